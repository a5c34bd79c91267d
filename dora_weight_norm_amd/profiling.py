"""Summaries of rocprofv3 runs of bench.py, for the profiles/ folder.

Turns the CSV output of three rocprofv3 runs of the same bench command
(kernel trace with --stats, then --pmc FETCH_SIZE, then --pmc WRITE_SIZE),
and optionally a fourth (--pmc MfmaFlopsBF16 MfmaFlopsF32 MfmaUtil: the
matrix-core work each dispatch executed and the share of cycles the matrix
cores were busy), into

  profiles/<kernel-set>_<workload>.md   per-kernel durations, counters and
                                        the commands that produced them;
  profiles/traffic_<workload>.json      measured HBM bytes per norm call, per
                                        compose call and per compose backward
                                        call, read by bench.py.

FETCH_SIZE and WRITE_SIZE are reported in KiB per dispatch. Each is scaled by
what the same counter reads for a plain device copy of known size (bench.py
--copy-calibration runs one of 1 GiB), so that the figures are bytes.

    python -m dora_weight_norm_amd.profiling --workload NAME --kt DIR --fetch DIR --write DIR \
        --cmd-kt "..." --cmd-fetch "..." --cmd-write "..." [--mfma DIR --cmd-mfma "..."] [--out profiles]
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
CALIB_BYTES = 1 << 30   # bench.py --copy-calibration copies this many bytes


def _code_only(text: str) -> str:
    """C/C++ source without comments and trailing blanks: a change to the
    comments alone leaves the kernels, and so the counters, as they were."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":                       # string or character literal, kept whole
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            while i < n and text[i] != "\n":
                i += 1
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return "\n".join(line.rstrip() for line in "".join(out).splitlines() if line.strip())


def source_hash() -> str:
    """Hash of the HIP sources' code (comments excluded): measured traffic is
    only valid for this code."""
    h = hashlib.sha256()
    for path in sorted(glob.glob(os.path.join(HERE, "csrc", "*"))):
        with open(path, encoding="utf-8") as f:
            h.update(os.path.basename(path).encode())
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


# Itanium-ABI codes of the template arguments the library's kernels take.
_MANGLED_TYPES = {"t": "unsigned short", "DF16_": "_Float16", "f": "float", "b": "bool", "i": "int"}


def demangle_ours(name: str) -> str:
    """A kernel name of this library as rocprofv3 prints it demangled.

    rocprofv3 leaves a name mangled when its demangler does not know a type
    in it (_Float16, code DF16_). The library's kernels are templates in
    namespace dora::(anonymous) over types and integers only, so their
    names are decoded here: identifier, then template arguments (types of
    _MANGLED_TYPES and integer literals L<type><value>E). Other names are
    returned as they are."""
    m = re.match(r"_ZN4dora12_GLOBAL__N_1(\d+)", name)
    if not m:
        return name
    i = m.end()
    ident = name[i:i + int(m.group(1))]
    i += len(ident)
    args = []
    if name.startswith("I", i):
        i += 1
        while i < len(name) and name[i] != "E":
            lit = re.match(r"L([a-z])(n?\d+)E", name[i:])
            if lit:
                val = lit.group(2).replace("n", "-")
                args.append({"0": "false", "1": "true"}[val] if lit.group(1) == "b" else val)
                i += lit.end()
                continue
            for code, typ in _MANGLED_TYPES.items():
                if name.startswith(code, i):
                    args.append(typ)
                    i += len(code)
                    break
            else:
                return name   # not a form this decoder knows
    targs = f"<{', '.join(args)}>" if args else ""
    return f"void dora::(anonymous namespace)::{ident}{targs}()"


def kernel_role(name: str) -> str | None:
    """Which part of the hot path a kernel belongs to (None: not ours)."""
    name = demangle_ours(name)
    if "dora::" not in name:
        return None
    if "compose_bwd" in name:
        return "compose_bwd"
    if "compose_kernel" in name:
        # compose_kernel<T, VEC, ADD>: ADD = true is the layer output
        return "layer_output" if re.search(r"compose_kernel<[^>]*true>", name) else "compose"
    return "norm"   # the norm call's kernels, and the widening and casts around it


def short_name(name: str) -> str:
    n = demangle_ours(name).replace("(anonymous namespace)::", "").replace("unsigned short", "bf16")
    n = n.replace("_Float16", "f16")
    n = re.sub(r"\(dora::NormPlan.*$|\(.*$", "", n)
    n = n.replace("void dora::", "").replace("dora::", "")
    m = re.match(r"norm_fast_kernel<(.*)>", n)
    if m:
        args = [a.strip() for a in m.group(1).split(",")]
        mode = {"0": "W pass", "1": "Gram pass", "2": "Gram term + assembly", "3": "W pass + G blocks",
                "4": "W pass + Gram term"}.get(args[-1], args[-1])
        n = f"norm_fast_kernel<{', '.join(args)}> ({mode})"
    m = re.match(r"norm_dense_kernel<(.*)>", n)
    if m:
        n = f"norm_dense_kernel<{m.group(1)}> (dense pass)"
    return n


def is_main_pass(name: str) -> bool:
    """The norm call's main pass: the W pass, or the dense pass where the plan takes it."""
    short = short_name(name)
    return "(W pass" in short or "(dense pass)" in short


def _one(pattern: str) -> str:
    hits = sorted(glob.glob(pattern))
    if not hits:
        raise FileNotFoundError(pattern)
    return hits[0]


def read_stats(kt_dir: str):
    rows = list(csv.DictReader(open(_one(os.path.join(kt_dir, "*kernel_stats.csv")))))
    out = []
    for r in rows:
        out.append({"name": r["Name"], "calls": int(r["Calls"]), "avg_us": float(r["AverageNs"]) / 1e3,
                    "min_us": float(r["MinNs"]) / 1e3, "max_us": float(r["MaxNs"]) / 1e3,
                    "total_us": float(r["TotalDurationNs"]) / 1e3})
    return out


def read_counter(pmc_dir: str, counter: str):
    rows = list(csv.DictReader(open(_one(os.path.join(pmc_dir, "*counter_collection.csv")))))
    per = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return per


def calibration(per: dict) -> float:
    """KiB the counter reports for the 1 GiB copy: the largest copy dispatch."""
    best = 0.0
    for name, vals in per.items():
        if "copy" in name and "dora::" not in name:
            best = max(best, max(vals))
    if best <= 0:
        raise RuntimeError("no copy dispatch found for the calibration")
    return (CALIB_BYTES / 1024.0) / best


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", required=True)
    ap.add_argument("--kt", required=True)
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--cmd-kt", required=True)
    ap.add_argument("--cmd-fetch", required=True)
    ap.add_argument("--cmd-write", required=True)
    ap.add_argument("--mfma", default=None)
    ap.add_argument("--cmd-mfma", default=None)
    ap.add_argument("--out", default=os.path.join(os.path.dirname(HERE), "profiles"))
    args = ap.parse_args()

    stats = read_stats(args.kt)
    fetch = read_counter(args.fetch, "FETCH_SIZE")
    write = read_counter(args.write, "WRITE_SIZE")
    f_scale, w_scale = calibration(fetch), calibration(write)
    mflops, mutil = {}, {}
    if args.mfma:
        for counter in ("MfmaFlopsBF16", "MfmaFlopsF32"):
            for name, vals in read_counter(args.mfma, counter).items():
                mflops[name] = mflops.get(name, 0.0) + sum(vals) / len(vals)
        mutil = {name: sum(v) / len(v) for name, v in read_counter(args.mfma, "MfmaUtil").items()}

    ours = [s for s in stats if kernel_role(s["name"])]
    # Calls of each part: every kernel of a part runs at least once per call,
    # so the least-called kernel of the part counts its calls.
    part_calls = {}
    for s in ours:
        role = kernel_role(s["name"])
        part_calls[role] = min(part_calls.get(role, s["calls"]), s["calls"])
    steps = part_calls["compose"]
    traffic = {"norm": 0.0, "compose": 0.0, "compose_bwd": 0.0, "layer_output": 0.0}
    w_pass_bytes = None   # HBM bytes of one W-pass launch
    w_pass_mfma = None    # (executed MFMA flops, MFMA busy %) of one W-pass launch
    w_pass_us = None      # the W-pass kernel's average duration
    lines = []
    for s in sorted(ours, key=lambda s: -s["total_us"]):
        role = kernel_role(s["name"])
        fk = fetch.get(s["name"], [])
        wk = write.get(s["name"], [])
        fb = (sum(fk) / len(fk)) * 1024 * f_scale if fk else float("nan")
        wb = (sum(wk) / len(wk)) * 1024 * w_scale if wk else float("nan")
        per_step = s["calls"] / part_calls[role]
        if fk and wk:
            traffic[role] += (fb + wb) * per_step
            if role == "norm" and is_main_pass(s["name"]):
                w_pass_bytes = fb + wb
        if role == "norm" and is_main_pass(s["name"]):
            w_pass_us = s["avg_us"]
        mcols = ""
        if args.mfma:
            mf, mu = mflops.get(s["name"]), mutil.get(s["name"])
            mcols = (f" {mf / 1e9:.2f} |" if mf is not None else " — |") + (f" {mu:.1f} |" if mu is not None else " — |")
            if role == "norm" and is_main_pass(s["name"]) and mf is not None:
                w_pass_mfma = (mf, mu)
        lines.append(f"| {short_name(s['name'])} | {role} | {s['calls']} | {s['avg_us']:.2f} | {s['min_us']:.2f} | "
                     f"{s['max_us']:.2f} | {fb / 1e6:.2f} | {wb / 1e6:.2f} |" + mcols)
    def part_us(role):
        return sum(s["avg_us"] * s["calls"] / part_calls[role] for s in ours if kernel_role(s["name"]) == role)

    norm_us, comp_us = part_us("norm"), part_us("compose")
    bwd_us = part_us("compose_bwd") if "compose_bwd" in part_calls else 0.0
    # The longest single launch of a step decides which roofline bench.py
    # reports as the dominant kernel.
    step_kernels = [s for s in ours if kernel_role(s["name"]) in ("norm", "compose")]
    longest = max(step_kernels, key=lambda s: s["avg_us"])

    os.makedirs(args.out, exist_ok=True)
    tj = {"workload": args.workload, "source_hash": source_hash(),
          "norm_bytes_per_call": traffic["norm"], "compose_bytes_per_call": traffic["compose"],
          "fetch_scale": f_scale, "write_scale": w_scale,
          "compose_bwd_bytes_per_call": traffic["compose_bwd"],
          "w_pass_bytes_per_launch": w_pass_bytes,
          "w_pass_us_per_launch": w_pass_us,
          "w_pass_mfma_flops_per_launch": w_pass_mfma[0] if w_pass_mfma else None,
          "w_pass_mfma_busy_pct": w_pass_mfma[1] if w_pass_mfma else None,
          "norm_us_per_call": norm_us, "compose_us_per_call": comp_us, "compose_bwd_us_per_call": bwd_us,
          "longest_step_kernel": {"name": short_name(longest["name"]), "part": kernel_role(longest["name"]),
                                  "avg_us": longest["avg_us"]},
          "commands": {"fetch": args.cmd_fetch, "write": args.cmd_write}}
    with open(os.path.join(args.out, f"traffic_{args.workload}.json"), "w") as f:
        json.dump(tj, f, indent=1)
        f.write("\n")
    mhead = " MFMA GF | MFMA busy % |" if args.mfma else ""
    msep = "---|---|" if args.mfma else ""
    md = [f"# Norm and compose kernels, workload {args.workload}", "",
          "rocprofv3 kernel trace (durations) and counter passes (HBM bytes"
          + ("; matrix-core work and busy share" if args.mfma else "") + ") of the same bench.py",
          "command. Bytes and MFMA work are per dispatch; bytes are scaled by the copy calibration below.", "",
          "| kernel | part | calls | avg µs | min µs | max µs | FETCH MB | WRITE MB |" + mhead,
          "|---|---|---|---|---|---|---|---|" + msep] + lines + [
          "",
          f"- compose calls in the trace: {steps}; norm call = sum of its kernels = {norm_us:.2f} µs; "
          f"compose call = {comp_us:.2f} µs",
          f"- longest single launch of a step: {short_name(longest['name'])} ({longest['avg_us']:.2f} µs)",
          f"- HBM traffic per norm call: {traffic['norm'] / 1e6:.1f} MB (W-pass launch: "
          f"{(w_pass_bytes or 0) / 1e6:.1f} MB); per compose call: {traffic['compose'] / 1e6:.1f} MB",
          f"- compose backward call (timed on its own after the steps) = {bwd_us:.2f} µs; HBM traffic "
          f"{traffic['compose_bwd'] / 1e6:.1f} MB",
          f"- copy calibration (1 GiB device copy): FETCH_SIZE x{f_scale:.3f}, WRITE_SIZE x{w_scale:.3f}",
          f"- HIP sources hash (code without comments): {tj['source_hash']}", "",
          "Commands:", "", "```", args.cmd_kt, args.cmd_fetch, args.cmd_write]
    md += ([args.cmd_mfma] if args.mfma and args.cmd_mfma else []) + ["```", ""]
    with open(os.path.join(args.out, f"norm_compose_{args.workload}.md"), "w") as f:
        f.write("\n".join(md))
    print("\n".join(md))
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
