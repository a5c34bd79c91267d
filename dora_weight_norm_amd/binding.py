"""ctypes binding of libdora (include/dora.h).

Argument marshalling only: tensors are checked for device, dtype, shape and
layout, their data pointers and the current HIP stream are handed to the C
ABI, and outputs are allocated with torch. Every step of the computation
runs in libdora's kernels; there is no fallback path. If ``libdora.so`` is
missing, every call raises.

The function names match the C entry points.
"""

from __future__ import annotations

import contextlib
import ctypes
import os

import torch

__all__ = [
    "LIB_PATH",
    "DoraError",
    "load",
    "dora_version",
    "dora_status_string",
    "dora_norm_chunk_size",
    "dora_norm_workspace_size",
    "dora_norm_plan_info",
    "dora_factored_norm",
    "dora_magnitude_scale",
    "dora_norm_to_dtype",
    "dora_layer_output",
    "dora_compose",
    "DORA_BF16",
    "DORA_F32",
    "DORA_F16",
    "PLAN_FIELDS",
    "dora_compose_backward",
    "dora_compose_backward_workspace_size",
    "dora_factored_norm_marked",
    "dora_factored_norm_noalloc",
    "NOALLOC_SCRATCH_BYTES",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdora.so")

DORA_BF16 = 0
DORA_F32 = 1
DORA_F16 = 2
DEFAULT_BUDGET = 256 << 20
NOALLOC_SCRATCH_BYTES = 32 << 20   # DORA_NOALLOC_SCRATCH_BYTES

PLAN_FIELDS = (
    "mode", "tile_cols", "col_tiles", "gram_tile_cols", "gram_col_tiles", "fast_cfg", "gen_cfg",
    "gram_fast_cfg", "gram_gen_cfg", "granule", "granules", "w_ranges", "gram_ranges", "workspace_bytes",
    "w_grid", "gram_grid", "lds_bytes", "tile_rows", "gram_folded", "gram_symmetric", "gram_term_fused",
    "w_launch", "offsets32", "dense_row_tiles", "dense_col_tiles", "die_groups",
)

_lib = None
_c_i64 = ctypes.c_int64
_c_sz = ctypes.c_size_t
_c_p = ctypes.c_void_p
_c_f = ctypes.c_float
_c_i = ctypes.c_int


class DoraError(RuntimeError):
    """A libdora call returned a non-zero status."""

    def __init__(self, func: str, status: int):
        self.status = status
        super().__init__(f"{func}: {dora_status_string(status)} (status {status})")


def load():
    """Load libdora.so (after torch, so it binds to torch's HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -m dora_weight_norm_amd.build` "
            "or __graft_entry__.build()"
        )
    lib = ctypes.CDLL(LIB_PATH)
    sig = {
        "dora_status_string": (ctypes.c_char_p, [_c_i]),
        "dora_version": (_c_i, []),
        "dora_norm_chunk_size": (_c_i, [_c_i64, _c_i64, _c_sz, ctypes.POINTER(_c_i64)]),
        "dora_norm_workspace_size": (_c_i, [_c_i64, _c_i64, _c_i64, _c_i, _c_f, _c_sz, ctypes.POINTER(_c_sz)]),
        "dora_norm_plan_info": (_c_i, [_c_i64, _c_i64, _c_i64, _c_i, _c_f, _c_sz, ctypes.POINTER(_c_i64), _c_i]),
        "dora_factored_norm": (_c_i, [_c_p, _c_p, _c_p, _c_i, _c_i64, _c_i64, _c_i64, _c_f, _c_sz, _c_p, _c_sz,
                                      _c_p, _c_p, _c_f, _c_p, _c_p]),
        "dora_factored_norm_marked": (_c_i, [_c_p, _c_p, _c_p, _c_i, _c_i64, _c_i64, _c_i64, _c_f, _c_sz, _c_p,
                                             _c_sz, _c_p, _c_p, _c_f, _c_p, _c_p, ctypes.POINTER(_c_p), _c_i]),
        "dora_factored_norm_noalloc": (_c_i, [_c_p, _c_p, _c_p, _c_i, _c_i64, _c_i64, _c_i64, _c_f, _c_sz, _c_p,
                                              _c_p, _c_f, _c_p, _c_p]),
        "dora_magnitude_scale": (_c_i, [_c_p, _c_p, _c_f, _c_i64, _c_p, _c_p]),
        "dora_norm_to_dtype": (_c_i, [_c_p, _c_i64, _c_i, _c_p, _c_p]),
        "dora_compose": (_c_i, [_c_p, _c_p, _c_p, _c_f, _c_i, _c_i64, _c_i64, _c_p, _c_p]),
        "dora_layer_output": (_c_i, [_c_p, _c_p, _c_p, _c_f, _c_i, _c_i64, _c_i64, _c_p, _c_p]),
        "dora_compose_backward_workspace_size": (_c_i, [_c_i64, _c_i64, ctypes.POINTER(_c_sz)]),
        "dora_compose_backward": (_c_i, [_c_p, _c_p, _c_p, _c_p, _c_f, _c_i, _c_i64, _c_i64, _c_p, _c_p, _c_p,
                                         _c_p, _c_f, _c_p, _c_p, _c_sz, _c_p]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _call(name: str, *args) -> None:
    st = getattr(load(), name)(*args)
    if st != 0:
        raise DoraError(name, st)


def dora_version() -> int:
    return load().dora_version()


def dora_status_string(status: int) -> str:
    return load().dora_status_string(status).decode()


def _dtype_code(dtype) -> int:
    if dtype in (torch.bfloat16, "bf16", DORA_BF16):
        return DORA_BF16
    if dtype in (torch.float32, "f32", DORA_F32):
        return DORA_F32
    if dtype in (torch.float16, "f16", DORA_F16):
        return DORA_F16
    raise TypeError(f"unsupported dtype {dtype}; libdora takes bfloat16, float16 or float32")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t: torch.Tensor, name: str):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (row-major)")


def _out_like(t, name: str, shape, dtype, device):
    """A caller-supplied output buffer: on `device`, contiguous, exactly
    `shape` and `dtype` (the C ABI cannot see allocation sizes, so a short
    or mistyped buffer is refused here, before any launch)."""
    _dev(t, name)
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")


def _workspace(t, name: str, need: int, device):
    """A caller-supplied workspace: on `device`, contiguous, at least `need` bytes."""
    _dev(t, name)
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if t.numel() * t.element_size() < need:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes; {need} are needed")


def _on(stream):
    """Allocations made inside belong to `stream` (torch's caching allocator
    then reuses their memory only after the work queued on `stream`), so
    temporaries freed on return cannot be handed to other work while the
    kernels launched on `stream` still use them."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def dora_norm_chunk_size(d_out: int, d_in: int, budget_bytes: int = DEFAULT_BUDGET) -> int:
    cs = _c_i64()
    _call("dora_norm_chunk_size", d_out, d_in, budget_bytes, ctypes.byref(cs))
    return cs.value


def dora_norm_workspace_size(d_out: int, d_in: int, r: int, dtype, s: float,
                             budget_bytes: int = DEFAULT_BUDGET) -> int:
    ws = _c_sz()
    _call("dora_norm_workspace_size", d_out, d_in, r, _dtype_code(dtype), s, budget_bytes, ctypes.byref(ws))
    return ws.value


def dora_norm_plan_info(d_out: int, d_in: int, r: int, dtype, s: float,
                        budget_bytes: int = DEFAULT_BUDGET) -> dict:
    buf = (_c_i64 * len(PLAN_FIELDS))()
    _call("dora_norm_plan_info", d_out, d_in, r, _dtype_code(dtype), s, budget_bytes, buf, len(PLAN_FIELDS))
    return dict(zip(PLAN_FIELDS, list(buf)))


def dora_factored_norm(W, A, B, s: float, budget_bytes: int = DEFAULT_BUDGET, m=None, eps: float = 1e-6,
                       workspace=None, wnorm=None, g=None, stream=None, events=None):
    """wnorm = ||W + s B A||_row (fp32) and, if m is given, g = m / max(wnorm, eps).

    W [d_out, d_in], A [r, d_in], B [d_out, r], all of one dtype (bfloat16,
    float16 or float32), on the GPU. Returns (wnorm, g); g is None when m is
    None. `events` (a sequence of recorded torch.cuda.Event objects or None
    entries) selects dora_factored_norm_marked, which records them between
    the call's launches.
    """
    for t, nm in ((W, "W"), (A, "A"), (B, "B")):
        _dev(t, nm)
    if W.dim() != 2 or A.dim() != 2 or B.dim() != 2:
        raise ValueError("W, A, B must be 2-D")
    d_out, d_in = W.shape
    r = A.shape[0]
    if A.shape[1] != d_in or tuple(B.shape) != (d_out, r):
        raise ValueError(f"shape mismatch: W {tuple(W.shape)}, A {tuple(A.shape)}, B {tuple(B.shape)}")
    if not (W.dtype == A.dtype == B.dtype):
        raise TypeError("W, A, B must share one dtype")
    if not (W.device == A.device == B.device):
        raise ValueError("W, A, B must be on one device")
    dt = _dtype_code(W.dtype)
    dev = W.device
    ws_bytes = dora_norm_workspace_size(d_out, d_in, r, dt, s, budget_bytes)
    if workspace is not None:
        _workspace(workspace, "workspace", ws_bytes, dev)
    if wnorm is not None:
        _out_like(wnorm, "wnorm", (d_out,), torch.float32, dev)
    if m is not None:
        _out_like(m, "m", (d_out,), torch.float32, dev)
        if g is not None:
            _out_like(g, "g", (d_out,), torch.float32, dev)
    with _on(stream):
        if workspace is None and ws_bytes > 0:
            workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        if wnorm is None:
            wnorm = torch.empty(d_out, dtype=torch.float32, device=dev)
        if m is not None and g is None:
            g = torch.empty(d_out, dtype=torch.float32, device=dev)
        args = (_ptr(W), _ptr(A), _ptr(B), dt, d_out, d_in, r, s, budget_bytes, _ptr(workspace),
                0 if workspace is None else workspace.numel() * workspace.element_size(),
                _ptr(wnorm), _ptr(m), eps, _ptr(g) if m is not None else None, _stream(stream))
        if events is None:
            _call("dora_factored_norm", *args)
        else:
            handles = [None if e is None else int(getattr(e, "cuda_event", e)) for e in events]
            if any(h == 0 for h in handles):
                raise ValueError("an event has no HIP handle yet (record it once first)")
            arr = (_c_p * max(len(handles), 1))(*handles)
            _call("dora_factored_norm_marked", *args, arr, len(handles))
    return wnorm, (g if m is not None else None)


def dora_factored_norm_marked(W, A, B, s: float, events, **kw):
    """dora_factored_norm with HIP events recorded between its launches
    (events[0] before the first, events[i] after the i-th; None entries
    skipped). Same keywords and results as dora_factored_norm."""
    return dora_factored_norm(W, A, B, s, events=list(events), **kw)


def dora_factored_norm_noalloc(W, A, B, s: float, budget_bytes: int = DEFAULT_BUDGET, m=None, eps: float = 1e-6,
                               wnorm=None, g=None, stream=None):
    """dora_factored_norm with the library's per-GPU scratch array as its
    workspace (the C call allocates nothing). wnorm and g may be passed in,
    so that the call itself allocates nothing either. Returns (wnorm, g)."""
    for t, nm in ((W, "W"), (A, "A"), (B, "B")):
        _dev(t, nm)
    if W.dim() != 2 or A.dim() != 2 or B.dim() != 2:
        raise ValueError("W, A, B must be 2-D")
    d_out, d_in = W.shape
    r = A.shape[0]
    if A.shape[1] != d_in or tuple(B.shape) != (d_out, r):
        raise ValueError(f"shape mismatch: W {tuple(W.shape)}, A {tuple(A.shape)}, B {tuple(B.shape)}")
    if not (W.dtype == A.dtype == B.dtype):
        raise TypeError("W, A, B must share one dtype")
    if not (W.device == A.device == B.device):
        raise ValueError("W, A, B must be on one device")
    dev = W.device
    if wnorm is not None:
        _out_like(wnorm, "wnorm", (d_out,), torch.float32, dev)
    if m is not None:
        _out_like(m, "m", (d_out,), torch.float32, dev)
        if g is not None:
            _out_like(g, "g", (d_out,), torch.float32, dev)
    with _on(stream):
        if wnorm is None:
            wnorm = torch.empty(d_out, dtype=torch.float32, device=dev)
        if m is not None and g is None:
            g = torch.empty(d_out, dtype=torch.float32, device=dev)
        _call("dora_factored_norm_noalloc", _ptr(W), _ptr(A), _ptr(B), _dtype_code(W.dtype), d_out, d_in, r, s,
              budget_bytes, _ptr(wnorm), _ptr(m), eps, _ptr(g) if m is not None else None, _stream(stream))
    return wnorm, (g if m is not None else None)


def dora_magnitude_scale(m, wnorm, eps: float = 1e-6, g=None, stream=None):
    """g = m / max(wnorm, eps), fp32 [d_out]."""
    _dev(m, "m")
    if m.dtype != torch.float32 or m.dim() != 1:
        raise ValueError("m must be float32 [d_out]")
    _out_like(wnorm, "wnorm", m.shape, torch.float32, m.device)
    if g is not None:
        _out_like(g, "g", m.shape, torch.float32, m.device)
    with _on(stream):
        if g is None:
            g = torch.empty_like(m)
        _call("dora_magnitude_scale", _ptr(m), _ptr(wnorm), eps, m.numel(), _ptr(g), _stream(stream))
    return g


def dora_norm_to_dtype(wnorm, dtype, out=None, stream=None):
    """wnorm (fp32 [n]) rounded to `dtype` (bfloat16, float16 or float32), nearest even."""
    _dev(wnorm, "wnorm")
    if wnorm.dtype != torch.float32 or wnorm.dim() != 1:
        raise ValueError("wnorm must be float32 [n]")
    tdt = {DORA_BF16: torch.bfloat16, DORA_F32: torch.float32, DORA_F16: torch.float16}[_dtype_code(dtype)]
    if out is not None:
        _out_like(out, "out", wnorm.shape, tdt, wnorm.device)
    with _on(stream):
        if out is None:
            out = torch.empty(wnorm.shape, dtype=tdt, device=wnorm.device)
        _call("dora_norm_to_dtype", _ptr(wnorm), wnorm.numel(), _dtype_code(dtype), _ptr(out), _stream(stream))
    return out


def _compose_call(name, base, lora, g, s, out, stream):
    for t, nm in ((base, "base"), (lora, "lora"), (g, "g")):
        _dev(t, nm)
    if base.shape != lora.shape or base.dtype != lora.dtype:
        raise ValueError("base and lora must share shape and dtype")
    if base.dim() != 2:
        raise ValueError("base and lora must be [T, d_out]")
    T, d_out = base.shape
    if g.dtype != torch.float32 or g.shape != (d_out,):
        raise ValueError("g must be float32 [d_out]")
    if not (base.device == lora.device == g.device):
        raise ValueError("base, lora and g must be on one device")
    dt = _dtype_code(base.dtype)
    if out is not None:
        _out_like(out, "out", base.shape, base.dtype, base.device)
    with _on(stream):
        if out is None:
            out = torch.empty_like(base)
        _call(name, _ptr(base), _ptr(lora), _ptr(g), s, dt, T, d_out, _ptr(out), _stream(stream))
    return out


def dora_compose(base, lora, g, s: float, out=None, stream=None):
    """out = (g - 1) * base + g * (s * lora), with g [d_out] scaling columns of [T, d_out]."""
    return _compose_call("dora_compose", base, lora, g, s, out, stream)


def dora_layer_output(base, lora, g, s: float, y=None, stream=None):
    """y = base + ((g - 1) * base + g * (s * lora)): the DoRA layer output, one rounding."""
    return _compose_call("dora_layer_output", base, lora, g, s, y, stream)

def dora_compose_backward_workspace_size(T: int, d_out: int) -> int:
    ws = _c_sz()
    _call("dora_compose_backward_workspace_size", T, d_out, ctypes.byref(ws))
    return ws.value


def dora_compose_backward(dy, base, lora, g, s: float, need_dg: bool = True, wnorm=None, eps: float = 1e-6,
                          d_base=None, d_lora=None, workspace=None, stream=None):
    """Gradients of delta = (g - 1) * base + g * (s * lora), the row norm detached.

    Returns (d_base, d_lora, dg, dm): d_base and d_lora like dy; dg fp32
    [d_out] (None when need_dg is False: the magnitude is frozen, base and
    lora are then not read and may be None); dm = dg / max(wnorm, eps) when
    wnorm is given.
    """
    _dev(dy, "dy")
    _dev(g, "g")
    if dy.dim() != 2:
        raise ValueError("dy must be [T, d_out]")
    T, d_out = dy.shape
    if g.dtype != torch.float32 or g.shape != (d_out,):
        raise ValueError("g must be float32 [d_out]")
    if need_dg:
        for t, nm in ((base, "base"), (lora, "lora")):
            _dev(t, nm)
            if t.shape != dy.shape or t.dtype != dy.dtype:
                raise ValueError(f"{nm} must match dy")
    if wnorm is not None:
        if not need_dg:
            raise ValueError("dm needs dg")
        _dev(wnorm, "wnorm")
        if wnorm.dtype != torch.float32 or wnorm.shape != (d_out,):
            raise ValueError("wnorm must be float32 [d_out]")
    dt = _dtype_code(dy.dtype)
    dev = dy.device
    if g.device != dev:
        raise ValueError("g must be on dy's device")
    if d_base is not None:
        _out_like(d_base, "d_base", dy.shape, dy.dtype, dev)
    if d_lora is not None:
        _out_like(d_lora, "d_lora", dy.shape, dy.dtype, dev)
    ws_bytes = dora_compose_backward_workspace_size(T, d_out) if need_dg else 0
    if workspace is not None and ws_bytes > 0:
        _workspace(workspace, "workspace", ws_bytes, dev)
    with _on(stream):
        d_base = torch.empty_like(dy) if d_base is None else d_base
        d_lora = torch.empty_like(dy) if d_lora is None else d_lora
        dg = torch.empty(d_out, dtype=torch.float32, device=dev) if need_dg else None
        dm = torch.empty(d_out, dtype=torch.float32, device=dev) if wnorm is not None else None
        if workspace is None and ws_bytes > 0:
            workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        _call("dora_compose_backward", _ptr(dy), _ptr(base if need_dg else None), _ptr(lora if need_dg else None),
              _ptr(g), s, dt, T, d_out, _ptr(d_base), _ptr(d_lora), _ptr(dg), _ptr(wnorm), eps, _ptr(dm),
              _ptr(workspace), ws_bytes if workspace is not None else 0, _stream(stream))
    return d_base, d_lora, dg, dm
