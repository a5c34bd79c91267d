// C ABI of libdora: argument checks, the norm's work plan, and launches.
// Every check runs on the host before anything is enqueued; a failed check
// returns a status and touches no device state.
#include <math.h>
#include <string.h>

#include <vector>

#include "../../include/dora.h"
#include "dora_launch.h"
#include "dora_plan.h"

using dora::NormPlan;

namespace {

constexpr int kVersion = 10000;  // 1.0.0
constexpr size_t kAlign = 256;

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool valid_dtype(int dt) { return dt == DORA_BF16 || dt == DORA_F32; }
int64_t esize(int dt) { return dt == DORA_BF16 ? 2 : 4; }
int64_t epc(int dt) { return dt == DORA_BF16 ? 8 : 4; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Byte ranges [a, a+na) and [b, b+nb) intersect (empty ranges never do).
bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
  if (a == nullptr || b == nullptr || na <= 0 || nb <= 0) return false;
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + (uintptr_t)nb && pb < pa + (uintptr_t)na;
}

// Upper bounds that keep every index and grid dimension in range.
constexpr int64_t kMaxDim = (int64_t)1 << 31;
constexpr int64_t kMaxRank = (int64_t)1 << 16;

int choose_cfg(int dtype, int64_t r) {
  if (dtype == DORA_F32) return r <= 32 ? dora::kF32R32 : dora::kF32R128;
  if (r <= 64) return dora::kBf16R64;
  if (r <= 128) return dora::kBf16R128;
  if (r <= 256) return dora::kBf16R256;
  if (r <= 384) return dora::kBf16R384;
  if (r <= 512) return dora::kBf16R512;
  return dora::kBf16R768;
}

int compute_maxseg(const NormPlan& p) {
  const int64_t T = dora::n_tiles(p);
  int maxseg = 1;
  for (int x = 0; x < p.X; ++x) {
    const int64_t nk = dora::range_lo(p.n_kt, p.X, x + 1) - dora::range_lo(p.n_kt, p.X, x);
    const int64_t U = T * nk;
    for (int64_t t = 0; t < T; ++t) {
      const int sa = dora::slot_of(U, p.P, t * nk), sb = dora::slot_of(U, p.P, t * nk + nk - 1);
      if (sb - sa + 1 > maxseg) maxseg = sb - sa + 1;
    }
  }
  return maxseg;
}

void layout(NormPlan& p) {
  const int64_t xs = (int64_t)p.X * p.maxseg;
  size_t off = 0;
  p.off_base = off;
  off = align_up(off + (size_t)(xs * p.ld_w) * 4, kAlign);
  p.off_cross = off;
  off = align_up(off + (size_t)(xs * p.n_nt * p.ld_w) * 4, kAlign);
  p.off_g = off;
  off = align_up(off + (size_t)(xs * p.ga_rows * p.ga_cols) * 4, kAlign);
  p.off_ghi = off;
  off = align_up(off + (size_t)(p.r32 * p.r32) * (p.dtype == DORA_BF16 ? 2 : 4), kAlign);
  p.off_glo = off;
  if (p.dtype == DORA_BF16) off = align_up(off + (size_t)(p.r32 * p.r32) * 2, kAlign);
  p.off_ba = off;
  off = align_up(off + (size_t)((int64_t)p.n_cb * p.ld_w) * 4, kAlign);
  p.ws_bytes = off;
}

dora_status check_sizes(int64_t d_out, int64_t d_in, int64_t r) {
  if (d_out < 0 || d_in < 0 || r < 0) return DORA_ERR_INVALID_ARG;
  if (d_out >= kMaxDim || d_in >= kMaxDim || r >= kMaxRank) return DORA_ERR_INVALID_ARG;
  return DORA_OK;
}

dora_status make_plan(int64_t d_out, int64_t d_in, int64_t r, int dtype, float s, size_t budget,
                      NormPlan* out) {
  if (!valid_dtype(dtype)) return DORA_ERR_UNSUPPORTED_DTYPE;
  dora_status st = check_sizes(d_out, d_in, r);
  if (st != DORA_OK) return st;
  NormPlan p;
  memset(&p, 0, sizeof(p));
  p.d_out = d_out;
  p.d_in = d_in;
  p.r = r;
  p.dtype = dtype;
  if (d_out == 0) {
    p.mode = dora::kModeEmpty;
    *out = p;
    return DORA_OK;
  }
  if (s == 0.0f || r == 0 || d_in == 0) {
    p.mode = dora::kModeRowOnly;
    *out = p;
    return DORA_OK;
  }
  p.mode = dora::kModeFactored;
  p.cfg = choose_cfg(dtype, r);
  const dora::TileShape ts = dora::tile_shape(p.cfg);
  p.mt = ts.wm * ts.mb * 32;
  p.ntc = ts.wn * ts.nb * 32;
  p.kt = ts.kt;
  p.n_mt_w = (int)ceil_div(d_out, p.mt);
  p.n_mt_a = (int)ceil_div(r, p.mt);
  p.n_nt = (int)ceil_div(r, p.ntc);
  p.n_kt = ceil_div(d_in, p.kt);
  p.ld_w = (int64_t)p.n_mt_w * p.mt;
  p.ga_rows = (int64_t)p.n_mt_a * p.mt;
  p.ga_cols = (int64_t)p.n_nt * p.ntc;
  p.r32 = ceil_div(r, 32) * 32;
  p.n_cb = (int)ceil_div(p.r32, dora::kGramCB);

  // Most parallel split first: one d_in range per die, every compute unit
  // busy. Then fewer workgroups, which shrink the partials.
  const int X0 = (int)(p.n_kt < dora::kDies ? p.n_kt : dora::kDies);
  const int cand[][2] = {{X0, dora::kGrid / X0}, {1, 64}, {1, 16}, {1, 4}, {1, 1}};
  for (const auto& c : cand) {
    p.X = c[0];
    p.P = c[1];
    // Never more workgroups per range than work units in its smallest range:
    // then no workgroup is empty, and the partials of a tile are exactly
    // those of workgroups slot_of(first unit) .. slot_of(last unit).
    const int64_t u_min = dora::n_tiles(p) * (p.n_kt / p.X);
    if (u_min < p.P) p.P = (int)u_min;
    p.maxseg = compute_maxseg(p);
    layout(p);
    if (p.ws_bytes <= budget) {
      *out = p;
      return DORA_OK;
    }
  }
  return DORA_ERR_BUDGET;
}

// Host replay of the kernels' work split: every (range, tile, stage) unit is
// owned by exactly one workgroup, segment indices stay below maxseg, and the
// reduction's enumeration of a tile's segments matches the producers.
bool plan_self_check(const NormPlan& p) {
  if (p.mode != dora::kModeFactored) return true;
  const int64_t T = dora::n_tiles(p);
  for (int x = 0; x < p.X; ++x) {
    const int64_t nk = dora::range_lo(p.n_kt, p.X, x + 1) - dora::range_lo(p.n_kt, p.X, x);
    if (nk <= 0) return false;
    const int64_t U = T * nk;
    std::vector<int> cover((size_t)U, 0);
    std::vector<int> seg_of((size_t)(T * p.maxseg), -1);  // producer slot per (tile, seg)
    for (int slot = 0; slot < p.P; ++slot) {
      int64_t u = dora::unit_lo(U, p.P, slot);
      const int64_t ue = dora::unit_lo(U, p.P, slot + 1);
      while (u < ue) {
        const int64_t t = u / nk, i0 = u - t * nk;
        const int64_t i1 = (ue - u < nk - i0) ? i0 + (ue - u) : nk;
        const int seg = slot - dora::slot_of(U, p.P, t * nk);
        if (seg < 0 || seg >= p.maxseg) return false;
        int& prod = seg_of[(size_t)(t * p.maxseg + seg)];
        if (prod != -1) return false;
        prod = slot;
        for (int64_t i = i0; i < i1; ++i) cover[(size_t)(t * nk + i)] += 1;
        u += i1 - i0;
      }
    }
    for (int64_t w = 0; w < U; ++w)
      if (cover[(size_t)w] != 1) return false;
    for (int64_t t = 0; t < T; ++t) {
      const int sa = dora::slot_of(U, p.P, t * nk), sb = dora::slot_of(U, p.P, t * nk + nk - 1);
      for (int sl = sa; sl <= sb; ++sl) {
        const int k = sl - sa;
        if (k >= p.maxseg) return false;
        if (seg_of[(size_t)(t * p.maxseg + k)] != sl) return false;   // every slot in range produced
      }
      for (int k = sb - sa + 1; k < p.maxseg; ++k)
        if (seg_of[(size_t)(t * p.maxseg + k)] != -1) return false;
    }
  }
  return true;
}

dora_status hip_status(hipError_t e) { return e == hipSuccess ? DORA_OK : DORA_ERR_HIP; }

}  // namespace

extern "C" {

const char* dora_status_string(int status) {
  switch (status) {
    case DORA_OK: return "ok";
    case DORA_ERR_INVALID_ARG: return "invalid argument";
    case DORA_ERR_UNSUPPORTED_DTYPE: return "unsupported dtype";
    case DORA_ERR_BUDGET: return "workspace needed exceeds the byte budget";
    case DORA_ERR_WORKSPACE: return "workspace too small or misaligned";
    case DORA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int dora_version(void) { return kVersion; }

dora_status dora_norm_chunk_size(int64_t d_out, int64_t d_in, size_t budget_bytes, int64_t* cs) {
  if (cs == nullptr || d_out < 0 || d_in < 0) return DORA_ERR_INVALID_ARG;
  if (d_out == 0 || d_in == 0) {
    *cs = d_in;
    return DORA_OK;
  }
  const uint64_t raw = (uint64_t)budget_bytes / (4ull * (uint64_t)d_out);
  uint64_t al = (raw / 64) * 64;
  if (al < 64) al = 64;
  *cs = (int64_t)(al < (uint64_t)d_in ? al : (uint64_t)d_in);
  return DORA_OK;
}

dora_status dora_norm_workspace_size(int64_t d_out, int64_t d_in, int64_t r, int dtype, float s,
                                     size_t budget_bytes, size_t* ws_bytes) {
  if (ws_bytes == nullptr || !isfinite(s)) return DORA_ERR_INVALID_ARG;
  NormPlan p;
  const dora_status st = make_plan(d_out, d_in, r, dtype, s, budget_bytes, &p);
  if (st != DORA_OK) return st;
  *ws_bytes = p.ws_bytes;
  return DORA_OK;
}

dora_status dora_norm_plan_info(int64_t d_out, int64_t d_in, int64_t r, int dtype, float s,
                                size_t budget_bytes, int64_t* info, int n_info) {
  if (info == nullptr || n_info < 0 || !isfinite(s)) return DORA_ERR_INVALID_ARG;
  NormPlan p;
  const dora_status st = make_plan(d_out, d_in, r, dtype, s, budget_bytes, &p);
  if (st != DORA_OK) return st;
  if (!plan_self_check(p)) return DORA_ERR_INVALID_ARG;
  const int64_t vals[] = {p.mode, p.cfg, p.mt, p.ntc, p.kt, p.n_mt_w, p.n_mt_a, p.n_nt, p.n_kt,
                          p.X, p.P, p.maxseg, (int64_t)p.ws_bytes,
                          p.mode == dora::kModeFactored ? (int64_t)p.X * p.P : 0,
                          p.mode == dora::kModeFactored ? (int64_t)dora::main_kernel_lds_bytes(p.cfg) : 0};
  const int nv = (int)(sizeof(vals) / sizeof(vals[0]));
  for (int i = 0; i < n_info && i < nv; ++i) info[i] = vals[i];
  for (int i = nv; i < n_info; ++i) info[i] = -1;
  return DORA_OK;
}

dora_status dora_factored_norm(const void* W, const void* A, const void* B, int dtype, int64_t d_out,
                               int64_t d_in, int64_t r, float s, size_t budget_bytes, void* workspace,
                               size_t workspace_bytes, float* wnorm, const float* m, float eps, float* g,
                               void* stream) {
  if (!valid_dtype(dtype)) return DORA_ERR_UNSUPPORTED_DTYPE;
  dora_status st = check_sizes(d_out, d_in, r);
  if (st != DORA_OK) return st;
  if (!isfinite(s)) return DORA_ERR_INVALID_ARG;
  if (m != nullptr && (!isfinite(eps) || !(eps > 0.0f))) return DORA_ERR_INVALID_ARG;
  NormPlan p;
  st = make_plan(d_out, d_in, r, dtype, s, budget_bytes, &p);
  if (st != DORA_OK) return st;
  if (p.mode == dora::kModeEmpty) return DORA_OK;

  const int64_t es = esize(dtype);
  const int64_t nW = d_out * d_in * es, nA = r * d_in * es, nB = d_out * r * es, nV = d_out * 4;
  const bool factored = p.mode == dora::kModeFactored;
  if (wnorm == nullptr) return DORA_ERR_INVALID_ARG;
  if (nW > 0 && W == nullptr) return DORA_ERR_INVALID_ARG;
  if (factored && (A == nullptr || B == nullptr)) return DORA_ERR_INVALID_ARG;
  if (m != nullptr && g == nullptr) return DORA_ERR_INVALID_ARG;
  if (!aligned(W, (size_t)es) || !aligned(wnorm, 4) || !aligned(m, 4) || !aligned(g, 4))
    return DORA_ERR_INVALID_ARG;
  if (factored && (!aligned(A, (size_t)es) || !aligned(B, (size_t)es))) return DORA_ERR_INVALID_ARG;
  const void* gout = (m != nullptr) ? g : nullptr;
  const int64_t nWs = factored ? (int64_t)p.ws_bytes : 0;
  // Outputs must not overlap inputs, the workspace or each other; g may be m itself.
  const void* ins[] = {W, factored ? A : nullptr, factored ? B : nullptr};
  const int64_t nin[] = {nW, nA, nB};
  for (int i = 0; i < 3; ++i) {
    if (overlap(wnorm, nV, ins[i], nin[i]) || overlap(gout, nV, ins[i], nin[i])) return DORA_ERR_INVALID_ARG;
    if (overlap(workspace, nWs, ins[i], nin[i])) return DORA_ERR_INVALID_ARG;
  }
  if (overlap(wnorm, nV, gout, nV) || overlap(wnorm, nV, m, nV)) return DORA_ERR_INVALID_ARG;
  if (gout != nullptr && gout != m && overlap(gout, nV, m, nV)) return DORA_ERR_INVALID_ARG;
  if (overlap(workspace, nWs, wnorm, nV) || overlap(workspace, nWs, gout, nV) || overlap(workspace, nWs, m, nV))
    return DORA_ERR_INVALID_ARG;

  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (!factored) {
    const bool vec = aligned(W, 16) && (d_in % epc(dtype)) == 0;
    return hip_status(dora::launch_norm_rowonly(W, dtype, d_out, d_in, vec, m, eps, wnorm, gout ? g : nullptr, hs));
  }
  if (workspace_bytes < p.ws_bytes) return DORA_ERR_WORKSPACE;
  if (p.ws_bytes > 0 && (workspace == nullptr || !aligned(workspace, kAlign))) return DORA_ERR_WORKSPACE;
  // The fast main kernel addresses a tile's rows with 32-bit byte offsets.
  const uint64_t tile_span = (uint64_t)(p.mt > p.ntc ? p.mt : p.ntc) * (uint64_t)d_in * (uint64_t)es;
  p.vec_in = aligned(W, 16) && aligned(A, 16) && (d_in % epc(dtype)) == 0 && tile_span < (1ull << 32);
  p.vec_b = aligned(B, 16) && (r % epc(dtype)) == 0;
  return hip_status(dora::launch_norm_factored(p, W, A, B, workspace, s, m, eps, wnorm, g, hs));
}

dora_status dora_magnitude_scale(const float* m, const float* wnorm, float eps, int64_t d_out, float* g,
                                 void* stream) {
  if (d_out < 0 || d_out >= kMaxDim || !isfinite(eps) || !(eps > 0.0f)) return DORA_ERR_INVALID_ARG;
  if (d_out == 0) return DORA_OK;
  if (m == nullptr || wnorm == nullptr || g == nullptr) return DORA_ERR_INVALID_ARG;
  if (!aligned(m, 4) || !aligned(wnorm, 4) || !aligned(g, 4)) return DORA_ERR_INVALID_ARG;
  const int64_t nV = d_out * 4;
  if (g != m && overlap(g, nV, m, nV)) return DORA_ERR_INVALID_ARG;
  if (g != wnorm && overlap(g, nV, wnorm, nV)) return DORA_ERR_INVALID_ARG;
  return hip_status(dora::launch_magnitude(m, wnorm, eps, d_out, g, static_cast<hipStream_t>(stream)));
}

dora_status dora_compose(const void* base, const void* lora, const float* g, float s, int dtype, int64_t T,
                         int64_t d_out, void* out, void* stream) {
  if (!valid_dtype(dtype)) return DORA_ERR_UNSUPPORTED_DTYPE;
  if (T < 0 || d_out < 0 || T >= kMaxDim * 64 || d_out >= kMaxDim || !isfinite(s)) return DORA_ERR_INVALID_ARG;
  if (T == 0 || d_out == 0) return DORA_OK;
  if (base == nullptr || lora == nullptr || g == nullptr || out == nullptr) return DORA_ERR_INVALID_ARG;
  const int64_t es = esize(dtype);
  if (!aligned(base, (size_t)es) || !aligned(lora, (size_t)es) || !aligned(out, (size_t)es) || !aligned(g, 4))
    return DORA_ERR_INVALID_ARG;
  const int64_t nE = T * d_out * es;
  if (out != base && overlap(out, nE, base, nE)) return DORA_ERR_INVALID_ARG;
  if (out != lora && overlap(out, nE, lora, nE)) return DORA_ERR_INVALID_ARG;
  if (overlap(out, nE, g, d_out * 4)) return DORA_ERR_INVALID_ARG;
  const bool vec = (d_out % epc(dtype)) == 0 && aligned(base, 16) && aligned(lora, 16) && aligned(out, 16);
  return hip_status(
      dora::launch_compose(base, lora, g, s, dtype, T, d_out, out, vec, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
