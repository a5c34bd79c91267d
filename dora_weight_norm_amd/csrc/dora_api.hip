// C ABI of libdora: argument checks, the norm's work plan, and launches.
// Every check runs on the host before anything is enqueued; a failed check
// returns a status and touches no device state.
#include <math.h>
#include <string.h>

#include <atomic>
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

bool valid_dtype(int dt) { return dt == DORA_BF16 || dt == DORA_F32 || dt == DORA_F16; }
int64_t esize(int dt) { return dt == DORA_F32 ? 4 : 2; }
int64_t epc(int dt) { return dt == DORA_F32 ? 4 : 8; }

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

// Column tiling over r and the kernel configurations of both passes. Up to
// r = 256 the W pass takes all of r in one column tile (64, 128 or 256
// columns); above, tall matrices take 256 x 384 tiles (eight waves of
// 128 x 96 accumulators) up to r = 768 where they pad r no more than
// 192-column tiles do, and otherwise 256-row tiles of 192 or 256 columns
// (whichever pads r less). The column tiles of one row tile run on one die,
// so W is still read from HBM about once. 256-row tiles need fewer loads per MFMA
// than 128-row ones, but with r <= 256 they halve the workgroups per d_in
// range, so the d_in split goes twice as fine and each workgroup gets half
// the stages. Their saving outweighs the fixed cost of the shorter ranges
// only when there are at least kTallMinRowTiles row tiles (so that 8
// ranges fill the chip) and d_in is at least kTallMinDepth (so that even
// 16 ranges leave each workgroup 8 stages of 64); otherwise 128-row tiles
// are kept. The Gram pass uses narrower tiles so that its few rows still
// spread over many workgroups.
constexpr int64_t kTallMinRowTiles = dora::kGrid / 8;
constexpr int64_t kTallMinDepth = 8192;
void choose_tiles(NormPlan& p) {
  const int64_t r = p.r;
  if (p.dtype == DORA_F32) {
    if (r <= 32) {
      p.ntc = 32, p.fcfg = dora::kFastF32, p.gcfg = dora::kGenF32;
    } else {
      p.ntc = 128, p.fcfg = dora::kFastF128, p.gcfg = dora::kGenF128;
    }
    p.ntc_g = p.ntc, p.fcfg_g = p.fcfg, p.gcfg_g = p.gcfg;
    p.gran = 32;
  } else {
    const bool tall = ceil_div(p.d_out, 256) >= kTallMinRowTiles && p.d_in >= kTallMinDepth;
    if (r <= 64) {
      p.ntc = 64, p.fcfg = tall ? dora::kFastT64 : dora::kFastB64, p.gcfg = dora::kGenB64;
    } else if (r <= 128) {
      p.ntc = 128, p.fcfg = tall ? dora::kFastT128 : dora::kFastB128, p.gcfg = dora::kGenB128;
    } else if (r <= 256) {
      p.ntc = 256, p.fcfg = tall ? dora::kFastT256 : dora::kFastB256, p.gcfg = dora::kGenB256;
    } else if (tall && (r <= 384 || (r <= 768 && ceil_div(r, 384) * 384 <= ceil_div(r, 192) * 192))) {
      p.ntc = 384, p.fcfg = dora::kFastT384, p.gcfg = dora::kGenT192;
    } else if (r <= 384 || ceil_div(r, 192) * 192 <= ceil_div(r, 256) * 256) {
      p.ntc = 192, p.fcfg = dora::kFastT192, p.gcfg = dora::kGenT192;
    } else {
      p.ntc = 256, p.fcfg = dora::kFastT256, p.gcfg = dora::kGenB256;
    }
    // Gram pass: square tiles of 64 where their upper triangle times 8 d_in
    // ranges fits the chip (r <= 384): with half the rows per tile each
    // workgroup loads half as much, against 128-row tiles (measured: 70.2
    // against 68.6 us for the norm call at 8192 x 8192, r = 384; slower at
    // r = 768, where 64-row tiles make 78 of them). Their column count is
    // kept a multiple of 128, the general kernel's tile (which runs the Gram
    // pass when the inputs do not allow 16-byte loads).
    if (p.ntc == 64) {
      p.ntc_g = 64, p.fcfg_g = dora::kFastB64, p.gcfg_g = dora::kGenB64;
    } else if (dora::tri_count(2 * ceil_div(r, 128)) * 8 <= dora::kGrid) {
      p.ntc_g = 64, p.fcfg_g = dora::kFastG64, p.gcfg_g = dora::kGenB128;
    } else {
      p.ntc_g = 128, p.fcfg_g = dora::kFastB128, p.gcfg_g = dora::kGenB128;
    }
    p.gran = 64;
  }
  p.ntc_gen = p.fcfg == dora::kFastT384 ? 192 : p.ntc;
  p.n_nt = (int)ceil_div(r, p.ntc);
  p.n_nt_g = p.fcfg_g == dora::kFastG64 ? (int)(2 * ceil_div(r, 128)) : (int)ceil_div(r, p.ntc_g);
}

// Column tiles of the W pass on either kernel: the cross partials are laid
// out for the larger count.
int64_t cross_tiles(const NormPlan& p) {
  const int64_t gen = ceil_div(p.r, p.ntc_gen);
  return p.n_nt > gen ? p.n_nt : gen;
}

// Gram partial planes the workspace holds: the Gram pass writes xg, the W
// pass with the Gram blocks folded in writes xw.
int gram_planes(const NormPlan& p) { return p.gfold && p.xw > p.xg ? p.xw : p.xg; }

// Gram-term partial planes: n_bt from the streaming kernel, n_cb from the
// general one.
int64_t ba_planes(const NormPlan& p) { return p.n_bt > p.n_cb ? p.n_bt : p.n_cb; }

void layout(NormPlan& p) {
  size_t off = 0;
  p.off_base = off;
  off = align_up(off + (size_t)((int64_t)p.xw * p.ld_w) * 4, kAlign);
  p.off_cross = off;
  off = align_up(off + (size_t)((int64_t)p.xw * cross_tiles(p) * p.ld_w) * 4, kAlign);
  p.off_ba = off;
  off = align_up(off + (size_t)(ba_planes(p) * p.ld_w) * 4, kAlign);
  p.off_g = off;
  off = align_up(off + (size_t)((int64_t)gram_planes(p) * p.ga_rows * p.ga_cols) * 4, kAlign);
  p.off_gg = off;
  off = align_up(off + (size_t)(p.rg * p.rg) * 4, kAlign);   // bf16 hi and lo, or fp32
  p.off_bf = off;
  // fp16: B widened to fp32 [d_out][r] (separate Gram-term pass), or B
  // split into bf16 [d_out][B_hi | B_lo], rg columns each (Gram term in
  // the W pass); the region holds the larger.
  if (p.dtype == DORA_F16) off = align_up(off + (size_t)(p.d_out * p.rg) * 4, kAlign);
  p.off_cnt = off;
  off = align_up(off + (size_t)ceil_div(p.d_out, dora::fast_rows(p.fcfg)) * 4, kAlign);   // arrival counters
  p.ws_bytes = off;
}

dora_status check_sizes(int64_t d_out, int64_t d_in, int64_t r) {
  if (d_out < 0 || d_in < 0 || r < 0) return DORA_ERR_INVALID_ARG;
  if (d_out >= kMaxDim || d_in >= kMaxDim || r >= kMaxRank) return DORA_ERR_INVALID_ARG;
  return DORA_OK;
}

// d_in ranges of the W pass: the power of two (<= 32 and <= the granule
// count) whose grid fills whole rounds of kGrid workgroups best; ties go to
// fewer ranges (fewer partials).
int choose_w_ranges(int64_t tiles, int64_t n_gran) {
  int best = 1;
  double best_eff = -1.0;
  for (int X = 1; X <= 32 && X <= n_gran; X *= 2) {
    const int64_t wg = tiles * X;
    const int64_t rounds = (wg + dora::kGrid - 1) / dora::kGrid;
    const double eff = (double)wg / (double)(rounds * dora::kGrid);
    if (eff > best_eff + 1e-9) {
      best_eff = eff;
      best = X;
    }
  }
  return best;
}

// d_in ranges of the Gram pass: the largest power of two (<= max_x and <=
// the granule count) that keeps the grid within kGrid workgroups and the written
// partial Gram matrices (what the reduction reads) within kGramPartialCap
// bytes.
constexpr int64_t kGramPartialCap = (int64_t)16 << 20;
int choose_g_ranges(int64_t tiles, int64_t n_gran, int64_t plane_bytes, int max_x) {
  int X = 1;
  while (X * 2 <= max_x && X * 2 <= n_gran && tiles * X * 2 <= dora::kGrid &&
         plane_bytes * X * 2 <= kGramPartialCap)
    X *= 2;
  return X;
}

// Dense mode (see NormMode): 16-bit inputs where B A costs less than the
// factored terms, d_in and r in whole 16-byte chunks, and every dense
// operand within a 32-bit buffer descriptor (A whole, 64 rows of W or of
// B). B A costs d_out d_in r multiply-adds: less than G = A A^T (r^2 d_in)
// when r >= d_out, and less than the Gram term B G (d_out r^2) when
// r > d_in. The first rule applies at every size, the second up to 4096
// rows, where the dense pass measured faster (taller matrices keep the W
// pass, whose tiles reuse their operands more). Its partials share the
// workspace with the factored layout, which stays valid as the fallback;
// the workspace is the larger of the two.
constexpr int64_t kDenseMaxRowsRankAboveDin = 4096;
void plan_dense(NormPlan& p, size_t budget) {
  if (p.mode != dora::kModeFactored || (p.dtype != DORA_BF16 && p.dtype != DORA_F16)) return;
  const bool cheaper = p.r >= p.d_out || (p.r > p.d_in && p.d_out <= kDenseMaxRowsRankAboveDin);
  if (!cheaper || p.d_in % 8 != 0 || p.r % 8 != 0) return;
  const uint64_t lim = 1ull << 31;
  if ((uint64_t)p.r * (uint64_t)p.d_in * 2u >= lim || (uint64_t)dora::kDenseRows * (uint64_t)p.d_in * 2u >= lim ||
      (uint64_t)dora::kDenseRows * (uint64_t)p.r * 2u >= lim)
    return;
  const int64_t n_rt = ceil_div(p.d_out, dora::kDenseRows), n_ct = ceil_div(p.d_in, dora::kDenseCols);
  const int64_t grid = n_rt * ceil_div(n_ct, dora::kDies) * dora::kDies;
  if (grid >= lim) return;
  const int64_t ld = ceil_div(p.d_out, 64) * 64;
  const size_t bytes = (size_t)(ceil_div(n_ct * ld * 4, (int64_t)kAlign) * (int64_t)kAlign);
  const size_t ws = bytes > p.ws_bytes ? bytes : p.ws_bytes;
  if (ws > budget) return;
  p.mode = dora::kModeDense;
  p.dn_rt = (int)n_rt;
  p.dn_ct = (int)n_ct;
  p.ld_d = ld;
  p.off_dense = 0;
  p.ws_bytes = ws;
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
  choose_tiles(p);
  p.n_gran = ceil_div(d_in, p.gran);
  p.ld_w = ceil_div(d_out, dora::kRowPadW) * dora::kRowPadW;
  p.ga_rows = ceil_div(r, dora::kRowPadG) * dora::kRowPadG;
  p.ga_cols = (int64_t)p.n_nt_g * p.ntc_g;
  const int64_t rq = dtype == DORA_F32 ? 32 : 64;   // (16-bit: the Gram term's parts meet on 64-deep stages)
  p.rg = ceil_div(r, rq) * rq;
  // Tiles of the separate Gram-term pass (run when the Gram term is not
  // inside the W pass: G folded into the W pass, the general path): the
  // streaming kernel covers up to 384 columns of G in one tile (bf16; 128
  // for fp32, and for fp16, whose separate Gram term runs in fp32) and uses
  // 256-column tiles beyond; the general kernel uses kGramCols.
  if (dtype == DORA_BF16) {
    p.bcfg = p.rg <= 384 ? (int)ceil_div(p.rg, 128) : 2;
  } else {
    p.bcfg = 1;
  }
  p.n_bt = (int)ceil_div(p.rg, 128 * (int64_t)p.bcfg);
  p.n_cb = (int)ceil_div(p.rg, dora::kGramCols);

  const int64_t tiles_w = ceil_div(d_out, dora::fast_rows(p.fcfg)) * p.n_nt;
  // G = A A^T folds into the streaming W pass when one column tile of at
  // most 128 columns holds all of A's rows and every 32x32 block of G finds
  // a wave (one per wave). Every wave then reads two more fragments and runs
  // one more MFMA per K16 step; on wider tiles those LDS reads cost the W
  // pass as much as the separate Gram pass takes.
  const int64_t nbc = p.rg / 32;
  p.gfold = p.n_nt == 1 && p.ntc <= 128 &&
            nbc * nbc <= (int64_t)dora::fast_waves(p.fcfg) * ceil_div(d_out, dora::fast_rows(p.fcfg));
  // The 128 x 128 and 64 x 64 Gram tiles are square, so only those on and
  // above the diagonal are computed (the reduction reads the rest
  // transposed); with a third less work per range, the Gram pass can split
  // d_in further.
  p.gsym = p.fcfg_g == dora::kFastB128 || p.fcfg_g == dora::kFastG64;
  const int64_t ntg = p.n_nt_g;
  const int64_t tiles_g = p.gsym ? dora::tri_count(ntg) : ceil_div(r, dora::fast_rows(p.fcfg_g)) * p.n_nt_g;
  const int64_t plane = p.ga_rows * p.ga_cols * 4;
  const int64_t written = p.gsym ? plane * dora::tri_count(ntg) / (ntg * ntg) : plane;
  int xw = choose_w_ranges(tiles_w, p.n_gran);
  // Square tiles: at most 16 ranges, so the reduction sums each element's
  // partials in one round trip of loads.
  int xg = choose_g_ranges(tiles_g, p.n_gran, written, p.gsym ? 16 : 64);
  // Fit the budget: fewer Gram ranges first, then fewer W ranges.
  for (;;) {
    p.xw = xw;
    p.xg = xg;
    layout(p);
    if (p.ws_bytes <= budget) {
      // The W pass that carries the Gram term runs in the die grid of two
      // range groups where its grid allows (B's rows, which its epilogue
      // reads, then leave memory for two dies instead of one per range).
      // A grid of several rounds takes four range groups where they fit:
      // between rounds each die's L2 sees its share of W go through and
      // loses A, so every round fetches the die's ranges of A again, and
      // four groups give each die half as many ranges as two do, halving
      // those bytes (B's rows then leave memory for four dies instead of
      // two). With G folded in, the plain order was faster.
      const int64_t n_mt = ceil_div(d_out, dora::fast_rows(p.fcfg));
      const bool rounds = (int64_t)p.xw * n_mt * p.n_nt > dora::kGrid;
      if (p.gfold) {
        p.die_groups = 0;
      } else if (rounds && dora::die_grid_fits(4, p.xw, n_mt, p.n_nt)) {
        p.die_groups = 4;
      } else {
        p.die_groups = dora::die_grid_fits(2, p.xw, n_mt, p.n_nt) ? 2 : 0;
      }
      plan_dense(p, budget);
      *out = p;
      return DORA_OK;
    }
    if (xg > 1) {
      xg /= 2;
    } else if (xw > 1) {
      xw /= 2;
    } else {
      return DORA_ERR_BUDGET;
    }
  }
}

// Host replay of the plan: the ranges tile d_in exactly and are non-empty,
// every grid fits, and every partial the kernels write lies inside its
// workspace region.
bool plan_self_check(const NormPlan& p) {
  if (p.mode != dora::kModeFactored && p.mode != dora::kModeDense) return true;
  if (p.mode == dora::kModeDense) {
    // Dense tiles cover d_out and d_in; the partials fit the workspace.
    if (p.dn_rt < 1 || p.dn_ct < 1 || (int64_t)p.dn_rt * dora::kDenseRows < p.d_out ||
        (int64_t)p.dn_ct * dora::kDenseCols < p.d_in || p.ld_d < p.d_out ||
        p.ws_bytes < p.off_dense + (size_t)((int64_t)p.dn_ct * p.ld_d) * 4)
      return false;
  }
  for (int pass = 0; pass < 2; ++pass) {
    const int X = pass ? p.xg : p.xw;
    if (X < 1 || X > p.n_gran) return false;
    if (dora::range_k0(p, X, 0) != 0 || dora::range_k0(p, X, X) != p.d_in) return false;
    for (int x = 0; x < X; ++x)
      if (dora::range_k0(p, X, x + 1) <= dora::range_k0(p, X, x)) return false;
  }
  // Row tiles of every kernel: no tile has fewer than 64 rows, and a plan's
  // general-kernel tile is never taller than its streaming tile (256 rows
  // only with a 256-row streaming tile), so these bounds cover both.
  const int64_t rows_w = ceil_div(p.d_out, 64) * 64, rows_g = ceil_div(p.r, 64) * 64;
  const int fw = dora::fast_rows(p.fcfg), fg = dora::fast_rows(p.fcfg_g);
  if (ceil_div(p.d_out, fw) * fw > p.ld_w || rows_w > p.ld_w) return false;
  if (ceil_div(p.r, fg) * fg > p.ga_rows || rows_g > p.ga_rows) return false;
  if ((int64_t)p.n_nt * p.ntc < p.r || p.ga_cols < p.r || p.rg > p.ga_cols) return false;
  const int64_t grid_w = p.xw * ceil_div(p.d_out, 64) * p.n_nt;
  const int64_t grid_g = p.xg * ceil_div(p.r, 64) * p.n_nt_g;
  if (grid_w >= ((int64_t)1 << 31) || grid_g >= ((int64_t)1 << 31)) return false;
  if (p.die_groups != 0 && !dora::die_grid_fits(p.die_groups, p.xw, ceil_div(p.d_out, fw), p.n_nt)) return false;
  if (p.off_cross < p.off_base + (size_t)(p.xw * p.ld_w) * 4) return false;
  if (p.off_ba < p.off_cross + (size_t)(p.xw * p.n_nt * p.ld_w) * 4) return false;
  if (p.off_g < p.off_ba + (size_t)(ba_planes(p) * p.ld_w) * 4) return false;
  if (p.off_gg < p.off_g + (size_t)((int64_t)gram_planes(p) * p.ga_rows * p.ga_cols) * 4) return false;
  if (p.off_bf < p.off_gg + (size_t)(p.rg * p.rg) * 4) return false;
  if (p.off_cnt < p.off_bf + (p.dtype == DORA_F16 ? (size_t)(p.d_out * p.rg) * 4 : 0)) return false;
  return p.ws_bytes >= p.off_cnt + (size_t)ceil_div(p.d_out, fw) * 4;
}

// Host replay of the streaming W pass's workgroup order (w_tile): every
// (range, row tile, column tile) exactly once. O(grid) time and memory, so
// only for plan queries, on grids of up to 2^22 workgroups.
bool w_order_covers_grid(const NormPlan& p) {
  if (p.mode != dora::kModeFactored && p.mode != dora::kModeDense) return true;
  const int64_t n_mt = ceil_div(p.d_out, dora::fast_rows(p.fcfg)), grid = (int64_t)p.xw * n_mt * p.n_nt;
  if (grid > ((int64_t)1 << 22)) return true;
  std::vector<bool> seen((size_t)grid, false);
  for (int64_t b = 0; b < grid; ++b) {
    int x, n;
    int64_t m;
    dora::w_tile(b, p.xw, n_mt, p.n_nt, p.die_groups, &x, &m, &n);
    if (x < 0 || x >= p.xw || m < 0 || m >= n_mt || n < 0 || n >= p.n_nt) return false;
    const size_t id = (size_t)((m * p.n_nt + n) * p.xw + x);
    if (seen[id]) return false;
    seen[id] = true;
  }
  return true;
}

// The streaming kernel addresses every operand tile through a buffer
// descriptor with 32-bit byte offsets, and marks masked loads with the
// offset 2^31 (past every descriptor's range). So each descriptor must span
// less than 2^31 bytes: the tallest row tile of W or A (the W pass's tile
// rows, its column tile over A's rows, and the Gram pass's square tiles) by
// d_in, and the Gram-term operands (B's rows by r, the stored Gram matrix's
// rows by its width).
bool offsets_fit_32(const NormPlan& p) {
  if (p.mode != dora::kModeFactored && p.mode != dora::kModeDense) return true;
  const uint64_t es = (uint64_t)esize(p.dtype);
  uint64_t rows = (uint64_t)dora::fast_rows(p.fcfg);
  const uint64_t others[] = {(uint64_t)p.ntc, (uint64_t)dora::fast_rows(p.fcfg_g), (uint64_t)p.ntc_g};
  for (uint64_t o : others) rows = o > rows ? o : rows;
  const uint64_t tile_span = rows * (uint64_t)p.d_in * es;
  const uint64_t b_span = rows * (uint64_t)p.r * es;
  const uint64_t g_span = rows * 2ull * (uint64_t)p.rg * es;
  return tile_span < (1ull << 31) && b_span < (1ull << 31) && g_span < (1ull << 31);
}

dora_status hip_status(hipError_t e) { return e == hipSuccess ? DORA_OK : DORA_ERR_HIP; }

dora_status compose_checked(const void* base, const void* lora, const float* g, float s, int dtype, int64_t T,
                            int64_t d_out, void* out, bool add_base, void* stream) {
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
  return hip_status(dora::launch_compose(base, lora, g, s, dtype, T, d_out, out, vec, add_base,
                                         static_cast<hipStream_t>(stream)));
}

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
  if (!plan_self_check(p) || !w_order_covers_grid(p)) return DORA_ERR_INVALID_ARG;
  const bool f = p.mode == dora::kModeFactored || p.mode == dora::kModeDense;   // (dense: its fallback)
  const int64_t grid_w = f ? p.xw * ceil_div(p.d_out, dora::fast_rows(p.fcfg)) * p.n_nt : 0;
  const int64_t grid_g = !f ? 0
                             : p.xg * (p.gsym ? dora::tri_count(p.n_nt_g)
                                              : ceil_div(p.r, dora::fast_rows(p.fcfg_g)) * p.n_nt_g);
  const int64_t vals[] = {p.mode, p.ntc, p.n_nt, p.ntc_g, p.n_nt_g, p.fcfg, p.gcfg, p.fcfg_g, p.gcfg_g, p.gran,
                          p.n_gran, p.xw, p.xg, (int64_t)p.ws_bytes, grid_w, grid_g,
                          f ? (int64_t)dora::fast_kernel_lds_bytes(p.fcfg) : 0, f ? dora::fast_rows(p.fcfg) : 0,
                          f ? p.gfold : 0, f ? p.gsym : 0, f ? (int64_t)(!p.gfold) : 0,
                          f ? (p.mode == dora::kModeDense || p.gfold ? 0 : 2) : 0, f ? (int64_t)offsets_fit_32(p) : 1,
                          p.mode == dora::kModeDense ? p.dn_rt : 0, p.mode == dora::kModeDense ? p.dn_ct : 0,
                          f ? p.die_groups : 0};
  const int nv = (int)(sizeof(vals) / sizeof(vals[0]));
  for (int i = 0; i < n_info && i < nv; ++i) info[i] = vals[i];
  for (int i = nv; i < n_info; ++i) info[i] = -1;
  return DORA_OK;
}

}  // extern "C"

namespace {

// Scratch memory of dora_factored_norm_noalloc: the norm's workspace for
// callers that cannot allocate. Each GPU the library runs on holds its own
// copy, at its own address, until the process ends. On the host this name
// is only a stand-in for the symbol; host code uses the device address
// that hipGetSymbolAddress returns, looked up once per device below.
static __device__ __align__(256) char scratch[DORA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
// Device address of `scratch` on each GPU, set by the first no-alloc call
// on that GPU and never changed afterwards (concurrent first calls store
// the same value).
std::atomic<void*> g_scratch_addr[kMaxDevices];

// The device address of `scratch` on the GPU that `stream` belongs to (the
// current GPU for the null stream), looked up with that GPU current.
dora_status scratch_address(hipStream_t stream, void** out) {
  int dev = -1;
  if (stream != nullptr) {
    hipDevice_t d = -1;
    if (hipStreamGetDevice(stream, &d) != hipSuccess) return DORA_ERR_HIP;
    dev = d;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return DORA_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return DORA_ERR_HIP;
  void* ptr = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return DORA_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return DORA_ERR_HIP;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return DORA_ERR_HIP;
    if (e != hipSuccess || ptr == nullptr) return DORA_ERR_HIP;
    g_scratch_addr[dev].store(ptr, std::memory_order_release);
  }
  *out = ptr;
  return DORA_OK;
}

// The factored norm behind every norm entry point. With use_scratch the
// workspace is this GPU's `scratch` (workspace and workspace_bytes are
// ignored), looked up after every argument check has passed.
dora_status factored_norm(const void* W, const void* A, const void* B, int dtype, int64_t d_out, int64_t d_in,
                          int64_t r, float s, size_t budget_bytes, void* workspace, size_t workspace_bytes,
                          float* wnorm, const float* m, float eps, float* g, void* stream, const hipEvent_t* events,
                          int n_events, bool use_scratch = false) {
  if (use_scratch) {
    workspace = nullptr;
    workspace_bytes = DORA_NOALLOC_SCRATCH_BYTES;
    if (budget_bytes > DORA_NOALLOC_SCRATCH_BYTES) budget_bytes = DORA_NOALLOC_SCRATCH_BYTES;
  }
  if (!valid_dtype(dtype)) return DORA_ERR_UNSUPPORTED_DTYPE;
  dora_status st = check_sizes(d_out, d_in, r);
  if (st != DORA_OK) return st;
  if (!isfinite(s)) return DORA_ERR_INVALID_ARG;
  if (m != nullptr && (!isfinite(eps) || !(eps > 0.0f))) return DORA_ERR_INVALID_ARG;
  NormPlan p;
  st = make_plan(d_out, d_in, r, dtype, s, budget_bytes, &p);
  if (st != DORA_OK) return st;
  if (p.mode == dora::kModeEmpty) return DORA_OK;
  if (!plan_self_check(p)) return DORA_ERR_INVALID_ARG;

  const int64_t es = esize(dtype);
  const int64_t nW = d_out * d_in * es, nA = r * d_in * es, nB = d_out * r * es, nV = d_out * 4;
  const bool factored = p.mode == dora::kModeFactored || p.mode == dora::kModeDense;   // (A and B are read)
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
    return hip_status(
        dora::launch_norm_rowonly(W, dtype, d_out, d_in, vec, m, eps, wnorm, gout ? g : nullptr, hs, events, n_events));
  }
  if (use_scratch && p.ws_bytes > 0) {
    // (`scratch` is its own allocation: it overlaps no caller buffer.)
    st = scratch_address(hs, &workspace);
    if (st != DORA_OK) return st;
  }
  if (workspace_bytes < p.ws_bytes) return DORA_ERR_WORKSPACE;
  if (p.ws_bytes > 0 && (workspace == nullptr || !aligned(workspace, kAlign))) return DORA_ERR_WORKSPACE;
  if (p.mode == dora::kModeDense) {
    if (aligned(W, 16) && aligned(A, 16) && aligned(B, 16))
      return hip_status(dora::launch_norm_dense(p, W, A, B, workspace, s, m, eps, wnorm, g, hs, events, n_events));
    p.mode = dora::kModeFactored;   // the 16-byte loads need aligned rows: the factored path, same workspace
  }
  p.vec_b = aligned(B, 16) && (r % epc(dtype)) == 0;
  p.fast = aligned(W, 16) && aligned(A, 16) && (d_in % epc(dtype)) == 0 && p.vec_b && offsets_fit_32(p);
  if (!p.fast && p.ntc != p.ntc_gen) {
    // The general kernel's own column tiling (the layout holds its partials).
    p.ntc = p.ntc_gen;
    p.n_nt = (int)ceil_div(r, p.ntc);
    if (!plan_self_check(p)) return DORA_ERR_INVALID_ARG;
  }
  return hip_status(dora::launch_norm_factored(p, W, A, B, workspace, s, m, eps, wnorm, g, hs, events, n_events));
}

}  // namespace

extern "C" {

dora_status dora_factored_norm(const void* W, const void* A, const void* B, int dtype, int64_t d_out,
                               int64_t d_in, int64_t r, float s, size_t budget_bytes, void* workspace,
                               size_t workspace_bytes, float* wnorm, const float* m, float eps, float* g,
                               void* stream) {
  return factored_norm(W, A, B, dtype, d_out, d_in, r, s, budget_bytes, workspace, workspace_bytes, wnorm, m, eps,
                       g, stream, nullptr, 0);
}

dora_status dora_factored_norm_noalloc(const void* W, const void* A, const void* B, int dtype, int64_t d_out,
                                       int64_t d_in, int64_t r, float s, size_t budget_bytes, float* wnorm,
                                       const float* m, float eps, float* g, void* stream) {
  return factored_norm(W, A, B, dtype, d_out, d_in, r, s, budget_bytes, nullptr, 0, wnorm, m, eps, g, stream, nullptr,
                       0, true);
}

dora_status dora_factored_norm_marked(const void* W, const void* A, const void* B, int dtype, int64_t d_out,
                                      int64_t d_in, int64_t r, float s, size_t budget_bytes, void* workspace,
                                      size_t workspace_bytes, float* wnorm, const float* m, float eps, float* g,
                                      void* stream, void* const* events, int n_events) {
  if (n_events < 0 || (n_events > 0 && events == nullptr)) return DORA_ERR_INVALID_ARG;
  return factored_norm(W, A, B, dtype, d_out, d_in, r, s, budget_bytes, workspace, workspace_bytes, wnorm, m, eps,
                       g, stream, reinterpret_cast<const hipEvent_t*>(events),
                       n_events < dora::kMaxLaunchEvents ? n_events : dora::kMaxLaunchEvents);
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

dora_status dora_norm_to_dtype(const float* wnorm, int64_t n, int dtype, void* out, void* stream) {
  if (!valid_dtype(dtype)) return DORA_ERR_UNSUPPORTED_DTYPE;
  if (n < 0 || n >= kMaxDim) return DORA_ERR_INVALID_ARG;
  if (n == 0) return DORA_OK;
  const int64_t es = esize(dtype);
  if (wnorm == nullptr || out == nullptr || !aligned(wnorm, 4) || !aligned(out, (size_t)es))
    return DORA_ERR_INVALID_ARG;
  if (overlap(out, n * es, wnorm, n * 4)) return DORA_ERR_INVALID_ARG;
  return hip_status(dora::launch_cast(wnorm, n, dtype, out, static_cast<hipStream_t>(stream)));
}

dora_status dora_compose(const void* base, const void* lora, const float* g, float s, int dtype, int64_t T,
                         int64_t d_out, void* out, void* stream) {
  return compose_checked(base, lora, g, s, dtype, T, d_out, out, false, stream);
}

dora_status dora_layer_output(const void* base, const void* lora, const float* g, float s, int dtype, int64_t T,
                              int64_t d_out, void* y, void* stream) {
  return compose_checked(base, lora, g, s, dtype, T, d_out, y, true, stream);
}

dora_status dora_compose_backward_workspace_size(int64_t T, int64_t d_out, size_t* ws_bytes) {
  if (ws_bytes == nullptr || T < 0 || d_out < 0 || T >= kMaxDim * 64 || d_out >= kMaxDim) return DORA_ERR_INVALID_ARG;
  *ws_bytes = dora::compose_bwd_workspace_bytes(T, d_out);
  return DORA_OK;
}

dora_status dora_compose_backward(const void* dy, const void* base, const void* lora, const float* g, float s,
                                  int dtype, int64_t T, int64_t d_out, void* d_base, void* d_lora, float* dg,
                                  const float* wnorm, float eps, float* dm, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  if (!valid_dtype(dtype)) return DORA_ERR_UNSUPPORTED_DTYPE;
  if (T < 0 || d_out < 0 || T >= kMaxDim * 64 || d_out >= kMaxDim || !isfinite(s)) return DORA_ERR_INVALID_ARG;
  if (dm != nullptr && (dg == nullptr || wnorm == nullptr || !isfinite(eps) || !(eps > 0.0f)))
    return DORA_ERR_INVALID_ARG;
  if (d_out == 0) return DORA_OK;
  const bool need_rows = T > 0 && (d_base != nullptr || d_lora != nullptr || dg != nullptr);
  if (g == nullptr || !aligned(g, 4)) return DORA_ERR_INVALID_ARG;
  if (need_rows && dy == nullptr) return DORA_ERR_INVALID_ARG;
  if (dg != nullptr && T > 0 && (base == nullptr || lora == nullptr)) return DORA_ERR_INVALID_ARG;
  const int64_t es = esize(dtype);
  const void* elems[] = {dy, dg ? base : nullptr, dg ? lora : nullptr, d_base, d_lora};
  for (const void* p : elems)
    if (p != nullptr && !aligned(p, (size_t)es)) return DORA_ERR_INVALID_ARG;
  if (!aligned(dg, 4) || !aligned(dm, 4) || !aligned(wnorm, 4)) return DORA_ERR_INVALID_ARG;
  // Outputs overlap no input and no other output.
  const int64_t nE = T * d_out * es, nV = d_out * 4;
  const void* ins[] = {dy, dg ? base : nullptr, dg ? lora : nullptr, g, wnorm};
  const int64_t nin[] = {nE, nE, nE, nV, nV};
  const void* outs[] = {d_base, d_lora, dg, dm};
  const int64_t nout[] = {nE, nE, nV, nV};
  for (int o = 0; o < 4; ++o) {
    for (int i = 0; i < 5; ++i)
      if (overlap(outs[o], nout[o], ins[i], nin[i])) return DORA_ERR_INVALID_ARG;
    for (int o2 = o + 1; o2 < 4; ++o2)
      if (overlap(outs[o], nout[o], outs[o2], nout[o2])) return DORA_ERR_INVALID_ARG;
  }
  const size_t need = dora::compose_bwd_workspace_bytes(T, d_out);
  if (dg != nullptr && need > 0) {
    if (workspace_bytes < need) return DORA_ERR_WORKSPACE;
    if (workspace == nullptr || !aligned(workspace, kAlign)) return DORA_ERR_WORKSPACE;
    for (int o = 0; o < 4; ++o)
      if (overlap(workspace, (int64_t)need, outs[o], nout[o])) return DORA_ERR_INVALID_ARG;
    for (int i = 0; i < 5; ++i)
      if (overlap(workspace, (int64_t)need, ins[i], nin[i])) return DORA_ERR_INVALID_ARG;
  }
  if (!need_rows && dg == nullptr) return DORA_OK;
  bool vec = (d_out % epc(dtype)) == 0;
  for (const void* p : elems)
    if (p != nullptr && !aligned(p, 16)) vec = false;
  return hip_status(dora::launch_compose_bwd(dy, base, lora, g, s, dtype, T, d_out, d_base, d_lora, dg, wnorm, eps,
                                             dm, workspace, vec, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
