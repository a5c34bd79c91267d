// Work plan of the factored row norm: column tiling over r, the split of
// d_in into ranges (one set of partial sums per range), the kernel
// configurations and the workspace layout. Shared by the host planner and
// the kernels so both derive ranges from the same integer formulas.
#pragma once

#include <stddef.h>
#include <stdint.h>

#if defined(__HIPCC__)
#define DORA_HD __host__ __device__ __forceinline__
#else
#define DORA_HD inline
#endif

namespace dora {

// MI355X: 256 compute units in 8 dies (XCDs) of 32. Workgroup b of a launch
// is placed on die b % 8, so workgroups b, b+8, b+16, ... share one die's L2.
constexpr int kDies = 8;
constexpr int kGrid = 256;           // compute units
constexpr int kThreads = 256;        // 4 waves of 64
constexpr int kRowPadW = 256;        // W-pass partial rows (ld_w) are padded to a multiple of this
constexpr int kRowPadG = 128;        // Gram partial rows (ga_rows) are padded to a multiple of this

// Streaming kernel configurations. Each holds MT rows (of W, or of A in the
// Gram pass) by NTC columns (rows of A) per workgroup; the column operand
// and the row operand go through a ring of LDS slots by direct loads.
enum FastCfg : int {
  kFastB64 = 0,    // bf16, 128 x 64, 8 waves
  kFastB128 = 1,   // bf16, 128 x 128, 8 waves
  kFastB256 = 2,   // bf16, 128 x 256, 8 waves
  kFastT192 = 3,   // bf16, 256 x 192, 8 waves
  kFastT256 = 4,   // bf16, 256 x 256, 8 waves
  kFastF32 = 5,    // fp32, 128 x 32, 4 waves
  kFastF128 = 6,   // fp32, 128 x 128, 8 waves
  kFastT64 = 7,    // bf16, 256 x 64, 8 waves
  kFastT128 = 8,   // bf16, 256 x 128, 8 waves
  kFastT384 = 9,   // bf16, 256 x 384, 8 waves of 128 x 96 (lean register mode)
  kFastG64 = 10,   // bf16, 64 x 64, 4 waves (Gram pass, square tiles)
};
// Rows per workgroup tile, and waves per workgroup, of a streaming
// configuration.
DORA_HD int fast_rows(int cfg) {
  if (cfg == kFastG64) return 64;
  return cfg == kFastT64 || cfg == kFastT128 || cfg == kFastT192 || cfg == kFastT256 || cfg == kFastT384 ? 256
                                                                                                       : 128;
}
DORA_HD int fast_waves(int cfg) { return cfg == kFastF32 || cfg == kFastG64 ? 4 : 8; }
constexpr int kGramCols = 64;      // columns of G per Gram-term tile (general kernel)

// Number of tiles on and above the diagonal of an nt x nt tile grid, and
// the (row, column) tile of upper-triangle tile t in row-major order.
DORA_HD int64_t tri_count(int64_t nt) { return nt * (nt + 1) / 2; }
DORA_HD void tri_tile(int t, int nt, int* m, int* n) {
  int row = 0;
  while (t >= nt - row) {
    t -= nt - row;
    ++row;
  }
  *m = row;
  *n = row + t;
}

// General kernel (any alignment): WM x WN waves, each owning MB x NB blocks
// of 32x32 accumulators; KT is the d_in depth of one LDS stage.
struct TileShape {
  int wm, wn, mb, nb, kt;
};
enum TileCfg : int {
  kGenB64 = 0,    // bf16, 128 x 64 tiles
  kGenB128 = 1,   // bf16, 128 x 128
  kGenB256 = 2,   // bf16, 128 x 256
  kGenT192 = 3,   // bf16, 256 x 192
  kGenF32 = 5,    // fp32, 128 x 32
  kGenF128 = 6,   // fp32, 128 x 128
};
DORA_HD TileShape tile_shape(int cfg) {
  switch (cfg) {
    case kGenB64: return TileShape{2, 2, 2, 1, 64};
    case kGenB128: return TileShape{1, 4, 4, 1, 64};
    case kGenB256: return TileShape{1, 4, 4, 2, 64};
    case kGenT192: return TileShape{4, 2, 2, 3, 64};
    case kGenF32: return TileShape{4, 1, 1, 1, 32};
    default: return TileShape{1, 4, 4, 1, 32};
  }
}

// kModeDense: the dense fused pass over tiles of W + s B A (16-bit types,
// r >= d_out, or r > d_in with at most 4096 rows); the plan's factored
// fields stay valid, so a call whose pointers do not allow its 16-byte
// loads runs the factored path instead, in the same workspace.
enum NormMode : int { kModeEmpty = 0, kModeRowOnly = 1, kModeFactored = 2, kModeDense = 3 };
constexpr int kDenseRows = 64;     // rows of W per dense tile
constexpr int kDenseCols = 128;    // columns of W (d_in) per dense tile

struct NormPlan {
  int64_t d_out, d_in, r;
  int dtype;            // 0 = bf16, 1 = fp32, 2 = fp16
  int mode;             // NormMode
  int ntc;              // W pass: columns of one column tile (a multiple of 32)
  int ntc_gen;          // W pass: column tile width of the general kernel (the streaming
                        // 384-column tile falls back to 192-column general tiles)
  int n_nt;             // W pass: column tiles over r
  int fcfg;             // W pass: FastCfg used when the inputs allow 16-byte loads
  int gcfg;             // W pass: TileCfg used otherwise
  int ntc_g, n_nt_g;    // Gram pass: column tile width and count
  int fcfg_g, gcfg_g;   // Gram pass: kernel configurations
  int fast;             // set per call: 1 = streaming kernel, 0 = general kernel
  int vec_b;            // set per call: B rows allow aligned 16-byte loads
  int gran;             // d_in granule in elements: range boundaries are multiples of it
  int64_t n_gran;       // granules over d_in
  int xw;               // d_in ranges of the W pass
  int xg;               // d_in ranges of the Gram pass
  int gsym;             // the streaming Gram pass computes only the tiles on and above
                        // the diagonal (square kFastB128 or kFastG64 tiles; G is symmetric)
  int gfold;            // the streaming W pass also computes G (no Gram pass); its
                        // Gram partials are then per W-pass range (xw planes)
  int64_t ld_w;         // padded W rows of the base / cross partials
  int64_t ga_rows;      // padded A rows of the Gram partials
  int64_t ga_cols;      // padded Gram columns: n_nt * ntc
  int64_t rg;           // side of the reduced Gram matrix: r rounded up to 64 for the
                        // 16-bit types (their Gram term runs over a depth of several
                        // parts in 64-deep stages, so the seams between the parts must
                        // fall on stage boundaries), to 32 for fp32
  int bcfg;             // Gram-term pass (streaming kernel): 128-column blocks per tile (bf16)
  int n_bt;             // Gram-term column tiles of the streaming kernel
  int n_cb;             // Gram-term column tiles of the general kernel (kGramCols columns each)
  size_t off_base;      // [xw][ld_w] fp32 base partials
  size_t off_cross;     // [xw][n_nt][ld_w] fp32 cross partials
  size_t off_ba;        // [max(n_bt, n_cb)][ld_w] fp32 Gram-term partials
  size_t off_g;         // [max(xg, xw if gfold)][ga_rows][ga_cols] fp32 Gram partials
  size_t off_gg;        // reduced Gram matrix: bf16 [rg][Ghi | Glo], fp32 [rg][rg]
  size_t off_bf;        // fp16 inputs only: B widened to fp32 [d_out][r], or split to bf16 [d_out][B_hi | B_lo]
  size_t off_cnt;       // [row tiles of the W pass] uint32 arrival counters (assembly in the W pass)
  int asm_fused;        // set per call: the W pass with the Gram term also assembles wnorm and g
  int die_groups;       // W pass with the Gram term: d_in range groups of its die grid
                        // (w_tile), 0 for the plain order
  int dn_rt, dn_ct;     // dense mode: row tiles over d_out, column tiles over d_in
  int64_t ld_d;         // dense mode: padded rows of the column-tile partials
  size_t off_dense;     // dense mode: [dn_ct][ld_d] fp32 partial sums of (W + s B A)^2
  size_t ws_bytes;
};

// Division done in 32 bits whenever both operands fit, which is much
// cheaper on the GPU, and in 64 bits otherwise.
DORA_HD int64_t div_u(int64_t a, int64_t b) {
  if (((uint64_t)a | (uint64_t)b) < (1ull << 32)) return (int64_t)((uint32_t)a / (uint32_t)b);
  return a / b;
}

// First granule of d_in range x of X (ranges split the granules as evenly
// as integers allow; every range is non-empty when X <= n_gran).
DORA_HD int64_t range_lo(int64_t n_gran, int X, int x) { return div_u(n_gran * x, X); }

// First and one-past-last element of d_in range x.
DORA_HD int64_t range_k0(const NormPlan& p, int X, int x) {
  const int64_t k = range_lo(p.n_gran, X, x) * p.gran;
  return k < p.d_in ? k : p.d_in;
}

// Whether the W pass's grid of X d_in ranges x n_mt row tiles x n_nt column
// tiles takes the die grid of `groups` range groups (see w_tile).
DORA_HD bool die_grid_fits(int groups, int X, int64_t n_mt, int n_nt) {
  if (groups < 1 || groups > kDies || kDies % groups != 0) return false;
  return X % groups == 0 && n_mt % (kDies / groups) == 0;
}

// Tile (d_in range x, row tile m, column tile n) of W-pass workgroup b, for
// a grid of X ranges, n_mt row tiles and n_nt column tiles. Workgroups are
// dealt to the kDies dies in turn (die = b mod kDies), each die with its
// own L2, and launch in increasing b. In every order the column tiles of
// one (range, row tile) run on one die, kDies apart in launch order, so
// the W rows they share come from memory once.
//  - groups > 0 (die grid): the dies form `groups` range groups by kDies /
//    groups row groups; a die runs the ranges of its range group with the
//    row tiles of its row group. A's columns of a range are then fetched by
//    kDies / groups dies and B's rows of a row tile (read in the epilogue)
//    by `groups` dies, instead of once and kDies times (groups = kDies, die
//    = range, the plain order at X = kDies). Needs die_grid_fits.
//  - groups == 0: x = b mod X, then row tiles and column tiles; with
//    several column tiles, (range, row tile) pairs in that order by die.
DORA_HD void w_tile(int64_t b, int X, int64_t n_mt, int n_nt, int groups, int* x, int64_t* m, int* n) {
  if (groups > 0) {
    const int lo = (int)(b % kDies);
    const int64_t g8 = b / kDies;
    *n = (int)(g8 % n_nt);
    const int64_t s = g8 / n_nt;   // (range, row tile) pair of this die
    const int xa = X / groups, rows = kDies / groups;
    *x = (lo % groups) * xa + (int)(s % xa);
    *m = (s / xa) * rows + lo / groups;
    return;
  }
  if (n_nt > 1 && (X * n_mt * n_nt) % (kDies * n_nt) == 0) {
    const int lo = (int)(b % kDies);
    const int64_t g8 = b / kDies;
    *n = (int)(g8 % n_nt);
    const int64_t u = (g8 / n_nt) * kDies + lo;
    *x = (int)(u % X);
    *m = u / X;
    return;
  }
  *x = (int)(b % X);
  const int64_t t = b / X;
  *m = t / n_nt;
  *n = (int)(t - *m * n_nt);
}

}  // namespace dora
