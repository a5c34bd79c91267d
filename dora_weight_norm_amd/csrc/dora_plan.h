// Work plan of the factored row norm: tile shapes, the split of d_in across
// the MI355X dies, the even split of each die's work across its compute
// units, and the workspace layout. Shared by the host planner and the
// kernels so both derive segment indices from the same integer formulas.
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
constexpr int kGrid = 256;           // one norm workgroup per compute unit
constexpr int kThreads = 256;        // 4 waves of 64
constexpr int kGramCB = 64;          // columns of G per Gram-term workgroup
constexpr int kGramRows = 256;       // rows of B per Gram-term workgroup (32 per wave, 8 waves)

// Tile shapes of the norm's main kernel. The workgroup is WM x WN waves (4 or 8);
// each wave owns MB x NB blocks of 32x32 fp32 accumulators. KT is the d_in
// depth of one LDS stage, in elements.
struct TileShape {
  int wm, wn, mb, nb, kt;
};

enum TileCfg : int {
  kBf16R64 = 0,   // r <= 64  : 256 x 64 tiles
  kBf16R128 = 1,  // r <= 128 : 128 x 128
  kBf16R256 = 2,  // r <= 256 : 128 x 256
  kBf16R384 = 3,  // r <= 384 : 128 x 384
  kBf16R512 = 4,  // r <= 512 : 64 x 512
  kBf16R768 = 5,  // r >  512 : 64 x 768 (several column tiles beyond 768)
  kF32R32 = 6,    // fp32, r <= 32 : 128 x 32
  kF32R128 = 7,   // fp32, r > 32  : 128 x 128 (several column tiles beyond 128)
  kNumTileCfg = 8
};

DORA_HD TileShape tile_shape(int cfg) {
  switch (cfg) {
    case kBf16R64: return TileShape{2, 2, 4, 1, 64};
    case kBf16R128: return TileShape{1, 4, 4, 1, 64};
    case kBf16R256: return TileShape{1, 4, 4, 2, 64};
    case kBf16R384: return TileShape{2, 4, 2, 3, 64};
    case kBf16R512: return TileShape{1, 4, 2, 4, 64};
    case kBf16R768: return TileShape{1, 4, 2, 6, 32};
    case kF32R32: return TileShape{4, 1, 1, 1, 32};
    default: return TileShape{1, 4, 4, 1, 32};
  }
}

enum NormMode : int { kModeEmpty = 0, kModeRowOnly = 1, kModeFactored = 2 };

struct NormPlan {
  int64_t d_out, d_in, r;
  int dtype;            // 0 = bf16, 1 = fp32
  int mode;             // NormMode
  int cfg;              // TileCfg
  int vec_in;           // W and A rows allow aligned 16-byte loads
  int vec_b;            // B rows allow aligned 16-byte loads
  int mt, ntc, kt;      // tile rows, tile columns, stage depth
  int n_mt_w;           // row tiles over W
  int n_mt_a;           // row tiles over A (they produce G = A A^T)
  int n_nt;             // column tiles over r
  int64_t n_kt;         // stages over d_in
  int X;                // d_in ranges (one per die when X == 8)
  int P;                // workgroups per range; grid = X * P
  int maxseg;           // most workgroups that share one (range, tile)
  int64_t ld_w;         // n_mt_w * mt: padded row count of the W partials
  int64_t ga_rows;      // n_mt_a * mt
  int64_t ga_cols;      // n_nt * ntc
  int64_t r32;          // r rounded up to 32: side of the reduced Gram matrix
  int n_cb;             // 64-column blocks of G in the Gram-term kernel
  size_t off_base, off_cross, off_g, off_ghi, off_glo, off_ba;
  size_t ws_bytes;
};

// The split below is integer arithmetic on counts that fit 32 bits for any
// realistic shape; the 64-bit forms are kept for the rest (the division is
// done in 32 bits whenever both operands fit, which is much cheaper on the GPU).
DORA_HD int64_t div_u(int64_t a, int64_t b) {
  if (((uint64_t)a | (uint64_t)b) < (1ull << 32)) return (int64_t)((uint32_t)a / (uint32_t)b);
  return a / b;
}

// First stage of d_in range x (ranges split n_kt stages as evenly as integers allow).
DORA_HD int64_t range_lo(int64_t n_kt, int X, int x) { return div_u(n_kt * x, X); }

// Work units of one range are (tile, stage) pairs, tile-major. Workgroup s
// of P takes units [unit_lo(s), unit_lo(s+1)).
DORA_HD int64_t unit_lo(int64_t U, int P, int s) { return div_u(U * s, P); }

// The workgroup whose unit range holds unit w (0 <= w < U).
DORA_HD int slot_of(int64_t U, int P, int64_t w) { return (int)div_u((w + 1) * P - 1, U); }

DORA_HD int64_t n_tiles(const NormPlan& p) { return (int64_t)(p.n_mt_w + p.n_mt_a) * p.n_nt; }

}  // namespace dora
