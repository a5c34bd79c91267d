// Factored DoRA row norm on gfx950.
//
// ||W + sBA||^2_row = ||W||^2_row + 2s <W, BA>_row + s^2 ||BA||^2_row
// ("DoRA优化技术解析：从内存瓶颈到高效实现", cyqw.cn, §1.2 and §1.2.1;
// "Scaling DoRA", alanhou.org, "Factored Norm").
//
// Launches, in stream order:
//   Gram pass     G = A A^T: rows of A against rows of A, d_in cut into
//                 ranges; one partial G tile per (tile, range).
//   gram_reduce   sums the partials in a fixed order; for bf16 it stores G
//                 as an unevaluated sum of two bf16 matrices Ghi + Glo.
//   W pass        one workgroup per (row tile of W, column tile over r,
//                 d_in range): U = W A^T on the matrix cores, dotted with B
//                 row by row at the end (cross term; U is never stored), and
//                 the W fragments squared on the way (base term). On the
//                 streaming path (every dtype) each workgroup then runs its
//                 share of the Gram term's depth, B against (s/2) G, in the
//                 same accumulators: the dot with B at the end is then
//                 cross + (s/2) ba, since the Gram term (B G) . B is linear
//                 in B G. (fp16: B and G as bf16 hi + lo, on the bf16
//                 matrix cores.)
//   assemble      fixed-order sums of all partials;
//                 wnorm = sqrt(max(base + 2s cross + s^2 ba, 0)) and
//                 g = m / max(wnorm, eps) without contraction, with
//                 correctly rounded sqrt and division (same page, §1.2.2,
//                 §5.2, §6.2).
// Otherwise (the general kernels, and G folded into the W pass) the Gram
// term is a pass of its own after the W pass: (B G) on the matrix cores
// (B Ghi + B Glo for bf16; fp32 for fp16, on B widened), dotted with B,
// with the assembly fused in when one tile covers all of G's columns.
// When the streaming W pass has a single column tile of at most 128 columns
// (all of A's rows in each stage) it also computes the blocks of G, and the
// order becomes W pass, gram_reduce, Gram term: the separate Gram pass, and
// its second read of A, are skipped.
// The passes run the streaming kernel when W, A and B allow aligned 16-byte
// loads, and the general kernels otherwise; both write the same partials.
//
// When s == 0 or r == 0 the cross and Gram terms vanish and only a row
// sum-of-squares kernel runs (same page, §5.1, notes of Algorithm 1).
#include "dora_device.h"
#include "dora_launch.h"
#include "dora_plan.h"

namespace dora {

namespace {

constexpr int kGramCB = kGramCols;   // columns of G per Gram-term workgroup
constexpr int kGramRows = 256;  // rows of B per Gram-term workgroup (32 per wave, 8 waves)

// s_waitcnt with vmcnt(N) and lgkmcnt(0), expcnt left alone (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// Workgroup barrier that orders memory only through the explicit waits
// before it: unlike __syncthreads it does not wait for every outstanding
// load, so direct-to-LDS loads of later stages stay in flight across it.
// The memory clobber keeps the compiler from moving LDS accesses across.
__device__ __forceinline__ void barrier_keep_loads() { asm volatile("s_barrier" ::: "memory"); }

// Compile-time flag carried into generic lambdas.
template <bool V>
struct Tag {
  static constexpr bool value = V;
};

// Out-of-range buffer offset: a buffer load at it returns zeros.
constexpr uint32_t kOob = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes, 0x00020000);
}

// ---------------------------------------------------------------------------
// Streaming kernel (inputs allow aligned 16-byte loads).
//
// Workgroup = WM x WN waves = one (row tile, column tile, d_in range) of MT
// rows (W; A in the Gram pass; B in the Gram-term stages) and NTC columns
// (rows of A; rows of the stored Gram matrix in the Gram-term stages). Wave
// (wm, wn) owns MB x NB blocks of 32x32 accumulators. Each KT-deep stage of
// both operands (MT + NTC rows) arrives in one of NS LDS ring slots by
// direct-to-LDS loads (64 lanes x 16 B = 1 KiB per instruction) issued NS-1
// stages ahead, so several stages of loads are in flight while the matrix
// cores work; one barrier per stage publishes a slot and retires the one
// reused next. The waits before the barrier leave the younger stages'
// loads outstanding (an ordinary __syncthreads would drain them all).
// The fragments of the next K16 step are read into one of two register
// sets while the current step's MFMAs run.
// ---------------------------------------------------------------------------
template <typename T, int WM, int WN, int MB, int NB, int KT, int NS>
struct FastK {
  static constexpr int ESZ = Elem<T>::esz;
  static constexpr int EPC = Elem<T>::epc;
  static constexpr int FC = Elem<T>::frag_chunks;
  static constexpr int NW = WM * WN;
  static constexpr int NT = NW * 64;
  static constexpr int MT = WM * MB * 32;
  static constexpr int NTC = WN * NB * 32;
  static constexpr int RB = KT * ESZ;            // bytes of one LDS row
  static constexpr int CPR = RB / 16;            // 16-byte chunks per LDS row
  static constexpr int RPB = 1024 / RB;          // LDS rows per 1 KiB direct-load block
  static constexpr int KSTEPS = KT / 16;
  static constexpr int SLOT = (MT + NTC) * RB;   // bytes of one ring slot
  static constexpr int MBLK = MT * RB / 1024;    // blocks holding row-operand rows
  static constexpr int BPW = SLOT / 1024 / NW;   // direct-load blocks per wave per stage
  static constexpr int BPW_M = MBLK / NW;        // of which row-operand blocks
  // Epilogue: each wave stages B for its rows and columns, one 32-row block
  // (round) at a time, in a private region of one or two round buffers.
  static constexpr int RBB = NB * 32 * ESZ;      // bytes of one staged B row segment
  static constexpr int CPRB = RBB / 16;
  // XOR mask of the staged-B swizzle: the largest power of two below 8 that
  // divides the row's chunk count, so a swizzled chunk stays in its row.
  static constexpr int BSW = CPRB % 8 == 0 ? 7 : (CPRB % 4 == 0 ? 3 : (CPRB % 2 == 0 ? 1 : 0));
  static constexpr int RW = 32 * RBB;            // bytes of one round
  static constexpr int LPR = RW / 1024;          // direct loads per round
  static constexpr int NBUF = MB > 1 ? 2 : 1;    // round buffers per wave
  static constexpr int WB = NBUF * RW;           // bytes of a wave's region
  static constexpr int WPS = SLOT / WB;          // waves staging B in one ring slot
  static constexpr int WX = NW > WPS * NS ? NW - WPS * NS : 0;   // waves staging B past the ring
  static constexpr int REDB = 2 * WN * MT * 4;  // bytes of the epilogue's per-row sums (cross, base)
  // Lean register mode, for waves of 12 or more accumulator blocks (the
  // 256 x 384 tile: 192 accumulators per lane at two waves per SIMD, so at
  // most 64 registers for everything else): one set of fragments instead
  // of two, load offsets formed at each load from one per-lane register per
  // row length, and the epilogue's row sums kept at the end of the last ring
  // slot (past the B staging regions of the waves that use that slot).
  static constexpr bool LEAN = MB * NB >= 12;
  static constexpr int LAST_WAVES = NW > WPS * (NS - 1) ? NW - WPS * (NS - 1) : 0;   // waves staging B in the last slot
  static_assert(!LEAN || (WX == 0 && LAST_WAVES * WB + REDB <= SLOT), "lean: row sums fit the last slot");
  static_assert(NW == 4 || NW == 8, "four or eight waves");
  static_assert(CPR == 8 || CPR == 4, "LDS rows are 64 or 128 bytes");
  static_assert(KSTEPS * 2 * FC == CPR, "K16 steps cover the stage");
  static_assert(SLOT % (1024 * NW) == 0 && MBLK % NW == 0, "a stage splits evenly over the waves");
  static_assert(RW % 1024 == 0 && RBB % 16 == 0, "B stages in whole 1 KiB blocks");
  static_assert(WPS >= 1, "a wave's B fits one ring slot");
  static_assert(NS >= 2 && NS <= 4 && NS * SLOT + WX * WB + (LEAN ? 0 : REDB) <= 160 * 1024,
                "gfx950 has 160 KiB of LDS");
  static_assert(BPW * (NS - 1) < 64 && LPR < 64, "outstanding loads fit vmcnt");
  static_assert(KSTEPS % 2 == 0, "fragment buffers alternate within a stage");
};

// Physical 16-byte chunk of logical chunk c in LDS row `row`: an XOR swizzle
// under which the 16 lanes that one LDS cycle serves (64 banks of 4 bytes)
// hit distinct banks for both the fragment reads and the direct loads.
template <int CPR>
__device__ __forceinline__ int fswz(int row, int c) {
  if constexpr (CPR == 8) {
    return c ^ ((row >> 1) & 7);
  } else {
    return c ^ ((row >> 2) & 3);
  }
}

// What one launch of the streaming kernel computes.
//   kPassW     U = W A^T per (row tile, column tile, d_in range); epilogue:
//              base and cross partials.
//   kPassGram  G = A A^T partial tiles per d_in range.
//   kPassWG    kPassW, and in the same pass the blocks of G = A A^T for the
//              d_in range: the column operand is all of A's rows (one column
//              tile), so its stages in LDS are exactly what G needs. Wave q of
//              row tile m computes the 32x32 block m + n_mt * q of G (if it
//              exists) with one more MFMA per K16 step and stores it as that
//              range's Gram partial; no separate Gram pass runs.
//   kPassBG    (B G) over the virtual depth [B | B] . [Ghi ; Glo] (bf16) or
//              B . G (fp32) per (row tile, column tile of G); epilogue: dot
//              with B. With a single column tile the Gram term of each row is
//              complete in its workgroup, which then assembles wnorm and g;
//              otherwise it stores per-tile partials for the assembly kernel.
//   kPassWB    kPassW, then, in the same accumulators, the workgroup's share
//              (d_in range x of X takes part x of X of the virtual depth) of
//              the kPassBG product against the reduced Gram matrix scaled by
//              s/2. Since rowsum(B . (U + (s/2) B G)) = cross + (s/2) ba, the
//              epilogue's dot with B then yields cross + (s/2) ba per (range,
//              column tile), and no separate Gram-term pass runs.
enum PassKind : int { kPassW = 0, kPassGram = 1, kPassBG = 2, kPassWG = 3, kPassWB = 4 };

// Scalars and outputs of the final assembly (used by kPassBG only).
struct AssembleArgs {
  float s, eps;
  const float* m;
  float* wnorm;
  float* g;
};

// sum_{i < n} p[i * stride], added in increasing i. The loads are issued
// kSumBatch at a time (they do not depend on the running sum), so a long sum
// costs n / kSumBatch memory round trips instead of n; the order of the
// additions, and so the result, is that of the plain loop.
constexpr int kSumBatch = 16;
__device__ __forceinline__ float ordered_sum(const float* p, int64_t stride, int n) {
  float acc = 0.f;
  int i = 0;
  for (; i + kSumBatch <= n; i += kSumBatch) {
    float v[kSumBatch];
#pragma unroll
    for (int u = 0; u < kSumBatch; ++u) v[u] = p[(int64_t)(i + u) * stride];
#pragma unroll
    for (int u = 0; u < kSumBatch; ++u) acc += v[u];
  }
  if (i < n) {
    float v[kSumBatch];
#pragma unroll
    for (int u = 0; u < kSumBatch; ++u) v[u] = (i + u < n) ? p[(int64_t)(i + u) * stride] : 0.f;
#pragma unroll
    for (int u = 0; u < kSumBatch; ++u)
      if (i + u < n) acc += v[u];
  }
  return acc;
}

// wnorm = sqrt(max(base + 2s cross + s^2 ba, 0)) and g = m / max(wnorm, eps),
// every operation separately rounded (no contraction), sqrt and division
// correctly rounded ("DoRA优化技术解析", cyqw.cn, §1.2.2, §5.2, §6.2). base and
// cross are summed from their partials in a fixed order.
__device__ __forceinline__ void assemble_sums(float base, float cross, float ba, float s, float eps, const float* m,
                                              float* wnorm, float* g, int64_t j) {
  const float two_s = s + s;
  const float s2 = __fmul_rn(s, s);
  float val = __fadd_rn(__fadd_rn(base, __fmul_rn(two_s, cross)), __fmul_rn(s2, ba));
  val = (val < 0.f) ? 0.f : val;
  const float wn = sqrtf(val);
  wnorm[j] = wn;
  if (m != nullptr) {
    const float d = (wn < eps) ? eps : wn;
    g[j] = m[j] / d;
  }
}

// ordered_sum over partials that other workgroups of the running kernel
// stored as device-scope atomics: each load is a device-scope atomic load
// too, so it reads the value those stores made visible on every die and
// never a stale line of this die's L2.
__device__ __forceinline__ float ordered_sum_device(const float* p, int64_t stride, int n) {
  float acc = 0.f;
  for (int i = 0; i < n; i += kSumBatch) {
    float v[kSumBatch];
#pragma unroll
    for (int u = 0; u < kSumBatch; ++u)
      v[u] = (i + u < n) ? __hip_atomic_load(p + (int64_t)(i + u) * stride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                         : 0.f;
#pragma unroll
    for (int u = 0; u < kSumBatch; ++u)
      if (i + u < n) acc += v[u];
  }
  return acc;
}

// Row j's base and cross partials summed in plane order, then assembled.
// DEVICE: the partials were stored as device-scope atomics by workgroups of
// the running kernel (the W pass's own assembly); otherwise by an earlier
// kernel.
template <bool DEVICE = false>
__device__ __forceinline__ void assemble_row(const NormPlan& p, const char* ws, float s, float eps, const float* m,
                                             float* wnorm, float* g, int64_t j, float ba) {
  const float* part_base = reinterpret_cast<const float*>(ws + p.off_base);
  const float* part_cross = reinterpret_cast<const float*>(ws + p.off_cross);
  // Cross partials are planes (x, n) in the order x * n_nt + n.
  const float base = DEVICE ? ordered_sum_device(part_base + j, p.ld_w, p.xw) : ordered_sum(part_base + j, p.ld_w, p.xw);
  const float cross = DEVICE ? ordered_sum_device(part_cross + j, p.ld_w, p.xw * p.n_nt)
                             : ordered_sum(part_cross + j, p.ld_w, p.xw * p.n_nt);
  assemble_sums(base, cross, ba, s, eps, m, wnorm, g, j);
}

template <typename T, int WM, int WN, int MB, int NB, int KT, int NS, int MODE>
__global__ __launch_bounds__(WM * WN * 64, 1) void norm_fast_kernel(NormPlan p, const T* __restrict__ Msrc,
                                                                    const T* __restrict__ A,
                                                                    const T* __restrict__ B,
                                                                    char* __restrict__ ws, AssembleArgs aa) {
  using C = FastK<T, WM, WN, MB, NB, KT, NS>;
  constexpr int NW = C::NW, MT = C::MT, NTC = C::NTC, RB = C::RB, CPR = C::CPR, RPB = C::RPB;
  constexpr int FC = C::FC, EPC = C::EPC, ESZ = C::ESZ, KSTEPS = C::KSTEPS, BPW = C::BPW;
  constexpr bool GRAM = MODE == kPassGram;
  constexpr bool BG = MODE == kPassBG;
  constexpr bool GF = MODE == kPassWG;               // Gram blocks folded into the W pass
  constexpr bool WB = MODE == kPassWB;               // Gram-term stages after the W stages
  constexpr bool WP = MODE == kPassW || GF || WB;    // W pass
  static_assert((GRAM ? kRowPadG : kRowPadW) % MT == 0, "row tiles divide the plan's row padding");
  constexpr int NG = sizeof(T) == 2 ? 2 : 1;   // parts of the stored Gram matrix (hi, lo)
  // fp16 with the Gram term in the W pass: the stored Gram matrix is bf16
  // hi + lo as for bf16, and B comes split exactly into bf16 hi + lo (by
  // the Gram reduction, into the workspace as [d_out][B_hi | B_lo], rg
  // columns each); the virtual depth runs over three parts, [B_hi | B_lo |
  // B_hi] against [Ghi ; Ghi ; Glo], on the bf16 matrix cores (B_lo Glo,
  // about 2^-16 of the term, is left out).
  constexpr bool F16G = WB && __is_same(T, f16_t);
  constexpr int NV = F16G ? 3 : NG;             // parts of the virtual depth
  __shared__ __attribute__((aligned(1024))) char r0[C::SLOT];
  __shared__ __attribute__((aligned(1024))) char r1[C::SLOT];
  __shared__ __attribute__((aligned(1024))) char r2[NS > 2 ? C::SLOT : 16];
  __shared__ __attribute__((aligned(1024))) char r3[NS > 3 ? C::SLOT : 16];
  __shared__ __attribute__((aligned(1024))) char bx[(!GRAM && C::WX > 0) ? C::WX * C::WB : 16];
  __shared__ float red_arr[(GRAM || C::LEAN) ? 1 : 2 * WN * MT];
  // Slot j of the ring (j < NS); slots past NS are never named, so their
  // placeholder arrays take no LDS.
  auto ring = [&](int j) __attribute__((always_inline)) -> char* {
    if constexpr (NS == 2) {
      return j == 0 ? r0 : r1;
    } else if constexpr (NS == 3) {
      return j == 0 ? r0 : (j == 1 ? r1 : r2);
    } else {
      return j == 0 ? r0 : (j == 1 ? r1 : (j == 2 ? r2 : r3));
    }
  };
  // The epilogue's per-row sums of each column group, [WN][MT] for the
  // cross term and [WN][MT] for the base term: their own array, or in lean
  // mode the end of the last ring slot.
  float* const red = C::LEAN ? reinterpret_cast<float*>(ring(NS - 1) + C::SLOT - C::REDB) : red_arr;
  float* const red_base = red + WN * MT;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int lrow = lane & 31, lgrp = lane >> 5;

  // Tile of this workgroup.
  const int X = BG ? 1 : (GRAM ? p.xg : p.xw);
  const int n_nt = BG ? p.n_bt : (GRAM ? (int)(p.ga_cols / NTC) : p.n_nt);
  const int64_t m_rows = GRAM ? p.r : p.d_out;
  int x = blockIdx.x % X;
  const int t = blockIdx.x / X;
  int m = t / n_nt, n = t - m * n_nt;
  if constexpr (GRAM) {
    if (MT == NTC && p.gsym) tri_tile(t, n_nt, &m, &n);   // upper-triangle tiles only
  }
  if constexpr (WP) {
    // W pass: the order of w_tile (by die; the die grid where planned).
    int64_t mm;
    w_tile(blockIdx.x, X, (m_rows + MT - 1) / MT, n_nt, p.die_groups, &x, &mm, &n);
    m = (int)mm;
  }
  const int64_t mrow0 = (int64_t)m * MT;
  const int64_t n0 = (int64_t)n * NTC;
  const int64_t d_in = p.d_in;
  const int64_t m_left = m_rows - mrow0;
  // Valid rows of the tile (none for a square Gram tile past r: the Gram
  // columns are padded to 128, so 64-row tiles can start at or past r).
  const int m_lim = m_left <= 0 ? 0 : (m_left < MT ? (int)m_left : MT);

  // Stages of the tile, in two phases.
  //  1. (every mode but kPassBG) Msrc rows (W, or A in the Gram pass)
  //     against A's rows over this workgroup's d_in range [k0, k1).
  //  2. (kPassBG; kPassWB after phase 1) B's rows against rows of the
  //     stored Gram matrix over the virtual depth [v0, v0 + n_bs KT) of
  //     [0, NV rg): B's columns against Ghi, then again against Glo (fp16:
  //     B_hi against Ghi, B_lo against Ghi, B_hi against Glo). rg is a
  //     whole number of stages, so no stage straddles a seam.
  const int64_t k0 = BG ? 0 : range_k0(p, X, x);
  const int64_t k1 = BG ? 0 : range_k0(p, X, x + 1);
  const int n_st = (int)((k1 - k0 + KT - 1) / KT);   // phase-1 stages (>= 1 unless kPassBG)
  int n_bs = 0;
  int64_t v0 = 0;
  if constexpr (BG || WB) {
    const int64_t vg = (int64_t)NV * p.rg / KT;     // stages of the whole virtual depth
    const int64_t g0 = div_u(vg * x, X);
    n_bs = (int)(div_u(vg * (x + 1), X) - g0);
    v0 = g0 * KT;
  }
  // First stage of phase 2: right after phase 1, except for fp16 with the
  // Gram term, whose phase-2 stages run in a loop of their own (another
  // MFMA type; a branch between the two inside one loop makes the
  // compiler spill the accumulators): there phase 1 is padded with zero
  // stages to a whole group of NS.
  const int p2s = F16G ? (n_st + NS - 1) / NS * NS : n_st;
  const int n_tot = p2s + n_bs;

  // Every operand goes through a buffer descriptor spanning the tile's valid
  // rows: rows past the matrix read as zeros.
  const uint32_t m_rowb = (uint32_t)(d_in * ESZ), n_rowb = m_rowb;
  // (In the Gram-term pass a column tile may start past r, since rg pads r;
  // its A descriptor, never read there, then spans no rows.)
  const int n_lim = p.r - n0 < NTC ? (p.r > n0 ? (int)(p.r - n0) : 0) : NTC;
  const __amdgpu_buffer_rsrc_t mrs = make_rsrc(Msrc + mrow0 * d_in, (uint32_t)m_lim * m_rowb);
  const __amdgpu_buffer_rsrc_t ars = make_rsrc(A + n0 * d_in, (uint32_t)n_lim * n_rowb);
  // (phase-2 row operand: B, or for fp16 its bf16 split, 2 rg wide)
  const int64_t b_ld = F16G ? 2 * p.rg : p.r;
  const T* Bp = F16G ? reinterpret_cast<const T*>(ws + p.off_bf) : B;
  const uint32_t b_rowb = (uint32_t)(b_ld * ESZ), g_rowb = (uint32_t)((int64_t)NG * p.rg * ESZ);
  const int g_lim = p.rg - n0 < NTC ? (int)(p.rg - n0) : NTC;
  const T* Gs = reinterpret_cast<const T*>(ws + p.off_gg);
  const __amdgpu_buffer_rsrc_t brs = make_rsrc(Bp + mrow0 * b_ld, (uint32_t)m_lim * b_rowb);
  const __amdgpu_buffer_rsrc_t grs = make_rsrc(Gs + n0 * NG * p.rg, (uint32_t)g_lim * g_rowb);

  // Direct loads: this wave fills blocks wave, wave + NW, ...; lane l lands at
  // byte 16*l of its block, which is LDS row blk*RPB + l/CPR, physical chunk
  // l % CPR. The logical chunk (and so the global k offset) does not depend
  // on the block, because blocks start on swizzle-period boundaries.
  const int l_row = lane / CPR;
  const int a_chunk = fswz<CPR>(wave * RPB + l_row, lane % CPR);
  // Blocks b < BPW_M of every wave hold row-operand rows, the rest the
  // column operand's rows; doff for phase 1, eoff for phase 2.
  // (Lean mode keeps only the per-lane parts, one per row length, and adds
  // each block's first row at the load.)
  constexpr int BPW_ARR = C::LEAN ? 1 : BPW;
  uint32_t doff[BPW_ARR], eoff[BPW_ARR];
  if constexpr (!C::LEAN) {
#pragma unroll
    for (int b = 0; b < BPW; ++b) {
      const int row = (b * NW + wave) * RPB + l_row;
      doff[b] = b < C::BPW_M ? (uint32_t)row * m_rowb + (uint32_t)(a_chunk * 16)
                             : (uint32_t)(row - MT) * n_rowb + (uint32_t)(a_chunk * 16);
      eoff[b] = b < C::BPW_M ? (uint32_t)row * b_rowb + (uint32_t)(a_chunk * 16)
                             : (uint32_t)(row - MT) * g_rowb + (uint32_t)(a_chunk * 16);
    }
  }
  // Lean mode: offset of block 0 for this lane, one per row length (W and
  // A rows in phase 1 share d_in; B rows and Gram rows in phase 2), and the
  // uniform step from one of the wave's blocks to the next (NW blocks of RPB
  // rows). Block BPW_M, the column operand's first, starts at the same row
  // of its operand as block 0 of the row operand (MBLK * RPB == MT).
  const uint32_t base_m = (uint32_t)(wave * RPB + l_row) * m_rowb + (uint32_t)(a_chunk * 16);
  const uint32_t base_b = (uint32_t)(wave * RPB + l_row) * b_rowb + (uint32_t)(a_chunk * 16);
  const uint32_t base_g = (uint32_t)(wave * RPB + l_row) * g_rowb + (uint32_t)(a_chunk * 16);
  const uint32_t step_m = (uint32_t)(NW * RPB) * m_rowb, step_b = (uint32_t)(NW * RPB) * b_rowb,
                 step_g = (uint32_t)(NW * RPB) * g_rowb;
  const int lane_k = a_chunk * EPC;   // this lane's first element within a stage's depth

  // Blocks [b0, b1) of this wave's share of stage i into a ring slot.
  // Stages past the tile (the loop runs a whole number of unrolled groups)
  // and chunks past the valid depth read as zeros, so every step issues the
  // same loads. (gtag: Tag<true> in the loop over fp16's Gram-term stages,
  // all of whose loads are of phase 2.)
  auto issue_blocks = [&](int i, char* slot, int b0, int b1, auto gtag) __attribute__((always_inline)) {
    const bool ph2 = (F16G && decltype(gtag)::value) || BG || (WB && i >= p2s);   // uniform
    const int j = i - p2s;
    const bool in = ph2 ? j < n_bs : i < n_st;
    // Column-operand depth ks (phase 2: into the virtual depth), and the
    // depths km into the row operand's rows (B's in phase 2) and kc into
    // the column operand's (phase 2: rows of [Ghi | Glo]).
    int64_t ks, km, kc;
    if constexpr (F16G) {
      // fp16's three parts run over [B_hi | B_lo | B_hi] and [Ghi ; Ghi ;
      // Glo]: km is the virtual depth k2 in parts 0 and 1 and k2 - 2 rg in
      // part 2, kc is k2 in part 0 and k2 - rg after. (32-bit: k2 < 3 rg.)
      const int32_t rg = (int32_t)p.rg, k2 = (int32_t)v0 + j * KT;
      const int32_t kr = k2 >= rg ? k2 - rg : k2;
      ks = ph2 ? (int64_t)k2 : k0 + (int64_t)i * KT;
      km = ph2 ? (int64_t)(kr >= rg ? kr - rg : k2) : ks;
      kc = ph2 ? (int64_t)kr : ks;
    } else {
      ks = ph2 ? v0 + (int64_t)j * KT : k0 + (int64_t)i * KT;
      km = (ph2 && ks >= p.rg) ? ks - p.rg : ks;   // B's columns against Ghi, then Glo
      kc = ks;
    }
    const uint32_t kb_m = (uint32_t)((in ? km : 0) * ESZ), kb_n = (uint32_t)((in ? kc : 0) * ESZ);
    if constexpr (C::LEAN) {
      // Valid elements left in the operands' rows from this stage's depth
      // (uniform; 0 past the tile), against which each lane's first element
      // is compared in 32 bits. Gram rows and fp16's split B rows (zero past
      // r) are never short.
      const int64_t lm = in ? ((F16G && ph2) ? (int64_t)KT : (ph2 ? p.r : d_in) - km) : 0;
      const int64_t ln = in ? (ph2 ? (int64_t)KT : d_in - ks) : 0;
      const int32_t rm = (int32_t)(lm < KT ? lm : KT), rn = (int32_t)(ln < KT ? ln : KT);
      const bool okm = lane_k < rm, okn = lane_k < rn;
#pragma unroll
      for (int b = 0; b < BPW; ++b) {
        if (b < b0 || b >= b1) continue;
        // Block b starts whole steps of NW blocks past the operand's first
        // block; the offset is formed at the load, none is kept across the
        // loop.
        uint32_t vo = b < C::BPW_M ? (ph2 ? base_b : base_m) + (uint32_t)b * (ph2 ? step_b : step_m)
                                   : (ph2 ? base_g : base_m) + (uint32_t)(b - C::BPW_M) * (ph2 ? step_g : step_m);
        asm volatile("" : "+v"(vo));
        void* dst = slot + (b * NW + wave) * 1024;
        const uint32_t off = (b < C::BPW_M ? okm : okn) ? vo : kOob;
        const int kb = (int)(b < C::BPW_M ? kb_m : kb_n);
        if (b < C::BPW_M) {
          const __amdgpu_buffer_rsrc_t rs = ph2 ? brs : mrs;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)dst, 16, off, kb, 0,
                                                   0);
        } else {
          const __amdgpu_buffer_rsrc_t rs = ph2 ? grs : ars;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)dst, 16, off, kb, 0,
                                                   0);
        }
      }
      return;
    }
    const bool ok_m = in && ((F16G && ph2) || km + (int64_t)a_chunk * EPC < (ph2 ? p.r : d_in));
    const bool ok_n = in && (ph2 || ks + (int64_t)a_chunk * EPC < d_in);
#pragma unroll
    for (int b = 0; b < BPW; ++b) {
      if (b < b0 || b >= b1) continue;
      // (Offsets are computed before the builtin call: a conditional
      // expression inside its argument list made hipcc's host pass drop the
      // kernel's launch stub.)
      void* dst = slot + (b * NW + wave) * 1024;
      const uint32_t o = ph2 ? eoff[b < BPW_ARR ? b : 0] : doff[b < BPW_ARR ? b : 0];
      const uint32_t off = (b < C::BPW_M ? ok_m : ok_n) ? o : kOob;
      const int kb = (int)(b < C::BPW_M ? kb_m : kb_n);
      if (b < C::BPW_M) {
        const __amdgpu_buffer_rsrc_t rs = ph2 ? brs : mrs;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)dst, 16, off, kb, 0, 0);
      } else {
        const __amdgpu_buffer_rsrc_t rs = ph2 ? grs : ars;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)dst, 16, off, kb, 0, 0);
      }
    }
  };

  f32x16 acc[MB][NB];
#pragma unroll
  for (int a = 0; a < MB; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;
  float sq[MB];
#pragma unroll
  for (int a = 0; a < MB; ++a) sq[a] = 0.f;
  // Folded Gram block of this wave: rows gI, columns gJ (32-blocks of G).
  int gI = 0, gJ = 0;
  bool has_g = false;
  f32x16 gacc;
#pragma unroll
  for (int v = 0; v < 16; ++v) gacc[v] = 0.f;
  if constexpr (GF) {
    const int nbc = (int)(p.rg / 32);
    const int n_mt = (int)((p.d_out + MT - 1) / MT);
    const int gb = m + n_mt * wave;
    has_g = gb < nbc * nbc;
    gI = has_g ? gb / nbc : 0;
    gJ = has_g ? gb - gI * nbc : 0;
  }

  // Fragments of one K16 step: F[a] row operand, F[MB + b] column operand,
  // F[MB + NB] and F[MB + NB + 1] the folded Gram block's row and column
  // blocks of A.
  constexpr int NGF = GF ? 2 : 0;
  typedef u32x4 Frag[MB + NB + NGF][FC];
  // Lean mode: every fragment of a lane sits in rows with the same swizzle
  // ((lrow >> 1) & 7: the blocks start on multiples of 16 rows), so a step's
  // addresses are one per-lane offset plus constants; it is formed at each
  // step rather than kept per step and slot.
  const uint32_t ysw = (uint32_t)(lgrp ^ ((lrow >> 1) & 7));
  auto read_step = [&](const char* slot, int s, Frag& F) __attribute__((always_inline)) {
    if constexpr (C::LEAN) {
      static_assert(FC == 1 && CPR == 8, "lean mode: 16-bit types, 128-byte LDS rows");
      uint32_t y = ysw;
      asm volatile("" : "+v"(y));
      const uint32_t x = (((uint32_t)(2 * s)) ^ y) * 16u + (uint32_t)lrow * RB;
      const char* rb = slot + wm * MB * 32 * RB + x;
      const char* cb = slot + (MT + wn * NB * 32) * RB + x;
#pragma unroll
      for (int a = 0; a < MB; ++a) F[a][0] = *reinterpret_cast<const u32x4*>(rb + a * 32 * RB);
#pragma unroll
      for (int b = 0; b < NB; ++b) F[MB + b][0] = *reinterpret_cast<const u32x4*>(cb + b * 32 * RB);
      return;
    }
#pragma unroll
    for (int f = 0; f < FC; ++f) {
      const int c = s * 2 * FC + lgrp * FC + f;
      const int co = fswz<CPR>(lrow, c) * 16;
#pragma unroll
      for (int a = 0; a < MB; ++a)
        F[a][f] = *reinterpret_cast<const u32x4*>(slot + ((wm * MB + a) * 32 + lrow) * RB + co);
#pragma unroll
      for (int b = 0; b < NB; ++b)
        F[MB + b][f] = *reinterpret_cast<const u32x4*>(slot + (MT + (wn * NB + b) * 32 + lrow) * RB + co);
      if constexpr (GF) {
        F[MB + NB][f] = *reinterpret_cast<const u32x4*>(slot + (MT + gI * 32 + lrow) * RB + co);
        F[MB + NB + 1][f] = *reinterpret_cast<const u32x4*>(slot + (MT + gJ * 32 + lrow) * RB + co);
      }
    }
  };
  // (gtag: Tag<true> in the loop over fp16's Gram-term stages)
  auto mfma_step = [&](const Frag& F, bool w_stage, int s, auto gtag) __attribute__((always_inline)) {
    if constexpr (F16G && decltype(gtag)::value) {
      // Gram-term stage (fp16): B's bf16 parts against the bf16 Gram rows.
#pragma unroll
      for (int a = 0; a < MB; ++a)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[a][b] = Mfma<bf16_t>::run(F[a], F[MB + b], acc[a][b]);
      return;
    }
#pragma unroll
    for (int a = 0; a < MB; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[a][b] = Mfma<T>::run(F[a], F[MB + b], acc[a][b]);
    if constexpr (GF) gacc = Mfma<T>::run(F[MB + NB], F[MB + NB + 1], gacc);
    if constexpr (WP) {
      // The WN waves of a row group hold the same row fragments, so K16 step
      // s is squared by column group s % WN alone (a wave-uniform branch);
      // the epilogue adds the groups' sums. Rows of B (phase 2) are not part
      // of the base term.
      if (s % WN == wn) {
#pragma unroll
        for (int a = 0; a < MB; ++a)
#pragma unroll
          for (int f = 0; f < FC; ++f) {
            const float q = chunk_sumsq(F[a][f], T());
            sq[a] += (WB && !w_stage) ? 0.f : q;
          }
      }
    }
  };
  // Pipeline. Stage j lives in ring slot j % NS. In stage i, K16 step s+1's
  // fragments are read while step s's MFMAs run. Before the last step: wait
  // for this wave's fragment reads of stage i and its loads of stage i+1
  // (the NS-2 younger stages stay in flight), barrier (stage i is in
  // registers in every wave and stage i+1 has landed everywhere), load stage
  // i+NS into the slot stage i vacated and read stage i+1's first step. The
  // stage count is rounded up to whole unrolled groups (the extra stages are
  // zeros), so the loop body is straight-line code with fixed load counts.
  const int n_pad = (n_tot + NS - 1) / NS * NS;
  // With two slots an odd last stage runs after the loop on its own, rather
  // than as a stage of zeros beside it in the unrolled pair. The extra code
  // stays within the register budget of tiles of up to 6 blocks per wave;
  // larger ones keep the zero stage (their tail spilled).
  constexpr bool PEEL = NS == 2 && MB * NB <= 6 && !F16G;
  const int n_loop = PEEL ? (n_tot & ~1) : n_pad;   // stages the unrolled loop runs
  Frag H[C::LEAN ? 1 : 2];
  // With two slots each stage's loads are spread over the stage before it:
  // the row-operand blocks (the HBM stream) right after the barrier that
  // frees their slot, the column-operand blocks a few at a time after each
  // of the first KSTEPS-1 steps' fragment reads. A wave stalls while the
  // address unit takes a burst of load instructions; spread out, the
  // stalls fall between MFMA steps (in lean mode, with one fragment set,
  // the other wave of the SIMD cannot cover them at all).
  constexpr bool SPREAD = NS == 2;
  constexpr int COL_PER_STEP = (BPW - C::BPW_M + KSTEPS - 2) / (KSTEPS - 1);
  if constexpr (SPREAD) {
    issue_blocks(0, ring(0), 0, BPW, Tag<false>{});
    issue_blocks(1, ring(1), 0, C::BPW_M, Tag<false>{});
    wait_vm_lgkm0<C::BPW_M>();   // stage 0 complete; stage 1's row-operand blocks in flight
  } else {
#pragma unroll
    for (int j = 0; j < NS; ++j) issue_blocks(j, ring(j), 0, BPW, Tag<false>{});
    wait_vm_lgkm0<(NS - 1) * BPW>();   // stage 0 complete; stages 1 .. NS-1 in flight
  }
  barrier_keep_loads();
  read_step(ring(0), 0, H[0]);
  if constexpr (C::LEAN) {
    // One fragment set: step s's MFMAs, then step s+1's fragments into the
    // same registers (the other wave of the SIMD keeps its matrix core busy
    // meanwhile). After the last step of stage i every wave has read all of
    // stage i: wait for stage i+1's loads, barrier, reload stage i's slot
    // with stage i+NS, read stage i+1's first step.
    auto lean_group = [&](int i0, auto gtag) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        const int i = i0 + j;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
          __builtin_amdgcn_sched_barrier(0);
          mfma_step(H[0], i < n_st, s, gtag);
          __builtin_amdgcn_sched_barrier(0);
          if (s + 1 < KSTEPS) {
            read_step(ring(j), s + 1, H[0]);
            if constexpr (SPREAD) {
              // Column-operand blocks of stage i+1 (its slot was freed at
              // the last barrier; its row-operand blocks went out then).
              const int c0 = C::BPW_M + s * COL_PER_STEP;
              const int c1 = c0 + COL_PER_STEP < BPW ? c0 + COL_PER_STEP : BPW;
              __builtin_amdgcn_sched_barrier(0);
              issue_blocks(i + 1, ring((j + 1) % NS), c0, c1, gtag);
            }
          } else {
            wait_vm_lgkm0<(NS - 2) * BPW>();   // (with two slots: every load issued so far)
            barrier_keep_loads();
            if constexpr (SPREAD) {
              issue_blocks(i + NS, ring(j), 0, C::BPW_M, gtag);
            } else {
              issue_blocks(i + NS, ring(j), 0, BPW, gtag);
            }
            read_step(ring((j + 1) % NS), 0, H[0]);
          }
        }
      }
    };
    for (int i0 = 0; i0 < (F16G ? p2s : n_pad); i0 += NS) lean_group(i0, Tag<false>{});
    if constexpr (F16G) {
      for (int i0 = p2s; i0 < n_pad; i0 += NS) lean_group(i0, Tag<true>{});
    }
  } else {
  auto plain_group = [&](int i0, auto gtag) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int i = i0 + j;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        if (s + 1 < KSTEPS) {
          read_step(ring(j), s + 1, H[(s + 1) & 1]);
          if constexpr (SPREAD) {
            const int c0 = C::BPW_M + s * COL_PER_STEP;
            const int c1 = c0 + COL_PER_STEP < BPW ? c0 + COL_PER_STEP : BPW;
            __builtin_amdgcn_sched_barrier(0);
            issue_blocks(i + 1, ring((j + 1) % NS), c0, c1, gtag);
          }
        } else {
          wait_vm_lgkm0<(NS - 2) * BPW>();
          barrier_keep_loads();
          if constexpr (SPREAD) {
            issue_blocks(i + NS, ring(j), 0, C::BPW_M, gtag);
          } else {
            issue_blocks(i + NS, ring(j), 0, BPW, gtag);
          }
          read_step(ring((j + 1) % NS), 0, H[0]);
        }
        __builtin_amdgcn_sched_barrier(0);
        mfma_step(H[s & 1], i < n_st, s, gtag);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  for (int i0 = 0; i0 < (F16G ? p2s : n_loop); i0 += NS) plain_group(i0, Tag<false>{});
  if constexpr (F16G) {
    for (int i0 = p2s; i0 < n_loop; i0 += NS) plain_group(i0, Tag<true>{});
  }
  }
  if constexpr (PEEL && !C::LEAN) {
    if (n_tot & 1) {
      // The odd last stage (slot 0): its loads landed and its first step's
      // fragments were read at the loop's last barrier.
      const int i = n_tot - 1;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        if (s + 1 < KSTEPS) read_step(ring(0), s + 1, H[(s + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
        mfma_step(H[s & 1], i < n_st, s, Tag<false>{});
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  // The ring is reused below: drain the trailing (zero) loads everywhere.
  wait_vm_lgkm0<0>();
  barrier_keep_loads();

  if constexpr (GRAM) {
    float* gdst = reinterpret_cast<float*>(ws + p.off_g) +
                  ((int64_t)x * p.ga_rows + mrow0 + wm * MB * 32) * p.ga_cols + n0 + wn * NB * 32;
#pragma unroll
    for (int a = 0; a < MB; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          gdst[(int64_t)(a * 32 + acc_row(v, lgrp)) * p.ga_cols + b * 32 + lrow] = acc[a][b][v];
  } else {
    const int64_t wrow0 = mrow0 + wm * MB * 32;   // first row of this wave
    if constexpr (GF) {
      if (has_g) {
        float* gdst = reinterpret_cast<float*>(ws + p.off_g) + ((int64_t)x * p.ga_rows + gI * 32) * p.ga_cols + gJ * 32;
#pragma unroll
        for (int v = 0; v < 16; ++v) gdst[(int64_t)acc_row(v, lgrp) * p.ga_cols + lrow] = gacc[v];
      }
    }
    if constexpr (WP) {
      // Base term: each column group's sum over its K16 steps (the two
      // k-halves of a row live in lanes l and l+32); the groups are added in
      // order with the cross sums below.
#pragma unroll
      for (int a = 0; a < MB; ++a) {
        const float qs = sq[a] + __shfl_xor(sq[a], 32, 64);
        if (lgrp == 0) red_base[wn * MT + wm * MB * 32 + a * 32 + lrow] = qs;
      }
    }
    // Dot each accumulator row with its B row over this wave's columns. B
    // is staged per 32-row block (round) in the wave's own LDS region (the
    // ring is free after the last barrier), the next round's loads in flight
    // while this round is used; then the column groups are added in order.
    char* bb;
    if constexpr (C::WX > 0) {
      bb = wave < C::WPS * NS ? ring(wave / C::WPS) + (wave % C::WPS) * C::WB : bx + (wave - C::WPS * NS) * C::WB;
    } else {
      bb = ring(wave / C::WPS) + (wave % C::WPS) * C::WB;
    }
    const int64_t w_left = p.d_out - wrow0;
    const int w_lim = w_left <= 0 ? 0 : (w_left < MB * 32 ? (int)w_left : MB * 32);
    const uint32_t brow_bytes = (uint32_t)(p.r * ESZ);
    const int64_t c0 = n0 + wn * NB * 32;       // first column of this wave
    const __amdgpu_buffer_rsrc_t brs = make_rsrc(B + wrow0 * p.r + (c0 < p.r ? c0 : 0), (uint32_t)w_lim * brow_bytes);
    auto issue_b = [&](int a, char* buf) __attribute__((always_inline)) {
#pragma unroll
      for (int q = 0; q < C::LPR; ++q) {
        const int slot16 = q * 64 + lane;
        const int row = slot16 / C::CPRB, c = (slot16 % C::CPRB) ^ (row & C::BSW);
        const uint32_t off = (c0 + (int64_t)c * EPC < p.r)
                                 ? (uint32_t)(a * 32 + row) * brow_bytes + (uint32_t)(c * 16) : kOob;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(brs, (__attribute__((address_space(3))) void*)(buf + q * 1024), 16,
                                                 off, 0, 0, 0);
      }
    };
    issue_b(0, bb);
    if constexpr (MB > 1) issue_b(1, bb + C::RW);
#pragma unroll
    for (int a = 0; a < MB; ++a) {
      const char* buf = bb + (a & 1) * C::RW;
      if (a + 1 < MB) {
        wait_vm_lgkm0<C::LPR>();   // round a landed; round a+1 in flight
      } else {
        wait_vm_lgkm0<0>();
      }
      float pa[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) pa[v] = 0.f;
      if constexpr (FC == 1) {
        // (16-bit types) B's 32x32 block in the accumulator layout (row acc_row(v), column
        // lrow), made by two MFMAs: the row-operand fragments are B's rows
        // (16-byte reads of the staged rows, as for W), the column operand
        // the 0/1 selector E_h with E_h[k][j] = 1 iff j = k + 16h. Each
        // output is one product by 1.0, so the block is exact; eight 16-byte
        // reads replace 64 two-byte reads per lane.
        const uint32_t one = __is_same(T, bf16_t) ? 0x3F80u : 0x3C00u;
        u32x4 E[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int e = lrow - 8 * lgrp - 16 * h;   // this lane's 1.0 sits at k-element e, if 0 <= e < 8
#pragma unroll
          for (int w = 0; w < 4; ++w) E[h][w] = (e == 2 * w ? one : 0u) | ((e == 2 * w + 1 ? one : 0u) << 16);
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          u32x4 f[2];
#pragma unroll
          for (int h = 0; h < 2; ++h)
            f[h] = *reinterpret_cast<const u32x4*>(buf + lrow * C::RBB +
                                                   (((4 * b + 2 * h + lgrp) ^ (lrow & C::BSW)) * 16));
          f32x16 bb32;
#pragma unroll
          for (int v = 0; v < 16; ++v) bb32[v] = 0.f;
          bb32 = Mfma<T>::run(&f[0], &E[0], bb32);
          bb32 = Mfma<T>::run(&f[1], &E[1], bb32);
#pragma unroll
          for (int v = 0; v < 16; ++v) pa[v] = fmaf(acc[a][b][v], bb32[v], pa[v]);
        }
      } else {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int col = b * 32 + lrow;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int row = acc_row(v, lgrp);
            const T bv = *reinterpret_cast<const T*>(buf + row * C::RBB + (((col / EPC) ^ (row & C::BSW)) * 16) +
                                                     (col % EPC) * ESZ);
            pa[v] = fmaf(acc[a][b][v], to_f32(bv), pa[v]);
          }
        }
      }
      const float tot = sum32_transpose(pa, lane);
      if ((lane & 1) == 0) red[wn * MT + wm * MB * 32 + a * 32 + acc_row((lane & 31) >> 1, lgrp)] = tot;
      if (a + 2 < MB) {
        wait_vm_lgkm0<C::LPR>();   // this round's LDS reads are done before its buffer is refilled
        issue_b(a + 2, bb + (a & 1) * C::RW);
      }
    }
    __syncthreads();
    if (BG && n_nt == 1) {
      // The whole Gram term of each row is here: assemble the tile's rows.
      if (tid < MT && mrow0 + tid < p.d_out) {
        float ba = 0.f;
#pragma unroll
        for (int gi = 0; gi < WN; ++gi) ba += red[gi * MT + tid];
        assemble_row(p, ws, aa.s, aa.eps, aa.m, aa.wnorm, aa.g, mrow0 + tid, ba);
      }
    } else {
      float* part = reinterpret_cast<float*>(ws + (BG ? p.off_ba : p.off_cross));
      const int64_t plane = (int64_t)x * n_nt + n;
      // With the assembly in this pass (asm_fused) the partials are stored
      // as device-scope atomics: written through to where every die reads
      // them, so no write-back of the die's L2 is needed before they are
      // counted in (below).
      const bool dev = WB && p.asm_fused;
      if (tid < MT) {
        float cs = 0.f;
#pragma unroll
        for (int gi = 0; gi < WN; ++gi) cs += red[gi * MT + tid];
        float* cp = part + plane * p.ld_w + mrow0 + tid;
        if (dev) {
          __hip_atomic_store(cp, cs, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
          *cp = cs;
        }
        if constexpr (WP) {
          if (n == 0) {
            float bs = 0.f;
#pragma unroll
            for (int gi = 0; gi < WN; ++gi) bs += red_base[gi * MT + tid];
            float* bp = reinterpret_cast<float*>(ws + p.off_base) + (int64_t)x * p.ld_w + mrow0 + tid;
            if (dev) {
              __hip_atomic_store(bp, bs, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            } else {
              *bp = bs;
            }
          }
        }
      }
      if constexpr (WB) {
        if (p.asm_fused) {
          // The row tile's last workgroup to finish assembles its rows
          // (nobody waits). Each wave waits until its device-scope partial
          // stores are acknowledged (vmcnt(0): the device has them), then
          // one thread counts the workgroup in with a device-scope atomic
          // add; the workgroup that brings the count to the row tile's
          // total sums every partial of its rows in the fixed plane order,
          // with device-scope loads. Every access to the partials and the
          // counter is a device-scope atomic and the count is taken only
          // after the stores completed, so the last workgroup reads every
          // partial; no fence is needed (a release fence would write back
          // the die's whole L2, an acquire fence would invalidate it under
          // the workgroups still streaming W). The counters were zeroed by
          // the reduction launched before this pass.
          __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's stores have completed
          __syncthreads();
          int* last = reinterpret_cast<int*>(red);   // the row sums are consumed
          if (tid == 0) {
            unsigned* cnt = reinterpret_cast<unsigned*>(ws + p.off_cnt) + m;
            const unsigned total = (unsigned)(X * n_nt);
            const unsigned old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            *last = old + 1u == total;
          }
          __syncthreads();
          if (*last != 0 && tid < MT && mrow0 + tid < p.d_out)
            assemble_row<true>(p, ws, aa.s, aa.eps, aa.m, aa.wnorm, aa.g, mrow0 + tid, 0.f);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// General kernel (any alignment): one workgroup per (row tile, column tile,
// d_in range); both operands are staged through two LDS buffers by
// element-wise register loads with explicit zero fill, one stage ahead.
// ---------------------------------------------------------------------------
template <int A_, int B_>
struct CMax {
  static constexpr int v = A_ > B_ ? A_ : B_;
};

template <typename T, int WM, int WN, int MB, int NB, int KT>
struct GenK {
  static constexpr int ESZ = Elem<T>::esz;
  static constexpr int EPC = Elem<T>::epc;
  static constexpr int FC = Elem<T>::frag_chunks;
  static constexpr int NW = WM * WN;            // waves per workgroup
  static constexpr int NT = NW * 64;            // threads per workgroup
  static constexpr int MT = WM * MB * 32;
  static constexpr int NTC = WN * NB * 32;
  static constexpr int RB = KT * ESZ;           // bytes of one LDS row
  static constexpr int CPR = RB / 16;           // 16-byte chunks per LDS row
  static constexpr int KSTEPS = KT / 16;
  static constexpr int ROWS = MT + NTC;
  static constexpr int STAGE = ROWS * RB;
  static constexpr int NCH = ROWS * CPR;
  static constexpr int CPT = NCH / NT;          // chunks per thread
  static constexpr int RSTEP = NT / CPR;        // row step between a thread's chunks
  // Epilogue: B rows of one 32-row block of the tile, the tile's NTC columns.
  static constexpr int RBB = NTC * ESZ;         // bytes of one staged B row
  static constexpr int CPRB = RBB / 16;         // 16-byte chunks per staged B row
  static constexpr int BROUND = 32 * RBB;       // bytes of one staged 32-row B block
  static constexpr int ROUNDS = WM * MB;        // 32-row blocks per tile
  static constexpr int L0 = CMax<STAGE, BROUND>::v;
  static constexpr int RED = (WN + 1) * MT * 4; // per-wave cross sums and base sums
  static_assert(NW == 4 || NW == 8, "four or eight waves");
  static_assert(NCH % NT == 0, "stage must split evenly over the threads");
  static_assert(MT % RSTEP == 0, "M rows end on a thread-row boundary");
  static_assert(KSTEPS * 2 * FC == CPR, "K16 steps cover the stage");
  static_assert(CPRB % 8 == 0, "staged B rows hold whole swizzle groups");
  static_assert(2 * L0 + RED <= 160 * 1024, "gfx950 has 160 KiB of LDS per workgroup");
};

template <typename T, int WM, int WN, int MB, int NB, int KT, bool GRAM>
__global__ __launch_bounds__(WM * WN * 64, 1) void norm_gen_kernel(NormPlan p, const T* __restrict__ Msrc,
                                                                   const T* __restrict__ A,
                                                                   const T* __restrict__ B,
                                                                   char* __restrict__ ws) {
  using C = GenK<T, WM, WN, MB, NB, KT>;
  constexpr int MT = C::MT, NTC = C::NTC, RB = C::RB, CPR = C::CPR, FC = C::FC, EPC = C::EPC;
  constexpr int ESZ = C::ESZ, NT = C::NT;
  __shared__ __attribute__((aligned(1024))) char s0[C::L0];
  __shared__ __attribute__((aligned(1024))) char s1[C::L0];
  __shared__ __attribute__((aligned(16))) float sred[C::RED / 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wmi = wave / WN, wni = wave % WN;
  const int lrow = lane & 31, lgrp = lane >> 5;

  const int X = GRAM ? p.xg : p.xw;
  const int n_nt = GRAM ? (int)(p.ga_cols / NTC) : p.n_nt;
  const int64_t m_rows = GRAM ? p.r : p.d_out;
  const int x = blockIdx.x % X;
  const int t = blockIdx.x / X;
  const int m = t / n_nt, n = t - m * n_nt;
  const int64_t d_in = p.d_in;
  const int64_t k0 = range_k0(p, X, x), k1 = range_k0(p, X, x + 1);
  const int n_st = (int)((k1 - k0 + KT - 1) / KT);

  const int64_t mrow0 = (int64_t)m * MT;
  const T* msrc = Msrc + mrow0 * d_in;
  const int64_t m_left = m_rows - mrow0;
  const int m_lim = m_left < MT ? (int)m_left : MT;   // valid rows of this tile
  const int64_t n0 = (int64_t)n * NTC;
  const T* nsrc = A + n0 * d_in;
  // (In the Gram-term pass a column tile may start past r, since rg pads r;
  // its A descriptor, never read there, then spans no rows.)
  const int n_lim = p.r - n0 < NTC ? (p.r > n0 ? (int)(p.r - n0) : 0) : NTC;

  f32x16 acc[MB][NB];
#pragma unroll
  for (int a = 0; a < MB; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;
  // Base term: wave wni squares blocks a = (wni % MB) + i*WN of its rows
  // (every block exactly once when MB >= WN; waves past MB repeat a block
  // and their sums are dropped).
  constexpr int SQB = MB >= WN ? MB / WN : 1;
  float sq[SQB];
#pragma unroll
  for (int i = 0; i < SQB; ++i) sq[i] = 0.f;

  // Stage i of the range (elements k0 + i*KT ..), zero past d_in and past
  // the valid rows.
  auto reg_stage = [&](int i, char* sb) __attribute__((always_inline)) {
    const int cch = tid % CPR, row0 = tid / CPR;
    const int64_t k = k0 + (int64_t)i * KT + (int64_t)cch * EPC;
    u32x4 st[C::CPT];
#pragma unroll
    for (int j = 0; j < C::CPT; ++j) {
      const int row = row0 + j * C::RSTEP;
      if (j < MT / C::RSTEP) {
        st[j] = load_chunk(msrc + (int64_t)row * d_in, k, d_in, row < m_lim, false);
      } else {
        const int nr = row - MT;
        st[j] = load_chunk(nsrc + (int64_t)nr * d_in, k, d_in, nr < n_lim, false);
      }
    }
#pragma unroll
    for (int j = 0; j < C::CPT; ++j) {
      const int row = row0 + j * C::RSTEP;
      *reinterpret_cast<u32x4*>(sb + row * RB + swz<CPR>(row, cch) * 16) = st[j];
    }
  };

  auto load_frags = [&](const char* sb, int ks, u32x4 (&fa)[MB][FC], u32x4 (&fb)[NB][FC],
                        u32x4 (&fs)[SQB][FC]) __attribute__((always_inline)) {
#pragma unroll
    for (int f = 0; f < FC; ++f) {
      const int ch = ks * 2 * FC + lgrp * FC + f;
#pragma unroll
      for (int a = 0; a < MB; ++a) {
        const int row = wmi * MB * 32 + a * 32 + lrow;
        fa[a][f] = *reinterpret_cast<const u32x4*>(sb + row * RB + swz<CPR>(row, ch) * 16);
      }
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int row = MT + wni * NB * 32 + b * 32 + lrow;
        fb[b][f] = *reinterpret_cast<const u32x4*>(sb + row * RB + swz<CPR>(row, ch) * 16);
      }
#pragma unroll
      for (int i = 0; i < SQB; ++i) {
        const int row = wmi * MB * 32 + ((wni % MB) + i * WN) * 32 + lrow;
        fs[i][f] = *reinterpret_cast<const u32x4*>(sb + row * RB + swz<CPR>(row, ch) * 16);
      }
    }
  };
  auto compute = [&](const char* sb) __attribute__((always_inline)) {
    u32x4 fa[2][MB][FC], fb[2][NB][FC], fs[2][SQB][FC];
    load_frags(sb, 0, fa[0], fb[0], fs[0]);
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
      const int c = ks & 1;
      if (ks + 1 < C::KSTEPS) load_frags(sb, ks + 1, fa[c ^ 1], fb[c ^ 1], fs[c ^ 1]);
#pragma unroll
      for (int a = 0; a < MB; ++a)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[a][b] = Mfma<T>::run(fa[c][a], fb[c][b], acc[a][b]);
      if constexpr (!GRAM) {
#pragma unroll
        for (int i = 0; i < SQB; ++i) {
          float qs = 0.f;
#pragma unroll
          for (int f = 0; f < FC; ++f) qs += chunk_sumsq(fs[c][i][f], T());
          sq[i] += qs;
        }
      }
    }
  };

  reg_stage(0, s0);
  __syncthreads();
  int i = 0;
  for (; i + 1 < n_st; i += 2) {
    compute(s0);
    reg_stage(i + 1, s1);
    __syncthreads();
    compute(s1);
    if (i + 2 < n_st) reg_stage(i + 2, s0);
    __syncthreads();
  }
  if (i < n_st) {
    compute(s0);
    __syncthreads();
  }

  if constexpr (!GRAM) {
    float* part_base = reinterpret_cast<float*>(ws + p.off_base);
    float* part_cross = reinterpret_cast<float*>(ws + p.off_cross);
    float* red_c = sred;              // [WN][MT] cross sums of each wave's columns
    float* red_b = sred + WN * MT;    // [MT] base sums
    // Base term: the two k-halves of each row live in lanes l and l+32.
#pragma unroll
    for (int i2 = 0; i2 < SQB; ++i2) {
      const float qs = sq[i2] + __shfl_xor(sq[i2], 32, 64);
      if (wni < MB && lgrp == 0) red_b[wmi * MB * 32 + ((wni % MB) + i2 * WN) * 32 + lrow] = qs;
    }
    // Cross term, one 32-row block of the tile per round: its B rows (the
    // tile's NTC columns) are staged in LDS; the owning waves multiply
    // their accumulators by B and sum over their columns with a lane
    // transpose-reduction.
    for (int rho = 0; rho < C::ROUNDS; ++rho) {
      const int wr = rho / MB, a = rho % MB;
      const int rbase = rho * 32;
      const int rows = m_lim - rbase < 32 ? (m_lim - rbase > 0 ? m_lim - rbase : 0) : 32;
      const T* bsrc = B + (mrow0 + rbase) * p.r + n0;
      for (int qq = tid; qq < 32 * C::CPRB; qq += NT) {
        const int row = qq / C::CPRB, ch = qq % C::CPRB;
        const u32x4 v = load_chunk(bsrc + (int64_t)row * p.r, (int64_t)ch * EPC, p.r - n0, row < rows, false);
        *reinterpret_cast<u32x4*>(s0 + row * C::RBB + ((ch ^ (row & 7)) * 16)) = v;
      }
      __syncthreads();
#pragma unroll
      for (int wr2 = 0; wr2 < WM; ++wr2)
#pragma unroll
        for (int a2 = 0; a2 < MB; ++a2) {
          if (wr2 == wr && a2 == a && wmi == wr) {
            float pa[16];
#pragma unroll
            for (int v = 0; v < 16; ++v) pa[v] = 0.f;
#pragma unroll
            for (int b = 0; b < NB; ++b) {
              const int col = wni * NB * 32 + b * 32 + lrow;
#pragma unroll
              for (int v = 0; v < 16; ++v) {
                const int row = acc_row(v, lgrp);
                const T bv = *reinterpret_cast<const T*>(s0 + row * C::RBB + (((col / EPC) ^ (row & 7)) * 16) +
                                                         (col % EPC) * ESZ);
                pa[v] = fmaf(acc[a2][b][v], to_f32(bv), pa[v]);
              }
            }
            const float tot = sum32_transpose(pa, lane);
            if ((lane & 1) == 0) red_c[wni * MT + rbase + acc_row((lane & 31) >> 1, lgrp)] = tot;
          }
        }
      __syncthreads();
    }
    for (int R = tid; R < MT; R += NT) {
      const int64_t grow = mrow0 + R;
      float cs = 0.f;
#pragma unroll
      for (int wn = 0; wn < WN; ++wn) cs += red_c[wn * MT + R];
      part_cross[((int64_t)x * p.n_nt + n) * p.ld_w + grow] = cs;
      if (n == 0) part_base[(int64_t)x * p.ld_w + grow] = red_b[R];
    }
  } else {
    // G = A A^T partial for rows mrow0.. of A and columns n0.. .
    float* gdst = reinterpret_cast<float*>(ws + p.off_g) + (int64_t)x * p.ga_rows * p.ga_cols;
#pragma unroll
    for (int a = 0; a < MB; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t gi = mrow0 + wmi * MB * 32 + a * 32 + acc_row(v, lgrp);
          const int64_t gj = n0 + wni * NB * 32 + b * 32 + lrow;
          gdst[gi * p.ga_cols + gj] = acc[a][b][v];
        }
  }
}

// ---------------------------------------------------------------------------
// gram_reduce: G[i][j] = sum over the Gram pass's ranges, in range order.
// One thread per element, consecutive j in consecutive lanes.
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ void store_gram(char* ws, const NormPlan& p, int64_t i, int64_t j, float v) {
  const int64_t rg = p.rg;
  if constexpr (sizeof(T) == 2) {
    // Row i of the stored matrix: [hi(G[i][0..rg)), lo(G[i][0..rg))].
    bf16_t* gg = reinterpret_cast<bf16_t*>(ws + p.off_gg) + i * 2 * rg;
    const bf16_t h = f32_to_bf16_rne(v);
    gg[j] = h;
    gg[rg + j] = f32_to_bf16_rne(v - bf16_bits_to_f32(h));
  } else {
    reinterpret_cast<float*>(ws + p.off_gg)[i * rg + j] = v;
  }
}

// One workgroup of 1024 threads per 32 x 32 block (bi, bj) of G on or above
// the diagonal, one element per thread: each element sums its x partials in
// increasing x (kSumBatch planes per round trip), reading only blocks on or
// above the diagonal, which every Gram pass computes. The block is written
// as G[bi][bj] and, off the diagonal, transposed through LDS as G[bj][bi],
// so every global access is along a row. The stored matrix is gscale * G
// (one rounded product per element): s/2 when the W pass runs the Gram term
// in its own accumulators, 1 otherwise.
//
// fp16 with the Gram term in the W pass: the workgroups past the n_red
// reduction blocks split B exactly into bf16 hi + lo (f16_split_bf16) for
// it, into the workspace as [d_out][B_hi | B_lo], each part rg columns wide
// and zero past r.
constexpr int kReduceThreads = 1024;

// Workgroups of the split of B: each covers whole rows, ppr rows per pass
// of 1024 threads (one 8-column chunk per thread), at most kSplitBlocks.
constexpr int kSplitBlocks = 512;
DORA_HD int split_rows_per_pass(int64_t rg) {
  const int64_t cpr = rg / 8;
  return cpr < kReduceThreads ? (int)(kReduceThreads / cpr) : 1;
}
int64_t split_blocks(const NormPlan& p) {
  const int64_t rpp = split_rows_per_pass(p.rg);
  const int64_t n = (p.d_out + rpp - 1) / rpp;
  return n < kSplitBlocks ? n : kSplitBlocks;
}

__device__ void split_b(const NormPlan& p, const f16_t* __restrict__ B, char* __restrict__ ws, int blk, int nblk) {
  const int cpr = (int)(p.rg / 8);                        // 8-column chunks per part
  const int cw = cpr < kReduceThreads ? cpr : kReduceThreads;   // threads across a row
  const int rpp = kReduceThreads / cw;
  const int ro = (int)threadIdx.x / cw, c0 = (int)threadIdx.x - ro * cw;
  if (ro >= rpp) return;
  bf16_t* dst = reinterpret_cast<bf16_t*>(ws + p.off_bf);
  const bool vec = (p.r & 7) == 0 && (reinterpret_cast<uintptr_t>(B) & 15) == 0;
  for (int64_t i = (int64_t)blk * rpp + ro; i < p.d_out; i += (int64_t)nblk * rpp) {
    const f16_t* row = B + i * p.r;
    bf16_t* out = dst + i * 2 * p.rg;
    for (int c8 = c0; c8 < cpr; c8 += cw) {
      const int64_t c = (int64_t)c8 * 8;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (vec) {
        if (c < p.r) v = *reinterpret_cast<const u32x4*>(row + c);
      } else {
        f16x8 h;
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = c + e < p.r ? row[c + e] : (f16_t)0;
        v = __builtin_bit_cast(u32x4, h);
      }
      *reinterpret_cast<u32x4*>(out + c) = f16_split_bf16(v, false);
      *reinterpret_cast<u32x4*>(out + p.rg + c) = f16_split_bf16(v, true);
    }
  }
}

template <typename T>
__global__ __launch_bounds__(kReduceThreads) void gram_reduce_kernel(NormPlan p, char* __restrict__ ws, float gscale,
                                                                     const f16_t* __restrict__ Bsplit, int n_red) {
  constexpr int RG = kReduceThreads / 32;   // row groups; each thread owns 32 / RG rows
  constexpr int RPT = 32 / RG;
  __shared__ float tile[32][33];
  if ((int)blockIdx.x >= n_red) {
    split_b(p, Bsplit, ws, (int)blockIdx.x - n_red, (int)gridDim.x - n_red);
    return;
  }
  if (p.asm_fused && blockIdx.x == 0) {
    // arrival counters of the W pass that follows (which assembles)
    unsigned* cnt = reinterpret_cast<unsigned*>(ws + p.off_cnt);
    const int64_t n_mt = (p.d_out + fast_rows(p.fcfg) - 1) / fast_rows(p.fcfg);
    for (int64_t i = threadIdx.x; i < n_mt; i += kReduceThreads) cnt[i] = 0u;
  }
  int bi, bj;
  tri_tile(blockIdx.x, (int)(p.rg / 32), &bi, &bj);
  const int c = threadIdx.x % 32, grp = threadIdx.x / 32;
  const float* part_g = reinterpret_cast<const float*>(ws + p.off_g);
  const int64_t plane = p.ga_rows * p.ga_cols;
  const int64_t j = (int64_t)bj * 32 + c;
  float acc[RPT];
  const float* src[RPT];
  bool live[RPT];
#pragma unroll
  for (int q = 0; q < RPT; ++q) {
    const int64_t i = (int64_t)bi * 32 + grp + RG * q;
    acc[q] = 0.f;
    live[q] = i < p.r && j < p.r;
    src[q] = part_g + i * p.ga_cols + j;
  }
  for (int x0 = 0; x0 < p.xg; x0 += kSumBatch) {
    float v[RPT][kSumBatch];
#pragma unroll
    for (int q = 0; q < RPT; ++q)
#pragma unroll
      for (int u = 0; u < kSumBatch; ++u)
        v[q][u] = (live[q] && x0 + u < p.xg) ? src[q][(int64_t)(x0 + u) * plane] : 0.f;
#pragma unroll
    for (int q = 0; q < RPT; ++q)
#pragma unroll
      for (int u = 0; u < kSumBatch; ++u)
        if (x0 + u < p.xg) acc[q] += v[q][u];
  }
#pragma unroll
  for (int q = 0; q < RPT; ++q) {
    const int row = grp + RG * q;
    acc[q] = __fmul_rn(acc[q], gscale);
    store_gram<T>(ws, p, (int64_t)bi * 32 + row, j, acc[q]);
    tile[row][c] = acc[q];
  }
  if (bi == bj) return;
  __syncthreads();
#pragma unroll
  for (int q = 0; q < RPT; ++q) {
    const int row = grp + RG * q;   // row of the transposed block: column `row` of the tile
    store_gram<T>(ws, p, (int64_t)bj * 32 + row, (int64_t)bi * 32 + c, tile[c][row]);
  }
}

// ---------------------------------------------------------------------------
// gram_term: ba[j] = sum_l (B G)[j,l] B[j,l], split over 64-column blocks of G.
// Workgroup (row group, column block): the block's 64 rows of G (G is
// symmetric, so they are its columns, K-contiguous) are staged in LDS once
// per K chunk; each wave contracts 32 rows of B with them on the matrix
// cores (bf16: B Ghi + B Glo), dots the result with B's entries in those
// columns, and writes one partial per row and column block.
// ---------------------------------------------------------------------------
template <typename T>
struct GramCfg {
  static constexpr int KC = 192;                          // K chunk staged at once
  static constexpr int NG = sizeof(T) == 2 ? 2 : 1;       // hi and lo parts
  static constexpr int EPC = Elem<T>::epc;
  static constexpr int RBYTES = KC * (int)sizeof(T);      // bytes of one staged G row
  static constexpr int CPRG = RBYTES / 16;                // 16-byte chunks per staged row
  static constexpr int PART = kGramCB * RBYTES;           // bytes of one staged part
  static constexpr int LDS = NG * PART;
  static constexpr int NBLK = LDS / 1024;                 // direct-load blocks per chunk
  static constexpr int WAVES = kGramRows / 32;
  static constexpr int NKS = KC / 16;                     // K16 steps per chunk
  static constexpr int FC = Elem<T>::frag_chunks;
  static_assert(NBLK % WAVES == 0 && PART % 1024 == 0, "staging splits evenly over the waves");
  static_assert(CPRG % 8 == 0, "swizzle stays inside a staged row");
};

template <typename T>
__global__ __launch_bounds__(kGramRows * 2, 1) void gram_term_kernel(NormPlan p, const T* __restrict__ B,
                                                                     char* __restrict__ ws) {
  using C = GramCfg<T>;
  constexpr int EPC = C::EPC, FC = C::FC;
  __shared__ __attribute__((aligned(1024))) char sg[C::LDS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lrow = lane & 31, lgrp = lane >> 5;
  const int64_t r = p.r, rg = p.rg;
  const int64_t c0 = (int64_t)blockIdx.y * kGramCB;
  const int64_t j0 = (int64_t)blockIdx.x * kGramRows + wave * 32;
  const int64_t arow = j0 + lrow;
  const bool arow_ok = arow < p.d_out;
  const T* brow = B + arow * r;
  const bool bvec = p.vec_b != 0;

  // B's entries in this block's columns for the epilogue, fetched up front.
  float bval[2][16];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int64_t col = c0 + q * 32 + lrow;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t row = j0 + acc_row(v, lgrp);
      bval[q][v] = (row < p.d_out && col < r) ? to_f32(B[row * r + col]) : 0.f;
    }
  }

  f32x16 acc[2];
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[q][v] = 0.f;

  for (int64_t k0 = 0; k0 < rg; k0 += C::KC) {
    u32x4 fa[C::NKS][FC];   // this lane's B fragments for the chunk
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks)
#pragma unroll
      for (int f = 0; f < FC; ++f)
        fa[ks][f] = load_chunk(brow, k0 + ks * 16 + (int64_t)(lgrp * FC + f) * EPC, r, arow_ok, bvec);
    __syncthreads();   // the previous chunk is fully consumed
    // Stage rows c0.. of G (hi, lo) for k in [k0, k0 + KC) by direct loads;
    // each lane fetches the chunk that lands on its LDS slot under the swizzle.
#pragma unroll
    for (int i = 0; i < C::NBLK / C::WAVES; ++i) {
      const int blk = i * C::WAVES + wave;
      const int part = blk / (C::PART / 1024);
      const int slot16 = (blk % (C::PART / 1024)) * 64 + lane;
      const int row = slot16 / C::CPRG, ch = (slot16 % C::CPRG) ^ (row & 7);
      int64_t grow = c0 + row, gk = k0 + (int64_t)ch * EPC;
      grow = grow < rg ? grow : rg - 1;          // past the matrix: a real row, never used
      gk = gk < rg ? gk : rg - EPC;
      const char* src = ws + p.off_gg + (grow * C::NG * rg + part * rg + gk) * (int64_t)sizeof(T);
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                       (__attribute__((address_space(3))) void*)(sg + blk * 1024), 16, 0, 0);
    }
    wait_lds_loads();
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int row = q * 32 + lrow;
#pragma unroll
        for (int part = 0; part < C::NG; ++part) {
          u32x4 fb[FC];
#pragma unroll
          for (int f = 0; f < FC; ++f) {
            const int ch = ks * 2 * FC + lgrp * FC + f;
            fb[f] = *reinterpret_cast<const u32x4*>(sg + part * C::PART + row * C::RBYTES + ((ch ^ (row & 7)) * 16));
          }
          acc[q] = Mfma<T>::run(fa[ks], fb, acc[q]);
        }
      }
    }
  }

  // Dot with B's entries in this block's columns, then sum over the columns.
  float pa[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) pa[v] = fmaf(acc[0][v], bval[0][v], acc[1][v] * bval[1][v]);
  const float tot = sum32_transpose(pa, lane);
  const int64_t row = j0 + acc_row((lane & 31) >> 1, lgrp);
  if ((lane & 1) == 0 && row < p.d_out)
    reinterpret_cast<float*>(ws + p.off_ba)[(int64_t)blockIdx.y * p.ld_w + row] = tot;
}

// ---------------------------------------------------------------------------
// assemble: per row, fixed-order sums of the partials, then
// wnorm = sqrt(max(base + 2s cross + s^2 ba, 0)) and g = m / max(wnorm, eps),
// every operation separately rounded (no contraction), sqrt and division
// correctly rounded. One thread per row; reads are coalesced. n_ba = 0 when
// the cross partials already hold cross + (s/2) ba (ba is then 0 here).
// ---------------------------------------------------------------------------
constexpr int kAsmThreads = 256;   // threads per assembly workgroup

// `split` threads per row (a power of two, at most 64): thread q of a row
// sums planes [n q / split, n (q+1) / split) of each kind in increasing
// order, the three kinds in lock step (each batch issues all its loads
// before any addition); then every thread adds its row's split partial sums
// in the order q = 0, 1, ..., and the row's first thread assembles. With
// split = 1 this is the plain sum over the planes in order. The host picks
// the smallest split that leaves each thread one batch of loads, so rows
// with many partials (many d_in ranges or column tiles) are summed by
// several threads at once.
__global__ __launch_bounds__(kAsmThreads) void assemble_kernel(NormPlan p, const char* __restrict__ ws, int n_ba,
                                                               float s, const float* m, float eps, float* wnorm,
                                                               float* g, int split) {
  const int64_t t = (int64_t)blockIdx.x * kAsmThreads + threadIdx.x;
  const int64_t j = t / split;
  const int q = (int)(t % split);
  const bool live = j < p.d_out;
  const float* pb = reinterpret_cast<const float*>(ws + p.off_base) + j;
  const float* pc = reinterpret_cast<const float*>(ws + p.off_cross) + j;
  const float* pa = reinterpret_cast<const float*>(ws + p.off_ba) + j;
  const int nb = p.xw, nc = p.xw * p.n_nt, na = n_ba;
  const int b0 = nb * q / split, b1 = nb * (q + 1) / split;
  const int c0 = nc * q / split, c1 = nc * (q + 1) / split;
  const int a0 = na * q / split, a1 = na * (q + 1) / split;
  const int len = (b1 - b0) > (c1 - c0) ? ((b1 - b0) > (a1 - a0) ? b1 - b0 : a1 - a0)
                                        : ((c1 - c0) > (a1 - a0) ? c1 - c0 : a1 - a0);
  float base = 0.f, cross = 0.f, ba = 0.f;
  for (int i = 0; i < len; i += kSumBatch) {
    float vb[kSumBatch], vc[kSumBatch], va[kSumBatch];
#pragma unroll
    for (int u = 0; u < kSumBatch; ++u) {
      vb[u] = (live && b0 + i + u < b1) ? pb[(int64_t)(b0 + i + u) * p.ld_w] : 0.f;
      vc[u] = (live && c0 + i + u < c1) ? pc[(int64_t)(c0 + i + u) * p.ld_w] : 0.f;
      va[u] = (live && a0 + i + u < a1) ? pa[(int64_t)(a0 + i + u) * p.ld_w] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kSumBatch; ++u) {
      if (b0 + i + u < b1) base += vb[u];
      if (c0 + i + u < c1) cross += vc[u];
      if (a0 + i + u < a1) ba += va[u];
    }
  }
  if (split > 1) {
    // The row's threads are consecutive lanes of one wave.
    const int first = (int)(threadIdx.x & 63) - q;
    float tb = __shfl(base, first, 64), tc = __shfl(cross, first, 64), ta = __shfl(ba, first, 64);
    for (int i = 1; i < split; ++i) {
      tb += __shfl(base, first + i, 64);
      tc += __shfl(cross, first + i, 64);
      ta += __shfl(ba, first + i, 64);
    }
    base = tb, cross = tc, ba = ta;
  }
  if (live && q == 0) assemble_sums(base, cross, ba, s, eps, m, wnorm, g, j);
}

hipError_t launched(hipStream_t st, Marks& mk);

// assemble_kernel over all rows, with the smallest split (threads per row)
// that leaves each thread at most one batch of kSumBatch planes per kind.
hipError_t launch_assemble(const NormPlan& p, const char* ws, int n_ba, float s, const float* m, float eps,
                           float* wnorm, float* g, hipStream_t st, Marks& mk) {
  const int nc = p.xw * p.n_nt;
  const int n = p.xw > nc ? (p.xw > n_ba ? p.xw : n_ba) : (nc > n_ba ? nc : n_ba);
  int split = 1;
  while (split < 64 && (n + split - 1) / split > kSumBatch) split *= 2;
  const int64_t threads = p.d_out * split;
  hipLaunchKernelGGL(assemble_kernel, dim3((unsigned)((threads + kAsmThreads - 1) / kAsmThreads)), dim3(kAsmThreads),
                     0, st, p, ws, n_ba, s, m, eps, wnorm, g, split);
  return launched(st, mk);
}

// ---------------------------------------------------------------------------
// Row sum of squares only (s == 0, r == 0 or d_in == 0): one workgroup per
// row.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads) void norm_rowonly_kernel(const T* __restrict__ W, int64_t d_in, bool vec,
                                                                const float* m, float eps, float* wnorm,
                                                                float* g) {
  constexpr int EPC = Elem<T>::epc;
  __shared__ float wsum[4];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const T* wr = W + row * d_in;
  float acc = 0.f;
  for (int64_t k = (int64_t)tid * EPC; k < d_in; k += (int64_t)kThreads * EPC)
    acc += chunk_sumsq(load_chunk(wr, k, d_in, true, vec), T());
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if ((tid & 63) == 0) wsum[tid >> 6] = acc;
  __syncthreads();
  if (tid == 0) {
    float v = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
    v = (v < 0.f) ? 0.f : v;
    const float wn = sqrtf(v);
    wnorm[row] = wn;
    if (m != nullptr) {
      const float d = (wn < eps) ? eps : wn;
      g[row] = m[row] / d;
    }
  }
}

__global__ __launch_bounds__(kThreads) void magnitude_kernel(const float* m, const float* wnorm, float eps,
                                                             int64_t n, float* g) {
  const int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (j >= n) return;
  const float wn = wnorm[j];
  const float d = (wn < eps) ? eps : wn;
  g[j] = m[j] / d;
}

// out[j] = wnorm[j] rounded to the storage type (round to nearest even),
// the cast that ends Algorithm 1 ("DoRA优化技术解析", cyqw.cn, §5.1, step 7).
template <typename T>
__global__ __launch_bounds__(kThreads) void cast_kernel(const float* wnorm, int64_t n, T* out) {
  const int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (j < n) out[j] = from_f32<T>(wnorm[j]);
}

// out[i] = in[i] as fp32 (exact).
__global__ __launch_bounds__(kThreads) void widen_kernel(const f16_t* in, int64_t n, float* out) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i < n) out[i] = (float)in[i];
}

int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Timing marks of one norm call (dora_factored_norm_marked): event 0 on the
// stream before the call's first launch, event i after its i-th launch, for
// as many events as the caller gave, null entries skipped. Local to the call.
hipError_t record_mark(Marks& mk, int i, hipStream_t st) {
  return (i < mk.n && mk.ev[i] != nullptr) ? hipEventRecord(mk.ev[i], st) : hipSuccess;
}

hipError_t begin_marks(Marks& mk, hipStream_t st) {
  mk.next = 1;
  return record_mark(mk, 0, st);
}

// The status of the launch just made, and its end marker if one is due.
hipError_t launched(hipStream_t st, Marks& mk) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return record_mark(mk, mk.next++, st);
}

template <typename T, int WM, int WN, int MB, int NB, int KT, int NS, int MODE>
hipError_t launch_fast(const NormPlan& p, const void* M, const void* A, const void* B, char* ws,
                       const AssembleArgs& aa, hipStream_t st, Marks& mk) {
  using C = FastK<T, WM, WN, MB, NB, KT, NS>;
  int64_t grid;
  if (MODE == kPassBG) {
    grid = ceil_div64(p.d_out, C::MT) * p.n_bt;   // n_bt * NTC covers rg
  } else {
    const bool gram = MODE == kPassGram;
    const int64_t rows = gram ? p.r : p.d_out;
    const int64_t cols = gram ? p.ga_cols : (int64_t)p.n_nt * p.ntc;
    const int64_t tiles = (gram && C::MT == C::NTC && p.gsym) ? tri_count(cols / C::NTC)
                                                               : ceil_div64(rows, C::MT) * (cols / C::NTC);
    grid = (gram ? p.xg : p.xw) * tiles;
  }
  hipLaunchKernelGGL((norm_fast_kernel<T, WM, WN, MB, NB, KT, NS, MODE>), dim3((unsigned)grid), dim3(C::NT), 0, st,
                     p, static_cast<const T*>(M), static_cast<const T*>(A), static_cast<const T*>(B), ws, aa);
  return launched(st, mk);
}

template <typename T, int WM, int WN, int MB, int NB, int KT, bool GRAM>
hipError_t launch_gen(const NormPlan& p, const void* M, const void* A, const void* B, char* ws, hipStream_t st, Marks& mk) {
  using C = GenK<T, WM, WN, MB, NB, KT>;
  const int64_t rows = GRAM ? p.r : p.d_out;
  const int64_t cols = GRAM ? p.ga_cols : (int64_t)p.n_nt * p.ntc;
  const int64_t grid = (GRAM ? p.xg : p.xw) * ceil_div64(rows, C::MT) * (cols / C::NTC);
  hipLaunchKernelGGL((norm_gen_kernel<T, WM, WN, MB, NB, KT, GRAM>), dim3((unsigned)grid), dim3(C::NT), 0, st, p,
                     static_cast<const T*>(M), static_cast<const T*>(A), static_cast<const T*>(B), ws);
  return launched(st, mk);
}

// H is the 16-bit storage type (bf16 or fp16); fp32 uses the F* configurations.
template <int MODE, typename H>
hipError_t launch_pass(const NormPlan& p, int fcfg, int gcfg, const void* M, const void* A, const void* B,
                       char* ws, hipStream_t st, Marks& mk, const AssembleArgs& aa = AssembleArgs{}) {
  constexpr bool GRAM = MODE == kPassGram;
  if (p.fast) {
    // The Gram pass only uses these configurations (64 and 128 columns).
    switch (fcfg) {
      case kFastB64: return launch_fast<H, 4, 2, 1, 1, 64, 4, MODE>(p, M, A, B, ws, aa, st, mk);
      case kFastB128: return launch_fast<H, 2, 4, 2, 1, 64, 4, MODE>(p, M, A, B, ws, aa, st, mk);
      case kFastG64: return launch_fast<H, 2, 2, 1, 1, 64, 4, MODE>(p, M, A, B, ws, aa, st, mk);
      case kFastF32: return launch_fast<float, 4, 1, 1, 1, 32, 4, MODE>(p, M, A, B, ws, aa, st, mk);
      case kFastF128: return launch_fast<float, 2, 4, 2, 1, 32, 4, MODE>(p, M, A, B, ws, aa, st, mk);
      default: break;
    }
    if constexpr (!GRAM) {
      switch (fcfg) {
        case kFastT64: return launch_fast<H, 4, 2, 2, 1, 64, 3, MODE>(p, M, A, B, ws, aa, st, mk);
        case kFastT128: return launch_fast<H, 4, 2, 2, 2, 64, 3, MODE>(p, M, A, B, ws, aa, st, mk);
        case kFastB256: return launch_fast<H, 2, 4, 2, 2, 64, 3, MODE>(p, M, A, B, ws, aa, st, mk);
        case kFastT192: return launch_fast<H, 4, 2, 2, 3, 64, 2, MODE>(p, M, A, B, ws, aa, st, mk);
        case kFastT384:
          if constexpr (MODE == kPassWG) return hipErrorInvalidValue;   // never planned
          else return launch_fast<H, 2, 4, 4, 3, 64, 2, MODE>(p, M, A, B, ws, aa, st, mk);
        case kFastT256:
          if constexpr (MODE == kPassWG) return hipErrorInvalidValue;   // never planned
          else return launch_fast<H, 4, 2, 2, 4, 64, 2, MODE>(p, M, A, B, ws, aa, st, mk);
        default: break;
      }
    }
    return hipErrorInvalidValue;
  }
  if constexpr (MODE == kPassWG || MODE == kPassWB) {
    return hipErrorInvalidValue;   // the general kernel never takes G or the Gram term in
  } else {
    switch (gcfg) {
      case kGenB64: return launch_gen<H, 2, 2, 2, 1, 64, GRAM>(p, M, A, B, ws, st, mk);
      case kGenB128: return launch_gen<H, 1, 4, 4, 1, 64, GRAM>(p, M, A, B, ws, st, mk);
      case kGenB256: return launch_gen<H, 1, 4, 4, 2, 64, GRAM>(p, M, A, B, ws, st, mk);
      case kGenT192: return launch_gen<H, 4, 2, 2, 3, 64, GRAM>(p, M, A, B, ws, st, mk);
      case kGenF32: return launch_gen<float, 4, 1, 1, 1, 32, GRAM>(p, M, A, B, ws, st, mk);
      case kGenF128: return launch_gen<float, 1, 4, 4, 1, 32, GRAM>(p, M, A, B, ws, st, mk);
      default: return hipErrorInvalidValue;
    }
  }
}

template <int MODE>
hipError_t launch_pass(const NormPlan& p, int fcfg, int gcfg, const void* M, const void* A, const void* B,
                       char* ws, hipStream_t st, Marks& mk, const AssembleArgs& aa = AssembleArgs{}) {
  return p.dtype == 2 ? launch_pass<MODE, f16_t>(p, fcfg, gcfg, M, A, B, ws, st, mk, aa)
                      : launch_pass<MODE, bf16_t>(p, fcfg, gcfg, M, A, B, ws, st, mk, aa);
}

template <typename T>
hipError_t launch_tail(const NormPlan& p, const void* B, char* ws, float s, const float* m, float eps,
                       float* wnorm, float* g, hipStream_t st, Marks& mk) {
  if (p.fast) {
    // Gram term on the matrix cores; with one column tile the assembly is
    // fused in, otherwise a small kernel adds the column-tile partials.
    const AssembleArgs aa{s, eps, m, wnorm, g};
    hipError_t e;
    if constexpr (sizeof(T) == 2) {
      switch (p.bcfg) {
        case 1: e = launch_fast<bf16_t, 2, 4, 1, 1, 64, 2, kPassBG>(p, B, nullptr, B, ws, aa, st, mk); break;
        case 2: e = launch_fast<bf16_t, 2, 4, 1, 2, 64, 2, kPassBG>(p, B, nullptr, B, ws, aa, st, mk); break;
        case 3: e = launch_fast<bf16_t, 2, 4, 1, 3, 64, 2, kPassBG>(p, B, nullptr, B, ws, aa, st, mk); break;
        default: return hipErrorInvalidValue;
      }
    } else {
      e = launch_fast<float, 2, 4, 1, 1, 32, 2, kPassBG>(p, B, nullptr, B, ws, aa, st, mk);
    }
    if (e != hipSuccess || p.n_bt == 1) return e;
    return launch_assemble(p, ws, p.n_bt, s, m, eps, wnorm, g, st, mk);
  }
  hipLaunchKernelGGL((gram_term_kernel<T>), dim3((unsigned)((p.d_out + kGramRows - 1) / kGramRows), (unsigned)p.n_cb),
                     dim3(kGramRows * 2), 0, st, p, static_cast<const T*>(B), ws);
  hipError_t e = launched(st, mk);
  if (e != hipSuccess) return e;
  return launch_assemble(p, ws, p.n_cb, s, m, eps, wnorm, g, st, mk);
}

}  // namespace

// ---------------------------------------------------------------------------
// Dense fused row norm, for r >= d_out or r > d_in (16-bit types): per tile of
// kDenseMT rows by kDenseNT columns of d_in, the tile of W + s B A is formed
// in the accumulators and squared, and its row sums are stored as one
// partial per (column tile, row); a second kernel adds each row's partials
// in column-tile order and takes the root. The definition itself
// ("DoRA优化技术解析", cyqw.cn, §1.1: ||W + s B A||_row), never materialised:
// where r >= d_out, the factored form's Gram matrix A A^T (r^2 d_in
// multiply-adds) outweighs B A (d_out r d_in), and where r > d_in its Gram
// term B G (d_out r^2) does, so this path does less work and needs no Gram
// reduction.
//
// Workgroup = NW waves (2 x NW/2), each owning 32 rows and 128 / (NW/2)
// columns of the tile in 32x32 accumulator blocks. The
// depth r goes through a ring of kDenseNS LDS slots, kDenseKT = 64 deep per
// stage: B's tile rows (128 bytes each, swizzled like the W pass's rows)
// and A's k-rows (kDenseNT columns, 16-byte chunks XOR-swizzled by 2 (k & 3)
// so the transposed reads below hit distinct banks). A row-major A is
// k-major for B A; each lane's column-operand fragment (8 consecutive k of
// one column) is read with two ds_read_b64_tr_b16: in each 16-lane group,
// lane m points at k-row m / 4 and columns 4 (m % 4) + [0, 4), and lane i
// receives the 4 k-rows of column i. W's tile (64 rows x 256 bytes, chunks
// XOR-swizzled by row & 15) is loaded first and enters the accumulator
// layout in the epilogue through selector MFMAs, as B does in the W pass.
// ---------------------------------------------------------------------------
typedef short short4v __attribute__((ext_vector_type(4)));
constexpr int kDenseMT = kDenseRows, kDenseNT = kDenseCols, kDenseKT = 64, kDenseNS = 6;
constexpr int kDenseWaves = 8;
constexpr int kDenseBBytes = kDenseMT * kDenseKT * 2;     // B part of a stage (8 KiB)
constexpr int kDenseABytes = kDenseKT * kDenseNT * 2;     // A part of a stage (16 KiB)
constexpr int kDenseSlot = kDenseBBytes + kDenseABytes;
constexpr int kDenseWBytes = kDenseMT * kDenseNT * 2;     // W tile (16 KiB)
static_assert(kDenseNS * kDenseSlot + kDenseWBytes <= 160 * 1024, "gfx950 has 160 KiB of LDS");

template <typename T, int NW>
__global__ __launch_bounds__(NW * 64, 1) void norm_dense_kernel(NormPlan p, const T* __restrict__ W,
                                                                      const T* __restrict__ A,
                                                                      const T* __restrict__ B, float s,
                                                                      float* __restrict__ part) {
  static_assert(sizeof(T) == 2, "16-bit types");
  // NW waves as 2 x WN; wave (wm, wn) owns rows 32 wm + [0, 32) and NBW
  // 32-column blocks from column 32 NBW wn.
  constexpr int WN = NW / 2, NBW = kDenseNT / 32 / WN;
  constexpr int BPW = kDenseSlot / 1024 / NW;                 // direct-load blocks per wave per stage
  constexpr int WPW = kDenseWBytes / 1024 / NW;               // W-tile blocks per wave
  static_assert(NW == 4 || NW == 8, "four or eight waves");
  static_assert(BPW * (kDenseNS - 1) + WPW < 64, "outstanding loads fit vmcnt");
  __shared__ __attribute__((aligned(1024))) char lds[kDenseNS * kDenseSlot + kDenseWBytes];
  char* const wt = lds + kDenseNS * kDenseSlot;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN, lrow = lane & 31, lgrp = lane >> 5;

  // Tile: all row tiles of one column tile run on one die (die = blockIdx
  // mod kDies), so A's columns come from memory once per die.
  const int die = blockIdx.x % kDies, u = blockIdx.x / kDies;
  const int rt = u % p.dn_rt, ct = (u / p.dn_rt) * kDies + die;
  if (ct >= p.dn_ct) return;   // (the grid rounds the column tiles up to whole dies)
  const int64_t i0 = (int64_t)rt * kDenseMT, j0 = (int64_t)ct * kDenseNT;
  const int64_t d_in = p.d_in, r = p.r;
  const int rows = p.d_out - i0 < kDenseMT ? (int)(p.d_out - i0) : kDenseMT;   // valid rows of the tile
  const int64_t cols = d_in - j0;                                              // valid columns past j0
  // Descriptors over the tile's rows: rows past them read as zeros.
  const __amdgpu_buffer_rsrc_t brs = make_rsrc(B + i0 * r, (uint32_t)(rows * r * 2));
  const __amdgpu_buffer_rsrc_t ars = make_rsrc(A + j0, (uint32_t)((r * d_in - j0) * 2));
  const __amdgpu_buffer_rsrc_t wrs = make_rsrc(W + i0 * d_in + j0, (uint32_t)((rows * d_in - j0) * 2));
  const int n_st = (int)((r + kDenseKT - 1) / kDenseKT);

  // Stage t into slot `sl`: block q of a stage (q = wave + NW n) is B rows
  // 8q + [0, 8) for q < 8, else A k-rows 4 (q - 8) + [0, 4). Chunks past r or
  // d_in, and stages past the depth, read as zeros.
  auto issue = [&](int t, char* sl) __attribute__((always_inline)) {
    const int64_t k0 = (int64_t)t * kDenseKT;
    const bool in = t < n_st;
#pragma unroll
    for (int n = 0; n < BPW; ++n) {
      const int q = wave + NW * n;
      uint32_t off;
      if (q < 8) {
        const int row = q * 8 + (lane >> 3);
        const int c = (lane & 7) ^ ((row >> 1) & 7);
        const int64_t k = k0 + c * 8;
        off = (in && k < r) ? (uint32_t)(row * r + k) * 2u : kOob;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(brs, (__attribute__((address_space(3))) void*)(sl + q * 1024), 16,
                                                 off, 0, 0, 0);
      } else {
        const int kr = (q - 8) * 4 + (lane >> 4);
        const int c = (lane & 15) ^ (2 * (kr & 3));
        off = (in && c * 8 < cols) ? (uint32_t)((k0 + kr) * d_in + c * 8) * 2u : kOob;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ars, (__attribute__((address_space(3))) void*)(sl + q * 1024), 16,
                                                 off, 0, 0, 0);
      }
    }
  };
  // W's tile: block q = wave + NW n holds rows 4q + [0, 4).
#pragma unroll
  for (int n = 0; n < WPW; ++n) {
    const int q = wave + NW * n;
    const int row = q * 4 + (lane >> 4);
    const int c = (lane & 15) ^ (row & 15);
    const uint32_t off = c * 8 < cols ? (uint32_t)(row * d_in + c * 8) * 2u : kOob;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, (__attribute__((address_space(3))) void*)(wt + q * 1024), 16, off,
                                             0, 0, 0);
  }
  auto slot = [&](int t) __attribute__((always_inline)) -> char* { return lds + (t % kDenseNS) * kDenseSlot; };
#pragma unroll
  for (int t = 0; t < kDenseNS; ++t) issue(t, slot(t));
  wait_vm_lgkm0<(kDenseNS - 1) * BPW>();   // W's tile and stage 0 complete
  barrier_keep_loads();

  // Fragments of K16 step st of a stage: X = B rows (16 bytes), Y[b] = A's
  // columns 32 (NBW wn + b) + (lane mod 32), 8 consecutive k each.
  struct Frag {
    u32x4 x, y[NBW];
  };
  const int m16 = lane & 15, g16 = lane >> 4;
  const int kq = 8 * (g16 >> 1) + (m16 >> 2);            // k-row within a step (before + 4 h)
  const int jq = 16 * (g16 & 1) + 4 * (m16 & 3);         // column within a 32-column block
  auto read = [&](const char* sl, int st, Frag& F) __attribute__((always_inline)) {
    const int row = wm * 32 + lrow;
    F.x = *reinterpret_cast<const u32x4*>(sl + row * 128 + (((2 * st + lgrp) ^ ((row >> 1) & 7)) * 16));
#pragma unroll
    for (int b = 0; b < NBW; ++b) {
      const int jj = (wn * NBW + b) * 32 + jq;
      short4v h[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int kr = 16 * st + kq + 4 * hh;
        const int phys = (jj >> 3) ^ (2 * (kr & 3));
        h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) short4v*)(sl + kDenseBBytes + kr * (kDenseNT * 2) + phys * 16 + (jj & 7) * 2));
      }
      F.y[b] = u32x4{(uint32_t)(uint16_t)h[0][0] | ((uint32_t)(uint16_t)h[0][1] << 16),
                     (uint32_t)(uint16_t)h[0][2] | ((uint32_t)(uint16_t)h[0][3] << 16),
                     (uint32_t)(uint16_t)h[1][0] | ((uint32_t)(uint16_t)h[1][1] << 16),
                     (uint32_t)(uint16_t)h[1][2] | ((uint32_t)(uint16_t)h[1][3] << 16)};
    }
  };
  f32x16 acc[NBW];
#pragma unroll
  for (int b = 0; b < NBW; ++b)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[b][v] = 0.f;
  Frag F[2];
  read(slot(0), 0, F[0]);
  for (int i = 0; i < n_st; ++i) {
    char* cur = slot(i);
#pragma unroll
    for (int st = 0; st < kDenseKT / 16; ++st) {
      if (st + 1 < kDenseKT / 16) {
        read(cur, st + 1, F[(st + 1) & 1]);
      } else {
        wait_vm_lgkm0<(kDenseNS - 2) * BPW>();   // stage i+1 landed; later stages in flight
        barrier_keep_loads();
        issue(i + kDenseNS, cur);
        if (i + 1 < n_st) read(slot(i + 1), 0, F[0]);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int b = 0; b < NBW; ++b) acc[b] = Mfma<T>::run(&F[st & 1].x, &F[st & 1].y[b], acc[b]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  wait_vm_lgkm0<0>();   // the trailing (zero) stages land before the ring is reused
  barrier_keep_loads();

  // Epilogue: W's 32x32 blocks in the accumulator layout (two MFMAs each
  // against 0/1 selectors, exact), then sum over this wave's columns of
  // (W + s (B A))^2 per row, across the 32 column lanes, then the WN
  // column waves in order.
  const uint32_t one = __is_same(T, bf16_t) ? 0x3F80u : 0x3C00u;
  u32x4 E[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int e = lrow - 8 * lgrp - 16 * h;
#pragma unroll
    for (int w = 0; w < 4; ++w) E[h][w] = (e == 2 * w ? one : 0u) | ((e == 2 * w + 1 ? one : 0u) << 16);
  }
  float pa[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) pa[v] = 0.f;
#pragma unroll
  for (int b = 0; b < NBW; ++b) {
    const int row = wm * 32 + lrow;
    u32x4 f[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = ((wn * NBW + b) * 32 + 16 * h) / 8 + lgrp;
      f[h] = *reinterpret_cast<const u32x4*>(wt + row * (kDenseNT * 2) + ((c ^ (row & 15)) * 16));
    }
    f32x16 wb;
#pragma unroll
    for (int v = 0; v < 16; ++v) wb[v] = 0.f;
    wb = Mfma<T>::run(&f[0], &E[0], wb);
    wb = Mfma<T>::run(&f[1], &E[1], wb);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float val = fmaf(s, acc[b][v], wb[v]);
      pa[v] = fmaf(val, val, pa[v]);
    }
  }
  const float tot = sum32_transpose(pa, lane);
  float* red = reinterpret_cast<float*>(lds);   // (the ring is free)
  if ((lane & 1) == 0) red[wn * kDenseMT + wm * 32 + acc_row((lane & 31) >> 1, lgrp)] = tot;
  __syncthreads();
  if (tid < rows) {
    float t = red[tid];
#pragma unroll
    for (int q = 1; q < WN; ++q) t += red[q * kDenseMT + tid];
    part[(int64_t)ct * p.ld_d + i0 + tid] = t;
  }
}

// wnorm[j] = sqrt of the sum of row j's column-tile partials, added in
// column-tile order, and g (the same assembly as the factored path's with
// the cross and Gram terms zero).
__global__ __launch_bounds__(kThreads) void assemble_dense_kernel(NormPlan p, const float* __restrict__ part,
                                                                  float s, const float* m, float eps, float* wnorm,
                                                                  float* g) {
  const int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (j >= p.d_out) return;
  const float tot = ordered_sum(part + j, p.ld_d, p.dn_ct);
  assemble_sums(tot, 0.f, 0.f, s, eps, m, wnorm, g, j);
}

hipError_t launch_norm_dense(const NormPlan& p, const void* W, const void* A, const void* B, void* ws_, float s,
                             const float* m, float eps, float* wnorm, float* g, hipStream_t st,
                             const hipEvent_t* events, int n_events) {
  char* ws = static_cast<char*>(ws_);
  float* part = reinterpret_cast<float*>(ws + p.off_dense);
  Marks mk{events, events != nullptr ? n_events : 0, 0};
  hipError_t e = begin_marks(mk, st);
  if (e != hipSuccess) return e;
  const unsigned grid = (unsigned)((int64_t)p.dn_rt * ((p.dn_ct + kDies - 1) / kDies) * kDies);
  constexpr int NW = kDenseWaves;
  if (p.dtype == 0)
    hipLaunchKernelGGL((norm_dense_kernel<bf16_t, NW>), dim3(grid), dim3(NW * 64), 0, st,
                       p, static_cast<const bf16_t*>(W), static_cast<const bf16_t*>(A),
                       static_cast<const bf16_t*>(B), s, part);
  else
    hipLaunchKernelGGL((norm_dense_kernel<f16_t, NW>), dim3(grid), dim3(NW * 64), 0, st,
                       p, static_cast<const f16_t*>(W), static_cast<const f16_t*>(A),
                       static_cast<const f16_t*>(B), s, part);
  e = launched(st, mk);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(assemble_dense_kernel, dim3((unsigned)((p.d_out + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                     st, p, part, s, m, eps, wnorm, g);
  return launched(st, mk);
}

hipError_t launch_norm_factored(const NormPlan& p, const void* W, const void* A, const void* B, void* ws_,
                                float s, const float* m, float eps, float* wnorm, float* g,
                                hipStream_t st, const hipEvent_t* events, int n_events) {
  char* ws = static_cast<char*>(ws_);
  Marks mk{events, events != nullptr ? n_events : 0, 0};
  const bool fold = p.fast && p.gfold;
  // On the streaming path the Gram term runs in the W pass's accumulators
  // against (s/2) G: bf16 and fp16 against its bf16 hi + lo parts (fp16
  // splitting B's fragments into bf16 hi + lo as well), fp32 against fp32.
  const bool fuse = p.fast && !p.gfold;
  hipError_t e = begin_marks(mk, st);
  if (e != hipSuccess) return e;
  if (fold) {
    e = launch_pass<kPassWG>(p, p.fcfg, p.gcfg, W, A, B, ws, st, mk);   // W pass with G folded in
  } else {
    e = launch_pass<kPassGram>(p, p.fcfg_g, p.gcfg_g, A, A, B, ws, st, mk);   // Gram pass
  }
  if (e != hipSuccess) return e;
  NormPlan q = p;
  if (fold) q.xg = p.xw;   // one Gram partial per W-pass range
  // The W pass assembles only when its workgroups run in one round and each
  // row has at most one batch of partials: every workgroup then waits once
  // for its partial stores to reach the device and for its count, against
  // the separate assembly launch that saves; over several rounds those
  // waits add up, and with many partials per row one thread per row sums
  // them too slowly.
  const int64_t w_grid = (int64_t)p.xw * ((p.d_out + fast_rows(p.fcfg) - 1) / fast_rows(p.fcfg)) * p.n_nt;
  const bool asm_in_w = fuse && w_grid <= kGrid && (int64_t)p.xw * p.n_nt <= kSumBatch;
  q.asm_fused = asm_in_w ? 1 : 0;   // the reduction zeroes the W pass's arrival counters
  // G is kept as bf16 hi + lo for the bf16 Gram term (bf16, and fp16 with
  // the Gram term in the W pass), in fp32 otherwise (fp32, and fp16's own
  // Gram-term pass, which runs in fp32 on B widened: fp16's range cannot
  // hold every G).
  // (fp16 with the Gram term in the W pass: B's split rides along.)
  const bool split = fuse && p.dtype == 2;
  const int64_t n_red = tri_count(p.rg / 32);
  const int64_t n_split = split ? split_blocks(p) : 0;
  hipLaunchKernelGGL((p.dtype == 0 || split) ? gram_reduce_kernel<bf16_t> : gram_reduce_kernel<float>,
                     dim3((unsigned)(n_red + n_split)), dim3(kReduceThreads), 0, st, q, ws, fuse ? 0.5f * s : 1.0f,
                     split ? static_cast<const f16_t*>(B) : nullptr, (int)n_red);
  e = launched(st, mk);
  if (e != hipSuccess) return e;
  if (fuse) {
    // W pass with the Gram term; its cross partials hold cross + (s/2) ba,
    // and (asm_in_w) the last workgroup of each row tile assembles wnorm
    // and g, else the assembly kernel follows.
    NormPlan pw = p;
    pw.asm_fused = asm_in_w ? 1 : 0;
    e = launch_pass<kPassWB>(pw, p.fcfg, p.gcfg, W, A, B, ws, st, mk, AssembleArgs{s, eps, m, wnorm, g});
    if (e != hipSuccess || asm_in_w) return e;
    return launch_assemble(p, ws, 0, s, m, eps, wnorm, g, st, mk);
  }
  if (!fold) {
    e = launch_pass<kPassW>(p, p.fcfg, p.gcfg, W, A, B, ws, st, mk);   // W pass
    if (e != hipSuccess) return e;
  }
  if (p.dtype == 0) return launch_tail<bf16_t>(p, B, ws, s, m, eps, wnorm, g, st, mk);
  if (p.dtype == 2) {
    // fp16: the Gram term runs in fp32 on B widened (exactly) into the workspace.
    float* Bf = reinterpret_cast<float*>(ws + p.off_bf);
    const int64_t nB = p.d_out * p.r;
    hipLaunchKernelGGL(widen_kernel, dim3((unsigned)((nB + kThreads - 1) / kThreads)), dim3(kThreads), 0, st,
                       static_cast<const f16_t*>(B), nB, Bf);
    e = launched(st, mk);
    if (e != hipSuccess) return e;
    return launch_tail<float>(p, Bf, ws, s, m, eps, wnorm, g, st, mk);
  }
  return launch_tail<float>(p, B, ws, s, m, eps, wnorm, g, st, mk);
}

hipError_t launch_norm_rowonly(const void* W, int dtype, int64_t d_out, int64_t d_in, bool vec, const float* m,
                               float eps, float* wnorm, float* g, hipStream_t st, const hipEvent_t* events,
                               int n_events) {
  Marks mk{events, events != nullptr ? n_events : 0, 0};
  const hipError_t e = begin_marks(mk, st);
  if (e != hipSuccess) return e;
  if (dtype == 0)
    hipLaunchKernelGGL((norm_rowonly_kernel<bf16_t>), dim3((unsigned)d_out), dim3(kThreads), 0, st,
                       static_cast<const bf16_t*>(W), d_in, vec, m, eps, wnorm, g);
  else if (dtype == 2)
    hipLaunchKernelGGL((norm_rowonly_kernel<f16_t>), dim3((unsigned)d_out), dim3(kThreads), 0, st,
                       static_cast<const f16_t*>(W), d_in, vec, m, eps, wnorm, g);
  else
    hipLaunchKernelGGL((norm_rowonly_kernel<float>), dim3((unsigned)d_out), dim3(kThreads), 0, st,
                       static_cast<const float*>(W), d_in, vec, m, eps, wnorm, g);
  return launched(st, mk);
}

hipError_t launch_magnitude(const float* m, const float* wnorm, float eps, int64_t n, float* g, hipStream_t st) {
  hipLaunchKernelGGL(magnitude_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0, st, m,
                     wnorm, eps, n, g);
  return hipGetLastError();
}

hipError_t launch_cast(const float* wnorm, int64_t n, int dtype, void* out, hipStream_t st) {
  const dim3 grid((unsigned)((n + kThreads - 1) / kThreads));
  if (dtype == 0)
    hipLaunchKernelGGL(cast_kernel<bf16_t>, grid, dim3(kThreads), 0, st, wnorm, n, static_cast<bf16_t*>(out));
  else if (dtype == 2)
    hipLaunchKernelGGL(cast_kernel<f16_t>, grid, dim3(kThreads), 0, st, wnorm, n, static_cast<f16_t*>(out));
  else
    hipLaunchKernelGGL(cast_kernel<float>, grid, dim3(kThreads), 0, st, wnorm, n, static_cast<float*>(out));
  return hipGetLastError();
}

size_t fast_kernel_lds_bytes(int cfg) {
#define DORA_LDS(NS, ...)                                                                        \
  (size_t)(FastK<__VA_ARGS__, NS>::SLOT * NS + FastK<__VA_ARGS__, NS>::WX * FastK<__VA_ARGS__, NS>::WB + \
           FastK<__VA_ARGS__, NS>::REDB)
  switch (cfg) {
    case kFastB64: return DORA_LDS(4, bf16_t, 4, 2, 1, 1, 64);
    case kFastB128: return DORA_LDS(4, bf16_t, 2, 4, 2, 1, 64);
    case kFastG64: return DORA_LDS(4, bf16_t, 2, 2, 1, 1, 64);
    case kFastB256: return DORA_LDS(3, bf16_t, 2, 4, 2, 2, 64);
    case kFastT64: return DORA_LDS(3, bf16_t, 4, 2, 2, 1, 64);
    case kFastT128: return DORA_LDS(3, bf16_t, 4, 2, 2, 2, 64);
    case kFastT192: return DORA_LDS(2, bf16_t, 4, 2, 2, 3, 64);
    case kFastT256: return DORA_LDS(2, bf16_t, 4, 2, 2, 4, 64);
    case kFastT384: return (size_t)FastK<bf16_t, 2, 4, 4, 3, 64, 2>::SLOT * 2;   // row sums inside the ring
    case kFastF32: return DORA_LDS(4, float, 4, 1, 1, 1, 32);
    case kFastF128: return DORA_LDS(4, float, 2, 4, 2, 1, 32);
    default: return 0;
  }
#undef DORA_LDS
}

size_t gen_kernel_lds_bytes(int cfg) {
#define DORA_LDS(...) (size_t)(2 * GenK<__VA_ARGS__>::L0 + GenK<__VA_ARGS__>::RED)
  switch (cfg) {
    case kGenB64: return DORA_LDS(bf16_t, 2, 2, 2, 1, 64);
    case kGenB128: return DORA_LDS(bf16_t, 1, 4, 4, 1, 64);
    case kGenB256: return DORA_LDS(bf16_t, 1, 4, 4, 2, 64);
    case kGenT192: return DORA_LDS(bf16_t, 4, 2, 2, 3, 64);
    case kGenF32: return DORA_LDS(float, 4, 1, 1, 1, 32);
    case kGenF128: return DORA_LDS(float, 1, 4, 4, 1, 32);
    default: return 0;
  }
#undef DORA_LDS
}

}  // namespace dora
