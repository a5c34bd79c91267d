// Factored DoRA row norm on gfx950.
//
// ||W + sBA||^2_row = ||W||^2_row + 2s <W, BA>_row + s^2 ||BA||^2_row
// ("DoRA优化技术解析：从内存瓶颈到高效实现", cyqw.cn, §1.2 and §1.2.1;
// "Scaling DoRA", alanhou.org, "Factored Norm").
//
// Four launches:
//   norm_main    one pass over W and A on the matrix cores. Rows of W and
//                rows of A are stacked as one M dimension and contracted
//                against A over d_in. W rows give U = W A^T, which is dotted
//                with B row by row in the epilogue (cross term) and never
//                stored; the same W fragments are squared (base term). A
//                rows give G = A A^T partials.
//                d_in is split into one range per die so each die's L2 holds
//                the slice of A its 32 workgroups share; inside a range the
//                (tile, stage) work units are cut evenly across workgroups.
//   gram_reduce  sums the G partials in a fixed order; for bf16 it stores G
//                as an unevaluated sum of two bf16 matrices, G ~ Ghi + Glo.
//   gram_term    (B G) on the matrix cores (B Ghi + B Glo), dotted with B,
//                per 64-column block of G (Gram term partials).
//   assemble     fixed-order sums of all partials;
//                wnorm = sqrt(max(base + 2s cross + s^2 ba, 0)) and
//                g = m / max(wnorm, eps) without contraction, with correctly
//                rounded sqrt and division (same page, §1.2.2, §5.2, §6.2).
//
// When s == 0 or r == 0 the cross and Gram terms vanish and only a row
// sum-of-squares kernel runs (same page, §5.1, notes of Algorithm 1).
#include "dora_device.h"
#include "dora_launch.h"
#include "dora_plan.h"

namespace dora {

namespace {

template <int A_, int B_>
struct CMax {
  static constexpr int v = A_ > B_ ? A_ : B_;
};

// ---------------------------------------------------------------------------
// norm_main
// ---------------------------------------------------------------------------
template <typename T, int WM, int WN, int MB, int NB, int KT>
struct MainCfg {
  static constexpr int ESZ = Elem<T>::esz;
  static constexpr int EPC = Elem<T>::epc;
  static constexpr int FC = Elem<T>::frag_chunks;
  static constexpr int MT = WM * MB * 32;
  static constexpr int NTC = WN * NB * 32;
  static constexpr int RB = KT * ESZ;           // bytes of one LDS row
  static constexpr int CPR = RB / 16;           // 16-byte chunks per LDS row
  static constexpr int KSTEPS = KT / 16;
  static constexpr int NW = WM * WN;            // waves per workgroup
  static constexpr int NT = NW * 64;            // threads per workgroup
  static constexpr int ROWS = MT + NTC;
  static constexpr int STAGE = ROWS * RB;
  static constexpr int NCH = ROWS * CPR;
  static constexpr int CPT = NCH / NT;          // chunks per thread (register path)
  static constexpr int RSTEP = NT / CPR;        // row step between a thread's chunks
  static constexpr int RPB = 1024 / RB;         // LDS rows per 1 KiB direct-load block
  static constexpr int MBLK = MT * RB / 1024;   // direct-load blocks of the M rows
  static constexpr int NBLKS = NTC * RB / 1024; // direct-load blocks of the N rows
  static constexpr int BPW_M = MBLK / NW, BPW_N = NBLKS / NW, BPW = BPW_M + BPW_N;
  // Epilogue: one 32-row block of U at a time, in fp32.
  static constexpr int UR = 32;                 // rows handled per epilogue round
  static constexpr int UPITCH = NTC * 4 + 16;   // bytes per U row in LDS
  static constexpr int TPR = NT / UR;           // threads per row in the dot product
  static constexpr int CPTH = NTC / TPR;        // columns per thread in the dot product
  static constexpr int UBUF = UR * UPITCH;
  static constexpr int RED = 2 * MT * 4;        // cross and base row sums
  static constexpr int L0 = CMax<STAGE, UBUF>::v;
  static constexpr int L1 = CMax<STAGE, RED>::v;
  static_assert(NW == 4 || NW == 8, "four or eight waves");
  static_assert(NCH % NT == 0, "stage must split evenly over the threads");
  static_assert(MT % RSTEP == 0, "M rows end on a thread-row boundary");
  static_assert(KSTEPS * 2 * FC == CPR, "K16 steps cover the stage");
  static_assert(MBLK % NW == 0 && NBLKS % NW == 0, "direct-load blocks split evenly over the waves");
  static_assert(CPTH % EPC == 0 && (TPR & (TPR - 1)) == 0, "dot-product split");
  static_assert(L0 + L1 <= 160 * 1024, "gfx950 has 160 KiB of LDS per workgroup");
};

// Main kernel. Work unit = (tile, d_in stage). A tile is MT rows (of W, or
// of A for the Gram matrix) by NTC columns of U (rows of A); a stage is KT
// elements of d_in. The stages of one tile stream through two LDS buffers:
// a full stage arrives by direct global->LDS loads (global_load_lds_dwordx4,
// 64 lanes x 16 B into 1 KiB of LDS per instruction) issued before the
// previous stage's matrix work, so the copy overlaps the MFMAs and needs no
// staging registers. Each lane picks the global chunk that lands on its LDS
// slot under the XOR swizzle; rows past the matrix edge load a clamped real
// row, and those accumulator rows and columns are never used. A ragged last
// stage, or inputs that do not allow aligned 16-byte loads (VEC == false),
// go through registers with explicit zero fill.
template <typename T, int WM, int WN, int MB, int NB, int KT, bool VEC>
__global__ __launch_bounds__(WM * WN * 64, 1) void norm_main_kernel(NormPlan p, const T* __restrict__ W,
                                                                 const T* __restrict__ A,
                                                                 const T* __restrict__ B,
                                                                 char* __restrict__ ws) {
  using C = MainCfg<T, WM, WN, MB, NB, KT>;
  constexpr int MT = C::MT, NTC = C::NTC, RB = C::RB, CPR = C::CPR, FC = C::FC, EPC = C::EPC;
  constexpr int ESZ = C::ESZ, NW = C::NW, NT = C::NT;
  __shared__ __attribute__((aligned(1024))) char s0[C::L0];
  __shared__ __attribute__((aligned(1024))) char s1[C::L1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wmi = wave / WN, wni = wave % WN;
  const int lrow = lane & 31, lgrp = lane >> 5;

  const int X = p.X, P = p.P;
  const int x = blockIdx.x % X;
  const int slot = blockIdx.x / X;
  const int64_t kb = range_lo(p.n_kt, X, x);
  const int64_t nk = range_lo(p.n_kt, X, x + 1) - kb;
  const int64_t U = n_tiles(p) * nk;
  int64_t u = unit_lo(U, P, slot);
  const int64_t u_end = unit_lo(U, P, slot + 1);

  float* part_base = reinterpret_cast<float*>(ws + p.off_base);
  float* part_cross = reinterpret_cast<float*>(ws + p.off_cross);
  float* part_g = reinterpret_cast<float*>(ws + p.off_g);
  const int64_t d_in = p.d_in;
  const int64_t row_bytes = d_in * ESZ;

  while (u < u_end) {
    const int64_t t = u / nk;
    const int64_t i0 = u - t * nk;
    const int64_t i1 = (u_end - u < nk - i0) ? i0 + (u_end - u) : nk;
    const int seg = slot - slot_of(U, P, t * nk);
    const int m = (int)(t / p.n_nt);
    const int n = (int)(t % p.n_nt);
    const bool is_w = m < p.n_mt_w;
    const int64_t mrow0 = is_w ? (int64_t)m * MT : (int64_t)(m - p.n_mt_w) * MT;
    const T* msrc = (is_w ? W : A) + mrow0 * d_in;
    const int64_t m_left = (is_w ? p.d_out : p.r) - mrow0;
    const int m_lim = m_left < MT ? (int)m_left : MT;   // valid rows of this tile
    const int64_t n0 = (int64_t)n * NTC;
    const T* nsrc = A + n0 * d_in;
    const int n_lim = p.r - n0 < NTC ? (int)(p.r - n0) : NTC;
    const bool do_sq = is_w && n == 0;

    // Direct loads go through one buffer descriptor per operand, spanning
    // exactly the tile's valid rows: a lane whose row lies past the matrix
    // edge is out of range and reads zeros. doff holds each lane's byte
    // offset (at k = 0) for every 1 KiB LDS block this wave loads.
    const int m_bytes = (int)((uint32_t)m_lim * (uint32_t)row_bytes);
    const int n_bytes = (int)((uint32_t)n_lim * (uint32_t)row_bytes);
    uint32_t doff[C::BPW];
    {
      const int sub = lane / CPR, phys = lane % CPR;
#pragma unroll
      for (int i = 0; i < C::BPW; ++i) {
        const bool mrow = i < C::BPW_M;
        const int blk = mrow ? i * NW + wave : C::MBLK + (i - C::BPW_M) * NW + wave;
        const int row = blk * C::RPB + sub;
        const int lr = mrow ? row : row - MT;
        doff[i] = (uint32_t)lr * (uint32_t)row_bytes + (uint32_t)(swz<CPR>(row, phys) * 16);
      }
    }

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

    auto dma_stage = [&](int64_t kt, char* sb) __attribute__((always_inline)) {
      const uint32_t koff = (uint32_t)(kt * (KT * ESZ));
      const bool full = (kt + 1) * KT <= d_in;
      if (full) {
#pragma unroll
        for (int i = 0; i < C::BPW; ++i) {
          const bool mrow = i < C::BPW_M;
          const int blk = mrow ? i * NW + wave : C::MBLK + (i - C::BPW_M) * NW + wave;
          lds_load16(mrow ? (const void*)msrc : (const void*)nsrc, mrow ? m_bytes : n_bytes, sb + blk * 1024, doff[i],
                     koff);
        }
      } else {
        const int sub = lane / CPR, phys = lane % CPR;
#pragma unroll
        for (int i = 0; i < C::BPW; ++i) {
          const bool mrow = i < C::BPW_M;
          const int blk = mrow ? i * NW + wave : C::MBLK + (i - C::BPW_M) * NW + wave;
          char* dst = sb + blk * 1024;
          const int row = blk * C::RPB + sub;
          const int64_t k = kt * KT + (int64_t)swz<CPR>(row, phys) * EPC;
          if (k < d_in) {
            lds_load16(mrow ? (const void*)msrc : (const void*)nsrc, mrow ? m_bytes : n_bytes, dst, doff[i], koff);
          } else {
            *reinterpret_cast<u32x4*>(dst + lane * 16) = u32x4{0u, 0u, 0u, 0u};
          }
        }
      }
    };

    auto reg_stage = [&](int64_t kt, char* sb) __attribute__((always_inline)) {
      const int cch = tid % CPR, row0 = tid / CPR;   // NT threads cover RSTEP rows per pass
      const int64_t k = kt * KT + (int64_t)cch * EPC;
      u32x4 st[C::CPT];
#pragma unroll
      for (int i = 0; i < C::CPT; ++i) {
        const int row = row0 + i * C::RSTEP;
        if (i < MT / C::RSTEP) {
          st[i] = load_chunk(msrc + (int64_t)row * d_in, k, d_in, row < m_lim, VEC);
        } else {
          const int nr = row - MT;
          st[i] = load_chunk(nsrc + (int64_t)nr * d_in, k, d_in, nr < n_lim, VEC);
        }
      }
#pragma unroll
      for (int i = 0; i < C::CPT; ++i) {
        const int row = row0 + i * C::RSTEP;
        *reinterpret_cast<u32x4*>(sb + row * RB + swz<CPR>(row, cch) * 16) = st[i];
      }
    };

    // One stage on the matrix cores. Fragments are double-buffered across
    // the K16 steps: step ks+1 is read from LDS while step ks's MFMAs run.
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
#pragma unroll
        for (int i = 0; i < SQB; ++i) {
          float q = 0.f;
#pragma unroll
          for (int f = 0; f < FC; ++f) q += chunk_sumsq(fs[c][i][f], T());
          sq[i] += q;
        }
      }
    };

    // Prefetch stage `nxt` into `dst` (direct loads before the matrix work,
    // or registers after it), consume `src`, then barrier.
    auto step = [&](const char* src, char* dst, int64_t nxt, bool more) __attribute__((always_inline)) {
      if constexpr (VEC) {
        if (more) dma_stage(nxt, dst);
        __builtin_amdgcn_sched_barrier(0);
        compute(src);
      } else {
        compute(src);
        if (more) reg_stage(nxt, dst);
      }
      __syncthreads();
    };

    if constexpr (VEC) dma_stage(kb + i0, s0);
    else reg_stage(kb + i0, s0);
    __syncthreads();
    int64_t it = i0;
    for (; it + 1 < i1; it += 2) {
      step(s0, s1, kb + it + 1, true);
      step(s1, s0, kb + it + 2, it + 2 < i1);
    }
    if (it < i1) step(s0, s1, 0, false);

    const int64_t pslot = (int64_t)x * p.maxseg + seg;
    if (is_w) {
      float* red_c = reinterpret_cast<float*>(s1);   // [MT] cross row sums
      float* red_b = red_c + MT;                     // [MT] base row sums
      // Base term: the two k-halves of each row live in lanes l and l+32.
#pragma unroll
      for (int i = 0; i < SQB; ++i) {
        const float q = sq[i] + __shfl_xor(sq[i], 32, 64);
        if (do_sq && wni < MB && lgrp == 0) red_b[wmi * MB * 32 + ((wni % MB) + i * WN) * 32 + lrow] = q;
      }
      // Cross term, one 32-row block of U at a time: the owning waves write
      // it to LDS straight from their accumulators, then every row is dotted
      // with B. The B chunks of the next round are loaded during this one.
      const int ur = tid / C::TPR, part = tid % C::TPR;   // row in the round, column part
      const int64_t gc0 = n0 + (int64_t)part * C::CPTH;
      constexpr int NBC = C::CPTH / EPC;                  // B chunks per thread per round
      u32x4 bcur[NBC], bnxt[NBC];
      auto load_b = [&](int lr, u32x4 (&dst)[NBC]) __attribute__((always_inline)) {
        const T* brow = B + (mrow0 + lr) * p.r;
        const bool row_ok = lr < m_lim;
#pragma unroll
        for (int c = 0; c < NBC; ++c) dst[c] = load_chunk(brow, gc0 + c * EPC, p.r, row_ok, VEC);
      };
      load_b(ur, bcur);
#pragma unroll
      for (int a = 0; a < MB; ++a) {
#pragma unroll
        for (int wr = 0; wr < WM; ++wr) {
          const int lr = wr * MB * 32 + a * 32 + ur;         // tile row of this thread this round
          if (wmi == wr) {
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
              for (int v = 0; v < 16; ++v) {
                const int cc = wni * NB * 32 + b * 32 + lrow;
                *reinterpret_cast<float*>(s0 + acc_row(v, lgrp) * C::UPITCH + cc * 4) = acc[a][b][v];
              }
          }
          __syncthreads();
          const bool last = (a + 1 == MB) && (wr + 1 == WM);
          if (!last) {
            const int nlr = (wr + 1 < WM) ? (wr + 1) * MB * 32 + a * 32 + ur : (a + 1) * 32 + ur;
            load_b(nlr, bnxt);
          }
          float dsum = 0.f;
#pragma unroll
          for (int c = 0; c < NBC; ++c) {
            const float* up = reinterpret_cast<const float*>(s0 + ur * C::UPITCH + (part * C::CPTH + c * EPC) * 4);
            float bf[EPC];
            if constexpr (sizeof(T) == 2) {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                bf[2 * e] = __uint_as_float(bcur[c][e] << 16);
                bf[2 * e + 1] = __uint_as_float(bcur[c][e] & 0xffff0000u);
              }
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e) bf[e] = __uint_as_float(bcur[c][e]);
            }
#pragma unroll
            for (int e = 0; e < EPC; ++e) dsum = fmaf(up[e], bf[e], dsum);
          }
#pragma unroll
          for (int off = C::TPR / 2; off >= 1; off >>= 1) dsum += __shfl_xor(dsum, off, 64);
          if (part == 0) red_c[lr] = dsum;
          __syncthreads();
          if (!last) {
#pragma unroll
            for (int c = 0; c < NBC; ++c) bcur[c] = bnxt[c];
          }
        }
      }
      for (int R = tid; R < MT; R += NT) {
        const int64_t grow = mrow0 + R;
        part_cross[(pslot * p.n_nt + n) * p.ld_w + grow] = red_c[R];
        if (do_sq) part_base[pslot * p.ld_w + grow] = red_b[R];
      }
      __syncthreads();
    } else {
      // G = A A^T partial for rows mrow0.. of A and columns n0.. .
      float* gdst = part_g + pslot * p.ga_rows * p.ga_cols;
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
    u += i1 - i0;
  }
}

// ---------------------------------------------------------------------------
// gram_reduce: G[i][j] = sum over d_in ranges and segments, fixed order.
// Eight lanes per element, lane x summing range x's segments; the eight
// range sums are then combined by a fixed xor tree.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads) void gram_reduce_kernel(NormPlan p, char* __restrict__ ws) {
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t idx = gid >> 3;
  const int x = (int)(gid & 7);
  const int64_t r32 = p.r32;
  const bool live = idx < r32 * r32;
  const int64_t i = live ? idx / r32 : 0, j = live ? idx % r32 : 0;
  const float* part_g = reinterpret_cast<const float*>(ws + p.off_g);
  float acc = 0.f;
  if (live && x < p.X && i < p.r && j < p.r) {
    const int ma = (int)(i / p.mt), n = (int)(j / p.ntc);
    const int64_t t = (int64_t)(p.n_mt_w + ma) * p.n_nt + n;
    const int64_t nk = range_lo(p.n_kt, p.X, x + 1) - range_lo(p.n_kt, p.X, x);
    const int64_t U = n_tiles(p) * nk;
    const int sa = slot_of(U, p.P, t * nk), sb = slot_of(U, p.P, t * nk + nk - 1);
    for (int s = sa; s <= sb; ++s) {
      const int64_t ps = (int64_t)x * p.maxseg + (s - sa);
      acc += part_g[(ps * p.ga_rows + i) * p.ga_cols + j];
    }
  }
  acc += __shfl_xor(acc, 1, 64);
  acc += __shfl_xor(acc, 2, 64);
  acc += __shfl_xor(acc, 4, 64);
  if (!live || x != 0) return;
  if constexpr (sizeof(T) == 2) {
    bf16_t* ghi = reinterpret_cast<bf16_t*>(ws + p.off_ghi);
    bf16_t* glo = reinterpret_cast<bf16_t*>(ws + p.off_glo);
    const bf16_t h = f32_to_bf16_rne(acc);
    const float rem = acc - bf16_bits_to_f32(h);
    ghi[idx] = h;
    glo[idx] = f32_to_bf16_rne(rem);
  } else {
    reinterpret_cast<float*>(ws + p.off_ghi)[idx] = acc;
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
  const int64_t r = p.r, r32 = p.r32;
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

  for (int64_t k0 = 0; k0 < r32; k0 += C::KC) {
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
      grow = grow < r32 ? grow : r32 - 1;          // past the matrix: a real row, never used
      gk = gk < r32 ? gk : r32 - EPC;
      const char* src = ws + (part == 0 ? p.off_ghi : p.off_glo) + (grow * r32 + gk) * (int64_t)sizeof(T);
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                       (__attribute__((address_space(3))) void*)(sg + blk * 1024), 16, 0, 0);
    }
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
// correctly rounded.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void assemble_kernel(NormPlan p, const char* __restrict__ ws, float s,
                                                            const float* m, float eps, float* wnorm, float* g) {
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t j = gid >> 3;
  const int x = (int)(gid & 7);
  const bool live = j < p.d_out;
  const float* part_base = reinterpret_cast<const float*>(ws + p.off_base);
  const float* part_cross = reinterpret_cast<const float*>(ws + p.off_cross);
  const float* part_ba = reinterpret_cast<const float*>(ws + p.off_ba);
  // Lane x: range x's base and cross partials.
  float base = 0.f, cross = 0.f;
  if (live && x < p.X) {
    const int mt_idx = (int)(j / p.mt);
    const int64_t nk = range_lo(p.n_kt, p.X, x + 1) - range_lo(p.n_kt, p.X, x);
    const int64_t U = n_tiles(p) * nk;
    for (int n = 0; n < p.n_nt; ++n) {
      const int64_t t = (int64_t)mt_idx * p.n_nt + n;
      const int sa = slot_of(U, p.P, t * nk), sb = slot_of(U, p.P, t * nk + nk - 1);
      for (int sl = sa; sl <= sb; ++sl) {
        const int64_t ps = (int64_t)x * p.maxseg + (sl - sa);
        cross += part_cross[(ps * p.n_nt + n) * p.ld_w + j];
        if (n == 0) base += part_base[ps * p.ld_w + j];
      }
    }
  }
  base += __shfl_xor(base, 1, 64);
  base += __shfl_xor(base, 2, 64);
  base += __shfl_xor(base, 4, 64);
  cross += __shfl_xor(cross, 1, 64);
  cross += __shfl_xor(cross, 2, 64);
  cross += __shfl_xor(cross, 4, 64);
  if (!live || x != 0) return;
  float ba = 0.f;
  for (int cb = 0; cb < p.n_cb; ++cb) ba += part_ba[(int64_t)cb * p.ld_w + j];
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

// ---------------------------------------------------------------------------
// Row sum of squares only (s == 0, r == 0 or d_in == 0).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads) void norm_rowonly_kernel(const T* __restrict__ W, int64_t d_out,
                                                                int64_t d_in, bool vec, const float* m,
                                                                float eps, float* wnorm, float* g) {
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

template <typename T, int WM, int WN, int MB, int NB, int KT>
hipError_t launch_main(const NormPlan& p, const void* W, const void* A, const void* B, char* ws,
                       hipStream_t st) {
  constexpr int NT = WM * WN * 64;
  if (p.vec_in && p.vec_b)
    hipLaunchKernelGGL((norm_main_kernel<T, WM, WN, MB, NB, KT, true>), dim3(p.X * p.P), dim3(NT), 0, st,
                       p, static_cast<const T*>(W), static_cast<const T*>(A), static_cast<const T*>(B), ws);
  else
    hipLaunchKernelGGL((norm_main_kernel<T, WM, WN, MB, NB, KT, false>), dim3(p.X * p.P), dim3(NT), 0,
                       st, p, static_cast<const T*>(W), static_cast<const T*>(A), static_cast<const T*>(B), ws);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_tail(const NormPlan& p, const void* B, char* ws, float s, const float* m, float eps,
                       float* wnorm, float* g, hipStream_t st) {
  const int64_t n_g = p.r32 * p.r32;
  hipLaunchKernelGGL((gram_reduce_kernel<T>), dim3((unsigned)((8 * n_g + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, st, p, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((gram_term_kernel<T>), dim3((unsigned)((p.d_out + kGramRows - 1) / kGramRows), (unsigned)p.n_cb),
                     dim3(kGramRows * 2), 0, st, p, static_cast<const T*>(B), ws);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(assemble_kernel, dim3((unsigned)((8 * p.d_out + kThreads - 1) / kThreads)), dim3(kThreads), 0, st,
                     p, ws, s, m, eps, wnorm, g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_norm_factored(const NormPlan& p, const void* W, const void* A, const void* B, void* ws_,
                                float s, const float* m, float eps, float* wnorm, float* g,
                                hipStream_t st) {
  char* ws = static_cast<char*>(ws_);
  hipError_t e = hipErrorInvalidValue;
  switch (p.cfg) {
    case kBf16R64: e = launch_main<bf16_t, 2, 2, 4, 1, 64>(p, W, A, B, ws, st); break;
    case kBf16R128: e = launch_main<bf16_t, 1, 4, 4, 1, 64>(p, W, A, B, ws, st); break;
    case kBf16R256: e = launch_main<bf16_t, 1, 4, 4, 2, 64>(p, W, A, B, ws, st); break;
    case kBf16R384: e = launch_main<bf16_t, 2, 4, 2, 3, 64>(p, W, A, B, ws, st); break;
    case kBf16R512: e = launch_main<bf16_t, 1, 4, 2, 4, 64>(p, W, A, B, ws, st); break;
    case kBf16R768: e = launch_main<bf16_t, 1, 4, 2, 6, 32>(p, W, A, B, ws, st); break;
    case kF32R32: e = launch_main<float, 4, 1, 1, 1, 32>(p, W, A, B, ws, st); break;
    case kF32R128: e = launch_main<float, 1, 4, 4, 1, 32>(p, W, A, B, ws, st); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  if (p.dtype == 0) return launch_tail<bf16_t>(p, B, ws, s, m, eps, wnorm, g, st);
  return launch_tail<float>(p, B, ws, s, m, eps, wnorm, g, st);
}

hipError_t launch_norm_rowonly(const void* W, int dtype, int64_t d_out, int64_t d_in, bool vec, const float* m,
                               float eps, float* wnorm, float* g, hipStream_t st) {
  if (dtype == 0)
    hipLaunchKernelGGL((norm_rowonly_kernel<bf16_t>), dim3((unsigned)d_out), dim3(kThreads), 0, st,
                       static_cast<const bf16_t*>(W), d_out, d_in, vec, m, eps, wnorm, g);
  else
    hipLaunchKernelGGL((norm_rowonly_kernel<float>), dim3((unsigned)d_out), dim3(kThreads), 0, st,
                       static_cast<const float*>(W), d_out, d_in, vec, m, eps, wnorm, g);
  return hipGetLastError();
}

hipError_t launch_magnitude(const float* m, const float* wnorm, float eps, int64_t n, float* g, hipStream_t st) {
  hipLaunchKernelGGL(magnitude_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0, st, m,
                     wnorm, eps, n, g);
  return hipGetLastError();
}

size_t main_kernel_lds_bytes(int cfg) {
  switch (cfg) {
    case kBf16R64: return MainCfg<bf16_t, 2, 2, 4, 1, 64>::L0 + MainCfg<bf16_t, 2, 2, 4, 1, 64>::L1;
    case kBf16R128: return MainCfg<bf16_t, 1, 4, 4, 1, 64>::L0 + MainCfg<bf16_t, 1, 4, 4, 1, 64>::L1;
    case kBf16R256: return MainCfg<bf16_t, 1, 4, 4, 2, 64>::L0 + MainCfg<bf16_t, 1, 4, 4, 2, 64>::L1;
    case kBf16R384: return MainCfg<bf16_t, 2, 4, 2, 3, 64>::L0 + MainCfg<bf16_t, 2, 4, 2, 3, 64>::L1;
    case kBf16R512: return MainCfg<bf16_t, 1, 4, 2, 4, 64>::L0 + MainCfg<bf16_t, 1, 4, 2, 4, 64>::L1;
    case kBf16R768: return MainCfg<bf16_t, 1, 4, 2, 6, 32>::L0 + MainCfg<bf16_t, 1, 4, 2, 6, 32>::L1;
    case kF32R32: return MainCfg<float, 4, 1, 1, 1, 32>::L0 + MainCfg<float, 4, 1, 1, 1, 32>::L1;
    case kF32R128: return MainCfg<float, 1, 4, 4, 1, 32>::L0 + MainCfg<float, 1, 4, 4, 1, 32>::L1;
    default: return 0;
  }
}

}  // namespace dora
