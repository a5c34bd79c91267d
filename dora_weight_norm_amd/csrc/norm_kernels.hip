// Factored DoRA row norm on gfx950.
//
// ||W + sBA||^2_row = ||W||^2_row + 2s <W, BA>_row + s^2 ||BA||^2_row
// ("DoRA优化技术解析：从内存瓶颈到高效实现", cyqw.cn, §1.2 and §1.2.1;
// "Scaling DoRA", alanhou.org, "Factored Norm").
//
// Three launches:
//   norm_main    one pass over W and A on the matrix cores. Rows of W and
//                rows of A are stacked as one M dimension and contracted
//                against A over d_in. W rows give U = W A^T, which is dotted
//                with B row by row in the epilogue (cross term) and never
//                stored; the same W fragments are squared on the vector ALU
//                (base term). A rows give G = A A^T partials.
//                d_in is split into one range per die so each die's L2 holds
//                the slice of A its 32 workgroups share; inside a range the
//                (tile, stage) work units are cut evenly across workgroups.
//   gram_reduce  sums the G partials in a fixed order; for bf16 it stores G
//                as an unevaluated sum of two bf16 matrices, G ~ Ghi + Glo.
//   norm_finish  (B G) on the matrix cores (B Ghi + B Glo), dotted with B
//                (Gram term); sums the base/cross partials in a fixed order;
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
  static constexpr int ROWS = MT + NTC;
  static constexpr int STAGE = ROWS * RB;
  static constexpr int NCH = ROWS * CPR;
  static constexpr int CPT = NCH / kThreads;    // chunks per thread (register path)
  static constexpr int RSTEP = kThreads / CPR;  // row step between a thread's chunks
  static constexpr int RPB = 1024 / RB;         // LDS rows per 1 KiB direct-load block
  static constexpr int MBLK = MT * RB / 1024;   // direct-load blocks of the M rows
  static constexpr int NBLKS = NTC * RB / 1024; // direct-load blocks of the N rows
  static constexpr int BPW_M = MBLK / 4, BPW_N = NBLKS / 4, BPW = BPW_M + BPW_N;
  // Epilogue: U rows of one 32-row block per wave row (WM*32 rows) in fp32.
  static constexpr int UR = WM * 32;            // rows handled per epilogue round
  static constexpr int UPITCH = NTC * 4 + 16;   // bytes per U row in LDS
  static constexpr int TPR = kThreads / UR;     // threads per row in the dot product
  static constexpr int CPTH = NTC / TPR;        // columns per thread in the dot product
  static constexpr int UBUF = UR * UPITCH;
  static constexpr int RED = 2 * MT * 4;        // cross and base row sums
  static constexpr int L0 = CMax<STAGE, UBUF>::v;
  static constexpr int L1 = CMax<STAGE, RED>::v;
  static_assert(WM * WN == 4, "four waves");
  static_assert(NCH % kThreads == 0, "stage must split evenly over the threads");
  static_assert(MT % RSTEP == 0, "M rows end on a thread-row boundary");
  static_assert(KSTEPS * 2 * FC == CPR, "K16 steps cover the stage");
  static_assert(MBLK % 4 == 0 && NBLKS % 4 == 0, "direct-load blocks split evenly over the waves");
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
__global__ __launch_bounds__(kThreads, 1) void norm_main_kernel(NormPlan p, const T* __restrict__ W,
                                                                 const T* __restrict__ A,
                                                                 const T* __restrict__ B,
                                                                 char* __restrict__ ws) {
  using C = MainCfg<T, WM, WN, MB, NB, KT>;
  constexpr int MT = C::MT, NTC = C::NTC, RB = C::RB, CPR = C::CPR, FC = C::FC, EPC = C::EPC;
  constexpr int ESZ = C::ESZ;
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

    // Byte offsets (k = 0) of this lane's direct-load chunks, from the tile's
    // first row; one per 1 KiB block this wave loads.
    uint32_t doff[C::BPW];
    {
      const int sub = lane / CPR, phys = lane % CPR;
#pragma unroll
      for (int i = 0; i < C::BPW; ++i) {
        const bool mrow = i < C::BPW_M;
        const int blk = mrow ? i * 4 + wave : C::MBLK + (i - C::BPW_M) * 4 + wave;
        const int row = blk * C::RPB + sub;
        const int lr = mrow ? row : row - MT;
        const int lim = mrow ? m_lim : n_lim;
        const int rr = lr < lim ? lr : lim - 1;
        doff[i] = (uint32_t)rr * (uint32_t)row_bytes + (uint32_t)(swz<CPR>(row, phys) * 16);
      }
    }

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

    // Direct loads of stage kt. In a ragged last stage (only when d_in is not
    // a multiple of KT) lanes whose chunk lies past d_in are masked off the
    // load and write zeros to their LDS slot instead.
    auto dma_stage = [&](int64_t kt, char* sb) __attribute__((always_inline)) {
      const char* mb_ = reinterpret_cast<const char*>(msrc) + kt * (KT * ESZ);
      const char* nb_ = reinterpret_cast<const char*>(nsrc) + kt * (KT * ESZ);
      const bool full = (kt + 1) * KT <= d_in;
      if (full) {
#pragma unroll
        for (int i = 0; i < C::BPW; ++i) {
          const bool mrow = i < C::BPW_M;
          const int blk = mrow ? i * 4 + wave : C::MBLK + (i - C::BPW_M) * 4 + wave;
          const char* src = (mrow ? mb_ : nb_) + doff[i];
          __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                           (__attribute__((address_space(3))) void*)(sb + blk * 1024), 16, 0, 0);
        }
      } else {
        const int sub = lane / CPR, phys = lane % CPR;
#pragma unroll
        for (int i = 0; i < C::BPW; ++i) {
          const bool mrow = i < C::BPW_M;
          const int blk = mrow ? i * 4 + wave : C::MBLK + (i - C::BPW_M) * 4 + wave;
          const char* src = (mrow ? mb_ : nb_) + doff[i];
          char* dst = sb + blk * 1024;
          const int row = blk * C::RPB + sub;
          const int64_t k = kt * KT + (int64_t)swz<CPR>(row, phys) * EPC;
          if (k < d_in) {
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                             (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
          } else {
            *reinterpret_cast<u32x4*>(dst + lane * 16) = u32x4{0u, 0u, 0u, 0u};
          }
        }
      }
    };

    auto reg_stage = [&](int64_t kt, char* sb) __attribute__((always_inline)) {
      const int cch = tid % CPR, row0 = tid / CPR;
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

    auto compute = [&](const char* sb) __attribute__((always_inline)) {
#pragma unroll
      for (int ks = 0; ks < C::KSTEPS; ++ks) {
        u32x4 fa[MB][FC], fb[NB][FC];
#pragma unroll
        for (int a = 0; a < MB; ++a) {
          const int row = wmi * MB * 32 + a * 32 + lrow;
#pragma unroll
          for (int f = 0; f < FC; ++f) {
            const int ch = ks * 2 * FC + lgrp * FC + f;
            fa[a][f] = *reinterpret_cast<const u32x4*>(sb + row * RB + swz<CPR>(row, ch) * 16);
          }
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int row = MT + wni * NB * 32 + b * 32 + lrow;
#pragma unroll
          for (int f = 0; f < FC; ++f) {
            const int ch = ks * 2 * FC + lgrp * FC + f;
            fb[b][f] = *reinterpret_cast<const u32x4*>(sb + row * RB + swz<CPR>(row, ch) * 16);
          }
        }
#pragma unroll
        for (int a = 0; a < MB; ++a)
#pragma unroll
          for (int b = 0; b < NB; ++b) acc[a][b] = Mfma<T>::run(fa[a], fb[b], acc[a][b]);
        if (do_sq) {
#pragma unroll
          for (int a = 0; a < MB; ++a)
            if (a % WN == wni) {
              float q = 0.f;
#pragma unroll
              for (int f = 0; f < FC; ++f) q += chunk_sumsq(fa[a][f], T());
              sq[a] += q;
            }
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
      for (int a = 0; a < MB; ++a)
        if (do_sq && (a % WN) == wni) {
          const float q = sq[a] + __shfl_xor(sq[a], 32, 64);
          if (lgrp == 0) red_b[wmi * MB * 32 + a * 32 + lrow] = q;
        }
      // Cross term, one 32-row block per wave row at a time: U goes to LDS
      // straight from the accumulators, then each row is dotted with B.
      const int ur = tid / C::TPR, part = tid % C::TPR;   // row in the round, column part
      const int uwm = ur / 32, ua = ur % 32;
      const int64_t gc0 = n0 + (int64_t)part * C::CPTH;
#pragma unroll
      for (int a = 0; a < MB; ++a) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int rr = wmi * 32 + acc_row(v, lgrp);
            const int cc = wni * NB * 32 + b * 32 + lrow;
            *reinterpret_cast<float*>(s0 + rr * C::UPITCH + cc * 4) = acc[a][b][v];
          }
        __syncthreads();
        const int lr = uwm * MB * 32 + a * 32 + ua;       // tile row of this thread
        const int64_t grow = mrow0 + lr;
        const T* brow = B + grow * p.r;
        const bool row_ok = lr < m_lim;
        float dsum = 0.f;
#pragma unroll
        for (int c = 0; c < C::CPTH; c += EPC) {
          const u32x4 bv = load_chunk(brow, gc0 + c, p.r, row_ok, VEC);
          const float* up = reinterpret_cast<const float*>(s0 + ur * C::UPITCH + (part * C::CPTH + c) * 4);
          float bf[EPC];
          if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              bf[2 * e] = __uint_as_float(bv[e] << 16);
              bf[2 * e + 1] = __uint_as_float(bv[e] & 0xffff0000u);
            }
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) bf[e] = __uint_as_float(bv[e]);
          }
#pragma unroll
          for (int e = 0; e < EPC; ++e) dsum = fmaf(up[e], bf[e], dsum);
        }
#pragma unroll
        for (int off = C::TPR / 2; off >= 1; off >>= 1) dsum += __shfl_xor(dsum, off, 64);
        if (part == 0) red_c[lr] = dsum;
        __syncthreads();
      }
      for (int R = tid; R < MT; R += kThreads) {
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
// gram_reduce: G[i][j] = sum over ranges and segments, fixed order.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads) void gram_reduce_kernel(NormPlan p, char* __restrict__ ws) {
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t r32 = p.r32;
  if (idx >= r32 * r32) return;
  const int64_t i = idx / r32, j = idx % r32;
  const float* part_g = reinterpret_cast<const float*>(ws + p.off_g);
  float acc = 0.f;
  if (i < p.r && j < p.r) {
    const int ma = (int)(i / p.mt), n = (int)(j / p.ntc);
    const int64_t t = (int64_t)(p.n_mt_w + ma) * p.n_nt + n;
    for (int x = 0; x < p.X; ++x) {
      const int64_t kb = range_lo(p.n_kt, p.X, x);
      const int64_t nk = range_lo(p.n_kt, p.X, x + 1) - kb;
      const int64_t U = n_tiles(p) * nk;
      const int sa = slot_of(U, p.P, t * nk), sb = slot_of(U, p.P, t * nk + nk - 1);
      for (int s = sa; s <= sb; ++s) {
        if (unit_lo(U, p.P, s) == unit_lo(U, p.P, s + 1)) continue;
        const int64_t ps = (int64_t)x * p.maxseg + (s - sa);
        acc += part_g[(ps * p.ga_rows + i) * p.ga_cols + j];
      }
    }
  }
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
// norm_finish: ba = rowsum((B G) * B), base/cross partial sums, assembly.
// One workgroup per 32 rows; wave w takes column blocks w, w+4, ...
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads) void norm_finish_kernel(NormPlan p, const T* __restrict__ B,
                                                               const char* __restrict__ ws, float s,
                                                               const float* m, float eps,
                                                               float* wnorm, float* g) {
  constexpr int EPC = Elem<T>::epc, FC = Elem<T>::frag_chunks;
  constexpr int NBG = 4;   // column blocks per wave per pass
  __shared__ float red[4 * 16 * 64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 31, lgrp = lane >> 5;
  const int64_t j0 = (int64_t)blockIdx.x * 32;
  const int64_t r = p.r, r32 = p.r32;
  const bool bvec = p.vec_b != 0;
  const int nblk = (int)(r32 / 32);
  const int64_t arow = j0 + lrow;
  const bool arow_ok = arow < p.d_out;
  const T* brow = B + arow * r;

  float pr[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) pr[v] = 0.f;

  for (int g0 = 0; g0 < nblk; g0 += 4 * NBG) {
    f32x16 acc[NBG];
#pragma unroll
    for (int q = 0; q < NBG; ++q)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[q][v] = 0.f;
    for (int64_t k0 = 0; k0 < r32; k0 += 16) {
      u32x4 fa[FC];
#pragma unroll
      for (int f = 0; f < FC; ++f)
        fa[f] = load_chunk(brow, k0 + (int64_t)(lgrp * FC + f) * EPC, r, arow_ok, bvec);
#pragma unroll
      for (int q = 0; q < NBG; ++q) {
        const int nb = g0 + q * 4 + wave;
        if (nb >= nblk) continue;
        const int64_t grow = (int64_t)nb * 32 + lrow;
        if constexpr (sizeof(T) == 2) {
          const bf16_t* ghi = reinterpret_cast<const bf16_t*>(ws + p.off_ghi) + grow * r32 + k0 + lgrp * 8;
          const bf16_t* glo = reinterpret_cast<const bf16_t*>(ws + p.off_glo) + grow * r32 + k0 + lgrp * 8;
          u32x4 fh = *reinterpret_cast<const u32x4*>(ghi);
          u32x4 fl = *reinterpret_cast<const u32x4*>(glo);
          acc[q] = Mfma<T>::run(fa, &fh, acc[q]);
          acc[q] = Mfma<T>::run(fa, &fl, acc[q]);
        } else {
          const float* g32 = reinterpret_cast<const float*>(ws + p.off_ghi) + grow * r32 + k0 + lgrp * 8;
          u32x4 fb[2];
          fb[0] = *reinterpret_cast<const u32x4*>(g32);
          fb[1] = *reinterpret_cast<const u32x4*>(g32 + 4);
          acc[q] = Mfma<T>::run(fa, fb, acc[q]);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < NBG; ++q) {
      const int nb = g0 + q * 4 + wave;
      if (nb >= nblk) continue;
      const int64_t col = (int64_t)nb * 32 + lrow;
      if (col >= r) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = j0 + acc_row(v, lgrp);
        if (row < p.d_out) pr[v] = fmaf(acc[q][v], to_f32(B[row * r + col]), pr[v]);
      }
    }
  }

#pragma unroll
  for (int v = 0; v < 16; ++v) red[(wave * 16 + v) * 64 + lane] = pr[v];
  __syncthreads();

  if (tid < 32) {
    const int R = tid;
    const int64_t j = j0 + R;
    if (j < p.d_out) {
      const int v = (R / 8) * 4 + (R & 3);
      const int gq = (R & 7) / 4;
      float ba = 0.f;
      for (int w = 0; w < 4; ++w) {
        const float* src = red + (w * 16 + v) * 64 + gq * 32;
        float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 32; ++i) s4[i & 3] += src[i];
        ba += (s4[0] + s4[1]) + (s4[2] + s4[3]);
      }
      const float* part_base = reinterpret_cast<const float*>(ws + p.off_base);
      const float* part_cross = reinterpret_cast<const float*>(ws + p.off_cross);
      const int mt_idx = (int)(j / p.mt);
      float base = 0.f, cross = 0.f;
      for (int x = 0; x < p.X; ++x) {
        const int64_t kb = range_lo(p.n_kt, p.X, x);
        const int64_t nk = range_lo(p.n_kt, p.X, x + 1) - kb;
        const int64_t U = n_tiles(p) * nk;
        for (int n = 0; n < p.n_nt; ++n) {
          const int64_t t = (int64_t)mt_idx * p.n_nt + n;
          const int sa = slot_of(U, p.P, t * nk), sb = slot_of(U, p.P, t * nk + nk - 1);
          for (int sl = sa; sl <= sb; ++sl) {
            if (unit_lo(U, p.P, sl) == unit_lo(U, p.P, sl + 1)) continue;
            const int64_t ps = (int64_t)x * p.maxseg + (sl - sa);
            cross += part_cross[(ps * p.n_nt + n) * p.ld_w + j];
            if (n == 0) base += part_base[ps * p.ld_w + j];
          }
        }
      }
      // wnorm = sqrt(max(base + 2s*cross + s^2*ba, 0)), each operation rounded.
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
  if (p.vec_in && p.vec_b)
    hipLaunchKernelGGL((norm_main_kernel<T, WM, WN, MB, NB, KT, true>), dim3(p.X * p.P), dim3(kThreads), 0, st,
                       p, static_cast<const T*>(W), static_cast<const T*>(A), static_cast<const T*>(B), ws);
  else
    hipLaunchKernelGGL((norm_main_kernel<T, WM, WN, MB, NB, KT, false>), dim3(p.X * p.P), dim3(kThreads), 0,
                       st, p, static_cast<const T*>(W), static_cast<const T*>(A), static_cast<const T*>(B), ws);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_tail(const NormPlan& p, const void* B, char* ws, float s, const float* m, float eps,
                       float* wnorm, float* g, hipStream_t st) {
  const int64_t n_g = p.r32 * p.r32;
  hipLaunchKernelGGL((gram_reduce_kernel<T>), dim3((unsigned)((n_g + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, st, p, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((norm_finish_kernel<T>), dim3((unsigned)((p.d_out + 31) / 32)), dim3(kThreads), 0, st,
                     p, static_cast<const T*>(B), ws, s, m, eps, wnorm, g);
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
    case kBf16R384: e = launch_main<bf16_t, 1, 4, 4, 3, 64>(p, W, A, B, ws, st); break;
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
    case kBf16R384: return MainCfg<bf16_t, 1, 4, 4, 3, 64>::L0 + MainCfg<bf16_t, 1, 4, 4, 3, 64>::L1;
    case kBf16R512: return MainCfg<bf16_t, 1, 4, 2, 4, 64>::L0 + MainCfg<bf16_t, 1, 4, 2, 4, 64>::L1;
    case kBf16R768: return MainCfg<bf16_t, 1, 4, 2, 6, 32>::L0 + MainCfg<bf16_t, 1, 4, 2, 6, 32>::L1;
    case kF32R32: return MainCfg<float, 4, 1, 1, 1, 32>::L0 + MainCfg<float, 4, 1, 1, 1, 32>::L1;
    case kF32R128: return MainCfg<float, 1, 4, 4, 1, 32>::L0 + MainCfg<float, 1, 4, 4, 1, 32>::L1;
    default: return 0;
  }
}

}  // namespace dora
