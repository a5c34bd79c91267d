// Stable DoRA magnitude compose on gfx950:
//
//   out[t,j] = (g[j] - 1) * base[t,j] + g[j] * (s * lora[t,j])
//
// ("DoRA优化技术解析：从内存瓶颈到高效实现", cyqw.cn, §2.1, §2.1.1, §5.2.)
// The backward of the same map (the row norm detached) is below: d_base,
// d_lora and, unless the magnitude is frozen, dg by a deterministic
// two-stage column reduction.
//
// One HBM pass: base and lora are streamed once, out written once, g read
// once per thread into registers. Each thread owns one 16-byte column strip
// (8 bf16 or 4 fp32 columns) and walks rows with a stride of the grid's
// row count, keeping several rows' loads in flight. Loads are non-temporal
// (nothing here is reused, so they should not displace anything from the
// L2 or the Infinity Cache); stores are ordinary: measured on MI355X,
// non-temporal stores cost 2-4% of the pass at 4096 x 4096 and at
// 8192 x 8192. Arithmetic is fp32: s*lora first, then one fused
// multiply-add g*(s*lora) + (g-1)*base, rounded once (RNE) to the storage
// type.
//
// The same kernel with ADD writes the layer output instead of the delta,
// y = base + delta (same page, §2.1.1: the compose result is added to the
// base projection): delta is formed as above in fp32, base is added in
// fp32, and y is rounded once to the storage type. That saves the separate
// addition's extra pass (read base and delta, write y) and its second
// rounding.
#include <type_traits>

#include "dora_device.h"
#include "dora_launch.h"

namespace dora {

namespace {

constexpr int kUnroll = 4;

template <typename T, int VEC>
struct Strip;
template <typename T>
struct Strip<T, 1> {
  using V = T;
};
template <>
struct Strip<bf16_t, 8> {
  using V = u32x4;
};
template <>
struct Strip<f16_t, 8> {
  using V = u32x4;
};
template <>
struct Strip<float, 4> {
  using V = u32x4;
};

template <typename T, int VEC>
__device__ __forceinline__ void unpack(const typename Strip<T, VEC>::V& v, float (&f)[VEC]) {
  if constexpr (VEC == 1) {
    f[0] = to_f32(v);
  } else if constexpr (std::is_same<T, f16_t>::value) {
    const f16x8 h = __builtin_bit_cast(f16x8, v);   // the whole vector at once
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = (float)h[i];
  } else if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(v[i] << 16);
      f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
  }
}

template <typename T, int VEC>
__device__ __forceinline__ typename Strip<T, VEC>::V pack(const float (&f)[VEC]) {
  if constexpr (VEC == 1) {
    return from_f32<T>(f[0]);
  } else if constexpr (std::is_same<T, f16_t>::value) {
    f16x8 h;
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = (f16_t)f[i];   // round to nearest even
    return __builtin_bit_cast(u32x4, h);
  } else if constexpr (sizeof(T) == 2) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      v[i] = (uint32_t)f32_to_bf16_rne(f[2 * i]) | ((uint32_t)f32_to_bf16_rne(f[2 * i + 1]) << 16);
    return v;
  } else {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(f[i]);
    return v;
  }
}

template <typename T, int VEC, bool ADD>
__global__ __launch_bounds__(256) void compose_kernel(const T* base, const T* lora, const float* __restrict__ g,
                                                      float s, int64_t T_rows, int64_t d_out, T* out) {
  using V = typename Strip<T, VEC>::V;
  const int64_t cg = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (cg >= d_out / VEC) return;
  const int64_t c0 = cg * VEC;
  float gv[VEC], gm1[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    gv[e] = g[c0 + e];
    gm1[e] = gv[e] - 1.0f;
  }
  const int64_t step = (int64_t)gridDim.y * kUnroll;
  for (int64_t t0 = (int64_t)blockIdx.y * kUnroll; t0 < T_rows; t0 += step) {
    V bv[kUnroll], lv[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (t0 + u < T_rows) {
        const int64_t off = (t0 + u) * d_out + c0;
        bv[u] = __builtin_nontemporal_load(reinterpret_cast<const V*>(base + off));
        lv[u] = __builtin_nontemporal_load(reinterpret_cast<const V*>(lora + off));
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (t0 + u < T_rows) {
        float b[VEC], l[VEC], o[VEC];
        unpack<T, VEC>(bv[u], b);
        unpack<T, VEC>(lv[u], l);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const float sl = s * l[e];
          o[e] = fmaf(gv[e], sl, gm1[e] * b[e]);
          if constexpr (ADD) o[e] = o[e] + b[e];
        }
        const int64_t off = (t0 + u) * d_out + c0;
        *reinterpret_cast<V*>(out + off) = pack<T, VEC>(o);
      }
    }
  }
}

template <typename T, int VEC, bool ADD>
hipError_t launch(const void* base, const void* lora, const float* g, float s, int64_t T_rows, int64_t d_out,
                  void* out, hipStream_t st) {
  const int64_t ncg = d_out / VEC;
  int64_t tpb = ((ncg + 63) / 64) * 64;
  if (tpb > 256) tpb = 256;
  const int64_t bx = (ncg + tpb - 1) / tpb;
  // About 32 workgroups per compute unit over 256 CUs (8 resident at a
  // time; at 8192 columns each workgroup then streams one group of kUnroll
  // rows): many short row strips balance the tail of the grid best.
  int64_t by = 8192 / bx;
  if (by < 1) by = 1;
  const int64_t row_iters = (T_rows + kUnroll - 1) / kUnroll;
  if (by > row_iters) by = row_iters;
  if (by > 65535) by = 65535;
  hipLaunchKernelGGL((compose_kernel<T, VEC, ADD>), dim3((unsigned)bx, (unsigned)by), dim3((unsigned)tpb), 0, st,
                     static_cast<const T*>(base), static_cast<const T*>(lora), g, s, T_rows, d_out,
                     static_cast<T*>(out));
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Compose backward. For L = sum(dy * delta) with delta as above and the row
// norm detached ("DoRA优化技术解析", cyqw.cn, §4.2, §5.2, §6.1 Table 9 report
// this fused backward; its formulas are the plain derivative):
//   d_base[t,j] = (g[j] - 1) * dy[t,j]
//   d_lora[t,j] = g[j] * (s * dy[t,j])
//   dg[j]       = sum_t dy[t,j] * (base[t,j] + s * lora[t,j])
// Each thread owns one 16-byte column strip and a fixed set of rows, as in
// the forward; with DG it also accumulates its rows' dg terms in fp32
// (fma(dy, fma(s, lora, base), acc), rows in increasing order; in a narrow
// workgroup each row lane does so, and the lanes' sums are then added in
// lane order) and stores one partial per (row block, column). A second
// kernel adds the row-block partials in a fixed order, so dg is
// reproducible; no float atomics.
// With the magnitude frozen (no dg), base and lora are not read at all.
// ---------------------------------------------------------------------------
constexpr int kBwdMaxRowBlocks = 256;
constexpr int64_t kBwdPlainMinBytes = (int64_t)64 << 20;     // per output tensor
constexpr int64_t kInfinityCacheBytes = (int64_t)256 << 20;  // MI355X
constexpr int kBwdTargetBlocks = 256;   // about one workgroup per compute unit

template <typename T, int VEC, bool DG, bool NTS>
__global__ __launch_bounds__(256) void compose_bwd_kernel(const T* dy, const T* base, const T* lora,
                                                          const float* __restrict__ g, float s, int64_t T_rows,
                                                          int64_t d_out, T* d_base, T* d_lora, float* part) {
  using V = typename Strip<T, VEC>::V;
  // threadIdx.x: column strip; threadIdx.y: row lane. A narrow workgroup
  // (few column strips) carries blockDim.y row lanes, so that it still has
  // several waves; lane y of row block b takes rows (b * blockDim.y + y) *
  // kUnroll + ..., stepping gridDim.y * blockDim.y * kUnroll.
  __shared__ float lanes[256 * VEC];
  const int nl = blockDim.y, ly = threadIdx.y;
  const int64_t cg = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool col_ok = cg < d_out / VEC;
  const int64_t c0 = col_ok ? cg * VEC : 0;
  float gv[VEC], gm1[VEC], acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    gv[e] = col_ok ? g[c0 + e] : 0.f;
    gm1[e] = gv[e] - 1.0f;
    acc[e] = 0.f;
  }
  const int64_t step = (int64_t)gridDim.y * nl * kUnroll;
  for (int64_t t0 = ((int64_t)blockIdx.y * nl + ly) * kUnroll; col_ok && t0 < T_rows; t0 += step) {
    V yv[kUnroll], bv[kUnroll], lv[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (t0 + u < T_rows) {
        const int64_t off = (t0 + u) * d_out + c0;
        yv[u] = __builtin_nontemporal_load(reinterpret_cast<const V*>(dy + off));
        if constexpr (DG) {
          bv[u] = __builtin_nontemporal_load(reinterpret_cast<const V*>(base + off));
          lv[u] = __builtin_nontemporal_load(reinterpret_cast<const V*>(lora + off));
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (t0 + u < T_rows) {
        float y[VEC], ob[VEC], ol[VEC];
        unpack<T, VEC>(yv[u], y);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          ob[e] = gm1[e] * y[e];
          ol[e] = gv[e] * (s * y[e]);
        }
        if constexpr (DG) {
          float b[VEC], l[VEC];
          unpack<T, VEC>(bv[u], b);
          unpack<T, VEC>(lv[u], l);
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[e] = fmaf(y[e], fmaf(s, l[e], b[e]), acc[e]);
        }
        const int64_t off = (t0 + u) * d_out + c0;
        if constexpr (NTS) {
          if (d_base != nullptr) __builtin_nontemporal_store(pack<T, VEC>(ob), reinterpret_cast<V*>(d_base + off));
          if (d_lora != nullptr) __builtin_nontemporal_store(pack<T, VEC>(ol), reinterpret_cast<V*>(d_lora + off));
        } else {
          if (d_base != nullptr) *reinterpret_cast<V*>(d_base + off) = pack<T, VEC>(ob);
          if (d_lora != nullptr) *reinterpret_cast<V*>(d_lora + off) = pack<T, VEC>(ol);
        }
      }
    }
  }
  if constexpr (DG) {
    if (nl > 1) {
      // The row lanes' sums, added in lane order by lane 0.
#pragma unroll
      for (int e = 0; e < VEC; ++e) lanes[(ly * blockDim.x + threadIdx.x) * VEC + e] = acc[e];
      __syncthreads();
      if (ly == 0) {
        for (int k = 1; k < nl; ++k)
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[e] += lanes[(k * blockDim.x + threadIdx.x) * VEC + e];
      }
    }
    if (ly == 0 && col_ok) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) part[(int64_t)blockIdx.y * d_out + c0 + e] = acc[e];
    }
  }
}

// dg[j] = sum of the row-block partials; optionally dm[j] = dg[j] /
// max(wnorm[j], eps) (correctly rounded division). One workgroup owns 64
// columns; its four waves each sum a contiguous quarter of the row blocks in
// increasing order (loads issued kBwdBatch at a time, added in order), then
// wave 0 adds the four quarter sums in order. The order is fixed by n_part
// alone, so dg is reproducible.
constexpr int kBwdCols = 64;
constexpr int kBwdSplit = 4;
constexpr int kBwdBatch = 8;

__global__ __launch_bounds__(256) void compose_bwd_reduce_kernel(const float* part, int n_part, int64_t d_out,
                                                                 float* dg, const float* wnorm, float eps,
                                                                 float* dm) {
  __shared__ float red[kBwdSplit][kBwdCols];
  const int c = threadIdx.x % kBwdCols;
  const int q = threadIdx.x / kBwdCols;
  const int64_t j = (int64_t)blockIdx.x * kBwdCols + c;
  const bool live = j < d_out;
  const int y0 = (int)(((int64_t)n_part * q) / kBwdSplit);
  const int y1 = (int)(((int64_t)n_part * (q + 1)) / kBwdSplit);
  float acc = 0.f;
  if (live) {
    const float* col = part + j;
    int y = y0;
    for (; y + kBwdBatch <= y1; y += kBwdBatch) {
      float v[kBwdBatch];
#pragma unroll
      for (int u = 0; u < kBwdBatch; ++u) v[u] = col[(int64_t)(y + u) * d_out];
#pragma unroll
      for (int u = 0; u < kBwdBatch; ++u) acc += v[u];
    }
    for (; y < y1; ++y) acc += col[(int64_t)y * d_out];
  }
  red[q][c] = acc;
  __syncthreads();
  if (q != 0 || !live) return;
  float tot = red[0][c];
#pragma unroll
  for (int k = 1; k < kBwdSplit; ++k) tot += red[k][c];
  dg[j] = tot;
  if (dm != nullptr) {
    const float wn = wnorm[j];
    const float d = (wn < eps) ? eps : wn;
    dm[j] = tot / d;
  }
}

// Launch shape of the backward: one thread per 16-byte strip, and about
// kBwdTargetBlocks workgroups in all (at most max_by row blocks). Fewer,
// longer row strips stream as fast and leave fewer dg partials to reduce.
// A workgroup of fewer than 256 strips gets 256 / tpb row lanes (rows of
// its block taken in turn), so it still has four waves.
struct Grid2 {
  int64_t tpb, bx, by;
  int64_t lanes() const { return tpb <= 128 ? 256 / tpb : 1; }
};
Grid2 strip_grid(int64_t T_rows, int64_t d_out, int vec, int64_t max_by) {
  const int64_t ncg = d_out / vec;
  int64_t tpb = ((ncg + 63) / 64) * 64;
  if (tpb > 256) tpb = 256;
  if (tpb < 64) tpb = 64;
  const int64_t bx = (ncg + tpb - 1) / tpb;
  int64_t by = kBwdTargetBlocks / (bx > 0 ? bx : 1);
  if (by < 1) by = 1;
  const int64_t row_iters = (T_rows + kUnroll - 1) / kUnroll;
  if (by > row_iters) by = row_iters;
  if (by > max_by) by = max_by;
  return Grid2{tpb, bx, by};
}

template <typename T, int VEC>
hipError_t launch_bwd(const void* dy, const void* base, const void* lora, const float* g, float s, int64_t T_rows,
                      int64_t d_out, void* d_base, void* d_lora, float* dg, const float* wnorm, float eps, float* dm,
                      float* part, hipStream_t st) {
  const Grid2 q = strip_grid(T_rows, d_out, VEC, kBwdMaxRowBlocks);
  if (q.by > 0 && q.bx > 0) {
    // Ordinary stores where each output exceeds kBwdPlainMinBytes and both
    // together fit the 256 MiB Infinity Cache, non-temporal ones otherwise.
    // Measured on MI355X (bf16, interleaved in one process): ordinary stores
    // take 6% off the pass at 8192 x 8192 (2 x 128 MiB of output), and add
    // 4-5% at 4096 x 4096 and 8192 x 512, 5% at 8192 x 12288, 6% at
    // 16384 x 8192 and 8192 x 28672.
    const int64_t out_bytes = T_rows * d_out * (int64_t)sizeof(T);
    const bool nts = !(out_bytes > kBwdPlainMinBytes && 2 * out_bytes <= kInfinityCacheBytes);
    const dim3 grid((unsigned)q.bx, (unsigned)q.by), block((unsigned)q.tpb, (unsigned)q.lanes());
    const T* dy_t = static_cast<const T*>(dy);
    const T* base_t = static_cast<const T*>(base);
    const T* lora_t = static_cast<const T*>(lora);
    T* db_t = static_cast<T*>(d_base);
    T* dl_t = static_cast<T*>(d_lora);
    if (dg != nullptr && nts)
      hipLaunchKernelGGL((compose_bwd_kernel<T, VEC, true, true>), grid, block, 0, st, dy_t, base_t, lora_t, g, s,
                         T_rows, d_out, db_t, dl_t, part);
    else if (dg != nullptr)
      hipLaunchKernelGGL((compose_bwd_kernel<T, VEC, true, false>), grid, block, 0, st, dy_t, base_t, lora_t, g, s,
                         T_rows, d_out, db_t, dl_t, part);
    else if (nts)
      hipLaunchKernelGGL((compose_bwd_kernel<T, VEC, false, true>), grid, block, 0, st, dy_t, base_t, lora_t, g, s,
                         T_rows, d_out, db_t, dl_t, part);
    else
      hipLaunchKernelGGL((compose_bwd_kernel<T, VEC, false, false>), grid, block, 0, st, dy_t, base_t, lora_t, g, s,
                         T_rows, d_out, db_t, dl_t, part);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (dg != nullptr) {
    hipLaunchKernelGGL(compose_bwd_reduce_kernel, dim3((unsigned)((d_out + kBwdCols - 1) / kBwdCols)),
                       dim3(kBwdCols * kBwdSplit), 0, st, part,
                       (int)q.by, d_out, dg, wnorm, eps, dm);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_compose(const void* base, const void* lora, const float* g, float s, int dtype, int64_t T,
                          int64_t d_out, void* out, bool vec, bool add_base, hipStream_t st) {
#define DORA_COMPOSE(ADD)                                                                      \
  switch (dtype) {                                                                             \
    case 0:                                                                                    \
      return vec ? launch<bf16_t, 8, ADD>(base, lora, g, s, T, d_out, out, st)                 \
                 : launch<bf16_t, 1, ADD>(base, lora, g, s, T, d_out, out, st);                \
    case 2:                                                                                    \
      return vec ? launch<f16_t, 8, ADD>(base, lora, g, s, T, d_out, out, st)                  \
                 : launch<f16_t, 1, ADD>(base, lora, g, s, T, d_out, out, st);                 \
    default:                                                                                   \
      return vec ? launch<float, 4, ADD>(base, lora, g, s, T, d_out, out, st)                  \
                 : launch<float, 1, ADD>(base, lora, g, s, T, d_out, out, st);                 \
  }
  if (add_base) {
    DORA_COMPOSE(true)
  }
  DORA_COMPOSE(false)
#undef DORA_COMPOSE
}

size_t compose_bwd_workspace_bytes(int64_t T, int64_t d_out) {
  // The most row blocks any strip width (element, fp32 or 16-bit vectors)
  // can take (see strip_grid).
  int64_t by = 0;
  for (int vec : {1, 4, 8}) {
    const int64_t b = strip_grid(T, d_out, vec, kBwdMaxRowBlocks).by;
    by = b > by ? b : by;
  }
  return (size_t)(by * d_out) * 4;
}

hipError_t launch_compose_bwd(const void* dy, const void* base, const void* lora, const float* g, float s, int dtype,
                              int64_t T, int64_t d_out, void* d_base, void* d_lora, float* dg, const float* wnorm,
                              float eps, float* dm, void* ws, bool vec, hipStream_t st) {
  float* part = static_cast<float*>(ws);
  switch (dtype) {
    case 0:
      return vec ? launch_bwd<bf16_t, 8>(dy, base, lora, g, s, T, d_out, d_base, d_lora, dg, wnorm, eps, dm, part, st)
                 : launch_bwd<bf16_t, 1>(dy, base, lora, g, s, T, d_out, d_base, d_lora, dg, wnorm, eps, dm, part, st);
    case 2:
      return vec ? launch_bwd<f16_t, 8>(dy, base, lora, g, s, T, d_out, d_base, d_lora, dg, wnorm, eps, dm, part, st)
                 : launch_bwd<f16_t, 1>(dy, base, lora, g, s, T, d_out, d_base, d_lora, dg, wnorm, eps, dm, part, st);
    default:
      return vec ? launch_bwd<float, 4>(dy, base, lora, g, s, T, d_out, d_base, d_lora, dg, wnorm, eps, dm, part, st)
                 : launch_bwd<float, 1>(dy, base, lora, g, s, T, d_out, d_base, d_lora, dg, wnorm, eps, dm, part, st);
  }
}

}  // namespace dora
