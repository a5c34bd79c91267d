// Device-side helpers shared by the libdora kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dora {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Storage types: bf16 is carried as its 16 raw bits; fp16 is the native
// half type.
typedef uint16_t bf16_t;
typedef _Float16 f16_t;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

template <typename T>
struct Elem;
template <>
struct Elem<bf16_t> {
  static constexpr int esz = 2;
  static constexpr int epc = 8;         // elements per 16-byte chunk
  static constexpr int frag_chunks = 1; // 16-byte chunks per MFMA operand fragment
};
template <>
struct Elem<f16_t> {
  static constexpr int esz = 2;
  static constexpr int epc = 8;
  static constexpr int frag_chunks = 1;
};
template <>
struct Elem<float> {
  static constexpr int esz = 4;
  static constexpr int epc = 4;
  static constexpr int frag_chunks = 2;
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// Round-to-nearest-even fp32 -> bf16 (hardware v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16_t f32_to_bf16_rne(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(bf16_t, h);
}

__device__ __forceinline__ float to_f32(bf16_t v) { return bf16_bits_to_f32(v); }

// Eight fp16 values of a 16-byte chunk split exactly into bf16 hi + lo:
// hi = the value rounded to bf16, lo = the remainder. fp16 carries 11
// significant bits and bf16 8 over a wider exponent range, so the
// remainder (at most 4 bits) is exact in bf16 and hi + lo equals the value.
// Returns the hi parts, or the lo parts, in the same element order.
__device__ __forceinline__ u32x4 f16_split_bf16(const u32x4& v, bool lo) {
  const f16x8 h = __builtin_bit_cast(f16x8, v);   // (by value: no address taken)
  u32x4 r;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float a = (float)h[2 * w], b = (float)h[2 * w + 1];
    uint32_t ha = f32_to_bf16_rne(a), hb = f32_to_bf16_rne(b);
    if (lo) {
      ha = f32_to_bf16_rne(a - bf16_bits_to_f32(ha));
      hb = f32_to_bf16_rne(b - bf16_bits_to_f32(hb));
    }
    r[w] = ha | (hb << 16);
  }
  return r;
}
__device__ __forceinline__ float to_f32(f16_t v) { return (float)v; }
__device__ __forceinline__ float to_f32(float v) { return v; }

template <typename T>
__device__ __forceinline__ T from_f32(float f);
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float f) { return f32_to_bf16_rne(f); }
template <>
__device__ __forceinline__ f16_t from_f32<f16_t>(float f) { return (f16_t)f; }   // round to nearest even
template <>
__device__ __forceinline__ float from_f32<float>(float f) { return f; }

// Sum of squares of the elements held in one 16-byte chunk. For bf16 the
// pairs go through v_dot2_f32_bf16 (each bf16 square is exact in fp32). The
// chunk is reinterpreted as a whole: bit-casting its 32-bit elements one by
// one inside an unrolled loop was compiled into four dots of element 0.
__device__ __forceinline__ float chunk_sumsq(const u32x4& v, bf16_t) {
  const bf16x8 h = __builtin_bit_cast(bf16x8, v);
  float q = 0.f;
  q = __builtin_amdgcn_fdot2_f32_bf16(h.s01, h.s01, q, false);
  q = __builtin_amdgcn_fdot2_f32_bf16(h.s23, h.s23, q, false);
  q = __builtin_amdgcn_fdot2_f32_bf16(h.s45, h.s45, q, false);
  q = __builtin_amdgcn_fdot2_f32_bf16(h.s67, h.s67, q, false);
  return q;
}
// fp16: v_dot2_f32_f16 on pairs (each fp16 square is exact in fp32).
__device__ __forceinline__ float chunk_sumsq(const u32x4& v, f16_t) {
  const f16x8 h = __builtin_bit_cast(f16x8, v);
  float q = 0.f;
  q = __builtin_amdgcn_fdot2(h.s01, h.s01, q, false);
  q = __builtin_amdgcn_fdot2(h.s23, h.s23, q, false);
  q = __builtin_amdgcn_fdot2(h.s45, h.s45, q, false);
  q = __builtin_amdgcn_fdot2(h.s67, h.s67, q, false);
  return q;
}
__device__ __forceinline__ float chunk_sumsq(const u32x4& v, float) {
  const float a = __uint_as_float(v[0]), b = __uint_as_float(v[1]);
  const float c = __uint_as_float(v[2]), d = __uint_as_float(v[3]);
  return fmaf(a, a, b * b) + fmaf(c, c, d * d);
}

// One 16-byte chunk of a row: elements [k, k+EPC) of `row`, zero-filled past
// d_in or when the row is out of range. `vec` means the row start and d_in
// allow an aligned 16-byte load.
template <typename T>
__device__ __forceinline__ u32x4 load_chunk(const T* row, int64_t k, int64_t d_in, bool row_ok,
                                            bool vec) {
  u32x4 v = {0u, 0u, 0u, 0u};
  if (!row_ok || k >= d_in) return v;
  if (vec) return *reinterpret_cast<const u32x4*>(row + k);
  constexpr int EPC = Elem<T>::epc;
  T tmp[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) tmp[e] = (k + e < d_in) ? row[k + e] : T(0);
  __builtin_memcpy(&v, tmp, 16);
  return v;
}

// One 16-byte-per-lane direct load into LDS: lane l's 16 bytes from
// base + voff + soff land at lds + 16*l. The buffer descriptor spans
// [base, base + nbytes); a lane whose offset lies past it reads zeros.
__device__ __forceinline__ void lds_load16(const void* base, int nbytes, void* lds, uint32_t voff, uint32_t soff) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nbytes,
                                                                        0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}

// Wait until every direct-to-LDS load this wave issued has landed (vmcnt 0;
// the export and LDS counters are left alone). Called before the barrier
// that hands the loaded data to the other waves.
__device__ __forceinline__ void wait_lds_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// XOR swizzle of 16-byte chunks inside LDS rows of CPR chunks, so that the
// 32 rows one MFMA fragment read touches spread over all LDS banks.
template <int CPR>
__device__ __forceinline__ int swz(int row, int c) {
  if constexpr (CPR == 8) {
    return c ^ (row & 7);
  } else {
    static_assert(CPR == 4, "LDS rows are 64 or 128 bytes");
    return c ^ ((row >> 1) & 3);
  }
}

// acc += A_frag * B_frag over one 16-deep slice of K.
// bf16: one v_mfma_f32_32x32x16_bf16; fp16: one v_mfma_f32_32x32x16_f16.
// fp32: eight v_mfma_f32_32x32x2_f32,
// element e of both fragments forming the e-th pair of K indices.
template <typename T>
struct Mfma;
template <>
struct Mfma<bf16_t> {
  static __device__ __forceinline__ f32x16 run(const u32x4* a, const u32x4* b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[0]),
                                                   __builtin_bit_cast(bf16x8, b[0]), c, 0, 0, 0);
  }
};
template <>
struct Mfma<f16_t> {
  static __device__ __forceinline__ f32x16 run(const u32x4* a, const u32x4* b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a[0]), __builtin_bit_cast(f16x8, b[0]),
                                                  c, 0, 0, 0);
  }
};
template <>
struct Mfma<float> {
  static __device__ __forceinline__ f32x16 run(const u32x4* a, const u32x4* b, f32x16 c) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[h][e]), __uint_as_float(b[h][e]),
                                                 c, 0, 0, 0);
    return c;
  }
};

// Row (within a 32x32 block) of accumulator register v for this lane:
// lanes 0-31 hold rows {0-3, 8-11, 16-19, 24-27}, lanes 32-63 the other four
// of each group of eight; the column is lane % 32.
__device__ __forceinline__ int acc_row(int v, int lgrp) { return 8 * (v >> 2) + 4 * lgrp + (v & 3); }

// Lane exchange inside each 32-lane half: value of lane (i ^ M).
template <int M>
__device__ __forceinline__ float swz_xor(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x1F | (M << 10)));
}

// Sum 16 per-lane values over the 32 lanes of each wave half, returning in
// lane i (of its half) the total of value index (i >> 1). Each exchange
// halves the values a lane keeps, so the 16 sums cost 16 lane exchanges.
// The summation order is fixed, so results are reproducible.
__device__ __forceinline__ float sum32_transpose(const float (&p)[16], int lane) {
  const int i = lane & 31;
  float q8[8], q4[4], q2[2];
  const bool b4 = (i & 16) != 0, b3 = (i & 8) != 0, b2 = (i & 4) != 0, b1 = (i & 2) != 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float keep = b4 ? p[8 + j] : p[j];
    const float send = b4 ? p[j] : p[8 + j];
    q8[j] = keep + swz_xor<16>(send);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float keep = b3 ? q8[4 + j] : q8[j];
    const float send = b3 ? q8[j] : q8[4 + j];
    q4[j] = keep + swz_xor<8>(send);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float keep = b2 ? q4[2 + j] : q4[j];
    const float send = b2 ? q4[j] : q4[2 + j];
    q2[j] = keep + swz_xor<4>(send);
  }
  const float keep = b1 ? q2[1] : q2[0];
  const float send = b1 ? q2[0] : q2[1];
  const float q1 = keep + swz_xor<2>(send);
  return q1 + swz_xor<1>(q1);
}

}  // namespace dora
