// Device helpers shared by the decode kernels: cross-lane reductions, bf16
// rounding, and the end of a partition (merge of the workgroup's waves,
// then either the final normalisation or the split-K partial).
#pragma once

#include "internal.h"

namespace kvp {

// Rescale threshold (base-2 exponent): a row's running max is only raised
// when a block's score exceeds it by more than this, so weights stay
// <= 2^kRescaleSlack and the accumulators are rescaled rarely.  The result
// is exact either way: numerator and denominator share the same stale max.
constexpr float kRescaleSlack = 8.0f;

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// Two fp32 values rounded to nearest-even bf16 and packed (low half = a);
// one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(unsigned, v);
}

__device__ __forceinline__ uint16_t bf16_rne(float f) { return (uint16_t)(pack_bf16x2(f, 0.f) & 0xffffu); }

__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// max / sum over lanes l, l^16, l^32, l^48 (the four 16-lane rows) with the
// gfx950 row-swap permutes.
__device__ __forceinline__ float rows_max(float x) {
  const unsigned u = __float_as_uint(x);
  auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const unsigned v = __float_as_uint(x);
  auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float rows_sum(float x) {
  const unsigned u = __float_as_uint(x);
  auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const unsigned v = __float_as_uint(x);
  auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <typename OutT>
__device__ __forceinline__ void store_out(void* out, size_t idx, float v) {
  if constexpr (sizeof(OutT) == 2)
    ((uint16_t*)out)[idx] = bf16_rne(v);
  else
    ((float*)out)[idx] = v;
}

// End of one (partition, head group): the waves left their running max
// m_s[w][h] (base 2), weight sum l_s[w][h] and unnormalised output
// o_s[w][h][d] in LDS (synchronised by the caller).  With M = max_w m_w,
//   num = sum_w 2^(m_w - M) o_w,   den = sum_w 2^(m_w - M) l_w.
// A row held by one partition stores num/den (times the V scale of an FP8
// pool, 1 otherwise); otherwise the partition's (M, den, num) go to the
// workspace for decode_reduce.
template <typename OutT, int D, int ROWS>
__device__ __forceinline__ void finish_partition(const DecodeParams& P, float (*o_s)[ROWS][D + 1],
                                                 float (*m_s)[ROWS], float (*l_s)[ROWS], int s, int h0, int nh,
                                                 int part, int nparts) {
  for (int i = threadIdx.x; i < nh * D; i += kThreads) {
    const int hh = i / D, d = i - hh * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, m_s[w][hh]);
    float num = 0.f, den = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = __builtin_amdgcn_exp2f(m_s[w][hh] - M);
        num += f * o_s[w][hh][d];
        den += f * l_s[w][hh];
      }
    }
    const size_t row_h = (size_t)s * P.num_q_heads + h0 + hh;
    if (nparts == 1) {
      store_out<OutT>(P.out, row_h * D + d, den > 0.f ? num / den * P.v_scale : 0.f);
    } else {
      P.part_o[(row_h * P.num_parts + part) * D + d] = num;
      if (d == 0) {
        P.part_ml[(row_h * P.num_parts + part) * 2 + 0] = M;
        P.part_ml[(row_h * P.num_parts + part) * 2 + 1] = den;
      }
    }
  }
}

}  // namespace kvp
