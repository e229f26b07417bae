// Second pass of split-K paged decode attention: merge the partitions of a
// row.  Partition p left its running max m_p (base 2), its weight sum l_p
// and its unnormalised output o_p; with M = max_p m_p
//     out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p,
// the same log-sum-exp merge the decode kernels use between their waves.
// Rows that fit in one partition were finished by the first pass.
//
// One wave per (sequence, query head); each lane owns D/64 output
// dimensions.
#include "decode_common.h"

namespace kvp {
namespace {

constexpr int kRowsPerWg = 4;  // waves, one query-head row each

template <int D, typename OutT>
__global__ __launch_bounds__(64 * kRowsPerWg) void decode_reduce_kernel(const DecodeParams P) {
  const int s = blockIdx.y;
  const RowSpan rs = row_span(P.seq_lens[s], P.window, P.max_blocks, P.bshift);
  const int nparts = (rs.nblocks + P.part_blocks - 1) / P.part_blocks;
  if (nparts <= 1) return;
  const int h = blockIdx.x * kRowsPerWg + (threadIdx.x >> 6);
  if (h >= P.num_q_heads) return;
  const int lane = threadIdx.x & 63;
  const size_t row_h = (size_t)s * P.num_q_heads + h;
  const float* ml = P.part_ml + row_h * P.num_parts * 2;
  const float* o = P.part_o + row_h * P.num_parts * D;

  // Every lane reads all partitions' (m, l) (the same addresses across the
  // wave) together with its own output dimensions of all partitions, so the
  // whole merge waits on one round of loads; longer rows go in chunks with
  // a running max.
  constexpr int PER = D / 64;  // output dimensions per lane
  constexpr int CH = 16;       // partitions per chunk
  float M = -INFINITY, den = 0.f, num[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) num[e] = 0.f;
  for (int p0 = 0; p0 < nparts; p0 += CH) {
    float m[CH], l[CH], v[CH][PER];
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int p = p0 + u < nparts ? p0 + u : nparts - 1;
      m[u] = p0 + u < nparts ? ml[2 * p] : -INFINITY;
      l[u] = ml[2 * p + 1];
#pragma unroll
      for (int e = 0; e < PER; ++e) v[u][e] = o[(size_t)p * D + lane + 64 * e];
    }
    float Mc = M;
#pragma unroll
    for (int u = 0; u < CH; ++u) Mc = fmaxf(Mc, m[u]);
    if (Mc == -INFINITY) continue;
    const float a = __builtin_amdgcn_exp2f(M - Mc);
    den *= a;
#pragma unroll
    for (int e = 0; e < PER; ++e) num[e] *= a;
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const float w = __builtin_amdgcn_exp2f(m[u] - Mc);
      den += w * l[u];
#pragma unroll
      for (int e = 0; e < PER; ++e) num[e] += w * v[u][e];
    }
    M = Mc;
  }
  const float inv = den > 0.f ? P.v_scale / den : 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) store_out<OutT>(P.out, row_h * D + lane + 64 * e, num[e] * inv);
}

template <int D, typename OutT>
hipError_t launch_t(const DecodeParams& p, hipStream_t stream) {
  const dim3 grid((p.num_q_heads + kRowsPerWg - 1) / kRowsPerWg, p.num_seqs);
  hipLaunchKernelGGL((decode_reduce_kernel<D, OutT>), grid, dim3(64 * kRowsPerWg), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_reduce(const DecodeParams& p, int dtype, int head_dim, hipStream_t stream) {
  // bf16 and FP8 pools produce bf16 outputs, fp32 pools fp32
  if (head_dim == 128) return dtype != 0 ? launch_t<128, uint16_t>(p, stream) : launch_t<128, float>(p, stream);
  return dtype != 0 ? launch_t<64, uint16_t>(p, stream) : launch_t<64, float>(p, stream);
}

}  // namespace kvp
