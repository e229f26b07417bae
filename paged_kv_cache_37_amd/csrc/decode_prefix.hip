// Shared-prefix (cascade) pass of paged decode attention on the CDNA4 matrix
// cores (bf16 or FP8 pools).
//
// When every sequence of a batch starts with the same physical blocks (a
// cached prefix that all of them reference: [Pool] "Finding a prefix again"
// and [Memory] "How vLLM recognizes a reusable prefix" describe how
// requests come to share blocks; [Optimizing] "Copy-on-Write (CoW) for
// Parallel Sampling and Prefix Caching" how a shared block stays one
// physical block), attention over those keys is one dense problem per KV
// head: all S * G query rows against the same prefix keys.  This pass
// computes it once per KV head instead of once per sequence: a wave takes
// 16 query rows (the 16 columns of the MFMA B operand, drawn from any
// sequences) and a quarter of the prefix blocks; the workgroup's four waves
// merge in LDS and leave, per (sequence, query head), the running max (base
// 2), the weight sum and the unnormalised output.  The streaming pass then
// attends only the private tails, and the merge pass combines the two.
// Only full blocks are hashed and reused ([Pool] "Finding a prefix again",
// [Memory] "How vLLM recognizes a reusable prefix"), so every shared prefix
// block is full and none of its slots is masked.
#include "mfma_tile.h"

namespace kvp {
namespace {

template <int D, int DEPTH, bool FP8, int BS>  // BS = log2(block size / 16)
__global__ __launch_bounds__(kThreads, 2) void decode_prefix_kernel(const DecodeParams P) {
  constexpr int NBUF = DEPTH + 1;
  __shared__ float o_s[kWaves][16][D + 1];
  __shared__ float m_s[kWaves][16];
  __shared__ float l_s[kWaves][16];
  __shared__ int ids_s[kWaves][kMaxPrefixBlocks / kWaves];

  const int G = P.group;
  const int rows = P.num_seqs * G;  // query rows per KV head
  const int tiles = (rows + 15) >> 4;
  // Workgroup i runs on XCD i mod 8: number the work XCD by XCD so that the
  // row tiles of one KV head, which all read that head's prefix, share one
  // XCD's L2 (one head's prefix, not all of them, per L2).
  const int nwg = gridDim.x, x = blockIdx.x & 7, k = blockIdx.x >> 3;
  const int idx = x * (nwg >> 3) + min(x, nwg & 7) + k;
  const int kvh = idx / tiles;
  const int tile = idx - kvh * tiles;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // Query row of this lane's B column: tile * 16 + lane % 16 = s * G + g.
  MfmaRow<D> st;
  {
    const int r = tile * 16 + (lane & 15);
    const int s = r / G, g = r - (r / G) * G;
    const uint16_t* qp = (const uint16_t*)P.q + ((size_t)s * P.num_q_heads + kvh * G + g) * D + 8 * (lane >> 4);
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) st.qop[kk] = r < rows ? *(const uint4_v*)(qp + 32 * kk) : uint4_v{0, 0, 0, 0};
  }
  st.reset();

  // This wave's contiguous quarter of the prefix tiles (16 tokens each; a
  // 32-token block holds two); their ids from the first entries of row 0,
  // the same in every row.
  const int nb = P.prefix_blocks << BS;
  const int j0 = (int)(((long long)nb * wave) >> 2), j1 = (int)(((long long)nb * (wave + 1)) >> 2);
  const int cnt = j1 - j0;
  // The blocks of the wave's tiles, staged in LDS.  The row tiles of one KV head all
  // read the same blocks: each starts its walk at a different tile, so that
  // concurrent waves spread over the L2 channels.
  for (int i = lane; i < cnt; i += 64) ids_s[wave][i] = P.block_tables[(j0 + i) >> BS];
  const int rot = cnt > 0 ? (int)(((long long)tile * 37) % cnt) : 0;
  const void* pool = P.pool_layer;
  const MfmaLanes la = mfma_lanes<D, BS>(P.num_kv_heads, kvh, lane);
  int issued = 0;
  auto issue = [&](MfmaTiles<D, FP8>& t) {
    const int k = issued < cnt ? issued : cnt - 1;  // past the end: re-read the last block (a cache hit)
    const int kr = k + rot < cnt ? k + rot : k + rot - cnt;
    mfma_issue<BS>(t, pool, la, __builtin_amdgcn_readfirstlane(ids_s[wave][kr]), (j0 + kr) & ((1 << BS) - 1),
                   P.num_blocks);
    ++issued;
  };

  if (cnt > 0) {
    MfmaTiles<D, FP8> buf[NBUF];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      issue(buf[d]);
      __builtin_amdgcn_sched_barrier(0);
    }
    for (int k0 = 0; k0 < cnt; k0 += NBUF) {
#pragma unroll
      for (int u = 0; u < NBUF; ++u) {
        if (k0 + u >= cnt) break;
        issue(buf[(u + DEPTH) % NBUF]);
        __builtin_amdgcn_sched_barrier(0);
        // every prefix block is full: only a tile outside the pool is masked
        st.step(buf[u], 0, 0, nb * kBlock, nb, P.scale_log2, lane);
      }
    }
  }

  // Merge the four waves: M = max_w m_w, L = sum_w 2^(m_w - M) l_w,
  // O = sum_w 2^(m_w - M) o_w, per query row.
  const float l_tot = rows_sum(st.l_run);
  if (lane < 16) {
    m_s[wave][lane] = st.m_run;
    l_s[wave][lane] = l_tot;
  }
  const int q4 = lane >> 4;
#pragma unroll
  for (int n = 0; n < D / 16; ++n)
#pragma unroll
    for (int r = 0; r < 4; ++r) o_s[wave][4 * q4 + r][32 * (n >> 1) + 2 * (lane & 15) + (n & 1)] = st.acc[n][r];
  __syncthreads();
  for (int i = threadIdx.x; i < 16 * D; i += kThreads) {
    const int rr = i / D, d = i - rr * D;
    const int r = tile * 16 + rr;
    if (r >= rows) continue;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, m_s[w][rr]);
    float num = 0.f, den = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = __builtin_amdgcn_exp2f(m_s[w][rr] - M);
        num += f * o_s[w][rr][d];
        den += f * l_s[w][rr];
      }
    }
    const int s = r / G, g = r - (r / G) * G;
    const size_t qh = (size_t)s * P.num_q_heads + kvh * G + g;
    P.pre_o[qh * D + d] = num;
    if (d == 0) {
      P.pre_ml[qh * 2 + 0] = M;
      P.pre_ml[qh * 2 + 1] = den;
    }
  }
}

template <int D>
hipError_t launch_p(const DecodeParams& p, unsigned grid, hipStream_t stream) {
  const dim3 g(grid), b(kThreads);
  if (p.kv_fp8 && p.bshift)
    hipLaunchKernelGGL((decode_prefix_kernel<D, 2, true, 1>), g, b, 0, stream, p);
  else if (p.kv_fp8)
    hipLaunchKernelGGL((decode_prefix_kernel<D, 2, true, 0>), g, b, 0, stream, p);
  else if (p.bshift)
    hipLaunchKernelGGL((decode_prefix_kernel<D, 2, false, 1>), g, b, 0, stream, p);
  else
    hipLaunchKernelGGL((decode_prefix_kernel<D, 2, false, 0>), g, b, 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_prefix(const DecodeParams& p, int head_dim, hipStream_t stream) {
  const long long tiles = ((long long)p.num_seqs * p.group + 15) / 16;
  const long long grid = tiles * p.num_kv_heads;
  if (grid <= 0 || grid > 0x7fffffff) return hipErrorInvalidValue;
  if (head_dim == 128) return launch_p<128>(p, (unsigned)grid, stream);
  if (head_dim == 64) return launch_p<64>(p, (unsigned)grid, stream);
  return hipErrorInvalidValue;
}

}  // namespace kvp
