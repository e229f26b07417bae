// Paged decode attention on the CDNA4 matrix cores (bf16 or FP8 pools),
// partitioned form: one workgroup per (partition of a block-table row, KV
// head [, chunk of 16 query heads], sequence).
//
// Its four waves take the partition's table entries round robin.  Per
// 16-token block a wave reads the physical block id from the row
// ("PagedAttention: Virtual Memory for LLMs" in "Optimizing KV Cache Memory
// Management in vLLM with PagedAttention and Dynamic Block Allocation": the
// kernel looks the block up in the table and computes the address), keeps
// the next DEPTH blocks' K/V tiles in flight, and runs the MFMA step of
// mfma_tile.h (S^T = K Q^T for the whole query-head group, online softmax,
// O += P V).  The waves' (max, sum, O) merge in LDS; a row held by one
// partition is normalised and stored at once, otherwise its partial result
// goes to the workspace for decode_reduce.  Tiles are read with
// non-temporal loads (NT) when no block is listed by two rows, each line
// then being read once, and with cached loads when rows share blocks.
#include "mfma_tile.h"

namespace kvp {
namespace {

// Occupancy target (waves per SIMD) the register allocation is held to.
#ifndef KVP_MFMA_WAVES_PER_EU
#define KVP_MFMA_WAVES_PER_EU 2
#endif

template <int D, int DEPTH, bool FP8, int BS, bool NT>  // BS = log2(block size / 16)
__global__ __launch_bounds__(kThreads, KVP_MFMA_WAVES_PER_EU) void decode_mfma_kernel(const DecodeParams P) {
  constexpr int NBUF = DEPTH + 1;
  __shared__ float o_s[kWaves][16][D + 1];
  __shared__ float m_s[kWaves][16];
  __shared__ float l_s[kWaves][16];

  // Grid (head groups, sequences, partitions): consecutive workgroups, which
  // the dispatcher deals round robin to the eight XCDs, differ in head group
  // first, so every XCD gets the same share of every row.
  const int kvh = blockIdx.x / P.qgroups;
  const int qg = blockIdx.x - kvh * P.qgroups;
  const int s = blockIdx.y;
  const int part = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h0 = kvh * P.group + qg * P.heads_per_wg;
  const int nh = min(P.heads_per_wg, P.group - qg * P.heads_per_wg);

  // Lane i holds the id of tile part * part_blocks + i of the row.  With
  // 16-token blocks tile j is table entry j, and the sequence length, the
  // table entries and the queries are independent loads, issued together;
  // 32-token blocks need the length first (a window may start in a block's
  // second tile).
  const int ctx = P.seq_lens[s];
  const int32_t* row = P.block_tables + (size_t)s * P.max_blocks;
  const int jl = part * P.part_blocks + lane;
  int my_id = 0;
  if (BS == 0 && lane < P.part_blocks && jl < P.max_blocks) my_id = row[jl];
  MfmaRow<D> st;
  st.template load_q<FP8>((const uint16_t*)P.q, (size_t)s * P.num_q_heads + h0, nh, lane);
  const RowSpan rs = row_span(ctx, P.window, P.max_blocks, BS);
  const int t0 = BS ? rs.t0 : 0;
  if (BS != 0 && lane < P.part_blocks && jl < rs.nblocks) my_id = row[(t0 + jl) >> BS];
  const int nparts = (rs.nblocks + P.part_blocks - 1) / P.part_blocks;
  if (rs.nblocks == 0) {
    if (part == 0)
      for (int i = threadIdx.x; i < nh * D; i += kThreads)
        ((uint16_t*)P.out)[((size_t)s * P.num_q_heads + h0) * D + i] = 0;
    return;
  }
  if (part >= nparts) return;
  const int jb = part * P.part_blocks;
  const int nbp = min(P.part_blocks, rs.nblocks - jb);

  const void* pool = P.pool_layer;
  const MfmaLanes la = mfma_lanes<D, BS, FP8>(P.num_kv_heads, kvh, lane);
  st.reset();
  const int so = rs.start_off;
  const int send = rs.start_off + rs.n;

  // Tiles of this wave: wave, wave + 4, ...; `cnt` of them.
  const int cnt = nbp > wave ? (nbp - wave + kWaves - 1) / kWaves : 0;
  auto issue = [&](int k, MfmaTiles<D, FP8>& t) {
    if (k >= cnt) {  // past the end: loads of a line just read (this row's queries)
      mfma_issue_hot(t, (const uint16_t*)P.q + ((size_t)s * P.num_q_heads + h0) * D);
      return;
    }
    mfma_issue<BS, NT>(t, pool, la, __builtin_amdgcn_readlane(my_id, wave + k * kWaves),
                       (t0 + jb + wave + k * kWaves) & ((1 << BS) - 1), P.num_blocks);
  };

  // Software pipeline: the loads of block k + DEPTH are issued before block k
  // is computed; the scheduling barrier keeps the compiler from sinking them
  // below the compute, so DEPTH blocks stay in flight while one is consumed.
  if (cnt > 0) {
    MfmaTiles<D, FP8> buf[NBUF];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      issue(d, buf[d]);
      __builtin_amdgcn_sched_barrier(0);  // keep the blocks in issue order
    }
    for (int k0 = 0; k0 < cnt; k0 += NBUF) {
#pragma unroll
      for (int u = 0; u < NBUF; ++u) {
        if (k0 + u >= cnt) break;
        issue(k0 + u + DEPTH, buf[(u + DEPTH) % NBUF]);
        __builtin_amdgcn_sched_barrier(0);
        st.step(buf[u], jb + wave + (k0 + u) * kWaves, so, send, rs.nblocks, P.scale_log2, lane);
      }
    }
  }

  // Wave totals: the sum over the four row groups; the max is already uniform.
  const float l_tot = rows_sum(st.l_run);
  if (lane < 16) {
    m_s[wave][lane] = st.m_run;
    l_s[wave][lane] = l_tot;
  }
  const int q4 = lane >> 4;
#pragma unroll
  for (int n = 0; n < D / 16; ++n)
#pragma unroll
    for (int r = 0; r < 4; ++r) o_s[wave][4 * q4 + r][acc_dim<FP8>(n, lane & 15)] = st.acc[n][r];
  __syncthreads();
  finish_partition<uint16_t, D, 16>(P, o_s, m_s, l_s, s, h0, nh, part, nparts);
}

template <int D, bool FP8, int BS, bool NT>
hipError_t launch_d(const DecodeParams& p, hipStream_t stream) {
  const dim3 grid(p.num_kv_heads * p.qgroups, p.num_seqs, p.num_parts);
  const dim3 block(kThreads);
  switch (p.depth) {
    case 1: hipLaunchKernelGGL((decode_mfma_kernel<D, 1, FP8, BS, NT>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((decode_mfma_kernel<D, 2, FP8, BS, NT>), grid, block, 0, stream, p); break;
    case 3: hipLaunchKernelGGL((decode_mfma_kernel<D, 3, FP8, BS, NT>), grid, block, 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D, bool NT>
hipError_t launch_dn(const DecodeParams& p, hipStream_t stream) {
  if (p.kv_fp8) return p.bshift ? launch_d<D, true, 1, NT>(p, stream) : launch_d<D, true, 0, NT>(p, stream);
  return p.bshift ? launch_d<D, false, 1, NT>(p, stream) : launch_d<D, false, 0, NT>(p, stream);
}

template <int D>
hipError_t launch_dt(const DecodeParams& p, hipStream_t stream) {
  return p.nt_loads ? launch_dn<D, true>(p, stream) : launch_dn<D, false>(p, stream);
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeParams& p, int head_dim, hipStream_t stream) {
  if (head_dim == 128) return launch_dt<128>(p, stream);
  if (head_dim == 64) return launch_dt<64>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace kvp
