// Paged decode attention on the CDNA4 matrix cores (bf16 pools).
//
// One workgroup = (partition of a block-table row, KV head [, chunk of 16
// query heads], sequence); its four waves take the partition's table
// entries round robin.  Per 16-token block a wave
//   1. reads the physical block id from the row ("PagedAttention: Virtual
//      Memory for LLMs" in "Optimizing KV Cache Memory Management in vLLM
//      with PagedAttention and Dynamic Block Allocation": the kernel looks the
//      block up in the table and computes the address);
//   2. has the K tile (4 KiB for head_dim 128) and V tile of the next DEPTH
//      blocks already in flight (16-byte loads into a ring of registers);
//   3. S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (16 tokens x up to 16 query
//      heads of the group; the KV tile is loaded once for the whole group);
//   4. masks slots outside the attended span, exponentiates in base 2
//      against the row's running max, which is raised (with a rescale of the
//      accumulators) only when a score exceeds it by more than 2^8;
//   5. O += P V with v_mfma_f32_16x16x16_bf16, P rounded to bf16 (the
//      running sum uses the same rounded weights).
// The waves' (max, sum, O) merge in LDS; a row held by one partition is
// normalised and stored at once, otherwise the last workgroup of the row to
// finish merges the partitions (decode_common.h).
//
// Operand layouts (16x16 MFMA, lane l, row group q = l / 16):
//   A of 16x16x32 : A[l % 16][8q .. 8q+7]      -> K[token l%16][32kk + 8q ..]
//   B of 16x16x32 : B[8q .. 8q+7][l % 16]      -> Q[head l%16][32kk + 8q ..]
//   C             : C[4q + r][l % 16], r<4     -> S[token 4q+r][head l%16]
//   A of 16x16x16 : A[l % 16][4q .. 4q+3]      -> P[head l%16][token 4q..4q+3]
//                   (exactly the C layout above, no shuffle needed)
//   B of 16x16x16 : B[4q .. 4q+3][l % 16]      -> V[token 4q..4q+3][dim]
// The V tile is stored as [4][D][4] (four slots of one dimension adjacent),
// so one 16-byte load gives a lane two dimensions x four tokens: the B
// operands of two PV MFMAs (column j of MFMA 2m+e is dimension 32m+2j+e).
#include "decode_common.h"

namespace kvp {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short short4v;
typedef __attribute__((ext_vector_type(8))) short short8v;
typedef __attribute__((ext_vector_type(4))) float float4v;
typedef __attribute__((ext_vector_type(4))) unsigned uint4v;

template <int D>
struct Tiles {
  uint4v k[D / 32];  // K operand: token l%16, dims 32kk + 8q .. +7
  uint4v v[D / 32];  // V operand: tokens 4q..4q+3 of dims 32m + 2(l%16), +1
  bool bad;          // block id outside the pool: contributes nothing
};

template <int D, int DEPTH>
__global__ __launch_bounds__(kThreads, 2) void decode_mfma_kernel(const DecodeParams P) {
  constexpr int KK = D / 32;  // QK^T MFMAs per block (k = 32 dims each)
  constexpr int NV = D / 16;  // PV MFMAs per block (16 output dims each)
  constexpr int NBUF = DEPTH + 1;
  __shared__ float o_s[kWaves][16][D + 1];
  __shared__ float m_s[kWaves][16];
  __shared__ float l_s[kWaves][16];

  const int part = blockIdx.x;
  const int kvh = blockIdx.y / P.qgroups;
  const int qg = blockIdx.y - kvh * P.qgroups;
  const int s = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h0 = kvh * P.group + qg * P.heads_per_wg;
  const int nh = min(P.heads_per_wg, P.group - qg * P.heads_per_wg);

  const RowSpan rs = row_span(P.seq_lens[s], P.window, P.max_blocks);
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

  // Physical ids of this partition's table entries: lane i holds entry jb+i.
  const int32_t* row = P.block_tables + (size_t)s * P.max_blocks + jb;
  const int my_id = lane < nbp ? row[lane] : 0;

  // Q as the B operand of S^T = K Q^T: column = query head l%16 of this group.
  const int g = lane & 15;
  const int q4 = lane >> 4;
  uint4v qop[KK];
  {
    const uint16_t* qp = (const uint16_t*)P.q + ((size_t)s * P.num_q_heads + h0 + g) * D + 8 * q4;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qop[kk] = g < nh ? *(const uint4v*)(qp + 32 * kk) : uint4v{0, 0, 0, 0};
  }

  const uint16_t* pool = (const uint16_t*)P.pool_layer;
  const size_t tile = (size_t)16 * D;
  const size_t blk_stride = 2 * (size_t)P.num_kv_heads * tile;
  const size_t k_off = (size_t)kvh * tile;              // K tile of this head
  const size_t v_rel = (size_t)P.num_kv_heads * tile;  // V tile = K tile + v_rel
  const int k_lane = (lane & 15) * D + 8 * q4;         // + 32 kk
  const int v_lane = (q4 * D + 2 * (lane & 15)) * 4;   // + 128 m

  float m_run = -INFINITY;  // running max of row (head) l%16, base 2
  float l_run = 0.f;        // this lane's share of the row's weight sum
  float4v acc[NV];
#pragma unroll
  for (int n = 0; n < NV; ++n) acc[n] = float4v{0.f, 0.f, 0.f, 0.f};

  const int so = rs.start_off;
  const int send = rs.start_off + rs.n;

  // Table entries of this wave: wave, wave + 4, ...; `cnt` of them.
  const int cnt = nbp > wave ? (nbp - wave + kWaves - 1) / kWaves : 0;

  auto issue = [&](int k, Tiles<D>& t) {
    const int kc = k < cnt ? k : cnt - 1;  // past the end: re-read the last block (a cache hit)
    int id = __builtin_amdgcn_readlane(my_id, wave + kc * kWaves);
    t.bad = (unsigned)id >= (unsigned)P.num_blocks;
    if (t.bad) id = 0;
    const uint16_t* kt = pool + (size_t)id * blk_stride + k_off;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) t.k[kk] = *(const uint4v*)(kt + k_lane + 32 * kk);
#pragma unroll
    for (int m = 0; m < D / 32; ++m) t.v[m] = *(const uint4v*)(kt + v_rel + v_lane + 128 * m);
  };

  auto compute = [&](int k, Tiles<D>& t) {
    const int J = jb + wave + k * kWaves;  // table entry
    float4v sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, t.k[kk]),
                                                     __builtin_bit_cast(bf16x8, qop[kk]), sacc, 0, 0, 0);
    float sv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) sv[r] = sacc[r] * P.scale_log2;
    const bool edge = t.bad || (J == 0 && so > 0) || (J == rs.nblocks - 1 && (send & 15) != 0);
    if (edge) {
      unsigned vm[2];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int u0 = J * 16 + 4 * q4 + 2 * half;
        const bool a = !t.bad && u0 >= so && u0 < send;
        const bool b = !t.bad && u0 + 1 >= so && u0 + 1 < send;
        if (!a) sv[2 * half] = -INFINITY;
        if (!b) sv[2 * half + 1] = -INFINITY;
        vm[half] = (a ? 0xffffu : 0u) | (b ? 0xffff0000u : 0u);
      }
#pragma unroll
      for (int m = 0; m < D / 32; ++m) {
        t.v[m].x &= vm[0];
        t.v[m].y &= vm[1];
        t.v[m].z &= vm[0];
        t.v[m].w &= vm[1];
      }
    }
    const float lmax = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    if (__any(lmax > m_run + kRescaleSlack)) {
      const float m_new = fmaxf(m_run, rows_max(lmax));
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      m_run = m_new;
      l_run *= alpha;
      // rows of O in this lane are heads 4*q4 + r
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float ar = __shfl(alpha, 4 * q4 + r);
#pragma unroll
        for (int n = 0; n < NV; ++n) acc[n][r] *= ar;
      }
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    const unsigned p01 = pack_bf16x2(__builtin_amdgcn_exp2f(sv[0] - m_use), __builtin_amdgcn_exp2f(sv[1] - m_use));
    const unsigned p23 = pack_bf16x2(__builtin_amdgcn_exp2f(sv[2] - m_use), __builtin_amdgcn_exp2f(sv[3] - m_use));
    l_run += (bf16_lo(p01) + bf16_hi(p01)) + (bf16_lo(p23) + bf16_hi(p23));
    const short4v pa = __builtin_bit_cast(short4v, (unsigned __attribute__((ext_vector_type(2)))){p01, p23});
#pragma unroll
    for (int m = 0; m < D / 32; ++m) {
      const short8v vv = __builtin_bit_cast(short8v, t.v[m]);
      acc[2 * m] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, __builtin_shufflevector(vv, vv, 0, 1, 2, 3),
                                                             acc[2 * m], 0, 0, 0);
      acc[2 * m + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, __builtin_shufflevector(vv, vv, 4, 5, 6, 7),
                                                                 acc[2 * m + 1], 0, 0, 0);
    }
  };

  // Software pipeline: the loads of block k + DEPTH are issued before block k
  // is computed; the scheduling barrier keeps the compiler from sinking them
  // below the compute, so DEPTH blocks stay in flight while one is consumed.
  if (cnt > 0) {
    Tiles<D> buf[NBUF];
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
        compute(k0 + u, buf[u]);
      }
    }
  }

  // Wave totals: the sum over the four row groups; the max is already uniform.
  l_run = rows_sum(l_run);
  if (lane < 16) {
    m_s[wave][lane] = m_run;
    l_s[wave][lane] = l_run;
  }
#pragma unroll
  for (int n = 0; n < NV; ++n)
#pragma unroll
    for (int r = 0; r < 4; ++r) o_s[wave][4 * q4 + r][32 * (n >> 1) + 2 * (lane & 15) + (n & 1)] = acc[n][r];
  __syncthreads();
  finish_partition<uint16_t, D, 16>(P, o_s, m_s, l_s, s, h0, nh, part, nparts);
}

template <int D>
hipError_t launch_d(const DecodeParams& p, hipStream_t stream) {
  const dim3 grid(p.num_parts, p.num_kv_heads * p.qgroups, p.num_seqs);
  const dim3 block(kThreads);
  switch (p.depth) {
    case 1: hipLaunchKernelGGL((decode_mfma_kernel<D, 1>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((decode_mfma_kernel<D, 2>), grid, block, 0, stream, p); break;
    case 3: hipLaunchKernelGGL((decode_mfma_kernel<D, 3>), grid, block, 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeParams& p, int head_dim, hipStream_t stream) {
  if (head_dim == 128) return launch_d<128>(p, stream);
  if (head_dim == 64) return launch_d<64>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace kvp
