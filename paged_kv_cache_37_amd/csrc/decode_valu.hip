// Paged decode attention on the vector ALUs (fp32 and bf16 pools).
//
// Same decomposition as the matrix-core kernel -- a workgroup per
// (partition, KV head [, query-head chunk], sequence), four waves taking the
// partition's table entries round robin, one block of prefetch -- but QK^T
// and PV are plain fp32 FMAs (bf16 x bf16 dot2 for QK^T on bf16 pools).
//
// Per block and wave, for a group of GT query heads sharing the KV head:
//   K: lane l holds token l/4 and the 16-byte chunks c, c+4, c+8, ... of its
//      row (c = l%4): a partial dot product per head, summed over the four
//      lanes of the quad with DPP.
//   V: lane l holds the four tokens 4(l/16)..+3 of a few dimensions (the V
//      tile is [4][D][4]); the four weights come from the lanes owning those
//      tokens, the output partial is summed over the four row groups once at
//      the end.
// The addressing is the pages' paged lookup: entry j of the row names the
// physical block, the slot is the offset inside it ("PagedAttention: Virtual
// Memory for LLMs" in "Optimizing KV Cache Memory Management in vLLM with
// PagedAttention and Dynamic Block Allocation").
#include "decode_common.h"

namespace kvp {
namespace {

typedef __attribute__((ext_vector_type(4))) unsigned uint4v;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;


// Sum over the four lanes of a quad (DPP quad permutations).
__device__ __forceinline__ float quad_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));  // [1,0,3,2]
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));  // [2,3,0,1]
  return x;
}

// Element type traits: E elements per 16-byte chunk.
template <typename T>
struct Elt;
template <>
struct Elt<float> {
  static constexpr int E = 4;
};
template <>
struct Elt<uint16_t> {
  static constexpr int E = 8;
};

template <typename T, int D, int GT, int DEPTH>
__global__ __launch_bounds__(kThreads) void decode_valu_kernel(const DecodeParams P) {
  constexpr int NBUF = DEPTH + 1;
  constexpr int E = Elt<T>::E;
  constexpr int KCH = D / E / 4;      // K chunks per lane (a row has D/E chunks over 4 lanes)
  constexpr int VCH = D * 4 / E / 16;  // V chunks per lane (a row group holds D*4 elements over 16 lanes)
  constexpr int VDIM = E / 4;          // dimensions per V chunk
  __shared__ float o_s[kWaves][GT][D + 1];
  __shared__ float m_s[kWaves][GT];
  __shared__ float l_s[kWaves][GT];

  // Grid (head groups, sequences, partitions): consecutive workgroups, which
  // the dispatcher deals round robin to the eight XCDs, differ in head group
  // first, so every XCD gets the same share of every row.
  const int kvh = blockIdx.x / P.qgroups;
  const int qg = blockIdx.x - kvh * P.qgroups;
  const int s = blockIdx.y;
  const int part = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h0 = kvh * P.group + qg * GT;
  const int nh = min(GT, P.group - qg * GT);

  // Lane i holds the id of tile part * part_blocks + i of the row (with
  // 16-token blocks, table entry part * part_blocks + i, loaded together
  // with the sequence length; 32-token blocks need the length first).
  const int ctx = P.seq_lens[s];
  const int32_t* row = P.block_tables + (size_t)s * P.max_blocks;
  const int jl = part * P.part_blocks + lane;
  int my_id = 0;
  if (P.bshift == 0 && lane < P.part_blocks && jl < P.max_blocks) my_id = row[jl];
  const RowSpan rs = row_span(ctx, P.window, P.max_blocks, P.bshift);
  const int t0 = rs.t0;  // 0 with 16-token blocks
  if (P.bshift != 0 && lane < P.part_blocks && jl < rs.nblocks) my_id = row[(t0 + jl) >> P.bshift];
  const int nparts = (rs.nblocks + P.part_blocks - 1) / P.part_blocks;
  T* out = (T*)P.out;
  if (rs.nblocks == 0) {
    if (part == 0)
      for (int i = threadIdx.x; i < nh * D; i += kThreads) out[((size_t)s * P.num_q_heads + h0) * D + i] = T(0);
    return;
  }
  if (part >= nparts) return;
  const int jb = part * P.part_blocks;
  const int nbp = min(P.part_blocks, rs.nblocks - jb);

  const int kt_tok = lane >> 2;  // token whose K row this lane reads
  const int kc = lane & 3;
  const int vq = lane >> 4;      // token quad whose V this lane reads
  const int vj = lane & 15;

  // This lane's slice of the group's queries, matching its K chunks: four
  // 32-bit words per chunk (two bf16 values each, or one fp32 value).
  unsigned qw[GT][KCH][4];
  {
    const T* qbase = (const T*)P.q + ((size_t)s * P.num_q_heads + h0) * D;
#pragma unroll
    for (int g = 0; g < GT; ++g)
#pragma unroll
      for (int i = 0; i < KCH; ++i) {
        uint4v w = {0, 0, 0, 0};
        if (g < nh) w = *(const uint4v*)(qbase + g * D + (kc + 4 * i) * E);
        qw[g][i][0] = w.x;
        qw[g][i][1] = w.y;
        qw[g][i][2] = w.z;
        qw[g][i][3] = w.w;
      }
  }

  const T* pool = (const T*)P.pool_layer;
  const size_t tile = (size_t)(16 << P.bshift) * D;  // one head's K (or V) tile of a block
  const size_t blk_stride = 2 * (size_t)P.num_kv_heads * tile;
  const size_t k_off = (size_t)kvh * tile;
  const size_t v_rel = (size_t)P.num_kv_heads * tile;
  const int so = rs.start_off;
  const int send = rs.start_off + rs.n;

  float m_run[GT], l_run[GT], acc[GT][VCH][VDIM];
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    m_run[g] = -INFINITY;
    l_run[g] = 0.f;
#pragma unroll
    for (int i = 0; i < VCH; ++i)
#pragma unroll
      for (int e = 0; e < VDIM; ++e) acc[g][i][e] = 0.f;
  }

  struct Tiles {
    uint4v k[KCH];
    uint4v v[VCH];
    bool bad;
  };
  const int cnt = nbp > wave ? (nbp - wave + kWaves - 1) / kWaves : 0;
  auto issue = [&](int k, Tiles& t) {
    const int kl = k < cnt ? k : cnt - 1;  // past the end: re-read the last block (a cache hit)
    int id = __builtin_amdgcn_readlane(my_id, wave + kl * kWaves);  // block of tile jb + wave + kl * kWaves
    const int sub = (t0 + jb + wave + kl * kWaves) & ((1 << P.bshift) - 1);
    t.bad = (unsigned)id >= (unsigned)P.num_blocks;
    if (t.bad) id = 0;
    const T* base = pool + (size_t)id * blk_stride + (size_t)sub * 16 * D + k_off;
#pragma unroll
    for (int i = 0; i < KCH; ++i) t.k[i] = *(const uint4v*)(base + kt_tok * D + (kc + 4 * i) * E);
#pragma unroll
    for (int i = 0; i < VCH; ++i) t.v[i] = *(const uint4v*)(base + v_rel + vq * D * 4 + (vj + 16 * i) * E);
  };

  auto compute = [&](int k, const Tiles& t) {
    const bool bad = t.bad;
    const int J = jb + wave + k * kWaves;
    // scores of token kt_tok for every head of the group
    float sc[GT];
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      float a = 0.f;
#pragma unroll
      for (int i = 0; i < KCH; ++i) {
        const unsigned w[4] = {t.k[i].x, t.k[i].y, t.k[i].z, t.k[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (sizeof(T) == 2)
            a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[e]),
                                                __builtin_bit_cast(bf16x2, qw[g][i][e]), a, false);
          else
            a = fmaf(__uint_as_float(w[e]), __uint_as_float(qw[g][i][e]), a);
        }
      }
      sc[g] = quad_sum(a) * P.scale_log2;
    }
    const int u = J * 16 + kt_tok;
    const bool valid = !bad && u >= so && u < send;
    // validity of the four tokens whose V this lane holds
    bool vvalid[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int uv = J * 16 + 4 * vq + r;
      vvalid[r] = !bad && uv >= so && uv < send;
    }
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      const float x = valid ? sc[g] : -INFINITY;
      float mx = x;
      mx = fmaxf(mx, __shfl_xor(mx, 4));
      mx = fmaxf(mx, __shfl_xor(mx, 8));
      mx = rows_max(mx);
      const float m_new = fmaxf(m_run[g], mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run[g] - m_use);
      m_run[g] = m_new;
      const float p = __builtin_amdgcn_exp2f(x - m_use);
      l_run[g] = l_run[g] * alpha + p;
      float pr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) pr[r] = __shfl(p, 16 * vq + 4 * r);
#pragma unroll
      for (int i = 0; i < VCH; ++i) {
        const unsigned w[4] = {t.v[i].x, t.v[i].y, t.v[i].z, t.v[i].w};
#pragma unroll
        for (int e = 0; e < VDIM; ++e) {
          float vals[4];
          if constexpr (sizeof(T) == 2) {
            vals[0] = bf16_lo(w[2 * e]);
            vals[1] = bf16_hi(w[2 * e]);
            vals[2] = bf16_lo(w[2 * e + 1]);
            vals[3] = bf16_hi(w[2 * e + 1]);
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) vals[r] = __uint_as_float(w[r]);
          }
          float a = acc[g][i][e] * alpha;
#pragma unroll
          for (int r = 0; r < 4; ++r) a = fmaf(pr[r], vvalid[r] ? vals[r] : 0.f, a);
          acc[g][i][e] = a;
        }
      }
    }
  };

  // Software pipeline: block k + DEPTH is in flight while block k is computed.
  if (cnt > 0) {
    Tiles buf[NBUF];
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

  // Wave totals: sum weights over tokens (one lane per token: stride-4 lanes),
  // sum outputs over the four token quads.
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    float l = l_run[g];
    l += __shfl_xor(l, 4);
    l += __shfl_xor(l, 8);
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    l_run[g] = l;
#pragma unroll
    for (int i = 0; i < VCH; ++i)
#pragma unroll
      for (int e = 0; e < VDIM; ++e) {
        float a = acc[g][i][e];
        a += __shfl_xor(a, 16);
        a += __shfl_xor(a, 32);
        acc[g][i][e] = a;
      }
  }
  if (lane == 0)
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      m_s[wave][g] = m_run[g];
      l_s[wave][g] = l_run[g];
    }
  if (lane < 16)
#pragma unroll
    for (int g = 0; g < GT; ++g)
#pragma unroll
      for (int i = 0; i < VCH; ++i)
#pragma unroll
        for (int e = 0; e < VDIM; ++e) o_s[wave][g][(vj + 16 * i) * VDIM + e] = acc[g][i][e];
  __syncthreads();
  finish_partition<T, D, GT>(P, o_s, m_s, l_s, s, h0, nh, part, nparts);
}

template <typename T, int D, int GT>
hipError_t launch_g(const DecodeParams& p, const dim3& grid, hipStream_t stream) {
  const dim3 block(kThreads);
  switch (p.depth) {
    case 1: hipLaunchKernelGGL((decode_valu_kernel<T, D, GT, 1>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((decode_valu_kernel<T, D, GT, 2>), grid, block, 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_typed(const DecodeParams& p, hipStream_t stream) {
  const dim3 grid(p.num_kv_heads * p.qgroups, p.num_seqs, p.num_parts);
  switch (p.heads_per_wg) {
    case 1: return launch_g<T, D, 1>(p, grid, stream);
    case 2: return launch_g<T, D, 2>(p, grid, stream);
    case 4: return launch_g<T, D, 4>(p, grid, stream);
    case 8:
      if constexpr (sizeof(T) == 4 && D == 128) return hipErrorInvalidValue;  // would spill; never planned
      else return launch_g<T, D, 8>(p, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_valu(const DecodeParams& p, int dtype, int head_dim, hipStream_t stream) {
  if (dtype == 0) return head_dim == 128 ? launch_typed<float, 128>(p, stream) : launch_typed<float, 64>(p, stream);
  return head_dim == 128 ? launch_typed<uint16_t, 128>(p, stream) : launch_typed<uint16_t, 64>(p, stream);
}

}  // namespace kvp
