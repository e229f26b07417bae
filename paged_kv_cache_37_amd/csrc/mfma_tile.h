// One wave's paged-attention step over a 16-token block on the CDNA4 matrix
// cores (bf16 pools), shared by the partitioned and the streaming kernels.
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
// The accumulator of PV MFMA n, register r, lane l is therefore
//   O[head 4q + r][dim 32(n/2) + 2(l%16) + n%2].
// An FP8 pool has the same layout with one-byte E4M3 codes: a lane widens
// 8 codes per operand to the 8 bf16 values above (exact), so the MFMAs are
// the same; the K scale is folded into the softmax scale and the V scale
// into the final normalisation by the callers.  FP8 K is loaded 16 codes
// per lane (dims 64 (kk / 2) + 16 q .. +15: the first 8 for QK MFMA kk
// even, the rest for kk odd), so that every load takes 64-byte runs of
// the K rows as with bf16; the queries follow the same dim order (qk_dim).
// FP8 V is loaded 16 codes per lane too: dims 4 (l%16) .. +3 and 64 + 4
// (l%16) .. +3 of tokens 4q..4q+3, so PV MFMA n = 4h + e takes dim
// 64 h + 4 (l%16) + e as column l%16 (acc_dim gives the mapping of each
// pool type).
//
// Tile loads are ordinary cached loads or non-temporal ones (mfma_issue's
// NT): a batch whose blocks each belong to one row reads every line once,
// and non-temporal loads then stream them past the caches.
#pragma once

#include <type_traits>

#include "decode_common.h"
#include "fp8.h"

namespace kvp {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_v;
typedef __attribute__((ext_vector_type(4))) short short4_v;
typedef __attribute__((ext_vector_type(8))) short short8_v;
typedef __attribute__((ext_vector_type(4))) float float4_v;
typedef __attribute__((ext_vector_type(4))) unsigned uint4_v;
typedef __attribute__((ext_vector_type(2))) unsigned uint2_v;

// A block's K and V operands for one wave (as loaded: bf16 values, or FP8 codes).
template <int D, bool FP8 = false>
struct MfmaTiles {
  using Op = std::conditional_t<FP8, uint2_v, uint4_v>;
  static constexpr int NV = FP8 ? D / 64 : D / 32;
  Op k[D / 32];      // token l%16, dims 32kk + 8q .. +7
  uint4_v v[NV];     // bf16: tokens 4q..4q+3 of dims 32m + 2(l%16), +1;
                     // FP8: the same tokens of dims 64h + 4(l%16) .. +3
  bool bad;          // block id outside the pool: contributes nothing
};

// Output dim held by PV accumulator n of lane column c (= l%16).
template <bool FP8>
__device__ __forceinline__ constexpr int acc_dim(int n, int c) {
  return FP8 ? 64 * (n >> 2) + 4 * c + (n & 3) : 32 * (n >> 1) + 2 * c + (n & 1);
}

// Per-wave addressing of one KV head's tiles inside a block.  A block of
// 16 << BS tokens holds, per head, a K tile [B][D] and a V tile
// [B/4][D][4]; its 16-token tile u is rows 16u.. of the K tile and quads
// 4u.. of the V tile, both at element offset 16 u D.
struct MfmaLanes {
  size_t blk_stride;  // elements per physical block (all heads, K and V)
  size_t k_off;       // this head's K tile inside a block
  size_t v_rel;       // V tile = K tile + v_rel
  int k_lane;         // this lane's K element offset (+ 32 kk; FP8: + 64 per 16-code load)
  int v_lane;         // this lane's V element offset (+ 128 m; FP8: + 256 h)
};

// First of the 8 dims that lanes of row group q supply to QK MFMA kk (the
// K operand and the query operand alike).
template <bool FP8>
__device__ __forceinline__ constexpr int qk_dim(int kk, int q) {
  return FP8 ? 64 * (kk >> 1) + 16 * q + 8 * (kk & 1) : 32 * kk + 8 * q;
}

template <int D, int BS, bool FP8>  // BS = log2(block size / 16)
__device__ __forceinline__ MfmaLanes mfma_lanes(int num_kv_heads, int kvh, int lane) {
  const size_t tile = (size_t)(16 << BS) * D;
  MfmaLanes a;
  a.blk_stride = 2 * (size_t)num_kv_heads * tile;
  a.k_off = (size_t)kvh * tile;
  a.v_rel = (size_t)num_kv_heads * tile;
  a.k_lane = (lane & 15) * D + qk_dim<FP8>(0, lane >> 4);
  a.v_lane = ((lane >> 4) * D + (FP8 ? 4 : 2) * (lane & 15)) * 4;
  return a;
}

// A tile load, cached or non-temporal (a compile-time choice: the two
// forms of one load would otherwise be merged into the cached one).
template <bool NT, typename T>
__device__ __forceinline__ T tile_load(const T* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

// Issue the loads of tile `sub` (< 1 << BS) of physical block `id` (the
// block id is checked against the pool size here).
template <int BS, bool NT, int D, bool FP8>
__device__ __forceinline__ void mfma_issue(MfmaTiles<D, FP8>& t, const void* __restrict__ pool, const MfmaLanes& a,
                                           int id, int sub, int num_blocks) {
  using E = std::conditional_t<FP8, uint8_t, uint16_t>;
  using Op = typename MfmaTiles<D, FP8>::Op;
  t.bad = (unsigned)id >= (unsigned)num_blocks;
  if (t.bad) id = 0;
  const E* kt = (const E*)pool + (size_t)id * a.blk_stride + (size_t)(BS ? sub : 0) * 16 * D + a.k_off;
  if constexpr (FP8) {
#pragma unroll
    for (int k2 = 0; k2 < D / 64; ++k2) {
      const uint4_v c = tile_load<NT>((const uint4_v*)(kt + a.k_lane + 64 * k2));
      t.k[2 * k2] = uint2_v{c.x, c.y};
      t.k[2 * k2 + 1] = uint2_v{c.z, c.w};
    }
  } else {
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) t.k[kk] = tile_load<NT>((const Op*)(kt + a.k_lane + 32 * kk));
  }
  if constexpr (FP8) {
#pragma unroll
    for (int h = 0; h < D / 64; ++h) t.v[h] = tile_load<NT>((const uint4_v*)(kt + a.v_rel + a.v_lane + 256 * h));
  } else {
#pragma unroll
    for (int m = 0; m < D / 32; ++m) t.v[m] = tile_load<NT>((const uint4_v*)(kt + a.v_rel + a.v_lane + 128 * m));
  }
}

// As many loads as mfma_issue issues, each one dword of the 128 bytes at
// `hot` (16-byte aligned, a line the wave has just read, so a cache hit):
// ring slots past the end of a wave's tiles keep the loop's load count
// without reading a tile again.  Dword loads cannot be merged with the
// tile loads they stand beside (which would lose the non-temporal hint).
// Their values are never used.
template <int D, bool FP8>
__device__ __forceinline__ void mfma_issue_hot(MfmaTiles<D, FP8>& t, const void* __restrict__ hot) {
  const unsigned* h = (const unsigned*)hot;
  if constexpr (FP8) {
#pragma unroll
    for (int k2 = 0; k2 < D / 64; ++k2) {
      t.k[2 * k2] = uint2_v{h[k2], 0u};
      t.k[2 * k2 + 1] = uint2_v{0u, 0u};
    }
#pragma unroll
    for (int m = 0; m < D / 64; ++m) t.v[m] = uint4_v{h[16 + m], 0u, 0u, 0u};
  } else {
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) t.k[kk] = uint4_v{h[kk], 0u, 0u, 0u};
#pragma unroll
    for (int m = 0; m < D / 32; ++m) t.v[m] = uint4_v{h[16 + m], 0u, 0u, 0u};
  }
  t.bad = true;
}

// Running softmax state of one wave for up to 16 query heads of a group.
template <int D>
struct MfmaRow {
  uint4_v qop[D / 32];  // Q as the B operand: column = head l%16
  float m_run;          // running max of head l%16 (base 2), uniform over row groups
  float l_run;          // this lane's share of head l%16's weight sum
  float4_v acc[D / 16];

  // Row 4 (l/16) + r4 of the accumulators (one query head) as D fp32
  // values at dst (a partial result), or times inv as D bf16 values at
  // dst (the output); each lane stores the dims its columns hold.
  template <bool FP8>
  __device__ __forceinline__ void store_partial(float* dst, int r4, int lane) const {
    const int c = lane & 15;
    if constexpr (FP8) {
#pragma unroll
      for (int h = 0; h < D / 64; ++h)
        *(float4_v*)(dst + acc_dim<true>(4 * h, c)) =
            float4_v{acc[4 * h][r4], acc[4 * h + 1][r4], acc[4 * h + 2][r4], acc[4 * h + 3][r4]};
    } else {
#pragma unroll
      for (int m = 0; m < D / 32; ++m)
        *(float2*)(dst + acc_dim<false>(2 * m, c)) = make_float2(acc[2 * m][r4], acc[2 * m + 1][r4]);
    }
  }
  template <bool FP8>
  __device__ __forceinline__ void store_out(uint16_t* dst, int r4, float inv, int lane) const {
    const int c = lane & 15;
    if constexpr (FP8) {
#pragma unroll
      for (int h = 0; h < D / 64; ++h)
        *(uint2_v*)(dst + acc_dim<true>(4 * h, c)) =
            uint2_v{pack_bf16x2(acc[4 * h][r4] * inv, acc[4 * h + 1][r4] * inv),
                    pack_bf16x2(acc[4 * h + 2][r4] * inv, acc[4 * h + 3][r4] * inv)};
    } else {
#pragma unroll
      for (int m = 0; m < D / 32; ++m)
        *(unsigned*)(dst + acc_dim<false>(2 * m, c)) = pack_bf16x2(acc[2 * m][r4] * inv, acc[2 * m + 1][r4] * inv);
    }
  }

  __device__ __forceinline__ void reset() {
    m_run = -INFINITY;
    l_run = 0.f;
#pragma unroll
    for (int n = 0; n < D / 16; ++n) acc[n] = float4_v{0.f, 0.f, 0.f, 0.f};
  }

  // Queries of heads h0 .. h0+nh-1 of sequence s (zero for the padding
  // columns), in the dim order of the K operand of an FP8 or bf16 pool.
  template <bool FP8>
  __device__ __forceinline__ void load_q(const uint16_t* __restrict__ q, size_t row_base, int nh, int lane) {
    const int g = lane & 15;
    const uint16_t* qp = q + (row_base + g) * D;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
      qop[kk] = g < nh ? *(const uint4_v*)(qp + qk_dim<FP8>(kk, lane >> 4)) : uint4_v{0, 0, 0, 0};
  }

  // One tile: tile J of a row span whose attended slots are [so, send)
  // (slots counted from its first tile) and which has `nblocks` tiles.
  template <bool FP8>
  __device__ __forceinline__ void step(MfmaTiles<D, FP8>& t, int J, int so, int send, int nblocks, float scale_log2,
                                       int lane) {
    const int q4 = lane >> 4;
    // K operands as bf16; V operands (bf16: per 32-dim group m, two dims x
    // four tokens; FP8: per output MFMA n, one dim x four tokens) as bf16
    uint4_v kop[D / 32];
    constexpr int NVO = FP8 ? D / 16 : D / 32;
    std::conditional_t<FP8, uint2_v, uint4_v> vop[NVO];
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      if constexpr (FP8) kop[kk] = fp8_widen8(t.k[kk]);
      else kop[kk] = t.k[kk];
    }
#pragma unroll
    for (int i = 0; i < NVO; ++i) {
      if constexpr (FP8) vop[i] = fp8_widen4(t.v[i >> 2][i & 3]);
      else vop[i] = t.v[i];
    }
    float4_v sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_v, kop[kk]),
                                                     __builtin_bit_cast(bf16x8_v, qop[kk]), sacc, 0, 0, 0);
    float sv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) sv[r] = sacc[r] * scale_log2;
    const bool edge = t.bad || (J == 0 && so > 0) || (J == nblocks - 1 && (send & 15) != 0);
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
      for (int i = 0; i < NVO; ++i) {
        vop[i].x &= vm[0];
        vop[i].y &= vm[1];
        if constexpr (!FP8) {
          vop[i].z &= vm[0];
          vop[i].w &= vm[1];
        }
      }
    }
    // The running max is raised only when a score exceeds it by more than
    // 2^kRescaleSlack; then the accumulators are rescaled.
    const float lmax = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    if (__any(lmax > m_run + kRescaleSlack)) {
      const float m_new = fmaxf(m_run, rows_max(lmax));
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float ar = __shfl(alpha, 4 * q4 + r);  // rows of O here are heads 4*q4 + r
#pragma unroll
        for (int n = 0; n < D / 16; ++n) acc[n][r] *= ar;
      }
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(sv[r] - m_use);
    l_run += (p[0] + p[1]) + (p[2] + p[3]);
    // P = P_hi + P_lo, both bf16: the two PV products together carry the
    // weights to ~2^-17 relative instead of bf16's 2^-9.
    const unsigned h01 = pack_bf16x2(p[0], p[1]), h23 = pack_bf16x2(p[2], p[3]);
    const unsigned l01 = pack_bf16x2(p[0] - bf16_lo(h01), p[1] - bf16_hi(h01));
    const unsigned l23 = pack_bf16x2(p[2] - bf16_lo(h23), p[3] - bf16_hi(h23));
    const short4_v pa_hi = __builtin_bit_cast(short4_v, uint2_v{h01, h23});
    const short4_v pa_lo = __builtin_bit_cast(short4_v, uint2_v{l01, l23});
    if constexpr (FP8) {
#pragma unroll
      for (int n = 0; n < D / 16; ++n) {
        const short4_v vn = __builtin_bit_cast(short4_v, vop[n]);
        acc[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa_hi, vn, acc[n], 0, 0, 0);
        acc[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa_lo, vn, acc[n], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int m = 0; m < D / 32; ++m) {
        const short8_v vv = __builtin_bit_cast(short8_v, vop[m]);
        const short4_v v0 = __builtin_shufflevector(vv, vv, 0, 1, 2, 3);
        const short4_v v1 = __builtin_shufflevector(vv, vv, 4, 5, 6, 7);
        acc[2 * m] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa_hi, v0, acc[2 * m], 0, 0, 0);
        acc[2 * m + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa_hi, v1, acc[2 * m + 1], 0, 0, 0);
        acc[2 * m] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa_lo, v0, acc[2 * m], 0, 0, 0);
        acc[2 * m + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa_lo, v1, acc[2 * m + 1], 0, 0, 0);
      }
    }
  }
};

}  // namespace kvp
