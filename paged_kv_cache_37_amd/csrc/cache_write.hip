// cache_write: store new tokens' K and V into their pool slots.
//
// "Optimizing KV Cache Memory Management in vLLM with PagedAttention and
// Dynamic Block Allocation", section The Block Manager and Dynamic
// Allocation Lifecycle: prefill writes the prompt's K/V into its blocks,
// decode writes the new token's K/V into the free slot of the last block.
// A slot is block * B + offset (section PagedAttention: Virtual Memory for
// LLMs: block floor(i/B), offset i mod B), B = 16 << bshift.
//
// One work item = (token, KV head, 16-byte chunk of head_dim).  K: the
// token's chunk is one 16-byte store into its row of the K tile.  V lives
// quad-interleaved ([B/4][D][4]: slot t of dimension d at ((t/4)*D + d)*4 +
// t%4, B = 16 or 32), so one token's values are 4 elements apart.  A token
// whose slot starts a quad, followed by three tokens in the quad's next
// three slots (a prompt or chunk written into its blocks in order), leads
// the quad: it transposes the four tokens' chunks in registers and stores
// every dimension's four slots together, 64 contiguous bytes (32 for FP8);
// the other three skip their V stores.  Every other token (decode's one
// token per sequence, a chunk's first and last few tokens, any other slot
// pattern) stores its own values one by one.  Bits are copied, never
// converted, except into an FP8 pool, where each bf16 value becomes its
// E4M3 code (fp8.h: nearest code of x * (1 / scale), saturating) and a
// chunk is 8 values.
#include "fp8.h"

namespace kvp {
namespace {

typedef __attribute__((ext_vector_type(4))) unsigned uint4v;

// Whether tokens t .. t+3 write the four slots of one quad in order: slots
// s, s+1, s+2, s+3 with s a multiple of 4 inside the pool.
__device__ __forceinline__ bool whole_quad(const int32_t* __restrict__ slots, long t, int num_tokens,
                                           int pool_slots) {
  if (t < 0 || t + 3 >= num_tokens) return false;
  const int s0 = slots[t];
  return s0 >= 0 && (s0 & 3) == 0 && s0 + 3 < pool_slots && slots[t + 1] == s0 + 1 && slots[t + 2] == s0 + 2 &&
         slots[t + 3] == s0 + 3;
}

// Four tokens' 16-byte chunks (x[i] = token i) -> the quad's 64 bytes of
// those dimensions, dimension by dimension, four slots each.
__device__ __forceinline__ void quad_transpose(const uint4v (&x)[4], uint4v (&o)[4], uint16_t) {
  // bf16: word j of a chunk holds dims 2j (low half) and 2j+1 (high half)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const unsigned a = x[0][j], b = x[1][j], c = x[2][j], d = x[3][j];
    o[j] = uint4v{(a & 0xffffu) | (b << 16), (c & 0xffffu) | (d << 16),            // dim 2j: slots 0,1 | 2,3
                  (a >> 16) | (b & 0xffff0000u), (c >> 16) | (d & 0xffff0000u)};  // dim 2j+1
  }
}
__device__ __forceinline__ void quad_transpose(const uint4v (&x)[4], uint4v (&o)[4], uint32_t) {
  // fp32: word j is dim j
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = uint4v{x[0][j], x[1][j], x[2][j], x[3][j]};
}

template <typename W>  // W = element bits: uint16_t (bf16) or uint32_t (fp32)
__global__ __launch_bounds__(256) void cache_write_kernel(W* __restrict__ pool, const W* __restrict__ k_new,
                                                          const W* __restrict__ v_new,
                                                          const int32_t* __restrict__ slots, int num_tokens,
                                                          int num_blocks, int bshift, int num_kv_heads, int D) {
  constexpr int E = 16 / sizeof(W);
  const int chunks = D / E;
  const long items = (long)num_tokens * num_kv_heads * chunks;
  const int B = 16 << bshift;
  const int pool_slots = num_blocks * B;
  const size_t tile = (size_t)B * D;
  for (long it = (long)blockIdx.x * 256 + threadIdx.x; it < items; it += (long)gridDim.x * 256) {
    const int c = (int)(it % chunks);
    const long th = it / chunks;
    const int h = (int)(th % num_kv_heads);
    const long t = th / num_kv_heads;
    const int slot = slots[t];
    if (slot < 0 || slot >= pool_slots) continue;
    const int blk = slot >> (4 + bshift), off = slot & (B - 1);
    W* base = pool + (size_t)blk * 2 * num_kv_heads * tile;
    const size_t src = ((size_t)t * num_kv_heads + h) * D + (size_t)c * E;
    *(uint4v*)(base + h * tile + (size_t)off * D + (size_t)c * E) = *(const uint4v*)(k_new + src);
    W* vq = base + (num_kv_heads + h) * tile + ((size_t)(off >> 2) * D + (size_t)c * E) * 4;
    if ((slot & 3) == 0 && whole_quad(slots, t, num_tokens, pool_slots)) {
      uint4v x[4], o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = *(const uint4v*)(v_new + src + (size_t)i * num_kv_heads * D);
      quad_transpose(x, o, W{});
#pragma unroll
      for (int j = 0; j < 4; ++j) ((uint4v*)vq)[j] = o[j];
    } else if (!whole_quad(slots, t - (slot & 3), num_tokens, pool_slots)) {  // not led by another token
      W ve[E];
      const uint4v vv = *(const uint4v*)(v_new + src);
      __builtin_memcpy(ve, &vv, 16);
#pragma unroll
      for (int e = 0; e < E; ++e) vq[e * 4 + (off & 3)] = ve[e];
    }
  }
}

// FP8 pool: bf16 inputs, 8 values (16 bytes in, 8 codes out) per token and
// chunk; a led quad's codes go out as 32 contiguous bytes.
__global__ __launch_bounds__(256) void cache_write_fp8_kernel(uint8_t* __restrict__ pool,
                                                              const uint16_t* __restrict__ k_new,
                                                              const uint16_t* __restrict__ v_new,
                                                              const int32_t* __restrict__ slots, int num_tokens,
                                                              int num_blocks, int bshift, int num_kv_heads, int D,
                                                              float inv_k, float inv_v) {
  const int chunks = D / 8;
  const long items = (long)num_tokens * num_kv_heads * chunks;
  const int B = 16 << bshift;
  const int pool_slots = num_blocks * B;
  const size_t tile = (size_t)B * D;
  for (long it = (long)blockIdx.x * 256 + threadIdx.x; it < items; it += (long)gridDim.x * 256) {
    const int c = (int)(it % chunks);
    const long th = it / chunks;
    const int h = (int)(th % num_kv_heads);
    const long t = th / num_kv_heads;
    const int slot = slots[t];
    if (slot < 0 || slot >= pool_slots) continue;
    const int blk = slot >> (4 + bshift), off = slot & (B - 1);
    uint8_t* base = pool + (size_t)blk * 2 * num_kv_heads * tile;
    const size_t src = ((size_t)t * num_kv_heads + h) * D + (size_t)c * 8;
    *(fp8_u2*)(base + h * tile + (size_t)off * D + (size_t)c * 8) = fp8_quant8(*(const fp8_u4*)(k_new + src), inv_k);
    uint8_t* vq = base + (num_kv_heads + h) * tile + ((size_t)(off >> 2) * D + (size_t)c * 8) * 4;
    if ((slot & 3) == 0 && whole_quad(slots, t, num_tokens, pool_slots)) {
      fp8_u2 vc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) vc[i] = fp8_quant8(*(const fp8_u4*)(v_new + src + (size_t)i * num_kv_heads * D), inv_v);
      // dimension e's word: the four slots' codes, slot 0 in the low byte
      unsigned w[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        w[e] = 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[e] |= (((e < 4 ? vc[i].x : vc[i].y) >> (8 * (e & 3))) & 0xffu) << (8 * i);
      }
      ((uint4v*)vq)[0] = uint4v{w[0], w[1], w[2], w[3]};
      ((uint4v*)vq)[1] = uint4v{w[4], w[5], w[6], w[7]};
    } else if (!whole_quad(slots, t - (slot & 3), num_tokens, pool_slots)) {  // not led by another token
      const fp8_u2 vc = fp8_quant8(*(const fp8_u4*)(v_new + src), inv_v);
#pragma unroll
      for (int e = 0; e < 8; ++e) vq[e * 4 + (off & 3)] = (uint8_t)(((e < 4 ? vc.x : vc.y) >> (8 * (e & 3))) & 0xffu);
    }
  }
}

}  // namespace

hipError_t launch_cache_write(void* pool_layer, int dtype, int num_blocks, int bshift, int num_kv_heads, int head_dim,
                              const void* k_new, const void* v_new, const int32_t* slots, int num_tokens,
                              float inv_k_scale, float inv_v_scale, hipStream_t stream) {
  const int E = dtype == 0 ? 4 : 8;
  const long items = (long)num_tokens * num_kv_heads * (head_dim / E);
  long blocks = (items + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  if (dtype == 2)
    hipLaunchKernelGGL(cache_write_fp8_kernel, dim3(blocks), dim3(256), 0, stream, (uint8_t*)pool_layer,
                       (const uint16_t*)k_new, (const uint16_t*)v_new, slots, num_tokens, num_blocks, bshift,
                       num_kv_heads, head_dim, inv_k_scale, inv_v_scale);
  else if (dtype == 1)
    hipLaunchKernelGGL(cache_write_kernel<uint16_t>, dim3(blocks), dim3(256), 0, stream, (uint16_t*)pool_layer,
                       (const uint16_t*)k_new, (const uint16_t*)v_new, slots, num_tokens, num_blocks, bshift,
                       num_kv_heads, head_dim);
  else
    hipLaunchKernelGGL(cache_write_kernel<uint32_t>, dim3(blocks), dim3(256), 0, stream, (uint32_t*)pool_layer,
                       (const uint32_t*)k_new, (const uint32_t*)v_new, slots, num_tokens, num_blocks, bshift,
                       num_kv_heads, head_dim);
  return hipGetLastError();
}

}  // namespace kvp
