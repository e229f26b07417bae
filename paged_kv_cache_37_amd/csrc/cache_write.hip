// cache_write: store new tokens' K and V into their pool slots.
//
// "Optimizing KV Cache Memory Management in vLLM with PagedAttention and
// Dynamic Block Allocation", section The Block Manager and Dynamic
// Allocation Lifecycle: prefill writes the prompt's K/V into its blocks,
// decode writes the new token's K/V into the free slot of the last block.
// A slot is block * B + offset (section PagedAttention: Virtual Memory for
// LLMs: block floor(i/B), offset i mod B), B = 16 << bshift.
//
// One work item = (token, KV head, 16-byte chunk of head_dim): the K chunk
// is one 16-byte store into the row of the K tile; the V chunk's elements go
// to the quad-interleaved V tile ([4][D][4]: slot t of dimension d at
// ((t/4)*D + d)*4 + t%4, t < block size: 16 or 32).  Bits are copied, never converted, except into an
// FP8 pool, where each bf16 value becomes its E4M3 code (fp8.h: nearest code
// of x * (1 / scale), saturating) and a chunk is 8 values.
#include "fp8.h"

namespace kvp {
namespace {

typedef __attribute__((ext_vector_type(4))) unsigned uint4v;

template <typename W>  // W = element bits: uint16_t (bf16) or uint32_t (fp32)
__global__ __launch_bounds__(256) void cache_write_kernel(W* __restrict__ pool, const W* __restrict__ k_new,
                                                          const W* __restrict__ v_new,
                                                          const int32_t* __restrict__ slots, int num_tokens,
                                                          int num_blocks, int bshift, int num_kv_heads, int D) {
  constexpr int E = 16 / sizeof(W);
  const int chunks = D / E;
  const long items = (long)num_tokens * num_kv_heads * chunks;
  const int B = 16 << bshift;
  const size_t tile = (size_t)B * D;
  for (long it = (long)blockIdx.x * 256 + threadIdx.x; it < items; it += (long)gridDim.x * 256) {
    const int c = (int)(it % chunks);
    const long th = it / chunks;
    const int h = (int)(th % num_kv_heads);
    const int t = (int)(th / num_kv_heads);
    const int slot = slots[t];
    if (slot < 0 || slot >= num_blocks * B) continue;
    const int blk = slot >> (4 + bshift), off = slot & (B - 1);
    W* base = pool + (size_t)blk * 2 * num_kv_heads * tile;
    const size_t src = ((size_t)t * num_kv_heads + h) * D + (size_t)c * E;
    *(uint4v*)(base + h * tile + (size_t)off * D + (size_t)c * E) = *(const uint4v*)(k_new + src);
    const uint4v vv = *(const uint4v*)(v_new + src);
    W ve[E];
    __builtin_memcpy(ve, &vv, 16);
    W* vt = base + (num_kv_heads + h) * tile + ((size_t)(off >> 2) * D + (size_t)c * E) * 4 + (off & 3);
#pragma unroll
    for (int e = 0; e < E; ++e) vt[e * 4] = ve[e];
  }
}

// FP8 pool: bf16 inputs, 8 values (16 bytes in, 8 codes out) per work item.
__global__ __launch_bounds__(256) void cache_write_fp8_kernel(uint8_t* __restrict__ pool,
                                                              const uint16_t* __restrict__ k_new,
                                                              const uint16_t* __restrict__ v_new,
                                                              const int32_t* __restrict__ slots, int num_tokens,
                                                              int num_blocks, int bshift, int num_kv_heads, int D,
                                                              float inv_k, float inv_v) {
  const int chunks = D / 8;
  const long items = (long)num_tokens * num_kv_heads * chunks;
  const int B = 16 << bshift;
  const size_t tile = (size_t)B * D;
  for (long it = (long)blockIdx.x * 256 + threadIdx.x; it < items; it += (long)gridDim.x * 256) {
    const int c = (int)(it % chunks);
    const long th = it / chunks;
    const int h = (int)(th % num_kv_heads);
    const int t = (int)(th / num_kv_heads);
    const int slot = slots[t];
    if (slot < 0 || slot >= num_blocks * B) continue;
    const int blk = slot >> (4 + bshift), off = slot & (B - 1);
    uint8_t* base = pool + (size_t)blk * 2 * num_kv_heads * tile;
    const size_t src = ((size_t)t * num_kv_heads + h) * D + (size_t)c * 8;
    *(fp8_u2*)(base + h * tile + (size_t)off * D + (size_t)c * 8) = fp8_quant8(*(const fp8_u4*)(k_new + src), inv_k);
    const fp8_u2 vc = fp8_quant8(*(const fp8_u4*)(v_new + src), inv_v);
    uint8_t* vt = base + (num_kv_heads + h) * tile + ((size_t)(off >> 2) * D + (size_t)c * 8) * 4 + (off & 3);
#pragma unroll
    for (int e = 0; e < 8; ++e) vt[e * 4] = (uint8_t)(((e < 4 ? vc.x : vc.y) >> (8 * (e & 3))) & 0xffu);
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
