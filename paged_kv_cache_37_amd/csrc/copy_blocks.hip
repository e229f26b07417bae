// Device block copy for copy-on-write ([Optimizing] "Copy-on-Write (CoW) for
// Parallel Sampling and Prefix Caching" in "Optimizing KV Cache Memory
// Management in vLLM with PagedAttention and Dynamic Block Allocation": a
// sequence about to write into a block it shares gets a new physical block
// holding a copy of the shared one, and its table entry is repointed; the
// host bookkeeping does the allocation, reference counts and table update,
// this kernel the copy).
//
// One workgroup per (pair, layer): the block's K and V tiles of every KV head
// are one contiguous run of block_bytes, copied with 16-byte loads and
// stores.  A pair naming a block outside the pool, or src == dst, is skipped.
#include "internal.h"

namespace kvp {
namespace {

typedef __attribute__((ext_vector_type(4))) unsigned uint4_c;

__global__ __launch_bounds__(256) void copy_blocks_kernel(char* base, int num_blocks, size_t layer_bytes,
                                                          size_t block_bytes, const int32_t* src,
                                                          const int32_t* dst) {
  const int i = blockIdx.x;
  const int s = src[i], d = dst[i];
  if ((unsigned)s >= (unsigned)num_blocks || (unsigned)d >= (unsigned)num_blocks || s == d) return;
  const char* from = base + blockIdx.y * layer_bytes + (size_t)s * block_bytes;
  char* to = base + blockIdx.y * layer_bytes + (size_t)d * block_bytes;
  const size_t n16 = block_bytes / 16;
  for (size_t k = threadIdx.x; k < n16; k += 256) ((uint4_c*)to)[k] = ((const uint4_c*)from)[k];
}

}  // namespace

hipError_t launch_copy_blocks(void* pool_base, int num_layers, int num_blocks, size_t block_bytes, const int32_t* src,
                              const int32_t* dst, int num_pairs, hipStream_t stream) {
  if (num_layers > 65535) return hipErrorInvalidValue;
  const dim3 grid(num_pairs, num_layers);
  hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(256), 0, stream, (char*)pool_base, num_blocks,
                     (size_t)num_blocks * block_bytes, block_bytes, src, dst);
  return hipGetLastError();
}

}  // namespace kvp
