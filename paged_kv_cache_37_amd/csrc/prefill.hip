// Multi-token (prefill / chunked-prefill) paged attention: the kernel and
// its launch (the workgroup body is prefill_body.inc; the cascade decode
// kernel runs the same body for its shared-prefix pass).
#include "prefill_common.h"

namespace kvp {
namespace {

template <int D, bool FP8, int BS>
__global__ __launch_bounds__(kThreads, 2) void prefill_kernel(const PrefillParams PF) {
  using namespace pf;
  constexpr bool PREFIX = false;
  __shared__ PfLds<D> lds;
  PfLds<D>& L = lds;
  const int wg = blockIdx.x;
#include "prefill_body.inc"
}

template <int D, bool FP8>
hipError_t launch_pf(const PrefillParams& p, unsigned grid, hipStream_t stream) {
  if (p.bshift)
    hipLaunchKernelGGL((prefill_kernel<D, FP8, 1>), dim3(grid), dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((prefill_kernel<D, FP8, 0>), dim3(grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, int head_dim, bool fp8, hipStream_t stream) {
  const long long grid = (long long)p.num_seqs * p.num_kv_heads * p.qtiles;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  const unsigned g = (unsigned)grid;
  if (head_dim == 128) return fp8 ? launch_pf<128, true>(p, g, stream) : launch_pf<128, false>(p, g, stream);
  if (head_dim == 64) return fp8 ? launch_pf<64, true>(p, g, stream) : launch_pf<64, false>(p, g, stream);
  return hipErrorInvalidValue;
}

}  // namespace kvp
