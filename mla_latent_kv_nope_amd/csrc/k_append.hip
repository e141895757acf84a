// mla_append_latent: write new latent rows (c_kv || RoPE(k_pe)) into the paged
// cache, optionally as fp8 E4M3FN codes with one fp32 scale per token (the
// per-token work is append_token in append.hpp).
#include "append.hpp"

namespace mla {
namespace {

// PART: the row comes from fp32 partial sums (summed in chunk order, rounded
// to bf16) instead of bf16 c_kv / k_pe inputs.
template <bool FP8, bool PART>
__global__ __launch_bounds__(256) void k_append(AppendArgs a) {
  append_token<FP8, PART>(a, blockIdx.x * 4 + (threadIdx.x >> 6), threadIdx.x & 63);
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
  if (a.n_tokens == 0) return hipSuccess;
  const dim3 grid((a.n_tokens + 3) / 4), block(256);
  if (a.part != nullptr) {
    if (a.fp8) hipLaunchKernelGGL((k_append<true, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_append<false, true>), grid, block, 0, s, a);
  } else {
    if (a.fp8) hipLaunchKernelGGL((k_append<true, false>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_append<false, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace mla
