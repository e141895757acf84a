// mla_project_append, first half: the down-projection of new tokens' hidden
// states into the latent row, y[t] = w_down . h[t] (d_c latent outputs, then
// d_rope RoPE-key outputs).
//
// Method: the cached latent is the down-projection of the hidden state
// ("DeepSeek-V2拆解：MLA与MoE如何把KV缓存压降93.3%", sheratonhq.com, section
// 2.1: down_proj = nn.Linear(d_model, kv_rank), c_kv = down_proj(h), appended
// to the cache), and the RoPE key has its own projection in the decoupled
// branch (same section); d_model = 7168 is the DeepSeek-V3 width
// ("LLM推理优化的新范式：从内存墙到计算墙的跨越", zskr.cn, section 2.1).
//
// A decode step projects a few dozen tokens against an 8 MB weight, so the
// GEMM is weight-read bound and is cut along the reduction: workgroup
// (column tile nt, chunk ks) computes outputs [32 nt, +32) of every token over
// d_model elements [256 ks, +256) and writes fp32 partial sums; the append
// kernel adds the chunks in order and rounds to bf16.  Both operands are
// contiguous along the reduction axis (h rows, w_down rows), so they go from
// global memory straight into 32x32x16 bf16 MFMA registers, all loads of a
// wave in flight at once.
#include "mla_common.hpp"
#include "mla_internal.hpp"

namespace mla {
namespace {

__global__ __launch_bounds__(128) void k_down(ProjectArgs a) {
  constexpr int KS = kDownChunk / 16;             // MFMA steps per chunk
  const int nt = blockIdx.x, ks = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 31, half = lane >> 5;
  const int k0 = ks * kDownChunk + 8 * half;
  // B operand: weight row (output) 32 nt + r, elements k0 + 16 s + [0, 8)
  const uint16_t* wrow = a.w_down + static_cast<int64_t>(nt * 32 + r) * a.d_model + k0;
  bf16x8 bv[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) bv[s] = *reinterpret_cast<const bf16x8*>(wrow + 16 * s);
  // two waves take alternate blocks of 32 tokens
  for (int t0 = 32 * wave; t0 < a.T; t0 += 64) {
    const int t = min(t0 + r, a.T - 1);           // rows past the last token: any valid row
    const uint16_t* hrow = a.h + static_cast<int64_t>(t) * a.d_model + k0;
    bf16x8 av[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) av[s] = *reinterpret_cast<const bf16x8*>(hrow + 16 * s);
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < KS; ++s) acc = mfma32(av[s], bv[s], acc);
    // acc[i] is token t0 + 8(i/4) + 4 half + i%4, output 32 nt + r
    float* dst = a.part + static_cast<int64_t>(ks) * a.T * a.N + nt * 32 + r;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int tok = t0 + 8 * (i >> 2) + 4 * half + (i & 3);
      if (tok < a.T) dst[static_cast<int64_t>(tok) * a.N] = acc[i];
    }
  }
}

}  // namespace

hipError_t launch_down(const ProjectArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (a.N % 32 != 0 || a.d_model % kDownChunk != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_down, dim3(a.N / 32, a.d_model / kDownChunk), dim3(128), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
