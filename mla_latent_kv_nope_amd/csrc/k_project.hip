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
// (column tile nt, group ks, token block tb) takes outputs [32 nt, +32) of
// tokens [32 tb, +32) over the kDownGroup chunks of 256 d_model elements
// starting at chunk kDownGroup ks, one chunk per wave; the waves' sums are
// added in chunk order through LDS and written as one fp32 partial, and the
// append kernel adds the groups' partials in order and rounds to bf16.  Both operands are
// contiguous along the reduction axis (h rows, w_down rows), so they go from
// global memory straight into 32x32x16 bf16 MFMA registers, all loads of a
// wave in flight at once.
#include "mla_common.hpp"
#include "mla_internal.hpp"

namespace mla {
namespace {

__global__ __launch_bounds__(64 * kDownGroup) void k_down(ProjectArgs a) {
  constexpr int KS = kDownChunk / 16;             // MFMA steps per chunk
  __shared__ float red[kDownGroup - 1][32][33];   // waves 1.. hand their sums to wave 0
  // 1-D grid, XCD-aware: workgroups are dealt round-robin over the 8 XCDs,
  // and the token blocks of one (column tile, group) pair take consecutive
  // slots of one XCD, so its weight slice leaves HBM once
  const int ntb = (a.T + 31) / 32, ng = down_groups(a.d_model);
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int pair = 8 * (slot / ntb) + xcd;
  if (pair >= (a.N / 32) * ng) return;          // (the pair count is padded to a multiple of 8)
  const int nt = pair % (a.N / 32), ks = pair / (a.N / 32), t0 = 32 * (slot % ntb);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 31, half = lane >> 5;
  const int chunk = ks * kDownGroup + wave;
  const bool has = chunk < a.d_model / kDownChunk;   // the last group may be short
  const int k0 = chunk * kDownChunk + 8 * half;
  // B operand: weight row (output) 32 nt + r, elements k0 + 16 s + [0, 8)
  const uint16_t* wrow = a.w_down + static_cast<int64_t>(nt * 32 + r) * a.d_model + k0;
  bf16x8 bv[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) bv[s] = has ? *reinterpret_cast<const bf16x8*>(wrow + 16 * s) : bf16x8{};
  const int t = min(t0 + r, a.T - 1);           // rows past the last token: any valid row
  const uint16_t* hrow = a.h + static_cast<int64_t>(t) * a.d_model + k0;
  bf16x8 av[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) av[s] = has ? *reinterpret_cast<const bf16x8*>(hrow + 16 * s) : bf16x8{};
  f32x16 acc = {};
#pragma unroll
  for (int s = 0; s < KS; ++s) acc = mfma32(av[s], bv[s], acc);
  // acc[i] is token t0 + 8(i/4) + 4 half + i%4, output 32 nt + r
  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < 16; ++i) red[wave - 1][8 * (i >> 2) + 4 * half + (i & 3)][r] = acc[i];
  }
  __syncthreads();
  if (wave == 0) {
    // the group's chunks in order: ((c0 + c1) + c2) + c3
#pragma unroll
    for (int w = 0; w < kDownGroup - 1; ++w)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] += red[w][8 * (i >> 2) + 4 * half + (i & 3)][r];
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
  const int64_t pairs = (static_cast<int64_t>(a.N / 32) * down_groups(a.d_model) + 7) / 8 * 8;
  const int64_t grid = pairs * ((a.T + 31) / 32);
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_down, dim3(static_cast<unsigned>(grid)), dim3(64 * kDownGroup), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
