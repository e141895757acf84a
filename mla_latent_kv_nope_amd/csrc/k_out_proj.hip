// mla_out_proj: out[b][h] = W_UV[h]^T . o_lat[b][h].
//
// Method: W_UV is absorbed into the output side ("DeepSeek-V2拆解：MLA与MoE如何把
// KV缓存压降93.3%", sheratonhq.com, section 2.1), so the attention result stays
// in the d_c-wide latent space until this per-head projection.
//
// A per-head batched GEMM [B x d_c] x [d_c x d_v] on 32x32x16 bf16 MFMA.  The
// o_lat operand is contiguous along the reduction axis and is loaded straight
// into registers.  W_UV[h] is stored [d_c][d_v] (contiguous along the output
// axis), so the whole head's weight is staged in LDS and read back with the
// gfx950 transpose read, which hands each lane four consecutive reduction
// elements of its output column.  Workgroup = one head, 4 waves x 32 output
// columns; the weight is read from HBM once.
#include "mla_common.hpp"
#include "mla_internal.hpp"

namespace mla {
namespace {

template <int DC, int DV>
__global__ __launch_bounds__(256) void k_out_proj(OutProjArgs a) {
  constexpr int DVP = DV < 32 ? 32 : DV;        // columns padded to the MFMA width
  constexpr int ROW = DVP + 8;                  // LDS row stride (elements), padded against bank conflicts
  constexpr int NWV = DVP / 32;
  constexpr int KC = DC / 16;
  static_assert(DVP % 32 == 0 && DC % 16 == 0, "tile shape");
  __shared__ __attribute__((aligned(16))) uint16_t w[DC * ROW];

  const int h = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int B = a.B, H = a.H;

  // stage W_UV[h] (zero-padded columns) with 16-byte loads
  const uint16_t* wsrc = a.w_uv + static_cast<int64_t>(h) * DC * DV;
  constexpr int CPR = DVP / 8;
  for (int i = threadIdx.x; i < DC * CPR; i += blockDim.x) {
    const int r = i / CPR, c8 = (i - r * CPR) * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (c8 < DV) v = *reinterpret_cast<const uint4*>(wsrc + r * DV + c8);
    *reinterpret_cast<uint4*>(&w[r * ROW + c8]) = v;
  }
  __syncthreads();
  if (wave >= NWV) return;

  // transpose-read addressing: source lane 4r+q of its 16-lane group reads
  // reduction row (8*g + r [+4]) at columns [16*(G%2) + 4q, +4) of this wave's 32
  const int G = lane >> 4, j = lane & 15, r = j >> 2, q = j & 3, g = lane >> 5;
  const int col0 = wave * 32 + 16 * (G & 1) + 4 * q;
  const int half = lane >> 5;

  for (int b0 = 0; b0 < B; b0 += 32) {
    const int br = b0 + (lane & 31);
    const bool ok = br < B;
    const uint16_t* orow = a.o_lat + (static_cast<int64_t>(ok ? br : 0) * H + h) * DC + 8 * half;
    f32x16 acc = {};
    const bf16x8 z = {};
#pragma unroll 8
    for (int k = 0; k < KC; ++k) {
      const bf16x8 av = *reinterpret_cast<const bf16x8*>(orow + 16 * k);
      const int row = 16 * k + 8 * g + r;
      const bf16x4 lo = lds_read_tr16(&w[row * ROW + col0]);
      const bf16x4 hi = lds_read_tr16(&w[(row + 4) * ROW + col0]);
      const bf16x8 bv = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      acc = mfma32(ok ? av : z, bv, acc);
    }
    const int c = wave * 32 + (lane & 31);
    if (c < DV) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int b = b0 + 8 * (i >> 2) + 4 * half + (i & 3);
        if (b < B) a.out[(static_cast<int64_t>(b) * H + h) * DV + c] = f32_to_bf16_bits(acc[i]);
      }
    }
  }
}

}  // namespace

bool out_proj_supported(int d_c, int d_v) {
  return (d_c == 512 && d_v == 128) || (d_c == 32 && d_v == 16);
}

hipError_t launch_out_proj(const OutProjArgs& a, hipStream_t s) {
  if (a.d_c == 512 && a.d_v == 128) {
    hipLaunchKernelGGL((k_out_proj<512, 128>), dim3(a.H), dim3(256), 0, s, a);
  } else if (a.d_c == 32 && a.d_v == 16) {
    hipLaunchKernelGGL((k_out_proj<32, 16>), dim3(a.H), dim3(256), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mla
