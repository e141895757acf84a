// mla_out_proj: out[b][h] = W_UV[h]^T . o_lat[b][h].
//
// Method: W_UV is absorbed into the output side ("DeepSeek-V2拆解：MLA与MoE如何把
// KV缓存压降93.3%", sheratonhq.com, section 2.1), so the attention result stays
// in the d_c-wide latent space until this per-head projection.
//
// A per-head batched GEMM [B x d_c] x [d_c x d_v] on 32x32x16 bf16 MFMA.  One
// wave computes a 32 x 32 output tile (32 batch rows x 32 columns of one head).
// The o_lat operand is contiguous along the reduction axis and goes straight
// into MFMA registers.  W_UV[h] is stored [d_c][d_v] (contiguous along the
// output axis), so the wave's [d_c x 32] slice is copied to LDS and read back
// with the gfx950 transpose read, which hands each lane four consecutive
// reduction elements of its output column.  Every global load of a wave is in
// flight at once: the kernel is a single memory round trip per wave.
#include "mla_common.hpp"
#include "mla_internal.hpp"

namespace mla {
namespace {

template <int DC, int DV>
__global__ __launch_bounds__(64) void k_out_proj(OutProjArgs a) {
  constexpr int NCOL = 32;                      // output columns per wave (MFMA N)
  constexpr int KC = DC / 16;                   // reduction chunks
  static_assert(DC % 16 == 0 && (DC * NCOL) % 512 == 0, "tile shape");
  // [DC][32] bf16 slice, row-major; 16 consecutive lanes of a transpose read
  // touch 4 rows x 32 bytes, which fall in distinct banks
  __shared__ __attribute__((aligned(1024))) uint16_t w[DC * NCOL];

  const int h = blockIdx.x;
  const int v0 = blockIdx.y * NCOL;
  const int b0 = blockIdx.z * 32;
  const int lane = threadIdx.x;
  const int B = a.B, H = a.H;

  // stage W_UV[h][:, v0:v0+32].  With whole 32-column slices, 16-byte
  // global->LDS copies: lane l of copy k moves elements [8(l%4), +8) of row
  // 16k + l/4, which is exactly LDS byte 1024k + 16l of the row-major slice.
  const uint16_t* wsrc = a.w_uv + static_cast<int64_t>(h) * DC * DV;
  if constexpr (DV % NCOL == 0) {
#pragma unroll
    for (int k = 0; k < DC * NCOL / 512; ++k) {
      const int i = k * 64 + lane;
      const uint16_t* src = wsrc + (i >> 2) * DV + v0 + (i & 3) * 8;
      __builtin_amdgcn_global_load_lds(
          reinterpret_cast<const void*>(src),
          reinterpret_cast<lds_void_t*>(reinterpret_cast<uintptr_t>(w) + 1024 * k), 16, 0, 0);
    }
  } else {
    for (int i = lane; i < DC * (NCOL / 8); i += 64) {
      const int r = i >> 2, c8 = (i & 3) * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (v0 + c8 < DV) v = *reinterpret_cast<const uint4*>(wsrc + r * DV + v0 + c8);
      *reinterpret_cast<uint4*>(&w[r * NCOL + c8]) = v;
    }
  }

  // o_lat rows b0 + lane%32, all loads in flight together with the copies
  const int half = lane >> 5;
  const int br = b0 + (lane & 31);
  const bool ok = br < B;
  const uint16_t* orow = a.o_lat + (static_cast<int64_t>(ok ? br : 0) * H + h) * DC + 8 * half;
  bf16x8 av[KC];
  const bf16x8 z = {};
#pragma unroll
  for (int k = 0; k < KC; ++k) {
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(orow + 16 * k);
    av[k] = ok ? v : z;
  }
  wait_vmcnt<0>();
  __syncthreads();

  // transpose-read addressing: source lane 4r+q of its 16-lane group reads
  // reduction row (8*g + r [+4]) at columns [16*(G%2) + 4q, +4) of this slice
  const int G = lane >> 4, j = lane & 15, rr = j >> 2, q = j & 3, g = lane >> 5;
  const int col0 = 16 * (G & 1) + 4 * q;
  f32x16 acc = {};
#pragma unroll
  for (int k = 0; k < KC; ++k) {
    const int row = 16 * k + 8 * g + rr;
    const bf16x4 lo = lds_read_tr16(&w[row * NCOL + col0]);
    const bf16x4 hi = lds_read_tr16(&w[(row + 4) * NCOL + col0]);
    const bf16x8 bv = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    acc = mfma32(av[k], bv, acc);
  }
  const int c = v0 + (lane & 31);
  if (c < DV) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int b = b0 + 8 * (i >> 2) + 4 * half + (i & 3);
      if (b < B) a.out[(static_cast<int64_t>(b) * H + h) * DV + c] = f32_to_bf16_bits(acc[i]);
    }
  }
}

}  // namespace

bool out_proj_supported(int d_c, int d_v) {
  return (d_c == 512 && d_v == 128) || (d_c == 32 && d_v == 16);
}

hipError_t launch_out_proj(const OutProjArgs& a, hipStream_t s) {
  if (a.d_c == 512 && a.d_v == 128) {
    hipLaunchKernelGGL((k_out_proj<512, 128>), dim3(a.H, 128 / 32, (a.B + 31) / 32), dim3(64), 0, s, a);
  } else if (a.d_c == 32 && a.d_v == 16) {
    hipLaunchKernelGGL((k_out_proj<32, 16>), dim3(a.H, 1, (a.B + 31) / 32), dim3(64), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mla
