// mla_absorb_q: q[b][h] = (W_UK[h] . q_nope[b][h]) || RoPE(q_pe[b][h], q_pos[b]).
//
// Method: W_UK is absorbed into the query side ("DeepSeek-V2拆解：MLA与MoE如何把KV
// 缓存压降93.3%", sheratonhq.com, section 2.1); the reordered path multiplies Q
// by the up-projection weight before scoring against the compressed cache
// ("LLM推理优化的新范式：从内存墙到计算墙的跨越", zskr.cn, sections 2.1-2.2; the
// fused Q x W_DK kernel of section 4.2).
//
// A per-head batched GEMM [B x d_nope] x [d_nope x d_c] on 32x32x16 bf16 MFMA.
// Both operands are contiguous along the reduction axis (q_nope rows, W_UK
// rows), so they are loaded straight into MFMA registers.  Workgroup = one
// head x 128 latent columns (4 waves x 32 columns); the weight slice stays in
// registers while the batch is swept in blocks of 32 rows.  The weights are
// read exactly once, which is what bounds this kernel.
#include "mla_common.hpp"
#include "mla_internal.hpp"

namespace mla {
namespace {

#pragma clang fp contract(off)
__device__ __forceinline__ void rope_pair_q(float x0, float x1, int i, int d_rope, int pos,
                                            double base, float* y0, float* y1) {
  const double theta = pow(base, -2.0 * static_cast<double>(i) / static_cast<double>(d_rope));
  const double ang = static_cast<double>(pos) * theta;
  double s, c;
  sincos(ang, &s, &c);
  const double a = static_cast<double>(x0), b = static_cast<double>(x1);
  const double p0 = a * c;
  const double p1 = b * s;
  const double p2 = a * s;
  const double p3 = b * c;
  *y0 = static_cast<float>(p0 - p1);
  *y1 = static_cast<float>(p2 + p3);
}
#pragma clang fp contract(on)

template <int DC, int DN>
__global__ __launch_bounds__(256) void k_absorb(AbsorbArgs a) {
  constexpr int COLS = DC < 128 ? DC : 128;  // latent columns per workgroup
  constexpr int NWV = COLS / 32;             // waves doing MFMA
  constexpr int KC = DN / 16;                // reduction chunks
  static_assert(COLS % 32 == 0 && DN % 16 == 0, "tile shape");
  const int h = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int B = a.B, H = a.H;
  const int R = DC + a.d_rope;

  if (wave < NWV) {
    const int c = blockIdx.y * COLS + wave * 32 + (lane & 31);
    const int half = lane >> 5;
    bf16x8 wreg[KC];
    const uint16_t* wrow = a.w_uk + (static_cast<int64_t>(h) * DC + c) * DN + 8 * half;
#pragma unroll
    for (int k = 0; k < KC; ++k) wreg[k] = *reinterpret_cast<const bf16x8*>(wrow + 16 * k);

    for (int b0 = 0; b0 < B; b0 += 32) {
      const int br = b0 + (lane & 31);
      f32x16 acc = {};
      // every lane runs the MFMAs; rows past the batch contribute zeros
      const bool ok = br < B;
      const uint16_t* qrow = a.q_nope + (static_cast<int64_t>(ok ? br : 0) * H + h) * DN + 8 * half;
      const bf16x8 z = {};
#pragma unroll
      for (int k = 0; k < KC; ++k) {
        bf16x8 v = *reinterpret_cast<const bf16x8*>(qrow + 16 * k);
        acc = mfma32(ok ? v : z, wreg[k], acc);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int b = b0 + 8 * (i >> 2) + 4 * half + (i & 3);
        if (b < B) a.q_out[(static_cast<int64_t>(b) * H + h) * R + c] = f32_to_bf16_bits(acc[i]);
      }
    }
  }

  if (blockIdx.y == 0) {
    const int pairs = a.d_rope / 2;
    for (int idx = threadIdx.x; idx < B * pairs; idx += blockDim.x) {
      const int b = idx / pairs, i = idx - b * pairs;
      const uint32_t v = *reinterpret_cast<const uint32_t*>(
          a.q_pe + (static_cast<int64_t>(b) * H + h) * a.d_rope + 2 * i);
      float y0, y1;
      rope_pair_q(bf16_bits_to_f32(static_cast<uint16_t>(v & 0xffffu)),
                  bf16_bits_to_f32(static_cast<uint16_t>(v >> 16)), i, a.d_rope, a.q_pos[b],
                  a.rope_base, &y0, &y1);
      const uint32_t packed = static_cast<uint32_t>(f32_to_bf16_bits(y0)) |
                              (static_cast<uint32_t>(f32_to_bf16_bits(y1)) << 16);
      *reinterpret_cast<uint32_t*>(a.q_out + (static_cast<int64_t>(b) * H + h) * R + DC + 2 * i) =
          packed;
    }
  }
}

}  // namespace

bool absorb_supported(int d_c, int d_nope) {
  return (d_c == 512 && d_nope == 128) || (d_c == 32 && d_nope == 16);
}

hipError_t launch_absorb(const AbsorbArgs& a, hipStream_t s) {
  const dim3 block(256);
  if (a.d_c == 512 && a.d_nope == 128) {
    hipLaunchKernelGGL((k_absorb<512, 128>), dim3(a.H, 512 / 128), block, 0, s, a);
  } else if (a.d_c == 32 && a.d_nope == 16) {
    hipLaunchKernelGGL((k_absorb<32, 16>), dim3(a.H, 1), block, 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mla
