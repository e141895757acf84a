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
// rows), so they are loaded straight into MFMA registers.
#include "mla_common.hpp"
#include "mla_internal.hpp"

namespace mla {
namespace {

// Rotation angles of RoPE pair i at position pos: pos * base^(-2i / d_rope),
// evaluated in double precision (sine and cosine included).
__device__ __forceinline__ void rope_angle(int i, int d_rope, int pos, double base, double* s, double* c) {
  const double theta = pow(base, -2.0 * static_cast<double>(i) / static_cast<double>(d_rope));
  sincos(static_cast<double>(pos) * theta, s, c);
}

#pragma clang fp contract(off)
// (x0, x1) rotated by the angle with sine s and cosine c; products and sums in
// double precision, unfused, rounded once to fp32
__device__ __forceinline__ void rope_rotate(float x0, float x1, double s, double c, float* y0, float* y1) {
  const double a = static_cast<double>(x0), b = static_cast<double>(x1);
  const double p0 = a * c;
  const double p1 = b * s;
  const double p2 = a * s;
  const double p3 = b * c;
  *y0 = static_cast<float>(p0 - p1);
  *y1 = static_cast<float>(p2 + p3);
}
#pragma clang fp contract(on)

// Workgroups [0, n_gemm): the W_UK GEMM, one head x 128 latent columns
// (4 waves x 32 columns) x 32 batch rows each; every global load of a wave is
// in flight at once.  Workgroups [n_gemm, n_gemm + B * ceil(H / 32)): the RoPE
// half of the query for one batch row and 32 heads; the d_rope/2 angles of the
// row's position are evaluated once per workgroup.
template <int DC, int DN>
__global__ __launch_bounds__(256) void k_absorb(AbsorbArgs a, int n_gemm) {
  constexpr int COLS = DC < 128 ? DC : 128;  // latent columns per workgroup
  constexpr int NCB = DC / COLS;             // column blocks per head
  constexpr int KC = DN / 16;                // reduction chunks
  static_assert(COLS % 32 == 0 && DN % 16 == 0, "tile shape");
  const int B = a.B, H = a.H;
  const int R = DC + a.d_rope;

  if (static_cast<int>(blockIdx.x) >= n_gemm) {
    // RoPE workgroup: batch row b, heads [hb, hb + 32); one pair per thread and
    // pass, all loads of the workgroup in flight together
    constexpr int HPW = 32;                    // heads per RoPE workgroup
    __shared__ double sc[2][64];
    const int id = blockIdx.x - n_gemm;
    const int hgrp = (H + HPW - 1) / HPW;
    const int b = id / hgrp, hb = (id - b * hgrp) * HPW;
    const int pairs = a.d_rope / 2;            // <= 32
    if (static_cast<int>(threadIdx.x) < pairs) {
      double sn, cs;
      rope_angle(threadIdx.x, a.d_rope, a.q_pos[b], a.rope_base, &sn, &cs);
      sc[0][threadIdx.x] = sn;
      sc[1][threadIdx.x] = cs;
    }
    constexpr int PASSES = HPW * 32 / 256;
    uint32_t v[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int idx = p * 256 + threadIdx.x;
      const int h = hb + idx / pairs, i = idx % pairs;
      v[p] = (idx < HPW * pairs && h < H)
                 ? *reinterpret_cast<const uint32_t*>(a.q_pe + (static_cast<int64_t>(b) * H + h) * a.d_rope + 2 * i)
                 : 0u;
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int idx = p * 256 + threadIdx.x;
      const int h = hb + idx / pairs, i = idx % pairs;
      if (idx < HPW * pairs && h < H) {
        float y0, y1;
        rope_rotate(bf16_bits_to_f32(static_cast<uint16_t>(v[p] & 0xffffu)),
                    bf16_bits_to_f32(static_cast<uint16_t>(v[p] >> 16)), sc[0][i], sc[1][i], &y0, &y1);
        const uint32_t packed = static_cast<uint32_t>(f32_to_bf16_bits(y0)) |
                                (static_cast<uint32_t>(f32_to_bf16_bits(y1)) << 16);
        *reinterpret_cast<uint32_t*>(a.q_out + (static_cast<int64_t>(b) * H + h) * R + DC + 2 * i) = packed;
      }
    }
    return;
  }

  int id = blockIdx.x;
  const int cbk = id % NCB;
  id /= NCB;
  const int h = id % H;
  const int b0 = (id / H) * 32;              // batch rows [b0, b0 + 32)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (wave >= COLS / 32) return;
  const int c = cbk * COLS + wave * 32 + (lane & 31);
  const int half = lane >> 5;
  const int br = b0 + (lane & 31);
  const bool ok = br < B;
  bf16x8 wreg[KC], qv[KC];
  const uint16_t* wrow = a.w_uk + (static_cast<int64_t>(h) * DC + c) * DN + 8 * half;
  const uint16_t* qrow = a.q_nope + (static_cast<int64_t>(ok ? br : 0) * H + h) * DN + 8 * half;
  const bf16x8 z = {};
#pragma unroll
  for (int k = 0; k < KC; ++k) {
    wreg[k] = *reinterpret_cast<const bf16x8*>(wrow + 16 * k);
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(qrow + 16 * k);
    qv[k] = ok ? v : z;   // rows past the batch contribute zeros
  }
  f32x16 acc = {};
#pragma unroll
  for (int k = 0; k < KC; ++k) acc = mfma32(qv[k], wreg[k], acc);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int b = b0 + 8 * (i >> 2) + 4 * half + (i & 3);
    if (b < B) a.q_out[(static_cast<int64_t>(b) * H + h) * R + c] = f32_to_bf16_bits(acc[i]);
  }
}

}  // namespace

bool absorb_supported(int d_c, int d_nope) {
  return (d_c == 512 && d_nope == 128) || (d_c == 32 && d_nope == 16);
}

hipError_t launch_absorb(const AbsorbArgs& a, hipStream_t s) {
  const dim3 block(256);
  const int rb = (a.B + 31) / 32;
  if (a.d_c == 512 && a.d_nope == 128) {
    const int n_gemm = a.H * 4 * rb;
    hipLaunchKernelGGL((k_absorb<512, 128>), dim3(n_gemm + a.B * ((a.H + 31) / 32)), block, 0, s, a, n_gemm);
  } else if (a.d_c == 32 && a.d_nope == 16) {
    const int n_gemm = a.H * rb;
    hipLaunchKernelGGL((k_absorb<32, 16>), dim3(n_gemm + a.B * ((a.H + 31) / 32)), block, 0, s, a, n_gemm);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mla
