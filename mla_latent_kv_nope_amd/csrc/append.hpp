// The append of one new latent row (c_kv || RoPE(k_pe), optionally as fp8
// E4M3FN codes with one fp32 scale per token) into the paged cache, as a
// device function: the body of mla_append_latent's kernel, also run by the
// absorb kernel's extra workgroups when the two are launched together.
//
// Method: only the latent is cached and new tokens are appended before use
// ("DeepSeek-V2拆解：MLA与MoE如何把KV缓存压降93.3%", sheratonhq.com, section 2.1);
// the RoPE key lives in its own decoupled branch (same section), so it is
// rotated once here and stored rotated.  fp8 storage is the option named in
// "LLM推理优化的新范式：从内存墙到计算墙的跨越" (zskr.cn) section 5.
//
// One wave per token.  The row is split across lanes: lane l owns c_kv
// elements [8l, 8l+8) (one 16-byte load) and RoPE pair l.
#pragma once

#include "mla_common.hpp"
#include "mla_internal.hpp"

namespace mla {
namespace append_detail {

// fp32 -> E4M3FN code: nearest, ties to the even code, |q| >= 448 clamps to
// 448, NaN -> 0x7F.  The sign of a result that rounds to zero is kept.
__device__ __forceinline__ uint32_t e4m3fn_encode(float q) {
  const uint32_t sign = (__float_as_uint(q) >> 24) & 0x80u;
  const float a = fabsf(q);
  if (a != a) return 0x7Fu;
  if (!(a < 448.0f)) return sign | 0x7Eu;
  uint32_t code;
  if (a < 0x1p-6f) {
    // subnormal codes are the multiples of 2^-9; 8 * 2^-9 is the smallest normal
    code = static_cast<uint32_t>(__builtin_rintf(a * 512.0f));
  } else {
    int e;
    const float m = frexpf(a, &e);             // a = m * 2^e, m in [0.5, 1)
    const float frac = (2.0f * m - 1.0f) * 8.0f;  // exact: 3 fraction bits to keep
    // a mantissa that rounds up to 8 carries into the exponent field
    code = (static_cast<uint32_t>(e + 6) << 3) + static_cast<uint32_t>(__builtin_rintf(frac));
  }
  return sign | code;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}

#pragma clang fp contract(off)
// RoFormer rotation of pair i at position pos, in fp64, rounded to fp32.
__device__ __forceinline__ void rope_pair(float x0, float x1, int i, int d_rope, int pos,
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

}  // namespace append_detail

// PART: the row comes from fp32 partial sums (summed in chunk order, rounded
// to bf16) instead of bf16 c_kv / k_pe inputs.
// One wave per token: lane `lane` of the wave that writes token `tok`.
template <bool FP8, bool PART>
__device__ __forceinline__ void append_token(const AppendArgs& a, int tok, int lane) {
  if (tok >= a.n_tokens) return;
  const int seq = a.seq_ids[tok];
  const int pos = a.positions[tok];
  if (seq < 0 || seq >= a.num_seqs || pos < 0) return;
  const int pidx = pos >> a.page_size_log2;
  if (pidx >= a.max_pages) return;
  const int page = a.block_table[static_cast<int64_t>(seq) * a.max_pages + pidx];
  if (page < 0 || page >= a.num_pages) return;
  const int ps = 1 << a.page_size_log2;
  const int64_t row = static_cast<int64_t>(page) * ps + (pos & (ps - 1));
  const int d_c = a.d_c, d_rope = a.d_rope, R = d_c + d_rope;

  // c_kv: 8 elements per lane
  const bool has_c = 8 * lane < d_c;
  const bool has_r = 2 * lane < d_rope;
  uint4 cv = make_uint4(0, 0, 0, 0);
  uint32_t kp = 0;
  if constexpr (PART) {
    // sum the reduction chunks of this token's row in order, round to bf16
    const int64_t stride = static_cast<int64_t>(a.n_tokens) * R;
    const float* prow = a.part + static_cast<int64_t>(tok) * R;
    // eight chunks' loads in flight at a time, then added in chunk order
    constexpr int U = 8;
    float c[8] = {}, k0 = 0.f, k1 = 0.f;
    for (int p0 = 0; p0 < a.n_part; p0 += U) {
      float4 lo[U], hi[U];
      float2 kk[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float* src = prow + static_cast<int64_t>(p0 + u) * stride;
        const bool live = p0 + u < a.n_part;
        lo[u] = live && has_c ? *reinterpret_cast<const float4*>(src + 8 * lane) : float4{};
        hi[u] = live && has_c ? *reinterpret_cast<const float4*>(src + 8 * lane + 4) : float4{};
        kk[u] = live && has_r ? *reinterpret_cast<const float2*>(src + d_c + 2 * lane) : float2{};
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (p0 + u < a.n_part) {
          c[0] += lo[u].x; c[1] += lo[u].y; c[2] += lo[u].z; c[3] += lo[u].w;
          c[4] += hi[u].x; c[5] += hi[u].y; c[6] += hi[u].z; c[7] += hi[u].w;
          k0 += kk[u].x;
          k1 += kk[u].y;
        }
      }
    }
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = static_cast<uint32_t>(f32_to_bf16_bits(c[2 * j])) |
             (static_cast<uint32_t>(f32_to_bf16_bits(c[2 * j + 1])) << 16);
    cv = make_uint4(w[0], w[1], w[2], w[3]);
    kp = static_cast<uint32_t>(f32_to_bf16_bits(k0)) | (static_cast<uint32_t>(f32_to_bf16_bits(k1)) << 16);
  } else {
    if (has_c) cv = *reinterpret_cast<const uint4*>(a.c_kv + static_cast<int64_t>(tok) * d_c + 8 * lane);
    if (has_r) kp = *reinterpret_cast<const uint32_t*>(a.k_pe + static_cast<int64_t>(tok) * d_rope + 2 * lane);
  }
  // RoPE pair per lane
  float r0 = 0.f, r1 = 0.f;
  if (has_r) {
    const float x0 = bf16_bits_to_f32(static_cast<uint16_t>(kp & 0xffffu));
    const float x1 = bf16_bits_to_f32(static_cast<uint16_t>(kp >> 16));
    if (a.rope) append_detail::rope_pair(x0, x1, lane, d_rope, pos, a.rope_base, &r0, &r1);
    else { r0 = x0; r1 = x1; }
  }

  if constexpr (!FP8) {
    uint16_t* dst = static_cast<uint16_t*>(a.pool) + row * R;
    if (has_c) *reinterpret_cast<uint4*>(dst + 8 * lane) = cv;
    if (has_r) {
      const uint32_t packed = static_cast<uint32_t>(f32_to_bf16_bits(r0)) |
                              (static_cast<uint32_t>(f32_to_bf16_bits(r1)) << 16);
      *reinterpret_cast<uint32_t*>(dst + d_c + 2 * lane) = packed;
    }
  } else {
    float c[8];
    const uint32_t w[4] = {cv.x, cv.y, cv.z, cv.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      c[2 * j] = bf16_bits_to_f32(static_cast<uint16_t>(w[j] & 0xffffu));
      c[2 * j + 1] = bf16_bits_to_f32(static_cast<uint16_t>(w[j] >> 16));
    }
    float m = fmaxf(fabsf(r0), fabsf(r1));
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(c[j]));
    const float absmax = append_detail::wave_max(m);
    const float scale = __fdiv_rn(absmax, 448.0f);
    uint8_t* dst = static_cast<uint8_t*>(a.pool) + row * R;
    if (has_c) {
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t e0 = scale > 0.f ? append_detail::e4m3fn_encode(__fdiv_rn(c[j], scale)) : 0u;
        const uint32_t e1 = scale > 0.f ? append_detail::e4m3fn_encode(__fdiv_rn(c[4 + j], scale)) : 0u;
        lo |= e0 << (8 * j);
        hi |= e1 << (8 * j);
      }
      *reinterpret_cast<uint2*>(dst + 8 * lane) = make_uint2(lo, hi);
    }
    if (has_r) {
      const uint32_t e0 = scale > 0.f ? append_detail::e4m3fn_encode(__fdiv_rn(r0, scale)) : 0u;
      const uint32_t e1 = scale > 0.f ? append_detail::e4m3fn_encode(__fdiv_rn(r1, scale)) : 0u;
      *reinterpret_cast<uint16_t*>(dst + d_c + 2 * lane) = static_cast<uint16_t>(e0 | (e1 << 8));
    }
    if (lane == 0) a.scales[row] = scale;
  }
}

}  // namespace mla
