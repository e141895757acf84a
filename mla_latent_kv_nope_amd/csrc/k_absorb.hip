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

  // GEMM workgroup: head h, latent columns [cbk*COLS, +COLS), batch rows
  // [b0, b0 + 32).  The W_UK slice and the q_nope rows are copied into LDS with
  // 16-byte global->LDS copies (row r's 16-byte chunk j stored at chunk
  // j ^ (r % CH)), read back as MFMA operands without bank conflicts, and the
  // 32 x COLS result goes back through LDS to leave as 16-byte stores.
  constexpr int CH = DN / 8;                 // 16-byte chunks per row
  constexpr int ROWB = DN * 2;
  static_assert((CH & (CH - 1)) == 0 && (COLS * ROWB) % 1024 == 0 && (32 * ROWB) % 1024 == 0,
                "copy shapes");
  __shared__ __attribute__((aligned(1024))) char wl[COLS * ROWB];   // W_UK slice [COLS][DN]
  __shared__ __attribute__((aligned(1024))) char ql[32 * ROWB];     // q_nope rows [32][DN]
  __shared__ __attribute__((aligned(16))) uint16_t ol[32 * (COLS + 8)];  // result [32][COLS]
  int id = blockIdx.x;
  const int cbk = id % NCB;
  id /= NCB;
  const int h = id % H;
  const int b0 = (id / H) * 32;              // batch rows [b0, b0 + 32)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int NWAVES = 4;

  // copies: lane l of 1 KB block k fills row (1024k + 16l) / ROWB, chunk
  // position p = l % CH with source chunk p ^ (row % CH)
  const uint16_t* wsrc = a.w_uk + (static_cast<int64_t>(h) * DC + cbk * COLS) * DN;
  for (int k = wave; k < COLS * ROWB / 1024; k += NWAVES) {
    const int r = (1024 * k + 16 * lane) / ROWB, pch = lane % CH;
    const uint16_t* src = wsrc + r * DN + 8 * (pch ^ (r % CH));
    lds_dma16_v(src, lds_addr(wl + 1024 * k));
  }
  for (int k = wave; k < 32 * ROWB / 1024; k += NWAVES) {
    const int r = (1024 * k + 16 * lane) / ROWB, pch = lane % CH;
    const int br = b0 + r < B ? b0 + r : b0;   // rows past the batch: any valid row
    const uint16_t* src = a.q_nope + (static_cast<int64_t>(br) * H + h) * DN + 8 * (pch ^ (r % CH));
    lds_dma16_v(src, lds_addr(ql + 1024 * k));
  }
  wait_vmcnt<0>();
  __syncthreads();

  if (wave < COLS / 32) {
    // A = q rows (lane: row l%32, k = 8(l/32) + [0,8) of each 16-wide step),
    // B = W_UK rows (lane: column l%32, same k)
    const int r = lane & 31, half = lane >> 5;
    const int cw = wave * 32 + r;
    f32x16 acc = {};
#pragma unroll
    for (int k = 0; k < DN / 16; ++k) {
      const int ch = 2 * k + half;
      const bf16x8 av = *reinterpret_cast<const bf16x8*>(ql + r * ROWB + 16 * (ch ^ (r % CH)));
      const bf16x8 bv = *reinterpret_cast<const bf16x8*>(wl + cw * ROWB + 16 * (ch ^ (cw % CH)));
      acc = mfma32(av, bv, acc);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int rr = 8 * (i >> 2) + 4 * half + (i & 3);
      ol[rr * (COLS + 8) + cw] = f32_to_bf16_bits(acc[i]);
    }
  }
  __syncthreads();
  // rows of the result: COLS columns = COLS * 2 bytes each, 16 bytes per store
  constexpr int SPR = COLS / 8;              // 16-byte stores per row
  for (int i = threadIdx.x; i < 32 * SPR; i += 64 * NWAVES) {
    const int rr = i / SPR, c8 = i - rr * SPR;
    if (b0 + rr < B)
      *reinterpret_cast<uint4*>(a.q_out + (static_cast<int64_t>(b0 + rr) * H + h) * R + cbk * COLS + 8 * c8) =
          *reinterpret_cast<const uint4*>(&ol[rr * (COLS + 8) + 8 * c8]);
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
