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
#include "append.hpp"
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

// One workgroup per (head h, 128 latent columns, 32 batch rows): the W_UK
// GEMM of that tile (4 waves x 32 columns), plus the RoPE half of the query for
// its share of the rows: the NCB column-block workgroups of a (head, 32 rows)
// tile each rotate 32 / NCB rows, one (row, pair) per thread with its angle
// evaluated in fp64.  Every workgroup needs 40 KB of LDS, so four fit on a CU
// and a 64-row batch at 128 heads runs in a single round of 1024 workgroups.
template <int DC, int DN>
__device__ __forceinline__ void absorb_block(const AbsorbArgs& a, int bid) {
  constexpr int COLS = DC < 128 ? DC : 128;  // latent columns per workgroup
  constexpr int NCB = DC / COLS;             // column blocks per head
  static_assert(COLS % 32 == 0 && DN % 16 == 0 && 32 % NCB == 0, "tile shape");
  const int B = a.B, H = a.H;
  const int R = DC + a.d_rope;

  // GEMM workgroup: head h, latent columns [cbk*COLS, +COLS), batch rows
  // [b0, b0 + 32).  The W_UK slice and the q_nope rows are copied into LDS with
  // 16-byte global->LDS copies (row r's 16-byte chunk j stored at chunk
  // j ^ (r % CH)), read back as MFMA operands without bank conflicts, and the
  // 32 x COLS result goes back through LDS to leave as 16-byte stores.
  constexpr int CH = DN / 8;                 // 16-byte chunks per row
  constexpr int ROWB = DN * 2;
  static_assert((CH & (CH - 1)) == 0 && (COLS * ROWB) % 1024 == 0 && (32 * ROWB) % 1024 == 0,
                "copy shapes");
  // the W_UK slice [COLS][DN]; after the MFMAs, the result [32][COLS] (padded
  // rows) in the same space
  constexpr int WL_BYTES = COLS * ROWB;
  constexpr int OL_BYTES = 32 * (COLS + 8) * 2;
  __shared__ __attribute__((aligned(1024))) char wl[WL_BYTES > OL_BYTES ? WL_BYTES : OL_BYTES];
  __shared__ __attribute__((aligned(1024))) char ql[32 * ROWB];     // q_nope rows [32][DN]
  uint16_t* const ol = reinterpret_cast<uint16_t*>(wl);
  int id = bid;
  const int cbk = id % NCB;
  id /= NCB;
  const int h = id % H;
  const int b0 = (id / H) * 32;              // batch rows [b0, b0 + 32)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int NWAVES = 4;

  // RoPE half of the query: rows [b0 + cbk * RPW, +RPW) of head h, one
  // (row, pair) per thread; its q_pe load is issued with the copies below
  constexpr int RPW = 32 / NCB;              // rows rotated by this workgroup
  const int pairs = a.d_rope / 2;
  const int rrow = static_cast<int>(threadIdx.x) / pairs, rpair = static_cast<int>(threadIdx.x) - rrow * pairs;
  const int rb = b0 + cbk * RPW + rrow;
  const bool rope_lane = rrow < RPW && rb < B;
  const uint32_t qpe =
      rope_lane ? *reinterpret_cast<const uint32_t*>(a.q_pe + (static_cast<int64_t>(rb) * H + h) * a.d_rope + 2 * rpair)
                : 0u;

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
  // the angle needs only the row's position: read with scalar loads (their
  // own counter), it is evaluated while the copies are in flight
  // (q_pos is read-only for the whole kernel; the constant address space
  // lets the compiler use scalar loads)
  const auto* qpos_c = (const __attribute__((address_space(4))) int32_t*)(a.q_pos);
  int rpos = 0;
#pragma unroll
  for (int j = 0; j < RPW; ++j) {
    const int bj = b0 + cbk * RPW + j;
    const int pj = bj < B ? qpos_c[bj] : 0;
    rpos = rrow == j ? pj : rpos;
  }
  double sn = 0.0, cs = 1.0;
  if (rope_lane) rope_angle(rpair, a.d_rope, rpos, a.rope_base, &sn, &cs);
  wait_vmcnt<0>();
  if (rope_lane) {
    float y0, y1;
    rope_rotate(bf16_bits_to_f32(static_cast<uint16_t>(qpe & 0xffffu)),
                bf16_bits_to_f32(static_cast<uint16_t>(qpe >> 16)), sn, cs, &y0, &y1);
    const uint32_t packed = static_cast<uint32_t>(f32_to_bf16_bits(y0)) |
                            (static_cast<uint32_t>(f32_to_bf16_bits(y1)) << 16);
    *reinterpret_cast<uint32_t*>(a.q_out + (static_cast<int64_t>(rb) * H + h) * R + DC + 2 * rpair) = packed;
  }
  __syncthreads();

  f32x16 acc = {};
  const int r = lane & 31, half = lane >> 5;
  const int cw = wave * 32 + r;
  if (wave < COLS / 32) {
    // A = q rows (lane: row l%32, k = 8(l/32) + [0,8) of each 16-wide step),
    // B = W_UK rows (lane: column l%32, same k)
#pragma unroll
    for (int k = 0; k < DN / 16; ++k) {
      const int ch = 2 * k + half;
      const bf16x8 av = *reinterpret_cast<const bf16x8*>(ql + r * ROWB + 16 * (ch ^ (r % CH)));
      const bf16x8 bv = *reinterpret_cast<const bf16x8*>(wl + cw * ROWB + 16 * (ch ^ (cw % CH)));
      acc = mfma32(av, bv, acc);
    }
  }
  __syncthreads();                           // the W_UK slice is read; its space takes the result
  if (wave < COLS / 32) {
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

template <int DC, int DN>
__global__ __launch_bounds__(256) void k_absorb(AbsorbArgs a) {
  absorb_block<DC, DN>(a, blockIdx.x);
}

// The absorb workgroups, then ceil(n_tokens / 4) workgroups that append the
// step's new latent rows (one wave per token).  The two parts touch disjoint
// memory; the append workgroups come last, so they run in the absorb's tail
// instead of holding back absorb workgroups.
template <int DC, int DN, bool FP8>
__global__ __launch_bounds__(256) void k_absorb_append(AbsorbArgs a, AppendArgs p, int n_absorb) {
  const int bid = blockIdx.x;
  if (bid >= n_absorb) {
    append_token<FP8, false>(p, (bid - n_absorb) * 4 + (threadIdx.x >> 6), threadIdx.x & 63);
    return;
  }
  absorb_block<DC, DN>(a, bid);
}

}  // namespace

bool absorb_supported(int d_c, int d_nope) {
  return (d_c == 512 && d_nope == 128) || (d_c == 32 && d_nope == 16);
}

hipError_t launch_absorb_append(const AbsorbArgs& a, const AppendArgs& p, hipStream_t s) {
  const dim3 block(256);
  const int rb = (a.B + 31) / 32;
  if (a.d_rope / 2 * (32 / (a.d_c < 128 ? 1 : a.d_c / 128)) > 256) return hipErrorInvalidValue;
  if (p.part != nullptr) return hipErrorInvalidValue;
  const int n_app = (p.n_tokens + 3) / 4;
  if (a.d_c == 512 && a.d_nope == 128) {
    const int n_abs = a.H * 4 * rb;
    if (p.fp8) hipLaunchKernelGGL((k_absorb_append<512, 128, true>), dim3(n_abs + n_app), block, 0, s, a, p, n_abs);
    else hipLaunchKernelGGL((k_absorb_append<512, 128, false>), dim3(n_abs + n_app), block, 0, s, a, p, n_abs);
  } else if (a.d_c == 32 && a.d_nope == 16) {
    const int n_abs = a.H * rb;
    if (p.fp8) hipLaunchKernelGGL((k_absorb_append<32, 16, true>), dim3(n_abs + n_app), block, 0, s, a, p, n_abs);
    else hipLaunchKernelGGL((k_absorb_append<32, 16, false>), dim3(n_abs + n_app), block, 0, s, a, p, n_abs);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_absorb(const AbsorbArgs& a, hipStream_t s) {
  const dim3 block(256);
  const int rb = (a.B + 31) / 32;
  if (a.d_rope / 2 * (32 / (a.d_c < 128 ? 1 : a.d_c / 128)) > 256) return hipErrorInvalidValue;
  if (a.d_c == 512 && a.d_nope == 128) {
    hipLaunchKernelGGL((k_absorb<512, 128>), dim3(a.H * 4 * rb), block, 0, s, a);
  } else if (a.d_c == 32 && a.d_nope == 16) {
    hipLaunchKernelGGL((k_absorb<32, 16>), dim3(a.H * rb), block, 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mla
