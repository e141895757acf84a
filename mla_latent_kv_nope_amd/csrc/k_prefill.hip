// mla_prefill_paged: causal attention of a chunk of new tokens per sequence in
// the explicit (un-absorbed) form.
//
// Method: folding W_UK into the query pays off only in decode; in prefill the
// reordering lowers the arithmetic intensity (zskr.cn "LLM推理优化的新范式：从内存
// 墙到计算墙的跨越", section 2.2, the per-stage table), so prefill up-projects
// the cached latent to per-head K and V (K_h = C . W_UK[h], V_h = C . W_UV[h];
// "DeepSeek-V2拆解：MLA与MoE如何把KV缓存压降93.3%", sheratonhq.com, section 2.1)
// and runs dense attention over them, the RoPE key part shared by all heads.
// Long prompts arrive in chunks ("vLLM 部署 DeepSeek V3" page, chunked prefill
// of 2048-4096 tokens); a chunk's new token i of sequence b is the cached
// token at position seq_lens[b] - n_b + i and attends to positions <= its own.
//
// Two kernels:
//   k_up       one workgroup of eight waves (two per SIMD) per (head, 1024
//              tokens), launched once for K and once for V: the head's
//              [512 x 128] weight sits in LDS and is read with the gfx950
//              transpose read; each wave computes 64 tokens x 128 columns
//              (two 32-token blocks sharing every weight operand), its latent
//              rows going from the paged pool straight into MFMA registers in
//              eight parts of the reduction, the next part loading while this
//              part's MFMAs run; an fp8 cache's codes become bf16 (code *
//              scale) at the MFMA.  K_nope is written [h][t][128] and V transposed
//              per 32-token tile, [h][t / 32][128][32] (the MFMA operands are
//              swapped for V), so a key tile of one head is one contiguous
//              8 KB run in each; the head-0 workgroups of the K launch
//              also write the shared RoPE keys [t][64] as bf16.
//   k_prefill  one workgroup of four waves per (sequence, head, 128 new
//              tokens); each wave owns 32 queries.  K_nope, RoPE-key and V^T
//              tiles of 32 keys stream from the workspace through a four-slot
//              LDS ring filled by global->LDS copies three tiles ahead.  The
//              score tile is computed transposed, S^T = K . Q^T (32x32x16 bf16
//              MFMA, Q in registers), so each lane holds 16 keys of one query:
//              the online-softmax row max needs one cross-half exchange, and
//              P^T goes straight from the accumulators into the B operand of
//              O^T = V^T . P^T, whose accumulators keep the query on the lane
//              as well.  The softmax offset moves only when a row max rises by
//              more than 8 (base 2), so rescaling O is rare.
//   Workgroups of one (sequence, head) sit on one XCD (blockIdx mod 8), so
//   their K/V tiles are shared through that XCD's L2; the query tiles that
//   see the most keys start first.
#include <type_traits>

#include "mla_common.hpp"
#include "prefill.hpp"

namespace mla {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLazy = 8.f;                // base-2 headroom of the softmax offset

// Page row holding token t of a block-table row (ids outside the pool read
// page 0: results are then unspecified but every access stays in bounds).
__device__ __forceinline__ int64_t pool_row(const int32_t* bt_row, int t, int lg, int num_pages) {
  int page = bt_row[t >> lg];
  if (static_cast<unsigned>(page) >= static_cast<unsigned>(num_pages)) page = 0;
  return (static_cast<int64_t>(page) << lg) + (t & ((1 << lg) - 1));
}

__device__ __forceinline__ int seq_tokens(const PrefillArgs& a, int b) {
  const int s = a.seq_lens[b];
  return s < 0 ? 0 : (s > a.s_cap ? a.s_cap : s);
}

// V^T keeps each aligned 32-token block in the order the P.V product reads
// it: 16-byte chunk 2 s + g holds the keys 16 s + 4 g + [0, 4) and
// 16 s + 8 + 4 g + [0, 4), i.e. token k = 16 s + 8 e + 4 g + i sits at
// slot 8 (2 s + g) + 4 e + i.
__device__ __forceinline__ int vt_slot(int k) {
  const int s = k >> 4, e = (k >> 3) & 1, g = (k >> 2) & 1, i = k & 3;
  return 8 * (2 * s + g) + 4 * e + i;
}

// Lanes 2m (even) and 2m + 1 (odd) each hold values x0, x1 of two adjacent
// rows (index i, i + 1) in their own column.  Returns, as two bf16 in one
// word, the even lane's row i of both columns (its own x0, the odd lane's x0)
// and the odd lane's row i + 1 of both columns (the even lane's x1, its own
// x1): the odd lane hands over x0, the even lane x1, by one DPP swap.
__device__ __forceinline__ uint32_t pair_transpose(float x0, float x1, int odd) {
  const float send = odd ? x0 : x1;
  const float recv = __int_as_float(__builtin_amdgcn_update_dpp(
      0, __float_as_int(send), 0xB1 /* quad_perm 1,0,3,2 */, 0xF, 0xF, false));
  return odd ? pack_bf16x2(recv, x1) : pack_bf16x2(x0, recv);
}

// ---------------------------------------------------------------------------
// Up-projection
// ---------------------------------------------------------------------------
// kUpWaves waves per workgroup (two per SIMD), the reduction in kUpParts
// parts of 512 / kUpParts elements
constexpr int kUpWaves = 8, kUpParts = 8;

template <bool IS_V, bool FP8>
__global__ __launch_bounds__(64 * kUpWaves) void k_up(PrefillArgs a) {
  constexpr int WROW = kPfDh * 2;                             // bytes per weight row
  __shared__ __attribute__((aligned(1024))) char wl[kPfDc * WROW];   // 128 KB
  const int h = blockIdx.x;
  const int b = blockIdx.z;
  const int tb = blockIdx.y * kUpTokens;
  const int S = seq_tokens(a, b);
  if (tb >= S) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  // W[h] [512][128]: chunk c of row k stored at c ^ 2 (k mod 4), so a
  // transpose read's 16-lane group touches 4 rows in distinct banks
  const uint16_t* wsrc = (IS_V ? a.w_uv : a.w_uk) + static_cast<int64_t>(h) * kPfDc * kPfDh;
  for (int k = wave; k < kPfDc / 4; k += kUpWaves) {
    const int r = 4 * k + (lane >> 4);
    const int c = (lane & 15) ^ (2 * (r & 3));
    lds_dma16_v(wsrc + r * kPfDh + 8 * c, lds_addr(wl + 1024 * k));
  }

  const int r = lane & 31, half = lane >> 5;
  const int G = lane >> 4, rr = (lane & 15) >> 2, q = lane & 3;
  const int32_t* bt = a.block_table + static_cast<int64_t>(b) * a.max_pages;
  const int tend = tb + kUpTokens < S ? tb + kUpTokens : S;
  // pool row of token t0 + r (rows past the sequence repeat its last token,
  // so every 32-token block the attention reads holds finite values)
  auto row_of = [&](int t0) {
    const int t = t0 + r < S ? t0 + r : S - 1;
    return pool_row(bt, t, a.page_size_log2, a.num_pages);
  };
  // Latent elements as loaded: 8 bf16 (16 bytes) or, for an fp8 cache, 8
  // E4M3 codes (8 bytes) turned into bf16 as code * scale at the MFMA (the
  // same rounding the fp8 decode applies)
  using Raw = typename std::conditional<FP8, uint2, bf16x8>::type;
  constexpr int ES = FP8 ? 1 : 2;                              // bytes per element
  const char* pool = static_cast<const char*>(a.pool);
  auto row_ptr = [&](int64_t prow) { return pool + (prow * kPfRow + 8 * half) * ES; };
  auto to_bf16 = [&](const Raw& v, float sc) -> bf16x8 {
    if constexpr (FP8) {
      return __builtin_bit_cast(bf16x8, make_uint4(fp8x2_to_bf16x2_scaled<false>(v.x, sc), fp8x2_to_bf16x2_scaled<true>(v.x, sc),
                                                   fp8x2_to_bf16x2_scaled<false>(v.y, sc), fp8x2_to_bf16x2_scaled<true>(v.y, sc)));
    } else {
      (void)sc;
      return v;
    }
  };
  // each wave takes two 32-token blocks, so every weight operand read from
  // LDS feeds two MFMAs; the reduction runs in kUpParts parts through two
  // alternating register sets, the next part's loads in flight during this
  // part's MFMAs (the row pointers are formed once per block, so no wait for
  // a page id ever waits for those loads)
  constexpr int kStride = kUpWaves * 64;                       // tokens per pass of the workgroup
  constexpr int KS = kPfDc / 16 / kUpParts;                    // 16-element steps per part
  Raw qa[2][KS], qb[2][KS];
  int64_t prow[2] = {0, 0};
  float sc[2] = {1.f, 1.f};
  auto load_q = [&](Raw (*dst)[KS], int qq) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const char* base = row_ptr(prow[rb]);
#pragma unroll
      for (int s = 0; s < KS; ++s) dst[rb][s] = *reinterpret_cast<const Raw*>(base + (16 * KS * qq + 16 * s) * ES);
    }
  };
  auto set_rows = [&](int tq) {
    prow[0] = row_of(tq);
    prow[1] = row_of(tq + 32);
    if constexpr (FP8) {
      sc[0] = a.scales[prow[0]];
      sc[1] = a.scales[prow[1]];
    }
  };
  int t0 = tb + 64 * wave;
  if (t0 < tend) {
    set_rows(t0);
    load_q(qa, 0);
  }
  wait_vmcnt<0>();
  __syncthreads();
  for (; t0 < tend; t0 += kStride) {
    const int64_t prow_now[2] = {prow[0], prow[1]};
    const float sc_now[2] = {sc[0], sc[1]};
    f32x16 acc[2][4] = {};
    // the lane's part of each weight read address, per 32-column tile ct
    // (row 8 half + rr, the swizzled column chunk), formed here from a fresh
    // lane id so that it is not hoisted out of the loop: every read is one of
    // these four plus an immediate
    uint32_t wlane[4];
    {
      const int fl = lane_id_fresh();
      const int fhalf = fl >> 5, fG = fl >> 4, frr = (fl & 15) >> 2, fq = fl & 3;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const int col0 = 32 * ct + 16 * (fG & 1) + 4 * fq;
        wlane[ct] = static_cast<uint32_t>((8 * fhalf + frr) * WROW + ((col0 >> 3) ^ (2 * frr)) * 16 + (col0 & 7) * 2);
      }
    }
    auto compute_q = [&](const Raw (*av)[KS], int qq) {
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int row0 = 16 * (KS * qq + s);                   // + 8 half + rr in wlane
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          const bf16x4 lo = lds_read_tr16(wl + wlane[ct] + row0 * WROW);
          const bf16x4 hi = lds_read_tr16(wl + wlane[ct] + (row0 + 4) * WROW);
          const bf16x8 bv = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            const bf16x8 x = to_bf16(av[rb][s], sc_now[rb]);
            if constexpr (IS_V) acc[rb][ct] = mfma32(bv, x, acc[rb][ct]);
            else acc[rb][ct] = mfma32(x, bv, acc[rb][ct]);
          }
        }
        // (one 16-element step at a time: weight reads are not hoisted over
        // later steps, which would hold their operands in registers)
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    static_assert(kUpParts % 2 == 0, "parts alternate between the two register sets");
#pragma unroll
    for (int qq = 0; qq < kUpParts; qq += 2) {
      load_q(qb, qq + 1);
      compute_q(qa, qq);
      if (qq + 2 < kUpParts) {
        load_q(qa, qq + 2);
      } else if (t0 + kStride < tend) {
        set_rows(t0 + kStride);
        load_q(qa, 0);
      }
      compute_q(qb, qq + 1);
    }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int tblk = t0 + 32 * rb;
      // a block that starts past the sequence is not stored (its rows may lie
      // beyond the workspace's token capacity)
      if (tblk >= tend) break;
      if constexpr (!IS_V) {
        // the RoPE key rows (shared by all heads) go to the workspace once,
        // as bf16, from the head-0 workgroups: lane (r, half) moves elements
        // [32 half, +32) of token tblk + r's rotated key
        if (h == 0) {
          uint4* dst = reinterpret_cast<uint4*>(a.kr + (static_cast<int64_t>(b) * a.s_pad + tblk + r) * kPfDr + 32 * half);
          const char* src = pool + (prow_now[rb] * kPfRow + kPfDc + 32 * half) * ES;
          if constexpr (FP8) {
            const uint4 c0 = reinterpret_cast<const uint4*>(src)[0];
            const uint4 c1 = reinterpret_cast<const uint4*>(src)[1];
            const float f = sc_now[rb];
            const uint32_t w[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
            for (int k = 0; k < 4; ++k)
              dst[k] = make_uint4(fp8x2_to_bf16x2_scaled<false>(w[2 * k], f), fp8x2_to_bf16x2_scaled<true>(w[2 * k], f),
                                  fp8x2_to_bf16x2_scaled<false>(w[2 * k + 1], f), fp8x2_to_bf16x2_scaled<true>(w[2 * k + 1], f));
          } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) dst[k] = reinterpret_cast<const uint4*>(src)[k];
          }
        }
        // acc[rb][ct][i]: token tblk + 8 (i/4) + 4 half + i%4, column 32 ct + r;
        // the lane's part of the address is in the base pointer, the rest is
        // uniform
        // (the stride is made opaque here so that its 64 multiples are formed
        // at the stores in scalar registers, not hoisted out of the loop)
        int64_t ts = kPfDh;                                             // token stride
        __asm__ volatile("" : "+s"(ts));
        // lanes 2m and 2m + 1 swap one value (a 2 x 2 transpose), so each
        // stores two adjacent columns of one token as one 4-byte word: the
        // even lane token 8 (i/4) + i%4, the odd lane the next token
        uint16_t* kb = a.kn + ((static_cast<int64_t>(b) * a.H + h) * a.s_pad + tblk) * kPfDh +
                       4 * half * ts + (r & ~1);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
          for (int i = 0; i < 16; i += 2)
            *reinterpret_cast<uint32_t*>(kb + (8 * (i >> 2) + (i & 3) + (r & 1)) * ts + 32 * ct) =
                pair_transpose(acc[rb][ct][i], acc[rb][ct][i + 1], r & 1);
      } else {
        // acc[rb][ct][i]: column 32 ct + 8 (i/4) + 4 half + i%4, token tblk + r,
        // stored at slot vt_slot(r) of its 32-token block; the lane's part of
        // the address is in the base pointer, the rest is uniform
        // (the stride is made opaque here so that its 64 multiples are formed
        // at the stores in scalar registers, not hoisted out of the loop)
        int64_t cs = kPfKTile;                                          // column stride
        __asm__ volatile("" : "+s"(cs));
        // lanes 2m and 2m + 1 hold adjacent slots; after the 2 x 2 transpose
        // each stores both slots of one column as one 4-byte word: the even
        // lane column 32 ct + 8 (i/4) + 4 half + i%4, the odd lane the next
        uint16_t* vb = a.vt + ((static_cast<int64_t>(b) * a.H + h) * a.s_pad + tblk) * kPfDh +
                       4 * half * cs + vt_slot(r & ~1);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
          for (int i = 0; i < 16; i += 2)
            *reinterpret_cast<uint32_t*>(vb + (32 * ct + 8 * (i >> 2) + (i & 3) + (r & 1)) * cs) =
                pair_transpose(acc[rb][ct][i], acc[rb][ct][i + 1], r & 1);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Attention
// ---------------------------------------------------------------------------
// One ring slot: K_nope [32][128] (chunk c of key row r at c ^ (r mod 16)),
// K_rope [32][64] (chunk c at c ^ (r mod 8)), V^T [128][32] in vt_slot order
// (chunk c of row j at c ^ ((j / 4) mod 4)).
constexpr int kSlotKn = 0, kSlotKr = 8192, kSlotVt = 12288, kSlotBytes = 20480;
constexpr int kAhead = 3;                   // key tiles in flight while one is computed
constexpr int kSlots = kAhead + 1;          // ring slots (80 KB)
constexpr int kCopiesPerTile = 5;           // global->LDS copies per wave per tile

// s_waitcnt vmcnt(5 k): all but this wave's copies of its k most recently
// issued tiles have landed
__device__ __forceinline__ void wait_tiles_behind(int k) {
  if (k >= 2) wait_vmcnt<2 * kCopiesPerTile>();
  else if (k == 1) wait_vmcnt<kCopiesPerTile>();
  else wait_vmcnt<0>();
}

#pragma clang fp contract(off)
// RoPE pair (x0, x1) at angle pos * theta (theta = base^(-2i / 64), computed
// on the host): angle, sine, cosine and the rotation in double precision,
// rounded once to fp32
__device__ __forceinline__ void rope_pair64(float x0, float x1, double theta, int pos,
                                            float* y0, float* y1) {
  double s, c;
  sincos(static_cast<double>(pos) * theta, &s, &c);
  const double u = static_cast<double>(x0), v = static_cast<double>(x1);
  const double p0 = u * c;
  const double p1 = v * s;
  const double p2 = u * s;
  const double p3 = v * c;
  *y0 = static_cast<float>(p0 - p1);
  *y1 = static_cast<float>(p2 + p3);
}
#pragma clang fp contract(on)

__global__ __launch_bounds__(256, 2) void k_prefill(PrefillArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds[kSlots * kSlotBytes];   // 80 KB
  const int QT = a.q_tiles;
  const int L = blockIdx.x, xcd = L & 7, slot = L >> 3;
  const int u = 8 * (slot / QT) + xcd;                 // (sequence, head) unit
  if (u >= a.B * a.H) return;
  const int qt = QT - 1 - slot % QT;
  const int b = u / a.H, h = u - b * a.H;
  const int q0 = a.q_start[b];
  const int n = a.q_start[b + 1] - q0;
  const int nc = min(n, a.max_q_len);                  // new tokens computed
  if (kPfQTile * qt >= nc) return;
  const int S = seq_tokens(a, b);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar registers
  const int r = lane & 31, half = lane >> 5;

  // keys the workgroup needs: up to the position of its last new token
  const int last_i = min(kPfQTile * qt + kPfQTile - 1, nc - 1);
  const int kend = min(S, S - n + last_i + 1);
  const int NT = kend > 0 ? (kend + kPfKTile - 1) / kPfKTile : 0;
  // this wave's queries and their positions (-1: sees nothing)
  const int i = kPfQTile * qt + 32 * wave + r;
  const int row = q0 + i;
  const bool live = i < nc && row >= 0 && row < a.T;
  const int pos = i < nc ? S - n + i : -1;
  const int wlast = min(kPfQTile * qt + 32 * wave + 31, nc - 1);
  const int pw = kPfQTile * qt + 32 * wave < nc ? S - n + wlast : -1;   // wave's last position
  const int pfirst = S - n + kPfQTile * qt + 32 * wave;                    // and its first

  // Q as the B operand: step s < 8 holds q_nope[16 s + 8 half, +8), steps
  // 8..11 the rotated q_pe[16 (s - 8) + 8 half, +8) (pairs 8 (s - 8) + 4 half + e)
  bf16x8 qv[12];
  const bf16x8 zero = {};
  if (live) {
    const uint16_t* qn = a.q_nope + (static_cast<int64_t>(row) * a.H + h) * kPfDh + 8 * half;
#pragma unroll
    for (int s = 0; s < 8; ++s) qv[s] = *reinterpret_cast<const bf16x8*>(qn + 16 * s);
    const uint16_t* qp = a.q_pe + (static_cast<int64_t>(row) * a.H + h) * kPfDr + 8 * half;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint4 raw = *reinterpret_cast<const uint4*>(qp + 16 * s);
      const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
      uint32_t o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float y0, y1;
        rope_pair64(bf16_bits_to_f32(static_cast<uint16_t>(w[e] & 0xffffu)),
                    bf16_bits_to_f32(static_cast<uint16_t>(w[e] >> 16)),
                    a.rope_theta[8 * s + 4 * half + e], pos, &y0, &y1);
        o[e] = static_cast<uint32_t>(f32_to_bf16_bits(y0)) |
               (static_cast<uint32_t>(f32_to_bf16_bits(y1)) << 16);
      }
      qv[8 + s] = __builtin_bit_cast(bf16x8, make_uint4(o[0], o[1], o[2], o[3]));
    }
  } else {
#pragma unroll
    for (int s = 0; s < 12; ++s) qv[s] = zero;
  }

  const uint16_t* kr_b = a.kr + static_cast<int64_t>(b) * a.s_pad * kPfDr;
  const uint16_t* kn_bh = a.kn + (static_cast<int64_t>(b) * a.H + h) * a.s_pad * kPfDh;
  const uint16_t* vt_bh = a.vt + (static_cast<int64_t>(b) * a.H + h) * a.s_pad * kPfDh;
  // copies of key tile nt into slot base: 8 K_nope, 4 K_rope and 8 V^T copies
  // of 1 KB, five per wave; lane l of a copy fills LDS bytes [16 l, +16).
  // Each lane's sources for tile 0 are formed once; tile nt adds a uniform
  // offset (nt tiles of 32 tokens) to each of them
  const uint16_t* src_kn[2];
  const uint16_t* src_vt[2];
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2) {
    const int k = wave + 4 * k2;
    const int kr = 4 * k + (lane >> 4);
    src_kn[k2] = kn_bh + kr * kPfDh + 8 * ((lane & 15) ^ (kr & 15));
    const int j = 16 * k + (lane >> 2);
    src_vt[k2] = vt_bh + j * kPfKTile + 8 * ((lane & 3) ^ ((j >> 2) & 3));
  }
  const uint16_t* src_kr;
  {
    const int kr = 8 * wave + (lane >> 3);
    src_kr = kr_b + kr * kPfDr + 8 * ((lane & 7) ^ (kr & 7));
  }
  auto issue = [&](int nt, char* base) {
    const int64_t t0 = static_cast<int64_t>(kPfKTile) * nt;
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
      lds_dma16_v(src_kn[k2] + t0 * kPfDh, lds_addr(base + kSlotKn + 1024 * (wave + 4 * k2)));
    lds_dma16_v(src_kr + t0 * kPfDr, lds_addr(base + kSlotKr + 1024 * wave));
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
      lds_dma16_v(src_vt[k2] + t0 * kPfDh, lds_addr(base + kSlotVt + 1024 * (wave + 4 * k2)));
  };

  float m = kNegInf, l = 0.f;
  f32x16 o[4] = {};
  for (int k = 0; k < kAhead && k < NT; ++k) issue(k, lds + k * kSlotBytes);
  for (int nt = 0; nt < NT; ++nt) {
    // tiles nt + 1 .. nt + kAhead - 1 may still be in flight
    wait_tiles_behind(min(kAhead - 1, NT - 1 - nt));
    __syncthreads();                       // tile nt landed everywhere; the slot of tile nt - 1 is free
    if (nt + kAhead < NT) issue(nt + kAhead, lds + ((nt + kAhead) % kSlots) * kSlotBytes);
    const int t0 = kPfKTile * nt;
    if (t0 > pw) continue;                 // every key of the tile is after this wave's queries
    const char* sb = lds + (nt % kSlots) * kSlotBytes;

    // S^T tile: acc[e] is key t0 + 8 (e/4) + 4 half + e%4 of query r
    f32x16 sacc = {};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bf16x8 kv = *reinterpret_cast<const bf16x8*>(sb + kSlotKn + r * 256 + 16 * ((2 * s + half) ^ (r & 15)));
      sacc = mfma32(kv, qv[s], sacc);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bf16x8 kv = *reinterpret_cast<const bf16x8*>(sb + kSlotKr + r * 128 + 16 * ((2 * s + half) ^ (r & 7)));
      sacc = mfma32(kv, qv[8 + s], sacc);
    }

    // online softmax in base 2 (m is the running max of scale * log2(e) *
    // score); keys after a query's position are -inf, which only tiles
    // reaching past the wave's first position need; a query that has seen no
    // key yet keeps m = -inf with offset 0 (so p = 0, not NaN)
    if (t0 + kPfKTile - 1 > pfirst) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = t0 + 8 * (e >> 2) + 4 * half + (e & 3);
        sacc[e] = key <= pos ? sacc[e] : kNegInf;
      }
    }
    float tmax = kNegInf;
#pragma unroll
    for (int e = 0; e < 16; ++e) tmax = fmaxf(tmax, sacc[e]);
    tmax = max_across_half_waves(tmax) * a.scale_log2;
    // the offset moves only when the row max rises by more than kLazy, so
    // p <= 2^kLazy (exact in bf16 and the fp32 sums) and the rescale below is
    // rare; the final division by the row sum cancels whatever offset is used
    const float mn = tmax > m + kLazy ? tmax : m;
    const float mu = mn == kNegInf ? 0.f : mn;
    const float alpha = __builtin_amdgcn_exp2f(m - mu);
    m = mn;
    float ls = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[e], a.scale_log2, -mu));
      sacc[e] = p;
      ls += p;
    }
    l = l * alpha + ls;
    if (__any(alpha != 1.f)) {             // rescale only when some row max moved
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[cb][e] *= alpha;
    }

    // O^T += V^T . P^T over the 32 keys in two 16-key steps; step s2 uses the
    // keys {16 s2 + 4 half + [0,4), 16 s2 + 8 + 4 half + [0,4)} on both sides
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const uint4 pk = make_uint4(pack_bf16x2(sacc[8 * s2 + 0], sacc[8 * s2 + 1]),
                                  pack_bf16x2(sacc[8 * s2 + 2], sacc[8 * s2 + 3]),
                                  pack_bf16x2(sacc[8 * s2 + 4], sacc[8 * s2 + 5]),
                                  pack_bf16x2(sacc[8 * s2 + 6], sacc[8 * s2 + 7]));
      const bf16x8 pb = __builtin_bit_cast(bf16x8, pk);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const int j = 32 * cb + r;
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(sb + kSlotVt + j * 64 +
                                                           16 * ((2 * s2 + half) ^ ((j >> 2) & 3)));
        o[cb] = mfma32(va, pb, o[cb]);
      }
    }
  }

  // normalise; o[cb][e] is O[query r][32 cb + 8 (e/4) + 4 half + e%4]
  const float lt = sum_across_half_waves(l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  __syncthreads();                         // every wave is done with the ring
  char* st = lds + 8192 * wave;            // [32 queries][128] bf16, chunk c at c ^ (query mod 16)
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint2 v = make_uint2(pack_bf16x2(o[cb][4 * g] * inv, o[cb][4 * g + 1] * inv),
                                 pack_bf16x2(o[cb][4 * g + 2] * inv, o[cb][4 * g + 3] * inv));
      *reinterpret_cast<uint2*>(st + r * 256 + 16 * ((4 * cb + g) ^ (r & 15)) + 8 * half) = v;
    }
  if (live && half == 0 && a.lse != nullptr)
    a.lse[static_cast<int64_t>(row) * a.H + h] =
        lt > 0.f ? (m + __builtin_log2f(lt)) * 0.69314718055994531f : kNegInf;
  __syncthreads();
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int k = lane + 64 * it;
    const int qr = k >> 4, c = k & 15;
    const int qi = kPfQTile * qt + 32 * wave + qr;
    const int orow = q0 + qi;
    if (qi < nc && orow >= 0 && orow < a.T) {
      const uint4 v = *reinterpret_cast<const uint4*>(st + qr * 256 + 16 * (c ^ (qr & 15)));
      *reinterpret_cast<uint4*>(a.out + (static_cast<int64_t>(orow) * a.H + h) * kPfDh + 8 * c) = v;
    }
  }
}

}  // namespace

bool prefill_supported(int d_c, int d_rope, int d_nope, int d_v) {
  return d_c == kPfDc && d_rope == kPfDr && d_nope == kPfDh && d_v == kPfDh;
}

int64_t prefill_s_pad(int64_t s_cap) { return (s_cap + kPfKTile - 1) / kPfKTile * kPfKTile; }

size_t prefill_workspace_bytes(int B, int H, int64_t s_cap) {
  const size_t one = static_cast<size_t>(B) * H * kPfDh * prefill_s_pad(s_cap) * 2;
  const size_t rope = static_cast<size_t>(B) * kPfDr * prefill_s_pad(s_cap) * 2;
  return 2 * ((one + 255) / 256 * 256) + (rope + 255) / 256 * 256;
}

size_t prefill_kv_bytes(int B, int H, int64_t s_cap) {
  const size_t one = static_cast<size_t>(B) * H * kPfDh * prefill_s_pad(s_cap) * 2;
  return (one + 255) / 256 * 256;
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s, hipEvent_t up0, hipEvent_t up1,
                          hipEvent_t at0, hipEvent_t at1) {
  if (a.B <= 0 || a.T <= 0 || a.q_tiles <= 0) return hipSuccess;
  const int64_t units = (static_cast<int64_t>(a.B) * a.H + 7) / 8 * 8;
  const int64_t grid = units * a.q_tiles;
  if (grid > 0x7fffffff || a.B > 65535) return hipErrorInvalidValue;
  const int ytiles = (a.s_cap + kUpTokens - 1) / kUpTokens;
  if (up0) (void)hipEventRecord(up0, s);
  if (a.fp8) {
    hipLaunchKernelGGL((k_up<false, true>), dim3(a.H, ytiles, a.B), dim3(64 * kUpWaves), 0, s, a);
    hipLaunchKernelGGL((k_up<true, true>), dim3(a.H, ytiles, a.B), dim3(64 * kUpWaves), 0, s, a);
  } else {
    hipLaunchKernelGGL((k_up<false, false>), dim3(a.H, ytiles, a.B), dim3(64 * kUpWaves), 0, s, a);
    hipLaunchKernelGGL((k_up<true, false>), dim3(a.H, ytiles, a.B), dim3(64 * kUpWaves), 0, s, a);
  }
  if (up1) (void)hipEventRecord(up1, s);
  if (at0) (void)hipEventRecord(at0, s);
  hipLaunchKernelGGL(k_prefill, dim3(static_cast<unsigned>(grid)), dim3(256), 0, s, a);
  if (at1) (void)hipEventRecord(at1, s);
  return hipGetLastError();
}

}  // namespace mla
