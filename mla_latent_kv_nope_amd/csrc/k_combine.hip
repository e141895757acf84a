// Merge of the pieces of split sequences (second phase of mla_decode_paged),
// alone or fused with the output projection W_UV.
//
// Method: a sequence cut into pieces p with normalised partial outputs O_p and
// log-sum-exp lse_p has lse = log sum_p exp(lse_p) and
// o_lat = sum_p exp(lse_p - lse) O_p; the split itself is this library's own
// design (the pages do not describe one).  The fused form applies W_UV on the
// output side ("DeepSeek-V2拆解：MLA与MoE如何把KV缓存压降93.3%",
// sheratonhq.com, section 2.1) while the merged latent rows are still on
// chip: operator fusion to cut memory round trips ("当MoE遇见MLA，推理效率的
// '黄金搭档'", agent.csdn.net, section 2.3; "LLM推理优化的新范式：从内存墙到
// 计算墙的跨越", zskr.cn, section 4.2).
//
// Partial slots (written by k_split): slot w + b of piece w of query sequence
// b holds bf16 rows [16 ceil(H/16)][d_c] (normalised O) and fp32 lse [H].  The
// pieces of sequence b are w = (plan[b] + pc) / quota .. (plan[b + 1] - 1) /
// quota, plan[] being cost positions and pc the per-sequence start cost.
// Both kernels add the pieces in piece order in fp32, each weighted by
// exp(lse_p - max lse), and divide by the sum of the weights.
#include "mla_common.hpp"
#include "mla_internal.hpp"

namespace mla {
namespace {

// Pieces of query sequence b: first piece wf and count np (0: no tokens).
struct PieceRange {
  int wf, np;
};
__device__ __forceinline__ PieceRange piece_range(const DecodeArgs& a, int b) {
  const int c0 = a.plan[b], c1 = a.plan[b + 1], quota = a.plan[a.B + 1], pc = a.plan[a.B + 2];
  if (c1 == c0) return {0, 0};
  const int wf = (c0 + pc) / quota, wl = (c1 - 1) / quota;
  return {wf, wl - wf + 1};
}

// Merged row chunks of head h of query sequence b: chunk k of this thread is
// 8 columns starting at col[k]; acc[k] receives the merged fp32 values (not
// yet rounded), the return value is the merged lse.  np >= 1.  PG pieces'
// chunks are in flight per round trip; the arithmetic (and so the result) is
// the same for every PG.
template <int CPT, int PG = 4>
__device__ __forceinline__ float merge_chunks(const DecodeArgs& a, int b, PieceRange pr, int h,
                                              const int (&col)[CPT], float (&acc)[CPT][8]) {
  const int H = a.H, HP = (H + 15) & ~15;
  const int64_t slot0 = static_cast<int64_t>(pr.wf) + b;
  uint4 t[PG][CPT];
  float l[PG];
  // rows and lse of pieces k0 .. k0 + PG - 1, all loads in flight together
  auto load_group = [&](int k0) {
#pragma unroll
    for (int k = 0; k < PG; ++k) {
      const bool ok = k0 + k < pr.np;
      const int64_t slot = slot0 + (ok ? k0 + k : 0);
      const uint16_t* row = a.part_o + (slot * HP + h) * a.d_c;
#pragma unroll
      for (int c = 0; c < CPT; ++c) t[k][c] = *reinterpret_cast<const uint4*>(row + col[c]);
      l[k] = ok ? a.part_lse[slot * H + h] : -INFINITY;
    }
  };
  load_group(0);
  float mx = -INFINITY;
  for (int k0 = PG; k0 < pr.np; k0 += PG) {         // more than PG pieces: their maximum first
    float x[PG];
#pragma unroll
    for (int k = 0; k < PG; ++k) x[k] = k0 + k < pr.np ? a.part_lse[(slot0 + k0 + k) * H + h] : -INFINITY;
#pragma unroll
    for (int k = 0; k < PG; ++k) mx = fmaxf(mx, x[k]);
  }
#pragma unroll
  for (int k = 0; k < PG; ++k) mx = fmaxf(mx, l[k]);
  float sum = 0.f;
  for (int k0 = 0; k0 < pr.np; k0 += PG) {
    if (k0 > 0) load_group(k0);
#pragma unroll
    for (int k = 0; k < PG; ++k) {
      if (k0 + k >= pr.np) break;
      const float wgt = expf(l[k] - mx);
      sum += wgt;
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const uint32_t u[4] = {t[k][c].x, t[k][c].y, t[k][c].z, t[k][c].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lo = __uint_as_float(u[e] << 16), hi = __uint_as_float(u[e] & 0xffff0000u);
          if (k0 + k == 0) {
            acc[c][2 * e] = lo * wgt;
            acc[c][2 * e + 1] = hi * wgt;
          } else {
            acc[c][2 * e] += lo * wgt;
            acc[c][2 * e + 1] += hi * wgt;
          }
        }
      }
    }
  }
  const float inv = 1.0f / sum;
#pragma unroll
  for (int c = 0; c < CPT; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[c][e] *= inv;
  return mx + logf(sum);
}

__device__ __forceinline__ uint4 pack_bf16x8(const float (&v)[8]) {
  return make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                    pack_bf16x2(v[6], v[7]));
}

// ---------------------------------------------------------------------------
// k_combine: one workgroup per (query sequence, RPW heads); TPR threads per
// head row, each merging CPT 16-byte chunks (a row's threads read 16 * TPR
// contiguous bytes per chunk), 16 / CPT pieces in flight (CPT 1: for batches
// too small to fill the GPU with 16-head workgroups).  Writes o_lat / lse of
// split sequences and o_lat = 0, lse = -inf for sequences with no tokens; a
// whole sequence in one piece was written by k_split.
template <int DC, int CPT>
__global__ __launch_bounds__(64 * (DC / 128 > 0 ? DC / 128 : 1)) void k_combine(DecodeArgs a) {
  constexpr int THREADS = 64 * (DC / 128 > 0 ? DC / 128 : 1);
  constexpr int TPR = DC / 8 / CPT;
  constexpr int RPW = THREADS / TPR;                 // head rows per workgroup
  static_assert(CPT * TPR * 8 == DC && RPW * TPR == THREADS, "row split");
  const int H = a.H, HGR = (H + RPW - 1) / RPW;
  const int b = blockIdx.x / HGR;
  const int h = (blockIdx.x % HGR) * RPW + threadIdx.x / TPR;
  if (h >= H) return;                                // (no barrier in this kernel)
  const int r = threadIdx.x % TPR;
  uint16_t* const orow = a.o_lat + (static_cast<int64_t>(b) * H + h) * DC;
  const PieceRange pr = piece_range(a, b);
  if (pr.np == 0) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) *reinterpret_cast<uint4*>(orow + 8 * (r + TPR * c)) = make_uint4(0, 0, 0, 0);
    if (a.lse != nullptr && r == 0) a.lse[static_cast<int64_t>(b) * H + h] = -INFINITY;
    return;
  }
  if (pr.np == 1) return;
  int col[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) col[c] = 8 * (r + TPR * c);
  float acc[CPT][8];
  const float lse = merge_chunks<CPT, (16 / CPT < 4 ? 4 : 16 / CPT)>(a, b, pr, h, col, acc);
#pragma unroll
  for (int c = 0; c < CPT; ++c) *reinterpret_cast<uint4*>(orow + col[c]) = pack_bf16x8(acc[c]);
  if (a.lse != nullptr && r == 0) a.lse[static_cast<int64_t>(b) * H + h] = lse;
}

// ---------------------------------------------------------------------------
// k_combine_proj (d_c 512, d_v 128): one workgroup of 8 waves per (head h,
// 32 query sequences).  W_UV[h] (128 KB) is copied global->LDS while the
// workgroup merges the pieces of its 32 rows (16 threads per row, 4 chunks
// each) into bf16 o_lat rows in LDS (32 KB; also written out when the caller
// asks for o_lat); then wave w computes output columns [16w, 16w + 16) of all
// 32 rows on 16x16x32 bf16 MFMAs, A (o_lat rows) by 16-byte LDS reads and B
// (W_UV columns) by transpose reads.  Every sequence is merged here, a whole
// one from its single piece (weight exp(0) = 1: the same bf16 row).
// LDS layouts (16-byte chunks permuted within a row; whole rows still land
// in whole lines):
//   W_UV[h] [512][128] (256-byte rows): chunk c of row k at c ^ 2 (k mod 4),
//     so the 4 rows x 32 bytes a transpose read's 16-lane group touches fall
//     in distinct banks;
//   o_lat [32][512] (1 KB rows): chunk j of row m at j ^ (m mod 16), so the 16
//     rows an A read touches at one chunk spread over the banks.
// Grid: blocks L = 8 RB (h / 8) + 8 rb + h % 8 for RB row blocks: all row
// blocks of one head share blockIdx mod 8, hence one XCD and its L2 copy of
// W_UV[h].
constexpr int kCpRows = 32;

// Merge of rows row0 .. row0 + 8 CPT - 1 (query sequences) of head h into
// bf16 o_lat rows in LDS (chunk j of row m at j ^ (m mod 16)), and to o_lat
// / lse when asked: 64 / CPT threads per row, thread (m, r) taking chunks
// r + (64 / CPT) k, k < CPT, with 16 / CPT pieces in flight.  Rows past the
// batch (and sequences without tokens) are zero.
template <int CPT>
__device__ __forceinline__ void merge_rows(const DecodeArgs& a, int h, int row0, char* ol) {
  constexpr int DC = 512, TPR = 64 / CPT;
  const int H = a.H, BQ = a.B;
  const int m = threadIdx.x / TPR, r = threadIdx.x % TPR;
  const int bq = row0 + m;
  const PieceRange pr = bq < BQ ? piece_range(a, bq) : PieceRange{0, 0};
  int col[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) col[c] = 8 * (r + TPR * c);
  float acc[CPT][8];
  float lse = -INFINITY;
  if (pr.np > 0) {
    lse = merge_chunks<CPT, 16 / CPT>(a, bq, pr, h, col, acc);
  } else {
#pragma unroll
    for (int c = 0; c < CPT; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[c][e] = 0.f;
  }
  uint4 pk[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    pk[c] = pack_bf16x8(acc[c]);
    *reinterpret_cast<uint4*>(ol + m * (DC * 2) + 16 * ((r + TPR * c) ^ (m & 15))) = pk[c];
  }
  if (bq < BQ) {
    if (a.o_lat != nullptr) {
      uint16_t* const orow = a.o_lat + (static_cast<int64_t>(bq) * H + h) * DC;
#pragma unroll
      for (int c = 0; c < CPT; ++c) *reinterpret_cast<uint4*>(orow + col[c]) = pk[c];
    }
    if (a.lse != nullptr && r == 0) a.lse[static_cast<int64_t>(bq) * H + h] = lse;
  }
}

__global__ __launch_bounds__(512) void k_combine_proj(DecodeArgs a, const uint16_t* w_uv, uint16_t* out) {
  constexpr int DC = 512, DV = 128, MR = kCpRows;
  constexpr int WROW = DV * 2;                       // bytes per W_UV row
  __shared__ __attribute__((aligned(1024))) char wl[DC * WROW];       // 128 KB
  __shared__ __attribute__((aligned(1024))) char ol[MR * DC * 2];     // 32 KB
  const int H = a.H, BQ = a.B;
  const int RB = (BQ + MR - 1) / MR;
  const int L = blockIdx.x;
  const int h = (L / (8 * RB)) * 8 + (L & 7);
  const int rb = (L >> 3) % RB;
  if (h >= H) return;                                // uniform per workgroup, before any barrier
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  // ---- W_UV copy
  // copy i (0..127) fills LDS bytes [1024 i, +1024) = W rows 4i .. 4i + 3:
  // lane l fills row 4i + l/16 at chunk position l % 16 with logical chunk
  // (l % 16) ^ 2 (row mod 4); wave w issues copies 16w .. 16w + 15
  {
    const uint16_t* wsrc = w_uv + static_cast<int64_t>(h) * DC * DV;
    const int rr = lane >> 4, pos = lane & 15;
    const int cl = pos ^ (2 * rr);
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      const int i = 16 * wave + n;
      lds_dma16_v(wsrc + (4 * i + rr) * DV + 8 * cl, lds_addr(wl + 1024 * i));
    }
  }

  // ---- merge: with few rows in the block, each row is spread over more
  // threads (fewer chunks each) and more pieces are in flight per round trip
  const int nrows = min(MR, BQ - rb * MR);
  if (nrows <= 8) merge_rows<1>(a, h, rb * MR, ol);
  else if (nrows <= 16) merge_rows<2>(a, h, rb * MR, ol);
  else merge_rows<4>(a, h, rb * MR, ol);
  wait_vmcnt<0>();
  __syncthreads();

  // ---- out[rows][16 wave .. +16) = o_lat rows . W_UV[h]
  const int g = lane >> 4, j = lane & 15;
  const int tr = j >> 2, tq = j & 3;                 // transpose-read source row / column quad
  const int col0 = 16 * wave + 4 * tq;               // W column of this lane's 8-byte read
  const uint32_t wb = static_cast<uint32_t>((((col0 >> 3) ^ (2 * tr)) * 16) + (col0 & 7) * 2);
  f32x4 acc[2] = {};
#pragma unroll 4
  for (int s = 0; s < DC / 32; ++s) {
    // B: rows 32 s + 8 g + tr and + 4 (both = tr mod 4), k slots 8 g .. 8 g + 7
    const char* wp = wl + (32 * s + 8 * g + tr) * WROW + wb;
    const bf16x4 lo = lds_read_tr16(wp);
    const bf16x4 hi = lds_read_tr16(wp + 4 * WROW);
    const bf16x8 bv = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      // A: row 16 t + j, logical chunk 4 s + g
      const int row = 16 * t + j;
      const bf16x8 av = *reinterpret_cast<const bf16x8*>(ol + row * (DC * 2) + 16 * ((4 * s + g) ^ j));
      acc[t] = mfma16(av, bv, acc[t]);
    }
  }
  // acc[t][i]: row 16 t + 4 g + i, column 16 wave + j
  const int v = 16 * wave + j;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = rb * MR + 16 * t + 4 * g + i;
      if (b < BQ) out[(static_cast<int64_t>(b) * H + h) * DV + v] = f32_to_bf16_bits(acc[t][i]);
    }
}

}  // namespace

hipError_t launch_combine(const DecodeArgs& a, hipStream_t s) {
  const int64_t hg16 = (a.H + 15) / 16, hg4 = (a.H + 3) / 4;
  if (a.d_c == 512) {
    // 16 heads per workgroup while that fills the compute units; else 4
    if (a.B * hg16 >= 256)
      hipLaunchKernelGGL((k_combine<512, 4>), dim3(static_cast<unsigned>(a.B * hg16)), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((k_combine<512, 1>), dim3(static_cast<unsigned>(a.B * hg4)), dim3(256), 0, s, a);
  } else if (a.d_c == 32) {
    hipLaunchKernelGGL((k_combine<32, 1>), dim3(static_cast<unsigned>(a.B * hg16)), dim3(64), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

bool combine_proj_supported(int d_c, int d_v) { return d_c == 512 && d_v == 128; }

hipError_t launch_combine_proj(const DecodeArgs& a, const uint16_t* w_uv, uint16_t* out, hipStream_t s) {
  if (a.d_c != 512) return hipErrorInvalidValue;
  const int rb = (a.B + kCpRows - 1) / kCpRows;
  const int64_t blocks = static_cast<int64_t>((a.H + 7) / 8) * 8 * rb;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_combine_proj, dim3(static_cast<unsigned>(blocks)), dim3(512), 0, s, a, w_uv, out);
  return hipGetLastError();
}

}  // namespace mla
