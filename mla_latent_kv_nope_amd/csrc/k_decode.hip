// mla_decode_paged: single-query softmax attention of all heads over the paged
// latent cache, with the latent used as V (absorbed MLA decode).
//
// Method: "DeepSeek-V2拆解：MLA与MoE如何把KV缓存压降93.3%" (sheratonhq.com)
// section 2.1 (cache only the latent; absorb W_UK / W_UV) and
// "LLM推理优化的新范式：从内存墙到计算墙的跨越" (zskr.cn) section 2.2 (the
// reordered path scores Q.W_UK directly against the compressed cache).  The
// split into partial results merged by their log-sum-exp is this library's
// own design; the pages do not describe one.
//
// This file holds the first of two kernels enqueued on the caller's stream:
//   k_split   every workgroup first derives the plan (tiles per sequence,
//             32 tokens each, on a cost line that may charge each sequence a
//             fixed start cost; quota = ceil(total cost / parts)); workgroup w
//             then takes the tiles at cost positions [w*quota, (w+1)*quota)
//             of the concatenated batch; a range may cover the tail of one
//             sequence and the head of the next.  A piece that is a whole sequence
//             writes o_lat/lse directly (unless o_lat is null); otherwise the
//             piece's normalised O (bf16 rows [head][d_c]) and lse (fp32) go
//             to slot w + b of the workspace.
//   The second (k_combine.hip) merges the pieces by their log-sum-exp, alone
//   or together with the W_UV output projection.
//
// k_split design (gfx950): one workgroup of NW waves holds every head of one
// sequence piece (NW = 8 for up to 128 heads), so each 32-token tile of
// 576-element rows is fetched from HBM once and shared by all heads.  Tiles
// are gathered page by page with direct global->LDS 16-byte copies into a ring
// of NBUF buffers (two tiles in flight while two are in use); 16-byte chunks
// are XOR-swizzled within 1 KB blocks of 8 rows so that the row-strided MFMA
// operand reads spread over the LDS banks.  One barrier per tile: step it
// computes S(it) = K_tile . Q^T and its softmax, publishes P(it) (bf16, PV
// A-operand order) to a double-buffered LDS slot, and accumulates
// O += P(it - 1) . V_tile(it - 1) on 16x16x32 bf16 MFMAs with V read by the
// LDS transpose read.  The softmax is base-2 with a per-head exponent offset
// fixed by the piece's first tile; a piece whose scores later exceed it by
// more than kHeadroom is recomputed once with the true maxima.
//   General layout (the tiny dims): every wave scores 16 heads (Q in 72
//        VGPRs; the head's row max is shared by four lanes) and accumulates
//        O for all heads over its d_c / NW columns.
//   Specialised layout (d_c 512, d_rope 64, NW 8, bf16 or fp8 cache): waves
//        0-3 score 32 heads each, every K operand read feeding the MFMAs of
//        two 16-head groups (Q in 144 VGPRs, four independent accumulator
//        chains), and accumulate O for 2 column blocks; waves 4-7 accumulate
//        O for 6 column blocks each and issue all tile copies, so the
//        copies' issue stalls never hold up the scoring waves.  An fp8 cache
//        stays fp8 in LDS: the scoring waves convert their K reads to bf16 in
//        registers, and V reaches the P.V MFMAs through 8-bit transpose
//        reads; the per-token scale multiplies the scores and P.
#include <atomic>
#include <type_traits>

#include "mla_common.hpp"
#include "mla_internal.hpp"

namespace mla {
namespace {

constexpr float kLn2 = 0.69314718055994530942f;
// With the exponent offset fixed per piece, P = 2^(x - m) stays below
// 2^kHeadroom (far inside fp32 and bf16 range) unless a score exceeds the
// offset by more than that; such a piece is recomputed with its true maximum.
constexpr float kHeadroom = 64.0f;  // log2 units

// What starting one more piece inside a workgroup's range costs, in tiles
// (the query load, the ring's refill and the partial store; measured about
// 3-4 tiles of steady-state work): the plan charges it per sequence when the
// batch's lengths differ.
constexpr int kPieceCost = 4;

// MFMA operand reads kept in flight ahead of their MFMA: QK^T of the general
// layout, and the specialised layout's K reads (each feeding two MFMAs; a
// second read in flight costs a spill reload per tile, and is slower)
constexpr int kQkAhead = 4;
constexpr int kQk2Ahead = 1;
constexpr int kQk8Ahead = 2;   // (fp8 cache: 16-byte reads, each feeding four MFMAs)

template <int DC, int DR, int NW, bool FP8 = false>
struct DecodeCfg {
  static constexpr int R = DC + DR;
  static constexpr int ROWB = 2 * R;                 // bytes per bf16 row
  static constexpr int CPR = ROWB / 16;              // 16-byte chunks per row
  // Blocked LDS layout (rows of a multiple of 8 chunks): the tile is a grid of
  // 1 KB blocks of 8 rows x 8 chunks; inside a block, chunk c of row r sits at
  // position r*8 + (c ^ r).  Otherwise plain row-major.
  static constexpr bool BLOCKED = (CPR % 8) == 0;
  static constexpr int CG = CPR / 8;                 // chunk groups per row (blocked)
  static constexpr int TILE_BYTES = kTile * ROWB;
  static constexpr int INSTR = kTile * CPR / 64;     // 1 KB wave loads per tile
  static constexpr int THREADS = 64 * NW;
  // tile loads are issued by the last LW waves (the others start computing
  // right after each barrier); loader i issues blocks i, i + LW, ...
  // Specialised layout (d_c 512, d_rope 64, 8 waves, bf16 or fp8 cache):
  // waves 0-3 score 32 heads each, waves 4-7 accumulate most of O and issue
  // every tile copy (bf16: loader i copies the tile's 8-row group i).
  static constexpr bool SPEC = NW == 8 && DC == 512 && DR == 64;
  static constexpr int LW = SPEC ? 4 : NW;
  static constexpr int LD_HI = (INSTR + LW - 1) / LW;  // loads of loaders < INSTR % LW (or all)
  static constexpr int LD_LO = INSTR / LW;
  static constexpr int K32 = R / 32;                 // full 32-wide QK chunks
  static constexpr bool K16 = (R % 32) == 16;        // one 16-wide tail chunk
  static constexpr int VCB = DC / 16;                // PV column blocks
  static constexpr int LDS_MAX = 160 * 1024;
  static constexpr int nbuf() {
    int n = 2;
    while ((n + 1) * TILE_BYTES <= LDS_MAX && (n - 1) * LD_HI <= 63 && n < 4) ++n;
    return n;
  }
  // fp8 cache (specialised layout only): the tiles stay fp8 in a ring of NBUF
  // slots of F8S_SLOT bytes (nope blocks, rope blocks, then the 32 fp32
  // scales; the layout is described at the copies)
  static_assert(!FP8 || SPEC, "the fp8 cache runs in the specialised layout");
  static constexpr bool SPEC8 = SPEC && FP8;
  static constexpr int F8S_ROPE = kTile * DC;           // rope blocks after the 16 KB of nope blocks
  static constexpr int F8S_SCL = kTile * R;             // scales after the two rope blocks
  static constexpr int F8S_SLOT = (kTile * R + 4 * kTile + 1023) / 1024 * 1024;
  static constexpr int NBUF = FP8 ? 7 : nbuf();
  static constexpr int SLOT_BYTES = SPEC8 ? F8S_SLOT : TILE_BYTES;
  static_assert(R % 16 == 0 && DC % 16 == 0, "dims");
  static_assert((kTile * CPR) % 64 == 0, "tile load split");
  static_assert(SPEC8 || (NBUF - 2) * LD_HI <= 63, "vmcnt range");
  static_assert(!SPEC8 || (DC == 16 * kTile && DR == 2 * kTile && (NBUF - 2) * 5 <= 63 && F8S_SLOT % 1024 == 0),
                "fp8 slot: 16 nope blocks, 2 rope blocks, the scales; up to 5 copies per loader and tile");
  static_assert(!BLOCKED || TILE_BYTES % 1024 == 0, "blocked tiles keep the low 10 address bits free");
};

// byte offset of (row t, 16-byte chunk c) inside a tile buffer
template <class Cfg>
__device__ __forceinline__ uint32_t lds_off(int t, int c) {
  if constexpr (Cfg::BLOCKED)
    return ((t >> 3) * Cfg::CG + (c >> 3)) * 1024 + (t & 7) * 128 + (((c & 7) ^ (t & 7)) * 16);
  else
    return t * Cfg::ROWB + c * 16;
}

// waits until at most `pending` tiles' loads of this wave (L loads per tile)
// are outstanding
template <int NBUF, int L>
__device__ __forceinline__ void wait_tiles(int pending) {
  if constexpr (NBUF >= 4) {
    if (pending >= 2) { wait_vmcnt<2 * L>(); return; }
  }
  if constexpr (NBUF >= 3) {
    if (pending >= 1) { wait_vmcnt<L>(); return; }
  }
  wait_vmcnt<0>();
}

// waits until at most `pending` (0 <= pending <= P, wave-uniform) groups of L
// vector memory operations of this wave are outstanding
template <int P, int L>
__device__ __forceinline__ void wait_pending(int pending) {
  if constexpr (P == 0) {
    wait_vmcnt<0>();
  } else {
    if (pending >= P) {
      wait_vmcnt<P * L>();
      return;
    }
    wait_pending<P - 1, L>(pending);
  }
}

// Scheduling hint for a run of N MFMAs, each fed by RD LDS reads: issue the
// reads of the first AHEAD MFMAs, then alternate one MFMA with the reads of
// the MFMA AHEAD places later.  Bounds the registers held by in-flight reads.
template <int N, int RD, int AHEAD_MAX>
__device__ __forceinline__ void sched_interleave() {
  constexpr int AHEAD = AHEAD_MAX < N ? AHEAD_MAX : N - 1;
  static_assert(AHEAD >= 1, "run too short");
  __builtin_amdgcn_sched_group_barrier(0x100, RD * AHEAD, 0);
#pragma unroll
  for (int i = 0; i < N - AHEAD; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, RD, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
}

__device__ __forceinline__ int clamp_len(int s, int cap) { return s < 0 ? 0 : (s > cap ? cap : s); }

// ---------------------------------------------------------------------------
// HBC (specialised layout only): 16-head blocks whose scores and O are
// computed, ceil(H / 16) rounded up to 1 or NW; the general layout always
// computes NW blocks.
template <int DC, int DR, int NW, bool FP8, int HBC>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW),
                          amdgpu_waves_per_eu((NW + 3) / 4, (NW + 3) / 4)))
void k_split(DecodeArgs a, int32_t* __restrict__ plan, const int32_t* __restrict__ seq_lens,
             const int32_t* __restrict__ block_table) {
  using Cfg = DecodeCfg<DC, DR, NW, FP8>;
  constexpr int R = Cfg::R, ROWB = Cfg::ROWB, CPR = Cfg::CPR;
  constexpr int CPW = Cfg::VCB / NW;          // PV column blocks per wave
  constexpr int PROW = 2 * kTile;             // bytes of one head's P row (bf16 per token)
  constexpr int PSLOT = 16 * NW * PROW;       // P of one tile, all heads
  static_assert(Cfg::VCB % NW == 0, "column blocks split evenly over the waves");
  static_assert(PROW == 64, "P rows are four 16-byte chunks");
  static_assert(!Cfg::BLOCKED || CPW % 4 == 0, "blocked PV reads start at a multiple of 4 column blocks");
  // tile ring, then two P slots (the second also carries the per-head 1/l at
  // the end of a piece; the first the overflow vote)
  __shared__ __attribute__((aligned(1024))) char lds[Cfg::NBUF * Cfg::SLOT_BYTES + 2 * PSLOT];
  char* const pbuf = lds + Cfg::NBUF * Cfg::SLOT_BYTES;
  int* const vote = reinterpret_cast<int*>(pbuf);
  float* const inv_share = reinterpret_cast<float*>(pbuf + PSLOT);

  // Piece index of this workgroup.  Workgroups are dispatched round-robin
  // over the 8 XCDs (blockIdx % 8); consecutive pieces, which are mostly the
  // pieces of one sequence, go to the same XCD so that they share its L2 for
  // the query and the block-table row.  A bijection on [0, num_parts).
  const int w = [&] {
    const int i = blockIdx.x, P = a.num_parts;
    const int x = i & 7, q8 = P >> 3, r8 = P & 7;
    return x * q8 + min(x, r8) + (i >> 3);
  }();

  // plan, seq_lens and block_table are read with scalar loads (restrict lets
  // the compiler prove nothing here writes them); scalar loads wait on their
  // own counter, so they never force a wait for the in-flight tile loads.
  const int B = a.B, H = a.H;
  const int HB = (H + 15) >> 4;               // 16-head blocks
  const int cap = a.max_pages << a.page_size_log2;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // ---- plan, computed by every workgroup.  The batch is a cost line: each
  // non-empty sequence costs its tiles plus pc (0 or kPieceCost) before its
  // first tile; quota = ceil(total cost / parts) and workgroup w takes the
  // tiles at cost positions [w * quota, (w + 1) * quota).  With ragged
  // lengths some workgroups' ranges hold several sequence starts, each one
  // more piece to run, and pc = kPieceCost spreads that cost; when every
  // non-empty sequence has the same tile count, pc = 0 (ranges then fall on
  // sequence starts or hold at most one, and a charge would only shift tiles
  // between workgroups).  Thread i sums the tiles and non-empty sequences of
  // a chunk of C consecutive sequences (and notes whether their tile counts
  // differ); wave scans plus the wave totals (in the P slots, unused until
  // the first tile) give each chunk's first position.  Workgroup 0 also
  // stores the cost prefix sums, the total, the quota and pc for the merge
  // kernels.
  // Query sequence v is new token qi = v % q_len of cache sequence cs =
  // v / q_len and sees len_of(cs, qi) tokens (the cache sequence's length less
  // its later new tokens).  (cs, qi) pairs are walked incrementally: one
  // division per thread here and one per workgroup for the piece loop.
  const int QL = a.q_len;
  auto len_of = [&](int cs, int qi) { return clamp_len(seq_lens[cs] - (QL - 1 - qi), cap); };
  auto tiles_len = [](int len) { return (len + kTile - 1) / kTile; };
  auto next_query = [&](int& cs, int& qi) {
    if (++qi == QL) {
      qi = 0;
      ++cs;
    }
  };
  int* const scan = reinterpret_cast<int*>(pbuf);
  const int C = (B + Cfg::THREADS - 1) / Cfg::THREADS;
  const int k0 = static_cast<int>(threadIdx.x) * C;
  const int cs0 = k0 / QL, qi0 = k0 - cs0 * QL;   // query sequence k0
  // Tiles of query sequence k0 + j of the chunk (walked as (cs, qi)); the plan
  // needs them in up to three passes.  With one sequence per thread (B <= 512,
  // the usual case) the length is loaded once, here, and no pass loops.
  const bool one = C == 1;
  const int n_one = (one && k0 < B) ? tiles_len(len_of(cs0, qi0)) : 0;
  int csum = 0, cne = 0;                        // tiles, non-empty sequences
  int n_first = -1;                             // tile count of the first non-empty one
  bool differs = false;                         // another one unlike it
  if (one) {
    csum = n_one;
    cne = n_one > 0;
    n_first = n_one > 0 ? n_one : -1;
  } else {
    int cs = cs0, qi = qi0;
    for (int j = 0; j < C; ++j, next_query(cs, qi))
      if (k0 + j < B) {
        const int n = tiles_len(len_of(cs, qi));
        csum += n;
        cne += n > 0;
        if (n > 0) {
          differs |= n_first >= 0 && n != n_first;
          if (n_first < 0) n_first = n;
        }
      }
  }
  int incl = csum;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d);
    if (lane >= d) incl += v;
  }
  // the wave's reference: the first lane holding a non-empty sequence
  const uint64_t has = __builtin_amdgcn_ballot_w64(n_first >= 0);
  const int ref = has != 0 ? __builtin_amdgcn_readlane(n_first, __builtin_ctzll(has)) : -1;
  differs |= n_first >= 0 && n_first != ref;
  const bool wave_differs = __builtin_amdgcn_ballot_w64(differs) != 0;
  if (lane == 63) {
    scan[wave] = incl;
    scan[NW + wave] = wave_differs;
    scan[2 * NW + wave] = ref;
  }
  __syncthreads();
  int total = 0, before = 0, ragged = 0, ref_all = -1;
  for (int i = 0; i < NW; ++i) {
    const int v = scan[i], r = scan[2 * NW + i];
    total += v;
    ragged |= scan[NW + i] | (r >= 0 && ref_all >= 0 && r != ref_all);
    if (ref_all < 0) ref_all = r;
    if (i < wave) before += v;
  }
  const int excl = before + incl - csum;       // tiles before this thread's chunk
  const int pc = ragged ? kPieceCost : 0;
  // cost positions: with a start cost, the non-empty sequences before each
  // chunk are counted too (a second scan, in words of its own)
  int total_c = total, excl_c = excl;
  if (pc != 0) {
    int incl_n = cne;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl_n, d);
      if (lane >= d) incl_n += v;
    }
    if (lane == 63) scan[3 * NW + wave] = incl_n;
    __syncthreads();
    int total_n = 0, before_n = 0;
    for (int i = 0; i < NW; ++i) {
      const int v = scan[3 * NW + i];
      total_n += v;
      if (i < wave) before_n += v;
    }
    total_c += pc * total_n;
    excl_c += pc * (before_n + incl_n - cne);
  }
  const int quota = total_c > 0 ? (total_c + a.num_parts - 1) / a.num_parts : 1;
  auto cost_of = [&](int n) { return n > 0 ? n + pc : 0; };
  if (w == 0) {
    if (one) {
      if (k0 < B) plan[k0] = excl_c;
    } else {
      int p0 = excl_c;
      int cs = cs0, qi = qi0;
      for (int j = 0; j < C; ++j, next_query(cs, qi))
        if (k0 + j < B) {
          plan[k0 + j] = p0;
          p0 += cost_of(tiles_len(len_of(cs, qi)));
        }
    }
    if (threadIdx.x == 0) {
      plan[B] = total_c;
      plan[B + 1] = quota;
      plan[B + 2] = pc;
    }
  }
  int g = w * quota;
  const int gend = min(g + quota, total_c);
  if (g >= gend) return;
  __syncthreads();                              // wave totals read before reuse
  // the chunk holding cost position g names the sequence containing it
  if (excl_c <= g && g < excl_c + csum + pc * cne) {
    if (one) {
      scan[0] = k0;
      scan[1] = excl_c;
    } else {
      int p0 = excl_c;
      int cs = cs0, qi = qi0;
      for (int j = 0; j < C; ++j, next_query(cs, qi)) {
        const int n = k0 + j < B ? cost_of(tiles_len(len_of(cs, qi))) : 0;
        if (g < p0 + n) {
          scan[0] = k0 + j;
          scan[1] = p0;
          break;
        }
        p0 += n;
      }
    }
  }
  __syncthreads();
  int b = scan[0];
  int t0 = scan[1];                             // cost position where sequence b starts
  int b_cs = b / QL, b_qi = b - b_cs * QL;      // its cache sequence and new-token index
  const int quad = lane >> 4;          // k slice (operands) / token quad (S) / head quad (O)
  const int l16 = lane & 15;
  const int lg = a.page_size_log2;
  const int ps = 1 << lg;
  const int hbase = wave * 16;         // QK: first head of this wave
  const bool qk_wave = hbase < H;
  const int cb0 = wave * CPW;          // PV: first column block of this wave
  constexpr int REM = Cfg::INSTR % Cfg::LW;
  const int loader = wave - (NW - Cfg::LW);      // loader index, negative for non-loaders
  const bool hi_loader = loader >= 0 && (REM == 0 || loader < REM);
  const bool lo_loader = loader >= 0 && !hi_loader;

  // The tile ring needs no initialisation: every row of every tile that is
  // read is copied first (a row past the sequence end copies the tile's first
  // row, a real token; a row whose page id lies outside the pool copies from
  // inside the pool), and ring slots beyond a piece's tile count are never
  // read.


  // Per-lane LDS byte offsets (relative to a tile buffer) of the MFMA operand
  // reads; every other operand address is one of these plus an immediate.  They
  // are recomputed from lane_id_fresh at each tile (a handful of VALU ops) so
  // that no register is held for them across the tile loop.
  // QK: row l16 (+16 per token block), chunk 4kc + quad: an even/odd base plus
  // 1 KB per chunk group (blocked) or 64 bytes per kc (row-major).  In the
  // blocked layout the odd base is the even one with chunk bit 2 flipped.
  struct QkBases { uint32_t even, odd, tail; };
  auto qk_bases = [&]() -> QkBases {
    const int l = lane_id_fresh();
    const int r = l & 15, q = l >> 4;
    QkBases qb;
    qb.even = lds_off<Cfg>(r, q);
    qb.odd = Cfg::BLOCKED ? (qb.even ^ 64u) : lds_off<Cfg>(r, 4 + q);
    // QK tail (16-wide, row-major layouts only): chunk 4*K32 + (quad & 1) of
    // row l16; lanes with quad >= 2 read the same in-row chunk and discard it
    qb.tail = Cfg::K16 ? lds_off<Cfg>(r, 4 * Cfg::K32 + (q & 1)) : 0u;
    return qb;
  };
  // fp8 K operand reads (specialised layout): chunk 4m + quad of row 16tbk +
  // l16 at even + 8192 tbk + 1024 (m / 2) when m % 2 == tbk, else at odd (the
  // even base with chunk bit 2 flipped) + the same; rope chunk quad at rope +
  // 1024 tbk past the nope blocks.
  struct K8Bases { uint32_t even, odd, rope; };
  auto k8_bases = [&]() -> K8Bases {
    const int l = lane_id_fresh();
    const int r = l & 15, q = l >> 4;
    K8Bases kb;
    kb.even = static_cast<uint32_t>(4096 * (r >> 3) + 128 * (r & 7) + 16 * (q ^ (r & 7)));
    kb.odd = kb.even ^ 64u;
    kb.rope = static_cast<uint32_t>(64 * r + 16 * (q ^ (r >> 2)));
    return kb;
  };
  // PV transpose reads: source lane 4r+q of its group reads row 4*quad + r (+16),
  // chunk 2cb + q/2, bytes 8*(q%2).  Blocked: the base for cb % 4 = m is the
  // base for m = 0 with chunk bits 1-2 xor m, plus 1 KB per cb/4; row-major:
  // one base plus 32 bytes per cb.
  auto pv_base0 = [&]() -> uint32_t {
    const int l = lane_id_fresh();
    const int trr = (l & 15) >> 2, trq = l & 3;
    return lds_off<Cfg>(4 * (l >> 4) + trr, trq >> 1) + (trq & 1) * 8;
  };
  // P slots: row h (one head, 64 bytes) holds the head's P in PV k-slot order;
  // 16-byte chunk q (k slots 8q..8q+7) sits at chunk q ^ ((h >> 2) & 3), so the
  // 16 rows read or written by a 16-lane group fall in distinct banks.
  auto p_lane_off = [&]() -> uint32_t {
    const int l = lane_id_fresh();
    const int r = l & 15;
    return static_cast<uint32_t>(r * PROW + (((l >> 4) ^ (r >> 2)) & 3) * 16);
  };
  // Tile loads (blocked): lane l of every 1 KB load fills row l/8 of its block
  // with logical chunk (l%8) ^ (l/8); the per-lane source offset is the same for
  // every block.  Recomputed per tile (see lane_id_fresh) to keep registers free.
  struct LdLane { int r; uint32_t off, fb; };
  auto ld_lane = [&]() -> LdLane {
    const int l = lane_id_fresh();
    const int r = l >> 3;
    const uint32_t c16 = (((l & 7) ^ r) * 16);
    return {r, r * ROWB + c16, c16};   // fb: same chunk of the block's first row
  };

  while (g < gend) {
    const int S = len_of(b_cs, b_qi);
    const int nt = tiles_len(S);
    const int first = t0 + pc;                  // cost position of its first tile
    const int t1 = first + nt;
    const int lt0 = max(g - first, 0), lt1 = min(gend, t1) - first;
    if (lt1 <= lt0) break;                      // the range ends before the sequence's first tile
    const int ntiles = lt1 - lt0;
    // a piece that is a whole sequence writes o_lat / lse itself, unless the
    // caller merges every piece afterwards (o_lat null: merged with the
    // output projection)
    const bool whole = a.o_lat != nullptr && (lt0 == 0) && (lt1 == nt);
    const int32_t* bt = block_table + static_cast<int64_t>(b_cs) * a.max_pages;
    const char* pool = static_cast<const char*>(a.pool);
    const int64_t page_bytes = static_cast<int64_t>(ROWB) << lg;

    // Page ids of the piece's first 64 pages, one per lane, loaded once per
    // piece: the tile loop reads them with v_readlane instead of a scalar
    // memory load (whose latency would stall every tile issue).
    const int pfirst = (lt0 * kTile) >> lg;
    const int pg_lane = pfirst + lane < a.max_pages ? bt[pfirst + lane] : -1;
    auto page_id = [&](int tok) -> int {
      const int rel = (tok >> lg) - pfirst;      // uniform
      return rel < 64 ? __builtin_amdgcn_readlane(pg_lane, rel) : bt[tok >> lg];
    };
    // Rows past the sequence (or on a page id outside the pool) load the same
    // chunk of the tile's first row instead, which is always a valid token.
    auto page_base = [&](int tok) -> const char* {
      const int pg = page_id(tok);
      return (pg >= 0 && pg < a.num_pages) ? pool + pg * page_bytes + (tok & (ps - 1)) * ROWB
                                           : nullptr;
    };
    auto issue_general = [&](int tok0, char* dst_tile) {
      if constexpr (Cfg::SPEC) {
        // loader i copies the tile's 8-row group i (see the fast path)
        if (loader >= 0) {
          const LdLane ll = ld_lane();
          const char* row0 = page_base(tok0);
          const char* fb = row0 ? row0 : pool;
          const int rtok = tok0 + 8 * loader;      // first token of the row group
          const char* rb = rtok >= S ? nullptr
                           : (ps >= kTile || loader < 2) ? row0 + 8 * loader * ROWB : page_base(rtok);
          const bool ok = rb != nullptr && row0 != nullptr && rtok + ll.r < S;
          const char* src = ok ? rb + ll.off : fb + ll.fb;
          const uint32_t dst = lds_addr(dst_tile) + static_cast<uint32_t>(loader) * Cfg::CG * 1024;
#pragma unroll
          for (int k = 0; k < Cfg::CG; ++k) lds_dma16_v(src + k * 128, dst + k * 1024);
        }
        return;
      }
      const LdLane ll = ld_lane();
      const int ld_r = ll.r;
      const uint32_t ld_off = ll.off, ld_fb = ll.fb;
      const char* row0 = page_base(tok0);
      const char* fb = row0 ? row0 : pool;
#pragma unroll
      for (int k = 0; k < Cfg::LD_HI; ++k) {
        const int blk = k * Cfg::LW + loader;        // 1 KB block of the tile this load fills
        if (loader >= 0 && blk < Cfg::INSTR) {
          const char* src;
          if constexpr (Cfg::BLOCKED) {
            const int bi = blk / Cfg::CG, bj = blk - bi * Cfg::CG;
            const int rtok = tok0 + 8 * bi;          // first token of the block's 8 rows
            // a block past the sequence end looks nothing up (its page may not exist)
            const char* rb = rtok >= S ? nullptr
                             : (ps >= kTile || bi < 2) ? row0 + 8 * bi * ROWB : page_base(rtok);
            const bool ok = rb != nullptr && row0 != nullptr && rtok + ld_r < S;
            src = ok ? rb + bj * 128 + ld_off : fb + bj * 128 + ld_fb;
          } else {
            const int pos = blk * 64 + lane_id_fresh();  // chunk position in the row-major tile
            const int t = pos / CPR;
            const int c = pos - t * CPR;
            const char* rb = (ps >= kTile || t < 16) ? row0
                             : (tok0 + 16 < S ? page_base(tok0 + 16) : nullptr);
            const bool ok = rb != nullptr && row0 != nullptr && tok0 + t < S;
            src = ok ? rb + ((ps >= kTile || t < 16) ? t : t - 16) * ROWB + c * 16 : fb + c * 16;
          }
          lds_dma16_v(src, lds_addr(dst_tile + blk * 1024));
        }
      }
    };
    // ---- fp8 cache, specialised layout: the tile stays fp8 in its ring slot.
    // Nope columns: 16 blocks of 1 KB, block 4rg + cg holding rows 8rg .. 8rg
    // + 7 and 16-byte chunks 8cg .. 8cg + 7, chunk c of row t at byte 128(t %
    // 8) + 16((c ^ sw(t)) % 8) with sw(t) = t % 8 ^ 4(t / 16 % 2).  Rope
    // columns: 2 blocks of 16 rows x 4 chunks, chunk c of row t at 64(t % 16) +
    // 16(c ^ (t / 4 % 4)).  Then the 32 fp32 scales.  Every 16-byte K operand
    // read (8 lanes: 8 rows, one chunk) and every 8-bit transpose read of V
    // (16 lanes: 8 rows of one chunk, rows t and t + 16 among them) falls on
    // distinct banks.  Loader i copies column group i of the four row groups,
    // then rope block i (i < 2) or the scales (i = 2): 5, 5, 5 and 4 copies.
    // A row past the sequence (or on a page outside the pool) copies the same
    // chunk of the tile's first row; masked scores take no scale.
    auto issue_f8 = [&](int lt, int buf) {
      if (loader < 0) return;
      const int tok0 = lt * kTile;
      const uint32_t dst = lds_addr(lds + buf * Cfg::SLOT_BYTES);
      const uint8_t* const pool8 = static_cast<const uint8_t*>(a.pool);
      const int64_t pb8 = static_cast<int64_t>(R) << lg;
      const int pg0 = page_id(tok0);
      const bool ok0 = pg0 >= 0 && pg0 < a.num_pages;
      const uint8_t* row0 = ok0 ? pool8 + pg0 * pb8 + (tok0 & (ps - 1)) * R : pool8;
      const int l = lane_id_fresh();
      if (ps >= kTile && tok0 + kTile <= S && ok0) {
        // one contiguous tile: scalar block base + the lane's fixed offset
        const uint32_t ca = 16u * ((l & 7) ^ (l >> 3));
        const uint32_t oa = (l >> 3) * R + ca, ob = (l >> 3) * R + (ca ^ 64u);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          lds_dma16(row0 + 8 * j * R + 128 * loader, j < 2 ? oa : ob, dst + (4 * j + loader) * 1024);
        if (loader < 2) {
          const uint32_t orp = (l >> 2) * R + 512 + 16 * ((l & 3) ^ (l >> 4));
          lds_dma16(row0 + 16 * loader * R, orp, dst + Cfg::F8S_ROPE + loader * 1024);
        } else if (loader == 2 && l < kTile / 4) {
          lds_dma16_v(a.scales + static_cast<int64_t>(pg0) * ps + (tok0 & (ps - 1)) + 4 * l, dst + Cfg::F8S_SCL);
        }
        return;
      }
      // rows 16 .. 31 lie on the next page when pages hold 16 tokens
      const int pg1 = ps >= kTile ? pg0 : (tok0 + 16 < S ? page_id(tok0 + 16) : -1);
      const bool ok1 = pg1 >= 0 && pg1 < a.num_pages;
      auto row_src = [&](int t, int byte) -> const uint8_t* {
        const bool hi = t >= 16;
        const bool ok = ok0 && (hi ? ok1 : true) && tok0 + t < S;
        return ok ? pool8 + (hi ? pg1 : pg0) * pb8 + ((tok0 + t) & (ps - 1)) * R + byte : row0 + byte;
      };
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = 8 * j + (l >> 3);
        const int c = 8 * loader + ((l & 7) ^ (l >> 3) ^ (j < 2 ? 0 : 4));
        lds_dma16_v(row_src(t, 16 * c), dst + (4 * j + loader) * 1024);
      }
      if (loader < 2) {
        const int t = 16 * loader + (l >> 2);
        lds_dma16_v(row_src(t, 512 + 16 * ((l & 3) ^ (l >> 4))), dst + Cfg::F8S_ROPE + loader * 1024);
      } else if (loader == 2 && l < kTile / 4) {
        const int t = 4 * l;                         // tokens t .. t + 3, one page
        const bool hi = t >= 16;
        const bool ok = ok0 && (hi ? ok1 : true) && tok0 + t < S;
        const float* src = ok ? a.scales + static_cast<int64_t>(hi ? pg1 : pg0) * ps + ((tok0 + t) & (ps - 1))
                              : (ok0 ? a.scales + static_cast<int64_t>(pg0) * ps + (tok0 & (ps - 1)) : a.scales);
        lds_dma16_v(src, dst + Cfg::F8S_SCL);
      }
    };
    auto issue_tile = [&](int lt, int buf) {
      if constexpr (Cfg::SPEC8) {
        issue_f8(lt, buf);
        return;
      }
      const int tok0 = lt * kTile;
      char* dst_tile = lds + buf * Cfg::TILE_BYTES;
      if constexpr (Cfg::BLOCKED) {
        // Fast path: a whole tile of valid tokens inside one page is one
        // contiguous run; every load is (scalar block base) + (the lane's fixed
        // offset), with nothing to select per lane.
        if (ps >= kTile && tok0 + kTile <= S) {
          const int pg = page_id(tok0);
          if (pg >= 0 && pg < a.num_pages) {
            const char* tile0 = pool + pg * page_bytes + (tok0 & (ps - 1)) * ROWB;
            const uint32_t ld_off = ld_lane().off;
            if constexpr (Cfg::SPEC) {
              // loader i copies the 8-row group i (9 KB contiguous in the
              // page): blocks 9i .. 9i + 8, source and LDS offsets with
              // constant strides
              static_assert(Cfg::LD_HI == Cfg::CG && Cfg::INSTR == Cfg::LW * Cfg::CG, "one row group per loader");
              if (loader >= 0) {
                const char* src = tile0 + loader * 8 * ROWB;
                const uint32_t dst = lds_addr(dst_tile) + static_cast<uint32_t>(loader) * Cfg::CG * 1024;
#pragma unroll
                for (int k = 0; k < Cfg::CG; ++k) lds_dma16(src + k * 128, ld_off, dst + k * 1024);
              }
              return;
            }
#pragma unroll
            for (int k = 0; k < Cfg::LD_HI; ++k) {
              const int blk = k * Cfg::LW + loader;
              if (loader >= 0 && blk < Cfg::INSTR) {
                const int bi = blk / Cfg::CG, bj = blk - bi * Cfg::CG;
                lds_dma16(tile0 + (8 * bi * ROWB + bj * 128), ld_off, lds_addr(dst_tile + blk * 1024));
              }
            }
            return;
          }
        }
      }
      issue_general(tok0, dst_tile);
    };

    if constexpr (Cfg::SPEC) {
    // ---- Specialised roles.  QK waves (0-3): S^T (32 tokens x 32 heads) as
    // two 16-head groups sharing every K operand read (K tile rows are the A
    // operand from LDS; Q of 32 heads x 576 in 144 VGPRs), softmax, P
    // published to LDS, and O for column blocks [2w, 2w + 2).  PV waves
    // (4-7): O for column blocks [8 + 6(w - 4), +6), and every tile copy.  One
    // barrier per tile as in the general path: step it computes S(it) and
    // PV(it - 1).
    constexpr int QH = 32, NQW = 4, QCB = 2, PCB = 6;
    constexpr int AHEAD = Cfg::NBUF - 2;
    // head blocks computed (HBC), 16-head groups per scoring wave (NG), and
    // the scoring waves' K reads in flight (each feeds NG MFMAs; one group
    // leaves the registers for more)
    static_assert(HBC == 1 || HBC == NW, "head blocks computed: 1 or all");
    constexpr int NG = HBC == 1 ? 1 : 2;
    constexpr int QD = NG == 1 ? 6 : (FP8 ? kQk8Ahead : kQk2Ahead);
    static_assert(NQW * QH == 16 * NW && NQW * QCB + (NW - NQW) * PCB == Cfg::VCB && Cfg::BLOCKED &&
                  Cfg::LW == NW - NQW && Cfg::INSTR % Cfg::LW == 0 && AHEAD >= 1, "specialised shape");
    const bool qkw = wave < NQW;

    auto sync_tile = [&](int it) {
      if (!qkw) {
        const int pending = min(ntiles - 1 - it, AHEAD - 1);
        if constexpr (FP8) {
          if (loader == 3) wait_pending<AHEAD - 1, 4>(pending);
          else wait_pending<AHEAD - 1, 5>(pending);
        } else {
          wait_tiles<AHEAD + 2, Cfg::LD_HI>(pending);
        }
      }
      block_barrier();
    };
    // a score far above the offset anywhere in the workgroup: redo the piece
    // with each head's true maximum as its offset (cannot overflow again)
    auto vote_again = [&](bool overflow) -> bool {
      __syncthreads();                 // P slots are free from here on
      if (threadIdx.x == 0) *vote = 0;
      __syncthreads();
      if (__builtin_amdgcn_ballot_w64(overflow) != 0 && lane == 0) *vote = 1;
      __syncthreads();
      const bool again = *vote != 0;
      __syncthreads();
      return again;
    };
    // O += P . V over all head blocks and column blocks [cbf, cbf + NC): B (V,
    // transpose reads) held for the wave's column blocks while the head
    // blocks' A operands (P rows) stream past, read AD head blocks ahead.
    // fp8: one 8-bit transpose read per column block: source lane 2k + h of
    // group `quad` reads row T = k < 4 ? 4quad + k : 16 + 4quad + k - 4 (the P
    // k-slot order), bytes 8h .. 8h + 7 of chunk cb, and lane l16 receives
    // column 16cb + l16 of the 8 rows; the codes convert exactly to bf16.
    auto pv8_base = [&]() -> uint32_t {
      const int l = lane_id_fresh();
      const int q = l >> 4, k = (l & 15) >> 1, h = l & 1;
      const int t = k < 4 ? 4 * q + k : 16 + 4 * q + k - 4;
      const int sw = (t & 7) ^ (4 * (t >> 4));
      return static_cast<uint32_t>(4096 * (t >> 3) + 128 * (t & 7) + 16 * sw + 8 * h);
    };
    auto pv_cols = [&](const char* tb, int pslot, int cbf, auto& oo) {
      constexpr int NC = sizeof(oo[0]) / sizeof(oo[0][0]);
      bf16x8 vb[NC];
      if constexpr (FP8) {
        const uint32_t pb = pv8_base();
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const int cb = cbf + c;
          // (the chunk xor touches address bits 4-6 only)
          const v2i32 r = lds_read_tr8(tb + ((pb ^ static_cast<uint32_t>(16 * (cb & 7))) + 1024 * (cb >> 3)));
          const uint4 y = {fp8x2_to_bf16x2<false>(static_cast<uint32_t>(r[0])),
                           fp8x2_to_bf16x2<true>(static_cast<uint32_t>(r[0])),
                           fp8x2_to_bf16x2<false>(static_cast<uint32_t>(r[1])),
                           fp8x2_to_bf16x2<true>(static_cast<uint32_t>(r[1]))};
          vb[c] = __builtin_bit_cast(bf16x8, y);
        }
      } else {
        const uint32_t pb = pv_base0();
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const int cb = cbf + c;
          const char* p0 = tb + ((pb ^ static_cast<uint32_t>(32 * (cb & 3))) + 1024 * (cb >> 2));
          const bf16x4 v0 = lds_read_tr16(p0);
          const bf16x4 v1 = lds_read_tr16(p0 + 16 * ROWB);
          vb[c] = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
        }
      }
      const char* pa_base = pbuf + pslot * PSLOT + p_lane_off();
      constexpr int AD = HBC < 3 ? HBC : 3;
      bf16x8 abuf[AD];
#pragma unroll
      for (int i = 0; i < AD; ++i) abuf[i] = *reinterpret_cast<const bf16x8*>(pa_base + i * 16 * PROW);
#pragma unroll
      for (int hb = 0; hb < HBC; ++hb) {
        const bf16x8 pa = abuf[hb % AD];
        if (hb + AD < HBC) abuf[hb % AD] = *reinterpret_cast<const bf16x8*>(pa_base + (hb + AD) * 16 * PROW);
#pragma unroll
        for (int c = 0; c < NC; ++c) oo[hb][c] = mfma16(pa, vb[c], oo[hb][c]);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // normalised O of this wave's column blocks to o_lat (whole sequence) or
    // to the piece's partial slot, both bf16 rows [head][d_c]
    auto store_o = [&](int cbf, auto& oo) {
      constexpr int NC = sizeof(oo[0]) / sizeof(oo[0][0]);
      const int fl = lane_id_fresh();
      const int fq = fl >> 4, f16 = fl & 15;
#pragma unroll
      for (int hb = 0; hb < HBC; ++hb) {
        if (hb < HB) {
          f32x4 scv;
#pragma unroll
          for (int i = 0; i < 4; ++i) scv[i] = inv_share[hb * 16 + 4 * fq + i];
#pragma unroll
          for (int c = 0; c < NC; ++c) oo[hb][c] *= scv;
        }
      }
      // the tile ring is free: the block goes to LDS as bf16 rows of one
      // head, then every thread copies whole rows out with 16-byte stores.
      // Rows are 1040 bytes apart, so the rows of a store's four 16-lane
      // groups (4 rows apart) start 64 bytes apart modulo the 256 bytes of one
      // pass over the banks.
      constexpr int ROWE = DC + 8;                             // elements per staged row
      static_assert(16 * NW * ROWE * 2 <= Cfg::NBUF * Cfg::SLOT_BYTES, "row staging fits the ring");
      uint16_t* const st = reinterpret_cast<uint16_t*>(lds);
      // heads 4fq + i and 4fq + i + 1 of a column rounded as one pair (one
      // conversion instruction), stored as two halves.  The fp8 layout's
      // scoring waves (two column blocks) keep the rounding one value at a
      // time: with the pairs there they reload three spilled registers per
      // tile instead of one.
#pragma unroll
      for (int hb = 0; hb < HBC; ++hb) {
        if (hb < HB) {
          if constexpr (FP8 && NC == QCB) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int h = hb * 16 + 4 * fq + i;
#pragma unroll
              for (int c = 0; c < NC; ++c)
                st[h * ROWE + 16 * (cbf + c) + f16] = f32_to_bf16_bits(oo[hb][c][i]);
            }
          } else {
#pragma unroll
            for (int i = 0; i < 4; i += 2) {
              const int h = hb * 16 + 4 * fq + i;
#pragma unroll
              for (int c = 0; c < NC; ++c) {
                const uint32_t pk = pack_bf16x2(oo[hb][c][i], oo[hb][c][i + 1]);
                st[h * ROWE + 16 * (cbf + c) + f16] = static_cast<uint16_t>(pk);
                st[(h + 1) * ROWE + 16 * (cbf + c) + f16] = static_cast<uint16_t>(pk >> 16);
              }
            }
          }
        }
      }
      __syncthreads();
      uint16_t* const rows = whole ? a.o_lat + static_cast<int64_t>(b) * H * DC
                                   : a.part_o + (static_cast<int64_t>(w) + b) * (HB * 16) * DC;
      uint4* const dst = reinterpret_cast<uint4*>(rows);
      for (int i = threadIdx.x; i < H * (DC / 8); i += Cfg::THREADS) {
        const int h = i / (DC / 8), c8 = i - h * (DC / 8);
        dst[i] = *reinterpret_cast<const uint4*>(st + h * ROWE + 8 * c8);
      }
    };

    if (qkw) {
      const int hq = QH * wave;                   // first head of this wave
      // a wave whose heads are all past the computed blocks only takes part
      // in the barriers and its (empty) share of O
      const bool scores = hq < 16 * HBC;
      // Q of NG 16-head groups g: lane holds head hq + 16g + l16, elements
      // [32kc + 8quad, +8) of chunk kc (bf16 cache), or [64(kc / 2) + 16quad +
      // 8(kc % 2), +8) (fp8 cache: one 16-byte K read feeds chunks kc, kc + 1)
      bf16x8 qg[NG][Cfg::K32];
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const int h = hq + 16 * g + l16;
        const bool hv = h < H;
        const uint16_t* qrow = a.q + (static_cast<int64_t>(b) * H + (hv ? h : 0)) * R;
        const bf16x8 z = {};
#pragma unroll
        for (int kc = 0; kc < Cfg::K32; ++kc) {
          const int e = FP8 ? 64 * (kc >> 1) + 16 * quad + 8 * (kc & 1) : 32 * kc + 8 * quad;
          const bf16x8 v = *reinterpret_cast<const bf16x8*>(qrow + e);
          qg[g][kc] = hv ? v : z;
        }
      }
      f32x4 oo[HBC][QCB];
      float m_use[2] = {-INFINITY, -INFINITY};   // exponent offset per head group (set by the first tile)
      // this lane's largest exponent argument (score . scale_log2 - offset)
      // since the offset was set: the overflow test and, for a recompute, the
      // true maximum, with no cross-lane reduction per tile
      float y_max[2] = {-INFINITY, -INFINITY};
      float l_part[2] = {0.f, 0.f};              // this lane's shares of the denominators
      // S^T (32 tokens x 32 heads) of one tile as four 16x16 accumulator
      // chains (token block x head group): each K operand read (row 16tbk +
      // l16, 16-byte chunk 4kc + quad) feeds the MFMAs of both head groups.
      // Then the softmax of each group and P to slot pslot.  A tile that runs
      // past the sequence end is a separate copy of the body (MASK), so the
      // steady-state tiles carry no masking.
      auto score2 = [&](const char* tb, int tok0, bool set_offset, int pslot) {
        auto body = [&](auto mask_t) {
          constexpr bool MASK = decltype(mask_t)::value;
          f32x4 sacc[NG][2] = {};
          if constexpr (FP8) {
            // 16-byte K reads j = 2m + tbk (row 16tbk + l16, chunk 4m + quad;
            // m = 8 reads the rope chunk quad), each converted exactly into the
            // bf16 A operands of chunks 2m and 2m + 1
            const K8Bases kb = k8_bases();
            auto k_ptr = [&](int j) {
              const int m = j >> 1, tbk = j & 1;
              const uint32_t off = m < 8 ? ((((m & 1) ^ tbk) ? kb.odd : kb.even) + 8192 * tbk + 1024 * (m >> 1))
                                         : Cfg::F8S_ROPE + kb.rope + 1024 * tbk;
              return reinterpret_cast<const uint4*>(tb + off);
            };
            constexpr int NR = Cfg::K32;
            uint4 kbuf[QD];
#pragma unroll
            for (int i = 0; i < QD; ++i) kbuf[i] = *k_ptr(i);
#pragma unroll
            for (int j = 0; j < NR; ++j) {
              const uint4 kv = kbuf[j % QD];
              if (j + QD < NR) kbuf[j % QD] = *k_ptr(j + QD);
              const int m = j >> 1, tbk = j & 1;
              const uint4 c0 = {fp8x2_to_bf16x2<false>(kv.x), fp8x2_to_bf16x2<true>(kv.x),
                                fp8x2_to_bf16x2<false>(kv.y), fp8x2_to_bf16x2<true>(kv.y)};
              const uint4 c1 = {fp8x2_to_bf16x2<false>(kv.z), fp8x2_to_bf16x2<true>(kv.z),
                                fp8x2_to_bf16x2<false>(kv.w), fp8x2_to_bf16x2<true>(kv.w)};
#pragma unroll
              for (int g = 0; g < NG; ++g)
                sacc[g][tbk] = mfma16(__builtin_bit_cast(bf16x8, c0), qg[g][2 * m], sacc[g][tbk]);
#pragma unroll
              for (int g = 0; g < NG; ++g)
                sacc[g][tbk] = mfma16(__builtin_bit_cast(bf16x8, c1), qg[g][2 * m + 1], sacc[g][tbk]);
              __builtin_amdgcn_sched_barrier(0);
            }
          } else {
            const QkBases qb = qk_bases();
            auto a_ptr = [&](int i) {
              const int kc = i >> 1, tbk = i & 1;
              return reinterpret_cast<const bf16x8*>(tb + ((kc & 1) ? qb.odd : qb.even) + tbk * 16 * ROWB +
                                                     1024 * (kc >> 1));
            };
            constexpr int NQ = 2 * Cfg::K32;
            bf16x8 abuf[QD];
#pragma unroll
            for (int i = 0; i < QD; ++i) abuf[i] = *a_ptr(i);
#pragma unroll
            for (int i = 0; i < NQ; ++i) {
              const bf16x8 av = abuf[i % QD];
              if (i + QD < NQ) abuf[i % QD] = *a_ptr(i + QD);
#pragma unroll
              for (int g = 0; g < NG; ++g) sacc[g][i & 1] = mfma16(av, qg[g][i >> 1], sacc[g][i & 1]);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
          // fp8: the score of token t is scale_t (q . code_t), and P carries
          // scale_t into P . V (a masked token's scale, possibly never
          // written, is not used: its P is zero and its scale taken as zero)
          float sc[8];
          if constexpr (FP8) {
            const float* sp = reinterpret_cast<const float*>(tb + Cfg::F8S_SCL) + 4 * quad;
            const f32x4 lo = *reinterpret_cast<const f32x4*>(sp);
            const f32x4 hi = *reinterpret_cast<const f32x4*>(sp + 16);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              sc[i] = (!MASK || tok0 + 4 * quad + i < S) ? lo[i] : 0.f;
              sc[4 + i] = (!MASK || tok0 + 16 + 4 * quad + i < S) ? hi[i] : 0.f;
            }
          }
          const uint32_t poff = p_lane_off();
          // sacc[g][tbk][i] is token 16tbk + 4quad + i of head hq + 16g + l16
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            float x[8];
#pragma unroll
            for (int tbk = 0; tbk < 2; ++tbk)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int t = 16 * tbk + 4 * quad + i;
                const float v = FP8 ? sacc[g][tbk][i] * sc[4 * tbk + i] : sacc[g][tbk][i];
                x[4 * tbk + i] = (!MASK || tok0 + t < S) ? v : -INFINITY;
              }
            if (set_offset) {                       // first tile: O is still zero
              float mt = -INFINITY;
#pragma unroll
              for (int i = 0; i < 8; ++i) mt = fmaxf(mt, x[i]);
              m_use[g] = max_across_half_waves(max_across_quarter_pairs(mt)) * a.scale_log2;
            }
            uint32_t pu[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float y0 = fmaf(x[2 * j], a.scale_log2, -m_use[g]);
              const float y1 = fmaf(x[2 * j + 1], a.scale_log2, -m_use[g]);
              y_max[g] = fmaxf(y_max[g], fmaxf(y0, y1));
              const float p0 = __builtin_amdgcn_exp2f(y0);
              const float p1 = __builtin_amdgcn_exp2f(y1);
              l_part[g] += p0 + p1;
              if constexpr (FP8) pu[j] = pack_bf16x2(p0 * sc[2 * j], p1 * sc[2 * j + 1]);
              else pu[j] = pack_bf16x2(p0, p1);
            }
            // P in PV A-operand order: k slot 8quad + j <-> token (j < 4 ? 4quad + j : 16 + 4quad + j - 4)
            *reinterpret_cast<bf16x8*>(pbuf + pslot * PSLOT + (hq + 16 * g) * PROW + poff) =
                __builtin_bit_cast(bf16x8, pu);
          }
        };
        if (!scores) return;
        if (tok0 + kTile <= S)
          body(std::false_type{});
        else
          body(std::true_type{});
      };

      for (int pass = 0;; ++pass) {
#pragma unroll
        for (int hb = 0; hb < HBC; ++hb)
#pragma unroll
          for (int c = 0; c < QCB; ++c) oo[hb][c] = f32x4{};
        l_part[0] = l_part[1] = 0.f;
        y_max[0] = y_max[1] = -INFINITY;
        sync_tile(0);
        score2(lds, lt0 * kTile, pass == 0, 0);
        for (int it = 1; it < ntiles; ++it) {
          sync_tile(it);
          score2(lds + (it % Cfg::NBUF) * Cfg::SLOT_BYTES, (lt0 + it) * kTile, false, it & 1);
          pv_cols(lds + ((it - 1) % Cfg::NBUF) * Cfg::SLOT_BYTES, (it - 1) & 1, QCB * wave, oo);
        }
        block_barrier();
        pv_cols(lds + ((ntiles - 1) % Cfg::NBUF) * Cfg::SLOT_BYTES, (ntiles - 1) & 1, QCB * wave, oo);
        const bool again = vote_again(y_max[0] > kHeadroom || y_max[1] > kHeadroom);
        if (!again || pass > 0) break;   // the second pass starts at the true maximum
#pragma unroll
        for (int g = 0; g < NG; ++g)
          m_use[g] += max_across_half_waves(max_across_quarter_pairs(y_max[g]));
      }
      // 1/l and lse of this wave's heads (four lanes hold a head)
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const float l_tot = sum_across_half_waves(sum_across_quarter_pairs(l_part[g]));
        const float lse_nat = (m_use[g] + log2f(l_tot)) * kLn2;
        const int h = hq + 16 * g + l16;
        if (quad == 0) {
          inv_share[h] = 1.0f / l_tot;
          if (h < H) {
            if (whole) {
              if (a.lse != nullptr) a.lse[static_cast<int64_t>(b) * H + h] = lse_nat;
            } else {
              a.part_lse[(static_cast<int64_t>(w) + b) * H + h] = lse_nat;
            }
          }
        }
      }
      __syncthreads();
      store_o(QCB * wave, oo);
    } else {
      const int cbf = NQW * QCB + PCB * (wave - NQW);
      f32x4 oo[HBC][PCB];
      for (int pass = 0;; ++pass) {
#pragma unroll
        for (int hb = 0; hb < HBC; ++hb)
#pragma unroll
          for (int c = 0; c < PCB; ++c) oo[hb][c] = f32x4{};
#pragma unroll
        for (int i = 0; i < AHEAD; ++i)
          if (i < ntiles) issue_tile(lt0 + i, i);
        sync_tile(0);
        if (AHEAD < ntiles) issue_tile(lt0 + AHEAD, AHEAD % Cfg::NBUF);
        for (int it = 1; it < ntiles; ++it) {
          sync_tile(it);
          if (it + AHEAD < ntiles) issue_tile(lt0 + it + AHEAD, (it + AHEAD) % Cfg::NBUF);
          pv_cols(lds + ((it - 1) % Cfg::NBUF) * Cfg::SLOT_BYTES, (it - 1) & 1, cbf, oo);
        }
        block_barrier();
        pv_cols(lds + ((ntiles - 1) % Cfg::NBUF) * Cfg::SLOT_BYTES, (ntiles - 1) & 1, cbf, oo);
        const bool again = vote_again(false);
        if (!again || pass > 0) break;
      }
      __syncthreads();
      store_o(cbf, oo);
    }
    } else {
    // query registers (QK waves): lane holds head hbase + l16, elements
    // [32kc + 8*quad, +8)
    bf16x8 qreg[Cfg::K32];
    bf16x8 qtail = {};  // elements [32*K32 + 8*quad, +8) for quad < 2, zero otherwise
    {
      const int h = hbase + l16;
      const bool hv = h < H;
      const uint16_t* qrow = a.q + (static_cast<int64_t>(b) * H + (hv ? h : 0)) * R;
      const bf16x8 z = {};
#pragma unroll
      for (int kc = 0; kc < Cfg::K32; ++kc) {
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(qrow + 32 * kc + 8 * quad);
        qreg[kc] = hv ? v : z;
      }
      if constexpr (Cfg::K16) {
        const bool tv = hv && quad < 2;
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(qrow + 32 * Cfg::K32 + 8 * (quad & 1));
        qtail = tv ? v : z;
      }
    }

    // O of this wave: heads 16hb + 4quad + i (all heads), columns
    // 16(cb0 + c) + l16
    f32x4 o[NW][CPW];
    float m_use = -INFINITY;   // exponent offset for this lane's head (set by the first tile)
    float m_seen = -INFINITY;  // running maximum of this head's scores
    float l_part = 0.f;        // this lane's share of the softmax denominator
    for (int pass = 0;; ++pass) {
#pragma unroll
    for (int hb = 0; hb < NW; ++hb)
#pragma unroll
      for (int c = 0; c < CPW; ++c) o[hb][c] = f32x4{};
    l_part = 0.f;
    bool overflow = false;

    // Software pipeline over tiles: iteration `it` computes S(it) = K(it).Q^T
    // and its softmax (QK waves: 16 heads each), publishes P(it) in P slot it%2,
    // then accumulates PV(it - 1) (every wave: all heads, its own columns; P of
    // the previous tile, V from its still-resident ring slot).  Two ring slots
    // are read per iteration, so AHEAD = NBUF - 2 tiles are in flight; the one
    // barrier per tile both releases a ring slot and publishes P.
    constexpr int AHEAD = Cfg::NBUF - 2;
    static_assert(AHEAD >= 1, "ring too small");
#pragma unroll
    for (int i = 0; i < AHEAD; ++i)
      if (i < ntiles) issue_tile(lt0 + i, i);

    // ---- S^T = K_tile . Q^T.  MFMA i covers chunk kc = i/2 of token block
    // tbk = i%2 (two independent accumulator chains, interleaved).  A operand =
    // row 16tbk + l16, 16-byte chunk 4kc + quad: an even/odd base plus
    // immediates.  Operands are read QD MFMAs ahead through a rotating set of
    // registers; sched_barrier pins the issue order.
    auto qk = [&](const char* tb, f32x4* sacc) {
      sacc[0] = f32x4{};
      sacc[1] = f32x4{};
      constexpr int NQ = 2 * Cfg::K32;
      constexpr int QD = NQ < kQkAhead ? NQ : kQkAhead;
      const QkBases qb = qk_bases();
      auto a_ptr = [&](int i) {
        const int kc = i >> 1, tbk = i & 1;
        return reinterpret_cast<const bf16x8*>(
            tb + ((kc & 1) ? qb.odd : qb.even) + tbk * 16 * ROWB +
            (Cfg::BLOCKED ? 1024 * (kc >> 1) : 64 * (kc & ~1)));
      };
      bf16x8 abuf[QD];
#pragma unroll
      for (int i = 0; i < QD; ++i) abuf[i] = *a_ptr(i);
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
        sacc[i & 1] = mfma16(abuf[i % QD], qreg[i >> 1], sacc[i & 1]);
        if (i + QD < NQ) abuf[i % QD] = *a_ptr(i + QD);
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (Cfg::K16) {
        // the last 16 elements as a 32-wide chunk whose upper half is zero on
        // both operands: one MFMA shape for the whole accumulator chain (a
        // 16x16x16 MFMA reading this accumulator right after a 16x16x32 one
        // has been seen to read stale accumulator registers)
        const bf16x8 z = {};
#pragma unroll
        for (int tbk = 0; tbk < 2; ++tbk) {
          const bf16x8 av = *reinterpret_cast<const bf16x8*>(tb + qb.tail + tbk * 16 * ROWB);
          sacc[tbk] = mfma16(quad < 2 ? av : z, qtail, sacc[tbk]);
        }
      }
    };

    // ---- online softmax of one tile; sacc[tb][i] is token 16tb + 4*quad + i,
    // head l16.  Returns P as the PV A operand: k slot 8*quad + j <-> token
    // (j < 4 ? 4quad + j : 16 + 4quad + j - 4).
    auto softmax = [&](const f32x4* sacc, int tok0, bool set_offset) -> bf16x8 {
      auto xval = [&](int tbk, int i) -> float { return sacc[tbk][i]; };
      float x[8];
      float mt;
      if (tok0 + kTile <= S) {                    // whole tile valid: no mask
#pragma unroll
        for (int tbk = 0; tbk < 2; ++tbk)
#pragma unroll
          for (int i = 0; i < 4; ++i) x[4 * tbk + i] = xval(tbk, i);
        mt = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                   fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
      } else {
        mt = -INFINITY;
#pragma unroll
        for (int tbk = 0; tbk < 2; ++tbk)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = 16 * tbk + 4 * quad + i;
            const float v = (tok0 + t < S) ? xval(tbk, i) : -INFINITY;
            x[4 * tbk + i] = v;
            mt = fmaxf(mt, v);
          }
      }
      // scores are raw dot products here; the base-2 scale is applied once to
      // the maximum and fused into the exponent argument below
      mt = max_across_half_waves(max_across_quarter_pairs(mt)) * a.scale_log2;
      m_seen = fmaxf(m_seen, mt);
      if (set_offset) m_use = mt;                 // first tile: O is still zero
      overflow |= mt > m_use + kHeadroom;
      uint32_t pu[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // v_exp_f32 directly: arguments <= kHeadroom, results below 2^-126 of
        // the maximum may flush to zero
        const float p0 = __builtin_amdgcn_exp2f(fmaf(x[2 * j], a.scale_log2, -m_use));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(x[2 * j + 1], a.scale_log2, -m_use));
        l_part += p0 + p1;
        pu[j] = pack_bf16x2(p0, p1);
      }
      return __builtin_bit_cast(bf16x8, pu);
    };

    auto p_store = [&](int pslot, bf16x8 pa) {
      *reinterpret_cast<bf16x8*>(pbuf + pslot * PSLOT + hbase * PROW + p_lane_off()) = pa;
    };

    // ---- O += P . V_tile over all head blocks and this wave's CPW column
    // blocks.  B (V, transpose reads: source lane 4r+q of group `quad` reads
    // token rows 4*quad + r and 16 + 4*quad + r at channels 16cb + 4q) is held
    // for CG column blocks while the head blocks' A operands (P rows, one
    // 16-byte read each) stream past.
    auto pv = [&](const char* tb, int pslot) {
      // tile buffers are 4 KB aligned, so the xor may be applied after adding
      // the buffer address
      // (blocked: cb0 is a multiple of 4, so the wave's first column block
      // only moves the base by whole 1 KB blocks, which the xor leaves alone)
      const uint32_t pb = pv_base0() + (Cfg::BLOCKED ? 1024 * (cb0 >> 2) : 32 * cb0);
      auto v_read = [&](int c) {                  // column block cb0 + c
        const int imm = Cfg::BLOCKED ? 1024 * (c >> 2) : 32 * c;
        const char* p0 = tb + (Cfg::BLOCKED ? (pb ^ static_cast<uint32_t>(32 * (c & 3))) : pb) + imm;
        const bf16x4 v0 = lds_read_tr16(p0);
        const bf16x4 v1 = lds_read_tr16(p0 + 16 * ROWB);
        return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
      };
      const char* pa_base = pbuf + pslot * PSLOT + p_lane_off();
      constexpr int CG = CPW < 4 ? CPW : 4;
#pragma unroll
      for (int c0 = 0; c0 < CPW; c0 += CG) {
        bf16x8 vb[CG];
#pragma unroll
        for (int c = 0; c < CG; ++c) vb[c] = v_read(c0 + c);
        // every head block, also those past H (never stored): no branches, so
        // the A reads can run AD head blocks ahead
        constexpr int AD = NW < 3 ? NW : 3;
        bf16x8 abuf[AD];
#pragma unroll
        for (int i = 0; i < AD; ++i) abuf[i] = *reinterpret_cast<const bf16x8*>(pa_base + i * 16 * PROW);
#pragma unroll
        for (int hb = 0; hb < NW; ++hb) {
          const bf16x8 pa = abuf[hb % AD];
          if (hb + AD < NW) abuf[hb % AD] = *reinterpret_cast<const bf16x8*>(pa_base + (hb + AD) * 16 * PROW);
#pragma unroll
          for (int c = 0; c < CG; ++c) o[hb][c0 + c] = mfma16(pa, vb[c], o[hb][c0 + c]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };

    // waits for tile it, then issues the loads of tile it + AHEAD into the
    // ring slot the barrier just released
    // The waves of the first half get the matrix core first on their SIMD and
    // would idle at the next barrier; they issue their share of the loads at
    // the end of the step instead (the slot is free from this step's barrier
    // on), while the second half issues right after the barrier.
    const bool late_issue = wave < NW / 2;
    auto wait_and_sync = [&](int it) {
      const int pending = min(ntiles - 1 - it, AHEAD - 1);
      if (hi_loader) wait_tiles<AHEAD + 2, Cfg::LD_HI>(pending);
      else if (lo_loader) wait_tiles<AHEAD + 2, Cfg::LD_LO>(pending);
      else wait_vmcnt<0>();
      block_barrier();
      if (!late_issue && it + AHEAD < ntiles) issue_tile(lt0 + it + AHEAD, (it + AHEAD) % Cfg::NBUF);
    };
    auto late = [&](int it) {
      if (late_issue && it + AHEAD < ntiles) issue_tile(lt0 + it + AHEAD, (it + AHEAD) % Cfg::NBUF);
    };

    // QK + softmax of one tile, P published to its slot (QK waves only)
    auto score_tile = [&](const char* tb, int tok0, bool set_offset, int pslot) {
      if (qk_wave) {
        f32x4 sacc[2];
        qk(tb, sacc);
        p_store(pslot, softmax(sacc, tok0, set_offset));
      }
    };

    // first tile: QK + softmax (sets the exponent offset on the first pass);
    // then each step computes S(it), its softmax and P(it), and PV(it - 1)
    wait_and_sync(0);
    score_tile(lds, lt0 * kTile, pass == 0, 0);
    late(0);
    for (int it = 1; it < ntiles; ++it) {
      wait_and_sync(it);
      score_tile(lds + (it % Cfg::NBUF) * Cfg::TILE_BYTES, (lt0 + it) * kTile, false, it & 1);
      pv(lds + ((it - 1) % Cfg::NBUF) * Cfg::TILE_BYTES, (it - 1) & 1);
      late(it);
    }
    // last tile's PV (its ring slot is not refilled: no later loads)
    block_barrier();
    pv(lds + ((ntiles - 1) % Cfg::NBUF) * Cfg::TILE_BYTES, (ntiles - 1) & 1);

    // a score far above the offset anywhere in the workgroup: redo the piece
    // with each head's true maximum as its offset (cannot overflow again)
    __syncthreads();                 // P slots are free from here on
    if (threadIdx.x == 0) *vote = 0;
    __syncthreads();
    if (__builtin_amdgcn_ballot_w64(overflow) != 0 && lane == 0) *vote = 1;
    __syncthreads();
    const bool again = *vote != 0;
    __syncthreads();
    if (!again || pass > 0) break;   // the second pass starts at the true maximum
    m_use = m_seen;
    }  // pass

    // ---- epilogue: the QK waves publish 1/l of their heads and write the lse;
    // every wave normalises and writes its columns of O
    const float l_tot = sum_across_half_waves(sum_across_quarter_pairs(l_part));
    const float lse_nat = (m_use + log2f(l_tot)) * kLn2;
    const int64_t slot = static_cast<int64_t>(w) + b;
    if (qk_wave && quad == 0) {
      inv_share[hbase + l16] = 1.0f / l_tot;
      if (hbase + l16 < H) {
        if (whole) {
          if (a.lse != nullptr) a.lse[static_cast<int64_t>(b) * H + hbase + l16] = lse_nat;
        } else {
          a.part_lse[slot * H + hbase + l16] = lse_nat;
        }
      }
    }
    __syncthreads();
    // (lane-derived values below come from lane_id_fresh so that none of them
    // is hoisted into a register held across the tile loop)
    const int fl = lane_id_fresh();
    const int fq = fl >> 4, f16 = fl & 15;
#pragma unroll
    for (int hb = 0; hb < NW; ++hb) {
      if (hb < HB) {
        f32x4 scv;
#pragma unroll
        for (int i = 0; i < 4; ++i) scv[i] = inv_share[hb * 16 + 4 * fq + i];
#pragma unroll
        for (int c = 0; c < CPW; ++c) o[hb][c] *= scv;
      }
    }

    {
      // o_lat[b] (whole sequence) or the piece's partial slot, bf16 rows
      // [head][d_c]: lane (quad, l16) writes column 16(cb0 + c) + l16 of heads
      // 16hb + 4quad + i; heads past H get an offset beyond the buffer's
      // range, whose stores the hardware drops
      uint16_t* const rows = whole ? a.o_lat + static_cast<int64_t>(b) * H * DC
                                   : a.part_o + slot * (HB * 16) * DC;
      const auto rs = make_rsrc(rows, H * DC * 2);
#pragma unroll
      for (int hb = 0; hb < NW; ++hb) {
        if (hb < HB) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int h = hb * 16 + 4 * fq + i;
            const uint32_t vo = h < H ? static_cast<uint32_t>(h * DC + 16 * cb0 + f16) * 2 : 0x80000000u;
#pragma unroll
            for (int c = 0; c < CPW; ++c)
              __builtin_amdgcn_raw_buffer_store_b16(static_cast<short>(f32_to_bf16_bits(o[hb][c][i])), rs,
                                                    vo, 32 * c, 0);
          }
        }
      }
    }

    }  // general path

    // next piece: the next non-empty sequence
    g = first + lt1;
    t0 = t1;
    ++b;
    next_query(b_cs, b_qi);
    while (b < B && len_of(b_cs, b_qi) == 0) {
      ++b;
      next_query(b_cs, b_qi);
    }
    // all waves must be done reading the ring and the shared 1/l before the
    // next piece refills them
    __syncthreads();
  }
}

template <int DC, int DR, int NW, bool FP8 = false, int HBC = NW>
hipError_t launch_split(const DecodeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((k_split<DC, DR, NW, FP8, HBC>), dim3(a.num_parts), dim3(64 * NW), 0, s, a,
                     a.plan, a.seq_lens, a.block_table);
  return hipGetLastError();
}

}  // namespace

bool decode_supported(int d_c, int d_rope, int H, bool fp8) {
  if (H < 1 || H > 128) return false;
  if (fp8) return d_c == 512 && d_rope == 64;
  if (d_c == 512 && d_rope == 64) return true;
  if (d_c == 32 && d_rope == 16) return H <= 32;
  return false;
}

// One piece per compute unit of the current device.  The count is cached per
// device in atomics (a racing first query stores the same value).
int decode_auto_parts(int B, int H) {
  (void)B;
  (void)H;
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cus[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < kMaxDevices) {
    const int c = cus[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  if (dev < kMaxDevices) cus[dev].store(n, std::memory_order_relaxed);
  return n;
}

WorkspaceLayout decode_workspace_layout(int B, int H, int d_c, int num_parts) {
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  WorkspaceLayout L;
  L.plan_off = 0;
  L.part_o_off = up(sizeof(int32_t) * (static_cast<size_t>(B) + 3));
  const size_t slots = static_cast<size_t>(num_parts) + B;
  const size_t hpad = (static_cast<size_t>(H) + 15) / 16 * 16;
  L.part_lse_off = L.part_o_off + up(sizeof(uint16_t) * slots * hpad * d_c);
  L.total = L.part_lse_off + up(sizeof(float) * slots * H);
  return L;
}

hipError_t launch_split_phase(const DecodeArgs& a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  hipError_t e = hipSuccess;
  if (ev0 && (e = hipEventRecord(ev0, s)) != hipSuccess) return e;
  // d_c 512: eight waves whatever H (<= 128).  With fewer heads the rows past H
  // carry zero queries and are never stored; the tile stream, not the MFMA
  // work, sets the time at small H, and one or two waves per workgroup could
  // not keep enough copies in flight (V2-Lite, H = 16: 145 us with one wave,
  // against a 9.5 us roofline).
  if (a.d_c == 512 && a.d_rope == 64 && a.fp8) {
    if (a.H <= 16) e = launch_split<512, 64, 8, true, 1>(a, s);
    else e = launch_split<512, 64, 8, true>(a, s);
  } else if (a.fp8) {
    return hipErrorInvalidValue;
  } else if (a.d_c == 512 && a.d_rope == 64) {
    // up to 16 heads: only the first head block is scored and accumulated
    if (a.H <= 16) e = launch_split<512, 64, 8, false, 1>(a, s);
    else e = launch_split<512, 64, 8>(a, s);
  } else if (a.d_c == 32 && a.d_rope == 16) {
    if (a.H <= 16) e = launch_split<32, 16, 1>(a, s);
    else e = launch_split<32, 16, 2>(a, s);
  } else {
    return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  if (ev1 && (e = hipEventRecord(ev1, s)) != hipSuccess) return e;
  return hipSuccess;
}

}  // namespace mla
