// Internal launch interface between the C ABI layer (mla_api.cpp) and the
// kernel translation units.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

// Tokens per decode tile; the split plan and the decode kernel cut work in
// whole tiles.
constexpr int kTile = 32;

// Heads handled by one wave of the decode kernel (16x16 MFMA columns).
constexpr int kHeadsPerWave = 16;

struct AppendArgs {
  int d_c, d_rope, page_size_log2, max_pages, num_pages, num_seqs, n_tokens;
  bool fp8, rope;
  double rope_base;
  const uint16_t* c_kv;
  const uint16_t* k_pe;
  // Instead of c_kv / k_pe: fp32 partial rows part[n_part][n_tokens][d_c +
  // d_rope], summed in order and rounded to bf16 (the down-projection's
  // reduction chunks).  nullptr = read c_kv / k_pe.
  const float* part;
  int n_part;
  const int32_t* positions;
  const int32_t* seq_ids;
  const int32_t* block_table;
  void* pool;
  float* scales;
};

// Split-K down-projection of mla_project_append: part[ks][t][n] = the sum,
// in chunk order, of the fp32 sums over the 256-element chunks
// kDownGroup ks .. kDownGroup ks + kDownGroup - 1 of h[t][k] w_down[n][k].
constexpr int kDownChunk = 256;
constexpr int kDownGroup = 4;                 // chunks per workgroup, summed in order
constexpr int down_groups(int d_model) { return (d_model / kDownChunk + kDownGroup - 1) / kDownGroup; }
struct ProjectArgs {
  int T, N, d_model;         // tokens, outputs (d_c + d_rope), reduction length
  const uint16_t* h;         // bf16 [T][d_model]
  const uint16_t* w_down;    // bf16 [N][d_model]
  float* part;               // fp32 [down_groups(d_model)][T][N]
};

struct AbsorbArgs {
  int B, H, d_c, d_rope, d_nope;
  double rope_base;
  const uint16_t* q_nope;
  const uint16_t* q_pe;
  const int32_t* q_pos;
  const uint16_t* w_uk;
  uint16_t* q_out;
};

struct OutProjArgs {
  int B, H, d_c, d_v;
  const uint16_t* o_lat;
  const uint16_t* w_uv;
  uint16_t* out;
};

// Workspace of mla_decode_paged, carved from the caller's buffer:
//   plan      int32 [B + 1] cost-line prefix sums (tiles, plus pc before
//             each non-empty sequence), then int32 quota and int32 pc
//   part_o    bf16 [num_parts + B][16 ceil(H/16)][d_c]  normalised partial
//             outputs, one row per head
//   part_lse  fp32 [num_parts + B][H]
// A partial computed by workgroup w for sequence b lives in slot w + b.
//
// With q_len > 1 (several new tokens per sequence, scored in one pass), the
// kernels work on B = (cache sequences) x q_len query sequences: query
// sequence v is token i = v % q_len of cache sequence v / q_len, reads that
// sequence's block-table row and sees its first seq_lens[v / q_len] -
// (q_len - 1 - i) tokens (causal among the new tokens).  q_len = 1 is
// single-token decode.
struct DecodeArgs {
  int B, H, d_c, d_rope, page_size_log2, max_pages, num_pages, num_parts, q_len;
  bool fp8;
  float scale_log2;  // softmax_scale * log2(e)
  const uint16_t* q;
  const void* pool;
  const float* scales;
  const int32_t* block_table;
  const int32_t* seq_lens;
  int32_t* plan;
  uint16_t* part_o;
  float* part_lse;
  uint16_t* o_lat;
  float* lse;
};

struct WorkspaceLayout {
  size_t plan_off, part_o_off, part_lse_off, total;
};

WorkspaceLayout decode_workspace_layout(int B, int H, int d_c, int num_parts);

// Size of the device scratch array that mla_decode_paged_noalloc uses as its
// workspace, and its address on the current device (looked up once per
// device; no allocation).
constexpr size_t kNoAllocScratchBytes = size_t{64} << 20;
hipError_t noalloc_scratch(void** ptr);
int decode_auto_parts(int B, int H);

hipError_t launch_append(const AppendArgs& a, hipStream_t s);
hipError_t launch_down(const ProjectArgs& a, hipStream_t s);
hipError_t launch_absorb(const AbsorbArgs& a, hipStream_t s);
// launch_absorb and launch_append (bf16 / fp8 rows from c_kv and k_pe, not
// from partial sums) as one launch
hipError_t launch_absorb_append(const AbsorbArgs& a, const AppendArgs& p, hipStream_t s);
hipError_t launch_out_proj(const OutProjArgs& a, hipStream_t s);
// split kernel (with its plan); `ev0`/`ev1` (may be null) are recorded
// immediately before and after it.  With a.o_lat null every piece, a whole
// sequence included, goes to its partial slot.
hipError_t launch_split_phase(const DecodeArgs& a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1);
// merge of split sequences into a.o_lat / a.lse
hipError_t launch_combine(const DecodeArgs& a, hipStream_t s);
// merge of every sequence (after a split phase with o_lat null) and the
// projection out[b][h] = W_UV[h]^T o_lat[b][h]; writes a.o_lat, a.lse when
// not null
hipError_t launch_combine_proj(const DecodeArgs& a, const uint16_t* w_uv, uint16_t* out, hipStream_t s);
bool combine_proj_supported(int d_c, int d_v);

bool decode_supported(int d_c, int d_rope, int H, bool fp8);
bool absorb_supported(int d_c, int d_nope);
bool out_proj_supported(int d_c, int d_v);

}  // namespace mla
