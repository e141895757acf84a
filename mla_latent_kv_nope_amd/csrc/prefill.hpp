// Internal launch interface of the explicit-form prefill (mla_prefill_paged).
// Arguments arrive here already validated by the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

// Built for the DeepSeek-V2/V3 head shape only: latent 512, RoPE part 64,
// per-head nope key and value width 128.
constexpr int kPfDc = 512, kPfDr = 64, kPfDh = 128;
constexpr int kPfRow = kPfDc + kPfDr;       // cached row width (elements)
constexpr int kPfQTile = 128;               // new tokens per attention workgroup
constexpr int kPfKTile = 32;                // keys per attention tile
constexpr int kUpTokens = 1024;             // tokens per up-projection workgroup

struct PrefillArgs {
  int B, H, T, page_size_log2, max_pages, num_pages;
  int s_cap;          // max_pages * page_size: tokens a block-table row can address
  int s_pad;          // s_cap rounded up to a whole key tile: workspace token stride
  int max_q_len;      // new tokens computed per sequence (the first max_q_len)
  int q_tiles;        // ceil(max_q_len / kPfQTile)
  float scale_log2;   // softmax_scale * log2(e)
  double rope_theta[kPfDr / 2];   // RoPE angle per position of pair i: base^(-2i / d_rope)
  const uint16_t* q_nope;      // [T][H][128]
  const uint16_t* q_pe;        // [T][H][64], un-rotated
  const int32_t* q_start;      // [B + 1]
  const void* pool;            // [num_pages][page_size][576] bf16, or E4M3 codes
  const float* scales;         // [num_pages][page_size] (fp8 cache), else nullptr
  bool fp8;
  const int32_t* block_table;  // [B][max_pages]
  const int32_t* seq_lens;     // [B]
  const uint16_t* w_uk;        // [H][512][128]
  const uint16_t* w_uv;        // [H][512][128]
  uint16_t* kn;                // workspace [B][H][s_pad][128]: K_nope = C . W_UK[h]
  uint16_t* vt;                // workspace [B][H][s_pad / 32][128][32]: V^T per 32-token tile, V = C . W_UV[h]
  uint16_t* kr;                // workspace [B][s_pad][64]: the rotated RoPE keys, bf16
  uint16_t* out;               // [T][H][128]
  float* lse;                  // [T][H] or nullptr
};

bool prefill_supported(int d_c, int d_rope, int d_nope, int d_v);
// Workspace bytes (kn, vt, then kr, each 256-byte aligned) for B sequences
// whose block-table rows address s_cap tokens; prefill_kv_bytes is the size
// of each of kn and vt (the offsets of vt and kr).
size_t prefill_workspace_bytes(int B, int H, int64_t s_cap);
size_t prefill_kv_bytes(int B, int H, int64_t s_cap);
int64_t prefill_s_pad(int64_t s_cap);
// Launches the up-projection and the attention kernel on stream s.  Optional
// event pairs bracket each of the two kernels (nullptr: none).
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s, hipEvent_t up0, hipEvent_t up1,
                          hipEvent_t at0, hipEvent_t at1);

}  // namespace mla
