// C ABI of libmla (declared in include/mla.h): argument validation, workspace
// layout, dispatch to the kernels and status codes.  Every check here runs
// before any HIP call, so invalid host arguments enqueue nothing.
#include "../../include/mla.h"

#include <hip/hip_runtime.h>

#include <cmath>

#include "mla_internal.hpp"
#include "prefill.hpp"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int log2_exact(int v) {
  if (v <= 0 || (v & (v - 1)) != 0) return -1;
  int l = 0;
  while ((1 << l) < v) ++l;
  return l;
}

// Dimension checks shared by all calls.
mla_status_t check_dims(const mla_dims_t* d) {
  if (d == nullptr) return MLA_ERR_INVALID_ARG;
  if (d->n_heads <= 0 || d->d_c <= 0 || d->d_rope <= 0 || d->d_nope <= 0 || d->d_v <= 0 ||
      d->page_size <= 0)
    return MLA_ERR_INVALID_ARG;
  if (d->d_rope % 2 != 0) return MLA_ERR_INVALID_ARG;
  if (d->cache_dtype != MLA_CACHE_BF16 && d->cache_dtype != MLA_CACHE_FP8_E4M3)
    return MLA_ERR_INVALID_ARG;
  if (!std::isfinite(d->rope_base) || d->rope_base <= 0.0) return MLA_ERR_INVALID_ARG;
  if (!std::isfinite(d->softmax_scale) || !(d->softmax_scale > 0.f)) return MLA_ERR_INVALID_ARG;
  const bool v3 = d->d_c == 512 && d->d_rope == 64 && d->d_nope == 128 && d->d_v == 128;
  const bool tiny = d->d_c == 32 && d->d_rope == 16 && d->d_nope == 16 && d->d_v == 16;
  if (!v3 && !tiny) return MLA_ERR_UNSUPPORTED;
  if (d->n_heads > (tiny ? 32 : 128)) return MLA_ERR_UNSUPPORTED;
  const int lg = log2_exact(d->page_size);
  if (lg < 4 || lg > 8) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

thread_local const char* g_last_hip_error = "no HIP error";

mla_status_t from_hip(hipError_t e) {
  if (e == hipSuccess) return MLA_OK;
  g_last_hip_error = hipGetErrorString(e);
  return MLA_ERR_HIP;
}

int effective_parts(int32_t num_splits, int B, int H) {
  return num_splits > 0 ? num_splits : mla::decode_auto_parts(B, H);
}

}  // namespace

extern "C" {

const char* mla_status_string(int32_t s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
  }
  return "MLA_ERR_UNKNOWN";
}

const char* mla_last_hip_error(void) { return g_last_hip_error; }

size_t mla_cache_bytes_per_token(const mla_dims_t* d) {
  if (d == nullptr || d->d_c <= 0 || d->d_rope < 0) return 0;
  const size_t r = static_cast<size_t>(d->d_c) + static_cast<size_t>(d->d_rope);
  if (d->cache_dtype == MLA_CACHE_BF16) return 2 * r;
  if (d->cache_dtype == MLA_CACHE_FP8_E4M3) return r + 4;
  return 0;
}

}  // extern "C"

namespace {

// Argument checks and kernel arguments of mla_append_latent; *empty is set
// when there is nothing to append (then `a` is not filled).
mla_status_t append_args(const mla_dims_t* d, const void* c_kv, const void* k_pe, const int32_t* positions,
                         const int32_t* seq_ids, const int32_t* block_table, int32_t num_seqs,
                         int32_t max_pages, int32_t num_pages, int32_t n_tokens, void* pool, float* scales,
                         uint32_t flags, mla::AppendArgs* a, bool* empty) {
  const mla_status_t st = check_dims(d);
  if (st != MLA_OK) return st;
  if (n_tokens < 0 || num_seqs <= 0 || max_pages <= 0 || num_pages <= 0) return MLA_ERR_INVALID_ARG;
  if ((flags & ~MLA_APPEND_NO_ROPE) != 0) return MLA_ERR_INVALID_ARG;
  *empty = n_tokens == 0;
  if (*empty) return MLA_OK;
  if (!c_kv || !k_pe || !positions || !seq_ids || !block_table || !pool) return MLA_ERR_INVALID_ARG;
  const bool fp8 = d->cache_dtype == MLA_CACHE_FP8_E4M3;
  if (fp8 != (scales != nullptr)) return MLA_ERR_INVALID_ARG;
  if (!aligned(c_kv, 16) || !aligned(k_pe, 4) || !aligned(pool, 16) || !aligned(positions, 4) ||
      !aligned(seq_ids, 4) || !aligned(block_table, 4) || (fp8 && !aligned(scales, 4)))
    return MLA_ERR_INVALID_ARG;
  *a = mla::AppendArgs{};
  a->d_c = d->d_c;
  a->d_rope = d->d_rope;
  a->page_size_log2 = log2_exact(d->page_size);
  a->max_pages = max_pages;
  a->num_pages = num_pages;
  a->num_seqs = num_seqs;
  a->n_tokens = n_tokens;
  a->fp8 = fp8;
  a->rope = (flags & MLA_APPEND_NO_ROPE) == 0;
  a->rope_base = d->rope_base;
  a->c_kv = static_cast<const uint16_t*>(c_kv);
  a->k_pe = static_cast<const uint16_t*>(k_pe);
  a->positions = positions;
  a->seq_ids = seq_ids;
  a->block_table = block_table;
  a->pool = pool;
  a->scales = scales;
  return MLA_OK;
}

// Argument checks and kernel arguments of mla_absorb_q.
mla_status_t absorb_args(const mla_dims_t* d, const void* q_nope, const void* q_pe, const int32_t* q_pos,
                         const void* w_uk, int32_t B, void* q_out, mla::AbsorbArgs* a) {
  const mla_status_t st = check_dims(d);
  if (st != MLA_OK) return st;
  if (B <= 0) return MLA_ERR_INVALID_ARG;
  if (!q_nope || !q_pe || !q_pos || !w_uk || !q_out) return MLA_ERR_INVALID_ARG;
  if (!aligned(q_nope, 16) || !aligned(q_pe, 4) || !aligned(q_pos, 4) || !aligned(w_uk, 16) ||
      !aligned(q_out, 16))
    return MLA_ERR_INVALID_ARG;
  if (!mla::absorb_supported(d->d_c, d->d_nope)) return MLA_ERR_UNSUPPORTED;
  *a = mla::AbsorbArgs{};
  a->B = B;
  a->H = d->n_heads;
  a->d_c = d->d_c;
  a->d_rope = d->d_rope;
  a->d_nope = d->d_nope;
  a->rope_base = d->rope_base;
  a->q_nope = static_cast<const uint16_t*>(q_nope);
  a->q_pe = static_cast<const uint16_t*>(q_pe);
  a->q_pos = q_pos;
  a->w_uk = static_cast<const uint16_t*>(w_uk);
  a->q_out = static_cast<uint16_t*>(q_out);
  return MLA_OK;
}

}  // namespace

extern "C" {

mla_status_t mla_append_latent(const mla_dims_t* d, const void* c_kv, const void* k_pe,
                               const int32_t* positions, const int32_t* seq_ids,
                               const int32_t* block_table, int32_t num_seqs, int32_t max_pages,
                               int32_t num_pages, int32_t n_tokens, void* pool, float* scales,
                               uint32_t flags, void* stream) {
  mla::AppendArgs a;
  bool empty = false;
  const mla_status_t st = append_args(d, c_kv, k_pe, positions, seq_ids, block_table, num_seqs, max_pages,
                                      num_pages, n_tokens, pool, scales, flags, &a, &empty);
  if (st != MLA_OK || empty) return st;
  return from_hip(mla::launch_append(a, static_cast<hipStream_t>(stream)));
}

mla_status_t mla_append_absorb(const mla_dims_t* d, const void* c_kv, const void* k_pe,
                               const int32_t* positions, const int32_t* seq_ids,
                               const int32_t* block_table, int32_t num_seqs, int32_t max_pages,
                               int32_t num_pages, int32_t n_tokens, void* pool, float* scales,
                               uint32_t flags, const void* q_nope, const void* q_pe, const int32_t* q_pos,
                               const void* w_uk, int32_t B, void* q_out, void* stream) {
  mla::AppendArgs p;
  bool empty = false;
  mla_status_t st = append_args(d, c_kv, k_pe, positions, seq_ids, block_table, num_seqs, max_pages,
                                num_pages, n_tokens, pool, scales, flags, &p, &empty);
  if (st != MLA_OK) return st;
  mla::AbsorbArgs a;
  st = absorb_args(d, q_nope, q_pe, q_pos, w_uk, B, q_out, &a);
  if (st != MLA_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (empty) return from_hip(mla::launch_absorb(a, s));
  return from_hip(mla::launch_absorb_append(a, p, s));
}

namespace {
bool project_supported(const mla_dims_t* d, int32_t d_model) {
  return (d->d_c + d->d_rope) % 32 == 0 && d_model > 0 && d_model % mla::kDownChunk == 0 &&
         d_model <= (1 << 16);
}
size_t project_ws_bytes(const mla_dims_t* d, int32_t d_model, int32_t n_tokens) {
  return sizeof(float) * static_cast<size_t>(mla::down_groups(d_model)) * static_cast<size_t>(n_tokens) *
         static_cast<size_t>(d->d_c + d->d_rope);
}
}  // namespace

size_t mla_project_append_workspace_size(const mla_dims_t* d, int32_t d_model, int32_t n_tokens) {
  if (check_dims(d) != MLA_OK || n_tokens < 0 || !project_supported(d, d_model)) return 0;
  return project_ws_bytes(d, d_model, n_tokens);
}

mla_status_t mla_project_append(const mla_dims_t* d, int32_t d_model, const void* h, const void* w_down,
                                const int32_t* positions, const int32_t* seq_ids,
                                const int32_t* block_table, int32_t num_seqs, int32_t max_pages,
                                int32_t num_pages, int32_t n_tokens, void* pool, float* scales,
                                void* workspace, size_t ws_bytes, void* stream) {
  const mla_status_t st = check_dims(d);
  if (st != MLA_OK) return st;
  if (n_tokens < 0 || num_seqs <= 0 || max_pages <= 0 || num_pages <= 0 || d_model <= 0)
    return MLA_ERR_INVALID_ARG;
  if (!project_supported(d, d_model)) return MLA_ERR_UNSUPPORTED;
  if (n_tokens == 0) return MLA_OK;
  if (!h || !w_down || !positions || !seq_ids || !block_table || !pool || !workspace)
    return MLA_ERR_INVALID_ARG;
  const bool fp8 = d->cache_dtype == MLA_CACHE_FP8_E4M3;
  if (fp8 != (scales != nullptr)) return MLA_ERR_INVALID_ARG;
  if (!aligned(h, 16) || !aligned(w_down, 16) || !aligned(pool, 16) || !aligned(positions, 4) ||
      !aligned(seq_ids, 4) || !aligned(block_table, 4) || !aligned(workspace, 256) ||
      (fp8 && !aligned(scales, 4)))
    return MLA_ERR_INVALID_ARG;
  if (ws_bytes < project_ws_bytes(d, d_model, n_tokens)) return MLA_ERR_WORKSPACE;
  mla::ProjectArgs p{};
  p.T = n_tokens;
  p.N = d->d_c + d->d_rope;
  p.d_model = d_model;
  p.h = static_cast<const uint16_t*>(h);
  p.w_down = static_cast<const uint16_t*>(w_down);
  p.part = static_cast<float*>(workspace);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = mla::launch_down(p, s);
  if (e != hipSuccess) return from_hip(e);
  mla::AppendArgs a{};
  a.d_c = d->d_c;
  a.d_rope = d->d_rope;
  a.page_size_log2 = log2_exact(d->page_size);
  a.max_pages = max_pages;
  a.num_pages = num_pages;
  a.num_seqs = num_seqs;
  a.n_tokens = n_tokens;
  a.fp8 = fp8;
  a.rope = true;
  a.rope_base = d->rope_base;
  a.part = p.part;
  a.n_part = mla::down_groups(d_model);
  a.positions = positions;
  a.seq_ids = seq_ids;
  a.block_table = block_table;
  a.pool = pool;
  a.scales = scales;
  return from_hip(mla::launch_append(a, s));
}

mla_status_t mla_absorb_q(const mla_dims_t* d, const void* q_nope, const void* q_pe,
                          const int32_t* q_pos, const void* w_uk, int32_t B, void* q_out,
                          void* stream) {
  mla::AbsorbArgs a;
  const mla_status_t st = absorb_args(d, q_nope, q_pe, q_pos, w_uk, B, q_out, &a);
  if (st != MLA_OK) return st;
  return from_hip(mla::launch_absorb(a, static_cast<hipStream_t>(stream)));
}

size_t mla_decode_workspace_size(const mla_dims_t* d, int32_t B, int32_t num_splits) {
  if (check_dims(d) != MLA_OK || B <= 0 || num_splits < 0) return 0;
  if (!mla::decode_supported(d->d_c, d->d_rope, d->n_heads, d->cache_dtype == MLA_CACHE_FP8_E4M3)) return 0;
  const int parts = effective_parts(num_splits, B, d->n_heads);
  return mla::decode_workspace_layout(B, d->n_heads, d->d_c, parts).total;
}

namespace {

// Both decode entry points: q_len new tokens per cache sequence (1 = plain
// decode), run as B * q_len query sequences.
mla_status_t decode_impl(const mla_dims_t* d, const void* q, const void* pool, const float* scales,
                         const int32_t* block_table, int32_t max_pages, int32_t num_pages,
                         const int32_t* seq_lens, int32_t B, int32_t q_len, int32_t num_splits,
                         void* workspace, size_t ws_bytes, void* o_lat, float* lse, const void* w_uv,
                         void* out, hipEvent_t e0, hipEvent_t e1, void* stream, bool use_scratch = false) {
  const mla_status_t st = check_dims(d);
  if (st != MLA_OK) return st;
  if (B <= 0 || max_pages <= 0 || num_pages <= 0 || num_splits < 0) return MLA_ERR_INVALID_ARG;
  if (q_len < 1 || q_len > MLA_MAX_Q_LEN || static_cast<int64_t>(B) * q_len > (int64_t{1} << 24))
    return MLA_ERR_INVALID_ARG;
  // with `out`, the merge kernel also applies W_UV and o_lat is optional
  const bool proj = out != nullptr;
  if (!q || !pool || !block_table || !seq_lens || (!use_scratch && !workspace) || (!proj && !o_lat) ||
      (proj && !w_uv))
    return MLA_ERR_INVALID_ARG;
  const bool fp8 = d->cache_dtype == MLA_CACHE_FP8_E4M3;
  if (fp8 != (scales != nullptr)) return MLA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(pool, 16) || !aligned(block_table, 4) || !aligned(seq_lens, 4) ||
      (!use_scratch && !aligned(workspace, 256)) || (o_lat && !aligned(o_lat, 16)) ||
      (lse && !aligned(lse, 4)) || (fp8 && !aligned(scales, 16)) || (proj && !aligned(w_uv, 16)) ||
      (proj && !aligned(out, 16)))
    return MLA_ERR_INVALID_ARG;
  if (!mla::decode_supported(d->d_c, d->d_rope, d->n_heads, fp8)) return MLA_ERR_UNSUPPORTED;
  if (proj && !mla::combine_proj_supported(d->d_c, d->d_v)) return MLA_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(max_pages) * d->page_size > (int64_t{1} << 30)) return MLA_ERR_UNSUPPORTED;
  const int BQ = B * q_len;                     // query sequences
  const int parts = effective_parts(num_splits, BQ, d->n_heads);
  const mla::WorkspaceLayout L = mla::decode_workspace_layout(BQ, d->n_heads, d->d_c, parts);
  if (use_scratch) {
    // the library's device scratch: sizes beyond it are refused before any
    // HIP call; then its address on the current device
    if (L.total > mla::kNoAllocScratchBytes) return MLA_ERR_WORKSPACE;
    const hipError_t e = mla::noalloc_scratch(&workspace);
    if (e != hipSuccess) return from_hip(e);
    ws_bytes = mla::kNoAllocScratchBytes;
  }
  if (ws_bytes < L.total) return MLA_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  mla::DecodeArgs a{};
  a.B = BQ;
  a.q_len = q_len;
  a.H = d->n_heads;
  a.d_c = d->d_c;
  a.d_rope = d->d_rope;
  a.page_size_log2 = log2_exact(d->page_size);
  a.max_pages = max_pages;
  a.num_pages = num_pages;
  a.num_parts = parts;
  a.fp8 = fp8;
  a.scale_log2 = static_cast<float>(static_cast<double>(d->softmax_scale) * 1.4426950408889634);
  a.q = static_cast<const uint16_t*>(q);
  a.pool = pool;
  a.scales = scales;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.plan = reinterpret_cast<int32_t*>(ws + L.plan_off);
  a.part_o = reinterpret_cast<uint16_t*>(ws + L.part_o_off);
  a.part_lse = reinterpret_cast<float*>(ws + L.part_lse_off);
  // the split kernel writes whole sequences to o_lat itself only without the
  // projection; with it every piece goes to the workspace
  a.o_lat = proj ? nullptr : static_cast<uint16_t*>(o_lat);
  a.lse = proj ? nullptr : lse;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = mla::launch_split_phase(a, s, e0, e1);
  if (e != hipSuccess) return from_hip(e);
  if (proj) {
    a.o_lat = static_cast<uint16_t*>(o_lat);
    a.lse = lse;
    e = mla::launch_combine_proj(a, static_cast<const uint16_t*>(w_uv), static_cast<uint16_t*>(out), s);
  } else {
    e = mla::launch_combine(a, s);
  }
  return from_hip(e);
}

}  // namespace

mla_status_t mla_decode_paged(const mla_dims_t* d, const void* q, const void* pool,
                              const float* scales, const int32_t* block_table, int32_t max_pages,
                              int32_t num_pages, const int32_t* seq_lens, int32_t B,
                              int32_t num_splits, void* workspace, size_t ws_bytes, void* o_lat,
                              float* lse, void* stream) {
  return decode_impl(d, q, pool, scales, block_table, max_pages, num_pages, seq_lens, B, 1, num_splits,
                     workspace, ws_bytes, o_lat, lse, nullptr, nullptr, nullptr, nullptr, stream);
}

mla_status_t mla_decode_paged_multi(const mla_dims_t* d, const void* q, const void* pool,
                                    const float* scales, const int32_t* block_table, int32_t max_pages,
                                    int32_t num_pages, const int32_t* seq_lens, int32_t B, int32_t q_len,
                                    int32_t num_splits, void* workspace, size_t ws_bytes, void* o_lat,
                                    float* lse, void* stream) {
  return decode_impl(d, q, pool, scales, block_table, max_pages, num_pages, seq_lens, B, q_len,
                     num_splits, workspace, ws_bytes, o_lat, lse, nullptr, nullptr, nullptr, nullptr, stream);
}

mla_status_t mla_decode_paged_noalloc(const mla_dims_t* d, const void* q, const void* pool,
                                      const float* scales, const int32_t* block_table, int32_t max_pages,
                                      int32_t num_pages, const int32_t* seq_lens, int32_t B, int32_t q_len,
                                      int32_t num_splits, void* o_lat, float* lse, void* stream) {
  return decode_impl(d, q, pool, scales, block_table, max_pages, num_pages, seq_lens, B, q_len,
                     num_splits, nullptr, 0, o_lat, lse, nullptr, nullptr, nullptr, nullptr, stream, true);
}

size_t mla_decode_noalloc_max_bytes(void) { return mla::kNoAllocScratchBytes; }

mla_status_t mla_decode_paged_timed(const mla_dims_t* d, const void* q, const void* pool,
                                    const float* scales, const int32_t* block_table, int32_t max_pages,
                                    int32_t num_pages, const int32_t* seq_lens, int32_t B, int32_t q_len,
                                    int32_t num_splits, void* workspace, size_t ws_bytes, void* o_lat,
                                    float* lse, void* ev_start, void* ev_stop, void* stream) {
  return decode_impl(d, q, pool, scales, block_table, max_pages, num_pages, seq_lens, B, q_len,
                     num_splits, workspace, ws_bytes, o_lat, lse, nullptr, nullptr,
                     static_cast<hipEvent_t>(ev_start), static_cast<hipEvent_t>(ev_stop), stream);
}

mla_status_t mla_decode_paged_out(const mla_dims_t* d, const void* q, const void* pool,
                                  const float* scales, const int32_t* block_table, int32_t max_pages,
                                  int32_t num_pages, const int32_t* seq_lens, int32_t B, int32_t q_len,
                                  int32_t num_splits, const void* w_uv, void* workspace, size_t ws_bytes,
                                  void* out, void* o_lat, float* lse, void* ev_start, void* ev_stop,
                                  void* stream) {
  if (out == nullptr) return MLA_ERR_INVALID_ARG;
  return decode_impl(d, q, pool, scales, block_table, max_pages, num_pages, seq_lens, B, q_len,
                     num_splits, workspace, ws_bytes, o_lat, lse, w_uv, out,
                     static_cast<hipEvent_t>(ev_start), static_cast<hipEvent_t>(ev_stop), stream);
}

size_t mla_prefill_workspace_size(const mla_dims_t* d, int32_t B, int32_t max_pages) {
  if (check_dims(d) != MLA_OK || B <= 0 || max_pages <= 0) return 0;
  if (!mla::prefill_supported(d->d_c, d->d_rope, d->d_nope, d->d_v)) return 0;
  const int64_t s_cap = static_cast<int64_t>(max_pages) * d->page_size;
  if (s_cap > (int64_t{1} << 24)) return 0;
  return mla::prefill_workspace_bytes(B, d->n_heads, s_cap);
}

}  // extern "C"

namespace {

mla_status_t prefill_impl(const mla_dims_t* d, const void* q_nope, const void* q_pe, const int32_t* q_start,
                          int32_t T, int32_t max_q_len, const void* pool, const float* scales,
                          const int32_t* block_table, int32_t max_pages, int32_t num_pages,
                          const int32_t* seq_lens, int32_t B, const void* w_uk, const void* w_uv,
                          void* workspace, size_t ws_bytes, void* out, float* lse, hipEvent_t e0,
                          hipEvent_t e1, void* stream) {
  const mla_status_t st = check_dims(d);
  if (st != MLA_OK) return st;
  if (T < 0 || max_q_len < 0 || B <= 0 || max_pages <= 0 || num_pages <= 0) return MLA_ERR_INVALID_ARG;
  if (!mla::prefill_supported(d->d_c, d->d_rope, d->d_nope, d->d_v)) return MLA_ERR_UNSUPPORTED;
  const bool fp8 = d->cache_dtype == MLA_CACHE_FP8_E4M3;
  const int64_t s_cap = static_cast<int64_t>(max_pages) * d->page_size;
  if (s_cap > (int64_t{1} << 24)) return MLA_ERR_UNSUPPORTED;
  if (B > 65535 || max_q_len > (1 << 24) ||
      (static_cast<int64_t>(B) * d->n_heads + 7) / 8 * 8 * ((max_q_len + mla::kPfQTile - 1) / mla::kPfQTile) >
          0x7fffffff)
    return MLA_ERR_UNSUPPORTED;
  if (fp8 != (scales != nullptr)) return MLA_ERR_INVALID_ARG;
  if (T == 0 || max_q_len == 0) return MLA_OK;
  if (!q_nope || !q_pe || !q_start || !pool || !block_table || !seq_lens || !w_uk || !w_uv ||
      !workspace || !out)
    return MLA_ERR_INVALID_ARG;
  if (!aligned(q_nope, 16) || !aligned(q_pe, 16) || !aligned(q_start, 4) || !aligned(pool, 16) ||
      !aligned(block_table, 4) || !aligned(seq_lens, 4) || !aligned(w_uk, 16) || !aligned(w_uv, 16) ||
      !aligned(workspace, 256) || !aligned(out, 16) || (lse && !aligned(lse, 4)) ||
      (fp8 && !aligned(scales, 4)))
    return MLA_ERR_INVALID_ARG;
  const size_t need = mla::prefill_workspace_bytes(B, d->n_heads, s_cap);
  if (ws_bytes < need) return MLA_ERR_WORKSPACE;
  mla::PrefillArgs a{};
  a.B = B;
  a.H = d->n_heads;
  a.T = T;
  a.page_size_log2 = log2_exact(d->page_size);
  a.max_pages = max_pages;
  a.num_pages = num_pages;
  a.s_cap = static_cast<int>(s_cap);
  a.s_pad = static_cast<int>(mla::prefill_s_pad(s_cap));
  a.max_q_len = max_q_len;
  a.q_tiles = (max_q_len + mla::kPfQTile - 1) / mla::kPfQTile;
  a.scale_log2 = static_cast<float>(static_cast<double>(d->softmax_scale) * 1.4426950408889634);
  for (int i = 0; i < mla::kPfDr / 2; ++i)
    a.rope_theta[i] = std::pow(d->rope_base, -2.0 * i / static_cast<double>(mla::kPfDr));
  a.q_nope = static_cast<const uint16_t*>(q_nope);
  a.q_pe = static_cast<const uint16_t*>(q_pe);
  a.q_start = q_start;
  a.pool = pool;
  a.scales = scales;
  a.fp8 = fp8;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.w_uk = static_cast<const uint16_t*>(w_uk);
  a.w_uv = static_cast<const uint16_t*>(w_uv);
  char* ws = static_cast<char*>(workspace);
  const size_t kv = mla::prefill_kv_bytes(B, d->n_heads, s_cap);
  a.kn = reinterpret_cast<uint16_t*>(ws);
  a.vt = reinterpret_cast<uint16_t*>(ws + kv);
  a.kr = reinterpret_cast<uint16_t*>(ws + 2 * kv);
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  return from_hip(mla::launch_prefill(a, static_cast<hipStream_t>(stream), nullptr, nullptr, e0, e1));
}

}  // namespace

extern "C" {

mla_status_t mla_prefill_paged(const mla_dims_t* d, const void* q_nope, const void* q_pe,
                               const int32_t* q_start, int32_t T, int32_t max_q_len, const void* pool,
                               const float* scales, const int32_t* block_table, int32_t max_pages,
                               int32_t num_pages, const int32_t* seq_lens, int32_t B, const void* w_uk,
                               const void* w_uv, void* workspace, size_t ws_bytes, void* out, float* lse,
                               void* stream) {
  return prefill_impl(d, q_nope, q_pe, q_start, T, max_q_len, pool, scales, block_table, max_pages, num_pages,
                      seq_lens, B, w_uk, w_uv, workspace, ws_bytes, out, lse, nullptr, nullptr, stream);
}

mla_status_t mla_prefill_paged_timed(const mla_dims_t* d, const void* q_nope, const void* q_pe,
                                     const int32_t* q_start, int32_t T, int32_t max_q_len, const void* pool,
                                     const float* scales, const int32_t* block_table, int32_t max_pages,
                                     int32_t num_pages, const int32_t* seq_lens, int32_t B, const void* w_uk,
                                     const void* w_uv, void* workspace, size_t ws_bytes, void* out, float* lse,
                                     void* ev_start, void* ev_stop, void* stream) {
  return prefill_impl(d, q_nope, q_pe, q_start, T, max_q_len, pool, scales, block_table, max_pages, num_pages,
                      seq_lens, B, w_uk, w_uv, workspace, ws_bytes, out, lse, static_cast<hipEvent_t>(ev_start),
                      static_cast<hipEvent_t>(ev_stop), stream);
}



mla_status_t mla_out_proj(const mla_dims_t* d, const void* o_lat, const void* w_uv, int32_t B,
                          void* out, void* stream) {
  const mla_status_t st = check_dims(d);
  if (st != MLA_OK) return st;
  if (B <= 0) return MLA_ERR_INVALID_ARG;
  if (!o_lat || !w_uv || !out) return MLA_ERR_INVALID_ARG;
  if (!aligned(o_lat, 16) || !aligned(w_uv, 16) || !aligned(out, 16)) return MLA_ERR_INVALID_ARG;
  if (!mla::out_proj_supported(d->d_c, d->d_v)) return MLA_ERR_UNSUPPORTED;
  mla::OutProjArgs a{};
  a.B = B;
  a.H = d->n_heads;
  a.d_c = d->d_c;
  a.d_v = d->d_v;
  a.o_lat = static_cast<const uint16_t*>(o_lat);
  a.w_uv = static_cast<const uint16_t*>(w_uv);
  a.out = static_cast<uint16_t*>(out);
  return from_hip(mla::launch_out_proj(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
