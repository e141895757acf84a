/*
 * mla.h - C ABI of libmla: Multi-head Latent Attention (MLA) decode with the
 * up-projections absorbed, over a paged latent cache, for AMD MI355X (gfx950).
 *
 * The method (as stated on the source pages):
 *   - Only the low-rank joint latent c_kv (width d_c) of each token is cached;
 *     per-head K and V are what c_kv becomes through the up-projections W_UK
 *     and W_UV.  ("DeepSeek-V2拆解：MLA与MoE如何把KV缓存压降93.3%",
 *     sheratonhq.com, section 2.1.)
 *   - W_UK can be absorbed on the query side and W_UV on the output side, so K
 *     and V are never materialised (same page, section 2.1; "LLM推理优化的新范式：
 *     从内存墙到计算墙的跨越", zskr.cn, section 2.2: reordering by associativity).
 *   - Position information travels in a separate decoupled-RoPE branch
 *     (sheratonhq.com section 2.1; zskr.cn section 2.1): a d_rope-wide rotated
 *     key shared by all heads, and a per-head rotated query part.
 *   - The new token's latent is appended to the cache before attention reads it
 *     (sheratonhq.com section 2.1, the compression sketch appends then returns).
 *   - The cache is paged with a block size (fsdata.site "DeepSeek V3 MLA",
 *     section 3.1: block_size=16, PagedAttention adapted to the latent space)
 *     and may be stored in fp8 (zskr.cn section 5; fsdata.site section 3.1).
 *
 * Conventions used by every call:
 *   - All array pointers are DEVICE pointers to dense row-major buffers owned
 *     by the caller; shapes are given as [dim0][dim1]...  bf16 means the
 *     16-bit bfloat16 format.  The library keeps no pointer after a call.
 *   - Each call only enqueues kernels on `stream` (a hipStream_t; NULL = the
 *     default stream).  It never synchronises and never allocates device
 *     memory (mla_decode_paged takes a caller-provided workspace).
 *   - Host-visible arguments are validated before anything is enqueued; a
 *     failed check returns MLA_ERR_INVALID_ARG / MLA_ERR_UNSUPPORTED /
 *     MLA_ERR_WORKSPACE and enqueues nothing.  A failed launch returns
 *     MLA_ERR_HIP.  No C++ exception crosses the ABI.
 *   - Values that live on the device (seq_lens, block-table entries,
 *     positions, seq_ids) are not checked on the host.  Kernels treat
 *     out-of-range values defensively instead of faulting: a page id outside
 *     [0, num_pages) is never dereferenced (the append skips the token, as it
 *     does a position beyond the block table; the attention kernels read a
 *     row inside the pool in its place) and seq_lens are clamped to
 *     [0, max_pages * page_size].  Results for the sequences concerned are
 *     unspecified; other sequences of the call are unaffected.
 *   - Outputs must not alias inputs.  Calls on different streams that write
 *     the same buffers race.
 *
 * Cached row layout (one per token, per layer): elements [0, d_c) hold c_kv,
 * elements [d_c, d_c + d_rope) hold k_pe already rotated at the token's
 * position.  Pool: [num_pages][page_size][d_c + d_rope] of bf16, or of uint8
 * E4M3FN codes plus a scale array [num_pages][page_size] of fp32.  Token t of
 * sequence b lives in row (block_table[b][t / page_size], t % page_size).
 *
 * RoPE (a reading; the pages only name the decoupled branch): RoFormer's
 * rotation of consecutive pairs (2i, 2i+1) by angle pos * rope_base^(-2i/d_rope);
 * the angle and its sine and cosine are evaluated in fp64.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1,   /* null pointer, non-positive size, misalignment, bad flag */
  MLA_ERR_UNSUPPORTED = 2,   /* dimensions outside the compiled instantiations */
  MLA_ERR_WORKSPACE = 3,     /* workspace smaller than mla_decode_workspace_size() */
  MLA_ERR_HIP = 4            /* a HIP launch or runtime call failed */
} mla_status_t;

typedef enum {
  MLA_CACHE_BF16 = 0,        /* bf16 rows */
  MLA_CACHE_FP8_E4M3 = 1     /* OCP E4M3FN codes + one fp32 scale per token */
} mla_cache_dtype_t;

/* Model dimensions, passed by pointer to every call (40 bytes, no padding).
 * Supported: (d_c, d_rope, d_nope, d_v) in {(512, 64, 128, 128), (32, 16, 16, 16)};
 * 1 <= n_heads <= 128; page_size a power of two in [16, 256]. */
typedef struct {
  int32_t n_heads;           /* H: query heads */
  int32_t d_c;               /* latent width (c_kv) */
  int32_t d_rope;            /* decoupled RoPE width (q_pe, k_pe); even */
  int32_t d_nope;            /* per-head non-positional query/key width */
  int32_t d_v;               /* per-head value width */
  int32_t page_size;         /* tokens per cache page */
  int32_t cache_dtype;       /* mla_cache_dtype_t */
  float softmax_scale;       /* > 0; multiplies the whole score, e.g. 1/sqrt(d_nope + d_rope) */
  double rope_base;          /* RoPE base, e.g. 10000 */
} mla_dims_t;

/* Append flag: store k_pe as given (no rotation).  Used to test placement. */
#define MLA_APPEND_NO_ROPE 1u

/*
 * mla_append_latent - write n_tokens new latent rows into the paged cache.
 * Source: the cache keeps only the latent, appended token by token before use
 * (sheratonhq.com section 2.1); the RoPE key is computed once per token in its
 * own branch (same section), so it is rotated here and stored rotated.
 *
 *   c_kv        bf16 [n_tokens][d_c]
 *   k_pe        bf16 [n_tokens][d_rope], un-rotated
 *   positions   int32 [n_tokens]: position of each token in its sequence; it
 *               selects the slot and is the RoPE position
 *   seq_ids     int32 [n_tokens]: row of block_table owning each token
 *   block_table int32 [num_seqs][max_pages]
 *   num_pages   pages in the pool
 *   pool        bf16 or uint8 [num_pages][page_size][d_c + d_rope] (written)
 *   scales      fp32 [num_pages][page_size] (fp8 cache only, else NULL; written)
 *   flags       0 or MLA_APPEND_NO_ROPE
 * Each row is (c_kv || RoPE(k_pe, position)) rounded to bf16.  For the fp8
 * cache the row is formed in fp32 (the rotation rounded from fp64 to fp32),
 * scale = absmax(row) / 448 (an fp32 division), and each code is the E4M3FN
 * value nearest to row[i] / scale (ties to even, clamped to +-448); a row of
 * zeros stores scale 0 and zero codes.  Two tokens that map to the same slot
 * race.  n_tokens == 0 is a no-op.
 */
mla_status_t mla_append_latent(const mla_dims_t* dims, const void* c_kv, const void* k_pe,
                               const int32_t* positions, const int32_t* seq_ids,
                               const int32_t* block_table, int32_t num_seqs, int32_t max_pages,
                               int32_t num_pages, int32_t n_tokens, void* pool, float* scales,
                               uint32_t flags, void* stream);

/*
 * mla_project_append - down-project new tokens' hidden states into latent
 * rows and append them: mla_append_latent of c_kv = bf16(W_DKV . h) and
 * k_pe = bf16(W_KR . h).
 * Source: the cached latent is the down-projection of the hidden state, and
 * only it is appended to the cache (sheratonhq.com section 2.1, the
 * down_proj = nn.Linear(d_model, kv_rank) sketch); the RoPE key is projected
 * in its own decoupled branch (same section); d_model = 7168 for DeepSeek-V3
 * (zskr.cn section 2.1).
 *
 *   d_model     hidden width, a positive multiple of 256 (<= 65536)
 *   h           bf16 [n_tokens][d_model]
 *   w_down      bf16 [d_c + d_rope][d_model] (nn.Linear layout): rows
 *               [0, d_c) are W_DKV, rows [d_c, d_c + d_rope) are W_KR
 *   workspace   device buffer of at least mla_project_append_workspace_size()
 *               bytes, 256-byte aligned (fp32 partial sums; no initialisation)
 *   other arguments as for mla_append_latent (RoPE always applied)
 * Each output is accumulated in fp32 (in 256-element chunks of d_model; the
 * chunk sums are added in order within runs of four chunks, and the run sums
 * in order) and rounded once to bf16; the row is then stored
 * exactly as mla_append_latent stores it.  Supported when d_c + d_rope is a
 * multiple of 32 (else MLA_ERR_UNSUPPORTED).  n_tokens == 0 is a no-op.
 */
size_t mla_project_append_workspace_size(const mla_dims_t* dims, int32_t d_model, int32_t n_tokens);
mla_status_t mla_project_append(const mla_dims_t* dims, int32_t d_model, const void* h,
                                const void* w_down, const int32_t* positions,
                                const int32_t* seq_ids, const int32_t* block_table,
                                int32_t num_seqs, int32_t max_pages, int32_t num_pages,
                                int32_t n_tokens, void* pool, float* scales, void* workspace,
                                size_t ws_bytes, void* stream);

/*
 * mla_prefill_workspace_size - bytes of device workspace mla_prefill_paged
 * needs for B sequences whose block-table rows hold max_pages pages: the
 * per-head K_nope and V of every addressable token and the shared RoPE keys,
 * bf16: with P = round_up(max_pages * page_size, 32), two 256-byte aligned
 * blocks of B * n_heads * 128 * P * 2 bytes and one of B * 64 * P * 2 bytes.
 * Returns 0 for unsupported dims, B <= 0, max_pages <= 0 or
 * max_pages * page_size > 2^24.
 */
size_t mla_prefill_workspace_size(const mla_dims_t* dims, int32_t B, int32_t max_pages);

/*
 * mla_prefill_paged - causal attention of a chunk of new tokens per sequence,
 * in the explicit form.
 * Source: reordering by associativity raises decode's arithmetic intensity
 * but lowers prefill's (zskr.cn section 2.2, the per-stage table), so prefill
 * materialises K_h = C . W_UK[h] and V_h = C . W_UV[h] from the cached latent
 * (sheratonhq.com section 2.1) and runs dense attention; long prompts are
 * processed in chunks (the vLLM deployment page, chunked prefill).
 *
 * The chunk's tokens must already be in the cache (mla_append_latent).  The
 * n_b = q_start[b + 1] - q_start[b] new tokens of sequence b are its last n_b
 * cached tokens: new token i sits at position seq_lens[b] - n_b + i and
 * attends to the cached tokens at positions <= its own (a new token at a
 * negative position sees nothing: out = 0, lse = -inf).
 *
 *   q_nope      bf16 [T][H][d_nope]; rows [q_start[b], q_start[b + 1]) are
 *               sequence b's new tokens in order
 *   q_pe        bf16 [T][H][d_rope], un-rotated (rotated here at the token's
 *               position)
 *   q_start     int32 [B + 1] (device): non-decreasing row offsets
 *   max_q_len   host bound on n_b: only the first max_q_len new tokens of a
 *               longer chunk are computed (the others are neither read nor
 *               written; positions still follow from n_b)
 *   pool, scales, block_table, max_pages, num_pages, seq_lens: as for
 *               mla_decode_paged (an fp8 cache is dequantised as code * scale
 *               rounded to bf16, as in decode)
 *   w_uk, w_uv  bf16 [H][d_c][d_nope] and [H][d_c][d_v]
 *   workspace   >= mla_prefill_workspace_size() bytes, 256-byte aligned (no
 *               initialisation; every call rebuilds it)
 *   out         bf16 [T][H][d_v] (written): sum_t p_t V_h[t]
 *   lse         fp32 [T][H] natural-log normaliser of the scores, or NULL
 * with s_t = softmax_scale * (q_nope . K_h[t] + RoPE(q_pe) . k_rot[t]).
 * K and V are rounded to bf16 in the workspace, scores and the softmax are
 * fp32, P is rounded to bf16 for the P.V product.  Supported for d_c 512,
 * d_rope 64 and d_nope = d_v = 128, B <= 65535, max_q_len <= 2^24 and
 * max_pages * page_size <= 2^24 (else MLA_ERR_UNSUPPORTED); MLA_ERR_WORKSPACE
 * when ws_bytes is too small, MLA_ERR_INVALID_ARG for NULL or misaligned
 * pointers (16 bytes for the bf16 arrays and the pool) or scales given for a
 * bf16 cache / missing for an fp8 one, all before anything is enqueued.
 * Rows outside [0, T) are neither read nor written.  T == 0 or
 * max_q_len == 0 is a no-op.
 */
mla_status_t mla_prefill_paged(const mla_dims_t* dims, const void* q_nope, const void* q_pe,
                               const int32_t* q_start, int32_t T, int32_t max_q_len,
                               const void* pool, const float* scales, const int32_t* block_table,
                               int32_t max_pages, int32_t num_pages, const int32_t* seq_lens, int32_t B,
                               const void* w_uk, const void* w_uv, void* workspace,
                               size_t ws_bytes, void* out, float* lse, void* stream);

/*
 * mla_absorb_q - fold W_UK into the query and rotate the RoPE query part.
 * Source: W_UK is absorbed into the query projection (sheratonhq.com section
 * 2.1); the reordered path multiplies Q by the up-projection weight before
 * scoring against the compressed cache (zskr.cn sections 2.1-2.2, and the
 * fused Q x W_DK kernel named in section 4.2).
 *
 *   q_nope  bf16 [B][H][d_nope]
 *   q_pe    bf16 [B][H][d_rope], un-rotated
 *   q_pos   int32 [B]: query position (the last cached position, seq_len - 1)
 *   w_uk    bf16 [H][d_c][d_nope]: K_h = C . W_UK[h]
 *   q_out   bf16 [B][H][d_c + d_rope] (written):
 *             q_out[b][h][0:d_c]   = W_UK[h] . q_nope[b][h]   (fp32 accumulate)
 *             q_out[b][h][d_c:]    = RoPE(q_pe[b][h], q_pos[b])
 */
mla_status_t mla_absorb_q(const mla_dims_t* dims, const void* q_nope, const void* q_pe,
                          const int32_t* q_pos, const void* w_uk, int32_t B, void* q_out,
                          void* stream);

/*
 * mla_append_absorb - mla_append_latent and mla_absorb_q of one decode step in
 * a single launch: the append's workgroups (one wave per new token) run after
 * the absorption's, in its tail, instead of as a kernel of their own.
 * Source: the step appends the new latent rows before attending
 * (sheratonhq.com section 2.1) and absorbs W_UK into the query (same section;
 * zskr.cn sections 2.2 and 4.2, the fused Q x W_DK kernel); kernel fusion
 * against launch and memory round trips (zskr.cn section 4.2).
 *
 * Arguments c_kv .. flags as for mla_append_latent, q_nope .. q_out as for
 * mla_absorb_q; both sets are checked as those calls check them (the first
 * failing check's status is returned, nothing is enqueued then).  Results are
 * those of mla_append_latent followed by mla_absorb_q: the two write disjoint
 * memory (pool rows and scales; q_out) and read nothing the other writes, so
 * their order does not matter.  n_tokens = 0 only absorbs.
 */
mla_status_t mla_append_absorb(const mla_dims_t* dims, const void* c_kv, const void* k_pe,
                               const int32_t* positions, const int32_t* seq_ids,
                               const int32_t* block_table, int32_t num_seqs, int32_t max_pages,
                               int32_t num_pages, int32_t n_tokens, void* pool, float* scales,
                               uint32_t flags, const void* q_nope, const void* q_pe,
                               const int32_t* q_pos, const void* w_uk, int32_t B, void* q_out,
                               void* stream);

/*
 * mla_decode_workspace_size - bytes of device workspace mla_decode_paged needs
 * for this batch size and split count (num_splits as in mla_decode_paged).
 * Returns 0 for unsupported dims or B <= 0.
 */
size_t mla_decode_workspace_size(const mla_dims_t* dims, int32_t B, int32_t num_splits);

/*
 * mla_decode_paged - single-query softmax attention of every head over its
 * sequence's cached latent rows; the latent is used as V.
 * Source: the core of MLA decode in the absorbed form (sheratonhq.com section
 * 2.1; zskr.cn section 2.2); bandwidth-bound on reading the latent cache
 * (fsdata.site section 6, decode bandwidth should approach the peak).
 *
 *   q           bf16 [B][H][d_c + d_rope] from mla_absorb_q
 *   pool        cache as written by mla_append_latent; scales for fp8 else NULL
 *   block_table int32 [B][max_pages]
 *   seq_lens    int32 [B]: tokens of each sequence (0 allowed)
 *   num_splits  number of equal shares the batch is cut into, each processed
 *               by one workgroup (a share may span sequences, a sequence may
 *               span shares); shares are equal in 32-token tiles, plus a
 *               fixed cost of 4 tiles per sequence start when the sequences'
 *               tile counts differ; 0 = automatic (fills the GPU)
 *   workspace   device buffer of at least mla_decode_workspace_size() bytes,
 *               256-byte aligned; contents need no initialisation
 *   o_lat       bf16 [B][H][d_c] (written): sum_t p_t c_kv[t]
 *   lse         fp32 [B][H] natural-log normaliser of the scores, or NULL
 * with s_t = softmax_scale * (q[b][h] . row_t) over t < seq_lens[b] and
 * p = softmax(s).  A sequence of length 0 yields o_lat = 0 and lse = -inf.
 * Results differ between split counts only by floating-point rounding.
 * fp8 cache (d_c = 512, d_rope = 64 only, else MLA_ERR_UNSUPPORTED): row_t is
 * the dequantised row code * scale[t] (zskr.cn section 5, mixed-precision
 * FP8 cache; fsdata.site section 3.1).  The codes enter the products exactly
 * (every e4m3 value is a bf16 value) and the token's scale multiplies its
 * score q . code_t and its softmax weight (p_t * scale[t], rounded to bf16 for
 * the P . V product).
 */
mla_status_t mla_decode_paged(const mla_dims_t* dims, const void* q, const void* pool,
                              const float* scales, const int32_t* block_table, int32_t max_pages,
                              int32_t num_pages, const int32_t* seq_lens, int32_t B,
                              int32_t num_splits, void* workspace, size_t ws_bytes, void* o_lat,
                              float* lse, void* stream);

/* Largest q_len mla_decode_paged_multi accepts. */
#define MLA_MAX_Q_LEN 16

/*
 * mla_decode_paged_multi - mla_decode_paged for q_len new tokens per sequence
 * in one pass, each attending causally: the verification pass of speculative
 * decoding with multi-token-prediction drafts.
 * Source: draft tokens from the multi-token-prediction layers are verified by
 * the main model in one parallel pass (deepseek.csdn.net section 6;
 * agent.csdn.net section 5.3, item 3); each query is the absorbed MLA decode
 * query above.  Reading: the q_len new tokens are already appended, as the
 * last q_len tokens of each sequence, and new token i (0-based) sees the
 * context and new tokens 0..i.
 *
 *   q           bf16 [B][q_len][H][d_c + d_rope] from mla_absorb_q called on
 *               B * q_len rows with positions seq_lens[b] - q_len + i
 *   q_len       1 .. MLA_MAX_Q_LEN (1 is exactly mla_decode_paged)
 *   seq_lens    int32 [B]: tokens of each sequence including its q_len new
 *               ones; new token i sees its first seq_lens[b] - (q_len - 1 - i)
 *               tokens (none if that is <= 0: o_lat = 0, lse = -inf)
 *   workspace   at least mla_decode_workspace_size(dims, B * q_len, num_splits)
 *               bytes
 *   o_lat       bf16 [B][q_len][H][d_c] (written), lse fp32 [B][q_len][H] or NULL
 * Other arguments, errors and results as for mla_decode_paged; q_len outside
 * 1 .. MLA_MAX_Q_LEN is MLA_ERR_INVALID_ARG.  The workgroups of the q_len
 * new tokens of a sequence are placed side by side on one XCD, where their
 * reads of the same pages can share that XCD's L2.
 */
mla_status_t mla_decode_paged_multi(const mla_dims_t* dims, const void* q, const void* pool,
                                    const float* scales, const int32_t* block_table,
                                    int32_t max_pages, int32_t num_pages, const int32_t* seq_lens,
                                    int32_t B, int32_t q_len, int32_t num_splits, void* workspace,
                                    size_t ws_bytes, void* o_lat, float* lse, void* stream);

/*
 * mla_decode_paged_out - mla_decode_paged_multi and mla_out_proj in one call:
 * the kernel that merges the split pieces also applies W_UV, with the merged
 * latent rows of a head still on chip, so o_lat never has to be written and
 * read back (d_c = 512, d_v = 128 only, else MLA_ERR_UNSUPPORTED).
 * Source: W_UV absorbed on the output side (sheratonhq.com section 2.1);
 * operators fused to save memory round trips (agent.csdn.net section 2.3;
 * zskr.cn section 4.2).
 *
 *   w_uv        bf16 [H][d_c][d_v], as for mla_out_proj
 *   out         bf16 [B][q_len][H][d_v] (written): W_UV[h]^T . o_lat[b][i][h]
 *   o_lat       bf16 [B][q_len][H][d_c] written when not NULL
 *   lse         fp32 [B][q_len][H] written when not NULL
 *   ev_start, ev_stop  caller-owned HIP events (hipEvent_t) recorded
 *               immediately before and after the split attention kernel, or
 *               NULL (for measurements)
 * Other arguments, the workspace size (mla_decode_workspace_size(dims,
 * B * q_len, num_splits)) and errors as for mla_decode_paged_multi; out NULL
 * or w_uv NULL is MLA_ERR_INVALID_ARG.  o_lat and lse are bit-equal to those
 * of mla_decode_paged_multi on the same inputs and split count; out is the
 * projection of that bf16 o_lat with fp32 accumulation (it may differ from
 * mla_out_proj's result in the order of the fp32 additions).
 */
mla_status_t mla_decode_paged_out(const mla_dims_t* dims, const void* q, const void* pool,
                                  const float* scales, const int32_t* block_table,
                                  int32_t max_pages, int32_t num_pages, const int32_t* seq_lens,
                                  int32_t B, int32_t q_len, int32_t num_splits, const void* w_uv,
                                  void* workspace, size_t ws_bytes, void* out, void* o_lat,
                                  float* lse, void* ev_start, void* ev_stop, void* stream);

/*
 * mla_out_proj - apply W_UV on the output side.
 * Source: W_UV is absorbed into the output projection (sheratonhq.com section 2.1).
 *
 *   o_lat  bf16 [B][H][d_c]
 *   w_uv   bf16 [H][d_c][d_v]: V_h = C . W_UV[h]
 *   out    bf16 [B][H][d_v] (written): out[b][h] = W_UV[h]^T . o_lat[b][h] (fp32 accumulate)
 */
mla_status_t mla_out_proj(const mla_dims_t* dims, const void* o_lat, const void* w_uv, int32_t B,
                          void* out, void* stream);

/*
 * mla_cache_bytes_per_token - bytes one token occupies in one layer's cache:
 * 2 (d_c + d_rope) for bf16, (d_c + d_rope) + 4 for fp8 plus its scale.
 * Source: MHA caches 2 n_h d_h elements per token per layer, MLA only the
 * latent (sheratonhq.com sections 2.1 and 4.2); here plus the RoPE key.
 * Returns 0 for a NULL or invalid dims.
 */
size_t mla_cache_bytes_per_token(const mla_dims_t* dims);

/* Human-readable name of a status code (static storage); any value is
 * accepted (an int, so that a code outside the enumeration is not an invalid
 * enum value), unknown ones give "MLA_ERR_UNKNOWN". */
const char* mla_status_string(int32_t status);

/* Description of the HIP error behind the calling thread's most recent
 * MLA_ERR_HIP (static storage; "no HIP error" if there was none). */
const char* mla_last_hip_error(void);

/*
 * mla_decode_paged_noalloc - mla_decode_paged_multi without a caller
 * workspace, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).
 * The workspace is a device array inside the library of
 * mla_decode_noalloc_max_bytes() = 64 MiB, present on every device the
 * library is loaded on until the process ends; the call allocates nothing
 * (it looks the array's address up once per device).  Calls whose
 * mla_decode_workspace_size(dims, B * q_len, num_splits) exceeds it return
 * MLA_ERR_WORKSPACE before anything is enqueued (with 128 heads and
 * automatic splits on 256 compute units: B * q_len up to 254).
 * All calls on one device share the array: calls that may overlap on one
 * device (different streams, several threads) race and must not be issued;
 * every call writes the parts of the array it reads first, so nothing needs
 * clearing between calls.  Arguments, other errors and results as for
 * mla_decode_paged_multi.
 */
mla_status_t mla_decode_paged_noalloc(const mla_dims_t* dims, const void* q, const void* pool,
                                      const float* scales, const int32_t* block_table,
                                      int32_t max_pages, int32_t num_pages, const int32_t* seq_lens,
                                      int32_t B, int32_t q_len, int32_t num_splits, void* o_lat,
                                      float* lse, void* stream);
/* Bytes of the device array mla_decode_paged_noalloc uses as workspace. */
size_t mla_decode_noalloc_max_bytes(void);

/*
 * mla_decode_paged_timed, mla_prefill_paged_timed - mla_decode_paged_multi and
 * mla_prefill_paged with two caller-owned HIP events (hipEvent_t values
 * created by the caller, or NULL) recorded on `stream` immediately before and
 * after the call's main kernel: the split attention of decode, the attention
 * kernel of prefill.  For measurements; arguments, errors and results are
 * otherwise those of the plain calls, and nothing is kept between calls.  A
 * failing event record returns MLA_ERR_HIP.
 */
mla_status_t mla_decode_paged_timed(const mla_dims_t* dims, const void* q, const void* pool,
                                    const float* scales, const int32_t* block_table,
                                    int32_t max_pages, int32_t num_pages, const int32_t* seq_lens,
                                    int32_t B, int32_t q_len, int32_t num_splits, void* workspace,
                                    size_t ws_bytes, void* o_lat, float* lse, void* ev_start,
                                    void* ev_stop, void* stream);
mla_status_t mla_prefill_paged_timed(const mla_dims_t* dims, const void* q_nope, const void* q_pe,
                                     const int32_t* q_start, int32_t T, int32_t max_q_len,
                                     const void* pool, const float* scales, const int32_t* block_table,
                                     int32_t max_pages, int32_t num_pages, const int32_t* seq_lens,
                                     int32_t B, const void* w_uk, const void* w_uv, void* workspace,
                                     size_t ws_bytes, void* out, float* lse, void* ev_start,
                                     void* ev_stop, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
