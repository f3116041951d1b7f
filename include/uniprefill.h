/*
 * uniprefill.h - C ABI of the packed, chunked prefill operator for MI355X
 * (gfx950): causal attention over a continuously batched packed prefill with
 * fused block-importance mass, block scores, top-p block selection and
 * compaction of the kept tokens.
 *
 * Sources of the operations (web pages; no code exists on them):
 *  - UniPrefill paper entry (chatpaper), abstract: a token-level prefill
 *    accelerator packaged as a continuous-batching operator.
 *  - UniPrefill review, "Key Terms & Definitions" (Top-p Token Selection) and
 *    "Method & Key Results": the input is split into token blocks, an
 *    importance per block is estimated at a full-attention layer, the fewest
 *    blocks whose cumulative importance reaches p are kept, and the dropped
 *    tokens skip all later sublayers.
 *  - Ultralytics glossary "Chunked Prefill", "How chunked prefill works": a
 *    prompt fed in pieces gives each piece's queries the keys and values
 *    stored by the pieces before it together with the piece's own, masked by
 *    position so that no query sees a later token; "Related serving
 *    techniques": the KV cache lives in fixed-size pages.
 *  - Prepacking summary, "Technical framework" / "Key design": prompts are
 *    concatenated into one sequence with a block-diagonal attention mask and
 *    per-prompt positions.
 *
 * The pages give no importance formula.  This library's definition: the
 * importance of key block b of a segment is the softmax probability mass
 * that the rows of the segment's last query block put on b, summed over all
 * query heads and those rows, normalised over the segment's blocks; the
 * first and last blocks are always kept and count toward p.
 *
 * Conventions for every call
 *  - All pointers are device pointers unless marked (host).
 *  - The caller allocates everything: inputs, outputs (sized to the
 *    capacities named below), KV caches and workspaces.  The library
 *    allocates and frees no memory and keeps no device state.
 *  - Every call is asynchronous on ``stream`` (a hipStream_t; NULL = the
 *    null stream) and never synchronises, except the debug aid
 *    up_check_batch (and up_prefill_attn with UP_DEBUG_CHECKS set).
 *  - Arguments are validated on the host before any launch; on failure the
 *    call returns a negative status, launches nothing, writes no output and
 *    sets the text returned by up_last_error() for the calling thread.  A
 *    failed launch returns UP_ERR_DEVICE.
 *  - Device-side preconditions are the caller's: cu_seqlens non-decreasing
 *    with every segment holding >= 1 token, cu_seqlens[S] <= T, positions
 *    strictly increasing inside a segment and >= that segment's ctx_len,
 *    page ids in [0, num_pages), num_pages * Hkv < 2^27 (cache rows are
 *    addressed with 32-bit indices), slots in range, cu_blocks consistent
 *    with cu_seqlens and block_size.
 *  - The library is thread-safe; its only global state is the thread-local
 *    error text.
 */
#ifndef UNIPREFILL_H
#define UNIPREFILL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int up_status;
#define UP_OK 0
#define UP_ERR_INVALID (-1)     /* bad argument (null pointer, size, range)      */
#define UP_ERR_UNSUPPORTED (-2) /* valid but not built (head dim, block size...) */
#define UP_ERR_WORKSPACE (-3)   /* workspace smaller than the size query says    */
#define UP_ERR_DEVICE (-4)      /* a HIP launch failed; text has hipGetErrorString */

/* Element type of q, k, v, the caches and out.  A plain integer rather than
 * an enum, so that any value a caller passes is well defined and can be
 * refused (UP_ERR_UNSUPPORTED). */
typedef int32_t up_dtype;
#define UP_F32 0
#define UP_BF16 1

/* Text describing the last non-OK status returned on this thread. */
const char* up_last_error(void);
/* Library version string, e.g. "uniprefill 0.1 gfx950". */
const char* up_version(void);

/*
 * One packed batch (one engine step).  Segment s owns packed rows
 * [cu_seqlens[s], cu_seqlens[s+1]); it continues a prompt that already has
 * ctx_lens[s] tokens in the paged KV cache (0 for a fresh prompt).  Cached
 * token i of segment s has position i and lives at page
 * block_table[s * max_pages + i / page_size], offset i % page_size.  The
 * segment's own token t has position positions[t] and its K/V go to slot
 * slot_mapping[t] = page * page_size + offset.
 */
typedef struct up_batch {
  int32_t num_seqs;             /* (host) S >= 1; every segment holds >= 1 token (a
                                   device precondition, checked by up_check_batch)     */
  int32_t num_tokens;           /* (host) T: row capacity of the packed arrays; the
                                   tokens in use are cu_seqlens[S] <= T (device value)   */
  const int32_t* cu_seqlens;    /* [S+1], cu_seqlens[0] = 0                              */
  const int32_t* ctx_lens;      /* [S] cached tokens before each segment                */
  const int32_t* positions;     /* [T] per-prompt positions (gapped after compaction)   */
  const int32_t* slot_mapping;  /* [T] KV slot of each token, >= 0                       */
  const int32_t* block_table;   /* [S, max_pages] page ids; may be NULL if every
                                   ctx_len is 0                                          */
  int32_t max_pages;            /* (host) row length of block_table                      */
  int32_t page_size;            /* (host) tokens per page; must be 16                    */
} up_batch;

/*
 * Scoring scope (score_scope arguments below).
 *  UP_SCOPE_SEGMENT: a scored segment's blocks are its own tokens, counted
 *    from its first one; cached keys enter the softmax normaliser only.
 *  UP_SCOPE_PROMPT: whole-prompt scoring for the final chunk of a chunked
 *    prompt (review, Method & Key Results: importance per block of the
 *    input; glossary, How chunked prefill works: a chunk sees the cached
 *    keys of the earlier chunks): a scored segment's blocks are those of its
 *    whole prompt, the ctx_len cached tokens first, so cached blocks are
 *    scored and selected too.  Needs ctx_lens and a block table; device
 *    precondition: ctx_lens[s] of every scored segment a multiple of
 *    block_size (so the prompt's last block is the segment's last block).
 *    Unscored segments keep their own blocks.  Built for UP_BF16.
 */
#define UP_SCOPE_SEGMENT 0
#define UP_SCOPE_PROMPT 1

/*
 * Block offsets: cu_blocks[s+1] - cu_blocks[s] = ceil((o_s + n_s) /
 * block_size), cu_blocks[0] = 0, where o_s = ctx_lens[s] for a scored
 * segment (score_flags[s] != 0) under UP_SCOPE_PROMPT and 0 otherwise;
 * blocks are counted from that start (the last one may be short).
 * cu_blocks: [S+1] int32 output.  block_size: a multiple of 16 in [16, 256]
 * (UP_ERR_UNSUPPORTED otherwise), the same value in every call of one step.
 * score_flags may be NULL (no segment scored).
 */
up_status up_block_offsets(const up_batch* batch, int32_t block_size, const uint8_t* score_flags,
                           int32_t score_scope, int32_t* cu_blocks, void* stream);

/*
 * Workspace bytes up_prefill_attn needs for this batch shape: the work list
 * of query tiles (and, for UP_F32, score items), plus for UP_BF16 with
 * scoring the per-row run sums of the segments' last blocks.  block_size:
 * the block size up_prefill_attn will be called with when it gets
 * score_flags, else 0; score_scope as it will be called with (the bound for
 * UP_SCOPE_PROMPT counts max_pages * page_size cached tokens per segment).
 * Returns 0 for an unsupported shape.
 */
size_t up_attn_workspace_bytes(const up_batch* batch, up_dtype dtype, int32_t Hq, int32_t Hkv,
                               int32_t D, int32_t block_size, int32_t score_scope);

/*
 * Attention with rotary positions, KV-cache write and fused block mass.
 *
 * Defined by: Ultralytics glossary "Chunked Prefill", "How chunked prefill
 * works" (a piece of a prompt sees the KV stored by the pieces before it and
 * its own tokens, masked by position, and the pieces together give the same
 * result as one pass) and "Related serving techniques" (KV in fixed-size
 * pages); Prepacking summary, "Technical framework" (packed prompts with a
 * block-diagonal mask and positions restarting per prompt); UniPrefill
 * review, "Method & Key Results" (block importance estimated at a
 * full-attention layer inside the prefill, hence the fused block mass).
 *
 * Computes, for every token t of every segment s and every query head h
 * (KV head g = h / (Hq / Hkv)):
 *   out[t,h,:] = sum_j softmax_j(sm_scale * q'[t,h,:] . K'[j,g,:]) V[j,g,:]
 * over the keys j visible to t: the segment's ctx_len cached keys
 * (positions 0..ctx-1) and its own tokens u with positions[u] <=
 * positions[t]; with window > 0 only keys with position >
 * positions[t] - window.  Keys of other segments are never visible (packed
 * block-diagonal mask).  q' and K' are q and k rotated by their positions
 * (rotate-half pairs (i, i + D/2), angle position * rope_theta^(-2i/D));
 * rope_theta <= 0 disables the rotation.
 *
 * First writes the rotated K and V of every token t to the caches at
 * slot_mapping[t]; attention then reads all keys through the caches.
 *
 * For every segment with score_flags[s] != 0 it also writes the block mass
 *   block_mass[(cu_blocks[s] + b) * Hq + h] =
 *     sum over rows t of the segment's last block (local rows
 *     [(nb-1)*block_size, n)) of the softmax probability that row t, head h,
 *     puts on the segment's own keys of block b
 * (cached keys enter the softmax normaliser but are not scored).  Under
 * UP_SCOPE_PROMPT the blocks b are those of the whole prompt (cached keys
 * included, see UP_SCOPE_PROMPT) and the rows those of its last block.
 * Entries of unflagged segments are not written.
 *
 * dtype: UP_F32 (q, k, v, caches, out float32) or UP_BF16 (all bf16;
 *        products on bf16 matrix cores, softmax and accumulation in fp32).
 * Hq % Hkv == 0 (else UP_ERR_INVALID).  Built: Hq / Hkv <= 32 (any
 * group size: 4 for Llama-3, 7 for 28 query over 4 KV heads), Hkv <= 255,
 * D in {64, 128}, at most 4096 segments per call
 * (num_seqs); other values return UP_ERR_UNSUPPORTED.
 * q [T, Hq, D], k, v [T, Hkv, D] row-major, read-only.
 * k_cache, v_cache [num_pages, Hkv, page_size, D], read and written.
 * sm_scale: logit scale; <= 0 selects 1/sqrt(D).
 * score_flags [S] u8, may be NULL (no scoring); then cu_blocks and
 *        block_mass may be NULL.  block_size and score_scope as in
 *        up_block_offsets (UP_SCOPE_PROMPT with UP_F32: UP_ERR_UNSUPPORTED).
 * block_mass [NB, Hq] f32 (NB = cu_blocks[S]).
 * out [T, Hq, D] (dtype); lse [T, Hq] f32 natural-log normaliser of each
 *        row's scaled logits, or NULL.
 * workspace: at least up_attn_workspace_bytes(...) bytes, 16-byte aligned.
 * q, k, v, k_cache, v_cache and out must be 16-byte aligned and lse 4-byte
 * aligned (UP_ERR_INVALID otherwise): rows move as 16-byte chunks.
 */
up_status up_prefill_attn(const up_batch* batch, up_dtype dtype, int32_t Hq, int32_t Hkv,
                          int32_t D, const void* q, const void* k, const void* v, void* k_cache,
                          void* v_cache, float rope_theta, int32_t window, float sm_scale,
                          const uint8_t* score_flags, int32_t block_size, int32_t score_scope,
                          const int32_t* cu_blocks, float* block_mass, void* out, float* lse,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * The same attention call for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same arguments and results as up_prefill_attn, without
 * the workspace.  Its scratch (work list, queue counters, per-run score
 * sums) is a device array of UP_NOALLOC_SCRATCH_BYTES that the library
 * holds on every GPU it runs on until the process ends; the call allocates
 * nothing and frees nothing.  A call that needs more scratch than that
 * (up_attn_workspace_bytes for the same arguments) returns
 * UP_ERR_WORKSPACE and launches nothing.  Every call on one GPU uses the
 * same array, so calls that overlap on one GPU (on different streams, or
 * from different threads without ordering) race and give wrong results;
 * calls ordered on one stream are safe.  Nothing in the scratch has to start
 * at zero.
 */
#define UP_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
up_status up_prefill_attn_noalloc(const up_batch* batch, up_dtype dtype, int32_t Hq, int32_t Hkv,
                                  int32_t D, const void* q, const void* k, const void* v,
                                  void* k_cache, void* v_cache, float rope_theta, int32_t window,
                                  float sm_scale, const uint8_t* score_flags, int32_t block_size,
                                  int32_t score_scope, const int32_t* cu_blocks,
                                  float* block_mass, void* out, float* lse, void* stream);

/*
 * Block scores (UniPrefill review, "Method & Key Results": an importance per
 * token block, estimated at a full-attention layer; "Key Terms &
 * Definitions", Top-p Token Selection: importances normalised so that
 * their cumulative sum can be compared with p).  No page gives a formula;
 * this library's reading is the normalised block mass.
 * For a flagged segment s, score[b] = m_b / sum_b' m_b' with
 * m_b = sum_h block_mass[b, h] (the importance of each own block,
 * normalised over the segment).  Unflagged segments get score 0 for every
 * block.  scores [NB] f32.
 */
up_status up_block_scores(const up_batch* batch, int32_t Hq, int32_t block_size,
                          const int32_t* cu_blocks, const uint8_t* score_flags,
                          const float* block_mass, float* scores, void* stream);

/*
 * Top-p block selection per flagged segment (review, Top-p Token Selection:
 * the fewest blocks whose cumulative importance reaches p).  The first and
 * last blocks are always kept and count toward p.  The others are taken in
 * order of decreasing score (ties: lower block first) while the running sum
 * is below the target.  Exact integer arithmetic: q_b = floor(score_b *
 * 2^40), target = ceil(floor(p * 2^22 + 1/2) * sum_b q_b / 2^22); sums are
 * order-independent, so the result does not depend on thread scheduling.
 * p >= 1 keeps every block.  Scores must be finite, >= 0 and sum to < 2 per
 * segment.  Unflagged segments keep all blocks.
 * p: host double in [0, 1].  keep [NB] u8 (1 = kept); kept_blocks [S] i32
 * number of kept blocks per segment (may be NULL).
 */
up_status up_topp_select(const up_batch* batch, int32_t block_size, const int32_t* cu_blocks,
                         const uint8_t* score_flags, double p, const float* scores,
                         uint8_t* keep, int32_t* kept_blocks, void* stream);

/*
 * Block scores and top-p selection in one launch: the same results as
 * up_block_scores followed by up_topp_select with the same arguments (one
 * workgroup per segment computes its scores, writes them, and selects on
 * them), for callers that want both without the second launch.
 */
up_status up_score_select(const up_batch* batch, int32_t Hq, int32_t block_size,
                          const int32_t* cu_blocks, const uint8_t* score_flags, double p,
                          const float* block_mass, float* scores, uint8_t* keep,
                          int32_t* kept_blocks, void* stream);

/* One row tensor to compact: rows of row_bytes bytes, [T, row] -> [T_kept, row]. */
typedef struct up_rows {
  const void* src;
  void* dst;
  int64_t row_bytes; /* > 0; 16-byte multiples with 16-byte aligned pointers copy fastest */
} up_rows;

/* Workspace bytes up_compact needs. */
size_t up_compact_workspace_bytes(int32_t num_seqs, int32_t num_blocks);

/*
 * Compaction of the kept tokens (review, Method & Key Results: dropped
 * tokens are removed from all later sublayers).  Token t of segment s is
 * kept when its block (local index / block_size) has keep[cu_blocks[s] + b]
 * != 0; under UP_SCOPE_PROMPT a scored segment's own token i is in block
 * (ctx_lens[s] + i) / block_size of its prompt (score_flags and
 * score_scope as given to up_block_offsets; score_flags may be NULL with
 * UP_SCOPE_SEGMENT).  Outputs, in ascending original order:
 *   index_map [T cap] i32: packed index of each kept token;
 *   cu_seqlens_out [S+1] i32: per-segment kept counts, prefix-summed;
 *   num_kept [1] i32 (device);
 *   rows[i].dst[j] = rows[i].src[index_map[j]] byte for byte (positions and
 *   KV slots are compacted by passing them as 4-byte row tensors).
 * num_blocks (host): capacity >= cu_blocks[S].
 * workspace: at least up_compact_workspace_bytes(S, num_blocks) bytes.
 */
up_status up_compact(const up_batch* batch, int32_t block_size, const int32_t* cu_blocks,
                     const uint8_t* score_flags, int32_t score_scope, const uint8_t* keep,
                     int32_t num_blocks, int32_t n_rows, const up_rows* rows /* (host) array of n_rows */,
                     int32_t* index_map, int32_t* cu_seqlens_out, int32_t* num_kept,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Whole-prompt scoring (UP_SCOPE_PROMPT): the KV slots of the kept cached
 * tokens of every scored segment, for the later layers' attention over the
 * kept context (review, Method & Key Results: dropped tokens take no part
 * in later sublayers).  Cached token u (position u) of scored segment s is
 * kept when block u / block_size of its prompt is; its slot is
 * block_table[s * max_pages + u / page_size] * page_size + u % page_size.
 * Outputs, segment by segment, positions ascending:
 *   slots [slots_cap] i32 (entries past slots_cap are not written; a cap of
 *   num_seqs * max_pages * page_size always suffices);
 *   cu_slots_out [S+1] i32: per-segment counts, prefix-summed;
 *   num_slots [1] i32 (device): the total.
 * cu_blocks, score_flags and keep as given to up_compact under
 * UP_SCOPE_PROMPT; workspace as for up_compact.
 */
up_status up_kept_cache_slots(const up_batch* batch, int32_t block_size, const int32_t* cu_blocks,
                              const uint8_t* score_flags, const uint8_t* keep, int32_t num_blocks,
                              int32_t* slots, int32_t slots_cap, int32_t* cu_slots_out,
                              int32_t* num_slots, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * Later-layer linear map on the kept tokens (UniPrefill review, Method & Key
 * Results: dropped tokens skip every later sublayer, so the later layers'
 * matrix products run on the compacted rows; paper entry, abstract).  bf16
 * in and out, float32 accumulation:
 *   act = UP_ACT_NONE:   y[m][n] = sum_k x[m][k] * w[n][k]          y [rows, n_out]
 *   act = UP_ACT_SWIGLU: y[m][f] = silu(g) * u, g and u the sums for w's
 *     gate row and up row of feature f (silu(z) = z / (1 + e^-z); the
 *     SwiGLU gate of Llama-style MLPs, Shazeer 2020)             y [rows, n_out / 2]
 *     w holds gate and up rows interleaved in groups of 32: rows 64q..64q+31
 *     are the gate rows of features 32q..32q+31, rows 64q+32..64q+63 their
 *     up rows.
 * x: [rows_cap, k_in] row-major bf16, 16-byte aligned; w: [n_out, k_in]
 * row-major bf16 (the [out, in] layout), 16-byte aligned; y: 8-byte aligned.
 * rows_in_use (device, may be NULL): rows used = min(*rows_in_use,
 * rows_cap), e.g. the num_kept that up_compact wrote, so no host
 * synchronisation is needed; NULL uses rows_cap.  Rows of y at or beyond
 * the rows used are not written.  n_out: a multiple of 256; k_in: a
 * multiple of 64; x and w each under 4 GiB (UP_ERR_UNSUPPORTED otherwise).
 */
/*
 * Later causal linear-attention layer on the kept tokens (UniPrefill paper
 * entry, abstract: linear/full hybrid models; review, Method & Key Results:
 * dropped tokens skip every later sublayer).  For every segment s (rows
 * [cu_seqlens[s], cu_seqlens[s+1]), e.g. the cu_seqlens_out of up_compact)
 * and query head h with KV head g = h / (Hq / Hkv), phi(x) = elu(x) + 1
 * (Katharopoulos et al. 2020):
 *   out[t][h] = phi(q_t,h)^T S_t / (phi(q_t,h) . z_t),
 *   S_t = sum over the segment's rows r <= t of phi(k_r,g) v_r,g^T,
 *   z_t = sum of phi(k_r,g).
 * q, k, v: bf16 rows (token r's head j at base + r * stride + j * head_dim;
 * strides in elements, multiples of 8, so the q, k and v column ranges of
 * one [rows, (Hq + 2 Hkv) * head_dim] projection output can be passed
 * directly), 16-byte aligned.  out: [rows, Hq, head_dim] bf16; rows outside
 * the segments are not written.  head_dim must be 128 (UP_ERR_UNSUPPORTED);
 * num_seqs at most 65535.
 * Device precondition: cu_seqlens non-decreasing.
 */
up_status up_linear_attn_bf16(const int32_t* cu_seqlens, int32_t num_seqs, const void* q,
                              int64_t q_stride, const void* k, int64_t k_stride, const void* v,
                              int64_t v_stride, int32_t Hq, int32_t Hkv, int32_t head_dim,
                              void* out, void* stream);

/*
 * The same layer computed chunk-parallel (the recurrence above is linear in
 * (S, z), so a segment's running sums can be formed per part and summed):
 * every segment is cut into parts of 1024 rows; the parts' own sums are
 * computed in parallel, summed in part order per segment and head, and
 * every part's outputs then computed in parallel from the sums of the parts
 * before it.  Same results up to the order of float32 additions; the
 * sequential depth is one part instead of the whole segment.  rows: rows of
 * q, k, v and out (cu_seqlens[num_seqs] <= rows is a device precondition;
 * rows / 1024 + num_seqs + 1 <= 65535).  workspace: device scratch of
 * up_linear_attn_workspace_bytes(rows, num_seqs, Hq) bytes (66 KB per
 * query head and part slot), 16-byte aligned, owned by the caller; its
 * contents on entry do not matter.  Other arguments and errors as for
 * up_linear_attn_bf16; a short workspace returns UP_ERR_WORKSPACE.
 */
size_t up_linear_attn_workspace_bytes(int32_t rows, int32_t num_seqs, int32_t Hq);
up_status up_linear_attn_bf16_parts(const int32_t* cu_seqlens, int32_t num_seqs, int32_t rows,
                                    const void* q, int64_t q_stride, const void* k,
                                    int64_t k_stride, const void* v, int64_t v_stride, int32_t Hq,
                                    int32_t Hkv, int32_t head_dim, void* out, void* workspace,
                                    size_t workspace_bytes, void* stream);

#define UP_ACT_NONE 0
#define UP_ACT_SWIGLU 1
up_status up_linear_bf16(const void* x, const void* w, void* y, int32_t rows_cap,
                         const int32_t* rows_in_use, int32_t n_out, int32_t k_in, int32_t act,
                         void* stream);

/*
 * Profiling aid (not part of the operator).  With both arguments non-NULL
 * (hipEvent_t handles created by the caller), up_prefill_attn calls made
 * afterwards on this thread record attn_start on their stream right before
 * the attention kernel is launched and attn_stop right after it, so the
 * kernel's own duration can be read with hipEventElapsedTime.  (NULL, NULL)
 * turns it off.  The events must outlive the calls that record them.
 */
up_status up_profile_attn_events(void* attn_start, void* attn_stop);
/* The same for the rotary/cache-write kernel that up_prefill_attn launches first. */
up_status up_profile_rope_events(void* rope_start, void* rope_stop);

/*
 * Measurement aids (not part of the operator): what the chip sustains, to
 * set beside its published peaks.
 *  - up_peak_mfma_bf16: `workgroups` workgroups of four waves; every wave
 *    runs iters x 4 bf16 products of 32x32x16 (32768 flops each), so one
 *    launch does workgroups * 4 * iters * 4 * 32768 flops.  sink: [workgroups
 *    * 256] float output (a fold of the accumulators, no meaning).
 *  - up_peak_copy: copies `bytes` (a multiple of 16; src and dst 16-byte
 *    aligned, not overlapping) from src to dst with 16-byte loads and stores.
 * Both are asynchronous on ``stream``; time them with events.
 */
up_status up_peak_mfma_bf16(int32_t workgroups, int32_t iters, float* sink, void* stream);
up_status up_peak_copy(const void* src, void* dst, size_t bytes, void* stream);

/*
 * Debug aid (not part of the operator): checks the batch's device-side
 * preconditions listed at the top of this header on the device, reading
 * only inside each array's extent (cu_seqlens [S+1], ctx_lens [S],
 * positions and slot_mapping [T], block_table [S, max_pages]).  num_pages
 * > 0 also checks page ids and slots against a cache of num_pages pages;
 * 0 skips those two range checks.  err_word: one int32 of device scratch.
 * Synchronises ``stream``; returns UP_OK, or UP_ERR_INVALID with
 * up_last_error() naming every violated condition.
 *
 * With the environment variable UP_DEBUG_CHECKS set to a non-zero integer
 * (read on every call), up_prefill_attn runs this check (num_pages = 0,
 * the workspace's first word as err_word) before it launches anything, and
 * returns its status if the batch fails it; with score_scope
 * UP_SCOPE_PROMPT it also checks that every scored segment's ctx_len is a
 * multiple of block_size.
 */
up_status up_check_batch(const up_batch* batch, int32_t num_pages, int32_t* err_word,
                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* UNIPREFILL_H */
