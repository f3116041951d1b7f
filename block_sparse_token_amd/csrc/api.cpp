// Host side of the C ABI declared in include/uniprefill.h: argument
// validation, workspace carving and kernel launches.  No allocation and no
// device state; only the batch check (a debug aid) synchronises.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include "../../include/uniprefill.h"
#include "common.h"

static_assert(UP_NOALLOC_SCRATCH_BYTES == up::kNoAllocScratchBytes,
              "the header states the no-allocation scratch size");

namespace {

thread_local std::string g_err;
thread_local hipEvent_t g_attn_ev[2] = {nullptr, nullptr};
thread_local hipEvent_t g_rope_ev[2] = {nullptr, nullptr};

up_status fail(up_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

up_status device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return UP_OK;
  return fail(UP_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool valid_block_size(int b) { return b >= 16 && b <= up::kMaxBlockSize && b % 16 == 0; }
#define BLOCK_SIZE_RULE "block_size must be a multiple of 16 in [16, 256] (got %d)"

up_status check_batch(const up_batch* b, bool need_positions) {
  if (!b) return fail(UP_ERR_INVALID, "batch is NULL");
  if (b->num_seqs <= 0) return fail(UP_ERR_INVALID, "num_seqs must be >= 1 (got %d)", b->num_seqs);
  if (b->num_tokens < b->num_seqs)
    return fail(UP_ERR_INVALID, "num_tokens (%d) < num_seqs (%d)", b->num_tokens, b->num_seqs);
  if (!b->cu_seqlens) return fail(UP_ERR_INVALID, "cu_seqlens is NULL");
  if (need_positions) {
    if (!b->ctx_lens) return fail(UP_ERR_INVALID, "ctx_lens is NULL");
    if (!b->positions) return fail(UP_ERR_INVALID, "positions is NULL");
    if (!b->slot_mapping) return fail(UP_ERR_INVALID, "slot_mapping is NULL");
    if (b->page_size != up::kPageSize)
      return fail(UP_ERR_UNSUPPORTED, "page_size must be %d (got %d)", up::kPageSize,
                  b->page_size);
    if (b->block_table && b->max_pages <= 0)
      return fail(UP_ERR_INVALID, "max_pages must be >= 1 with a block table");
  }
  return UP_OK;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// whole-prompt scoring reads the cached lengths, and its workspace bound
// uses the block table's width (cached tokens <= max_pages * page_size)
up_status check_scope(const up_batch* b, int32_t scope) {
  if (scope != UP_SCOPE_SEGMENT && scope != UP_SCOPE_PROMPT)
    return fail(UP_ERR_INVALID, "score_scope must be UP_SCOPE_SEGMENT or UP_SCOPE_PROMPT (got %d)",
                scope);
  if (scope == UP_SCOPE_PROMPT && (!b->ctx_lens || !b->block_table || b->max_pages <= 0))
    return fail(UP_ERR_INVALID, "whole-prompt scoring needs ctx_lens and a block table");
  return UP_OK;
}

up::BlockOrigin block_origin(const up_batch* b, const uint8_t* flags, int32_t scope) {
  up::BlockOrigin bo;
  bo.ctx_lens = b->ctx_lens;
  bo.flags = flags;
  bo.prompt_scope = scope == UP_SCOPE_PROMPT && flags;
  return bo;
}

// UP_DEBUG_CHECKS=1 in the environment: up_prefill_attn checks the batch's
// device-side preconditions first (and synchronises on the result).
bool debug_checks() {
  const char* v = getenv("UP_DEBUG_CHECKS");
  return v && atoi(v) != 0;
}

// grid > 0: also check that every segment flagged in score_flags has a
// ctx_len that is a multiple of grid (whole-prompt scoring).
up_status run_check(const up_batch* b, int32_t num_pages, int32_t* err, hipStream_t st,
                    const uint8_t* score_flags = nullptr, int grid = 0) {
  hipError_t e = up::launch_check_batch(b->cu_seqlens, b->ctx_lens, b->positions,
                                        b->slot_mapping, b->block_table, score_flags, b->num_seqs,
                                        b->num_tokens, b->max_pages, num_pages, grid, err, st);
  if (e != hipSuccess) return device_status(e, "batch check launch");
  int32_t bits = 0;
  e = hipMemcpyAsync(&bits, err, sizeof bits, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return device_status(e, "batch check read-back");
  if (!bits) return UP_OK;
  static const char* what[] = {"cu_seqlens[0] != 0",
                               "a segment has no token",
                               "cu_seqlens[S] > num_tokens",
                               "negative ctx_lens",
                               "positions not increasing inside a segment or below ctx_len",
                               "slot out of range",
                               "page id out of range",
                               "block table too short or missing for cached tokens",
                               "a scored segment's ctx_len is not a multiple of block_size"};
  std::string msg = "batch check failed:";
  for (int i = 0; i < 9; ++i)
    if (bits & (1 << i)) {
      msg += " ";
      msg += what[i];
      msg += ";";
    }
  g_err = msg;
  return UP_ERR_INVALID;
}

int positions_per_tile(up_dtype dt, int D, int G) {
  return dt == UP_BF16 ? up::attn_bf16_positions_per_tile(D, G)
                       : up::attn_f32_positions_per_tile(D, G);
}

}  // namespace

namespace {
up_status check_linear_attn(const int32_t* cu_seqlens, int32_t num_seqs, const void* q,
                            int64_t q_stride, const void* k, int64_t k_stride, const void* v,
                            int64_t v_stride, int32_t Hq, int32_t Hkv, int32_t head_dim,
                            void* out) {
  if (!cu_seqlens || !q || !k || !v || !out)
    return fail(UP_ERR_INVALID, "cu_seqlens, q, k, v and out must be non-NULL");
  if (num_seqs <= 0 || num_seqs > 65535)
    return fail(UP_ERR_INVALID, "num_seqs must be in [1, 65535] (got %d)", num_seqs);
  if (Hkv <= 0 || Hq <= 0 || Hq % Hkv)
    return fail(UP_ERR_INVALID, "Hq (%d) must be a positive multiple of Hkv (%d)", Hq, Hkv);
  if (head_dim != 128) return fail(UP_ERR_UNSUPPORTED, "head_dim must be 128 (got %d)", head_dim);
  if (q_stride < (int64_t)Hq * head_dim || k_stride < (int64_t)Hkv * head_dim ||
      v_stride < (int64_t)Hkv * head_dim || (q_stride | k_stride | v_stride) % 8)
    return fail(UP_ERR_INVALID, "row strides must hold all heads and be multiples of 8 elements");
  if ((((uintptr_t)q) | ((uintptr_t)k) | ((uintptr_t)v)) & 15)
    return fail(UP_ERR_INVALID, "q, k and v must be 16-byte aligned");
  if (((uintptr_t)out) & 1) return fail(UP_ERR_INVALID, "out must be 2-byte aligned");
  return UP_OK;
}
}  // namespace

extern "C" {

const char* up_last_error(void) { return g_err.c_str(); }

const char* up_version(void) { return "uniprefill 0.1 gfx950"; }

up_status up_check_batch(const up_batch* batch, int32_t num_pages, int32_t* err_word,
                         void* stream) {
  up_status st = check_batch(batch, true);
  if (st) return st;
  if (!err_word) return fail(UP_ERR_INVALID, "err_word is NULL");
  if (num_pages < 0) return fail(UP_ERR_INVALID, "num_pages must be >= 0 (got %d)", num_pages);
  return run_check(batch, num_pages, err_word, as_stream(stream));
}

up_status up_profile_attn_events(void* attn_start, void* attn_stop) {
  if ((attn_start == nullptr) != (attn_stop == nullptr))
    return fail(UP_ERR_INVALID, "pass two events or none");
  g_attn_ev[0] = reinterpret_cast<hipEvent_t>(attn_start);
  g_attn_ev[1] = reinterpret_cast<hipEvent_t>(attn_stop);
  return UP_OK;
}

up_status up_profile_rope_events(void* rope_start, void* rope_stop) {
  if ((rope_start == nullptr) != (rope_stop == nullptr))
    return fail(UP_ERR_INVALID, "pass two events or none");
  g_rope_ev[0] = reinterpret_cast<hipEvent_t>(rope_start);
  g_rope_ev[1] = reinterpret_cast<hipEvent_t>(rope_stop);
  return UP_OK;
}

up_status up_peak_mfma_bf16(int32_t workgroups, int32_t iters, float* sink, void* stream) {
  if (workgroups < 1 || iters < 1)
    return fail(UP_ERR_INVALID, "workgroups and iters must be >= 1 (got %d, %d)", workgroups, iters);
  if (!sink) return fail(UP_ERR_INVALID, "sink is NULL");
  return device_status(up::launch_peak_mfma(workgroups, iters, sink, as_stream(stream)),
                       "peak mfma launch");
}

up_status up_peak_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst) return fail(UP_ERR_INVALID, "src and dst must be non-NULL");
  if ((((uintptr_t)src) | ((uintptr_t)dst) | bytes) & 15)
    return fail(UP_ERR_INVALID, "src, dst and bytes must be multiples of 16");
  return device_status(up::launch_peak_copy(src, dst, bytes, as_stream(stream)), "peak copy launch");
}

up_status up_linear_attn_bf16(const int32_t* cu_seqlens, int32_t num_seqs, const void* q,
                              int64_t q_stride, const void* k, int64_t k_stride, const void* v,
                              int64_t v_stride, int32_t Hq, int32_t Hkv, int32_t head_dim,
                              void* out, void* stream) {
  up_status st = check_linear_attn(cu_seqlens, num_seqs, q, q_stride, k, k_stride, v, v_stride,
                                   Hq, Hkv, head_dim, out);
  if (st) return st;
  return device_status(up::launch_linear_attn_bf16(cu_seqlens, num_seqs, 0, q, q_stride, k,
                                                   k_stride, v, v_stride, Hq, Hkv, out, nullptr,
                                                   as_stream(stream)),
                       "linear attention launch");
}

size_t up_linear_attn_workspace_bytes(int32_t rows, int32_t num_seqs, int32_t Hq) {
  if (rows < 0 || num_seqs <= 0 || Hq <= 0) return 0;
  return up::linear_attn_workspace_bytes(rows, num_seqs, Hq);
}

up_status up_linear_attn_bf16_parts(const int32_t* cu_seqlens, int32_t num_seqs, int32_t rows,
                                    const void* q, int64_t q_stride, const void* k,
                                    int64_t k_stride, const void* v, int64_t v_stride, int32_t Hq,
                                    int32_t Hkv, int32_t head_dim, void* out, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  up_status st = check_linear_attn(cu_seqlens, num_seqs, q, q_stride, k, k_stride, v, v_stride,
                                   Hq, Hkv, head_dim, out);
  if (st) return st;
  if (rows < 0) return fail(UP_ERR_INVALID, "rows must be >= 0 (got %d)", rows);
  const int part = up::linear_attn_part_rows();
  if ((int64_t)rows / part + num_seqs + 1 > 65535)
    return fail(UP_ERR_UNSUPPORTED, "rows / %d + num_seqs + 1 must be <= 65535", part);
  if (!workspace) return fail(UP_ERR_INVALID, "workspace is NULL");
  if (((uintptr_t)workspace) & 15) return fail(UP_ERR_INVALID, "workspace must be 16-byte aligned");
  const size_t need = up::linear_attn_workspace_bytes(rows, num_seqs, Hq);
  if (workspace_bytes < need)
    return fail(UP_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  return device_status(up::launch_linear_attn_bf16(cu_seqlens, num_seqs, rows, q, q_stride, k,
                                                   k_stride, v, v_stride, Hq, Hkv, out, workspace,
                                                   as_stream(stream)),
                       "linear attention launch");
}

up_status up_linear_bf16(const void* x, const void* w, void* y, int32_t rows_cap,
                         const int32_t* rows_in_use, int32_t n_out, int32_t k_in, int32_t act,
                         void* stream) {
  if (!x || !w || !y) return fail(UP_ERR_INVALID, "x, w and y must be non-NULL");
  if (rows_cap < 0) return fail(UP_ERR_INVALID, "rows_cap must be >= 0 (got %d)", rows_cap);
  if (n_out <= 0 || n_out % 256)
    return fail(UP_ERR_UNSUPPORTED, "n_out must be a positive multiple of 256 (got %d)", n_out);
  if (k_in <= 0 || k_in % 64)
    return fail(UP_ERR_UNSUPPORTED, "k_in must be a positive multiple of 64 (got %d)", k_in);
  if (act != UP_ACT_NONE && act != UP_ACT_SWIGLU)
    return fail(UP_ERR_INVALID, "act must be UP_ACT_NONE or UP_ACT_SWIGLU (got %d)", act);
  if ((double)rows_cap * k_in * 2 >= 4294967296.0 || (double)n_out * k_in * 2 >= 4294967296.0)
    return fail(UP_ERR_UNSUPPORTED, "x and w must each be under 4 GiB (32-bit row offsets)");
  // one workgroup per 256 x 256 output tile (plus at most 7 x 32 idle ones)
  if ((double)((rows_cap + 255) / 256) * (n_out / 256) + 224.0 >= 2147483648.0)
    return fail(UP_ERR_UNSUPPORTED, "more than 2^31 output tiles");
  if ((((uintptr_t)x) | ((uintptr_t)w)) & 15)
    return fail(UP_ERR_INVALID, "x and w must be 16-byte aligned");
  if (((uintptr_t)y) & 7) return fail(UP_ERR_INVALID, "y must be 8-byte aligned");
  return device_status(up::launch_linear_bf16(x, w, y, rows_cap, rows_in_use, n_out, k_in, act,
                                              as_stream(stream)),
                       "linear launch");
}

up_status up_block_offsets(const up_batch* batch, int32_t block_size, const uint8_t* score_flags,
                           int32_t score_scope, int32_t* cu_blocks, void* stream) {
  up_status st = check_batch(batch, false);
  if (st) return st;
  st = check_scope(batch, score_scope);
  if (st) return st;
  if (!valid_block_size(block_size))
    return fail(UP_ERR_UNSUPPORTED, BLOCK_SIZE_RULE, block_size);
  if (!cu_blocks) return fail(UP_ERR_INVALID, "cu_blocks is NULL");
  return device_status(up::launch_block_offsets(batch->cu_seqlens,
                                                block_origin(batch, score_flags, score_scope),
                                                batch->num_seqs, block_size, cu_blocks,
                                                as_stream(stream)),
                       "block offsets launch");
}

namespace {
// bf16 scoring scratch: runs of min(block, 64) keys of every block, one
// value per last-block row and head, plus one total per last-block row and
// head of every segment
// Upper bound on the blocks of a call (cu_blocks[S]): every token in use
// and, for whole-prompt scoring, every cached token the block table can
// hold, plus one partial block per segment.
size_t block_cap(const up_batch* b, int block_size, int scope) {
  const size_t cached =
      scope == UP_SCOPE_PROMPT ? (size_t)b->num_seqs * b->max_pages * up::kPageSize : 0;
  return ((size_t)b->num_tokens + cached + block_size - 1) / block_size + b->num_seqs;
}
size_t score_runs(const up_batch* b, int block_size, int scope) {
  return block_cap(b, block_size, scope) * (size_t)(block_size / up::score_run_len(block_size));
}
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
}  // namespace

size_t up_attn_workspace_bytes(const up_batch* batch, up_dtype dtype, int32_t Hq, int32_t Hkv,
                               int32_t D, int32_t block_size, int32_t score_scope) {
  if (!batch || Hkv <= 0 || Hq <= 0 || Hq % Hkv) return 0;
  const int G = Hq / Hkv;
  if (G > 32) return 0;
  const int P = positions_per_tile(dtype, D, G);
  if (P <= 0) return 0;
  size_t bytes = 16 + sizeof(int2) * up::work_capacity(batch->num_tokens, batch->num_seqs, P);
  if (dtype == UP_BF16 && block_size != 0) {
    if (!valid_block_size(block_size)) return 0;
    bytes = align256(bytes);
    bytes += sizeof(float) * score_runs(batch, block_size, score_scope) * block_size * Hq;
    bytes += sizeof(float) * (size_t)batch->num_seqs * block_size * Hq;
  }
  return bytes;
}

namespace {
// The attention call with its scratch in `workspace`: a caller's buffer, or
// (noalloc) the library's per-device scratch array.
up_status prefill_attn_impl(const up_batch* batch, up_dtype dtype, int32_t Hq, int32_t Hkv,
                            int32_t D, const void* q, const void* k, const void* v,
                            void* k_cache, void* v_cache, float rope_theta, int32_t window,
                            float sm_scale, const uint8_t* score_flags, int32_t block_size,
                            int32_t score_scope, const int32_t* cu_blocks, float* block_mass,
                            void* out, float* lse, void* workspace, size_t workspace_bytes,
                            void* stream, bool noalloc) {
  up_status st = check_batch(batch, true);
  if (st) return st;
  st = check_scope(batch, score_scope);
  if (st) return st;
  if (score_scope == UP_SCOPE_PROMPT && dtype != UP_BF16)
    return fail(UP_ERR_UNSUPPORTED, "whole-prompt scoring is built for the bf16 path only");
  if (dtype != UP_F32 && dtype != UP_BF16) return fail(UP_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv)
    return fail(UP_ERR_INVALID, "Hq (%d) must be a positive multiple of Hkv (%d)", Hq, Hkv);
  const int G = Hq / Hkv;
  if (G > 32) return fail(UP_ERR_UNSUPPORTED, "Hq / Hkv must be at most 32 (got %d)", G);
  if (Hkv > 255) return fail(UP_ERR_UNSUPPORTED, "at most 255 KV heads (got %d)", Hkv);
  if (D != 64 && D != 128) return fail(UP_ERR_UNSUPPORTED, "head dim must be 64 or 128 (got %d)", D);
  if (!q || !k || !v || !k_cache || !v_cache || !out)
    return fail(UP_ERR_INVALID, "q, k, v, k_cache, v_cache and out must be non-NULL");
  // rows move as 16-byte chunks (global-to-LDS copies, vector loads and stores)
  if ((((uintptr_t)q) | ((uintptr_t)k) | ((uintptr_t)v) | ((uintptr_t)k_cache) |
       ((uintptr_t)v_cache) | ((uintptr_t)out)) & 15)
    return fail(UP_ERR_INVALID, "q, k, v, k_cache, v_cache and out must be 16-byte aligned");
  if (((uintptr_t)lse) & 3) return fail(UP_ERR_INVALID, "lse must be 4-byte aligned");
  if (!noalloc) {
    if (!workspace) return fail(UP_ERR_INVALID, "workspace is NULL");
    if (((uintptr_t)workspace) & 15)
      return fail(UP_ERR_INVALID, "workspace must be 16-byte aligned");
  }
  if (!(rope_theta == rope_theta) || !(sm_scale == sm_scale))
    return fail(UP_ERR_INVALID, "rope_theta and sm_scale must not be NaN");
  if (score_flags) {
    if (!valid_block_size(block_size))
      return fail(UP_ERR_UNSUPPORTED, BLOCK_SIZE_RULE, block_size);
    if (!cu_blocks || !block_mass)
      return fail(UP_ERR_INVALID, "scoring needs cu_blocks and block_mass");
    // one block-mass workgroup per possible block of the call
    if (block_cap(batch, block_size, score_scope) > 0x7fffffff)
      return fail(UP_ERR_UNSUPPORTED, "too many blocks in one call");
  }
  if (batch->num_seqs > up::kMaxSeqsPlan)
    return fail(UP_ERR_UNSUPPORTED, "at most %d segments per call (got %d)", up::kMaxSeqsPlan,
                batch->num_seqs);
  const size_t need =
      up_attn_workspace_bytes(batch, dtype, Hq, Hkv, D, score_flags ? block_size : 0, score_scope);
  if (noalloc) {
    if (need > up::kNoAllocScratchBytes)
      return fail(UP_ERR_WORKSPACE,
                  "this call needs %zu bytes of scratch; the no-allocation entry point holds %zu "
                  "(fewer tokens, segments or cached pages per call, or up_prefill_attn with a "
                  "workspace)",
                  need, up::kNoAllocScratchBytes);
    // the GPU's scratch array, after every argument check
    const hipError_t e = up::noalloc_scratch(&workspace);
    if (e != hipSuccess) return device_status(e, "no-allocation scratch lookup");
    workspace_bytes = up::kNoAllocScratchBytes;
  }
  if (workspace_bytes < need)
    return fail(UP_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);

  hipStream_t s = as_stream(stream);
  if (debug_checks()) {
    const bool prompt = score_flags && score_scope == UP_SCOPE_PROMPT;
    st = run_check(batch, 0, (int32_t*)workspace, s, score_flags, prompt ? block_size : 0);
    if (st) return st;
  }
  const bool bf16 = dtype == UP_BF16;
  const int P = positions_per_tile(dtype, D, G);
  const int cap = (int)up::work_capacity(batch->num_tokens, batch->num_seqs, P);

  // rotary frequencies in turns per position: theta^(-2j/D) / (2 pi)
  double rev[up::kMaxRopePairs] = {0};
  const int rope = rope_theta > 0.f;
  if (rope)
    for (int j = 0; j < D / 2; ++j)
      rev[j] = pow((double)rope_theta, -2.0 * j / D) / (2.0 * 3.141592653589793238462643383279502884);

  up::RopeArgs ra;
  ra.k = k;
  ra.v = v;
  ra.k_cache = k_cache;
  ra.v_cache = v_cache;
  ra.cu_seqlens = batch->cu_seqlens;
  ra.positions = batch->positions;
  ra.slot_mapping = batch->slot_mapping;
  ra.S = batch->num_seqs;
  ra.T = batch->num_tokens;
  ra.Hkv = Hkv;
  ra.rope = rope;
  for (int j = 0; j < up::kMaxRopePairs; ++j) ra.rope_rev[j] = rev[j];
  hipError_t e;
  if (g_rope_ev[0]) {
    e = hipEventRecord(g_rope_ev[0], s);
    if (e != hipSuccess) return device_status(e, "profiling event record");
  }
  e = up::launch_rope_kv(ra, bf16, D, s);
  if (e != hipSuccess) return device_status(e, "rope/kv-write launch");
  if (g_rope_ev[1]) {
    e = hipEventRecord(g_rope_ev[1], s);
    if (e != hipSuccess) return device_status(e, "profiling event record");
  }

  int32_t* count = (int32_t*)workspace;
  int2* items = (int2*)((char*)workspace + 16);
  // the bf16 kernel scores inside its attention items: no score items
  e = up::launch_plan(batch->cu_seqlens, batch->ctx_lens, bf16 ? nullptr : score_flags,
                      batch->num_seqs, P, window, items, count, cap, s);
  if (e != hipSuccess) return device_status(e, "work-plan launch");

  up::AttnArgs a;
  a.q = q;
  a.out = out;
  a.lse = lse;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.cu_seqlens = batch->cu_seqlens;
  a.ctx_lens = batch->ctx_lens;
  a.positions = batch->positions;
  a.slot_mapping = batch->slot_mapping;
  a.block_table = batch->block_table;
  a.score_flags = score_flags;
  a.cu_blocks = cu_blocks;
  a.block_mass = block_mass;
  a.score_part = nullptr;
  a.score_lse = nullptr;
  if (bf16 && score_flags) {
    a.score_part = (float*)((char*)workspace + align256(16 + sizeof(int2) * (size_t)cap));
    a.score_lse = a.score_part + score_runs(batch, block_size, score_scope) * block_size * Hq;
  }
  a.items = items;
  a.item_count = count;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = G;
  a.max_pages = batch->max_pages;
  a.block_size = block_size;
  a.score_scope = score_flags && score_scope == UP_SCOPE_PROMPT;
  a.window = window > 0 ? window : 0;
  a.rope = rope;
  a.scale = sm_scale > 0.f ? sm_scale : (float)(1.0 / sqrt((double)D));
  a.scale_log2 = (float)((double)a.scale * 1.4426950408889634073599246810018921);
  for (int j = 0; j < up::kMaxRopePairs; ++j) a.rope_rev[j] = rev[j];
  if (g_attn_ev[0]) {
    e = hipEventRecord(g_attn_ev[0], s);
    if (e != hipSuccess) return device_status(e, "profiling event record");
  }
  e = bf16 ? up::launch_attn_bf16(a, D, cap, s) : up::launch_attn_f32(a, D, cap, s);
  if (e != hipSuccess) return device_status(e, "attention launch");
  if (g_attn_ev[1]) {
    e = hipEventRecord(g_attn_ev[1], s);
    if (e != hipSuccess) return device_status(e, "profiling event record");
  }
  if (bf16 && score_flags) {
    e = up::launch_block_mass(a, batch->num_seqs, (int)block_cap(batch, block_size, score_scope),
                              s);
    if (e != hipSuccess) return device_status(e, "block mass launch");
  }
  return UP_OK;
}

}  // namespace

up_status up_prefill_attn(const up_batch* batch, up_dtype dtype, int32_t Hq, int32_t Hkv,
                          int32_t D, const void* q, const void* k, const void* v, void* k_cache,
                          void* v_cache, float rope_theta, int32_t window, float sm_scale,
                          const uint8_t* score_flags, int32_t block_size, int32_t score_scope,
                          const int32_t* cu_blocks, float* block_mass, void* out, float* lse,
                          void* workspace, size_t workspace_bytes, void* stream) {
  return prefill_attn_impl(batch, dtype, Hq, Hkv, D, q, k, v, k_cache, v_cache, rope_theta,
                           window, sm_scale, score_flags, block_size, score_scope, cu_blocks,
                           block_mass, out, lse, workspace, workspace_bytes, stream, false);
}

up_status up_prefill_attn_noalloc(const up_batch* batch, up_dtype dtype, int32_t Hq, int32_t Hkv,
                                  int32_t D, const void* q, const void* k, const void* v,
                                  void* k_cache, void* v_cache, float rope_theta, int32_t window,
                                  float sm_scale, const uint8_t* score_flags, int32_t block_size,
                                  int32_t score_scope, const int32_t* cu_blocks,
                                  float* block_mass, void* out, float* lse, void* stream) {
  return prefill_attn_impl(batch, dtype, Hq, Hkv, D, q, k, v, k_cache, v_cache, rope_theta,
                           window, sm_scale, score_flags, block_size, score_scope, cu_blocks,
                           block_mass, out, lse, nullptr, 0, stream, true);
}

up_status up_block_scores(const up_batch* batch, int32_t Hq, int32_t block_size,
                          const int32_t* cu_blocks, const uint8_t* score_flags,
                          const float* block_mass, float* scores, void* stream) {
  up_status st = check_batch(batch, false);
  if (st) return st;
  if (Hq <= 0) return fail(UP_ERR_INVALID, "Hq must be >= 1");
  if (!valid_block_size(block_size))
    return fail(UP_ERR_UNSUPPORTED, BLOCK_SIZE_RULE, block_size);
  if (!cu_blocks || !scores) return fail(UP_ERR_INVALID, "cu_blocks and scores must be non-NULL");
  if (score_flags && !block_mass) return fail(UP_ERR_INVALID, "block_mass is NULL");
  return device_status(up::launch_block_scores(batch->cu_seqlens, cu_blocks, score_flags,
                                               block_mass, scores, batch->num_seqs, Hq,
                                               as_stream(stream)),
                       "block scores launch");
}

up_status up_topp_select(const up_batch* batch, int32_t block_size, const int32_t* cu_blocks,
                         const uint8_t* score_flags, double p, const float* scores,
                         uint8_t* keep, int32_t* kept_blocks, void* stream) {
  up_status st = check_batch(batch, false);
  if (st) return st;
  if (!valid_block_size(block_size))
    return fail(UP_ERR_UNSUPPORTED, BLOCK_SIZE_RULE, block_size);
  if (!(p >= 0.0 && p <= 1.0)) return fail(UP_ERR_INVALID, "p must be in [0, 1] (got %g)", p);
  if (!cu_blocks || !keep) return fail(UP_ERR_INVALID, "cu_blocks and keep must be non-NULL");
  if (score_flags && !scores) return fail(UP_ERR_INVALID, "scores is NULL");
  const uint32_t p_fx = (uint32_t)floor(ldexp(p, 22) + 0.5);
  const int keep_all = p >= 1.0;
  return device_status(up::launch_topp(cu_blocks, score_flags, scores, keep, kept_blocks,
                                       batch->num_seqs, p_fx, keep_all, as_stream(stream)),
                       "top-p launch");
}

up_status up_score_select(const up_batch* batch, int32_t Hq, int32_t block_size,
                          const int32_t* cu_blocks, const uint8_t* score_flags, double p,
                          const float* block_mass, float* scores, uint8_t* keep,
                          int32_t* kept_blocks, void* stream) {
  up_status st = check_batch(batch, false);
  if (st) return st;
  if (Hq <= 0) return fail(UP_ERR_INVALID, "Hq must be >= 1");
  if (!valid_block_size(block_size))
    return fail(UP_ERR_UNSUPPORTED, BLOCK_SIZE_RULE, block_size);
  if (!(p >= 0.0 && p <= 1.0)) return fail(UP_ERR_INVALID, "p must be in [0, 1] (got %g)", p);
  if (!cu_blocks || !scores || !keep)
    return fail(UP_ERR_INVALID, "cu_blocks, scores and keep must be non-NULL");
  if (score_flags && !block_mass) return fail(UP_ERR_INVALID, "block_mass is NULL");
  const uint32_t p_fx = (uint32_t)floor(ldexp(p, 22) + 0.5);
  return device_status(up::launch_score_select(cu_blocks, score_flags, block_mass, scores, Hq,
                                               keep, kept_blocks, batch->num_seqs, p_fx, p >= 1.0,
                                               as_stream(stream)),
                       "score/select launch");
}

size_t up_compact_workspace_bytes(int32_t num_seqs, int32_t num_blocks) {
  (void)num_seqs;
  if (num_blocks <= 0) return 0;
  return 2 * sizeof(int32_t) * ((size_t)num_blocks + 4);
}

up_status up_compact(const up_batch* batch, int32_t block_size, const int32_t* cu_blocks,
                     const uint8_t* score_flags, int32_t score_scope, const uint8_t* keep,
                     int32_t num_blocks, int32_t n_rows, const up_rows* rows,
                     int32_t* index_map, int32_t* cu_seqlens_out, int32_t* num_kept,
                     void* workspace, size_t workspace_bytes, void* stream) {
  up_status st = check_batch(batch, false);
  if (st) return st;
  st = check_scope(batch, score_scope);
  if (st) return st;
  if (!valid_block_size(block_size))
    return fail(UP_ERR_UNSUPPORTED, BLOCK_SIZE_RULE, block_size);
  if (!cu_blocks || !keep || !index_map || !cu_seqlens_out || !num_kept)
    return fail(UP_ERR_INVALID, "cu_blocks, keep, index_map, cu_seqlens_out, num_kept must be non-NULL");
  if (num_blocks < batch->num_seqs)
    return fail(UP_ERR_INVALID, "num_blocks (%d) < num_seqs (%d)", num_blocks, batch->num_seqs);
  if (n_rows < 0 || n_rows > up::kMaxRowTensors)
    return fail(UP_ERR_UNSUPPORTED, "n_rows must be in [0, %d] (got %d)", up::kMaxRowTensors, n_rows);
  if (n_rows && !rows) return fail(UP_ERR_INVALID, "rows is NULL");
  up::RowCopy rc[up::kMaxRowTensors];
  for (int i = 0; i < n_rows; ++i) {
    if (!rows[i].src || !rows[i].dst || rows[i].row_bytes <= 0)
      return fail(UP_ERR_INVALID, "rows[%d]: src/dst NULL or row_bytes <= 0", i);
    rc[i].src = (const uint8_t*)rows[i].src;
    rc[i].dst = (uint8_t*)rows[i].dst;
    rc[i].row_bytes = rows[i].row_bytes;
  }
  if (!workspace) return fail(UP_ERR_INVALID, "workspace is NULL");
  const size_t need = up_compact_workspace_bytes(batch->num_seqs, num_blocks);
  if (workspace_bytes < need)
    return fail(UP_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  int32_t* block_out = (int32_t*)workspace;
  int32_t* block_seg = block_out + num_blocks + 4;
  return device_status(up::launch_compact(batch->cu_seqlens, cu_blocks,
                                          block_origin(batch, score_flags, score_scope), keep,
                                          batch->num_seqs,
                                          num_blocks, block_size, rc, n_rows, index_map,
                                          cu_seqlens_out, num_kept, block_out, block_seg,
                                          as_stream(stream)),
                       "compaction launch");
}

}  // extern "C"

up_status up_kept_cache_slots(const up_batch* batch, int32_t block_size, const int32_t* cu_blocks,
                              const uint8_t* score_flags, const uint8_t* keep, int32_t num_blocks,
                              int32_t* slots, int32_t slots_cap, int32_t* cu_slots_out,
                              int32_t* num_slots, void* workspace, size_t workspace_bytes,
                              void* stream) {
  up_status st = check_batch(batch, false);
  if (st) return st;
  st = check_scope(batch, UP_SCOPE_PROMPT);
  if (st) return st;
  if (!valid_block_size(block_size))
    return fail(UP_ERR_UNSUPPORTED, BLOCK_SIZE_RULE, block_size);
  if (!cu_blocks || !score_flags || !keep || !slots || !cu_slots_out || !num_slots)
    return fail(UP_ERR_INVALID,
                "cu_blocks, score_flags, keep, slots, cu_slots_out and num_slots must be non-NULL");
  if (num_blocks < batch->num_seqs)
    return fail(UP_ERR_INVALID, "num_blocks (%d) < num_seqs (%d)", num_blocks, batch->num_seqs);
  if (slots_cap < 0) return fail(UP_ERR_INVALID, "slots_cap must be >= 0 (got %d)", slots_cap);
  if (!workspace) return fail(UP_ERR_INVALID, "workspace is NULL");
  const size_t need = up_compact_workspace_bytes(batch->num_seqs, num_blocks);
  if (workspace_bytes < need)
    return fail(UP_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  int32_t* block_out = (int32_t*)workspace;
  int32_t* block_seg = block_out + num_blocks + 4;
  return device_status(
      up::launch_kept_cache_slots(batch->cu_seqlens, cu_blocks, keep,
                                  block_origin(batch, score_flags, UP_SCOPE_PROMPT),
                                  batch->block_table, batch->max_pages, batch->num_seqs,
                                  num_blocks, block_size, slots, slots_cap, cu_slots_out,
                                  num_slots, block_out, block_seg, as_stream(stream)),
      "kept cache slots launch");
}
