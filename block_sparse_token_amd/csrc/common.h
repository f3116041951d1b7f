// Internal declarations shared by the host entry points and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

namespace up {

// ---------------------------------------------------------------- limits
constexpr int kPageSize = 16;
constexpr int kMaxSeqsPlan = 4096;  // segments per call the work planner handles
constexpr int kMaxRopePairs = 64;   // D / 2 for D = 128
constexpr int kMaxBlockSize = 256;  // block sizes: multiples of 16 in [16, 256]
// scratch of the no-allocation attention entry point, per GPU
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;

// The bf16 attention sweep records the log2-sum-exp of every run of this
// many consecutive scored keys (a run never straddles a 64-key tile, and a
// block is a whole number of runs).
__host__ __device__ inline int score_run_len(int block_size) {
  return (block_size % 64) == 0 ? 64 : (block_size % 32) == 0 ? 32 : 16;
}

// ---------------------------------------------------------------- work items
// One attention work item = (segment, query tile) or a score item for a
// flagged segment (tile == kScoreTile).  Launched once per KV head.
constexpr int kScoreTile = -1;

// Work list layout inside the attention workspace (bytes):
//   [0, 16): int32 item count
//   [16, ...): int2 items[capacity]
inline size_t work_capacity(int T, int S, int positions_per_tile) {
  return (size_t)((T + positions_per_tile - 1) / positions_per_tile) + 2 * (size_t)S + 1;
}

// ---------------------------------------------------------------- kernel parameters
// Where a segment's blocks start: at its own first token, or, for a scored
// segment under whole-prompt scoring, at its prompt's first token (the
// cached tokens form the first blocks; their count is a multiple of the
// block size).  ``of(s)`` is the number of the segment's tokens before its
// own first one that its blocks cover.
struct BlockOrigin {
  const int32_t* ctx_lens;
  const uint8_t* flags;
  int prompt_scope;
  __device__ inline int of(int s) const {
    return (prompt_scope && flags && flags[s]) ? ctx_lens[s] : 0;
  }
};

struct AttnArgs {
  const void* q;
  void* out;
  float* lse;
  const void* k_cache;
  const void* v_cache;
  const int32_t* cu_seqlens;
  const int32_t* ctx_lens;
  const int32_t* positions;
  const int32_t* slot_mapping;
  const int32_t* block_table;
  const uint8_t* score_flags;
  const int32_t* cu_blocks;
  float* block_mass;
  // bf16 path, scored segments: run and row log2-sum-exps of the last
  // block's rows (score_part [runs][block][Hq], score_lse [S][block][Hq])
  float* score_part;
  float* score_lse;
  const int2* items;
  const int32_t* item_count;
  int Hq, Hkv, G, max_pages, block_size, window, rope;
  int score_scope;   // 1: scored segments are scored over their whole prompt
  float scale;       // logit scale (1/sqrt(D) by default)
  float scale_log2;  // scale * log2(e)
  // rotary frequencies: rev[j] = theta^(-2j/D) / (2 pi) (turns per position)
  double rope_rev[kMaxRopePairs];
};

struct RopeArgs {
  const void* k;
  const void* v;
  void* k_cache;
  void* v_cache;
  const int32_t* cu_seqlens;
  const int32_t* positions;
  const int32_t* slot_mapping;
  int S, T, Hkv, rope;
  double rope_rev[kMaxRopePairs];
};

// ---------------------------------------------------------------- launchers
// All return hipSuccess or the launch error.
// violation bits reported by launch_check_batch
constexpr int kCheckCuStart = 1 << 0;     // cu_seqlens[0] != 0
constexpr int kCheckSegment = 1 << 1;     // a segment with fewer than one token
constexpr int kCheckCuEnd = 1 << 2;       // cu_seqlens[S] > num_tokens
constexpr int kCheckCtx = 1 << 3;         // ctx_lens < 0
constexpr int kCheckPositions = 1 << 4;   // not strictly increasing, or first < ctx
constexpr int kCheckSlots = 1 << 5;       // slot < -1 or beyond the page pool
constexpr int kCheckPages = 1 << 6;       // page id < 0 or beyond the page pool
constexpr int kCheckBlockTable = 1 << 7;  // table too short for ctx + n, or missing
constexpr int kCheckBlockGrid = 1 << 8;   // scored ctx_len not a multiple of `grid`
// grid > 0 (with score_flags): the whole-prompt scoring precondition
hipError_t launch_check_batch(const int32_t* cu_seqlens, const int32_t* ctx_lens,
                              const int32_t* positions, const int32_t* slot_mapping,
                              const int32_t* block_table, const uint8_t* score_flags, int S,
                              int T, int max_pages, int num_pages, int grid, int32_t* err,
                              hipStream_t st);
// blocks_cap: at least cu_blocks[S] (workgroups past it exit at once)
// Device address of this GPU's no-allocation scratch (kNoAllocScratchBytes,
// 256-byte aligned); looked up once per device, with that device current.
hipError_t noalloc_scratch(void** ptr);
hipError_t launch_block_mass(const AttnArgs& a, int S, int blocks_cap, hipStream_t st);
hipError_t launch_peak_mfma(int workgroups, int iters, float* sink, hipStream_t st);
hipError_t launch_peak_copy(const void* src, void* dst, size_t bytes, hipStream_t st);
// ws NULL: one workgroup per (query head, segment); else the
// chunk-parallel form over parts, ws of linear_attn_workspace_bytes(rows,
// S, Hq) bytes
int linear_attn_part_rows();
size_t linear_attn_workspace_bytes(int rows, int S, int Hq);
hipError_t launch_linear_attn_bf16(const int32_t* cu_seqlens, int S, int rows, const void* q,
                                   long q_stride, const void* k, long k_stride, const void* v,
                                   long v_stride, int Hq, int Hkv, void* out, void* ws,
                                   hipStream_t st);
hipError_t launch_linear_bf16(const void* x, const void* w, void* y, int rows_cap,
                              const int32_t* rows_dev, int N, int K, int act, hipStream_t st);
hipError_t launch_block_offsets(const int32_t* cu_seqlens, const BlockOrigin& bo, int S, int block_size,
                                int32_t* cu_blocks, hipStream_t st);
hipError_t launch_plan(const int32_t* cu_seqlens, const int32_t* ctx_lens,
                       const uint8_t* score_flags, int S, int positions_per_tile, int window,
                       int2* items, int32_t* count, int capacity, hipStream_t st);
hipError_t launch_rope_kv(const RopeArgs& a, bool bf16, int D, hipStream_t st);
int attn_bf16_positions_per_tile(int D, int G);
hipError_t launch_attn_bf16(const AttnArgs& a, int D, int capacity, hipStream_t st);
int attn_f32_positions_per_tile(int D, int G);
hipError_t launch_attn_f32(const AttnArgs& a, int D, int capacity, hipStream_t st);
hipError_t launch_block_scores(const int32_t* cu_seqlens, const int32_t* cu_blocks,
                               const uint8_t* flags, const float* mass, float* scores, int S,
                               int Hq, hipStream_t st);
hipError_t launch_score_select(const int32_t* cu_blocks, const uint8_t* flags, const float* mass,
                               float* scores, int Hq, uint8_t* keep, int32_t* kept_blocks, int S,
                               uint32_t p_fx, int keep_all, hipStream_t st);
hipError_t launch_topp(const int32_t* cu_blocks, const uint8_t* flags, const float* scores,
                       uint8_t* keep, int32_t* kept_blocks, int S, uint32_t p_fx, int keep_all,
                       hipStream_t st);
struct RowCopy {
  const uint8_t* src;
  uint8_t* dst;
  int64_t row_bytes;
};
constexpr int kMaxRowTensors = 16;
hipError_t launch_kept_cache_slots(const int32_t* cu_seqlens, const int32_t* cu_blocks,
                                   const uint8_t* keep, const BlockOrigin& bo,
                                   const int32_t* block_table, int max_pages, int S,
                                   int num_blocks, int block_size, int32_t* slots, int slots_cap,
                                   int32_t* cu_out, int32_t* num_out, int32_t* block_out,
                                   int32_t* block_seg, hipStream_t st);
hipError_t launch_compact(const int32_t* cu_seqlens, const int32_t* cu_blocks, const BlockOrigin& bo,
                          const uint8_t* keep, int S, int num_blocks, int block_size,
                          const RowCopy* rows, int n_rows, int32_t* index_map,
                          int32_t* cu_seqlens_out, int32_t* num_kept, int32_t* block_out,
                          int32_t* block_seg, hipStream_t st);

}  // namespace up
