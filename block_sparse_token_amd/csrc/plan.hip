// Batch metadata kernels: block offsets and the attention work list.
//
// The work list puts score items (two QK^T sweeps over a segment's last
// query block) first, then query tiles segment by segment.
#include "common.h"

namespace up {

// cu_blocks[s+1] = cu_blocks[s] + ceil((origin_s + n_s) / B); one workgroup,
// chunked scan.
__global__ __launch_bounds__(1024) void block_offsets_kernel(const int32_t* __restrict__ cu_seqlens,
                                                             BlockOrigin bo, int S, int B,
                                                             int32_t* __restrict__ cu_blocks) {
  __shared__ int32_t wsum[16];
  __shared__ int32_t carry;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  if (tid == 0) {
    carry = 0;
    cu_blocks[0] = 0;
  }
  __syncthreads();
  for (int base = 0; base < S; base += 1024) {
    const int s = base + tid;
    int v = 0;
    if (s < S) v = (cu_seqlens[s + 1] - cu_seqlens[s] + bo.of(s) + B - 1) / B;
    // inclusive wave scan
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wid] = x;
    __syncthreads();
    int off = carry;
    for (int w = 0; w < wid; ++w) off += wsum[w];
    if (s < S) cu_blocks[s + 1] = off + x;
    __syncthreads();
    if (tid == 1023) carry = off + x;
    __syncthreads();
  }
}

hipError_t launch_block_offsets(const int32_t* cu_seqlens, const BlockOrigin& bo, int S,
                                int block_size, int32_t* cu_blocks, hipStream_t st) {
  hipLaunchKernelGGL(block_offsets_kernel, dim3(1), dim3(1024), 0, st, cu_seqlens, bo, S,
                     block_size, cu_blocks);
  return hipGetLastError();
}

// One workgroup.  Segments fall in two classes: memory-bound ones, whose
// rows fit in one wave of a tile (8 n <= P: decodes, the tails of short
// segments), and the rest.  Within its class a segment is ranked by the
// visible-key count of its last row (ctx + n, or the window), heaviest
// first, ties by index; its tiles are listed from the last (most keys) to
// the first, so neighbouring items read the same segment's keys and the
// workgroups that run together on one XCD share its L2.  The two class
// lists are then merged in proportion (item i of a class of N items sits at
// fraction (2i + 1) / 2N, memory-bound first on ties), so that workgroups
// streaming cached keys run beside workgroups bound by the matrix cores,
// and the lightest items of both end the list.  Score items precede all
// tiles.
__device__ inline bool memory_bound_segment(int n, int P) { return 8 * n <= P; }
constexpr int kClassBit = 1 << 30;

// Items of the other class (Y, NY items) ahead of item i of class X (NX
// items): #{j : (2j + 1) NX < (2i + 1) NY}, with <= instead of < when a
// Y item at the same fraction goes first (ties_ahead: X is the
// compute-bound class).  The quotient runs in double: numerator and NX are
// integers below 2^53, and their quotient is at least 1/NX away from any
// integer it does not equal, far more than its rounding error, so floor
// and ceil are exact.
__device__ inline int merged_before(int i, int NX, int NY, bool ties_ahead) {
  if (NY == 0) return 0;
  const double q = ((2.0 * i + 1.0) * NY) / NX;
  const int c = ties_ahead ? ((int)floor(q) + 1) / 2 : (int)ceil(q) / 2;
  return min(c, NY);
}

__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* __restrict__ cu_seqlens,
                                                    const int32_t* __restrict__ ctx_lens,
                                                    const uint8_t* __restrict__ score_flags,
                                                    int S, int P, int window,
                                                    int2* __restrict__ items,
                                                    int32_t* __restrict__ count, int capacity) {
  __shared__ int32_t key[kMaxSeqsPlan];
  __shared__ int32_t order[kMaxSeqsPlan];  // memory-bound class first, each by rank
  __shared__ int32_t cu_t[kMaxSeqsPlan + 1];
  __shared__ int32_t wsum[16];
  __shared__ int32_t carry, n_score, n_mem;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  if (tid == 0) {
    carry = 0;
    n_score = 0;
    n_mem = 0;
    cu_t[0] = 0;
  }
  __syncthreads();
  for (int base = 0; base < S; base += 1024) {
    const int s = base + tid;
    bool mem = false;
    if (s < S) {
      const int n = cu_seqlens[s + 1] - cu_seqlens[s];
      int k = ctx_lens[s] + n;
      if (window > 0) k = min(k, window + P);
      // the class rides in bit 30 of the key (key counts clamped below it)
      mem = memory_bound_segment(n, P);
      key[s] = min(k, kClassBit - 1) | (mem ? kClassBit : 0);
    }
    const unsigned long long m = __ballot(mem);
    if (lane == 0 && m) atomicAdd(&n_mem, __popcll(m));
  }
  __syncthreads();
  const int S_mem = n_mem;
  for (int s = tid; s < S; s += 1024) {
    const int ks = key[s];
    const bool mem = (ks & kClassBit) != 0;
    int r = 0;
    for (int t = 0; t < S; ++t) {
      const int kt = key[t];
      // same class, heavier (or as heavy and earlier)
      r += (((kt ^ ks) & kClassBit) == 0) & ((kt > ks) | ((kt == ks) & (t < s)));
    }
    order[(mem ? 0 : S_mem) + r] = s;
    if (score_flags && score_flags[s]) atomicAdd(&n_score, 1);
  }
  __syncthreads();
  // tiles per segment in class-then-rank order, prefix-summed
  for (int base = 0; base < S; base += 1024) {
    const int r = base + tid;
    int v = 0;
    if (r < S) {
      const int s = order[r];
      v = (cu_seqlens[s + 1] - cu_seqlens[s] + P - 1) / P;
    }
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wid] = x;
    __syncthreads();
    int off = carry;
    for (int w = 0; w < wid; ++w) off += wsum[w];
    if (r < S) cu_t[r + 1] = off + x;
    __syncthreads();
    if (tid == 1023) carry = off + x;
    __syncthreads();
  }
  const int n_tiles = cu_t[S];
  const int n_mem_tiles = cu_t[S_mem];
  const int ns = n_score;
  if (tid == 0) {
    int k = 0;
    if (score_flags)
      for (int r = 0; r < S && k < ns; ++r)
        if (score_flags[order[r]]) items[k++] = make_int2(order[r], kScoreTile);
    *count = min(n_tiles + ns, capacity);
  }
  const int NM = n_mem_tiles, NC = n_tiles - n_mem_tiles;
  for (int i = tid; i < n_tiles; i += 1024) {
    int lo = 0, hi = S - 1;  // position r with cu_t[r] <= i < cu_t[r+1]
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (cu_t[mid] <= i) lo = mid; else hi = mid - 1;
    }
    const int s = order[lo];
    const int nt = cu_t[lo + 1] - cu_t[lo];
    const int j = nt - 1 - (i - cu_t[lo]);
    const bool mem = i < n_mem_tiles;
    const int ic = mem ? i : i - n_mem_tiles;
    const int pos = ic + (mem ? merged_before(ic, NM, NC, false) : merged_before(ic, NC, NM, true));
    if (ns + pos < capacity) items[ns + pos] = make_int2(s, j);
  }
}

// Device-side preconditions of a batch, as violation bits OR-ed into
// err[0] (see kCheck* in common.h).  One thread per segment walks its
// tokens; every index is clamped into its array, so a malformed batch is
// reported, never followed.
__global__ __launch_bounds__(256) void check_zero_kernel(int32_t* err) {
  if (threadIdx.x == 0) err[0] = 0;
}

__global__ __launch_bounds__(256) void check_batch_kernel(const int32_t* __restrict__ cu_seqlens,
                                                          const int32_t* __restrict__ ctx_lens,
                                                          const int32_t* __restrict__ positions,
                                                          const int32_t* __restrict__ slot_mapping,
                                                          const int32_t* __restrict__ block_table,
                                                          const uint8_t* __restrict__ score_flags,
                                                          int S, int T, int max_pages,
                                                          int num_pages, int grid, int32_t* err) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= S) return;
  int bits = 0;
  if (s == 0 && cu_seqlens[0] != 0) bits |= kCheckCuStart;
  if (s == S - 1 && cu_seqlens[S] > T) bits |= kCheckCuEnd;
  const int a = min(max(cu_seqlens[s], 0), T), b = min(max(cu_seqlens[s + 1], 0), T);
  if (cu_seqlens[s + 1] - cu_seqlens[s] < 1) bits |= kCheckSegment;
  const int c = ctx_lens[s];
  if (c < 0) bits |= kCheckCtx;
  // whole-prompt scoring: a scored segment's cached tokens fill whole blocks
  if (grid > 0 && score_flags && score_flags[s] && c % grid) bits |= kCheckBlockGrid;
  for (int t = a; t < b; ++t) {
    const int p = positions[t];
    if (t == a ? p < c : p <= positions[t - 1]) bits |= kCheckPositions;
    const int sl = slot_mapping[t];
    if (sl < 0 || (num_pages > 0 && sl >= num_pages * kPageSize)) bits |= kCheckSlots;
  }
  if (block_table) {
    const long need = ((long)max(c, 0) + kPageSize - 1) / kPageSize;
    if (need > max_pages) bits |= kCheckBlockTable;
    const int m = (int)min(need, (long)max_pages);
    for (int i = 0; i < m; ++i) {
      const int pg = block_table[(long)s * max_pages + i];
      if (pg < 0 || (num_pages > 0 && pg >= num_pages)) bits |= kCheckPages;
    }
  } else if (c > 0) {
    bits |= kCheckBlockTable;
  }
  if (bits) atomicOr(err, bits);
}

hipError_t launch_check_batch(const int32_t* cu_seqlens, const int32_t* ctx_lens,
                              const int32_t* positions, const int32_t* slot_mapping,
                              const int32_t* block_table, const uint8_t* score_flags, int S,
                              int T, int max_pages, int num_pages, int grid, int32_t* err,
                              hipStream_t st) {
  hipLaunchKernelGGL(check_zero_kernel, dim3(1), dim3(64), 0, st, err);
  hipLaunchKernelGGL(check_batch_kernel, dim3((S + 255) / 256), dim3(256), 0, st, cu_seqlens,
                     ctx_lens, positions, slot_mapping, block_table, score_flags, S, T, max_pages,
                     num_pages, grid, err);
  return hipGetLastError();
}

hipError_t launch_plan(const int32_t* cu_seqlens, const int32_t* ctx_lens,
                       const uint8_t* score_flags, int S, int positions_per_tile, int window,
                       int2* items, int32_t* count, int capacity, hipStream_t st) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, st, cu_seqlens, ctx_lens, score_flags,
                     S, positions_per_tile, window, items, count, capacity);
  return hipGetLastError();
}

}  // namespace up
