// Batch metadata kernels: block offsets and the attention work list.
//
// The work list orders query tiles by decreasing cost (keys each tile's last
// row can see) so the longest tiles start first and the tail of the launch
// holds the short ones.  Score items (two QK^T sweeps over a segment's last
// query block) go first.
#include "common.h"

namespace up {

// cu_blocks[s+1] = cu_blocks[s] + ceil(n_s / B); one workgroup, chunked scan.
__global__ __launch_bounds__(1024) void block_offsets_kernel(const int32_t* __restrict__ cu_seqlens,
                                                             int S, int B,
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
    if (s < S) v = (cu_seqlens[s + 1] - cu_seqlens[s] + B - 1) / B;
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

hipError_t launch_block_offsets(const int32_t* cu_seqlens, int S, int block_size,
                                int32_t* cu_blocks, hipStream_t st) {
  hipLaunchKernelGGL(block_offsets_kernel, dim3(1), dim3(1024), 0, st, cu_seqlens, S, block_size,
                     cu_blocks);
  return hipGetLastError();
}

constexpr int kBuckets = 2048;  // cost buckets of 64 keys; the last one is open-ended

__device__ inline int tile_cost(int c, int n, int P, int j, int window) {
  int last_row = min((j + 1) * P, n);  // rows [jP, last_row)
  int vis = c + last_row;
  if (window > 0) vis = min(vis, window + P);
  return vis;
}

// One workgroup.  Segment tile prefix sums live in LDS (S <= kMaxSeqsPlan).
__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* __restrict__ cu_seqlens,
                                                    const int32_t* __restrict__ ctx_lens,
                                                    const uint8_t* __restrict__ score_flags,
                                                    int S, int P, int window,
                                                    int2* __restrict__ items,
                                                    int32_t* __restrict__ count, int capacity) {
  __shared__ int32_t cu_t[kMaxSeqsPlan + 1];
  __shared__ int32_t hist[kBuckets];
  __shared__ int32_t wsum[16];
  __shared__ int32_t carry, n_score;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  for (int b = tid; b < kBuckets; b += 1024) hist[b] = 0;
  if (tid == 0) {
    carry = 0;
    n_score = 0;
    cu_t[0] = 0;
  }
  __syncthreads();
  // tiles per segment, prefix-summed; count flagged segments
  for (int base = 0; base < S; base += 1024) {
    const int s = base + tid;
    int v = 0;
    if (s < S) {
      const int n = cu_seqlens[s + 1] - cu_seqlens[s];
      v = (n + P - 1) / P;
      if (score_flags && score_flags[s]) atomicAdd(&n_score, 1);
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
    if (s < S) cu_t[s + 1] = off + x;
    __syncthreads();
    if (tid == 1023) carry = off + x;
    __syncthreads();
  }
  const int n_tiles = cu_t[S];
  const int ns = n_score;
  int total = n_tiles + ns;
  if (total > capacity) total = capacity;  // cannot happen for a valid batch
  // score items first, in segment order
  if (tid == 0) {
    int k = 0;
    if (score_flags)
      for (int s = 0; s < S && k < ns; ++s)
        if (score_flags[s]) items[k++] = make_int2(s, kScoreTile);
    *count = total;
  }
  // histogram of tile costs
  for (int i = tid; i < n_tiles; i += 1024) {
    int lo = 0, hi = S - 1;  // find s with cu_t[s] <= i < cu_t[s+1]
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (cu_t[mid] <= i) lo = mid; else hi = mid - 1;
    }
    const int s = lo, j = i - cu_t[s];
    const int n = cu_seqlens[s + 1] - cu_seqlens[s];
    const int b = min(kBuckets - 1, tile_cost(ctx_lens[s], n, P, j, window) >> 6);
    atomicAdd(&hist[b], 1);
  }
  __syncthreads();
  // exclusive scan in decreasing-cost order: offset[b] = ns + sum_{b' > b} hist[b']
  if (tid == 0) {
    int acc = ns;
    for (int b = kBuckets - 1; b >= 0; --b) {
      int h = hist[b];
      hist[b] = acc;
      acc += h;
    }
  }
  __syncthreads();
  for (int i = tid; i < n_tiles; i += 1024) {
    int lo = 0, hi = S - 1;
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (cu_t[mid] <= i) lo = mid; else hi = mid - 1;
    }
    const int s = lo, j = i - cu_t[s];
    const int n = cu_seqlens[s + 1] - cu_seqlens[s];
    const int b = min(kBuckets - 1, tile_cost(ctx_lens[s], n, P, j, window) >> 6);
    const int slot = atomicAdd(&hist[b], 1);
    if (slot < capacity) items[slot] = make_int2(s, j);
  }
}

hipError_t launch_plan(const int32_t* cu_seqlens, const int32_t* ctx_lens,
                       const uint8_t* score_flags, int S, int positions_per_tile, int window,
                       int2* items, int32_t* count, int capacity, hipStream_t st) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, st, cu_seqlens, ctx_lens, score_flags,
                     S, positions_per_tile, window, items, count, capacity);
  return hipGetLastError();
}

}  // namespace up
