// Compaction of the kept tokens (UniPrefill review, "Method & Key Results":
// the removed tokens take no part in any later sublayer, so later layers see
// only the kept rows).
//
// Under whole-prompt scoring a scored segment's first blocks are its cached
// tokens (BlockOrigin): they hold none of the call's rows, and a second
// entry lists the KV slots of the kept ones instead.
//
// Pass 1 (one workgroup): exclusive scan over blocks of (kept ? length : 0)
// gives each kept block's first output row, the per-segment output offsets
// (cu_seqlens_out) and the kept count.  Pass 2: the rows of one block are
// contiguous in the input and in the output, so each kept block is a
// contiguous byte range per row tensor; workgroups copy slices of those
// ranges with 16-byte vector loads and stores and write the index map.
//
// Calls with at most kFusedBlocks blocks under segment scope skip pass 1:
// each copying workgroup sums the kept lengths of the blocks before its own
// (a few hundred at most, with the block offsets staged in LDS), so one
// launch does the whole compaction; the launch saved is most of the pass's
// time at those sizes.
#include "common.h"

namespace up {

// cached = false: each block counts its kept own rows; cached = true: each
// kept block of cached tokens counts its B tokens.
__global__ __launch_bounds__(1024) void compact_scan_kernel(
    const int32_t* __restrict__ cu_seqlens, const int32_t* __restrict__ cu_blocks,
    const uint8_t* __restrict__ keep, BlockOrigin bo, bool cached, int S, int B,
    int32_t* __restrict__ block_out,
    int32_t* __restrict__ block_seg, int32_t* __restrict__ cu_out, int32_t* __restrict__ num_kept) {
  __shared__ int32_t wsum[16];
  __shared__ int32_t carry;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int NB = cu_blocks[S];
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < NB; base += 1024) {
    const int k = base + tid;
    int v = 0, s = 0;
    if (k < NB) {
      int lo = 0, hi = S - 1;  // segment with cu_blocks[s] <= k < cu_blocks[s+1]
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cu_blocks[mid] <= k) lo = mid; else hi = mid - 1;
      }
      s = lo;
      const int n = cu_seqlens[s + 1] - cu_seqlens[s];
      const int i0 = (k - cu_blocks[s]) * B - bo.of(s);  // first own row of the block
      // (a cached block holds min(B, -i0) cached tokens; B whenever the
      // cached length is on the block grid, as whole-prompt scoring requires)
      if (cached) v = keep[k] && i0 < 0 ? min(B, -i0) : 0;
      else v = keep[k] && i0 >= 0 ? min(B, n - i0) : 0;
      block_seg[k] = s;
    }
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wid] = x;
    __syncthreads();
    int off = carry;
    for (int w = 0; w < wid; ++w) off += wsum[w];
    const int excl = off + x - v;
    if (k < NB) block_out[k] = excl;
    __syncthreads();
    if (tid == 1023) carry = off + x;
    __syncthreads();
  }
  // every segment's output offset, also for a segment without blocks (it
  // starts where the next block's rows go, or at the total); the barrier
  // above orders these reads after the workgroup's block_out writes
  const int total = carry;
  for (int s = tid; s < S; s += 1024) {
    const int k = cu_blocks[s];
    cu_out[s] = k < NB ? block_out[k] : total;
  }
  if (tid == 0) {
    cu_out[S] = total;
    *num_kept = total;
  }
}

struct GatherArgs {
  const int32_t* cu_seqlens;
  const int32_t* cu_blocks;
  BlockOrigin bo;
  const uint8_t* keep;
  const int32_t* block_out;
  const int32_t* block_seg;
  int32_t* index_map;
  int32_t* cu_out;    // (one-launch path) per-segment output offsets [S+1]
  int32_t* num_kept;  // (one-launch path)
  int S, B, n_rows;
  RowCopy rows[kMaxRowTensors];
};

__device__ inline void copy_range(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                  long nbytes, int part, int nparts) {
  const int tid = threadIdx.x;
  const bool vec = ((((uintptr_t)src) | ((uintptr_t)dst) | (uintptr_t)nbytes) & 15) == 0;
  if (vec) {
    const long n16 = nbytes >> 4;
    const long per = (n16 + nparts - 1) / nparts;
    const long a = part * per, b = min(n16, a + per);
    const uint4* s4 = (const uint4*)src;
    uint4* d4 = (uint4*)dst;
    long i = a + tid;
    for (; i + 3 * 256 < b; i += 4 * 256) {
      const uint4 x0 = s4[i], x1 = s4[i + 256], x2 = s4[i + 512], x3 = s4[i + 768];
      d4[i] = x0;
      d4[i + 256] = x1;
      d4[i + 512] = x2;
      d4[i + 768] = x3;
    }
    for (; i < b; i += 256) d4[i] = s4[i];
  } else if (((((uintptr_t)src) | ((uintptr_t)dst) | (uintptr_t)nbytes) & 3) == 0) {
    const long n4 = nbytes >> 2;
    const long per = (n4 + nparts - 1) / nparts;
    const long a = part * per, b = min(n4, a + per);
    const uint32_t* s4 = (const uint32_t*)src;
    uint32_t* d4 = (uint32_t*)dst;
    for (long i = a + tid; i < b; i += 256) d4[i] = s4[i];
  } else {
    const long per = (nbytes + nparts - 1) / nparts;
    const long a = part * per, b = min(nbytes, a + per);
    for (long i = a + tid; i < b; i += 256) dst[i] = src[i];
  }
}

__global__ __launch_bounds__(256) void compact_gather_kernel(GatherArgs g) {
  const int k = blockIdx.x;
  const int NB = g.cu_blocks[g.S];
  if (k >= NB || !g.keep[k]) return;
  const int s = g.block_seg[k];
  const int n = g.cu_seqlens[s + 1] - g.cu_seqlens[s];
  const int i0 = (k - g.cu_blocks[s]) * g.B - g.bo.of(s);
  if (i0 < 0) return;  // a block of cached tokens: no rows in this call
  const int len = min(g.B, n - i0);
  const int src_row = g.cu_seqlens[s] + i0;
  const int dst_row = g.block_out[k];
  const int part = blockIdx.y, nparts = gridDim.y;
  if (part == 0)
    for (int r = threadIdx.x; r < len; r += 256) g.index_map[dst_row + r] = src_row + r;
  for (int t = 0; t < g.n_rows; ++t) {
    const long rb = g.rows[t].row_bytes;
    copy_range(g.rows[t].src + (long)src_row * rb, g.rows[t].dst + (long)dst_row * rb, len * rb,
               part, nparts);
  }
}

// Kept cached tokens of whole-prompt-scored segments: token u of block k
// goes to slots[block_out[k] + u - first token of k] as its KV slot
// block_table[s][u / 16] * 16 + u % 16 (never past slots_cap).
__global__ __launch_bounds__(256) void kept_cache_slots_kernel(
    const int32_t* __restrict__ cu_blocks, const uint8_t* __restrict__ keep, BlockOrigin bo,
    const int32_t* __restrict__ block_table, int max_pages, int S, int B,
    const int32_t* __restrict__ block_out, const int32_t* __restrict__ block_seg,
    int32_t* __restrict__ slots, int slots_cap) {
  const int k = blockIdx.x;
  if (k >= cu_blocks[S] || !keep[k]) return;
  const int s = block_seg[k];
  const int u0 = (k - cu_blocks[s]) * B;
  const int c = bo.of(s);
  if (u0 >= c) return;  // a block of the segment's own rows
  // only cached tokens (u < c), so the block table is read inside its prefix
  for (int r = threadIdx.x; r < min(B, c - u0); r += 256) {
    const int u = u0 + r, d = block_out[k] + r;
    if (d < slots_cap)
      slots[d] = block_table[(long)s * max_pages + (u >> 4)] * kPageSize + (u & (kPageSize - 1));
  }
}

// One launch, segment scope, NB <= kFusedBlocks (so S <= kFusedBlocks too):
// workgroup (k, part) sums (kept ? length : 0) over blocks j < k itself.
// Every part-0 workgroup writes its segment's output offset when k is the
// segment's first block, and the one of the last block the kept count.
constexpr int kFusedBlocks = 2048;
__global__ __launch_bounds__(256) void compact_fused_kernel(GatherArgs g) {
  __shared__ int32_t cb[kFusedBlocks + 1], cs[kFusedBlocks + 1];
  __shared__ int32_t wsum[4];
  const int k = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int S = g.S, B = g.B;
  for (int i = tid; i <= S; i += 256) {
    cb[i] = g.cu_blocks[i];
    cs[i] = g.cu_seqlens[i];
  }
  __syncthreads();
  const int NB = cb[S];
  if (k >= NB) return;
  // segment of block j, and its kept own rows (segment scope: blocks start
  // at the segment's first token)
  auto seg_of = [&](int j) {
    int lo = 0, hi = S - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (cb[mid] <= j) lo = mid; else hi = mid - 1;
    }
    return lo;
  };
  auto kept_len = [&](int j, int sj) {
    const int i0 = (j - cb[sj]) * B;
    return g.keep[j] ? min(B, cs[sj + 1] - cs[sj] - i0) : 0;
  };
  int part = 0;
  for (int j = tid; j < k; j += 256) part += kept_len(j, seg_of(j));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o, 64);
  if (lane == 0) wsum[wid] = part;
  __syncthreads();
  const int dst_row = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  const int s = seg_of(k);
  const int i0 = (k - cb[s]) * B;
  const int len = kept_len(k, s);
  if (blockIdx.y == 0 && tid == 0) {
    if (k == cb[s]) g.cu_out[s] = dst_row;
    if (k == NB - 1) {
      g.cu_out[S] = dst_row + len;
      *g.num_kept = dst_row + len;
    }
  }
  if (!len) return;
  const int src_row = cs[s] + i0;
  const int p = blockIdx.y, nparts = gridDim.y;
  if (p == 0)
    for (int r = tid; r < len; r += 256) g.index_map[dst_row + r] = src_row + r;
  for (int t = 0; t < g.n_rows; ++t) {
    const long rb = g.rows[t].row_bytes;
    copy_range(g.rows[t].src + (long)src_row * rb, g.rows[t].dst + (long)dst_row * rb, len * rb,
               p, nparts);
  }
}

hipError_t launch_kept_cache_slots(const int32_t* cu_seqlens, const int32_t* cu_blocks,
                                   const uint8_t* keep, const BlockOrigin& bo,
                                   const int32_t* block_table, int max_pages, int S,
                                   int num_blocks, int block_size, int32_t* slots, int slots_cap,
                                   int32_t* cu_out, int32_t* num_out, int32_t* block_out,
                                   int32_t* block_seg, hipStream_t st) {
  hipLaunchKernelGGL(compact_scan_kernel, dim3(1), dim3(1024), 0, st, cu_seqlens, cu_blocks, keep,
                     bo, true, S, block_size, block_out, block_seg, cu_out, num_out);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kept_cache_slots_kernel, dim3(num_blocks), dim3(256), 0, st, cu_blocks, keep,
                     bo, block_table, max_pages, S, block_size, block_out, block_seg, slots,
                     slots_cap);
  return hipGetLastError();
}

hipError_t launch_compact(const int32_t* cu_seqlens, const int32_t* cu_blocks, const BlockOrigin& bo,
                          const uint8_t* keep, int S, int num_blocks, int block_size,
                          const RowCopy* rows, int n_rows, int32_t* index_map,
                          int32_t* cu_seqlens_out, int32_t* num_kept, int32_t* block_out,
                          int32_t* block_seg, hipStream_t st) {
  const bool fused = !bo.prompt_scope && num_blocks <= kFusedBlocks;
  if (!fused) {
    hipLaunchKernelGGL(compact_scan_kernel, dim3(1), dim3(1024), 0, st, cu_seqlens, cu_blocks,
                       keep, bo, false, S, block_size, block_out, block_seg, cu_seqlens_out,
                       num_kept);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  GatherArgs g;
  g.cu_seqlens = cu_seqlens;
  g.cu_blocks = cu_blocks;
  g.bo = bo;
  g.keep = keep;
  g.block_out = block_out;
  g.block_seg = block_seg;
  g.index_map = index_map;
  g.cu_out = cu_seqlens_out;
  g.num_kept = num_kept;
  g.S = S;
  g.B = block_size;
  g.n_rows = n_rows;
  long max_block_bytes = 0;
  for (int i = 0; i < n_rows; ++i) {
    g.rows[i] = rows[i];
    max_block_bytes = max_block_bytes > rows[i].row_bytes * block_size
                          ? max_block_bytes
                          : rows[i].row_bytes * block_size;
  }
  // split each block's copy into ~64 KiB slices
  int parts = (int)((max_block_bytes + 65535) / 65536);
  if (parts < 1) parts = 1;
  if (parts > 64) parts = 64;
  if (fused)
    hipLaunchKernelGGL(compact_fused_kernel, dim3(num_blocks, parts), dim3(256), 0, st, g);
  else
    hipLaunchKernelGGL(compact_gather_kernel, dim3(num_blocks, parts), dim3(256), 0, st, g);
  return hipGetLastError();
}

}  // namespace up
