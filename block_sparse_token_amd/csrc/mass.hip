// Block mass of the scored segments for the bf16 attention path: the
// softmax probability mass that the rows of a segment's last block put on
// each of its own key blocks (UniPrefill review, "Key Terms & Definitions"
// (Top-p Token Selection) and "Method & Key Results": importance per token
// block; the pages give no formula, the reading used is this mass).  The
// attention items store, per last-block row and head, the log2-sum-exp of
// every run of 64, 32 or 16 own keys (the largest dividing the block) and
// the row's total; the mass of
// block b is the sum over rows of exp2(run - total) over b's runs.
#include "common.h"

namespace up {

// Block mass of every scored segment from the run and row log2-sum-exps
// the attention items stored.  One workgroup per block of the call (grid:
// an upper bound on the blocks; workgroups past cu_blocks[S], and those of
// unscored segments, exit at once).  Wave 0 finds the block's segment by a
// 64-way search over cu_blocks; the segment's last-block row totals are
// staged in LDS 32 heads at a time, and thread (row group rg, head hl) sums
// exp2(run - total) over rows rg, rg + 8, ... and the block's runs, every
// load of a row group issued before its sums; the 8 row groups are then
// added in a fixed order (deterministic).  Runs that start after a row's
// own key are not read (they hold no visible key and were not all written).
__global__ __launch_bounds__(256) void block_mass_kernel(const int32_t* __restrict__ cu_seqlens,
                                                         const uint8_t* __restrict__ score_flags,
                                                         const int32_t* __restrict__ cu_blocks,
                                                         const int32_t* __restrict__ ctx_lens,
                                                         int prompt_scope,
                                                         const float* __restrict__ score_part,
                                                         const float* __restrict__ score_lse,
                                                         int Hq, int B, int S,
                                                         float* __restrict__ mass) {
  __shared__ float tot[kMaxBlockSize * 32];
  __shared__ float red[8 * 32];
  __shared__ int seg;
  const int k = blockIdx.x;
  if (k >= cu_blocks[S]) return;
  const int tid = threadIdx.x;
  if (tid < 64) {
    // segment s with cu_blocks[s] <= k < cu_blocks[s+1]: the answer lies in
    // [lo, hi]; each round probes 64 evenly spaced candidates
    int lo = 0, hi = S - 1;
    while (hi > lo) {
      const int step = (hi - lo + 63) / 64;
      const int c = lo + tid * step;
      const bool le = c <= hi && cu_blocks[c] <= k;
      const unsigned long long m = __ballot(le);
      // last probe with cu_blocks[c] <= k (probe 0 = lo always qualifies);
      // the probe after it, if there is one, bounds the answer from above
      const int last = 63 - __clzll((long long)m);
      const int nlo = lo + last * step;
      if (last < 63) hi = min(hi, nlo + step - 1);
      lo = nlo;
    }
    if (tid == 0) seg = lo;
  }
  __syncthreads();
  const int s = seg;
  if (!score_flags[s]) return;
  const int b = k - cu_blocks[s];
  const int n = cu_seqlens[s + 1] - cu_seqlens[s];
  // whole-prompt scoring: blocks from the prompt's first token; off = the
  // cached tokens they cover (a multiple of B, so the last block is the
  // segment's own last block either way)
  const int off = prompt_scope ? ctx_lens[s] : 0;
  const int r0 = ((n + B - 1) / B - 1) * B, rows = n - r0;
  const int Q = score_run_len(B), rpb = B / Q;
  const long run0 = ((long)cu_blocks[s] + b) * rpb;
  const int rg = tid >> 5, hl = tid & 31;
  // runs of block b that start at or before the row's own key: j < nj(rl)
  for (int hc = 0; hc < Hq; hc += 32) {
    const int h = hc + hl;
    __syncthreads();
    for (int x = tid; x < rows * 32; x += 256) {
      const int rl = x >> 5, hh = hc + (x & 31);
      tot[x] = hh < Hq ? score_lse[((long)s * B + rl) * Hq + hh] : 0.f;
    }
    __syncthreads();
    float acc = 0.f;
    if (h < Hq) {
      for (int rl = rg; rl < rows; rl += 8) {
        const float t = tot[rl * 32 + hl];
        const int visible_end = off + r0 + rl;  // the row's own key
        for (int j = 0; j < rpb && b * B + j * Q <= visible_end; ++j)
          acc += exp2f(score_part[((run0 + j) * B + rl) * Hq + h] - t);
      }
    }
    red[tid] = acc;
    __syncthreads();
    if (rg == 0 && h < Hq) {
      float m = 0.f;
#pragma unroll
      for (int g8 = 0; g8 < 8; ++g8) m += red[g8 * 32 + hl];
      mass[((long)cu_blocks[s] + b) * Hq + h] = m;
    }
  }
}

hipError_t launch_block_mass(const AttnArgs& a, int S, int blocks_cap, hipStream_t st) {
  hipLaunchKernelGGL(block_mass_kernel, dim3(blocks_cap), dim3(256), 0, st, a.cu_seqlens,
                     a.score_flags, a.cu_blocks, a.ctx_lens, a.score_scope, a.score_part,
                     a.score_lse, a.Hq, a.block_size, S, a.block_mass);
  return hipGetLastError();
}

}  // namespace up
