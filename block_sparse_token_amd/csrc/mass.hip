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
// the attention items stored.  Workgroup (s, y) handles blocks y, y +
// kMassGroups, ... of segment s, 32 heads at a time: thread (row group rg,
// head hl) sums exp2(run - total) over rows rg, rg + 8, ... (totals staged
// in LDS), then the 8 row groups are added in a fixed order.  Runs that
// start after a row's own key are not read (they hold no visible key and
// were not all written).
constexpr int kMassGroups = 32;
__global__ __launch_bounds__(256) void block_mass_kernel(const int32_t* __restrict__ cu_seqlens,
                                                         const uint8_t* __restrict__ score_flags,
                                                         const int32_t* __restrict__ cu_blocks,
                                                         const int32_t* __restrict__ ctx_lens,
                                                         int prompt_scope,
                                                         const float* __restrict__ score_part,
                                                         const float* __restrict__ score_lse,
                                                         int Hq, int B, float* __restrict__ mass) {
  __shared__ float tot[kMaxBlockSize * 32];
  __shared__ float red[8 * 32];
  const int s = blockIdx.x;
  if (!score_flags[s]) return;
  const int n = cu_seqlens[s + 1] - cu_seqlens[s];
  // whole-prompt scoring: blocks from the prompt's first token; off = the
  // cached tokens they cover (a multiple of B, so the last block is the
  // segment's own last block either way)
  const int off = prompt_scope ? ctx_lens[s] : 0;
  const int nb = (off + n + B - 1) / B;
  if ((int)blockIdx.y >= nb) return;
  const int r0 = ((n + B - 1) / B - 1) * B, rows = n - r0;
  const int Q = score_run_len(B), rpb = B / Q;
  const long run_base = (long)cu_blocks[s] * rpb;
  const int tid = threadIdx.x, rg = tid >> 5, hl = tid & 31;
  for (int hc = 0; hc < Hq; hc += 32) {
    const int h = hc + hl;
    __syncthreads();
    for (int x = tid; x < rows * 32; x += 256) {
      const int rl = x >> 5, hh = hc + (x & 31);
      tot[x] = hh < Hq ? score_lse[((long)s * B + rl) * Hq + hh] : 0.f;
    }
    __syncthreads();
    for (int b = blockIdx.y; b < nb; b += kMassGroups) {
      float acc = 0.f;
      if (h < Hq) {
#pragma unroll 4
        for (int rl = rg; rl < rows; rl += 8) {
          const float t = tot[rl * 32 + hl];
          for (int j = 0; j < rpb && b * B + j * Q <= off + r0 + rl; ++j)
            acc += exp2f(score_part[((run_base + b * rpb + j) * B + rl) * Hq + h] - t);
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
      __syncthreads();
    }
  }
}

hipError_t launch_block_mass(const AttnArgs& a, int S, hipStream_t st) {
  hipLaunchKernelGGL(block_mass_kernel, dim3(S, kMassGroups), dim3(256), 0, st, a.cu_seqlens,
                     a.score_flags, a.cu_blocks, a.ctx_lens, a.score_scope, a.score_part,
                     a.score_lse, a.Hq, a.block_size, a.block_mass);
  return hipGetLastError();
}

}  // namespace up
