// Block scores and top-p block selection.
//
// Scores: the importance of each own block of a scored segment is its
// softmax mass from the segment's last query block summed over heads,
// normalised over the segment's blocks (the pages leave the importance
// measure open; UniPrefill review, "Method & Key Results": importance is
// evaluated per block at a full-attention layer).
//
// Selection (review, "Key Terms & Definitions", Top-p Token Selection): the
// fewest blocks whose cumulative importance reaches p.  The first and last
// blocks are always kept and count toward p; the rest are taken by
// decreasing score, ties to the lower block, while the running sum is below
// the target.  All sums are exact 64-bit integers (q_b = floor(score_b 2^40)),
// so the selection is independent of the order threads add them in.  One
// workgroup per segment finds the cut with an MSB-first radix select on the
// float bit patterns (histograms of q per 8-bit digit in LDS), then resolves
// blocks tied with the cut value by an ascending-index prefix sum.
#include "common.h"

namespace up {

constexpr int kSelThreads = 256;

__device__ inline float block_sum_f(float x, float* sh) {
  // deterministic tree reduction over the workgroup
  const int tid = threadIdx.x;
  sh[tid] = x;
  __syncthreads();
  for (int o = kSelThreads / 2; o > 0; o >>= 1) {
    if (tid < o) sh[tid] += sh[tid + o];
    __syncthreads();
  }
  const float r = sh[0];
  __syncthreads();
  return r;
}

// Scores of segment s (one workgroup).
__device__ inline void segment_scores(const int32_t* __restrict__ cu_blocks,
                                      const uint8_t* __restrict__ flags,
                                      const float* __restrict__ mass, float* __restrict__ scores,
                                      int Hq, int s, float* sh) {
  const int b0 = cu_blocks[s], nb = cu_blocks[s + 1] - b0;
  if (!flags || !flags[s]) {
    for (int k = threadIdx.x; k < nb; k += kSelThreads) scores[b0 + k] = 0.f;
    return;
  }
  float part = 0.f;
  for (int k = threadIdx.x; k < nb; k += kSelThreads) {
    const float* m = mass + (long)(b0 + k) * Hq;
    float mk = 0.f;
    for (int h = 0; h < Hq; ++h) mk += m[h];
    part += mk;
  }
  const float tot = block_sum_f(part, sh);
  for (int k = threadIdx.x; k < nb; k += kSelThreads) {
    const float* m = mass + (long)(b0 + k) * Hq;
    float mk = 0.f;
    for (int h = 0; h < Hq; ++h) mk += m[h];
    scores[b0 + k] = mk / tot;
  }
}

__global__ __launch_bounds__(kSelThreads) void block_scores_kernel(
    const int32_t* __restrict__ cu_blocks, const uint8_t* __restrict__ flags,
    const float* __restrict__ mass, float* __restrict__ scores, int Hq) {
  __shared__ float sh[kSelThreads];
  segment_scores(cu_blocks, flags, mass, scores, Hq, blockIdx.x, sh);
}

hipError_t launch_block_scores(const int32_t* cu_seqlens, const int32_t* cu_blocks,
                               const uint8_t* flags, const float* mass, float* scores, int S,
                               int Hq, hipStream_t st) {
  (void)cu_seqlens;
  hipLaunchKernelGGL(block_scores_kernel, dim3(S), dim3(kSelThreads), 0, st, cu_blocks, flags,
                     mass, scores, Hq);
  return hipGetLastError();
}

__device__ inline uint64_t fx_score(float s) {
  // floor(s * 2^40); s is finite, >= 0 and < 2, so the product is exact
  return (uint64_t)((double)s * 1099511627776.0);
}

struct ToppShared {
  unsigned long long hq[256];
  unsigned long long red[kSelThreads];
  unsigned long long s_need, s_carry;
  uint32_t s_prefix;
  int s_kept;
};

// Keep mask of segment s (one workgroup).
__device__ inline void segment_topp(const int32_t* __restrict__ cu_blocks,
                                    const uint8_t* __restrict__ flags,
                                    const float* __restrict__ scores, uint8_t* __restrict__ keep,
                                    int32_t* __restrict__ kept_blocks, uint32_t p_fx, int keep_all,
                                    int s, ToppShared& S) {
  unsigned long long* hq = S.hq;
  unsigned long long* red = S.red;
  unsigned long long& s_need = S.s_need;
  unsigned long long& s_carry = S.s_carry;
  uint32_t& s_prefix = S.s_prefix;
  int& s_kept = S.s_kept;
  const int tid = threadIdx.x;
  const int b0 = cu_blocks[s], nb = cu_blocks[s + 1] - b0;
  const float* sc = scores + b0;
  uint8_t* kp = keep + b0;
  if (keep_all || !flags || !flags[s] || nb <= 2) {
    for (int k = tid; k < nb; k += kSelThreads) kp[k] = 1;
    if (kept_blocks && tid == 0) kept_blocks[s] = nb;
    return;
  }
  // total Q and the forced blocks' share
  unsigned long long part = 0;
  for (int k = tid; k < nb; k += kSelThreads) part += fx_score(sc[k]);
  red[tid] = part;
  __syncthreads();
  for (int o = kSelThreads / 2; o > 0; o >>= 1) {
    if (tid < o) red[tid] += red[tid + o];
    __syncthreads();
  }
  if (tid == 0) {
    const unsigned long long Q = red[0];
    const unsigned long long target = ((unsigned long long)p_fx * Q + ((1ull << 22) - 1)) >> 22;
    const unsigned long long forced = fx_score(sc[0]) + fx_score(sc[nb - 1]);
    s_need = target > forced ? target - forced : 0ull;
    s_prefix = 0;
    s_kept = 2;
    s_carry = 0;
  }
  for (int k = tid; k < nb; k += kSelThreads) kp[k] = (k == 0 || k == nb - 1) ? 1 : 0;
  __syncthreads();
  if (s_need == 0) {
    if (kept_blocks && tid == 0) kept_blocks[s] = 2;
    return;
  }
  // free blocks' total: if it cannot reach the need, keep everything
  part = 0;
  for (int k = 1 + tid; k < nb - 1; k += kSelThreads) part += fx_score(sc[k]);
  red[tid] = part;
  __syncthreads();
  for (int o = kSelThreads / 2; o > 0; o >>= 1) {
    if (tid < o) red[tid] += red[tid + o];
    __syncthreads();
  }
  if (red[0] < s_need) {
    for (int k = tid; k < nb; k += kSelThreads) kp[k] = 1;
    if (kept_blocks && tid == 0) kept_blocks[s] = nb;
    return;
  }
  __syncthreads();
  // radix select on the score bit patterns, most significant digit first
  const uint32_t* bits = (const uint32_t*)sc;
  uint32_t mask = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int b = tid; b < 256; b += kSelThreads) hq[b] = 0;
    __syncthreads();
    const uint32_t prefix = s_prefix;
    for (int k = 1 + tid; k < nb - 1; k += kSelThreads) {
      const uint32_t key = bits[k];
      if ((key & mask) == prefix) atomicAdd(&hq[(key >> shift) & 255u], fx_score(sc[k]));
    }
    __syncthreads();
    // Highest bin b* with (mass of bins above b*) + hq[b*] >= need, and the
    // mass above it.  Wave 0: lane i holds bins 255-4i .. 252-4i (descending),
    // an exclusive scan over lanes gives each lane the mass above its bins,
    // and the first lane (in bin order) whose bins reach the need decides.
    if (tid < 64) {
      const int lane = tid;
      unsigned long long v[4], loc = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[j] = hq[255 - 4 * lane - j];
        loc += v[j];
      }
      unsigned long long incl = loc;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const unsigned long long y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
      }
      const unsigned long long need = s_need;
      unsigned long long cum = incl - loc;  // mass of all bins above this lane's
      int hit = -1;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (hit < 0 && cum + v[j] >= need) hit = j;
        if (hit < 0) cum += v[j];
      }
      const unsigned long long found = __ballot(hit >= 0);
      // no bin reaches the need: b* = 0 with every bin counted above it
      const int first = found ? __ffsll((long long)found) - 1 : 63;
      if (lane == first) {
        const int bstar = hit >= 0 ? 255 - 4 * lane - hit : 0;
        s_need = need - cum;
        s_prefix = prefix | ((uint32_t)bstar << shift);
      }
    }
    mask |= 255u << shift;
    __syncthreads();
  }
  const uint32_t cut = s_prefix;
  const unsigned long long need_tie = s_need;  // still needed from blocks equal to cut
  // blocks strictly above the cut are kept; ties in ascending index order
  int kept_local = 0;
  for (int base = 1; base < nb - 1; base += kSelThreads) {
    const int k = base + tid;
    unsigned long long v = 0;
    bool tie = false;
    if (k < nb - 1) {
      const uint32_t key = bits[k];
      if (key > cut) {
        kp[k] = 1;
        ++kept_local;
      } else if (key == cut) {
        tie = true;
        v = fx_score(sc[k]);
      }
    }
    // exclusive scan of tie values in index order
    red[tid] = v;
    __syncthreads();
    for (int o = 1; o < kSelThreads; o <<= 1) {
      const unsigned long long y = tid >= o ? red[tid - o] : 0ull;
      __syncthreads();
      red[tid] += y;
      __syncthreads();
    }
    const unsigned long long excl = s_carry + red[tid] - v;
    if (tie && excl < need_tie) {
      kp[k] = 1;
      ++kept_local;
    }
    __syncthreads();
    if (tid == kSelThreads - 1) s_carry += red[tid];
    __syncthreads();
  }
  if (kept_local) atomicAdd(&s_kept, kept_local);
  __syncthreads();
  if (kept_blocks && tid == 0) kept_blocks[s] = s_kept;
}

__global__ __launch_bounds__(kSelThreads) void topp_kernel(const int32_t* __restrict__ cu_blocks,
                                                         const uint8_t* __restrict__ flags,
                                                         const float* __restrict__ scores,
                                                         uint8_t* __restrict__ keep,
                                                         int32_t* __restrict__ kept_blocks,
                                                         uint32_t p_fx, int keep_all) {
  __shared__ ToppShared sh;
  segment_topp(cu_blocks, flags, scores, keep, kept_blocks, p_fx, keep_all, blockIdx.x, sh);
}

// Scores and selection of one segment in one workgroup: the scores it
// writes are read back by the same workgroup after a barrier (a
// workgroup-scope release and acquire, so every thread sees them).
__global__ __launch_bounds__(kSelThreads) void score_select_kernel(
    const int32_t* __restrict__ cu_blocks, const uint8_t* __restrict__ flags,
    const float* __restrict__ mass, float* __restrict__ scores, int Hq,
    uint8_t* __restrict__ keep, int32_t* __restrict__ kept_blocks, uint32_t p_fx, int keep_all) {
  __shared__ float shf[kSelThreads];
  __shared__ ToppShared sh;
  segment_scores(cu_blocks, flags, mass, scores, Hq, blockIdx.x, shf);
  __syncthreads();
  segment_topp(cu_blocks, flags, scores, keep, kept_blocks, p_fx, keep_all, blockIdx.x, sh);
}

hipError_t launch_score_select(const int32_t* cu_blocks, const uint8_t* flags, const float* mass,
                               float* scores, int Hq, uint8_t* keep, int32_t* kept_blocks, int S,
                               uint32_t p_fx, int keep_all, hipStream_t st) {
  hipLaunchKernelGGL(score_select_kernel, dim3(S), dim3(kSelThreads), 0, st, cu_blocks, flags,
                     mass, scores, Hq, keep, kept_blocks, p_fx, keep_all);
  return hipGetLastError();
}

hipError_t launch_topp(const int32_t* cu_blocks, const uint8_t* flags, const float* scores,
                       uint8_t* keep, int32_t* kept_blocks, int S, uint32_t p_fx, int keep_all,
                       hipStream_t st) {
  hipLaunchKernelGGL(topp_kernel, dim3(S), dim3(kSelThreads), 0, st, cu_blocks, flags, scores,
                     keep, kept_blocks, p_fx, keep_all);
  return hipGetLastError();
}

}  // namespace up
