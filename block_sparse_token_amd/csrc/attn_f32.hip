// float32 path of the attention operator (one thread per packed query row,
// fp32 FMA dot products, exact expf).  Same semantics, work list, key
// addressing and fused block mass as the bf16 matrix-core kernel; it serves
// the small fp32 workloads where the tolerance is relative 1e-5.
#include "common.h"

namespace up {

template <int D>
struct CfgF {
  static constexpr int THREADS = 128;  // packed rows per workgroup
  static constexpr int BN = 32;        // keys per tile
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = BN * D * 4;
  static constexpr int POS_OFF = V_OFF + BN * D * 4;
  static constexpr int RED_OFF = POS_OFF + BN * 4;
  static constexpr int RED_BYTES = THREADS * 2 * 4;
  static constexpr int LDS_BYTES = RED_OFF + RED_BYTES;
};

constexpr int kPosInv = 0x7fffffff;

struct SegF {
  int s, q0, n, c;
};

__device__ inline long cache_row_f(const AttnArgs& a, const SegF& sg, int g, int u, int D) {
  int page, off;
  if (u < sg.c) {
    page = a.block_table[(long)sg.s * a.max_pages + (u >> 4)];
    off = u & 15;
  } else {
    const int slot = a.slot_mapping[sg.q0 + u - sg.c];
    page = slot >> 4;
    off = slot & 15;
  }
  return (((long)page * a.Hkv + g) * kPageSize + off) * (long)D;
}

template <int D, bool kWithV>
__device__ inline void stage_tile_f(const AttnArgs& a, const SegF& sg, int g, int u0, int u_end,
                                    char* lds) {
  const float* kc = (const float*)a.k_cache;
  const float* vc = (const float*)a.v_cache;
  float* sK = (float*)(lds + CfgF<D>::K_OFF);
  float* sV = (float*)(lds + CfgF<D>::V_OFF);
  int* sP = (int*)(lds + CfgF<D>::POS_OFF);
  constexpr int BN = CfgF<D>::BN;
  for (int idx = threadIdx.x; idx < BN * D / 4; idx += CfgF<D>::THREADS) {
    const int kk = idx / (D / 4), c4 = idx % (D / 4);
    const int u = u0 + kk;
    float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
    if (u < u_end) {
      const long row = cache_row_f(a, sg, g, u, D);
      kv = *(const float4*)(kc + row + c4 * 4);
      if (kWithV) vv = *(const float4*)(vc + row + c4 * 4);
    }
    *(float4*)(sK + kk * D + c4 * 4) = kv;
    if (kWithV) *(float4*)(sV + kk * D + c4 * 4) = vv;
  }
  for (int kk = threadIdx.x; kk < BN; kk += CfgF<D>::THREADS) {
    const int u = u0 + kk;
    sP[kk] = u >= u_end ? kPosInv : (u < sg.c ? u : a.positions[sg.q0 + u - sg.c]);
  }
}

template <int D>
__device__ inline void load_q_f(const AttnArgs& a, long qrow, bool valid, int pos, float (&q)[D]) {
  const float* src = (const float*)a.q;
  for (int d = 0; d < D; ++d) q[d] = valid ? src[qrow + d] : 0.f;
  if (a.rope && valid) {
    for (int j = 0; j < D / 2; ++j) {
      double t = (double)pos * a.rope_rev[j];
      t -= rint(t);
      float s, c;
      sincosf((float)(t * 6.283185307179586476925286766559), &s, &c);
      const float x1 = q[j], x2 = q[j + D / 2];
      q[j] = x1 * c - x2 * s;
      q[j + D / 2] = x2 * c + x1 * s;
    }
  }
}

__device__ inline bool visible_f(int kp, int qp, int window) {
  return kp <= qp && (window <= 0 || kp > qp - window);
}

// first virtual key index whose position is >= target (serial binary search)
__device__ inline int first_key_f(const AttnArgs& a, const SegF& sg, int target) {
  if (target <= 0) return 0;
  if (target <= sg.c) return target;
  int lo = 0, hi = min(sg.n, target - sg.c);
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a.positions[sg.q0 + mid] >= target) hi = mid; else lo = mid + 1;
  }
  return sg.c + lo;
}

template <int D>
__device__ void attn_item_f(const AttnArgs& a, int s, int jt, int g, char* lds) {
  constexpr int BN = CfgF<D>::BN;
  SegF sg;
  sg.s = s;
  sg.q0 = a.cu_seqlens[s];
  sg.n = a.cu_seqlens[s + 1] - sg.q0;
  sg.c = a.ctx_lens[s];
  const int G = a.G;
  const int P = CfgF<D>::THREADS / G;
  const int r = threadIdx.x;
  const int i_first = jt * P;
  const int i_last = min(sg.n, i_first + P) - 1;
  const int i = i_first + r / G, hh = r % G;
  const bool valid = (r < P * G) && (i <= i_last);
  const int qp = valid ? a.positions[sg.q0 + i] : -1;
  const long qrow = ((long)(sg.q0 + i) * a.Hq + g * G + hh) * D;
  float q[D], acc[D];
  load_q_f<D>(a, qrow, valid, qp, q);
  for (int d = 0; d < D; ++d) acc[d] = 0.f;
  float m = -INFINITY, l = 0.f;
  const int u_end = sg.c + i_last + 1;
  int u_lo = 0;
  if (a.window > 0) u_lo = first_key_f(a, sg, a.positions[sg.q0 + i_first] - a.window + 1);
  const float* sK = (const float*)(lds + CfgF<D>::K_OFF);
  const float* sV = (const float*)(lds + CfgF<D>::V_OFF);
  const int* sP = (const int*)(lds + CfgF<D>::POS_OFF);
  for (int u0 = (u_lo / BN) * BN; u0 < u_end; u0 += BN) {
    __syncthreads();
    stage_tile_f<D, true>(a, sg, g, u0, u_end, lds);
    __syncthreads();
    float sc[BN];
    float mx = -INFINITY;
    for (int kk = 0; kk < BN; ++kk) {
      float dot = 0.f;
      for (int d = 0; d < D; ++d) dot = fmaf(q[d], sK[kk * D + d], dot);
      dot *= a.scale;
      if (!visible_f(sP[kk], qp, a.window)) dot = -INFINITY;
      sc[kk] = dot;
      mx = fmaxf(mx, dot);
    }
    if (mx == -INFINITY) continue;  // nothing visible to this row in the tile
    const float mnew = fmaxf(m, mx);
    const float alpha = expf(m - mnew);  // 0 when m = -inf
    for (int d = 0; d < D; ++d) acc[d] *= alpha;
    l *= alpha;
    for (int kk = 0; kk < BN; ++kk) {
      const float p = expf(sc[kk] - mnew);
      l += p;
      for (int d = 0; d < D; ++d) acc[d] = fmaf(p, sV[kk * D + d], acc[d]);
    }
    m = mnew;
  }
  if (!valid) return;
  float* out = (float*)a.out;
  const float inv = 1.f / l;
  for (int d = 0; d < D; ++d) out[qrow + d] = acc[d] * inv;
  if (a.lse) a.lse[qrow / D] = m + logf(l);
}

template <int D>
__device__ void score_item_f(const AttnArgs& a, int s, int g, char* lds) {
  constexpr int BN = CfgF<D>::BN;
  constexpr int NT = CfgF<D>::THREADS;
  SegF sg;
  sg.s = s;
  sg.q0 = a.cu_seqlens[s];
  sg.n = a.cu_seqlens[s + 1] - sg.q0;
  sg.c = a.ctx_lens[s];
  const int G = a.G, B = a.block_size;
  const int nb = (sg.n + B - 1) / B;
  const int r0 = (nb - 1) * B;
  const int rows_total = (sg.n - r0) * G;
  // a pass covers whole tokens (NTG rows, a multiple of G), so thread t
  // holds head t % G in every pass
  const int NTG = (NT / G) * G;
  const int passes = (rows_total + NTG - 1) / NTG;
  const long mbase = a.cu_blocks[s];
  const float* sK = (const float*)(lds + CfgF<D>::K_OFF);
  const int* sP = (const int*)(lds + CfgF<D>::POS_OFF);
  float* red = (float*)(lds + CfgF<D>::RED_OFF);
  // a tile of BN = 32 own keys aligned to the segment start meets at most
  // two blocks (block sizes are multiples of 16)
  for (int ps = passes - 1; ps >= 0; --ps) {
    const int rbeg = ps * NTG, rend = min(rows_total, rbeg + NTG);
    const int r = rbeg + threadIdx.x;
    const bool valid = r < rend;
    const int i = r0 + r / G, hh = r % G;
    const int i_first = r0 + rbeg / G, i_last = r0 + (rend - 1) / G;
    const int qp = valid ? a.positions[sg.q0 + i] : -1;
    const long qrow = ((long)(sg.q0 + i) * a.Hq + g * G + hh) * D;
    float q[D];
    load_q_f<D>(a, qrow, valid, qp, q);
    const int u_end = sg.c + i_last + 1;
    int u_lo = 0;
    if (a.window > 0) u_lo = first_key_f(a, sg, a.positions[sg.q0 + i_first] - a.window + 1);
    float m = -INFINITY, l = 0.f;
    for (int u0 = (u_lo / BN) * BN; u0 < u_end; u0 += BN) {
      __syncthreads();
      stage_tile_f<D, false>(a, sg, g, u0, u_end, lds);
      __syncthreads();
      for (int kk = 0; kk < BN; ++kk) {
        float dot = 0.f;
        for (int d = 0; d < D; ++d) dot = fmaf(q[d], sK[kk * D + d], dot);
        dot *= a.scale;
        if (!visible_f(sP[kk], qp, a.window)) continue;
        if (dot > m) {
          l = l * expf(m - dot) + 1.f;
          m = dot;
        } else {
          l += expf(dot - m);
        }
      }
    }
    const float inv = valid ? 1.f / l : 0.f;
    const int own_end = i_last + 1;
    const int n_tiles = (own_end + BN - 1) / BN;
    for (int mt = 0; mt < n_tiles; ++mt) {
      const int u0 = sg.c + mt * BN;
      __syncthreads();
      stage_tile_f<D, false>(a, sg, g, u0, u_end, lds);
      __syncthreads();
      float part[2] = {0.f, 0.f};
      if (valid) {
        for (int kk = 0; kk < BN; ++kk) {
          if (!visible_f(sP[kk], qp, a.window)) continue;
          float dot = 0.f;
          for (int d = 0; d < D; ++d) dot = fmaf(q[d], sK[kk * D + d], dot);
          dot *= a.scale;
          const float p = expf(dot - m) * inv;
          const int bt = (mt * BN + kk) / B - (mt * BN) / B;
          if (bt == 0) part[0] += p; else part[1] += p;
        }
      }
      red[threadIdx.x * 2 + 0] = part[0];
      red[threadIdx.x * 2 + 1] = part[1];
      __syncthreads();
      if ((int)threadIdx.x < 2 * G) {
        const int bt = threadIdx.x / G, h2 = threadIdx.x % G;
        float tot = 0.f;
        for (int t = h2; t < NT; t += G) tot += red[t * 2 + bt];  // fixed order
        const int kb = (mt * BN) / B + bt;
        // the block's keys in this tile (bt = 1 only if a block starts inside it)
        const bool here = bt == 0 || kb * B < min((mt + 1) * BN, own_end);
        if (kb < nb && here) {
          float* dst = a.block_mass + (mbase + kb) * a.Hq + g * G + h2;
          // first contribution: the pass processed first, the tile holding
          // the block's first key
          const bool first = (ps == passes - 1) && kb * B >= mt * BN;
          if (first) *dst = tot;
          else *dst += tot;
        }
      }
    }
    __syncthreads();
  }
}

template <int D>
__global__ __launch_bounds__(128) void attn_f32_kernel(AttnArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int item = blockIdx.x / a.Hkv;
  const int g = blockIdx.x % a.Hkv;
  if (item >= *a.item_count) return;
  const int2 it = a.items[item];
  if (it.y == kScoreTile) score_item_f<D>(a, it.x, g, lds);
  else attn_item_f<D>(a, it.x, it.y, g, lds);
}

int attn_f32_positions_per_tile(int D, int G) {
  (void)D;
  return 128 / G;
}

hipError_t launch_attn_f32(const AttnArgs& a, int D, int capacity, hipStream_t st) {
  dim3 grid((unsigned)capacity * a.Hkv);
  if (D == 128)
    hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(128), CfgF<128>::LDS_BYTES, st, a);
  else
    hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(128), CfgF<64>::LDS_BYTES, st, a);
  return hipGetLastError();
}

}  // namespace up
