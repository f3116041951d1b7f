// Packed, paged, chunked causal attention on bf16 matrix cores (gfx950), with
// the block-importance mass of each scored segment fused into the same
// launch.
//
// What is computed (UniPrefill review, "Method & Key Results"; glossary page
// "Chunked Prefill", "How chunked prefill works"; Prepacking summary,
// "Technical framework"): each token attends the cached keys of its own
// prompt plus its segment's keys at positions <= its own (optionally inside
// a sliding window), never keys of other packed segments.
//
// Layout of the work:
//  * GQA packing: for KV head g the query rows of heads g*G .. g*G+G-1 are
//    interleaved, packed row r = local_token * G + head_in_group.  A
//    workgroup (4 waves) owns 128*RB consecutive packed rows, so every K/V
//    tile staged in LDS feeds all G query heads that read it.
//  * A wave owns RB blocks of 32 packed rows.  S^T = K Q^T and O^T = V^T P^T
//    run on v_mfma_f32_32x32x16_bf16: the S^T accumulator already holds, per
//    lane, 16 keys of one query row, which is the B-operand layout P^T needs
//    once keys are permuted within each 16-key step (V^T is stored in LDS
//    with the same permutation).  Row statistics (max, sum) therefore live in
//    one lane pair (l, l^32).
//  * Keys are addressed through the page table (cached prefix) or the slot
//    of each own token, so the same kernel serves packed prefill, chunked
//    prefill over a paged cache, decodes and gapped positions after
//    compaction.
//  * Score items: for a scored segment and KV head, a first QK^T sweep over
//    every visible key gives the exact softmax normaliser of the rows of the
//    segment's last query block; a second sweep over the segment's own keys
//    sums those probabilities per key block.  The result is written to
//    block_mass[block, head] in a fixed order (deterministic).
#include "common.h"

namespace up {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int D_, int RB_>
struct Cfg {
  static constexpr int D = D_;
  static constexpr int RB = RB_;
  static constexpr int NW = 4;
  static constexpr int ROWS = 32 * RB * NW;  // packed rows per workgroup
  static constexpr int BN = 64;              // keys per tile
  static constexpr int KC = D / 16;          // 16-wide d steps (QK^T)
  static constexpr int DB = D / 32;          // 32-wide d blocks (PV)
  static constexpr int KSTR = D * 2 + 16;    // LDS bytes per K row
  static constexpr int VSTR = BN * 2 + 16;   // LDS bytes per V^T row
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = K_OFF + BN * KSTR;
  static constexpr int POS_OFF = V_OFF + D * VSTR;
  static constexpr int RED_OFF = POS_OFF + BN * 4;
  static constexpr int RED_BYTES = NW * 4 * 32 * 4;  // [wave][block in tile][head] f32
  static constexpr int MISC_OFF = RED_OFF + RED_BYTES;
  static constexpr int LDS_BYTES = MISC_OFF + 64;
  static constexpr int KCH = D / 32;  // 16-byte chunks of K per thread per tile
};

constexpr int kPosInvalid = 0x7fffffff;
constexpr float kNegBig = -1.0e30f;

struct Seg {
  int s, q0, n, c;
};

__device__ inline long cache_row(const AttnArgs& a, const Seg& sg, int g, int u, int D) {
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

__device__ inline int key_position(const AttnArgs& a, const Seg& sg, int u) {
  return u < sg.c ? u : a.positions[sg.q0 + u - sg.c];
}

// First virtual key index u in [0, c + n) whose position is >= target.
// Positions are increasing in u and pos(u) >= u.  Wave-cooperative 64-ary
// search; every lane returns the same value.
__device__ inline int first_key_at_or_after(const AttnArgs& a, const Seg& sg, int target) {
  if (target <= 0) return 0;
  if (target <= sg.c) return target;
  // Own index j: the answer lies in [lo, hi]; j = hi is known to qualify
  // (pos(c + j) >= c + j), every probe at or beyond hi counts as qualifying.
  int lo = 0, hi = min(sg.n, target - sg.c);
  const int lane = threadIdx.x & 63;
  while (hi > lo) {
    const int step = (hi - lo + 63) / 64;
    const int j = lo + lane * step;
    bool ge = true;
    if (j < hi) ge = a.positions[sg.q0 + j] >= target;
    const unsigned long long m = __ballot(ge);
    // first qualifying probe; 64 stands for the probe at hi
    const int first = m ? __ffsll((long long)m) - 1 : 64;
    if (first == 0) {
      hi = lo;
    } else {
      const int nlo = lo + (first - 1) * step + 1;
      hi = min(hi, lo + first * step);
      lo = nlo;
    }
  }
  return sg.c + lo;
}

// ----------------------------------------------------------------------------
// tile staging: global -> registers -> LDS
// ----------------------------------------------------------------------------
template <class C>
struct TileRegs {
  uint4 k[C::KCH];
  uint4 v[4];
  int pos;
};

template <class C, bool kWithV>
__device__ inline void tile_load(const AttnArgs& a, const Seg& sg, int g, int u0, int u_end,
                                 TileRegs<C>& r) {
  const int tid = threadIdx.x;
  const uint16_t* kc = (const uint16_t*)a.k_cache;
  const uint16_t* vc = (const uint16_t*)a.v_cache;
  {  // K: key tid/4, bytes [part * D/2, +D/2) of its row
    const int kk = tid >> 2, part = tid & 3;
    const int u = u0 + kk;
    if (u < u_end) {
      const long row = cache_row(a, sg, g, u, C::D);
      const uint4* src = (const uint4*)(kc + row + part * (C::D / 4));
#pragma unroll
      for (int i = 0; i < C::KCH; ++i) r.k[i] = src[i];
    } else {
#pragma unroll
      for (int i = 0; i < C::KCH; ++i) r.k[i] = make_uint4(0, 0, 0, 0);
    }
  }
  if (kWithV) {  // V: keys quad*4 .. +3, d in [octet*8, +8)
    if (tid < 2 * C::D) {
      const int quad = (tid & 63) >> 2, octet = (tid >> 6) * 4 + (tid & 3);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int u = u0 + quad * 4 + e;
        if (u < u_end) {
          const long row = cache_row(a, sg, g, u, C::D);
          r.v[e] = *(const uint4*)(vc + row + octet * 8);
        } else {
          r.v[e] = make_uint4(0, 0, 0, 0);
        }
      }
    }
  }
  if (tid < C::BN) {
    const int u = u0 + tid;
    r.pos = u < u_end ? key_position(a, sg, u) : kPosInvalid;
  }
}

// key index within a 16-key step -> LDS column of V^T (quads 0,1,2,3 -> 0,2,1,3)
__device__ inline int vt_col(int kk) {
  const int q = (kk >> 2) & 3;
  const int cq = ((q & 1) << 1) | (q >> 1);
  return (kk & ~15) | (cq << 2) | (kk & 3);
}

template <class C, bool kWithV>
__device__ inline void tile_store(char* lds, const TileRegs<C>& r) {
  const int tid = threadIdx.x;
  {
    const int kk = tid >> 2, part = tid & 3;
    uint4* dst = (uint4*)(lds + C::K_OFF + kk * C::KSTR + part * (C::D / 2) * 1);
#pragma unroll
    for (int i = 0; i < C::KCH; ++i) dst[i] = r.k[i];
  }
  if (kWithV && tid < 2 * C::D) {
    const int quad = (tid & 63) >> 2, octet = (tid >> 6) * 4 + (tid & 3);
    const int col = vt_col(quad * 4);  // 4 consecutive keys stay together
    // r.v[e] holds d = octet*8 .. +7 of key quad*4+e; write V^T[d][col + e]
    const uint16_t* ve[4] = {(const uint16_t*)&r.v[0], (const uint16_t*)&r.v[1],
                             (const uint16_t*)&r.v[2], (const uint16_t*)&r.v[3]};
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      uint2 w;
      w.x = (uint32_t)ve[0][x] | ((uint32_t)ve[1][x] << 16);
      w.y = (uint32_t)ve[2][x] | ((uint32_t)ve[3][x] << 16);
      *(uint2*)(lds + C::V_OFF + (octet * 8 + x) * C::VSTR + col * 2) = w;
    }
  }
  if (tid < C::BN) ((int*)(lds + C::POS_OFF))[tid] = r.pos;
}

// ----------------------------------------------------------------------------
// Q fragments with rotary embedding
// ----------------------------------------------------------------------------
// Lane l (h = l / 32) of row-block rb holds, for d-step kc, q[row][kc*16 + h*8 + e].
template <class C>
__device__ inline void load_q(const AttnArgs& a, long qrow_elem, bool valid, int pos,
                              bf16x8 (&qf)[C::KC]) {
  const int h = (threadIdx.x & 63) >> 5;
  const uint16_t* q = (const uint16_t*)a.q;
  float x[C::KC][8];
#pragma unroll
  for (int kc = 0; kc < C::KC; ++kc) {
    uint4 raw = make_uint4(0, 0, 0, 0);
    if (valid) raw = *(const uint4*)(q + qrow_elem + kc * 16 + h * 8);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[kc][2 * e] = __uint_as_float(w[e] << 16);
      x[kc][2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
  }
  if (a.rope && valid) {
#pragma unroll
    for (int kc = 0; kc < C::KC / 2; ++kc) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = kc * 16 + h * 8 + e;
        double t = (double)pos * a.rope_rev[j];
        t -= rint(t);
        const float s = __builtin_amdgcn_sinf((float)t);
        const float c = __builtin_amdgcn_cosf((float)t);
        const float x1 = x[kc][e], x2 = x[kc + C::KC / 2][e];
        x[kc][e] = x1 * c - x2 * s;
        x[kc + C::KC / 2][e] = x2 * c + x1 * s;
      }
    }
  }
#pragma unroll
  for (int kc = 0; kc < C::KC; ++kc)
#pragma unroll
    for (int e = 0; e < 8; ++e) qf[kc][e] = (__bf16)x[kc][e];
}

// ----------------------------------------------------------------------------
// S^T = K Q^T for one 64-key tile: s[rb][mb], mb = 32-key half of the tile
// ----------------------------------------------------------------------------
template <class C>
__device__ inline void qk_tile(const char* lds, const bf16x8 (&qf)[C::RB][C::KC],
                               f32x16 (&s)[C::RB][2]) {
  const int l = threadIdx.x & 63, h = l >> 5, kr = l & 31;
#pragma unroll
  for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[rb][mb][i] = 0.f;
#pragma unroll
  for (int kc = 0; kc < C::KC; ++kc) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const bf16x8 kf =
          *(const bf16x8*)(lds + C::K_OFF + (mb * 32 + kr) * C::KSTR + (kc * 16 + h * 8) * 2);
#pragma unroll
      for (int rb = 0; rb < C::RB; ++rb)
        s[rb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[rb][kc], s[rb][mb], 0, 0, 0);
    }
  }
}

// Visibility mask of this lane's 32 keys for one row.
template <class C>
__device__ inline void apply_mask(const char* lds, int qpos, int window, f32x16 (&s)[2]) {
  const int l = threadIdx.x & 63, h = l >> 5;
  const int* kp = (const int*)(lds + C::POS_OFF);
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int jg = 0; jg < 4; ++jg) {
      const int4 p4 = *(const int4*)(kp + mb * 32 + jg * 8 + h * 4);
      const int pp[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bool vis = pp[e] <= qpos;
        if (window > 0) vis = vis && (pp[e] > qpos - window);
        if (!vis) s[mb][jg * 4 + e] = -INFINITY;
      }
    }
  }
}

__device__ inline float wave_pair_max(float x) {
  return fmaxf(x, __shfl_xor(x, 32, 64));
}

// ----------------------------------------------------------------------------
// attention item: one query tile of one segment, one KV head
// ----------------------------------------------------------------------------
template <class C>
__device__ void attn_item(const AttnArgs& a, int s, int jt, int g, char* lds) {
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, h = l >> 5;
  Seg sg;
  sg.s = s;
  sg.q0 = a.cu_seqlens[s];
  sg.n = a.cu_seqlens[s + 1] - sg.q0;
  sg.c = a.ctx_lens[s];
  const int G = a.G;
  const int P = C::ROWS / G;
  const int i_first = jt * P;
  const int i_last = min(sg.n, i_first + P) - 1;

  int qpos[C::RB];
  bool rvalid[C::RB];
  long qrow[C::RB];
  bf16x8 qf[C::RB][C::KC];
#pragma unroll
  for (int rb = 0; rb < C::RB; ++rb) {
    const int r = (w * C::RB + rb) * 32 + (l & 31);
    const int i = i_first + r / G, hh = r % G;
    rvalid[rb] = (r < P * G) && (i <= i_last);
    qpos[rb] = rvalid[rb] ? a.positions[sg.q0 + i] : -1;
    qrow[rb] = ((long)(sg.q0 + i) * a.Hq + g * G + hh) * C::D;
    load_q<C>(a, qrow[rb], rvalid[rb], qpos[rb], qf[rb]);
  }
  const int pos_first = a.positions[sg.q0 + i_first];
  const int pos_last = a.positions[sg.q0 + i_last];
  const int u_end = sg.c + i_last + 1;
  int u_lo = 0;
  if (a.window > 0) {
    int* misc = (int*)(lds + C::MISC_OFF);
    if (w == 0) {
      const int r = first_key_at_or_after(a, sg, pos_first - a.window + 1);
      if (l == 0) misc[0] = r;
    }
    __syncthreads();
    u_lo = misc[0];
    __syncthreads();
  }

  f32x16 o[C::RB][C::DB];
  float m[C::RB], lsum[C::RB];
#pragma unroll
  for (int rb = 0; rb < C::RB; ++rb) {
    m[rb] = kNegBig;
    lsum[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[rb][db][i] = 0.f;
  }
  const float sl2 = a.scale_log2;

  TileRegs<C> regs;
  const int t0 = (u_lo / C::BN) * C::BN;
  tile_load<C, true>(a, sg, g, t0, u_end, regs);
  for (int u0 = t0; u0 < u_end; u0 += C::BN) {
    __syncthreads();
    tile_store<C, true>(lds, regs);
    __syncthreads();
    if (u0 + C::BN < u_end) tile_load<C, true>(a, sg, g, u0 + C::BN, u_end, regs);

    f32x16 sacc[C::RB][2];
    qk_tile<C>(lds, qf, sacc);
    const int kpos0 = ((const int*)(lds + C::POS_OFF))[0];
    const bool full = (u0 + C::BN - 1 <= sg.c + i_first) &&
                      (a.window <= 0 || kpos0 > pos_last - a.window);
    bf16x8 pf[C::RB][4];
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb) {
      if (!full) apply_mask<C>(lds, qpos[rb], a.window, sacc[rb]);
      float mx = kNegBig;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[rb][mb][i]);
      mx = wave_pair_max(mx);
      const float mnew = fmaxf(m[rb], mx);
      const float alpha = __builtin_amdgcn_exp2f((m[rb] - mnew) * sl2);
      m[rb] = mnew;
      const float mb2 = mnew * sl2;
      float rs = 0.f;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = __builtin_amdgcn_exp2f(sacc[rb][mb][i] * sl2 - mb2);
          sacc[rb][mb][i] = p;
          rs += p;
        }
      lsum[rb] = lsum[rb] * alpha + rs;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[rb][db][i] *= alpha;
      // P^T B-operand for 16-key step ks: regs (ks%2)*8 .. +8 of half ks/2
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[rb][ks][e] = (__bf16)sacc[rb][ks >> 1][(ks & 1) * 8 + e];
    }
    // O^T += V^T P^T
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const bf16x8 vf = *(const bf16x8*)(lds + C::V_OFF + (db * 32 + (l & 31)) * C::VSTR +
                                           (ks * 16 + h * 8) * 2);
#pragma unroll
        for (int rb = 0; rb < C::RB; ++rb)
          o[rb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[rb][ks], o[rb][db], 0, 0, 0);
      }
    }
  }

  // epilogue: normalise and store rows; lane holds d = db*32 + jg*8 + h*4 + e
  uint16_t* out = (uint16_t*)a.out;
#pragma unroll
  for (int rb = 0; rb < C::RB; ++rb) {
    const float ltot = lsum[rb] + __shfl_xor(lsum[rb], 32, 64);
    if (!rvalid[rb]) continue;
    const float inv = 1.f / ltot;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        bf16x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(o[rb][db][jg * 4 + e] * inv);
        *(bf16x4*)(out + qrow[rb] + db * 32 + jg * 8 + h * 4) = v4;
      }
    if (a.lse && h == 0) {
      const long row = qrow[rb] / C::D;
      a.lse[row] = (m[rb] * sl2 + __log2f(ltot)) * 0.69314718055994530942f;
    }
  }
}

// ----------------------------------------------------------------------------
// score item: block mass of the last query block of segment s, KV head g
// ----------------------------------------------------------------------------
template <class C>
__device__ void score_item(const AttnArgs& a, int s, int g, char* lds) {
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, h = l >> 5;
  Seg sg;
  sg.s = s;
  sg.q0 = a.cu_seqlens[s];
  sg.n = a.cu_seqlens[s + 1] - sg.q0;
  sg.c = a.ctx_lens[s];
  const int G = a.G, B = a.block_size;
  const int nb = (sg.n + B - 1) / B;
  const int r0 = (nb - 1) * B;
  const int rows_total = (sg.n - r0) * G;
  const int passes = (rows_total + C::ROWS - 1) / C::ROWS;
  const long mbase = (long)a.cu_blocks[s];
  const float sl2 = a.scale_log2;
  float* red = (float*)(lds + C::RED_OFF);
  const int nbt = B >= 64 ? 1 : 64 / B;  // blocks per 64-key tile

  for (int ps = passes - 1; ps >= 0; --ps) {
    const int rbeg = ps * C::ROWS;
    const int rend = min(rows_total, rbeg + C::ROWS);
    const int i_first = r0 + rbeg / G;
    const int i_last = r0 + (rend - 1) / G;
    int qpos[C::RB];
    bool rvalid[C::RB];
    bf16x8 qf[C::RB][C::KC];
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb) {
      const int r = rbeg + (w * C::RB + rb) * 32 + (l & 31);
      const int i = r0 + r / G, hh = r % G;
      rvalid[rb] = r < rend;
      qpos[rb] = rvalid[rb] ? a.positions[sg.q0 + i] : -1;
      const long qrow = ((long)(sg.q0 + i) * a.Hq + g * G + hh) * C::D;
      load_q<C>(a, qrow, rvalid[rb], qpos[rb], qf[rb]);
    }
    const int pos_first = a.positions[sg.q0 + i_first];
    const int u_end = sg.c + i_last + 1;
    int u_lo = 0;
    if (a.window > 0) {
      int* misc = (int*)(lds + C::MISC_OFF);
      if (w == 0) {
        const int r = first_key_at_or_after(a, sg, pos_first - a.window + 1);
        if (l == 0) misc[0] = r;
      }
      __syncthreads();
      u_lo = misc[0];
      __syncthreads();
    }
    // sweep 1: row max and normaliser over all visible keys
    float m[C::RB], lsum[C::RB];
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb) {
      m[rb] = kNegBig;
      lsum[rb] = 0.f;
    }
    TileRegs<C> regs;
    const int t0 = (u_lo / C::BN) * C::BN;
    tile_load<C, false>(a, sg, g, t0, u_end, regs);
    for (int u0 = t0; u0 < u_end; u0 += C::BN) {
      __syncthreads();
      tile_store<C, false>(lds, regs);
      __syncthreads();
      if (u0 + C::BN < u_end) tile_load<C, false>(a, sg, g, u0 + C::BN, u_end, regs);
      f32x16 sacc[C::RB][2];
      qk_tile<C>(lds, qf, sacc);
#pragma unroll
      for (int rb = 0; rb < C::RB; ++rb) {
        apply_mask<C>(lds, qpos[rb], a.window, sacc[rb]);
        float mx = kNegBig;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[rb][mb][i]);
        mx = wave_pair_max(mx);
        const float mnew = fmaxf(m[rb], mx);
        const float alpha = __builtin_amdgcn_exp2f((m[rb] - mnew) * sl2);
        m[rb] = mnew;
        float rs = 0.f;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int i = 0; i < 16; ++i) rs += __builtin_amdgcn_exp2f(sacc[rb][mb][i] * sl2 - mnew * sl2);
        lsum[rb] = lsum[rb] * alpha + rs;
      }
    }
    float inv[C::RB];
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb) {
      const float lt = lsum[rb] + __shfl_xor(lsum[rb], 32, 64);
      inv[rb] = rvalid[rb] ? 1.f / lt : 0.f;
    }
    // sweep 2: own keys in 64-key tiles from the segment start
    const int own_end = i_last + 1;  // own keys visible to some row of this pass
    const int n_tiles = (own_end + C::BN - 1) / C::BN;
    int mt0 = 0;
    if (u_lo > sg.c) mt0 = (u_lo - sg.c) / C::BN;
    if (ps != passes - 1) {
      // later passes only add; earlier tiles with no visible keys add nothing
    } else {
      mt0 = 0;  // the first pass writes every block once
    }
    tile_load<C, false>(a, sg, g, sg.c + mt0 * C::BN, u_end, regs);
    for (int mt = mt0; mt < n_tiles; ++mt) {
      const int u0 = sg.c + mt * C::BN;
      __syncthreads();
      tile_store<C, false>(lds, regs);
      __syncthreads();
      if (mt + 1 < n_tiles) tile_load<C, false>(a, sg, g, u0 + C::BN, u_end, regs);
      f32x16 sacc[C::RB][2];
      qk_tile<C>(lds, qf, sacc);
      float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int rb = 0; rb < C::RB; ++rb) {
        apply_mask<C>(lds, qpos[rb], a.window, sacc[rb]);
        const float mb2 = m[rb] * sl2;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float p = __builtin_amdgcn_exp2f(sacc[rb][mb][i] * sl2 - mb2) * inv[rb];
            const int kk = mb * 32 + (i >> 2) * 8 + h * 4 + (i & 3);
            const int bt = B >= 64 ? 0 : kk / B;
            // bt < 4; select without dynamic register indexing
#pragma unroll
            for (int b = 0; b < 4; ++b)
              if (b == bt) part[b] += p;
          }
      }
      // reduce over lanes holding rows of the same head (lane % G)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        float x = part[b];
        x += __shfl_xor(x, 32, 64);
        for (int o = 16; o >= G; o >>= 1) x += __shfl_xor(x, o, 64);
        part[b] = x;
      }
      if (l < G) {
#pragma unroll
        for (int b = 0; b < 4; ++b) red[(w * 4 + b) * 32 + l] = part[b];
      }
      __syncthreads();
      if (tid < nbt * G) {
        const int bt = tid / G, hh = tid % G;
        float tot = 0.f;
#pragma unroll
        for (int ww = 0; ww < C::NW; ++ww) tot += red[(ww * 4 + bt) * 32 + hh];
        const int kb = (mt * C::BN) / B + bt;
        if (kb < nb) {
          float* dst = a.block_mass + (mbase + kb) * a.Hq + g * G + hh;
          const bool first = (ps == passes - 1) && (B <= C::BN || ((mt * C::BN) % B) == 0);
          if (first) *dst = tot;
          else *dst += tot;
        }
      }
    }
    __syncthreads();
  }
}

template <int D, int RB>
__global__ __launch_bounds__(256) void attn_bf16_kernel(AttnArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  using C = Cfg<D, RB>;
  const int item = blockIdx.x / a.Hkv;
  const int g = blockIdx.x % a.Hkv;
  if (item >= *a.item_count) return;
  const int2 it = a.items[item];
  if (it.y == kScoreTile) score_item<C>(a, it.x, g, lds);
  else attn_item<C>(a, it.x, it.y, g, lds);
}

constexpr int kRB = 1;

int attn_bf16_positions_per_tile(int D, int G) {
  (void)D;
  return (32 * kRB * 4) / G;
}

hipError_t launch_attn_bf16(const AttnArgs& a, int D, int capacity, hipStream_t st) {
  dim3 grid((unsigned)capacity * a.Hkv);
  if (D == 128) {
    using C = Cfg<128, kRB>;
    hipLaunchKernelGGL((attn_bf16_kernel<128, kRB>), grid, dim3(256), C::LDS_BYTES, st, a);
  } else {
    using C = Cfg<64, kRB>;
    hipLaunchKernelGGL((attn_bf16_kernel<64, kRB>), grid, dim3(256), C::LDS_BYTES, st, a);
  }
  return hipGetLastError();
}

}  // namespace up
