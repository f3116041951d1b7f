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
//    workgroup (8 waves, 2 per SIMD) owns 256 consecutive packed rows, so
//    every K/V tile staged in LDS feeds all G query heads that read it.
//  * A wave owns 32 packed rows.  S^T = K Q^T and O^T = V^T P^T run on
//    v_mfma_f32_32x32x16_bf16: the S^T accumulator holds, per lane, 16 keys
//    of one query row, which is the B-operand layout P^T needs once keys are
//    permuted within each 16-key step (V^T is stored in LDS with the same
//    permutation).  Row statistics (max, sum) live in one lane pair (l, l^32).
//  * Key tiles of 64 go through a three-stage pipeline: cache-row indices
//    (page table or per-token slot) two tiles ahead, K/V data one tile ahead
//    in registers, and a double-buffered LDS stage, one barrier per tile.
//    Eight threads stage each key (four move a quarter of its K row, four a
//    quarter of its V row); V stays row-major in LDS and its V^T fragments
//    come from ds_read_b64_tr_b16 transpose reads.
//  * Online softmax in exp2 with the scale folded in and a lazily raised
//    running max (rescale only when a tile's max is 2^8 above it).
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
// native vector for staged 16-byte chunks (HIP's uint4 is a struct with a
// union, which the optimiser may leave on the stack)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
// global-address-space views, so loads from computed addresses stay global_load
// (a flat load would also hold the LDS counter the compute phase waits on)
typedef __attribute__((address_space(1))) const u32x4 gu32x4;
typedef __attribute__((address_space(1))) const int gint;

template <int D_>
struct Cfg {
  static constexpr int D = D_;
  static constexpr int NW = 8;
  static constexpr int THREADS = NW * 64;
  static constexpr int ROWS = 32 * NW;      // packed rows per workgroup
  static constexpr int BN = 64;             // keys per tile
  static constexpr int KC = D / 16;         // 16-wide d steps (QK^T)
  static constexpr int DB = D / 32;         // 32-wide d blocks (PV)
  // LDS row strides (bytes).  K rows are read 16 bytes per lane, 32 rows at a
  // time: a stride of 4 banks mod 64 keeps 16 lanes on distinct banks.  V rows
  // are read with ds_read_b64_tr_b16 (4 rows x 32 bytes per 16 lanes, two
  // groups per cycle): a stride of 16 banks mod 64 keeps those disjoint.
  static constexpr int KSTR = D * 2 + 16;
  static constexpr int VSTR = 320;
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = K_OFF + BN * KSTR;
  static constexpr int POS_OFF = V_OFF + BN * VSTR;
  static constexpr int BUF_BYTES = POS_OFF + BN * 4;
  static constexpr int RED_OFF = 2 * BUF_BYTES;
  static constexpr int RED_BYTES = NW * 4 * 32 * 4;  // [wave][block in tile][head] f32
  static constexpr int MISC_OFF = RED_OFF + RED_BYTES;
  static constexpr int LDS_BYTES = MISC_OFF + 64;
  // loaders: 8 threads per key; parts 0-3 move a quarter K row, 4-7 a quarter V row
  static constexpr int PART_BYTES = D / 2;
  static constexpr int PCH = PART_BYTES / 16;  // 16-byte chunks per thread (2 or 4)
  static_assert(VSTR >= D * 2, "V row stride");
};

constexpr int kPosInvalid = 0x7fffffff;
constexpr float kNegBig = -1.0e30f;

struct Seg {
  int s, q0, n, c;
};

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
// tile pipeline: indices -> registers -> LDS
// ----------------------------------------------------------------------------
// Thread t stages key t/8 of the tile: parts 0-3 a quarter of its K row,
// parts 4-7 a quarter of its V row.  Keys past the visible range are clamped
// to the last visible one (real, finite data) and get position INT_MAX so the
// mask removes them; no branch depends on per-key data.
template <class C, bool kWithV>
struct Pipe {
  int row;    // cache row (page * Hkv + g) * 16 + offset
  int ipos;   // key position from the index stage
  int dpos;   // the same, latched with the data stage
  u32x4 d0, d1, d2, d3;  // staged data (d2, d3 unused when D = 64)

  __device__ inline void index(const AttnArgs& a, const Seg& sg, int g, int u0, int u_end) {
    const int kk = threadIdx.x >> 3;
    const int u = u0 + kk;
    const int uu = min(u, u_end - 1);
    const bool cached = uu < sg.c;
    const int own = max(uu - sg.c, 0);
    // select the index address arithmetically (a select of two kernel-argument
    // pointers would be turned into a per-lane load of the argument itself)
    const uintptr_t bt = (uintptr_t)(a.block_table + (long)sg.s * a.max_pages + (uu >> 4));
    const uintptr_t sm = (uintptr_t)(a.slot_mapping + sg.q0 + own);
    const int val = *(gint*)(cached ? bt : sm);
    const int page = cached ? val : (val >> 4);
    const int off = cached ? (uu & 15) : (val & 15);
    row = (page * a.Hkv + g) * kPageSize + off;
    const int opos = a.positions[sg.q0 + min(own, sg.n - 1)];
    ipos = u < u_end ? (cached ? uu : opos) : kPosInvalid;
  }

  // Loads and stores are unconditional (a K-only sweep moves V too, unused),
  // so the staged registers never live across divergent control flow.
  __device__ inline void load(const AttnArgs& a) {
    const int part = threadIdx.x & 7;
    dpos = ipos;
    const uintptr_t kb = (uintptr_t)a.k_cache, vb = (uintptr_t)a.v_cache;
    const uintptr_t base = kb + (uintptr_t)(part >> 2) * (vb - kb);
    gu32x4* src = (gu32x4*)(base + ((long)row * C::D + (part & 3) * (C::PART_BYTES / 2)) * 2);
    d0 = src[0];
    d1 = src[1];
    if constexpr (C::PCH == 4) {
      d2 = src[2];
      d3 = src[3];
    }
  }

  __device__ inline void store(char* buf) const {
    const int kk = threadIdx.x >> 3, part = threadIdx.x & 7;
    char* dst = part < 4 ? buf + C::K_OFF + kk * C::KSTR + part * C::PART_BYTES
                         : buf + C::V_OFF + kk * C::VSTR + (part - 4) * C::PART_BYTES;
    ((u32x4*)dst)[0] = d0;
    ((u32x4*)dst)[1] = d1;
    if constexpr (C::PCH == 4) {
      ((u32x4*)dst)[2] = d2;
      ((u32x4*)dst)[3] = d3;
    }
    if (part == 0) ((int*)(buf + C::POS_OFF))[kk] = dpos;
  }
};

// Runs body(buf, u0) over the key tiles [t0, u_end) in steps of 64 with the
// index/data/LDS pipeline.  Every thread of the workgroup must call it.
template <class C, bool kWithV, class Body>
__device__ inline void sweep(const AttnArgs& a, const Seg& sg, int g, int t0, int u_end,
                             char* lds, Body&& body) {
  const int nt = (u_end - t0 + C::BN - 1) / C::BN;
  if (nt <= 0) return;
  Pipe<C, kWithV> p;
  p.index(a, sg, g, t0, u_end);
  p.load(a);
  if (nt > 1) p.index(a, sg, g, t0 + C::BN, u_end);
  __syncthreads();  // the previous user of the buffers is done
  p.store(lds);
  __syncthreads();
  if (nt > 1) {
    p.load(a);
    if (nt > 2) p.index(a, sg, g, t0 + 2 * C::BN, u_end);
  }
  for (int t = 0; t < nt; ++t) {
    char* buf = lds + (t & 1) * C::BUF_BYTES;
    body((const char*)buf, t0 + t * C::BN);
    if (t + 1 < nt) p.store(lds + ((t + 1) & 1) * C::BUF_BYTES);
    __syncthreads();
    if (t + 2 < nt) {
      p.load(a);
      if (t + 3 < nt) p.index(a, sg, g, t0 + (t + 3) * C::BN, u_end);
    }
  }
}

// ----------------------------------------------------------------------------
// Q fragments with rotary embedding
// ----------------------------------------------------------------------------
// Lane l (h = l / 32) holds, for d-step kc, q[row][kc*16 + h*8 + e].
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

// S^T = K Q^T for one 64-key tile: s[mb], mb = 32-key half of the tile
template <class C>
__device__ inline void qk_tile(const char* buf, const bf16x8 (&qf)[C::KC], f32x16 (&s)[2]) {
  const int l = threadIdx.x & 63, h = l >> 5, kr = l & 31;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) s[mb][i] = 0.f;
#pragma unroll
  for (int kc = 0; kc < C::KC; ++kc) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const bf16x8 kf =
          *(const bf16x8*)(buf + C::K_OFF + (mb * 32 + kr) * C::KSTR + (kc * 16 + h * 8) * 2);
      s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kc], s[mb], 0, 0, 0);
    }
  }
}

// Visibility mask of this lane's 32 keys for its row.
template <class C>
__device__ inline void apply_mask(const char* buf, int qpos, int window, f32x16 (&s)[2]) {
  const int l = threadIdx.x & 63, h = l >> 5;
  const int* kp = (const int*)(buf + C::POS_OFF);
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

__device__ inline float pair_max(float x) { return fmaxf(x, __shfl_xor(x, 32, 64)); }

__device__ inline int window_start(const AttnArgs& a, const Seg& sg, int pos_first, char* lds,
                                   int misc_off) {
  if (a.window <= 0) return 0;
  int* misc = (int*)(lds + misc_off);
  if (threadIdx.x < 64) {
    const int r = first_key_at_or_after(a, sg, pos_first - a.window + 1);
    if (threadIdx.x == 0) misc[0] = r;
  }
  __syncthreads();
  const int r = misc[0];
  __syncthreads();
  return r;
}

// ----------------------------------------------------------------------------
// attention item: one query tile of one segment, one KV head
// ----------------------------------------------------------------------------
// Row max over this lane's 32 keys and its partner lane's, scaled to log2 units.
__device__ inline float scaled_row_max(const f32x16 (&s)[2], float sl2) {
  float mx = kNegBig;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[mb][e]);
  return pair_max(mx) * sl2;
}

// The running max is only raised (and O, l rescaled) when a tile's max
// exceeds it by more than kLazy (log2 units); probabilities are computed
// against the stale max and stay below 2^kLazy, exact after the final
// division by l.
constexpr float kLazy = 8.0f;

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

  const int r = w * 32 + (l & 31);
  const int i = i_first + r / G, hh = r % G;
  const bool rvalid = i <= i_last;
  const int qpos = rvalid ? a.positions[sg.q0 + i] : -1;
  const long qrow = ((long)(sg.q0 + i) * a.Hq + g * G + hh) * C::D;
  bf16x8 qf[C::KC];
  load_q<C>(a, qrow, rvalid, qpos, qf);
  const int pos_first = a.positions[sg.q0 + i_first];
  const int pos_last = a.positions[sg.q0 + i_last];
  const int u_end = sg.c + i_last + 1;
  const int u_lo = window_start(a, sg, pos_first, lds, C::MISC_OFF);
  const int window = a.window;
  const int full_limit = sg.c + i_first;
  const float sl2 = a.scale_log2;

  f32x16 o[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[db][e] = 0.f;
  float ms = kNegBig, lsum = 0.f;  // running max (log2 units) and partial row sum

  sweep<C, true>(a, sg, g, (u_lo / C::BN) * C::BN, u_end, lds, [&](const char* buf, int u0) {
    f32x16 sacc[2];
    qk_tile<C>(buf, qf, sacc);
    const int kpos0 = ((const int*)(buf + C::POS_OFF))[0];
    const bool full = (u0 + C::BN - 1 <= full_limit) && (window <= 0 || kpos0 > pos_last - window);
    if (!full) apply_mask<C>(buf, qpos, window, sacc);
    const float mx = scaled_row_max(sacc, sl2);
    if (__any(mx > ms + kLazy)) {
      const float mnew = fmaxf(ms, mx);
      const float alpha = __builtin_amdgcn_exp2f(ms - mnew);
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[db][e] *= alpha;
      ms = mnew;
    }
    float rs = 0.f;
    bf16x8 pf[4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[mb][e], sl2, -ms));
        rs += pv;
        pf[mb * 2 + (e >> 3)][e & 7] = (__bf16)pv;
      }
    lsum += rs;
    // O^T += V^T P^T; 16-key step ks uses S^T registers (ks%2)*8.. of half ks/2.
    // V^T fragment of lane l (d = l%32, h = l/32): keys ks*16 + h*4 + 0..3 and
    // ks*16 + 8 + h*4 + 0..3 at d, via two transpose reads in which lane
    // 4a+b of each 16-lane group points at V[key0 + a][d0 + 4b].
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const char* vp = buf + C::V_OFF + (ks * 16 + h * 4 + ((l & 15) >> 2)) * C::VSTR +
                         (db * 32 + (l & 16) + 4 * (l & 3)) * 2;
        const bf16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (__attribute__((address_space(3))) bf16x4*)(vp));
        const bf16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (__attribute__((address_space(3))) bf16x4*)(vp + 8 * C::VSTR));
        const bf16x8 vf = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ks], o[db], 0, 0, 0);
      }
    }
  });

  // epilogue: normalise and store; lane holds d = db*32 + jg*8 + h*4 + e
  const float ltot = lsum + __shfl_xor(lsum, 32, 64);
  if (!rvalid) return;
  uint16_t* out = (uint16_t*)a.out;
  const float inv = 1.f / ltot;
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int jg = 0; jg < 4; ++jg) {
      bf16x4 v4;
#pragma unroll
      for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(o[db][jg * 4 + e] * inv);
      *(bf16x4*)(out + qrow + db * 32 + jg * 8 + h * 4) = v4;
    }
  if (a.lse && h == 0) a.lse[qrow / C::D] = (ms + __log2f(ltot)) * 0.69314718055994530942f;
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
  const int window = a.window;
  float* red = (float*)(lds + C::RED_OFF);
  const int nbt = B >= 64 ? 1 : 64 / B;  // blocks per 64-key tile

  for (int ps = passes - 1; ps >= 0; --ps) {
    const int rbeg = ps * C::ROWS;
    const int rend = min(rows_total, rbeg + C::ROWS);
    const int i_first = r0 + rbeg / G;
    const int i_last = r0 + (rend - 1) / G;
    const int r = rbeg + w * 32 + (l & 31);
    const int i = r0 + r / G, hh = r % G;
    const bool rvalid = r < rend;
    const int qpos = rvalid ? a.positions[sg.q0 + i] : -1;
    bf16x8 qf[C::KC];
    load_q<C>(a, ((long)(sg.q0 + i) * a.Hq + g * G + hh) * C::D, rvalid, qpos, qf);
    const int u_end = sg.c + i_last + 1;
    const int u_lo = window_start(a, sg, a.positions[sg.q0 + i_first], lds, C::MISC_OFF);
    // sweep 1: row max and normaliser over all visible keys
    float m = kNegBig, lsum = 0.f;
    sweep<C, false>(a, sg, g, (u_lo / C::BN) * C::BN, u_end, lds, [&](const char* buf, int u0) {
      f32x16 sacc[2];
      qk_tile<C>(buf, qf, sacc);
      apply_mask<C>(buf, qpos, window, sacc);
      float mx = kNegBig;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[mb][e]);
      mx = pair_max(mx);
      const float mnew = fmaxf(m, mx);
      const float alpha = __builtin_amdgcn_exp2f((m - mnew) * sl2);
      m = mnew;
      float rs = 0.f;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) rs += __builtin_amdgcn_exp2f(sacc[mb][e] * sl2 - mnew * sl2);
      lsum = lsum * alpha + rs;
    });
    const float lt = lsum + __shfl_xor(lsum, 32, 64);
    const float inv = rvalid ? 1.f / lt : 0.f;
    const float mb2 = m * sl2;
    // sweep 2: own keys in 64-key tiles from the segment start.  The first
    // pass (the one holding the segment's last row) writes every block.
    const int first_pass = ps == passes - 1;
    int mt0 = 0;
    if (!first_pass && u_lo > sg.c) mt0 = (u_lo - sg.c) / C::BN;
    sweep<C, false>(a, sg, g, sg.c + mt0 * C::BN, u_end, lds, [&](const char* buf, int u0) {
      f32x16 sacc[2];
      qk_tile<C>(buf, qf, sacc);
      apply_mask<C>(buf, qpos, window, sacc);
      float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = __builtin_amdgcn_exp2f(sacc[mb][e] * sl2 - mb2) * inv;
          const int kk = mb * 32 + (e >> 2) * 8 + h * 4 + (e & 3);
          const int bt = B >= 64 ? 0 : kk / B;
#pragma unroll
          for (int b = 0; b < 4; ++b)
            if (b == bt) part[b] += p;
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
        const int bt = tid / G, h2 = tid % G;
        float tot = 0.f;
#pragma unroll
        for (int ww = 0; ww < C::NW; ++ww) tot += red[(ww * 4 + bt) * 32 + h2];
        const int mt = (u0 - sg.c) / C::BN;
        const int kb = (mt * C::BN) / B + bt;
        if (kb < nb) {
          float* dst = a.block_mass + (mbase + kb) * a.Hq + g * G + h2;
          if (first_pass && (B <= C::BN || ((mt * C::BN) % B) == 0)) *dst = tot;
          else *dst += tot;
        }
      }
    });
  }
}

template <int D>
__global__ __launch_bounds__(512) void attn_bf16_kernel(AttnArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  using C = Cfg<D>;
  const int item = blockIdx.x / a.Hkv;
  const int g = blockIdx.x % a.Hkv;
  if (item >= *a.item_count) return;
  const int2 it = a.items[item];
  if (it.y == kScoreTile) score_item<C>(a, it.x, g, lds);
  else attn_item<C>(a, it.x, it.y, g, lds);
}

int attn_bf16_positions_per_tile(int D, int G) {
  (void)D;
  return Cfg<128>::ROWS / G;
}

hipError_t launch_attn_bf16(const AttnArgs& a, int D, int capacity, hipStream_t st) {
  dim3 grid((unsigned)capacity * a.Hkv);
  hipError_t e;
  if (D == 128) {
    using C = Cfg<128>;
    e = hipFuncSetAttribute((const void*)attn_bf16_kernel<128>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_bf16_kernel<128>), grid, dim3(C::THREADS), C::LDS_BYTES, st, a);
  } else {
    using C = Cfg<64>;
    e = hipFuncSetAttribute((const void*)attn_bf16_kernel<64>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_bf16_kernel<64>), grid, dim3(C::THREADS), C::LDS_BYTES, st, a);
  }
  return hipGetLastError();
}

}  // namespace up
