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
//    permuted within each 16-key step; V^T fragments come from
//    ds_read_b64_tr_b16 transpose reads of row-major V.  Row statistics (max,
//    sum) live in one lane pair (l, l^32).
//  * Key tiles of 64 arrive by direct global->LDS copies (no staging
//    registers): the cache-row index and position of every key four tiles
//    ahead go to a small LDS ring, the K and V rows two tiles ahead go to one
//    of four tile buffers (a tile is read in two steps: waves 4-7 finish it
//    one step late).  Each wave waits only for its own copies of the next
//    tile (an exact count of its outstanding copies), then one barrier per
//    tile publishes it.
//  * Softmax in exp2 with the scale folded in, against a per-row reference
//    max fixed at the row's first tile with a visible key: the steady loop
//    computes no row max and never rescales O.  A tile whose probabilities
//    pass 2^64 sends the item through a second loop with a running max that
//    is raised (and O, l rescaled) when a tile's max is 2^8 above it.
//  * Block importance of a scored segment: the items holding the rows of
//    its last block store, per row and head, the log2-sum-exp of every run
//    of 64, 32 or 16 own keys (the largest dividing the block) and the row's
//    total log2-sum-exp (key tiles
//    are aligned to the segment's first own key, so runs never straddle a
//    tile); block_mass_kernel (mass.hip) then sums exp2(run - total) over
//    the rows and runs of each block in a fixed order (deterministic).
#include <type_traits>

#include "common.h"
#include "lds_copy.h"

namespace up {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int D_>
struct Cfg {
  static constexpr int D = D_;
  static constexpr int NW = 8;
  static constexpr int THREADS = NW * 64;
  static constexpr int ROWS = 32 * NW;  // packed rows per workgroup
  static constexpr int BN = 64;         // keys per tile
  static constexpr int KC = D / 16;     // 16-wide d steps (QK^T)
  static constexpr int DB = D / 32;     // 32-wide d blocks (PV)
  // A K or V tile is 64 unpadded rows of 2D bytes whose 16-byte chunks are
  // XOR-swizzled per row (swk / swv).  Wave w copies the rows of keys
  // w*KPW .. w*KPW+KPW-1, RPW rows (1 KiB) per copy instruction.
  static constexpr int RBYTES = 2 * D;
  static constexpr int CPR = RBYTES / 16;  // chunks per row
  static constexpr int RPW = 64 / CPR;     // rows per copy instruction
  static constexpr int KPW = BN / NW;      // keys per wave
  static constexpr int WPW = KPW / RPW;    // copy instructions per wave per matrix
  // pipeline depth: data LA tiles ahead, indices IA = 2 LA tiles ahead
  static constexpr int LA = 2;
  static constexpr int IA = 2 * LA;
  // tile t is read in steps t and t+1 (waves 4-7 finish it a step late) and
  // tiles t+1, t+2 are landing: four buffers
  static constexpr int NBUF = 4;
  static constexpr int NRING = 8;  // ring slots (power of two, > IA)
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = BN * RBYTES;
  static constexpr int BUF_BYTES = 2 * BN * RBYTES;
  // ring slot: [0, 256) cache-row source value per key, [256, 512) position
  static constexpr int RING_OFF = NBUF * BUF_BYTES;
  static constexpr int RING_BYTES = 2 * BN * 4;
  static constexpr int MISC_OFF = RING_OFF + NRING * RING_BYTES;
  // rotary frequencies (turns per position) of the D/2 pairs, float64
  static constexpr int ROPE_OFF = MISC_OFF + 64;
  static constexpr int LDS_BYTES = ROPE_OFF + (D / 2) * 8;
  // copies one wave issues per tile step: two index copies, K and V rows
  static constexpr int COPIES_IDX = 2;
  static constexpr int COPIES_DATA = 2 * WPW;
  static constexpr int COPIES_STEP = COPIES_IDX + COPIES_DATA;
  static_assert(WPW >= 1 && WPW * RPW == KPW, "copy split");
  static_assert(LA == 2, "the prologue's wait counts assume two data tiles ahead");
  static_assert(NRING > IA && (NRING & (NRING - 1)) == 0, "ring size");
  static_assert(NBUF == 4, "buffer rotation");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

// Chunk swizzles.  K fragments are read 16 rows x one 16-byte chunk per 16
// lanes; V^T fragments by ds_read_b64_tr_b16, 4 rows x two chunks per 16
// lanes, two such groups per cycle.  The XOR patterns put each of those
// access sets on distinct banks.
template <int D>
__device__ inline int swk(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
template <int D>
__device__ inline int swv(int r) {
  return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
}

constexpr int kPosInvalid = 0x7fffffff;
constexpr float kNegBig = -1.0e30f;

struct Seg {
  int s, q0, n, c;
};

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
// tile staging
// ----------------------------------------------------------------------------
// Keys outside [0, u_end) are clamped to the nearest key in it (real,
// finite data) and get position INT_MAX, so the mask removes them; every
// copy reads inside its array and no branch depends on per-key data.
template <class C>
struct Stager {
  const AttnArgs& a;
  const Seg& sg;
  int g, t0, u_end, w, lane;
  char* lds;
  uint32_t l0;

  __device__ inline int buf_off(int k) const { return (k & (C::NBUF - 1)) * C::BUF_BYTES; }
  __device__ inline int ring_off(int k) const {
    return C::RING_OFF + (k & (C::NRING - 1)) * C::RING_BYTES;
  }

  // tile k: wave 0 brings, for key `lane`, the page-table entry (cached key)
  // or slot (own key) and the key's position into ring slot k
  __device__ inline void index(int k) const {
    if (w != 0) return;
    const int u = t0 + k * C::BN + lane;
    const int uu = max(min(u, u_end - 1), 0);
    const bool cached = uu < sg.c;
    const int own = max(uu - sg.c, 0);
    // the source is selected arithmetically (a select of two kernel-argument
    // pointers becomes a per-lane load of the argument)
    const uintptr_t bt = (uintptr_t)(a.block_table + (long)sg.s * a.max_pages + (uu >> 4));
    const uintptr_t sm = (uintptr_t)(a.slot_mapping + sg.q0 + own);
    const uintptr_t ps = (uintptr_t)(a.positions + sg.q0 + min(own, sg.n - 1));
    const uint32_t dst = l0 + ring_off(k);
    lds_copy4(cached ? bt : sm, dst);
    lds_copy4(ps, dst + C::BN * 4);
  }

  // tile k: K and V rows of this wave's keys into buffer k % NBUF, chunk
  // (i % CPR) ^ sw(r) of row r to LDS chunk slot i % CPR; then the ring's
  // position entries of these keys are finalised (cached key: u; past the
  // visible range: INT_MAX)
  __device__ inline void data(int k) const {
    const int u0 = t0 + k * C::BN;
    const int* rv = (const int*)(lds + ring_off(k));
    int* rp = (int*)(lds + ring_off(k) + C::BN * 4);
    const uint32_t dst = l0 + buf_off(k);
    const int pc = lane % C::CPR;
    // every ring entry this wave needs, in one round trip
    int val[C::WPW];
#pragma unroll
    for (int x = 0; x < C::WPW; ++x) val[x] = rv[w * C::KPW + x * C::RPW + lane / C::CPR];
#pragma unroll
    for (int x = 0; x < C::WPW; ++x) {
      const int rbase = w * C::KPW + x * C::RPW;
      const int r = rbase + lane / C::CPR;
      const int uu = max(min(u0 + r, u_end - 1), 0);
      const bool cached = uu < sg.c;
      const int page = cached ? val[x] : (val[x] >> 4);
      const int off = cached ? (uu & 15) : (val[x] & 15);
      // 24-bit product: Hkv <= 255 (checked by the host), page * Hkv < 2^27
      // (a documented precondition on the cache size)
      const long rowb = (long)((__umul24(page, a.Hkv) + g) * kPageSize + off) * C::RBYTES;
      lds_copy16((uintptr_t)a.k_cache + rowb + (pc ^ swk<C::D>(r)) * 16,
             dst + C::K_OFF + rbase * C::RBYTES);
      lds_copy16((uintptr_t)a.v_cache + rowb + (pc ^ swv<C::D>(r)) * 16,
             dst + C::V_OFF + rbase * C::RBYTES);
    }
    // positions: a cached key's is its index, one outside the key range
    // (past the visible end, or before key 0) gets INT_MAX; an own key
    // keeps the copied one (no write)
#pragma unroll
    for (int x = 0; x < C::WPW; ++x) {
      const int r = w * C::KPW + x * C::RPW + lane / C::CPR;
      const int u = u0 + r;
      if (pc == 0 && (u >= u_end || u < sg.c)) rp[r] = (u < u_end && u >= 0) ? u : kPosInvalid;
    }
  }
};

// Pipeline over the key tiles [t0, u_end) in steps of 64.  Tile step t:
// index copies of tile t+4, data copies of tile t+2, the step's work on tile
// t (and t-1), wait until this wave's copies of tile t+1 have landed,
// barrier.  Copies past the last tile are clamped and unused.  Every thread
// of the workgroup runs the same steps.
template <class C>
__device__ inline void sweep_prologue(const Stager<C>& st) {
  lds_only_barrier();  // the previous users of the buffers and the ring are done
#pragma unroll
  for (int k = 0; k < C::IA; ++k) st.index(k);
  lds_copy_wait<0>();
  lds_only_barrier();
#pragma unroll
  for (int k = 0; k < C::LA; ++k) st.data(k);
  lds_copy_wait<C::COPIES_DATA>();  // tile 0 has landed
  lds_only_barrier();
}
// Only tiles that exist are copied: step t issues the index copies of tile
// t+IA and the data copies of tile t+LA only while those are below nt, and
// waits for everything but what it issued.
template <class C>
__device__ inline void sweep_issue(const Stager<C>& st, int t, int nt) {
  if (t + C::IA < nt) st.index(t + C::IA);
  if (t + C::LA < nt) st.data(t + C::LA);
}
template <class C>
__device__ inline void sweep_step_end(int t, int nt) {
  const bool w0 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) == 0;
  if (t + C::IA < nt) {
    if (w0) lds_copy_wait<C::COPIES_STEP>();
    else lds_copy_wait<C::COPIES_DATA>();
  } else if (t + C::LA < nt) {
    lds_copy_wait<C::COPIES_DATA>();
  } else {
    lds_copy_wait<0>();
  }
  lds_only_barrier();
}

// ----------------------------------------------------------------------------
// Q fragments with rotary embedding
// ----------------------------------------------------------------------------
// x of quad lane k in every lane of the quad (DPP quad_perm(k, k, k, k));
// k is a constant after unrolling
__device__ inline float quad_bcast(float x, int k) {
  const int v = __float_as_int(x);
  switch (k) {
    case 0: return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x00, 0xf, 0xf, false));
    case 1: return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x55, 0xf, 0xf, false));
    case 2: return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0xaa, 0xf, 0xf, false));
    default: return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0xff, 0xf, 0xf, false));
  }
}

// Lane l (h = l / 32) holds, for d-step kc, q[row][kc*16 + h*8 + e].
// Pair j = kc*16 + h*8 + e (kc < KC/2) rotates elements j and j + D/2 by
// the angle pos * rev[j] turns, reduced to (-1/2, 1/2] in float64 before the
// hardware sin/cos (which take turns).  `rev` is the frequency table in LDS.
template <class C>
__device__ inline void load_q(const AttnArgs& a, long qrow_elem, bool valid, int pos,
                              const double* rev, bf16x8 (&qf)[C::KC]) {
  const int l = threadIdx.x & 63, h = l >> 5;
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
  constexpr int NP = C::KC / 2;  // d-steps of the first half
  auto rotate = [&](int kc, int e, float s, float c) {
    const float x1 = x[kc][e], x2 = x[kc + NP][e];
    x[kc][e] = x1 * c - x2 * s;
    x[kc + NP][e] = x2 * c + x1 * s;
  };
  if (a.rope && valid) {
    if ((a.G & 3) == 0) {
      // G a multiple of 4: the four lanes of a quad hold four heads of one
      // token (same position, same h), so quad lane k computes the angles
      // of d-step k (mod NP) once and each d-step's values are broadcast
      // from its lane (all four lanes share the row's validity)
      const int k = (l & 3) % NP;
      float so[8], co[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        double t = (double)pos * rev[k * 16 + h * 8 + e];
        t -= rint(t);
        so[e] = __builtin_amdgcn_sinf((float)t);
        co[e] = __builtin_amdgcn_cosf((float)t);
      }
#pragma unroll
      for (int kc = 0; kc < NP; ++kc)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          rotate(kc, e, quad_bcast(so[e], kc), quad_bcast(co[e], kc));
        }
    } else {
#pragma unroll
      for (int kc = 0; kc < NP; ++kc)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          double t = (double)pos * rev[kc * 16 + h * 8 + e];
          t -= rint(t);
          rotate(kc, e, __builtin_amdgcn_sinf((float)t), __builtin_amdgcn_cosf((float)t));
        }
    }
  }
#pragma unroll
  for (int kc = 0; kc < C::KC; ++kc)
#pragma unroll
    for (int e = 0; e < 8; ++e) qf[kc][e] = (__bf16)x[kc][e];
}

// LDS fragment addresses.  Per lane, the byte offset inside a tile buffer
// of its K fragment for each 16-wide d step kc (key row kr = l%32, chunk
// (2kc + h) ^ swk(kr)) and of its V^T transpose-read start for each 32-wide d
// block db (row h*4 + (l%16)/4 of each 16-key step).  Neither swizzle
// depends on the 32-key half, the 16-key step or the upper 8 keys of a
// step, so those stay immediate offsets of the reads.
typedef __attribute__((address_space(3))) const bf16x8 lbf16x8;
typedef __attribute__((address_space(3))) bf16x4 lbf16x4;
template <class C>
struct FragOffsets {
  uint32_t k[C::KC], v[C::DB];
  __device__ inline FragOffsets() {
    const int l = threadIdx.x & 63, h = l >> 5, kr = l & 31;
#pragma unroll
    for (int kc = 0; kc < C::KC; ++kc)
      k[kc] = C::K_OFF + kr * C::RBYTES + (((kc * 2 + h) ^ swk<C::D>(kr)) << 4);
    const int R = h * 4 + ((l & 15) >> 2);
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      const int cv = db * 4 + ((l & 16) >> 3) + ((l & 3) >> 1);
      v[db] = C::V_OFF + R * C::RBYTES + ((cv ^ swv<C::D>(R)) << 4) + 8 * (l & 1);
    }
  }
};
// A tile's fragment addresses: the offsets plus the buffer's LDS address.
// The empty asm keeps each sum in one register, so the compiler folds the
// constant parts into the reads instead of keeping one register per read.
template <class C>
struct TileFrag {
  uint32_t k[C::KC], v[C::DB];
  __device__ inline TileFrag(const FragOffsets<C>& f, uint32_t base) {
#pragma unroll
    for (int kc = 0; kc < C::KC; ++kc) {
      k[kc] = f.k[kc] + base;
      asm("" : "+v"(k[kc]));
    }
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      v[db] = f.v[db] + base;
      asm("" : "+v"(v[db]));
    }
  }
};

// S^T = K Q^T for one 64-key tile: s[mb], mb = 32-key half of the tile
template <class C>
__device__ inline void qk_tile(const TileFrag<C>& tf, const bf16x8 (&qf)[C::KC],
                               f32x16 (&s)[2]) {
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) s[mb][i] = 0.f;
#pragma unroll
  for (int kc = 0; kc < C::KC; ++kc) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const bf16x8 kf = *(lbf16x8*)(uintptr_t)(tf.k[kc] + mb * 32 * C::RBYTES);
      s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kc], s[mb], 0, 0, 0);
    }
  }
}

// Visibility mask of this lane's 32 keys for its row.
__device__ inline void apply_mask(const int* kp, int qpos, int window, f32x16 (&s)[2]) {
  const int l = threadIdx.x & 63, h = l >> 5;
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

// Reductions over the lane pair (l, l^32): v_permlane32_swap of x with
// itself leaves x(l % 32) in one result and x(l % 32 + 32) in the other.
__device__ inline float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

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
constexpr float kRefUnset = -1.0e29f;         // ms above this: a reference is set
constexpr float kRefMaxSum = 1.8446744e19f;   // 2^64

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
  load_q<C>(a, qrow, rvalid, qpos, (const double*)(lds + C::ROPE_OFF), qf);
  const int pos_first = a.positions[sg.q0 + i_first];
  const int pos_last = a.positions[sg.q0 + i_last];
  const int u_end = sg.c + i_last + 1;
  const int u_lo = window_start(a, sg, pos_first, lds, C::MISC_OFF);
  const int window = a.window;
  const int full_limit = sg.c + i_first;
  const float sl2 = a.scale_log2;

  f32x16 o[C::DB];
  float ms, lsum;   // reference or running max (log2 units), partial row sum
  f32x16 sacc[2];   // S^T of the tile between QK and softmax

  // Key tiles are aligned to the segment's first own key (key index c), so
  // every 16-key step of a tile covers one run of 16 own keys; the first
  // tile may start before key 0 (those keys are masked).
  const int t0 = u_lo >= sg.c ? sg.c + ((u_lo - sg.c) / C::BN) * C::BN
                              : sg.c - ((sg.c - u_lo + C::BN - 1) / C::BN) * C::BN;
  const int nt = (u_end - t0 + C::BN - 1) / C::BN;

  // Block importance (scored segments): the rows of the segment's last
  // block store, per row and head, the log2-sum-exp of each run of Qs own
  // keys (Qs = 64, 32 or 16, the largest dividing the block) and their
  // total log2-sum-exp; mass of block
  // b = sum over those rows of exp2(run - total) over b's runs
  // (block_mass_kernel).
  const int Bs = a.block_size;
  const bool scored = a.score_flags != nullptr && a.score_flags[s] != 0;
  const int nbs = scored ? (sg.n + Bs - 1) / Bs : 0;
  const int r0s = scored ? (nbs - 1) * Bs : 0;
  const bool item_scores = scored && i_last >= r0s;       // same in every lane
  const bool row_scores = item_scores && rvalid && i >= r0s && h == 0;
  const int Qs = scored ? score_run_len(Bs) : C::BN;
  const int run_base = scored ? a.cu_blocks[s] * (Bs / Qs) : 0;
  // first key of the scored blocks: the segment's first own key, or key 0
  // when the whole prompt is scored (cached length a multiple of the block)
  const int c0 = (scored && a.score_scope) ? 0 : sg.c;
  float* run_lse = row_scores ? a.score_part + (long)(i - r0s) * a.Hq + g * G + hh : nullptr;
  const long run_stride = (long)Bs * a.Hq;  // between consecutive runs
  const Stager<C> st{a,   sg,  g, t0, u_end, __builtin_amdgcn_readfirstlane(w),
                     l, lds, lds_addr_of(lds)};

  // S^T of tile t, masked where the tile is not entirely visible
  const FragOffsets<C> fo;
  const uint32_t l0 = lds_addr_of(lds);
  auto qk = [&](int t) {
    const TileFrag<C> tf(fo, l0 + st.buf_off(t));
    const int* kpos = (const int*)(lds + st.ring_off(t) + C::BN * 4);
    qk_tile<C>(tf, qf, sacc);
    const int u0 = t0 + t * C::BN;
    const bool full = u0 >= 0 && (u0 + C::BN - 1 <= full_limit) &&
                      (window <= 0 || kpos[0] > pos_last - window);
    if (!full) apply_mask(kpos, qpos, window, sacc);
  };
  // probabilities of S^T (tile t) against ms, their row sum, O^T += V^T P^T
  // sc: std::true_type in the loop instances that score (items holding a
  // scored segment's last-block rows, and the rescaling loop); the others
  // carry none of that code
  auto probs_pv = [&](int t, auto sc) {
    constexpr bool SC = decltype(sc)::value;
    const TileFrag<C> tf(fo, l0 + st.buf_off(t));
    bf16x8 pf[4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        pf[mb * 2 + (e >> 3)][e & 7] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sacc[mb][e], sl2, -ms));
    // row sum of the bf16 probabilities the PV product uses, two per dot2
    // (per 16-key step where runs are scored)
    const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
    float rk[4];
    float rs;
    if constexpr (SC) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        float x0 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[ks][0], pf[ks][1]}, one2, 0.f, false);
        float x1 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[ks][2], pf[ks][3]}, one2, 0.f, false);
        x0 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[ks][4], pf[ks][5]}, one2, x0, false);
        x1 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[ks][6], pf[ks][7]}, one2, x1, false);
        rk[ks] = x0 + x1;
      }
      rs = (rk[0] + rk[1]) + (rk[2] + rk[3]);
    } else {
      float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        rs0 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[ks][0], pf[ks][1]}, one2, rs0, false);
        rs1 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[ks][2], pf[ks][3]}, one2, rs1, false);
        rs0 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[ks][4], pf[ks][5]}, one2, rs0, false);
        rs1 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[ks][6], pf[ks][7]}, one2, rs1, false);
      }
      rs = rs0 + rs1;
    }
    lsum += rs;
    // 16-key step ks uses S^T registers (ks%2)*8.. of half ks/2.  V^T
    // fragment of lane l (d = l%32, h = l/32): keys ks*16 + h*4 + 0..3 and
    // ks*16 + 8 + h*4 + 0..3 at d, via two transpose reads in which lane
    // 4a+b of each 16-lane group points at V[key0 + a][d0 + 4b].
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const uint32_t vp = tf.v[db] + ks * 16 * C::RBYTES;
        const bf16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lbf16x4*)(uintptr_t)vp);
        const bf16x4 hi4 =
            __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lbf16x4*)(uintptr_t)(vp + 8 * C::RBYTES));
        const bf16x8 vf = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ks], o[db], 0, 0, 0);
      }
    }
    // scored segment, last block's rows, tile with scored keys: the
    // log2-sum-exp of each run of Qs keys from c0 (after the products, so
    // the branch does not split the softmax and PV work)
    const int u0 = t0 + t * C::BN;
    if (SC && item_scores && u0 + C::BN > c0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int q = Qs == 16 ? j : Qs == 32 ? (j >> 1) : 0;
        const bool head = Qs == 16 || (Qs == 32 && (j & 1) == 0) || (Qs == 64 && j == 0);
        if (!head) continue;
        const float part = Qs == 16 ? rk[j] : Qs == 32 ? rk[j] + rk[j + 1] : rs;
        const float x = pair_sum(part);
        const int ustart = u0 + q * Qs;
        if (row_scores && ustart >= c0 && ustart < sg.c + sg.n)
          run_lse[(long)(run_base + (ustart - c0) / Qs) * run_stride] = ms + __log2f(x);
      }
    }
    return rs;
  };
  // Fast path (reference max): a row's reference is its max over its first
  // tile with a visible key (before that O and l are zero, so setting it
  // costs nothing) and stays fixed, so the steady loop has no row max and
  // no rescaling.  Later probabilities may exceed 1: bf16 and fp32 keep
  // their relative precision there and the final division by l
  // normalises.  A tile whose row sum passes 2^64 marks the item, which is
  // then recomputed by the rescaling path.
  bool bad = false;
  auto softmax_pv_ref = [&](int t, auto sc) {
    if (__any(ms <= kRefUnset)) {
      const float mx = scaled_row_max(sacc, sl2);
      ms = ms > kRefUnset ? ms : fmaxf(ms, mx);
    }
    const float rs = probs_pv(t, sc);
    bad = bad || !(rs <= kRefMaxSum);
  };
  // Rescaling path: the running max is raised (and O, l rescaled) when a
  // tile's max exceeds it by more than kLazy.
  auto softmax_pv_rescale = [&](int t) {
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
    probs_pv(t, std::true_type{});
  };

  // The two waves that share a SIMD (w and w+4) work on different stages:
  // waves 0-3 run QK, softmax and PV of tile t in step t; waves 4-7 run
  // softmax and PV of tile t-1, then QK of tile t.  While one issues matrix
  // instructions the other mostly runs the vector softmax.  Waves 4-7 finish
  // the last tile after the loop.
  const bool lead = w < C::NW / 2;
  // A wave whose rows all lie past the item's last token (short segments,
  // decodes) only stages and synchronises.
  const bool active = __any(rvalid);
  auto run = [&](auto rescale, auto sc) {
    constexpr bool R = decltype(rescale)::value;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[db][e] = 0.f;
    ms = kNegBig;
    lsum = 0.f;
    auto spv = [&](int t) {
      if constexpr (R) softmax_pv_rescale(t);
      else softmax_pv_ref(t, sc);
    };
    sweep_prologue(st);
    for (int t = 0; t < nt; ++t) {
      // the two waves of a SIMD issue their copies at different points of
      // the step, so the copies of a step never all queue at once
      if (lead) {
        if (active) qk(t);
        sweep_issue(st, t, nt);
        if (active) spv(t);
      } else {
        if (t > 0 && active) spv(t - 1);
        if (active) qk(t);
        sweep_issue(st, t, nt);
      }
      sweep_step_end<C>(t, nt);
    }
    // waves 4-7 finish the last tile (its buffer is no longer written)
    if (!lead && active) spv(nt - 1);
    lds_copy_wait<0>();
  };
  int* misc = (int*)(lds + C::MISC_OFF);
  if (tid == 0) misc[1] = 0;  // published by the prologue's barriers
  if (item_scores) run(std::false_type{}, std::true_type{});
  else run(std::false_type{}, std::false_type{});
  if (__any(bad) && l == 0) misc[1] = 1;
  lds_only_barrier();
  if (misc[1]) run(std::true_type{}, std::true_type{});

  // epilogue: normalise and store; lane holds d = db*32 + jg*8 + h*4 + e
  const float ltot = pair_sum(lsum);
  if (row_scores) {
    a.score_lse[((long)s * Bs + (i - r0s)) * a.Hq + g * G + hh] = ms + __log2f(ltot);
    // runs before the first tile (outside the window of every row here)
    for (int q = 0; q < (t0 - c0) / Qs; ++q)
      run_lse[(long)(run_base + q) * run_stride] = -INFINITY;
  }
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

template <int D>
__global__ __launch_bounds__(512) void attn_bf16_kernel(AttnArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  using C = Cfg<D>;
  const int item = blockIdx.x / a.Hkv;
  const int g = blockIdx.x % a.Hkv;
  if (item >= *a.item_count) return;
  // the rotary frequency table into LDS (read per lane by the query load)
  if (a.rope && threadIdx.x < D / 2)
    ((double*)(lds + C::ROPE_OFF))[threadIdx.x] = a.rope_rev[threadIdx.x];
  __syncthreads();
  const int2 it = a.items[item];
  attn_item<C>(a, it.x, it.y, g, lds);
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
