// Causal linear attention over the kept tokens of each packed segment, on
// bf16 matrix cores (gfx950): a later linear-attention layer of a
// linear/full hybrid running on the compacted rows only.
//
// What is computed (UniPrefill paper entry, abstract: linear/full hybrid
// models; review, "Method & Key Results": dropped tokens skip every later
// sublayer): per segment and query head h (KV head g = h / G), with
// phi(x) = elu(x) + 1 (Katharopoulos et al., "Transformers are RNNs",
// 2020), o_t = phi(q_t)^T S_t / (phi(q_t) . z_t), S_t = sum over s <= t of
// phi(k_s) v_s^T, z_t = sum of phi(k_s), s ranging over the segment's own
// tokens in order.
//
// Chunked form: the segment is walked in chunks of 64 tokens by one
// workgroup per (segment, query head), four waves, two workgroups per
// compute unit.  For chunk c with
// states S, z of the chunks before it:
//   A   = mask(phi(Q_c) phi(K_c)^T)           (64 x 64, key <= query)
//   o_c = (A V_c + phi(Q_c) S) / (A 1 + phi(Q_c) z)
//   S  += phi(K_c)^T V_c,   z += phi(K_c)^T 1
// All products run on v_mfma_f32_32x32x16_bf16, the row sums A 1 and the
// key sums phi(K_c)^T 1 too (against a ones operand).  S stays in float32
// registers (wave w owns output columns 32w..32w+31, which are the columns
// of the outputs it computes); the product phi(Q_c) S takes it from there
// as the bf16 pair hi + lo (hi the rounding of S, lo that of the
// remainder), so S enters with about 16 significant bits.  With no copy of
// S in LDS, two workgroups share a compute unit.  The denominators use the
// same bf16 A and phi(K) as the numerators.
//
// LDS: phi(Q), phi(K) and V are stored token-major as loaded (16-byte
// stores), A as A^T (key-major, 8-byte stores from the product's
// accumulator).  Products that contract over tokens or keys take their
// operands with ds_read_b64_tr_b16 transpose reads: two reads give a lane
// the 8 keys {4h..4h+3, 8+4h..8+4h+3} of a 16-key step (h = lane / 32),
// the same permutation on both operands.  The 16-byte chunks of a row are
// XOR-swizzled so that both the row reads (16 rows of one chunk) and the
// transpose reads (4 rows of a 64-byte chunk group) fall on distinct banks.
#include "common.h"
#include "lds_copy.h"

namespace up {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const bf16x8 lbf16x8;
typedef __attribute__((address_space(3))) bf16x4 lbf16x4;

constexpr int kC = 64;   // tokens per chunk
constexpr int kD = 128;  // head dimension
constexpr int kThreads = 256;
// LDS layout (bytes)
constexpr int QF = 0;                  // phi(Q) [64][128]   rows of 256 B
constexpr int KF = QF + kC * kD * 2;   // phi(K) [64][128]
constexpr int VF = KF + kC * kD * 2;   // V [64][128]
constexpr int AT = VF + kC * kD * 2;   // A^T [64 keys][64 queries], rows of 128 B
constexpr int ZF = AT + kC * kC * 2;   // z [128] f32
constexpr int DN = ZF + kD * 4;        // phi(Q) . z per row [64] f32
constexpr int kLdsBytes = DN + kC * 4;
static_assert(2 * kLdsBytes <= 160 * 1024, "two workgroups per compute unit");

// chunk swizzles: 256-byte rows (16 chunks): (r & 3) picks the 64-byte
// chunk group and (r >> 2) & 3 the chunk in it, a bijection over any 16
// consecutive rows that sends 4 consecutive rows to 4 different groups;
// 128-byte rows (8 chunks): rows r and r + 2 in different 64-byte groups,
// (r >> 2) & 3 inside the group
__device__ inline int sw256(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ inline int sw128(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }
// byte offset of element (r, e) in a row-major bf16 tile with 256-byte rows
__device__ inline int off256(int r, int e) { return r * 256 + (((e >> 3) ^ sw256(r)) << 4) + (e & 7) * 2; }
// ... with 128-byte rows
__device__ inline int off128(int r, int e) { return r * 128 + (((e >> 3) ^ sw128(r)) << 4) + (e & 7) * 2; }

// The 8 keys (tokens) {k0 + 4h + 0..3, k0 + 8 + 4h + 0..3} of column
// c0 + lane % 32 of a token-major tile (element offsets from `off`), by two
// transpose reads: in each 16-lane group, lane 4a + b points at row
// k0 + 4h + a (then + 8), columns c0 + 16 ((lane >> 4) & 1) + 4b.. + 3, and
// receives column c0 + lane % 32 of those four rows.
template <int (*OFF)(int, int)>
__device__ inline bf16x8 tr_frag(uint32_t base, int k0, int c0) {
  const int l = threadIdx.x & 63, h = l >> 5;
  const int r = k0 + 4 * h + ((l & 15) >> 2);
  const int c = c0 + (l & 16) + 4 * (l & 3);
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lbf16x4*)(uintptr_t)(base + OFF(r, c)));
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lbf16x4*)(uintptr_t)(base + OFF(r + 8, c)));
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ inline float phi(float x) { return x > 0.f ? x + 1.f : __expf(x); }

// Chunk-parallel form (when the caller passes a workspace): each segment
// is cut into parts of kPart tokens.  Part p of segment s has the slot
// cu_seqlens[s] / kPart + s + p, distinct for all parts and below
// rows / kPart + S + 1.  Pass 1 runs every part but a segment's last in
// parallel and stores the part's own (S, z) sums; pass 2 turns them, per
// segment and head, into running sums over the parts (inclusive); pass 3
// runs every part in parallel from the running sum of the parts before it
// and writes the outputs.  The recurrence is linear in (S, z), so the
// result is the same up to the order of float32 additions.
constexpr int kPart = 1024;
constexpr int kState = kD * kD + kD;  // floats of (S, z) per part and query head

struct LinAttnArgs {
  const int32_t* cu_seqlens;
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  long q_stride, k_stride, v_stride;  // elements between consecutive tokens
  int Hq, Hkv;
  uint16_t* out;  // [rows, Hq, 128]
  float* ws;      // [slots, Hq, kState] (chunk-parallel form)
  int S;
};

__device__ inline int part_slot(const int32_t* cu, int s) { return cu[s] / kPart + s; }

__device__ inline float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// MODE 0: whole segments (blockIdx.y = segment).  MODE 1: part states
// (blockIdx.y = slot; no outputs).  MODE 2: part outputs from the running
// sums of the parts before.
template <int MODE>
__global__ __launch_bounds__(kThreads, 2) void linear_attn_bf16_kernel(LinAttnArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int h = blockIdx.x;
  const int g = h / (a.Hq / a.Hkv);
  int t_begin, t_end, slot = 0, p = 0;
  if (MODE == 0) {
    t_begin = a.cu_seqlens[blockIdx.y];
    t_end = a.cu_seqlens[blockIdx.y + 1];
  } else {
    // the segment owning this slot: the last one whose first slot is <= it
    slot = blockIdx.y;
    int lo = 0, hi = a.S - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (part_slot(a.cu_seqlens, mid) <= slot) lo = mid;
      else hi = mid - 1;
    }
    p = slot - part_slot(a.cu_seqlens, lo);
    const int a0 = a.cu_seqlens[lo], n = a.cu_seqlens[lo + 1] - a0;
    const int np = (n + kPart - 1) / kPart;
    // a slot between two segments' parts, or a segment's last part (whose
    // sums no later part reads)
    if (p < 0 || p >= np || (MODE == 1 && p == np - 1)) return;
    t_begin = a0 + p * kPart;
    t_end = min(a0 + n, t_begin + kPart);
  }
  const int tid = threadIdx.x, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t L0 = lds_addr_of(lds);

  // S and z start at zero, or at the running sums of the parts before
  f32x16 sacc[4];  // S[32i + row][32w + col] blocks, i = d_in block
  if (MODE == 2 && p > 0) {
    const float* prev = a.ws + ((long)(slot - 1) * a.Hq + h) * kState;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[i][e] = prev[(i * 16 + e) * kThreads + tid];
    if (tid < kD) ((float*)(lds + ZF))[tid] = prev[kD * kD + tid];
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[i][e] = 0.f;
    if (tid < kD * 4 / 16) *(u32x4*)(lds + ZF + tid * 16) = u32x4{0u, 0u, 0u, 0u};
  }
  __syncthreads();

  // the chunk's raw q, k, v rows: thread tid handles (row p / 16, 16-byte
  // column chunk p % 16) for p = tid + 256 i (q only where outputs are made)
  u32x4 rq[4], rk[4], rv[4];
  auto load_q = [&](int t0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = tid + kThreads * i, r = p >> 4, c = p & 15;
      rq[i] = u32x4{0u, 0u, 0u, 0u};
      if (MODE != 1 && t0 + r < t_end)
        rq[i] = *(const u32x4*)(a.q + (long)(t0 + r) * a.q_stride + (long)h * kD + c * 8);
    }
  };
  auto load_kv = [&](int t0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = tid + kThreads * i, r = p >> 4, c = p & 15;
      rk[i] = rv[i] = u32x4{0u, 0u, 0u, 0u};
      if (t0 + r < t_end) {
        const long t = t0 + r;
        rk[i] = *(const u32x4*)(a.k + t * a.k_stride + (long)g * kD + c * 8);
        rv[i] = *(const u32x4*)(a.v + t * a.v_stride + (long)g * kD + c * 8);
      }
    }
  };
  const bf16x8 ones = {(__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f,
                       (__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f};

  if (MODE == 1) load_kv(t_begin);
  for (int t0 = t_begin; t0 < t_end; t0 += kC) {
    const int nrows = min(kC, t_end - t0);
    if (MODE != 1) {
      load_q(t0);
      load_kv(t0);
    }
    // (a) the chunk's phi(q), phi(k), v into LDS, token-major; rows past
    // the segment are zero (not phi(0)), so they add nothing to A, S or z
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = tid + kThreads * i, r = p >> 4, c = p & 15;
      const bool ok = r < nrows;
      bf16x8 fq, fk;
      const uint16_t* q16 = (const uint16_t*)&rq[i];
      const uint16_t* k16 = (const uint16_t*)&rk[i];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        fq[e] = ok ? (__bf16)phi(bf2f(q16[e])) : (__bf16)0.f;
        fk[e] = ok ? (__bf16)phi(bf2f(k16[e])) : (__bf16)0.f;
      }
      if (MODE != 1) *(bf16x8*)(lds + QF + off256(r, c * 8)) = fq;
      *(bf16x8*)(lds + KF + off256(r, c * 8)) = fk;
      *(u32x4*)(lds + VF + off256(r, c * 8)) = rv[i];
    }
    // part sums: the next chunk's rows are loaded while this one is
    // computed (the outputs' registers leave no room for that elsewhere)
    if (MODE == 1 && t0 + kC < t_end) load_kv(t0 + kC);
    __syncthreads();

    if (MODE != 1) {
    // (b) wave w: block of A (query rows 32 (w >> 1).., keys 32 (w & 1)..),
    // masked, to LDS as A^T in bf16 (a lane holds 4 consecutive queries of
    // one key: 8-byte stores)
    {
      const int mr = w >> 1, nc = w & 1;
      f32x16 acc2[2];
#pragma unroll
      for (int e = 0; e < 16; ++e) acc2[0][e] = acc2[1][e] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8 qa = *(lbf16x8*)(uintptr_t)(L0 + QF + off256(mr * 32 + l32, ks * 16 + hl * 8));
        const bf16x8 kb = *(lbf16x8*)(uintptr_t)(L0 + KF + off256(nc * 32 + l32, ks * 16 + hl * 8));
        acc2[ks & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kb, acc2[ks & 1], 0, 0, 0);
      }
      const f32x16 acc = acc2[0] + acc2[1];
      const int key = nc * 32 + l32;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        bf16x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = mr * 32 + jj * 8 + hl * 4 + e;
          v4[e] = (__bf16)(key <= row ? acc[jj * 4 + e] : 0.f);
        }
        *(bf16x4*)(lds + AT + off128(key, mr * 32 + jj * 8 + hl * 4)) = v4;
      }
    }
    // (c) phi(Q) . z per row (z of the chunks before this one): row
    // r = tid / 4, quarter x = tid % 4 of the head dimension
    {
      const int r = tid >> 2, x = tid & 3;
      float d = 0.f;
      const float* z = (const float*)(lds + ZF) + x * 32;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8 qv = *(const bf16x8*)(lds + QF + off256(r, x * 32 + j * 8));
        const float4 z0 = *(const float4*)(z + j * 8), z1 = *(const float4*)(z + j * 8 + 4);
        d += (float)qv[0] * z0.x + (float)qv[1] * z0.y + (float)qv[2] * z0.z + (float)qv[3] * z0.w +
             (float)qv[4] * z1.x + (float)qv[5] * z1.y + (float)qv[6] * z1.z + (float)qv[7] * z1.w;
      }
      d += __shfl_xor(d, 1, 64);
      d += __shfl_xor(d, 2, 64);
      if (x == 0) ((float*)(lds + DN))[r] = d;
    }
    __syncthreads();

    // (d) wave w: the transposed outputs O^T = V^T A^T + S^T phi(Q)^T of
    // head dimensions 32w.. for both 32-query blocks, over A 1 + phi(Q) z.
    // A lane then holds 16 dimensions of one query (4 consecutive per
    // register group: 8-byte stores) and needs one denominator per block.
    // V^T and A^T come by transpose reads (keys permuted alike); A 1 from
    // the same A fragments against ones.  S^T comes from this wave's own
    // registers: for the 16 rows of step ks of S, the lane of column c and
    // half h holds rows 4h + 0..3 and 8 + 4h + 0..3, which with phi(Q)'s
    // head dimensions read in the same order (two 8-byte reads) is an
    // operand as it stands; S enters as the bf16 pair hi + lo.
    {
      f32x16 acc[2], den[2];  // numerators; denominator part A 1
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[mb][e] = den[mb][e] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 vt = tr_frag<off256>(L0 + VF, ks * 16, w * 32);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const bf16x8 at = tr_frag<off128>(L0 + AT, ks * 16, mb * 32);
          acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vt, at, acc[mb], 0, 0, 0);
          den[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones, at, den[mb], 0, 0, 0);
        }
      }
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const int i = ks >> 1, j0 = (ks & 1) * 2;
        bf16x8 sh, sl;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = sacc[i][j0 * 4 + e];
          sh[e] = (__bf16)x;
          sl[e] = (__bf16)(x - (float)sh[e]);
        }
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const int qr = mb * 32 + l32;
          const bf16x4 q0 = *(const bf16x4*)(lds + QF + off256(qr, ks * 16 + hl * 4));
          const bf16x4 q1 = *(const bf16x4*)(lds + QF + off256(qr, ks * 16 + 8 + hl * 4));
          const bf16x8 qb = {q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3]};
          acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sh, qb, acc[mb], 0, 0, 0);
          acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sl, qb, acc[mb], 0, 0, 0);
        }
      }
      const float* dqz = (const float*)(lds + DN);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int qr = mb * 32 + l32;
        if (qr < nrows) {
          // every element of den[mb] in this lane is its query's A 1
          const float inv = 1.f / (den[mb][0] + dqz[qr]);
          uint16_t* orow = a.out + ((long)(t0 + qr) * a.Hq + h) * kD + w * 32 + hl * 4;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            bf16x4 v4;
#pragma unroll
            for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(acc[mb][jj * 4 + e] * inv);
            *(bf16x4*)(orow + jj * 8) = v4;
          }
        }
      }
    }
    }  // MODE != 1

    // (e) this chunk's phi(K)^T V into S (registers; wave w's columns), and
    // its key sums phi(K)^T 1 for the 32 head dimensions 32w.. into z (every
    // wave has read z for the denominators before the last barrier)
    {
      f32x16 zacc;
#pragma unroll
      for (int e = 0; e < 16; ++e) zacc[e] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 vb = tr_frag<off256>(L0 + VF, ks * 16, w * 32);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bf16x8 ka = tr_frag<off256>(L0 + KF, ks * 16, i * 32);
          sacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, vb, sacc[i], 0, 0, 0);
          if (i == w) zacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, ones, zacc, 0, 0, 0);
        }
      }
      // every column of zacc holds the same sums: lanes 0 and 32 (column 0)
      // add rows 8jj + 4h + e of block w
      if (l32 == 0) {
        float* z = (float*)(lds + ZF) + w * 32 + hl * 4;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
          for (int e = 0; e < 4; ++e) z[jj * 8 + e] += zacc[jj * 4 + e];
      }
    }
    __syncthreads();
  }
  if (MODE == 1) {
    float* own = a.ws + ((long)slot * a.Hq + h) * kState;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) own[(i * 16 + e) * kThreads + tid] = sacc[i][e];
    if (tid < kD) own[kD * kD + tid] = ((const float*)(lds + ZF))[tid];
  }
}

// pass 2: per (query head, segment, block of 256 state elements), the part
// sums of parts 0..np-2 become running sums (inclusive), in part order,
// eight parts' values loaded ahead of their stores; slots at or past
// `slots` (a batch that breaks cu_seqlens[S] <= rows) are left alone
__global__ __launch_bounds__(256) void linear_attn_prefix_kernel(const int32_t* __restrict__ cu,
                                                                 float* __restrict__ ws, int Hq,
                                                                 int slots) {
  const int h = blockIdx.x, s = blockIdx.y, e = blockIdx.z * 256 + threadIdx.x;
  const int a0 = cu[s], n = cu[s + 1] - a0;
  const int np = (n + kPart - 1) / kPart;
  const long first = part_slot(cu, s);
  if (np < 3 || first < 0 || first + np - 2 >= slots || e >= kState) return;
  const long step = (long)Hq * kState;
  float* x = ws + (first * Hq + h) * kState + e;
  float r = 0.f;
  const int m = np - 1;
  for (int q0 = 0; q0 < m; q0 += 8) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = q0 + j < m ? x[(q0 + j) * step] : 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      r += v[j];
      if (q0 + j < m) x[(q0 + j) * step] = r;
    }
  }
}

}  // namespace

int linear_attn_part_rows() { return kPart; }

size_t linear_attn_workspace_bytes(int rows, int S, int Hq) {
  return (size_t)(rows / kPart + S + 1) * Hq * kState * sizeof(float);
}

hipError_t launch_linear_attn_bf16(const int32_t* cu_seqlens, int S, int rows, const void* q,
                                   long q_stride, const void* k, long k_stride, const void* v,
                                   long v_stride, int Hq, int Hkv, void* out, void* ws,
                                   hipStream_t st) {
  LinAttnArgs a;
  a.cu_seqlens = cu_seqlens;
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.q_stride = q_stride;
  a.k_stride = k_stride;
  a.v_stride = v_stride;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.out = (uint16_t*)out;
  a.ws = (float*)ws;
  a.S = S;
  for (const void* f : {(const void*)linear_attn_bf16_kernel<0>,
                        (const void*)linear_attn_bf16_kernel<1>,
                        (const void*)linear_attn_bf16_kernel<2>}) {
    hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e != hipSuccess) return e;
  }
  // heads fastest: the workgroups of one segment (or part) go out together,
  // and a compute unit that finishes a short one takes the next
  if (!ws) {
    hipLaunchKernelGGL(linear_attn_bf16_kernel<0>, dim3(Hq, S), dim3(kThreads), kLdsBytes, st, a);
    return hipGetLastError();
  }
  const int slots = rows / kPart + S + 1;
  hipLaunchKernelGGL(linear_attn_bf16_kernel<1>, dim3(Hq, slots), dim3(kThreads), kLdsBytes, st, a);
  hipLaunchKernelGGL(linear_attn_prefix_kernel, dim3(Hq, S, (kState + 255) / 256), dim3(256), 0,
                     st, cu_seqlens, a.ws, Hq, slots);
  hipLaunchKernelGGL(linear_attn_bf16_kernel<2>, dim3(Hq, slots), dim3(kThreads), kLdsBytes, st, a);
  return hipGetLastError();
}

}  // namespace up
