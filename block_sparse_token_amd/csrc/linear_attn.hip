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
// All four products run on v_mfma_f32_32x32x16_bf16.  S stays in float32
// registers (wave w owns output columns 32w..32w+31, which are the columns
// of the outputs it computes); the product phi(Q_c) S takes it from there
// as the bf16 pair hi + lo (hi the rounding of S, lo that of the
// remainder), so S enters with about 16 significant bits.  With no copy of
// S in LDS, two workgroups share a compute unit.  The denominators use the same bf16 A and phi(K) as the
// numerators.  LDS tiles are row-major with 16-byte chunks XOR-swizzled per
// row, so fragment reads of 16 rows fall on distinct banks; phi(K) and V
// are also stored transposed (key-minor), which is the layout the products
// over keys read.
#include "common.h"
#include "lds_copy.h"

namespace up {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const bf16x8 lbf16x8;

constexpr int kC = 64;   // tokens per chunk
constexpr int kD = 128;  // head dimension
constexpr int kThreads = 256;
// LDS layout (bytes)
constexpr int QF = 0;                  // phi(Q) [64][128]   rows of 256 B
constexpr int KF = QF + kC * kD * 2;   // phi(K) [64][128]
constexpr int KT = KF + kC * kD * 2;   // phi(K)^T [128][64] rows of 128 B
constexpr int VT = KT + kD * kC * 2;   // V^T [128][64]
constexpr int AB = VT + kD * kC * 2;   // A [64][64]         rows of 128 B
constexpr int ZF = AB + kC * kC * 2;   // z [128] f32
constexpr int DN = ZF + kD * 4;        // denominators [64] f32
constexpr int kLdsBytes = DN + kC * 4;
static_assert(2 * kLdsBytes <= 160 * 1024, "two workgroups per compute unit");

// byte offset of element (r, e) in a row-major bf16 tile with 256-byte rows
__device__ inline int off256(int r, int e) { return r * 256 + ((((e >> 3) ^ (r & 15))) << 4) + (e & 7) * 2; }
// ... with 128-byte rows
__device__ inline int off128(int r, int e) { return r * 128 + ((((e >> 3) ^ ((r >> 1) & 7))) << 4) + (e & 7) * 2; }

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
  // column chunk p % 16) for p = tid + 256 i
  u32x4 rq[4], rk[4], rv[4];
  auto load_chunk = [&](int t0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = tid + kThreads * i, r = p >> 4, c = p & 15;
      rq[i] = rk[i] = rv[i] = u32x4{0u, 0u, 0u, 0u};
      if (t0 + r < t_end) {
        const long t = t0 + r;
        if (MODE != 1) rq[i] = *(const u32x4*)(a.q + t * a.q_stride + (long)h * kD + c * 8);
        rk[i] = *(const u32x4*)(a.k + t * a.k_stride + (long)g * kD + c * 8);
        rv[i] = *(const u32x4*)(a.v + t * a.v_stride + (long)g * kD + c * 8);
      }
    }
  };

  for (int t0 = t_begin; t0 < t_end; t0 += kC) {
    const int nrows = min(kC, t_end - t0);
    load_chunk(t0);
    // (a) the chunk's phi(q), phi(k), v into LDS; rows past the segment are
    // zero (not phi(0)), so they add nothing to A, S or z
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = tid + kThreads * i, r = p >> 4, c = p & 15;
      const bool ok = r < nrows;
      bf16x8 fq, fk;
      const uint16_t* q16 = (const uint16_t*)&rq[i];
      const uint16_t* k16 = (const uint16_t*)&rk[i];
      const uint16_t* v16 = (const uint16_t*)&rv[i];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        fq[e] = ok ? (__bf16)phi(bf2f(q16[e])) : (__bf16)0.f;
        fk[e] = ok ? (__bf16)phi(bf2f(k16[e])) : (__bf16)0.f;
      }
      if (MODE != 1) {
        *(bf16x8*)(lds + QF + off256(r, c * 8)) = fq;
        *(bf16x8*)(lds + KF + off256(r, c * 8)) = fk;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        *(__bf16*)(lds + KT + off128(c * 8 + e, r)) = fk[e];
        *(uint16_t*)(lds + VT + off128(c * 8 + e, r)) = v16[e];
      }
    }
    __syncthreads();

    if (MODE != 1) {
    // (b) wave w: A block (rows 32 (w >> 1).., keys 32 (w & 1)..), masked,
    // to LDS in bf16
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
      for (int jj = 0; jj < 4; ++jj)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = mr * 32 + jj * 8 + hl * 4 + e;
          *(__bf16*)(lds + AB + off128(row, key)) = (__bf16)(key <= row ? acc[jj * 4 + e] : 0.f);
        }
    }
    __syncthreads();

    // (c) denominators: row r = tid / 4, quarter x = tid % 4 sums A[r][16x..]
    // and phi(Q)[r][32x..] . z (z of the chunks before this one)
    {
      const int r = tid >> 2, x = tid & 3;
      float d = 0.f;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const bf16x8 av = *(const bf16x8*)(lds + AB + off128(r, x * 16 + j * 8));
#pragma unroll
        for (int e = 0; e < 8; ++e) d += (float)av[e];
      }
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

    // (d) wave w: outputs of columns 32w.. for both 32-row blocks:
    // A V + phi(Q) S, divided by the row's denominator.  S comes from this
    // wave's own registers: for the 16 rows of step ks, lane (c, half 0)
    // holds rows 8jj + 0..3 of column c and lane (c, half 1) rows 8jj +
    // 4..7; one v_permlane32_swap per register pair gives each lane the 8
    // consecutive rows the product reads, split into bf16 hi + lo.
    {
      f32x16 acc[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[mb][e] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 vb = *(lbf16x8*)(uintptr_t)(L0 + VT + off128(w * 32 + l32, ks * 16 + hl * 8));
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const bf16x8 aa = *(lbf16x8*)(uintptr_t)(L0 + AB + off128(mb * 32 + l32, ks * 16 + hl * 8));
          acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aa, vb, acc[mb], 0, 0, 0);
        }
      }
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const int i = ks >> 1, j0 = (ks & 1) * 2;
        bf16x8 sh, sl;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(sacc[i][j0 * 4 + e]),
                                                          __float_as_uint(sacc[i][j0 * 4 + 4 + e]),
                                                          false, false);
          const float lo_rows = __uint_as_float(r[0]), hi_rows = __uint_as_float(r[1]);
          sh[e] = (__bf16)lo_rows;
          sl[e] = (__bf16)(lo_rows - (float)sh[e]);
          sh[4 + e] = (__bf16)hi_rows;
          sl[4 + e] = (__bf16)(hi_rows - (float)sh[4 + e]);
        }
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const bf16x8 qa = *(lbf16x8*)(uintptr_t)(L0 + QF + off256(mb * 32 + l32, ks * 16 + hl * 8));
          acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, sh, acc[mb], 0, 0, 0);
          acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, sl, acc[mb], 0, 0, 0);
        }
      }
      const float* den = (const float*)(lds + DN);
      const int col = w * 32 + l32;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int row = mb * 32 + jj * 8 + hl * 4 + e;
            if (row < nrows) {
              const float o = acc[mb][jj * 4 + e] / den[row];
              *(__bf16*)(a.out + ((long)(t0 + row) * a.Hq + h) * kD + col) = (__bf16)o;
            }
          }
    }
    }  // MODE != 1

    // (e) this chunk's phi(K)^T V into S (registers; wave w's columns), and
    // its keys into z once every wave has read z for the denominators
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 vb = *(lbf16x8*)(uintptr_t)(L0 + VT + off128(w * 32 + l32, ks * 16 + hl * 8));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8 ka = *(lbf16x8*)(uintptr_t)(L0 + KT + off128(i * 32 + l32, ks * 16 + hl * 8));
        sacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, vb, sacc[i], 0, 0, 0);
      }
    }
    {
      const int d = tid >> 1, half = tid & 1;
      float zs = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8 kv = *(const bf16x8*)(lds + KT + off128(d, half * 32 + j * 8));
#pragma unroll
        for (int e = 0; e < 8; ++e) zs += (float)kv[e];
      }
      zs += __shfl_xor(zs, 1, 64);
      if (half == 0) ((float*)(lds + ZF))[d] += zs;
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
