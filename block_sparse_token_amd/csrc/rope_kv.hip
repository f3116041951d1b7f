// Rotary embedding of the new keys and the paged KV-cache write.
//
// Every new token's K (rotated by its position) and V are stored at its slot
// (page * 16 + offset) of the caches [num_pages, Hkv, 16, D], which is how
// the prefill keeps its keys and values for later chunks (glossary page
// "Chunked Prefill": a chunk attends the cached K/V of earlier chunks; its
// "Related serving techniques" section: the cache is kept in fixed-size
// pages).  Rotation: pairs (j, j + D/2), angle = position * theta^(-2j/D).
//
// bf16: one wave per token; lane (head, group of 8 pairs) moves 16-byte
// chunks of the K halves and V and computes its 8 angles once, reused for
// every head it visits.  fp32: one thread per (token, pair index j), walking
// the KV heads.
#include "common.h"

namespace up {

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  __device__ static float ld(const float* p) { return *p; }
  __device__ static void st(float* p, float x) { *p = x; }
};
template <>
struct Elem<uint16_t> {
  __device__ static float ld(const uint16_t* p) { return __uint_as_float(((uint32_t)*p) << 16); }
  __device__ static void st(uint16_t* p, float x) {
    __bf16 b = (__bf16)x;
    *p = __builtin_bit_cast(uint16_t, b);
  }
};

// cos/sin of 2*pi*turns for turns = pos * rev, reduced to [-0.5, 0.5) in fp64.
template <bool kAccurate>
__device__ inline void rope_cs(int pos, double rev, float& c, float& s) {
  double t = (double)pos * rev;
  t -= rint(t);
  if (kAccurate) {
    sincosf((float)(t * 6.283185307179586476925286766559), &s, &c);
  } else {
    // hardware sin/cos take their input in turns
    s = __builtin_amdgcn_sinf((float)t);
    c = __builtin_amdgcn_cosf((float)t);
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void rope_kv_kernel(RopeArgs a) {
  constexpr int H = D / 2;
  constexpr int TOK_PER_BLOCK = 256 / H;
  const int t = blockIdx.x * TOK_PER_BLOCK + threadIdx.x / H;
  const int j = threadIdx.x % H;
  if (t >= a.T) return;
  const int T_used = a.cu_seqlens[a.S];
  if (t >= T_used) return;
  const int slot = a.slot_mapping[t];
  if (slot < 0) return;
  const int page = slot / kPageSize, off = slot % kPageSize;
  float c = 1.f, s = 0.f;
  if (a.rope) rope_cs<std::is_same<T, float>::value>(a.positions[t], a.rope_rev[j], c, s);
  const T* k = (const T*)a.k;
  const T* v = (const T*)a.v;
  T* kc = (T*)a.k_cache;
  T* vc = (T*)a.v_cache;
  for (int g = 0; g < a.Hkv; ++g) {
    const size_t src = ((size_t)t * a.Hkv + g) * D;
    const size_t dst = (((size_t)page * a.Hkv + g) * kPageSize + off) * D;
    const float x1 = Elem<T>::ld(k + src + j), x2 = Elem<T>::ld(k + src + j + H);
    Elem<T>::st(kc + dst + j, x1 * c - x2 * s);
    Elem<T>::st(kc + dst + j + H, x2 * c + x1 * s);
    vc[dst + j] = v[src + j];
    vc[dst + j + H] = v[src + j + H];
  }
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4 gcu32x4;
typedef __attribute__((address_space(1))) u32x4 gu32x4;

__device__ inline float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ inline uint32_t bf_pack(float lo, float hi) {
  const __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

template <int D>
__global__ __launch_bounds__(256) void rope_kv_bf16_kernel(RopeArgs a) {
  constexpr int H = D / 2;
  constexpr int PG = H / 8;     // groups of 8 pairs per head
  constexpr int HPI = 64 / PG;  // heads per pass of the wave
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T || t >= a.cu_seqlens[a.S]) return;
  const int slot = a.slot_mapping[t];
  if (slot < 0) return;
  const int page = slot / kPageSize, off = slot % kPageSize;
  const int jg = lane % PG, gl = lane / PG;
  const int pos = a.rope ? a.positions[t] : 0;
  float c[8], s[8];
  bool angles = false;
  const uint16_t* k = (const uint16_t*)a.k;
  const uint16_t* v = (const uint16_t*)a.v;
  uint16_t* kc = (uint16_t*)a.k_cache;
  uint16_t* vc = (uint16_t*)a.v_cache;
  for (int g0 = 0; g0 < a.Hkv; g0 += HPI) {
    const int g = g0 + gl;
    if (g >= a.Hkv) break;
    const size_t src = ((size_t)t * a.Hkv + g) * D + jg * 8;
    const size_t dst = (((size_t)page * a.Hkv + g) * kPageSize + off) * D + jg * 8;
    const u32x4 k1 = *(gcu32x4*)(k + src), k2 = *(gcu32x4*)(k + src + H);
    const u32x4 v1 = *(gcu32x4*)(v + src), v2 = *(gcu32x4*)(v + src + H);
    // the angles once per token, after the first pass's loads are out, so
    // their arithmetic runs while the loads are in flight
    if (!angles) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        c[e] = 1.f;
        s[e] = 0.f;
      }
      if (a.rope)
#pragma unroll
        for (int e = 0; e < 8; ++e) rope_cs<false>(pos, a.rope_rev[jg * 8 + e], c[e], s[e]);
      angles = true;
    }
    u32x4 y1, y2;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float a0 = bf_lo(k1[q]), a1 = bf_hi(k1[q]);
      const float b0 = bf_lo(k2[q]), b1 = bf_hi(k2[q]);
      const int e0 = 2 * q, e1 = 2 * q + 1;
      y1[q] = bf_pack(a0 * c[e0] - b0 * s[e0], a1 * c[e1] - b1 * s[e1]);
      y2[q] = bf_pack(b0 * c[e0] + a0 * s[e0], b1 * c[e1] + a1 * s[e1]);
    }
    *(gu32x4*)(kc + dst) = y1;
    *(gu32x4*)(kc + dst + H) = y2;
    *(gu32x4*)(vc + dst) = v1;
    *(gu32x4*)(vc + dst + H) = v2;
  }
}

hipError_t launch_rope_kv(const RopeArgs& a, bool bf16, int D, hipStream_t st) {
  if (bf16) {
    dim3 grid((a.T + 3) / 4);
    if (D == 128) hipLaunchKernelGGL((rope_kv_bf16_kernel<128>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((rope_kv_bf16_kernel<64>), grid, dim3(256), 0, st, a);
  } else {
    const int tpb = 256 / (D / 2);
    dim3 grid((a.T + tpb - 1) / tpb);
    if (D == 128) hipLaunchKernelGGL((rope_kv_kernel<float, 128>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((rope_kv_kernel<float, 64>), grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace up
