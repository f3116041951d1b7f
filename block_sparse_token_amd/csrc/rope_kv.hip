// Rotary embedding of the new keys and the paged KV-cache write.
//
// Every new token's K (rotated by its position) and V are stored at its slot
// (page * 16 + offset) of the caches [num_pages, Hkv, 16, D], which is how
// the prefill keeps its keys and values for later chunks (glossary page
// "Chunked Prefill": a chunk attends the cached K/V of earlier chunks; its
// "Related serving techniques" section: the cache is kept in fixed-size
// pages).  Rotation: pairs (j, j + D/2), angle = position * theta^(-2j/D).
//
// One thread per (token, pair index j); it walks the KV heads, so each angle
// is computed once per token.  Loads and stores of a wave cover contiguous
// half rows.
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

hipError_t launch_rope_kv(const RopeArgs& a, bool bf16, int D, hipStream_t st) {
  const int tpb = 256 / (D / 2);
  dim3 grid((a.T + tpb - 1) / tpb);
  if (bf16) {
    if (D == 128) hipLaunchKernelGGL((rope_kv_kernel<uint16_t, 128>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((rope_kv_kernel<uint16_t, 64>), grid, dim3(256), 0, st, a);
  } else {
    if (D == 128) hipLaunchKernelGGL((rope_kv_kernel<float, 128>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((rope_kv_kernel<float, 64>), grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace up
