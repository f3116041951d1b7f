// Linear maps of a later layer on bf16 matrix cores (gfx950): Y = X W^T over
// the token rows in use, optionally with the SwiGLU gate fused into the
// epilogue.
//
// Why it is part of the path (UniPrefill review, "Method & Key Results";
// UniPrefill paper entry, abstract): tokens dropped at the selection layer
// skip every later sublayer, so the later layers' matrix products run on the
// compacted rows only; this is where the method saves its work.  The shapes
// are Llama-3.1-8B's (hidden 4096, 32 query / 8 KV heads of 128, MLP width
// 14336 gated by SwiGLU: silu(x Wg^T) * (x Wu^T), Shazeer, "GLU Variants
// Improve Transformer", 2020).
//
// Layout: X [rows, K] and W [N, K] row-major bf16 (W in the [out, in] layout
// of a linear layer), Y [rows, N] bf16, or [rows, N/2] with the gate, whose
// W holds gate and up rows interleaved in groups of 32 (rows 64q..64q+31:
// gate rows of features 32q..32q+31; rows 64q+32..64q+63: their up rows).
// The number of rows in use may live on the device (the kept count the
// compaction wrote), so no host synchronisation sits between the two.
//
// Work: a workgroup of 8 waves (2 per SIMD) computes one 256-token x
// 256-feature tile of Y^T = W X^T; wave (wn, wm) owns 128 features x 64
// tokens as 4 x 2 blocks of v_mfma_f32_32x32x16_bf16 (A = W rows, B = X
// rows: both read as 16 contiguous bytes of one row per lane).  K advances
// in stages of 64: the two 256 x 64 operand tiles of a stage arrive in LDS
// by direct global->LDS copies issued one stage ahead (two stage buffers,
// 128 KiB), one barrier per stage.  A 128-byte LDS row holds its eight
// 16-byte chunks XOR-swizzled by (row >> 1) & 7, so the 16 rows one
// fragment read touches per pass fall on distinct banks.
//
// Tile order (8 XCDs with private L2): tiles are grouped in chunks of 32
// (CM token tiles x CN feature tiles) that one XCD's 32 compute units run
// side by side, sharing CM X panels and CN W panels in that XCD's L2;
// chunks go to XCDs round robin (workgroup b runs on XCD b mod 8), so the
// tiles that exit early because fewer rows are in use spread over all XCDs.
#include "common.h"
#include "lds_copy.h"

namespace up {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) const bf16x8 lbf16x8;

constexpr int kBM = 256;                  // tokens per tile
constexpr int kBN = 256;                  // features (rows of W) per tile
constexpr int kBK = 64;                   // k per stage
constexpr int kThreads = 512;             // 8 waves
constexpr int kRowBytes = kBK * 2;        // one tile row in LDS
constexpr int kTileBytes = 256 * kRowBytes;
constexpr int kStageBytes = 2 * kTileBytes;  // X tile, then W tile
constexpr int kLdsBytes = 2 * kStageBytes;
constexpr int kCopies = kTileBytes / (kThreads * 16);  // per thread per tile
constexpr int kChunkTiles = 32;
constexpr int kXcds = 8;
static_assert(kCopies * kThreads * 16 == kTileBytes, "copy split");
static_assert(kLdsBytes <= 160 * 1024, "LDS");

struct LinearArgs {
  const uint8_t* x;
  const uint8_t* w;
  uint16_t* y;
  const int32_t* rows_dev;
  int rows_cap, N, K, act;
  int tiles_m, tiles_n, cm, cn, chunks_n, chunks;
};

__device__ inline int swz(int r) { return (r >> 1) & 7; }

// Per-lane source offsets of a stage's copies.  Copy j of wave w moves tile
// rows rb..rb+7, rb = (4w + j) * 8; lane i brings global chunk
// (i % 8) ^ swz(row) of row rb + i / 8 to LDS chunk slot i % 8 of that row.
// X rows past the rows in use read the last row in use (finite data; their
// results are not stored).  The offsets are 32-bit (the host checks that
// both matrices are under 4 GiB); a stage only moves the common base.
struct CopyOffsets {
  uint32_t x[kCopies], w[kCopies];
  __device__ inline CopyOffsets(const LinearArgs& a, int m0, int n0, int M, int wv, int lane) {
    const uint32_t ldb = (uint32_t)a.K * 2;
    const int sub = lane >> 3, slot = lane & 7;
#pragma unroll
    for (int j = 0; j < kCopies; ++j) {
      const int r = (wv * kCopies + j) * 8 + sub;
      const uint32_t c = (uint32_t)(slot ^ swz(r)) << 4;
      x[j] = (uint32_t)min(m0 + r, M - 1) * ldb + c;
      w[j] = (uint32_t)(n0 + r) * ldb + c;
    }
  }
};

// copies of stage kt (k in [64 kt, 64 kt + 64)) into the stage buffer at
// LDS address `stage`
__device__ inline void stage_copies(const LinearArgs& a, const CopyOffsets& co, int kt,
                                    uint32_t stage, int wv) {
  const uint8_t* xs = a.x + (long)kt * kRowBytes;
  const uint8_t* ws = a.w + (long)kt * kRowBytes;
#pragma unroll
  for (int j = 0; j < kCopies; ++j) {
    const int rb = (wv * kCopies + j) * 8;
    lds_copy16_sv(xs, co.x[j], stage + rb * kRowBytes);
    lds_copy16_sv(ws, co.w[j], stage + kTileBytes + rb * kRowBytes);
  }
}

__device__ inline float silu(float x) { return x / (1.f + __expf(-x)); }

__global__ __launch_bounds__(kThreads) void linear_bf16_kernel(LinearArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  // workgroup -> (chunk, tile in chunk) -> (token tile, feature tile)
  const int b = blockIdx.x;
  const int slot = b / kXcds;
  const int chunk = (slot / kChunkTiles) * kXcds + b % kXcds;
  if (chunk >= a.chunks) return;
  const int pos = slot % kChunkTiles;
  const int tm = (chunk / a.chunks_n) * a.cm + pos / a.cn;
  const int tn = (chunk % a.chunks_n) * a.cn + pos % a.cn;
  if (tm >= a.tiles_m) return;
  int M = a.rows_cap;
  if (a.rows_dev) M = min(M, *a.rows_dev);
  const int m0 = tm * kBM, n0 = tn * kBN;
  if (m0 >= M) return;

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = w & 1, wm = w >> 1;
  const uint32_t l0 = lds_addr_of(lds);
  // per lane, for k16 step ks: row lane % 32 of a 32-row block, chunk
  // (2 ks + h) swizzled by that row (block and wave offsets are multiples
  // of 32 rows, which leave the swizzle unchanged)
  uint32_t koff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    koff[ks] = (lane & 31) * kRowBytes + ((((ks << 1) | h) ^ swz(lane & 31)) << 4);

  f32x16 acc[4][2];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[nb][mb][e] = 0.f;

  const int nk = a.K / kBK;
  const CopyOffsets co(a, m0, n0, M, w, lane);
  stage_copies(a, co, 0, l0, w);
  for (int kt = 0; kt < nk; ++kt) {
    // stage kt has landed (every wave waited for its own copies before the
    // barrier) and every wave is done reading the other buffer
    lds_copy_wait<0>();
    lds_only_barrier();
    if (kt + 1 < nk) stage_copies(a, co, kt + 1, l0 + ((kt + 1) & 1) * kStageBytes, w);
    const uint32_t xb = l0 + (kt & 1) * kStageBytes + wm * 64 * kRowBytes;
    const uint32_t wb = l0 + (kt & 1) * kStageBytes + kTileBytes + wn * 128 * kRowBytes;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 af[4], bx[2];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        af[nb] = *(lbf16x8*)(uintptr_t)(wb + koff[ks] + nb * 32 * kRowBytes);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        bx[mb] = *(lbf16x8*)(uintptr_t)(xb + koff[ks] + mb * 32 * kRowBytes);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[nb], bx[mb], acc[nb][mb], 0, 0, 0);
    }
  }

  // epilogue: lane holds Y^T[n][m] for m = its token, n = 8 jj + 4 h + e of
  // each 32-feature block
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int m = m0 + wm * 64 + mb * 32 + (lane & 31);
    if (m >= M) continue;
    if (a.act == 0) {
      uint16_t* yrow = a.y + (long)m * a.N + n0 + wn * 128;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          bf16x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (__bf16)acc[nb][mb][jj * 4 + e];
          *(bf16x4*)(yrow + nb * 32 + jj * 8 + h * 4) = v;
        }
    } else {
      const int F = a.N / 2;
      uint16_t* yrow = a.y + (long)m * F + n0 / 2 + wn * 64;
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          bf16x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            v[e] = (__bf16)(silu(acc[2 * p][mb][jj * 4 + e]) * acc[2 * p + 1][mb][jj * 4 + e]);
          *(bf16x4*)(yrow + p * 32 + jj * 8 + h * 4) = v;
        }
    }
  }
}

}  // namespace

hipError_t launch_linear_bf16(const void* x, const void* w, void* y, int rows_cap,
                              const int32_t* rows_dev, int N, int K, int act, hipStream_t st) {
  if (rows_cap == 0) return hipSuccess;
  LinearArgs a;
  a.x = (const uint8_t*)x;
  a.w = (const uint8_t*)w;
  a.y = (uint16_t*)y;
  a.rows_dev = rows_dev;
  a.rows_cap = rows_cap;
  a.N = N;
  a.K = K;
  a.act = act;
  a.tiles_m = (rows_cap + kBM - 1) / kBM;
  a.tiles_n = N / kBN;
  // chunk shape CM x CN = 32 tiles: an XCD's L2 fetches CM + CN panels per
  // chunk, fewest for the squarest shape (4 x 8 = 12 panels, against 18 for
  // 2 x 16), so CN is the first of 8, 4, 16, 2 that divides the feature tiles
  a.cn = 1;
  for (int c : {8, 4, 16, 2})
    if (a.tiles_n % c == 0) {
      a.cn = c;
      break;
    }
  a.cm = kChunkTiles / a.cn;
  a.chunks_n = a.tiles_n / a.cn;
  a.chunks = ((a.tiles_m + a.cm - 1) / a.cm) * a.chunks_n;
  // every (chunk, tile) pair gets a workgroup: whole rounds of 8 chunks
  const long grid = (long)((a.chunks + kXcds - 1) / kXcds) * kXcds * kChunkTiles;
  hipError_t e = hipFuncSetAttribute((const void*)linear_bf16_kernel,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(linear_bf16_kernel, dim3((unsigned)grid), dim3(kThreads), kLdsBytes, st, a);
  return hipGetLastError();
}

}  // namespace up
