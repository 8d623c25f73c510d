// HIP kernels of the block-diffusion denoising step, written for gfx950 (CDNA4).
//
// Dense contractions (QKV/O projections, router logits, expert SwiGLU FFNs,
// LM head) run on MFMA: v_mfma_f32_16x16x32_bf16 for bf16 (fp8 expert weights
// are widened to bf16 in registers with the gfx950 scaled converters), and
// v_mfma_f32_16x16x4_f32 for float32 models.  At the batch sizes of a
// denoising step these contractions stream weights from HBM with few rows,
// so every tile keeps all rows of its token group and splits the reduction
// dimension across the waves of the workgroup to keep enough loads in flight.
//
// Integer decisions (router top-k, expert permutation, unmask selection,
// retention selection) use wavefront shuffles/ballots and LDS scans with
// fixed tie rules, so they are deterministic and reproducible bit for bit.
// No kernel uses floating-point atomics.
#include "dllm_internal.h"

#include <math.h>

#include <type_traits>

namespace dllm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// scalar helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf2f(uint16_t u) { return __uint_as_float(((uint32_t)u) << 16); }

__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)0x7fc0;  // NaN stays NaN
  u += 0x7fffu + ((u >> 16) & 1u);                                // nearest, ties to even
  return (uint16_t)(u >> 16);
}

template <typename T> __device__ __forceinline__ float ld1(const T* p);
template <> __device__ __forceinline__ float ld1<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ld1<uint16_t>(const uint16_t* p) { return bf2f(*p); }
template <typename T> __device__ __forceinline__ void st1(T* p, float v);
template <> __device__ __forceinline__ void st1<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void st1<uint16_t>(uint16_t* p, float v) { *p = f2bf(v); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Block-wide sum over blockDim.x threads (multiple of 64); every thread gets
// the total.  Fixed reduction order: deterministic.
__device__ float block_sum(float v, float* tmp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) tmp[wave] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += tmp[i];
  return t;
}

// Block-wide exclusive prefix sum of ints (blockDim.x multiple of 64, <= 1024).
__device__ int block_exclusive_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  __syncthreads();
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  int base = 0, tot = 0;
  for (int i = 0; i < nw; ++i) {
    if (i < wave) base += tmp[i];
    tot += tmp[i];
  }
  *total = tot;
  return base + x - v;
}

// ---------------------------------------------------------------------------
// MFMA fragment operations.  A wave computes a 16x16 tile D = A B with A rows
// = tokens and B columns = weight rows.  Lane l holds row/column (l % 16) and
// the 8 consecutive reduction elements starting at 8 * (l / 16) of a 32-wide
// chunk; the accumulator holds D[4 * (l / 16) + v][l % 16], v = 0..3.
// ---------------------------------------------------------------------------

template <int MODE> struct Op;

template <> struct Op<MODE_BF16> {
  static constexpr int KL = 8;        // reduction elements per lane and fragment
  static constexpr int KC = 4 * KL;   // reduction elements per fragment
  typedef uint16_t TA;
  typedef uint16_t TW;
  typedef uint4 AF;
  typedef uint4 WF;
  __device__ static AF lda(const TA* p) { return *(const uint4*)p; }
  __device__ static AF za() { return make_uint4(0, 0, 0, 0); }
  __device__ static WF ldw(const TW* p) { return *(const uint4*)p; }
  __device__ static void mma(f32x4& c, const AF& a, const WF& w) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, w), c, 0, 0, 0);
  }
};

// fp8 weights: one 16-byte load per lane covers 16 reduction elements, so a
// fragment spans 64 (lane group g holds 16 g .. 16 g + 15) and feeds two
// MFMAs, the first taking elements 0..7 of every lane group and the second
// 8..15.  The activation fragment holds the same 16 elements per lane, so the
// two operands pair every reduction index with itself.
struct A16 { uint4 lo, hi; };
template <> struct Op<MODE_FP8> {
  static constexpr int KL = 16;
  static constexpr int KC = 4 * KL;
  typedef uint16_t TA;
  typedef uint8_t TW;
  typedef A16 AF;
  typedef uint4 WF;
  __device__ static AF lda(const TA* p) { return A16{*(const uint4*)p, *(const uint4*)(p + 8)}; }
  __device__ static AF za() { return A16{make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0)}; }
  __device__ static WF ldw(const TW* p) { return *(const uint4*)p; }
  // OCP E4M3FN -> bf16 is exact (3 mantissa bits, exponent range inside bf16).
  __device__ static bf16x8 widen(const uint2& w) {
    bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, false);
    bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, true);
    bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, false);
    bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, true);
    bf16x8 r;
    r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
    r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
    return r;
  }
  __device__ static void mma(f32x4& c, const AF& a, const WF& w) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a.lo), widen(make_uint2(w.x, w.y)), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a.hi), widen(make_uint2(w.z, w.w)), c, 0, 0, 0);
  }
};

struct F8x { float4 a, b; };

template <> struct Op<MODE_F32> {
  static constexpr int KL = 8;
  static constexpr int KC = 4 * KL;
  typedef float TA;
  typedef float TW;
  typedef F8x AF;
  typedef F8x WF;
  __device__ static AF lda(const TA* p) { return F8x{((const float4*)p)[0], ((const float4*)p)[1]}; }
  __device__ static AF za() { return F8x{make_float4(0, 0, 0, 0), make_float4(0, 0, 0, 0)}; }
  __device__ static WF ldw(const TW* p) { return lda(p); }
  __device__ static void mma(f32x4& c, const AF& a, const WF& w) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a.x, w.a.x, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a.y, w.a.y, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a.z, w.a.z, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a.w, w.a.w, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b.x, w.b.x, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b.y, w.b.y, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b.z, w.b.z, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b.w, w.b.w, c, 0, 0, 0);
  }
};

// Calls f(std::integral_constant<int, U>) with the largest U <= UMAX (a power
// of two) dividing the chunk count; UMAX keeps the register footprint of the
// widest row-tile variant near 128 VGPRs.  Only U <= UMAX are instantiated.
template <int U> using IC = std::integral_constant<int, U>;
template <int UMAX, class F>
__host__ __device__ __forceinline__ void pick_u(int ch, F&& f) {
  if constexpr (UMAX >= 16) { if (ch % 16 == 0) { f(IC<16>{}); return; } }
  if constexpr (UMAX >= 8) { if (ch % 8 == 0) { f(IC<8>{}); return; } }
  if constexpr (UMAX >= 4) { if (ch % 4 == 0) { f(IC<4>{}); return; } }
  if constexpr (UMAX >= 2) { if (ch % 2 == 0) { f(IC<2>{}); return; } }
  f(IC<1>{});
}

#ifndef DLLM_UCAP_FP8
#define DLLM_UCAP_FP8 8
#endif
template <int MODE> struct UCap { static constexpr int v = MODE == MODE_F32 ? 4 : (MODE == MODE_FP8 ? DLLM_UCAP_FP8 : 8); };

// One batch of U 32-wide reduction chunks for NRT row tiles (16 rows each)
// and NW weight matrices sharing the A rows (NW = 2: gate and up).  Every
// load of the batch is issued before the first MFMA, so a wavefront keeps
// U * NW weight fragments (U * NW KB) in flight.
template <int MODE, int NRT, int NW, int U>
__device__ __forceinline__ void mma_batch(f32x4 (&acc)[NW][NRT], const typename Op<MODE>::TA* const (&ap)[NRT],
                                          const bool (&av)[NRT], const typename Op<MODE>::TW* const (&wp)[NW],
                                          int k) {
  typedef Op<MODE> O;
  typename O::WF wf[NW][U];
  typename O::AF af[NRT][U];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int w = 0; w < NW; ++w) wf[w][u] = O::ldw(wp[w] + k + 32 * u);
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int u = 0; u < U; ++u) af[rt][u] = av[rt] ? O::lda(ap[rt] + k + 32 * u) : O::za();
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int w = 0; w < NW; ++w) O::mma(acc[w][rt], af[rt][u], wf[w][u]);
}

// Whole-line form of mma_batch for bf16 weights (U even): a fragment-order
// load reads 16 weight rows x 64 bytes, half of each 128-byte line, and the
// number of lines in flight, not bytes, limits a CU.  Here each load reads 8
// rows x 128 bytes (load i of matrix w: rows 8 (i & 1) + lane / 8, reduction
// elements 64 (i >> 1) + 8 (lane % 8)); the wavefront writes the U KB of each
// matrix to its own LDS block (16 rows at a pitch of 64 U + 16 bytes) and reads
// it back in fragment order (lane l: row l % 16, elements 32 u + 8 (l / 16)).
// wlo / whi: this lane's row in the first / second group of 8 rows, at the
// lane's 8-element offset; wl: the wavefront's NW * 16 * (64 U + 16) bytes.
template <int NRT, int NW, int U>
__device__ __forceinline__ void mma_batch_lines(f32x4 (&acc)[NW][NRT], const uint16_t* const (&ap)[NRT],
                                                const bool (&av)[NRT], const uint16_t* const (&wlo)[NW],
                                                const uint16_t* const (&whi)[NW], int k, uint8_t* wl) {
  static_assert(U % 2 == 0, "whole lines take two 32-element chunks per row");
  constexpr int P = 64 * U + 16;
  typedef Op<MODE_BF16> O;
  const int lane = threadIdx.x & 63;
  const int lr = lane >> 3, lq = lane & 7;
  __builtin_amdgcn_wave_barrier();   // the previous batch's LDS reads stay before these writes
  uint4 wv[NW][U];
#pragma unroll
  for (int w = 0; w < NW; ++w)
#pragma unroll
    for (int i = 0; i < U; ++i) wv[w][i] = *(const uint4*)(((i & 1) ? whi[w] : wlo[w]) + k + 64 * (i >> 1));
  typename O::AF af[NRT][U];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int u = 0; u < U; ++u) af[rt][u] = av[rt] ? O::lda(ap[rt] + k + 32 * u) : O::za();
#pragma unroll
  for (int w = 0; w < NW; ++w)
#pragma unroll
    for (int i = 0; i < U; ++i)
      *(uint4*)(wl + w * 16 * P + (8 * (i & 1) + lr) * P + (64 * (i >> 1) + 8 * lq) * 2) = wv[w][i];
  // other lanes' writes are read back; a wavefront's LDS operations complete in order
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const uint4 wf = *(const uint4*)(wl + w * 16 * P + (lane & 15) * P + (32 * u + 8 * (lane >> 4)) * 2);
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) O::mma(acc[w][rt], af[rt][u], wf);
    }
}

// Sum the K-split partial accumulators of the NWAVE wavefronts into wave 0.
// red holds (NWAVE - 1) * NRT * 4 * 64 floats.
template <int NRT, int NWAVE>
__device__ __forceinline__ void reduce_waves(f32x4 (&acc)[NRT], float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();   // previous users of red are done
  if (wave > 0) {
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[(((wave - 1) * NRT + rt) * 4 + v) * 64 + lane] = acc[rt][v];
  }
  __syncthreads();
  if (wave == 0) {
    if constexpr (NRT <= 2) {
      for (int w = 1; w < NWAVE; ++w)
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[rt][v] += red[(((w - 1) * NRT + rt) * 4 + v) * 64 + lane];
    } else {
      // wide tiles: one wavefront's partials at a time keeps the loads in
      // flight to 4 * NRT registers
#pragma unroll 1
      for (int w = 1; w < NWAVE; ++w)
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[rt][v] += red[(((w - 1) * NRT + rt) * 4 + v) * 64 + lane];
    }
  }
}

// ---------------------------------------------------------------------------
// dense GEMM: C[M, N] (=|+=) A[M, K] W[N, K]^T.  Workgroup = 8 wavefronts
// splitting K; tile = 16 * NRT rows x 16 columns.  Rows of A may be gathered
// through row_map; the row count may live on the device (M_dev).
// ---------------------------------------------------------------------------

constexpr int kGemmWaves = 8;

template <int MODE, int NRT, int U>
__global__ __launch_bounds__(64 * kGemmWaves, NRT >= 4 ? 2 : 4) void k_gemm(const typename Op<MODE>::TA* __restrict__ A, int lda,
                                                          const int32_t* __restrict__ row_map, int M,
                                                          const int32_t* __restrict__ M_dev,
                                                          const typename Op<MODE>::TW* __restrict__ W, int ldw,
                                                          int N, int K, float* __restrict__ C, int ldc,
                                                          int accumulate, float* __restrict__ ss_part) {
  typedef typename Op<MODE>::TA TA;
  typedef typename Op<MODE>::TW TW;
  __shared__ float red[(kGemmWaves - 1) * NRT * 4 * 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (M_dev) M = *M_dev;
  const int row0 = blockIdx.y * 16 * NRT;
  if (row0 >= M) return;
  const int col0 = blockIdx.x * 16;
  const int kper = K / kGemmWaves;
  const TA* ap[NRT];
  bool av[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const int r = row0 + rt * 16 + (lane & 15);
    av[rt] = r < M;
    const int src = av[rt] ? (row_map ? row_map[r] : r) : 0;
    ap[rt] = A + (size_t)src * lda + 8 * (lane >> 4);
  }
  const int col = col0 + (lane & 15);
  // ragged last tile: lanes past N re-read row N-1 and never store
  const TW* wp[1] = {W + (size_t)min(col, N - 1) * ldw + 8 * (lane >> 4)};
  constexpr bool kLines = MODE == MODE_BF16 && U % 2 == 0;
  // wave 0 fetches the C tile it accumulates into before the K loop
  float cin[NRT][4];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = row0 + rt * 16 + 4 * (lane >> 4) + v;
      cin[rt][v] = (accumulate && wave == 0 && row < M && col < N) ? C[(size_t)row * ldc + col] : 0.f;
    }
  f32x4 acc[1][NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) acc[0][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (kLines) {
    __shared__ __align__(16) uint8_t wlds[kGemmWaves * 16 * (64 * U + 16)];
    const TW* wlo[1] = {W + (size_t)min(col0 + (lane >> 3), N - 1) * ldw + 8 * (lane & 7)};
    const TW* whi[1] = {W + (size_t)min(col0 + 8 + (lane >> 3), N - 1) * ldw + 8 * (lane & 7)};
    for (int k = wave * kper; k < (wave + 1) * kper; k += 32 * U)
      mma_batch_lines<NRT, 1, U>(acc, ap, av, wlo, whi, k, wlds + wave * 16 * (64 * U + 16));
  } else {
    for (int k = wave * kper; k < (wave + 1) * kper; k += 32 * U) mma_batch<MODE, NRT, 1, U>(acc, ap, av, wp, k);
  }
  reduce_waves<NRT, kGemmWaves>(acc[0], red);
  if (wave != 0) return;
  float out[NRT][4];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int v = 0; v < 4; ++v) out[rt][v] = cin[rt][v] + acc[0][rt][v];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = row0 + rt * 16 + 4 * (lane >> 4) + v;
      if (row < M && col < N) C[(size_t)row * ldc + col] = out[rt][v];
    }
  if (!ss_part) return;
  // per row: sum of squares of the tile's 16 columns (lanes 16 g .. 16 g + 15),
  // the 4 NRT shuffle chains interleaved
  float q[NRT][4];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int v = 0; v < 4; ++v) q[rt][v] = out[rt][v] * out[rt][v];
#pragma unroll
  for (int o = 1; o < 16; o <<= 1)
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int v = 0; v < 4; ++v) q[rt][v] += __shfl_xor(q[rt][v], o, 64);
  if ((lane & 15) == 0)
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = row0 + rt * 16 + 4 * (lane >> 4) + v;
        if (row < M) ss_part[(size_t)row * gridDim.x + blockIdx.x] = q[rt][v];
      }
}

template <int MODE, int NRT, int U>
static void gemm_launch_one(dim3 grid, const void* A, int lda, const int32_t* row_map, int M, const int32_t* M_dev,
                            const void* W, int ldw, int N, int K, float* C, int ldc, int acc, float* ss_part,
                            hipStream_t s) {
  typedef typename Op<MODE>::TA TA;
  typedef typename Op<MODE>::TW TW;
  hipLaunchKernelGGL((k_gemm<MODE, NRT, U>), grid, dim3(64 * kGemmWaves), 0, s, (const TA*)A, lda, row_map, M,
                     M_dev, (const TW*)W, ldw, N, K, C, ldc, acc, ss_part);
}

template <int MODE, int NRT>
static void gemm_launch_u(dim3 grid, const void* A, int lda, const int32_t* row_map, int M, const int32_t* M_dev,
                          const void* W, int ldw, int N, int K, float* C, int ldc, int acc, float* ss_part,
                          hipStream_t s) {
  // bf16 (whole-line loads through LDS): batches of 2 chunks (measured best of
  // 2, 4 and 8 at the layer step); f32: one batch per wavefront for up to 2
  // row tiles (W + A fragments ~110 VGPRs)
  constexpr int UMAX = MODE == MODE_BF16 ? (NRT <= 2 ? 2 : UCap<MODE>::v / NRT)
                                         : (NRT <= 2 ? UCap<MODE>::v : UCap<MODE>::v / NRT);
  const int chunks = K / (32 * kGemmWaves);   // 32-wide chunks per wavefront
  pick_u<UMAX>(chunks, [&](auto u) {
    gemm_launch_one<MODE, NRT, decltype(u)::value>(grid, A, lda, row_map, M, M_dev, W, ldw, N, K, C, ldc, acc,
                                                   ss_part, s);
  });
}

// 16-row tiles per workgroup for a GEMM over M rows and `col_tiles` column
// tiles: one tile when the column tiles alone give fewer workgroups than CUs
// (twice the workgroups, each reading half the activations), else 2 (M <= 32)
// or 4.
static int rows_tiles(int M, int col_tiles) {
  if (M <= 16) return 1;
  if (M <= 32) return col_tiles < 256 ? 1 : 2;
  return 4;
}

template <int MODE>
static hipError_t gemm_dispatch(const void* A, int lda, const int32_t* row_map, int M, const int32_t* M_dev,
                                const void* W, int ldw, int N, int K, float* C, int ldc, int acc, float* ss_part,
                                hipStream_t s) {
  const int nrt = rows_tiles(M, (N + 15) / 16);
  dim3 grid((N + 15) / 16, (M + 16 * nrt - 1) / (16 * nrt));
  if (nrt == 1) gemm_launch_u<MODE, 1>(grid, A, lda, row_map, M, M_dev, W, ldw, N, K, C, ldc, acc, ss_part, s);
  else if (nrt == 2) gemm_launch_u<MODE, 2>(grid, A, lda, row_map, M, M_dev, W, ldw, N, K, C, ldc, acc, ss_part, s);
  else gemm_launch_u<MODE, 4>(grid, A, lda, row_map, M, M_dev, W, ldw, N, K, C, ldc, acc, ss_part, s);
  return hipGetLastError();
}

hipError_t launch_gemm(int mode, const void* A, int lda, const int32_t* row_map, int M,
                       const int32_t* M_dev, const void* W, int ldw, int N, int K, float* C,
                       int ldc, int accumulate, hipStream_t s, float* ss_part) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (mode == MODE_F32)
    return gemm_dispatch<MODE_F32>(A, lda, row_map, M, M_dev, W, ldw, N, K, C, ldc, accumulate, ss_part, s);
  return gemm_dispatch<MODE_BF16>(A, lda, row_map, M, M_dev, W, ldw, N, K, C, ldc, accumulate, ss_part, s);
}

// ---------------------------------------------------------------------------
// LDS-tiled bf16 GEMM for long passes (prefill, the batched projections and the
// batched LM head), C = A W^T with A [M][K] and W [N][K], both K-contiguous.
// One BM x BN output tile per workgroup of 4 wavefronts (BM/2 x BN/2 each);
// K in stages of 64.  Each global load instruction of a wavefront reads 8
// whole 128-byte row segments (8 lanes x 16 bytes per row): the number of
// cache lines a load touches, not its bytes, limits how fast a CU pulls data,
// and the MFMA fragment order (16 rows x 64 bytes per instruction) touched
// twice as many.  Two register sets keep the loads of stages ks + 1 and
// ks + 2 in flight while stage ks is read from LDS, so a load has two stages
// of MFMA work to arrive in (one stage hid too little of the latency: the
// loop waited on memory at every barrier).  A register set is written to
// the LDS slot of its stage (two slots) right before the barrier that
// publishes it.  A slot holds the stage as rows of 64 bf16 at a pitch of 144
// bytes (A rows, then W rows), so that the fragment reads (lane l: row l %
// 16, 16 bytes at k chunk 4c + l / 16) fall on distinct banks.  After the K
// loop the fp32 tile is written to LDS and the epilogue walks it with all 256
// threads.
// ---------------------------------------------------------------------------

constexpr int kTM = 128, kTN = 128, kTK = 64;      // kTM: largest row tile; kTN: column tile of the fused epilogues
__host__ __device__ constexpr int tile_pitch(int kt) { return kt * 2 + 16; }   // LDS row pitch of a stage (bytes)
constexpr int kTileLd = kTN + 4;                   // fp32 row pitch of a kTN-column output tile in LDS
// LDS of a BM x BN tile: two stage slots, or the output tile that aliases them
__host__ __device__ constexpr int tile_lds_bytes(int bm, int bn = kTN, int kt = kTK, int kg = 1) {
  return kg * 2 * (bm + bn) * tile_pitch(kt) > bm * (bn + 4) * 4 ? kg * 2 * (bm + bn) * tile_pitch(kt)
                                                                  : bm * (bn + 4) * 4;
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Pipeline depth of the projections: two register sets of loads in flight for
// the 32- and 64-row tiles; one for 128-row tiles, where a second set costs a
// workgroup per CU (probe at 1024 x 6144 x 2048: 59.0 -> 42.2 us with one).
template <int BM> constexpr int kTileDepth = BM >= 128 ? 1 : 2;

// Accumulates a BM x BN tile and leaves it in LDS as float [BM][BN + 4]
// (rows m0.., columns n0..); ends with a barrier.  NW wavefronts in an NW/2 x
// 2 grid: wavefront (wm, wn) owns rows BM/(NW/2) wm .. and columns BN/2 wn ...
// Tile row r reads A row row_map[m0 + r] when row_map is given, else m0 + r;
// rows past M repeat the last row (their outputs are unused), as do W rows
// past N.
//
// KG > 1: KG groups of NW wavefronts split the reduction into KG equal
// parts, each with its own stage slots (the K loop is KG times shorter, so
// KG times fewer dependent load round trips per group); the parts are summed
// in LDS in a fixed order (last group first).  Needs K a multiple of KG KT.
template <int BM, int BN = kTN, int DEPTH = 2, int NW = 4, int KT = kTK, bool PAIR = false, int KG = 1>
__device__ void gemm_tile_bf16(const uint16_t* __restrict__ A, int lda, int M, const uint16_t* __restrict__ W,
                               int ldw, int N, int K, int m0, int n0, uint8_t* lds,
                               const int32_t* __restrict__ row_map = nullptr) {
  constexpr int WR = BM / (NW / 2);                // rows per wavefront
  constexpr int RT = WR / 16, CT = BN / 32;        // row / column fragments per wavefront
  constexpr int SEG = KT / 8;                      // 16-byte segments of a staged row
  constexpr int RPL = 64 / SEG * NW;               // tile rows one load instruction of the group covers
  constexpr int AL = BM / RPL, L = AL + BN / RPL;  // load instructions per thread per stage
  static_assert(BM % RPL == 0 && BN % RPL == 0 && WR % 16 == 0 && KT % 64 == 0, "tile shape");
  static_assert(KG == 1 || KG == 2 || KG == 4, "reduction groups");
  constexpr int PITCH = tile_pitch(KT);
  constexpr int SLOT = (BM + BN) * PITCH;
  const int lane = threadIdx.x & 63, kg = (threadIdx.x >> 6) / NW, wave = (threadIdx.x >> 6) % NW;
  const int kofs = kg * (K / KG);                  // first reduction element of this group
  K /= KG;
  lds += kg * 2 * SLOT;
  const int wm = wave >> 1, wn = wave & 1;
  const int q = lane % SEG, rr = lane / SEG;       // 16-byte chunk and row of this lane in a load
  const uint16_t* src[L];
  int dst[L];
#pragma unroll
  for (int i = 0; i < AL; ++i) {
    const int r = (wave + NW * i) * (64 / SEG) + rr;
    int row = m0 + r;
    row = row < M ? row : M - 1;
    src[i] = A + (size_t)(row_map ? row_map[row] : row) * lda + kofs + q * 8;
    dst[i] = r * PITCH + q * 16;
  }
#pragma unroll
  for (int i = 0; i < BN / RPL; ++i) {
    const int r = (wave + NW * i) * (64 / SEG) + rr;
    // PAIR (64-column tiles): tile columns 0..31 and 32..63 are W rows n0 ..
    // n0 + 31 and n0 + 64 .. n0 + 95, the two halves of 32 rotation pairs
    int row = PAIR ? n0 + (r & 31) + ((r >> 5) << 6) : n0 + r;
    row = row < N ? row : N - 1;
    src[AL + i] = W + (size_t)row * ldw + kofs + q * 8;
    dst[AL + i] = (BM + r) * PITCH + q * 16;
  }
  f32x4 acc[RT][CT];
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int j = 0; j < CT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int fr = lane & 15, fq = lane >> 4;         // fragment row and k chunk of this lane
  const int nk = K / KT;
  auto load = [&](u32x4(&st)[L], int ks) {
#pragma unroll
    for (int i = 0; i < L; ++i) st[i] = *(const u32x4*)(src[i] + ks * KT);
    // keep the loads here, ahead of the MFMAs they are meant to overlap
    __builtin_amdgcn_sched_barrier(0);
  };
  auto store = [&](const u32x4(&st)[L], int slot) {
    uint8_t* sl = lds + slot * SLOT;
#pragma unroll
    for (int i = 0; i < L; ++i) *(u32x4*)(sl + dst[i]) = st[i];
  };
  auto compute = [&](int slot) {
    const uint8_t* sa = lds + slot * SLOT;
    const uint8_t* sw = sa + BM * PITCH;
#pragma unroll
    for (int c = 0; c < KT / 32; ++c) {
      u32x4 af[RT], wf[CT];
#pragma unroll
      for (int i = 0; i < RT; ++i) af[i] = *(const u32x4*)(sa + ((wm * RT + i) * 16 + fr) * PITCH + (4 * c + fq) * 16);
#pragma unroll
      for (int j = 0; j < CT; ++j) wf[j] = *(const u32x4*)(sw + ((wn * CT + j) * 16 + fr) * PITCH + (4 * c + fq) * 16);
#pragma unroll
      for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int j = 0; j < CT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af[i]),
                                                              __builtin_bit_cast(bf16x8, wf[j]), acc[i][j], 0, 0, 0);
    }
  };
  u32x4 s0[L], s1[L];
  if constexpr (DEPTH == 1) {
    // one register set: the loads of stage ks + 1 overlap the products of ks
    load(s0, 0);
    store(s0, 0);
    __syncthreads();
    for (int ks = 0; ks < nk; ++ks) {
      if (ks + 1 < nk) load(s0, ks + 1);
      compute(ks & 1);
      if (ks + 1 < nk) store(s0, (ks + 1) & 1);
      __syncthreads();   // stage ks + 1 is in LDS; stage ks is no longer read
    }
  } else {
  // even stages live in slot 0 and register set s0, odd ones in slot 1 and s1
  load(s0, 0);
  if (nk > 1) load(s1, 1);
  store(s0, 0);
  __syncthreads();
  if (nk > 2) load(s0, 2);
  for (int ks = 0; ks < nk; ks += 2) {
    // slot 0: stage ks; s1: stage ks + 1; s0: stage ks + 2 in flight
    compute(0);
    if (ks + 1 < nk) store(s1, 1);
    __syncthreads();   // stage ks + 1 is in slot 1; slot 0 is no longer read
    if (ks + 1 >= nk) break;
    if (ks + 3 < nk) load(s1, ks + 3);
    compute(1);
    if (ks + 2 < nk) store(s0, 0);
    __syncthreads();   // stage ks + 2 is in slot 0; slot 1 is no longer read
    if (ks + 4 < nk) load(s0, ks + 4);
  }
  }
  // the slots are dead: the output tile aliases them
  // accumulator (i, j)[v]: row WR wm + 16 i + 4 (lane / 16) + v, column BN/2 wn + 16 j + lane % 16
  float* t = (float*)(lds - kg * 2 * SLOT);
  auto put = [&](bool add) {
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int j = 0; j < CT; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float& d = t[(wm * WR + i * 16 + 4 * (lane >> 4) + v) * (BN + 4) + wn * (BN / 2) + j * 16 + (lane & 15)];
          d = add ? d + acc[i][j][v] : acc[i][j][v];
        }
  };
  if (kg == KG - 1) put(false);
#pragma unroll
  for (int g = KG - 2; g >= 0; --g) {
    __syncthreads();
    if (kg == g) put(true);
  }
  __syncthreads();
}

// C (float, [M][ldc]) += tile, with per-row sums of squares of the new values
// per 16-column group in ss_part[row][N / 16] (as the streaming GEMM writes).
template <int BM, int BN, int KT, int KG = 1>
__global__ __launch_bounds__(256 * KG) void k_gemm_tiled_acc(const uint16_t* __restrict__ A, int lda, int M,
                                                             const uint16_t* __restrict__ W, int ldw, int N, int K,
                                                             float* __restrict__ C, int ldc, float* __restrict__ ss_part) {
  extern __shared__ __align__(16) uint8_t tile_lds[];
  constexpr int G = BN / 16, LD = BN + 4;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  gemm_tile_bf16<BM, BN, kTileDepth<BM>, 4, KT, false, KG>(A, lda, M, W, ldw, N, K, m0, n0, tile_lds);
  const float* t = (const float*)tile_lds;
  // thread: one row, one 16-column group per pass
  for (int p = threadIdx.x; p < BM * G; p += 256 * KG) {
    const int r = p / G, g = p % G;
    const int row = m0 + r, c0 = n0 + 16 * g;
    if (row >= M || c0 >= N) continue;
    float* cr = C + (size_t)row * ldc + c0;
    float q = 0.f;
#pragma unroll
    for (int c = 0; c < 16; c += 4) {
      float4 v = *(const float4*)(cr + c);
      v.x += t[r * LD + 16 * g + c];
      v.y += t[r * LD + 16 * g + c + 1];
      v.z += t[r * LD + 16 * g + c + 2];
      v.w += t[r * LD + 16 * g + c + 3];
      *(float4*)(cr + c) = v;
      q += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
    if (ss_part) ss_part[(size_t)row * (N / 16) + (c0 >> 4)] = q;
  }
}

// QKV projection of a long pass with RoPE and the K/V cache scatter.  BN =
// 128: the column tile lies inside the q, k or v part (HD multiple of 128)
// and covers whole heads, so each rotation pair (j, j + dh/2) is in the tile.
// BN = 64 (d_h = 128 only): the tile holds columns j0 .. j0 + 31 and j0 + 64
// .. j0 + 95 of one head (j0 = 0 or 32), the two halves of 32 rotation pairs.
template <int BM, int BN>
__global__ __launch_bounds__(256) void k_qkv_rope_tiled(const uint16_t* __restrict__ X, const uint16_t* __restrict__ W,
                                                        int M, int D, int H, int dh, int n_tok, int pos0, double base,
                                                        uint16_t* __restrict__ q, uint16_t* __restrict__ kdst,
                                                        uint16_t* __restrict__ vdst, long long k_row_stride,
                                                        long long k_head_stride, int k_pos0) {
  extern __shared__ __align__(16) uint8_t tile_lds[];
  constexpr bool PAIR = BN == 64;
  constexpr int NP = BN / 2, LD = BN + 4;          // rotation pairs per tile row; LDS row pitch (floats)
  const int HD = H * dh;
  const int m0 = blockIdx.y * BM;
  // first W row of the tile: a head block of 128 columns, then j0 within it
  const int n0 = PAIR ? (blockIdx.x >> 1) * 128 + (blockIdx.x & 1) * 32 : blockIdx.x * BN;
  gemm_tile_bf16<BM, BN, kTileDepth<BM>, 4, kTK, PAIR>(X, D, M, W, D, 3 * HD, D, m0, n0, tile_lds);
  const float* t = (const float*)tile_lds;
  const int part = n0 / HD;                       // 0 q, 1 k, 2 v
  const int half = dh >> 1;
  const double two_pi = 6.283185307179586476925286766559;
  const double inv_two_pi = 0.15915494309189533576888376337251;
  // thread: one rotation pair (fixed column) of rows threadIdx.x / NP, + 256 /
  // NP, ..., so theta is computed once per thread
  const int pc = threadIdx.x % NP;
  const int cl = PAIR ? pc : (pc / half) * dh + (pc % half);   // tile column of the pair's first element
  const int cl2 = PAIR ? pc + 32 : cl + half;                   // and of its second
  const int col = PAIR ? n0 + pc : n0 + cl;                     // W row (output column) of the first
  const int hh = (col % HD) / dh, j = col % dh;
  const double theta = part < 2 ? pow(base, -2.0 * (double)j / (double)dh) : 0.0;
  for (int r = threadIdx.x / NP; r < BM; r += 256 / NP) {
    const int i = m0 + r;
    if (i >= M) break;
    float x1 = t[r * LD + cl], x2 = t[r * LD + cl2];
    const int rr = i / n_tok, jt = i % n_tok;
    if (part < 2) {
      double ang = (double)(pos0 + jt) * theta;
      ang -= two_pi * rint(ang * inv_two_pi);
      float sn, cs;
      sincosf((float)ang, &sn, &cs);
      const float y1 = x1 * cs - x2 * sn, y2 = x2 * cs + x1 * sn;
      x1 = y1;
      x2 = y2;
    }
    uint16_t* dst;
    if (part == 0) dst = q + ((size_t)(rr * H + hh) * n_tok + jt) * dh;
    else dst = (part == 1 ? kdst : vdst) + (size_t)(rr * k_row_stride + hh * k_head_stride) + (size_t)(k_pos0 + jt) * dh;
    dst[j] = f2bf(x1);
    dst[j + half] = f2bf(x2);
  }
}

bool gemm_tiled_ok(int mode, int M, int N, int K) {
  return mode == MODE_BF16 && M >= kTM && N % 64 == 0 && K % kTK == 0;
}

#ifndef DLLM_GEMM_MIN_WG
#define DLLM_GEMM_MIN_WG 256
#endif
#ifndef DLLM_OPROJ_KG
#define DLLM_OPROJ_KG 2
#endif

hipError_t launch_gemm_tiled_acc(const void* A, int lda, int M, const void* W, int ldw, int N, int K, float* C,
                                 int ldc, float* ss_part, hipStream_t s) {
  // the largest tile that still gives every CU a workgroup: fewer, larger
  // tiles re-read less of A and W from L2
  auto go = [&](auto bm_c, auto bn_c, auto kt_c, auto kg_c) {
    constexpr int BM = decltype(bm_c)::value, BN = decltype(bn_c)::value, KT = decltype(kt_c)::value;
    constexpr int KG = decltype(kg_c)::value;
    dim3 grid(N / BN, (M + BM - 1) / BM);
    hipLaunchKernelGGL((k_gemm_tiled_acc<BM, BN, KT, KG>), grid, dim3(256 * KG), tile_lds_bytes(BM, BN, KT, KG), s,
                       (const uint16_t*)A, lda, M, (const uint16_t*)W, ldw, N, K, C, ldc, ss_part);
  };
  auto tiles = [&](int bm, int bn) { return (N % bn ? 0 : N / bn) * ((M + bm - 1) / bm); };
  if (tiles(128, 128) >= DLLM_GEMM_MIN_WG) go(IC<128>{}, IC<128>{}, IC<64>{}, IC<1>{});
  else if (tiles(64, 128) >= DLLM_GEMM_MIN_WG) go(IC<64>{}, IC<128>{}, IC<64>{}, IC<1>{});
  else if (tiles(64, 64) >= DLLM_GEMM_MIN_WG) {
    // 128-deep stages halve the barriers of the small tile (probe at 512 x
    // 2048 x 2048: 17.4 -> 13.3 us)
    // Two wavefront groups split the reduction (8 stages each instead of
    // 16; one workgroup per CU): the batched step's 512 x 2048 x 2048
    // projection measured 0.5-1.3 % faster per 20-layer step; four groups of
    // 64-deep stages measured between the two.
    if (DLLM_OPROJ_KG == 2 && K % 256 == 0) go(IC<64>{}, IC<64>{}, IC<128>{}, IC<2>{});
    else if (K % 128 == 0) go(IC<64>{}, IC<64>{}, IC<128>{}, IC<1>{});
    else go(IC<64>{}, IC<64>{}, IC<64>{}, IC<1>{});
  } else go(IC<32>{}, IC<64>{}, IC<64>{}, IC<1>{});
  return hipGetLastError();
}

bool qkv_tiled_ok(int mode, int M, int D, int H, int dh) {
  return mode == MODE_BF16 && M >= kTM && (H * dh) % kTN == 0 && kTN % dh == 0 && D % kTK == 0;
}

hipError_t launch_qkv_rope_tiled(const void* X, const void* W, int rows, int n_tok, int D, int H, int dh, int pos0,
                                 float base, void* q, void* kdst, void* vdst, long long k_row_stride,
                                 long long k_head_stride, int k_pos0, hipStream_t s) {
  const int M = rows * n_tok;
  // the tallest row tile that still gives every CU a workgroup
  const int ncol = 3 * H * dh / kTN;
  auto go = [&](auto bm_c, auto bn_c) {
    constexpr int BM = decltype(bm_c)::value, BN = decltype(bn_c)::value;
    dim3 grid(3 * H * dh / BN, (M + BM - 1) / BM);
    hipLaunchKernelGGL((k_qkv_rope_tiled<BM, BN>), grid, dim3(256), tile_lds_bytes(BM, BN), s, (const uint16_t*)X,
                       (const uint16_t*)W, M, D, H, dh, n_tok, pos0, (double)base, (uint16_t*)q, (uint16_t*)kdst,
                       (uint16_t*)vdst, k_row_stride, k_head_stride, k_pos0);
  };
  if (ncol * ((M + 127) / 128) >= DLLM_GEMM_MIN_WG) go(IC<128>{}, IC<128>{});
  else if (dh == 128) go(IC<64>{}, IC<64>{});   // paired 64-column tiles
  else if (ncol * ((M + 63) / 64) >= DLLM_GEMM_MIN_WG) go(IC<64>{}, IC<128>{});
  else go(IC<32>{}, IC<128>{});
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Router logits with the pre-MoE RMSNorm folded in: C[M, E] = x W^T with
// x = h / sqrt(mean(h^2) + eps) * gain formed while the A fragments load.
// The K range is split over gridDim.z workgroups (more CUs pull h and W);
// slice z writes partial logits C[z][row][col] (slice-major: a wavefront's
// stores cover whole 64-byte runs), summed by the selection kernel.
// mean(h^2) comes from ss_part[row][0 .. n_part) (per-column-tile sums of
// squares written by the producer of h), summed in a fixed order.  The
// normalized activations are also stored (for the expert GEMMs) straight from
// the A fragments: 32-column chunk c by workgroup column c mod gridDim.x, for
// the rows of its row tiles, so every element is written once.
// ---------------------------------------------------------------------------

template <int MODE> struct NormA;
template <> struct NormA<MODE_BF16> {
  __device__ static void store(uint16_t* p, const uint4& v) { *(uint4*)p = v; }
  __device__ static uint4 make(const float* hp, const float* gp, float inv) {
    const float4 h0 = ((const float4*)hp)[0], h1 = ((const float4*)hp)[1];
    const float4 g0 = ((const float4*)gp)[0], g1 = ((const float4*)gp)[1];
    uint4 r;
    r.x = (uint32_t)f2bf(h0.x * inv * g0.x) | ((uint32_t)f2bf(h0.y * inv * g0.y) << 16);
    r.y = (uint32_t)f2bf(h0.z * inv * g0.z) | ((uint32_t)f2bf(h0.w * inv * g0.w) << 16);
    r.z = (uint32_t)f2bf(h1.x * inv * g1.x) | ((uint32_t)f2bf(h1.y * inv * g1.y) << 16);
    r.w = (uint32_t)f2bf(h1.z * inv * g1.z) | ((uint32_t)f2bf(h1.w * inv * g1.w) << 16);
    return r;
  }
};
template <> struct NormA<MODE_F32> {
  __device__ static void store(float* p, const F8x& v) {
    ((float4*)p)[0] = v.a;
    ((float4*)p)[1] = v.b;
  }
  __device__ static F8x make(const float* hp, const float* gp, float inv) {
    const float4 h0 = ((const float4*)hp)[0], h1 = ((const float4*)hp)[1];
    const float4 g0 = ((const float4*)gp)[0], g1 = ((const float4*)gp)[1];
    return F8x{make_float4(h0.x * inv * g0.x, h0.y * inv * g0.y, h0.z * inv * g0.z, h0.w * inv * g0.w),
               make_float4(h1.x * inv * g1.x, h1.y * inv * g1.y, h1.z * inv * g1.z, h1.w * inv * g1.w)};
  }
};

template <int MODE, int NRT, int U, int CT>
__global__ __launch_bounds__(64 * kGemmWaves, NRT >= 4 ? 2 : 4) void k_router_norm(
    const float* __restrict__ h, const float* __restrict__ gain, const float* __restrict__ ss_part, int n_part,
    float eps, int M, const typename Op<MODE>::TW* __restrict__ W, int N, int K, float* __restrict__ C,
    typename Op<MODE>::TA* __restrict__ x) {
  typedef typename Op<MODE>::TW TW;
  typedef typename Op<MODE>::AF AF;
  __shared__ float red[(kGemmWaves - 1) * NRT * 4 * 64];
  __shared__ float inv_s[16 * NRT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row0 = blockIdx.y * 16 * NRT;
  const int col0 = blockIdx.x * 16 * CT;   // CT 16-column tiles share the normalized A fragments
  const int kper = K / gridDim.z / kGemmWaves;   // K split over gridDim.z workgroups, then 8 waves
  // the first weight batch does not depend on the normalization: request it first
  const TW* wp[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) wp[ct] = W + (size_t)min(col0 + 16 * ct + (lane & 15), N - 1) * K + 8 * (lane >> 4);
  int k = (blockIdx.z * kGemmWaves + wave) * kper;
  const int kend = k + kper;
  typename Op<MODE>::WF wf[CT][U];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int u = 0; u < U; ++u) wf[ct][u] = Op<MODE>::ldw(wp[ct] + k + 32 * u);
  // 1 / rms of the tile's rows: 16 threads per row, partials summed in a fixed order
  for (int r = tid >> 4; r < 16 * NRT; r += (64 * kGemmWaves) >> 4) {
    const int row = row0 + r;
    float q = 0.f;
    if (row < M) {
      const float* sp = ss_part + (size_t)row * n_part;
      int p = tid & 15;
      for (; p + 7 * 16 < n_part; p += 8 * 16) {   // 8 loads in flight
        float t[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) t[j] = sp[p + 16 * j];
#pragma unroll
        for (int j = 0; j < 8; ++j) q += t[j];
      }
      for (; p < n_part; p += 16) q += sp[p];
    }
    q += __shfl_xor(q, 1, 64);
    q += __shfl_xor(q, 2, 64);
    q += __shfl_xor(q, 4, 64);
    q += __shfl_xor(q, 8, 64);
    if ((tid & 15) == 0) inv_s[r] = 1.0f / sqrtf(q / (float)K + eps);
  }
  __syncthreads();
  const float* hp[NRT];
  float inv[NRT];
  bool av[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const int r = rt * 16 + (lane & 15);
    av[rt] = row0 + r < M;
    inv[rt] = inv_s[r];
    hp[rt] = h + (size_t)(av[rt] ? row0 + r : 0) * K + 8 * (lane >> 4);
  }
  f32x4 acc[CT][NRT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) acc[ct][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (;;) {
    AF af[NRT][U];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int kk = k + 32 * u + 8 * (lane >> 4);
        af[rt][u] = av[rt] ? NormA<MODE>::make(hp[rt] + k + 32 * u, gain + kk, inv[rt]) : Op<MODE>::za();
      }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (((k >> 5) + u) % gridDim.x == blockIdx.x)   // this workgroup's chunks of x
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
          if (av[rt]) NormA<MODE>::store(x + (size_t)(row0 + rt * 16 + (lane & 15)) * K + k + 32 * u + 8 * (lane >> 4),
                                         af[rt][u]);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) Op<MODE>::mma(acc[ct][rt], af[rt][u], wf[ct][u]);
    k += 32 * U;
    if (k >= kend) break;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int u = 0; u < U; ++u) wf[ct][u] = Op<MODE>::ldw(wp[ct] + k + 32 * u);
  }
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) reduce_waves<NRT, kGemmWaves>(acc[ct], red);
  if (wave != 0) return;
  // this K slice's partial logits: C[z][row][col]
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int col = col0 + 16 * ct + (lane & 15);
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = row0 + rt * 16 + 4 * (lane >> 4) + v;
        if (row < M && col < N) C[((size_t)blockIdx.z * M + row) * N + col] = acc[ct][rt][v];
      }
  }
}

// Router logits of a 64-row x 64-column tile over one K slice (bf16, 256+
// experts): the slice's rows are normalised once into LDS (bf16) by all 512
// threads, then wavefront (c, g) = (wave % 4, wave / 4) multiplies 16
// columns by the slice's g-th half, and the two halves are summed in LDS
// (second half first, then the first added to it) before the partial logits
// are stored.  The normalised activations x are written as in k_router_norm
// (32-column chunk c by workgroup column c mod gridDim.x).
constexpr int kRtRows = 64, kRtCols = 64;
template <int KS>
__global__ __launch_bounds__(512) void k_router_norm_lds(const float* __restrict__ h, const float* __restrict__ gain,
                                                         const float* __restrict__ ss_part, int n_part, float eps,
                                                         int M, const uint16_t* __restrict__ W, int N, int K,
                                                         float* __restrict__ C, uint16_t* __restrict__ x) {
  constexpr int PITCH = KS + 8;                     // bf16 elements per staged row
  constexpr int KH = KS / 2, NCH = KH / 32;         // reduction elements / 32-wide chunks per half
  __shared__ __align__(16) uint16_t xa[kRtRows * PITCH];
  __shared__ float inv_s[kRtRows];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = wave & 3, g = wave >> 2;
  const int row0 = blockIdx.y * kRtRows, col0 = blockIdx.x * kRtCols;
  const int kz = blockIdx.z * KS;                  // this workgroup's K slice
  // weight fragments of the wavefront's 16 columns and K half: requested first
  uint4 wf[NCH];
  {
    const int col = min(col0 + 16 * c + (lane & 15), N - 1);
    const uint16_t* wp = W + (size_t)col * K + kz + g * KH + 8 * (lane >> 4);
#pragma unroll
    for (int j = 0; j < NCH; ++j) wf[j] = *(const uint4*)(wp + 32 * j);
  }
  // 1 / rms of the tile's rows: 16 threads per row, partials summed in a fixed order
  for (int r = tid >> 4; r < kRtRows; r += 512 >> 4) {
    const int row = row0 + r;
    float q = 0.f;
    if (row < M) {
      const float* sp = ss_part + (size_t)row * n_part;
      int p = tid & 15;
      for (; p + 7 * 16 < n_part; p += 8 * 16) {
        float t[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) t[j] = sp[p + 16 * j];
#pragma unroll
        for (int j = 0; j < 8; ++j) q += t[j];
      }
      for (; p < n_part; p += 16) q += sp[p];
    }
    q += __shfl_xor(q, 1, 64);
    q += __shfl_xor(q, 2, 64);
    q += __shfl_xor(q, 4, 64);
    q += __shfl_xor(q, 8, 64);
    if ((tid & 15) == 0) inv_s[r] = 1.0f / sqrtf(q / (float)K + eps);
  }
  __syncthreads();
  // normalised rows of the slice -> LDS (rows past M are zero) and x
  for (int u = tid; u < kRtRows * (KS / 8); u += 512) {
    const int r = u / (KS / 8), k8 = (u % (KS / 8)) * 8;
    const int row = row0 + r, kk = kz + k8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row < M) {
      v = NormA<MODE_BF16>::make(h + (size_t)row * K + kk, gain + kk, inv_s[r]);
      if ((kk >> 5) % gridDim.x == blockIdx.x) *(uint4*)(x + (size_t)row * K + kk) = v;
    }
    *(uint4*)(xa + r * PITCH + k8) = v;
  }
  __syncthreads();
  f32x4 acc[kRtRows / 16];
#pragma unroll
  for (int rt = 0; rt < kRtRows / 16; ++rt) acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < NCH; ++j)
#pragma unroll
    for (int rt = 0; rt < kRtRows / 16; ++rt) {
      const uint4 a = *(const uint4*)(xa + (rt * 16 + (lane & 15)) * PITCH + g * KH + 32 * j + 8 * (lane >> 4));
      acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                        __builtin_bit_cast(bf16x8, wf[j]), acc[rt], 0, 0, 0);
    }
  __syncthreads();   // the staged rows are dead: the halves' exchange aliases them
  float* red = (float*)xa;                          // [4 column waves][kRtRows / 16][4][64]
  if (g == 1) {
#pragma unroll
    for (int rt = 0; rt < kRtRows / 16; ++rt)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[((c * (kRtRows / 16) + rt) * 4 + v) * 64 + lane] = acc[rt][v];
  }
  __syncthreads();
  if (g == 1) return;
  const int col = col0 + 16 * c + (lane & 15);
#pragma unroll
  for (int rt = 0; rt < kRtRows / 16; ++rt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = row0 + rt * 16 + 4 * (lane >> 4) + v;
      const float z = red[((c * (kRtRows / 16) + rt) * 4 + v) * 64 + lane] + acc[rt][v];
      if (row < M && col < N) C[((size_t)blockIdx.z * M + row) * N + col] = z;
    }
}

template <int MODE, int NRT, int CT = 1>
static void router_norm_launch(dim3 grid, const float* h, const float* gain, const float* ss_part, int n_part,
                               float eps, int M, const void* W, int N, int K, float* C, void* x, hipStream_t s) {
  typedef typename Op<MODE>::TA TA;
  typedef typename Op<MODE>::TW TW;
  // A fragments are formed from float32 h and gains: half the plain GEMM's batch
  constexpr int UC = (NRT <= 2 ? UCap<MODE>::v : UCap<MODE>::v / NRT) / 2;
  constexpr int UMAX = UC > 1 ? UC : 1;
  const int chunks = K / grid.z / (32 * kGemmWaves);
  pick_u<UMAX>(chunks, [&](auto u) {
    hipLaunchKernelGGL((k_router_norm<MODE, NRT, decltype(u)::value, CT>), grid, dim3(64 * kGemmWaves), 0, s, h, gain,
                       ss_part, n_part, eps, M, (const TW*)W, N, K, C, (TA*)x);
  });
}

#ifndef DLLM_ROUTER_LDS
#define DLLM_ROUTER_LDS 1
#endif

int router_k_split(int K) { return K / 256 < kRouterSplit ? K / 256 : kRouterSplit; }

hipError_t launch_router_norm(int mode, const float* h, const float* gain, const float* ss_part, int n_part,
                              float eps, int M, const void* W, int N, int K, float* C, void* x, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  const int nrt = M <= 32 ? 1 : 4;   // 16-row tiles up to 32 rows (twice the workgroups; measured faster)
  // 64-row tiles: 4 column tiles per workgroup share the normalized rows (a
  // quarter of the float32 h reads)
  const int ct = (nrt == 4 && N >= 256) ? 4 : 1;
  dim3 grid((N + 16 * ct - 1) / (16 * ct), (M + 16 * nrt - 1) / (16 * nrt), router_k_split(K));
#define DLLM_RN(MD, NR, CTV) router_norm_launch<MD, NR, CTV>(grid, h, gain, ss_part, n_part, eps, M, W, N, K, C, x, s)
  if (mode == MODE_F32) {
    if (nrt == 1) DLLM_RN(MODE_F32, 1, 1);
    else if (ct == 4) DLLM_RN(MODE_F32, 4, 4);
    else DLLM_RN(MODE_F32, 4, 1);
  } else {
    if (nrt == 1) DLLM_RN(MODE_BF16, 1, 1);
    else if (ct == 4 && DLLM_ROUTER_LDS && K / grid.z == 256 && N % kRtCols == 0)
      hipLaunchKernelGGL((k_router_norm_lds<256>), dim3(N / kRtCols, (M + kRtRows - 1) / kRtRows, grid.z), dim3(512),
                         0, s, h, gain, ss_part, n_part, eps, M, (const uint16_t*)W, N, K, C, (uint16_t*)x);
    else if (ct == 4) DLLM_RN(MODE_BF16, 4, 4);
    else DLLM_RN(MODE_BF16, 4, 1);
  }
#undef DLLM_RN
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Fused QKV projection + 1D RoPE + scatter.  A workgroup computes the column
// pair (c, c + dh/2) of one head for 16 * NRT token rows: the two 16-column
// tiles are exactly the rotate-half partners, so the epilogue rotates q and k
// in registers and writes q, k and v straight into the attention layouts
// (q: [rows][H][n_tok][dh]; k/v: cache positions or the block scratch).
// Angles: theta_i = base^(-2i/dh) and pos * theta in double precision,
// reduced by whole turns, then sincosf.
// ---------------------------------------------------------------------------

template <int MODE, int NRT, int U>
__global__ __launch_bounds__(64 * kGemmWaves, NRT >= 4 ? 2 : 4) void k_qkv_rope(
    const typename Op<MODE>::TA* __restrict__ X, const typename Op<MODE>::TW* __restrict__ W, int M, int D, int H,
    int dh, int n_tok, int pos0, double base, typename Op<MODE>::TA* __restrict__ q,
    typename Op<MODE>::TA* __restrict__ kdst, typename Op<MODE>::TA* __restrict__ vdst, long long k_row_stride,
    long long k_head_stride, int k_pos0) {
  typedef typename Op<MODE>::TA TA;
  typedef typename Op<MODE>::TW TW;
  __shared__ float red[(kGemmWaves - 1) * NRT * 4 * 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = dh >> 1;
  const int pairs_per_head = half / 16;
  const int tile = blockIdx.x;                 // 0 .. 3 * H * pairs_per_head - 1
  const int part = tile / (H * pairs_per_head);  // 0 q, 1 k, 2 v
  const int hh = (tile / pairs_per_head) % H;
  const int j0 = (tile % pairs_per_head) * 16;   // column within the head's first half
  const int row0 = blockIdx.y * 16 * NRT;
  const int HD = H * dh;
  const int col_a = part * HD + hh * dh + j0 + (lane & 15);
  const TW* wp[2] = {W + (size_t)col_a * D + 8 * (lane >> 4), W + (size_t)(col_a + half) * D + 8 * (lane >> 4)};
  const TA* ap[NRT];
  bool av[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const int r = row0 + rt * 16 + (lane & 15);
    av[rt] = r < M;
    ap[rt] = X + (size_t)(av[rt] ? r : 0) * D + 8 * (lane >> 4);
  }
  f32x4 acc[2][NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    acc[0][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc[1][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int kper = D / kGemmWaves;
  if constexpr (MODE == MODE_BF16 && U % 2 == 0) {
    __shared__ __align__(16) uint8_t wlds[kGemmWaves * 2 * 16 * (64 * U + 16)];
    const int rl = part * HD + hh * dh + j0 + (lane >> 3);   // whole-line rows of the first matrix
    const TW* wlo[2] = {W + (size_t)rl * D + 8 * (lane & 7), W + (size_t)(rl + half) * D + 8 * (lane & 7)};
    const TW* whi[2] = {W + (size_t)(rl + 8) * D + 8 * (lane & 7), W + (size_t)(rl + 8 + half) * D + 8 * (lane & 7)};
    for (int k = wave * kper; k < (wave + 1) * kper; k += 32 * U)
      mma_batch_lines<NRT, 2, U>(acc, ap, av, wlo, whi, k, wlds + wave * 2 * 16 * (64 * U + 16));
  } else {
    for (int k = wave * kper; k < (wave + 1) * kper; k += 32 * U) mma_batch<MODE, NRT, 2, U>(acc, ap, av, wp, k);
  }
  reduce_waves<NRT, kGemmWaves>(acc[0], red);
  reduce_waves<NRT, kGemmWaves>(acc[1], red);
  if (wave != 0) return;
  const int j = j0 + (lane & 15);
  const double theta = pow(base, -2.0 * (double)j / (double)dh);
  const double two_pi = 6.283185307179586476925286766559;
  const double inv_two_pi = 0.15915494309189533576888376337251;
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = row0 + rt * 16 + 4 * (lane >> 4) + v;
      if (i >= M) continue;
      const int r = i / n_tok, jt = i % n_tok;
      float x1 = acc[0][rt][v], x2 = acc[1][rt][v];
      if (part < 2) {
        double ang = (double)(pos0 + jt) * theta;
        ang -= two_pi * rint(ang * inv_two_pi);   // any whole turn removed leaves sin, cos unchanged
        float sn, cs;
        sincosf((float)ang, &sn, &cs);
        const float y1 = x1 * cs - x2 * sn, y2 = x2 * cs + x1 * sn;
        x1 = y1;
        x2 = y2;
      }
      TA* dst;
      if (part == 0) dst = q + ((size_t)(r * H + hh) * n_tok + jt) * dh;
      else dst = (part == 1 ? kdst : vdst) + (size_t)(r * k_row_stride + hh * k_head_stride) + (size_t)(k_pos0 + jt) * dh;
      st1<TA>(dst + j, x1);
      st1<TA>(dst + j + half, x2);
    }
}

template <int MODE, int NRT, int U>
static void qkv_launch_one(dim3 grid, const void* X, const void* W, int M, int D, int H, int dh, int n_tok, int pos0,
                           float base, void* q, void* kd, void* vd, long long krs, long long khs, int kp0,
                           hipStream_t s) {
  typedef typename Op<MODE>::TA TA;
  typedef typename Op<MODE>::TW TW;
  hipLaunchKernelGGL((k_qkv_rope<MODE, NRT, U>), grid, dim3(64 * kGemmWaves), 0, s, (const TA*)X, (const TW*)W, M, D,
                     H, dh, n_tok, pos0, (double)base, (TA*)q, (TA*)kd, (TA*)vd, krs, khs, kp0);
}

template <int MODE>
static void qkv_dispatch(const void* X, const void* W, int M, int D, int H, int dh, int n_tok, int pos0, float base,
                         void* q, void* kd, void* vd, long long krs, long long khs, int kp0, hipStream_t s) {
  // 16-row tiles up to 32 rows: twice the workgroups, the second read of each
  // weight tile from L2 (measured faster with whole-line loads)
  const int nrt = M <= 32 ? 1 : 4;
  dim3 grid(3 * H * (dh / 32), (M + 16 * nrt - 1) / (16 * nrt));
  const int chunks = D / (32 * kGemmWaves);
  auto go = [&](auto nrt_c) {
    constexpr int NRT = decltype(nrt_c)::value;
    // bf16: batches of 2 chunks on the whole-line path (measured best of 2 and 4)
    constexpr int UMAX = MODE == MODE_BF16 ? 2 : UCap<MODE>::v / (NRT >= 2 ? NRT : 2);
    pick_u<(UMAX > 0 ? UMAX : 1)>(chunks, [&](auto u) {
      qkv_launch_one<MODE, NRT, decltype(u)::value>(grid, X, W, M, D, H, dh, n_tok, pos0, base, q, kd, vd, krs, khs,
                                                     kp0, s);
    });
  };
  if (nrt == 1) go(IC<1>{});
  else if (nrt == 2) go(IC<2>{});
  else go(IC<4>{});
}

hipError_t launch_qkv_rope(int mode, const void* X, const void* W, int rows, int n_tok, int D, int H, int dh,
                           int pos0, float base, void* q, void* kdst, void* vdst, long long k_row_stride,
                           long long k_head_stride, int k_pos0, hipStream_t s) {
  const int M = rows * n_tok;
  if (M == 0) return hipSuccess;
  if (mode == MODE_F32)
    qkv_dispatch<MODE_F32>(X, W, M, D, H, dh, n_tok, pos0, base, q, kdst, vdst, k_row_stride, k_head_stride, k_pos0, s);
  else
    qkv_dispatch<MODE_BF16>(X, W, M, D, H, dh, n_tok, pos0, base, q, kdst, vdst, k_row_stride, k_head_stride, k_pos0,
                            s);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// embedding gather + RMSNorm, RMSNorm, combine + RMSNorm
// ---------------------------------------------------------------------------

template <typename T>
__device__ void norm_store(float* hrow, const float* gain, float eps, int D, T* xrow, float* tmp) {
  float ss = 0.f;
  for (int i = threadIdx.x; i < D; i += blockDim.x) ss += hrow[i] * hrow[i];
  ss = block_sum(ss, tmp);
  const float inv = 1.0f / sqrtf(ss / (float)D + eps);
  for (int i = threadIdx.x; i < D; i += blockDim.x) st1<T>(xrow + i, hrow[i] * inv * gain[i]);
}

// Masked positions -> LM-head rows.  Entry e lists masked position (s, j) in
// (s, j) order.  gm (guidance) 0: head row e is model row s.  1 (CFG pairs):
// head rows 2e, 2e+1 are model rows 2s (cond), 2s+1 (uncond).  2 (three-way):
// head rows 4e..4e+3 are model rows 3s (full), 3s+1 (image-only), 3s+2
// (uncond) and 3s+2 again, so an entry fills one 4-row accumulator group.
// seq_off[s] = first entry of sequence s.  Whole workgroup.
__device__ void mask_list_block(const int32_t* __restrict__ ids, int n_seq, int LB, int mask_id, int gm,
                                int32_t* __restrict__ row_map, int32_t* __restrict__ entry_pos,
                                int32_t* __restrict__ seq_off, int32_t* __restrict__ n_rows,
                                int32_t* __restrict__ n_entries, int* tmp) {
  const int n = n_seq * LB;
  int base = 0;
  for (int c0 = 0; c0 < n; c0 += blockDim.x) {
    const int i = c0 + threadIdx.x;
    const int f = (i < n && ids[i] == mask_id) ? 1 : 0;
    int total;
    const int e = base + block_exclusive_scan(f, tmp, &total);
    if (i < n && i % LB == 0) seq_off[i / LB] = e;
    if (f) {
      const int s = i / LB, j = i % LB;
      entry_pos[e] = i;
      if (gm == 2) {
#pragma unroll
        for (int v = 0; v < 4; ++v) row_map[4 * e + v] = (3 * s + min(v, 2)) * LB + j;
      } else if (gm == 1) {
        row_map[2 * e] = (2 * s) * LB + j;
        row_map[2 * e + 1] = (2 * s + 1) * LB + j;
      } else {
        row_map[e] = i;
      }
    }
    base += total;
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    seq_off[n_seq] = base;
    *n_entries = base;
    *n_rows = base * (gm == 2 ? 4 : gm + 1);
  }
}

struct MaskListArgs {
  const int32_t* ids;
  int n_seq, LB, mask_id, gm;
  int32_t *row_map, *entry_pos, *seq_off, *n_rows, *n_entries;
};

template <typename T>
__global__ __launch_bounds__(256) void k_embed_norm(const int32_t* __restrict__ ids, int ids_stride,
                                                    int n_tok, int rep, int n_embed,
                                                    const T* __restrict__ embed,
                                                    const float* __restrict__ gain, float eps, int D,
                                                    float* __restrict__ h, T* __restrict__ x, MaskListArgs ml,
                                                    uint32_t* __restrict__ zero_words, int n_zero) {
  __shared__ float tmp[16];
  __shared__ int itmp[32];
  if (blockIdx.x == gridDim.x - 1) {   // the extra workgroup: per-pass accumulators and the mask list
    for (int z = threadIdx.x; z < n_zero; z += blockDim.x) zero_words[z] = 0u;
    if (ml.ids)
      mask_list_block(ml.ids, ml.n_seq, ml.LB, ml.mask_id, ml.gm, ml.row_map, ml.entry_pos, ml.seq_off, ml.n_rows,
                      ml.n_entries, itmp);
    return;
  }
  const int i = blockIdx.x;               // model row r = i / n_tok, token j = i % n_tok
  const int r = i / n_tok, j = i % n_tok;
  // ids outside the table read the [MASK] row (last row) instead of faulting
  int id = ids[(size_t)(r / rep) * ids_stride + j];
  if (id < 0 || id >= n_embed) id = n_embed - 1;
  const T* e = embed + (size_t)id * D;
  float* hrow = h + (size_t)i * D;
  T* xrow = x + (size_t)i * D;
  constexpr int kPer = 16;   // register-resident row for D <= 16 * blockDim.x
  const int per = D / blockDim.x;
  if (D % blockDim.x == 0 && per <= kPer) {
    float v[kPer], g[kPer];
    float ss = 0.f;
#pragma unroll
    for (int m = 0; m < kPer; ++m)
      if (m < per) {
        const int c = threadIdx.x + m * blockDim.x;
        v[m] = ld1<T>(e + c);
        g[m] = gain[c];
      }
#pragma unroll
    for (int m = 0; m < kPer; ++m)
      if (m < per) ss += v[m] * v[m];
    ss = block_sum(ss, tmp);
    const float inv = 1.0f / sqrtf(ss / (float)D + eps);
#pragma unroll
    for (int m = 0; m < kPer; ++m)
      if (m < per) {
        const int c = threadIdx.x + m * blockDim.x;
        hrow[c] = v[m];
        st1<T>(xrow + c, v[m] * inv * g[m]);
      }
    return;
  }
  for (int c = threadIdx.x; c < D; c += blockDim.x) hrow[c] = ld1<T>(e + c);
  __syncthreads();
  norm_store<T>(hrow, gain, eps, D, xrow, tmp);
}

hipError_t launch_embed_norm(int mode, const int32_t* ids, int ids_stride, int rows, int n_tok,
                             int rep, int n_embed, const void* embed, const float* gain, float eps,
                             int D, float* h, void* x, const int32_t* ml_ids, int n_seq, int LB, int mask_id,
                             int gm, int32_t* row_map, int32_t* entry_pos, int32_t* seq_off, int32_t* n_rows,
                             int32_t* n_entries, uint32_t* zero_words, int n_zero, hipStream_t s) {
  const int M = rows * n_tok;
  if (M == 0) return hipSuccess;
  MaskListArgs ml{ml_ids, n_seq, LB, mask_id, gm, row_map, entry_pos, seq_off, n_rows, n_entries};
  // one workgroup per token row, plus one for the zeroing and the mask list
  if (mode == MODE_F32)
    hipLaunchKernelGGL(k_embed_norm<float>, dim3(M + 1), dim3(256), 0, s, ids, ids_stride, n_tok, rep, n_embed,
                       (const float*)embed, gain, eps, D, h, (float*)x, ml, zero_words, n_zero);
  else
    hipLaunchKernelGGL(k_embed_norm<uint16_t>, dim3(M + 1), dim3(256), 0, s, ids, ids_stride, n_tok, rep, n_embed,
                       (const uint16_t*)embed, gain, eps, D, h, (uint16_t*)x, ml, zero_words, n_zero);
  return hipGetLastError();
}

// h[t] += sum_j Y[slot_pos[t, j]] (slot t k + j when slot_pos is null) + Y[S + t]
// (shared), in a fixed order, with Y in the activation type (the expert
// kernels round each gated output row to bf16 in the bf16 paths; float32
// sums); then x = RMSNorm(h) with the next gains.  One
// workgroup per token; each thread keeps its NF float4 of the row in
// registers between the sum of squares and the normalised store.
template <typename T> __device__ __forceinline__ void st4(T* p, float a, float b, float c, float d);
template <> __device__ __forceinline__ void st4<float>(float* p, float a, float b, float c, float d) {
  *(float4*)p = make_float4(a, b, c, d);
}
template <> __device__ __forceinline__ void st4<uint16_t>(uint16_t* p, float a, float b, float c, float d) {
  *(uint2*)p = make_uint2((uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16), (uint32_t)f2bf(c) | ((uint32_t)f2bf(d) << 16));
}

// Four consecutive expert outputs (float32, or bf16 in the bf16 paths) as float.
template <typename T> __device__ __forceinline__ float4 ld4(const T* p);
template <> __device__ __forceinline__ float4 ld4<float>(const float* p) { return *(const float4*)p; }
template <> __device__ __forceinline__ float4 ld4<uint16_t>(const uint16_t* p) {
  const uint2 u = *(const uint2*)p;
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                     __uint_as_float(u.y & 0xffff0000u));
}

template <typename T, int NF>
__global__ __launch_bounds__(256) void k_combine_norm(float* __restrict__ h, const T* __restrict__ Y,
                                                      const int32_t* __restrict__ slot_pos, int D, int k,
                                                      int S, int shared, const float* __restrict__ gain,
                                                      float eps, T* __restrict__ x) {
  __shared__ float tmp[16];
  __shared__ int rows[17];
  const int t = blockIdx.x;
  if (threadIdx.x < k) rows[threadIdx.x] = slot_pos ? slot_pos[t * k + threadIdx.x] : t * k + threadIdx.x;
  if (threadIdx.x == 0) rows[k] = S + t;
  __syncthreads();
  const int nr = k + (shared ? 1 : 0);
  float4* h4 = (float4*)(h + (size_t)t * D);
  const int D4 = D >> 2;
  float4 a[NF];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NF; ++i) {
    const int f = threadIdx.x + 256 * i;
    if (f < D4) {
      float4 v = h4[f];
#pragma unroll 8
      for (int j = 0; j < nr; ++j) {
        const float4 y = ld4<T>(Y + (size_t)rows[j] * D + 4 * f);
        v.x += y.x; v.y += y.y; v.z += y.z; v.w += y.w;
      }
      h4[f] = v;
      ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
      a[i] = v;
    }
  }
  ss = block_sum(ss, tmp);
  const float inv = 1.0f / sqrtf(ss / (float)D + eps);
  const float4* g4 = (const float4*)gain;
  T* xr = x + (size_t)t * D;
#pragma unroll
  for (int i = 0; i < NF; ++i) {
    const int f = threadIdx.x + 256 * i;
    if (f < D4) {
      const float4 g = g4[f];
      st4<T>(xr + 4 * f, a[i].x * inv * g.x, a[i].y * inv * g.y, a[i].z * inv * g.z, a[i].w * inv * g.w);
    }
  }
}

hipError_t launch_combine_norm(int mode, float* h, const void* Y, const int32_t* slot_pos, int M,
                               int D, int k, int S, int shared, const float* gain, float eps,
                               void* x, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (D % 4 || D > kMaxHidden || k > 16) return hipErrorInvalidValue;
  auto go = [&](auto nf_c) {
    constexpr int NF = decltype(nf_c)::value;
    if (mode == MODE_F32)
      hipLaunchKernelGGL((k_combine_norm<float, NF>), dim3(M), dim3(256), 0, s, h, (const float*)Y, slot_pos, D, k,
                         S, shared, gain, eps, (float*)x);
    else
      hipLaunchKernelGGL((k_combine_norm<uint16_t, NF>), dim3(M), dim3(256), 0, s, h, (const uint16_t*)Y, slot_pos,
                         D, k, S, shared, gain, eps, (uint16_t*)x);
  };
  const int nf = (D / 4 + 255) / 256;   // float4 per thread
  if (nf <= 1) go(IC<1>{});
  else if (nf <= 2) go(IC<2>{});
  else if (nf <= 4) go(IC<4>{});
  else go(IC<8>{});
  return hipGetLastError();
}


// ---------------------------------------------------------------------------
// Block-wise attention (bidirectional inside a block, left to right across
// blocks), split over the key range; each workgroup handles one query block
// of one (row, head) and a range of keys (kAttnSplit for the float kernel
// below; the matrix-core kernels take their ranges from attn_plan), with an
// online softmax over 32-key tiles.  Every key a workgroup sees is visible to
// all of its queries: in a denoising step the keys are the (retained) prefix
// plus the block itself, and in an append pass the keys end at the query
// block's end.
// ---------------------------------------------------------------------------

struct AttnGeo {
  int LBp, TPQ, KT;
};

__host__ __device__ inline int pow2_at_least(int x) {
  int p = 8;
  while (p < x) p <<= 1;
  return p;
}

template <typename T>
__device__ __forceinline__ const T* key_row(const T* cache, const T* blk, const int32_t* kept,
                                            int kept_stride, int r, int h, int H, int LB, int dh,
                                            long long row_stride, long long head_stride, int i,
                                            int n_pref, int append) {
  if (append || i < n_pref) {
    const int pos = (!append && kept) ? kept[r * kept_stride + i] : i;
    return cache + (size_t)(r * row_stride + h * head_stride) + (size_t)pos * dh;
  }
  return blk + ((size_t)(r * H + h) * LB + (i - n_pref)) * dh;
}

template <typename T>
__global__ __launch_bounds__(256) void k_attn_partial(
    const T* __restrict__ q, int H, int dh, int n_tok, int LB, const T* __restrict__ kc,
    const T* __restrict__ vc, long long row_stride, long long head_stride, const T* __restrict__ bk,
    const T* __restrict__ bv, const int32_t* __restrict__ kept, const int32_t* __restrict__ n_kept,
    int kept_stride, int n_pref_all, int append, int P, int n_splits, float* __restrict__ part_o,
    float* __restrict__ part_ml) {
  extern __shared__ float smem[];
  const int LBp = pow2_at_least(LB);
  const int TPQ = 256 / LBp;
  const int KT = 32;
  const int ldk = dh + 1;
  float* sQ = smem;                    // [LBp][dh]
  float* sK = sQ + LBp * dh;           // [KT][dh+1]
  float* sV = sK + KT * ldk;           // [KT][dh+1]
  float* sP = sV + KT * ldk;           // [LBp][KT]
  const int bx = blockIdx.x, qb = blockIdx.y, sp = blockIdx.z;
  const int r = bx / H, h = bx % H;
  const int n_pref = append ? 0 : (kept ? n_kept[r] : n_pref_all);
  const int nk = append ? P + (qb + 1) * LB : n_pref + LB;
  const int k0 = sp * kAttnSplit;
  if (k0 >= nk) return;
  const int k1 = min(nk, k0 + kAttnSplit);
  const float scale = 1.0f / sqrtf((float)dh);
  const T* qsrc = q + ((size_t)(r * H + h) * n_tok + qb * LB) * dh;
  for (int e = threadIdx.x; e < LBp * dh; e += 256) {
    const int qi = e / dh, d = e % dh;
    sQ[e] = qi < LB ? ld1<T>(qsrc + (size_t)qi * dh + d) * scale : 0.f;
  }
  const int t = threadIdx.x;
  const int qi = t / TPQ, sub = t % TPQ;
  const int kpt = KT / TPQ > 0 ? KT / TPQ : 1;   // keys per thread in a tile
  const int dpt = dh / TPQ;                      // output dims per thread
  float m = -INFINITY, l = 0.f;
  float o[128 / 4];                              // dh / TPQ <= 32
  for (int i = 0; i < dpt; ++i) o[i] = 0.f;
  for (int kt = k0; kt < k1; kt += KT) {
    __syncthreads();
    for (int e = threadIdx.x; e < KT * dh; e += 256) {
      const int kk = e / dh, d = e % dh;
      const int ki = kt + kk;
      float kvk = 0.f, kvv = 0.f;
      if (ki < k1) {
        const T* kr = key_row<T>(kc, bk, kept, kept_stride, r, h, H, LB, dh, row_stride, head_stride, ki,
                                 n_pref, append);
        const T* vr = key_row<T>(vc, bv, kept, kept_stride, r, h, H, LB, dh, row_stride, head_stride, ki,
                                 n_pref, append);
        kvk = ld1<T>(kr + d);
        kvv = ld1<T>(vr + d);
      }
      sK[kk * ldk + d] = kvk;
      sV[kk * ldk + d] = kvv;
    }
    __syncthreads();
    // scores of this thread's keys
    float sc[32];
    float tmax = -INFINITY;
    for (int j = 0; j < kpt; ++j) {
      const int kk = sub + j * TPQ;
      float a = -INFINITY;
      if (kk < KT && kt + kk < k1) {
        a = 0.f;
        for (int d = 0; d < dh; ++d) a += sQ[qi * dh + d] * sK[kk * ldk + d];
      }
      sc[j] = a;
      tmax = fmaxf(tmax, a);
    }
    for (int off = 1; off < TPQ; off <<= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, off, 64));
    const float mn = fmaxf(m, tmax);
    const float corr = (m == -INFINITY) ? 0.f : expf(m - mn);
    float psum = 0.f;
    for (int j = 0; j < kpt; ++j) {
      const int kk = sub + j * TPQ;
      const float p = (sc[j] == -INFINITY) ? 0.f : expf(sc[j] - mn);
      psum += p;
      if (kk < KT) sP[qi * KT + kk] = p;
    }
    for (int off = 1; off < TPQ; off <<= 1) psum += __shfl_xor(psum, off, 64);
    l = l * corr + psum;
    m = mn;
    __syncthreads();
    for (int i = 0; i < dpt; ++i) {
      const int d = sub * dpt + i;
      float a = o[i] * corr;
      for (int kk = 0; kk < KT; ++kk) a += sP[qi * KT + kk] * sV[kk * ldk + d];
      o[i] = a;
    }
  }
  if (qi < LB) {
    const size_t base = ((size_t)(bx * gridDim.y + qb) * n_splits + sp);
    float* po = part_o + (base * LBp + qi) * dh;
    for (int i = 0; i < dpt; ++i) po[sub * dpt + i] = o[i];
    if (sub == 0) {
      part_ml[(base * LBp + qi) * 2 + 0] = m;
      part_ml[(base * LBp + qi) * 2 + 1] = l;
    }
  }
}

// B operand of O += P V for output columns 16 dt .. 16 dt + 15, from a 32-key
// V tile held row-major in LDS (row pitch ld bf16): slot j of lane (g, c16)
// is V[key 16 (j / 4) + 4 g + j % 4][16 dt + c16], the key order of the P
// fragments.  Two transposed LDS reads (ds_read_b64_tr_b16) instead of eight
// 2-byte reads: in each 16-lane group g, lane 4 a + b gives the address of
// key 4 g + a (then 16 + 4 g + a), columns 16 dt + 4 b .. + 3, and every lane
// receives its own column c16 of the group's four keys.  Every lane of the
// wavefront takes part, so callers reach it with the whole wavefront active.
// A pitch of DH + 16 puts the rows one half-wavefront reads 8 banks apart.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x8 pv_operand(const uint16_t* vt, int ld, int dt, int g, int c16) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  uint16_t* p = const_cast<uint16_t*>(vt) + (4 * g + (c16 >> 2)) * ld + 16 * dt + 4 * (c16 & 3);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 16 * ld));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// bf16 matrix-core variant for blocks of <= 32 queries.  A workgroup of 4
// wavefronts covers kAttnSplitMfma consecutive keys of one (row, head, query
// block); wavefront w owns the 32-key tile at split start + 32 w:
//   - its K and V rows are requested before any arithmetic: unconditional
//     16-byte loads from one base pointer when the tile lies contiguously in
//     one buffer, otherwise per-key row pointers resolved once (one lookup
//     per lane, including the retained-position indirection) and handed out
//     by shuffles, so no load waits on another;
//   - S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (A = 16 key rows, B = 16
//     query rows, both contiguous 16-byte row segments; Q staged once per
//     workgroup through LDS), so each lane ends up with the scores of one
//     query (lane % 16) for 4 keys of each 16-key half -- the A-operand layout
//     of P for the P V product;
//   - softmax over the tile, O = P V with V staged through the wave's own LDS
//     tile and read as the B operand.
// The four (m, l, O) states meet in LDS (aliasing the tiles, after a
// barrier); wavefront w merges output column tiles w, w + 4, ... and writes
// that slice of the workgroup's partial.
template <int DH>
__global__ __launch_bounds__(256) void k_attn_mfma(
    const uint16_t* __restrict__ q, int H, int n_tok, int LB, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, long long row_stride, long long head_stride,
    const uint16_t* __restrict__ bk, const uint16_t* __restrict__ bv, const int32_t* __restrict__ kept,
    const int32_t* __restrict__ n_kept, int kept_stride, int n_pref_all, int append, int P, int n_splits,
    float* __restrict__ part_o, float* __restrict__ part_ml) {
  constexpr int NW = 4;
  constexpr int NKC = DH / 32;              // 32-wide chunks of the head dimension
  constexpr int NDT = DH / 16;              // 16-wide output column tiles
  constexpr int VLD = DH + 16;              // padded LDS row of a V tile (bf16)
  constexpr int QLD = DH + 8;               // padded LDS row of Q (bf16)
  constexpr int OLD = DH + 4;               // padded LDS row of a merge slot (float)
  constexpr int SEGS = DH / 8;              // 16-byte segments per key row
  constexpr int VSEG = (32 * SEGS) / 64;    // V segments per lane
  static_assert(NW * 32 == kAttnSplitMfma, "split = 4 tiles of 32 keys");
  extern __shared__ __align__(16) uint8_t attn_smem_raw[];
  uint16_t* vt_all = (uint16_t*)attn_smem_raw;          // [NW][32][VLD]
  uint16_t* qs = vt_all + NW * 32 * VLD;                 // [32][QLD]
  float* mO = (float*)attn_smem_raw;                     // [NW][32][OLD] (after the tiles are dead)
  float* mM = mO + NW * 32 * OLD;                        // [NW][32]
  float* mL = mM + NW * 32;                              // [NW][32]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int bx = blockIdx.x, qb = blockIdx.y, sp = blockIdx.z;
  const int r = bx / H, h = bx % H;
  const int n_pref = append ? 0 : (kept ? n_kept[r] : n_pref_all);
  const int nk = append ? P + (qb + 1) * LB : n_pref + LB;
  const int kw0 = sp * kAttnSplitMfma + wave * 32;
  const int kw1 = min(nk, kw0 + 32);
  const int g = lane >> 4, c16 = lane & 15;
  uint4 kf[2][NKC];
  uint4 vr[VSEG];
  const bool in_cache = !append && kept == nullptr && kw0 + 32 <= n_pref;
  const bool in_block = !append && kw0 >= n_pref && kw0 + 32 <= nk;
  const bool in_app = append && kw0 + 32 <= nk;
  if (in_cache || in_block || in_app) {
    const size_t base = in_block ? ((size_t)(r * H + h) * LB + (kw0 - n_pref)) * DH
                                 : (size_t)(r * row_stride + h * head_stride) + (size_t)kw0 * DH;
    const uint16_t* kb = (in_block ? bk : kc) + base;
    const uint16_t* vb = (in_block ? bv : vc) + base;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int c = 0; c < NKC; ++c) kf[kt][c] = *(const uint4*)(kb + (kt * 16 + c16) * DH + 32 * c + 8 * g);
#pragma unroll
    for (int j = 0; j < VSEG; ++j) vr[j] = *(const uint4*)(vb + (size_t)(lane + 64 * j) * 8);
  } else {
    // lane resolves key kw0 + (lane & 31); keys at or past kw1 are never loaded
    const int kl = kw0 + (lane & 31);
    const uint16_t* kpl = kc;
    const uint16_t* vpl = vc;
    if (kl < kw1) {
      kpl = key_row<uint16_t>(kc, bk, kept, kept_stride, r, h, H, LB, DH, row_stride, head_stride, kl, n_pref, append);
      vpl = key_row<uint16_t>(vc, bv, kept, kept_stride, r, h, H, LB, DH, row_stride, head_stride, kl, n_pref, append);
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int kk = kt * 16 + c16;
      const uint16_t* kr = (const uint16_t*)__shfl((long long)kpl, kk, 64);
      const bool ok = kw0 + kk < kw1;
#pragma unroll
      for (int c = 0; c < NKC; ++c) kf[kt][c] = ok ? *(const uint4*)(kr + 32 * c + 8 * g) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < VSEG; ++j) {
      const int sg = lane + 64 * j;
      const int kk = sg / SEGS, part = sg % SEGS;
      const uint16_t* vp = (const uint16_t*)__shfl((long long)vpl, kk, 64);
      vr[j] = kw0 + kk < kw1 ? *(const uint4*)(vp + part * 8) : make_uint4(0, 0, 0, 0);
    }
  }
  // Q of the query block -> LDS (rows past LB are zero) -> B-operand fragments
  for (int sg = threadIdx.x; sg < 32 * SEGS; sg += 64 * NW) {
    const int qi = sg / SEGS, part = sg % SEGS;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (qi < LB) val = *(const uint4*)(q + ((size_t)(r * H + h) * n_tok + qb * LB + qi) * DH + part * 8);
    *(uint4*)(qs + qi * QLD + part * 8) = val;
  }
  __syncthreads();
  uint4 qf[2][NKC];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int c = 0; c < NKC; ++c) qf[qt][c] = *(const uint4*)(qs + (qt * 16 + c16) * QLD + 32 * c + 8 * g);
  f32x4 o[2][NDT];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[qt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_q[2] = {-INFINITY, -INFINITY}, l_q[2] = {0.f, 0.f};   // statistics of query qt * 16 + c16
  if (kw0 < nk) {
    const float scale = 1.0f / sqrtf((float)DH);
    uint16_t* vt = vt_all + wave * 32 * VLD;
#pragma unroll
    for (int j = 0; j < VSEG; ++j) {
      const int sg = lane + 64 * j;
      *(uint4*)(vt + (sg / SEGS) * VLD + (sg % SEGS) * 8) = vr[j];
    }
    f32x4 s[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        s[kt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NKC; ++c)
          s[kt][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[kt][c]),
                                                              __builtin_bit_cast(bf16x8, qf[qt][c]), s[kt][qt], 0, 0, 0);
      }
    // softmax per query over the tile: lane holds query c16 (+16 qt), keys 16 kt + 4 g + v
    bf16x8 pa[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      float sv[8];
      float tmax = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int ki = kw0 + kt * 16 + 4 * g + v;
          const float x = ki < kw1 ? s[kt][qt][v] * scale : -INFINITY;
          sv[kt * 4 + v] = x;
          tmax = fmaxf(tmax, x);
        }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      float ps = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float pj = sv[j] == -INFINITY ? 0.f : expf(sv[j] - tmax);
        ps += pj;
        pa[qt][j] = (__bf16)pj;
      }
      ps += __shfl_xor(ps, 16, 64);
      ps += __shfl_xor(ps, 32, 64);
      m_q[qt] = tmax;
      l_q[qt] = ps;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // O = P V
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const bf16x8 vb = pv_operand(vt, VLD, dt, g, c16);
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) o[qt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[qt], vb, o[qt][dt], 0, 0, 0);
    }
  }
  __syncthreads();   // tiles dead: the merge slots alias them
  // accumulator rows are queries qt * 16 + 4 g + v
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) mO[(wave * 32 + qt * 16 + 4 * g + v) * OLD + dt * 16 + c16] = o[qt][dt][v];
    if (g == 0) {
      mM[wave * 32 + qt * 16 + c16] = m_q[qt];
      mL[wave * 32 + qt * 16 + c16] = l_q[qt];
    }
  }
  __syncthreads();
  const size_t part = (size_t)(bx * gridDim.y + qb) * n_splits + sp;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int qi = qt * 16 + 4 * g + v;
      float ms[NW], mx = -INFINITY;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        ms[w] = mM[w * 32 + qi];
        mx = fmaxf(mx, ms[w]);
      }
      float f[NW], L = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        f[w] = ms[w] == -INFINITY ? 0.f : expf(ms[w] - mx);
        L += f[w] * mL[w * 32 + qi];
      }
      for (int dt = wave; dt < NDT; dt += NW) {
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) acc += f[w] * mO[(w * 32 + qi) * OLD + dt * 16 + c16];
        part_o[(part * 32 + qi) * DH + dt * 16 + c16] = acc;
      }
      if (wave == 0 && c16 == 0) {
        part_ml[(part * 32 + qi) * 2 + 0] = mx;
        part_ml[(part * 32 + qi) * 2 + 1] = L;
      }
    }
}

// Streaming variant for contiguous key ranges: no retained-prefix
// indirection, and in a denoising step a prefix length that is a multiple of
// 32, so no 32-key tile straddles the cache and the block buffer.  A
// workgroup of 4 wavefronts covers `split` consecutive keys of one (row,
// head, query block); wavefront w takes the 32-key tiles w, w + 4, ... of
// that range with an online softmax (running max m, sum l and unnormalised
// O per query; a new tile with maximum m' rescales them by e^(m - m')).  The
// next tile's K is requested right after the current S product and its V
// right after the current V reached LDS, and the loop body has no branch, so
// the compiler waits only for the tile in use.  Rows of a partial tile read
// the tile's last valid row instead (finite values, weight 0).  Keys below
// kbeg are masked out (weight 0): a compacted retained prefix is padded with
// kbeg < 32 zero rows in front to a whole number of tiles.  With one
// split the workgroup normalises and writes the output and the log-sum-exp
// itself (out != null); otherwise it writes a partial like k_attn_mfma.
template <int DH>
struct StreamTile {
  static constexpr int NKC = DH / 32, VSEG = DH / 16, SEGS = DH / 8;
  __device__ __forceinline__ static void load_k(u32x4 (&kf)[2][NKC], const uint16_t* __restrict__ kb, int last) {
    const int lane = threadIdx.x & 63, g = lane >> 4, c16 = lane & 15;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int row = min(kt * 16 + c16, last);
#pragma unroll
      for (int c = 0; c < NKC; ++c) kf[kt][c] = *(const u32x4*)(kb + row * DH + 32 * c + 8 * g);
    }
  }
  __device__ __forceinline__ static void load_v(u32x4 (&vr)[VSEG], const uint16_t* __restrict__ vb, int last) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < VSEG; ++j) {
      const int sg = lane + 64 * j;
      const int row = min(sg / SEGS, last);
      vr[j] = *(const u32x4*)(vb + row * DH + (sg % SEGS) * 8);
    }
  }
};

template <int DH>
__global__ __launch_bounds__(256, 2) void k_attn_stream(
    const uint16_t* __restrict__ q, int H, int n_tok, int LB, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, long long row_stride, long long head_stride,
    const uint16_t* __restrict__ bk, const uint16_t* __restrict__ bv, int n_pref, int append, int P,
    int n_splits, int split, float* __restrict__ part_o, float* __restrict__ part_ml, uint16_t* __restrict__ out,
    float* __restrict__ lse, int kbeg) {
  constexpr int NW = 4;
  constexpr int NKC = DH / 32;
  constexpr int NDT = DH / 16;
  constexpr int VLD = DH + 16;              // padded LDS row of a V tile (bf16)
  constexpr int QLD = DH + 8;               // padded LDS row of Q (bf16)
  constexpr int OLD = DH + 4;               // padded LDS row of a merge slot (float)
  constexpr int SEGS = DH / 8;
  constexpr int VSEG = (32 * SEGS) / 64;
  typedef StreamTile<DH> TL;
  extern __shared__ __align__(16) uint8_t attn_smem_raw[];
  uint16_t* vt_all = (uint16_t*)attn_smem_raw;          // [NW][32][VLD]
  uint16_t* qs = vt_all + NW * 32 * VLD;                 // [32][QLD]
  float* mO = (float*)attn_smem_raw;                     // [NW][32][OLD] (after the tiles are dead)
  float* mM = mO + NW * 32 * OLD;                        // [NW][32]
  float* mL = mM + NW * 32;                              // [NW][32]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int bx = blockIdx.x, qb = blockIdx.y, sp = blockIdx.z;
  const int r = bx / H, h = bx % H;
  const int np = append ? 0 : n_pref;
  const int nk = append ? P + (qb + 1) * LB : np + LB;
  const int kend = min(nk, sp * split + split);
  const int k_first = sp * split + 32 * wave;
  const int nt = k_first < kend ? (kend - k_first + 32 * NW - 1) / (32 * NW) : 0;   // this wavefront's tiles
  const size_t hoff = (size_t)r * row_stride + (size_t)h * head_stride;
  const size_t boff = (size_t)(r * H + h) * LB;
  // first key of a tile -> its K / V rows in the cache or the block buffer
  auto kptr = [&](int k0) { return (!append && k0 >= np) ? bk + (boff + (k0 - np)) * DH : kc + hoff + (size_t)k0 * DH; };
  auto vptr = [&](int k0) { return (!append && k0 >= np) ? bv + (boff + (k0 - np)) * DH : vc + hoff + (size_t)k0 * DH; };
  const int g = lane >> 4, c16 = lane & 15;
  u32x4 kf[2][NKC];
  u32x4 vr[VSEG];
  if (nt > 0) {
    TL::load_k(kf, kptr(k_first), min(31, kend - 1 - k_first));
    TL::load_v(vr, vptr(k_first), min(31, kend - 1 - k_first));
  }
  // Q of the query block -> LDS (rows past LB are zero) -> B-operand fragments
  for (int sg = threadIdx.x; sg < 32 * SEGS; sg += 64 * NW) {
    const int qi = sg / SEGS, part = sg % SEGS;
    u32x4 val = u32x4{0u, 0u, 0u, 0u};
    if (qi < LB) val = *(const u32x4*)(q + ((size_t)(r * H + h) * n_tok + qb * LB + qi) * DH + part * 8);
    *(u32x4*)(qs + qi * QLD + part * 8) = val;
  }
  __syncthreads();
  u32x4 qf[2][NKC];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int c = 0; c < NKC; ++c) qf[qt][c] = *(const u32x4*)(qs + (qt * 16 + c16) * QLD + 32 * c + 8 * g);
  f32x4 o[2][NDT];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[qt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // running max (log2 units) and sum of query qt * 16 + c16: scores are
  // scaled by log2(e) / sqrt(d_h) so the exponentials are single v_exp_f32
  float m_q[2] = {-INFINITY, -INFINITY}, l_q[2] = {0.f, 0.f};
  const float scale = 1.4426950408889634f / sqrtf((float)DH);
  uint16_t* vt = vt_all + wave * 32 * VLD;
  // one tile at key k0: S^T = K Q^T, (next K), softmax update, V -> LDS, (next V), O += P V
  auto tile = [&](int k0, auto pf) {
    constexpr bool PF = decltype(pf)::value;
    f32x4 sc[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        sc[kt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NKC; ++c)
          sc[kt][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[kt][c]),
                                                               __builtin_bit_cast(bf16x8, qf[qt][c]), sc[kt][qt], 0, 0, 0);
      }
    const int kn = k0 + 32 * NW;
    if (PF) TL::load_k(kf, kptr(kn), min(31, kend - 1 - kn));
    bf16x8 pa[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      float sv[8];
      float tmax = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int ki = k0 + kt * 16 + 4 * g + v;
          const float x = (ki < kend && ki >= kbeg) ? sc[kt][qt][v] * scale : -INFINITY;
          sv[kt * 4 + v] = x;
          tmax = fmaxf(tmax, x);
        }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      const float mn = fmaxf(m_q[qt], tmax);    // finite: every tile holds a valid key
      const float alpha = __builtin_amdgcn_exp2f(m_q[qt] - mn);   // 0 on the first tile
      float ps = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float pj = __builtin_amdgcn_exp2f(sv[j] - mn);
        ps += pj;
        pa[qt][j] = (__bf16)pj;
      }
      ps += __shfl_xor(ps, 16, 64);
      ps += __shfl_xor(ps, 32, 64);
      l_q[qt] = l_q[qt] * alpha + ps;
      m_q[qt] = mn;
      // accumulator rows are queries 4 g + v: their factor sits in lane 4 g + v;
      // once the running maxima settle no query's max moves and the rescale
      // is skipped (a wavefront-uniform test)
      if (__ballot(alpha != 1.0f)) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float av = __shfl(alpha, 4 * g + v, 64);
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) o[qt][dt][v] *= av;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < VSEG; ++j) {
      const int sg = lane + 64 * j;
      *(u32x4*)(vt + (sg / SEGS) * VLD + (sg % SEGS) * 8) = vr[j];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (PF) TL::load_v(vr, vptr(kn), min(31, kend - 1 - kn));
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const bf16x8 vb = pv_operand(vt, VLD, dt, g, c16);
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) o[qt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[qt], vb, o[qt][dt], 0, 0, 0);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  int k0 = k_first;
#pragma unroll 1
  for (int t = 0; t + 1 < nt; ++t, k0 += 32 * NW) tile(k0, std::true_type{});
  if (nt > 0) tile(k0, std::false_type{});
  __syncthreads();   // tiles dead: the merge slots alias them
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) mO[(wave * 32 + qt * 16 + 4 * g + v) * OLD + dt * 16 + c16] = o[qt][dt][v];
    if (g == 0) {
      mM[wave * 32 + qt * 16 + c16] = m_q[qt];
      mL[wave * 32 + qt * 16 + c16] = l_q[qt];
    }
  }
  __syncthreads();
  const size_t part = (size_t)(bx * gridDim.y + qb) * n_splits + sp;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int qi = qt * 16 + 4 * g + v;
      float ms[NW], mx = -INFINITY;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        ms[w] = mM[w * 32 + qi];
        mx = fmaxf(mx, ms[w]);
      }
      float f[NW], L = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        f[w] = ms[w] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms[w] - mx);
        L += f[w] * mL[w * 32 + qi];
      }
      mx *= 0.69314718055994531f;   // back to natural-log units for the log-sum-exp and the partials
      if (out) {   // the only split: final output row of query qi
        if (qi < LB) {
          const float inv = 1.0f / L;
          uint16_t* op = out + ((size_t)r * n_tok + qb * LB + qi) * (H * DH) + h * DH;
          for (int dt = wave; dt < NDT; dt += NW) {
            float acc = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) acc += f[w] * mO[(w * 32 + qi) * OLD + dt * 16 + c16];
            op[dt * 16 + c16] = f2bf(acc * inv);
          }
          if (lse && wave == 0 && c16 == 0) lse[((size_t)r * H + h) * n_tok + qb * LB + qi] = mx + logf(L);
        }
        continue;
      }
      for (int dt = wave; dt < NDT; dt += NW) {
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) acc += f[w] * mO[(w * 32 + qi) * OLD + dt * 16 + c16];
        part_o[(part * 32 + qi) * DH + dt * 16 + c16] = acc;
      }
      if (wave == 0 && c16 == 0) {
        part_ml[(part * 32 + qi) * 2 + 0] = mx;
        part_ml[(part * 32 + qi) * 2 + 1] = L;
      }
    }
}

// Append passes (a clean forward of whole blocks): query block qb of a row
// sees the cached keys and the pass's own keys through its block, P + (qb +
// 1) L_B of them (block-causal).  k_attn_stream gives each query block its
// own workgroup, so a pass of n blocks streams each (row, head)'s keys n
// times.  Here a workgroup of 4 wavefronts takes 4 consecutive query blocks
// of one (row, head): every 32-key tile of K and V is loaded once into LDS
// (double-buffered, the next tile's loads in flight during the products) and
// read by each wavefront whose block still sees it.  Wavefront w keeps its
// own online softmax over all of its block's keys (base 2, as in
// k_attn_stream; rows of a partial tile read the last key instead, weight 0),
// so there is no merge, and writes its normalised output rows and their
// log-sum-exp.
template <int DH>
__global__ __launch_bounds__(256, 2) void k_attn_append(const uint16_t* __restrict__ q, int H, int n_tok, int LB,
                                                        const uint16_t* __restrict__ kc,
                                                        const uint16_t* __restrict__ vc, long long row_stride,
                                                        long long head_stride, int P, uint16_t* __restrict__ out,
                                                        float* __restrict__ lse) {
  constexpr int NW = 4, NKC = DH / 32, NDT = DH / 16, LD = DH + 8;   // LD: padded LDS row of K (bf16)
  constexpr int VLD = DH + 16;                                        // padded LDS row of V (bf16)
  constexpr int SEGS = DH / 8;                                        // 16-byte segments of a key row
  constexpr int LPT = (32 * SEGS + 255) / 256;                        // loads per thread, per matrix and tile
  __shared__ __align__(16) uint16_t ks[2 * 32 * LD];
  __shared__ __align__(16) uint16_t vs[2 * 32 * VLD];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int r = blockIdx.x / H, h = blockIdx.x % H;
  const int nqb = n_tok / LB;
  const int qb = blockIdx.y * NW + wave;                 // this wavefront's query block
  const bool live = qb < nqb;
  const int nk_w = live ? P + (qb + 1) * LB : 0;         // its keys
  const int qb_last = min(nqb, (int)(blockIdx.y + 1) * NW) - 1;
  const int nk_max = P + (qb_last + 1) * LB;             // keys of the workgroup's last block
  const int ntile = (nk_max + 31) / 32;
  const size_t hoff = (size_t)r * row_stride + (size_t)h * head_stride;
  const uint16_t* kb = kc + hoff;
  const uint16_t* vb = vc + hoff;
  // Q fragments from global memory, as the B operand (query row qt 16 + c16,
  // elements 32 c + 8 g ..); rows past L_B are zero
  u32x4 qf[2][NKC];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int c = 0; c < NKC; ++c) {
      const int row = qt * 16 + c16;
      qf[qt][c] = (live && row < LB)
                      ? *(const u32x4*)(q + ((size_t)(r * H + h) * n_tok + qb * LB + row) * DH + 32 * c + 8 * g)
                      : u32x4{0u, 0u, 0u, 0u};
    }
  // the workgroup's share of one tile: 16-byte segment sg = tid + 256 j of
  // key row sg / SEGS (clamped to the last key), for K and for V
  u32x4 kr[LPT], vr[LPT];
  auto fetch = [&](int t) {
#pragma unroll
    for (int j = 0; j < LPT; ++j) {
      const int sg = threadIdx.x + 256 * j;
      if (sg < 32 * SEGS) {
        const int key = min(32 * t + sg / SEGS, nk_max - 1);
        kr[j] = *(const u32x4*)(kb + (size_t)key * DH + (sg % SEGS) * 8);
        vr[j] = *(const u32x4*)(vb + (size_t)key * DH + (sg % SEGS) * 8);
      }
    }
  };
  auto put = [&](int slot) {
#pragma unroll
    for (int j = 0; j < LPT; ++j) {
      const int sg = threadIdx.x + 256 * j;
      if (sg < 32 * SEGS) {
        *(u32x4*)(ks + (slot * 32 + sg / SEGS) * LD + (sg % SEGS) * 8) = kr[j];
        *(u32x4*)(vs + (slot * 32 + sg / SEGS) * VLD + (sg % SEGS) * 8) = vr[j];
      }
    }
  };
  f32x4 o[2][NDT];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[qt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_q[2] = {-INFINITY, -INFINITY}, l_q[2] = {0.f, 0.f};   // of query qt 16 + c16, log2 units
  const float scale = 1.4426950408889634f / sqrtf((float)DH);
  fetch(0);
  put(0);
  __syncthreads();
  for (int t = 0; t < ntile; ++t) {
    if (t + 1 < ntile) fetch(t + 1);
    const int k0 = 32 * t;
    if (k0 < nk_w) {   // wavefront-uniform: the tile holds at least one of this block's keys
      const uint16_t* kt_s = ks + (t & 1) * 32 * LD;
      const uint16_t* vt_s = vs + (t & 1) * 32 * VLD;
      f32x4 sc[2][2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        u32x4 kf[NKC];
#pragma unroll
        for (int c = 0; c < NKC; ++c) kf[c] = *(const u32x4*)(kt_s + (kt * 16 + c16) * LD + 32 * c + 8 * g);
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          sc[kt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c = 0; c < NKC; ++c)
            sc[kt][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[c]),
                                                                 __builtin_bit_cast(bf16x8, qf[qt][c]), sc[kt][qt], 0,
                                                                 0, 0);
        }
      }
      bf16x8 pa[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        float sv[8];
        float tmax = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int ki = k0 + kt * 16 + 4 * g + v;
            const float x = ki < nk_w ? sc[kt][qt][v] * scale : -INFINITY;
            sv[kt * 4 + v] = x;
            tmax = fmaxf(tmax, x);
          }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        const float mn = fmaxf(m_q[qt], tmax);   // finite: the tile holds a valid key
        const float alpha = __builtin_amdgcn_exp2f(m_q[qt] - mn);
        float ps = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float pj = __builtin_amdgcn_exp2f(sv[j] - mn);
          ps += pj;
          pa[qt][j] = (__bf16)pj;
        }
        ps += __shfl_xor(ps, 16, 64);
        ps += __shfl_xor(ps, 32, 64);
        l_q[qt] = l_q[qt] * alpha + ps;
        m_q[qt] = mn;
        if (__ballot(alpha != 1.0f)) {
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float av = __shfl(alpha, 4 * g + v, 64);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) o[qt][dt][v] *= av;
          }
        }
      }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const bf16x8 vbf = pv_operand(vt_s, VLD, dt, g, c16);
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
          o[qt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[qt], vbf, o[qt][dt], 0, 0, 0);
      }
    }
    if (t + 1 < ntile) put((t + 1) & 1);
    __syncthreads();   // tile t + 1 is in its slot; slot t % 2 is no longer read
  }
  if (!live) return;
  // accumulator rows are queries qt 16 + 4 g + v; their max and sum sit in lane 4 g + v
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float lq = __shfl(l_q[qt], 4 * g + v, 64);
      const float mq = __shfl(m_q[qt], 4 * g + v, 64);
      const int qi = qt * 16 + 4 * g + v;
      if (qi < LB) {
        uint16_t* op = out + ((size_t)r * n_tok + qb * LB + qi) * (H * DH) + h * DH;
        const float inv = 1.0f / lq;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) op[dt * 16 + c16] = f2bf(o[qt][dt][v] * inv);
        if (lse && c16 == 0) lse[((size_t)r * H + h) * n_tok + qb * LB + qi] = mq * 0.69314718055994531f + logf(lq);
      }
    }
}

static size_t attn_smem(int LB, int dh) {
  const int LBp = pow2_at_least(LB);
  return sizeof(float) * ((size_t)LBp * dh + 2 * 32 * (dh + 1) + (size_t)LBp * 32);
}

static size_t attn_mfma_smem(int dh) {
  const size_t tiles = ((size_t)4 * 32 * (dh + 16) + 32 * (dh + 8)) * sizeof(uint16_t);
  const size_t merge = ((size_t)4 * 32 * (dh + 4) + 2 * 4 * 32) * sizeof(float);
  return tiles > merge ? tiles : merge;
}

static bool attn_mfma_ok(int mode, int LB, int dh) {
  return mode != MODE_F32 && LB <= 32 && (dh == 32 || dh == 64 || dh == 128);
}

AttnPlan attn_plan(int mode, int rows, int H, int n_tok, int LB, int dh, int nk_max, int gather, int n_pref,
                   int append) {
  AttnPlan pl;
  if (!attn_mfma_ok(mode, LB, dh)) {
    pl.kind = kAttnFloat;
    pl.split = kAttnSplit;
  } else if (gather || (!append && n_pref % 32 != 0)) {
    pl.kind = kAttnMfma;
    pl.split = kAttnSplitMfma;
  } else if (append && n_tok / LB >= 4 && rows * H * ((n_tok / LB + 3) / 4) >= kAttnAppendMinWg) {
    // append pass of 4+ query blocks: 4 blocks share each key tile
    pl.kind = kAttnAppend;
    pl.split = nk_max;
  } else {
    // about one workgroup per compute unit: few long key ranges stream best,
    // and one split lets the kernel write the output without a merge pass
    const int units = rows * H * (n_tok / LB);
    const int max_splits = (nk_max + kAttnSplitMfma - 1) / kAttnSplitMfma;
    int ns = units >= kAttnStreamUnits ? 1 : (kAttnStreamUnits + units - 1) / units;
    ns = ns < max_splits ? ns : max_splits;
    const int per = (nk_max + ns - 1) / ns;
    pl.kind = kAttnStream;
    pl.split = (per + kAttnSplitMfma - 1) / kAttnSplitMfma * kAttnSplitMfma;
  }
  pl.n_splits = (nk_max + pl.split - 1) / pl.split;
  return pl;
}

// Retained prefix K and V of every layer, row and head copied into a
// contiguous buffer: rows [0, pad) zero, rows [pad, pad + n) the kept
// positions kept[r][0 .. n) in their (ascending) order, so the streaming
// attention reads the retained prefix as whole 32-key tiles (masking the
// first pad keys).  Grid: (rows x H, row segments / 256, layers); one
// 16-byte segment of K and of V per thread.
__global__ __launch_bounds__(256) void k_kv_compact(const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
                                                    long long src_layer, long long src_row, long long src_head,
                                                    const int32_t* __restrict__ kept, int kept_stride, int n, int pad,
                                                    int H, int dh, uint16_t* __restrict__ kd,
                                                    uint16_t* __restrict__ vd, long long dst_layer, long long dst_row,
                                                    long long dst_head) {
  const int r = blockIdx.x / H, h = blockIdx.x % H, l = blockIdx.z;
  const int segs = dh / 8;
  const int e = blockIdx.y * 256 + threadIdx.x;
  if (e >= (pad + n) * segs) return;
  const int i = e / segs, sg = e % segs;
  const size_t dof = (size_t)l * dst_layer + (size_t)r * dst_row + (size_t)h * dst_head + (size_t)i * dh + sg * 8;
  uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
  if (i >= pad) {
    const size_t so = (size_t)l * src_layer + (size_t)r * src_row + (size_t)h * src_head +
                      (size_t)kept[(size_t)r * kept_stride + (i - pad)] * dh + sg * 8;
    kv = *(const uint4*)(kc + so);
    vv = *(const uint4*)(vc + so);
  }
  *(uint4*)(kd + dof) = kv;
  *(uint4*)(vd + dof) = vv;
}

hipError_t launch_kv_compact(const void* kc, const void* vc, long long src_layer, long long src_row,
                             long long src_head, const int32_t* kept, int kept_stride, int n, int pad, int rows, int H,
                             int dh, int layers, void* kd, void* vd, long long dst_layer, long long dst_row,
                             long long dst_head, hipStream_t s) {
  const int total = (pad + n) * (dh / 8);
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(k_kv_compact, dim3(rows * H, (total + 255) / 256, layers), dim3(256), 0, s, (const uint16_t*)kc,
                     (const uint16_t*)vc, src_layer, src_row, src_head, kept, kept_stride, n, pad, H, dh,
                     (uint16_t*)kd, (uint16_t*)vd, dst_layer, dst_row, dst_head);
  return hipGetLastError();
}

// Merge of the key-split partials of one (row, head, query block):
// out = sum_s e^(m_s - M) O_s / sum_s e^(m_s - M) l_s with M = max_s m_s, and
// lse = M + log(sum_s e^(m_s - M) l_s).  kCombineTpo threads share one
// (query, 4 output columns) group: thread `sub` folds splits sub, sub + TPO,
// ... with every load of a chunk in flight at once (online rescaling between
// chunks), then the group's states merge by shuffles.  Partials hold LBp query
// rows each.
constexpr int kCombineTpo = 2;
constexpr int kCombineChunk = 8;

template <typename T>
__global__ __launch_bounds__(256) void k_attn_combine(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_ml, int H, int dh,
                                                      int n_tok, int LB, int LBp, int n_splits, int split,
                                                      int n_pref_all, const int32_t* __restrict__ n_kept,
                                                      int append, int P, T* __restrict__ out,
                                                      float* __restrict__ lse) {
  constexpr int TPO = kCombineTpo, CH = kCombineChunk;
  const int bx = blockIdx.x, qb = blockIdx.y;
  const int r = bx / H, h = bx % H;
  const int cols4 = dh >> 2;
  const int e = blockIdx.z * blockDim.x + threadIdx.x;
  const int og = e / TPO, sub = e % TPO;
  const bool live = og < LB * cols4;
  const int qi = live ? og / cols4 : 0, d = live ? (og % cols4) * 4 : 0;
  const int n_pref = append ? 0 : (n_kept ? n_kept[r] : n_pref_all);
  const int nk = append ? P + (qb + 1) * LB : n_pref + LB;
  const int ns = live ? min(n_splits, (nk + split - 1) / split) : 0;
  const size_t base0 = (size_t)(bx * gridDim.y + qb) * n_splits;
  float M = -INFINITY, L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = sub; s0 < ns; s0 += CH * TPO) {
    float2 ml[CH];
    float4 po[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int sj = s0 + j * TPO;
      if (sj < ns) {
        const size_t row = (base0 + sj) * LBp + qi;
        ml[j] = *(const float2*)(part_ml + row * 2);
        po[j] = *(const float4*)(part_o + row * dh + d);
      } else {
        ml[j] = make_float2(-INFINITY, 0.f);
        po[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    float mc = M;
#pragma unroll
    for (int j = 0; j < CH; ++j) mc = fmaxf(mc, ml[j].x);
    const float f = M == -INFINITY ? 0.f : expf(M - mc);
    L *= f;
    acc.x *= f; acc.y *= f; acc.z *= f; acc.w *= f;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const float w = ml[j].x == -INFINITY ? 0.f : expf(ml[j].x - mc);
      L += w * ml[j].y;
      acc.x += w * po[j].x; acc.y += w * po[j].y; acc.z += w * po[j].z; acc.w += w * po[j].w;
    }
    M = mc;
  }
#pragma unroll
  for (int o = 1; o < TPO; o <<= 1) {
    const float Mo = __shfl_xor(M, o, 64), Lo = __shfl_xor(L, o, 64);
    const float ax = __shfl_xor(acc.x, o, 64), ay = __shfl_xor(acc.y, o, 64);
    const float az = __shfl_xor(acc.z, o, 64), aw = __shfl_xor(acc.w, o, 64);
    const float mx = fmaxf(M, Mo);
    const float fa = M == -INFINITY ? 0.f : expf(M - mx);
    const float fb = Mo == -INFINITY ? 0.f : expf(Mo - mx);
    L = L * fa + Lo * fb;
    acc.x = acc.x * fa + ax * fb; acc.y = acc.y * fa + ay * fb;
    acc.z = acc.z * fa + az * fb; acc.w = acc.w * fa + aw * fb;
    M = mx;
  }
  if (!live || sub != 0) return;
  const float inv = 1.0f / L;
  T* op = out + ((size_t)r * n_tok + qb * LB + qi) * (H * dh) + h * dh + d;
  st1<T>(op + 0, acc.x * inv);
  st1<T>(op + 1, acc.y * inv);
  st1<T>(op + 2, acc.z * inv);
  st1<T>(op + 3, acc.w * inv);
  if (lse && d == 0) lse[((size_t)r * H + h) * n_tok + qb * LB + qi] = M + logf(L);
}

static hipError_t launch_attn_combine(int mode, const float* part_o, const float* part_ml, int rows, int H,
                                      int dh, int n_tok, int LB, int n_splits, int split, int n_pref,
                                      const int32_t* n_kept, int append, int P, void* out, float* lse,
                                      hipStream_t s) {
  const int LBp = attn_mfma_ok(mode, LB, dh) ? 32 : pow2_at_least(LB);   // query rows per partial
  const int threads = LB * (dh / 4) * kCombineTpo;
  dim3 grid(rows * H, n_tok / LB, (threads + 255) / 256);
  if (mode == MODE_F32)
    hipLaunchKernelGGL(k_attn_combine<float>, grid, dim3(256), 0, s, part_o, part_ml, H, dh, n_tok, LB, LBp,
                       n_splits, split, n_pref, n_kept, append, P, (float*)out, lse);
  else
    hipLaunchKernelGGL(k_attn_combine<uint16_t>, grid, dim3(256), 0, s, part_o, part_ml, H, dh, n_tok, LB, LBp,
                       n_splits, split, n_pref, n_kept, append, P, (uint16_t*)out, lse);
  return hipGetLastError();
}

hipError_t launch_attn(const AttnPlan& pl, int mode, const void* q, int rows, int H, int dh, int n_tok, int LB,
                       const void* kc, const void* vc, long long row_stride, long long head_stride, const void* bk,
                       const void* bv, const int32_t* kept, const int32_t* n_kept, int kept_stride, int n_pref,
                       int append, int P, float* part_o, float* part_ml, void* out, float* lse, hipStream_t s,
                       int kbeg) {
  const int n_splits = pl.n_splits;
  dim3 grid(rows * H, n_tok / LB, n_splits);
  if (pl.kind == kAttnAppend) {
    dim3 ga(rows * H, (n_tok / LB + 3) / 4);
#define DLLM_ATTN_APPEND(DHV)                                                                                    \
  hipLaunchKernelGGL(k_attn_append<DHV>, ga, dim3(256), 0, s, (const uint16_t*)q, H, n_tok, LB, (const uint16_t*)kc, \
                     (const uint16_t*)vc, row_stride, head_stride, P, (uint16_t*)out, lse)
    if (dh == 128) DLLM_ATTN_APPEND(128);
    else if (dh == 64) DLLM_ATTN_APPEND(64);
    else DLLM_ATTN_APPEND(32);
#undef DLLM_ATTN_APPEND
    return hipGetLastError();
  }
  if (pl.kind == kAttnStream) {
    const size_t smm = attn_mfma_smem(dh);
    uint16_t* fo = n_splits == 1 ? (uint16_t*)out : nullptr;
#define DLLM_ATTN_STREAM(DHV)                                                                                   \
  hipLaunchKernelGGL(k_attn_stream<DHV>, grid, dim3(256), smm, s, (const uint16_t*)q, H, n_tok, LB,            \
                     (const uint16_t*)kc, (const uint16_t*)vc, row_stride, head_stride, (const uint16_t*)bk,   \
                     (const uint16_t*)bv, n_pref, append, P, n_splits, pl.split, part_o, part_ml, fo, lse, kbeg)
    if (dh == 128) DLLM_ATTN_STREAM(128);
    else if (dh == 64) DLLM_ATTN_STREAM(64);
    else DLLM_ATTN_STREAM(32);
#undef DLLM_ATTN_STREAM
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || n_splits == 1) return e;
  } else if (pl.kind == kAttnMfma) {
    const size_t smm = attn_mfma_smem(dh);
#define DLLM_ATTN_MFMA(DHV)                                                                                     \
  hipLaunchKernelGGL(k_attn_mfma<DHV>, grid, dim3(256), smm, s, (const uint16_t*)q, H, n_tok, LB, (const uint16_t*)kc, \
                     (const uint16_t*)vc, row_stride, head_stride, (const uint16_t*)bk, (const uint16_t*)bv, kept,     \
                     n_kept, kept_stride, n_pref, append, P, n_splits, part_o, part_ml)
    if (dh == 128) DLLM_ATTN_MFMA(128);
    else if (dh == 64) DLLM_ATTN_MFMA(64);
    else DLLM_ATTN_MFMA(32);
#undef DLLM_ATTN_MFMA
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else {
    const size_t sm = attn_smem(LB, dh);
    if (mode == MODE_F32)
      hipLaunchKernelGGL(k_attn_partial<float>, grid, dim3(256), sm, s, (const float*)q, H, dh, n_tok, LB,
                         (const float*)kc, (const float*)vc, row_stride, head_stride, (const float*)bk,
                         (const float*)bv, kept, n_kept, kept_stride, n_pref, append, P, n_splits,
                         part_o, part_ml);
    else
      hipLaunchKernelGGL(k_attn_partial<uint16_t>, grid, dim3(256), sm, s, (const uint16_t*)q, H, dh, n_tok,
                         LB, (const uint16_t*)kc, (const uint16_t*)vc, row_stride, head_stride,
                         (const uint16_t*)bk, (const uint16_t*)bv, kept, n_kept, kept_stride, n_pref,
                         append, P, n_splits, part_o, part_ml);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_attn_combine(mode, part_o, part_ml, rows, H, dh, n_tok, LB, n_splits, pl.split, n_pref, n_kept,
                             append, P, out, lse, s);
}

// Attention probability mass on every prefix key, summed over heads and the
// block's queries: mass[r][i] += sum_h sum_q exp(q.k_i / sqrt(dh) - lse_q).
// One writer per key, layers in order: deterministic.
template <typename T>
__global__ __launch_bounds__(256) void k_attn_mass(const T* __restrict__ q, const float* __restrict__ lse,
                                                   int H, int dh, int LB, const T* __restrict__ kc,
                                                   long long row_stride, long long head_stride, int P,
                                                   float* __restrict__ mass, int mass_stride,
                                                   float* __restrict__ part) {
  extern __shared__ float smem[];
  const int ldk = dh + 1;
  float* sK = smem;               // [64][dh+1]
  float* sQ = sK + 64 * ldk;      // [LB][dh]
  float* sL = sQ + LB * dh;       // [LB]
  const int r = blockIdx.x, base = blockIdx.y * 64;
  const int t = threadIdx.x, kk = t >> 2, qs = t & 3;
  const float scale = 1.0f / sqrtf((float)dh);
  float acc = 0.f;
  // with part: workgroup z takes head z alone and writes its partial mass
  const int h_lo = part ? blockIdx.z : 0, h_hi = part ? blockIdx.z + 1 : H;
  for (int h = h_lo; h < h_hi; ++h) {
    __syncthreads();
    const T* qsrc = q + (size_t)(r * H + h) * LB * dh;
    for (int e = t; e < LB * dh; e += 256) sQ[e] = ld1<T>(qsrc + e) * scale;
    for (int e = t; e < LB; e += 256) sL[e] = lse[((size_t)r * H + h) * LB + e];
    for (int e = t; e < 64 * dh; e += 256) {
      const int kr = e / dh, d = e % dh;
      const int i = base + kr;
      sK[kr * ldk + d] = i < P ? ld1<T>(kc + (size_t)(r * row_stride + h * head_stride) + (size_t)i * dh + d) : 0.f;
    }
    __syncthreads();
    if (base + kk < P) {
      for (int qi = qs; qi < LB; qi += 4) {
        float a = 0.f;
        for (int d = 0; d < dh; ++d) a += sQ[qi * dh + d] * sK[kk * ldk + d];
        acc += expf(a - sL[qi]);
      }
    }
  }
  acc += __shfl_xor(acc, 1, 64);
  acc += __shfl_xor(acc, 2, 64);
  if (qs == 0 && base + kk < P) {
    if (part) part[((size_t)blockIdx.z * gridDim.x + r) * mass_stride + base + kk] = acc;
    else mass[(size_t)r * mass_stride + base + kk] += acc;
  }
}

// The same per-head mass on matrix cores (bf16, block <= 32): workgroup (row
// x head, 128 keys), wavefront w takes keys 32 w .. 32 w + 31 of the range:
// S^T = K Q^T as in the streaming attention, p = e^(s / sqrt(d) - lse) of
// each query, summed over the block's queries (in registers, then across the
// 16 query lanes by shuffles).  part[h][r][key].
template <int DH>
__global__ __launch_bounds__(256) void k_attn_mass_mfma(const uint16_t* __restrict__ q, const float* __restrict__ lse,
                                                        int H, int LB, const uint16_t* __restrict__ kc,
                                                        long long row_stride, long long head_stride, int P,
                                                        float* __restrict__ part, int mass_stride) {
  constexpr int NKC = DH / 32, QLD = DH + 8, SEGS = DH / 8;
  __shared__ __align__(16) uint16_t qs[32 * QLD];
  __shared__ float ls[32];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, c16 = lane & 15;
  const int rows = gridDim.x / H, r = blockIdx.x / H, h = blockIdx.x % H;
  const int k0 = blockIdx.y * 128 + 32 * wave;
  u32x4 kf[2][NKC];
  if (k0 < P)
    StreamTile<DH>::load_k(kf, kc + (size_t)r * row_stride + (size_t)h * head_stride + (size_t)k0 * DH,
                           min(31, P - 1 - k0));
  for (int sg = threadIdx.x; sg < 32 * SEGS; sg += 256) {
    const int qi = sg / SEGS, pt = sg % SEGS;
    u32x4 val = u32x4{0u, 0u, 0u, 0u};
    if (qi < LB) val = *(const u32x4*)(q + ((size_t)(r * H + h) * LB + qi) * DH + pt * 8);
    *(u32x4*)(qs + qi * QLD + pt * 8) = val;
  }
  if (threadIdx.x < 32) ls[threadIdx.x] = threadIdx.x < LB ? lse[((size_t)r * H + h) * LB + threadIdx.x] : 0.f;
  __syncthreads();
  if (k0 >= P) return;
  u32x4 qf[2][NKC];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int c = 0; c < NKC; ++c) qf[qt][c] = *(const u32x4*)(qs + (qt * 16 + c16) * QLD + 32 * c + 8 * g);
  const float scale = 1.0f / sqrtf((float)DH);
  float ms[2][4];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
    for (int v = 0; v < 4; ++v) ms[kt][v] = 0.f;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NKC; ++c)
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[kt][c]),
                                                    __builtin_bit_cast(bf16x8, qf[qt][c]), sc, 0, 0, 0);
      const int qi = qt * 16 + c16;   // accumulator (v) of lane (g, c16): key 16 kt + 4 g + v, query qi
      if (qi < LB) {
#pragma unroll
        for (int v = 0; v < 4; ++v) ms[kt][v] += expf(sc[v] * scale - ls[qi]);
      }
    }
  }
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float x = ms[kt][v];
      x += __shfl_xor(x, 1, 64);
      x += __shfl_xor(x, 2, 64);
      x += __shfl_xor(x, 4, 64);
      x += __shfl_xor(x, 8, 64);
      const int key = k0 + kt * 16 + 4 * g + v;
      if (c16 == 0 && key < P) part[((size_t)h * rows + r) * mass_stride + key] = x;
    }
}

// mass[r][p] += sum over heads h = 0, 1, ... of part[h][r][p] (fixed order).
__global__ __launch_bounds__(256) void k_mass_reduce(const float* __restrict__ part, int rows, int H, int P,
                                                     float* __restrict__ mass, int mass_stride) {
  const int r = blockIdx.y, p = blockIdx.x * 256 + threadIdx.x;
  if (p >= P) return;
  float a = 0.f;
  for (int h = 0; h < H; ++h) a += part[((size_t)h * rows + r) * mass_stride + p];
  mass[(size_t)r * mass_stride + p] += a;
}

hipError_t launch_attn_mass(int mode, const void* q, const float* lse, int rows, int H, int dh, int LB,
                            const void* kc, long long row_stride, long long head_stride, int P,
                            float* mass, int mass_stride, hipStream_t s, float* part) {
  if (P == 0) return hipSuccess;
  // with a partial buffer ([H][rows][mass_stride]): one workgroup per (row,
  // 64 keys, head), then a fixed-order sum over heads
  dim3 grid(rows, (P + 63) / 64, part ? H : 1);
  const size_t sm = sizeof(float) * (64 * (dh + 1) + LB * dh + LB);
  if (part && mode != MODE_F32 && LB <= 32 && (dh == 32 || dh == 64 || dh == 128)) {
    dim3 gm(rows * H, (P + 127) / 128);
    auto go = [&](auto dh_c) {
      hipLaunchKernelGGL((k_attn_mass_mfma<decltype(dh_c)::value>), gm, dim3(256), 0, s, (const uint16_t*)q, lse, H,
                         LB, (const uint16_t*)kc, row_stride, head_stride, P, part, mass_stride);
    };
    if (dh == 128) go(IC<128>{});
    else if (dh == 64) go(IC<64>{});
    else go(IC<32>{});
  } else if (mode == MODE_F32)
    hipLaunchKernelGGL(k_attn_mass<float>, grid, dim3(256), sm, s, (const float*)q, lse, H, dh, LB,
                       (const float*)kc, row_stride, head_stride, P, mass, mass_stride, part);
  else
    hipLaunchKernelGGL(k_attn_mass<uint16_t>, grid, dim3(256), sm, s, (const uint16_t*)q, lse, H, dh, LB,
                       (const uint16_t*)kc, row_stride, head_stride, P, mass, mass_stride, part);
  if (part)
    hipLaunchKernelGGL(k_mass_reduce, dim3((P + 255) / 256, rows), dim3(256), 0, s, part, rows, H, P, mass,
                       mass_stride);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Router: sigmoid scores (float64 evaluation rounded to float32), selection
// key = score + bias in float32, top-k with ties to the lower expert id,
// gates = selected scores normalised to sum 1 (summed in selection order).
//
// One wavefront per token.  The k-th largest key is found by a radix select
// on an order-preserving 32-bit code of the key: 32 steps, each a handful of
// ballots and scalar popcounts, with no cross-lane shuffle chain.  Keys above
// the threshold are taken, keys equal to it fill the remaining slots lowest
// expert id first, and the k winners are ranked among themselves (key
// descending, id ascending) through a small per-wave LDS area.
// ---------------------------------------------------------------------------

// Words of LDS one wavefront of topk_token uses.
constexpr int kTopkLdsWords = 5 * 16;

// Order-preserving code: for non-NaN a, b: a > b  <=>  code(a) > code(b);
// -0 and +0 share a code.  Every non-NaN float maps to a code >= 1.
__device__ __forceinline__ uint32_t sortable_u32(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Number of set bits of m at lanes below the calling lane.
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Makes the wave's own LDS stores visible to all its lanes.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One whole wavefront (all 64 lanes active): selection for token `tok` from
// its E <= 256 logits, each the sum of n_split partials (logits[z zs + tok E
// + e], slice stride zs, summed in z order), k <= 16.  w = kTopkLdsWords words of LDS owned by this
// wave.  Results go to idx/gates (and idx_copy when not null) at
// [tok * k + rank]; lane r < k returns the expert of rank r, other lanes -1.
// z_out (optional, inspection): the summed logits [tok][E] the keys came from.
__device__ __forceinline__ int topk_token(const float* __restrict__ logits, int n_split, size_t zs,
                                           const float* __restrict__ bias, int tok, int E, int k,
                                           int32_t* __restrict__ idx, float* __restrict__ gates,
                                           int32_t* __restrict__ idx_copy, float* __restrict__ z_out,
                                           uint32_t* w) {
  const int lane = threadIdx.x & 63;
  float sc[4];
  uint32_t u[4];
  float lg[4];
  if (n_split == kRouterSplit) {   // partials [kRouterSplit][tok][e]: all 8 loads of a logit in flight
    float pz[4][kRouterSplit];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = j * 64 + lane;
      const float* p = logits + (size_t)tok * E + (e < E ? e : 0);
#pragma unroll
      for (int z = 0; z < kRouterSplit; ++z) pz[j][z] = p[z * zs];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float a = pz[j][0];
#pragma unroll
      for (int z = 1; z < kRouterSplit; ++z) a += pz[j][z];
      lg[j] = a;
    }
  } else {   // partials [n_split][tok][e], summed in split order
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = j * 64 + lane;
      float a = 0.f;
      if (e < E)
        for (int z = 0; z < n_split; ++z) a += logits[z * zs + (size_t)tok * E + e];
      lg[j] = a;
    }
  }
  if (z_out) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (j * 64 + lane < E) z_out[(size_t)tok * E + j * 64 + lane] = lg[j];
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = j * 64 + lane;
    if (e < E) {
      const double z = (double)lg[j];
      sc[j] = (float)(1.0 / (1.0 + exp(-z)));
      u[j] = sortable_u32(sc[j] + bias[e]);
    } else {
      sc[j] = 0.f;
      u[j] = 0u;   // below every real key
    }
  }
  // threshold T = k-th largest code = the largest T with #{code >= T} >= k
  uint32_t T = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = T | (1u << b);
    int n = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) n += __popcll(__ballot(u[j] >= c));
    if (n >= k) T = c;
  }
  int need = k;
#pragma unroll
  for (int j = 0; j < 4; ++j) need -= __popcll(__ballot(u[j] > T));
  uint32_t* su = w;                 // [16] codes of the winners (expert order)
  uint32_t* se = w + 16;            // [16] their expert ids
  float* ss = (float*)(w + 32);     // [16] their scores
  uint32_t* oe = w + 48;            // [16] expert ids in rank order
  float* os = (float*)(w + 64);     // [16] scores in rank order
  int base = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {     // expert id order: j major, lane minor
    const bool eq = u[j] == T;
    const uint64_t beq = __ballot(eq);
    const bool take = u[j] > T || (eq && lanes_below(beq) < need);
    const int neq = __popcll(beq);
    need -= neq < need ? neq : need;
    const uint64_t bt = __ballot(take);
    if (take) {
      const int p = base + lanes_below(bt);
      su[p] = u[j];
      se[p] = (uint32_t)(j * 64 + lane);
      ss[p] = sc[j];
    }
    base += __popcll(bt);
  }
  wave_lds_sync();
  if (lane < k) {
    const uint32_t mu = su[lane], me = se[lane];
    int r = 0;
    for (int m = 0; m < k; ++m) {
      const uint32_t ou = su[m], oi = se[m];
      r += (ou > mu || (ou == mu && oi < me)) ? 1 : 0;
    }
    oe[r] = me;
    os[r] = ss[lane];
  }
  wave_lds_sync();
  float sum = 0.f;
  for (int m = 0; m < k; ++m) sum += os[m];
  if (lane < k) {
    const int e = (int)oe[lane];
    const size_t o = (size_t)tok * k + lane;
    idx[o] = e;
    gates[o] = os[lane] / sum;
    if (idx_copy) idx_copy[o] = e;
    return e;
  }
  return -1;
}

// Four tokens per workgroup.  masks (optional, kMaskWords words, zero before
// the launch) accumulates the bit set of the experts any token selected.
__global__ __launch_bounds__(256) void k_router_topk(const float* __restrict__ logits, int n_split,
                                                     const float* __restrict__ bias, int M, int E, int k,
                                                     int32_t* __restrict__ idx, float* __restrict__ gates,
                                                     int32_t* __restrict__ idx_copy, uint32_t* __restrict__ masks,
                                                     float* __restrict__ z_out) {
  __shared__ uint32_t wl[4][kTopkLdsWords];
  __shared__ uint32_t bits[kMaskWords];
  const int wave = threadIdx.x >> 6;
  const int tok = blockIdx.x * 4 + wave;
  if (threadIdx.x < kMaskWords) bits[threadIdx.x] = 0u;
  __syncthreads();
  if (tok < M) {
    const int e = topk_token(logits, n_split, (size_t)M * E, bias, tok, E, k, idx, gates, idx_copy, z_out, wl[wave]);
    if (masks && e >= 0) atomicOr(&bits[e >> 5], 1u << (e & 31));
  }
  __syncthreads();
  if (masks && threadIdx.x < kMaskWords && bits[threadIdx.x]) atomicOr(&masks[threadIdx.x], bits[threadIdx.x]);
}

hipError_t launch_router_topk(const float* logits, int n_split, const float* bias, int M, int E, int k,
                              int32_t* idx, float* gates, int32_t* idx_copy, uint32_t* masks, hipStream_t s,
                              float* z_out) {
  if (M == 0) return hipSuccess;
  hipLaunchKernelGGL(k_router_topk, dim3((M + 3) / 4), dim3(256), 0, s, logits, n_split, bias, M, E, k, idx, gates,
                     idx_copy, masks, z_out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Token permutation: expert-major order of the (token, slot) pairs, one
// thread per slot over S / 256 workgroups.  Every workgroup counts the
// expert ids of all S slots in LDS (each expert's total, and its count in
// the slots before the workgroup's own range), scans the totals into the
// expert offsets off[e], and gives each of its slots a place among its
// expert's slots: the count before its range plus an LDS counter.  Slot s
// goes to row off[e] + place.  The first workgroup also writes off[] and the
// work items {expert, first row, rows, 0} that cover each expert's rows in
// chunks, longest first: the shared expert's (index E, all M tokens, rows S
// ..) lead, then the routed items by decreasing row count, so a launch's last
// workgroups run its shortest items.  The order of the slots within an
// expert, and so which rows share an item, varies between runs; no result
// depends on it: every row is computed on its own (a product row depends
// only on its own input row), and the combine reads each slot's row through
// slot_pos.
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void k_permute(const int32_t* __restrict__ idx, const float* __restrict__ gates,
                                                 int M, int E, int k, int shared, int chunk,
                                                 int32_t* __restrict__ off, int32_t* __restrict__ tok,
                                                 float* __restrict__ gate_sorted, int32_t* __restrict__ slot_pos,
                                                 int4* __restrict__ items, int32_t* __restrict__ n_items) {
  __shared__ int cnt[256], before[256], here[256];
  __shared__ int tmp[32];
  __shared__ int hist[65], bcur[65];   // routed items per row count; next list place per row count
  const int tid = threadIdx.x;         // blockDim.x = 256 >= E: one expert per thread in the scans
  const int S = M * k;
  const int first = blockIdx.x * 256;
  const int s = first + tid;
  cnt[tid] = 0;
  before[tid] = 0;
  here[tid] = 0;
  __syncthreads();
  // histogram of all slots; ids of slots before this range also go to before[]
  int i = tid;
  for (; i + 3 * 256 < S; i += 4 * 256) {   // four loads in flight
    int e4[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) e4[u] = idx[i + u * 256];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      atomicAdd(&cnt[e4[u]], 1);
      if (i + u * 256 < first) atomicAdd(&before[e4[u]], 1);
    }
  }
  for (; i < S; i += 256) {
    const int e = idx[i];
    atomicAdd(&cnt[e], 1);
    if (i < first) atomicAdd(&before[e], 1);
  }
  __syncthreads();
  const int ce = tid < E ? cnt[tid] : 0;
  int total;
  const int ex_off = block_exclusive_scan(ce, tmp, &total);
  __syncthreads();   // every thread has read cnt[]: it now holds the offsets
  cnt[tid] = ex_off;
  __syncthreads();
  if (s < S) {
    const int e = idx[s];
    const int pos = cnt[e] + before[e] + atomicAdd(&here[e], 1);
    tok[pos] = s / k;
    gate_sorted[pos] = gates[s];
    slot_pos[s] = pos;
  }
  if (shared && s < M) tok[S + s] = s;
  if (blockIdx.x != 0) return;
  // first workgroup: expert offsets and the work list
  const int nc = (ce + chunk - 1) / chunk;   // this expert's items
  int n_routed;
  (void)block_exclusive_scan(nc, tmp, &n_routed);
  const int sh_chunks = shared ? (M + chunk - 1) / chunk : 0;
  if (tid < E) off[tid] = ex_off;
  if (tid < 65) hist[tid] = 0;
  __syncthreads();
  for (int j = 0; j < nc; ++j) atomicAdd(&hist[min(chunk, ce - j * chunk)], 1);
  __syncthreads();
  if (tid == 0) {
    int acc = sh_chunks;
    for (int rsz = 64; rsz >= 1; --rsz) {
      bcur[rsz] = acc;
      acc += hist[rsz];
    }
    off[E] = S;
    off[E + 1] = S + (shared ? M : 0);
    *n_items = sh_chunks + n_routed;
  }
  for (int j = tid; j < sh_chunks; j += 256) items[j] = make_int4(E, S + j * chunk, min(chunk, M - j * chunk), 0);
  __syncthreads();
  for (int j = 0; j < nc; ++j) {
    const int rows = min(chunk, ce - j * chunk);
    items[atomicAdd(&bcur[rows], 1)] = make_int4(tid, ex_off + j * chunk, rows, 0);
  }
}

hipError_t launch_permute(const int32_t* idx, const float* gates, int M, int E, int k, int shared, int chunk,
                          int32_t* off, int32_t* tok, float* gate_sorted, int32_t* slot_pos, int4* items,
                          int32_t* n_items, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (E < 1 || E > 256 || chunk < 1 || chunk > 64 || k < 1) return hipErrorInvalidValue;
  const int S = M * k;
  hipLaunchKernelGGL(k_permute, dim3((S + 255) / 256), dim3(256), 0, s, idx, gates, M, E, k, shared, chunk, off,
                     tok, gate_sorted, slot_pos, items, n_items);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Grouped expert SwiGLU FFN over the work items (expert, 32-row chunk).
//  gate/up: Hmid[row] = silu(x W_g^T) * (x W_u^T) for 16 features per
//           workgroup; 8 wavefronts split the hidden dimension, each with
//           its gate and up fragments in flight together;
//  down:    Y[row] = gate_row * (Hmid[row] W_d^T); each wavefront owns 16
//           outputs over the whole expert width.
// The row-tile count of an item is a template parameter chosen per
// workgroup, so loads and MFMAs are fully unrolled.  fp8 weights carry one
// float32 scale per output row, applied to the accumulated dot product.
// ---------------------------------------------------------------------------

constexpr int kExpWaves = 8;
// 16-row MFMA tiles of an expert work item
constexpr int kExpNrt = kRowChunk / 16;
#ifndef DLLM_GU_MINBLK
#define DLLM_GU_MINBLK 4
#endif
#ifndef DLLM_DN_MINBLK
#define DLLM_DN_MINBLK 4
#endif
#ifndef DLLM_GU_CT_FP8
#define DLLM_GU_CT_FP8 2
#endif
#ifndef DLLM_DN_CT_FP8
#define DLLM_DN_CT_FP8 4
#endif

// Weight fragments of one batch (U chunks) for NW matrices.
template <int MODE, int NW, int U>
__device__ __forceinline__ void load_w(typename Op<MODE>::WF (&wf)[NW][U],
                                       const typename Op<MODE>::TW* const (&wp)[NW], int k) {
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int w = 0; w < NW; ++w) wf[w][u] = Op<MODE>::ldw(wp[w] + k + Op<MODE>::KC * u);
}

// Weight fragments of chunks kc .. kc + U - 1 (Op<MODE>::KC reduction
// elements each) from uniform bases wb[] at the lane's 32-bit element offset
// lo (one offset register serves all NW matrices), chunk stride cs elements:
// KC in the row-major layout, 64 KL in the packed fragment layout.
template <int MODE, int NW, int U>
__device__ __forceinline__ void load_wc(typename Op<MODE>::WF (&wf)[NW][U],
                                        const typename Op<MODE>::TW* const (&wb)[NW], uint32_t lo, int kc, int cs) {
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      // byte offset in 32 bits from a uniform base: the scalar-base + vector
      // offset addressing form
      const uint32_t bo = (lo + (uint32_t)((kc + u) * cs)) * (uint32_t)sizeof(typename Op<MODE>::TW);
      wf[w][u] = Op<MODE>::ldw((const typename Op<MODE>::TW*)((const char*)wb[w] + bo));
    }
}

template <int MODE, int NRT, int U>
__device__ __forceinline__ void load_a(typename Op<MODE>::AF (&af)[NRT][U], const typename Op<MODE>::TA* const (&ap)[NRT],
                                       const bool (&av)[NRT], int k) {
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int u = 0; u < U; ++u) af[rt][u] = av[rt] ? Op<MODE>::lda(ap[rt] + k + Op<MODE>::KC * u) : Op<MODE>::za();
}

template <int MODE, int NRT, int NW, int U>
__device__ __forceinline__ void mma_apply(f32x4 (&acc)[NW][NRT], const typename Op<MODE>::AF (&af)[NRT][U],
                                          const typename Op<MODE>::WF (&wf)[NW][U]) {
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int w = 0; w < NW; ++w) Op<MODE>::mma(acc[w][rt], af[rt][u], wf[w][u]);
}

// The weight batch depends only on (expert, columns) and is issued first; the
// token gather for the A rows resolves while those loads are in flight.
// Gate/up MFMA loop of one chunk (cnt <= 16 * NRT rows) over CT 16-column
// tiles (matrices gate 0, up 0, gate 1, up 1, ... sharing every A fragment)
// whose first weight batch wf (from wb at this wave's k offset) is already
// requested: rows_tok gives the source token of row rr, rows_out its Hmid
// row.  NRT 16-row tiles are allocated; the loads and products of unused ones
// are skipped at run time (one code path keeps the register allocation free
// of spills).
template <int MODE, int NRT, int U, int CT>
__device__ void gateup_compute(const ExpertArgs& a, int e, int cnt, int col0, bool shared_e, float* red,
                               const int* rows_out, const int* rows_tok, typename Op<MODE>::WF (&wf)[2 * CT][U],
                               const typename Op<MODE>::TW* const (&wb)[2 * CT], uint32_t lo, int cs) {
  typedef typename Op<MODE>::TA TA;
  constexpr int KC = Op<MODE>::KC, KL = Op<MODE>::KL, NM = 2 * CT;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int D = a.D;
  const int Fe = shared_e ? a.Fs : a.F;
  const int kper = D / kExpWaves;
  const int k0 = wave * kper;
  const int nrt = (cnt + 15) >> 4;   // row tiles in use (cnt <= 16 * NRT)
  const TA* X = (const TA*)a.X;
  const TA* ap[NRT];
  bool av[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const int rr = rt * 16 + (lane & 15);
    av[rt] = rr < cnt;
    const int src = av[rt] ? rows_tok[rr] : 0;
    ap[rt] = X + (size_t)src * D + KL * (lane >> 4);
  }
  f32x4 acc[NM][NRT];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) acc[m][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k = k0;;) {
    // one row tile at a time keeps the A fragments to U registers groups
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      if (rt < nrt) {
        typename Op<MODE>::AF af[U];
#pragma unroll
        for (int u = 0; u < U; ++u) af[u] = av[rt] ? Op<MODE>::lda(ap[rt] + k + KC * u) : Op<MODE>::za();
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int m = 0; m < NM; ++m) Op<MODE>::mma(acc[m][rt], af[u], wf[m][u]);
      }
    }
    k += KC * U;
    if (k >= k0 + kper) break;
    load_wc<MODE, NM, U>(wf, wb, lo, k / KC, cs);
  }
#pragma unroll
  for (int m = 0; m < NM; ++m) reduce_waves<NRT, kExpWaves>(acc[m], red);
  if (wave != 0) return;   // only wave 0 stores
  TA* Hm = (TA*)a.Hmid;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int col = col0 + 16 * ct + (lane & 15);
    float sg = 1.f, su = 1.f;
    if (MODE == MODE_FP8 && !shared_e) {
      sg = a.sg[(size_t)e * a.F + col];
      su = a.su[(size_t)e * a.F + col];
    }
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int rr = rt * 16 + 4 * (lane >> 4) + v;
        if (rr < cnt && col < Fe) {
          const float g = acc[2 * ct][rt][v] * sg, u = acc[2 * ct + 1][rt][v] * su;
          st1<TA>(Hm + (size_t)rows_out[rr] * a.Fmax + col, g / (1.0f + expf(-g)) * u);
        }
      }
  }
}

// One gate/up chunk of expert e (shared_e: the shared expert), columns col0
// .. col0 + 16 CT - 1: the first weight batch is requested first, then
// `stage()` (whole workgroup: stages rows_out / rows_tok behind a barrier and
// returns the row count, 1 .. 32) runs while those loads are in flight.  WM
// is the weight format, UMAX the largest batch.  Tile ct of a matrix starts
// 16 ct D elements after tile 0 in both weight layouts.
template <int WM, int UMAX, int NRT = 2, bool PK = false, int CT = 1, class Stage>
__device__ void gateup_chunk(const ExpertArgs& a, int e, int col0, bool shared_e, float* red, const int* rows_out,
                             const int* rows_tok, Stage& stage) {
  typedef typename Op<WM>::TW TW;
  constexpr int KC = Op<WM>::KC, KL = Op<WM>::KL;
  const int chunks = a.D / (KC * kExpWaves);
  pick_u<UMAX>(chunks, [&](auto u) {
    constexpr int UU = decltype(u)::value;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int D = a.D;
    const int col = col0 + (lane & 15);
    const TW* wg = shared_e ? (const TW*)a.swg : (const TW*)a.wg + (size_t)e * a.F * D;
    const TW* wu = shared_e ? (const TW*)a.swu : (const TW*)a.wu + (size_t)e * a.F * D;
    // row-major: lane l reads row col at k + KL (l / 16); packed (PK, routed
    // experts only): fragment (col0 / 16, k / KC) is 64 lanes x KL elements
    const uint32_t lo = PK ? ((col0 >> 4) * (D / KC) * 64 + lane) * KL : col * D + KL * (lane >> 4);   // < F * D
    constexpr int cs = PK ? 64 * KL : KC;
    const TW* wb[2 * CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      wb[2 * ct] = wg + (size_t)16 * ct * D;
      wb[2 * ct + 1] = wu + (size_t)16 * ct * D;
    }
    typename Op<WM>::WF wf[2 * CT][UU];
    load_wc<WM, 2 * CT, UU>(wf, wb, lo, wave * (D / kExpWaves) / KC, cs);
    const int cnt = stage();
    gateup_compute<WM, NRT, UU, CT>(a, e, cnt, col0, shared_e, red, rows_out, rows_tok, wf, wb, lo, cs);
  });
}

// Down-projection MFMA loop of one chunk with its first weight batch in wf
// (unused 16-row tiles skipped at run time); CT 16-column tiles per wavefront
// share every A fragment.
template <int MODE, int NRT, int U, int CT>
__device__ void down_compute(const ExpertArgs& a, int e, int cnt, int col0, bool shared_e, const int* rows_out,
                             typename Op<MODE>::WF (&wf)[CT][U], const typename Op<MODE>::TW* const (&wp)[CT]) {
  typedef typename Op<MODE>::TA TA;
  constexpr int KC = Op<MODE>::KC, KL = Op<MODE>::KL;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int D = a.D;
  const int Ke = shared_e ? a.Fs : a.F;
  const int nrt = (cnt + 15) >> 4;
  const TA* Hm = (const TA*)a.Hmid;
  const TA* ap[NRT];
  bool av[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const int rr = rt * 16 + (lane & 15);
    av[rt] = rr < cnt;
    ap[rt] = Hm + (size_t)rows_out[av[rt] ? rr : 0] * a.Fmax + KL * (lane >> 4);
  }
  f32x4 acc[CT][NRT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) acc[ct][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k = 0;;) {
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      if (rt < nrt) {
        typename Op<MODE>::AF af[U];
#pragma unroll
        for (int u = 0; u < U; ++u) af[u] = av[rt] ? Op<MODE>::lda(ap[rt] + k + KC * u) : Op<MODE>::za();
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) Op<MODE>::mma(acc[ct][rt], af[u], wf[ct][u]);
      }
    }
    k += KC * U;
    if (k >= Ke) break;
    load_w<MODE, CT, U>(wf, wp, k);
  }
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int col = col0 + (wave * CT + ct) * 16 + (lane & 15);
    float sd = 1.f;
    if (MODE == MODE_FP8 && !shared_e) sd = a.sd[(size_t)e * D + col];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int rr = rt * 16 + 4 * (lane >> 4) + v;
        if (rr < cnt) {
          const int row = rows_out[rr];
          const float g = shared_e ? 1.f : a.gate_rows[row];
          st1<typename Op<MODE>::TA>((typename Op<MODE>::TA*)a.Y + (size_t)row * D + col, acc[ct][rt][v] * sd * g);
        }
      }
  }
}

// One down-projection chunk (output columns col0 .. col0 + 64 CT - 1, 16 CT
// per wave): first weight batch requested, then `stage()`, then the MFMA loop.
template <int WM, int UMAX, int NRT = 2, int CT = 1, class Stage>
__device__ void down_chunk(const ExpertArgs& a, int e, int col0, bool shared_e, const int* rows_out, Stage& stage) {
  typedef typename Op<WM>::TW TW;
  constexpr int KL = Op<WM>::KL;
  const int Ke = shared_e ? a.Fs : a.F;
  const int chunks = Ke / Op<WM>::KC;
  pick_u<UMAX>(chunks, [&](auto u) {
    constexpr int UU = decltype(u)::value;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const TW* wd = shared_e ? (const TW*)a.swd : (const TW*)a.wd + (size_t)e * a.D * a.F;
    const TW* wp[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
      wp[ct] = wd + (size_t)(col0 + (wave * CT + ct) * 16 + (lane & 15)) * Ke + KL * (lane >> 4);
    typename Op<WM>::WF wf[CT][UU];
    load_w<WM, CT, UU>(wf, wp, 0);
    const int cnt = stage();
    down_compute<WM, NRT, UU, CT>(a, e, cnt, col0, shared_e, rows_out, wf, wp);
  });
}

// Slot-order choice of workgroup unit `unit`, without any barrier or vector
// memory access: units 0 .. n-1 are the experts selected by any token (the
// bit set accumulated by the router, read with uniform loads) in ascending
// id order; the shared expert's 32-row chunks follow; later units have no
// work.  Returns {expert or E (shared) or -1, first token of the shared chunk}.
__device__ int2 slot_unit(const ExpertArgs& a, int unit) {
  uint32_t mw[kMaskWords];
#pragma unroll
  for (int w = 0; w < kMaskWords; ++w) mw[w] = a.masks[w];   // all requested before the first use
  int n = 0, e = -1;
#pragma unroll
  for (int w = 0; w < kMaskWords; ++w) {
    uint32_t m = mw[w];
    const int c = __popc(m);
    if (e < 0 && unit < n + c) {
      for (int r = unit - n; r > 0; --r) m &= m - 1u;   // drop the lower set bits
      e = w * 32 + __ffs(m) - 1;
    }
    n += c;
  }
  if (e >= 0) return make_int2(e, 0);
  const int t0 = (unit - n) * kRowChunk;
  return (a.swg && t0 < a.M) ? make_int2(a.E, t0) : make_int2(-1, 0);
}

// Slots of slot-order mode (M <= kDirectMaxTokens tokens, top_k <= 16).
constexpr int kSlotOrderMaxSlots = kDirectMaxTokens * 16;

// The routed expert of slots tid, tid + blockDim.x, ... (-1 past S).  The
// address does not depend on the workgroup's expert, so kernels request it
// first and it overlaps the expert-set reads of slot_unit.
template <int NPRE>
__device__ __forceinline__ void load_route(const ExpertArgs& a, int (&rv)[NPRE]) {
#pragma unroll
  for (int j = 0; j < NPRE; ++j) {
    const int s = threadIdx.x + j * blockDim.x;
    rv[j] = s < a.S ? a.route[s] : -1;
  }
}

// Whole workgroup: the slots s (route[s] == e, rv from load_route) of routed
// expert e in ascending order into slots[] (at most one per token), the first
// kRowChunk of them also as row maps (rows_tok may be null); ends with a
// barrier; returns the count.
template <int NPRE>
__device__ int stage_slots(const ExpertArgs& a, int e, const int (&rvs)[NPRE], int* rows_out, int* rows_tok,
                           int* slots, int* wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  int base = 0;
#pragma unroll
  for (int pass = 0; pass < NPRE; ++pass) {
    const int s0 = pass * blockDim.x;
    if (s0 < a.S) {   // uniform
      const int s = s0 + tid;
      const bool hit = rvs[pass] == e;
      const uint64_t b = __ballot(hit);
      int* ws = wsum + (pass & 1) * 16;   // alternate halves: no barrier needed after the reads
      if (lane == 0) ws[wave] = __popcll(b);
      __syncthreads();
      int before = 0, tot = 0;
      for (int w = 0; w < nw; ++w) {
        const int c = ws[w];
        before += w < wave ? c : 0;
        tot += c;
      }
      if (hit) {
        const int pos = base + before + lanes_below(b);
        slots[pos] = s;
        if (pos < kRowChunk) {
          rows_out[pos] = s;
          if (rows_tok) rows_tok[pos] = s / a.k;
        }
      }
      base += tot;
    }
  }
  __syncthreads();
  return base;
}

// Grouped expert kernels.  Row maps of a chunk of at most kRowChunk rows
// (output row of Hmid / Y, source token) live in LDS:
//  - slot-order mode (route != null): workgroup (unit, column tile), unit
//    chosen by slot_unit; a routed expert's rows are its slots (token = slot /
//    k), 32 at a time; shared chunk rows are tokens t0 .. (output row S + t).
//  - work-list mode: workgroup t handles tile t of the permutation's items,
//    rows start .. start + cnt - 1 with tokens tok[row].
// CT 16-column tiles per workgroup (fp8: 2, so a workgroup streams as many
// weight bytes as a bf16 one of 1 tile).
template <int MODE, bool PK, int CT>
__global__ __launch_bounds__(64 * kExpWaves, DLLM_GU_MINBLK) void k_expert_gateup(ExpertArgs a) {
  constexpr int SM = MODE == MODE_FP8 ? MODE_BF16 : MODE;   // shared expert weights
  // 4 fragments x (gate, up) = 8 KB of weights in flight per wavefront; with
  // 16 wavefronts per CU that saturates HBM without exceeding 128 VGPRs
  constexpr int UMAX = UCap<MODE>::v / (2 * CT);
  __shared__ float red[(kExpWaves - 1) * kExpNrt * 4 * 64];
  __shared__ int rows_out[kRowChunk], rows_tok[kRowChunk];
  __shared__ int slots[kDirectMaxTokens], wsum[32];
  const int tid = threadIdx.x;
  const int tiles = a.Fmax / (16 * CT);
  if (a.route) {
    // units past the touched experts and the shared chunks exit on the expert
    // set alone, before any other load (a wavefront ends only once its loads
    // return); the routing is first needed after the first weight batch
    const int unit = blockIdx.x / tiles, col0 = (blockIdx.x % tiles) * 16 * CT;
    const int2 ch = slot_unit(a, unit);
    const int e = ch.x;
    if (e < 0) return;
    const bool sh = e == a.E;
    if (col0 >= (sh ? a.Fs : a.F)) return;
    int rv[kSlotOrderMaxSlots / (64 * kExpWaves)];
    if (!sh) load_route(a, rv);
    if (sh) {
      auto st = [&]() -> int {
        const int n = min(kRowChunk, a.M - ch.y);
        if (tid < n) {
          rows_out[tid] = a.S + ch.y + tid;
          rows_tok[tid] = ch.y + tid;
        }
        __syncthreads();
        return n;
      };
      gateup_chunk<SM, UMAX, kExpNrt, false, CT>(a, e, col0, true, red, rows_out, rows_tok, st);
      return;
    }
    int cnt = 0;
    auto st0 = [&]() -> int {
      cnt = stage_slots(a, e, rv, rows_out, rows_tok, slots, wsum);
      return min(cnt, kRowChunk);
    };
    gateup_chunk<MODE, UMAX, kExpNrt, PK, CT>(a, e, col0, false, red, rows_out, rows_tok, st0);
    for (int c0 = kRowChunk; c0 < cnt; c0 += kRowChunk) {   // heavily routed expert
      auto st = [&]() -> int {
        const int n = min(kRowChunk, cnt - c0);
        __syncthreads();
        if (tid < n) {
          rows_out[tid] = slots[c0 + tid];
          rows_tok[tid] = slots[c0 + tid] / a.k;
        }
        __syncthreads();
        return n;
      };
      gateup_chunk<MODE, UMAX, kExpNrt, PK, CT>(a, e, col0, false, red, rows_out, rows_tok, st);
    }
    return;
  }
  const int n_tiles = *a.n_items * tiles;
  for (int t = blockIdx.x; t < n_tiles; t += gridDim.x) {
    const int4 item = a.items[t / tiles];
    const int e = item.x, start = item.y, cnt = item.z;
    const bool sh = e == a.E;
    const int col0 = (t % tiles) * 16 * CT;
    if (col0 >= (sh ? a.Fs : a.F)) continue;
    auto st = [&]() -> int {
      __syncthreads();
      if (tid < cnt) {
        rows_out[tid] = start + tid;
        rows_tok[tid] = a.tok[start + tid];
      }
      __syncthreads();
      return cnt;
    };
    if (sh) gateup_chunk<SM, UMAX, kExpNrt, false, CT>(a, e, col0, true, red, rows_out, rows_tok, st);
    else gateup_chunk<MODE, UMAX, kExpNrt, PK, CT>(a, e, col0, false, red, rows_out, rows_tok, st);
  }
}

// CT 16-column tiles per wavefront (2 for bf16 and fp8: the row staging is
// paid once per 128 output columns).
template <int MODE, int CT>
__global__ __launch_bounds__(256, DLLM_DN_MINBLK) void k_expert_down(ExpertArgs a) {
  constexpr int SM = MODE == MODE_FP8 ? MODE_BF16 : MODE;
  // CT tiles share every activation fragment; batches of UCap / CT chunks keep
  // the loop within 128 VGPRs (fp8: 4 tiles, bf16: 2, f32: 1)
  constexpr int UMAX = UCap<MODE>::v / CT;
  constexpr int UMAXS = UCap<SM>::v / CT;   // shared expert (bf16 beside fp8 experts)
  __shared__ int rows_out[kRowChunk];
  __shared__ int slots[kDirectMaxTokens], wsum[32];
  const int tid = threadIdx.x;
  const int tiles = a.D / (64 * CT);
  if (a.route) {
    // surplus units exit on the expert set alone (see k_expert_gateup)
    const int unit = blockIdx.x / tiles, col0 = (blockIdx.x % tiles) * 64 * CT;
    const int2 ch = slot_unit(a, unit);
    const int e = ch.x;
    if (e < 0) return;
    int rv[kSlotOrderMaxSlots / 256];
    if (e != a.E) load_route(a, rv);
    if (e == a.E) {
      auto st = [&]() -> int {
        const int n = min(kRowChunk, a.M - ch.y);
        if (tid < n) rows_out[tid] = a.S + ch.y + tid;
        __syncthreads();
        return n;
      };
      down_chunk<SM, UMAXS, kExpNrt, CT>(a, e, col0, true, rows_out, st);
      return;
    }
    int cnt = 0;
    auto st0 = [&]() -> int {
      cnt = stage_slots(a, e, rv, rows_out, nullptr, slots, wsum);
      return min(cnt, kRowChunk);
    };
    down_chunk<MODE, UMAX, kExpNrt, CT>(a, e, col0, false, rows_out, st0);
    for (int c0 = kRowChunk; c0 < cnt; c0 += kRowChunk) {
      auto st = [&]() -> int {
        const int n = min(kRowChunk, cnt - c0);
        __syncthreads();
        if (tid < n) rows_out[tid] = slots[c0 + tid];
        __syncthreads();
        return n;
      };
      down_chunk<MODE, UMAX, kExpNrt, CT>(a, e, col0, false, rows_out, st);
    }
    return;
  }
  const int n_tiles = *a.n_items * tiles;
  for (int t = blockIdx.x; t < n_tiles; t += gridDim.x) {
    const int4 item = a.items[t / tiles];
    const int e = item.x, start = item.y, cnt = item.z;
    const bool sh = e == a.E;
    const int col0 = (t % tiles) * 64 * CT;
    auto st = [&]() -> int {
      __syncthreads();
      if (tid < cnt) rows_out[tid] = start + tid;
      __syncthreads();
      return cnt;
    };
    if (sh) down_chunk<SM, UMAXS, kExpNrt, CT>(a, e, col0, true, rows_out, st);
    else down_chunk<MODE, UMAX, kExpNrt, CT>(a, e, col0, false, rows_out, st);
  }
}

// ---------------------------------------------------------------------------
// Work-list expert kernels (passes of more than kDirectMaxTokens tokens:
// batched steps, prefill).  Each wavefront owns its output columns over the
// whole reduction, so no partial sums cross wavefronts; the item's input rows
// are gathered into LDS one reduction stage at a time and shared by the
// wavefronts; an fp8 weight fragment is widened to bf16 once for all row
// tiles.  A stage's weight batch is requested before the rows are staged, so
// both loads are in flight together.
// ---------------------------------------------------------------------------

constexpr int kWlWaves = 4;                   // wavefronts per workgroup
#ifndef DLLM_WL_MINBLK
#define DLLM_WL_MINBLK 2                          // workgroups per CU the register budget allows
#endif
#ifndef DLLM_WL_ROWS
#define DLLM_WL_ROWS 64
#endif
#ifndef DLLM_WL_KS
#define DLLM_WL_KS 128
#endif
constexpr int kWlRows = DLLM_WL_ROWS;         // rows of a work item (16-row MFMA tiles: kWlRows / 16)
constexpr int kWlStage = DLLM_WL_KS;          // reduction elements per stage (fp8: 2 x 64, bf16: 4 x 32)
// Narrow column blocks: more, shorter workgroups per item.  At the batched
// step (about 16 rows per expert) the kernels stream weights at a rate per
// workgroup that does not grow with its width, so a launch is done when its
// last workgroup is; measured at 512 rows x 256 experts (fp8): gate/up 108 ->
// 89 us going from 2 to 1 tiles per wavefront, down 69 -> 62 us going from 4
// to 2 tiles with 4 workgroups per CU, then 56.8 -> 55.1 us with 1 tile and
// up to 8 workgroups per CU (items longest first).
#ifndef DLLM_WL_GU_CT
#define DLLM_WL_GU_CT 1
#endif
#ifndef DLLM_WL_DN_CT
#define DLLM_WL_DN_CT 1
#endif
#ifndef DLLM_WL_GU_MINBLK
#define DLLM_WL_GU_MINBLK DLLM_WL_MINBLK
#endif
#ifndef DLLM_WL_DN_MINBLK
#define DLLM_WL_DN_MINBLK 6
#endif
#ifndef DLLM_WL_DN_DB
#define DLLM_WL_DN_DB 0
#endif
constexpr int kWlGuCt = DLLM_WL_GU_CT;        // 16-column tiles of gate (and of up) per wavefront
constexpr int kWlDnCt = DLLM_WL_DN_CT;        // 16-column tiles per wavefront, down projection
constexpr int kWlPitch = kWlStage * 2 + 16;   // LDS bytes per staged row

// A weight fragment as MFMA operands: bf16 one 16x16x32 operand, fp8 two
// (elements 0..7 and 8..15 of each lane's 16, widened exactly).
template <int WM> struct WideW;
template <> struct WideW<MODE_BF16> { bf16x8 w0; };
template <> struct WideW<MODE_FP8> { bf16x8 w0, w1; };
template <int WM> __device__ __forceinline__ WideW<WM> widen_w(const uint4& w);
template <> __device__ __forceinline__ WideW<MODE_BF16> widen_w<MODE_BF16>(const uint4& w) {
  return {__builtin_bit_cast(bf16x8, w)};
}
template <> __device__ __forceinline__ WideW<MODE_FP8> widen_w<MODE_FP8>(const uint4& w) {
  return {Op<MODE_FP8>::widen(make_uint2(w.x, w.y)), Op<MODE_FP8>::widen(make_uint2(w.z, w.w))};
}

// The matching activation fragment from a staged LDS row at chunk element
// offset kk: lane l reads KL elements at kk + KL (l / 16).
template <int WM> struct ARow;
template <> struct ARow<MODE_BF16> { bf16x8 a0; };
template <> struct ARow<MODE_FP8> { bf16x8 a0, a1; };
template <int WM> __device__ __forceinline__ ARow<WM> lds_arow(const uint8_t* row, int kk);
template <> __device__ __forceinline__ ARow<MODE_BF16> lds_arow<MODE_BF16>(const uint8_t* row, int kk) {
  const int lane = threadIdx.x & 63;
  return {__builtin_bit_cast(bf16x8, *(const uint4*)(row + (kk + 8 * (lane >> 4)) * 2))};
}
template <> __device__ __forceinline__ ARow<MODE_FP8> lds_arow<MODE_FP8>(const uint8_t* row, int kk) {
  const int lane = threadIdx.x & 63;
  const uint8_t* p = row + (kk + 16 * (lane >> 4)) * 2;
  return {__builtin_bit_cast(bf16x8, *(const uint4*)p), __builtin_bit_cast(bf16x8, *(const uint4*)(p + 16))};
}
__device__ __forceinline__ void mma_aw(f32x4& c, const ARow<MODE_BF16>& a, const WideW<MODE_BF16>& w) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.a0, w.w0, c, 0, 0, 0);
}
__device__ __forceinline__ void mma_aw(f32x4& c, const ARow<MODE_FP8>& a, const WideW<MODE_FP8>& w) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.a0, w.w0, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.a1, w.w1, c, 0, 0, 0);
}

// acc[m][rt] += rows (cnt <= kWlRows: row r is A[a_rows[r] * lda ...]) x W_m^T over
// K reduction elements, for the NM 16-column weight tiles of this wavefront:
// tile m's lane element offset is lo (32 bits) from base wb[m], chunk c at
// + c cs elements (row-major: cs = KC, packed fragments: 64 KL).  Uses `sa`
// (two slots of kWlRows rows x kWlPitch bytes of LDS; DB: two stages in
// flight, else one).
template <int WM, int NM, bool DB>
__device__ void wl_mma_rows(f32x4 (&acc)[NM][kWlRows / 16], const uint16_t* __restrict__ A, int lda,
                            const int* a_rows, int cnt, int K, const typename Op<WM>::TW* const (&wb)[NM],
                            uint32_t lo, int cs, uint8_t* sa) {
  constexpr int KC = Op<WM>::KC, U = kWlStage / KC, NRT = kWlRows / 16;
  constexpr int SEGS = kWlStage / 8;                        // 16-byte segments per staged row
  constexpr int LPT = kWlRows * SEGS / (64 * kWlWaves);     // staging loads per thread
  constexpr int RSTEP = 64 * kWlWaves / SEGS;               // rows between a thread's segments
  constexpr int SLOT = kWlRows * kWlPitch;                  // LDS bytes of one staged stage
  static_assert(U >= 1 && LPT >= 1 && (64 * kWlWaves) % SEGS == 0, "stage shape");
  typedef typename Op<WM>::WF WF;
  const int lane = threadIdx.x & 63, tid = threadIdx.x;
  const int nrt = (cnt + 15) >> 4;
  const int seg = tid % SEGS, r0 = tid / SEGS;
  const int nst = K / kWlStage;
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) acc[m][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto fetch_rows = [&](uint4 (&st)[LPT], int s) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int r = r0 + i * RSTEP;
      st[i] = r < cnt ? *(const uint4*)(A + (size_t)a_rows[r] * lda + s * kWlStage + seg * 8)
                      : make_uint4(0, 0, 0, 0);
    }
  };
  auto put_rows = [&](const uint4 (&st)[LPT], int s) {
    uint8_t* slot = sa + (s & 1) * SLOT;
#pragma unroll
    for (int i = 0; i < LPT; ++i) *(uint4*)(slot + (r0 + i * RSTEP) * kWlPitch + seg * 16) = st[i];
  };
  auto compute = [&](const WF (&wf)[NM][U], int s) {
    const uint8_t* ar = sa + (s & 1) * SLOT + (lane & 15) * kWlPitch;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      WideW<WM> w[NM];
#pragma unroll
      for (int m = 0; m < NM; ++m) w[m] = widen_w<WM>(wf[m][u]);
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        if (rt < nrt) {
          const ARow<WM> a = lds_arow<WM>(ar + rt * 16 * kWlPitch, u * KC);
#pragma unroll
          for (int m = 0; m < NM; ++m) mma_aw(acc[m][rt], a, w[m]);
        }
      }
    }
  };
  if constexpr (!DB) {
    // one stage at a time: its weight batch, then its rows through LDS
    for (int s = 0; s < nst; ++s) {
      WF wf[NM][U];
      load_wc<WM, NM, U>(wf, wb, lo, s * U, cs);
      uint4 st[LPT];
      fetch_rows(st, s);
      __syncthreads();   // the previous stage is no longer read
      put_rows(st, 0);
      __syncthreads();
      compute(wf, 0);
    }
    return;
  }
  // Two stages in flight: before stage s is multiplied, the rows and then the
  // weights of stage s + 1 are requested (vector loads retire in order, so
  // waiting for the rows later does not wait for those weights); scheduling
  // barriers keep the compiler from sinking the requests below the products.
  WF wa[NM][U], wn[NM][U];
  {
    uint4 st[LPT];
    fetch_rows(st, 0);
    load_wc<WM, NM, U>(wa, wb, lo, 0, cs);
    put_rows(st, 0);
    __syncthreads();
  }
  for (int s = 0; s < nst; s += 2) {
    {
      uint4 st[LPT];
      const bool more = s + 1 < nst;
      if (more) {
        fetch_rows(st, s + 1);
        load_wc<WM, NM, U>(wn, wb, lo, (s + 1) * U, cs);
      }
      __builtin_amdgcn_sched_barrier(0);
      compute(wa, s);
      __builtin_amdgcn_sched_barrier(0);
      if (more) put_rows(st, s + 1);
      __syncthreads();
      if (!more) break;
    }
    {
      uint4 st[LPT];
      const bool more = s + 2 < nst;
      if (more) {
        fetch_rows(st, s + 2);
        load_wc<WM, NM, U>(wa, wb, lo, (s + 2) * U, cs);
      }
      __builtin_amdgcn_sched_barrier(0);
      compute(wn, s + 1);
      __builtin_amdgcn_sched_barrier(0);
      if (more) put_rows(st, s + 2);
      __syncthreads();
    }
  }
}

// Gate/up + SwiGLU of one item (expert e, cnt rows: input tokens tok_s[],
// output rows out_s[] of Hmid) for the columns col0 .. col0 + 16 CT waves - 1
// of gate and of up (wavefront w owns tiles col0/16 + CT w + ct).
template <int WM, bool PK>
__device__ void wl_gateup(const ExpertArgs& a, int e, bool shared_e, int cnt, int col0, const int* tok_s,
                          const int* out_s, uint8_t* sa) {
  typedef typename Op<WM>::TW TW;
  constexpr int KC = Op<WM>::KC, KL = Op<WM>::KL, CT = kWlGuCt, NM = 2 * CT;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int D = a.D;
  const int Fe = shared_e ? a.Fs : a.F;
  const TW* wg = shared_e ? (const TW*)a.swg : (const TW*)a.wg + (size_t)e * a.F * D;
  const TW* wu = shared_e ? (const TW*)a.swu : (const TW*)a.wu + (size_t)e * a.F * D;
  const int t0 = (col0 >> 4) + wave * CT;          // first 16-column tile of this wavefront
  const int ntile = Fe >> 4;
  const TW* wb[NM];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    // a tile past the width reads tile 0 (its results are not stored)
    const int t = t0 + ct < ntile ? t0 + ct : 0;
    const size_t off = PK ? (size_t)t * (D / KC) * 64 * KL : (size_t)16 * t * D;
    wb[2 * ct] = wg + off;
    wb[2 * ct + 1] = wu + off;
  }
  const uint32_t lo = PK ? (uint32_t)(lane * KL) : (uint32_t)((lane & 15) * D + KL * (lane >> 4));
  const int cs = PK ? 64 * KL : KC;
  f32x4 acc[NM][kWlRows / 16];
  wl_mma_rows<WM, NM, true>(acc, (const uint16_t*)a.X, D, tok_s, cnt, D, wb, lo, cs, sa);
  uint16_t* Hm = (uint16_t*)a.Hmid;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int col = 16 * (t0 + ct) + (lane & 15);
    if (t0 + ct >= ntile) continue;
    float sg = 1.f, su = 1.f;
    if (WM == MODE_FP8) {
      sg = a.sg[(size_t)e * a.F + col];
      su = a.su[(size_t)e * a.F + col];
    }
#pragma unroll
    for (int rt = 0; rt < kWlRows / 16; ++rt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int rr = rt * 16 + 4 * (lane >> 4) + v;
        if (rr < cnt) {
          const float g = acc[2 * ct][rt][v] * sg, u = acc[2 * ct + 1][rt][v] * su;
          Hm[(size_t)out_s[rr] * a.Fmax + col] = f2bf(g / (1.0f + expf(-g)) * u);
        }
      }
  }
}

// Down projection of one item: Y[out_s[r]] = gate(r) (Hmid[out_s[r]] W_d^T) for
// the output columns col0 .. col0 + 16 CT waves - 1.
template <int WM>
__device__ void wl_down(const ExpertArgs& a, int e, bool shared_e, int cnt, int col0, const int* out_s,
                        uint8_t* sa) {
  typedef typename Op<WM>::TW TW;
  constexpr int KC = Op<WM>::KC, KL = Op<WM>::KL, CT = kWlDnCt;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int D = a.D;
  const int Ke = shared_e ? a.Fs : a.F;
  const TW* wd = shared_e ? (const TW*)a.swd : (const TW*)a.wd + (size_t)e * D * a.F;
  const int t0 = (col0 >> 4) + wave * CT;
  const TW* wb[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) wb[ct] = wd + (size_t)16 * (t0 + ct) * Ke;
  const uint32_t lo = (uint32_t)((lane & 15) * Ke + KL * (lane >> 4));
  f32x4 acc[CT][kWlRows / 16];
  wl_mma_rows<WM, CT, DLLM_WL_DN_DB != 0>(acc, (const uint16_t*)a.Hmid, a.Fmax, out_s, cnt, Ke, wb, lo, KC, sa);
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int col = 16 * (t0 + ct) + (lane & 15);
    const float sd = WM == MODE_FP8 ? a.sd[(size_t)e * D + col] : 1.f;
#pragma unroll
    for (int rt = 0; rt < kWlRows / 16; ++rt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int rr = rt * 16 + 4 * (lane >> 4) + v;
        if (rr < cnt) {
          const int row = out_s[rr];
          const float gt = shared_e ? 1.f : a.gate_rows[row];
          st1<uint16_t>((uint16_t*)a.Y + (size_t)row * D + col, acc[ct][rt][v] * sd * gt);
        }
      }
  }
}

#ifndef DLLM_WL_XCD_ROWS
#define DLLM_WL_XCD_ROWS 2048
#endif
constexpr int kWlXcdRows = DLLM_WL_XCD_ROWS;   // token rows from which items are dealt per XCD

// Work-list unit of workgroup t: item and column block; false past the list.
// Workgroups are dealt to the 8 XCDs in turn (t to XCD t % 8).  For passes of
// kWlXcdRows token rows or more (prefill), the items go to the XCDs in turn as
// well (item i to XCD i % 8, in list order on each): the B column blocks of an
// item run on one XCD and its L2 fetches the item's rows once, and every XCD
// gets the same mix of long and short items.  Otherwise (the denoising step,
// where items are short and the weights dominate), and when the grid is too
// small for that layout, workgroup t takes item t / B, column block t % B.
__device__ __forceinline__ bool wl_unit(int t, int n_items, int B, int rows, int& item, int& cb) {
  if (rows >= kWlXcdRows && 8 * B * ((n_items + 7) / 8) <= (int)gridDim.x) {
    const int x = t & 7, k = t >> 3;
    item = x + 8 * (k / B);
    cb = k % B;
  } else {
    item = t / B;
    cb = t % B;
  }
  return item < n_items;
}

template <int MODE, bool PK>
__global__ __launch_bounds__(64 * kWlWaves, DLLM_WL_GU_MINBLK) void k_expert_gateup_wl(ExpertArgs a) {
  constexpr int SM = MODE_BF16;   // shared expert weights
  __shared__ __align__(16) uint8_t sa[2 * kWlRows * kWlPitch];
  __shared__ int tok_s[kWlRows], out_s[kWlRows];
  const int cols = 16 * kWlGuCt * kWlWaves;
  const int blocks = (a.Fmax + cols - 1) / cols;
  int it, cb;
  if (!wl_unit(blockIdx.x, *a.n_items, blocks, a.M, it, cb)) return;
  const int4 item = a.items[it];
  const int e = item.x, start = item.y, cnt = item.z;
  const bool sh = e == a.E;
  const int col0 = cb * cols;
  if (col0 >= (sh ? a.Fs : a.F)) return;
  if (threadIdx.x < cnt) {
    out_s[threadIdx.x] = start + threadIdx.x;
    tok_s[threadIdx.x] = a.tok[start + threadIdx.x];
  }
  __syncthreads();
  if (sh) wl_gateup<SM, false>(a, e, true, cnt, col0, tok_s, out_s, sa);
  else wl_gateup<MODE, PK>(a, e, false, cnt, col0, tok_s, out_s, sa);
}

template <int MODE>
__global__ __launch_bounds__(64 * kWlWaves, DLLM_WL_DN_MINBLK) void k_expert_down_wl(ExpertArgs a) {
  constexpr int SM = MODE_BF16;
  // one staging slot unless the stages are double-buffered
  __shared__ __align__(16) uint8_t sa[(DLLM_WL_DN_DB ? 2 : 1) * kWlRows * kWlPitch];
  __shared__ int out_s[kWlRows];
  const int cols = 16 * kWlDnCt * kWlWaves;
  const int blocks = a.D / cols;
  int it, cb;
  if (!wl_unit(blockIdx.x, *a.n_items, blocks, a.M, it, cb)) return;
  const int4 item = a.items[it];
  const int e = item.x, start = item.y, cnt = item.z;
  const bool sh = e == a.E;
  if (threadIdx.x < cnt) out_s[threadIdx.x] = start + threadIdx.x;
  __syncthreads();
  if (sh) wl_down<SM>(a, e, true, cnt, cb * cols, out_s, sa);
  else wl_down<MODE>(a, e, false, cnt, cb * cols, out_s, sa);
}

// Shapes the work-list kernels cover: bf16 activations (bf16 or fp8 experts),
// hidden size and expert widths in whole stages and column blocks.
static bool wl_ok(int mode, int D, int F, int Fs) {
  if (mode == MODE_F32) return false;
  return D % kWlStage == 0 && F % kWlStage == 0 && Fs % kWlStage == 0 && D % (16 * kWlDnCt * kWlWaves) == 0 &&
         F % 16 == 0 && Fs % 16 == 0;
}

int expert_item_rows(int mode, int D, int F, int Fs) { return wl_ok(mode, D, F, Fs) ? kWlRows : kRowChunk; }

// Workgroup units: slot-order mode min(E, S) routed-expert bound + the shared
// expert's 32-row chunks; work-list mode max_items (units past the device item
// count exit at once).
static int expert_units(const ExpertArgs& a, int max_items) {
  if (!a.route) return max_items;
  return (a.E < a.S ? a.E : a.S) + (a.swg ? (a.M + kRowChunk - 1) / kRowChunk : 0);
}

hipError_t launch_expert_gateup(int mode, const ExpertArgs& a, int max_items, hipStream_t s) {
  const int units = expert_units(a, max_items);
  if (units == 0) return hipSuccess;
  if (!a.route && wl_ok(mode, a.D, a.F, a.Fs)) {
    const int cols = 16 * kWlGuCt * kWlWaves;
    dim3 g((unsigned)(max_items * ((a.Fmax + cols - 1) / cols)));
    auto go = [&](auto pk) {
      constexpr bool PK = decltype(pk)::value;
      if (mode == MODE_BF16) hipLaunchKernelGGL((k_expert_gateup_wl<MODE_BF16, PK>), g, dim3(64 * kWlWaves), 0, s, a);
      else hipLaunchKernelGGL((k_expert_gateup_wl<MODE_FP8, PK>), g, dim3(64 * kWlWaves), 0, s, a);
    };
    if (a.gu_packed) go(std::true_type{});
    else go(std::false_type{});
    return hipGetLastError();
  }
  const int ct = mode == MODE_FP8 ? DLLM_GU_CT_FP8 : 1;   // column tiles per workgroup
  dim3 g1(units * (a.Fmax / (16 * ct)));
  dim3 b1(64 * kExpWaves);
  auto go = [&](auto pk) {
    constexpr bool PK = decltype(pk)::value;
    if (mode == MODE_F32) hipLaunchKernelGGL((k_expert_gateup<MODE_F32, PK, 1>), g1, b1, 0, s, a);
    else if (mode == MODE_BF16) hipLaunchKernelGGL((k_expert_gateup<MODE_BF16, PK, 1>), g1, b1, 0, s, a);
    else hipLaunchKernelGGL((k_expert_gateup<MODE_FP8, PK, DLLM_GU_CT_FP8>), g1, b1, 0, s, a);
  };
  if (a.gu_packed) go(std::true_type{});
  else go(std::false_type{});
  return hipGetLastError();
}

hipError_t launch_expert_down(int mode, const ExpertArgs& a, int max_items, hipStream_t s) {
  const int units = expert_units(a, max_items);
  if (units == 0) return hipSuccess;
  if (!a.route && wl_ok(mode, a.D, a.F, a.Fs)) {
    dim3 g((unsigned)(max_items * (a.D / (16 * kWlDnCt * kWlWaves))));
    if (mode == MODE_BF16) hipLaunchKernelGGL((k_expert_down_wl<MODE_BF16>), g, dim3(64 * kWlWaves), 0, s, a);
    else hipLaunchKernelGGL((k_expert_down_wl<MODE_FP8>), g, dim3(64 * kWlWaves), 0, s, a);
    return hipGetLastError();
  }
  if (mode == MODE_F32) hipLaunchKernelGGL((k_expert_down<MODE_F32, 1>), dim3(units * (a.D / 64)), dim3(256), 0, s, a);
  else if (mode == MODE_BF16) hipLaunchKernelGGL((k_expert_down<MODE_BF16, 2>), dim3(units * (a.D / 128)), dim3(256), 0, s, a);
  // fp8: 4 output tiles per wavefront (a workgroup's weight bytes match the bf16 kernel's 2 tiles)
  else hipLaunchKernelGGL((k_expert_down<MODE_FP8, DLLM_DN_CT_FP8>), dim3(units * (a.D / (64 * DLLM_DN_CT_FP8))), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Masked positions -> LM-head rows (standalone launch of mask_list_block).
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(1024) void k_mask_list(const int32_t* __restrict__ ids, int n_seq, int LB,
                                                    int mask_id, int gm, int32_t* __restrict__ row_map,
                                                    int32_t* __restrict__ entry_pos, int32_t* __restrict__ seq_off,
                                                    int32_t* __restrict__ n_rows, int32_t* __restrict__ n_entries) {
  __shared__ int tmp[32];
  mask_list_block(ids, n_seq, LB, mask_id, gm, row_map, entry_pos, seq_off, n_rows, n_entries, tmp);
}

hipError_t launch_mask_list(const int32_t* ids, int n_seq, int LB, int mask_id, int gm, int32_t* row_map,
                            int32_t* entry_pos, int32_t* seq_off, int32_t* n_rows, int32_t* n_entries,
                            hipStream_t s) {
  hipLaunchKernelGGL(k_mask_list, dim3(1), dim3(1024), 0, s, ids, n_seq, LB, mask_id, gm, row_map,
                     entry_pos, seq_off, n_rows, n_entries);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Confidence.  Partials over kHeadCols columns: (max, argmax, second max,
// sum exp(l - max), sum exp(l - max) (l - max)); CFG mixes the (cond,
// uncond) logits first.  The merge combines partials in column order.
// ---------------------------------------------------------------------------

struct Top2 {
  float m1;
  int i1;
  float m2;
};

__device__ __forceinline__ Top2 top2_merge(Top2 a, Top2 b) {
  Top2 r;
  if (b.m1 > a.m1 || (b.m1 == a.m1 && b.i1 < a.i1)) {
    r.m1 = b.m1;
    r.i1 = b.i1;
    r.m2 = fmaxf(a.m1, b.m2);
  } else {
    r.m1 = a.m1;
    r.i1 = a.i1;
    r.m2 = fmaxf(a.m2, b.m1);
  }
  return r;
}

__global__ __launch_bounds__(256) void k_conf_partial(const float* __restrict__ logits,
                                                      const int32_t* __restrict__ n_entries,
                                                      const int32_t* __restrict__ row_of_entry, int V,
                                                      int cfg, float cfg_scale, float* __restrict__ part) {
  __shared__ float sm1[4], sm2[4];
  __shared__ int si1[4];
  __shared__ float tmp[16];
  const int ent = blockIdx.y;
  if (ent >= *n_entries) return;
  const int tile = blockIdx.x;
  const int c = tile * kHeadCols + threadIdx.x;
  const int row = row_of_entry ? row_of_entry[ent] : ent;
  float l = -INFINITY;
  if (c < V) {
    if (cfg) {
      const float lc = logits[(size_t)(2 * row) * V + c];
      const float lu = logits[(size_t)(2 * row + 1) * V + c];
      l = lu + cfg_scale * (lc - lu);
    } else {
      l = logits[(size_t)row * V + c];
    }
  }
  Top2 t{l, c < V ? c : 0x7fffffff, -INFINITY};
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    Top2 u{__shfl_xor(t.m1, o, 64), __shfl_xor(t.i1, o, 64), __shfl_xor(t.m2, o, 64)};
    t = top2_merge(t, u);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    sm1[wave] = t.m1;
    si1[wave] = t.i1;
    sm2[wave] = t.m2;
  }
  __syncthreads();
  Top2 b{sm1[0], si1[0], sm2[0]};
  for (int w = 1; w < 4; ++w) b = top2_merge(b, Top2{sm1[w], si1[w], sm2[w]});
  const float e = (c < V) ? expf(l - b.m1) : 0.f;
  const float s1 = block_sum(e, tmp);
  const float s2 = block_sum((c < V) ? e * (l - b.m1) : 0.f, tmp);
  if (threadIdx.x == 0) {
    float* p = part + ((size_t)ent * gridDim.x + tile) * 5;
    p[0] = b.m1;
    p[1] = __int_as_float(b.i1);
    p[2] = b.m2;
    p[3] = s1;
    p[4] = s2;
  }
}

hipError_t launch_conf_partial(const float* logits, const int32_t* n_entries, const int32_t* row_of_entry,
                               int max_entries, int V, int cfg, float cfg_scale, float* part,
                               hipStream_t s) {
  if (max_entries == 0) return hipSuccess;
  dim3 grid((V + kHeadCols - 1) / kHeadCols, max_entries);
  hipLaunchKernelGGL(k_conf_partial, grid, dim3(kHeadCols), 0, s, logits, n_entries, row_of_entry, V, cfg,
                     cfg_scale, part);
  return hipGetLastError();
}

__global__ __launch_bounds__(64) void k_conf_merge(const float* __restrict__ part,
                                                   const int32_t* __restrict__ n_entries, int ntiles,
                                                   int vocab_lo, const int32_t* __restrict__ entry_pos,
                                                   int strategy, float* __restrict__ conf,
                                                   int32_t* __restrict__ xhat) {
  const int ent = blockIdx.x;
  if (ent >= *n_entries) return;
  const int lane = threadIdx.x;
  // each lane merges tiles lane, lane+64, ... in order; then a fixed butterfly
  Top2 t{-INFINITY, 0x7fffffff, -INFINITY};
  float M = -INFINITY;
  for (int i = lane; i < ntiles; i += 64) {
    const float* p = part + ((size_t)ent * ntiles + i) * 5;
    t = top2_merge(t, Top2{p[0], __float_as_int(p[1]), p[2]});
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    Top2 u{__shfl_xor(t.m1, o, 64), __shfl_xor(t.i1, o, 64), __shfl_xor(t.m2, o, 64)};
    t = top2_merge(t, u);
  }
  M = t.m1;
  float s1 = 0.f, s2 = 0.f;
  for (int i = lane; i < ntiles; i += 64) {
    const float* p = part + ((size_t)ent * ntiles + i) * 5;
    const float w = expf(p[0] - M);
    s1 += w * p[3];
    s2 += w * (p[4] + (p[0] - M) * p[3]);
  }
  s1 = wave_sum(s1);
  s2 = wave_sum(s2);
  if (lane == 0) {
    float c;
    if (strategy == 0) c = 1.0f / s1;
    else if (strategy == 1) c = (1.0f - expf(t.m2 - M)) / s1;
    else c = s2 / s1 - logf(s1);
    const int pos = entry_pos[ent];
    conf[pos] = c;
    xhat[pos] = vocab_lo + t.i1;
  }
}

hipError_t launch_conf_merge(const float* part, const int32_t* n_entries, int max_entries, int V,
                             int vocab_lo, const int32_t* entry_pos, int strategy, float* conf,
                             int32_t* xhat, int n_pos, hipStream_t s) {
  (void)n_pos;
  if (max_entries == 0) return hipSuccess;
  const int ntiles = (V + kHeadCols - 1) / kHeadCols;
  hipLaunchKernelGGL(k_conf_merge, dim3(max_entries), dim3(64), 0, s, part, n_entries, ntiles, vocab_lo,
                     entry_pos, strategy, conf, xhat);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// LM head over the masked rows with the confidence partials fused into the
// epilogue: each workgroup computes 16 vocabulary columns for up to 16 * NRT
// head rows and reduces, per entry (one row, a CFG pair mixed with gs_a, or
// a three-way group mixed as l_u + gs_a (l_img - l_u) + gs_b (l_full - l_img)), the partial
// (max, argmax, 2nd max, sum exp(l - max), sum exp(l - max)(l - max)) over its
// columns.  Logits never leave registers.  part: [entry][ntiles][5].
// row_map null: head row r is X row r; n_rows_dev null: max_rows rows.
// ---------------------------------------------------------------------------

template <int MODE, int NRT, int U>
__global__ __launch_bounds__(64 * kGemmWaves, NRT >= 4 ? 2 : 4) void k_head_conf(
    const typename Op<MODE>::TA* __restrict__ X, int D, const int32_t* __restrict__ row_map,
    const int32_t* __restrict__ n_rows_dev, int max_rows, const typename Op<MODE>::TW* __restrict__ W, int V, int gm,
    float gs_a, float gs_b, float* __restrict__ part) {
  typedef typename Op<MODE>::TA TA;
  typedef typename Op<MODE>::TW TW;
  __shared__ float red[(kGemmWaves - 1) * NRT * 4 * 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int M = n_rows_dev ? *n_rows_dev : max_rows;
  const int row0 = blockIdx.y * 16 * NRT;
  if (row0 >= M) return;
  const int tile = blockIdx.x, ntiles = gridDim.x;
  const int col = tile * 16 + (lane & 15);
  const TW* wp[1] = {W + (size_t)min(col, V - 1) * D + 8 * (lane >> 4)};
  const TA* ap[NRT];
  bool av[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const int r = row0 + rt * 16 + (lane & 15);
    av[rt] = r < M;
    ap[rt] = X + (size_t)(av[rt] ? (row_map ? row_map[r] : r) : 0) * D + 8 * (lane >> 4);
  }
  f32x4 acc[1][NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) acc[0][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int kper = D / kGemmWaves;
  if constexpr (MODE == MODE_BF16 && U % 2 == 0) {
    __shared__ __align__(16) uint8_t wlds[kGemmWaves * 16 * (64 * U + 16)];
    const TW* wlo[1] = {W + (size_t)min(tile * 16 + (lane >> 3), V - 1) * D + 8 * (lane & 7)};
    const TW* whi[1] = {W + (size_t)min(tile * 16 + 8 + (lane >> 3), V - 1) * D + 8 * (lane & 7)};
    for (int kk = wave * kper; kk < (wave + 1) * kper; kk += 32 * U)
      mma_batch_lines<NRT, 1, U>(acc, ap, av, wlo, whi, kk, wlds + wave * 16 * (64 * U + 16));
  } else {
    for (int kk = wave * kper; kk < (wave + 1) * kper; kk += 32 * U) mma_batch<MODE, NRT, 1, U>(acc, ap, av, wp, kk);
  }
  reduce_waves<NRT, kGemmWaves>(acc[0], red);
  if (wave != 0) return;
  const bool cvalid = col < V;
  const int npv = gm == 2 ? 1 : (gm == 1 ? 2 : 4);   // entries per 4 accumulator rows
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    if (row0 + rt * 16 < M) {   // uniform: tiles without rows are skipped
      // entries of rows 4 g + v: the reductions over the 16 columns held by the
      // lanes with the same (lane >> 4) run interleaved across entries
      float l[4];
      int row[4];
      Top2 t[4];
#pragma unroll
      for (int pv = 0; pv < 4; ++pv) {
        if (gm == 2) {
          const float lf = acc[0][rt][0], li = acc[0][rt][1], lu = acc[0][rt][2];
          l[pv] = lu + gs_a * (li - lu) + gs_b * (lf - li);
          row[pv] = row0 + rt * 16 + 4 * (lane >> 4);
        } else if (gm == 1) {
          const float lc = acc[0][rt][2 * (pv & 1)], lu = acc[0][rt][2 * (pv & 1) + 1];
          l[pv] = lu + gs_a * (lc - lu);
          row[pv] = row0 + rt * 16 + 4 * (lane >> 4) + 2 * (pv & 1);
        } else {
          l[pv] = acc[0][rt][pv];
          row[pv] = row0 + rt * 16 + 4 * (lane >> 4) + pv;
        }
        if (!cvalid) l[pv] = -INFINITY;
        t[pv] = Top2{l[pv], cvalid ? col : 0x7fffffff, -INFINITY};
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1)
#pragma unroll
        for (int pv = 0; pv < 4; ++pv) {
          Top2 u{__shfl_xor(t[pv].m1, o, 64), __shfl_xor(t[pv].i1, o, 64), __shfl_xor(t[pv].m2, o, 64)};
          t[pv] = top2_merge(t[pv], u);
        }
      float s1[4], s2[4];
#pragma unroll
      for (int pv = 0; pv < 4; ++pv) {
        const float e = cvalid ? expf(l[pv] - t[pv].m1) : 0.f;
        s1[pv] = e;
        s2[pv] = cvalid ? e * (l[pv] - t[pv].m1) : 0.f;
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1)
#pragma unroll
        for (int pv = 0; pv < 4; ++pv) {
          s1[pv] += __shfl_xor(s1[pv], o, 64);
          s2[pv] += __shfl_xor(s2[pv], o, 64);
        }
      if ((lane & 15) == 0)
#pragma unroll
        for (int pv = 0; pv < 4; ++pv)
          if (pv < npv && row[pv] < M) {
            const int ent = gm == 2 ? row[pv] >> 2 : (gm == 1 ? row[pv] >> 1 : row[pv]);
            float* p = part + ((size_t)ent * ntiles + tile) * 5;
            p[0] = t[pv].m1;
            p[1] = __int_as_float(t[pv].i1);
            p[2] = t[pv].m2;
            p[3] = s1[pv];
            p[4] = s2[pv];
          }
    }
  }
}

template <int MODE, int NRT, int U>
static void head_launch_one(dim3 grid, const void* X, int D, const int32_t* row_map, const int32_t* n_rows,
                            int max_rows, const void* W, int V, int gm, float gs_a, float gs_b, float* part,
                            hipStream_t s) {
  typedef typename Op<MODE>::TA TA;
  typedef typename Op<MODE>::TW TW;
  hipLaunchKernelGGL((k_head_conf<MODE, NRT, U>), grid, dim3(64 * kGemmWaves), 0, s, (const TA*)X, D, row_map, n_rows,
                     max_rows, (const TW*)W, V, gm, gs_a, gs_b, part);
}

hipError_t launch_head_conf(int mode, const void* X, int D, const int32_t* row_map, const int32_t* n_rows,
                            int max_rows, const void* W, int V, int gm, float gs_a, float gs_b, float* part,
                            hipStream_t s) {
  if (max_rows == 0) return hipSuccess;
  const int nrt = max_rows <= 16 ? 1 : (max_rows <= 32 ? 2 : 4);
  dim3 grid((V + 15) / 16, (max_rows + 16 * nrt - 1) / (16 * nrt));
  const int chunks = D / (32 * kGemmWaves);
  auto go = [&](auto nrt_c) {
    constexpr int NRT = decltype(nrt_c)::value;
    if (mode == MODE_F32)
      pick_u<(NRT <= 2 ? 4 : 1)>(chunks, [&](auto u) {
        head_launch_one<MODE_F32, NRT, decltype(u)::value>(grid, X, D, row_map, n_rows, max_rows, W, V, gm, gs_a,
                                                           gs_b, part, s);
      });
    else   // whole-line path: batches of 2 chunks (measured best of 2, 4 and 8)
      pick_u<(NRT <= 2 ? 2 : 1)>(chunks, [&](auto u) {
        head_launch_one<MODE_BF16, NRT, decltype(u)::value>(grid, X, D, row_map, n_rows, max_rows, W, V, gm, gs_a,
                                                            gs_b, part, s);
      });
  };
  if (nrt == 1) go(IC<1>{});
  else if (nrt == 2) go(IC<2>{});
  else go(IC<4>{});
  return hipGetLastError();
}

// LM head of a pass with many head rows (a batch of sequences, or the
// prefix-confidence pass of an append): the LDS-tiled GEMM over BM head rows
// (gathered through row_map) x 128 vocabulary columns, so every weight row
// streams once per BM head rows instead of once per 16 * NRT, then the same
// confidence partials as k_head_conf over the tile's 128 columns.  Launch
// order: only the row tiles that hold head rows (n_rows of max_rows) take
// workgroups, from the front of the grid; the surplus workgroups at the end
// exit at once (spread through the grid they cost as much as real tiles).
// The row tiles of one column tile take consecutive workgroups, which the
// dispatcher deals to different XCDs: they run together and the weight tile
// streams from HBM about once (measured faster than keeping them on one XCD).
// Epilogue: S =
// 256 / (entries in the tile) threads per entry; thread s holds the guided
// logits of columns s, s + S, ... of the output tile in registers and scans
// them twice (top two, then the exponential sums); the S partial results merge
// with log2(S) exchanges.  GM (the guidance mode) fixes the rows per entry, so
// both scans unroll.  part: [entry][ceil(V / 128)][5].
#ifndef DLLM_HEAD_DEPTH
#define DLLM_HEAD_DEPTH 1   // two register sets halve the workgroups a CU holds: slower here
#endif
template <int BM, int GM>
__global__ __launch_bounds__(256) void k_head_tiled(const uint16_t* __restrict__ X, int D,
                                                    const int32_t* __restrict__ row_map,
                                                    const int32_t* __restrict__ n_rows_dev, int max_rows,
                                                    const uint16_t* __restrict__ W, int V, float gs_a, float gs_b,
                                                    float* __restrict__ part) {
  extern __shared__ __align__(16) uint8_t tile_lds[];
  constexpr int RPE = GM == 2 ? 4 : (GM == 1 ? 2 : 1);   // head rows per entry
  constexpr int S = 256 * RPE / BM;                       // threads per entry: 2 .. 16
  constexpr int NC = kTN / S;                             // columns per thread
  const int M = n_rows_dev ? min(*n_rows_dev, max_rows) : max_rows;
  if (M <= 0) return;
  const int nrt = (M + BM - 1) / BM, ntiles = (V + kTN - 1) / kTN;   // row tiles holding head rows
  const int tile = blockIdx.x / nrt;
  const int m0 = (blockIdx.x % nrt) * BM, n0 = tile * kTN;
  if (tile >= ntiles) return;   // uniform: past the live tiles
  gemm_tile_bf16<BM, kTN, DLLM_HEAD_DEPTH>(X, D, M, W, D, V, D, m0, n0, tile_lds, row_map);
  const float* t = (const float*)tile_lds;
  const int e = threadIdx.x / S, sg = threadIdx.x % S;
  const int r0 = e * RPE;
  const float* tr = t + r0 * kTileLd + sg;
  const int cend = min(kTN, V - n0);   // valid columns of this tile
  float l[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const float* p = tr + S * i;
    float x;
    if (GM == 2) {
      const float lf = p[0], li = p[kTileLd], lu = p[2 * kTileLd];
      x = lu + gs_a * (li - lu) + gs_b * (lf - li);
    } else if (GM == 1) {
      const float lc = p[0], lu = p[kTileLd];
      x = lu + gs_a * (lc - lu);
    } else {
      x = p[0];
    }
    l[i] = sg + S * i < cend ? x : -INFINITY;
  }
  Top2 tp{-INFINITY, 0x7fffffff, -INFINITY};
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    if (l[i] > tp.m1) {
      tp.m2 = tp.m1;
      tp.m1 = l[i];
      tp.i1 = n0 + sg + S * i;
    } else {
      tp.m2 = fmaxf(tp.m2, l[i]);
    }
  }
#pragma unroll
  for (int o = 1; o < S; o <<= 1) {
    Top2 u{__shfl_xor(tp.m1, o, 64), __shfl_xor(tp.i1, o, 64), __shfl_xor(tp.m2, o, 64)};
    tp = top2_merge(tp, u);
  }
  float s1 = 0.f, s2 = 0.f;
#pragma unroll
  for (int i = 0; i < NC; ++i)
    if (l[i] != -INFINITY) {
      const float d = l[i] - tp.m1;
      const float ex = expf(d);
      s1 += ex;
      s2 += ex * d;
    }
#pragma unroll
  for (int o = 1; o < S; o <<= 1) {
    s1 += __shfl_xor(s1, o, 64);
    s2 += __shfl_xor(s2, o, 64);
  }
  if (sg == 0 && m0 + r0 < M) {
    float* pp = part + ((size_t)((m0 + r0) / RPE) * ntiles + tile) * 5;
    pp[0] = tp.m1;
    pp[1] = __int_as_float(tp.i1);
    pp[2] = tp.m2;
    pp[3] = s1;
    pp[4] = s2;
  }
}

// The tiled head needs more than 32 head rows and enough 128 x 128 tiles to
// give every CU one; below that the streaming kernel has more parallelism.
bool head_tiled_ok(int mode, int max_rows, int V) {
  return mode == MODE_BF16 && max_rows > 32 && (V + kTN - 1) / kTN * ((max_rows + kTM - 1) / kTM) >= kHeadTiledMin;
}

int head_partial_tiles(int mode, int max_rows, int V) {
  return head_tiled_ok(mode, max_rows, V) ? (V + kTN - 1) / kTN : (V + 15) / 16;
}

hipError_t launch_head(int mode, const void* X, int D, const int32_t* row_map, const int32_t* n_rows, int max_rows,
                       const void* W, int V, int gm, float gs_a, float gs_b, float* part, hipStream_t s) {
  if (max_rows == 0) return hipSuccess;
  if (!head_tiled_ok(mode, max_rows, V))
    return launch_head_conf(mode, X, D, row_map, n_rows, max_rows, W, V, gm, gs_a, gs_b, part, s);
  // 128-row tiles: the two row tiles of a column tile fetch it about twice.
  // A 256-row tile of 8 wavefronts reads each vocabulary tile once but
  // measured slower (256 head rows x 157,184 ids: 272 vs 251 us): the
  // tile's loop, not HBM, sets the pace.
  const int bm = max_rows > 64 ? 128 : 64;
  dim3 grid((V + kTN - 1) / kTN * ((max_rows + bm - 1) / bm));
  auto go = [&](auto bm_c, auto gm_c) {
    constexpr int BM = decltype(bm_c)::value, GM = decltype(gm_c)::value;
    hipLaunchKernelGGL((k_head_tiled<BM, GM>), grid, dim3(256), tile_lds_bytes(BM), s, (const uint16_t*)X, D, row_map,
                       n_rows, max_rows, (const uint16_t*)W, V, gs_a, gs_b, part);
  };
  auto go_bm = [&](auto gm_c) {
    if (bm == 128) go(IC<128>{}, gm_c);
    else go(IC<64>{}, gm_c);
  };
  if (gm == 2) go_bm(IC<2>{});
  else if (gm == 1) go_bm(IC<1>{});
  else go_bm(IC<0>{});
  return hipGetLastError();
}

// Merge the confidence partials of one entry (one wavefront; lanes over tiles
// in a fixed order) into (confidence, argmax id).  Up to 64 * kConfTpl tiles
// are read once into registers (all loads in flight together) and reused by
// both passes.
constexpr int kConfTpl = 8;

__device__ __forceinline__ void conf_merge_entry(const float* __restrict__ part, int ent, int ntiles, int strategy,
                                                 float* c_out, int* i_out) {
  const int lane = threadIdx.x & 63;
  Top2 t{-INFINITY, 0x7fffffff, -INFINITY};
  float s1 = 0.f, s2 = 0.f;
  if (ntiles <= 64 * kConfTpl) {
    float q[kConfTpl][5];
#pragma unroll
    for (int j = 0; j < kConfTpl; ++j) {
      const int i = lane + 64 * j;
      if (i < ntiles) {
        const float* p = part + ((size_t)ent * ntiles + i) * 5;
#pragma unroll
        for (int f = 0; f < 5; ++f) q[j][f] = p[f];
      } else {
        q[j][0] = -INFINITY;
        q[j][1] = __int_as_float(0x7fffffff);
        q[j][2] = -INFINITY;
        q[j][3] = 0.f;
        q[j][4] = 0.f;
      }
    }
#pragma unroll
    for (int j = 0; j < kConfTpl; ++j) t = top2_merge(t, Top2{q[j][0], __float_as_int(q[j][1]), q[j][2]});
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      Top2 u{__shfl_xor(t.m1, o, 64), __shfl_xor(t.i1, o, 64), __shfl_xor(t.m2, o, 64)};
      t = top2_merge(t, u);
    }
    const float M = t.m1;
#pragma unroll
    for (int j = 0; j < kConfTpl; ++j)
      if (q[j][0] != -INFINITY) {
        const float w = expf(q[j][0] - M);
        s1 += w * q[j][3];
        s2 += w * (q[j][4] + (q[j][0] - M) * q[j][3]);
      }
  } else {
    // more tiles than registers: both passes walk the lane's tiles (lane,
    // lane + 64, ...) in the same order in chunks of kConfTpl, each chunk's
    // loads issued together
    const float* pe = part + (size_t)ent * ntiles * 5;
    for (int base = 0; base < ntiles; base += 64 * kConfTpl) {
      float q[kConfTpl][3];
#pragma unroll
      for (int j = 0; j < kConfTpl; ++j) {
        const int i = base + lane + 64 * j;
        if (i < ntiles) {
#pragma unroll
          for (int f = 0; f < 3; ++f) q[j][f] = pe[(size_t)i * 5 + f];
        } else {
          q[j][0] = -INFINITY;
          q[j][1] = __int_as_float(0x7fffffff);
          q[j][2] = -INFINITY;
        }
      }
#pragma unroll
      for (int j = 0; j < kConfTpl; ++j) t = top2_merge(t, Top2{q[j][0], __float_as_int(q[j][1]), q[j][2]});
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      Top2 u{__shfl_xor(t.m1, o, 64), __shfl_xor(t.i1, o, 64), __shfl_xor(t.m2, o, 64)};
      t = top2_merge(t, u);
    }
    const float M = t.m1;
    for (int base = 0; base < ntiles; base += 64 * kConfTpl) {
      float q[kConfTpl][3];
#pragma unroll
      for (int j = 0; j < kConfTpl; ++j) {
        const int i = base + lane + 64 * j;
        if (i < ntiles) {
          q[j][0] = pe[(size_t)i * 5];
          q[j][1] = pe[(size_t)i * 5 + 3];
          q[j][2] = pe[(size_t)i * 5 + 4];
        } else {
          q[j][0] = -INFINITY;
        }
      }
#pragma unroll
      for (int j = 0; j < kConfTpl; ++j)
        if (q[j][0] != -INFINITY) {
          const float w = expf(q[j][0] - M);
          s1 += w * q[j][1];
          s2 += w * (q[j][2] + (q[j][0] - M) * q[j][1]);
        }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {   // both sums, interleaved
    s1 += __shfl_xor(s1, o, 64);
    s2 += __shfl_xor(s2, o, 64);
  }
  const float M = t.m1;
  if (strategy == 0) *c_out = 1.0f / s1;
  else if (strategy == 1) *c_out = (1.0f - expf(t.m2 - M)) / s1;
  else *c_out = s2 / s1 - logf(s1);
  *i_out = t.i1;
}

// ---------------------------------------------------------------------------
// Commit: quota n = ceil(r / (T - t)); threshold mode n = max(n, #{c > tau});
// the n masked positions of highest confidence (ties to the lower position)
// take their argmax ids.  One wavefront per sequence, lane = block position.
// ---------------------------------------------------------------------------

// Core of the commit for one sequence: lane j < LB holds the block id at
// position j, its confidence cj and argmax id xj (read only when the position
// is [MASK]).
// ids_out may alias the block ids the caller read: each lane writes only the
// position whose id it already holds.
__device__ __forceinline__ void select_commit_vals(int s, int id, float cj, int xj, float* __restrict__ conf, int LB,
                                                   int mask_id, int steps, int t, int use_threshold, float threshold,
                                                   int32_t* ids_out, int32_t* __restrict__ remaining) {
  const int j = threadIdx.x & 63;
  const bool in = j < LB;
  const bool m = in && id == mask_id;
  const float c = m ? cj : -INFINITY;
  const int r = __popcll(__ballot(m));
  int n = 0;
  if (r > 0) {
    n = (r + (steps - t) - 1) / (steps - t);
    if (use_threshold) {
      const int above = __popcll(__ballot(m && c > threshold));
      n = max(n, above);
    }
    n = min(n, r);
  }
  // rank among the masked positions: confidences through LDS (broadcast
  // reads, no cross-lane dependency chain); masked ones only
  __shared__ float cs[64];
  cs[j] = c;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const uint64_t mb = __ballot(m);
  int rank = 0;
  for (int i = 0; i < LB; ++i) {
    const float ci = cs[i];
    if (((mb >> i) & 1ull) && (ci > c || (ci == c && i < j))) rank++;
  }
  const bool commit = m && rank < n;
  if (in) {
    ids_out[s * LB + j] = commit ? xj : id;
    if (!m) conf[s * LB + j] = -INFINITY;
  }
  if (j == 0) remaining[s] = r - n;
}

__device__ __forceinline__ void select_commit_seq(int s, const int32_t* ids_in, float* __restrict__ conf,
                                                  const int32_t* __restrict__ xhat, int LB, int mask_id, int steps,
                                                  int t, int use_threshold, float threshold,
                                                  int32_t* ids_out, int32_t* __restrict__ remaining) {
  const int j = threadIdx.x & 63;
  const bool in = j < LB;
  const int id = in ? ids_in[s * LB + j] : 0;
  const bool m = in && id == mask_id;
  select_commit_vals(s, id, m ? conf[s * LB + j] : -INFINITY, m ? xhat[s * LB + j] : 0, conf, LB, mask_id, steps, t,
                     use_threshold, threshold, ids_out, remaining);
}

__global__ __launch_bounds__(64) void k_select_commit(const int32_t* ids_in, float* __restrict__ conf,
                                                      const int32_t* __restrict__ xhat, int LB, int mask_id,
                                                      int steps, int t, int use_threshold, float threshold,
                                                      int32_t* ids_out, int32_t* __restrict__ remaining) {
  select_commit_seq(blockIdx.x, ids_in, conf, xhat, LB, mask_id, steps, t, use_threshold, threshold, ids_out,
                    remaining);
}

// Per sequence: merge the confidence partials of its masked entries (one
// wavefront per entry), then commit the quota (wavefront 0).
__global__ __launch_bounds__(1024) void k_conf_select(const float* __restrict__ part, int ntiles,
                                                     const int32_t* __restrict__ seq_off,
                                                     const int32_t* __restrict__ entry_pos, int vocab_lo, int strategy,
                                                     const int32_t* ids_in, float* __restrict__ conf,
                                                     int32_t* __restrict__ xhat, int LB, int mask_id, int steps,
                                                     int t, int use_threshold, float threshold,
                                                     int32_t* ids_out, int32_t* __restrict__ remaining) {
  const int s = blockIdx.x, wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nw = blockDim.x >> 6;
  __shared__ float sconf[64];
  __shared__ int sxhat[64];
  // the block ids for the commit, requested before the merge
  const int id = (wave == 0 && lane < LB) ? ids_in[s * LB + lane] : 0;
  const int e0 = seq_off[s], e1 = seq_off[s + 1];
  for (int ent = e0 + wave; ent < e1; ent += nw) {
    float c;
    int i;
    conf_merge_entry(part, ent, ntiles, strategy, &c, &i);
    if (lane == 0) {
      const int pos = entry_pos[ent];
      conf[pos] = c;
      xhat[pos] = vocab_lo + i;
      sconf[pos - s * LB] = c;
      sxhat[pos - s * LB] = vocab_lo + i;
    }
  }
  __syncthreads();   // the merged entries of this sequence are in LDS
  if (wave == 0) {
    const bool m = lane < LB && id == mask_id;
    select_commit_vals(s, id, m ? sconf[lane] : -INFINITY, m ? sxhat[lane] : 0, conf, LB, mask_id, steps, t,
                       use_threshold, threshold, ids_out, remaining);
  }
}

// Merge only, one wavefront (workgroup) per entry over the whole grid: for
// passes with many partials the per-sequence workgroups of k_conf_select put
// all the partial reads on n_seq CUs.  k_select_commit then commits per
// sequence from conf / xhat (the same merge and commit functions, so the same
// decisions).  Entries past seq_off[n_seq] exit.
__global__ __launch_bounds__(64) void k_conf_merge_wide(const float* __restrict__ part, int ntiles,
                                                        const int32_t* __restrict__ seq_off, int n_seq,
                                                        const int32_t* __restrict__ entry_pos, int vocab_lo,
                                                        int strategy, float* __restrict__ conf,
                                                        int32_t* __restrict__ xhat) {
  const int ent = blockIdx.x;
  if (ent >= seq_off[n_seq]) return;
  const int pos = entry_pos[ent];
  float c;
  int i;
  conf_merge_entry(part, ent, ntiles, strategy, &c, &i);
  if (threadIdx.x == 0) {
    conf[pos] = c;
    xhat[pos] = vocab_lo + i;
  }
}

constexpr long long kConfWideMin = 65536;   // entries x partials from which the merge spreads over the grid

hipError_t launch_conf_select(const float* part, int ntiles, const int32_t* seq_off, const int32_t* entry_pos,
                              int vocab_lo, int strategy, const int32_t* ids_in, float* conf, int32_t* xhat,
                              int n_seq, int LB, int mask_id, int steps, int t, int use_threshold, float threshold,
                              int32_t* ids_out, int32_t* remaining, hipStream_t s) {
  if ((long long)n_seq * LB * ntiles >= kConfWideMin) {
    hipLaunchKernelGGL(k_conf_merge_wide, dim3(n_seq * LB), dim3(64), 0, s, part, ntiles, seq_off, n_seq, entry_pos,
                       vocab_lo, strategy, conf, xhat);
    hipLaunchKernelGGL(k_select_commit, dim3(n_seq), dim3(64), 0, s, ids_in, conf, xhat, LB, mask_id, steps, t,
                       use_threshold, threshold, ids_out, remaining);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_conf_select, dim3(n_seq), dim3(1024), 0, s, part, ntiles, seq_off, entry_pos, vocab_lo,
                     strategy, ids_in, conf, xhat, LB, mask_id, steps, t, use_threshold, threshold, ids_out,
                     remaining);
  return hipGetLastError();
}

hipError_t launch_select_commit(const int32_t* ids_in, const float* conf, const int32_t* xhat, int n_seq,
                                int LB, int mask_id, int steps, int t, int use_threshold, float threshold,
                                int32_t* ids_out, int32_t* remaining, hipStream_t s) {
  hipLaunchKernelGGL(k_select_commit, dim3(n_seq), dim3(64), 0, s, ids_in, const_cast<float*>(conf), xhat,
                     LB, mask_id, steps, t, use_threshold, threshold, ids_out, remaining);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Retention: per model row, keep the prefix positions of highest score (ties
// to the lower position), listed in ascending order.  Positions fall into two
// pools (visual ids, everything else) when prefix ids are given, else one;
// each pool keeps its own count.  Radix select on the float bits (scores are
// >= 0, so the bits order like the values), then an ordered compaction.  One
// workgroup per row.
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(1024) void k_retention(const float* __restrict__ score, int P, int stride,
                                                    const int32_t* __restrict__ pids, int vis_lo, int vis_hi,
                                                    float r_text, float r_image, int32_t* __restrict__ kept,
                                                    int32_t* __restrict__ n_kept) {
  __shared__ int hist[256];
  __shared__ int tmp[32];
  __shared__ uint32_t s_prefix;
  __shared__ int s_need;
  const int r = blockIdx.x, tid = threadIdx.x;
  const float* sr = score + (size_t)r * stride;
  const int32_t* ir = pids ? pids + (size_t)r * stride : nullptr;
  int32_t* kr = kept + (size_t)r * stride;
  auto pool_of = [&](int i) -> int {
    if (!ir) return 0;
    const int id = ir[i];
    return (id >= vis_lo && id < vis_hi) ? 1 : 0;
  };
  auto key_of = [&](int i) -> uint32_t { return __float_as_uint(fmaxf(sr[i], 0.f)); };
  int c1 = 0;
  if (ir)
    for (int i = tid; i < P; i += 1024) c1 += pool_of(i);
  int n_img;
  (void)block_exclusive_scan(c1, tmp, &n_img);
  const int size[2] = {P - n_img, n_img};
  const int want[2] = {keep_count(r_text, size[0]), keep_count(r_image, size[1])};
  // per pool: 0 keeps nothing, 1 keeps all, 2 keeps the top want[p]
  int mode[2];
  uint32_t T[2] = {0u, 0u};
  int need[2] = {0, 0};
  for (int p = 0; p < 2; ++p) {
    mode[p] = want[p] <= 0 ? 0 : (want[p] >= size[p] ? 1 : 2);
    if (mode[p] != 2) continue;   // uniform
    __syncthreads();              // the previous pool's threshold has been read
    if (tid == 0) {
      s_prefix = 0;
      s_need = want[p];
    }
    uint32_t pmask = 0;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      for (int b = tid; b < 256; b += 1024) hist[b] = 0;
      __syncthreads();
      const uint32_t prefix = s_prefix;
      for (int i = tid; i < P; i += 1024) {
        if (pool_of(i) != p) continue;
        const uint32_t u = key_of(i);
        if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 255], 1);
      }
      __syncthreads();
      if (tid == 0) {
        int need_p = s_need, cum = 0, sel = 0;
        for (int b = 255; b >= 0; --b) {
          if (cum + hist[b] >= need_p) {
            sel = b;
            break;
          }
          cum += hist[b];
        }
        s_need = need_p - cum;
        s_prefix = prefix | ((uint32_t)sel << shift);
      }
      pmask |= 255u << shift;
      __syncthreads();
    }
    T[p] = s_prefix;     // the want[p]-th largest key of the pool
    need[p] = s_need;    // how many keys equal to it are kept
  }
  // ordered compaction; the tie ranks of both pools share one packed scan
  int tie_base0 = 0, tie_base1 = 0, out_base = 0;
  for (int c0 = 0; c0 < P; c0 += 1024) {
    const int i = c0 + tid;
    int p = 0;
    uint32_t u = 0;
    if (i < P) {
      p = pool_of(i);
      u = key_of(i);
    }
    const bool tie = i < P && mode[p] == 2 && u == T[p];
    int tt;
    const int tr = block_exclusive_scan(tie ? (p ? (1 << 16) : 1) : 0, tmp, &tt);
    const int trank = p ? (tr >> 16) : (tr & 0xffff);
    const int tbase = p ? tie_base1 : tie_base0;
    const int keep =
        (i < P && (mode[p] == 1 || (mode[p] == 2 && (u > T[p] || (tie && tbase + trank < need[p]))))) ? 1 : 0;
    int kt;
    const int pos = block_exclusive_scan(keep, tmp, &kt);
    if (keep) kr[out_base + pos] = i;
    tie_base0 += tt & 0xffff;
    tie_base1 += tt >> 16;
    out_base += kt;
  }
  if (tid == 0) n_kept[r] = want[0] + want[1];
}

hipError_t launch_retention(const float* score, int rows, int P, int stride, const int32_t* pids, int vis_lo,
                            int vis_hi, float r_text, float r_image, int32_t* kept, int32_t* n_kept,
                            hipStream_t s) {
  hipLaunchKernelGGL(k_retention, dim3(rows), dim3(1024), 0, s, score, P, stride, pids, vis_lo, vis_hi, r_text,
                     r_image, kept, n_kept);
  return hipGetLastError();
}

// Key norms of appended prefix positions, for the key-norm + confidence
// retention score: per (row, position) the sum over heads of |K_h| of one
// layer, written into (first layer) or added to knorm[row][P0 + j].  One
// wavefront per position; each lane takes 16-byte chunks and the chunks of a
// head sit in an aligned group of lanes, so a head's sum of squares is a
// butterfly inside its group.
template <typename T>
__global__ __launch_bounds__(256) void k_key_norm(const T* __restrict__ kc, int rows, int n_tok, int H, int dh,
                                                  long long row_stride, long long head_stride, int P0,
                                                  float* __restrict__ knorm, int stride, int accumulate) {
  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= rows * n_tok) return;   // uniform per wavefront
  const int r = w / n_tok, j = w % n_tok;
  constexpr int kEl = 16 / (int)sizeof(T);
  const int cph = dh / kEl;        // chunks per head: a power of two in 4..32
  const int nch = H * cph;
  const T* base = kc + (size_t)r * row_stride + (size_t)(P0 + j) * dh;
  float acc = 0.f;
  for (int c0 = 0; c0 < nch; c0 += 64) {
    const int c = c0 + lane;
    float ss = 0.f;
    if (c < nch) {
      const T* p = base + (size_t)(c / cph) * head_stride + (c % cph) * kEl;
      if constexpr (sizeof(T) == 4) {
        const float4 v = *(const float4*)p;
        ss = v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
      } else {
        const uint4 v = *(const uint4*)p;
        const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float lo = __uint_as_float(wd[q] << 16), hi = __uint_as_float(wd[q] & 0xffff0000u);
          ss += lo * lo + hi * hi;
        }
      }
    }
    for (int o = 1; o < cph; o <<= 1) ss += __shfl_xor(ss, o, 64);
    if (c < nch && (lane % cph) == 0) acc += sqrtf(ss);
  }
  acc = wave_sum(acc);
  if (lane == 0) {
    float* d = knorm + (size_t)r * stride + P0 + j;
    *d = accumulate ? *d + acc : acc;
  }
}

hipError_t launch_key_norm(int mode, const void* kc, int rows, int n_tok, int H, int dh, long long row_stride,
                           long long head_stride, int P0, float* knorm, int stride, int accumulate,
                           hipStream_t s) {
  const int waves = rows * n_tok;
  if (waves == 0) return hipSuccess;
  dim3 grid((waves + 3) / 4);
  if (mode == MODE_F32)
    hipLaunchKernelGGL(k_key_norm<float>, grid, dim3(256), 0, s, (const float*)kc, rows, n_tok, H, dh, row_stride,
                       head_stride, P0, knorm, stride, accumulate);
  else
    hipLaunchKernelGGL(k_key_norm<uint16_t>, grid, dim3(256), 0, s, (const uint16_t*)kc, rows, n_tok, H, dh,
                       row_stride, head_stride, P0, knorm, stride, accumulate);
  return hipGetLastError();
}

// Top-1 probability of appended prefix positions from the LM-head partials
// of their rows (row m = model row m / n_tok, token m % n_tok): one wavefront
// per row, written to pconf[row][P0 + token].
__global__ __launch_bounds__(1024) void k_prefix_conf(const float* __restrict__ part, int ntiles, int M, int n_tok,
                                                      int P0, int stride, float* __restrict__ pconf) {
  const int m = blockIdx.x * 16 + (threadIdx.x >> 6);
  if (m >= M) return;   // uniform per wavefront; the merge uses no barrier
  float c;
  int i;
  conf_merge_entry(part, m, ntiles, 0, &c, &i);
  if ((threadIdx.x & 63) == 0) pconf[(size_t)(m / n_tok) * stride + P0 + m % n_tok] = c;
}

hipError_t launch_prefix_conf(const float* part, int ntiles, int M, int n_tok, int P0, int stride, float* pconf,
                              hipStream_t s) {
  if (M == 0) return hipSuccess;
  hipLaunchKernelGGL(k_prefix_conf, dim3((M + 15) / 16), dim3(1024), 0, s, part, ntiles, M, n_tok, P0, stride,
                     pconf);
  return hipGetLastError();
}

// Prefix ids of appended positions (modality pools): out[row][P0 + j].
__global__ __launch_bounds__(256) void k_store_ids(const int32_t* __restrict__ ids, int ids_stride, int rows,
                                                   int n_tok, int P0, int stride, int32_t* __restrict__ out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows * n_tok) return;
  const int r = i / n_tok, j = i % n_tok;
  out[(size_t)r * stride + P0 + j] = ids[(size_t)r * ids_stride + j];
}

hipError_t launch_store_ids(const int32_t* ids, int ids_stride, int rows, int n_tok, int P0, int stride,
                            int32_t* out, hipStream_t s) {
  const int n = rows * n_tok;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_store_ids, dim3((n + 255) / 256), dim3(256), 0, s, ids, ids_stride, rows, n_tok, P0, stride,
                     out);
  return hipGetLastError();
}

// Key-norm + confidence retention score of every prefix position:
// score = alpha * knorm / mean(knorm) + (1 - alpha) * pconf, the mean over
// the row's P positions (0 when all norms are 0).  One workgroup per row.
__global__ __launch_bounds__(1024) void k_retention_score(const float* __restrict__ knorm,
                                                          const float* __restrict__ pconf, int P, int stride,
                                                          float alpha, float* __restrict__ score) {
  __shared__ float tmp[16];
  const int r = blockIdx.x;
  const float* kr = knorm + (size_t)r * stride;
  const float* cr = pconf + (size_t)r * stride;
  float* sr = score + (size_t)r * stride;
  float acc = 0.f;
  for (int i = threadIdx.x; i < P; i += blockDim.x) acc += kr[i];
  const float tot = block_sum(acc, tmp);
  const float inv_mean = tot > 0.f ? (float)P / tot : 0.f;
  for (int i = threadIdx.x; i < P; i += blockDim.x) sr[i] = alpha * (kr[i] * inv_mean) + (1.f - alpha) * cr[i];
}

hipError_t launch_retention_score(const float* knorm, const float* pconf, int rows, int P, int stride, float alpha,
                                  float* score, hipStream_t s) {
  if (P == 0) return hipSuccess;
  hipLaunchKernelGGL(k_retention_score, dim3(rows), dim3(1024), 0, s, knorm, pconf, P, stride, alpha, score);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Packed fragment layout of expert gate/up weights.  For each matrix [rows][K]
// (rows = F of one expert), with KL = 16 for fp8 and 8 otherwise and KC = 4 KL,
// fragment (t, c) of rows 16 t .. 16 t + 15 and reduction chunk KC c .. KC c +
// KC - 1 holds, for lane l = 0..63, the KL elements W[16 t + l % 16][KC c +
// KL (l / 16) .. + KL - 1] at lane offset KL l: exactly what lane l of a
// weight-fragment load reads, so one fragment is one contiguous 64 x KL-element
// read.  Fragments are ordered (matrix, t, c).  One wavefront copies one
// fragment.
// ---------------------------------------------------------------------------

template <int ES>
__global__ __launch_bounds__(256) void k_pack_fragments(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                        long long n_frag, int rows, int K) {
  constexpr int KL = ES == 1 ? 16 : 8;   // elements per lane and fragment (16 bytes; 32 for float32)
  constexpr int KC = 4 * KL;
  const long long f = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (f >= n_frag) return;
  const int lane = threadIdx.x & 63;
  const int kch = K / KC, rt = rows / 16;
  const int c = (int)(f % kch);
  const long long mt = f / kch;                  // matrix * rt + t
  const int t = (int)(mt % rt);
  const long long mat = mt / rt;
  const size_t s_off = ((size_t)mat * rows + (size_t)t * 16 + (lane & 15)) * K + (size_t)c * KC + KL * (lane >> 4);
  const size_t d_off = ((size_t)f * 64 + lane) * KL;
  if constexpr (ES == 4) {
    const uint4* sp = (const uint4*)(src + 4 * s_off);
    uint4* dp = (uint4*)(dst + 4 * d_off);
    dp[0] = sp[0];
    dp[1] = sp[1];
  } else {
    *(uint4*)(dst + ES * d_off) = *(const uint4*)(src + ES * s_off);
  }
}

hipError_t launch_pack_fragments(const void* src, void* dst, long long n_mats, int rows, int K, int es,
                                 hipStream_t s) {
  const int kc = es == 1 ? 64 : 32;
  const long long n_frag = n_mats * (rows / 16) * (K / kc);
  if (n_frag == 0) return hipSuccess;
  dim3 grid((unsigned)((n_frag + 3) / 4));
  if (es == 1)
    hipLaunchKernelGGL(k_pack_fragments<1>, grid, dim3(256), 0, s, (const uint8_t*)src, (uint8_t*)dst, n_frag, rows, K);
  else if (es == 2)
    hipLaunchKernelGGL(k_pack_fragments<2>, grid, dim3(256), 0, s, (const uint8_t*)src, (uint8_t*)dst, n_frag, rows, K);
  else
    hipLaunchKernelGGL(k_pack_fragments<4>, grid, dim3(256), 0, s, (const uint8_t*)src, (uint8_t*)dst, n_frag, rows, K);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// small utilities
// ---------------------------------------------------------------------------

__global__ void k_fill_f32(float* p, float v, long long n) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t launch_fill_f32(float* p, float v, long long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, v, n);
  return hipGetLastError();
}

__global__ void k_decode_fp8(const uint8_t* codes, int n, float* out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i * 8 >= n) return;
  uint2 w = make_uint2(0, 0);
  uint8_t b[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int j = 0; j < 8; ++j)
    if (i * 8 + j < n) b[j] = codes[i * 8 + j];
  w.x = b[0] | (b[1] << 8) | (b[2] << 16) | ((uint32_t)b[3] << 24);
  w.y = b[4] | (b[5] << 8) | (b[6] << 16) | ((uint32_t)b[7] << 24);
  const bf16x8 v = Op<MODE_FP8>::widen(w);
  for (int j = 0; j < 8; ++j)
    if (i * 8 + j < n) out[i * 8 + j] = (float)v[j];
}

hipError_t launch_decode_fp8(const uint8_t* codes, int n, float* out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int nt = (n + 7) / 8;
  hipLaunchKernelGGL(k_decode_fp8, dim3((nt + 255) / 256), dim3(256), 0, s, codes, n, out);
  return hipGetLastError();
}

}  // namespace dllm
