// Seeded synthetic inputs on the GPU (input preparation only; none of the
// denoising step's arithmetic).  The same counter streams as
// dllm_inputs/counter.py, bit for bit:
//  - Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
//    easy as 1, 2, 3", SC 2011): key = (seed, tag * 65536 + layer), counter =
//    (j mod 2^32, j div 2^32, expert, 0) for the j-th element pair of a matrix;
//  - a weight is the centred sum of four 16-bit uniforms times a float32
//    factor (one rounding), stored as float32, bfloat16 (round to nearest
//    even) or E4M3FN codes with a float32 scale per row (amax / 448, codes
//    rounded to nearest even in double precision, saturated at 448);
//  - a uniform value in [-h, h) is ((w0 >> 8) - 2^23) * (h / 2^23).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

struct U4 {
  uint32_t x, y, z, w;
};

__device__ __forceinline__ U4 philox(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)c0 * 0xD2511F53ull;
    const uint64_t p1 = (uint64_t)c2 * 0xCD9E8D57ull;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return U4{c0, c1, c2, c3};
}

__device__ __forceinline__ int ih4(uint32_t a, uint32_t b) {
  return (int)(a & 0xFFFFu) + (int)(a >> 16) + (int)(b & 0xFFFFu) + (int)(b >> 16) - 131070;
}

// elements 2j and 2j + 1 of a stream, as float32
__device__ __forceinline__ void pair(unsigned long long j, uint32_t expert, uint32_t seed, uint32_t kl, float k,
                                     float* a, float* b) {
  const U4 r = philox((uint32_t)j, (uint32_t)(j >> 32), expert, 0u, seed, kl);
  // exact integers in float32, one rounded product each
  *a = __fmul_rn((float)ih4(r.x, r.y), k);
  *b = __fmul_rn((float)ih4(r.z, r.w), k);
}

__device__ __forceinline__ uint16_t bf16_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__global__ void k_normal(void* out, int dtype, long long n, uint32_t seed, uint32_t kl, uint32_t expert, float k) {
  const long long npair = (n + 1) / 2;
  for (long long j = blockIdx.x * (long long)blockDim.x + threadIdx.x; j < npair;
       j += (long long)gridDim.x * blockDim.x) {
    float a, b;
    pair((unsigned long long)j, expert, seed, kl, k, &a, &b);
    const long long i = 2 * j;
    if (dtype == 0) {
      float* o = (float*)out;
      o[i] = a;
      if (i + 1 < n) o[i + 1] = b;
    } else {
      uint16_t* o = (uint16_t*)out;
      o[i] = bf16_rne(a);
      if (i + 1 < n) o[i + 1] = bf16_rne(b);
    }
  }
}

// E4M3FN code of x = v / scale (double), rounded to nearest even, saturated
// at 448: normal magnitudes (>= 2^-6) keep 3 mantissa bits of their double
// bits, smaller ones are multiples of 2^-9.
__device__ __forceinline__ uint8_t e4m3_code(double x) {
  const bool neg = x < 0.0 || (x == 0.0 && __double_as_longlong(x) < 0);
  double a = fabs(x);
  a = a < 448.0 ? a : 448.0;
  int c;
  if (a >= 0.015625) {
    const unsigned long long u = (unsigned long long)__double_as_longlong(a);
    const unsigned long long lsb = (u >> 49) & 1ull;
    const unsigned long long ur = (u + ((1ull << 48) - 1ull) + lsb) & ~((1ull << 49) - 1ull);
    const int e = (int)((ur >> 52) & 0x7FFull) - 1023;
    const int m = (int)((ur >> 49) & 7ull);
    c = ((e + 7) << 3) | m;
    c = c < 0x7E ? c : 0x7E;
  } else {
    c = (int)rint(a * 512.0);
  }
  return (uint8_t)(c | (neg ? 0x80 : 0));
}

// One workgroup per row of a [rows][cols] matrix stream (cols even, <= 8192).
__global__ __launch_bounds__(256) void k_normal_fp8(uint8_t* codes, float* scales, int rows, int cols, uint32_t seed,
                                                    uint32_t kl, uint32_t expert0, float k) {
  __shared__ float vals[8192];
  __shared__ float red[256];
  const int row = blockIdx.x;
  if (row >= rows) return;
  // blockIdx.y: the expert within the batch; its matrix follows the previous one
  const uint32_t expert = expert0 + blockIdx.y;
  codes += (size_t)blockIdx.y * rows * cols;
  scales += (size_t)blockIdx.y * rows;
  const unsigned long long j0 = (unsigned long long)row * (cols / 2);
  float amax = 0.f;
  for (int p = threadIdx.x; p < cols / 2; p += blockDim.x) {
    float a, b;
    pair(j0 + p, expert, seed, kl, k, &a, &b);
    vals[2 * p] = a;
    vals[2 * p + 1] = b;
    amax = fmaxf(amax, fmaxf(fabsf(a), fabsf(b)));
  }
  red[threadIdx.x] = amax;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + s]);
    __syncthreads();
  }
  float sc = (float)((double)red[0] / 448.0);
  if (sc == 0.f) sc = 1.f;
  for (int i = threadIdx.x; i < cols; i += blockDim.x)
    codes[(size_t)row * cols + i] = e4m3_code((double)vals[i] / (double)sc);
  if (threadIdx.x == 0) scales[row] = sc;
}

__global__ void k_uniform(float* out, long long n, uint32_t seed, uint32_t kl, float h) {
  for (long long j = blockIdx.x * (long long)blockDim.x + threadIdx.x; j < n; j += (long long)gridDim.x * blockDim.x) {
    const U4 r = philox((uint32_t)j, (uint32_t)((unsigned long long)j >> 32), 0u, 0u, seed, kl);
    out[j] = __fmul_rn((float)((int)(r.x >> 8) - (1 << 23)), h);
  }
}

int grid_for(long long work) {
  long long g = (work + 255) / 256;
  if (g > 65536) g = 65536;
  return (int)(g < 1 ? 1 : g);
}

}  // namespace

extern "C" {

// n values of the (seed, tag, layer, expert) stream into d_out (dtype 0:
// float32, 1: bfloat16 bits), standard-deviation factor k.  0 on success,
// -1 on a bad argument, -3 on a launch error.
int dllm_inputs_normal(void* d_out, int dtype, long long n, uint32_t seed, uint32_t tag, uint32_t layer,
                       uint32_t expert, float k, void* stream) {
  if (!d_out || n < 0 || (dtype != 0 && dtype != 1)) return -1;
  if (n == 0) return 0;
  hipLaunchKernelGGL(k_normal, dim3(grid_for((n + 1) / 2)), dim3(256), 0, (hipStream_t)stream, d_out, dtype, n, seed,
                     tag * 65536u + layer, expert, k);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

// n_experts consecutive [rows][cols] matrices (experts expert .. expert +
// n_experts - 1, each its own stream), quantized per row to E4M3FN codes and
// float32 scales.  cols even and <= 8192.
int dllm_inputs_normal_fp8(uint8_t* d_codes, float* d_scales, int rows, int cols, int n_experts, uint32_t seed,
                           uint32_t tag, uint32_t layer, uint32_t expert, float k, void* stream) {
  if (!d_codes || !d_scales || rows < 0 || cols < 2 || cols % 2 || cols > 8192 || n_experts < 0 ||
      n_experts > 65535)
    return -1;
  if (rows == 0 || n_experts == 0) return 0;
  hipLaunchKernelGGL(k_normal_fp8, dim3(rows, n_experts), dim3(256), 0, (hipStream_t)stream, d_codes, d_scales, rows,
                     cols, seed, tag * 65536u + layer, expert, k);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

// n uniform float32 values in [-h, h) (h_scaled = h / 2^23).
int dllm_inputs_uniform(float* d_out, long long n, uint32_t seed, uint32_t tag, uint32_t layer, float h_scaled,
                        void* stream) {
  if (!d_out || n < 0) return -1;
  if (n == 0) return 0;
  hipLaunchKernelGGL(k_uniform, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream, d_out, n, seed,
                     tag * 65536u + layer, h_scaled);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

// Interface revision of the entry points above; the Python caller refuses a
// library built from other sources.
int dllm_inputs_abi_version(void) { return 2; }

}  // extern "C"
