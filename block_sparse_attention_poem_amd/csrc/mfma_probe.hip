// On-card bf16 MFMA rate probes (measurement only; not part of libpoem's hot path).
//
// Every wave issues independent chains of v_mfma_f32_32x32x16_bf16 on register
// operands: no memory traffic, no LDS, no vector work inside the loop. The rate they
// reach under the card's own clock and power management is a practical ceiling for
// the attention kernels, beside the 2.5 PFLOP/s quoted at 2.4 GHz. The constant probe
// feeds every MFMA the same few-bit operands; the random probe rotates through eight
// operand pairs of random sign and mantissa bits, so the multiplier inputs change from
// one MFMA to the next as they do when a kernel streams real K and V fragments (the
// switching power, and with it the clock the power limit allows, depends on that).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kChains = 4;      // independent accumulators per wave
constexpr int kThreads = 256;   // four waves, one per SIMD

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mfma_peak_kernel(float* sink, int iters) {
  const uint32_t t = threadIdx.x;
  // operands depend on the thread so the compiler cannot fold the products
  const u32x4 wa = {0x3f803f80u ^ (t & 7), 0x3f803f80u, 0x3f003f00u, 0x3f803f80u};
  const u32x4 wb = {0x3e803e80u, 0x3f803f80u ^ (t & 3), 0x3f803f80u, 0x3f003f00u};
  const bf16x8 a = __builtin_bit_cast(bf16x8, wa);
  const bf16x8 b = __builtin_bit_cast(bf16x8, wb);
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = f32x16{};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  // a store that (almost) never happens keeps the loop alive without memory traffic
  if (s == -1.0f) sink[blockIdx.x * kThreads + t] = s;
}

// integer hash (the MurmurHash3 32-bit finalizer)
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x85ebca6bu;
  x ^= x >> 13;
  x *= 0xc2b2ae35u;
  x ^= x >> 16;
  return x;
}

// two bf16 values of random sign and mantissa with the exponent of 2^-1: |v| in [0.5, 1)
__device__ __forceinline__ uint32_t rand_bf16x2(uint32_t key) { return (mix32(key) & 0x807F807Fu) | 0x3F003F00u; }

constexpr int kOperands = 8;  // operand pairs a wave rotates through

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mfma_random_kernel(float* sink, int iters, uint32_t seed) {
  const uint32_t t = blockIdx.x * kThreads + threadIdx.x;
  bf16x8 a[kOperands], b[kOperands];
#pragma unroll
  for (int j = 0; j < kOperands; ++j) {
    const uint32_t k = seed ^ (t * 64u + j * 8u);
    const u32x4 wa = {rand_bf16x2(k), rand_bf16x2(k + 1), rand_bf16x2(k + 2), rand_bf16x2(k + 3)};
    const u32x4 wb = {rand_bf16x2(k + 4), rand_bf16x2(k + 5), rand_bf16x2(k + 6), rand_bf16x2(k + 7)};
    a[j] = __builtin_bit_cast(bf16x8, wa);
    b[j] = __builtin_bit_cast(bf16x8, wb);
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = f32x16{};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int u = 0; u < kOperands; ++u)
      acc[u % kChains] =
          __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[u], b[(3 * u + 1) % kOperands], acc[u % kChains], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  if (s == -1.0f) sink[t] = s;
}

}  // namespace

extern "C" {

// Enqueues blocks x 256 threads, each wave running iters x 4 MFMAs of 32x32x16 bf16
// (32768 FLOP each). Returns the FLOP count enqueued, or -1 if the launch failed.
// sink: device fp32 [blocks * 256], written only in a case that does not arise.
double poem_probe_mfma_bf16(float* sink, int blocks, int iters, void* stream) {
  hipLaunchKernelGGL(mfma_peak_kernel, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream), sink,
                     iters);
  if (hipGetLastError() != hipSuccess) return -1.0;
  return (double)blocks * (kThreads / 64) * (double)iters * kChains * 32768.0;
}

// As poem_probe_mfma_bf16 with random operands (eight pairs per wave from `seed`), each
// wave running iters x 8 MFMAs. Returns the FLOP count enqueued, or -1 on failure.
double poem_probe_mfma_bf16_random(float* sink, int blocks, int iters, uint32_t seed, void* stream) {
  hipLaunchKernelGGL(mfma_random_kernel, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream), sink,
                     iters, seed);
  if (hipGetLastError() != hipSuccess) return -1.0;
  return (double)blocks * (kThreads / 64) * (double)iters * kOperands * 32768.0;
}

}  // extern "C"
