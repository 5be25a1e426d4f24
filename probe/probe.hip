// Measurement helpers for the benchmark, built into their own library
// (libsa_probe.so) and kept out of the attention library's ABI.
//
//   sa_probe_clock   one wavefront samples the shader clock counter
//                    (s_memtime, one tick per engine clock) against the
//                    constant-rate real-time counter (s_memrealtime) over a
//                    bounded window.  Launched on its own stream next to
//                    another kernel, it reads off the engine clock the chip
//                    runs that kernel at.
//   sa_probe_mfma    a dense loop of independent 32x32x16 bf16 MFMAs on every
//                    SIMD: the matrix rate the chip reaches with nothing else
//                    to do.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr int kMaxSamples = 256;
constexpr long long kMaxSpins = 100000000;  // safety bound on the sampling loop

// out[2 s] = engine-clock count, out[2 s + 1] = real-time count of sample s
// (one sample every `every` real-time ticks, and one at the end);
// out[2 kMaxSamples] = samples taken.  Ends after `window` real-time ticks, kMaxSamples samples or
// kMaxSpins iterations, whichever comes first.
__global__ __launch_bounds__(64) void clock_sampler(uint64_t* out, uint64_t window,
                                                    uint64_t every) {
  if (threadIdx.x != 0) return;
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  uint64_t next = r0;
  int n = 0;
  for (long long spin = 0; spin < kMaxSpins && n < kMaxSamples; ++spin) {
    const uint64_t r = __builtin_amdgcn_s_memrealtime();
    if (r >= next) {
      const uint64_t m = __builtin_amdgcn_s_memtime();
      out[2 * n] = m;
      out[2 * n + 1] = r;
      ++n;
      next = r + every;
    }
    if (r - r0 >= window) break;
  }
  if (n < kMaxSamples) {  // a last sample at the end, so the samples span the whole run
    out[2 * n] = __builtin_amdgcn_s_memtime();
    out[2 * n + 1] = __builtin_amdgcn_s_memrealtime();
    ++n;
  }
  out[2 * kMaxSamples] = (uint64_t)n;
}

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
constexpr int kChains = 8;  // independent accumulators per wavefront

__global__ __launch_bounds__(256) void mfma_loop(float* out, int iters) {
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(1e-3f * (float)((threadIdx.x + e) & 7));
    b[e] = (__bf16)(1e-3f * (float)(e + 1));
  }
  for (int i = 0; i < iters; ++i)
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

__attribute__((visibility("default"))) int sa_probe_clock_max_samples() { return kMaxSamples; }

// out: device, 2 * kMaxSamples + 1 uint64 values.  Returns a hipError_t.
__attribute__((visibility("default"))) int sa_probe_clock(uint64_t* out, uint64_t window,
                                                          uint64_t every, void* stream) {
  if (!out || every == 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(clock_sampler, dim3(1), dim3(64), 0, (hipStream_t)stream, out, window,
                     every);
  return (int)hipGetLastError();
}

// out: device, blocks * 256 floats.  Executes blocks * 4 * iters * kChains
// MFMAs of 2 * 32 * 32 * 16 flops.  Returns a hipError_t.
__attribute__((visibility("default"))) int sa_probe_mfma(float* out, int blocks, int iters,
                                                         void* stream) {
  if (!out || blocks <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_loop, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters);
  return (int)hipGetLastError();
}

__attribute__((visibility("default"))) int sa_probe_mfma_chains() { return kChains; }

}  // extern "C"
