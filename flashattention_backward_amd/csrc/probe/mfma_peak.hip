// Sustained matrix-core throughput of the whole chip, and the shader clock it runs at (not
// part of the attention library; built into libfab_probe.so and run by bench.py
// --mfma-peak).  The measurement behind the practical ceiling of the attention kernels:
// the dense bf16 peak assumes every MFMA pipe busy at the 2.4 GHz peak clock, and the
// question is what clock the chip holds when they are.
//
// Every wave runs `iters` rounds of eight independent v_mfma_f32_32x32x16_bf16 (eight
// accumulators, so no MFMA waits on another's result), and lane 0 records the shader-clock
// counter (s_memtime) and the 100 MHz real-time counter (s_memrealtime) around the loop.
// Their ratio is the wave's average shader clock.  The matrix cores' power, and so the clock
// the chip holds, depends on how many operand bits change from one MFMA to the next:
//   mode 0  all eight MFMAs of a round read the same small operands (few bits change)
//   mode 1  each chain has its own pseudo-random operands of unit size, as attention's
//           Q, K, V, dO tiles are (most bits change between consecutive MFMAs)
#include <hip/hip_runtime.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
constexpr int kChains = 8;

// Pseudo-random value in [-2, 2) from a lane, chain and element index (an integer hash).
__device__ __forceinline__ float hashed_unit(unsigned x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return (float)(x & 0xffff) * (4.f / 65536.f) - 2.f;
}

__global__ __launch_bounds__(256) void mfma_peak_kernel(unsigned long long* out, int iters, int mode) {
  const int lane = threadIdx.x & 63;
  bf16x8 a[kChains], b[kChains];
#pragma unroll
  for (int k = 0; k < kChains; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const unsigned id = ((unsigned)blockIdx.x * 256 + threadIdx.x) * 64 + k * 8 + e;
      a[k][e] = (__bf16)(mode == 0 ? 0.001f * (float)(lane + e) : hashed_unit(2 * id));
      b[k][e] = (__bf16)(mode == 0 ? 0.002f * (float)(lane - e) : hashed_unit(2 * id + 1));
    }
  f32x16 acc[kChains];
#pragma unroll
  for (int k = 0; k < kChains; ++k) acc[k] = f32x16{};
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  // the operands pass through an empty asm after the counters are read, so no MFMA can be
  // scheduled before them
#pragma unroll
  for (int k = 0; k < kChains; ++k) asm volatile("" : "+v"(a[k]), "+v"(b[k]));
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < kChains; ++k) acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[k], b[k], acc[k], 0, 0, 0);
  }
  float sum = 0.f;
#pragma unroll
  for (int k = 0; k < kChains; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) sum += acc[k][r];
  // ... and every result is consumed before the closing counters are read
  asm volatile("" : "+v"(sum));
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  if (lane == 0) {
    const size_t wave = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    out[4 * wave + 0] = t1 - t0;
    out[4 * wave + 1] = r1 - r0;
    out[4 * wave + 2] = (unsigned long long)__float_as_uint(sum);
    out[4 * wave + 3] = 0;
  }
}

}  // namespace

extern "C" {

// Launch the probe on `stream`: `blocks` workgroups of 4 waves, each wave `iters` rounds of
// eight MFMAs, operands per `mode` (0 or 1, above).  out: device memory of blocks * 4 * 4
// uint64 (per wave: shader-clock ticks, real-time ticks at 100 MHz, the bits of a checksum,
// 0).  Returns 0, 1 for invalid arguments, or 2 if the launch failed.
int fab_probe_mfma(unsigned long long* out, int blocks, int iters, int mode, void* stream) {
  if (out == nullptr || blocks < 1 || iters < 1 || mode < 0 || mode > 1) return 1;
  hipLaunchKernelGGL(mfma_peak_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters, mode);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
