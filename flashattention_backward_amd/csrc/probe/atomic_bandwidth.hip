// Measurement kernels behind the choice of a deterministic dQ pass over fp32 atomics (not
// part of the attention library; built into libfab_probe.so and run by bench.py --atomics).
//
// flash_bwd.rs's main step adds every (key tile, query tile) contribution to dQ with atomic
// adds.  Each such contribution is one 64-row x 128-column fp32 block, 32 KiB.  These kernels
// stream 32 KiB tiles of an fp32 buffer from every workgroup, `iters` tiles per workgroup,
// and do to every element of a tile one of:
//   mode 0  a no-return fp32 atomic add, tiles scattered over the buffer
//   mode 1  the same, each XCD's workgroups confined to their own eighth of the buffer
//   mode 2  a plain store
//   mode 3  a plain read-modify-write (load, add, store), what a non-atomic owner would do
// The payload is blocks * iters * 32 KiB in every mode.
#include <hip/hip_runtime.h>

namespace {

constexpr int kTile = 8192;  // floats per tile (32 KiB)

__device__ __forceinline__ int pick_tile(int wg, int it, int ntiles, int xcd_local) {
  if (xcd_local) {  // workgroups are dispatched round-robin over the 8 XCDs: wg % 8 = XCD
    const int per = ntiles / 8, x = wg % 8, s = wg / 8;
    return x * per + (s * 5 + it * 3) % per;
  }
  return (wg * 37 + it * 11) % ntiles;
}

__global__ __launch_bounds__(256) void probe_kernel(float* buf, int ntiles, int iters, int mode) {
  const int wg = blockIdx.x;
  for (int it = 0; it < iters; ++it) {
    float* t = buf + (size_t)pick_tile(wg, it, ntiles, mode == 1) * kTile;
#pragma unroll 4
    for (int e = threadIdx.x; e < kTile; e += 256) {
      if (mode <= 1) {
        __hip_atomic_fetch_add(t + e, 1.0f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else if (mode == 2) {
        t[e] = (float)e;
      } else {
        t[e] = t[e] + 1.0f;
      }
    }
  }
}

}  // namespace

extern "C" {

// Launch one probe on `stream`.  buf: device memory of ntiles * 32 KiB (ntiles a positive
// multiple of 8).  Returns 0, 1 for invalid arguments, or 2 if the launch failed.
int fab_probe_launch(float* buf, int ntiles, int blocks, int iters, int mode, void* stream) {
  if (buf == nullptr || ntiles < 8 || ntiles % 8 != 0 || blocks < 1 || iters < 1 || mode < 0 || mode > 3)
    return 1;
  hipLaunchKernelGGL(probe_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, buf, ntiles, iters, mode);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
