// Step 1 of the backward (boostr flash_bwd.rs, "Step 1: Preprocessing"):
//   D[row] = sum_d dO[row, d] * o[row, d]   (float32), one row per (b, h, query),
// stored next to the row's LSE rescaled to base 2 (the unit of the kernels' exp2), as the
// per-row statistics {LSE * log2(e), D} the main kernels stage with each query tile.
//
// HBM-bound: each row is read once from each of dO and o.  Lanes load 16 contiguous bytes
// each, so a wavefront reads whole rows with fully coalesced 16-byte loads; the lanes that
// share a row reduce their partial sums with cross-lane shuffles.
#include "common.h"
#include "launch.h"

namespace fab {

// Lanes that share a row: its number of 16-byte chunks rounded up to a power of two, at most
// 64 (a lane sums chunks sub, sub + L, ...; lanes past the last chunk idle).
constexpr int lanes_per_row(int chunks) {
  int l = 1;
  while (l < chunks && l < 64) l *= 2;
  return l;
}

template <class T, int HD>
__global__ __launch_bounds__(256) void preprocess_kernel(const PreParams p) {
  constexpr int E = 16 / sizeof(T);          // elements per 16-byte load
  constexpr int CH = HD / E;                 // 16-byte chunks per row
  constexpr int L = lanes_per_row(CH);
  constexpr int ROWS_PER_PASS = 256 / L;
  constexpr int PASSES = 4;
  const int tid = threadIdx.x;
  const int sub = tid % L;
  const long long row_base = (long long)blockIdx.x * (ROWS_PER_PASS * PASSES);
  const long long rows = (long long)p.BH * p.Sq_pad;
  const T* dO = (const T*)p.dO;
  const T* o = (const T*)p.o;
#pragma unroll
  for (int pass = 0; pass < PASSES; ++pass) {
    const long long row = row_base + pass * ROWS_PER_PASS + tid / L;  // padded row index
    const int bh = (int)(row / p.Sq_pad), m = (int)(row % p.Sq_pad);
    const bool valid = row < rows && m < p.Sq;
    const long long src_row = (long long)bh * p.Sq + m;
    float acc = 0.f;
#pragma unroll
    for (int c = sub; c < CH; c += L) {
      if (!valid) continue;
      const size_t off = (size_t)src_row * HD + c * E;
      if constexpr (sizeof(T) == 2) {
        typedef T v8 __attribute__((ext_vector_type(8)));
        const v8 a = *reinterpret_cast<const v8*>(dO + off);
        const v8 b = *reinterpret_cast<const v8*>(o + off);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc += (float)a[e] * (float)b[e];
      } else {
        const f32x4 a = *reinterpret_cast<const f32x4*>(dO + off);
        const f32x4 b = *reinterpret_cast<const f32x4*>(o + off);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc += a[e] * b[e];
      }
    }
#pragma unroll
    for (int w = L / 2; w > 0; w >>= 1) acc += __shfl_xor(acc, w, L);
    if (sub == 0 && row < rows) {
      // A row with LSE = -inf may attend no key (a window can leave a row without keys); it
      // gets the padding rows' +inf, so that exp2(score - lse2) is 0 on all its pairs.
      const float lse = valid ? p.lse[src_row] : -__builtin_inff();
      const float l2 = lse == -__builtin_inff() ? __builtin_inff() : lse * kLog2e;
      *reinterpret_cast<float2*>(p.stats + 2 * row) = make_float2(l2, valid ? acc : 0.f);
    }
  }
}

template <class T, int HD>
static hipError_t go(const PreParams& p, hipStream_t s, LaunchInfo* info) {
  constexpr int rows_per_block = (256 / lanes_per_row(HD / (16 / sizeof(T)))) * 4;
  const long long rows = (long long)p.BH * p.Sq_pad;
  const long long grid = (rows + rows_per_block - 1) / rows_per_block;
  if (info) *info = LaunchInfo{"preprocess", (int)grid, 256, 0};
  hipLaunchKernelGGL((preprocess_kernel<T, HD>), dim3((unsigned)grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <class T>
static hipError_t go_hd(const PreParams& p, int hd, hipStream_t s, LaunchInfo* info) {
  switch (hd) {
    case 32: return go<T, 32>(p, s, info);
    case 64: return go<T, 64>(p, s, info);
    case 96: return go<T, 96>(p, s, info);
    case 128: return go<T, 128>(p, s, info);
    default: return go<T, 256>(p, s, info);
  }
}

hipError_t launch_preprocess(const PreParams& p, int dt, int hd, hipStream_t s, LaunchInfo* info) {
  if (dt == kBF16) return go_hd<bf16>(p, hd, s, info);
  if (dt == kF16) return go_hd<f16>(p, hd, s, info);
  return go_hd<float>(p, hd, s, info);
}

}  // namespace fab
