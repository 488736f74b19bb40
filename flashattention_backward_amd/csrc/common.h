// Device-side building blocks shared by the gfx950 kernels: element types, 8-element
// operand fragments, the 32x32 MFMA step, and global/LDS vector moves.
//
// MFMA lane layout used throughout (v_mfma_f32_32x32x16_{bf16,f16}; fp32 issues eight
// v_mfma_f32_32x32x2_f32 over the same fragment):
//   A operand (32 x 16, row i, column k): lane l holds A[l % 32][8 * (l / 32) + t], t < 8
//   B operand (16 x 32, row k, column j): lane l holds B[8 * (l / 32) + t][l % 32]
//   C/D       (32 x 32):                  lane l, register r holds
//                                         D[8 * (r / 4) + 4 * (l / 32) + r % 4][l % 32]
// A contraction over an index that an accumulator holds "in lane" (rows of C) uses the
// accumulator's registers 8s..8s+7 as one fragment; slot t then stands for row
// 16 s + 8 (t / 4) + 4 (l / 32) + t % 4, and the other operand is read from a tile whose
// rows were stored in the matching permuted order (perm16 below).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fab {

typedef __bf16 bf16;
typedef _Float16 f16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <class T> struct Frag;
template <> struct Frag<bf16> { typedef bf16x8 type; };
template <> struct Frag<f16> { typedef f16x8 type; };
template <> struct Frag<float> { typedef f32x8 type; };

// acc += A * B over one 16-wide slice of the contraction.
__device__ __forceinline__ void mma(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x16& acc, const f16x8& a, const f16x8& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x16& acc, const f32x8& a, const f32x8& b) {
#pragma unroll
  for (int t = 0; t < 8; ++t) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t], b[t], acc, 0, 0, 0);
}

// acc += A * B with the accumulator pinned to AGPRs (the "a" constraint).  Used for the
// long-lived accumulators (dK, dV, dQ) so that the register allocator never moves them
// between the AGPR and VGPR files; the short-lived score tiles use mma() in VGPRs.
// Hazards handled here, because the compiler does not look inside the asm: `s_nop 1` gives
// the two wait states needed between a VALU write of an A/B operand and the MFMA reading it;
// consecutive MFMAs accumulating into the same registers need none; reads of the
// accumulators after the last MFMA must go through mma_drain() first.
__device__ __forceinline__ void mma_a(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mma_a(f32x16& acc, const f16x8& a, const f16x8& b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// Wait states between the last accumulating MFMA and any other access to its registers
// (more than the 8 passes plus the read latency of a 32x32x16 MFMA).  Every accumulator is an
// operand, so no accumulating MFMA can be scheduled after the wait and no read before it.
__device__ __forceinline__ void mma_drain(f32x16 (&a)[4]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(a[0]), "+a"(a[1]), "+a"(a[2]), "+a"(a[3]));
}
__device__ __forceinline__ void mma_drain(f32x16 (&a)[2]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(a[0]), "+a"(a[1]));
}

// 8 consecutive elements <-> fragment.  16-bit types move as one 16-byte access, fp32 as
// two, so only 16-byte alignment is ever required.
template <class T>
__device__ __forceinline__ typename Frag<T>::type ld8(const T* p) {
  typedef typename Frag<T>::type F;
  if constexpr (sizeof(T) == 2) {
    return *reinterpret_cast<const F*>(p);
  } else {
    f32x4 lo = *reinterpret_cast<const f32x4*>(p);
    f32x4 hi = *reinterpret_cast<const f32x4*>(p + 4);
    F r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
  }
}

template <class T>
__device__ __forceinline__ void st8(T* p, const typename Frag<T>::type& v) {
  typedef typename Frag<T>::type F;
  if constexpr (sizeof(T) == 2) {
    *reinterpret_cast<F*>(p) = v;
  } else {
    *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
  }
}

template <class T>
__device__ __forceinline__ typename Frag<T>::type zero8() {
  typename Frag<T>::type r;
#pragma unroll
  for (int t = 0; t < 8; ++t) r[t] = (T)0.0f;
  return r;
}

// Four elements taken from slot e of four fragments, stored contiguously (8 or 16 bytes).
template <class T>
__device__ __forceinline__ void st4_column(T* p, const typename Frag<T>::type* rows, int e) {
  if constexpr (sizeof(T) == 2) {
    typedef T v4 __attribute__((ext_vector_type(4)));
    *reinterpret_cast<v4*>(p) = v4{rows[0][e], rows[1][e], rows[2][e], rows[3][e]};
  } else {
    *reinterpret_cast<f32x4*>(p) = f32x4{rows[0][e], rows[1][e], rows[2][e], rows[3][e]};
  }
}

// Registers 8s..8s+7 of an accumulator, rounded to T (round to nearest even).
template <class T>
__device__ __forceinline__ typename Frag<T>::type acc_slice(const f32x16& acc, int s) {
  typename Frag<T>::type r;
#pragma unroll
  for (int t = 0; t < 8; ++t) r[t] = (T)acc[8 * s + t];
  return r;
}

// Position of row m (0..15) inside a 16-row group of a transposed tile, chosen so that the
// rows one lane half contracts over (see the header comment) are 8 contiguous elements:
// lane half 0 reads rows {0..3, 8..11} at positions 0..7, lane half 1 rows {4..7, 12..15}
// at positions 8..15.  Runs of four rows starting at a multiple of 4 stay contiguous.
__device__ __forceinline__ int perm16(int m) {
  return 8 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------------------
// Swizzled 16-bit tiles in LDS.  A tile row holds HD elements (2*HD bytes, no padding); the
// 16-byte chunk c of row r is stored at chunk position c ^ swz<HD>(r).  The XOR pattern is
// chosen so that both access shapes the kernels use are free of bank conflicts on gfx950
// (measured): a b128 read of one chunk from 32 consecutive rows, and a ds_read_b64_tr_b16
// of a 4-row x 16-column block by each 16-lane group.
template <int HD>
__device__ __forceinline__ int swz(int r) {
  if constexpr (HD == 128) return 4 * (r & 3) + ((r >> 2) & 3);
  else return 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}
template <int HD>
__device__ __forceinline__ int swz_off(int r, int c) {
  return r * (2 * HD) + 16 * (c ^ swz<HD>(r));
}

typedef __attribute__((address_space(3))) char lds_char;
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

template <class T>
__device__ __forceinline__ typename Frag<T>::type lds_frag(const char* base, int byte_off) {
  return *reinterpret_cast<const typename Frag<T>::type*>(base + byte_off);
}

// Transposed fragment from a row-major 16-bit tile: two ds_read_b64_tr_b16.  In each 16-lane
// group, source lane i addresses 4 consecutive elements of row (row0 + i / 4) starting at
// column (col0 + 4 * (i % 4)); the result gives group lane i the four rows row0..row0+3 of
// column col0 + i.  The two reads cover rows row0..+3 and row0+8..+11 (the permuted row order
// of an accumulator-sourced operand, see perm16).
template <class T>
__device__ __forceinline__ typename Frag<T>::type lds_frag_tr(const char* base, int off_lo, int off_hi) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(const lds_char*)(base + off_lo));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(const lds_char*)(base + off_hi));
  const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(typename Frag<T>::type, v);
}

// 16 bytes from global memory straight into LDS (global_load_lds_dwordx4): lane l of the wave
// writes lds_wave_base + 16 * l.  lds_wave_base must be the same for the whole wave.
__device__ __forceinline__ void g2lds16(const void* src, char* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(lds_char*)lds_wave_base, 16, 0, 0);
}

__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Work-item mapping shared by the launches: workgroup ids are dispatched round-robin over
// the 8 XCDs, so id w runs on XCD w % 8.  When the independent units (kv-head groups) split
// evenly over the XCDs, give each XCD whole units so that their tiles share its L2; the
// second index ("step") then runs in dispatch order inside each XCD.
struct WorkItem { int unit; int step; };
__device__ __forceinline__ WorkItem map_work(int wg, int n_units, int units_per_xcd) {
  WorkItem r;
  if (units_per_xcd > 0) {
    const int x = wg & 7, s = wg >> 3;
    r.unit = x * units_per_xcd + s % units_per_xcd;
    r.step = s / units_per_xcd;
  } else {
    r.unit = wg % n_units;
    r.step = wg / n_units;
  }
  return r;
}

}  // namespace fab
