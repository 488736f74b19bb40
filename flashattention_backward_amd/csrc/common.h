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
typedef int i32x4 __attribute__((ext_vector_type(4)));

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
// Hazards are handled by the caller, because the compiler does not look inside the asm: a
// VALU write of an A/B operand needs two wait states before the MFMA reads it.  NOP = true
// (the default) puts them in front (`s_nop 1`); callers pass NOP = false where no vector
// instruction writes the operands (operands read from LDS, or a 16-bit P / dS fragment
// after its first MFMA).  A lone wave issues about one instruction every five cycles, an
// s_nop included, so each dropped nop shortens the step.  The build checks the compiled code
// for this hazard (asm_check.py).  Consecutive
// MFMAs accumulating into the same registers need no wait states; reads of the
// accumulators after the last MFMA must go through mma_drain() first.
template <bool NOP = true>
__device__ __forceinline__ void mma_a(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  if constexpr (NOP) asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  else asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
template <bool NOP = true>
__device__ __forceinline__ void mma_a(f32x16& acc, const f16x8& a, const f16x8& b) {
  if constexpr (NOP) asm("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  else asm("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// Wait states between the last accumulating MFMA and any other access to its registers
// (more than the 8 passes plus the read latency of a 32x32x16 MFMA).  Every accumulator is an
// operand, so no accumulating MFMA can be scheduled after the wait and no read before it.
__device__ __forceinline__ void mma_drain(f32x16 (&a)[8]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(a[0]), "+a"(a[1]), "+a"(a[2]), "+a"(a[3]),
               "+a"(a[4]), "+a"(a[5]), "+a"(a[6]), "+a"(a[7]));
}
__device__ __forceinline__ void mma_drain(f32x16 (&a)[4]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(a[0]), "+a"(a[1]), "+a"(a[2]), "+a"(a[3]));
}
__device__ __forceinline__ void mma_drain(f32x16 (&a)[2]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(a[0]), "+a"(a[1]));
}
__device__ __forceinline__ void mma_drain(f32x16 (&a)[3]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(a[0]), "+a"(a[1]), "+a"(a[2]));
}
__device__ __forceinline__ void mma_drain(f32x16 (&a)[1]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(a[0]));
}
// Two wait states after the accumulators were last written by vector instructions (their
// zero initialisation, which the compiler may emit as AGPR moves anywhere before the first
// MFMA): the asm reads and writes them, so every such write precedes it, and no inline-asm
// MFMA, which the compiler's hazard handling does not see, can follow a write too closely.
__device__ __forceinline__ void mma_ready(f32x16 (&a)[8]) {
  asm volatile("s_nop 1" : "+a"(a[0]), "+a"(a[1]), "+a"(a[2]), "+a"(a[3]), "+a"(a[4]), "+a"(a[5]),
               "+a"(a[6]), "+a"(a[7]));
}
__device__ __forceinline__ void mma_ready(f32x16 (&a)[4]) {
  asm volatile("s_nop 1" : "+a"(a[0]), "+a"(a[1]), "+a"(a[2]), "+a"(a[3]));
}
__device__ __forceinline__ void mma_ready(f32x16 (&a)[3]) {
  asm volatile("s_nop 1" : "+a"(a[0]), "+a"(a[1]), "+a"(a[2]));
}
__device__ __forceinline__ void mma_ready(f32x16 (&a)[2]) { asm volatile("s_nop 1" : "+a"(a[0]), "+a"(a[1])); }
__device__ __forceinline__ void mma_ready(f32x16 (&a)[1]) { asm volatile("s_nop 1" : "+a"(a[0])); }
// The same with the accumulator in VGPRs, as volatile asm: the statements keep their order
// relative to each other and to order_point(), which lets a loop state exactly where vector
// work goes between MFMAs.  mma_v0 starts a contraction (accumulator input 0); its output
// may not share registers with the operands (early clobber).  Reads of the result by the
// vector ALU must follow mma_vdrain().  NOP as for mma_a.
template <bool NOP = true>
__device__ __forceinline__ void mma_v(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  if constexpr (NOP) asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
  else asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
template <bool NOP = true>
__device__ __forceinline__ void mma_v(f32x16& acc, const f16x8& a, const f16x8& b) {
  if constexpr (NOP) asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
  else asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
template <bool NOP = true>
__device__ __forceinline__ void mma_v0(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  if constexpr (NOP) asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
  else asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
template <bool NOP = true>
__device__ __forceinline__ void mma_v0(f32x16& acc, const f16x8& a, const f16x8& b) {
  if constexpr (NOP) asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
  else asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
// Wait states between an mma_v result and vector-ALU reads of it (19 cover the longest
// MFMA-write to VALU-read distance of a 32x32 MFMA).
__device__ __forceinline__ void mma_vdrain(f32x16 (&a)[2]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(a[0]), "+v"(a[1]));
}
__device__ __forceinline__ void mma_vdrain(f32x16 (&a)[1]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(a[0]));
}
// Marks a point in the volatile-asm order by which x must have been computed.
__device__ __forceinline__ void order_point(float& x) { asm volatile("" : "+v"(x)); }

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
// 16-bit tiles in LDS.  Two access shapes must be free of bank conflicts on gfx950 (64 banks
// of 4 bytes, 256 bytes per cycle):
//   * a b128 read of one 16-byte chunk from 16 consecutive rows (operands that contract over
//     the head dim: 16 lanes, 256 bytes);
//   * a ds_read_b64_tr_b16 half-wave, which reads 4 consecutive rows x 64 bytes (4 chunks
//     starting at a multiple of 4) for operands that contract over rows.
// HD = 128: rows in groups of four; row b of a group starts 320 bytes (80 dwords, 16 banks
// mod 64) after row b - 1, groups are 1232 bytes (308 dwords, 4 mod 16) apart.  The four
// rows of a transposed read then cover disjoint 16-bank windows, and 16 consecutive rows
// start at 16 distinct multiples of 4 banks.  Every offset stays affine (row data are
// contiguous, whole groups shift by a constant), so unrolled loops use immediate offsets.
// HD = 64: unpadded 128-byte rows (two per bank cycle), chunk c of row r at position
// c ^ swz64(r); the row parity selects the half of the bank cycle.
__device__ __forceinline__ int swz64(int r) { return 4 * ((r >> 1) & 1) + ((r >> 2) & 3); }

template <int HD>
struct TileLayout;

template <>
struct TileLayout<128> {
  static constexpr int ROWB = 256;                 // data bytes per row
  static constexpr int SLOT = 320, GROUP = 1232;   // row stride in a group, group stride
  static constexpr int GPG = GROUP / 16;           // 16-byte granules per group (77)
  // Bytes of a tile of `rows` rows; byte shift of `n` rows (both multiples of 4).
  static constexpr int bytes(int rows) { return rows / 4 * GROUP; }
  static constexpr int rows(int n) { return n / 4 * GROUP; }
  // Byte offset of 16-byte chunk c of row r.
  __device__ static __forceinline__ int off(int r, int c) {
    return (r >> 2) * GROUP + (r & 3) * SLOT + 16 * c;
  }
  // Row and chunk whose data the granule at byte 16 gi holds; the gap granules after a row
  // (4 of them, 1 after the last row of a group) repeat chunks of that row.
  __device__ static __forceinline__ void granule(int gi, int& r, int& c) {
    const int g = gi / GPG, q = gi - g * GPG;
    const int b = min(q / (SLOT / 16), 3);
    c = q - b * (SLOT / 16);
    if (c >= 16) c -= 16;
    r = 4 * g + b;
  }
};

template <>
struct TileLayout<64> {
  static constexpr int ROWB = 128;
  static constexpr int bytes(int rows) { return rows * ROWB; }
  static constexpr int rows(int n) { return n * ROWB; }  // n a multiple of 16
  __device__ static __forceinline__ int off(int r, int c) { return r * ROWB + 16 * (c ^ swz64(r)); }
  __device__ static __forceinline__ void granule(int gi, int& r, int& c) {
    r = gi >> 3;
    c = (gi & 7) ^ swz64(r);
  }
};

// D=256: the same grouping with 512-byte rows.  Rows of a group are 576 B apart (16 banks) and
// groups 2320 B apart (580 dwords, 4 mod 16), so a b128 read of 16 rows and a transposed
// half-wave read (4 rows x 32 B) both hit distinct banks.
template <>
struct TileLayout<256> {
  static constexpr int ROWB = 512;
  static constexpr int SLOT = 576, GROUP = 2320;
  static constexpr int GPG = GROUP / 16;  // 145
  static constexpr int bytes(int rows) { return rows / 4 * GROUP; }
  static constexpr int rows(int n) { return n / 4 * GROUP; }
  __device__ static __forceinline__ int off(int r, int c) {
    return (r >> 2) * GROUP + (r & 3) * SLOT + 16 * c;
  }
  // gap granules (4 after each row, 1 after the group) repeat chunks of the row before them
  __device__ static __forceinline__ void granule(int gi, int& r, int& c) {
    const int g = gi / GPG, q = gi - g * GPG;
    const int b = min(q / (SLOT / 16), 3);
    c = q - b * (SLOT / 16);
    if (c >= 32) c -= 32;
    if (c >= 32) c -= 32;
    r = 4 * g + b;
  }
};

// Head dims 96 and 32 keep the geometry of 128 and 64: a row uses the first 12 (4) of the
// 16 (8) chunks its slot has room for, so every read is one the wider layout makes without
// bank conflicts.  The granules past a row's data load repeats of its first chunks (the
// copy fills whole tile images), which nothing reads.
template <>
struct TileLayout<96> : TileLayout<128> {
  __device__ static __forceinline__ void granule(int gi, int& r, int& c) {
    TileLayout<128>::granule(gi, r, c);
    if (c >= 12) c -= 12;
  }
};

template <>
struct TileLayout<32> : TileLayout<64> {
  __device__ static __forceinline__ void granule(int gi, int& r, int& c) {
    TileLayout<64>::granule(gi, r, c);
    if (c >= 4) c -= 4;
  }
};

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

// Direct global->LDS copies use buffer loads with the LDS bit (buffer_load_dwordx4 ... lds):
// lane l of the wave writes 16 bytes at lds_wave_base + 16 * l, read from byte offset
// voff + soff of a raw buffer resource.  The buffer form (rather than global_load_lds) keeps
// the compiler's LDS wait counting exact: a flat-encoded load that also writes LDS makes
// every later LDS wait drain to zero while it is in flight, and the prefetch here is in
// flight across whole compute steps.
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw (unstrided) buffer resource over `bytes` bytes from `base`; dword 3 is the gfx9
// default (32-bit data format, no swizzle).  Reads at offsets >= bytes return zero.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// AUX: the cache-policy bits of the load (gfx950: 1 = sc0, 2 = nt, 16 = sc1).
template <int AUX = 0>
__device__ __forceinline__ void b2lds16(rsrc_t r, unsigned voff, unsigned soff, char* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(lds_char*)lds_wave_base,
                                           16, voff, soff, 0, AUX);
}

// Copy rows [row0, row0 + ROWS) of a row-major [*, HD] tensor slice (rows 0 .. last_row,
// starting at `src`) into an LDS tile in TileLayout<HD>, with direct loads spread over `nw`
// waves (this one is wave w).  Rows past `last_row` are loaded from `last_row` (finite data;
// callers mask them).  Lanes past the tile's last granule do not load.
template <class T, int HD, int ROWS>
__device__ __forceinline__ void load_tile(char* tile, const T* src, int row0, int last_row,
                                          int w, int nw, int lane) {
  typedef TileLayout<HD> L;
  constexpr int NG = L::bytes(ROWS) / 16;  // granules in the tile
  constexpr int NI = (NG + 63) / 64;       // wave instructions (1 KB each)
  const rsrc_t r = make_rsrc(src, (unsigned)(last_row + 1) * HD * sizeof(T));
#pragma unroll
  for (int k = 0; k < (NI + 3) / 4; ++k) {
    const int q = w + nw * k;
    if (q < NI) {
      const int gi = 64 * q + lane;
      if (NG % 64 == 0 || gi < NG) {
        int rr, c;
        L::granule(gi, rr, c);
        const int row = min(row0 + rr, last_row);
        b2lds16(r, (unsigned)((row * HD + 8 * c) * sizeof(T)), 0u, tile + 1024 * q);
      }
    }
  }
}

// The same copy split into single instructions, so that a prefetch can be spread over a
// compute step instead of stalling the wave's issue at one point.  The source is a buffer
// resource over whole rows; the tile's first row is selected by a uniform byte offset
// (soffset), so each instruction needs no per-lane address arithmetic.  Rows past the end
// of the resource read as zeros.  Every wave issues KMAX instructions: where the tile has no
// instruction left for a wave, it writes to `spare` (1 KB of LDS nothing reads), which keeps
// the per-wave load count uniform for the vmcnt waits.  The tile's last instruction may
// cover fewer granules than lanes; only its valid lanes load.
template <class T, int HD, int ROWS>
struct TileDma {
  typedef TileLayout<HD> L;
  static constexpr int NG = L::bytes(ROWS) / 16;
  static constexpr int NI = (NG + 63) / 64;   // wave instructions for the whole tile
  static constexpr int KMAX = (NI + 3) / 4;   // instructions each of 4 waves issues
  static constexpr bool kSpare = 4 * KMAX > NI;
  static constexpr int TAIL = NG % 64;        // valid lanes of the last instruction (0: all)
  int w;
  unsigned src_off[KMAX];  // byte offset of this lane's granule of instruction k from row 0
  __device__ __forceinline__ void init(int wave, int lane) {
    w = wave;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      int r, c;
      L::granule(64 * (w + 4 * k) + lane, r, c);
      src_off[k] = (unsigned)((r * HD + 8 * c) * sizeof(T));
    }
  }
  // Instruction k of this wave: the tile whose first row starts at byte `soff` of `r`.
  __device__ __forceinline__ void issue(int k, char* tile, rsrc_t r, unsigned soff, char* spare,
                                        int lane) const {
    const int q = w + 4 * k;
    if (kSpare && 4 * k + 3 >= NI) {  // instruction k does not exist for every wave
      char* dst = q < NI ? tile + 1024 * q : spare;
      if (TAIL == 0 || q != NI - 1 || lane < TAIL) b2lds16(r, src_off[k], soff, dst);
    } else if (TAIL != 0 && 4 * k + 3 >= NI - 1) {
      if (q != NI - 1 || lane < TAIL) b2lds16(r, src_off[k], soff, tile + 1024 * q);
    } else {
      b2lds16(r, src_off[k], soff, tile + 1024 * q);
    }
  }
};

__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Workgroup barrier for the staging loops.  __syncthreads() also waits for every outstanding
// global memory operation of the wave (vmcnt(0)), which would stall on the tiles being
// prefetched; here each wave first drains only its LDS reads (so no wave can still be reading
// a buffer that the next step's prefetch overwrites) and the caller waits explicitly for the
// tile the next step needs (wait_vm_le).  The asm blocks with a memory clobber stop the
// compiler from moving LDS accesses across the barrier; the LDS wait is issued through the
// builtin so that the compiler's own wait-count tracking knows every earlier LDS read has
// completed (it does not look inside asm text).
__device__ __forceinline__ void barrier_lds() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt at "no wait"
  asm volatile("s_barrier" ::: "memory");
}

// Wait until at most N vector-memory operations of this wave are outstanding (loads return
// in order, so everything issued before the last N has landed).  gfx9 s_waitcnt encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4] and lgkmcnt [11:8] left at "no wait".
template <int N>
__device__ __forceinline__ void wait_vm_le() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}



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

// Keys a query row may attend (top-left indices): [lo(m), hi(m)], empty when lo > hi.
// Every key is below Sk; with the causal mask no key is past the row itself; with a window of
// `win` keys (win > 0) a key is more than m - win and, without the causal mask, less than
// m + win.  win = 0 means no window (the host passes 0 for windows too wide to cut anything).
// Both bounds are non-decreasing in m, so a block of rows [m_a, m_b] sees keys within
// [lo(m_a), hi(m_b)], and sees every key of [n_a, n_b] iff lo(m_b) <= n_a and hi(m_a) >= n_b.
struct KeyRange {
  int Sk, causal, win;
  __device__ __forceinline__ int lo(int m) const { return win > 0 ? max(m - win + 1, 0) : 0; }
  __device__ __forceinline__ int hi(int m) const {
    return min(Sk - 1, causal ? m : (win > 0 ? m + win - 1 : Sk - 1));
  }
  // Query rows that may attend key n (n < Sk), unclamped: [rows_lo(n), rows_hi(n)].
  __device__ __forceinline__ int rows_lo(int n) const {
    return causal ? n : (win > 0 ? n - win + 1 : -(1 << 29));
  }
  __device__ __forceinline__ int rows_hi(int n) const { return win > 0 ? n + win - 1 : (1 << 29); }
};

}  // namespace fab
