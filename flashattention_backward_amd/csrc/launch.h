// Host-side launch interface between the C ABI (api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>

namespace fab {

enum Dt { kF32 = 0, kF16 = 1, kBF16 = 2 };

constexpr float kLog2eHost = 1.4426950408889634f;

// Per-row statistics the backward kernels consume, written by the preprocess:
// stats[(b*H + h) * Sq_pad + i] = {LSE[b,h,i] * log2(e), D[b,h,i]}, Sq_pad = Sq rounded up to
// kStatsRows; padding rows hold {+inf, 0} so that they contribute nothing.
constexpr int kStatsRows = 64;
inline int stats_rows(int Sq) { return (Sq + kStatsRows - 1) / kStatsRows * kStatsRows; }

// Rows and keys a dS slab covers: every row block and key block either step-2 kernel may
// touch (query tiles of up to 128 rows, key tiles of up to 256 keys).
inline long long ds_rows(int Sq) { return (Sq + 127LL) / 128 * 128; }
inline long long ds_keys(int Sk) { return (Sk + 255LL) / 256 * 256; }

struct PreParams {
  const void* dO;
  const void* o;
  const float* lse;
  float* stats;
  int BH, Sq, Sq_pad;
};

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, H_kv, Sq, Sk;
  int causal;
  int win;           // sliding window in keys, 0 = none (see KeyRange in common.h)
  float scale;       // softmax scale
  float scale_log2;  // scale * log2(e)
  int n_units;       // B * H_kv
  int units_per_xcd; // > 0 when n_units % 8 == 0
};

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* dO;
  const float* stats;  // see PreParams
  // Set on the dQ kernel of fab_bwd (16-bit path): the kernel forms its rows' statistics
  // itself from o and lse, as the preprocess would, and writes them to stats_out for the
  // dK/dV kernel that follows.  Null otherwise (the statistics come from the preprocess).
  const void* o;
  const float* lse;
  float* stats_out;
  void* dq;
  void* dk;
  void* dv;
  // Stored dS (16-bit path; null when dQ recomputes dS): the dK/dV kernel writes every dS
  // fragment it forms, the dQ kernel that follows reads them back.  Per (b, h) a slab of
  // ds_slab bytes: 1 KB fragments of 32 keys x 16 query rows (see bwd16.hip), the fragment of
  // row block r (rows 16 r ..) and key block k (keys 32 k ..) at byte
  // ((r / 8 * ds_nk32 + k) * 8 + r % 8) * 1024 of the slab.
  void* ds;
  unsigned ds_slab;  // bytes per (b, h): ds_rows(Sq) * ds_keys(Sk) * 2
  int ds_nk32;       // key blocks per slab row: ds_keys(Sk) / 32
  int B, H, H_kv, Sq, Sk, Sq_pad;
  int causal;
  int win;            // sliding window in keys, 0 = none (see KeyRange in common.h)
  float scale;
  float scale_log2;  // scale * log2(e), never zero or subnormal
  float mask_s;      // a score replaced by mask_s gets exponent mask_s * scale_log2 = -inf
  int n_units;
  int units_per_xcd;
};

struct LaunchInfo {
  const char* name;
  int grid, block, lds_bytes;
};

hipError_t launch_preprocess(const PreParams& p, int dt, int hd, hipStream_t s, LaunchInfo* info);
// fp32 inputs: launch_fwd, launch_bwd_dkdv, launch_bwd_dq; bf16/fp16: the *16 launchers.
hipError_t launch_fwd(const FwdParams& p, int dt, int hd, hipStream_t s, LaunchInfo* info);
hipError_t launch_fwd16(const FwdParams& p, int dt, int hd, hipStream_t s, LaunchInfo* info);
hipError_t launch_bwd_dkdv(const BwdParams& p, int dt, int hd, hipStream_t s, LaunchInfo* info);
hipError_t launch_bwd_dq(const BwdParams& p, int dt, int hd, hipStream_t s, LaunchInfo* info);
hipError_t launch_bwd_dkdv16(const BwdParams& p, int dt, int hd, hipStream_t s, LaunchInfo* info);
hipError_t launch_bwd_dq16(const BwdParams& p, int dt, int hd, hipStream_t s, LaunchInfo* info);
// Both recomputing step-2 kernels in one launch (row statistics from a preprocess first), and
// whether the problem is small enough for it (the two grids together fit the device at once).
bool bwd_small16_fits(const BwdParams& p, int hd);
hipError_t launch_bwd_small16(const BwdParams& p, int dt, int hd, hipStream_t s, LaunchInfo* info);
// dQ = scale * dS K from the dS fragments the dK/dV kernel stored (p.ds set).
hipError_t launch_bwd_dq_ds16(const BwdParams& p, int dt, int hd, hipStream_t s, LaunchInfo* info);

}  // namespace fab
