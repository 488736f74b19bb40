// Host-side launch interface between the C ABI (api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>

namespace fab {

enum Dt { kF32 = 0, kF16 = 1, kBF16 = 2 };

constexpr float kLog2eHost = 1.4426950408889634f;

struct PreParams {
  const void* dO;
  const void* o;
  float* delta;
  long long rows;  // B * H * Sq
};

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, H_kv, Sq, Sk;
  int causal;
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
  const float* lse;
  const float* delta;
  void* dq;
  void* dk;
  void* dv;
  int B, H, H_kv, Sq, Sk;
  int causal;
  float scale;
  float scale_log2;
  int n_units;
  int units_per_xcd;
};

struct LaunchInfo {
  const char* name;
  int grid, block, lds_bytes;
};

hipError_t launch_preprocess(const PreParams& p, int dt, int hd, hipStream_t s, LaunchInfo* info);
hipError_t launch_fwd(const FwdParams& p, int dt, int hd, hipStream_t s, LaunchInfo* info);
hipError_t launch_bwd_dkdv(const BwdParams& p, int dt, int hd, hipStream_t s, LaunchInfo* info);
hipError_t launch_bwd_dq(const BwdParams& p, int dt, int hd, hipStream_t s, LaunchInfo* info);

}  // namespace fab
