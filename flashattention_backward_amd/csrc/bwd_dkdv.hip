// The generic path: fp32 inputs (v_mfma_f32_32x32x2f32: fp32 products and sums) at head dims
// 32, 64, 96 and 128; bf16 and fp16 inputs use the tiled dK/dV kernel of bwd16.hip.
//
// Main backward step for dK and dV (boostr flash_bwd.rs, "Step 2: Main backward kernel",
// whose launch gives every workgroup one tile of keys: grid (batch*heads, ceil(Sk/BLOCK_N))
// with K, V, Q and dO tiles in shared memory).
//
// KV-tile outer: a workgroup owns BN = 128 keys of one (batch, kv head) and keeps their K
// and V operand fragments in registers for its whole life.  It walks every query head of
// the kv-head group and every query tile that the causal mask lets reach its keys, so the
// group sum of dK and dV happens in registers and each output row is written exactly once.
// Per query tile it recomputes
//   S = Q K^T,  P = exp2(S * scale*log2e - LSE*log2e),  dP = dO V^T,  dS = P (dP - D),
//   dV += P^T dO,  dK += dS^T Q            (dK takes the factor `scale` at the end)
// with the four contractions on the matrix cores.  dQ is produced by the separate
// query-outer kernel (bwd_dq.hip), so no atomics are needed.
//
// Wave w (of 4) owns keys [32w, 32w + 32) of the tile.  Q and dO tiles are staged in LDS
// twice: row-major (operand of S and dP, which contract over the head dim) and transposed
// with rows permuted by perm16 (operand of dV and dK, which contract over query rows held
// "in lane" by the S / dP accumulators).
#include "common.h"
#include "launch.h"

namespace fab {

template <class T, int HD>
struct DkdvCfg {
  static constexpr int NW = 4;
  static constexpr int BN = 32 * NW;                   // keys per workgroup
  static constexpr int BM = sizeof(T) == 4 ? 32 : 64;  // query rows per step
  static constexpr int ES = sizeof(T);
  static constexpr int PAD = 16 / ES;                  // +16 bytes per LDS row
  static constexpr int LDR = HD + PAD;                 // row-major tile [BM][LDR]
  static constexpr int LDT = BM + PAD;                 // transposed tile [HD][LDT]
  static constexpr int SZ_R = BM * LDR;
  static constexpr int SZ_T = HD * LDT;
  static constexpr int LDS_BYTES = (2 * SZ_R + 2 * SZ_T) * ES + 2 * BM * 4;
};

template <class T, int HD>
__global__ __launch_bounds__(256) void bwd_dkdv_kernel(const BwdParams p) {
  typedef DkdvCfg<T, HD> C;
  typedef typename Frag<T>::type F;
  constexpr int BM = C::BM, BN = C::BN, LDR = C::LDR, LDT = C::LDT;
  constexpr int NC = HD / 16;   // 16-wide slices of the head dim
  constexpr int NDB = HD / 32;  // 32-wide blocks of the head dim
  constexpr int NMB = BM / 32;  // 32-row blocks of the query tile

  __shared__ __attribute__((aligned(16))) char smem[C::LDS_BYTES];
  T* sQ = reinterpret_cast<T*>(smem);
  T* sdO = sQ + C::SZ_R;
  T* sQt = sdO + C::SZ_R;
  T* sdOt = sQt + C::SZ_T;
  float* sL = reinterpret_cast<float*>(sdOt + C::SZ_T);
  float* sD = sL + BM;

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, hl = lane >> 5, c32 = lane & 31;

  const WorkItem wi = map_work(blockIdx.x, p.n_units, p.units_per_xcd);
  const int b = wi.unit / p.H_kv, g = wi.unit % p.H_kv;
  const int n0 = wi.step * BN;
  const int G = p.H / p.H_kv;
  const int Sq = p.Sq, Sk = p.Sk;

  const size_t kv_off = (size_t)(b * p.H_kv + g) * Sk * HD;
  const T* Kg = (const T*)p.k + kv_off;
  const T* Vg = (const T*)p.v + kv_off;

  // This lane's key row and its K, V fragments (B operands of S = Q K^T and dP = dO V^T).
  const int nw0 = n0 + 32 * w;
  const int nrow = nw0 + c32;
  F kf[NC], vf[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (nrow < Sk) {
      kf[c] = ld8(Kg + (size_t)nrow * HD + 16 * c + 8 * hl);
      vf[c] = ld8(Vg + (size_t)nrow * HD + 16 * c + 8 * hl);
    } else {
      kf[c] = zero8<T>();
      vf[c] = zero8<T>();
    }
  }

  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }

  // query tiles holding a row that may attend one of these keys (rows [r_lo, r_hi])
  const KeyRange kr{Sk, p.causal, p.win};
  const int r_lo = max(kr.rows_lo(n0), 0), r_hi = min(kr.rows_hi(min(n0 + BN, Sk) - 1), Sq - 1);
  const int i_first = r_lo / BM;
  const int i_end = r_hi >= r_lo ? r_hi / BM + 1 : i_first;

  for (int hh = 0; hh < G; ++hh) {
    const int hq = g * G + hh;
    const size_t q_off = (size_t)(b * p.H + hq) * Sq;
    const T* Qg = (const T*)p.q + q_off * HD;
    const T* dOg = (const T*)p.dO + q_off * HD;
    const float* Stg = p.stats + (size_t)(b * p.H + hq) * p.Sq_pad * 2;

    for (int it = i_first; it < i_end; ++it) {
      const int m0 = it * BM;
      __syncthreads();  // every wave is done reading the previous tile
      {
        // Stage Q and dO: a unit is 4 rows x 8 columns of one tensor.
        constexpr int NCH = HD / 8, NRQ = BM / 4, UNITS = 2 * NRQ * NCH;
        for (int u = tid; u < UNITS; u += 256) {
          const int tsel = u / (NRQ * NCH);
          const int rem = u % (NRQ * NCH);
          const int rq = rem / NCH, ch = rem % NCH;
          const T* src = tsel ? dOg : Qg;
          T* dR = tsel ? sdO : sQ;
          T* dT = tsel ? sdOt : sQt;
          F rows[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int m = m0 + 4 * rq + r;
            rows[r] = m < Sq ? ld8(src + (size_t)m * HD + 8 * ch) : zero8<T>();
            st8(dR + (4 * rq + r) * LDR + 8 * ch, rows[r]);
          }
          const int mr = 4 * rq;
          const int pos = (mr & ~15) + perm16(mr & 15);
#pragma unroll
          for (int e = 0; e < 8; ++e) st4_column<T>(dT + (8 * ch + e) * LDT + pos, rows, e);
        }
        for (int t = tid; t < BM; t += 256) {
          const int m = m0 + t;
          sL[t] = m < Sq ? Stg[2 * m] : __builtin_inff();
          sD[t] = m < Sq ? Stg[2 * m + 1] : 0.f;
        }
      }
      __syncthreads();

      // Keys of this wave that no query row of the tile may attend: nothing to add.
      if (kr.hi(m0 + BM - 1) < nw0 || kr.lo(m0) > nw0 + 31) continue;

      f32x16 S[NMB], dP[NMB];
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
        S[mb] = f32x16{};
        dP[mb] = f32x16{};
      }
#pragma unroll
      for (int c = 0; c < NC; ++c) {
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) {
          const int off = (32 * mb + c32) * LDR + 16 * c + 8 * hl;
          mma(S[mb], ld8(sQ + off), kf[c]);
          mma(dP[mb], ld8(sdO + off), vf[c]);
        }
      }

      const bool need_mask = kr.hi(m0) < nw0 + 31 || kr.lo(m0 + BM - 1) > nw0;
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ml = 32 * mb + 8 * (r >> 2) + 4 * hl + (r & 3);
          float pv = fast_exp2(S[mb][r] * p.scale_log2 - sL[ml]);
          if (need_mask) {
            const int mg = m0 + ml;
            if (nrow < kr.lo(mg) || nrow > kr.hi(mg)) pv = 0.f;
          }
          S[mb][r] = pv;
          dP[mb][r] = pv * (dP[mb][r] - sD[ml]);
        }
      }

#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const F pa = acc_slice<T>(S[mb], ks);
          const F da = acc_slice<T>(dP[mb], ks);
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const int off = (32 * db + c32) * LDT + 32 * mb + 16 * ks + 8 * hl;
            mma(dv[db], pa, ld8(sdOt + off));
            mma(dk[db], da, ld8(sQt + off));
          }
        }
      }
    }
  }

  // Epilogue: accumulator rows are this wave's keys, columns the head dim.
  T* dKg = (T*)p.dk + kv_off;
  T* dVg = (T*)p.dv + kv_off;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int n = nw0 + 8 * (r >> 2) + 4 * hl + (r & 3);
      if (n < Sk) {
        dKg[(size_t)n * HD + 32 * db + c32] = (T)(dk[db][r] * p.scale);
        dVg[(size_t)n * HD + 32 * db + c32] = (T)dv[db][r];
      }
    }
  }
}

template <class T, int HD>
static hipError_t go(const BwdParams& p, hipStream_t s, LaunchInfo* info) {
  typedef DkdvCfg<T, HD> C;
  const int n_kt = (p.Sk + C::BN - 1) / C::BN;
  const int grid = p.n_units * n_kt;
  if (info) *info = LaunchInfo{"bwd_dkdv", grid, 256, C::LDS_BYTES};
  hipLaunchKernelGGL((bwd_dkdv_kernel<T, HD>), dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

// fp32 inputs only; bf16 and fp16 inputs run the tiled dK/dV kernel of bwd16.hip.
hipError_t launch_bwd_dkdv(const BwdParams& p, int dt, int hd, hipStream_t s, LaunchInfo* info) {
  (void)dt;
  switch (hd) {
    case 32: return go<float, 32>(p, s, info);
    case 64: return go<float, 64>(p, s, info);
    case 96: return go<float, 96>(p, s, info);
    default: return go<float, 128>(p, s, info);
  }
}

}  // namespace fab
