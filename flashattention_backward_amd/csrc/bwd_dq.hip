// The generic path for fp32 inputs (v_mfma_f32_32x32x2f32: fp32 products and sums) at head
// dims 32, 64, 96 and 128; bf16 and fp16 inputs use the tiled dQ kernel of bwd16.hip.
//
// Main backward step for dQ, query-tile outer (the dQ pass of rustytorch's
// rtx-flash-metal-attention backward.rs, which dispatches one threadgroup per block of
// queries per (batch, head)).  A workgroup owns BM = 128 query rows of one (batch, head);
// wave w (of 4) owns rows [32w, 32w + 32) and keeps their Q and dO operand fragments, LSE
// and D in registers.  It walks the key tiles that the causal mask lets those rows see and
// recomputes, per tile of BN = 64 keys,
//   S^T = K Q^T,  P^T = exp2(S^T * scale*log2e - LSE*log2e),  dP^T = V dO^T,
//   dS^T = P^T (dP^T - D),  dQ += dS K           (dQ takes the factor `scale` at the end)
// Computing the transposed scores puts one query row in each lane, so LSE and D are plain
// per-lane scalars and dS^T's registers already form the A operand of dQ = dS K.  K is
// staged twice in LDS: row-major (operand of S^T) and transposed with rows permuted by
// perm16 (operand of dS K).  Every dQ element is written once: no atomics, deterministic.
#include "common.h"
#include "launch.h"

namespace fab {

template <class T, int HD>
struct DqCfg {
  static constexpr int NW = 4;
  static constexpr int BM = 32 * NW;  // query rows per workgroup
  static constexpr int BN = 64;       // keys per step
  static constexpr int ES = sizeof(T);
  static constexpr int PAD = 16 / ES;
  static constexpr int LDR = HD + PAD;  // row-major [BN][LDR]
  static constexpr int LDT = BN + PAD;  // transposed [HD][LDT]
  static constexpr int SZ_R = BN * LDR;
  static constexpr int SZ_T = HD * LDT;
  static constexpr int LDS_BYTES = (2 * SZ_R + SZ_T) * ES;
};

template <class T, int HD>
__global__ __launch_bounds__(256) void bwd_dq_kernel(const BwdParams p) {
  typedef DqCfg<T, HD> C;
  typedef typename Frag<T>::type F;
  constexpr int BM = C::BM, BN = C::BN, LDR = C::LDR, LDT = C::LDT;
  constexpr int NC = HD / 16;
  constexpr int NDB = HD / 32;
  constexpr int NNB = BN / 32;

  __shared__ __attribute__((aligned(16))) char smem[C::LDS_BYTES];
  T* sK = reinterpret_cast<T*>(smem);
  T* sV = sK + C::SZ_R;
  T* sKt = sV + C::SZ_R;

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, hl = lane >> 5, c32 = lane & 31;
  const int Sq = p.Sq, Sk = p.Sk;
  const bool causal = p.causal != 0;
  const int G = p.H / p.H_kv;
  const int n_qt = (Sq + BM - 1) / BM;

  // unit = (b, kv head); step enumerates (query tile, head in group), heaviest tile first.
  const WorkItem wi = map_work(blockIdx.x, p.n_units, p.units_per_xcd);
  const int b = wi.unit / p.H_kv, g = wi.unit % p.H_kv;
  const int hq = g * G + wi.step % G;
  const int tq = wi.step / G;
  const int it = causal ? n_qt - 1 - tq : tq;
  const int m0 = it * BM;
  const int mw0 = m0 + 32 * w;
  const int m = mw0 + c32;  // this lane's query row

  const size_t q_off = (size_t)(b * p.H + hq) * Sq;
  const size_t kv_off = (size_t)(b * p.H_kv + g) * Sk * HD;
  const T* Qg = (const T*)p.q + q_off * HD;
  const T* dOg = (const T*)p.dO + q_off * HD;
  const T* Kg = (const T*)p.k + kv_off;
  const T* Vg = (const T*)p.v + kv_off;

  F qf[NC], dof[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (m < Sq) {
      qf[c] = ld8(Qg + (size_t)m * HD + 16 * c + 8 * hl);
      dof[c] = ld8(dOg + (size_t)m * HD + 16 * c + 8 * hl);
    } else {
      qf[c] = zero8<T>();
      dof[c] = zero8<T>();
    }
  }
  const float* Stg = p.stats + (size_t)(b * p.H + hq) * p.Sq_pad * 2;
  const float lse2 = m < Sq ? Stg[2 * m] : __builtin_inff();
  const float dl = m < Sq ? Stg[2 * m + 1] : 0.f;

  f32x16 dq[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dq[db] = f32x16{};

  // key tiles holding a key some row of this tile may attend
  const KeyRange kr{Sk, p.causal, p.win};
  const int k_lo = kr.lo(m0), k_hi = kr.hi(min(m0 + BM, Sq) - 1);
  const int j_begin = k_lo / BN;
  const int j_end = k_hi >= k_lo ? k_hi / BN + 1 : j_begin;

  for (int j = j_begin; j < j_end; ++j) {
    const int n0 = j * BN;
    __syncthreads();
    {
      constexpr int NCH = HD / 8, NRQ = BN / 4, UNITS = 2 * NRQ * NCH;
      for (int u = tid; u < UNITS; u += 256) {
        const int tsel = u / (NRQ * NCH);  // 0: K (row-major + transposed), 1: V
        const int rem = u % (NRQ * NCH);
        const int rq = rem / NCH, ch = rem % NCH;
        const T* src = tsel ? Vg : Kg;
        T* dR = tsel ? sV : sK;
        F rows[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int n = n0 + 4 * rq + r;
          rows[r] = n < Sk ? ld8(src + (size_t)n * HD + 8 * ch) : zero8<T>();
          st8(dR + (4 * rq + r) * LDR + 8 * ch, rows[r]);
        }
        if (tsel == 0) {
          const int nr = 4 * rq;
          const int pos = (nr & ~15) + perm16(nr & 15);
#pragma unroll
          for (int e = 0; e < 8; ++e) st4_column<T>(sKt + (8 * ch + e) * LDT + pos, rows, e);
        }
      }
    }
    __syncthreads();

    if (kr.hi(mw0 + 31) < n0 || kr.lo(mw0) > n0 + BN - 1) continue;  // no row of this wave sees these keys

    f32x16 St[NNB], dPt[NNB];
#pragma unroll
    for (int nb = 0; nb < NNB; ++nb) {
      St[nb] = f32x16{};
      dPt[nb] = f32x16{};
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int nb = 0; nb < NNB; ++nb) {
        const int off = (32 * nb + c32) * LDR + 16 * c + 8 * hl;
        mma(St[nb], ld8(sK + off), qf[c]);
        mma(dPt[nb], ld8(sV + off), dof[c]);
      }
    }

    const bool need_mask = kr.hi(mw0) < n0 + BN - 1 || kr.lo(mw0 + 31) > n0;
#pragma unroll
    for (int nb = 0; nb < NNB; ++nb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pv = fast_exp2(St[nb][r] * p.scale_log2 - lse2);
        if (need_mask) {
          const int n = n0 + 32 * nb + 8 * (r >> 2) + 4 * hl + (r & 3);
          if (n < kr.lo(m) || n > kr.hi(m)) pv = 0.f;
        }
        dPt[nb][r] = pv * (dPt[nb][r] - dl);
      }
    }

#pragma unroll
    for (int nb = 0; nb < NNB; ++nb) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const F da = acc_slice<T>(dPt[nb], ks);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int off = (32 * db + c32) * LDT + 32 * nb + 16 * ks + 8 * hl;
          mma(dq[db], da, ld8(sKt + off));
        }
      }
    }
  }

  // Epilogue: accumulator rows are this wave's query rows, columns the head dim.
  T* dQg = (T*)p.dq + q_off * HD;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int mr = mw0 + 8 * (r >> 2) + 4 * hl + (r & 3);
      if (mr < Sq) dQg[(size_t)mr * HD + 32 * db + c32] = (T)(dq[db][r] * p.scale);
    }
  }
}

template <class T, int HD>
static hipError_t go(const BwdParams& p, hipStream_t s, LaunchInfo* info) {
  typedef DqCfg<T, HD> C;
  const int n_qt = (p.Sq + C::BM - 1) / C::BM;
  const int grid = p.n_units * (p.H / p.H_kv) * n_qt;
  if (info) *info = LaunchInfo{"bwd_dq", grid, 256, C::LDS_BYTES};
  hipLaunchKernelGGL((bwd_dq_kernel<T, HD>), dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

// fp32 inputs only; bf16 and fp16 inputs run the tiled dQ kernel of bwd16.hip.
hipError_t launch_bwd_dq(const BwdParams& p, int dt, int hd, hipStream_t s, LaunchInfo* info) {
  (void)dt;
  switch (hd) {
    case 32: return go<float, 32>(p, s, info);
    case 64: return go<float, 64>(p, s, info);
    case 96: return go<float, 96>(p, s, info);
    default: return go<float, 128>(p, s, info);
  }
}

}  // namespace fab
