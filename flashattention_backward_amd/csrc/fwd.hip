// The generic path: fp32 inputs (v_mfma_f32_32x32x2f32: fp32 products and sums) at head dims
// 32, 64, 96 and 128; bf16 and fp16 inputs use the tiled forward of fwd16.hip.
//
// Supporting forward: O = softmax(scale Q K^T over the allowed keys) V and the row LSE
// (natural log), which the backward consumes (boostr autograd_attention.rs,
// var_flash_attention: the forward returns (output, lse) and the lse stays internal to the
// backward).  Query-tile outer with an online softmax over key tiles.
//
// A workgroup owns BM = 128 query rows of one (batch, head); wave w owns rows
// [32w, 32w + 32) and keeps their Q fragments in registers.  Per key tile of BN = 64 it
// computes S^T = K Q^T (one query row per lane, so the running max and sum are per-lane
// scalars combined with the other lane half), then O^T += V^T P^T with P^T's registers as
// the B operand and V staged transposed in LDS with rows permuted by perm16.
#include "common.h"
#include "launch.h"

namespace fab {

template <class T, int HD>
struct FwdCfg {
  static constexpr int NW = 4;
  static constexpr int BM = 32 * NW;
  static constexpr int BN = 64;
  static constexpr int ES = sizeof(T);
  static constexpr int PAD = 16 / ES;
  static constexpr int LDR = HD + PAD;  // K row-major [BN][LDR]
  static constexpr int LDT = BN + PAD;  // V transposed [HD][LDT]
  static constexpr int SZ_R = BN * LDR;
  static constexpr int SZ_T = HD * LDT;
  static constexpr int LDS_BYTES = (SZ_R + SZ_T) * ES;
};

template <class T, int HD>
__global__ __launch_bounds__(256) void fwd_kernel(const FwdParams p) {
  typedef FwdCfg<T, HD> C;
  typedef typename Frag<T>::type F;
  constexpr int BM = C::BM, BN = C::BN, LDR = C::LDR, LDT = C::LDT;
  constexpr int NC = HD / 16;
  constexpr int NDB = HD / 32;
  constexpr int NNB = BN / 32;

  __shared__ __attribute__((aligned(16))) char smem[C::LDS_BYTES];
  T* sK = reinterpret_cast<T*>(smem);
  T* sVt = sK + C::SZ_R;

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, hl = lane >> 5, c32 = lane & 31;
  const int Sq = p.Sq, Sk = p.Sk;
  const bool causal = p.causal != 0;
  const int G = p.H / p.H_kv;
  const int n_qt = (Sq + BM - 1) / BM;

  const WorkItem wi = map_work(blockIdx.x, p.n_units, p.units_per_xcd);
  const int b = wi.unit / p.H_kv, g = wi.unit % p.H_kv;
  const int hq = g * G + wi.step % G;
  const int tq = wi.step / G;
  const int it = causal ? n_qt - 1 - tq : tq;
  const int m0 = it * BM;
  const int mw0 = m0 + 32 * w;
  const int m = mw0 + c32;

  const size_t q_off = (size_t)(b * p.H + hq) * Sq;
  const size_t kv_off = (size_t)(b * p.H_kv + g) * Sk * HD;
  const T* Qg = (const T*)p.q + q_off * HD;
  const T* Kg = (const T*)p.k + kv_off;
  const T* Vg = (const T*)p.v + kv_off;

  F qf[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c)
    qf[c] = m < Sq ? ld8(Qg + (size_t)m * HD + 16 * c + 8 * hl) : zero8<T>();

  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
  float mrun = -1e30f;  // running max of the log2-domain scores of row m (finite start)
  float lsum = 0.f;     // this lane half's share of the row sum

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
        const int tsel = u / (NRQ * NCH);  // 0: K row-major, 1: V transposed
        const int rem = u % (NRQ * NCH);
        const int rq = rem / NCH, ch = rem % NCH;
        const T* src = tsel ? Vg : Kg;
        F rows[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int n = n0 + 4 * rq + r;
          rows[r] = n < Sk ? ld8(src + (size_t)n * HD + 8 * ch) : zero8<T>();
        }
        if (tsel == 0) {
#pragma unroll
          for (int r = 0; r < 4; ++r) st8(sK + (4 * rq + r) * LDR + 8 * ch, rows[r]);
        } else {
          const int nr = 4 * rq;
          const int pos = (nr & ~15) + perm16(nr & 15);
#pragma unroll
          for (int e = 0; e < 8; ++e) st4_column<T>(sVt + (8 * ch + e) * LDT + pos, rows, e);
        }
      }
    }
    __syncthreads();

    if (kr.hi(mw0 + 31) < n0 || kr.lo(mw0) > n0 + BN - 1) continue;  // no row of this wave sees these keys

    f32x16 St[NNB];
#pragma unroll
    for (int nb = 0; nb < NNB; ++nb) St[nb] = f32x16{};
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int nb = 0; nb < NNB; ++nb)
        mma(St[nb], ld8(sK + (32 * nb + c32) * LDR + 16 * c + 8 * hl), qf[c]);
    }

    const bool need_mask = kr.hi(mw0) < n0 + BN - 1 || kr.lo(mw0 + 31) > n0;
    float mx = -__builtin_inff();
#pragma unroll
    for (int nb = 0; nb < NNB; ++nb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = St[nb][r] * p.scale_log2;
        if (need_mask) {
          const int n = n0 + 32 * nb + 8 * (r >> 2) + 4 * hl + (r & 3);
          if (n < kr.lo(m) || n > kr.hi(m)) x = -__builtin_inff();
        }
        St[nb][r] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(mrun, mx);
    const float alpha = fast_exp2(mrun - mnew);
    float ps = 0.f;
#pragma unroll
    for (int nb = 0; nb < NNB; ++nb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = fast_exp2(St[nb][r] - mnew);
        St[nb][r] = pv;
        ps += pv;
      }
    }
    lsum = lsum * alpha + ps;
    mrun = mnew;
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] *= alpha;

#pragma unroll
    for (int nb = 0; nb < NNB; ++nb) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const F pb = acc_slice<T>(St[nb], ks);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          mma(o[db], ld8(sVt + (32 * db + c32) * LDT + 32 * nb + 16 * ks + 8 * hl), pb);
      }
    }
  }

  const float ltot = lsum + __shfl_xor(lsum, 32);
  if (m < Sq) {
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;  // a row with no key: O = 0, LSE = -inf
    T* Og = (T*)p.o + (q_off + m) * HD;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * db + 8 * q4 + 4 * hl;
        if constexpr (sizeof(T) == 2) {
          typedef T v4 __attribute__((ext_vector_type(4)));
          *reinterpret_cast<v4*>(Og + d) =
              v4{(T)(o[db][4 * q4] * inv), (T)(o[db][4 * q4 + 1] * inv),
                 (T)(o[db][4 * q4 + 2] * inv), (T)(o[db][4 * q4 + 3] * inv)};
        } else {
          *reinterpret_cast<f32x4*>(Og + d) =
              f32x4{o[db][4 * q4] * inv, o[db][4 * q4 + 1] * inv, o[db][4 * q4 + 2] * inv,
                    o[db][4 * q4 + 3] * inv};
        }
      }
    }
    if (hl == 0) p.lse[q_off + m] = (mrun + __log2f(ltot)) * kLn2;
  }
}

template <class T, int HD>
static hipError_t go(const FwdParams& p, hipStream_t s, LaunchInfo* info) {
  typedef FwdCfg<T, HD> C;
  const int n_qt = (p.Sq + C::BM - 1) / C::BM;
  const int grid = p.n_units * (p.H / p.H_kv) * n_qt;
  if (info) *info = LaunchInfo{"fwd", grid, 256, C::LDS_BYTES};
  hipLaunchKernelGGL((fwd_kernel<T, HD>), dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

// fp32 inputs only; bf16 and fp16 inputs run the tiled forward of fwd16.hip.
hipError_t launch_fwd(const FwdParams& p, int dt, int hd, hipStream_t s, LaunchInfo* info) {
  (void)dt;
  switch (hd) {
    case 32: return go<float, 32>(p, s, info);
    case 64: return go<float, 64>(p, s, info);
    case 96: return go<float, 96>(p, s, info);
    default: return go<float, 128>(p, s, info);
  }
}

}  // namespace fab
