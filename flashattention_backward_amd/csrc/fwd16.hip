// Supporting forward for 16-bit inputs, tiled for gfx950: O = softmax(scale Q K^T over the
// allowed keys) V and the row LSE (natural log), which the backward consumes (boostr
// autograd_attention.rs, var_flash_attention: the forward returns (output, lse) and the lse
// stays internal to the backward).  Query-tile outer with an online softmax over key tiles.
//
// A workgroup owns BM = 128 query rows of one (batch, head) and walks the key tiles the
// causal mask lets it see; wave w owns rows [32 w, 32 w + 32) with their Q fragments in
// registers.  Per tile of BN = 64 keys: S^T = K Q^T (one query row per lane, keys in the
// accumulator registers), the online softmax per lane, then O^T += V^T P^T with P^T taken
// straight from the score registers as the B operand and V^T read from the row-major V tile
// with the LDS transpose read.  One query row per lane in both S^T and O^T, so the running
// max, the rescale factor and the final normalisation are per-lane scalars.
//
// K and V tiles arrive by direct-to-LDS buffer loads into a double buffer (the prefetch of
// the next tile is spread over the S MFMAs); up to head dim 128, 2 x 2 tiles of 64 rows fit
// two workgroups per CU, i.e. two waves per SIMD; at 256 one workgroup fills the CU's LDS
// and its waves have the whole register file for the 256-wide accumulators.  Rescaling is lazy: O and the row sum are rescaled only when
// some row's maximum grew by more than 2^8 since the last rescale, so P <= 2^8 always.
#include "common.h"
#include "launch.h"

namespace fab {

template <int HD>
struct Fwd16 {
  typedef TileLayout<HD> L;
  static constexpr int BM = 128, BN = 64;
  static constexpr int TILE = L::bytes(BN);  // one K or V tile
  static constexpr int BUF = 2 * TILE;
  static constexpr int STAGES = 2;
  typedef TileDma<bf16, HD, BN> Dma;  // (the element type only sets the row size)
  static constexpr int KMAX = Dma::KMAX;
  static constexpr int SPARE = Dma::kSpare ? 1024 : 0;
  static constexpr int LDS = STAGES * BUF + SPARE;
  static constexpr int OROW = HD * 2 + 16;  // epilogue: row pitch of the 16-bit output tile
  static constexpr int WG_PER_CU = HD <= 128 ? 2 : 1;
  static_assert(LDS <= 160 * 1024 / WG_PER_CU, "LDS budget per workgroup");
  static_assert(4 * 32 * OROW <= LDS, "the output tiles of the four waves fit the staging buffers");
};

template <class T, int HD>
__global__ __launch_bounds__(256, (HD <= 128 ? 2 : 1)) void fwd16_kernel(const FwdParams p) {
  typedef Fwd16<HD> C;
  typedef typename C::L L;
  typedef typename Frag<T>::type F;
  constexpr int NC = HD / 16, NDB = HD / 32;
  static_assert(C::KMAX <= NC, "a tile's prefetch is spread over the head-dim slices");
  constexpr int BM = C::BM, BN = C::BN;
  constexpr float kLazy = 8.f;  // log2 growth of a row maximum tolerated without rescaling

  __shared__ __attribute__((aligned(1024))) char smem[C::LDS];
  char* const spare = smem + C::STAGES * C::BUF;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, hl = lane >> 5, c32 = lane & 31;
  const int Sq = p.Sq, Sk = p.Sk;
  const bool causal = p.causal != 0;
  const int G = p.H / p.H_kv;
  const int n_qt = (Sq + BM - 1) / BM;

  const WorkItem wi = map_work(blockIdx.x, p.n_units, p.units_per_xcd);
  const int b = wi.unit / p.H_kv, g = wi.unit % p.H_kv;
  const int hq = g * G + wi.step % G;
  const int tq = wi.step / G;
  const int it = causal ? n_qt - 1 - tq : tq;  // heaviest query tiles first
  const int m0 = it * BM;
  const int mw0 = m0 + 32 * w;
  const int m = mw0 + c32;  // this lane's query row

  const size_t q_off = (size_t)(b * p.H + hq) * Sq;
  const size_t kv_off = (size_t)(b * p.H_kv + g) * Sk * HD;
  const T* Qg = (const T*)p.q + q_off * HD;

  F qf[NC];
  {
    const int mc = min(m, Sq - 1);  // rows past Sq compute on a valid row; never stored
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) qf[cc] = ld8(Qg + (size_t)mc * HD + 16 * cc + 8 * hl);
  }

  // LDS offsets.  A operand of S^T (K rows 32 nb + c32, chunk 2 cc + hl); A operand of O^T
  // (V^T, transposed read of the V tile: 16-lane group (hl, dh), lane i in the group).
  int a_off[NC];
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) a_off[cc] = L::off(c32, 2 * cc + hl);
  const int gi16 = lane & 15, dh = (lane >> 4) & 1;
  int t_off[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int sec = 0; sec < 2; ++sec) {
      const int r = 4 * hl + 8 * sec + (gi16 >> 2);
      const int col = 32 * db + 16 * dh + 4 * (gi16 & 3);
      t_off[db][sec] = L::off(r, col >> 3) + 2 * (col & 7);
    }

  // key tiles holding a key some row of this tile may attend
  const KeyRange kr{Sk, p.causal, p.win};
  const int k_lo = kr.lo(m0), k_hi = kr.hi(min(m0 + BM, Sq) - 1);
  const int j_begin = k_lo / BN;
  const int j_end = k_hi >= k_lo ? k_hi / BN + 1 : j_begin;

  TileDma<T, HD, BN> kvdma;
  kvdma.init(w, lane);
  const rsrc_t rk = make_rsrc((const T*)p.k + kv_off, (unsigned)((size_t)Sk * HD * sizeof(T)));
  const rsrc_t rv = make_rsrc((const T*)p.v + kv_off, (unsigned)((size_t)Sk * HD * sizeof(T)));
  constexpr unsigned TILEB = BN * HD * sizeof(T);
  auto issue_part = [&](int j, char* buf, int k) {
    kvdma.issue(k, buf, rk, (unsigned)j * TILEB, spare, lane);
    kvdma.issue(k, buf + C::TILE, rv, (unsigned)j * TILEB, spare, lane);
  };
#pragma unroll
  for (int k = 0; k < C::KMAX; ++k) issue_part(j_begin, smem + (j_begin & 1) * C::BUF, k);
  wait_vm_all();
  barrier_lds();

  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
  float mrun = -1e30f;  // running maximum of this row's log2-domain scores (finite start)
  float lsum = 0.f;     // this lane half's share of the row sum of P

  // One key tile.  The stage being read and the stage being prefetched are restrict
  // pointers, so the compiler knows the direct-to-LDS prefetch does not write what the step
  // reads and does not make those reads wait for it.
  auto step_body = [&](const char* __restrict__ cur, char* __restrict__ nxt, int j) {
    const bool pf = j + 1 < j_end;
    const int n0 = j * BN;
    // ---- S^T = K Q^T for the tile's two 32-key blocks; the next tile's prefetch is spread
    // over these MFMAs.
    f32x16 St[2];
    St[0] = f32x16{};
    St[1] = f32x16{};
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      const F k0 = lds_frag<T>(cur, a_off[cc]);
      const F k1 = lds_frag<T>(cur + L::rows(32), a_off[cc]);
      if (pf && cc < C::KMAX) issue_part(j + 1, nxt, cc);
      mma(St[0], k0, qf[cc]);
      mma(St[1], k1, qf[cc]);
    }
    // ---- scores in the log2 domain; masked ones are -inf.  Register r of block nb holds key
    // n0 + 32 nb + 4 hl + off, off = 8 (r / 4) + r % 4, of row m; it is seen iff
    // kr.lo(m) <= key <= kr.hi(m).  Only steps that cut some row's keys test.
    const float c2 = p.scale_log2;
    // On steps that cut some row's keys the scores are scaled here and the cut ones set to
    // -inf.  Elsewhere the scale is applied inside the exponent's fma below (one vector
    // instruction per score fewer): the row maximum of the scaled scores is then c2 times the
    // maximum of the raw ones, or times their minimum when c2 < 0.
    const bool cut = kr.hi(mw0) < n0 + BN - 1 || kr.lo(mw0 + 31) > n0;
    float mx;
    if (cut) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int base = n0 + 32 * nb + 4 * hl;
        const int a = kr.lo(m) - base, z = kr.hi(m) - base;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = 8 * (r >> 2) + (r & 3);
          St[nb][r] = (off >= a && off <= z) ? St[nb][r] * c2 : -__builtin_inff();
        }
      }
      mx = -__builtin_inff();
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, St[nb][r]);
    } else if (c2 >= 0.f) {
      float hi = -__builtin_inff();
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) hi = fmaxf(hi, St[nb][r]);
      mx = hi * c2;
    } else {
      float lo = __builtin_inff();
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) lo = fminf(lo, St[nb][r]);
      mx = lo * c2;
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // ---- lazy rescale (wave-uniform decision): only when some row's maximum grew by more
    // than kLazy; rows whose maximum did not grow get alpha = 1.
    if (__any(mx > mrun + kLazy)) {
      const float mnew = fmaxf(mrun, mx);
      const float alpha = fast_exp2(mrun - mnew);
      mrun = mnew;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[db] *= alpha;
    }
    // ---- P = exp2(score - mrun) <= 2^kLazy, its row sum, and its 16-bit fragments
    // (fragment (nb, ks): registers 8 ks .. 8 ks + 7 of block nb), the B operand of O^T.
    F pb[2][2];
    const float sc = cut ? 1.f : c2;  // the scores' remaining scale factor
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = fast_exp2(St[nb][r] * sc - mrun);
        lsum += pv;
        pb[nb][r >> 3][r & 7] = (T)pv;
      }
    // ---- O^T += V^T P^T: A operand = transposed read of the V tile (rows = keys).
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int ro = L::rows(32 * nb + 16 * ks);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const F va = lds_frag_tr<T>(cur + C::TILE, t_off[db][0] + ro, t_off[db][1] + ro);
          mma(o[db], va, pb[nb][ks]);
        }
      }
  };

  for (int j = j_begin; j < j_end; ++j) {
    step_body(smem + (j & 1) * C::BUF, smem + ((j + 1) & 1) * C::BUF, j);
    wait_vm_all();  // the next tile has landed
    barrier_lds();  // and nobody reads this one any more before it is overwritten
  }

  // ---- epilogue: O = O^T / rowsum (register r of block db holds column 32 db + 8 (r / 4) +
  // 4 hl + r % 4 of this lane's row); LSE in natural log.  A row that may attend no key
  // (possible with a window) gets O = 0 and LSE = log 0 = -inf.  Each wave writes its 32 rows
  // into a row-major tile of its own in LDS (the stage buffers are free: the loop ended on a
  // barrier after every wave's loads) and stores it by whole rows, 16 bytes per lane.
  const float ltot = lsum + __shfl_xor(lsum, 32);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  char* const otile = smem + w * (32 * C::OROW);
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      typedef T v4 __attribute__((ext_vector_type(4)));
      const int d = 32 * db + 8 * q4 + 4 * hl;
      *reinterpret_cast<v4*>(otile + c32 * C::OROW + 2 * d) =
          v4{(T)(o[db][4 * q4] * inv), (T)(o[db][4 * q4 + 1] * inv),
             (T)(o[db][4 * q4 + 2] * inv), (T)(o[db][4 * q4 + 3] * inv)};
    }
  asm volatile("" ::: "memory");  // the wave reads back only what it wrote, in order
  T* const Og = (T*)p.o + q_off * HD;
  constexpr int CPR = HD / 8;  // 16-byte chunks per row
#pragma unroll
  for (int i = 0; i < CPR / 2; ++i) {
    const int q = 64 * i + lane, row = q / CPR, ch = q % CPR;
    typedef T v8 __attribute__((ext_vector_type(8)));
    const v8 val = *reinterpret_cast<const v8*>(otile + row * C::OROW + 16 * ch);
    if (mw0 + row < Sq) *reinterpret_cast<v8*>(Og + (size_t)(mw0 + row) * HD + 8 * ch) = val;
  }
  if (m < Sq && hl == 0) p.lse[q_off + m] = (mrun + __log2f(ltot)) * kLn2;
}

template <class T, int HD>
static hipError_t go16(const FwdParams& p, hipStream_t s, LaunchInfo* info) {
  typedef Fwd16<HD> C;
  const int n_qt = (p.Sq + C::BM - 1) / C::BM;
  const int grid = p.n_units * (p.H / p.H_kv) * n_qt;
  if (info) *info = LaunchInfo{"fwd16", grid, 256, C::LDS};
  hipLaunchKernelGGL((fwd16_kernel<T, HD>), dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <class T>
static hipError_t fwd_hd(const FwdParams& p, int hd, hipStream_t s, LaunchInfo* info) {
  switch (hd) {
    case 32: return go16<T, 32>(p, s, info);
    case 64: return go16<T, 64>(p, s, info);
    case 96: return go16<T, 96>(p, s, info);
    case 128: return go16<T, 128>(p, s, info);
    default: return go16<T, 256>(p, s, info);
  }
}

hipError_t launch_fwd16(const FwdParams& p, int dt, int hd, hipStream_t s, LaunchInfo* info) {
  return dt == kBF16 ? fwd_hd<bf16>(p, hd, s, info) : fwd_hd<f16>(p, hd, s, info);
}

}  // namespace fab
