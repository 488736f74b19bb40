// The step-2 kernels for 16-bit inputs (bf16, fp16), tiled for gfx950: the key-tile outer
// dK/dV kernel, and dQ in one of two ways -- a query-tile outer kernel that recomputes S and dP,
// or, when the workspace holds room for it, a contraction dQ = scale dS K over the dS values
// the dK/dV kernel stored ("stored dS").
//
// Both kernels stage their streamed operand tiles with direct global->LDS loads
// (buffer_load_dwordx4 ... lds) into a ring of stage buffers, so the next tiles arrive while
// the current one is consumed and each step needs one barrier.  Tiles are row-major in the
// bank-conflict-free layouts of TileLayout (common.h); operands that contract over rows are
// read with the LDS transpose read (lds_frag_tr) instead of keeping a transposed copy.  The
// buffer loads are range-checked: rows past the end of the tensor read as zeros and rows
// past a head's end read the next head's rows, finite values that the masks and the padding
// rows' statistics (LSE = +inf, D = 0) neutralise.  (The dK/dV kernel's resident V tile is
// loaded once, with its rows clamped to the last valid key.)
//
// Per-row statistics: stats[(b*H + h) * Sq_pad + i] = {LSE * log2(e), D} with
// Sq_pad = Sq rounded up to 64, written by the preprocess kernel or, on fab_bwd's path, by
// the dQ kernel's prologue.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace fab {

// Cache policy of the stored-dS traffic (gfx950 bits: 1 = sc0, 2 = nt, 16 = sc1): dS is
// written once and read once, by another kernel, so both sides stream it (nt) rather than
// let it displace the Q, dO and K tiles that neighbouring workgroups share through the L2
// (measured: 0.870 against 0.913 ms for the whole backward at B=2, H=32, S=4096, D=128).
#ifndef FAB_DS_STORE_AUX
#define FAB_DS_STORE_AUX 2
#endif
#ifndef FAB_DS_LOAD_AUX
#define FAB_DS_LOAD_AUX 2
#endif

// =======================================================================================
// dK, dV: key-tile outer (boostr flash_bwd.rs "Step 2": one workgroup per tile of keys).
// A workgroup owns BN keys of one (batch, kv head) and walks every query head of the group
// and every query tile (BM rows) the mask (causal, window) lets reach its keys.  Up to head
// dim 128 a wave owns 64 keys, so every Q / dO element read from LDS feeds 64 keys: its 4 waves
// form a 2 x 2 grid over BN = 128 keys (wave (kb, qh) owns keys [64 kb, 64 kb + 64) and the
// query rows [32 qh, 32 qh + 32) of each 64-row tile), or, in the wide variant, a 4 x 1 grid
// over BN = 256 keys and 32-row tiles, which halves the number of workgroups and with them the
// fixed cost of each (the launcher takes it where the grid still gives every CU at least two
// workgroups).  At head dim 256 the dK, dV accumulators of 64 keys would not fit, so the grid
// is 4 x 1 with BN = 128: wave kb owns keys [32 kb, 32 kb + 32) and all of a 32-row tile.  A wave's K
// fragments stay in registers and the V tile in LDS for the workgroup's life (there is no room
// for V in registers beside the dK, dV accumulators and the score tiles); dK and dV accumulate
// in AGPRs, and with two query halves they are summed through LDS at the end.
// =======================================================================================
template <int HD, bool WIDE>
struct Dkdv16 {
  typedef TileLayout<HD> L;
  // Wave grid: KG groups of keys x QH halves of the query tile.  Up to head dim 128 a wave owns
  // KB = 2 blocks of 32 keys and half of a 64-row query tile (2 x 2 grid), or in the wide
  // variant all of a 32-row tile (4 x 1 grid); at 256 its dK, dV accumulators allow one block,
  // so a wave owns 32 keys and all of a 32-row tile (4 x 1 grid).
  static constexpr int KB = HD <= 128 ? 2 : 1, QH = (KB == 2 && !WIDE) ? 2 : 1, KG = 4 / QH;
  static constexpr int BN = 32 * KB * KG, BM = 32 * QH;
  static constexpr int TILE = L::bytes(BM);    // one Q or dO tile
  static constexpr int STATS = 1024;           // {lse2, D} of 128 rows (one wave-wide load)
  static constexpr int BUF = 2 * TILE + STATS; // one stage: Q, dO, stats
  static constexpr int VT = L::bytes(BN);      // V tile of the workgroup
  static constexpr int STAGES = HD <= 128 ? 3 : 2;  // tiles in flight: current + prefetched
  typedef TileDma<bf16, HD, BM> Dma;           // (the element type only sets the row size)
  static constexpr int KMAX = Dma::KMAX;
  static constexpr int SPARE = Dma::kSpare ? 1024 : 0;  // target of padding loads
  static constexpr int LDS = STAGES * BUF + VT + SPARE;
  static constexpr int RED = QH > 1 ? 2 * 64 * HD * 4 : 0;  // epilogue: partial dK or dV exchange
  static constexpr int OROW = HD * 2 + 16;     // epilogue: row pitch of the 16-bit output tile
  static constexpr int OUT = BN * OROW;        // epilogue: the tile's output rows
  // Loads each wave issues per stage (Q and dO; wave 0 adds the statistics), and the dS
  // fragments it stores per step when dS is stored.
  static constexpr int ISSUE = 2 * KMAX;
  static constexpr int DS_STORES = 2 * KB;
  static_assert(RED + OUT <= LDS, "reduction and output tiles must fit in the staging buffers");
  static_assert(LDS <= 160 * 1024, "LDS budget");
  static_assert(TILE % 16 == 0 && VT % 16 == 0, "granule alignment");
};

// The kernel body, for workgroup `wg` of the launch, with C::LDS bytes of LDS at `smem`
// (1024-byte aligned); the kernels below run it on their own or beside the dQ body.
template <class T, int HD, bool WIDE>
__device__ __forceinline__ void dkdv16_body(const BwdParams& p, int wg, char* smem) {
  typedef Dkdv16<HD, WIDE> C;
  typedef typename Frag<T>::type F;
  typedef TileDma<T, HD, C::BM> Dma;
  constexpr int NC = HD / 16, NDB = HD / 32;
  static_assert(C::KMAX <= NC, "a tile's prefetch is spread over the head-dim slices");
  constexpr int BM = C::BM, BN = C::BN, KB = C::KB, STAGES = C::STAGES;
  typedef typename C::L L;
  constexpr unsigned ROWB = HD * sizeof(T);

  char* const vtile = smem + C::STAGES * C::BUF;
  char* const spare = vtile + C::VT;  // only used when the tile DMA needs padding loads

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform per wave
  const int lane = tid & 63, hl = lane >> 5, c32 = lane & 31;
  const int kb = w % C::KG, qh = w / C::KG;

  const WorkItem wi = map_work(wg, p.n_units, p.units_per_xcd);
  const int b = wi.unit / p.H_kv, g = wi.unit % p.H_kv;
  const int n0 = wi.step * BN;
  const int G = p.H / p.H_kv;
  const int Sq = p.Sq, Sk = p.Sk, Sq_pad = p.Sq_pad;
  const size_t kv_off = (size_t)(b * p.H_kv + g) * Sk * HD;
  const T* Kg = (const T*)p.k + kv_off;
  const T* Vg = (const T*)p.v + kv_off;

  // ---- V tile -> LDS once for the workgroup's life; K fragments -> registers
  load_tile<T, HD, BN>(vtile, Vg, n0, Sk - 1, w, 4, lane);
  const int nw0 = n0 + 32 * KB * kb;
  F kf[KB][NC];
#pragma unroll
  for (int nb = 0; nb < KB; ++nb) {
    const int n = min(nw0 + 32 * nb + c32, Sk - 1);
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) kf[nb][cc] = ld8(Kg + (size_t)n * HD + 16 * cc + 8 * hl);
  }

  f32x16 dk[KB][NDB], dv[KB][NDB];
#pragma unroll
  for (int nb = 0; nb < KB; ++nb) {
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      dk[nb][db] = f32x16{};
      dv[nb][db] = f32x16{};
    }
    mma_ready(dk[nb]);
    mma_ready(dv[nb]);
  }

  // ---- per-lane LDS offsets
  // A operand (Q or dO rows): row 32 qh + c32, chunk 2 cc + hl
  int a_off[NC];
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) a_off[cc] = L::off(32 * qh + c32, 2 * cc + hl);
  // B operand of P^T dO / dS^T Q, transposed read: 16-lane group (hl, dh), lane i in group
  const int gi16 = lane & 15, dh = (lane >> 4) & 1;
  int t_off[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int sec = 0; sec < 2; ++sec) {
      const int r = 32 * qh + 4 * hl + 8 * sec + (gi16 >> 2);
      const int col = 32 * db + 16 * dh + 4 * (gi16 & 3);
      t_off[db][sec] = L::off(r, col >> 3) + 2 * (col & 7);
    }
  // B operand of dP = dO V^T: V rows 32 (KB kb + nb) + c32 have the same layout offsets as the
  // A operand rows 32 qh + c32 shifted by a whole number of row groups, so they are a_off
  // plus a wave constant.
  const char* const vrows = vtile + L::rows(32 * KB * kb) - L::rows(32 * qh);

  // ---- iteration space: every query head of the group and every query tile holding a row
  // that may attend one of these keys (rows [r_lo, r_hi]).  Tiles run from the last one
  // down, heads inside: step s is tile i_last - s / G of head s % G.  Without a window every
  // key tile's sequence starts at the same (tile, head), so the workgroups of a group that
  // run together on an XCD read the same Q and dO tile at about the same time and share it
  // through that XCD's L2.
  const int n_qt = (Sq + BM - 1) / BM;
  const KeyRange kr{Sk, p.causal, p.win};
  const int r_lo = max(kr.rows_lo(n0), 0), r_hi = min(kr.rows_hi(min(n0 + BN, Sk) - 1), Sq - 1);
  const int i_first = r_lo / BM, i_last = r_hi / BM;
  const int per = r_hi >= r_lo ? i_last - i_first + 1 : 0;
  const int total = G * per;
  // The wave's 32 rows from mw0 see all of its 32 KB keys from nw0 iff
  // kr.hi(mw0) >= nw0 + 32 KB - 1 and kr.lo(mw0 + 31) <= nw0, i.e. iff full_lo <= mw0 <= full_hi:
  const int full_lo = nw0 + 32 * KB - 1 > Sk - 1 ? (1 << 30)
                      : p.causal ? nw0 + 32 * KB - 1 : (p.win > 0 ? nw0 + 32 * KB - p.win : -(1 << 30));
  const int full_hi = p.win > 0 ? nw0 + p.win - 32 : (1 << 30);

  // Buffer resources over the rows of the group's query heads (Q, dO) and their row
  // statistics.  A tile is selected by a uniform byte offset; rows past a head's end read the
  // next head's rows or, past the group, zeros: finite values that the padding rows'
  // statistics (lse = +inf) turn into P = 0.  The prefetch issued after the last step reads
  // past the group (zeros) into a stage nothing reads any more.
  const size_t row0 = (size_t)(b * p.H + g * G) * Sq;
  const rsrc_t rq = make_rsrc((const T*)p.q + row0 * HD, (unsigned)((size_t)G * Sq * ROWB));
  const rsrc_t rdo = make_rsrc((const T*)p.dO + row0 * HD, (unsigned)((size_t)G * Sq * ROWB));
  const rsrc_t rst = make_rsrc(p.stats + (size_t)(b * p.H + g * G) * Sq_pad * 2,
                               (unsigned)((size_t)G * Sq_pad * 8));

  // Stored dS (p.ds set): every dS fragment of the step is also written to the slab of its
  // query head, for the dQ kernel that follows.  The resource spans the group's G slabs (the
  // host keeps that below 4 GB).  A lane's 16 bytes of a fragment (key c32, 8 query rows) go
  // to byte 16 (2 c32 + hl): the two lane halves of one key side by side, which is what the
  // dQ kernel's transposed LDS reads of 4 keys x 16 rows want.
  const bool store_ds = p.ds != nullptr;
  const rsrc_t rds = make_rsrc(store_ds ? (const char*)p.ds + (size_t)(b * p.H + g * G) * p.ds_slab
                                        : (const char*)p.q,
                               store_ds ? (unsigned)G * p.ds_slab : 0u);
  const unsigned ds_voff = 16u * (2 * c32 + hl);
  const int k32w = nw0 >> 5;

  Dma qdma;
  qdma.init(w, lane);
  // Head and tile of the next stage to prefetch, advanced once per issued stage.  Past the
  // last step the offsets leave the group (or wrap): those reads are range-checked zeros or
  // in-range rows, landing in a stage nothing reads.
  int ph = 0, pit = i_last;
  auto issue_part = [&](char* buf, int k, unsigned q_soff, unsigned st_soff) {
    qdma.issue(k, buf, rq, q_soff, spare, lane);
    qdma.issue(k, buf + C::TILE, rdo, q_soff, spare, lane);
    if (k == 0 && w == 0) b2lds16(rst, 16u * lane, st_soff, buf + 2 * C::TILE);
  };
  auto next_offsets = [&](unsigned& q_soff, unsigned& st_soff) {
    q_soff = (unsigned)(ph * Sq + pit * BM) * ROWB;
    st_soff = (unsigned)(ph * Sq_pad + pit * BM) * 8u;
    if (++ph == G) {
      ph = 0;
      --pit;
    }
  };
  auto issue = [&](char* buf) {
    unsigned qs, ss;
    next_offsets(qs, ss);
#pragma unroll
    for (int k = 0; k < C::KMAX; ++k) issue_part(buf, k, qs, ss);
  };

  // Ring of STAGES tile buffers: step s computes on buffer s % STAGES while the tiles of the
  // next STAGES - 1 steps are in flight.
#pragma unroll
  for (int st = 0; st < STAGES - 1; ++st) issue(smem + st * C::BUF);
  wait_vm_le<C::ISSUE * (STAGES - 2)>();  // V, K and stage 0 have landed
  barrier_lds();

  const float mask_s = p.mask_s;

  // One step.  The stage being read, the resident V tile and the stage being prefetched are
  // passed as restrict pointers: the compiler then knows that the direct-to-LDS prefetch does
  // not write what this step reads, and does not make the step's LDS reads wait for it.
  //
  // The step is ordered so that the matrix cores always have work while the vector ALU
  // computes the softmax: S first; then dP, with the exponentials of P (which need only S)
  // computed while its MFMAs run; then dV += P^T dO for the first 16 rows while dS of those
  // rows is formed; dK += dS^T Q for them while the last exponentials are formed; dV for the
  // second 16 rows while their dS is formed; and last dK for the second 16 rows.
  // Operands that open a step: the Q fragments of every head-dim slice and the statistics of
  // this lane's 16 rows (register r of a block holds row m_base + off(r), off(r) = 8 (r / 4) +
  // r % 4).  They are read from the stage of the next step while the current step's last
  // MFMAs run, so a step starts with them in registers.
  F aq[NC];
  float l2[16], dl[16];

  auto load_step_operands = [&](const char* __restrict__ buf) {
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) aq[cc] = lds_frag<T>(buf, a_off[cc]);
    const float* st = reinterpret_cast<const float*>(buf + 2 * C::TILE);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ml = 32 * qh + 8 * j + 4 * hl;
      const f32x4 s01 = *reinterpret_cast<const f32x4*>(st + 2 * ml);
      const f32x4 s23 = *reinterpret_cast<const f32x4*>(st + 2 * ml + 4);
      l2[4 * j + 0] = s01[0]; dl[4 * j + 0] = s01[1];
      l2[4 * j + 1] = s01[2]; dl[4 * j + 1] = s01[3];
      l2[4 * j + 2] = s23[0]; dl[4 * j + 2] = s23[1];
      l2[4 * j + 3] = s23[2]; dl[4 * j + 3] = s23[3];
    }
  };
  load_step_operands(smem);

  // One step on stage `cur`; `nb1` is the stage of the next step and `nxt` the stage being
  // prefetched (step s + STAGES - 1; with two stages it is `nb1` itself).  The workgroup
  // barrier that ends the step sits before its last MFMAs: by then every read of `cur` has
  // completed, and the next step's operands are read from `nb1` while those MFMAs run.
  auto step_body = [&](const char* __restrict__ cur, const char* __restrict__ vrows,
                       char* __restrict__ nxt, const char* nb1, int m0, int hh) {
    unsigned pq_soff, pst_soff;
    next_offsets(pq_soff, pst_soff);
    const int mw0 = m0 + 32 * qh;
    // dS fragment (nb, ks) of this step: row block mw0 / 16 + ks, key block k32w + nb.
    const unsigned ds_soff = (unsigned)hh * p.ds_slab +
                             (unsigned)((((mw0 >> 7) * p.ds_nk32 + k32w) * 8 + ((mw0 >> 4) & 7)) * 1024);

    // ---- S = Q K^T for the wave's key blocks; the prefetch is spread over it, one instruction
    // per head-dim slice, so the wave never stalls on a burst of loads.
    f32x16 S[KB], dP[KB];
#pragma unroll
    for (int nb = 0; nb < KB; ++nb) S[nb] = f32x16{};
    // Operands of dP = dO V^T stream through a window LEAD head-dim slices deep; the first
    // LEAD slices are read here, under the S MFMAs (LDS latency under load is several MFMAs).
    constexpr int LEAD = NC >= 8 ? 3 : 2;
    F ad[NC], bv[KB][NC];
    auto read_dp_operands = [&](int cc) {
      ad[cc] = lds_frag<T>(cur + C::TILE, a_off[cc]);
#pragma unroll
      for (int nb = 0; nb < KB; ++nb) bv[nb][cc] = lds_frag<T>(vrows + L::rows(32 * nb), a_off[cc]);
    };
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      if (cc < C::KMAX) issue_part(nxt, cc, pq_soff, pst_soff);
      if (cc < LEAD) read_dp_operands(cc);
#pragma unroll
      for (int nb = 0; nb < KB; ++nb) mma(S[nb], aq[cc], kf[nb][cc]);
      __builtin_amdgcn_sched_barrier(0);
    }

    // Masking, only on steps that cut some row's keys (the causal diagonal, a window's
    // edges, the last key tile): a cut score is replaced by mask_s, whose exponent is -inf,
    // so P = 0 and dS = 0 there.  Key n (this lane's column of block nb) may be seen by the
    // rows [kr.rows_lo(n), kr.rows_hi(n)] if n < Sk; register r holds row m_base + off(r).
    if (mw0 < full_lo || mw0 > full_hi) {
      const int m_base = mw0 + 4 * hl;
#pragma unroll
      for (int nb = 0; nb < KB; ++nb) {
        const int n = nw0 + 32 * nb + c32;
        const int a = n < Sk ? kr.rows_lo(n) - m_base : (1 << 30);
        const int z = kr.rows_hi(n) - m_base;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = 8 * (r >> 2) + (r & 3);
          S[nb][r] = (off >= a && off <= z) ? S[nb][r] : mask_s;
        }
      }
    }

    __builtin_amdgcn_sched_barrier(0);
    // ---- dP = dO V^T, with P = exp2(S scale log2e - lse2) computed in place of S (and its
    // 16-bit copy, the A operand of dV += P^T dO) while the MFMAs run.  Fragment (nb, ks)
    // holds registers 8 ks .. 8 ks + 7 of block nb.  The MFMAs are volatile asm and every
    // exponential is pinned between them with order_point(), so the interleave is exact.
    // A lane's NE exponentials go in the order registers 0..7 of every block (the A operands
    // of the first dV MFMAs), then registers 8..15.  The dP MFMAs take NE_DP of them, about as
    // many as their issue time covers (an exponential with its fma and conversion takes about
    // two thirds of an MFMA's), and never fewer than registers 0..7; the rest run under the
    // dK MFMAs of rows 0..15, which otherwise leave the vector ALU idle.
    F pa[KB][2], da[KB][2];
    // The dS fragments of rows 16 ks .. 16 ks + 15 go out as soon as they are formed.
    auto store_ds_rows = [&](int ks) {
      if (store_ds) {
#pragma unroll
        for (int nb = 0; nb < KB; ++nb)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, da[nb][ks]), rds, ds_voff,
                                                 ds_soff + (unsigned)(nb * 8192 + ks * 1024),
                                                 FAB_DS_STORE_AUX);
      }
    };
    constexpr int NE = 16 * KB;
    constexpr int NE_FIT = NC * KB * 3 / 2;
    constexpr int NE_DP = NE < NE_FIT ? NE : (NE_FIT > 8 * KB ? NE_FIT : 8 * KB);
    constexpr int PER_CC = (NE_DP + NC - 1) / NC;   // exponentials per head-dim slice
    constexpr int PER_NB = (PER_CC + KB - 1) / KB;  // ... after each of its MFMAs
    auto pexp = [&](int e) {
      const int j = e % (8 * KB), nb = j % KB, r = 8 * (e / (8 * KB)) + j / KB;
      float sv = S[nb][r];
      order_point(sv);  // not before the MFMA that precedes it in the interleave
      float x = fast_exp2(sv * p.scale_log2 - l2[r]);
      order_point(x);
      S[nb][r] = x;
      pa[nb][r >> 3][r & 7] = (T)x;
    };
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      if (cc + LEAD < NC) read_dp_operands(cc + LEAD);
#pragma unroll
      for (int nb = 0; nb < KB; ++nb) {
        if (cc == 0) mma_v0<false>(dP[nb], ad[cc], bv[nb][cc]);
        else mma_v<false>(dP[nb], ad[cc], bv[nb][cc]);
#pragma unroll
        for (int k = nb * PER_NB; k < (nb + 1) * PER_NB && k < PER_CC; ++k)
          if (cc * PER_CC + k < NE_DP) pexp(cc * PER_CC + k);
      }
    }
    mma_vdrain(dP);
    __builtin_amdgcn_sched_barrier(0);

    // dS = P (dP - D) for register r of block nb, into its 16-bit fragment.
    auto ds = [&](int nb, int r) {
      da[nb][r >> 3][r & 7] = (T)(S[nb][r] * (dP[nb][r] - dl[r]));
    };
    // B operands, transposed reads of the dO and Q tiles: d block db, row slice ks.
    auto b_do = [&](int db, int ks) {
      return lds_frag_tr<T>(cur + C::TILE, t_off[db][0] + L::rows(16) * ks, t_off[db][1] + L::rows(16) * ks);
    };
    auto b_q = [&](int db, int ks) {
      return lds_frag_tr<T>(cur, t_off[db][0] + L::rows(16) * ks, t_off[db][1] + L::rows(16) * ks);
    };

    // ---- dV += P^T dO, rows 0..15 of the wave, with dS of those rows formed meanwhile.
    F bo[NDB], bq[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) bo[db] = b_do(db, 0);
    constexpr int PER_MMA = (8 + NDB - 1) / NDB;  // dS elements per MFMA of a 16-row slice
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      bq[db] = b_q(db, 0);
#pragma unroll
      for (int nb = 0; nb < KB; ++nb) {
        if (db == 0) mma_a<true>(dv[nb][db], pa[nb][0], bo[db]);  // first use of pa[nb][0]
        else mma_a<false>(dv[nb][db], pa[nb][0], bo[db]);
#pragma unroll
        for (int k = 0; k < PER_MMA; ++k) {
          const int e = (KB * db + nb) * PER_MMA + k;  // rows 0..7 of every block
          if (e < 8 * KB) ds(e % KB, e / KB);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    store_ds_rows(0);
    // ---- dK += dS^T Q, rows 0..15, with the remaining exponentials formed meanwhile.
    constexpr int NR = NE - NE_DP;
    constexpr int PER_MMA_E = (NR + NDB * KB - 1) / (NDB * KB);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      bo[db] = b_do(db, 1);
#pragma unroll
      for (int nb = 0; nb < KB; ++nb) {
        if (db == 0) mma_a<true>(dk[nb][db], da[nb][0], bq[db]);  // first use of da[nb][0]
        else mma_a<false>(dk[nb][db], da[nb][0], bq[db]);
#pragma unroll
        for (int k = 0; k < PER_MMA_E; ++k) {
          const int e = (KB * db + nb) * PER_MMA_E + k;
          if (e < NR) pexp(NE_DP + e);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // ---- dV += P^T dO for rows 16..31, reading the last B operands of this stage, with dS of
    // rows 16..31 formed meanwhile.
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      bq[db] = b_q(db, 1);
#pragma unroll
      for (int nb = 0; nb < KB; ++nb) {
        if (db == 0) mma_a<true>(dv[nb][db], pa[nb][1], bo[db]);  // first use of pa[nb][1]
        else mma_a<false>(dv[nb][db], pa[nb][1], bo[db]);
#pragma unroll
        for (int k = 0; k < PER_MMA; ++k) {
          const int e = (KB * db + nb) * PER_MMA + k;
          if (e < 8 * KB) ds(e % KB, 8 + e / KB);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    store_ds_rows(1);
    // ---- end of the step for the workgroup: the next stage has landed (the loads of the one
    // after it may stay in flight) and no wave reads `cur` any more.  Vector memory operations
    // retire in issue order, stores among loads, so the wait names how many were issued after
    // the next stage's loads: the prefetch issued in this step and, with stored dS, the stores
    // of the previous step and of this one, which then have two steps to retire.
    if (store_ds) wait_vm_le<C::ISSUE * (STAGES - 2) + C::DS_STORES * (STAGES - 1)>();
    else wait_vm_le<C::ISSUE * (STAGES - 2)>();
    barrier_lds();
    load_step_operands(nb1);
    // ---- dK += dS^T Q for rows 16..31 while the next step's operands arrive.
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int nb = 0; nb < KB; ++nb) {
        if (db == 0) mma_a<true>(dk[nb][db], da[nb][1], bq[db]);
        else mma_a<false>(dk[nb][db], da[nb][1], bq[db]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  int cb = 0;  // buffer of step s
  int it = i_last, hh = 0;
  for (int s = 0; s < total; ++s) {
    const int nb1 = cb == STAGES - 1 ? 0 : cb + 1;                     // (s + 1) % STAGES
    const int nb2 = STAGES == 2 ? nb1 : (cb >= 1 ? cb - 1 : STAGES - 1);  // (s + STAGES - 1) % STAGES
    step_body(smem + cb * C::BUF, vrows, smem + nb2 * C::BUF, smem + nb1 * C::BUF, it * BM, hh);
    cb = nb1;
    if (++hh == G) {
      hh = 0;
      --it;
    }
  }
  // the epilogue reuses the staging buffers: every prefetch must have landed
  wait_vm_all();
  barrier_lds();

#pragma unroll
  for (int nb = 0; nb < KB; ++nb) {
    mma_drain(dk[nb]);
    mma_drain(dv[nb]);
  }

  // ---- epilogue.  With two query halves the qh = 1 waves hand their partial sums to the
  // qh = 0 waves via LDS, which add them; the accumulators of a wave pair have identical
  // layouts, so the exchange is lane-major and conflict free.  A lane's sums lie down one
  // column (16 keys of column 32 db + c32), so the storing waves write them, scaled and rounded
  // to 16 bits, into a row-major tile in LDS and store that tile by whole rows: 16 bytes per
  // lane and 1 KB per store instruction, instead of one 2-byte element per lane.  Rows are
  // OROW bytes apart, so the two half-waves' 2-byte writes (rows 4 apart: 16 banks apart)
  // never collide.
  char* const otile = smem + C::RED + kb * (32 * KB * C::OROW);
  T* dKg = (T*)p.dk + kv_off;
  T* dVg = (T*)p.dv + kv_off;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    if constexpr (C::QH > 1) {
      float* red = reinterpret_cast<float*>(smem) + kb * (32 * KB * HD);
      if (qh == 1) {
#pragma unroll
        for (int nb = 0; nb < KB; ++nb)
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              const f32x16& a = pass == 0 ? dk[nb][db] : dv[nb][db];
              const int slot = (nb * NDB + db) * 4 + r4;
              *reinterpret_cast<f32x4*>(red + (slot * 64 + lane) * 4) =
                  f32x4{a[4 * r4], a[4 * r4 + 1], a[4 * r4 + 2], a[4 * r4 + 3]};
            }
      }
      __syncthreads();
    }
    if (qh == 0) {
      const float sc = pass == 0 ? p.scale : 1.f;
#pragma unroll
      for (int nb = 0; nb < KB; ++nb)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const f32x16& a = pass == 0 ? dk[nb][db] : dv[nb][db];
            f32x4 o = f32x4{};
            if constexpr (C::QH > 1) {
              const float* red = reinterpret_cast<const float*>(smem) + kb * (32 * KB * HD);
              const int slot = (nb * NDB + db) * 4 + r4;
              o = *reinterpret_cast<const f32x4*>(red + (slot * 64 + lane) * 4);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int row = 32 * nb + 8 * r4 + 4 * hl + e;  // key nw0 + row
              *reinterpret_cast<T*>(otile + row * C::OROW + 2 * (32 * db + c32)) =
                  (T)((a[4 * r4 + e] + o[e]) * sc);
            }
          }
      // the wave reads back only what it wrote: its LDS accesses complete in order
      asm volatile("" ::: "memory");
      T* const dst = pass == 0 ? dKg : dVg;
      constexpr int CPR = HD / 8;  // 16-byte chunks per row
#pragma unroll
      for (int i = 0; i < KB * CPR / 2; ++i) {
        const int q = 64 * i + lane, row = q / CPR, ch = q % CPR;
        typedef T v8 __attribute__((ext_vector_type(8)));
        const v8 val = *reinterpret_cast<const v8*>(otile + row * C::OROW + 16 * ch);
        if (nw0 + row < Sk) *reinterpret_cast<v8*>(dst + (size_t)(nw0 + row) * HD + 8 * ch) = val;
      }
    }
    __syncthreads();
  }
}

template <class T, int HD, bool WIDE>
__global__ __launch_bounds__(256) void bwd_dkdv16_kernel(const BwdParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[Dkdv16<HD, WIDE>::LDS];
  dkdv16_body<T, HD, WIDE>(p, blockIdx.x, smem);
}

// =======================================================================================
// dQ: query-tile outer.  A workgroup owns BM = 128 query rows of one (batch, head); wave w
// owns 32 of them, with their Q and dO fragments, LSE and D in registers (one query row per
// lane).  Per step of BN = 32 NB keys it recomputes S^T = K Q^T and dP^T = V dO^T, forms
// dS^T = P^T (dP^T - D) and adds dS K into the dQ accumulators.  K and V tiles stream
// through a ring of LDS stages (three for 32-key steps, two for 64-key steps), which keeps
// two workgroups, i.e. two waves per SIMD, on a CU.  On fab_bwd's path the kernel also forms
// its rows' D and base-2 LSE (step 1) and writes them for the dK/dV kernel.
// =======================================================================================
template <int HD, int NB>
struct Dq16 {
  typedef TileLayout<HD> L;
  static constexpr int BM = 128, BN = 32 * NB;  // one 32-row block per wave, NB key blocks
  static constexpr int TILE = L::bytes(BN);     // one K or V tile
  static constexpr int BUF = 2 * TILE;
  static constexpr int STAGES = NB == 1 ? 3 : 2;
  typedef TileDma<bf16, HD, BN> Dma;  // (the element type only sets the row size)
  static constexpr int KMAX = Dma::KMAX;
  static constexpr int SPARE = Dma::kSpare ? 1024 : 0;  // target of padding loads
  static constexpr int LDS = STAGES * BUF + SPARE;
  static constexpr int ISSUE = 2 * KMAX;  // loads each wave issues per stage
  static constexpr int OROW = HD * 2 + 16;  // epilogue: row pitch of the 16-bit output tile
  // Two workgroups (two waves per SIMD) per CU up to head dim 128; at 256 the Q, dO fragments
  // and dQ accumulators of a wave take more than half the register file, so one.
  static constexpr int WG_PER_CU = HD <= 128 ? 2 : 1;
  static_assert(LDS <= 160 * 1024 / WG_PER_CU, "LDS per workgroup");
  static_assert(4 * 32 * OROW <= LDS, "the output tiles of the four waves fit the staging buffers");
};

template <class T, int HD, int NB>
__device__ __forceinline__ void dq16_body(const BwdParams& p, int wg, char* smem) {
  typedef Dq16<HD, NB> C;
  typedef typename Frag<T>::type F;
  constexpr int NC = HD / 16, NDB = HD / 32;
  static_assert(C::KMAX <= NC, "a tile's prefetch is spread over the head-dim slices");
  constexpr int BM = C::BM, BN = C::BN, STAGES = C::STAGES;
  typedef typename C::L L;

  char* const spare = smem + C::STAGES * C::BUF;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform per wave
  const int lane = tid & 63, hl = lane >> 5, c32 = lane & 31;
  const int Sq = p.Sq, Sk = p.Sk;
  const bool causal = p.causal != 0;
  const int G = p.H / p.H_kv;
  const int n_qt = (Sq + BM - 1) / BM;

  const WorkItem wi = map_work(wg, p.n_units, p.units_per_xcd);
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
  const T* dOg = (const T*)p.dO + q_off * HD;
  const T* Kg = (const T*)p.k + kv_off;
  const T* Vg = (const T*)p.v + kv_off;

  F qf[NC], dof[NC];
  float lse2, dl;
  {
    const int mc = min(m, Sq - 1);
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      qf[cc] = ld8(Qg + (size_t)mc * HD + 16 * cc + 8 * hl);
      dof[cc] = ld8(dOg + (size_t)mc * HD + 16 * cc + 8 * hl);
    }
    if (p.stats_out != nullptr) {
      // Step 1 fused: D = sum_d dO * O of this lane's row, over the two lanes that hold it,
      // and the row's LSE in base 2 (a row with LSE = -inf attends no key and, like a
      // padding row, gets +inf).  The dK/dV kernel reads both from stats_out.
      const T* Og = (const T*)p.o + q_off * HD;
      float acc = 0.f;
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        const F of = ld8(Og + (size_t)mc * HD + 16 * cc + 8 * hl);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc += (float)dof[cc][e] * (float)of[e];
      }
      acc += __shfl_xor(acc, 32);
      const float lse = m < Sq ? p.lse[q_off + m] : -__builtin_inff();
      lse2 = lse == -__builtin_inff() ? __builtin_inff() : lse * kLog2e;
      dl = m < Sq ? acc : 0.f;
      if (hl == 0 && m < p.Sq_pad)
        *reinterpret_cast<float2*>(p.stats_out + ((size_t)(b * p.H + hq) * p.Sq_pad + m) * 2) =
            make_float2(lse2, dl);
    } else {
      const float* st = p.stats + ((size_t)(b * p.H + hq) * p.Sq_pad + mc) * 2;
      lse2 = m < Sq ? st[0] : __builtin_inff();
      dl = m < Sq ? st[1] : 0.f;
    }
  }

  f32x16 dq[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dq[db] = f32x16{};
  mma_ready(dq);

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

  // K and V tiles of the kv head through buffer resources: a tile is selected by a uniform
  // byte offset, keys past Sk read as zeros (and are masked), and the prefetches issued past
  // the last tile land in stages nothing reads any more.
  TileDma<T, HD, BN> kvdma;
  kvdma.init(w, lane);
  const rsrc_t rk = make_rsrc(Kg, (unsigned)((size_t)Sk * HD * sizeof(T)));
  const rsrc_t rv = make_rsrc(Vg, (unsigned)((size_t)Sk * HD * sizeof(T)));
  constexpr unsigned TILEB = BN * HD * sizeof(T);  // source bytes of one key tile
  auto issue_part = [&](int j, char* buf, int k) {
    kvdma.issue(k, buf, rk, (unsigned)j * TILEB, spare, lane);
    kvdma.issue(k, buf + C::TILE, rv, (unsigned)j * TILEB, spare, lane);
  };
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
#pragma unroll
    for (int k = 0; k < C::KMAX; ++k) issue_part(j_begin + s, smem + s * C::BUF, k);
  wait_vm_le<C::ISSUE * (STAGES - 2)>();  // Q, dO, statistics and stage 0 have landed
  barrier_lds();
  const float mask_s = p.mask_s;

  // One step of BN keys; restrict pointers as in the dK/dV kernel.  `nxt` receives the tile
  // STAGES - 1 steps ahead.
  auto step_body = [&](const char* __restrict__ cur, char* __restrict__ nxt, int j) {
    const int n0 = j * BN;
    f32x16 St[NB], dPt[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      St[nb] = f32x16{};
      dPt[nb] = f32x16{};
    }
    // ---- S^T = K Q^T and dP^T = V dO^T per 32-key block; the prefetch is spread over them.
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      if (cc < C::KMAX) issue_part(j + STAGES - 1, nxt, cc);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const F ak = lds_frag<T>(cur + L::rows(32 * nb), a_off[cc]);
        const F av = lds_frag<T>(cur + C::TILE + L::rows(32 * nb), a_off[cc]);
        mma(St[nb], ak, qf[cc]);
        mma(dPt[nb], av, dof[cc]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_sched_barrier(0);
    F da[NB][2];
    // Masking, only on steps that cut some row's keys (the causal diagonal, a window's
    // edges, the last key tile): a cut score is replaced by mask_s, whose exponent is -inf.
    // Register r of block nb holds key n0 + 32 nb + 4 hl + off(r), off = 8 (r / 4) + r % 4,
    // of row m (one row per lane); it may be seen iff kr.lo(m) <= key <= kr.hi(m).
    if (kr.hi(mw0) < n0 + BN - 1 || kr.lo(mw0 + 31) > n0) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int base = n0 + 32 * nb + 4 * hl;
        const int a = kr.lo(m) - base, z = kr.hi(m) - base;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = 8 * (r >> 2) + (r & 3);
          St[nb][r] = (off >= a && off <= z) ? St[nb][r] : mask_s;
        }
      }
    }
    // dS for register r of block nb.
    auto elem = [&](int nb, int r) {
      const float pv = fast_exp2(St[nb][r] * p.scale_log2 - lse2);
      da[nb][r >> 3][r & 7] = (T)(pv * (dPt[nb][r] - dl));
    };
    // ---- dQ += dS K, one 16-key slice (sl = 2 nb + ks) at a time; the dS of the next slice
    // is formed while the current slice's MFMAs run.
#pragma unroll
    for (int r = 0; r < 8; ++r) elem(0, r);
    constexpr int PER = (8 + NDB - 1) / NDB;  // next-slice elements per MFMA
#pragma unroll
    for (int sl = 0; sl < 2 * NB; ++sl) {
      const int nb = sl >> 1, ks = sl & 1;
      const int ro = L::rows(32 * nb + 16 * ks);
      F bk = lds_frag_tr<T>(cur, t_off[0][0] + ro, t_off[0][1] + ro);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        F bk_n;
        if (db + 1 < NDB) bk_n = lds_frag_tr<T>(cur, t_off[db + 1][0] + ro, t_off[db + 1][1] + ro);
        if (db == 0) mma_a<true>(dq[db], da[nb][ks], bk);  // first use of this dS slice
        else mma_a<false>(dq[db], da[nb][ks], bk);
        if (sl + 1 < 2 * NB) {
#pragma unroll
          for (int k = 0; k < PER; ++k)
            if (db * PER + k < 8) elem((sl + 1) >> 1, 8 * ((sl + 1) & 1) + db * PER + k);
        }
        if (db + 1 < NDB) bk = bk_n;
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  int cb = 0;  // buffer of step j
  for (int j = j_begin; j < j_end; ++j) {
    const int pb = cb == 0 ? STAGES - 1 : cb - 1;  // (j + STAGES - 1) % STAGES
    step_body(smem + cb * C::BUF, smem + pb * C::BUF, j);
    wait_vm_le<C::ISSUE * (STAGES - 2)>();  // tile j + 1 has landed
    barrier_lds();
    cb = cb == STAGES - 1 ? 0 : cb + 1;
  }
  wait_vm_all();  // no prefetch of this wave is still writing LDS ...
  barrier_lds();  // ... nor of any other: the stage buffers are free for the output tiles

  // ---- epilogue: dQ = scale * acc.  A lane's values lie down one column (16 rows of column
  // 32 db + c32), so each wave writes its 32 rows, rounded to 16 bits, into a row-major tile
  // of its own in LDS and stores that by whole rows: 16 bytes per lane instead of one 2-byte
  // element.  Rows are OROW bytes apart, so the two half-waves' writes (rows 4 apart: 16 banks
  // apart) never collide.
  mma_drain(dq);
  char* const otile = smem + w * (32 * C::OROW);
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 8 * (r >> 2) + 4 * hl + (r & 3);
      *reinterpret_cast<T*>(otile + row * C::OROW + 2 * (32 * db + c32)) = (T)(dq[db][r] * p.scale);
    }
  asm volatile("" ::: "memory");  // the wave reads back only what it wrote, in order
  T* dQg = (T*)p.dq + q_off * HD;
  constexpr int CPR = HD / 8;  // 16-byte chunks per row
#pragma unroll
  for (int i = 0; i < CPR / 2; ++i) {
    const int q = 64 * i + lane, row = q / CPR, ch = q % CPR;
    typedef T v8 __attribute__((ext_vector_type(8)));
    const v8 val = *reinterpret_cast<const v8*>(otile + row * C::OROW + 16 * ch);
    if (mw0 + row < Sq) *reinterpret_cast<v8*>(dQg + (size_t)(mw0 + row) * HD + 8 * ch) = val;
  }
}

template <class T, int HD, int NB>
__global__ __launch_bounds__(256, (HD <= 128 ? 2 : 1)) void bwd_dq16_kernel(const BwdParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[Dq16<HD, NB>::LDS];
  dq16_body<T, HD, NB>(p, blockIdx.x, smem);
}

// Key blocks of 32 per step of the dQ kernel (1: 32-key steps through a three-stage ring;
// 2: 64-key steps through a double buffer, which pays the per-step barrier, waits and
// scalar bookkeeping half as often and measures 2% faster at head dim 128).
#ifndef FAB_DQ_NB
#define FAB_DQ_NB 2
#endif
constexpr int kDqNB = FAB_DQ_NB;

// =======================================================================================
// Both recomputing step-2 kernels in one launch, for problems whose two grids together fit
// the device in one round: the first n_dkdv workgroups (rounded up to a multiple of the 8
// XCDs, so that the dQ workgroups keep the XCD order of their own grid; the padding ones
// exit at once) run the dK/dV body with 128-key tiles, the rest the dQ body.  Separate
// launches would leave half the device idle in each; here both halves run at once.  The
// row statistics come from a preprocess launch before it.
// =======================================================================================
template <class T, int HD>
__global__ __launch_bounds__(256) void bwd_small16_kernel(const BwdParams p, int n_dkdv, int n_dkdv_pad) {
  constexpr int L1 = Dkdv16<HD, false>::LDS, L2 = Dq16<HD, kDqNB>::LDS;
  __shared__ __attribute__((aligned(1024))) char smem[L1 > L2 ? L1 : L2];
  const int wg = blockIdx.x;
  if (wg < n_dkdv_pad) {
    if (wg < n_dkdv) dkdv16_body<T, HD, false>(p, wg, smem);
  } else {
    dq16_body<T, HD, kDqNB>(p, wg - n_dkdv_pad, smem);
  }
}

// =======================================================================================
// dQ from stored dS: once the dK/dV kernel has written every dS fragment, dQ = scale * dS K is
// a plain contraction, without recomputing S and dP.  A workgroup of eight waves owns 256
// query-row slots -- 128 rows of two query heads of one kv-head group when the group has an
// even number of heads, else 256 rows of one head -- and each wave 32 rows of one head.  Per
// step of 64 keys it stages the K tile, which all eight waves share, and each wave its own dS
// fragments in LDS by direct loads, and accumulates dQ in AGPRs.  The kernel streams dS from
// HBM once; what it moves besides is the K tile of every step, so a workgroup covers as many
// rows per K tile as the LDS allows.
// A stored fragment holds, for each of its 32 keys, 16 query rows: two 8-byte runs of four
// consecutive rows per lane half (see the dK/dV kernel).  The MFMA wants one query row per lane
// and keys along the 8 slots of its operand, so the fragment is read with the transposing LDS
// read: in a 16-lane group, lane 4 q + c addresses rows 4 c .. 4 c + 3 of key q0 + q, and lane
// i receives query row i of keys q0 .. q0 + 3.  The dS operand carries keys in natural order
// (slot t of lane half h: key 8 h + t of a 16-key slice), and so does the K operand, read
// transposed from the row-major K tile.
// =======================================================================================

// K tile of a stored-dS step: 64 rows of HD elements without padding, 16-byte chunk c of row r
// at r * 2 HD + 16 * (c ^ kswz(r)).  A transposed half-wave read (4 consecutive rows, 64 bytes
// of each) then covers four different 16-bank windows: rows of 256 or 512 bytes start on the
// same bank and are spread by the XOR, rows of 128 bytes alternate halves of the bank cycle
// and the XOR spreads row pairs, and rows of 64 or 192 bytes fall on distinct windows as they
// are.  kswz(r) depends only on r mod 4, so a slice of 16 rows further is a constant offset.
template <int HD>
__device__ __forceinline__ int kswz(int r) {
  if constexpr (HD == 128 || HD == 256) return 4 * (r & 3);
  else if constexpr (HD == 64) return 4 * ((r >> 1) & 1);
  else return 0;
}

template <int HD>
struct DqDs16 {
  static constexpr int NW = 8;                  // waves
  static constexpr int ROWS = 32 * NW;          // query-row slots of a workgroup
  static constexpr int BN = 64;                 // keys per step
  static constexpr int FRAG = 1024;             // one dS fragment: 32 keys x 16 rows
  // Row block r of a stage (its two fragments) starts at r * RB: the 128 bytes past the
  // fragments put the two row blocks a wave reads in one instruction on different banks.
  static constexpr int RB = 2 * FRAG + 128;
  static constexpr int DSB = 2 * NW * RB;       // dS part of a stage
  static constexpr int ROWB = 2 * HD;           // bytes per K row (16-bit elements)
  static constexpr int CPR = HD / 8;            // 16-byte chunks per K row
  static constexpr int KT = BN * ROWB;          // K tile
  static constexpr int KNI = KT / 1024;         // 1 KB direct loads per K tile
  static constexpr int KMAX = (KNI + NW - 1) / NW;  // ... issued by each wave
  static constexpr bool kSpare = NW * KMAX > KNI;   // waves past the tile load into `spare`
  static constexpr int SPARE = kSpare ? 1024 : 0;
  static constexpr int BUF = DSB + KT;
  static constexpr int STAGES_FIT = (160 * 1024 - SPARE) / BUF;
  static constexpr int STAGES = STAGES_FIT > 4 ? 4 : STAGES_FIT;
  static constexpr int LDS = STAGES * BUF + SPARE;
  static constexpr int ISSUE = KMAX + 4;        // loads each wave issues per stage
  static constexpr int OROW = HD * 2 + 16;      // epilogue: row pitch of the 16-bit output tile
  static_assert(KT % 1024 == 0, "whole direct loads per K tile");
  static_assert(STAGES >= 2, "a double buffer at least");
  static_assert(NW * 32 * OROW <= LDS, "the output tiles of the waves fit the staging buffers");
  static_assert(BUF % 16 == 0 && RB % 256 == 128, "granule alignment, banks");
};

template <class T, int HD>
__global__ __launch_bounds__(512, 1) void bwd_dq_ds16_kernel(const BwdParams p) {
  typedef DqDs16<HD> C;
  typedef typename Frag<T>::type F;
  constexpr int NDB = HD / 32, BN = C::BN, STAGES = C::STAGES, NW = C::NW;

  __shared__ __attribute__((aligned(1024))) char smem[C::LDS];
  char* const spare = smem + STAGES * C::BUF;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform per wave
  const int lane = tid & 63, c32 = lane & 31, hl = lane >> 5;
  const int Sq = p.Sq, Sk = p.Sk;
  const int G = p.H / p.H_kv;
  // Two heads of the group per workgroup when G is even (128 rows each), else one (256 rows).
  const int NH = (G & 1) ? 1 : 2;
  const int RPH = C::ROWS / NH;                 // rows per head in the workgroup
  const int WPH = NW / NH;                      // waves per head
  const int n_qt = (Sq + RPH - 1) / RPH;

  const WorkItem wi = map_work(blockIdx.x, p.n_units, p.units_per_xcd);
  const int b = wi.unit / p.H_kv, g = wi.unit % p.H_kv;
  const int hs = wi.step % (G / NH), tq = wi.step / (G / NH);
  const int it = p.causal ? n_qt - 1 - tq : tq;  // heaviest query tiles first
  const int hq = g * G + hs * NH + w / WPH;      // this wave's query head
  const int m0 = it * RPH;
  const int mw0 = m0 + 32 * (w % WPH);           // this wave's first row

  const size_t q_off = (size_t)(b * p.H + hq) * Sq;
  const T* Kg = (const T*)p.k + (size_t)(b * p.H_kv + g) * Sk * HD;

  f32x16 dq[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dq[db] = f32x16{};
  mma_ready(dq);

  // Per-lane LDS offsets of the transposed reads.  16-lane group grp = lane / 16: lane half
  // h = grp / 2 (keys 8 h ..), and sub = grp % 2 selects the wave's second row block (dS) or
  // the second 16 columns of a 32-column block of K; in the group, lane 4 q + c.
  const int grp = lane >> 4, hh = grp >> 1, sub = grp & 1, qd = (lane >> 2) & 3, cq = lane & 3;
  // dS: key 8 hh + 4 sec + qd of a 16-key slice, rows 4 cq .. 4 cq + 3 of row block 2 w + sub;
  // slice sl adds (sl / 2) fragments and (sl % 2) * 16 keys, sec = 1 four keys.
  const int ds_off = (2 * w + sub) * C::RB + 32 * (8 * hh + qd) + 16 * (cq & 1) + 8 * (cq >> 1);
  // K: key row 8 hh + 4 sec + qd of the slice, columns 32 db + 16 sub + 4 cq .. + 3.
  int k_off[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int sec = 0; sec < 2; ++sec) {
      const int r = 8 * hh + 4 * sec + qd;
      const int col = 32 * db + 16 * sub + 4 * cq;
      k_off[db][sec] = C::DSB + r * C::ROWB + 16 * ((col >> 3) ^ kswz<HD>(r)) + 2 * (col & 7);
    }

  // key tiles holding a key some row of the workgroup may attend
  const KeyRange kr{Sk, p.causal, p.win};
  const int k_lo = kr.lo(m0), k_hi = kr.hi(min(m0 + RPH, Sq) - 1);
  const int j_begin = k_lo / BN;
  const int j_end = k_hi >= k_lo ? k_hi / BN + 1 : j_begin;

  // The dS fragments of a row block exist (were written by the dK/dV kernel) where the block
  // sees some key of the key block; the others are never written and read as zeros here.
  // This lane's row block (2 w + sub of the workgroup) sees keys [v_lo, v_hi]; rows past Sq
  // carry nothing (their dQ is not stored), so their block is left empty.
  const int rb0 = mw0 + 16 * sub;
  const int v_lo = rb0 < Sq ? kr.lo(rb0) : 1;
  const int v_hi = rb0 < Sq ? kr.hi(min(rb0 + 15, Sq - 1)) : 0;

  // Loads: the K tile through buffer loads (keys past Sk read as zeros), spread over the
  // waves, and each wave's own dS fragments (its two row blocks x the step's two key blocks)
  // from the slab of its head.  The prefetches issued past the last step land in stages
  // nothing reads any more (their offsets read zeros past the tensor or the slab).
  const rsrc_t rk = make_rsrc(Kg, (unsigned)((size_t)Sk * HD * sizeof(T)));
  const rsrc_t rds = make_rsrc((const char*)p.ds + (size_t)(b * p.H + hq) * p.ds_slab, p.ds_slab);
  unsigned k_src[C::KMAX];  // this lane's source offset in the K tile, per instruction
#pragma unroll
  for (int k = 0; k < C::KMAX; ++k) {
    const int gidx = 64 * (w + NW * k) + lane;  // granule of the tile image
    const int r = gidx / C::CPR, slot = gidx % C::CPR;
    k_src[k] = (unsigned)(r * C::ROWB + 16 * (slot ^ kswz<HD>(r)));
  }
  const unsigned ds_row = (unsigned)((mw0 >> 7) * p.ds_nk32) * 8u + (unsigned)((mw0 >> 4) & 7);
  auto issue_part = [&](int j, char* buf, int k) {
    if (k < C::KMAX) {
      const int q = w + NW * k;
      char* dst = (!C::kSpare || q < C::KNI) ? buf + C::DSB + 1024 * q : spare;
      b2lds16(rk, k_src[k], (unsigned)j * C::KT, dst);
    }
    if (k < 4) {
      const int rbw = k & 1, kb = k >> 1;
      b2lds16<FAB_DS_LOAD_AUX>(rds, 16u * lane, (ds_row + (unsigned)(2 * j + kb) * 8u + rbw) * 1024u,
                               buf + (2 * w + rbw) * C::RB + kb * C::FRAG);
    }
  };
  constexpr int NPART = C::KMAX > 4 ? C::KMAX : 4;
#pragma unroll
  for (int st = 0; st < STAGES - 1; ++st)
#pragma unroll
    for (int k = 0; k < NPART; ++k) issue_part(j_begin + st, smem + st * C::BUF, k);
  wait_vm_le<C::ISSUE * (STAGES - 2)>();  // stage 0 has landed
  barrier_lds();

  // One step of BN keys on stage `cur`; `nxt` receives the stage STAGES - 1 steps ahead.
  auto step_body = [&](const char* __restrict__ cur, char* __restrict__ nxt, int j) {
    const int n0 = j * BN;
    // Steps where some row of the wave may not see some key read the validity of each dS
    // fragment; elsewhere every fragment was written.
    const bool edge = kr.hi(mw0) < n0 + BN - 1 || kr.lo(mw0 + 31) > n0;
    bool valid[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key0 = n0 + 32 * kb;
      valid[kb] = v_lo <= v_hi && key0 <= v_hi && key0 + 31 >= v_lo;
    }
    int part = 0;
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) {
      const int kb = sl >> 1, ks = sl & 1;
      const int so = kb * C::FRAG + ks * 512;  // slice offset in a row block
      F a = lds_frag_tr<T>(cur, ds_off + so, ds_off + so + 128);
      if (edge && !valid[kb]) a = zero8<T>();
      const int ro = 16 * sl * C::ROWB;
      F bk = lds_frag_tr<T>(cur, k_off[0][0] + ro, k_off[0][1] + ro);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        F bk_n;
        if (db + 1 < NDB) bk_n = lds_frag_tr<T>(cur, k_off[db + 1][0] + ro, k_off[db + 1][1] + ro);
        if (db == 0) mma_a<true>(dq[db], a, bk);  // first use of this slice's dS operand
        else mma_a<false>(dq[db], a, bk);
        if (part < NPART) issue_part(j + STAGES - 1, nxt, part++);
        if (db + 1 < NDB) bk = bk_n;
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    while (part < NPART) issue_part(j + STAGES - 1, nxt, part++);
  };

  int cb = 0;  // buffer of step j
  for (int j = j_begin; j < j_end; ++j) {
    const int pb = cb == 0 ? STAGES - 1 : cb - 1;  // (j + STAGES - 1) % STAGES
    step_body(smem + cb * C::BUF, smem + pb * C::BUF, j);
    wait_vm_le<C::ISSUE * (STAGES - 2)>();  // stage j + 1 has landed
    barrier_lds();
    cb = cb == STAGES - 1 ? 0 : cb + 1;
  }
  wait_vm_all();  // no prefetch of this wave is still writing LDS ...
  barrier_lds();  // ... nor of any other: the stage buffers are free for the output tiles

  // ---- epilogue: dQ = scale * acc, staged through a row-major tile per wave and stored by
  // whole rows (16 bytes per lane), as in the recomputing dQ kernel.
  mma_drain(dq);
  char* const otile = smem + w * (32 * C::OROW);
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 8 * (r >> 2) + 4 * hl + (r & 3);
      *reinterpret_cast<T*>(otile + row * C::OROW + 2 * (32 * db + c32)) = (T)(dq[db][r] * p.scale);
    }
  asm volatile("" ::: "memory");  // the wave reads back only what it wrote, in order
  T* dQg = (T*)p.dq + q_off * HD;
  constexpr int CPR = HD / 8;  // 16-byte chunks per row
#pragma unroll
  for (int i = 0; i < CPR / 2; ++i) {
    const int q = 64 * i + lane, row = q / CPR, ch = q % CPR;
    typedef T v8 __attribute__((ext_vector_type(8)));
    const v8 val = *reinterpret_cast<const v8*>(otile + row * C::OROW + 16 * ch);
    if (mw0 + row < Sq) *reinterpret_cast<v8*>(dQg + (size_t)(mw0 + row) * HD + 8 * ch) = val;
  }
}

template <class T, int HD, bool WIDE>
static hipError_t go_dkdv_cfg(const BwdParams& p, hipStream_t s, LaunchInfo* info) {
  typedef Dkdv16<HD, WIDE> C;
  const int n_kt = (p.Sk + C::BN - 1) / C::BN;
  const int grid = p.n_units * n_kt;
  if (info) *info = LaunchInfo{WIDE ? "bwd_dkdv16_wide" : "bwd_dkdv16", grid, 256, C::LDS};
  hipLaunchKernelGGL((bwd_dkdv16_kernel<T, HD, WIDE>), dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

// Compute units of the current device (queried once per process).
static int device_cus() {
  static const int n = [] {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
      (void)hipGetLastError();
      return 256;
    }
    return cus;
  }();
  return n;
}

// The wide (256-key) workgroups halve the per-workgroup fixed cost, but one workgroup per CU
// leaves the heaviest-first order nothing to balance: they are used only where the grid still
// gives every CU at least two of them.
template <class T, int HD>
static hipError_t go_dkdv(const BwdParams& p, hipStream_t s, LaunchInfo* info) {
  if constexpr (HD <= 128) {
    const long long wide_grid = (long long)p.n_units * ((p.Sk + 255) / 256);
    if (wide_grid >= 2LL * device_cus()) return go_dkdv_cfg<T, HD, true>(p, s, info);
  }
  return go_dkdv_cfg<T, HD, false>(p, s, info);
}

template <class T, int HD>
static hipError_t go_dq(const BwdParams& p, hipStream_t s, LaunchInfo* info) {
  typedef Dq16<HD, kDqNB> C;
  const int n_qt = (p.Sq + C::BM - 1) / C::BM;
  const int grid = p.n_units * (p.H / p.H_kv) * n_qt;
  if (info) *info = LaunchInfo{"bwd_dq16", grid, 256, C::LDS};
  hipLaunchKernelGGL((bwd_dq16_kernel<T, HD, kDqNB>), dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <class T, int HD>
static hipError_t go_dq_ds(const BwdParams& p, hipStream_t s, LaunchInfo* info) {
  typedef DqDs16<HD> C;
  const int G = p.H / p.H_kv, NH = (G & 1) ? 1 : 2;
  const int n_qt = (p.Sq + C::ROWS / NH - 1) / (C::ROWS / NH);
  const int grid = p.n_units * (G / NH) * n_qt;
  if (info) *info = LaunchInfo{"bwd_dq_ds16", grid, 64 * C::NW, C::LDS};
  hipLaunchKernelGGL((bwd_dq_ds16_kernel<T, HD>), dim3(grid), dim3(64 * C::NW), 0, s, p);
  return hipGetLastError();
}

template <class T>
static hipError_t dq_ds_hd(const BwdParams& p, int hd, hipStream_t s, LaunchInfo* info) {
  switch (hd) {
    case 32: return go_dq_ds<T, 32>(p, s, info);
    case 64: return go_dq_ds<T, 64>(p, s, info);
    case 96: return go_dq_ds<T, 96>(p, s, info);
    case 128: return go_dq_ds<T, 128>(p, s, info);
    default: return go_dq_ds<T, 256>(p, s, info);
  }
}

template <class T>
static hipError_t dkdv_hd(const BwdParams& p, int hd, hipStream_t s, LaunchInfo* info) {
  switch (hd) {
    case 32: return go_dkdv<T, 32>(p, s, info);
    case 64: return go_dkdv<T, 64>(p, s, info);
    case 96: return go_dkdv<T, 96>(p, s, info);
    case 128: return go_dkdv<T, 128>(p, s, info);
    default: return go_dkdv<T, 256>(p, s, info);
  }
}

template <class T>
static hipError_t dq_hd(const BwdParams& p, int hd, hipStream_t s, LaunchInfo* info) {
  switch (hd) {
    case 32: return go_dq<T, 32>(p, s, info);
    case 64: return go_dq<T, 64>(p, s, info);
    case 96: return go_dq<T, 96>(p, s, info);
    case 128: return go_dq<T, 128>(p, s, info);
    default: return go_dq<T, 256>(p, s, info);
  }
}

// Workgroups of the two recomputing step-2 kernels when they share one launch (128-key dK/dV
// tiles, the dK/dV count rounded up to whole rounds of the XCDs) and whether that launch fits
// the device in one round.
static void small_counts(const BwdParams& p, int hd, int& n_dkdv, int& n_dkdv_pad, int& n_dq) {
  const int bn = hd == 256 ? Dkdv16<256, false>::BN : Dkdv16<128, false>::BN;
  n_dkdv = p.n_units * ((p.Sk + bn - 1) / bn);
  n_dkdv_pad = (n_dkdv + 7) / 8 * 8;
  n_dq = p.n_units * (p.H / p.H_kv) * ((p.Sq + 127) / 128);
}

bool bwd_small16_fits(const BwdParams& p, int hd) {
  int n_dkdv, n_pad, n_dq;
  small_counts(p, hd, n_dkdv, n_pad, n_dq);
  return (long long)n_pad + n_dq <= device_cus();
}

template <class T, int HD>
static hipError_t go_small(const BwdParams& p, hipStream_t s, LaunchInfo* info) {
  int n_dkdv, n_pad, n_dq;
  small_counts(p, HD, n_dkdv, n_pad, n_dq);
  constexpr int L1 = Dkdv16<HD, false>::LDS, L2 = Dq16<HD, kDqNB>::LDS;
  if (info) *info = LaunchInfo{"bwd_small16", n_pad + n_dq, 256, L1 > L2 ? L1 : L2};
  hipLaunchKernelGGL((bwd_small16_kernel<T, HD>), dim3(n_pad + n_dq), dim3(256), 0, s, p, n_dkdv, n_pad);
  return hipGetLastError();
}

template <class T>
static hipError_t small_hd(const BwdParams& p, int hd, hipStream_t s, LaunchInfo* info) {
  switch (hd) {
    case 32: return go_small<T, 32>(p, s, info);
    case 64: return go_small<T, 64>(p, s, info);
    case 96: return go_small<T, 96>(p, s, info);
    case 128: return go_small<T, 128>(p, s, info);
    default: return go_small<T, 256>(p, s, info);
  }
}

hipError_t launch_bwd_small16(const BwdParams& p, int dt, int hd, hipStream_t s, LaunchInfo* info) {
  return dt == kBF16 ? small_hd<bf16>(p, hd, s, info) : small_hd<f16>(p, hd, s, info);
}

hipError_t launch_bwd_dkdv16(const BwdParams& p, int dt, int hd, hipStream_t s, LaunchInfo* info) {
  return dt == kBF16 ? dkdv_hd<bf16>(p, hd, s, info) : dkdv_hd<f16>(p, hd, s, info);
}

hipError_t launch_bwd_dq16(const BwdParams& p, int dt, int hd, hipStream_t s, LaunchInfo* info) {
  return dt == kBF16 ? dq_hd<bf16>(p, hd, s, info) : dq_hd<f16>(p, hd, s, info);
}

hipError_t launch_bwd_dq_ds16(const BwdParams& p, int dt, int hd, hipStream_t s, LaunchInfo* info) {
  return dt == kBF16 ? dq_ds_hd<bf16>(p, hd, s, info) : dq_ds_hd<f16>(p, hd, s, info);
}

}  // namespace fab
