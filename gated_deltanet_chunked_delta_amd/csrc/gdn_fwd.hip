// gdn_fwd.hip -- forward chunk loop of the gated delta rule on gfx950.
//
// One workgroup owns one (segment, head): a run of consecutive 64-token chunks
// of one sequence.  It has Dv/16 waves when Dv = 128 (eight, two per SIMD) and
// four otherwise; wave w keeps the 16-column slices [16 w NTW, 16 (w+1) NTW)
// (NTW = Dv / (16 waves)) of the fp32 state h = S^T (Dk x Dv) in accumulator
// registers for the whole run, so
// the serial chain U = Ut - W h, h' = Gam_C h + Kt^T U never leaves registers.
// Everything that does not depend on h (decay cumsum, the decay-masked K K^T,
// the unit-lower-triangular solve, W and Ut, the masked Q K^T) is computed
// per chunk from LDS tiles by all waves together, while the next chunk's
// q/k/v/g/beta are already on their way from HBM into registers.
//
// Chunk algebra (rows r, i of one chunk; gam = inclusive cumsum of g):
//   A  = strict_lower(diag(beta) (K K^T) * exp(gam_r - gam_i))
//   T  = (I + A)^-1,  W = T diag(beta exp(gam)) K,  Ut = T diag(beta) V
//   U  = Ut - W h
//   O  = scale (diag(exp(gam)) Q h + P U),  P = (Q K^T) * exp(gam_r - gam_i) * [i <= r]
//   h' = exp(gam_last) h + K^T diag(exp(gam_last - gam)) U
// This is the "hardware-friendly algebraic reformulation" the "FlashQLA
// resource" page lists (section 3) in its exact form: it equals the token
// recurrence up to rounding.
//
// Intra-card context parallelism ("FlashQLA resource", section 3: gate-driven,
// automatic, for long sequences and few heads).  The plan cuts each sequence
// into segments, one workgroup each, all independent.  A segment that does not
// start its sequence starts from a zero state some chunks earlier, at the
// latest chunk wb with  sum_{c=wb}^{cb-1} Lambda_c <= ln 2^-24, where
// Lambda_c = sum over the chunk's tokens of g_t + log max(1, |1 - beta_t |k_t|^2|)
// bounds log ||transition||_2 (||I - beta k k^T||_2 = max(1, |1 - beta |k|^2|)).
// Those lead-in chunks only advance the state; from chunk cb on, the state
// differs from the true one by the true state at wb carried through chunks
// wb..cb-1, at most 2^-24 of its norm, i.e. fp32 round-off.  Where the bound is
// not reached (weak decay) the run starts at the sequence start from h0 and is
// exact; the gate decay usually makes the lead-in a few chunks long.
//
// The same kernels, without an output, replay the forward for the backward
// pass and store the state at every chunk start.
#include <type_traits>

#include <cstddef>

#include "gdn_device.h"
#include "gdn_internal.h"
#include "gdn_tiles.h"

namespace gdn {

// Every tile is row-major.  Products that need the columns of K or V read them
// with LDS transpose loads, from copies whose bf16 rows are padded by 16
// elements (which keeps the transpose loads free of bank conflicts); the
// tiles read along their rows (Q, W, P, T, and K once more for Q K^T) are
// padded by 4, where 8-byte row reads run at full rate and 16 would not.
template <class E, int DK, int DV>
struct alignas(16) FwdSmem {
  static constexpr int LQ = ldpad<E>(DK);                 // sQ, sKR, sW row stride
  static constexpr int LT = ldpad<E>(CH);                 // P, scaled T
  static constexpr int LO = DV + 16 / (int)sizeof(E);     // output staging (16-byte rows)
  static constexpr int PADC = sizeof(E) == 2 ? 16 : 4;    // tiles read through transpose loads
  static constexpr int LK = DK + PADC;
  static constexpr int LV = DV + PADC;
  E Q[CH * LQ];
  E KR[CH * LQ];  // K, for its rows
  E K[CH * LK];   // K, for its columns
  E V[CH * LV];
  E W[CH * LQ];   // holds -W
  E P[CH * LT];
  E TBG[CH * LT];  // T diag(beta Gam), the X operand of W
  E TB[CH * LT];   // T diag(beta), the X operand of Ut
  E O[CH * LO];
  // the chunk's scalar record, as laid out in memory (tail: Lambda_c, Gam_C)
  alignas(16) float gam[CH], Gam[CH], ek[CH], beta[CH], bg[CH], tail[4];
};

// ------------------------------------------------------------------ prefetch

// The raw tiles of one chunk, held in registers between the global load and
// the LDS store so that the next chunk's loads overlap the current chunk's
// compute.  K and V move as 4-row x 16-byte blocks, Q as single 16-byte
// vectors, all stored row-major (K twice, at the two strides).  The loads, and
// those of T, are non-temporal: the forward ran shorter so, the replay much
// shorter.
template <class E, int DK, int DV, int NT, bool NEED_Q, bool NEED_V, bool PREP>
struct TileLoader {
  static constexpr int VEC = 16 / (int)sizeof(E);
  static constexpr int NBK = (CH / 4) * (DK / VEC);
  static constexpr int NBV = NEED_V ? (CH / 4) * (DV / VEC) : 0;
  static constexpr int NB = (NBK + NBV + NT - 1) / NT;     // blocks per thread
  static constexpr int NQV = NEED_Q ? (CH * (DK / VEC) + NT - 1) / NT : 0;
  typedef E vec_t __attribute__((__vector_size__(16)));
  vec_t blk[NB > 0 ? NB : 1][4];
  vec_t qv[NQV > 0 ? NQV : 1];
  f32x4 rv;  // this thread's piece of the chunk's scalar record (threads < RECF / 4)

  __device__ __forceinline__ void load(const FwdParams& p, int64_t tok0, int rows, int h, const float* rec) {
    load_kv(p, tok0, rows, h, rec);
    load_q(p, tok0, rows, h);
  }

  // K / V blocks and the scalar record
  __device__ __forceinline__ void load_kv(const FwdParams& p, int64_t tok0, int rows, int h, const float* rec) {
    const int H = p.H;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int id = threadIdx.x + b * NT;
      if (id < NBK + NBV) {
        const bool isk = id < NBK;
        const int loc = isk ? id : id - NBK;
        const int D = isk ? DK : DV;
        const int r0 = (loc / (D / VEC)) * 4, c0 = (loc % (D / VEC)) * VEC;
        const E* src = static_cast<const E*>(isk ? p.k : p.v) + (tok0 * H + h) * D + c0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (r0 + j < rows)
            blk[b][j] = __builtin_nontemporal_load(reinterpret_cast<const vec_t*>(src + (int64_t)(r0 + j) * H * D));
          else
            for (int e = 0; e < VEC; ++e) blk[b][j][e] = (E)0.f;
        }
      }
    }
    if (threadIdx.x < RECF / 4) rv = *reinterpret_cast<const f32x4*>(rec + 4 * threadIdx.x);
  }

  __device__ __forceinline__ void load_q(const FwdParams& p, int64_t tok0, int rows, int h) {
    const int H = p.H;
#pragma unroll
    for (int v = 0; v < NQV; ++v) {
      const int id = threadIdx.x + v * NT;
      if (id < CH * (DK / VEC)) {
        const int r = id / (DK / VEC), c0 = (id % (DK / VEC)) * VEC;
        if (r < rows)
          qv[v] = __builtin_nontemporal_load(
              reinterpret_cast<const vec_t*>(static_cast<const E*>(p.q) + ((tok0 + r) * H + h) * DK + c0));
        else
          for (int e = 0; e < VEC; ++e) qv[v][e] = (E)0.f;
      }
    }
  }
  // the scalar record into LDS (gam .. tail are contiguous there as in memory)
  template <class S>
  __device__ __forceinline__ void store_rec(S& s) const {
    static_assert(offsetof(S, tail) == offsetof(S, gam) + 5 * CH * sizeof(float), "record layout");
    if (threadIdx.x < RECF / 4) *reinterpret_cast<f32x4*>(&s.gam[4 * threadIdx.x]) = rv;
  }

  // Divide every row of K and Q by its L2 norm (q / k pre-processing).  A row's
  // DK/VEC vectors sit on consecutive lanes, and K / V blocks never share a
  // wave; every lane of the workgroup must call this.
  __device__ __forceinline__ void normalize() {
    constexpr int BPR = DK / VEC;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const bool isk = threadIdx.x + b * NT < NBK;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) ss += to_f(blk[b][j][e]) * to_f(blk[b][j][e]);
        ss = lane_group_sum<BPR>(isk ? ss : 0.f);
        const float sc = rsqrtf(ss + QK_NORM_EPS);
        if (isk) {
#pragma unroll
          for (int e = 0; e < VEC; ++e) blk[b][j][e] = to_e<E>(to_f(blk[b][j][e]) * sc);
        }
      }
    }
#pragma unroll
    for (int v = 0; v < NQV; ++v) {
      const bool valid = threadIdx.x + v * NT < CH * (DK / VEC);
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) ss += to_f(qv[v][e]) * to_f(qv[v][e]);
      ss = lane_group_sum<BPR>(valid ? ss : 0.f);
      const float sc = rsqrtf(ss + QK_NORM_EPS);
#pragma unroll
      for (int e = 0; e < VEC; ++e) qv[v][e] = to_e<E>(to_f(qv[v][e]) * sc);
    }
  }

  template <class S>
  __device__ __forceinline__ void store(S& s) const {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int id = threadIdx.x + b * NT;
      if (id < NBK + NBV) {
        const bool isk = id < NBK;
        const int loc = isk ? id : id - NBK;
        const int D = isk ? DK : DV;
        const int r0 = (loc / (D / VEC)) * 4, c0 = (loc % (D / VEC)) * VEC;
        E* dst = isk ? s.K : s.V;
        const int ld = isk ? S::LK : S::LV;
#pragma unroll
        for (int j = 0; j < 4; ++j) *reinterpret_cast<vec_t*>(dst + (r0 + j) * ld + c0) = blk[b][j];
        if (NEED_Q && isk) {  // the row copy serves Q K^T, which only the forward proper forms
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < VEC; e += 4)
              st4<E>(s.KR + (r0 + j) * S::LQ + c0 + e, blk[b][j][e], blk[b][j][e + 1], blk[b][j][e + 2],
                     blk[b][j][e + 3]);
        }
      }
    }
#pragma unroll
    for (int v = 0; v < NQV; ++v) {
      const int id = threadIdx.x + v * NT;
      if (id < CH * (DK / VEC)) {
        const int r = id / (DK / VEC), c0 = (id % (DK / VEC)) * VEC;
#pragma unroll
        for (int e = 0; e < VEC; e += 4)
          st4<E>(s.Q + r * S::LQ + c0 + e, qv[v][e], qv[v][e + 1], qv[v][e + 2], qv[v][e + 3]);
      }
    }
  }
};

// ------------------------------------------------------------------ one chunk

// Phases of the forward's phase clock: 0 before the first chunk; per chunk 1
// staging, 2 P and T's landing, 3 -W and Ut, 4 the state chain, 5 the output
// stores; 6 after the last chunk; slot 7 counts the chunks run.
using FwdClock = PhaseClock<8>;
// [forward, replay][workgroup][wave][phase] (an instrumented build only)
__device__ uint32_t gdn_clock_fwd[kPhaseClock ? 2 : 1][kPhaseClock ? CLOCK_BLOCKS : 1][8 * 8];

// OUT:  forward (writes o) vs replay (no output).  Either stores the chunk-start
//       state when p.hs is set.
// Waves per workgroup: 8 when the state has 128 value columns (one 16-column
// tile per wave, two waves per SIMD), else 4.
template <int DV>
struct FwdWaves { static constexpr int NW = DV == 128 ? 8 : 4; };

// Every chunk's T and scalar record are read from p.t_in / p.rec (written by
// the chunk-parallel T solve beforehand).
// USAVE: every chunk's U is written to p.us.
template <class E, int DK, int DV, bool OUT, bool PREP, bool USAVE>
struct Chunk {
  static constexpr int NW = FwdWaves<DV>::NW;
  static constexpr int NT = NW * 64;
  static constexpr int NTW = DV / (16 * NW);  // 16-column tiles of the state per wave
  using S = FwdSmem<E, DK, DV>;
  using Loader = TileLoader<E, DK, DV, NT, OUT, true, PREP>;

  // One lower 16x16 tile (rt, ct) of P = (Q K^T) * M, formed transposed (key
  // rows, query columns) so that each lane stores four consecutive entries of
  // a row of P at once.
  __device__ __forceinline__ static void p_tile(S* sp, int rt, int ct, int g, int c16) {
    constexpr int LQ = S::LQ, LT = S::LT;
    f32x4 acc = zero4();
#pragma unroll
    for (int kb = 0; kb < DK / 32; ++kb)
      mma(acc, ld_frag(sp->KR, LQ, 16 * ct + c16, 32 * kb), ld_frag(sp->Q, LQ, 16 * rt + c16, 32 * kb));
    const f32x4 gc4 = *reinterpret_cast<const f32x4*>(&sp->gam[16 * ct + 4 * g]);
    const int r = 16 * rt + c16;
    const float gr = sp->gam[r];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = 16 * ct + 4 * g + i;
      acc[i] = (c <= r) ? acc[i] * __expf(gr - gc4[i]) : 0.f;
    }
    st_tile_cm<E>(sp->P, LT, 16 * ct, 16 * rt, acc);
  }

  // A chunk's stores that wait for the next chunk: its U (the replay, from
  // registers) and its output tile (the forward proper, from LDS, where the
  // next chunk writes O only in its state-chain phase).  Loads and stores
  // retire through one counter, and at the next chunk's start the compiler's
  // wait for the prefetched tiles also covered the stores issued after them
  // (it cannot count the stores of a loop iteration exactly), so stores issued
  // at the end of a chunk were waited for there in full.  Held back to just
  // after the next chunk's T lands (its last load wait before the state
  // chain), they complete during the chain.
  struct Held {
    f32x4 u[4][NTW];
    E* us = nullptr;   // where the held U goes (none held: nullptr)
    E* ulo = nullptr;  // and its rounding residual (bf16)
    int64_t otok0 = 0;
    int orows = 0;     // rows of the held output tile (none held: 0)
  };
  __device__ static void flush(S* sp, const FwdParams& p, Held& hd, int h) {
    constexpr bool ULO = USAVE && std::is_same<E, bf16>::value;
    const int tid = threadIdx.x, n0 = wave_id() * (DV / NW);
    if constexpr (USAVE && !OUT) {
      // U as DV/16 column blocks of [CH][16], each contiguous (a wave's stores
      // fill whole lines; rows past the end are zero: beta = 0 there)
      if (hd.us) {
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
          for (int nt = 0; nt < NTW; ++nt) {
            st_tile_rows<E>(hd.us + (n0 + 16 * nt) * CH, 16, 16 * rt, 0, hd.u[rt][nt]);
            if constexpr (ULO) st_tile_rows<E>(hd.ulo + (n0 + 16 * nt) * CH, 16, 16 * rt, 0, bf16_residual(hd.u[rt][nt]));
          }
        hd.us = nullptr;
      }
    }
    if constexpr (OUT) {
      // the output tile, coalesced
      constexpr int OVEC = 16 / (int)sizeof(E), LO = S::LO;
      typedef E ovec_t __attribute__((__vector_size__(16)));
      for (int e = tid; e < hd.orows * (DV / OVEC); e += NT) {
        const int r = e / (DV / OVEC), c0 = (e % (DV / OVEC)) * OVEC;
        st_out(reinterpret_cast<ovec_t*>(static_cast<E*>(p.o) + ((hd.otok0 + r) * p.H + h) * DV + c0),
               *reinterpret_cast<const ovec_t*>(&sp->O[r * LO + c0]));
      }
      hd.orows = 0;
    }
  }

  // Process the chunk whose tiles `ld` holds; prefetch the next chunk (if any)
  // into `ld`.  hacc: this wave's state columns (chunk start on entry, chunk end
  // on exit).  LEAD: a lead-in chunk before the segment proper, which only
  // advances the state (nothing is written).
  // t_in: this chunk's T; nrec: the next chunk's scalar record.
  // us_chunk: where this chunk's U = Ut - W h goes (nullable).  hd: the
  // previous chunk's held stores (issued here), then this chunk's.
  template <bool LEAD>
  __device__ static void step(S& s0, const FwdParams& p, Loader& ld, int64_t tok0, int rows, int64_t ntok0,
                              int nrows, int h, E* hs_chunk, const float* t_in, const float* nrec, E* us_chunk,
                              E* ulo_chunk, f32x4 (&hacc)[DK / 16][NTW], Held& hd, FwdClock& clk) {
    constexpr bool OUTC = OUT && !LEAD, USAVEC = USAVE && !LEAD;
    constexpr int LQ = S::LQ, LT = S::LT, LO = S::LO;
    const int tid = threadIdx.x, l = lane_id(), w = wave_id(), g = l >> 4, c16 = l & 15;
    const int H = p.H;
    const int n0 = w * (DV / NW);  // first state column of this wave

    // T (its bf16 value plane for bf16 inputs) is requested first and lands
    // in LDS at the end of phase 2
    TPart<E, NT> tp;
    tp.template load<true>(t_in);

    // ---- 1. tiles into LDS, scalars, prefetch of the next chunk
    S* sp = lds_opaque(&s0);
    if (PREP && p.prep.qk_norm) ld.normalize();
    ld.store(*sp);
    ld.store_rec(*sp);
    __syncthreads();
    clk.mark(1);
    sp = lds_opaque(sp);

    // ---- 2. for the output, the ten lower 16x16 tiles of P = (Q K^T) * M, tile j
    //         on wave j % NW (at most two tiles a wave with eight waves)
    if constexpr (OUTC) {
#pragma unroll
      for (int j = 0; j < (10 + NW - 1) / NW; ++j) {
        const int pid = w + NW * j;
        const int rt = pid < 1 ? 0 : (pid < 3 ? 1 : (pid < 6 ? 2 : 3));
        const int ct = pid - (rt * (rt + 1)) / 2;
        if (pid < 10) p_tile(sp, rt, ct, g, c16);
      }
    }
    // T lands as its two column-scaled operands (scaled in fp32, rounded once)
#pragma unroll
    for (int i = 0; i < TPart<E, NT>::NP; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int e = 8 * (tid + i * NT) + 4 * j, r = e / CH, c = e % CH;
        const f32x4 bg4 = *reinterpret_cast<const f32x4*>(&sp->bg[c]);
        const f32x4 bt4 = *reinterpret_cast<const f32x4*>(&sp->beta[c]);
        const f32x4 tv = tp.get(i, j);
        st4f<E>(&sp->TBG[r * LT + c], tv * bg4);
        st4f<E>(&sp->TB[r * LT + c], tv * bt4);
      }
    if constexpr (!LEAD) {
      // the stores held back from the previous chunk, and the chunk-start
      // state, as h (Dk x Dv) in 4 x 16 blocks
      flush(sp, p, hd, h);
      if (hs_chunk) {
#pragma unroll
        for (int t = 0; t < DK / 16; ++t)
#pragma unroll
          for (int nt = 0; nt < NTW; ++nt) st_blk_row4<E>(hs_chunk, 16 * t + 4 * g, n0 + 16 * nt, DV, hacc[t][nt]);
      }
    }
    __syncthreads();
    clk.mark(2);
    sp = lds_opaque(sp);

    // ---- 3. the next chunk's k, v, scalar record (and q) start their way from HBM
    if (nrows > 0) {
      ld.load_kv(p, ntok0, nrows, h, nrec);
      if (OUT) ld.load_q(p, ntok0, nrows, h);
    }

    // ---- 4. -W = -T diag(beta Gam) K for row tile w % 4 (key column tiles split
    //         between w / 4 = 0, 1 with eight waves); Ut = T diag(beta) V for this
    //         wave's state columns.
    {
      constexpr int CTW = (DK / 16) / (NW / 4);
      const int rt = w & 3, ct0 = (w >> 2) * CTW;
      Frag<E> xw[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) xw[kb] = ld_frag(sp->TBG, LT, 16 * rt + c16, 32 * kb);
      // formed transposed (key rows), so each lane stores four consecutive
      // entries of a row of -W at once
#pragma unroll
      for (int cc = 0; cc < CTW; ++cc) {
        const int ct = ct0 + cc;
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) mma(acc, ld_fragC_q<E>(sp->K, S::LK, 32 * kb, 16 * ct), xw[kb]);
        st_tile_cm<E>(sp->W, LQ, 16 * ct, 16 * rt, -acc);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    sp = lds_opaque(sp);
    f32x4 u[4][NTW];
    {
      Frag<E> yv[NTW][2];
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) yv[nt][kb] = ld_fragC_q<E>(sp->V, S::LV, 32 * kb, n0 + 16 * nt);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        Frag<E> xb[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) xb[kb] = ld_frag(sp->TB, LT, 16 * rt + c16, 32 * kb);
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
          u[rt][nt] = zero4();
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) mma(u[rt][nt], xb[kb], yv[nt][kb]);
        }
      }
    }
    __syncthreads();
    clk.mark(3);
    sp = lds_opaque(sp);

    // ---- 5. state chain: U = Ut - W h ; O = scale (diag(Gam) Q h + P U) ; h' = Gam_C h + K^T (ek * U)
    Frag<E> hf[NTW][DK / 32];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
      for (int kb = 0; kb < DK / 32; ++kb) pack_frag(hf[nt][kb], hacc[2 * kb][nt], hacc[2 * kb + 1][nt]);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      Frag<E> xw[DK / 32];
#pragma unroll
      for (int kb = 0; kb < DK / 32; ++kb) xw[kb] = ld_frag(sp->W, LQ, 16 * rt + c16, 32 * kb);
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb) mma(u[rt][nt], xw[kb], hf[nt][kb]);
    }
    // U out (held for the next chunk; flush); the forward proper writes the
    // rounded operand fragments it forms anyway (bf16: and the residual of
    // that rounding, for the backward's decay gradient, whose row terms
    // u_r . (dS' k_r) can cancel far below their parts)
    constexpr bool ULO = USAVE && std::is_same<E, bf16>::value;
    if (USAVEC && !OUT) {
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) hd.u[rt][nt] = u[rt][nt];
      hd.us = us_chunk;
      hd.ulo = ulo_chunk;
    }
    if (OUTC) {
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        Frag<E> uf[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) pack_frag(uf[kb], u[2 * kb][nt], u[2 * kb + 1][nt]);
        if (USAVEC) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) st_fragC_q<E>(us_chunk + (n0 + 16 * nt) * CH, 16, 32 * kb, 0, uf[kb]);
          if constexpr (ULO) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
              Frag<E> lf;
              pack_frag(lf, bf16_residual(u[2 * kb][nt]), bf16_residual(u[2 * kb + 1][nt]));
              st_fragC_q<E>(ulo_chunk + (n0 + 16 * nt) * CH, 16, 32 * kb, 0, lf);
            }
          }
        }
        // O^T = scale (h^T Q^T diag(Gam) + U^T P^T): value rows, chunk-row
        // columns, so each lane stores four consecutive entries of a row of O
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          f32x4 o = zero4();
#pragma unroll
          for (int kb = 0; kb < DK / 32; ++kb) mma(o, hf[nt][kb], ld_frag(sp->Q, LQ, 16 * rt + c16, 32 * kb));
          o = o * sp->Gam[16 * rt + c16];
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) mma(o, uf[kb], ld_frag(sp->P, LT, 16 * rt + c16, 32 * kb));
          st_tile_cm<E>(sp->O, LO, n0 + 16 * nt, 16 * rt, o * p.scale);
        }
      }
    }
    {
      const float gc = sp->tail[1];
      f32x4 e0[2], e1[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        e0[kb] = *reinterpret_cast<const f32x4*>(&sp->ek[32 * kb + 4 * g]);
        e1[kb] = *reinterpret_cast<const f32x4*>(&sp->ek[32 * kb + 16 + 4 * g]);
      }
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        Frag<E> us[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) pack_frag_scaled(us[kb], u[2 * kb][nt], u[2 * kb + 1][nt], e0[kb], e1[kb]);
#pragma unroll
        for (int t = 0; t < DK / 16; ++t) {
          hacc[t][nt] = hacc[t][nt] * gc;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) mma(hacc[t][nt], ld_fragC_q<E>(sp->K, S::LK, 32 * kb, 16 * t), us[kb]);
        }
      }
    }
    __syncthreads();
    clk.mark(4);
    sp = lds_opaque(sp);

    // ---- 6. the output tile stays in LDS until the next chunk (flush)
    if constexpr (OUTC) {
      hd.otok0 = tok0;
      hd.orows = rows;
    }
    clk.mark(5);
  }

  // Issue the loads of chunk wb, the first of a run (before the state is
  // loaded, so that the two are in flight together).
  __device__ static void prime(Loader& ld, const FwdParams& p, int64_t seq0, int len, int64_t chunk0, int wb,
                               int ce, int h) {
    if (wb < ce) ld.load(p, seq0 + (int64_t)wb * CH, min(CH, len - wb * CH), h, p.rec + ((chunk0 + wb) * p.H + h) * RECF);
  }
  // Run chunks [wb, ce) of sequence (seq0, len) from the state in hacc: chunks
  // before cb are the lead-in (the state advances, nothing is written), chunks
  // from cb on write their outputs.  ld: primed for chunk wb.
  __device__ static void run(S& s, const FwdParams& p, int64_t seq0, int len, int64_t chunk0, int wb, int cb,
                             int ce, int h, f32x4 (&hacc)[DK / 16][NTW], Loader& ld, FwdClock& clk) {
    const size_t SS = (size_t)DK * DV;
    E* hs = static_cast<E*>(p.hs);
    Held hd;
    // the lead-in and the segment proper as two loops, each with its own
    // register allocation
    auto chunk = [&](auto lead, int c) {
      const int64_t tok0 = seq0 + (int64_t)c * CH;
      const int rows = min(CH, len - c * CH);
      const bool more = c + 1 < ce;
      const int nrows = more ? min(CH, len - (c + 1) * CH) : 0;
      const float* tin = p.t_in + ((chunk0 + c) * p.H + h) * (size_t)(CH * CH);
      const float* nrec = more ? p.rec + ((chunk0 + c + 1) * p.H + h) * RECF : nullptr;
      if constexpr (decltype(lead)::value) {
        step<true>(s, p, ld, tok0, rows, tok0 + CH, nrows, h, nullptr, tin, nrec, nullptr, nullptr, hacc, hd, clk);
      } else {
        E* hsc = hs ? hs + ((chunk0 + c) * p.H + h) * SS : nullptr;
        const size_t uoff = ((chunk0 + c) * p.H + h) * (size_t)(CH * DV);
        E* usc = USAVE ? static_cast<E*>(p.us) + uoff : nullptr;
        E* ulc = USAVE && p.ulo ? static_cast<E*>(p.ulo) + uoff : nullptr;
        step<false>(s, p, ld, tok0, rows, tok0 + CH, nrows, h, hsc, tin, nrec, usc, ulc, hacc, hd, clk);
      }
    };
    for (int c = wb; c < cb; ++c) chunk(std::true_type{}, c);
    for (int c = cb; c < ce; ++c) chunk(std::false_type{}, c);
    flush(lds_opaque(&s), p, hd, h);  // the last chunk's (after its final barrier)
    clk.set(7, ce - wb);
  }
};

// State h = S^T (fp32 [DK][DV]) <-> this wave's accumulator tiles (its DV/NW columns).
template <class E, int DK, int DV>
__device__ void load_state(f32x4 (&hacc)[DK / 16][DV / (16 * FwdWaves<DV>::NW)], const float* src) {
  constexpr int NW = FwdWaves<DV>::NW, NTW = DV / (16 * NW);
  const int l = lane_id(), w = wave_id(), g = l >> 4, c16 = l & 15;
#pragma unroll
  for (int t = 0; t < DK / 16; ++t)
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        hacc[t][nt][i] = src ? src[(16 * t + 4 * g + i) * DV + w * (DV / NW) + 16 * nt + c16] : 0.f;
}
template <class E, int DK, int DV>
__device__ void store_state(const f32x4 (&hacc)[DK / 16][DV / (16 * FwdWaves<DV>::NW)], float* dst) {
  constexpr int NW = FwdWaves<DV>::NW, NTW = DV / (16 * NW);
  const int l = lane_id(), w = wave_id(), g = l >> 4, c16 = l & 15;
#pragma unroll
  for (int t = 0; t < DK / 16; ++t)
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[(16 * t + 4 * g + i) * DV + w * (DV / NW) + 16 * nt + c16] = hacc[t][nt][i];
}

template <class E, int DK, int DV>
__device__ void init_smem(FwdSmem<E, DK, DV>& s) {
  using Sm = FwdSmem<E, DK, DV>;
  // The upper-triangular part of P is never written by the chunk loop and must
  // read as zero.
  for (int e = threadIdx.x; e < CH * CH; e += blockDim.x) {
    const int r = e >> 6, c = e & 63;
    s.P[r * Sm::LT + c] = to_e<E>(0.f);
  }
  __syncthreads();
}

// One workgroup per (segment, head).  A segment that does not start its
// sequence begins with a lead-in from a zero state over the chunks before it
// whose log-bounds sum to ln 2^-24 or less, so that its state at the segment
// start equals the exact one to fp32 rounding; if no such lead-in exists the
// run starts at the sequence start from h0 (exact, and serial for that
// segment).
template <class E, int DK, int DV, bool OUT, bool PREP, bool USAVE>
__global__ __launch_bounds__(64 * FwdWaves<DV>::NW) void gdn_fwd_seg(FwdParams p) {
  __shared__ FwdSmem<E, DK, DV> s;
  FwdClock clk;
  clk.start();
  const SegDesc sd = p.seq.seg_of(p.segs, blockIdx.x);
  if (sd.n < 0) return;  // the plan found the device cu_seqlens inconsistent
  const int h = blockIdx.y, n = sd.n;
  const int nseg = p.seq.nseg_of(p.seg_first, n);
  const int64_t seq0 = p.seq.start(n), chunk0 = p.seq.first_chunk(p.chunk_first, n);
  const int len = p.seq.len(n);
  const size_t SS = (size_t)DK * DV;
  const int wb = sd.c_begin > 0 ? lead_in_begin(p.rec, chunk0, p.H, h, sd.c_begin) : 0;
  f32x4 hacc[DK / 16][DV / (16 * FwdWaves<DV>::NW)];
  using C = Chunk<E, DK, DV, OUT, PREP, USAVE>;
  typename C::Loader ld;
  C::prime(ld, p, seq0, len, chunk0, wb, sd.c_end, h);
  init_smem(s);
  load_state<E, DK, DV>(hacc, (wb == 0 && p.h0) ? p.h0 + ((size_t)n * p.H + h) * SS : nullptr);
  clk.mark(0);
  C::run(s, p, seq0, len, chunk0, wb, sd.c_begin, sd.c_end, h, hacc, ld, clk);
  if (sd.s == nseg - 1 && p.hT) store_state<E, DK, DV>(hacc, p.hT + ((size_t)n * p.H + h) * SS);
  if constexpr (kPhaseClock) {
    clk.mark(6);
    const int blk = blockIdx.x + blockIdx.y * gridDim.x;
    if (blk < CLOCK_BLOCKS) clk.flush(gdn_clock_fwd[OUT ? 0 : 1][blk]);
  }
}

template <class E, int DK, int DV>
hipError_t launch_fwd_t(const FwdParams& p, int nseg_total, hipStream_t st) {
  dim3 grid(nseg_total, p.H), block(64 * FwdWaves<DV>::NW);
  const bool out = p.o != nullptr;
  const bool prep = p.prep.qk_norm || p.prep.gate_act;
  // T and the scalar records are solved beforehand; the replay always writes
  // U, the forward proper on request
  if (!p.t_in || !p.rec) return hipErrorInvalidValue;
  if (!out && !p.us) return hipErrorInvalidValue;
  const bool us = p.us != nullptr;
  // in bf16, U's rounding residual is stored with U
  if (std::is_same<E, bf16>::value && us && !p.ulo) return hipErrorInvalidValue;
  if (prep) {
    if (out && us) hipLaunchKernelGGL((gdn_fwd_seg<E, DK, DV, true, true, true>), grid, block, 0, st, p);
    else if (out) hipLaunchKernelGGL((gdn_fwd_seg<E, DK, DV, true, true, false>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((gdn_fwd_seg<E, DK, DV, false, true, true>), grid, block, 0, st, p);
  } else {
    if (out && us) hipLaunchKernelGGL((gdn_fwd_seg<E, DK, DV, true, false, true>), grid, block, 0, st, p);
    else if (out) hipLaunchKernelGGL((gdn_fwd_seg<E, DK, DV, true, false, false>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((gdn_fwd_seg<E, DK, DV, false, false, true>), grid, block, 0, st, p);
  }
  return hipGetLastError();
}

hipError_t launch_fwd(int dtype, int DK, int DV, const FwdParams& p, int nseg_total, hipStream_t st) {
  if (dtype == 1) {
    if (DK == 128 && DV == 128) return launch_fwd_t<bf16, 128, 128>(p, nseg_total, st);
    if (DK == 64 && DV == 64) return launch_fwd_t<bf16, 64, 64>(p, nseg_total, st);
    if (DK == 64 && DV == 128) return launch_fwd_t<bf16, 64, 128>(p, nseg_total, st);
    if (DK == 128 && DV == 64) return launch_fwd_t<bf16, 128, 64>(p, nseg_total, st);
  } else {
    if (DK == 64 && DV == 64) return launch_fwd_t<float, 64, 64>(p, nseg_total, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn

#ifdef GDN_PHASE_CLOCK
// The forward's and the replay's phase clocks ([2][CLOCK_BLOCKS][8 waves][8
// phases] uint32 cycles) to host memory; an instrumented build only.
extern "C" int gdn_clock_read_fwd(uint32_t* host) {
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(gdn::gdn_clock_fwd), sizeof(gdn::gdn_clock_fwd));
}
#endif
