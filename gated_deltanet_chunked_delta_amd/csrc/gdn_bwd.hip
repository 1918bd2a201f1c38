// gdn_bwd.hip -- backward pass of the chunked gated delta rule on gfx950.
//
// The backward ("FlashQLA resource", sections 3 and 5: fused backward kernels
// with intra-card sequence parallelism) runs in three stages after the forward
// replay (gdn_fwd.hip in replay mode stores the state h_c at every chunk start):
//
//  1. Reverse chain (this file, gdn_rev_seg): per (segment, head), from the
//     last chunk to the first, the gradient dh' at each chunk END is stored and
//     carried back through the chunk:
//        dU = scale P^T dO + diag(ek) K dh'
//        dh = scale (diag(Gam) Q)^T dO + Gam_C dh' - W^T dU
//     The dh' chain lives in accumulator registers (wave w owns 16 columns).
//     Long sequences are cut into segments exactly as in the forward; a
//     segment that does not end its sequence starts from dh' = 0 some chunks
//     after its end (the lead-in, until the chunks' log-bounds sum to
//     ln 2^-24 or less -- the transpose of the forward transition has the same
//     norm bound), else from the sequence end and dhT.
//
//  2. Chunk gradients (gdn_grad_kernel): every chunk independently, given h_c
//     and dh'_c, evaluates the reverse-mode derivative of the chunk algebra
//     (with D_ri = exp(gam_r - gam_i), M = D * [i <= r], ek = exp(gam_last - gam)):
//        GP = scale (dO U^T) * [i <= r]
//        GW = -dU h^T,  XW = T^T GW,  XU = T^T dU
//        GT = dU (diag(beta) V)^T + GW (diag(beta Gam) K)^T
//        GA = strict_lower(-T^T GT T^T),  E = diag(beta) (GA * D)
//        dQ = scale diag(Gam) dO h^T + (GP*M) K
//        dK = (GP*M)^T Q + diag(ek) U dh'^T + diag(beta Gam) XW + (E + E^T) K
//        dV = diag(beta) XU
//        dbeta_r = XU_r.v_r + Gam_r XW_r.k_r + sum_i GA_ri D_ri (k_r.k_i)
//        dgam_r  = scale Gam_r q_r.(dO h^T)_r + beta_r Gam_r XW_r.k_r
//                  + rowsum_r(GP*P) - colsum_r(GP*P) + rowsum_r(GA*A) - colsum_r(GA*A)
//                  - ek_r k_r.(U dh'^T)_r
//                  + [r = last] (Gam_C <h, dh'> + sum_i ek_i k_i.(U dh'^T)_i)
//        dg = reverse cumulative sum of dgam within the chunk.
//     A short final chunk is handled as a 64-row chunk whose extra rows have
//     zero beta and g (and, in the chunk-gradient kernel, zero q, k, v, dO);
//     the reverse chain loads copies of the last real row there and masks the
//     two terms that would see them, which leaves every real gradient unchanged.
#include <type_traits>

#include <cstddef>

#include "gdn_device.h"
#include "gdn_internal.h"
#include "gdn_tiles.h"

namespace gdn {

// ======================================================================== reverse chain

// Every staged tile is row-major.  Products that need the columns of K, of
// diag(scale Gam) Q or of dO read them with LDS transpose loads, from copies
// whose bf16 rows are padded by 16 elements (conflict-free for transpose
// loads); tiles read along their rows are padded by 4 (where 8-byte row reads
// run at full rate).
template <class E, int DK, int DV>
struct alignas(16) RevSmem {
  static constexpr int LQ = ldpad<E>(DK);
  static constexpr int LT = ldpad<E>(CH);
  static constexpr int PADC = sizeof(E) == 2 ? 16 : 4;
  static constexpr int LKC = DK + PADC, LDO = DV + PADC;
  E Q[CH * LQ];    // row-major, X of Q K^T
  E K[CH * LQ];    // row-major, X/Y of K K^T, X of K dh'
  E KC[CH * LKC];  // K again, read down its columns (X of W^T)
  E QS[CH * LKC];  // diag(scale Gam) Q (zero past the sequence end), read down its columns (X of (Gam Q)^T dO)
  E DO[CH * LDO];  // dO, read down its columns (Y of P^T dO and (Gam Q)^T dO)
  E WT[DK * LT];   // -W^T
  E PT[CH * LT];   // scale * P^T
  E TBG[CH * LT];  // T diag(beta Gam), Y of W^T
  // the chunk's scalar record, as laid out in memory (tail: Lambda_c, Gam_C)
  alignas(16) float gam[CH], Gam[CH], ek[CH], beta[CH], bg[CH], tail[4];
};

// Phases of the reverse chain's phase clock: 0 before the first chunk; per
// chunk 1 staging, 2 scale P^T and -W^T, 3 dU and the state-gradient update;
// 4 after the last chunk; slot 7 counts the chunks run.
using RevClock = PhaseClock<8>;
// [workgroup][wave][phase] (an instrumented build only)
__device__ uint32_t gdn_clock_rev[kPhaseClock ? CLOCK_BLOCKS : 1][8 * 8];

// Waves per workgroup of the reverse chain: 8 when the state gradient has 128
// value columns (one 16-column tile per wave, two waves per SIMD), else 4.
template <int DV>
struct RevWaves { static constexpr int NW = DV == 128 ? 8 : 4; };

// One chunk of the reverse chain (wave w owns Dv/NW columns of the state
// gradient).  Every chunk's T and scalar record are read from p.t_in / p.rec
// (written by the chunk-parallel T solve beforehand).
template <class E, int DK, int DV, bool PREP>
struct RevChunk {
  static constexpr int NW = RevWaves<DV>::NW, NT = 64 * NW, NTW = DV / (16 * NW);
  using S = RevSmem<E, DK, DV>;
  // The next chunk's tiles, in flight in registers during the current chunk:
  // the first half of the threads holds K and the second half Q (one register
  // set, kq), and dO sits on the first NT / 2 * (DV / DK) threads.
  static constexpr int KQT = NT / 2;  // threads per K (or Q) tile
  struct Loader {
    TilePart<E, KQT, DK> kq;
    TilePart<E, NT, DV> d;
    RecordPart rec;
    // this thread's pieces of T (its bf16 value plane for bf16 inputs) and
    // beta Gam of their 8 columns (the same columns for every piece)
    TPart<E, NT> t;
    f32x4 tbg[2];
    // Gam of the rows of each kq block (Q half), as loaded: the scaling waits
    // for the staging, so that nothing waits for these loads meanwhile
    f32x4 sc[TilePart<E, KQT, DK>::NB > 0 ? TilePart<E, KQT, DK>::NB : 1];
  };
  __device__ __forceinline__ static bool q_half() { return threadIdx.x >= KQT; }
  __device__ __forceinline__ static int kq_tid() { return threadIdx.x & (KQT - 1); }

  __device__ static void issue(Loader& ld, const RevParams& p, int64_t tok0, int rows, int h, const float* rec,
                              const float* t) {
    const int H = p.H;
    const void* src = q_half() ? p.q : p.k;
    // every load of the prefetch is non-temporal: the chain ran shorter so
    // (the forward chain did not)
    ld.kq.template load<false, true>(static_cast<const E*>(src) + (tok0 * H + h) * DK, (int64_t)H * DK, rows,
                                     kq_tid());
    ld.d.template load<false, true>(static_cast<const E*>(p.dout) + (tok0 * H + h) * DV, (int64_t)H * DV, rows);
    ld.rec.load(rec);
    ld.t.template load<true>(t);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      ld.tbg[j] = *reinterpret_cast<const f32x4*>(rec + 4 * CH + (8 * threadIdx.x) % CH + 4 * j);
    constexpr int NBK = TilePart<E, KQT, DK>::NB;
#pragma unroll
    for (int b = 0; b < NBK; ++b) {
      const int r0 = TilePart<E, KQT, DK>::block_row(b, kq_tid());
      if (q_half() && r0 >= 0) ld.sc[b] = *reinterpret_cast<const f32x4*>(rec + CH + r0);  // Gam
    }
  }

  // One lower 16x16 tile (rt, ct) of scale P^T, P = (Q K^T) * M, with the rows
  // past the sequence end masked.
  __device__ __forceinline__ static void pt_tile(S* sp, const RevParams& p, int rt, int ct, int g, int c16,
                                                 int rows) {
    constexpr int LQ = S::LQ, LT = S::LT;
    f32x4 acc = zero4();
#pragma unroll
    for (int kb = 0; kb < DK / 32; ++kb)
      mma(acc, ld_frag(sp->Q, LQ, 16 * rt + c16, 32 * kb), ld_frag(sp->K, LQ, 16 * ct + c16, 32 * kb));
    const f32x4 gr4 = *reinterpret_cast<const f32x4*>(&sp->gam[16 * rt + 4 * g]);
    const int c = 16 * ct + c16;
    const float gc = sp->gam[c];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * rt + 4 * g + i;
      acc[i] = (c <= r && r < rows) ? p.scale * acc[i] * __expf(gr4[i] - gc) : 0.f;
    }
    st_tile_cm<E>(sp->PT, LT, 16 * rt, 16 * ct, acc);
  }

  // dh: gradient at the chunk end on entry, at the chunk start on exit.
  // Prefetches chunk (ntok0, nrows) into ld (nrows = 0: none).
  // nt_in, nrec: the next chunk's T and scalar record.  LEAD: a
  // lead-in chunk after the segment proper, which only advances the gradient
  // (nothing is written).
  //
  // Besides, for the decay gradient, the row terms e_r = ek_r u_r . (dS' k_r)
  // (dS' = this chunk's end gradient, u_r = row r of its U) summed over this
  // wave's value columns go to ep_chunk[w][r].  Their sum over r can be far
  // smaller than its parts (strong decay leaves little else in dg), so both
  // factors are carried to about 16 bits: dS' as its bf16 value plus the bf16
  // residual (two products with K), U as the stored bf16 value plus its stored
  // residual (us_chunk, ulo_chunk).
  template <bool LEAD>
  __device__ static void step(S& s0, const RevParams& p, Loader& ld, int rows, int64_t ntok0, int nrows, int h,
                              E* dhs_chunk, const float* nt_in, const float* nrec, const E* us_chunk,
                              const E* ulo_chunk, float* ep_chunk, f32x4 (&dh)[DK / 16][NTW], RevClock& clk) {
    constexpr int LQ = S::LQ, LT = S::LT;
    constexpr bool LO = std::is_same<E, bf16>::value;  // U and dS' need their residuals
    const int tid = threadIdx.x, l = lane_id(), w = wave_id(), g = l >> 4, c16 = l & 15;
    const int n0 = w * (DV / NW);
    // this wave's columns of U (and its residual) for the row terms, read now
    // and used in phase 5
    CPiece<E> uhp[4][NTW], ulp[4][NTW];
    if constexpr (!LEAD) {
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
          uhp[rt][nt].template load<true>(us_chunk + (n0 + 16 * nt) * CH, 16 * rt);
          if constexpr (LO) ulp[rt][nt].template load<true>(ulo_chunk + (n0 + 16 * nt) * CH, 16 * rt);
        }
    }

    // ---- 1. gradient at the chunk end out; tiles into LDS; scalars
    S* sp = lds_opaque(&s0);
    // stored as dh' (Dk x Dv) in 4 x 16 blocks
    if constexpr (!LEAD) {
#pragma unroll
      for (int t = 0; t < DK / 16; ++t)
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) st_blk_row4<E>(dhs_chunk, 16 * t + 4 * g, n0 + 16 * nt, DV, dh[t][nt]);
    }
    S& s1 = *sp;
    if (PREP && p.prep.qk_norm) ld.kq.normalize_rows(kq_tid());
    if (q_half()) {
      // the second Q copy's row scales: scale Gam, zero past the sequence end
      constexpr int NBK = TilePart<E, KQT, DK>::NB;
      f32x4 sc[NBK > 0 ? NBK : 1];
#pragma unroll
      for (int b = 0; b < NBK; ++b) {
        const int r0 = TilePart<E, KQT, DK>::block_row(b, kq_tid());
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[b][i] = r0 + i < rows ? p.scale * ld.sc[b][i] : 0.f;
      }
      ld.kq.template store_rows2<true>(s1.Q, LQ, s1.QS, S::LKC, sc, kq_tid());
    } else {
      ld.kq.template store_rows2<false>(s1.K, LQ, s1.KC, S::LKC, ld.sc, kq_tid());
    }
    ld.d.store_rows16(s1.DO, S::LDO);
    // T lands as T diag(beta Gam) (scaled in fp32, rounded once)
#pragma unroll
    for (int i = 0; i < TPart<E, NT>::NP; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int e = 8 * (tid + i * NT) + 4 * j, r = e / CH, c = e % CH;
        st4f<E>(&s1.TBG[r * LT + c], ld.t.get(i, j) * ld.tbg[j]);
      }
    static_assert(offsetof(S, tail) == offsetof(S, gam) + 5 * CH * sizeof(float), "record layout");
    ld.rec.store(s1.gam);
    __syncthreads();
    clk.mark(1);

    // ---- 2. the next chunk's tiles, T and record start their way from HBM
    if (nrows > 0) issue(ld, p, ntok0, nrows, h, nrec, nt_in);

    // ---- 3. Q K^T -> scale P^T: the ten lower 16x16 tiles, tile j on wave j % NW
    //         (at most two tiles a wave with eight waves)
    {
      S* sq = lds_opaque(&s0);
#pragma unroll
      for (int j = 0; j < (10 + NW - 1) / NW; ++j) {
        const int pid = w + NW * j;
        const int rt = pid < 1 ? 0 : (pid < 3 ? 1 : (pid < 6 ? 2 : 3));
        const int ct = pid - (rt * (rt + 1)) / 2;
        if (pid < 10) pt_tile(sq, p, rt, ct, g, c16, rows);
      }
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- 4. -W^T = -K^T diag(beta Gam) T^T: (Dk/16) x 4 tiles, KTW key tiles x
    //         RTW chunk-row tiles per wave
    {
      S& s = *lds_opaque(&s0);
      constexpr int NKT = DK / 16;
      constexpr int KTW = NKT >= NW ? NKT / NW : 1;
      constexpr int RTW = NKT >= NW ? 4 : 4 * NKT / NW;
      const int kt0 = (w % (NKT / KTW)) * KTW, rt0 = (w / (NKT / KTW)) * RTW;
      Frag<E> yt[RTW][2];
#pragma unroll
      for (int rr = 0; rr < RTW; ++rr)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) yt[rr][kb] = ld_frag(s.TBG, LT, 16 * (rt0 + rr) + c16, 32 * kb);
#pragma unroll
      for (int dd = 0; dd < KTW; ++dd) {
        const int dt = kt0 + dd;
        Frag<E> xk[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) xk[kb] = ld_fragC_q<E>(s.KC, S::LKC, 32 * kb, 16 * dt);
        // W itself (chunk rows, key columns), stored transposed: each lane
        // writes four consecutive entries of a row of -W^T at once
#pragma unroll
        for (int rr = 0; rr < RTW; ++rr) {
          f32x4 acc = zero4();
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) mma(acc, yt[rr][kb], xk[kb]);
          st_tile_cm<E>(s.WT, LT, 16 * (rt0 + rr), 16 * dt, -acc);
        }
      }
    }
    __syncthreads();
    clk.mark(2);

    // ---- 5. dU = diag(ek) K dh' + scale P^T dO ;  dh = Gam_C dh' + scale (Gam Q)^T dO - W^T dU
    f32x4 du[4][NTW];
    {
      S& s = *lds_opaque(&s0);
      Frag<E> hf[NTW][DK / 32], hflo[NTW][DK / 32];
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb) {
          pack_frag(hf[nt][kb], dh[2 * kb][nt], dh[2 * kb + 1][nt]);
          if constexpr (LO && !LEAD) pack_frag(hflo[nt][kb], bf16_residual(dh[2 * kb][nt]), bf16_residual(dh[2 * kb + 1][nt]));
        }
      Frag<E> yd[NTW][2];
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) yd[nt][kb] = ld_fragC_q<E>(s.DO, S::LDO, 32 * kb, n0 + 16 * nt);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        Frag<E> xk[DK / 32];
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb) xk[kb] = ld_frag(s.K, LQ, 16 * rt + c16, 32 * kb);
        const f32x4 e4 = *reinterpret_cast<const f32x4*>(&s.ek[16 * rt + 4 * g]);
        Frag<E> xp[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) xp[kb] = ld_frag(s.PT, LT, 16 * rt + c16, 32 * kb);
        f32x4 er = zero4();  // row terms of this lane's rows, over its columns
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
          f32x4 acc = zero4();
#pragma unroll
          for (int kb = 0; kb < DK / 32; ++kb) mma(acc, xk[kb], hf[nt][kb]);
          if constexpr (!LEAD) {
            f32x4 z = acc;  // K dS'^T: this lane's rows, column n0 + 16 nt + c16
            f32x4 u = uhp[rt][nt].get();
            if constexpr (LO) {
              f32x4 zl = zero4();
#pragma unroll
              for (int kb = 0; kb < DK / 32; ++kb) mma(zl, xk[kb], hflo[nt][kb]);
              z = z + zl;
              u = u + ulp[rt][nt].get();
            }
            er = er + u * z;
          }
          acc = acc * e4;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) mma(acc, xp[kb], yd[nt][kb]);
          du[rt][nt] = acc;
        }
        if constexpr (!LEAD) {
          er = er * e4;
#pragma unroll
          for (int i = 0; i < 4; ++i) er[i] = row16_sum(er[i]);
          if (c16 == 0) st_out(reinterpret_cast<f32x4*>(ep_chunk + w * CH + 16 * rt + 4 * g), er);
        }
      }
      const float gc = s.tail[1];
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        Frag<E> uf[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) pack_frag(uf[kb], du[2 * kb][nt], du[2 * kb + 1][nt]);
#pragma unroll
        for (int t = 0; t < DK / 16; ++t) {
          dh[t][nt] = dh[t][nt] * gc;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
            mma(dh[t][nt], ld_fragC_q<E>(s.QS, S::LKC, 32 * kb, 16 * t), yd[nt][kb]);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) mma(dh[t][nt], ld_frag(s.WT, LT, 16 * t + c16, 32 * kb), uf[kb]);
        }
      }
    }
    __syncthreads();
    clk.mark(3);
  }

  // Issue the loads of chunk we - 1, the first of a run (before the state
  // gradient is loaded, so that the two are in flight together).
  __device__ static void prime(Loader& ld, const RevParams& p, int64_t seq0, int len, int64_t chunk0, int cb, int we,
                               int h) {
    const int c = we - 1;
    if (c >= cb)
      issue(ld, p, seq0 + (int64_t)c * CH, min(CH, len - c * CH), h, p.rec + ((chunk0 + c) * p.H + h) * RECF,
            p.t_in + ((chunk0 + c) * p.H + h) * (size_t)(CH * CH));
  }
  // Chunks we-1 down to cb from the gradient in dh: chunks at or after ce are
  // the lead-in (the gradient advances, nothing is written), chunks below ce
  // write their chunk-end gradients.  ld: primed for chunk we - 1.
  __device__ static void run(S& s, const RevParams& p, int64_t seq0, int len, int64_t chunk0, int cb, int ce, int we,
                             int h, f32x4 (&dh)[DK / 16][DV / (16 * RevWaves<DV>::NW)], Loader& ld, RevClock& clk) {
    const size_t SS = (size_t)DK * DV;
    constexpr bool LOU = std::is_same<E, bf16>::value;
    E* dhs = static_cast<E*>(p.dhs);
    // the lead-in and the segment proper as two loops, each with its own
    // register allocation
    auto chunk = [&](auto lead, int c) {
      const int rows = min(CH, len - c * CH);
      const bool more = c - 1 >= cb;
      const int64_t ntok0 = seq0 + (int64_t)(c - 1) * CH;
      const int nrows = more ? min(CH, len - (c - 1) * CH) : 0;
      const float* ntin = more ? p.t_in + ((chunk0 + c - 1) * p.H + h) * (size_t)(CH * CH) : nullptr;
      const float* nrec = more ? p.rec + ((chunk0 + c - 1) * p.H + h) * RECF : nullptr;
      if constexpr (decltype(lead)::value) {
        step<true>(s, p, ld, rows, ntok0, nrows, h, nullptr, ntin, nrec, nullptr, nullptr, nullptr, dh, clk);
      } else {
        const size_t ci = (chunk0 + c) * p.H + h;
        const E* usc = static_cast<const E*>(p.us) + ci * (CH * DV);
        const E* ulc = LOU ? static_cast<const E*>(p.ulo) + ci * (CH * DV) : nullptr;
        step<false>(s, p, ld, rows, ntok0, nrows, h, dhs + ci * SS, ntin, nrec, usc, ulc, p.ep + ci * (EPW * CH), dh,
                    clk);
      }
    };
    for (int c = we - 1; c >= ce; --c) chunk(std::true_type{}, c);
    for (int c = ce - 1; c >= cb; --c) chunk(std::false_type{}, c);
    clk.set(7, we - cb);
  }
};

template <class E, int DK, int DV>
__device__ void rev_load(f32x4 (&acc)[DK / 16][DV / (16 * RevWaves<DV>::NW)], const float* src) {
  constexpr int NW = RevWaves<DV>::NW, NTW = DV / (16 * NW);
  const int l = lane_id(), w = wave_id(), g = l >> 4, c16 = l & 15;
#pragma unroll
  for (int t = 0; t < DK / 16; ++t)
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[t][nt][i] = src ? src[(16 * t + 4 * g + i) * DV + w * (DV / NW) + 16 * nt + c16] : 0.f;
}
template <class E, int DK, int DV>
__device__ void rev_store(const f32x4 (&acc)[DK / 16][DV / (16 * RevWaves<DV>::NW)], float* dst) {
  constexpr int NW = RevWaves<DV>::NW, NTW = DV / (16 * NW);
  const int l = lane_id(), w = wave_id(), g = l >> 4, c16 = l & 15;
#pragma unroll
  for (int t = 0; t < DK / 16; ++t)
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = (16 * t + 4 * g + i) * DV + w * (DV / NW) + 16 * nt + c16;
        dst[e] = acc[t][nt][i];
      }
}

template <class E, int DK, int DV>
__device__ void rev_init_smem(RevSmem<E, DK, DV>& s) {
  using Sm = RevSmem<E, DK, DV>;
  // the tiles of P^T above the diagonal are never written
  for (int e = threadIdx.x; e < CH * CH; e += blockDim.x) s.PT[(e >> 6) * Sm::LT + (e & 63)] = to_e<E>(0.f);
  __syncthreads();
}

// One segment of the reverse chain.  A segment that ends before its sequence
// does starts from dh' = 0 a few chunks later (the lead-in, until the chunks'
// log-bounds sum to ln 2^-24 or less; else from the sequence end and dhT), so
// every segment runs independently of the others.
template <class E, int DK, int DV, bool PREP>
__global__ __launch_bounds__(64 * RevWaves<DV>::NW) void gdn_rev_seg(RevParams p) {
  __shared__ RevSmem<E, DK, DV> s;
  RevClock clk;
  clk.start();
  const SegDesc sd = p.seq.seg_of(p.segs, blockIdx.x);
  if (sd.n < 0) return;  // the plan found the device cu_seqlens inconsistent
  const int h = blockIdx.y, n = sd.n;
  const int64_t seq0 = p.seq.start(n), chunk0 = p.seq.first_chunk(p.chunk_first, n);
  const int len = p.seq.len(n), nch = (len + CH - 1) / CH;
  const size_t SS = (size_t)DK * DV;
  const int we = sd.c_end < nch ? lead_in_end(p.rec, chunk0, p.H, h, sd.c_end, nch) : nch;
  f32x4 dh[DK / 16][DV / (16 * RevWaves<DV>::NW)];
  using C = RevChunk<E, DK, DV, PREP>;
  typename C::Loader ld;
  C::prime(ld, p, seq0, len, chunk0, sd.c_begin, we, h);
  rev_init_smem(s);
  rev_load<E, DK, DV>(dh, (we == nch && p.dhT) ? p.dhT + ((size_t)n * p.H + h) * SS : nullptr);
  clk.mark(0);
  C::run(s, p, seq0, len, chunk0, sd.c_begin, sd.c_end, we, h, dh, ld, clk);
  if (sd.c_begin == 0 && p.dh0) rev_store<E, DK, DV>(dh, p.dh0 + ((size_t)n * p.H + h) * SS);
  if constexpr (kPhaseClock) {
    clk.mark(4);
    const int blk = blockIdx.x + blockIdx.y * gridDim.x;
    if (blk < CLOCK_BLOCKS) clk.flush(gdn_clock_rev[blk]);
  }
}

template <class E, int DK, int DV>
hipError_t launch_rev_t(const RevParams& p, int nseg_total, hipStream_t st) {
  const dim3 block(64 * RevWaves<DV>::NW);
  const dim3 grid(nseg_total, p.H);
  // T and the scalar records are solved beforehand; U (with its bf16 residual)
  // is stored by the forward or its replay
  if (!p.t_in || !p.rec || !p.us || !p.ep) return hipErrorInvalidValue;
  if (std::is_same<E, bf16>::value && !p.ulo) return hipErrorInvalidValue;
  if (p.prep.qk_norm || p.prep.gate_act) hipLaunchKernelGGL((gdn_rev_seg<E, DK, DV, true>), grid, block, 0, st, p);
  else hipLaunchKernelGGL((gdn_rev_seg<E, DK, DV, false>), grid, block, 0, st, p);
  return hipGetLastError();
}

hipError_t launch_rev(int dtype, int DK, int DV, const RevParams& p, int nseg_total, hipStream_t st) {
  if (dtype == 1) {
    if (DK == 128 && DV == 128) return launch_rev_t<bf16, 128, 128>(p, nseg_total, st);
    if (DK == 64 && DV == 64) return launch_rev_t<bf16, 64, 64>(p, nseg_total, st);
    if (DK == 64 && DV == 128) return launch_rev_t<bf16, 64, 128>(p, nseg_total, st);
    if (DK == 128 && DV == 64) return launch_rev_t<bf16, 128, 64>(p, nseg_total, st);
  } else {
    if (DK == 64 && DV == 64) return launch_rev_t<float, 64, 64>(p, nseg_total, st);
  }
  return hipErrorInvalidValue;
}

// ======================================================================== chunk gradients

template <class E, int DK, int DV>
struct GradLayout {
  static constexpr int PADE = 16 / (int)sizeof(E);
  static constexpr int LK = DK + PADE;  // row-major [64][DK] E
  static constexpr int LV = DV + PADE;  // row-major [64][DV] E
  static constexpr int LT = CH + 4;     // transposed [D][64] E: an accumulator tile's columns as rows
  static constexpr int LA = CH + 4;     // fp32 [64][64]
  static constexpr int cmax(int a, int b) { return a > b ? a : b; }
  static constexpr int SLOT = cmax(cmax(CH * LK * (int)sizeof(E), CH * LV * (int)sizeof(E)),
                                   cmax(cmax(DK, DV) * LT * (int)sizeof(E), CH * LA * 4));
  static constexpr int NSLOT = 9;
};

template <class E, int DK, int DV>
struct alignas(16) GradSmem {
  using L = GradLayout<E, DK, DV>;
  alignas(16) char slot[L::NSLOT][L::SLOT];
  // the chunk's scalar record, as laid out in memory (tail: Lambda_c, Gam_C)
  alignas(16) float gam[CH], Gam[CH], ek[CH], beta[CH], bg[CH], tail[4];
  float pg[4][CH], pb[4][CH];  // row sums of the per-wave dgam / dbeta terms, by column group
  float p7[4][CH], c7[4][CH];  // row sums of GP*P by column tile, column sums by row tile
  float c9[2][CH];             // column sums of T * (dU V^T) by row half
  float c10[2][CH];            // column sums of GA*A by row half
  float ph[8];
};

// slot roles (each slot holds one tile at a time; the kernel's phases hand
// them on: Q -> GW^T -> dV, U -> GT^T, dO -> dQ, KD -> dK, scale P^T -> Z^T,
// dU^T -> E^T; slot GP holds (GP * M)^T)
enum { SK = 0, SGP = 1, SQ = 2, SV = 3, SDO = 4, ST = 5, SKD = 6, SP = 7, SDU = 8 };

// A 64 x 64 fp32 matrix in one LDS slot, kept for near-fp32 products (PFrag).
// E = float stores it as is (row stride LA).  E = bf16 stores its bf16 hi and
// lo parts (x = hi + lo, lo the rounded residual) as two planes of row stride
// LP: each value is split once, when written, and fragments load ready to
// multiply.  row(): k-slots along row r; col(): k-slots down column c0 + lane%16;
// cpiece(): the accumulator-tile piece at (r0, c0), as fp32.
template <class E> struct PMat;
template <> struct PMat<float> {
  static constexpr int LA = CH + 4;
  float* m;
  __device__ __forceinline__ explicit PMat(void* slot) : m(static_cast<float*>(slot)) {}
  __device__ __forceinline__ void put4(int r, int c0, const f32x4& x) const {
    *reinterpret_cast<f32x4*>(&m[r * LA + c0]) = x;
  }
  __device__ __forceinline__ PFrag<float> row(int r, int k0) const { return PFrag<float>(ld_frag(m, LA, r, k0)); }
  __device__ __forceinline__ PFrag<float> col(int k0, int c0) const {
    return PFrag<float>(ld_fragT<float>(m, LA, c0 + (lane_id() & 15), k0, 1.f));
  }
  __device__ __forceinline__ Frag<float> col_e(int k0, int c0) const {
    return ld_fragT<float>(m, LA, c0 + (lane_id() & 15), k0, 1.f);
  }
  __device__ __forceinline__ f32x4 cpiece(int r0, int c0) const { return ld_cpiece<float>(m, LA, r0, c0); }
};
template <> struct PMat<bf16> {
  static constexpr int LP = CH + 4;  // bf16 elements per row: 8-byte aligned rows
  bf16* hi;
  bf16* lo;
  typedef bf16 b4_t __attribute__((__vector_size__(8)));
  __device__ __forceinline__ explicit PMat(void* slot)
      : hi(static_cast<bf16*>(slot)), lo(static_cast<bf16*>(slot) + CH * LP) {}
  __device__ __forceinline__ void put4(int r, int c0, const f32x4& x) const {
    b4_t h, l;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h[i] = (bf16)x[i];
      l[i] = (bf16)(x[i] - (float)h[i]);
    }
    *reinterpret_cast<b4_t*>(&hi[r * LP + c0]) = h;
    *reinterpret_cast<b4_t*>(&lo[r * LP + c0]) = l;
  }
  __device__ __forceinline__ PFrag<bf16> row(int r, int k0) const {
    PFrag<bf16> f;
    f.hi = ld_frag(hi, LP, r, k0);
    f.lo = ld_frag(lo, LP, r, k0);
    return f;
  }
  __device__ __forceinline__ PFrag<bf16> col(int k0, int c0) const {
    PFrag<bf16> f;
    f.hi = ld_fragC_q<bf16>(hi, LP, k0, c0);
    f.lo = ld_fragC_q<bf16>(lo, LP, k0, c0);
    return f;
  }
  __device__ __forceinline__ Frag<bf16> col_e(int k0, int c0) const { return ld_fragC_q<bf16>(hi, LP, k0, c0); }
  __device__ __forceinline__ f32x4 cpiece(int r0, int c0) const {
    return ld_cpiece<bf16>(hi, LP, r0, c0) + ld_cpiece<bf16>(lo, LP, r0, c0);
  }
  // 8 consecutive elements of row r from c0, already split into their parts
  __device__ __forceinline__ void put8(int r, int c0, const bf16x8& h, const bf16x8& l) const {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      *reinterpret_cast<b4_t*>(&hi[r * LP + c0 + 4 * j]) = b4_t{h[4 * j], h[4 * j + 1], h[4 * j + 2], h[4 * j + 3]};
      *reinterpret_cast<b4_t*>(&lo[r * LP + c0 + 4 * j]) = b4_t{l[4 * j], l[4 * j + 1], l[4 * j + 2], l[4 * j + 3]};
    }
  }
};

// One thread's share of a chunk's T on its way from global memory (as the T
// solve stores it) into a PMat: fp32 pieces, or for bf16 inputs the stored
// value and residual planes, which are already the PMat's two parts.  The
// bf16 planes are read with non-temporal loads (measured slightly shorter).
template <class E, int NT> struct TStage;
template <int NT> struct TStage<float, NT> {
  static constexpr int NP = CH * CH / (4 * NT);
  f32x4 v[NP];
  __device__ __forceinline__ void load(const float* t, int tid) {
#pragma unroll
    for (int i = 0; i < NP; ++i) v[i] = *reinterpret_cast<const f32x4*>(t + 4 * (tid + i * NT));
  }
  __device__ __forceinline__ void put(const PMat<float>& m, int tid) const {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int e = 4 * (tid + i * NT);
      m.put4(e / CH, e % CH, v[i]);
    }
  }
};
template <int NT> struct TStage<bf16, NT> {
  static constexpr int NP = CH * CH / (8 * NT);
  static_assert(NP * 8 * NT == CH * CH, "whole pieces of T per thread");
  bf16x8 h[NP], l[NP];
  __device__ __forceinline__ void load(const float* t, int tid) {
    const bf16* b = reinterpret_cast<const bf16*>(t);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      h[i] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(b + 8 * (tid + i * NT)));
      l[i] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(b + CH * CH + 8 * (tid + i * NT)));
    }
  }
  __device__ __forceinline__ void put(const PMat<bf16>& m, int tid) const {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int e = 8 * (tid + i * NT);
      m.put8(e / CH, e % CH, h[i], l[i]);
    }
  }
};

// Requests into L2 the inputs that the staging of workgroup b + nwg reads (b
// this workgroup's linear index, nwg the compute units; the last workgroups
// take the last one): its scalar record, K, Q, dO (sequences of one length;
// with cu_seqlens only the chunk-indexed inputs), U and T, one 4-byte load
// per 128-byte L2 line (one load per 64 bytes measured no faster), folded into
// the returned value.  The LDS holds one
// workgroup per compute unit and workgroups are dealt to the XCDs round-robin,
// so that workgroup runs on this XCD and starts about when this one ends:
// its staging then reads from L2.
template <class E, int DK, int DV>
__device__ __forceinline__ uint32_t l2_prefetch_next(const GradParams& p, int tid) {
  constexpr int NT = 512;
  constexpr int KP = DK * (int)sizeof(E) / 128, VP = DV * (int)sizeof(E) / 128;  // pieces per row
  constexpr int NK = CH * KP, NDO = CH * VP, NU = CH * DV * (int)sizeof(E) / 128, NTP = CH * CH * 4 / 128,
                NR = (RECF * 4 + 127) / 128;
  constexpr int O_Q = NK, O_DO = 2 * NK, O_U = O_DO + NDO, O_T = O_U + NU, O_R = O_T + NTP, NPF = O_R + NR;
  const int nlin = gridDim.x * gridDim.y;
  const int tgt = min((int)(blockIdx.x + blockIdx.y * gridDim.x) + p.nwg, nlin - 1);
  const int ci = tgt % gridDim.x, h = tgt / gridDim.x, H = p.H;
  const bool tok = p.seq.cu == nullptr;  // token-indexed inputs without a table load
  const int2 ct = tok ? p.seq.chunk_of(nullptr, ci) : make_int2(0, 0);
  const int64_t tok0 = (int64_t)ct.x * p.seq.T + (int64_t)ct.y * CH;
  const int rmax = min(CH, p.seq.T - ct.y * CH) - 1;
  const size_t cb = (size_t)ci * H + h;
  const char* kb = static_cast<const char*>(p.k) + (tok0 * H + h) * DK * sizeof(E);
  const char* qb = static_cast<const char*>(p.q) + (tok0 * H + h) * DK * sizeof(E);
  const char* db = static_cast<const char*>(p.dout) + (tok0 * H + h) * DV * sizeof(E);
  const char* ub = static_cast<const char*>(p.us) + cb * (CH * DV * sizeof(E));
  const char* tb = reinterpret_cast<const char*>(p.t_in + cb * (CH * CH));
  const char* rb = reinterpret_cast<const char*>(p.rec + cb * RECF);
  uint32_t acc = 0;
#pragma unroll
  for (int j = 0; j < (NPF + NT - 1) / NT; ++j) {
    int i = min(tid + j * NT, NPF - 1);
    if (!tok && i < O_U) i = O_U + i % NU;
    const char* a;
    if (i < O_Q) a = kb + (int64_t)min(i / KP, rmax) * H * DK * sizeof(E) + (i % KP) * 128;
    else if (i < O_DO) a = qb + (int64_t)min((i - O_Q) / KP, rmax) * H * DK * sizeof(E) + ((i - O_Q) % KP) * 128;
    else if (i < O_U) a = db + (int64_t)min((i - O_DO) / VP, rmax) * H * DV * sizeof(E) + ((i - O_DO) % VP) * 128;
    else if (i < O_T) a = ub + (i - O_U) * 128;
    else if (i < O_R) a = tb + (i - O_T) * 128;
    else a = rb + min((i - O_R) * 128, RECF * 4 - 4);
    acc ^= *reinterpret_cast<const uint32_t*>(a);
  }
  return acc;
}

// One chunk per workgroup of 8 waves.  Wave w works on column group cw = w % 4
// (key columns [cw Dk/4, (cw+1) Dk/4), value columns [cw Dv/4, ...)) and row
// half rh = w / 4 (row tiles 2 rh, 2 rh + 1) of every per-row product, so two
// waves share each SIMD and every accumulator array is half the size it would
// be with four waves.  Sums over rows or columns that cross those halves go
// through small LDS arrays with a single writer per entry (deterministic).
// Accumulator tiles that later products read down their columns are stored
// transposed (M^T row-major, the lane's four rows of a column as one piece);
// reads across the other way use the LDS transpose loads.
// Phases of the gradient kernel's phase clock: one per barrier interval (1
// staging, 2 K K^T * D and P, 3 dU and G_P, 4 G_W / dQ1 / U dh'^T, 5 X_W / dQ /
// G_T, 6 Z, 7 G_A and E, 8 dK and the row sums), 9 the final stores.
using GradClock = PhaseClock<10>;
// [workgroup][wave][phase] (an instrumented build only)
__device__ uint32_t gdn_clock_grad[kPhaseClock ? CLOCK_BLOCKS : 1][8 * 10];

template <class E, int DK, int DV, bool PREP>
__global__ __launch_bounds__(512) void gdn_grad_kernel(GradParams p) {
  GradClock clk;
  clk.start();
  using L = GradLayout<E, DK, DV>;
  constexpr int NT = 512;
  constexpr int LK = L::LK, LV = L::LV, LT = L::LT;
  constexpr int CTK = DK / 64, CTV = DV / 64;  // 16-wide column tiles per column group
  // P5 (dU) partition: with at least eight 16-wide value tiles every wave takes
  // its own value tiles over all four row tiles, so no two waves request the
  // same dh' fragments; otherwise the column group / row half split of the
  // other products
  constexpr bool P5ALL = (DV / 16) % 8 == 0;
  constexpr int P5C = P5ALL ? DV / 128 : CTV, P5R = P5ALL ? 4 : 2;
  __shared__ GradSmem<E, DK, DV> s;
  auto slotE = [&](int i) { return reinterpret_cast<E*>(s.slot[i]); };

  const int tid = threadIdx.x, l = lane_id(), w = wave_id(), g = l >> 4, c16 = l & 15;
  const int cw = w & 3, rh = w >> 2;
  const int2 ctab = p.seq.chunk_of(p.chunk_tab, blockIdx.x);
  if (ctab.x < 0) return;  // the plan found the device cu_seqlens inconsistent
  const int n = ctab.x, jc = ctab.y, h = blockIdx.y, H = p.H;
  const int len = p.seq.len(n);
  const int64_t tok0 = p.seq.start(n) + (int64_t)jc * CH;
  const int rows = min(CH, len - jc * CH);
  const size_t SS = (size_t)DK * DV;
  // h_c and dh'_c of this chunk, both stored as Dk x Dv matrices in 4 x 16 blocks (st_blk)
  const E* hs = static_cast<const E*>(p.hs) + ((size_t)blockIdx.x * H + h) * SS;
  const E* dhs = static_cast<const E*>(p.dhs) + ((size_t)blockIdx.x * H + h) * SS;
  const int d0 = cw * (DK / 4), n0 = cw * (DV / 4);
  const int p5n0 = P5ALL ? w * (DV / 8) : n0, p5r0 = P5ALL ? 0 : 2 * rh;
  const float scale = p.scale;

  E* sK = slotE(SK);
  const PMat<E> Tm(s.slot[ST]);                                // T (row-major)
  f32x4* sKD = reinterpret_cast<f32x4*>(s.slot[SKD]);           // KD: tile (rt, ct), lane l at (4 rt + ct) 64 + l
  E* sPT = slotE(SP);                                           // scale P^T
  E* sDUT = slotE(SDU);                                         // dU^T

  // ---- P1: staging, in the order the phases need it: the chunk's scalar
  //          record (written by the T solve: decay cumsum and exponentials,
  //          beta, beta Gam, Gam_C) and K, Q (waves 0..3 and 4..7) are
  //          requested first and stored before the first barrier; U, dO (waves
  //          0..3 and 4..7) and T stay in flight during P2 and are stored at
  //          its end.  Rows past the end are zero.  Every load is issued by
  //          every lane (rows past the end read the last row and are zeroed
  //          when stored), so that the compiler knows how many loads are in
  //          flight behind each one it waits for; with loads under branches
  //          it waited for all of them.
  const int ht = tid & (NT / 2 - 1);
  typedef E vec_t __attribute__((__vector_size__(16)));
  constexpr int UVEC = 16 / (int)sizeof(E), UPC = CH * DV / UVEC / (NT / 2);  // U pieces per thread
  vec_t upc[UPC];  // U (waves 0..3) or dO (waves 4..7)
  TStage<E, NT> tst;
  {
    using GS = GradSmem<E, DK, DV>;
    static_assert(offsetof(GS, tail) == offsetof(GS, gam) + 5 * CH * sizeof(float), "record layout");
    const f32x4 rv =
        *reinterpret_cast<const f32x4*>(p.rec + ((size_t)blockIdx.x * H + h) * RECF + 4 * min(tid, RECF / 4 - 1));
    const E* q = static_cast<const E*>(p.q) + (tok0 * H + h) * DK;
    const E* k = static_cast<const E*>(p.k) + (tok0 * H + h) * DK;
    // U of this chunk as the forward (or its replay) formed it: DV/16 column
    // blocks of [CH][16], zero past the end; contiguous, so 16-byte piece i
    // of the whole [CH x DV] matrix sits at element 16 i / sizeof(E).  dO by
    // rows, 16-byte piece i at row i / (DV / UVEC).
    const E* u = static_cast<const E*>(p.us) + ((size_t)blockIdx.x * H + h) * (CH * DV);
    const E* d = static_cast<const E*>(p.dout) + (tok0 * H + h) * DV;
    TilePart<E, NT / 2, DK> tkq;
    tkq.template load<false, true>(rh == 0 ? k : q, (int64_t)H * DK, rows, ht);
#pragma unroll
    for (int i = 0; i < UPC; ++i) {
      const int pc = ht + i * (NT / 2);
      const int rd = min(pc / (DV / UVEC), rows - 1), cd = pc % (DV / UVEC);
      const E* src = rh == 0 ? u + pc * UVEC : d + (int64_t)rd * H * DV + cd * UVEC;
      upc[i] = *reinterpret_cast<const vec_t*>(src);
    }
    tst.load(p.t_in + ((size_t)blockIdx.x * H + h) * (CH * CH), tid);
    for (int e = tid; e < 4 * CH; e += NT) {
      (&s.p7[0][0])[e] = 0.f;
      (&s.c7[0][0])[e] = 0.f;
    }
    if (tid < RECF / 4) *reinterpret_cast<f32x4*>(&s.gam[4 * tid]) = rv;
    if (PREP && p.prep.qk_norm) tkq.normalize_rows(ht);
    tkq.store_zrows(rh == 0 ? sK : slotE(SQ), LK, rows, ht);
  }
  __syncthreads();
  clk.mark(1);
  // dh' down this wave's P5 value columns, requested now (behind the tiles
  // still in flight): quad transposes in P5 turn its row pieces into columns;
  // its products use the contiguous k-slot order
  RawFrag<E> dkraw[P5C][DK / 32];
#pragma unroll
  for (int nt = 0; nt < P5C; ++nt)
#pragma unroll
    for (int kb = 0; kb < DK / 32; ++kb) dkraw[nt][kb] = raw_fragC_q8_st<E>(dhs, DV, 32 * kb, p5n0 + 16 * nt);

  // ---- P2: KD = strict_lower(K K^T * D) -> slot KD; P = (Q K^T) * M, kept in
  //          fp32 registers for P7 and stored as scale P^T for P5.  Wave w
  //          takes P tiles w and w + 8 (those P7 gives it) and KD tiles w - 2
  //          and w + 4 (2 <= w < 6); the six zero tiles of P^T are written too.
  f32x4 pkeep[2];
  {
    constexpr int NJ = 3;
    f32x4 acc[NJ];
    Frag<E> xr[NJ][DK / 32], xc[NJ][DK / 32];
    auto tile = [&](int j, bool& valid, bool& isp, int& rt, int& ct) {
      valid = j < 2 || (w >= 2 && w < 6);
      isp = j == 0 || (j == 1 && w < 2);
      const int tt = j == 0 ? w : (j == 1 ? (w < 2 ? w + 8 : w - 2) : w + 4);
      rt = tt < 1 ? 0 : (tt < 3 ? 1 : (tt < 6 ? 2 : 3));
      ct = tt - rt * (rt + 1) / 2;
    };
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      bool valid, isp;
      int rt, ct;
      tile(j, valid, isp, rt, ct);
      const E* X = isp ? slotE(SQ) : sK;
      if (valid) {
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb) {
          xr[j][kb] = ld_frag(X, LK, 16 * rt + c16, 32 * kb);
          xc[j][kb] = ld_frag(sK, LK, 16 * ct + c16, 32 * kb);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      bool valid, isp;
      int rt, ct;
      tile(j, valid, isp, rt, ct);
      acc[j] = zero4();
      if (valid) {
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb) mma(acc[j], xr[j][kb], xc[j][kb]);
      }
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      bool valid, isp;
      int rt, ct;
      tile(j, valid, isp, rt, ct);
      if (valid) {
        const int c = 16 * ct + c16;
        const float gc = s.gam[c];
        const f32x4 gr4 = *reinterpret_cast<const f32x4*>(&s.gam[16 * rt + 4 * g]);
        f32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * rt + 4 * g + i;
          const float dm = __expf(gr4[i] - gc);
          v[i] = (isp ? c <= r : c < r) ? acc[j][i] * dm : 0.f;
        }
        if (isp) {
          if (j < 2) pkeep[j] = v;
          st_tile_cm<E>(sPT, LT, 16 * rt, 16 * ct, v * scale);
        } else {
          sKD[(4 * rt + ct) * 64 + l] = v;
        }
      }
    }
    if (w < 6) {  // P's strictly upper tiles (rt < ct), as zero tiles of P^T
      const int rt = w < 3 ? 0 : (w < 5 ? 1 : 2), ct = w < 3 ? w + 1 : (w < 5 ? w - 1 : 3);
      st_tile_cm<E>(sPT, LT, 16 * rt, 16 * ct, zero4());
    }
  }
  // the rest of the staging: U, dO and T (split into its bf16 parts)
  if (rh == 0) {
#pragma unroll
    for (int i = 0; i < UPC; ++i) {
      const int pc = ht + i * (NT / 2);            // piece index
      const int blk = pc / (CH * 16 / UVEC);       // column block
      const int r = (pc % (CH * 16 / UVEC)) / (16 / UVEC), c = blk * 16 + (pc % (16 / UVEC)) * UVEC;
      *reinterpret_cast<vec_t*>(slotE(SV) + r * LV + c) = upc[i];
    }
  } else {
#pragma unroll
    for (int i = 0; i < UPC; ++i) {
      const int pc = ht + i * (NT / 2);
      const int r = pc / (DV / UVEC), c = (pc % (DV / UVEC)) * UVEC;
      *reinterpret_cast<vec_t*>(slotE(SDO) + r * LV + c) = r < rows ? upc[i] : vec_t{};
    }
  }
  tst.put(Tm, tid);
  __syncthreads();
  clk.mark(2);

  // per-lane partial sums of this wave's rows (row tiles 2 rh + j)
  f32x4 rg[2], rb[2];  // dgam / dbeta terms
  float hdh = 0.f;
#pragma unroll
  for (int j = 0; j < 2; ++j) { rg[j] = zero4(); rb[j] = zero4(); }

  // rows of h and dh' at this wave's key columns (the operands of P6):
  // requested now, in flight during P5
  Frag<E> hn[CTK][DV / 32], dhn[CTK][DV / 32];
#pragma unroll
  for (int dt = 0; dt < CTK; ++dt)
#pragma unroll
    for (int kb = 0; kb < DV / 32; ++kb) {
      hn[dt][kb] = ld_frag8_st(hs, DV, d0 + 16 * dt + c16, 32 * kb);
      dhn[dt][kb] = ld_frag8_st(dhs, DV, d0 + 16 * dt + c16, 32 * kb);
    }

  // ---- P5: dU = diag(ek) K dh' + scale P^T dO (P5 rows and value columns) -> dU^T;
  //          GP = scale (dO U^T) * [i <= r] (tiles w, w + 8): GP*P row / column
  //          sums, (GP * M)^T -> slot GP; Q down the own key columns
  Frag<E> qr[2][CTK];
  {
    f32x4 du[P5R][P5C];
    Frag<E> dk_[P5C][DK / 32];
#pragma unroll
    for (int nt = 0; nt < P5C; ++nt)
#pragma unroll
      for (int kb = 0; kb < DK / 32; ++kb) dk_[nt][kb] = finish_frag(dkraw[nt][kb]);
#pragma unroll
    for (int nt = 0; nt < P5C; ++nt) {
      Frag<E> dor[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) dor[kb] = ld_fragC_q<E>(slotE(SDO), LV, 32 * kb, p5n0 + 16 * nt);
#pragma unroll
      for (int j = 0; j < P5R; ++j) {
        const int rt = p5r0 + j;
        f32x4 kd = zero4();
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb) mma(kd, ld_frag8(sK, LK, 16 * rt + c16, 32 * kb), dk_[nt][kb]);
        kd = kd * *reinterpret_cast<const f32x4*>(&s.ek[16 * rt + 4 * g]);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) mma(kd, ld_frag(sPT, LT, 16 * rt + c16, 32 * kb), dor[kb]);
        du[j][nt] = kd;
      }
    }
#pragma unroll
    for (int j = 0; j < P5R; ++j)
#pragma unroll
      for (int nt = 0; nt < P5C; ++nt) st_tile_cm<E>(sDUT, LT, 16 * (p5r0 + j), p5n0 + 16 * nt, du[j][nt]);
  }
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const int ti = w + 8 * jj;
    if (ti < 10) {
      const int rt = ti < 1 ? 0 : (ti < 3 ? 1 : (ti < 6 ? 2 : 3)), ct = ti - rt * (rt + 1) / 2;
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < DV / 32; ++kb)
        mma(acc, ld_frag(slotE(SDO), LV, 16 * rt + c16, 32 * kb), ld_frag(slotE(SV), LV, 16 * ct + c16, 32 * kb));
      const int c = 16 * ct + c16;
      const f32x4 pv = pkeep[jj];
      f32x4 rs4, gpm;
      float csum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rt + 4 * g + i;
        const float gp = (c <= r) ? scale * acc[i] : 0.f;
        // the diagonal entry enters row sum r and column sum r with opposite
        // signs: left out of both, it cannot leave a rounding residue in dgam_r
        // (which strong decay would make larger than dgam itself)
        const float gpp = (c < r) ? gp * pv[i] : 0.f;
        rs4[i] = gpp;
        csum += gpp;
        gpm[i] = (c <= r) ? gp * __expf(s.gam[r] - s.gam[c]) : 0.f;
      }
      st_tile_cm<E>(slotE(SGP), LT, 16 * rt, 16 * ct, gpm);
#pragma unroll
      for (int i = 0; i < 4; ++i) rs4[i] = row16_sum(rs4[i]);
      csum += __shfl_xor(csum, 16, 64);
      csum += __shfl_xor(csum, 32, 64);
      if (c16 == 0) *reinterpret_cast<f32x4*>(&s.p7[ct][16 * rt + 4 * g]) = rs4;
      if (g == 0) s.c7[rt][c] = -csum;
    }
  }
  if (w < 6) {  // the strictly upper tiles of (GP * M)^T are zero
    const int rt = w < 3 ? 0 : (w < 5 ? 1 : 2), ct = w < 3 ? w + 1 : (w < 5 ? w - 1 : 3);
    st_tile_cm<E>(slotE(SGP), LT, 16 * rt, 16 * ct, zero4());
  }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int dt = 0; dt < CTK; ++dt) qr[kb][dt] = ld_fragC_q<E>(slotE(SQ), LK, 32 * kb, d0 + 16 * dt);
  __syncthreads();
  clk.mark(3);
  // V rows 16 cw .. 16 cw + 15, the operand of GT in P9 (every tile of a wave
  // there has column tile cw): requested here, so that the loads are in
  // flight during P6 and P8 (rows past the end are copies of the last one;
  // beta = 0 there removes them).  Contiguous k order, one 16-byte read per
  // fragment.
  Frag<E> vf[DV / 32];
  {
    const E* v = static_cast<const E*>(p.v) + (tok0 * H + h) * DV;
    const int vrow = min(16 * cw + c16, rows - 1);
#pragma unroll
    for (int kb = 0; kb < DV / 32; ++kb) vf[kb] = ld_frag8(v + (int64_t)vrow * H * DV, 0, 0, 32 * kb);
  }

  // ---- P6: GW = -dU h^T, dQ1 = dO h^T, Udh = U dh'^T (own rows and key columns);
  //          GW -> slot Q as GW^T (Q was last read in P5)
  // (the state operands are rows of the stored h and dh', so these products
  //  use the contiguous k-slot order: one 16-byte read per fragment, each
  //  loaded once and used for both key-column tiles)
  f32x4 gw[2][CTK], dq1[2][CTK], udh[2][CTK];
  // <h, dh'> over the whole state: the two row halves share each column group's part
#pragma unroll
  for (int dt = 0; dt < CTK; ++dt)
#pragma unroll
    for (int kb = 0; kb < DV / 32; ++kb)
      if ((kb & 1) == rh) hdh = frag_dot(hn[dt][kb], dhn[dt][kb], hdh);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int rt = 2 * rh + j;
    f32x4 a[CTK], b[CTK], c[CTK];
#pragma unroll
    for (int dt = 0; dt < CTK; ++dt) a[dt] = b[dt] = c[dt] = zero4();
#pragma unroll
    for (int kb = 0; kb < DV / 32; ++kb) {
      const Frag<E> xdu = ld_fragC_q8<E>(sDUT, LT, 32 * kb, 16 * rt);
      const Frag<E> xdo = ld_frag8(slotE(SDO), LV, 16 * rt + c16, 32 * kb);
      const Frag<E> xu = ld_frag8(slotE(SV), LV, 16 * rt + c16, 32 * kb);
#pragma unroll
      for (int dt = 0; dt < CTK; ++dt) {
        mma(a[dt], xdu, hn[dt][kb]);
        mma(b[dt], xdo, hn[dt][kb]);
        mma(c[dt], xu, dhn[dt][kb]);
      }
    }
#pragma unroll
    for (int dt = 0; dt < CTK; ++dt) {
      const Frag<E> qown = rh ? qr[1][dt] : qr[0][dt];
      gw[j][dt] = zero4() - a[dt];
      dq1[j][dt] = b[dt];
      udh[j][dt] = c[dt];
      const f32x4 gm4 = *reinterpret_cast<const f32x4*>(&s.Gam[16 * rt + 4 * g]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float qv = frag_at(qown, 4 * j + i);
        rg[j][i] += scale * gm4[i] * qv * b[dt][i];
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) { pin(rg[j]); pin(rb[j]); }
  pin(hdh);
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int dt = 0; dt < CTK; ++dt) st_tile_cm<E>(slotE(SQ), LT, 16 * (2 * rh + j), d0 + 16 * dt, gw[j][dt]);
  __syncthreads();
  clk.mark(4);

  // ---- P8: XW = T^T GW (own rows); row dots; dK partial (with GPM^T Q); dQ;
  //          then GT
  f32x4 dkacc[2][CTK];
  {
    const E* sGWT = slotE(SQ);
#pragma unroll
    for (int dt = 0; dt < CTK; ++dt) {
      Frag<E> gwf[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) gwf[kb] = ld_frag(sGWT, LT, d0 + 16 * dt + c16, 32 * kb);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int rt = 2 * rh + j;
        f32x4 xw = zero4();
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) mma(xw, Tm.col_e(32 * kb, 16 * rt), gwf[kb]);
        f32x4 pq = zero4();  // GPM^T Q (GPM is final since P7)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) mma(pq, ld_frag(slotE(SGP), LT, 16 * rt + c16, 32 * kb), qr[kb][dt]);
        const f32x4 kv4 = ld_cpiece<E>(sK, LK, 16 * rt, d0 + 16 * dt);
        const f32x4 gm4 = *reinterpret_cast<const f32x4*>(&s.Gam[16 * rt + 4 * g]);
        const f32x4 bg4 = *reinterpret_cast<const f32x4*>(&s.bg[16 * rt + 4 * g]);
        const f32x4 ek4 = *reinterpret_cast<const f32x4*>(&s.ek[16 * rt + 4 * g]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float xk = xw[i] * kv4[i];
          rb[j][i] += gm4[i] * xk;
          rg[j][i] += bg4[i] * xk;
          dkacc[j][dt][i] = bg4[i] * xw[i] + ek4[i] * udh[j][dt][i] + pq[i];
        }
      }
    }
  }
  // dQ = scale diag(Gam) dQ1 + GPM K, final here (slot dO was last read in P6)
  {
    E* sDQ = slotE(SDO);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int dt = 0; dt < CTK; ++dt) {
        const int rt = 2 * rh + j;
        f32x4 a = zero4();
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          mma(a, ld_fragC_q<E>(slotE(SGP), LT, 32 * kb, 16 * rt), ld_fragC_q<E>(sK, LK, 32 * kb, d0 + 16 * dt));
        const f32x4 gm4 = *reinterpret_cast<const f32x4*>(&s.Gam[16 * rt + 4 * g]);
        st_tile_rows<E>(sDQ, LK, 16 * rt, d0 + 16 * dt, dq1[j][dt] * gm4 * scale + a);
      }
  }

  // ---- P9 (same phase): GT = dU V^T diag(beta) + GW K^T diag(beta Gam) -> slot
  //          V as GT^T (PMat; U was last read in P6).  The dbeta term
  //          sum_c (T^T dU)[r][c] V[r][c] is the column sum
  //          sum_i T[i][r] (dU V^T)[i][r], taken here from the first product.
  const PMat<E> GTT(s.slot[SV]);
  {
    const int c = 16 * cw + c16;
    float tm = 0.f;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int rt = rh + 2 * j;
      f32x4 a = zero4(), b = zero4();
#pragma unroll
      for (int kb = 0; kb < DV / 32; ++kb) mma(a, ld_fragC_q8<E>(sDUT, LT, 32 * kb, 16 * rt), vf[kb]);
#pragma unroll
      for (int kb = 0; kb < DK / 32; ++kb)
        mma(b, ld_fragC_q<E>(slotE(SQ), LT, 32 * kb, 16 * rt), ld_frag(sK, LK, c, 32 * kb));
      const f32x4 t4 = Tm.cpiece(16 * rt, 16 * cw);
      const float bc = s.beta[c], bgc = s.bg[c];
      f32x4 gt;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        gt[i] = bc * a[i] + bgc * b[i];
        tm += t4[i] * a[i];
      }
      GTT.put4(c, 16 * rt + 4 * g, gt);
    }
    tm += __shfl_xor(tm, 16, 64);
    tm += __shfl_xor(tm, 32, 64);
    if (g == 0) s.c9[rh][c] = tm;
  }
  __syncthreads();
  clk.mark(5);

  uint32_t pf;  // the prefetch below, folded; consumed after the last barrier

  // ---- P10: Z = GT T^T (own row tiles, column tile cw) -> slot P as Z^T (last
  //           read in P5), GA = strict_lower(-T^T Z) (own rows); E -> slot dU
  //           as E^T (dU^T is last read before the barrier in the middle).  XU = T^T dU (own rows and value columns) -> dV into
  //           slot Q (GW^T was last read in P9).  The rows of T^T for this
  //           wave's row tiles serve XU (in E) and GA (near fp32).
  PFrag<E> ttp[2][2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) ttp[j][kb] = Tm.col(32 * kb, 16 * (2 * rh + j));
  {
    E* sDV = slotE(SQ);
#pragma unroll
    for (int nt = 0; nt < CTV; ++nt) {
      Frag<E> duf[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) duf[kb] = ld_frag(sDUT, LT, n0 + 16 * nt + c16, 32 * kb);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int rt = 2 * rh + j;
        f32x4 xu = zero4();
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) mma(xu, e_part(ttp[j][kb]), duf[kb]);
        const f32x4 b4 = *reinterpret_cast<const f32x4*>(&s.beta[16 * rt + 4 * g]);
        st_tile_rows<E>(sDV, LV, 16 * rt, n0 + 16 * nt, xu * b4);
      }
    }
  }
  {
    // both products take fp32 operands (PFrag: near-fp32 products); the two
    // row halves of a column group each form half of Z and exchange it through
    // LDS, stored transposed so that Z's columns read back as rows
    const PMat<E> ZT(s.slot[SP]);
    {
      PFrag<E> trow[2];  // rows 16 cw.. of T
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) trow[kb] = Tm.row(16 * cw + c16, 32 * kb);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int rt = 2 * rh + j;
        f32x4 z = zero4();
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) mma(z, GTT.col(32 * kb, 16 * rt), trow[kb]);
        ZT.put4(16 * cw + c16, 16 * rt + 4 * g, z);
      }
    }
    __syncthreads();
    clk.mark(6);
    pf = l2_prefetch_next<E, DK, DV>(p, tid);
    PFrag<E> zf[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) zf[kb] = ZT.row(16 * cw + c16, 32 * kb);
    const int c = 16 * cw + c16;
    float csum = 0.f;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int rt = 2 * rh + j;
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) mma(acc, ttp[j][kb], zf[kb]);
      // KD's upper tiles were never written (and are zero)
      const f32x4 kd4 = cw <= rt ? sKD[(4 * rt + cw) * 64 + l] : zero4();
      f32x4 ev;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rt + 4 * g + i;
        const float gav = (c < r) ? -acc[i] : 0.f;
        const float gaa = gav * s.beta[r] * kd4[i];
        rg[j][i] += gaa;
        csum += gaa;
        rb[j][i] += gav * kd4[i];
        ev[i] = (c < r) ? s.beta[r] * gav * __expf(s.gam[r] - s.gam[c]) : 0.f;
      }
      st_tile_cm<E>(sDUT, LT, 16 * rt, 16 * cw, ev);
    }
    csum += __shfl_xor(csum, 16, 64);
    csum += __shfl_xor(csum, 32, 64);
    if (g == 0) s.c10[rh][c] = -csum;
  }
  __syncthreads();
  clk.mark(7);

  // e_r = ek_r k_r.(U dh'^T)_r, the reverse chain's row terms (summed here over
  // its waves): it enters dgam_r with a minus sign and the last row with a plus,
  // so dg_r gets sum_{i < r} e_i, formed as a prefix sum (adding and then
  // cancelling it leaves a rounding residue that strong decay would make larger
  // than dg itself).  Every wave loads them (a branch around the loads made
  // the compiler wait for them at once); wave 0 uses them at the end.
  float epv[RevWaves<DV>::NW];
  {
    const float* ep = p.ep + ((size_t)blockIdx.x * H + h) * (EPW * CH);
#pragma unroll
    for (int ww = 0; ww < RevWaves<DV>::NW; ++ww) epv[ww] = ep[ww * CH + l];
  }

  // ---- P11: dK = dK partial + (E + E^T) K (own rows and key columns) -> slot KD
  //           (last read in P10).  The three gradient tiles are written out
  //           after the last barrier, so that no load of this kernel waits
  //           behind a store.
  {
    E* sDK = slotE(SKD);
    const E* sET = sDUT;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int dt = 0; dt < CTK; ++dt) {
        const int rt = 2 * rh + j;
        f32x4 b = dkacc[j][dt];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const Frag<E> kc = ld_fragC_q<E>(sK, LK, 32 * kb, d0 + 16 * dt);
          mma(b, ld_fragC_q<E>(sET, LT, 32 * kb, 16 * rt), kc);  // rows of E
          mma(b, ld_frag(sET, LT, 16 * rt + c16, 32 * kb), kc);   // rows of E^T
        }
        st_tile_rows<E>(sDK, LK, 16 * rt, d0 + 16 * dt, b);
      }
  }

  // ---- P12: reductions, dbeta, dg
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    f32x4 a = rg[j], b = rb[j];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = row16_sum(a[i]);
      b[i] = row16_sum(b[i]);
    }
    if (c16 == 0) {
      *reinterpret_cast<f32x4*>(&s.pg[cw][16 * (2 * rh + j) + 4 * g]) = a;
      *reinterpret_cast<f32x4*>(&s.pb[cw][16 * (2 * rh + j) + 4 * g]) = b;
    }
  }
  {
    const float b = wave_sum(hdh);
    if (l == 0) s.ph[w] = b;
  }
  __syncthreads();
  clk.mark(8);
  // The prefetch's loads and the row terms e end here, before the first
  // store: the compiler cannot count the stores of the tile loops below (their
  // trip count depends on the rows), so a wait after them for a load issued
  // before them waited for every one of them too (wave 0's sums did).
  float esum = 0.f;
#pragma unroll
  for (int ww = 0; ww < RevWaves<DV>::NW; ++ww) esum += epv[ww];
  asm volatile("" ::"v"(pf), "v"(esum));
  store_tile<E, DV, NT>(slotE(SQ), LV, static_cast<E*>(p.dv) + (tok0 * H + h) * DV, (int64_t)H * DV, rows);
  if (PREP && p.prep.qk_norm) {
    // gradients with respect to the raw q and k (the kernel saw them normalised)
    store_tile_unnorm<E, DK, NT>(slotE(SDO), LK, static_cast<const E*>(p.q) + (tok0 * H + h) * DK, (int64_t)H * DK,
                                 static_cast<E*>(p.dq) + (tok0 * H + h) * DK, (int64_t)H * DK, rows);
    store_tile_unnorm<E, DK, NT>(slotE(SKD), LK, static_cast<const E*>(p.k) + (tok0 * H + h) * DK, (int64_t)H * DK,
                                 static_cast<E*>(p.dk) + (tok0 * H + h) * DK, (int64_t)H * DK, rows);
  } else {
    store_tile<E, DK, NT>(slotE(SDO), LK, static_cast<E*>(p.dq) + (tok0 * H + h) * DK, (int64_t)H * DK, rows);
    store_tile<E, DK, NT>(slotE(SKD), LK, static_cast<E*>(p.dk) + (tok0 * H + h) * DK, (int64_t)H * DK, rows);
  }
  if (w == 0) {
    const int r = l;
    float dgm = s.c10[0][r] + s.c10[1][r], db = s.c9[0][r] + s.c9[1][r];
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      dgm += s.pg[ww][r] + s.p7[ww][r] + s.c7[ww][r];
      db += s.pb[ww][r];
    }
    if (r == CH - 1) {
      float extra = 0.f;
#pragma unroll
      for (int ww = 0; ww < 8; ++ww) extra += s.tail[1] * s.ph[ww];
      dgm += extra;
    }
    const float e = esum;
    // dg_r = sum_{r' >= r} dgam_r' (suffix scan = prefix scan over reversed
    // lanes) + sum_{i < r} e_i (exclusive prefix scan)
    const float rev = __shfl(dgm, CH - 1 - r, 64);
    const float sc = wave_incl_scan(rev);
    const float ei = wave_incl_scan(e);
    const float ex = __shfl_up(ei, 1, 64);
    const float dgv = __shfl(sc, CH - 1 - r, 64) + (r == 0 ? 0.f : ex);
    if (r < rows) {
      const int64_t si = (tok0 + r) * H + h;
      if (PREP && p.prep.gate_act) {
        // chain rule through g = -s softplus(a) and beta = sigmoid(b)
        const float s_h = p.prep.gate_scale ? p.prep.gate_scale[h] : 1.f;
        const float bs = sigmoid_f(to_f(static_cast<const E*>(p.beta)[si]));
        p.dg[si] = -s_h * sigmoid_f(p.g[si]) * dgv;
        static_cast<E*>(p.dbeta)[si] = to_e<E>(db * bs * (1.f - bs));
      } else {
        p.dg[si] = dgv;
        static_cast<E*>(p.dbeta)[si] = to_e<E>(db);
      }
    }
  }
  if constexpr (kPhaseClock) {
    clk.mark(9);
    const int blk = blockIdx.x + blockIdx.y * gridDim.x;
    if (blk < CLOCK_BLOCKS) clk.flush(gdn_clock_grad[blk]);
  }
}

template <class E, int DK, int DV>
hipError_t launch_grad_t(const GradParams& p, int nchunk_total, hipStream_t st) {
  // the scalar records and T are solved beforehand (as for the chains)
  if (!p.t_in || !p.rec || !p.us || !p.ep) return hipErrorInvalidValue;
  if (p.prep.qk_norm || p.prep.gate_act)
    hipLaunchKernelGGL((gdn_grad_kernel<E, DK, DV, true>), dim3(nchunk_total, p.H), dim3(512), 0, st, p);
  else
    hipLaunchKernelGGL((gdn_grad_kernel<E, DK, DV, false>), dim3(nchunk_total, p.H), dim3(512), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_grad(int dtype, int DK, int DV, const GradParams& p, int nchunk_total, hipStream_t st) {
  if (dtype == 1) {
    if (DK == 128 && DV == 128) return launch_grad_t<bf16, 128, 128>(p, nchunk_total, st);
    if (DK == 64 && DV == 64) return launch_grad_t<bf16, 64, 64>(p, nchunk_total, st);
    if (DK == 64 && DV == 128) return launch_grad_t<bf16, 64, 128>(p, nchunk_total, st);
    if (DK == 128 && DV == 64) return launch_grad_t<bf16, 128, 64>(p, nchunk_total, st);
  } else {
    if (DK == 64 && DV == 64) return launch_grad_t<float, 64, 64>(p, nchunk_total, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn

#ifdef GDN_PHASE_CLOCK
// The reverse chain's ([CLOCK_BLOCKS][8 waves][8 phases]) and the gradient
// kernel's ([CLOCK_BLOCKS][8 waves][10 phases]) phase clocks, uint32 cycles, to
// host memory; an instrumented build only.
extern "C" int gdn_clock_read_rev(uint32_t* host) {
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(gdn::gdn_clock_rev), sizeof(gdn::gdn_clock_rev));
}
extern "C" int gdn_clock_read_grad(uint32_t* host) {
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(gdn::gdn_clock_grad), sizeof(gdn::gdn_clock_grad));
}
#endif
