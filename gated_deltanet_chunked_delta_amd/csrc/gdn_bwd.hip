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

template <class E, int DK, int DV>
struct alignas(16) RevSmem {
  static constexpr int LQ = ldpad<E>(DK);
  static constexpr int LT = ldpad<E>(CH);
  static constexpr int LA = CH + 4;
  E Q[CH * LQ];    // row-major, X of Q K^T
  E K[CH * LQ];    // row-major, X/Y of K K^T, X of K dh'
  E KT[DK * LT];   // K^T, X of W^T
  E QT[DK * LT];   // Q^T, X of (Gam Q)^T dO
  E DOT[DV * LT];  // dO^T, Y of P^T dO and (Gam Q)^T dO
  E WT[DK * LT];   // -W^T
  E PT[CH * LT];   // scale * P^T
  float T[CH * LA];
  // the chunk's scalar record, as laid out in memory (tail: Lambda_c, Gam_C)
  alignas(16) float gam[CH], Gam[CH], ek[CH], beta[CH], bg[CH], tail[4];
  alignas(16) float sGam[CH];  // scale Gam, zero past the sequence end
};

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
  };
  __device__ __forceinline__ static bool q_half() { return threadIdx.x >= KQT; }
  __device__ __forceinline__ static int kq_tid() { return threadIdx.x & (KQT - 1); }

  __device__ static void issue(Loader& ld, const RevParams& p, int64_t tok0, int rows, int h, const float* rec) {
    const int H = p.H;
    const void* src = q_half() ? p.q : p.k;
    ld.kq.load(static_cast<const E*>(src) + (tok0 * H + h) * DK, (int64_t)H * DK, rows, kq_tid());
    ld.d.load(static_cast<const E*>(p.dout) + (tok0 * H + h) * DV, (int64_t)H * DV, rows);
    ld.rec.load(rec);
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
      sp->PT[c * LT + r] = to_e<E>((c <= r && r < rows) ? p.scale * acc[i] * __expf(gr4[i] - gc) : 0.f);
    }
  }

  // dh: gradient at the chunk end on entry, at the chunk start on exit.
  // Prefetches chunk (ntok0, nrows) into ld (nrows = 0: none).  Returns Lambda_c.
  // t_in: this chunk's T; nrec: the next chunk's scalar record.  LEAD: a
  // lead-in chunk after the segment proper, which only advances the gradient
  // (nothing is written).
  template <bool LEAD>
  __device__ static void step(S& s0, const RevParams& p, Loader& ld, int rows, int64_t ntok0, int nrows, int h,
                              E* dhs_chunk, const float* t_in, const float* nrec, f32x4 (&dh)[DK / 16][NTW]) {
    constexpr int LQ = S::LQ, LT = S::LT, LA = S::LA;
    constexpr int TPT = CH * CH / (4 * NT);  // 4-float pieces of T per thread
    const int tid = threadIdx.x, l = lane_id(), w = wave_id(), g = l >> 4, c16 = l & 15;
    const int n0 = w * (DV / NW);

    // ---- 1. gradient at the chunk end out; tiles into LDS; scalars
    S* sp = lds_opaque(&s0);
    // stored as S (Dv x Dk) in 4 x 16 blocks: the lane's four rows of one
    // column are contiguous
    if constexpr (!LEAD) {
#pragma unroll
      for (int t = 0; t < DK / 16; ++t)
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) st4f<E>(dhs_chunk + st_blk(n0 + 16 * nt + c16, 16 * t + 4 * g, DK), dh[t][nt]);
    }
    S& s1 = *sp;
    if (PREP && p.prep.qk_norm) ld.kq.normalize_rows(kq_tid());
    {
      const bool qh = q_half();
      ld.kq.store(qh ? s1.Q : s1.K, LQ, qh ? s1.QT : s1.KT, LT, kq_tid());
    }
    ld.d.store(nullptr, 0, s1.DOT, LT);
    static_assert(offsetof(S, tail) == offsetof(S, gam) + 5 * CH * sizeof(float), "record layout");
    ld.rec.store(s1.gam);
    if (tid >= CH / 4 && tid < CH / 2) {
      // the threads that hold Gam form scale Gam, zero past the sequence end
      const int r0 = 4 * tid - CH;
      f32x4 sg;
#pragma unroll
      for (int i = 0; i < 4; ++i) sg[i] = r0 + i < rows ? p.scale * ld.rec.rv[i] : 0.f;
      *reinterpret_cast<f32x4*>(&s1.sGam[r0]) = sg;
    }
    __syncthreads();

    // ---- 2. Q K^T -> scale P^T: the ten lower 16x16 tiles, tile j on wave j % NW
    //         (at most two tiles a wave with eight waves).  T is requested now,
    //         past the staging, and lands in LDS at the end of this phase.
    f32x4 tv[TPT];
#pragma unroll
    for (int i = 0; i < TPT; ++i) tv[i] = *reinterpret_cast<const f32x4*>(t_in + 4 * (tid + i * NT));
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
    {
      S& s = *lds_opaque(&s0);
#pragma unroll
      for (int i = 0; i < TPT; ++i) {
        const int e = 4 * (tid + i * NT);
        *reinterpret_cast<f32x4*>(&s.T[(e / CH) * LA + e % CH]) = tv[i];
      }
    }
    __syncthreads();

    // ---- 3. the next chunk's tiles start their way from HBM
    if (nrows > 0) issue(ld, p, ntok0, nrows, h, nrec);

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
        for (int kb = 0; kb < 2; ++kb) yt[rr][kb] = ld_frag_f32<E>(s.T, LA, 16 * (rt0 + rr) + c16, 32 * kb);
#pragma unroll
      for (int dd = 0; dd < KTW; ++dd) {
        const int dt = kt0 + dd;
        Frag<E> xk[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) xk[kb] = ld_frag_kscaled<E>(s.KT, LT, 16 * dt + c16, 32 * kb, s.bg);
#pragma unroll
        for (int rr = 0; rr < RTW; ++rr) {
          f32x4 acc = zero4();
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) mma(acc, xk[kb], yt[rr][kb]);
#pragma unroll
          for (int i = 0; i < 4; ++i) s.WT[(16 * dt + 4 * g + i) * LT + 16 * (rt0 + rr) + c16] = to_e<E>(-acc[i]);
        }
      }
    }
    __syncthreads();

    // ---- 5. dU = diag(ek) K dh' + scale P^T dO ;  dh = Gam_C dh' + scale (Gam Q)^T dO - W^T dU
    f32x4 du[4][NTW];
    {
      S& s = *lds_opaque(&s0);
      Frag<E> hf[NTW][DK / 32];
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb) pack_frag(hf[nt][kb], dh[2 * kb][nt], dh[2 * kb + 1][nt]);
      Frag<E> yd[NTW][2];
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) yd[nt][kb] = ld_frag(s.DOT, LT, n0 + 16 * nt + c16, 32 * kb);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        Frag<E> xk[DK / 32];
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb) xk[kb] = ld_frag(s.K, LQ, 16 * rt + c16, 32 * kb);
        const f32x4 e4 = *reinterpret_cast<const f32x4*>(&s.ek[16 * rt + 4 * g]);
        Frag<E> xp[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) xp[kb] = ld_frag(s.PT, LT, 16 * rt + c16, 32 * kb);
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
          f32x4 acc = zero4();
#pragma unroll
          for (int kb = 0; kb < DK / 32; ++kb) mma(acc, xk[kb], hf[nt][kb]);
          acc = acc * e4;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) mma(acc, xp[kb], yd[nt][kb]);
          du[rt][nt] = acc;
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
            mma(dh[t][nt], ld_frag_kscaled<E>(s.QT, LT, 16 * t + c16, 32 * kb, s.sGam), yd[nt][kb]);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) mma(dh[t][nt], ld_frag(s.WT, LT, 16 * t + c16, 32 * kb), uf[kb]);
        }
      }
    }
    __syncthreads();
  }

  // Issue the loads of chunk we - 1, the first of a run (before the state
  // gradient is loaded, so that the two are in flight together).
  __device__ static void prime(Loader& ld, const RevParams& p, int64_t seq0, int len, int64_t chunk0, int cb, int we,
                               int h) {
    const int c = we - 1;
    if (c >= cb) issue(ld, p, seq0 + (int64_t)c * CH, min(CH, len - c * CH), h, p.rec + ((chunk0 + c) * p.H + h) * RECF);
  }
  // Chunks we-1 down to cb from the gradient in dh: chunks at or after ce are
  // the lead-in (the gradient advances, nothing is written), chunks below ce
  // write their chunk-end gradients.  ld: primed for chunk we - 1.
  __device__ static void run(S& s, const RevParams& p, int64_t seq0, int len, int64_t chunk0, int cb, int ce, int we,
                             int h, f32x4 (&dh)[DK / 16][DV / (16 * RevWaves<DV>::NW)], Loader& ld) {
    const size_t SS = (size_t)DK * DV;
    E* dhs = static_cast<E*>(p.dhs);
    // the lead-in and the segment proper as two loops, each with its own
    // register allocation
    auto chunk = [&](auto lead, int c) {
      const int rows = min(CH, len - c * CH);
      const bool more = c - 1 >= cb;
      const int64_t ntok0 = seq0 + (int64_t)(c - 1) * CH;
      const int nrows = more ? min(CH, len - (c - 1) * CH) : 0;
      const float* tin = p.t_in + ((chunk0 + c) * p.H + h) * (size_t)(CH * CH);
      const float* nrec = more ? p.rec + ((chunk0 + c - 1) * p.H + h) * RECF : nullptr;
      if constexpr (decltype(lead)::value) step<true>(s, p, ld, rows, ntok0, nrows, h, nullptr, tin, nrec, dh);
      else step<false>(s, p, ld, rows, ntok0, nrows, h, dhs + ((chunk0 + c) * p.H + h) * SS, tin, nrec, dh);
    };
    for (int c = we - 1; c >= ce; --c) chunk(std::true_type{}, c);
    for (int c = ce - 1; c >= cb; --c) chunk(std::false_type{}, c);
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
  // T's strictly-upper blocks and the tiles of P^T above the diagonal are never written
  for (int e = threadIdx.x; e < CH * CH; e += blockDim.x) {
    s.T[(e >> 6) * Sm::LA + (e & 63)] = 0.f;
    s.PT[(e >> 6) * Sm::LT + (e & 63)] = to_e<E>(0.f);
  }
  __syncthreads();
}

// One segment of the reverse chain.  A segment that ends before its sequence
// does starts from dh' = 0 a few chunks later (the lead-in, until the chunks'
// log-bounds sum to ln 2^-24 or less; else from the sequence end and dhT), so
// every segment runs independently of the others.
template <class E, int DK, int DV, bool PREP>
__global__ __launch_bounds__(64 * RevWaves<DV>::NW) void gdn_rev_seg(RevParams p) {
  __shared__ RevSmem<E, DK, DV> s;
  const SegDesc sd = p.segs[blockIdx.x];
  const int h = blockIdx.y, n = sd.n;
  const int64_t seq0 = p.seq.start(n), chunk0 = p.chunk_first[n];
  const int len = p.seq.len(n), nch = (len + CH - 1) / CH;
  const size_t SS = (size_t)DK * DV;
  const int we = sd.c_end < nch ? lead_in_end(p.rec, chunk0, p.H, h, sd.c_end, nch) : nch;
  f32x4 dh[DK / 16][DV / (16 * RevWaves<DV>::NW)];
  using C = RevChunk<E, DK, DV, PREP>;
  typename C::Loader ld;
  C::prime(ld, p, seq0, len, chunk0, sd.c_begin, we, h);
  rev_init_smem(s);
  rev_load<E, DK, DV>(dh, (we == nch && p.dhT) ? p.dhT + ((size_t)n * p.H + h) * SS : nullptr);
  C::run(s, p, seq0, len, chunk0, sd.c_begin, sd.c_end, we, h, dh, ld);
  if (sd.c_begin == 0 && p.dh0) rev_store<E, DK, DV>(dh, p.dh0 + ((size_t)n * p.H + h) * SS);
}

template <class E, int DK, int DV>
hipError_t launch_rev_t(const RevParams& p, int nseg_total, hipStream_t st) {
  const dim3 block(64 * RevWaves<DV>::NW);
  const dim3 grid(nseg_total, p.H);
  // T and the scalar records are solved beforehand
  if (!p.t_in || !p.rec) return hipErrorInvalidValue;
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
  static constexpr int LT = CH + 4;     // transposed [D][64] E
  static constexpr int LA = CH + 4;     // fp32 [64][64]
  static constexpr int cmax(int a, int b) { return a > b ? a : b; }
  static constexpr int SLOT = cmax(cmax(CH * LK * (int)sizeof(E), CH * LV * (int)sizeof(E)),
                                   cmax(DK * LT * (int)sizeof(E), CH * LA * 4));
  static constexpr int NSLOT = 9;
};

template <class E, int DK, int DV>
struct alignas(16) GradSmem {
  using L = GradLayout<E, DK, DV>;
  alignas(16) char slot[L::NSLOT][L::SLOT];
  alignas(16) float gam[CH], Gam[CH], ek[CH], beta[CH], bg[CH];
  float pg[4][CH], pb[4][CH];  // row sums of the per-wave dgam / dbeta terms, by column group
  float p7[4][CH], c7[4][CH];  // row sums of GP*P by column tile, column sums by row tile
  float c9[2][CH];             // column sums of T * (dU V^T) by row half
  float c10[2][CH];            // column sums of GA*A by row half
  float ph[8];
  float GamC;
};

// slot roles
enum { SK = 0, SKT = 1, SQ = 2, SV = 3, SDO = 4, ST = 5, SKD = 6, SP = 7, SDU = 8 };

// A 64 x 64 fp32 matrix in one LDS slot, kept for near-fp32 products (PFrag).
// E = float stores it as is (row stride LA).  E = bf16 stores its bf16 hi and
// lo parts (x = hi + lo, lo the rounded residual) as two planes of row stride
// LP: each value is split once, when written, and fragments load ready to
// multiply.  row(): k-slots along row r; col(): k-slots down column c0 + lane%16.
template <class E> struct PMat;
template <> struct PMat<float> {
  static constexpr int LA = CH + 4;
  float* m;
  __device__ __forceinline__ explicit PMat(void* slot) : m(static_cast<float*>(slot)) {}
  __device__ __forceinline__ void put(int r, int c, float x) const { m[r * LA + c] = x; }
  __device__ __forceinline__ void put4(int r, int c0, const f32x4& x) const {
    *reinterpret_cast<f32x4*>(&m[r * LA + c0]) = x;
  }
  __device__ __forceinline__ float at(int r, int c) const { return m[r * LA + c]; }
  __device__ __forceinline__ Frag<float> row_e(int r, int k0) const { return ld_frag(m, LA, r, k0); }
  __device__ __forceinline__ PFrag<float> row(int r, int k0) const { return PFrag<float>(ld_frag(m, LA, r, k0)); }
  __device__ __forceinline__ PFrag<float> col(int k0, int c0) const {
    return PFrag<float>(ld_fragT<float>(m, LA, c0 + (lane_id() & 15), k0, 1.f));
  }
};
template <> struct PMat<bf16> {
  static constexpr int LP = CH + 4;  // bf16 elements per row: 8-byte aligned rows
  bf16* hi;
  bf16* lo;
  typedef bf16 b4_t __attribute__((__vector_size__(8)));
  __device__ __forceinline__ explicit PMat(void* slot)
      : hi(static_cast<bf16*>(slot)), lo(static_cast<bf16*>(slot) + CH * LP) {}
  __device__ __forceinline__ static void split(float x, bf16& h, bf16& l) {
    h = (bf16)x;
    l = (bf16)(x - (float)h);
  }
  __device__ __forceinline__ void put(int r, int c, float x) const {
    bf16 h, l;
    split(x, h, l);
    hi[r * LP + c] = h;
    lo[r * LP + c] = l;
  }
  __device__ __forceinline__ void put4(int r, int c0, const f32x4& x) const {
    b4_t h, l;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bf16 a, b;
      split(x[i], a, b);
      h[i] = a;
      l[i] = b;
    }
    *reinterpret_cast<b4_t*>(&hi[r * LP + c0]) = h;
    *reinterpret_cast<b4_t*>(&lo[r * LP + c0]) = l;
  }
  __device__ __forceinline__ float at(int r, int c) const { return (float)hi[r * LP + c] + (float)lo[r * LP + c]; }
  __device__ __forceinline__ Frag<bf16> row_e(int r, int k0) const { return ld_frag(hi, LP, r, k0); }
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
};

// One chunk per workgroup of 8 waves.  Wave w works on column group cw = w % 4
// (key columns [cw Dk/4, (cw+1) Dk/4), value columns [cw Dv/4, ...)) and row
// half rh = w / 4 (row tiles 2 rh, 2 rh + 1) of every per-row product, so two
// waves share each SIMD and every accumulator array is half the size it would
// be with four waves.  Sums over rows or columns that cross those halves go
// through small LDS arrays with a single writer per entry (deterministic).
template <class E, int DK, int DV, bool PREP>
__global__ __launch_bounds__(512) void gdn_grad_kernel(GradParams p) {
  using L = GradLayout<E, DK, DV>;
  constexpr int NT = 512;
  constexpr int LK = L::LK, LV = L::LV, LT = L::LT, LA = L::LA;
  constexpr int CTK = DK / 64, CTV = DV / 64;  // 16-wide column tiles per column group
  // P5 (dU) partition: with at least eight 16-wide value tiles every wave takes
  // its own value tiles over all four row tiles, so no two waves request the
  // same dh' fragments; otherwise the column group / row half split of the
  // other products
  constexpr bool P5ALL = (DV / 16) % 8 == 0;
  constexpr int P5C = P5ALL ? DV / 128 : CTV, P5R = P5ALL ? 4 : 2;
  __shared__ GradSmem<E, DK, DV> s;
  auto slotE = [&](int i) { return reinterpret_cast<E*>(s.slot[i]); };
  auto slotF = [&](int i) { return reinterpret_cast<float*>(s.slot[i]); };

  const int tid = threadIdx.x, l = lane_id(), w = wave_id(), g = l >> 4, c16 = l & 15;
  const int cw = w & 3, rh = w >> 2;
  const int2 ctab = p.chunk_tab[blockIdx.x];
  const int n = ctab.x, jc = ctab.y, h = blockIdx.y, H = p.H;
  const int len = p.seq.len(n);
  const int64_t tok0 = p.seq.start(n) + (int64_t)jc * CH;
  const int rows = min(CH, len - jc * CH);
  const size_t SS = (size_t)DK * DV;
  // h_c and dh'_c of this chunk, both stored as S-shaped (Dv x Dk) matrices in 4 x 16 blocks (st_blk)
  const E* hs = static_cast<const E*>(p.hs) + ((size_t)blockIdx.x * H + h) * SS;
  const E* dhs = static_cast<const E*>(p.dhs) + ((size_t)blockIdx.x * H + h) * SS;
  const int d0 = cw * (DK / 4), n0 = cw * (DV / 4);
  const int p5n0 = P5ALL ? w * (DV / 8) : n0, p5r0 = P5ALL ? 0 : 2 * rh;
  const float scale = p.scale;

  E* sK = slotE(SK);
  E* sKT = slotE(SKT);
  const PMat<E> TT(s.slot[ST]);  // T^T (so that T^T's rows, the most read, load as rows)
  float* sKD = slotF(SKD);
  float* sP = slotF(SP);
  E* sDU = slotE(SDU);

  // ---- P1: staging (all four tiles in flight at once; rows past the end are
  //          zero); zero T (unless given), P and the cross-wave sum arrays.
  //          dh' down this wave's value columns (the operand of P5) is
  //          requested after the tiles have landed and stays in flight until
  //          P5; its products use the contiguous k-slot order (one 16-byte
  //          read per fragment).
  Frag<E> dk_[P5C][DK / 32];
  {
    const E* q = static_cast<const E*>(p.q) + (tok0 * H + h) * DK;
    const E* k = static_cast<const E*>(p.k) + (tok0 * H + h) * DK;
    // U of this chunk as the forward (or its replay) formed it: DV/16 column
    // blocks of [CH][16], zero past the end; contiguous, so 16-byte piece i
    // of the whole [CH x DV] matrix sits at element 16 i / sizeof(E)
    const E* u = static_cast<const E*>(p.us) + ((size_t)blockIdx.x * H + h) * (CH * DV);
    const E* d = static_cast<const E*>(p.dout) + (tok0 * H + h) * DV;
    // waves 0..3 bring K and Q, waves 4..7 U and dO
    const int ht = tid & (NT / 2 - 1);
    TilePart<E, NT / 2, DK> tk, tq;
    TilePart<E, NT / 2, DV> td;
    typedef E vec_t __attribute__((__vector_size__(16)));
    constexpr int UVEC = 16 / (int)sizeof(E), UPC = CH * DV / UVEC / (NT / 2);  // pieces per thread
    vec_t upc[UPC];
    if (rh == 0) {
      tk.template load<true>(k, (int64_t)H * DK, rows, ht);
      tq.template load<true>(q, (int64_t)H * DK, rows, ht);
    } else {
#pragma unroll
      for (int i = 0; i < UPC; ++i) upc[i] = *reinterpret_cast<const vec_t*>(u + (ht + i * (NT / 2)) * UVEC);
      td.template load<true>(d, (int64_t)H * DV, rows, ht);
    }
    // T (requested after the tiles)
    constexpr int TPT = CH * CH / (4 * NT);
    const float* tin = p.t_in + ((size_t)blockIdx.x * H + h) * (CH * CH);
    f32x4 tvals[TPT];
#pragma unroll
    for (int i = 0; i < TPT; ++i) tvals[i] = *reinterpret_cast<const f32x4*>(tin + 4 * (tid + i * NT));
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int e = 4 * (tid + i * NT);
      *reinterpret_cast<f32x4*>(&sP[(e >> 6) * LA + (e & 63)]) = zero4();
    }
    for (int e = tid; e < 4 * CH; e += NT) {
      (&s.p7[0][0])[e] = 0.f;
      (&s.c7[0][0])[e] = 0.f;
    }
    if (w == 0) {
      const bool valid = l < rows;
      const int64_t si = (tok0 + l) * H + h;
      float gr = valid ? p.g[si] : 0.f;
      float bt = valid ? to_f(static_cast<const E*>(p.beta)[si]) : 0.f;
      if (PREP && p.prep.gate_act && valid) {
        gr = -(p.prep.gate_scale ? p.prep.gate_scale[h] : 1.f) * softplus_f(gr);
        bt = sigmoid_f(bt);
      }
      const float gm = wave_incl_scan(gr);
      const float gC = __shfl(gm, 63, 64);
      const float Gm = __expf(gm);
      s.gam[l] = gm;
      s.Gam[l] = Gm;
      s.ek[l] = __expf(gC - gm);
      s.beta[l] = bt;
      s.bg[l] = bt * Gm;
      if (l == 0) s.GamC = __expf(gC);
    }
    if (PREP && p.prep.qk_norm && rh == 0) {
      tk.normalize_rows(ht);
      tq.normalize_rows(ht);
    }
    if (rh == 0) {
      tk.store(sK, LK, sKT, LT, ht);
      tq.store(slotE(SQ), LK, nullptr, 0, ht);
    } else {
#pragma unroll
      for (int i = 0; i < UPC; ++i) {
        const int pc = ht + i * (NT / 2);            // piece index
        const int blk = pc / (CH * 16 / UVEC);       // column block
        const int r = (pc % (CH * 16 / UVEC)) / (16 / UVEC), c = blk * 16 + (pc % (16 / UVEC)) * UVEC;
        *reinterpret_cast<vec_t*>(slotE(SV) + r * LV + c) = upc[i];
      }
      td.store(slotE(SDO), LV, nullptr, 0, ht);
    }
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int e = 4 * (tid + i * NT);
#pragma unroll
      for (int q = 0; q < 4; ++q) TT.put((e & 63) + q, e >> 6, tvals[i][q]);
    }
  }
  __syncthreads();
  // dh' down this wave's P5 value columns, requested only now: every
  // workgroup stages its tiles at about the same time, and the tiles arrive
  // sooner without the state queued beside them
#pragma unroll
  for (int nt = 0; nt < P5C; ++nt)
#pragma unroll
    for (int kb = 0; kb < DK / 32; ++kb) dk_[nt][kb] = ld_frag8_st(dhs, DK, p5n0 + 16 * nt + c16, 32 * kb);

  // ---- P2: KD = strict_lower(K K^T * D), P = (Q K^T) * M  (20 lower tiles:
  //          tile w + 8j for wave w, all fragment reads issued before the products)
  {
    constexpr int NJ = 3;
    f32x4 acc[NJ];
    Frag<E> xr[NJ][DK / 32], xc[NJ][DK / 32];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int ti = w + 8 * j, tt = ti >= 10 ? ti - 10 : ti;
      const int rt = tt < 1 ? 0 : (tt < 3 ? 1 : (tt < 6 ? 2 : 3)), ct = tt - rt * (rt + 1) / 2;
      const E* X = ti >= 10 ? slotE(SQ) : sK;
      if (ti < 20) {
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb) {
          xr[j][kb] = ld_frag(X, LK, 16 * rt + c16, 32 * kb);
          xc[j][kb] = ld_frag(sK, LK, 16 * ct + c16, 32 * kb);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      acc[j] = zero4();
      if (w + 8 * j < 20) {
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb) mma(acc[j], xr[j][kb], xc[j][kb]);
      }
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int ti = w + 8 * j, tt = ti >= 10 ? ti - 10 : ti;
      const int rt = tt < 1 ? 0 : (tt < 3 ? 1 : (tt < 6 ? 2 : 3)), ct = tt - rt * (rt + 1) / 2;
      if (ti < 20) {
        const int c = 16 * ct + c16;
        const float gc = s.gam[c];
        const f32x4 gr4 = *reinterpret_cast<const f32x4*>(&s.gam[16 * rt + 4 * g]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * rt + 4 * g + i;
          const float dm = __expf(gr4[i] - gc);
          if (ti < 10) sKD[r * LA + c] = (c < r) ? acc[j][i] * dm : 0.f;
          else sP[r * LA + c] = (c <= r) ? acc[j][i] * dm : 0.f;
        }
      }
    }
  }
  __syncthreads();

  // per-lane partial sums of this wave's rows (row tiles 2 rh + j)
  f32x4 rg[2], rb[2];  // dgam / dbeta terms
  // e_r = ek_r k_r.(U dh'^T)_r, kept apart: it enters dgam_r with a minus sign
  // and the last row with a plus, so dg_r gets sum_{i < r} e_i, formed as a
  // prefix sum (adding and then cancelling it leaves a rounding residue that
  // strong decay would make larger than dg itself)
  f32x4 re[2];
  float hdh = 0.f;
#pragma unroll
  for (int j = 0; j < 2; ++j) { rg[j] = zero4(); rb[j] = zero4(); re[j] = zero4(); }

  // h and dh' down this wave's key columns (the operands of P6): requested now,
  // in flight during P5, quad-transposed in P6
  RawFrag<E> hraw[CTK][DV / 32], dhraw[CTK][DV / 32];
#pragma unroll
  for (int dt = 0; dt < CTK; ++dt)
#pragma unroll
    for (int kb = 0; kb < DV / 32; ++kb) {
      hraw[dt][kb] = raw_fragC_q8_st<E>(hs, DK, 32 * kb, d0 + 16 * dt);
      dhraw[dt][kb] = raw_fragC_q8_st<E>(dhs, DK, 32 * kb, d0 + 16 * dt);
    }

  // ---- P5: dU = diag(ek) K dh' + scale P^T dO (P5 rows and value columns)
  f32x4 du[P5R][P5C];
  {
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
        for (int kb = 0; kb < 2; ++kb) mma(kd, ld_fragT<E>(sP, LA, 16 * rt + c16, 32 * kb, scale), dor[kb]);
        du[j][nt] = kd;
      }
    }
  }
#pragma unroll
  for (int j = 0; j < P5R; ++j)
#pragma unroll
    for (int nt = 0; nt < P5C; ++nt) st_tile_rows<E>(sDU, LV, 16 * (p5r0 + j), p5n0 + 16 * nt, du[j][nt]);
  __syncthreads();

  // ---- P6: GW = -dU h^T, dQ1 = dO h^T, Udh = U dh'^T (own rows and key columns)
  Frag<E> qr[2][CTK];  // Q down the own key columns, all rows
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int dt = 0; dt < CTK; ++dt) qr[kb][dt] = ld_fragC_q<E>(slotE(SQ), LK, 32 * kb, d0 + 16 * dt);
  // (the state operands come from memory on both sides of these products, so
  //  they use the contiguous k-slot order: one 16-byte LDS read per fragment,
  //  each loaded once and used for both key-column tiles)
  f32x4 gw[2][CTK], dq1[2][CTK], udh[2][CTK];
  Frag<E> hn[CTK][DV / 32], dhn[CTK][DV / 32];
#pragma unroll
  for (int dt = 0; dt < CTK; ++dt)
#pragma unroll
    for (int kb = 0; kb < DV / 32; ++kb) {
      hn[dt][kb] = finish_frag(hraw[dt][kb]);
      dhn[dt][kb] = finish_frag(dhraw[dt][kb]);
      // <h, dh'> over the whole state: the two row halves share each column group's part
      if ((kb & 1) == rh) hdh = frag_dot(hn[dt][kb], dhn[dt][kb], hdh);
    }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int rt = 2 * rh + j;
    f32x4 a[CTK], b[CTK], c[CTK];
#pragma unroll
    for (int dt = 0; dt < CTK; ++dt) a[dt] = b[dt] = c[dt] = zero4();
#pragma unroll
    for (int kb = 0; kb < DV / 32; ++kb) {
      const Frag<E> xdu = ld_frag8(sDU, LV, 16 * rt + c16, 32 * kb);
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
      const int dcol = d0 + 16 * dt + c16;
      // k at the lane's four rows of key column dcol: four consecutive entries of K^T
      const f32x4 kv4 = ld4f<E>(sKT + dcol * LT + 16 * rt + 4 * g);
      const f32x4 gm4 = *reinterpret_cast<const f32x4*>(&s.Gam[16 * rt + 4 * g]);
      const f32x4 ek4 = *reinterpret_cast<const f32x4*>(&s.ek[16 * rt + 4 * g]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float qv = frag_at(qown, 4 * j + i);
        rg[j][i] += scale * gm4[i] * qv * b[dt][i];
        re[j][i] += ek4[i] * kv4[i] * c[dt][i];
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) { pin(rg[j]); pin(rb[j]); pin(re[j]); }
  pin(hdh);
  __syncthreads();  // Q reads done: slot Q becomes GW
  {
    E* sGW = slotE(SQ);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int dt = 0; dt < CTK; ++dt) st_tile_rows<E>(sGW, LK, 16 * (2 * rh + j), d0 + 16 * dt, gw[j][dt]);
  }

  // ---- P7: GP = scale (dO U^T) * [i <= r]; GP*P row / column sums; P -> GP * M
  for (int ti = w; ti < 10; ti += 8) {
    int rt = 0;
    while ((rt + 1) * (rt + 2) / 2 <= ti) ++rt;
    const int ct = ti - rt * (rt + 1) / 2;
    f32x4 acc = zero4();
#pragma unroll
    for (int kb = 0; kb < DV / 32; ++kb)
      mma(acc, ld_frag(slotE(SDO), LV, 16 * rt + c16, 32 * kb), ld_frag(slotE(SV), LV, 16 * ct + c16, 32 * kb));
    const int c = 16 * ct + c16;
    f32x4 rs4;
    float csum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * rt + 4 * g + i;
      const float gp = (c <= r) ? scale * acc[i] : 0.f;
      // the diagonal entry enters row sum r and column sum r with opposite
      // signs: left out of both, it cannot leave a rounding residue in dgam_r
      // (which strong decay would make larger than dgam itself)
      const float gpp = (c < r) ? gp * sP[r * LA + c] : 0.f;
      rs4[i] = gpp;
      csum += gpp;
      sP[r * LA + c] = (c <= r) ? gp * __expf(s.gam[r] - s.gam[c]) : 0.f;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) rs4[i] = row16_sum(rs4[i]);
    csum += __shfl_xor(csum, 16, 64);
    csum += __shfl_xor(csum, 32, 64);
    if (c16 == 0) *reinterpret_cast<f32x4*>(&s.p7[ct][16 * rt + 4 * g]) = rs4;
    if (g == 0) s.c7[rt][c] = -csum;
  }
  __syncthreads();

  // V rows 16 cw .. 16 cw + 15, the operand of P9 (every tile of a wave there
  // has column tile cw; slot V holds U by then): read from global now so that
  // the loads are in flight during P8 (rows past the end are copies of the last
  // one; beta = 0 there removes them).  Contiguous k order, one 16-byte read
  // per fragment.
  Frag<E> vf[DV / 32];
  {
    const E* v = static_cast<const E*>(p.v) + (tok0 * H + h) * DV;
    const int vrow = min(16 * cw + c16, rows - 1);
#pragma unroll
    for (int kb = 0; kb < DV / 32; ++kb) vf[kb] = ld_frag8(v + (int64_t)vrow * H * DV, 0, 0, 32 * kb);
  }

  // ---- P8: XW = T^T GW (own rows); row dots; dK partial (with GPM^T Q); dQ
  f32x4 dkacc[2][CTK];
  {
    const E* sGW = slotE(SQ);
    // K is re-read here: an opaque pointer keeps the compiler from holding the
    // values read in P6 in registers (or scratch) until now
    const E* sKTr = lds_opaque(sKT);
#pragma unroll
    for (int dt = 0; dt < CTK; ++dt) {
      Frag<E> gwf[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) gwf[kb] = ld_fragC_q<E>(sGW, LK, 32 * kb, d0 + 16 * dt);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int rt = 2 * rh + j;
        f32x4 xw = zero4();
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) mma(xw, TT.row_e(16 * rt + c16, 32 * kb), gwf[kb]);
        const int dcol = d0 + 16 * dt + c16;
        f32x4 pq = zero4();  // GPM^T Q (GPM is final since P7)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) mma(pq, ld_fragT<E>(sP, LA, 16 * rt + c16, 32 * kb, 1.f), qr[kb][dt]);
        const f32x4 kv4 = ld4f<E>(sKTr + dcol * LT + 16 * rt + 4 * g);
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
  // dQ = scale diag(Gam) dQ1 + GPM K, final here (slot dO was last read in P7)
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
          mma(a, ld_frag_f32<E>(sP, LA, 16 * rt + c16, 32 * kb), ld_frag(sKT, LT, d0 + 16 * dt + c16, 32 * kb));
        const f32x4 gm4 = *reinterpret_cast<const f32x4*>(&s.Gam[16 * rt + 4 * g]);
        st_tile_rows<E>(sDQ, LK, 16 * rt, d0 + 16 * dt, dq1[j][dt] * gm4 * scale + a);
      }
  }
  __syncthreads();

  // ---- P9: GT = dU V^T diag(beta) + GW K^T diag(beta Gam) -> slot V (PMat).
  //          The dbeta term sum_c (T^T dU)[r][c] V[r][c] is the column sum
  //          sum_i T[i][r] (dU V^T)[i][r], taken here from the first product.
  const PMat<E> GTm(s.slot[SV]);
  {
    const int c = 16 * cw + c16;
    float tm = 0.f;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int rt = rh + 2 * j;
      f32x4 a = zero4(), b = zero4();
#pragma unroll
      for (int kb = 0; kb < DV / 32; ++kb) mma(a, ld_frag8(sDU, LV, 16 * rt + c16, 32 * kb), vf[kb]);
#pragma unroll
      for (int kb = 0; kb < DK / 32; ++kb)
        mma(b, ld_frag(slotE(SQ), LK, 16 * rt + c16, 32 * kb), ld_frag(sK, LK, c, 32 * kb));
      // U (slot V) is no longer read: every wave finished P7 before the barrier above
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rt + 4 * g + i;
        GTm.put(r, c, s.beta[c] * a[i] + s.bg[c] * b[i]);
        tm += TT.at(c, r) * a[i];
      }
    }
    tm += __shfl_xor(tm, 16, 64);
    tm += __shfl_xor(tm, 32, 64);
    if (g == 0) s.c9[rh][c] = tm;
  }
  __syncthreads();

  // ---- P10: Z = GT T^T (own row tiles, column tile cw) -> slot P (last read in
  //           P8), GA = strict_lower(-T^T Z) (own rows); E -> S = E + E^T (slot KD)
  // XU = T^T dU (own rows and value columns) -> dV into slot Q (GW was last read in P9)
  // The rows of T^T for this wave's row tiles serve XU (in E) and GA (near fp32).
  PFrag<E> ttp[2][2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      ttp[j][kb] = TT.row(16 * (2 * rh + j) + c16, 32 * kb);
  {
    E* sDV = slotE(SQ);
#pragma unroll
    for (int nt = 0; nt < CTV; ++nt) {
      Frag<E> duf[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) duf[kb] = ld_fragC_q<E>(sDU, LV, 32 * kb, n0 + 16 * nt);
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
      PFrag<E> tcol[2];  // rows 16 cw.. of T
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) tcol[kb] = TT.col(32 * kb, 16 * cw);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int rt = 2 * rh + j;
        f32x4 z = zero4();
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) mma(z, GTm.row(16 * rt + c16, 32 * kb), tcol[kb]);
        ZT.put4(16 * cw + c16, 16 * rt + 4 * g, z);
      }
    }
    __syncthreads();
    PFrag<E> zf[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) zf[kb] = ZT.row(16 * cw + c16, 32 * kb);
    const int c = 16 * cw + c16;
    float csum = 0.f;
    f32x4 ga[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int rt = 2 * rh + j;
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) mma(acc, ttp[j][kb], zf[kb]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rt + 4 * g + i;
        const float gav = (c < r) ? -acc[i] : 0.f;
        const float kd = sKD[r * LA + c];
        const float gaa = gav * s.beta[r] * kd;
        rg[j][i] += gaa;
        csum += gaa;
        rb[j][i] += gav * kd;
        ga[j][i] = gav;
      }
    }
    csum += __shfl_xor(csum, 16, 64);
    csum += __shfl_xor(csum, 32, 64);
    if (g == 0) s.c10[rh][c] = -csum;
    __syncthreads();  // every wave has read its KD entries: slot KD becomes S
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * (2 * rh + j) + 4 * g + i;
        if (c <= r) {
          const float ev = s.beta[r] * ga[j][i] * __expf(s.gam[r] - s.gam[c]);
          sKD[r * LA + c] = ev;
          if (c < r) sKD[c * LA + r] = ev;
        }
      }
  }
  __syncthreads();

  // ---- P11: dK = dK partial + S K (own rows and key columns) -> slot K
  //           (free since P9).  The three gradient tiles are written out after
  //           the last barrier, so that no load of this kernel waits behind a store.
  {
    E* sDK = slotE(SK);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int dt = 0; dt < CTK; ++dt) {
        const int rt = 2 * rh + j;
        f32x4 b = dkacc[j][dt];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          mma(b, ld_frag_f32<E>(sKD, LA, 16 * rt + c16, 32 * kb), ld_frag(sKT, LT, d0 + 16 * dt + c16, 32 * kb));
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
    // slot T is free since P10
    float* pe = reinterpret_cast<float*>(s.slot[ST]);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      f32x4 e = re[j];
#pragma unroll
      for (int i = 0; i < 4; ++i) e[i] = row16_sum(e[i]);
      if (c16 == 0) *reinterpret_cast<f32x4*>(&pe[cw * CH + 16 * (2 * rh + j) + 4 * g]) = e;
    }
    const float b = wave_sum(hdh);
    if (l == 0) s.ph[w] = b;
  }
  __syncthreads();
  store_tile<E, DV, NT>(slotE(SQ), LV, static_cast<E*>(p.dv) + (tok0 * H + h) * DV, (int64_t)H * DV, rows);
  if (PREP && p.prep.qk_norm) {
    // gradients with respect to the raw q and k (the kernel saw them normalised)
    store_tile_unnorm<E, DK, NT>(slotE(SDO), LK, static_cast<const E*>(p.q) + (tok0 * H + h) * DK, (int64_t)H * DK,
                                 static_cast<E*>(p.dq) + (tok0 * H + h) * DK, (int64_t)H * DK, rows);
    store_tile_unnorm<E, DK, NT>(slotE(SK), LK, static_cast<const E*>(p.k) + (tok0 * H + h) * DK, (int64_t)H * DK,
                                 static_cast<E*>(p.dk) + (tok0 * H + h) * DK, (int64_t)H * DK, rows);
  } else {
    store_tile<E, DK, NT>(slotE(SDO), LK, static_cast<E*>(p.dq) + (tok0 * H + h) * DK, (int64_t)H * DK, rows);
    store_tile<E, DK, NT>(slotE(SK), LK, static_cast<E*>(p.dk) + (tok0 * H + h) * DK, (int64_t)H * DK, rows);
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
      for (int ww = 0; ww < 8; ++ww) extra += s.GamC * s.ph[ww];
      dgm += extra;
    }
    const float* pe = reinterpret_cast<const float*>(s.slot[ST]);
    float e = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) e += pe[ww * CH + r];
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
}

template <class E, int DK, int DV>
hipError_t launch_grad_t(const GradParams& p, int nchunk_total, hipStream_t st) {
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
