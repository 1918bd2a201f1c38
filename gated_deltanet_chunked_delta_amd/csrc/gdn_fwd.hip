// gdn_fwd.hip -- forward chunk loop of the gated delta rule on gfx950.
//
// One workgroup owns one (segment, head): a run of consecutive 64-token chunks
// of one sequence.  Wave w of the workgroup keeps columns [16w, 16w+16) of the
// fp32 state h = S^T (Dk x Dv) in accumulator registers for the whole run, so
// the serial chain U = Ut - W h, h' = Gam_C h + Kt^T U never leaves registers.
// Everything that does not depend on h (decay cumsum, the decay-masked K K^T,
// the unit-lower-triangular solve, W and Ut, the masked Q K^T) is computed
// per chunk from LDS tiles by all waves together.
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
// into segments.  Phase 1 runs every segment from a zero state (segment 0 from
// h0), writing provisional outputs, the segment's end state b_s and
// Lambda_s = sum over its tokens of g_t + log max(1, |1 - beta_t |k_t|^2|),
// a bound on log ||transition||_2 since ||I - beta k k^T||_2 = max(1, |1 - beta |k|^2|).
// Phase 3 adds, for each segment s >= 1, the effect of the true incoming state
// H_s = b_{s-1}: delta <- H_s, and per chunk  o += scale (diag(Gam) Q delta - P W delta),
// delta <- Gam_C delta - K^T diag(ek) W delta, until the accumulated bound
// exp(sum Lambda) drops under 2^-24 (fp32 round-off), which the gate decay
// makes happen after a few chunks.  H_s = b_{s-1} is exact to that bound only
// if every interior segment decays below it; a workgroup checks that from the
// Lambda_s values and otherwise the (sequence, head) is recomputed serially.
#include "gdn_device.h"
#include "gdn_internal.h"
#include "gdn_tiles.h"

namespace gdn {

template <class E, int DK, int DV>
struct alignas(16) FwdSmem {
  static constexpr int LQ = ldpad<E>(DK);  // sQ, sK, sW row stride
  static constexpr int LT = ldpad<E>(CH);  // transposed tiles and 64x64 E matrices
  static constexpr int LA = CH + 4;        // fp32 64x64 matrices
  static constexpr int LO = ldpad<E>(DV);  // output staging
  static constexpr int A_BYTES = CH * LA * 4;
  static constexpr int O_BYTES = CH * LO * (int)sizeof(E);
  E Q[CH * LQ];
  E K[CH * LQ];
  E KT[DK * LT];
  E VT[DV * LT];
  E W[CH * LQ];   // holds -W
  E P[CH * LT];
  float T[CH * LA];
  union {
    float A[CH * LA];
    E O[(O_BYTES > A_BYTES ? O_BYTES : A_BYTES) / sizeof(E)];
  };
  alignas(16) float gam[CH], Gam[CH], ek[CH], beta[CH], bg[CH], graw[CH], lam[CH];
  float GamC;
};

// ------------------------------------------------------------------ one chunk

enum : int { M_WRITE_O = 1, M_STORE_H = 2, M_CORR = 4 };

template <class E, int DK, int DV>
struct FwdCtx {
  static constexpr int NW = DV / 16;
  static constexpr int NT = NW * 64;
  static constexpr int KT_ = DK / 16;  // state row tiles per wave
  using S = FwdSmem<E, DK, DV>;
};

// Process one chunk.  hacc: this wave's state columns (state at chunk start on
// entry, at chunk end on exit).  Returns the chunk's log-bound Lambda_c.
template <class E, int DK, int DV>
__device__ float chunk_step(FwdSmem<E, DK, DV>& s, const FwdParams& p, int64_t tok0, int rows,
                            int h, int mode, E* hs_chunk, f32x4 (&hacc)[DK / 16]) {
  using C = FwdCtx<E, DK, DV>;
  using Sm = FwdSmem<E, DK, DV>;
  constexpr int NW = C::NW, NT = C::NT;
  constexpr int LQ = Sm::LQ, LT = Sm::LT, LA = Sm::LA, LO = Sm::LO;
  const int tid = threadIdx.x, l = lane_id(), w = wave_id(), g = l >> 4, c16 = l & 15;
  const bool corr = mode & M_CORR;
  const bool need_q = mode & M_WRITE_O;
  const bool need_v = !corr;
  const int H = p.H;

  // ---- 0. per-chunk start state out (backward replay)
  if (hs_chunk) {
#pragma unroll
    for (int t = 0; t < DK / 16; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        E* dst = hs_chunk + (16 * t + 4 * g + i) * DV + 16 * w + c16;
        float val = hacc[t][i];
        if (corr) val += to_f(*dst);
        *dst = to_e<E>(val);
      }
  }

  // ---- 1. staging
  {
    const E* q = static_cast<const E*>(p.q) + (tok0 * H + h) * DK;
    const E* k = static_cast<const E*>(p.k) + (tok0 * H + h) * DK;
    const E* v = static_cast<const E*>(p.v) + (tok0 * H + h) * DV;
    stage_tile<E, DK, NT>(k, (int64_t)H * DK, rows, s.K, LQ, s.KT, LT);
    if (need_q) stage_tile<E, DK, NT>(q, (int64_t)H * DK, rows, s.Q, LQ, nullptr, 0);
    if (need_v) stage_tile<E, DV, NT>(v, (int64_t)H * DV, rows, nullptr, 0, s.VT, LT);
    if (w == 0) {
      const bool valid = l < rows;
      const int64_t si = (tok0 + l) * H + h;
      float gr = valid ? p.g[si] : 0.f;
      float bt = valid ? to_f(static_cast<const E*>(p.beta)[si]) : 0.f;
      float gm = wave_incl_scan(gr);
      float gC = __shfl(gm, 63, 64);
      float Gm = __expf(gm);
      s.gam[l] = gm;
      s.Gam[l] = Gm;
      s.ek[l] = __expf(gC - gm);
      s.beta[l] = bt;
      s.bg[l] = bt * Gm;
      s.graw[l] = gr;
      if (l == 0) s.GamC = __expf(gC);
    }
  }
  __syncthreads();

  // ---- 2. K K^T (lower tiles) -> A, lambda
  for (int ti = w; ti < 10; ti += NW) {
    int rt = 0;
    while ((rt + 1) * (rt + 2) / 2 <= ti) ++rt;
    const int ct = ti - rt * (rt + 1) / 2;
    f32x4 acc = zero4();
#pragma unroll
    for (int kb = 0; kb < DK / 32; ++kb)
      mma(acc, ld_frag(s.K, LQ, 16 * rt + c16, 32 * kb), ld_frag(s.K, LQ, 16 * ct + c16, 32 * kb));
    const int c = 16 * ct + c16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * rt + 4 * g + i;
      float val = (c < r) ? s.beta[r] * acc[i] * __expf(s.gam[r] - s.gam[c]) : 0.f;
      s.A[r * LA + c] = val;
      if (r == c) s.lam[r] = s.graw[r] + __logf(fmaxf(1.f, fabsf(1.f - s.beta[r] * acc[i])));
    }
  }
  __syncthreads();
  // lane 0's sum: every wave reduces the same values in the same order, so the
  // value (and the loop decisions taken on it) is identical across the workgroup
  const float lam_c = __shfl(wave_sum(s.lam[l]), 0, 64);

  // ---- 3a. diagonal solve (wave 0) || Q K^T -> P and Q h (other waves)
  f32x4 qh[4];
  if (w == 0) solve_diag(s.A, s.T);
  if (need_q) {
    const int nw = NW > 1 ? NW - 1 : 1, w0 = NW > 1 ? w - 1 : w;
    if (w0 >= 0) {
      for (int ti = w0; ti < 10; ti += nw) {
        int rt = 0;
        while ((rt + 1) * (rt + 2) / 2 <= ti) ++rt;
        const int ct = ti - rt * (rt + 1) / 2;
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb)
          mma(acc, ld_frag(s.Q, LQ, 16 * rt + c16, 32 * kb), ld_frag(s.K, LQ, 16 * ct + c16, 32 * kb));
        const int c = 16 * ct + c16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * rt + 4 * g + i;
          float val = (c <= r) ? acc[i] * __expf(s.gam[r] - s.gam[c]) : 0.f;
          s.P[r * LT + c] = to_e<E>(val);
        }
      }
    }
    // Q h for this wave's columns
    Frag<E> hf[DK / 32];
#pragma unroll
    for (int kb = 0; kb < DK / 32; ++kb) pack_frag(hf[kb], hacc[2 * kb], hacc[2 * kb + 1]);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      qh[rt] = zero4();
#pragma unroll
      for (int kb = 0; kb < DK / 32; ++kb) mma(qh[rt], ld_frag(s.Q, LQ, 16 * rt + c16, 32 * kb), hf[kb]);
    }
  }
  __syncthreads();

  // ---- 3b. off-diagonal solve levels
  if (w < 3) solve_offdiag(s.A, s.T, w + 1, w);
  __syncthreads();
  if (w < 2) solve_offdiag(s.A, s.T, w + 2, w);
  __syncthreads();
  if (w == 0) solve_offdiag(s.A, s.T, 3, 0);
  __syncthreads();

  // ---- 5. -W = -T diag(beta Gam) K  (all waves) ; Ut = T diag(beta) V (own columns)
  for (int ti = w; ti < 4 * (DK / 16); ti += NW) {
    const int rt = ti / (DK / 16), ct = ti % (DK / 16);
    f32x4 acc = zero4();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      mma(acc, ld_frag_scaled<E>(s.T, LA, 16 * rt + c16, 32 * kb, s.bg), ld_frag(s.KT, LT, 16 * ct + c16, 32 * kb));
#pragma unroll
    for (int i = 0; i < 4; ++i) s.W[(16 * rt + 4 * g + i) * LQ + 16 * ct + c16] = to_e<E>(-acc[i]);
  }
  f32x4 u[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    u[rt] = zero4();
    if (need_v) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        mma(u[rt], ld_frag_scaled<E>(s.T, LA, 16 * rt + c16, 32 * kb, s.beta), ld_frag(s.VT, LT, 16 * w + c16, 32 * kb));
    }
  }
  __syncthreads();

  // ---- 6. state chain: U = Ut - W h ; O ; h' = GamC h + K^T (ek * U)
  {
    Frag<E> hf[DK / 32];
#pragma unroll
    for (int kb = 0; kb < DK / 32; ++kb) pack_frag(hf[kb], hacc[2 * kb], hacc[2 * kb + 1]);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int kb = 0; kb < DK / 32; ++kb) mma(u[rt], ld_frag(s.W, LQ, 16 * rt + c16, 32 * kb), hf[kb]);
  }
  if (need_q) {
    Frag<E> uf[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) pack_frag(uf[kb], u[2 * kb], u[2 * kb + 1]);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      f32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = qh[rt][i] * s.Gam[16 * rt + 4 * g + i];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) mma(o, ld_frag(s.P, LT, 16 * rt + c16, 32 * kb), uf[kb]);
      o = o * p.scale;
      if (!corr) {
#pragma unroll
        for (int i = 0; i < 4; ++i) s.O[(16 * rt + 4 * g + i) * LO + 16 * w + c16] = to_e<E>(o[i]);
      } else if (mode & M_WRITE_O) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * rt + 4 * g + i;
          if (r < rows) {
            E* dst = static_cast<E*>(p.o) + ((tok0 + r) * H + h) * DV + 16 * w + c16;
            *dst = to_e<E>(to_f(*dst) + o[i]);
          }
        }
      }
    }
  }
  {
    const float gc = s.GamC;
    Frag<E> us[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x4 e0, e1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        e0[i] = s.ek[32 * kb + 4 * g + i];
        e1[i] = s.ek[32 * kb + 16 + 4 * g + i];
      }
      pack_frag_scaled(us[kb], u[2 * kb], u[2 * kb + 1], e0, e1);
    }
#pragma unroll
    for (int t = 0; t < DK / 16; ++t) {
      hacc[t] = hacc[t] * gc;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) mma(hacc[t], ld_frag(s.KT, LT, 16 * t + c16, 32 * kb), us[kb]);
    }
  }
  __syncthreads();

  // ---- 7. output tile out (coalesced)
  if ((mode & M_WRITE_O) && !corr) {
    constexpr int VEC = 16 / sizeof(E);
    typedef E vec_t __attribute__((__vector_size__(16)));
    for (int e = tid; e < CH * (DV / VEC); e += NT) {
      const int r = e / (DV / VEC), c0 = (e % (DV / VEC)) * VEC;
      if (r < rows) {
        vec_t x;
#pragma unroll
        for (int j = 0; j < VEC; ++j) x[j] = s.O[r * LO + c0 + j];
        *reinterpret_cast<vec_t*>(static_cast<E*>(p.o) + ((tok0 + r) * H + h) * DV + c0) = x;
      }
    }
  }
  return lam_c;
}

template <class E, int DK, int DV>
__device__ void load_state(f32x4 (&hacc)[DK / 16], const float* src) {
  const int l = lane_id(), w = wave_id(), g = l >> 4, c16 = l & 15;
#pragma unroll
  for (int t = 0; t < DK / 16; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) hacc[t][i] = src ? src[(16 * t + 4 * g + i) * DV + 16 * w + c16] : 0.f;
}
template <class E, int DK, int DV>
__device__ void store_state(const f32x4 (&hacc)[DK / 16], float* dst, const float* add) {
  const int l = lane_id(), w = wave_id(), g = l >> 4, c16 = l & 15;
#pragma unroll
  for (int t = 0; t < DK / 16; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = (16 * t + 4 * g + i) * DV + 16 * w + c16;
      dst[e] = hacc[t][i] + (add ? add[e] : 0.f);
    }
}

template <class E, int DK, int DV>
__device__ void init_smem(FwdSmem<E, DK, DV>& s) {
  using Sm = FwdSmem<E, DK, DV>;
  // Upper-triangular parts of P and T are never written by the chunk loop and
  // must read as zero.
  for (int e = threadIdx.x; e < CH * CH; e += blockDim.x) {
    const int r = e >> 6, c = e & 63;
    s.P[r * Sm::LT + c] = to_e<E>(0.f);
    s.T[r * Sm::LA + c] = 0.f;
  }
  __syncthreads();
}

template <class E, int DK, int DV>
__global__ __launch_bounds__(DV / 16 * 64) void gdn_fwd_kernel(FwdParams p) {
  __shared__ FwdSmem<E, DK, DV> s;
  const SegDesc sd = p.segs[blockIdx.x];
  const int h = blockIdx.y;
  const int n = sd.n;
  const int seg0 = p.seg_first[n];
  const int nseg = p.seg_first[n + 1] - seg0;
  const int64_t seq0 = p.seq.start(n);
  const int len = p.seq.len(n);
  const size_t SS = (size_t)DK * DV;
  const int64_t chunk0 = p.chunk_first[n];
  E* hs = static_cast<E*>(p.hs);
  const int base_mode = (p.o ? M_WRITE_O : 0) | (hs ? M_STORE_H : 0);
  f32x4 hacc[DK / 16];

  auto run = [&](int cb, int ce, int mode) {
    for (int c = cb; c < ce; ++c) {
      const int64_t tok0 = seq0 + (int64_t)c * CH;
      const int rows = min(CH, len - c * CH);
      E* hsc = hs ? hs + ((chunk0 + c) * p.H + h) * SS : nullptr;
      chunk_step<E, DK, DV>(s, p, tok0, rows, h, mode, hsc, hacc);
    }
  };

  if (p.phase == 1) {
    init_smem(s);
    load_state<E, DK, DV>(hacc, (sd.s == 0 && p.h0) ? p.h0 + ((size_t)n * p.H + h) * SS : nullptr);
    float lam = 0.f;
    for (int c = sd.c_begin; c < sd.c_end; ++c) {
      const int64_t tok0 = seq0 + (int64_t)c * CH;
      const int rows = min(CH, len - c * CH);
      E* hsc = hs ? hs + ((chunk0 + c) * p.H + h) * SS : nullptr;
      lam += chunk_step<E, DK, DV>(s, p, tok0, rows, h, base_mode, hsc, hacc);
    }
    if (nseg == 1) {
      if (p.hT) store_state<E, DK, DV>(hacc, p.hT + ((size_t)n * p.H + h) * SS, nullptr);
    } else {
      store_state<E, DK, DV>(hacc, p.bstate + ((size_t)blockIdx.x * p.H + h) * SS, nullptr);
      if (threadIdx.x == 0) p.lam[(size_t)blockIdx.x * p.H + h] = lam;
    }
    return;
  }

  // ---- phase 3: boundary corrections
  if (nseg == 1 || sd.s == 0) return;
  bool ok = true;
  for (int j = 1; j + 1 < nseg; ++j) ok = ok && (p.lam[(size_t)(seg0 + j) * p.H + h] <= LN_EPS);
  init_smem(s);
  if (!ok) {
    // Gates do not decay fast enough to cut this sequence: one workgroup redoes it serially.
    if (sd.s != 1) return;
    load_state<E, DK, DV>(hacc, p.h0 ? p.h0 + ((size_t)n * p.H + h) * SS : nullptr);
    const int nch = (len + CH - 1) / CH;
    run(0, nch, base_mode);
    if (p.hT) store_state<E, DK, DV>(hacc, p.hT + ((size_t)n * p.H + h) * SS, nullptr);
    return;
  }
  load_state<E, DK, DV>(hacc, p.bstate + ((size_t)(blockIdx.x - 1) * p.H + h) * SS);
  float cum = 0.f;
  int c = sd.c_begin;
  for (; c < sd.c_end && cum > LN_EPS; ++c) {
    const int64_t tok0 = seq0 + (int64_t)c * CH;
    const int rows = min(CH, len - c * CH);
    E* hsc = hs ? hs + ((chunk0 + c) * p.H + h) * SS : nullptr;
    cum += chunk_step<E, DK, DV>(s, p, tok0, rows, h, base_mode | M_CORR, hsc, hacc);
  }
  if (sd.s == nseg - 1 && p.hT) {
    // hT = b_last + (the correction propagated through the whole last segment, if it got there)
    const float* b = p.bstate + ((size_t)blockIdx.x * p.H + h) * SS;
    if (c == sd.c_end) store_state<E, DK, DV>(hacc, p.hT + ((size_t)n * p.H + h) * SS, b);
    else {
      f32x4 z[DK / 16];
      for (int t = 0; t < DK / 16; ++t) z[t] = zero4();
      store_state<E, DK, DV>(z, p.hT + ((size_t)n * p.H + h) * SS, b);
    }
  }
}

template <class E, int DK, int DV>
hipError_t launch_fwd_t(const FwdParams& p, int nseg_total, hipStream_t st) {
  dim3 grid(nseg_total, p.H), block(DV / 16 * 64);
  hipLaunchKernelGGL((gdn_fwd_kernel<E, DK, DV>), grid, block, 0, st, p);
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
