// gdn_tsolve.hip -- every chunk's T = (I + diag(beta) A)^-1, A = strict_lower(K K^T * D),
// solved for all chunks at once.
//
// T is the UT-transform matrix of the chunked form (the per-chunk "in-LDS
// solve" of the forward and backward kernels the "FlashQLA resource" page
// describes in section 3).  It depends on the chunk's k, g and beta only, not on
// the state, so it is formed here, chunk-parallel, before the serial chunk
// chains; they and the gradient kernel read it back instead
// of solving on their critical path.
//
// One workgroup of three waves per (chunk, head) -- the column solve has three
// block columns, the diagonal solve two pairs of blocks -- and 35 KiB of LDS
// (T takes the place of K once K K^T is formed), so four workgroups share a
// compute unit and one's solve overlaps another's loads.
// Rows past a sequence end are zero in K and carry beta = 0, so their rows and
// columns of T are those of the identity.  Beside T it writes the chunk's
// scalar record (decay cumsum and exponentials, beta, the log-bound; layout in
// gdn_internal.h), which the chunk chains and the gradient kernel read instead
// of g and beta.
#include "gdn_internal.h"
#include "gdn_tiles.h"

namespace gdn {
namespace {

template <class E, int DK>
struct TSolveSmem {
  static constexpr int LK = DK + 16 / (int)sizeof(E);  // row-major [64][DK] E
  static constexpr int LA = CH + 4;                    // fp32 [64][64]
  static constexpr int KB = CH * LK * (int)sizeof(E), TB = CH * LA * 4;
  alignas(16) char kt[KB > TB ? KB : TB];  // K, then T
  alignas(16) float KD[CH * LA];
  float gam[CH], beta[CH], graw[CH], kk[CH];  // kk: |k_r|^2
  __device__ E* K() { return reinterpret_cast<E*>(kt); }
  __device__ float* T() { return reinterpret_cast<float*>(kt); }
};

template <class E, int DK, bool PREP>
__global__ __launch_bounds__(192) void gdn_tsolve(TSolveParams p) {
  constexpr int NT = 192;
  using S = TSolveSmem<E, DK>;
  constexpr int LK = S::LK, LA = S::LA;
  __shared__ S s;
  const int tid = threadIdx.x, l = lane_id(), w = wave_id(), g = l >> 4, c16 = l & 15;
  const int2 ct = p.seq.chunk_of(p.chunk_tab, blockIdx.x);
  if (ct.x < 0) return;  // the plan found the device cu_seqlens inconsistent
  const int n = ct.x, h = blockIdx.y, H = p.H;
  const int64_t tok0 = p.seq.start(n) + (int64_t)ct.y * CH;
  const int rows = min(CH, p.seq.len(n) - ct.y * CH);

  TilePart<E, NT, DK> tk;
  tk.template load<true>(static_cast<const E*>(p.k) + (tok0 * H + h) * DK, (int64_t)H * DK, rows, tid);
  if (w == 0) {
    const bool valid = l < rows;
    const int64_t si = (tok0 + l) * H + h;
    float gr = valid ? p.g[si] : 0.f;
    float bt = valid ? to_f(static_cast<const E*>(p.beta)[si]) : 0.f;
    if (PREP && p.prep.gate_act && valid) {
      gr = -(p.prep.gate_scale ? p.prep.gate_scale[h] : 1.f) * softplus_f(gr);
      bt = sigmoid_f(bt);
    }
    s.gam[l] = wave_incl_scan(gr);
    s.beta[l] = bt;
    s.graw[l] = gr;
  }
  if (PREP && p.prep.qk_norm) tk.normalize_rows(tid);
  tk.store(s.K(), LK, nullptr, 0, tid);
  __syncthreads();

  // KD = strict_lower(K K^T * D): the ten lower 16x16 tiles, tile t = w + 3j
  // for wave w (row tile r, column tile t - r(r+1)/2); every fragment read of a
  // wave is issued before its products
  {
    constexpr int NJ = 4;
    f32x4 acc[NJ];
    Frag<E> xr[NJ][DK / 32], xc[NJ][DK / 32];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int ti = w + 3 * j;
      const int rt = ti < 1 ? 0 : (ti < 3 ? 1 : (ti < 6 ? 2 : 3)), ctl = ti - rt * (rt + 1) / 2;
      if (ti < 10) {
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb) {
          xr[j][kb] = ld_frag(s.K(), LK, 16 * rt + c16, 32 * kb);
          xc[j][kb] = ld_frag(s.K(), LK, 16 * ctl + c16, 32 * kb);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      acc[j] = zero4();
      if (w + 3 * j < 10) {
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb) mma(acc[j], xr[j][kb], xc[j][kb]);
      }
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int ti = w + 3 * j;
      const int rt = ti < 1 ? 0 : (ti < 3 ? 1 : (ti < 6 ? 2 : 3)), ctl = ti - rt * (rt + 1) / 2;
      if (ti < 10) {
        const int c = 16 * ctl + c16;
        const float gc = s.gam[c];
        const f32x4 gr4 = *reinterpret_cast<const f32x4*>(&s.gam[16 * rt + 4 * g]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * rt + 4 * g + i;
          s.KD[r * LA + c] = (c < r) ? acc[j][i] * __expf(gr4[i] - gc) : 0.f;
        }
        if (rt == ctl) {  // a diagonal tile (wave-uniform): |k_r|^2, for the log-bound
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (16 * rt + 4 * g + i == c) s.kk[c] = acc[j][i];
        }
      }
    }
  }
  __syncthreads();
  // K is dead: its space becomes T, whose six blocks above the diagonal are
  // zero; the diagonal blocks (two per wave), then one block column per wave
  float* sT = s.T();
  for (int e = tid; e < 6 * 64; e += NT) {
    const int blk = e >> 6, q = e & 63;  // block (I, J), I < J, in order (0,1) (0,2) (0,3) (1,2) (1,3) (2,3)
    const int I = blk < 3 ? 0 : (blk < 5 ? 1 : 2), J = blk < 3 ? blk + 1 : (blk < 5 ? blk - 1 : 3);
    *reinterpret_cast<f32x4*>(&sT[(16 * I + (q >> 2)) * LA + 16 * J + 4 * (q & 3)]) = zero4();
  }
  if (w < 2) {
    solve_diag_pair(s.KD, sT, w, 3 - w, s.beta);
  } else {
    // the scalar record, while waves 0 and 1 solve
    float* rec = p.rec_out + ((size_t)blockIdx.x * H + h) * RECF;
    const float gm = s.gam[l], gC = s.gam[CH - 1], bt = s.beta[l];
    const float Gm = __expf(gm);
    rec[l] = gm;
    rec[CH + l] = Gm;
    rec[2 * CH + l] = __expf(gC - gm);
    rec[3 * CH + l] = bt;
    rec[4 * CH + l] = bt * Gm;
    const float lam = __shfl(wave_sum(s.graw[l] + __logf(fmaxf(1.f, fabsf(1.f - bt * s.kk[l])))), 0, 64);
    if (l < 4) rec[5 * CH + l] = l == 0 ? lam : (l == 1 ? __expf(gC) : 0.f);
  }
  __syncthreads();
  solve_columns(s.KD, sT, w, s.beta);
  __syncthreads();
  // out as fp32 (fp32 inputs) or as its bf16 value and residual planes
  float* dst = p.t_out + ((size_t)blockIdx.x * H + h) * (CH * CH);
  for (int e = 4 * tid; e < CH * CH; e += 4 * NT) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(&sT[(e >> 6) * LA + (e & 63)]);
    if constexpr (std::is_same<E, bf16>::value) {
      bf16x4 hi, lo;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hi[i] = (bf16)x[i];
        lo[i] = (bf16)(x[i] - (float)hi[i]);
      }
      st_out(reinterpret_cast<bf16x4*>(reinterpret_cast<bf16*>(dst) + e), hi);
      st_out(reinterpret_cast<bf16x4*>(reinterpret_cast<bf16*>(dst) + CH * CH + e), lo);
    } else {
      st_out(reinterpret_cast<f32x4*>(dst + e), x);
    }
  }
}

template <class E, int DK>
hipError_t launch_tsolve_t(const TSolveParams& p, int nchunk_total, hipStream_t st) {
  const dim3 grid(nchunk_total, p.H), block(192);
  if (p.prep.qk_norm || p.prep.gate_act) hipLaunchKernelGGL((gdn_tsolve<E, DK, true>), grid, block, 0, st, p);
  else hipLaunchKernelGGL((gdn_tsolve<E, DK, false>), grid, block, 0, st, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tsolve(int dtype, int DK, const TSolveParams& p, int nchunk_total, hipStream_t st) {
  if (nchunk_total <= 0) return hipSuccess;
  if (dtype == 1) {
    if (DK == 128) return launch_tsolve_t<bf16, 128>(p, nchunk_total, st);
    if (DK == 64) return launch_tsolve_t<bf16, 64>(p, nchunk_total, st);
  } else {
    if (DK == 64) return launch_tsolve_t<float, 64>(p, nchunk_total, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
