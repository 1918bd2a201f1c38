// gdn_decode.hip -- one recurrent decode step of the gated delta rule on gfx950.
//
// After a prefill, each new token of a sequence advances the state by one step
// of the recurrence ("Qwen's FlashQLA targets the expensive bit of long-context
// AI", section "What happened", and "FlashQLA resource", section 4: the kernels
// serve training and inference).  With h = S^T (Dk x Dv) the step is
//     p = h^T k,   u = beta (v - e^g p),   h' = e^g h + k u^T,   o = scale h'^T q,
// the same algebra as S' = e^g S (I - beta k k^T) + beta v k^T, o = scale S' q.
// With the optional pre-processing, q and k are first divided by their L2
// norms and g, beta are formed from logits (as in the chunk kernels).
//
// Every column j of h evolves independently given (q, k, v_j, g, beta): a
// workgroup owns a 32-column slice of one (sequence, head) state.  Its 256
// threads hold 4 consecutive columns of DK/32 rows each (16-byte loads, each
// row of the slice read as one 128-byte segment), the two column sums p and o
// are reduced over the row groups through LDS, and the updated slice is
// written back in place.  The step is bound by HBM: the fp32 state is read and
// written once (2 Dk Dv 4 bytes per sequence and head), with non-temporal
// accesses since nothing reuses it within the step.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int DEC_COLS = 32;  // state columns per workgroup
constexpr int DEC_NT = 256;   // threads: 8 column quads x 32 row groups

template <class E>
__device__ __forceinline__ float ld1(const void* p, int64_t i) {
  return to_f(static_cast<const E*>(p)[i]);
}

template <class E, int DK, int DV>
__global__ __launch_bounds__(DEC_NT) void gdn_decode_kernel(DecodeParams p) {
  constexpr int RPT = DK / 32;  // rows per thread
  __shared__ float red[32][DEC_COLS + 1];
  __shared__ float uj[DEC_COLS];
  const int tid = threadIdx.x, tc = tid & 7, tr = tid >> 3;
  const int nh = blockIdx.x, n = nh / p.H, h = nh - n * p.H;
  const int slot = p.state_idx ? p.state_idx[n] : n;
  if (slot < 0 || slot >= p.num_slots) return;  // padding entry (uniform per workgroup)
  const int c0 = blockIdx.y * DEC_COLS + 4 * tc;  // this thread's first state column
  float* hs = p.state + ((int64_t)slot * p.H + h) * DK * DV;
  const int64_t qk = (int64_t)nh * DK;

  float gl = p.g[nh], bt = ld1<E>(p.beta, nh);
  if (p.prep.gate_act) {
    gl = -(p.prep.gate_scale ? p.prep.gate_scale[h] : 1.f) * softplus_f(gl);
    bt = sigmoid_f(bt);
  }
  const float a = __expf(gl);
  // optional L2 normalisation of q and k: wave 0 forms both norms
  __shared__ float inv_norm[2];
  if (p.prep.qk_norm) {
    if (tid < 64) {
      float sk = 0.f, sq = 0.f;
#pragma unroll
      for (int i = tid; i < DK; i += 64) {
        const float kk = ld1<E>(p.k, qk + i), qq = ld1<E>(p.q, qk + i);
        sk += kk * kk;
        sq += qq * qq;
      }
      sk = wave_sum(sk);
      sq = wave_sum(sq);
      if (tid == 0) {
        inv_norm[0] = rsqrtf(sk + QK_NORM_EPS);
        inv_norm[1] = rsqrtf(sq + QK_NORM_EPS);
      }
    }
    __syncthreads();
  }

  // own rows of the slice and the matching k, q entries
  f32x4 hv[RPT];
  float kv[RPT], qv[RPT];
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int i = tr + 32 * m;
    hv[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(hs + (int64_t)i * DV + c0));
    kv[m] = ld1<E>(p.k, qk + i);
    qv[m] = ld1<E>(p.q, qk + i);
  }

  if (p.prep.qk_norm) {
    const float ik = inv_norm[0], iq = inv_norm[1];
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
      kv[m] *= ik;
      qv[m] *= iq;
    }
  }

  // p_j = sum_i h_ij k_i over this thread's rows, then over the 32 row groups
  f32x4 part = zero4();
#pragma unroll
  for (int m = 0; m < RPT; ++m) part = part + hv[m] * kv[m];
#pragma unroll
  for (int e = 0; e < 4; ++e) red[tr][4 * tc + e] = part[e];
  __syncthreads();
  if (tid < DEC_COLS) {
    float s = 0.f;
#pragma unroll 8
    for (int r = 0; r < 32; ++r) s += red[r][tid];
    const int j = blockIdx.y * DEC_COLS + tid;
    uj[tid] = bt * (ld1<E>(p.v, (int64_t)nh * DV + j) - a * s);
  }
  __syncthreads();

  // h' = e^g h + k u^T (written back), o_j = scale sum_i h'_ij q_i
  const f32x4 u4 = *reinterpret_cast<const f32x4*>(&uj[4 * tc]);
  part = zero4();
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int i = tr + 32 * m;
    const f32x4 hn = hv[m] * a + u4 * kv[m];
    __builtin_nontemporal_store(hn, reinterpret_cast<f32x4*>(hs + (int64_t)i * DV + c0));
    part = part + hn * qv[m];
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) red[tr][4 * tc + e] = part[e];
  __syncthreads();
  if (tid < DEC_COLS) {
    float s = 0.f;
#pragma unroll 8
    for (int r = 0; r < 32; ++r) s += red[r][tid];
    const int j = blockIdx.y * DEC_COLS + tid;
    static_cast<E*>(p.o)[(int64_t)nh * DV + j] = to_e<E>(p.scale * s);
  }
}

template <class E, int DK, int DV>
hipError_t launch_decode_t(const DecodeParams& p, hipStream_t st) {
  hipLaunchKernelGGL((gdn_decode_kernel<E, DK, DV>), dim3(p.N * p.H, DV / DEC_COLS), dim3(DEC_NT), 0, st, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(int dtype, int DK, int DV, const DecodeParams& p, hipStream_t st) {
  if (p.N * p.H == 0) return hipSuccess;
  if (dtype == 1) {
    if (DK == 128 && DV == 128) return launch_decode_t<bf16, 128, 128>(p, st);
    if (DK == 64 && DV == 64) return launch_decode_t<bf16, 64, 64>(p, st);
    if (DK == 64 && DV == 128) return launch_decode_t<bf16, 64, 128>(p, st);
    if (DK == 128 && DV == 64) return launch_decode_t<bf16, 128, 64>(p, st);
  } else {
    if (DK == 128 && DV == 128) return launch_decode_t<float, 128, 128>(p, st);
    if (DK == 64 && DV == 64) return launch_decode_t<float, 64, 64>(p, st);
    if (DK == 64 && DV == 128) return launch_decode_t<float, 64, 128>(p, st);
    if (DK == 128 && DV == 64) return launch_decode_t<float, 128, 64>(p, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
