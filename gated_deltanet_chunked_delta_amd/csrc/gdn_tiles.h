// gdn_tiles.h -- LDS tile helpers shared by the forward and backward kernels:
// the 64x64 unit-lower-triangular solve and global->LDS tile staging.
#pragma once
#include "gdn_device.h"

namespace gdn {

// ------------------------------------------------------------------ helpers

// 16x16x16 fp32 product  acc += X[xr0.., xk0..] * Y  where Y's k rows are the
// C-layout rows 4g+i held in yreg[i].  X is fp32 row-major in LDS.
__device__ __forceinline__ void mm16_xreg(f32x4& acc, const float* X, int ldx, int xr0, int xk0,
                                          const f32x4& yreg) {
  const int l = lane_id(), g = l >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float a = X[(xr0 + (l & 15)) * ldx + xk0 + 4 * g + i];
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, yreg[i], acc, 0, 0, 0);
  }
}
// acc += diag(rs) X[xr0.., xk0..] * Y[yk0.., yc0..], both fp32 row-major in LDS
// (16x16x16); rs (a row scale of X) may be null.
__device__ __forceinline__ void mm16_xy(f32x4& acc, const float* X, int ldx, int xr0, int xk0,
                                        const float* Y, int ldy, int yk0, int yc0,
                                        const float* rs = nullptr) {
  const int l = lane_id(), g = l >> 4;
  const float sc = rs ? rs[xr0 + (l & 15)] : 1.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float a = sc * X[(xr0 + (l & 15)) * ldx + xk0 + 4 * g + i];
    float b = Y[(yk0 + 4 * g + i) * ldy + yc0 + (l & 15)];
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
  }
}

// Off-diagonal 16x16 block of T = (I + A)^-1 (block rows/cols of 16):
//   T_IJ = -T_II * sum_{K=J}^{I-1} A_IK T_KJ
// with A = diag(rs) Araw (rs null: A = Araw).
__device__ void solve_offdiag(const float* A, float* T, int I, int J, const float* rs = nullptr) {
  constexpr int LA = CH + 4;
  f32x4 y = zero4();
  for (int K = J; K < I; ++K) mm16_xy(y, A, LA, 16 * I, 16 * K, T, LA, 16 * K, 16 * J, rs);
  f32x4 t = zero4();
  mm16_xreg(t, T, LA, 16 * I, 16 * I, y);
  const int l = lane_id(), g = l >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) T[(16 * I + 4 * g + i) * LA + 16 * J + (l & 15)] = -t[i];
}

// Diagonal 16x16 blocks of T by forward substitution; one wave, lane = 16*b + j
// owns column j of block b.  (I + A) T = I  =>  T_rj = d_rj - sum_{i<r} A_ri T_ij.
__device__ void solve_diag(const float* A, float* T, const float* rs = nullptr) {
  constexpr int LA = CH + 4;
  const int l = lane_id(), b = l >> 4, j = l & 15;
  const float* Ab = A + (16 * b) * LA + 16 * b;
  float t[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) t[r] = (r == j) ? 1.f : 0.f;
#pragma unroll
  for (int i = 0; i < 15; ++i) {
#pragma unroll
    for (int r = i + 1; r < 16; ++r) t[r] -= (rs ? rs[16 * b + r] : 1.f) * Ab[r * LA + i] * t[i];
  }
  float* Tb = T + (16 * b) * LA + 16 * b;
#pragma unroll
  for (int r = 0; r < 16; ++r) Tb[r * LA + j] = t[r];
}

// ------------------------------------------------------------------ staging

template <class E>
__device__ __forceinline__ void st4(E* dst, E a, E b, E c, E d);
template <>
__device__ __forceinline__ void st4<bf16>(bf16* dst, bf16 a, bf16 b, bf16 c, bf16 d) {
  *reinterpret_cast<bf16x4*>(dst) = bf16x4{a, b, c, d};
}
template <>
__device__ __forceinline__ void st4<float>(float* dst, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4*>(dst) = f32x4{a, b, c, d};
}

// Copy a [CH x D] tile (rows >= rows are zero) from global (row stride gld
// elements) into LDS row-major (dst, ld) and/or transposed (dstT, ldT).
template <class E, int D, int NT>
__device__ __forceinline__ void stage_tile(const E* __restrict__ src, int64_t gld, int rows,
                                           E* dst, int ld, E* dstT, int ldT) {
  constexpr int VEC = 16 / sizeof(E);
  constexpr int CG = D / VEC;          // vector columns per row
  constexpr int NB = (CH / 4) * CG;    // 4-row blocks
  typedef E vec_t __attribute__((__vector_size__(16)));
  for (int blk = threadIdx.x; blk < NB; blk += NT) {
    const int r0 = (blk / CG) * 4, c0 = (blk % CG) * VEC;
    vec_t x[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (r0 + j < rows) x[j] = *reinterpret_cast<const vec_t*>(src + (int64_t)(r0 + j) * gld + c0);
      else
        for (int e = 0; e < VEC; ++e) x[j][e] = (E)0.f;
    }
    if (dst) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < VEC; e += 4)
          st4<E>(dst + (r0 + j) * ld + c0 + e, x[j][e], x[j][e + 1], x[j][e + 2], x[j][e + 3]);
    }
    if (dstT) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) st4<E>(dstT + (c0 + e) * ldT + r0, x[0][e], x[1][e], x[2][e], x[3][e]);
    }
  }
}


// Solve T = (I + diag(rs) Araw)^-1 for a 64x64 strictly-lower Araw (fp32, row
// stride CH+4) into T, using waves 0..2 of the workgroup.  Must be called by
// every thread (it contains barriers); T's strictly-upper blocks must already
// be zero.  On return (after the final barrier) T is complete.
__device__ __forceinline__ void solve_T(const float* A, float* T, const float* rs) {
  const int w = wave_id();
  if (w == 0) solve_diag(A, T, rs);
  __syncthreads();
  if (w < 3) solve_offdiag(A, T, w + 1, w, rs);
  __syncthreads();
  if (w < 2) solve_offdiag(A, T, w + 2, w, rs);
  __syncthreads();
  if (w == 0) solve_offdiag(A, T, 3, 0, rs);
  __syncthreads();
}

}  // namespace gdn
