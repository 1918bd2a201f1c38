// gdn_tiles.h -- LDS tile helpers shared by the forward and backward kernels:
// the 64x64 unit-lower-triangular solve, register prefetch of chunk tiles and
// their stores into LDS, and coalesced tile writes.
#pragma once
#include "gdn_device.h"
#include "gdn_internal.h"

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
// acc += diag(rs) X[xr0.., xk0..] * Y with Y in registers as above (rs may be null).
__device__ __forceinline__ void mm16_xreg_scaled(f32x4& acc, const float* X, int ldx, int xr0, int xk0,
                                                 const f32x4& yreg, const float* rs) {
  const int l = lane_id(), g = l >> 4;
  const float sc = rs ? rs[xr0 + (l & 15)] : 1.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float a = sc * X[(xr0 + (l & 15)) * ldx + xk0 + 4 * g + i];
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

// Two diagonal 16x16 blocks (ba, bb) of T by forward substitution in one wave,
// with no cross-lane traffic: lane j (< 16) owns column j of block ba, lane
// 16 + j column j of block bb (lanes 32..63 repeat lanes 0..31 and write
// nothing).  Left-looking: row r of the block is
//   T_rj = [r = j] - rs_r sum_{i<r} A_ri T_ij,
// with A's rows read as 16-byte vectors so the reads run ahead of the
// dependent dot products.
__device__ __forceinline__ void solve_diag_pair(const float* A, float* T, int ba, int bb, const float* rs) {
  constexpr int LA = CH + 4;
  const int l = lane_id(), j = l & 15;
  const int b = (l & 16) ? bb : ba;
  const float* Ab = A + (16 * b) * LA + 16 * b;
  float t[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) t[r] = (r == j) ? 1.f : 0.f;
#pragma unroll
  for (int r = 1; r < 16; ++r) {
    f32x4 a[4];
#pragma unroll
    for (int q = 0; q < (r + 3) / 4; ++q) a[q] = *reinterpret_cast<const f32x4*>(Ab + r * LA + 4 * q);
    float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
    for (int i = 0; i < r; ++i) {
      if (i & 1) acc1 += a[i >> 2][i & 3] * t[i];
      else acc0 += a[i >> 2][i & 3] * t[i];
    }
    t[r] -= (rs ? rs[16 * b + r] : 1.f) * (acc0 + acc1);
  }
  if (l < 32) {
    float* Tb = T + (16 * b) * LA + 16 * b;
#pragma unroll
    for (int r = 0; r < 16; ++r) Tb[r * LA + j] = t[r];
  }
}

// All off-diagonal 16x16 blocks of T (after the diagonal blocks), one block
// column per wave: wave J (< 3) forms T_IJ for I = J+1 .. 3 in order,
//   T_IJ = -T_II * sum_{K=J}^{I-1} A_IK T_KJ,
// keeping the blocks it has finished in registers (in accumulator layout,
// which is the B-operand layout of the 16x16x4 fp32 product) so that no
// barrier separates them.  Complete after the caller's next barrier.
template <int J>
__device__ __forceinline__ void solve_column(const float* A, float* T, const float* rs) {
  constexpr int LA = CH + 4;
  const int l = lane_id(), g = l >> 4;
  f32x4 tk[3];  // tk[I - J - 1] = T_IJ
#pragma unroll
  for (int I = J + 1; I < 4; ++I) {
    f32x4 y = zero4();
    mm16_xy(y, A, LA, 16 * I, 16 * J, T, LA, 16 * J, 16 * J, rs);
#pragma unroll
    for (int K = J + 1; K < I; ++K) mm16_xreg_scaled(y, A, LA, 16 * I, 16 * K, tk[K - J - 1], rs);
    f32x4 t = zero4();
    mm16_xreg(t, T, LA, 16 * I, 16 * I, y);
    t = zero4() - t;
    tk[I - J - 1] = t;
#pragma unroll
    for (int i = 0; i < 4; ++i) T[(16 * I + 4 * g + i) * LA + 16 * J + (l & 15)] = t[i];
  }
}
__device__ __forceinline__ void solve_columns(const float* A, float* T, int w, const float* rs) {
  if (w == 0) solve_column<0>(A, T, rs);
  else if (w == 1) solve_column<1>(A, T, rs);
  else if (w == 2) solve_column<2>(A, T, rs);
}

}  // namespace gdn

namespace gdn {

// Register prefetch of up to three [CH x D_t] tiles of one chunk (D_t = 0:
// tensor absent), moved as 4-row x 16-byte blocks so that each block can be
// written to LDS row-major and/or transposed.  Every tensor has its own
// compile-time block loop, so no pointer or stride is ever selected at run
// time.  Rows at or past `rows` are loaded from the last valid row (finite
// data); the kernels mask those rows through beta = 0, g = 0 and their output
// masks, which leaves every real result unchanged.  load() only issues global
// loads; store() consumes them.
template <class E, int NT, int D>
struct TilePart {
  static constexpr int VEC = 16 / (int)sizeof(E);
  static constexpr int NBLK = D > 0 ? (CH / 4) * (D / VEC) : 0;
  static constexpr int NB = (NBLK + NT - 1) / NT;
  static constexpr int BPR = D > 0 ? D / VEC : 1;  // blocks per 4-row group
  typedef E vec_t __attribute__((__vector_size__(16)));
  vec_t blk[NB > 0 ? NB : 1][4];
  template <bool NTL>
  __device__ __forceinline__ static vec_t ld_vec(const char* p) {
    if constexpr (NTL) return __builtin_nontemporal_load(reinterpret_cast<const vec_t*>(p));
    else return *reinterpret_cast<const vec_t*>(p);
  }

  // ZFILL: rows at or past `rows` become zero instead of copies of the last row.
  // src is the same for every lane; each load is addressed as src + a 32-bit
  // byte offset (the host keeps 64 rows of a tile under 2 GiB), one address
  // register per load.
  // NTL: non-temporal loads.
  template <bool ZFILL = false, bool NTL = false>
  __device__ __forceinline__ void load(const E* src, int64_t gld, int rows, int tid = threadIdx.x) {
    const char* base = reinterpret_cast<const char*>(src);
    const uint32_t ldb = (uint32_t)gld * (uint32_t)sizeof(E);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int id = tid + b * NT;
      if (NB * NT == NBLK || id < NBLK) {
        const int r0 = (id / BPR) * 4, c0 = (id % BPR) * VEC;
        const uint32_t cb = (uint32_t)c0 * (uint32_t)sizeof(E);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (ZFILL) {
            blk[b][j] = vec_t{};
            if (r0 + j < rows) blk[b][j] = ld_vec<NTL>(base + ((uint32_t)(r0 + j) * ldb + cb));
          } else {
            blk[b][j] = ld_vec<NTL>(base + ((uint32_t)min(r0 + j, rows - 1) * ldb + cb));
          }
        }
      }
    }
  }
  // Divide every row by its L2 norm (q / k pre-processing).  A row's D/VEC
  // blocks sit on consecutive lanes; every lane of the wave must call this.
  __device__ __forceinline__ void normalize_rows(int tid = threadIdx.x) {
    if constexpr (NB > 0) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const bool valid = NB * NT == NBLK || tid + b * NT < NBLK;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float ss = 0.f;
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            const float x = to_f(blk[b][j][e]);
            ss += x * x;
          }
          ss = lane_group_sum<BPR>(valid ? ss : 0.f);
          const float sc = rsqrtf(ss + QK_NORM_EPS);
#pragma unroll
          for (int e = 0; e < VEC; ++e) blk[b][j][e] = to_e<E>(to_f(blk[b][j][e]) * sc);
        }
      }
    }
  }
  // The tile row-major twice: as loaded at dst (8-byte stores, any stride)
  // and at dst2 (16-byte stores: ld2 * sizeof(E) a multiple of 16), the rows
  // r0 .. r0 + 3 of block b of the second copy scaled by sc[b][0 .. 3] when
  // SCALE2 (computed in fp32, rounded once).
  template <bool SCALE2>
  __device__ __forceinline__ void store_rows2(E* dst, int ld, E* dst2, int ld2, const f32x4 (&sc)[NB > 0 ? NB : 1],
                                              int tid = threadIdx.x) const {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int id = tid + b * NT;
      if (NB * NT == NBLK || id < NBLK) {
        const int r0 = (id / BPR) * 4, c0 = (id % BPR) * VEC;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
          for (int e = 0; e < VEC; e += 4)
            st4<E>(dst + (r0 + j) * ld + c0 + e, blk[b][j][e], blk[b][j][e + 1], blk[b][j][e + 2], blk[b][j][e + 3]);
          vec_t v = blk[b][j];
          if (SCALE2) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) v[e] = to_e<E>(to_f(v[e]) * sc[b][j]);
          }
          *reinterpret_cast<vec_t*>(dst2 + (r0 + j) * ld2 + c0) = v;
        }
      }
    }
  }
  // The tile row-major with 16-byte stores (ld * sizeof(E) a multiple of 16).
  __device__ __forceinline__ void store_rows16(E* dst, int ld, int tid = threadIdx.x) const {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int id = tid + b * NT;
      if (NB * NT == NBLK || id < NBLK) {
        const int r0 = (id / BPR) * 4, c0 = (id % BPR) * VEC;
#pragma unroll
        for (int j = 0; j < 4; ++j) *reinterpret_cast<vec_t*>(dst + (r0 + j) * ld + c0) = blk[b][j];
      }
    }
  }
  // First row of each of this thread's blocks (blocks past the tile: -1).
  __device__ __forceinline__ static int block_row(int b, int tid = threadIdx.x) {
    const int id = tid + b * NT;
    return (NB * NT == NBLK || id < NBLK) ? (id / BPR) * 4 : -1;
  }
  // The tile row-major at dst (8-byte stores), rows at or past `rows` as
  // zeros (for a tile loaded without ZFILL, whose extra rows repeat the last).
  __device__ __forceinline__ void store_zrows(E* dst, int ld, int rows, int tid = threadIdx.x) const {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int id = tid + b * NT;
      if (NB * NT == NBLK || id < NBLK) {
        const int r0 = (id / BPR) * 4, c0 = (id % BPR) * VEC;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const vec_t v = r0 + j < rows ? blk[b][j] : vec_t{};
#pragma unroll
          for (int e = 0; e < VEC; e += 4) st4<E>(dst + (r0 + j) * ld + c0 + e, v[e], v[e + 1], v[e + 2], v[e + 3]);
        }
      }
    }
  }
  __device__ __forceinline__ void store(E* dst, int ld, E* dstT, int ldT, int tid = threadIdx.x) const {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int id = tid + b * NT;
      if (NB * NT == NBLK || id < NBLK) {
        const int r0 = (id / BPR) * 4, c0 = (id % BPR) * VEC;
        if (dst) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < VEC; e += 4)
              st4<E>(dst + (r0 + j) * ld + c0 + e, blk[b][j][e], blk[b][j][e + 1], blk[b][j][e + 2], blk[b][j][e + 3]);
        }
        if (dstT) {
#pragma unroll
          for (int e = 0; e < VEC; ++e)
            st4<E>(dstT + (c0 + e) * ldT + r0, blk[b][0][e], blk[b][1][e], blk[b][2][e], blk[b][3][e]);
        }
      }
    }
  }
};

// Copy rows [0, rows) of a [CH x D] row-major LDS tile (row stride ld) to
// global memory (row stride gld) in 16-byte pieces.
template <class E, int D, int NT>
__device__ __forceinline__ void store_tile(const E* src, int ld, E* dst, int64_t gld, int rows) {
  constexpr int VEC = 16 / (int)sizeof(E);
  typedef E vec_t __attribute__((__vector_size__(16)));
  for (int e = threadIdx.x; e < rows * (D / VEC); e += NT) {
    const int r = e / (D / VEC), c0 = (e % (D / VEC)) * VEC;
    *reinterpret_cast<vec_t*>(dst + (int64_t)r * gld + c0) = *reinterpret_cast<const vec_t*>(src + r * ld + c0);
  }
}

// Write a C-layout accumulator tile (lane: rows r0+4g..+3 of column c0+lane%16)
// into a row-major E matrix, four consecutive columns per lane after a quad
// transpose.
template <class E, bool NTS = false>
__device__ __forceinline__ void st_tile_rows(E* base, int ld, int r0, int c0, const f32x4& acc) {
  const int l = lane_id(), g = l >> 4, q = (l >> 2) & 3, b = l & 3;
  st4_transposed<E, NTS>(base + (r0 + 4 * g + b) * ld + c0 + 4 * q, acc);
}

// Lead-ins of the segment runs.  The transition of the state (or of its
// gradient) over chunks a..b-1 has norm at most exp(sum_c Lambda_c), Lambda_c
// the chunk log-bounds of the scalar records.  A segment whose run starts from
// a zero state that many chunks before its first (after its last, for the
// reverse chain) has its boundary state exact to 2^-24 once the sum is at or
// below LN_EPS.  Every lane of every wave computes the same value.
//
// Forward: the largest wb <= cb with sum_{c=wb}^{cb-1} Lambda_c <= LN_EPS, else
// 0 (the run then starts at the sequence start, from h0: exact).
__device__ __forceinline__ int lead_in_begin(const float* rec, int64_t chunk0, int H, int h, int cb) {
  const int l = lane_id();
  float acc = 0.f;  // sum over the chunks of earlier windows
  for (int base = cb - 1; base >= 0; base -= 64) {
    const int c = base - l;
    const float lam = c >= 0 ? rec[((chunk0 + c) * H + h) * RECF + 5 * CH] : 0.f;
    const float run = acc + wave_incl_scan(lam);  // sum over chunks c .. cb - 1
    const unsigned long long hit = __ballot(c >= 0 && run <= LN_EPS);
    if (hit) return base - (__ffsll((long long)hit) - 1);
    acc = __shfl(run, 63, 64);
  }
  return 0;
}
// Reverse chain: the smallest we >= ce with sum_{c=ce}^{we-1} Lambda_c <= LN_EPS,
// else nch (the run then starts at the sequence end, from dhT: exact).
__device__ __forceinline__ int lead_in_end(const float* rec, int64_t chunk0, int H, int h, int ce, int nch) {
  const int l = lane_id();
  float acc = 0.f;
  for (int base = ce; base < nch; base += 64) {
    const int c = base + l;
    const float lam = c < nch ? rec[((chunk0 + c) * H + h) * RECF + 5 * CH] : 0.f;
    const float run = acc + wave_incl_scan(lam);  // sum over chunks ce .. c
    const unsigned long long hit = __ballot(c < nch && run <= LN_EPS);
    if (hit) return base + __ffsll((long long)hit);
    acc = __shfl(run, 63, 64);
  }
  return nch;
}

// A chunk's T as the T solve stores it (one 16 KiB entry per chunk and head):
// fp32 64 x 64 row-major for fp32 inputs; for bf16 inputs two bf16 64 x 64
// row-major planes, the value rounded to bf16 (the "hi" plane) and then the
// residual T - hi rounded to bf16 (the "lo" plane), so that hi + lo carries T
// to about 16 bits.  The chains use T only as a bf16 matrix-core operand
// (scaled by a column factor and rounded) and read the hi plane alone; the
// gradient kernel's near-fp32 products read both.
//
// TPart: one thread's share of the chunk's (hi) T, in pieces of 8 consecutive
// elements, piece i at element 8 (tid + i NT); get(i, j) gives elements
// 8 (tid + i NT) + 4 j .. + 3 as fp32.
template <class E, int NT>
struct TPart;
template <int NT>
struct TPart<float, NT> {
  static constexpr int NP = CH * CH / (8 * NT);
  static_assert(NP * 8 * NT == CH * CH && (8 * NT) % CH == 0, "whole rows of T per pass");
  f32x4 v[NP][2];
  template <bool NTL = false>
  __device__ __forceinline__ void load(const float* t, int tid = threadIdx.x) {
#pragma unroll
    for (int i = 0; i < NP; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const f32x4* p = reinterpret_cast<const f32x4*>(t + 8 * (tid + i * NT) + 4 * j);
        v[i][j] = NTL ? __builtin_nontemporal_load(p) : *p;
      }
  }
  __device__ __forceinline__ f32x4 get(int i, int j) const { return v[i][j]; }
};
template <int NT>
struct TPart<bf16, NT> {
  static constexpr int NP = CH * CH / (8 * NT);
  static_assert(NP * 8 * NT == CH * CH && (8 * NT) % CH == 0, "whole rows of T per pass");
  bf16x8 v[NP];
  template <bool NTL = false>
  __device__ __forceinline__ void load(const float* t, int tid = threadIdx.x) {
    const bf16* hi = reinterpret_cast<const bf16*>(t);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const bf16x8* p = reinterpret_cast<const bf16x8*>(hi + 8 * (tid + i * NT));
      v[i] = NTL ? __builtin_nontemporal_load(p) : *p;
    }
  }
  __device__ __forceinline__ f32x4 get(int i, int j) const {
    return f32x4{(float)v[i][4 * j], (float)v[i][4 * j + 1], (float)v[i][4 * j + 2], (float)v[i][4 * j + 3]};
  }
};

// This thread's 16-byte piece of a chunk's scalar record (threads < RECF / 4),
// prefetched with the chunk's tiles; store() writes it to LDS, where the
// record's arrays lie as in memory.
struct RecordPart {
  f32x4 rv;
  __device__ __forceinline__ void load(const float* rec) {
    if (threadIdx.x < RECF / 4) rv = *reinterpret_cast<const f32x4*>(rec + 4 * threadIdx.x);
  }
  __device__ __forceinline__ void store(float* dst) const {
    if (threadIdx.x < RECF / 4) *reinterpret_cast<f32x4*>(dst + 4 * threadIdx.x) = rv;
  }
};

// Gradient of a row-normalised input: rows of `grad` (LDS, row stride ld) are
// the gradient with respect to x / sqrt(|x|^2 + eps); `raw` (global, row stride
// gld) holds x.  Writes dx = (grad - x (x.grad) / n^2) / n, n^2 = |x|^2 + eps,
// for rows [0, rows) to dst (global) in 16-byte pieces.
template <class E, int D, int NT>
__device__ __forceinline__ void store_tile_unnorm(const E* grad, int ld, const E* raw, int64_t gld, E* dst,
                                                  int64_t dgld, int rows) {
  constexpr int VEC = 16 / (int)sizeof(E), BPR = D / VEC;
  typedef E vec_t __attribute__((__vector_size__(16)));
  static_assert((CH * BPR) % NT == 0 || NT % (CH * BPR) == 0, "whole lane groups per pass");
  for (int e = threadIdx.x; e < CH * BPR; e += NT) {
    const int r = e / BPR, c0 = (e % BPR) * VEC;
    const bool valid = r < rows;
    vec_t x = vec_t{}, d = vec_t{};
    if (valid) {
      x = *reinterpret_cast<const vec_t*>(raw + (int64_t)r * gld + c0);
      d = *reinterpret_cast<const vec_t*>(grad + r * ld + c0);
    }
    float ss = 0.f, dot = 0.f;
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      ss += to_f(x[i]) * to_f(x[i]);
      dot += to_f(x[i]) * to_f(d[i]);
    }
    ss = lane_group_sum<BPR>(ss) + QK_NORM_EPS;
    dot = lane_group_sum<BPR>(dot);
    const float inv = rsqrtf(ss), proj = dot / ss;
    vec_t out;
#pragma unroll
    for (int i = 0; i < VEC; ++i) out[i] = to_e<E>((to_f(d[i]) - to_f(x[i]) * proj) * inv);
    if (valid) *reinterpret_cast<vec_t*>(dst + (int64_t)r * dgld + c0) = out;
  }
}

}  // namespace gdn
