// gdn_device.h -- device-side building blocks shared by the GDN kernels (gfx950).
//
// Matrix products run on the CDNA4 matrix cores with 16x16 output tiles:
//   bf16 operands: v_mfma_f32_16x16x32_bf16  (one instruction per 32-deep k-block)
//   fp32 operands: v_mfma_f32_16x16x4_f32    (eight instructions per 32-deep k-block)
// Accumulator ("C") layout of a 16x16 fp32 tile in a wave of 64 lanes:
//   lane l holds C[4*(l/16) + i][l % 16] in acc[i], i = 0..3.
//
// k-permutation.  Inside one 32-deep k-block, lane l (lane group g = l/16) feeds
// eight operand slots j = 0..7 that stand for the logical k index
//   kperm(g, j) = 4g + j          (j < 4)
//               = 16 + 4g + j - 4 (j >= 4).
// The matrix core pairs slot j of the A operand with slot j of the B operand in
// the same lane group, so any fixed slot->k map gives the right sum as long as A
// and B use the same one.  This particular map is chosen because it is exactly
// what a lane already holds of two vertically stacked C tiles (rows 4g..4g+3 of
// each): an accumulator tile pair can be fed back as an operand along k with no
// data movement across lanes.
//
// Operand sources:
//   "X" operand (A side, m = row):  row-major matrix in LDS, k contiguous.
//   "Y" operand (B side, n = col):  the product is C = X * Y^T, Y row-major with
//                                   k contiguous -- the "NT" form.
//   register operand: a pair of C tiles stacked along k.
#pragma once
#include <hip/hip_runtime.h>

#include <type_traits>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int CH = 64;  // chunk length (rows per chunk)

// ln(2^-24): a boundary state whose propagated contribution is bounded by
// exp(sum of per-token log-bounds) * |state| stops mattering once that factor
// is below fp32's unit round-off.
constexpr float LN_EPS = -16.635532333438686f;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Returns the LDS pointer p unchanged while hiding its value from the
// optimizer: address arithmetic derived from the result cannot be hoisted
// above or shared across this point.  Kernels whose LDS exceeds the 64 KiB
// reach of a ds instruction's immediate offset call it at each phase, so that
// per-lane LDS addresses are formed where they are used instead of being
// precomputed once and held (or spilled) across the whole chunk loop.
template <class T>
__device__ __forceinline__ T* lds_opaque(T* p) {
  uint32_t a = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) T*)p);
  asm volatile("" : "+s"(a));
  return (T*)((__attribute__((address_space(3))) T*)(uintptr_t)a);
}

__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// Cycles per phase of a workgroup, for an instrumented build only (compiled
// with GDN_PHASE_CLOCK; otherwise every call is empty).  Each wave reads the
// shader clock (s_memtime) at mark(i) and adds the cycles since its previous
// mark to phase i; the sums stay in registers until flush(), which lane 0
// writes out once at the end, so that no store enters the phases measured.
#ifdef GDN_PHASE_CLOCK
constexpr bool kPhaseClock = true;
#else
constexpr bool kPhaseClock = false;
#endif
template <int NPH>
struct PhaseClock {
  uint64_t last;
  uint32_t acc[NPH];
  __device__ __forceinline__ void start() {
    if constexpr (kPhaseClock) {
#pragma unroll
      for (int i = 0; i < NPH; ++i) acc[i] = 0;
      last = __builtin_amdgcn_s_memtime();
    }
  }
  __device__ __forceinline__ void mark(int i) {
    if constexpr (kPhaseClock) {
      const uint64_t t = __builtin_amdgcn_s_memtime();
      acc[i] += (uint32_t)(t - last);
      last = t;
    }
  }
  // a count kept in slot i instead of cycles (the chunks a chain ran)
  __device__ __forceinline__ void set(int i, uint32_t v) {
    if constexpr (kPhaseClock) acc[i] = v;
  }
  // dst: this workgroup's [waves][NPH] record
  __device__ __forceinline__ void flush(uint32_t* dst) const {
    if constexpr (kPhaseClock) {
      if ((threadIdx.x & 63) == 0) {
#pragma unroll
        for (int i = 0; i < NPH; ++i) dst[wave_id() * NPH + i] = acc[i];
      }
    }
  }
};
// Workgroups whose phase cycles are kept (the first ones of the grid).
constexpr int CLOCK_BLOCKS = 512;

// ---------------------------------------------------------------------------
// Operand fragments: eight k-slots per lane.
template <class E> struct Frag;
template <> struct Frag<bf16> { bf16x8 v; };
template <> struct Frag<float> { f32x4 lo, hi; };

__device__ __forceinline__ void mma(f32x4& acc, const Frag<bf16>& a, const Frag<bf16>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[j], b.lo[j], acc, 0, 0, 0);
#pragma unroll
  for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[j], b.hi[j], acc, 0, 0, 0);
}

// Load the eight k-slots of row `row` of a row-major LDS matrix (k contiguous),
// for the k-block starting at k0.  Slots: [k0+4g .. +3], [k0+16+4g .. +3].
__device__ __forceinline__ Frag<bf16> ld_frag(const bf16* base, int ld, int row, int k0) {
  const int g = lane_id() >> 4;
  const bf16* p = base + row * ld + k0 + 4 * g;
  bf16x4 a = *reinterpret_cast<const bf16x4*>(p);
  bf16x4 b = *reinterpret_cast<const bf16x4*>(p + 16);
  Frag<bf16> f;
  f.v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return f;
}
__device__ __forceinline__ Frag<float> ld_frag(const float* base, int ld, int row, int k0) {
  const int g = lane_id() >> 4;
  const float* p = base + row * ld + k0 + 4 * g;
  Frag<float> f;
  f.lo = *reinterpret_cast<const f32x4*>(p);
  f.hi = *reinterpret_cast<const f32x4*>(p + 16);
  return f;
}

// Fragment of row `row` of a row-major E matrix (LDS or global) in the
// "contiguous" k-slot order: slot j of lane group g is k0 + 8g + j, one 16-byte
// read per lane.  Both operands of a product must use the same order; this one
// serves products whose operands both come from memory.
__device__ __forceinline__ Frag<bf16> ld_frag8(const bf16* base, int ld, int row, int k0) {
  const int g = lane_id() >> 4;
  Frag<bf16> f;
  f.v = *reinterpret_cast<const bf16x8*>(base + row * ld + k0 + 8 * g);
  return f;
}
__device__ __forceinline__ Frag<float> ld_frag8(const float* base, int ld, int row, int k0) {
  const int g = lane_id() >> 4;
  const float* p = base + row * ld + k0 + 8 * g;
  Frag<float> f;
  f.lo = *reinterpret_cast<const f32x4*>(p);
  f.hi = *reinterpret_cast<const f32x4*>(p + 4);
  return f;
}

// Register operand from two accumulator tiles stacked along k (t0: k0..k0+15,
// t1: k0+16..k0+31), each slot multiplied by a per-k scale (s0 for t0's rows,
// s1 for t1's rows).
__device__ __forceinline__ void pack_frag(Frag<bf16>& f, const f32x4& t0, const f32x4& t1) {
  f.v = bf16x8{(bf16)t0[0], (bf16)t0[1], (bf16)t0[2], (bf16)t0[3],
               (bf16)t1[0], (bf16)t1[1], (bf16)t1[2], (bf16)t1[3]};
}
__device__ __forceinline__ void pack_frag(Frag<float>& f, const f32x4& t0, const f32x4& t1) {
  f.lo = t0;
  f.hi = t1;
}
template <class E>
__device__ __forceinline__ void pack_frag_scaled(Frag<E>& f, const f32x4& t0, const f32x4& t1,
                                                 const f32x4& s0, const f32x4& s1) {
  pack_frag(f, t0 * s0, t1 * s1);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Operand of a near-fp32 product, from an fp32 fragment.  For E = float it is
// that fragment (fp32 matrix-core products).  For E = bf16 it is the pair
// x = hi + lo of bf16 fragments (hi = x rounded, lo = the exact residual x - hi
// rounded): the product hi*hi + hi*lo + lo*hi (lo*lo dropped) carries about 16
// significant bits of each operand, with three bf16 instructions per 32-deep
// k-block in place of eight fp32 ones.
template <class E> struct PFrag;
template <> struct PFrag<float> {
  Frag<float> f;
  __device__ __forceinline__ explicit PFrag(const Frag<float>& x) : f(x) {}
  __device__ __forceinline__ PFrag() {}
};
template <> struct PFrag<bf16> {
  Frag<bf16> hi, lo;
  __device__ __forceinline__ PFrag() {}
  __device__ __forceinline__ explicit PFrag(const Frag<float>& x) {
    pack_frag(hi, x.lo, x.hi);
    f32x4 rl, rh;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      rl[i] = x.lo[i] - (float)hi.v[i];
      rh[i] = x.hi[i] - (float)hi.v[4 + i];
    }
    pack_frag(lo, rl, rh);
  }
};
__device__ __forceinline__ void mma(f32x4& acc, const PFrag<float>& a, const PFrag<float>& b) { mma(acc, a.f, b.f); }
__device__ __forceinline__ void mma(f32x4& acc, const PFrag<bf16>& a, const PFrag<bf16>& b) {
  mma(acc, a.lo, b.hi);
  mma(acc, a.hi, b.lo);
  mma(acc, a.hi, b.hi);
}
// The E-operand part of a PFrag (the rounded value for bf16).
__device__ __forceinline__ const Frag<float>& e_part(const PFrag<float>& a) { return a.f; }
__device__ __forceinline__ const Frag<bf16>& e_part(const PFrag<bf16>& a) { return a.hi; }

// fp32 -> storage type
template <class E> __device__ __forceinline__ E to_e(float x);
template <> __device__ __forceinline__ bf16 to_e<bf16>(float x) { return (bf16)x; }
template <> __device__ __forceinline__ float to_e<float>(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f(float x) { return x; }

// Fragment of row `row` of an fp32 row-major LDS matrix, converted to E.
template <class E>
__device__ __forceinline__ Frag<E> ld_frag_f32(const float* base, int ld, int row, int k0) {
  const int g = lane_id() >> 4;
  const float* p = base + row * ld + k0 + 4 * g;
  Frag<E> f;
  pack_frag(f, *reinterpret_cast<const f32x4*>(p), *reinterpret_cast<const f32x4*>(p + 16));
  return f;
}

// Fragment of row m of M^T for an fp32 row-major M (so the k-slots walk down
// column m of M), times sc, converted to E.
template <class E>
__device__ __forceinline__ Frag<E> ld_fragT(const float* M, int ld, int m, int k0, float sc) {
  const int g = lane_id() >> 4;
  const float* p = M + (k0 + 4 * g) * ld + m;
  f32x4 a, b;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    a[j] = sc * p[j * ld];
    b[j] = sc * p[(16 + j) * ld];
  }
  Frag<E> f;
  pack_frag(f, a, b);
  return f;
}

// Four consecutive E values as fp32, and the reverse.
template <class E>
__device__ __forceinline__ f32x4 ld4f(const E* p);
template <>
__device__ __forceinline__ f32x4 ld4f<bf16>(const bf16* p) {
  const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
template <>
__device__ __forceinline__ f32x4 ld4f<float>(const float* p) {
  return *reinterpret_cast<const f32x4*>(p);
}
// A store of data that the storing kernel never reads back (its output, or a
// buffer that a later kernel reads from HBM anyway): non-temporal.  The chain
// kernels' state stores and the T solve's store of T use it (the chains ran
// shorter with it); the gradient kernel's stores of dq, dk, dv ran slower with
// it and are plain stores.
template <class V>
__device__ __forceinline__ void st_out(V* p, const V& v) {
  __builtin_nontemporal_store(v, p);
}

template <class E>
__device__ __forceinline__ void st4f(E* p, const f32x4& v);
template <>
__device__ __forceinline__ void st4f<bf16>(bf16* p, const f32x4& v) {
  *reinterpret_cast<bf16x4*>(p) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
}
template <>
__device__ __forceinline__ void st4f<float>(float* p, const f32x4& v) {
  *reinterpret_cast<f32x4*>(p) = v;
}

// DPP move within rows of 16 lanes (quad permutations and row mirrors, whose
// source lanes always exist, so no fill value is needed and none is set up).
template <int CTRL>
__device__ __forceinline__ int dpp_mov(int x) {
  return __builtin_amdgcn_mov_dpp(x, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, dpp_mov<CTRL>(__builtin_bit_cast(int, x)));
}

// x from lane (lane ^ X) of the same quad (DPP quad permutation, no LDS).
template <int X>
__device__ __forceinline__ float quad_xor(float x) {
  constexpr int ctrl = (0 ^ X) | ((1 ^ X) << 2) | ((2 ^ X) << 4) | ((3 ^ X) << 6);
  return dpp_mov<ctrl>(x);
}

// Forces x to be computed here: the compiler may not sink the arithmetic that
// produces it past this point (which would keep its inputs alive instead).
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(f32x4& x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float t = x[i];
    asm volatile("" : "+v"(t));
    x[i] = t;
  }
}

// Sum over the 16 lanes of each DPP row (lanes 16r .. 16r+15), in every lane.
__device__ __forceinline__ float row16_sum(float x) {
  x += quad_xor<1>(x);
  x += quad_xor<2>(x);
  x += dpp_mov<0x141>(x);  // half-row mirror
  x += dpp_mov<0x140>(x);  // row mirror
  return x;
}

// Sum over each aligned group of N (8 or 16) consecutive lanes, in every lane
// of the group.  Every lane of the wave must execute it.
template <int N>
__device__ __forceinline__ float lane_group_sum(float x) {
  static_assert(N == 8 || N == 16, "lane groups of 8 or 16");
  x += quad_xor<1>(x);
  x += quad_xor<2>(x);
  x += dpp_mov<0x141>(x);
  if (N == 16) x += dpp_mov<0x140>(x);
  return x;
}

// Input pre-processing (see PrepParams): 1 / sqrt(sum of squares + eps) for the
// L2 normalisation of q and k, and the gate / beta activations with their
// derivatives.
constexpr float QK_NORM_EPS = 1e-6f;
__device__ __forceinline__ float softplus_f(float x) { return x > 20.f ? x : log1pf(__expf(x)); }
__device__ __forceinline__ float sigmoid_f(float x) { return 1.f / (1.f + __expf(-x)); }

// 4x4 transpose across each aligned quad of lanes: lane b of the quad holds
// column b of a 4x4 block (v[i] = M[i][b]) and gets row b (v[j] = M[b][j]);
// applied to rows it gives columns.  Two butterfly stages: 2x2 blocks are
// exchanged with lane b^2, then single entries with lane b^1.
__device__ __forceinline__ f32x4 quad_transpose(f32x4 v) {
  const int b = threadIdx.x & 3;
  {
    const bool lo = (b & 2) == 0;
    const float r0 = quad_xor<2>(lo ? v[2] : v[0]);
    const float r1 = quad_xor<2>(lo ? v[3] : v[1]);
    v = lo ? f32x4{v[0], v[1], r0, r1} : f32x4{r0, r1, v[2], v[3]};
  }
  {
    const bool lo = (b & 1) == 0;
    const float r0 = quad_xor<1>(lo ? v[1] : v[0]);
    const float r1 = quad_xor<1>(lo ? v[3] : v[2]);
    v = lo ? f32x4{v[0], r0, v[2], r1} : f32x4{r0, v[1], r1, v[3]};
  }
  return v;
}

// quad_transpose for four 16-bit values held as two packed dwords
// (d0 = v0 | v1 << 16, d1 = v2 | v3 << 16).
template <int X>
__device__ __forceinline__ uint32_t quad_xor_u(uint32_t x) {
  constexpr int ctrl = (0 ^ X) | ((1 ^ X) << 2) | ((2 ^ X) << 4) | ((3 ^ X) << 6);
  return (uint32_t)dpp_mov<ctrl>((int)x);
}
__device__ __forceinline__ void quad_transpose16(uint32_t& d0, uint32_t& d1) {
  const int b = threadIdx.x & 3;
  // 2x2 blocks with lane b^2: lanes 0, 1 take the partner's first dword as
  // their second, lanes 2, 3 the partner's second dword as their first
  const uint32_t a = quad_xor_u<2>(d0), c = quad_xor_u<2>(d1);
  const bool lo = (b & 2) == 0;
  const uint32_t n0 = lo ? d0 : c, n1 = lo ? a : d1;
  // single entries with lane b^1: even lanes keep their low halves and append
  // the partner's, odd lanes put the partner's high half below their own (one
  // byte permute with a per-lane selector)
  const uint32_t sel = (b & 1) ? 0x03020706u : 0x05040100u;
  const uint32_t x0 = quad_xor_u<1>(n0), x1 = quad_xor_u<1>(n1);
  d0 = __builtin_amdgcn_perm(x0, n0, sel);
  d1 = __builtin_amdgcn_perm(x1, n1, sel);
}

// LDS transpose read (ds_read_b64_tr_b16, CDNA4).  Every lane names an 8-byte
// piece (four 16-bit elements, 8-byte aligned); within each group of 16 lanes,
// lane 4a + b receives element b of the pieces named by lanes a, 4 + a, 8 + a and
// 12 + a of its group, in that order.  Reading rows r0 + L/4 at columns
// c0 + 4 (L % 4) (lane L) therefore hands lane l the four elements
// M[r0 + 4 (l/16) + j][c0 + l % 16], j = 0..3: one column piece of a 16 x 16
// block, laid out as an accumulator tile holds it.
__device__ __forceinline__ bf16x4 ds_read_tr16(const bf16* p) {
  typedef short s4 __attribute__((ext_vector_type(4)));
  const s4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)(p));
  return __builtin_bit_cast(bf16x4, v);
}
// The column piece above: rows r0 + 4g .. r0 + 4g + 3 of column c0 + lane%16 of
// a row-major LDS matrix (rows 8-byte aligned, c0 a multiple of 4).
__device__ __forceinline__ bf16x4 ld_cpiece_tr(const bf16* base, int ld, int r0, int c0) {
  const int l = lane_id();
  return ds_read_tr16(base + (r0 + (l >> 2)) * ld + c0 + 4 * (l & 3));
}

// Fragment whose k-slots walk down column col0 + lane%16 of a row-major E
// matrix in LDS (rows k0+4g.., k0+16+4g..: the operand layout of an accumulator
// tile pair).  bf16: two transpose reads; fp32: 4-element row pieces turned
// into column pieces by quad transposes.  col0 must be a multiple of 4; all 64
// lanes must take part.
template <class E>
__device__ __forceinline__ Frag<E> ld_fragC_q(const E* base, int ld, int k0, int col0);
template <>
__device__ __forceinline__ Frag<bf16> ld_fragC_q<bf16>(const bf16* base, int ld, int k0, int col0) {
  const bf16x4 a = ld_cpiece_tr(base, ld, k0, col0), b = ld_cpiece_tr(base, ld, k0 + 16, col0);
  Frag<bf16> f;
  f.v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return f;
}
template <>
__device__ __forceinline__ Frag<float> ld_fragC_q<float>(const float* base, int ld, int k0, int col0) {
  const int l = lane_id(), g = l >> 4, q = (l >> 2) & 3, b = l & 3;
  const float* p = base + (k0 + 4 * g + b) * ld + col0 + 4 * q;
  Frag<float> f;
  f.lo = quad_transpose(*reinterpret_cast<const f32x4*>(p));
  f.hi = quad_transpose(*reinterpret_cast<const f32x4*>(p + 16 * ld));
  return f;
}

// ld_fragC_q in the contiguous k-slot order (pairs with ld_frag8): k-slots
// k0 + 8g .. k0 + 8g + 7 down column col0 + lane%16 of a row-major LDS matrix.
template <class E>
__device__ __forceinline__ Frag<E> ld_fragC_q8(const E* base, int ld, int k0, int col0);
template <>
__device__ __forceinline__ Frag<bf16> ld_fragC_q8<bf16>(const bf16* base, int ld, int k0, int col0) {
  const int l = lane_id();
  const bf16* p = base + (k0 + 8 * (l >> 4) + ((l & 15) >> 2)) * ld + col0 + 4 * (l & 3);
  const bf16x4 a = ds_read_tr16(p), b = ds_read_tr16(p + 4 * ld);
  Frag<bf16> f;
  f.v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return f;
}
template <>
__device__ __forceinline__ Frag<float> ld_fragC_q8<float>(const float* base, int ld, int k0, int col0) {
  const int l = lane_id();
  const float* p = base + (k0 + 8 * (l >> 4)) * ld + col0 + (l & 15);
  Frag<float> f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f.lo[j] = p[j * ld];
    f.hi[j] = p[(4 + j) * ld];
  }
  return f;
}

// Rows r0 + 4g .. r0 + 4g + 3 of column c0 + lane%16 of a row-major LDS
// matrix, as fp32: the piece of an accumulator tile at (r0, c0).
template <class E>
__device__ __forceinline__ f32x4 ld_cpiece(const E* base, int ld, int r0, int c0);
template <>
__device__ __forceinline__ f32x4 ld_cpiece<bf16>(const bf16* base, int ld, int r0, int c0) {
  const bf16x4 v = ld_cpiece_tr(base, ld, r0, c0);
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
template <>
__device__ __forceinline__ f32x4 ld_cpiece<float>(const float* base, int ld, int r0, int c0) {
  const int l = lane_id();
  const float* p = base + (r0 + 4 * (l >> 4)) * ld + c0 + (l & 15);
  return f32x4{p[0], p[ld], p[2 * ld], p[3 * ld]};
}

// An accumulator tile (rows r0.., columns c0..) stored transposed, into the
// row-major matrix M^T: the lane's four rows of its column are one piece.
template <class E>
__device__ __forceinline__ void st_tile_cm(E* baseT, int ldT, int r0, int c0, const f32x4& acc) {
  const int l = lane_id();
  st4f<E>(baseT + (c0 + (l & 15)) * ldT + r0 + 4 * (l >> 4), acc);
}

// Element offset of M[r][c] in a matrix of ncol columns kept as 4 x 16 blocks,
// each row-major and contiguous (64 elements: one 128-byte line for bf16),
// blocks in row-major order.  Four or eight consecutive columns of one row, and
// the same columns of four consecutive rows, fall into whole lines, so such a
// matrix can be read along its rows and, after a quad transpose, down its
// columns with every fetched line fully used.  The stored chunk states are
// h (Dk x Dv) in this layout: h[d][v] at st_blk(d, v, Dv).
__host__ __device__ constexpr int64_t st_blk(int r, int c, int ncol) {
  return ((int64_t)(r >> 2) * (ncol >> 4) + (c >> 4)) * 64 + ((r & 3) << 4) + (c & 15);
}

// ld_frag8 from a blocked matrix of DK columns: row v, columns k0 + 8g ..
// k0 + 8g + 7 (k0 a multiple of 16).
__device__ __forceinline__ Frag<bf16> ld_frag8_st(const bf16* base, int DK, int v, int k0) {
  const int g = lane_id() >> 4;
  Frag<bf16> f;
  f.v = *reinterpret_cast<const bf16x8*>(base + st_blk(v, k0 + 8 * g, DK));
  return f;
}
__device__ __forceinline__ Frag<float> ld_frag8_st(const float* base, int DK, int v, int k0) {
  const int g = lane_id() >> 4;
  const float* p = base + st_blk(v, k0 + 8 * g, DK);
  Frag<float> f;
  f.lo = *reinterpret_cast<const f32x4*>(p);
  f.hi = *reinterpret_cast<const f32x4*>(p + 4);
  return f;
}

// ld_fragC_q8_st split in two: the loads (issued early, kept in flight) and the
// quad transposes (once the data is needed).
template <class E> struct RawFrag;
template <> struct RawFrag<bf16> { uint32_t x0, x1, y0, y1; };
template <> struct RawFrag<float> { f32x4 lo, hi; };
template <class E>
__device__ __forceinline__ RawFrag<E> raw_fragC_q8_st(const E* base, int DK, int k0, int col0) {
  const int l = lane_id(), g = l >> 4, q = (l >> 2) & 3, b = l & 3;
  const E* p = base + st_blk(k0 + 8 * g + b, col0 + 4 * q, DK);
  RawFrag<E> r;
  if constexpr (std::is_same<E, bf16>::value) {
    typedef uint32_t u32x2 __attribute__((__vector_size__(8)));
    const u32x2 x = *reinterpret_cast<const u32x2*>(p), y = *reinterpret_cast<const u32x2*>(p + DK * 4);
    r.x0 = x[0]; r.x1 = x[1]; r.y0 = y[0]; r.y1 = y[1];
  } else {
    r.lo = *reinterpret_cast<const f32x4*>(p);
    r.hi = *reinterpret_cast<const f32x4*>(p + DK * 4);
  }
  return r;
}
__device__ __forceinline__ Frag<bf16> finish_frag(RawFrag<bf16> r) {
  typedef uint32_t u32x4 __attribute__((__vector_size__(16)));
  quad_transpose16(r.x0, r.x1);
  quad_transpose16(r.y0, r.y1);
  Frag<bf16> f;
  f.v = __builtin_bit_cast(bf16x8, u32x4{r.x0, r.x1, r.y0, r.y1});
  return f;
}
__device__ __forceinline__ Frag<float> finish_frag(const RawFrag<float>& r) {
  Frag<float> f;
  f.lo = quad_transpose(r.lo);
  f.hi = quad_transpose(r.hi);
  return f;
}

// ld_fragC_q in the contiguous k-slot order (pairs with ld_frag8), from a
// blocked chunk state: k-slots walk down key column
// col0 + lane%16 (col0 a multiple of 16) over value rows k0 + 8g .. k0 + 8g + 7
// (k0 a multiple of 8); each 4-row piece is one block row of 16 keys.
template <class E>
__device__ __forceinline__ Frag<E> ld_fragC_q8_st(const E* base, int DK, int k0, int col0);
template <>
__device__ __forceinline__ Frag<bf16> ld_fragC_q8_st<bf16>(const bf16* base, int DK, int k0, int col0) {
  const int l = lane_id(), g = l >> 4, q = (l >> 2) & 3, b = l & 3;
  const bf16* p = base + st_blk(k0 + 8 * g + b, col0 + 4 * q, DK);
  typedef uint32_t u32x2 __attribute__((__vector_size__(8)));
  typedef uint32_t u32x4 __attribute__((__vector_size__(16)));
  u32x2 x = *reinterpret_cast<const u32x2*>(p);
  u32x2 y = *reinterpret_cast<const u32x2*>(p + DK * 4);  // four rows down: the next block row
  uint32_t x0 = x[0], x1 = x[1], y0 = y[0], y1 = y[1];
  quad_transpose16(x0, x1);
  quad_transpose16(y0, y1);
  Frag<bf16> f;
  f.v = __builtin_bit_cast(bf16x8, u32x4{x0, x1, y0, y1});
  return f;
}
template <>
__device__ __forceinline__ Frag<float> ld_fragC_q8_st<float>(const float* base, int DK, int k0, int col0) {
  const int l = lane_id(), g = l >> 4, q = (l >> 2) & 3, b = l & 3;
  const float* p = base + st_blk(k0 + 8 * g + b, col0 + 4 * q, DK);
  Frag<float> f;
  f.lo = quad_transpose(*reinterpret_cast<const f32x4*>(p));
  f.hi = quad_transpose(*reinterpret_cast<const f32x4*>(p + DK * 4));
  return f;
}

// The inverse of ld_fragC_q: a fragment whose k-slots walk down column
// col0 + lane%16 (rows k0+4g.., k0+16+4g..) stored into a row-major E matrix as
// two quad-transposed 4-column row pieces.  All 64 lanes must take part.
template <class E, bool NTS = false>
__device__ __forceinline__ void st_fragC_q(E* base, int ld, int k0, int col0, const Frag<E>& f) {
  const int l = lane_id(), g = l >> 4, q = (l >> 2) & 3, b = l & 3;
  E* p = base + (k0 + 4 * g + b) * ld + col0 + 4 * q;
  if constexpr (sizeof(E) == 2) {
    typedef uint32_t u32x2 __attribute__((__vector_size__(8)));
    typedef uint32_t u32x4 __attribute__((__vector_size__(16)));
    const u32x4 v = __builtin_bit_cast(u32x4, f.v);
    uint32_t x0 = v[0], x1 = v[1], y0 = v[2], y1 = v[3];
    quad_transpose16(x0, x1);
    quad_transpose16(y0, y1);
    if constexpr (NTS) {
      st_out(reinterpret_cast<u32x2*>(p), u32x2{x0, x1});
      st_out(reinterpret_cast<u32x2*>(p + 16 * ld), u32x2{y0, y1});
    } else {
      *reinterpret_cast<u32x2*>(p) = u32x2{x0, x1};
      *reinterpret_cast<u32x2*>(p + 16 * ld) = u32x2{y0, y1};
    }
  } else {
    if constexpr (NTS) {
      st_out(reinterpret_cast<f32x4*>(p), quad_transpose(f.lo));
      st_out(reinterpret_cast<f32x4*>(p + 16 * ld), quad_transpose(f.hi));
    } else {
      *reinterpret_cast<f32x4*>(p) = quad_transpose(f.lo);
      *reinterpret_cast<f32x4*>(p + 16 * ld) = quad_transpose(f.hi);
    }
  }
}

// x - bf16(x), elementwise: what rounding x to bf16 drops (x = hi + residual,
// the residual itself rounded to bf16 when stored).
__device__ __forceinline__ f32x4 bf16_residual(const f32x4& x) {
  f32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = x[i] - (float)(bf16)x[i];
  return r;
}

// The C-layout piece (rows r0+4g .. r0+4g+3 of column lane%16) of a row-major
// E matrix with 16 columns, read as one 4-column row piece per lane and
// quad-transposed: load() issues the read, get() returns the values as fp32.
// All 64 lanes must take part in get().
template <class E> struct CPiece;
template <> struct CPiece<bf16> {
  uint32_t x0, x1;
  template <bool NTL = false>
  __device__ __forceinline__ void load(const bf16* blk, int r0) {
    const int l = lane_id(), g = l >> 4, q = (l >> 2) & 3, b = l & 3;
    typedef uint32_t u32x2 __attribute__((__vector_size__(8)));
    const u32x2* p = reinterpret_cast<const u32x2*>(blk + (r0 + 4 * g + b) * 16 + 4 * q);
    const u32x2 v = NTL ? __builtin_nontemporal_load(p) : *p;
    x0 = v[0];
    x1 = v[1];
  }
  __device__ __forceinline__ f32x4 get() {
    uint32_t a = x0, c = x1;
    quad_transpose16(a, c);
    const float v0 = __builtin_bit_cast(float, a << 16), v1 = __builtin_bit_cast(float, a & 0xFFFF0000u);
    const float v2 = __builtin_bit_cast(float, c << 16), v3 = __builtin_bit_cast(float, c & 0xFFFF0000u);
    return f32x4{v0, v1, v2, v3};
  }
};
template <> struct CPiece<float> {
  f32x4 v;
  template <bool NTL = false>
  __device__ __forceinline__ void load(const float* blk, int r0) {
    const int l = lane_id(), g = l >> 4, q = (l >> 2) & 3, b = l & 3;
    const f32x4* p = reinterpret_cast<const f32x4*>(blk + (r0 + 4 * g + b) * 16 + 4 * q);
    v = NTL ? __builtin_nontemporal_load(p) : *p;
  }
  __device__ __forceinline__ f32x4 get() const { return quad_transpose(v); }
};

// Four fp32 values of a C-layout column piece -> E, quad-transposed into a row
// piece and stored (4 consecutive columns of row `row`).
template <class E, bool NTS = false>
__device__ __forceinline__ void st4_transposed(E* p, const f32x4& v) {
  if constexpr (sizeof(E) == 2) {
    typedef uint32_t u32x2 __attribute__((__vector_size__(8)));
    u32x2 x = __builtin_bit_cast(u32x2, bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]});
    uint32_t x0 = x[0], x1 = x[1];
    quad_transpose16(x0, x1);
    if constexpr (NTS) st_out(reinterpret_cast<u32x2*>(p), u32x2{x0, x1});
    else *reinterpret_cast<u32x2*>(p) = u32x2{x0, x1};
  } else {
    if constexpr (NTS) st_out(reinterpret_cast<f32x4*>(p), quad_transpose(v));
    else *reinterpret_cast<f32x4*>(p) = quad_transpose(v);
  }
}

// Rows r0 .. r0 + 3 of column c0 + lane%16 (an accumulator tile's column
// piece, c0 a multiple of 16) into a blocked matrix of ncol columns (st_blk):
// quad-transposed first, so that the lane holds row r0 + lane%4 at columns
// c0 + 4 ((lane / 4) % 4) .. + 3 and stores them as one piece.  All 64 lanes
// must take part.
template <class E>
__device__ __forceinline__ void st_blk_row4(E* base, int r0, int c0, int ncol, const f32x4& x) {
  const int l = lane_id(), q = (l >> 2) & 3, b = l & 3;
  st4_transposed<E, true>(base + st_blk(r0 + b, c0 + 4 * q, ncol), x);
}

// acc + sum over the eight k-slots of a[j] * b[j] (bf16 pairs on the dot
// product unit, fp32 accumulation).
__device__ __forceinline__ float frag_dot(const Frag<bf16>& a, const Frag<bf16>& b, float acc) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  struct Pairs { bf16x2_t p[4]; };
  const Pairs pa = __builtin_bit_cast(Pairs, a.v), pb = __builtin_bit_cast(Pairs, b.v);
#pragma unroll
  for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_fdot2_f32_bf16(pa.p[i], pb.p[i], acc, false);
  return acc;
}
__device__ __forceinline__ float frag_dot(const Frag<float>& a, const Frag<float>& b, float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) acc += a.lo[i] * b.lo[i] + a.hi[i] * b.hi[i];
  return acc;
}

// Value of k-slot j of a fragment, as fp32.
__device__ __forceinline__ float frag_at(const Frag<bf16>& f, int j) { return (float)f.v[j]; }
__device__ __forceinline__ float frag_at(const Frag<float>& f, int j) { return j < 4 ? f.lo[j] : f.hi[j - 4]; }

// Wave-wide inclusive prefix sum (64 lanes).
__device__ __forceinline__ float wave_incl_scan(float x) {
  const int l = lane_id();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    float y = __shfl_up(x, o, 64);
    if (l >= o) x += y;
  }
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Row-major LDS leading dimensions: 4 extra elements per row stagger rows
// across LDS banks for the 8-/16-byte fragment reads.
template <class E> constexpr int ldpad(int n) { return n + 4; }

// Per-chunk work description, written by the plan kernel.
struct SegDesc {
  int n;        // sequence index
  int c_begin;  // first chunk (index within the sequence)
  int c_end;    // one past the last chunk
  int s;        // segment index within the sequence
};

struct SeqInfo {
  const int32_t* cu;   // device cu_seqlens [N+1] or nullptr for uniform length T
  int T;               // tokens per sequence when cu == nullptr
  int segc;            // chunks per segment (the plan's)
  __device__ __forceinline__ int64_t start(int n) const { return cu ? (int64_t)cu[n] : (int64_t)n * T; }
  __device__ __forceinline__ int len(int n) const { return cu ? cu[n + 1] - cu[n] : T; }
  // (sequence, chunk within it) of global chunk c: computed for sequences of
  // one length (no load in front of a workgroup's first requests), else the
  // plan's table
  __device__ __forceinline__ int2 chunk_of(const int2* tab, int c) const {
    if (cu) return tab[c];
    const int nch = max(1, (T + CH - 1) / CH);
    return make_int2(c / nch, c % nch);
  }
  // The plan's tables, computed the same way for sequences of one length
  // (ceil(T / CH) chunks each, cut into segments of segc chunks; an empty
  // sequence has one segment without chunks), so that no plan runs for them.
  __device__ __forceinline__ int nseg_per_seq() const {
    const int nch = (T + CH - 1) / CH;
    return nch == 0 ? 1 : (nch + segc - 1) / segc;
  }
  __device__ __forceinline__ SegDesc seg_of(const SegDesc* tab, int j) const {
    if (cu) return tab[j];
    const int nch = (T + CH - 1) / CH, ns = nseg_per_seq();
    const int n = j / ns, s = j % ns;
    return SegDesc{n, min(nch, s * segc), min(nch, (s + 1) * segc), s};
  }
  __device__ __forceinline__ int nseg_of(const int* seg_first, int n) const {
    return cu ? seg_first[n + 1] - seg_first[n] : nseg_per_seq();
  }
  __device__ __forceinline__ int64_t first_chunk(const int* chunk_first, int n) const {
    return cu ? chunk_first[n] : (int64_t)n * ((T + CH - 1) / CH);
  }
};

}  // namespace gdn
