// gdn_internal.h -- host/device parameter blocks and launchers (not part of the ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_device.h"

namespace gdn {

// Forward chunk loop (also the backward's forward-state replay).
// Optional input pre-processing applied inside the kernels: q and k divided by
// their L2 norm over the head dimension (qk_norm), and gate / beta given as
// logits (gate_act): g = -gate_scale[h] softplus(a), beta = sigmoid(b).
struct PrepParams {
  int qk_norm;
  int gate_act;
  const float* gate_scale;  // nullable [H]: 1
};

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const void* beta;
  const float* h0;         // nullable
  void* o;                 // nullable: replay mode writes no output
  float* hT;               // nullable
  float scale;
  int H;
  SeqInfo seq;
  const SegDesc* segs;     // [total segments]
  const int* seg_first;    // [N+1]
  const int* chunk_first;  // [N+1]
  void* hs;                // nullable: [total chunks][H] chunk start states h, Dk x Dv in st_blk order (dtype)
  void* us;                // nullable: [total chunks][H][DV/16][CH][16] U = Ut - W h of each chunk in 16-column blocks (dtype)
  void* ulo;               // nullable (bf16 only, with us): U - bf16(U) rounded to bf16, laid out as us
  // [total chunks][H][CH][CH] fp32 row-major T = (I + diag(beta) A)^-1 of each chunk
  const float* t_in;
  const float* rec;        // [total chunks][H][RECF] scalar records
  PrepParams prep;
};

// Scalar record of a chunk (fp32, RECF values, 16-byte multiple), written by
// the T solve beside T and read by the chunk chains in place of g and beta:
//   [0, 64)    gam_r = sum_{i<=r} g_i         [64, 128)  Gam_r = exp(gam_r)
//   [128, 192) ek_r = exp(gam_63 - gam_r)      [192, 256) beta_r
//   [256, 320) bg_r = beta_r Gam_r             320: Lambda_c, 321: exp(gam_63), 322..323: 0
// (g, beta after the optional activation; rows past a sequence end have g = 0,
// beta = 0).  Lambda_c = sum_r [g_r + log max(1, |1 - beta_r |k_r|^2|)] is the
// chunk's log-bound on the norm of its state transition.
constexpr int RECF = 5 * CH + 4;

// Slots per chunk and head of the partial row terms e_r (RevParams::ep): one
// per wave of the reverse chain (at most eight).
constexpr int EPW = 8;

// Every chunk's T = (I + diag(beta) strict_lower(K K^T * D))^-1, chunk-parallel.
struct TSolveParams {
  const void* k;
  const float* g;
  const void* beta;
  float* t_out;            // [total chunks][H][CH][CH] fp32 row-major
  float* rec_out;          // [total chunks][H][RECF] scalar records
  int H;
  SeqInfo seq;
  const int2* chunk_tab;   // [total chunks] (sequence, chunk index within it)
  PrepParams prep;
};

// Reverse state-gradient chain of the backward.
struct RevParams {
  const void* q;
  const void* k;
  const float* g;
  const void* beta;
  const void* dout;
  const float* dhT;        // nullable
  float* dh0;              // nullable
  float scale;
  int H;
  SeqInfo seq;
  const SegDesc* segs;
  const int* seg_first;
  const int* chunk_first;
  void* dhs;               // [total chunks][H] gradient at each chunk END, Dk x Dv, st_blk order (dtype)
  const float* t_in;       // chunk matrices T (as FwdParams)
  const float* rec;        // scalar records (as FwdParams)
  // Each chunk's U (us, and for bf16 its rounding residual ulo; layout as
  // FwdParams) and, written here, the row terms
  //   e_r = exp(gam_last - gam_r) u_r . (dS' k_r)
  // of the decay gradient, per wave of this kernel: ep[chunk][H][EPW][CH], the
  // partial sums over each wave's value columns (the gradient kernel adds them)
  const void* us;
  const void* ulo;
  float* ep;
  PrepParams prep;
};

// Chunk-parallel gradients of the backward.
struct GradParams {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const void* beta;
  const void* dout;
  const void* hs;          // chunk start states
  const void* dhs;         // chunk end state gradients
  const void* us;          // each chunk's U = Ut - W h ([total chunks][H][DV/16][CH][16] column blocks, dtype)
  const float* t_in;       // chunk matrices T (as FwdParams)
  const float* rec;        // scalar records (as FwdParams)
  const float* ep;         // per-wave partial row terms e_r of the reverse chain (RevParams)
  void* dq;
  void* dk;
  void* dv;
  void* dbeta;
  float* dg;
  float scale;
  int H;
  SeqInfo seq;
  const int2* chunk_tab;   // [total chunks] (sequence, chunk index within it)
  PrepParams prep;
  int nwg;                 // compute units (workgroups resident at once: one per compute unit)
};

// One recurrent decode step: N sequences x H heads, one token each.
struct DecodeParams {
  const void* q;              // [N, H, DK]
  const void* k;              // [N, H, DK]
  const void* v;              // [N, H, DV]
  const float* g;             // [N, H]
  const void* beta;           // [N, H]
  float* state;               // [num_slots, H, DK, DV] fp32 h = S^T, updated in place
  const int32_t* state_idx;   // nullable [N]: state slot of sequence n (out of range: skipped)
  int num_slots;
  void* o;                    // [N, H, DV]
  float scale;
  int N, H;
  PrepParams prep;
};

hipError_t launch_plan(SeqInfo seq, int N, int segc, int total_tokens, int nchunk_cap, int nseg_cap,
                       int* chunk_first, int* seg_first, SegDesc* segs, int2* chunk_tab, hipStream_t st);
hipError_t launch_tsolve(int dtype, int DK, const TSolveParams& p, int nchunk_total, hipStream_t st);
hipError_t launch_fwd(int dtype, int DK, int DV, const FwdParams& p, int nseg_total, hipStream_t st);
hipError_t launch_rev(int dtype, int DK, int DV, const RevParams& p, int nseg_total, hipStream_t st);
hipError_t launch_grad(int dtype, int DK, int DV, const GradParams& p, int nchunk_total, hipStream_t st);
hipError_t launch_decode(int dtype, int DK, int DV, const DecodeParams& p, hipStream_t st);

}  // namespace gdn
