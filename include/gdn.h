/*
 * gdn.h -- C ABI of the MI355X (gfx950) chunked Gated DeltaNet prefill library.
 *
 * Operation.  The pages this library follows ("Qwen's FlashQLA targets the
 * expensive bit of long-context AI", section "What happened"; "FlashQLA
 * resource", section 2 "What It Actually Is") describe the forward and backward
 * pass of Gated DeltaNet (GDN) chunked prefill.  They print no formula; the
 * computation is the published gated delta rule, per sequence and head:
 *
 *     S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,    S_0 = h0^T
 *     o_t = scale * S_t q_t,                                               hT = S_T^T
 *
 * with S a Dv x Dk matrix, evaluated chunk by chunk (64 tokens) in the exact
 * WY/UT form ("FlashQLA resource", section 3: an algebraic reformulation that
 * keeps full precision).  Long sequences with few heads are split into
 * segments that run side by side on one GPU; the exponential decay of the
 * gates bounds how far a segment boundary's state must be propagated
 * ("FlashQLA resource", section 3, gate-driven intra-card context parallelism;
 * section 5 for the backward pass).  The split changes the result by at most
 * 2^-24 of the norm of the state (or state gradient) at a segment boundary
 * carried across it, so a split and an unsplit run differ at fp32 round-off
 * level (the tests hold them to 1e-5 relative, elementwise).
 *
 * Layouts (row-major, last dimension contiguous, all pointers device memory
 * unless stated otherwise; every tensor pointer 16-byte aligned):
 *   q, k                [B, T, H, Dk]   dtype
 *   v, o                [B, T, H, Dv]   dtype
 *   beta                [B, T, H]       dtype
 *   g                   [B, T, H]       fp32, natural-log decay (<= 0 in the tested domain)
 *   h0, hT, dhT, dh0    [N, H, Dk, Dv]  fp32, h = S^T
 *   do, dq, dk, dv, dbeta   like o, q, k, v, beta; dg like g (fp32)
 * Variable-length batches: B == 1, sequences packed along T, described by
 * cu_seqlens (int32 [N+1], cu[0] = 0, non-decreasing, cu[N] = T).  The
 * recurrence restarts at every sequence start.  Without cu_seqlens, N = B.
 *
 * Supported: dtype GDN_BF16 with Dk, Dv in {64, 128}; GDN_F32 with Dk = Dv = 64.
 *
 * Ownership.  The caller owns every buffer, including the workspace, whose size
 * the *_workspace_size functions report for the same arguments.  The library
 * allocates no device memory and keeps no state besides a per-device cache of
 * the compute-unit count and a thread-local error string.
 *
 * Asynchrony.  Calls enqueue kernels on the caller's HIP stream and return
 * without synchronising.  Buffers must stay valid until the stream has passed
 * the call.  Two calls that share a workspace must be ordered on one stream.
 *
 * Errors.  All argument checks run before anything is enqueued: a call that
 * returns GDN_E_INVALID / GDN_E_UNSUPPORTED / GDN_E_WORKSPACE has written
 * nothing.  GDN_E_HIP reports a failed launch (the message carries HIP's
 * error string).  gdn_last_error() returns a description of the last non-OK
 * status on the calling thread.  Nothing throws or aborts across this ABI.
 * Non-finite inputs propagate; they are not detected.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 11

typedef enum {
  GDN_OK = 0,
  GDN_E_INVALID = 1,     /* null pointer, bad size, misalignment, bad cu_seqlens, ... */
  GDN_E_UNSUPPORTED = 2, /* dtype / head-size combination not built */
  GDN_E_WORKSPACE = 3,   /* workspace missing or smaller than *_workspace_size */
  GDN_E_HIP = 4          /* a HIP launch or query failed */
} gdn_status;

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

/* Arguments shared by forward and backward. */
typedef struct {
  int32_t dtype;               /* gdn_dtype of q, k, v, beta (and o, do, dq, dk, dv, dbeta) */
  int32_t B, T, H, Dk, Dv;     /* with cu_seqlens: B == 1 and T = total packed tokens */
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const void* beta;
  const float* h0;             /* nullable: zero initial state */
  float scale;                 /* output scale; the usual choice is Dk^-0.5 */
  const int32_t* cu_seqlens;   /* nullable device pointer [N+1] */
  const int32_t* cu_seqlens_host; /* host copy of the same [N+1]; required with cu_seqlens.  The
                                  host copy sizes the work and the workspace; the kernels read
                                  the device copy.  If the device copy starts at a nonzero
                                  value, ends at a value other than T, has a negative length or
                                  gives other chunk or segment totals than the host copy, the
                                  call writes no output (o, hT and the gradients are left as
                                  they were) and reads nothing past its buffers; the status is
                                  still GDN_OK, since nothing is checked on the host side. */
  int32_t num_seqs;            /* N: len(cu_seqlens) - 1, or B when cu_seqlens is NULL */
  int32_t cp_mode;             /* intra-card sequence splitting: 0 = automatic,
                                  -1 = off (one segment per sequence and head),
                                  k > 0 = segments of k chunks (64 tokens each) */
  void* workspace;             /* device scratch of at least workspace_bytes */
  size_t workspace_bytes;
  /* Optional input pre-processing inside the kernels (0 = off):
   *   qk_norm:  q and k are raw; each (token, head) vector is divided by
   *             sqrt(|x|^2 + 1e-6) before use;
   *   gate_act: g and beta hold logits a, b; the kernels use
   *             g = -gate_scale[h] * softplus(a) and beta = sigmoid(b).
   * The backward then returns dq, dk, dg, dbeta with respect to these raw
   * inputs.  Outputs o, hT and the states are unchanged in meaning. */
  int32_t qk_norm;
  int32_t gate_act;
  const float* gate_scale;     /* nullable [H] fp32 (1 when NULL); only with gate_act */
} gdn_common_args;

typedef struct {
  gdn_common_args a;
  void* o;                     /* [B,T,H,Dv] dtype, written */
  float* hT;                   /* nullable [N,H,Dk,Dv] fp32, written */
  void* h_save;                /* nullable, 16-byte aligned, gdn_chunk_states_bytes(&a) bytes: the
                                  state at the start of every 64-token chunk, written for a later
                                  gdn_chunk_bwd (layout below) */
  float* t_save;               /* nullable, 16-byte aligned, gdn_chunk_t_bytes(&a) bytes: every
                                  chunk's matrix T (below), written for a later gdn_chunk_bwd */
} gdn_fwd_args;

typedef struct {
  gdn_common_args a;           /* the forward's inputs; the backward recomputes what it needs */
  const void* h_saved;         /* nullable: h_save of a gdn_chunk_fwd call on the same inputs;
                                  given, the backward reads the chunk states instead of
                                  recomputing them (no forward replay) */
  const float* t_saved;        /* nullable: t_save of a gdn_chunk_fwd call on the same inputs;
                                  given, the backward reads every chunk's T instead of solving
                                  for it once itself */
  const void* do_;             /* [B,T,H,Dv] dtype: gradient of o */
  const float* dhT;            /* nullable [N,H,Dk,Dv]: gradient of hT (NULL = zero) */
  void* dq;                    /* [B,T,H,Dk] dtype, written */
  void* dk;                    /* [B,T,H,Dk] dtype, written */
  void* dv;                    /* [B,T,H,Dv] dtype, written */
  void* dbeta;                 /* [B,T,H] dtype, written */
  float* dg;                   /* [B,T,H] fp32, written */
  float* dh0;                  /* nullable [N,H,Dk,Dv] fp32, written */
} gdn_bwd_args;

/* Bytes of device workspace gdn_chunk_fwd / gdn_chunk_bwd need for these
 * arguments (pointers other than cu_seqlens_host are not read, except that the
 * forward needs less when t_save is non-NULL and the backward less when
 * h_saved or t_saved is).  Returns 0 and sets the error string when the
 * arguments are invalid. */
size_t gdn_chunk_fwd_workspace_size(const gdn_fwd_args* args);
size_t gdn_chunk_bwd_workspace_size(const gdn_bwd_args* args);

/* Bytes of the saved chunk states (h_save / h_saved) for these arguments:
 * C * H * (Dk * Dv + 64 * Dv) elements of the input dtype (bf16: C * H *
 * (Dk * Dv + 2 * 64 * Dv)), C = sum over sequences of ceil(len / 64).  The
 * first C * H * Dk * Dv elements are the
 * states: state (c, h) is h (= S^T, Dk x Dv) at the start of chunk c (chunks
 * numbered sequence after sequence), rounded to the dtype, stored at element
 * offset (c * H + h) * Dk * Dv in 4 x 16 blocks: h[i][j] (key i, value j) sits at
 *     ((i / 4) * (Dv / 16) + j / 16) * 64 + (i % 4) * 16 + j % 16
 * (each block row-major and contiguous, blocks in row-major order), so that
 * the state can be read both along and across its rows in whole cache lines.
 * Then, at element offset C * H * Dk * Dv + (c * H + h) * 64 * Dv, each
 * chunk's value residual U = T (diag(beta) V - diag(beta Gam) K h), 64 x Dv
 * (h the chunk-start state, Gam_r = exp(G_r), T and G as for
 * gdn_chunk_t_bytes; rows past a sequence's end are zero), stored as Dv / 16
 * column blocks of 64 x 16, each row-major and contiguous: U[r][j] sits at
 *     (j / 16) * 1024 + r * 16 + j % 16.
 * For bf16 a third part follows, at element offset C * H * (Dk * Dv + 64 * Dv),
 * laid out like U: bf16(U - bf16(U)), the residual of U's rounding (the
 * backward's decay gradient takes U to about 16 bits).
 * Returns 0 and sets the error string for invalid arguments (and returns 0
 * without error when there are no tokens). */
size_t gdn_chunk_states_bytes(const gdn_common_args* a);

/* Bytes of the saved chunk matrices (t_save / t_saved): C * H * (64 * 64 + 324)
 * fp32 values, C as above.  Entry (c, h), 16 KiB at element offset
 * (c * H + h) * 4096, holds the 64 x 64 row-major lower-triangular matrix
 *     T = (I + diag(beta) strict_lower((K K^T) * D))^-1,   D[r][i] = exp(G_r - G_i),
 * of chunk c and head h (K: the chunk's 64 keys as rows, after the optional
 * normalisation; beta after the optional activation; G_r the running sum of
 * g over the chunk up to row r), the inverse of the chunk's unit lower-
 * triangular system in the WY/UT form ("FlashQLA resource", section 3).  Rows
 * past a sequence's end have beta = 0 (rows of the identity).  For fp32 inputs
 * the entry is T in fp32; for bf16 inputs it is two 64 x 64 row-major bf16
 * planes, T rounded to bf16 and then the residual T - that value rounded to
 * bf16 (their sum carries T to about 16 significant bits; the forward and
 * reverse state chains read the first plane only).  After the
 * C * H matrices, at element offset C * H * 4096 + (c * H + h) * 324, the
 * chunk's scalar record (g, beta after the optional activation; rows past a
 * sequence end have g = beta = 0): G_r (64 values), exp(G_r), exp(G_63 - G_r),
 * beta_r, beta_r exp(G_r), then Lambda = sum_r [g_r + log max(1, |1 - beta_r
 * |k_r|^2|)] (the log-bound on the chunk's state transition), exp(G_63), 0, 0.
 * Returns 0 and sets the error string for invalid arguments (and returns 0
 * without error when there are no tokens). */
size_t gdn_chunk_t_bytes(const gdn_common_args* a);

/* Forward: o and (optionally) hT, the chunk states and the chunk matrices T
 * -- the chunked prefill forward pass ("FlashQLA resource", section 2 "What It
 * Actually Is", and section 3 for the reformulated chunk form and the
 * intra-card splitting; "Qwen's FlashQLA targets the expensive bit of
 * long-context AI", section "What happened").  stream is a hipStream_t (NULL =
 * default stream). */
gdn_status gdn_chunk_fwd(const gdn_fwd_args* args, void* stream);

/* Bytes of the scratch array gdn_chunk_fwd_noalloc uses in place of a workspace. */
#define GDN_NOALLOC_SCRATCH_BYTES (64u << 20)

/* gdn_chunk_fwd without a workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  Same arguments and results as gdn_chunk_fwd, except that
 * a.workspace / a.workspace_bytes are ignored: the work tables (and, when
 * t_save is NULL, every chunk's T and scalar record) go to a scratch array
 * of GDN_NOALLOC_SCRATCH_BYTES (64 MiB) that the library holds on each device
 * it runs on, from its load until the process ends.  Arguments whose
 * gdn_chunk_fwd_workspace_size exceeds that size are rejected with
 * GDN_E_WORKSPACE before anything is enqueued (without t_save that is about
 * 3,700 chunk-heads, e.g. 16 heads of 15,000 tokens; with t_save the tables
 * alone, a few bytes per chunk).  The call allocates nothing: no hipMalloc,
 * hipFree or allocating library routine, and no timing events
 * (gdn_profile_enable does not apply to it).  Every call on one device shares
 * that device's scratch, which keeps the last call's contents (the forward
 * reads nothing it has not written in the same call): calls that overlap on
 * one device -- on different streams, or from several threads without
 * ordering -- race and give undefined results; order them on one stream.
 * The first call on a device looks the scratch address up (not under graph
 * capture on that device, which forbids that query in some runtimes: make one
 * call outside capture first). */
gdn_status gdn_chunk_fwd_noalloc(const gdn_fwd_args* args, void* stream);

/* Backward: gradients of <do, o> + <dhT, hT> with respect to q, k, v, beta, g
 * and (optionally) h0 -- the matching backward pass ("FlashQLA resource",
 * section 2, and section 5 for its intra-card splitting; "Qwen's FlashQLA
 * targets the expensive bit of long-context AI", section "What happened").  It
 * recomputes the forward states from the inputs unless h_saved provides them,
 * and solves for each chunk's T once unless t_saved provides them.  stream as
 * for gdn_chunk_fwd. */
gdn_status gdn_chunk_bwd(const gdn_bwd_args* args, void* stream);

/* One recurrent decode step: every listed sequence takes one new token and
 * advances its state in place.  The pages present the kernels as serving
 * training and inference ("Qwen's FlashQLA targets the expensive bit of
 * long-context AI", section "What happened"; "FlashQLA resource", section 4);
 * after a prefill (gdn_chunk_fwd with hT) the state continues token by token
 * with the same recurrence, per sequence n and head:
 *     S <- exp(g) S (I - beta k k^T) + beta v k^T,      o = scale * S q
 * with the state stored as h = S^T (fp32 [Dk, Dv], as hT of the forward).
 *
 * Layouts (row-major, last dimension contiguous, device memory, every pointer
 * 16-byte aligned except g and beta):
 *   q, k [N, H, Dk], v, o [N, H, Dv] dtype;  g [N, H] fp32;  beta [N, H] dtype;
 *   state [num_slots, H, Dk, Dv] fp32, read and written in place.
 * state_idx (nullable int32 [N], device): sequence n uses slot state_idx[n];
 * an index outside [0, num_slots) marks a padding entry, which is skipped
 * (its o is not written).  NULL means slot n (num_slots >= N).  Two
 * sequences of one call must not share a slot.
 * Supported: bf16 and fp32 with Dk, Dv in {64, 128}.  Errors as for the chunk
 * calls (checked before anything is enqueued); asynchronous on `stream`. */
typedef struct {
  int32_t dtype;               /* gdn_dtype of q, k, v, beta, o */
  int32_t N, H, Dk, Dv;
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const void* beta;
  float scale;
  float* state;
  const int32_t* state_idx;
  int32_t num_slots;
  void* o;
  int32_t qk_norm;             /* as in gdn_common_args */
  int32_t gate_act;
  const float* gate_scale;
} gdn_decode_args;

gdn_status gdn_decode_step(const gdn_decode_args* args, void* stream);

/* Per-kernel timing, for benchmarks (off by default).  While enabled, every
 * kernel the library launches is bracketed by a pair of HIP events recorded on
 * the call's stream.  gdn_profile_read waits for the recorded events, adds
 * their elapsed times to per-kernel totals and writes up to `max` entries:
 * the kernel's name (static storage), total milliseconds and launch count.
 * It returns the number of distinct kernels seen since the last reset (or -1
 * on a HIP error).  gdn_profile_reset clears the totals.  Not thread-safe with
 * respect to concurrent calls on other threads. */
int gdn_profile_enable(int on);
int gdn_profile_read(int max, const char** names, double* ms, int* launches);
void gdn_profile_reset(void);

/* Thread-local description of the last non-OK status ("" if none). */
const char* gdn_last_error(void);

/* GDN_ABI_VERSION of the library. */
int gdn_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* GDN_H */
