// gdn_api.hip -- host side of the C ABI declared in include/gdn.h:
// argument validation, the segment plan's sizes, workspace layout and the
// launch sequence on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "gdn.h"
#include "gdn_internal.h"

namespace {

thread_local std::string g_err;

gdn_status fail(gdn_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

constexpr int CHUNK = gdn::CH;

size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

// Compute units of the current device, cached per device.
int cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

struct Plan {
  int N = 0;
  int nchunk = 0;       // total chunks over all sequences
  int nseg = 0;         // total segments over all sequences
  int segc = 1;         // chunks per segment
  bool cp = false;      // some sequence has more than one segment
  // workspace offsets (bytes)
  size_t o_chunk_first = 0, o_seg_first = 0, o_segs = 0, o_chunk_tab = 0;
  size_t o_hs = 0, o_us = 0, o_ulo = 0, o_dhs = 0, o_ts = 0, o_ep = 0, total = 0;
};

bool supported(int dtype, int Dk, int Dv) {
  if (dtype == GDN_BF16) return (Dk == 64 || Dk == 128) && (Dv == 64 || Dv == 128);
  if (dtype == GDN_F32) return Dk == 64 && Dv == 64;
  return false;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

gdn_status check_prep(int qk_norm, int gate_act, const float* gate_scale) {
  if ((qk_norm != 0 && qk_norm != 1) || (gate_act != 0 && gate_act != 1))
    return fail(GDN_E_INVALID, "qk_norm and gate_act must be 0 or 1");
  if (gate_scale && !gate_act) return fail(GDN_E_INVALID, "gate_scale is only used with gate_act");
  if (!aligned(gate_scale, 4)) return fail(GDN_E_INVALID, "gate_scale misaligned");
  return GDN_OK;
}

gdn_status check_common(const gdn_common_args& a) {
  if (a.dtype != GDN_F32 && a.dtype != GDN_BF16) return fail(GDN_E_UNSUPPORTED, "unknown dtype %d", a.dtype);
  if (a.B < 1 || a.T < 0 || a.H < 1 || a.Dk < 1 || a.Dv < 1)
    return fail(GDN_E_INVALID, "bad sizes B=%d T=%d H=%d Dk=%d Dv=%d", a.B, a.T, a.H, a.Dk, a.Dv);
  if (!supported(a.dtype, a.Dk, a.Dv))
    return fail(GDN_E_UNSUPPORTED, "unsupported combination dtype=%d Dk=%d Dv=%d", a.dtype, a.Dk, a.Dv);
  const long long tokens = (long long)a.B * a.T;
  if (tokens * a.H * std::max(a.Dk, a.Dv) >= (1LL << 40)) return fail(GDN_E_INVALID, "problem too large");
  if (tokens > 0) {
    if (!a.q || !a.k || !a.v || !a.g || !a.beta) return fail(GDN_E_INVALID, "null input pointer");
    if (!aligned(a.q, 16) || !aligned(a.k, 16) || !aligned(a.v, 16))
      return fail(GDN_E_INVALID, "q, k and v must be 16-byte aligned");
    if (!aligned(a.g, 4) || !aligned(a.beta, a.dtype == GDN_F32 ? 4 : 2))
      return fail(GDN_E_INVALID, "g / beta misaligned");
  }
  if (!aligned(a.h0, 4)) return fail(GDN_E_INVALID, "h0 misaligned");
  if (a.cu_seqlens) {
    if (a.B != 1) return fail(GDN_E_INVALID, "cu_seqlens requires B == 1 (got %d)", a.B);
    if (!a.cu_seqlens_host) return fail(GDN_E_INVALID, "cu_seqlens needs its host copy cu_seqlens_host");
    if (a.num_seqs < 1) return fail(GDN_E_INVALID, "num_seqs must be >= 1 with cu_seqlens");
    const int32_t* cu = a.cu_seqlens_host;
    if (cu[0] != 0) return fail(GDN_E_INVALID, "cu_seqlens[0] must be 0");
    for (int n = 0; n < a.num_seqs; ++n)
      if (cu[n + 1] < cu[n]) return fail(GDN_E_INVALID, "cu_seqlens must be non-decreasing (index %d)", n);
    if (cu[a.num_seqs] != a.T) return fail(GDN_E_INVALID, "cu_seqlens[N] = %d != T = %d", cu[a.num_seqs], a.T);
  } else if (a.cu_seqlens_host) {
    return fail(GDN_E_INVALID, "cu_seqlens_host given without cu_seqlens");
  } else if (a.num_seqs != a.B) {
    return fail(GDN_E_INVALID, "num_seqs (%d) must equal B (%d) without cu_seqlens", a.num_seqs, a.B);
  }
  if (a.cp_mode < -1) return fail(GDN_E_INVALID, "cp_mode must be -1, 0 or a positive chunk count");
  return check_prep(a.qk_norm, a.gate_act, a.gate_scale);
}

gdn::PrepParams prep_of(int qk_norm, int gate_act, const float* gate_scale) {
  gdn::PrepParams pp;
  pp.qk_norm = qk_norm;
  pp.gate_act = gate_act;
  pp.gate_scale = gate_scale;
  return pp;
}

// Segment length, totals and workspace layout.  `bwd` adds the backward's arrays
// (without the chunk states when the caller provides them: `saved`).  `t_given`:
// the caller provides (forward: takes) the chunk matrices T, which otherwise live
// in the workspace (solved first, read by every later kernel).
Plan make_plan(const gdn_common_args& a, bool bwd, int cus, bool saved = false, bool t_given = false) {
  Plan p;
  p.N = a.num_seqs;
  std::vector<int> nch(p.N);
  long long total = 0;
  int maxc = 0;
  for (int n = 0; n < p.N; ++n) {
    const int len = a.cu_seqlens ? a.cu_seqlens_host[n + 1] - a.cu_seqlens_host[n] : a.T;
    nch[n] = (len + CHUNK - 1) / CHUNK;
    total += nch[n];
    maxc = std::max(maxc, nch[n]);
  }
  p.nchunk = (int)total;
  if (a.cp_mode == -1) {
    p.segc = std::max(1, maxc);
  } else if (a.cp_mode > 0) {
    p.segc = a.cp_mode;
  } else {
    // Automatic: aim for about one workgroup per compute unit, but never cut
    // segments shorter than 8 chunks -- each segment but a sequence's first
    // (last, in the reverse chain) runs a few lead-in chunks before its own
    // (the gate-decay horizon).
    const long long work = total * a.H;
    const long long per = (work + cus - 1) / std::max(1, cus);
    p.segc = (int)std::max<long long>(8, per);
    p.segc = std::max(1, std::min(p.segc, std::max(1, maxc)));
    // Sequences of several lengths round up to more workgroups than compute
    // units, and the chains then run in two rounds.  Among longer segments,
    // take the one that minimises rounds x chunks per segment (the chain
    // time of the slowest compute unit), when there are only a few rounds.
    const int ncu = std::max(1, cus);
    auto rounds = [&](int sc) {
      long long w = 0;
      for (int n = 0; n < p.N; ++n) w += nch[n] == 0 ? 1 : (nch[n] + sc - 1) / sc;
      return (w * a.H + ncu - 1) / ncu;
    };
    const long long r0 = rounds(p.segc);
    if (r0 > 1 && r0 <= 8) {
      long long best = r0 * p.segc;
      int bestc = p.segc;
      for (long long r = r0 - 1; r >= 1; --r) {
        // the shortest segment length (up to the longest sequence) with at most r rounds
        int lo = bestc, hi = std::max(1, maxc);
        if (rounds(hi) > r) break;
        while (lo < hi) {
          const int mid = lo + (hi - lo) / 2;
          if (rounds(mid) <= r) hi = mid;
          else lo = mid + 1;
        }
        if (r * lo < best) { best = r * lo; bestc = lo; }
      }
      p.segc = bestc;
    }
  }
  long long nseg = 0;
  for (int n = 0; n < p.N; ++n) nseg += nch[n] == 0 ? 1 : (nch[n] + p.segc - 1) / p.segc;
  p.nseg = (int)nseg;
  p.cp = p.nseg > p.N;
  const size_t SS = (size_t)a.Dk * a.Dv;
  const size_t esz = a.dtype == GDN_BF16 ? 2 : 4;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align_up(bytes); return o; };
  p.o_chunk_first = take(sizeof(int) * (p.N + 1));
  p.o_seg_first = take(sizeof(int) * (p.N + 1));
  p.o_segs = take(sizeof(gdn::SegDesc) * p.nseg);
  p.o_chunk_tab = take(sizeof(int2) * std::max(1, p.nchunk));
  // T of every chunk, then every chunk's scalar record
  const size_t tbytes = sizeof(float) * (CHUNK * CHUNK + gdn::RECF) * (size_t)std::max(1, p.nchunk) * a.H;
  if (!bwd && !t_given) p.o_ts = take(tbytes);
  if (bwd) {
    if (!saved) {
      p.o_hs = take(esz * SS * (size_t)std::max(1, p.nchunk) * a.H);
      p.o_us = take(esz * CHUNK * (size_t)a.Dv * std::max(1, p.nchunk) * a.H);
      if (a.dtype == GDN_BF16) p.o_ulo = take(esz * CHUNK * (size_t)a.Dv * std::max(1, p.nchunk) * a.H);
    }
    // the chunk matrices T, solved once and read by the later kernels
    if (!t_given) p.o_ts = take(tbytes);
    p.o_dhs = take(esz * SS * (size_t)std::max(1, p.nchunk) * a.H);
    // the reverse chain's per-wave row terms of the decay gradient
    p.o_ep = take(sizeof(float) * gdn::EPW * CHUNK * (size_t)std::max(1, p.nchunk) * a.H);
  }
  p.total = off;
  return p;
}

template <class T>
T* at(void* base, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(base) + off); }

// ---------------------------------------------------------------- per-kernel timing
struct ProfRec { const char* name; hipEvent_t a, b; };
struct ProfTotal { const char* name; double ms; int n; };
bool g_prof = false;
std::vector<ProfRec> g_pending;
std::vector<hipEvent_t> g_pool;
std::vector<ProfTotal> g_totals;

hipEvent_t prof_event() {
  if (!g_pool.empty()) { hipEvent_t e = g_pool.back(); g_pool.pop_back(); return e; }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Set while an allocation-free call runs on this thread: no timing events are
// created for it.
thread_local bool t_noalloc = false;

// Launch through f() on stream s, bracketed by events when timing is enabled.
template <class F>
hipError_t timed(const char* name, hipStream_t s, F f) {
  if (!g_prof || t_noalloc) return f();
  ProfRec r{name, prof_event(), prof_event()};
  const bool ok_a = r.a && hipEventRecord(r.a, s) == hipSuccess;
  hipError_t e = f();
  const bool ok_b = r.b && hipEventRecord(r.b, s) == hipSuccess;
  if (ok_a && ok_b) {
    g_pending.push_back(r);
  } else {  // an unrecorded pair is not timed; its events go back to the pool
    if (r.a) g_pool.push_back(r.a);
    if (r.b) g_pool.push_back(r.b);
  }
  return e;
}

gdn_status hip_fail(hipError_t e, const char* what) {
  return fail(GDN_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

gdn::SeqInfo seq_info(const gdn_common_args& a, int segc) {
  gdn::SeqInfo s;
  s.cu = a.cu_seqlens;
  s.T = a.T;
  s.segc = segc;
  return s;
}

// The plan kernel fills the work tables from the device cu_seqlens; for
// sequences of one length (no cu_seqlens) the kernels compute the same tables
// themselves and it does not run.
hipError_t plan_tables(const gdn_common_args& a, const Plan& pl, const gdn::SeqInfo& sq, void* ws, hipStream_t s) {
  if (!sq.cu) return hipSuccess;
  return timed("plan", s, [&] {
    return gdn::launch_plan(sq, pl.N, pl.segc, a.T, pl.nchunk, pl.nseg, at<int>(ws, pl.o_chunk_first),
                            at<int>(ws, pl.o_seg_first), at<gdn::SegDesc>(ws, pl.o_segs),
                            at<int2>(ws, pl.o_chunk_tab), s);
  });
}

long long count_chunks(const gdn_common_args& a) {
  long long chunks = 0;
  for (int n = 0; n < a.num_seqs; ++n) {
    const int len = a.cu_seqlens ? a.cu_seqlens_host[n + 1] - a.cu_seqlens_host[n] : a.T;
    chunks += (len + CHUNK - 1) / CHUNK;
  }
  return chunks;
}

// The saved-states buffer: the chunk states, then every chunk's U, then (bf16)
// every chunk's U rounding residual.
size_t states_part_bytes(const gdn_common_args& a) {
  return (size_t)count_chunks(a) * a.H * a.Dk * a.Dv * (a.dtype == GDN_BF16 ? 2 : 4);
}
size_t u_part_bytes(const gdn_common_args& a) {
  return (size_t)count_chunks(a) * a.H * CHUNK * a.Dv * (a.dtype == GDN_BF16 ? 2 : 4);
}

}  // namespace

extern "C" {

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

int gdn_profile_enable(int on) {
  const int was = g_prof ? 1 : 0;
  g_prof = on != 0;
  return was;
}

void gdn_profile_reset(void) {
  for (ProfRec& r : g_pending) {
    (void)hipEventSynchronize(r.b);
    g_pool.push_back(r.a);
    g_pool.push_back(r.b);
  }
  g_pending.clear();
  g_totals.clear();
}

int gdn_profile_read(int max, const char** names, double* ms, int* launches) {
  int rc = 0;
  for (ProfRec& r : g_pending) {
    float t = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&t, r.a, r.b) != hipSuccess) rc = -1;
    ProfTotal* tot = nullptr;
    for (ProfTotal& x : g_totals)
      if (std::strcmp(x.name, r.name) == 0) tot = &x;
    if (!tot) { g_totals.push_back({r.name, 0.0, 0}); tot = &g_totals.back(); }
    tot->ms += t;
    tot->n += 1;
    g_pool.push_back(r.a);
    g_pool.push_back(r.b);
  }
  g_pending.clear();
  if (rc) { fail(GDN_E_HIP, "profile: event query failed"); return -1; }
  for (int i = 0; i < (int)g_totals.size() && i < max; ++i) {
    if (names) names[i] = g_totals[i].name;
    if (ms) ms[i] = g_totals[i].ms;
    if (launches) launches[i] = g_totals[i].n;
  }
  return (int)g_totals.size();
}

const char* gdn_last_error(void) { return g_err.c_str(); }

size_t gdn_chunk_fwd_workspace_size(const gdn_fwd_args* args) {
  if (!args) { fail(GDN_E_INVALID, "null args"); return 0; }
  if (check_common(args->a) != GDN_OK) return 0;
  return make_plan(args->a, false, cu_count(), false, args->t_save != nullptr).total;
}

size_t gdn_chunk_bwd_workspace_size(const gdn_bwd_args* args) {
  if (!args) { fail(GDN_E_INVALID, "null args"); return 0; }
  if (check_common(args->a) != GDN_OK) return 0;
  return make_plan(args->a, true, cu_count(), args->h_saved != nullptr, args->t_saved != nullptr).total;
}

size_t gdn_chunk_states_bytes(const gdn_common_args* a) {
  if (!a) { fail(GDN_E_INVALID, "null args"); return 0; }
  if (check_common(*a) != GDN_OK) return 0;
  return states_part_bytes(*a) + u_part_bytes(*a) * (a->dtype == GDN_BF16 ? 2 : 1);
}

size_t gdn_chunk_t_bytes(const gdn_common_args* a) {
  if (!a) { fail(GDN_E_INVALID, "null args"); return 0; }
  if (check_common(*a) != GDN_OK) return 0;
  return (size_t)count_chunks(*a) * a->H * (CHUNK * CHUNK + gdn::RECF) * sizeof(float);
}

}  // extern "C"

namespace {

// Checks of the forward's own arguments (beyond check_common).
gdn_status check_fwd(const gdn_fwd_args* args) {
  if (!args) return fail(GDN_E_INVALID, "null args");
  const gdn_common_args& a = args->a;
  gdn_status st = check_common(a);
  if (st != GDN_OK) return st;
  if ((long long)a.B * a.T > 0 && !args->o) return fail(GDN_E_INVALID, "null output o");
  if (!aligned(args->o, 16)) return fail(GDN_E_INVALID, "o must be 16-byte aligned");
  if (!aligned(args->hT, 4)) return fail(GDN_E_INVALID, "hT misaligned");
  if (!aligned(args->h_save, 16)) return fail(GDN_E_INVALID, "h_save must be 16-byte aligned");
  if (!aligned(args->t_save, 16)) return fail(GDN_E_INVALID, "t_save must be 16-byte aligned");
  return GDN_OK;
}

// The forward's launches with workspace ws (at least pl.total bytes).
gdn_status fwd_launch(const gdn_fwd_args* args, const Plan& pl, void* ws, void* stream) {
  const gdn_common_args& a = args->a;
  hipStream_t s = static_cast<hipStream_t>(stream);
  gdn::SeqInfo sq = seq_info(a, pl.segc);
  hipError_t e = plan_tables(a, pl, sq, ws, s);
  if (e != hipSuccess) return hip_fail(e, "plan launch");
  gdn::FwdParams p{};
  p.q = a.q; p.k = a.k; p.v = a.v; p.g = a.g; p.beta = a.beta; p.h0 = a.h0;
  p.o = args->o; p.hT = args->hT; p.scale = a.scale; p.H = a.H; p.seq = sq;
  p.segs = at<gdn::SegDesc>(ws, pl.o_segs);
  p.seg_first = at<int>(ws, pl.o_seg_first);
  p.chunk_first = at<int>(ws, pl.o_chunk_first);
  p.hs = args->h_save;  // nullable: the chunk states (and U) are stored only on request
  p.us = args->h_save ? static_cast<char*>(args->h_save) + states_part_bytes(a) : nullptr;
  p.ulo = args->h_save && a.dtype == GDN_BF16 ? static_cast<char*>(p.us) + u_part_bytes(a) : nullptr;
  p.prep = prep_of(a.qk_norm, a.gate_act, a.gate_scale);
  // every chunk's T, solved chunk-parallel (into the caller's buffer when it
  // keeps T) and read by the chunk chain
  float* ts = args->t_save ? args->t_save : at<float>(ws, pl.o_ts);
  float* rec = ts + (size_t)pl.nchunk * a.H * CHUNK * CHUNK;  // the chunks' scalar records
  if (pl.nchunk > 0) {
    gdn::TSolveParams tp{};
    tp.k = a.k; tp.g = a.g; tp.beta = a.beta; tp.t_out = ts; tp.rec_out = rec; tp.H = a.H; tp.seq = sq;
    tp.chunk_tab = at<int2>(ws, pl.o_chunk_tab);
    tp.prep = p.prep;
    e = timed("tsolve", s, [&] { return gdn::launch_tsolve(a.dtype, a.Dk, tp, pl.nchunk, s); });
    if (e != hipSuccess) return hip_fail(e, "T solve launch");
  }
  p.t_in = ts;
  p.rec = rec;
  e = timed("fwd", s, [&] { return gdn::launch_fwd(a.dtype, a.Dk, a.Dv, p, pl.nseg, s); });
  if (e != hipSuccess) return hip_fail(e, "forward launch");
  return GDN_OK;
}

// Scratch of the allocation-free forward: one copy per device, held from the
// library's load until the process ends.  Host code never passes this name to
// a kernel or a copy (on the host it is only a stand-in for the symbol); it
// uses the device address hipGetSymbolAddress returns for the current device.
constexpr size_t NOALLOC_SCRATCH = (size_t)GDN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[NOALLOC_SCRATCH];

// The scratch's device address on the current device, looked up once per
// device (under a lock: concurrent first calls from several threads).
gdn_status scratch_ptr(void** out) {
  static std::mutex mu;
  static void* cache[64] = {nullptr};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(GDN_E_UNSUPPORTED, "device index %d beyond the scratch table", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (!cache[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    cache[dev] = ptr;
  }
  *out = cache[dev];
  return GDN_OK;
}

}  // namespace

extern "C" {

gdn_status gdn_chunk_fwd(const gdn_fwd_args* args, void* stream) {
  gdn_status st = check_fwd(args);
  if (st != GDN_OK) return st;
  const gdn_common_args& a = args->a;
  const Plan pl = make_plan(a, false, cu_count(), false, args->t_save != nullptr);
  if (!a.workspace || a.workspace_bytes < pl.total)
    return fail(GDN_E_WORKSPACE, "workspace of %zu bytes needed, %zu given", pl.total,
                a.workspace ? a.workspace_bytes : (size_t)0);
  return fwd_launch(args, pl, a.workspace, stream);
}

gdn_status gdn_chunk_fwd_noalloc(const gdn_fwd_args* args, void* stream) {
  gdn_status st = check_fwd(args);
  if (st != GDN_OK) return st;
  const Plan pl = make_plan(args->a, false, cu_count(), false, args->t_save != nullptr);
  if (pl.total > NOALLOC_SCRATCH)
    return fail(GDN_E_WORKSPACE,
                "gdn_chunk_fwd_noalloc: these arguments need %zu bytes of scratch, more than its %zu "
                "(pass t_save, or use gdn_chunk_fwd with a workspace)", pl.total, NOALLOC_SCRATCH);
  void* ws = nullptr;
  st = scratch_ptr(&ws);
  if (st != GDN_OK) return st;
  t_noalloc = true;
  st = fwd_launch(args, pl, ws, stream);
  t_noalloc = false;
  return st;
}

gdn_status gdn_chunk_bwd(const gdn_bwd_args* args, void* stream) {
  if (!args) return fail(GDN_E_INVALID, "null args");
  const gdn_common_args& a = args->a;
  gdn_status st = check_common(a);
  if (st != GDN_OK) return st;
  const bool any = (long long)a.B * a.T > 0;
  if (any && (!args->do_ || !args->dq || !args->dk || !args->dv || !args->dbeta || !args->dg))
    return fail(GDN_E_INVALID, "null gradient pointer");
  if (!aligned(args->do_, 16) || !aligned(args->dq, 16) || !aligned(args->dk, 16) || !aligned(args->dv, 16))
    return fail(GDN_E_INVALID, "do, dq, dk and dv must be 16-byte aligned");
  if (!aligned(args->dg, 4) || !aligned(args->dbeta, a.dtype == GDN_F32 ? 4 : 2) || !aligned(args->dhT, 4) ||
      !aligned(args->dh0, 4))
    return fail(GDN_E_INVALID, "dg / dbeta / dhT / dh0 misaligned");
  if (!aligned(args->h_saved, 16)) return fail(GDN_E_INVALID, "h_saved must be 16-byte aligned");
  if (!aligned(args->t_saved, 16)) return fail(GDN_E_INVALID, "t_saved must be 16-byte aligned");
  const bool saved = args->h_saved != nullptr;
  const bool t_given = args->t_saved != nullptr;
  const Plan pl = make_plan(a, true, cu_count(), saved, t_given);
  if (!a.workspace || a.workspace_bytes < pl.total)
    return fail(GDN_E_WORKSPACE, "workspace of %zu bytes needed, %zu given", pl.total,
                a.workspace ? a.workspace_bytes : (size_t)0);
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = a.workspace;
  gdn::SeqInfo sq = seq_info(a, pl.segc);
  hipError_t e = plan_tables(a, pl, sq, ws, s);
  if (e != hipSuccess) return hip_fail(e, "plan launch");
  // 1. forward replay: state at every chunk start (unless the forward saved them)
  gdn::FwdParams p{};
  p.prep = prep_of(a.qk_norm, a.gate_act, a.gate_scale);
  p.q = a.q; p.k = a.k; p.v = a.v; p.g = a.g; p.beta = a.beta; p.h0 = a.h0;
  p.o = nullptr; p.hT = nullptr; p.scale = a.scale; p.H = a.H; p.seq = sq;
  p.segs = at<gdn::SegDesc>(ws, pl.o_segs);
  p.seg_first = at<int>(ws, pl.o_seg_first);
  p.chunk_first = at<int>(ws, pl.o_chunk_first);
  // chunk matrices T: the caller's, else solved chunk-parallel here (the same
  // kernel as the forward's, so the same values); every later kernel reads them
  const float* ts = t_given ? args->t_saved : at<float>(ws, pl.o_ts);
  const float* rec = ts + (size_t)pl.nchunk * a.H * CHUNK * CHUNK;  // the chunks' scalar records
  if (!t_given && pl.nchunk > 0) {
    gdn::TSolveParams tp{};
    tp.k = a.k; tp.g = a.g; tp.beta = a.beta; tp.t_out = at<float>(ws, pl.o_ts);
    tp.rec_out = at<float>(ws, pl.o_ts) + (size_t)pl.nchunk * a.H * CHUNK * CHUNK; tp.H = a.H; tp.seq = sq;
    tp.chunk_tab = at<int2>(ws, pl.o_chunk_tab);
    tp.prep = p.prep;
    e = timed("tsolve", s, [&] { return gdn::launch_tsolve(a.dtype, a.Dk, tp, pl.nchunk, s); });
    if (e != hipSuccess) return hip_fail(e, "T solve launch");
  }
  p.t_in = ts;
  p.rec = rec;
  if (saved) {
    p.hs = const_cast<void*>(args->h_saved);
    p.us = static_cast<char*>(const_cast<void*>(args->h_saved)) + states_part_bytes(a);
    p.ulo = a.dtype == GDN_BF16 ? static_cast<char*>(p.us) + u_part_bytes(a) : nullptr;
  } else {
    p.hs = at<void>(ws, pl.o_hs);
    p.us = at<void>(ws, pl.o_us);
    p.ulo = a.dtype == GDN_BF16 ? at<void>(ws, pl.o_ulo) : nullptr;
    e = timed("replay", s, [&] { return gdn::launch_fwd(a.dtype, a.Dk, a.Dv, p, pl.nseg, s); });
    if (e != hipSuccess) return hip_fail(e, "replay launch");
  }
  // 2. reverse chain: state gradient at every chunk end, dh0
  gdn::RevParams r{};
  r.q = a.q; r.k = a.k; r.g = a.g; r.beta = a.beta; r.dout = args->do_; r.dhT = args->dhT; r.dh0 = args->dh0;
  r.scale = a.scale; r.H = a.H; r.seq = sq;
  r.segs = p.segs; r.seg_first = p.seg_first; r.chunk_first = p.chunk_first;
  r.dhs = at<void>(ws, pl.o_dhs);
  r.t_in = ts;
  r.rec = rec;
  r.us = p.us;
  r.ulo = p.ulo;
  r.ep = at<float>(ws, pl.o_ep);
  r.prep = p.prep;
  e = timed("rev", s, [&] { return gdn::launch_rev(a.dtype, a.Dk, a.Dv, r, pl.nseg, s); });
  if (e != hipSuccess) return hip_fail(e, "reverse launch");
  // 3. chunk-parallel gradients
  if (pl.nchunk > 0) {
    gdn::GradParams gp{};
    gp.q = a.q; gp.k = a.k; gp.v = a.v; gp.g = a.g; gp.beta = a.beta; gp.dout = args->do_;
    gp.hs = p.hs; gp.dhs = r.dhs; gp.us = p.us; gp.t_in = ts; gp.rec = rec; gp.ep = r.ep;
    gp.dq = args->dq; gp.dk = args->dk; gp.dv = args->dv; gp.dbeta = args->dbeta; gp.dg = args->dg;
    gp.scale = a.scale; gp.H = a.H; gp.seq = sq;
    gp.chunk_tab = at<int2>(ws, pl.o_chunk_tab);
    gp.prep = p.prep;
    gp.nwg = cu_count();
    e = timed("grad", s, [&] { return gdn::launch_grad(a.dtype, a.Dk, a.Dv, gp, pl.nchunk, s); });
    if (e != hipSuccess) return hip_fail(e, "gradient launch");
  }
  return GDN_OK;
}

gdn_status gdn_decode_step(const gdn_decode_args* args, void* stream) {
  if (!args) return fail(GDN_E_INVALID, "null args");
  const gdn_decode_args& a = *args;
  if (a.dtype != GDN_F32 && a.dtype != GDN_BF16) return fail(GDN_E_UNSUPPORTED, "unknown dtype %d", a.dtype);
  if (a.N < 0 || a.H < 1 || a.Dk < 1 || a.Dv < 1)
    return fail(GDN_E_INVALID, "bad sizes N=%d H=%d Dk=%d Dv=%d", a.N, a.H, a.Dk, a.Dv);
  if (!((a.Dk == 64 || a.Dk == 128) && (a.Dv == 64 || a.Dv == 128)))
    return fail(GDN_E_UNSUPPORTED, "unsupported head sizes Dk=%d Dv=%d", a.Dk, a.Dv);
  if ((long long)a.N * a.H >= (1LL << 31)) return fail(GDN_E_INVALID, "problem too large");
  if (a.N == 0) return GDN_OK;
  if (!a.q || !a.k || !a.v || !a.g || !a.beta || !a.state || !a.o) return fail(GDN_E_INVALID, "null pointer");
  if (!aligned(a.q, 16) || !aligned(a.k, 16) || !aligned(a.v, 16) || !aligned(a.o, 16) || !aligned(a.state, 16))
    return fail(GDN_E_INVALID, "q, k, v, o and state must be 16-byte aligned");
  if (!aligned(a.g, 4) || !aligned(a.beta, a.dtype == GDN_F32 ? 4 : 2) || !aligned(a.state_idx, 4))
    return fail(GDN_E_INVALID, "g / beta / state_idx misaligned");
  if (a.num_slots < (a.state_idx ? 0 : a.N))
    return fail(GDN_E_INVALID, "num_slots (%d) must be >= N (%d) without state_idx", a.num_slots, a.N);
  if (gdn_status ps = check_prep(a.qk_norm, a.gate_act, a.gate_scale); ps != GDN_OK) return ps;
  gdn::DecodeParams p{};
  p.q = a.q; p.k = a.k; p.v = a.v; p.g = a.g; p.beta = a.beta;
  p.state = a.state; p.state_idx = a.state_idx; p.num_slots = a.num_slots;
  p.o = a.o; p.scale = a.scale; p.N = a.N; p.H = a.H;
  p.prep = prep_of(a.qk_norm, a.gate_act, a.gate_scale);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = timed("decode", s, [&] { return gdn::launch_decode(a.dtype, a.Dk, a.Dv, p, s); });
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return GDN_OK;
}

}  // extern "C"
