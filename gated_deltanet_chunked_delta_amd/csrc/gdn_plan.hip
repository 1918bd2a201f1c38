// gdn_plan.hip -- device-side work plan: which chunks each workgroup owns.
//
// Every sequence n is cut into ceil(len_n / 64) chunks (the last one may be
// short) and its chunks into segments of `segc` chunks.  One small workgroup
// derives, from the device copy of cu_seqlens (or the uniform length T):
//   chunk_first[n]  first global chunk index of sequence n   ([N+1] prefix)
//   seg_first[n]    first global segment index of sequence n ([N+1] prefix)
//   segs[j]         (sequence, chunk range, segment index) of global segment j
//   chunk_tab[c]    (sequence, chunk index within it) of global chunk c
// An empty sequence gets one segment with no chunks, so that its final state
// (h0) and its initial-state gradient (dhT) still pass through.
#include "gdn_internal.h"

namespace gdn {

constexpr int PLAN_NT = 1024;

// Up to 64 sequences: one wave scans the counts with lane shuffles, and the
// prefixes stay in LDS for the table fill (no barrier-stepped block scan, no
// round trip through global memory).
constexpr int PLAN_SMALL = 64;

__device__ __forceinline__ int wave_incl_scan_i(int x) {
  const int l = lane_id();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (l >= o) x += y;
  }
  return x;
}

// The host sized the workspace and the grids from its copy of cu_seqlens
// (nchunk_cap chunks, nseg_cap segments).  If the device copy disagrees in a way
// that would change those totals or reach past the packed tokens (cu[0] != 0,
// cu[N] != total_tokens, a negative length), every table entry is marked
// invalid (sequence index -1) and the kernels that read the tables write
// nothing; no table is written past its capacity either way.
__device__ void mark_invalid(int nchunk_cap, int nseg_cap, SegDesc* segs, int2* chunk_tab) {
  for (int j = threadIdx.x; j < nseg_cap; j += PLAN_NT) segs[j] = SegDesc{-1, 0, 0, 0};
  for (int c = threadIdx.x; c < nchunk_cap; c += PLAN_NT) chunk_tab[c] = make_int2(-1, 0);
}

__global__ __launch_bounds__(PLAN_NT) void gdn_plan_kernel(SeqInfo seq, int N, int segc, int total_tokens,
                                                          int nchunk_cap, int nseg_cap, int* chunk_first,
                                                          int* seg_first, SegDesc* segs, int2* chunk_tab) {
  __shared__ int sc[PLAN_NT], ss[PLAN_NT];
  __shared__ int carry_c, carry_s, bad;
  const int tid = threadIdx.x;
  if (tid == 0) bad = seq.cu && (seq.cu[0] != 0 || seq.cu[N] != total_tokens);
  __syncthreads();
  if (seq.cu)
    for (int n = tid; n < N; n += PLAN_NT)
      if (seq.len(n) < 0) bad = 1;
  __syncthreads();
  if (bad) {
    mark_invalid(nchunk_cap, nseg_cap, segs, chunk_tab);
    return;
  }
  if (N <= PLAN_SMALL) {
    // sc[n] / ss[n]: first chunk / segment of sequence n, n <= N
    if (tid < 64) {
      int nc = 0, ns = 0;
      if (tid < N) {
        nc = (seq.len(tid) + CH - 1) / CH;
        ns = nc == 0 ? 1 : (nc + segc - 1) / segc;
      }
      const int ic = wave_incl_scan_i(nc), is = wave_incl_scan_i(ns);
      if (tid < N) {
        sc[tid] = ic - nc;
        ss[tid] = is - ns;
        chunk_first[tid] = ic - nc;
        seg_first[tid] = is - ns;
      }
      if (tid == 63) {
        sc[N] = ic;
        ss[N] = is;
        chunk_first[N] = ic;
        seg_first[N] = is;
      }
    }
    __syncthreads();
    const int total_s = ss[N], total_c = sc[N];
    if (total_s != nseg_cap || total_c != nchunk_cap) {
      mark_invalid(nchunk_cap, nseg_cap, segs, chunk_tab);
      return;
    }
    for (int j = tid; j < total_s; j += PLAN_NT) {
      int n = 0, hi = N - 1;
      while (n < hi) {
        const int mid = (n + hi + 1) >> 1;
        if (ss[mid] <= j) n = mid; else hi = mid - 1;
      }
      const int s = j - ss[n];
      const int nc = sc[n + 1] - sc[n];
      SegDesc d;
      d.n = n;
      d.s = s;
      d.c_begin = min(nc, s * segc);
      d.c_end = min(nc, (s + 1) * segc);
      segs[j] = d;
    }
    for (int c = tid; c < total_c; c += PLAN_NT) {
      // the last sequence whose first chunk is <= c owns c (empty sequences share
      // their prefix with the next one)
      int n = 0, hi = N - 1;
      while (n < hi) {
        const int mid = (n + hi + 1) >> 1;
        if (sc[mid] <= c) n = mid; else hi = mid - 1;
      }
      chunk_tab[c] = make_int2(n, c - sc[n]);
    }
    return;
  }
  if (tid == 0) { carry_c = 0; carry_s = 0; }
  __syncthreads();
  for (int base = 0; base < N; base += PLAN_NT) {
    const int n = base + tid;
    int nc = 0, ns = 0;
    if (n < N) {
      const int len = seq.len(n);
      nc = (len + CH - 1) / CH;
      ns = nc == 0 ? 1 : (nc + segc - 1) / segc;
    }
    sc[tid] = nc;
    ss[tid] = ns;
    __syncthreads();
    // inclusive Hillis-Steele scan over the tile
    for (int o = 1; o < PLAN_NT; o <<= 1) {
      int a = tid >= o ? sc[tid - o] : 0, b = tid >= o ? ss[tid - o] : 0;
      __syncthreads();
      sc[tid] += a;
      ss[tid] += b;
      __syncthreads();
    }
    if (n < N) {
      chunk_first[n] = carry_c + sc[tid] - nc;
      seg_first[n] = carry_s + ss[tid] - ns;
    }
    __syncthreads();
    if (tid == PLAN_NT - 1) {
      carry_c += sc[tid];
      carry_s += ss[tid];
    }
    __syncthreads();
  }
  if (tid == 0) {
    chunk_first[N] = carry_c;
    seg_first[N] = carry_s;
  }
  __syncthreads();
  __threadfence();
  const int total_s = carry_s, total_c = carry_c;
  if (total_s != nseg_cap || total_c != nchunk_cap) {
    mark_invalid(nchunk_cap, nseg_cap, segs, chunk_tab);
    return;
  }
  // fill the tables: locate the owning sequence by binary search over the prefixes
  for (int j = tid; j < total_s; j += PLAN_NT) {
    int lo = 0, hi = N - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (seg_first[mid] <= j) lo = mid; else hi = mid - 1;
    }
    // skip sequences that own no segment (none do: every sequence has >= 1)
    const int n = lo, s = j - seg_first[n];
    const int nc = (seq.len(n) + CH - 1) / CH;
    SegDesc d;
    d.n = n;
    d.s = s;
    d.c_begin = min(nc, s * segc);
    d.c_end = min(nc, (s + 1) * segc);
    segs[j] = d;
  }
  for (int c = tid; c < total_c; c += PLAN_NT) {
    int lo = 0, hi = N - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (chunk_first[mid] <= c) lo = mid; else hi = mid - 1;
    }
    // sequences with zero chunks share their prefix with the next one; the
    // search lands on the last sequence whose first chunk is <= c, which owns c
    chunk_tab[c] = make_int2(lo, c - chunk_first[lo]);
  }
}

hipError_t launch_plan(SeqInfo seq, int N, int segc, int total_tokens, int nchunk_cap, int nseg_cap,
                       int* chunk_first, int* seg_first, SegDesc* segs, int2* chunk_tab, hipStream_t st) {
  hipLaunchKernelGGL(gdn_plan_kernel, dim3(1), dim3(PLAN_NT), 0, st, seq, N, segc, total_tokens, nchunk_cap,
                     nseg_cap, chunk_first, seg_first, segs, chunk_tab);
  return hipGetLastError();
}

}  // namespace gdn
