// Kernels of batch calls: per-request settings (temperature, top-k, top-p,
// temperature-0 requests mixed with sampled ones) and the nucleus (top-p)
// cut.
//
// Method: page "vLLM speculative decoding이 기각 토큰을 다시 뽑는 이유"
// (velog), section "vLLM 커널은 이 규칙을 어떻게 옮겼나": temperature, top_k
// and top_p are applied to the logits before the test, so p (and q) are the
// adjusted laws; section "기본값 greedy 드래프트에서도 분포가 지켜질까": a
// temperature-0 request is decided by argmax matching.
//
// The nucleus of a row is the shortest prefix, in (logit desc, index asc)
// order, of the law left by temperature and top-k whose mass reaches top_p.
// It is a prefix in key order, so it is one cut key kappa: a token is kept iff
// make_key(logit, index) >= kappa.  Whether a token is in the nucleus is an
// integer decision taken on cumulative masses, so those masses are fp64:
// exp((l - l_max) / T) in double precision for every token that can matter.
#pragma once

#include <type_traits>

#include "sv_kernels.hpp"

namespace sv {

// Inclusive prefix sum over the lanes of a wave, in lane order.
__device__ __forceinline__ double wave_incl_scan_d(double v) {
  const int lane = lane_id();
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const double o = __shfl_up(v, (unsigned)d);
    if (lane >= d) v += o;
  }
  return v;
}

// Mass of logit l relative to the row's largest logit lm, at 1/T = it: the
// unnormalised probability exp(l / T - lm / T), in fp64.
__device__ __forceinline__ double nucleus_mass(double lm, float l, double it) {
  return exp(((double)l - lm) * it);
}

// 64 / ln2 (bins of ln2 / 64 nats per unit exponent), and 1.5 * 2^52: an
// fp64 value near it is rounded to an integer by its own precision (the
// integer sits in the low mantissa bits).
constexpr double kNucInvStep = 0x1.71547652b82fep+6;
constexpr double kNucRound = 0x1.8p52;

// Paths of the nucleus passes over full rows (below): with at most
// kNucSplitRows rows with top-p in a call, each row is cut into NS =
// max(2, min(kNucMaxSplit, kNucItemTarget / rows)) chunks, about one wave of
// workgroups over the chip (rows x NS <= kNucItems); with more, one
// workgroup per row.  plan = {rows, NS} (NS = 1: one workgroup per row).
constexpr int kNucSplitRows = 512, kNucItems = 1024, kNucMaxSplit = 16, kNucItemTarget = 512;
__device__ __forceinline__ void plan_nucleus(int n, int* plan) {
  int ns = 1;
  if (n > 0 && n <= kNucSplitRows) {
    ns = kNucItemTarget / n < kNucMaxSplit ? kNucItemTarget / n : kNucMaxSplit;
    ns = ns < 2 ? 2 : ns;  // n * ns <= kNucItems
  }
  plan[0] = n;
  plan[1] = ns;
}

// ===========================================================================
// Classify pass: one workgroup reads the per-request settings (or, where an
// array is null, the call's single setting T0 / K0 / top_p 1), validates
// them, and writes one ReqInfo per request.  An invalid request emits
// nothing (tokens -1, n = 0, p(x) = q(x) = 0) and sets kErrBadParam.  A
// ragged layout is checked first (cu[0] = 0, 0 <= cu[b+1] - cu[b] <= G, and
// cu[B] = 0 when the call passed no draft tokens or draft rows):
// if it fails anywhere, every request is invalid, no per-position output is
// written (their positions are unknown) and kErrBadLayout is set.  The pass
// also clears the call's error word before any other kernel can set a bit.
// ===========================================================================
__global__ __launch_bounds__(1024) void classify_kernel(const float* __restrict__ T, const int32_t* __restrict__ K,
                                                        const float* __restrict__ P, float T0, int K0, int B, int G,
                                                        int V, int max_top_k, int cand_cap, Layout L,
                                                        const int32_t* __restrict__ parents,
                                                        ReqInfo* __restrict__ info, int* __restrict__ err,
                                                        int32_t* __restrict__ out, int32_t* __restrict__ nacc,
                                                        float* __restrict__ p_draft, float* __restrict__ q_draft,
                                                        float* __restrict__ beta, int draft_rows,
                                                        int* __restrict__ nplan, int* __restrict__ nlist,
                                                        int no_drafts) {
  __shared__ int bad_layout, nlisted;
  if (threadIdx.x == 0) {
    atomicExch(err, 0);
    bad_layout = 0;
    nlisted = 0;
  }
  __syncthreads();
  if (L.cu) {
    for (int b = threadIdx.x; b < B; b += blockDim.x) {
      const int64_t c0 = L.cu[b], c1 = L.cu[b + 1];
      if ((b == 0 && c0 != 0) || c1 - c0 < 0 || c1 - c0 > G) bad_layout = 1;
    }
    // A call that passed no draft tokens (or no draft rows) has no draft
    // position to read: every length must be 0.
    if (no_drafts && threadIdx.x == 0 && L.cu[B] != 0) bad_layout = 1;
  }
  __syncthreads();
  const bool all_bad = bad_layout != 0;
  if (all_bad && threadIdx.x == 0) atomicOr(err, kErrBadLayout);
  for (int b = threadIdx.x; b < B; b += blockDim.x) {
    const float t = T ? T[b] : T0;
    const int k = K ? K[b] : K0;
    const float p = P ? P[b] : 1.f;
    bool ok = !all_bad && __builtin_isfinite(t) && t >= 0.f && k >= 0 && (k >= V || k <= max_top_k) &&
              p > 0.f && p <= 1.f;
    if (ok && parents) {
      // Tree drafts: node i's parent is an earlier node.
      const int g = L.len(b, G);
      for (int i = 1; i <= g && ok; ++i) {
        const int pa = parents[L.tok(b, G, i - 1)];
        ok = pa >= 0 && pa < i;
      }
    }
    ReqInfo r;
    r.kind = kReqInvalid;
    r.c = 0.f;
    r.K = 0;
    r.top_p = p;
    r.T = t;
    r.cut = 0;
    r.pad[0] = r.pad[1] = 0;
    if (ok) {
      if (t == 0.f) {
        r.kind = kReqGreedy;
      } else {
        r.c = (float)(1.4426950408889634 / (double)t);
        if (k > 0 && k < V && k <= cand_cap) {
          r.kind = kReqTopk;  // exact top-k by candidates
          r.K = k;
        } else {
          r.kind = kReqFull;
          if (k > 0 && k < V) r.K = k;  // a cut at the k-th key of the full row
          r.cut = (p < 1.f || r.K > 0) ? 1 : 0;
        }
      }
    }
    info[b] = r;
    if (nlist && r.kind == kReqFull && r.top_p < 1.f) {
      // The request's rows that take a nucleus (any order: rows are
      // independent): target rows 0..g, and its draft logit rows.
      const int g = L.len(b, G), nr = g + 1 + (draft_rows ? g : 0);
      const int at = atomicAdd(&nlisted, nr);
      for (int j = 0; j <= g; ++j) nlist[at + j] = b * (G + 1) + j;
      if (draft_rows)
        for (int j = 0; j < g; ++j) nlist[at + g + 1 + j] = B * (G + 1) + b * G + j;
    }
    if (!ok) {
      if (!all_bad) atomicOr(err, kErrBadParam);
      for (int j = 0; j <= G; ++j) out[(size_t)b * (G + 1) + j] = -1;
      nacc[b] = 0;
      if (!all_bad) {
        const int g = L.len(b, G);
        for (int j = 0; j < g; ++j) {
          if (p_draft) p_draft[L.tok(b, G, j)] = 0.f;
          if (q_draft) q_draft[L.tok(b, G, j)] = 0.f;
          if (beta) beta[L.tok(b, G, j)] = 0.f;
        }
      }
    }
  }
  if (nplan) {
    __syncthreads();
    if (threadIdx.x == 0) {
      const int n = nlisted;
      plan_nucleus(n, nplan);
    }
  }
}

// Whether padded row `row` exists for its request (ragged calls).
__device__ __forceinline__ bool row_exists(const Layout& L, int rows_t, int G, int row) {
  if (!L.cu) return true;
  if (row < rows_t) {
    const int b = row / (G + 1);
    return row - b * (G + 1) <= L.len(b, G);
  }
  const int r = row - rows_t, b = r / G;
  return r - b * G < L.len(b, G);
}

// The same by a whole workgroup of NT threads.
template <int NT>
__device__ __forceinline__ void block_sort_desc(uint64_t* a, int n) {
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < n / 2; i += NT) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool desc = (lo & size) == 0;
        const uint64_t x = a[lo], y = a[hi];
        if ((x < y) == desc) {
          a[lo] = y;
          a[hi] = x;
        }
      }
      __syncthreads();
    }
  }
}

// Walks sorted keys a[0, n) (descending) by one wave, starting from mass A:
// returns the first index t whose running mass A + e_0 + ... + e_t reaches
// target, and that running mass in *zk.  If rounding leaves the target
// unreached, the last index and the total.
template <typename M>
__device__ __forceinline__ int wave_walk(const uint64_t* a, int n, double A, double target, M&& mass, double* zk) {
  const int lane = lane_id();
  double base = A;
  for (int i0 = 0; i0 < n; i0 += kWave) {
    const int i = i0 + lane;
    const uint64_t k = i < n ? a[i] : 0ull;
    const double e = k ? mass(key_value(k)) : 0.0;
    const double inc = base + wave_incl_scan_d(e);
    const uint64_t hit = ballot(i < n && inc >= target);
    if (hit) {
      const int l = (int)__builtin_ctzll(hit);
      *zk = __shfl(inc, l);
      return i0 + l;
    }
    base = __shfl(inc, kWave - 1);
  }
  *zk = base;
  return n - 1;
}

// ===========================================================================
// Nucleus of a top-k row: one wave per row (four rows per workgroup).  The
// row's k candidate keys are sorted (descending), their fp64 masses summed
// and walked, and the candidates after the cut are zeroed in place.
// ===========================================================================
__global__ __launch_bounds__(256) void nucleus_topk_kernel(uint64_t* __restrict__ cand, int kstride, int rows_t,
                                                           int nrows, int G, const ReqInfo* __restrict__ info,
                                                           Layout L) {
  __shared__ uint64_t keys_sh[4][1024];
  const int w = threadIdx.x / kWave, lane = lane_id();
  const int row = blockIdx.x * 4 + w;
  if (row >= nrows) return;
  const ReqInfo ri = info[row_request(row, rows_t, G)];
  if (ri.kind != kReqTopk || !(ri.top_p < 1.f)) return;
  if (!row_exists(L, rows_t, G, row)) return;
  const int K = ri.K;  // 1 <= K <= 1024 (validated by the host bound)
  int n2 = kWave;
  while (n2 < K) n2 <<= 1;
  uint64_t* ks = keys_sh[w];
  uint64_t* src = cand + (size_t)row * kstride;
  for (int i = lane; i < n2; i += kWave) ks[i] = i < K ? src[i] : 0ull;
  wave_lds_sync();
  wave_sort_desc(ks, n2);
  const uint64_t top = ks[0];
  if (top == 0ull) return;
  const double lm = (double)key_value(top), it = 1.0 / (double)ri.T;
  double z = 0.0;
  for (int i = lane; i < K; i += kWave) {
    const uint64_t k = ks[i];
    if (k) z += nucleus_mass(lm, key_value(k), it);
  }
  z = wave_sum_d(z);
  double zk;
  const int t = wave_walk(ks, K, 0.0, (double)ri.top_p * z, [&](float l) { return nucleus_mass(lm, l, it); }, &zk);
  for (int i = lane; i < K; i += kWave) src[i] = i <= t ? ks[i] : 0ull;
}

// ===========================================================================
// Nucleus of a full row (no top-k candidates).  The steps, as nucleus_row
// runs them with one workgroup per row; with few such rows in a call, the
// same steps are split over chunks of each row (the nucleus passes further
// below):
//
//   pass 1  a histogram of fp64 mass over bins ln2 / 64 nats wide, the row's
//           largest logit and its total mass Z, in one read of the row (the
//           softmax pass skips these rows).
//   scan    the bin where the running mass, from the largest logit down,
//           reaches top_p Z, and the mass A of the bins before it.
//   pass 2  the bin's tokens are collected into LDS (at most kNucCap; the
//           histogram's storage), sorted by key and walked from A: the first
//           token that reaches top_p Z is the cut.
//   refine  (a bin with more than kNucCap tokens, e.g. many equal logits)
//           radix passes over the keys of that bin, 8 bits at a time below
//           their common prefix, each keeping the digit that holds the cut,
//           until at most kNucCap tokens remain.
//
// The grid.  With 1/T = it and C = 64 it / ln2, token l falls in bin
// k(l) = round(y), y = l C - rint(a C) (the exact product plus an integer,
// rounded once by one fma), for an anchor a fixed before pass 1 reads the
// row: 0 for a row split over chunks (every chunk bins alike), the largest
// logit of a first look for a row read by one workgroup.  k is
// non-decreasing in l, so the bins cut the row in key order.  With kmax the bin of the row's largest logit, every mass
// of the nucleus passes is taken in the unit 2^((y - kmax) / 64) =
// 2^((k - kmax) / 64) 2^(f / 64), f = y - k in [-1/2, 1/2]: a bin sums its
// tokens' 2^(f / 64) and its power of two is applied once, and the walk and
// the refinement take each token's mass the same way, so all of them agree
// to rounding.  The row's masses exp((l - lmax) / T) are these times
// g = 2^((kmax - y(lmax)) / 64), applied to the kept mass at the end.
//
// The window.  A workgroup holds kNucBins consecutive bins in LDS, bin k in
// slot k mod kNucBins.  Before any token is added, the largest logit l0 of
// the vectors the workgroup loads first places the window at bins
// (k0 + R - kNucBins, k0 + R], k0 = k(l0), R = kNucRise.  A token below the
// window adds its mass exp((l - l0) / T) to a spare sum; a token above it is
// listed (at most kNucRiseCap) until the workgroup's maximum is known, and
// the window then moves up to (kmax - kNucBins, kmax]: the bins it leaves go
// into the spare sum, the listed tokens into their bins.  Either way every
// bin within kNucBins - R bins (38.8 nats) of kmax holds its exact sum; the
// tokens further below carry less than 2^31 e^-38.8 < 3.1e-8 of Z in total,
// so the cut (top_p <= 1 - 2^-24) falls among the held bins.  A row whose
// list overflows (e.g. ascending logits) or whose bins leave fp64's exact
// integers is binned again with its maximum known (anchor and window at the
// maximum): one more read, for that row only.  Rows under a large top-k take
// that form from the start (the softmax pass before their top-k cut gives
// the maximum).
// ===========================================================================
constexpr int kNucBins = 4096;      // slots of the window: ln2 / 64 nats each
constexpr int kNucRise = 512;       // bins of the window above the first look's maximum
constexpr int kNucRiseCap = 256;    // tokens listed above the window
constexpr double kNucRange = 0x1.0p49;  // |y| bound of the window's bins (exact fp64 integers)
// A workgroup per row (or per chunk): 512 threads, two vectors per thread in
// flight (build knobs SV_NUC_NT, SV_NUC_U).  Measured on MI355X against
// 256 x 2, 256 x 4, 512 x 3, 1024 x 1 and 1024 x 2 (with the earlier pass 1
// that read the row after the softmax pass): the fastest or within 1% on the
// mixed, ragged and sampler-match workloads.
#ifndef SV_NUC_NT
#define SV_NUC_NT 512
#endif
#ifndef SV_NUC_U
#define SV_NUC_U 2
#endif
struct NucShape {
  static constexpr int NT = SV_NUC_NT, U = SV_NUC_U;
};
constexpr int kCutThreads = 512;  // kcut_full_kernel
constexpr int kNucCap = 2048;

// Streams the row through the workgroup: fv(values, y0) for each 16-byte
// vector this thread owns (elements y0 .. y0 + EPV - 1), fs(value, y) for the
// scalar head and tail.  Chunks of U vectors per thread; the next chunk's
// loads are issued before the current one is processed, so a wave's memory
// requests stay in flight while it computes.
// Elements [a, e) of the row (indices as in the whole row).
template <typename ET, int NT, int U, typename FV, typename FS>
__device__ __forceinline__ void row_stream(const ET* rp, int a, int e, FV&& fv, FS&& fs) {
  constexpr int EPV = Elem<ET>::kPerVec, STEP = NT * U;
  Slice<ET> sl(rp, a, e);
  const int tid = threadIdx.x;
  if (tid < sl.nscalar()) {
    const int y = sl.scalar_index(tid);
    fs(Elem<ET>::load1(rp + y), y);
  }
  const uint4* vp = sl.vecs();
  const int nv = sl.nvec, nfull = nv / STEP;
  auto proc = [&](const uint4& v, int i) {
    float f[EPV];
    Elem<ET>::unpack(v, f);
    fv(f, sl.vec_index0(i));
  };
  if (nfull > 0) {
    uint4 cur[U];
#pragma unroll
    for (int u = 0; u < U; ++u) cur[u] = load_stream(vp + tid + u * NT);
    for (int c = 0; c < nfull; ++c) {
      const int i0 = c * STEP + tid;
      uint4 nxt[U];
      if (c + 1 < nfull) {
#pragma unroll
        for (int u = 0; u < U; ++u) nxt[u] = load_stream(vp + i0 + STEP + u * NT);
      } else {
#pragma unroll
        for (int u = 0; u < U; ++u) nxt[u] = cur[u];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) proc(cur[u], i0 + u * NT);
#pragma unroll
      for (int u = 0; u < U; ++u) cur[u] = nxt[u];
    }
  }
  // The last partial chunk: fewer than U vectors for some threads.
  const int i0 = nfull * STEP + tid;
  uint4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int i = i0 + u * NT;
    v[u] = i < nv ? load_stream(vp + i) : make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (i0 + u * NT < nv) proc(v[u], i0 + u * NT);
}

template <typename ET, int NT, int U, typename FV, typename FS>
__device__ __forceinline__ void row_stream(const ET* rp, int V, FV&& fv, FS&& fs) {
  row_stream<ET, NT, U>(rp, 0, V, fv, fs);
}

// Calls f(logit, index) for every element of the row this thread owns.
template <typename ET, int NT, int U, typename F>
__device__ __forceinline__ void row_foreach(const ET* rp, int V, F&& f) {
  constexpr int EPV = Elem<ET>::kPerVec;
  row_stream<ET, NT, U>(
      rp, V,
      [&](const float (&fv)[EPV], int y0) {
#pragma unroll
        for (int k = 0; k < EPV; ++k) f(fv[k], y0 + k);
      },
      f);
}

// The window of the nucleus passes (kNucBins slots), one LDS array per
// kernel; dead once the cut bin is chosen, it then holds the collected keys
// of that bin.
__device__ __forceinline__ double* nucleus_hist_lds() {
  __shared__ double hm[kNucBins];
  return hm;
}

// Tokens listed above the window, and a reduction buffer, for pass 1.
struct NucRise {
  float l[kNucRiseCap];
  int n;
  float red[NucShape::NT / kWave];
};
__device__ __forceinline__ NucRise* nucleus_rise_lds() {
  __shared__ NucRise s;
  return &s;
}

// Largest logit of a row, from the softmax pass's partials (every lane of
// every wave gets it).
__device__ __forceinline__ float nucleus_lmax(const float2* part, int row, int S) {
  float lmax = -INFINITY;
  for (int k = lane_id(); k < S; k += kWave) lmax = fmaxf(lmax, part[(size_t)row * S + k].x);
  return wave_max_f(lmax);
}

// Writes a row's softmax partials as one split (max, mass) and empty ones,
// for a row whose softmax pass was skipped.  By the whole workgroup.
__device__ __forceinline__ void nucleus_write_part(float2* part, int row, int S, float lmax, float Z) {
  for (int k = threadIdx.x; k < S; k += blockDim.x)
    part[(size_t)row * S + k] = k == 0 ? make_float2(lmax, Z) : make_float2(-INFINITY, 0.f);
}

// Largest value over the workgroup (NT threads), to every thread.  Ends with
// a barrier.
template <int NT>
__device__ __forceinline__ float block_max_f(float v, float* red) {
  constexpr int NW = NT / kWave;
  v = wave_max_f(v);
  if (lane_id() == 0) red[threadIdx.x / kWave] = v;
  __syncthreads();
  float m = red[0];
#pragma unroll
  for (int k = 1; k < NW; ++k) m = fmaxf(m, red[k]);
  __syncthreads();
  return m;
}

// Sum over the workgroup (NT threads), to every thread.  Ends with a barrier.
template <int NT>
__device__ __forceinline__ double block_sum_d(double v, double* red) {
  constexpr int NW = NT / kWave;
  v = wave_sum_d(v);
  if (lane_id() == 0) red[threadIdx.x / kWave] = v;
  __syncthreads();
  double s = 0.0;
#pragma unroll
  for (int k = 0; k < NW; ++k) s += red[k];
  __syncthreads();
  return s;
}

// 2^(f/64) for |f| <= 1/2: exp(c f), c = ln2 / 64, by its Taylor polynomial
// of degree 4 (|c f| <= 0.0055, truncation below 4e-14 relative).
__device__ __forceinline__ double exp2_frac64(double f) {
  constexpr double c = 0.6931471805599453 / 64.0;
  constexpr double a2 = c * c / 2.0, a3 = a2 * c / 3.0, a4 = a3 * c / 4.0;
  double q = fma(f, a4, a3);
  q = fma(f, q, a2);
  q = fma(f, q, c);
  return fma(f, q, 1.0);
}

// 2^(j/64) for an integer j <= 2^16 (tab[i] = 2^(i/64)); 0 below fp64's
// range.
__device__ __forceinline__ double exp2_64ths(double j, const double* tab) {
  const int k = (int)fmin(fmax(j, -1048576.0), 65536.0);
  return ldexp(tab[k & 63], k >> 6);
}

// 2^(e/64) for real e <= 2^16 (0 below fp64's range).
__device__ __forceinline__ double exp2_64(double e, const double* tab) {
  const double n = rint(e);
  return e > -1048576.0 ? exp2_64ths(n, tab) * exp2_frac64(e - n) : 0.0;
}

// The bin grid of a row: t(l) = fma(l, C, B) rounds l C + B once to an
// integer (B = kNucRound - rint(a C), an integer near kNucRound, for anchor
// a), so token l is in bin k(l) = t(l) - kNucRound, with y = l C + B -
// kNucRound and f = y - k = fma(l, C, B - t(l)) (an exact integer added to
// the exact product, rounded once).  Exact while |y| < 2^51.
struct NucGrid {
  double B, C, kmax;  // offset, bins per unit of logit, bin of the largest logit
};
__device__ __forceinline__ double nuc_grid_B(double anchor, double C) { return kNucRound - rint(anchor * C); }
__device__ __forceinline__ double nuc_t(float l, const NucGrid& g) { return fma((double)l, g.C, g.B); }

// A token's mass in the grid's unit, 2^((y - kmax) / 64).
__device__ __forceinline__ double nuc_mass(const NucGrid& g, float l, const double* tab) {
  const double t = nuc_t(l, g);
  const double m = exp2_64ths(t - kNucRound - g.kmax, tab) * exp2_frac64(fma((double)l, g.C, g.B - t));
  return l == -INFINITY ? 0.0 : m;
}

// Result of pass 1 over a slice: the grid and window top kmax, the logit l0
// that placed the window, the largest logit lmax (-inf: none finite), and
// this thread's spare masses: sp in units of exp((l - l0) / T), sb in the
// grid's unit.  ok false: the row must be binned again with its maximum
// known.
struct NucP1 {
  NucGrid g;
  float l0, lmax;
  bool ok;
  double sp, sb;
};

// Pass 1 over elements [a_, e_) of a row into the window hm (kNucBins slots,
// zeroed by the caller, who also clears the rise list's count before a
// barrier); tab[i] = 2^(i/64).  LOOK: the window is placed by a first look
// at the vectors the workgroup loads first (the next ones while those hold
// no finite logit), and the anchor is l0 when anchor_l0, else `anchor`.
// !LOOK: the row's largest logit lm is known and is both anchor and l0; with
// FLOOR a token whose key is below kfloor adds nothing.  Workgroup-uniform
// result after a barrier.
template <typename ET, int NT, int U, bool LOOK, bool FLOOR>
__device__ NucP1 nucleus_pass1(const ET* rp, int a_, int e_, bool anchor_l0, double anchor, float lm, double it,
                               uint64_t kfloor, const double* tab, double* hm) {
  constexpr int EPV = Elem<ET>::kPerVec, STEP = NT * U, S = kNucBins;
  NucRise* rl = nucleus_rise_lds();
  const double C = it * kNucInvStep;
  Slice<ET> sl(rp, a_, e_);
  const int tid = threadIdx.x;
  float sv = -INFINITY;
  int sy = 0;
  if (tid < sl.nscalar()) {
    sy = sl.scalar_index(tid);
    sv = Elem<ET>::load1(rp + sy);
  }
  const uint4* vp = sl.vecs();
  const int nv = sl.nvec, nch = (nv + STEP - 1) / STEP;
  const uint4 ninf = make_uint4(Elem<ET>::kNegInfWord, Elem<ET>::kNegInfWord, Elem<ET>::kNegInfWord,
                                Elem<ET>::kNegInfWord);
  // Chunk c's vectors of this thread; past the slice's end the load is
  // clamped into it (unconditional) and the value replaced by -inf.
  auto load = [&](int c, uint4(&v)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = c * STEP + u * NT + tid;
      const uint4 x = load_stream(vp + (i < nv ? i : nv - 1));
      v[u] = i < nv ? x : ninf;
    }
  };
  uint4 cur[U];
  int c = 0;
  if (nch > 0) load(0, cur);
  float l0 = lm;
  if constexpr (LOOK) {
    for (;;) {
      float tm = c == 0 ? sv : -INFINITY;
      if (c < nch) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float f[EPV];
          Elem<ET>::unpack(cur[u], f);
#pragma unroll
          for (int k = 0; k < EPV; ++k) tm = fmaxf(tm, f[k]);
        }
      }
      l0 = block_max_f<NT>(tm, rl->red);
      if (l0 != -INFINITY || c + 1 >= nch) break;  // uniform
      ++c;  // chunks before c hold no finite logit (no mass)
      load(c, cur);
    }
  }
  NucP1 r;
  r.g.B = kNucRound;
  r.g.C = C;
  r.g.kmax = 0.0;
  r.l0 = l0;
  r.lmax = -INFINITY;
  r.ok = true;
  r.sp = 0.0;
  r.sb = 0.0;
  if (l0 == -INFINITY) return r;  // no finite logit in the slice (uniform)
  r.g.B = nuc_grid_B(LOOK ? (anchor_l0 ? (double)l0 : anchor) : (double)lm, C);
  const double B = r.g.B;
  // The window (lo, hi] in bins, as t values.
  const double hi = nuc_t(l0, r.g) + (double)kNucRise, lo = hi - (double)S;
  float tmax = -INFINITY;
  double sp = 0.0;
  // Below the window a token lies more than 38.8 nats under l0, and all of
  // them carry less than 3.1e-8 of Z: their masses are taken in fp32 (about
  // 1e-5 relative), so Z keeps about 1e-12 relative accuracy.
  const float c2 = (float)(it * 1.4426950408889634);
  auto add = [&](float l, int y) {
    tmax = fmaxf(tmax, l);
    if (FLOOR && make_key(l, (uint32_t)y) < kfloor) return;
    const double t = fma((double)l, C, B);
    if (t > lo && t <= hi) {
      atomicAdd(&hm[__double2loint(t) & (S - 1)], exp2_frac64(fma((double)l, C, B - t)));
    } else if (t > hi) {
      const int pos = atomicAdd(&rl->n, 1);
      if (pos < kNucRiseCap) rl->l[pos] = l;
    } else {
      const float m = __builtin_amdgcn_exp2f((l - l0) * c2);
      sp += m > 0.f ? (double)m : 0.0;  // 0 for -inf and NaN
    }
  };
  if (tid < sl.nscalar()) add(sv, sy);
  for (; c < nch; ++c) {
    uint4 nxt[U];
    if (c + 1 < nch) load(c + 1, nxt);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float f[EPV];
      Elem<ET>::unpack(cur[u], f);
      const int y0 = sl.vec_index0(c * STEP + u * NT + tid);
#pragma unroll
      for (int k = 0; k < EPV; ++k) add(f[k], y0 + k);
    }
    if (c + 1 < nch) {
#pragma unroll
      for (int u = 0; u < U; ++u) cur[u] = nxt[u];
    }
  }
  r.sp = sp;
  const float lmax = block_max_f<NT>(tmax, rl->red);  // its barrier also ends every add
  r.lmax = lmax;
  if (lmax == -INFINITY) return r;  // every token -inf (uniform)
  const int nr = rl->n;
  const double tmx = nuc_t(lmax, r.g);
  const double kmax = tmx - kNucRound;
  r.g.kmax = kmax;
  r.ok = nr <= kNucRiseCap && fabs(fma((double)lmax, C, B - kNucRound)) < kNucRange &&
         fabs(fma((double)l0, C, B - kNucRound)) < kNucRange;
  if (r.ok && nr > 0) {
    // The window moves up to (kmax - S, kmax]: bins (lo, kmax - S] leave it
    // (slot i holds bin hi - dist, dist = (hi - i) mod S; t values).
    const double shift = tmx - hi;  // > 0: a listed token lies above hi
    const int top = __double2loint(hi);
    double sb = 0.0;
    for (int i = tid; i < S; i += NT) {
      const int dist = (top - i) & (S - 1);
      if ((double)dist >= (double)S - shift) {
        const double v = hm[i];
        if (v != 0.0) sb += v * exp2_64ths(-((double)dist + shift), tab);
        hm[i] = 0.0;
      }
    }
    __syncthreads();
    for (int i = tid; i < nr; i += NT) {
      const float l = rl->l[i];
      const double t = fma((double)l, C, B);
      const double v = exp2_frac64(fma((double)l, C, B - t));
      if (t > tmx - (double)S) atomicAdd(&hm[__double2loint(t) & (S - 1)], v);
      else sb += v * exp2_64ths(t - tmx, tab);
    }
    __syncthreads();
    r.sb = sb;
  }
  return r;
}

// Bin masses in the grid's unit, in place: slot i of a window with top bin
// kmax (top = kmax mod 2^32) holds gap j = (top - i) mod kNucBins and is
// multiplied by 2^(-j/64).  Returns the total, bins plus every thread's
// spare (already in the grid's unit), to every thread.  Starts after a
// barrier and ends with one.
template <int NT>
__device__ __forceinline__ double nucleus_unfactor(double* hm, int top, double spare, const double* tab,
                                                   double* red) {
  double z = spare;
  for (int i = threadIdx.x; i < kNucBins; i += NT) {
    const double v = hm[i];
    if (v != 0.0) {
      const int j = (top - i) & (kNucBins - 1);
      const double m = v * ldexp(tab[(-j) & 63], (-j) >> 6);
      hm[i] = m;
      z += m;
    }
  }
  return block_sum_d<NT>(z, red);
}

// Scan of the window by a workgroup of NT threads in gap order (gap j in
// slot (top - j) mod kNucBins): thread t owns gaps [t * PER, (t + 1) * PER);
// its interval of running mass is (incl[t - 1], incl[t]], so the intervals
// tile [0, total].  Writes the first non-empty gap where the running mass
// reaches target to *bin_out (-1 if none) and the mass of the gaps before it
// to *A_out.  Ends with a barrier.
template <int NT>
__device__ __forceinline__ void nucleus_pick(const double* hm, int top, double target, double* incl_sh,
                                             double* red_s, int* bin_out, double* A_out) {
  constexpr int PER = kNucBins / NT, NW = NT / kWave;
  const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
  auto at = [&](int j) { return hm[(top - j) & (kNucBins - 1)]; };
  if (tid == 0) *bin_out = -1;
  double loc = 0.0;
  for (int k = 0; k < PER; ++k) loc += at(tid * PER + k);
  double inc = wave_incl_scan_d(loc);
  if (lane == kWave - 1) red_s[w] = inc;
  __syncthreads();
  for (int k = 0; k < w && k < NW; ++k) inc += red_s[k];
  incl_sh[tid] = inc;
  __syncthreads();
  const double start = tid == 0 ? 0.0 : incl_sh[tid - 1];
  if (start < target && target <= inc) {
    double cum = start;
    int pick = -1;
    double pickA = start;
    for (int k = 0; k < PER; ++k) {
      const int j = tid * PER + k;
      const double v = at(j);
      if (!(v > 0.0)) continue;
      pick = j;  // last non-empty gap so far: the choice if rounding leaves the target unreached
      pickA = cum;
      const double nxt = cum + v;
      if (nxt >= target) break;
      cum = nxt;
    }
    *bin_out = pick;
    *A_out = pickA;
  }
  __syncthreads();
}

// Pass 2 over elements [a, e): push(l, y) for every token with in_bin(l).
// The test of a vector's tokens first (branch-free), then the rare tokens of
// the chosen bin.
template <typename ET, int NT, int U, typename B, typename P>
__device__ __forceinline__ void nucleus_collect(const ET* rp, int a, int e, B&& in_bin, P&& push) {
  row_stream<ET, NT, U>(
      rp, a, e,
      [&](const float (&fv)[Elem<ET>::kPerVec], int y0) {
        constexpr int EPV = Elem<ET>::kPerVec;
        bool m[EPV];
        bool any = false;
#pragma unroll
        for (int k = 0; k < EPV; ++k) {
          m[k] = in_bin(fv[k]);
          any |= m[k];
        }
        if (any) {
#pragma unroll
          for (int k = 0; k < EPV; ++k)
            if (m[k]) push(fv[k], y0 + k);
        }
      },
      [&](float l, int y) {
        if (in_bin(l)) push(l, y);
      });
}

// The whole nucleus of one row by one workgroup (every step above;
// refinement of an over-full bin included).  known: the row's maximum is
// read from the softmax partials (rows under a large top-k, whose softmax
// pass ran, and rows the split passes send back), else pass 1 finds it.  A
// row without top-k gets its softmax partials written here.
template <typename ET>
__device__ __forceinline__ void nucleus_row(int row, const ET* __restrict__ lt, const ET* __restrict__ ld, int rows_t,
                                            int G, int V, int S, float2* __restrict__ part,
                                            const ReqInfo* __restrict__ info, RowCut* __restrict__ cut,
                                            const Layout& L, bool known) {
  constexpr int NT = NucShape::NT, U = NucShape::U, NW = NT / kWave;
  static_assert(kNucBins % NT == 0, "bins per thread");
  static_assert(kNucCap * sizeof(uint64_t) <= kNucBins * sizeof(double), "keys alias the histogram");
  const ReqInfo ri = info[row_request(row, rows_t, G)];
  if (ri.kind != kReqFull || !(ri.top_p < 1.f)) return;  // uniform over the workgroup
  const ET* rp = row_ptr(L, lt, ld, rows_t, G, row);
  if (!rp) return;  // past the request's draft length
  // Under a large top-k the nucleus is taken over the top-k law: tokens below
  // the k-cut (written by kcut_full_kernel) have no mass here.
  const bool own_part = ri.K == 0;  // the softmax pass skipped the row
  const uint64_t kfloor = ri.K > 0 ? cut[row].kappa : 0ull;
  auto below = [&](float l, int y) { return kfloor != 0ull && make_key(l, (uint32_t)y) < kfloor; };
  double* hm = nucleus_hist_lds();
  uint64_t* keys = reinterpret_cast<uint64_t*>(hm);
  NucRise* rl = nucleus_rise_lds();
  __shared__ double tab[64];
  __shared__ double red_d[NW], red_s[NW];
  // The scan's running sums and the refinement's digit counts live at
  // different times.
  __shared__ union {
    double incl[NT];
    struct {
      double m[256];
      uint32_t c[256];
    } dig;
  } scr;
  double* dm = scr.dig.m;
  uint32_t* dc = scr.dig.c;
  __shared__ uint64_t red_k[2][NW];
  __shared__ double sh_A;
  __shared__ int sh_bin, sh_n;
  __shared__ uint32_t sh_cnt;
  __shared__ uint64_t sh_prefix;
  __shared__ int sh_plen;
  const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
  const double it = 1.0 / (double)ri.T;

  for (int i = tid; i < kNucBins; i += NT) hm[i] = 0.0;
  if (tid < 64) tab[tid] = exp2((double)tid / 64.0);
  if (tid == 0) {
    rl->n = 0;
    sh_prefix = 0ull;  // fixed top bits of the cut key (refinement)
    sh_plen = 0;
    sh_n = 0;
  }
  __syncthreads();

  // Pass 1: the window, the row's maximum and the spare masses.
  NucP1 p;
  if (known) {
    const float lm = nucleus_lmax(part, row, S);
    if (kfloor != 0ull) p = nucleus_pass1<ET, NT, U, false, true>(rp, 0, V, false, 0.0, lm, it, kfloor, tab, hm);
    else p = nucleus_pass1<ET, NT, U, false, false>(rp, 0, V, false, 0.0, lm, it, 0ull, tab, hm);
  } else {
    p = nucleus_pass1<ET, NT, U, true, false>(rp, 0, V, true, 0.0, 0.f, it, 0ull, tab, hm);
    if (!p.ok) {
      // Binned again with the maximum known.
      const float lm = p.lmax;
      for (int i = tid; i < kNucBins; i += NT) hm[i] = 0.0;
      if (tid == 0) rl->n = 0;
      __syncthreads();
      p = nucleus_pass1<ET, NT, U, false, false>(rp, 0, V, false, 0.0, lm, it, 0ull, tab, hm);
    }
  }
  const float lmax = p.lmax;
  if (lmax == -INFINITY) {
    // No finite logit: no cut.
    if (own_part) nucleus_write_part(part, row, S, lmax, 0.f);
    if (tid == 0) cut[row] = RowCut{kfloor, lmax, INFINITY};
    return;
  }
  const NucGrid g = p.g;
  const int top = __double2loint(g.kmax + kNucRound);
  const double sp = p.sp * exp2_64(fma((double)p.l0, g.C, g.B - kNucRound - g.kmax), tab);
  const double Z = nucleus_unfactor<NT>(hm, top, sp + p.sb, tab, red_d);
  // Grid unit -> exp((l - lmax) / T).
  const double gf = exp2_frac64(-fma((double)lmax, g.C, g.B - kNucRound - g.kmax));
  if (own_part) nucleus_write_part(part, row, S, lmax, (float)(Z * gf));
  const double target = (double)ri.top_p * Z;

  nucleus_pick<NT>(hm, top, target, scr.incl, red_s, &sh_bin, &sh_A);
  const int jstar = sh_bin;
  if (jstar < 0) {
    // No mass (degenerate row): no cut.
    if (tid == 0) cut[row] = RowCut{kfloor, lmax, (float)(1.0 / (Z * gf))};
    return;
  }
  const double tstar = kNucRound + (g.kmax - (double)jstar);
  auto in_bin = [&](float l) { return nuc_t(l, g) == tstar; };
  auto mass = [&](float l) { return nuc_mass(g, l, tab); };

  // Pass 2: collect the keys of the bin (at most kNucCap are kept; the count
  // tells whether the bin needs refining).  filter_key: bin and key prefix.
  auto collect = [&](int plen, uint64_t prefix) {
    nucleus_collect<ET, NT, U>(rp, 0, V, in_bin, [&](float l, int y) {
      if (below(l, y)) return;
      const uint64_t k = make_key(l, (uint32_t)y);
      if (plen > 0 && (plen == 64 ? k != prefix : (k >> (64 - plen)) != (prefix >> (64 - plen)))) return;
      const int pos = atomicAdd(&sh_n, 1);
      if (pos < kNucCap) keys[pos] = k;
    });
  };
  collect(0, 0ull);
  __syncthreads();
  // Refinement of an over-full bin: radix over the keys below their common
  // prefix, 8 bits at a time, keeping the digit that holds the cut.
  if (sh_n > kNucCap) {
    if (tid == 0) sh_cnt = (uint32_t)sh_n;
    uint64_t kmin = ~0ull, kmax = 0ull;
    row_foreach<ET, NT, U>(rp, V, [&](float l, int y) {
      if (in_bin(l) && !below(l, y)) {
        const uint64_t k = make_key(l, (uint32_t)y);
        kmin = k < kmin ? k : kmin;
        kmax = k > kmax ? k : kmax;
      }
    });
    kmax = wave_max_u64(kmax);
    kmin = ~wave_max_u64(~kmin);
    if (lane == 0) {
      red_k[0][w] = kmin;
      red_k[1][w] = kmax;
    }
    __syncthreads();
    if (tid == 0) {
      uint64_t a = red_k[0][0], z = red_k[1][0];
      for (int k = 1; k < NW; ++k) {
        a = red_k[0][k] < a ? red_k[0][k] : a;
        z = red_k[1][k] > z ? red_k[1][k] : z;
      }
      const int plen = a == z ? 64 : __builtin_clzll(a ^ z);
      sh_plen = plen;
      sh_prefix = plen == 0 ? 0ull : (plen == 64 ? z : (z & (~0ull << (64 - plen))));
    }
    __syncthreads();
    while (sh_cnt > (uint32_t)kNucCap && sh_plen < 64) {
      const int plen = sh_plen;
      const uint64_t prefix = sh_prefix;
      const int nb = 64 - plen < 8 ? 64 - plen : 8;
      const int shift = 64 - plen - nb;
      for (int i = tid; i < 256; i += NT) {
        dm[i] = 0.0;
        dc[i] = 0u;
      }
      __syncthreads();
      row_foreach<ET, NT, U>(rp, V, [&](float l, int y) {
        if (!in_bin(l) || below(l, y)) return;
        const uint64_t k = make_key(l, (uint32_t)y);
        if (plen > 0 && (k >> (64 - plen)) != (prefix >> (64 - plen))) return;
        const int dig = (int)((k >> shift) & ((1ull << nb) - 1ull));
        atomicAdd(&dm[dig], mass(l));
        atomicAdd(&dc[dig], 1u);
      });
      __syncthreads();
      if (tid == 0) {
        double cum = sh_A;
        int pick = -1;
        double pickA = cum;
        for (int dig = (1 << nb) - 1; dig >= 0; --dig) {  // descending keys first
          if (dc[dig] == 0u) continue;
          pick = dig;
          pickA = cum;
          const double nxt = cum + dm[dig];
          if (nxt >= target) break;
          cum = nxt;
        }
        if (pick >= 0) {  // always: the digits hold the sh_cnt > 0 tokens of the prefix
          sh_prefix = prefix | ((uint64_t)pick << shift);
          sh_plen = plen + nb;
          sh_A = pickA;
          sh_cnt = dc[pick];
        } else {
          sh_plen = 64;
          sh_cnt = 0u;
        }
      }
      __syncthreads();
    }
    if (tid == 0) sh_n = 0;
    __syncthreads();
    collect(sh_plen, sh_prefix);
    __syncthreads();
  }

  // Sort the collected keys and walk them from the mass of the bins above.
  const int n = sh_n < kNucCap ? sh_n : kNucCap;
  int n2 = 2;
  while (n2 < n) n2 <<= 1;
  for (int i = n + tid; i < n2; i += NT) keys[i] = 0ull;
  __syncthreads();
  block_sort_desc<NT>(keys, n2);
  if (w == 0) {
    double zk;
    const int t = n > 0 ? wave_walk(keys, n, sh_A, target, mass, &zk) : -1;
    if (lane == 0) {
      if (t >= 0) cut[row] = RowCut{keys[t], lmax, (float)(1.0 / (zk * gf))};
      else cut[row] = RowCut{kfloor, lmax, (float)(1.0 / (Z * gf))};
    }
  }
}


// ===========================================================================
// Nucleus passes over full rows.  classify_kernel lists the rows with top-p
// (how many there are is known only on the device).  With more than
// kNucSplitRows of them, nucleus_part_kernel runs nucleus_row on each, one
// workgroup per row.  With fewer, one workgroup per row would leave most of
// the chip idle (a row then streams at the rate of one workgroup's loads in
// flight), so each row is cut into NS contiguous chunks (plan_nucleus) and
// the steps of nucleus_row run as separate passes:
//   part     per chunk: pass 1 (its window on the row's common grid, anchor
//            0, or the row's maximum under a large top-k) into the
//            workspace;
//   scan     per row: the chunks' windows merged at the row's largest
//            logit (bins below the merged window join the spare mass); the
//            bin where the running mass reaches top_p Z, and the mass A of
//            the bins before it; the row's softmax partials;
//   collect  per chunk: the keys of that bin, appended to the row's buffer;
//   finish   per row: sort and walk the keys from A.  A bin of more than
//            kNucCap keys, or a row a chunk could not bin (see the window
//            above), is resolved by nucleus_row with the maximum known.
// The passes of the path not taken exit at once.
// ===========================================================================
// A chunk's record: its window's slots, then kmax, l0, the spare sums (units
// of exp((l - l0) / T), and of the grid), lmax and ok.
constexpr int kNucPartStride = kNucBins + 8;
enum : int32_t { kNucNoCut = 0, kNucCutBin = 1, kNucRedo = 2 };

struct NucState {
  double A, Z;        // mass of the bins before the cut bin; the row's mass (grid unit)
  double B, kmax;     // the grid's offset and the bin of the row's maximum
  double tstar;       // kNucRound + the cut bin
  double gf;          // grid unit -> exp((l - lmax) / T)
  uint64_t kfloor;    // the row's large top-k cut key (0: none)
  int32_t status;     // kNucNoCut (the row's RowCut is written), kNucCutBin, kNucRedo
  uint32_t n;         // keys of the cut bin found by the collect pass
};

__device__ __forceinline__ int nucleus_splits(const int* plan) { return plan[1]; }

// Chunk s of NS over a row of V tokens: boundaries on multiples of 64
// elements (16-byte alignment relative to the row start is kept).
__device__ __forceinline__ void nucleus_chunk(int V, int NS, int s, int* a, int* e) {
  const int c = (((V + NS - 1) / NS) + 63) & ~63;
  const int lo = s * c < V ? s * c : V;
  *a = lo;
  *e = lo + c < V ? lo + c : V;
}

// part: one workgroup per (listed row, chunk); with NS = 1, nucleus_row per
// listed row.
template <typename ET>
__global__ __launch_bounds__(NucShape::NT) void nucleus_part_kernel(const ET* __restrict__ lt, const ET* __restrict__ ld,
                                                           int rows_t, int G, int V, int S,
                                                           float2* __restrict__ part,
                                                           const ReqInfo* __restrict__ info,
                                                           RowCut* __restrict__ cut, Layout L,
                                                           const int* __restrict__ plan,
                                                           const int* __restrict__ list,
                                                           double* __restrict__ hpart) {
  constexpr int NT = NucShape::NT, U = NucShape::U, NW = NT / kWave;
  const int NS = nucleus_splits(plan);
  const int item = blockIdx.x;
  if (item >= plan[0] * NS) return;
  if (NS == 1) {
    const int row = list[item];
    nucleus_row<ET>(row, lt, ld, rows_t, G, V, S, part, info, cut, L,
                    info[row_request(row, rows_t, G)].K > 0);
    return;
  }
  const int r = item / NS, s = item - r * NS;
  const int row = list[r];
  const ReqInfo ri = info[row_request(row, rows_t, G)];
  const ET* rp = row_ptr(L, lt, ld, rows_t, G, row);
  const uint64_t kfloor = ri.K > 0 ? cut[row].kappa : 0ull;
  double* hm = nucleus_hist_lds();
  NucRise* rl = nucleus_rise_lds();
  __shared__ double tab[64];
  __shared__ double red_d[NW];
  const int tid = threadIdx.x;
  const double it = 1.0 / (double)ri.T;
  for (int i = tid; i < kNucBins; i += NT) hm[i] = 0.0;
  if (tid < 64) tab[tid] = exp2((double)tid / 64.0);
  if (tid == 0) rl->n = 0;
  __syncthreads();
  int a, e;
  nucleus_chunk(V, NS, s, &a, &e);
  NucP1 p;
  if (ri.K > 0) {
    // Under a large top-k: the maximum is known; the grid's anchor is it.
    const float lm = nucleus_lmax(part, row, S);
    p = nucleus_pass1<ET, NT, U, false, true>(rp, a, e, false, 0.0, lm, it, kfloor, tab, hm);
  } else {
    p = nucleus_pass1<ET, NT, U, true, false>(rp, a, e, false, 0.0, 0.f, it, 0ull, tab, hm);
  }
  const double sp = block_sum_d<NT>(p.sp, red_d);
  const double sb = block_sum_d<NT>(p.sb, red_d);
  // The chunk's slots as accumulated (each bin's power of two is applied
  // after the merge), then its record.
  double* out = hpart + (size_t)item * kNucPartStride;
  for (int i = tid; i < kNucBins; i += NT) out[i] = hm[i];
  if (tid == 0) {
    out[kNucBins + 0] = p.g.kmax;
    out[kNucBins + 1] = (double)p.l0;
    out[kNucBins + 2] = sp;
    out[kNucBins + 3] = sb;
    out[kNucBins + 4] = (double)p.lmax;
    out[kNucBins + 5] = p.ok ? 1.0 : 0.0;
  }
}

// scan: one workgroup per listed row.
__global__ __launch_bounds__(NucShape::NT) void nucleus_scan_kernel(int rows_t, int G, int S,
                                                                   float2* __restrict__ part,
                                                                   const ReqInfo* __restrict__ info,
                                                                   RowCut* __restrict__ cut,
                                                                   const int* __restrict__ plan,
                                                                   const int* __restrict__ list,
                                                                   const double* __restrict__ hpart,
                                                                   NucState* __restrict__ state) {
  constexpr int NT = NucShape::NT, NW = NT / kWave;
  const int NS = nucleus_splits(plan);
  const int r = blockIdx.x;
  if (NS < 2 || r >= plan[0]) return;
  const int row = list[r];
  const ReqInfo ri = info[row_request(row, rows_t, G)];
  const uint64_t kfloor = ri.K > 0 ? cut[row].kappa : 0ull;
  const bool own_part = ri.K == 0;
  __shared__ double hm[kNucBins];
  __shared__ double incl[NT], red_s[NW], tab[64];
  __shared__ double ck_kmax[kNucMaxSplit], ck_d[kNucMaxSplit];
  __shared__ float ck_lmax[kNucMaxSplit];
  __shared__ double sh_A;
  __shared__ int sh_bin;
  const int tid = threadIdx.x;
  const double* src = hpart + (size_t)r * NS * kNucPartStride;
  const double it = 1.0 / (double)ri.T, C = it * kNucInvStep;
  // The grid's anchor: 0, or the row's maximum under a large top-k.
  const NucGrid g0{ri.K > 0 ? nuc_grid_B((double)nucleus_lmax(part, row, S), C) : kNucRound, C, 0.0};
  const double B = g0.B;
  float lmax = -INFINITY;
  bool ok = true;
  for (int c = 0; c < NS; ++c) {
    const double* rec = src + (size_t)c * kNucPartStride + kNucBins;
    const float lc = (float)rec[4];
    lmax = fmaxf(lmax, lc);
    ok = ok && (lc == -INFINITY || rec[5] != 0.0);
  }
  if (tid < 64) tab[tid] = exp2((double)tid / 64.0);
  if (lmax == -INFINITY || !ok) {
    // No finite logit (no cut), or a chunk that could not bin its tokens
    // (the finish pass bins the row with this maximum).
    if (own_part) nucleus_write_part(part, row, S, lmax, 0.f);
    if (tid == 0) {
      if (lmax == -INFINITY) cut[row] = RowCut{kfloor, lmax, INFINITY};
      NucState st{};
      st.kfloor = kfloor;
      st.status = lmax == -INFINITY ? kNucNoCut : kNucRedo;
      state[r] = st;
    }
    return;
  }
  const double kmax = nuc_t(lmax, g0) - kNucRound;
  const int top = __double2loint(kmax + kNucRound);
  if (tid < NS) {
    const double* rec = src + (size_t)tid * kNucPartStride + kNucBins;
    ck_kmax[tid] = rec[0];
    ck_lmax[tid] = (float)rec[4];
    ck_d[tid] = kmax - rec[0];  // >= 0: how far the chunk's window lies below the row's
  }
  __syncthreads();
  // Slot i of every window holds a bin congruent to i: chunk c's bin at
  // chunk gap jc = (top_c - i) mod kNucBins lies at the row's gap jc + d_c,
  // in the row's window if that is below kNucBins, else below it (spare).
  double sb = 0.0;
  for (int i = tid; i < kNucBins; i += NT) {
    double v = 0.0;
    for (int c = 0; c < NS; ++c) {
      if (ck_lmax[c] == -INFINITY) continue;
      const double x = src[(size_t)c * kNucPartStride + i];
      if (x == 0.0) continue;
      const int topc = __double2loint(ck_kmax[c] + kNucRound);
      const double jr = (double)((topc - i) & (kNucBins - 1)) + ck_d[c];
      if (jr < (double)kNucBins) v += x;
      else sb += x * exp2_64ths(-jr, tab);
    }
    hm[i] = v;
  }
  if (tid < NS && ck_lmax[tid] != -INFINITY) {
    // The chunk's spare sums in the row's grid unit.
    const double* rec = src + (size_t)tid * kNucPartStride + kNucBins;
    sb += rec[3] * exp2_64ths(-ck_d[tid], tab);
    sb += rec[2] * exp2_64(fma(rec[1], C, B - kNucRound - kmax), tab);
  }
  __syncthreads();
  const double Z = nucleus_unfactor<NT>(hm, top, sb, tab, red_s);
  const double gf = exp2_frac64(-fma((double)lmax, C, B - kNucRound - kmax));
  if (own_part) nucleus_write_part(part, row, S, lmax, (float)(Z * gf));
  const double target = (double)ri.top_p * Z;
  nucleus_pick<NT>(hm, top, target, incl, red_s, &sh_bin, &sh_A);
  if (tid == 0) {
    const int jstar = sh_bin;
    if (jstar < 0) cut[row] = RowCut{kfloor, lmax, (float)(1.0 / (Z * gf))};  // no mass: no cut
    NucState st;
    st.A = sh_A;
    st.Z = Z;
    st.B = B;
    st.kmax = kmax;
    st.tstar = kNucRound + (kmax - (double)jstar);
    st.gf = gf;
    st.kfloor = kfloor;
    st.status = jstar < 0 ? kNucNoCut : kNucCutBin;
    st.n = 0u;
    state[r] = st;
  }
}

// collect: one workgroup per (listed row, chunk); keys of the cut bin are
// appended to the row's buffer (the first kNucCap of them are stored).
template <typename ET>
__global__ __launch_bounds__(NucShape::NT) void nucleus_collect_kernel(const ET* __restrict__ lt,
                                                              const ET* __restrict__ ld, int rows_t, int G,
                                                              int V, const ReqInfo* __restrict__ info, Layout L,
                                                              const int* __restrict__ plan,
                                                              const int* __restrict__ list,
                                                              NucState* __restrict__ state,
                                                              uint64_t* __restrict__ gkeys) {
  constexpr int NT = NucShape::NT, U = NucShape::U;
  const int NS = nucleus_splits(plan);
  const int item = blockIdx.x;
  if (NS < 2 || item >= plan[0] * NS) return;
  const int r = item / NS, s = item - r * NS;
  if (state[r].status != kNucCutBin) return;
  const double tstar = state[r].tstar, gB = state[r].B;
  const uint64_t kfloor = state[r].kfloor;
  const int row = list[r];
  const ReqInfo ri = info[row_request(row, rows_t, G)];
  const ET* rp = row_ptr(L, lt, ld, rows_t, G, row);
  const double C = (1.0 / (double)ri.T) * kNucInvStep;
  int a, e;
  nucleus_chunk(V, NS, s, &a, &e);
  uint32_t* cnt = &state[r].n;
  uint64_t* dst = gkeys + (size_t)r * kNucCap;
  nucleus_collect<ET, NT, U>(
      rp, a, e, [&](float l) { return fma((double)l, C, gB) == tstar; },
      [&](float l, int y) {
        const uint64_t k = make_key(l, (uint32_t)y);
        if (kfloor != 0ull && k < kfloor) return;
        const uint32_t pos = atomicAdd(cnt, 1u);
        if (pos < (uint32_t)kNucCap) dst[pos] = k;
      });
}

// finish: one workgroup per listed row.
template <typename ET>
__global__ __launch_bounds__(NucShape::NT) void nucleus_finish_kernel(const ET* __restrict__ lt,
                                                             const ET* __restrict__ ld, int rows_t, int G, int V,
                                                             int S, float2* __restrict__ part,
                                                             const ReqInfo* __restrict__ info,
                                                             RowCut* __restrict__ cut, Layout L,
                                                             const int* __restrict__ plan,
                                                             const int* __restrict__ list,
                                                             const NucState* __restrict__ state,
                                                             const uint64_t* __restrict__ gkeys) {
  constexpr int NT = NucShape::NT;
  const int NS = nucleus_splits(plan);
  const int r = blockIdx.x;
  if (NS < 2 || r >= plan[0]) return;
  const NucState st = state[r];
  if (st.status == kNucNoCut) return;  // the scan wrote the row's cut
  const int row = list[r];
  if (st.status == kNucRedo || st.n > (uint32_t)kNucCap) {
    // A row a chunk could not bin, or an over-full bin (many equal or
    // near-equal logits): the one-workgroup pass with the maximum known.
    nucleus_row<ET>(row, lt, ld, rows_t, G, V, S, part, info, cut, L, true);
    return;
  }
  const ReqInfo ri = info[row_request(row, rows_t, G)];
  uint64_t* keys = reinterpret_cast<uint64_t*>(nucleus_hist_lds());
  __shared__ double tab[64];
  const int tid = threadIdx.x;
  const float lmax = nucleus_lmax(part, row, S);
  const NucGrid g{st.B, (1.0 / (double)ri.T) * kNucInvStep, st.kmax};
  const int n = (int)st.n;
  int n2 = 2;
  while (n2 < n) n2 <<= 1;
  const uint64_t* src = gkeys + (size_t)r * kNucCap;
  for (int i = tid; i < n2; i += NT) keys[i] = i < n ? src[i] : 0ull;
  if (tid < 64) tab[tid] = exp2((double)tid / 64.0);
  __syncthreads();
  block_sort_desc<NT>(keys, n2);
  if (tid < kWave) {
    const double target = (double)ri.top_p * st.Z;
    double zk;
    const int t =
        n > 0 ? wave_walk(keys, n, st.A, target, [&](float l) { return nuc_mass(g, l, tab); }, &zk) : -1;
    if (tid == 0) {
      if (t >= 0) cut[row] = RowCut{keys[t], lmax, (float)(1.0 / (zk * st.gf))};
      else cut[row] = RowCut{st.kfloor, lmax, (float)(1.0 / (st.Z * st.gf))};
    }
  }
}

// ===========================================================================
// Top-k above the candidate capacity, over a full row: the kept set is the k
// largest keys (logit desc, index asc), so it is one cut key kappa, the k-th
// largest key.  kappa is found by radix select over the 64-bit key, 12 bits
// per pass from the top (the row's tokens counted into an LDS histogram of
// the next digit among those sharing the prefix found so far), until the
// bucket holding the k-th key has at most kNucCap keys; the bucket's keys are
// then collected, sorted and the k-th taken.  The same collect pass sums the
// mass of every key above the bucket; the kept mass Z_k adds the bucket's
// kept keys.  Writes cut[row] = {kappa, row maximum, 1 / Z_k} (masses
// exp2((l - max) c), fp32 terms summed in fp64).  Keys are distinct, so at
// most six passes (12, 24, ..., 60, 64 bits) reach a bucket of one key; rows
// of N(0, 9) logits need two.  A nucleus over this law is cut afterwards by
// the nucleus passes, which read kappa as their floor.
// ===========================================================================
constexpr int kCutBits = 12, kCutBins = 1 << kCutBits;

__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
  const int lane = lane_id();
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const uint32_t o = (uint32_t)__shfl_up((int)v, (unsigned)d);
    if (lane >= d) v += o;
  }
  return v;
}

template <typename ET>
__global__ __launch_bounds__(kCutThreads) void kcut_full_kernel(const ET* __restrict__ lt, const ET* __restrict__ ld,
                                                                int rows_t, int G, int V, int S,
                                                                const float2* __restrict__ part,
                                                                const ReqInfo* __restrict__ info,
                                                                RowCut* __restrict__ cut, Layout L) {
  constexpr int NT = kCutThreads, NW = NT / kWave, PER = kCutBins / NT;
  static_assert(kCutBins % NT == 0, "digits per thread");
  const int row = blockIdx.x;
  const ReqInfo ri = info[row_request(row, rows_t, G)];
  if (ri.kind != kReqFull || ri.K <= 0) return;  // uniform over the workgroup
  const ET* rp = row_ptr(L, lt, ld, rows_t, G, row);
  if (!rp) return;  // past the request's draft length
  __shared__ uint32_t hist[kCutBins];
  __shared__ uint64_t keys[kNucCap];
  __shared__ uint32_t red_u[NW];
  __shared__ double red_d[NW];
  __shared__ int sh_digit;
  __shared__ uint32_t sh_need, sh_cnt, sh_n;
  const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;

  float lmax = -INFINITY;
  for (int k = lane; k < S; k += kWave) lmax = fmaxf(lmax, part[(size_t)row * S + k].x);
  lmax = wave_max_f(lmax);
  const float c = ri.c;
  auto in_prefix = [](uint64_t k, uint64_t prefix, int plen) {
    return plen == 0 || (k >> (64 - plen)) == (prefix >> (64 - plen));
  };

  uint64_t prefix = 0ull;
  int plen = 0;
  uint32_t need = (uint32_t)ri.K;  // rank of the cut key among the keys with the prefix (1-based)
  uint32_t cnt = (uint32_t)V;      // keys with the prefix
  while (cnt > (uint32_t)kNucCap && plen < 64) {
    const int nb = 64 - plen < kCutBits ? 64 - plen : kCutBits;
    const int shift = 64 - plen - nb;
    const int nbins = 1 << nb;
    for (int i = tid; i < kCutBins; i += NT) hist[i] = 0u;
    __syncthreads();
    row_foreach<ET, NT, 2>(rp, V, [&](float l, int y) {
      const uint64_t k = make_key(l, (uint32_t)y);
      if (in_prefix(k, prefix, plen)) atomicAdd(&hist[(uint32_t)(k >> shift) & (uint32_t)(nbins - 1)], 1u);
    });
    __syncthreads();
    // Thread t owns positions [PER t, PER t + PER) of the digits in
    // descending order (digit nbins - 1 - position): running counts then
    // rank keys from the largest.
    uint32_t loc = 0u;
    for (int q = 0; q < PER; ++q) {
      const int pos = PER * tid + q;
      if (pos < nbins) loc += hist[nbins - 1 - pos];
    }
    uint32_t inc = wave_incl_scan_u32(loc);
    if (lane == kWave - 1) red_u[w] = inc;
    __syncthreads();
    for (int k = 0; k < w; ++k) inc += red_u[k];
    const uint32_t start = inc - loc;
    if (start < need && need <= inc) {  // exactly one thread
      uint32_t cum = start;
      for (int q = 0; q < PER; ++q) {
        const int d = nbins - 1 - (PER * tid + q);
        const uint32_t h = hist[d];
        if (cum + h >= need) {
          sh_digit = d;
          sh_need = need - cum;
          sh_cnt = h;
          break;
        }
        cum += h;
      }
    }
    __syncthreads();
    prefix |= (uint64_t)(uint32_t)sh_digit << shift;
    plen += nb;
    need = sh_need;
    cnt = sh_cnt;
    __syncthreads();  // every thread has read the choice before the next clear
  }

  // Collect the bucket (at most kNucCap keys) and sum the mass above it.
  if (tid == 0) sh_n = 0u;
  __syncthreads();
  double za = 0.0;
  row_foreach<ET, NT, 2>(rp, V, [&](float l, int y) {
    const uint64_t k = make_key(l, (uint32_t)y);
    if (in_prefix(k, prefix, plen)) {
      const uint32_t pos = atomicAdd(&sh_n, 1u);
      if (pos < (uint32_t)kNucCap) keys[pos] = k;
    } else if (plen > 0 && (k >> (64 - plen)) > (prefix >> (64 - plen))) {
      za += (double)__builtin_amdgcn_exp2f((l - lmax) * c);
    }
  });
  za = wave_sum_d(za);
  if (lane == 0) red_d[w] = za;
  __syncthreads();
  double zabove = 0.0;
  for (int k = 0; k < NW; ++k) zabove += red_d[k];
  const int n = sh_n < (uint32_t)kNucCap ? (int)sh_n : kNucCap;
  int n2 = 2;
  while (n2 < n) n2 <<= 1;
  for (int i = n + tid; i < n2; i += NT) keys[i] = 0ull;
  __syncthreads();
  block_sort_desc<NT>(keys, n2);
  if (w == 0) {
    // The kept part of the bucket: its `need` largest keys.
    double zb = 0.0;
    for (int i = lane; i < (int)need && i < n; i += kWave)
      zb += (double)__builtin_amdgcn_exp2f((key_value(keys[i]) - lmax) * c);
    zb = wave_sum_d(zb);
    if (lane == 0) {
      const uint64_t kappa = need >= 1u && (int)need <= n ? keys[need - 1] : 0ull;
      cut[row] = RowCut{kappa, lmax, (float)(1.0 / (zabove + zb))};
    }
  }
}

// ===========================================================================
// Acceptance probability of every draft position: beta_j = sum_y
// min(p_j(y), q_j(y)) (page "초안 모델로 생성 속도를 높이는 추측 디코딩",
// section "수락률 α와 기대 속도 향상": alpha is its expectation).  Launched
// only when a caller asks for beta.
// ===========================================================================

// Top-k requests with draft logits (MODE 0) or probabilities (MODE 2): one
// wave per (request, position), over the kept tokens of p.  MODE 0 sorts q's
// kept tokens by token index in the wave's LDS and searches them.
template <int MODE>
__global__ __launch_bounds__(256) void beta_topk_kernel(const uint64_t* __restrict__ cand,
                                                        const float* __restrict__ qp, int B, int G, int kstride,
                                                        int rows_t, const ReqInfo* __restrict__ info, Layout L,
                                                        float* __restrict__ beta) {
  __shared__ uint64_t qs_sh[MODE == 0 ? 4 : 1][MODE == 0 ? 1024 : 1];
  const int w = threadIdx.x / kWave, lane = lane_id();
  const int pos = blockIdx.x * 4 + w;
  if (pos >= B * G) return;  // wave-uniform; no workgroup barrier below
  const int b = pos / G, j = pos - b * G;
  const ReqInfo ri = info[b];
  if (ri.kind != kReqTopk || j >= L.len(b, G)) return;
  const int K = ri.K;
  const float c = ri.c;
  const uint64_t* pk = cand + ((size_t)b * (G + 1) + j) * kstride;
  const CandStats sp = cand_stats(pk, K, c);
  float part = 0.f;
  if (MODE == 0) {
    const uint64_t* qk = cand + ((size_t)rows_t + (size_t)b * G + j) * kstride;
    const CandStats sq = cand_stats(qk, K, c);
    // q's kept tokens as ((index + 1) << 32 | value bits), sorted descending.
    uint64_t* qs = qs_sh[MODE == 0 ? w : 0];
    int n2 = kWave;
    while (n2 < K) n2 <<= 1;
    for (int i = lane; i < n2; i += kWave) {
      uint64_t e = 0ull;
      if (i < K) {
        const uint64_t k = qk[i];
        if (k) e = ((uint64_t)(key_index(k) + 1u) << 32) | (uint64_t)__float_as_uint(key_value(k));
      }
      qs[i] = e;
    }
    wave_lds_sync();
    wave_sort_desc(qs, n2);
    for (int i = lane; i < K; i += kWave) {
      const uint64_t k = pk[i];
      if (!k) continue;
      const uint32_t y1 = key_index(k) + 1u;
      const float p = __builtin_amdgcn_exp2f((key_value(k) - sp.m) * c) * sp.inv_z;
      float q = 0.f;
      int lo = 0, hi = n2 - 1;
      while (lo <= hi) {
        const int mid = (lo + hi) >> 1;
        const uint32_t idx = (uint32_t)(qs[mid] >> 32);
        if (idx == y1) {
          q = __builtin_amdgcn_exp2f((__uint_as_float((uint32_t)qs[mid]) - sq.m) * c) * sq.inv_z;
          break;
        }
        if (idx > y1) lo = mid + 1;
        else hi = mid - 1;
      }
      part += fminf(p, q);
    }
  } else {
    const float* qrow = qp + L.tok(b, G, j) * (size_t)L.ds;
    for (int i = lane; i < K; i += kWave) {
      const uint64_t k = pk[i];
      if (!k) continue;
      const float p = __builtin_amdgcn_exp2f((key_value(k) - sp.m) * c) * sp.inv_z;
      part += fminf(p, qrow[key_index(k)]);
    }
  }
  part = wave_sum_f(part);
  if (lane == 0) beta[L.tok(b, G, j)] = part;
}

// Requests without top-k (draft logits or probabilities): one workgroup per
// (request, position) reads both rows once more (16-byte vectors), with the
// stats (or nucleus cuts) of the row pass.  QP: q given as fp32
// probabilities.
template <typename ET, bool QP>
__global__ __launch_bounds__(256) void beta_full_kernel(const ET* __restrict__ lt, const ET* __restrict__ ld,
                                                        const float* __restrict__ qp,
                                                        const float2* __restrict__ part, int G, int V, int S,
                                                        int rows_t, const ReqInfo* __restrict__ info,
                                                        const RowCut* __restrict__ cut, Layout L,
                                                        float* __restrict__ beta) {
  constexpr int NT = 256, NW = NT / kWave, EPV = Elem<ET>::kPerVec;
  const int b = blockIdx.x / G, j = blockIdx.x - b * G;
  const ReqInfo ri = info[b];
  if (ri.kind != kReqFull || j >= L.len(b, G)) return;  // uniform over the workgroup
  const float c = ri.c;
  const bool nuc = ri.cut != 0;
  const size_t rt = (size_t)b * (G + 1) + j, rd = (size_t)rows_t + (size_t)b * G + j;
  // Row stats: the nucleus cut, or the merged softmax partials.
  float mp, izp, mq = 0.f, izq = 0.f;
  uint64_t kp = 0ull, kq = 0ull;
  if (nuc) {
    const RowCut a = cut[rt];
    mp = a.m;
    izp = a.inv_z;
    kp = a.kappa;
    if (!QP) {
      const RowCut d = cut[rd];
      mq = d.m;
      izq = d.inv_z;
      kq = d.kappa;
    }
  } else {
    float Z;
    merge_row_lane(part + rt * S, S, c, mp, Z);
    izp = 1.f / Z;
    if (!QP) {
      merge_row_lane(part + rd * S, S, c, mq, Z);
      izq = 1.f / Z;
    }
  }
  const ET* rp = lt + L.trow(b, G, j) * (size_t)L.ts;
  const size_t dq = L.tok(b, G, j) * (size_t)L.ds;
  const ET* rq = QP ? nullptr : ld + dq;
  const float* rqp = QP ? qp + dq : nullptr;
  auto term = [&](float l, float lq, int y) -> float {
    float p = __builtin_amdgcn_exp2f((l - mp) * c) * izp;
    if (nuc && make_key(l, (uint32_t)y) < kp) p = 0.f;
    float q = lq;  // QP: the given probability
    if (!QP) {
      q = __builtin_amdgcn_exp2f((lq - mq) * c) * izq;
      if (nuc && make_key(lq, (uint32_t)y) < kq) q = 0.f;
    }
    return fminf(p, q);
  };
  Slice<ET> sl(rp, 0, V);
  const bool q_vec = !QP && ((((uintptr_t)rp) ^ ((uintptr_t)rq)) & 15u) == 0u;
  const uint4* vp = sl.vecs();
  const uint4* vq = q_vec ? (const uint4*)(rq + sl.head) : nullptr;
  float acc = 0.f;
  const int tid = threadIdx.x;
  if (tid < sl.nscalar()) {
    const int y = sl.scalar_index(tid);
    acc += term(Elem<ET>::load1(rp + y), QP ? rqp[y] : Elem<ET>::load1(rq + y), y);
  }
  for (int i = tid; i < sl.nvec; i += NT) {
    float fp[EPV], fq[EPV];
    Elem<ET>::unpack(load_stream(vp + i), fp);
    const int y0 = sl.vec_index0(i);
    if (q_vec) {
      Elem<ET>::unpack(load_stream(vq + i), fq);
    } else {
#pragma unroll
      for (int k = 0; k < EPV; ++k) fq[k] = QP ? rqp[y0 + k] : Elem<ET>::load1(rq + y0 + k);
    }
#pragma unroll
    for (int k = 0; k < EPV; ++k) acc += term(fp[k], fq[k], y0 + k);
  }
  acc = wave_sum_f(acc);
  __shared__ float red[NW];
  if (lane_id() == 0) red[tid / kWave] = acc;
  __syncthreads();
  if (tid == 0) {
    float t = 0.f;
    for (int k = 0; k < NW; ++k) t += red[k];
    beta[L.tok(b, G, j)] = t;
  }
}

// ===========================================================================
// Sampler-match verification ([P3] "mlxcel의 프롬프트 조회" on the manual
// page: a proposal is accepted only if it equals the token the target's
// sampler draws at that position).  Node i of request b (0 = the root, i >= 1
// the draft token X[i-1], parent given or i - 1) has target row (b, i); every
// node gets a fresh sample from its row's adjusted law by the Exp(1) race on
// the stream of (b, i) (temperature 0: the row's argmax); the walk from the
// root follows the child whose token equals the sample (the lowest-indexed
// one) and emits the sample where no child matches.
// ===========================================================================

// One race descriptor per target row of a request without top-k (n: the
// node, rb: the request); other rows get n = -1.  One thread per row.
__global__ __launch_bounds__(256) void match_prep_kernel(const float2* __restrict__ part, int S, int rows_t, int G,
                                                         const ReqInfo* __restrict__ info,
                                                         const RowCut* __restrict__ cut, Layout L,
                                                         RaceDesc* __restrict__ rdesc,
                                                         unsigned long long* __restrict__ rslots) {
  const int row = blockIdx.x * 256 + threadIdx.x;
  if (row >= rows_t) return;
  const int b = row / (G + 1), j = row - b * (G + 1);
  RaceDesc d;
  d.n = -1;
  d.mask_tok = -1;
  d.resid = 0;
  d.rb = b;
  d.mp = d.inv_zp = d.mq = d.inv_zq = 0.f;
  d.c = 0.f;
  d.pad2[0] = d.pad2[1] = d.pad2[2] = 0;
  d.kp = d.kq = 0ull;
  d.prow = d.qrow = 0;
  const ReqInfo ri = info[b];
  if (ri.kind == kReqFull && j <= L.len(b, G)) {
    d.n = j;
    d.c = ri.c;
    if (ri.cut) {
      const RowCut rc = cut[row];
      d.mp = rc.m;
      d.inv_zp = rc.inv_z;
      d.kp = rc.kappa;
    } else {
      float M, Z;
      merge_row_lane(part + (size_t)row * S, S, ri.c, M, Z);
      d.mp = M;
      d.inv_zp = 1.f / Z;
    }
    d.prow = (int64_t)(L.trow(b, G, j) * (size_t)L.ts);
  }
  rdesc[row] = d;
  rslots[3 * (size_t)row] = 0ull;
}

// Samples of the rows of top-k requests: the Exp(1) race over the kept
// tokens.  One wave per row.
__global__ __launch_bounds__(256) void sample_topk_kernel(const uint64_t* __restrict__ cand, int kstride, int rows_t,
                                                          int G, const ReqInfo* __restrict__ info, Layout L,
                                                          uint32_t k0, uint32_t k1, int32_t* __restrict__ samples) {
  const int w = threadIdx.x / kWave, lane = lane_id();
  const int row = blockIdx.x * 4 + w;
  if (row >= rows_t) return;
  const int b = row / (G + 1), j = row - b * (G + 1);
  const ReqInfo ri = info[b];
  if (ri.kind != kReqTopk || j > L.len(b, G)) return;
  const uint64_t* pk = cand + (size_t)row * kstride;
  const CandStats sp = cand_stats(pk, ri.K, ri.c);
  uint64_t best = 0ull;
  for (int i = lane; i < ri.K; i += kWave) {
    const uint64_t k = pk[i];
    if (!k) continue;
    const uint32_t y = key_index(k);
    const float p = __builtin_amdgcn_exp2f((key_value(k) - sp.m) * ri.c) * sp.inv_z;
    if (p > 0.f) {
      const uint4 r = race_block(k0, k1, (uint32_t)b, (uint32_t)j, y);
      const float E = (y & 1u) ? exp1_from_words(r.z, r.w) : exp1_from_words(r.x, r.y);
      const uint64_t kk = make_key(p * __builtin_amdgcn_rcpf(E), y);
      best = kk > best ? kk : best;
    }
  }
  best = wave_max_u64(best);
  if (lane == 0) samples[row] = best ? (int32_t)key_index(best) : -1;
}

// Samples of full rows: race_full_kernel runs over (row, vocabulary split)
// with one descriptor per row (match_prep_kernel), the one-stage Exp(1) race
// over the row's kept tokens on the race stream of (request, node); this
// pass moves each row's winning key into its sample (-1 if no token had
// mass, which a row's own maximum rules out).  One thread per row.
__global__ __launch_bounds__(256) void match_samples_kernel(int rows_t, const RaceDesc* __restrict__ desc,
                                                            const unsigned long long* __restrict__ slots,
                                                            int32_t* __restrict__ samples) {
  const int row = blockIdx.x * 256 + threadIdx.x;
  if (row >= rows_t || desc[row].n < 0) return;
  const unsigned long long win = slots[3 * (size_t)row];
  samples[row] = win ? (int32_t)key_index(win) : -1;
}

// The walk, one wave per request: p_parent(x) of every node (its acceptance
// probability once the parent is reached; also beta), then the path.
template <typename ET>
__global__ __launch_bounds__(64) void match_walk_kernel(const ET* __restrict__ lt, const float2* __restrict__ part,
                                                        const uint64_t* __restrict__ part64,
                                                        const uint64_t* __restrict__ cand, int kstride, int S, int G,
                                                        int V, const ReqInfo* __restrict__ info,
                                                        const RowCut* __restrict__ cut, Layout L,
                                                        const int32_t* __restrict__ X,
                                                        const int32_t* __restrict__ parents,
                                                        const int32_t* __restrict__ samples,
                                                        int32_t* __restrict__ out, int32_t* __restrict__ nacc,
                                                        int32_t* __restrict__ path_nodes,
                                                        float* __restrict__ p_draft, float* __restrict__ q_draft,
                                                        Stats stats, int* __restrict__ err) {
  const int b = blockIdx.x, lane = lane_id();
  const ReqInfo ri = info[b];
  const size_t r0 = (size_t)b * (G + 1);
  if (ri.kind == kReqInvalid) {  // outputs other than the path cleared by classify_kernel
    if (path_nodes)
      for (int j = lane; j <= G; j += kWave) path_nodes[r0 + j] = -1;
    return;
  }
  const int g = L.len(b, G);
  auto sample_of = [&](int i) -> int {
    if (ri.kind == kReqGreedy) {
      uint64_t m = 0ull;
      for (int k = 0; k < S; ++k) {
        const uint64_t v = part64[(r0 + i) * S + k];
        m = v > m ? v : m;
      }
      return (int)key_index(m);
    }
    return samples[r0 + i];
  };
  auto parent_of = [&](int i) -> int { return parents ? parents[L.tok(b, G, i - 1)] : i - 1; };
  // Acceptance probability of node i (>= 1): p_parent(x_i).
  auto write_node = [&](int i, float pd, bool valid) {
    const size_t t = L.tok(b, G, i - 1);
    if (p_draft) p_draft[t] = pd;
    if (q_draft) q_draft[t] = valid ? 1.f : 0.f;
    if (stats.beta) stats.beta[t] = pd;
  };
  if (ri.kind == kReqTopk) {
    for (int i = 1; i <= g; ++i) {  // wave-cooperative per node
      const int x = X[L.tok(b, G, i - 1)];
      const bool valid = x >= 0 && x < V;
      const uint64_t* pk = cand + (r0 + parent_of(i)) * kstride;
      const CandStats sp = cand_stats(pk, ri.K, ri.c);
      const float pd = valid ? cand_prob(pk, ri.K, sp, ri.c, x) : 0.f;
      if (lane == 0) {
        write_node(i, pd, valid);
        if (!valid) atomicOr(err, kErrBadToken);
      }
    }
  } else {
    for (int i0 = 1; i0 <= g; i0 += kWave) {
      const int i = i0 + lane;
      if (i > g) continue;
      const int x = X[L.tok(b, G, i - 1)];
      const bool valid = x >= 0 && x < V;
      const int pa = parent_of(i);
      float pd = 0.f;
      if (valid) {
        if (ri.kind == kReqGreedy) {
          pd = x == sample_of(pa) ? 1.f : 0.f;
        } else {
          const size_t rp = r0 + pa;
          const float l = Elem<ET>::load1(lt + L.trow(b, G, pa) * (size_t)L.ts + x);
          if (ri.cut) {
            const RowCut rc = cut[rp];
            pd = make_key(l, (uint32_t)x) < rc.kappa ? 0.f : __builtin_amdgcn_exp2f((l - rc.m) * ri.c) * rc.inv_z;
          } else {
            float M, Z;
            merge_row_lane(part + rp * S, S, ri.c, M, Z);
            pd = __builtin_amdgcn_exp2f((l - M) * ri.c) / Z;
          }
        }
      }
      write_node(i, pd, valid);
      if (!valid) atomicOr(err, kErrBadToken);
    }
  }
  // Walk from the root.
  int cur = 0, d = 0;
  for (;;) {
    const int t = sample_of(cur);
    int child = -1;
    if (t < 0) {
      // no sample (cannot happen: a row's law always has positive mass)
    } else if (!parents) {
      if (cur < g && X[L.tok(b, G, cur)] == t) child = cur + 1;
    } else {
      for (int i0 = 1; i0 <= g && child < 0; i0 += kWave) {
        const int i = i0 + lane;
        const bool m = i <= g && parents[L.tok(b, G, i - 1)] == cur && X[L.tok(b, G, i - 1)] == t;
        const uint64_t mask = ballot(m);
        if (mask) child = i0 + (int)__builtin_ctzll(mask);
      }
    }
    if (lane == 0) out[r0 + d] = t;
    if (child < 0) break;
    if (lane == 0 && path_nodes) path_nodes[r0 + d] = child;
    ++d;
    cur = child;
  }
  for (int j = lane; j <= G; j += kWave) {
    if (j > d) out[r0 + j] = -1;
    if (path_nodes && j >= d) path_nodes[r0 + j] = -1;
  }
  if (lane == 0) {
    nacc[b] = d;
    count_round(stats, b, g, d);
  }
}

}  // namespace sv
