// HIP kernels of libspecverify for gfx950.
//
// Launch sequence of one call (every kernel on the caller's stream):
//   row pass     one workgroup per (logit row, vocabulary split):
//                  softmax rows  -> (max, sum exp) partials
//                  top-k rows    -> exactly k (value, index) keys per row
//                  argmax rows   -> (max, lowest index) partial keys
//   accept pass  one wave per request: merge the partials, p(x_j), q(x_j),
//                the accept tests, the first-rejection scan, outputs; with
//                top-k it also runs the recovered/bonus race over the k kept
//                tokens
//   race pass    (no top-k) one workgroup per (request, vocabulary split):
//                the Exp(1) race over the full row n; the last workgroup of a
//                request to finish writes its token
//
// Method: page "vLLM speculative decoding이 기각 토큰을 다시 뽑는 이유"
// (velog): the per-position test of section "드래프트가 제안하고 타깃이
// 판정한다", the residual of section "왜 하필 max(p − q, 0)인가", the fp64
// uniform and the Exp(1) race of section "vLLM 커널은 이 규칙을 어떻게
// 옮겼나", the one-hot draft and the greedy kernel of section "기본값 greedy
// 드래프트에서도 분포가 지켜질까"; Algorithm 1 on page "초안 모델로 생성
// 속도를 높이는 추측 디코딩", section "방법".
#pragma once

#include "sv_device.hpp"

// Build knobs of the top-k row pass (measured defaults).
#ifndef SV_TOPK_COMPACT_INLINE
#define SV_TOPK_COMPACT_INLINE __noinline__  // rare; kept out of the streaming loop's code
#endif

namespace sv {

// Error word bits.
constexpr int kErrBadToken = 1;
constexpr int kErrBadParam = 2;
constexpr int kErrBadLayout = 4;

// Where rows, draft tokens and per-position outputs live.  Kernels index
// their own workspace by the padded (request, position) pair: target row
// b * (G + 1) + j, draft row b * G + j.  A ragged call (cu not null) gives
// request b the draft positions cu[b] .. cu[b + 1] - 1 (g_b of them): its
// target rows are packed at cu[b] + b + j (j <= g_b); its draft rows, draft
// tokens and p / q outputs at cu[b] + j (j < g_b).  Strides are in elements.
// The classify pass has checked cu (cu[0] = 0, 0 <= g_b <= G) before any
// kernel reads it.
struct Layout {
  const int32_t* cu;
  int64_t ts, ds;
  __device__ __forceinline__ int len(int b, int G) const { return cu ? cu[b + 1] - cu[b] : G; }
  __device__ __forceinline__ size_t tok(int b, int G, int j) const {
    return cu ? (size_t)cu[b] + (size_t)j : (size_t)b * (size_t)G + (size_t)j;
  }
  __device__ __forceinline__ size_t trow(int b, int G, int j) const {
    return cu ? (size_t)cu[b] + (size_t)b + (size_t)j : (size_t)b * (size_t)(G + 1) + (size_t)j;
  }
};

// Optional statistics of a call: per-position acceptance probability beta
// (laid out like the draft tokens) and per-request counters [B][3] (+=
// draft positions, accepted drafts, 1).
struct Stats {
  float* beta;
  int64_t* counters;
};

// Adds this call's round to request b's counters (one writer per request).
__device__ __forceinline__ void count_round(const Stats& st, int b, int g, int n) {
  if (!st.counters) return;
  int64_t* c = st.counters + 3 * (size_t)b;
  c[0] += g;
  c[1] += n;
  c[2] += 1;
}

// Bitonic sort of a[0, n) into descending order by one wave (n a power of
// two; LDS).
template <typename PK>
__device__ __forceinline__ void wave_sort_desc(PK a, int n) {
  const int lane = lane_id();
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = lane; i < n / 2; i += kWave) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool desc = (lo & size) == 0;
        const uint64_t x = a[lo], y = a[hi];
        if ((x < y) == desc) {
          a[lo] = y;
          a[hi] = x;
        }
      }
      wave_lds_sync();
    }
  }
}

// The logit row of padded row index `row` (target rows first), or null if
// the request has no such row (ragged calls).
template <typename ET>
__device__ __forceinline__ const ET* row_ptr(const Layout& L, const ET* lt, const ET* ld, int rows_t, int G,
                                             int row) {
  if (row < rows_t) {
    const int b = row / (G + 1), j = row - b * (G + 1);
    if (L.cu && j > L.len(b, G)) return nullptr;
    return lt + L.trow(b, G, j) * (size_t)L.ts;
  }
  const int r = row - rows_t, b = r / G, j = r - b * G;
  if (L.cu && j >= L.len(b, G)) return nullptr;
  return ld + L.tok(b, G, j) * (size_t)L.ds;
}

// Per-request settings of a batch call (written by the classify pass).  In a
// call with one setting for every request the kernels get a null pointer.
enum : int32_t { kReqInvalid = 0, kReqGreedy = 1, kReqTopk = 2, kReqFull = 3 };
struct __align__(16) ReqInfo {
  int32_t kind;  // kReq*
  float c;       // log2(e) / T (sampled requests)
  int32_t K;     // top-k: of a kReqTopk request (its candidates), or of a
                 // kReqFull request whose k exceeds the candidate capacity
                 // (a cut over the full row); 0 otherwise
  float top_p;   // < 1: nucleus cut
  float T;       // temperature
  int32_t cut;   // kReqFull: 1 if its rows carry a RowCut (top-p or large k)
  int32_t pad[2];
};

// Request of a logit row: rows [0, rows_t) are target rows b * (G + 1) + j,
// the rest draft rows b * G + j.
__device__ __forceinline__ int row_request(int row, int rows_t, int G) {
  return row < rows_t ? row / (G + 1) : (row - rows_t) / G;
}

// Nucleus cut of a full row: tokens with key >= kappa are kept (kappa 0: no
// cut); m is the row's largest logit and inv_z the inverse kept mass in units
// of exp2((l - m) * c).
struct __align__(16) RowCut {
  uint64_t kappa;
  float m, inv_z;
};

// Per-request race descriptor written by the accept pass (no top-k).
struct __align__(16) RaceDesc {
  int32_t n;         // race position (first rejection or G); -1: no race
  int32_t mask_tok;  // one-hot: token removed from the residual, else -1
  int32_t resid;     // 1: weights max(p - q, 0), q from draft logits; 2: q given as
                     // probabilities; 0: weights p
  int32_t rb;        // request of the race stream (counter (y >> 1, n, rb, 1))
  float mp, inv_zp, mq, inv_zq;  // softmax stats of target row n / draft row n
  float c;                       // log2(e) / T of the request
  int32_t pad2[3];
  uint64_t kp, kq;               // nucleus cuts of target row n / draft row n (0: none)
  int64_t prow, qrow;            // element offsets of target row n and of draft row n
};

// A contiguous slice [a, e) of one logit row split into a scalar head (until
// the first 16-byte boundary), full 16-byte vectors, and a scalar tail.
template <typename ET>
struct Slice {
  const ET* row;
  int a, head, nvec, tail0, e;
  __device__ __forceinline__ Slice(const ET* r, int a_, int e_) : row(r), a(a_), e(e_) {
    constexpr int EPV = Elem<ET>::kPerVec;
    const uintptr_t addr = (uintptr_t)(r + a_);
    const int mis = (int)(((16u - (uint32_t)(addr & 15u)) & 15u) / sizeof(ET));
    const int n = e_ - a_;
    head = mis < n ? mis : n;
    nvec = (n - head) / EPV;
    tail0 = a_ + head + nvec * EPV;
  }
  __device__ __forceinline__ const uint4* vecs() const { return (const uint4*)(row + a + head); }
  __device__ __forceinline__ int vec_index0(int i) const { return a + head + i * Elem<ET>::kPerVec; }
  // Scalar elements: k in [0, nscalar) -> element index.
  __device__ __forceinline__ int nscalar() const { return head + (e - tail0); }
  __device__ __forceinline__ int scalar_index(int k) const { return k < head ? a + k : tail0 + (k - head); }
};

// ===========================================================================
// Row pass 1: online softmax partials.  For each (row, split): m = max logit,
// s = sum_y exp2((l_y - m) * c) with c = log2(e) / T.
// ===========================================================================
//
// Single-setting calls on dense rows may also pass `gath` and `slots`: the
// workgroup whose split holds the draft token x_j of its row stores that
// row's logit l(x_j) in gath[row] (the accept decisions then need no gather
// of their own), and split 0 of target row (b, 0) clears request b's race
// slot for the race that follows.
template <typename ET, int NT, int U>
__global__ __launch_bounds__(NT) void rows_softmax_kernel(const ET* __restrict__ lt, const ET* __restrict__ ld,
                                                          int rows_t, int V, int S, int seg, float c,
                                                          float2* __restrict__ part, int* __restrict__ err,
                                                          const ReqInfo* __restrict__ info, int G, Layout L,
                                                          const int32_t* __restrict__ X = nullptr,
                                                          float* __restrict__ gath = nullptr,
                                                          unsigned long long* __restrict__ slots = nullptr) {
  constexpr int EPV = Elem<ET>::kPerVec;
  const int blk = blockIdx.x;
  const int row = blk / S, s = blk - row * S;
  if (info) {
    // Batch call: only rows of requests without top-k; per-request T.  Rows
    // with top-p and no top-k are left to the nucleus pass, which finds
    // their maximum and mass in the read that bins them.
    const ReqInfo ri = info[row_request(row, rows_t, G)];
    if (ri.kind != kReqFull || (ri.top_p < 1.f && ri.K == 0)) return;
    c = ri.c;
  } else if (blk == 0 && threadIdx.x == 0) {
    *err = 0;
  }
  const ET* rp = row_ptr(L, lt, ld, rows_t, G, row);
  if (!rp) return;  // past the request's draft length
  const int a = s * seg;
  const int e = min(V, a + seg);
  // The row's draft token (one wave-uniform load, issued before the stream
  // and used after it).
  int xg = -1;
  if (gath) {
    const int b = row < rows_t ? row / (G + 1) : (row - rows_t) / G;
    const int j = row < rows_t ? row - b * (G + 1) : (row - rows_t) - b * G;
    if (j < G) xg = X[(size_t)b * G + j];
    if (slots && threadIdx.x == 0 && s == 0 && row < rows_t && j == 0) slots[3 * (size_t)b] = 0ull;
  }
  Slice<ET> sl(rp, a, e);
  float m = -INFINITY, sum = 0.f;
  const int tid = threadIdx.x;
  if (tid < sl.nscalar()) {
    m = Elem<ET>::load1(rp + sl.scalar_index(tid));
    sum = (m == -INFINITY) ? 0.f : 1.f;
  }
  const uint4* vp = sl.vecs();
  const uint4 ninf = make_uint4(Elem<ET>::kNegInfWord, Elem<ET>::kNegInfWord, Elem<ET>::kNegInfWord,
                                Elem<ET>::kNegInfWord);
  for (int i0 = tid; i0 < sl.nvec; i0 += NT * U) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * NT;
      v[u] = i < sl.nvec ? load_stream(vp + i) : ninf;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float f[EPV];
      Elem<ET>::unpack(v[u], f);
      float vm = f[0];
#pragma unroll
      for (int k = 1; k < EPV; ++k) vm = fmaxf(vm, f[k]);
      if (vm > m) {
        sum = (m == -INFINITY) ? 0.f : sum * __builtin_amdgcn_exp2f((m - vm) * c);
        m = vm;
      }
      if (m != -INFINITY) {
        // (l - m) c, not fma(l, c, -m c): the rounding of m c (up to |m c|
        // 2^-24, large at low temperature) would shift every exponent.
#pragma unroll
        for (int k = 0; k < EPV; ++k) sum += __builtin_amdgcn_exp2f((f[k] - m) * c);
      }
    }
  }
  if (tid == NT - 1 && xg >= a && xg < e) gath[row] = Elem<ET>::load1(rp + xg);
  wave_lse(m, sum, c);
  __shared__ float2 red[NT / kWave];
  const int w = tid / kWave;
  if (lane_id() == 0) red[w] = make_float2(m, sum);
  __syncthreads();
  if (tid == 0) {
    float M = red[0].x, Sm = red[0].y;
    for (int k = 1; k < NT / kWave; ++k) lse_merge(M, Sm, red[k].x, red[k].y, c);
    part[blk] = make_float2(M, Sm);
  }
}

// ===========================================================================
// Row pass 2: argmax partials (greedy).  Key = (value, lowest index).
// ===========================================================================
template <typename ET, int NT, int U>
__global__ __launch_bounds__(NT) void rows_argmax_kernel(const ET* __restrict__ lt, int V, int S, int seg,
                                                         uint64_t* __restrict__ part, int* __restrict__ err,
                                                         const ReqInfo* __restrict__ info, int G, Layout L) {
  constexpr int EPV = Elem<ET>::kPerVec;
  const int blk = blockIdx.x;
  const int row = blk / S, s = blk - row * S;
  if (info) {
    // Batch call: target rows of temperature-0 requests only.
    if (info[row / (G + 1)].kind != kReqGreedy) return;
  } else if (blk == 0 && threadIdx.x == 0) {
    *err = 0;
  }
  const ET* rp = row_ptr(L, lt, lt, row + 1, G, row);
  if (!rp) return;  // past the request's draft length
  const int a = s * seg;
  const int e = min(V, a + seg);
  Slice<ET> sl(rp, a, e);
  const int tid = threadIdx.x;
  float bv = -INFINITY;
  int bi = -1;
  uint64_t best = 0;
  if (tid < sl.nscalar()) {
    const int y = sl.scalar_index(tid);
    best = make_key(Elem<ET>::load1(rp + y), (uint32_t)y);
  }
  const uint4* vp = sl.vecs();
  for (int i0 = tid; i0 < sl.nvec; i0 += NT * U) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * NT;
      v[u] = i < sl.nvec ? load_stream(vp + i) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * NT;
      if (i < sl.nvec) {
        float f[EPV];
        Elem<ET>::unpack(v[u], f);
        float vm = f[0];
#pragma unroll
        for (int k = 1; k < EPV; ++k) vm = fmaxf(vm, f[k]);
        // Strict '>' in ascending index order keeps the first maximum: a
        // vector only matters if its largest value beats the running one,
        // and then through the first of its elements that holds it.
        if (vm > bv || bi < 0) {
          int kk = 0;  // the lowest k with f[k] == vm
#pragma unroll
          for (int k = EPV - 1; k >= 0; --k)
            if (f[k] == vm) kk = k;
          bv = vm;
          bi = sl.vec_index0(i) + kk;
        }
      }
    }
  }
  if (bi >= 0) {
    const uint64_t kv = make_key(bv, (uint32_t)bi);
    best = kv > best ? kv : best;
  }
  best = wave_max_u64(best);
  __shared__ uint64_t red[NT / kWave];
  if (lane_id() == 0) red[tid / kWave] = best;
  __syncthreads();
  if (tid == 0) {
    uint64_t m = red[0];
    for (int k = 1; k < NT / kWave; ++k) m = red[k] > m ? red[k] : m;
    part[blk] = m;
  }
}

// ===========================================================================
// Row pass 3: exact top-k in one read of the row.
//
// WPR waves per row (RPB rows per workgroup) stream interleaved 16-byte
// vectors.  A vector that may hold a key above the running threshold tau is
// stashed in the wave's LDS; stashed vectors are appended in bulk to the
// wave's key buffer, keeping only keys above the current tau.  Compactions
// (a coarse histogram bound, or an exact radix select when the buffer is
// nearly full) raise tau and publish bounds through LDS: every published
// value has at least K retained keys at or above it, so it is a lower bound
// of the row's K-th largest key and any wave may skip elements at or below
// it.  At the end the surviving keys of the row's waves are merged, selected
// once more and written in descending key order.
// ===========================================================================

// K-th largest of the n (> K) distinct keys in buf, by radix select over the
// bytes of the key (from the top; bytes shared by every key are skipped).
// Returns a threshold t such that exactly K keys are >= t: the K-th largest
// key itself, or (when the last examined digit bucket is taken whole) that
// bucket's prefix with zero low bits.
template <typename PK, typename PH>
__device__ uint64_t wave_select_kth(PK buf, int n, int K, PH hist) {
  const int lane = lane_id();
  uint64_t orv = 0, andv = ~0ull;
  for (int i = lane; i < n; i += kWave) {
    const uint64_t k = buf[i];
    orv |= k;
    andv &= k;
  }
  orv = wave_or_u64(orv);
  andv = wave_and_u64(andv);
  const uint64_t varying = orv ^ andv;
  uint64_t prefix = 0, pmask = 0;
  int need = K;
  for (int shift = 56; shift >= 0; shift -= 8) {
    const uint64_t byte_mask = 0xFFull << shift;
    if ((varying & byte_mask) == 0) {
      prefix |= andv & byte_mask;
      pmask |= byte_mask;
      continue;
    }
    for (int bkt = lane; bkt < 256; bkt += kWave) hist[bkt] = 0u;
    wave_lds_sync();
    for (int i = lane; i < n; i += kWave) {
      const uint64_t k = buf[i];
      if ((k & pmask) == prefix)
        __hip_atomic_fetch_add(&hist[(uint32_t)(k >> shift) & 255u], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    wave_lds_sync();
    const uint32_t h0 = hist[4 * lane + 0], h1 = hist[4 * lane + 1];
    const uint32_t h2 = hist[4 * lane + 2], h3 = hist[4 * lane + 3];
    const uint32_t lsum = h0 + h1 + h2 + h3;
    // Inclusive suffix sum over lanes: counts of buckets >= 4 * lane.
    uint32_t incl = lsum;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const uint32_t t = (uint32_t)__shfl_down((int)incl, o);
      if (lane + o < kWave) incl += t;
    }
    const uint32_t above = incl - lsum;
    const bool mine = above < (uint32_t)need && (uint32_t)need <= incl;
    int dl = 0;
    uint32_t ab = above, hd = 0;
    if (mine) {
      if (ab + h3 >= (uint32_t)need) {
        dl = 3; hd = h3;
      } else {
        ab += h3;
        if (ab + h2 >= (uint32_t)need) {
          dl = 2; hd = h2;
        } else {
          ab += h2;
          if (ab + h1 >= (uint32_t)need) {
            dl = 1; hd = h1;
          } else {
            ab += h1;
            dl = 0; hd = h0;
          }
        }
      }
    }
    const uint64_t owner = ballot(mine);
    const int src = (int)__builtin_ctzll(owner);
    const int d = __shfl(4 * lane + dl, src);
    const uint32_t above_d = (uint32_t)__shfl((int)ab, src);
    const uint32_t count_d = (uint32_t)__shfl((int)hd, src);
    need -= (int)above_d;
    prefix |= (uint64_t)(uint32_t)d << shift;
    pmask |= byte_mask;
    wave_lds_sync();  // every lane has read hist before the next pass clears it
    if (count_d == (uint32_t)need) return prefix;  // the whole bucket is taken
  }
  return prefix;
}

// Keeps the keys >= thr, in order, in place; returns how many.
template <typename PK>
__device__ int wave_keep_ge(PK buf, int n, uint64_t thr) {
  const int lane = lane_id();
  int out = 0;
  for (int base = 0; base < n; base += kWave) {
    const int i = base + lane;
    const uint64_t k = i < n ? buf[i] : 0ull;
    const bool keep = i < n && k >= thr;
    const uint64_t m = ballot(keep);
    if (keep) buf[out + lanes_below(m)] = k;
    out += __builtin_popcountll(m);
  }
  wave_lds_sync();
  return out;
}

// Key bounds from the value bits only, in one histogram pass: for rank r
// (r = r1, r2) returns q such that at least r of the n keys are >= q (q keeps
// the bits above the highest bit where the keys' values differ, the next 8
// bits of the bucket holding the r-th largest, and zeros below); 0 when
// n < r.
template <typename PK, typename PH>
__device__ uint2 wave_coarse_select2(PK buf, int n, int r1, int r2, PH hist) {
  const int lane = lane_id();
  uint32_t orv = 0u, andv = ~0u;
  for (int i = lane; i < n; i += kWave) {
    const uint32_t h = (uint32_t)(buf[i] >> 32);
    orv |= h;
    andv &= h;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    orv |= (uint32_t)__shfl_xor((int)orv, m);
    andv &= (uint32_t)__shfl_xor((int)andv, m);
  }
  const uint32_t var = orv ^ andv;
  if (var == 0u) return make_uint2(n >= r1 ? andv : 0u, n >= r2 ? andv : 0u);
  const int hb = 31 - __builtin_clz(var);
  const int shift = hb >= 7 ? hb - 7 : 0;
  const uint32_t high = (shift + 8 >= 32) ? 0u : (~0u << (shift + 8));
  for (int bkt = lane; bkt < 256; bkt += kWave) hist[bkt] = 0u;
  wave_lds_sync();
  for (int i = lane; i < n; i += kWave)
    __hip_atomic_fetch_add(&hist[((uint32_t)(buf[i] >> 32) >> shift) & 255u], 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_WORKGROUP);
  wave_lds_sync();
  const uint32_t h0 = hist[4 * lane + 0], h1 = hist[4 * lane + 1];
  const uint32_t h2 = hist[4 * lane + 2], h3 = hist[4 * lane + 3];
  const uint32_t lsum = h0 + h1 + h2 + h3;
  uint32_t incl = lsum;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t t = (uint32_t)__shfl_down((int)incl, o);
    if (lane + o < kWave) incl += t;
  }
  const uint32_t above = incl - lsum;
  uint32_t res[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int r = t == 0 ? r1 : r2;
    res[t] = 0u;
    if (n < r) continue;  // wave-uniform
    const uint32_t need = (uint32_t)r;
    const bool mine = above < need && need <= incl;
    int dl = 0;
    if (mine) {
      if (above + h3 >= need) dl = 3;
      else if (above + h3 + h2 >= need) dl = 2;
      else if (above + h3 + h2 + h1 >= need) dl = 1;
    }
    const uint64_t owner = ballot(mine);
    const int d = __shfl(4 * lane + dl, (int)__builtin_ctzll(owner));
    res[t] = (andv & high) | ((uint32_t)d << shift);
  }
  wave_lds_sync();
  return make_uint2(res[0], res[1]);
}

// Lower bound of the row's K-th largest key from what the waves published:
// every wave w retains >= ceil(K/NW) keys >= q[w], so >= K keys are >= min_w
// q[w]; the publisher of kth retains K keys >= kth.
template <int NW, typename PK>
__device__ __forceinline__ uint64_t shared_bound(PK q_sh, PK kth_sh) {
  uint64_t mn = ~0ull;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint64_t q = __hip_atomic_load(q_sh + w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    mn = q < mn ? q : mn;
  }
  const uint64_t k = __hip_atomic_load(kth_sh, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  return k > mn ? k : mn;
}

// Shrinks one wave's candidate buffer and returns the wave's new threshold
// (insert keys > tau).  Publishes a coarse ceil(K/NW)-th bound; if the buffer
// is still above `guard` keys (or `exact` is set and it holds more than K),
// the exact K-th largest is selected and published too.  Only keys below a
// valid bound are ever dropped.
template <int NW, typename PK, typename PH>
__device__ SV_TOPK_COMPACT_INLINE uint64_t topk_compact(PK bw, PH hw, PH cntp, PK q_sh, PK kth_sh, int w, uint64_t tau,
                                                       int K, int guard, bool exact) {
  const int lane = lane_id();
  const int K4 = (K + NW - 1) / NW;
  wave_lds_sync();
  int n = __builtin_amdgcn_readfirstlane(*cntp);
  if (!exact && n >= K4) {
    const uint2 q = wave_coarse_select2(bw, n, K4, K, hw);
    if (lane == 0) {
      __hip_atomic_fetch_max(q_sh + w, (uint64_t)q.x << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      if (q.y) __hip_atomic_fetch_max(kth_sh, (uint64_t)q.y << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  }
  const uint64_t sb = shared_bound<NW>(q_sh, kth_sh);
  tau = sb > tau ? sb : tau;
  n = wave_keep_ge(bw, n, tau);
  if (n > guard || (exact && n > K)) {
    const uint64_t kth = wave_select_kth(bw, n, K, hw);
    if (lane == 0) __hip_atomic_fetch_max(kth_sh, kth, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    tau = kth > tau ? kth : tau;
    n = wave_keep_ge(bw, n, tau);
  }
  // The combined bound goes to one word that the streaming loop reads.
  if (lane == 0) {
    *cntp = (uint32_t)n;
    __hip_atomic_fetch_max(kth_sh + 1, tau, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  wave_lds_sync();
  return tau;
}

#ifndef SV_TOPK_TRIG_STEP
#define SV_TOPK_TRIG_STEP 32  // keys added between two compactions of a wave buffer
#endif

// Float value below which no key can beat tau (-inf for keys at or below
// the -inf keys).
__device__ __forceinline__ float tau_value(uint64_t tau) {
  const uint32_t o = (uint32_t)(tau >> 32);
  return (o <= 0x007FFFFFu) ? -INFINITY : key_value(tau);
}

// Appends this lane's elements with key > tau to the wave buffer at
// positions from a ballot prefix count; returns the new (wave-uniform) count.
template <int EPV, typename PK>
__device__ __forceinline__ int topk_append(const float* f, uint32_t idx0, uint32_t vmask, uint64_t tau, float tau_v,
                                           PK bw, int cnt) {
#pragma unroll
  for (int k = 0; k < EPV; ++k) {
    const bool cand = (vmask & (1u << k)) && f[k] >= tau_v;
    if (ballot(cand) == 0ull) continue;
    const uint64_t key = cand ? make_key(f[k], idx0 + (uint32_t)k) : 0ull;
    const bool hit = key > tau;
    const uint64_t m = ballot(hit);
    if (hit) bw[cnt + lanes_below(m)] = key;
    cnt += __builtin_popcountll(m);
  }
  return cnt;
}

#ifndef SV_TOPK_STASH_FLUSH
#define SV_TOPK_STASH_FLUSH 64  // stashed vectors that trigger the bulk append
#endif
constexpr int kTopkStashFlush = SV_TOPK_STASH_FLUSH;
constexpr int kTopkStash = kTopkStashFlush + kWave;  // a step adds at most one wave's worth

// Prefilter for bf16 vectors against a positive threshold: for positive
// values the bf16 bit pattern orders like a signed 16-bit integer, and every
// negative pattern is below every positive one.
__device__ __forceinline__ bool bf16_vec_reaches(const uint4& v, short thr16) {
  typedef short s2 __attribute__((ext_vector_type(2)));
  const s2 a = __builtin_bit_cast(s2, v.x), b = __builtin_bit_cast(s2, v.y);
  const s2 c = __builtin_bit_cast(s2, v.z), d = __builtin_bit_cast(s2, v.w);
  const s2 m = __builtin_elementwise_max(__builtin_elementwise_max(a, b), __builtin_elementwise_max(c, d));
  const short mm = m.x > m.y ? m.x : m.y;
  return mm >= thr16;
}

// WPR waves share one row; a workgroup holds RPB rows.  Fewer waves per row
// track the row's running k-th key more tightly (fewer keys pass the
// filter); more waves per row shorten each row's latency.
template <typename ET, int CAPW, int U, int WPR, int RPB>
__global__ __launch_bounds__(WPR * RPB * kWave) void rows_topk_kernel(const ET* __restrict__ lt,
                                                                       const ET* __restrict__ ld, int rows_t,
                                                                       int nrows, int V, int K,
                                                                       uint64_t* __restrict__ cand,
                                                                       int* __restrict__ err,
                                                                       const ReqInfo* __restrict__ info, int G,
                                                                       int kstride, Layout L) {
  constexpr int NT = WPR * RPB * kWave, NW = NT / kWave;
  constexpr int GT = WPR * kWave;   // threads per row
  constexpr int EPV = Elem<ET>::kPerVec;
  constexpr int kGuard = CAPW - kWave * EPV;  // room for one more step's keys
  __shared__ uint64_t buf[NW][CAPW];
  __shared__ uint32_t hist[NW][256];
  __shared__ uint64_t q_sh[NW];
  __shared__ uint64_t kth_sh[RPB][2];  // per row: best k-th bound; best combined bound
  __shared__ uint32_t cnt_sh[NW];
  __shared__ uint32_t lm_sh[RPB][WPR * kWave];
  __shared__ uint64_t stash_v[NW][2 * kTopkStash];  // 16-byte vectors as two words
  __shared__ uint32_t stash_i[NW][kTopkStash];
  const int tid = threadIdx.x, w = tid / kWave;
  const int g = w / WPR, wg = w % WPR, gtid = tid % GT;
  const int row = blockIdx.x * RPB + g;
  bool row_ok = row < nrows;
  const ET* rp = nullptr;
  if (info) {
    // Batch call: rows of top-k requests only, each with its own k (<= the
    // stride); a skipped row streams nothing but joins every barrier.
    const ReqInfo ri = info[row_request(row_ok ? row : 0, rows_t, G)];
    row_ok = row_ok && ri.kind == kReqTopk;
    if (row_ok) rp = row_ptr(L, lt, ld, rows_t, G, row);
    row_ok = row_ok && rp != nullptr;
    K = __builtin_amdgcn_readfirstlane(row_ok ? ri.K : 1);  // one row per wave: wave-uniform
  } else {
    if (blockIdx.x == 0 && tid == 0) *err = 0;
    if (row_ok) rp = row_ptr(L, lt, ld, rows_t, G, row);
  }
  if (tid < NW) {
    q_sh[tid] = 0ull;
    cnt_sh[tid] = 0u;
  }
  if (tid < 2 * RPB) kth_sh[tid / 2][tid % 2] = 0ull;
  __syncthreads();
  if (!row_ok) rp = lt;  // not read: the slice is empty
  Slice<ET> sl(rp, 0, row_ok ? V : 0);
  lds_u64* bw = (lds_u64*)buf[w];
  lds_u32* hw = (lds_u32*)hist[w];
  lds_u32* cntp = (lds_u32*)&cnt_sh[w];
  lds_u64* qg = (lds_u64*)(q_sh + g * WPR);
  lds_u64* kg = (lds_u64*)kth_sh[g];
  const int K4 = (K + WPR - 1) / WPR;
  int trig = K4 + SV_TOPK_TRIG_STEP;
  uint64_t tau = 0ull;
  float tau_v = -INFINITY;
  int cnt = 0;  // keys in this wave's buffer (wave-uniform; in LDS only around compactions)

  // Scalar head and tail (fewer than 2 * EPV elements): one per thread.
  {
    float f[EPV];
#pragma unroll
    for (int k = 0; k < EPV; ++k) f[k] = -INFINITY;
    uint32_t idx = 0, vm = 0u;
    if (gtid < sl.nscalar()) {
      idx = (uint32_t)sl.scalar_index(gtid);
      f[0] = Elem<ET>::load1(rp + idx);
      vm = 1u;
    }
    cnt = topk_append<EPV>(f, idx, vm, tau, tau_v, bw, cnt);
  }
  const uint4* vp = sl.vecs();
  const uint32_t full = (1u << EPV) - 1u;

  // Candidate vectors are stashed, not walked: a step where some lane's
  // vector may hold a key >= tau writes those lanes' vectors (and their first
  // token index) to the wave's LDS stash with one masked store, so a step
  // costs a few instructions however many lanes it stops.  Once the stash
  // holds a wave's worth of vectors, every lane takes one of them and the
  // wave appends their keys > tau (the current tau: tau only rises, so every
  // key that beats the row's final bound was stashed and is appended).
  int sc = 0;  // stashed vectors (wave-uniform)
  lds_u64* sv_w = (lds_u64*)stash_v[w];
  lds_u32* si_w = (lds_u32*)stash_i[w];
  auto flush = [&]() {
    wave_lds_sync();
    for (int e0 = 0; e0 < sc; e0 += kWave) {
      const int e = e0 + lane_id();
      float f[EPV];
      uint32_t idx0 = 0u, vm = 0u;
      if (e < sc) {
        const uint64_t lo = sv_w[2 * e], hi = sv_w[2 * e + 1];
        Elem<ET>::unpack(make_uint4((uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)), f);
        idx0 = si_w[e];
        vm = full;
      } else {
#pragma unroll
        for (int k = 0; k < EPV; ++k) f[k] = -INFINITY;
      }
      if (cnt > kGuard) {
        if (lane_id() == 0) *cntp = (uint32_t)cnt;
        tau = topk_compact<WPR>(bw, hw, cntp, qg, kg, wg, tau, K, kGuard, false);
        tau_v = tau_value(tau);
        cnt = (int)__builtin_amdgcn_readfirstlane(*cntp);
      }
      cnt = topk_append<EPV>(f, idx0, vm, tau, tau_v, bw, cnt);
      if (cnt > trig) {
        if (lane_id() == 0) *cntp = (uint32_t)cnt;
        tau = topk_compact<WPR>(bw, hw, cntp, qg, kg, wg, tau, K, kGuard, false);
        tau_v = tau_value(tau);
        cnt = (int)__builtin_amdgcn_readfirstlane(*cntp);
        trig = max(K4 + SV_TOPK_TRIG_STEP, cnt + SV_TOPK_TRIG_STEP);
      }
    }
    sc = 0;
    wave_lds_sync();
  };
  auto filter = [&](const uint4& vv, int i, bool packed, short thr16) {
    const bool valid = i < sl.nvec;
    bool maybe;
    if (packed) {
      maybe = valid && bf16_vec_reaches(vv, thr16);
    } else {
      float f[EPV];
      Elem<ET>::unpack(vv, f);
      float vm = f[0];
#pragma unroll
      for (int k = 1; k < EPV; ++k) vm = fmaxf(vm, f[k]);
      maybe = valid && vm >= tau_v;
    }
    const uint64_t mm = ballot(maybe);
    if (mm == 0ull) return;
    if (maybe) {
      const int slot = sc + lanes_below(mm);
      sv_w[2 * slot] = (uint64_t)vv.x | ((uint64_t)vv.y << 32);
      sv_w[2 * slot + 1] = (uint64_t)vv.z | ((uint64_t)vv.w << 32);
      si_w[slot] = (uint32_t)sl.vec_index0(i);
    }
    sc += __builtin_popcountll(mm);
    if (sc >= kTopkStashFlush) flush();
  };

  // Warm start.  Every lane's largest element of the row's first batch is a
  // distinct element, so the K-th largest of those WPR * 64 maxima has at
  // least K elements at or above it: a valid threshold from the start, far
  // above what one wave's first batch alone would give.
  uint4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int i = u * GT + gtid;
    v[u] = sl.nvec > 0 ? load_stream(vp + (i < sl.nvec ? i : sl.nvec - 1)) : make_uint4(0u, 0u, 0u, 0u);
  }
  {
    float lm = -INFINITY;
    bool has = false;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (u * GT + gtid < sl.nvec) {
        float f[EPV];
        Elem<ET>::unpack(v[u], f);
#pragma unroll
        for (int k = 0; k < EPV; ++k) lm = fmaxf(lm, f[k]);
        has = true;
      }
    }
    lm_sh[g][wg * kWave + lane_id()] = has ? ord32(lm) : 0u;
    __syncthreads();
    if (K <= WPR * kWave) {
      uint32_t mine[WPR];
#pragma unroll
      for (int r = 0; r < WPR; ++r) mine[r] = lm_sh[g][r * kWave + lane_id()];
      // Largest t with at least K maxima >= t, i.e. the K-th largest.
      uint32_t t = 0u;
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t c = t | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int r = 0; r < WPR; ++r) cnt += __builtin_popcountll(ballot(mine[r] >= c));
        if (cnt >= K) t = c;
      }
      if (t != 0u) {
        const uint64_t t0 = ((uint64_t)t << 32) - 1ull;
        if (t0 > tau) tau = t0;
      }
    }
    tau_v = tau_value(tau);
    const bool packed = sizeof(ET) == 2 && tau_v > 0.f;
    const short thr16 = (short)(__float_as_uint(tau_v) >> 16);
    // Rolling pipeline: once a slot is filtered its register is refilled
    // with the slot's next vector, so U - 1 loads per lane stay in flight and
    // no register is moved (a move would wait for every pending load).
#pragma unroll
    for (int u = 0; u < U; ++u) {
      filter(v[u], u * GT + gtid, packed, thr16);
      if (sl.nvec > 0) v[u] = load_stream(vp + min(GT * U + u * GT + gtid, sl.nvec - 1));
    }
  }
  for (int i0 = GT * U; i0 < sl.nvec; i0 += GT * U) {
    {
      const uint64_t sb = __hip_atomic_load(kg + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      if (sb > tau) tau = sb;
      tau_v = tau_value(tau);
    }
    const bool packed = sizeof(ET) == 2 && tau_v > 0.f;
    const short thr16 = (short)(__float_as_uint(tau_v) >> 16);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      filter(v[u], i0 + u * GT + gtid, packed, thr16);
      // Past the end the request repeats the last vector (one cache line).
      v[u] = load_stream(vp + min(i0 + GT * U + u * GT + gtid, sl.nvec - 1));
    }
  }
  if (sc > 0) flush();
  // Each wave reduces to at most K keys, then the row's first wave merges.
  if (lane_id() == 0) *cntp = (uint32_t)cnt;
  tau = topk_compact<WPR>(bw, hw, cntp, qg, kg, wg, tau, K, kGuard, true);
  __syncthreads();
  // A wave that compacted early may hold keys below the final bound: they
  // are dropped here (valid: the bound has K retained keys at or above it).
  const uint64_t fin = shared_bound<WPR>(qg, kg);
  int mine = wave_keep_ge(bw, (int)cnt_sh[w], fin > tau ? fin : tau);
  __syncthreads();
  if (lane_id() == 0) cnt_sh[w] = (uint32_t)mine;
  __syncthreads();
  lds_u64* b0 = (lds_u64*)buf[g * WPR];
  if (wg > 0) {
    int off = 0;
    for (int k = 0; k < wg; ++k) off += (int)cnt_sh[g * WPR + k];
    for (int i = lane_id(); i < mine; i += kWave) b0[off + i] = bw[i];
  }
  __syncthreads();
  if (wg == 0 && row_ok) {
    int n = 0;
    for (int k = 0; k < WPR; ++k) n += (int)cnt_sh[g * WPR + k];
    if (n > K) {
      const uint64_t thr = wave_select_kth(b0, n, K, hw);
      n = wave_keep_ge(b0, n, thr);
    }
    // The kept set is exact, but the order in which its keys were appended
    // depends on when each wave saw which bound; the row's candidates are
    // written in descending key order so that every later sum over them runs
    // in the same order on every call.
    uint64_t* dst = cand + (size_t)row * kstride;
    if (K <= kWave) {
      const int lane = lane_id();
      uint64_t v = lane < n ? b0[lane] : 0ull;
      // Bitonic sort across the wave's lanes (one key each), descending.
#pragma unroll
      for (int size = 2; size <= kWave; size <<= 1) {
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
          const uint64_t o = shfl_xor_u64(v, stride);
          const bool keep_max = ((lane & stride) == 0) == ((lane & size) == 0);
          v = keep_max ? (o > v ? o : v) : (o < v ? o : v);
        }
      }
      if (lane < K) dst[lane] = v;
    } else {
      int n2 = kWave;
      while (n2 < n) n2 <<= 1;
      for (int i = n + lane_id(); i < n2; i += kWave) b0[i] = 0ull;
      wave_lds_sync();
      wave_sort_desc(b0, n2);
      for (int i = lane_id(); i < K; i += kWave) dst[i] = i < n ? b0[i] : 0ull;
    }
  }
}

// ===========================================================================
// Accept pass, top-k rows: one wave per request.
// ===========================================================================
struct CandStats {
  float m;        // max kept logit
  float inv_z;    // 1 / sum exp2((l - m) c) over the kept tokens
  double inv_zd;  // the same in fp64 (the sum itself is exact, unit_fixed)
};

__device__ __forceinline__ CandStats cand_stats(const uint64_t* ck, int K, float c) {
  const int lane = lane_id();
  float m = -INFINITY;
  for (int i = lane; i < K; i += kWave) {
    const uint64_t k = ck[i];
    if (k) m = fmaxf(m, key_value(k));
  }
  m = wave_max_f(m);
  uint64_t z = 0ull;
  for (int i = lane; i < K; i += kWave) {
    const uint64_t k = ck[i];
    if (k) z += unit_fixed(__builtin_amdgcn_exp2f((key_value(k) - m) * c));
  }
  z = wave_sum_u64(z);
  return CandStats{m, 1.f / ((float)z * 0x1.0p-52f), 1.0 / ((double)z * 0x1.0p-52)};
}

// Probability of a kept token of logit v under stats st (fp32): the weight
// of a race on p.  Residual weights are taken in fp64 (test_prob).
__device__ __forceinline__ float cand_p(float v, CandStats st, float c) {
  return __builtin_amdgcn_exp2f((v - st.m) * c) * st.inv_z;
}

// Below this an fp32 probability may have lost digits to underflow; the
// accept test then takes it again in fp64 (test_prob).
constexpr float kTestProbFloor = 0x1.0p-100f;

// Race key of a candidate whose residual d = p - q (fp64) is positive, with
// variate E: the score w / E in the log domain, log2(d) - log2(E), so that
// residuals far below fp32's range (down to fp64's) keep their order.  Every
// residual race over candidates takes its keys this way.
__device__ __forceinline__ uint64_t resid_key(double d, float E, uint32_t y) {
  int ex;
  const double m = frexp(d, &ex);  // d = m 2^ex, m in [1/2, 1)
  return make_key((float)ex + __builtin_amdgcn_logf((float)m) - __builtin_amdgcn_logf(E), y);
}

// Probability of token x under a kept set (0 if x is not kept), and in *pd
// the same for the accept test: the fp32 value, or test_prob's below
// kTestProbFloor (a wave-uniform branch, almost never taken).
__device__ __forceinline__ float cand_prob(const uint64_t* ck, int K, CandStats st, float c, int x, double* pd) {
  const int lane = lane_id();
  float p = 0.f;
  float v = -INFINITY;
  for (int i = lane; i < K; i += kWave) {
    const uint64_t k = ck[i];
    if (k && (int)key_index(k) == x) {
      p = __builtin_amdgcn_exp2f((key_value(k) - st.m) * c) * st.inv_z;
      v = key_value(k);
    }
  }
  p = wave_sum_f(p);
  *pd = p;
  if (p < kTestProbFloor) {
    v = wave_max_f(v);
    *pd = v == -INFINITY ? 0.0 : test_prob(v, st.m, c, (double)st.inv_z);
  }
  return p;
}
__device__ __forceinline__ float cand_prob(const uint64_t* ck, int K, CandStats st, float c, int x) {
  double unused;
  return cand_prob(ck, K, st, c, x, &unused);
}

// MODE 0: prob (q from draft candidates), 1: onehot, 2: q given as
// probabilities (qp rows).  One 256-thread workgroup per request: the four
// waves compute p(x_j), q(x_j) and the accept test of different positions;
// wave 0 then finds the first rejection and runs the race over the kept
// tokens of row n.  Dynamic LDS: G bytes.
template <int MODE>
__global__ __launch_bounds__(256) void accept_topk_kernel(const uint64_t* __restrict__ cand,
                                                          const int32_t* __restrict__ X, int G, int V, int K,
                                                          int rows_t, float c, uint32_t k0, uint32_t k1,
                                                          int32_t* __restrict__ out, int32_t* __restrict__ nacc,
                                                          float* __restrict__ p_draft, float* __restrict__ q_draft,
                                                          int* __restrict__ err, const ReqInfo* __restrict__ info,
                                                          int kstride, Layout L, const float* __restrict__ qp,
                                                          Stats stats) {
  extern __shared__ uint8_t rejected[];  // [G]
  __shared__ uint64_t qkeys[1024];
  __shared__ int n_sh;
  const int b = blockIdx.x;
  if (info) {
    // Batch call: top-k requests only, with their own k and T.
    const ReqInfo ri = info[b];
    if (ri.kind != kReqTopk) return;
    K = ri.K;
    c = ri.c;
  }
  const int g = L.len(b, G);  // this request's draft positions
  const int lane = lane_id(), w = threadIdx.x / kWave;
  constexpr int NW = 4;
  const uint64_t* ct = cand + (size_t)b * (G + 1) * kstride;
  const uint64_t* cd = cand + ((size_t)rows_t + (size_t)b * G) * kstride;
  for (int j = w; j < g; j += NW) {
    const size_t xj = L.tok(b, G, j);
    const int x = X[xj];
    const bool valid = x >= 0 && x < V;
    const CandStats sp = cand_stats(ct + (size_t)j * kstride, K, c);
    double pd = 0.0, qd = valid ? 1.0 : 0.0;
    const float px = valid ? cand_prob(ct + (size_t)j * kstride, K, sp, c, x, &pd) : 0.f;
    float qx = valid ? 1.f : 0.f;
    if (MODE == 0) {
      const CandStats sq = cand_stats(cd + (size_t)j * kstride, K, c);
      qx = valid ? cand_prob(cd + (size_t)j * kstride, K, sq, c, x, &qd) : 0.f;
    } else if (MODE == 2) {
      qx = valid ? qp[xj * (size_t)L.ds + x] : 0.f;
      qd = qx;
    }
    if (lane == 0) {
      if (p_draft) p_draft[xj] = px;
      if (q_draft) q_draft[xj] = qx;
      if (MODE == 1 && stats.beta) stats.beta[xj] = px;  // one-hot q: beta = p(x)
      if (!valid) atomicOr(err, kErrBadToken);
      const uint4 r = accept_block(k0, k1, (uint32_t)b, (uint32_t)j);
      const double u = unit_from_words(r.x, r.y);
      const bool acc = valid && (MODE != 1 ? (qd > 0.0 && u <= pd / qd) : (u <= pd));
      rejected[j] = acc ? 0 : 1;
    }
  }
  __syncthreads();
  if (w == 0) {
    int n = g;
    for (int j0 = 0; j0 < g; j0 += kWave) {
      const uint64_t m = ballot(j0 + lane < g && rejected[j0 + lane] != 0);
      if (m) {
        n = j0 + (int)__builtin_ctzll(m);
        break;
      }
    }
    if (lane == 0) n_sh = n;
  }
  __syncthreads();
  const int n = n_sh;
  if (MODE == 0 && n < g) {
    const uint64_t* cq = cd + (size_t)n * kstride;
    for (int i = threadIdx.x; i < K; i += 256) qkeys[i] = cq[i];
  }
  __syncthreads();
  if (w != 0) return;
  // Recovered (n < g) or bonus (n == g) token by the Exp(1) race over the
  // kept tokens of target row n.
  const uint64_t* cp = ct + (size_t)n * kstride;
  const CandStats sp = cand_stats(cp, K, c);
  CandStats sq{0.f, 0.f, 0.0};
  if (MODE == 0 && n < g) sq = cand_stats(qkeys, K, c);
  const int xn = n < g ? X[L.tok(b, G, n)] : -1;
  const float* qrow = (MODE == 2 && n < g) ? qp + L.tok(b, G, n) * (size_t)L.ds : nullptr;
  uint64_t best_w = 0ull, best_p = 0ull;
  for (int i = lane; i < K; i += kWave) {
    const uint64_t k = cp[i];
    if (!k) continue;
    const uint32_t y = key_index(k);
    const float p = cand_p(key_value(k), sp, c);
    float wgt = p;
    double wd = 0.0;  // the residual (MODE 0 / 2, n < g)
    if (n < g) {
      // The residual in fp64 from the exact kept-set sums: where the two
      // laws nearly agree it is a small difference of numbers near 1.
      if (MODE == 0) {
        double q = 0.0;
        for (int t = 0; t < K; ++t) {
          const uint64_t kq = qkeys[t];
          if (kq && key_index(kq) == y) q = test_prob(key_value(kq), sq.m, c, sq.inv_zd);
        }
        wd = test_prob(key_value(k), sp.m, c, sp.inv_zd) - q;
      } else if (MODE == 2) {
        wd = test_prob(key_value(k), sp.m, c, sp.inv_zd) - (double)qrow[y];
      } else if ((int)y == xn) {
        wgt = 0.f;
      }
    }
    const uint4 r = race_block(k0, k1, (uint32_t)b, (uint32_t)n, y);
    const float E = (y & 1u) ? exp1_from_words(r.z, r.w) : exp1_from_words(r.x, r.y);
    if ((MODE == 0 || MODE == 2) && n < g) {
      if (wd > 0.0) {
        const uint64_t kk = resid_key(wd, E, y);
        best_w = kk > best_w ? kk : best_w;
      }
    } else if (wgt > 0.f) {
      const uint64_t kk = make_key(wgt * __builtin_amdgcn_rcpf(E), y);
      best_w = kk > best_w ? kk : best_w;
    }
    if (p > 0.f) {
      const uint64_t kk = make_key(p * __builtin_amdgcn_rcpf(E), y);
      best_p = kk > best_p ? kk : best_p;
    }
  }
  best_w = wave_max_u64(best_w);
  best_p = wave_max_u64(best_p);
  const uint64_t win = best_w ? best_w : best_p;  // zero residual mass: race on p
  int32_t* o = out + (size_t)b * (G + 1);
  for (int j = lane; j <= G; j += kWave) {
    int32_t t = -1;
    if (j < n) t = X[L.tok(b, G, j)];
    else if (j == n) t = win ? (int32_t)key_index(win) : -1;
    o[j] = t;
  }
  if (lane == 0) {
    nacc[b] = n;
    count_round(stats, b, g, n);
  }
}

// The same for K <= 64 and gamma <= 16 (every top-k call of the measured
// shapes): one 512-thread workgroup per request stages all of its candidate
// rows in LDS with one coalesced load (lane i of a row's wave holds key i),
// then each of the eight waves takes a position; wave 0 races over row n.
// The arithmetic is that of accept_topk_kernel key for key (the same
// reductions over the same lanes), so both kernels give the same bits.
constexpr int kSmallK = 64, kSmallG = 16;

template <int MODE>
__global__ __launch_bounds__(512) void accept_topk_small_kernel(const uint64_t* __restrict__ cand,
                                                                const int32_t* __restrict__ X, int G, int V, int K,
                                                                int rows_t, float c, uint32_t k0, uint32_t k1,
                                                                int32_t* __restrict__ out, int32_t* __restrict__ nacc,
                                                                float* __restrict__ p_draft,
                                                                float* __restrict__ q_draft, int* __restrict__ err,
                                                                const ReqInfo* __restrict__ info, int kstride,
                                                                Layout L, const float* __restrict__ qp,
                                                                Stats stats) {
  __shared__ uint64_t keys[2 * kSmallG + 1][kSmallK];
  __shared__ uint8_t rejected[kSmallG];
  const int b = blockIdx.x;
  if (info) {
    const ReqInfo ri = info[b];
    if (ri.kind != kReqTopk) return;  // uniform over the workgroup
    K = ri.K;
    c = ri.c;
  }
  const int g = L.len(b, G);
  const int lane = lane_id(), w = threadIdx.x / kWave;
  constexpr int NW = 8;
  const int nt = g + 1, nrow = nt + (MODE == 0 ? g : 0);
  const uint64_t* ct = cand + (size_t)b * (G + 1) * kstride;
  const uint64_t* cd = cand + ((size_t)rows_t + (size_t)b * G) * kstride;
  for (int e = threadIdx.x; e < nrow * kSmallK; e += NW * kWave) {
    const int r = e / kSmallK, i = e - r * kSmallK;
    const uint64_t* src = r < nt ? ct + (size_t)r * kstride : cd + (size_t)(r - nt) * kstride;
    keys[r][i] = i < K ? src[i] : 0ull;
  }
  __syncthreads();
  // Softmax over a kept set held one key per lane: (m, 1 / z) as cand_stats.
  auto stats_of = [&](uint64_t k) -> CandStats {
    const float m = wave_max_f(k ? key_value(k) : -INFINITY);
    const uint64_t z = wave_sum_u64(k ? unit_fixed(__builtin_amdgcn_exp2f((key_value(k) - m) * c)) : 0ull);
    return CandStats{m, 1.f / ((float)z * 0x1.0p-52f), 1.0 / ((double)z * 0x1.0p-52)};
  };
  auto prob_of = [&](uint64_t k, CandStats st, int x, double* pd) -> float {
    const bool hit = k && (int)key_index(k) == x;
    const float p = wave_sum_f(hit ? __builtin_amdgcn_exp2f((key_value(k) - st.m) * c) * st.inv_z : 0.f);
    *pd = p;
    if (p < kTestProbFloor) {  // as cand_prob
      const float v = wave_max_f(hit ? key_value(k) : -INFINITY);
      *pd = v == -INFINITY ? 0.0 : test_prob(v, st.m, c, (double)st.inv_z);
    }
    return p;
  };
  for (int j = w; j < g; j += NW) {
    const size_t xj = L.tok(b, G, j);
    const int x = X[xj];
    const bool valid = x >= 0 && x < V;
    const uint64_t kp = keys[j][lane];
    double pd = 0.0, qd = valid ? 1.0 : 0.0;
    const float px = valid ? prob_of(kp, stats_of(kp), x, &pd) : 0.f;
    float qx = valid ? 1.f : 0.f;
    if (MODE == 0) {
      const uint64_t kq = keys[nt + j][lane];
      qx = valid ? prob_of(kq, stats_of(kq), x, &qd) : 0.f;
    } else if (MODE == 2) {
      qx = valid ? qp[xj * (size_t)L.ds + x] : 0.f;
      qd = qx;
    }
    if (lane == 0) {
      if (p_draft) p_draft[xj] = px;
      if (q_draft) q_draft[xj] = qx;
      if (MODE == 1 && stats.beta) stats.beta[xj] = px;  // one-hot q: beta = p(x)
      if (!valid) atomicOr(err, kErrBadToken);
      const uint4 r = accept_block(k0, k1, (uint32_t)b, (uint32_t)j);
      const double u = unit_from_words(r.x, r.y);
      const bool acc = valid && (MODE != 1 ? (qd > 0.0 && u <= pd / qd) : (u <= pd));
      rejected[j] = acc ? 0 : 1;
    }
  }
  __syncthreads();
  if (w != 0) return;
  const int n = [&] {
    const uint64_t m = ballot(lane < g && rejected[lane] != 0);
    return m ? (int)__builtin_ctzll(m) : g;
  }();
  // Recovered (n < g) or bonus (n == g) token: the Exp(1) race over the kept
  // tokens of target row n; the residual's q(y) is looked up among draft row
  // n's keys by broadcasting them one lane at a time.
  const uint64_t kp = keys[n][lane];
  const CandStats sp = stats_of(kp);
  const int xn = n < g ? X[L.tok(b, G, n)] : -1;
  // q(y) of the residual in fp64 (as accept_topk_kernel), looked up among
  // draft row n's keys by broadcasting them one lane at a time.
  double q = 0.0;
  if (MODE == 0 && n < g) {
    const uint64_t kq = keys[nt + n][lane];
    const CandStats sq = stats_of(kq);
    const double myq = kq ? test_prob(key_value(kq), sq.m, c, sq.inv_zd) : 0.0;
    const uint32_t myqi = kq ? key_index(kq) : 0xFFFFFFFFu;
    const uint32_t y = key_index(kp);
    const uint64_t myqb = (uint64_t)__double_as_longlong(myq);
    for (int t = 0; t < K; ++t) {
      const uint32_t yt = (uint32_t)__builtin_amdgcn_readlane((int)myqi, t);
      const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)myqb, t);
      const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(myqb >> 32), t);
      if (kp && yt == y) q = __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
    }
  } else if (MODE == 2 && n < g && kp) {
    q = (double)qp[L.tok(b, G, n) * (size_t)L.ds + key_index(kp)];
  }
  uint64_t best_w = 0ull, best_p = 0ull;
  if (kp) {
    const uint32_t y = key_index(kp);
    const float p = cand_p(key_value(kp), sp, c);
    float wgt = p;
    if (n < g && MODE == 1 && (int)y == xn) wgt = 0.f;
    const uint4 r = race_block(k0, k1, (uint32_t)b, (uint32_t)n, y);
    const float E = (y & 1u) ? exp1_from_words(r.z, r.w) : exp1_from_words(r.x, r.y);
    if ((MODE == 0 || MODE == 2) && n < g) {
      const double wd = test_prob(key_value(kp), sp.m, c, sp.inv_zd) - q;  // the residual, log-domain key
      if (wd > 0.0) best_w = resid_key(wd, E, y);
    } else if (wgt > 0.f) {
      best_w = make_key(wgt * __builtin_amdgcn_rcpf(E), y);
    }
    if (p > 0.f) best_p = make_key(p * __builtin_amdgcn_rcpf(E), y);
  }
  best_w = wave_max_u64(best_w);
  best_p = wave_max_u64(best_p);
  const uint64_t win = best_w ? best_w : best_p;  // zero residual mass: race on p
  int32_t* o = out + (size_t)b * (G + 1);
  for (int j = lane; j <= G; j += kWave) {
    int32_t t = -1;
    if (j < n) t = X[L.tok(b, G, j)];
    else if (j == n) t = win ? (int32_t)key_index(win) : -1;
    o[j] = t;
  }
  if (lane == 0) {
    nacc[b] = n;
    count_round(stats, b, g, n);
  }
}

// ===========================================================================
// Accept pass, full rows (no top-k): one wave per request.
// ===========================================================================
__device__ __forceinline__ void merge_partials(const float2* part, int S, float c, float& M, float& Z) {
  const int lane = lane_id();
  float m = -INFINITY, s = 0.f;
  for (int k = lane; k < S; k += kWave) {
    const float2 v = part[k];
    lse_merge(m, s, v.x, v.y, c);
  }
  wave_lse(m, s, c);
  M = m;
  Z = s;
}

// Merge of one row's S partials by one lane, in order; the loads run four
// ahead of the merges.
__device__ __forceinline__ void merge_row_lane(const float2* part, int S, float c, float& M, float& Z) {
  float m = -INFINITY, s = 0.f;
  int k = 0;
  for (; k + 4 <= S; k += 4) {
    const float2 v0 = part[k], v1 = part[k + 1], v2 = part[k + 2], v3 = part[k + 3];
    lse_merge(m, s, v0.x, v0.y, c);
    lse_merge(m, s, v1.x, v1.y, c);
    lse_merge(m, s, v2.x, v2.y, c);
    lse_merge(m, s, v3.x, v3.y, c);
  }
  for (; k < S; ++k) {
    const float2 v = part[k];
    lse_merge(m, s, v.x, v.y, c);
  }
  M = m;
  Z = s;
}

// One wave per request; lane j handles position j (chunks of 64 positions):
// merged softmax stats, the gathered logit, p(x_j), q(x_j) and the accept
// test all run in parallel, and the first rejection is one ballot.  In a batch
// call (info not null) only requests without top-k are handled here, each
// with its own T, and rows with a nucleus cut take their stats from `cut`.
// MODE 0: prob, 1: onehot, 2: q given as probabilities (qp rows).
template <typename ET, int MODE>
__global__ __launch_bounds__(64) void accept_full_kernel(const ET* __restrict__ lt, const ET* __restrict__ ld,
                                                         const float2* __restrict__ part,
                                                         const int32_t* __restrict__ X, int G, int V, int S,
                                                         int rows_t, float c, uint32_t k0, uint32_t k1,
                                                         int32_t* __restrict__ out, int32_t* __restrict__ nacc,
                                                         float* __restrict__ p_draft, float* __restrict__ q_draft,
                                                         RaceDesc* __restrict__ desc,
                                                         unsigned long long* __restrict__ slots,
                                                         int* __restrict__ err, const ReqInfo* __restrict__ info,
                                                         const RowCut* __restrict__ cut, Layout L,
                                                         const float* __restrict__ qp, Stats stats) {
  const int b = blockIdx.x;
  const int lane = lane_id();
  bool nuc = false;
  if (info) {
    const ReqInfo ri = info[b];
    if (ri.kind != kReqFull) {
      if (lane == 0) desc[b].n = -1;  // no full-row race for this request
      return;
    }
    c = ri.c;
    nuc = ri.cut != 0;
  }
  const int g = L.len(b, G);  // this request's draft positions
  // Probability of token x (logit l) in padded row r, merged by one lane.
  // *pd: the same for the accept test (test_prob).
  auto prob_lane = [&](size_t r, float l, int x, double* pd) -> float {
    if (nuc) {
      const RowCut rc = cut[r];
      if (make_key(l, (uint32_t)x) < rc.kappa) {
        *pd = 0.0;
        return 0.f;
      }
      *pd = test_prob(l, rc.m, c, (double)rc.inv_z);
      return __builtin_amdgcn_exp2f((l - rc.m) * c) * rc.inv_z;
    }
    float M, Z;
    merge_row_lane(part + r * S, S, c, M, Z);
    *pd = test_prob(l, M, c, 1.0 / (double)Z);
    return __builtin_amdgcn_exp2f((l - M) * c) / Z;
  };
  int n = g;
  for (int j0 = 0; j0 < g; j0 += kWave) {
    const int j = j0 + lane;
    bool rej = false;
    if (j < g) {
      const size_t xj = L.tok(b, G, j);
      const int x = X[xj];
      const bool valid = x >= 0 && x < V;
      const size_t rt = (size_t)b * (G + 1) + j;
      double pd = 0.0, qd = valid ? 1.0 : 0.0;
      const float px =
          valid ? prob_lane(rt, Elem<ET>::load1(lt + L.trow(b, G, j) * (size_t)L.ts + x), x, &pd) : 0.f;
      float qx = valid ? 1.f : 0.f;
      if (MODE == 0) {
        const size_t rd = (size_t)b * G + j;
        qx = valid ? prob_lane((size_t)rows_t + rd, Elem<ET>::load1(ld + xj * (size_t)L.ds + x), x, &qd) : 0.f;
      } else if (MODE == 2) {
        qx = valid ? qp[xj * (size_t)L.ds + x] : 0.f;
        qd = qx;
      }
      if (q_draft) q_draft[xj] = qx;
      if (p_draft) p_draft[xj] = px;
      if (MODE == 1 && stats.beta) stats.beta[xj] = px;  // one-hot q: beta = p(x)
      if (!valid) atomicOr(err, kErrBadToken);
      const uint4 r = accept_block(k0, k1, (uint32_t)b, (uint32_t)j);
      const double u = unit_from_words(r.x, r.y);
      const bool acc = valid && (MODE != 1 ? (qd > 0.0 && u <= pd / qd) : (u <= pd));
      rej = !acc;
    }
    const uint64_t m = ballot(rej);
    if (n == g && m) n = j0 + (int)__builtin_ctzll(m);
  }
  // Stats of padded row r for the race, merged by the whole wave.
  auto race_stats = [&](size_t r, float& M, float& inv_z, uint64_t& kap) {
    if (nuc) {
      const RowCut rc = cut[r];
      M = rc.m;
      inv_z = rc.inv_z;
      kap = rc.kappa;
    } else {
      float Z;
      merge_partials(part + r * S, S, c, M, Z);
      inv_z = 1.f / Z;
      kap = 0ull;
    }
  };
  RaceDesc d;
  d.n = n;
  d.mask_tok = (MODE == 1 && n < g) ? X[L.tok(b, G, n)] : -1;
  d.resid = n < g ? (MODE == 0 ? 1 : (MODE == 2 ? 2 : 0)) : 0;
  d.rb = b;
  race_stats((size_t)b * (G + 1) + n, d.mp, d.inv_zp, d.kp);
  d.mq = 0.f;
  d.inv_zq = 0.f;
  d.kq = 0ull;
  d.c = c;
  d.pad2[0] = d.pad2[1] = d.pad2[2] = 0;
  if (d.resid == 1) race_stats((size_t)rows_t + (size_t)b * G + n, d.mq, d.inv_zq, d.kq);
  d.prow = (int64_t)(L.trow(b, G, n) * (size_t)L.ts);
  d.qrow = d.resid ? (int64_t)(L.tok(b, G, n) * (size_t)L.ds) : 0;
  int32_t* o = out + (size_t)b * (G + 1);
  for (int j = lane; j <= G; j += kWave) o[j] = j < n ? X[L.tok(b, G, j)] : -1;
  if (lane == 0) {
    nacc[b] = n;
    desc[b] = d;
    slots[3 * b] = 0ull;  // best race key
    count_round(stats, b, g, n);
  }
}

// ===========================================================================
// Race pass (no top-k): Exp(1) race over the full row n of each request.
// ===========================================================================
// Scores w / E with w = p - q (residual), p with the draft token masked
// (one-hot), or p (bonus).  Each thread keeps its best (score, index) in
// ascending index order (strict '>' keeps the lowest index); the workgroup
// merges (value, index) keys; the request's workgroups merge with a 64-bit
// atomic max, and race_finish_kernel writes the token.  CUT: rows may carry a
// nucleus cut (tokens with key < kp / kq have p = 0 / q = 0).  QP: q is given
// as fp32 probabilities (rows of qp).
//
// race_scan is one thread's pass over its part of the slice for one kind of
// weight, chosen per workgroup outside the streaming loop: RES 0 (p, with
// the one-hot draft token masked), 1 (max(p - q, 0), q from draft logits; QV:
// the draft row shares the target row's 16-byte alignment and is read in
// vectors), 2 (q given as fp32 probabilities); EVEN: vectors start on even
// tokens, so tokens 2m and 2m + 1 share one Philox block.
//
// Weights are kept in the row's own units, w / inv_zp (the exponentials
// exp2((l - m) c) of the target row, the draft's scaled by inv_zq / inv_zp):
// one factor for every token of the row, so the race's winner is unchanged.
struct RaceRow {
  float mp, mq, ratio, c, kvp, kvq;  // row maxima of p and q; ratio = inv_zq / inv_zp
  int kip, kiq, mask_tok;
  bool cut_p, cut_q;
};

// A residual race over two peaked rows (both normalisers below 1 + 1/16, in
// units of the rows' largest exponential; low temperature): a token at the
// maximum of both rows has weight 1 - Zp / Zq, which fp32 rounds to 0 once
// the rows' masses off their maxima are below 2^-24, and the other tokens'
// residuals can lie below fp32's range.  Such rows take race_scan_tail:
// log-domain scores, and the tokens whose two exponentials are equal (the
// same gap below each row's maximum: the tokens at both maxima, and others)
// set aside, since their residual e (1 / Zp - 1 / Zq) shares one factor that
// the finish takes in fp64 from Z = n + c + t: n the count of maximal
// tokens, c the mass of the other set-aside tokens (the same in both rows),
// t the rest of the row's mass off its maximum (per-split sums, times 2^64
// so that they do not flush).
constexpr float kTailInvZ = 1.0f / 1.0625f;
constexpr float kTailShift = 64.f;
struct TailAcc {
  float tp, tq, np, nq, tc;
  uint64_t ukey;
};
// Draft logits: also two normalisers within 2^-10 of each other, where 1 -
// Zp / Zq is as small and the rows' masses off their maxima, without the
// tokens of equal gap, can still be small.  Draft probabilities given: a
// peaked target row.
__device__ __forceinline__ bool tail_race(const RaceDesc& d) {
  if (d.resid == 1)
    return (d.inv_zp > kTailInvZ && d.inv_zq > kTailInvZ) || fabsf(d.inv_zp - d.inv_zq) < 0x1.0p-10f * d.inv_zq;
  return d.resid == 2 && d.inv_zp > kTailInvZ;
}

template <typename ET, int NT, int RES, bool QV, bool EVEN>
__device__ __forceinline__ uint64_t race_scan(const Slice<ET>& sl, const ET* rq, const float* rqp, const RaceRow& r,
                                              float inv_zp, uint32_t k0, uint32_t k1, uint32_t ub, uint32_t un) {
  constexpr int EPV = Elem<ET>::kPerVec;
  const int tid = threadIdx.x;
  float best = 0.f;  // scores are positive; best_y < 0 until a token scores
  int best_y = -1;
  // Nucleus cuts as float compares: key(l, y) >= kappa iff l > value(kappa),
  // or l equals it and y <= index(kappa); kappa = 0 keeps every token.
  auto weight = [&](float lp, float lq, int y) -> float {
    float p = __builtin_amdgcn_exp2f((lp - r.mp) * r.c);
    if (r.cut_p && !(lp > r.kvp || (lp == r.kvp && y <= r.kip))) p = 0.f;
    if (RES == 0) return p;  // the one-hot draft token is masked per vector
    float q;
    if (RES == 1) {
      q = __builtin_amdgcn_exp2f((lq - r.mq) * r.c);
      if (r.cut_q && !(lq > r.kvq || (lq == r.kvq && y <= r.kiq))) q = 0.f;
      return fmaxf(fmaf(-q, r.ratio, p), 0.f);
    }
    return fmaxf(fmaf(-lq, 1.f / inv_zp, p), 0.f);  // RES 2: q given as a probability
  };
  // A score equal to the thread's best loses (ties go to the lowest index,
  // and a thread visits its tokens in ascending order).  A token cannot win
  // the row if w <= S t, with t = 1 - u (the race variate E = -ln(1 - t) >=
  // t) and S the largest best score of any lane at the last exchange: such
  // tokens skip the logarithm.  The test uses t's lower bound ~hi 2^-32
  // (hi: the high Philox word) and folds 2^-32 and the rounding margin into
  // `bar`; a bar shared by the wave keeps whole waves on the short path.
  constexpr float kBarScale = kRaceSkip * 0x1.0p-32f;
  float bar = 0.f;
  auto consider = [&](float w, uint32_t lo, uint32_t hi, int y) {
    if (!(w <= bar * (float)(~hi))) {
      const float sc = w * __builtin_amdgcn_rcpf(exp1_from_words(lo, hi));  // E = 0 gives +inf
      if (sc > best) {
        best = sc;
        best_y = y;
        bar = fmaxf(bar, sc * kBarScale);
      }
    }
  };
  const uint4* vp = sl.vecs();
  const uint4* vq = QV ? (const uint4*)(rq + sl.a + sl.head) : nullptr;
  auto race_vec = [&](const uint4& pv, const uint4& qv, int i) {
    float fp[EPV], fq[EPV];
    Elem<ET>::unpack(pv, fp);
    const int y0 = sl.vec_index0(i);
    if (RES == 0 && (uint32_t)(r.mask_tok - y0) < (uint32_t)EPV) {
#pragma unroll
      for (int k = 0; k < EPV; ++k)
        if (k == r.mask_tok - y0) fp[k] = -INFINITY;
    }
    if (RES == 2) {
#pragma unroll
      for (int k = 0; k < EPV; ++k) fq[k] = rqp[y0 + k];
    } else if (RES == 1 && QV) {
      Elem<ET>::unpack(qv, fq);
    } else if (RES == 1) {
#pragma unroll
      for (int k = 0; k < EPV; ++k) fq[k] = Elem<ET>::load1(rq + y0 + k);
    } else {
#pragma unroll
      for (int k = 0; k < EPV; ++k) fq[k] = 0.f;
    }
    if (EVEN) {
      // The vector's EPV / 2 race blocks (counter (y >> 1, n, b, 1)) at once.
      uint4 rr[EPV / 2];
#pragma unroll
      for (int m = 0; m < EPV / 2; ++m) rr[m] = make_uint4((uint32_t)(y0 >> 1) + (uint32_t)m, un, ub, 1u);
      philox10_multi<EPV / 2>(rr, k0, k1);
#pragma unroll
      for (int m = 0; m < EPV / 2; ++m) {
        const int y = y0 + 2 * m;
        consider(weight(fp[2 * m], fq[2 * m], y), rr[m].x, rr[m].y, y);
        consider(weight(fp[2 * m + 1], fq[2 * m + 1], y + 1), rr[m].z, rr[m].w, y + 1);
      }
    } else {
#pragma unroll
      for (int k = 0; k < EPV; ++k) {
        const int y = y0 + k;
        const uint4 rr = race_block(k0, k1, ub, un, (uint32_t)y);
        if (y & 1) consider(weight(fp[k], fq[k], y), rr.z, rr.w, y);
        else consider(weight(fp[k], fq[k], y), rr.x, rr.y, y);
      }
    }
  };
  const uint4 zero4 = make_uint4(0u, 0u, 0u, 0u);
  // Two vectors per iteration (more independent Philox chains in flight);
  // the trip count is the same for every lane, so the whole wave takes part
  // in the exchange of the bar.
  for (int base = 0; base < sl.nvec; base += 2 * NT) {
    const int i0 = base + tid, i1 = i0 + NT;
    const bool h0 = i0 < sl.nvec, h1 = i1 < sl.nvec;
    const uint4 p0 = h0 ? load_stream(vp + i0) : zero4, p1 = h1 ? load_stream(vp + i1) : zero4;
    const uint4 q0 = (QV && h0) ? load_stream(vq + i0) : zero4;
    const uint4 q1 = (QV && h1) ? load_stream(vq + i1) : zero4;
    if (h0) race_vec(p0, q0, i0);
    if (h1) race_vec(p1, q1, i1);
    bar = wave_max_f(bar);
  }
  uint64_t key = best_y >= 0 ? make_key(best, (uint32_t)best_y) : 0ull;
  // Scalar head and tail: keyed directly, so index order does not matter.
  if (tid < sl.nscalar()) {
    const int y = sl.scalar_index(tid);
    const uint4 rr = race_block(k0, k1, ub, un, (uint32_t)y);
    const float lq = RES == 2 ? rqp[y] : (RES == 1 ? Elem<ET>::load1(rq + y) : 0.f);
    float w = weight(Elem<ET>::load1(sl.row + y), lq, y);
    if (RES == 0 && y == r.mask_tok) w = 0.f;
    if (w > 0.f) {
      const float E = (y & 1) ? exp1_from_words(rr.z, rr.w) : exp1_from_words(rr.x, rr.y);
      const uint64_t kk = make_key(w * __builtin_amdgcn_rcpf(E), (uint32_t)y);
      key = kk > key ? kk : key;
    }
  }
  return key;
}

// The scan of a residual race over two peaked rows (tail_race), element by
// element over [a, e) (a rare path: plain loads, one Philox block per
// token).  Scores are taken in the log domain, log2(w) - log2(E) with w in
// units of the target row's largest exponential, so that no residual mass
// the oracle's fp64 keeps (down to 2^-1074) is lost: w = 2^gp (1 - 2^(gq -
// gp) Zp / Zq), g = (l - m) c.  Tokens kept in both rows with gp == gq are
// set aside (ukey: largest gp - log2(E), lowest index) for the finish; the
// counts of maximal tokens and the masses c, tp, tq (times 2^64) are summed
// into *ta.
//
// log2 of a positive fp32 value, its denormals included (the hardware log
// takes them as 0): a denormal's bits are its value in units of 2^-149.
__device__ __forceinline__ float log2_pos(float v) {
  const uint32_t b = __float_as_uint(v);
  return b < 0x00800000u ? __builtin_amdgcn_logf((float)b) - 149.f : __builtin_amdgcn_logf(v);
}

// With the draft given as probabilities (RES 2: q(y) = qp[y]), w = 2^gp -
// q(y) Zp, taken as gp + log2(1 - 2^(log2 q(y) + log2 Zp - gp)); the target
// row's maximal tokens are left to the finish, which weighs each with
// p - q = 1 / Zp - q(y) in fp64 (Zp = np + tp).
template <typename ET, int RES>
__device__ __forceinline__ uint64_t race_scan_tail(const ET* rp, const ET* rq, const float* rqp, int a, int e,
                                                   const RaceRow& r, float inv_zp, uint32_t k0, uint32_t k1,
                                                   uint32_t ub, uint32_t un, int nt, TailAcc* ta) {
  uint64_t key = 0ull;
  if constexpr (RES == 2) {
    const float lzp = -__builtin_amdgcn_logf(inv_zp);  // log2 Zp
#pragma unroll 1
    for (int y = a + (int)threadIdx.x; y < e; y += nt) {
      const float lp = Elem<ET>::load1(rp + y);
      const bool kp = !r.cut_p || lp > r.kvp || (lp == r.kvp && y <= r.kip);
      const float gp = (lp - r.mp) * r.c;
      const bool ip = kp && lp == r.mp;  // a kept maximal token (a tie past a cut is not kept)
      ta->tp += (kp && !ip) ? __builtin_amdgcn_exp2f(gp + kTailShift) : 0.f;
      ta->np += ip ? 1.f : 0.f;
      if (!kp || ip) continue;  // p = 0, or a maximal token (the finish)
      const float qy = rqp[y];
      float lw = gp;
      if ((__float_as_uint(qy) & 0x7FFFFFFFu) != 0u) {
        const float lf = log2_pos(qy) + lzp - gp;
        if (!(lf < 0.f)) continue;  // q >= p: no residual
        lw = gp + __builtin_amdgcn_logf(1.f - __builtin_amdgcn_exp2f(lf));
      }
      if (!(lw > -1074.f)) continue;  // below fp64's range, as in the oracle
      const uint4 rr = race_block(k0, k1, ub, un, (uint32_t)y);
      const float E = (y & 1) ? exp1_from_words(rr.z, rr.w) : exp1_from_words(rr.x, rr.y);
      const uint64_t k = make_key(lw - __builtin_amdgcn_logf(E), (uint32_t)y);
      key = k > key ? k : key;
    }
    return key;
  }
#pragma unroll 1
  for (int y = a + (int)threadIdx.x; y < e; y += nt) {
    const float lp = Elem<ET>::load1(rp + y), lq = Elem<ET>::load1(rq + y);
    const bool kp = !r.cut_p || lp > r.kvp || (lp == r.kvp && y <= r.kip);
    const bool kq = !r.cut_q || lq > r.kvq || (lq == r.kvq && y <= r.kiq);
    const float gp = (lp - r.mp) * r.c, gq = (lq - r.mq) * r.c;
    const bool ip = kp && lp == r.mp, iq = kq && lq == r.mq;  // kept maximal tokens
    const bool common = kp && kq && gp == gq;  // equal exponentials (both maxima: gp = gq = 0)
    const float ep = kp ? __builtin_amdgcn_exp2f(gp + kTailShift) : 0.f;
    const float eq = kq ? __builtin_amdgcn_exp2f(gq + kTailShift) : 0.f;
    ta->np += ip ? 1.f : 0.f;
    ta->nq += iq ? 1.f : 0.f;
    if (common) {
      ta->tc += ip ? 0.f : ep;
    } else {
      ta->tp += ip ? 0.f : ep;
      ta->tq += iq ? 0.f : eq;
    }
    if (!kp) continue;  // p = 0: no residual
    const uint4 rr = race_block(k0, k1, ub, un, (uint32_t)y);
    const float E = (y & 1) ? exp1_from_words(rr.z, rr.w) : exp1_from_words(rr.x, rr.y);
    const float nle = -__builtin_amdgcn_logf(E);  // E = 0: +inf
    if (common) {
      const uint64_t k = make_key(gp + nle, (uint32_t)y);
      ta->ukey = k > ta->ukey ? k : ta->ukey;
      continue;
    }
    const float f = kq ? __builtin_amdgcn_exp2f(gq - gp) * r.ratio : 0.f;
    if (!(f < 1.f)) continue;  // q >= p: no residual
    const float lw = gp + __builtin_amdgcn_logf(1.f - f);
    if (!(lw > -1074.f)) continue;  // below fp64's range, as in the oracle
    const uint64_t k = make_key(lw + nle, (uint32_t)y);
    key = k > key ? k : key;
  }
  return key;
}

// The race over split s of the row a descriptor names: this workgroup's best
// (score, index) key, 0 if no token of the split has weight (every thread
// gets the workgroup's key).  A residual race over two peaked rows
// (tail_race) also stores the split's tails, counts and set-aside key in
// tpart[slot] and tkey[slot] (tpart null: never).
template <typename ET, int NT, bool CUT, bool QP>
__device__ __forceinline__ uint64_t race_split(const RaceDesc& d, const ET* __restrict__ lt, const ET* __restrict__ ld,
                                               const float* __restrict__ qp, int V, int s, int seg, uint32_t k0,
                                               uint32_t k1, float4* __restrict__ tpart = nullptr,
                                               unsigned long long* __restrict__ tkey = nullptr, size_t slot = 0) {
  const ET* rp = lt + d.prow;
  const ET* rq = (!QP && d.resid) ? ld + d.qrow : nullptr;
  const float* rqp = (QP && d.resid) ? qp + d.qrow : nullptr;
  const int a = s * seg;
  const int e = min(V, a + seg);
  const int tid = threadIdx.x;
  RaceRow r;
  r.c = d.c;
  r.mp = d.mp;
  r.mq = d.mq;
  r.ratio = d.inv_zq / d.inv_zp;
  r.mask_tok = d.mask_tok;
  r.cut_p = CUT && d.kp != 0ull;
  r.cut_q = CUT && d.kq != 0ull;
  r.kvp = r.cut_p ? key_value(d.kp) : 0.f;
  r.kvq = r.cut_q ? key_value(d.kq) : 0.f;
  r.kip = r.cut_p ? (int)key_index(d.kp) : 0;
  r.kiq = r.cut_q ? (int)key_index(d.kq) : 0;
  const uint32_t ub = (uint32_t)d.rb, un = (uint32_t)d.n;
  Slice<ET> sl(rp, a, e);
  // The draft row is read with 16-byte vectors only if it shares the target
  // row's alignment (rows start at different offsets when V * size is not a
  // multiple of 16); otherwise element by element.
  const bool q_vec = rq && ((((uintptr_t)(rp + a)) ^ ((uintptr_t)(rq + a))) & 15u) == 0u;
  const bool even = ((a + sl.head) & 1) == 0;
  uint64_t key;
  if (!d.resid) {
    key = even ? race_scan<ET, NT, 0, false, true>(sl, rq, rqp, r, d.inv_zp, k0, k1, ub, un)
               : race_scan<ET, NT, 0, false, false>(sl, rq, rqp, r, d.inv_zp, k0, k1, ub, un);
  } else if (tpart && tail_race(d)) {
    TailAcc ta{0.f, 0.f, 0.f, 0.f, 0.f, 0ull};
    if constexpr (QP) key = race_scan_tail<ET, 2>(rp, rq, rqp, a, e, r, d.inv_zp, k0, k1, ub, un, NT, &ta);
    else key = race_scan_tail<ET, 1>(rp, rq, rqp, a, e, r, d.inv_zp, k0, k1, ub, un, NT, &ta);
    // The split's sums in a fixed order (waves, then lanes).
    ta.tp = wave_sum_f(ta.tp);
    ta.tq = wave_sum_f(ta.tq);
    ta.np = wave_sum_f(ta.np);
    ta.nq = wave_sum_f(ta.nq);
    ta.tc = wave_sum_f(ta.tc);
    ta.ukey = wave_max_u64(ta.ukey);
    __shared__ float4 tred[NT / kWave];
    __shared__ float cred[NT / kWave];
    __shared__ uint64_t ured[NT / kWave];
    if (lane_id() == 0) {
      tred[tid / kWave] = make_float4(ta.tp, ta.tq, ta.np, ta.nq);
      cred[tid / kWave] = ta.tc;
      ured[tid / kWave] = ta.ukey;
    }
    __syncthreads();
    if (tid == 0) {
      float4 t = tred[0];
      float tc = cred[0];
      uint64_t u = ured[0];
      for (int k = 1; k < NT / kWave; ++k) {
        t.x += tred[k].x;
        t.y += tred[k].y;
        t.z += tred[k].z;
        t.w += tred[k].w;
        tc += cred[k];
        u = ured[k] > u ? ured[k] : u;
      }
      tpart[2 * slot] = t;
      tpart[2 * slot + 1] = make_float4(tc, 0.f, 0.f, 0.f);
      tkey[slot] = u;
    }
  } else if (QP) {
    key = even ? race_scan<ET, NT, 2, false, true>(sl, rq, rqp, r, d.inv_zp, k0, k1, ub, un)
               : race_scan<ET, NT, 2, false, false>(sl, rq, rqp, r, d.inv_zp, k0, k1, ub, un);
  } else if (q_vec) {
    key = even ? race_scan<ET, NT, 1, true, true>(sl, rq, rqp, r, d.inv_zp, k0, k1, ub, un)
               : race_scan<ET, NT, 1, true, false>(sl, rq, rqp, r, d.inv_zp, k0, k1, ub, un);
  } else {
    key = even ? race_scan<ET, NT, 1, false, true>(sl, rq, rqp, r, d.inv_zp, k0, k1, ub, un)
               : race_scan<ET, NT, 1, false, false>(sl, rq, rqp, r, d.inv_zp, k0, k1, ub, un);
  }
  key = wave_max_u64(key);
  __shared__ uint64_t red[NT / kWave];
  if (lane_id() == 0) red[tid / kWave] = key;
  __syncthreads();
  uint64_t bk = red[0];
  for (int k = 1; k < NT / kWave; ++k) bk = red[k] > bk ? red[k] : bk;
  return bk;
}

template <typename ET, int NT, bool CUT, bool QP>
__global__ __launch_bounds__(NT) void race_full_kernel(const ET* __restrict__ lt, const ET* __restrict__ ld,
                                                       const float* __restrict__ qp, int V, int S, int seg,
                                                       uint32_t k0, uint32_t k1, const RaceDesc* __restrict__ desc,
                                                       unsigned long long* __restrict__ slots,
                                                       float4* __restrict__ tpart = nullptr,
                                                       unsigned long long* __restrict__ tkey = nullptr) {
  const int b = blockIdx.x / S, s = blockIdx.x - b * S;
  const RaceDesc d = desc[b];
  if (d.n < 0) return;
  const uint64_t bk = race_split<ET, NT, CUT, QP>(d, lt, ld, qp, V, s, seg, k0, k1, tpart, tkey, blockIdx.x);
  // Device-scope atomic max: coherent across XCDs; read by the next launch.
  if (threadIdx.x == 0 && bk) atomicMax(&slots[3 * b], (unsigned long long)bk);
}

// Accept pass and race in one launch (single-setting calls over full rows,
// dense rows, G < 64): workgroup (b, s) first takes request b's accept
// decisions itself, then races split s of row n.  The request's row partials
// are staged in LDS with one coalesced load (dynamic LDS: (2G+1) S float2,
// G+1 rows without draft logits); wave 0 then takes the decisions (lane j =
// position j: p(x_j), q(x_j) from the logits the row pass gathered, the fp64
// test, the first rejection by one ballot).  Every workgroup of a request
// reaches the same n from the same inputs; workgroup 0 writes the outputs and
// the descriptor race_finish_kernel reads.  The row pass has cleared the race
// slots.
template <typename ET, int MODE>
__global__ __launch_bounds__(256) void accept_race_kernel(const ET* __restrict__ lt, const ET* __restrict__ ld,
                                                          const float2* __restrict__ part,
                                                          const float* __restrict__ gath,
                                                          const int32_t* __restrict__ X, int G, int V, int S,
                                                          int rows_t, float c, uint32_t k0, uint32_t k1, int Sr,
                                                          int segr, int32_t* __restrict__ out,
                                                          int32_t* __restrict__ nacc, float* __restrict__ p_draft,
                                                          float* __restrict__ q_draft, RaceDesc* __restrict__ desc,
                                                          unsigned long long* __restrict__ slots,
                                                          int* __restrict__ err, float4* __restrict__ tpart,
                                                          unsigned long long* __restrict__ tkey) {
  extern __shared__ float2 psh[];  // [rows of the request][S]
  __shared__ RaceDesc dsh;
  const int b = blockIdx.x / Sr, s = blockIdx.x - b * Sr;
  const int tid = threadIdx.x, w = tid / kWave, lane = lane_id();
  const int nt = G + 1, nrq = nt + (MODE == 0 ? G : 0);
  const float2* pt = part + (size_t)b * nt * S;                            // target rows 0..G
  const float2* pd = part + ((size_t)rows_t + (size_t)b * G) * S;          // draft rows 0..G-1
  // Wave 0's per-position inputs are loaded first, so that their latency
  // overlaps the staging of the partials (a gathered value is used only
  // where the token is valid).
  int x = -1;
  float gp = 0.f, gq = 0.f;
  if (w == 0 && lane < G) {
    x = X[(size_t)b * G + lane];
    gp = gath[(size_t)b * nt + lane];
    if (MODE == 0) gq = gath[(size_t)rows_t + (size_t)b * G + lane];
  }
  for (int e = tid; e < nrq * S; e += 256) psh[e] = e < nt * S ? pt[e] : pd[e - nt * S];
  __syncthreads();
  if (w == 0) {
    // The arithmetic of accept_full_kernel: each lane merges its rows'
    // partials in order (p(x_j), q(x_j)); the race rows n are merged by the
    // wave.  The results are bit-identical to that kernel's.
    const int j = lane;
    bool rej = false;
    float px = 0.f, qx = 0.f;
    double pdt = 0.0, qdt = 0.0;  // the same for the accept test (test_prob)
    bool valid = false;
    if (j < G) {
      valid = x >= 0 && x < V;
      if (valid) {
        float M, Z;
        merge_row_lane(psh + j * S, S, c, M, Z);
        px = __builtin_amdgcn_exp2f((gp - M) * c) / Z;
        pdt = test_prob(gp, M, c, 1.0 / (double)Z);
        qx = 1.f;
        qdt = 1.0;
        if (MODE == 0) {
          merge_row_lane(psh + (nt + j) * S, S, c, M, Z);
          qx = __builtin_amdgcn_exp2f((gq - M) * c) / Z;
          qdt = test_prob(gq, M, c, 1.0 / (double)Z);
        }
      }
      const uint4 r = accept_block(k0, k1, (uint32_t)b, (uint32_t)j);
      const double u = unit_from_words(r.x, r.y);
      const bool acc = valid && (MODE != 1 ? (qdt > 0.0 && u <= pdt / qdt) : (u <= pdt));
      rej = !acc;
    }
    const uint64_t m = ballot(rej);
    const int n = m ? (int)__builtin_ctzll(m) : G;
    RaceDesc d;
    d.n = n;
    d.mask_tok = (MODE == 1 && n < G) ? __shfl(x, n) : -1;
    d.resid = (MODE == 0 && n < G) ? 1 : 0;
    d.rb = b;
    float Z;
    merge_partials(psh + n * S, S, c, d.mp, Z);
    d.inv_zp = 1.f / Z;
    d.mq = 0.f;
    d.inv_zq = 0.f;
    if (d.resid) {
      merge_partials(psh + (nt + n) * S, S, c, d.mq, Z);
      d.inv_zq = 1.f / Z;
    }
    d.c = c;
    d.pad2[0] = d.pad2[1] = d.pad2[2] = 0;
    d.kp = d.kq = 0ull;
    d.prow = (int64_t)(((size_t)b * nt + n) * (size_t)V);
    d.qrow = d.resid ? (int64_t)(((size_t)b * G + n) * (size_t)V) : 0;
    if (lane == 0) dsh = d;
    if (s == 0) {
      if (j < G) {
        if (p_draft) p_draft[(size_t)b * G + j] = px;
        if (q_draft) q_draft[(size_t)b * G + j] = MODE == 1 ? (valid ? 1.f : 0.f) : qx;
        if (!valid) atomicOr(err, kErrBadToken);
      }
      if (j <= G) out[(size_t)b * nt + j] = j < n ? x : -1;
      if (lane == 0) {
        nacc[b] = n;
        desc[b] = d;
      }
    }
  }
  __syncthreads();
  const RaceDesc d = dsh;
  const uint64_t bk = race_split<ET, 256, false, false>(d, lt, ld, (const float*)nullptr, V, s, segr, k0, k1, tpart,
                                                        tkey, blockIdx.x);
  if (threadIdx.x == 0 && bk) atomicMax(&slots[3 * b], (unsigned long long)bk);
}

// Writes each request's race winner to out[request][n].  A residual race
// over two peaked rows first weighs the tokens its splits set aside (the
// tails and counts of splits 0..Sr-1 summed in order).  If the residual had
// no positive weight (possible only when p and q agree to rounding) the draw
// is taken from p_n instead, by the whole workgroup over the row (rare).
template <typename ET, int NT, bool CUT>
__global__ __launch_bounds__(NT) void race_finish_kernel(const ET* __restrict__ lt, int G, int V, uint32_t k0,
                                                         uint32_t k1, const RaceDesc* __restrict__ desc,
                                                         const unsigned long long* __restrict__ slots,
                                                         int32_t* __restrict__ out,
                                                         const float4* __restrict__ tpart = nullptr,
                                                         const unsigned long long* __restrict__ tkey = nullptr,
                                                         int Sr = 0, const float* __restrict__ qp = nullptr) {
  const int b = blockIdx.x, tid = threadIdx.x;
  const RaceDesc d = desc[b];
  const int n = d.n;
  if (n < 0) return;
  const float c = d.c;
  int32_t* dst = out + (size_t)b * (G + 1) + n;
  unsigned long long win = slots[3 * b];
  __shared__ uint64_t red[NT / kWave];
  if (tpart && qp && d.resid == 2 && tail_race(d)) {
    // Draft probabilities given: the target row's maximal tokens, each with
    // p - q = 1 / Zp - q(y) in fp64 (Zp = np + tp, the scan's sums), found
    // by one more pass over the row (rare rows only).
    double tp = 0.0, np = 0.0;
    for (int s = 0; s < Sr; ++s) {
      const float4 t = tpart[2 * ((size_t)b * Sr + s)];
      tp += t.x;
      np += t.z;
    }
    const double zp = np + 0x1.0p-64 * tp;
    const ET* rp = lt + d.prow;
    const float* rq = qp + d.qrow;
    uint64_t km = 0ull;
    for (int y = tid; y < V; y += NT) {
      const float l = Elem<ET>::load1(rp + y);
      if (l != d.mp || (CUT && make_key(l, (uint32_t)y) < d.kp)) continue;  // kept maximal tokens
      const double w = (1.0 / zp - (double)rq[y]) * zp;
      if (!(w > 0.0)) continue;
      const uint4 r = race_block(k0, k1, (uint32_t)d.rb, (uint32_t)n, (uint32_t)y);
      const float E = (y & 1) ? exp1_from_words(r.z, r.w) : exp1_from_words(r.x, r.y);
      const uint64_t kk = make_key((float)log2(w) - __builtin_amdgcn_logf(E), (uint32_t)y);
      km = kk > km ? kk : km;
    }
    km = wave_max_u64(km);
    if (lane_id() == 0) red[tid / kWave] = km;
    __syncthreads();
    for (int k = 0; k < NT / kWave; ++k) win = red[k] > win ? red[k] : win;
    __syncthreads();
  } else if (tpart && tail_race(d)) {
    double tp = 0.0, tq = 0.0, np = 0.0, nq = 0.0, tc = 0.0;
    uint64_t u = 0ull;
    for (int s = 0; s < Sr; ++s) {
      const size_t slot = (size_t)b * Sr + s;
      const float4 t = tpart[2 * slot];
      tp += t.x;
      tq += t.y;
      np += t.z;
      nq += t.w;
      tc += tpart[2 * slot + 1].x;
      const uint64_t k = tkey[slot];
      u = k > u ? k : u;
    }
    // The set-aside tokens' factor 1 / Zp - 1 / Zq, taken in fp64 (the
    // precision of the residual's definition) from Z = n + c + t (the sums
    // carry the scan's factor 2^64), in units of the target row's largest
    // exponential (times Zp); their best score gp - log2(E) plus its log2.
    const double zp = np + 0x1.0p-64 * (tc + tp), zq = nq + 0x1.0p-64 * (tc + tq);
    const double wt = (1.0 / zp - 1.0 / zq) * zp;
    if (u && wt > 0.0) {
      const uint64_t kk = make_key((float)log2(wt) + key_value(u), key_index(u));
      win = kk > win ? kk : win;
    }
  }
  if (win) {
    if (tid == 0) *dst = (int32_t)key_index(win);
    return;
  }
  const ET* rp = lt + d.prow;
  const uint32_t ub = (uint32_t)d.rb, un = (uint32_t)n;
  uint64_t kp = 0ull;
  for (int y = tid; y < V; y += NT) {
    const float l = Elem<ET>::load1(rp + y);
    float p = __builtin_amdgcn_exp2f((l - d.mp) * c) * d.inv_zp;
    if (CUT && make_key(l, (uint32_t)y) < d.kp) p = 0.f;
    if (p > 0.f) {
      const uint4 r = race_block(k0, k1, ub, un, (uint32_t)y);
      const float E = (y & 1) ? exp1_from_words(r.z, r.w) : exp1_from_words(r.x, r.y);
      const uint64_t kk = make_key(p * __builtin_amdgcn_rcpf(E), (uint32_t)y);
      kp = kk > kp ? kk : kp;
    }
  }
  kp = wave_max_u64(kp);
  if (lane_id() == 0) red[tid / kWave] = kp;
  __syncthreads();
  if (tid == 0) {
    uint64_t bk = red[0];
    for (int k = 1; k < NT / kWave; ++k) bk = red[k] > bk ? red[k] : bk;
    *dst = bk ? (int32_t)key_index(bk) : -1;
  }
}

// ===========================================================================
// Accept pass, greedy: one wave per request.
// ===========================================================================
__global__ __launch_bounds__(64) void accept_greedy_kernel(const uint64_t* __restrict__ part,
                                                           const int32_t* __restrict__ X, int G, int V, int S,
                                                           int32_t* __restrict__ out, int32_t* __restrict__ nacc,
                                                           int32_t* __restrict__ targ, int* __restrict__ err,
                                                           const ReqInfo* __restrict__ info,
                                                           float* __restrict__ p_draft, float* __restrict__ q_draft,
                                                           Layout L, Stats stats) {
  // Lane j handles position j (chunks of 64): the target argmax of row j
  // (max over the row's partial keys), written to out[j] for now, and the
  // match test; the first mismatch is one ballot.  In a batch call only
  // temperature-0 requests are handled; their p(x_j) is the temperature-0
  // law (1 on the argmax, else 0) and q(x_j) = 1.
  const int b = blockIdx.x;
  if (info && info[b].kind != kReqGreedy) return;
  const int g = L.len(b, G);  // this request's draft positions
  const int lane = lane_id();
  int32_t* o = out + (size_t)b * (G + 1);
  int n = g;
  int x0 = -1;  // this lane's draft token in the first chunk of positions
  for (int j0 = 0; j0 <= g; j0 += kWave) {
    const int j = j0 + lane;
    bool mis = false;
    if (j <= g) {
      // The draft token and the row's partial keys are loaded together,
      // eight partials in flight at a time.
      const size_t xj = j < g ? L.tok(b, G, j) : 0;
      const int x = j < g ? X[xj] : -1;
      if (j0 == 0) x0 = x;
      const uint64_t* pj = part + ((size_t)b * (G + 1) + j) * S;
      uint64_t m = 0ull;
      for (int k0 = 0; k0 < S; k0 += 8) {
        uint64_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = k0 + u < S ? pj[k0 + u] : 0ull;
#pragma unroll
        for (int u = 0; u < 8; ++u) m = v[u] > m ? v[u] : m;
      }
      const int a = (int)key_index(m);
      o[j] = a;
      if (targ) targ[(size_t)b * (G + 1) + j] = a;
      if (j < g) {
        const bool valid = x >= 0 && x < V;
        if (!valid) atomicOr(err, kErrBadToken);
        mis = !valid || x != a;
        if (p_draft) p_draft[xj] = mis ? 0.f : 1.f;
        if (q_draft) q_draft[xj] = 1.f;
        if (stats.beta) stats.beta[xj] = mis ? 0.f : 1.f;
      }
    }
    const uint64_t mm = ballot(mis);
    if (n == g && mm) n = j0 + (int)__builtin_ctzll(mm);
  }
  // Accepted drafts before n, the target argmax (already in place) at n,
  // padding after: each lane rewrites only positions of its own lane.
  for (int j = lane; j <= G; j += kWave) {
    if (j < n) o[j] = j < kWave ? x0 : X[L.tok(b, G, j)];
    else if (j > n) o[j] = -1;
  }
  if (lane == 0) {
    nacc[b] = n;
    count_round(stats, b, g, n);
  }
}

// Measurement only: the streaming-read ceiling the row passes are compared
// with.  One workgroup per chunk of `chunk` 16-byte vectors, read with the
// row passes' nontemporal loads, U in flight per thread; nothing is written
// unless the xor of a workgroup's words hits one fixed value (which keeps
// the loads alive and is otherwise never true in practice).
template <int U>
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ p, int64_t nvec, int64_t chunk,
                                                          uint32_t* __restrict__ sink) {
  const int64_t c0 = (int64_t)blockIdx.x * chunk;
  const int64_t c1 = c0 + chunk < nvec ? c0 + chunk : nvec;
  uint32_t acc = 0u;
  for (int64_t i0 = c0 + threadIdx.x; i0 < c1; i0 += 256 * U) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = i0 + (int64_t)u * 256;
      v[u] = i < c1 ? load_stream(p + i) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x & 255] = acc;
}

// Copies the error word of a call into a caller's device word.
__global__ __launch_bounds__(64) void copy_word_kernel(const int32_t* __restrict__ src, int32_t* __restrict__ dst) {
  if (threadIdx.x == 0) *dst = *src;
}

}  // namespace sv
