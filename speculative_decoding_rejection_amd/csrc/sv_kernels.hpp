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

namespace sv {

// Error word bits.
constexpr int kErrBadToken = 1;

// Per-request race descriptor written by the accept pass (no top-k).
struct __align__(16) RaceDesc {
  int32_t n;         // race position (first rejection or G)
  int32_t mask_tok;  // one-hot: token removed from the residual, else -1
  int32_t resid;     // 1: weights max(p - q, 0); 0: weights p
  int32_t pad;
  float mp, inv_zp, mq, inv_zq;  // softmax stats of target row n / draft row n
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
template <typename ET, int NT, int U>
__global__ __launch_bounds__(NT) void rows_softmax_kernel(const ET* __restrict__ lt, const ET* __restrict__ ld,
                                                          int rows_t, int V, int S, int seg, float c,
                                                          float2* __restrict__ part, int* __restrict__ err) {
  constexpr int EPV = Elem<ET>::kPerVec;
  const int blk = blockIdx.x;
  const int row = blk / S, s = blk - row * S;
  if (blk == 0 && threadIdx.x == 0) *err = 0;
  const ET* rp = row < rows_t ? lt + (size_t)row * V : ld + (size_t)(row - rows_t) * V;
  const int a = s * seg;
  const int e = min(V, a + seg);
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
      v[u] = i < sl.nvec ? vp[i] : ninf;
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
        const float mc = m * c;
#pragma unroll
        for (int k = 0; k < EPV; ++k) sum += __builtin_amdgcn_exp2f(fmaf(f[k], c, -mc));
      }
    }
  }
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
                                                         uint64_t* __restrict__ part, int* __restrict__ err) {
  constexpr int EPV = Elem<ET>::kPerVec;
  const int blk = blockIdx.x;
  const int row = blk / S, s = blk - row * S;
  if (blk == 0 && threadIdx.x == 0) *err = 0;
  const ET* rp = lt + (size_t)row * V;
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
      v[u] = i < sl.nvec ? vp[i] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * NT;
      if (i < sl.nvec) {
        float f[EPV];
        Elem<ET>::unpack(v[u], f);
        // Strict '>' in ascending index order keeps the first maximum.
#pragma unroll
        for (int k = 0; k < EPV; ++k) {
          if (f[k] > bv || bi < 0) {
            bv = f[k];
            bi = sl.vec_index0(i) + k;
          }
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
// One workgroup (4 waves) per row; the waves stream interleaved 16-byte
// vectors.  Each wave keeps the keys that beat a running threshold tau in its
// own LDS buffer.  When the buffer would overflow, an exact radix select over
// the buffer finds its K-th largest key, the buffer keeps exactly those K, and
// tau rises to it.  tau is shared through LDS: every published value is the
// K-th largest of K keys some wave retains, hence a lower bound of the row's
// K-th largest key, so any wave may skip elements at or below it.  At the end
// the surviving keys of the four waves are merged and selected once more.
// ===========================================================================

// K-th largest of the n (> K) distinct keys in buf, by radix select over the
// bytes of the key (from the top; bytes shared by every key are skipped).
// Returns a threshold t such that exactly K keys are >= t: the K-th largest
// key itself, or (when the last examined digit bucket is taken whole) that
// bucket's prefix with zero low bits.
__device__ uint64_t wave_select_kth(const uint64_t* buf, int n, int K, uint32_t* hist) {
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
      if ((k & pmask) == prefix) atomicAdd(&hist[(uint32_t)(k >> shift) & 255u], 1u);
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
__device__ int wave_keep_ge(uint64_t* buf, int n, uint64_t thr) {
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

template <int CAPW>
struct TopkWave {
  uint64_t* buf;
  uint32_t* hist;
  uint64_t* tau_shared;
  uint64_t tau;   // insert keys > tau
  float tau_v;    // value part of tau (-inf when tau is at or below -inf keys)
  int cnt;
  int K;

  __device__ __forceinline__ void set_tau(uint64_t t) {
    tau = t;
    const uint32_t o = (uint32_t)(t >> 32);
    tau_v = (o <= 0x007FFFFFu) ? -INFINITY : key_value(t);
  }
  __device__ __forceinline__ void refresh() {
    const uint64_t ts = __hip_atomic_load(tau_shared, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (ts > tau) set_tau(ts);
  }
  // Reduces the buffer to its K largest keys (and drops keys below tau).
  __device__ void compact() {
    wave_lds_sync();
    if (cnt > K) {
      const uint64_t thr = wave_select_kth(buf, cnt, K, hist);
      if (thr > tau) {
        set_tau(thr);
        if (lane_id() == 0) atomicMax((unsigned long long*)tau_shared, (unsigned long long)thr);
      }
    }
    cnt = wave_keep_ge(buf, cnt, tau);
  }
  // Offers up to EPV elements per lane (slot k valid if bit k of vmask).
  template <int EPV>
  __device__ __forceinline__ void offer(const float* f, uint32_t idx0, uint32_t vmask) {
    float vm = -INFINITY;
#pragma unroll
    for (int k = 0; k < EPV; ++k)
      if (vmask & (1u << k)) vm = fmaxf(vm, f[k]);
    const bool maybe = vmask != 0u && vm >= tau_v;
    if (ballot(maybe) == 0ull) return;
#pragma unroll
    for (int k = 0; k < EPV; ++k) {
      const uint64_t key = (vmask & (1u << k)) ? make_key(f[k], idx0 + (uint32_t)k) : 0ull;
      bool hit = key > tau;
      uint64_t m = ballot(hit);
      if (m == 0ull) continue;
      int nh = __builtin_popcountll(m);
      if (cnt + nh > CAPW) {
        compact();
        hit = key > tau;
        m = ballot(hit);
        nh = __builtin_popcountll(m);
      }
      if (hit) buf[cnt + lanes_below(m)] = key;
      cnt += nh;
    }
  }
};

template <typename ET, int CAPW, int U>
__global__ __launch_bounds__(256) void rows_topk_kernel(const ET* __restrict__ lt, const ET* __restrict__ ld,
                                                        int rows_t, int V, int K, uint64_t* __restrict__ cand,
                                                        int* __restrict__ err) {
  constexpr int NT = 256, NW = NT / kWave;
  constexpr int EPV = Elem<ET>::kPerVec;
  __shared__ uint64_t buf[NW][CAPW];
  __shared__ uint32_t hist[NW][256];
  __shared__ uint64_t tau_shared;
  __shared__ int counts[NW];
  const int row = blockIdx.x;
  const int tid = threadIdx.x, w = tid / kWave;
  if (row == 0 && tid == 0) *err = 0;
  if (tid == 0) tau_shared = 0ull;
  __syncthreads();
  const ET* rp = row < rows_t ? lt + (size_t)row * V : ld + (size_t)(row - rows_t) * V;
  Slice<ET> sl(rp, 0, V);
  TopkWave<CAPW> st{buf[w], hist[w], &tau_shared, 0ull, -INFINITY, 0, K};

  // Scalar head and tail (fewer than 2 * EPV elements): one slot per thread.
  {
    float f[EPV];
    uint32_t idx = 0, vm = 0u;
#pragma unroll
    for (int k = 0; k < EPV; ++k) f[k] = -INFINITY;
    if (tid < sl.nscalar()) {
      idx = (uint32_t)sl.scalar_index(tid);
      f[0] = Elem<ET>::load1(rp + idx);
      vm = 1u;
    }
    st.template offer<EPV>(f, idx, vm);
  }
  const uint4* vp = sl.vecs();
  const uint32_t full = (1u << EPV) - 1u;
  for (int i0 = 0; i0 < sl.nvec; i0 += NT * U) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * NT + tid;
      v[u] = i < sl.nvec ? vp[i] : make_uint4(0u, 0u, 0u, 0u);
    }
    st.refresh();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * NT + tid;
      float f[EPV];
      Elem<ET>::unpack(v[u], f);
      st.template offer<EPV>(f, (uint32_t)sl.vec_index0(i), i < sl.nvec ? full : 0u);
    }
  }
  // Each wave reduces to at most K keys, then wave 0 merges the four.
  st.refresh();
  st.compact();
  if (lane_id() == 0) counts[w] = st.cnt;
  __syncthreads();
  if (w > 0) {
    int off = 0;
    for (int k = 0; k < w; ++k) off += counts[k];
    for (int i = lane_id(); i < st.cnt; i += kWave) buf[0][off + i] = st.buf[i];
  }
  __syncthreads();
  if (w == 0) {
    int n = 0;
    for (int k = 0; k < NW; ++k) n += counts[k];
    st.cnt = n;
    st.tau = 0ull;  // select among all merged keys
    if (n > K) {
      const uint64_t thr = wave_select_kth(st.buf, n, K, st.hist);
      n = wave_keep_ge(st.buf, n, thr);
    }
    uint64_t* dst = cand + (size_t)row * K;
    for (int i = lane_id(); i < K; i += kWave) dst[i] = i < n ? st.buf[i] : 0ull;
  }
}

// ===========================================================================
// Accept pass, top-k rows: one wave per request.
// ===========================================================================
struct CandStats {
  float m;      // max kept logit
  float inv_z;  // 1 / sum exp2((l - m) c) over the kept tokens
};

__device__ __forceinline__ CandStats cand_stats(const uint64_t* ck, int K, float c) {
  const int lane = lane_id();
  float m = -INFINITY;
  for (int i = lane; i < K; i += kWave) {
    const uint64_t k = ck[i];
    if (k) m = fmaxf(m, key_value(k));
  }
  m = wave_max_f(m);
  float z = 0.f;
  for (int i = lane; i < K; i += kWave) {
    const uint64_t k = ck[i];
    if (k) z += __builtin_amdgcn_exp2f((key_value(k) - m) * c);
  }
  z = wave_sum_f(z);
  return CandStats{m, 1.f / z};
}

// Probability of token x under a kept set (0 if x is not kept).
__device__ __forceinline__ float cand_prob(const uint64_t* ck, int K, CandStats st, float c, int x) {
  const int lane = lane_id();
  float p = 0.f;
  for (int i = lane; i < K; i += kWave) {
    const uint64_t k = ck[i];
    if (k && (int)key_index(k) == x) p = __builtin_amdgcn_exp2f((key_value(k) - st.m) * c) * st.inv_z;
  }
  return wave_sum_f(p);
}

// MODE 0: prob (q from draft candidates), 1: onehot.
template <int MODE>
__global__ __launch_bounds__(64) void accept_topk_kernel(const uint64_t* __restrict__ cand,
                                                         const int32_t* __restrict__ X, int G, int V, int K,
                                                         int rows_t, float c, uint32_t k0, uint32_t k1,
                                                         int32_t* __restrict__ out, int32_t* __restrict__ nacc,
                                                         float* __restrict__ p_draft, float* __restrict__ q_draft,
                                                         int* __restrict__ err) {
  const int b = blockIdx.x;
  const int lane = lane_id();
  const uint64_t* ct = cand + (size_t)b * (G + 1) * K;
  const uint64_t* cd = cand + ((size_t)rows_t + (size_t)b * G) * K;
  int n = G;
  for (int j = 0; j < G; ++j) {
    const int x = X[(size_t)b * G + j];
    const bool valid = x >= 0 && x < V;
    const CandStats sp = cand_stats(ct + (size_t)j * K, K, c);
    const float px = valid ? cand_prob(ct + (size_t)j * K, K, sp, c, x) : 0.f;
    float qx = valid ? 1.f : 0.f;
    if (MODE == 0) {
      const CandStats sq = cand_stats(cd + (size_t)j * K, K, c);
      qx = valid ? cand_prob(cd + (size_t)j * K, K, sq, c, x) : 0.f;
      if (q_draft && lane == 0) q_draft[(size_t)b * G + j] = qx;
    }
    if (p_draft && lane == 0) p_draft[(size_t)b * G + j] = px;
    if (!valid && lane == 0) atomicOr(err, kErrBadToken);
    if (n == G) {
      const uint4 r = accept_block(k0, k1, (uint32_t)b, (uint32_t)j);
      const double u = unit_from_words(r.x, r.y);
      const bool acc = valid && (MODE == 0 ? (qx > 0.f && u <= (double)px / (double)qx) : (u <= (double)px));
      if (!acc) n = j;
    }
  }
  // Recovered (n < G) or bonus (n == G) token by the Exp(1) race over the
  // kept tokens of target row n.
  const uint64_t* cp = ct + (size_t)n * K;
  const CandStats sp = cand_stats(cp, K, c);
  CandStats sq{0.f, 0.f};
  const uint64_t* cq = cd + (size_t)n * K;
  if (MODE == 0 && n < G) sq = cand_stats(cq, K, c);
  const int xn = n < G ? X[(size_t)b * G + n] : -1;
  uint64_t best_w = 0ull, best_p = 0ull;
  for (int i = lane; i < K; i += kWave) {
    const uint64_t k = cp[i];
    if (!k) continue;
    const uint32_t y = key_index(k);
    const float p = __builtin_amdgcn_exp2f((key_value(k) - sp.m) * c) * sp.inv_z;
    float w = p;
    if (n < G) {
      if (MODE == 0) {
        float q = 0.f;
        for (int t = 0; t < K; ++t) {
          const uint64_t kq = cq[t];
          if (kq && key_index(kq) == y) q = __builtin_amdgcn_exp2f((key_value(kq) - sq.m) * c) * sq.inv_z;
        }
        w = fmaxf(p - q, 0.f);
      } else if ((int)y == xn) {
        w = 0.f;
      }
    }
    const uint4 r = race_block(k0, k1, (uint32_t)b, (uint32_t)n, y);
    const float E = (y & 1u) ? exp1_from_words(r.z, r.w) : exp1_from_words(r.x, r.y);
    if (w > 0.f) {
      const uint64_t kk = make_key(E > 0.f ? w / E : INFINITY, y);
      best_w = kk > best_w ? kk : best_w;
    }
    if (p > 0.f) {
      const uint64_t kk = make_key(E > 0.f ? p / E : INFINITY, y);
      best_p = kk > best_p ? kk : best_p;
    }
  }
  best_w = wave_max_u64(best_w);
  best_p = wave_max_u64(best_p);
  const uint64_t win = best_w ? best_w : best_p;  // zero residual mass: race on p
  int32_t* o = out + (size_t)b * (G + 1);
  for (int j = lane; j <= G; j += kWave) {
    int32_t t = -1;
    if (j < n) t = X[(size_t)b * G + j];
    else if (j == n) t = win ? (int32_t)key_index(win) : -1;
    o[j] = t;
  }
  if (lane == 0) nacc[b] = n;
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

template <typename ET, int MODE>
__global__ __launch_bounds__(64) void accept_full_kernel(const ET* __restrict__ lt, const ET* __restrict__ ld,
                                                         const float2* __restrict__ part,
                                                         const int32_t* __restrict__ X, int G, int V, int S,
                                                         int rows_t, float c, uint32_t k0, uint32_t k1,
                                                         int32_t* __restrict__ out, int32_t* __restrict__ nacc,
                                                         float* __restrict__ p_draft, float* __restrict__ q_draft,
                                                         RaceDesc* __restrict__ desc,
                                                         unsigned long long* __restrict__ slots,
                                                         int* __restrict__ err) {
  const int b = blockIdx.x;
  const int lane = lane_id();
  int n = G;
  for (int j = 0; j < G; ++j) {
    const int x = X[(size_t)b * G + j];
    const bool valid = x >= 0 && x < V;
    const size_t rt = (size_t)b * (G + 1) + j;
    float M, Z;
    merge_partials(part + rt * S, S, c, M, Z);
    float px = 0.f;
    if (valid) px = __builtin_amdgcn_exp2f((Elem<ET>::load1(lt + rt * V + x) - M) * c) / Z;
    float qx = valid ? 1.f : 0.f;
    if (MODE == 0) {
      const size_t rd = (size_t)b * G + j;
      float Mq, Zq;
      merge_partials(part + ((size_t)rows_t + rd) * S, S, c, Mq, Zq);
      qx = valid ? __builtin_amdgcn_exp2f((Elem<ET>::load1(ld + rd * V + x) - Mq) * c) / Zq : 0.f;
      if (q_draft && lane == 0) q_draft[rd] = qx;
    }
    if (p_draft && lane == 0) p_draft[(size_t)b * G + j] = px;
    if (!valid && lane == 0) atomicOr(err, kErrBadToken);
    if (n == G) {
      const uint4 r = accept_block(k0, k1, (uint32_t)b, (uint32_t)j);
      const double u = unit_from_words(r.x, r.y);
      const bool acc = valid && (MODE == 0 ? (qx > 0.f && u <= (double)px / (double)qx) : (u <= (double)px));
      if (!acc) n = j;
    }
  }
  float Mp, Zp;
  merge_partials(part + ((size_t)b * (G + 1) + n) * S, S, c, Mp, Zp);
  RaceDesc d;
  d.n = n;
  d.mask_tok = (MODE == 1 && n < G) ? X[(size_t)b * G + n] : -1;
  d.resid = (MODE == 0 && n < G) ? 1 : 0;
  d.pad = 0;
  d.mp = Mp;
  d.inv_zp = 1.f / Zp;
  d.mq = 0.f;
  d.inv_zq = 0.f;
  if (d.resid) {
    float Mq, Zq;
    merge_partials(part + ((size_t)rows_t + (size_t)b * G + n) * S, S, c, Mq, Zq);
    d.mq = Mq;
    d.inv_zq = 1.f / Zq;
  }
  int32_t* o = out + (size_t)b * (G + 1);
  for (int j = lane; j <= G; j += kWave) o[j] = j < n ? X[(size_t)b * G + j] : -1;
  if (lane == 0) {
    nacc[b] = n;
    desc[b] = d;
    slots[3 * b + 0] = 0ull;  // best residual key
    slots[3 * b + 1] = 0ull;  // best p key (zero-mass fallback)
    slots[3 * b + 2] = 0ull;  // finished workgroups
  }
}

// ===========================================================================
// Race pass (no top-k): Exp(1) race over the full row n of each request.
// ===========================================================================
template <typename ET, int NT>
__global__ __launch_bounds__(NT) void race_full_kernel(const ET* __restrict__ lt, const ET* __restrict__ ld, int G,
                                                       int V, int S, int seg, float c, uint32_t k0, uint32_t k1,
                                                       const RaceDesc* __restrict__ desc,
                                                       unsigned long long* __restrict__ slots,
                                                       int32_t* __restrict__ out) {
  constexpr int EPV = Elem<ET>::kPerVec;
  const int b = blockIdx.x / S, s = blockIdx.x - b * S;
  const RaceDesc d = desc[b];
  const int n = d.n;
  const ET* rp = lt + ((size_t)b * (G + 1) + n) * V;
  const ET* rq = d.resid ? ld + ((size_t)b * G + n) * V : nullptr;
  const int a = s * seg;
  const int e = min(V, a + seg);
  uint64_t best_w = 0ull, best_p = 0ull;
  auto score = [&](float lp, float lq, uint32_t y, uint4& blk, uint32_t& blk_id) {
    const uint32_t pair = y >> 1;
    if (pair != blk_id) {
      blk = race_block(k0, k1, (uint32_t)b, (uint32_t)n, y);
      blk_id = pair;
    }
    const float E = (y & 1u) ? exp1_from_words(blk.z, blk.w) : exp1_from_words(blk.x, blk.y);
    const float p = __builtin_amdgcn_exp2f((lp - d.mp) * c) * d.inv_zp;
    float w;
    if (d.resid) {
      const float q = __builtin_amdgcn_exp2f((lq - d.mq) * c) * d.inv_zq;
      w = fmaxf(p - q, 0.f);
      if (p > 0.f) {
        const uint64_t kk = make_key(E > 0.f ? p / E : INFINITY, y);
        best_p = kk > best_p ? kk : best_p;
      }
    } else {
      w = ((int)y == d.mask_tok) ? 0.f : p;
    }
    if (w > 0.f) {
      const uint64_t kk = make_key(E > 0.f ? w / E : INFINITY, y);
      best_w = kk > best_w ? kk : best_w;
    }
  };
  Slice<ET> sl(rp, a, e);
  // The draft row is read with 16-byte vectors only if it shares the target
  // row's alignment (rows start at different offsets when V * size is not a
  // multiple of 16); otherwise element by element.
  const bool q_vec = rq && ((((uintptr_t)(rp + a)) ^ ((uintptr_t)(rq + a))) & 15u) == 0u;
  const int tid = threadIdx.x;
  uint4 blk = make_uint4(0, 0, 0, 0);
  uint32_t blk_id = 0xFFFFFFFFu;
  if (tid < sl.nscalar()) {
    const int y = sl.scalar_index(tid);
    score(Elem<ET>::load1(rp + y), rq ? Elem<ET>::load1(rq + y) : 0.f, (uint32_t)y, blk, blk_id);
  }
  const uint4* vp = sl.vecs();
  const uint4* vq = q_vec ? (const uint4*)(rq + a + sl.head) : nullptr;
  for (int i = tid; i < sl.nvec; i += NT) {
    float fp[EPV], fq[EPV];
    Elem<ET>::unpack(vp[i], fp);
    const int y0 = sl.vec_index0(i);
    if (q_vec) {
      Elem<ET>::unpack(vq[i], fq);
    } else {
#pragma unroll
      for (int k = 0; k < EPV; ++k) fq[k] = rq ? Elem<ET>::load1(rq + y0 + k) : 0.f;
    }
#pragma unroll
    for (int k = 0; k < EPV; ++k) score(fp[k], fq[k], (uint32_t)(y0 + k), blk, blk_id);
  }
  best_w = wave_max_u64(best_w);
  best_p = wave_max_u64(best_p);
  __shared__ uint64_t red[2][NT / kWave];
  const int w = tid / kWave;
  if (lane_id() == 0) {
    red[0][w] = best_w;
    red[1][w] = best_p;
  }
  __syncthreads();
  if (tid == 0) {
    uint64_t bw = red[0][0], bp = red[1][0];
    for (int k = 1; k < NT / kWave; ++k) {
      bw = red[0][k] > bw ? red[0][k] : bw;
      bp = red[1][k] > bp ? red[1][k] : bp;
    }
    unsigned long long* sl3 = slots + 3 * b;
    if (bw) atomicMax(&sl3[0], (unsigned long long)bw);
    if (bp) atomicMax(&sl3[1], (unsigned long long)bp);
    __threadfence();
    const unsigned long long done = atomicAdd(&sl3[2], 1ull);
    if (done == (unsigned long long)(S - 1)) {
      // Last workgroup of this request: every other one has published.
      __threadfence();
      const unsigned long long fw = atomicAdd(&sl3[0], 0ull);
      const unsigned long long fp2 = atomicAdd(&sl3[1], 0ull);
      const unsigned long long win = fw ? fw : fp2;
      out[(size_t)b * (G + 1) + n] = win ? (int32_t)key_index(win) : -1;
    }
  }
}

// ===========================================================================
// Accept pass, greedy: one wave per request.
// ===========================================================================
__global__ __launch_bounds__(64) void accept_greedy_kernel(const uint64_t* __restrict__ part,
                                                           const int32_t* __restrict__ X, int G, int V, int S,
                                                           int32_t* __restrict__ out, int32_t* __restrict__ nacc,
                                                           int32_t* __restrict__ targ, int* __restrict__ err) {
  const int b = blockIdx.x;
  const int lane = lane_id();
  int n = G;
  int32_t* o = out + (size_t)b * (G + 1);
  for (int j = 0; j <= G; ++j) {
    const uint64_t* pj = part + ((size_t)b * (G + 1) + j) * S;
    uint64_t m = 0ull;
    for (int k = lane; k < S; k += kWave) m = pj[k] > m ? pj[k] : m;
    m = wave_max_u64(m);
    const int a = (int)key_index(m);
    if (targ && lane == 0) targ[(size_t)b * (G + 1) + j] = a;
    if (n == G) {
      if (j < G) {
        const int x = X[(size_t)b * G + j];
        const bool valid = x >= 0 && x < V;
        if (!valid && lane == 0) atomicOr(err, kErrBadToken);
        if (!valid || x != a) {
          n = j;
          if (lane == 0) o[j] = a;
        } else if (lane == 0) {
          o[j] = x;
        }
      } else if (lane == 0) {
        o[G] = a;  // bonus
      }
    } else {
      if (j < G) {
        const int x = X[(size_t)b * G + j];
        if (!(x >= 0 && x < V) && lane == 0) atomicOr(err, kErrBadToken);
      }
      if (lane == 0) o[j] = -1;
    }
  }
  if (lane == 0) nacc[b] = n;
}

}  // namespace sv
