// Device-side building blocks of libspecverify (gfx950, wave64).
//
// Counter-based uniforms, the (value, index) order keys used by top-k and
// argmax, logit unpacking, and wave-level reductions.  Everything here is
// independent of the CPU oracle: the Philox below is written from the
// definition in Salmon et al., "Parallel Random Numbers: As Easy as 1, 2, 3"
// (SC'11).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Philox4x32-10.  Round: (c0,c1,c2,c3) -> (hi(B*c2)^c1^k0, lo(B*c2),
// hi(A*c0)^c3^k1, lo(A*c0)) with A = 0xD2511F53, B = 0xCD9E8D57; the key
// advances by the golden-ratio and sqrt(3)-1 Weyl increments between rounds.
// ---------------------------------------------------------------------------
// a ^ b ^ k in one VALU instruction (gfx950's three-input bit operation,
// truth table 0x96); k is wave-uniform (the key schedule).  The builtin, not
// inline assembly, so the scheduler can interleave independent Philox blocks.
__device__ __forceinline__ uint32_t xor3_sk(uint32_t a, uint32_t b, uint32_t k) {
  return __builtin_amdgcn_bitop3_b32(a, b, k, 0x96);
}

// Requires a wave-uniform key (k0, k1).
__device__ __forceinline__ uint4 philox10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    // 32 x 32 -> 64-bit products: one v_mad_u64_u32 each on gfx950 (about
    // 1.4x the throughput of separate low and high multiplies).
    const uint64_t pa = (uint64_t)c.x * 0xD2511F53ull;
    const uint64_t pb = (uint64_t)c.z * 0xCD9E8D57ull;
    c = make_uint4(xor3_sk((uint32_t)(pb >> 32), c.y, k0), (uint32_t)pb, xor3_sk((uint32_t)(pa >> 32), c.w, k1),
                   (uint32_t)pa);
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

// N independent blocks advanced round by round together, so that N
// multiply-xor chains are in flight at once (bit-identical to philox10).
template <int N>
__device__ __forceinline__ void philox10_multi(uint4 (&c)[N], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const uint64_t pa = (uint64_t)c[i].x * 0xD2511F53ull;
      const uint64_t pb = (uint64_t)c[i].z * 0xCD9E8D57ull;
      c[i] = make_uint4(xor3_sk((uint32_t)(pb >> 32), c[i].y, k0), (uint32_t)pb,
                        xor3_sk((uint32_t)(pa >> 32), c[i].w, k1), (uint32_t)pa);
    }
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
}

// Stream layout: the accept uniform of (b, j) is counter (0, j, b, 0), words
// 0/1; the race uniform of token y at position j is counter (y>>1, j, b, 1),
// words 0/1 for even y, 2/3 for odd y.
__device__ __forceinline__ uint4 accept_block(uint32_t k0, uint32_t k1, uint32_t b, uint32_t j) {
  return philox10(make_uint4(0u, j, b, 0u), k0, k1);
}
__device__ __forceinline__ uint4 race_block(uint32_t k0, uint32_t k1, uint32_t b, uint32_t j, uint32_t y) {
  return philox10(make_uint4(y >> 1, j, b, 1u), k0, k1);
}

// (lo, hi) -> u = (top 53 bits + 1) * 2^-53 in (0, 1], exact in fp64.
__device__ __forceinline__ double unit_from_words(uint32_t lo, uint32_t hi) {
  const uint64_t k53 = ((((uint64_t)hi) << 32) | lo) >> 11;
  return (double)(k53 + 1ull) * 0x1.0p-53;
}

// E = -ln(u) for the same u, to about 7e-7 relative error in fp32.  The
// gap t = 1 - u = (2^53 - 1 - k53) * 2^-53 is exact in integers (the
// complement of the 53 bits); for t < 1/16, -ln(1 - t) = t + t^2/2 + ...
// truncated after t^5/5 (next term below 2e-7 relative), so precision holds
// as u -> 1 where u itself, rounded to fp32, would collapse to 1; otherwise
// -ln(u) = -ln(2) log2(u) with the hardware log2 on u rounded to fp32
// (|log2 u| >= 0.093 there).  E = 0 only for u == 1.
__device__ __forceinline__ float exp1_from_words(uint32_t lo, uint32_t hi) {
  const float t = fmaf((float)(~lo >> 11), 0x1.0p-53f, (float)(~hi) * 0x1.0p-32f);
  const float u = fmaf((float)((lo >> 11) + 1u), 0x1.0p-53f, (float)hi * 0x1.0p-32f);
  const float ser = t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, 0.2f, 0.25f), 0.33333334f), 0.5f), 1.0f);
  const float lg = -0.6931471805599453f * __builtin_amdgcn_logf(u);
  return t < 0.0625f ? ser : lg;
}

// The exact gap t = 1 - u of the same u, rounded to fp32.  -ln(1 - t) >= t,
// so a race score w / E never exceeds w / t: a token with w <= s t cannot
// beat a score s, and its logarithm need not be taken.
__device__ __forceinline__ float unit_gap_from_words(uint32_t lo, uint32_t hi) {
  return fmaf((float)(~lo >> 11), 0x1.0p-53f, (float)(~hi) * 0x1.0p-32f);
}
// Factor that keeps the skip test exact under fp32 rounding: E is computed
// within 1e-6 relative of -ln(u) and t within 2^-24 of the gap, so a token
// with w <= s t (1 - 2^-16) scores below s as computed.
constexpr float kRaceSkip = 1.0f - 0x1.0p-16f;

// ---------------------------------------------------------------------------
// Order keys.  key(v, i) = ord32(v) << 32 | ~i: larger key <=> larger value,
// then smaller index.  ord32 maps IEEE bits to an unsigned order with -0
// folded onto +0 (they compare equal as values).  Key 0 is below every real
// key (it would be a NaN pattern) and marks "no element".
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t ord32(float v) {
  uint32_t b = __float_as_uint(v);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ uint64_t make_key(float v, uint32_t idx) {
  return (((uint64_t)ord32(v)) << 32) | (uint64_t)(~idx);
}
__device__ __forceinline__ float key_value(uint64_t key) {
  const uint32_t o = (uint32_t)(key >> 32);
  const uint32_t b = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __uint_as_float(b);
}
__device__ __forceinline__ uint32_t key_index(uint64_t key) { return ~(uint32_t)key; }

// ---------------------------------------------------------------------------
// Streaming 16-byte load: logits are read once per call, so the load is
// marked nontemporal (it does not displace reusable lines in the caches);
// measured on MI355X this lifts a plain streaming read from about 79% to
// about 89% of the HBM peak.
// ---------------------------------------------------------------------------
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const u32x4_t t = __builtin_nontemporal_load((const u32x4_t*)p);
  return make_uint4(t.x, t.y, t.z, t.w);
}

// ---------------------------------------------------------------------------
// Logit unpacking from 16-byte vectors.
// ---------------------------------------------------------------------------
template <typename ET> struct Elem;
template <> struct Elem<float> {
  static constexpr int kPerVec = 4;
  static constexpr uint32_t kNegInfWord = 0xFF800000u;
  __device__ static __forceinline__ void unpack(const uint4& v, float* out) {
    out[0] = __uint_as_float(v.x);
    out[1] = __uint_as_float(v.y);
    out[2] = __uint_as_float(v.z);
    out[3] = __uint_as_float(v.w);
  }
  __device__ static __forceinline__ float load1(const float* p) { return *p; }
};
// bfloat16 held as raw 16-bit patterns: the value is the upper half of a
// binary32, so widening is a shift.
template <> struct Elem<uint16_t> {
  static constexpr int kPerVec = 8;
  static constexpr uint32_t kNegInfWord = 0xFF80FF80u;
  __device__ static __forceinline__ void unpack(const uint4& v, float* out) {
    out[0] = __uint_as_float(v.x << 16);
    out[1] = __uint_as_float(v.x & 0xFFFF0000u);
    out[2] = __uint_as_float(v.y << 16);
    out[3] = __uint_as_float(v.y & 0xFFFF0000u);
    out[4] = __uint_as_float(v.z << 16);
    out[5] = __uint_as_float(v.z & 0xFFFF0000u);
    out[6] = __uint_as_float(v.w << 16);
    out[7] = __uint_as_float(v.w & 0xFFFF0000u);
  }
  __device__ static __forceinline__ float load1(const uint16_t* p) {
    return __uint_as_float(((uint32_t)*p) << 16);
  }
};

// ---------------------------------------------------------------------------
// Wave helpers.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() {
  return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}
__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }
// Number of set bits of `mask` below this lane.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}
// Orders this wave's LDS accesses: everything before completes before
// anything after is issued (LDS is processed in order per wave).
// LDS-qualified element types.  Helpers that take pointers to these compile
// their accesses to ds_* instructions even when they are not inlined; through
// a generic pointer they would be FLAT accesses, which also count as vector
// memory operations, so every wait on them would wait for the row's pending
// loads as well.
typedef __attribute__((address_space(3))) uint64_t lds_u64;
typedef __attribute__((address_space(3))) uint32_t lds_u32;

__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
  const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)v, src);
  const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(v >> 32), src);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, m);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), m);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const uint64_t o = shfl_xor_u64(v, m);
    v = o > v ? o : v;
  }
  return v;
}
__device__ __forceinline__ uint64_t wave_or_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v |= shfl_xor_u64(v, m);
  return v;
}
__device__ __forceinline__ uint64_t wave_and_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v &= shfl_xor_u64(v, m);
  return v;
}
__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}
__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

// A probability as the accept test compares it: exp2((l - m) c) inv_z from
// the fp32 row statistics, evaluated in fp64.  A draft token's q(x) can lie
// below fp32's smallest normal, 2^-126, at low temperatures while p(x) / q(x)
// is large; in fp64 it reaches 2^-1074, as in the oracle's arithmetic.
// Contraction off: the product is rounded on its own, so that a later
// p - q of two equal laws is exactly 0.
__device__ __forceinline__ double test_prob(float l, float m, float c, double inv_z) {
#pragma clang fp contract(off)
  return exp2(((double)l - (double)m) * (double)c) * inv_z;
}

// Sums of exponentials t in [0, 1] that do not depend on the order of the
// terms: each term is truncated to a multiple of 2^-52 (NaN counts as 0) and
// the integers are added exactly; at most 1024 terms keep the total below
// 2^62.  Two kept sets that hold the same logits in different orders then
// get the same normaliser, so their laws agree token by token (and p - q is
// exactly 0 where the logits agree).
__device__ __forceinline__ uint64_t unit_fixed(float t) { return t > 0.f ? (uint64_t)(t * 0x1.0p52f) : 0ull; }
__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor_u64(v, m);
  return v;
}
__device__ __forceinline__ float wave_sum_fixed(uint64_t v) { return (float)wave_sum_u64(v) * 0x1.0p-52f; }

// Online softmax pair (m = max logit, s = sum exp2((l - m) * c)) merge.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2, float c) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) {
    m = M;
    s = 0.f;
    return;
  }
  s = s * __builtin_amdgcn_exp2f((m - M) * c) + s2 * __builtin_amdgcn_exp2f((m2 - M) * c);
  m = M;
}
__device__ __forceinline__ void wave_lse(float& m, float& s, float c) {
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) {
    const float m2 = __shfl_xor(m, k);
    const float s2 = __shfl_xor(s, k);
    lse_merge(m, s, m2, s2, c);
  }
}

}  // namespace sv
