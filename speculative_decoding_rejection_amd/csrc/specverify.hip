// libspecverify C ABI: argument validation, workspace plan, kernel launches.
// Declarations and the contract of every entry point: include/specverify.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <map>
#include <mutex>
#include <vector>

#include "specverify.h"
#include "sv_batch.hpp"

namespace {

using sv::RaceDesc;
using sv::ReqInfo;
using sv::RowCut;

constexpr int kRowThreads = 256;
#ifndef SV_ROW_UNROLL
#define SV_ROW_UNROLL 4
#endif
constexpr int kRowUnroll = SV_ROW_UNROLL;  // vectors per thread in flight in the softmax and argmax row passes
#ifndef SV_TOPK_UNROLL
#define SV_TOPK_UNROLL 12
#endif
constexpr int kTopkUnroll = SV_TOPK_UNROLL;
constexpr int kMaxTopK = 1024;
constexpr int kMaxGamma = 16384;  // the top-k accept pass keeps one byte per position in LDS
constexpr size_t kWsAlign = 256;
constexpr int kEntryProb = 0, kEntryOnehot = 1, kEntryGreedy = 2;
// A call whose logits total at most this many bytes splits its rows into
// pieces of at least kSmallMinSeg elements (else 8192 / 2048).
constexpr size_t kSmallCallBytes = (size_t)64 << 20;
#ifndef SV_SMALL_MIN_SEG
#define SV_SMALL_MIN_SEG 2048
#endif
constexpr int kSmallMinSeg = SV_SMALL_MIN_SEG;
constexpr size_t kFusedLdsBytes = 32768;
// Measured on MI355X (race splits per request, us per call): fp32 full rows
// (B 256, V 151936) 4 / 6 / 8 / 16 splits: 414 / 412.5 / 418 / 421.5; one-hot
// bf16 (B 512, V 262144) 2 / 3 / 4 / 8: 317 / 316 / 312 / 312.5; bf16 full
// rows (B 512, V 128256) 2 / 3 / 4 / 8: 276 / 252 / 241.5 / 244.
constexpr int kFusedRaceMinSeg = 24576;
// Calls of at most kSmallCallBytes (8 requests, gamma 4, V 32000, fp32: race
// splits of at least 256 / 512 / 1024 / 2048 / 4096 tokens, us per call:
// 21.5 / 18.8 / 18.1 / 18.8 / 20.6).
constexpr int kSmallFusedRaceMinSeg = 1024;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Everything a call needs, derived from the parameters alone.
struct Plan {
  int B, G, V, dtype, esize;
  int K;          // active top-k (0 = off)
  int kcap;       // candidate keys stored per row (K rounded to its kernel tier)
  float c;        // log2(e) / T
  int rows_t, rows_d;
  int S, seg;     // row-pass splits of the vocabulary (softmax / argmax)
  int Sr, segr;   // race-pass splits
  size_t off_err, off_part, off_cand, off_desc, off_slots, off_info, off_cut, total;
  size_t off_gath;  // gathered draft-token logits, one float per row (full-row single-setting calls)
  size_t off_tpart, off_tkey;  // per race split: masses, counts and set-aside key of a peaked residual race
  bool fused;       // full rows, G < 64: accept and race in one launch (accept_race_kernel)
  int Srr, segrr;                           // row-race splits (sampler-match)
  size_t off_rdesc, off_rslots, off_samples;  // per-row race descriptors, slots, samples
  // Nucleus of few rows split across workgroups: plan, row list, chunk
  // histograms, per-row state, collected keys (batch calls with top-p).
  size_t off_nplan = 0, off_nlist = 0, off_nhist = 0, off_nstate = 0, off_nkeys = 0;
  int nuc_rows = 0, nuc_items = 0;  // grids of the per-row and per-chunk passes
  sv::Layout L;   // rows, tokens, outputs (dense: rows V apart, every request G positions)
  bool big_k;     // batch plans: a top-k above kcap is possible (full-row cut)
};

// Splits per row so that rows x splits stays within target_blocks (one
// round of workgroups at full occupancy: 256 CUs x 8 workgroups of 256
// threads = 2048), each split at least min_seg elements.
int splits_for(int rows, int V, int target_blocks, int min_seg) {
  int s = target_blocks / rows;
  int smax = V / min_seg;
  if (smax < 1) smax = 1;
  if (s > smax) s = smax;
  if (s < 1) s = 1;
  return s;
}

int seg_for(int V, int S) {
  // Split boundaries on multiples of 64 elements keep 16-byte alignment
  // relative to the row start.
  int seg = (V + S - 1) / S;
  seg = (seg + 63) / 64 * 64;
  return seg;
}

sv_status make_plan(const sv_params* p, int entry, Plan* pl) {
  if (!p) return SV_ERR_INVALID_ARG;
  if (p->batch < 1 || p->gamma < 1 || p->vocab < 1) return SV_ERR_INVALID_ARG;
  if (p->dtype != SV_F32 && p->dtype != SV_BF16) return SV_ERR_DTYPE;
  if (p->top_k < 0) return SV_ERR_INVALID_ARG;
  if (entry != kEntryGreedy && !(p->temperature > 0.f && std::isfinite(p->temperature))) return SV_ERR_INVALID_ARG;
  const int64_t B = p->batch, G = p->gamma, V = p->vocab;
  if (G > kMaxGamma) return SV_ERR_UNSUPPORTED;
  const int64_t rows = B * (2 * G + 1);
  if (rows > (int64_t)INT32_MAX / 64 || V > (int64_t)INT32_MAX - 1024) return SV_ERR_INVALID_ARG;
  Plan q{};
  q.B = (int)B;
  q.G = (int)G;
  q.V = (int)V;
  q.dtype = p->dtype;
  q.esize = p->dtype == SV_F32 ? 4 : 2;
  q.K = (entry != kEntryGreedy && p->top_k > 0 && p->top_k < p->vocab) ? p->top_k : 0;
  if (q.K > kMaxTopK) return SV_ERR_UNSUPPORTED;
  q.kcap = q.K;
  q.c = entry == kEntryGreedy ? 0.f : (float)(1.4426950408889634 / (double)p->temperature);
  q.rows_t = (int)(B * (G + 1));
  q.rows_d = (int)(B * G);  // sized for the prob entry; unused by the others
  const size_t nrows = (size_t)q.rows_t + (size_t)q.rows_d;
  // Splits of the row pass over `rows` rows.  Few rows: shorter splits, so
  // that the pass still spreads over the chip and each workgroup's share is
  // one or two rounds of loads.
  auto row_splits = [&](size_t rows, int* seg) {
    const bool sm = rows * (size_t)q.V * (size_t)q.esize <= kSmallCallBytes;
    *seg = seg_for(q.V, splits_for((int)rows, q.V, 2048, sm ? kSmallMinSeg : 8192));
    return (q.V + *seg - 1) / *seg;
  };
  // The sampled entries plan the splits over target and draft rows (the
  // plan a batch call with the same settings starts from, so that its row
  // sums merge alike); greedy reads only the target rows and takes an
  // argmax, which no split changes.  The partials area fits either, so one
  // workspace size serves every entry.
  int seg_all = 0, seg_t = 0;
  const int S_all = row_splits(nrows, &seg_all), S_t = row_splits((size_t)q.rows_t, &seg_t);
  const size_t part_slots = std::max(nrows * (size_t)S_all, (size_t)q.rows_t * (size_t)S_t);
  q.S = entry == kEntryGreedy ? S_t : S_all;
  q.seg = entry == kEntryGreedy ? seg_t : seg_all;
  const bool small = nrows * (size_t)q.V * (size_t)q.esize <= kSmallCallBytes;
  // Accept and race in one launch when the request's row partials fit the
  // fused kernel's LDS staging.
  q.fused = entry != kEntryGreedy && q.K == 0 && q.G < 64 &&
            (size_t)(2 * q.G + 1) * (size_t)q.S * 8 <= kFusedLdsBytes;
  // Race splits.  Every workgroup of the fused kernel takes its request's
  // accept decisions before it races, so large fused calls race longer
  // splits (at least kFusedRaceMinSeg tokens); small fused calls, bound by
  // latency, race shorter ones (kSmallFusedRaceMinSeg).  The race state is
  // sized for the most splits any entry takes (the shortest minimum), so
  // that one workspace size serves every entry.
  auto race_splits = [&](int min_seg, int* seg) {
    *seg = seg_for(q.V, splits_for(q.B, q.V, 4096, min_seg));
    return (q.V + *seg - 1) / *seg;
  };
  int seg_ws = 0;
  const int Sr_ws = race_splits(small ? std::min(kSmallMinSeg, kSmallFusedRaceMinSeg) : 2048, &seg_ws);
  q.Sr = race_splits(small ? (q.fused ? kSmallFusedRaceMinSeg : kSmallMinSeg) : (q.fused ? kFusedRaceMinSeg : 2048),
                     &q.segr);
  size_t off = 0;
  q.off_err = off;
  off = align_up(off + sizeof(int), kWsAlign);
  q.off_part = off;
  // Row-pass partials: float2 (softmax) or uint64 (argmax), both 8 bytes.
  off = align_up(off + part_slots * 8, kWsAlign);
  q.off_cand = off;
  off = align_up(off + (q.K ? nrows * (size_t)q.kcap * 8 : 0), kWsAlign);
  q.off_desc = off;
  off = align_up(off + (size_t)q.B * sizeof(RaceDesc), kWsAlign);
  q.off_slots = off;
  off = align_up(off + (size_t)q.B * 3 * 8, kWsAlign);
  q.off_gath = off;
  off = align_up(off + nrows * sizeof(float), kWsAlign);
  q.off_tpart = off;
  off = align_up(off + (size_t)q.B * (size_t)Sr_ws * 32, kWsAlign);
  q.off_tkey = off;
  off = align_up(off + (size_t)q.B * (size_t)Sr_ws * 8, kWsAlign);
  q.off_info = q.off_cut = off;
  q.total = off;
  q.L = sv::Layout{nullptr, (int64_t)q.V, (int64_t)q.V};
  *pl = q;
  return SV_OK;
}

// The largest top-k a batch call may use: sampling->max_top_k, or the call's
// single top_k when there are no per-request settings.
int batch_max_top_k(const sv_params* p, const sv_sampling* sm) {
  if (sm) return sm->max_top_k;
  return (p->top_k > 0 && p->top_k < p->vocab) ? p->top_k : 0;
}

// Plan of a batch call: the scalar plan's layout sized for the largest top-k
// kept as candidates (at most kMaxTopK: a larger top-k is a cut over the full
// row), plus per-request settings and per-row cuts (top-p, large top-k).
sv_status make_batch_plan(const sv_params* p, const sv_sampling* sm, Plan* pl) {
  if (!p) return SV_ERR_INVALID_ARG;
  if (sm && !sm->temperature) return SV_ERR_INVALID_ARG;
  if (!sm && !(std::isfinite(p->temperature) && p->temperature >= 0.f)) return SV_ERR_INVALID_ARG;
  const int mk = batch_max_top_k(p, sm);
  if (mk < 0 || p->top_k < 0) return SV_ERR_INVALID_ARG;
  // Candidates per row; none when the call's one setting is a large top-k.
  const int cap = (!sm && mk > kMaxTopK) ? 0 : (mk < kMaxTopK ? mk : kMaxTopK);
  sv_params q = *p;
  q.temperature = 1.f;
  q.top_k = p->vocab > 1 ? (cap < p->vocab - 1 ? cap : p->vocab - 1) : 0;
  sv_status s = make_plan(&q, kEntryProb, pl);
  if (s != SV_OK) return s;
  pl->c = 0.f;
  // A kind of request may hold only part of the batch: the softmax and
  // argmax passes split rows as if a quarter of them were theirs.
  const int act = (pl->rows_t + pl->rows_d + 3) / 4;
  const int S = splits_for(act, pl->V, 2048, 8192);
  if (S > pl->S) {
    pl->seg = seg_for(pl->V, S);
    pl->S = (pl->V + pl->seg - 1) / pl->seg;
    size_t off = pl->off_part;
    off = align_up(off + ((size_t)pl->rows_t + (size_t)pl->rows_d) * (size_t)pl->S * 8, kWsAlign);
    const size_t shift = off > pl->off_cand ? off - pl->off_cand : 0;  // later sections move up
    pl->off_cand += shift;
    pl->off_desc += shift;
    pl->off_slots += shift;
    pl->off_gath += shift;
    pl->off_tpart += shift;
    pl->off_tkey += shift;
    pl->total += shift;
  }
  size_t off = pl->total;
  pl->off_info = off;
  off = align_up(off + (size_t)pl->B * sizeof(ReqInfo), kWsAlign);
  pl->off_cut = off;
  pl->big_k = mk > pl->kcap && pl->V > 1;  // some request may take a full-row top-k cut
  if ((sm && sm->top_p) || pl->big_k)
    off = align_up(off + ((size_t)pl->rows_t + (size_t)pl->rows_d) * sizeof(RowCut), kWsAlign);
  // Sampler-match: one sample per target row; the full-row race over rows
  // is ALU-bound, so it splits rows finely (at least 2048 tokens a split).
  pl->Srr = splits_for(pl->rows_t, pl->V, 8192, 2048);
  pl->segrr = seg_for(pl->V, pl->Srr);
  pl->Srr = (pl->V + pl->segrr - 1) / pl->segrr;
  pl->off_rdesc = off;
  off = align_up(off + (size_t)pl->rows_t * sizeof(RaceDesc), kWsAlign);
  pl->off_rslots = off;
  off = align_up(off + (size_t)pl->rows_t * 3 * 8, kWsAlign);
  pl->off_samples = off;
  off = align_up(off + (size_t)pl->rows_t * 4, kWsAlign);
  if (sm && sm->top_p) {
    const int nr = pl->rows_t + pl->rows_d;
    pl->nuc_rows = nr < sv::kNucSplitRows ? nr : sv::kNucSplitRows;
    const int64_t items = (int64_t)pl->nuc_rows * sv::kNucMaxSplit;
    pl->nuc_items = items < sv::kNucItems ? (int)items : sv::kNucItems;
    pl->off_nplan = off;
    off = align_up(off + 4 * sizeof(int), kWsAlign);
    pl->off_nlist = off;
    off = align_up(off + (size_t)nr * sizeof(int), kWsAlign);
    pl->off_nhist = off;
    off = align_up(off + (size_t)pl->nuc_items * sv::kNucPartStride * sizeof(double), kWsAlign);
    pl->off_nstate = off;
    off = align_up(off + (size_t)pl->nuc_rows * sizeof(sv::NucState), kWsAlign);
    pl->off_nkeys = off;
    off = align_up(off + (size_t)pl->nuc_rows * sv::kNucCap * sizeof(uint64_t), kWsAlign);
  }
  pl->total = off;
  return SV_OK;
}

// ---------------------------------------------------------------------------
// Per-kernel timing (measurement only).
// ---------------------------------------------------------------------------
constexpr int kFamilies = 3;
constexpr size_t kMaxTimed = 65536;
bool g_timing = false;
std::vector<std::pair<hipEvent_t, hipEvent_t>> g_events[kFamilies];
size_t g_used[kFamilies] = {0, 0, 0};

struct TimedLaunch {
  int fam;
  hipStream_t st;
  hipEvent_t stop = nullptr;
  // f < 0: not timed (a launch inside a span timed as a whole).
  TimedLaunch(int f, hipStream_t s) : fam(f), st(s) {
    if (fam < 0 || !g_timing || g_used[fam] >= kMaxTimed) return;
    auto& ev = g_events[fam];
    if (g_used[fam] == ev.size()) {
      hipEvent_t a, b;
      if (hipEventCreate(&a) != hipSuccess) return;
      if (hipEventCreate(&b) != hipSuccess) {
        (void)hipEventDestroy(a);
        return;
      }
      ev.emplace_back(a, b);
    }
    if (hipEventRecord(ev[g_used[fam]].first, st) != hipSuccess) return;
    stop = ev[g_used[fam]].second;
  }
  void done() {
    if (!stop) return;
    if (hipEventRecord(stop, st) == hipSuccess) ++g_used[fam];
    stop = nullptr;
  }
};

sv_status check_launch() { return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP; }

// ---------------------------------------------------------------------------
// Side streams of a batch call's row phase.  The rows of different kinds of
// request are disjoint and each kind has its own row kernels, so the top-k
// rows and the temperature-0 rows are streamed on two side streams while the
// full rows take the caller's stream: a kind that holds few rows no longer
// runs alone on the chip.  Fork and join are events recorded on the caller's
// stream and the side streams (stream order is kept; a capture of the
// caller's stream takes the side streams in).  Created once per device
// (non-blocking, default priority); the lock covers the enqueue of a fork and
// its join, so concurrent host threads do not interleave the shared events.
// ---------------------------------------------------------------------------
struct SideStreams {
  hipStream_t s[2] = {nullptr, nullptr};
  hipEvent_t fork = nullptr, join[2] = {nullptr, nullptr};
};
std::mutex g_side_mu;
std::map<int, SideStreams> g_side;

// With g_side_mu held.  Null if the streams do not exist and cannot be made
// now (then the row phase runs on the caller's stream alone, and a later call
// tries again): they are not created while `st` is being captured into a
// graph, so that a capture is never disturbed by their creation.
SideStreams* side_streams(hipStream_t st) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  auto it = g_side.find(dev);
  if (it != g_side.end()) return &it->second;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) {
    (void)hipGetLastError();
    return nullptr;
  }
  SideStreams ss;
  bool ok = true;
  for (int i = 0; i < 2 && ok; ++i) ok = hipStreamCreateWithFlags(&ss.s[i], hipStreamNonBlocking) == hipSuccess;
  ok = ok && hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) == hipSuccess;
  for (int i = 0; i < 2 && ok; ++i) ok = hipEventCreateWithFlags(&ss.join[i], hipEventDisableTiming) == hipSuccess;
  if (!ok) {
    for (hipStream_t h : ss.s)
      if (h) (void)hipStreamDestroy(h);
    for (hipEvent_t e : {ss.fork, ss.join[0], ss.join[1]})
      if (e) (void)hipEventDestroy(e);
    (void)hipGetLastError();  // the failure is not the caller's launch error
    return nullptr;
  }
  return &g_side.emplace(dev, ss).first->second;
}

bool aligned(const void* ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

// null_tokens: a ragged batch call may pass no draft tokens (every draft
// length 0, checked on the device).
sv_status check_common(const Plan& pl, const void* target_logits, const int32_t* draft_tokens, int32_t* out_tokens,
                       int32_t* num_accepted, void* workspace, size_t workspace_bytes, bool null_tokens = false) {
  if (!target_logits || (!draft_tokens && !null_tokens) || !out_tokens || !num_accepted) return SV_ERR_INVALID_ARG;
  if (!aligned(target_logits, (size_t)pl.esize)) return SV_ERR_DTYPE;
  if (!aligned(draft_tokens, 4) || !aligned(out_tokens, 4) || !aligned(num_accepted, 4)) return SV_ERR_INVALID_ARG;
  if (!workspace || !aligned(workspace, kWsAlign) || workspace_bytes < pl.total) return SV_ERR_WORKSPACE;
  return SV_OK;
}

template <typename ET>
sv_status run_rows_softmax(const Plan& pl, const void* lt, const void* ld, int nrows, char* ws, hipStream_t st,
                           const ReqInfo* info = nullptr, int fam = 0, const int32_t* X = nullptr) {
  TimedLaunch t(fam, st);
  float* gath = X ? (float*)(ws + pl.off_gath) : nullptr;
  unsigned long long* slots = X ? (unsigned long long*)(ws + pl.off_slots) : nullptr;
  hipLaunchKernelGGL((sv::rows_softmax_kernel<ET, kRowThreads, kRowUnroll>), dim3(nrows * pl.S),
                     dim3(kRowThreads), 0, st, (const ET*)lt, (const ET*)ld, pl.rows_t, pl.V, pl.S, pl.seg, pl.c,
                     (float2*)(ws + pl.off_part), (int*)(ws + pl.off_err), info, pl.G, pl.L, X, gath, slots);
  t.done();
  return check_launch();
}

#ifndef SV_TOPK_CAPW64
#define SV_TOPK_CAPW64 768  // per-wave key buffer for k <= 64
#endif
#ifndef SV_TOPK_WPR
#define SV_TOPK_WPR 2  // waves per row in the top-k row pass (k > 64)
#endif

#ifndef SV_TOPK_RPB
#define SV_TOPK_RPB 2  // rows per workgroup in the top-k row pass (k > 64)
#endif

// For k <= 64: one row per 256-thread workgroup, 4 waves per row (measured
// on MI355X against 2 rows of 2 waves: headline row pass 1332 -> 1319 us,
// mixed batch 1% faster, sampler-match 1-2% slower).
#ifndef SV_TOPK_WPR64
#define SV_TOPK_WPR64 4
#endif
#ifndef SV_TOPK_RPB64
#define SV_TOPK_RPB64 1
#endif

template <typename ET, int CAPW, int WPR = SV_TOPK_WPR, int RPB = SV_TOPK_RPB>
void launch_rows_topk(const Plan& pl, const void* lt, const void* ld, int nrows, uint64_t* cand, int* err,
                      hipStream_t st, const ReqInfo* info) {
  hipLaunchKernelGGL((sv::rows_topk_kernel<ET, CAPW, kTopkUnroll, WPR, RPB>), dim3((nrows + RPB - 1) / RPB),
                     dim3(WPR * RPB * 64), 0, st, (const ET*)lt, (const ET*)ld, pl.rows_t, nrows, pl.V, pl.K,
                     cand, err, info, pl.G, pl.kcap, pl.L);
}

// pl.K: the top-k of every row, or (batch call) the largest one; rows are
// stored pl.kcap keys apart.
template <typename ET>
sv_status run_rows_topk(const Plan& pl, const void* lt, const void* ld, int nrows, char* ws, hipStream_t st,
                        const ReqInfo* info = nullptr, int fam = 0) {
  TimedLaunch t(fam, st);
  uint64_t* cand = (uint64_t*)(ws + pl.off_cand);
  int* err = (int*)(ws + pl.off_err);
  // Buffer capacity per wave: >= K + 64 * (elements per vector) for one
  // vector step after a compaction, and >= WPR * K for the final merge.
  if (pl.K <= 64) {
    launch_rows_topk<ET, SV_TOPK_CAPW64, SV_TOPK_WPR64, SV_TOPK_RPB64>(pl, lt, ld, nrows, cand, err, st, info);
  } else if (pl.K <= 256) {
    launch_rows_topk<ET, 1024>(pl, lt, ld, nrows, cand, err, st, info);
  } else {
    launch_rows_topk<ET, 4096>(pl, lt, ld, nrows, cand, err, st, info);
  }
  t.done();
  return check_launch();
}

template <typename ET, bool CUT, bool QP>
sv_status run_race(const Plan& pl, const void* lt, const void* ld, uint32_t k0, uint32_t k1, char* ws, int32_t* out,
                   hipStream_t st) {
  TimedLaunch t(2, st);
  RaceDesc* desc = (RaceDesc*)(ws + pl.off_desc);
  unsigned long long* slots = (unsigned long long*)(ws + pl.off_slots);
  float4* tpart = (float4*)(ws + pl.off_tpart);
  unsigned long long* tkey = (unsigned long long*)(ws + pl.off_tkey);
  hipLaunchKernelGGL((sv::race_full_kernel<ET, 256, CUT, QP>), dim3(pl.B * pl.Sr), dim3(256), 0, st,
                     (const ET*)lt, QP ? (const ET*)nullptr : (const ET*)ld, QP ? (const float*)ld : nullptr, pl.V,
                     pl.Sr, pl.segr, k0, k1, (const RaceDesc*)desc, slots, tpart, tkey);
  hipLaunchKernelGGL((sv::race_finish_kernel<ET, 256, CUT>), dim3(pl.B), dim3(256), 0, st, (const ET*)lt, pl.G,
                     pl.V, k0, k1, (const RaceDesc*)desc, (const unsigned long long*)slots, out,
                     (const float4*)tpart, (const unsigned long long*)tkey, pl.Sr,
                     QP ? (const float*)ld : (const float*)nullptr);
  t.done();
  return check_launch();
}

// One sample per target row of a full-row request (sampler-match): the
// full-row race over every such row (descriptors and slots per row), then
// the winners to `samples`.
template <typename ET, bool CUT>
sv_status run_row_race(const Plan& pl, const void* lt, uint32_t k0, uint32_t k1, char* ws, hipStream_t st) {
  TimedLaunch t(2, st);
  const RaceDesc* rdesc = (const RaceDesc*)(ws + pl.off_rdesc);
  unsigned long long* rslots = (unsigned long long*)(ws + pl.off_rslots);
  hipLaunchKernelGGL((sv::race_full_kernel<ET, 256, CUT, false>), dim3(pl.rows_t * pl.Srr), dim3(256), 0, st,
                     (const ET*)lt, (const ET*)nullptr, (const float*)nullptr, pl.V, pl.Srr, pl.segrr, k0, k1, rdesc,
                     rslots);
  hipLaunchKernelGGL(sv::match_samples_kernel, dim3((pl.rows_t + 255) / 256), dim3(256), 0, st, pl.rows_t, rdesc,
                     (const unsigned long long*)rslots, (int32_t*)(ws + pl.off_samples));
  t.done();
  return check_launch();
}

// Accept pass over top-k candidates: the staged small kernel when every
// request keeps at most 64 tokens and has at most 16 positions, else the
// general one.  K: the call's top-k, or its largest (the candidate stride).
template <int MODE>
void launch_accept_topk(const Plan& pl, const uint64_t* cand, const int32_t* X, int K, float c, uint32_t k0,
                        uint32_t k1, int32_t* out, int32_t* nacc, float* p_draft, float* q_draft, int* err,
                        const ReqInfo* info, const float* qp, sv::Stats stats, hipStream_t st) {
  if (pl.kcap <= sv::kSmallK && pl.G <= sv::kSmallG) {
    hipLaunchKernelGGL((sv::accept_topk_small_kernel<MODE>), dim3(pl.B), dim3(512), 0, st, cand, X, pl.G, pl.V, K,
                       pl.rows_t, c, k0, k1, out, nacc, p_draft, q_draft, err, info, pl.kcap, pl.L, qp, stats);
  } else {
    hipLaunchKernelGGL((sv::accept_topk_kernel<MODE>), dim3(pl.B), dim3(256), (size_t)pl.G, st, cand, X, pl.G,
                       pl.V, K, pl.rows_t, c, k0, k1, out, nacc, p_draft, q_draft, err, info, pl.kcap, pl.L, qp,
                       stats);
  }
}

template <typename ET, int MODE>
sv_status verify_sampled(const Plan& pl, uint64_t seed, const void* lt, const void* ld, const int32_t* X,
                         int32_t* out, int32_t* nacc, float* p_draft, float* q_draft, char* ws, hipStream_t st) {
  const int nrows = pl.rows_t + (MODE == 0 ? pl.rows_d : 0);
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  int* err = (int*)(ws + pl.off_err);
  sv_status s;
  if (pl.K) {
    s = run_rows_topk<ET>(pl, lt, ld, nrows, ws, st);
    if (s != SV_OK) return s;
    TimedLaunch t(1, st);
    launch_accept_topk<MODE>(pl, (const uint64_t*)(ws + pl.off_cand), X, pl.kcap, pl.c, k0, k1, out, nacc, p_draft,
                             q_draft, err, (const ReqInfo*)nullptr, (const float*)nullptr,
                             sv::Stats{nullptr, nullptr}, st);
    t.done();
    return check_launch();
  }
  RaceDesc* desc = (RaceDesc*)(ws + pl.off_desc);
  unsigned long long* slots = (unsigned long long*)(ws + pl.off_slots);
  if (pl.fused) {
    // Row pass (with the draft tokens' logits and the race slots cleared),
    // then accept and race in one launch, then the finish.
    s = run_rows_softmax<ET>(pl, lt, ld, nrows, ws, st, nullptr, 0, X);
    if (s != SV_OK) return s;
    TimedLaunch t(2, st);
    const size_t lds = (size_t)(pl.G + 1 + (MODE == 0 ? pl.G : 0)) * pl.S * sizeof(float2);
    hipLaunchKernelGGL((sv::accept_race_kernel<ET, MODE>), dim3(pl.B * pl.Sr), dim3(256), lds, st, (const ET*)lt,
                       (const ET*)ld, (const float2*)(ws + pl.off_part), (const float*)(ws + pl.off_gath), X, pl.G,
                       pl.V, pl.S, pl.rows_t, pl.c, k0, k1, pl.Sr, pl.segr, out, nacc, p_draft, q_draft, desc, slots,
                       err, (float4*)(ws + pl.off_tpart), (unsigned long long*)(ws + pl.off_tkey));
    hipLaunchKernelGGL((sv::race_finish_kernel<ET, 256, false>), dim3(pl.B), dim3(256), 0, st, (const ET*)lt, pl.G,
                       pl.V, k0, k1, (const RaceDesc*)desc, (const unsigned long long*)slots, out,
                       (const float4*)(ws + pl.off_tpart), (const unsigned long long*)(ws + pl.off_tkey), pl.Sr);
    t.done();
    return check_launch();
  }
  s = run_rows_softmax<ET>(pl, lt, ld, nrows, ws, st);
  if (s != SV_OK) return s;
  {
    TimedLaunch t(1, st);
    hipLaunchKernelGGL((sv::accept_full_kernel<ET, MODE>), dim3(pl.B), dim3(64), 0, st, (const ET*)lt,
                       (const ET*)ld, (const float2*)(ws + pl.off_part), X, pl.G, pl.V, pl.S, pl.rows_t, pl.c, k0,
                       k1, out, nacc, p_draft, q_draft, desc, slots, err, (const ReqInfo*)nullptr,
                       (const RowCut*)nullptr, pl.L, (const float*)nullptr, sv::Stats{nullptr, nullptr});
    t.done();
    s = check_launch();
    if (s != SV_OK) return s;
  }
  return run_race<ET, false, false>(pl, lt, ld, k0, k1, ws, out, st);
}

template <typename ET>
sv_status verify_greedy(const Plan& pl, const void* lt, const int32_t* X, int32_t* out, int32_t* nacc,
                        int32_t* targ, char* ws, hipStream_t st) {
  int* err = (int*)(ws + pl.off_err);
  uint64_t* part = (uint64_t*)(ws + pl.off_part);
  {
    TimedLaunch t(0, st);
    hipLaunchKernelGGL((sv::rows_argmax_kernel<ET, kRowThreads, kRowUnroll>), dim3(pl.rows_t * pl.S),
                       dim3(kRowThreads), 0, st, (const ET*)lt, pl.V, pl.S, pl.seg, part, err,
                       (const ReqInfo*)nullptr, pl.G, pl.L);
    t.done();
    sv_status s = check_launch();
    if (s != SV_OK) return s;
  }
  TimedLaunch t(1, st);
  hipLaunchKernelGGL(sv::accept_greedy_kernel, dim3(pl.B), dim3(64), 0, st, (const uint64_t*)part, X, pl.G, pl.V,
                     pl.S, out, nacc, targ, err, (const ReqInfo*)nullptr, (float*)nullptr, (float*)nullptr, pl.L,
                     sv::Stats{nullptr, nullptr});
  t.done();
  return check_launch();
}

// A batch call: per-request settings (device arrays, or the call's single
// setting), greedy, top-k and full-row requests, draft logits, one-hot drafts
// or draft probabilities (MODE 0 / 1 / 2), dense or ragged rows.  Every
// kernel of a kind runs over every (padded) row or request and skips those
// of other kinds or beyond a request's draft length.
struct BatchArgs {
  const float* T;
  const int32_t* K;
  const float* P;
  float T0;
  int K0, max_top_k;
  const int32_t* parents;  // sampler-match trees (null: chains)
  int no_drafts;           // ragged call without draft tokens or draft rows: every length must be 0
};

template <typename ET, int MODE>
sv_status verify_batch(const Plan& pl, const BatchArgs& ba, uint64_t seed, const void* lt, const void* ld,
                       const int32_t* X, const sv_outputs& o, char* ws, hipStream_t st) {
  int32_t* out = o.out_tokens;
  int32_t* nacc = o.num_accepted;
  float* p_draft = o.p_draft;
  float* q_draft = o.q_draft;
  float* beta = o.beta;
  int64_t* counters = o.counters;
  const int nrows = pl.rows_t + (MODE == 0 ? pl.rows_d : 0);  // MODE 3 (sampler-match): target rows only
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  int* err = (int*)(ws + pl.off_err);
  ReqInfo* info = (ReqInfo*)(ws + pl.off_info);
  RowCut* cut = (RowCut*)(ws + pl.off_cut);
  uint64_t* part64 = (uint64_t*)(ws + pl.off_part);
  const bool nuc = ba.P != nullptr;        // top-p settings given: nucleus passes
  const bool use_cut = nuc || pl.big_k;    // full rows may carry a RowCut
  const float* qp = MODE == 2 ? (const float*)ld : nullptr;
  const void* ldl = MODE == 0 ? ld : nullptr;  // draft logits, if any
  sv_status s;
  {
    TimedLaunch t(0, st);
    hipLaunchKernelGGL(sv::classify_kernel, dim3(1), dim3(1024), 0, st, ba.T, ba.K, ba.P, ba.T0, ba.K0, pl.B, pl.G,
                       pl.V, ba.max_top_k, pl.kcap, pl.L, MODE == 3 ? ba.parents : (const int32_t*)nullptr, info,
                       err, out, nacc, p_draft, q_draft, beta, MODE == 0 ? 1 : 0,
                       nuc ? (int*)(ws + pl.off_nplan) : (int*)nullptr,
                       nuc ? (int*)(ws + pl.off_nlist) : (int*)nullptr, ba.no_drafts);
    t.done();
    if ((s = check_launch()) != SV_OK) return s;
  }
  // The side streams join the caller's stream after the row phase, or (when
  // the kernels are not timed by family) at the end of the call: the
  // full-row requests' accept and race read nothing the side streams write,
  // so they run beside the top-k and temperature-0 row passes.  Sampler-match
  // samples read the top-k candidates and join first.
  const bool late_join = MODE != 3 && !g_timing;
  std::unique_lock<std::mutex> lock(g_side_mu);
  SideStreams* side = nullptr;
  hipStream_t s_topk = st, s_arg = st;
  // The caller's stream waits for both side streams (also after a failed
  // launch); the lock is released once the join is enqueued.
  auto join = [&]() -> sv_status {
    sv_status r = SV_OK;
    if (s_topk != st &&
        (hipEventRecord(side->join[0], s_topk) != hipSuccess || hipEventRecord(side->join[1], s_arg) != hipSuccess ||
         hipStreamWaitEvent(st, side->join[0], 0) != hipSuccess ||
         hipStreamWaitEvent(st, side->join[1], 0) != hipSuccess))
      r = SV_ERR_HIP;
    s_topk = s_arg = st;
    if (lock.owns_lock()) lock.unlock();
    return r;
  };
  {
    // Row phase: top-k rows (candidates, then their nucleus, then the
    // top-k requests' accept pass) on side stream 0, temperature-0 rows
    // (argmax, then their accept pass) on side stream 1, full rows (softmax
    // partials, then a large top-k's cut and the nucleus) on the caller's
    // stream.  The three write disjoint parts of the workspace and of the
    // outputs.
    TimedLaunch t(0, st);
    side = side_streams(st);
    if (side && hipEventRecord(side->fork, st) == hipSuccess &&
        hipStreamWaitEvent(side->s[0], side->fork, 0) == hipSuccess &&
        hipStreamWaitEvent(side->s[1], side->fork, 0) == hipSuccess) {
      s_topk = side->s[0];
      s_arg = side->s[1];
    }
    sv_status rs = SV_OK;
    if (pl.K > 0) {
      rs = run_rows_topk<ET>(pl, lt, ldl, nrows, ws, s_topk, info, -1);
      if (rs == SV_OK && nuc)
        hipLaunchKernelGGL(sv::nucleus_topk_kernel, dim3((nrows + 3) / 4), dim3(256), 0, s_topk,
                           (uint64_t*)(ws + pl.off_cand), pl.kcap, pl.rows_t, nrows, pl.G, (const ReqInfo*)info,
                           pl.L);
    }
    if (rs == SV_OK)
      hipLaunchKernelGGL((sv::rows_argmax_kernel<ET, kRowThreads, kRowUnroll>), dim3(pl.rows_t * pl.S),
                         dim3(kRowThreads), 0, s_arg, (const ET*)lt, pl.V, pl.S, pl.seg, part64, err,
                         (const ReqInfo*)info, pl.G, pl.L);
    if constexpr (MODE != 3) {
      // The accept passes of top-k and temperature-0 requests (and the
      // former's beta) depend only on their own row passes: they run on
      // those passes' streams, beside the full rows' softmax and nucleus
      // passes.  Each writes only its own requests' outputs.
      if (rs == SV_OK) {
        const sv::Stats stats{beta, counters};
        if (pl.K > 0) {
          launch_accept_topk<MODE>(pl, (const uint64_t*)(ws + pl.off_cand), X, pl.kcap, 0.f, k0, k1, out, nacc,
                                   p_draft, q_draft, err, (const ReqInfo*)info, qp, stats, s_topk);
          if (beta && MODE != 1)
            hipLaunchKernelGGL((sv::beta_topk_kernel<MODE>), dim3((pl.B * pl.G + 3) / 4), dim3(256), 0, s_topk,
                               (const uint64_t*)(ws + pl.off_cand), qp, pl.B, pl.G, pl.kcap, pl.rows_t,
                               (const ReqInfo*)info, pl.L, beta);
        }
        hipLaunchKernelGGL(sv::accept_greedy_kernel, dim3(pl.B), dim3(64), 0, s_arg, (const uint64_t*)part64, X,
                           pl.G, pl.V, pl.S, out, nacc, (int32_t*)nullptr, err, (const ReqInfo*)info, p_draft,
                           q_draft, pl.L, stats);
      }
    }
    if (rs == SV_OK) rs = run_rows_softmax<ET>(pl, lt, ldl, nrows, ws, st, info, -1);
    if (rs == SV_OK && pl.big_k)  // top-k above the candidate capacity: the k-th key of the full row, before any nucleus
      hipLaunchKernelGGL((sv::kcut_full_kernel<ET>), dim3(nrows), dim3(sv::kCutThreads), 0, st, (const ET*)lt,
                         (const ET*)ldl, pl.rows_t, pl.G, pl.V, pl.S, (const float2*)(ws + pl.off_part),
                         (const ReqInfo*)info, cut, pl.L);
    if (rs == SV_OK && nuc) {
      // The classify pass listed the top-p rows and picked one workgroup per
      // row or, for few rows, rows split across workgroups (the part pass's
      // grid covers both); the passes of the other path exit at once.
      int* nplan = (int*)(ws + pl.off_nplan);
      int* nlist = (int*)(ws + pl.off_nlist);
      double* nhist = (double*)(ws + pl.off_nhist);
      sv::NucState* nstate = (sv::NucState*)(ws + pl.off_nstate);
      uint64_t* nkeys = (uint64_t*)(ws + pl.off_nkeys);
      float2* sp = (float2*)(ws + pl.off_part);
      const dim3 nt(sv::NucShape::NT);
      hipLaunchKernelGGL((sv::nucleus_part_kernel<ET>), dim3(pl.nuc_items > nrows ? pl.nuc_items : nrows), nt, 0,
                         st, (const ET*)lt, (const ET*)ldl, pl.rows_t, pl.G, pl.V, pl.S, sp, (const ReqInfo*)info,
                         cut, pl.L, (const int*)nplan, (const int*)nlist, nhist);
      hipLaunchKernelGGL(sv::nucleus_scan_kernel, dim3(pl.nuc_rows), nt, 0, st, pl.rows_t, pl.G, pl.S, sp,
                         (const ReqInfo*)info, cut, (const int*)nplan, (const int*)nlist, (const double*)nhist,
                         nstate);
      hipLaunchKernelGGL((sv::nucleus_collect_kernel<ET>), dim3(pl.nuc_items), nt, 0, st, (const ET*)lt,
                         (const ET*)ldl, pl.rows_t, pl.G, pl.V, (const ReqInfo*)info, pl.L, (const int*)nplan,
                         (const int*)nlist, nstate, nkeys);
      hipLaunchKernelGGL((sv::nucleus_finish_kernel<ET>), dim3(pl.nuc_rows), nt, 0, st, (const ET*)lt,
                         (const ET*)ldl, pl.rows_t, pl.G, pl.V, pl.S, sp, (const ReqInfo*)info, cut, pl.L,
                         (const int*)nplan, (const int*)nlist, (const sv::NucState*)nstate,
                         (const uint64_t*)nkeys);
    }
    if (rs == SV_OK) rs = check_launch();
    if (rs != SV_OK || !late_join) {
      const sv_status js = join();
      if (rs == SV_OK) rs = js;
    }
    if (rs != SV_OK) return rs;
    t.done();
  }
  if (MODE == 3) {
    // Sampler-match: a sample for every node's row, then the walk.
    {
      TimedLaunch t(1, st);
      hipLaunchKernelGGL(sv::match_prep_kernel, dim3((pl.rows_t + 255) / 256), dim3(256), 0, st,
                         (const float2*)(ws + pl.off_part), pl.S, pl.rows_t, pl.G, (const ReqInfo*)info,
                         (const RowCut*)(use_cut ? cut : nullptr), pl.L, (RaceDesc*)(ws + pl.off_rdesc),
                         (unsigned long long*)(ws + pl.off_rslots));
      if (pl.K > 0)
        hipLaunchKernelGGL(sv::sample_topk_kernel, dim3((pl.rows_t + 3) / 4), dim3(256), 0, st,
                           (const uint64_t*)(ws + pl.off_cand), pl.kcap, pl.rows_t, pl.G, (const ReqInfo*)info, pl.L,
                           k0, k1, (int32_t*)(ws + pl.off_samples));
      t.done();
      if ((s = check_launch()) != SV_OK) return s;
    }
    s = use_cut ? run_row_race<ET, true>(pl, lt, k0, k1, ws, st) : run_row_race<ET, false>(pl, lt, k0, k1, ws, st);
    if (s != SV_OK) return s;
    TimedLaunch t(1, st);
    hipLaunchKernelGGL((sv::match_walk_kernel<ET>), dim3(pl.B), dim3(64), 0, st, (const ET*)lt,
                       (const float2*)(ws + pl.off_part), (const uint64_t*)part64,
                       (const uint64_t*)(ws + pl.off_cand), pl.kcap, pl.S, pl.G, pl.V, (const ReqInfo*)info,
                       (const RowCut*)(use_cut ? cut : nullptr), pl.L, X, ba.parents,
                       (const int32_t*)(ws + pl.off_samples), out, nacc, o.path_nodes, p_draft, q_draft,
                       sv::Stats{beta, counters}, err);
    t.done();
    return check_launch();
  }
  RaceDesc* desc = (RaceDesc*)(ws + pl.off_desc);
  unsigned long long* slots = (unsigned long long*)(ws + pl.off_slots);
  // Full-row requests (the top-k and temperature-0 ones are accepted on the
  // side streams): accept, beta and race on the caller's stream, then the
  // join if it is still pending.
  auto tail = [&]() -> sv_status {
    sv_status r;
    {
      TimedLaunch t(1, st);
      const sv::Stats stats{beta, counters};
      hipLaunchKernelGGL((sv::accept_full_kernel<ET, MODE>), dim3(pl.B), dim3(64), 0, st, (const ET*)lt,
                         (const ET*)ldl, (const float2*)(ws + pl.off_part), X, pl.G, pl.V, pl.S, pl.rows_t, 0.f, k0,
                         k1, out, nacc, p_draft, q_draft, desc, slots, err, (const ReqInfo*)info,
                         (const RowCut*)(use_cut ? cut : nullptr), pl.L, qp, stats);
      t.done();
      if ((r = check_launch()) != SV_OK) return r;
    }
    if (beta && MODE != 1) {
      // Acceptance probability of every position of requests without top-k:
      // one more read of their target and draft rows.
      TimedLaunch t(1, st);
      hipLaunchKernelGGL((sv::beta_full_kernel<ET, MODE == 2>), dim3(pl.B * pl.G), dim3(256), 0, st,
                         (const ET*)lt, (const ET*)ldl, qp, (const float2*)(ws + pl.off_part), pl.G, pl.V, pl.S,
                         pl.rows_t, (const ReqInfo*)info, (const RowCut*)(use_cut ? cut : nullptr), pl.L, beta);
      t.done();
      if ((r = check_launch()) != SV_OK) return r;
    }
    constexpr bool QP = MODE == 2;
    if (use_cut) return run_race<ET, true, QP>(pl, lt, ld, k0, k1, ws, out, st);
    return run_race<ET, false, QP>(pl, lt, ld, k0, k1, ws, out, st);
  };
  const sv_status ts = tail();
  const sv_status js = join();
  return ts != SV_OK ? ts : js;
}

// A single-setting call whose top-k exceeds the candidate capacity (and is
// below the vocabulary) runs as a batch call with that one setting: the
// top-k is a cut over each full row.
bool large_top_k(const sv_params* p) { return p && p->top_k > kMaxTopK && p->top_k < p->vocab; }

// The probabilistic-draft call once planned: argument checks against the
// plan, then the kernels on `workspace`.
sv_status prob_planned(const Plan& pl, uint64_t seed, const void* target_logits, const void* draft_logits,
                       const int32_t* draft_tokens, int32_t* out_tokens, int32_t* num_accepted, float* p_draft,
                       float* q_draft, void* workspace, size_t workspace_bytes, void* stream) {
  sv_status s = check_common(pl, target_logits, draft_tokens, out_tokens, num_accepted, workspace, workspace_bytes);
  if (s != SV_OK) return s;
  if (!draft_logits) return SV_ERR_INVALID_ARG;
  if (!aligned(draft_logits, (size_t)pl.esize)) return SV_ERR_DTYPE;
  if ((p_draft && !aligned(p_draft, 4)) || (q_draft && !aligned(q_draft, 4))) return SV_ERR_INVALID_ARG;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  if (pl.dtype == SV_F32)
    return verify_sampled<float, 0>(pl, seed, target_logits, draft_logits, draft_tokens, out_tokens, num_accepted,
                                    p_draft, q_draft, ws, st);
  return verify_sampled<uint16_t, 0>(pl, seed, target_logits, draft_logits, draft_tokens, out_tokens, num_accepted,
                                     p_draft, q_draft, ws, st);
}

// ---------------------------------------------------------------------------
// Scratch of spec_verify_prob_noalloc: a device array in the library's code
// object (each GPU that loads it holds its own copy until the process ends).
// Host code never uses the array's name as an address: its device address
// is looked up once per device with hipGetSymbolAddress (with that device
// current) and kept in g_noalloc_ptr.  Calls on one GPU share its copy.
// ---------------------------------------------------------------------------
constexpr size_t kNoAllocScratchBytes = SV_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
std::mutex g_noalloc_mu;
char* g_noalloc_ptr[kMaxDevices] = {};

}  // namespace

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

sv_status noalloc_scratch(char** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SV_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SV_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_noalloc_mu);
  if (!g_noalloc_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return SV_ERR_HIP;
    }
    g_noalloc_ptr[dev] = (char*)p;
  }
  *out = g_noalloc_ptr[dev];
  return SV_OK;
}

}  // namespace

extern "C" {

size_t sv_workspace_bytes(const sv_params* params) {
  if (large_top_k(params)) return sv_workspace_bytes_batch(params, nullptr);
  Plan pl;
  if (make_plan(params, kEntryProb, &pl) != SV_OK) {
    // Greedy parameters may carry any temperature.
    if (make_plan(params, kEntryGreedy, &pl) != SV_OK) return 0;
  }
  return pl.total;
}

const char* sv_status_string(sv_status s) {
  switch (s) {
    case SV_OK: return "ok";
    case SV_ERR_INVALID_ARG: return "invalid argument (size, temperature, top_k or null pointer)";
    case SV_ERR_DTYPE: return "unsupported dtype or misaligned logits";
    case SV_ERR_WORKSPACE: return "workspace missing, misaligned (256 B) or smaller than sv_workspace_bytes()";
    case SV_ERR_HIP: return "HIP runtime or kernel launch failure";
    case SV_ERR_UNSUPPORTED: return "unsupported: gamma above 16384, or (no-alloc entry) a top_k above 1024";
    case SV_ERR_SCRATCH: return "the call needs more device scratch than spec_verify_prob_noalloc holds (16 MiB)";
  }
  return "unknown status";
}

sv_status spec_verify_prob(const sv_params* params, const void* target_logits, const void* draft_logits,
                           const int32_t* draft_tokens, int32_t* out_tokens, int32_t* num_accepted, float* p_draft,
                           float* q_draft, void* workspace, size_t workspace_bytes, void* stream) {
  if (large_top_k(params)) {
    if (!(params->temperature > 0.f && std::isfinite(params->temperature))) return SV_ERR_INVALID_ARG;
    if (!draft_logits) return SV_ERR_INVALID_ARG;
    const sv_outputs o{out_tokens, num_accepted, p_draft, q_draft, nullptr, nullptr, nullptr};
    return spec_verify_batch(params, nullptr, nullptr, target_logits, draft_logits, draft_tokens, &o, workspace,
                             workspace_bytes, stream);
  }
  Plan pl;
  sv_status s = make_plan(params, kEntryProb, &pl);
  if (s != SV_OK) return s;
  return prob_planned(pl, params->seed, target_logits, draft_logits, draft_tokens, out_tokens, num_accepted,
                      p_draft, q_draft, workspace, workspace_bytes, stream);
}

sv_status spec_verify_prob_noalloc(const sv_params* params, const void* target_logits, const void* draft_logits,
                                   const int32_t* draft_tokens, int32_t* out_tokens, int32_t* num_accepted,
                                   float* p_draft, float* q_draft, int32_t* error_word, void* stream) {
  if (large_top_k(params)) return SV_ERR_UNSUPPORTED;  // the full-row cut runs as a batch call (side streams)
  Plan pl;
  sv_status s = make_plan(params, kEntryProb, &pl);
  if (s != SV_OK) return s;
  if (pl.total > kNoAllocScratchBytes) return SV_ERR_SCRATCH;
  if (error_word && !aligned(error_word, 4)) return SV_ERR_INVALID_ARG;
  char* ws = nullptr;
  if ((s = noalloc_scratch(&ws)) != SV_OK) return s;
  s = prob_planned(pl, params->seed, target_logits, draft_logits, draft_tokens, out_tokens, num_accepted, p_draft,
                   q_draft, ws, kNoAllocScratchBytes, stream);
  if (s != SV_OK || !error_word) return s;
  hipLaunchKernelGGL(sv::copy_word_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream,
                     (const int32_t*)(ws + pl.off_err), error_word);
  return check_launch();
}

sv_status spec_verify_onehot(const sv_params* params, const void* target_logits, const int32_t* draft_tokens,
                             int32_t* out_tokens, int32_t* num_accepted, float* p_draft, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (large_top_k(params)) {
    if (!(params->temperature > 0.f && std::isfinite(params->temperature))) return SV_ERR_INVALID_ARG;
    const sv_outputs o{out_tokens, num_accepted, p_draft, nullptr, nullptr, nullptr, nullptr};
    return spec_verify_batch(params, nullptr, nullptr, target_logits, nullptr, draft_tokens, &o, workspace,
                             workspace_bytes, stream);
  }
  Plan pl;
  sv_status s = make_plan(params, kEntryOnehot, &pl);
  if (s != SV_OK) return s;
  s = check_common(pl, target_logits, draft_tokens, out_tokens, num_accepted, workspace, workspace_bytes);
  if (s != SV_OK) return s;
  if (p_draft && !aligned(p_draft, 4)) return SV_ERR_INVALID_ARG;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  if (pl.dtype == SV_F32)
    return verify_sampled<float, 1>(pl, params->seed, target_logits, nullptr, draft_tokens, out_tokens, num_accepted,
                                    p_draft, nullptr, ws, st);
  return verify_sampled<uint16_t, 1>(pl, params->seed, target_logits, nullptr, draft_tokens, out_tokens,
                                     num_accepted, p_draft, nullptr, ws, st);
}

sv_status spec_verify_greedy(const sv_params* params, const void* target_logits, const int32_t* draft_tokens,
                             int32_t* out_tokens, int32_t* num_accepted, int32_t* target_argmax, void* workspace,
                             size_t workspace_bytes, void* stream) {
  Plan pl;
  sv_status s = make_plan(params, kEntryGreedy, &pl);
  if (s != SV_OK) return s;
  s = check_common(pl, target_logits, draft_tokens, out_tokens, num_accepted, workspace, workspace_bytes);
  if (s != SV_OK) return s;
  if (target_argmax && !aligned(target_argmax, 4)) return SV_ERR_INVALID_ARG;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  if (pl.dtype == SV_F32)
    return verify_greedy<float>(pl, target_logits, draft_tokens, out_tokens, num_accepted, target_argmax, ws, st);
  return verify_greedy<uint16_t>(pl, target_logits, draft_tokens, out_tokens, num_accepted, target_argmax, ws, st);
}

size_t sv_workspace_bytes_batch(const sv_params* params, const sv_sampling* sampling) {
  Plan pl;
  if (make_batch_plan(params, sampling, &pl) != SV_OK) return 0;
  return pl.total;
}

sv_status spec_verify_batch(const sv_params* params, const sv_sampling* sampling, const sv_layout* layout,
                            const void* target_logits, const void* draft, const int32_t* draft_tokens,
                            const sv_outputs* outputs, void* workspace, size_t workspace_bytes, void* stream) {
  Plan pl;
  sv_status s = make_batch_plan(params, sampling, &pl);
  if (s != SV_OK) return s;
  if (!outputs) return SV_ERR_INVALID_ARG;
  const sv_outputs o = *outputs;
  // A ragged call whose every draft length is 0 has no draft tokens or rows
  // to pass; their pointers may then be null (the classify pass checks that
  // the offsets end at 0).
  const bool ragged = layout && layout->cu_draft;
  s = check_common(pl, target_logits, draft_tokens, o.out_tokens, o.num_accepted, workspace, workspace_bytes, ragged);
  if (s != SV_OK) return s;
  int kind = draft ? SV_DRAFT_LOGITS : SV_DRAFT_ONEHOT;
  if (layout) {
    kind = layout->draft_kind;
    if (kind != SV_DRAFT_LOGITS && kind != SV_DRAFT_ONEHOT && kind != SV_DRAFT_PROBS && kind != SV_DRAFT_MATCH)
      return SV_ERR_INVALID_ARG;
    if ((kind == SV_DRAFT_LOGITS || kind == SV_DRAFT_PROBS) && !draft && !ragged) return SV_ERR_INVALID_ARG;
    if (layout->parents && (kind != SV_DRAFT_MATCH || !aligned(layout->parents, 4))) return SV_ERR_INVALID_ARG;
    const int64_t ts = layout->target_stride ? layout->target_stride : pl.V;
    const int64_t ds = layout->draft_stride ? layout->draft_stride : pl.V;
    if (ts < pl.V || ds < pl.V) return SV_ERR_INVALID_ARG;
    pl.L = sv::Layout{layout->cu_draft, ts, ds};
    if (layout->cu_draft && !aligned(layout->cu_draft, 4)) return SV_ERR_INVALID_ARG;
  }
  if (kind == SV_DRAFT_LOGITS && !aligned(draft, (size_t)pl.esize)) return SV_ERR_DTYPE;
  if (kind == SV_DRAFT_PROBS && !aligned(draft, 4)) return SV_ERR_INVALID_ARG;
  if (sampling && ((sampling->temperature && !aligned(sampling->temperature, 4)) ||
                   (sampling->top_k && !aligned(sampling->top_k, 4)) || (sampling->top_p && !aligned(sampling->top_p, 4))))
    return SV_ERR_INVALID_ARG;
  if ((o.p_draft && !aligned(o.p_draft, 4)) || (o.q_draft && !aligned(o.q_draft, 4)) ||
      (o.beta && !aligned(o.beta, 4)) || (o.counters && !aligned(o.counters, 8)))
    return SV_ERR_INVALID_ARG;
  BatchArgs ba;
  ba.T = sampling ? sampling->temperature : nullptr;
  ba.K = sampling ? sampling->top_k : nullptr;
  ba.P = sampling ? sampling->top_p : nullptr;
  ba.T0 = params->temperature;
  ba.K0 = params->top_k;
  ba.max_top_k = batch_max_top_k(params, sampling);
  ba.parents = layout ? layout->parents : nullptr;
  ba.no_drafts = !draft_tokens || ((kind == SV_DRAFT_LOGITS || kind == SV_DRAFT_PROBS) && !draft);
  if (o.path_nodes && !aligned(o.path_nodes, 4)) return SV_ERR_INVALID_ARG;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const uint64_t seed = params->seed;
  const void* d = (kind == SV_DRAFT_ONEHOT || kind == SV_DRAFT_MATCH) ? nullptr : draft;
  if (kind == SV_DRAFT_MATCH) {
    if (pl.dtype == SV_F32) return verify_batch<float, 3>(pl, ba, seed, target_logits, nullptr, draft_tokens, o, ws, st);
    return verify_batch<uint16_t, 3>(pl, ba, seed, target_logits, nullptr, draft_tokens, o, ws, st);
  }
  if (pl.dtype == SV_F32) {
    if (kind == SV_DRAFT_LOGITS)
      return verify_batch<float, 0>(pl, ba, seed, target_logits, d, draft_tokens, o, ws, st);
    if (kind == SV_DRAFT_PROBS)
      return verify_batch<float, 2>(pl, ba, seed, target_logits, d, draft_tokens, o, ws, st);
    return verify_batch<float, 1>(pl, ba, seed, target_logits, nullptr, draft_tokens, o, ws, st);
  }
  if (kind == SV_DRAFT_LOGITS)
    return verify_batch<uint16_t, 0>(pl, ba, seed, target_logits, d, draft_tokens, o, ws, st);
  if (kind == SV_DRAFT_PROBS)
    return verify_batch<uint16_t, 2>(pl, ba, seed, target_logits, d, draft_tokens, o, ws, st);
  return verify_batch<uint16_t, 1>(pl, ba, seed, target_logits, nullptr, draft_tokens, o, ws, st);
}

sv_status sv_read_device_error(const void* workspace, int32_t* host_code, void* stream) {
  if (!workspace || !host_code) return SV_ERR_INVALID_ARG;
  hipStream_t st = (hipStream_t)stream;
  if (hipStreamSynchronize(st) != hipSuccess) return SV_ERR_HIP;
  if (hipMemcpy(host_code, workspace, sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess) return SV_ERR_HIP;
  return SV_OK;
}

sv_status sv_kernel_timing_enable(int enable) {
  g_timing = enable != 0;
  return SV_OK;
}

sv_status sv_kernel_timing_reset(void) {
  for (int f = 0; f < kFamilies; ++f) g_used[f] = 0;
  return SV_OK;
}

sv_status sv_kernel_timing_read(int family, double* total_ms, int64_t* launches) {
  if (family < 0 || family >= kFamilies || !total_ms || !launches) return SV_ERR_INVALID_ARG;
  double tot = 0.0;
  for (size_t i = 0; i < g_used[family]; ++i) {
    const auto& ev = g_events[family][i];
    if (hipEventSynchronize(ev.second) != hipSuccess) return SV_ERR_HIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, ev.first, ev.second) != hipSuccess) return SV_ERR_HIP;
    tot += ms;
  }
  *total_ms = tot;
  *launches = (int64_t)g_used[family];
  return SV_OK;
}

sv_status sv_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes < 16 || bytes % 16 || !aligned(buf, 16) || !aligned(sink, 4)) return SV_ERR_INVALID_ARG;
  const int64_t nvec = (int64_t)(bytes / 16);
  const int64_t chunk = 32768;  // 512 KB per workgroup, the size of a headline logit row
  const int64_t nblk = (nvec + chunk - 1) / chunk;
  if (nblk > INT32_MAX) return SV_ERR_INVALID_ARG;
  hipLaunchKernelGGL(sv::stream_read_kernel<8>, dim3((unsigned)nblk), dim3(256), 0, (hipStream_t)stream,
                     (const uint4*)buf, nvec, chunk, sink);
  return check_launch();
}

}  // extern "C"
