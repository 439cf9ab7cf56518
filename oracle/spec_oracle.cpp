// Plain fp64 CPU oracle for the speculative-sampling verifier.
//
// TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
// load or call this file.  It is used by the test suite, by the smoke check
// and by the CPU-baseline leg of the benchmark, and by nothing else.  It
// shares no code, header, table or constant with the GPU library: it carries
// its own Philox4x32-10 and its own decoding of the logit formats.
//
// Sources (the reference pages; titles as printed):
//   [P1] "초안 모델로 생성 속도를 높이는 추측 디코딩" (cortexys.team),
//        section "방법" (Algorithm 1 of Leviathan et al.) and section
//        "수락률 α와 기대 속도 향상" (Eq. 1).
//   [P3] "투기적 디코딩" (mlxcel.ai manual), sections "기본 라운드" and
//        "정확성 기준".
//   [P4] "vLLM speculative decoding이 기각 토큰을 다시 뽑는 이유" (velog),
//        sections "드래프트가 제안하고 타깃이 판정한다" (the per-position test),
//        "왜 하필 max(p − q, 0)인가" (the residual, Appendix A.1),
//        "vLLM 커널은 이 규칙을 어떻게 옮겼나" (fp64 uniforms, the Exp(1)
//        race, sampling constraints), "기본값 greedy 드래프트에서도 분포가
//        지켜질까" (one-hot q and the greedy kernel).
//
// Readings where the pages are silent (each is listed with its reason in the
// design notes of the repository):
//   * temperature, then top-k, then top-p, the same settings for p and q;
//   * top-k keeps exactly k tokens ranked by (logit desc, index asc);
//   * top-p keeps the shortest prefix of the law left by top-k, in the same
//     order, whose probability reaches top_p (at least one token), and
//     renormalises over it;
//   * a request with temperature 0 takes the greedy rule, and its p(x_j) is
//     the temperature-0 law (1 on the target argmax, else 0) with q(x_j) = 1;
//   * a draft given as probabilities (vLLM's draft_probs) is q as given: no
//     temperature, top-k, top-p or renormalisation is applied to it;
//   * a request with g draft positions (0 <= g <= gamma) uses target rows
//     0..g and positions 0..g-1; its uniforms are those of the same (b, j);
//   * sampler-match ([P3] "mlxcel의 프롬프트 조회"): every node of the draft
//     (a chain, or a tree given by parent indices) gets a fresh sample from
//     its row's adjusted law, drawn by the same Exp(1) race over the whole
//     law as the recovered and bonus draws, on the race stream of (b, node);
//     from the root, the walk follows the child whose token equals
//     the sample (the lowest-indexed child if several do) and emits the
//     sample where no child matches.
//   * every argmax and every race tie goes to the lowest index;
//   * uniforms are Philox4x32-10 words mapped to (k53 + 1) * 2^-53 in (0, 1];
//     accept stream counter (0, j, b, 0), race stream counter
//     (y >> 1, j, b, 1) with words (0,1) for even y and (2,3) for odd y;
//   * accept iff q(x) > 0 and u <= p(x)/q(x) (equality accepts);
//   * Exp(1) variate E = -ln(u); E == 0 gives an infinite race score;
//   * a residual of zero total mass falls back to w = p;
//   * an out-of-range draft token counts as rejected and raises a flag.
//
// Decision margins (diagnostics; they decide which results a comparison may
// exempt as near ties, [P3] "정확성 기준": a different reduction order can
// flip near-equal tokens): accept_margin, race_margin and nucleus_margin
// below, each pinned on hand-computed values.
//
// Parity unpinned by the pages: the tie rules at exact equality (race ties,
// accept at u == p/q) are events of probability ~2^-53 that no sampling test
// can observe; they are this oracle's definition only.  The Philox keying and
// bit mapping are pinned against themselves only through the documented
// counter layout.
//
// Every loop is the definition written out, in fp64, in ascending index
// order.  No blocking, no fusion, no reordering.  Requests are independent, so
// the batch loop is an OpenMP parallel-for over requests; nothing inside a
// request is parallel.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <numeric>
#include <vector>

#ifdef _OPENMP
#include <omp.h>
#endif

namespace {

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy
// as 1, 2, 3", SC'11).  One round maps counter (c0,c1,c2,c3) under key
// (k0,k1) to (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1, lo(M0*c0));
// the key is bumped by the Weyl constants before every round after the first.
// ---------------------------------------------------------------------------
const uint32_t kPhiloxM0 = 0xD2511F53u;
const uint32_t kPhiloxM1 = 0xCD9E8D57u;
const uint32_t kPhiloxW0 = 0x9E3779B9u;
const uint32_t kPhiloxW1 = 0xBB67AE85u;

void philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
  uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
  uint32_t k0 = key_in[0], k1 = key_in[1];
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += kPhiloxW0;
      k1 += kPhiloxW1;
    }
    uint64_t prod0 = (uint64_t)kPhiloxM0 * (uint64_t)c0;
    uint64_t prod1 = (uint64_t)kPhiloxM1 * (uint64_t)c2;
    uint32_t hi0 = (uint32_t)(prod0 >> 32), lo0 = (uint32_t)prod0;
    uint32_t hi1 = (uint32_t)(prod1 >> 32), lo1 = (uint32_t)prod1;
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n1 = lo1;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    uint32_t n3 = lo0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

// Two 32-bit words -> a double in (0, 1]: the top 53 bits of (hi:lo), plus
// one, times 2^-53.  Exact in fp64; never 0, which the page on vLLM's kernel
// gives as the reason for drawing the uniform in float64.
double words_to_unit(uint32_t lo, uint32_t hi) {
  uint64_t bits = ((uint64_t)hi << 32) | (uint64_t)lo;
  uint64_t k53 = bits >> 11;
  return (double)(k53 + 1) * std::ldexp(1.0, -53);
}

double uniform_accept(uint64_t seed, uint32_t b, uint32_t j) {
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t ctr[4] = {0u, j, b, 0u};
  uint32_t w[4];
  philox4x32_10(ctr, key, w);
  return words_to_unit(w[0], w[1]);
}

double uniform_race(uint64_t seed, uint32_t b, uint32_t j, uint32_t y) {
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t ctr[4] = {y >> 1, j, b, 1u};
  uint32_t w[4];
  philox4x32_10(ctr, key, w);
  if ((y & 1u) == 0u) return words_to_unit(w[0], w[1]);
  return words_to_unit(w[2], w[3]);
}

// ---------------------------------------------------------------------------
// Logit decoding.  dtype 0: IEEE binary32.  dtype 1: bfloat16, i.e. the upper
// 16 bits of a binary32.  Both embed exactly in fp64.
// ---------------------------------------------------------------------------
double decode_logit(const void* row, int dtype, int64_t y) {
  if (dtype == 0) {
    float f;
    std::memcpy(&f, (const char*)row + 4 * y, 4);
    return (double)f;
  }
  uint16_t h;
  std::memcpy(&h, (const char*)row + 2 * y, 2);
  uint32_t bits = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &bits, 4);
  return (double)f;
}

size_t elem_bytes(int dtype) { return dtype == 0 ? 4 : 2; }

// ---------------------------------------------------------------------------
// Decision margins.  Each is the relative (or, for the nucleus, absolute
// probability) distance of a decision from its boundary; 1 where no decision
// could flip.
// ---------------------------------------------------------------------------

// The accept test u <= p(x) / q(x), written u q(x) <= p(x): relative gap
// |u q - p| / max(u q, p).  An invalid token or q(x) = 0 rejects whatever u
// is (no boundary); p = u q = 0 cannot occur since u > 0 and q > 0 there.
double accept_margin(double u, double px, double qx, bool valid) {
  if (!valid || !(qx > 0.0)) return 1.0;
  const double lhs = u * qx, rhs = px;
  const double den = std::max(lhs, rhs);
  return den > 0.0 ? std::fabs(lhs - rhs) / den : 0.0;
}

// The race winner against the runner-up: (s1 - s2) / s1 for the two largest
// scores.  One candidate (s2 absent): 1.  An infinite winner (E = 0) is
// flipped only by another infinite score.
double race_margin(int ncand, double s1, double s2) {
  if (ncand < 2) return 1.0;
  if (std::isinf(s1)) return std::isinf(s2) ? 0.0 : 1.0;
  return (s1 - s2) / s1;
}

// The nucleus stops at the s-th kept token (rank order) because the running
// mass C_s reaches top_p while C_(s-1) did not: the decision has the two
// sides C_s - top_p and top_p - C_(s-1).  At s = 1 only the first exists (at
// least one token is always kept, so nothing is decided below it).
double nucleus_margin(int s, double C, double Cprev, double top_p) {
  if (s <= 1) return C - top_p;
  return std::min(C - top_p, top_p - Cprev);
}

// The adjusted distribution of one position: temperature, then top-k, then
// top-p, then softmax ([P4] "vLLM 커널은 이 규칙을 어떻게 옮겼나": the sampling
// constraints are applied to the logits before the test, so p is the adjusted
// law; the page lists them as temperature, top_k, top_p).  top_p >= 1 is off.
// *cut_margin (if not NULL) receives nucleus_margin of the stop, or 1 when
// top-p is off.
std::vector<double> row_probs(const void* row, int dtype, int V, double T, int top_k, double top_p = 1.0,
                              double* cut_margin = nullptr) {
  std::vector<double> l(V);
  for (int y = 0; y < V; ++y) l[y] = decode_logit(row, dtype, y);

  // Rank by (logit desc, index asc): a stable sort on descending logit keeps
  // equal logits in ascending index order.  Ranking on l equals ranking on
  // l / T for T > 0.
  std::vector<int> order(V);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int a, int c) { return l[a] > l[c]; });

  std::vector<char> keep(V, 1);
  if (top_k > 0 && top_k < V) {
    std::fill(keep.begin(), keep.end(), 0);
    for (int r = 0; r < top_k; ++r) keep[order[r]] = 1;
  }

  std::vector<double> z(V, 0.0);
  double m = -std::numeric_limits<double>::infinity();
  for (int y = 0; y < V; ++y) {
    if (!keep[y]) continue;
    z[y] = l[y] / T;
    if (z[y] > m) m = z[y];
  }
  double Z = 0.0;
  for (int y = 0; y < V; ++y)
    if (keep[y]) Z += std::exp(z[y] - m);
  std::vector<double> p(V, 0.0);
  for (int y = 0; y < V; ++y)
    if (keep[y]) p[y] = std::exp(z[y] - m) / Z;
  if (cut_margin) *cut_margin = 1.0;
  if (!(top_p < 1.0)) return p;

  // Nucleus: walk the kept tokens in rank order, adding their probability
  // under the top-k law, and stop at the first token where the running mass
  // reaches top_p.
  double C = 0.0, Cprev = 0.0;
  int s = 0;
  for (int r = 0; r < V; ++r) {
    const int y = order[r];
    if (!keep[y]) continue;
    Cprev = C;
    C += p[y];
    ++s;
    if (C >= top_p) break;
  }
  if (cut_margin) *cut_margin = nucleus_margin(s, C, Cprev, top_p);
  std::vector<char> nucleus(V, 0);
  for (int r = 0, taken = 0; r < V && taken < s; ++r) {
    const int y = order[r];
    if (!keep[y]) continue;
    nucleus[y] = 1;
    ++taken;
  }
  double Zn = 0.0;
  for (int y = 0; y < V; ++y)
    if (nucleus[y]) Zn += std::exp(z[y] - m);
  for (int y = 0; y < V; ++y) p[y] = nucleus[y] ? std::exp(z[y] - m) / Zn : 0.0;
  return p;
}

// Greedy target token: the lowest index attaining the maximum raw logit.
int row_argmax(const void* row, int dtype, int V) {
  int best = 0;
  double bv = decode_logit(row, dtype, 0);
  for (int y = 1; y < V; ++y) {
    double v = decode_logit(row, dtype, y);
    if (v > bv) { bv = v; best = y; }
  }
  return best;
}

// Exp(1) race ([P4] "vLLM 커널은 이 규칙을 어떻게 옮겼나"): the argmax over
// tokens with w_y > 0 of w_y / E_y, E_y = -ln u_y i.i.d. Exp(1), is a sample
// from w / sum(w) with no normalisation.  Strict '>' keeps the lowest index on
// ties.  *margin receives (s1 - s2) / s1 for the top two scores.
int race(const std::vector<double>& w, uint64_t seed, uint32_t b, uint32_t j, double* margin) {
  const double inf = std::numeric_limits<double>::infinity();
  int best = -1, ncand = 0;
  double s1 = -inf, s2 = -inf;
  for (size_t y = 0; y < w.size(); ++y) {
    if (!(w[y] > 0.0)) continue;
    ++ncand;
    double u = uniform_race(seed, b, j, (uint32_t)y);
    double E = -std::log(u);
    double s = (E == 0.0) ? inf : w[y] / E;
    if (s > s1) {
      s2 = s1;
      s1 = s;
      best = (int)y;
    } else if (s > s2) {
      s2 = s;
    }
  }
  if (margin) *margin = race_margin(ncand, s1, s2);
  return best;
}

enum { MODE_PROB = 0, MODE_ONEHOT = 1, MODE_GREEDY = 2, MODE_NAIVE = 3, MODE_PROBS = 4 };

struct Problem {
  int mode, B, G, V, dtype, top_k;
  double T;
  uint64_t seed;
  double top_p = 1.0;
};

// One request: Algorithm 1's verification part ([P1] "방법"; [P4]
// "드래프트가 제안하고 타깃이 판정한다").  Positions j = 0..G-1 carry draft
// tokens; row G of the target is the bonus position.  Returns 1 if a draft
// token was out of range, else 0.
int verify_one(const Problem& P, uint32_t b, const char* Lt, const char* Ld, const float* Qp, const int32_t* X,
               int32_t* out, int32_t* n_out, double* p_draft, double* q_draft, int32_t* target_argmax,
               double* beta, double* acc_margin, double* race_margin, double* cut_margin = nullptr) {
  const int G = P.G, V = P.V;
  const size_t row_bytes = (size_t)V * elem_bytes(P.dtype);
  const double nan = std::numeric_limits<double>::quiet_NaN();
  int bad_token = 0;
  std::vector<char> valid(G);
  for (int j = 0; j < G; ++j) {
    valid[j] = (X[j] >= 0 && X[j] < V);
    if (!valid[j]) bad_token = 1;
  }
  if (acc_margin)
    for (int j = 0; j < G; ++j) acc_margin[j] = nan;
  if (race_margin) *race_margin = nan;
  if (cut_margin) *cut_margin = 1.0;

  if (P.mode == MODE_GREEDY) {
    // Temperature 0: accept iff the draft token is the target argmax ([P1]
    // "방법"; [P4] "기본값 greedy 드래프트에서도 분포가 지켜질까"); the target
    // argmax replaces the first mismatch, and is the bonus after G matches.
    std::vector<int> a(G + 1);
    for (int j = 0; j <= G; ++j) a[j] = row_argmax(Lt + (size_t)j * row_bytes, P.dtype, V);
    int n = G;
    for (int j = 0; j < G; ++j) {
      if (!valid[j] || X[j] != a[j]) { n = j; break; }
    }
    for (int j = 0; j < n; ++j) out[j] = X[j];
    out[n] = a[n];
    for (int j = n + 1; j <= G; ++j) out[j] = -1;
    *n_out = n;
    if (target_argmax)
      for (int j = 0; j <= G; ++j) target_argmax[j] = a[j];
    return bad_token;
  }

  const bool has_q = (P.mode == MODE_PROB || P.mode == MODE_NAIVE || P.mode == MODE_PROBS);
  std::vector<std::vector<double>> p(G + 1), q(has_q ? G : 0);
  double cm = 1.0, cmj = 1.0;
  for (int j = 0; j <= G; ++j) {
    p[j] = row_probs(Lt + (size_t)j * row_bytes, P.dtype, V, P.T, P.top_k, P.top_p, &cmj);
    cm = std::min(cm, cmj);
  }
  for (int j = 0; j < (has_q ? G : 0); ++j) {
    if (P.mode == MODE_PROBS) {
      // The drafter's probabilities, as given.
      q[j].assign(V, 0.0);
      for (int y = 0; y < V; ++y) q[j][y] = (double)Qp[(size_t)j * V + y];
      continue;
    }
    q[j] = row_probs(Ld + (size_t)j * row_bytes, P.dtype, V, P.T, P.top_k, P.top_p, &cmj);
    cm = std::min(cm, cmj);
  }
  if (cut_margin) *cut_margin = cm;

  // p(x_j) and q(x_j) for every draft position (q := 1 for a one-hot draft).
  std::vector<double> px(G), qx(G);
  for (int j = 0; j < G; ++j) {
    px[j] = valid[j] ? p[j][X[j]] : 0.0;
    if (has_q) qx[j] = valid[j] ? q[j][X[j]] : 0.0;
    else qx[j] = valid[j] ? 1.0 : 0.0;
    if (p_draft) p_draft[j] = px[j];
    if (q_draft) q_draft[j] = qx[j];
    if (beta) {
      // Acceptance rate of position j: sum_y min(p, q) ([P4] "왜 하필
      // max(p − q, 0)인가", Theorem 3.5).  For one-hot q it is p(x).
      if (has_q) {
        double s = 0.0;
        for (int y = 0; y < V; ++y) s += std::min(p[j][y], q[j][y]);
        beta[j] = s;
      } else {
        beta[j] = px[j];
      }
    }
  }

  // Front-to-back test with one independent uniform per position; the first
  // rejection ends the scan ([P4] "드래프트가 제안하고 타깃이 판정한다").
  int n = G;
  for (int j = 0; j < G; ++j) {
    double u = uniform_accept(P.seed, b, (uint32_t)j);
    bool accept;
    if (!valid[j]) {
      accept = false;
    } else if (has_q) {
      accept = (qx[j] > 0.0) && (u <= px[j] / qx[j]);
    } else {
      accept = (u <= px[j]);
    }
    if (acc_margin) acc_margin[j] = accept_margin(u, px[j], qx[j], valid[j]);
    if (!accept) { n = j; break; }
  }

  std::vector<double> w(V, 0.0);
  if (n < G) {
    if (P.mode == MODE_PROB || P.mode == MODE_PROBS) {
      // Residual norm(max(0, p - q)) ([P4] "왜 하필 max(p − q, 0)인가").
      double mass = 0.0;
      for (int y = 0; y < V; ++y) {
        w[y] = std::max(p[n][y] - q[n][y], 0.0);
        mass += w[y];
      }
      // Zero mass needs p = q at row n: reached when an out-of-range draft
      // token forces the rejection of a position whose two laws agree.
      if (!(mass > 0.0)) w = p[n];
    } else if (P.mode == MODE_ONEHOT) {
      // One-hot q: the residual is p with the draft token masked ([P4]
      // "기본값 greedy 드래프트에서도 분포가 지켜질까").
      w = p[n];
      if (valid[n]) w[X[n]] = 0.0;
      double mass = 0.0;
      for (int y = 0; y < V; ++y) mass += w[y];
      if (!(mass > 0.0)) w = p[n];  // unreachable: p(x) = 1 always accepts
    } else {
      // MODE_NAIVE, test-only: resample from p after a rejection, the wrong
      // rule that [P4] "Java로 규칙을 재현해 본 결과" shows to double count.
      w = p[n];
    }
  } else {
    // All G accepted: one more token from p at the bonus position.
    w = p[G];
  }
  int tok = race(w, P.seed, b, (uint32_t)n, race_margin);

  for (int j = 0; j < n; ++j) out[j] = X[j];
  out[n] = tok;
  for (int j = n + 1; j <= G; ++j) out[j] = -1;
  *n_out = n;
  return bad_token;
}

// Sampler-match verification of one request ([P3] "mlxcel의 프롬프트 조회":
// a proposal is accepted only if it equals the token the target's sampler
// draws at that position; lossless for one-hot proposals).  Nodes 0..g: node
// 0 is the root (the last context token), node i >= 1 carries the draft
// token X[i-1] and has parent par[i-1] in 0..i-1 (NULL: i-1, a chain).  Row
// i of Lt is the target's law after node i's path.  Outputs: out[0..d] the
// d accepted tokens and the sample that ends the walk, *n_out = d, nodes[k]
// the k-th accepted node; p_draft[i-1] = p_parent(X[i-1]), the probability
// that node i is accepted once its parent is reached.  Returns 1 if a draft
// token is out of range.
int verify_match(const Problem& P, uint32_t b, const char* Lt, const int32_t* X, const int32_t* par, int32_t* out,
                 int32_t* n_out, int32_t* nodes, double* p_draft, double* race_margin, double* cut_margin) {
  const int g = P.G, V = P.V;
  const size_t row_bytes = (size_t)V * elem_bytes(P.dtype);
  int bad = 0;
  std::vector<std::vector<double>> p(g + 1);
  std::vector<int> s(g + 1);
  std::vector<double> margin(g + 1, 1.0);  // each node's race margin
  double cm = 1.0;
  for (int i = 0; i <= g; ++i) {
    const char* row = Lt + (size_t)i * row_bytes;
    if (P.mode == MODE_GREEDY) {
      s[i] = row_argmax(row, P.dtype, V);  // the temperature-0 sampler
    } else {
      double c = 1.0;
      p[i] = row_probs(row, P.dtype, V, P.T, P.top_k, P.top_p, &c);
      cm = std::min(cm, c);
      // A fresh draw from the node's law: the Exp(1) race over its tokens
      // on the race stream of (b, node), as for a recovered or bonus token.
      s[i] = race(p[i], P.seed, b, (uint32_t)i, &margin[i]);
    }
  }
  for (int i = 1; i <= g; ++i) {
    const int x = X[i - 1];
    const int pa = par ? par[i - 1] : i - 1;
    const bool valid = x >= 0 && x < V;
    if (!valid) bad = 1;
    if (p_draft) {
      if (P.mode == MODE_GREEDY) p_draft[i - 1] = (valid && x == s[pa]) ? 1.0 : 0.0;
      else p_draft[i - 1] = valid ? p[pa][x] : 0.0;
    }
  }
  int cur = 0, d = 0;
  double rm = 1.0;  // over the nodes the walk visits: only their samples are used
  for (;;) {
    const int t = s[cur];
    rm = std::min(rm, margin[cur]);
    int child = -1;
    for (int i = 1; i <= g; ++i) {
      const int pa = par ? par[i - 1] : i - 1;
      if (pa == cur && X[i - 1] == t) {
        child = i;
        break;
      }
    }
    out[d] = t;
    if (child < 0) break;
    if (nodes) nodes[d] = child;
    ++d;
    cur = child;
  }
  *n_out = d;
  if (race_margin) *race_margin = rm;
  if (cut_margin) *cut_margin = cm;
  return bad;
}

}  // namespace

extern "C" {

// Philox4x32-10 on one counter block.
void sv_ref_philox4x32_10(const uint32_t* ctr4, const uint32_t* key2, uint32_t* out4) {
  philox4x32_10(ctr4, key2, out4);
}

double sv_ref_uniform_accept(uint64_t seed, uint32_t b, uint32_t j) { return uniform_accept(seed, b, j); }

double sv_ref_uniform_race(uint64_t seed, uint32_t b, uint32_t j, uint32_t y) {
  return uniform_race(seed, b, j, y);
}

// Adjusted distribution of one row (length V) into p_out.  Returns 0.
int sv_ref_row_probs(const void* row, int dtype, int V, double T, int top_k, double* p_out) {
  std::vector<double> p = row_probs(row, dtype, V, T, top_k);
  std::copy(p.begin(), p.end(), p_out);
  return 0;
}

// Adjusted distribution with top-p (top_p >= 1: off); *cut_margin as in
// row_probs.  Returns 0.
int sv_ref_row_probs_p(const void* row, int dtype, int V, double T, int top_k, double top_p, double* p_out,
                       double* cut_margin) {
  std::vector<double> p = row_probs(row, dtype, V, T, top_k, top_p, cut_margin);
  std::copy(p.begin(), p.end(), p_out);
  return 0;
}

int sv_ref_row_argmax(const void* row, int dtype, int V) { return row_argmax(row, dtype, V); }

// Exp(1) race over weights w[0..V) on the race stream of (seed, b, j).
int sv_ref_race(const double* w, int V, uint64_t seed, uint32_t b, uint32_t j, double* margin) {
  std::vector<double> wv(w, w + V);
  return race(wv, seed, b, j, margin);
}

// The decision margins, for pinning.
double sv_ref_accept_margin(double u, double px, double qx, int valid) { return accept_margin(u, px, qx, valid != 0); }
double sv_ref_race_margin(int ncand, double s1, double s2) { return race_margin(ncand, s1, s2); }
double sv_ref_nucleus_margin(int s, double C, double Cprev, double top_p) { return nucleus_margin(s, C, Cprev, top_p); }

// Batched verifier.
//   mode: 0 prob, 1 onehot, 2 greedy, 3 naive (test-only, deliberately wrong)
//   Lt: [nreq][G+1][V] logits; Ld: [nreq][G][V] (prob and naive only)
//   X: [nreq][G] int32 draft tokens
//   req_ids: request index b of each request for the Philox streams
//            (NULL: b = 0..nreq-1)
//   outputs: out_tokens [nreq][G+1], num_accepted [nreq];
//   optional (NULL to skip): p_draft, q_draft [nreq][G]; target_argmax
//   [nreq][G+1] (greedy); beta, acc_margin [nreq][G]; race_margin [nreq];
//   bad_token [nreq] (1 where a draft token is out of range).
// Returns 0 on success, -1 on invalid arguments.
int sv_ref_verify(int mode, int nreq, int G, int V, int dtype, double T, int top_k, uint64_t seed,
                  const void* Lt, const void* Ld, const int32_t* X, const int32_t* req_ids,
                  int32_t* out_tokens, int32_t* num_accepted, double* p_draft, double* q_draft,
                  int32_t* target_argmax, double* beta, double* acc_margin, double* race_margin,
                  int32_t* bad_token, int nthreads) {
  if (nreq < 0 || G < 1 || V < 1 || (dtype != 0 && dtype != 1) || mode < 0 || mode > 3) return -1;
  if (mode != MODE_GREEDY && !(T > 0.0)) return -1;
  if (top_k < 0) return -1;
  if (!Lt || !X || !out_tokens || !num_accepted) return -1;
  if ((mode == MODE_PROB || mode == MODE_NAIVE) && !Ld) return -1;
  Problem P{mode, nreq, G, V, dtype, top_k, T, seed};
  const size_t row_bytes = (size_t)V * elem_bytes(dtype);
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int r = 0; r < nreq; ++r) {
    uint32_t b = req_ids ? (uint32_t)req_ids[r] : (uint32_t)r;
    const char* lt = (const char*)Lt + (size_t)r * (G + 1) * row_bytes;
    const char* ld = Ld ? (const char*)Ld + (size_t)r * G * row_bytes : nullptr;
    int bad = verify_one(P, b, lt, ld, nullptr, X + (size_t)r * G, out_tokens + (size_t)r * (G + 1), num_accepted + r,
                         p_draft ? p_draft + (size_t)r * G : nullptr, q_draft ? q_draft + (size_t)r * G : nullptr,
                         target_argmax ? target_argmax + (size_t)r * (G + 1) : nullptr,
                         beta ? beta + (size_t)r * G : nullptr, acc_margin ? acc_margin + (size_t)r * G : nullptr,
                         race_margin ? race_margin + r : nullptr);
    if (bad_token) bad_token[r] = bad;
  }
  return 0;
}

// Batched verifier with per-request settings and ragged draft lengths.
//   draft_kind: 0 draft logits (Ld, rows like Lt), 1 one-hot drafts (Ld
//   unused), 2 draft probabilities (Qp: fp32 rows, q as given), 3 token-only
//   drafts verified by sampler-match (parents: [sum g_r] parent node of each
//   draft node, in 0..i-1, packed like the tokens; NULL: chains; path_nodes
//   [nreq][G+1]: accepted nodes in order, -1 after; a request whose parents
//   break that rule emits nothing and gets bad_param).
//   lengths[r]: draft positions of request r, 0..G (NULL: all G).  Rows are
//   packed request after request: request r's g_r + 1 target rows start at
//   row sum_{r' < r} (g_r' + 1), its g_r draft rows (logits or
//   probabilities), draft tokens and p_draft / q_draft / beta / acc_margin
//   entries at sum_{r' < r} g_r'.  out_tokens is [nreq][G+1], -1 after the
//   emitted token.
//   T[r]: temperature, 0 = greedy request; K[r]: top-k (0 or >= V: off);
//   P[r]: top-p in (0, 1], 1 = off; all three as the caller's fp32 / int32.
//   max_top_k: a top_k in (max_top_k, V) makes the request invalid.
//   An invalid request (T negative, NaN or infinite; top_k negative or above
//   max_top_k and below V; top_p NaN, <= 0 or > 1) emits nothing: out_tokens
//   all -1, num_accepted 0, p_draft / q_draft / beta 0, bad_param 1.
//   Greedy requests: the argmax rule; p_draft[j] = 1 if x_j is the target
//   argmax of row j else 0, q_draft[j] = 1.
//   cut_margin [nreq]: the smallest top-p boundary margin over the request's
//   rows (1 without top-p).  Other arguments as sv_ref_verify.
int sv_ref_verify_ex(int draft_kind, int nreq, int G, int V, int dtype, const float* T, const int32_t* K,
                     const float* Pp, int max_top_k, uint64_t seed, const void* Lt, const void* Ld, const float* Qp,
                     const int32_t* X, const int32_t* lengths, const int32_t* req_ids, int32_t* out_tokens,
                     int32_t* num_accepted, double* p_draft, double* q_draft, double* beta, double* acc_margin,
                     double* race_margin, double* cut_margin, int32_t* bad_token, int32_t* bad_param,
                     const int32_t* parents, int32_t* path_nodes, int nthreads) {
  if (nreq < 0 || G < 0 || V < 1 || (dtype != 0 && dtype != 1) || draft_kind < 0 || draft_kind > 3) return -1;
  if (!Lt || !X || !out_tokens || !num_accepted || !T || !K || !Pp) return -1;
  if (draft_kind == 0 && !Ld) return -1;
  if (draft_kind == 2 && !Qp) return -1;
  const int mode = draft_kind == 0 ? MODE_PROB : (draft_kind == 2 ? MODE_PROBS : MODE_ONEHOT);
  std::vector<size_t> d0(nreq + 1, 0);  // packed draft offset of each request
  for (int r = 0; r < nreq; ++r) {
    const int g = lengths ? lengths[r] : G;
    if (g < 0 || g > G) return -1;
    d0[r + 1] = d0[r] + (size_t)g;
  }
  const size_t row_bytes = (size_t)V * elem_bytes(dtype);
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int r = 0; r < nreq; ++r) {
    const uint32_t b = req_ids ? (uint32_t)req_ids[r] : (uint32_t)r;
    const int g = (int)(d0[r + 1] - d0[r]);
    const size_t t0 = d0[r] + (size_t)r;  // first target row
    const double t = (double)T[r], pp = (double)Pp[r];
    const int k = K[r];
    const bool ok = std::isfinite(t) && t >= 0.0 && k >= 0 && (k >= V || k <= max_top_k) && pp > 0.0 &&
                    pp <= 1.0;
    int32_t* o = out_tokens + (size_t)r * (G + 1);
    double* pd = p_draft ? p_draft + d0[r] : nullptr;
    double* qd = q_draft ? q_draft + d0[r] : nullptr;
    for (int j = 0; j <= G; ++j) o[j] = -1;
    if (bad_param) bad_param[r] = ok ? 0 : 1;
    if (cut_margin) cut_margin[r] = 1.0;
    if (race_margin) race_margin[r] = 1.0;
    if (acc_margin)
      for (int j = 0; j < g; ++j) acc_margin[d0[r] + j] = 1.0;
    if (!ok) {
      num_accepted[r] = 0;
      for (int j = 0; j < g; ++j) {
        if (pd) pd[j] = 0.0;
        if (qd) qd[j] = 0.0;
        if (beta) beta[d0[r] + j] = 0.0;
      }
      if (bad_token) bad_token[r] = 0;
      continue;
    }
    const char* lt = (const char*)Lt + t0 * row_bytes;
    const char* ld = (draft_kind == 0) ? (const char*)Ld + d0[r] * row_bytes : nullptr;
    const float* qp = (draft_kind == 2) ? Qp + d0[r] * (size_t)V : nullptr;
    const int32_t* x = X + d0[r];
    if (path_nodes)
      for (int j = 0; j <= G; ++j) path_nodes[(size_t)r * (G + 1) + j] = -1;
    if (draft_kind == 3) {
      // Sampler-match over a chain or a tree; q is one-hot (1 for a valid
      // draft token) and beta = p_draft.
      const int32_t* par = parents ? parents + d0[r] : nullptr;
      bool tree_ok = true;
      for (int i = 1; par && i <= g; ++i) tree_ok = tree_ok && par[i - 1] >= 0 && par[i - 1] < i;
      if (!tree_ok) {
        if (bad_param) bad_param[r] = 1;
        num_accepted[r] = 0;
        for (int j = 0; j < g; ++j) {
          if (pd) pd[j] = 0.0;
          if (qd) qd[j] = 0.0;
          if (beta) beta[d0[r] + j] = 0.0;
        }
        if (bad_token) bad_token[r] = 0;
        continue;
      }
      Problem P{t == 0.0 ? (int)MODE_GREEDY : (int)MODE_ONEHOT, nreq, g, V, dtype, k, t, seed, pp};
      int bad = verify_match(P, b, lt, x, par, o, num_accepted + r,
                             path_nodes ? path_nodes + (size_t)r * (G + 1) : nullptr, pd,
                             race_margin ? race_margin + r : nullptr, cut_margin ? cut_margin + r : nullptr);
      for (int j = 0; j < g; ++j) {
        if (qd) qd[j] = (x[j] >= 0 && x[j] < V) ? 1.0 : 0.0;
        if (beta) beta[d0[r] + j] = pd ? pd[j] : 0.0;
      }
      if (bad_token) bad_token[r] = bad;
      continue;
    }
    Problem P{t == 0.0 ? (int)MODE_GREEDY : mode, nreq, g, V, dtype, k, t, seed, pp};
    std::vector<int32_t> targ(g + 1);
    int bad = verify_one(P, b, lt, ld, qp, x, o, num_accepted + r, pd, qd, targ.data(),
                         beta ? beta + d0[r] : nullptr, acc_margin ? acc_margin + d0[r] : nullptr,
                         race_margin ? race_margin + r : nullptr, cut_margin ? cut_margin + r : nullptr);
    if (P.mode == MODE_GREEDY) {
      // The temperature-0 law is one-hot on the target argmax.
      for (int j = 0; j < g; ++j) {
        if (pd) pd[j] = (x[j] == targ[j]) ? 1.0 : 0.0;
        if (qd) qd[j] = 1.0;
        if (beta) beta[d0[r] + j] = (x[j] == targ[j]) ? 1.0 : 0.0;
      }
    }
    if (bad_token) bad_token[r] = bad;
  }
  return 0;
}

// Number of threads the OpenMP runtime will use for the batch loop.
int sv_ref_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

}  // extern "C"
