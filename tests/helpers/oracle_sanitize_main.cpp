// Drives the fp64 oracle (oracle/spec_oracle.cpp, linked in) through its C
// entry points on small seeded inputs and edge cases, for a build with
// AddressSanitizer and UndefinedBehaviorSanitizer (test infrastructure; the
// test that builds and runs it is tests/test_oracle_sanitize.py).  Exits
// non-zero if an entry point rejects a valid call, accepts an invalid one, or
// returns an output outside its documented range.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <vector>

extern "C" {
void sv_ref_philox4x32_10(const uint32_t* ctr4, const uint32_t* key2, uint32_t* out4);
double sv_ref_uniform_accept(uint64_t seed, uint32_t b, uint32_t j);
double sv_ref_uniform_race(uint64_t seed, uint32_t b, uint32_t j, uint32_t y);
int sv_ref_row_probs_p(const void* row, int dtype, int V, double T, int top_k, double top_p, double* p_out,
                       double* cut_margin);
int sv_ref_row_argmax(const void* row, int dtype, int V);
int sv_ref_race(const double* w, int V, uint64_t seed, uint32_t b, uint32_t j, double* margin);
double sv_ref_accept_margin(double u, double px, double qx, int valid);
double sv_ref_race_margin(int ncand, double s1, double s2);
double sv_ref_nucleus_margin(int s, double C, double Cprev, double top_p);
int sv_ref_verify(int mode, int nreq, int G, int V, int dtype, double T, int top_k, uint64_t seed, const void* Lt,
                  const void* Ld, const int32_t* X, const int32_t* req_ids, int32_t* out_tokens,
                  int32_t* num_accepted, double* p_draft, double* q_draft, int32_t* target_argmax, double* beta,
                  double* acc_margin, double* race_margin, int32_t* bad_token, int nthreads);
int sv_ref_verify_ex(int draft_kind, int nreq, int G, int V, int dtype, const float* T, const int32_t* K,
                     const float* Pp, int max_top_k, uint64_t seed, const void* Lt, const void* Ld, const float* Qp,
                     const int32_t* X, const int32_t* lengths, const int32_t* req_ids, int32_t* out_tokens,
                     int32_t* num_accepted, double* p_draft, double* q_draft, double* beta, double* acc_margin,
                     double* race_margin, double* cut_margin, int32_t* bad_token, int32_t* bad_param,
                     const int32_t* parents, int32_t* path_nodes, int nthreads);
}

namespace {

int failures = 0;
#define CHECK(c)                                                  \
  do {                                                            \
    if (!(c)) {                                                   \
      std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
      ++failures;                                                 \
    }                                                             \
  } while (0)

// Input generator only (xorshift64*), no verifier arithmetic.
struct Gen {
  uint64_t s;
  uint32_t next() {
    s ^= s >> 12;
    s ^= s << 25;
    s ^= s >> 27;
    return (uint32_t)((s * 0x2545F4914F6CDD1Dull) >> 32);
  }
  float logit() { return ((float)(next() % 20001u) - 10000.f) * 6e-4f; }  // [-6, 6]
  int token(int V) { return (int)(next() % (uint32_t)V); }
};

uint16_t to_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

// Logits of n rows of V as fp32 or bf16 bytes; a few -inf entries.
std::vector<uint8_t> rows(Gen& g, int n, int V, int dtype) {
  std::vector<uint8_t> out((size_t)n * V * (dtype == 0 ? 4 : 2));
  for (size_t i = 0; i < (size_t)n * V; ++i) {
    float f = g.logit();
    if (g.next() % 17u == 0u && i % (size_t)V != 0) f = -std::numeric_limits<float>::infinity();
    if (dtype == 0) std::memcpy(&out[i * 4], &f, 4);
    else {
      const uint16_t h = to_bf16(f);
      std::memcpy(&out[i * 2], &h, 2);
    }
  }
  return out;
}

void check_tokens(const std::vector<int32_t>& out, const std::vector<int32_t>& n, int nreq, int G, int V,
                  const int32_t* lengths) {
  for (int r = 0; r < nreq; ++r) {
    const int g = lengths ? lengths[r] : G;
    CHECK(n[r] >= 0 && n[r] <= g);
    for (int j = 0; j <= G; ++j) {
      const int32_t t = out[(size_t)r * (G + 1) + j];
      if (j <= n[r]) CHECK(t >= -1 && t < V);
      else CHECK(t == -1);
    }
  }
}

void scalar_entry_points(Gen& g) {
  const uint32_t ctr[4] = {1, 2, 3, 4}, key[2] = {5, 6};
  uint32_t o[4];
  sv_ref_philox4x32_10(ctr, key, o);
  for (uint32_t b = 0; b < 64; ++b) {
    const double u = sv_ref_uniform_accept(42, b, b % 7), v = sv_ref_uniform_race(42, b, 3, 1000 + b);
    CHECK(u > 0.0 && u <= 1.0 && v > 0.0 && v <= 1.0);
  }
  for (int dtype = 0; dtype < 2; ++dtype) {
    for (int V : {1, 2, 5, 64, 65, 300}) {
      std::vector<uint8_t> row = rows(g, 1, V, dtype);
      std::vector<double> p(V);
      for (double tp : {1e-30, 0.5, 0.9, 1.0}) {
        for (int k : {0, 1, 3, V}) {
          double cm = 0.0;
          CHECK(sv_ref_row_probs_p(row.data(), dtype, V, 0.7, k, tp, p.data(), &cm) == 0);
          double s = 0.0;
          for (double x : p) s += x;
          CHECK(std::fabs(s - 1.0) < 1e-9);
        }
      }
      const int a = sv_ref_row_argmax(row.data(), dtype, V);
      CHECK(a >= 0 && a < V);
      std::vector<double> w(V, 0.0);
      double m = 0.0;
      CHECK(sv_ref_race(w.data(), V, 1, 0, 0, &m) == -1);  // no mass: no winner
      w[V - 1] = 1.0;
      CHECK(sv_ref_race(w.data(), V, 1, 0, 0, &m) == V - 1);
      CHECK(m == 1.0);  // one candidate
    }
  }
  CHECK(sv_ref_accept_margin(0.5, 0.25, 0.5, 1) == 0.0);
  CHECK(sv_ref_race_margin(1, 1.0, -1.0) == 1.0);
  CHECK(sv_ref_nucleus_margin(1, 0.5, 0.0, 0.25) == 0.25);
}

void dense_verify(Gen& g) {
  for (int dtype = 0; dtype < 2; ++dtype) {
    for (int mode = 0; mode < 4; ++mode) {
      const int nreq = 5, G = 3, V = 37;
      std::vector<uint8_t> lt = rows(g, nreq * (G + 1), V, dtype), ld = rows(g, nreq * G, V, dtype);
      std::vector<int32_t> X(nreq * G);
      for (auto& x : X) x = g.token(V);
      X[1] = V;  // out of range: rejected and flagged
      X[4] = -3;
      std::vector<int32_t> out(nreq * (G + 1)), n(nreq), ta(nreq * (G + 1)), bad(nreq);
      std::vector<double> pd(nreq * G), qd(nreq * G), beta(nreq * G), am(nreq * G), rm(nreq);
      for (int k : {0, 4, V}) {
        const int rc = sv_ref_verify(mode, nreq, G, V, dtype, 0.8, k, 42, lt.data(), ld.data(), X.data(), nullptr,
                                     out.data(), n.data(), pd.data(), qd.data(), ta.data(), beta.data(), am.data(),
                                     rm.data(), bad.data(), 2);
        CHECK(rc == 0);
        check_tokens(out, n, nreq, G, V, nullptr);
        CHECK(bad[0] == 1 && bad[1] == 1);
      }
    }
  }
  // Invalid arguments are refused.
  std::vector<int32_t> out(8), n(2);
  CHECK(sv_ref_verify(0, 2, 0, 5, 0, 1.0, 0, 1, nullptr, nullptr, nullptr, nullptr, out.data(), n.data(), nullptr,
                      nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 1) == -1);
  CHECK(sv_ref_verify(1, 2, 1, 5, 0, 0.0, 0, 1, nullptr, nullptr, nullptr, nullptr, out.data(), n.data(), nullptr,
                      nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 1) == -1);
}

void batch_verify(Gen& g) {
  const int nreq = 7, G = 4, V = 50;
  const int32_t lengths[nreq] = {0, 4, 2, 1, 3, 4, 0};
  int total = 0;
  for (int r = 0; r < nreq; ++r) total += lengths[r];
  const float T[nreq] = {0.f, 0.7f, 1.f, 0.8f, std::numeric_limits<float>::quiet_NaN(), 1.3f, 0.5f};
  const int32_t K[nreq] = {0, 5, 0, 3, 0, 20, 1};
  const float P[nreq] = {1.f, 1.f, 0.9f, 0.5f, 1.f, 1.f, 1e-20f};
  for (int dtype = 0; dtype < 2; ++dtype) {
    for (int kind = 0; kind < 4; ++kind) {
      for (bool ragged : {false, true}) {
        const int32_t* len = ragged ? lengths : nullptr;
        const int nt = ragged ? total + nreq : nreq * (G + 1), nd = ragged ? total : nreq * G;
        std::vector<uint8_t> lt = rows(g, nt, V, dtype), ld = rows(g, nd, V, dtype);
        std::vector<float> qp((size_t)nd * V);
        for (int r = 0; r < nd; ++r) {
          double s = 0.0;
          for (int y = 0; y < V; ++y) s += (qp[(size_t)r * V + y] = (float)(g.next() % 7u));
          for (int y = 0; y < V; ++y) qp[(size_t)r * V + y] = s > 0 ? (float)(qp[(size_t)r * V + y] / s) : 0.f;
        }
        std::vector<int32_t> X(nd), par(nd);
        for (auto& x : X) x = g.token(V);
        int off = 0;
        for (int r = 0; r < nreq; ++r) {
          const int gr = ragged ? lengths[r] : G;
          for (int i = 0; i < gr; ++i) par[off + i] = (int32_t)(g.next() % (uint32_t)(i + 1));
          off += gr;
        }
        std::vector<int32_t> out(nreq * (G + 1)), n(nreq), bt(nreq), bp(nreq), pn(nreq * (G + 1));
        std::vector<double> pd(nd), qd(nd), beta(nd), am(nd), rm(nreq), cm(nreq);
        const int rc = sv_ref_verify_ex(kind, nreq, G, V, dtype, T, K, P, 8, 42, lt.data(), ld.data(), qp.data(),
                                        X.data(), len, nullptr, out.data(), n.data(), pd.data(), qd.data(),
                                        beta.data(), am.data(), rm.data(), cm.data(), bt.data(), bp.data(),
                                        kind == 3 ? par.data() : nullptr, kind == 3 ? pn.data() : nullptr, 2);
        CHECK(rc == 0);
        check_tokens(out, n, nreq, G, V, len);
        CHECK(bp[4] == 1 && bp[5] == 1);  // NaN temperature; top-k above max_top_k
        for (int r = 0; r < nreq; ++r)
          if (bp[r]) CHECK(n[r] == 0 && out[(size_t)r * (G + 1)] == -1);
      }
    }
  }
  // A length outside 0..G is refused.
  const int32_t badlen[2] = {0, 5};
  const float T2[2] = {1.f, 1.f};
  const int32_t K2[2] = {0, 0};
  const float P2[2] = {1.f, 1.f};
  std::vector<uint8_t> lt = rows(g, 10, 8, 0);
  std::vector<int32_t> X(8, 0), out(10), n(2);
  CHECK(sv_ref_verify_ex(1, 2, 4, 8, 0, T2, K2, P2, 0, 1, lt.data(), nullptr, nullptr, X.data(), badlen, nullptr,
                         out.data(), n.data(), nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                         nullptr, nullptr, 1) == -1);
}

}  // namespace

int main() {
  Gen g{0x9E3779B97F4A7C15ull};
  scalar_entry_points(g);
  dense_verify(g);
  batch_verify(g);
  if (failures) {
    std::fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  std::printf("oracle sanitizer run: ok\n");
  return 0;
}
