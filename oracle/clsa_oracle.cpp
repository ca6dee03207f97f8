// Plain fp64 CPU oracle of one CLSA decode / prefill step, in C++17.
//
// TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU-baseline leg
// load this library.  It shares no code with the HIP path (the product) nor with the Python oracle
// or the Python input generator: it regenerates every input itself from the generator definition
// below, so that agreement with them is evidence, not a tautology.
//
// What it computes (page titles as published; sections named on the page):
//  * [SUM] picx.dev summary of "You Only Index Once: Cross-Layer Sparse Attention with Shared
//    Routing", Methodology > Architecture Overview: eq. 2, routing scores I_t = q_idx,t . K_idx^T and
//    S_t = TopK(I_t, k) computed once per step; eq. 3, every cross-decoder layer l attends with its
//    own query Q_t^(l) to the selected rows K_{S_t}, V_{S_t} of the one shared cache.
//  * [FORUM] zhichai.net explainer "... (CLSA) Explained", Background: attention is
//    softmax(Q K^T / sqrt(d_k)) V; Ablations: the variant without the shared index recomputes the
//    routing in every layer (clsa_oracle_row_layer_routing).
// Readings where the pages leave a step open: plain dot-product scores (no scale, no activation);
// a decode row sees its whole sequence, prefill row t sees tokens 0..t; |S_t| = min(k, visible);
// ties at the k-th score go to the lower index; S_t ascending; one S_t for every layer and head;
// scale 1/sqrt(head_dim); query head h reads KV head floor(h * Hkv / Hq).
//
// Input generator definition (Steele, Lea & Flood, "Fast splittable pseudorandom number
// generators", OOPSLA 2014, for the SplitMix64 output function):
//  * mix(z): z += 0x9E3779B97F4A7C15; z = (z ^ z>>30) * 0xBF58476D1CE4E5B9;
//    z = (z ^ z>>27) * 0x94D049BB133111EB; return z ^ z>>31   (all mod 2^64)
//  * tensor key = mix(mix(seed) ^ tensor_id); draw j of element i = mix(key + 4 i + j)
//  * uniform integer in [lo, hi] = lo + ((draw0 >> 32) * (hi - lo + 1)) >> 32, divided by den
//  * ~N(0,1): the twelve 16-bit fields of draws 0..2 summed, minus 393210, over 65536
//  * fp32 -> bf16 round to nearest even on the bit pattern
//  * needles: K_idx of a planted token is bf16(2 * q_idx of its row); positions drawn by rejection,
//    attempt a of row b uses mix(key_needle + (b << 32) + a), position = (x >> 32) * n >> 32
//  * tensor ids: q_idx 1, K_idx 2, Q 3, K 4, V 5, needles 6, per-layer indexer queries 8.
#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <unordered_map>
#include <vector>

namespace {

constexpr uint64_t kTidQIdx = 1, kTidKIdx = 2, kTidQ = 3, kTidK = 4, kTidV = 5, kTidNeedle = 6;

uint64_t mix(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

uint64_t tensor_key(uint64_t seed, uint64_t tid) { return mix(mix(seed) ^ tid); }

uint16_t bf16_rne(float x) {
  uint32_t u;
  std::memcpy(&u, &x, 4);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

double bf16_value(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return (double)f;
}

uint16_t uniform_bits(uint64_t key, uint64_t i, int lo, int hi, int den) {
  const uint64_t x = mix(key + 4 * i);
  const uint64_t v = ((x >> 32) * (uint64_t)(hi - lo + 1)) >> 32;
  return bf16_rne((float)((int64_t)v + lo) / (float)den);
}

uint16_t normal_bits(uint64_t key, uint64_t i) {
  int64_t total = 0;
  for (int j = 0; j < 3; ++j) {
    const uint64_t x = mix(key + 4 * i + (uint64_t)j);
    for (int f = 0; f < 4; ++f) total += (int64_t)((x >> (16 * f)) & 0xFFFFu);
  }
  return bf16_rne((float)(total - 393210) / 65536.0f);
}

}  // namespace

extern "C" {

// A workload as the generator defines it.  mode 0 = decode (row b is sequence b and sees all of
// it), 1 = prefill of sequence 0 (row t sees tokens 0..t).
typedef struct {
  int32_t mode;
  int32_t batch;
  const int64_t* seq_lens;  // [batch]
  int32_t d_idx, topk, n_layers, hq, hkv, head_dim;
  int32_t idx_lo, idx_hi, idx_den, needles;
  uint64_t seed;
} clsa_oracle_workload;

// ---- generator, exported so the tests can compare it with the Python generator --------------
uint16_t clsa_oracle_gen_uniform(uint64_t seed, uint64_t tid, uint64_t i, int lo, int hi, int den) {
  return uniform_bits(tensor_key(seed, tid), i, lo, hi, den);
}
uint16_t clsa_oracle_gen_normal(uint64_t seed, uint64_t tid, uint64_t i) {
  return normal_bits(tensor_key(seed, tid), i);
}
// The first `count` needle positions of row `row` in a sequence of n tokens.  Returns 0, or 1 when
// count > n (no such set of distinct positions exists).
int clsa_oracle_gen_needles(uint64_t seed, int64_t row, int64_t n, int32_t count, int64_t* out) {
  if (count < 0 || (int64_t)count > n) return 1;
  const uint64_t key = tensor_key(seed, kTidNeedle);
  std::vector<int64_t> got;
  for (uint64_t attempt = 0; (int32_t)got.size() < count; ++attempt) {
    const uint64_t x = mix(key + (((uint64_t)row << 32) + attempt));
    const int64_t p = (int64_t)(((x >> 32) * (uint64_t)n) >> 32);
    if (std::find(got.begin(), got.end(), p) == got.end()) got.push_back(p);
  }
  std::copy(got.begin(), got.end(), out);
  return 0;
}

// ---- eq. 2, first half: I[j] = q . K[j] over the n visible tokens ----------------------------
void clsa_oracle_scores(const double* q, const double* k_rows, int64_t n, int32_t d, double* out) {
  for (int64_t j = 0; j < n; ++j) {
    double s = 0.0;
    for (int32_t c = 0; c < d; ++c) s += q[c] * k_rows[j * d + c];
    out[j] = s;
  }
}

// ---- eq. 2, second half: S = TopK(I, k) ------------------------------------------------------
// Full sort by (score descending, index ascending), the first min(k, n) kept, returned
// ascending; idx has k entries, -1 after the count.  -0.0 == +0.0 under this comparison.
void clsa_oracle_topk(const double* scores, int64_t n, int32_t k, int32_t* idx, int32_t* count) {
  std::vector<int64_t> order((size_t)n);
  for (int64_t j = 0; j < n; ++j) order[(size_t)j] = j;
  std::sort(order.begin(), order.end(), [&](int64_t a, int64_t b) {
    if (scores[a] != scores[b]) return scores[a] > scores[b];
    return a < b;
  });
  const int64_t m = std::min<int64_t>(k, n);
  std::sort(order.begin(), order.begin() + m);
  for (int32_t i = 0; i < k; ++i) idx[i] = i < m ? (int32_t)order[(size_t)i] : -1;
  *count = (int32_t)m;
}

// ---- eq. 3 with the attention of [FORUM] Background ------------------------------------------
// q [Lc, Hq, hd]; k_sel, v_sel [m, Hkv, hd] (the same m selected rows for every layer and head);
// out [Lc, Hq, hd].  scale <= 0 means 1/sqrt(hd).
void clsa_oracle_attention(const double* q, const double* k_sel, const double* v_sel, int64_t m, int32_t lc,
                           int32_t hq, int32_t hkv, int32_t hd, double scale, double* out) {
  if (scale <= 0.0) scale = 1.0 / std::sqrt((double)hd);
  std::vector<double> logit((size_t)m);
  for (int32_t l = 0; l < lc; ++l)
    for (int32_t h = 0; h < hq; ++h) {
      const int32_t g = (int32_t)(((int64_t)h * hkv) / hq);
      const double* qv = q + ((int64_t)l * hq + h) * hd;
      double mx = -INFINITY;
      for (int64_t i = 0; i < m; ++i) {
        const double* kv = k_sel + (i * hkv + g) * hd;
        double s = 0.0;
        for (int32_t d = 0; d < hd; ++d) s += qv[d] * kv[d];
        logit[(size_t)i] = s * scale;
        mx = std::max(mx, logit[(size_t)i]);
      }
      double den = 0.0;
      double* o = out + ((int64_t)l * hq + h) * hd;
      for (int32_t d = 0; d < hd; ++d) o[d] = 0.0;
      for (int64_t i = 0; i < m; ++i) {
        const double p = std::exp(logit[(size_t)i] - mx);
        den += p;
        const double* vv = v_sel + (i * hkv + g) * hd;
        for (int32_t d = 0; d < hd; ++d) o[d] += p * vv[d];
      }
      for (int32_t d = 0; d < hd; ++d) o[d] /= den;
    }
}

// ---- one query row of the step, inputs regenerated from the workload definition -------------
namespace {

constexpr uint64_t kTidQIdxLayer = 8;

// What a query row sees: its sequence, the cache row of its first token, its n visible tokens
// and their indexer keys (n x d_idx, needles included).  Returns false on a bad argument.
struct RowInputs {
  int32_t seq = 0;
  int64_t base = 0, n = 0;
  std::vector<double> k_idx;
};

bool row_inputs(const clsa_oracle_workload* w, int32_t row, RowInputs* in) {
  if (w == nullptr || w->batch < 1 || w->head_dim < 1 || w->hkv < 1 || w->hq % w->hkv != 0) return false;
  std::vector<int64_t> cu((size_t)w->batch + 1, 0);
  for (int32_t b = 0; b < w->batch; ++b) cu[(size_t)b + 1] = cu[(size_t)b] + w->seq_lens[b];
  const bool decode = w->mode == 0;
  const int32_t n_rows = decode ? w->batch : (int32_t)w->seq_lens[0];
  if (row < 0 || row >= n_rows) return false;
  in->seq = decode ? row : 0;
  in->n = decode ? w->seq_lens[row] : (int64_t)row + 1;
  in->base = cu[(size_t)in->seq];
  const int32_t d = w->d_idx;
  const uint64_t kq = tensor_key(w->seed, kTidQIdx), kk = tensor_key(w->seed, kTidKIdx);
  // needles planted in this row's sequence: global token -> the q_idx row it copies
  std::unordered_map<int64_t, int64_t> needle;
  if (w->needles > 0) {
    std::vector<int64_t> pos((size_t)w->needles);
    if (decode) {
      if (clsa_oracle_gen_needles(w->seed, in->seq, w->seq_lens[in->seq], w->needles, pos.data())) return false;
      for (int64_t p : pos) needle[in->base + p] = in->seq;
    } else {
      if (clsa_oracle_gen_needles(w->seed, 0, w->seq_lens[0], w->needles, pos.data())) return false;
      for (int64_t p : pos) needle[p] = w->seq_lens[0] - 1;
    }
  }
  in->k_idx.assign((size_t)(in->n * d), 0.0);
  for (int64_t j = 0; j < in->n; ++j) {
    const int64_t t = in->base + j;
    const auto it = needle.find(t);
    for (int32_t c = 0; c < d; ++c) {
      uint16_t bits;
      if (it != needle.end())
        bits = bf16_rne(2.0f * (float)bf16_value(uniform_bits(kq, (uint64_t)(it->second * d + c), w->idx_lo,
                                                               w->idx_hi, w->idx_den)));
      else
        bits = uniform_bits(kk, (uint64_t)(t * d + c), w->idx_lo, w->idx_hi, w->idx_den);
      in->k_idx[(size_t)(j * d + c)] = bf16_value(bits);
    }
  }
  return true;
}

// Attention of layers layer0 .. layer0 + lc - 1 of `row` over the m selected local tokens sel[],
// read from the one shared cache; out [lc, Hq, hd].
void attend_row(const clsa_oracle_workload* w, int32_t row, const RowInputs& in, int32_t layer0, int32_t lc,
                const int32_t* sel, int64_t m, double* out) {
  const int32_t hd = w->head_dim, L = w->n_layers, hq = w->hq, hkv = w->hkv;
  const uint64_t kqa = tensor_key(w->seed, kTidQ), kka = tensor_key(w->seed, kTidK), kva = tensor_key(w->seed, kTidV);
  std::vector<double> q((size_t)lc * hq * hd), ks((size_t)m * hkv * hd), vs((size_t)m * hkv * hd);
  const int64_t qrow = (int64_t)row * L * hq * hd + (int64_t)layer0 * hq * hd;
  for (int64_t e = 0; e < (int64_t)lc * hq * hd; ++e) q[(size_t)e] = bf16_value(normal_bits(kqa, (uint64_t)(qrow + e)));
  for (int64_t i = 0; i < m; ++i) {
    const int64_t t = in.base + sel[i];
    for (int64_t e = 0; e < (int64_t)hkv * hd; ++e) {
      ks[(size_t)(i * hkv * hd + e)] = bf16_value(normal_bits(kka, (uint64_t)(t * hkv * hd + e)));
      vs[(size_t)(i * hkv * hd + e)] = bf16_value(normal_bits(kva, (uint64_t)(t * hkv * hd + e)));
    }
  }
  clsa_oracle_attention(q.data(), ks.data(), vs.data(), m, lc, hq, hkv, hd, 0.0, out);
}

}  // namespace

// idx [topk] (ascending, -1 padded), count, out [L, Hq, hd]; scores [visible tokens] optional.
// Returns 0, or 1 on a bad argument.
int clsa_oracle_row(const clsa_oracle_workload* w, int32_t row, int32_t* idx, int32_t* count, double* out,
                    double* scores_out) {
  RowInputs in;
  if (!row_inputs(w, row, &in)) return 1;
  const int32_t d = w->d_idx;
  const uint64_t kq = tensor_key(w->seed, kTidQIdx);
  std::vector<double> qv((size_t)d), sc((size_t)in.n);
  for (int32_t c = 0; c < d; ++c)
    qv[(size_t)c] = bf16_value(uniform_bits(kq, (uint64_t)((int64_t)row * d + c), w->idx_lo, w->idx_hi, w->idx_den));
  clsa_oracle_scores(qv.data(), in.k_idx.data(), in.n, d, sc.data());
  if (scores_out != nullptr) std::copy(sc.begin(), sc.end(), scores_out);
  clsa_oracle_topk(sc.data(), in.n, w->topk, idx, count);
  // one selection for every layer and head
  attend_row(w, row, in, 0, w->n_layers, idx, *count, out);
  return 0;
}

// The ablation without the shared index (zhichai.net explainer, Ablations: per-layer recompute;
// picx.dev summary, Complexity Comparison: eta L N instead of eta N): layer l scores the row's
// visible tokens with its OWN indexer query (tensor id 8, element (row, l, c) of [R, L, d_idx]),
// selects its own set and attends with its own query over that set.
// idx [L, topk], count [L], out [L, Hq, hd].  Returns 0, or 1 on a bad argument.
int clsa_oracle_row_layer_routing(const clsa_oracle_workload* w, int32_t row, int32_t* idx, int32_t* count,
                                  double* out) {
  RowInputs in;
  if (!row_inputs(w, row, &in)) return 1;
  const int32_t d = w->d_idx, L = w->n_layers;
  const uint64_t kql = tensor_key(w->seed, kTidQIdxLayer);
  std::vector<double> qv((size_t)d), sc((size_t)in.n);
  for (int32_t l = 0; l < L; ++l) {
    for (int32_t c = 0; c < d; ++c)
      qv[(size_t)c] = bf16_value(uniform_bits(kql, (uint64_t)(((int64_t)row * L + l) * d + c), w->idx_lo, w->idx_hi,
                                              w->idx_den));
    clsa_oracle_scores(qv.data(), in.k_idx.data(), in.n, d, sc.data());
    int32_t* li = idx + (int64_t)l * w->topk;
    clsa_oracle_topk(sc.data(), in.n, w->topk, li, count + l);
    attend_row(w, row, in, l, 1, li, count[l], out + (int64_t)l * w->hq * w->head_dim);
  }
  return 0;
}

// The rows `rows[0..n)` spread over `threads` host threads, each row computed by the
// single-threaded clsa_oracle_row.  idx [n, topk], count [n], out [n, L*Hq*hd].  Writes the wall
// time of the computation to *seconds.  Returns 0, or 1 if any row failed.
int clsa_oracle_rows(const clsa_oracle_workload* w, const int32_t* rows, int32_t n, int32_t threads, int32_t* idx,
                     int32_t* count, double* out, double* seconds) {
  if (threads < 1) threads = 1;
  const int64_t per = (int64_t)w->n_layers * w->hq * w->head_dim;
  std::vector<int> fail((size_t)threads, 0);
  const auto t0 = std::chrono::steady_clock::now();
  std::vector<std::thread> pool;
  for (int32_t t = 0; t < threads; ++t)
    pool.emplace_back([&, t]() {
      for (int32_t i = t; i < n; i += threads)
        fail[(size_t)t] |= clsa_oracle_row(w, rows[i], idx + (int64_t)i * w->topk, count + i, out + i * per, nullptr);
    });
  for (auto& th : pool) th.join();
  *seconds = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
  for (int f : fail)
    if (f) return 1;
  return 0;
}

// clsa_oracle_row_layer_routing over rows[0..n) on `threads` host threads.  idx [n, L, topk],
// count [n, L], out [n, L*Hq*hd].  Returns 0, or 1 if any row failed.
int clsa_oracle_rows_layer_routing(const clsa_oracle_workload* w, const int32_t* rows, int32_t n, int32_t threads,
                                   int32_t* idx, int32_t* count, double* out) {
  if (threads < 1) threads = 1;
  const int64_t L = w->n_layers, per = L * w->hq * w->head_dim;
  std::vector<int> fail((size_t)threads, 0);
  std::vector<std::thread> pool;
  for (int32_t t = 0; t < threads; ++t)
    pool.emplace_back([&, t]() {
      for (int32_t i = t; i < n; i += threads)
        fail[(size_t)t] |= clsa_oracle_row_layer_routing(w, rows[i], idx + (int64_t)i * L * w->topk, count + i * L,
                                                         out + i * per);
    });
  for (auto& th : pool) th.join();
  for (int f : fail)
    if (f) return 1;
  return 0;
}

}  // extern "C"
