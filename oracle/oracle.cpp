// Plain CPU oracle for the batched speculative-verify + SAM-draft step.
//
// TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or
// call this file: only tests/, __graft_entry__.smoke() and the cpu_baseline
// leg of bench.py use it. It shares no code, header, table or constant with
// the HIP library; the two meet only in the seeded inputs they are given.
//
// Sources (the pages this follows):
//   [P1] "SAM投机推理：长序列强化学习训练加速利器" (CANN cann-recipes-train
//        article), §1.1 "SAM 原理" and §3.1.2 "拒绝采样加速".
//   [P2] speculative-sampling guide "1. 投机采样到底在解决什么问题"
//        (m.nxbn.cn), §2.2 "验证阶段的并行打分机制".
//   [P3] notes "投机采样" (gogongxt.com), section "贪婪验证，拒绝采样" and
//        its subsections "贪婪采样" / "拒绝采样", and "SGLang 的实现".
//   [P4] SAM-Decoding summary (developer.volcengine.com), §2 "Suffix
//        Automaton", §3 "Suffix Automaton Construction", "Drafting with
//        Suffix Automaton", "Update of Suffix Automaton".
//
// Every function is a direct, slow statement of a definition: a std::map
// suffix automaton built by Blumer's online construction, and per-sequence
// verification in double precision. No blocking, fusion or reordering.
//
// Pins: each function is checked in tests/ against values fixed by the pages
// or by mathematics (worked example, brute force, closed forms, chi-square).
// Functions without such a pin: none.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <map>
#include <thread>
#include <vector>

namespace {

// ---------------------------------------------------------------------------
// Suffix automaton ([P1] §1.1; [P4] §2 "Suffix Automaton", §3 "Suffix
// Automaton Construction").
//
// A state is an endpos-equivalence class of substrings of the text S. next is
// the transition function, link the suffix link (the state of the longest
// proper suffix whose endpos set differs). min_endpos records the smallest end
// position shared by the state's strings (its first occurrence), which
// [P1] §1.1 and [P4] §3 say the dynamic automaton maintains while it grows.
// State 0 is the root (empty string): len 0, link -1, min_endpos -1.
// ---------------------------------------------------------------------------
struct OracleSAM {
  std::vector<int32_t> len, link, minend;
  std::vector<std::map<int32_t, int32_t>> next;
  std::vector<int32_t> text;  // the committed tokens S[0..n-1]
  int32_t last = 0;
  int32_t last_walk_hops = 0;

  OracleSAM() { add_state(0, -1, -1); }

  int32_t add_state(int32_t l, int32_t lk, int32_t me) {
    len.push_back(l);
    link.push_back(lk);
    minend.push_back(me);
    next.emplace_back();
    return (int32_t)len.size() - 1;
  }

  // Blumer et al. (1984) online extension by one token c appended at
  // 0-indexed position i = n. The new state `cur` is created before any
  // clone, so ids follow creation order.
  void extend(int32_t c) {
    const int32_t i = (int32_t)text.size();
    const int32_t cur = add_state(len[last] + 1, -1, i);
    int32_t p = last;
    while (p != -1 && next[p].find(c) == next[p].end()) {
      next[p][c] = cur;
      p = link[p];
    }
    if (p == -1) {
      link[cur] = 0;
    } else {
      const int32_t q = next[p][c];
      if (len[p] + 1 == len[q]) {
        link[cur] = q;
      } else {
        // endpos(clone) = endpos(q) ∪ {i}; i is the largest position seen, so
        // the first occurrence of the clone's strings is that of q.
        const int32_t clone = add_state(len[p] + 1, link[q], minend[q]);
        next[clone] = next[q];
        while (p != -1) {
          auto it = next[p].find(c);
          if (it == next[p].end() || it->second != q) break;
          it->second = clone;
          p = link[p];
        }
        link[q] = clone;
        link[cur] = clone;
      }
    }
    last = cur;
    text.push_back(c);
  }

  // Drafting ([P1] §1.1, the ABCBC example; [P4] "Drafting with Suffix
  // Automaton"): from the state of the whole text, follow suffix links until a
  // state has an outgoing next edge. That state holds the longest suffix of S
  // that occurred earlier; its min_endpos locates the first such occurrence and
  // the tokens after it are the draft. A match of length 0 (the walk reached
  // the root) gives no draft; a draft that would run past the end of S is cut
  // at the end of S.
  int32_t draft(int32_t K, int32_t* out, int32_t* match_len) {
    int32_t s = last;
    int32_t hops = 0;
    while (s != 0 && next[s].empty()) {
      s = link[s];
      ++hops;
    }
    last_walk_hops = hops;
    for (int32_t j = 0; j < K; ++j) out[j] = -1;
    const int32_t L = len[s];
    *match_len = L;
    if (L == 0) return 0;
    const int32_t n = (int32_t)text.size();
    const int32_t p = minend[s];
    const int32_t d = std::min<int32_t>(K, n - 1 - p);
    for (int32_t j = 0; j < d; ++j) out[j] = text[p + 1 + j];
    return d;
  }

  // Draft tree from several candidates (an extension of the drafting above
  // to the tree layout the tree verifier takes; the pages draft one
  // candidate): the state the draft walk reaches, then up to M - 1 of its
  // suffix-link ancestors (each a shorter suffix of S whose occurrences are a
  // superset, down to the root, excluded), each giving the tokens after its
  // first occurrence (K at most, cut at the end of S). The candidates are
  // merged into a trie in that order: node 0 is the root; a candidate walks
  // down the children with its tokens and adds a node where none matches, so
  // a node's children appear in the order their candidates came. Returns the
  // node count; tok/par receive node i's token and parent (root: -1, -1).
  int32_t draft_tree(int32_t K, int32_t M, int32_t* tok, int32_t* par,
                     int32_t* match_len) {
    int32_t s = last;
    while (s != 0 && next[s].empty()) s = link[s];
    *match_len = len[s];
    int32_t nn = 1;
    tok[0] = par[0] = -1;
    const int32_t n = (int32_t)text.size();
    for (int32_t i = 0; i < M && s != 0 && len[s] > 0; ++i, s = link[s]) {
      const int32_t p = minend[s];
      const int32_t d = std::min<int32_t>(K, n - 1 - p);
      int32_t cur = 0;
      for (int32_t j = 0; j < d; ++j) {
        const int32_t t = text[p + 1 + j];
        int32_t found = -1;
        for (int32_t v = 1; v < nn; ++v)
          if (par[v] == cur && tok[v] == t) found = v;
        if (found < 0) {
          found = nn++;
          par[found] = cur;
          tok[found] = t;
        }
        cur = found;
      }
    }
    return nn;
  }

  // Match-state transfer on a fixed automaton ([P4] "Drafting with Suffix
  // Automaton", "Update of Suffix Automaton", state transfer of Algorithm 1):
  // (s, l) is the state of the longest suffix of a generated text that occurs
  // in this automaton's reference text, and that suffix's length. Appending
  // token t: if s has a transition on t it is taken and the match grows by
  // one; otherwise suffix links are followed to the first state with such a
  // transition, and the match becomes that state's longest string plus t; if
  // even the root has none, the match is empty (root, 0).
  void match_step(int32_t& s, int32_t& l, int32_t t) const {
    while (true) {
      auto it = next[s].find(t);
      if (it != next[s].end()) {
        s = it->second;
        l += 1;
        return;
      }
      if (s == 0) {
        l = 0;
        return;
      }
      s = link[s];
      l = len[s];
    }
  }

  // Draft from a match state: the tokens that followed the first occurrence
  // of the matched suffix in the reference text (min_endpos of s), cut at the
  // end of the text; an empty match gives no draft.
  int32_t draft_from(int32_t s, int32_t l, int32_t K, int32_t* out) const {
    for (int32_t j = 0; j < K; ++j) out[j] = -1;
    if (l == 0) return 0;
    const int32_t n = (int32_t)text.size();
    const int32_t p = minend[s];
    const int32_t d = std::min<int32_t>(K, n - 1 - p);
    for (int32_t j = 0; j < d; ++j) out[j] = text[p + 1 + j];
    return d;
  }

  int64_t num_edges() const {
    int64_t e = 0;
    for (const auto& m : next) e += (int64_t)m.size();
    return e;
  }
};

// ---------------------------------------------------------------------------
// Verification ([P2] §2.2; [P3] "贪婪采样" and "拒绝采样"; [P1] §1.1 and
// §3.1.2).
// ---------------------------------------------------------------------------

// Status bits (same meaning as the library's, defined here independently).
constexpr int32_t ST_TOKEN_RANGE = 1 << 1;
constexpr int32_t ST_DRAFT_LEN = 1 << 2;
constexpr int32_t ST_NONFINITE = 1 << 3;
constexpr int32_t ST_TEMPERATURE = 1 << 4;
constexpr int32_t ST_NO_UNIFORMS = 1 << 5;
constexpr int32_t ST_TOP_P = 1 << 7;
constexpr int32_t ST_TREE = 1 << 8;

// bfloat16 is the upper half of an IEEE binary32: widen by appending 16 zero
// bits.
double bf16_to_double(uint16_t h) {
  uint32_t bits = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &bits, sizeof f);
  return (double)f;
}

void load_row(const void* logits, int dtype, int64_t row, int64_t V,
              std::vector<double>& out) {
  out.resize((size_t)V);
  if (dtype == 0) {
    const float* r = (const float*)logits + row * V;
    for (int64_t i = 0; i < V; ++i) out[(size_t)i] = (double)r[i];
  } else {
    const uint16_t* r = (const uint16_t*)logits + row * V;
    for (int64_t i = 0; i < V; ++i) out[(size_t)i] = bf16_to_double(r[i]);
  }
}

// Lowest index among the maxima ([P3] "贪婪采样": the token the target model
// rates most probable).
int64_t argmax_lowest(const std::vector<double>& l) {
  int64_t best = 0;
  for (int64_t i = 1; i < (int64_t)l.size(); ++i)
    if (l[(size_t)i] > l[(size_t)best]) best = i;
  return best;
}

// p = softmax(l / T), written as w_i = exp((l_i - m) / T), Z = sum w, p = w/Z.
void softmax_T(const std::vector<double>& l, double T, std::vector<double>& p) {
  double m = -std::numeric_limits<double>::infinity();
  for (double v : l) m = std::max(m, v);
  p.resize(l.size());
  double Z = 0.0;
  for (size_t i = 0; i < l.size(); ++i) {
    p[i] = std::exp((l[i] - m) / T);
    Z += p[i];
  }
  for (double& v : p) v /= Z;
}

// Inverse CDF in ascending token order: the smallest i with
// sum_{k<=i} w_k > u * sum(w). If rounding leaves no such i, the largest i with
// w_i > 0. lo/hi receive the normalised CDF just before and at the chosen
// index, so a caller can tell how close u was to a breakpoint.
int64_t inv_cdf(const std::vector<double>& w, double u, double* lo, double* hi) {
  double S = 0.0;
  for (double v : w) S += v;
  const double t = u * S;
  double c = 0.0;
  int64_t last_pos = -1;
  for (size_t i = 0; i < w.size(); ++i) {
    const double prev = c;
    c += w[i];
    if (w[i] > 0.0) last_pos = (int64_t)i;
    if (c > t) {
      *lo = prev / S;
      *hi = c / S;
      return (int64_t)i;
    }
  }
  *lo = *hi = 1.0;
  return last_pos;
}

// A row is usable when it holds no NaN, no +inf, and at least one entry above
// -inf (-inf marks a token with probability 0).
bool finite_row(const std::vector<double>& l) {
  bool any_above_neg_inf = false;
  for (double v : l) {
    if (std::isnan(v)) return false;
    if (v == std::numeric_limits<double>::infinity()) return false;
    if (v > -std::numeric_limits<double>::infinity()) any_above_neg_inf = true;
  }
  return any_above_neg_inf;
}

// Truncation of a sampling distribution before verification ([P3] "SGLang
// 的实现": the target probabilities are renormalised by top-k, then by top-p,
// before the speculative-sampling kernel sees them; one value of each per
// request, applied to every position of that request). Read as:
//   top-k (1 <= k < V): keep the tokens whose logit is at least the k-th
//     largest logit (counted with multiplicity; tokens tied with it are all
//     kept), drop the rest;
//   top-p (0 < top_p < 1), on what top-k kept: going down the distinct logit
//     values, keep every token of each value until the kept probability,
//     relative to what top-k kept, first reaches top_p (that whole group of
//     tied tokens included);
//   then renormalise. k <= 0 or k >= V, and top_p = 1, leave p as it is.
// p is overwritten with the truncated distribution. Returns the threshold
// logit (keep l >= threshold; -inf when nothing is dropped). *margin receives
// how far, relative to the mass top-k kept, the top-p decision was from
// flipping (the smaller of the gaps to top_p on both sides of the chosen
// group); NaN when top-p made no decision.
double truncate(const std::vector<double>& l, std::vector<double>& p, int32_t top_k,
                double top_p, double* margin) {
  const int64_t V = (int64_t)l.size();
  const double ninf = -std::numeric_limits<double>::infinity();
  *margin = std::numeric_limits<double>::quiet_NaN();
  const bool use_k = top_k >= 1 && top_k < V;
  const bool use_p = top_p < 1.0;
  if (!use_k && !use_p) return ninf;
  std::vector<int64_t> order((size_t)V);
  for (int64_t i = 0; i < V; ++i) order[(size_t)i] = i;
  std::sort(order.begin(), order.end(),
            [&](int64_t a, int64_t b) { return l[(size_t)a] > l[(size_t)b]; });
  double thr = ninf;
  if (use_k) thr = l[(size_t)order[(size_t)(top_k - 1)]];
  if (use_p) {
    double Zk = 0.0;
    for (int64_t i = 0; i < V; ++i)
      if (l[(size_t)i] >= thr) Zk += p[(size_t)i];
    const double target = top_p * Zk;
    double cum = 0.0;
    int64_t g = 0;
    while (g < V && l[(size_t)order[(size_t)g]] >= thr) {
      const double v = l[(size_t)order[(size_t)g]];
      const double before = cum;
      int64_t e = g;
      while (e < V && l[(size_t)order[(size_t)e]] == v) cum += p[(size_t)order[(size_t)e++]];
      if (cum >= target) {
        thr = v;
        *margin = std::min(target - before, cum - target) / Zk;
        break;
      }
      g = e;
    }
  }
  double Z = 0.0;
  for (int64_t i = 0; i < V; ++i) {
    if (l[(size_t)i] < thr) p[(size_t)i] = 0.0;
    Z += p[(size_t)i];
  }
  for (double& v : p) v /= Z;
  return thr;
}

struct VerifyIO {
  const void* logits;
  int dtype;
  int B, K, V;
  const int32_t* draft;
  const int32_t* draft_len;
  const float* q;  // [B,K,V] or null (one-hot q = delta at the draft token)
  const float* temperature;
  const float* uniforms;  // [B,K+1] or null
  int32_t* out_tokens;    // [B,K+1]
  int32_t* num_emitted;   // [B]
  double* p_draft;        // [B,K] target probability of each draft token
  double* alpha;          // [B,K] acceptance threshold min(1,p/q) (NaN unused)
  double* cdf_lo;         // [B] normalised CDF breakpoints of the final draw
  double* cdf_hi;         // [B]
  int32_t* status;        // [B] (OR-ed)
  const int32_t* top_k;   // [B] or null (no top-k)
  const float* top_p;     // [B] or null (no top-p)
  double* trunc_thr;      // [B,K+1] threshold logit of each row used (NaN unused)
  double* trunc_margin;   // [B,K+1] top-p decision margin (NaN: none)
};

// One sequence of the step ([P2] §2.2: K+1 target distributions from one
// forward; judge the drafts in order; at the first rejection drop the rest and
// resample there; [P1] §3.1.2: a recovered token at the rejected position, a
// bonus token when every draft is accepted).
void verify_one(const VerifyIO& io, int b) {
  const int K = io.K;
  const int64_t V = io.V;
  const int64_t R = K + 1;
  int32_t* out = io.out_tokens + (int64_t)b * R;
  double* pd = io.p_draft + (int64_t)b * K;
  double* al = io.alpha + (int64_t)b * K;
  for (int j = 0; j < K; ++j) {
    pd[j] = -1.0;
    al[j] = std::numeric_limits<double>::quiet_NaN();
  }
  io.cdf_lo[b] = io.cdf_hi[b] = std::numeric_limits<double>::quiet_NaN();
  if (io.trunc_thr)
    for (int64_t j = 0; j < R; ++j)
      io.trunc_thr[(int64_t)b * R + j] = io.trunc_margin[(int64_t)b * R + j] =
          std::numeric_limits<double>::quiet_NaN();

  const int32_t d = io.draft_len[b];
  const double T = (double)io.temperature[b];
  int32_t st = 0;
  if (d < 0 || d > K) st |= ST_DRAFT_LEN;
  // T = 0 is greedy; a positive T must be a finite float no smaller than the
  // smallest normal float (below it 1/T is not representable in float).
  if (!(T == 0.0 || (T >= (double)std::numeric_limits<float>::min() &&
                     std::isfinite(T))))
    st |= ST_TEMPERATURE;
  if (T > 0.0 && io.uniforms == nullptr) st |= ST_NO_UNIFORMS;
  const int32_t top_k = io.top_k ? io.top_k[b] : 0;
  const double top_p = io.top_p ? (double)io.top_p[b] : 1.0;
  if (!(top_p > 0.0 && top_p <= 1.0)) st |= ST_TOP_P;
  if (st == 0) {
    for (int j = 0; j < d; ++j) {
      const int32_t x = io.draft[(int64_t)b * K + j];
      if (x < 0 || x >= V) st |= ST_TOKEN_RANGE;
    }
  }
  std::vector<std::vector<double>> rows((size_t)(st ? 0 : d + 1));
  for (int j = 0; st == 0 && j <= d; ++j) {
    load_row(io.logits, io.dtype, (int64_t)b * R + j, V, rows[(size_t)j]);
    if (!finite_row(rows[(size_t)j])) st |= ST_NONFINITE;
  }
  if (st != 0) {
    io.status[b] |= st;
    return;
  }

  for (int64_t j = 0; j < R; ++j) out[j] = -1;

  if (T == 0.0) {
    // Greedy ([P3] "贪婪采样"): accept a draft iff it equals the target's
    // argmax; at the first mismatch emit the argmax and stop; if all d pass,
    // emit the argmax of row d.
    for (int j = 0; j < d; ++j) {
      const int32_t x = io.draft[(int64_t)b * K + j];
      const int64_t a = argmax_lowest(rows[(size_t)j]);
      if (x != a) {
        out[j] = (int32_t)a;
        io.num_emitted[b] = j + 1;
        return;
      }
      out[j] = x;
    }
    out[d] = (int32_t)argmax_lowest(rows[(size_t)d]);
    io.num_emitted[b] = d + 1;
    return;
  }

  // Sampling ([P2] §2.2; [P1] §1.1: accept x drawn from q iff eps <= alpha(x),
  // alpha = min(1, p/q); on rejection draw from norm(max(0, p - q)); one-hot q
  // when the drafts come with no probabilities, [P3] "SGLang 的实现").
  const float* u = io.uniforms + (int64_t)b * R;
  std::vector<double> p, w;
  // p_j: softmax(l_j / T), truncated when the request asks for it.
  auto target = [&](int j) {
    softmax_T(rows[(size_t)j], T, p);
    double mg;
    const double thr = truncate(rows[(size_t)j], p, top_k, top_p, &mg);
    if (io.trunc_thr) {
      io.trunc_thr[(int64_t)b * R + j] = thr;
      io.trunc_margin[(int64_t)b * R + j] = mg;
    }
  };
  for (int j = 0; j < d; ++j) {
    const int32_t x = io.draft[(int64_t)b * K + j];
    target(j);
    pd[j] = p[(size_t)x];
    double qx = 1.0;
    if (io.q) qx = (double)io.q[((int64_t)b * K + j) * V + x];
    double ratio;
    if (qx > 0.0)
      ratio = p[(size_t)x] / qx;
    else
      ratio = p[(size_t)x] > 0.0 ? 1.0 : 0.0;
    al[j] = std::min(1.0, ratio);
    if ((double)u[j] <= ratio) {
      out[j] = x;
      continue;
    }
    // Rejected: residual max(0, p - q); for one-hot q, p with x removed.
    w.assign(p.size(), 0.0);
    if (io.q) {
      const float* qr = io.q + ((int64_t)b * K + j) * V;
      for (int64_t i = 0; i < V; ++i)
        w[(size_t)i] = std::max(0.0, p[(size_t)i] - (double)qr[i]);
    } else {
      w = p;
      w[(size_t)x] = 0.0;
    }
    double S = 0.0;
    for (double v : w) S += v;
    if (!(S > 0.0)) w = p;  // only when p == q exactly
    out[j] = (int32_t)inv_cdf(w, (double)u[K], &io.cdf_lo[b], &io.cdf_hi[b]);
    io.num_emitted[b] = j + 1;
    return;
  }
  // Every draft accepted: bonus token from the target at row d.
  target(d);
  out[d] = (int32_t)inv_cdf(p, (double)u[K], &io.cdf_lo[b], &io.cdf_hi[b]);
  io.num_emitted[b] = d + 1;
}


// Verification of a draft tree ([P3] gogongxt notes "SGLang 的实现": the
// target-only tree sampling walks the draft tree depth by depth; at a node the
// children are tried in sibling order, each adding its target probability to
// a running sum, and the first child whose running sum reaches the depth's
// coin is accepted, the sum starting again at the next depth; when no child
// passes, the children's probabilities are taken out of the target and the
// final token is drawn from what is left; with both of the page's thresholds
// at 1, which makes the walk lossless). Read as:
//   node 0 is the root (the last committed token); node i >= 1 holds a
//   drafted token and a parent p < i; row i of the logits scores the token
//   after the path root..i; the children of a node are taken in increasing
//   node index and must carry distinct tokens;
//   T > 0: at depth t (t tokens accepted so far) with coin u[t], child c_k is
//   accepted iff u[t] <= sum_{k' <= k} p(x_{c_k'}); if none, the final token is
//   drawn with u[N-1] from p with the children's tokens removed; at a leaf
//   (every draft on the path accepted) it is drawn from the leaf's row;
//   T = 0: the child whose token is the row's argmax is accepted, else the
//   argmax is emitted (also at a leaf).
// Outputs per sequence: the emitted tokens, the node each came from (the
// accepted child, or for the last token the node whose row it was drawn
// from), their number; gap[b, t] is the smallest distance between u[t] and
// the running sums at depth t (tie detection), cdf_lo/hi as in orc_verify.
struct TreeIO {
  const void* logits;
  int dtype, B, N, V;
  const int32_t* tokens;   // [B,N]
  const int32_t* parent;   // [B,N]
  const int32_t* n_nodes;  // [B]
  const float* temperature;
  const float* uniforms;   // [B,N]
  int32_t* out_tokens;     // [B,N]
  int32_t* out_nodes;      // [B,N]
  int32_t* num_emitted;    // [B]
  double* gap;             // [B,N]
  double* cdf_lo;
  double* cdf_hi;
  int32_t* status;
};

void verify_tree_one(const TreeIO& io, int b) {
  const int N = io.N;
  const int64_t V = io.V;
  int32_t* out = io.out_tokens + (int64_t)b * N;
  int32_t* onode = io.out_nodes + (int64_t)b * N;
  double* gap = io.gap + (int64_t)b * N;
  for (int i = 0; i < N; ++i) {
    out[i] = onode[i] = -1;
    gap[i] = std::numeric_limits<double>::quiet_NaN();
  }
  io.cdf_lo[b] = io.cdf_hi[b] = std::numeric_limits<double>::quiet_NaN();
  const int n = io.n_nodes[b];
  const double T = (double)io.temperature[b];
  const int32_t* tok = io.tokens + (int64_t)b * N;
  const int32_t* par = io.parent + (int64_t)b * N;
  int32_t st = 0;
  if (!(T == 0.0 || (T >= (double)std::numeric_limits<float>::min() && std::isfinite(T))))
    st |= ST_TEMPERATURE;
  if (T > 0.0 && io.uniforms == nullptr) st |= ST_NO_UNIFORMS;
  std::vector<std::vector<int>> kids;
  if (n < 1 || n > N) {
    st |= ST_TREE;
  } else {
    kids.resize((size_t)n);
    if (par[0] != -1) st |= ST_TREE;
    for (int i = 1; i < n; ++i) {
      if (par[i] < 0 || par[i] >= i || tok[i] < 0 || tok[i] >= V) {
        st |= ST_TREE;
        continue;
      }
      for (int c : kids[(size_t)par[i]])
        if (tok[c] == tok[i]) st |= ST_TREE;
      kids[(size_t)par[i]].push_back(i);
    }
  }
  std::vector<std::vector<double>> rows;
  if (st == 0) {
    rows.resize((size_t)n);
    for (int i = 0; i < n; ++i) {
      load_row(io.logits, io.dtype, (int64_t)b * N + i, V, rows[(size_t)i]);
      if (!finite_row(rows[(size_t)i])) st |= ST_NONFINITE;
    }
  }
  if (st) {
    io.status[b] |= st;
    return;
  }
  const float* u = io.uniforms ? io.uniforms + (int64_t)b * N : nullptr;
  int cur = 0, depth = 0;
  std::vector<double> p, w;
  while (true) {
    const std::vector<int>& ch = kids[(size_t)cur];
    int next = -1;
    if (T == 0.0) {
      const int64_t a = argmax_lowest(rows[(size_t)cur]);
      for (int c : ch)
        if (tok[c] == a) next = c;
      if (next < 0) {
        out[depth] = (int32_t)a;
        onode[depth] = cur;
        io.num_emitted[b] = depth + 1;
        return;
      }
    } else {
      softmax_T(rows[(size_t)cur], T, p);
      if (!ch.empty()) {
        const double ut = (double)u[depth];
        double run = 0.0, g = std::numeric_limits<double>::infinity();
        for (int c : ch) {
          run += p[(size_t)tok[c]];
          g = std::min(g, std::fabs(ut - run));
          if (next < 0 && ut <= run) next = c;
        }
        gap[depth] = g;
      }
      if (next < 0) {
        // no child passed (or a leaf): draw from p without the children
        w = p;
        for (int c : ch) w[(size_t)tok[c]] = 0.0;
        double S = 0.0;
        for (double v : w) S += v;
        if (!(S > 0.0)) w = p;
        out[depth] = (int32_t)inv_cdf(w, (double)u[N - 1], &io.cdf_lo[b], &io.cdf_hi[b]);
        onode[depth] = cur;
        io.num_emitted[b] = depth + 1;
        return;
      }
    }
    out[depth] = tok[next];
    onode[depth] = next;
    cur = next;
    ++depth;
  }
}
}  // namespace

// ---------------------------------------------------------------------------
// C interface used by the Python test harness (ctypes).
// ---------------------------------------------------------------------------
extern "C" {

void* orc_sam_new(void) { return new OracleSAM(); }

int32_t orc_sam_draft_tree(void* h, int32_t K, int32_t M, int32_t* tok, int32_t* par,
                           int32_t* match_len) {
  return ((OracleSAM*)h)->draft_tree(K, M, tok, par, match_len);
}
void orc_sam_free(void* h) { delete (OracleSAM*)h; }

void orc_sam_extend(void* h, const int32_t* toks, int64_t n) {
  OracleSAM* s = (OracleSAM*)h;
  for (int64_t i = 0; i < n; ++i) s->extend(toks[i]);
}

int32_t orc_sam_draft(void* h, int32_t K, int32_t* draft, int32_t* match_len) {
  return ((OracleSAM*)h)->draft(K, draft, match_len);
}

int32_t orc_sam_last_walk_hops(void* h) { return ((OracleSAM*)h)->last_walk_hops; }
int64_t orc_sam_num_states(void* h) { return (int64_t)((OracleSAM*)h)->len.size(); }
int64_t orc_sam_num_edges(void* h) { return ((OracleSAM*)h)->num_edges(); }
int64_t orc_sam_length(void* h) { return (int64_t)((OracleSAM*)h)->text.size(); }
int32_t orc_sam_last(void* h) { return ((OracleSAM*)h)->last; }

// Advances B match states (state[b], mlen[b]) in the automaton h (the static
// automaton of [P4] §3) by tokens[b, 0..counts[b]) (row stride ld).
void orc_sam_match(void* h, int32_t B, int32_t* state, int32_t* mlen,
                   const int32_t* tokens, int64_t ld, const int32_t* counts) {
  const OracleSAM* s = (const OracleSAM*)h;
  for (int32_t b = 0; b < B; ++b)
    for (int32_t j = 0; j < counts[b]; ++j)
      s->match_step(state[b], mlen[b], tokens[(int64_t)b * ld + j]);
}

// Static drafts of B match states; returns nothing, writes draft [B,K] and
// draft_len [B].
void orc_sam_static_draft(void* h, int32_t B, const int32_t* state,
                          const int32_t* mlen, int32_t K, int32_t* draft,
                          int32_t* draft_len) {
  const OracleSAM* s = (const OracleSAM*)h;
  for (int32_t b = 0; b < B; ++b)
    draft_len[b] = s->draft_from(state[b], mlen[b], K, draft + (int64_t)b * K);
}

// Copies the structure out. edges receives [E,3] rows (src, token, dst) in
// ascending (src, token) order.
void orc_sam_export(void* h, int32_t* len, int32_t* link, int32_t* minend,
                    int32_t* edges) {
  const OracleSAM* s = (const OracleSAM*)h;
  int64_t e = 0;
  for (size_t i = 0; i < s->len.size(); ++i) {
    len[i] = s->len[i];
    link[i] = s->link[i];
    minend[i] = s->minend[i];
    for (const auto& kv : s->next[i]) {
      edges[3 * e + 0] = (int32_t)i;
      edges[3 * e + 1] = kv.first;
      edges[3 * e + 2] = kv.second;
      ++e;
    }
  }
}

// Verification of a batch. Sequences are independent; nthreads > 1 splits them
// over std::threads (the arithmetic of each sequence is unchanged).
// Log-probabilities of emitted tokens (for RL rollouts; [P1] §2.1 compares
// draft-token logprobs between decoding paths): for j < num_emitted[b],
// logprob[b, j] = log softmax(l_{b,j} / T)[out[b, j]] with T the sequence's
// temperature, or T = 1 for a greedy sequence (T = 0): the model's own
// log-probability. Entries past num_emitted are NaN.
void orc_logprobs(const void* logits, int32_t dtype, int32_t B, int32_t K,
                  int32_t V, const int32_t* out_tokens, const int32_t* num_emitted,
                  const float* temperature, double* logprob) {
  const int32_t R = K + 1;
  std::vector<double> row;
  for (int32_t b = 0; b < B; ++b) {
    const double T = temperature[b] > 0.0f ? (double)temperature[b] : 1.0;
    for (int32_t j = 0; j < R; ++j) {
      double& o = logprob[(int64_t)b * R + j];
      o = std::numeric_limits<double>::quiet_NaN();
      if (j >= num_emitted[b]) continue;
      const int32_t x = out_tokens[(int64_t)b * R + j];
      if (x < 0 || x >= V) continue;
      load_row(logits, dtype, (int64_t)b * R + j, V, row);
      double m = -std::numeric_limits<double>::infinity();
      for (int32_t i = 0; i < V; ++i) m = std::max(m, row[i] / T);
      double z = 0.0;
      for (int32_t i = 0; i < V; ++i) z += std::exp(row[i] / T - m);
      o = row[x] / T - m - std::log(z);
    }
  }
}

void orc_verify(const void* logits, int32_t dtype, int32_t B, int32_t K,
                int32_t V, const int32_t* draft, const int32_t* draft_len,
                const float* q, const float* temperature, const float* uniforms,
                int32_t* out_tokens, int32_t* num_emitted, double* p_draft,
                double* alpha, double* cdf_lo, double* cdf_hi, int32_t* status,
                const int32_t* top_k, const float* top_p, double* trunc_thr,
                double* trunc_margin, int32_t nthreads) {
  VerifyIO io{logits,      dtype,    B,          K,           V,
              draft,       draft_len, q,         temperature, uniforms,
              out_tokens,  num_emitted, p_draft, alpha,       cdf_lo,
              cdf_hi,      status,   top_k,     top_p,       trunc_thr,
              trunc_margin};
  if (nthreads <= 1) {
    for (int b = 0; b < B; ++b) verify_one(io, b);
    return;
  }
  std::vector<std::thread> ts;
  for (int t = 0; t < nthreads; ++t)
    ts.emplace_back([&, t] {
      for (int b = t; b < B; b += nthreads) verify_one(io, b);
    });
  for (auto& th : ts) th.join();
}

void orc_verify_tree(const void* logits, int32_t dtype, int32_t B, int32_t N,
                     int32_t V, const int32_t* tokens, const int32_t* parent,
                     const int32_t* n_nodes, const float* temperature,
                     const float* uniforms, int32_t* out_tokens, int32_t* out_nodes,
                     int32_t* num_emitted, double* gap, double* cdf_lo,
                     double* cdf_hi, int32_t* status, int32_t nthreads) {
  TreeIO io{logits,      dtype,    B,          N,         V,     tokens,
            parent,      n_nodes,  temperature, uniforms, out_tokens, out_nodes,
            num_emitted, gap,      cdf_lo,     cdf_hi,    status};
  if (nthreads <= 1) {
    for (int b = 0; b < B; ++b) verify_tree_one(io, b);
    return;
  }
  std::vector<std::thread> ts;
  for (int t = 0; t < nthreads; ++t)
    ts.emplace_back([&, t] {
      for (int b = t; b < B; b += nthreads) verify_tree_one(io, b);
    });
  for (auto& th : ts) th.join();
}

// One whole step for a batch of oracle automata: draft from each automaton,
// verify against the logits, extend each automaton by what was emitted.
// Used to time the oracle beside the GPU. draft/draft_len/match_len receive
// the drafts used. Sequences are independent: nthreads > 1 splits each of the
// three phases over std::threads (every automaton is touched by one thread).
void orc_step(void** sams, int32_t B, int32_t K, int32_t V, const void* logits,
              int32_t dtype, const float* temperature, const float* uniforms,
              int32_t* draft, int32_t* draft_len, int32_t* match_len,
              int32_t* out_tokens, int32_t* num_emitted, double* p_draft,
              double* alpha, double* cdf_lo, double* cdf_hi, int32_t* status,
              int32_t nthreads) {
  auto each = [&](auto fn) {
    if (nthreads <= 1) {
      for (int b = 0; b < B; ++b) fn(b);
      return;
    }
    std::vector<std::thread> ts;
    for (int t = 0; t < nthreads; ++t)
      ts.emplace_back([&, t] {
        for (int b = t; b < B; b += nthreads) fn(b);
      });
    for (auto& th : ts) th.join();
  };
  each([&](int b) {
    draft_len[b] =
        ((OracleSAM*)sams[b])->draft(K, draft + (int64_t)b * K, &match_len[b]);
  });
  orc_verify(logits, dtype, B, K, V, draft, draft_len, nullptr, temperature,
             uniforms, out_tokens, num_emitted, p_draft, alpha, cdf_lo, cdf_hi,
             status, nullptr, nullptr, nullptr, nullptr, nthreads);
  each([&](int b) {
    if (status[b]) return;
    OracleSAM* s = (OracleSAM*)sams[b];
    for (int j = 0; j < num_emitted[b]; ++j)
      s->extend(out_tokens[(int64_t)b * (K + 1) + j]);
  });
}

}  // extern "C"
