// Host planner of the fixed sparse candidate tree (exact ranking).
//
// aicassindra.com "Medusa deep dive", "From top-k heads to a sparse candidate
// tree": the Cartesian product of the per-head shortlists is pruned ahead of
// time to a fixed sparse tree that gives more branches to confident, early
// heads.  Rule used here: candidate (r_1..r_D) scores
//     prod_{d=1..D} decay^d / (r_d + 1) = decay^(D(D+1)/2) / prod (r_d + 1)
// and the first N under (score desc, D asc, tuple asc) are kept.  A child
// scores strictly below its parent (decay < 1), so the kept set is closed
// under taking ancestors.  Scores are compared exactly: in the log domain when
// they are clearly apart, otherwise by cross-multiplied big integers, so ties
// at the cut-off (common: scores are ratios of small integers) are resolved by
// the stated order and not by rounding.
// Two more ways to a tree: the N candidates of largest acceptance product
// under measured per-rank rates (plan_from_rates), and caller-given node
// tables, validated (plan_from_tables).

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "tree_plan.h"

namespace medusa {

namespace {

// little-endian base-2^32 unsigned integer, only what the comparison needs
struct Big {
  std::vector<uint32_t> w{1};
  void mul(uint32_t f) {
    uint64_t carry = 0;
    for (auto& x : w) {
      uint64_t v = (uint64_t)x * f + carry;
      x = (uint32_t)v;
      carry = v >> 32;
    }
    if (carry) w.push_back((uint32_t)carry);
  }
  void mul_pow(uint32_t f, int e) {
    for (int i = 0; i < e; ++i) mul(f);
  }
};
int cmp(const Big& a, const Big& b) {
  size_t na = a.w.size(), nb = b.w.size();
  while (na > 1 && a.w[na - 1] == 0) --na;
  while (nb > 1 && b.w[nb - 1] == 0) --nb;
  if (na != nb) return na < nb ? -1 : 1;
  for (size_t i = na; i-- > 0;)
    if (a.w[i] != b.w[i]) return a.w[i] < b.w[i] ? -1 : 1;
  return 0;
}

struct Cand {
  uint8_t D;
  uint8_t r[kPlanMaxDepth];
  double logscore;   // fixed rule: log of the score
  double score;      // rates rule: the score itself
};

struct Ranker {
  uint32_t num, den;
  // exact: score(a) > score(b)?
  // num^Ea / (den^Ea * Pa)  vs  num^Eb / (den^Eb * Pb)
  int cmp_exact(const Cand& a, const Cand& b) const {
    const int Ea = a.D * (a.D + 1) / 2, Eb = b.D * (b.D + 1) / 2;
    const int e = std::min(Ea, Eb);
    Big lhs, rhs;   // lhs = num^(Ea-e) den^(Eb-e) Pb ; rhs = num^(Eb-e) den^(Ea-e) Pa
    lhs.mul_pow(num, Ea - e);
    lhs.mul_pow(den, Eb - e);
    for (int d = 0; d < b.D; ++d) lhs.mul(b.r[d] + 1u);
    rhs.mul_pow(num, Eb - e);
    rhs.mul_pow(den, Ea - e);
    for (int d = 0; d < a.D; ++d) rhs.mul(a.r[d] + 1u);
    return cmp(lhs, rhs);   // > 0: score(a) > score(b)
  }
  bool before(const Cand& a, const Cand& b) const {
    const double diff = a.logscore - b.logscore;
    int c;
    if (std::fabs(diff) > 1e-9) c = diff > 0 ? 1 : -1;
    else c = cmp_exact(a, b);
    if (c != 0) return c > 0;
    if (a.D != b.D) return a.D < b.D;
    return std::lexicographical_compare(a.r, a.r + a.D, b.r, b.r + b.D);
  }
};

bool tuple_less(const Cand& a, const Cand& b) {
  if (a.D != b.D) return a.D < b.D;
  return std::lexicographical_compare(a.r, a.r + a.D, b.r, b.r + b.D);
}

std::string key_of(const int* k, int K, int N, int dn, int dd) {
  std::string s;
  for (int i = 0; i < K; ++i) s += std::to_string(k[i]) + ",";
  s += "|" + std::to_string(N) + "|" + std::to_string(dn) + "/" + std::to_string(dd);
  return s;
}

std::mutex g_mu;
std::map<std::string, std::shared_ptr<const TreePlanHost>> g_cache;

// Node tables of a kept candidate set: root first, then by depth and rank
// tuple (so a parent precedes its children); nullptr if the set is not closed
// under taking ancestors.
std::shared_ptr<TreePlanHost> tables_of(std::vector<Cand>& kept, std::string* err) {
  std::sort(kept.begin(), kept.end(), tuple_less);
  auto plan = std::make_shared<TreePlanHost>();
  const int T = (int)kept.size() + 1;
  plan->T = T;
  plan->parent.assign(T, -1);
  plan->depth.assign(T, 0);
  plan->rank.assign(T, -1);
  std::map<std::vector<int>, int> index;
  index[{}] = 0;
  for (int i = 1; i < T; ++i) {
    const Cand& c = kept[i - 1];
    std::vector<int> t(c.r, c.r + c.D);
    index[t] = i;
    std::vector<int> par(t.begin(), t.end() - 1);
    auto it = index.find(par);
    if (it == index.end()) {
      *err = "tree: kept set is not closed under ancestors";
      return nullptr;
    }
    plan->parent[i] = it->second;
    plan->depth[i] = c.D;
    plan->rank[i] = c.r[c.D - 1];
  }
  return plan;
}

}  // namespace

int64_t full_tree_candidates(const int* k, int K) {
  int64_t total = 0, prod = 1;
  for (int i = 0; i < K; ++i) {
    if (prod > (int64_t)1 << 40) return -1;
    prod *= k[i];
    total += prod;
  }
  return total;
}

std::shared_ptr<const TreePlanHost> get_tree_plan(const int* k, int K, int N, int dn, int dd,
                                                  std::string* err) {
  const std::string key = key_of(k, K, N, dn, dd);
  {
    std::lock_guard<std::mutex> g(g_mu);
    auto it = g_cache.find(key);
    if (it != g_cache.end()) return it->second;
  }
  const int64_t total = full_tree_candidates(k, K);
  if (total < 0 || total > kPlanMaxCandidates) {
    *err = "tree: too many candidate tuples to rank (" + std::to_string(total) + ")";
    return nullptr;
  }
  const int64_t keep = N < 0 ? total : N;
  if (keep > total) {
    *err = "tree: N exceeds the number of candidate tuples";
    return nullptr;
  }
  if (keep + 1 > kPlanMaxT) {
    *err = "tree: N + 1 exceeds the node limit";
    return nullptr;
  }
  std::vector<Cand> all;
  all.reserve((size_t)total);
  const double ld = std::log((double)dn / (double)dd);
  for (int D = 1; D <= K; ++D) {
    Cand c{};
    c.D = (uint8_t)D;
    std::vector<int> r(D, 0);
    while (true) {
      double ls = 0.5 * D * (D + 1) * ld;
      for (int d = 0; d < D; ++d) {
        c.r[d] = (uint8_t)r[d];
        ls -= std::log((double)(r[d] + 1));
      }
      c.logscore = ls;
      all.push_back(c);
      int d = D - 1;
      while (d >= 0 && ++r[d] == k[d]) r[d--] = 0;
      if (d < 0) break;
    }
  }
  Ranker rk{(uint32_t)dn, (uint32_t)dd};
  if (keep < total) {
    std::sort(all.begin(), all.end(), [&](const Cand& a, const Cand& b) { return rk.before(a, b); });
    all.resize((size_t)keep);
  }
  auto plan = tables_of(all, err);
  if (!plan) return nullptr;
  std::lock_guard<std::mutex> g(g_mu);
  auto it = g_cache.find(key);
  if (it != g_cache.end()) return it->second;
  g_cache[key] = plan;
  return plan;
}

// aicassindra.com "Medusa deep dive", "From top-k heads to a sparse candidate
// tree" (the tree shape is a tuned budget) and "What it costs on a CPU-bound
// SLM" (expected acceptance length multiplies throughput).  Candidate
// (r_1..r_D) scores q[0][r_1] * q[1][r_2] * ... (float64, from depth 1 down):
// the probability that its path is accepted when heads are independent given
// the hidden state.  The N best under (score desc, D asc, tuple asc) are kept;
// q <= 1 keeps a child's score at or below its parent's, so the kept set is
// closed under ancestors.  Expected tokens = 1 + the kept scores summed in node
// order.  Not cached (rates change as they are measured).
std::shared_ptr<const TreePlanHost> plan_from_rates(const int* k, int K, int N, const double* q,
                                                    double* expected, std::string* err) {
  const int64_t total = full_tree_candidates(k, K);
  if (total < 0 || total > kPlanMaxCandidates) {
    *err = "tree: too many candidate tuples to rank (" + std::to_string(total) + ")";
    return nullptr;
  }
  const int64_t keep = N < 0 ? total : N;
  if (keep > total) {
    *err = "tree: N exceeds the number of candidate tuples";
    return nullptr;
  }
  if (keep + 1 > kPlanMaxT) {
    *err = "tree: N + 1 exceeds the node limit";
    return nullptr;
  }
  std::vector<Cand> all;
  all.reserve((size_t)total);
  for (int D = 1; D <= K; ++D) {
    Cand c{};
    c.D = (uint8_t)D;
    std::vector<int> r(D, 0);
    while (true) {
      double sc = 1.0;
      for (int d = 0; d < D; ++d) {
        c.r[d] = (uint8_t)r[d];
        sc = sc * q[d * kPlanRankCols + r[d]];
      }
      c.score = sc;
      all.push_back(c);
      int d = D - 1;
      while (d >= 0 && ++r[d] == k[d]) r[d--] = 0;
      if (d < 0) break;
    }
  }
  if (keep < total) {
    std::sort(all.begin(), all.end(), [](const Cand& a, const Cand& b) {
      if (a.score != b.score) return a.score > b.score;
      return tuple_less(a, b);
    });
    all.resize((size_t)keep);
  }
  auto plan = tables_of(all, err);
  if (!plan) return nullptr;
  // expected tokens in node order (the root contributes the 1)
  double e = 1.0;
  std::vector<double> node_score(plan->T, 1.0);
  for (int i = 1; i < plan->T; ++i) {
    node_score[i] = node_score[plan->parent[i]] * q[(plan->depth[i] - 1) * kPlanRankCols + plan->rank[i]];
    e = e + node_score[i];
  }
  if (expected) *expected = e;
  return plan;
}

std::shared_ptr<const TreePlanHost> plan_from_tables(const int* k, int K, const int* parent,
                                                     const int* rank, int T, std::string* err) {
  if (T < 1 || T > kPlanMaxT) {
    *err = "tree: T must be in [1, 256]";
    return nullptr;
  }
  if (parent[0] != -1) {
    *err = "tree: node 0 must be the root (parent -1)";
    return nullptr;
  }
  auto plan = std::make_shared<TreePlanHost>();
  plan->T = T;
  plan->parent.assign(T, -1);
  plan->depth.assign(T, 0);
  plan->rank.assign(T, -1);
  std::vector<uint32_t> seen((size_t)T * 16, 0);   // (parent, rank) taken
  for (int i = 1; i < T; ++i) {
    const int p = parent[i], r = rank[i];
    if (p < 0 || p >= i) {
      *err = "tree: parent[i] must lie in [0, i)";
      return nullptr;
    }
    const int D = plan->depth[p] + 1;
    if (D > K || r < 0 || r >= k[D - 1]) {
      *err = "tree: node deeper than K or rank outside the head's shortlist";
      return nullptr;
    }
    if (D < plan->depth[i - 1]) {
      *err = "tree: depths must not decrease along the node order";
      return nullptr;
    }
    if (seen[(size_t)p * 16 + r]++) {
      *err = "tree: two children of one node share a rank";
      return nullptr;
    }
    plan->parent[i] = p;
    plan->depth[i] = D;
    plan->rank[i] = r;
  }
  return plan;
}

}  // namespace medusa
