// Host planner of the fixed sparse candidate tree (see tree_plan.cpp).
#pragma once

#include <cstdint>
#include <memory>
#include <string>
#include <vector>

namespace medusa {

constexpr int kPlanMaxDepth = 16;
constexpr int kPlanMaxT = 256;
constexpr int64_t kPlanMaxCandidates = 4000000;
constexpr int kPlanRankCols = 16;   // columns of a rate table (ranks per head)

struct TreePlanHost {
  int T = 0;
  std::vector<int> parent, depth, rank;
};

// s_1 + s_1 s_2 + ... (candidates of the full tree), -1 on overflow.
int64_t full_tree_candidates(const int* k, int K);

// Cached, immutable plan; nullptr with *err set when the request is invalid.
std::shared_ptr<const TreePlanHost> get_tree_plan(const int* k, int K, int N, int decay_num,
                                                  int decay_den, std::string* err);

// The N candidates of largest path acceptance product under rates
// q[d * kPlanRankCols + r] in [0, 1] (checked by the caller); *expected =
// expected tokens per step.  N = -1 keeps every candidate.
std::shared_ptr<const TreePlanHost> plan_from_rates(const int* k, int K, int N, const double* q,
                                                    double* expected, std::string* err);

// A tree given as parent and rank per node: parent[0] = -1, 0 <= parent[i] <
// i, depths (derived) never decrease along the node order and stay <= K, rank
// below the head's shortlist size, one child per (parent, rank).
std::shared_ptr<const TreePlanHost> plan_from_tables(const int* k, int K, const int* parent,
                                                     const int* rank, int T, std::string* err);

}  // namespace medusa
