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

struct TreePlanHost {
  int T = 0;
  std::vector<int> parent, depth, rank;
};

// s_1 + s_1 s_2 + ... (candidates of the full tree), -1 on overflow.
int64_t full_tree_candidates(const int* k, int K);

// Cached, immutable plan; nullptr with *err set when the request is invalid.
std::shared_ptr<const TreePlanHost> get_tree_plan(const int* k, int K, int N, int decay_num,
                                                  int decay_den, std::string* err);

}  // namespace medusa
