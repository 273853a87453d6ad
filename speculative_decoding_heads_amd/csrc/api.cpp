// C ABI of libmedusa.so (declared in include/medusa.h): argument validation,
// workspace sizing and dispatch to the HIP kernels.  Host code only.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <string>

#include "../../include/medusa.h"
#include "kernels.h"
#include "tree_plan.h"

using namespace medusa;

namespace {

thread_local std::string g_err;

int fail(int status, const std::string& msg) {
  g_err = msg;
  return status;
}
int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MEDUSA_OK;
  return fail(MEDUSA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool dtype_ok(int32_t dt) { return dt == MEDUSA_F32 || dt == MEDUSA_BF16; }
size_t elem_size(int32_t dt) { return dt == MEDUSA_BF16 ? 2 : 4; }
size_t round_up(size_t x) { return (x + 255) & ~(size_t)255; }
hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

int check_k(const int32_t* k_host, int32_t K, int32_t kmax_or_zero) {
  if (!k_host) return fail(MEDUSA_ERR_ARG, "k_host is NULL");
  if (K < 1 || K > MEDUSA_MAX_HEADS) return fail(MEDUSA_ERR_ARG, "K out of range [1, 16]");
  for (int i = 0; i < K; ++i) {
    if (k_host[i] < 1 || k_host[i] > MEDUSA_MAX_K)
      return fail(MEDUSA_ERR_ARG, "k_host[i] out of range [1, 16]");
    if (kmax_or_zero > 0 && k_host[i] > kmax_or_zero)
      return fail(MEDUSA_ERR_ARG, "k_host[i] exceeds kmax");
  }
  return MEDUSA_OK;
}

}  // namespace

extern "C" {

int medusa_abi_version(void) { return MEDUSA_ABI_VERSION; }

const char* medusa_status_str(int status) {
  switch (status) {
    case MEDUSA_OK: return "ok";
    case MEDUSA_ERR_ARG: return "invalid argument";
    case MEDUSA_ERR_UNSUPPORTED: return "unsupported configuration";
    case MEDUSA_ERR_WORKSPACE: return "workspace missing or too small";
    case MEDUSA_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

const char* medusa_last_error(void) { return g_err.c_str(); }

// ------------------------------------------------------------------- heads
size_t medusa_heads_workspace(int64_t rows, int32_t H, int32_t n_heads, int32_t include_base,
                              int32_t dtype) {
  if (rows <= 0 || H <= 0 || n_heads <= 0 || !dtype_ok(dtype)) return 0;
  const int R = include_base + n_heads;
  return round_up((size_t)rows * R * H * elem_size(dtype));
}

int medusa_heads(const void* x, int64_t rows, int32_t H, const void* W, int32_t n_heads,
                 const void* LM, int32_t V, int32_t dtype, int32_t include_base, void* u_out,
                 float* logits, void* ws, size_t ws_bytes, void* stream) {
  if (rows < 0) return fail(MEDUSA_ERR_ARG, "rows < 0");
  if (!dtype_ok(dtype)) return fail(MEDUSA_ERR_ARG, "dtype must be MEDUSA_F32 or MEDUSA_BF16");
  if (H <= 0 || V <= 0) return fail(MEDUSA_ERR_ARG, "H and V must be positive");
  if (n_heads < 0 || n_heads > MEDUSA_MAX_HEADS) return fail(MEDUSA_ERR_ARG, "n_heads out of range");
  if (include_base != 0 && include_base != 1) return fail(MEDUSA_ERR_ARG, "include_base must be 0 or 1");
  const int R = include_base + n_heads;
  if (R < 1) return fail(MEDUSA_ERR_ARG, "no output head requested");
  if (rows == 0) return MEDUSA_OK;
  if (!x || !LM || !logits) return fail(MEDUSA_ERR_ARG, "x, LM and logits must be non-NULL");
  if (n_heads > 0 && !W) return fail(MEDUSA_ERR_ARG, "W is NULL with n_heads > 0");
  if (rows * R > INT32_MAX / 2 || (int64_t)n_heads * H > INT32_MAX / 2)
    return fail(MEDUSA_ERR_UNSUPPORTED, "too many rows");
  if (dtype == MEDUSA_BF16) {
    if (H % 128 != 0) return fail(MEDUSA_ERR_UNSUPPORTED, "bf16 heads need H % 128 == 0");
    if (!aligned16(x) || !aligned16(LM) || (W && !aligned16(W)) || (u_out && !aligned16(u_out)))
      return fail(MEDUSA_ERR_ARG, "bf16 operands must be 16-byte aligned");
  }
  hipStream_t st = as_stream(stream);
  const void* gemm_x = x;
  if (n_heads > 0 || u_out) {
    void* u = u_out;
    if (!u) {
      const size_t need = medusa_heads_workspace(rows, H, n_heads, include_base, dtype);
      if (!ws || ws_bytes < need) return fail(MEDUSA_ERR_WORKSPACE, "heads: workspace too small");
      u = ws;
    }
    int s = hip_status(run_heads_hidden(x, (int)rows, H, W, n_heads, dtype, u, R, include_base, st),
                       "heads hidden");
    if (s) return s;
    gemm_x = u;
  }
  // Head rows walk the LM weights' K chunks backwards, verify rows (n_heads =
  // 0) forwards: a step's two LM passes then each start on what the other
  // read last, which the last-level cache still holds.
  return hip_status(run_lm_logits(gemm_x, (int)(rows * R), H, LM, V, dtype, logits, st,
                                  n_heads > 0),
                    "LM projection");
}

int medusa_heads_hidden(const void* x, int64_t rows, int32_t H, const void* W, int32_t n_heads,
                        int32_t dtype, int32_t include_base, void* u_out, void* stream) {
  if (rows < 0) return fail(MEDUSA_ERR_ARG, "rows < 0");
  if (!dtype_ok(dtype)) return fail(MEDUSA_ERR_ARG, "dtype must be MEDUSA_F32 or MEDUSA_BF16");
  if (H <= 0) return fail(MEDUSA_ERR_ARG, "H must be positive");
  if (n_heads < 1 || n_heads > MEDUSA_MAX_HEADS) return fail(MEDUSA_ERR_ARG, "n_heads out of range [1, 16]");
  if (include_base != 0 && include_base != 1) return fail(MEDUSA_ERR_ARG, "include_base must be 0 or 1");
  const int R = include_base + n_heads;
  if (rows == 0) return MEDUSA_OK;
  if (!x || !W || !u_out) return fail(MEDUSA_ERR_ARG, "x, W and u_out must be non-NULL");
  if (rows * R > INT32_MAX / 2 || (int64_t)n_heads * H > INT32_MAX / 2)
    return fail(MEDUSA_ERR_UNSUPPORTED, "too many rows");
  if (dtype == MEDUSA_BF16) {
    if (H % 128 != 0) return fail(MEDUSA_ERR_UNSUPPORTED, "bf16 heads need H % 128 == 0");
    if (!aligned16(x) || !aligned16(W) || !aligned16(u_out))
      return fail(MEDUSA_ERR_ARG, "bf16 operands must be 16-byte aligned");
  }
  return hip_status(run_heads_hidden(x, (int)rows, H, W, n_heads, dtype, u_out, R, include_base,
                                     as_stream(stream)),
                    "heads hidden");
}

int medusa_lm_logits(const void* x, int64_t rows, int32_t H, const void* LM, int32_t V,
                     int32_t dtype, int32_t reverse_k, float* logits, void* stream) {
  if (rows < 0) return fail(MEDUSA_ERR_ARG, "rows < 0");
  if (!dtype_ok(dtype)) return fail(MEDUSA_ERR_ARG, "dtype must be MEDUSA_F32 or MEDUSA_BF16");
  if (H <= 0 || V <= 0) return fail(MEDUSA_ERR_ARG, "H and V must be positive");
  if (reverse_k != 0 && reverse_k != 1) return fail(MEDUSA_ERR_ARG, "reverse_k must be 0 or 1");
  if (rows == 0) return MEDUSA_OK;
  if (!x || !LM || !logits) return fail(MEDUSA_ERR_ARG, "x, LM and logits must be non-NULL");
  if (rows > INT32_MAX / 2) return fail(MEDUSA_ERR_UNSUPPORTED, "too many rows");
  if (dtype == MEDUSA_BF16) {
    if (H % 128 != 0) return fail(MEDUSA_ERR_UNSUPPORTED, "bf16 rows need H % 128 == 0");
    if (!aligned16(x) || !aligned16(LM)) return fail(MEDUSA_ERR_ARG, "bf16 operands must be 16-byte aligned");
  }
  return hip_status(run_lm_logits(x, (int)rows, H, LM, V, dtype, logits, as_stream(stream),
                                  reverse_k == 1),
                    "LM projection");
}

// ------------------------------------------------------------------- MTP-style heads
static int mtp_check(int32_t b, int32_t H, int32_t K, int32_t F, int32_t nq, int32_t nkv, int32_t d,
              int32_t Pmax, int32_t V) {
  if (b < 0) return fail(MEDUSA_ERR_ARG, "b < 0");
  if (K < 1 || K > MEDUSA_MAX_HEADS) return fail(MEDUSA_ERR_ARG, "K out of range [1, 16]");
  if (H <= 0 || F <= 0 || V <= 0) return fail(MEDUSA_ERR_ARG, "H, F and V must be positive");
  if (nq < 1 || nkv < 1 || nq % nkv != 0) return fail(MEDUSA_ERR_ARG, "need nq % nkv == 0");
  if (d != 64 && d != 128) return fail(MEDUSA_ERR_UNSUPPORTED, "MTP attention supports d = 64 or 128");
  if (H % 128 != 0 || F % 128 != 0 || (nq * d) % 128 != 0)
    return fail(MEDUSA_ERR_UNSUPPORTED, "MTP heads need H, F and nq * d multiples of 128");
  if (Pmax < 1) return fail(MEDUSA_ERR_ARG, "Pmax must be positive");
  if ((int64_t)b * K > INT32_MAX / 4 || (int64_t)b * (K + 1) > INT32_MAX / 4)
    return fail(MEDUSA_ERR_UNSUPPORTED, "too many rows");
  if ((int64_t)(nq + 2 * nkv) * d > INT32_MAX / 4 || (int64_t)2 * F > INT32_MAX / 4)
    return fail(MEDUSA_ERR_UNSUPPORTED, "layer too wide");
  return MEDUSA_OK;
}

size_t medusa_mtp_workspace(int32_t b, int32_t H, int32_t K, int32_t F, int32_t nq, int32_t nkv,
                            int32_t d, int32_t Pmax, int32_t keep_u) {
  if (b <= 0 || K < 1 || H <= 0 || F <= 0 || nq < 1 || nkv < 1 || nq % nkv || Pmax < 1) return 0;
  if (d != 64 && d != 128) return 0;
  return round_up(mtp_layout(b, H, K, F, nq, nkv, d, Pmax, keep_u == 0).bytes);
}

int medusa_mtp_draft(const void* h, int32_t b, int32_t H, int32_t K, const void* g1,
                     const void* Wqkv, const void* Wo, const void* g2, const void* Wgu,
                     const void* Wd, int32_t F, float eps, void* Kh, void* Vh,
                     const int32_t* seq_len, int32_t nq, int32_t nkv, int32_t d, int32_t Pmax,
                     const void* LM, int32_t V, void* u_out, float* logits, void* ws,
                     size_t ws_bytes, void* stream) {
  if (int s = mtp_check(b, H, K, F, nq, nkv, d, Pmax, V)) return s;
  if (!(eps >= 0.f && std::isfinite(eps))) return fail(MEDUSA_ERR_ARG, "eps must be finite and >= 0");
  if (b == 0) return MEDUSA_OK;
  if (!h || !g1 || !Wqkv || !Wo || !g2 || !Wgu || !Wd || !Kh || !Vh || !seq_len || !LM || !logits)
    return fail(MEDUSA_ERR_ARG, "NULL pointer");
  const void* al[] = {h, g1, Wqkv, Wo, g2, Wgu, Wd, Kh, Vh, LM, u_out, ws};
  for (const void* p : al)
    if (p && !aligned16(p)) return fail(MEDUSA_ERR_ARG, "MTP operands must be 16-byte aligned");
  const size_t need = medusa_mtp_workspace(b, H, K, F, nq, nkv, d, Pmax, u_out != nullptr);
  if (!ws || ws_bytes < need) return fail(MEDUSA_ERR_WORKSPACE, "mtp_draft: workspace too small");
  MtpArgs a{h, b, H, K, F, g1, Wqkv, Wo, g2, Wgu, Wd, eps, Kh, Vh, seq_len, nq, nkv, d, Pmax, LM, V};
  return hip_status(run_mtp_draft(a, u_out, logits, ws, as_stream(stream)), "mtp_draft");
}

// ------------------------------------------------------------------- verify logits + partials
size_t medusa_verify_workspace(int64_t rows, int32_t H, int32_t V, int32_t dtype, int32_t mode) {
  if (rows <= 0 || H <= 0 || V <= 0 || !dtype_ok(dtype)) return 0;
  if (mode != MEDUSA_GREEDY && mode != MEDUSA_TYPICAL && mode != MEDUSA_REJECT) return 0;
  if (rows > INT32_MAX / 2) return 0;
  // rejection sampling works from the same tempered statistics as typical
  return round_up(verify_workspace((int)rows, V, H, dtype, mode == MEDUSA_GREEDY ? kGreedy : kTypical));
}

int medusa_verify_logits(const void* x, int64_t rows, int32_t H, const void* LM, int32_t V,
                         int32_t dtype, int32_t mode, float temperature, float* logits, void* ws,
                         size_t ws_bytes, void* stream) {
  if (rows < 0) return fail(MEDUSA_ERR_ARG, "rows < 0");
  if (!dtype_ok(dtype)) return fail(MEDUSA_ERR_ARG, "dtype must be MEDUSA_F32 or MEDUSA_BF16");
  if (H <= 0 || V <= 0) return fail(MEDUSA_ERR_ARG, "H and V must be positive");
  if (mode != MEDUSA_GREEDY && mode != MEDUSA_TYPICAL && mode != MEDUSA_REJECT)
    return fail(MEDUSA_ERR_ARG, "mode must be GREEDY, TYPICAL or REJECT");
  if (mode != MEDUSA_GREEDY && !(temperature > 0.f && std::isfinite(temperature)))
    return fail(MEDUSA_ERR_ARG, "temperature must be positive and finite");
  if (rows == 0) return MEDUSA_OK;
  if (!x || !LM || !logits) return fail(MEDUSA_ERR_ARG, "x, LM and logits must be non-NULL");
  if (rows > INT32_MAX / 2) return fail(MEDUSA_ERR_UNSUPPORTED, "too many rows");
  if (dtype == MEDUSA_BF16) {
    if (H % 128 != 0) return fail(MEDUSA_ERR_UNSUPPORTED, "bf16 rows need H % 128 == 0");
    if (!aligned16(x) || !aligned16(LM)) return fail(MEDUSA_ERR_ARG, "bf16 operands must be 16-byte aligned");
  }
  const size_t need = medusa_verify_workspace(rows, H, V, dtype, mode);
  if (!ws || ws_bytes < need) return fail(MEDUSA_ERR_WORKSPACE, "verify: workspace too small");
  if (!aligned16(ws)) return fail(MEDUSA_ERR_ARG, "workspace must be 16-byte aligned");
  const float tmp = mode != MEDUSA_GREEDY ? temperature : 1.0f;
  return hip_status(run_verify_logits(x, (int)rows, H, LM, V, dtype, logits,
                                      mode == MEDUSA_GREEDY ? kGreedy : kTypical, tmp, ws,
                                      as_stream(stream)),
                    "verify logits");
}

// ------------------------------------------------------------------- top-k
size_t medusa_topk_workspace(int32_t b, int32_t K, int32_t V, int32_t kmax) {
  if (b <= 0 || K <= 0 || V <= 0 || kmax <= 0) return 0;
  const size_t n = topk_workspace(b, K, V, kmax);
  return n ? round_up(n) : 0;
}

int medusa_topk(const float* logits, int32_t b, int32_t K, int32_t V, const int32_t* k_host,
                int32_t kmax, int32_t root_mode, float temperature, uint64_t seed, uint64_t step,
                int32_t* root, int32_t* idx, float* val, void* ws, size_t ws_bytes,
                void* stream) {
  if (b < 0) return fail(MEDUSA_ERR_ARG, "b < 0");
  if (V <= 0) return fail(MEDUSA_ERR_ARG, "V must be positive");
  if (kmax < 1 || kmax > MEDUSA_MAX_K) return fail(MEDUSA_ERR_ARG, "kmax out of range [1, 16]");
  if (int s = check_k(k_host, K, kmax)) return s;
  for (int i = 0; i < K; ++i)
    if (k_host[i] > V) return fail(MEDUSA_ERR_ARG, "k_i exceeds V");
  if (root_mode != MEDUSA_GREEDY && root_mode != MEDUSA_TYPICAL && root_mode != MEDUSA_ROOT_GIVEN)
    return fail(MEDUSA_ERR_ARG, "root_mode must be GREEDY, TYPICAL or ROOT_GIVEN");
  if (root_mode == MEDUSA_TYPICAL && !(temperature > 0.f && std::isfinite(temperature)))
    return fail(MEDUSA_ERR_ARG, "temperature must be positive and finite");
  if (b == 0) return MEDUSA_OK;
  if (!logits || !root || !idx || !val) return fail(MEDUSA_ERR_ARG, "NULL pointer");
  if ((int64_t)b * (K + 1) > 65535) return fail(MEDUSA_ERR_UNSUPPORTED, "b * (K+1) > 65535");
  const size_t need = medusa_topk_workspace(b, K, V, kmax);
  if (need && (!ws || ws_bytes < need)) return fail(MEDUSA_ERR_WORKSPACE, "topk: workspace too small");
  if (!aligned16(ws)) return fail(MEDUSA_ERR_ARG, "workspace must be 16-byte aligned");
  TopkArgs a{};
  a.b = b; a.K = K; a.V = V; a.kmax = kmax; a.root_mode = root_mode;
  a.temperature = temperature; a.seed = seed; a.step = step;
  for (int i = 0; i < K; ++i) a.k[i] = k_host[i];
  return hip_status(run_topk(logits, a, root, idx, val, ws, as_stream(stream)), "topk");
}

// ------------------------------------------------------------------- tree
static int plan_for(const int32_t* k_host, int32_t K, int32_t N, int32_t dn, int32_t dd,
                    std::shared_ptr<const TreePlanHost>* out) {
  if (int s = check_k(k_host, K, 0)) return s;
  if (N < -1) return fail(MEDUSA_ERR_ARG, "N must be >= 0, or -1 for the full tree");
  if (dn <= 0 || dd <= 0 || dn >= dd || dd > 1000000)
    return fail(MEDUSA_ERR_ARG, "decay must be a fraction in (0, 1)");
  const int64_t total = full_tree_candidates(k_host, K);
  if (N > total && total >= 0) return fail(MEDUSA_ERR_ARG, "N exceeds the candidate count");
  const int64_t keep = N < 0 ? total : N;
  if (keep < 0 || keep + 1 > MEDUSA_MAX_T) return fail(MEDUSA_ERR_UNSUPPORTED, "tree exceeds 256 nodes");
  std::string err;
  auto p = get_tree_plan(k_host, K, N, dn, dd, &err);
  if (!p) return fail(MEDUSA_ERR_UNSUPPORTED, err);
  *out = p;
  return MEDUSA_OK;
}

int medusa_tree_plan(const int32_t* k_host, int32_t K, int32_t N, int32_t decay_num,
                     int32_t decay_den, int32_t* parent, int32_t* depth, int32_t* rank,
                     int32_t T_cap, int32_t* T_out) {
  std::shared_ptr<const TreePlanHost> p;
  if (int s = plan_for(k_host, K, N, decay_num, decay_den, &p)) return s;
  if (T_out) *T_out = p->T;
  if (!parent && !depth && !rank) return MEDUSA_OK;
  if (T_cap < p->T) return fail(MEDUSA_ERR_ARG, "T_cap smaller than the tree");
  for (int i = 0; i < p->T; ++i) {
    if (parent) parent[i] = p->parent[i];
    if (depth) depth[i] = p->depth[i];
    if (rank) rank[i] = p->rank[i];
  }
  return MEDUSA_OK;
}

int medusa_build_tree(const int32_t* k_host, int32_t K, int32_t N, int32_t decay_num,
                      int32_t decay_den, const int32_t* root, const int32_t* idx, int32_t b,
                      int32_t kmax, const int32_t* seq_len, int32_t* tokens, int32_t* pos,
                      int32_t* parent, int32_t* depth, uint64_t* anc, int32_t anc_words,
                      void* stream) {
  std::shared_ptr<const TreePlanHost> p;
  if (int s = plan_for(k_host, K, N, decay_num, decay_den, &p)) return s;
  if (kmax < 1 || kmax > MEDUSA_MAX_K) return fail(MEDUSA_ERR_ARG, "kmax out of range [1, 16]");
  for (int i = 0; i < K; ++i)
    if (k_host[i] > kmax) return fail(MEDUSA_ERR_ARG, "k_i exceeds kmax");
  if (b < 0) return fail(MEDUSA_ERR_ARG, "b < 0");
  if (anc_words < (p->T + 63) / 64) return fail(MEDUSA_ERR_ARG, "anc_words < ceil(T / 64)");
  if (b == 0) return MEDUSA_OK;
  if (!root || !idx || !seq_len || !tokens || !pos || !parent || !depth || !anc)
    return fail(MEDUSA_ERR_ARG, "NULL pointer");
  TreeDev t{};
  t.T = p->T; t.K = K; t.kmax = kmax; t.anc_words = anc_words;
  for (int i = 0; i < p->T; ++i) {
    t.parent[i] = (int16_t)p->parent[i];
    t.depth[i] = (uint8_t)p->depth[i];
    t.rank[i] = (uint8_t)(p->rank[i] < 0 ? 0 : p->rank[i]);
  }
  return hip_status(run_build_tree(t, root, idx, b, seq_len, tokens, pos, parent, depth, anc,
                                   as_stream(stream)),
                    "build_tree");
}

// ------------------------------------------------------------------- top-k + tree, one launch
static int topk_tree_common(const float* logits, int32_t b, int32_t K, int32_t V,
                            const int32_t* k_host, int32_t kmax, int32_t root_mode,
                            float temperature, uint64_t seed, uint64_t step,
                            const int32_t* seq_len, int32_t* root, int32_t* idx, float* val,
                            int32_t* tokens, int32_t* pos, int32_t* parent, int32_t* depth,
                            uint64_t* anc, int32_t anc_words, void* ws, size_t ws_bytes,
                            void* stream, const std::shared_ptr<const TreePlanHost>& p);

static int topk_tree_args(int32_t b, int32_t K, int32_t V, const int32_t* k_host, int32_t kmax,
                          int32_t root_mode, float temperature) {
  if (b < 0) return fail(MEDUSA_ERR_ARG, "b < 0");
  if (V <= 0) return fail(MEDUSA_ERR_ARG, "V must be positive");
  if (kmax < 1 || kmax > MEDUSA_MAX_K) return fail(MEDUSA_ERR_ARG, "kmax out of range [1, 16]");
  if (int s = check_k(k_host, K, kmax)) return s;
  for (int i = 0; i < K; ++i)
    if (k_host[i] > V) return fail(MEDUSA_ERR_ARG, "k_i exceeds V");
  if (root_mode != MEDUSA_GREEDY && root_mode != MEDUSA_TYPICAL && root_mode != MEDUSA_ROOT_GIVEN)
    return fail(MEDUSA_ERR_ARG, "root_mode must be GREEDY, TYPICAL or ROOT_GIVEN");
  if (root_mode == MEDUSA_TYPICAL && !(temperature > 0.f && std::isfinite(temperature)))
    return fail(MEDUSA_ERR_ARG, "temperature must be positive and finite");
  return MEDUSA_OK;
}

int medusa_topk_tree(const float* logits, int32_t b, int32_t K, int32_t V, const int32_t* k_host,
                     int32_t kmax, int32_t N, int32_t decay_num, int32_t decay_den,
                     int32_t root_mode, float temperature, uint64_t seed, uint64_t step,
                     const int32_t* seq_len, int32_t* root, int32_t* idx, float* val,
                     int32_t* tokens, int32_t* pos, int32_t* parent, int32_t* depth, uint64_t* anc,
                     int32_t anc_words, void* ws, size_t ws_bytes, void* stream) {
  if (int s = topk_tree_args(b, K, V, k_host, kmax, root_mode, temperature)) return s;
  std::shared_ptr<const TreePlanHost> p;
  if (int s = plan_for(k_host, K, N, decay_num, decay_den, &p)) return s;
  return topk_tree_common(logits, b, K, V, k_host, kmax, root_mode, temperature, seed, step,
                          seq_len, root, idx, val, tokens, pos, parent, depth, anc, anc_words, ws,
                          ws_bytes, stream, p);
}

int medusa_topk_tree_tables(const float* logits, int32_t b, int32_t K, int32_t V,
                            const int32_t* k_host, int32_t kmax, const int32_t* plan_parent,
                            const int32_t* plan_rank, int32_t T, int32_t root_mode,
                            float temperature, uint64_t seed, uint64_t step,
                            const int32_t* seq_len, int32_t* root, int32_t* idx, float* val,
                            int32_t* tokens, int32_t* pos, int32_t* parent, int32_t* depth,
                            uint64_t* anc, int32_t anc_words, void* ws, size_t ws_bytes,
                            void* stream) {
  if (int s = topk_tree_args(b, K, V, k_host, kmax, root_mode, temperature)) return s;
  if (!plan_parent || !plan_rank) return fail(MEDUSA_ERR_ARG, "plan tables are NULL");
  std::string err;
  auto p = plan_from_tables(k_host, K, plan_parent, plan_rank, T, &err);
  if (!p) return fail(MEDUSA_ERR_ARG, err);
  return topk_tree_common(logits, b, K, V, k_host, kmax, root_mode, temperature, seed, step,
                          seq_len, root, idx, val, tokens, pos, parent, depth, anc, anc_words, ws,
                          ws_bytes, stream, p);
}

static int topk_tree_common(const float* logits, int32_t b, int32_t K, int32_t V,
                            const int32_t* k_host, int32_t kmax, int32_t root_mode,
                            float temperature, uint64_t seed, uint64_t step,
                            const int32_t* seq_len, int32_t* root, int32_t* idx, float* val,
                            int32_t* tokens, int32_t* pos, int32_t* parent, int32_t* depth,
                            uint64_t* anc, int32_t anc_words, void* ws, size_t ws_bytes,
                            void* stream, const std::shared_ptr<const TreePlanHost>& p) {
  if (anc_words < (p->T + 63) / 64) return fail(MEDUSA_ERR_ARG, "anc_words < ceil(T / 64)");
  if (b == 0) return MEDUSA_OK;
  if (!logits || !root || !idx || !val || !seq_len || !tokens || !pos || !parent || !depth || !anc)
    return fail(MEDUSA_ERR_ARG, "NULL pointer");
  if ((int64_t)b * (K + 1) > 65535) return fail(MEDUSA_ERR_UNSUPPORTED, "b * (K+1) > 65535");
  const size_t need = medusa_topk_workspace(b, K, V, kmax);
  if (need && (!ws || ws_bytes < need)) return fail(MEDUSA_ERR_WORKSPACE, "topk: workspace too small");
  if (!aligned16(ws)) return fail(MEDUSA_ERR_ARG, "workspace must be 16-byte aligned");
  TopkArgs a{};
  a.b = b; a.K = K; a.V = V; a.kmax = kmax; a.root_mode = root_mode;
  a.temperature = temperature; a.seed = seed; a.step = step;
  for (int i = 0; i < K; ++i) a.k[i] = k_host[i];
  TreeDev t{};
  t.T = p->T; t.K = K; t.kmax = kmax; t.anc_words = anc_words;
  for (int i = 0; i < p->T; ++i) {
    t.parent[i] = (int16_t)p->parent[i];
    t.depth[i] = (uint8_t)p->depth[i];
    t.rank[i] = (uint8_t)(p->rank[i] < 0 ? 0 : p->rank[i]);
  }
  TreeOut o{seq_len, tokens, pos, parent, depth, anc};
  return hip_status(run_topk(logits, a, root, idx, val, ws, as_stream(stream), &t, &o), "topk_tree");
}

// ------------------------------------------------------------------- Hydra draft
static std::shared_ptr<const TreePlanHost> hydra_plan(const int32_t* k_host, int32_t K,
                                                      const int32_t* plan_parent,
                                                      const int32_t* plan_rank, int32_t T,
                                                      std::string* err) {
  if (!k_host || K < 1 || K > MEDUSA_MAX_HEADS || !plan_parent || !plan_rank) {
    *err = "need k_host, 1 <= K <= 16 and the plan tables";
    return nullptr;
  }
  return plan_from_tables(k_host, K, plan_parent, plan_rank, T, err);
}

static TreeDev tree_dev(const TreePlanHost& p, int K, int kmax, int anc_words) {
  TreeDev t{};
  t.T = p.T; t.K = K; t.kmax = kmax; t.anc_words = anc_words;
  for (int i = 0; i < p.T; ++i) {
    t.parent[i] = (int16_t)p.parent[i];
    t.depth[i] = (uint8_t)p.depth[i];
    t.rank[i] = (uint8_t)(p.rank[i] < 0 ? 0 : p.rank[i]);
  }
  return t;
}

size_t medusa_hydra_workspace(int32_t b, int32_t H, int32_t V, const int32_t* k_host, int32_t K,
                              int32_t kmax, const int32_t* plan_parent, const int32_t* plan_rank,
                              int32_t T) {
  if (b <= 0 || H <= 0 || V <= 0 || kmax < 1 || kmax > MEDUSA_MAX_K) return 0;
  std::string err;
  auto p = hydra_plan(k_host, K, plan_parent, plan_rank, T, &err);
  if (!p) return 0;
  return round_up(hydra_workspace(b, H, V, kmax, hydra_shape(tree_dev(*p, K, kmax, 1))));
}

int medusa_hydra_draft(const void* h, int32_t b, int32_t H, const void* E, int32_t V,
                       const void* W, int32_t K, const void* LM, const int32_t* k_host,
                       int32_t kmax, const int32_t* plan_parent, const int32_t* plan_rank,
                       int32_t T, int32_t root_mode, float temperature, uint64_t seed,
                       uint64_t step, const int32_t* seq_len, int32_t* root, int32_t* tokens,
                       int32_t* pos, int32_t* parent, int32_t* depth, uint64_t* anc,
                       int32_t anc_words, float* logits_out, void* ws, size_t ws_bytes,
                       void* stream) {
  if (int s = topk_tree_args(b, K, V, k_host, kmax, root_mode, temperature)) return s;
  if (H <= 0) return fail(MEDUSA_ERR_ARG, "H must be positive");
  if (H % 128 != 0) return fail(MEDUSA_ERR_UNSUPPORTED, "Hydra draft needs H % 128 == 0");
  std::string err;
  auto p = hydra_plan(k_host, K, plan_parent, plan_rank, T, &err);
  if (!p) return fail(MEDUSA_ERR_ARG, err);
  if (anc_words < (p->T + 63) / 64) return fail(MEDUSA_ERR_ARG, "anc_words < ceil(T / 64)");
  if (b == 0) return MEDUSA_OK;
  if (!h || !E || !W || !LM || !root || !seq_len || !tokens || !pos || !parent || !depth || !anc)
    return fail(MEDUSA_ERR_ARG, "NULL pointer");
  if (!aligned16(h) || !aligned16(E) || !aligned16(W) || !aligned16(LM) || !aligned16(ws))
    return fail(MEDUSA_ERR_ARG, "h, E, W, LM and the workspace must be 16-byte aligned");
  const TreeDev t = tree_dev(*p, K, kmax, anc_words);
  const HydraShape hs = hydra_shape(t);
  int widest = 1;
  for (int d = 0; d < hs.D; ++d) widest = hs.n[d] > widest ? hs.n[d] : widest;
  if ((int64_t)b * widest > 32767) return fail(MEDUSA_ERR_UNSUPPORTED, "b * (widest depth) > 32767");
  const size_t need = medusa_hydra_workspace(b, H, V, k_host, K, kmax, plan_parent, plan_rank, T);
  if (!ws || ws_bytes < need) return fail(MEDUSA_ERR_WORKSPACE, "hydra: workspace too small");
  TopkArgs a{};
  a.b = b; a.K = K; a.V = V; a.kmax = kmax; a.root_mode = root_mode;
  a.temperature = temperature; a.seed = seed; a.step = step;
  for (int i = 0; i < K; ++i) a.k[i] = k_host[i];
  TreeOut o{seq_len, tokens, pos, parent, depth, anc};
  return hip_status(run_hydra_draft(h, E, W, LM, H, a, t, o, root, logits_out, ws,
                                    as_stream(stream)),
                    "hydra draft");
}

// ------------------------------------------------------------------- attention
static int attn_check(int32_t b, int32_t T, int32_t nq, int32_t nkv, int32_t d, int32_t Pmax,
                      int32_t dtype) {
  if (!dtype_ok(dtype)) return fail(MEDUSA_ERR_ARG, "dtype must be MEDUSA_F32 or MEDUSA_BF16");
  if (b < 0 || T < 1 || T > MEDUSA_MAX_T) return fail(MEDUSA_ERR_ARG, "need b >= 0, 1 <= T <= 256");
  if (nq < 1 || nkv < 1 || nq % nkv != 0) return fail(MEDUSA_ERR_ARG, "need nq % nkv == 0");
  if (Pmax < T) return fail(MEDUSA_ERR_ARG, "Pmax < T");
  if (dtype == MEDUSA_BF16 && d != 64 && d != 128)
    return fail(MEDUSA_ERR_UNSUPPORTED, "bf16 attention supports d = 64 or 128");
  if (dtype == MEDUSA_F32 && (d < 1 || d > 256))
    return fail(MEDUSA_ERR_UNSUPPORTED, "f32 attention supports d <= 256");
  if (dtype == MEDUSA_F32 && Pmax > 16384)
    return fail(MEDUSA_ERR_UNSUPPORTED, "f32 attention supports Pmax <= 16384");
  // the plan's grid is (sequence, kv head) x row groups (at most one per
  // 16-row block) x key partitions (at most 16 and at most one per 64 keys)
  if ((int64_t)b * nkv * std::min((Pmax + 63) / 64, 16) * ((T * (nq / nkv) + 15) / 16) >
      INT32_MAX / 4)
    return fail(MEDUSA_ERR_UNSUPPORTED, "attention grid too large");
  if (dtype == MEDUSA_F32 && (int64_t)b * T * nq > INT32_MAX / 2)
    return fail(MEDUSA_ERR_UNSUPPORTED, "attention grid too large");
  return MEDUSA_OK;
}

size_t medusa_tree_attn_workspace(int32_t b, int32_t T, int32_t nq, int32_t nkv, int32_t d,
                                  int32_t Pmax, int32_t dtype) {
  if (b <= 0 || T < 1 || nq < 1 || nkv < 1 || nq % nkv || Pmax < T || !dtype_ok(dtype)) return 0;
  return round_up(attn_plan(b, T, nq, nkv, d, Pmax, dtype).ws_bytes);
}

int medusa_tree_attn(const void* Q, const void* Kc, const void* Vc, const int32_t* seq_len,
                     const uint64_t* anc, int32_t anc_words, int32_t b, int32_t T, int32_t nq,
                     int32_t nkv, int32_t d, int32_t Pmax, float scale, int32_t dtype, void* O,
                     void* ws, size_t ws_bytes, void* stream) {
  if (int s = attn_check(b, T, nq, nkv, d, Pmax, dtype)) return s;
  if (anc_words < (T + 63) / 64 || anc_words > MEDUSA_MAX_T / 64)
    return fail(MEDUSA_ERR_ARG, "anc_words must be in [ceil(T/64), 4]");
  if (!std::isfinite(scale)) return fail(MEDUSA_ERR_ARG, "scale must be finite");
  if (b == 0) return MEDUSA_OK;
  if (!Q || !Kc || !Vc || !seq_len || !anc || !O) return fail(MEDUSA_ERR_ARG, "NULL pointer");
  if (dtype == MEDUSA_BF16 && (!aligned16(Q) || !aligned16(Kc) || !aligned16(Vc) || !aligned16(O)))
    return fail(MEDUSA_ERR_ARG, "bf16 attention operands must be 16-byte aligned");
  AttnPlan p = attn_plan(b, T, nq, nkv, d, Pmax, dtype);
  if (p.ws_bytes && (!ws || ws_bytes < p.ws_bytes))
    return fail(MEDUSA_ERR_WORKSPACE, "tree_attn: workspace too small");
  return hip_status(run_tree_attn(Q, Kc, Vc, seq_len, anc, anc_words, b, T, nq, nkv, d, Pmax, scale,
                                  dtype, O, ws, p, as_stream(stream)),
                    "tree_attn");
}

static_assert(MEDUSA_NOALLOC_SCRATCH_BYTES == kAttnScratchBytes,
              "the header states the size of the static scratch");

int medusa_tree_attn_noalloc(const void* Q, const void* Kc, const void* Vc,
                             const int32_t* seq_len, const uint64_t* anc, int32_t anc_words,
                             int32_t b, int32_t T, int32_t nq, int32_t nkv, int32_t d,
                             int32_t Pmax, float scale, int32_t dtype, void* O, void* stream) {
  if (int s = attn_check(b, T, nq, nkv, d, Pmax, dtype)) return s;
  if (anc_words < (T + 63) / 64 || anc_words > MEDUSA_MAX_T / 64)
    return fail(MEDUSA_ERR_ARG, "anc_words must be in [ceil(T/64), 4]");
  if (!std::isfinite(scale)) return fail(MEDUSA_ERR_ARG, "scale must be finite");
  if (b == 0) return MEDUSA_OK;
  if (!Q || !Kc || !Vc || !seq_len || !anc || !O) return fail(MEDUSA_ERR_ARG, "NULL pointer");
  if (dtype == MEDUSA_BF16 && (!aligned16(Q) || !aligned16(Kc) || !aligned16(Vc) || !aligned16(O)))
    return fail(MEDUSA_ERR_ARG, "bf16 attention operands must be 16-byte aligned");
  AttnPlan p = attn_plan(b, T, nq, nkv, d, Pmax, dtype);
  if (p.ws_bytes > attn_scratch_bytes())
    return fail(MEDUSA_ERR_UNSUPPORTED,
                "tree_attn_noalloc: the split-KV partials of this shape exceed the "
                "MEDUSA_NOALLOC_SCRATCH_BYTES of static scratch");
  void* ws = nullptr;
  if (p.ws_bytes) {
    hipError_t e = attn_scratch(&ws);
    if (e != hipSuccess) return hip_status(e, "tree_attn_noalloc (scratch address)");
  }
  return hip_status(run_tree_attn(Q, Kc, Vc, seq_len, anc, anc_words, b, T, nq, nkv, d, Pmax, scale,
                                  dtype, O, ws, p, as_stream(stream)),
                    "tree_attn_noalloc");
}

// ------------------------------------------------------------------- accept
size_t medusa_accept_workspace(int32_t b, int32_t T) {
  if (b <= 0 || T <= 0) return 0;
  return round_up(accept_workspace(b, T));
}

int medusa_accept(const float* base_logits, const int32_t* tokens, const int32_t* parent,
                  const int32_t* depth, int32_t b, int32_t T, int32_t V, int32_t K, int32_t mode,
                  float temperature, float eps, float delta, uint64_t seed, uint64_t step,
                  int32_t* L, int32_t* path, int32_t* acc_tokens, int32_t* bonus, void* ws,
                  size_t ws_bytes, void* stream) {
  if (b < 0 || T < 1 || T > MEDUSA_MAX_T) return fail(MEDUSA_ERR_ARG, "need b >= 0, 1 <= T <= 256");
  if (V < 1) return fail(MEDUSA_ERR_ARG, "V must be positive");
  if (K < 1 || K > MEDUSA_MAX_HEADS) return fail(MEDUSA_ERR_ARG, "K out of range [1, 16]");
  if (mode != MEDUSA_GREEDY && mode != MEDUSA_TYPICAL && mode != MEDUSA_REJECT)
    return fail(MEDUSA_ERR_ARG, "mode must be GREEDY, TYPICAL or REJECT");
  if (mode != MEDUSA_GREEDY && !(temperature > 0.f && std::isfinite(temperature)))
    return fail(MEDUSA_ERR_ARG, "temperature must be positive and finite");
  if (mode == MEDUSA_TYPICAL &&
      (!(eps > 0.f && std::isfinite(eps)) || !(delta > 0.f && std::isfinite(delta))))
    return fail(MEDUSA_ERR_ARG, "eps and delta must be positive and finite");
  if (b == 0) return MEDUSA_OK;
  if (!base_logits || !tokens || !parent || !depth || !L || !path || !acc_tokens || !bonus)
    return fail(MEDUSA_ERR_ARG, "NULL pointer");
  if ((int64_t)b * T > INT32_MAX / 2) return fail(MEDUSA_ERR_UNSUPPORTED, "b * T too large");
  const size_t need = medusa_accept_workspace(b, T);
  if (!ws || ws_bytes < need) return fail(MEDUSA_ERR_WORKSPACE, "accept: workspace too small");
  if (!aligned16(ws)) return fail(MEDUSA_ERR_ARG, "workspace must be 16-byte aligned");
  const float tmp = mode != MEDUSA_GREEDY ? temperature : 1.0f;
  return hip_status(run_accept(base_logits, tokens, parent, depth, b, T, V, K, mode, tmp, eps,
                               delta, seed, step, L, path, acc_tokens, bonus, ws,
                               as_stream(stream)),
                    "accept");
}

// ------------------------------------------------------------------- acceptance + rollback
int medusa_accept_compact(const float* base_logits, const int32_t* tokens, const int32_t* parent,
                          const int32_t* depth, int32_t b, int32_t T, int32_t V, int32_t K,
                          int32_t mode, float temperature, float eps, float delta, uint64_t seed,
                          uint64_t step, int32_t* L, int32_t* path, int32_t* acc_tokens,
                          int32_t* bonus, void* Kc, void* Vc, int32_t* seq_len, int32_t nkv,
                          int32_t Pmax, int32_t d, int32_t dtype, const void* verify_ws,
                          void* ws, size_t ws_bytes, void* stream) {
  if (b < 0 || T < 1 || T > MEDUSA_MAX_T) return fail(MEDUSA_ERR_ARG, "need b >= 0, 1 <= T <= 256");
  if (V < 1) return fail(MEDUSA_ERR_ARG, "V must be positive");
  if (K < 1 || K > MEDUSA_MAX_HEADS) return fail(MEDUSA_ERR_ARG, "K out of range [1, 16]");
  if (mode != MEDUSA_GREEDY && mode != MEDUSA_TYPICAL && mode != MEDUSA_REJECT)
    return fail(MEDUSA_ERR_ARG, "mode must be GREEDY, TYPICAL or REJECT");
  if (mode != MEDUSA_GREEDY && !(temperature > 0.f && std::isfinite(temperature)))
    return fail(MEDUSA_ERR_ARG, "temperature must be positive and finite");
  if (mode == MEDUSA_TYPICAL &&
      (!(eps > 0.f && std::isfinite(eps)) || !(delta > 0.f && std::isfinite(delta))))
    return fail(MEDUSA_ERR_ARG, "eps and delta must be positive and finite");
  if (!dtype_ok(dtype)) return fail(MEDUSA_ERR_ARG, "dtype must be MEDUSA_F32 or MEDUSA_BF16");
  if (nkv < 1 || Pmax < 1 || d < 1) return fail(MEDUSA_ERR_ARG, "bad shape");
  if ((d * elem_size(dtype)) % 16 != 0) return fail(MEDUSA_ERR_UNSUPPORTED, "d * sizeof(dtype) must be a multiple of 16");
  if (b == 0) return MEDUSA_OK;
  if (!base_logits || !tokens || !parent || !depth || !L || !path || !acc_tokens || !bonus)
    return fail(MEDUSA_ERR_ARG, "NULL pointer");
  if (!Kc || !Vc || !seq_len) return fail(MEDUSA_ERR_ARG, "NULL pointer");
  if (!aligned16(Kc) || !aligned16(Vc)) return fail(MEDUSA_ERR_ARG, "cache must be 16-byte aligned");
  if ((int64_t)b * T > INT32_MAX / 2) return fail(MEDUSA_ERR_UNSUPPORTED, "b * T too large");
  const size_t need = medusa_accept_workspace(b, T);
  if (!ws || ws_bytes < need) return fail(MEDUSA_ERR_WORKSPACE, "accept: workspace too small");
  if (!aligned16(ws)) return fail(MEDUSA_ERR_ARG, "workspace must be 16-byte aligned");
  const float tmp = mode != MEDUSA_GREEDY ? temperature : 1.0f;
  KvRollback kv{Kc, Vc, seq_len, nkv, Pmax, d, dtype};
  const void* parts = verify_ws && verify_uses_parts((int64_t)b * T, V) ? verify_ws : nullptr;
  return hip_status(run_accept(base_logits, tokens, parent, depth, b, T, V, K, mode, tmp, eps,
                               delta, seed, step, L, path, acc_tokens, bonus, ws,
                               as_stream(stream), &kv, parts),
                    "accept_compact");
}

// ------------------------------------------------------------------- compaction
int medusa_kv_compact(void* Kc, void* Vc, int32_t* seq_len, const int32_t* path,
                      const int32_t* L, int32_t b, int32_t nkv, int32_t Pmax, int32_t d, int32_t K,
                      int32_t dtype, void* stream) {
  if (!dtype_ok(dtype)) return fail(MEDUSA_ERR_ARG, "dtype must be MEDUSA_F32 or MEDUSA_BF16");
  if (b < 0 || nkv < 1 || Pmax < 1 || d < 1) return fail(MEDUSA_ERR_ARG, "bad shape");
  if (K < 0 || K > MEDUSA_MAX_HEADS) return fail(MEDUSA_ERR_ARG, "K out of range [0, 16]");
  if ((d * elem_size(dtype)) % 16 != 0) return fail(MEDUSA_ERR_UNSUPPORTED, "d * sizeof(dtype) must be a multiple of 16");
  if (b == 0) return MEDUSA_OK;
  if (!Kc || !Vc || !seq_len || !path || !L) return fail(MEDUSA_ERR_ARG, "NULL pointer");
  if (!aligned16(Kc) || !aligned16(Vc)) return fail(MEDUSA_ERR_ARG, "cache must be 16-byte aligned");
  return hip_status(run_kv_compact(Kc, Vc, seq_len, path, L, b, nkv, Pmax, d, K, dtype,
                                   as_stream(stream)),
                    "kv_compact");
}

// ------------------------------------------------------------------- state between steps
int medusa_kv_append(void* Kc, void* Vc, const int32_t* seq_len, const void* Knew,
                     const void* Vnew, int32_t b, int32_t nkv, int32_t Pmax, int32_t T, int32_t d,
                     int32_t dtype, void* stream) {
  if (!dtype_ok(dtype)) return fail(MEDUSA_ERR_ARG, "dtype must be MEDUSA_F32 or MEDUSA_BF16");
  if (b < 0 || nkv < 1 || d < 1 || T < 1 || T > MEDUSA_MAX_T || Pmax < T)
    return fail(MEDUSA_ERR_ARG, "need b >= 0, nkv >= 1, d >= 1, 1 <= T <= 256, Pmax >= T");
  if ((d * elem_size(dtype)) % 16 != 0) return fail(MEDUSA_ERR_UNSUPPORTED, "d * sizeof(dtype) must be a multiple of 16");
  if ((int64_t)b * nkv > INT32_MAX) return fail(MEDUSA_ERR_UNSUPPORTED, "b * nkv too large");
  if (b == 0) return MEDUSA_OK;
  if (!Kc || !Vc || !seq_len || !Knew || !Vnew) return fail(MEDUSA_ERR_ARG, "NULL pointer");
  if (!aligned16(Kc) || !aligned16(Vc) || !aligned16(Knew) || !aligned16(Vnew))
    return fail(MEDUSA_ERR_ARG, "cache and new rows must be 16-byte aligned");
  return hip_status(run_kv_append(Kc, Vc, seq_len, Knew, Vnew, b, nkv, Pmax, T, d, dtype,
                                  as_stream(stream)),
                    "kv_append");
}

int medusa_next_hidden(const void* O, const int32_t* path, const int32_t* L, int32_t b,
                       int32_t T, int32_t K, int32_t H, int32_t dtype, void* h, void* stream) {
  if (!dtype_ok(dtype)) return fail(MEDUSA_ERR_ARG, "dtype must be MEDUSA_F32 or MEDUSA_BF16");
  if (b < 0 || T < 1 || T > MEDUSA_MAX_T || H < 1) return fail(MEDUSA_ERR_ARG, "need b >= 0, 1 <= T <= 256, H >= 1");
  if (K < 0 || K > MEDUSA_MAX_HEADS) return fail(MEDUSA_ERR_ARG, "K out of range [0, 16]");
  if ((H * elem_size(dtype)) % 16 != 0) return fail(MEDUSA_ERR_UNSUPPORTED, "H * sizeof(dtype) must be a multiple of 16");
  if (b == 0) return MEDUSA_OK;
  if (!O || !path || !L || !h) return fail(MEDUSA_ERR_ARG, "NULL pointer");
  if (!aligned16(O) || !aligned16(h)) return fail(MEDUSA_ERR_ARG, "O and h must be 16-byte aligned");
  return hip_status(run_next_hidden(O, path, L, b, T, K, H, dtype, h, as_stream(stream)),
                    "next_hidden");
}

// ------------------------------------------------------------------- tree budget
int medusa_tree_plan_rates(const int32_t* k_host, int32_t K, int32_t N, const double* q,
                           int32_t* parent, int32_t* depth, int32_t* rank, int32_t T_cap,
                           int32_t* T_out, double* expected_tokens) {
  if (int s = check_k(k_host, K, 0)) return s;
  if (!q) return fail(MEDUSA_ERR_ARG, "q is NULL");
  if (N < -1) return fail(MEDUSA_ERR_ARG, "N must be >= 0, or -1 for the full tree");
  for (int d = 0; d < K; ++d)
    for (int r = 0; r < k_host[d]; ++r) {
      const double v = q[d * MEDUSA_MAX_K + r];
      if (!(v >= 0.0 && v <= 1.0)) return fail(MEDUSA_ERR_ARG, "rates must lie in [0, 1]");
    }
  const int64_t total = full_tree_candidates(k_host, K);
  if (N > total && total >= 0) return fail(MEDUSA_ERR_ARG, "N exceeds the candidate count");
  const int64_t keep = N < 0 ? total : N;
  if (keep < 0 || keep + 1 > MEDUSA_MAX_T) return fail(MEDUSA_ERR_UNSUPPORTED, "tree exceeds 256 nodes");
  std::string err;
  double e = 0.0;
  auto p = plan_from_rates(k_host, K, N, q, &e, &err);
  if (!p) return fail(MEDUSA_ERR_UNSUPPORTED, err);
  if (T_out) *T_out = p->T;
  if (expected_tokens) *expected_tokens = e;
  if (!parent && !depth && !rank) return MEDUSA_OK;
  if (T_cap < p->T) return fail(MEDUSA_ERR_ARG, "T_cap smaller than the tree");
  for (int i = 0; i < p->T; ++i) {
    if (parent) parent[i] = p->parent[i];
    if (depth) depth[i] = p->depth[i];
    if (rank) rank[i] = p->rank[i];
  }
  return MEDUSA_OK;
}

int medusa_accept_tally(const int32_t* L, const int32_t* path, int32_t b, const int32_t* k_host,
                        int32_t K, const int32_t* plan_parent, const int32_t* plan_rank,
                        int32_t T, int64_t* accepted, int64_t* offered, void* stream) {
  if (int s = check_k(k_host, K, 0)) return s;
  if (b < 0) return fail(MEDUSA_ERR_ARG, "b < 0");
  if (!plan_parent || !plan_rank) return fail(MEDUSA_ERR_ARG, "plan tables are NULL");
  std::string err;
  auto p = plan_from_tables(k_host, K, plan_parent, plan_rank, T, &err);
  if (!p) return fail(MEDUSA_ERR_ARG, err);
  if (b == 0) return MEDUSA_OK;
  if (!L || !path || !accepted || !offered) return fail(MEDUSA_ERR_ARG, "NULL pointer");
  if (((uintptr_t)accepted & 7u) || ((uintptr_t)offered & 7u))
    return fail(MEDUSA_ERR_ARG, "counts must be 8-byte aligned");
  TreeDev t{};
  t.T = p->T; t.K = K; t.kmax = MEDUSA_MAX_K; t.anc_words = (p->T + 63) / 64;
  for (int i = 0; i < p->T; ++i) {
    t.parent[i] = (int16_t)p->parent[i];
    t.depth[i] = (uint8_t)p->depth[i];
    t.rank[i] = (uint8_t)(p->rank[i] < 0 ? 0 : p->rank[i]);
  }
  return hip_status(run_accept_tally(L, path, b, K, t, accepted, offered, as_stream(stream)),
                    "accept_tally");
}

// ------------------------------------------------------------------- yardstick
int medusa_stream_read(const void* buf, size_t bytes, uint32_t never, void* sink, void* stream) {
  if (bytes % 16) return fail(MEDUSA_ERR_ARG, "stream_read: bytes must be a multiple of 16");
  if (bytes == 0) return MEDUSA_OK;
  if (!buf || !sink) return fail(MEDUSA_ERR_ARG, "NULL pointer");
  if (!aligned16(buf) || ((uintptr_t)sink & 3))
    return fail(MEDUSA_ERR_ARG, "stream_read: buf must be 16-byte and sink 4-byte aligned");
  return hip_status(run_stream_read(buf, bytes, never, static_cast<uint32_t*>(sink),
                                    as_stream(stream)),
                    "stream_read");
}

}  // extern "C"
