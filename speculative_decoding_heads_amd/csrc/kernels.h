// Internal launchers of the Medusa HIP kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace medusa {

enum { kF32 = 0, kBF16 = 1 };
// kRootGiven: root_mode only; kReject: acceptance mode only
enum { kGreedy = 0, kTypical = 1, kRootGiven = 2, kReject = 3 };

constexpr int kMaxHeads = 16;   // Medusa heads K
constexpr int kMaxK = 16;       // shortlist size per head
constexpr int kMaxT = 256;      // tree nodes including the root
constexpr int kMaxAncWords = kMaxT / 64;

// ---- heads / LM projection (gemm.hip)
hipError_t run_heads_hidden(const void* x, int M, int H, const void* W, int n_heads, int dtype,
                            void* u, int R, int base, hipStream_t st);
// rev: the weight-streaming kernel walks K backwards (same products, another
// summation order); see medusa_heads.
// ldc: logits row stride in floats (0: V).
// stream_w: the weights are read with the non-temporal hint where the
// weight-stream kernel runs (for the last pass over them in a step); the
// logits are the same either way.
hipError_t run_lm_logits(const void* x, int M, int H, const void* LM, int V, int dtype,
                         float* logits, hipStream_t st, bool rev = false, int64_t ldc = 0,
                         bool stream_w = false);
// LM projection of the verify rows plus acceptance partials per (row, weight
// tile) in ws: a header (kPartsHeader bytes, the int32 fields below), then
// [rows][ntiles] argmax keys (u64, greedy) or RowStat (typical).  The header
// records what the partials were made for; acceptance uses them only when
// every field matches its own call (else it reads the logits).
constexpr size_t kPartsHeader = 256;
enum { kHdrTiles = 0, kHdrKind = 1, kHdrRows = 2, kHdrCols = 3, kHdrInvTemp = 4, kHdrMagic = 5 };
constexpr int kPartsMagic = 0x4D445653;
int verify_tiles(int M, int N, int Kd, int dtype);
// whether run_verify_logits leaves partials (else acceptance reads the logits)
bool verify_uses_parts(int64_t M, int64_t N);
size_t verify_workspace(int M, int N, int Kd, int dtype, int mode);
hipError_t run_verify_logits(const void* x, int M, int H, const void* LM, int V, int dtype,
                             float* logits, int mode, float temperature, void* ws, hipStream_t st);

// ---- MTP-style heads: one transformer layer per head, batched over heads
// (gemm.hip: the layer's GEMMs; mtp.hip: RMSNorm and the draft driver)
hipError_t run_mtp_qkv(const uint16_t* a, int M, int H, const uint16_t* Wqkv, int heads, int nq,
                       int nkv, int d, uint16_t* Q, uint16_t* Kc, uint16_t* Vc,
                       const int* seq_len, int Pmax, hipStream_t st);
hipError_t run_mtp_resid(const uint16_t* x, int64_t ldx, int64_t sx, int M, int Kd,
                         const uint16_t* W, int N, int heads, uint16_t* O, int64_t so,
                         int64_t ldo, const uint16_t* R, int64_t sr, int64_t ldr, hipStream_t st);
hipError_t run_mtp_swiglu(const uint16_t* a, int M, int H, const uint16_t* Wgu, int F, int heads,
                          uint16_t* z, hipStream_t st);
struct MtpArgs {
  const void* h;                       // [b, H]
  int b, H, K, F;
  const void *g1, *Wqkv, *Wo, *g2, *Wgu, *Wd;
  float eps;
  void *Kh, *Vh;                       // [K, b, nkv, Pmax, d]
  const int* seq_len;                  // [b]
  int nq, nkv, d, Pmax;
  const void* LM;
  int V;
};

// ---- top-k shortlists and root (topk.hip)
struct TopkArgs {
  int b, K, V, kmax;
  int root_mode;
  float temperature;
  uint64_t seed, step;
  int k[kMaxHeads];
};
// ---- tree plan on the device, passed by value (tree.hip, topk.hip)
struct TreeDev {
  int T, K, kmax, anc_words;
  int16_t parent[kMaxT];
  uint8_t depth[kMaxT];
  uint8_t rank[kMaxT];
};
// outputs of the tree gather; tokens == nullptr when no tree is built
struct TreeOut {
  const int* seq_len;
  int* tokens;
  int* pos;
  int* parent;
  int* depth;
  uint64_t* anc;
};

size_t topk_workspace(int b, int K, int V, int kmax);
// With tree != nullptr the same launch also writes the tree tables and tokens.
hipError_t run_topk(const float* logits, const TopkArgs& a, int* root, int* idx, float* val,
                    void* ws, hipStream_t st, const TreeDev* tree = nullptr,
                    const TreeOut* tree_out = nullptr);

// ---- Hydra-style sequential draft (hydra.hip)
// Row counts of the plan's depths: n[d] nodes at depth d, first node first[d]
// (nodes come in depth order).  Returns the largest parent row count
// b * max_{d < D} n[d] the per-depth passes use (D = the deepest depth).
struct HydraShape {
  int D;
  int first[kMaxHeads + 1], n[kMaxHeads + 1];
};
HydraShape hydra_shape(const TreeDev& t);
size_t hydra_workspace(int b, int H, int V, int kmax, const HydraShape& hs);
// h [b,H], E [V,H], W [K,H,H], LM [V,H] bf16; k per head in a.k; the root
// as in run_topk (a.root_mode); the tree tables, positions and tokens into o;
// logits_out (optional) [b,T,V]: row (s, p) = the head logits node p's
// children were drawn from, for every node above the deepest depth.
hipError_t run_hydra_draft(const void* h, const void* E, const void* W, const void* LM, int H,
                           const TopkArgs& a, const TreeDev& t, const TreeOut& o, int* root,
                           float* logits_out, void* ws, hipStream_t st);

// ---- sampling rows of softmax(x / T) in float64 (topk.hip)
// Row of sequence s: base + s*seq_stride + (row_sel ? row_sel[s] : 0) * V.
// The draw goes to out[s] and, if out2 is given, to out2[s * out2_stride].
// ws: sample_workspace(b) bytes, 16-byte aligned (per-slice partial sums).
constexpr int kSampSlices = 64;
constexpr int kSampExcl = 16;    // tokens a draw can exclude (the children of one node)
size_t sample_workspace(int b);
hipError_t run_sample_rows(const float* base, int64_t seq_stride, const int* row_sel, int b, int V,
                           float temperature, uint64_t seed, uint64_t step, uint64_t draw,
                           int* out, void* ws, hipStream_t st, int* out2 = nullptr,
                           int out2_stride = 0, const int* excl = nullptr);

hipError_t run_build_tree(const TreeDev& t, const int* root, const int* idx, int b,
                          const int* seq_len, int* tokens, int* pos, int* parent, int* depth,
                          uint64_t* anc, hipStream_t st);

// ---- tree attention (attn.hip)
struct AttnPlan {
  int nsplit;        // key-range partitions per (sequence, kv head)
  int rowgroups;     // workgroups along the query rows of one kv head
  int rb;            // 16-row blocks per wave
  size_t ws_bytes;
  int tiles_per_split;  // 64-key tiles per partition
  int bpg;           // 16-row blocks per row group (<= 8 rb)
  int nbuf;          // K/V tiles in the LDS ring (4, or 2: two workgroups per CU)
};
AttnPlan attn_plan(int b, int T, int nq, int nkv, int d, int Pmax, int dtype);
// MTP draft workspace regions (byte offsets) and the attention plan it uses
struct MtpLayout {
  size_t a, a2, x1, q, o, z, u, seq, anc, attn, bytes;
  AttnPlan plan;
};
MtpLayout mtp_layout(int M, int H, int K, int F, int nq, int nkv, int d, int Pmax, bool own_u);
hipError_t run_mtp_draft(const MtpArgs& a, void* u_out, float* logits, void* ws, hipStream_t st);
// the static scratch of the no-allocation attention call: its size, and its
// device address on the current device (looked up once per device)
constexpr size_t kAttnScratchBytes = size_t(16) << 20;
size_t attn_scratch_bytes();
hipError_t attn_scratch(void** out);
hipError_t run_tree_attn(const void* Q, const void* Kc, const void* Vc, const int* seq_len,
                         const uint64_t* anc, int anc_words, int b, int T, int nq, int nkv, int d,
                         int Pmax, float scale, int dtype, void* O, void* ws, const AttnPlan& p,
                         hipStream_t st);

// ---- acceptance (accept.hip)
// KV cache of the rollback fused into the acceptance walk
struct KvRollback {
  void* Kc;
  void* Vc;
  int* seq_len;
  int nkv, Pmax, d, dtype;
};
size_t accept_workspace(int b, int T);
hipError_t run_accept(const float* base_logits, const int* tokens, const int* parent,
                      const int* depth, int b, int T, int V, int K, int mode, float temperature,
                      float eps, float delta, uint64_t seed, uint64_t step, int* L, int* path,
                      int* acc_tokens, int* bonus, void* ws, hipStream_t st,
                      const KvRollback* kv = nullptr, const void* parts = nullptr);

// ---- compaction (compact.hip)
// ---- state between steps (loop.hip)
hipError_t run_kv_append(void* Kc, void* Vc, const int* seq_len, const void* Knew,
                         const void* Vnew, int b, int nkv, int Pmax, int T, int d, int dtype,
                         hipStream_t st);
hipError_t run_next_hidden(const void* O, const int* path, const int* L, int b, int T, int K,
                           int H, int dtype, void* h, hipStream_t st);
// offered / accepted counts per (depth - 1, rank), [K][16] int64, added to
hipError_t run_accept_tally(const int* L, const int* path, int b, int K, const TreeDev& t,
                            int64_t* accepted, int64_t* offered, hipStream_t st);

hipError_t run_kv_compact(void* Kc, void* Vc, int* seq_len, const int* path, const int* L, int b,
                          int nkv, int Pmax, int d, int K, int dtype, hipStream_t st);

// ---- yardstick (probe.hip): a plain read of `bytes` (a multiple of 16)
hipError_t run_stream_read(const void* buf, size_t bytes, uint32_t never, uint32_t* sink,
                           hipStream_t st);

}  // namespace medusa
