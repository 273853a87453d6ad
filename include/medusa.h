/*
 * medusa.h - C ABI of libmedusa.so: one Medusa draft-and-verify step on an
 * AMD Instinct MI355X (gfx950), in hand-written HIP kernels.
 *
 * Sources (web pages on Medusa heads, cited by title and section):
 *   [deep-dive]  aicassindra.com, "Medusa deep dive" (tm_medusa_deep)
 *   [glossary]   inferensys.com, "Medusa Heads"
 *   [guide]      aiunderstanding.org, "Medusa Decoding Heads"
 *   [zackli]     zackli.ai, "Speculative Decoding Deep Dive II: Medusa, MTP"
 *
 * Conventions for every call:
 *   - Device pointers are caller-owned device memory (for instance a torch
 *     tensor's data_ptr()), contiguous, row-major, in the layout given.
 *     Pointers marked "host" are ordinary host memory, read during the call.
 *   - A call validates its arguments on the host first; on failure it returns
 *     a negative status, launches nothing and sets medusa_last_error().
 *   - On success a call has only ENQUEUED its kernels on `stream` (a
 *     hipStream_t; NULL = the default stream) and returns MEDUSA_OK.  No call
 *     allocates or frees device memory, synchronises, or copies device data
 *     to the host.  A failed launch returns MEDUSA_ERR_HIP.
 *   - Scratch memory is a caller-provided workspace `ws` of at least the
 *     size the matching *_workspace() query returns (host-only queries),
 *     16-byte aligned.  Its contents need no initialisation and are
 *     overwritten by every call.
 *   - Floating-point inputs must be finite.  Values that only the device
 *     sees (token ids, seq_len, L, path) are range-checked by the kernels:
 *     an out-of-range seq_len gives NaN attention rows for that sequence and
 *     leaves the cache untouched in compaction; out-of-range tokens are
 *     rejected by acceptance.
 *   - Calls are reentrant.  The only library state is an immutable cache of
 *     tree plans keyed by (k, N, decay), guarded by a mutex, and the static
 *     device scratch of medusa_tree_attn_noalloc (one array per GPU, shared by
 *     every call of that entry point on the GPU).
 *   - Calls that share buffers must be ordered on one stream by the caller.
 */
#ifndef MEDUSA_H
#define MEDUSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MEDUSA_ABI_VERSION 1

typedef enum {
  MEDUSA_OK = 0,
  MEDUSA_ERR_ARG = -1,          /* invalid argument (null, range, alignment) */
  MEDUSA_ERR_UNSUPPORTED = -2,  /* valid but outside what the kernels handle */
  MEDUSA_ERR_WORKSPACE = -3,    /* workspace missing or too small */
  MEDUSA_ERR_HIP = -4           /* a HIP launch failed */
} medusa_status;

typedef enum { MEDUSA_F32 = 0, MEDUSA_BF16 = 1 } medusa_dtype;   /* logits are always f32 */
typedef enum { MEDUSA_GREEDY = 0, MEDUSA_TYPICAL = 1 } medusa_mode;
/* root_mode of medusa_topk / medusa_topk_tree only: root[] is an input (the
 * previous step's next token, see medusa_next_hidden). */
#define MEDUSA_ROOT_GIVEN 2
/* mode of medusa_accept / medusa_accept_compact / medusa_verify_logits only:
 * exact rejection sampling over the tree (see medusa_accept). */
#define MEDUSA_REJECT 3

/* Limits of the library. */
#define MEDUSA_MAX_HEADS 16     /* Medusa heads K */
#define MEDUSA_MAX_K 16         /* shortlist size per head */
#define MEDUSA_MAX_T 256        /* tree nodes including the root */

int medusa_abi_version(void);
const char* medusa_status_str(int status);
/* Message of the last failed call on this host thread ("" if none). */
const char* medusa_last_error(void);

/* ---------------------------------------------------------------------------
 * medusa_heads - K residual Medusa heads sharing one LM projection.
 * [deep-dive] "The heads are residual blocks, not linear layers":
 *   head_i(h) = LMproj(h + SiLU(W_i h)),  SiLU(z) = z * sigmoid(z);
 * [deep-dive] "What this deep dive assumes" / [zackli] "Medusa" (Head_0): the
 * base head LMproj(h) owns t+1 and Medusa head i owns t+i+1.  The same call
 * with n_heads = 0 is the base model's original output head applied to the
 * verification rows ([glossary], verification phase).
 *
 *   x       [rows, H]            hidden states (dtype)
 *   W       [n_heads, H, H]      head weights, [head][out][in] (dtype); NULL
 *                                 allowed when n_heads == 0
 *   LM      [V, H]               shared LM projection (dtype)
 *   include_base  1: output slot 0 is the base head LMproj(x)
 *   u_out   [rows, R, H] or NULL hidden state of every head, R =
 *                                 include_base + n_heads: slot 0 = x (base),
 *                                 then x + SiLU(W_i x) rounded to dtype.  NULL:
 *                                 kept in the workspace.
 *   logits  [rows, R, V] f32     logits[r, j, :] = LM . u[r, j, :]
 * bf16 needs H % 128 == 0 and 16-byte aligned x, W, LM, u_out.  rows == 0 is
 * a no-op.  Arithmetic: bf16 operands, f32 accumulation (MFMA); f32 path in
 * f32 throughout.  With n_heads > 0 the bf16 LM projection sums the K chunks
 * in the reverse order of the n_heads = 0 call (so a step's two passes over
 * LM each begin on the weights the other read last, still in the last-level
 * cache); logits of the same row from the two forms can differ by rounding.
 * ------------------------------------------------------------------------- */
size_t medusa_heads_workspace(int64_t rows, int32_t H, int32_t n_heads, int32_t include_base,
                              int32_t dtype);
int medusa_heads(const void* x, int64_t rows, int32_t H, const void* W, int32_t n_heads,
                 const void* LM, int32_t V, int32_t dtype, int32_t include_base, void* u_out,
                 float* logits, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * medusa_heads_hidden / medusa_lm_logits - the two halves of medusa_heads as
 * calls of their own (the same kernels; each call is one GEMM), for callers
 * that schedule or time them apart.  [deep-dive] "The heads are residual
 * blocks, not linear layers": the residual block, then the shared LM
 * projection.
 *
 * medusa_heads_hidden: u_out [rows, R, H] (dtype), R = include_base + n_heads
 *   (n_heads >= 1): slot 0 = x when include_base, then x + SiLU(W_i x)
 *   rounded to dtype, exactly as medusa_heads writes u_out.
 * medusa_lm_logits: logits [rows, V] f32 = x [rows, H] . LM^T.  reverse_k = 1
 *   sums the K chunks in the order medusa_heads uses for head rows, 0 in the
 *   order it uses with n_heads = 0 (verify rows).
 * medusa_heads(x, W, n_heads > 0, ..., u_out, logits) is bit for bit
 * medusa_heads_hidden(x, ..., u_out) then medusa_lm_logits(u_out viewed as
 * [rows * R, H], reverse_k = 1); with n_heads = 0 it is medusa_lm_logits(x,
 * reverse_k = 0).  Requirements and errors as medusa_heads.
 * ------------------------------------------------------------------------- */
int medusa_heads_hidden(const void* x, int64_t rows, int32_t H, const void* W, int32_t n_heads,
                        int32_t dtype, int32_t include_base, void* u_out, void* stream);
int medusa_lm_logits(const void* x, int64_t rows, int32_t H, const void* LM, int32_t V,
                     int32_t dtype, int32_t reverse_k, float* logits, void* stream);

/* ---------------------------------------------------------------------------
 * medusa_topk - per-head shortlists and the root token.
 * [deep-dive] "From top-k heads to a sparse candidate tree": keep the top k_i
 * tokens of head i.  Order: logit descending, equal logits by the lower
 * vocabulary index (-0.0 == +0.0).
 *
 *   logits [b, K+1, V] f32       slot 0 = base head, slot i = Medusa head i
 *   k_host [K] (host)            shortlist sizes, 1 <= k_i <= kmax <= 16, k_i <= V
 *   root_mode  GREEDY: root = argmax of slot 0 (lowest index on ties).
 *              TYPICAL: root = a sample from softmax(slot0 / temperature) in
 *              float64: the smallest i whose running sum of
 *              exp((x_i - max x)/T) exceeds u * (the full sum), with
 *              u = (splitmix64(seed ^ step<<32 ^ s<<8 ^ 0) >> 40) * 2^-24
 *              for sequence s (SplitMix64: Steele, Lea, Flood 2014).
 *              The sums are taken over 64 vocabulary slices and combined, so
 *              a draw can differ from a serial float64 running sum only when
 *              u * sum lies within rounding of a running sum.
 *              ROOT_GIVEN: root[] holds the root tokens on entry (the next
 *              token the previous step produced) and is left as it is.
 *   root   [b] i32; idx [b, K, kmax] i32 (descending; -1 past k_i);
 *   val    [b, K, kmax] f32 (the logits; -inf past k_i)
 *   ws     medusa_topk_workspace bytes: the float64 sampler's per-slice
 *          partial sums (64 slices per sequence).
 * ------------------------------------------------------------------------- */
size_t medusa_topk_workspace(int32_t b, int32_t K, int32_t V, int32_t kmax);
int medusa_topk(const float* logits, int32_t b, int32_t K, int32_t V, const int32_t* k_host,
                int32_t kmax, int32_t root_mode, float temperature, uint64_t seed, uint64_t step,
                int32_t* root, int32_t* idx, float* val, void* ws, size_t ws_bytes,
                void* stream);

/* ---------------------------------------------------------------------------
 * medusa_tree_plan (host only) / medusa_build_tree - the fixed sparse tree.
 * [deep-dive] "From top-k heads to a sparse candidate tree": the Cartesian
 * product of shortlists is pruned ahead of time to a fixed sparse tree with
 * more branches through confident, early heads, laid out as a flat node
 * sequence with a matching attention mask and position ids; [zackli]
 * "Medusa": Anc(i), and s_1 + s_1 s_2 + ... nodes for the full tree.
 *
 * A candidate is a rank tuple (r_1..r_D), r_d < k_d: rank r_d of head d at
 * depth d.  The N kept candidates are the first N under (score descending,
 * D ascending, tuple ascending), score = prod_{d=1..D} decay^d / (r_d + 1),
 * decay = decay_num / decay_den in (0, 1), compared exactly.  N = -1 keeps
 * all (full tree).  Node 0 is the root; then candidates by depth, tuples
 * ascending within a depth, so parent[i] < i.  T = N + 1 <= 256.
 *
 * medusa_tree_plan fills host arrays parent/depth/rank [T_cap] (rank = the
 * tuple's last rank; -1 for the root) and *T_out.
 * medusa_build_tree, per sequence s (all device):
 *   tokens[s, 0] = root[s];  tokens[s, i] = idx[s, depth_i - 1, rank_i]
 *   pos[s, i]    = seq_len[s] + depth_i
 *   parent[T], depth[T] i32; anc [T, anc_words] u64: bit (j % 64) of word
 *   j / 64 in row i is set iff j == i or j is an ancestor of i.
 * idx is [b, K, kmax] as written by medusa_topk.
 * ------------------------------------------------------------------------- */
int medusa_tree_plan(const int32_t* k_host, int32_t K, int32_t N, int32_t decay_num,
                     int32_t decay_den, int32_t* parent, int32_t* depth, int32_t* rank,
                     int32_t T_cap, int32_t* T_out);
int medusa_build_tree(const int32_t* k_host, int32_t K, int32_t N, int32_t decay_num,
                      int32_t decay_den, const int32_t* root, const int32_t* idx, int32_t b,
                      int32_t kmax, const int32_t* seq_len, int32_t* tokens, int32_t* pos,
                      int32_t* parent, int32_t* depth, uint64_t* anc, int32_t anc_words,
                      void* stream);

/* ---------------------------------------------------------------------------
 * medusa_topk_tree - medusa_topk and medusa_build_tree in one launch (the
 * shortlist of head i and the tokens of the tree nodes at depth i come from
 * the same workgroup).  Same arguments, layouts and outputs as the two calls
 * made in sequence: the shortlist arguments of medusa_topk, the tree
 * arguments of medusa_build_tree (the tree uses the same k_host and kmax),
 * with seq_len [b] device.  Outputs are bit-identical to the two-call path.
 * Errors: the union of both calls' checks; nothing is launched on error.
 * ------------------------------------------------------------------------- */
int medusa_topk_tree(const float* logits, int32_t b, int32_t K, int32_t V, const int32_t* k_host,
                     int32_t kmax, int32_t N, int32_t decay_num, int32_t decay_den,
                     int32_t root_mode, float temperature, uint64_t seed, uint64_t step,
                     const int32_t* seq_len, int32_t* root, int32_t* idx, float* val,
                     int32_t* tokens, int32_t* pos, int32_t* parent, int32_t* depth, uint64_t* anc,
                     int32_t anc_words, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * medusa_tree_attn - one tree-masked attention layer of the verify pass.
 * [glossary] tree attention: all branches share the prefix KV cache and all
 * nodes are scored in one pass; [deep-dive]: a node attends only to its
 * ancestors.  For sequence b with P = seq_len[b], node i and q head h
 * (kv head g = floor(h * nkv / nq)):
 *   O[b, i, h*d:(h+1)*d] = softmax_j(scale * q . k_j) v_j
 * over j in [0, P) and the tree slots P + a, a in Anc(i) u {i}.
 *   Q  [b, T, nq, d] (dtype)     the tree nodes' queries
 *   Kc, Vc [b, nkv, Pmax, d]     cache; the tree nodes' K/V at slots P..P+T-1
 *   anc [T, anc_words] u64       as written by medusa_build_tree
 *   O  [b, T, nq*d] (dtype)
 * Requires P + T <= Pmax per sequence (else NaN rows for that sequence),
 * nq % nkv == 0, T <= 256; bf16: d in {64, 128}, 16-byte aligned pointers;
 * f32: d <= 256, Pmax <= 16384.  bf16 arithmetic: MFMA products, f32 softmax,
 * probabilities rounded to bf16 for the PV product, O rounded to bf16.
 * ------------------------------------------------------------------------- */
size_t medusa_tree_attn_workspace(int32_t b, int32_t T, int32_t nq, int32_t nkv, int32_t d,
                                  int32_t Pmax, int32_t dtype);
int medusa_tree_attn(const void* Q, const void* Kc, const void* Vc, const int32_t* seq_len,
                     const uint64_t* anc, int32_t anc_words, int32_t b, int32_t T, int32_t nq,
                     int32_t nkv, int32_t d, int32_t Pmax, float scale, int32_t dtype, void* O,
                     void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * medusa_tree_attn_noalloc - medusa_tree_attn for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, checks, kernels and outputs as
 * medusa_tree_attn, without the workspace: the split-KV partials live in a
 * static device array of MEDUSA_NOALLOC_SCRATCH_BYTES that each GPU the
 * library runs on holds until the process ends (its address is looked up on
 * the first call on a device, with that device current; the stream must
 * belong to the current device).  The call allocates and frees nothing.
 * Shapes whose partials (medusa_tree_attn_workspace bytes) exceed the array
 * return MEDUSA_ERR_UNSUPPORTED and launch nothing.  Every call on a GPU
 * shares that GPU's array and leaves its partials there: calls that overlap
 * on one GPU (other streams, other host threads) race and must be ordered by
 * the caller.  Nothing in the array needs to start at zero.
 * ------------------------------------------------------------------------- */
#define MEDUSA_NOALLOC_SCRATCH_BYTES (16u << 20)
int medusa_tree_attn_noalloc(const void* Q, const void* Kc, const void* Vc,
                             const int32_t* seq_len, const uint64_t* anc, int32_t anc_words,
                             int32_t b, int32_t T, int32_t nq, int32_t nkv, int32_t d,
                             int32_t Pmax, float scale, int32_t dtype, void* O, void* stream);

/* ---------------------------------------------------------------------------
 * medusa_accept - acceptance, the accepted path and the next token.
 * [guide] "Deep Dive": accept the longest prefix matching what the model
 * would have produced; [glossary]: stop at the first rejection, roll back,
 * the base model gives the next token; [deep-dive] "Typical acceptance, not
 * exact rejection sampling": accept when p(x) > min(eps, delta * exp(-H)).
 *   base_logits [b, T, V] f32    verify logits of every node
 *   tokens [b, T], parent [T], depth [T]   as from medusa_build_tree
 *   GREEDY : child c of p accepted iff tokens[c] == argmax base_logits[p]
 *            (lowest index on ties).
 *   TYPICAL: q = softmax(base_logits[p] / temperature), H = -sum q ln q;
 *            accepted iff q[tokens[c]] > min(eps, delta * exp(-H)).
 *   A node is fully accepted when it and all its ancestors below the root
 *   are.  L[b] = the largest depth of a fully accepted node (0..K); the chosen
 *   node is the lowest node index at that depth.
 *   path [b, K+1]       node indices root .. chosen node, -1 padded
 *   acc_tokens [b, K+1] their tokens, -1 padded
 *   bonus [b]           next token at the chosen node: argmax (GREEDY) or a
 *                       float64 sample from softmax(x / temperature) with
 *                       counter draw 1 (TYPICAL; same rule as medusa_topk)
 *   REJECT (exact rejection sampling; [guide] "Deep Dive": rejection against
 *   the original model keeps its output distribution; [deep-dive]: the heads
 *   give no proposal distribution of their own): the candidates of a node
 *   are point-mass proposals tried in node order.  With p = softmax(
 *   base_logits[n] / temperature) at node n, its j-th child c (token t) is
 *   taken when u * (1 - r) < p[t], r = the p of the children tried before it
 *   and u = counter draw 16 * depth(n) + j keyed by splitmix64(seed); the
 *   walk moves to the first taken child, from the root down.  L and the
 *   chosen node are where it stops.  bonus: counter draw 1 from p at the
 *   chosen node with its children's tokens removed (they were all
 *   rejected), from the full p when it has none.  Every emitted token is
 *   then distributed as p at its position.  p comes from the float32
 *   statistics of the typical path (taken in float64), so a decision can
 *   differ from exact arithmetic only when u * (1 - r) lies within that
 *   rounding of p[t].  eps and delta are not used.
 * ------------------------------------------------------------------------- */
size_t medusa_accept_workspace(int32_t b, int32_t T);
int medusa_accept(const float* base_logits, const int32_t* tokens, const int32_t* parent,
                  const int32_t* depth, int32_t b, int32_t T, int32_t V, int32_t K, int32_t mode,
                  float temperature, float eps, float delta, uint64_t seed, uint64_t step,
                  int32_t* L, int32_t* path, int32_t* acc_tokens, int32_t* bonus, void* ws,
                  size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * medusa_kv_compact - rollback of the speculative KV entries.
 * [glossary]: roll back to the last accepted position; the speculative KV
 * cache manages the tree's key/value entries.  For every sequence s with
 * P = seq_len[s] (device) and d = 0..L[s]:
 *   Kc[s, :, P + d, :] <- Kc[s, :, P + path[s, d], :]   (same for Vc)
 * as if from a snapshot (sources are read before they are overwritten), then
 * seq_len[s] = P + L[s] + 1.  In place; stale slots past the new length are
 * left as they are.  Requires path[s, d] >= d (breadth-first node order, as
 * produced by medusa_accept) and (d * sizeof(dtype)) % 16 == 0.
 * ------------------------------------------------------------------------- */
int medusa_kv_compact(void* Kc, void* Vc, int32_t* seq_len, const int32_t* path,
                      const int32_t* L, int32_t b, int32_t nkv, int32_t Pmax, int32_t d, int32_t K,
                      int32_t dtype, void* stream);

/* ---------------------------------------------------------------------------
 * medusa_accept_compact - medusa_accept followed by medusa_kv_compact, with
 * the rollback done by the acceptance walk's own workgroup (one launch less).
 * Arguments: those of medusa_accept, then the cache arguments of
 * medusa_kv_compact (Kc, Vc [b, nkv, Pmax, d] dtype, seq_len [b] device, in:
 * P, out: P + L + 1; K is medusa_accept's K), then verify_ws: NULL, or the
 * workspace of the medusa_verify_logits call that wrote base_logits (same
 * rows b*T, V, mode and temperature); with it the per-node argmax /
 * softmax statistics come from its partials instead of a pass over
 * base_logits.  The statistics then differ only in float32 rounding, so the
 * outputs are the same except for a node whose typical-acceptance margin is
 * within that rounding.  The partials carry a record of the call that made
 * them (rows, V, greedy keys or tempered statistics, temperature); when it
 * does not match this call the kernel reads base_logits instead (slower, and
 * never past the partials).  Errors: the union of both calls' checks; nothing
 * is launched on error.
 * ------------------------------------------------------------------------- */
int medusa_accept_compact(const float* base_logits, const int32_t* tokens, const int32_t* parent,
                          const int32_t* depth, int32_t b, int32_t T, int32_t V, int32_t K,
                          int32_t mode, float temperature, float eps, float delta, uint64_t seed,
                          uint64_t step, int32_t* L, int32_t* path, int32_t* acc_tokens,
                          int32_t* bonus, void* Kc, void* Vc, int32_t* seq_len, int32_t nkv,
                          int32_t Pmax, int32_t d, int32_t dtype, const void* verify_ws,
                          void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * medusa_verify_logits - the verify-rows LM projection of medusa_heads
 * (n_heads = 0, include_base = 1: logits [rows, V] f32 = x [rows, H] . LM^T)
 * that also leaves, in ws, the acceptance statistics of every row per weight
 * tile: the argmax key (GREEDY) or the online softmax statistics of
 * logits / temperature (TYPICAL and REJECT).  medusa_accept_compact consumes them
 * (verify_ws), so acceptance does not re-read the logits.  Below 2^24 logits
 * (rows * V) re-reading is cheaper: then no partials are kept and
 * medusa_accept_compact reads the logits as without verify_ws.  [glossary]
 * verification phase: the original output head scores every candidate.
 *   x [rows, H], LM [V, H] (dtype); logits [rows, V] f32, as medusa_heads.
 *   ws: medusa_verify_workspace(rows, H, V, dtype, mode) bytes, 16-byte
 *       aligned, device, caller-owned; contents are opaque.
 * logits are bit-identical to medusa_heads.  Errors as medusa_heads.
 * Cache use (no effect on any value): this call, the step's last pass over
 * LM, reads LM with the non-temporal hint where the weight-stream kernel
 * runs (at most 80 rows over a vocabulary that is a multiple of 128 and at
 * least 30720), and stores the logits non-temporally when it keeps partials;
 * medusa_heads and medusa_lm_logits read LM without the hint, so a verify
 * call that follows them on the same LM finds much of it in the
 * last-level cache.
 * ------------------------------------------------------------------------- */
size_t medusa_verify_workspace(int64_t rows, int32_t H, int32_t V, int32_t dtype, int32_t mode);
int medusa_verify_logits(const void* x, int64_t rows, int32_t H, const void* LM, int32_t V,
                         int32_t dtype, int32_t mode, float temperature, float* logits, void* ws,
                         size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * medusa_kv_append / medusa_next_hidden - state carried between steps.
 * [glossary] (decoding loop; speculative KV cache): the tree's key/value
 * entries join the cache behind the accepted prefix for the verification
 * pass, and the next step drafts from the hidden state at the last accepted
 * position; [deep-dive] "What this deep dive assumes": the heads run off one
 * hidden state.
 *
 * medusa_kv_append, per sequence s with P = seq_len[s] (device):
 *   Kc[s, g, P + j, :] = Knew[s, g, j, :]   j = 0..T-1, every kv head g
 *   (same for Vc / Vnew).  Knew, Vnew [b, nkv, T, d] in the cache dtype; the
 *   cache is [b, nkv, Pmax, d].  seq_len is not changed.  A sequence with
 *   P < 0 or P + T > Pmax is left untouched.  Requires d * sizeof(dtype) % 16
 *   == 0 and 16-byte aligned buffers.
 * medusa_next_hidden, per sequence s:
 *   h[s, :] = O[s, path[s, L[s]], :]          O [b, T, H], h [b, H] (dtype)
 *   i.e. the verification state of the chosen node (path and L as written by
 *   medusa_accept / medusa_accept_compact; O as from medusa_tree_attn).  The
 *   next step's root is that step's bonus token (root_mode MEDUSA_ROOT_GIVEN
 *   with root = bonus).  Invalid L or path entries leave h[s] untouched.
 *   Requires H * sizeof(dtype) % 16 == 0 and 16-byte aligned O and h.
 * ------------------------------------------------------------------------- */
int medusa_kv_append(void* Kc, void* Vc, const int32_t* seq_len, const void* Knew,
                     const void* Vnew, int32_t b, int32_t nkv, int32_t Pmax, int32_t T, int32_t d,
                     int32_t dtype, void* stream);
int medusa_next_hidden(const void* O, const int32_t* path, const int32_t* L, int32_t b,
                       int32_t T, int32_t K, int32_t H, int32_t dtype, void* h, void* stream);

/* ---------------------------------------------------------------------------
 * The tree budget: medusa_tree_plan_rates (host only), medusa_topk_tree_tables,
 * medusa_accept_tally.
 * [deep-dive] "From top-k heads to a sparse candidate tree": the tree shape is
 * a tuned budget, more candidates (higher acceptance) against a heavier pass;
 * "What it costs on a CPU-bound SLM": the expected acceptance length (tokens
 * confirmed per pass) multiplies throughput; "The conditional-independence
 * gap": every head sees the same hidden state and nothing else.
 *
 * Rates q [K][MEDUSA_MAX_K] f64 (row d = head d+1, column r = rank r; entries
 * r >= k_d ignored, the rest in [0, 1]): q[d][r] is the rate at which the
 * rank-r candidate of head d+1 is accepted when its parent was.  With heads
 * independent given the hidden state, candidate (r_1..r_D) is accepted with
 * probability q[0][r_1] * ... * q[D-1][r_D] (f64, in that order).
 *
 * medusa_tree_plan_rates keeps the N candidates of largest probability under
 * (probability descending, D ascending, tuple ascending) -- the N-candidate
 * tree of most expected tokens, closed under ancestors since q <= 1 -- and
 * returns the tree as medusa_tree_plan does (host arrays, same node order)
 * plus *expected_tokens = 1 + the kept probabilities summed in node order.
 * N = -1 keeps all.  The fixed rule of medusa_tree_plan is the case
 * q[d][r] = decay^(d+1) / (r + 1) (up to the order of exact ties).
 *
 * medusa_topk_tree_tables is medusa_topk_tree for a tree given by host
 * tables plan_parent / plan_rank [T] (as filled by either planner): node 0
 * the root (parent -1), 0 <= parent[i] < i, depths (derived from the parents)
 * never decreasing along the node order and <= K, rank[i] < k of its head,
 * no two children of one node with the same rank.  Outputs as
 * medusa_topk_tree for that tree.  MEDUSA_ERR_ARG on an invalid table.
 *
 * medusa_accept_tally adds one batch of steps to the counts accepted and
 * offered [K][MEDUSA_MAX_K] i64 (device, 8-byte aligned, zeroed by the caller
 * before the first batch; calls add): for sequence s with 0 <= L[s] <= K and
 * the accepted path path[s, 0..L[s]] (as written by medusa_accept), a node of
 * depth D and rank r was offered when its parent is path[s, D-1], and accepted
 * when it is path[s, D]; offered[D-1][r] and accepted[D-1][r] count them.
 * accepted / offered estimates q.  The tree is given by host tables as for
 * medusa_topk_tree_tables.  Calls that overlap on one counts buffer add
 * atomically.
 * ------------------------------------------------------------------------- */
int medusa_tree_plan_rates(const int32_t* k_host, int32_t K, int32_t N, const double* q,
                           int32_t* parent, int32_t* depth, int32_t* rank, int32_t T_cap,
                           int32_t* T_out, double* expected_tokens);
int medusa_topk_tree_tables(const float* logits, int32_t b, int32_t K, int32_t V,
                            const int32_t* k_host, int32_t kmax, const int32_t* plan_parent,
                            const int32_t* plan_rank, int32_t T, int32_t root_mode,
                            float temperature, uint64_t seed, uint64_t step,
                            const int32_t* seq_len, int32_t* root, int32_t* idx, float* val,
                            int32_t* tokens, int32_t* pos, int32_t* parent, int32_t* depth,
                            uint64_t* anc, int32_t anc_words, void* ws, size_t ws_bytes,
                            void* stream);
int medusa_accept_tally(const int32_t* L, const int32_t* path, int32_t b, const int32_t* k_host,
                        int32_t K, const int32_t* plan_parent, const int32_t* plan_rank,
                        int32_t T, int64_t* accepted, int64_t* offered, void* stream);

/* ---------------------------------------------------------------------------
 * medusa_hydra_draft - Hydra-style sequentially dependent draft heads.
 * zackli.ai "Speculative Decoding Deep Dive II: Medusa, MTP", "Medusa": the
 * Medusa heads never see the token just drafted (accuracy falls with the
 * offset); Hydra feeds that token to the later heads -- better drafts, less
 * parallelism.  Reading taken (the pages give one sentence): head d of the
 * residual form ([deep-dive] heads section) takes y = bf16(h + E[x]) in place
 * of h, E [V,H] the base model's input embedding and x the token one position
 * earlier on the candidate's path (the root for head 1):
 *   u = bf16(y + SiLU(W_d y)),  logits = LM u  (f32),
 * evaluated for every node of depth d-1; node (r_1..r_d) of the tree takes
 * rank r_d of its parent's top-k_d (descending, ties to the lower index).
 * With E = 0 this is the Medusa draft.  One LM pass per depth, sequential.
 *
 * h [b,H], E [V,H], W [K,H,H] (head d = W[d-1], out x in), LM [V,H]: bf16,
 * device, 16-byte aligned; H % 128 == 0.  k_host[K], kmax, the tree as host
 * tables plan_parent / plan_rank [T] (as for medusa_topk_tree_tables).  The
 * root: argmax (MEDUSA_GREEDY) or seeded sample at `temperature`
 * (MEDUSA_TYPICAL, counter draw 0) of LM h, or given in root[b]
 * (MEDUSA_ROOT_GIVEN); tokens outside [0, V) read as the nearest end.
 * Outputs (device) as medusa_topk_tree: root [b], tokens / pos [b,T] (pos =
 * seq_len[s] + depth), parent / depth [T], anc [T][anc_words].  logits_out
 * (optional, NULL = none) [b,T,V] f32: row (s, p) = the head logits that node
 * p's children were drawn from, for every node above the deepest depth.
 * ws: medusa_hydra_workspace() bytes, 16-byte aligned.  b * (the largest node
 * count of a depth above the deepest) must not exceed 32767
 * (MEDUSA_ERR_UNSUPPORTED).  The draft then feeds medusa_tree_attn and the
 * rest of the step unchanged.
 * ------------------------------------------------------------------------- */
size_t medusa_hydra_workspace(int32_t b, int32_t H, int32_t V, const int32_t* k_host, int32_t K,
                              int32_t kmax, const int32_t* plan_parent, const int32_t* plan_rank,
                              int32_t T);
int medusa_hydra_draft(const void* h, int32_t b, int32_t H, const void* E, int32_t V,
                       const void* W, int32_t K, const void* LM, const int32_t* k_host,
                       int32_t kmax, const int32_t* plan_parent, const int32_t* plan_rank,
                       int32_t T, int32_t root_mode, float temperature, uint64_t seed,
                       uint64_t step, const int32_t* seq_len, int32_t* root, int32_t* tokens,
                       int32_t* pos, int32_t* parent, int32_t* depth, uint64_t* anc,
                       int32_t anc_words, float* logits_out, void* ws, size_t ws_bytes,
                       void* stream);

/* ---------------------------------------------------------------------------
 * medusa_mtp_draft - MTP-style draft heads: one transformer layer per head.
 * zackli.ai "Speculative Decoding Deep Dive II: Medusa, MTP", "MTP": the
 * trunk's h_t feeds n heads that are transformer layers f_{h_i}, the logits
 * are f_u(f_{h_i}(h_t)) through one shared unembedding, and the drafts take
 * the same tree verification as Medusa heads.  Reading taken (the page gives
 * no layer shape): head i is one pre-norm layer of the trunk's kind at the
 * current position,
 *   a  = RMSNorm(h; g1_i)                 RMSNorm(x; g) = x / sqrt(mean(x^2) + eps) * g
 *   q, k, v = a Wq_i^T, a Wk_i^T, a Wv_i^T      (nq / nkv heads of dim d)
 *   o  = softmax(q k^T / sqrt(d)) v  over the head's cache [0, P) and (k, v)
 *        at slot P = seq_len[s]; q head j reads kv head floor(j * nkv / nq)
 *   x1 = h + o Wo_i^T,  a2 = RMSNorm(x1; g2_i)
 *   y  = x1 + (SiLU(a2 Wg_i^T) * (a2 Wu_i^T)) Wd_i^T
 * and the outputs are those of medusa_heads: u [b, K+1, H] (slot 0 = h, slot
 * i = y of head i) and logits [b, K+1, V] f32 = LM u, so medusa_topk_tree and
 * the rest of the step follow unchanged.
 *
 *   h [b, H]; g1, g2 [K, H]; Wqkv [K, (nq + 2 nkv) d, H] (rows: Wq, then Wk,
 *   then Wv); Wo [K, H, nq d]; Wgu [K, 2F, H] with rows 2j = Wg row j and
 *   2j+1 = Wu row j (interleaved); Wd [K, H, F]; LM [V, H]: bf16, device.
 *   Kh, Vh [K, b, nkv, Pmax, d] bf16: each head's cache; on return slot
 *   seq_len[s] of every head holds the current position's k, v (nothing is
 *   written for a sequence with seq_len outside [0, Pmax), whose attention
 *   rows are then NaN).  seq_len [b] device, not changed.
 *   u_out [b, K+1, H] bf16 or NULL (kept in the workspace); logits f32.
 *   ws: medusa_mtp_workspace(b, H, K, F, nq, nkv, d, Pmax, u_out != NULL)
 *   bytes, 16-byte aligned.
 * Requires H, F and nq*d multiples of 128, d in {64, 128}, nq % nkv == 0,
 * every pointer 16-byte aligned.  bf16 operands with f32 accumulation;
 * a, q, k, v, o, x1, a2, the SwiGLU product and y are stored in bf16.
 * ------------------------------------------------------------------------- */
size_t medusa_mtp_workspace(int32_t b, int32_t H, int32_t K, int32_t F, int32_t nq, int32_t nkv,
                            int32_t d, int32_t Pmax, int32_t keep_u);
int medusa_mtp_draft(const void* h, int32_t b, int32_t H, int32_t K, const void* g1,
                     const void* Wqkv, const void* Wo, const void* g2, const void* Wgu,
                     const void* Wd, int32_t F, float eps, void* Kh, void* Vh,
                     const int32_t* seq_len, int32_t nq, int32_t nkv, int32_t d, int32_t Pmax,
                     const void* LM, int32_t V, void* u_out, float* logits, void* ws,
                     size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * medusa_stream_read - a plain read of a device buffer, computing nothing of
 * the method: the yardstick for the weight streams.  [deep-dive] "What it
 * costs on a CPU-bound SLM": the step's pace is set by the memory traffic of
 * the weight reads; timing this call on a buffer of a weight stream's size
 * gives the read rate the part reaches for that many bytes.
 *   buf    device, `bytes` readable, 16-byte aligned; bytes a multiple of 16
 *          (bytes == 0 launches nothing)
 *   never  a 32-bit value; each thread folds the 32-bit words it read by
 *          XOR and writes `never` to sink[0] (device, 4 bytes) only when its
 *          fold equals `never`, so the loads cannot be elided; with a value
 *          no fold takes nothing is written
 * Returns MEDUSA_ERR_ARG for a NULL or misaligned pointer or a size that is
 * not a multiple of 16.
 * ------------------------------------------------------------------------- */
int medusa_stream_read(const void* buf, size_t bytes, uint32_t never, void* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MEDUSA_H */
