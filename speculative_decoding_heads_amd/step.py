"""One Medusa draft-and-verify step as a sequence of libmedusa calls.

This module only allocates device buffers (through torch) and enqueues the
library calls in loop order (inferensys.com "Medusa Heads": draft, verify,
accept and roll back); every part of the step runs in the HIP kernels.

    heads      : medusa_heads(h)            -> logits [b, K+1, V]
                 (fused: medusa_heads_hidden + medusa_lm_logits, the same kernels)
    shortlists : medusa_topk(logits)        -> root [b], idx [b, K, kmax]
    tree       : medusa_build_tree          -> tokens, pos, parent, depth, anc
    verify     : medusa_tree_attn(Q, Kc, Vc)-> O [b, T, nq*d]
                 medusa_heads(O, base only) -> base_logits [b, T, V]
    accept     : medusa_accept              -> L, path, acc_tokens, bonus
    rollback   : medusa_kv_compact          -> Kc, Vc, seq_len updated

With ``fused=True`` (the default) shortlists + tree run as medusa_topk_tree, the
verify logits as medusa_verify_logits (which also leaves the acceptance
statistics per weight tile) and accept + rollback as medusa_accept_compact on
those statistics: the same outputs, three launches fewer.
"""

import torch

from . import medusa as M


class VerifyStep:
    def __init__(self, cfg, device="cuda", plan=None, draft="medusa"):
        """plan: optional host tables (parent, rank) of the tree, e.g. from
        medusa_tree_plan_rates (the tree budget); default: the fixed tree of
        cfg.N candidates.  Either way the tree has cfg.T nodes.

        draft: "medusa" (the K heads on h, one launch for shortlists + tree) or
        "hydra" (medusa_hydra_draft: head d on h + E[previous token], one LM
        pass per depth; bf16 and the fused path only; x needs "E")."""
        self.cfg = c = cfg
        if draft not in ("medusa", "hydra", "mtp"):
            raise ValueError("draft must be 'medusa', 'hydra' or 'mtp'")
        self.draft = draft
        if plan is not None:
            parent, rank = list(plan[0]), list(plan[1])
            if len(parent) != c.T or len(rank) != c.T:
                raise ValueError(f"plan: expected {c.T} nodes, got {len(parent)}")
            plan = (parent, rank)
        self.plan = plan
        self.device = device
        dt = M.BF16 if c.dtype == "bf16" else M.F32
        self.dt = dt
        # acceptance mode; the root is drawn (typical, rejection) or the argmax
        self.mode = {"greedy": M.GREEDY, "typical": M.TYPICAL, "reject": M.REJECT}[c.mode]
        self.root_mode = M.GREEDY if self.mode == M.GREEDY else M.TYPICAL
        self.N = c.N
        T, K = c.T, c.K
        i32 = dict(dtype=torch.int32, device=device)
        f32 = dict(dtype=torch.float32, device=device)
        act = torch.bfloat16 if dt == M.BF16 else torch.float32
        self.logits = torch.empty(c.b, K + 1, c.V, **f32)
        self.u = torch.empty(c.b, K + 1, c.H, dtype=act, device=device)
        self.root = torch.empty(c.b, **i32)
        self.idx = torch.empty(c.b, K, c.kmax, **i32)
        self.val = torch.empty(c.b, K, c.kmax, **f32)
        self.tokens = torch.empty(c.b, T, **i32)
        self.pos = torch.empty(c.b, T, **i32)
        self.parent = torch.empty(T, **i32)
        self.depth = torch.empty(T, **i32)
        self.anc_words = (T + 63) // 64
        self.anc = torch.empty(T, self.anc_words, dtype=torch.int64, device=device)
        self.O = torch.empty(c.b, T, c.nq * c.d, dtype=act, device=device)
        self.base_logits = torch.empty(c.b, T, c.V, **f32)
        self.L = torch.empty(c.b, **i32)
        self.path = torch.empty(c.b, K + 1, **i32)
        self.acc_tokens = torch.empty(c.b, K + 1, **i32)
        self.bonus = torch.empty(c.b, **i32)
        self.ws_topk = M.workspace(M.medusa_topk_workspace(c.b, K, c.V, c.kmax), device)
        self.ws_attn = M.workspace(
            M.medusa_tree_attn_workspace(c.b, T, c.nq, c.nkv, c.d, c.Pmax, dt), device)
        self.ws_acc = M.workspace(M.medusa_accept_workspace(c.b, T), device)
        self.ws_verify = M.workspace(
            M.medusa_verify_workspace(c.b * T, c.nq * c.d, c.V, dt, self.mode), device)
        if draft == "hydra":
            if dt != M.BF16:
                raise ValueError("the Hydra draft runs in bf16")
            if self.plan is None:
                par, _, rk = M.medusa_tree_plan(c.k, c.N, c.decay.numerator, c.decay.denominator)
                self.plan = (list(par), list(rk))
            self.ws_hydra = M.workspace(
                M.medusa_hydra_workspace(c.b, c.H, c.V, c.k, c.kmax, *self.plan), device)
        if draft == "mtp":
            if dt != M.BF16:
                raise ValueError("the MTP draft runs in bf16")
            self.ws_mtp = None          # sized on first use (the layer width comes with x)

    def fit_cache(self, Pmax):
        """Size the attention workspace for a cache of Pmax slots per (sequence,
        kv head): the split of the keys, and with it the workspace, follows
        the cache's capacity.  Allocates only when the current one is short."""
        c = self.cfg
        need = M.medusa_tree_attn_workspace(c.b, c.T, c.nq, c.nkv, c.d, Pmax, self.dt)
        if need > self.ws_attn.numel():
            self.ws_attn = M.workspace(need, self.device)

    def run(self, x, step=0, stream=None, fused=True, root_given=False):
        """Enqueue one step.  x: dict of device tensors h, W, LM, Q, Kc, Vc, seq_len.

        root_given: the tree root is the previous step's next token (self.bonus)
        instead of the base head's argmax / sample (fused path only)."""
        root_mode = M.ROOT_GIVEN if root_given else self.root_mode
        root = self.bonus if root_given else self.root
        if self.draft == "hydra":
            if not fused:
                raise ValueError("the Hydra draft needs the fused path")
            self.draft_hydra(x, step, root_mode, root, stream)
        elif self.draft == "mtp":
            if not fused:
                raise ValueError("the MTP draft needs the fused path")
            self.draft_mtp(x, step, root_mode, root, stream)
        else:
            self.draft_medusa(x, step, root_mode, root, fused, stream)
        self.verify(x, step, fused, stream)

    def draft_medusa(self, x, step, root_mode, root, fused, stream=None):
        """The Medusa draft of one step: head logits, root, shortlists and tree.
        Fused path: the heads' residual GEMM and their LM pass as two calls
        (medusa_heads_hidden, medusa_lm_logits: the kernels of medusa_heads)."""
        c = self.cfg
        if fused:
            M.medusa_heads_hidden(x["h"], x["W"], self.u, include_base=1, stream=stream)
            M.medusa_lm_logits(self.u, x["LM"], self.logits, reverse_k=1, stream=stream)
        else:
            M.medusa_heads(x["h"], x["W"], x["LM"], self.logits, include_base=1, u_out=self.u,
                           stream=stream)
        if fused and self.plan is not None:
            M.medusa_topk_tree_tables(self.logits, c.k, c.kmax, self.plan[0], self.plan[1],
                                      root_mode, c.temperature, c.seed, step, x["seq_len"], root,
                                      self.idx, self.val, self.tokens, self.pos, self.parent,
                                      self.depth, self.anc, self.ws_topk, stream=stream)
        elif fused:
            M.medusa_topk_tree(self.logits, c.k, c.kmax, self.N, c.decay.numerator,
                               c.decay.denominator, root_mode, c.temperature, c.seed, step,
                               x["seq_len"], root, self.idx, self.val, self.tokens, self.pos,
                               self.parent, self.depth, self.anc, self.ws_topk, stream=stream)
        else:
            if self.plan is not None:
                raise ValueError("a given tree plan needs the fused path")
            M.medusa_topk(self.logits, c.k, c.kmax, self.root_mode, c.temperature, c.seed, step,
                          self.root, self.idx, self.val, self.ws_topk, stream=stream)
            M.medusa_build_tree(c.k, self.N, c.decay.numerator, c.decay.denominator, self.root,
                                self.idx, x["seq_len"], self.tokens, self.pos, self.parent,
                                self.depth, self.anc, stream=stream)

    def draft_mtp(self, x, step, root_mode, root, stream=None):
        """The MTP-style draft of one step: K transformer-layer heads on h
        (medusa_mtp_draft: head logits in the layout of medusa_heads), then
        shortlists and tree as for Medusa heads.  x needs "mtp": the layers'
        weights and caches (synth.make_mtp_inputs, on the device)."""
        c = self.cfg
        w = x["mtp"]
        if self.ws_mtp is None:
            F = w["Wd"].shape[2]
            self.ws_mtp = M.workspace(M.medusa_mtp_workspace(c.b, c.H, c.K, F, c.nq, c.nkv, c.d,
                                                             w["Kh"].shape[3]), self.device)
        M.medusa_mtp_draft(x["h"], w, x["LM"], w["Kh"], w["Vh"], x["seq_len"], self.logits,
                           u_out=self.u, ws=self.ws_mtp, stream=stream)
        M.medusa_topk_tree(self.logits, c.k, c.kmax, self.N, c.decay.numerator,
                           c.decay.denominator, root_mode, c.temperature, c.seed, step,
                           x["seq_len"], root, self.idx, self.val, self.tokens, self.pos,
                           self.parent, self.depth, self.anc, self.ws_topk, stream=stream)

    def draft_hydra(self, x, step, root_mode, root, stream=None):
        """The Hydra-style draft of one step: root, tree tables and tokens."""
        c = self.cfg
        M.medusa_hydra_draft(x["h"], x["E"], x["W"], x["LM"], c.k, c.kmax, self.plan[0],
                             self.plan[1], root_mode, c.temperature, c.seed, step, x["seq_len"],
                             root, self.tokens, self.pos, self.parent, self.depth, self.anc,
                             self.ws_hydra, stream=stream)

    def verify(self, x, step, fused, stream=None):
        """Tree attention, verification logits, acceptance and KV rollback."""
        c = self.cfg
        M.medusa_tree_attn(x["Q"], x["Kc"], x["Vc"], x["seq_len"], self.anc, self.O,
                           ws=self.ws_attn, stream=stream)
        if fused:
            M.medusa_verify_logits(self.O.view(c.b * c.T, c.nq * c.d), x["LM"],
                                   self.base_logits.view(c.b * c.T, c.V), self.mode,
                                   c.temperature, self.ws_verify, stream=stream)
            M.medusa_accept_compact(self.base_logits, self.tokens, self.parent, self.depth, c.K,
                                    self.mode, c.temperature, c.eps, c.delta, c.seed, step, self.L,
                                    self.path, self.acc_tokens, self.bonus, x["Kc"], x["Vc"],
                                    x["seq_len"], self.ws_acc, verify_ws=self.ws_verify,
                                    stream=stream)
        else:
            M.medusa_heads(self.O.view(c.b * c.T, c.nq * c.d), None, x["LM"],
                           self.base_logits.view(c.b * c.T, c.V), include_base=1, stream=stream)
            M.medusa_accept(self.base_logits, self.tokens, self.parent, self.depth, c.K, self.mode,
                            c.temperature, c.eps, c.delta, c.seed, step, self.L, self.path,
                            self.acc_tokens, self.bonus, self.ws_acc, stream=stream)
            M.medusa_kv_compact(x["Kc"], x["Vc"], x["seq_len"], self.path, self.L, stream=stream)


class VerifyLoop:
    """Consecutive steps with the state carried on the device (the decoding
    loop of inferensys.com "Medusa Heads"): before step s the step's tree K/V
    join the cache behind the accepted prefix (medusa_kv_append); the step runs
    the five fused calls, step s >= 1 with the previous step's next token as
    the tree root; after it the chosen node's verification state becomes the
    next hidden state (medusa_next_hidden).  seq_len advances by L + 1 per step
    (the compaction).  The tree Q / K / V of each step are inputs (the
    backbone that would produce them is not part of this path).

    Every call only enqueues kernels, so ``run`` can be captured in a HIP
    graph (``capture``) and replayed."""

    def __init__(self, cfg, device="cuda", plan=None, draft="medusa"):
        self.cfg = cfg
        self.step = VerifyStep(cfg, device, plan, draft)

    def run(self, x, Qs, Kn, Vn, step0=0, root_given_first=False, stream=None, after_step=None):
        """x: h, W, LM (and E for the Hydra draft), Kc, Vc, seq_len (state, updated
        in place); Qs [S, b, T, nq, d],
        Kn / Vn [S, b, nkv, T, d].  after_step(s) runs after each step (eager use only)."""
        st = self.step
        st.fit_cache(x["Kc"].shape[2])
        for s in range(Qs.shape[0]):
            M.medusa_kv_append(x["Kc"], x["Vc"], x["seq_len"], Kn[s], Vn[s], stream=stream)
            xs = dict(x)
            xs["Q"] = Qs[s]
            st.run(xs, step=step0 + s, stream=stream, root_given=(s > 0 or root_given_first))
            M.medusa_next_hidden(st.O, st.path, st.L, x["h"], stream=stream)
            if after_step is not None:
                after_step(s)

    def capture(self, x, Qs, Kn, Vn, step0=0, root_given_first=False):
        """A torch CUDA (HIP) graph of ``run``; replaying it advances the state."""
        self.step.fit_cache(x["Kc"].shape[2])   # no allocation under capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.run(x, Qs, Kn, Vn, step0=step0, root_given_first=root_given_first)
        return g



def loop_inputs(cfg, steps, seed_base=0, device="cuda"):
    """Seeded per-step tree Q / K / V for ``VerifyLoop`` (N(0, 1), rounded to the
    workload dtype): Qs [S, b, T, nq, d], Kn / Vn [S, b, nkv, T, d]."""
    from .synth import normal
    c = cfg
    Qs = normal((steps, c.b, c.T, c.nq, c.d), seed_base + 101, 1.0, c.dtype)
    Kn = normal((steps, c.b, c.nkv, c.T, c.d), seed_base + 102, 1.0, c.dtype)
    Vn = normal((steps, c.b, c.nkv, c.T, c.d), seed_base + 103, 1.0, c.dtype)
    return Qs.to(device), Kn.to(device), Vn.to(device)


def device_inputs(cfg, host, device="cuda"):
    """Copy host inputs (from ``synth.make_inputs``) to the device, plus seq_len = P."""
    x = {k: v.to(device) for k, v in host.items()}
    x["seq_len"] = torch.full((cfg.b,), cfg.P, dtype=torch.int32, device=device)
    return x
