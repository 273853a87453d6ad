"""Python binding of libmedusa.so: argument marshalling only.

Each function has the name of the C entry point it calls (include/medusa.h)
and takes torch tensors (device memory) plus plain integers.  Nothing here
computes any part of the step; torch provides device memory and the current
HIP stream.  A missing library raises ``MedusaLibraryError``; a failed call
raises ``MedusaError`` with the library's message.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmedusa.so")

F32, BF16 = 0, 1
GREEDY, TYPICAL = 0, 1
ROOT_GIVEN = 2          # root_mode only: root[] is an input
REJECT = 3              # acceptance mode only: exact rejection sampling
MAX_K = 16              # shortlist size per head at most (columns of a rate table)
MAX_T = 256

_lib = None


class MedusaLibraryError(RuntimeError):
    pass


class MedusaError(RuntimeError):
    def __init__(self, name, status, msg):
        super().__init__(f"{name} failed with status {status}: {msg}")
        self.status = status


_P = ctypes.c_void_p
_I32, _I64, _U64, _F = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float
_SZ = ctypes.c_size_t

_SIGS = {
    "medusa_abi_version": ([], _I32),
    "medusa_status_str": ([_I32], ctypes.c_char_p),
    "medusa_last_error": ([], ctypes.c_char_p),
    "medusa_heads_workspace": ([_I64, _I32, _I32, _I32, _I32], _SZ),
    "medusa_heads": ([_P, _I64, _I32, _P, _I32, _P, _I32, _I32, _I32, _P, _P, _P, _SZ, _P], _I32),
    "medusa_heads_hidden": ([_P, _I64, _I32, _P, _I32, _I32, _I32, _P, _P], _I32),
    "medusa_lm_logits": ([_P, _I64, _I32, _P, _I32, _I32, _I32, _P, _P], _I32),
    "medusa_topk_workspace": ([_I32, _I32, _I32, _I32], _SZ),
    "medusa_topk": ([_P, _I32, _I32, _I32, _P, _I32, _I32, _F, _U64, _U64, _P, _P, _P, _P, _SZ,
                     _P], _I32),
    "medusa_tree_plan": ([_P, _I32, _I32, _I32, _I32, _P, _P, _P, _I32, _P], _I32),
    "medusa_build_tree": ([_P, _I32, _I32, _I32, _I32, _P, _P, _I32, _I32, _P, _P, _P, _P, _P, _P,
                           _I32, _P], _I32),
    "medusa_tree_attn_workspace": ([_I32, _I32, _I32, _I32, _I32, _I32, _I32], _SZ),
    "medusa_tree_attn": ([_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _F, _I32,
                          _P, _P, _SZ, _P], _I32),
    "medusa_tree_attn_noalloc": ([_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                  _F, _I32, _P, _P], _I32),
    "medusa_mtp_workspace": ([_I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32], _SZ),
    "medusa_mtp_draft": ([_P, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _I32, _F, _P, _P, _P, _I32,
                          _I32, _I32, _I32, _P, _I32, _P, _P, _P, _SZ, _P], _I32),
    "medusa_accept_workspace": ([_I32, _I32], _SZ),
    "medusa_accept": ([_P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _F, _F, _F, _U64, _U64, _P, _P,
                       _P, _P, _P, _SZ, _P], _I32),
    "medusa_kv_compact": ([_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _P], _I32),
    "medusa_topk_tree": ([_P, _I32, _I32, _I32, _P, _I32, _I32, _I32, _I32, _I32, _F, _U64, _U64,
                          _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _P, _SZ, _P], _I32),
    "medusa_accept_compact": ([_P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _F, _F, _F, _U64, _U64,
                               _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _P, _P, _SZ, _P],
                              _I32),
    "medusa_verify_workspace": ([_I64, _I32, _I32, _I32, _I32], _SZ),
    "medusa_verify_logits": ([_P, _I64, _I32, _P, _I32, _I32, _I32, _F, _P, _P, _SZ, _P], _I32),
    "medusa_kv_append": ([_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _P], _I32),
    "medusa_next_hidden": ([_P, _P, _P, _I32, _I32, _I32, _I32, _I32, _P, _P], _I32),
    "medusa_tree_plan_rates": ([_P, _I32, _I32, _P, _P, _P, _P, _I32, _P, _P], _I32),
    "medusa_topk_tree_tables": ([_P, _I32, _I32, _I32, _P, _I32, _P, _P, _I32, _I32, _F, _U64, _U64,
                                 _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _P, _SZ, _P], _I32),
    "medusa_accept_tally": ([_P, _P, _I32, _P, _I32, _P, _P, _I32, _P, _P, _P], _I32),
    "medusa_hydra_workspace": ([_I32, _I32, _I32, _P, _I32, _I32, _P, _P, _I32], _SZ),
    "medusa_hydra_draft": ([_P, _I32, _I32, _P, _I32, _P, _I32, _P, _P, _I32, _P, _P, _I32, _I32,
                            _F, _U64, _U64, _P, _P, _P, _P, _P, _P, _P, _I32, _P, _P, _SZ, _P],
                           _I32),
    "medusa_stream_read": ([_P, _SZ, ctypes.c_uint32, _P, _P], _I32),
}
EXPORTS = tuple(_SIGS)


def lib():
    """Load libmedusa.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MedusaLibraryError(
                f"{LIB_PATH} is missing; build it with `python -m speculative_decoding_heads_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _check(name, status):
    if status != 0:
        msg = lib().medusa_last_error().decode()
        raise MedusaError(name, status, msg)


def _i32_host(values):
    arr = (ctypes.c_int32 * len(values))(*[int(v) for v in values])
    return arr


def _need(cond, what):
    """Shape / dtype agreement between the tensors of one call (the C ABI takes
    raw pointers and sizes, so a mismatch here would become an out-of-bounds
    access there)."""
    if not cond:
        raise ValueError(what)


def _shape(t, shape, name):
    _need(t is not None and tuple(t.shape) == tuple(shape),
          f"{name}: expected shape {tuple(shape)}, got {None if t is None else tuple(t.shape)}")


def _dt(t, dtype, name):
    _need(t.dtype == dtype, f"{name}: expected {dtype}, got {t.dtype}")


def _tree_T(k, N, decay_num, decay_den):
    kk = _i32_host(k)
    T = ctypes.c_int32(0)
    st = lib().medusa_tree_plan(kk, len(k), -1 if N is None else N, decay_num, decay_den, None,
                                None, None, 0, ctypes.byref(T))
    _check("medusa_tree_plan", st)
    return T.value


def dtype_code(t):
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise ValueError(f"unsupported dtype {t.dtype}")


# ------------------------------------------------------------------ workspace queries
def medusa_heads_workspace(rows, H, n_heads, include_base, dtype):
    return lib().medusa_heads_workspace(rows, H, n_heads, include_base, dtype)


def medusa_topk_workspace(b, K, V, kmax):
    return lib().medusa_topk_workspace(b, K, V, kmax)


def medusa_tree_attn_workspace(b, T, nq, nkv, d, Pmax, dtype):
    return lib().medusa_tree_attn_workspace(b, T, nq, nkv, d, Pmax, dtype)


def medusa_accept_workspace(b, T):
    return lib().medusa_accept_workspace(b, T)


def workspace(nbytes, device="cuda"):
    """A byte buffer for a call's scratch memory (at least 1 byte)."""
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ calls
def medusa_heads(x, W, LM, logits, include_base=1, u_out=None, ws=None, stream=None):
    rows, H = x.shape
    n_heads = 0 if W is None else W.shape[0]
    V = LM.shape[0]
    R = (1 if include_base else 0) + n_heads
    _shape(LM, (V, H), "LM")
    _dt(LM, x.dtype, "LM")
    if W is not None:
        _shape(W, (n_heads, H, H), "W")
        _dt(W, x.dtype, "W")
    _need(logits.numel() == rows * R * V and logits.shape[-1] == V, "logits: expected rows*R*V entries")
    _dt(logits, torch.float32, "logits")
    if u_out is not None:
        _need(u_out.numel() == rows * R * H and u_out.shape[-1] == H, "u_out: expected rows*R*H entries")
        _dt(u_out, x.dtype, "u_out")
    st = lib().medusa_heads(_ptr(x), rows, H, _ptr(W), n_heads, _ptr(LM), V, dtype_code(x),
                            include_base, _ptr(u_out), _ptr(logits), _ptr(ws),
                            0 if ws is None else ws.numel(), _stream(stream))
    _check("medusa_heads", st)


def medusa_heads_hidden(x, W, u_out, include_base=1, stream=None):
    """u_out [rows, include_base + K, H]: the residual blocks of medusa_heads."""
    rows, H = x.shape
    n_heads = W.shape[0]
    _shape(W, (n_heads, H, H), "W")
    _dt(W, x.dtype, "W")
    R = (1 if include_base else 0) + n_heads
    _need(u_out.numel() == rows * R * H and u_out.shape[-1] == H, "u_out: expected rows*R*H entries")
    _dt(u_out, x.dtype, "u_out")
    st = lib().medusa_heads_hidden(_ptr(x), rows, H, _ptr(W), n_heads, dtype_code(x),
                                   include_base, _ptr(u_out), _stream(stream))
    _check("medusa_heads_hidden", st)


def medusa_lm_logits(x, LM, logits, reverse_k=0, stream=None):
    """logits [rows, V] = x [rows, H] . LM^T (x may be any view with rows of H)."""
    H = x.shape[-1]
    rows = x.numel() // H
    V = LM.shape[0]
    _shape(LM, (V, H), "LM")
    _dt(LM, x.dtype, "LM")
    _need(x.is_contiguous(), "x must be contiguous")
    _need(logits.numel() == rows * V and logits.shape[-1] == V, "logits: expected rows*V entries")
    _dt(logits, torch.float32, "logits")
    st = lib().medusa_lm_logits(_ptr(x), rows, H, _ptr(LM), V, dtype_code(x), int(reverse_k),
                                _ptr(logits), _stream(stream))
    _check("medusa_lm_logits", st)


def _topk_shapes(logits, k, kmax, root, idx, val):
    b, K1, V = logits.shape
    _dt(logits, torch.float32, "logits")
    _need(len(k) == K1 - 1, "len(k) must equal the number of head rows K")
    _shape(root, (b,), "root")
    _shape(idx, (b, K1 - 1, kmax), "idx")
    _shape(val, (b, K1 - 1, kmax), "val")
    _dt(root, torch.int32, "root")
    _dt(idx, torch.int32, "idx")
    _dt(val, torch.float32, "val")


def _tree_shapes(T, b, seq_len, tokens, pos, parent, depth, anc):
    _shape(seq_len, (b,), "seq_len")
    _shape(tokens, (b, T), "tokens")
    _shape(pos, (b, T), "pos")
    _shape(parent, (T,), "parent")
    _shape(depth, (T,), "depth")
    _need(anc.dim() == 2 and anc.shape[0] == T and anc.shape[1] >= (T + 63) // 64,
          "anc: expected [T, >= ceil(T/64)]")
    for t, n in ((seq_len, "seq_len"), (tokens, "tokens"), (pos, "pos"), (parent, "parent"),
                 (depth, "depth")):
        _dt(t, torch.int32, n)
    _dt(anc, torch.int64, "anc")


def medusa_topk(logits, k, kmax, root_mode, temperature, seed, step, root, idx, val, ws,
                stream=None):
    b, K1, V = logits.shape
    _topk_shapes(logits, k, kmax, root, idx, val)
    st = lib().medusa_topk(_ptr(logits), b, K1 - 1, V, _i32_host(k), kmax, root_mode,
                           temperature, seed, step, _ptr(root), _ptr(idx), _ptr(val), _ptr(ws),
                           0 if ws is None else ws.numel(), _stream(stream))
    _check("medusa_topk", st)


def medusa_tree_plan(k, N, decay_num=4, decay_den=5):
    """Host-only: (parent, depth, rank) lists of the fixed tree."""
    kk = _i32_host(k)
    T = ctypes.c_int32(0)
    st = lib().medusa_tree_plan(kk, len(k), -1 if N is None else N, decay_num, decay_den, None,
                                None, None, 0, ctypes.byref(T))
    _check("medusa_tree_plan", st)
    n = T.value
    par, dep, rk = (ctypes.c_int32 * n)(), (ctypes.c_int32 * n)(), (ctypes.c_int32 * n)()
    st = lib().medusa_tree_plan(kk, len(k), -1 if N is None else N, decay_num, decay_den, par, dep,
                                rk, n, ctypes.byref(T))
    _check("medusa_tree_plan", st)
    return list(par), list(dep), list(rk)


def _rates_host(k, q):
    """q: K rows of per-rank rates (sequences or a [K, >=k_d] array) -> f64 [K][16]."""
    K = len(k)
    _need(len(q) == K, "q: expected one row of rates per head")
    buf = (ctypes.c_double * (K * MAX_K))()
    for d in range(K):
        row = [float(x) for x in q[d]]
        _need(len(row) >= k[d], "q: row d needs k[d] rates")
        for r in range(k[d]):
            buf[d * MAX_K + r] = row[r]
    return buf


def medusa_tree_plan_rates(k, N, q):
    """Host-only: (parent, depth, rank, expected tokens) of the N-candidate tree
    with the largest path acceptance products under per-rank rates q."""
    kk = _i32_host(k)
    qq = _rates_host(k, q)
    T = ctypes.c_int32(0)
    e = ctypes.c_double(0.0)
    NN = -1 if N is None else N
    st = lib().medusa_tree_plan_rates(kk, len(k), NN, qq, None, None, None, 0, ctypes.byref(T),
                                      ctypes.byref(e))
    _check("medusa_tree_plan_rates", st)
    n = T.value
    par, dep, rk = (ctypes.c_int32 * n)(), (ctypes.c_int32 * n)(), (ctypes.c_int32 * n)()
    st = lib().medusa_tree_plan_rates(kk, len(k), NN, qq, par, dep, rk, n, ctypes.byref(T),
                                      ctypes.byref(e))
    _check("medusa_tree_plan_rates", st)
    return list(par), list(dep), list(rk), e.value


def medusa_build_tree(k, N, decay_num, decay_den, root, idx, seq_len, tokens, pos, parent, depth,
                      anc, stream=None):
    b, K, kmax = idx.shape
    _need(len(k) == K, "len(k) must equal idx.shape[1]")
    _shape(root, (b,), "root")
    _tree_shapes(_tree_T(k, N, decay_num, decay_den), b, seq_len, tokens, pos, parent, depth, anc)
    st = lib().medusa_build_tree(_i32_host(k), len(k), -1 if N is None else N, decay_num,
                                 decay_den, _ptr(root), _ptr(idx), b, kmax, _ptr(seq_len),
                                 _ptr(tokens), _ptr(pos), _ptr(parent), _ptr(depth), _ptr(anc),
                                 anc.shape[1], _stream(stream))
    _check("medusa_build_tree", st)


def medusa_tree_attn(Q, Kc, Vc, seq_len, anc, O, scale=None, ws=None, stream=None):
    b, T, nq, d = Q.shape
    nkv, Pmax = Kc.shape[1], Kc.shape[2]
    _shape(Kc, (b, nkv, Pmax, d), "Kc")
    _shape(Vc, (b, nkv, Pmax, d), "Vc")
    _shape(seq_len, (b,), "seq_len")
    _dt(seq_len, torch.int32, "seq_len")
    _need(anc.dim() == 2 and anc.shape[0] == T, "anc: expected [T, words]")
    _need(O.numel() == b * T * nq * d, "O: expected b*T*nq*d entries")
    for t, n in ((Kc, "Kc"), (Vc, "Vc"), (O, "O")):
        _dt(t, Q.dtype, n)
    if scale is None:
        scale = d ** -0.5
    st = lib().medusa_tree_attn(_ptr(Q), _ptr(Kc), _ptr(Vc), _ptr(seq_len), _ptr(anc), anc.shape[1],
                                b, T, nq, nkv, d, Pmax, scale, dtype_code(Q), _ptr(O), _ptr(ws),
                                0 if ws is None else ws.numel(), _stream(stream))
    _check("medusa_tree_attn", st)


def medusa_tree_attn_noalloc(Q, Kc, Vc, seq_len, anc, O, scale=None, stream=None):
    """medusa_tree_attn with the split-KV partials in the library's static
    device scratch (no workspace; allocates nothing)."""
    b, T, nq, d = Q.shape
    nkv, Pmax = Kc.shape[1], Kc.shape[2]
    _shape(Kc, (b, nkv, Pmax, d), "Kc")
    _shape(Vc, (b, nkv, Pmax, d), "Vc")
    _shape(seq_len, (b,), "seq_len")
    _dt(seq_len, torch.int32, "seq_len")
    _need(anc.dim() == 2 and anc.shape[0] == T, "anc: expected [T, words]")
    _need(O.numel() == b * T * nq * d, "O: expected b*T*nq*d entries")
    for t, n in ((Kc, "Kc"), (Vc, "Vc"), (O, "O")):
        _dt(t, Q.dtype, n)
    if scale is None:
        scale = d ** -0.5
    st = lib().medusa_tree_attn_noalloc(_ptr(Q), _ptr(Kc), _ptr(Vc), _ptr(seq_len), _ptr(anc),
                                        anc.shape[1], b, T, nq, nkv, d, Pmax, scale,
                                        dtype_code(Q), _ptr(O), _stream(stream))
    _check("medusa_tree_attn_noalloc", st)


def medusa_mtp_workspace(b, H, K, F, nq, nkv, d, Pmax, keep_u=True):
    return lib().medusa_mtp_workspace(b, H, K, F, nq, nkv, d, Pmax, 1 if keep_u else 0)


def medusa_mtp_draft(h, w, LM, Kh, Vh, seq_len, logits, u_out=None, eps=1e-6, ws=None,
                     stream=None):
    """MTP-style draft heads.  w: dict of bf16 device tensors g1 [K, H],
    Wqkv [K, (nq + 2 nkv) d, H], Wo [K, H, nq d], g2 [K, H], Wgu [K, 2F, H]
    (gate / up rows interleaved), Wd [K, H, F]; Kh, Vh [K, b, nkv, Pmax, d]."""
    b, H = h.shape
    K, _, nkv, Pmax, d = Kh.shape
    F = w["Wd"].shape[2]
    nq = w["Wo"].shape[2] // d
    V = LM.shape[0]
    _shape(w["g1"], (K, H), "g1")
    _shape(w["g2"], (K, H), "g2")
    _shape(w["Wqkv"], (K, (nq + 2 * nkv) * d, H), "Wqkv")
    _shape(w["Wo"], (K, H, nq * d), "Wo")
    _shape(w["Wgu"], (K, 2 * F, H), "Wgu")
    _shape(w["Wd"], (K, H, F), "Wd")
    _shape(Vh, (K, b, nkv, Pmax, d), "Vh")
    _shape(LM, (V, H), "LM")
    _shape(seq_len, (b,), "seq_len")
    _dt(seq_len, torch.int32, "seq_len")
    for t, n in [(h, "h"), (LM, "LM"), (Kh, "Kh"), (Vh, "Vh")] + [(w[k], k) for k in
                                                                  ("g1", "Wqkv", "Wo", "g2", "Wgu",
                                                                   "Wd")]:
        _dt(t, torch.bfloat16, n)
    _need(logits.numel() == b * (K + 1) * V and logits.shape[-1] == V,
          "logits: expected b*(K+1)*V entries")
    _dt(logits, torch.float32, "logits")
    if u_out is not None:
        _need(u_out.numel() == b * (K + 1) * H, "u_out: expected b*(K+1)*H entries")
        _dt(u_out, torch.bfloat16, "u_out")
    st = lib().medusa_mtp_draft(_ptr(h), b, H, K, _ptr(w["g1"]), _ptr(w["Wqkv"]), _ptr(w["Wo"]),
                                _ptr(w["g2"]), _ptr(w["Wgu"]), _ptr(w["Wd"]), F, eps, _ptr(Kh),
                                _ptr(Vh), _ptr(seq_len), nq, nkv, d, Pmax, _ptr(LM), V,
                                _ptr(u_out), _ptr(logits), _ptr(ws),
                                0 if ws is None else ws.numel(), _stream(stream))
    _check("medusa_mtp_draft", st)


def _accept_shapes(base_logits, tokens, parent, depth, K, L, path, acc_tokens, bonus):
    b, T, V = base_logits.shape
    _dt(base_logits, torch.float32, "base_logits")
    _shape(tokens, (b, T), "tokens")
    _shape(parent, (T,), "parent")
    _shape(depth, (T,), "depth")
    _shape(L, (b,), "L")
    _shape(path, (b, K + 1), "path")
    _shape(acc_tokens, (b, K + 1), "acc_tokens")
    _shape(bonus, (b,), "bonus")
    for t, n in ((tokens, "tokens"), (parent, "parent"), (depth, "depth"), (L, "L"),
                 (path, "path"), (acc_tokens, "acc_tokens"), (bonus, "bonus")):
        _dt(t, torch.int32, n)


def medusa_accept(base_logits, tokens, parent, depth, K, mode, temperature, eps, delta, seed, step,
                  L, path, acc_tokens, bonus, ws, stream=None):
    b, T, V = base_logits.shape
    _accept_shapes(base_logits, tokens, parent, depth, K, L, path, acc_tokens, bonus)
    st = lib().medusa_accept(_ptr(base_logits), _ptr(tokens), _ptr(parent), _ptr(depth), b, T, V, K,
                             mode, temperature, eps, delta, seed, step, _ptr(L), _ptr(path),
                             _ptr(acc_tokens), _ptr(bonus), _ptr(ws),
                             0 if ws is None else ws.numel(), _stream(stream))
    _check("medusa_accept", st)


def _cache_shapes(Kc, Vc, seq_len, b):
    _need(Kc.dim() == 4 and Kc.shape[0] == b, "Kc: expected [b, nkv, Pmax, d]")
    _shape(Vc, tuple(Kc.shape), "Vc")
    _dt(Vc, Kc.dtype, "Vc")
    _shape(seq_len, (b,), "seq_len")
    _dt(seq_len, torch.int32, "seq_len")


def medusa_kv_compact(Kc, Vc, seq_len, path, L, stream=None):
    b, nkv, Pmax, d = Kc.shape
    K = path.shape[1] - 1
    _cache_shapes(Kc, Vc, seq_len, b)
    _shape(path, (b, K + 1), "path")
    _shape(L, (b,), "L")
    st = lib().medusa_kv_compact(_ptr(Kc), _ptr(Vc), _ptr(seq_len), _ptr(path), _ptr(L), b, nkv,
                                 Pmax, d, K, dtype_code(Kc), _stream(stream))
    _check("medusa_kv_compact", st)


def medusa_topk_tree(logits, k, kmax, N, decay_num, decay_den, root_mode, temperature, seed, step,
                     seq_len, root, idx, val, tokens, pos, parent, depth, anc, ws, stream=None):
    b, K1, V = logits.shape
    _topk_shapes(logits, k, kmax, root, idx, val)
    _tree_shapes(_tree_T(k, N, decay_num, decay_den), b, seq_len, tokens, pos, parent, depth, anc)
    st = lib().medusa_topk_tree(_ptr(logits), b, K1 - 1, V, _i32_host(k), kmax,
                                -1 if N is None else N, decay_num, decay_den, root_mode,
                                temperature, seed, step, _ptr(seq_len), _ptr(root), _ptr(idx),
                                _ptr(val), _ptr(tokens), _ptr(pos), _ptr(parent), _ptr(depth),
                                _ptr(anc), anc.shape[1], _ptr(ws), 0 if ws is None else ws.numel(),
                                _stream(stream))
    _check("medusa_topk_tree", st)


def medusa_topk_tree_tables(logits, k, kmax, plan_parent, plan_rank, root_mode, temperature, seed,
                            step, seq_len, root, idx, val, tokens, pos, parent, depth, anc, ws,
                            stream=None):
    """medusa_topk_tree for a tree given by host tables (plan_parent, plan_rank)."""
    b, K1, V = logits.shape
    T = len(plan_parent)
    _need(len(plan_rank) == T, "plan_rank: expected one rank per node")
    _topk_shapes(logits, k, kmax, root, idx, val)
    _tree_shapes(T, b, seq_len, tokens, pos, parent, depth, anc)
    st = lib().medusa_topk_tree_tables(_ptr(logits), b, K1 - 1, V, _i32_host(k), kmax,
                                       _i32_host(plan_parent), _i32_host(plan_rank), T, root_mode,
                                       temperature, seed, step, _ptr(seq_len), _ptr(root), _ptr(idx),
                                       _ptr(val), _ptr(tokens), _ptr(pos), _ptr(parent),
                                       _ptr(depth), _ptr(anc), anc.shape[1], _ptr(ws),
                                       0 if ws is None else ws.numel(), _stream(stream))
    _check("medusa_topk_tree_tables", st)


def medusa_accept_tally(L, path, k, plan_parent, plan_rank, accepted, offered, stream=None):
    """Add one batch of steps to accepted / offered [K, 16] int64 (device)."""
    b = L.shape[0]
    K = len(k)
    T = len(plan_parent)
    _need(len(plan_rank) == T, "plan_rank: expected one rank per node")
    _shape(L, (b,), "L")
    _shape(path, (b, K + 1), "path")
    _dt(L, torch.int32, "L")
    _dt(path, torch.int32, "path")
    for t, n in ((accepted, "accepted"), (offered, "offered")):
        _shape(t, (K, MAX_K), n)
        _dt(t, torch.int64, n)
    st = lib().medusa_accept_tally(_ptr(L), _ptr(path), b, _i32_host(k), K,
                                   _i32_host(plan_parent), _i32_host(plan_rank), T,
                                   _ptr(accepted), _ptr(offered), _stream(stream))
    _check("medusa_accept_tally", st)


def medusa_accept_compact(base_logits, tokens, parent, depth, K, mode, temperature, eps, delta,
                          seed, step, L, path, acc_tokens, bonus, Kc, Vc, seq_len, ws,
                          verify_ws=None, stream=None):
    b, T, V = base_logits.shape
    _accept_shapes(base_logits, tokens, parent, depth, K, L, path, acc_tokens, bonus)
    _cache_shapes(Kc, Vc, seq_len, b)
    _, nkv, Pmax, d = Kc.shape
    st = lib().medusa_accept_compact(_ptr(base_logits), _ptr(tokens), _ptr(parent), _ptr(depth), b,
                                     T, V, K, mode, temperature, eps, delta, seed, step, _ptr(L),
                                     _ptr(path), _ptr(acc_tokens), _ptr(bonus), _ptr(Kc), _ptr(Vc),
                                     _ptr(seq_len), nkv, Pmax, d, dtype_code(Kc), _ptr(verify_ws),
                                     _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream))
    _check("medusa_accept_compact", st)


def medusa_verify_workspace(rows, H, V, dtype, mode):
    return lib().medusa_verify_workspace(rows, H, V, dtype, mode)


def medusa_verify_logits(x, LM, logits, mode, temperature, ws, stream=None):
    rows, H = x.shape
    V = LM.shape[0]
    _shape(LM, (V, H), "LM")
    _dt(LM, x.dtype, "LM")
    _need(logits.numel() == rows * V and logits.shape[-1] == V, "logits: expected rows*V entries")
    _dt(logits, torch.float32, "logits")
    st = lib().medusa_verify_logits(_ptr(x), rows, H, _ptr(LM), V, dtype_code(x), mode, temperature,
                                    _ptr(logits), _ptr(ws), 0 if ws is None else ws.numel(),
                                    _stream(stream))
    _check("medusa_verify_logits", st)


def medusa_kv_append(Kc, Vc, seq_len, Knew, Vnew, stream=None):
    """Tree K/V [b, nkv, T, d] into cache slots seq_len .. seq_len+T-1."""
    b, nkv, Pmax, d = Kc.shape
    _cache_shapes(Kc, Vc, seq_len, b)
    _need(Knew.dim() == 4 and Knew.shape[0] == b and Knew.shape[1] == nkv and Knew.shape[3] == d,
          "Knew: expected [b, nkv, T, d]")
    _shape(Vnew, tuple(Knew.shape), "Vnew")
    _dt(Knew, Kc.dtype, "Knew")
    _dt(Vnew, Kc.dtype, "Vnew")
    T = Knew.shape[2]
    st = lib().medusa_kv_append(_ptr(Kc), _ptr(Vc), _ptr(seq_len), _ptr(Knew), _ptr(Vnew), b, nkv,
                                Pmax, T, d, dtype_code(Kc), _stream(stream))
    _check("medusa_kv_append", st)


def medusa_next_hidden(O, path, L, h, stream=None):
    """h[s] = O[s, path[s, L[s]]] (O [b, T, H] or [b, T, nq, d]; h [b, H])."""
    b, T = O.shape[0], O.shape[1]
    H = O[0, 0].numel()
    K = path.shape[1] - 1
    _shape(path, (b, K + 1), "path")
    _shape(L, (b,), "L")
    _dt(path, torch.int32, "path")
    _dt(L, torch.int32, "L")
    _need(h.numel() == b * H and h.shape[0] == b, "h: expected [b, H]")
    _dt(h, O.dtype, "h")
    st = lib().medusa_next_hidden(_ptr(O), _ptr(path), _ptr(L), b, T, K, H, dtype_code(O), _ptr(h),
                                  _stream(stream))
    _check("medusa_next_hidden", st)


def medusa_stream_read(buf, sink, never=0x9E3779B9, stream=None):
    """Plain read of the whole of `buf` (a device tensor, 16-byte multiple):
    the yardstick for the weight streams.  Each thread folds the 32-bit words
    it read by XOR and writes `never` to sink (a 4-byte device tensor) only
    when its fold equals it."""
    _need(buf.is_contiguous(), "buf must be contiguous")
    nbytes = buf.numel() * buf.element_size()
    _need(sink.numel() * sink.element_size() >= 4, "sink: expected at least 4 bytes")
    st = lib().medusa_stream_read(_ptr(buf), nbytes, never & 0xFFFFFFFF, _ptr(sink), _stream(stream))
    _check("medusa_stream_read", st)


def medusa_hydra_workspace(b, H, V, k, kmax, plan_parent, plan_rank):
    return lib().medusa_hydra_workspace(b, H, V, _i32_host(k), len(k), kmax,
                                        _i32_host(plan_parent), _i32_host(plan_rank),
                                        len(plan_parent))


def medusa_hydra_draft(h, E, W, LM, k, kmax, plan_parent, plan_rank, root_mode, temperature, seed,
                       step, seq_len, root, tokens, pos, parent, depth, anc, ws, logits_out=None,
                       stream=None):
    """Hydra-style draft: per-depth heads on h + E[previous token] (bf16)."""
    b, H = h.shape
    V = E.shape[0]
    K = len(k)
    T = len(plan_parent)
    _need(len(plan_rank) == T, "plan_rank: expected one rank per node")
    _shape(E, (V, H), "E")
    _shape(W, (K, H, H), "W")
    _shape(LM, (V, H), "LM")
    for t, n in ((h, "h"), (E, "E"), (W, "W"), (LM, "LM")):
        _dt(t, torch.bfloat16, n)
    _shape(root, (b,), "root")
    _dt(root, torch.int32, "root")
    _tree_shapes(T, b, seq_len, tokens, pos, parent, depth, anc)
    if logits_out is not None:
        _shape(logits_out, (b, T, V), "logits_out")
        _dt(logits_out, torch.float32, "logits_out")
    st = lib().medusa_hydra_draft(_ptr(h), b, H, _ptr(E), V, _ptr(W), K, _ptr(LM), _i32_host(k),
                                  kmax, _i32_host(plan_parent), _i32_host(plan_rank), T, root_mode,
                                  temperature, seed, step, _ptr(seq_len), _ptr(root), _ptr(tokens),
                                  _ptr(pos), _ptr(parent), _ptr(depth), _ptr(anc), anc.shape[1],
                                  _ptr(logits_out), _ptr(ws), 0 if ws is None else ws.numel(),
                                  _stream(stream))
    _check("medusa_hydra_draft", st)
