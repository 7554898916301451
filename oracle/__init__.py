"""fp64 CPU oracle for differential softmax attention.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
cpu_baseline leg are the only callers. The product path never imports this
package, and this package imports nothing from the product.

It wraps ``diffattn_oracle.c`` (plain loops in double) and arranges numpy
arrays into the per-head blocks the C code takes. Layouts follow the product's
token-major convention: ``[batch, tokens, heads, dim]``.

What it computes, with the pages it follows:
  - ``lambda_init``, ``lam``: "Differential Transformer: Noise-Canceling
    Attention by Subtraction", section "Making lambda learnable and stable".
  - ``v1_forward``, ``decode``: the DiffAttn formula of "The mechanism" on the
    same page and of "softmax can't say zero, so it subtracts", section
    "The mechanism, exactly"; the epilogue of "The row no longer sums to one".
  - ``v2_forward``: "softmax can't say zero, so it subtracts", section
    "DIFF V2: what the authors changed", and the "Differential Transformer V2"
    write-up (paired heads of one GQA group, contiguous group heads).
  - ``gather_pages``: the storage convention of the paged decodes (a cache
    held in fixed-size pages listed by a block table) read back as a
    contiguous cache; the paged decodes compute ``decode`` / ``v2_decode`` of
    that cache.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def _load():
    global _lib
    if _lib is None:
        path = _build.LIB
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
            _build.build(force=True)
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.oracle_lambda_init.restype = ctypes.c_double
        lib.oracle_lambda_init.argtypes = [ctypes.c_int]
        lib.oracle_lambda.restype = None
        lib.oracle_lambda.argtypes = [dp, dp, dp, dp, ctypes.c_int, ctypes.c_int, ctypes.c_int, dp]
        lib.oracle_diff_head.restype = ctypes.c_int
        lib.oracle_diff_head.argtypes = [dp, dp, dp, dp, dp, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, dp, ctypes.c_int,
                                         ctypes.c_double, ctypes.POINTER(ctypes.c_int32),
                                         ctypes.c_int, dp]
        lib.oracle_rmsnorm_scale.restype = None
        lib.oracle_rmsnorm_scale.argtypes = [dp, ctypes.c_int, ctypes.c_int, dp,
                                             ctypes.c_double, ctypes.c_double]
        lib.oracle_diff_head_bwd.restype = ctypes.c_int
        lib.oracle_diff_head_bwd.argtypes = [dp, dp, dp, dp, dp, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_int, dp, ctypes.c_int,
                                             ctypes.c_double, dp, dp, dp, dp, dp, dp, dp]
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        _lib = lib
    return _lib


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def lambda_init(layer: int) -> float:
    """0.8 - 0.6 exp(-0.3 (l - 1)), l counted from 1."""
    return float(_load().oracle_lambda_init(int(layer)))


def lam(lq1, lk1, lq2, lk2, layer: int) -> np.ndarray:
    """exp(lq1.lk1) - exp(lq2.lk2) + lambda_init(layer), per row of [n, dim]."""
    a = [_f64(x) for x in (lq1, lk1, lq2, lk2)]
    if a[0].ndim == 1:
        a = [x[None, :] for x in a]
    n, dim = a[0].shape
    out = np.empty(n, dtype=np.float64)
    _load().oracle_lambda(*(_ptr(x) for x in a), n, dim, int(layer), _ptr(out))
    return out


def _head(q1, q2, k1, k2, v, lam_rows, causal, scale, rows):
    """q1, q2: [nq, d]; k1, k2: [nk, d]; v: [nk, dv]; lam_rows: [nq]."""
    q1, q2, k1, k2, v, lam_rows = (_f64(x) for x in (q1, q2, k1, k2, v, lam_rows))
    nq, d = q1.shape
    nk, dv = v.shape
    if rows is None:
        nrows, rp = nq, None
    else:
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
        nrows, rp = rows.size, rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    out = np.empty((nrows, dv), dtype=np.float64)
    rc = _load().oracle_diff_head(_ptr(q1), _ptr(q2), _ptr(k1), _ptr(k2), _ptr(v), nq, nk, d, dv,
                                  _ptr(lam_rows), int(bool(causal)), float(scale), rp, nrows,
                                  _ptr(out))
    if rc != 0:
        raise ValueError("oracle: a requested row sees no key (or allocation failed)")
    return out


def _epilogue(o, g, eps, lambda_init_value):
    o = np.ascontiguousarray(o, dtype=np.float64)
    nrows, dv = o.shape
    gkeep = None if g is None else _f64(g)   # keep the buffer alive across the call
    gp = None if gkeep is None else _ptr(gkeep)
    _load().oracle_rmsnorm_scale(_ptr(o), nrows, dv, gp, float(eps), float(lambda_init_value))
    return o


def default_scale(d: int) -> float:
    return 1.0 / np.sqrt(d)


def v1_forward(q1, q2, k1, k2, v, lam_heads, causal=True, epilogue=True, lambda_init_value=0.8,
               g=None, eps=1e-5, scale=None, rows=None):
    """DIFF V1 forward.

    q1, q2: [B, Nq, H, d]; k1, k2: [B, Nk, H, d]; v: [B, Nk, H, dv]; lam_heads: [H].
    rows: None for every output, else an int array [n, 3] of (b, h, i).
    Returns [B, Nq, H, dv] (rows is None) or [n, dv].
    """
    q1, q2, k1, k2, v = (np.asarray(x) for x in (q1, q2, k1, k2, v))
    B, Nq, H, d = q1.shape
    dv = v.shape[3]
    s = default_scale(d) if scale is None else float(scale)
    lam_heads = np.asarray(lam_heads, dtype=np.float64).reshape(-1)
    if rows is None:
        out = np.empty((B, Nq, H, dv), dtype=np.float64)
        for b in range(B):
            for h in range(H):
                o = _head(q1[b, :, h], q2[b, :, h], k1[b, :, h], k2[b, :, h], v[b, :, h],
                          np.full(Nq, lam_heads[h]), causal, s, None)
                if epilogue:
                    o = _epilogue(o, g, eps, lambda_init_value)
                out[b, :, h] = o
        return out
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    out = np.empty((rows.shape[0], dv), dtype=np.float64)
    for b in np.unique(rows[:, 0]):
        for h in np.unique(rows[rows[:, 0] == b, 1]):
            sel = np.nonzero((rows[:, 0] == b) & (rows[:, 1] == h))[0]
            o = _head(q1[b, :, h], q2[b, :, h], k1[b, :, h], k2[b, :, h], v[b, :, h],
                      np.full(Nq, lam_heads[h]), causal, s, rows[sel, 2])
            if epilogue:
                o = _epilogue(o, g, eps, lambda_init_value)
            out[sel] = o
    return out


def decode(q1, q2, k1c, k2c, vc, lam_heads, cache_lens=None, epilogue=True, lambda_init_value=0.8,
           g=None, eps=1e-5, scale=None, pairs=None):
    """DIFF V1 decode: one query per (b, h) against the first cache_lens[b] cached keys.

    q1, q2: [B, H, d]; k1c, k2c: [B, L, H, d]; vc: [B, L, H, dv].
    pairs: None for every (b, h), else an int array [n, 2] of (b, h); returns [B, H, dv] or [n, dv].
    """
    q1, q2 = np.asarray(q1), np.asarray(q2)
    B, H, d = q1.shape
    L = k1c.shape[1]
    dv = vc.shape[3]
    s = default_scale(d) if scale is None else float(scale)
    lens = np.full(B, L, dtype=np.int64) if cache_lens is None else np.asarray(cache_lens, np.int64)
    lam_heads = np.asarray(lam_heads, dtype=np.float64).reshape(-1)
    if pairs is None:
        pairs = np.array([(b, h) for b in range(B) for h in range(H)], dtype=np.int64)
        full = True
    else:
        pairs = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
        full = False
    out = np.empty((pairs.shape[0], dv), dtype=np.float64)
    for n, (b, h) in enumerate(pairs):
        n_b = int(lens[b])
        o = _head(q1[b, h][None], q2[b, h][None], k1c[b, :n_b, h], k2c[b, :n_b, h],
                  vc[b, :n_b, h], np.array([lam_heads[h]]), False, s, None)
        if epilogue:
            o = _epilogue(o, g, eps, lambda_init_value)
        out[n] = o[0]
    return out.reshape(B, H, dv) if full else out


def sigmoid(z):
    """1 / (1 + e^-z) in fp64: DIFF V2's lambda from its projected logit ("softmax can't say
    zero", section "DIFF V2: what the authors changed")."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def v2_forward(q, k, v, lam_tok, causal=True, scale=None, rows=None, lam_logits=False):
    """DIFF V2 forward (no per-head norm).

    q: [B, N, 2h, d]; k, v: [B, N, h_kv, d]; lam_tok: [B, N, h], lambda itself or, with
    lam_logits, the projected logits (lambda = sigmoid of them).
    Pair p takes query heads 2p (map 1) and 2p+1 (map 2); both read KV head
    2p // (2h / h_kv), since the heads of one GQA group are contiguous.
    rows: None, or an int array [n, 3] of (b, p, i). Returns [B, N, h, d] or [n, d].
    """
    q, k, v, lam_tok = (np.asarray(x) for x in (q, k, v, lam_tok))
    if lam_logits:
        lam_tok = sigmoid(lam_tok)
    B, N, H2, d = q.shape
    h = H2 // 2
    hkv = k.shape[2]
    group = H2 // hkv
    s = default_scale(d) if scale is None else float(scale)
    if rows is None:
        out = np.empty((B, N, h, v.shape[3]), dtype=np.float64)
        for b in range(B):
            for p in range(h):
                g = (2 * p) // group
                out[b, :, p] = _head(q[b, :, 2 * p], q[b, :, 2 * p + 1], k[b, :, g], k[b, :, g],
                                     v[b, :, g], lam_tok[b, :, p], causal, s, None)
        return out
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    out = np.empty((rows.shape[0], v.shape[3]), dtype=np.float64)
    for b in np.unique(rows[:, 0]):
        for p in np.unique(rows[rows[:, 0] == b, 1]):
            sel = np.nonzero((rows[:, 0] == b) & (rows[:, 1] == p))[0]
            g = (2 * p) // group
            out[sel] = _head(q[b, :, 2 * p], q[b, :, 2 * p + 1], k[b, :, g], k[b, :, g],
                             v[b, :, g], lam_tok[b, :, p], causal, s, rows[sel, 2])
    return out

def v2_decode(q, kc, vc, lam_pairs, cache_lens=None, scale=None, pairs=None, lam_logits=False):
    """DIFF V2 decode: the new token's query heads against the first cache_lens[b] cached keys.

    Each pair p subtracts query head 2p+1's attention from head 2p's with the token's lambda, both
    over the KV head of their GQA group ("softmax can't say zero", section "DIFF V2: what the
    authors changed"); no norm. q: [B, 2h, d]; kc, vc: [B, L, h_kv, d]; lam_pairs: [B, h]
    (logits whose sigmoid is lambda, with lam_logits).
    pairs: None for every (b, p), else an int array [n, 2] of (b, p); returns [B, h, d] or [n, d].
    """
    q, kc, vc, lam_pairs = (np.asarray(x) for x in (q, kc, vc, lam_pairs))
    if lam_logits:
        lam_pairs = sigmoid(lam_pairs)
    B, H2, d = q.shape
    L, hkv = kc.shape[1], kc.shape[2]
    group = H2 // hkv
    s = default_scale(d) if scale is None else float(scale)
    lens = np.full(B, L, dtype=np.int64) if cache_lens is None else np.asarray(cache_lens, np.int64)
    full = pairs is None
    if full:
        pairs = np.array([(b, p) for b in range(B) for p in range(H2 // 2)], dtype=np.int64)
    pairs = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    out = np.empty((pairs.shape[0], vc.shape[3]), dtype=np.float64)
    for n, (b, p) in enumerate(pairs):
        n_b = int(lens[b])
        g = (2 * p) // group
        out[n] = _head(q[b, 2 * p][None], q[b, 2 * p + 1][None], kc[b, :n_b, g], kc[b, :n_b, g],
                       vc[b, :n_b, g], np.array([lam_pairs[b, p]]), False, s, None)[0]
    return out.reshape(B, H2 // 2, -1) if full else out


def gather_pages(pool, block_table, length: int, page_size: int):
    """A paged cache read back as a contiguous one: token t of sequence b is row t % page_size of
    pool page block_table[b, t // page_size] (the storage convention of the paged decodes).
    pool: [P, page_size, H, D]; block_table: [B, >= ceil(length / page_size)]. Returns [B, length, H, D]."""
    pool, table = np.asarray(pool), np.asarray(block_table, dtype=np.int64)
    B = table.shape[0]
    out = np.empty((B, length) + pool.shape[2:], dtype=pool.dtype)
    for b in range(B):
        for t in range(length):
            out[b, t] = pool[table[b, t // page_size], t % page_size]
    return out


def v1_backward(q1, q2, k1, k2, v, lam_heads, dy, causal=True, epilogue=True, lambda_init_value=0.8,
                g=None, eps=1e-5, scale=None):
    """Gradients of the DIFF V1 forward (v1_forward) with respect to every input, for L = sum(dy * y).

    The RMSNorm part follows from y = k w o / r with r = sqrt(mean_c o_c^2 + eps), k = 1 - lambda_init
    ("Noise-Canceling Attention by Subtraction", section "Making lambda learnable and stable"):
    dL/dw_c = sum dy_c k o_c / r and dL/do = (du - u mean_c(du_c u_c)) / r with u = o / r,
    du = k w dy. The map part is oracle_diff_head_bwd. Shapes as v1_forward; dy: [B, N, H, dv].
    Returns a dict with dq1, dq2, dk1, dk2, dv (shaped like the inputs), dlam [H] and dg [dv]
    (None without epilogue).
    """
    q1, q2, k1, k2, v, dy = (np.asarray(x, dtype=np.float64) for x in (q1, q2, k1, k2, v, dy))
    B, Nq, H, d = q1.shape
    Nk, dv = k1.shape[1], v.shape[3]
    s = default_scale(d) if scale is None else float(scale)
    lam_heads = np.asarray(lam_heads, dtype=np.float64).reshape(-1)
    grads = {k: np.zeros_like(x) for k, x in (("dq1", q1), ("dq2", q2), ("dk1", k1), ("dk2", k2), ("dv", v))}
    dlam = np.zeros(H)
    dg = np.zeros(dv) if epilogue else None
    w = np.ones(dv) if g is None else np.asarray(g, dtype=np.float64)
    kappa = 1.0 - lambda_init_value
    L = _load()
    for b in range(B):
        for h in range(H):
            lam_rows = np.full(Nq, lam_heads[h])
            args = [_f64(x[b, :, h]) for x in (q1, q2, k1, k2, v)]
            o = _head(*args, lam_rows, causal, s, None)                 # [Nq, dv], pre-norm
            gy = dy[b, :, h]
            if epilogue:
                r = np.sqrt(np.mean(o * o, axis=1, keepdims=True) + eps)
                u = o / r
                dg += np.sum(gy * kappa * u, axis=0)
                du = kappa * w[None, :] * gy
                go = (du - u * np.mean(du * u, axis=1, keepdims=True)) / r
            else:
                go = gy
            go = _f64(go)
            outs = [np.empty((Nq, d)), np.empty((Nq, d)), np.empty((Nk, d)), np.empty((Nk, d)),
                    np.empty((Nk, dv)), np.empty(Nq)]
            rc = L.oracle_diff_head_bwd(*(_ptr(x) for x in args), Nq, Nk, d, dv, _ptr(lam_rows),
                                        int(bool(causal)), s, _ptr(go), *(_ptr(x) for x in outs))
            if rc != 0:
                raise ValueError("oracle_diff_head_bwd failed (a row with no visible key?)")
            for key, x in zip(("dq1", "dq2", "dk1", "dk2", "dv"), outs[:5]):
                grads[key][b, :, h] = x
            dlam[h] += outs[5].sum()
    grads["dlam"] = dlam
    grads["dg"] = dg
    return grads


def lambda_backward(lq1, lk1, lq2, lk2, dlam):
    """Gradients of lambda = exp(lq1 . lk1) - exp(lq2 . lk2) + lambda_init with respect to the four
    vectors ("Noise-Canceling Attention by Subtraction", section "Making lambda learnable and
    stable"), one row per head: d/dlq1 = dlam exp(lq1 . lk1) lk1, d/dlk1 = dlam exp(lq1 . lk1) lq1,
    and the same with a minus sign for the second pair."""
    lq1, lk1, lq2, lk2 = (np.atleast_2d(np.asarray(x, dtype=np.float64)) for x in (lq1, lk1, lq2, lk2))
    dlam = np.asarray(dlam, dtype=np.float64).reshape(-1, 1)
    e1 = np.exp(np.sum(lq1 * lk1, axis=1, keepdims=True))
    e2 = np.exp(np.sum(lq2 * lk2, axis=1, keepdims=True))
    return dict(dlq1=dlam * e1 * lk1, dlk1=dlam * e1 * lq1, dlq2=-dlam * e2 * lk2, dlk2=-dlam * e2 * lq2)


def v1_train_stats(q1, q2, k1, k2, v, causal=True, scale=None):
    """What the training forward saves for the backward pass, from the definitions:
    lse [B, H, Nq, 2]: per row and map log2(sum_j exp(s q . k_j)) * ... expressed in base 2 of the
    scaled scores, i.e. log2(e) * ln(sum_j exp(s q . k_j)) over the visible keys;
    maps [B, Nq, H, 2, dv]: A1 V and A2 V (each map's attention output, lambda = 0)."""
    q1, q2, k1, k2, v = (np.asarray(x, dtype=np.float64) for x in (q1, q2, k1, k2, v))
    B, Nq, H, d = q1.shape
    Nk, dv = k1.shape[1], v.shape[3]
    s = default_scale(d) if scale is None else float(scale)
    lse = np.empty((B, H, Nq, 2))
    maps = np.empty((B, Nq, H, 2, dv))
    for b in range(B):
        for h in range(H):
            for m, (q, k) in enumerate(((q1, k1), (q2, k2))):
                qq, kk = _f64(q[b, :, h]), _f64(k[b, :, h])
                maps[b, :, h, m] = _head(qq, qq, kk, kk, _f64(v[b, :, h]), np.zeros(Nq), causal, s, None)
                z = s * (qq @ kk.T)                                     # natural-unit logits
                for i in range(Nq):
                    n = Nk if not causal else min(Nk, i + (Nk - Nq) + 1)
                    zi = z[i, :n]
                    mx = zi.max()
                    lse[b, h, i, m] = (mx + np.log(np.sum(np.exp(zi - mx)))) / np.log(2.0)
    return lse, maps


def v2_backward(q, k, v, lam_tok, dy, causal=True, scale=None, lam_logits=False):
    """Gradients of the DIFF V2 forward (v2_forward) for L = sum(dy * out).

    Pair p is the V1 head difference of query heads 2p and 2p+1 over the group's K and V with a
    per-row lambda and no norm ("softmax can't say zero", section "DIFF V2: what the authors
    changed"), so each pair is oracle_diff_head_bwd with K1 = K2 = K_g and go = dy; K and V
    gradients add up over the heads of the group. With lam_logits the lambda gradient is carried
    through the sigmoid: dL/dz = dL/dlambda * lambda (1 - lambda).
    q: [B, Nq, 2h, d]; k, v: [B, Nk, h_kv, d]; lam_tok: [B, Nq, h]; dy: [B, Nq, h, d]. Nq may be
    smaller than Nk: the queries are then the last Nq rows of the sequence (query i sees keys
    j <= i + Nk - Nq), whose gradients are exact for them and, for keys past Nk - Nq, complete
    (no earlier query sees those keys).
    Returns a dict with dq, dk, dv (shaped like the inputs) and dlam [B, Nq, h].
    """
    q, k, v, dy = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dy))
    lam_tok = np.asarray(lam_tok, dtype=np.float64)
    lam_val = sigmoid(lam_tok) if lam_logits else lam_tok
    B, N, H2, d = q.shape
    Nk = k.shape[1]
    h, hkv = H2 // 2, k.shape[2]
    group = H2 // hkv
    s = default_scale(d) if scale is None else float(scale)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dlam = np.zeros((B, N, h))
    L = _load()
    for b in range(B):
        for p in range(h):
            g = (2 * p) // group
            args = [_f64(q[b, :, 2 * p]), _f64(q[b, :, 2 * p + 1]), _f64(k[b, :, g]), _f64(k[b, :, g]),
                    _f64(v[b, :, g])]
            lam_rows = _f64(lam_val[b, :, p])
            outs = [np.empty((N, d)), np.empty((N, d)), np.empty((Nk, d)), np.empty((Nk, d)),
                    np.empty((Nk, v.shape[3])), np.empty(N)]
            rc = L.oracle_diff_head_bwd(*(_ptr(x) for x in args), N, Nk, d, v.shape[3], _ptr(lam_rows),
                                        int(bool(causal)), s, _ptr(_f64(dy[b, :, p])), *(_ptr(x) for x in outs))
            if rc != 0:
                raise ValueError("oracle_diff_head_bwd failed")
            dq[b, :, 2 * p] = outs[0]
            dq[b, :, 2 * p + 1] = outs[1]
            dk[b, :, g] += outs[2] + outs[3]
            dv[b, :, g] += outs[4]
            dlam[b, :, p] = outs[5] * (lam_rows * (1.0 - lam_rows) if lam_logits else 1.0)
    return dict(dq=dq, dk=dk, dv=dv, dlam=dlam)


def v2_train_stats(q, k, v, causal=True, scale=None):
    """What the V2 training forward saves, from the definitions: lse [B, h, N, 2], the base-2
    log-sum-exp of query heads 2p and 2p+1 over their group's keys, and maps [B, N, h, 2, d], the
    two heads' attention outputs A_{2p} V and A_{2p+1} V. It is v1_train_stats with Q1, Q2 the
    pair's heads and K1 = K2 = K_g, V = V_g."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, N, H2, d = q.shape
    h, hkv = H2 // 2, k.shape[2]
    group = H2 // hkv
    gk = np.stack([k[:, :, (2 * p) // group] for p in range(h)], axis=2)      # [B, N, h, d]
    gv = np.stack([v[:, :, (2 * p) // group] for p in range(h)], axis=2)
    return v1_train_stats(q[:, :, 0::2], q[:, :, 1::2], gk, gk, gv, causal=causal, scale=scale)


# ------------------------------------------------------------------------------------------------
# fp8 score operands. OCP e4m3: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0
# holds the subnormals m * 2^-9; the largest finite value is 448 (field 15, mantissa 6); field 15
# with mantissa 7 is NaN; there is no infinity.
# ------------------------------------------------------------------------------------------------

def e4m3_encode(x):
    """Codes (uint8) of fp32 values, rounded to nearest with ties to even. Magnitudes from 464 up
    (448 plus half a step) have no finite code and give NaN (0x7f), as does NaN."""
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x.astype(np.float64))
    code = np.zeros(x.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    code[sub] = np.rint(a[sub] / 2.0 ** -9).astype(np.int64)          # 0..8; 8 is the first normal
    nrm = ~sub & np.isfinite(a)
    mant, ex = np.frexp(a[nrm])                                          # a = mant * 2^ex, mant in [0.5, 1)
    e = ex - 1                                                           # a = (2 mant) * 2^e, 2 mant in [1, 2)
    q = np.rint((2.0 * mant - 1.0) * 8.0).astype(np.int64)              # 0..8
    e = e + (q == 8)
    q = np.where(q == 8, 0, q)
    code[nrm] = ((e + 7) << 3) | q
    code[(a >= 464.0) | np.isnan(a)] = 0x7F
    code = code | np.where(np.signbit(x), 0x80, 0)
    return code.astype(np.uint8)


def e4m3_decode(code):
    """Values (float64) of e4m3 codes; NaN for 0x7f and 0xff."""
    c = np.asarray(code, dtype=np.int64)
    E, m = (c >> 3) & 15, c & 7
    v = np.where(E == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (E - 7))
    v = np.where((E == 15) & (m == 7), np.nan, v)
    return np.where(c & 0x80, -v, v)


def quantize_fp8(x):
    """Dynamic absmax quantisation of a [B, N, H, dim] score operand, one scale per (batch, head)
    slice (the granularity the pages leave open): amax = max |x|, s = amax / 448 and
    r = 448 / amax in fp32 (both 1 when amax is 0), code = e4m3(x * r) with the product in fp32;
    x is about code * s. Returns (codes uint8, s [B, H] fp32).
    "softmax can't say zero, so it subtracts", section "Outliers, and the low-bit claim"."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=(1, 3))                               # [B, H]
    pos = amax > 0
    safe = np.where(pos, amax, np.float32(1.0)).astype(np.float32)
    s = np.where(pos, safe / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    r = np.where(pos, np.float32(448.0) / safe, np.float32(1.0)).astype(np.float32)
    codes = e4m3_encode(x * r[:, None, :, None])
    return codes, s


def dequantize_fp8(codes, s):
    """code * s per (batch, head) slice, in float64."""
    return e4m3_decode(codes) * np.asarray(s, dtype=np.float64)[:, None, :, None]
