"""CPU oracle of the sparse MoE layer forward (ctypes wrapper around liboracle.so).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The HIP library
and its Python binding never import it, and the two share no code: the only
common module is ``workloads`` (seeded random inputs, no layer arithmetic).

The arithmetic lives in ``moe_oracle.c`` (plain loops, fp64 accumulation,
``-ffp-contract=off``); this file only marshals numpy arrays and chains the
steps in the order the layer defines them:
logits -> exact top-k + softmax gates -> counts / offsets / stable expert-major
permutation / LIS -> per-row expert FFN -> weighted combine (+ shared experts).
Two variants of the dispatch are also here: the replica split of one heavy
expert (odd ranks of its flat assignment order go to an extra slot), and the
nested-width decode where each (token, slot) carries a width of 2, 3 or 4 bits
and rows are grouped by (expert, width).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

OK, ERR_ARG, ERR_NONFINITE = 0, 1, 2
F32, BF16 = 0, 1
ROUND_NONE, ROUND_BF16, ROUND_F32 = 0, 1, 2
SWIGLU, RELU = 0, 1
INT4_GROUP = 128


class OracleError(RuntimeError):
    pass


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (plain C11 + OpenMP, no contraction)."""
    if force or not os.path.exists(_LIB_PATH) or \
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    with _lock:
        if _lib is None:
            build()
            L = C.CDLL(_LIB_PATH)
            p, i, i64, d = C.c_void_p, C.c_int, C.c_int64, C.c_double
            L.orc_router_logits.argtypes = [p, i, p, p, i, i, i, p]
            L.orc_topk_gates.argtypes = [p, i, i, i, p, p]
            L.orc_permute.argtypes = [p, i, i, i, p, p, p, p, p]
            L.orc_expert_rows.argtypes = [p, i, i, i, i, p, p, p, i, i, p, p, i, p]
            L.orc_combine.argtypes = [p, p, p, p, i, i, i, p]
            L.orc_dequant_int4.argtypes = [p, p, p, i64, i, i, p]
            L.orc_replica_split.argtypes = [p, i, i, i, i, p]
            L.orc_dequant_mwq.argtypes = [p, p, p, p, p, p, p, i64, i, i, i, p]
            L.orc_floe_rows.argtypes = [p, i, i, p, p, p, p, p, p, i, p, p, p, p]
            L.orc_log_softmax_rows.argtypes = [p, i, i, p]
            L.orc_grid_topk.argtypes = [p, p, i, i, i, i, p, p]
            L.orc_atomic_rows.argtypes = [p, i, p, p, i, p, p, i, i, p, i, p]
            L.orc_round_bf16.argtypes = [d]
            L.orc_round_bf16.restype = d
            for f in ("orc_router_logits", "orc_topk_gates", "orc_permute", "orc_expert_rows",
                      "orc_combine", "orc_dequant_int4", "orc_replica_split", "orc_dequant_mwq",
                      "orc_floe_rows", "orc_log_softmax_rows", "orc_grid_topk",
                      "orc_atomic_rows"):
                getattr(L, f).restype = C.c_int
            _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _check(rc, what):
    if rc != OK:
        raise OracleError("%s failed with code %d" % (what, rc))


def _dt(a):
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    raise TypeError("expected bf16 bits (uint16) or float32, got %s" % a.dtype)


def round_bf16(v: float) -> float:
    return lib().orc_round_bf16(float(v))


# --- steps ---------------------------------------------------------------

def router_logits(x, w_r, b_r=None):
    x = np.ascontiguousarray(x)
    w_r = np.ascontiguousarray(w_r)
    assert _dt(x) == _dt(w_r)
    T, d = x.shape
    E = w_r.shape[0]
    out = np.empty((T, E), np.float32)
    b = None if b_r is None else np.ascontiguousarray(b_r, np.float32)
    _check(lib().orc_router_logits(_ptr(x), _dt(x), _ptr(w_r), _ptr(b), T, d, E, _ptr(out)),
           "router_logits")
    return out


def topk_gates(logits, k):
    logits = np.ascontiguousarray(logits, np.float32)
    T, E = logits.shape
    idx = np.empty((T, k), np.int32)
    gate = np.empty((T, k), np.float32)
    _check(lib().orc_topk_gates(_ptr(logits), T, E, k, _ptr(idx), _ptr(gate)), "topk_gates")
    return idx, gate


def permute(idx, E):
    idx = np.ascontiguousarray(idx, np.int32)
    T, k = idx.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    row_assign = np.empty(T * k, np.int32)
    assign_row = np.empty(T * k, np.int32)
    lis = np.empty(1, np.float64)
    _check(lib().orc_permute(_ptr(idx), T, E, k, _ptr(counts), _ptr(offsets), _ptr(row_assign),
                             _ptr(assign_row), _ptr(lis)), "permute")
    return counts, offsets, row_assign, assign_row, float(lis[0])


def replica_split(idx, E, heavy):
    """Assignments of expert ``heavy`` alternate with the replica slot E (odd ranks)."""
    idx = np.ascontiguousarray(idx, np.int32)
    T, k = idx.shape
    out = np.empty_like(idx)
    _check(lib().orc_replica_split(_ptr(idx), T, E, k, int(heavy), _ptr(out)), "replica_split")
    return out


def heavy_hitter(counts):
    """The most-loaded expert (lowest id among equal counts)."""
    counts = np.asarray(counts)
    return int(np.flatnonzero(counts == counts.max())[0])


def expert_rows(x, w_gate, w_up, w_down, act, h_round, tok, exp_id):
    """fp64 expert outputs for (token, expert) pairs.  Weights [E,F,d] / [E,d,F]."""
    x = np.ascontiguousarray(x)
    w_up = np.ascontiguousarray(w_up)
    w_down = np.ascontiguousarray(w_down)
    w_gate = None if w_gate is None else np.ascontiguousarray(w_gate)
    T, d = x.shape
    F = w_up.shape[-2]
    assert w_up.shape[-1] == d and w_down.shape[-2:] == (d, F)
    tok = np.ascontiguousarray(tok, np.int32)
    exp_id = np.ascontiguousarray(exp_id, np.int32)
    n = tok.shape[0]
    Y = np.empty((n, d), np.float64)
    a = SWIGLU if act == "swiglu" else RELU
    _check(lib().orc_expert_rows(_ptr(x), _dt(x), d, F, a, _ptr(w_gate), _ptr(w_up),
                                 _ptr(w_down), _dt(w_up), h_round, _ptr(tok), _ptr(exp_id), n,
                                 _ptr(Y)), "expert_rows")
    return Y


def combine(Y, assign_row, gate, Ys=None):
    gate = np.ascontiguousarray(gate, np.float32)
    T, k = gate.shape
    Y = np.ascontiguousarray(Y, np.float64)
    d = Y.shape[1]
    ar = None if assign_row is None else np.ascontiguousarray(assign_row, np.int32)
    Ys = None if Ys is None else np.ascontiguousarray(Ys, np.float64)
    y = np.empty((T, d), np.float32)
    _check(lib().orc_combine(_ptr(Y), _ptr(ar), _ptr(gate), _ptr(Ys), T, k, d, _ptr(y)),
           "combine")
    return y


def dequant_int4(q, scale, zero, group=INT4_GROUP):
    """INT4 words [.., N, K/8] + fp16 scale/zero [.., N, K/group] -> bf16 bits [.., N, K]."""
    q = np.ascontiguousarray(q, np.int32)
    scale = np.ascontiguousarray(scale, np.uint16)
    zero = np.ascontiguousarray(zero, np.uint16)
    K = q.shape[-1] * 8
    rows = int(np.prod(q.shape[:-1]))
    out = np.empty(q.shape[:-1] + (K,), np.uint16)
    _check(lib().orc_dequant_int4(_ptr(q), _ptr(scale), _ptr(zero), rows, K, group, _ptr(out)),
           "dequant_int4")
    return out


def dequant_mwq(m, bits, group=INT4_GROUP):
    """Nested INT2 + residual planes (one projection, leading dims kept) decoded at
    width ``bits`` (2, 3 or 4) -> bf16 bits [.., N, K]."""
    q2 = np.ascontiguousarray(m.q2, np.int32)
    K = q2.shape[-1] * 16
    rows = int(np.prod(q2.shape[:-1]))
    out = np.empty(q2.shape[:-1] + (K,), np.uint16)
    arrs = [np.ascontiguousarray(a, dt) for a, dt in ((m.s2, np.uint16), (m.z2, np.uint16),
                                                       (m.p3, np.int32), (m.a3, np.uint16),
                                                       (m.p4, np.int32), (m.a4, np.uint16))]
    _check(lib().orc_dequant_mwq(_ptr(q2), *[_ptr(a) for a in arrs], rows, K, group, int(bits),
                                 _ptr(out)), "dequant_mwq")
    return out


def mwq_groups(idx, bits, E):
    """Rows grouped by (expert, bit width): group v = 3*e + (b - 2) for the width b
    of each assignment (a width outside 2..4 is read as the nearest of them), then
    the stable group-major permutation over 3E groups.  Returns (group ids [T][k],
    counts [3E], offsets [3E+1], row_assign, assign_row)."""
    b = np.clip(np.asarray(bits, np.int64), 2, 4)
    vidx = (np.asarray(idx, np.int64) * 3 + (b - 2)).astype(np.int32)
    counts, offsets, row_assign, assign_row, _ = permute(vidx, 3 * E)
    return vidx, counts, offsets, row_assign, assign_row


def dequant_int2(q2, s2, z2, group=INT4_GROUP):
    """INT2 weights (the base of the nested format) -> bf16 bits [.., N, K]:
    bf16_RNE(fp32(fp32(q) - z) * s), the nested decode at width 2."""
    q2 = np.ascontiguousarray(q2, np.int32)
    K = q2.shape[-1] * 16
    rows = int(np.prod(q2.shape[:-1]))
    out = np.empty(q2.shape[:-1] + (K,), np.uint16)
    s2 = np.ascontiguousarray(s2, np.uint16)
    z2 = np.ascontiguousarray(z2, np.uint16)
    _check(lib().orc_dequant_mwq(_ptr(q2), _ptr(s2), _ptr(z2), None, None, None, None, rows, K,
                                 group, 2, _ptr(out)), "dequant_int2")
    return out


def floe_threshold(samples, sparsity):
    """Threshold for a target sparsity from the empirical CDF of |activations|
    ("FloE" -- Assumptions & free parameters: per-expert thresholds from the
    empirical CDF; reading: its inverse at the target level), i.e. the smallest
    sample value t with F_hat(t) >= sparsity, the ceil(sparsity * n)-th smallest
    |sample|.  Channels with |u| <= t are then pruned."""
    a = np.sort(np.abs(np.asarray(samples, np.float64)).ravel())
    if a.size == 0:
        raise OracleError("floe_threshold: no samples")
    r = max(1, int(np.ceil(sparsity * a.size)))
    return float(a[r - 1])


def floe_rows(x, w_gate, w_up_dec, w_down, thr, tok, exp_id, u_given=None):
    """Sparse-down expert rows (see orc_floe_rows).  Returns (Y [n][d] fp64,
    u [n][F] fp64, keep [n][F] uint8)."""
    x = np.ascontiguousarray(x, np.uint16)
    tok = np.ascontiguousarray(tok, np.int32)
    exp_id = np.ascontiguousarray(exp_id, np.int32)
    n, d, F = tok.size, x.shape[1], w_up_dec.shape[1]
    Y = np.empty((n, d), np.float64)
    u = np.empty((n, F), np.float64)
    keep = np.empty((n, F), np.uint8)
    ug = None if u_given is None else np.ascontiguousarray(u_given, np.float32)
    arrs = [np.ascontiguousarray(a, np.uint16) for a in (w_gate, w_up_dec, w_down)]
    thr = np.ascontiguousarray(thr, np.float32)
    _check(lib().orc_floe_rows(_ptr(x), d, F, _ptr(arrs[0]), _ptr(arrs[1]), _ptr(arrs[2]),
                               _ptr(thr), _ptr(tok), _ptr(exp_id), n, _ptr(ug), _ptr(u),
                               _ptr(keep), _ptr(Y)), "floe_rows")
    return Y, u, keep


def log_softmax_rows(l):
    l = np.ascontiguousarray(l, np.float32)
    T, n = l.shape
    out = np.empty_like(l)
    _check(lib().orc_log_softmax_rows(_ptr(l), T, n, _ptr(out)), "log_softmax_rows")
    return out


def grid_topk(pr, pc, K):
    """Exact top-K of S_ij = fp32(pr[i] + pc[j]) per token (ties to the lower id
    i*Nc + j), ids in ascending order, gates = softmax over the chosen S."""
    pr = np.ascontiguousarray(pr, np.float32)
    pc = np.ascontiguousarray(pc, np.float32)
    T, Nr = pr.shape
    Nc = pc.shape[1]
    idx = np.empty((T, K), np.int32)
    gate = np.empty((T, K), np.float32)
    _check(lib().orc_grid_topk(_ptr(pr), _ptr(pc), T, Nr, Nc, K, _ptr(idx), _ptr(gate)),
           "grid_topk")
    return idx, gate


def atomic_rows(x, w_in, w_out_t, idx, gate, act, tok):
    """fp64 outputs of the atomic experts of tokens ``tok`` (see orc_atomic_rows)."""
    x = np.ascontiguousarray(x, np.uint16)
    w_in = np.ascontiguousarray(w_in, np.uint16)
    w_out_t = np.ascontiguousarray(w_out_t, np.uint16)
    idx = np.ascontiguousarray(idx, np.int32)
    gate = np.ascontiguousarray(gate, np.float32)
    tok = np.ascontiguousarray(tok, np.int32)
    d, N = w_out_t.shape
    Y = np.empty((tok.size, d), np.float64)
    _check(lib().orc_atomic_rows(_ptr(x), d, _ptr(w_in), _ptr(w_out_t), N, _ptr(idx), _ptr(gate),
                                 idx.shape[1], 0 if act == "silu" else 1, _ptr(tok), tok.size,
                                 _ptr(Y)), "atomic_rows")
    return Y


def atomic_layer_forward(wl, pr=None, pc=None, tokens=None):
    """The atomic-expert layer on the CPU: router logits of the grid's rows and
    columns, their log-softmax, exact top-K over the grid with gates, the
    expert-major permutation over N = nr*nc experts with LIS, the atomic expert
    outputs and the shared MLP.  ``pr``/``pc``: given row / column
    log-probabilities (e.g. the GPU's), on which the selection is taken."""
    cfg = wl.cfg
    T, K, N = cfg.T, cfg.k, cfg.nr * cfg.nc
    lr = router_logits(wl.x, wl.w_router, None)
    lc = router_logits(wl.x, wl.w_col, None)
    own_pr, own_pc = log_softmax_rows(lr), log_softmax_rows(lc)
    PR = own_pr if pr is None else np.ascontiguousarray(pr, np.float32)
    PC = own_pc if pc is None else np.ascontiguousarray(pc, np.float32)
    idx, gate = grid_topk(PR, PC, K)
    counts, offsets, row_assign, assign_row, lis = permute(idx, N)
    out = dict(logits_r=lr, logits_c=lc, pr=own_pr, pc=own_pc, idx=idx, gate=gate, counts=counts,
               offsets=offsets, row_assign=row_assign, assign_row=assign_row, lis=lis)
    toks = np.arange(T, dtype=np.int32) if tokens is None else np.asarray(tokens, np.int32)
    Y = atomic_rows(wl.x, wl.w_in, wl.w_out_t, idx, gate, cfg.act, toks)
    Ys = None
    if cfg.n_shared:
        Ys = expert_rows(wl.x, wl.ws_gate[None], wl.ws_up[None], wl.ws_down[None], "swiglu",
                         ROUND_BF16, toks, np.zeros_like(toks))
    out["tokens"] = toks
    out["y"] = combine(Y, None, np.ones((toks.size, 1), np.float32), Ys)
    return out


# --- the layer -----------------------------------------------------------

def _h_round(wl):
    return ROUND_BF16 if wl.cfg.dtype == "bf16" else ROUND_F32


def dense_expert_weights(wl, experts=None):
    """Routed expert weights as dense arrays (INT4 decoded with the oracle's rule).

    Nested-quantised layers have 3E virtual experts v = e*3 + (bits - 2): expert e
    decoded at 2, 3 and 4 bits."""
    if wl.cfg.mwq:
        E = wl.cfg.E
        sel = range(3 * E) if experts is None else experts
        out = []
        for m, shape_src in ((wl.m_gate, wl.w_gate), (wl.m_up, wl.w_up), (wl.m_down, wl.w_down)):
            if m is None:
                out.append(None)
                continue
            full = np.zeros((3 * E,) + shape_src.shape[1:], np.uint16)
            for v in sel:
                e, b = v // 3, v % 3 + 2
                one = type(m)(*[a[e] for a in (m.q2, m.s2, m.z2, m.p3, m.a3, m.p4, m.a4)])
                full[v] = dequant_mwq(one, b)
            out.append(full)
        return tuple(out)
    if not wl.cfg.int4:
        return wl.w_gate, wl.w_up, wl.w_down
    E = wl.cfg.E
    sel = range(E) if experts is None else experts
    out = []
    for qw, shape_src in ((wl.q_gate, wl.w_gate), (wl.q_up, wl.w_up), (wl.q_down, wl.w_down)):
        if qw is None:          # ReLU experts have no gate projection
            out.append(None)
            continue
        full = np.zeros(shape_src.shape, np.uint16)
        for e in sel:
            full[e] = dequant_int4(qw.q[e], qw.scale[e], qw.zero[e])
        out.append(full)
    return tuple(out)


def replica_dense_weights(rep):
    """The replica's INT4 projections ([1, N, K]) decoded with the oracle's rule."""
    out = []
    for qw in (rep.q_gate, rep.q_up, rep.q_down):
        out.append(None if qw is None else dequant_int4(qw.q, qw.scale, qw.zero))
    return tuple(out)


def layer_forward(wl, logits=None, tokens=None, routing_only=False, replica=None, floe_u=None):
    """Run the whole layer on the CPU.

    ``logits``: if given (e.g. the GPU's fp32 logits), routing uses them instead
    of the oracle's own; that pins every integer output to one fp32 input.
    ``tokens``: optional subset of token ids whose y is computed (routing,
    counts, permutation and LIS always cover all T tokens).
    ``floe_u``: sparse-down layers only -- up-projection outputs [T*k][F] fp32 in
    expert-major row order (e.g. the GPU's) on which the keep/prune decisions
    are taken, as ``logits`` is for routing.
    Returns a dict of every intermediate and output.
    """
    cfg = wl.cfg
    T, d, E, k = cfg.T, cfg.d, cfg.E, cfg.k
    own_logits = router_logits(wl.x, wl.w_router, wl.b_router)
    lg = own_logits if logits is None else np.ascontiguousarray(logits, np.float32)
    idx, gate = topk_gates(lg, k)
    counts, offsets, row_assign, assign_row, lis = permute(idx, E)
    out = dict(logits=own_logits, idx=idx, gate=gate, counts=counts, offsets=offsets,
               row_assign=row_assign, assign_row=assign_row, lis=lis)
    if replica is not None:
        # the replica of expert `replica.heavy` is slot E; its share of that
        # expert's assignments and the recount over E+1 slots
        idx2 = replica_split(idx, E, replica.heavy)
        counts2, offsets2, row_assign2, assign_row2, lis2 = permute(idx2, E + 1)
        out.update(base_counts=counts, base_lis=lis, idx=idx2, counts=counts2,
                   offsets=offsets2, row_assign=row_assign2, assign_row=assign_row2, lis=lis2)
        idx, row_assign, assign_row = idx2, row_assign2, assign_row2
    if cfg.mwq:
        vidx, vcounts, voffsets, vra, var_ = mwq_groups(idx, wl.bits, E)
        out.update(mwq_idx=vidx, mwq_counts=vcounts, mwq_offsets=voffsets,
                   mwq_row_assign=vra, mwq_assign_row=var_)
        idx, row_assign, assign_row = vidx, vra, var_
    if routing_only:
        return out
    if tokens is None:
        # every row in expert-major order, recombined through assign_row
        toks = np.arange(T, dtype=np.int32)
        pt = (row_assign // k).astype(np.int32)
        pe = idx.reshape(-1)[row_assign]
        ar = assign_row
    else:
        # a token subset, in its own flat slot order
        toks = np.asarray(tokens, np.int32)
        pt = np.repeat(toks, k)
        pe = idx[toks].reshape(-1)
        ar = None
    if cfg.floe:
        ug = None
        if floe_u is not None:
            fu = np.asarray(floe_u, np.float32)
            ug = fu if tokens is None else fu[assign_row[(toks[:, None] * k + np.arange(k)).ravel()]]
        wu = dequant_int2(wl.u2_up.q2, wl.u2_up.s2, wl.u2_up.z2)
        Y, u, keep = floe_rows(wl.x, wl.w_gate, wu, wl.w_down, wl.floe_thr, pt, pe, ug)
        out.update(tokens=toks, Y=Y, Ys=None, floe_u=u, floe_keep=keep)
        if tokens is None:
            # channels a row of each expert keeps (rows are expert-major)
            nnz = np.zeros(E, np.int64)
            for e in range(E):
                sel = pe == e
                if sel.any():
                    nnz[e] = int(keep[sel].any(axis=0).sum())
            out["floe_nnz"] = nnz
        Ys = None
        if cfg.n_shared:
            Ys = expert_rows(wl.x, wl.ws_gate[None], wl.ws_up[None], wl.ws_down[None], "swiglu",
                             _h_round(wl), toks, np.zeros_like(toks))
            out["Ys"] = Ys
        out["y"] = combine(Y, ar, gate[toks], Ys)
        return out
    needed = sorted(set(int(e) for e in pe if e < (3 * E if cfg.mwq else E)))
    wg, wu, wd = dense_expert_weights(wl, needed)
    if replica is not None:
        rg, ru, rd = replica_dense_weights(replica)
        wg = None if wg is None else np.concatenate([wg, rg], axis=0)
        wu = np.concatenate([wu, ru], axis=0)
        wd = np.concatenate([wd, rd], axis=0)
    Y = expert_rows(wl.x, wg, wu, wd, cfg.act, _h_round(wl), pt, pe)
    Ys = None
    if cfg.n_shared:
        Ys = expert_rows(wl.x, wl.ws_gate[None], wl.ws_up[None], wl.ws_down[None], "swiglu",
                         _h_round(wl), toks, np.zeros_like(toks))
    out["tokens"] = toks
    out["Y"] = Y
    out["Ys"] = Ys
    out["y"] = combine(Y, ar, gate[toks], Ys)
    return out
