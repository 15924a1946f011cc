"""Seeded tensor generation for the MoE workloads.

Every tensor is drawn from its own ``numpy.random.Generator(PCG64(SeedSequence(
[cfg_id, tensor_id, expert])))`` so any tensor regenerates on its own, on any
machine, bit for bit.  Values are drawn in fp32 (x ~ N(0,1), every weight ~
N(0, 0.02^2)) and, for bf16 workloads, rounded to bf16 with round-to-nearest-
even.  bf16 arrays are returned as ``uint16`` bit patterns.

Nothing here computes any part of the layer: the INT4 *encoding* below is
input preparation (it turns bf16 weights into nibbles, scales and zero points);
the *decoding* that the layer performs lives separately in the oracle and in
the HIP kernels.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Optional

import numpy as np

from .configs import CONFIGS, WorkloadConfig

# tensor ids inside a workload's seed space
TID_X, TID_WR, TID_WGATE, TID_WUP, TID_WDOWN = 0, 1, 2, 3, 4
TID_SGATE, TID_SUP, TID_SDOWN, TID_ZIPF = 5, 6, 7, 8
TID_BITS = 9   # per-assignment bit widths of the nested-quantisation workload
TID_XCAL = 10  # calibration activations (sparsity thresholds)
TID_WRCOL = 11 # column router of the atomic-expert grid (the row router uses TID_WR)
ATOMIC_CHUNK = 1024  # atomic experts per seeded chunk
FLOE_CAL_TOKENS = 64

W_STD = 0.02
INT4_GROUP = 128


def _rng(cfg_id: int, tid: int, expert: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg_id, tid, expert])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round-to-nearest-even (finite inputs)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).copy()
    u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (u >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(cfg_id, tid, expert, shape, scale, bf16):
    a = _rng(cfg_id, tid, expert).standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        a *= np.float32(scale)
    return f32_to_bf16_bits(a) if bf16 else a


def _per_expert(fn, n, threads=8):
    with ThreadPoolExecutor(max(1, min(threads, n))) as ex:
        return np.stack(list(ex.map(fn, range(n))))


def quantize_int4_rows(w_bits: np.ndarray, fractional_zero: bool = False):
    """Asymmetric group-wise INT4 encoding of bf16 weight rows.

    ``w_bits``: [N, K] bf16 bits, K a multiple of 128.  Returns (q [N, K/8] int32
    with nibble i of word j holding K-index 8j+i, low nibble first; scale and
    zero as fp16 bits [N, K/128]).  Per group of 128 along K: s = fp16((hi-lo)/15),
    z = fp16(clamp(rint(-lo/s), 0, 15)) and q = clamp(rint(w/s) + z, 0, 15);
    a constant group gets s = 1, z = 0.  With ``fractional_zero`` the zero
    point keeps its fraction (z = fp16(clamp(-lo/s, 0, 15)), q = clamp(rint(w/s + z),
    0, 15)), which exercises the decode rule with non-integer z.
    """
    N, K = w_bits.shape
    assert K % INT4_GROUP == 0
    w = bf16_bits_to_f32(w_bits).reshape(N, K // INT4_GROUP, INT4_GROUP)
    lo = w.min(axis=2)
    hi = w.max(axis=2)
    const = hi == lo
    s16 = ((hi - lo) / np.float32(15.0)).astype(np.float16)
    s16[const] = np.float16(1.0)
    s = s16.astype(np.float32)
    if fractional_zero:
        z16 = np.clip(-lo / s, 0.0, 15.0).astype(np.float16)
    else:
        z16 = np.clip(np.rint(-lo / s), 0.0, 15.0).astype(np.float16)
    z16[const] = np.float16(0.0)
    z = z16.astype(np.float32)
    if fractional_zero:
        q = np.clip(np.rint(w / s[..., None] + z[..., None]), 0, 15)
    else:
        q = np.clip(np.rint(w / s[..., None]) + z[..., None], 0, 15)
    q = q.astype(np.uint32).reshape(N, K // 8, 8)
    shifts = (np.arange(8, dtype=np.uint32) * np.uint32(4))[None, None, :]
    words = np.bitwise_or.reduce(q << shifts, axis=2).astype(np.uint32)
    return words.view(np.int32), s16.view(np.uint16), z16.view(np.uint16)


def _int2_base(w, N, K):
    """INT2 base of the nested format on float64 groups w [N, G, 128]."""
    lo = w.min(axis=2)
    hi = w.max(axis=2)
    const = hi == lo
    s16 = ((hi - lo) / 3.0).astype(np.float16)
    s16[const] = np.float16(1.0)
    s = s16.astype(np.float64)
    z16 = np.clip(np.rint(-lo / s), 0.0, 3.0).astype(np.float16)
    z16[const] = np.float16(0.0)
    z = z16.astype(np.float64)
    q = np.clip(np.rint(w / s[..., None]) + z[..., None], 0, 3)
    return q, s16, z16, s, z


def _pack_q2(q, N, K):
    qv = q.astype(np.uint32).reshape(N, K // 16, 16)
    i16 = np.arange(16, dtype=np.uint32)
    sh2 = (2 * (4 * (i16 % 4) + i16 // 4))[None, None, :]
    return np.bitwise_or.reduce(qv << sh2, axis=2).astype(np.uint32).view(np.int32)


def quantize_int2_rows(w_bits: np.ndarray):
    """Asymmetric INT2 (group 128 along K) of bf16 rows: the base of the nested
    format alone (see quantize_mwq_rows).  Returns q2 [N, K/16] int32 in the
    byte-transposed order, s2, z2 fp16 bits [N, K/128]."""
    N, K = w_bits.shape
    assert K % INT4_GROUP == 0
    w = bf16_bits_to_f32(w_bits).astype(np.float64).reshape(N, K // INT4_GROUP, INT4_GROUP)
    q, s16, z16, _, _ = _int2_base(w, N, K)
    return _pack_q2(q, N, K), s16.view(np.uint16), z16.view(np.uint16)


def quantize_mwq_rows(w_bits: np.ndarray):
    """Nested INT2 + two binary residual planes (group 128 along K) of bf16 rows.

    ``w_bits``: [N, K] bf16 bits, K a multiple of 128.  Per group: an asymmetric
    INT2 base (s2 = fp16((hi-lo)/3), z2 = fp16(clamp(rint(-lo/s2), 0, 3)),
    q2 = clamp(rint(w/s2) + z2, 0, 3); a constant group gets s2 = 1, z2 = 0), then
    for b = 3, 4 the sign bit r_b of the remaining error (1 where it is >= 0) and
    a_b = fp16(mean |error|) -- the closed-form binary fit of the residual.  The
    errors are taken in float64 (this is the input quantiser, not the decode).
    Returns q2 [N, K/16] int32, s2, z2, a3, a4 fp16 bits [N, K/128], p3, p4
    [N, K/32] int32, in the byte-transposed storage order of the nested format:
    K-index 16j + 4m + b in 2-bit field 4b + m of q2 word j, K-index 32j + 4i + b
    in bit 8b + i of plane word j."""
    N, K = w_bits.shape
    assert K % INT4_GROUP == 0
    G = K // INT4_GROUP
    w = bf16_bits_to_f32(w_bits).astype(np.float64).reshape(N, G, INT4_GROUP)
    q, s16, z16, s, z = _int2_base(w, N, K)
    approx = (q - z[..., None]) * s[..., None]
    planes, mags = [], []
    for _ in range(2):
        err = w - approx
        r = err >= 0
        a16 = np.abs(err).mean(axis=2).astype(np.float16)
        a = a16.astype(np.float64)[..., None]
        approx = approx + np.where(r, a, -a)
        planes.append(r.reshape(N, K))
        mags.append(a16)
    q2 = _pack_q2(q, N, K)
    i32 = np.arange(32, dtype=np.uint32)
    sh1 = (8 * (i32 % 4) + i32 // 4)[None, None, :]

    def pack_bits(r):
        return np.bitwise_or.reduce(r.reshape(N, K // 32, 32).astype(np.uint32) << sh1,
                                    axis=2).astype(np.uint32).view(np.int32)
    return (q2, s16.view(np.uint16), z16.view(np.uint16), pack_bits(planes[0]),
            mags[0].view(np.uint16), pack_bits(planes[1]), mags[1].view(np.uint16))


@dataclass
class MwqWeights:
    """Nested-quantised weights of one projection, all experts (see quantize_mwq_rows)."""
    q2: np.ndarray      # [E, N, K/16] int32
    s2: np.ndarray      # [E, N, K/128] fp16 bits
    z2: np.ndarray
    p3: np.ndarray      # [E, N, K/32] int32
    a3: np.ndarray      # [E, N, K/128] fp16 bits
    p4: np.ndarray
    a4: np.ndarray


@dataclass
class Int2Weights:
    """INT2 weights of one projection, all experts (see quantize_int2_rows)."""
    q2: np.ndarray      # [E, N, K/16] int32
    s2: np.ndarray      # [E, N, K/128] fp16 bits
    z2: np.ndarray


def sparsity_thresholds(x_cal_bits: np.ndarray, w_up_bits: np.ndarray, sparsity: float):
    """Per-expert magnitude thresholds of the up-projection output for a target
    sparsity: for expert e, the ceil(sparsity * n)-th smallest of the n values
    |x_cal . W_up[e]^T| over a calibration batch (float64, unquantised weights).
    These are layer parameters produced offline; the layer only compares against
    them."""
    xc = bf16_bits_to_f32(x_cal_bits).astype(np.float64)
    out = np.empty(w_up_bits.shape[0], np.float32)
    for e in range(w_up_bits.shape[0]):
        a = np.abs(xc @ bf16_bits_to_f32(w_up_bits[e]).astype(np.float64).T).ravel()
        r = max(1, int(math.ceil(sparsity * a.size)))
        out[e] = np.float32(np.partition(a, r - 1)[r - 1])
    return out


@dataclass
class Int4Weights:
    q: np.ndarray       # [E, N, K/8] int32
    scale: np.ndarray   # [E, N, K/128] fp16 bits (uint16)
    zero: np.ndarray    # [E, N, K/128] fp16 bits (uint16)


@dataclass
class Workload:
    cfg: WorkloadConfig
    x: np.ndarray                    # [T, d]   bf16 bits (uint16) or fp32
    w_router: np.ndarray             # [E, d]   activation dtype
    b_router: np.ndarray             # [E]      fp32
    w_gate: Optional[np.ndarray]     # [E, F, d] (None for ReLU)
    w_up: np.ndarray                 # [E, F, d] (W_in for ReLU)
    w_down: np.ndarray               # [E, d, F]
    ws_gate: Optional[np.ndarray] = None   # [S*F_s, d] shared experts, concatenated along F
    ws_up: Optional[np.ndarray] = None
    ws_down: Optional[np.ndarray] = None   # [d, S*F_s]
    q_gate: Optional[Int4Weights] = None
    q_up: Optional[Int4Weights] = None
    q_down: Optional[Int4Weights] = None
    m_gate: Optional[MwqWeights] = None    # nested INT2+residual weights (mwq configs)
    m_up: Optional[MwqWeights] = None
    m_down: Optional[MwqWeights] = None
    bits: Optional[np.ndarray] = None      # [T, k] int32 bit width of each assignment
    w_col: Optional[np.ndarray] = None     # [nc, d] column router (atomic configs; w_router = rows)
    w_in: Optional[np.ndarray] = None      # [N, d] atomic input vectors
    w_out_t: Optional[np.ndarray] = None   # [d, N] atomic output vectors as columns
    w_out_rows: Optional[np.ndarray] = None  # [N, d] the same output vectors as rows
    u2_up: Optional[Int2Weights] = None    # INT2 up projection (floe configs)
    floe_thr: Optional[np.ndarray] = None  # [E] fp32 |up output| threshold per expert

    @property
    def bf16(self) -> bool:
        return self.cfg.dtype == "bf16"


def router_bias(cfg: WorkloadConfig, beta: Optional[float] = None) -> np.ndarray:
    """Router bias per the config's recipe (fp32)."""
    E = cfg.E
    beta = cfg.beta if beta is None else beta
    e = np.arange(E, dtype=np.float64)
    if cfg.bias == "zero":
        b = np.zeros(E)
    elif cfg.bias == "log_inv":           # b_e = 0.5 ln(1/(e+1))
        b = 0.5 * np.log(1.0 / (e + 1.0))
    elif cfg.bias == "neg_log":           # b_e = -beta ln(e+1)
        b = -beta * np.log(e + 1.0)
    elif cfg.bias == "zipf":              # b_e = -1.1 beta ln(r_e), r_e a seeded rank in 1..E
        ranks = _rng(cfg.cfg_id, TID_ZIPF).permutation(E) + 1
        b = -1.1 * beta * np.log(ranks.astype(np.float64))
    else:
        raise ValueError(cfg.bias)
    return b.astype(np.float32)


def _make_atomic(cfg, threads):
    """Atomic-expert workload: row / column routers and the two atomic matrices,
    drawn in seeded chunks of ATOMIC_CHUNK experts."""
    T, d, N = cfg.T, cfg.d, cfg.nr * cfg.nc
    wid = CONFIGS[cfg.weights_of].cfg_id if cfg.weights_of else cfg.cfg_id
    x = _normal(cfg.cfg_id, TID_X, 0, (T, d), 1.0, True)
    w_row = _normal(wid, TID_WR, 0, (cfg.nr, d), W_STD, True)
    w_col = _normal(wid, TID_WRCOL, 0, (cfg.nc, d), W_STD, True)
    nch = (N + ATOMIC_CHUNK - 1) // ATOMIC_CHUNK

    def chunks(tid):
        def one(c):
            n = min(ATOMIC_CHUNK, N - c * ATOMIC_CHUNK)
            return _normal(wid, tid, c, (n, d), W_STD, True)
        with ThreadPoolExecutor(max(1, min(threads, nch))) as ex:
            return np.concatenate(list(ex.map(one, range(nch))), axis=0)
    w_in = chunks(TID_WUP)
    w_out_rows = chunks(TID_WDOWN)                      # [N][d]: expert n's output vector
    w_out_t = np.ascontiguousarray(w_out_rows.T)        # [d][N]: the same values transposed
    wl = Workload(cfg, x, w_row, np.zeros(cfg.nr, np.float32), None, w_in, w_out_t)
    wl.w_col, wl.w_in, wl.w_out_t, wl.w_out_rows = w_col, w_in, w_out_t, w_out_rows
    if cfg.n_shared:
        Fs = cfg.n_shared * cfg.F_shared
        wl.ws_gate = _normal(wid, TID_SGATE, 0, (Fs, d), W_STD, True)
        wl.ws_up = _normal(wid, TID_SUP, 0, (Fs, d), W_STD, True)
        wl.ws_down = _normal(wid, TID_SDOWN, 0, (d, Fs), W_STD, True)
    return wl


def make_workload(cfg, beta: Optional[float] = None, fractional_zero: bool = False,
                  threads: int = 8) -> Workload:
    """Draw every tensor of a workload.  ``cfg`` is a WorkloadConfig or a name."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    if cfg.atomic:
        assert cfg.dtype == "bf16" and cfg.E == cfg.nr * cfg.nc
        return _make_atomic(cfg, threads)
    bf16 = cfg.dtype == "bf16"
    T, d, E, F = cfg.T, cfg.d, cfg.E, cfg.F
    wid = CONFIGS[cfg.weights_of].cfg_id if cfg.weights_of else cfg.cfg_id
    if cfg.x_rows_of:
        src = CONFIGS[cfg.x_rows_of]
        assert src.d == d and T <= src.T
        x = _normal(src.cfg_id, TID_X, 0, (src.T, d), 1.0, bf16)[:T].copy()
    else:
        x = _normal(cfg.cfg_id, TID_X, 0, (T, d), 1.0, bf16)
    w_router = _normal(wid, TID_WR, 0, (E, d), W_STD, bf16)
    b_router = router_bias(cfg, beta)

    def mk(tid, shape):
        return _per_expert(lambda e: _normal(wid, tid, e, shape, W_STD, bf16), E, threads)

    w_gate = mk(TID_WGATE, (F, d)) if cfg.act == "swiglu" else None
    w_up = mk(TID_WUP, (F, d))
    w_down = mk(TID_WDOWN, (d, F))
    wl = Workload(cfg, x, w_router, b_router, w_gate, w_up, w_down)
    if cfg.n_shared:
        Fs = cfg.n_shared * cfg.F_shared
        wl.ws_gate = _normal(wid, TID_SGATE, 0, (Fs, d), W_STD, bf16)
        wl.ws_up = _normal(wid, TID_SUP, 0, (Fs, d), W_STD, bf16)
        wl.ws_down = _normal(wid, TID_SDOWN, 0, (d, Fs), W_STD, bf16)
    if cfg.int4:
        assert bf16, "INT4 experts carry bf16 activations"

        def q4(w):
            parts = [None] * E

            def one(e):
                parts[e] = quantize_int4_rows(w[e], fractional_zero)
            with ThreadPoolExecutor(max(1, min(threads, E))) as ex:
                list(ex.map(one, range(E)))
            return Int4Weights(np.stack([p[0] for p in parts]),
                               np.stack([p[1] for p in parts]),
                               np.stack([p[2] for p in parts]))
        wl.q_gate = q4(w_gate) if w_gate is not None else None
        wl.q_up = q4(w_up)
        wl.q_down = q4(w_down)
    if cfg.mwq:
        assert bf16, "nested-quantised experts carry bf16 activations"

        def qm(w):
            parts = [None] * E

            def one(e):
                parts[e] = quantize_mwq_rows(w[e])
            with ThreadPoolExecutor(max(1, min(threads, E))) as ex:
                list(ex.map(one, range(E)))
            return MwqWeights(*[np.stack([p[i] for p in parts]) for i in range(7)])
        wl.m_gate = qm(w_gate) if w_gate is not None else None
        wl.m_up = qm(w_up)
        wl.m_down = qm(w_down)
        # per-assignment bit widths, uniform over {2, 3, 4} (the pages' learned
        # bit-width router is not part of this workload)
        wl.bits = (_rng(cfg.cfg_id, TID_BITS).integers(0, 3, size=(T, cfg.k)) + 2).astype(np.int32)
    if cfg.floe:
        assert bf16 and cfg.act == "swiglu", "the sparse-down layer is a bf16 SwiGLU layer"
        parts = [None] * E

        def one(e):
            parts[e] = quantize_int2_rows(w_up[e])
        with ThreadPoolExecutor(max(1, min(threads, E))) as ex:
            list(ex.map(one, range(E)))
        wl.u2_up = Int2Weights(*[np.stack([p[i] for p in parts]) for i in range(3)])
        x_cal = _normal(cfg.cfg_id, TID_XCAL, 0, (FLOE_CAL_TOKENS, d), 1.0, True)
        wl.floe_thr = sparsity_thresholds(x_cal, w_up, cfg.sparsity)
    return wl



@dataclass
class Replica:
    """An INT4 copy of one routed expert, appended to the layer as slot E.

    ``heavy`` is the expert it copies; the projections hold one expert each
    ([1, F, d] / [1, d, F] logical shapes, same packing as Int4Weights)."""
    heavy: int
    q_gate: Optional[Int4Weights]
    q_up: Int4Weights
    q_down: Int4Weights


def make_replica(wl: Workload, heavy: int, fractional_zero: bool = False) -> Replica:
    """Quantise expert ``heavy`` of ``wl`` with the input quantiser (INT4 layers:
    copy its existing INT4 weights)."""
    def one(qw, w):
        if qw is not None:
            return Int4Weights(qw.q[heavy:heavy + 1].copy(), qw.scale[heavy:heavy + 1].copy(),
                               qw.zero[heavy:heavy + 1].copy())
        if w is None:
            return None
        q, s, z = quantize_int4_rows(w[heavy], fractional_zero)
        return Int4Weights(q[None], s[None], z[None])
    if wl.cfg.dtype != "bf16":
        raise ValueError("the INT4 replica needs bf16 activations")
    return Replica(int(heavy), one(wl.q_gate, wl.w_gate), one(wl.q_up, wl.w_up),
                   one(wl.q_down, wl.w_down))
