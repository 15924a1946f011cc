"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each test ties one oracle step to a closed form, an invariant, brute force on
tiny inputs, a hand-worked fixture under tests/golden/, or an independent
library routine (numpy fp64 matmul / argsort / bincount, torch's bf16 cast).
The mutation test at the end plants plausible mistakes in a copy of the oracle
and checks that this file catches each of them.
"""
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from workloads import get_config, make_workload
from workloads.gen import bf16_bits_to_f32, f32_to_bf16_bits, quantize_int4_rows

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _topk_brute(l, k):
    """Full sort by (value descending, id ascending); -0.0 == +0.0 under IEEE."""
    order = sorted(range(len(l)), key=lambda e: (-float(l[e]) + 0.0, e))
    return order[:k]


# ---------------------------------------------------------------- bf16 rounding

def test_round_bf16_table_matches_torch_cast():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    vals = np.concatenate([
        rng.standard_normal(4000).astype(np.float32),
        (rng.standard_normal(4000) * 1e-30).astype(np.float32),
        (rng.standard_normal(4000) * 1e30).astype(np.float32),
        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 257.0, 259.0, 2 ** -130,
                  0.0, -0.0], np.float32),
    ])
    ref = torch.from_numpy(vals).to(torch.bfloat16).to(torch.float32).numpy()
    got = np.array([oracle.round_bf16(float(v)) for v in vals], np.float64).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    # the generator's fp32 -> bf16 conversion follows the same rule
    assert np.array_equal(bf16_bits_to_f32(f32_to_bf16_bits(vals)).view(np.uint32),
                          ref.view(np.uint32))


def test_round_bf16_is_a_single_rounding_from_fp64():
    # 1 + 2^-8 + 2^-40 lies above the bf16 midpoint 1 + 2^-8: one rounding gives
    # 1 + 2^-7; rounding through fp32 first would land on the midpoint and tie to 1.
    assert oracle.round_bf16(1 + 2 ** -8 + 2 ** -40) == 1 + 2 ** -7
    assert oracle.round_bf16(1 + 2 ** -8) == 1.0          # tie -> even
    assert oracle.round_bf16(1 + 3 * 2 ** -8) == 1 + 2 ** -6  # tie -> even


# ---------------------------------------------------------------- logits

def test_router_logits_match_numpy_fp64():
    rng = np.random.default_rng(1)
    T, d, E = 37, 24, 5
    x = rng.standard_normal((T, d)).astype(np.float32)
    w = (rng.standard_normal((E, d)) * 0.3).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32)
    got = oracle.router_logits(x, w, b)
    ref = (x.astype(np.float64) @ w.astype(np.float64).T + b.astype(np.float64)).astype(np.float32)
    np.testing.assert_allclose(got, ref, rtol=2e-7, atol=1e-7)
    # bf16 inputs are widened exactly
    xb, wb = f32_to_bf16_bits(x), f32_to_bf16_bits(w)
    got = oracle.router_logits(xb, wb, None)
    ref = (bf16_bits_to_f32(xb).astype(np.float64) @ bf16_bits_to_f32(wb).astype(np.float64).T)
    np.testing.assert_allclose(got, ref.astype(np.float32), rtol=2e-7, atol=1e-7)


# ---------------------------------------------------------------- top-k

@pytest.mark.parametrize("E,k", [(1, 1), (2, 1), (5, 2), (8, 2), (16, 5), (64, 6), (64, 64)])
def test_topk_matches_full_sort(E, k):
    rng = np.random.default_rng(E * 100 + k)
    T = 60
    l = rng.standard_normal((T, E)).astype(np.float32)
    # exact ties and signed zeros in half the rows
    alphabet = np.array([-1.0, -0.0, 0.0, 0.5, 1.0], np.float32)
    l[::2] = alphabet[rng.integers(0, 5, size=(T // 2, E))]
    idx, _ = oracle.topk_gates(l, k)
    for t in range(T):
        assert list(idx[t]) == _topk_brute(l[t], k), (t, l[t])


@pytest.mark.parametrize("E", [1, 2, 3, 4])
def test_topk_exhaustive_small_alphabet(E):
    alphabet = [-1.0, -0.0, 0.0, 1.0]
    rows = np.array(list(itertools.product(alphabet, repeat=E)), np.float32)
    for k in range(1, E + 1):
        idx, gate = oracle.topk_gates(rows, k)
        for t in range(rows.shape[0]):
            assert list(idx[t]) == _topk_brute(rows[t], k)
        assert np.all(np.abs(gate.astype(np.float64).sum(1) - 1.0) <= 1e-6)


def test_topk_shift_invariance():
    rng = np.random.default_rng(3)
    l = (rng.integers(-64, 64, size=(200, 16)) / 8.0).astype(np.float32)  # exact grid
    i1, g1 = oracle.topk_gates(l, 4)
    i2, g2 = oracle.topk_gates(l + np.float32(2.5), 4)
    assert np.array_equal(i1, i2)
    assert np.array_equal(g1, g2)


def test_topk_rejects_nonfinite():
    l = np.zeros((2, 4), np.float32)
    l[1, 2] = np.nan
    with pytest.raises(oracle.OracleError):
        oracle.topk_gates(l, 2)
    l[1, 2] = np.inf
    with pytest.raises(oracle.OracleError):
        oracle.topk_gates(l, 2)


# ---------------------------------------------------------------- gates

def test_gates_closed_forms():
    rng = np.random.default_rng(4)
    l = rng.standard_normal((500, 8)).astype(np.float32) * 3
    i1, g1 = oracle.topk_gates(l, 1)
    assert np.all(g1 == 1.0)                      # k = 1: exactly one
    i2, g2 = oracle.topk_gates(l, 2)
    l0 = np.take_along_axis(l, i2[:, :1], 1)[:, 0].astype(np.float64)
    l1 = np.take_along_axis(l, i2[:, 1:2], 1)[:, 0].astype(np.float64)
    sig = 1.0 / (1.0 + np.exp(l1 - l0))           # k = 2: g0 = sigmoid(l0 - l1)
    np.testing.assert_allclose(g2[:, 0], sig, rtol=0, atol=1e-7)
    np.testing.assert_allclose(g2[:, 1], 1 - sig, rtol=0, atol=1e-7)
    assert np.all(g2[:, 0] >= g2[:, 1])
    eq = np.zeros((3, 6), np.float32)            # equal logits: 1/k each
    for k in (1, 2, 3, 6):
        _, g = oracle.topk_gates(eq, k)
        assert np.all(g == np.float32(1.0 / k))
    # k = E: the full softmax, in sorted order
    i8, g8 = oracle.topk_gates(l, 8)
    lf = l.astype(np.float64)
    sm = np.exp(lf - lf.max(1, keepdims=True))
    sm /= sm.sum(1, keepdims=True)
    np.testing.assert_allclose(g8, np.take_along_axis(sm, i8, 1), rtol=0, atol=1e-7)
    assert np.all(np.abs(g8.astype(np.float64).sum(1) - 1) <= 1e-6)


# ---------------------------------------------------------------- counts / permutation / LIS

def _check_permutation(idx, E):
    T, k = idx.shape
    counts, offsets, row_assign, assign_row, lis = oracle.permute(idx, E)
    flat = idx.reshape(-1)
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert counts.sum() == T * k
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts)
    assert np.array_equal(row_assign, np.argsort(flat, kind="stable"))
    assert np.array_equal(assign_row[row_assign], np.arange(T * k))
    assert np.array_equal(np.sort(row_assign), np.arange(T * k))
    for e in range(E):
        seg = row_assign[offsets[e]:offsets[e + 1]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg // k) > 0)      # token order inside an expert
    if T:
        exact = Fraction(E * int(counts.max()), T * k)
        assert lis == float(exact)                 # one correctly rounded division
        assert 1.0 <= lis <= E / k
    else:
        assert math.isnan(lis)
    return counts, offsets, row_assign, assign_row, lis


def test_permutation_golden_worked_example():
    fields = {}
    with open(os.path.join(GOLDEN, "lis_worked_example.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                key, *vals = line.split()
                fields[key] = vals
    E, k = int(fields["E"][0]), int(fields["K"][0])
    idx = np.array(fields["IDX"], np.int32).reshape(-1, k)
    counts, offsets, row_assign, assign_row, lis = oracle.permute(idx, E)
    assert list(counts) == [int(v) for v in fields["COUNTS"]]
    assert list(offsets) == [int(v) for v in fields["OFFSETS"]]
    assert list(row_assign) == [int(v) for v in fields["ROW_ASSIGN"]]
    assert list(assign_row) == [int(v) for v in fields["ASSIGN_ROW"]]
    assert lis == float(fields["LIS"][0])


@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (7, 8, 2), (100, 64, 6), (333, 8, 1), (50, 3, 3)])
def test_permutation_invariants_random(T, E, k):
    rng = np.random.default_rng(T * E + k)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    _check_permutation(idx, E)


def test_permutation_empty_and_degenerate():
    _check_permutation(np.zeros((0, 2), np.int32), 8)           # T = 0: LIS NaN
    E, k, T = 8, 2, 64
    rr = np.array([[(t * k + j) % E for j in range(k)] for t in range(T)], np.int32)
    assert _check_permutation(rr, E)[4] == 1.0                  # round-robin: balanced
    same = np.tile(np.array([[5, 2]], np.int32), (T, 1))
    c = _check_permutation(same, E)
    assert c[4] == E / k                                        # all on the same k
    assert list(np.nonzero(c[0])[0]) == [2, 5]                 # empty experts elsewhere


# ---------------------------------------------------------------- expert FFN and layer

def _silu(v):
    return v / (1.0 + np.exp(-v))


def _np_ffn(x, wg, wu, wd, act, h_round):
    """numpy fp64 matmul formulation of one expert on a block of tokens."""
    x = x.astype(np.float64)
    u = x @ wu.astype(np.float64).T
    h = _silu(x @ wg.astype(np.float64).T) * u if act == "swiglu" else np.maximum(u, 0.0)
    if h_round == oracle.ROUND_F32:
        h = h.astype(np.float32).astype(np.float64)
    return h @ wd.astype(np.float64).T


@pytest.mark.parametrize("act", ["swiglu", "relu"])
def test_expert_rows_dense_ffn(act):
    rng = np.random.default_rng(5)
    T, d, F, E = 9, 24, 40, 3                    # d != F catches a transposed operand
    x = rng.standard_normal((T, d)).astype(np.float32)
    wg = (rng.standard_normal((E, F, d)) * 0.2).astype(np.float32)
    wu = (rng.standard_normal((E, F, d)) * 0.2).astype(np.float32)
    wd = (rng.standard_normal((E, d, F)) * 0.2).astype(np.float32)
    tok = np.repeat(np.arange(T), E).astype(np.int32)
    ex = np.tile(np.arange(E), T).astype(np.int32)
    Y = oracle.expert_rows(x, wg if act == "swiglu" else None, wu, wd, act, oracle.ROUND_NONE,
                           tok, ex)
    for e in range(E):
        ref = _np_ffn(x, wg[e], wu[e], wd[e], act, oracle.ROUND_NONE)
        np.testing.assert_allclose(Y[ex == e], ref, rtol=1e-12, atol=1e-13)


def test_expert_rows_scalar_closed_form_and_silu_zero():
    x = np.array([[0.75], [0.0], [-1.5]], np.float32)
    wg = np.array([[[2.0]]], np.float32)
    wu = np.array([[[-0.5]]], np.float32)
    wd = np.array([[[3.0]]], np.float32)
    Y = oracle.expert_rows(x, wg, wu, wd, "swiglu", oracle.ROUND_NONE,
                           np.arange(3, dtype=np.int32), np.zeros(3, np.int32))
    for t in range(3):
        xv = float(x[t, 0])
        g = 2.0 * xv
        ref = (g / (1 + math.exp(-g))) * (-0.5 * xv) * 3.0
        assert abs(Y[t, 0] - ref) <= 1e-15
    assert Y[1, 0] == 0.0                                      # silu(0) = 0


def _tiny_f32(T=48, d=32, F=40, E=6, k=2, **kw):
    return make_workload(get_config("tiny_fp32", T=T, d=d, F=F, E=E, k=k, **kw))


def _dense_masked_y(wl, idx, gate):
    """Every expert on every token, times a one-hot gate matrix (no permutation)."""
    cfg = wl.cfg
    G = np.zeros((cfg.T, cfg.E))
    for t in range(cfg.T):
        for j in range(cfg.k):
            G[t, idx[t, j]] += float(gate[t, j])
    y = np.zeros((cfg.T, cfg.d))
    for e in range(cfg.E):
        Ye = _np_ffn(wl.x, wl.w_gate[e], wl.w_up[e], wl.w_down[e], cfg.act, oracle.ROUND_F32)
        y += G[:, e:e + 1] * Ye
    return y


def test_layer_matches_dense_masked_formulation():
    wl = _tiny_f32()
    out = oracle.layer_forward(wl)
    ref = _dense_masked_y(wl, out["idx"], out["gate"])
    np.testing.assert_allclose(out["y"], ref, rtol=1e-6, atol=1e-9)
    sub = oracle.layer_forward(wl, tokens=[5, 0, 47])          # token subset path agrees
    np.testing.assert_allclose(sub["y"], out["y"][[5, 0, 47]], rtol=1e-7, atol=1e-12)


def test_layer_single_expert_is_dense_ffn():
    wl = _tiny_f32(E=1, k=1)
    out = oracle.layer_forward(wl)
    assert np.all(out["gate"] == 1.0) and np.all(out["idx"] == 0)
    ref = _np_ffn(wl.x, wl.w_gate[0], wl.w_up[0], wl.w_down[0], "swiglu", oracle.ROUND_F32)
    np.testing.assert_allclose(out["y"], ref, rtol=1e-6, atol=1e-9)


def test_layer_all_experts_is_dense_softmax_mixture():
    wl = _tiny_f32(E=4, k=4)
    out = oracle.layer_forward(wl)
    lf = out["logits"].astype(np.float64)
    sm = np.exp(lf - lf.max(1, keepdims=True))
    sm /= sm.sum(1, keepdims=True)
    y = np.zeros((wl.cfg.T, wl.cfg.d))
    for e in range(4):
        y += sm[:, e:e + 1] * _np_ffn(wl.x, wl.w_gate[e], wl.w_up[e], wl.w_down[e], "swiglu",
                                     oracle.ROUND_F32)
    np.testing.assert_allclose(out["y"], y, rtol=1e-5, atol=1e-8)


def test_layer_token_permutation_equivariance():
    wl = _tiny_f32()
    out = oracle.layer_forward(wl)
    perm = np.random.default_rng(6).permutation(wl.cfg.T)
    wl.x = wl.x[perm].copy()
    out2 = oracle.layer_forward(wl)
    assert np.array_equal(out2["idx"], out["idx"][perm])
    assert np.array_equal(out2["counts"], out["counts"])
    assert out2["lis"] == out["lis"]
    np.testing.assert_array_equal(out2["y"], out["y"][perm])


def test_layer_shared_experts_add_dense_term():
    wl = _tiny_f32(n_shared=2, F_shared=16)
    assert wl.ws_gate.shape == (32, wl.cfg.d)
    out = oracle.layer_forward(wl)
    routed = _dense_masked_y(wl, out["idx"], out["gate"])
    shared = _np_ffn(wl.x, wl.ws_gate, wl.ws_up, wl.ws_down, "swiglu", oracle.ROUND_F32)
    np.testing.assert_allclose(out["y"], routed + shared, rtol=1e-6, atol=1e-9)
    assert out["counts"].sum() == wl.cfg.T * wl.cfg.k           # shared not counted


def test_tiny_workload_bias_skews_load():
    out = oracle.layer_forward(make_workload("tiny_fp32"), routing_only=True)
    # b_0 exceeds b_1 by 0.35 against logit noise of ~0.23 std: expert 0 nearly always wins
    assert out["counts"][0] >= 0.85 * 64 and out["lis"] > 3.0


# ---------------------------------------------------------------- INT4 decode

def _pack(nibbles):
    nib = np.asarray(nibbles, np.uint32).reshape(-1, 8)
    return np.bitwise_or.reduce(nib << (np.arange(8, dtype=np.uint32) * 4), axis=1) \
        .astype(np.uint32).view(np.int32)


def test_int4_golden_table():
    rows = []
    with open(os.path.join(GOLDEN, "int4_dequant_table.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                q, s, z, v = line.split()
                rows.append((int(q), int(s, 16), int(z, 16), float(v)))
    for q, s, z, v in rows:
        K = 128
        words = _pack([q] * K)[None]                       # one row, one group
        out = oracle.dequant_int4(words, np.array([[s]], np.uint16), np.array([[z]], np.uint16))
        vals = bf16_bits_to_f32(out)
        assert np.all(vals == np.float32(v)), (q, hex(s), hex(z), vals[0, 0], v)


def test_int4_nibble_order_and_groups():
    K, N = 256, 3
    rng = np.random.default_rng(7)
    q = rng.integers(0, 16, size=(N, K))
    words = _pack(q.reshape(-1)).reshape(N, K // 8)
    s = np.full((N, K // 128), 0x3C00, np.uint16)          # s = 1
    z = np.zeros((N, K // 128), np.uint16)
    z[:, 1] = 0x4000                                       # z = 2 on the second group only
    out = bf16_bits_to_f32(oracle.dequant_int4(words, s, z))
    exp = q.astype(np.float32)
    exp[:, 128:] -= 2
    assert np.array_equal(out, exp)


def test_int4_quantization_error_bound():
    rng = np.random.default_rng(8)
    w = f32_to_bf16_bits((rng.standard_normal((16, 512)) * 0.02).astype(np.float32))
    for frac in (False, True):
        q, s, z = quantize_int4_rows(w, fractional_zero=frac)
        wh = bf16_bits_to_f32(oracle.dequant_int4(q, s, z)).astype(np.float64)
        wf = bf16_bits_to_f32(w).astype(np.float64).reshape(16, 4, 128)
        s64 = np.frombuffer(s.tobytes(), np.float16).astype(np.float64).reshape(16, 4, 1)
        err = np.abs(wh.reshape(16, 4, 128) - wf)
        # half a quantisation step, plus half a bf16 ulp of the decoded value, plus
        # one step where the top of the group is clipped at 15
        bound = 0.5 * s64 + np.abs(wf) * 2.0 ** -8 + 1e-9
        inside = err <= bound
        assert inside.mean() > 0.97, inside.mean()
        assert np.all(err <= 1.0 * s64 + np.abs(wf) * 2.0 ** -8 + 1e-9)


# ---------------------------------------------------------------- replica dispatch

def _golden(name):
    fields = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                key, *vals = line.split()
                fields[key] = vals
    return fields


def test_replica_split_golden_worked_example():
    g = _golden("replica_split_example.txt")
    E, k, heavy = int(g["E"][0]), int(g["K"][0]), int(g["HEAVY"][0])
    idx = np.array(g["IDX"], np.int32).reshape(-1, k)
    counts0, _, _, _, lis0 = oracle.permute(idx, E)
    assert oracle.heavy_hitter(counts0) == heavy
    assert lis0 == float(g["LIS_BEFORE"][0])
    idx2 = oracle.replica_split(idx, E, heavy)
    assert list(idx2.reshape(-1)) == [int(v) for v in g["IDX_SPLIT"]]
    counts, offsets, row_assign, assign_row, lis = oracle.permute(idx2, E + 1)
    assert list(counts) == [int(v) for v in g["COUNTS"]]
    assert list(offsets) == [int(v) for v in g["OFFSETS"]]
    assert list(row_assign) == [int(v) for v in g["ROW_ASSIGN"]]
    assert list(assign_row) == [int(v) for v in g["ASSIGN_ROW"]]
    assert lis == float(g["LIS"][0])


@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (37, 8, 2), (200, 64, 6), (333, 8, 1), (9, 3, 3)])
def test_replica_split_closed_forms(T, E, k):
    rng = np.random.default_rng(1000 + T * E + k)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    counts0, _, _, _, _ = oracle.permute(idx, E)
    heavy = oracle.heavy_hitter(counts0)
    n = int(counts0[heavy])
    idx2 = oracle.replica_split(idx, E, heavy)
    counts, offsets, row_assign, assign_row, lis = oracle.permute(idx2, E + 1)
    # the heavy expert keeps ceil(n/2), the replica gets floor(n/2), the rest unchanged
    assert counts[heavy] == (n + 1) // 2 and counts[E] == n // 2
    others = [e for e in range(E) if e != heavy]
    assert list(counts[others]) == list(counts0[others])
    assert counts.sum() == T * k
    # only assignments of the heavy expert move, each to the replica slot
    moved = idx2 != idx
    assert np.all(idx[moved] == heavy) and np.all(idx2[moved] == E)
    # the moved ones are every second heavy assignment, counting from the second
    heavy_flat = np.flatnonzero(idx.reshape(-1) == heavy)
    assert list(np.flatnonzero(moved.reshape(-1))) == list(heavy_flat[1::2])
    assert lis == (E + 1) * counts.max() / (T * k)
    assert lis <= (E + 1) * max(counts0.max(), 1) / (T * k)


def test_replica_of_exact_weights_leaves_the_layer_unchanged():
    """A replica whose decoded weights equal the original expert's makes the
    split invisible: y is the same bits with and without it."""
    from workloads import make_replica
    wl = make_workload(get_config("mixtral_prefill_bf16", T=48, d=256, F=256))
    r0 = oracle.layer_forward(wl, routing_only=True)
    heavy = oracle.heavy_hitter(r0["counts"])
    rep = make_replica(wl, heavy)
    # make the original expert exactly the replica's decoded weights
    for name, qw in (("w_gate", rep.q_gate), ("w_up", rep.q_up), ("w_down", rep.q_down)):
        getattr(wl, name)[heavy] = oracle.dequant_int4(qw.q[0], qw.scale[0], qw.zero[0])
    base = oracle.layer_forward(wl)
    split = oracle.layer_forward(wl, replica=rep)
    assert split["counts"][-1] > 0
    assert np.array_equal(base["y"], split["y"])
    # and a lossy replica does change y (the split is really applied)
    wl2 = make_workload(get_config("mixtral_prefill_bf16", T=48, d=256, F=256))
    lossy = oracle.layer_forward(wl2, replica=make_replica(wl2, heavy))
    assert not np.array_equal(oracle.layer_forward(wl2)["y"], lossy["y"])


# ---------------------------------------------------------------- nested (MWQ) decode

def _mwq_one(q, r3, r4, s, z, a3, a4):
    """One 32-wide row (K = 128 so one group) whose first weight carries the given codes."""
    from workloads import MwqWeights
    q2 = np.zeros((1, 8), np.uint32)
    q2[0, 0] = q
    p3 = np.zeros((1, 4), np.uint32)
    p3[0, 0] = r3
    p4 = np.zeros((1, 4), np.uint32)
    p4[0, 0] = r4
    g = lambda v: np.array([[v]], np.uint16)
    return MwqWeights(q2.view(np.int32), g(s), g(z), p3.view(np.int32), g(a3), p4.view(np.int32),
                      g(a4))


def test_mwq_golden_table():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "mwq_dequant_table.txt"))
            if l.strip() and not l.startswith("#") and not l.startswith("q ")]
    assert len(rows) >= 9
    for q, r3, r4, s, z, a3, a4, b2, b3, b4 in rows:
        m = _mwq_one(int(q), int(r3), int(r4), int(s, 16), int(z, 16), int(a3, 16), int(a4, 16))
        for bits, want in ((2, b2), (3, b3), (4, b4)):
            got = oracle.dequant_mwq(m, bits)[0, 0]
            assert got == int(want, 16), (q, r3, r4, bits, hex(got), want)


def test_mwq_storage_positions():
    """One non-zero code at a time lands on the K-index the storage order names:
    q2 word j, field 4b+m -> K-index 16j+4m+b; plane word j, bit 8b+i -> 32j+4i+b."""
    from workloads import MwqWeights
    K = 128
    one = lambda v: np.full((1, 1), v, np.uint16)
    s, z, a = one(0x3C00), one(0x0000), one(0x3800)     # s = 1, z = 0, a = 0.5
    for word, field, want in ((0, 0, 0), (0, 1, 4), (0, 4, 1), (0, 5, 5), (0, 15, 15), (1, 6, 16 + 9),
                              (7, 11, 112 + 14)):
        q2 = np.zeros((1, K // 16), np.uint32)
        q2[0, word] = np.uint32(3) << np.uint32(2 * field)
        zero_p = np.zeros((1, K // 32), np.int32)
        m = MwqWeights(q2.view(np.int32), s, z, zero_p, a, zero_p, a)
        w2 = oracle.dequant_mwq(m, 2)[0]
        assert w2[want] == 0x4040 and np.count_nonzero(w2) == 1, (word, field)   # 3.0
    for word, bit, want in ((0, 0, 0), (0, 1, 4), (0, 8, 1), (0, 9, 5), (0, 31, 31), (3, 20, 96 + 18)):
        p = np.zeros((1, K // 32), np.uint32)
        p[0, word] = np.uint32(1) << np.uint32(bit)
        q2 = np.zeros((1, K // 16), np.int32)
        zero_p = np.zeros((1, K // 32), np.int32)
        w3 = oracle.dequant_mwq(MwqWeights(q2, s, z, p.view(np.int32), a, zero_p, a), 3)[0]
        assert w3[want] == 0x3F00 and np.count_nonzero(w3 == 0x3F00) == 1, (word, bit)  # +0.5
        assert np.all(np.delete(w3, want) == 0xBF00)                                   # -0.5


def test_mwq_nesting_and_reductions():
    from workloads import quantize_mwq_rows
    rng = np.random.default_rng(31)
    w = f32_to_bf16_bits((rng.standard_normal((24, 256)) * 0.02).astype(np.float32))
    m1 = quantize_mwq_rows(w)
    from workloads import MwqWeights
    m = MwqWeights(*m1)
    w2, w3, w4 = (oracle.dequant_mwq(m, b) for b in (2, 3, 4))
    # width 2 reads neither plane, width 3 not the second
    flip = MwqWeights(m.q2, m.s2, m.z2, ~m.p3, m.a3 ^ np.uint16(0x0155), ~m.p4,
                      m.a4 ^ np.uint16(0x0133))
    assert np.array_equal(oracle.dequant_mwq(flip, 2), w2)
    flip4 = MwqWeights(m.q2, m.s2, m.z2, m.p3, m.a3, ~m.p4, m.a4 ^ np.uint16(0x0133))
    assert np.array_equal(oracle.dequant_mwq(flip4, 3), w3)
    # zero residual magnitudes: each wider decode equals the narrower one
    zero = np.zeros_like(m.a3)
    assert np.array_equal(oracle.dequant_mwq(MwqWeights(m.q2, m.s2, m.z2, m.p3, zero, m.p4, zero), 4), w2)
    # the base is the INT4 rule on the same codes: spread each 2-bit field into a nibble
    N, K = w.shape
    fields = (m.q2.view(np.uint32)[:, :, None] >> (np.arange(16, dtype=np.uint32) * 2)) & 3
    i16 = np.arange(16)
    q = fields[:, :, 4 * (i16 % 4) + i16 // 4].reshape(N, K)   # K-index 4m+b in field 4b+m
    nib = np.bitwise_or.reduce(q.reshape(N, K // 8, 8) << (np.arange(8, dtype=np.uint32) * 4),
                               axis=2).astype(np.uint32).view(np.int32)
    assert np.array_equal(oracle.dequant_int4(nib, m.s2, m.z2), w2)
    # the residual planes shrink the error of the input quantiser on average
    wf = bf16_bits_to_f32(w).astype(np.float64)
    errs = [np.abs(bf16_bits_to_f32(x) - wf).mean() for x in (w2, w3, w4)]
    assert errs[0] > errs[1] > errs[2]


def test_mwq_groups_closed_forms():
    """Grouping by (expert, width): an expert's groups add up to its count, rows of
    one expert stay in flat order across its groups split by width, and widths
    outside 2..4 read as the nearest of them."""
    rng = np.random.default_rng(5)
    T, E, k = 300, 7, 3
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    bits = rng.integers(2, 5, size=(T, k)).astype(np.int32)
    vidx, c3, o3, ra3, ar3 = oracle.mwq_groups(idx, bits, E)
    counts, offsets, ra, ar, _ = oracle.permute(idx, E)
    assert np.array_equal(c3.reshape(E, 3).sum(axis=1), counts)
    assert np.array_equal(o3[::3], offsets)
    flat_idx, flat_b = idx.reshape(-1), bits.reshape(-1)
    for e in range(E):
        rows = ra3[o3[3 * e]:o3[3 * e + 3]]
        assert np.all(flat_idx[rows] == e)
        assert np.all(np.diff(flat_b[rows]) >= 0)              # widths ascending
        for j in range(3):
            grp = ra3[o3[3 * e + j]:o3[3 * e + j + 1]]
            assert np.all(np.diff(grp) > 0) and np.all(flat_b[grp] == j + 2)
    assert np.array_equal(ar3[ra3], np.arange(T * k))
    wild = bits.copy()
    wild[bits == 2] = rng.choice([-5, 0, 1, 2], size=int((bits == 2).sum()))
    wild[bits == 4] = rng.choice([4, 5, 100], size=int((bits == 4).sum()))
    for a, b in zip(oracle.mwq_groups(idx, wild, E), (vidx, c3, o3, ra3, ar3)):
        assert np.array_equal(a, b)


def test_mwq_layer_at_one_width_is_the_plain_layer():
    """All assignments at one width: rows group exactly as the plain routing and
    y equals the plain layer on the weights decoded at that width."""
    import dataclasses
    wl = make_workload(get_config("mixtral_mwq_decode", T=24, d=256, F=256, x_rows_of=None,
                                  weights_of=None))
    for b in (2, 4):
        wl.bits = np.full_like(wl.bits, b)
        mw = oracle.layer_forward(wl)
        plain = dataclasses.replace(wl, cfg=dataclasses.replace(wl.cfg, mwq=False))
        plain.w_gate = oracle.dequant_mwq(wl.m_gate, b)
        plain.w_up = oracle.dequant_mwq(wl.m_up, b)
        plain.w_down = oracle.dequant_mwq(wl.m_down, b)
        ref = oracle.layer_forward(plain)
        assert np.array_equal(mw["counts"], ref["counts"]) and mw["lis"] == ref["lis"]
        E = wl.cfg.E
        assert np.array_equal(mw["mwq_counts"].reshape(E, 3)[:, b - 2], ref["counts"])
        assert np.array_equal(mw["row_assign"], ref["row_assign"])
        assert np.array_equal(mw["y"], ref["y"])


# ---------------------------------------------------------------- sparse down (FloE)

def _floe_small(T=6, d=256, F=384, E=3, seed=3):
    rng = np.random.default_rng(seed)
    b = lambda *sh: f32_to_bf16_bits((rng.standard_normal(sh) * 0.05).astype(np.float32))
    x = f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    return x, b(E, F, d), b(E, F, d), b(E, d, F)


def test_floe_keep_all_is_the_dense_expert():
    """A threshold below zero keeps every channel: the rows equal the pinned dense
    SwiGLU expert (same fp64 arithmetic, bit for bit)."""
    x, wg, wu, wd = _floe_small()
    tok = np.array([0, 1, 2, 3, 4, 5, 0, 2], np.int32)
    ex = np.array([0, 0, 1, 1, 2, 2, 2, 0], np.int32)
    Y, u, keep = oracle.floe_rows(x, wg, wu, wd, np.full(3, -1.0, np.float32), tok, ex)
    ref = oracle.expert_rows(x, wg, wu, wd, "swiglu", oracle.ROUND_BF16, tok, ex)
    assert keep.all() and np.array_equal(Y, ref)
    # u is the fp64 up projection (numpy matmul)
    xf = bf16_bits_to_f32(x).astype(np.float64)
    for p_, (t, e) in enumerate(zip(tok, ex)):
        ref_u = bf16_bits_to_f32(wu[e]).astype(np.float64) @ xf[t]
        assert np.allclose(u[p_], ref_u, rtol=1e-12, atol=1e-12)


def test_floe_prune_all_and_given_decisions():
    x, wg, wu, wd = _floe_small(seed=4)
    tok = np.arange(6, dtype=np.int32)
    ex = np.array([0, 1, 2, 0, 1, 2], np.int32)
    Y, _, keep = oracle.floe_rows(x, wg, wu, wd, np.full(3, np.inf, np.float32), tok, ex)
    assert not keep.any() and np.all(Y == 0.0)
    # decisions follow the given values, not the oracle's own u
    Y0, u, _ = oracle.floe_rows(x, wg, wu, wd, np.zeros(3, np.float32), tok, ex)
    Yz, _, kz = oracle.floe_rows(x, wg, wu, wd, np.zeros(3, np.float32), tok, ex,
                                 u_given=np.zeros((6, 384), np.float32))
    assert not kz.any() and np.all(Yz == 0.0)
    Ys, _, ks = oracle.floe_rows(x, wg, wu, wd, np.zeros(3, np.float32), tok, ex,
                                 u_given=u.astype(np.float32))
    assert np.array_equal(ks, (np.abs(u.astype(np.float32)) > 0).astype(np.uint8))


def test_floe_single_row_equals_dense_with_pruned_columns_zeroed():
    """For one row, pruning channel f is the dense expert with column f of W_down
    zeroed (an independent route through the pinned dense routine)."""
    x, wg, wu, wd = _floe_small(seed=5)
    for t, e in ((0, 0), (3, 2), (5, 1)):
        tok, ex = np.array([t], np.int32), np.array([e], np.int32)
        _, u, _ = oracle.floe_rows(x, wg, wu, wd, np.full(3, -1.0, np.float32), tok, ex)
        thr = np.full(3, np.float32(np.quantile(np.abs(u[0]), 0.8)), np.float32)
        Y, _, keep = oracle.floe_rows(x, wg, wu, wd, thr, tok, ex)
        assert 0.1 < keep.mean() < 0.3
        wd2 = wd.copy()
        wd2[e][:, keep[0] == 0] = 0
        ref = oracle.expert_rows(x, wg, wu, wd2, "swiglu", oracle.ROUND_BF16, tok, ex)
        assert np.array_equal(Y, ref)


def test_floe_threshold_is_the_empirical_quantile():
    """The inverse empirical CDF at the target level: numpy's inverted-CDF
    quantile, and the fraction of samples at or below it is ceil(k n)/n."""
    rng = np.random.default_rng(9)
    for n, k in ((1000, 0.9), (917, 0.8), (5, 0.5), (64, 1.0)):
        a = rng.standard_normal(n)
        t = oracle.floe_threshold(a, k)
        assert t == float(np.quantile(np.abs(a), k, method="inverted_cdf"))
        assert (np.abs(a) <= t).sum() == max(1, math.ceil(k * n))
    # the workload's calibrated thresholds are the same reading
    from workloads.gen import FLOE_CAL_TOKENS, TID_XCAL, _normal
    wl = make_workload(get_config("mixtral_floe_decode", d=256, F=512, x_rows_of=None,
                                  weights_of=None))
    xc = bf16_bits_to_f32(_normal(wl.cfg.cfg_id, TID_XCAL, 0, (FLOE_CAL_TOKENS, 256), 1.0,
                                  True)).astype(np.float64)
    for e in range(wl.cfg.E):
        samples = xc @ bf16_bits_to_f32(wl.w_up[e]).astype(np.float64).T
        assert np.float32(oracle.floe_threshold(samples, 0.9)) == wl.floe_thr[e]


def test_floe_layer_keep_all_is_the_plain_layer():
    """Thresholds below zero: the sparse-down layer is the plain layer on the
    decoded INT2 up weights."""
    import dataclasses
    wl = make_workload(get_config("mixtral_floe_decode", T=20, d=256, F=512, x_rows_of=None,
                                  weights_of=None))
    wl.floe_thr = np.full(wl.cfg.E, -1.0, np.float32)
    fl = oracle.layer_forward(wl)
    plain = dataclasses.replace(wl, cfg=dataclasses.replace(wl.cfg, floe=False))
    plain.w_up = oracle.dequant_int2(wl.u2_up.q2, wl.u2_up.s2, wl.u2_up.z2)
    ref = oracle.layer_forward(plain)
    assert np.array_equal(fl["y"], ref["y"]) and fl["floe_keep"].all()
    assert np.array_equal(fl["floe_nnz"], np.where(ref["counts"] > 0, 512, 0))


# ---------------------------------------------------------------- atomic experts (OmniMoE)

def _grid_brute(pr, pc, K):
    """Full sort of every cell by (S descending, id ascending); S in fp32."""
    T, Nr = pr.shape
    Nc = pc.shape[1]
    out = np.empty((T, K), np.int64)
    for t in range(T):
        S = (pr[t][:, None] + pc[t][None, :]).astype(np.float32).ravel()
        ids = np.arange(Nr * Nc)
        order = np.lexsort((ids, -S.astype(np.float64)))
        out[t] = np.sort(order[:K])
    return out


@pytest.mark.parametrize("Nr,Nc,K,quant", [(4, 8, 5, True), (7, 3, 21, False), (16, 32, 64, True),
                                           (9, 9, 1, True), (5, 12, 17, False)])
def test_grid_topk_matches_brute_force(Nr, Nc, K, quant):
    rng = np.random.default_rng(Nr * 100 + Nc + K)
    T = 12
    pr = rng.standard_normal((T, Nr)).astype(np.float32)
    pc = rng.standard_normal((T, Nc)).astype(np.float32)
    if quant:   # a small alphabet: many exact ties in the sums
        pr = np.round(pr * 2) / 2
        pc = np.round(pc * 2) / 2
    idx, gate = oracle.grid_topk(pr, pc, K)
    assert np.array_equal(idx, _grid_brute(pr, pc, K))
    assert np.allclose(gate.astype(np.float64).sum(1), 1.0, atol=1e-6)


def test_grid_all_cells_gates_are_the_product_distribution():
    """K = N: the gates are softmax(l_r)_i * softmax(l_c)_j (the row and column
    log-probabilities add)."""
    rng = np.random.default_rng(2)
    lr = rng.standard_normal((6, 5)).astype(np.float32)
    lc = rng.standard_normal((6, 7)).astype(np.float32)
    pr, pc = oracle.log_softmax_rows(lr), oracle.log_softmax_rows(lc)
    idx, gate = oracle.grid_topk(pr, pc, 35)
    sr = np.exp(lr - lr.max(1, keepdims=True)); sr /= sr.sum(1, keepdims=True)
    sc = np.exp(lc - lc.max(1, keepdims=True)); sc /= sc.sum(1, keepdims=True)
    assert np.array_equal(idx, np.tile(np.arange(35), (6, 1)))
    ref = (sr[:, :, None] * sc[:, None, :]).reshape(6, 35)
    assert np.allclose(gate, ref, rtol=2e-6, atol=1e-8)


def test_grid_one_column_is_the_coarse_router():
    """Nc = 1: the column log-probability is 0, so the grid's top-K is the coarse
    top-k of the row logits (same set; gates equal)."""
    rng = np.random.default_rng(8)
    lr = rng.standard_normal((20, 12)).astype(np.float32)
    pr = oracle.log_softmax_rows(lr)
    pc = oracle.log_softmax_rows(np.zeros((20, 1), np.float32))
    assert np.all(pc == 0.0)
    for K in (1, 3, 12):
        idx, gate = oracle.grid_topk(pr, pc, K)
        cidx, cgate = oracle.topk_gates(lr, K)
        for t in range(20):
            o = np.argsort(cidx[t])
            assert np.array_equal(idx[t], cidx[t][o])
            assert np.allclose(gate[t], cgate[t][o], rtol=1e-6, atol=1e-7)


def _atomic_small(**over):
    kw = dict(T=24, d=256, nr=8, nc=16, E=128, k=16, F_shared=128)
    kw.update(over)
    return make_workload(get_config("omni_atomic", **kw))


def test_atomic_top1_relu_one_column_is_the_coarse_relu_layer():
    """K = 1, Nc = 1, ReLU: each token runs one width-1 ReLU expert with gate 1,
    which is the coarse ReLU layer with d_ff = 1 and top-1, bit for bit."""
    import dataclasses
    wl = _atomic_small(nr=12, nc=1, E=12, k=1, n_shared=0)
    wl.cfg = dataclasses.replace(wl.cfg, act="relu")
    at = oracle.atomic_layer_forward(wl)
    E, d = 12, wl.cfg.d
    lr = oracle.router_logits(wl.x, wl.w_router, None)
    cidx, cgate = oracle.topk_gates(lr, 1)
    assert np.array_equal(at["idx"], cidx) and np.all(cgate == 1.0)
    Y = oracle.expert_rows(wl.x, None, wl.w_in.reshape(E, 1, d),
                           np.ascontiguousarray(wl.w_out_t.T.reshape(E, d, 1)), "relu",
                           oracle.ROUND_BF16, np.arange(wl.cfg.T, dtype=np.int32), cidx[:, 0])
    assert np.array_equal(at["y"], oracle.combine(Y, None, cgate))


def test_atomic_silu_single_unit_closed_form():
    """One token, one unit: y = w_out * bf16(silu(x . w_in)), gate 1."""
    x = f32_to_bf16_bits(np.array([[1.0, 0.5]], np.float32))
    w_in = f32_to_bf16_bits(np.array([[1.5, 1.0]], np.float32))
    w_out_t = f32_to_bf16_bits(np.array([[2.0], [-0.25]], np.float32))
    idx = np.zeros((1, 1), np.int32)
    Y = oracle.atomic_rows(x, w_in, w_out_t, idx, np.ones((1, 1), np.float32), "silu",
                           np.zeros(1, np.int32))
    h = 2.0 / (1.0 + math.exp(-2.0))           # silu(2)
    a = float(bf16_bits_to_f32(f32_to_bf16_bits(np.array([h], np.float32)))[0])
    assert np.array_equal(Y, np.array([[2.0 * a, -0.25 * a]]))


def test_atomic_gate_scaled_value_rounded_once():
    """Two units with gates g and 1 - g: each contributes w_out * bf16(g * silu(u)),
    the gate inside the one bf16 rounding."""
    x = f32_to_bf16_bits(np.array([[1.0, 0.5]], np.float32))
    w_in = f32_to_bf16_bits(np.array([[1.5, 1.0], [0.5, -1.0]], np.float32))   # u = 2, 0
    w_out_t = f32_to_bf16_bits(np.array([[1.0, 3.0], [-2.0, 1.0]], np.float32))  # [d][N]
    idx = np.array([[0, 1]], np.int32)
    g = np.array([[0.75, 0.25]], np.float32)
    Y = oracle.atomic_rows(x, w_in, w_out_t, idx, g, "silu", np.zeros(1, np.int32))
    rb = lambda v: float(bf16_bits_to_f32(f32_to_bf16_bits(np.array([v], np.float32)))[0])
    a0 = rb(0.75 * (2.0 / (1.0 + math.exp(-2.0))))   # 1.3212 -> 1.3203125
    assert a0 != 0.75 * rb(2.0 / (1.0 + math.exp(-2.0)))
    assert Y[0, 0] == 1.0 * a0 + 3.0 * 0.0 and Y[0, 1] == -2.0 * a0   # silu(0) = 0


def test_atomic_layer_grid_relabelling_equivariance():
    """Swapping grid rows (and the atomic experts of those rows) or transposing the
    grid (rows <-> columns) relabels experts and leaves y unchanged."""
    wl = _atomic_small()
    ref = oracle.atomic_layer_forward(wl)
    nr, nc, d = 8, 16, wl.cfg.d
    perm = np.random.default_rng(3).permutation(nr)
    w2 = make_workload(get_config("omni_atomic", T=24, d=256, nr=8, nc=16, E=128, k=16,
                                  F_shared=128))
    w2.w_router = wl.w_router[perm]
    cell = (perm[:, None] * nc + np.arange(nc)[None, :]).ravel()   # new id -> old id
    w2.w_in = wl.w_in[cell]
    w2.w_out_t = np.ascontiguousarray(wl.w_out_t[:, cell])
    out = oracle.atomic_layer_forward(w2)
    assert np.allclose(out["y"], ref["y"], rtol=0, atol=1e-9)
    assert np.array_equal(np.sort(cell[out["idx"]], axis=1), ref["idx"])
    # transpose: rows and columns swap roles, id i*nc + j becomes j*nr + i
    import dataclasses
    w3 = make_workload(get_config("omni_atomic", T=24, d=256, nr=16, nc=8, E=128, k=16,
                                  F_shared=128))
    w3.w_router, w3.w_col = wl.w_col, wl.w_router
    tcell = (np.arange(nr)[None, :] * nc + np.arange(nc)[:, None]).ravel()   # (j, i) -> i*nc+j
    w3.w_in = wl.w_in[tcell]
    w3.w_out_t = np.ascontiguousarray(wl.w_out_t[:, tcell])
    out3 = oracle.atomic_layer_forward(w3)
    assert np.allclose(out3["y"], ref["y"], rtol=0, atol=1e-9)
    assert np.array_equal(out3["counts"].sum(), ref["counts"].sum())


# ---------------------------------------------------------------- planted mistakes

MUTANTS = [
    ("topk tie to higher id", "if (best < 0 || l[e] > l[best]) best = e;",
     "if (best < 0 || l[e] >= l[best]) best = e;"),
    ("bias dropped", "if (b_r) s += (double)b_r[e];", "(void)b_r;"),
    ("gate not normalised", "(float)(exp((double)l[out[j]] - m) / sum);",
     "(float)(exp((double)l[out[j]] - m));"),
    ("lis uses k twice", "(double)((int64_t)T * k);", "(double)((int64_t)T * k * k);"),
    ("unstable permutation", "int32_t row = offsets[e] + seen[e]++;",
     "int32_t row = offsets[e + 1] - 1 - seen[e]++;"),
    ("silu sign", "v = (g / (1.0 + exp(-g))) * u;", "v = (g / (1.0 + exp(g))) * u;"),
    ("down operand transposed",
     "size_t wo = (e * (size_t)d + (size_t)i) * (size_t)F;\n        double s = 0.0;\n"
     "        for (int f = 0; f < F; ++f) s += h[f] * elem(w_down, wdt, wo + f);",
     "size_t wo = e * (size_t)d * (size_t)F;\n        double s = 0.0;\n"
     "        for (int f = 0; f < F; ++f) s += h[f] * elem(w_down, wdt, wo + (size_t)f * d + i);"),
    ("combine drops shared term", "if (Ys) s += Ys[(size_t)t * d + i];", "(void)Ys;"),
    ("int4 high nibble first", "(word >> (4 * (kk % 8))) & 0xFu;",
     "(word >> (4 * (7 - kk % 8))) & 0xFu;"),
    ("int4 zero added", "float a = (float)nib - z;", "float a = (float)nib + z;"),
    ("bf16 rounding truncates", "double r = nearbyint(ldexp(v, -q));",
     "double r = trunc(ldexp(v, -q));"),
    ("replica takes even ranks", "idx_out[a] = (rank % 2 == 1) ? E : e;",
     "idx_out[a] = (rank % 2 == 0) ? E : e;"),
    ("replica split counts every expert", "    if (e == heavy) {\n      idx_out[a]",
     "    if (e >= 0) {\n      idx_out[a]"),
    ("mwq residual sign flipped", "        w = w + (bit ? m : -m);\n      }\n      if (bits == 4)",
     "        w = w + (bit ? -m : m);\n      }\n      if (bits == 4)"),
    ("floe mask inverted", "int keep = mag > (double)thr[e];", "int keep = mag < (double)thr[e];"),
    ("floe silu on the up output", "h[f] = orc_round_bf16((g / (1.0 + exp(-g))) * u);",
     "h[f] = orc_round_bf16((u / (1.0 + exp(-u))) * g);"),
    ("floe h not rounded", "h[f] = orc_round_bf16((g / (1.0 + exp(-g))) * u);",
     "h[f] = (g / (1.0 + exp(-g))) * u;"),
    ("floe given values ignored", "double mag = u_given ? fabs((double)u_given[(size_t)p * F + f]) : fabs(u);",
     "double mag = fabs(u);"),
    ("grid ties to the higher id", "return (x->id < y->id) ? -1 : (x->id > y->id);",
     "return (x->id > y->id) ? -1 : (x->id < y->id);"),
    ("grid slots left in score order", "qsort(out, (size_t)K, sizeof(int32_t), cmp_int32);",
     "(void)cmp_int32;"),
    ("atomic activation swapped", "double h = act == 0 ? u / (1.0 + exp(-u)) : (u > 0.0 ? u : 0.0);",
     "double h = act == 1 ? u / (1.0 + exp(-u)) : (u > 0.0 ? u : 0.0);"),
    ("atomic output vectors read as rows", "y[i] += a * bf16_to_double(w_out[(size_t)i * N + e]);",
     "y[i] += a * bf16_to_double(w_out[e * (size_t)d + i]);"),
    ("atomic gate outside the rounding", "double a = orc_round_bf16((double)gate[t * K + s] * h);",
     "double a = (double)gate[t * K + s] * orc_round_bf16(h);"),
    ("mwq second plane read from the first", "((uint32_t)p4[r * (K / 32) + kk / 32] >> mwq_bit(kk))",
     "((uint32_t)p3[r * (K / 32) + kk / 32] >> mwq_bit(kk))"),
    ("mwq 2-bit fields in natural order", "(w2 >> (2 * mwq_field(kk))) & 0x3u;",
     "(w2 >> (2 * (kk % 16))) & 0x3u;"),
    ("mwq residual bits in natural order", "  return 8 * (i % 4) + i / 4;", "  return i;"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(name, old, new, tmp_path):
    """A copy of the oracle with one plausible mistake must fail this file's pins."""
    import subprocess
    import sys
    src = open(oracle._SRC).read()
    assert old in src, "mutation anchor not found: " + name
    mdir = tmp_path / "oracle"
    mdir.mkdir()
    (mdir / "moe_oracle.c").write_text(src.replace(old, new, 1))
    (mdir / "__init__.py").write_text(open(os.path.join(os.path.dirname(oracle._SRC),
                                                        "__init__.py")).read())
    env = dict(os.environ)
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env["PYTHONPATH"] = str(tmp_path) + os.pathsep + root
    env["ORACLE_MUTANT_RUN"] = "1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.abspath(__file__), "-k", "not planted_mistake"],
                       cwd=str(tmp_path), env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, "pins did not catch mutant: %s\n%s" % (name, r.stdout[-2000:])
    assert "failed" in r.stdout or "error" in r.stdout.lower()
