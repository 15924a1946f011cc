"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Integers (top-k indices in slot order, counts, offsets, permutation, LIS) must
match bit for bit given the same fp32 logits: the oracle's routing is fed the
GPU's logits.  Floats: logits within 1e-4 (bf16 layers) / 1e-5 (fp32), gates
within 1e-6, y within max-abs 2e-2 and relative L2 1e-2 (bf16) or 1e-5 (fp32).
"""
import functools
import math

import numpy as np
import pytest

import oracle
from workloads import get_config, make_workload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_mixture_experts_wavefront_amd as moe
    moe.lib()  # raises if libmoe.so is missing: no fallback path exists


def _moe():
    import sparse_mixture_experts_wavefront_amd as moe
    return moe


def _say(msg):
    print("\n[case] " + msg, flush=True)


@functools.lru_cache(maxsize=None)
def _workload(name, **over):
    return make_workload(get_config(name, **over) if over else get_config(name))


def _tol(wl):
    return (1e-5, 1e-5, 1e-5) if wl.cfg.dtype == "f32" else (1e-4, 2e-2, 1e-2)


def run_layer(wl, logits=None, flags=0):
    from sparse_mixture_experts_wavefront_amd.device_inputs import to_device
    moe = _moe()
    layer, x = to_device(wl)
    lg = None if logits is None else torch.from_numpy(logits).cuda()
    y, aux = moe.layer_forward(layer, x, logits=lg, flags=flags)
    torch.cuda.synchronize()
    T, k = wl.cfg.T, wl.cfg.k
    out = {n: t.cpu().numpy() for n, t in aux.items()}
    out["row_assign"] = out["row_assign"][:T * k]
    out["assign_row"] = out["assign_row"][:T * k]
    out["y"] = y.cpu().numpy()
    out["lis"] = float(out["lis"][0])
    return out


def check_routing(wl, g):
    """Routing integers bit-exact and gates/logits within tolerance."""
    ltol = _tol(wl)[0]
    ref = oracle.layer_forward(wl, logits=g["logits"], routing_only=True)
    err = np.abs(g["logits"].astype(np.float64) - ref["logits"].astype(np.float64)).max() \
        if wl.cfg.T else 0.0
    assert err <= ltol, "logits max-abs %g" % err
    assert np.array_equal(g["idx"], ref["idx"])
    assert np.array_equal(g["counts"], ref["counts"])
    assert np.array_equal(g["offsets"], ref["offsets"])
    assert np.array_equal(g["row_assign"], ref["row_assign"])
    assert np.array_equal(g["assign_row"], ref["assign_row"])
    assert g["lis"] == ref["lis"] or (math.isnan(g["lis"]) and math.isnan(ref["lis"]))
    if wl.cfg.T:
        assert np.abs(g["gates"] - ref["gate"]).max() <= 1e-6
        assert np.abs(g["gates"].astype(np.float64).sum(1) - 1.0).max() <= 1e-6
    return ref


def check_y(wl, g, tokens=None):
    _, atol, rtol = _tol(wl)
    ref = oracle.layer_forward(wl, logits=g["logits"], tokens=tokens)
    gy = g["y"] if tokens is None else g["y"][np.asarray(tokens)]
    ry = ref["y"].astype(np.float64)
    d = np.abs(gy.astype(np.float64) - ry)
    rel = np.linalg.norm(gy.astype(np.float64) - ry) / max(np.linalg.norm(ry), 1e-30)
    print("  y max-abs %.3e rel-L2 %.3e (|y| max %.3e)" % (d.max(), rel, np.abs(ry).max()),
          flush=True)
    assert d.max() <= atol, "y max-abs %g" % d.max()
    assert rel <= rtol, "y rel-L2 %g" % rel


# ---------------------------------------------------------------- parity-size workloads

SMALL = {
    "tiny_fp32": ("tiny_fp32", {}),
    "switch_small": ("switch_bf16", dict(T=300, d=256, F=384)),
    "mixtral_small": ("mixtral_prefill_bf16", dict(T=333, d=512, F=640)),
    "decode_small": ("mixtral_decode_bf16", dict(T=16, d=512, F=1024, x_rows_of=None,
                                                 weights_of=None)),
    # several K slices per weight strip in the streaming kernels (regression:
    # row-block selection must stay compile-time there)
    "decode_multi_kslice": ("mixtral_decode_bf16", dict(T=16, d=2048, F=1536, x_rows_of=None,
                                                        weights_of=None)),
    "int4_multi_kslice": ("mixtral_int4_decode", dict(T=48, d=2048, F=1536, x_rows_of=None,
                                                      weights_of=None)),
    "decode_relu_small": ("switch_bf16", dict(T=40, d=512, F=1024)),
    "deepseek_small": ("deepseek_v2_lite_bf16", dict(T=257, d=256, F=192, F_shared=64)),
    "int4_small": ("mixtral_int4_decode", dict(T=64, d=512, F=1024, x_rows_of=None,
                                               weights_of=None)),
    "int4_relu_small": ("mixtral_int4_decode", dict(T=33, d=512, F=1024, act="relu",
                                                    x_rows_of=None, weights_of=None)),
    "int4_prefill_small": ("mixtral_int4_decode", dict(T=300, d=256, F=384, x_rows_of=None,
                                                       weights_of=None)),
    "single_token": ("mixtral_prefill_bf16", dict(T=1, d=512, F=640)),
    # small-batch routing: router GEMM split in 128-wide K blocks
    # (d % 256 != 0), and not split at all (d % 128 != 0: the routing
    # workgroup's own GEMM)
    "route_split_128": ("mixtral_decode_bf16", dict(T=48, d=1664, F=512, x_rows_of=None,
                                                    weights_of=None)),
    "route_unsplit": ("mixtral_decode_bf16", dict(T=8, d=200, F=256, x_rows_of=None,
                                                  weights_of=None)),
    # INT4 row-split down with 8 K parts of 512 (4 groups each: 8-byte scale staging)
    "int4_down_8parts": ("mixtral_int4_decode", dict(T=32, d=1024, F=4096, x_rows_of=None,
                                                     weights_of=None)),
}


@pytest.mark.parametrize("case", list(SMALL))
def test_layer_parity_small(case):
    name, over = SMALL[case]
    _say("%s %s" % (case, over))
    wl = _workload(name, **over)
    g = run_layer(wl)
    check_routing(wl, g)
    check_y(wl, g)


BF16_ROWS = {
    "switch_small": ("switch_bf16", dict(T=300, d=256, F=384)),
    "mixtral_small": ("mixtral_prefill_bf16", dict(T=333, d=512, F=640)),
    "deepseek_small": ("deepseek_v2_lite_bf16", dict(T=257, d=256, F=256, F_shared=64)),
    "deepseek_full": ("deepseek_v2_lite_bf16", {}),
}


@pytest.mark.parametrize("case", list(BF16_ROWS))
def test_bf16_rows_flag(case):
    """MOE_F_BF16_ROWS (tiled path, d_ff a multiple of 128): the gate-scaled
    expert rows travel as bf16 between the down pass and the combine (one more
    rounding per row, the same tolerance); the result stays run-to-run
    deterministic and differs from the fp32-row one (the flag took effect)."""
    name, over = BF16_ROWS[case]
    _say("bf16 rows %s %s" % (case, over))
    moe = _moe()
    wl = _workload(name, **over)
    g = run_layer(wl, flags=moe.MOE_F_BF16_ROWS)
    check_routing(wl, g)
    check_y(wl, g)
    g2 = run_layer(wl, flags=moe.MOE_F_BF16_ROWS)
    assert np.array_equal(g["y"], g2["y"])
    g32 = run_layer(wl)
    assert not np.array_equal(g["y"], g32["y"])


def test_int4_fractional_zero_point():
    _say("int4 fractional zero point")
    cfg = get_config("mixtral_int4_decode", T=40, d=512, F=1024, x_rows_of=None, weights_of=None)
    wl = make_workload(cfg, fractional_zero=True)
    assert np.any(wl.q_up.zero.view(np.float16) % 1 != 0)
    g = run_layer(wl)
    check_routing(wl, g)
    check_y(wl, g)


@pytest.mark.parametrize("T", [200, 64])
def test_all_tokens_one_expert_and_empty_experts(T):
    _say("all tokens routed to expert 3 (k=1), seven empty experts, T=%d" % T)
    wl = make_workload(get_config("switch_bf16", T=T, d=512, F=512))
    wl.b_router = np.zeros(8, np.float32)
    wl.b_router[3] = 100.0
    g = run_layer(wl)
    ref = check_routing(wl, g)
    assert ref["counts"][3] == T and ref["lis"] == 8.0
    check_y(wl, g)


def test_single_expert_and_k_equals_e():
    _say("E=1 k=1 and E=4 k=4")
    for over in (dict(E=1, k=1), dict(E=4, k=4)):
        wl = make_workload(get_config("mixtral_prefill_bf16", T=70, d=256, F=256, **over))
        g = run_layer(wl)
        check_routing(wl, g)
        check_y(wl, g)


def test_empty_batch():
    _say("T=0")
    moe = _moe()
    from sparse_mixture_experts_wavefront_amd.device_inputs import to_device
    wl = make_workload(get_config("mixtral_prefill_bf16", T=4, d=256, F=256))
    layer, x = to_device(wl)
    r = moe.LayerRunner(layer, 0)
    r(x[:0])
    torch.cuda.synchronize()
    idx = torch.zeros(0, 2, dtype=torch.int32, device="cuda")
    counts, offsets, _, _, lis = moe.permute(idx, 8)
    torch.cuda.synchronize()
    assert counts.cpu().numpy().sum() == 0 and math.isnan(float(lis.cpu()[0]))


@pytest.mark.parametrize("name,over", [
    ("deepseek_v2_lite_bf16", dict(T=257, d=256, F=192, F_shared=64)),
    ("mixtral_decode_bf16", dict(T=16, d=2048, F=1536, x_rows_of=None, weights_of=None)),
    ("mixtral_int4_decode", dict(T=64, d=1024, F=1024, x_rows_of=None, weights_of=None)),
])
def test_deterministic_rerun(name, over):
    _say("bitwise determinism %s %s" % (name, over))
    wl = _workload(name, **over)
    a = run_layer(wl)
    b = run_layer(wl)
    assert np.array_equal(a["y"], b["y"]) and np.array_equal(a["logits"], b["logits"])


def test_token_permutation_equivariance():
    _say("token permutation equivariance")
    wl = make_workload(get_config("mixtral_prefill_bf16", T=150, d=256, F=256))
    a = run_layer(wl)
    perm = np.random.default_rng(11).permutation(150)
    wl.x = wl.x[perm].copy()
    b = run_layer(wl)
    assert np.array_equal(b["idx"], a["idx"][perm])
    assert np.array_equal(b["counts"], a["counts"])
    assert np.array_equal(b["y"], a["y"][perm])


# ---------------------------------------------------------------- entry points alone

def test_route_topk_ties_and_signed_zero():
    _say("route_topk with given logits: ties, signed zeros")
    moe = _moe()
    rng = np.random.default_rng(12)
    for E, k in ((8, 2), (64, 6), (5, 5), (3, 1), (17, 8)):
        alphabet = np.array([-1.0, -0.0, 0.0, 0.25, 1.0], np.float32)
        lg = alphabet[rng.integers(0, 5, size=(100, E))]
        lg[50:] = rng.standard_normal((50, E)).astype(np.float32)
        _, idx, gate = moe.route_topk(None, None, None, k, logits=torch.from_numpy(lg).cuda(),
                                      logits_given=True)
        torch.cuda.synchronize()
        ridx, rgate = oracle.topk_gates(lg, k)
        assert np.array_equal(idx.cpu().numpy(), ridx), (E, k)
        assert np.abs(gate.cpu().numpy() - rgate).max() <= 1e-6


def test_permute_multiblock_path():
    _say("permute: multi-block path (T*k > fused limit), skewed")
    moe = _moe()
    rng = np.random.default_rng(13)
    for T, E, k in ((8192, 64, 6), (20000, 8, 1), (3000, 16, 8)):
        p = rng.zipf(1.3, size=(T, E)).astype(np.float64)
        idx = np.argsort(-p + rng.random((T, E)) * 1e-3, axis=1)[:, :k].astype(np.int32)
        c, o, ra, ar, lis = moe.permute(torch.from_numpy(idx).cuda(), E)
        torch.cuda.synchronize()
        rc, ro, rra, rar, rlis = oracle.permute(idx, E)
        assert np.array_equal(c.cpu().numpy(), rc) and np.array_equal(o.cpu().numpy(), ro)
        assert np.array_equal(ra.cpu().numpy(), rra) and np.array_equal(ar.cpu().numpy(), rar)
        assert float(lis.cpu()[0]) == rlis


def test_permute_single_block_mid_sizes():
    _say("permute: one 1024-thread block (fused limit < T*k <= 8192), skewed and edge sizes")
    moe = _moe()
    rng = np.random.default_rng(17)
    for T, E, k in ((2049, 8, 1), (4096, 8, 1), (4096, 64, 2), (1365, 64, 6), (3000, 1, 2),
                    (2730, 3, 3), (1100, 37, 2)):
        p = rng.zipf(1.3, size=(T, E)).astype(np.float64)
        idx = np.argsort(-p + rng.random((T, E)) * 1e-3, axis=1)[:, :k].astype(np.int32)
        c, o, ra, ar, lis = moe.permute(torch.from_numpy(idx).cuda(), E)
        torch.cuda.synchronize()
        rc, ro, rra, rar, rlis = oracle.permute(idx, E)
        assert np.array_equal(c.cpu().numpy(), rc) and np.array_equal(o.cpu().numpy(), ro)
        assert np.array_equal(ra.cpu().numpy(), rra) and np.array_equal(ar.cpu().numpy(), rar)
        assert float(lis.cpu()[0]) == rlis


def test_grouped_ffn_single_dense_expert_and_combine():
    _say("grouped_ffn with offsets NULL (one dense expert), combine alone")
    moe = _moe()
    from sparse_mixture_experts_wavefront_amd.device_inputs import to_device
    wl = make_workload(get_config("mixtral_prefill_bf16", T=130, d=256, F=320, E=1, k=1))
    layer, x = to_device(wl)
    y_rows = moe.grouped_ffn(x, 1, 1, "swiglu", layer.routed)
    torch.cuda.synchronize()
    Y = oracle.expert_rows(wl.x, wl.w_gate, wl.w_up, wl.w_down, "swiglu", oracle.ROUND_BF16,
                           np.arange(130, dtype=np.int32), np.zeros(130, np.int32))
    d = np.abs(y_rows.cpu().numpy() - Y)
    assert d.max() <= 2e-2 and np.linalg.norm(y_rows.cpu().numpy() - Y) / np.linalg.norm(Y) <= 1e-2
    # combine: gathers k rows per token in slot order plus a shared term
    rng = np.random.default_rng(14)
    T, k, dd = 50, 3, 64
    rows = rng.standard_normal((T * k, dd)).astype(np.float32)
    ar = rng.permutation(T * k).astype(np.int32)
    ys = rng.standard_normal((T, dd)).astype(np.float32)
    y = moe.combine(torch.from_numpy(rows).cuda(), torch.from_numpy(ar).cuda(), T, k,
                    torch.from_numpy(ys).cuda())
    torch.cuda.synchronize()
    ref = np.zeros((T, dd), np.float32)
    for t in range(T):
        s = rows[ar[t * k]].copy()
        for j in range(1, k):
            s = s + rows[ar[t * k + j]]
        ref[t] = s + ys[t]
    assert np.array_equal(y.cpu().numpy(), ref)           # same fp32 order: bitwise


# ---------------------------------------------------------------- full-size workloads

FULL = ["tiny_fp32", "switch_bf16", "mixtral_decode_bf16", "mixtral_prefill_bf16",
        "deepseek_v2_lite_bf16", "mixtral_int4_decode"]


@pytest.mark.parametrize("name", FULL)
def test_layer_parity_full_size(name):
    """Full configs in the benchmark's launch configuration; y on every token,
    so every row tile, half tile and K slice of the launch is compared."""
    _say("full-size %s" % name)
    wl = _workload(name)
    g = run_layer(wl)
    ref = check_routing(wl, g)
    check_y(wl, g)
    print("  LIS %.6f counts %s" % (ref["lis"], ref["counts"][:16]), flush=True)
