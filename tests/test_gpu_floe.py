"""Parity of the contextual sparse down-projection layer (moe_layer_forward_floe)
with the CPU oracle.

Keep/prune decisions are floating-point comparisons deciding integers, so both
sides take them on the same fp32 values: the oracle decides on the GPU's up
outputs (as routing uses the GPU's logits), and those outputs are checked
against the oracle's own fp64 ones.  Then every integer (routing, counts,
offsets, LIS, kept-channel counts and lists per expert) must match bit for bit,
and y within max-abs 2e-2 and relative L2 1e-2.
"""
import functools

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


def _say(msg):
    print("\n[case] " + msg, flush=True)


@functools.lru_cache(maxsize=None)
def _workload(name, **over):
    return make_workload(get_config(name, **over) if over else get_config(name))


def run_floe_layer(wl):
    import sparse_mixture_experts_wavefront_amd as moe
    from sparse_mixture_experts_wavefront_amd.device_inputs import floe_to_device, to_device
    layer, x = to_device(wl)
    y, aux = moe.layer_forward(layer, x, floe=floe_to_device(wl))
    torch.cuda.synchronize()
    T, k = wl.cfg.T, wl.cfg.k
    g = {n: t.cpu().numpy() for n, t in aux.items()}
    for n in ("row_assign", "assign_row"):
        g[n] = g[n][:T * k]
    g["floe_u"] = g["floe_u"][:T * k]
    g["lis"] = float(g["lis"][0])
    g["y"] = y.cpu().numpy()
    return g


def check_floe(wl, g, tokens=None):
    ref = oracle.layer_forward(wl, logits=g["logits"], floe_u=g["floe_u"], tokens=tokens)
    for n in ("idx", "counts", "offsets", "row_assign", "assign_row"):
        assert np.array_equal(g[n], ref[n]), n
    assert g["lis"] == ref["lis"]
    E, F = wl.cfg.E, wl.cfg.F
    if tokens is None:
        # the GPU's up outputs against the oracle's fp64 ones
        du = np.abs(g["floe_u"].astype(np.float64) - ref["floe_u"])
        assert du.max() <= 1e-4 * max(1.0, np.abs(ref["floe_u"]).max()), du.max()
        # kept channels per expert: counts and ascending lists
        assert np.array_equal(g["floe_nnz"], ref["floe_nnz"])
        pe = ref["idx"].reshape(-1)[ref["row_assign"]]
        for e in range(E):
            if ref["counts"][e] == 0:
                continue
            union = np.flatnonzero(ref["floe_keep"][pe == e].any(axis=0))
            assert np.array_equal(g["floe_channels"][e][:len(union)], union), e
    gy = g["y"] if tokens is None else g["y"][np.asarray(tokens)]
    ry = ref["y"].astype(np.float64)
    d = np.abs(gy.astype(np.float64) - ry)
    rel = np.linalg.norm(gy.astype(np.float64) - ry) / max(np.linalg.norm(ry), 1e-30)
    kept = ref["floe_keep"].mean()
    print("  kept %.3f of channels per row; y max-abs %.3e rel-L2 %.3e" % (kept, d.max(), rel),
          flush=True)
    assert d.max() <= 2e-2, "y max-abs %g" % d.max()
    if np.linalg.norm(ry) > 0:
        assert rel <= 1e-2, "y rel-L2 %g" % rel
    else:
        assert np.all(gy == 0)
    return ref


def _small(T=16, d=512, F=1024, **over):
    return _workload("mixtral_floe_decode", T=T, d=d, F=F, x_rows_of=None, weights_of=None, **over)


SMALL = {
    "decode": lambda: _small(),
    "one_token": lambda: _small(T=1),
    # more than 16 rows per expert: several passes in the gate and down kernels
    "many_rows": lambda: _small(T=64, E=4),
    # K ranges that leave waves idle in the INT2 up pass (d: 3 iterations of 512)
    "ragged": lambda: _small(T=24, d=1536, F=2560),
    # a few active experts among 64: blocks are numbered over the active ones
    # (lane = expert up to 63) and the gate chunks over their lists
    "few_of_many": lambda: _small(T=3, E=64),
    "shared_experts": lambda: _workload("deepseek_v2_lite_bf16", T=40, d=512, F=512, E=16, k=4,
                                        F_shared=256, floe=True, sparsity=0.9),
}


@pytest.mark.parametrize("case", list(SMALL))
def test_floe_layer_parity_small(case):
    _say("floe layer %s" % case)
    wl = SMALL[case]()
    g = run_floe_layer(wl)
    check_floe(wl, g)


@pytest.mark.parametrize("thr", [-1.0, np.inf])
def test_floe_layer_keep_all_and_prune_all(thr):
    """Every channel kept (the lists cover all of d_ff) or none (y = 0)."""
    import dataclasses
    _say("floe layer thresholds %s" % thr)
    wl = dataclasses.replace(_small(T=20))
    wl.floe_thr = np.full(wl.cfg.E, thr, np.float32)
    g = run_floe_layer(wl)
    ref = check_floe(wl, g)
    if thr < 0:
        assert np.all(g["floe_nnz"][ref["counts"] > 0] == wl.cfg.F)
    else:
        assert np.all(g["floe_nnz"] == 0) and np.all(g["y"] == 0)


@pytest.mark.parametrize("name", ["mixtral_floe_decode", "mixtral_floe_decode_t1"])
def test_floe_layer_full_size(name):
    _say("floe layer full-size %s" % name)
    wl = _workload(name)
    g = run_floe_layer(wl)
    check_floe(wl, g)
