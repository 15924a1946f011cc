"""Parity of the replica dispatch (moe_replica_split, moe_layer_forward_replica)
with the CPU oracle.

The heavy expert's odd-ranked assignments run on an INT4 copy of it as slot E.
Integers of the split routing (counts over E+1 slots, offsets, permutation,
LIS over E+1 slots, the base LIS) must match bit for bit given the GPU's fp32
logits; y within max-abs 2e-2 and relative L2 1e-2 against the oracle layer
with the replica's INT4 weights decoded by the oracle's own rule.
"""
import functools

import numpy as np
import pytest

import oracle
from workloads import get_config, make_replica, make_workload

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


@pytest.mark.parametrize("T,E,k", [(16, 8, 2), (1, 8, 2), (333, 16, 8), (4096, 8, 1),
                                   (8192, 64, 6)])
def test_replica_split_matches_oracle(T, E, k):
    _say("replica split T=%d E=%d k=%d" % (T, E, k))
    moe = _moe()
    rng = np.random.default_rng(T + 7 * E + k)
    p = rng.zipf(1.3, size=(T, E)).astype(np.float64)
    idx = np.argsort(-p + rng.random((T, E)) * 1e-3, axis=1)[:, :k].astype(np.int32)
    di = torch.from_numpy(idx).cuda()
    c, o, ra, ar, lis = moe.permute(di, E)
    rc, _, _, _, _ = oracle.permute(idx, E)
    heavy = oracle.heavy_hitter(rc)
    out = moe.replica_split(di, c, o, ar, E, heavy)
    torch.cuda.synchronize()
    idx2 = oracle.replica_split(idx, E, heavy)
    c2, o2, ra2, ar2, lis2 = oracle.permute(idx2, E + 1)
    assert np.array_equal(out["idx"].cpu().numpy(), idx2)
    assert np.array_equal(out["counts"].cpu().numpy(), c2)
    assert np.array_equal(out["offsets"].cpu().numpy(), o2)
    assert np.array_equal(out["row_assign"].cpu().numpy()[:T * k], ra2)
    assert np.array_equal(out["assign_row"].cpu().numpy()[:T * k], ar2)
    assert float(out["lis"].cpu()[0]) == lis2


def run_replica_layer(wl):
    """Plain layer call (its counts name the heavy expert), then the replica layer."""
    from sparse_mixture_experts_wavefront_amd.device_inputs import replica_to_device, to_device
    moe = _moe()
    layer, x = to_device(wl)
    _, aux0 = moe.layer_forward(layer, x)
    torch.cuda.synchronize()
    heavy = oracle.heavy_hitter(aux0["counts"].cpu().numpy())
    rep = make_replica(wl, heavy)
    y, aux = moe.layer_forward(layer, x, replica=replica_to_device(rep))
    torch.cuda.synchronize()
    T, k = wl.cfg.T, wl.cfg.k
    g = {n: t.cpu().numpy() for n, t in aux.items()}
    g["row_assign"] = g["row_assign"][:T * k]
    g["assign_row"] = g["assign_row"][:T * k]
    g["lis"] = float(g["lis"][0])
    g["lis_base"] = float(g["lis_base"][0])
    g["y"] = y.cpu().numpy()
    return rep, g


def check_replica(wl, rep, g, tokens=None):
    ref = oracle.layer_forward(wl, logits=g["logits"], replica=rep, tokens=tokens)
    plain = oracle.layer_forward(wl, logits=g["logits"], routing_only=True)
    assert np.array_equal(g["idx"], plain["idx"])              # the router's own choice
    assert np.array_equal(g["counts"], ref["counts"])          # E + 1 slots
    assert np.array_equal(g["offsets"], ref["offsets"])
    assert np.array_equal(g["row_assign"], ref["row_assign"])
    assert np.array_equal(g["assign_row"], ref["assign_row"])
    assert g["lis"] == ref["lis"]
    assert g["lis_base"] == ref["base_lis"] == plain["lis"]
    gy = g["y"] if tokens is None else g["y"][np.asarray(tokens)]
    ry = ref["y"].astype(np.float64)
    d = np.abs(gy.astype(np.float64) - ry)
    rel = np.linalg.norm(gy.astype(np.float64) - ry) / max(np.linalg.norm(ry), 1e-30)
    print("  LIS %.4f -> %.4f; y max-abs %.3e rel-L2 %.3e" % (g["lis_base"], g["lis"], d.max(), rel),
          flush=True)
    assert d.max() <= 2e-2, "y max-abs %g" % d.max()
    assert rel <= 1e-2, "y rel-L2 %g" % rel
    return ref


SMALL = {
    # T > 64: the replica's projections decoded to bf16; it runs as expert E of
    # the main tiled launches (E + 1 = 65 for the DeepSeek shape: the tile map's
    # second 64-expert chunk)
    "switch_small": ("switch_bf16", dict(T=300, d=256, F=384)),
    "mixtral_small": ("mixtral_prefill_bf16", dict(T=333, d=512, F=640)),
    "deepseek_small": ("deepseek_v2_lite_bf16", dict(T=257, d=256, F=256, F_shared=64)),
    # T <= 64: the replica runs through the weight-streaming INT4 kernel
    "decode_small": ("mixtral_decode_bf16", dict(T=16, d=512, F=1024, x_rows_of=None,
                                                 weights_of=None)),
    "decode_relu_small": ("switch_bf16", dict(T=40, d=512, F=1024)),
}


@pytest.mark.parametrize("case", list(SMALL))
def test_replica_layer_parity_small(case):
    name, over = SMALL[case]
    _say("replica layer %s %s" % (case, over))
    wl = _workload(name, **over)
    rep, g = run_replica_layer(wl)
    check_replica(wl, rep, g)


@pytest.mark.parametrize("name", ["switch_bf16", "deepseek_v2_lite_bf16"])
def test_replica_layer_full_size(name):
    """The two skewed configurations; y on every token."""
    _say("replica layer full-size %s" % name)
    wl = _workload(name)
    rep, g = run_replica_layer(wl)
    check_replica(wl, rep, g)
    assert g["lis"] < g["lis_base"]
