"""Parity of the nested low-bit expert path (moe_mwq_group, moe_layer_forward_mwq)
with the CPU oracle.

Every (token, slot) assignment runs its expert at its own width (2, 3 or 4 bits,
the lower widths nested in the higher ones); rows are grouped by (expert, width).
Integers (the router's routing, counts, offsets, LIS; the grouping over 3E
groups) must match bit for bit given the GPU's fp32 logits; y within max-abs
2e-2 and relative L2 1e-2 against the oracle layer, which decodes every weight
with its own fp32 rule and runs the experts in fp64.
"""
import dataclasses
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


def _moe():
    import sparse_mixture_experts_wavefront_amd as moe
    return moe


def _say(msg):
    print("\n[case] " + msg, flush=True)


@functools.lru_cache(maxsize=None)
def _workload(name, **over):
    return make_workload(get_config(name, **over) if over else get_config(name))


@pytest.mark.parametrize("T,E,k", [(16, 8, 2), (1, 8, 2), (333, 21, 8), (9000, 8, 2), (0, 8, 2)])
def test_mwq_group_matches_oracle(T, E, k):
    """Grouping alone, widths including values outside 2..4 (read as the nearest);
    9000 x 2 assignments take the multi-block permutation."""
    _say("mwq group T=%d E=%d k=%d" % (T, E, k))
    moe = _moe()
    rng = np.random.default_rng(T + 5 * E + k)
    idx = np.array([rng.permutation(E)[:k] for _ in range(T)], np.int32).reshape(T, k)
    widths = rng.integers(0, 7, size=(T, k)).astype(np.int32)
    out = moe.mwq_group(torch.from_numpy(idx).cuda(), torch.from_numpy(widths).cuda(), E)
    torch.cuda.synchronize()
    vidx, c3, o3, ra3, ar3 = oracle.mwq_groups(idx, widths, E)
    assert np.array_equal(out["group_idx"].cpu().numpy(), vidx)
    assert np.array_equal(out["counts"].cpu().numpy(), c3)
    assert np.array_equal(out["offsets"].cpu().numpy(), o3)
    assert np.array_equal(out["row_assign"].cpu().numpy()[:T * k], ra3)
    assert np.array_equal(out["assign_row"].cpu().numpy()[:T * k], ar3)


def run_mwq_layer(wl):
    from sparse_mixture_experts_wavefront_amd.device_inputs import mwq_to_device, to_device
    moe = _moe()
    layer, x = to_device(wl)
    ex, widths = mwq_to_device(wl)
    y, aux = moe.layer_forward(layer, x, mwq=ex, widths=widths)
    torch.cuda.synchronize()
    T, k = wl.cfg.T, wl.cfg.k
    g = {n: t.cpu().numpy() for n, t in aux.items()}
    for n in ("row_assign", "assign_row", "mwq_row_assign", "mwq_assign_row"):
        g[n] = g[n][:T * k]
    g["lis"] = float(g["lis"][0])
    g["y"] = y.cpu().numpy()
    return g


def check_mwq(wl, g, tokens=None):
    ref = oracle.layer_forward(wl, logits=g["logits"], tokens=tokens)
    for n in ("idx", "counts", "offsets", "row_assign", "assign_row"):
        assert np.array_equal(g[n], ref[n]), n                  # the router's own routing
    assert g["lis"] == ref["lis"]
    for n in ("mwq_idx", "mwq_counts", "mwq_offsets", "mwq_row_assign", "mwq_assign_row"):
        assert np.array_equal(g[n], ref[n]), n                  # (expert, width) groups
    gy = g["y"] if tokens is None else g["y"][np.asarray(tokens)]
    ry = ref["y"].astype(np.float64)
    d = np.abs(gy.astype(np.float64) - ry)
    rel = np.linalg.norm(gy.astype(np.float64) - ry) / max(np.linalg.norm(ry), 1e-30)
    print("  groups %s; y max-abs %.3e rel-L2 %.3e" % (g["mwq_counts"].tolist(), d.max(), rel),
          flush=True)
    assert d.max() <= 2e-2, "y max-abs %g" % d.max()
    assert rel <= 1e-2, "y rel-L2 %g" % rel
    return ref


def _small(T=16, d=512, F=1024, **over):
    return _workload("mixtral_mwq_decode", T=T, d=d, F=F, x_rows_of=None, weights_of=None, **over)


def _with_widths(wl, fn):
    w2 = dataclasses.replace(wl)
    w2.bits = fn(wl.bits).astype(np.int32)
    return w2


SMALL = {
    "decode_mixed": lambda: _small(),
    "one_token": lambda: _small(T=1),
    # passes of 16 rows with one, two or three widths present
    "many_rows": lambda: _small(T=64, E=4),
    # K ranges that leave waves with nothing (d: 3 iterations of 512, F: 5)
    "ragged_k": lambda: _small(T=24, d=1536, F=2560),
    # T*k = 4 of 20 experts: the grid covers four experts, numbered over those with rows
    "few_of_many": lambda: _small(T=2, E=20),
    "relu_k1": lambda: _workload("switch_bf16", T=40, d=512, F=1024, mwq=True),
    "shared_experts": lambda: _workload("deepseek_v2_lite_bf16", T=48, d=512, F=512, E=16, k=4,
                                        F_shared=256, mwq=True),
}


@pytest.mark.parametrize("case", list(SMALL))
def test_mwq_layer_parity_small(case):
    _say("mwq layer %s" % case)
    wl = SMALL[case]()
    g = run_mwq_layer(wl)
    check_mwq(wl, g)


@pytest.mark.parametrize("width", [2, 3, 4])
def test_mwq_layer_one_width(width):
    """All assignments at one width: one table and one accumulator per pass."""
    _say("mwq layer one width %d" % width)
    wl = _with_widths(_small(T=32), lambda b: np.full_like(b, width))
    g = run_mwq_layer(wl)
    check_mwq(wl, g)
    E = wl.cfg.E
    assert np.array_equal(g["mwq_counts"].reshape(E, 3)[:, width - 2], g["counts"])


def test_mwq_layer_full_size():
    """Mixtral-shaped nested experts, a 16-token decode step, every token checked."""
    _say("mwq layer full-size mixtral_mwq_decode")
    wl = _workload("mixtral_mwq_decode")
    g = run_mwq_layer(wl)
    check_mwq(wl, g)
