"""Parity of the atomic-expert layer (moe_atomic_layer_forward) with the CPU oracle.

The selection over the router grid is decided on fp32 scores, so the oracle
selects on the GPU's row and column log-probabilities (checked against its own
fp64 ones); then the kept experts, their counts, offsets, the expert-major
permutation and LIS must match bit for bit, gates within 2e-6, and y within
max-abs 2e-2 and relative L2 1e-2.
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
def _workload(**over):
    return make_workload(get_config("omni_atomic", **over))


def run_atomic(wl, schedule="auto", layouts=("dense", "rows")):
    import sparse_mixture_experts_wavefront_amd as moe
    from sparse_mixture_experts_wavefront_amd.device_inputs import atomic_to_device
    layer, x = atomic_to_device(wl, schedule=schedule, layouts=layouts)
    y, aux = moe.atomic_layer_forward(layer, x)
    torch.cuda.synchronize()
    g = {n: t.cpu().numpy() for n, t in aux.items()}
    n = wl.cfg.T * wl.cfg.k
    g["row_assign"], g["assign_row"] = g["row_assign"][:n], g["assign_row"][:n]
    g["lis"] = float(g["lis"][0])
    g["y"] = y.cpu().numpy()
    return g


def check_atomic(wl, g, tokens=None, full_routing=True, ref=None):
    if ref is None:
        ref = oracle.atomic_layer_forward(wl, pr=g["logp_row"], pc=g["logp_col"], tokens=tokens)
    for a, b in (("logp_row", "pr"), ("logp_col", "pc")):
        dlp = np.abs(g[a].astype(np.float64) - ref[b].astype(np.float64)).max()
        assert dlp <= 1e-4, (a, dlp)
    assert np.array_equal(g["idx"], ref["idx"])
    assert np.allclose(g["gates"], ref["gate"], rtol=2e-5, atol=2e-6)
    if full_routing:
        for n in ("counts", "offsets", "row_assign", "assign_row"):
            assert np.array_equal(g[n], ref[n]), n
        assert g["lis"] == ref["lis"]
    gy = g["y"] if tokens is None else g["y"][np.asarray(tokens)]
    ry = ref["y"].astype(np.float64)
    d = np.abs(gy.astype(np.float64) - ry)
    rel = np.linalg.norm(gy.astype(np.float64) - ry) / max(np.linalg.norm(ry), 1e-30)
    print("  LIS %.3f; y max-abs %.3e rel-L2 %.3e" % (g["lis"], d.max(), rel), flush=True)
    assert d.max() <= 2e-2, "y max-abs %g" % d.max()
    assert rel <= 1e-2, "y rel-L2 %g" % rel


SMALL = {
    "small": dict(T=48, d=256, nr=8, nc=32, E=256, k=16, F_shared=128),
    "one_token": dict(T=1, d=256, nr=8, nc=32, E=256, k=16, F_shared=128),
    "top1": dict(T=40, d=256, nr=8, nc=32, E=256, k=1, n_shared=0),
    "all_cells": dict(T=20, d=256, nr=4, nc=32, E=128, k=128, F_shared=128),
    "ragged": dict(T=300, d=384, nr=20, nc=64, E=1280, k=100, F_shared=256),
    # 96 x 256 cells per tile, 3/4 kept: more kept cells than a tile lists in
    # LDS, so the input GEMM takes its dense-tile path
    "dense_tiles": dict(T=96, d=256, nr=8, nc=32, E=256, k=192, F_shared=128),
    # N = 384: the last column tile of the input GEMM is half outside the grid
    "odd_width": dict(T=300, d=256, nr=12, nc=32, E=384, k=40, F_shared=128),
    # the largest grid (1024 x 1024 = 1,048,576 experts): sort of 1024 column
    # scores, 4 rows per thread, 32768 bitmap words per token
    "max_grid": dict(T=3, d=128, nr=1024, nc=1024, E=1024 * 1024, k=4096, F_shared=128),
}


@pytest.mark.parametrize("case", list(SMALL))
def test_atomic_layer_parity_small(case):
    _say("atomic layer %s %s" % (case, SMALL[case]))
    wl = _workload(**SMALL[case])
    g = run_atomic(wl, schedule="dense")
    check_atomic(wl, g)


# expert-centric schedule: d a multiple of 512 (one to eight 512-wide chunks per
# lane); T > 16 exercises the token chunks of the output side, T = 1 and top-1
# leave most experts without rows
EC_SMALL = {
    "ec_small": dict(T=48, d=512, nr=8, nc=32, E=256, k=16, F_shared=128),
    "ec_one_token": dict(T=1, d=512, nr=8, nc=32, E=256, k=16, F_shared=128),
    "ec_top1": dict(T=40, d=1024, nr=8, nc=32, E=256, k=1, n_shared=0),
    "ec_all_cells": dict(T=20, d=512, nr=4, nc=32, E=128, k=128, F_shared=128),
    "ec_ragged": dict(T=300, d=1024, nr=20, nc=64, E=1280, k=100, F_shared=256),
    "ec_wide": dict(T=17, d=4096, nr=8, nc=32, E=256, k=24, F_shared=128),
    "ec_sixteen": dict(T=16, d=2048, nr=12, nc=32, E=384, k=40, F_shared=128),
    # 16 tokens x 64 units = 1024 rows in one 256-unit range: more than a round
    # stages in LDS, so the output side reads rows and tokens from memory
    "ec_unstaged": dict(T=16, d=512, nr=8, nc=32, E=256, k=64, F_shared=128),
}


@pytest.mark.parametrize("case", list(EC_SMALL))
def test_atomic_layer_expert_centric_small(case):
    _say("atomic layer expert-centric %s %s" % (case, EC_SMALL[case]))
    wl = _workload(**EC_SMALL[case])
    g = run_atomic(wl, schedule="expert_centric", layouts=("rows",))
    ref = oracle.atomic_layer_forward(wl, pr=g["logp_row"], pc=g["logp_col"])
    check_atomic(wl, g, ref=ref)
    # the dense schedule on the same inputs: the same routing, y within tolerance
    gd = run_atomic(wl, schedule="dense", layouts=("dense",))
    for n in ("idx", "counts", "offsets", "row_assign", "assign_row"):
        assert np.array_equal(gd[n], g[n]), n
    check_atomic(wl, gd, ref=ref)


def test_atomic_auto_schedule_picks_by_tokens():
    """auto: expert-centric up to 64 tokens when w_out_rows is given, dense above;
    either layout alone forces its schedule; the results agree with the oracle."""
    _say("atomic auto schedule")
    base = dict(d=512, nr=8, nc=32, E=256, k=16, F_shared=128)
    for T, layouts in ((64, ("dense", "rows")), (65, ("dense", "rows")), (65, ("rows",)),
                       (30, ("dense",))):
        wl = _workload(T=T, **base)
        g = run_atomic(wl, schedule="auto", layouts=layouts)
        check_atomic(wl, g)


def test_atomic_layer_tied_scores():
    """Router weights of zero: every cell scores the same, the lowest K ids win."""
    _say("atomic layer tied scores")
    import dataclasses
    wl = dataclasses.replace(_workload(**SMALL["small"]))
    wl.w_router = np.zeros_like(wl.w_router)
    wl.w_col = np.zeros_like(wl.w_col)
    g = run_atomic(wl)
    assert np.array_equal(g["idx"], np.tile(np.arange(16), (48, 1)))
    check_atomic(wl, g)


def test_atomic_layer_full_size():
    """102,400 atomic experts, top-4096, 4096 tokens: routing, permutation and y
    on every token."""
    _say("atomic layer full-size omni_atomic")
    wl = make_workload("omni_atomic")
    g = run_atomic(wl)
    ref = oracle.atomic_layer_forward(wl, pr=g["logp_row"], pc=g["logp_col"])
    assert np.array_equal(g["idx"], ref["idx"])
    for n in ("counts", "offsets", "row_assign", "assign_row"):
        assert np.array_equal(g[n], ref[n]), n
    assert g["lis"] == ref["lis"]
    gy = g["y"].astype(np.float64)
    ry = ref["y"].astype(np.float64)
    d = np.abs(gy - ry)
    rel = np.linalg.norm(gy - ry) / np.linalg.norm(ry)
    print("  LIS %.3f; y max-abs %.3e rel-L2 %.3e" % (g["lis"], d.max(), rel), flush=True)
    assert d.max() <= 2e-2 and rel <= 1e-2
    # the expert-centric schedule at the same size (the bench times both)
    _say("atomic layer full-size omni_atomic, expert-centric")
    ge = run_atomic(wl, schedule="expert_centric", layouts=("rows",))
    for n in ("idx", "counts", "offsets", "row_assign", "assign_row"):
        assert np.array_equal(ge[n], g[n]), n
    check_atomic(wl, ge, ref=ref)


def test_atomic_layer_full_width_decode():
    """The full grid (102,400 experts, top-4096, d 2048) at 16 tokens, where the
    automatic schedule is expert-centric; every token checked."""
    _say("atomic layer full width, 16 tokens (expert-centric)")
    wl = make_workload(get_config("omni_atomic", T=16))
    g = run_atomic(wl, schedule="auto", layouts=("rows",))
    check_atomic(wl, g)
