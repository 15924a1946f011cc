"""The layer under HIP graph capture.

moe_layer_forward enqueues kernels only (no host synchronisation, no memset
or copy nodes, no allocation), so a caller can capture one call in a graph
and replay it.  Each case runs the layer eagerly on two inputs, captures one
call, then replays the graph several times with the program's own eager work
and synchronisations between the replays, changing the captured input buffer
in place, and checks every replay bit for bit against the eager output for
the input it held (the kernels are deterministic, so equal inputs give equal
bits).
"""
import functools

import numpy as np
import pytest

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


CASES = {
    # weight streaming (bf16), k = 2: down pass adds into y directly
    "decode": ("mixtral_decode_bf16", dict(T=16, d=512, F=1024, x_rows_of=None, weights_of=None)),
    # INT4 row-split kernels, split router GEMM, down K parts + combine
    "int4_decode": ("mixtral_int4_decode", dict(T=64, d=512, F=1024, x_rows_of=None,
                                                weights_of=None)),
    # tiled path, k = 1, two down K slices + combine
    "switch": ("switch_bf16", dict(T=300, d=256, F=384)),
    # tiled path, top-6 of 64 with shared experts, multi-block permutation
    "deepseek": ("deepseek_v2_lite_bf16", dict(T=600, d=256, F=192, F_shared=64)),
    # fp32 layer
    "tiny_fp32": ("tiny_fp32", {}),
}


def _second_input(x, seed):
    """A different input of the same shape and dtype (a seeded permutation of
    x's rows, sign-flipped), so the routing and the output change."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    perm = torch.randperm(x.shape[0], generator=g).to(x.device)
    return (-x[perm]).contiguous()


@pytest.mark.parametrize("case", list(CASES))
def test_layer_graph_replay_matches_eager(case):
    import sparse_mixture_experts_wavefront_amd as moe
    from sparse_mixture_experts_wavefront_amd.device_inputs import to_device
    name, over = CASES[case]
    _say("graph replay %s" % case)
    wl = _workload(name, **over)
    layer, x = to_device(wl)
    x2 = _second_input(x, 7)
    runner = moe.LayerRunner(layer, wl.cfg.T)
    ref = {}
    for tag, xi in (("a", x), ("b", x2)):
        runner(xi)
        torch.cuda.synchronize()
        ref[tag] = runner.y.clone()
    assert not torch.equal(ref["a"], ref["b"])

    xin = x.clone()  # the buffer the graph reads
    runner(xin)      # warm-up on the capture buffers before capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        runner(xin)
    torch.cuda.synchronize()

    other = moe.LayerRunner(layer, wl.cfg.T)  # eager work between the replays
    for rep, tag in enumerate(["a", "b", "a", "b"]):
        xin.copy_(x if tag == "a" else x2)
        graph.replay()
        other(x2 if tag == "a" else x)
        torch.cuda.synchronize()
        got = runner.y.clone()
        assert torch.equal(got, ref[tag]), "replay %d (%s): max-abs %g" % (
            rep, tag, (got - ref[tag]).abs().max().item())
        assert torch.equal(other.y, ref["b" if tag == "a" else "a"])
