"""moe_layer_forward_noalloc (the layer with the library's static device array
as workspace) against moe_layer_forward with a caller workspace.

Both run the same kernels on the same inputs, so every output -- routing
integers, LIS, gates, logits and y -- must agree bit for bit.  Two calls in a
row, the second with fewer tokens, check that the array's leftover contents
from the first call do not leak into the second.
"""
import pytest

from workloads import get_config, make_workload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_mixture_experts_wavefront_amd as moe
    moe.lib()


AUX = ("logits", "idx", "gates", "counts", "offsets", "row_assign", "assign_row", "lis")


def _aux(T, E, k, dev):
    return dict(logits=torch.empty(T, E, dtype=torch.float32, device=dev),
                idx=torch.empty(T, k, dtype=torch.int32, device=dev),
                gates=torch.empty(T, k, dtype=torch.float32, device=dev),
                counts=torch.empty(E, dtype=torch.int32, device=dev),
                offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
                row_assign=torch.empty(T * k, dtype=torch.int32, device=dev),
                assign_row=torch.empty(T * k, dtype=torch.int32, device=dev),
                lis=torch.empty(1, dtype=torch.float64, device=dev))


def _run_both(layer, x, out_dtype):
    from sparse_mixture_experts_wavefront_amd import api
    T = x.shape[0]
    E, k, d = layer.n_experts, layer.top_k, layer.d_model
    y_ref, aux_ref = api.layer_forward(layer, x, out_dtype=out_dtype)
    aux = _aux(T, E, k, x.device)
    y = torch.full((T, d), float("nan"), dtype=out_dtype, device=x.device)
    api.layer_forward_noalloc(layer, x, y, aux=aux)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref), "y differs"
    for n in AUX:
        a, b = aux[n], aux_ref[n]
        if n in ("row_assign", "assign_row"):
            b = b[:T * k]
        assert torch.equal(a, b), n
    return y


@pytest.mark.parametrize("name,over,t2", [
    ("mixtral_decode_bf16", dict(T=16, d=1024, F=2048, x_rows_of=None, weights_of=None), 7),
    ("mixtral_int4_decode", dict(T=64, d=1024, F=2048, x_rows_of=None, weights_of=None), 9),
    ("deepseek_v2_lite_bf16", dict(T=96, d=512, F=256, F_shared=256), 33),
    ("tiny_fp32", dict(), 20),
])
def test_noalloc_matches_layer_forward(name, over, t2):
    from sparse_mixture_experts_wavefront_amd.device_inputs import to_device
    print("\n[case] noalloc %s %s then T=%d" % (name, over, t2), flush=True)
    wl = make_workload(get_config(name, **over))
    layer, x = to_device(wl)
    _run_both(layer, x, torch.float32)
    # second call, fewer tokens: the array still holds the first call's values
    _run_both(layer, x[:t2].contiguous(), torch.float32)
    if wl.cfg.dtype == "bf16":
        _run_both(layer, x[:t2].contiguous(), torch.bfloat16)


def test_noalloc_rejects_oversized_calls():
    import sparse_mixture_experts_wavefront_amd as moe
    from sparse_mixture_experts_wavefront_amd import _binding as B
    from sparse_mixture_experts_wavefront_amd import api
    from sparse_mixture_experts_wavefront_amd.device_inputs import to_device
    wl = make_workload(get_config("mixtral_decode_bf16", T=16, d=1024, F=2048, x_rows_of=None,
                                  weights_of=None))
    layer, x = to_device(wl)
    cap = api.noalloc_scratch_bytes()
    assert cap == 64 << 20
    # the largest T whose workspace fits, and one past it (x rows repeated:
    # nothing runs for the rejected call, the accepted one just has to match)
    T = 16
    while layer.workspace_size(T * 2) <= cap:
        T *= 2
    lo, hi = T, T * 2
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if layer.workspace_size(mid) <= cap:
            lo = mid
        else:
            hi = mid
    big = x.repeat((hi + 15) // 16, 1)[:hi].contiguous()
    y = torch.empty(hi, layer.d_model, dtype=torch.float32, device=x.device)
    with pytest.raises(B.MoeError) as ei:
        api.layer_forward_noalloc(layer, big, y)
    assert ei.value.status == B.MOE_ERR_WORKSPACE
    assert b"static" in moe.lib().moe_last_error()
    # the largest accepted size runs and matches the workspace call
    _run_both(layer, big[:lo].contiguous(), torch.float32)
