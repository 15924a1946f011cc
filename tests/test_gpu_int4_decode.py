"""The INT4 weight decode inside the streaming FFN kernels, bit for bit.

Asymmetric group-wise INT4 (D^2MoE -- Figure 8: the low-bit weights are decoded
inside the GEMM kernel): W = bf16_RNE(fp32(fp32(q) - z) * s) per group of 128
along K.  Seen through the layer's output with tolerances, a decode that is off
by one bf16 ulp in a few weights would pass; here it cannot:

* token rows are one-hot, x_t = +-e_{k_t}, so every projection sum has a single
  non-zero term and returns one weight exactly;
* the down projection is an INT4 identity (q = 1 on the diagonal, scale 1,
  zero 0), so y_rows[t][n] = h[t][n] exactly for n < F;
* ReLU expert: h[t][f] = max(0, +-W_in[f][k_t]), a bf16 weight already;
* SwiGLU expert: the gate decodes to 30 everywhere (silu(30) == 30 in fp32) and
  h[t][f] = bf16_RNE(30 * W_up[f][k_t]), the product being exact in fp32.

The k_t cover all eight nibble positions of a word and many groups; the zero
points mix integers, fractions >= 2^-10 (the fused decode form) and tiny
fractions (the two-operation form), the latter confined to some blocks of rows
so that both forms run in one launch.  Expected values come from the oracle's
decode rule.
"""
import numpy as np
import pytest

import oracle

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


def _rand_int4(rng, N, K, tiny_rows):
    """Random INT4 words, fp16 scales of both signs over many binades, and zero
    points: integers 0..15, fractions >= 2^-10, and in rows `tiny_rows` also
    fractions below 2^-10 (for which fp32(q) - z is not exact)."""
    q = rng.integers(0, 2 ** 32, size=(N, K // 8), dtype=np.uint64).astype(np.uint32)
    G = K // 128
    mag = np.exp2(rng.uniform(-14, 3, size=(N, G))) * (1 + rng.random((N, G)))
    s = (mag * rng.choice([-1.0, 1.0], size=(N, G))).astype(np.float16)
    kind = rng.integers(0, 3, size=(N, G))
    z = np.where(kind == 0, rng.integers(0, 16, size=(N, G)).astype(np.float64),
                 np.where(kind == 1, rng.uniform(2.0 ** -10, 15.0, size=(N, G)), 0.0))
    tiny = np.zeros((N, G), bool)
    tiny[tiny_rows] = rng.random((len(tiny_rows), G)) < 0.5
    z = np.where(tiny, rng.uniform(1e-6, 2.0 ** -11, size=(N, G)), z).astype(np.float16)
    return q.view(np.int32), s.view(np.uint16), z.view(np.uint16)


def _identity_int4(N, K):
    """INT4 words of the [N][K] identity (q = 1 at k == n), scale 1, zero 0."""
    q = np.zeros((N, K // 8), np.uint32)
    n = np.arange(min(N, K))
    q[n, n // 8] = np.uint32(1) << (4 * (n % 8)).astype(np.uint32)
    G = K // 128
    s = np.full((N, G), 1.0, np.float16)
    z = np.zeros((N, G), np.float16)
    return q.view(np.int32), s.view(np.uint16), z.view(np.uint16)


def _bf16_to_f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _f32_to_bf16_rne(v):
    b = np.ascontiguousarray(v, np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def _proj(moe, q, s, z):
    dev = "cuda"
    return moe.Int4Proj(torch.from_numpy(q[None].copy()).to(dev),
                        torch.from_numpy(s[None].copy()).view(torch.float16).to(dev),
                        torch.from_numpy(z[None].copy()).view(torch.float16).to(dev))


def _one_hot(T, d, ks, signs):
    x = np.zeros((T, d), np.float32)
    x[np.arange(T), ks] = signs
    return torch.from_numpy(x).to(torch.bfloat16).cuda()


@pytest.mark.parametrize("T,d,F", [(64, 2048, 512), (16, 1024, 512), (37, 1536, 512)])
def test_relu_int4_decode_bit_exact(T, d, F):
    _say("int4 decode bit-exact, ReLU expert, T=%d d=%d F=%d" % (T, d, F))
    import sparse_mixture_experts_wavefront_amd as moe
    rng = np.random.default_rng(1000 + T)
    # blocks of 64 W_in rows: the first half of the blocks get tiny zero points
    tiny_rows = [r for r in range(F) if (r // 64) % 2 == 0]
    qi, si, zi = _rand_int4(rng, F, d, tiny_rows)
    qd, sd, zd = _identity_int4(d, F)
    ks = (np.arange(T) * 37 + 5) % d               # k mod 8 runs through all 8 nibbles
    signs = np.where(np.arange(T) % 2 == 0, 1.0, -1.0)
    ex = moe.ExpertWeights(q_up=_proj(moe, qi, si, zi), q_down=_proj(moe, qd, sd, zd))
    y = moe.grouped_ffn(_one_hot(T, d, ks, signs), 1, 1, "relu", ex, d_ff=F)
    torch.cuda.synchronize()
    W = _bf16_to_f32(oracle.dequant_int4(qi, si, zi))          # [F][d]
    h = np.maximum(W[:, ks].T * signs[:, None], 0.0).astype(np.float32)
    want = np.zeros((T, d), np.float32)
    want[:, :F] = h                                            # (d >= F here)
    got = y.cpu().numpy()
    bad = np.argwhere(got != want)
    assert bad.size == 0, "first mismatches (t, n): %s" % bad[:5].tolist()


@pytest.mark.parametrize("T,d,F", [(64, 2048, 512), (20, 1024, 1024)])
def test_swiglu_int4_decode_bit_exact(T, d, F):
    _say("int4 decode bit-exact, SwiGLU expert, T=%d d=%d F=%d" % (T, d, F))
    import sparse_mixture_experts_wavefront_amd as moe
    rng = np.random.default_rng(2000 + T)
    tiny_rows = [r for r in range(F) if (r // 64) % 2 == 1]
    qu, su, zu = _rand_int4(rng, F, d, tiny_rows)
    G = d // 128
    # gate: q = 15 everywhere, scale 2, zero 0 -> 30
    qg = np.full((F, d // 8), -1, np.int32)
    sg = np.full((F, G), 2.0, np.float16).view(np.uint16)
    zg = np.zeros((F, G), np.float16).view(np.uint16)
    qd, sd, zd = _identity_int4(d, F)
    ks = (np.arange(T) * 53 + 3) % d
    ex = moe.ExpertWeights(q_gate=_proj(moe, qg, sg, zg), q_up=_proj(moe, qu, su, zu),
                           q_down=_proj(moe, qd, sd, zd))
    y = moe.grouped_ffn(_one_hot(T, d, ks, np.ones(T)), 1, 1, "swiglu", ex, d_ff=F)
    torch.cuda.synchronize()
    Wu = _bf16_to_f32(oracle.dequant_int4(qu, su, zu))
    h = _bf16_to_f32(_f32_to_bf16_rne(np.float32(30.0) * Wu[:, ks].T))
    want = np.zeros((T, d), np.float32)
    want[:, :F] = h                                            # (d >= F here)
    got = y.cpu().numpy()
    bad = np.argwhere(got != want)
    assert bad.size == 0, "first mismatches (t, n): %s" % bad[:5].tolist()
