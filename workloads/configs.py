"""The seven synthetic workloads of the sparse MoE layer forward.

Shapes follow the model families the pages measure on: a Switch-Transformer-like
top-1 ReLU layer, a Mixtral-8x7B-shaped top-2 SwiGLU layer (decode and prefill),
a DeepSeek-V2-Lite-shaped layer with 64 fine-grained routed experts plus two
always-active shared experts, and a Mixtral-shaped decode with asymmetric INT4
expert weights (group 128 along K, fp16 scale and zero point, 8 nibbles per
int32), and the same decode with nested INT2-to-INT4 weights and a bit width
per assignment.  The pages print no d_model or d_ff; these sizes are those of
the published model families.

Router-bias constants ``beta`` were found by ``oracle/tune_router_bias.py``
(it calls only the oracle) so that the Load Imbalance Score of the routed
assignment lands near the values the Replicate-and-Quantize page reports for
raw routing (about 2 for an 8-expert Switch layer and about 4 for
DeepSeek-V2-Lite; that page, "Core claim").
"""
from dataclasses import dataclass, field
from typing import Optional


@dataclass(frozen=True)
class WorkloadConfig:
    name: str
    cfg_id: int          # first word of every tensor's SeedSequence
    T: int               # tokens in this call
    d: int               # d_model
    E: int               # routed experts
    k: int               # top-k
    F: int               # routed expert d_ff
    act: str             # "swiglu" | "relu"
    dtype: str           # activation / weight dtype: "f32" | "bf16"
    n_shared: int = 0    # always-active shared experts
    F_shared: int = 0    # d_ff of each shared expert
    bias: str = "zero"   # router-bias recipe: "zero" | "log_inv" | "neg_log" | "zipf"
    beta: float = 0.0    # bias strength for "neg_log" / "zipf"
    int4: bool = False   # expert weights as asymmetric INT4, group 128 along K
    mwq: bool = False    # nested INT2 + binary residual planes, per-assignment bit width
    floe: bool = False   # INT2 up projection, gate/down channels kept where |up| > threshold
    sparsity: float = 0.0  # target fraction of pruned channels (floe thresholds)
    atomic: bool = False   # atomic experts on an nr x nc router grid: E = nr*nc, k = K
    nr: int = 0
    nc: int = 0
    x_rows_of: Optional[str] = None   # take the first T rows of this workload's x
    weights_of: Optional[str] = None  # reuse this workload's router/expert weights
    notes: str = field(default="", compare=False)


CONFIGS = {
    "tiny_fp32": WorkloadConfig(
        "tiny_fp32", 0, T=64, d=128, E=8, k=2, F=256, act="swiglu", dtype="f32",
        bias="log_inv",
        notes="b_e = 0.5*ln(1/(e+1)), e 0-based"),
    "switch_bf16": WorkloadConfig(
        "switch_bf16", 1, T=4096, d=768, E=8, k=1, F=3072, act="relu", dtype="bf16",
        bias="neg_log", beta=0.204,
        notes="b_e = -beta*ln(e+1), beta tuned so LIS ~ 2"),
    "mixtral_decode_bf16": WorkloadConfig(
        "mixtral_decode_bf16", 2, T=16, d=4096, E=8, k=2, F=14336, act="swiglu",
        dtype="bf16", x_rows_of="mixtral_prefill_bf16",
        weights_of="mixtral_prefill_bf16"),
    "mixtral_prefill_bf16": WorkloadConfig(
        "mixtral_prefill_bf16", 2, T=4096, d=4096, E=8, k=2, F=14336, act="swiglu",
        dtype="bf16"),
    "deepseek_v2_lite_bf16": WorkloadConfig(
        "deepseek_v2_lite_bf16", 3, T=8192, d=2048, E=64, k=6, F=1408, act="swiglu",
        dtype="bf16", n_shared=2, F_shared=1408, bias="zipf", beta=0.269,
        notes="b_e = -1.1*beta*ln(r_e), r_e a seeded rank 1..64, beta tuned so LIS ~ 4"),
    "mixtral_int4_decode": WorkloadConfig(
        "mixtral_int4_decode", 4, T=64, d=4096, E=8, k=2, F=14336, act="swiglu",
        dtype="bf16", int4=True, x_rows_of="mixtral_prefill_bf16",
        weights_of="mixtral_prefill_bf16"),
    "mixtral_mwq_decode": WorkloadConfig(
        "mixtral_mwq_decode", 5, T=16, d=4096, E=8, k=2, F=14336, act="swiglu",
        dtype="bf16", mwq=True, x_rows_of="mixtral_prefill_bf16",
        weights_of="mixtral_prefill_bf16",
        notes="nested INT2 base + binary residual planes, bit width per assignment "
              "uniform over {2, 3, 4}"),
    "omni_atomic": WorkloadConfig(
        "omni_atomic", 7, T=4096, d=2048, E=320 * 320, k=4096, F=1, act="silu", dtype="bf16",
        atomic=True, nr=320, nc=320, n_shared=1, F_shared=1536,
        notes="102,400 atomic experts on a 320 x 320 router grid, top-4096 per token, "
              "SiLU units, one shared SwiGLU MLP (d_ff 1536)"),
    "omni_atomic_decode": WorkloadConfig(
        "omni_atomic_decode", 7, T=16, d=2048, E=320 * 320, k=4096, F=1, act="silu",
        dtype="bf16", atomic=True, nr=320, nc=320, n_shared=1, F_shared=1536,
        notes="the atomic-expert layer above at 16 tokens (a decode step): only the "
              "experts some token keeps need their parameters read"),
    "mixtral_floe_decode": WorkloadConfig(
        "mixtral_floe_decode", 6, T=16, d=4096, E=8, k=2, F=14336, act="swiglu",
        dtype="bf16", floe=True, sparsity=0.9, x_rows_of="mixtral_prefill_bf16",
        weights_of="mixtral_prefill_bf16",
        notes="INT2 up projection; per-expert thresholds for 90% pruned up outputs, "
              "calibrated on 64 seeded tokens"),
    "mixtral_floe_decode_t1": WorkloadConfig(
        "mixtral_floe_decode_t1", 6, T=1, d=4096, E=8, k=2, F=14336, act="swiglu",
        dtype="bf16", floe=True, sparsity=0.9, x_rows_of="mixtral_prefill_bf16",
        weights_of="mixtral_prefill_bf16", notes="one-token decode step"),
}


def get_config(name: str, **overrides) -> WorkloadConfig:
    """Return a named config, optionally with fields replaced (e.g. a smaller T)."""
    import dataclasses
    c = CONFIGS[name]
    return dataclasses.replace(c, **overrides) if overrides else c
