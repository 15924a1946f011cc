"""MI355X (gfx950) sparse Mixture-of-Experts layer forward.

The layer runs in hand-written HIP kernels behind the C ABI of include/moe.h
(libmoe.so, built in-tree by ``build.py``).  This package is the thin Python
binding: torch supplies device memory and the HIP stream.
"""
from ._binding import (MOE_ACT_RELU, MOE_ACT_SWIGLU, MOE_DT_BF16, MOE_DT_F32,  # noqa: F401
                       MOE_F_BF16_ROWS, MOE_F_LOGITS_GIVEN, MOE_F_NONDETERMINISTIC_COMBINE,
                       MOE_F_VALIDATE_ONLY, MoeError, lib)
from .api import (AtomicLayer, AtomicRunner, ExpertWeights, FloeExperts,  # noqa: F401
                  Int4Proj, LayerRunner, MoeLayer, MoeReplica, MwqExperts, MwqProj,
                  atomic_layer_forward, combine, grouped_ffn, grouped_ffn_mwq, layer_forward,
                  mwq_group, permute, replica_split, route_topk)
