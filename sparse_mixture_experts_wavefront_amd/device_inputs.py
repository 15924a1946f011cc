"""Upload a seeded workload (numpy, from ``workloads``) to device tensors."""
from __future__ import annotations

import numpy as np
import torch

from .api import (AtomicLayer, ExpertWeights, FloeExperts, Int4Proj, MoeLayer, MoeReplica, MwqExperts,
                  MwqProj)


def _t(a: np.ndarray, dev, bf16: bool):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if bf16:
        t = t.view(torch.bfloat16)
    return t.to(dev)


def _q(qw, dev):
    return Int4Proj(torch.from_numpy(np.ascontiguousarray(qw.q)).to(dev),
                    torch.from_numpy(np.ascontiguousarray(qw.scale)).view(torch.float16).to(dev),
                    torch.from_numpy(np.ascontiguousarray(qw.zero)).view(torch.float16).to(dev))


def to_device(wl, device="cuda"):
    """Returns (MoeLayer, x) for a ``workloads.Workload``."""
    cfg = wl.cfg
    bf = cfg.dtype == "bf16"
    if cfg.mwq or cfg.floe:
        routed = ExpertWeights()   # nested or sparse-down experts: see mwq_to_device, floe_to_device
    elif cfg.int4:
        routed = ExpertWeights(q_gate=None if wl.q_gate is None else _q(wl.q_gate, device),
                               q_up=_q(wl.q_up, device), q_down=_q(wl.q_down, device))
    else:
        routed = ExpertWeights(
            w_gate=None if wl.w_gate is None else _t(wl.w_gate, device, bf),
            w_up=_t(wl.w_up, device, bf), w_down=_t(wl.w_down, device, bf))
    shared = None
    if cfg.n_shared:
        shared = ExpertWeights(w_gate=_t(wl.ws_gate, device, bf), w_up=_t(wl.ws_up, device, bf),
                               w_down=_t(wl.ws_down, device, bf))
    layer = MoeLayer(cfg.d, cfg.F, cfg.E, cfg.k, cfg.act, _t(wl.w_router, device, bf),
                     torch.from_numpy(wl.b_router).to(device), routed, cfg.n_shared,
                     cfg.F_shared, shared)
    return layer, _t(wl.x, device, bf)


def replica_to_device(rep, device="cuda"):
    """MoeReplica for a ``workloads.Replica`` (INT4, one expert per projection)."""
    return MoeReplica(rep.heavy, _q(rep.q_up, device), _q(rep.q_down, device),
                      None if rep.q_gate is None else _q(rep.q_gate, device))


def _m(mw, dev):
    f16 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).view(torch.float16).to(dev)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return MwqProj(i32(mw.q2), f16(mw.s2), f16(mw.z2), i32(mw.p3), f16(mw.a3), i32(mw.p4),
                   f16(mw.a4))


def mwq_to_device(wl, device="cuda"):
    """(MwqExperts, widths [T][k] int32) for a nested-expert ``workloads.Workload``."""
    ex = MwqExperts(_m(wl.m_up, device), _m(wl.m_down, device),
                    None if wl.m_gate is None else _m(wl.m_gate, device))
    widths = torch.from_numpy(np.ascontiguousarray(wl.bits, dtype=np.int32)).to(device)
    return ex, widths


def floe_to_device(wl, device="cuda"):
    """FloeExperts for a sparse-down ``workloads.Workload`` (W_down transposed on
    the device to channel-major [E][F][d])."""
    f16 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).view(torch.float16).to(device)
    wd = _t(wl.w_down, device, True)
    return FloeExperts(torch.from_numpy(np.ascontiguousarray(wl.u2_up.q2)).to(device),
                       f16(wl.u2_up.s2), f16(wl.u2_up.z2), _t(wl.w_gate, device, True),
                       wd.transpose(1, 2).contiguous(),
                       torch.from_numpy(np.ascontiguousarray(wl.floe_thr)).to(device))


def atomic_to_device(wl, device="cuda", schedule="auto", layouts=("dense", "rows")):
    """(AtomicLayer, x) for an atomic-expert ``workloads.Workload``; ``layouts``
    picks which copies of the output vectors go to the device: "dense" (w_out
    [d][N]) and/or "rows" (w_out_rows [N][d])."""
    cfg = wl.cfg
    shared = None
    if cfg.n_shared:
        shared = ExpertWeights(w_gate=_t(wl.ws_gate, device, True), w_up=_t(wl.ws_up, device, True),
                               w_down=_t(wl.ws_down, device, True))
    layer = AtomicLayer(cfg.d, cfg.nr, cfg.nc, cfg.k, _t(wl.w_router, device, True),
                        _t(wl.w_col, device, True), _t(wl.w_in, device, True),
                        _t(wl.w_out_t, device, True) if "dense" in layouts else None,
                        cfg.n_shared, cfg.F_shared, shared,
                        w_out_rows=_t(wl.w_out_rows, device, True) if "rows" in layouts else None,
                        schedule=schedule)
    return layer, _t(wl.x, device, True)
