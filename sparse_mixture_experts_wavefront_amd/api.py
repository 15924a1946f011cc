"""Python face of the MoE layer forward: the five C-ABI calls on torch tensors.

Torch provides device memory and the current HIP stream; all arithmetic runs in
libmoe.so.  Function names match the C entry points without the ``moe_`` prefix.
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass, field
from typing import Optional

import torch

from . import _binding as B


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return B.MOE_DT_BF16
    if t.dtype == torch.float32:
        return B.MOE_DT_F32
    raise TypeError("unsupported dtype %s" % t.dtype)


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return C.c_void_p(t.data_ptr())


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ws(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


@dataclass
class Int4Proj:
    """One projection's group-wise INT4 weights (all experts)."""
    q: torch.Tensor       # int32 [E][N][K/8]
    scale: torch.Tensor   # fp16 [E][N][K/128]
    zero: torch.Tensor    # fp16 [E][N][K/128]

    def struct(self):
        return B.W4(_p(self.q), _p(self.scale), _p(self.zero))


@dataclass
class ExpertWeights:
    """Dense (bf16/fp32) or INT4 expert weights.  Dense: w_gate/w_up [E][F][d], w_down [E][d][F]."""
    w_gate: Optional[torch.Tensor] = None
    w_up: Optional[torch.Tensor] = None
    w_down: Optional[torch.Tensor] = None
    q_gate: Optional[Int4Proj] = None
    q_up: Optional[Int4Proj] = None
    q_down: Optional[Int4Proj] = None
    _keep: list = field(default_factory=list, repr=False)

    def struct(self, dtype: int) -> B.Experts:
        e = B.Experts()
        e.dtype = dtype
        e.w_gate, e.w_up, e.w_down = _p(self.w_gate), _p(self.w_up), _p(self.w_down)
        self._keep = []
        for name in ("q_gate", "q_up", "q_down"):
            q = getattr(self, name)
            if q is not None:
                s = q.struct()
                self._keep.append(s)
                setattr(e, name, C.pointer(s))
        return e


@dataclass
class MoeLayer:
    """Device-resident weights of one MoE layer and its shape."""
    d_model: int
    d_ff: int
    n_experts: int
    top_k: int
    act: str                      # "swiglu" | "relu"
    w_router: torch.Tensor        # [E][d] in the activation dtype
    b_router: Optional[torch.Tensor]
    routed: ExpertWeights
    n_shared: int = 0
    d_ff_shared: int = 0
    shared: Optional[ExpertWeights] = None

    @property
    def act_code(self):
        return B.MOE_ACT_SWIGLU if self.act == "swiglu" else B.MOE_ACT_RELU

    def desc(self) -> B.LayerDesc:
        dt = _dt(self.w_router)
        L = B.LayerDesc()
        L.d_model, L.d_ff, L.n_experts, L.top_k = self.d_model, self.d_ff, self.n_experts, self.top_k
        L.act, L.act_dtype = self.act_code, dt
        L.w_router, L.b_router = _p(self.w_router), _p(self.b_router)
        L.routed = self.routed.struct(dt)
        L.n_shared, L.d_ff_shared = self.n_shared, self.d_ff_shared
        if self.shared is not None:
            L.shared = self.shared.struct(dt)
        return L

    def workspace_size(self, T: int) -> int:
        n = C.c_size_t(0)
        L = self.desc()
        B.check(B.lib().moe_workspace_size(C.byref(L), T, C.byref(n)), "moe_workspace_size")
        return n.value


@dataclass
class MoeReplica:
    """INT4 copy of routed expert ``expert`` (one expert per projection), run as slot E."""
    expert: int
    q_up: Int4Proj
    q_down: Int4Proj
    q_gate: Optional[Int4Proj] = None
    _keep: list = field(default_factory=list, repr=False)

    def struct(self) -> B.Replica:
        r = B.Replica()
        r.expert = self.expert
        self._keep = []
        for name in ("q_gate", "q_up", "q_down"):
            q = getattr(self, name)
            if q is not None:
                st = q.struct()
                self._keep.append(st)
                setattr(r, name, C.pointer(st))
        return r


@dataclass
class MwqProj:
    """One projection's nested 2/3/4-bit weights (all experts), storage order of moe.h."""
    q2: torch.Tensor      # int32 [E][N][K/16]
    s2: torch.Tensor      # fp16 [E][N][K/128]
    z2: torch.Tensor
    p3: torch.Tensor      # int32 [E][N][K/32]
    a3: torch.Tensor      # fp16 [E][N][K/128]
    p4: torch.Tensor
    a4: torch.Tensor

    def struct(self):
        return B.WMwq(*[_p(getattr(self, n)) for n in ("q2", "s2", "z2", "p3", "a3", "p4", "a4")])


@dataclass
class MwqExperts:
    """Nested experts: gate/up with N = d_ff, down with N = d_model (gate None for ReLU)."""
    up: MwqProj
    down: MwqProj
    gate: Optional[MwqProj] = None
    _keep: list = field(default_factory=list, repr=False)

    def struct(self) -> B.MwqExperts:
        m = B.MwqExperts()
        self._keep = []
        for name in ("gate", "up", "down"):
            q = getattr(self, name)
            if q is not None:
                st = q.struct()
                self._keep.append(st)
                setattr(m, name, C.pointer(st))
        return m


@dataclass
class FloeExperts:
    """Sparse-down experts: INT2 up (q2, s2, z2 as in MwqProj), bf16 gate [E][F][d],
    bf16 W_down transposed [E][F][d], fp32 thresholds [E]."""
    q2: torch.Tensor
    s2: torch.Tensor
    z2: torch.Tensor
    w_gate: torch.Tensor
    w_down_t: torch.Tensor
    threshold: torch.Tensor
    _keep: list = field(default_factory=list, repr=False)

    def struct(self) -> B.FloeExperts:
        up = B.WMwq(_p(self.q2), _p(self.s2), _p(self.z2), None, None, None, None)
        self._keep = [up]
        return B.FloeExperts(C.pointer(up), _p(self.w_gate), _p(self.w_down_t),
                             _p(self.threshold))


# ---- the five calls -----------------------------------------------------------

def route_topk(x, w_router, b_router, k, logits=None, logits_given=False, flags=0):
    """Returns (logits [T][E] fp32, idx [T][k] int32, gate [T][k] fp32)."""
    dev = (logits if logits_given else x).device
    T = (logits if logits_given else x).shape[0]
    E = (logits.shape[1] if logits_given else w_router.shape[0])
    d = 8 if logits_given and x is None else x.shape[1]
    if logits is None:
        logits = torch.empty(T, E, dtype=torch.float32, device=dev)
    idx = torch.empty(T, k, dtype=torch.int32, device=dev)
    gate = torch.empty(T, k, dtype=torch.float32, device=dev)
    f = flags | (B.MOE_F_LOGITS_GIVEN if logits_given else 0)
    xdt = _dt(x) if x is not None else B.MOE_DT_BF16
    B.check(B.lib().moe_route_topk(_p(x), xdt, _p(w_router), _p(b_router), T, d, E, k,
                                   _p(logits), _p(idx), _p(gate), f, _stream()),
            "moe_route_topk")
    return logits, idx, gate


def permute(idx, E, flags=0):
    """Returns (counts [E], offsets [E+1], row_assign [T*k], assign_row [T*k], lis [1] fp64)."""
    T, k = idx.shape
    dev = idx.device
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    row_assign = torch.empty(max(T * k, 1), dtype=torch.int32, device=dev)
    assign_row = torch.empty(max(T * k, 1), dtype=torch.int32, device=dev)
    lis = torch.empty(1, dtype=torch.float64, device=dev)
    nws = B.lib().moe_permute_workspace_size(T, E, k)
    ws = _ws(nws, dev)
    B.check(B.lib().moe_permute(_p(idx), T, E, k, _p(counts), _p(offsets), _p(row_assign),
                                _p(assign_row), _p(lis), _p(ws), ws.numel(), flags, _stream()),
            "moe_permute")
    return counts, offsets, row_assign[:T * k], assign_row[:T * k], lis


def grouped_ffn(x, E, k, act, experts: ExpertWeights, offsets=None, row_assign=None,
                topk_gate=None, d_ff=None, flags=0):
    """Gate-scaled expert outputs y_rows [T*k][d] fp32 in expert-major row order."""
    T, d = x.shape
    F = d_ff if d_ff is not None else (experts.w_up.shape[-2] if experts.w_up is not None
                                       else experts.q_up.q.shape[-2])
    a = B.MOE_ACT_SWIGLU if act == "swiglu" else B.MOE_ACT_RELU
    st = experts.struct(_dt(x))
    y_rows = torch.empty(max(T * k, 1), d, dtype=torch.float32, device=x.device)
    nws = B.lib().moe_grouped_ffn_workspace_size(T, d, F, E, k, a, C.byref(st))
    ws = _ws(nws, x.device)
    B.check(B.lib().moe_grouped_ffn(_p(x), _dt(x), T, d, F, E, k, a, C.byref(st), _p(offsets),
                                    _p(row_assign), _p(topk_gate), _p(y_rows), _p(ws), ws.numel(),
                                    flags, _stream()),
            "moe_grouped_ffn")
    return y_rows[:T * k]


def combine(y_rows, assign_row, T, k, y_shared=None, out_dtype=torch.float32, flags=0):
    d = y_rows.shape[1]
    y = torch.empty(T, d, dtype=out_dtype, device=y_rows.device)
    B.check(B.lib().moe_combine(_p(y_rows), _p(assign_row), T, k, d, _p(y_shared), _p(y),
                                _dt(y), flags, _stream()),
            "moe_combine")
    return y


class LayerRunner:
    """Holds the descriptor, workspace and aux buffers for repeated layer calls.

    With ``replica`` the layer runs moe_layer_forward_replica: aux then holds
    the split routing over E+1 slots and ``lis_base`` the router's own LIS.
    With ``mwq`` (nested experts) it runs moe_layer_forward_mwq; each call then
    takes the widths [T][k] and aux also holds the (expert, width) grouping
    (mwq_idx, mwq_counts, mwq_offsets, mwq_row_assign, mwq_assign_row)."""

    def __init__(self, layer: MoeLayer, T: int, out_dtype=torch.float32, want_aux=True,
                 replica: Optional[MoeReplica] = None, mwq: Optional[MwqExperts] = None,
                 floe: Optional[FloeExperts] = None):
        self.layer = layer
        self.T = T
        dev = layer.w_router.device
        self.desc = layer.desc()
        self.replica = replica
        self.rep = None if replica is None else replica.struct()
        self.mwq = mwq
        self.mwq_st = None if mwq is None else mwq.struct()
        self.floe = floe
        self.floe_st = None if floe is None else floe.struct()
        if replica is None and mwq is None and floe is None:
            self.ws = _ws(layer.workspace_size(T), dev)
        else:
            n = C.c_size_t(0)
            fn = ("moe_replica_workspace_size" if replica is not None else
                  "moe_mwq_workspace_size" if mwq is not None else "moe_floe_workspace_size")
            B.check(getattr(B.lib(), fn)(C.byref(self.desc), T, C.byref(n)), fn)
            self.ws = _ws(n.value, dev)
        self.lis_base = torch.empty(1, dtype=torch.float64, device=dev)
        E, k = layer.n_experts, layer.top_k
        S = 0 if replica is None else 1   # extra slot of the replica
        self.y = torch.empty(T, layer.d_model, dtype=out_dtype, device=dev)
        self.aux_t = None
        self.aux = None
        if want_aux:
            self.aux_t = dict(
                logits=torch.empty(T, E, dtype=torch.float32, device=dev),
                idx=torch.empty(T, k, dtype=torch.int32, device=dev),
                gates=torch.empty(T, k, dtype=torch.float32, device=dev),
                counts=torch.empty(E + S, dtype=torch.int32, device=dev),
                offsets=torch.empty(E + 1 + S, dtype=torch.int32, device=dev),
                row_assign=torch.empty(max(T * k, 1), dtype=torch.int32, device=dev),
                assign_row=torch.empty(max(T * k, 1), dtype=torch.int32, device=dev),
                lis=torch.empty(1, dtype=torch.float64, device=dev))
            self.aux = B.Aux(**{n: _p(t) for n, t in self.aux_t.items()})
        self.groups = None
        if want_aux and mwq is not None:
            g = dict(mwq_idx=torch.empty(T, k, dtype=torch.int32, device=dev),
                     mwq_counts=torch.empty(3 * E, dtype=torch.int32, device=dev),
                     mwq_offsets=torch.empty(3 * E + 1, dtype=torch.int32, device=dev),
                     mwq_row_assign=torch.empty(max(T * k, 1), dtype=torch.int32, device=dev),
                     mwq_assign_row=torch.empty(max(T * k, 1), dtype=torch.int32, device=dev))
            self.aux_t.update(g)
            self.groups = B.MwqGroups(*[_p(g[n]) for n in ("mwq_idx", "mwq_counts", "mwq_offsets",
                                                           "mwq_row_assign", "mwq_assign_row")])

        self.floe_aux = None
        if want_aux and floe is not None:
            F = layer.d_ff
            g = dict(floe_u=torch.empty(max(T * k, 1), F, dtype=torch.float32, device=dev),
                     floe_nnz=torch.empty(E, dtype=torch.int32, device=dev),
                     floe_channels=torch.empty(E, F, dtype=torch.int32, device=dev))
            self.aux_t.update(g)
            self.floe_aux = B.FloeAux(_p(g["floe_u"]), _p(g["floe_nnz"]), _p(g["floe_channels"]))

    def __call__(self, x, flags=0, widths=None):
        aux = C.byref(self.aux) if self.aux is not None else None
        if self.floe is not None:
            fa = C.byref(self.floe_aux) if self.floe_aux is not None else None
            B.check(B.lib().moe_layer_forward_floe(C.byref(self.desc), C.byref(self.floe_st),
                                                   _p(x), self.T, _p(self.y), _dt(self.y), aux,
                                                   fa, _p(self.ws), self.ws.numel(), flags,
                                                   _stream()),
                    "moe_layer_forward_floe")
        elif self.mwq is not None:
            if widths is None:
                raise ValueError("a layer with nested experts needs the widths [T][k]")
            groups = C.byref(self.groups) if self.groups is not None else None
            B.check(B.lib().moe_layer_forward_mwq(C.byref(self.desc), C.byref(self.mwq_st),
                                                  _p(widths), _p(x), self.T, _p(self.y),
                                                  _dt(self.y), aux, groups, _p(self.ws),
                                                  self.ws.numel(), flags, _stream()),
                    "moe_layer_forward_mwq")
        elif self.rep is None:
            B.check(B.lib().moe_layer_forward(C.byref(self.desc), _p(x), self.T, _p(self.y),
                                              _dt(self.y), aux, _p(self.ws), self.ws.numel(),
                                              flags, _stream()),
                    "moe_layer_forward")
        else:
            B.check(B.lib().moe_layer_forward_replica(C.byref(self.desc), C.byref(self.rep),
                                                      _p(x), self.T, _p(self.y), _dt(self.y), aux,
                                                      _p(self.lis_base), _p(self.ws),
                                                      self.ws.numel(), flags, _stream()),
                    "moe_layer_forward_replica")
        return self.y


def layer_forward(layer: MoeLayer, x, out_dtype=torch.float32, flags=0, logits=None,
                  replica: Optional[MoeReplica] = None, mwq: Optional[MwqExperts] = None,
                  widths=None, floe: Optional[FloeExperts] = None):
    """One layer call; returns (y, aux dict of device tensors).  With ``replica``
    aux describes the split routing and aux["lis_base"] the router's own LIS;
    with ``mwq`` (and ``widths`` [T][k] int32) the routed experts are nested
    low-bit ones and aux adds the (expert, width) grouping; with ``floe`` the
    routed experts are sparse-down ones and aux adds floe_u (up outputs, rows
    expert-major), floe_nnz and floe_channels (kept channels per expert)."""
    r = LayerRunner(layer, x.shape[0], out_dtype, replica=replica, mwq=mwq, floe=floe)
    if logits is not None:
        r.aux_t["logits"].copy_(logits)
        flags |= B.MOE_F_LOGITS_GIVEN
    y = r(x, flags, widths=widths)
    if replica is not None:
        r.aux_t["lis_base"] = r.lis_base
    return y, r.aux_t


def noalloc_scratch_bytes() -> int:
    """Size of the static device array behind layer_forward_noalloc."""
    return int(B.lib().moe_noalloc_scratch_bytes())


def layer_forward_noalloc(layer: MoeLayer, x, y, aux=None, flags=0):
    """moe_layer_forward_noalloc: the layer with the library's static device
    array as workspace (the call allocates nothing).  y [T][d] (fp32 or bf16)
    is written; aux, if given, is a dict of caller tensors named as the fields
    of moe_aux (any subset).  Returns y."""
    T = x.shape[0]
    desc = layer.desc()
    a = None
    if aux:
        a = B.Aux(**{n: _p(t) for n, t in aux.items()})
    B.check(B.lib().moe_layer_forward_noalloc(C.byref(desc), _p(x), T, _p(y), _dt(y),
                                              C.byref(a) if a is not None else None, flags,
                                              _stream()),
            "moe_layer_forward_noalloc")
    return y


def replica_split(idx, counts, offsets, assign_row, E, heavy, flags=0):
    """Split routing of expert ``heavy`` (see moe_replica_split); returns a dict."""
    T, k = idx.shape
    dev = idx.device
    out = dict(idx=torch.empty_like(idx),
               counts=torch.empty(E + 1, dtype=torch.int32, device=dev),
               offsets=torch.empty(E + 2, dtype=torch.int32, device=dev),
               row_assign=torch.empty(max(T * k, 1), dtype=torch.int32, device=dev),
               assign_row=torch.empty(max(T * k, 1), dtype=torch.int32, device=dev),
               lis=torch.empty(1, dtype=torch.float64, device=dev))
    B.check(B.lib().moe_replica_split(_p(idx), _p(counts), _p(offsets), _p(assign_row), T, E, k,
                                      int(heavy), _p(out["idx"]), _p(out["counts"]),
                                      _p(out["offsets"]), _p(out["row_assign"]),
                                      _p(out["assign_row"]), _p(out["lis"]), flags, _stream()),
            "moe_replica_split")
    return out


def mwq_group(idx, widths, E, flags=0):
    """(expert, width) grouping of nested experts (see moe_mwq_group); returns a dict
    with group_idx, counts [3E], offsets [3E+1], row_assign, assign_row."""
    T, k = idx.shape
    dev = idx.device
    out = dict(group_idx=torch.empty_like(idx),
               counts=torch.empty(3 * E, dtype=torch.int32, device=dev),
               offsets=torch.empty(3 * E + 1, dtype=torch.int32, device=dev),
               row_assign=torch.empty(max(T * k, 1), dtype=torch.int32, device=dev),
               assign_row=torch.empty(max(T * k, 1), dtype=torch.int32, device=dev))
    g = B.MwqGroups(*[_p(out[n]) for n in ("group_idx", "counts", "offsets", "row_assign",
                                            "assign_row")])
    ws = _ws(B.lib().moe_mwq_group_workspace_size(T, E, k), dev)
    B.check(B.lib().moe_mwq_group(_p(idx), _p(widths), T, E, k, C.byref(g), _p(ws), ws.numel(),
                                  flags, _stream()),
            "moe_mwq_group")
    return out


def grouped_ffn_mwq(x, E, k, act, experts: MwqExperts, offsets, row_assign, topk_gate=None,
                    flags=0):
    """Gate-scaled rows y_rows [T*k][d] fp32 of nested experts, rows grouped by
    (expert, width) as mwq_group leaves them."""
    T, d = x.shape
    F = experts.up.q2.shape[-2]
    a = B.MOE_ACT_SWIGLU if act == "swiglu" else B.MOE_ACT_RELU
    st = experts.struct()
    y_rows = torch.empty(max(T * k, 1), d, dtype=torch.float32, device=x.device)
    ws = _ws(B.lib().moe_grouped_ffn_mwq_workspace_size(T, F, k), x.device)
    B.check(B.lib().moe_grouped_ffn_mwq(_p(x), T, d, F, E, k, a, C.byref(st), _p(offsets),
                                        _p(row_assign), _p(topk_gate), _p(y_rows), _p(ws),
                                        ws.numel(), flags, _stream()),
            "moe_grouped_ffn_mwq")
    return y_rows[:T * k]


@dataclass
class AtomicLayer:
    """Atomic experts on an nr x nc router grid (see moe_atomic_layer_forward):
    w_row [nr][d], w_col [nc][d], w_in [N][d], w_out [d][N] and/or w_out_rows
    [N][d] bf16 (the same output vectors in the dense and the expert-centric
    layout); optional shared SwiGLU MLP; schedule "auto", "dense" or
    "expert_centric"."""
    d_model: int
    grid_rows: int
    grid_cols: int
    top_k: int
    w_row: torch.Tensor
    w_col: torch.Tensor
    w_in: torch.Tensor
    w_out: Optional[torch.Tensor]
    n_shared: int = 0
    d_ff_shared: int = 0
    shared: Optional[ExpertWeights] = None
    w_out_rows: Optional[torch.Tensor] = None
    schedule: str = "auto"

    def desc(self) -> B.AtomicLayerDesc:
        L = B.AtomicLayerDesc()
        L.d_model, L.grid_rows, L.grid_cols, L.top_k = (self.d_model, self.grid_rows,
                                                        self.grid_cols, self.top_k)
        L.w_row, L.w_col, L.w_in, L.w_out = (_p(self.w_row), _p(self.w_col), _p(self.w_in),
                                             _p(self.w_out))
        L.n_shared, L.d_ff_shared = self.n_shared, self.d_ff_shared
        if self.shared is not None:
            L.shared = self.shared.struct(B.MOE_DT_BF16)
        L.w_out_rows = _p(self.w_out_rows)
        L.schedule = {"auto": B.MOE_ATOMIC_AUTO, "dense": B.MOE_ATOMIC_DENSE,
                      "expert_centric": B.MOE_ATOMIC_EXPERT_CENTRIC}[self.schedule]
        return L


class AtomicRunner:
    """Descriptor, workspace and aux buffers for repeated atomic-layer calls."""

    def __init__(self, layer: AtomicLayer, T: int, out_dtype=torch.float32, want_aux=True):
        self.layer, self.T = layer, T
        dev = layer.w_row.device
        self.desc = layer.desc()
        n = C.c_size_t(0)
        B.check(B.lib().moe_atomic_workspace_size(C.byref(self.desc), T, C.byref(n)),
                "moe_atomic_workspace_size")
        self.ws = _ws(n.value, dev)
        self.y = torch.empty(T, layer.d_model, dtype=out_dtype, device=dev)
        nr, nc, K = layer.grid_rows, layer.grid_cols, layer.top_k
        N = nr * nc
        self.aux_t, self.aux = None, None
        if want_aux:
            self.aux_t = dict(
                logp_row=torch.empty(T, nr, dtype=torch.float32, device=dev),
                logp_col=torch.empty(T, nc, dtype=torch.float32, device=dev),
                idx=torch.empty(T, K, dtype=torch.int32, device=dev),
                gates=torch.empty(T, K, dtype=torch.float32, device=dev),
                counts=torch.empty(N, dtype=torch.int32, device=dev),
                offsets=torch.empty(N + 1, dtype=torch.int32, device=dev),
                row_assign=torch.empty(max(T * K, 1), dtype=torch.int32, device=dev),
                assign_row=torch.empty(max(T * K, 1), dtype=torch.int32, device=dev),
                lis=torch.empty(1, dtype=torch.float64, device=dev))
            self.aux = B.AtomicAux(**{k: _p(v) for k, v in self.aux_t.items()})

    def schedule_used(self) -> str:
        """The schedule the library runs for this layer and T (moe_atomic_schedule)."""
        v = C.c_int(-1)
        B.check(B.lib().moe_atomic_schedule(C.byref(self.desc), self.T, C.byref(v)),
                "moe_atomic_schedule")
        return {B.MOE_ATOMIC_DENSE: "dense", B.MOE_ATOMIC_EXPERT_CENTRIC: "expert_centric"}[v.value]

    def __call__(self, x, flags=0):
        aux = C.byref(self.aux) if self.aux is not None else None
        B.check(B.lib().moe_atomic_layer_forward(C.byref(self.desc), _p(x), self.T, _p(self.y),
                                                 _dt(self.y), aux, _p(self.ws), self.ws.numel(),
                                                 flags, _stream()),
                "moe_atomic_layer_forward")
        return self.y


def atomic_layer_forward(layer: AtomicLayer, x, out_dtype=torch.float32, flags=0):
    """One atomic-layer call; returns (y, aux dict of device tensors)."""
    r = AtomicRunner(layer, x.shape[0], out_dtype)
    y = r(x, flags)
    return y, r.aux_t
