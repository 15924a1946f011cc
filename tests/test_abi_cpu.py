"""C-ABI checks that need no GPU: exported symbols and host-side validation.

Every error path is forced from the host with MOE_F_VALIDATE_ONLY and fake,
never-dereferenced device addresses; no HIP call is made.
"""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    from sparse_mixture_experts_wavefront_amd import _binding as B
    if not os.path.exists(B.LIB_PATH):
        from sparse_mixture_experts_wavefront_amd import build
        build.build()
    return B.lib()


@pytest.fixture(scope="module")
def B():
    from sparse_mixture_experts_wavefront_amd import _binding
    return _binding


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", src)))


def test_every_declared_symbol_is_exported(L):
    names = _declared_functions()
    assert "moe_layer_forward" in names and len(names) >= 10
    for n in names:
        assert hasattr(L, n), "missing export " + n


def test_binding_lists_all_exports(B):
    assert sorted(B.EXPORTED) == _declared_functions()


FAKE = 0x10000  # aligned, never dereferenced under VALIDATE_ONLY


def _addr(i=0):
    return C.c_void_p(FAKE + 4096 * i)


def route(L, B, T=4, d=64, E=8, k=2, flags=None, x=True, w=True, logits=True, idx=True,
          xdt=1):
    f = B.MOE_F_VALIDATE_ONLY if flags is None else flags
    return L.moe_route_topk(_addr(1) if x else None, xdt, _addr(2) if w else None, None, T, d,
                            E, k, _addr(3) if logits else None, _addr(4) if idx else None, None,
                            f, None)


def test_route_validation(L, B):
    assert route(L, B) == B.MOE_OK
    assert route(L, B, k=0) == B.MOE_ERR_INVALID_ARG
    assert route(L, B, k=9, E=9) == B.MOE_ERR_UNSUPPORTED
    assert route(L, B, k=3, E=2) == B.MOE_ERR_INVALID_ARG
    assert route(L, B, E=0) == B.MOE_ERR_INVALID_ARG
    assert route(L, B, E=65) == B.MOE_ERR_UNSUPPORTED
    assert route(L, B, d=60) == B.MOE_ERR_INVALID_ARG
    assert route(L, B, T=-1) == B.MOE_ERR_INVALID_ARG
    assert route(L, B, x=False) == B.MOE_ERR_INVALID_ARG
    assert route(L, B, idx=False) == B.MOE_ERR_INVALID_ARG
    assert route(L, B, xdt=7) == B.MOE_ERR_INVALID_ARG
    assert route(L, B, flags=B.MOE_F_VALIDATE_ONLY | 64) == B.MOE_ERR_INVALID_ARG
    # logits given: x and w may be absent
    assert route(L, B, x=False, w=False,
                 flags=B.MOE_F_VALIDATE_ONLY | B.MOE_F_LOGITS_GIVEN) == B.MOE_OK
    # a successful validation clears the thread's error string
    assert L.moe_last_error() == b""
    assert route(L, B, x=False) == B.MOE_ERR_INVALID_ARG
    assert L.moe_last_error() == b"x must not be NULL"
    r = L.moe_route_topk(C.c_void_p(FAKE + 8), 1, _addr(2), None, 4, 64, 8, 2, _addr(3),
                         _addr(4), None, B.MOE_F_VALIDATE_ONLY, None)
    assert r == B.MOE_ERR_INVALID_ARG and b"aligned" in L.moe_last_error()
    assert route(L, B) == B.MOE_OK and L.moe_last_error() == b""


def test_permute_validation_and_workspace(L, B):
    VO = B.MOE_F_VALIDATE_ONLY

    def perm(T, E, k, ws=None, nbytes=0, counts=True):
        return L.moe_permute(_addr(1), T, E, k, _addr(2) if counts else None, _addr(3), _addr(4),
                             _addr(5), _addr(6), ws, nbytes, VO, None)
    assert perm(16, 8, 2) == B.MOE_OK                  # fused path needs no workspace
    assert L.moe_permute_workspace_size(16, 8, 2) == 0
    need = L.moe_permute_workspace_size(8192, 64, 6)
    assert need > 0
    assert perm(8192, 64, 6) == B.MOE_ERR_WORKSPACE
    assert perm(8192, 64, 6, _addr(7), need - 1) == B.MOE_ERR_WORKSPACE
    assert perm(8192, 64, 6, _addr(7), need) == B.MOE_OK
    assert perm(16, 8, 2, counts=False) == B.MOE_ERR_INVALID_ARG
    assert perm(0, 8, 2) == B.MOE_OK


def _experts(B, dtype=1, gate=True, int4=False):
    e = B.Experts()
    e.dtype = dtype
    keep = []
    if int4:
        for name in ("q_gate", "q_up", "q_down"):
            if name == "q_gate" and not gate:
                continue
            w = B.W4(_addr(10), _addr(11), _addr(12))
            keep.append(w)
            setattr(e, name, C.pointer(w))
    else:
        e.w_gate = _addr(10) if gate else None
        e.w_up, e.w_down = _addr(11), _addr(12)
    e._keep = keep
    return e


def test_grouped_ffn_validation(L, B):
    VO = B.MOE_F_VALIDATE_ONLY

    def ffn(T=16, d=128, F=256, E=8, k=2, act=0, ex=None, offsets=True, ra=True, ws=True,
            xdt=1):
        ex = ex or _experts(B)
        need = L.moe_grouped_ffn_workspace_size(T, d, F, E, k, act, C.byref(ex))
        return L.moe_grouped_ffn(_addr(1), xdt, T, d, F, E, k, act, C.byref(ex),
                                 _addr(2) if offsets else None, _addr(3) if ra else None, None,
                                 _addr(4), _addr(5) if ws else None, need, VO, None)
    assert ffn() == B.MOE_OK
    assert ffn(ws=False) == B.MOE_ERR_WORKSPACE
    assert ffn(offsets=False) == B.MOE_ERR_INVALID_ARG          # needs E == 1, k == 1
    assert ffn(offsets=False, E=1, k=1, ra=False) == B.MOE_OK
    assert ffn(ra=False) == B.MOE_ERR_INVALID_ARG               # k > 1 needs row_assign
    assert ffn(F=250) == B.MOE_ERR_INVALID_ARG
    assert ffn(ex=_experts(B, gate=False)) == B.MOE_ERR_INVALID_ARG       # SwiGLU needs gate
    assert ffn(ex=_experts(B, gate=False), act=1) == B.MOE_OK             # ReLU does not
    assert ffn(ex=_experts(B, dtype=0)) == B.MOE_ERR_INVALID_ARG          # dtype mismatch
    assert ffn(ex=_experts(B, int4=True)) == B.MOE_OK
    assert ffn(ex=_experts(B, int4=True), d=136) == B.MOE_ERR_INVALID_ARG  # K % 128
    assert ffn(ex=_experts(B, int4=True), xdt=0) == B.MOE_ERR_UNSUPPORTED


def test_combine_validation(L, B):
    VO = B.MOE_F_VALIDATE_ONLY
    assert L.moe_combine(_addr(1), _addr(2), 4, 2, 64, None, _addr(3), 0, VO, None) == B.MOE_OK
    assert L.moe_combine(_addr(1), None, 4, 2, 64, None, _addr(3), 0, VO, None) == \
        B.MOE_ERR_INVALID_ARG
    assert L.moe_combine(_addr(1), _addr(2), 4, 9, 64, None, _addr(3), 0, VO, None) == \
        B.MOE_ERR_INVALID_ARG
    assert L.moe_combine(_addr(1), _addr(2), 4, 2, 64, None, _addr(3), 5, VO, None) == \
        B.MOE_ERR_INVALID_ARG


def _desc(B, T_shared=False, int4=False):
    Ld = B.LayerDesc()
    Ld.d_model, Ld.d_ff, Ld.n_experts, Ld.top_k = 256, 512, 8, 2
    Ld.act, Ld.act_dtype = 0, 1
    Ld.w_router = _addr(20)
    Ld.routed = _experts(B, int4=int4)
    if T_shared:
        Ld.n_shared, Ld.d_ff_shared = 2, 64
        Ld.shared = _experts(B)
    return Ld


def test_layer_workspace_and_validation(L, B):
    Ld = _desc(B)
    n = C.c_size_t(0)
    assert L.moe_workspace_size(C.byref(Ld), 100, C.byref(n)) == B.MOE_OK
    small = n.value
    Ls = _desc(B, T_shared=True)
    n2 = C.c_size_t(0)
    assert L.moe_workspace_size(C.byref(Ls), 100, C.byref(n2)) == B.MOE_OK
    assert n2.value > small                                   # shared H and y_shared
    VO = B.MOE_F_VALIDATE_ONLY
    ws = C.c_void_p(FAKE * 16)
    assert L.moe_layer_forward(C.byref(Ld), _addr(1), 100, _addr(2), 0, None, ws, small, VO,
                               None) == B.MOE_OK
    assert L.moe_layer_forward(C.byref(Ld), _addr(1), 100, _addr(2), 0, None, ws, small - 1, VO,
                               None) == B.MOE_ERR_WORKSPACE
    assert L.moe_layer_forward(C.byref(Ld), _addr(1), 100, _addr(2), 0, None, ws, small,
                               VO | B.MOE_F_LOGITS_GIVEN, None) == B.MOE_ERR_INVALID_ARG
    Ld.top_k = 0
    assert L.moe_layer_forward(C.byref(Ld), _addr(1), 100, _addr(2), 0, None, ws, small, VO,
                               None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_layer_forward(None, _addr(1), 100, _addr(2), 0, None, ws, small, VO,
                               None) == B.MOE_ERR_INVALID_ARG
    Li = _desc(B, int4=True)
    assert L.moe_workspace_size(C.byref(Li), 64, C.byref(n)) == B.MOE_OK


def test_noalloc_validation(L, B):
    """The allocation-free layer call checks its arguments and the size of its
    static scratch on the host; nothing here touches a device."""
    VO = B.MOE_F_VALIDATE_ONLY
    cap = L.moe_noalloc_scratch_bytes()
    assert cap == 64 << 20
    Ld = _desc(B)
    n = C.c_size_t(0)

    def ws(T):
        assert L.moe_workspace_size(C.byref(Ld), T, C.byref(n)) == B.MOE_OK
        return n.value
    T = 100
    assert ws(T) <= cap
    assert L.moe_layer_forward_noalloc(C.byref(Ld), _addr(1), T, _addr(2), 0, None, VO,
                                       None) == B.MOE_OK
    assert L.moe_last_error() == b""
    big = T
    while ws(big) <= cap:
        big *= 2
    assert L.moe_layer_forward_noalloc(C.byref(Ld), _addr(1), big, _addr(2), 0, None, VO,
                                       None) == B.MOE_ERR_WORKSPACE
    assert b"static" in L.moe_last_error()
    assert L.moe_layer_forward_noalloc(C.byref(Ld), None, T, _addr(2), 0, None, VO,
                                       None) == B.MOE_ERR_INVALID_ARG
    assert L.moe_layer_forward_noalloc(C.byref(Ld), _addr(1), 0, None, 0, None, VO,
                                       None) == B.MOE_OK
    Ld.top_k = 0
    assert L.moe_layer_forward_noalloc(C.byref(Ld), _addr(1), T, _addr(2), 0, None, VO,
                                       None) == B.MOE_ERR_INVALID_ARG


def test_status_strings(L, B):
    for s in range(5):
        assert L.moe_status_string(s).decode().startswith("MOE_")


def _replica(B, expert=0, gate=True):
    r = B.Replica()
    r.expert = expert
    keep = []
    for name in ("q_gate", "q_up", "q_down"):
        if name == "q_gate" and not gate:
            continue
        w = B.W4(_addr(30), _addr(31), _addr(32))
        keep.append(w)
        setattr(r, name, C.pointer(w))
    r._keep = keep
    return r


def test_replica_validation_and_workspace(L, B):
    VO = B.MOE_F_VALIDATE_ONLY
    Ld = _desc(B)
    n0, n1 = C.c_size_t(0), C.c_size_t(0)
    assert L.moe_workspace_size(C.byref(Ld), 100, C.byref(n0)) == B.MOE_OK
    assert L.moe_replica_workspace_size(C.byref(Ld), 100, C.byref(n1)) == B.MOE_OK
    assert n1.value > 0 and n0.value > 0   # (the plain layer may hold K-slice partials instead)
    ws = C.c_void_p(FAKE * 16)

    def fwd(rep, nbytes=None, Ldesc=None):
        return L.moe_layer_forward_replica(C.byref(Ldesc or Ld), None if rep is None else C.byref(rep),
                                           _addr(1), 100, _addr(2), 0, None, _addr(3), ws,
                                           n1.value if nbytes is None else nbytes, VO, None)
    assert fwd(_replica(B, 3)) == B.MOE_OK
    assert fwd(_replica(B, 3), n1.value - 1) == B.MOE_ERR_WORKSPACE
    assert fwd(_replica(B, 8)) == B.MOE_ERR_INVALID_ARG          # expert out of range
    assert fwd(_replica(B, -1)) == B.MOE_ERR_INVALID_ARG
    assert fwd(None) == B.MOE_ERR_INVALID_ARG
    assert fwd(_replica(B, 3, gate=False)) == B.MOE_ERR_INVALID_ARG   # SwiGLU needs q_gate
    Lf = _desc(B)
    Lf.act_dtype = 0
    Lf.routed = _experts(B, dtype=0)
    assert fwd(_replica(B, 3), Ldesc=Lf) == B.MOE_ERR_UNSUPPORTED     # bf16 activations only

    def split(heavy, T=16, E=8, k=2, counts=True):
        return L.moe_replica_split(_addr(1), _addr(2) if counts else None, _addr(3), _addr(4), T,
                                   E, k, heavy, _addr(5), _addr(6), _addr(7), _addr(8), _addr(9),
                                   _addr(10), VO, None)
    assert split(0) == B.MOE_OK
    assert split(7) == B.MOE_OK
    assert split(8) == B.MOE_ERR_INVALID_ARG
    assert split(0, counts=False) == B.MOE_ERR_INVALID_ARG
    assert split(0, E=65) == B.MOE_ERR_UNSUPPORTED


def _mwq_experts(B, gate=True, hole=None):
    keep = []
    ex = B.MwqExperts()
    for j, name in enumerate(("gate", "up", "down")):
        if name == "gate" and not gate:
            continue
        ptrs = [_addr(40 + 8 * j + i) for i in range(7)]
        if hole is not None and name == hole[0]:
            ptrs[hole[1]] = None
        w = B.WMwq(*ptrs)
        keep.append(w)
        setattr(ex, name, C.pointer(w))
    ex._keep = keep
    return ex


def test_mwq_validation_and_workspace(L, B):
    VO = B.MOE_F_VALIDATE_ONLY
    Ld = _desc(B)
    Ld.d_model, Ld.d_ff = 512, 1024
    Ld.routed = B.Experts()          # not read by the nested layer
    n = C.c_size_t(0)
    assert L.moe_mwq_workspace_size(C.byref(Ld), 100, C.byref(n)) == B.MOE_OK
    assert n.value >= 100 * 2 * 1024 * 2 + 100 * 2 * 512 * 4     # H and the gate-scaled rows
    ws = C.c_void_p(FAKE * 16)
    groups = B.MwqGroups(_addr(60), _addr(61), _addr(62), _addr(63), _addr(64))

    def fwd(ex, nbytes=None, Ldesc=None, widths=True, T=100, g=groups):
        return L.moe_layer_forward_mwq(C.byref(Ldesc or Ld), None if ex is None else C.byref(ex),
                                       _addr(5) if widths else None, _addr(1), T, _addr(2), 0,
                                       None, None if g is None else C.byref(g), ws,
                                       n.value if nbytes is None else nbytes, VO, None)
    assert fwd(_mwq_experts(B)) == B.MOE_OK
    assert fwd(_mwq_experts(B), g=None) == B.MOE_OK
    assert fwd(_mwq_experts(B), n.value - 1) == B.MOE_ERR_WORKSPACE
    assert fwd(None) == B.MOE_ERR_INVALID_ARG
    assert fwd(_mwq_experts(B), widths=False) == B.MOE_ERR_INVALID_ARG
    assert fwd(_mwq_experts(B, gate=False)) == B.MOE_ERR_INVALID_ARG      # SwiGLU needs gate
    for hole in (("up", 0), ("down", 3), ("gate", 6), ("up", 1)):
        assert fwd(_mwq_experts(B, hole=hole)) == B.MOE_ERR_INVALID_ARG, hole
    Lr = _desc(B)
    Lr.d_model, Lr.d_ff, Lr.act = 512, 1024, 1
    Lr.routed = B.Experts()
    assert fwd(_mwq_experts(B, gate=False), Ldesc=Lr) == B.MOE_OK         # ReLU: no gate
    Lk = _desc(B)
    Lk.d_model, Lk.d_ff = 512, 640                                         # d_ff % 512 != 0
    Lk.routed = B.Experts()
    assert fwd(_mwq_experts(B), Ldesc=Lk) == B.MOE_ERR_UNSUPPORTED
    Le = _desc(B)
    Le.d_model, Le.d_ff, Le.n_experts = 512, 1024, 22                     # 3E > 64
    Le.routed = B.Experts()
    assert fwd(_mwq_experts(B), Ldesc=Le) == B.MOE_ERR_UNSUPPORTED
    Lf = _desc(B)
    Lf.d_model, Lf.d_ff, Lf.act_dtype = 512, 1024, 0
    Lf.routed = B.Experts()
    assert fwd(_mwq_experts(B), Ldesc=Lf) == B.MOE_ERR_UNSUPPORTED       # bf16 activations only

    def grp(T=16, E=8, k=2, nbytes=None, counts=True, widths=True):
        g = B.MwqGroups(None, _addr(61) if counts else None, _addr(62), None, None)
        need = L.moe_mwq_group_workspace_size(T, E, k)
        return L.moe_mwq_group(_addr(1), _addr(2) if widths else None, T, E, k, C.byref(g), ws,
                               need if nbytes is None else nbytes, VO, None)
    assert grp() == B.MOE_OK
    assert grp(E=21, k=8, T=333) == B.MOE_OK
    assert grp(E=22) == B.MOE_ERR_UNSUPPORTED
    assert grp(counts=False) == B.MOE_ERR_INVALID_ARG
    assert grp(widths=False) == B.MOE_ERR_INVALID_ARG
    assert grp(nbytes=16) == B.MOE_ERR_WORKSPACE
    assert L.moe_mwq_group_workspace_size(9000, 8, 2) > L.moe_mwq_group_workspace_size(16, 8, 2)

    def ffn(d=512, F=1024, act=0, nbytes=None, ex=None):
        need = L.moe_grouped_ffn_mwq_workspace_size(16, F, 2)
        return L.moe_grouped_ffn_mwq(_addr(1), 16, d, F, 8, 2, act,
                                     C.byref(ex or _mwq_experts(B)), _addr(2), _addr(3), None,
                                     _addr(4), ws, need if nbytes is None else nbytes, VO, None)
    assert ffn() == B.MOE_OK
    assert ffn(d=384) == B.MOE_ERR_UNSUPPORTED
    assert ffn(d=200) == B.MOE_ERR_INVALID_ARG
    assert ffn(nbytes=100) == B.MOE_ERR_WORKSPACE
    assert ffn(act=1, ex=_mwq_experts(B, gate=False)) == B.MOE_OK


def test_floe_validation_and_workspace(L, B):
    VO = B.MOE_F_VALIDATE_ONLY
    Ld = _desc(B)
    Ld.d_model, Ld.d_ff = 512, 1024
    Ld.routed = B.Experts()
    n = C.c_size_t(0)
    assert L.moe_floe_workspace_size(C.byref(Ld), 16, C.byref(n)) == B.MOE_OK
    assert n.value >= 16 * 2 * 1024 * (4 + 2) + 8 * 1024 * 5   # U, Hc, flags, lists
    ws = C.c_void_p(FAKE * 16)

    def experts(up=True, gate=True, down=True, thr=True, s2=True):
        w = B.WMwq(_addr(40), _addr(41) if s2 else None, _addr(42), None, None, None, None)
        ex = B.FloeExperts(C.pointer(w) if up else None, _addr(43) if gate else None,
                           _addr(44) if down else None, _addr(45) if thr else None)
        ex._keep = [w]
        return ex

    def fwd(ex, Ldesc=None, nbytes=None, T=16):
        return L.moe_layer_forward_floe(C.byref(Ldesc or Ld), None if ex is None else C.byref(ex),
                                        _addr(1), T, _addr(2), 0, None, None, ws,
                                        n.value if nbytes is None else nbytes, VO, None)
    assert fwd(experts()) == B.MOE_OK
    assert fwd(experts(), nbytes=n.value - 1) == B.MOE_ERR_WORKSPACE
    assert fwd(None) == B.MOE_ERR_INVALID_ARG
    for kw in ("up", "gate", "down", "thr", "s2"):
        assert fwd(experts(**{kw: False})) == B.MOE_ERR_INVALID_ARG, kw
    Lr = _desc(B)
    Lr.d_model, Lr.d_ff, Lr.act = 512, 1024, 1
    Lr.routed = B.Experts()
    assert fwd(experts(), Ldesc=Lr) == B.MOE_ERR_UNSUPPORTED            # SwiGLU only
    Lk = _desc(B)
    Lk.d_model, Lk.d_ff = 640, 1024
    Lk.routed = B.Experts()
    assert fwd(experts(), Ldesc=Lk) == B.MOE_ERR_UNSUPPORTED            # d_model % 512


def test_atomic_validation_and_workspace(L, B):
    VO = B.MOE_F_VALIDATE_ONLY

    def desc(d=256, nr=8, nc=32, K=16, shared=False):
        Ld = B.AtomicLayerDesc()
        Ld.d_model, Ld.grid_rows, Ld.grid_cols, Ld.top_k = d, nr, nc, K
        Ld.w_row, Ld.w_col, Ld.w_in, Ld.w_out = _addr(50), _addr(51), _addr(52), _addr(53)
        if shared:
            Ld.n_shared, Ld.d_ff_shared = 1, 128
            Ld.shared = _experts(B)
        return Ld
    Ld = desc()
    n = C.c_size_t(0)
    assert L.moe_atomic_workspace_size(C.byref(Ld), 48, C.byref(n)) == B.MOE_OK
    assert n.value >= 48 * 256 * 2 + 48 * 16 * 8     # the [T][N] hidden matrix, ids and gates
    ws = C.c_void_p(FAKE * 16)

    def fwd(Ldesc, nbytes=None, T=48, flags=VO):
        need = C.c_size_t(0)
        L.moe_atomic_workspace_size(C.byref(Ldesc), T, C.byref(need))
        return L.moe_atomic_layer_forward(C.byref(Ldesc), _addr(1), T, _addr(2), 0, None, ws,
                                          need.value if nbytes is None else nbytes, flags, None)
    assert fwd(Ld) == B.MOE_OK
    assert fwd(desc(shared=True)) == B.MOE_OK
    assert fwd(Ld, nbytes=n.value - 1) == B.MOE_ERR_WORKSPACE
    assert fwd(desc(K=0)) == B.MOE_ERR_INVALID_ARG
    assert fwd(desc(K=257)) == B.MOE_ERR_INVALID_ARG          # K > N
    assert fwd(desc(d=200)) == B.MOE_ERR_INVALID_ARG
    assert fwd(desc(nc=40)) == B.MOE_ERR_UNSUPPORTED          # nc % 32
    assert fwd(desc(nr=2000)) == B.MOE_ERR_UNSUPPORTED        # nr > 1024
    assert fwd(desc(nr=3, nc=32)) == B.MOE_ERR_UNSUPPORTED    # N % 128
    assert fwd(Ld, flags=VO | B.MOE_F_LOGITS_GIVEN) == B.MOE_ERR_INVALID_ARG
    bad = desc()
    bad.w_in = None
    assert fwd(bad) == B.MOE_ERR_INVALID_ARG


def test_atomic_schedule_resolution(L, B):
    """Which schedule a call runs, and what each schedule needs, all on the host."""
    VO = B.MOE_F_VALIDATE_ONLY

    def desc(d=512, dense=True, rows=True, schedule=0):
        Ld = B.AtomicLayerDesc()
        Ld.d_model, Ld.grid_rows, Ld.grid_cols, Ld.top_k = d, 8, 32, 16
        Ld.w_row, Ld.w_col, Ld.w_in = _addr(50), _addr(51), _addr(52)
        Ld.w_out = _addr(53) if dense else None
        Ld.w_out_rows = _addr(54) if rows else None
        Ld.schedule = schedule
        return Ld

    def sched(Ld, T):
        v = C.c_int(-1)
        r = L.moe_atomic_schedule(C.byref(Ld), T, C.byref(v))
        return r if r != B.MOE_OK else ("ec" if v.value == B.MOE_ATOMIC_EXPERT_CENTRIC else
                                        "dense" if v.value == B.MOE_ATOMIC_DENSE else v.value)
    assert sched(desc(), 1) == "ec"
    assert sched(desc(), 64) == "ec"
    assert sched(desc(), 65) == "dense"
    assert sched(desc(dense=False), 4096) == "ec"          # only the expert-major copy
    assert sched(desc(rows=False), 1) == "dense"
    assert sched(desc(d=256), 1) == "dense"                # d % 512: expert-centric not built
    assert sched(desc(d=256, dense=False), 1) == B.MOE_ERR_UNSUPPORTED
    assert sched(desc(dense=False, rows=False), 1) == B.MOE_ERR_INVALID_ARG
    assert sched(desc(schedule=B.MOE_ATOMIC_DENSE), 1) == "dense"
    assert sched(desc(schedule=B.MOE_ATOMIC_EXPERT_CENTRIC), 4096) == "ec"
    assert sched(desc(rows=False, schedule=B.MOE_ATOMIC_EXPERT_CENTRIC), 1) == \
        B.MOE_ERR_INVALID_ARG
    assert sched(desc(dense=False, schedule=B.MOE_ATOMIC_DENSE), 1) == B.MOE_ERR_INVALID_ARG
    assert sched(desc(d=4608, schedule=B.MOE_ATOMIC_EXPERT_CENTRIC), 1) == B.MOE_ERR_UNSUPPORTED
    assert sched(desc(schedule=7), 1) == B.MOE_ERR_INVALID_ARG
    assert L.moe_atomic_schedule(C.byref(desc()), 1, None) == B.MOE_ERR_INVALID_ARG
    # the workspace follows the schedule (each is checked against its own size)
    n_ec, n_dense = C.c_size_t(0), C.c_size_t(0)
    assert L.moe_atomic_workspace_size(C.byref(desc(schedule=2)), 64, C.byref(n_ec)) == B.MOE_OK
    assert L.moe_atomic_workspace_size(C.byref(desc(schedule=1)), 64, C.byref(n_dense)) == B.MOE_OK
    assert n_ec.value != n_dense.value
    ws = C.c_void_p(FAKE * 16)
    for Ld, n in ((desc(schedule=2), n_ec.value), (desc(schedule=1), n_dense.value)):
        assert L.moe_atomic_layer_forward(C.byref(Ld), _addr(1), 64, _addr(2), 0, None, ws, n,
                                          VO, None) == B.MOE_OK
        assert L.moe_atomic_layer_forward(C.byref(Ld), _addr(1), 64, _addr(2), 0, None, ws,
                                          n - 1, VO, None) == B.MOE_ERR_WORKSPACE
