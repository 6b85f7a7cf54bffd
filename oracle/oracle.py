"""ctypes front end of the fp64 reference checker in ``mom_oracle.c``.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg
of the benchmark may call this module; the GPU library never does.  Inputs are
converted exactly to float64 (fp32 and bfloat16 values are exact in fp64).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mom_oracle.c")
_LIB = os.path.join(_HERE, "_build", "libmom_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the checker with gcc (plain C99, OpenMP, IEEE double)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    os.makedirs(os.path.dirname(_LIB), exist_ok=True)
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c99", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        build(force=False)
        _lib = ctypes.CDLL(_LIB)
    return _lib


def _d(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def _i(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.int32)


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def threads() -> int:
    """Number of OpenMP threads the checker uses."""
    return int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))


def route(x, w_r, bias, K, want_logits=False):
    x, w_r, bias = _d(x), _d(w_r), _d(bias)
    n, D = x.shape
    M = w_r.shape[0]
    idx = np.empty((n, K), np.int32)
    w = np.empty((n, K), np.float64)
    lg = np.empty((n, M), np.float64) if want_logits else None
    lib().oracle_route(ctypes.c_int64(n), D, M, K, _p(x), _p(w_r), _p(bias), _p(idx), _p(w), _p(lg))
    return (idx, w, lg) if want_logits else (idx, w)


def dispatch(idx, B, T, M):
    idx = _i(idx)
    K = idx.shape[1]
    N = B * T * (K + 1)
    seg_off = np.empty((M + 1) * B + 1, np.int32)
    perm = np.empty(N, np.int32)
    inv = np.empty((B * T, K), np.int32)
    lib().oracle_dispatch(B, T, M, K, _p(idx), _p(seg_off), _p(perm), _p(inv))
    return seg_off, perm, inv


def gdn_step(q, k, v, a, c, S):
    """One recurrence step; S [dk][dv] is updated in place (float64)."""
    q, k, v = _d(q), _d(k), _d(v)
    assert S.dtype == np.float64 and S.flags.c_contiguous
    dk, dv = S.shape
    o = np.empty(dv, np.float64)
    lib().oracle_gdn_step(dk, dv, ctypes.c_double(a), ctypes.c_double(c), _p(q), _p(k), _p(v),
                          _p(S), _p(o))
    return o


def gdn_chain(q, k, v, a, c, S0=None):
    """Recurrence over one memory's own rows: returns (o [L][dv], S_final)."""
    q, k, v, a, c = _d(q), _d(k), _d(v), _d(a), _d(c)
    L, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else _d(S0).copy()
    o = np.empty((L, dv), np.float64)
    lib().oracle_gdn_chain(ctypes.c_int64(L), dk, dv, _p(q), _p(k), _p(v), _p(a), _p(c), _p(S), _p(o))
    return o, S


# update rules of a memory (mom_oracle.c): Gated DeltaNet, gated linear attention
RULES = {"gdn": 0, "gla": 1}


def gla_step(q, k, v, a, c, S):
    """One gated linear attention step; S [dk][dv] is updated in place (float64)."""
    q, k, v = _d(q), _d(k), _d(v)
    assert S.dtype == np.float64 and S.flags.c_contiguous
    dk, dv = S.shape
    o = np.empty(dv, np.float64)
    lib().oracle_gla_step(dk, dv, ctypes.c_double(a), ctypes.c_double(c), _p(q), _p(k), _p(v),
                          _p(S), _p(o))
    return o


def gla_chain(q, k, v, a, c, S0=None):
    """Gated linear attention over one memory's rows: returns (o [L][dv], S_final)."""
    q, k, v, a, c = _d(q), _d(k), _d(v), _d(a), _d(c)
    L, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else _d(S0).copy()
    o = np.empty((L, dv), np.float64)
    lib().oracle_gla_chain(ctypes.c_int64(L), dk, dv, _p(q), _p(k), _p(v), _p(a), _p(c), _p(S), _p(o))
    return o, S


def layer(dims, x, w_r, bias, w_q, w_k, w_v, alpha, beta, state0=None, mixed=False,
          want_qkv=False, rule="gdn"):
    """Whole layer forward.  dims = (B, T, D, H, dk, dv, M, K); rule "gdn" (Gated
    DeltaNet memories) or "gla" (gated linear attention memories)."""
    B, T, D, H, dk, dv, M, K = [int(v) for v in dims]
    NT = B * T
    args = [_d(a) for a in (x, w_r, bias, w_q, w_k, w_v, alpha, beta, state0)]
    res = dict(
        idx=np.empty((NT, K), np.int32), w=np.empty((NT, K)),
        o_routed=np.empty((NT, K, H, dv)), o_shared=np.empty((NT, H, dv)),
        out=np.empty((NT, H, dv)), out_mixed=np.empty((NT, H, dv)) if mixed else None,
        state=np.empty((B, M + 1, H, dk, dv)),
        q=np.empty((NT, H, dk)) if want_qkv else None,
        k=np.empty((NT, K + 1, H, dk)) if want_qkv else None,
        v=np.empty((NT, K + 1, H, dv)) if want_qkv else None)
    dims_a = np.array([B, T, D, H, dk, dv, M, K], np.int32)
    lib().oracle_layer_rule(RULES[rule], _p(dims_a), *[_p(a) for a in args], _p(res["idx"]), _p(res["w"]),
                       _p(res["o_routed"]), _p(res["o_shared"]), _p(res["out"]),
                       _p(res["out_mixed"]), _p(res["state"]), _p(res["q"]), _p(res["k"]),
                       _p(res["v"]))
    return res


def combine(inv, w, o_routed, o_shared):
    w, o_routed, o_shared = _d(w), _d(o_routed), _d(o_shared)
    inv = _i(inv)
    n, K = w.shape
    H, dv = o_shared.shape[1], o_shared.shape[2]
    out = np.empty((n, H, dv))
    lib().oracle_combine(ctypes.c_int64(n), K, H, dv, _p(inv), _p(w), _p(o_routed), _p(o_shared),
                         _p(out))
    return out


def segments(seg_off, seg_state, row_token, q, k, v, a, c, state, which=None, rule="gdn"):
    """Run the recurrence over packed segments.  `state` (float64 [n_state][H][dk][dv])
    is updated in place; returns o [N][H][dv] (rows of segments not run are NaN)."""
    seg_off, seg_state, row_token, which = _i(seg_off), _i(seg_state), _i(row_token), _i(which)
    q, k, v, a, c = _d(q), _d(k), _d(v), _d(a), _d(c)
    assert state.dtype == np.float64 and state.flags.c_contiguous
    N, H, dk = k.shape
    dv = v.shape[2]
    o = np.full((N, H, dv), np.nan)
    n_seg = seg_off.shape[0] - 1
    lib().oracle_segments_rule(RULES[rule], n_seg, _p(seg_off), _p(seg_state), _p(row_token), H, dk, dv, _p(q), _p(k),
                          _p(v), _p(a), _p(c), _p(state), _p(o), 0 if which is None else len(which),
                          _p(which))
    return o


def project_head(rows_tok, x, wq_h, wk_h, wv_h):
    """Projections of one head for the tokens rows_tok: (q, k normalised, v)."""
    rows_tok, x = _i(rows_tok), _d(x)
    wq_h, wk_h, wv_h = _d(wq_h), _d(wk_h), _d(wv_h)
    n = rows_tok.shape[0]
    D = x.shape[1]
    dk = (wk_h if wk_h is not None else wq_h).shape[0]
    dv = wv_h.shape[0] if wv_h is not None else 1
    q = np.empty((n, dk)) if wq_h is not None else None
    k = np.empty((n, dk)) if wk_h is not None else None
    v = np.empty((n, dv)) if wv_h is not None else None
    lib().oracle_project_head(ctypes.c_int64(n), _p(rows_tok), D, dk, dv, _p(x), _p(wq_h), _p(wk_h),
                              _p(wv_h), _p(q), _p(k), _p(v))
    return q, k, v


def segments_bwd(seg_off, seg_state, row_token, q, k, v, a, c, state0, d_o, dstate=None, n_state=None,
                 rule="gdn"):
    """Gradients of ``segments``: given dL/do (d_o [N][H][dv]) and dL/d(final
    state) (dstate [n_state][H][dk][dv], None = zeros), return a dict with
    dq [N][H][dk] (per row, as the query is used at that row), dk, dv, da, dc and
    dstate0 (dL/d(entering state)).  state0 None = zeros.  Each state slot may be
    used by at most one segment."""
    seg_off, seg_state, row_token = _i(seg_off), _i(seg_state), _i(row_token)
    q, k, v, a, c, state0, d_o, dstate = (_d(t) for t in (q, k, v, a, c, state0, d_o, dstate))
    N, H, dk = k.shape
    dv = v.shape[2]
    n_seg = seg_off.shape[0] - 1
    if n_state is None:
        n_state = (state0.shape[0] if state0 is not None else
                   dstate.shape[0] if dstate is not None else int(seg_state.max()) + 1)
    assert len(set(seg_state.tolist())) == n_seg, "a state slot may serve one segment only"
    res = dict(dq=np.zeros((N, H, dk)), dk=np.zeros((N, H, dk)), dv=np.zeros((N, H, dv)),
               da=np.zeros((N, H)), dc=np.zeros((N, H)), dstate0=np.empty((n_state, H, dk, dv)))
    lib().oracle_segments_bwd_rule(RULES[rule], n_seg, _p(seg_off), _p(seg_state), n_state, _p(row_token), H, dk,
                                   dv, _p(q), _p(k), _p(v), _p(a), _p(c), _p(state0), _p(d_o), _p(dstate),
                                   _p(res["dq"]), _p(res["dk"]), _p(res["dv"]), _p(res["da"]), _p(res["dc"]),
                                   _p(res["dstate0"]))
    return res


def combine_bwd(inv, w, o_routed, dout, n_rows=None):
    """Gradients of ``combine``: (d_routed [rows][H][dv] (rows no token reads are
    zero), d_shared [n][H][dv], dw [n][K])."""
    w, o_routed, dout = _d(w), _d(o_routed), _d(dout)
    inv = _i(inv)
    n, K = w.shape
    H, dv = dout.shape[1], dout.shape[2]
    rows = o_routed.shape[0] if n_rows is None else n_rows
    d_routed = np.zeros((rows, H, dv))
    d_shared = np.empty((n, H, dv))
    dw = np.empty((n, K))
    lib().oracle_combine_bwd(ctypes.c_int64(n), K, H, dv, _p(inv), _p(w), _p(o_routed), _p(dout), _p(d_routed),
                             _p(d_shared), _p(dw))
    return d_routed, d_shared, dw


def route_bwd(x, w_r, idx, w, dw):
    """Gradients of the router weights' loss with the top-k choice held fixed:
    (dx [n][D], dw_r [M][D], dbias [M])."""
    x, w_r, w, dw = _d(x), _d(w_r), _d(w), _d(dw)
    idx = _i(idx)
    n, D = x.shape
    M = w_r.shape[0]
    K = idx.shape[1]
    dx = np.empty((n, D))
    dwr = np.empty((M, D))
    db = np.empty(M)
    lib().oracle_route_bwd(ctypes.c_int64(n), D, M, K, _p(x), _p(w_r), _p(idx), _p(w), _p(dw), _p(dx), _p(dwr),
                           _p(db))
    return dx, dwr, db


def dispatch_bwd(idx, inv, M, d_alpha_p, d_beta_p, dq_rows):
    """The dispatch gathers in reverse: (d_alpha, d_beta [n][H][M+1], dq [n][H][dk])."""
    idx, inv = _i(idx), _i(inv)
    d_alpha_p, d_beta_p, dq_rows = _d(d_alpha_p), _d(d_beta_p), _d(dq_rows)
    n, K = idx.shape
    H, dk = dq_rows.shape[1], dq_rows.shape[2]
    da = np.empty((n, H, M + 1))
    db = np.empty((n, H, M + 1))
    dq = np.empty((n, H, dk))
    lib().oracle_dispatch_bwd(ctypes.c_int64(n), H, dk, M, K, _p(idx), _p(inv), _p(d_alpha_p), _p(d_beta_p),
                              _p(dq_rows), _p(da), _p(db), _p(dq))
    return da, db, dq


def layer_bwd(dims, x, w_r, bias, w_q, w_k, w_v, alpha, beta, dout, state0=None, dstate=None, rule="gdn"):
    """Gradients of the layer for the parts the layer's backward pass covers:
    combine, recurrence (all memories), dispatch gathers and router weights, the
    top-k choice held fixed.  Returns a dict with d_alpha, d_beta [NT][H][M+1],
    dq [NT][H][dk] (w.r.t. the projected queries), dk_rows/dv_rows (w.r.t. the
    packed projected keys and values), dx_router [NT][D] (the router's share of
    dx), dw_r [M][D], dbias [M], dstate0 [B][M+1][H][dk][dv], and the forward's
    routing (idx, w, seg_off, perm, inv) and packed rows for reference."""
    B, T, D, H, dk, dv, M, K = [int(v) for v in dims]
    NT, NR = B * T, B * T * K
    fw = layer(dims, x, w_r, bias, w_q, w_k, w_v, alpha, beta, state0=state0, want_qkv=True, rule=rule)
    idx, wgt = fw["idx"], fw["w"]
    seg_off, perm, inv = dispatch(idx, B, T, M)
    N = NR + NT
    # packed rows: k/v of (token, j) at inv[t][j], shared at NR + t; gates per row
    kp, vp = np.empty((N, H, dk)), np.empty((N, H, dv))
    ap, bp = np.empty((N, H)), np.empty((N, H))
    al = _d(alpha).reshape(NT, H, M + 1)
    be = _d(beta).reshape(NT, H, M + 1)
    for j in range(K):
        r = inv[:, j]
        kp[r], vp[r] = fw["k"][:, j], fw["v"][:, j]
        ap[r] = al[np.arange(NT), :, idx[:, j]]
        bp[r] = be[np.arange(NT), :, idx[:, j]]
    kp[NR:], vp[NR:] = fw["k"][:, K], fw["v"][:, K]
    ap[NR:], bp[NR:] = al[:, :, M], be[:, :, M]
    o_rows = np.zeros((N, H, dv))
    for j in range(K):
        o_rows[inv[:, j]] = fw["o_routed"][:, j]
    o_rows[NR:] = fw["o_shared"]
    d_rows, d_shared, dw = combine_bwd(inv, wgt, o_rows, dout, n_rows=N)
    d_rows[NR:] = d_shared
    n_seg = (M + 1) * B
    seg_state = np.array([(s % B) * (M + 1) + s // B for s in range(n_seg)], np.int32)
    S0 = None if state0 is None else _d(state0).reshape(B * (M + 1), H, dk, dv)
    dS = None if dstate is None else _d(dstate).reshape(B * (M + 1), H, dk, dv)
    g = segments_bwd(seg_off, seg_state, perm, fw["q"], kp, vp, ap, bp, S0, d_rows, dS, n_state=B * (M + 1),
                     rule=rule)
    da, db, dq = dispatch_bwd(idx, inv, M, g["da"], g["dc"], g["dq"])
    dx, dwr, dbias = route_bwd(x, w_r, idx, wgt, dw)
    return dict(d_alpha=da, d_beta=db, dq=dq, dk_rows=g["dk"], dv_rows=g["dv"], dx_router=dx, dw_r=dwr, dbias=dbias,
                dstate0=g["dstate0"].reshape(B, M + 1, H, dk, dv), idx=idx, w=wgt, seg_off=seg_off, perm=perm,
                inv=inv, dw=dw, d_rows=d_rows)
