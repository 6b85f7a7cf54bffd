"""Thin ctypes binding of libmom.so (argument marshalling only).

Every function named like a C entry point takes torch tensors that already
live on the GPU, passes their data pointers and the current HIP stream, and
raises MomError on a non-zero status.  No arithmetic of the layer happens in
Python: there is no CPU fallback, and a missing library raises at load time.

``MomLayer`` strings the entry points together for one layer forward or one
decode step, allocating its intermediates with torch (device memory only).
"""
from __future__ import annotations

import ctypes
import os

import torch

from .synth import LayerConfig

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmom.so")

DTYPE_F32, DTYPE_BF16 = 0, 1
WS_DISPATCH, WS_CHUNK, WS_ROUTE_BWD = 0, 1, 2


class MomError(RuntimeError):
    pass


class MomDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("B", "T", "D", "H", "dk", "dv", "M", "topk", "chunk", "dtype")]


_lib = None
_VP = ctypes.c_void_p
_I32 = ctypes.c_int32


def lib():
    """Load libmom.so (after torch, so both share torch's HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise MomError("libmom.so is not built (%s); run mixture_memories_recurrence_amd.build" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    D = ctypes.POINTER(MomDims)
    sigs = {
        "mom_route": [D, _VP, _VP, _VP, _VP, _VP, _VP],
        "mom_route_count": [D, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP],
        "mom_dispatch_counted": [D, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP],
        "mom_dispatch": [D, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP],
        "mom_dispatch_noalloc": [D] + [_VP] * 11,
        "mom_project": [D, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP],
        "mom_project_part": [D, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _VP],
        "mom_dispatch_part": [D, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _I32, _VP],
        "mom_dispatch_counted_part": [D, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t,
                                      _I32, _VP],
        "gdn_chunk_fwd": [D, _I32, _I32, _I32, _I32, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                          _VP, ctypes.c_size_t, _VP],
        "gla_chunk_fwd": [D, _I32, _I32, _I32, _I32, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                          _VP, ctypes.c_size_t, _VP],
        "gdn_chunk_bwd": [D, _I32, _I32, _I32, _I32] + [_VP] * 18 + [ctypes.c_size_t, _VP],
        "gla_chunk_bwd": [D, _I32, _I32, _I32, _I32] + [_VP] * 18 + [ctypes.c_size_t, _VP],
        "gdn_chunk_fwd_train": [D, _I32, _I32, _I32, _I32] + [_VP] * 12 + [ctypes.c_size_t, _VP],
        "gla_chunk_fwd_train": [D, _I32, _I32, _I32, _I32] + [_VP] * 12 + [ctypes.c_size_t, _VP],
        "gdn_chunk_bwd_saved": [D, _I32, _I32, _I32, _I32] + [_VP] * 18 + [ctypes.c_size_t, _VP],
        "gla_chunk_bwd_saved": [D, _I32, _I32, _I32, _I32] + [_VP] * 18 + [ctypes.c_size_t, _VP],
        "gdn_chunk_bwd_workspace_bytes": [D, _I32, _I32],
        "gdn_decode_step": [D, _I32, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP],
        "gla_decode_step": [D, _I32, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP],
        "gdn_decode_step_combined": [D, _I32] + [_VP] * 11,
        "gla_decode_step_combined": [D, _I32] + [_VP] * 11,
        "mom_combine": [D, _I32, _VP, _VP, _VP, _VP, _VP, _VP],
        "mom_combine_bwd": [D, _I32] + [_VP] * 8,
        "mom_route_bwd": [D] + [_VP] * 9 + [ctypes.c_size_t, _VP],
        "mom_dispatch_bwd": [D] + [_VP] * 9,
        "mom_workspace_bytes": [D, _I32],
        "gdn_chunk_workspace_bytes": [D, _I32, _I32],
        "mom_status_string": [_I32],
    }
    for name, args in sigs.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = _I32
    L.mom_workspace_bytes.restype = ctypes.c_size_t
    L.gdn_chunk_workspace_bytes.restype = ctypes.c_size_t
    L.gdn_chunk_bwd_workspace_bytes.restype = ctypes.c_size_t
    L.mom_status_string.restype = ctypes.c_char_p
    _lib = L
    return L


EXPORTS = ("mom_route", "mom_route_count", "mom_dispatch", "mom_dispatch_noalloc", "mom_dispatch_counted",
           "mom_dispatch_part", "mom_dispatch_counted_part",
           "mom_project", "mom_project_part", "gdn_chunk_fwd", "gla_chunk_fwd", "gdn_chunk_bwd", "gla_chunk_bwd",
           "gdn_chunk_fwd_train", "gla_chunk_fwd_train", "gdn_chunk_bwd_saved", "gla_chunk_bwd_saved",
           "gdn_decode_step", "gla_decode_step", "gdn_decode_step_combined", "gla_decode_step_combined",
           "mom_combine", "mom_combine_bwd", "mom_route_bwd", "mom_dispatch_bwd", "mom_workspace_bytes",
           "gdn_chunk_workspace_bytes", "gdn_chunk_bwd_workspace_bytes", "mom_status_string")


def dims_of(cfg: LayerConfig, B: int | None = None, T: int | None = None) -> MomDims:
    return MomDims(cfg.B if B is None else B, cfg.T if T is None else T, cfg.D, cfg.H, cfg.dk, cfg.dv, cfg.M,
                   cfg.K, cfg.chunk, DTYPE_BF16 if cfg.dtype == "bf16" else DTYPE_F32)


def _p(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise MomError("tensor is not on the GPU")
    if not t.is_contiguous():
        raise MomError("tensor is not contiguous")
    return _VP(t.data_ptr())


def _s(stream):
    return _VP(torch.cuda.current_stream().cuda_stream if stream is None else stream)


def _check(status, name):
    if status != 0:
        msg = lib().mom_status_string(status).decode()
        raise MomError("%s: %s (status %d)" % (name, msg, status))


def mom_route(dims, x, w_r, bias, idx, w, stream=None):
    _check(lib().mom_route(ctypes.byref(dims), _p(x), _p(w_r), _p(bias), _p(idx), _p(w), _s(stream)), "mom_route")


def mom_route_count(dims, x, w_r, bias, idx, w, ws, stream=None):
    """mom_route, also writing the dispatch's counts into ws for
    mom_dispatch_counted / mom_dispatch_counted_part."""
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().mom_route_count(ctypes.byref(dims), _p(x), _p(w_r), _p(bias), _p(idx), _p(w), _p(ws), nbytes,
                                 _s(stream)), "mom_route_count")


def mom_dispatch_counted(dims, idx, x, alpha, beta, seg_off, perm, inv, x_packed, alpha_p, beta_p, ws,
                         stream=None):
    """mom_dispatch reading the counts mom_route_count left in ws."""
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().mom_dispatch_counted(ctypes.byref(dims), _p(idx), _p(x), _p(alpha), _p(beta), _p(seg_off),
                                      _p(perm), _p(inv), _p(x_packed), _p(alpha_p), _p(beta_p), _p(ws), nbytes,
                                      _s(stream)), "mom_dispatch_counted")


def mom_dispatch(dims, idx, x, alpha, beta, seg_off, perm, inv, x_packed, alpha_p, beta_p, ws, stream=None):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().mom_dispatch(ctypes.byref(dims), _p(idx), _p(x), _p(alpha), _p(beta), _p(seg_off), _p(perm),
                              _p(inv), _p(x_packed), _p(alpha_p), _p(beta_p), _p(ws), nbytes, _s(stream)),
           "mom_dispatch")


def mom_dispatch_noalloc(dims, idx, x, alpha, beta, seg_off, perm, inv, x_packed, alpha_p, beta_p, stream=None):
    """mom_dispatch with the library's fixed scratch instead of a workspace (no
    allocation; calls that overlap on one GPU race)."""
    _check(lib().mom_dispatch_noalloc(ctypes.byref(dims), _p(idx), _p(x), _p(alpha), _p(beta), _p(seg_off),
                                      _p(perm), _p(inv), _p(x_packed), _p(alpha_p), _p(beta_p), _s(stream)),
           "mom_dispatch_noalloc")


PART_ALL, PART_SHARED, PART_ROUTED = 0, 1, 2


def mom_dispatch_part(dims, idx, x, alpha, beta, seg_off, perm, inv, x_packed, alpha_p, beta_p, ws, part,
                      stream=None):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().mom_dispatch_part(ctypes.byref(dims), _p(idx), _p(x), _p(alpha), _p(beta), _p(seg_off), _p(perm),
                                   _p(inv), _p(x_packed), _p(alpha_p), _p(beta_p), _p(ws), nbytes, part, _s(stream)),
           "mom_dispatch_part")


def mom_dispatch_counted_part(dims, idx, x, alpha, beta, seg_off, perm, inv, x_packed, alpha_p, beta_p, ws, part,
                              stream=None):
    """mom_dispatch_part reading the counts mom_route_count left in ws."""
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().mom_dispatch_counted_part(ctypes.byref(dims), _p(idx), _p(x), _p(alpha), _p(beta), _p(seg_off),
                                           _p(perm), _p(inv), _p(x_packed), _p(alpha_p), _p(beta_p), _p(ws), nbytes,
                                           part, _s(stream)), "mom_dispatch_counted_part")


def mom_project_part(dims, x, perm, seg_off, w_q, w_k, w_v, q, k, v, part, stream=None):
    _check(lib().mom_project_part(ctypes.byref(dims), _p(x), _p(perm), _p(seg_off), _p(w_q), _p(w_k), _p(w_v),
                                  _p(q), _p(k), _p(v), part, _s(stream)), "mom_project_part")


def mom_project(dims, x, perm, seg_off, w_q, w_k, w_v, q, k, v, stream=None):
    _check(lib().mom_project(ctypes.byref(dims), _p(x), _p(perm), _p(seg_off), _p(w_q), _p(w_k), _p(w_v), _p(q),
                             _p(k), _p(v), _s(stream)), "mom_project")


def gdn_chunk_fwd(dims, n_seg, n_rows, n_tok, n_state, seg_off, seg_state, row_token, q, k, v, alpha_p, beta_p,
                  state_in, state_out, o, ws=None, stream=None):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().gdn_chunk_fwd(ctypes.byref(dims), n_seg, n_rows, n_tok, n_state, _p(seg_off), _p(seg_state),
                               _p(row_token), _p(q), _p(k), _p(v), _p(alpha_p), _p(beta_p), _p(state_in),
                               _p(state_out), _p(o), _p(ws), nbytes, _s(stream)), "gdn_chunk_fwd")


def gla_chunk_fwd(dims, n_seg, n_rows, n_tok, n_state, seg_off, seg_state, row_token, q, k, v, alpha_p, beta_p,
                  state_in, state_out, o, ws=None, stream=None):
    """As gdn_chunk_fwd, for gated linear attention memories (S <- a S + c k v^T)."""
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().gla_chunk_fwd(ctypes.byref(dims), n_seg, n_rows, n_tok, n_state, _p(seg_off), _p(seg_state),
                               _p(row_token), _p(q), _p(k), _p(v), _p(alpha_p), _p(beta_p), _p(state_in),
                               _p(state_out), _p(o), _p(ws), nbytes, _s(stream)), "gla_chunk_fwd")


def chunk_fwd_train(rule, dims, n_seg, n_rows, n_tok, n_state, seg_off, seg_state, row_token, q, k, v, alpha_p,
                    beta_p, state_in, state_out, o, ws, stream=None):
    """gdn_chunk_fwd_train (rule "gdn") or gla_chunk_fwd_train (rule "gla"): the
    forward's outputs, and ws (gdn_chunk_bwd_workspace_bytes) keeps its chunk
    factors and states for chunk_bwd_saved."""
    name = {"gdn": "gdn_chunk_fwd_train", "gla": "gla_chunk_fwd_train"}[rule]
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(getattr(lib(), name)(ctypes.byref(dims), n_seg, n_rows, n_tok, n_state, _p(seg_off), _p(seg_state),
                                _p(row_token), _p(q), _p(k), _p(v), _p(alpha_p), _p(beta_p), _p(state_in),
                                _p(state_out), _p(o), _p(ws), nbytes, _s(stream)), name)


def chunk_bwd_saved(rule, dims, n_seg, n_rows, n_tok, n_state, seg_off, seg_state, row_token, q, k, v, alpha_p,
                    beta_p, state_in, d_o, dstate_out, dq, dk, dv, d_alpha, d_beta, dstate_in, ws, stream=None):
    """gdn_chunk_bwd_saved / gla_chunk_bwd_saved: the gradients, from the ws a
    chunk_fwd_train call of the same rule and inputs left."""
    name = {"gdn": "gdn_chunk_bwd_saved", "gla": "gla_chunk_bwd_saved"}[rule]
    _chunk_bwd(name, dims, n_seg, n_rows, n_tok, n_state, seg_off, seg_state, row_token, q, k, v, alpha_p, beta_p,
               state_in, d_o, dstate_out, dq, dk, dv, d_alpha, d_beta, dstate_in, ws, stream)


def _chunk_bwd(name, dims, n_seg, n_rows, n_tok, n_state, seg_off, seg_state, row_token, q, k, v, alpha_p, beta_p,
               state_in, d_o, dstate_out, dq, dk, dv, d_alpha, d_beta, dstate_in, ws, stream):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(getattr(lib(), name)(ctypes.byref(dims), n_seg, n_rows, n_tok, n_state, _p(seg_off), _p(seg_state),
                                _p(row_token), _p(q), _p(k), _p(v), _p(alpha_p), _p(beta_p), _p(state_in), _p(d_o),
                                _p(dstate_out), _p(dq), _p(dk), _p(dv), _p(d_alpha), _p(d_beta), _p(dstate_in),
                                _p(ws), nbytes, _s(stream)), name)


def gdn_chunk_bwd(dims, n_seg, n_rows, n_tok, n_state, seg_off, seg_state, row_token, q, k, v, alpha_p, beta_p,
                  state_in, d_o, dstate_out, dq, dk, dv, d_alpha, d_beta, dstate_in, ws, stream=None):
    """Gradients of gdn_chunk_fwd: dq (per row), dk, dv, d_alpha, d_beta, dstate_in."""
    _chunk_bwd("gdn_chunk_bwd", dims, n_seg, n_rows, n_tok, n_state, seg_off, seg_state, row_token, q, k, v,
               alpha_p, beta_p, state_in, d_o, dstate_out, dq, dk, dv, d_alpha, d_beta, dstate_in, ws, stream)


def gla_chunk_bwd(dims, n_seg, n_rows, n_tok, n_state, seg_off, seg_state, row_token, q, k, v, alpha_p, beta_p,
                  state_in, d_o, dstate_out, dq, dk, dv, d_alpha, d_beta, dstate_in, ws, stream=None):
    """Gradients of gla_chunk_fwd (same arguments as gdn_chunk_bwd)."""
    _chunk_bwd("gla_chunk_bwd", dims, n_seg, n_rows, n_tok, n_state, seg_off, seg_state, row_token, q, k, v,
               alpha_p, beta_p, state_in, d_o, dstate_out, dq, dk, dv, d_alpha, d_beta, dstate_in, ws, stream)


def gdn_chunk_bwd_workspace_bytes(dims, n_seg, n_rows):
    return int(lib().gdn_chunk_bwd_workspace_bytes(ctypes.byref(dims), n_seg, n_rows))


def gdn_decode_step(dims, n_seq, idx, inv, q, k, v, alpha, beta, states, o, stream=None):
    _check(lib().gdn_decode_step(ctypes.byref(dims), n_seq, _p(idx), _p(inv), _p(q), _p(k), _p(v), _p(alpha),
                                 _p(beta), _p(states), _p(o), _s(stream)), "gdn_decode_step")


def decode_step_combined(rule, dims, n_seq, idx, inv, w, q, k, v, alpha, beta, states, out, stream=None):
    """gdn_decode_step_combined (rule "gdn") or gla_decode_step_combined: the
    decode step with the combine folded in; out [n_seq, H, dv] fp32."""
    name = {"gdn": "gdn_decode_step_combined", "gla": "gla_decode_step_combined"}[rule]
    _check(getattr(lib(), name)(ctypes.byref(dims), n_seq, _p(idx), _p(inv), _p(w), _p(q), _p(k), _p(v), _p(alpha),
                                _p(beta), _p(states), _p(out), _s(stream)), name)


def gla_decode_step(dims, n_seq, idx, inv, q, k, v, alpha, beta, states, o, stream=None):
    """As gdn_decode_step, for gated linear attention memories."""
    _check(lib().gla_decode_step(ctypes.byref(dims), n_seq, _p(idx), _p(inv), _p(q), _p(k), _p(v), _p(alpha),
                                 _p(beta), _p(states), _p(o), _s(stream)), "gla_decode_step")


def mom_combine(dims, n_tok, inv, w, o_routed, o_shared, out, stream=None):
    _check(lib().mom_combine(ctypes.byref(dims), n_tok, _p(inv), _p(w), _p(o_routed), _p(o_shared), _p(out),
                             _s(stream)), "mom_combine")


def mom_combine_bwd(dims, n_tok, inv, w, o_routed, dout, d_o_routed, d_o_shared, dw, stream=None):
    _check(lib().mom_combine_bwd(ctypes.byref(dims), n_tok, _p(inv), _p(w), _p(o_routed), _p(dout), _p(d_o_routed),
                                 _p(d_o_shared), _p(dw), _s(stream)), "mom_combine_bwd")


def mom_route_bwd(dims, x, w_r, idx, w, dw, dx, dw_r, dbias, ws, stream=None):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().mom_route_bwd(ctypes.byref(dims), _p(x), _p(w_r), _p(idx), _p(w), _p(dw), _p(dx), _p(dw_r),
                               _p(dbias), _p(ws), nbytes, _s(stream)), "mom_route_bwd")


def mom_dispatch_bwd(dims, idx, inv, d_alpha_p, d_beta_p, dq_rows, d_alpha, d_beta, dq, stream=None):
    _check(lib().mom_dispatch_bwd(ctypes.byref(dims), _p(idx), _p(inv), _p(d_alpha_p), _p(d_beta_p), _p(dq_rows),
                                  _p(d_alpha), _p(d_beta), _p(dq), _s(stream)), "mom_dispatch_bwd")


def mom_workspace_bytes(dims, which):
    return int(lib().mom_workspace_bytes(ctypes.byref(dims), which))


def gdn_chunk_workspace_bytes(dims, n_seg, n_rows):
    return int(lib().gdn_chunk_workspace_bytes(ctypes.byref(dims), n_seg, n_rows))


def chunk_workspace(dims, n_seg, n_rows, device="cuda"):
    """A device buffer large enough for gdn_chunk_fwd (None when none is needed)."""
    n = gdn_chunk_workspace_bytes(dims, n_seg, n_rows)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


# ---------------------------------------------------------------- layer driver
def storage_dtype(cfg):
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def act_dtype(cfg):
    """Storage of q/k/v between the projection and the recurrence."""
    return torch.float16 if cfg.dtype == "bf16" else torch.float32


_AUX_STREAMS = {}


def _aux_streams(device):
    """The two extra streams every layer on this device shares, drawn once per
    process.  torch hands out its pooled streams round-robin, and the pool's
    streams share the GPU's few hardware queues (four by default) round-robin
    too, so every fourth stream drawn shares a queue with the default stream:
    a new pair per layer would, after a few layers, put a layer's second
    stream behind the first and run its two halves one after the other."""
    d = torch.device(device)
    key = d.index if d.index is not None else torch.cuda.current_device()
    if key not in _AUX_STREAMS:
        _AUX_STREAMS[key] = (torch.cuda.Stream(device=key), torch.cuda.Stream(device=key))
    return _AUX_STREAMS[key]


class MomLayer:
    """One MoM layer on the GPU: weights resident, intermediates allocated once
    per (B, T).  forward() and decode_step() only enqueue library calls."""

    def __init__(self, cfg: LayerConfig, w_r, bias, w_q, w_k, w_v, device="cuda", rule="gdn"):
        """rule: "gdn" (Gated DeltaNet memories) or "gla" (gated linear attention)."""
        if rule not in ("gdn", "gla"):
            raise MomError("unknown update rule %r" % rule)
        self.cfg = cfg
        self.rule = rule
        sd = storage_dtype(cfg)
        t = lambda a, dt: None if a is None else torch.as_tensor(a).to(device=device, dtype=dt).contiguous()
        self.w_r, self.w_q, self.w_k, self.w_v = t(w_r, sd), t(w_q, sd), t(w_k, sd), t(w_v, sd)
        self.bias = t(bias, torch.float32)
        self.device = device
        self._bufs = {}

    def buffers(self, B, T):
        key = (B, T)
        if key in self._bufs:
            return self._bufs[key]
        c, dev = self.cfg, self.device
        NT = B * T
        NR = NT * c.K
        N = NR + NT
        dims = dims_of(c, B, T)
        i32 = dict(dtype=torch.int32, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        ad = dict(dtype=act_dtype(c), device=dev)
        ws = max(mom_workspace_bytes(dims, WS_DISPATCH), 256)
        n_seg = (c.M + 1) * B
        seg_state = torch.tensor([(s % B) * (c.M + 1) + s // B for s in range(n_seg)], **i32)
        b = dict(
            dims=dims, B=B, NT=NT, NR=NR, N=N, n_seg=n_seg, seg_state=seg_state,
            # the shared memory's segments alone (rows NR + b T ..), for the overlapped forward
            seg_off_s=torch.tensor([NR + i * T for i in range(B + 1)], **i32),
            seg_state_s=seg_state[c.M * B:].clone(),
            ws_chunk_s=chunk_workspace(dims, B, N, dev),
            idx=torch.empty(NT, c.K, **i32), w=torch.empty(NT, c.K, **f32),
            seg_off=torch.empty(n_seg + 1, **i32), perm=torch.empty(N, **i32), inv=torch.empty(NT, c.K, **i32),
            alpha_p=torch.empty(N, c.H, **f32), beta_p=torch.empty(N, c.H, **f32),
            ws=torch.empty(ws, dtype=torch.uint8, device=dev),
            ws_chunk=chunk_workspace(dims, n_seg, N, dev),
            q=torch.empty(NT, c.H, c.dk, **ad), k=torch.empty(N, c.H, c.dk, **ad), v=torch.empty(N, c.H, c.dv, **ad),
            o=torch.empty(N, c.H, c.dv, **f32), out=torch.empty(NT, c.H, c.dv, **f32),
        )
        self._bufs[key] = b
        return b

    def route_dispatch_project(self, x, alpha, beta, b, stream=None):
        c, d = self.cfg, b["dims"]
        mom_route_count(d, x, self.w_r, self.bias, b["idx"], b["w"], b["ws"], stream)
        mom_dispatch_counted(d, b["idx"], x, alpha, beta, b["seg_off"], b["perm"], b["inv"], None, b["alpha_p"],
                             b["beta_p"], b["ws"], stream)
        mom_project(d, x, b["perm"], b["seg_off"], self.w_q, self.w_k, self.w_v, b["q"], b["k"], b["v"], stream)

    def forward(self, x, alpha, beta, state_in=None, state_out=None, B=None, T=None, stream=None, overlap=True,
                train=False):
        """x [B*T, D], alpha/beta [B*T, H, M+1]; state_in/out [B, M+1, H, dk, dv] fp32.
        Returns (out [B*T, H, dv] fp32, state_out, buffers).

        train: the recurrence runs as chunk_fwd_train (same outputs, bit for
        bit) and keeps its chunk factors and states for the next backward(),
        which then skips recomputing them.

        overlap (default, on the current stream): the shared memory needs no
        routing, so its rows, the queries with its keys and values, and its
        recurrence run on a second stream while the main stream routes and
        dispatches; the routed projection follows the shared one (so the shared
        recurrence runs beside it), then the routed recurrence; the combine
        waits for both.  Otherwise (or with an explicit
        stream) the same steps run in order on one stream."""
        c = self.cfg
        B = c.B if B is None else B
        T = c.T if T is None else T
        b = self.buffers(B, T)
        if state_out is None:
            state_out = torch.empty(B, c.M + 1, c.H, c.dk, c.dv, dtype=torch.float32, device=self.device)
        b["saved"] = None  # the forward overwrites what a saved pass read
        if overlap and stream is None:
            return self._forward_overlapped(x, alpha, beta, b, state_in, state_out, train)
        self.route_dispatch_project(x, alpha, beta, b, stream)
        args = (b["dims"], b["n_seg"], b["N"], b["NT"], B * (c.M + 1), b["seg_off"], b["seg_state"], b["perm"],
                b["q"], b["k"], b["v"], b["alpha_p"], b["beta_p"], state_in, state_out, b["o"])
        if train:
            chunk_fwd_train(self.rule, *args, self._grad_bufs(b)["ws"], stream)
            b["saved"] = "all"
        else:
            (gdn_chunk_fwd if self.rule == "gdn" else gla_chunk_fwd)(*args, b["ws_chunk"], stream)
        mom_combine(b["dims"], b["NT"], b["inv"], b["w"], b["o"], b["o"][b["NR"]:], b["out"], stream)
        return b["out"], state_out, b

    def _forward_overlapped(self, x, alpha, beta, b, state_in, state_out, train=False):
        c, d = self.cfg, b["dims"]
        B, N, NT = b["B"], b["N"], b["NT"]
        n_state = B * (c.M + 1)
        if train:
            g = self._grad_bufs(b, split=True)
            chunk = lambda *a: chunk_fwd_train(self.rule, *a)
            ws_r, ws_s = g["ws"], g["ws_s"]
        else:
            chunk = gdn_chunk_fwd if self.rule == "gdn" else gla_chunk_fwd
            ws_r, ws_s = b["ws_chunk"], b["ws_chunk_s"]
        main = torch.cuda.current_stream()
        side, ev = self._side_stream()
        ev[0].record(main)  # inputs ready
        side.wait_event(ev[0])
        s = side.cuda_stream
        mom_dispatch_part(d, None, x, alpha, beta, b["seg_off"], b["perm"], None, None, b["alpha_p"], b["beta_p"],
                          None, PART_SHARED, s)
        mom_project_part(d, x, None, None, self.w_q, self.w_k, self.w_v, b["q"], b["k"], b["v"], PART_SHARED, s)
        ev[1].record(side)  # queries ready
        chunk(d, B, N, NT, n_state, b["seg_off_s"], b["seg_state_s"], b["perm"], b["q"], b["k"], b["v"], b["alpha_p"],
              b["beta_p"], state_in, state_out, b["o"], ws_s, s)
        ev[2].record(side)  # shared memory done
        mom_route_count(d, x, self.w_r, self.bias, b["idx"], b["w"], b["ws"])
        mom_dispatch_counted_part(d, b["idx"], x, alpha, beta, b["seg_off"], b["perm"], b["inv"], None,
                                  b["alpha_p"], b["beta_p"], b["ws"], PART_ROUTED)
        # the routed projection starts when the shared one is done, so that the
        # shared recurrence (a few long chains) runs beside it, not behind it
        main.wait_event(ev[1])
        mom_project_part(d, x, b["perm"], b["seg_off"], self.w_q, self.w_k, self.w_v, b["q"], b["k"], b["v"],
                         PART_ROUTED)
        chunk(d, c.M * B, N, NT, n_state, b["seg_off"], b["seg_state"], b["perm"], b["q"], b["k"], b["v"],
              b["alpha_p"], b["beta_p"], state_in, state_out, b["o"], ws_r)
        main.wait_event(ev[2])
        mom_combine(d, NT, b["inv"], b["w"], b["o"], b["o"][b["NR"]:], b["out"])
        if train:
            b["saved"] = "split"
        return b["out"], state_out, b

    def _side_stream(self):
        """The second stream (default priority, one per device for the whole
        process) and this layer's events."""
        if getattr(self, "_ev", None) is None:
            self._ev = [torch.cuda.Event() for _ in range(7)]
        return _aux_streams(self.device)[0], self._ev

    def _third_stream(self):
        """A third stream (default priority, one per device for the whole
        process), for the router's gradients."""
        return _aux_streams(self.device)[1]

    def _grad_bufs(self, b, split=False):
        """Gradient buffers of shape b; ws serves the recompute backward, the
        training forward over all segments, or (split) its routed call, and
        ws_s its shared call (chunk slots are counted per call)."""
        c = self.cfg
        if "grad" not in b:
            dev, f32 = self.device, torch.float32
            N, H = b["N"], c.H
            nbytes = gdn_chunk_bwd_workspace_bytes(b["dims"], b["n_seg"], N)
            b["grad"] = dict(dq=torch.empty(N, H, c.dk, dtype=f32, device=dev),
                             dk=torch.empty(N, H, c.dk, dtype=f32, device=dev),
                             dv=torch.empty(N, H, c.dv, dtype=f32, device=dev),
                             d_alpha=torch.empty(N, H, dtype=f32, device=dev),
                             d_beta=torch.empty(N, H, dtype=f32, device=dev),
                             dstate_in=torch.empty(b["n_seg"], H, c.dk, c.dv, dtype=f32, device=dev),
                             ws=torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev))
        g = b["grad"]
        if split and "ws_s" not in g:
            nbytes = gdn_chunk_bwd_workspace_bytes(b["dims"], b["B"], b["N"])
            g["ws_s"] = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        return g

    def chunk_backward(self, b, d_o, dstate_out=None, state_in=None, stream=None):
        """Gradients of the memories' recurrence over the segments of the last
        forward with buffers b: d_o [N, H, dv] fp32 = dL/do per packed row,
        dstate_out [B, M+1, H, dk, dv] fp32 or None (zeros), state_in as given to
        forward.  Returns a dict of dq [N, H, dk] (per row), dk, dv, d_alpha,
        d_beta [N, H] and dstate_in, all fp32 (buffers reused per shape).
        After a train=True forward it reads the factors and states that forward
        kept (once: the next call recomputes them)."""
        g = self._grad_bufs(b)
        saved, b["saved"] = b.get("saved"), None
        if saved == "split":  # routed and shared segments, as the overlapped forward ran them
            self._chunk_bwd_call(b, PART_ROUTED, True, d_o, dstate_out, state_in, stream)
            self._chunk_bwd_call(b, PART_SHARED, True, d_o, dstate_out, state_in, stream)
        else:
            self._chunk_bwd_call(b, PART_ALL, saved == "all", d_o, dstate_out, state_in, stream)
        return g

    def _chunk_bwd_call(self, b, part, saved, d_o, dstate_out, state_in, stream):
        """One recurrence-gradient call over the routed segments, the shared
        memory's, or all; from the saved factors or recomputing them."""
        g, n_state = b["grad"], b["n_seg"]
        if part == PART_SHARED:
            n, off, st, ws = b["B"], b["seg_off_s"], b["seg_state_s"], g["ws_s"]
        else:
            n = n_state - b["B"] if part == PART_ROUTED else n_state
            off, st, ws = b["seg_off"], b["seg_state"], g["ws"]
        args = (b["dims"], n, b["N"], b["NT"], n_state, off, st, b["perm"], b["q"], b["k"], b["v"], b["alpha_p"],
                b["beta_p"], state_in, d_o, dstate_out, g["dq"], g["dk"], g["dv"], g["d_alpha"], g["d_beta"],
                g["dstate_in"], ws, stream)
        if saved:
            chunk_bwd_saved(self.rule, *args)
        else:
            (gdn_chunk_bwd if self.rule == "gdn" else gla_chunk_bwd)(*args)

    def backward(self, x, dout, b, dstate_out=None, state_in=None, stream=None):
        """Gradients of the layer's last forward (buffers b, input x) for the
        parts its backward pass covers: combine, the memories' recurrence, the
        dispatch gathers and the router weights (top-k held fixed).  dout
        [B*T, H, dv] fp32 = dL/dout; dstate_out = dL/d(final states) or None.
        Returns a dict (buffers reused per shape) of d_alpha, d_beta [B*T, H, M+1],
        dq [B*T, H, dk] (w.r.t. the projected queries), dk, dv [N, H, dk|dv]
        (w.r.t. the packed projected keys and values), dx_router [B*T, D] (the
        router's share of dL/dx), dw_r [M, D], dbias [M], dstate_in.

        Without an explicit stream the router's gradients run on a third stream
        beside the recurrence's, and after a train=True forward on two streams
        the shared memory's recurrence gradients run on the second; the current
        stream waits for both before the dispatch gradients, so the results are
        ordered on it.  With a stream everything runs in order on that stream."""
        c, d = self.cfg, b["dims"]
        if "lgrad" not in b:
            dev, f32 = self.device, torch.float32
            NT, N, H = b["NT"], b["N"], c.H
            b["lgrad"] = dict(d_o=torch.empty(N, H, c.dv, dtype=f32, device=dev),
                              dw=torch.empty(NT, c.K, dtype=f32, device=dev),
                              d_alpha=torch.empty(NT, H, c.M + 1, dtype=f32, device=dev),
                              d_beta=torch.empty(NT, H, c.M + 1, dtype=f32, device=dev),
                              dq=torch.empty(NT, H, c.dk, dtype=f32, device=dev),
                              dx_router=torch.empty(NT, c.D, dtype=f32, device=dev),
                              dw_r=torch.empty(c.M, c.D, dtype=f32, device=dev),
                              dbias=torch.empty(c.M, dtype=f32, device=dev),
                              ws=torch.empty(max(mom_workspace_bytes(d, WS_ROUTE_BWD), 256), dtype=torch.uint8,
                                             device=dev))
        lg = b["lgrad"]
        mom_combine_bwd(d, b["NT"], b["inv"], b["w"], b["o"], dout, lg["d_o"], lg["d_o"][b["NR"]:], lg["dw"], stream)
        route = lambda s: mom_route_bwd(d, x, self.w_r, b["idx"], b["w"], lg["dw"], lg["dx_router"], lg["dw_r"],
                                        lg["dbias"], lg["ws"], s)
        if b.get("saved") == "split" and stream is None:
            # after an overlapped training forward: the shared memory's
            # recurrence gradients (a few long walks that fill few CUs) run on
            # the second stream beside the routed memories', and the router's
            # (which need only dL/dw) on a third from the start
            b["saved"] = None
            g = b["grad"]
            main = torch.cuda.current_stream()
            side, ev = self._side_stream()
            side2 = self._third_stream()
            ev[3].record(main)  # dL/do and dL/dw ready
            side.wait_event(ev[3])
            side2.wait_event(ev[3])
            route(side2.cuda_stream)
            ev[5].record(side2)
            self._chunk_bwd_call(b, PART_SHARED, True, lg["d_o"], dstate_out, state_in, side.cuda_stream)
            ev[4].record(side)
            self._chunk_bwd_call(b, PART_ROUTED, True, lg["d_o"], dstate_out, state_in, None)
            main.wait_event(ev[4])
            main.wait_event(ev[5])
        elif stream is None:
            # the router's gradients (which need only dL/dw) beside the recurrence's
            main = torch.cuda.current_stream()
            side2 = self._third_stream()
            _, ev = self._side_stream()
            ev[3].record(main)
            side2.wait_event(ev[3])
            route(side2.cuda_stream)
            ev[5].record(side2)
            g = self.chunk_backward(b, lg["d_o"], dstate_out, state_in)
            main.wait_event(ev[5])
        else:
            g = self.chunk_backward(b, lg["d_o"], dstate_out, state_in, stream)
            route(stream)
        mom_dispatch_bwd(d, b["idx"], b["inv"], g["d_alpha"], g["d_beta"], g["dq"], lg["d_alpha"], lg["d_beta"],
                         lg["dq"], stream)
        return dict(d_alpha=lg["d_alpha"], d_beta=lg["d_beta"], dq=lg["dq"], dk=g["dk"], dv=g["dv"],
                    dx_router=lg["dx_router"], dw_r=lg["dw_r"], dbias=lg["dbias"],
                    dstate_in=g["dstate_in"].view(-1, c.M + 1, c.H, c.dk, c.dv))

    def decode_step(self, x_t, alpha, beta, states, stream=None):
        """One token for each of n_seq sequences: x_t [n_seq, D], alpha/beta
        [n_seq, H, M+1], states [n_seq, M+1, H, dk, dv] updated in place."""
        n_seq = x_t.shape[0]
        b = self.buffers(n_seq, 1)
        d = b["dims"]
        # route and histogram in one launch, then the dispatch without its count
        mom_route_count(d, x_t, self.w_r, self.bias, b["idx"], b["w"], b["ws"], stream)
        mom_dispatch_counted(d, b["idx"], x_t, alpha, beta, b["seg_off"], b["perm"], b["inv"], None, b["alpha_p"],
                             b["beta_p"], b["ws"], stream)
        mom_project(d, x_t, b["perm"], b["seg_off"], self.w_q, self.w_k, self.w_v, b["q"], b["k"], b["v"], stream)
        # the recurrent step with the combine folded in (no per-memory outputs)
        decode_step_combined(self.rule, d, n_seq, b["idx"], b["inv"], b["w"], b["q"], b["k"], b["v"], alpha, beta,
                             states, b["out"], stream)
        return b["out"], b
