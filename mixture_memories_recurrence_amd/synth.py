"""Seeded synthetic inputs for the Mixture-of-Memories layer.

This module only draws random numbers and rounds them to the storage format
(fp32, or bfloat16 round-to-nearest-even).  It holds none of the layer's
arithmetic, so both the GPU path and the CPU reference checker can consume its
output without sharing any of the method's code.

Layouts (row-major):
  x      [B*T, D]           token t_g = b*T + t
  w_r    [M, D]             router weight, one row per memory
  bias   [M] fp32 or None   router bias
  w_q    [H*dk, D]          shared query projection
  w_k    [M+1, H*dk, D]     per-memory key projection (index M = shared memory)
  w_v    [M+1, H*dv, D]     per-memory value projection
  alpha  [B*T, H, M+1] fp32 forget gate in [0.9, 1)
  beta   [B*T, H, M+1] fp32 write strength in [0, 1)
Draw order: x, w_r, bias, w_q, w_k, w_v, alpha, beta.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    B: int
    T: int
    D: int
    H: int
    dk: int
    dv: int
    M: int
    K: int
    dtype: str = "bf16"          # "f32" or "bf16": storage of x and the weights
    bias: str = "none"           # "none" | "normal" | "zipf"
    chunk: int = 64
    name: str = ""

    @property
    def n_tok(self) -> int:
        return self.B * self.T

    @property
    def n_routed(self) -> int:
        return self.B * self.T * self.K

    @property
    def n_rows(self) -> int:
        return self.n_routed + self.n_tok


# The five workloads the layer is measured and checked on.
CONFIGS = {
    "tiny_f32": LayerConfig(1, 256, 256, 2, 64, 64, 4, 2, "f32", "none", 64, "tiny_f32"),
    "l380m": LayerConfig(8, 2048, 1024, 4, 128, 256, 4, 2, "bf16", "none", 64, "l380m"),
    "l1b3": LayerConfig(4, 4096, 2048, 8, 128, 256, 4, 2, "bf16", "normal", 64, "l1b3"),
    "m16": LayerConfig(4, 4096, 1024, 4, 128, 256, 16, 4, "bf16", "zipf", 64, "m16"),
    "long32k": LayerConfig(1, 32768, 2048, 8, 128, 256, 4, 2, "bf16", "none", 64, "long32k"),
}
# decode workload that follows the long-context prefill
DECODE_SEQS = 256

# One Gated DeltaNet memory whose value width equals the 380M layer's active
# state (k + 1 = 3 memories of 256 value columns): the single enlarged memory
# the pages compare the mixture with, with no router.
SINGLE_MEMORY = dict(B=8, T=2048, H=4, dk=128, dv=768)


def round_bf16(a: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bfloat16 (ties to even), returned as fp32 values."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of an array whose values are already bfloat16-exact."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("array holds values that are not bfloat16-exact")
    return (u >> 16).astype(np.uint16)


def _store(a: np.ndarray, dtype: str) -> np.ndarray:
    a = a.astype(np.float32)
    return round_bf16(a) if dtype == "bf16" else a


def make_layer_inputs(cfg: LayerConfig, seed: int = 0) -> dict:
    """Draw every input of one layer forward.  Float tensors are fp32 arrays whose
    values are exactly representable in cfg.dtype."""
    g = np.random.Generator(np.random.PCG64(seed))
    NT, D, H, M = cfg.n_tok, cfg.D, cfg.H, cfg.M
    sd = 1.0 / math.sqrt(D)
    x = _store(g.standard_normal((NT, D)), cfg.dtype)
    w_r = _store(g.standard_normal((M, D)) * sd, cfg.dtype)
    if cfg.bias == "none":
        bias = None
    elif cfg.bias == "normal":
        bias = g.standard_normal(M).astype(np.float32)
    elif cfg.bias == "zipf":
        # log of a Zipf(s=1.2) pmf over memory ranks, up to an additive constant
        bias = (-1.2 * np.log(np.arange(1, M + 1, dtype=np.float64))).astype(np.float32)
    else:
        raise ValueError(cfg.bias)
    w_q = _store(g.standard_normal((H * cfg.dk, D)) * sd, cfg.dtype)
    w_k = _store(g.standard_normal((M + 1, H * cfg.dk, D)) * sd, cfg.dtype)
    w_v = _store(g.standard_normal((M + 1, H * cfg.dv, D)) * sd, cfg.dtype)
    alpha = g.uniform(0.9, 1.0, (NT, H, M + 1)).astype(np.float32)
    beta = g.uniform(0.0, 1.0, (NT, H, M + 1)).astype(np.float32)
    return dict(x=x, w_r=w_r, bias=bias, w_q=w_q, w_k=w_k, w_v=w_v, alpha=alpha, beta=beta)


def make_state(cfg: LayerConfig, n_seq: int, seed: int = 1, scale: float = 0.1) -> np.ndarray:
    """A seeded fp32 state tensor [n_seq, M+1, H, dk, dv] ~ N(0, scale^2)."""
    g = np.random.Generator(np.random.PCG64(seed))
    shape = (n_seq, cfg.M + 1, cfg.H, cfg.dk, cfg.dv)
    return (g.standard_normal(shape, dtype=np.float32) * np.float32(scale)).astype(np.float32)


def make_decode_step_inputs(cfg: LayerConfig, n_seq: int, seed: int) -> dict:
    """Per-step decode inputs: one new token for each of n_seq sequences."""
    g = np.random.Generator(np.random.PCG64(seed))
    x = _store(g.standard_normal((n_seq, cfg.D)), cfg.dtype)
    alpha = g.uniform(0.9, 1.0, (n_seq, cfg.H, cfg.M + 1)).astype(np.float32)
    beta = g.uniform(0.0, 1.0, (n_seq, cfg.H, cfg.M + 1)).astype(np.float32)
    return dict(x=x, alpha=alpha, beta=beta)


def make_chain_inputs(n_rows: int, H: int, dk: int, dv: int, seed: int, store: str = "f16") -> dict:
    """Inputs of the per-memory recurrence alone, in packed-row order: q ~ N(0,1),
    keys ~ N(0, 1/dk) (squared norm close to 1, like the layer's normalised keys),
    values ~ N(0,1), gates as in the layer.  Values are exact in the given storage
    format ("f16" or "f32")."""
    g = np.random.Generator(np.random.PCG64(seed))
    q = g.standard_normal((n_rows, H, dk))
    k = g.standard_normal((n_rows, H, dk)) / math.sqrt(dk)
    v = g.standard_normal((n_rows, H, dv))
    alpha = g.uniform(0.9, 1.0, (n_rows, H)).astype(np.float32)
    beta = g.uniform(0.0, 1.0, (n_rows, H)).astype(np.float32)
    cast = np.float16 if store == "f16" else np.float32
    return dict(q=q.astype(cast).astype(np.float32), k=k.astype(cast).astype(np.float32),
                v=v.astype(cast).astype(np.float32), alpha=alpha, beta=beta)


def make_chain_grads(n_rows: int, H: int, dk: int, dv: int, n_state: int, seed: int) -> dict:
    """Upstream gradients for the recurrence's backward pass: d_o = dL/do [n_rows][H][dv]
    and dstate = dL/d(final state) [n_state][H][dk][dv], both N(0,1) float32 (the
    gradient of a loss that sums random projections of the outputs and states)."""
    g = np.random.Generator(np.random.PCG64(seed))
    return dict(d_o=g.standard_normal((n_rows, H, dv)).astype(np.float32),
                dstate=g.standard_normal((n_state, H, dk, dv)).astype(np.float32))


def make_single_memory_inputs(B: int, T: int, H: int, dk: int, dv: int, seed: int) -> dict:
    """Inputs of one plain Gated DeltaNet memory over B sequences of T tokens
    (rows in token order): q ~ N(0,1), keys normalised per head, values ~
    N(0,1), gates as in the layer.  q, k, v are exact in half precision."""
    g = np.random.Generator(np.random.PCG64(seed))
    n = B * T
    q = g.standard_normal((n, H, dk))
    k = g.standard_normal((n, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = g.standard_normal((n, H, dv))
    alpha = g.uniform(0.9, 1.0, (n, H)).astype(np.float32)
    beta = g.uniform(0.0, 1.0, (n, H)).astype(np.float32)
    h = lambda a: a.astype(np.float16).astype(np.float32)
    return dict(q=h(q), k=h(k), v=h(v), alpha=alpha, beta=beta)
