"""Seeded synthetic workloads for the gated delta rule operator.

This module only draws inputs. It holds none of the operator's arithmetic, so the
HIP path and the CPU oracle can both be fed from it without sharing any code that
computes the method.

Shapes and distributions of the five workloads (all seeded, all synthetic):

  id  name           shape                                        dtype (q,k,v,o)  h0 / state
  0   tiny_fp32      B=1 H=2  T=256   d_k=d_v=64   chunk 64         fp32             zero
  1   train_1p3b     B=4 H=16 T=2048  d_k=d_v=128  chunk 64         bf16             zero
  2   long_ctx       B=1 H=16 T=32768 d_k=d_v=128  chunk 64         bf16             N(0, 0.02^2)
  3   varlen_packed  8 sequences, lengths ~ U{512..8192}, H=32, d=128 bf16             zero
  4   decode         256 sequences x H=32, d=128, 64 chained steps  bf16             N(0, 0.02^2)

Per token and head: q, k ~ N(0,1) then L2-normalised over d_k; v ~ N(0,1);
g = log(alpha) = -softplus(N(0,1)) so alpha is in (0,1); beta = sigmoid(N(0,1)).
The gates and the state are always fp32. bf16 casts round to nearest even.

Draw order for a seed: [varlen lengths], q, k, v, g_raw, b_raw, [h0]; for the
decode workload: state first, then the per-step q, k, v, g_raw, b_raw stacked
over the 64 steps.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    id: int
    name: str
    H: int
    dk: int
    dv: int
    dtype: str                      # "f32" or "bf16": dtype of q, k, v and o
    B: int = 1
    T: int = 0                      # tokens per batch row (fixed-length workloads)
    chunk: int = 64
    h0: bool = False                # nonzero initial state drawn
    varlen: int = 0                 # number of packed sequences (0: fixed length)
    len_range: tuple = (0, 0)       # inclusive range of packed sequence lengths
    decode_seqs: int = 0            # decode workload: independent sequences
    decode_steps: int = 0           # decode workload: chained steps
    state_std: float = 0.02
    notes: str = field(default="", compare=False)


WORKLOADS = {
    0: Workload(0, "tiny_fp32", H=2, dk=64, dv=64, dtype="f32", B=1, T=256),
    1: Workload(1, "train_1p3b", H=16, dk=128, dv=128, dtype="bf16", B=4, T=2048),
    2: Workload(2, "long_ctx", H=16, dk=128, dv=128, dtype="bf16", B=1, T=32768, h0=True),
    3: Workload(3, "varlen_packed", H=32, dk=128, dv=128, dtype="bf16", varlen=8,
                len_range=(512, 8192)),
    4: Workload(4, "decode", H=32, dk=128, dv=128, dtype="bf16", decode_seqs=256,
                decode_steps=64, h0=True),
}


def _unit(x: np.ndarray) -> np.ndarray:
    """Scale each vector along the last axis to unit L2 norm (fp32, no epsilon)."""
    return x / np.sqrt(np.sum(x.astype(np.float32) ** 2, axis=-1, keepdims=True, dtype=np.float32))


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(np.float32(0.0), x).astype(np.float32)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x))).astype(np.float32)


def _cast(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def _token_tensors(rng, shape_qk, shape_v, shape_gate, dtype, gate_scale, beta_scale=1.0):
    q = rng.standard_normal(shape_qk, dtype=np.float32)
    k = rng.standard_normal(shape_qk, dtype=np.float32)
    v = rng.standard_normal(shape_v, dtype=np.float32)
    g_raw = rng.standard_normal(shape_gate, dtype=np.float32)
    b_raw = rng.standard_normal(shape_gate, dtype=np.float32)
    g = (-np.float32(gate_scale) * _softplus(g_raw)).astype(np.float32)
    beta = (np.float32(beta_scale) * _sigmoid(b_raw)).astype(np.float32)
    return dict(q=_cast(_unit(q), dtype), k=_cast(_unit(k), dtype), v=_cast(v, dtype),
                g=torch.from_numpy(g), beta=torch.from_numpy(beta))


def varlen_lengths(w: Workload, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    lo, hi = w.len_range
    return rng.integers(lo, hi, size=w.varlen, endpoint=True).astype(np.int64)


def make_forward_inputs(w: Workload | int, seed: int | None = None, *, T: int | None = None,
                        B: int | None = None, H: int | None = None, lengths=None,
                        gate_scale: float = 1.0, h0: bool | None = None,
                        dtype: str | None = None, beta_scale: float = 1.0) -> dict:
    """Draw one forward-pass input set.

    Returns CPU tensors: q, k [B,T,H,dk], v [B,T,H,dv] in the workload dtype; g, beta
    [B,T,H] fp32; h0 [N,H,dv,dk] fp32 or None; cu_seqlens int32 [N+1] or None.
    Overrides (T, B, H, lengths, dtype) shrink a workload for quick tests while
    keeping its distributions. `gate_scale` multiplies -softplus (0.01 gives slow decay);
    `beta_scale` multiplies the sigmoid (2 gives beta in (0, 2), the negative-eigenvalue range).
    """
    if isinstance(w, int):
        w = WORKLOADS[w]
    seed = w.id if seed is None else seed
    rng = np.random.default_rng(seed)
    H = w.H if H is None else H
    dtype = w.dtype if dtype is None else dtype
    if w.varlen or lengths is not None:
        if lengths is None:
            lo, hi = w.len_range
            lengths = rng.integers(lo, hi, size=w.varlen, endpoint=True)
        lengths = np.asarray(lengths, dtype=np.int64)
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
        Bn, Tn, N = 1, int(cu[-1]), len(lengths)
        cu_seqlens = torch.from_numpy(cu)
    else:
        Bn = w.B if B is None else B
        Tn = w.T if T is None else T
        N = Bn
        cu_seqlens = None
    out = _token_tensors(rng, (Bn, Tn, H, w.dk), (Bn, Tn, H, w.dv), (Bn, Tn, H), dtype, gate_scale,
                         beta_scale)
    want_h0 = w.h0 if h0 is None else h0
    out["h0"] = (torch.from_numpy((rng.standard_normal((N, H, w.dv, w.dk), dtype=np.float32)
                                   * np.float32(w.state_std)).astype(np.float32))
                 if want_h0 else None)
    out["cu_seqlens"] = cu_seqlens
    out["meta"] = dict(workload=w.name, B=Bn, T=Tn, H=H, dk=w.dk, dv=w.dv, N=N, dtype=dtype,
                       chunk=w.chunk, seed=seed, gate_scale=gate_scale, beta_scale=beta_scale,
                       lengths=None if cu_seqlens is None else [int(x) for x in np.diff(cu_seqlens.numpy())])
    return out


def make_decode_inputs(w: Workload | int = 4, seed: int | None = None, *, N: int | None = None,
                       H: int | None = None, steps: int | None = None,
                       dtype: str | None = None, beta_scale: float = 1.0) -> dict:
    """Draw the decode workload: fp32 state [N,H,dv,dk] and `steps` stacked token sets
    q, k [steps,N,H,dk], v [steps,N,H,dv] (workload dtype), g, beta [steps,N,H] fp32."""
    if isinstance(w, int):
        w = WORKLOADS[w]
    seed = w.id if seed is None else seed
    rng = np.random.default_rng(seed)
    N = w.decode_seqs if N is None else N
    H = w.H if H is None else H
    steps = w.decode_steps if steps is None else steps
    dtype = w.dtype if dtype is None else dtype
    state = (rng.standard_normal((N, H, w.dv, w.dk), dtype=np.float32) * np.float32(w.state_std))
    out = _token_tensors(rng, (steps, N, H, w.dk), (steps, N, H, w.dv), (steps, N, H), dtype, 1.0,
                         beta_scale)
    out["state"] = torch.from_numpy(state.astype(np.float32))
    out["meta"] = dict(workload=w.name, N=N, H=H, dk=w.dk, dv=w.dv, steps=steps, dtype=dtype, seed=seed)
    return out


def make_cotangents(x: dict, seed: int, *, dhT: bool = True) -> dict:
    """Gradients of a synthetic loss with respect to the forward outputs of input set x:
    dO [B,T,H,dv] ~ N(0,1) in the input dtype, dhT [N,H,dv,dk] ~ N(0,1) fp32 (or None)."""
    m = x["meta"]
    rng = np.random.default_rng(seed)
    do = _cast(rng.standard_normal((m["B"], m["T"], m["H"], m["dv"]), dtype=np.float32), m["dtype"])
    dh = (torch.from_numpy(rng.standard_normal((m["N"], m["H"], m["dv"], m["dk"]), dtype=np.float32))
          if dhT else None)
    return dict(do=do, dhT=dh)


def channel_gates(x: dict, seed: int, *, gate_scale: float = 1.0) -> dict:
    """Replace the scalar gates of an input set (forward or decode) by one gate per key
    channel, with the same distribution: g = -gate_scale * softplus(N(0,1)) of shape
    g.shape + (d_k,), drawn from its own seeded generator (the other tensors are unchanged)."""
    rng = np.random.default_rng(seed)
    dk = x["meta"]["dk"]
    shape = tuple(x["g"].shape) + (dk,)
    g = -np.float32(gate_scale) * _softplus(rng.standard_normal(shape, dtype=np.float32))
    y = dict(x)
    y["g"] = torch.from_numpy(g.astype(np.float32))
    y["meta"] = dict(x["meta"], channel_gate=True)
    return y


def decoupled_gates(x: dict, seed: int) -> dict:
    """Replace beta of a channel-gate input set (forward or decode) by an erase gate
    g.shape (one per key channel) and a write gate of shape beta.shape + (d_v,), both
    sigmoid(N(0,1)), drawn from their own seeded generator."""
    rng = np.random.default_rng(seed)
    m = x["meta"]
    y = dict(x)
    y["erase"] = torch.from_numpy(_sigmoid(rng.standard_normal(tuple(x["g"].shape), dtype=np.float32)))
    y["write"] = torch.from_numpy(_sigmoid(rng.standard_normal(tuple(x["beta"].shape) + (m["dv"],),
                                                               dtype=np.float32)))
    y["meta"] = dict(m, decoupled=True)
    return y
