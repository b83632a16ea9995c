"""CPU fp64 oracle of the gated delta rule with decoupled channel-wise erase and write gates on
top of a channel-wise decay, and a chunkwise model of it.

TEST INFRASTRUCTURE. Only the test suite, the package smoke check and the CPU baseline
leg of the benchmark may import or run anything in this directory. It shares no code
with the HIP library.

Sources: record "LIT-137: Gated Delta Networks" (anthology-of-the-sota), "Standing in the
anthology" (Gated DeltaNet-2 "splits beta into a channel-wise erase gate and a channel-wise
write gate on top of KDA's channel-wise decay, and reduces to this recurrence when all three
are tied to scalars"), and practice "SOTA-135", "Where it is incomplete" (the erase gate is
"on the key", the write gate "on the value", and "the erased read then runs along a
reweighted key rather than the key itself"). No formula is printed; the reading taken here:
with the channel-wise decay applied first (kda.py), the read that is erased runs along the
key reweighted by the erase gate e_t in [0,1]^{d_k}, the written value is weighted by the
write gate w_t in [0,1]^{d_v}, and both are stored along the key itself:

    Sa  = S_{t-1} Diag(alpha_t)
    S_t = Sa - (Sa (e_t * k_t)) k_t^T + (w_t * v_t) k_t^T,      o_t = S_t q_t

(literally S_t = S_{t-1} Diag(alpha_t) (I - (e_t * k_t) k_t^T) + (w_t * v_t) k_t^T). With
e_t = beta_t 1 and w_t = beta_t 1 it is the channel-wise-decay recurrence, and with scalar
decays the gated delta rule.

`chunk_forward` restates it chunk by chunk (derived as for kda.py; E = the erase gates,
W = the write gates, rows per token):
    A     = strict_lower([sum_c e_r k_r k_i e^{gamma_r - gamma_i}])
    T     = (I + A)^{-1}
    Delta = T (W * V - (E * K * e^gamma) S^T)
    O     = (Q * e^gamma) S^T + P Delta,   P = lower_incl([sum_c q_r k_i e^{gamma_r - gamma_i}])
    S'    = S Diag(e^{gamma_last}) + Delta^T (K * e^{gamma_last - gamma})

Parity pins: tests/test_decoupled_oracle.py.
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular

from .recurrence import _f64, segments


def step_heads(S, q, k, v, g, e, w):
    """One token for H heads: S [H,d_v,d_k]; q, k, g, e [H,d_k]; v, w [H,d_v]."""
    Sa = S * np.exp(g)[:, None, :]
    u = np.einsum("hvk,hk->hv", Sa, e * k)               # the erased read, along e * k
    S = Sa + (w * v - u)[:, :, None] * k[:, None, :]
    o = np.einsum("hvk,hk->hv", S, q)
    return S, o


def forward(q, k, v, g, erase, write, h0=None, cu_seqlens=None):
    """Token-by-token forward pass. q, k, g, erase [B,T,H,d_k]; v, write [B,T,H,d_v];
    h0 [N,H,d_v,d_k] or None; cu_seqlens [N+1] or None. Returns o, hT (fp64)."""
    q, k, v, g, erase, write, h0 = (_f64(x) for x in (q, k, v, g, erase, write, h0))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    segs = segments(B, T, cu_seqlens)
    if cu_seqlens is not None and B != 1:
        raise ValueError("packed sequences need B == 1")
    f = lambda x, d: x.reshape(B * T, H, d)  # noqa: E731
    qf, kf, gf, ef = f(q, dk), f(k, dk), f(g, dk), f(erase, dk)
    vf, wf = f(v, dv), f(write, dv)
    o = np.full((B * T, H, dv), np.nan)
    hT = np.zeros((len(segs), H, dv, dk))
    for n, (s0, s1) in enumerate(segs):
        S = np.zeros((H, dv, dk)) if h0 is None else h0[n].copy()
        for t in range(s0, s1):
            S, o[t] = step_heads(S, qf[t], kf[t], vf[t], gf[t], ef[t], wf[t])
        hT[n] = S
    return o.reshape(B, T, H, dv), hT


def decode(state, q, k, v, g, erase, write):
    """One decode step: state [N,H,d_v,d_k]; q, k, g, erase [N,H,d_k]; v, write [N,H,d_v]."""
    state, q, k, v, g, erase, write = (_f64(x) for x in (state, q, k, v, g, erase, write))
    N, H, dv, dk = state.shape
    r = lambda x, d: x.reshape(N * H, d)  # noqa: E731
    S, o = step_heads(state.reshape(N * H, dv, dk), r(q, dk), r(k, dk), r(v, dv), r(g, dk), r(erase, dk),
                      r(write, dv))
    return S.reshape(N, H, dv, dk), o.reshape(N, H, dv)


def _chunk(S, q, k, v, g, e, w):
    n = k.shape[0]
    gamma = np.cumsum(g, axis=0)
    diff = gamma[:, None, :] - gamma[None, :, :]
    low = np.tril(np.ones((n, n), dtype=bool))
    X = np.exp(np.where(low[:, :, None], diff, -np.inf))
    A = np.tril(np.einsum("rc,ic,ric->ri", e * k, k, X), k=-1)
    P = np.einsum("rc,ic,ric->ri", q, k, X)
    T = solve_triangular(np.eye(n) + A, np.eye(n), lower=True, unit_diagonal=True)
    Delta = T @ (w * v - (e * k * np.exp(gamma)) @ S.T)
    O = (q * np.exp(gamma)) @ S.T + P @ Delta
    S_next = S * np.exp(gamma[-1])[None, :] + Delta.T @ (k * np.exp(gamma[-1] - gamma))
    return O, S_next


def chunk_forward(q, k, v, g, erase, write, h0=None, cu_seqlens=None, chunk=64):
    """Same interface as `forward`, through the chunkwise restatement."""
    q, k, v, g, erase, write, h0 = (_f64(x) for x in (q, k, v, g, erase, write, h0))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    segs = segments(B, T, cu_seqlens)
    f = lambda x, d: x.reshape(B * T, H, d)  # noqa: E731
    qf, kf, gf, ef = f(q, dk), f(k, dk), f(g, dk), f(erase, dk)
    vf, wf = f(v, dv), f(write, dv)
    o = np.zeros((B * T, H, dv))
    hT = np.zeros((len(segs), H, dv, dk))
    for n, (s0, s1) in enumerate(segs):
        for h in range(H):
            S = np.zeros((dv, dk)) if h0 is None else h0[n, h].copy()
            for c0 in range(s0, s1, chunk):
                c1 = min(c0 + chunk, s1)
                sl = slice(c0, c1)
                o[sl, h], S = _chunk(S, qf[sl, h], kf[sl, h], vf[sl, h], gf[sl, h], ef[sl, h], wf[sl, h])
            hT[n, h] = S
    return o.reshape(B, T, H, dv), hT
