"""CPU fp64 oracle of the gated delta rule with a channel-wise decay (one decay per key
channel), and a chunkwise model of it.

TEST INFRASTRUCTURE. Only the test suite, the package smoke check and the CPU baseline
leg of the benchmark may import or run anything in this directory. It shares no code
with the HIP library.

Sources: record "LIT-137: Gated Delta Networks" (anthology-of-the-sota), "Standing in the
anthology" (Kimi Delta Attention extends the gated delta rule "with a channel-wise
forgetting gate"), and practice "SOTA-135", "Sequence" (it "replaces the scalar decay with a
channel-wise one"). The pages give no formula; the reading taken here is the plainest one:
the scalar alpha_t of the gated delta rule becomes a vector alpha_t in (0,1]^{d_k}, one decay
per key channel, applied where the scalar one was (to the old memory, before the write):

    S_t = S_{t-1} Diag(alpha_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = S_t q_t

with S [d_v, d_k] (its columns are the key channels). With alpha_t the same in every channel
it is the gated delta rule of recurrence.py.

`forward` evaluates the step as Sa = S Diag(alpha); S = Sa + beta (v - Sa k) k^T.

`chunk_forward` restates it chunk by chunk (derived here). With gamma_r = sum_{j<=r} g_j the
in-chunk cumulative log decay of every channel (a row vector), Kh = K * e^gamma,
Kc = K * e^-gamma, Qh = Q * e^gamma (elementwise, row r scaled by e^{gamma_r}) and
Kd = K * e^{gamma_last - gamma}:
    A     = strict_lower(diag(beta) Kh Kc^T)        (A[r,i] = beta_r sum_c k_r k_i e^{gamma_r - gamma_i})
    T     = (I + A)^{-1},   Mmat = T diag(beta)
    Delta = Mmat (V - Kh S^T)
    O     = Qh S^T + P Delta,   P = lower_incl(Qh Kc^T)
    S'    = S Diag(e^{gamma_last}) + Delta^T Kd
The model forms A and P from exp of the per-element differences directly (never from the
e^{-gamma} factor, which can overflow), as the exact sums over channels.

Parity pins: tests/test_kda_oracle.py.
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular

from .recurrence import _f64, segments


def step_heads(S, q, k, v, g, beta):
    """One token for H heads: S [H,d_v,d_k]; q, k, g [H,d_k] (g = log alpha per channel);
    v [H,d_v]; beta [H]."""
    Sa = S * np.exp(g)[:, None, :]                       # decay every key channel (column)
    u = np.einsum("hvk,hk->hv", Sa, k)
    S = Sa + beta[:, None, None] * (v - u)[:, :, None] * k[:, None, :]
    o = np.einsum("hvk,hk->hv", S, q)
    return S, o


def forward(q, k, v, g, beta, h0=None, cu_seqlens=None):
    """Token-by-token forward pass. q, k, g [B,T,H,d_k]; v [B,T,H,d_v]; beta [B,T,H];
    h0 [N,H,d_v,d_k] or None; cu_seqlens [N+1] or None (then N = B). Returns o, hT (fp64)."""
    q, k, v, g, beta, h0 = (_f64(x) for x in (q, k, v, g, beta, h0))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    segs = segments(B, T, cu_seqlens)
    if cu_seqlens is not None and B != 1:
        raise ValueError("packed sequences need B == 1")
    qf, kf, gf = q.reshape(B * T, H, dk), k.reshape(B * T, H, dk), g.reshape(B * T, H, dk)
    vf, bf = v.reshape(B * T, H, dv), beta.reshape(B * T, H)
    o = np.full((B * T, H, dv), np.nan)
    hT = np.zeros((len(segs), H, dv, dk))
    for n, (s0, s1) in enumerate(segs):
        S = np.zeros((H, dv, dk)) if h0 is None else h0[n].copy()
        for t in range(s0, s1):
            S, o[t] = step_heads(S, qf[t], kf[t], vf[t], gf[t], bf[t])
        hT[n] = S
    return o.reshape(B, T, H, dv), hT


def decode(state, q, k, v, g, beta):
    """One decode step: state [N,H,d_v,d_k]; q, k, g [N,H,d_k]; v [N,H,d_v]; beta [N,H]."""
    state, q, k, v, g, beta = (_f64(x) for x in (state, q, k, v, g, beta))
    N, H, dv, dk = state.shape
    S, o = step_heads(state.reshape(N * H, dv, dk), q.reshape(N * H, dk), k.reshape(N * H, dk),
                      v.reshape(N * H, dv), g.reshape(N * H, dk), beta.reshape(N * H))
    return S.reshape(N, H, dv, dk), o.reshape(N, H, dv)


def _chunk(S, q, k, v, g, beta):
    n = k.shape[0]
    gamma = np.cumsum(g, axis=0)                                    # [n, d_k]
    diff = gamma[:, None, :] - gamma[None, :, :]                    # [r, i, c] = gamma_r - gamma_i
    low = np.tril(np.ones((n, n), dtype=bool))
    W = np.exp(np.where(low[:, :, None], diff, -np.inf))            # masked before the exp
    KK = np.einsum("rc,ic,ric->ri", k, k, W)
    QK = np.einsum("rc,ic,ric->ri", q, k, W)
    A = np.tril(beta[:, None] * KK, k=-1)
    T = solve_triangular(np.eye(n) + A, np.eye(n), lower=True, unit_diagonal=True)
    Kh, Qh = k * np.exp(gamma), q * np.exp(gamma)
    Kd = k * np.exp(gamma[-1] - gamma)
    Delta = (T * beta[None, :]) @ (v - Kh @ S.T)
    O = Qh @ S.T + QK @ Delta
    S_next = S * np.exp(gamma[-1])[None, :] + Delta.T @ Kd
    return O, S_next


def chunk_forward(q, k, v, g, beta, h0=None, cu_seqlens=None, chunk=64):
    """Same interface as `forward`, through the chunkwise restatement."""
    q, k, v, g, beta, h0 = (_f64(x) for x in (q, k, v, g, beta, h0))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    segs = segments(B, T, cu_seqlens)
    qf, kf, gf = q.reshape(B * T, H, dk), k.reshape(B * T, H, dk), g.reshape(B * T, H, dk)
    vf, bf = v.reshape(B * T, H, dv), beta.reshape(B * T, H)
    o = np.zeros((B * T, H, dv))
    hT = np.zeros((len(segs), H, dv, dk))
    for n, (s0, s1) in enumerate(segs):
        for h in range(H):
            S = np.zeros((dv, dk)) if h0 is None else h0[n, h].copy()
            for c0 in range(s0, s1, chunk):
                c1 = min(c0 + chunk, s1)
                o[c0:c1, h], S = _chunk(S, qf[c0:c1, h], kf[c0:c1, h], vf[c0:c1, h], gf[c0:c1, h], bf[c0:c1, h])
            hT[n, h] = S
    return o.reshape(B, T, H, dv), hT
