"""CPU fp64 model of the chunkwise-parallel form of the gated delta rule (WY
representation / UT transform carrying the gate), one stage at a time.

TEST INFRASTRUCTURE. Only the test suite, the package smoke check and the CPU
baseline leg of the benchmark may import or run anything in this directory. It
shares no code with the HIP library.

Sources: the parallel training algorithm built on the WY representation and the UT
transform is named in the paper note "Gated Delta Networks: Improving Mamba2 with
Delta Rule" (phantomic12 inference-research), mechanism paragraph; record "LIT-137"
(anthology-of-the-sota), "Key takeaways" (second item) and "Standing in the
anthology" (the WY-based chunkwise algorithm, extended to carry the gate); practice
"SOTA-135", section "Source". The pages name the method but print no formulas for
it, so the chunk equations below are derived from the recurrence
S_t = alpha_t S_{t-1} + beta_t (v_t - alpha_t S_{t-1} k_t) k_t^T:

For one chunk of n tokens entering with state S (rows r, i = 0..n-1 of the chunk):
    gamma_r = sum_{j<=r} g_j                      (log of the running decay product)
    A[r,i]  = beta_r (k_r . k_i) exp(gamma_r - gamma_i)   for i < r, else 0
    T       = (I + A)^{-1}                        (UT transform; unit lower triangular)
    W       = T diag(beta * exp(gamma)) K          U = T diag(beta) V
    Delta   = U - W S^T                           (rows: the effective writes delta_r)
    O       = diag(exp(gamma)) Q S^T + (Q K^T * exp(gamma_r - gamma_i) * [i <= r]) Delta
    S_next  = exp(gamma_{n-1}) S + Delta^T diag(exp(gamma_{n-1} - gamma)) K

Derivation: write S_r = e^{gamma_r} S + sum_{i<=r} e^{gamma_r-gamma_i} delta_i k_i^T with
delta_r = beta_r (v_r - alpha_r S_{r-1} k_r); substituting S_{r-1} into delta_r gives
(I + A) Delta = diag(beta) V - diag(beta e^gamma) K S^T. The mask includes the diagonal
because the query reads the state after the token's own write ("Gated DeltaNet"
module page, "How It Works").

The per-chunk transition is affine in the state: S_next = S M + Bc with
    M  = exp(gamma_{n-1}) I - W^T diag(exp(gamma_{n-1} - gamma)) K    [d_k, d_k]
    Bc = U^T diag(exp(gamma_{n-1} - gamma)) K                         [d_v, d_k]
which the tests compare with the explicit product of the per-token matrices
alpha_r (I - beta_r k_r k_r^T).

Parity pins: tests/test_oracle.py (equality with the token recurrence for chunk
sizes 1, 7, 16, 64 and with the brute-force per-chunk product).
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular


def chunk_factors(k, v, g, beta):
    """Chunk-local factors that do not depend on the state.

    k [n,d_k], v [n,d_v], g [n], beta [n] (float64). Returns a dict with gamma [n],
    A [n,n], T [n,n], W [n,d_k], U [n,d_v], Gamma_ratio [n,n] (exp(gamma_r - gamma_i)
    on and below the diagonal, 0 above).
    """
    n = k.shape[0]
    gamma = np.cumsum(g)
    lower = np.tril(np.ones((n, n), dtype=bool))
    diff = np.where(lower, gamma[:, None] - gamma[None, :], -np.inf)   # masked before exp
    ratio = np.exp(diff)
    A = np.tril(beta[:, None] * (k @ k.T) * ratio, k=-1)
    T = solve_triangular(np.eye(n) + A, np.eye(n), lower=True, unit_diagonal=True)
    W = T @ ((beta * np.exp(gamma))[:, None] * k)
    U = T @ (beta[:, None] * v)
    return dict(gamma=gamma, A=A, T=T, W=W, U=U, ratio=ratio)


def chunk_apply(S, q, k, f):
    """State-dependent part of one chunk: returns (Delta, O, S_next)."""
    gamma, ratio = f["gamma"], f["ratio"]
    Delta = f["U"] - f["W"] @ S.T
    O = np.exp(gamma)[:, None] * (q @ S.T) + ((q @ k.T) * ratio) @ Delta
    tail = np.exp(gamma[-1] - gamma)
    S_next = np.exp(gamma[-1]) * S + Delta.T @ (tail[:, None] * k)
    return Delta, O, S_next


def chunk_transition(k, f):
    """Affine per-chunk transition (M, Bc) with S_next = S @ M + Bc."""
    gamma = f["gamma"]
    tail = np.exp(gamma[-1] - gamma)
    M = np.exp(gamma[-1]) * np.eye(k.shape[1]) - f["W"].T @ (tail[:, None] * k)
    Bc = f["U"].T @ (tail[:, None] * k)
    return M, Bc


def sequence(q, k, v, g, beta, S0, chunk):
    """One sequence and head through the chunkwise form. q,k [L,d_k], v [L,d_v],
    g, beta [L], S0 [d_v,d_k]. Chunks start at token 0; only the last may be short.
    Returns (o [L,d_v], S_final, stages) where stages lists, per chunk, the entering
    state and the factors."""
    L = q.shape[0]
    S = np.array(S0, dtype=np.float64)
    o = np.zeros((L, v.shape[1]))
    stages = []
    for c0 in range(0, L, chunk):
        c1 = min(c0 + chunk, L)
        f = chunk_factors(k[c0:c1], v[c0:c1], g[c0:c1], beta[c0:c1])
        Delta, O, S_next = chunk_apply(S, q[c0:c1], k[c0:c1], f)
        stages.append(dict(start=c0, S_in=S, Delta=Delta, **f))
        o[c0:c1] = O
        S = S_next
    return o, S, stages


def forward(q, k, v, g, beta, h0=None, cu_seqlens=None, chunk=64):
    """Same interface as recurrence.forward (inputs already float64 arrays)."""
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if cu_seqlens is None:
        segs = [(b * T, (b + 1) * T) for b in range(B)]
    else:
        cu = [int(x) for x in np.asarray(cu_seqlens)]
        segs = [(cu[i], cu[i + 1]) for i in range(len(cu) - 1)]
    qf, kf, vf = q.reshape(-1, H, dk), k.reshape(-1, H, dk), v.reshape(-1, H, dv)
    gf, bf = g.reshape(-1, H), beta.reshape(-1, H)
    o = np.zeros((B * T, H, dv))
    hT = np.zeros((len(segs), H, dv, dk))
    for n, (s0, s1) in enumerate(segs):
        for h in range(H):
            S0 = np.zeros((dv, dk)) if h0 is None else np.asarray(h0[n, h], dtype=np.float64)
            if s1 == s0:
                hT[n, h] = S0
                continue
            o[s0:s1, h], hT[n, h], _ = sequence(qf[s0:s1, h], kf[s0:s1, h], vf[s0:s1, h],
                                                gf[s0:s1, h], bf[s0:s1, h], S0, chunk)
    return o.reshape(B, T, H, dv), hT
