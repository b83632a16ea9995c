"""CPU fp64 oracle of the gradients of the gated delta rule, and a chunkwise model of them.

TEST INFRASTRUCTURE. Only the test suite, the package smoke check and the CPU baseline
leg of the benchmark may import or run anything in this directory. It shares no code
with the HIP library.

The loss is any scalar L whose gradients with respect to the outputs are given: dO
(with respect to every o_t) and dhT (with respect to every final state; None = 0).
`backward` returns dL/dq, dL/dk, dL/dv, dL/dg, dL/dbeta and dL/dh0.

Sources: the recurrence and its step order are those of `recurrence.py` (paper note
"Gated Delta Networks: Improving Mamba2 with Delta Rule", mechanism paragraph; module page
"Gated DeltaNet", "How It Works"). The pages train the layer with this chunkwise algorithm
("parallel training algorithm", paper note; "training throughput", record "LIT-137") but
print no gradient formulas; everything below is derived here.

`backward` is reverse-mode differentiation of the token loop, one step at a time. The
forward step, for state P entering token t, is
    a = e^{g_t};  Sa = a P;  u = Sa k;  d = v - u;  S = Sa + beta d k^T;  o = S q
and its adjoint, with dS the gradient reaching S (from later tokens, or dhT):
    dS  += do q^T                 dq  = S^T do
    dbeta = d . (dS k)            dd  = beta dS k          dk  = beta dS^T d
    dv  = dd                      du  = -dd
    dSa = dS + du k^T             dk += Sa^T du
    dP  = a dSa                   dg  = a (dSa : P)        (":" = sum of the elementwise product)

`chunk_backward` restates the same gradients chunk by chunk, in the form the HIP kernels
compute (the notation of `chunkwise.py`, with E = diag(e^gamma), Ed = diag(e^{gamma_last -
gamma}), lam = e^{gamma_last}, X = K S^T, R = V - E X, Delta = Mm R with Mm = T diag(beta),
Y = E Q S^T, P = (Q K^T) * exp(gamma_i - gamma_r) * [r <= i]):
    chunk c forward:   O = Y + P Delta;   S' = lam S + Delta^T Ed K
    reverse over chunks, dS' the gradient reaching the state after the chunk:
        Z = K dS'^T,   dDelta = P^T dO + Ed Z,   dR = Mm^T dDelta (= dV)
        dS = lam dS' + (E dO)^T Q - (E dR)^T K            (the gradient for the chunk before)
    per chunk, given S and dS':
        dP  = dO Delta^T,  dPg = dP * exp(gamma_i - gamma_r) * [r <= i]
        dMm = dDelta R^T,  dT = dMm diag(beta),  dA = strict_lower(-T^T dT T^T)
        dQ  = E dO S + dPg K
        dK  = -E dR S + Ed Delta dS' + dPg^T Q + (dG + dG^T) K,  dG = dA * beta_r * Gamma
        dbeta_i = sum_r dMm[r,i] T[r,i] + sum_{m<i} dA[i,m] (k_i . k_m) Gamma[i,m]
        dgamma_r: (dO : Y)_r - (dR : E X)_r - z_r + (dP : P) row r - (dP : P) column r
                  + (dA : A) row r - (dA : A) column r,  z_r = Ed_r (Delta : Z)_r,
                  and the last row also gets lam (dS' : S) + sum_r z_r
        dg = reverse cumulative sum of dgamma within the chunk.

Parity pins: tests/test_backward_oracle.py (central finite differences of the forward
oracle, a closed form for beta = 0, and equality of the two functions here).
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular

from .recurrence import _f64, segments


def backward(q, k, v, g, beta, do, h0=None, dhT=None, cu_seqlens=None):
    """Gradients of a loss with output gradients dO [B,T,H,d_v] (and dhT [N,H,d_v,d_k] or
    None) through the token recurrence. Inputs as in recurrence.forward. Returns
    dq, dk [B,T,H,d_k], dv [B,T,H,d_v], dg, dbeta [B,T,H], dh0 [N,H,d_v,d_k] (float64)."""
    q, k, v, g, beta, do, h0, dhT = (_f64(x) for x in (q, k, v, g, beta, do, h0, dhT))
    B, T, H, dk_ = q.shape
    dv_ = v.shape[-1]
    segs = segments(B, T, cu_seqlens)
    if cu_seqlens is not None and B != 1:
        raise ValueError("packed sequences need B == 1")
    qf, kf, vf = q.reshape(B * T, H, dk_), k.reshape(B * T, H, dk_), v.reshape(B * T, H, dv_)
    gf, bf = g.reshape(B * T, H), beta.reshape(B * T, H)
    dof = do.reshape(B * T, H, dv_)
    dq = np.zeros_like(qf)
    dk = np.zeros_like(kf)
    dv = np.zeros_like(vf)
    dg = np.zeros_like(gf)
    db = np.zeros_like(bf)
    dh0 = np.zeros((len(segs), H, dv_, dk_))
    for n, (s0, s1) in enumerate(segs):
        for h in range(H):
            P = np.zeros((dv_, dk_)) if h0 is None else h0[n, h].copy()
            states = [P]                                   # state entering each token
            for t in range(s0, s1):
                a = np.exp(gf[t, h])
                Sa = a * P
                P = Sa + bf[t, h] * np.outer(vf[t, h] - Sa @ kf[t, h], kf[t, h])
                states.append(P)
            dS = np.zeros((dv_, dk_)) if dhT is None else dhT[n, h].copy()
            for t in range(s1 - 1, s0 - 1, -1):
                Pin, S = states[t - s0], states[t - s0 + 1]
                kt, qt, vt, b = kf[t, h], qf[t, h], vf[t, h], bf[t, h]
                a = np.exp(gf[t, h])
                Sa = a * Pin
                d = vt - Sa @ kt
                dS = dS + np.outer(dof[t, h], qt)
                dq[t, h] = S.T @ dof[t, h]
                dSk = dS @ kt
                db[t, h] = d @ dSk
                dd = b * dSk
                dkt = b * (dS.T @ d)
                dv[t, h] = dd
                du = -dd
                dSa = dS + np.outer(du, kt)
                dkt = dkt + Sa.T @ du
                dk[t, h] = dkt
                dg[t, h] = a * np.sum(dSa * Pin)
                dS = a * dSa
            dh0[n, h] = dS
    shp = (B, T, H)
    return (dq.reshape(*shp, dk_), dk.reshape(*shp, dk_), dv.reshape(*shp, dv_), dg.reshape(shp),
            db.reshape(shp), dh0)


def _chunk_locals(q, k, v, g, beta, C):
    """Per-chunk quantities of one chunk padded to C rows (padding rows: zero inputs,
    g = beta = 0, which keeps gamma constant past the chunk's end)."""
    n = k.shape[0]
    pad = lambda x: np.concatenate([x, np.zeros((C - n,) + x.shape[1:])]) if n < C else x
    q, k, v, g, beta = (pad(x) for x in (q, k, v, g, beta))
    gamma = np.cumsum(g)
    low = np.tril(np.ones((C, C), dtype=bool))
    Gam = np.exp(np.where(low, gamma[:, None] - gamma[None, :], -np.inf))   # Gamma[r,i], i <= r
    G = k @ k.T
    A = np.tril(beta[:, None] * G * Gam, k=-1)
    T = solve_triangular(np.eye(C) + A, np.eye(C), lower=True, unit_diagonal=True)
    Mm = T * beta[None, :]
    P = (q @ k.T) * Gam
    return dict(q=q, k=k, v=v, g=g, beta=beta, gamma=gamma, Gam=Gam, G=G, A=A, T=T, Mm=Mm, P=P,
                E=np.exp(gamma), Ed=np.exp(gamma[-1] - gamma), lam=np.exp(gamma[-1]))


def chunk_backward(q, k, v, g, beta, do, h0=None, dhT=None, cu_seqlens=None, chunk=64):
    """The gradients of `backward`, computed chunk by chunk (see the module docstring):
    a forward pass keeping the state entering each chunk, a reverse pass keeping the
    gradient leaving each chunk, then independent per-chunk gradients."""
    q, k, v, g, beta, do, h0, dhT = (_f64(x) for x in (q, k, v, g, beta, do, h0, dhT))
    B, T, H, dk_ = q.shape
    dv_ = v.shape[-1]
    C = chunk
    segs = segments(B, T, cu_seqlens)
    qf, kf, vf = q.reshape(B * T, H, dk_), k.reshape(B * T, H, dk_), v.reshape(B * T, H, dv_)
    gf, bf = g.reshape(B * T, H), beta.reshape(B * T, H)
    dof = do.reshape(B * T, H, dv_)
    out = dict(dq=np.zeros_like(qf), dk=np.zeros_like(kf), dv=np.zeros_like(vf),
               dg=np.zeros_like(gf), db=np.zeros_like(bf))
    dh0 = np.zeros((len(segs), H, dv_, dk_))
    for n, (s0, s1) in enumerate(segs):
        for h in range(H):
            starts = list(range(s0, s1, C))
            L = [_chunk_locals(qf[c0:min(c0 + C, s1), h], kf[c0:min(c0 + C, s1), h],
                               vf[c0:min(c0 + C, s1), h], gf[c0:min(c0 + C, s1), h],
                               bf[c0:min(c0 + C, s1), h], C) for c0 in starts]
            dO = []
            for c0 in starts:
                x = dof[c0:min(c0 + C, s1), h]
                dO.append(np.concatenate([x, np.zeros((C - x.shape[0], dv_))]))
            # forward: state entering each chunk
            S = np.zeros((dv_, dk_)) if h0 is None else h0[n, h].copy()
            Sin = []
            for f in L:
                Sin.append(S)
                R = f["v"] - f["E"][:, None] * (f["k"] @ S.T)
                Delta = f["Mm"] @ R
                S = f["lam"] * S + Delta.T @ (f["Ed"][:, None] * f["k"])
            # reverse: gradient reaching the state after each chunk
            dS = np.zeros((dv_, dk_)) if dhT is None else dhT[n, h].copy()
            dSout = [None] * len(L)
            for c in range(len(L) - 1, -1, -1):
                f = L[c]
                dSout[c] = dS
                Z = f["k"] @ dS.T
                dDelta = f["P"].T @ dO[c] + f["Ed"][:, None] * Z
                dR = f["Mm"].T @ dDelta
                dS = (f["lam"] * dS + (f["E"][:, None] * dO[c]).T @ f["q"]
                      - (f["E"][:, None] * dR).T @ f["k"])
            dh0[n, h] = dS
            # independent per-chunk gradients
            for c, (c0, f) in enumerate(zip(starts, L)):
                S, dSo, dOc = Sin[c], dSout[c], dO[c]
                K, Q, V, E, Ed, lam, bet = f["k"], f["q"], f["v"], f["E"], f["Ed"], f["lam"], f["beta"]
                X = K @ S.T
                R = V - E[:, None] * X
                Delta = f["Mm"] @ R
                Y = E[:, None] * (Q @ S.T)
                Z = K @ dSo.T
                dDelta = f["P"].T @ dOc + Ed[:, None] * Z
                dR = f["Mm"].T @ dDelta
                dP = np.tril(dOc @ Delta.T)
                dPg = dP * f["Gam"]
                dMm = dDelta @ R.T
                dT = dMm * bet[None, :]
                dA = np.tril(-f["T"].T @ dT @ f["T"].T, k=-1)
                dG = dA * bet[:, None] * f["Gam"]
                dQ = E[:, None] * (dOc @ S) + dPg @ K
                dK = (-(E[:, None] * dR) @ S + (Ed[:, None] * Delta) @ dSo + dPg.T @ Q
                      + (dG + dG.T) @ K)
                dbeta = np.sum(dMm * f["T"], axis=0) + np.sum(dA * f["G"] * f["Gam"], axis=1)
                PP = dP * f["P"]
                AA = dA * f["A"]
                z = Ed * np.sum(Delta * Z, axis=1)
                dgam = (np.sum(dOc * Y, axis=1) - np.sum(dR * (E[:, None] * X), axis=1) - z
                        + PP.sum(axis=1) - PP.sum(axis=0) + AA.sum(axis=1) - AA.sum(axis=0))
                dgam[-1] += lam * np.sum(dSo * S) + z.sum()
                dgc = np.cumsum(dgam[::-1])[::-1]
                m = min(C, s1 - c0)
                out["dq"][c0:c0 + m, h] = dQ[:m]
                out["dk"][c0:c0 + m, h] = dK[:m]
                out["dv"][c0:c0 + m, h] = dR[:m]
                out["dg"][c0:c0 + m, h] = dgc[:m]
                out["db"][c0:c0 + m, h] = dbeta[:m]
    shp = (B, T, H)
    return (out["dq"].reshape(*shp, dk_), out["dk"].reshape(*shp, dk_), out["dv"].reshape(*shp, dv_),
            out["dg"].reshape(shp), out["db"].reshape(shp), dh0)
