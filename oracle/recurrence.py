"""CPU fp64 oracle of the gated delta rule: the token-by-token recurrence.

TEST INFRASTRUCTURE. Only the test suite, the package smoke check and the CPU
baseline leg of the benchmark may import or run anything in this directory. The
HIP library never calls it, and it shares no code with the HIP library.

What it computes (per sequence and head, state S of shape [d_v, d_k]):

    S_t = S_{t-1} . alpha_t (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = S_t q_t

Sources:
  * recurrence: paper note "Gated Delta Networks: Improving Mamba2 with Delta Rule"
    (phantomic12 inference-research), mechanism paragraph; and record "LIT-137: Gated
    Delta Networks" (anthology-of-the-sota), section "Standing in the anthology".
  * order inside one step (decay of the old memory first, then the delta write, then
    the read of the updated memory): module page "Gated DeltaNet" (ai-model-reference),
    sections "How It Works" and "Math Or Compute Schema", and the compute-path diagram,
    whose output node is o_t = S_t q_t.

The step is evaluated in the expanded form alpha S + beta (v - alpha S k) k^T, which
equals the product form above exactly in real arithmetic (distribute the product).
The product form itself is evaluated, with explicit d_k x d_k matrices, only by the
tests that pin this module.

Parity pins: tests/test_oracle.py (closed forms, brute force, invariants).
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    """Exact widening of a CPU tensor / array (fp32 or bf16 values) to a float64 array."""
    if x is None:
        return None
    if hasattr(x, "detach"):              # torch tensor: bf16 -> fp32 is exact, fp32 -> fp64 exact
        import torch
        x = x.detach().to("cpu")
        if x.dtype == torch.bfloat16:
            x = x.float()
        return x.double().numpy()
    return np.asarray(x, dtype=np.float64)


def step(S, q, k, v, g, beta):
    """One token of the recurrence for one head.

    S [d_v, d_k] state before the token; q, k [d_k]; v [d_v]; g = log(alpha) scalar;
    beta scalar. Returns (S_t, o_t).
    """
    a = np.exp(g)                         # alpha_t: decays the old memory before the write
    S = a * S
    u = S @ k                             # what the decayed memory returns for key k
    S = S + beta * np.outer(v - u, k)     # delta-rule write of the residual along k
    o = S @ q                             # the query reads the updated memory
    return S, o


def step_heads(S, q, k, v, g, beta):
    """`step` applied to H independent heads at once: S [H,d_v,d_k]; q,k [H,d_k];
    v [H,d_v]; g, beta [H]. Heads never interact; the batch axis is only bookkeeping."""
    a = np.exp(g)[:, None, None]
    S = a * S
    u = np.einsum("hvk,hk->hv", S, k)
    S = S + beta[:, None, None] * (v - u)[:, :, None] * k[:, None, :]
    o = np.einsum("hvk,hk->hv", S, q)
    return S, o


def segments(B, T, cu_seqlens):
    """Token ranges [start, end) of each sequence in the flattened token axis."""
    if cu_seqlens is None:
        return [(b * T, (b + 1) * T) for b in range(B)]
    cu = [int(x) for x in np.asarray(_f64(cu_seqlens)).astype(np.int64)]
    return [(cu[i], cu[i + 1]) for i in range(len(cu) - 1)]


def forward(q, k, v, g, beta, h0=None, cu_seqlens=None, heads=None):
    """Whole-sequence forward pass, token by token.

    q, k [B,T,H,d_k]; v [B,T,H,d_v]; g, beta [B,T,H]; h0 [N,H,d_v,d_k] or None (zeros);
    cu_seqlens int [N+1] or None. With cu_seqlens, B must be 1 and each segment
    starts from its own h0[n] (packed variable-length sequences). Returns
    o [B,T,H,d_v] and hT [N,H,d_v,d_k] in float64. `heads` restricts the work to a
    subset of heads (outputs of other heads are left as NaN).
    """
    q, k, v, g, beta, h0 = (_f64(x) for x in (q, k, v, g, beta, h0))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    segs = segments(B, T, cu_seqlens)
    if cu_seqlens is not None and B != 1:
        raise ValueError("packed sequences need B == 1")
    hs = np.arange(H) if heads is None else np.asarray(heads)
    qf, kf, vf = q.reshape(B * T, H, dk), k.reshape(B * T, H, dk), v.reshape(B * T, H, dv)
    gf, bf = g.reshape(B * T, H), beta.reshape(B * T, H)
    o = np.full((B * T, H, dv), np.nan)
    hT = np.full((len(segs), H, dv, dk), np.nan)
    for n, (s0, s1) in enumerate(segs):
        S = np.zeros((len(hs), dv, dk)) if h0 is None else h0[n, hs].copy()
        for t in range(s0, s1):
            S, o[t, hs] = step_heads(S, qf[t, hs], kf[t, hs], vf[t, hs], gf[t, hs], bf[t, hs])
        hT[n, hs] = S
    return o.reshape(B, T, H, dv), hT


def decode(state, q, k, v, g, beta):
    """One decode step for every (sequence, head): state [N,H,d_v,d_k]; q,k [N,H,d_k];
    v [N,H,d_v]; g, beta [N,H]. Returns (new_state, o [N,H,d_v]) in float64; this is
    exactly one iteration of `forward`'s token loop with the state taken from memory."""
    state, q, k, v, g, beta = (_f64(x) for x in (state, q, k, v, g, beta))
    N, H, dv, dk = state.shape
    S = state.reshape(N * H, dv, dk)
    S, o = step_heads(S, q.reshape(N * H, dk), k.reshape(N * H, dk), v.reshape(N * H, dv),
                      g.reshape(N * H), beta.reshape(N * H))
    return S.reshape(N, H, dv, dk), o.reshape(N, H, dv)
