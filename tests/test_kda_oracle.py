"""Pins of the CPU fp64 oracle of the channel-wise-decay recurrence (oracle/kda.py).

Each compares the oracle with something other than its own formula: the pinned scalar-gate
oracle (the two must agree when every channel decays alike), closed forms (beta = 0; basis
keys with one decaying channel), the literal matrix product form on tiny shapes, and the
chunkwise restatement. Planted mistakes in copies of the step are each rejected.
"""
import numpy as np
import pytest

from oracle import kda as KD
from oracle import recurrence as R
from test_oracle import rand_inputs, rel


def kda_inputs(seed, T=40, H=2, dk=8, dv=6, gate_scale=1.0, h0=True, lengths=None, beta_scale=1.0):
    x = rand_inputs(seed, T=T, H=H, dk=dk, dv=dv, gate_scale=gate_scale, h0=h0, lengths=lengths)
    rng = np.random.default_rng(seed + 50)
    B, TT = x["q"].shape[:2]
    x["g"] = -gate_scale * np.logaddexp(0.0, rng.standard_normal((B, TT, H, dk)))
    x["beta"] = beta_scale * x["beta"]
    return x


def pin_scalar_reduction(fwd):
    """Every channel with the same decay: the scalar gated delta rule (pinned oracle)."""
    x = rand_inputs(11, T=50, H=2, dk=6, dv=5, h0=True)
    o, hT = R.forward(**x)
    xk = dict(x)
    xk["g"] = np.repeat(x["g"][..., None], 6, axis=-1)
    ok, hk = fwd(**xk)
    return max(rel(ok, o), rel(hk, hT))


def pin_decay_only(fwd):
    """beta = 0: S_t = h0 Diag(prod_{j<=t} alpha_j) column by column, o_t = S_t q_t."""
    x = kda_inputs(12, T=30, H=2, dk=5, dv=4, gate_scale=0.05)
    x["beta"] = np.zeros_like(x["beta"])
    o, hT = fwd(**x)
    P = np.exp(np.cumsum(x["g"][0], axis=0))                      # [T, H, dk]
    S = x["h0"][0][None] * P[:, :, None, :]                        # [T, H, dv, dk]
    o_cf = np.einsum("thvk,thk->thv", S, x["q"][0])
    return max(rel(o[0], o_cf), rel(hT[0], S[-1]))


def pin_basis_keys(fwd):
    """beta = 1, keys e_1..e_m, h0 = 0, channel c decaying by a_c per token and the others
    not at all: token i stores v_i in column i, which then decays by the later tokens'
    alpha of channel i only, so S e_i = v_i prod_{j>i} alpha_j[i] and the query e_t reads
    the token's own v_t (after the write)."""
    m, dk, dv = 5, 6, 3
    rng = np.random.default_rng(13)
    K = np.eye(dk)[:m]
    V = rng.standard_normal((m, dv))
    g = np.zeros((m, dk))
    g[:, 2] = -0.3
    g[:, 4] = -1.1
    x = dict(q=K[None, :, None], k=K[None, :, None], v=V[None, :, None], g=g[None, :, None],
             beta=np.ones((1, m, 1)))
    o, hT = fwd(**x)
    errs = [rel(o[0, :, 0], V)]
    for i in range(m):
        want = V[i] * np.exp(np.sum(g[i + 1:, i]))
        errs.append(rel(hT[0, 0] @ K[i], want))
    return max(errs)


def pin_literal_product(fwd):
    """The literal form S_{t-1} Diag(alpha_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T with
    explicit d_k x d_k matrices, beta up to 2, h0 != 0."""
    x = kda_inputs(14, T=12, H=1, dk=4, dv=3, beta_scale=2.0)
    o, hT = fwd(**x)
    S = x["h0"][0, 0].copy()
    errs = []
    for t in range(12):
        k = x["k"][0, t, 0]
        b = x["beta"][0, t, 0]
        S = S @ np.diag(np.exp(x["g"][0, t, 0])) @ (np.eye(4) - b * np.outer(k, k)) + b * np.outer(x["v"][0, t, 0], k)
        errs.append(rel(o[0, t, 0], S @ x["q"][0, t, 0]))
    errs.append(rel(hT[0, 0], S))
    return max(errs)


PINS = [pin_scalar_reduction, pin_decay_only, pin_basis_keys, pin_literal_product]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_kda_oracle_pins(pin):
    assert pin(KD.forward) < 1e-12


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_kda_chunkwise_model_pins(pin):
    assert pin(lambda **x: KD.chunk_forward(**x, chunk=4)) < 1e-11


@pytest.mark.parametrize("C", [1, 7, 16, 64])
@pytest.mark.parametrize("gate_scale", [1.0, 0.01])
def test_kda_chunkwise_equals_recurrence(C, gate_scale):
    x = kda_inputs(15, T=150, H=2, dk=8, dv=6, gate_scale=gate_scale)
    o, hT = KD.forward(**x)
    oc, hc = KD.chunk_forward(**x, chunk=C)
    assert max(rel(oc, o), rel(hc, hT)) < 1e-11


def test_kda_chunkwise_varlen_beta_to_2():
    x = kda_inputs(16, H=2, dk=8, dv=6, lengths=[70, 0, 5, 129], beta_scale=2.0)
    o, hT = KD.forward(**x)
    oc, hc = KD.chunk_forward(**x)
    assert max(rel(oc, o), rel(hc, hT)) < 1e-10


def test_kda_decode_is_one_step():
    x = kda_inputs(17, T=9, H=2, dk=8, dv=6)
    o, hT = KD.forward(**x)
    x8 = {n: (x[n][:, :8] if n in ("q", "k", "v", "g", "beta") else x[n]) for n in x}
    _, h8 = KD.forward(**x8)
    S, od = KD.decode(h8, x["q"][:, 8], x["k"][:, 8], x["v"][:, 8], x["g"][:, 8], x["beta"][:, 8])
    assert max(rel(od, o[:, 8]), rel(S, hT)) < 1e-13


# --------------------------------------------------------------- planted mistakes
def _loop(step):
    def fwd(q, k, v, g, beta, h0=None, cu_seqlens=None):
        B, T, H, dk = q.shape
        S = np.zeros((B, H, v.shape[-1], dk)) if h0 is None else np.array(h0, dtype=float)
        o = np.zeros((B, T, H, v.shape[-1]))
        for b in range(B):
            for t in range(T):
                S[b], o[b, t] = step(S[b], q[b, t], k[b, t], v[b, t], g[b, t], beta[b, t])
        return o, S
    return fwd


def _m_rows(S, q, k, v, g, b):          # decay on the value side (rows) instead of key channels
    Sa = S * np.exp(g)[:, :S.shape[1], None] if S.shape[1] <= g.shape[1] else S
    u = np.einsum("hvk,hk->hv", Sa, k)
    S = Sa + b[:, None, None] * (v - u)[:, :, None] * k[:, None, :]
    return S, np.einsum("hvk,hk->hv", S, q)


def _m_after(S, q, k, v, g, b):         # decay after the write
    u = np.einsum("hvk,hk->hv", S, k)
    S = (S + b[:, None, None] * (v - u)[:, :, None] * k[:, None, :]) * np.exp(g)[:, None, :]
    return S, np.einsum("hvk,hk->hv", S, q)


def _m_residual(S, q, k, v, g, b):      # residual read from the undecayed memory
    u = np.einsum("hvk,hk->hv", S, k)
    S = S * np.exp(g)[:, None, :] + b[:, None, None] * (v - u)[:, :, None] * k[:, None, :]
    return S, np.einsum("hvk,hk->hv", S, q)


def _m_mean_gate(S, q, k, v, g, b):     # channel gates collapsed to their mean
    gm = np.repeat(g.mean(axis=1, keepdims=True), g.shape[1], axis=1)
    return KD.step_heads(S, q, k, v, gm, b)


@pytest.mark.parametrize("mut", [_m_rows, _m_after, _m_residual, _m_mean_gate], ids=lambda m: m.__name__)
def test_kda_pins_reject_mutant(mut):
    assert max(pin(_loop(KD.step_heads)) for pin in PINS) < 1e-12
    assert max(pin(_loop(mut)) for pin in PINS) > 1e-6
