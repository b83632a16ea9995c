"""Pins of the CPU fp64 oracle of the decoupled erase/write-gate recurrence
(oracle/decoupled.py): reduction to the pinned channel-wise-decay oracle when both gates are
tied to beta, a closed form with the erase gate off (pure accumulation), a closed form for a
basis key whose erase gate removes only some channels, the literal matrix product form, and
the chunkwise restatement. Planted mistakes are each rejected.
"""
import numpy as np
import pytest

from oracle import decoupled as DC
from oracle import kda as KD
from test_kda_oracle import kda_inputs
from test_oracle import rel


def dc_inputs(seed, T=40, H=2, dk=8, dv=6, gate_scale=1.0, lengths=None):
    x = kda_inputs(seed, T=T, H=H, dk=dk, dv=dv, gate_scale=gate_scale, lengths=lengths)
    rng = np.random.default_rng(seed + 70)
    B, TT = x["q"].shape[:2]
    x["erase"] = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, TT, H, dk))))
    x["write"] = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, TT, H, dv))))
    del x["beta"]
    return x


def pin_tied_gates(fwd):
    """erase = beta 1 and write = beta 1: the channel-wise-decay recurrence (pinned oracle)."""
    x = kda_inputs(21, T=50, H=2, dk=6, dv=5)
    o, hT = KD.forward(**x)
    y = {n: x[n] for n in ("q", "k", "v", "g", "h0", "cu_seqlens")}
    y["erase"] = np.repeat(x["beta"][..., None], 6, axis=-1)
    y["write"] = np.repeat(x["beta"][..., None], 5, axis=-1)
    oy, hy = fwd(**y)
    return max(rel(oy, o), rel(hy, hT))


def pin_no_erase(fwd):
    """erase = 0, no decay: nothing is erased, S_t = h0 + sum_{j<=t} (w_j * v_j) k_j^T."""
    x = dc_inputs(22, T=30, H=2, dk=5, dv=4)
    x["erase"] = np.zeros_like(x["erase"])
    x["g"] = np.zeros_like(x["g"])
    o, hT = fwd(**x)
    wv = x["write"][0] * x["v"][0]
    S = x["h0"][0][None] + np.cumsum(np.einsum("thv,thk->thvk", wv, x["k"][0]), axis=0)
    return max(rel(o[0], np.einsum("thvk,thk->thv", S, x["q"][0])), rel(hT[0], S[-1]))


def pin_partial_erase(fwd):
    """No decay, h0 = 0; token 1 writes v1 under the unit key u = (e_1 + e_2)/sqrt(2), token 2
    writes v2 under the same key with erase gate (1, 0, ...) and write gate 1: the erased read
    along (e * u) = (1/sqrt2, 0, ...) returns v1 / 2, so S = v1 u^T + (v2 - v1/2) u^T."""
    dk, dv = 4, 3
    u = np.zeros(dk)
    u[:2] = 1 / np.sqrt(2)
    rng = np.random.default_rng(23)
    v1, v2 = rng.standard_normal(dv), rng.standard_normal(dv)
    er = np.zeros((2, dk))
    er[0] = 1.0
    er[1, 0] = 1.0
    x = dict(q=np.stack([u, u])[None, :, None], k=np.stack([u, u])[None, :, None],
             v=np.stack([v1, v2])[None, :, None], g=np.zeros((1, 2, 1, dk)), erase=er[None, :, None],
             write=np.ones((1, 2, 1, dv)))
    o, hT = fwd(**x)
    S = np.outer(v1, u) + np.outer(v2 - v1 / 2, u)
    return max(rel(hT[0, 0], S), rel(o[0, 1, 0], S @ u), rel(o[0, 0, 0], v1))


def pin_literal_product(fwd):
    """S_t = S_{t-1} Diag(alpha_t) (I - (e_t * k_t) k_t^T) + (w_t * v_t) k_t^T with explicit
    d_k x d_k matrices."""
    x = dc_inputs(24, T=12, H=1, dk=4, dv=3)
    o, hT = fwd(**x)
    S = x["h0"][0, 0].copy()
    errs = []
    for t in range(12):
        k, e = x["k"][0, t, 0], x["erase"][0, t, 0]
        S = (S @ np.diag(np.exp(x["g"][0, t, 0])) @ (np.eye(4) - np.outer(e * k, k))
             + np.outer(x["write"][0, t, 0] * x["v"][0, t, 0], k))
        errs.append(rel(o[0, t, 0], S @ x["q"][0, t, 0]))
    errs.append(rel(hT[0, 0], S))
    return max(errs)


PINS = [pin_tied_gates, pin_no_erase, pin_partial_erase, pin_literal_product]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_decoupled_oracle_pins(pin):
    assert pin(DC.forward) < 1e-12


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_decoupled_chunkwise_model_pins(pin):
    assert pin(lambda **x: DC.chunk_forward(**x, chunk=4)) < 1e-11


@pytest.mark.parametrize("C", [1, 7, 16, 64])
@pytest.mark.parametrize("gate_scale", [1.0, 0.01])
def test_decoupled_chunkwise_equals_recurrence(C, gate_scale):
    x = dc_inputs(25, T=150, H=2, dk=8, dv=6, gate_scale=gate_scale)
    o, hT = DC.forward(**x)
    oc, hc = DC.chunk_forward(**x, chunk=C)
    assert max(rel(oc, o), rel(hc, hT)) < 1e-11


def test_decoupled_chunkwise_varlen():
    x = dc_inputs(26, H=2, dk=8, dv=6, lengths=[70, 0, 5, 129])
    o, hT = DC.forward(**x)
    oc, hc = DC.chunk_forward(**x)
    assert max(rel(oc, o), rel(hc, hT)) < 1e-10


def test_decoupled_decode_is_one_step():
    x = dc_inputs(27, T=9, H=2, dk=8, dv=6)
    o, hT = DC.forward(**x)
    x8 = {n: (x[n][:, :8] if n in ("q", "k", "v", "g", "erase", "write") else x[n]) for n in x}
    _, h8 = DC.forward(**x8)
    S, od = DC.decode(h8, *(x[n][:, 8] for n in ("q", "k", "v", "g", "erase", "write")))
    assert max(rel(od, o[:, 8]), rel(S, hT)) < 1e-13


# --------------------------------------------------------------- planted mistakes
def _loop(step):
    def fwd(q, k, v, g, erase, write, h0=None, cu_seqlens=None):
        B, T, H, dk = q.shape
        S = np.zeros((B, H, v.shape[-1], dk)) if h0 is None else np.array(h0, dtype=float)
        o = np.zeros((B, T, H, v.shape[-1]))
        for b in range(B):
            for t in range(T):
                S[b], o[b, t] = step(S[b], q[b, t], k[b, t], v[b, t], g[b, t], erase[b, t], write[b, t])
        return o, S
    return fwd


def _m_erase_on_store(S, q, k, v, g, e, w):    # erase gate on the stored direction instead
    Sa = S * np.exp(g)[:, None, :]
    u = np.einsum("hvk,hk->hv", Sa, k)
    S = Sa - u[:, :, None] * (e * k)[:, None, :] + (w * v)[:, :, None] * k[:, None, :]
    return S, np.einsum("hvk,hk->hv", S, q)


def _m_write_on_read(S, q, k, v, g, e, w):     # write gate applied to the whole residual
    Sa = S * np.exp(g)[:, None, :]
    u = np.einsum("hvk,hk->hv", Sa, e * k)
    S = Sa + (w * (v - u))[:, :, None] * k[:, None, :]
    return S, np.einsum("hvk,hk->hv", S, q)


def _m_swap(S, q, k, v, g, e, w):              # erase and write gates confused (write on read)
    Sa = S * np.exp(g)[:, None, :]
    u = np.einsum("hvk,hk->hv", Sa, k) * w
    S = Sa + (e.mean(axis=1, keepdims=True) * v - u)[:, :, None] * k[:, None, :]
    return S, np.einsum("hvk,hk->hv", S, q)


@pytest.mark.parametrize("mut", [_m_erase_on_store, _m_write_on_read, _m_swap], ids=lambda m: m.__name__)
def test_decoupled_pins_reject_mutant(mut):
    assert max(pin(_loop(DC.step_heads)) for pin in PINS) < 1e-12
    assert max(pin(_loop(mut)) for pin in PINS) > 1e-6
