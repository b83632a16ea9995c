"""Pins of the CPU fp64 gradient oracle (oracle/backward.py).

The gradients are pinned to things other than their own formulas: central finite
differences of the pinned forward oracle (every input element of small problems), a closed
form for beta = 0, and the agreement of the two independent derivations in the module (the
token-by-token adjoint and the chunkwise restatement the HIP kernels follow). Planted
mistakes in a copy of the adjoint show that the finite-difference pin rejects them.
"""
import numpy as np
import pytest

from oracle import backward as BW
from oracle import recurrence as R
from test_oracle import rand_inputs, rel


def _loss_inputs(seed, T=7, H=2, dk=3, dv=2, gate_scale=1.0, lengths=None, beta_scale=1.0):
    x = rand_inputs(seed, T=T, H=H, dk=dk, dv=dv, gate_scale=gate_scale, h0=True, lengths=lengths)
    x["beta"] = beta_scale * x["beta"]
    rng = np.random.default_rng(seed + 100)
    B, TT = x["q"].shape[:2]
    do = rng.standard_normal((B, TT, H, dv))
    dhT = rng.standard_normal(x["h0"].shape)
    return x, do, dhT


def _loss(x, do, dhT):
    o, hT = R.forward(**x)
    return float(np.sum(o * do) + np.sum(hT * dhT))


def _fd_grads(x, do, dhT, eps=1e-6):
    """Central differences of the forward oracle's loss for every element of q, k, v, g,
    beta and h0."""
    out = {}
    for name in ("q", "k", "v", "g", "beta", "h0"):
        base = x[name]
        grad = np.zeros_like(base)
        it = np.nditer(base, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = dict(x)
            xp[name] = base.copy()
            xp[name][idx] += eps
            lp = _loss(xp, do, dhT)
            xp[name][idx] -= 2 * eps
            lm = _loss(xp, do, dhT)
            grad[idx] = (lp - lm) / (2 * eps)
        out[name] = grad
    return out


def _adjoint(bw, x, do, dhT):
    dq, dk, dv, dg, db, dh0 = bw(x["q"], x["k"], x["v"], x["g"], x["beta"], do, h0=x["h0"], dhT=dhT,
                                 cu_seqlens=x["cu_seqlens"])
    return dict(q=dq, k=dk, v=dv, g=dg, beta=db, h0=dh0)


def _fd_check(bw, x, do, dhT):
    fd = _fd_grads(x, do, dhT)
    an = _adjoint(bw, x, do, dhT)
    return max(rel(an[n], fd[n]) for n in fd)


@pytest.mark.parametrize("case", ["dense", "varlen", "weak_decay", "beta_to_2"])
def test_adjoint_matches_finite_differences(case):
    kw = dict(dense={}, varlen=dict(lengths=[3, 1, 4]), weak_decay=dict(gate_scale=0.02),
              beta_to_2=dict(beta_scale=2.0))[case]
    x, do, dhT = _loss_inputs(3, **kw)
    assert _fd_check(BW.backward, x, do, dhT) < 1e-7


def test_beta_zero_closed_form():
    """beta = 0: S_t = (prod_{j<=t} alpha_j) h0, so with L = sum_t do_t . o_t:
    dq_t = a_t h0^T do_t, dh0 = sum_t a_t do_t q_t^T, dg_j = sum_{t>=j} do_t . o_t,
    dk = dv = 0, and dbeta_t = sum_{s>=t} (a_s / a_t) (do_s . r_t)(k_t . q_s) with
    r_t = v_t - a_t h0 k_t (a_t = prod_{j<=t} alpha_j): the first-order effect of
    switching on token t's write, carried forward by the decay."""
    x = rand_inputs(4, T=9, H=1, dk=4, dv=3, gate_scale=0.1, h0=True)
    x["beta"] = np.zeros_like(x["beta"])
    do = np.random.default_rng(5).standard_normal(x["v"].shape)
    dq, dk, dv, dg, db, dh0 = BW.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], do, h0=x["h0"])
    h0 = x["h0"][0, 0]
    q, k, v, g, d = x["q"][0, :, 0], x["k"][0, :, 0], x["v"][0, :, 0], x["g"][0, :, 0], do[0, :, 0]
    a = np.cumprod(np.exp(g))
    o = a[:, None] * (q @ h0.T)
    assert rel(dq[0, :, 0], a[:, None] * (d @ h0)) < 1e-13
    assert rel(dh0[0, 0], np.einsum("t,tv,tk->vk", a, d, q)) < 1e-13
    assert rel(dg[0, :, 0], np.cumsum(np.sum(d * o, axis=1)[::-1])[::-1]) < 1e-13
    assert np.max(np.abs(dk)) == 0 and np.max(np.abs(dv)) == 0
    r = v - a[:, None] * (k @ h0.T)
    want = np.array([sum(a[s] / a[t] * (d[s] @ r[t]) * (k[t] @ q[s]) for s in range(t, len(a)))
                     for t in range(len(a))])
    assert rel(db[0, :, 0], want) < 1e-12


@pytest.mark.parametrize("C", [1, 5, 16, 64])
@pytest.mark.parametrize("gate_scale", [1.0, 0.01])
def test_chunkwise_gradients_equal_adjoint(C, gate_scale):
    x, do, dhT = _loss_inputs(6, T=70, H=2, dk=8, dv=6, gate_scale=gate_scale)
    ref = _adjoint(BW.backward, x, do, dhT)
    got = _adjoint(lambda *a, **kw: BW.chunk_backward(*a, chunk=C, **kw), x, do, dhT)
    for n in ref:
        assert rel(got[n], ref[n]) < 1e-10, n


def test_chunkwise_gradients_varlen_and_no_state():
    x, do, _ = _loss_inputs(7, H=2, dk=8, dv=6, lengths=[70, 0, 5, 64, 129])
    x["h0"] = None
    ref = _adjoint(BW.backward, x, do, None)
    got = _adjoint(BW.chunk_backward, x, do, None)
    for n in ref:
        assert rel(got[n], ref[n]) < 1e-10, n
    assert np.max(np.abs(ref["h0"][:, :, :, :])) > 0   # dh0 is defined even when h0 is absent


def test_chunkwise_gradients_beta_to_2():
    x, do, dhT = _loss_inputs(8, T=130, H=1, dk=8, dv=6, beta_scale=2.0)
    ref = _adjoint(BW.backward, x, do, dhT)
    got = _adjoint(BW.chunk_backward, x, do, dhT)
    for n in ref:
        assert rel(got[n], ref[n]) < 1e-9, n


# --------------------------------------------------------------- planted mistakes
def _mutant(drop):
    """A copy of the adjoint with one term removed or altered."""
    def bw(q, k, v, g, beta, do, h0=None, dhT=None, cu_seqlens=None):
        q, k, v, g, beta, do, h0, dhT = (np.asarray(a, dtype=np.float64) if a is not None else None
                                         for a in (q, k, v, g, beta, do, h0, dhT))
        B, T, H, dk_ = q.shape
        dv_ = v.shape[-1]
        outs = [np.zeros_like(q), np.zeros_like(k), np.zeros_like(v), np.zeros_like(g), np.zeros_like(beta)]
        dh0 = np.zeros((B, H, dv_, dk_))
        for b in range(B):
            for h in range(H):
                P = h0[b, h].copy()
                st = [P]
                for t in range(T):
                    a = np.exp(g[b, t, h])
                    Sa = a * P
                    P = Sa + beta[b, t, h] * np.outer(v[b, t, h] - Sa @ k[b, t, h], k[b, t, h])
                    st.append(P)
                dS = dhT[b, h].copy()
                for t in range(T - 1, -1, -1):
                    kt, qt, vt, bt = k[b, t, h], q[b, t, h], v[b, t, h], beta[b, t, h]
                    a = np.exp(g[b, t, h])
                    Sa = a * st[t]
                    d = vt - Sa @ kt
                    dS = dS + np.outer(do[b, t, h], qt)
                    outs[0][b, t, h] = st[t + 1].T @ do[b, t, h]
                    dSk = dS @ kt
                    outs[4][b, t, h] = d @ dSk
                    dd = bt * dSk
                    dkt = bt * (dS.T @ d) if drop != "write_key" else 0.0
                    outs[2][b, t, h] = dd
                    du = -dd
                    dSa = dS + np.outer(du, kt) if drop != "read_path" else dS
                    if drop != "read_key":
                        dkt = dkt + Sa.T @ du
                    outs[1][b, t, h] = dkt
                    outs[3][b, t, h] = a * np.sum(dSa * st[t]) if drop != "gate_uses_new" else a * np.sum(dSa * st[t + 1])
                    dS = a * dSa
                dh0[b, h] = dS
        return (*outs, dh0)
    return bw


@pytest.mark.parametrize("drop", ["write_key", "read_path", "read_key", "gate_uses_new"])
def test_finite_difference_pin_rejects_mutant(drop):
    x, do, dhT = _loss_inputs(9, T=5, H=1)
    assert _fd_check(_mutant(None), x, do, dhT) < 1e-7      # the harness itself passes
    assert _fd_check(_mutant(drop), x, do, dhT) > 1e-3
