"""GPU tests of the value range the bf16 forward path supports.

With bf16 inputs the matrix-core operands of the state propagation are fp16: the state and
diag(e^gamma) Q, K, Mmat and P, and the residual V - e^gamma K S^T and the effective writes
Delta = Mmat R (all accumulated in fp32). fp16 holds magnitudes up to 65504, with full relative
precision down to 6.1e-5. These cases pin the parity bound of the workloads (max error within
2e-2 of the output RMS) at the edges of the range stated in the header: values up to about 1e4,
initial states of standard deviation 100, keys longer than unit length, and small values.
"""
import numpy as np
import pytest
import torch

from gated_delta_rule_42_amd import binding as gb
from gated_delta_rule_42_amd import synthetic as SY
from oracle import ctwin

pytestmark = pytest.mark.gpu

TOL = 2e-2


def rel(x, ref):
    x, ref = np.asarray(x, np.float64), np.asarray(ref, np.float64)
    assert np.isfinite(x).all()
    return np.max(np.abs(x - ref)) / max(np.sqrt(np.mean(ref ** 2)), 1e-300)


def rescaled(seed, T, gate_scale, v_scale, h0_std, k_scale, beta_scale=1.0, dk=128, dv=128):
    w = SY.Workload(94, "range", H=2, dk=dk, dv=dv, dtype="bf16", B=1, T=T)
    x = SY.make_forward_inputs(w, seed=seed, gate_scale=gate_scale, h0=True, beta_scale=beta_scale)
    x["v"] = (x["v"].float() * v_scale).to(torch.bfloat16)
    x["k"] = (x["k"].float() * k_scale).to(torch.bfloat16)
    rng = np.random.default_rng(seed + 1)
    x["h0"] = torch.from_numpy((rng.standard_normal(tuple(x["h0"].shape)) * h0_std).astype(np.float32))
    return x


CASES = [
    # T, gate_scale, v_scale, h0_std, k_scale, beta_scale
    (300, 1.0, 2500.0, 100.0, 1.0, 1.0),    # |v| up to about 1e4, fast decay
    (300, 0.01, 2500.0, 100.0, 1.0, 1.0),   # the same with slow decay: the state accumulates
    (300, 0.01, 1.0, 100.0, 1.0, 2.0),      # h0 std 100, beta up to 2
    (300, 0.05, 1.0, 1.0, 1.4, 1.0),        # |k| = 1.4 (beta |k|^2 < 2: the recurrence contracts)
    (300, 0.05, 1e-3, 1e-3, 1.0, 1.0),      # small values
]


@pytest.mark.parametrize("T,gs,vs,hs,ks,bs", CASES)
def test_value_range(T, gs, vs, hs, ks, bs):
    x = rescaled(900 + int(np.log10(vs) * 3) + int(ks * 10), T, gs, vs, hs, ks, bs)
    print(f"[gpu] range T={T} gate={gs} v*{vs} h0 std {hs} k*{ks} beta*{bs}: "
          f"max|v| {x['v'].float().abs().max().item():.3g}", flush=True)
    dev = "cuda"
    q, k, v, g, b, h0 = (x[n].to(dev) for n in ("q", "k", "v", "g", "beta", "h0"))
    o, hT = gb.gdn_chunk_fwd(q, k, v, g, b, h0, o_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, hT_ref = ctwin.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"])
    eo, eh = rel(o.cpu().numpy(), o_ref), rel(hT.cpu().numpy(), hT_ref)
    print(f"      max|o| {np.abs(o_ref).max():.3g} max|S| {np.abs(hT_ref).max():.3g} "
          f"err(o)={eo:.3e} err(hT)={eh:.3e}", flush=True)
    assert eo <= TOL and eh <= TOL
