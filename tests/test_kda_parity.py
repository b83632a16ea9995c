"""GPU parity of the channel-wise-decay path (gdn_kda_chunk_fwd, gdn_kda_decode_step, through
the C ABI) against the CPU fp64 oracle (oracle/kda.py), with the forward pass's tolerances:
fp32 inputs max|x - ref| / max|ref| <= 1e-4; bf16 inputs max|x - ref| <= 2e-2 RMS(ref).
Outputs are compared in fp32 (o_dtype = fp32); bf16 outputs are checked bit for bit against
the fp32 ones rounded to nearest even.
"""
import numpy as np
import pytest
import torch

from gated_delta_rule_42_amd import binding as gb
from gated_delta_rule_42_amd import synthetic as SY
from oracle import kda as KD
from test_parity import err, to_np, tol

pytestmark = pytest.mark.gpu


def gpu_kda(x, o_dtype=torch.float32):
    dev = "cuda"
    t = {n: x[n].to(dev) for n in ("q", "k", "v", "g", "beta")}
    h0 = None if x["h0"] is None else x["h0"].to(dev)
    cu = None if x["cu_seqlens"] is None else x["cu_seqlens"].to(dev)
    o, hT = gb.gdn_kda_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], h0, cu, o_dtype=o_dtype)
    torch.cuda.synchronize()
    return o, hT


def check_kda(x, heads=None):
    dt = x["meta"]["dtype"]
    print(f"[gpu] kda_chunk_fwd {x['meta']}", flush=True)
    o, hT = (to_np(t) for t in gpu_kda(x))
    sl = (lambda t: t) if heads is None else (lambda t: None if t is None else t[:, :, heads].contiguous())
    slN = (lambda t: t) if heads is None else (lambda t: None if t is None else t[:, heads].contiguous())
    o_ref, h_ref = KD.forward(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["g"]), sl(x["beta"]), slN(x["h0"]),
                              x["cu_seqlens"])
    if heads is not None:
        o, hT = o[:, :, heads], hT[:, heads]
    eo, eh = err(o, o_ref, dt), err(hT, h_ref, dt)
    print(f"      err(o)={eo:.3e} err(hT)={eh:.3e} tol={tol(dt):.0e}", flush=True)
    assert eo <= tol(dt) and eh <= tol(dt)


KDA_SMALL = [
    # B, T, H, dk, dv, dtype, h0, gate_scale
    (1, 200, 2, 64, 64, "f32", True, 1.0),
    (2, 130, 2, 128, 128, "f32", True, 0.02),
    (1, 100, 2, 64, 128, "f32", False, 1.0),
    (2, 150, 2, 128, 128, "bf16", True, 1.0),
    (1, 257, 2, 128, 64, "bf16", True, 0.05),
    (1, 1, 2, 128, 128, "bf16", True, 1.0),
    (1, 190, 2, 128, 128, "f32", True, 5.0),     # strong decay: up to e^-30 per token
    (1, 200, 2, 64, 64, "bf16", False, 1.0),
    (1, 100, 2, 64, 128, "bf16", True, 1.0),
    (1, 190, 2, 128, 128, "bf16", True, 5.0),
]


@pytest.mark.parametrize("B,T,H,dk,dv,dtype,h0,gs", KDA_SMALL)
def test_kda_small(B, T, H, dk, dv, dtype, h0, gs):
    w = SY.Workload(99, f"kda_{dtype}", H=H, dk=dk, dv=dv, dtype=dtype, B=B, T=T)
    x = SY.make_forward_inputs(w, seed=5000 + T + dk + dv, h0=h0)
    check_kda(SY.channel_gates(x, 6000 + T, gate_scale=gs))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_kda_varlen_beta_to_2(dtype):
    w = SY.Workload(99, "kda_varlen", H=2, dk=128, dv=128, dtype=dtype, varlen=5)
    x = SY.make_forward_inputs(w, seed=51, lengths=[70, 0, 1, 64, 129], h0=True, beta_scale=2.0)
    check_kda(SY.channel_gates(x, 52, gate_scale=0.05))


def test_kda_bf16_output_is_rounded_fp32():
    w = SY.Workload(99, "kda_round", H=2, dk=128, dv=128, dtype="bf16", B=1, T=150)
    x = SY.channel_gates(SY.make_forward_inputs(w, seed=53, h0=True), 54)
    o32, h32 = gpu_kda(x, torch.float32)
    o16, h16 = gpu_kda(x, torch.bfloat16)
    assert o16.dtype == torch.bfloat16 and torch.equal(o32.to(torch.bfloat16), o16)
    assert torch.equal(h32, h16)


def test_kda_train_workload_sampled_heads():
    """The training-shape workload (B4 H16 T2048 d128, bf16) with channel-wise gates, in full
    on the GPU; the oracle computes heads 3 and 12."""
    x = SY.channel_gates(SY.make_forward_inputs(1), 55)
    check_kda(x, heads=[3, 12])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_kda_decode(dtype):
    d = SY.channel_gates(SY.make_decode_inputs(4, N=8, H=4, steps=3, dtype=dtype), 56)
    dev = "cuda"
    st = d["state"].to(dev).clone()
    S_ref = d["state"]
    for s in range(3):
        o = gb.gdn_kda_decode_step(*(d[n][s].to(dev) for n in ("q", "k", "v", "g", "beta")), st)
        torch.cuda.synchronize()
        S_ref, o_ref = KD.decode(S_ref, *(d[n][s] for n in ("q", "k", "v", "g", "beta")))
        eo, es = err(to_np(o), o_ref, dtype), err(to_np(st), S_ref, dtype)
        print(f"[gpu] kda_decode step {s} {dtype}: err(o)={eo:.2e} err(state)={es:.2e}", flush=True)
        assert eo <= tol(dtype) and es <= tol(dtype)
