"""GPU parity of the decoupled erase/write-gate path (gdn_decoupled_chunk_fwd,
gdn_decoupled_decode_step, through the C ABI) against the CPU fp64 oracle
(oracle/decoupled.py), with the forward pass's tolerances (fp32: max|x - ref| / max|ref| <=
1e-4; bf16: max|x - ref| <= 2e-2 RMS(ref)); outputs compared in fp32.
"""
import pytest
import torch

from gated_delta_rule_42_amd import binding as gb
from gated_delta_rule_42_amd import synthetic as SY
from oracle import decoupled as DC
from test_parity import err, to_np, tol

pytestmark = pytest.mark.gpu

GATES = ("q", "k", "v", "g", "erase", "write")


def dc_inputs(x, seed, gate_scale=1.0):
    return SY.decoupled_gates(SY.channel_gates(x, seed, gate_scale=gate_scale), seed + 1)


def check_dc(x, heads=None):
    dt = x["meta"]["dtype"]
    print(f"[gpu] decoupled_chunk_fwd {x['meta']}", flush=True)
    dev = "cuda"
    t = {n: x[n].to(dev) for n in GATES}
    h0 = None if x["h0"] is None else x["h0"].to(dev)
    cu = None if x["cu_seqlens"] is None else x["cu_seqlens"].to(dev)
    o, hT = gb.gdn_decoupled_chunk_fwd(*(t[n] for n in GATES), h0, cu, o_dtype=torch.float32)
    torch.cuda.synchronize()
    o, hT = to_np(o), to_np(hT)
    sl = (lambda a: a) if heads is None else (lambda a: a[:, :, heads].contiguous())
    h0r = x["h0"] if (heads is None or x["h0"] is None) else x["h0"][:, heads].contiguous()
    o_ref, h_ref = DC.forward(*(sl(x[n]) for n in GATES), h0r, x["cu_seqlens"])
    if heads is not None:
        o, hT = o[:, :, heads], hT[:, heads]
    eo, eh = err(o, o_ref, dt), err(hT, h_ref, dt)
    print(f"      err(o)={eo:.3e} err(hT)={eh:.3e} tol={tol(dt):.0e}", flush=True)
    assert eo <= tol(dt) and eh <= tol(dt)


DC_SMALL = [
    # B, T, H, dk, dv, dtype, h0, gate_scale
    (1, 200, 2, 64, 64, "f32", True, 1.0),
    (2, 130, 2, 128, 128, "f32", True, 0.02),
    (1, 100, 2, 128, 64, "bf16", False, 1.0),
    (2, 150, 2, 128, 128, "bf16", True, 1.0),
    (1, 1, 2, 64, 128, "bf16", True, 1.0),
]


@pytest.mark.parametrize("B,T,H,dk,dv,dtype,h0,gs", DC_SMALL)
def test_decoupled_small(B, T, H, dk, dv, dtype, h0, gs):
    w = SY.Workload(99, f"dc_{dtype}", H=H, dk=dk, dv=dv, dtype=dtype, B=B, T=T)
    x = SY.make_forward_inputs(w, seed=7000 + T + dk + dv, h0=h0)
    check_dc(dc_inputs(x, 7100 + T, gate_scale=gs))


def test_decoupled_varlen():
    w = SY.Workload(99, "dc_varlen", H=2, dk=128, dv=128, dtype="bf16", varlen=5)
    x = SY.make_forward_inputs(w, seed=71, lengths=[70, 0, 1, 64, 129], h0=True)
    check_dc(dc_inputs(x, 72, gate_scale=0.05))


def test_decoupled_train_workload_sampled_heads():
    check_dc(dc_inputs(SY.make_forward_inputs(1), 73), heads=[5, 9])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decoupled_decode(dtype):
    d = dc_inputs(SY.make_decode_inputs(4, N=8, H=4, steps=3, dtype=dtype), 74)
    st = d["state"].to("cuda").clone()
    S_ref = d["state"]
    for s in range(3):
        o = gb.gdn_decoupled_decode_step(*(d[n][s].to("cuda") for n in GATES), st)
        torch.cuda.synchronize()
        S_ref, o_ref = DC.decode(S_ref, *(d[n][s] for n in GATES))
        eo, es = err(to_np(o), o_ref, dtype), err(to_np(st), S_ref, dtype)
        print(f"[gpu] decoupled_decode step {s} {dtype}: err(o)={eo:.2e} err(state)={es:.2e}", flush=True)
        assert eo <= tol(dtype) and es <= tol(dtype)
