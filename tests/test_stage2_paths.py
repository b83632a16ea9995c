"""GPU tests of the two state-propagation kernels that serve 32-column tiles of unsplit chains
(bf16 inputs, 64 or more (sequence, head) pairs at d_v = 128, 128 or more at d_v = 64): the
default chunk_propagate_split_kernel, where chain waves step the state and output waves form o
from the fp16 state and Delta the chain waves leave in LDS, and the four-wave
chunk_propagate_bf16_kernel (GDN_SPLIT_OUT=0). Both run the same products in the same order, so
o (fp32 and bf16) and hT must agree bit for bit; the default path's agreement with the oracle is
covered by the full-size parity tests of the training shape."""
import pytest
import torch

from gated_delta_rule_42_amd import binding as gb
from gated_delta_rule_42_amd import synthetic as SY

pytestmark = pytest.mark.gpu

CASES = {
    # name: (workload, overrides)
    "train_shape": (1, {}),
    "ragged_h0": (1, dict(T=2000, h0=True)),
    "slow_decay_beta2": (1, dict(T=1000, h0=True, gate_scale=0.01, beta_scale=2.0)),
    "packed_64_pairs": (3, dict(lengths=[64, 1, 1900, 0, 4035], H=16)),
    "d64_128_pairs": (0, dict(B=8, T=700, H=16, h0=True, dtype="bf16")),
}


def _run(x, monkeypatch, split):
    monkeypatch.setenv("GDN_SPLIT_OUT", "1" if split else "0")
    q, k, v, g, b = (x[n].to("cuda") for n in ("q", "k", "v", "g", "beta"))
    h0 = None if x["h0"] is None else x["h0"].to("cuda")
    cu = None if x["cu_seqlens"] is None else x["cu_seqlens"].to("cuda")
    out = []
    for od in (torch.float32, torch.bfloat16):
        o, hT = gb.gdn_chunk_fwd(q, k, v, g, b, h0, cu, o_dtype=od)
        out += [o, hT]
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name", list(CASES))
def test_split_kernel_matches_four_wave_kernel(name, monkeypatch):
    wid, kw = CASES[name]
    x = SY.make_forward_inputs(wid, seed=40 + wid, **kw)
    m = x["meta"]
    pairs = m["N"] * m["H"]
    # the 32-column path: fewer than 256 tiles of 64 columns, at least 256 of 32
    assert pairs * (m["dv"] // 64) < 256 <= pairs * (m["dv"] // 32), m
    print(f"[gpu] stage-2 paths {name} {m}", flush=True)
    a = _run(x, monkeypatch, split=False)
    b = _run(x, monkeypatch, split=True)
    for u, w in zip(a, b):
        assert torch.isfinite(u.float()).all()
        assert torch.equal(u, w)
