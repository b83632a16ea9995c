"""gdn_chunk_fwd_noalloc (the forward pass on the library's own device scratch array) against
gdn_chunk_fwd on the same inputs, through the C ABI: two calls in a row, the second with a
smaller input (so it also runs on whatever the first call left in the shared array). The two
entry points run the same kernels, so their outputs must be bitwise equal."""
import pytest
import torch

from gated_delta_rule_42_amd import binding as gb
from gated_delta_rule_42_amd import synthetic as SY

pytestmark = pytest.mark.gpu


def _run(x, fn):
    dev = "cuda"
    t = [x[n].to(dev) for n in ("q", "k", "v", "g", "beta")]
    h0 = None if x["h0"] is None else x["h0"].to(dev)
    cu = None if x["cu_seqlens"] is None else x["cu_seqlens"].to(dev)
    o, hT = fn(*t, h0, cu)
    torch.cuda.synchronize()
    return o, hT


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_workspace_entry_point(dtype):
    big = SY.make_forward_inputs(SY.Workload(80, "noalloc_big", H=4, dk=128, dv=128, dtype=dtype, B=2, T=700),
                                 seed=41, gate_scale=0.05, h0=True)
    small = SY.make_forward_inputs(SY.Workload(80, "noalloc_small", H=2, dk=128, dv=128, dtype=dtype),
                                   seed=42, lengths=[130, 1, 64], gate_scale=0.05, h0=True)
    for x in (big, small):
        print(f"[gpu] noalloc {x['meta']}", flush=True)
        o_ref, h_ref = _run(x, gb.gdn_chunk_fwd)
        o, h = _run(x, gb.gdn_chunk_fwd_noalloc)
        assert torch.equal(o, o_ref) and torch.equal(h, h_ref)


@pytest.mark.parametrize("path", ["0", "1"])   # GDN_FUSED: two stages, one kernel
def test_noalloc_long_chain_split(path, monkeypatch):
    """The long-chain split keeps its segment records and per-segment rerun counts in the
    workspace, which here is the shared array holding the previous call's contents: forced
    segments of 3 chunks, a long input then a shorter one, bitwise equal to gdn_chunk_fwd."""
    monkeypatch.setenv("GDN_FUSED", path)
    monkeypatch.setenv("GDN_SEGMENT_CHUNKS", "3")
    big = SY.make_forward_inputs(SY.Workload(80, "noalloc_split_big", H=2, dk=128, dv=128, dtype="bf16", B=2, T=1300),
                                 seed=43, h0=True, beta_scale=2.0)
    small = SY.make_forward_inputs(SY.Workload(80, "noalloc_split_small", H=2, dk=128, dv=128, dtype="bf16"),
                                   seed=44, lengths=[700, 64, 0, 300], gate_scale=0.001, h0=True)
    for x in (big, small):
        print(f"[gpu] noalloc split path={path} {x['meta']}", flush=True)
        o_ref, h_ref = _run(x, gb.gdn_chunk_fwd)
        o, h = _run(x, gb.gdn_chunk_fwd_noalloc)
        assert torch.isfinite(o.float()).all()
        assert torch.equal(o, o_ref) and torch.equal(h, h_ref)


def test_noalloc_rejects_problems_beyond_its_scratch():
    """A problem whose workspace exceeds the array is refused with GDN_ERR_WORKSPACE before any
    work is enqueued (the call does not fall back to allocating)."""
    # fp32 inputs run the two stages, whose workspace holds fp32 chunk operators (about 33 KB
    # per chunk and head): 64 chunks x 32 heads need more than the 64 MiB array
    B, T, H, d = 1, 4096, 32, 128
    need = gb.gdn_chunk_fwd_workspace_bytes(B, T, H, d, d, B, False, dtype=torch.float32)
    assert need > (64 << 20)
    dev = "cuda"
    q = torch.zeros(B, T, H, d, dtype=torch.float32, device=dev)
    g = torch.zeros(B, T, H, device=dev)
    with pytest.raises(gb.GDNError, match="workspace"):
        gb.gdn_chunk_fwd_noalloc(q, q, q, g, g)
