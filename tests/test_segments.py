"""GPU tests of the long-chain split of the bf16 forward pass.

Few (sequence, head) pairs with many chunks leave most compute units idle in the sequential
state propagation, so the library cuts each sequence into segments: all segments run at once
(segment 0 from h0, the others from zero, recording their states at segment offsets 1, 2, 4,
..), then a second pass walks the segments in order from the true entering state until its
state equals a record bit for bit. The split must give o and hT bit for bit equal to the
unsplit pass, for every segment length, with and without matches:
  * fast decay (the workloads' gates): the entering state is forgotten within a chunk, so the
    second pass stops at offset 1 or 2 (offset 1 can differ in the last bit: a zero start
    feeds the matrix core's accumulate an exact zero where the true run feeds it the decayed
    state, tiny but not zero, and a few sums round the other way);
  * slow decay: no record ever matches and the second pass recomputes every segment;
  * medium decay: a match at a later record in some tiles (last-bit differences fade slowly
    once the decayed state is no longer negligible in the accumulate; where is data-dependent:
    the one-kernel path compares all 128 columns of a head at once, the two-stage path each
    64-column tile on its own).
GDN_SEGMENT_CHUNKS forces the segment length; the workspace's last region tells how many
chunks the second pass computed per segment. Cases with d_k = d_v = 128 run on both bf16 forward
paths (GDN_FUSED=0: two stages; 1: one kernel), each against its own unsplit pass.
"""
import numpy as np
import pytest
import torch

from gated_delta_rule_42_amd import binding as gb
from gated_delta_rule_42_amd import synthetic as SY
from oracle import ctwin

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2


def rel_rms(x, ref):
    x, ref = np.asarray(x, np.float64), np.asarray(ref, np.float64)
    assert np.isfinite(x).all()
    return np.max(np.abs(x - ref)) / max(np.sqrt(np.mean(ref ** 2)), 1e-30)


def run(x, seg_chunks, monkeypatch, o_dtype=torch.float32):
    """Forward pass with the split forced to `seg_chunks` (0: off); returns o, hT and the
    per-segment rerun counts [N, H, max(1, dv/64), ns] (None without a split)."""
    monkeypatch.setenv("GDN_SEGMENT_CHUNKS", str(seg_chunks))
    m = x["meta"]
    dev = "cuda"
    q, k, v, g, b = (x[n].to(dev) for n in ("q", "k", "v", "g", "beta"))
    h0 = None if x["h0"] is None else x["h0"].to(dev)
    cu = None if x["cu_seqlens"] is None else x["cu_seqlens"].to(dev)
    N = m["N"]
    need = gb.gdn_chunk_fwd_workspace_bytes(m["B"], m["T"], m["H"], m["dk"], m["dv"], N, cu is not None)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    o, hT = gb.gdn_chunk_fwd(q, k, v, g, b, h0, cu, o_dtype=o_dtype, workspace=ws)
    torch.cuda.synchronize()
    reran = None
    if seg_chunks > 0:
        nmax = (m["T"] + 63) // 64
        ns = (nmax + seg_chunks - 1) // seg_chunks
        if ns > 1:
            nt = max(1, m["dv"] // 64)
            reran = ws[need - 4 * N * m["H"] * nt * ns:].cpu().view(torch.int32).numpy().reshape(N, m["H"], nt, ns)
    monkeypatch.delenv("GDN_SEGMENT_CHUNKS")
    return o, hT, reran


def seq_chunks(x):
    m = x["meta"]
    lengths = m["lengths"] if m["lengths"] is not None else [m["T"]] * m["B"]
    return [(L + 63) // 64 for L in lengths]


def check_split(x, L, monkeypatch, expect):
    m = x["meta"]
    print(f"[gpu] split L={L} expect={expect} {m}", flush=True)
    o0, h0, _ = run(x, 0, monkeypatch)
    o1, h1, reran = run(x, L, monkeypatch)
    assert reran is not None
    assert torch.equal(o1, o0), "o differs from the unsplit pass"
    assert torch.equal(h1, h0), "hT differs from the unsplit pass"
    # second-pass work per segment s >= 1 of each sequence
    seen, early = [], []
    for n, nc in enumerate(seq_chunks(x)):
        for s in range(1, (nc + L - 1) // L):
            seg_len = min(L, nc - s * L)
            r = reran[n, :, :, s]
            seen += r.ravel().tolist()
            assert ((r >= 1) & (r <= seg_len)).all(), (n, s, r)
            if expect == "full":
                assert (r == seg_len).all(), (n, s, r)
            elif expect == "quick" and seg_len > 2:
                assert (r <= 2).all(), (n, s, r)
            elif expect == "early" and seg_len == L:
                early.append((r < seg_len).any())
    print(f"      chunks recomputed per segment: {sorted(set(seen))}", flush=True)
    if expect == "early":
        assert any(early), "no segment matched a record before its end"
    # and the oracle
    o_ref, hT_ref = ctwin.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], x["cu_seqlens"])
    eo, eh = rel_rms(o1.float().cpu().numpy(), o_ref), rel_rms(h1.cpu().numpy(), hT_ref)
    print(f"      err(o)={eo:.3e} err(hT)={eh:.3e}", flush=True)
    assert eo <= TOL_BF16 and eh <= TOL_BF16


CASES = [
    # B, T, H, dk, dv, L, gate_scale, beta_scale, expect
    (1, 849, 2, 128, 128, 1, 1.0, 2.0, "quick"),     # every chunk a segment
    (1, 849, 2, 128, 128, 3, 1.0, 2.0, "quick"),
    (2, 849, 2, 128, 128, 5, 1.0, 1.0, "quick"),
    (2, 849, 2, 128, 128, 5, 0.001, 2.0, "full"),    # no match anywhere
    (1, 6400, 2, 128, 128, 32, 0.1, 1.0, "early"),   # matches at a later record
    (1, 1000, 2, 64, 64, 3, 1.0, 2.0, "quick"),
    (1, 1000, 3, 64, 128, 2, 0.001, 1.0, "full"),
    (1, 1000, 2, 128, 64, 4, 1.0, 2.0, "quick"),
]
PATHS = ["0", "1"]   # GDN_FUSED: two stages, one kernel


def paths_of(dk, dv):
    return PATHS if dk == dv == 128 else ["0"]


@pytest.mark.parametrize("B,T,H,dk,dv,L,gs,bs,expect,path",
                         [c + (pth,) for c in CASES for pth in paths_of(c[3], c[4])])
def test_split_equals_unsplit(B, T, H, dk, dv, L, gs, bs, expect, path, monkeypatch):
    monkeypatch.setenv("GDN_FUSED", path)
    w = SY.Workload(95, "split", H=H, dk=dk, dv=dv, dtype="bf16", B=B, T=T)
    x = SY.make_forward_inputs(w, seed=500 + T + L, gate_scale=gs, h0=True, beta_scale=bs)
    check_split(x, L, monkeypatch, expect)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("L,gs,expect", [(3, 1.0, "quick"), (2, 0.001, "full")])
def test_split_varlen(L, gs, expect, path, monkeypatch):
    """Packed sequences of 700, 64, 0, 300 and 1 tokens: segments past a sequence's end are
    empty, a one-chunk sequence never reaches the second pass."""
    monkeypatch.setenv("GDN_FUSED", path)
    w = SY.Workload(95, "split_varlen", H=2, dk=128, dv=128, dtype="bf16")
    x = SY.make_forward_inputs(w, seed=77, lengths=[700, 64, 0, 300, 1], gate_scale=gs, h0=True,
                               beta_scale=2.0)
    check_split(x, L, monkeypatch, expect)


@pytest.mark.parametrize("path", PATHS)
def test_split_bf16_output_and_no_final_state(path, monkeypatch):
    """bf16 o through the split equals the unsplit bf16 o; hT not requested."""
    monkeypatch.setenv("GDN_FUSED", path)
    w = SY.Workload(95, "split_bf16o", H=2, dk=128, dv=128, dtype="bf16", B=1, T=1500)
    x = SY.make_forward_inputs(w, seed=78, h0=True)
    o0, _, _ = run(x, 0, monkeypatch, o_dtype=torch.bfloat16)
    o1, _, _ = run(x, 4, monkeypatch, o_dtype=torch.bfloat16)
    assert o1.dtype == torch.bfloat16 and torch.equal(o0, o1)


@pytest.mark.parametrize("path,ns", [("0", 8), ("1", 16)])
def test_long_context_split_equals_unsplit(path, ns, monkeypatch):
    """B1 H16 T32768 d128: the shape-chosen plan (two stages: 8 segments of 64 chunks; one
    kernel: 16 of 32) against the unsplit pass, bit for bit; with the workloads' decay the
    second pass stops at offset 1 or 2."""
    monkeypatch.delenv("GDN_SEGMENT_CHUNKS", raising=False)
    monkeypatch.setenv("GDN_FUSED", path)
    x = SY.make_forward_inputs(2)
    dev = "cuda"
    t = [x[n].to(dev) for n in ("q", "k", "v", "g", "beta")]
    h0 = x["h0"].to(dev)
    need = gb.gdn_chunk_fwd_workspace_bytes(1, 32768, 16, 128, 128, 1, False)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    o1, h1 = gb.gdn_chunk_fwd(*t, h0, workspace=ws)
    torch.cuda.synchronize()
    reran = ws[need - 4 * 16 * 2 * ns:].cpu().view(torch.int32).numpy().reshape(16, 2, ns)
    monkeypatch.setenv("GDN_SEGMENT_CHUNKS", "0")
    o0, h0r = gb.gdn_chunk_fwd(*t, h0)
    torch.cuda.synchronize()
    print(f"[gpu] long-context reran per segment: {reran[:, :, 1:].ravel().tolist()}", flush=True)
    assert torch.equal(o0, o1) and torch.equal(h0r, h1)
    assert (reran[:, :, 1:] <= 2).all()
