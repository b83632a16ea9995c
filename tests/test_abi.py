"""Host-side tests of the C ABI (no GPU needed): the library loads, exports every function
that include/gdn.h declares, sizes workspaces as documented, and rejects bad arguments
before any HIP call."""
import ctypes
import os
import re

import pytest

from gated_delta_rule_42_amd import binding as gb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

OK, ERR_NULL, ERR_SHAPE, ERR_DTYPE, ERR_ALIGN, ERR_UNSUP, ERR_WS = 0, -1, -2, -3, -4, -5, -6


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(gb.LIB_PATH):
        from gated_delta_rule_42_amd import build
        build.build()
    return gb.lib()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("gdn_chunk_fwd", "gdn_decode_step", "gdn_chunk_prepare", "gdn_chunk_propagate",
              "gdn_chunk_fwd_workspace_bytes", "gdn_status_string", "gdn_version"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name
    bound = {n for n, _, _ in gb._SIGNATURES}
    assert bound == set(declared_functions())


def test_only_c_abi_is_exported():
    """The shared object exports the gdn_* C functions and no C++ symbols of its own."""
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", gb.LIB_PATH], capture_output=True, text=True).stdout
    mine = [l.split()[-1] for l in out.splitlines() if " T " in l]
    assert set(declared_functions()) <= set(mine)
    assert not [m for m in mine if m.startswith("_ZN3gdn")]


def test_version_and_status_strings(L):
    assert gb.gdn_version() >= 100
    for s in range(-7, 1):
        assert len(gb.gdn_status_string(s)) >= 2
    assert gb.gdn_status_string(-99) == "unknown status"


def test_workspace_bytes(L, monkeypatch):
    monkeypatch.setenv("GDN_SEGMENT_CHUNKS", "0")   # the stage-1 regions alone
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    # B4 H16 T2048 bf16: 128 chunks x 16 heads
    nc, H = 4 * 32, 16
    expect = (al(nc * H * 128 * 4) + al(nc * H * 4096 * 2) + al(nc * H * 4096 * 2)
              + al(nc * H * 64 * 128 * 2) + nc * H * 64 * 128 * 2)   # + fp16 K and scaled Q
    assert gb.gdn_chunk_fwd_workspace_bytes(4, 2048, 16, 128, 128, 4, False) == expect
    # packed: bound floor((T + N*63)/64), plus the chunk table
    T, N, H = 1000, 5, 2
    ncb = (T + N * 63) // 64
    expect = al((2 * N + 1) * 4) + al(ncb * H * 128 * 4) + al(ncb * H * 4096 * 4) + ncb * H * 4096 * 4
    import torch
    assert gb.gdn_chunk_fwd_workspace_bytes(1, T, H, 64, 64, N, True, dtype=torch.float32) == expect
    assert gb.gdn_chunk_fwd_workspace_bytes(1, 0, 2, 64, 64, 1, False) == 0
    # rejected arguments give 0
    assert L.gdn_chunk_fwd_workspace_bytes(1, 10, 2, 96, 64, 1, 0, 64, 1) == 0
    assert L.gdn_chunk_fwd_workspace_bytes(1, 10, 2, 64, 64, 1, 0, 32, 1) == 0
    assert L.gdn_chunk_fwd_workspace_bytes(2, 10, 2, 64, 64, 3, 0, 64, 1) == 0
    assert L.gdn_chunk_fwd_workspace_bytes(2, 10, 2, 64, 64, 3, 1, 64, 1) == 0


def _fwd_base_bytes(B, T, H, d):
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    nc = B * ((T + 63) // 64)
    return (al(nc * H * 128 * 4) + al(nc * H * 4096 * 2) + al(nc * H * 4096 * 2)
            + al(nc * H * 64 * d * 2) + nc * H * 64 * d * 2)


def _seg_bytes(N, H, d, ns, sl):
    ncp = (sl - 1).bit_length()   # offsets 1, 2, 4, .. below sl
    return N * H * ns * (ncp + 2) * d * d * 4 + N * H * max(1, d // 64) * ns * 4


def test_segment_plan_workspace(L, monkeypatch):
    """The long-chain split's plan, read from the workspace size.

    Two-stage path (GDN_FUSED=0, and the default from 64 (sequence, head) pairs on): about 256
    work-groups of 64-column tiles with segments of at least 16 chunks, so the long-context shape
    (B1 H16 T32768 d128 bf16: 32 tiles) gets 8 segments of 64 chunks (6 records each), B2 H16
    T2048 (64 tiles) 2 of 16, the training shape (B4 H16 T2048: 256 tiles of 32 columns) and
    B8 none. One-kernel path (bf16 d128, the default below 64 pairs, GDN_FUSED=1): one
    work-group per pair, segments of at least 8 chunks: the long-context shape gets 16 of 32,
    B2 H16 T2048 4 of 8 and, forced, the training shape 4 of 8. fp32 inputs are never split;
    GDN_SEGMENT_CHUNKS forces a length or turns the split off."""
    import torch
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    monkeypatch.delenv("GDN_SEGMENT_CHUNKS", raising=False)
    monkeypatch.delenv("GDN_FUSED", raising=False)
    ws = gb.gdn_chunk_fwd_workspace_bytes
    # default paths: one kernel for the long-context shape and B2, two stages for B4 and B8
    assert ws(1, 32768, 16, 128, 128, 1, False) == al(_fwd_base_bytes(1, 32768, 16, 128)) + _seg_bytes(1, 16, 128, 16, 32)
    assert ws(2, 2048, 16, 128, 128, 2, False) == al(_fwd_base_bytes(2, 2048, 16, 128)) + _seg_bytes(2, 16, 128, 4, 8)
    for B in (4, 8):
        assert ws(B, 2048, 16, 128, 128, B, False) == _fwd_base_bytes(B, 2048, 16, 128)
    monkeypatch.setenv("GDN_FUSED", "0")
    assert ws(1, 32768, 16, 128, 128, 1, False) == al(_fwd_base_bytes(1, 32768, 16, 128)) + _seg_bytes(1, 16, 128, 8, 64)
    assert ws(2, 2048, 16, 128, 128, 2, False) == al(_fwd_base_bytes(2, 2048, 16, 128)) + _seg_bytes(2, 16, 128, 2, 16)
    monkeypatch.setenv("GDN_FUSED", "1")
    assert ws(4, 2048, 16, 128, 128, 4, False) == al(_fwd_base_bytes(4, 2048, 16, 128)) + _seg_bytes(4, 16, 128, 4, 8)
    # fewer than 16 chunks: no split on the one-kernel path
    assert ws(1, 15 * 64, 2, 128, 128, 1, False) == _fwd_base_bytes(1, 15 * 64, 2, 128)
    monkeypatch.delenv("GDN_FUSED")
    f32 = ws(1, 32768, 16, 128, 128, 1, False, dtype=torch.float32)
    assert f32 == ws(1, 32768, 256, 128, 128, 1, False, dtype=torch.float32) // 16
    # one head of d 64 (one tile): 256 segments wanted, but at least 16 chunks each: 32 x 16
    base = _fwd_base_bytes(1, 32768, 1, 64)
    assert ws(1, 32768, 1, 64, 64, 1, False) == al(base) + _seg_bytes(1, 1, 64, 32, 16)
    # fewer than 32 chunks: no split
    assert ws(1, 31 * 64, 1, 64, 64, 1, False) == _fwd_base_bytes(1, 31 * 64, 1, 64)
    monkeypatch.setenv("GDN_SEGMENT_CHUNKS", "3")
    base = _fwd_base_bytes(2, 849, 2, 128)   # 14 chunks per sequence: 5 segments of 3
    assert ws(2, 849, 2, 128, 128, 2, False) == al(base) + _seg_bytes(2, 2, 128, 5, 3)
    monkeypatch.setenv("GDN_SEGMENT_CHUNKS", "0")
    assert ws(1, 32768, 16, 128, 128, 1, False) == _fwd_base_bytes(1, 32768, 16, 128)


def test_bwd_workspace_bytes(L):
    """The backward workspace is the region list of its header: the forward's regions with
    fp32 operators, then T, the state entering each chunk and the state gradient, and for bf16
    inputs the K and Q images; T and the entering state are fp16 for bf16 inputs."""
    import torch
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731

    def expect(nc, H, dk, dv, bf16, varlen_n=None):
        fwd = (al((2 * varlen_n + 1) * 4) if varlen_n else 0) + al(nc * H * 128 * 4) \
            + al(nc * H * 4096 * 4) + nc * H * 4096 * 4
        e16 = 2 if bf16 else 4
        off = al(al(al(fwd) + nc * H * 4096 * e16) + nc * H * dv * dk * e16)
        end = off + nc * H * dv * dk * 4
        if bf16:
            end = al(al(end) + nc * H * 64 * dk * 2) + nc * H * 64 * dk * 2
        return end

    # B4 H16 T2048 d128: 128 chunks x 16 heads
    for dt, bf16 in ((torch.float32, False), (torch.bfloat16, True)):
        assert gb.gdn_chunk_bwd_workspace_bytes(4, 2048, 16, 128, 128, 4, False, dtype=dt) == \
            expect(128, 16, 128, 128, bf16)
    # packed, d_k != d_v: chunk bound floor((T + N*63)/64) and the chunk table
    T, N, H = 1000, 5, 2
    ncb = (T + N * 63) // 64
    for dt, bf16 in ((torch.float32, False), (torch.bfloat16, True)):
        assert gb.gdn_chunk_bwd_workspace_bytes(1, T, H, 64, 128, N, True, dtype=dt) == \
            expect(ncb, H, 64, 128, bf16, varlen_n=N)
    assert gb.gdn_chunk_bwd_workspace_bytes(1, 0, 2, 64, 64, 1, False) == 0


FAKE = 1 << 20  # an aligned, never dereferenced address: every call below fails validation


def fwd(L, q=FAKE, k=FAKE, v=FAKE, g=FAKE, b=FAKE, h0=None, o=FAKE, hT=None, cu=None, chunk=64,
        B=1, T=128, H=2, dk=64, dv=64, N=1, dtype=1, o_dtype=1, ws=None, wsb=0):
    return L.gdn_chunk_fwd(q, k, v, g, b, h0, o, hT, cu, chunk, B, T, H, dk, dv, N, dtype, o_dtype,
                           ws, wsb, None)


def test_chunk_fwd_rejects_before_any_launch(L):
    assert fwd(L, dtype=7) == ERR_DTYPE
    assert fwd(L, o_dtype=3) == ERR_DTYPE
    assert fwd(L, dtype=0, o_dtype=1) == ERR_DTYPE        # bf16 o needs bf16 inputs
    assert fwd(L, chunk=32) == ERR_UNSUP
    assert fwd(L, dk=96) == ERR_UNSUP
    assert fwd(L, dv=256) == ERR_UNSUP
    assert fwd(L, H=0) == ERR_SHAPE
    assert fwd(L, T=-1) == ERR_SHAPE
    assert fwd(L, B=2, N=1) == ERR_SHAPE
    assert fwd(L, B=2, N=2, cu=FAKE) == ERR_SHAPE          # packed sequences need B == 1
    assert fwd(L, q=None) == ERR_NULL
    assert fwd(L, o=None) == ERR_NULL
    assert fwd(L, g=None) == ERR_NULL
    assert fwd(L, v=FAKE + 2) == ERR_ALIGN
    assert fwd(L, h0=FAKE + 4) == ERR_ALIGN
    assert fwd(L, g=FAKE + 2) == ERR_ALIGN
    assert fwd(L) == ERR_WS                                # workspace required
    assert fwd(L, ws=FAKE, wsb=100) == ERR_WS              # too small
    need = L.gdn_chunk_fwd_workspace_bytes(1, 128, 2, 64, 64, 1, 0, 64, 1)
    assert fwd(L, ws=FAKE + 16, wsb=need) == ERR_ALIGN     # workspace needs 256 B alignment


def test_stage_entry_points_validate(L):
    assert L.gdn_chunk_prepare(None, FAKE, FAKE, FAKE, None, 64, 1, 128, 2, 64, 64, 1, 1, None, 0, None) == ERR_NULL
    assert L.gdn_chunk_prepare(FAKE, FAKE, FAKE, FAKE, None, 64, 1, 128, 2, 64, 64, 1, 1, None, 0, None) == ERR_WS
    assert L.gdn_chunk_propagate(FAKE, FAKE, None, None, FAKE, None, None, 64, 1, 128, 2, 64, 64, 1, 1,
                                 1, None, 0, None) == ERR_NULL
    assert L.gdn_chunk_propagate(FAKE, FAKE, FAKE, None, FAKE, None, None, 64, 1, 128, 2, 64, 64, 1, 3,
                                 0, None, 0, None) == ERR_DTYPE


def test_decode_rejects_before_any_launch(L):
    def dec(q=FAKE, state=FAKE, N=4, H=2, dk=128, dv=128, dtype=1, o_dtype=0):
        return L.gdn_decode_step(q, FAKE, FAKE, FAKE, FAKE, state, FAKE, N, H, dk, dv, dtype, o_dtype, None)
    assert dec(dtype=2) == ERR_DTYPE
    assert dec(o_dtype=5) == ERR_DTYPE
    assert dec(dk=32) == ERR_UNSUP
    assert dec(N=0) == ERR_SHAPE
    assert dec(q=None) == ERR_NULL
    assert dec(state=FAKE + 4) == ERR_ALIGN


def test_binding_refuses_cpu_tensors(L):
    import torch
    x = torch.zeros(1, 64, 2, 64)
    g = torch.zeros(1, 64, 2)
    with pytest.raises(ValueError):
        gb.gdn_chunk_fwd(x, x, x, g, g)
    with pytest.raises(ValueError):
        gb.gdn_decode_step(x[0], x[0], x[0], g[0], g[0], torch.zeros(1, 64, 2, 64, 64))


# ---------------------------------------------------------------- binding argument checks
# The C ABI sees raw pointers only, so the binding checks shapes and dtypes before any call:
# a mismatched tensor would otherwise be read or written out of bounds on the device. These
# run on CPU tensors; the shape and dtype checks come before the device check.
def _fwd_inputs(B=1, T=8, H=2, dk=64, dv=64, dtype=None):
    import torch
    dtype = dtype or torch.bfloat16
    q = torch.zeros(B, T, H, dk, dtype=dtype)
    return dict(q=q, k=q.clone(), v=torch.zeros(B, T, H, dv, dtype=dtype),
                g=torch.zeros(B, T, H), beta=torch.zeros(B, T, H))


@pytest.mark.parametrize("bad", ["k_dtype", "k_shape", "v_dtype", "v_rows", "g_dtype", "g_shape",
                                 "beta_shape", "h0_shape", "h0_dtype", "hT_shape", "o_shape",
                                 "cu_int64", "cu_2d"])
def test_binding_rejects_mismatched_forward_arguments(bad):
    import torch
    x = _fwd_inputs()
    kw = {}
    if bad == "k_dtype":
        x["k"] = x["k"].float()
    elif bad == "k_shape":
        x["k"] = torch.zeros(1, 8, 2, 32, dtype=torch.bfloat16)
    elif bad == "v_dtype":
        x["v"] = x["v"].float()
    elif bad == "v_rows":
        x["v"] = torch.zeros(1, 7, 2, 64, dtype=torch.bfloat16)
    elif bad == "g_dtype":
        x["g"] = x["g"].double()
    elif bad == "g_shape":
        x["g"] = torch.zeros(1, 8, 3)
    elif bad == "beta_shape":
        x["beta"] = torch.zeros(8, 2)
    elif bad == "h0_shape":
        kw["h0"] = torch.zeros(1, 2, 64, 32)
    elif bad == "h0_dtype":
        kw["h0"] = torch.zeros(1, 2, 64, 64, dtype=torch.bfloat16)
    elif bad == "hT_shape":
        kw["hT"] = torch.zeros(2, 2, 64, 64)
    elif bad == "o_shape":
        kw["o"] = torch.zeros(1, 8, 2, 32, dtype=torch.bfloat16)
    elif bad == "cu_int64":
        kw["cu_seqlens"] = torch.tensor([0, 8], dtype=torch.int64)
    elif bad == "cu_2d":
        kw["cu_seqlens"] = torch.tensor([[0, 8]], dtype=torch.int32)
    with pytest.raises(ValueError, match="gdn: "):
        gb.gdn_chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], **kw)


def test_binding_rejects_cpu_tensors_after_shape_checks():
    x = _fwd_inputs()
    with pytest.raises(ValueError, match="on a GPU"):
        gb.gdn_chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"])


@pytest.mark.parametrize("bad", ["state_bf16", "state_shape", "g_shape", "o_shape", "v_dtype"])
def test_binding_rejects_mismatched_decode_arguments(bad):
    import torch
    N, H, d = 2, 2, 64
    q = torch.zeros(N, H, d, dtype=torch.bfloat16)
    a = dict(q=q, k=q.clone(), v=q.clone(), g=torch.zeros(N, H), beta=torch.zeros(N, H),
             state=torch.zeros(N, H, d, d), o=None)
    if bad == "state_bf16":
        a["state"] = a["state"].bfloat16()
    elif bad == "state_shape":
        a["state"] = torch.zeros(N, H, d, 32)
    elif bad == "g_shape":
        a["g"] = torch.zeros(N, H, d)
    elif bad == "o_shape":
        a["o"] = torch.zeros(N, H, 32)
    elif bad == "v_dtype":
        a["v"] = a["v"].float()
    with pytest.raises(ValueError, match="gdn: "):
        gb.gdn_decode_step(a["q"], a["k"], a["v"], a["g"], a["beta"], a["state"], a["o"])


def test_binding_rejects_mismatched_backward_and_channel_gate_arguments():
    import torch
    x = _fwd_inputs()
    with pytest.raises(ValueError, match="do has"):
        gb.gdn_chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["v"].float())
    with pytest.raises(ValueError, match="g has shape"):   # channel-wise decay needs [B,T,H,dk]
        gb.gdn_kda_chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"])
    gc = torch.zeros(1, 8, 2, 64)
    with pytest.raises(ValueError, match="write has shape"):
        gb.gdn_decoupled_chunk_fwd(x["q"], x["k"], x["v"], gc, gc, torch.zeros(1, 8, 2, 32))
