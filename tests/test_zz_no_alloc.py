"""segpaged_decode_static: the decode entry point that allocates nothing.

Its scratch is the library's static device array instead of a caller
workspace; its results must equal those of segpaged_decode bit for bit (same
plan, same kernels).  Two calls in a row on the GPU, the second with a smaller
input, so the second reads a scratch the first has left full.  The size limit
is checked on the host before any GPU work, so that part runs on the CPU.
"""
import numpy as np
import pytest

import synth
from synth import custom_layout, GLOBAL, LOCAL
from head_aware_paged_page_amd import segpaged as sp


def _decode_both(w, torch):
    """segpaged_decode with the workload's workspace, then segpaged_decode_static."""
    args = dict(page_size=w.ps, group=w.G, n_seq=w.n_seq, n_slot=w.n_slot, h_row_ptr=w.td["row_ptr"],
                d_q_pos=w.d_q_dec, d_cls=w.d_cls, d_window=w.d_window, d_row_ptr=w.d_row_ptr,
                d_entries=w.d_entries, scale=w.scale)
    o_ref = torch.full_like(w.q_decode, float("nan"))
    l_ref = torch.full(w.q_decode.shape[:2], float("nan"), dtype=torch.float32, device="cuda")
    sp.decode(w.q_decode, w.k_pool, w.v_pool, out=o_ref, lse=l_ref, workspace=w.workspace, **args)
    o = torch.full_like(o_ref, float("nan"))
    l = torch.full_like(l_ref, float("nan"))
    sp.decode_static(w.q_decode, w.k_pool, w.v_pool, out=o, lse=l, **args)
    torch.cuda.synchronize()
    return o_ref, l_ref, o, l


@pytest.mark.gpu
def test_decode_static_matches_decode_on_two_calls():
    torch = pytest.importorskip("torch")
    from head_aware_paged_page_amd.workload import Workload
    big = synth.make_layout("32k")
    many = custom_layout(seg_lens=[[6000]] * 4, offline=[[0]] * 4, n_prefill=16, n_decode=1,
                         classes=[(GLOBAL, 0) if s % 2 == 0 else (LOCAL, 64) for s in range(50)], page_size=16,
                         head_dim=64, group=2, dtype="bf16", name="many_rows", seed=3)
    small = custom_layout(seg_lens=[[300, 77]], offline=[[0, -40]], n_prefill=20, n_decode=1,
                          classes=[(GLOBAL, 0), (LOCAL, 100)], page_size=16, head_dim=128, group=4, dtype="bf16",
                          name="small", seed=1)
    for lay in (big, many, small):     # each call smaller than the one before it
        print(f"[case] decode_static {lay.name}: {lay.n_slot} slots x {lay.n_seq} seqs", flush=True)
        w = Workload(lay, device="cuda")
        assert w.ws_decode <= sp.SP_STATIC_SCRATCH_BYTES
        o_ref, l_ref, o, l = _decode_both(w, torch)
        assert not torch.isnan(o_ref.float()).any() and not torch.isnan(l_ref).any()
        assert torch.equal(o, o_ref), lay.name
        assert torch.equal(l, l_ref), lay.name
        del w
        torch.cuda.empty_cache()


def test_decode_static_rejects_calls_beyond_its_scratch():
    """A call whose plan needs more than SP_STATIC_SCRATCH_BYTES fails with
    SP_EWORKSPACE before any GPU work (so this runs without a GPU); the message
    names both sizes."""
    import ctypes
    n_rows = 40000
    row_ptr = (np.arange(n_rows + 1, dtype=np.int64) * 700).astype(np.int32)
    need = sp.workspace_bytes(sp.SP_WS_DECODE, sp.SP_BF16, 128, 16, 16, 1, n_rows, None, row_ptr)
    assert need > sp.SP_STATIC_SCRATCH_BYTES
    L = sp.lib()
    fake = ctypes.c_void_p(256)        # never dereferenced: the call fails before any GPU work
    rc = L.segpaged_decode_static(sp.SP_BF16, 128, 16, 16, 1, n_rows, sp._ptr(row_ptr), fake, fake, fake, fake,
                                  fake, fake, fake, fake, 1 << 20, ctypes.c_float(0.088), fake, None, None)
    assert rc == sp.SP_EWORKSPACE
    msg = L.segpaged_last_error().decode()
    assert str(need) in msg and str(sp.SP_STATIC_SCRATCH_BYTES) in msg, msg
