"""Window-only storage and page release on the GPU.

With window-only storage each head keeps only the pages its queries can read
(local heads their window, retrieval heads their listed pages).  The kernels
are unchanged: relocation runs over the stored pages only, and prefill and
decode read the same logical tables with other physical ids, so their results
must be bit-identical to those of whole-chain storage and match the oracle.
In a decode loop, pages released after each token are filled with NaN (as if
another session had taken them): any read of a released page would show.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth
from synth import custom_layout, GLOBAL, LOCAL, RETRIEVAL
from oracle import attention as oatt
from oracle import rope as orope
from oracle import tables as otab
import head_aware_paged_page_amd.segpaged as sp

pytestmark = pytest.mark.gpu


def _wl(lay, **kw):
    from head_aware_paged_page_amd.workload import Workload
    print(f"[case] {lay.name} window_only={kw.get('window_only', False)}", flush=True)
    return Workload(lay, device="cuda", **kw)


def _host(t):
    return t.double().cpu().numpy()


def test_32k_window_only_equals_whole_chains_and_oracle():
    lay = synth.make_layout("32k")
    full = _wl(lay)
    win = _wl(lay, window_only=True)
    assert win.n_phys == 10 * 1883 + 54 * 22 and full.n_phys == 64 * 1883
    for w in (full, win):
        w.relocate()
        w.prefill(k=w.k_reloc)
        w.decode(k=w.k_reloc)
    torch.cuda.synchronize()
    assert torch.equal(full.out_prefill, win.out_prefill) and torch.equal(full.lse_prefill, win.lse_prefill)
    assert torch.equal(full.out_decode, win.out_decode) and torch.equal(full.lse_decode, win.lse_decode)
    # relocation touched exactly the stored segment keys, with the same results
    ctx = lay.ctx_len(0)
    on = np.concatenate([np.arange(o, o + l) for o, l in zip(lay.seg_online[0], lay.seg_len[0])])
    off = np.concatenate([np.arange(o, o + l) for o, l in zip(lay.seg_offline[0], lay.seg_len[0])])
    for slot in (int(np.nonzero(lay.cls == GLOBAL)[0][0]), int(np.nonzero(lay.cls == LOCAL)[0][0])):
        a = win.gather_keys(win.k_reloc, slot, 0)
        b = full.gather_keys(full.k_reloc, slot, 0)
        stored = ~np.isnan(a[:, 0])
        assert stored[ctx:].all() and np.array_equal(a[stored], b[stored])
        if lay.cls[slot] == LOCAL:      # pages 296..312 of the last segment reach position 30000 - 256 + 1
            assert stored[:ctx].sum() == 30000 - (25000 + 296 * 16)
        K, _ = win.unit_host(slot, 0)
        want = orope.relocate(K[:ctx], off, on, lay.theta)
        assert np.max(np.abs(a[:ctx][stored[:ctx]] - want[stored[:ctx]])) <= 2e-2
    # KV bytes per session
    page = 2 * 16 * 128 * 2
    print(f"[window] 32K session: {full.n_phys * page / 1e6:.1f} MB whole chains, {win.n_phys * page / 1e6:.1f} MB "
          f"window-only ({full.n_phys / win.n_phys:.2f}x); relocation items {len(full.tp['reloc'])} -> "
          f"{len(win.tp['reloc'])}")


def test_decode_loop_releases_pages_as_the_window_slides():
    """A 40-token decode after a 20-token prefill chunk: before each token the
    pages no later query can read are released and filled with NaN; the new
    token's tables come from the remaining chains; every output matches the
    oracle.  A local chain never holds more than its window's pages (plus one
    for a window that straddles pages) and those of the tokens still to come."""
    lens = [[300, 200]]
    ps, W1, W2 = 16, 32, 64
    nsp = -(-300 // ps) + -(-200 // ps)
    ret = np.sort(np.random.default_rng(4).choice(nsp, size=5, replace=False))
    lay = custom_layout(seg_lens=lens, offline=[[0, -77]], n_prefill=20, n_decode=40,
                        classes=[(GLOBAL, 0), (LOCAL, W1), (LOCAL, W2), (RETRIEVAL, 0)], page_size=ps, head_dim=128,
                        group=4, dtype="bf16", ret_lists={(3, 0): ret}, name="slide", seed=2)
    w = _wl(lay, window_only=True)
    G, E = lay.group, int(lay.new_base[0])
    w.relocate()
    w.prefill(k=w.k_reloc)
    torch.cuda.synchronize()
    ctx = lay.ctx_len(0)
    on = np.concatenate([np.arange(o, o + l) for o, l in zip(lay.seg_online[0], lay.seg_len[0])])
    off = np.concatenate([np.arange(o, o + l) for o, l in zip(lay.seg_offline[0], lay.seg_len[0])])
    KV = {}
    for slot in range(lay.n_slot):
        K, V = w.unit_host(slot, 0)
        K[:ctx] = orope.relocate(K[:ctx], off, on, lay.theta)
        KV[slot] = (K, V)
    for slot in range(lay.n_slot):                     # the prefill chunk itself
        O, _, _ = oatt.row_attention(lay, slot, 0, *KV[slot], _host(w.q_prefill[:, slot * G:(slot + 1) * G]),
                                     E + np.arange(lay.n_prefill))
        assert np.max(np.abs(_host(w.out_prefill[:, slot * G:(slot + 1) * G]) - O)) <= 2e-2
    q_all = synth.seq_queries(lay, 0, device="cuda")
    storage = w.tp["storage"].copy()
    chain_ptr = w.tp["chain_ptr"]
    o_storage = storage.astype(np.int64).copy()
    n_released = 0
    out = torch.empty((1, lay.n_slot * G, lay.head_dim), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((1, lay.n_slot * G), dtype=torch.float32, device="cuda")
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    for j in range(lay.n_decode):
        p = E + lay.n_prefill + j
        rel = sp.release_pages(**w.layout_args, page_size=ps, p_next=[p], chain_ptr=chain_ptr, storage=storage)
        o_rel, o_storage = otab.release(lay, o_storage, chain_ptr, [p])
        assert np.array_equal(rel, o_rel), f"released ids before token {j}"
        n_released += len(rel)
        if len(rel):
            ids = torch.as_tensor(rel.astype(np.int64), device="cuda")
            w.k_reloc[ids] = float("nan")
            w.v_pool[ids] = float("nan")
        for slot, Wl in ((1, W1), (2, W2)):   # live pages of a local chain: its window's, and those of later tokens
            live = int((storage[chain_ptr[slot]:chain_ptr[slot + 1]] >= 0).sum())
            assert live <= -(-Wl // ps) + 1 + -(-(E + lay.n_new - p) // ps), (slot, j, live)
        rp, ent = sp.tables_from_chains(**w.layout_args, q_lo=[p], q_hi=[p], page_size=ps, chain_ptr=chain_ptr,
                                        storage=storage)
        q = q_all[lay.n_prefill + j:lay.n_prefill + j + 1].contiguous()
        assert sp.workspace_bytes(sp.SP_WS_DECODE, sp.SP_BF16, 128, ps, G, 1, lay.n_slot, None, rp) <= ws.numel()
        sp.decode(q, w.k_reloc, w.v_pool, page_size=ps, group=G, n_seq=1, n_slot=lay.n_slot, h_row_ptr=rp,
                  d_q_pos=torch.tensor([p], dtype=torch.int32, device="cuda"), d_cls=w.d_cls, d_window=w.d_window,
                  d_row_ptr=torch.from_numpy(rp).cuda(), d_entries=torch.from_numpy(np.ascontiguousarray(ent)).cuda(),
                  scale=w.scale, out=out, lse=lse, workspace=ws)
        torch.cuda.synchronize()
        for slot in range(lay.n_slot):
            O, L, _ = oatt.row_attention(lay, slot, 0, *KV[slot], _host(q[:, slot * G:(slot + 1) * G]), [p])
            got = _host(out[:, slot * G:(slot + 1) * G])
            assert np.all(np.isfinite(got)), f"token {j}, slot {slot}: a released page was read"
            assert np.max(np.abs(got - O)) <= 2e-2, (j, slot)
            assert np.max(np.abs(lse[:, slot * G:(slot + 1) * G].double().cpu().numpy() - L)) <= 2e-2
    end = [E + lay.n_new]                               # the sequence is over: everything returns
    rel = sp.release_pages(**w.layout_args, page_size=ps, p_next=end, chain_ptr=chain_ptr, storage=storage)
    assert n_released + len(rel) == int((w.tp["storage"] >= 0).sum()) and (storage == -1).all()


@pytest.mark.parametrize("seed", range(12))
def test_window_only_random_layouts(seed):
    """The seeded random layouts of the whole-path test with window-only storage:
    prefill and decode bit-identical to whole-chain storage, and the stored
    keys' relocation identical too."""
    from test_random_layouts_gpu import _draw
    lay = _draw(seed)
    full = _wl(lay)
    win = _wl(lay, window_only=True)
    assert win.n_phys <= full.n_phys
    for w in (full, win):
        w.relocate()
        w.prefill(k=w.k_reloc)
        w.decode(k=w.k_reloc)
    torch.cuda.synchronize()
    assert torch.equal(full.out_prefill, win.out_prefill) and torch.equal(full.lse_prefill, win.lse_prefill)
    assert torch.equal(full.out_decode, win.out_decode) and torch.equal(full.lse_decode, win.lse_decode)
    for slot in range(lay.n_slot):
        for seq in range(lay.n_seq):
            a = win.gather_keys(win.k_reloc, slot, seq)
            b = full.gather_keys(full.k_reloc, slot, seq)
            stored = ~np.isnan(a[:, 0])
            assert np.array_equal(a[stored], b[stored]), (slot, seq)


@pytest.mark.parametrize("seed", range(16))
def test_window_only_random_wide_groups(seed):
    """The wide random layouts (groups 3 to 16, pages up to 64 keys, several
    query tiles per row) with window-only storage: prefill (and decode, for
    pages of 16 or 32 keys) bit-identical to whole-chain storage."""
    from test_random_layouts_gpu import _draw
    lay = _draw(seed, wide=True)
    full = _wl(lay)
    win = _wl(lay, window_only=True)
    assert win.n_phys <= full.n_phys
    dec = lay.page_size in (16, 32)
    for w in (full, win):
        w.relocate()
        w.prefill(k=w.k_reloc)
        if dec:
            w.decode(k=w.k_reloc)
    torch.cuda.synchronize()
    assert torch.equal(full.out_prefill, win.out_prefill) and torch.equal(full.lse_prefill, win.lse_prefill)
    if dec:
        assert torch.equal(full.out_decode, win.out_decode) and torch.equal(full.lse_decode, win.lse_decode)
