"""HIP path vs the fp64 oracle on the same seeded inputs (MI355X only).

Bounds: fp32 inputs (the tiny config) 1e-5 max-abs; bf16 inputs with fp32
accumulation 2e-2 max-abs; integer results (visible counts) exact.
Pools are pre-filled with NaN so that any read of a slot that holds no token
shows up in the outputs.
"""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth
from synth import custom_layout, GLOBAL, LOCAL, RETRIEVAL, DENSE
from oracle import attention as oatt
from oracle import rope as orope
from oracle import tables as otab

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}


def lse_tol(dtype, L):
    """The output bound holds for the log-sum-exp output too: max abs 2e-2 for bf16
    inputs; for fp32 inputs 1e-5 relative to |LSE| (at least 1e-5), since LSE is
    formed as m + log l in fp32."""
    return TOL["bf16"] if dtype == "bf16" else 1e-5 * max(1.0, float(np.max(np.abs(L))))


def _wl(lay, **kw):
    from head_aware_paged_page_amd.workload import Workload
    print(f"[case] {lay.name} G={lay.group} D={lay.head_dim} ps={lay.page_size} slots={lay.n_slot} "
          f"seqs={lay.n_seq}", flush=True)
    return Workload(lay, device="cuda", **kw)


_CACHE = {}


def cached(name):
    if name not in _CACHE:
        _CACHE.clear()
        torch.cuda.empty_cache()
        _CACHE[name] = _wl(synth.make_layout(name))
    return _CACHE[name]


def _host(t):
    return t.double().cpu().numpy()


def _seg_positions(lay, seq):
    if len(lay.seg_len[seq]) == 0:                       # a context with no reused segment
        return np.zeros(0, np.int64), np.zeros(0, np.int64)
    on = np.concatenate([np.arange(o, o + l) for o, l in zip(lay.seg_online[seq], lay.seg_len[seq])])
    off = np.concatenate([np.arange(o, o + l) for o, l in zip(lay.seg_offline[seq], lay.seg_len[seq])])
    return on, off


def check_prefill(w, rows=None, q_sample=None, k_pool=None, keys_fn=None):
    """Compare prefill outputs of the sampled rows (and query tokens) with the oracle."""
    lay = w.lay
    torch.cuda.synchronize()
    out, lse = _host(w.out_prefill), w.lse_prefill.cpu().numpy()
    rows = range(lay.n_slot * lay.n_seq) if rows is None else rows
    worst = 0.0
    for r in rows:
        slot, seq = divmod(r, lay.n_seq)
        K, V = w.unit_host(slot, seq)
        if keys_fn is not None:
            K = keys_fn(slot, seq, K)
        t0 = int(w.h_tok_ptr[seq])
        toks = np.arange(lay.n_prefill) if q_sample is None else q_sample
        q_pos = lay.new_base[seq] + toks
        heads = slice(slot * lay.group, (slot + 1) * lay.group)
        q = _host(w.q_prefill[t0 + toks, heads])
        O, L, cnt = oatt.row_attention(lay, slot, seq, K, V, q, q_pos)
        got = out[t0 + toks, heads]
        err = np.max(np.abs(got - O))
        worst = max(worst, err)
        assert np.all(np.isfinite(got)), f"row {r}: non-finite output"
        assert err <= TOL[lay.dtype], f"row {r} (class {lay.cls[slot]}): max abs err {err}"
        assert np.max(np.abs(lse[t0 + toks, heads] - L)) <= lse_tol(lay.dtype, L)
    return worst


def check_decode(w, rows=None, keys_fn=None):
    lay = w.lay
    torch.cuda.synchronize()
    out, lse = _host(w.out_decode), w.lse_decode.cpu().numpy()
    rows = range(lay.n_slot * lay.n_seq) if rows is None else rows
    for r in rows:
        slot, seq = divmod(r, lay.n_seq)
        K, V = w.unit_host(slot, seq)
        if keys_fn is not None:
            K = keys_fn(slot, seq, K)
        heads = slice(slot * lay.group, (slot + 1) * lay.group)
        q = _host(w.q_decode[seq:seq + 1, heads])
        O, L, cnt = oatt.row_attention(lay, slot, seq, K, V, q, [lay.new_base[seq] + lay.n_prefill])
        got = out[seq:seq + 1, heads]
        err = np.max(np.abs(got - O))
        assert np.all(np.isfinite(got)), f"row {r}: non-finite output"
        assert err <= TOL[lay.dtype], f"row {r} (class {lay.cls[slot]}): max abs err {err}"
        assert np.max(np.abs(lse[seq:seq + 1, heads] - L)) <= lse_tol(lay.dtype, L)


def check_relocate(w, rows=None):
    lay = w.lay
    torch.cuda.synchronize()
    rows = range(lay.n_slot * lay.n_seq) if rows is None else rows
    for r in rows:
        slot, seq = divmod(r, lay.n_seq)
        K, _ = w.unit_host(slot, seq)
        ctx = lay.ctx_len(seq)
        on, off = _seg_positions(lay, seq)
        want = orope.relocate(K[:ctx], off, on, lay.theta)
        got = w.gather_keys(w.k_reloc, slot, seq)
        if ctx:                                          # a row with reused keys
            err = np.max(np.abs(got[:ctx] - want))
            assert err <= TOL[lay.dtype], f"row {r}: relocation max abs err {err}"
        # new-token keys are not touched
        assert np.array_equal(got[ctx:], w.gather_keys(w.k_pool, slot, seq)[ctx:])


def _rows_by_class(lay, per_class=2, seed=0):
    rng = np.random.default_rng(seed)
    rows = set()
    for c in (GLOBAL, LOCAL, RETRIEVAL, DENSE):
        slots = np.nonzero(lay.cls == c)[0]
        for slot in rng.choice(slots, size=min(per_class, len(slots)), replace=False) if len(slots) else []:
            rows.add(int(slot) * lay.n_seq + int(rng.integers(0, lay.n_seq)))
    return sorted(rows)


# ---------------------------------------------------------------- tiny fp32 config: everything, 1e-5

def test_tiny_fp32_all_calls():
    w = _wl(synth.make_layout("tiny"))
    w.relocate()
    check_relocate(w)
    # Delta = 0 (first segment) is the identity, bit for bit
    lay = w.lay
    for slot in range(lay.n_slot):
        a = w.gather_keys(w.k_reloc, slot, 0)[:256]
        b = w.gather_keys(w.k_pool, slot, 0)[:256]
        assert np.array_equal(a, b)
    w.prefill()
    check_prefill(w)
    w.decode()
    check_decode(w)
    # end to end: relocated keys feed prefill and decode; oracle relocates in fp64
    def reloc_keys(slot, seq, K):
        ctx = lay.ctx_len(seq)
        on, off = _seg_positions(lay, seq)
        K = K.copy()
        K[:ctx] = orope.relocate(K[:ctx], off, on, lay.theta)
        return K
    w.prefill(k=w.k_reloc)
    check_prefill(w, keys_fn=reloc_keys)
    w.decode(k=w.k_reloc)
    check_decode(w, keys_fn=reloc_keys)


def test_relocate_plus_minus_delta_roundtrip():
    for name in ("tiny", "32k"):
        w = cached(name) if name != "tiny" else _wl(synth.make_layout(name))
        back = w.d_reloc.clone()
        back[:, 1] = -back[:, 1]
        w.relocate()
        from head_aware_paged_page_amd import segpaged as sp
        tmp = torch.empty_like(w.k_pool)
        tmp.copy_(w.k_reloc)
        sp.rope_relocate(w.k_reloc, tmp, w.ps, back, w.lay.theta)
        torch.cuda.synchronize()
        lay = w.lay
        for r in _rows_by_class(lay, 1) if name != "tiny" else range(lay.n_slot):
            slot, seq = divmod(r, lay.n_seq)
            a = w.gather_keys(tmp, slot, seq)
            b = w.gather_keys(w.k_pool, slot, seq)
            assert np.max(np.abs(a - b)) <= TOL[lay.dtype]


# ---------------------------------------------------------------- small bf16 layouts: several tiles, ragged tails

SMALL = [
    # (group, head_dim, page_size, seg_lens, n_prefill, classes)
    (4, 128, 16, [[300, 77, 513]], 70, [(GLOBAL, 0), (LOCAL, 100), (RETRIEVAL, 0), (DENSE, 0), (LOCAL, 1)]),
    (8, 128, 32, [[1000, 33], [64]], 45, [(LOCAL, 257), (GLOBAL, 0), (RETRIEVAL, 0)]),
    (1, 64, 16, [[200, 31]], 150, [(GLOBAL, 0), (LOCAL, 40), (LOCAL, 1)]),
    (2, 64, 64, [[129, 700]], 33, [(GLOBAL, 0), (LOCAL, 65)]),
    (16, 128, 16, [[17]], 9, [(GLOBAL, 0), (LOCAL, 5)]),
    (3, 128, 16, [[450], [90, 91]], 40, [(LOCAL, 64), (GLOBAL, 0)]),
]


def _small(i, dtype="bf16", seed=0):
    G, D, ps, lens, npf, classes = SMALL[i]
    r = np.random.default_rng(seed + i)
    off = [list(r.integers(-5000, 5000, size=len(l))) for l in lens]
    ret = {}
    for slot, (c, _) in enumerate(classes):
        if c == RETRIEVAL:
            for q in range(len(lens)):
                nsp = sum(-(-l // ps) for l in lens[q])
                ret[(slot, q)] = np.sort(r.choice(nsp, size=max(1, nsp // 3), replace=False))
    return custom_layout(seg_lens=lens, offline=off, n_prefill=npf, n_decode=1, classes=classes, page_size=ps,
                         head_dim=D, group=G, dtype=dtype, ret_lists=ret, name=f"small{i}", seed=seed)


@pytest.mark.parametrize("i", range(len(SMALL)))
def test_small_layouts_bf16(i):
    lay = _small(i)
    if lay.page_size == 64:
        w = _wl(lay)
        w.prefill()
        check_prefill(w)
        return
    w = _wl(lay)
    w.relocate()
    check_relocate(w)
    w.prefill()
    check_prefill(w)
    w.decode()
    check_decode(w)


@pytest.mark.parametrize("i", [0, 2])
def test_small_layouts_fp32(i):
    lay = _small(i, dtype="f32")
    w = _wl(lay)
    w.relocate()
    check_relocate(w)
    w.prefill()
    check_prefill(w)
    w.decode()
    check_decode(w)


def test_visible_counts_from_zero_queries():
    """Q = 0 makes every visible score 0: weights are exactly 1, so exp(LSE) is the
    visible count (exact in fp32 below 2^24) and the output is the mean of V."""
    for i in (0, 1):
        lay = _small(i)
        w = _wl(lay)
        zq = torch.zeros_like(w.q_prefill)
        zd = torch.zeros_like(w.q_decode)
        _, lse_p = w.prefill(q=zq)
        _, lse_d = w.decode(q=zd)
        torch.cuda.synchronize()
        lp, ld = lse_p.cpu().numpy(), lse_d.cpu().numpy()
        for slot in range(lay.n_slot):
            for seq in range(lay.n_seq):
                t0 = int(w.h_tok_ptr[seq])
                q_pos = lay.new_base[seq] + np.arange(lay.n_prefill)
                cnt = otab.visible_counts(lay, slot, seq, q_pos)
                got = np.rint(np.exp(lp[t0:t0 + lay.n_prefill, slot * lay.group:(slot + 1) * lay.group]))
                assert np.array_equal(got, np.repeat(cnt[:, None], lay.group, axis=1))
                cd = otab.visible_counts(lay, slot, seq, [lay.new_base[seq] + lay.n_prefill])
                gd = np.rint(np.exp(ld[seq, slot * lay.group:(slot + 1) * lay.group]))
                assert np.all(gd == cd[0])


def test_window_one_returns_own_value_bit_exact():
    lay = custom_layout(seg_lens=[[100, 40]], offline=[[0, 7]], n_prefill=37, n_decode=1, classes=[(LOCAL, 1)] * 2,
                        page_size=16, head_dim=128, group=4, dtype="bf16", name="w1")
    w = _wl(lay)
    out, _ = w.prefill()
    outd, _ = w.decode()
    torch.cuda.synchronize()
    for slot in range(2):
        V = synth.unit_values(lay, slot, 0, device="cuda")["new_v"]
        for g in range(4):
            assert torch.equal(out[:, slot * 4 + g], V[:37])
            assert torch.equal(outd[0, slot * 4 + g], V[37])


def test_free_list_permutation_gives_identical_outputs():
    """Physical placement must not change any result: another free-list permutation
    gives bit-identical outputs (the kernels' reduction order is logical)."""
    lay = _small(0)
    w1 = _wl(lay)
    o1 = w1.prefill()[0].clone()
    d1 = w1.decode()[0].clone()
    perm = np.random.default_rng(99).permutation(w1.n_phys + 5).astype(np.int32)
    w3 = _wl_free(lay, perm)
    assert not np.array_equal(w1.free, w3.free[: len(w1.free)])
    o3 = w3.prefill()[0]
    d3 = w3.decode()[0]
    torch.cuda.synchronize()
    assert torch.equal(o1, o3) and torch.equal(d1, d3)


def _wl_free(lay, free):
    from head_aware_paged_page_amd.workload import Workload
    return Workload(lay, device="cuda", free=free)


def test_class_reductions_on_gpu():
    """local with a window past every position, retrieval listing every segment page
    and dense all give the global result, bit for bit."""
    lens = [[300, 170]]
    nsp = -(-300 // 16) + -(-170 // 16)
    classes = [(GLOBAL, 0), (LOCAL, 10 ** 6), (RETRIEVAL, 0), (DENSE, 0)]
    lay = custom_layout(seg_lens=lens, offline=[[0, 0]], n_prefill=50, n_decode=1, classes=classes, page_size=16,
                        head_dim=128, group=4, dtype="bf16", ret_lists={(2, 0): list(range(nsp))}, name="red")
    # same values for every slot: overwrite the pools from slot 0's chain
    w = _wl(lay)
    for slot in range(1, 4):
        src, dst = w.chain_phys(0, 0), w.chain_phys(slot, 0)
        w.k_pool[dst] = w.k_pool[src]
        w.v_pool[dst] = w.v_pool[src]
    q = w.q_prefill.clone()
    for slot in range(1, 4):
        q[:, slot * 4:(slot + 1) * 4] = q[:, 0:4]
    out, _ = w.prefill(q=q)
    qd = w.q_decode.clone()
    for slot in range(1, 4):
        qd[:, slot * 4:(slot + 1) * 4] = qd[:, 0:4]
    outd, _ = w.decode(q=qd)
    torch.cuda.synchronize()
    for slot in range(1, 4):
        assert torch.equal(out[:, slot * 4:(slot + 1) * 4], out[:, 0:4])
        assert torch.equal(outd[:, slot * 4:(slot + 1) * 4], outd[:, 0:4])


# ---------------------------------------------------------------- full-size configs (sampled rows / queries)

@pytest.mark.parametrize("name", ["32k", "16k", "128k", "batch", "recovery32k"])
def test_full_config(name):
    w = cached(name)
    lay = w.lay
    rows = _rows_by_class(lay, 2)
    q_sample = None
    if lay.n_prefill > 256:
        rng = np.random.default_rng(1)
        q_sample = np.unique(np.concatenate([[0, 1, lay.n_prefill - 1], rng.integers(0, lay.n_prefill, 12)]))
    w.relocate()
    check_relocate(w, rows=rows[:3])
    w.prefill()
    check_prefill(w, rows=rows, q_sample=q_sample)
    w.decode()
    check_decode(w, rows=rows)


def test_end_to_end_32k():
    """GPU chain relocate -> prefill -> decode vs oracle relocation (fp64) -> attention."""
    w = cached("32k")
    lay = w.lay
    rows = _rows_by_class(lay, 2, seed=3)

    def reloc_keys(slot, seq, K):
        ctx = lay.ctx_len(seq)
        on, off = _seg_positions(lay, seq)
        K = K.copy()
        K[:ctx] = orope.relocate(K[:ctx], off, on, lay.theta)
        return K
    w.relocate()
    w.prefill(k=w.k_reloc)
    check_prefill(w, rows=rows, keys_fn=reloc_keys)
    w.decode(k=w.k_reloc)
    check_decode(w, rows=rows, keys_fn=reloc_keys)



def test_many_rows_with_splits():
    """More rows than fit a plan in the kernel arguments (200 > 128 for prefill,
    > 192 for decode), so the plan
    kernel writes both plans to the workspace, with rows long enough that prefill
    and decode both split them: the merge kernels then read the workspace plan."""
    classes = [(GLOBAL, 0) if s % 2 == 0 else (LOCAL, 64) for s in range(50)]
    lay = custom_layout(seg_lens=[[6000]] * 4, offline=[[0]] * 4, n_prefill=16, n_decode=1, classes=classes,
                        page_size=16, head_dim=64, group=2, dtype="bf16", name="many_rows", seed=3)
    assert lay.n_slot * lay.n_seq == 200
    w = _wl(lay)
    rows = [slot * lay.n_seq + seq for slot in (0, 1, 24, 48, 49) for seq in range(lay.n_seq)]
    w.prefill()
    check_prefill(w, rows=rows)
    w.decode()
    check_decode(w, rows=rows)


def _raw(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


@pytest.mark.parametrize("name", ["small0", "32k"])
def test_pack_unpack_pages_bit_exact(name):
    """Per-head visible-page pack (the pages the decode tables list, in table
    order) and unpack, against the oracle, bit for bit on the raw page bytes
    (NaN-filled empty slots included).  On the small layout two entries are
    pointed outside the pool: they pack as zeros and unpack to nothing."""
    from oracle import pack as opack
    import head_aware_paged_page_amd.segpaged as sp
    w = _wl(_small(0)) if name == "small0" else cached("32k")
    ent = torch.as_tensor(np.asarray(w.td["entries"]).reshape(-1, 4), dtype=torch.int32).clone()
    if name == "small0":
        ent[1, 0] = w.n_phys + 5
        ent[-1, 0] = -1
    n = ent.shape[0]
    d_ent = ent.cuda()
    k_out = torch.empty((n,) + tuple(w.k_pool.shape[1:]), dtype=w.k_pool.dtype, device="cuda")
    v_out = torch.empty((n,) + tuple(w.v_pool.shape[1:]), dtype=w.v_pool.dtype, device="cuda")
    sp.pack_pages(w.k_pool, w.v_pool, d_ent, n, k_out, v_out)
    k_zero, v_zero = torch.zeros_like(w.k_pool), torch.zeros_like(w.v_pool)
    sp.unpack_pages(k_out, v_out, d_ent, n, k_zero, v_zero)
    torch.cuda.synchronize()
    phys = ent[:, 0].numpy()
    kp, vp = opack.pack(_raw(w.k_pool), _raw(w.v_pool), phys)
    assert np.array_equal(_raw(k_out), kp) and np.array_equal(_raw(v_out), vp)
    ku, vu = opack.unpack(kp, vp, phys, np.zeros_like(kp, shape=w.k_pool.shape), np.zeros_like(vp, shape=w.v_pool.shape))
    assert np.array_equal(_raw(k_zero), ku) and np.array_equal(_raw(v_zero), vu)

@pytest.mark.parametrize("fill", ["ones", "random"])
def test_workspace_contents_do_not_matter(fill):
    """The prefill's work-ticket counter lives in the caller's workspace, which no
    call clears first (with the plan in the kernel arguments no plan kernel runs):
    each call counts under its own epoch.  At 128K the persistent workgroups take
    about 2400 of the 2624 items by ticket, so a counter that handed out a wrong or
    repeated item would change the outputs: they must be bit-identical whatever
    the workspace held before the call."""
    w = cached("128k")
    o_ref = w.prefill()[0].clone()
    d_ref = w.decode()[0].clone()
    if fill == "ones":
        w.workspace.fill_(0xFF)
    else:
        g = torch.Generator(device="cuda").manual_seed(7)
        w.workspace.copy_(torch.randint(0, 256, w.workspace.shape, dtype=torch.uint8, device="cuda", generator=g))
    o = w.prefill()[0]
    d = w.decode()[0]
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(d, d_ref)
