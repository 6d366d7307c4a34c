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
    """The log-sum-exp is formed from the scores in fp32 with no rounding of the
    inputs beyond their own precision (the queries enter the matrix cores as
    given): held to 1e-4 for bf16 inputs and 1e-5 for fp32 (about 1e-6 is
    measured in both; the fp32 m + log l keeps about seven digits)."""
    return {"bf16": 1e-4, "f32": 1e-5}[dtype]


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


def check_prefill(w, rows=None, q_sample=None, k_pool=None, keys_fn=None, lse_bound=None):
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
        assert np.max(np.abs(lse[t0 + toks, heads] - L)) <= (lse_bound or lse_tol(lay.dtype, L))
    return worst


def check_decode(w, rows=None, keys_fn=None, lse_bound=None):
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
        assert np.max(np.abs(lse[seq:seq + 1, heads] - L)) <= (lse_bound or lse_tol(lay.dtype, L))


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



def test_relocate_in_place_matches_out_of_place():
    """rope_relocate with the output buffer the input buffer (the bench's form:
    each pool replica rotated in place, by +delta and -delta in turn) writes
    exactly the bits the out-of-place call writes, on every page of the pool
    (a thread rewrites only the elements it read); and back by -delta in place
    returns the original keys within the relocation bound."""
    for name in ("tiny", "32k"):
        w = cached(name) if name != "tiny" else _wl(synth.make_layout(name))
        w.relocate()                                         # k_pool -> k_reloc
        tmp = w.k_pool.clone()
        w.relocate(k_in=tmp, k_out=tmp)                      # in place
        torch.cuda.synchronize()
        ib = torch.int32 if tmp.dtype == torch.float32 else torch.int16
        assert torch.equal(tmp.view(ib), w.k_reloc.view(ib)), f"{name}: in-place bits differ"
        w.relocate(k_in=tmp, k_out=tmp, back=True)           # and back
        torch.cuda.synchronize()
        lay = w.lay
        for r in _rows_by_class(lay, 1) if name != "tiny" else range(lay.n_slot):
            slot, seq = divmod(r, lay.n_seq)
            assert np.max(np.abs(w.gather_keys(tmp, slot, seq) - w.gather_keys(w.k_pool, slot, seq))) <= TOL[lay.dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_relocate_large_deltas(dtype):
    """Position deltas near the int32 limit (2^30 - 5, -999 900, -2^30 + 350):
    the angle is formed and reduced in fp64, so relocated keys still match the
    fp64 oracle at the dtype's bound; prefill and decode over them too."""
    lay = custom_layout(seg_lens=[[100, 50, 30]], offline=[[-(2 ** 30) + 5, 10 ** 6, 2 ** 30 - 200]], n_prefill=5,
                        n_decode=1, classes=[(GLOBAL, 0), (LOCAL, 40)], page_size=16,
                        head_dim=64 if dtype == "f32" else 128, group=2, dtype=dtype, name=f"bigdelta_{dtype}",
                        seed=11)
    w = _wl(lay)
    w.relocate()
    check_relocate(w)
    w.prefill()
    check_prefill(w)
    w.decode()
    check_decode(w)

# ---------------------------------------------------------------- small bf16 layouts: several tiles, ragged tails

SMALL = [
    # (group, head_dim, page_size, seg_lens, n_prefill, classes)
    (4, 128, 16, [[300, 77, 513]], 70, [(GLOBAL, 0), (LOCAL, 100), (RETRIEVAL, 0), (DENSE, 0), (LOCAL, 1)]),
    (8, 128, 32, [[1000, 33], [64]], 45, [(LOCAL, 257), (GLOBAL, 0), (RETRIEVAL, 0)]),
    (1, 64, 16, [[200, 31]], 150, [(GLOBAL, 0), (LOCAL, 40), (LOCAL, 1)]),
    (2, 64, 64, [[129, 700]], 33, [(GLOBAL, 0), (LOCAL, 65)]),
    (16, 128, 16, [[17]], 9, [(GLOBAL, 0), (LOCAL, 5)]),
    (3, 128, 16, [[450], [90, 91]], 40, [(LOCAL, 64), (GLOBAL, 0)]),
    (4, 128, 64, [[700, 65], [130]], 50, [(GLOBAL, 0), (LOCAL, 100)]),
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
    if lay.page_size == 64:                 # decode takes pages of 16 and 32 keys
        w = _wl(lay)
        w.relocate()
        check_relocate(w)
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


def test_fp32_pages_longer_than_a_wave():
    """fp32 attention over pages of 128 keys (the kernel scores a page 64 keys
    at a time), of 64 keys, and of sizes that do not divide 64 (24: two pages
    per step and 16 idle lanes; 48: one page per step; 5: twelve pages per
    step), against the oracle."""
    for ps, lens, npf in ((128, [[300, 70]], 20), (64, [[129, 700]], 33), (24, [[250, 61]], 30),
                          (48, [[97, 200]], 25), (5, [[83, 17]], 12)):
        lay = custom_layout(seg_lens=lens, offline=[[17, -900]], n_prefill=npf, n_decode=1,
                            classes=[(GLOBAL, 0), (LOCAL, 90)], page_size=ps, head_dim=64, group=2, dtype="f32",
                            ret_lists={}, name=f"f32_ps{ps}", seed=3)
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


# ---------------------------------------------------------------- full-size configs

@pytest.mark.parametrize("name", ["32k", "16k"])
def test_full_config_every_row(name):
    """Every (slot, seq) row of the 32K and 16K workloads, in the launch
    configuration bench.py times: relocation of every segment key, prefill of
    every query token and the decode token, against the oracle.  Segment 0 of
    both workloads keeps its position (offline base = online base = 0), so its
    relocated keys must equal the cached ones bit for bit in bf16."""
    w = cached(name)
    lay = w.lay
    w.relocate()
    check_relocate(w)
    torch.cuda.synchronize()
    n0 = int(lay.seg_len[0][0])
    assert lay.seg_online[0][0] == lay.seg_offline[0][0]
    for slot in range(lay.n_slot):
        a = w.gather_keys(w.k_reloc, slot, 0)[:n0]
        b = w.gather_keys(w.k_pool, slot, 0)[:n0]
        assert np.array_equal(a, b), f"slot {slot}: a zero shift changed bf16 keys"
    w.prefill()
    check_prefill(w)
    w.decode()
    check_decode(w)


@pytest.mark.parametrize("name", ["128k", "batch"])
def test_full_config_sampled(name):
    """The 128K and batch workloads at full size: two rows per class (and, at
    128K, sampled query tokens of the 2048-token chunk) against the oracle."""
    w = cached(name)
    lay = w.lay
    rows = _rows_by_class(lay, 2)
    q_sample = None
    if lay.n_prefill > 256:
        rng = np.random.default_rng(1)
        q_sample = np.unique(np.concatenate([[0, 1, lay.n_prefill - 1], rng.integers(0, lay.n_prefill, 12)]))
    w.relocate()
    check_relocate(w, rows=rows)
    w.prefill()
    check_prefill(w, rows=rows, q_sample=q_sample)
    w.decode()
    check_decode(w, rows=rows)


@pytest.mark.parametrize("part", [0, 1])
def test_recovery32k_every_query_tile(part):
    """Head-level recovery prefill (30000-token causal chunk over the 10 global
    slots): for every row, the last token of every 64-token query tile (where
    the diagonal bound cuts the tile's last key tile) plus one random token in
    every fourth tile, against the oracle.  The rows are split over two tests."""
    w = cached("recovery32k")
    lay = w.lay
    if part == 0:
        w.prefill()
        w.decode()
    tpt = 256 // lay.group
    last = np.arange(tpt - 1, lay.n_prefill, tpt)
    if last[-1] != lay.n_prefill - 1:
        last = np.append(last, lay.n_prefill - 1)
    rng = np.random.default_rng(7 + part)
    starts = np.arange(0, lay.n_prefill, 4 * tpt)
    extra = np.minimum(starts + rng.integers(0, tpt, len(starts)), lay.n_prefill - 1)
    q_sample = np.unique(np.concatenate([[0], last, extra]))
    rows = range(part * 5, part * 5 + 5)
    check_prefill(w, rows=rows, q_sample=q_sample)
    check_decode(w, rows=rows)


def _table_counts(w, which, q_pos_of_seq):
    """Visible keys of each (query, row) counted from the host tables alone."""
    import bench
    tab = w.tp if which == "prefill" else w.td
    return bench.table_visible_counts(tab["row_ptr"], tab["entries"], w.lay.cls, w.lay.window, w.lay.n_seq,
                                      q_pos_of_seq)


@pytest.mark.parametrize("name", ["32k", "16k", "128k", "batch"])
def test_full_size_visible_counts(name):
    """Q = 0 at full size: exp(LSE) of every (query, head) is the head's visible
    token count, exactly.  It must equal the oracle's visible set size and the
    count the benchmark derives from the host tables (its FLOP and byte
    numerators).  Every row and query at 32K and 16K; at 128K and batch every
    row, on sampled queries."""
    w = cached(name)
    lay = w.lay
    zq = torch.zeros_like(w.q_prefill)
    zd = torch.zeros_like(w.q_decode)
    _, lse_p = w.prefill(q=zq, out=torch.empty_like(zq), lse=torch.empty_like(w.lse_prefill))
    _, lse_d = w.decode(q=zd, out=torch.empty_like(zd), lse=torch.empty_like(w.lse_decode))
    torch.cuda.synchronize()
    cp = np.rint(np.exp(lse_p.double().cpu().numpy())).astype(np.int64)
    cd = np.rint(np.exp(lse_d.double().cpu().numpy())).astype(np.int64)
    toks = np.arange(lay.n_prefill)
    if name in ("128k", "batch"):
        rng = np.random.default_rng(5)
        toks = np.unique(np.concatenate([[0, lay.n_prefill - 1], rng.integers(0, lay.n_prefill, 6)]))
    q_pos = [lay.new_base[s] + toks for s in range(lay.n_seq)]
    d_pos = [np.asarray([lay.new_base[s] + lay.n_prefill]) for s in range(lay.n_seq)]
    tab_p = _table_counts(w, "prefill", q_pos)
    tab_d = _table_counts(w, "decode", d_pos)
    G = lay.group
    for slot in range(lay.n_slot):
        for seq in range(lay.n_seq):
            r = slot * lay.n_seq + seq
            t0 = int(w.h_tok_ptr[seq])
            want = otab.visible_counts(lay, slot, seq, q_pos[seq])
            got = cp[t0 + toks, slot * G:(slot + 1) * G]
            assert np.array_equal(got, np.repeat(want[:, None], G, axis=1)), f"prefill row {r}"
            assert np.array_equal(tab_p[r], want), f"host-table count, prefill row {r}"
            wd = otab.visible_counts(lay, slot, seq, d_pos[seq])
            assert np.all(cd[seq, slot * G:(slot + 1) * G] == wd[0]), f"decode row {r}"
            assert np.array_equal(tab_d[r], wd), f"host-table count, decode row {r}"


def _row_call(w, slots, which):
    """One prefill or decode call over the given slots of a workload (a slot may
    repeat), straight through the C ABI, reusing the workload's pools and tables.
    Returns (out, lse) laid out [tokens, len(slots) * G, D] / [tokens, len(slots) * G]."""
    import head_aware_paged_page_amd.segpaged as sp
    lay, G = w.lay, w.lay.group
    assert lay.n_seq == 1
    tab = w.tp if which == "prefill" else w.td
    rp, ent = tab["row_ptr"], tab["entries"]
    ents = [ent[rp[s]:rp[s + 1]] for s in slots]
    row_ptr = np.concatenate([[0], np.cumsum([len(e) for e in ents])]).astype(np.int32)
    entries = np.ascontiguousarray(np.concatenate(ents), dtype=np.int32)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    heads = torch.as_tensor(np.concatenate([np.arange(s * G, (s + 1) * G) for s in slots]), device="cuda")
    q_src = w.q_prefill if which == "prefill" else w.q_decode
    q = q_src.index_select(1, heads).contiguous()
    out, lse = torch.empty_like(q), torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    cls, win = dev(lay.cls[slots].astype(np.int32)), dev(lay.window[slots].astype(np.int32))
    kind = sp.SP_WS_PREFILL if which == "prefill" else sp.SP_WS_DECODE
    code = sp.SP_BF16 if lay.dtype == "bf16" else sp.SP_F32
    nb = sp.workspace_bytes(kind, code, w.D, w.ps, G, 1, len(slots), w.h_tok_ptr if which == "prefill" else None,
                            row_ptr)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    common = dict(page_size=w.ps, group=G, n_seq=1, n_slot=len(slots), h_row_ptr=row_ptr, d_cls=cls, d_window=win,
                  d_row_ptr=dev(row_ptr), d_entries=dev(entries), scale=w.scale, out=out, lse=lse, workspace=ws)
    if which == "prefill":
        sp.prefill(q, w.k_pool, w.v_pool, h_tok_ptr=w.h_tok_ptr, d_tok_ptr=w.d_tok_ptr, d_q_pos0=w.d_q_pos0,
                   **common)
    else:
        sp.decode(q, w.k_pool, w.v_pool, d_q_pos=w.d_q_dec, **common)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("which", ["prefill", "decode"])
def test_split_count_does_not_change_results(which):
    """The same 32K global row computed with different kv-split counts: alone in a
    call (many splits), inside the 64-row call (the bench's split), and repeated
    256 times in one call (no prefill split: the items then outnumber the CUs).

    The log-sum-exp (fp32 partials, merged in fp32) must agree to 2e-5.  The
    outputs may differ by the roundings that depend on the split: the softmax
    weights enter the P.V product in bf16 relative to each split's own running
    max (at most 2^-9 relative per weight, so 2^-9 * sum_j p_j |v_j| per side),
    the prefill's split partials are stored normalised in fp16 (2^-11 of the
    same sum per side), and the bf16 output rounding (one unit in the last
    place).  sum_j p_j |v_j| is taken from the oracle (attention over |v|)."""
    w = cached("32k")
    lay, G = w.lay, w.lay.group
    slot = int(np.nonzero(lay.cls == GLOBAL)[0][0])
    o_all, l_all = (w.prefill() if which == "prefill" else w.decode())
    torch.cuda.synchronize()
    ref_o = o_all[:, slot * G:(slot + 1) * G].clone()
    ref_l = l_all[:, slot * G:(slot + 1) * G].clone()
    o1, l1 = _row_call(w, [slot], which)
    on, ln = _row_call(w, [slot] * 256, which)
    K, V = w.unit_host(slot, 0)
    q_src = w.q_prefill if which == "prefill" else w.q_decode
    q_pos = lay.new_base[0] + (np.arange(lay.n_prefill) if which == "prefill" else np.asarray([lay.n_prefill]))
    wabs, _, _ = oatt.row_attention(lay, slot, 0, K, np.abs(V), _host(q_src[:, slot * G:(slot + 1) * G]), q_pos)
    per_side = 2.0 ** -9 + (2.0 ** -11 if which == "prefill" else 0.0)
    slack = torch.as_tensor(2 * per_side * wabs, dtype=torch.float32, device="cuda")
    worst_l = worst_o = worst_frac = 0.0
    for k in range(257):
        o, l = (o1, l1) if k == 0 else (on[:, (k - 1) * G:k * G], ln[:, (k - 1) * G:k * G])
        d = float((l - ref_l).abs().max())
        worst_l = max(worst_l, d)
        assert d <= 2e-5, f"call {k}: LSE differs by {d}"
        a, b = o.float(), ref_o.float()
        diff = (a - b).abs()
        bound = torch.maximum(a.abs(), b.abs()) * 2.0 ** -7 + slack
        worst_o = max(worst_o, float(diff.max()))
        worst_frac = max(worst_frac, float((diff / bound).max()))
        assert bool(torch.all(diff <= bound)), f"call {k}: outputs differ by {float(diff.max())}"
    print(f"[split] {which}: max LSE difference {worst_l:.2e}, max output difference {worst_o:.2e} "
          f"({worst_frac:.2f} of its bound)")


@pytest.mark.parametrize("which", ["prefill", "decode"])
def test_per_layer_calls_match_the_whole_call(which):
    """The 32K step's prefill and decode issued as one call per layer (its 8 KV
    heads), as the bench's per-layer block times them, against the one 64-slot
    call: each layer's rows get their own plan (finer kv splits when a layer holds
    few global rows), so the log-sum-exp must agree to 2e-5 and the outputs to the
    roundings that depend on the split (as in the split-count test), bounded here
    by the largest |v| of the pool's written pages instead of the per-row sum of
    p |v|."""
    from synth.configs import CONFIGS
    w = cached("32k")
    lay, G = w.lay, w.lay.group
    spl = CONFIGS["32k"]["n_kv"]                 # a layer's KV heads
    n_layers = lay.n_slot // spl
    o_all, l_all = (w.prefill() if which == "prefill" else w.decode())
    torch.cuda.synchronize()
    o_all, l_all = o_all.clone(), l_all.clone()
    vmax = float(torch.nan_to_num(w.v_pool.float().abs(), nan=0.0, posinf=0.0).amax())   # unused pages hold NaN
    per_side = 2.0 ** -9 + (2.0 ** -11 if which == "prefill" else 0.0)
    worst_l = worst_o = 0.0
    for layer in range(n_layers):
        slots = list(range(layer * spl, (layer + 1) * spl))
        o, l = _row_call(w, slots, which)
        heads = slice(layer * spl * G, (layer + 1) * spl * G)
        d = float((l - l_all[:, heads]).abs().max())
        worst_l = max(worst_l, d)
        assert d <= 2e-5, f"layer {layer}: LSE differs by {d}"
        a, b = o.float(), o_all[:, heads].float()
        diff = (a - b).abs()
        bound = torch.maximum(a.abs(), b.abs()) * 2.0 ** -7 + 2 * per_side * vmax
        worst_o = max(worst_o, float(diff.max()))
        assert bool(torch.all(diff <= bound)), f"layer {layer}: outputs differ by {float(diff.max())}"
    print(f"[per-layer] {which}: max LSE difference {worst_l:.2e}, max output difference {worst_o:.2e}")


def test_out_of_pool_pages_are_empty():
    """A table entry whose physical page lies outside the pool (>= n_phys, or
    negative) is read as a page with no tokens: prefill and decode then equal
    the oracle over the visible set less that page's tokens."""
    import head_aware_paged_page_amd.segpaged as sp
    lay = _small(0)
    w = _wl(lay)
    slot, G = 0, lay.group                       # a global row of 57 pages
    assert lay.cls[slot] == GLOBAL
    rp_p, rp_d = w.tp["row_ptr"], w.td["row_ptr"]
    drop_p = {int(rp_p[slot]) + 5: w.n_phys + 5, int(rp_p[slot]) + 30: -1}
    drop_d = {int(rp_d[slot]) + 11: w.n_phys, int(rp_d[slot]) + 40: -7}
    ent_p, ent_d = w.tp["entries"].copy(), w.td["entries"].copy()
    gone_p = [tuple(ent_p[i, 1:3]) for i in drop_p]
    gone_d = [tuple(ent_d[i, 1:3]) for i in drop_d]
    for i, v in drop_p.items():
        ent_p[i, 0] = v
    for i, v in drop_d.items():
        ent_d[i, 0] = v
    w.p_entries = torch.from_numpy(ent_p).cuda()
    w.d_entries = torch.from_numpy(ent_d).cuda()
    out, lse = w.prefill()
    outd, lsed = w.decode()
    torch.cuda.synchronize()
    K, V = w.unit_host(slot, 0)
    tpos, _tp, tsp, tnew = otab.tokens(lay, 0)

    def expect(q, p, gone):
        m = otab.visible(GLOBAL, 0, [], tpos, tsp, tnew, int(p))
        for s0, n in gone:
            m &= ~((tpos >= s0) & (tpos < s0 + n))
        return oatt.attend(q, K[m], V[m], w.scale)

    for t in range(lay.n_prefill):
        o, l = expect(_host(w.q_prefill[t, :G]), lay.new_base[0] + t, gone_p)
        assert np.max(np.abs(_host(out[t, :G]) - o)) <= TOL["bf16"]
        assert np.max(np.abs(lse[t, :G].double().cpu().numpy() - l)) <= TOL["bf16"]
    o, l = expect(_host(w.q_decode[0, :G]), lay.new_base[0] + lay.n_prefill, gone_d)
    assert np.max(np.abs(_host(outd[0, :G]) - o)) <= TOL["bf16"]
    assert np.max(np.abs(lsed[0, :G].double().cpu().numpy() - l)) <= TOL["bf16"]


@pytest.mark.parametrize("k_scale", [4.0, 8.0])
def test_large_key_magnitudes(k_scale):
    """Keys of standard deviation 4 and 8 against unit queries (logits of that
    spread): outputs within the bf16 bound and the log-sum-exp within 1e-4,
    which a query rounded after scaling (c * q to bf16) would not meet."""
    lay = custom_layout(seg_lens=[[3000, 1000]], offline=[[0, -500]], n_prefill=64, n_decode=1,
                        classes=[(GLOBAL, 0), (LOCAL, 256)], page_size=16, head_dim=128, group=4, dtype="bf16",
                        k_scale=k_scale, name=f"kscale{k_scale:g}", seed=5)
    w = _wl(lay)
    w.prefill()
    worst = check_prefill(w)
    w.decode()
    check_decode(w)
    print(f"[kscale] {k_scale}: prefill worst output error {worst:.2e}")


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
    # The relocated keys the GPU hands to attention are rounded to bf16, the
    # oracle's are not: the log-sum-exp inherits that input rounding, so it is
    # held to the output bound here.
    w.relocate()
    w.prefill(k=w.k_reloc)
    check_prefill(w, rows=rows, keys_fn=reloc_keys, lse_bound=TOL["bf16"])
    w.decode(k=w.k_reloc)
    check_decode(w, rows=rows, keys_fn=reloc_keys, lse_bound=TOL["bf16"])



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


def test_deep_merges_with_workspace_plans():
    """200 slots (more than either plan in the kernel arguments holds, so the
    plan kernel writes both plans to the workspace): one global row of 40 000
    keys and 199 short local rows.  The prefill planner cuts the long row at
    least 32 ways (checked through the workspace size the ABI reports: its
    partials), so the merge takes its row-per-workgroup path reading the
    workspace plan; the decode splits it too, merged by four waves per head."""
    import head_aware_paged_page_amd.segpaged as sp
    classes = [(GLOBAL, 0)] + [(LOCAL, 64)] * 199
    lay = custom_layout(seg_lens=[[40000]], offline=[[0]], n_prefill=64, n_decode=1, classes=classes,
                        page_size=16, head_dim=64, group=2, dtype="bf16", name="deep_merges", seed=5)
    assert lay.n_slot * lay.n_seq == 200
    w = _wl(lay)
    # prefill workspace: a few KB of plan arrays, then per split item a fp16
    # partial of 256 rows x 64 dims and 256 fp32 log-sum-exps (a lower bound
    # on the item count: 57 here)
    nb = sp.workspace_bytes(sp.SP_WS_PREFILL, sp.SP_BF16, 64, 16, 2, 1, 200, w.h_tok_ptr, w.tp["row_ptr"])
    parts = (nb - 4 * 4 * 201 - 512) // (256 * 64 * 2 + 256 * 4)
    assert parts >= 32, f"the long row is split {parts} ways"
    rows = [0, 1, 100, 199]
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


# ---------------------------------------------------------------- edge cases

def test_longest_rows_with_zero_queries():
    """The largest row one decode call takes: 1024 splits of 512 pages, 524 288
    pages of 16 keys (8.4 M keys), through prefill (64 tokens, every one) and
    decode.  With every query zero, attention is uniform, so each head's output
    is the mean of the visible values and the log-sum-exp is ln(count): one
    split missing or doubled would move it by 1e-3 at the decode.  The values
    are set to a pattern exact in bf16, v[pos, d] = ((pos + 3 d) mod 16) / 16,
    whose mean over the visible positions is counted exactly on the host."""
    ps, D, n_new = 16, 128, 65
    n_pages = 1024 * 512
    seg = (n_pages - (n_new + ps - 1) // ps) * ps     # the new tokens fill the last five pages
    lay = custom_layout(seg_lens=[[seg]], offline=[[0]], n_prefill=n_new - 1, n_decode=1, classes=[(GLOBAL, 0)],
                        page_size=ps, head_dim=D, group=4, dtype="bf16", name="longest_rows", seed=7)
    w = _wl(lay, relocated_pool=False)
    assert int(w.td["row_ptr"][-1]) == n_pages
    ent = torch.from_numpy(np.ascontiguousarray(w.td["entries"]).reshape(-1, 4)).to("cuda")
    phys, pos0 = ent[:, 0].long(), ent[:, 1].int()
    slots = torch.arange(ps, device="cuda", dtype=torch.int32)
    d3 = 3 * torch.arange(D, device="cuda", dtype=torch.int32)
    for c0 in range(0, n_pages, 1 << 16):                                 # [pages, D, ps], 65 536 pages at a time
        pos = pos0[c0:c0 + (1 << 16), None] + slots[None, :]
        vals = ((pos[:, None, :] + d3[None, :, None]) % 16).float().div_(16).to(torch.bfloat16)
        w.v_pool[phys[c0:c0 + (1 << 16)]] = vals
    del vals, pos
    w.q_prefill.zero_()
    w.q_decode.zero_()
    out_p, lse_p = w.prefill()
    out_d, lse_d = w.decode()
    torch.cuda.synchronize()

    def mean_pattern(count):
        per_res = np.full(16, count // 16, np.int64)
        per_res[: count % 16] += 1           # visible positions 0 .. count-1 by residue mod 16
        return np.array([np.sum(per_res * ((np.arange(16) + 3 * dd) % 16) / 16.0) / count for dd in range(D)])

    counts = [seg + t + 1 for t in range(n_new)]        # token t sees positions 0 .. seg + t
    got = torch.cat([out_p, out_d]).double().cpu().numpy()                # [tokens, heads, D]
    lse = torch.cat([lse_p, lse_d]).double().cpu().numpy()               # [tokens, heads]
    err = max(float(np.max(np.abs(got[t] - mean_pattern(c)[None, :]))) for t, c in enumerate(counts))
    lerr = max(float(np.max(np.abs(lse[t] - np.log(c)))) for t, c in enumerate(counts))
    print(f"[longest rows] {counts[-1]} keys: max abs error {err:.2e}, log-sum-exp {lerr:.2e}")
    assert err <= 1e-2
    assert lerr <= 1e-5


def test_calls_on_two_streams_at_once():
    """Two workloads (own pools, tables and workspaces) run relocate -> prefill
    -> decode on two streams at once, several times over: every output equals
    the same calls made one stream at a time, bit for bit."""
    lays = [synth.make_layout("16k"), _small(1)]
    ws = [_wl(l) for l in lays]
    want = []
    for w in ws:
        w.relocate()
        w.prefill(k=w.k_reloc)
        w.decode(k=w.k_reloc)
        torch.cuda.synchronize()
        want.append([t.clone() for t in (w.k_reloc, w.out_prefill, w.lse_prefill, w.out_decode, w.lse_decode)])
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for _ in range(5):
        for w in ws:
            for t in (w.out_prefill, w.lse_prefill, w.out_decode, w.lse_decode):
                t.zero_()
        torch.cuda.synchronize()
        for w, st in zip(ws, streams):
            with torch.cuda.stream(st):
                w.relocate(stream=st)
                w.prefill(k=w.k_reloc, stream=st)
                w.decode(k=w.k_reloc, stream=st)
        torch.cuda.synchronize()
        for w, ref in zip(ws, want):
            got = (w.k_reloc, w.out_prefill, w.lse_prefill, w.out_decode, w.lse_decode)
            for a, b in zip(got, ref):
                assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                                   b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


def test_empty_calls_write_nothing():
    """A relocation list of length 0 and a prefill call with no query tokens are
    valid no-ops: SP_OK, and the outputs keep what they held."""
    import head_aware_paged_page_amd.segpaged as sp
    lay = _small(2)
    w = _wl(lay)
    before = w.k_reloc.clone()
    sp.rope_relocate(w.k_pool, w.k_reloc, w.ps, w.d_reloc[:0], lay.theta)
    zero_tok = np.zeros(lay.n_seq + 1, np.int32)
    out = torch.full_like(w.q_prefill[:1], 7.0)
    lse = torch.full((1, w.Hq), 7.0, dtype=torch.float32, device="cuda")
    sp.prefill(w.q_prefill[:1], w.k_pool, w.v_pool, page_size=w.ps, group=w.G, n_seq=lay.n_seq, n_slot=lay.n_slot,
               h_tok_ptr=zero_tok, h_row_ptr=w.tp["row_ptr"], d_tok_ptr=torch.from_numpy(zero_tok).cuda(),
               d_q_pos0=w.d_q_pos0, d_cls=w.d_cls, d_window=w.d_window, d_row_ptr=w.p_row_ptr,
               d_entries=w.p_entries, scale=w.scale, out=out, lse=lse, workspace=w.workspace)
    torch.cuda.synchronize()
    # unwritten pool pages hold NaN: compare bit patterns
    assert torch.equal(w.k_reloc.view(torch.int16), before.view(torch.int16))
    assert bool((out.float() == 7.0).all()) and bool((lse == 7.0).all())


def test_sequence_without_query_tokens():
    """Two sequences, query tokens for the second only (tok_ptr = [0, 0, n]):
    the first sequence's rows have no work items, the second matches the oracle."""
    import head_aware_paged_page_amd.segpaged as sp
    lay = _small(1)                                   # two sequences, G = 8
    w = _wl(lay)
    n = lay.n_prefill
    tok = np.asarray([0, 0, n], np.int32)
    q = w.q_prefill[n:2 * n].contiguous()
    out, lse = torch.empty_like(q), torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    nb = sp.workspace_bytes(sp.SP_WS_PREFILL, sp.SP_BF16, w.D, w.ps, w.G, lay.n_seq, lay.n_slot, tok,
                            w.tp["row_ptr"])
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    sp.prefill(q, w.k_pool, w.v_pool, page_size=w.ps, group=w.G, n_seq=lay.n_seq, n_slot=lay.n_slot, h_tok_ptr=tok,
               h_row_ptr=w.tp["row_ptr"], d_tok_ptr=torch.from_numpy(tok).cuda(), d_q_pos0=w.d_q_pos0,
               d_cls=w.d_cls, d_window=w.d_window, d_row_ptr=w.p_row_ptr, d_entries=w.p_entries, scale=w.scale,
               out=out, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    for slot in range(lay.n_slot):
        K, V = w.unit_host(slot, 1)
        heads = slice(slot * lay.group, (slot + 1) * lay.group)
        O, L, _ = oatt.row_attention(lay, slot, 1, K, V, _host(q[:, heads]), lay.new_base[1] + np.arange(n))
        assert np.max(np.abs(_host(out[:, heads]) - O)) <= TOL["bf16"]
        assert np.max(np.abs(lse[:, heads].double().cpu().numpy() - L)) <= TOL["bf16"]


def test_retrieval_head_with_no_listed_page():
    """A retrieval head whose list is empty sees only the new tokens (causally):
    its table holds only new-token pages, and prefill and decode match the oracle."""
    lay = custom_layout(seg_lens=[[300, 90]], offline=[[0, 11]], n_prefill=40, n_decode=1,
                        classes=[(RETRIEVAL, 0), (GLOBAL, 0)], page_size=16, head_dim=128, group=4, dtype="bf16",
                        ret_lists={(0, 0): []}, name="ret_empty")
    w = _wl(lay)
    ent = w.tp["entries"][w.tp["row_ptr"][0]:w.tp["row_ptr"][1]]
    assert np.all(ent[:, 1] >= lay.new_base[0])       # new-token pages only
    w.prefill()
    check_prefill(w)
    w.decode()
    check_decode(w)
