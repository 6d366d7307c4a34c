"""Attention importance and token selection on the GPU against the oracle.

segpaged_token_importance: each slot's importance of every position (the
softmax probability mass the chunk's rows give it, with the prefill's lse)
against oracle.importance.row_importance in fp64.  Bound: the device computes
each probability from bf16 inputs (the queries as given) against the
prefill's log-sum-exp, so each probability (and a sum of them) is held to 2e-2
relative, the bf16 bound, plus 1e-6 absolute; fp32 inputs to 1e-4 relative plus
1e-7 (the fp32 log-sum-exp the prefill returns is itself held to 1e-5).
The probabilities of every row sum to 1, so each slot's importances sum to its
number of query rows (checked on the GPU result alone).

segpaged_select_tokens: integer work, bit-exact against oracle.importance on
seeded score arrays with many ties; at full size the selection made from the
device importances is checked to be a valid top-k of the oracle's scores within
the importance bound.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth
from synth import custom_layout, GLOBAL, LOCAL, RETRIEVAL, DENSE
from oracle import importance as oimp
import head_aware_paged_page_amd.segpaged as sp

pytestmark = pytest.mark.gpu

REL = {"bf16": 2e-2, "f32": 1e-4}
ABS = {"bf16": 1e-6, "f32": 1e-7}


def _wl(lay, **kw):
    from head_aware_paged_page_amd.workload import Workload
    print(f"[case] {lay.name} G={lay.group} D={lay.head_dim} ps={lay.page_size} slots={lay.n_slot} "
          f"seqs={lay.n_seq}", flush=True)
    return Workload(lay, device="cuda", **kw)


def _host(t):
    return t.double().cpu().numpy()


def check_importance(w, imp, pos_ptr, rows=None):
    lay = w.lay
    torch.cuda.synchronize()
    got_all = imp.double().cpu().numpy()
    rows = range(lay.n_slot * lay.n_seq) if rows is None else rows
    worst = 0.0
    for r in rows:
        slot, seq = divmod(r, lay.n_seq)
        K, _ = w.unit_host(slot, seq)
        t0 = int(w.h_tok_ptr[seq])
        q = _host(w.q_prefill[t0:t0 + lay.n_prefill, slot * lay.group:(slot + 1) * lay.group])
        q_pos = lay.new_base[seq] + np.arange(lay.n_prefill)
        n_pos = int(pos_ptr[seq + 1] - pos_ptr[seq])
        want = oimp.row_importance(lay, slot, seq, K, q, q_pos, n_pos)
        got = got_all[slot, pos_ptr[seq]:pos_ptr[seq + 1]]
        assert np.all(np.isfinite(got)), f"row {r}: non-finite importance"
        err = np.abs(got - want)
        bound = REL[lay.dtype] * want + ABS[lay.dtype]
        worst = max(worst, float(np.max(err / bound)))
        assert np.all(err <= bound), f"row {r} (class {lay.cls[slot]}): worst {np.max(err - bound)} over its bound"
    return worst


def check_row_sums(w, imp):
    """All positions covered: each slot's importances of a sequence sum to its rows."""
    lay = w.lay
    rows = lay.n_prefill * lay.group
    tot = imp.double().cpu().numpy()
    tol = 1e-3 if lay.dtype == "bf16" else 1e-5
    for slot in range(lay.n_slot):
        assert abs(tot[slot].sum() - rows * lay.n_seq) <= tol * rows * lay.n_seq, slot


SMALL = [
    # (group, head_dim, page_size, seg_lens, n_prefill, classes, dtype)
    (4, 128, 16, [[300, 77, 513]], 70, [(GLOBAL, 0), (LOCAL, 100), (RETRIEVAL, 0), (DENSE, 0), (LOCAL, 1)], "bf16"),
    (8, 128, 32, [[1000, 33], [64]], 45, [(LOCAL, 257), (GLOBAL, 0), (RETRIEVAL, 0)], "bf16"),
    (1, 64, 16, [[200, 31]], 600, [(GLOBAL, 0), (LOCAL, 40), (LOCAL, 1)], "bf16"),
    (16, 128, 16, [[17]], 9, [(GLOBAL, 0), (LOCAL, 5)], "bf16"),
    (2, 64, 32, [[1500, 33]], 300, [(GLOBAL, 0), (LOCAL, 300)], "bf16"),
    (4, 64, 16, [[300, 77]], 40, [(GLOBAL, 0), (LOCAL, 100), (RETRIEVAL, 0)], "f32"),
]


def _small(i):
    G, D, ps, lens, npf, classes, dt = SMALL[i]
    r = np.random.default_rng(40 + i)
    off = [list(r.integers(-5000, 5000, size=len(l))) for l in lens]
    ret = {}
    for slot, (c, _) in enumerate(classes):
        if c == RETRIEVAL:
            for q in range(len(lens)):
                nsp = sum(-(-l // ps) for l in lens[q])
                ret[(slot, q)] = np.sort(r.choice(nsp, size=max(1, nsp // 3), replace=False))
    return custom_layout(seg_lens=lens, offline=off, n_prefill=npf, n_decode=1, classes=classes, page_size=ps,
                         head_dim=D, group=G, dtype=dt, ret_lists=ret, name=f"imp{i}", seed=i)


@pytest.mark.parametrize("i", range(len(SMALL)))
def test_importance_small_layouts(i):
    """Several q-tiles (partial sums and their reduction), ragged tails, every class."""
    lay = _small(i)
    w = _wl(lay)
    w.prefill()
    imp, pos_ptr = w.importance()
    worst = check_importance(w, imp, pos_ptr)
    check_row_sums(w, imp)
    imp2, _ = w.importance()                 # a second call gives the same bits
    torch.cuda.synchronize()
    assert torch.equal(imp, imp2)
    print(f"[importance] {lay.name}: worst error {worst:.3f} of its bound")


@pytest.mark.parametrize("name", ["32k", "16k"])
def test_importance_full_config_every_row(name):
    w = synth.make_layout(name)
    w = _wl(w)
    w.prefill()
    imp, pos_ptr = w.importance()
    check_row_sums(w, imp)
    worst = check_importance(w, imp, pos_ptr)
    print(f"[importance] {name}: worst error {worst:.3f} of its bound")


def test_importance_128k_and_batch():
    """128K: every row sums to its 8192 query rows; the local rows against the
    oracle (a global row there costs the oracle minutes).  Batch: two rows per
    class against the oracle, every row's sum."""
    for name in ("128k", "batch"):
        lay = synth.make_layout(name)
        w = _wl(lay)
        w.prefill()
        imp, pos_ptr = w.importance()
        check_row_sums(w, imp)
        rng = np.random.default_rng(3)
        if name == "128k":
            rows = sorted(rng.choice(np.nonzero(lay.cls == LOCAL)[0], size=2, replace=False).tolist())
        else:
            rows = []
            for c in (GLOBAL, LOCAL, RETRIEVAL):
                for slot in rng.choice(np.nonzero(lay.cls == c)[0], size=2, replace=False):
                    rows.append(int(slot) * lay.n_seq + int(rng.integers(0, lay.n_seq)))
        worst = check_importance(w, imp, pos_ptr, rows=rows)
        print(f"[importance] {name}: worst error {worst:.3f} of its bound on rows {rows}")
        del w, imp
        torch.cuda.empty_cache()


@pytest.mark.parametrize("levels,long", [(0, False), (3, False), (64, False), (0, True), (5, True)])
def test_select_tokens_bit_exact(levels, long):
    """Seeded score arrays (levels > 0: many exact ties) through the selection:
    layer scores and selected positions equal the oracle's, bit for bit.
    Lists up to 32768 candidates are selected from LDS, longer ones from
    global memory (long=True adds one of 70000)."""
    n_layers, spl = 3, 5 if not long else 9
    lens = [1, 37, 1000, 4096, 30000] + ([70000] if long else [])
    pos_ptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    ks = [1, 10, 0, 4096, 7501] + ([17000] if long else [])
    sel_ptr = np.concatenate([[0], np.cumsum(ks)]).astype(np.int32)
    imp_h = synth.score_values(levels, n_layers * spl, int(pos_ptr[-1]), levels)
    imp = torch.from_numpy(imp_h).cuda()
    score = torch.full((n_layers, int(pos_ptr[-1])), float("nan"), dtype=torch.float32, device="cuda")
    sel = torch.full((n_layers, int(sel_ptr[-1])), -1, dtype=torch.int32, device="cuda")
    sp.select_tokens(imp, n_layers=n_layers, slots_per_layer=spl, n_seq=len(lens), h_pos_ptr=pos_ptr,
                     d_pos_ptr=torch.from_numpy(pos_ptr).cuda(), h_sel_ptr=sel_ptr,
                     d_sel_ptr=torch.from_numpy(sel_ptr).cuda(), score=score, sel=sel)
    torch.cuda.synchronize()
    score_h, sel_h = score.cpu().numpy(), sel.cpu().numpy()
    for l in range(n_layers):
        for s in range(len(lens)):
            a, b = pos_ptr[s], pos_ptr[s + 1]
            want_score = oimp.layer_scores(imp_h[l * spl:(l + 1) * spl, a:b])
            assert np.array_equal(score_h[l, a:b].view(np.uint32), want_score.view(np.uint32)), (l, s)
            want = oimp.select(want_score, ks[s])
            assert np.array_equal(sel_h[l, sel_ptr[s]:sel_ptr[s + 1]], want), (l, s)


def test_select_tokens_32k_end_to_end():
    """32K: importance of the reused segment positions from the device, then a
    quarter of them selected per layer.  The selection must be a valid top-k of
    the oracle's layer scores: nothing left out scores above anything taken by
    more than the importance bound allows."""
    lay = synth.make_layout("32k")
    w = _wl(lay)
    w.prefill()
    imp, pos_ptr = w.importance(span="segments")
    n_layers, spl = 8, 8
    n = int(pos_ptr[-1])
    k = n // 4
    sel_ptr = np.asarray([0, k], np.int32)
    score = torch.empty((n_layers, n), dtype=torch.float32, device="cuda")
    sel = torch.empty((n_layers, k), dtype=torch.int32, device="cuda")
    sp.select_tokens(imp, n_layers=n_layers, slots_per_layer=spl, n_seq=1, h_pos_ptr=pos_ptr,
                     d_pos_ptr=torch.from_numpy(pos_ptr).cuda(), h_sel_ptr=sel_ptr,
                     d_sel_ptr=torch.from_numpy(sel_ptr).cuda(), score=score, sel=sel)
    torch.cuda.synchronize()
    sel_h = sel.cpu().numpy()
    for l in (0, 5):
        want_imp = []
        for slot in range(l * spl, (l + 1) * spl):
            K, _ = w.unit_host(slot, 0)
            q = _host(w.q_prefill[:, slot * lay.group:(slot + 1) * lay.group])
            want_imp.append(oimp.row_importance(lay, slot, 0, K, q, lay.new_base[0] + np.arange(lay.n_prefill), n))
        ref = np.sum(want_imp, axis=0)
        s = sel_h[l]
        assert np.all(np.diff(s) > 0) and s[0] >= 0 and s[-1] < n
        taken = np.zeros(n, bool)
        taken[s] = True
        lo_taken, hi_left = ref[taken].min(), ref[~taken].max()
        slack = REL["bf16"] * max(lo_taken, hi_left) + 8 * ABS["bf16"]
        assert hi_left <= lo_taken + slack, (l, hi_left, lo_taken)


@pytest.mark.parametrize("seed", range(12))
def test_importance_random_layouts(seed):
    """The seeded random layouts of the whole-path test (every class, windows,
    retrieval lists, a sequence without a reused segment, several q-tiles):
    every row against the oracle, and every slot's sums."""
    from test_random_layouts_gpu import _draw
    lay = _draw(seed)
    w = _wl(lay)
    w.prefill()
    imp, pos_ptr = w.importance()
    check_row_sums(w, imp)
    worst = check_importance(w, imp, pos_ptr)
    print(f"[importance] {lay.name}: worst error {worst:.3f} of its bound")


def _wide_seeds():
    from test_random_layouts_gpu import _draw
    return [s for s in range(16) if _draw(s, wide=True).page_size in (16, 32)]


@pytest.mark.parametrize("seed", _wide_seeds())
def test_importance_random_wide_groups(seed):
    """The wide random layouts (groups 3, 5, 6, 12 and 16, several q-tiles per
    row) that use pages of 16 or 32 keys: every row against the oracle."""
    from test_random_layouts_gpu import _draw
    lay = _draw(seed, wide=True)
    w = _wl(lay)
    w.prefill()
    imp, pos_ptr = w.importance()
    check_row_sums(w, imp)
    worst = check_importance(w, imp, pos_ptr)
    print(f"[importance] {lay.name}: worst error {worst:.3f} of its bound")
