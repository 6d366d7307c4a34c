"""Pins of the oracle against what the pages and the mathematics fix (CPU only).

Each test checks the fp64 oracle against something other than itself: a
closed form, a textbook special case, a value worked out by hand or printed on
the pages, or a brute-force formulation written independently here.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import attention as oatt
from oracle import rope as orope
from oracle import tables as otab
from synth import custom_layout, GLOBAL, LOCAL, RETRIEVAL, DENSE

RNG = np.random.default_rng(1234)


# ------------------------------------------------------------------ rotary embedding

def test_rope_d2_is_textbook_rotation():
    """D = 2: w_0 = theta^0 = 1, so rope is the plane rotation by pos radians."""
    for pos in (0, 1, -3, 17, 2.5e4):
        x, y = 0.3, -1.7
        got = orope.rope(np.array([x, y]), pos, 10000.0)
        c, s = math.cos(pos), math.sin(pos)
        assert got == pytest.approx([c * x - s * y, s * x + c * y], abs=1e-12)


def test_rope_half_split_pairing_and_frequencies():
    """D = 4, theta = 1e4: w_0 = 1 and w_1 = 1e4^(-1/2) = 0.01; coordinate i pairs with i + D/2."""
    e0 = np.array([1.0, 0, 0, 0])
    e1 = np.array([0, 1.0, 0, 0])
    assert orope.rope(e0, 1, 1e4) == pytest.approx([math.cos(1), 0, math.sin(1), 0], abs=1e-15)
    assert orope.rope(e1, 100, 1e4) == pytest.approx([0, math.cos(1), 0, math.sin(1)], abs=1e-12)
    e3 = np.array([0, 0, 0, 1.0])          # second half rotates towards minus the first half
    assert orope.rope(e3, 100, 1e4) == pytest.approx([0, -math.sin(1), 0, math.cos(1)], abs=1e-12)


def test_rope_scores_depend_on_relative_position_only():
    """RoFormer property: <rope(q, m), rope(k, n)> is a function of m - n."""
    q, k = RNG.standard_normal(64), RNG.standard_normal(64)
    a = orope.rope(q, 700, 1e4) @ orope.rope(k, 300, 1e4)
    b = orope.rope(q, 5400, 1e4) @ orope.rope(k, 5000, 1e4)
    c = orope.rope(q, 400, 1e4) @ k
    assert a == pytest.approx(b, abs=1e-9) and a == pytest.approx(c, abs=1e-9)


@pytest.mark.parametrize("D", [2, 64, 128])
def test_relocate_closed_form(D):
    """A key rotated at old and relocated to new equals the key rotated at new directly."""
    k = RNG.standard_normal((8, D))
    for old, new in [(0, 5000), (-4096, 129000), (65536, 3), (131072, -131072), (7, 7)]:
        got = orope.relocate(orope.rope(k, old, 1e4), old, new, 1e4)
        assert np.max(np.abs(got - orope.rope(k, new, 1e4))) <= 1e-9 * np.max(np.abs(k))


def test_relocate_plus_minus_delta_is_identity():
    k = RNG.standard_normal((16, 128))
    for d in (1, 256, 4096, 65536, 131072):
        there = orope.relocate(k, 0, d, 1e4)
        back = orope.relocate(there, d, 0, 1e4)
        assert np.max(np.abs(back - k)) <= 1e-12 * 10


def test_relocate_zero_delta_is_identity():
    k = RNG.standard_normal((4, 128))
    for base in (0, 1000, -4096):
        assert np.max(np.abs(orope.relocate(k, base, base, 1e4) - k)) <= 1e-12


def test_relocate_preserves_pair_norms():
    k = RNG.standard_normal((4, 128))
    r = orope.relocate(k, 123, 98765, 1e4)
    n0 = k[:, :64] ** 2 + k[:, 64:] ** 2
    n1 = r[:, :64] ** 2 + r[:, 64:] ** 2
    assert np.max(np.abs(n0 - n1)) <= 1e-12


def test_relocate_equals_one_rotation_by_the_shift():
    """Rotations about the same planes compose additively: back by old then forward
    by new is one rotation by (new - old)."""
    k = RNG.standard_normal((4, 128))
    r = orope.relocate(k, 4096, 30000, 1e4)
    assert np.max(np.abs(r - orope.rope(k, 30000 - 4096, 1e4))) <= 1e-10


# ------------------------------------------------------------------ attention

def test_attend_two_keys_closed_form():
    """Two keys: weights are the logistic function of the score difference."""
    q = np.array([[1.0, 2.0]])
    K = np.array([[0.5, 0.0], [0.0, 1.0]])
    V = np.array([[1.0, 0.0], [0.0, 1.0]])
    o, lse = oatt.attend(q, K, V, 1.0)
    a, b = 0.5, 2.0
    w = 1.0 / (1.0 + math.exp(b - a))
    assert o[0] == pytest.approx([w, 1 - w], abs=1e-15)
    assert lse[0] == pytest.approx(math.log(math.exp(a) + math.exp(b)), abs=1e-14)


def test_attend_single_key_returns_its_value():
    v = RNG.standard_normal((1, 16))
    o, lse = oatt.attend(RNG.standard_normal((3, 16)), RNG.standard_normal((1, 16)), v, 0.25)
    assert np.array_equal(o, np.repeat(v, 3, axis=0))


def _rand_layout(ps, n_seg, seg_max, n_prefill, classes, seed):
    r = np.random.default_rng(seed)
    lens = [list(r.integers(1, seg_max + 1, size=n_seg))]
    off = [list(r.integers(-50, 50, size=n_seg))]
    lay = custom_layout(seg_lens=lens, offline=off, n_prefill=n_prefill, n_decode=1, classes=classes,
                        page_size=ps, head_dim=8, group=2)
    nsp = sum(-(-l // ps) for l in lens[0])
    for slot, (c, _w) in enumerate(classes):
        if c == RETRIEVAL:
            k = int(r.integers(0, nsp + 1))
            lay.ret_pages[(slot, 0)] = np.sort(r.choice(nsp, size=k, replace=False)).astype(np.int32)
    return lay


def _dense_mask(lay, slot, q_pos):
    """Brute-force visibility written from the class rules, independently of the
    oracle: one boolean per (query, token) from positions and segment offsets."""
    ps = lay.page_size
    c, w = int(lay.cls[slot]), int(lay.window[slot])
    listed = set(int(x) for x in lay.ret_pages.get((slot, 0), []))
    pos, is_new, ordinal = [], [], []
    base_ord = 0
    for ln, on in zip(lay.seg_len[0], lay.seg_online[0]):
        for o in range(int(ln)):
            pos.append(int(on) + o)
            is_new.append(False)
            ordinal.append(base_ord + o // ps)
        base_ord += -(-int(ln) // ps)
    for j in range(lay.n_new):
        pos.append(int(lay.new_base[0]) + j)
        is_new.append(True)
        ordinal.append(-1)
    M = np.zeros((len(q_pos), len(pos)), bool)
    for i, p in enumerate(q_pos):
        for j, t in enumerate(pos):
            if t > p:
                continue
            if c in (GLOBAL, DENSE):
                M[i, j] = True
            elif c == LOCAL:
                M[i, j] = p - t < w
            else:
                M[i, j] = is_new[j] or ordinal[j] in listed
    return M


@pytest.mark.parametrize("ps", [1, 2, 3, 4, 16])
def test_gather_oracle_matches_dense_masked_attention(ps):
    """The gather oracle equals full attention over all tokens with masked logits
    set to -inf (the masked formulation the method avoids), to 1e-12."""
    classes = [(GLOBAL, 0), (LOCAL, 1), (LOCAL, 5), (RETRIEVAL, 0), (DENSE, 0), (LOCAL, 40)]
    for seed in range(3):
        lay = _rand_layout(ps, 3, 13, 6, classes, seed)
        D, G = lay.head_dim, lay.group
        q_pos = list(range(int(lay.new_base[0]), int(lay.new_base[0]) + lay.n_new))
        for slot in range(lay.n_slot):
            ctx = lay.ctx_len(0)
            K = RNG.standard_normal((ctx + lay.n_new, D))
            V = RNG.standard_normal((ctx + lay.n_new, D))
            q = RNG.standard_normal((len(q_pos), G, D))
            O, L, cnt = oatt.row_attention(lay, slot, 0, K, V, q, q_pos)
            M = _dense_mask(lay, slot, q_pos)
            s = np.einsum("igd,td->igt", q, K) / math.sqrt(D)
            s = np.where(M[:, None, :], s, -np.inf)
            mx = s.max(axis=2, keepdims=True)
            e = np.exp(s - mx)
            O2 = np.einsum("igt,td->igd", e, V) / e.sum(axis=2)[..., None]
            L2 = mx[..., 0] + np.log(e.sum(axis=2))
            assert np.max(np.abs(O - O2)) <= 1e-12
            assert np.max(np.abs(L - L2)) <= 1e-12
            assert np.array_equal(cnt, M.sum(axis=1))


@pytest.mark.parametrize("ps", [1, 3, 4, 16])
def test_visible_counts_match_brute_force_mask(ps):
    """oracle.tables.visible_counts (the expected value of the GPU's count checks)
    equals the row sums of the brute-force mask, for every class, query position
    and page size, including retrieval lists that are empty or list every page."""
    classes = [(GLOBAL, 0), (LOCAL, 1), (LOCAL, 4), (LOCAL, 1000), (RETRIEVAL, 0), (RETRIEVAL, 0), (DENSE, 0)]
    for seed in range(4):
        lay = _rand_layout(ps, 4, 11, 7, classes, 100 + seed)
        nsp = sum(-(-int(l) // ps) for l in lay.seg_len[0])
        lay.ret_pages[(5, 0)] = np.arange(nsp, dtype=np.int32) if seed % 2 else np.zeros(0, np.int32)
        q_pos = list(range(int(lay.new_base[0]), int(lay.new_base[0]) + lay.n_new))
        for slot in range(lay.n_slot):
            want = _dense_mask(lay, slot, q_pos).sum(axis=1)
            assert np.array_equal(otab.visible_counts(lay, slot, 0, q_pos), want), (seed, slot)


def test_visible_counts_match_hand_fixture(golden_dir):
    """The visible sets worked out by hand in tests/golden/tiny_tables_by_hand.json
    fix the counts: global at p = 9 sees 10 tokens, local(3) at p = 10 and 13
    sees 3, retrieval at p = 11 sees 5, dense at p = 13 sees 14."""
    g, lay = _tiny_hand(golden_dir)
    for v in g["expected_visible"]:
        got = otab.visible_counts(lay, v["slot"], 0, [v["p"]])
        assert got.tolist() == [len(v["positions"])]
    assert [len(v["positions"]) for v in g["expected_visible"]] == [10, 3, 5, 14, 3]


def test_window_one_returns_own_value_and_zero_query_averages():
    lay = custom_layout(seg_lens=[[9, 4]], offline=[[0, 0]], n_prefill=3, n_decode=1,
                        classes=[(LOCAL, 1), (GLOBAL, 0)], page_size=4, head_dim=8, group=1)
    K = RNG.standard_normal((17, 8))
    V = RNG.standard_normal((17, 8))
    q_pos = [13, 14, 15, 16]
    O, _, cnt = oatt.row_attention(lay, 0, 0, K, V, RNG.standard_normal((4, 1, 8)), q_pos)
    assert np.array_equal(cnt, [1, 1, 1, 1])
    assert np.array_equal(O[:, 0], V[13:17])
    O, L, cnt = oatt.row_attention(lay, 1, 0, K, V, np.zeros((4, 1, 8)), q_pos)
    for i, p in enumerate(q_pos):
        assert cnt[i] == p + 1
        assert np.max(np.abs(O[i, 0] - V[: p + 1].mean(axis=0))) <= 1e-14
        assert L[i, 0] == pytest.approx(math.log(p + 1), abs=1e-14)


def test_class_reductions():
    """local with W beyond every position = global; retrieval listing every segment
    page = global; dense = global."""
    lens = [[7, 5, 9]]
    nsp = 2 + 2 + 3
    classes = [(GLOBAL, 0), (LOCAL, 10 ** 6), (RETRIEVAL, 0), (DENSE, 0)]
    lay = custom_layout(seg_lens=lens, offline=[[0, 3, -9]], n_prefill=5, n_decode=1, classes=classes,
                        page_size=4, head_dim=8, group=2, ret_lists={(2, 0): list(range(nsp))})
    K = RNG.standard_normal((27, 8))
    V = RNG.standard_normal((27, 8))
    q = RNG.standard_normal((6, 2, 8))
    q_pos = list(range(21, 27))
    ref = oatt.row_attention(lay, 0, 0, K, V, q, q_pos)
    for slot in (1, 2, 3):
        got = oatt.row_attention(lay, slot, 0, K, V, q, q_pos)
        assert np.array_equal(got[0], ref[0]) and np.array_equal(got[2], ref[2])


# ------------------------------------------------------------------ tables

def test_paged_block_walkthrough(golden_dir):
    """The 4-token-block walk-through printed on the PagedAttention page."""
    g = json.load(open(os.path.join(golden_dir, "paged_block_walkthrough.json")))
    lay = custom_layout(seg_lens=[[]], offline=[[]], n_prefill=g["prompt_tokens"],
                        n_decode=g["generated_tokens"], classes=[(GLOBAL, 0)], page_size=g["page_size"])
    storage, chain_ptr = otab.allocate(lay, np.asarray(g["free_list"]))
    assert storage.tolist() == g["expected_block_table"]
    used = len(storage)
    assert sorted(g["free_list"][used:]) == g["expected_unused_blocks"]
    tpos, tpage, _, _ = otab.tokens(lay, 0)
    slots = [[int(tpage[i]), int(tpos[i] - otab.chain(lay, 0)[tpage[i]]["pos_start"])] for i in range(len(tpos))]
    assert slots == g["expected_token_slots"]
    # after the second generated token, the table of a query at the last position reads all three blocks
    row_ptr, ent = otab.tables(lay, storage, chain_ptr, [8], [8])
    assert ent[:, 0].tolist() == g["expected_block_table"]


def _tiny_hand(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "tiny_tables_by_hand.json")))
    ret = {tuple(int(x) for x in k.split(",")): v for k, v in g["ret_lists"].items()}
    lay = custom_layout(seg_lens=[g["seg_lens"]], offline=[g["offline"]], n_prefill=g["n_prefill"],
                        n_decode=g["n_decode"], classes=[tuple(c) for c in g["classes"]],
                        page_size=g["page_size"], ret_lists=ret)
    return g, lay


def test_tables_by_hand(golden_dir):
    g, lay = _tiny_hand(golden_dir)
    storage, chain_ptr = otab.allocate(lay, np.asarray(g["free_list"]))
    assert storage.tolist() == g["expected_storage"]
    for call in ("prefill", "decode"):
        lo, hi = g[f"{call}_q"]
        row_ptr, ent = otab.tables(lay, storage, chain_ptr, [lo], [hi])
        rows = [ent[row_ptr[r]:row_ptr[r + 1]].tolist() for r in range(lay.n_slot)]
        assert rows == g[f"expected_{call}_rows"]
    assert otab.reloc_list(lay, storage, chain_ptr).tolist() == g["expected_reloc"]
    for v in g["expected_visible"]:
        tpos, _tp, tsp, tnew = otab.tokens(lay, 0)
        m = otab.visible(int(lay.cls[v["slot"]]), int(lay.window[v["slot"]]),
                         lay.ret_pages.get((v["slot"], 0), []), tpos, tsp, tnew, v["p"])
        assert tpos[m].tolist() == v["positions"]


def test_allocation_is_a_prefix_of_the_free_list_and_disjoint():
    lay = _rand_layout(4, 3, 20, 7, [(GLOBAL, 0), (LOCAL, 3), (RETRIEVAL, 0)], 5)
    free = np.random.default_rng(0).permutation(500)
    storage, chain_ptr = otab.allocate(lay, free)
    assert np.array_equal(storage, free[: len(storage)])
    assert len(set(storage.tolist())) == len(storage)
    with pytest.raises(MemoryError):
        otab.allocate(lay, free[: len(storage) - 1])


# ---------------------------------------------------------------- per-head page pack / unpack
from oracle import pack as opack  # noqa: E402


def _hand_pool(n_pages, ps, D):
    k = np.array([[[100 * p + 10 * s + d for d in range(D)] for s in range(ps)] for p in range(n_pages)], np.float64)
    v = np.array([[[-(100 * p + 10 * d + s) for s in range(ps)] for d in range(D)] for p in range(n_pages)], np.float64)
    return k, v


def test_pack_matches_hand_worked_example():
    """tests/golden/pack_by_hand.json: packed pages of a hand-written table, worked out by hand."""
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pack_by_hand.json")))
    k, v = _hand_pool(g["n_pages"], g["page_size"], g["head_dim"])
    kp, vp = opack.pack(k, v, np.array(g["phys"]))
    assert np.array_equal(kp, np.array(g["k_packed"], np.float64))
    assert np.array_equal(vp, np.array(g["v_packed"], np.float64))


def test_pack_unpack_round_trip_restores_exactly_the_listed_pages():
    rng = np.random.default_rng(5)
    k = rng.standard_normal((40, 16, 8))
    v = rng.standard_normal((40, 8, 16))
    phys = rng.choice(40, size=17, replace=False)
    kp, vp = opack.pack(k, v, phys)
    assert kp.nbytes + vp.nbytes == 17 * (k[0].nbytes + v[0].nbytes)   # bytes = listed pages only
    k2, v2 = opack.unpack(kp, vp, phys, np.zeros_like(k), np.zeros_like(v))
    listed = np.zeros(40, bool)
    listed[phys] = True
    assert np.array_equal(k2[listed], k[listed]) and np.array_equal(v2[listed], v[listed])
    assert not k2[~listed].any() and not v2[~listed].any()


# ---------------------------------------------------------------- window-only storage and page release

def _window_hand(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "window_storage_by_hand.json")))
    lay = custom_layout(seg_lens=[g["seg_lens"]], offline=[g["offline"]], n_prefill=g["n_prefill"],
                        n_decode=g["n_decode"], classes=[tuple(c) for c in g["classes"]], page_size=g["page_size"])
    return g, lay


def test_window_storage_by_hand(golden_dir):
    """tests/golden/window_storage_by_hand.json: stored pages, allocation, the
    relocation list, the prefill tables, then releases and decode tables step
    by step until the sequence ends, all worked out by hand."""
    g, lay = _window_hand(golden_dir)
    storage, chain_ptr = otab.allocate_window(lay, np.asarray(g["free_list"]), [g["keep_from"]])
    assert storage.tolist() == g["expected_storage"] and chain_ptr.tolist() == g["expected_chain_ptr"]
    assert otab.reloc_list(lay, storage, chain_ptr).tolist() == g["expected_reloc"]
    row_ptr, ent = otab.tables(lay, storage, chain_ptr, [9], [12])
    assert [ent[row_ptr[r]:row_ptr[r + 1]].tolist() for r in range(3)] == g["expected_prefill_rows"]
    freed = []
    for st in g["steps"]:
        rel, storage = otab.release(lay, storage, chain_ptr, [st["release_at"]])
        assert rel.tolist() == st["expected_released"]
        freed += rel.tolist()
        if "decode_at" in st:
            p = st["decode_at"]
            row_ptr, ent = otab.tables(lay, storage, chain_ptr, [p], [p])
            assert [ent[row_ptr[r]:row_ptr[r + 1]].tolist() for r in range(3)] == st["expected_decode_rows"]
    assert sorted(freed) == sorted(x for x in g["expected_storage"] if x >= 0) and (storage == -1).all()
    with pytest.raises(LookupError):          # a released page cannot appear in a table
        otab.tables(lay, storage, chain_ptr, [15], [15])


def test_walkthrough_end_of_sequence_release(golden_dir):
    """The PagedAttention page's walk-through: when the sequence ends, blocks 7, 1
    and 3 return to the pool, which then again holds all nine blocks."""
    g = json.load(open(os.path.join(golden_dir, "paged_block_walkthrough.json")))
    lay = custom_layout(seg_lens=[[]], offline=[[]], n_prefill=g["prompt_tokens"],
                        n_decode=g["generated_tokens"], classes=[(GLOBAL, 0)], page_size=g["page_size"])
    free = np.asarray(g["free_list"])
    storage, chain_ptr = otab.allocate_window(lay, free, [0])
    assert storage.tolist() == g["expected_block_table"]
    # while tokens remain to be generated nothing is released
    for p_next in range(0, otab.seq_end(lay, 0)):
        assert len(otab.release(lay, storage, chain_ptr, [p_next])[0]) == 0
    rel, after = otab.release(lay, storage, chain_ptr, [otab.seq_end(lay, 0)])
    assert rel.tolist() == [7, 1, 3]
    assert sorted(free[len(storage):].tolist()) == g["expected_unused_blocks"]
    assert sorted(free[len(storage):].tolist() + rel.tolist()) == sorted(g["free_list"]) and (after == -1).all()


def _needed_closed_form(lay, seq, c, W, listed, p_from):
    """Chain pages a head still needs once every query is at or after p_from, in
    closed form: none once the sequence is over; otherwise for local(W) the
    pages whose last position is at least p_from - W + 1, for retrieval the
    listed segment pages and the new-token pages, for the rest all pages."""
    out = []
    for pg in otab.chain(lay, seq):
        last = pg["pos_start"] + pg["n_valid"] - 1
        if p_from >= otab.seq_end(lay, seq):
            out.append(False)
        elif c == LOCAL:
            out.append(last >= p_from - W + 1)
        elif c == RETRIEVAL:
            out.append(pg["seg"] < 0 or pg["seg_page"] in set(int(x) for x in listed))
        else:
            out.append(True)
    return np.asarray(out)


@pytest.mark.parametrize("seed", range(5))
def test_window_storage_and_release_closed_form(seed):
    """On random layouts the stored pages after allocation, and the live pages
    after a release at every later position, are exactly the closed-form sets."""
    r = np.random.default_rng(300 + seed)
    ps = int(r.choice([1, 2, 4, 16]))
    lens = [list(r.integers(1, 40, size=int(r.integers(1, 4))))]
    classes = [(GLOBAL, 0), (LOCAL, int(r.integers(1, 30))), (LOCAL, 1), (RETRIEVAL, 0), (DENSE, 0),
               (LOCAL, 1000)]
    nsp = sum(-(-l // ps) for l in lens[0])
    listed = np.sort(r.choice(nsp, size=min(2, nsp), replace=False))
    lay = custom_layout(seg_lens=lens, offline=[[0] * len(lens[0])], n_prefill=int(r.integers(1, 9)),
                        n_decode=int(r.integers(1, 12)), classes=classes, page_size=ps,
                        ret_lists={(3, 0): listed})
    k0 = int(lay.new_base[0])
    storage, chain_ptr = otab.allocate_window(lay, r.permutation(4000), [k0])
    for slot, (c, W) in enumerate(classes):
        got = storage[chain_ptr[slot]:chain_ptr[slot + 1]] >= 0
        assert np.array_equal(got, _needed_closed_form(lay, 0, c, W, listed, k0)), slot
    assert len(set(storage[storage >= 0].tolist())) == int((storage >= 0).sum())
    for p_next in range(k0, otab.seq_end(lay, 0) + 2):
        rel, after = otab.release(lay, storage, chain_ptr, [p_next])
        for slot, (c, W) in enumerate(classes):
            live = after[chain_ptr[slot]:chain_ptr[slot + 1]] >= 0
            want = _needed_closed_form(lay, 0, c, W, listed, p_next)
            assert np.array_equal(live, want), (slot, p_next)
        assert sorted(rel.tolist()) == sorted(storage[(storage >= 0) & (after < 0)].tolist())


# ---------------------------------------------------------------- attention importance and token selection
from oracle import importance as oimp  # noqa: E402


def _imp_layout(ps, seed):
    classes = [(GLOBAL, 0), (LOCAL, 1), (LOCAL, 5), (RETRIEVAL, 0), (DENSE, 0), (LOCAL, 40)]
    return _rand_layout(ps, 3, 13, 6, classes, seed)


@pytest.mark.parametrize("ps", [1, 3, 4, 16])
def test_importance_equals_column_sums_of_dense_masked_softmax(ps):
    """Importance = column sums, over every query row and head, of the dense masked
    softmax matrix (the mask formulation of the same attention, built
    independently of the oracle's visible sets)."""
    for seed in range(3):
        lay = _imp_layout(ps, seed)
        D, G = lay.head_dim, lay.group
        q_pos = list(range(int(lay.new_base[0]), int(lay.new_base[0]) + lay.n_new))
        n_tok = lay.ctx_len(0) + lay.n_new
        for slot in range(lay.n_slot):
            K = RNG.standard_normal((n_tok, D))
            q = RNG.standard_normal((len(q_pos), G, D))
            got = oimp.row_importance(lay, slot, 0, K, q, q_pos, n_tok)
            M = _dense_mask(lay, slot, q_pos)
            s = np.einsum("igd,td->igt", q, K) / math.sqrt(D)
            s = np.where(M[:, None, :], s, -np.inf)
            e = np.exp(s - s.max(axis=2, keepdims=True))
            P = e / e.sum(axis=2, keepdims=True)
            want = P.sum(axis=(0, 1))                 # positions are 0 .. n_tok-1 in token order here
            assert np.max(np.abs(got - want)) <= 1e-12
            assert abs(got.sum() - len(q_pos) * G) <= 1e-10     # each row's probabilities sum to 1


def test_importance_zero_queries_closed_form():
    """Q = 0: every visible token of a query gets 1/|V(p)|; with positions 0..N-1
    contiguous, |V(p)| = p + 1 (global) or min(W, p + 1) (local W), so
    imp(t) = G * sum over queries p >= t (and p < t + W for local) of 1/|V(p)|."""
    lay = custom_layout(seg_lens=[[7, 5]], offline=[[0, 0]], n_prefill=6, n_decode=1,
                        classes=[(GLOBAL, 0), (LOCAL, 4)], page_size=4, head_dim=8, group=3)
    q_pos = list(range(12, 18))
    n = 18
    K = RNG.standard_normal((n, 8))
    for slot, W in ((0, None), (1, 4)):
        got = oimp.row_importance(lay, slot, 0, K, np.zeros((6, 3, 8)), q_pos, n)
        want = np.zeros(n)
        for t in range(n):
            for p in q_pos:
                if t <= p and (W is None or t > p - W):
                    want[t] += 3.0 / ((p + 1) if W is None else min(W, p + 1))
        assert np.max(np.abs(got - want)) <= 1e-14


def test_select_by_hand(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "select_by_hand.json")))
    score = np.asarray(g["score"], np.float32)
    for c in g["cases"]:
        assert oimp.select(score, c["k"]).tolist() == c["expected"]
    ls = g["layer_sum"]
    got = oimp.layer_scores(np.asarray(ls["slots"], np.float64))
    assert got.dtype == np.float32 and got.tolist() == ls["expected"]


def test_select_is_the_stable_descending_order():
    """Brute force on small random arrays with many ties: the selection is the
    first k of the positions sorted by (score descending, position ascending)."""
    r = np.random.default_rng(8)
    for _ in range(200):
        n = int(r.integers(1, 40))
        score = r.integers(0, 5, n).astype(np.float32) / 4
        k = int(r.integers(0, n + 1))
        ranked = sorted(range(n), key=lambda t: (-float(score[t]), t))
        assert oimp.select(score, k).tolist() == sorted(ranked[:k])
