"""Window-only storage and page release through the C ABI, on the CPU.

segpaged_build_tables_ex (with keep_from), segpaged_tables_from_chains and
segpaged_release_pages are host-only integer work: bit-exact against the
oracle (storage with its -1 holes, tables, relocation list as a set, released
ids in order) on the hand-worked fixture, random layouts stepped through a whole
decode, and the 32K workload; plus the errors they promise.
"""
import json
import os

import numpy as np
import pytest

import synth
from oracle import tables as otab
from synth import custom_layout, GLOBAL, LOCAL, RETRIEVAL, DENSE
from head_aware_paged_page_amd import segpaged as sp


def _layout_args(lay):
    a = lay.abi_arrays("prefill")
    return {k: a[k] for k in ("seg_ptr", "segs", "n_new", "cls", "window", "ret_ptr", "ret_pages")}


def _calls(lay):
    la = _layout_args(lay)
    ps = lay.page_size
    def tables(storage, chain_ptr, p_lo, p_hi):
        return sp.tables_from_chains(**la, q_lo=p_lo, q_hi=p_hi, page_size=ps, chain_ptr=chain_ptr, storage=storage)
    def release(storage, chain_ptr, p_next):
        return sp.release_pages(**la, page_size=ps, p_next=p_next, chain_ptr=chain_ptr, storage=storage)
    return tables, release


def _check_against_oracle(lay, free, keep_from, rows=None):
    """Build with keep_from, compare to the oracle, then step the decode: release
    at each next position and compare tables and released ids, to the end."""
    a = lay.abi_arrays("prefill")
    t = sp.build_tables_ex(**a, page_size=lay.page_size, free_list=free, keep_from=keep_from)
    o_storage, o_chain_ptr = otab.allocate_window(lay, free, keep_from)
    assert np.array_equal(t["chain_ptr"], o_chain_ptr)
    assert np.array_equal(t["storage"], o_storage)
    assert t["counts"][3] == int((o_storage >= 0).sum())
    rl = otab.reloc_list(lay, o_storage, o_chain_ptr)
    assert np.array_equal(t["reloc"][:, :3], rl[np.argsort(rl[:, 0], kind="stable")])
    row_ptr, ent = otab.tables(lay, o_storage, o_chain_ptr, a["q_lo"], a["q_hi"])
    assert np.array_equal(t["row_ptr"], row_ptr) and np.array_equal(t["entries"][:, :3], ent)
    tables, release = _calls(lay)
    storage = t["storage"].copy()
    for step in range(lay.n_decode + 1):
        p = lay.new_base + lay.n_prefill + step               # next query position of every sequence
        rel = release(storage, t["chain_ptr"], p)
        o_rel, o_storage = otab.release(lay, o_storage, o_chain_ptr, p)
        assert np.array_equal(rel, o_rel), f"released ids at step {step}"
        assert np.array_equal(storage, o_storage)
        if step < lay.n_decode:
            rp, en = tables(storage, t["chain_ptr"], p, p)
            orp, oen = otab.tables(lay, o_storage, o_chain_ptr, p, p)
            assert np.array_equal(rp, orp) and np.array_equal(en[:, :3], oen), f"decode tables at step {step}"
    assert (storage == -1).all()                               # the sequences are over: every page is back


def test_hand_fixture_through_the_library(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "window_storage_by_hand.json")))
    lay = custom_layout(seg_lens=[g["seg_lens"]], offline=[g["offline"]], n_prefill=g["n_prefill"],
                        n_decode=g["n_decode"], classes=[tuple(c) for c in g["classes"]], page_size=g["page_size"])
    a = lay.abi_arrays("prefill")
    t = sp.build_tables_ex(**a, page_size=4, free_list=np.asarray(g["free_list"]), keep_from=[g["keep_from"]])
    assert t["storage"].tolist() == g["expected_storage"] and t["chain_ptr"].tolist() == g["expected_chain_ptr"]
    assert t["counts"].tolist() == [15, 9, 6, 12]
    assert t["reloc"][:, :3].tolist() == sorted(g["expected_reloc"])
    assert [t["entries"][t["row_ptr"][r]:t["row_ptr"][r + 1], :3].tolist() for r in range(3)] == \
        g["expected_prefill_rows"]
    tables, release = _calls(lay)
    storage = t["storage"].copy()
    for st in g["steps"]:
        assert release(storage, t["chain_ptr"], [st["release_at"]]).tolist() == st["expected_released"]
        if "decode_at" in st:
            rp, en = tables(storage, t["chain_ptr"], [st["decode_at"]], [st["decode_at"]])
            assert [en[rp[r]:rp[r + 1], :3].tolist() for r in range(3)] == st["expected_decode_rows"]
    with pytest.raises(sp.SegPagedError) as e:           # a released page cannot be read
        tables(storage, t["chain_ptr"], [15], [15])
    assert e.value.status == sp.SP_EINVAL and "not stored" in str(e.value)


@pytest.mark.parametrize("seed", range(6))
def test_random_layouts_every_decode_step(seed):
    r = np.random.default_rng(700 + seed)
    ps = int(r.choice([1, 2, 4, 16]))
    n_seq = int(r.integers(1, 4))
    lens = [list(r.integers(1, 60, size=int(r.integers(0, 4)))) for _ in range(n_seq)]
    off = [list(r.integers(-300, 300, size=len(l))) for l in lens]
    classes = [(GLOBAL, 0), (LOCAL, int(r.integers(1, 40))), (RETRIEVAL, 0), (DENSE, 0), (LOCAL, 1),
               (LOCAL, int(r.integers(1, 9)))]
    ret = {}
    for q in range(n_seq):
        nsp = sum(-(-l // ps) for l in lens[q])
        ret[(2, q)] = np.sort(r.choice(nsp, size=int(r.integers(0, nsp + 1)), replace=False))
    lay = custom_layout(seg_lens=lens, offline=off, n_prefill=int(r.integers(1, 12)),
                        n_decode=int(r.integers(1, 20)), classes=classes, page_size=ps, ret_lists=ret)
    free = np.random.default_rng(seed).permutation(20000).astype(np.int32)
    _check_against_oracle(lay, free, lay.new_base.astype(np.int32))


def test_32k_window_storage_bit_exact():
    """The 32K workload with window-only storage: 20 018 of 120 512 chain pages
    stored (the 10 global slots whole, 1883 pages each; the 54 local slots
    17 segment pages ending at or after 30000 - 256 + 1, plus 5 new-token pages), compared
    with the oracle; then the decode token's release."""
    lay = synth.make_layout("32k")
    free = synth.free_list(lay, 120512)
    a = lay.abi_arrays("prefill")
    t = sp.build_tables_ex(**a, page_size=16, free_list=free, keep_from=a["q_lo"])
    o_storage, o_chain_ptr = otab.allocate_window(lay, free, a["q_lo"])
    assert np.array_equal(t["storage"], o_storage) and np.array_equal(t["chain_ptr"], o_chain_ptr)
    assert t["counts"][3] == 10 * 1883 + 54 * (17 + 5)     # local: 17 segment pages reach the window, 5 new
    row_ptr, ent = otab.tables(lay, o_storage, o_chain_ptr, a["q_lo"], a["q_hi"])
    assert np.array_equal(t["entries"][:, :3], ent)
    d = lay.abi_arrays("decode")
    tables, release = _calls(lay)
    storage = t["storage"].copy()
    rel = release(storage, t["chain_ptr"], d["q_lo"])
    o_rel, o_storage = otab.release(lay, o_storage, o_chain_ptr, d["q_lo"])
    assert np.array_equal(rel, o_rel) and np.array_equal(storage, o_storage)
    rp, en = tables(storage, t["chain_ptr"], d["q_lo"], d["q_hi"])
    orp, oen = otab.tables(lay, o_storage, o_chain_ptr, d["q_lo"], d["q_hi"])
    assert np.array_equal(en[:, :3], oen)


def test_whole_chain_build_is_unchanged():
    """keep_from = NULL is segpaged_build_tables: same storage, tables and list."""
    lay = synth.make_layout("16k")
    a = lay.abi_arrays("prefill")
    free = synth.free_list(lay, 66112 + 10)
    t0 = sp.build_tables(**a, page_size=16, free_list=free)
    t1 = sp.build_tables_ex(**a, page_size=16, free_list=free)
    for k in ("chain_ptr", "storage", "row_ptr", "entries", "reloc"):
        assert np.array_equal(t0[k], t1[k]), k
    assert t1["counts"][0] == t1["counts"][3] == t0["counts"][0]


def test_errors():
    lay = custom_layout(seg_lens=[[40]], offline=[[0]], n_prefill=5, n_decode=3,
                        classes=[(GLOBAL, 0), (LOCAL, 8)], page_size=4)
    a = lay.abi_arrays("prefill")
    free = np.arange(100, dtype=np.int32)
    with pytest.raises(sp.SegPagedError) as e:           # keep_from after the call's first query
        sp.build_tables_ex(**a, page_size=4, free_list=free, keep_from=[41])
    assert e.value.status == sp.SP_EINVAL
    t = sp.build_tables_ex(**a, page_size=4, free_list=free, keep_from=[40])
    with pytest.raises(sp.SegPagedError) as e:           # p_next before the new tokens
        sp.release_pages(**_layout_args(lay), page_size=4, p_next=[39], chain_ptr=t["chain_ptr"],
                         storage=t["storage"].copy())
    assert e.value.status == sp.SP_EINVAL
    with pytest.raises(sp.SegPagedError) as e:           # too short a free list for the stored pages
        sp.build_tables_ex(**a, page_size=4, free_list=free[: t["counts"][3] - 1], keep_from=[40])
    assert e.value.status == sp.SP_ENOMEM
    n = sp.build_tables_ex(**a, page_size=4, free_list=None, keep_from=[40], counts_only=True)["counts"]
    assert n.tolist() == t["counts"].tolist()
