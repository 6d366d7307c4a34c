"""The C ABI on the CPU: the library loads and exports every declared symbol, and
segpaged_build_tables (host-only) matches the oracle's allocation, tables and
relocation list bit-exactly, plus its error codes."""
import json
import os
import re

import numpy as np
import pytest

from oracle import tables as otab
import synth
from synth import custom_layout, GLOBAL, LOCAL, RETRIEVAL, DENSE
from head_aware_paged_page_amd import segpaged as sp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_declared_symbol():
    hdr = open(os.path.join(ROOT, "include", "segpaged.h")).read()
    body = re.sub(r"/\*.*?\*/", "", hdr, flags=re.S)
    names = set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", body, flags=re.M))
    names.discard("if")
    assert {"segpaged_build_tables", "rope_relocate", "segpaged_prefill", "segpaged_decode",
            "segpaged_workspace_bytes", "segpaged_strerror", "segpaged_last_error", "segpaged_version"} <= names
    L = sp.lib()
    for n in sorted(names):
        assert hasattr(L, n), f"{n} declared in segpaged.h but not exported"
    assert sp.version() == 100


def test_library_has_no_unresolved_internal_symbols():
    """Every kernel's host launch stub must be defined (a device-only builtin in a
    kernel body can make the host pass drop it silently)."""
    import subprocess
    out = subprocess.run(["nm", "-D", "--undefined-only", sp._LIB_PATH], capture_output=True, text=True).stdout
    bad = [l for l in out.splitlines() if "_ZN2sp" in l]
    assert not bad, bad[:5]


def _lib_tables(lay, call, free):
    return sp.build_tables(**lay.abi_arrays(call), page_size=lay.page_size, free_list=free)


def _compare(lay, free, rows=None):
    """Library vs oracle for the prefill and the decode call; `rows` limits the table rows compared."""
    storage, chain_ptr = otab.allocate(lay, free)
    for call in ("prefill", "decode"):
        a = lay.abi_arrays(call)
        t = _lib_tables(lay, call, free)
        assert np.array_equal(t["chain_ptr"], chain_ptr)
        assert np.array_equal(t["storage"], storage)
        if rows is None:
            row_ptr, ent = otab.tables(lay, storage, chain_ptr, a["q_lo"], a["q_hi"])
            assert np.array_equal(t["row_ptr"], row_ptr)
            assert np.array_equal(t["entries"][:, :3], ent)
            assert not t["entries"][:, 3].any()
        else:
            for r in rows:
                slot, seq = divmod(r, lay.n_seq)
                ent = otab.row_table(lay, storage, chain_ptr, slot, seq, a["q_lo"][seq], a["q_hi"][seq])
                got = t["entries"][t["row_ptr"][r]:t["row_ptr"][r + 1], :3]
                assert np.array_equal(got, ent), f"row {r} ({call})"
    # The relocation items are independent, so the library lists them in
    # ascending physical page; page ids are distinct, so the sorted list is
    # unique and compared whole.
    rl = otab.reloc_list(lay, storage, chain_ptr, rows=None if rows is None else set(rows))
    got = t["reloc"][:, :3]
    assert np.all(np.diff(got[:, 0]) > 0), "relocation list not in ascending physical page"
    if rows is not None:
        got = got[np.isin(got[:, 0], rl[:, 0])]
    assert np.array_equal(got, rl[np.argsort(rl[:, 0], kind="stable")])


@pytest.mark.parametrize("seed", range(6))
def test_random_layouts_bit_exact(seed):
    r = np.random.default_rng(seed)
    ps = int(r.choice([1, 2, 3, 4, 8, 16, 32]))
    n_seq = int(r.integers(1, 4))
    lens = [list(r.integers(1, 70, size=int(r.integers(0, 4)))) for _ in range(n_seq)]
    off = [list(r.integers(-300, 300, size=len(l))) for l in lens]
    classes = [(GLOBAL, 0), (LOCAL, int(r.integers(1, 90))), (RETRIEVAL, 0), (DENSE, 0), (LOCAL, 1)]
    ret = {}
    for q in range(n_seq):
        nsp = sum(-(-l // ps) for l in lens[q])
        k = int(r.integers(0, nsp + 1))
        ret[(2, q)] = np.sort(r.choice(nsp, size=k, replace=False))
    lay = custom_layout(seg_lens=lens, offline=off, n_prefill=int(r.integers(1, 40)), n_decode=1, classes=classes,
                        page_size=ps, ret_lists=ret)
    n = sp.build_tables(**lay.abi_arrays("prefill"), page_size=ps, free_list=None, counts_only=True)["counts"][0]
    free = np.random.default_rng(seed + 100).permutation(int(n) + 7).astype(np.int32)
    _compare(lay, free)


def test_tiny_config_bit_exact():
    lay = synth.make_layout("tiny")
    n = sp.build_tables(**lay.abi_arrays("prefill"), page_size=lay.page_size, free_list=None,
                        counts_only=True)["counts"][0]
    _compare(lay, synth.free_list(lay, int(n)))


@pytest.mark.parametrize("name", ["32k", "16k"])
def test_full_configs_bit_exact(name):
    lay = synth.make_layout(name)
    n = sp.build_tables(**lay.abi_arrays("prefill"), page_size=lay.page_size, free_list=None,
                        counts_only=True)["counts"][0]
    _compare(lay, synth.free_list(lay, int(n)))


@pytest.mark.parametrize("name", ["128k", "batch"])
def test_large_configs_sampled_rows_bit_exact(name):
    lay = synth.make_layout(name)
    n = sp.build_tables(**lay.abi_arrays("prefill"), page_size=lay.page_size, free_list=None,
                        counts_only=True)["counts"][0]
    free = synth.free_list(lay, int(n))
    rows_all = lay.n_slot * lay.n_seq
    rng = np.random.default_rng(7)
    # every class, plus the first and last rows
    rows = {0, rows_all - 1}
    for c in (GLOBAL, LOCAL, RETRIEVAL, DENSE):
        slots = np.nonzero(lay.cls == c)[0]
        if len(slots):
            slot = int(rng.choice(slots))
            rows.add(slot * lay.n_seq + int(rng.integers(0, lay.n_seq)))
    _compare(lay, free, rows=sorted(rows))


def test_hand_fixture_and_block_walkthrough(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "tiny_tables_by_hand.json")))
    ret = {tuple(int(x) for x in k.split(",")): v for k, v in g["ret_lists"].items()}
    lay = custom_layout(seg_lens=[g["seg_lens"]], offline=[g["offline"]], n_prefill=g["n_prefill"],
                        n_decode=g["n_decode"], classes=[tuple(c) for c in g["classes"]],
                        page_size=g["page_size"], ret_lists=ret)
    for call in ("prefill", "decode"):
        t = _lib_tables(lay, call, np.asarray(g["free_list"]))
        assert t["storage"].tolist() == g["expected_storage"]
        rows = [t["entries"][t["row_ptr"][r]:t["row_ptr"][r + 1], :3].tolist() for r in range(4)]
        assert rows == g[f"expected_{call}_rows"]
        assert t["reloc"][:, :3].tolist() == sorted(g["expected_reloc"])
    w = json.load(open(os.path.join(golden_dir, "paged_block_walkthrough.json")))
    lay = custom_layout(seg_lens=[[]], offline=[[]], n_prefill=w["prompt_tokens"], n_decode=w["generated_tokens"],
                        classes=[(GLOBAL, 0)], page_size=w["page_size"])
    a = lay.abi_arrays("decode")
    a["q_lo"] = a["q_hi"] = np.array([8], np.int32)   # the second generated token
    t = sp.build_tables(**a, page_size=w["page_size"], free_list=np.asarray(w["free_list"]))
    assert t["storage"].tolist() == w["expected_block_table"]
    assert t["entries"][:, 0].tolist() == w["expected_block_table"]
    assert sorted(w["free_list"][len(t["storage"]):]) == w["expected_unused_blocks"]


def _base_tiny():
    lay = custom_layout(seg_lens=[[10, 5]], offline=[[0, 0]], n_prefill=4, n_decode=1,
                        classes=[(GLOBAL, 0), (LOCAL, 3), (RETRIEVAL, 0)], page_size=4,
                        ret_lists={(2, 0): [0, 3]})
    return lay, lay.abi_arrays("prefill")


def _expect(code, **kw):
    lay, a = _base_tiny()
    free = kw.pop("free_list", np.arange(100, dtype=np.int32))
    a.update(kw)
    with pytest.raises(sp.SegPagedError) as e:
        sp.build_tables(**a, page_size=kw.pop("page_size", 4) if "page_size" in kw else 4, free_list=free)
    assert e.value.status == code


def test_error_codes():
    lay, a = _base_tiny()
    n = sp.build_tables(**a, page_size=4, free_list=None, counts_only=True)["counts"][0]
    _expect(sp.SP_ENOMEM, free_list=np.arange(n - 1, dtype=np.int32))
    _expect(sp.SP_EINVAL, free_list=np.array([0] + list(range(n)), np.int32))          # repeated page id
    _expect(sp.SP_EINVAL, free_list=np.array([-1] + list(range(n)), np.int32))         # negative page id
    _expect(sp.SP_EINVAL, cls=np.array([0, 7, 2], np.int32))                           # unknown class
    _expect(sp.SP_EINVAL, window=np.array([0, 0, 0], np.int32))                        # local window 0
    _expect(sp.SP_EINVAL, ret_pages=np.array([3, 0], np.int32))                        # not ascending
    _expect(sp.SP_EINVAL, ret_pages=np.array([0, 5], np.int32))                        # beyond the segment pages
    _expect(sp.SP_EINVAL, q_lo=np.array([14], np.int32))                               # query inside a segment
    _expect(sp.SP_EINVAL, q_hi=np.array([20], np.int32))                               # beyond the new tokens
    _expect(sp.SP_EINVAL, segs=np.array([[10, 0, 0], [5, 3, 0]], np.int32))           # overlapping segments
    _expect(sp.SP_EINVAL, segs=np.array([[10, 0, 0], [5, 2**31 - 3, 0]], np.int32))   # position overflow
    _expect(sp.SP_EINVAL, n_new=np.array([0], np.int32))
    with pytest.raises(sp.SegPagedError) as e:
        sp.build_tables(**a, page_size=0, free_list=np.arange(100, dtype=np.int32))
    assert e.value.status == sp.SP_EINVAL


def test_workspace_query_and_validation():
    rp = np.array([0, 3, 5], np.int32)
    b = sp.workspace_bytes(sp.SP_WS_DECODE, sp.SP_BF16, 128, 16, 4, 1, 2, None, rp)
    assert b >= 256 and b % 256 == 0
    with pytest.raises(sp.SegPagedError) as e:
        sp.workspace_bytes(sp.SP_WS_DECODE, sp.SP_BF16, 96, 16, 4, 1, 2, None, rp)
    assert e.value.status == sp.SP_EUNSUPPORTED
    with pytest.raises(sp.SegPagedError) as e:
        sp.workspace_bytes(sp.SP_WS_DECODE, sp.SP_BF16, 128, 16, 4, 1, 2, None, np.array([0, 3, 3], np.int32))
    assert e.value.status == sp.SP_EINVAL


def test_workspace_query_limits():
    # a decode row longer than one call's split capacity (1024 splits of at
    # most 512 pages), and a query group beyond 16 heads
    rp = np.array([0, 1024 * 512 + 1], np.int32)
    with pytest.raises(sp.SegPagedError) as e:
        sp.workspace_bytes(sp.SP_WS_DECODE, sp.SP_BF16, 128, 16, 4, 1, 1, None, rp)
    assert e.value.status == sp.SP_EUNSUPPORTED and "split capacity" in str(e.value)
    assert sp.workspace_bytes(sp.SP_WS_DECODE, sp.SP_BF16, 128, 16, 4, 1, 1, None,
                              np.array([0, 1024 * 512], np.int32)) > 0
    with pytest.raises(sp.SegPagedError) as e:
        sp.workspace_bytes(sp.SP_WS_DECODE, sp.SP_BF16, 128, 16, 17, 1, 1, None, np.array([0, 4], np.int32))
    assert e.value.status == sp.SP_EUNSUPPORTED


@pytest.mark.parametrize("seed", range(3))
def test_prefill_plan_does_not_depend_on_row_order(seed):
    # The planner scores rows of equal shape together: a permutation of the
    # rows of one sequence (same multiset of table lengths) must give the same
    # plan, hence the same workspace size, for any mix of lengths.
    r = np.random.default_rng(seed)
    for _ in range(40):
        n_slot = int(r.integers(2, 80))
        lens = r.choice(r.integers(1, 3000, size=int(r.integers(1, 6))), size=n_slot)
        tok = np.array([0, int(r.integers(1, 700))], np.int32)
        for ps in (16, 32):
            rp = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
            rq = np.concatenate([[0], np.cumsum(r.permutation(lens))]).astype(np.int32)
            a = sp.workspace_bytes(sp.SP_WS_PREFILL, sp.SP_BF16, 128, ps, 4, 1, n_slot, tok, rp)
            b = sp.workspace_bytes(sp.SP_WS_PREFILL, sp.SP_BF16, 128, ps, 4, 1, n_slot, tok, rq)
            assert a == b


@pytest.mark.parametrize("seed", range(4))
def test_bench_counts_from_host_tables_match_oracle(seed):
    """bench.py takes its FLOP and byte numerators from the host tables: the
    visible keys of each query counted from a row's entries and its class must
    equal the oracle's visible set sizes, for the prefill and the decode call."""
    import bench
    r = np.random.default_rng(50 + seed)
    ps = int(r.choice([1, 3, 4, 16]))
    n_seq = int(r.integers(1, 4))
    lens = [list(r.integers(1, 60, size=int(r.integers(0, 4)))) for _ in range(n_seq)]
    off = [list(r.integers(-300, 300, size=len(l))) for l in lens]
    classes = [(GLOBAL, 0), (LOCAL, int(r.integers(1, 70))), (RETRIEVAL, 0), (DENSE, 0), (LOCAL, 1)]
    ret = {}
    for q in range(n_seq):
        nsp = sum(-(-l // ps) for l in lens[q])
        ret[(2, q)] = np.sort(r.choice(nsp, size=int(r.integers(0, nsp + 1)), replace=False))
    lay = custom_layout(seg_lens=lens, offline=off, n_prefill=int(r.integers(1, 30)), n_decode=1, classes=classes,
                        page_size=ps, ret_lists=ret)
    n = sp.build_tables(**lay.abi_arrays("prefill"), page_size=ps, free_list=None, counts_only=True)["counts"][0]
    free = np.arange(int(n), dtype=np.int32)
    for call, toks in (("prefill", np.arange(lay.n_prefill)), ("decode", np.asarray([lay.n_prefill]))):
        t = _lib_tables(lay, call, free)
        q_pos = [lay.new_base[q] + toks for q in range(n_seq)]
        got = bench.table_visible_counts(t["row_ptr"], t["entries"], lay.cls, lay.window, n_seq, q_pos)
        for row in range(lay.n_slot * n_seq):
            slot, q = divmod(row, n_seq)
            assert np.array_equal(got[row], otab.visible_counts(lay, slot, q, q_pos[q])), (call, row)


@pytest.mark.parametrize("seed", range(4))
def test_visible_sets_from_tables_equal_the_oracle(seed):
    """The per-query visible token set derived from a library table and the
    class predicate (a key of an entry (pos_start, n_valid) is seen by a query
    at p when its position is <= p and, for local(W), > p - W) equals the
    oracle's visible set, position for position, for every query of the
    prefill and the decode call."""
    r = np.random.default_rng(900 + seed)
    ps = int(r.choice([1, 2, 4, 16]))
    n_seq = int(r.integers(1, 3))
    lens = [list(r.integers(1, 50, size=int(r.integers(0, 4)))) for _ in range(n_seq)]
    off = [list(r.integers(-99, 99, size=len(l))) for l in lens]
    classes = [(GLOBAL, 0), (LOCAL, int(r.integers(1, 40))), (RETRIEVAL, 0), (DENSE, 0), (LOCAL, 1)]
    ret = {}
    for q in range(n_seq):
        nsp = sum(-(-l // ps) for l in lens[q])
        ret[(2, q)] = np.sort(r.choice(nsp, size=int(r.integers(0, nsp + 1)), replace=False))
    lay = custom_layout(seg_lens=lens, offline=off, n_prefill=int(r.integers(1, 20)), n_decode=1, classes=classes,
                        page_size=ps, ret_lists=ret)
    n = sp.build_tables(**lay.abi_arrays("prefill"), page_size=ps, free_list=None, counts_only=True)["counts"][0]
    free = np.random.default_rng(seed).permutation(int(n) + 3).astype(np.int32)
    for call, toks in (("prefill", np.arange(lay.n_prefill)), ("decode", np.asarray([lay.n_prefill]))):
        t = _lib_tables(lay, call, free)
        for row in range(lay.n_slot * n_seq):
            slot, q = divmod(row, n_seq)
            ent = t["entries"][t["row_ptr"][row]:t["row_ptr"][row + 1]]
            keys = np.concatenate([np.arange(e[1], e[1] + e[2]) for e in ent])
            tpos, _tp, tsp, tnew = otab.tokens(lay, q)
            listed = lay.ret_pages.get((slot, q), [])
            for p in lay.new_base[q] + toks:
                mine = keys[keys <= p]
                if lay.cls[slot] == LOCAL:
                    mine = mine[mine > p - lay.window[slot]]
                want = tpos[otab.visible(int(lay.cls[slot]), int(lay.window[slot]), listed, tpos, tsp, tnew, int(p))]
                assert np.array_equal(np.sort(mine), np.sort(want)), (call, row, int(p))


def test_host_calls_from_many_threads():
    """The host calls keep no shared state (the error text is per thread): the
    table builder and the workspace query run from 8 threads at once (ctypes
    releases the interpreter lock during each call) give the results of the
    same calls made one at a time, and a failing call in one thread leaves the
    other threads' error text alone."""
    import threading
    lay = synth.make_layout("16k")
    arr = lay.abi_arrays("prefill")
    n = sp.build_tables(**arr, page_size=lay.page_size, free_list=None, counts_only=True)["counts"][0]
    free = np.random.default_rng(3).permutation(int(n) + 11).astype(np.int32)
    want = sp.build_tables(**arr, page_size=lay.page_size, free_list=free)
    tok = np.arange(lay.n_seq + 1, dtype=np.int32) * lay.n_prefill
    ws_want = sp.workspace_bytes(sp.SP_WS_PREFILL, sp.SP_BF16, lay.head_dim, lay.page_size, lay.group, lay.n_seq,
                                 lay.n_slot, tok, want["row_ptr"])
    errors, bad = [], []

    def work(i):
        try:
            for _ in range(5):
                if i % 4 == 3:       # a failing call: its message must stay in this thread
                    with pytest.raises(sp.SegPagedError) as e:
                        sp.workspace_bytes(sp.SP_WS_DECODE, sp.SP_BF16, 96, 16, 4, 1, 1, None,
                                           np.array([0, 4], np.int32))
                    if "head_dim" not in str(e.value):
                        bad.append(str(e.value))
                    continue
                got = sp.build_tables(**arr, page_size=lay.page_size, free_list=free)
                for k in ("row_ptr", "entries", "reloc", "storage"):
                    if not np.array_equal(got[k], want[k]):
                        bad.append(k)
                ws = sp.workspace_bytes(sp.SP_WS_PREFILL, sp.SP_BF16, lay.head_dim, lay.page_size, lay.group,
                                        lay.n_seq, lay.n_slot, tok, got["row_ptr"])
                if ws != ws_want:
                    bad.append("workspace")
        except Exception as ex:      # surfaced below
            errors.append(repr(ex))

    threads = [threading.Thread(target=work, args=(i,)) for i in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    assert not bad, bad[:5]
