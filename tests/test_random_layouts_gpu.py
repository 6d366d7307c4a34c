"""Randomised layouts through the whole path on the GPU, against the fp64 oracle.

Each seed draws a small layout: 1-3 sequences (one of them possibly without a
reused segment), 0-3 segments of up to 600 tokens each at random offline
positions, 1-6 slots of random class (global, local with a random window,
retrieval with a random page list, dense), query group 1-8, head_dim 64 or
128, page size 16 or 32, and up to 90 new tokens; a second family takes
groups 3, 5, 6, 12 and 16, pages of up to 64 keys and up to 200 new tokens.  Relocation, prefill (every
row, every query token) and decode (every row) are compared with the oracle
at the same bounds as the fixed-layout tests.  Every draw is seeded, so a
failure names a reproducible case.
"""
import numpy as np
import pytest

from synth import custom_layout, GLOBAL, LOCAL, RETRIEVAL, DENSE
from test_gpu_parity import _wl, check_prefill, check_decode, check_relocate

pytestmark = pytest.mark.gpu


def _draw(seed, wide=False):
    """wide: query groups that do not divide a wave's 32 rows (3, 5, 6, 12) and
    group 16, pages of 16, 32 or 64 keys, and up to 200 new tokens (several
    query tiles per row)."""
    r = np.random.default_rng((5000 if wide else 1000) + seed)
    n_seq = int(r.integers(1, 4))
    ps = int(r.choice([16, 32, 64] if wide else [16, 32]))
    D = int(r.choice([64, 128]))
    G = int(r.choice([3, 5, 6, 12, 16] if wide else [1, 2, 4, 8]))
    seg_lens, offline = [], []
    for q in range(n_seq):
        n_segs = int(r.integers(1, 4))
        if q == n_seq - 1 and n_seq > 1 and seed % 3 == 1:
            n_segs = 0                                 # a sequence with no reused segment
        lens = [int(x) for x in r.integers(1, 601, size=n_segs)]
        seg_lens.append(lens)
        offline.append([int(x) for x in r.integers(-5000, 5000, size=n_segs)])
    n_slot = int(r.integers(1, 7))
    classes, ret = [], {}
    for slot in range(n_slot):
        c = int(r.choice([GLOBAL, LOCAL, RETRIEVAL, DENSE]))
        classes.append((c, int(r.integers(1, 600)) if c == LOCAL else 0))
        if c == RETRIEVAL:
            for q in range(n_seq):
                nsp = sum(-(-l // ps) for l in seg_lens[q])
                k = int(r.integers(0, nsp + 1)) if nsp else 0
                ret[(slot, q)] = np.sort(r.choice(nsp, size=k, replace=False)) if k else np.zeros(0, np.int64)
    n_prefill = int(r.integers(1, 201 if wide else 91))
    return custom_layout(seg_lens=seg_lens, offline=offline, n_prefill=n_prefill, n_decode=1, classes=classes,
                         page_size=ps, head_dim=D, group=G, dtype="bf16", ret_lists=ret,
                         name=f"random{'_wide' if wide else ''}{seed}", seed=seed)


@pytest.mark.parametrize("seed", range(24))
def test_random_layout_whole_path(seed):
    lay = _draw(seed)
    w = _wl(lay)
    w.relocate()
    check_relocate(w)
    w.prefill()
    check_prefill(w)
    w.decode()
    check_decode(w)


@pytest.mark.parametrize("seed", range(16))
def test_random_layout_wide_groups(seed):
    """Groups 3, 5, 6, 12 and 16, pages up to 64 keys, several query tiles per
    row; decode where it takes the page size (16 or 32)."""
    lay = _draw(seed, wide=True)
    w = _wl(lay)
    w.relocate()
    check_relocate(w)
    w.prefill()
    check_prefill(w)
    if lay.page_size in (16, 32):
        w.decode()
        check_decode(w)
