"""ctypes binding of libsegpaged.so - argument marshalling only.

Every call maps one-to-one onto an ``extern "C"`` entry point declared in
``include/segpaged.h``; all work happens in the library (host table builder)
and its HIP kernels.  Device arguments are torch tensors on the GPU (torch only
supplies device memory and the current stream).  If the library has not been
built this module raises at import of the library, it never falls back.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

# SEGPAGED_LIB overrides the library path (for instance a build with the host
# code instrumented by AddressSanitizer).
_LIB_PATH = os.environ.get("SEGPAGED_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib",
                                                           "libsegpaged.so")

SP_OK, SP_EINVAL, SP_ENOMEM, SP_EHIP, SP_EUNSUPPORTED, SP_EWORKSPACE = 0, -1, -2, -3, -4, -5
SP_GLOBAL, SP_LOCAL, SP_RETRIEVAL, SP_DENSE = 0, 1, 2, 3
SP_F32, SP_BF16 = 0, 1
SP_WS_PREFILL, SP_WS_DECODE, SP_WS_IMPORTANCE = 0, 1, 2
SP_STATIC_SCRATCH_BYTES = 16 << 20

ENTRY_FIELDS = 4   # sp_entry / sp_reloc are 4 x int32


class Layout(ctypes.Structure):
    """sp_layout: the host calls' shared layout arguments (pointers into numpy arrays the caller keeps alive)."""
    _fields_ = [("n_seq", ctypes.c_int), ("seg_ptr", ctypes.c_void_p), ("segs", ctypes.c_void_p),
                ("n_new", ctypes.c_void_p), ("n_slot", ctypes.c_int), ("cls", ctypes.c_void_p),
                ("window", ctypes.c_void_p), ("ret_ptr", ctypes.c_void_p), ("ret_pages", ctypes.c_void_p),
                ("page_size", ctypes.c_int)]


class SegPagedError(RuntimeError):
    def __init__(self, status: int, call: str, msg: str):
        super().__init__(f"{call} failed: status {status} ({msg})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"libsegpaged.so not built at {_LIB_PATH}; run head_aware_paged_page_amd/build.py")
        L = ctypes.CDLL(_LIB_PATH)
        P, I, I64, D, F, SZ = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double, ctypes.c_float,
                               ctypes.c_size_t)
        L.segpaged_build_tables.argtypes = [I, P, P, P, P, P, I, P, P, P, P, I, I64, P, P, P, P, P, P, P]
        L.segpaged_build_tables_ex.argtypes = [P, P, P, P, I64, P, P, P, P, P, P, P]
        L.segpaged_tables_from_chains.argtypes = [P, P, P, P, P, P, P, P]
        L.segpaged_release_pages.argtypes = [P, P, P, P, P, P]
        L.rope_relocate.argtypes = [P, P, I, I, I, I64, I, P, D, P]
        L.segpaged_workspace_bytes.argtypes = [I, I, I, I, I, I, I, P, P, ctypes.POINTER(SZ)]
        L.segpaged_prefill.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, P, I64, F, P, P, P, SZ, P]
        L.segpaged_decode.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, I64, F, P, P, P, SZ, P]
        L.segpaged_decode_static.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, I64, F, P, P, P]
        L.segpaged_token_importance.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, I64, F, P, P, P, P,
                                                P, SZ, P]
        L.segpaged_select_tokens.argtypes = [I, I, I, P, P, P, P, P, P, P, P]
        L.segpaged_pack_pages.argtypes = [I, I, I, I64, P, P, P, I64, P, P, P]
        L.segpaged_unpack_pages.argtypes = [I, I, I, I64, P, P, P, P, P, I64, P]
        L.segpaged_strerror.restype = ctypes.c_char_p
        L.segpaged_strerror.argtypes = [I]
        L.segpaged_last_error.restype = ctypes.c_char_p
        L.segpaged_last_error.argtypes = []
        L.segpaged_version.restype = I
        for fn in ("segpaged_build_tables", "segpaged_build_tables_ex", "segpaged_tables_from_chains",
                   "segpaged_release_pages", "rope_relocate", "segpaged_workspace_bytes", "segpaged_prefill",
                   "segpaged_decode", "segpaged_decode_static", "segpaged_pack_pages", "segpaged_unpack_pages",
                   "segpaged_token_importance", "segpaged_select_tokens"):
            getattr(L, fn).restype = I
        _lib = L
    return _lib


def _check(rc: int, call: str):
    if rc != SP_OK:
        L = lib()
        msg = L.segpaged_last_error().decode() or L.segpaged_strerror(rc).decode()
        raise SegPagedError(rc, call, msg)


def _i32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.int32)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return SP_F32
    if t.dtype == torch.bfloat16:
        return SP_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


# --------------------------------------------------------------------------- host table builder

def build_tables(seg_ptr, segs, n_new, q_lo, q_hi, cls, window, ret_ptr, ret_pages, page_size, free_list,
                 counts_only=False):
    """segpaged_build_tables.  ``segs`` is [n_seg, 3] (len, online_base, offline_base).

    Returns dict(counts, chain_ptr, storage, row_ptr, entries [n, 4], reloc [n, 4]) as int32
    arrays (only ``counts`` when counts_only)."""
    L = lib()
    seg_ptr, segs, n_new, q_lo, q_hi = map(_i32, (seg_ptr, segs, n_new, q_lo, q_hi))
    cls, window, ret_ptr, ret_pages = map(_i32, (cls, window, ret_ptr, ret_pages))
    free_list = _i32(free_list)
    n_seq = len(n_new)
    n_slot = len(cls)
    counts = np.zeros(3, np.int64)
    n_free = 0 if free_list is None else len(free_list)
    args = [n_seq, _ptr(seg_ptr), _ptr(segs), _ptr(n_new), _ptr(q_lo), _ptr(q_hi), n_slot, _ptr(cls),
            _ptr(window), _ptr(ret_ptr), _ptr(ret_pages), page_size, n_free, _ptr(free_list)]
    rc = L.segpaged_build_tables(*args, None, None, None, None, None, _ptr(counts))
    _check(rc, "segpaged_build_tables")
    if counts_only:
        return dict(counts=counts)
    n_rows = n_slot * n_seq
    chain_ptr = np.zeros(n_rows + 1, np.int32)
    storage = np.zeros(max(1, counts[0]), np.int32)
    row_ptr = np.zeros(n_rows + 1, np.int32)
    entries = np.zeros((max(1, counts[1]), ENTRY_FIELDS), np.int32)
    reloc = np.zeros((max(1, counts[2]), ENTRY_FIELDS), np.int32)
    rc = L.segpaged_build_tables(*args, _ptr(chain_ptr), _ptr(storage), _ptr(row_ptr), _ptr(entries),
                                 _ptr(reloc), _ptr(counts))
    _check(rc, "segpaged_build_tables")
    return dict(counts=counts, chain_ptr=chain_ptr, storage=storage[: counts[0]], row_ptr=row_ptr,
                entries=entries[: counts[1]], reloc=reloc[: counts[2]])


def _layout(seg_ptr, segs, n_new, cls, window, ret_ptr, ret_pages, page_size):
    """(sp_layout, arrays it points into); keep the arrays alive while the layout is used."""
    arrs = [_i32(a) for a in (seg_ptr, segs, n_new, cls, window, ret_ptr, ret_pages)]
    seg_ptr, segs, n_new, cls, window, ret_ptr, ret_pages = arrs
    lay = Layout(len(n_new), _ptr(seg_ptr), _ptr(segs), _ptr(n_new), len(cls), _ptr(cls), _ptr(window),
                 _ptr(ret_ptr), _ptr(ret_pages), int(page_size))
    return lay, arrs


def build_tables_ex(seg_ptr, segs, n_new, q_lo, q_hi, cls, window, ret_ptr, ret_pages, page_size, free_list,
                    keep_from=None, counts_only=False):
    """segpaged_build_tables_ex: as build_tables, with window-only storage when
    keep_from is given (storage then holds -1 for pages not stored).  Returns
    dict(counts [4], chain_ptr, storage, row_ptr, entries [n, 4], reloc [n, 4])."""
    L = lib()
    lay, keep = _layout(seg_ptr, segs, n_new, cls, window, ret_ptr, ret_pages, page_size)
    q_lo, q_hi, keep_from, free_list = map(_i32, (q_lo, q_hi, keep_from, free_list))
    counts = np.zeros(4, np.int64)
    n_free = 0 if free_list is None else len(free_list)
    head = [ctypes.byref(lay), _ptr(q_lo), _ptr(q_hi), _ptr(keep_from), n_free, _ptr(free_list)]
    _check(L.segpaged_build_tables_ex(*head, None, None, None, None, None, _ptr(counts)), "segpaged_build_tables_ex")
    if counts_only:
        return dict(counts=counts)
    n_rows = lay.n_slot * lay.n_seq
    chain_ptr = np.zeros(n_rows + 1, np.int32)
    storage = np.zeros(max(1, counts[0]), np.int32)
    row_ptr = np.zeros(n_rows + 1, np.int32)
    entries = np.zeros((max(1, counts[1]), ENTRY_FIELDS), np.int32)
    reloc = np.zeros((max(1, counts[2]), ENTRY_FIELDS), np.int32)
    _check(L.segpaged_build_tables_ex(*head, _ptr(chain_ptr), _ptr(storage), _ptr(row_ptr), _ptr(entries),
                                      _ptr(reloc), _ptr(counts)), "segpaged_build_tables_ex")
    del keep
    return dict(counts=counts, chain_ptr=chain_ptr, storage=storage[: counts[0]], row_ptr=row_ptr,
                entries=entries[: counts[1]], reloc=reloc[: counts[2]])


def tables_from_chains(seg_ptr, segs, n_new, q_lo, q_hi, cls, window, ret_ptr, ret_pages, page_size, chain_ptr,
                       storage):
    """segpaged_tables_from_chains: (row_ptr, entries [n, 4]) of a call over existing chains."""
    L = lib()
    lay, keep = _layout(seg_ptr, segs, n_new, cls, window, ret_ptr, ret_pages, page_size)
    q_lo, q_hi, chain_ptr, storage = map(_i32, (q_lo, q_hi, chain_ptr, storage))
    n = ctypes.c_int64(0)
    head = [ctypes.byref(lay), _ptr(q_lo), _ptr(q_hi), _ptr(chain_ptr), _ptr(storage)]
    _check(L.segpaged_tables_from_chains(*head, None, None, ctypes.byref(n)), "segpaged_tables_from_chains")
    row_ptr = np.zeros(lay.n_slot * lay.n_seq + 1, np.int32)
    entries = np.zeros((max(1, n.value), ENTRY_FIELDS), np.int32)
    _check(L.segpaged_tables_from_chains(*head, _ptr(row_ptr), _ptr(entries), ctypes.byref(n)),
           "segpaged_tables_from_chains")
    del keep
    return row_ptr, entries[: n.value]


def release_pages(seg_ptr, segs, n_new, cls, window, ret_ptr, ret_pages, page_size, p_next, chain_ptr, storage):
    """segpaged_release_pages.  ``storage`` (int32 numpy) is updated in place;
    returns the released physical ids."""
    L = lib()
    lay, keep = _layout(seg_ptr, segs, n_new, cls, window, ret_ptr, ret_pages, page_size)
    p_next, chain_ptr = _i32(p_next), _i32(chain_ptr)
    assert storage.dtype == np.int32 and storage.flags.c_contiguous
    released = np.zeros(max(1, len(storage)), np.int32)
    n = ctypes.c_int64(0)
    _check(L.segpaged_release_pages(ctypes.byref(lay), _ptr(p_next), _ptr(chain_ptr), _ptr(storage), _ptr(released),
                                    ctypes.byref(n)), "segpaged_release_pages")
    del keep
    return released[: n.value]


# --------------------------------------------------------------------------- device calls

def rope_relocate(k_in, k_out, page_size: int, reloc_dev, theta: float, stream=None):
    """rope_relocate on K pools [n_phys, page_size, head_dim]; reloc_dev: int32 [n, 4] on the GPU."""
    n_phys, ps, D = k_in.shape
    assert ps == page_size and tuple(k_out.shape) == tuple(k_in.shape) and k_out.dtype == k_in.dtype
    n = reloc_dev.shape[0]
    rc = lib().rope_relocate(_dptr(k_in), _dptr(k_out), _dtype_code(k_in), page_size, D, n_phys, n,
                             _dptr(reloc_dev), float(theta), _stream(stream))
    _check(rc, "rope_relocate")


def workspace_bytes(kind: int, dtype: int, head_dim: int, page_size: int, group: int, n_seq: int, n_slot: int,
                    h_tok_ptr, h_row_ptr) -> int:
    out = ctypes.c_size_t(0)
    tp = _i32(h_tok_ptr)
    rp = _i32(h_row_ptr)
    rc = lib().segpaged_workspace_bytes(kind, dtype, head_dim, page_size, group, n_seq, n_slot, _ptr(tp), _ptr(rp),
                                        ctypes.byref(out))
    _check(rc, "segpaged_workspace_bytes")
    return out.value


def prefill(q, k_pool, v_pool, *, page_size, group, n_seq, n_slot, h_tok_ptr, h_row_ptr, d_tok_ptr, d_q_pos0,
            d_cls, d_window, d_row_ptr, d_entries, scale, out, lse, workspace, stream=None):
    """segpaged_prefill.  q/out [n_tok, n_slot*group, D]; pools [n_phys, ps, D] (K) and [n_phys, D, ps] (V)."""
    D = q.shape[-1]
    tp = _i32(h_tok_ptr)
    rp = _i32(h_row_ptr)
    rc = lib().segpaged_prefill(_dtype_code(q), D, page_size, group, n_seq, n_slot, _ptr(tp), _ptr(rp),
                                _dptr(d_tok_ptr), _dptr(d_q_pos0), _dptr(d_cls), _dptr(d_window), _dptr(d_row_ptr),
                                _dptr(d_entries), _dptr(q), _dptr(k_pool), _dptr(v_pool), k_pool.shape[0],
                                float(scale), _dptr(out), _dptr(lse), _dptr(workspace), workspace.numel(),
                                _stream(stream))
    _check(rc, "segpaged_prefill")


def decode(q, k_pool, v_pool, *, page_size, group, n_seq, n_slot, h_row_ptr, d_q_pos, d_cls, d_window, d_row_ptr,
           d_entries, scale, out, lse, workspace, stream=None):
    """segpaged_decode.  q/out [n_seq, n_slot*group, D]."""
    D = q.shape[-1]
    rp = _i32(h_row_ptr)
    rc = lib().segpaged_decode(_dtype_code(q), D, page_size, group, n_seq, n_slot, _ptr(rp), _dptr(d_q_pos),
                               _dptr(d_cls), _dptr(d_window), _dptr(d_row_ptr), _dptr(d_entries), _dptr(q),
                               _dptr(k_pool), _dptr(v_pool), k_pool.shape[0], float(scale), _dptr(out), _dptr(lse),
                               _dptr(workspace), workspace.numel(), _stream(stream))
    _check(rc, "segpaged_decode")


def decode_static(q, k_pool, v_pool, *, page_size, group, n_seq, n_slot, h_row_ptr, d_q_pos, d_cls, d_window,
                  d_row_ptr, d_entries, scale, out, lse, stream=None):
    """segpaged_decode_static: segpaged_decode with the library's static scratch (no workspace)."""
    D = q.shape[-1]
    rp = _i32(h_row_ptr)
    rc = lib().segpaged_decode_static(_dtype_code(q), D, page_size, group, n_seq, n_slot, _ptr(rp),
                                      _dptr(d_q_pos), _dptr(d_cls), _dptr(d_window), _dptr(d_row_ptr),
                                      _dptr(d_entries), _dptr(q), _dptr(k_pool), _dptr(v_pool), k_pool.shape[0],
                                      float(scale), _dptr(out), _dptr(lse), _stream(stream))
    _check(rc, "segpaged_decode_static")


def token_importance(q, k_pool, *, page_size, group, n_seq, n_slot, h_tok_ptr, h_row_ptr, d_tok_ptr, d_q_pos0,
                     d_cls, d_window, d_row_ptr, d_entries, scale, lse, h_pos_ptr, d_pos_ptr, imp, workspace,
                     stream=None):
    """segpaged_token_importance.  imp: fp32 [n_slot, h_pos_ptr[-1]] (written); lse from segpaged_prefill."""
    D = q.shape[-1]
    tp, rp, pp = _i32(h_tok_ptr), _i32(h_row_ptr), _i32(h_pos_ptr)
    rc = lib().segpaged_token_importance(_dtype_code(q), D, page_size, group, n_seq, n_slot, _ptr(tp), _ptr(rp),
                                         _dptr(d_tok_ptr), _dptr(d_q_pos0), _dptr(d_cls), _dptr(d_window),
                                         _dptr(d_row_ptr), _dptr(d_entries), _dptr(q), _dptr(k_pool),
                                         k_pool.shape[0], float(scale), _dptr(lse), _ptr(pp), _dptr(d_pos_ptr),
                                         _dptr(imp), _dptr(workspace), workspace.numel(), _stream(stream))
    _check(rc, "segpaged_token_importance")


def select_tokens(imp, *, n_layers, slots_per_layer, n_seq, h_pos_ptr, d_pos_ptr, h_sel_ptr, d_sel_ptr, score, sel,
                  stream=None):
    """segpaged_select_tokens.  score fp32 [n_layers, h_pos_ptr[-1]], sel int32 [n_layers, h_sel_ptr[-1]] (written)."""
    pp, sp_ = _i32(h_pos_ptr), _i32(h_sel_ptr)
    rc = lib().segpaged_select_tokens(n_layers, slots_per_layer, n_seq, _ptr(pp), _dptr(d_pos_ptr), _dptr(imp),
                                      _ptr(sp_), _dptr(d_sel_ptr), _dptr(score), _dptr(sel), _stream(stream))
    _check(rc, "segpaged_select_tokens")


def pack_pages(k_pool, v_pool, d_entries, n_entries: int, k_out, v_out, stream=None):
    """segpaged_pack_pages.  Pools [n_phys, ps, D] (K) and [n_phys, D, ps] (V); outputs [n_entries, ...] alike."""
    D = k_pool.shape[-1]
    rc = lib().segpaged_pack_pages(_dtype_code(k_pool), D, k_pool.shape[1], int(n_entries), _dptr(d_entries),
                                   _dptr(k_pool), _dptr(v_pool), k_pool.shape[0], _dptr(k_out), _dptr(v_out),
                                   _stream(stream))
    _check(rc, "segpaged_pack_pages")


def unpack_pages(k_in, v_in, d_entries, n_entries: int, k_pool, v_pool, stream=None):
    """segpaged_unpack_pages: packed page e back to pool page d_entries[e].phys."""
    D = k_pool.shape[-1]
    rc = lib().segpaged_unpack_pages(_dtype_code(k_pool), D, k_pool.shape[1], int(n_entries), _dptr(d_entries),
                                     _dptr(k_in), _dptr(v_in), _dptr(k_pool), _dptr(v_pool), k_pool.shape[0],
                                     _stream(stream))
    _check(rc, "segpaged_unpack_pages")


def version() -> int:
    return lib().segpaged_version()
