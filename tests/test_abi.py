"""The C-ABI library loads, exports what include/calibatt.h declares, and rejects
bad arguments on the host before anything is enqueued (CPU only).

Every call below is invalid by construction, so it returns before any HIP
call: device pointers are placeholders that are never dereferenced.
"""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "calibatt.h")

cal = pytest.importorskip("calibrated_block_sparse_skiplist_amd._lib")
lib = cal.lib
INVALID = cal.ERR_INVALID_ARG
P = 0x1000   # placeholder device address; never dereferenced by a rejected call


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(calibatt_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert set(names) == set(cal.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value


def test_version_and_error_string():
    assert lib.calibatt_version() == 100
    assert isinstance(lib.calibatt_last_error(), bytes)


def _view(T=1, L=1, H=2, N=1000, B=128, nb=8):
    return cal.SkipListView(T, L, H, N, B, nb, P, P, None)


def _sparse(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=None, H=2, N=1000, d=128, dtype=cal.BF16, scale=0.088,
             view=_view(), t=0, l=0, heads=None, nh=0)
    a.update(kw)
    return lib.calibatt_block_sparse_attn(a["q"], a["k"], a["v"], a["o"], a["lse"], a["H"], a["N"], a["d"],
                                          a["dtype"], a["scale"], ctypes.byref(a["view"]) if a["view"] else None,
                                          a["t"], a["l"], a["heads"], a["nh"], None)


@pytest.mark.parametrize("kw,msg", [
    (dict(q=None), "non-NULL"),
    (dict(d=96), "d = 96"),
    (dict(dtype=7), "dtype"),
    (dict(scale=0.0), "scale"),
    (dict(scale=float("nan")), "scale"),
    (dict(H=3), "skip list is for"),
    (dict(view=None), "NULL"),
    (dict(view=_view(B=32, nb=32)), "block size"),
    (dict(view=_view(nb=9)), "nb"),
    (dict(t=1), "outside the dictionary"),
    (dict(l=-1), "outside the dictionary"),
])
def test_block_sparse_rejects(kw, msg):
    assert _sparse(**kw) == INVALID
    assert msg in cal.last_error()


def test_block_sparse_rejects_bad_heads():
    bad = np.array([0, 2], dtype=np.int32)
    assert _sparse(heads=bad.ctypes.data, nh=2) == INVALID
    assert "out of range" in cal.last_error()
    dup = np.array([1, 1], dtype=np.int32)
    assert _sparse(heads=dup.ctypes.data, nh=2) == INVALID
    assert "twice" in cal.last_error()


def _anchor(N=600, F=3, R=10, C=20, anchors=(2, 7), d=64, dtype=cal.BF16):
    arr = np.array(anchors, dtype=np.int32)
    return lib.calibatt_anchor_attn(P, P, P, P, None, 1, N, d, dtype, 0.125, F, R, C,
                                    arr.ctypes.data if len(arr) else None, len(arr), None, 0, None)


@pytest.mark.parametrize("kw,msg", [
    (dict(N=601), "F*R*C"),
    (dict(anchors=(7, 2)), "ascending"),
    (dict(anchors=(2, 2)), "ascending"),
    (dict(anchors=(2, 10)), "outside"),
    (dict(anchors=()), "anchor"),
    (dict(d=32), "d = 32"),
])
def test_anchor_rejects(kw, msg):
    assert _anchor(**kw) == INVALID
    assert msg in cal.last_error()


def test_dispatch_rejects_missing_flags_and_bad_anchors():
    view = _view()
    st = lib.calibatt_layer_dispatch(P, P, P, P, None, 2, 1000, 128, cal.BF16, 0.088, ctypes.byref(view), 0, 0,
                                     None, 10, 10, 10, None, 0, None)
    assert st == INVALID and "rep_flags" in cal.last_error()
    flags = np.array([[[0, 1]]], dtype=np.uint8)
    anchors = np.array([3], dtype=np.int32)
    st = lib.calibatt_layer_dispatch(P, P, P, P, None, 2, 1000, 128, cal.BF16, 0.088, ctypes.byref(view), 0, 0,
                                     flags.ctypes.data, 10, 10, 11, anchors.ctypes.data, 1, None)
    assert st == INVALID and "F*R*C" in cal.last_error()


def test_compile_rejects():
    nnz = ctypes.c_int64(-1)
    assert lib.calibatt_compile_skiplist(None, 1, 1, 1, 100, 10, P, None, 0, None, ctypes.byref(nnz), None) == INVALID
    assert lib.calibatt_compile_skiplist(P, 1, 0, 1, 100, 10, P, None, 0, None, ctypes.byref(nnz), None) == INVALID
    assert lib.calibatt_compile_skiplist(P, 1, 1, 1, 10**6, 1, P, None, 0, None, ctypes.byref(nnz), None) == INVALID
    assert "exceeds" in cal.last_error()
    assert lib.calibatt_compile_skiplist(P, 1, 1, 1, 100, 10, P, P, -1, None, ctypes.byref(nnz), None) == INVALID
    assert lib.calibatt_compile_skiplist(P, 1, 1, 1, 100, 10, P, None, 0, None, None, None) == INVALID


def _iv_view(T=1, L=1, H=2, N=1000, B=128, nb=8, iv_ptr=P, iv=P):
    return cal.IntervalListView(T, L, H, N, B, nb, iv_ptr, iv, None)


@pytest.mark.parametrize("view,msg", [
    (None, "NULL"),
    (_iv_view(iv=None), "iv_ptr/iv"),
    (_iv_view(iv_ptr=None), "iv_ptr/iv"),
    (_iv_view(H=3), "skip list is for"),
    (_iv_view(B=96, nb=11), "block size"),
    (_iv_view(nb=7), "nb"),
    (_iv_view(T=0), "T and L"),
])
def test_interval_attention_rejects(view, msg):
    ref = ctypes.byref(view) if view is not None else None
    st = lib.calibatt_block_sparse_attn_iv(P, P, P, P, None, 2, 1000, 128, cal.BF16, 0.088, ref, 0, 0,
                                           None, 0, None)
    assert st == INVALID and msg in cal.last_error()
    flags = np.zeros((max(view.T, 1) if view else 1, 1, 2), dtype=np.uint8) if view else None
    st = lib.calibatt_layer_dispatch_iv(P, P, P, P, None, 2, 1000, 128, cal.BF16, 0.088, ref, 0, 0,
                                        flags.ctypes.data if flags is not None else None, 10, 10, 10, None, 0,
                                        None)
    assert st == INVALID and msg in cal.last_error()


def test_interval_dispatch_rejects_missing_flags():
    view = _iv_view()
    st = lib.calibatt_layer_dispatch_iv(P, P, P, P, None, 2, 1000, 128, cal.BF16, 0.088, ctypes.byref(view), 0,
                                        0, None, 10, 10, 10, None, 0, None)
    assert st == INVALID and "rep_flags" in cal.last_error()


def test_compile_intervals_rejects():
    n = ctypes.c_int64(-1)
    f = lib.calibatt_compile_intervals
    assert f(None, 1, 1, 1, 100, 10, P, None, 0, None, ctypes.byref(n), None) == INVALID
    assert f(P, 0, 1, 1, 100, 10, P, None, 0, None, ctypes.byref(n), None) == INVALID
    assert f(P, 1, 1, 1, 10**6, 1, P, None, 0, None, ctypes.byref(n), None) == INVALID
    assert "exceeds" in cal.last_error()
    assert f(P, 1, 1, 1, 100, 10, P, P, -1, None, ctypes.byref(n), None) == INVALID
    assert f(P, 1, 1, 1, 100, 10, None, None, 0, None, ctypes.byref(n), None) == INVALID


@pytest.mark.parametrize("kw,msg", [
    (dict(q=None), "non-NULL"), (dict(energy=None), "non-NULL"), (dict(d=32), "d = 32"), (dict(B=96), "block size"),
    (dict(scale=-1.0), "scale"), (dict(N=4097 * 64, B=64), "nb exceeds"), (dict(dtype=5), "dtype"),
])
def test_block_energy_rejects(kw, msg):
    a = dict(q=P, k=P, H=2, N=1000, d=128, dtype=cal.BF16, scale=0.088, B=128, energy=P)
    a.update(kw)
    st = lib.calibatt_block_energy(a["q"], a["k"], a["H"], a["N"], a["d"], a["dtype"], a["scale"], a["B"],
                                   a["energy"], None, 0, None, 0, None)
    assert st == INVALID and msg in cal.last_error()
    bad = np.array([2], dtype=np.int32)
    assert lib.calibatt_block_energy(P, P, 2, 1000, 128, cal.BF16, 0.088, 128, P, bad.ctypes.data, 1, None, 0,
                                     None) == INVALID


def test_block_energy_workspace_rejects():
    need = cal.energy_work_bytes(1000, 128)                # 8 * 8 * 128 floats for one head
    assert need == 8 * 8 * 128 * 4
    f = lib.calibatt_block_energy
    assert f(P, P, 2, 1000, 128, cal.BF16, 0.088, 128, P, None, 0, P, need - 4, None) == INVALID
    assert "work_bytes" in cal.last_error()
    assert f(P, P, 2, 1000, 128, cal.BF16, 0.088, 128, P, None, 0, P + 4, need, None) == INVALID
    assert "aligned" in cal.last_error()


@pytest.mark.parametrize("args,msg", [
    ((None, 4, 8, 0.5, P, None), "energy"), ((P, 4, 8, 0.5, None, None), "both NULL"), ((P, -1, 8, 0.5, P, None), "rows"),
    ((P, 4, 0, 0.5, P, None), "nb"), ((P, 4, 4097, 0.5, P, None), "nb"), ((P, 4, 8, 1.5, P, None), "tau"),
    ((P, 4, 8, float("nan"), P, None), "tau"), ((P, 4, 8, -0.1, None, P), "tau"),
])
def test_select_blocks_rejects(args, msg):
    assert lib.calibatt_select_blocks(*args, None) == INVALID and msg in cal.last_error()


@pytest.mark.parametrize("args,msg", [
    ((None, 4, 64, 0.5, P), "non-NULL"), ((P, 4, 64, 0.5, None), "non-NULL"), ((P, -1, 64, 0.5, P), "n must"),
    ((P, 4, 0, 0.5, P), "n_prompts"), ((P, 4, 64, 1.01, P), "rho"), ((P, 4, 64, float("inf"), P), "rho"),
])
def test_keep_frequency_rejects(args, msg):
    assert lib.calibatt_keep_frequency(*args, None) == INVALID and msg in cal.last_error()


def test_spatial_similarity_rejects():
    anchors = np.array([2, 7], dtype=np.int32)
    f = lib.calibatt_spatial_similarity
    def call(**kw):
        a = dict(q=P, k=P, H=1, N=600, d=64, dtype=cal.BF16, scale=0.125, F=3, R=10, C=20,
                 anchors=anchors.ctypes.data, ka=2, sim=P)
        a.update(kw)
        return f(a["q"], a["k"], a["H"], a["N"], a["d"], a["dtype"], a["scale"], a["F"], a["R"], a["C"],
                 a["anchors"], a["ka"], a["sim"], None, 0, None)
    assert call(sim=None) == INVALID
    assert call(q=None) == INVALID
    unsorted = np.array([7, 2], dtype=np.int32)
    assert call(anchors=unsorted.ctypes.data) == INVALID and "ascending" in cal.last_error()
    assert call(N=601) == INVALID and "F*R*C" in cal.last_error()
    assert call(d=32) == INVALID
    every = np.arange(10, dtype=np.int32)
    assert call(anchors=every.ctypes.data, ka=10) == INVALID and "every row" in cal.last_error()


def test_repetition_flags_rejects():
    anchors = np.array([1], dtype=np.int32)
    f = lib.calibatt_repetition_flags
    assert f(None, 1, 1, 1, 4, anchors.ctypes.data, 1, 0.87, P, None, None) == INVALID
    assert f(P, 1, 1, 1, 4, anchors.ctypes.data, 1, 0.87, None, None, None) == INVALID
    assert f(P, 0, 1, 1, 4, anchors.ctypes.data, 1, 0.87, P, None, None) == INVALID
    assert f(P, 1, 1, 1, 1, anchors.ctypes.data, 1, 0.87, P, None, None) == INVALID
    bad = np.array([3, 1], dtype=np.int32)
    assert f(P, 1, 1, 1, 4, bad.ctypes.data, 2, 0.87, P, None, None) == INVALID
    assert f(P, 1, 1, 1, 4, anchors.ctypes.data, 1, float("nan"), P, None, None) == INVALID


def test_product_path_does_not_import_the_oracle():
    import sys
    pkg = os.path.join(ROOT, "calibrated_block_sparse_skiplist_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"\boracle\b", src.replace("the oracle", "")), f


# ---------------------------------------------------------------------------
# Checked mode: host-side validation of list views (host arrays: no HIP call)
# ---------------------------------------------------------------------------
def _host_lists(T=2, L=2, H=3, N=1000, B=128, p=0.4, seed=0):
    import oracle
    nb = -(-N // B)
    rng = np.random.default_rng(seed)
    masks = (rng.random((T, L, H, nb, nb)) < p).astype(np.uint8)
    masks[0, 0, 1, 2] = 0                      # an empty row
    rp, ci, order = oracle.compile_skiplist(masks)
    iv_ptr, iv, _ = oracle.compile_intervals(masks)
    packed = (iv[:, 0].astype(np.int64) | (iv[:, 1].astype(np.int64) << 16)).astype(np.uint32)
    return dict(T=T, L=L, H=H, N=N, B=B, nb=nb, rp=rp.astype(np.int64), ci=ci.astype(np.int32),
                order=order.astype(np.int32), iv_ptr=iv_ptr.astype(np.int64), iv=packed)


def _validate_csr(d, rp=None, ci=None, order="keep", t=-1, l=-1):
    rp = d["rp"] if rp is None else rp
    ci = d["ci"] if ci is None else ci
    order = d["order"] if isinstance(order, str) else order
    view = cal.SkipListView(d["T"], d["L"], d["H"], d["N"], d["B"], d["nb"], rp.ctypes.data,
                            ci.ctypes.data if ci.size else P, order.ctypes.data if order is not None else None)
    return lib.calibatt_validate_skiplist(ctypes.byref(view), t, l, 1, None)


def _validate_runs(d, ptr=None, iv=None, t=-1, l=-1):
    ptr = d["iv_ptr"] if ptr is None else ptr
    iv = d["iv"] if iv is None else iv
    view = cal.IntervalListView(d["T"], d["L"], d["H"], d["N"], d["B"], d["nb"], ptr.ctypes.data,
                                iv.ctypes.data, d["order"].ctypes.data)
    return lib.calibatt_validate_intervals(ctypes.byref(view), t, l, 1, None)


def test_validate_accepts_compiled_lists():
    d = _host_lists()
    assert _validate_csr(d) == cal.OK, cal.last_error()
    assert _validate_csr(d, order=None) == cal.OK
    assert _validate_runs(d) == cal.OK, cal.last_error()
    for t in range(d["T"]):
        for l in range(d["L"]):
            assert _validate_csr(d, t=t, l=l) == cal.OK
            assert _validate_runs(d, t=t, l=l) == cal.OK


def _row_with(d, ptr_key, min_len):
    ptr = d[ptr_key]
    lens = np.diff(ptr)
    return int(np.flatnonzero(lens >= min_len)[0])


@pytest.mark.parametrize("case", ["out_of_range", "negative", "descending", "duplicate", "row_ptr_down",
                                  "row_ptr_start", "order_repeat", "order_range"])
def test_validate_rejects_bad_index_lists(case):
    d = _host_lists()
    rp, ci, order = d["rp"].copy(), d["ci"].copy(), d["order"].copy()
    row = _row_with(d, "rp", 2)
    j = int(rp[row])
    if case == "out_of_range":
        ci[j + 1] = d["nb"]
    elif case == "negative":
        ci[j] = -1
    elif case == "descending":
        ci[j], ci[j + 1] = ci[j + 1], ci[j]
    elif case == "duplicate":
        ci[j + 1] = ci[j]
    elif case == "row_ptr_down":
        rp[row + 1] = rp[row] - 1
    elif case == "row_ptr_start":
        rp[:] += 1
    elif case == "order_repeat":
        order[1] = order[0]
    else:
        order[5] = d["nb"]
    assert _validate_csr(d, rp=rp, ci=ci, order=order) == INVALID
    assert cal.last_error()
    # the record holding the bad row is rejected, a record before it is not (where there is one)
    rec = row // d["nb"] if case not in ("order_repeat", "order_range", "row_ptr_start") else 0
    t, l = divmod(rec // d["H"], d["L"])
    assert _validate_csr(d, rp=rp, ci=ci, order=order, t=t, l=l) == INVALID or case == "row_ptr_start"


@pytest.mark.parametrize("case", ["empty", "past_nb", "overlap", "adjacent", "descending", "too_many"])
def test_validate_rejects_bad_runs(case):
    d = _host_lists(p=0.3)
    ptr, iv = d["iv_ptr"].copy(), d["iv"].copy()
    row = _row_with(d, "iv_ptr", 2)
    j = int(ptr[row])
    lo0, hi0 = int(iv[j] & 0xffff), int(iv[j] >> 16)
    lo1, hi1 = int(iv[j + 1] & 0xffff), int(iv[j + 1] >> 16)
    pack = lambda lo, hi: np.uint32(lo | (hi << 16))
    if case == "empty":
        iv[j] = pack(lo0, lo0)
    elif case == "past_nb":
        iv[j + 1] = pack(lo1, d["nb"] + 1)
    elif case == "overlap":
        iv[j + 1] = pack(hi0 - 1, hi1)
    elif case == "adjacent":
        iv[j + 1] = pack(hi0, hi1)
    elif case == "descending":
        iv[j], iv[j + 1] = iv[j + 1], iv[j]
    else:
        # every block of a row as its own one-block run: more runs than ceil(nb/2)
        nb = d["nb"]
        new_ptr = ptr.copy()
        extra = nb - (ptr[row + 1] - ptr[row])
        new_ptr[row + 1:] += extra
        iv = np.concatenate([iv[:j], np.array([pack(c, c + 1) for c in range(nb)], np.uint32), iv[ptr[row + 1]:]])
        ptr = new_ptr
    assert _validate_runs(d, ptr=ptr, iv=iv) == INVALID
    assert cal.last_error()


def test_validate_rejects_bad_view_sizes():
    d = _host_lists()
    assert _validate_csr(d, t=2, l=0) == INVALID and "outside the dictionary" in cal.last_error()
    assert _validate_csr(d, t=0, l=-1) == INVALID
    d2 = dict(d, nb=d["nb"] + 1)
    assert _validate_csr(d2) == INVALID and "nb" in cal.last_error()
    assert lib.calibatt_validate_skiplist(None, -1, -1, 1, None) == INVALID


def test_checked_mode_switch():
    # the switch is thread-local state; toggling it makes no HIP call
    lib.calibatt_set_checked_mode(1)
    lib.calibatt_set_checked_mode(0)


def _validate_bm(T, L, H, N, B, bits, words=None, t=-1, l=-1):
    nb = -(-N // B)
    w = -(-nb // 64) if words is None else words
    view = cal.BitmapView(T, L, H, N, B, nb, w, bits.ctypes.data)
    return lib.calibatt_validate_bitmap(ctypes.byref(view), t, l, 1, None)


def test_validate_bitmaps():
    import oracle
    rng = np.random.default_rng(5)
    for N, B in ((1000, 128), (640 * 64, 64), (129, 1)):
        nb = -(-N // B)
        if nb > cal.MAX_NB:
            continue
        masks = (rng.random((1, 2, 2, nb, nb)) < 0.3).astype(np.uint8)
        bits = np.ascontiguousarray(oracle.compile_bitmap(masks))
        assert _validate_bm(1, 2, 2, N, B, bits) == cal.OK, cal.last_error()
        assert _validate_bm(1, 2, 2, N, B, bits, t=0, l=1) == cal.OK
        if nb % 64:
            bad = bits.copy()
            bad[3, -1] |= np.uint64(1) << np.uint64(63)      # a bit past nb
            assert _validate_bm(1, 2, 2, N, B, bad) == INVALID and "past nb" in cal.last_error()
            # the record holding row 3 is (0, 0); record (0, 1) is still fine
            assert _validate_bm(1, 2, 2, N, B, bad, t=0, l=0) == INVALID
            assert _validate_bm(1, 2, 2, N, B, bad, t=0, l=1) == cal.OK
        assert _validate_bm(1, 2, 2, N, B, bits, words=-(-nb // 64) + 1) == INVALID


def test_bitmap_calls_reject_bad_views():
    view = cal.BitmapView(1, 1, 2, 1000, 128, 8, 2, P)     # words must be ceil(8/64) = 1
    st = lib.calibatt_block_sparse_attn_bm(P, P, P, P, None, 2, 1000, 128, cal.BF16, 0.088, ctypes.byref(view), 0, 0,
                                           None, 0, None)
    assert st == INVALID and "words" in cal.last_error()
    assert lib.calibatt_block_sparse_attn_bm(P, P, P, P, None, 2, 1000, 128, cal.BF16, 0.088, None, 0, 0, None, 0,
                                             None) == INVALID
    assert lib.calibatt_compile_bitmap(None, 1, 1, 1, 100, 10, P, None) == INVALID
    assert lib.calibatt_compile_bitmap(P, 1, 1, 1, 100, 10, P + 4, None) == INVALID    # not 8-byte aligned
    view = cal.BitmapView(1, 1, 2, 1000, 128, 8, 1, P + 4)  # the kernels read whole 64-bit words
    st = lib.calibatt_block_sparse_attn_bm(P, P, P, P, None, 2, 1000, 128, cal.BF16, 0.088, ctypes.byref(view), 0, 0,
                                           None, 0, None)
    assert st == INVALID and "aligned" in cal.last_error()
