"""C-ABI checks that need no GPU: the library loads, exports every entry point that
include/hstu.h declares, and rejects invalid arguments on host data alone, with
the documented status and before any HIP call."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "hstu_jagged_pointwise_amd", "libhstu.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libhstu.so not built")


@pytest.fixture(scope="module")
def ops():
    from hstu_jagged_pointwise_amd import ops as o
    return o


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "hstu.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(\w+)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while", "for")))


def test_every_declared_symbol_is_exported(ops):
    names = _declared_functions()
    assert {"hstu_attn_fwd", "hstu_layer_fwd", "mfalcon_score"} <= set(names)
    for n in names:
        assert hasattr(ops.lib, n), n
    assert set(names) == set(ops.EXPORTED)
    assert ops.hstu_version() == 100


FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: every case below fails validation first


def _desc(ops, **kw):
    d = dict(batch=2, num_heads=2, d_qk=64, d_v=64, max_seq_len=16, num_pos_buckets=8,
             num_time_buckets=8, dtype_code=ops.HSTU_BF16, ln_eps=1e-5)
    d.update(kw)
    return ops.attn_desc(**d)


def _attn(ops, desc, off, q=FAKE, k=FAKE, v=FAKE, u=None, out=FAKE, ws=None, wsb=1 << 30):
    return ops.lib.hstu_attn_fwd(ctypes.byref(desc) if desc is not None else None,
                                 off.ctypes.data_as(ops._I64P) if off is not None else None,
                                 FAKE, None, q, k, v, None, None, u, None, None, out,
                                 ws if ws is not None else ctypes.c_void_p(0x100000), wsb, None)


GOOD_OFF = np.array([0, 5, 12], np.int64)


@pytest.mark.parametrize("case,status", [
    (dict(batch=-1), 1), (dict(num_heads=0), 1), (dict(d_qk=48), 2), (dict(d_v=256), 2),
    (dict(max_seq_len=0), 1), (dict(num_pos_buckets=0), 1), (dict(num_time_buckets=0), 1),
    (dict(dtype_code=7), 2),
])
def test_attn_desc_rejections(ops, case, status):
    d = _desc(ops, **case)
    off = GOOD_OFF if case.get("batch", 2) == 2 else np.zeros(1, np.int64)
    assert _attn(ops, d, off) == status
    assert ops.lib.hstu_last_error().decode() != ""


@pytest.mark.parametrize("off,status", [
    ([1, 5, 12], 1),        # offsets[0] != 0
    ([0, 7, 5], 1),         # decreasing
    ([0, 17, 20], 1),       # a sequence longer than max_seq_len
])
def test_offset_rejections(ops, off, status):
    assert _attn(ops, _desc(ops), np.array(off, np.int64)) == status


def test_pointer_and_workspace_rejections(ops):
    d = _desc(ops)
    assert _attn(ops, None, GOOD_OFF) == 1
    assert _attn(ops, d, None) == 1
    assert _attn(ops, d, GOOD_OFF, q=None) == 1
    assert _attn(ops, d, GOOD_OFF, out=None) == 1
    assert _attn(ops, d, GOOD_OFF, q=ctypes.c_void_p(0x10002)) == 1  # not 16-byte aligned
    assert _attn(ops, d, GOOD_OFF, wsb=16) == 3
    assert _attn(ops, d, GOOD_OFF, ws=ctypes.c_void_p(0x100010)) == 1  # workspace not 256-aligned
    bad_eps = _desc(ops, ln_eps=0.0)
    assert _attn(ops, bad_eps, GOOD_OFF, u=FAKE) == 1


def test_empty_batches_are_noops(ops):
    assert _attn(ops, _desc(ops, batch=0), np.zeros(1, np.int64), q=None, k=None, v=None,
                 out=None) == 0
    assert _attn(ops, _desc(ops), np.zeros(3, np.int64), q=None, k=None, v=None, out=None) == 0


def _attn_noalloc(ops, desc, off, q=FAKE, k=FAKE, v=FAKE, u=None, out=FAKE):
    return ops.lib.hstu_attn_fwd_noalloc(ctypes.byref(desc) if desc is not None else None,
                                         off.ctypes.data_as(ops._I64P) if off is not None else None,
                                         FAKE, None, q, k, v, None, None, u, None, None, out, None)


def test_noalloc_rejections(ops):
    """The allocation-free attention call validates like hstu_attn_fwd and rejects a call
    whose scratch need exceeds its fixed device array, all before any HIP call."""
    cap = ops.lib.hstu_attn_noalloc_scratch_bytes()
    assert cap == 64 << 20
    d = _desc(ops)
    assert _attn_noalloc(ops, None, GOOD_OFF) == 1
    assert _attn_noalloc(ops, d, None) == 1
    assert _attn_noalloc(ops, d, GOOD_OFF, q=None) == 1
    assert _attn_noalloc(ops, d, GOOD_OFF, out=ctypes.c_void_p(0x10008)) == 1
    assert _attn_noalloc(ops, _desc(ops, ln_eps=0.0), GOOD_OFF, u=FAKE) == 1
    assert _attn_noalloc(ops, _desc(ops, batch=0), np.zeros(1, np.int64), q=None, k=None,
                         v=None, out=None) == 0
    # a gated call needs 4 * H * d_v bytes of fp32 rows per token: find the first batch
    # that does not fit (one sequence per 4096 rows) and check both sides of the limit
    dd = dict(num_heads=8, d_qk=64, d_v=64, max_seq_len=4096)
    def need(rows):
        off = np.arange(0, rows + 1, 4096, dtype=np.int64)
        if off[-1] != rows:
            off = np.append(off, rows)
        return off, ops.hstu_attn_workspace_size(_desc(ops, batch=len(off) - 1, **dd), off)
    lo, hi = 4096, 1 << 20
    while hi - lo > 1:
        mid = (lo + hi) // 2
        lo, hi = (mid, hi) if need(mid)[1] <= cap else (lo, mid)
    off_ok, n_ok = need(lo)
    off_big, n_big = need(hi)
    assert n_ok <= cap < n_big
    assert _attn_noalloc(ops, _desc(ops, batch=len(off_big) - 1, **dd), off_big, u=FAKE) == 2
    assert "scratch" in ops.lib.hstu_last_error().decode()


def test_workspace_sizes(ops):
    d = _desc(ops, batch=4, max_seq_len=300)  # bf16, d=64: 128-row tiles
    off = np.array([0, 300, 301, 301, 500], np.int64)
    n = ops.hstu_attn_workspace_size(d, off)
    items = 3 + 1 + 0 + 2
    al = lambda x: (x + 255) // 256 * 256
    key_ranges = 500 // 32 + 4 + 1  # one (min, max) timestamp pair per 32-key block slot
    assert n == al(items * 8) + al(key_ranges * 16) + al(500 * 2 * 64 * 4)
    d32 = _desc(ops, dtype_code=ops.HSTU_F32, batch=4, max_seq_len=300)  # fp32: 64-row tiles
    assert ops.hstu_attn_workspace_size(d32, off) == al((5 + 1 + 0 + 4) * 8) + al(500 * 2 * 64 * 4)
    with pytest.raises(ops.HstuError) as e:
        ops.hstu_attn_workspace_size(_desc(ops, d_qk=33), GOOD_OFF)
    assert e.value.status == ops.HSTU_UNSUPPORTED


def _layer_desc(ops, **kw):
    a = _desc(ops)
    d = dict(d_model=128, residual=0, num_layers=1)
    d.update(kw)
    return ops.hstu_layer_desc(a, d["d_model"], d["residual"], d["num_layers"])


def _weights(ops, n=1, w1=FAKE):
    arr = (ops.hstu_layer_weights * n)()
    for i in range(n):
        arr[i] = ops.hstu_layer_weights(w1, None, None, None, None, None, FAKE, None)
    return arr


@pytest.mark.parametrize("case,status", [
    (dict(d_model=12), 2), (dict(residual=2), 1), (dict(num_layers=0), 1),
])
def test_layer_rejections(ops, case, status):
    d = _layer_desc(ops, **case)
    r = ops.lib.hstu_layer_fwd(ctypes.byref(d), GOOD_OFF.ctypes.data_as(ops._I64P), FAKE, None,
                               FAKE, _weights(ops), FAKE, ctypes.c_void_p(0x100000), 1 << 30, None)
    assert r == status


def test_layer_weight_rejections(ops):
    d = _layer_desc(ops)
    for arr in (None, _weights(ops, w1=None), _weights(ops, w1=ctypes.c_void_p(0x10004))):
        r = ops.lib.hstu_layer_fwd(ctypes.byref(d), GOOD_OFF.ctypes.data_as(ops._I64P), FAKE, None,
                                   FAKE, arr, FAKE, ctypes.c_void_p(0x100000), 1 << 30, None)
        assert r == 1


def _mf(ops, desc, hoff, coff, hist_ts=None, cand_ts=None, w_head=None, logit=None):
    return ops.lib.mfalcon_score(ctypes.byref(desc), hoff.ctypes.data_as(ops._I64P), FAKE, hist_ts,
                                 FAKE, coff.ctypes.data_as(ops._I64P), FAKE, cand_ts, FAKE,
                                 _weights(ops), w_head, FAKE, logit, ctypes.c_void_p(0x100000),
                                 1 << 30, None)


def test_mfalcon_rejections(ops):
    ld = _layer_desc(ops)
    hoff = np.array([0, 5, 12], np.int64)
    coff = np.array([0, 3, 9], np.int64)
    assert _mf(ops, ops.mfalcon_desc(ld, 0), hoff, coff) == 1                      # microbatch 0
    assert _mf(ops, ops.mfalcon_desc(ld, 4), hoff, coff, hist_ts=FAKE) == 1        # ts mismatch
    assert _mf(ops, ops.mfalcon_desc(ld, 4), hoff, coff, logit=FAKE) == 1          # logit w/o head
    ld.attn.max_seq_len = 16
    # a history of 16 plus its candidate exceeds N = 16; a history of 17 exceeds it alone
    assert _mf(ops, ops.mfalcon_desc(ld, 4), np.array([0, 5, 21], np.int64), coff) == 1
    assert _mf(ops, ops.mfalcon_desc(ld, 4), np.array([0, 5, 22], np.int64), coff) == 1
    # no candidates at all is a no-op
    assert _mf(ops, ops.mfalcon_desc(ld, 4), hoff, np.zeros(3, np.int64)) == 0


def test_mfalcon_cache_rejections(ops):
    """The cached M-FALCON calls check the cache and workspace before any launch."""
    ld = _layer_desc(ops)
    desc = ops.mfalcon_desc(ld, 4)
    hoff = np.array([0, 5, 12], np.int64)
    coff = np.array([0, 3, 9], np.int64)
    hp, cp = hoff.ctypes.data_as(ops._I64P), coff.ctypes.data_as(ops._I64P)
    n = ctypes.c_size_t(0)
    assert ops.lib.mfalcon_cache_size(ctypes.byref(desc), hp, ctypes.byref(n)) == 0
    cache = n.value
    assert cache > 0
    assert ops.lib.mfalcon_history_workspace_size(ctypes.byref(desc), hp, ctypes.byref(n)) == 0
    hws = n.value
    assert ops.lib.mfalcon_cached_workspace_size(ctypes.byref(desc), hp, cp, ctypes.byref(n)) == 0
    cws = n.value
    # the one-shot workspace holds the cache and both passes' scratch
    full = ctypes.c_size_t(0)
    assert ops.lib.mfalcon_workspace_size(ctypes.byref(desc), hp, cp, ctypes.byref(full)) == 0
    al = lambda x: (x + 255) // 256 * 256
    assert full.value == al(cache) + al(hws) + al(cws)
    hist = ops.lib.mfalcon_history
    big = ctypes.c_void_p(0x100000)
    assert hist(ctypes.byref(desc), hp, FAKE, None, FAKE, _weights(ops), big, cache - 1, big, 1 << 30,
                None) == 3                                             # cache too small
    assert hist(ctypes.byref(desc), hp, FAKE, None, FAKE, _weights(ops), ctypes.c_void_p(0x100010),
                cache, big, 1 << 30, None) == 1                        # cache not 256-aligned
    assert hist(ctypes.byref(desc), hp, FAKE, None, FAKE, _weights(ops), big, cache, big, 0,
                None) == 3                                             # workspace too small
    sc = ops.lib.mfalcon_score_cached
    args = lambda c, cb, ws, wsb, hts=None, cts=None: (ctypes.byref(desc), hp, FAKE, hts, c, cb, cp,
                                                        FAKE, cts, FAKE, _weights(ops), None, FAKE,
                                                        None, ws, wsb, None)
    assert sc(*args(big, cache - 1, big, 1 << 30)) == 3                 # cache too small
    assert sc(*args(big, cache, big, cws - 1)) == 3                     # workspace too small
    assert sc(*args(big, cache, big, 1 << 30, hts=FAKE)) == 1           # ts mismatch
    assert sc(ctypes.byref(desc), hp, FAKE, None, big, cache, None, FAKE, None, FAKE, _weights(ops),
              None, FAKE, None, big, 1 << 30, None) == 1                # no host cand offsets


def test_debug_buckets_rejections(ops):
    d = _desc(ops)
    f = ops.lib.hstu_debug_buckets
    assert f(ctypes.byref(d), GOOD_OFF.ctypes.data_as(ops._I64P), FAKE, None, 5, FAKE, FAKE,
             None) == 1
    assert f(ctypes.byref(d), GOOD_OFF.ctypes.data_as(ops._I64P), FAKE, None, 0, None, FAKE,
             None) == 1


def test_status_strings(ops):
    for s, name in enumerate(["HSTU_OK", "HSTU_INVALID_ARGUMENT", "HSTU_UNSUPPORTED",
                              "HSTU_WORKSPACE_TOO_SMALL", "HSTU_DEVICE_ERROR"]):
        assert ops.lib.hstu_status_string(s).decode() == name


def test_layer_bwd_rejections(ops):
    w = ops.hstu_layer_weights(FAKE, None, None, None, None, None, FAKE, None)
    off = np.array([0, 5, 12], np.int64)

    def call(desc, x=FAKE, dy=FAKE, ws=ctypes.c_void_p(0x100000), wsb=1 << 40):
        return ops.lib.hstu_layer_bwd(ctypes.byref(desc), off.ctypes.data_as(ops._I64P), FAKE, None,
                                      x, ctypes.byref(w), dy, None, None, ws, wsb, None)

    good = ops.hstu_layer_desc(_desc(ops), 64, 0, 1)
    wide = ops.hstu_layer_desc(_desc(ops, num_heads=16, d_v=128, d_qk=128), 64, 0, 1)
    assert call(wide) == ops.HSTU_UNSUPPORTED                 # H*d_v > 1024
    assert call(good, x=None) == ops.HSTU_INVALID_ARGUMENT    # x required
    assert call(good, dy=None) == ops.HSTU_INVALID_ARGUMENT   # d_y required
    assert call(good, wsb=16) == ops.HSTU_WORKSPACE_TOO_SMALL
    assert call(ops.hstu_layer_desc(_desc(ops), 60, 0, 1)) == ops.HSTU_UNSUPPORTED  # d_model % 8
    n = ctypes.c_size_t(0)
    assert ops.lib.hstu_layer_bwd_workspace_size(ctypes.byref(good), off.ctypes.data_as(ops._I64P),
                                                 ctypes.byref(n)) == ops.HSTU_OK and n.value > 0
