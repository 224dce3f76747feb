"""CPU tests of the C ABI: the library loads, exports every declared symbol,
and rejects invalid arguments on the host before any HIP call."""

import ctypes
import os
import re

import pytest

from hybrid_sliding_window_gqa_amd import _lib
from hybrid_sliding_window_gqa_amd._lib import HaKvView, HaShape

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def _declared_functions():
    text = ""
    for name in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if name.endswith(".h"):
            with open(os.path.join(ROOT, "include", name)) as f:
                text += f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_exports_every_declared_symbol(lib):
    declared = _declared_functions()
    assert set(declared) == set(_lib.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings(lib):
    assert lib.ha_abi_version() == _lib.ABI_VERSION
    assert _lib.status_str(0) == "HA_OK"
    assert _lib.status_str(4) == "HA_ERR_WORKSPACE"
    assert _lib.status_str(99) == "HA_ERR_UNKNOWN"


def good_shape(**kw):
    base = dict(num_q_heads=64, num_kv_heads=8, head_dim=128, window=128, page_size=16, softmax_scale=0.0)
    base.update(kw)
    return HaShape(**base)


FAKE = 0x1000  # never dereferenced: every call below fails validation first


def view(kind=_lib.HA_FULL, k=FAKE, v=FAKE, table=FAKE, stride=4, blocks=8):
    return HaKvView(kind, k, v, blocks, table, stride)


def decode_call(lib, shape, kv, batch=2, max_len=100, q=FAKE, dtype=0, splits=0, ws=None, ws_bytes=0,
                k_new=None, v_new=None):
    return lib.hybrid_attn_decode(ctypes.byref(shape) if shape is not None else None,
                                  ctypes.byref(kv) if kv is not None else None, FAKE, batch, max_len, q, k_new,
                                  v_new, dtype, FAKE, FAKE, splits, ws, ws_bytes, None)


@pytest.mark.parametrize(
    "shape_kw,status",
    [
        (dict(num_q_heads=60), _lib.HA_ERR_SHAPE),          # not a multiple of Hkv
        (dict(num_q_heads=8 * 32), _lib.HA_ERR_SHAPE),      # group 32 unsupported
        (dict(num_q_heads=24), _lib.HA_ERR_SHAPE),          # group 3 unsupported
        (dict(head_dim=96), _lib.HA_ERR_SHAPE),
        (dict(window=0), _lib.HA_ERR_SHAPE),
        (dict(window=-16), _lib.HA_ERR_SHAPE),
        (dict(window=(1 << 24) + 1), _lib.HA_ERR_SHAPE),
        (dict(page_size=8), _lib.HA_ERR_SHAPE),           # pages hold whole 16-token blocks
        (dict(page_size=48), _lib.HA_ERR_SHAPE),          # not a power of two
        (dict(page_size=0), _lib.HA_ERR_SHAPE),
        (dict(page_size=1 << 21), _lib.HA_ERR_SHAPE),
        (dict(num_kv_heads=0), _lib.HA_ERR_SHAPE),
        (dict(softmax_scale=float("nan")), _lib.HA_ERR_SHAPE),
    ],
)
def test_shape_errors(lib, shape_kw, status):
    assert decode_call(lib, good_shape(**shape_kw), view()) == status
    assert "" != lib.ha_last_error().decode()


@pytest.mark.parametrize("window", [1, 3, 16, 100, 1 << 24])
def test_any_window_from_one_is_accepted(lib, window):
    # the ring is stored as ceil(W / 16) blocks, so W need not be a multiple of
    # 16; validation then reaches the next argument (a NULL q)
    assert decode_call(lib, good_shape(window=window), view(), q=None) == _lib.HA_ERR_NULL


@pytest.mark.parametrize("page_size", [16, 32, 64, 1 << 20])
def test_power_of_two_page_sizes_are_accepted(lib, page_size):
    assert decode_call(lib, good_shape(page_size=page_size), view(), q=None) == _lib.HA_ERR_NULL


def test_page_table_row_beyond_int32_positions_is_rejected(lib):
    # a row of stride pages x page_size tokens must stay below 2^31 tokens
    s = good_shape(page_size=1 << 20)
    assert decode_call(lib, s, view(stride=1 << 11), q=None) == _lib.HA_ERR_NULL
    assert decode_call(lib, s, view(stride=(1 << 11) + 1)) == _lib.HA_ERR_RANGE


def test_null_and_range_errors(lib):
    s = good_shape()
    assert decode_call(lib, None, view()) == _lib.HA_ERR_NULL
    assert decode_call(lib, s, None) == _lib.HA_ERR_NULL
    assert decode_call(lib, s, view(k=None)) == _lib.HA_ERR_NULL
    assert decode_call(lib, s, view(table=None)) == _lib.HA_ERR_NULL
    assert decode_call(lib, s, view(stride=0)) == _lib.HA_ERR_RANGE
    assert decode_call(lib, s, view(), batch=-1) == _lib.HA_ERR_RANGE
    assert decode_call(lib, s, view(), q=None) == _lib.HA_ERR_NULL
    assert decode_call(lib, s, view(), dtype=7) == _lib.HA_ERR_UNSUPPORTED
    assert decode_call(lib, s, view(kind=3)) == _lib.HA_ERR_UNSUPPORTED
    assert decode_call(lib, s, view(), batch=70000) == _lib.HA_ERR_RANGE
    # the fused append needs both new-token tensors or neither
    assert decode_call(lib, s, view(), k_new=FAKE) == _lib.HA_ERR_NULL
    assert decode_call(lib, s, view(), v_new=FAKE) == _lib.HA_ERR_NULL


def test_decode_workspace_checked(lib):
    s = good_shape()
    # 8 sequences x 8 kv heads cannot fill 256 CUs twice over: the keys are split
    need = lib.hybrid_attn_workspace_size(ctypes.byref(s), _lib.HA_FULL, 1, 8, 32768, 0)
    splits = lib.hybrid_attn_decode_splits(ctypes.byref(s), _lib.HA_FULL, 8, 32768, 0)
    assert splits > 1
    assert need == 8 * 64 * splits * (128 + 1) * 4
    assert decode_call(lib, s, view(), batch=8, max_len=32768) == _lib.HA_ERR_WORKSPACE
    assert decode_call(lib, s, view(), batch=8, max_len=32768, ws=FAKE, ws_bytes=need - 1) == _lib.HA_ERR_WORKSPACE
    # 64 x 8 pairs give every CU two workgroups: one split, no merge, no workspace
    assert lib.hybrid_attn_decode_splits(ctypes.byref(s), _lib.HA_FULL, 64, 8193, 0) == 1
    assert lib.hybrid_attn_workspace_size(ctypes.byref(s), _lib.HA_FULL, 1, 64, 8193, 0) == 0
    # SWA decode and prefill need none
    assert lib.hybrid_attn_workspace_size(ctypes.byref(s), _lib.HA_SWA, 1, 64, 8193, 0) == 0
    # prefill: the staged chunk (K and V of every 16-token block); full layers add the
    # partial rows of work items split by keys: up to 64 parts per XCD, 384 rows x
    # (D + 1) floats each
    stage = ((8193 + 15) // 16 + 64) * 8 * 16 * 128 * 2 * 2
    assert lib.hybrid_attn_workspace_size(ctypes.byref(s), _lib.HA_SWA, 0, 64, 8193, 0) == stage
    assert lib.hybrid_attn_workspace_size(ctypes.byref(s), _lib.HA_FULL, 0, 64, 8193, 0) == \
        stage + 8 * 64 * 384 * (128 + 1) * 4
    assert lib.hybrid_attn_decode_splits(ctypes.byref(s), _lib.HA_SWA, 64, 8193, 0) == 1
    # a filled batch still splits a long sequence: at most 1024 blocks per workgroup
    # (a batch of short sequences and one of 900K tokens must not leave the long one
    # to its 8 workgroups)
    splits = lib.hybrid_attn_decode_splits(ctypes.byref(s), _lib.HA_FULL, 256, 900000, 0)
    assert splits > 1 and -(-(-(-900000 // 16)) // splits) <= 1024
    # explicit split count is honoured
    assert lib.hybrid_attn_decode_splits(ctypes.byref(s), _lib.HA_FULL, 64, 8193, 4) == 4


def test_append_and_prefill_errors(lib):
    s = good_shape()
    ring = view(kind=_lib.HA_SWA)
    pages = view(kind=_lib.HA_FULL)
    # wrong view kind
    assert lib.swa_ring_append(ctypes.byref(s), ctypes.byref(pages), FAKE, FAKE, 2, 10, FAKE, FAKE, 0,
                               None) == _lib.HA_ERR_UNSUPPORTED
    assert lib.full_pool_append(ctypes.byref(s), ctypes.byref(ring), FAKE, FAKE, 2, 10, FAKE, FAKE, 0,
                                None) == _lib.HA_ERR_UNSUPPORTED
    assert lib.swa_ring_append(ctypes.byref(s), ctypes.byref(ring), None, FAKE, 2, 10, FAKE, FAKE, 0,
                               None) == _lib.HA_ERR_NULL
    assert lib.swa_ring_append(ctypes.byref(s), ctypes.byref(ring), FAKE, FAKE, 2, -1, FAKE, FAKE, 0,
                               None) == _lib.HA_ERR_RANGE
    assert lib.swa_ring_append(ctypes.byref(s), ctypes.byref(ring), FAKE, FAKE, 2, 10, FAKE, FAKE, 2,
                               None) == _lib.HA_ERR_UNSUPPORTED
    # empty work is a successful no-op that touches nothing
    assert lib.swa_ring_append(ctypes.byref(s), ctypes.byref(ring), FAKE, FAKE, 0, 0, FAKE, FAKE, 0, None) == 0
    args = [FAKE, FAKE, 2, 10, 5, FAKE, FAKE, FAKE, 0, FAKE, FAKE, FAKE, 1 << 30, None]
    assert lib.hybrid_attn_prefill(ctypes.byref(s), ctypes.byref(pages), *args[:2], 2, 10, 11,
                                   *args[5:]) == _lib.HA_ERR_RANGE          # max_new > num_tokens
    bad = list(args)
    bad[5] = None
    assert lib.hybrid_attn_prefill(ctypes.byref(s), ctypes.byref(pages), *bad) == _lib.HA_ERR_NULL
    assert lib.hybrid_attn_prefill(ctypes.byref(s), ctypes.byref(pages), FAKE, FAKE, 0, 0, 0,
                                   *args[5:]) == 0
    small_ws = list(args)
    small_ws[12] = 100
    assert lib.hybrid_attn_prefill(ctypes.byref(s), ctypes.byref(pages), *small_ws) == _lib.HA_ERR_WORKSPACE


def test_errors_do_not_leak_between_calls(lib):
    s = good_shape()
    assert decode_call(lib, good_shape(head_dim=3), view()) == _lib.HA_ERR_SHAPE
    assert b"head_dim" in lib.ha_last_error()
    out = ctypes.c_int64()
    assert lib.window_safe_match(None, 0, None, 0, None, 4, ctypes.byref(out)) == 0
    assert out.value == 0
    assert lib.ha_last_error() == b""
    assert s.window == 128


def verify_call(lib, shape, kv, batch=2, max_len=100, nq=4, q=FAKE, k_new=FAKE, v_new=FAKE, dtype=0, splits=0,
                ws=None, ws_bytes=0):
    return lib.hybrid_attn_verify(ctypes.byref(shape) if shape is not None else None,
                                  ctypes.byref(kv) if kv is not None else None, FAKE, batch, max_len, nq, q, k_new,
                                  v_new, dtype, FAKE, FAKE, splits, ws, ws_bytes, None)


def test_verify_errors_and_workspace(lib):
    s = good_shape()                       # group 8
    ring = view(kind=_lib.HA_SWA)
    assert verify_call(lib, s, ring, nq=0) == _lib.HA_ERR_RANGE
    assert verify_call(lib, s, ring, nq=17) == _lib.HA_ERR_RANGE
    assert verify_call(lib, s, ring, nq=5) == _lib.HA_ERR_SHAPE          # 5 * 8 columns > 32
    assert verify_call(lib, good_shape(num_q_heads=8, num_kv_heads=8), ring, nq=16, k_new=None) == \
        _lib.HA_ERR_NULL                                                  # group 1: nq 16 allowed
    assert verify_call(lib, s, ring, k_new=None) == _lib.HA_ERR_NULL
    assert verify_call(lib, s, ring, v_new=None) == _lib.HA_ERR_NULL
    assert verify_call(lib, s, ring, q=None) == _lib.HA_ERR_NULL
    assert verify_call(lib, s, ring, batch=70000) == _lib.HA_ERR_RANGE
    assert verify_call(lib, s, ring, dtype=7) == _lib.HA_ERR_UNSUPPORTED
    assert verify_call(lib, None, ring) == _lib.HA_ERR_NULL
    # full layers: split-K partials need a workspace sized for nq rows per sequence
    need = lib.hybrid_attn_verify_workspace_size(ctypes.byref(s), _lib.HA_FULL, 8, 32772, 4, 0)
    splits = lib.hybrid_attn_decode_splits(ctypes.byref(s), _lib.HA_FULL, 8, 32772, 0)
    assert splits > 1 and need == 8 * 4 * 64 * splits * (128 + 1) * 4
    assert lib.hybrid_attn_verify_workspace_size(ctypes.byref(s), _lib.HA_FULL, 64, 8196, 4, 0) == 0   # one split
    assert verify_call(lib, s, view(), batch=8, max_len=32772) == _lib.HA_ERR_WORKSPACE
    assert verify_call(lib, s, view(), batch=8, max_len=32772, ws=FAKE, ws_bytes=need - 1) == _lib.HA_ERR_WORKSPACE
    assert lib.hybrid_attn_verify_workspace_size(ctypes.byref(s), _lib.HA_SWA, 64, 8196, 4, 0) == 0
    assert lib.hybrid_attn_verify_workspace_size(ctypes.byref(s), _lib.HA_FULL, 64, 8196, 5, 0) == 0   # invalid nq
    assert verify_call(lib, s, ring, batch=0) == _lib.HA_OK


def test_int8_view_errors(lib):
    s = good_shape()
    int8 = lambda kind, ks=FAKE, vs=FAKE: HaKvView(kind, FAKE, FAKE, 8, FAKE, 4, _lib.HA_KV_INT8, ks, vs)
    pages, ring = int8(_lib.HA_FULL), int8(_lib.HA_SWA)
    # scales are required, and the format must be known
    for bad, status in ((int8(_lib.HA_FULL, ks=None), _lib.HA_ERR_NULL),
                        (int8(_lib.HA_FULL, vs=None), _lib.HA_ERR_NULL),
                        (HaKvView(_lib.HA_FULL, FAKE, FAKE, 8, FAKE, 4, 7, FAKE, FAKE), _lib.HA_ERR_UNSUPPORTED)):
        assert decode_call(lib, s, bad) == status
        assert lib.full_pool_append(ctypes.byref(s), ctypes.byref(bad), FAKE, FAKE, 2, 10, FAKE, FAKE, 0,
                                    None) == status
    # prefill reads bf16 pools only
    args = [FAKE, FAKE, 2, 10, 5, FAKE, FAKE, FAKE, 0, FAKE, FAKE, FAKE, 1 << 30, None]
    assert lib.hybrid_attn_prefill(ctypes.byref(s), ctypes.byref(ring), *args) == _lib.HA_ERR_UNSUPPORTED
    # verify takes INT8 pools: validation reaches the NULL query (and a view
    # without scales is refused first)
    verify = lambda v, q: lib.hybrid_attn_verify(ctypes.byref(s), ctypes.byref(v), FAKE, 2, 100, 4, q, FAKE, FAKE,
                                                  0, FAKE, FAKE, 0, FAKE, 1 << 30, None)
    assert verify(pages, None) == _lib.HA_ERR_NULL
    assert verify(ring, None) == _lib.HA_ERR_NULL
    assert verify(int8(_lib.HA_FULL, ks=None), FAKE) == _lib.HA_ERR_NULL
    # the zero-initialised tail of a view is a bf16 pool
    assert HaKvView(_lib.HA_FULL, FAKE, FAKE, 8, FAKE, 4).kv_dtype == _lib.HA_KV_BF16


def test_read_errors(lib):
    s = good_shape()
    ring, pages = view(kind=_lib.HA_SWA), view(kind=_lib.HA_FULL)
    rd = lambda fn, v, **kw: fn(ctypes.byref(s), ctypes.byref(v), kw.get("pos0", FAKE), FAKE, kw.get("batch", 2),
                                kw.get("n", 10), kw.get("k", FAKE), FAKE, None)
    assert rd(lib.swa_ring_read, pages) == _lib.HA_ERR_UNSUPPORTED
    assert rd(lib.full_pool_read, ring) == _lib.HA_ERR_UNSUPPORTED
    assert rd(lib.swa_ring_read, ring, pos0=None) == _lib.HA_ERR_NULL
    assert rd(lib.full_pool_read, pages, k=None) == _lib.HA_ERR_NULL
    assert rd(lib.full_pool_read, pages, n=-1) == _lib.HA_ERR_RANGE
    assert rd(lib.swa_ring_read, ring, batch=0, n=0) == 0
    int8 = HaKvView(_lib.HA_FULL, FAKE, FAKE, 8, FAKE, 4, _lib.HA_KV_INT8, FAKE, FAKE)
    assert rd(lib.full_pool_read, int8) == _lib.HA_ERR_UNSUPPORTED


def noalloc_call(lib, shape, kv, batch=2, max_len=100, q=FAKE, splits=0):
    return lib.hybrid_attn_decode_noalloc(ctypes.byref(shape) if shape is not None else None,
                                          ctypes.byref(kv) if kv is not None else None, FAKE, batch, max_len, q,
                                          None, None, 0, FAKE, FAKE, splits, None)


def test_noalloc_decode_checks_its_scratch_limit_on_the_host(lib):
    s = good_shape()
    assert noalloc_call(lib, None, view()) == _lib.HA_ERR_NULL
    assert noalloc_call(lib, good_shape(head_dim=96), view()) == _lib.HA_ERR_SHAPE
    assert noalloc_call(lib, s, view(), q=None) == _lib.HA_ERR_NULL
    assert noalloc_call(lib, s, view(), batch=-1) == _lib.HA_ERR_RANGE
    assert noalloc_call(lib, s, view(), batch=0) == _lib.HA_OK
    # 8 sequences of 1M tokens split over many workgroups: partials beyond the static array
    need = lib.hybrid_attn_workspace_size(ctypes.byref(s), _lib.HA_FULL, 1, 8, 1 << 20, 0)
    assert need > _lib.HA_DECODE_SCRATCH_BYTES
    assert noalloc_call(lib, s, view(), batch=8, max_len=1 << 20) == _lib.HA_ERR_WORKSPACE
    assert b"static scratch" in lib.ha_last_error()
    # the same call with fewer splits fits
    assert lib.hybrid_attn_workspace_size(ctypes.byref(s), _lib.HA_FULL, 1, 8, 1 << 20, 64) <= \
        _lib.HA_DECODE_SCRATCH_BYTES


def test_probe_argument_errors(lib):
    s = good_shape()
    pages = view(kind=_lib.HA_FULL)
    ring = view(kind=_lib.HA_SWA)
    assert lib.ha_probe_paged_read(None, ctypes.byref(pages), FAKE, 2, FAKE, 1, None) == _lib.HA_ERR_NULL
    assert lib.ha_probe_paged_read(ctypes.byref(good_shape(head_dim=96)), ctypes.byref(pages), FAKE, 2, FAKE, 1,
                                   None) == _lib.HA_ERR_SHAPE
    assert lib.ha_probe_paged_read(ctypes.byref(s), ctypes.byref(ring), FAKE, 2, FAKE, 1, None) == \
        _lib.HA_ERR_UNSUPPORTED
    assert lib.ha_probe_paged_read(ctypes.byref(s), ctypes.byref(pages), None, 2, FAKE, 1, None) == _lib.HA_ERR_NULL
    assert lib.ha_probe_paged_read(ctypes.byref(s), ctypes.byref(pages), FAKE, -1, FAKE, 1, None) == \
        _lib.HA_ERR_RANGE
    assert lib.ha_probe_paged_read(ctypes.byref(s), ctypes.byref(pages), FAKE, 0, FAKE, 1, None) == _lib.HA_OK
    assert lib.ha_probe_mfma_bf16(0, 10, FAKE, None) == _lib.HA_ERR_RANGE
    assert lib.ha_probe_mfma_bf16(4, 0, FAKE, None) == _lib.HA_ERR_RANGE
    assert lib.ha_probe_mfma_bf16(4, 10, None, None) == _lib.HA_ERR_NULL
    assert lib.ha_probe_coissue(5, 4, 10, FAKE, None) == _lib.HA_ERR_RANGE
    assert lib.ha_probe_coissue(-1, 4, 10, FAKE, None) == _lib.HA_ERR_RANGE
    assert lib.ha_probe_coissue(0, 0, 10, FAKE, None) == _lib.HA_ERR_RANGE
    assert lib.ha_probe_coissue(0, 4, 0, FAKE, None) == _lib.HA_ERR_RANGE
    assert lib.ha_probe_coissue(2, 4, 10, None, None) == _lib.HA_ERR_NULL
