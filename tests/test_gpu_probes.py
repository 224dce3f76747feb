"""The measurement probes of include/ha_probe.h on the GPU. The paged read
probe must read exactly the K/V words of decode's walk over a page table (its
per-thread checksum equals the same fold over the pool's bytes, computed on
the host), whether or not its loads carry the non-temporal bit; the
matrix-core and co-issue probes must run in every mode and write their
sinks."""

import ctypes

import numpy as np
import pytest
import torch

import hybrid_sliding_window_gqa_amd as ha
from hybrid_sliding_window_gqa_amd import _lib

pytestmark = pytest.mark.gpu


def _expected_paged_read(k_words, v_words, table, lens, hkv, d, num_pages):
    """Host replica of the probe's fold: thread t of workgroup (kv head g,
    sequence b) XORs, over the blocks i = t/64, t/64 + 4, ... below
    ceil(len/16), words 0 and 3 of K's 16-byte unit (64 m + t%64) and words 1
    and 2 of V's, for every 32-channel slice m; a page id out of range reads
    zeros."""
    units = d // 32
    out = np.zeros((len(lens), hkv, 256), np.uint32)
    lane = np.arange(64)
    for b, n in enumerate(lens):
        nblk = min(-(-max(n, 0) // 16), table.shape[1])
        for g in range(hkv):
            for w in range(4):
                acc = np.zeros(64, np.uint32)
                for i in range(w, nblk, 4):
                    pg = int(table[b, i])
                    if not 0 <= pg < num_pages:
                        continue
                    for m in range(units):
                        u = 64 * m + lane
                        acc ^= k_words[pg, g, u, 0] ^ k_words[pg, g, u, 3] ^ v_words[pg, g, u, 1] ^ v_words[pg, g, u, 2]
                out[b, g, 64 * w:64 * w + 64] = acc
    return out


@pytest.mark.parametrize("d", [64, 128])
def test_paged_read_probe_reads_the_decode_walk(d):
    shape = ha.HeadShape(16, 4, d)
    lens = [1, 16, 17, 100, 300, 0, 129]
    per = [-(-n // 16) for n in lens]
    num_pages = sum(per) + 5
    pool = ha.FullPagePool(shape, num_pages, "cuda")
    gen = torch.Generator(device="cpu").manual_seed(11)
    for t in (pool.k, pool.v):
        bits = torch.randint(-32768, 32768, t.shape, generator=gen, dtype=torch.int32).to(torch.int16)
        t.view(torch.int16).copy_(bits.to("cuda"))
    rng = np.random.default_rng(3)
    perm = rng.permutation(num_pages)
    table = np.full((len(lens), max(per) + 1), -1, np.int32)
    off = 0
    for b, c in enumerate(per):
        table[b, :c] = perm[off:off + c]
        off += c
    table[3, 2] = num_pages + 7          # an out-of-range page id inside a sequence: read as zeros
    view = pool.view(torch.as_tensor(table, device="cuda"))
    kv_len = torch.as_tensor(np.array(lens, np.int32), device="cuda")
    k_words = pool.k.view(torch.int32).cpu().numpy().view(np.uint32).reshape(num_pages, 4, 16 * d // 8, 4)
    v_words = pool.v.view(torch.int32).cpu().numpy().view(np.uint32).reshape(num_pages, 4, 16 * d // 8, 4)
    want = _expected_paged_read(k_words, v_words, table, lens, 4, d, num_pages)
    lib = _lib.load()
    c_shape, c_view = shape.c(), view.c()
    for nt in (0, 1):
        sink = torch.full((len(lens) * 4 * 256,), -1, dtype=torch.int32, device="cuda")
        _lib.check(lib.ha_probe_paged_read(ctypes.byref(c_shape), ctypes.byref(c_view), kv_len.data_ptr(), len(lens),
                                           sink.data_ptr(), nt, None))
        torch.cuda.synchronize()
        got = sink.cpu().numpy().view(np.uint32).reshape(len(lens), 4, 256)
        assert np.array_equal(got, want), f"nontemporal={nt}"


def test_mfma_and_coissue_probes_run_in_every_mode():
    lib = _lib.load()
    sink = torch.full((8 * 512,), float("nan"), dtype=torch.float32, device="cuda")
    _lib.check(lib.ha_probe_mfma_bf16(8, 16, sink.data_ptr(), None))
    torch.cuda.synchronize()
    assert torch.isfinite(sink[:8 * 256]).all()
    for mode in range(5):
        sink.fill_(float("nan"))
        _lib.check(lib.ha_probe_coissue(mode, 8, 4, sink.data_ptr(), None))
        torch.cuda.synchronize()
        assert torch.isfinite(sink).all(), mode
