"""The seeded generators are deterministic and produce the workloads' shapes."""

import numpy as np
import torch

import synth


def test_structures_are_deterministic():
    for make in (synth.small_structure, synth.decode_structure, synth.chunked_structure,
                 synth.reuse_structure, synth.ragged_structure):
        a, b = make(), make()
        np.testing.assert_array_equal(a.hist, b.hist)
        np.testing.assert_array_equal(a.page_table, b.page_table)
        np.testing.assert_array_equal(a.ring_id, b.ring_id)


def test_page_tables_are_disjoint_permutations():
    s = synth.ragged_structure()
    used = s.page_table[s.page_table >= 0]
    assert len(np.unique(used)) == len(used)
    assert used.max() < s.num_pages
    # physical order differs from logical order
    assert not np.all(np.diff(s.page_table[0][s.page_table[0] >= 0]) == 1)


def test_workload_shapes():
    r = synth.ragged_structure()
    assert r.batch == 24
    assert (r.hist[:12] >= 1024).all() and (r.hist[:12] <= 65536).all()
    assert (r.hist[20:] >= 262144).all() and (r.hist[20:] <= 1 << 20).all()
    u = synth.reuse_structure()
    assert u.batch == 32 and (u.hist >= 4096).all() and (u.new >= 512).all()
    for b in range(u.batch):
        ev = u.extra["evicted"][b]
        assert len(ev) == int(np.floor(u.extra["frac"][b] * 128))
        assert (ev >= u.hist[b] - 128).all() and (ev < u.hist[b]).all()
    req, cached, valid = synth.reuse_tokens(u, 0)
    assert len(req) == u.hist[0] + u.new[0] and (req[: u.hist[0]] == cached).all()
    assert valid.sum() == u.hist[0] - len(u.extra["evicted"][0])


def test_values_reproducible_and_bf16_rounded():
    a = synth.normal_bf16((4, 8), "decode", 3, synth.K_VALUES, "cpu")
    b = synth.normal_bf16((4, 8), "decode", 3, synth.K_VALUES, "cpu")
    c = synth.normal_bf16((4, 8), "decode", 4, synth.K_VALUES, "cpu")
    assert a.dtype == torch.bfloat16
    assert torch.equal(a, b) and not torch.equal(a, c)
    f = synth.normal_f32((4, 8), "decode", 3, synth.K_VALUES, "cpu")
    assert torch.equal(f.to(torch.bfloat16), a)
