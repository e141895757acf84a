"""The seeded input generator: determinism, shapes, paging structure (CPU only)."""
import numpy as np
import pytest

from workload import configs, make_inputs, unused_slots


def test_deterministic():
    a = make_inputs(configs.TINY)
    b = make_inputs(configs.TINY)
    for k in ("seq_lens", "block_table", "q_nope", "q_pe", "c_kv", "k_pe", "w_uk", "w_uv"):
        assert np.array_equal(getattr(a, k), getattr(b, k)), k
    c = make_inputs(configs.TINY, seed=1)
    assert not np.array_equal(a.c_kv, c.c_kv)


def test_tiny_shapes_and_pages():
    inp = make_inputs(configs.TINY)
    assert list(inp.seq_lens) == [37, 64]
    assert inp.c_kv.shape == (101, 32) and inp.k_pe.shape == (101, 16)
    assert inp.w_uk.shape == (4, 32, 16) and inp.w_uv.shape == (4, 32, 16)
    bt = inp.block_table
    assert bt.shape == (2, 4)
    assert bt[0, 3] == -1
    used = bt[bt >= 0]
    assert len(set(used.tolist())) == len(used) == 7
    assert inp.num_pages == 10 and used.max() < 10
    spare, tail = unused_slots(inp)
    assert len(spare) == 3 and len(tail) == 48 - 37


def test_ragged_lengths():
    wl = configs.RAGGED.with_(batch=2000)
    rng = np.random.default_rng(0)
    from workload.generate import make_seq_lens
    s = make_seq_lens(wl, rng)
    assert s.min() >= 512 and s.max() <= 32768
    # log-uniform: median near sqrt(512 * 32768) = 4096
    assert 3000 < np.median(s) < 5600


@pytest.mark.parametrize("name", ["tiny"])
def test_value_distributions(name):
    wl = configs.get(name).with_(seq_lens=(4000, 4000), batch=2)
    inp = make_inputs(wl)
    from oracle import bf16_bits_to_f64
    c = bf16_bits_to_f64(inp.c_kv)
    w = bf16_bits_to_f64(inp.w_uk)
    assert abs(c.std() - 1) < 0.02
    assert abs(w.std() * np.sqrt(wl.d_c) - 1) < 0.1
