"""Structure of the seeded synthetic inputs (CPU)."""
import numpy as np
import pytest

import synth


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 2**-8 + 2**-20, 1.0 + 3 * 2**-8, -2.5, 0.0],
                 dtype=np.float32)
    got = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x))
    # 1+2^-8 is a tie -> even (1.0); just above the tie rounds up; 1+3*2^-8 tie -> 1+2^-6
    np.testing.assert_array_equal(got, np.array([1.0, 1.0, 1.0 + 2**-7, 1.0 + 2**-6, -2.5, 0.0],
                                                dtype=np.float32))


def test_tiny_config_structure_and_determinism():
    a = synth.make(0)
    b = synth.make(0)
    for f in ("h", "W", "idx", "p", "mask"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
    c = a.cfg
    assert a.h.shape == (c.N, c.d) and a.h.dtype == np.float32
    assert a.W.shape == (c.V, c.d)
    assert a.idx.shape == (c.N, c.K) and a.idx.dtype == np.int32
    assert a.idx.min() >= 0 and a.idx.max() < c.V
    assert all(len(set(r)) == c.K for r in a.idx)
    assert np.all(np.diff(a.p, axis=1) <= 0)
    M = a.p.sum(1)
    assert M.min() >= c.mass_lo - 1e-6 and M.max() <= c.mass_hi + 1e-6
    assert a.mask.dtype == np.uint8 and a.mask.all()
    assert abs(a.h.std() - 1.0) < 0.02
    assert abs(a.W.std() - 2.0 / np.sqrt(c.d)) < 0.01 * 2.0 / np.sqrt(c.d) * 5


def test_row_ranges_reproduce_the_full_draw():
    c = synth.config(1, N=20000)
    seed = 123
    full_idx = synth.make_topk_idx(c, seed)
    part = synth.make_topk_idx(c, seed, 8000, 17000)
    np.testing.assert_array_equal(part, full_idx[8000:17000])
    h = synth.make_h(synth.config(0, N=20000), seed, 9000, 9010)
    np.testing.assert_array_equal(h, synth.make_h(synth.config(0, N=20000), seed)[9000:9010])


def test_zipf_head_share():
    """Zipf(1.1) over 128256 puts about 46% of each row's 100 draws below 256."""
    c = synth.config(1, N=2000)
    idx = synth.make_topk_idx(c, 5)
    share = (idx < 256).mean()
    assert 0.40 < share < 0.52


@pytest.mark.parametrize("cid", [2, 4])
def test_packed_masks(cid):
    c = synth.config(cid)
    seed = synth.BASE_SEED + cid
    lens = synth.packed_lengths(c, seed)
    assert lens.sum() == c.N and lens[:-1].min() >= 512 and lens.max() <= 8192
    m = synth.make_mask(c, seed)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    assert np.all(m[starts] == 0)
    if cid == 2:
        assert m.sum() == c.N - len(lens)
    else:
        frac = 1 - m.mean()
        assert 0.09 < frac < 0.115


def test_teacher_logits_rows_are_reproducible_and_shaped():
    a = synth.make_teacher_logits(300, 1000, seed=5)
    b = synth.make_teacher_logits(300, 1000, seed=5, row_lo=120, row_hi=130, threads=1)
    assert a.dtype == np.uint16 and a.shape == (300, 1000)
    assert np.array_equal(a[120:130], b)
    f = synth.make_teacher_logits(4, 1000, seed=5, dtype="f32")
    assert f.dtype == np.float32
    # the frequency prior puts the largest logits at low token ids on average
    x = synth.bf16_bits_to_f32(a).astype(np.float64)
    top = np.argsort(-x, axis=1, kind="stable")[:, :10]
    assert np.median(top) < 200
