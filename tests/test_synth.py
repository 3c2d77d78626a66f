"""The seeded input generators (CPU): Philox known answers, the normal draw, recipes."""
import os

import numpy as np

from synth import philox as P
from synth import recipes as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")


def test_philox_known_answers():
    n = 0
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        v = [int(x, 16) for x in line.split()]
        out = P.philox4x32_10(*v[:6])
        assert [int(x) for x in out] == v[6:]
        n += 1
    assert n == 3


def test_normal_draw_is_exact_irwin_hall():
    idx = np.arange(200000, dtype=np.uint64)
    z = P.normal_f32(0, 7, idx)
    # value * 65536 is an integer in [-393210, 393210]
    k = z.astype(np.float64) * 65536
    assert np.array_equal(k, np.round(k)) and np.abs(k).max() <= 393210
    assert abs(z.mean()) < 0.01 and abs(z.var() - 1) < 0.01
    # rebuild one element by hand from the two Philox calls
    i = 123456789012
    a = P.philox4x32_10(i & 0xFFFFFFFF, i >> 32, 7, 0, 0, 0)
    b = P.philox4x32_10(i & 0xFFFFFFFF, i >> 32, 7, 1, 0, 0)
    halves = []
    for w in [int(x) for x in list(a) + list(b)]:
        halves += [w & 0xFFFF, w >> 16]
    want = sum((h + 0.5) / 65536 for h in halves[:12]) - 6
    assert float(P.normal_f32(0, 7, np.array([i], dtype=np.uint64))[0]) == want


def test_bf16_rounding_ties_to_even():
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -1.0 - 2 ** -8], dtype=np.float32)
    got = P.bf16_bits_to_f32(P.f32_to_bf16_bits(x))
    assert list(got) == [1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -1.0]


def test_recipes_plan_and_tables():
    cfg = R.make_config("C4")
    p = cfg.plan.reshape(-1)
    assert (p == 0).sum() == 48 and (p == 1).sum() == 29 and (p == 2).sum() == 19
    assert np.all(cfg.plan[-1] != 2)
    bt = R.block_table(cfg)
    assert bt.shape == (32, 1024)
    assert np.array_equal(np.sort(bt.reshape(-1)), np.arange(32 * 1024))
    assert not np.array_equal(bt.reshape(-1), np.arange(32 * 1024))
    c5 = R.make_config("C5")
    assert len(c5.lengths) == 128 and min(c5.lengths) >= 1024 and max(c5.lengths) <= 16384
    bt5 = R.block_table(c5)
    used = bt5[bt5 >= 0]
    assert used.size == R.num_blocks(c5) and np.unique(used).size == used.size
    f = R.factor_table(R.make_config("C2"))
    assert f.shape == (1, 2, 16, 128) and ((f == 10).sum(axis=-1) == 3).all()
    f3 = R.factor_table(R.make_config("C3"))
    assert f3.min() >= 0.5 and f3.max() <= 4.0
