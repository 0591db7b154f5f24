"""The CPU baseline's stratified row sample (bench.py): one block per stratum
of 16 blocks, the last block always in, rows sorted and unique, so that the
extrapolation by causal pairs covers the whole sequence evenly."""

import numpy as np

import bench


def test_stratified_rows_one_block_per_stratum_and_the_last():
    rng = np.random.default_rng(0)
    for L in (1, 127, 128, 129, 4096, 32768, 3000):
        rows = bench.stratified_rows(L, 128, 16, rng)
        assert np.all(np.diff(rows) > 0) and rows.min() >= 0 and rows.max() == L - 1
        blocks = sorted(set((rows // 128).tolist()))
        n_blocks = (L + 127) // 128
        strata = [b // 16 for b in blocks]
        # at most two blocks in the last stratum (its drawn block and the last block), one elsewhere
        for s in set(strata):
            assert strata.count(s) <= (2 if s == (n_blocks - 1) // 16 else 1)
        assert len(set(strata)) == (n_blocks + 15) // 16
        for b in blocks:  # whole blocks
            assert set(range(b * 128, min(L, b * 128 + 128))) <= set(rows.tolist())


def test_stratified_sample_fraction_of_the_long_prefill():
    rng = np.random.default_rng(0x51A7)
    rows = bench.stratified_rows(32768, 128, 16, rng)
    frac = (rows + 1).sum() / (32768 * 32769 / 2)
    assert 0.03 < frac < 0.12, frac
