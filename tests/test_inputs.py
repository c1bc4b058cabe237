"""Host checks of the seeded input helpers that the parity tests rely on."""
import numpy as np
import pytest

from mask_mods_amd import inputs


@pytest.mark.parametrize("B,H,S", [(2, 32, 8192), (2, 32, 2048), (1, 2, 1000), (1, 1, 5)])
def test_sample_rows_cover_every_query_block(B, H, S):
    """Every (b, h) keeps its first and last row, and every 128-row block of every (b, h)
    (the smallest forward workgroup) has at least one sampled row."""
    r = inputs.sample_rows(3, B, H, S)
    assert np.all(np.diff(r) > 0) and r.min() >= 0 and r.max() < B * H * S
    bh, i = r // S, r % S
    for x in range(B * H):
        rows = i[bh == x]
        assert rows.min() == 0 and rows.max() == S - 1
        assert set((rows // 128).tolist()) == set(range((S + 127) // 128))


def test_sample_rows_seeded():
    assert np.array_equal(inputs.sample_rows(5, 2, 4, 700), inputs.sample_rows(5, 2, 4, 700))
    assert not np.array_equal(inputs.sample_rows(5, 2, 4, 700), inputs.sample_rows(6, 2, 4, 700))
