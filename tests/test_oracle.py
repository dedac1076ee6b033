"""The fp64 oracle against what the pages and the mathematics fix (CPU only)."""
import numpy as np
import pytest

import pins
from sparse_top_latent_amd.workloads import make_random, make_tiny


@pytest.mark.parametrize("check", pins.BATTERY, ids=lambda c: c.__name__)
def test_oracle_pin(ref, check):
    msg = check(ref)
    assert msg is None, msg


def test_out_of_range_index_is_an_error(ref):
    w = make_random(40, 1, 2, 2, 8, 10, 4, p_unused=0.0)
    bad = w.idxs.copy()
    bad[0, 1, 2] = w.N
    with pytest.raises(ValueError):
        ref(w.q, w.kv_host(), w.sink, bad, w.scale)


def test_unreferenced_nan_rows_are_never_read(ref):
    # the generators poison unreferenced rows with NaN; the oracle must stay finite
    w = make_random(42, 2, 3, 4, 16, 64, 8, p_unused=0.2)
    kv = w.kv_host()
    assert (kv == 0x7FC0).any()
    out = ref(w.q, kv, w.sink, w.idxs, w.scale)
    assert np.isfinite(out).all()


def test_any_negative_index_is_unused(ref):
    w = make_random(41, 1, 2, 4, 16, 12, 6, p_unused=0.3)
    kv = w.kv_host()
    other = np.where(w.idxs < 0, -7, w.idxs).astype(np.int32)
    np.testing.assert_array_equal(ref(w.q, kv, w.sink, w.idxs, w.scale),
                                  ref(w.q, kv, w.sink, other, w.scale))
