"""The whole-unit code check used by the GPU parity tests (CPU only): codes
from the oracle itself pass; a flipped bit inside the band passes and is
counted; a flipped bit outside the band fails."""

import numpy as np
import pytest

import oracle
import parity_util
from parity_util import check_unit_codes


def test_unit_code_check_accepts_band_flips_only():
    rng = np.random.default_rng(3)
    k = rng.standard_normal((700, 128))
    W = oracle.hyperplanes(seed=4, R=10 * 30, d=128)
    # put key 5 almost on hyperplane 7 (table 0, bit 7) so that bit is in the band
    w = W[7].astype(np.float64)
    k[5] -= (w @ k[5]) / (w @ w) * w * (1 - 1e-9)
    ref, band, nb = oracle.encode_keys_band(k, W, 10, 30)
    assert nb >= 1 and band[0, 5] & (1 << 7)
    assert check_unit_codes(ref, band, ref.copy(), "same") == (0, nb)
    got = ref.copy()
    got[0, 5] ^= 1 << 7                        # inside the band: allowed, counted
    assert check_unit_codes(ref, band, got, "band flip") == (1, nb)
    l, i = np.argwhere(band == 0)[0]
    got[l, i] ^= 1                             # outside the band: refused
    with pytest.raises(AssertionError, match="outside the band"):
        check_unit_codes(ref, band, got, "planted")


def test_elementwise_error_has_a_floor():
    ref = np.array([1.0, -2.0, 1e-9, 0.0])
    got = ref + np.array([1e-3, 0.0, 1e-6, 0.0])
    # element 2: |1e-6| / max(1e-9, 1e-3 * 2) = 5e-4; element 0: 1e-3 / 1 = 1e-3
    assert np.isclose(parity_util.elem_rel_err(got, ref), 1e-3)
    assert parity_util.elem_rel_err(ref, ref) == 0.0
    assert parity_util.elem_rel_err(np.ones(3), np.zeros(3)) == 1.0
