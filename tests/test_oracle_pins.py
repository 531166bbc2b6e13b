"""The fp64 oracle against its pins (CPU only)."""

import pytest

from oracle_checks import ALL_CHECKS


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(orc, check):
    check(orc)


def test_oracle_rejects_bad_problems(orc):
    import numpy as np

    q = np.zeros((1, 3, 2, 4))
    k = np.zeros((1, 2, 2, 4))
    with pytest.raises(ValueError):
        orc.forward(q, k, k)  # Hq % Hkv != 0
    q = np.zeros((1, 2, 2, 4))
    with pytest.raises(ValueError):
        orc.forward(q, k, k, len_kv=[3])  # length past Lk
    m = np.zeros((1, 1, 2, 2))
    m[0, 0, 0, 1] = np.inf
    with pytest.raises(ValueError):
        orc.forward(q, k, k, mask=m)  # +inf is not an additive -inf mask
