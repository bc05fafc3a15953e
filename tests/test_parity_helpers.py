"""The parity helper's diagnostics beside the gates (tests/parity.py)."""
import numpy as np

import parity


def test_parity_diagnostic_counts_bf16_spacings():
    """The comparison helper's diagnostic beside the gate: an element counts
    when it is more than 30 bf16 spacings (2^(floor(log2 |v|) - 7)) from the
    reference; exact results count none."""
    want = np.array([1.0, 1.0, 1.5, -3.0, 0.0, 1024.0])
    got = want.copy()
    got[0] += 30.5 * 2.0 ** -7          # just beyond 30 spacings of 1.0
    got[1] += 29.5 * 2.0 ** -7          # just inside
    got[3] -= 31 * 2.0 ** -6            # -3.0 sits in [2, 4): spacing 2^-6
    got[5] += 20 * 8.0                  # 1024: spacing 8, inside
    info = parity.close(got, want, 1.0, 1.0, "diagnostic")
    assert info["n_over_30ulp_bf16"] == 2
    assert parity.close(want, want, 0.0, 0.0, "exact")["n_over_30ulp_bf16"] == 0
