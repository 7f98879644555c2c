"""The CPU oracle against facts fixed by the pages and by mathematics."""
import pytest

import oracle
from tests import oracle_pins


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check(oracle.default())


def test_bf16_bit_rule_matches_torch():
    """The pins' bfloat16 rule against torch's own fp32 -> bfloat16 conversion
    (a library routine), so the pins do not rest on the rule alone."""
    import numpy as np
    import torch
    rng = np.random.default_rng(21)
    bits = rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[~np.isnan(v)]
    want = torch.from_numpy(v.copy()).to(torch.bfloat16).to(torch.float32).numpy()
    got = oracle_pins.round16_ref(oracle_pins.BF16, v)
    assert np.array_equal(got.view(np.int32), want.view(np.int32))
