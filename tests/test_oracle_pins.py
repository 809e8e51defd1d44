"""The oracle against what the pages and mathematics fix (CPU only)."""
import pytest

import pins


@pytest.mark.parametrize("check", pins.ALL, ids=lambda f: f.__name__)
def test_pin(check):
    check()


@pytest.mark.parametrize("seed", [11, 12, 13])
def test_pins_more_seeds(seed):
    pins.check_attention_library(seed)
    pins.check_bias_closed_form(seed)
    pins.check_split_merge(seed)
    pins.check_evict_bruteforce(seed, trials=25)
    pins.check_lookup_bruteforce(seed)
