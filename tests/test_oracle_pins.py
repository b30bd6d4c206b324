"""The fp64 oracle against the pins in oracle_pins.py (CPU only)."""
import pytest

import oracle.attention as A
import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(A)


def test_fd_every_entry_gqa_window():
    P.pin_fd_every_entry(A, Hq=4, Hkv=2, S=16, D=8, window=5, seed=9)


def test_fd_sampled_tiny_workload_shape():
    P.pin_fd_sampled(A)


def test_visible_mask_reading():
    # window W counts the diagonal: W=1024 lets query i see keys max(0, i-1023) .. i
    m = A.visible_mask([0, 1023, 1024, 5000], range(6000), True, 1024)
    assert m[0].sum() == 1 and m[0, 0]
    assert m[1].sum() == 1024 and m[1, 0] and m[1, 1023]
    assert m[2].sum() == 1024 and not m[2, 0] and m[2, 1] and m[2, 1024]
    assert m[3].sum() == 1024 and m[3, 3977] and not m[3, 3976] and not m[3, 5001]
    with pytest.raises(ValueError):
        A.forward_backward(*(P._rng_inputs(0, 1, 2, 2, 4, 2)[:3]), None, False, 3, 1.0)
    with pytest.raises(ValueError):
        A.forward_backward(*(P._rng_inputs(0, 1, 3, 2, 4, 2)[:3]), None, True, 0, 1.0)


def test_kv_head_contiguous_groups():
    assert [A.kv_head(h, 64, 8) for h in range(0, 64, 7)] == [0, 0, 1, 2, 3, 4, 5, 6, 7, 7]
