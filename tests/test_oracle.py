"""The CPU oracle against its pins (no GPU needed)."""
import pytest

import oracle
import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle._load())


def test_dense_bruteforce_vs_library():
    P.pin_dense_vs_library()


def test_oracle_rejects_bad_tables():
    import torch
    q = torch.zeros(1, 2, 4)
    kc = torch.zeros(3, 1, 2, 4)
    with pytest.raises(ValueError):   # block id outside the pool inside the used range
        oracle.paged_attention(q, kc, kc, torch.tensor([[0, 7]], dtype=torch.int32),
                               torch.tensor([3], dtype=torch.int32), 1.0)
    with pytest.raises(ValueError):   # context longer than its table
        oracle.paged_attention(q, kc, kc, torch.tensor([[0, 1]], dtype=torch.int32),
                               torch.tensor([5], dtype=torch.int32), 1.0)
    # padding (-1) beyond the used blocks is never read
    out = oracle.paged_attention(q, kc, kc, torch.tensor([[0, -1]], dtype=torch.int32),
                                 torch.tensor([2], dtype=torch.int32), 1.0)
    assert out.shape == (1, 2, 4)
