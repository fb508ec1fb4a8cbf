"""The 2 MB-aligned arena (host logic; runs on a CPU tensor)."""
import pytest
import torch

from cg_streaming_vector_amd.arena import ALIGN, Arena


def test_arena_alignment_and_order():
    a = Arena(3 * ALIGN + 5 * ALIGN, "cpu")
    x = a.empty(1000, torch.float64)
    y = a.empty(ALIGN // 8 + 1, torch.float64)  # spills into a second slot
    z = a.put(torch.arange(10, dtype=torch.int32))
    assert x.data_ptr() % ALIGN == 0 and y.data_ptr() % ALIGN == 0 and z.data_ptr() % ALIGN == 0
    assert y.data_ptr() - x.data_ptr() == ALIGN
    assert z.data_ptr() - y.data_ptr() == 2 * ALIGN
    assert torch.equal(z, torch.arange(10, dtype=torch.int32))
    # the slots are distinct memory: filling one leaves its neighbours alone
    y.fill_(-2.0)
    x.fill_(1.5)
    assert float(y[0].item()) == -2.0 and float(y[-1].item()) == -2.0
    assert torch.equal(z, torch.arange(10, dtype=torch.int32))
    assert float(x[-1].item()) == 1.5
    assert Arena.slot(1) == ALIGN and Arena.slot(ALIGN) == ALIGN and Arena.slot(ALIGN + 1) == 2 * ALIGN


def test_arena_padding():
    a = Arena(8 * ALIGN, "cpu")
    x = a.empty(4 * ALIGN // 8, torch.float64, pad=1)  # a power-of-two size, one granule of padding
    y = a.empty(10, torch.float64)
    assert y.data_ptr() - x.data_ptr() == 5 * ALIGN


def test_arena_exhausted():
    a = Arena(ALIGN, "cpu")
    a.empty(10, torch.float64)
    with pytest.raises(MemoryError):
        a.empty(10, torch.float64)
