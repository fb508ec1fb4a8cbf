"""Host logic of the Python binding that runs without a GPU: how shared
contexts are keyed, and argument checks that must fire before anything is
enqueued."""
import pytest
import torch

import cg_streaming_vector_amd as bs


class _FakeContext:
    made = []

    def __init__(self, device):
        self.device = device
        _FakeContext.made.append(device)


def test_shared_contexts_are_keyed_by_device_and_stream(monkeypatch):
    monkeypatch.setattr(bs, "Context", _FakeContext)
    monkeypatch.setattr(bs, "_contexts", {})
    _FakeContext.made.clear()
    a = bs._shared_context(0, 0x1000)
    assert bs._shared_context(0, 0x1000) is a
    b = bs._shared_context(0, 0x2000)
    c = bs._shared_context(1, 0x1000)
    d = bs._shared_context(0, None)  # the null (default) stream
    assert len({id(a), id(b), id(c), id(d)}) == 4
    assert bs._shared_context(0, 0) is d
    assert _FakeContext.made == [0, 0, 1, 0]
    assert c.device == 1


def _cg_args(ng=6, nl=8, hist=None, iters=3):
    f = lambda n: torch.zeros(n, dtype=torch.float64)  # noqa: E731
    i = lambda n: torch.zeros(n, dtype=torch.int32)  # noqa: E731
    return (i(nl), i(ng + 1), i(nl), f(ng), f(ng), f(ng), f(ng), f(nl), iters), hist


def test_cg_solve_rejects_a_short_history_before_any_launch(monkeypatch):
    def no_lib():
        raise AssertionError("the library was reached")
    monkeypatch.setattr(bs, "_lib", no_lib)
    args, _ = _cg_args()
    for n in (0, 1, 3):
        with pytest.raises(ValueError, match="rr_hist"):
            bs.bs_cg_solve(*args, rr_hist=torch.zeros(n, dtype=torch.float64))
    with pytest.raises(ValueError, match="iters"):
        bs.bs_cg_solve(*args[:-1], -1)
    with pytest.raises(ValueError, match="inconsistent"):
        bs.bs_cg_solve(*_cg_args(ng=5)[0][:3], *[torch.zeros(6, dtype=torch.float64)] * 4,
                       torch.zeros(8, dtype=torch.float64), 3)


def test_a_plan_of_the_wrong_shape_is_rejected_before_any_launch(monkeypatch):
    """A gather plan is (n_blocks, 4) int32 blocks; row starts alone, or pairs,
    would make the kernel read past the array, so the binding refuses them
    before it reaches the library."""
    def no_lib():
        raise AssertionError("the library was reached")
    monkeypatch.setattr(bs, "_lib", no_lib)
    for bad in (torch.zeros(5, dtype=torch.int32), torch.zeros((5, 2), dtype=torch.int32),
                torch.zeros((0, 4), dtype=torch.int32)):
        with pytest.raises(ValueError, match="block_starts"):
            bs._plan_dev(bad)
    assert bs._plan_dev(None) == (None, 0)
    with pytest.raises(ValueError, match="block_starts"):
        bs.bs_bench_loop("gather", 4, [(torch.zeros(5, dtype=torch.int32), torch.zeros(3, dtype=torch.int32),
                                        torch.zeros(3, dtype=torch.float64), torch.zeros(4, dtype=torch.float64),
                                        torch.zeros((2, 2), dtype=torch.int32))], 1, n_blocks=2)
