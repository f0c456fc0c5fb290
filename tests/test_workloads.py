"""CPU tests of the seeded input generators (no method arithmetic here)."""
import torch

from zero_sharded_optimizer_step_amd import workloads as W


def test_flat_normal_slices_agree_and_pad_with_zeros(monkeypatch):
    monkeypatch.setattr(W, "CHUNK", 64)          # many chunks on a small tensor
    total = 1000
    whole = torch.empty(1100, dtype=torch.float32)
    W.flat_normal(whole, 0, total, 1.0, ("k",))
    assert (whole[total:] == 0).all() and (whole[:total] != 0).all()
    for lo, n in ((0, 1), (63, 2), (64, 64), (500, 600), (999, 1), (1000, 8), (1200, 8)):
        part = torch.full((n,), 7.0)
        W.flat_normal(part, lo, total, 1.0, ("k",))
        ref = torch.zeros(n)
        if lo < 1100:
            m = min(n, 1100 - lo)
            ref[:m] = whole[lo:lo + m]
        assert torch.equal(part, ref), (lo, n)


def test_flat_normal_keys_differ_and_repeat():
    a = W.flat_normal(torch.empty(100), 0, 100, 1.0, ("a",))
    b = W.flat_normal(torch.empty(100), 0, 100, 1.0, ("b",))
    c = W.flat_normal(torch.empty(100), 0, 100, 1.0, ("a",))
    assert torch.equal(a, c) and not torch.equal(a, b)


def test_poison_schedule_and_ragged_sizes():
    s = W.poison_schedule(200, 4, 50_000_000, 0.05, 0)
    hits = [p for p in s if p is not None]
    assert 2 <= len(hits) <= 25
    assert all(0 <= p.replica < 4 and 0 <= p.index < 50_000_000 and p.kind in (0, 1, 2) for p in hits)
    assert s == W.poison_schedule(200, 4, 50_000_000, 0.05, 0)
    sizes = W.ragged_sizes()
    assert len(sizes) == 2000 and min(sizes) >= 1000 and max(sizes) < 10**7
    assert 1.9e9 < sum(sizes) < 2.5e9


def test_plant_writes_nonfinite_codes():
    for dt in (torch.float16, torch.bfloat16):
        for kind, check in ((0, lambda x: x == float("inf")), (1, lambda x: x == float("-inf")),
                            (2, lambda x: x != x)):
            t = torch.zeros(10, dtype=dt)
            W.plant(t, W.Poison(0, 0, 3, kind))
            assert check(float(t[3])) and (t[:3] == 0).all()
