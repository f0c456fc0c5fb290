"""The device cast over every fp32 bit pattern, and the device decode of
every 16-bit code, through the C ABI.

A step with lr = 0, weight decay 0 and zero gradients leaves every master
unchanged (p * 1 - 0 * 0), so the parameters it writes are the cast alone.
All 2^32 fp32 patterns go through it as masters, four chunks of 2^30, in
both formats, and each code is compared with torch's round-to-nearest-even
cast of the same pattern on the device (NaN must stay NaN): subnormals, the
overflow edges, infinities and NaN payloads included."""
import pytest
import torch

import zero_sharded_optimizer_step_amd as Z  # noqa: F401  (the library path is what runs)
from zero_sharded_optimizer_step_amd.world import Hyper, SimulatedWorld

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("pdt", [torch.bfloat16, torch.float16])
def test_device_cast_of_every_fp32_pattern(pdt):
    chunk = 1 << 30
    print("device cast, every fp32 pattern, %s" % pdt, flush=True)
    world = SimulatedWorld(chunk, 1, n_replicas=1, alignment=8, grad_dtype=torch.bfloat16,
                           param_dtype=pdt)
    hp = Hyper(lr=0.0, weight_decay=0.0, max_grad_norm=0.0)
    idx = torch.arange(chunk, dtype=torch.int32, device="cuda")
    for c in range(4):
        start = c * chunk
        pat = idx + (start - (1 << 32) if start >= (1 << 31) else start)   # int32 wraps
        world.master[0].view(torch.int32).copy_(pat)
        world.exp_avg[0].zero_()
        world.exp_avg_sq[0].zero_()
        world.step(hp, 1)
        res = world.result()
        assert not res.overflow
        x = pat.view(torch.float32)
        got = world.full_params.view(torch.int16)
        ref = x.to(pdt).view(torch.int16)
        nan = torch.isnan(x)
        same = (got == ref) | nan
        if not bool(same.all()):
            bad = torch.nonzero(~same)[:5].flatten()
            raise AssertionError("chunk %d: patterns %s give %s, torch gives %s" % (
                c, [hex(int(v) & 0xFFFFFFFF) for v in pat[bad].tolist()],
                [hex(int(v) & 0xFFFF) for v in got[bad].tolist()],
                [hex(int(v) & 0xFFFF) for v in ref[bad].tolist()]))
        assert bool(world.full_params[nan].isnan().all()), "a NaN pattern lost its NaN"
        print("  chunk %d of 4 agrees" % (c + 1), flush=True)
        del pat, x, got, ref, nan, same
    del world
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16])
def test_device_decode_of_every_16_bit_code(dt):
    # One replica holding every code, reduced at scale 1: the fp32 slice is
    # each code widened, exactly (NaN codes widen to NaN), and the flag is
    # raised by the inf and NaN codes.
    n = 1 << 16
    print("device decode, every %s code" % dt, flush=True)
    world = SimulatedWorld(n, 1, n_replicas=1, alignment=8, grad_dtype=dt)
    codes = torch.arange(n, dtype=torch.int32, device="cuda").to(torch.int16)
    world.grads[0].view(torch.int16).copy_(codes)
    world.step(Hyper(), 1)
    assert world.result().overflow
    g = world.reduced_grad(0)[:n]
    ref = codes.view(dt).float()
    nan = torch.isnan(ref)
    assert torch.equal(g[~nan].view(torch.int32), ref[~nan].view(torch.int32))
    assert bool(torch.isnan(g[nan]).all())
