"""The main-loop schedule probe (coda_baseline_schedule_probe) on the GPU: with every LDS
element equal to one bf16 value c, each of a thread's 128 accumulator values gains
32 c^2 per step, and the reads-only kind adds 48 words (two bf16 c each) per step; both
sums are exact in their arithmetic for c = 1/8, so they are checked bit for bit. Step counts
that are not a multiple of the ring's 5 slots exercise the remainder steps. With a hashed
image every workgroup must still compute the same values, and a different seed others.
The kind with the zero-filling DMA runs on the all-zero image only: its sums are exactly 0."""
import numpy as np
import pytest

from gpu_util import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def coda():
    import torch
    import transformer_gemm_epilogue_amd as c
    assert torch.cuda.is_available()
    c.lib()
    return c


@pytest.mark.parametrize("kind", [0, 1, 2, 3, 4, 5, 6])
def test_schedule_probe_closed_form(coda, kind):
    import torch
    for steps, grid in ((1, 1), (7, 3), (23, 2)):
        log(f"schedule probe kind={kind} steps={steps} grid={grid}")
        out, cycles = coda.coda_baseline_schedule_probe(kind, steps, grid, fill=0.125)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        if kind != 3:
            assert np.all(got == np.float32(128 * 32 * 0.125 ** 2 * steps))
        else:
            word = 0x3E00 * 0x10001          # two bf16(1/8) per 32-bit word
            want = (48 * steps * word) % (1 << 32)
            assert np.all(got.view(np.uint32) == want)
        assert bool((cycles > 0).all())


@pytest.mark.parametrize("kind", [0, 2, 3, 4, 5, 6])
def test_schedule_probe_hashed_image(coda, kind):
    import torch
    log(f"schedule probe hashed kind={kind}")
    a, ca = coda.coda_baseline_schedule_probe(kind, 12, 4, seed=7)
    b, _ = coda.coda_baseline_schedule_probe(kind, 12, 4, seed=8)
    torch.cuda.synchronize()
    a = a.cpu().numpy().reshape(4, 512)
    b = b.cpu().numpy().reshape(4, 512)
    assert np.all(a.view(np.uint32) == a[:1].view(np.uint32))
    assert not np.array_equal(a.view(np.uint32), b.view(np.uint32))
    if kind != 3:
        assert np.all(np.isfinite(a))
    assert bool((ca > 0).all())


def test_schedule_probe_zero_fill_dma(coda):
    import torch
    for steps, grid in ((1, 1), (7, 3), (23, 2), (400, 256)):
        log(f"schedule probe kind=7 steps={steps} grid={grid}")
        out, cycles = coda.coda_baseline_schedule_probe(7, steps, grid, fill=0.0, seed=0)
        torch.cuda.synchronize()
        assert np.all(out.cpu().numpy() == 0.0)
        assert bool((cycles > 0).all())
