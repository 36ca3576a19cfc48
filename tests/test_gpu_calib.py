"""Measurement helpers on the GPU: the read-stream calibration reads every word of its buffer
(its XOR equals the host's) and the matrix-unit loop performs exactly the operations it
reports (its sums have a closed form: iterations x chains x the operand dot product)."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as t
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    return t


@pytest.fixture(scope="module")
def bl(torch):
    import bit_gemm_02_amd as m
    m.lib()
    return m


@pytest.mark.parametrize("nbytes", [16, 4096 * 16 + 48, 1 << 24, (1 << 26) + 16 * 7])
def test_calib_stream_reads_every_word(torch, bl, nbytes):
    g = torch.Generator(device="cpu").manual_seed(nbytes)
    x = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, generator=g)
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    bl.calib_stream(x.cuda(), out)
    torch.cuda.synchronize()
    ref = np.bitwise_xor.reduce(x.numpy().view(np.uint32))
    assert out.cpu().numpy().view(np.uint32)[0] == ref


@pytest.mark.parametrize("kind,per_step", [(0, 64), (1, 32)])
def test_calib_mfma_closed_form(torch, bl, kind, per_step):
    blocks, iters = 3, 100
    out = torch.full((256 * blocks,), -1, dtype=torch.int32, device="cuda")
    ops = bl.calib_mfma(kind, iters, blocks, out)
    torch.cuda.synchronize()
    assert ops == blocks * 4 * 8 * iters * (32768 if kind == 0 else 16384)
    assert bool((out == 8 * iters * per_step).all())
