"""The allocation-free weight quantization (bitlinear_quantize_weights_grouped_noalloc, its
partial sums in the library's fixed scratch) against the workspace form on the same weights,
through the C ABI: two calls in a row, the second with a smaller input, packed words and gamma
bit for bit.  Also refused: a problem count past the scratch's room (BL_MAX_GROUP)."""

import ctypes

import numpy as np
import pytest

import workloads

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


def _problems(bl, Ws, outs):
    arr = (bl._WeightProblem * len(Ws))()
    for i, (W, (P, g)) in enumerate(zip(Ws, outs)):
        arr[i] = bl._WeightProblem(W.data_ptr(), P.data_ptr(), g.data_ptr(), W.shape[0], W.shape[1])
    return arr


def _outputs(torch, Ws, fill):
    return [(torch.full((W.shape[0], W.shape[1] // 16), fill, dtype=torch.int32, device="cuda"),
             torch.full((1,), float(fill), dtype=torch.float32, device="cuda")) for W in Ws]


def test_noalloc_matches_workspace_form(torch, bl):
    L = bl.lib()
    stream = torch.cuda.current_stream().cuda_stream
    # Call 1: a Qwen3-4B-shaped set (seven tensors, the largest 9728 x 2560); call 2: two
    # smaller ragged tensors, so the second call uses fewer partial sums than the first left.
    sets = [[(4096, 2560), (1024, 2560), (1024, 2560), (2560, 4096), (9728, 2560), (9728, 2560),
             (2560, 9728)],
            [(300, 272), (17, 1040)]]
    for c, shapes in enumerate(sets):
        Ws = [torch.from_numpy(workloads.gaussian(s, (700, c, i), 0.02)).cuda() for i, s in enumerate(shapes)]
        ref = _outputs(torch, Ws, 0)
        ws = torch.empty(bl.quantize_weights_workspace_bytes(len(Ws)), dtype=torch.uint8, device="cuda")
        arr_ref = _problems(bl, Ws, ref)      # kept alive across the call
        rc = L.bitlinear_quantize_weights_grouped(ctypes.addressof(arr_ref), len(Ws), ws.data_ptr(),
                                                  ws.numel(), stream)
        assert rc == 0, rc
        got = _outputs(torch, Ws, 7)
        arr_got = _problems(bl, Ws, got)
        rc = L.bitlinear_quantize_weights_grouped_noalloc(ctypes.addressof(arr_got), len(Ws), stream)
        assert rc == 0, rc
        torch.cuda.synchronize()
        for i, ((P, g), (Pr, gr)) in enumerate(zip(got, ref)):
            assert torch.equal(P, Pr), (c, i)
            assert torch.equal(g, gr), (c, i, float(g), float(gr))


def test_noalloc_refuses_past_the_scratch(torch, bl):
    L = bl.lib()
    W = torch.zeros((16, 16), dtype=torch.float32, device="cuda")
    outs = _outputs(torch, [W] * 17, 0)
    arr = _problems(bl, [W] * 17, outs)
    assert L.bitlinear_quantize_weights_grouped_noalloc(ctypes.addressof(arr), 17, None) == -7
    assert L.bitlinear_quantize_weights_grouped_noalloc(None, 1, None) == -1
