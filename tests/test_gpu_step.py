"""Weight and activation quantization of one step in one call (bitlinear_quantize_step): codes,
gamma, activation codes and scales equal bit for bit to the two grouped calls it replaces, and
checked against the CPU oracle (gamma within 1e-6 with codes exact away from the rounding
boundary, activation codes exact and scales within 1e-6).  Cases: the Distillix-125M layer set's
weights with 2048-token inputs (the benchmark's step), ragged and bf16 inputs with a norm, inputs
longer than 4096 (two launches of their own), and one set empty.
"""

import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu

REL = 1e-6


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


def dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b) / np.maximum(np.abs(b), 1e-300))) if a.size else 0.0


def make(torch, w_shapes, x_specs, key):
    Ws = [workloads.gaussian(s, (330, i) + key, 0.02) for i, s in enumerate(w_shapes)]
    Xs, xin, gs = [], [], []
    for i, (M, K, dt, nm) in enumerate(x_specs):
        X = workloads.gaussian((M, K), (331, i) + key, 1.0)
        g = (np.float32(1) + workloads.gaussian((K,), (332, i) + key, 0.1)) if nm else None
        if dt == "bf16":
            bits = workloads.f32_to_bf16_bits(X)
            Xs.append(dev(torch, bits.view(np.int16)).view(torch.bfloat16))
            xin.append((bits, g, True))
        else:
            Xs.append(dev(torch, X))
            xin.append((X, g, False))
        gs.append(None if g is None else dev(torch, g))
    return Ws, [dev(torch, W) for W in Ws], xin, Xs, gs


def check(torch, bl, orc, w_shapes, x_specs, key):
    Ws_h, Ws, xin, Xs, gs = make(torch, w_shapes, x_specs, key)
    wo, xo = bl.quantize_step(Ws, Xs, gs, 1e-6)
    wo2 = bl.quantize_weights_grouped(Ws) if Ws else []
    xo2 = bl.quantize_acts_grouped(Xs, gs, 1e-6) if Xs else []
    torch.cuda.synchronize()
    for i, ((P, g), (P2, g2)) in enumerate(zip(wo, wo2)):
        assert torch.equal(P, P2) and torch.equal(g, g2), ("weights", key, i)
        gref, _ = orc.gamma(Ws_h[i])
        assert rel_err(g.cpu().numpy(), np.float32(gref)) <= REL, ("gamma", key, i)
    for i, ((q, s), (q2, s2)) in enumerate(zip(xo, xo2)):
        assert torch.equal(q, q2) and torch.equal(s, s2), ("acts", key, i)
        x, g, bf = xin[i]
        q_ref, s_ref = orc.quantize_acts(x, g, 1e-6, bf16=bf)
        assert np.array_equal(q.cpu().numpy(), q_ref), ("codes", key, i)
        sn = s.cpu().numpy()
        nz = s_ref != 0
        assert np.array_equal(sn == 0, ~nz) and rel_err(sn[nz], s_ref[nz]) <= REL, ("scales", key, i)


def test_step_distillix_layer(torch, bl, orc):
    wl = workloads.WORKLOADS["c2_distillix125m_layer"]
    check(torch, bl, orc, [(m.N, m.K) for m in wl.matrices],
          [(2048, m.K, "f32", False) for m in wl.matrices], (1,))


def test_step_ragged_bf16_norm(torch, bl, orc):
    check(torch, bl, orc, [(300, 272), (17, 1040), (1, 16)],
          [(130, 272, "bf16", True), (1, 1040, "bf16", False), (33, 4096, "bf16", True)], (2,))


@pytest.mark.parametrize("case", [0, 1, 2, 3])
def test_step_two_launch_cases(torch, bl, orc, case):
    """Rows longer than 4096, mixed dtypes, no activations, no weights."""
    w = [(256, 768), (64, 512)]
    x = [(64, 768, "f32", True)]
    if case == 0:
        x = x + [(8, 8192, "f32", False)]
    elif case == 1:
        x = x + [(8, 512, "bf16", False)]
    elif case == 2:
        x = []
    else:
        w = []
    check(torch, bl, orc, w, x, (3, case))
