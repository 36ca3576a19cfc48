"""GPU path vs the CPU oracle, element by element, through the C ABI.

Stage-wise parity (one legal code flip must not cascade):
  * gamma: relative error <= 1e-6 (the fp64 sums differ only in order);
  * packed codes: bit-exact against the oracle's codes computed with the GPU's gamma, and
    against the oracle's own gamma except where |W / gamma| lies within 1e-6 of 0.5 (counted);
  * int8 activations: bit-exact; scales: relative error <= 1e-6 (bit-exact without the norm);
  * int32 accumulators: bit-exact against the oracle run on the GPU's own packed weights and
    int8 activations;
  * fp32 outputs: relative error <= 1e-6 against the oracle epilogue on the same inputs, and
    exactly zero where the oracle gives zero.
Sizes here span several tiles and ragged tails; full workload sizes are in test_gpu_workloads.
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


def host(t):
    return t.cpu().numpy()


def words(t):
    return host(t).view(np.uint32)


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.maximum(np.abs(b), 1e-300)
    return np.max(np.abs(a - b) / den) if a.size else 0.0


def check_weights(torch, bl, orc, W, label=""):
    P, g = bl.quantize_weights(dev(torch, W))
    torch.cuda.synchronize()
    g_gpu = np.float32(host(g)[0])
    g_orc, g64 = orc.gamma(W)
    assert rel_err(g_gpu, g_orc) <= REL, (label, g_gpu, g_orc)
    # Bit-exact against the oracle's codes with the GPU's gamma.
    ref = orc.pack(orc.ternary_codes(W, g_gpu))
    assert np.array_equal(words(P), ref), label
    # Against the oracle's own gamma: flips only inside the 1e-6 band around 0.5.
    codes_gpu = orc.unpack(words(P), W.shape[1])
    codes_orc = orc.ternary_codes(W, g_orc)
    flips = codes_gpu != codes_orc
    if flips.any():
        t = np.abs(W.astype(np.float64) / g64)
        assert np.all(np.abs(t[flips] - 0.5) <= 1e-6), label
    return P, g, int(flips.sum())


@pytest.mark.parametrize("N,K", [(1, 16), (3, 48), (37, 80), (130, 272), (257, 1040),
                                 (64, 4096), (2048, 768)])
def test_quantize_weights(torch, bl, orc, N, K):
    W = workloads.gaussian((N, K), (100, N, K), 0.02)
    check_weights(torch, bl, orc, W, f"{N}x{K}")


def test_quantize_weights_special(torch, bl, orc):
    # Exact ties at |W / gamma| = 0.5 (gamma = 2).
    W = np.tile(np.array([1, -1, 3, 3], np.float32), (5, 8))
    P, g, _ = check_weights(torch, bl, orc, W, "ties")
    assert host(g)[0] == 2.0
    assert np.array_equal(orc.unpack(words(P), 32), np.tile(np.array([0, 0, 1, 1], np.int8), (5, 8)))
    # All zero: gamma = 0, codes 0.
    Z = np.zeros((7, 48), np.float32)
    P, g, _ = check_weights(torch, bl, orc, Z, "zeros")
    assert host(g)[0] == 0.0 and not words(P).any()
    # alpha * C round-trips to C.
    Cm = workloads.ternary((33, 96), (101,))
    P, _, _ = check_weights(torch, bl, orc, (np.float32(0.021) * Cm).astype(np.float32), "alphaC")
    assert np.array_equal(orc.unpack(words(P), 96), Cm)
    # Subnormal and huge magnitudes mixed with ordinary ones.
    S = workloads.gaussian((9, 64), (102,), 0.02)
    S[0, :8] = np.float32(1e-40)
    S[1, :4] = np.float32(3e38)
    check_weights(torch, bl, orc, S, "extremes")
    # gamma computed from data whose mean underflows to zero in fp32 (all codes must be 0).
    U = np.zeros((1, 16000), np.float32)
    U[0, 0] = np.float32(1.4e-45)
    P, g, _ = check_weights(torch, bl, orc, U, "underflow")
    assert host(g)[0] == 0.0 and not words(P).any()


def test_quantize_weights_deterministic(torch, bl):
    W = dev(torch, workloads.gaussian((1000, 1024), (103,), 0.02))
    P1, g1 = bl.quantize_weights(W)
    P2, g2 = bl.quantize_weights(W)
    assert torch.equal(P1, P2) and torch.equal(g1, g2)


def test_quantize_weights_empty(torch, bl):
    W = torch.empty((0, 64), dtype=torch.float32, device="cuda")
    P, g = bl.quantize_weights(W, gamma=torch.full((1,), 7.0, device="cuda"))
    assert host(g)[0] == 0.0 and P.numel() == 0


def test_quantize_weights_grouped_equals_single(torch, bl):
    shapes = [(64, 256), (17, 48), (300, 1024), (1, 16)]
    Ws = [dev(torch, workloads.gaussian(s, (104, i), 0.02)) for i, s in enumerate(shapes)]
    outs = bl.quantize_weights_grouped(Ws)
    for W, (P, g) in zip(Ws, outs):
        P1, g1 = bl.quantize_weights(W)
        assert torch.equal(P, P1) and torch.equal(g, g1)


@pytest.mark.parametrize("N,K", [(1, 16), (5, 48), (129, 256), (1000, 1040)])
def test_pack_codes(torch, bl, orc, N, K):
    Cm = workloads.ternary((N, K), (105, N, K))
    P = bl.pack_codes(dev(torch, Cm))
    assert np.array_equal(words(P), orc.pack(Cm))


ACT_SHAPES = [(1, 16), (1, 768), (3, 80), (16, 2048), (37, 272), (64, 9728), (5, 16384)]


@pytest.mark.parametrize("M,K", ACT_SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("norm", [False, True])
def test_quantize_acts(torch, bl, orc, M, K, dtype, norm):
    X = workloads.gaussian((M, K), (106, M, K), 1.0)
    if M > 2:
        X[1] = 0.0                     # all-zero row
        X[2] = 0.0
        X[2, K // 3] = -3.25           # one-hot row
    g = (np.float32(1) + workloads.gaussian((K,), (107, K), 0.1)) if norm else None
    if dtype == "bf16":
        bits = workloads.f32_to_bf16_bits(X)
        Xt = dev(torch, bits.view(np.int16)).view(torch.bfloat16)
        q_ref, s_ref = orc.quantize_acts(bits, g, 1e-6, bf16=True)
    else:
        Xt = dev(torch, X)
        q_ref, s_ref = orc.quantize_acts(X, g, 1e-6)
    q, s = bl.quantize_acts(Xt, None if g is None else dev(torch, g), 1e-6)
    torch.cuda.synchronize()
    assert np.array_equal(host(q), q_ref)
    if norm:
        assert rel_err(host(s)[s_ref != 0], s_ref[s_ref != 0]) <= REL
        assert np.array_equal(host(s) == 0, s_ref == 0)
    else:
        assert np.array_equal(host(s), s_ref)


def test_quantize_acts_edge_values(torch, bl, orc):
    X = workloads.gaussian((6, 64), (108,), 1.0)
    X[0, :] = 1e-40                    # subnormal row
    X[1, 5] = 3e38                     # huge element
    X[2] = np.array([127.0, 0.5, 1.5, 2.5, -3.5, -127.0, 0.25, 126.5] * 8, np.float32)  # ties
    X[3, :] = -0.0
    X[4, :] = 2.0 ** -130              # subnormal absmax, 127 / a overflows to inf
    X[4, 7] = 0.0
    q_ref, s_ref = orc.quantize_acts(X)
    q, s = bl.quantize_acts(dev(torch, X))
    assert np.array_equal(host(q), q_ref)
    assert np.array_equal(host(s), s_ref)


def test_quantize_acts_grouped_equals_single(torch, bl):
    Xs = [dev(torch, workloads.gaussian((m, k), (109, m, k), 1.0)) for m, k in
          [(3, 64), (1, 768), (40, 2048)]]
    gs = [None, dev(torch, np.ones(768, np.float32)), None]
    outs = bl.quantize_acts_grouped(Xs, gs, 1e-6)
    for X, g, (q, s) in zip(Xs, gs, outs):
        q1, s1 = bl.quantize_acts(X, g, 1e-6)
        assert torch.equal(q, q1) and torch.equal(s, s1)


FWD_SHAPES = [
    (1, 16, 16), (1, 50, 48), (1, 768, 768), (1, 257, 2048), (1, 64, 9728),
    (3, 33, 80), (8, 1536, 1536), (16, 2048, 768), (16, 100, 272),
    (17, 40, 64), (100, 130, 272), (129, 129, 1040), (256, 512, 768), (300, 257, 4096),
    (517, 1000, 1536),
    # Decode launch variants: activations staged in LDS up to its byte limit, and the
    # two- and four-row-group blocks that large layers get, with K a multiple of 256 or not.
    (4, 70, 12288), (2, 16400, 1040), (6, 8200, 80), (5, 16448, 272), (12, 16400, 512),
]


@pytest.mark.parametrize("M,N,K", FWD_SHAPES)
def test_forward(torch, bl, orc, M, N, K):
    W = workloads.gaussian((N, K), (110, M, N, K), 0.02)
    X = workloads.gaussian((M, K), (111, M, N, K), 1.0)
    Pt, gt = bl.quantize_weights(dev(torch, W))
    Xq, sx = bl.quantize_acts(dev(torch, X))
    Y, acc = bl.forward(Xq, sx, Pt, gt, return_acc=True)
    torch.cuda.synchronize()
    acc_ref, Y_ref = orc.forward(host(Xq), host(sx), words(Pt), host(gt)[0])
    assert np.array_equal(host(acc), acc_ref), (M, N, K)
    Yh = host(Y)
    assert np.array_equal(Yh == 0, Y_ref == 0)
    assert rel_err(Yh[Y_ref != 0], Y_ref[Y_ref != 0]) <= REL


# Shapes whose products have full tiles, so that without the int32 copy they take the
# straight-line epilogue (whole 128-byte row segments, lanes r and r ^ 8 exchanging pieces):
# 128 x 128 tiles with a row pitch that is not a multiple of 128 bytes (N = 260, 2060) and
# ragged last tiles, and 128 x 256 tiles (at least 256 units of 256 x 256 outputs), one set
# with a ragged last column tile (N = 8200).
FULL_TILE_SHAPES = [(256, 260, 512), (300, 640, 768), (1100, 2060, 256), (2048, 8192, 256),
                    (2048, 8200, 128)]


@pytest.mark.parametrize("M,N,K", FULL_TILE_SHAPES)
def test_forward_full_tiles(torch, bl, orc, M, N, K):
    W = workloads.gaussian((N, K), (117, M, N, K), 0.02)
    X = workloads.gaussian((M, K), (118, M, N, K), 1.0)
    P, g = bl.quantize_weights(dev(torch, W))
    Xq, sx = bl.quantize_acts(dev(torch, X))
    Y = bl.forward(Xq, sx, P, g)                              # full tiles: straight-line epilogue
    Y_gen, acc = bl.forward(Xq, sx, P, g, return_acc=True)    # general epilogue everywhere
    torch.cuda.synchronize()
    assert torch.equal(Y, Y_gen), (M, N, K)
    acc_ref, Y_ref = orc.forward(host(Xq), host(sx), words(P), host(g)[0])
    assert np.array_equal(host(acc), acc_ref), (M, N, K)
    Yh = host(Y)
    assert np.array_equal(Yh == 0, Y_ref == 0)
    assert rel_err(Yh[Y_ref != 0], Y_ref[Y_ref != 0]) <= REL


def test_forward_without_acc_matches(torch, bl):
    W = dev(torch, workloads.gaussian((300, 512), (112,), 0.02))
    X = dev(torch, workloads.gaussian((40, 512), (113,), 1.0))
    P, g = bl.quantize_weights(W)
    Xq, sx = bl.quantize_acts(X)
    Y1, _ = bl.forward(Xq, sx, P, g, return_acc=True)
    Y2 = bl.forward(Xq, sx, P, g)
    assert torch.equal(Y1, Y2)


def test_forward_extreme_codes(torch, bl, orc):
    """All +1 weights and all +127 activations reach the largest accumulator 127 K."""
    for M in (1, 200):
        K, N = 4096, 48
        Cm = np.ones((N, K), np.int8)
        Cm[1::2] = -1
        P = bl.pack_codes(dev(torch, Cm))
        Xq = dev(torch, np.full((M, K), 127, np.int8))
        sx = dev(torch, np.ones(M, np.float32))
        g = dev(torch, np.ones(1, np.float32))
        Y, acc = bl.forward(Xq, sx, P, g, return_acc=True)
        a = host(acc)
        assert np.all(a[:, 0::2] == 127 * K) and np.all(a[:, 1::2] == -127 * K)


def test_forward_grouped_equals_single(torch, bl):
    probs, singles = [], []
    for i, (M, N, K) in enumerate([(1, 768, 768), (2048, 256, 768), (16, 2048, 768), (300, 64, 2048)]):
        P, g = bl.quantize_weights(dev(torch, workloads.gaussian((N, K), (114, i), 0.02)))
        Xq, sx = bl.quantize_acts(dev(torch, workloads.gaussian((M, K), (115, i), 1.0)))
        Y = torch.empty((M, N), device="cuda")
        acc = torch.empty((M, N), dtype=torch.int32, device="cuda")
        probs.append(dict(X_q=Xq, x_scale=sx, W_packed=P, gamma=g, Y=Y, acc=acc))
        singles.append(bl.forward(Xq, sx, P, g, return_acc=True))
    bl.forward_grouped(probs)
    for p, (Y1, a1) in zip(probs, singles):
        assert torch.equal(p["Y"], Y1) and torch.equal(p["acc"], a1)


def test_forward_deterministic(torch, bl):
    P, g = bl.quantize_weights(dev(torch, workloads.gaussian((1024, 2048), (116,), 0.02)))
    for M in (1, 777):
        Xq, sx = bl.quantize_acts(dev(torch, workloads.gaussian((M, 2048), (117, M), 1.0)))
        a = bl.forward(Xq, sx, P, g)
        b = bl.forward(Xq, sx, P, g)
        assert torch.equal(a, b)
