"""Training-side products on the GPU against the CPU oracle.

* Transposed packing: bit-exact against the oracle's packing of the transposed codes.
* Weight-only forward (O9), input gradient (O10) and weight gradient with the pass-through,
  hard and soft scales (O11, O12): fp32 results within the bound the arithmetic gives
  (the library header states it): for a contraction of length L over terms a_i,
  |y - y_ref| <= scale * (L * 2^-24 + e_op) * sum |a_i| + 2^-23 |y_ref|,
  e_op = 2^-16 for operands carried as two bf16 parts (fp32 inputs; for the weight
  gradient also the fp32 product dY * s_x, 2^-24), 0 for bf16 inputs.  The bound is loose
  for long contractions, so the RMS of the error relative to sum |a_i| must also stay
  below 2^-20 + e_op / 4 (a realistic fp32 accumulation sits near sqrt(L) * 2^-24, the
  two-part representation near e_op / 3).
* Shapes: several tiles with ragged tails in every dimension, word counts that are not a
  multiple of the stage width, and the Qwen3-4B-shaped projections at full size with the
  oracle evaluated on sampled rows.
"""

import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


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


def as_input(torch, X, dtype):
    """(device tensor, fp32 values the oracle sees) for fp32 or bf16 inputs."""
    if dtype == "bf16":
        bits = workloads.f32_to_bf16_bits(X)
        return dev(torch, bits.view(np.int16)).view(torch.bfloat16), workloads.bf16_bits_to_f32(bits)
    return dev(torch, X), X


def check_bound(Y, ref, S, L, e_op, scale=1.0, label=""):
    Y = Y.astype(np.float64)
    ref = ref.astype(np.float64)
    err = np.abs(Y - ref)
    bound = scale * S * (L * U + e_op) + 2.0 ** -23 * np.abs(ref) + 1e-37
    worst = float(np.max(err / bound)) if err.size else 0.0
    assert worst <= 1.0, (label, worst)
    denom = scale * S
    live = denom > 0
    if np.any(live):
        rms = float(np.sqrt(np.mean((err[live] / denom[live]) ** 2)))
        assert rms <= 2.0 ** -20 + e_op / 4, (label, rms)
    assert np.all(err[~live] == 0), label


TRANSPOSE_SHAPES = [(16, 16), (32, 80), (48, 272), (208, 1040), (1024, 768)]


@pytest.mark.parametrize("N,K", TRANSPOSE_SHAPES)
def test_transpose_packed(torch, bl, orc, N, K):
    C = workloads.ternary((N, K), (400, N, K))
    P = bl.pack_codes(dev(torch, C))
    Pt = bl.transpose_packed(P)
    torch.cuda.synchronize()
    ref = orc.pack(np.ascontiguousarray(C.T)).view(np.int32)
    assert np.array_equal(host(Pt), ref)


WONLY_SHAPES = [(1, 16, 16), (5, 40, 80), (130, 200, 272), (257, 129, 1040), (64, 768, 2048),
                (300, 520, 144)]


@pytest.mark.parametrize("M,N,K", WONLY_SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_forward_wonly(torch, bl, orc, M, N, K, dtype):
    X = workloads.gaussian((M, K), (401, M, N, K), 1.0)
    if M > 2:
        X[1] = 0.0
    C = workloads.ternary((N, K), (402, M, N, K))
    g = np.float32(0.021)
    Xt, Xf = as_input(torch, X, dtype)
    Y = bl.forward_wonly(Xt, bl.pack_codes(dev(torch, C)), dev(torch, np.array([g], np.float32)))
    torch.cuda.synchronize()
    ref = orc.forward_wonly(Xf, C, g)
    S = float(g) * (np.abs(Xf.astype(np.float64)) @ np.abs(C.astype(np.float64)).T)
    check_bound(host(Y), ref, S, K, 2.0 ** -16 if dtype == "f32" else 0.0, label=(M, N, K, dtype))


GRAD_INPUT_SHAPES = [(1, 16, 16), (7, 80, 48), (130, 272, 200 // 16 * 16), (257, 1040, 129 * 16),
                     (96, 2048, 768)]


@pytest.mark.parametrize("M,N,K", GRAD_INPUT_SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_grad_input(torch, bl, orc, M, N, K, dtype):
    dY = workloads.gaussian((M, N), (403, M, N, K), 1.0)
    C = workloads.ternary((N, K), (404, M, N, K))
    g = np.float32(0.017)
    dYt, dYf = as_input(torch, dY, dtype)
    Wt = bl.transpose_packed(bl.pack_codes(dev(torch, C)))
    dX = bl.grad_input(dYt, Wt, dev(torch, np.array([g], np.float32)))
    torch.cuda.synchronize()
    ref = orc.grad_input(dYf, C, g)
    S = float(g) * (np.abs(dYf.astype(np.float64)) @ np.abs(C.astype(np.float64)))
    check_bound(host(dX), ref, S, N, 2.0 ** -16 if dtype == "f32" else 0.0, label=(M, N, K, dtype))


def ste_scale_np(kind, W, g, beta):
    if kind == 0:
        return np.ones(W.shape)
    t = (W / np.float32(g)).astype(np.float32).astype(np.float64)
    if kind == 1:
        return (np.abs(t) <= 1.0).astype(np.float64)
    return 1.0 / np.cosh(beta * t) ** 2


GRAD_WEIGHT_SHAPES = [(1, 16, 16), (33, 40, 80), (130, 200, 272), (257, 129, 1040), (512, 768, 2048),
                      (64, 130, 48)]


@pytest.mark.parametrize("M,N,K", GRAD_WEIGHT_SHAPES)
@pytest.mark.parametrize("kind", [0, 1, 2])
def test_grad_weight(torch, bl, orc, M, N, K, kind):
    dY = workloads.gaussian((M, N), (405, M, N, K), 1.0)
    X = workloads.gaussian((M, K), (406, M, N, K), 1.0)
    if M > 2:
        X[1] = 0.0                       # a zero row: s_x = 0
    q, s = orc.quantize_acts(X)
    W = workloads.gaussian((N, K), (407, N, K), 0.03)
    g = np.float32(0.02)
    beta = 2.0
    dW = bl.grad_weight(dev(torch, dY), dev(torch, q), dev(torch, s), dev(torch, np.array([g], np.float32)),
                        W=dev(torch, W) if kind else None, ste=kind, beta=beta)
    torch.cuda.synchronize()
    ref = orc.grad_weight(dY, kind, W=W if kind else None, gamma=g, beta=beta, Xq=q, sx=s)
    xh = np.abs(q.astype(np.float64) * s.astype(np.float64)[:, None])
    S = np.abs(dY.astype(np.float64)).T @ xh
    check_bound(host(dW), ref, S, M, 2.0 ** -16 + U, ste_scale_np(kind, W, g, beta), label=(M, N, K, kind))


def test_grad_weight_hard_mask_exact_boundaries(torch, bl, orc):
    """Weights at exactly |W / gamma| = 1 keep their gradient; the next float out drops it."""
    M, N, K = 8, 16, 32
    dY = workloads.gaussian((M, N), (408,), 1.0)
    q = np.ones((M, K), np.int8)
    s = np.full(M, 0.5, np.float32)
    g = np.float32(0.25)
    W = np.zeros((N, K), np.float32)
    W[:, 0::4] = g
    W[:, 1::4] = -g
    W[:, 2::4] = np.nextafter(g, np.float32(1))
    W[:, 3::4] = np.nextafter(-g, np.float32(-1))
    dW = host(bl.grad_weight(dev(torch, dY), dev(torch, q), dev(torch, s), dev(torch, np.array([g], np.float32)),
                             W=dev(torch, W), ste=bl.STE_HARD))
    ref = orc.grad_weight(dY, 1, W=W, gamma=g, Xq=q, sx=s)
    assert np.all(dW[:, 2::4] == 0) and np.all(dW[:, 3::4] == 0)
    assert np.count_nonzero(ref[:, 0::4]) > 0
    S = np.abs(dY.astype(np.float64)).T @ np.abs(q * s[:, None].astype(np.float64))
    check_bound(dW, ref, S, M, 2.0 ** -16 + U, ste_scale_np(1, W, g, 2.0), label="boundaries")


def test_grad_weight_empty_batch_and_noops(torch, bl):
    """M == 0: dW = 0 (an empty sum); M == 0 / N == 0 elsewhere: nothing is written."""
    g = dev(torch, np.array([0.02], np.float32))
    dW = torch.full((16, 32), 5.0, device="cuda")
    bl.grad_weight_grouped([dict(dY=torch.empty((0, 16), device="cuda"),
                                 X_q=torch.empty((0, 32), dtype=torch.int8, device="cuda"),
                                 x_scale=torch.empty(0, device="cuda"), gamma=g, dW=dW)])
    torch.cuda.synchronize()
    assert torch.count_nonzero(dW) == 0
    Y = torch.full((0, 64), 1.0, device="cuda")
    bl.forward_wonly_grouped([dict(X=torch.empty((0, 32), device="cuda"),
                                   W_packed=torch.zeros((64, 2), dtype=torch.int32, device="cuda"),
                                   gamma=g, Y=Y)])
    torch.cuda.synchronize()


def test_grouped_calls_match_single(torch, bl):
    """Several problems of mixed dtypes in one grouped call equal one call per problem."""
    specs = [(5, 40, 80, "f32"), (130, 200, 272, "bf16"), (64, 768, 512, "f32"), (3, 32, 16, "bf16")]
    probs, gp = [], []
    for i, (M, N, K, dt) in enumerate(specs):
        X, _ = as_input(torch, workloads.gaussian((M, K), (409, i), 1.0), dt)
        P = bl.pack_codes(dev(torch, workloads.ternary((N, K), (410, i))))
        gam = dev(torch, np.array([0.01 * (i + 1)], np.float32))
        probs.append(dict(X=X, W_packed=P, gamma=gam, Y=torch.empty((M, N), device="cuda")))
        dY, _ = as_input(torch, workloads.gaussian((M, N), (411, i), 1.0), dt)
        N16 = N // 16 * 16
        gp.append(dict(dY=dY[:, :N16].contiguous(), Wt_packed=bl.transpose_packed(P[:N16].contiguous()),
                       gamma=gam, dX=torch.empty((M, K), device="cuda")))
    bl.forward_wonly_grouped(probs)
    bl.grad_input_grouped(gp)
    torch.cuda.synchronize()
    Ys = [p["Y"].clone() for p in probs]
    dXs = [p["dX"].clone() for p in gp]
    for p, Y in zip(probs, Ys):
        p["Y"].zero_()
        bl.forward_wonly_grouped([p])
        torch.cuda.synchronize()
        assert torch.equal(p["Y"], Y)
    for p, dX in zip(gp, dXs):
        p["dX"].zero_()
        bl.grad_input_grouped([p])
        torch.cuda.synchronize()
        assert torch.equal(p["dX"], dX)


# Qwen3-4B-shaped projections at full size (the 8192-token training step), the oracle on
# sampled rows of the output.
FULL = [("gate", 9728, 2560), ("down", 2560, 9728), ("q", 4096, 2560)]


@pytest.mark.parametrize("name,N,K", FULL)
def test_full_size_sampled(torch, bl, orc, name, N, K):
    M = 8192
    rng = np.random.Generator(np.random.PCG64([412, N, K]))
    X = workloads.gaussian((M, K), (413, N, K), 1.0)
    dY = workloads.gaussian((M, N), (414, N, K), 1.0)
    C = workloads.ternary((N, K), (415, N, K))
    W = workloads.gaussian((N, K), (416, N, K), 0.02)
    g = np.float32(0.016)
    gt = dev(torch, np.array([g], np.float32))
    P = bl.pack_codes(dev(torch, C))
    Xt = dev(torch, X)
    Y = bl.forward_wonly(Xt, P, gt)
    dX = bl.grad_input(dev(torch, dY), bl.transpose_packed(P), gt)
    q_t, s_t = bl.quantize_acts(Xt)
    dW = bl.grad_weight(dev(torch, dY), q_t, s_t, gt, W=dev(torch, W), ste=bl.STE_SOFT)
    torch.cuda.synchronize()
    rows = np.sort(rng.choice(M, 6, replace=False))
    rows = np.unique(np.concatenate([rows, [0, M - 1]]))
    ref = orc.forward_wonly(X[rows], C, g)
    S = float(g) * (np.abs(X[rows].astype(np.float64)) @ np.abs(C.astype(np.float64)).T)
    check_bound(host(Y[rows]), ref, S, K, 2.0 ** -16, label=(name, "Y"))
    ref = orc.grad_input(dY[rows], C, g)
    S = float(g) * (np.abs(dY[rows].astype(np.float64)) @ np.abs(C.astype(np.float64)))
    check_bound(host(dX[rows]), ref, S, N, 2.0 ** -16, label=(name, "dX"))
    q, s = host(q_t), host(s_t)
    cols = np.unique(np.concatenate([np.sort(rng.choice(N, 6, replace=False)), [0, N - 1]]))
    ref = orc.grad_weight(np.ascontiguousarray(dY[:, cols]), 2, W=W[cols], gamma=g, beta=2.0, Xq=q, sx=s)
    xh = np.abs(q.astype(np.float64) * s.astype(np.float64)[:, None])
    S = np.abs(dY[:, cols].astype(np.float64)).T @ xh
    check_bound(host(dW[cols]), ref, S, M, 2.0 ** -16 + U, ste_scale_np(2, W[cols], g, 2.0),
                label=(name, "dW"))
