"""Quad rows on the GPU: the packer bit-exact against the layout written out here from the
oracle's two-bit packing, the step's weight quantization into quad rows bit-exact against the
rows call re-arranged, and the prefill product on quad rows bit for bit against the same call
on rows and against the oracle (accumulators exact, Y within 1e-6), from a few tiles with
ragged token and row counts up to the Qwen3-4B layer set at 8192 tokens."""

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


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b) / np.maximum(np.abs(b), 1e-300))) if a.size else 0.0


def quad_layout(P, N, K):
    """The documented layout, from the rows P [N][K/16]: word w of row n goes to word
    ((n / 4) * (K / 128) + w / 8) * 32 + 8 (n % 4) + w % 8."""
    S = K // 128
    rows = P.view(np.uint32).reshape(N // 4, 4, S, 8)       # [q][i][t][j]
    return rows.transpose(0, 2, 1, 3).reshape(-1)             # [q][t][i][j]


@pytest.mark.parametrize("N,K", [(4, 128), (8, 256), (36, 384), (100, 2560), (12, 9728)])
def test_pack_quad_rows(torch, bl, orc, N, K):
    C = workloads.ternary((N, K), (520, N, K))
    P = orc.pack(C)
    Q = bl.pack_quad_rows(dev(torch, P.view(np.int32).reshape(N, K // 16)))
    torch.cuda.synchronize()
    assert np.array_equal(host(Q).view(np.uint32).reshape(-1), quad_layout(P, N, K))


@pytest.mark.parametrize("shapes", [[(4, 128)], [(300, 512), (64, 2560), (8, 1024)],
                                    [(2560, 4096), (1024, 2560)], [(2560, 9728), (4096, 2560)]])
def test_quantize_step_quad_rows(torch, bl, shapes):
    """Same gamma, same activation results, and the rows call's words re-arranged (rows of up
    to 4096 values share the gamma pass's launch; 9728 takes the separate launches, as the
    Qwen3-4B set's down projection does in the benchmark step)."""
    Ws = [dev(torch, workloads.gaussian(s, (521, i) + s, 0.02)) for i, s in enumerate(shapes)]
    Xs = [dev(torch, workloads.gaussian((33, s[1]), (522, i) + s, 1.0)) for i, s in enumerate(shapes)]
    w_rows, x_rows = bl.quantize_step(Ws, Xs)
    w_quad, x_quad = bl.quantize_step(Ws, Xs, quad_rows=True)
    torch.cuda.synchronize()
    for (Pr, gr), (Pq, gq), s in zip(w_rows, w_quad, shapes):
        assert torch.equal(gr, gq), s
        assert np.array_equal(host(Pq).view(np.uint32).reshape(-1),
                              quad_layout(host(Pr).view(np.uint32), *s)), s
    for (a, b), (c, d) in zip(x_rows, x_quad):
        assert torch.equal(a, c) and torch.equal(b, d)


def forward_pair(torch, bl, problems):
    """Runs the rows call and the quad-row call on the same codes; returns both outputs."""
    rows, quad = [], []
    for p in problems:
        M, N = p["M"], p["N"]
        base = dict(X_q=p["Xq"], x_scale=p["sx"], gamma=p["g"])
        rows.append(dict(base, W_packed=p["P"], Y=torch.empty((M, N), device="cuda"),
                         acc=torch.empty((M, N), dtype=torch.int32, device="cuda")))
        quad.append(dict(base, W_packed=bl.pack_quad_rows(p["P"]),
                         Y=torch.full((M, N), float("nan"), device="cuda"),
                         acc=torch.empty((M, N), dtype=torch.int32, device="cuda")))
    bl.forward_grouped(rows)
    bl.forward_grouped(quad, quad_rows=True)
    torch.cuda.synchronize()
    return rows, quad


def make_problem(torch, bl, M, N, K, key):
    W = workloads.gaussian((N, K), (523, M, N, K) + key, 0.02)
    X = workloads.gaussian((M, K), (524, M, N, K) + key, 1.0)
    P, g = bl.quantize_weights(dev(torch, W))
    Xq, sx = bl.quantize_acts(dev(torch, X))
    return dict(M=M, N=N, K=K, P=P, g=g, Xq=Xq, sx=sx)


# Ragged tokens and rows over several tiles (128 x 128 tiles below 256 units of 256 x 256,
# 128 x 256 tiles from there), K from one stage to many.
SHAPES = [(17, 4, 128), (300, 132, 384), (129, 260, 2560), (1000, 512, 1024),
          (2048, 8192, 512)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_forward_quad_rows(torch, bl, orc, M, N, K):
    p = make_problem(torch, bl, M, N, K, (0,))
    rows, quad = forward_pair(torch, bl, [p])
    assert torch.equal(rows[0]["acc"], quad[0]["acc"]), (M, N, K)
    assert torch.equal(rows[0]["Y"], quad[0]["Y"]), (M, N, K)
    if M * N * K <= 300 * 260 * 2560:
        acc_ref, Y_ref = orc.forward(host(p["Xq"]), host(p["sx"]), host(p["P"]).view(np.uint32),
                                     host(p["g"])[0])
        assert np.array_equal(host(quad[0]["acc"]), acc_ref), (M, N, K)
        Y = host(quad[0]["Y"])
        assert np.array_equal(Y == 0, Y_ref == 0)
        assert rel_err(Y[Y_ref != 0], Y_ref[Y_ref != 0]) <= REL


def test_forward_quad_rows_grouped_mixed_shapes(torch, bl):
    """Several problems of different shapes in one launch (and an empty one skipped)."""
    ps = [make_problem(torch, bl, M, N, K, (1, i)) for i, (M, N, K) in
          enumerate([(200, 64, 256), (33, 1028, 640), (400, 300, 1152)])]
    rows, quad = forward_pair(torch, bl, ps)
    for a, b in zip(rows, quad):
        assert torch.equal(a["acc"], b["acc"]) and torch.equal(a["Y"], b["Y"])


@pytest.mark.parametrize("M,N,K", [(40, 132, 384), (2048, 4096, 1024)])
def test_forward_ex_quad_rows_residual(torch, bl, M, N, K):
    """The layer chain's product form (residual added in the epilogue, here also in place) on
    quad rows: bit for bit the rows call's."""
    p = make_problem(torch, bl, M, N, K, (2,))
    R = dev(torch, workloads.gaussian((M, N), (528, M, N, K), 1.0))
    outs = []
    for quad in (False, True):
        Y = R.clone()
        bl.forward_ex_grouped([dict(X_q=p["Xq"], x_scale=p["sx"], gamma=p["g"], Y=Y, residual=Y,
                                    W_packed=bl.pack_quad_rows(p["P"]) if quad else p["P"])],
                              quad_rows=quad)
        outs.append(Y)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]), (M, N, K)


def test_forward_quad_rows_layer_set(torch, bl, orc):
    """The Qwen3-4B layer set at 8192 tokens (the 128 x 256 tiles, as the benchmark step runs
    it): every accumulator and output equals the rows call's, and 1024 sampled entries of each
    projection (the corners among them) equal the oracle's, computed one by one."""
    mats = workloads.WORKLOADS["c5_qwen3_4b_layer"].matrices
    M = 8192
    ps = []
    for i, m in enumerate(mats):
        C = workloads.ternary((m.N, m.K), (525, i))
        P = bl.pack_codes(dev(torch, C))
        X = workloads.gaussian((M, m.K), (526, i), 1.0)
        Xq, sx = bl.quantize_acts(dev(torch, X))
        ps.append(dict(M=M, N=m.N, K=m.K, P=P, g=dev(torch, np.array([0.021], np.float32)),
                       Xq=Xq, sx=sx))
    rows, quad = forward_pair(torch, bl, ps)
    for a, b, m in zip(rows, quad, mats):
        assert torch.equal(a["acc"], b["acc"]), (m.N, m.K)
        assert torch.equal(a["Y"], b["Y"]), (m.N, m.K)
    rng = np.random.default_rng(527)
    for p, b, m in zip(ps, quad, mats):
        mi = np.concatenate([[0, M - 1, 0, M - 1], rng.integers(0, M, 1020)])
        ni = np.concatenate([[0, 0, m.N - 1, m.N - 1], rng.integers(0, m.N, 1020)])
        acc_ref, y_ref = orc.forward_entries(host(p["Xq"]), host(p["sx"]), host(p["P"]).view(np.uint32),
                                             0.021, mi, ni)
        assert np.array_equal(host(b["acc"])[mi, ni], acc_ref), (m.N, m.K)
        y = host(b["Y"])[mi, ni]
        assert np.array_equal(y == 0, y_ref == 0)
        assert rel_err(y[y_ref != 0], y_ref[y_ref != 0]) <= REL, (m.N, m.K)
