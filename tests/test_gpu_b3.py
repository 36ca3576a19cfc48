"""Base-3 weights on the GPU: the packer bit-exact against the oracle's base-3 packing (O13)
of the same codes, and the fused decode call on base-3 weights against the oracle (codes
bit-exact, scales and Y within 1e-6 as for the two-bit call) and bit for bit against the same
call on the two-bit layout (the integer sums, hence every output, are identical)."""

import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu

REL = 1e-6
GAMMA = np.float32(0.019)


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


@pytest.mark.parametrize("N,K", [(1, 16), (16, 80), (33, 96), (300, 768), (64, 2000), (129, 9728), (8, 12288)])
def test_pack_b3(torch, bl, orc, N, K):
    C = workloads.ternary((N, K), (500, N, K))
    B = bl.pack_b3(bl.pack_codes(dev(torch, C)))
    torch.cuda.synchronize()
    assert B.shape == (N, orc.b3_row_bytes(K)) and bl.b3_row_bytes(K) == orc.b3_row_bytes(K)
    assert np.array_equal(host(B), orc.pack_b3(C))


SHAPES = [(1, 1, 16), (1, 37, 80), (2, 300, 272), (1, 768, 768), (3, 2048, 768), (4, 129, 2000),
          (1, 96, 9728), (4, 40, 12288), (1, 4100, 2560), (2, 16400, 1040)]


def make(torch, bl, M, N, K, dtype, norm, key):
    X = workloads.gaussian((M, K), (501, M, N, K) + key, 1.0)
    if M > 1:
        X[1] = 0.0
    g = (np.float32(1) + workloads.gaussian((K,), (502, K) + key, 0.1)) if norm else None
    C = workloads.ternary((N, K), (503, N, K) + key)
    P = bl.pack_codes(dev(torch, C))
    if dtype == "bf16":
        bits = workloads.f32_to_bf16_bits(X)
        Xt, xin = dev(torch, bits.view(np.int16)).view(torch.bfloat16), bits
    else:
        Xt, xin = dev(torch, X), X
    gt = dev(torch, np.array([GAMMA], np.float32))
    nt = None if g is None else dev(torch, g)

    def outs():
        return dict(Y=torch.empty((M, N), device="cuda"),
                    X_q=torch.empty((M, K), dtype=torch.int8, device="cuda"),
                    x_scale=torch.empty(M, device="cuda"))
    b3 = dict(X=Xt, W_b3=bl.pack_b3(P), gamma=gt, norm_weight=nt, eps=1e-6, **outs())
    two = dict(X=Xt, W_packed=P, gamma=gt, norm_weight=nt, eps=1e-6, **outs())
    return b3, two, dict(x=xin, g=g, C=C, bf16=dtype == "bf16")


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("norm", [False, True])
def test_linear_b3(torch, bl, orc, M, N, K, dtype, norm):
    label = (M, N, K, dtype, norm)
    b3, two, ref = make(torch, bl, M, N, K, dtype, norm, (0,))
    bl.linear_b3_grouped([b3])
    bl.linear_grouped([two])
    torch.cuda.synchronize()
    for k in ("Y", "X_q", "x_scale"):
        assert torch.equal(b3[k], two[k]), (label, k)
    q_ref, s_ref = orc.quantize_acts(ref["x"], ref["g"], 1e-6, bf16=ref["bf16"])
    assert np.array_equal(host(b3["X_q"]), q_ref), label
    s = host(b3["x_scale"])
    nz = s_ref != 0
    assert rel_err(s[nz], s_ref[nz]) <= REL, label
    Y_ref = orc.epilogue(orc.matmul(q_ref, ref["C"]), s_ref, GAMMA)
    Y = host(b3["Y"])
    assert np.array_equal(Y == 0, Y_ref == 0), label
    assert rel_err(Y[Y_ref != 0], Y_ref[Y_ref != 0]) <= REL, label


def test_linear_b3_grouped_layer_set(torch, bl):
    """A whole decode layer set (Qwen3-4B shapes, one token) in one call: each output equals
    the two-bit call's."""
    mats = workloads.WORKLOADS["c5_qwen3_4b_layer"].matrices
    b3s, twos = [], []
    for i, m in enumerate(mats):
        b3, two, _ = make(torch, bl, 1, m.N, m.K, "f32", i % 2 == 0, (1, i))
        b3s.append(b3)
        twos.append(two)
    bl.linear_b3_grouped(b3s)
    bl.linear_grouped(twos)
    torch.cuda.synchronize()
    for a, b in zip(b3s, twos):
        assert torch.equal(a["Y"], b["Y"])


def test_linear_b3_rejects_prefill_sizes(torch, bl):
    b3, _, _ = make(torch, bl, 5, 64, 256, "f32", False, (2,))
    with pytest.raises(bl.BitLinearError) as e:
        bl.linear_b3_grouped([b3])
    assert e.value.status == -2
