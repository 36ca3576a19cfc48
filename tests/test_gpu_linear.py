"""The layer call (bitlinear_linear_grouped): steps 3 to 5 in one launch for decode-sized
token counts, against the CPU oracle and against the two-call GPU path.  Its layer form
(bitlinear_linear_ex_grouped) adds the output stages: a gated pair's activation, ReLU^2 and
the residual, checked against the oracle's activation (O7) and residual epilogue (O8) over
the oracle's products on the codes and scales the call reports.

Per call: codes and scales the product used (optional outputs) bit-exact / within 1e-6 of
the oracle's activation quantization, Y within 1e-6 of the oracle epilogue over the oracle's
exact integer product (zero exactly where the oracle gives zero), and Y equal to the two-call
path (bit for bit without the norm; with the norm the sum of squares is added in another
fixed order, so within 1e-6).
"""

import numpy as np
import pytest

import tie_band
import workloads

pytestmark = pytest.mark.gpu

REL = 1e-6
GAMMA = np.float32(0.021)


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


def make_call(torch, bl, M, N, K, dtype, norm, key, zero_row=False):
    """Inputs on both sides: host copies for the oracle, device tensors for the library."""
    X = workloads.gaussian((M, K), (200, M, N, K) + key, 1.0)
    if zero_row and M > 1:
        X[1] = 0.0
    g = (np.float32(1) + workloads.gaussian((K,), (201, K) + key, 0.1)) if norm else None
    C = workloads.ternary((N, K), (202, N, K) + key)
    P = bl.pack_codes(dev(torch, C))
    if dtype == "bf16":
        bits = workloads.f32_to_bf16_bits(X)
        Xt = dev(torch, bits.view(np.int16)).view(torch.bfloat16)
        xin = bits
    else:
        Xt = dev(torch, X)
        xin = X
    call = dict(X=Xt, W_packed=P, gamma=dev(torch, np.array([GAMMA], np.float32)),
                Y=torch.empty((M, N), dtype=torch.float32, device="cuda"),
                X_q=torch.empty((M, K), dtype=torch.int8, device="cuda"),
                x_scale=torch.empty(M, dtype=torch.float32, device="cuda"),
                norm_weight=None if g is None else dev(torch, g), eps=1e-6)
    ref = dict(x=xin, g=g, C=C, bf16=dtype == "bf16")
    return call, ref


def check_call(torch, bl, orc, call, ref, label):
    q_ref, s_ref = orc.quantize_acts(ref["x"], ref["g"], 1e-6, bf16=ref["bf16"])
    q, s, Y = host(call["X_q"]), host(call["x_scale"]), host(call["Y"])
    assert np.array_equal(q, q_ref), label
    nz = s_ref != 0
    assert np.array_equal(s == 0, ~nz), label
    assert rel_err(s[nz], s_ref[nz]) <= REL, label
    if ref["g"] is None:
        assert np.array_equal(s, s_ref), label
    Y_ref = orc.epilogue(orc.matmul(q_ref, ref["C"]), s_ref, GAMMA)
    assert np.array_equal(Y == 0, Y_ref == 0), label
    assert rel_err(Y[Y_ref != 0], Y_ref[Y_ref != 0]) <= REL, label
    # The two-call path on the same input.
    q2, s2 = bl.quantize_acts(call["X"], call["norm_weight"], 1e-6)
    Y2 = bl.forward(q2, s2, call["W_packed"], call["gamma"])
    torch.cuda.synchronize()
    assert torch.equal(call["X_q"], q2), label
    if ref["g"] is None:
        assert torch.equal(call["Y"], Y2), label
    else:
        assert rel_err(Y[Y_ref != 0], host(Y2)[Y_ref != 0]) <= 2 * REL, label


LINEAR_SHAPES = [
    (1, 1, 16), (1, 37, 48), (1, 768, 768), (2, 300, 272), (3, 2048, 768), (4, 129, 2048),
    (1, 96, 9728), (4, 40, 12288), (2, 5000, 1040),
    # Large layers: blocks of two and four 16-row groups.
    (1, 16400, 768), (3, 9000, 272),
]


@pytest.mark.parametrize("M,N,K", LINEAR_SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("norm", [False, True])
def test_linear_fused(torch, bl, orc, M, N, K, dtype, norm):
    assert bl.linear_fused(M, K)
    call, ref = make_call(torch, bl, M, N, K, dtype, norm, (0,), zero_row=True)
    bl.linear_grouped([call])
    torch.cuda.synchronize()
    check_call(torch, bl, orc, call, ref, (M, N, K, dtype, norm))


def test_linear_grouped_mixed(torch, bl, orc):
    """Fused calls of several K in one launch, next to calls that take the two-step path."""
    specs = [(1, 768, 768, "f32", False), (1, 256, 2048, "f32", True), (4, 100, 16384, "f32", False),
             (2, 64, 80, "bf16", True), (8, 300, 768, "f32", False), (1, 50, 65536, "f32", False),
             (33, 128, 1024, "bf16", True)]
    calls, refs = [], []
    for i, (M, N, K, dt, nm) in enumerate(specs):
        c, r = make_call(torch, bl, M, N, K, dt, nm, (1, i))
        calls.append(c)
        refs.append(r)
    assert [bl.linear_fused(c["X"].shape[0], c["X"].shape[1]) for c in calls] == \
        [True, True, False, True, False, False, False]
    bl.linear_grouped(calls)
    torch.cuda.synchronize()
    for i, (c, r) in enumerate(zip(calls, refs)):
        check_call(torch, bl, orc, c, r, specs[i])


def test_linear_optional_outputs_and_convenience(torch, bl, orc):
    """Without the X_q / x_scale outputs the fused call gives the same Y; bl.linear agrees."""
    call, ref = make_call(torch, bl, 3, 700, 1536, "f32", True, (2,))
    bl.linear_grouped([call])
    Y_full = call["Y"].clone()
    call2 = dict(call, X_q=None, x_scale=None, Y=torch.empty_like(Y_full))
    bl.linear_grouped([call2])
    Y3 = bl.linear(call["X"], call["W_packed"], call["gamma"], call["norm_weight"], 1e-6)
    torch.cuda.synchronize()
    assert torch.equal(call2["Y"], Y_full)
    assert torch.equal(Y3, Y_full)
    check_call(torch, bl, orc, call, ref, "outputs")
    # Beyond the fused size the convenience call takes the two-step path.
    X = dev(torch, workloads.gaussian((9, 256), (203,), 1.0))
    Y9 = bl.linear(X, call["W_packed"][:, :16].contiguous(), call["gamma"])
    q9, s9 = bl.quantize_acts(X)
    assert torch.equal(Y9, bl.forward(q9, s9, call["W_packed"][:, :16].contiguous(), call["gamma"]))


def test_linear_degenerate(torch, bl):
    """All-zero activations give zero codes, zero scales and Y == 0; empty calls are no-ops."""
    C = workloads.ternary((64, 512), (204,))
    P = bl.pack_codes(dev(torch, C))
    gamma = dev(torch, np.array([GAMMA], np.float32))
    X = torch.zeros((2, 512), dtype=torch.float32, device="cuda")
    Y = torch.full((2, 64), 7.0, device="cuda")
    Xq = torch.full((2, 512), 5, dtype=torch.int8, device="cuda")
    sx = torch.full((2,), 3.0, device="cuda")
    bl.linear_grouped([dict(X=X, W_packed=P, gamma=gamma, Y=Y, X_q=Xq, x_scale=sx)])
    torch.cuda.synchronize()
    assert torch.count_nonzero(Y) == 0 and torch.count_nonzero(Xq) == 0 and torch.count_nonzero(sx) == 0
    empty = torch.empty((0, 512), dtype=torch.float32, device="cuda")
    bl.linear_grouped([dict(X=empty, W_packed=P, gamma=gamma, Y=torch.empty((0, 64), device="cuda"))])
    torch.cuda.synchronize()


EX_SHAPES = [(1, 16, 16), (1, 300, 768), (2, 1000, 2048), (3, 129, 272), (4, 2048, 9728),
             (1, 4100, 1536)]


def ex_reference(orc, call, ref, C2, gamma2, kind, R):
    """Y from the oracle on the call's reported codes and scales, and for SwiGLU the fp64 value
    of h = silu(y1) * y2 before its fp32 rounding (else None)."""
    q, s = host(call["X_q"]), host(call["x_scale"])
    y1 = orc.epilogue(orc.matmul(q, ref["C"]), s, GAMMA)
    h64 = None
    if C2 is not None:
        y2 = orc.epilogue(orc.matmul(q, C2), s, gamma2)
        h = orc.ffn_act(kind, y1, y2)
        if kind == orc.SWIGLU:
            h64 = orc.ffn_act_f64(kind, y1, y2)
    elif kind != 0:
        h = orc.ffn_act(kind, y1)
    else:
        h = y1
    if R is not None:
        h = (h + R).astype(np.float32)      # one fp32 rounding of the fp32 sum
    return h, h64


@pytest.mark.parametrize("M,N,K", EX_SHAPES)
@pytest.mark.parametrize("kind", [0, 1, 2, 3])
@pytest.mark.parametrize("norm,residual", [(False, False), (True, True), (True, False)])
def test_linear_ex(torch, bl, orc, M, N, K, kind, norm, residual):
    label = (M, N, K, kind, norm, residual)
    call, ref = make_call(torch, bl, M, N, K, "f32", norm, (3, kind), zero_row=True)
    glu = kind in (bl.ACT_SWIGLU, bl.ACT_RELU2_GLU)
    C2 = workloads.ternary((N, K), (205, N, K, kind)) if glu else None
    gamma2 = np.float32(0.017)
    R = workloads.gaussian((M, N), (206, M, N), 3.0) if residual else None
    ex = dict(call, act=kind, residual=None if R is None else dev(torch, R))
    if glu:
        ex.update(W2_packed=bl.pack_codes(dev(torch, C2)), gamma2=dev(torch, np.array([gamma2], np.float32)))
    bl.linear_ex_grouped([ex])
    torch.cuda.synchronize()
    # Codes and scales the call used: the activation quantizer's.
    q_ref, s_ref = orc.quantize_acts(ref["x"], ref["g"], 1e-6)
    assert np.array_equal(host(call["X_q"]), q_ref), label
    s = host(call["x_scale"])
    nz = s_ref != 0
    assert np.array_equal(s == 0, ~nz), label
    assert rel_err(s[nz], s_ref[nz]) <= REL, label
    Y_ref, h64 = ex_reference(orc, call, ref, C2, gamma2, kind, R)
    Y = host(call["Y"])
    if kind == bl.ACT_SWIGLU:
        # The device library's exp against the host's: h may take the other rounding where the
        # oracle's fp64 h is at an fp32 tie, and Y is then exactly that h (plus the residual).
        flips = tie_band.check_values(Y, h64, label, add=R)
        if flips:
            print(f"{label}: {flips} of {Y.size} SwiGLU values at an fp32 tie took the other rounding")
    else:
        assert np.array_equal(Y, Y_ref), label


def test_linear_ex_mixed_group(torch, bl, orc):
    """Single projections and gated pairs of several K in one call (two launches), with and
    without the optional code outputs; the outputs equal those of one call per problem."""
    specs = [(1, 768, 768, 0, True), (1, 2048, 768, 1, False), (2, 640, 2048, 3, True),
             (4, 96, 9728, 2, True), (3, 1000, 1536, 0, False)]
    calls = []
    for i, (M, N, K, kind, res) in enumerate(specs):
        c, _ = make_call(torch, bl, M, N, K, "f32", True, (4, i))
        c["act"] = kind
        if kind in (bl.ACT_SWIGLU, bl.ACT_RELU2_GLU):
            c["W2_packed"] = bl.pack_codes(dev(torch, workloads.ternary((N, K), (207, i))))
            c["gamma2"] = dev(torch, np.array([0.019], np.float32))
        if res:
            c["residual"] = dev(torch, workloads.gaussian((M, N), (208, i), 1.0))
        if i % 2:
            c["X_q"] = c["x_scale"] = None
        calls.append(c)
    bl.linear_ex_grouped(calls)
    torch.cuda.synchronize()
    together = [c["Y"].clone() for c in calls]
    for c, Y in zip(calls, together):
        c["Y"].zero_()
        bl.linear_ex_grouped([c])
        torch.cuda.synchronize()
        assert torch.equal(c["Y"], Y)


def test_linear_ex_rejects(torch, bl):
    """Sizes past the fused form, a gated kind without its pair and a pair with a single
    kind are refused before anything runs."""
    call, _ = make_call(torch, bl, 5, 64, 256, "f32", False, (5,))
    with pytest.raises(bl.BitLinearError) as e:
        bl.linear_ex_grouped([call])
    assert e.value.status == -2
    call, _ = make_call(torch, bl, 2, 64, 256, "f32", False, (6,))
    with pytest.raises(bl.BitLinearError) as e:
        bl.linear_ex_grouped([dict(call, act=bl.ACT_SWIGLU)])
    assert e.value.status == -1
    with pytest.raises(bl.BitLinearError) as e:
        bl.linear_ex_grouped([dict(call, act=bl.ACT_NONE, W2_packed=call["W_packed"],
                                   gamma2=call["gamma"])])
    assert e.value.status == -4
