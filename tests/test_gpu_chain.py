"""Layer chain on the GPU against the CPU oracle, stage by stage.

* Activation quantization with the FFN activation in front (SwiGLU, gated ReLU^2, ReLU^2;
  with and without SubLN): codes bit-exact against the oracle's activation (O7) followed by
  its quantizer (O4); scales bit-exact without the norm, within 1e-6 with it.  SwiGLU's fp64
  exp comes from two different implementations, so an h may round the other way where the
  oracle's fp64 h lies within a few ulps of an fp32 rounding midpoint: every differing code
  must then be the oracle's quantization of that other rounding (tie_band), and is counted.
* Products with a residual: Y bit-exact against the oracle's residual epilogue (O8) on the
  same codes and scales (vector and scalar store paths, decode and prefill, residual
  aliasing the output).
* The whole chain of one layer (layer.py): every stage's output against the oracle run on the
  GPU's own inputs to that stage, so a legal difference cannot cascade.  At one and three
  tokens the chain takes the three-launch fused form (gate/up pair with the activation in
  the epilogue); its FFN hidden state h is checked against the oracle's activation of the
  oracle's gate and up outputs on the GPU's codes and scales.  The two forms also agree with
  each other on the same layer.
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


def check_ffn_quant(q, s, G, U, g, kind, orc, label):
    """Codes q and scales s of the FFN activation act(G, U) followed by the quantizer (norm
    weight g or None): exactly the oracle's (O7 then O4), except SwiGLU elements at an fp32
    tie of the oracle's fp64 h, which may take the other rounding (tie_band.check_act_codes).
    Returns the number of such elements."""
    glu = kind in (orc.SWIGLU, orc.RELU2_GLU)
    if kind == orc.SWIGLU:
        flips = tie_band.check_act_codes(q, s, orc.ffn_act_f64(kind, G, U), g, orc, label)
        if flips:
            print(f"{label}: {flips} of {q.size} SwiGLU values at an fp32 tie took the other rounding")
        return flips
    q_ref, s_ref = orc.quantize_acts(orc.ffn_act(kind, G, U if glu else None), g, 1e-6)
    assert np.array_equal(q, q_ref), label
    check_scales(s, s_ref, g is not None, label)
    return 0


def check_scales(s, s_ref, norm, label):
    nz = s_ref != 0
    assert np.array_equal(s == 0, ~nz), label
    assert rel_err(s[nz], s_ref[nz]) <= REL, label
    if not norm:
        assert np.array_equal(s, s_ref), label


ACT_SHAPES = [(1, 16), (3, 272), (7, 2048), (33, 6144), (5, 9728), (2, 16384)]


@pytest.mark.parametrize("M,K", ACT_SHAPES)
@pytest.mark.parametrize("kind", [1, 2, 3])
@pytest.mark.parametrize("norm", [False, True])
def test_act_quant_ffn(torch, bl, orc, M, K, kind, norm):
    G = workloads.gaussian((M, K), (300, M, K, kind), 2.0)
    U = workloads.gaussian((M, K), (301, M, K, kind), 1.0)
    if M > 2:
        G[1] = -np.abs(G[1])                # relu kills the row (all zeros for ReLU kinds)
        U[2] = 0.0                          # up row of zeros
    g = (np.float32(1) + workloads.gaussian((K,), (302, K), 0.1)) if norm else None
    glu = kind in (orc.SWIGLU, orc.RELU2_GLU)
    Xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
    sx = torch.empty(M, dtype=torch.float32, device="cuda")
    bl.quantize_acts_ex_grouped([dict(X=dev(torch, G), X2=dev(torch, U) if glu else None, act=kind,
                                      norm_weight=None if g is None else dev(torch, g),
                                      X_q=Xq, x_scale=sx, eps=1e-6)])
    torch.cuda.synchronize()
    check_ffn_quant(host(Xq), host(sx), G, U, g, kind, orc, (M, K, kind, norm))


@pytest.mark.parametrize("K", [272, 9728])
def test_act_quant_ffn_extreme_gates(torch, bl, orc, K):
    """SwiGLU with gate values where exp(-g) saturates or is tiny (|g| of 100, 700, 750),
    denormal and signed-zero gates, mixed with ordinary values: codes and scales as the
    oracle's (its exp from the host library), differences only at fp32 ties of h."""
    M = 6
    G = workloads.gaussian((M, K), (310, K), 2.0)
    U = workloads.gaussian((M, K), (311, K), 1.0)
    special = np.array([100.0, -100.0, 700.0, -700.0, 750.0, -750.0, 1e-40, -1e-40, 0.0, -0.0,
                        30.0, -30.0], np.float32)
    for m in range(M):
        idx = np.random.Generator(np.random.PCG64([312, m, K])).choice(K, size=special.size, replace=False)
        G[m, idx] = special
    G[M - 1, :] = np.float32(-750.0)        # a row whose h is all -0 or tiny: absmax from zeros
    Xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
    sx = torch.empty(M, dtype=torch.float32, device="cuda")
    bl.quantize_acts_ex_grouped([dict(X=dev(torch, G), X2=dev(torch, U), act=orc.SWIGLU, X_q=Xq,
                                      x_scale=sx)])
    torch.cuda.synchronize()
    check_ffn_quant(host(Xq), host(sx), G, U, None, orc.SWIGLU, orc, ("extremes", K))


def test_act_quant_ex_mixed_group(torch, bl, orc):
    """Plain, bf16 and activation problems in one call give what separate calls give."""
    A = workloads.gaussian((40, 768), (303,), 1.0)
    Bb = workloads.f32_to_bf16_bits(workloads.gaussian((9, 2048), (304,), 1.0))
    G = workloads.gaussian((17, 512), (305,), 1.5)
    U = workloads.gaussian((17, 512), (306,), 1.0)
    outs = [(torch.empty(s, dtype=torch.int8, device="cuda"), torch.empty(s[0], device="cuda"))
            for s in [(40, 768), (9, 2048), (17, 512)]]
    Bt = dev(torch, Bb.view(np.int16)).view(torch.bfloat16)
    bl.quantize_acts_ex_grouped([
        dict(X=dev(torch, A), X_q=outs[0][0], x_scale=outs[0][1]),
        dict(X=Bt, X_q=outs[1][0], x_scale=outs[1][1], norm_weight=dev(torch, np.ones(2048, np.float32))),
        dict(X=dev(torch, G), X2=dev(torch, U), act=2, X_q=outs[2][0], x_scale=outs[2][1]),
    ])
    torch.cuda.synchronize()
    qa, sa = orc.quantize_acts(A)
    qb, sb = orc.quantize_acts(Bb, np.ones(2048, np.float32), 1e-6, bf16=True)
    qc, sc = orc.quantize_acts(orc.ffn_act(2, G, U))
    assert np.array_equal(host(outs[0][0]), qa) and np.array_equal(host(outs[0][1]), sa)
    assert np.array_equal(host(outs[1][0]), qb) and rel_err(host(outs[1][1]), sb) <= REL
    assert np.array_equal(host(outs[2][0]), qc) and np.array_equal(host(outs[2][1]), sc)


FWD_RES = [(1, 40, 768), (3, 130, 272), (16, 2048, 512), (100, 130, 272), (300, 257, 1040),
           (517, 512, 768)]


@pytest.mark.parametrize("M,N,K", FWD_RES)
@pytest.mark.parametrize("alias", [False, True])
def test_forward_residual(torch, bl, orc, M, N, K, alias):
    C = workloads.ternary((N, K), (310, N, K))
    X = workloads.gaussian((M, K), (311, M, K), 1.0)
    R = workloads.gaussian((M, N), (312, M, N), 2.0)
    P = bl.pack_codes(dev(torch, C))
    Xq, sx = bl.quantize_acts(dev(torch, X))
    gamma = dev(torch, np.array([GAMMA], np.float32))
    Rt = dev(torch, R)
    Y = Rt if alias else torch.empty((M, N), dtype=torch.float32, device="cuda")
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda")
    bl.forward_ex_grouped([dict(X_q=Xq, x_scale=sx, W_packed=P, gamma=gamma, Y=Y, acc=acc, residual=Rt)])
    torch.cuda.synchronize()
    acc_ref = orc.matmul(host(Xq), C)
    assert np.array_equal(host(acc), acc_ref)
    Y_ref = orc.epilogue_residual(acc_ref, host(sx), GAMMA, R)
    assert np.array_equal(host(Y), Y_ref), (M, N, K, alias)


def make_layer(torch, bl, d, F, names, act, key, norms=True):
    from bit_gemm_02_amd.layer import LayerWeights
    shapes = {"q": (d, d), "k": (d // 2, d), "v": (d // 2, d), "qkv": (2 * d, d), "o": (d, d),
              "gate": (F, d), "up": (F, d), "down": (d, F)}
    packed, gamma, codes = {}, {}, {}
    for i, n in enumerate(names):
        C = workloads.ternary(shapes[n], (320, i) + key)
        codes[n] = C
        packed[n] = bl.pack_codes(dev(torch, C))
        gamma[n] = dev(torch, np.array([0.02 + 0.001 * i], np.float32))
    nrm = {}
    if norms:
        for i, (n, k) in enumerate([("attn", d), ("o", d), ("ffn", d), ("down", F)]):
            nrm[n] = dev(torch, np.float32(1) + workloads.gaussian((k,), (321, i) + key, 0.1))
    return LayerWeights(packed=packed, gamma=gamma, norms=nrm, act=act), codes


LAYERS = [
    (256, 512, ("q", "k", "v", "o", "gate", "up", "down"), 1),
    (256, 512, ("q", "k", "v", "o", "gate", "up", "down"), 2),
    (256, 768, ("qkv", "o", "up", "down"), 3),
    (272, 528, ("o", "gate", "up", "down"), 1),
]


@pytest.mark.parametrize("d,F,names,act", LAYERS)
@pytest.mark.parametrize("M", [1, 3, 64, 200])
def test_layer_chain_stagewise(torch, bl, orc, d, F, names, act, M):
    from bit_gemm_02_amd.layer import LayerChain
    w, codes = make_layer(torch, bl, d, F, names, act, (M, act, d))
    ch = LayerChain(w, M, keep_codes=True)
    assert ch.fused == (M <= 4)
    assert len(ch._calls) == (3 if ch.fused else 6)
    x = workloads.gaussian((M, d), (330, M, d), 1.0)
    a = workloads.gaussian((M, w.K("o")), (331, M, d), 1.0)
    ch.x.copy_(dev(torch, x))
    ch.attn.copy_(dev(torch, a))
    ch()
    torch.cuda.synchronize()
    gv = {n: np.float32(host(w.gamma[n])[0]) for n in names}
    nv = {n: host(t) for n, t in w.norms.items()}
    label = (d, F, names, act, M)
    # A1: input norm on x, SubLN on the attention output.
    if w.attn_in:
        q1, s1 = orc.quantize_acts(x, nv["attn"], 1e-6)
        assert np.array_equal(host(ch.xq), q1), label
        check_scales(host(ch.xs), s1, True, label)
    q2, s2 = orc.quantize_acts(a, nv["o"], 1e-6)
    assert np.array_equal(host(ch.aq), q2), label
    check_scales(host(ch.as_), s2, True, label)
    # P1: q/k/v on the GPU's codes; o with the residual x.
    for n in w.attn_in:
        Yr = orc.epilogue(orc.matmul(host(ch.xq), codes[n]), host(ch.xs), gv[n])
        assert np.array_equal(host(ch.y[n]), Yr), (label, n)
    x1 = orc.epilogue_residual(orc.matmul(host(ch.aq), codes["o"]), host(ch.as_), gv["o"], x)
    assert np.array_equal(host(ch.x1), x1), label
    # A2, P2 on the GPU's x1.
    q3, s3 = orc.quantize_acts(host(ch.x1), nv["ffn"], 1e-6)
    assert np.array_equal(host(ch.fq), q3), label
    check_scales(host(ch.fs), s3, True, label)
    up = orc.epilogue(orc.matmul(host(ch.fq), codes["up"]), host(ch.fs), gv["up"])
    gate = None
    if "gate" in names:
        gate = orc.epilogue(orc.matmul(host(ch.fq), codes["gate"]), host(ch.fs), gv["gate"])
    if ch.fused:
        # L2's epilogue: h = act(gate, up) from the pair's fp32 outputs.
        H = host(ch.h)
        check_hidden(H, gate, up, act, orc, label)
        # L3's quantization of the GPU's own h, with SubLN.
        q4, s4 = orc.quantize_acts(H, nv["down"], 1e-6)
        assert np.array_equal(host(ch.hq), q4), label
        check_scales(host(ch.hs), s4, True, label)
    else:
        assert np.array_equal(host(ch.up), up), label
        if gate is not None:
            assert np.array_equal(host(ch.gate), gate), label
        # A3: FFN activation + SubLN on the GPU's gate and up outputs.
        G, U = (host(ch.gate), host(ch.up)) if gate is not None else (host(ch.up), None)
        check_ffn_quant(host(ch.hq), host(ch.hs), G, U, nv["down"], act, orc, label)
    # P3: down with the residual x1, on the GPU's codes.
    out = orc.epilogue_residual(orc.matmul(host(ch.hq), codes["down"]), host(ch.hs), gv["down"],
                                host(ch.x1))
    assert np.array_equal(host(ch.out), out), label


def check_hidden(H, gate, up, kind, orc, label):
    """The fused epilogue's h against act(gate, up) of the oracle's gate and up outputs: bit-
    exact, except SwiGLU values at an fp32 tie of the oracle's fp64 h (the device library's exp
    against the host's), which may take the other rounding (tie_band.check_values)."""
    if kind != orc.SWIGLU:
        H_ref = orc.ffn_act(kind, gate, up) if gate is not None else orc.ffn_act(kind, up)
        assert np.array_equal(H, H_ref), label
        return
    flips = tie_band.check_values(H, orc.ffn_act_f64(kind, gate, up), label)
    if flips:
        print(f"{label}: {flips} of {H.size} SwiGLU values at an fp32 tie took the other rounding")


@pytest.mark.parametrize("d,F,names,act", LAYERS)
@pytest.mark.parametrize("M", [1, 2, 4])
def test_layer_chain_forms_agree(torch, bl, d, F, names, act, M):
    """Three-launch and six-launch forms on the same layer and input: the same codes at
    every stage and outputs within the last-bit differences of the norms' scales."""
    from bit_gemm_02_amd.layer import LayerChain
    w, _ = make_layer(torch, bl, d, F, names, act, (M, act, d, 7))
    fz = LayerChain(w, M, keep_codes=True)
    sx = LayerChain(w, M, fused=False)
    assert fz.fused and not sx.fused
    x = dev(torch, workloads.gaussian((M, d), (332, M, d), 1.0))
    a = dev(torch, workloads.gaussian((M, w.K("o")), (333, M, d), 1.0))
    for ch in (fz, sx):
        ch.x.copy_(x)
        ch.attn.copy_(a)
        ch()
    torch.cuda.synchronize()
    for name in ("xq", "aq", "fq", "hq"):
        if name == "xq" and not w.attn_in:
            continue
        diff = np.count_nonzero(host(getattr(fz, name)) != host(getattr(sx, name)))
        assert diff <= max(1, getattr(fz, name).numel() // 10000), (name, diff)
    for name in ["x1", "out"] + [f"y:{n}" for n in w.attn_in]:
        get = (lambda c: c.y[name[2:]]) if name.startswith("y:") else (lambda c: getattr(c, name))
        A, B = host(get(fz)), host(get(sx))
        scale = float(np.max(np.abs(B))) or 1.0
        assert np.allclose(A, B, rtol=1e-4, atol=1e-4 * scale), name


def test_layer_chain_graph_replay(torch, bl):
    """The chain's launches (six; three in the fused form at two tokens) captured in a HIP
    graph give the eager result on every replay, with eager work and synchronizations
    between the replays."""
    from bit_gemm_02_amd.layer import LayerChain
    for M in (64, 2):
        check_graph_replay(torch, bl, LayerChain, M)


def check_graph_replay(torch, bl, LayerChain, M):
    w, _ = make_layer(torch, bl, 256, 512, ("q", "k", "v", "o", "gate", "up", "down"), 1, (9,))
    ch = LayerChain(w, M)
    ch.x.copy_(dev(torch, workloads.gaussian((M, 256), (340,), 1.0)))
    ch.attn.copy_(dev(torch, workloads.gaussian((M, 256), (341,), 1.0)))
    ch()
    torch.cuda.synchronize()
    ref = ch.out.clone()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        ch(s)                               # warm the side stream
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        ch(s)
    for i in range(4):
        ch.out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ch.out, ref), i
        ch()                                # eager work between replays
        torch.cuda.synchronize()
