"""One-read weight quantization (sample, pass with a listed band, fix-up; taken for sets of at
least 64 MB of fp32 weights when the workspace holds its lists): gamma and every packed word
equal bit for bit to the two-read form's, and the codes equal the oracle's at the GPU's gamma
(gamma within 1e-6 of the oracle's).  Cases: Qwen3-4B-shaped projections in rows and quad rows
with their step activations; tensors that make the fix-up code its part of W again (a sample
ten times larger than the rest of the tensor, a list overflow from half the weights sitting on
the rounding boundary, all zeros, a NaN, an inf), ragged, one-row and empty tensors in a large
set; weights planted on the code boundary and its fp32 neighbours in a tensor whose band holds,
so that the fix-up decides them; the step call's activation rows in each launch they can take;
repeated calls giving the same words (the lists' order never reaches a result); and the step
call replayed from a captured HIP graph, with eager calls sharing its workspace in between.
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


def sampled_mask(N, K):
    """Weights the sample reads: the first 1024 of every 16384 (flat index)."""
    m = np.zeros(N * K, dtype=bool)
    for s in range(0, N * K, 16384):
        m[s:s + 1024] = True
    return m.reshape(N, K)


def check_set(torch, bl, orc, Ws_h, quad=False, acts=False, label=""):
    """One-read against two-read (bit for bit) and against the oracle."""
    Ws = [dev(torch, W) for W in Ws_h]
    total = sum(W.nbytes for W in Ws_h)
    assert total >= 64 << 20, "the set must be large enough for the one-read form"
    Xs = [dev(torch, workloads.gaussian((3, W.shape[1]), (611, i), 1.0)) for i, W in enumerate(Ws_h)] if acts else []
    if acts or quad:
        w1, x1 = bl.quantize_step(Ws, Xs, quad_rows=quad, one_read=True)
        w2, x2 = bl.quantize_step(Ws, Xs, quad_rows=quad, one_read=False)
        for (a, b), (c, d) in zip(x1, x2):
            assert torch.equal(a, c) and torch.equal(b, d), label
    else:
        w1 = bl.quantize_weights_grouped(Ws, one_read=True)
        w2 = bl.quantize_weights_grouped(Ws, one_read=False)
    torch.cuda.synchronize()
    for i, ((P1, g1), (P2, g2), W) in enumerate(zip(w1, w2, Ws_h)):
        tag = (label, i, W.shape)
        assert np.array_equal(host(g1).view(np.uint32), host(g2).view(np.uint32)), tag
        assert torch.equal(P1, P2), tag
        if W.size == 0:
            continue
        g_gpu = np.float32(host(g1)[0])
        g_orc, _ = orc.gamma(W)
        if np.isfinite(g_orc):
            assert abs(float(g_gpu) / float(g_orc) - 1.0) <= REL if g_orc != 0 else g_gpu == 0, tag
        else:
            assert not np.isfinite(g_gpu), tag
        ref = orc.pack(orc.ternary_codes(W, g_gpu))
        if quad:
            N, K = W.shape
            ref = ref.reshape(N // 4, 4, K // 128, 8).transpose(0, 2, 1, 3).reshape(-1)
        assert np.array_equal(host(P1).view(np.uint32).reshape(-1), ref.reshape(-1)), tag


QWEN = [(4096, 2560), (1024, 2560), (1024, 2560), (2560, 4096), (2560, 9728)]


@pytest.mark.parametrize("quad", [False, True])
def test_one_read_qwen_projections(torch, bl, orc, quad):
    Ws = [workloads.gaussian(s, (610, i), 0.02) for i, s in enumerate(QWEN)]
    check_set(torch, bl, orc, Ws, quad=quad, acts=True, label=("qwen", quad))


def test_one_read_grouped_call(torch, bl, orc):
    Ws = [workloads.gaussian(s, (612, i), 0.02) for i, s in enumerate(QWEN[:4])]
    check_set(torch, bl, orc, Ws, label="grouped")


def test_one_read_fallbacks(torch, bl, orc):
    base = workloads.gaussian((4096, 4096), (613, 0), 0.02)
    # Sample unrepresentative: the sampled pieces ten times larger (the band misses tau).
    skew = workloads.gaussian((1024, 2560), (613, 1), 0.02)
    skew[sampled_mask(*skew.shape)] *= np.float32(10)
    # Half the weights exactly on the boundary: |w| in {1, 3}, gamma = 2, tau = 1 (ties to 0);
    # every weight of magnitude 1 is listed, far more than a list holds.
    rng = np.random.default_rng(614)
    tie = np.where(rng.random((512, 2048)) < 0.5, 1.0, 3.0).astype(np.float32)
    tie *= np.where(rng.random(tie.shape) < 0.5, -1, 1).astype(np.float32)
    zero = np.zeros((256, 512), np.float32)
    nan = workloads.gaussian((64, 1024), (613, 2), 0.02)
    nan[17, 300] = np.nan
    inf = workloads.gaussian((64, 1024), (613, 3), 0.02)
    inf[5, 7] = -np.inf
    ragged = workloads.gaussian((1001, 2576), (613, 4), 0.02)
    one = workloads.gaussian((1, 16), (613, 5), 0.02)
    empty = np.zeros((0, 64), np.float32)
    Ws = [base, skew, tie, zero, nan, inf, ragged, one, empty]
    check_set(torch, bl, orc, Ws, label="fallbacks")


def test_one_read_tie_and_ragged_quad(torch, bl, orc):
    """The fall-back coding and the fix-up in the quad-row layout."""
    base = workloads.gaussian((4096, 4096), (615, 0), 0.02)
    rng = np.random.default_rng(616)
    tie = np.where(rng.random((512, 2048)) < 0.5, 1.0, 3.0).astype(np.float32)
    ragged = workloads.gaussian((1004, 2560), (615, 1), 0.02)
    check_set(torch, bl, orc, [base, tie, ragged], quad=True, label="quad fallbacks")


def test_one_read_repeatable(torch, bl):
    Ws = [dev(torch, workloads.gaussian(s, (617, i), 0.02)) for i, s in enumerate(QWEN[:4])]
    a = bl.quantize_weights_grouped(Ws, one_read=True)
    b = bl.quantize_weights_grouped(Ws, one_read=True)
    torch.cuda.synchronize()
    for (P1, g1), (P2, g2) in zip(a, b):
        assert torch.equal(P1, P2) and torch.equal(g1, g2)


def test_one_read_step_activation_routing(torch, bl, orc):
    """The step call's activation rows in every launch the one-read form routes them to: fp32
    rows of up to 4096 values with the sample, bf16 rows longer than 4096 with the fix-up, and
    the rest (fp32 rows longer than 4096, bf16 rows of up to 4096, a norm) as launches of their
    own; codes and scales against the two-read call and the oracle."""
    shapes = [(4096, 2560), (2560, 9728), (1024, 1024)]
    Ws = [dev(torch, workloads.gaussian(s, (618, i), 0.02)) for i, s in enumerate(shapes)]
    specs = [(17, 2560, False, False), (9, 9728, True, True), (5, 9728, False, False),
             (33, 1024, True, False), (3, 4096, False, True)]
    Xs, host_x, gs = [], [], []
    for i, (M, K, bf, nm) in enumerate(specs):
        X = workloads.gaussian((M, K), (619, i), 1.0)
        g = (np.float32(1) + workloads.gaussian((K,), (620, i), 0.1)) if nm else None
        if bf:
            bits = workloads.f32_to_bf16_bits(X)
            Xs.append(dev(torch, bits.view(np.int16)).view(torch.bfloat16))
            host_x.append((bits, g, True))
        else:
            Xs.append(dev(torch, X))
            host_x.append((X, g, False))
        gs.append(None if g is None else dev(torch, g))
    for quad in (False, True):
        w1, x1 = bl.quantize_step(Ws, Xs, gs, 1e-6, quad_rows=quad, one_read=True)
        w2, x2 = bl.quantize_step(Ws, Xs, gs, 1e-6, quad_rows=quad, one_read=False)
        torch.cuda.synchronize()
        for (P1, g1), (P2, g2) in zip(w1, w2):
            assert torch.equal(P1, P2) and torch.equal(g1, g2), quad
        for i, ((q1, s1), (q2, s2)) in enumerate(zip(x1, x2)):
            assert torch.equal(q1, q2) and torch.equal(s1, s2), (quad, i)
            x, g, bf = host_x[i]
            q_ref, s_ref = orc.quantize_acts(x, g, 1e-6, bf16=bf)
            assert np.array_equal(host(q1), q_ref), (quad, i)
            sn = host(s1)
            nz = s_ref != 0
            assert np.array_equal(sn == 0, ~nz), (quad, i)
            assert np.max(np.abs(sn[nz].astype(np.float64) / s_ref[nz] - 1.0)) <= REL, (quad, i)


def test_one_read_weights_on_the_threshold(torch, bl, orc):
    """Weights at the code boundary and its fp32 neighbours, inside a tensor whose sample gives
    a good band, so they are listed by the pass and decided by the fix-up."""
    rng = np.random.default_rng(621)
    W = workloads.gaussian((4096, 4096), (622, 0), 0.02)
    idx = rng.choice(W.size, size=600, replace=False)
    flat = W.reshape(-1)
    for _ in range(3):
        g32, _ = orc.gamma(W)
        # The boundary from the oracle's codes: the smallest fp32 magnitude coded nonzero.
        cand = np.float32(g32) * np.float32(0.5)
        probe = np.array([np.nextafter(cand, np.float32(0), dtype=np.float32), cand,
                          np.nextafter(cand, np.float32(1), dtype=np.float32),
                          np.nextafter(np.nextafter(cand, np.float32(1), dtype=np.float32),
                                       np.float32(1), dtype=np.float32)], np.float32)
        codes = orc.ternary_codes(probe.reshape(1, -1), g32)[0]
        lo_zero = probe[codes == 0].max()
        hi_one = probe[codes != 0].min()
        vals = np.array([lo_zero, hi_one, np.nextafter(lo_zero, np.float32(0), dtype=np.float32),
                         np.nextafter(hi_one, np.float32(1), dtype=np.float32)], np.float32)
        signs = np.where(np.arange(idx.size) % 2 == 0, 1, -1).astype(np.float32)
        flat[idx] = vals[np.arange(idx.size) % 4] * signs
    Ws = [W, workloads.gaussian((2560, 4096), (622, 1), 0.02)]
    check_set(torch, bl, orc, Ws, label="threshold")
    check_set(torch, bl, orc, Ws, quad=True, acts=True, label="threshold quad")


def test_one_read_single_tensor_call(torch, bl, orc):
    """bitlinear_quantize_weights on one 64 MB tensor (the one-read form through the single
    call) against the two-read call and the oracle."""
    W = workloads.gaussian((4096, 4096), (623, 0), 0.02)
    Wd = dev(torch, W)
    P1, g1 = bl.quantize_weights(Wd, one_read=True)
    P2, g2 = bl.quantize_weights(Wd, one_read=False)
    torch.cuda.synchronize()
    assert torch.equal(P1, P2) and torch.equal(g1, g2)
    g_gpu = np.float32(host(g1)[0])
    g_orc, _ = orc.gamma(W)
    assert abs(float(g_gpu) / float(g_orc) - 1.0) <= REL
    assert np.array_equal(host(P1).view(np.uint32), orc.pack(orc.ternary_codes(W, g_gpu)))


def test_one_read_graph_replays(torch, bl):
    """The step call in the one-read form captured in a HIP graph and replayed three times,
    with eager calls on other inputs in between (the workspace's lists, counts and band are
    rewritten by every call): every replay equals the eager call bit for bit."""
    shapes = [(4096, 2560), (2560, 9728)]
    Ws = [dev(torch, workloads.gaussian(s, (624, i), 0.02)) for i, s in enumerate(shapes)]
    Xs = [dev(torch, workloads.gaussian((65, s[1]), (625, i), 1.0)) for i, s in enumerate(shapes)]
    Wo = [dev(torch, workloads.gaussian(s, (626, i), 0.03)) for i, s in enumerate(shapes)]
    ref_w, ref_x = bl.quantize_step(Ws, Xs, quad_rows=True)
    torch.cuda.synchronize()
    outs_w = [(torch.empty_like(P), torch.empty_like(g)) for P, g in ref_w]
    outs_x = [(torch.empty_like(q), torch.empty_like(s)) for q, s in ref_x]
    nbytes = max(bl.quantize_weights_workspace_bytes(len(Ws)),
                 bl.quantize_weights_one_read_workspace_bytes(_problems(bl, Ws), len(Ws)))
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        bl.quantize_step(Ws, Xs, w_outputs=outs_w, x_outputs=outs_x, workspace=ws, quad_rows=True,
                         stream=stream)          # warm-up outside capture
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        bl.quantize_step(Ws, Xs, w_outputs=outs_w, x_outputs=outs_x, workspace=ws, quad_rows=True,
                         stream=stream)
    for rep in range(3):
        for P, g in outs_w:
            P.zero_()
            g.zero_()
        # Eager work on other weights through the same workspace between replays.
        bl.quantize_step(Wo, [], workspace=ws, quad_rows=True)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for (P, g), (P2, g2) in zip(outs_w, ref_w):
            assert torch.equal(P, P2) and torch.equal(g, g2), rep
        for (q, s), (q2, s2) in zip(outs_x, ref_x):
            assert torch.equal(q, q2) and torch.equal(s, s2), rep


def _problems(bl, Ws):
    import ctypes
    arr = (bl._WeightProblem * len(Ws))()
    for i, W in enumerate(Ws):
        N, K = W.shape
        arr[i] = bl._WeightProblem(W.data_ptr(), None, None, N, K)
    return arr
