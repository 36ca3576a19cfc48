"""Full-size parity on every workload shape, in the launch configuration the benchmark times
(one grouped weight quantization, one grouped activation quantization and one grouped
forward over the whole layer set).

Per matrix and token count:
  * gamma within 1e-6 relative; packed codes bit-exact against the oracle's codes computed
    with the GPU's gamma (every weight), flips against the oracle's own gamma only inside the
    1e-6 band around |W / gamma| = 0.5 (counted);
  * int8 activations bit-exact and scales within 1e-6 (every element);
  * int32 accumulators: exact integer Freivalds check acc v == X_q (C^T v) over all of them
    (C unpacked by the oracle from the GPU's packed words), plus bit-exact equality with the
    oracle on sampled entries (corners and random positions);
  * fp32 outputs: equal (within 1e-6 relative) to the oracle epilogue applied to the
    accumulators, everywhere, and to the oracle's sampled entries.
"""

import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu

REL = 1e-6
SAMPLES = 384


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
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.cpu().numpy()


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if a.size == 0:
        return 0.0
    return float(np.max(np.abs(a - b) / np.maximum(np.abs(b), 1e-300)))


def freivalds(acc, Xq, C, rounds=2, seed=0):
    """Exact integer check of acc == Xq C^T (all partial sums stay below 2^53 in fp64)."""
    g = np.random.Generator(np.random.PCG64([seed, acc.shape[0], acc.shape[1]]))
    Cf = C.astype(np.float64)
    Xf = Xq.astype(np.float64)
    Af = acc.astype(np.float64)
    for _ in range(rounds):
        v = g.integers(-1000, 1001, size=acc.shape[1]).astype(np.float64)
        lhs = Af @ v
        rhs = Xf @ (Cf.T @ v)
        assert np.array_equal(lhs, rhs)


def sample_positions(M, N, seed):
    g = np.random.Generator(np.random.PCG64([seed, M, N]))
    m = np.concatenate([[0, 0, M - 1, M - 1], g.integers(0, M, SAMPLES)])
    n = np.concatenate([[0, N - 1, 0, N - 1], g.integers(0, N, SAMPLES)])
    return m.astype(np.int64), n.astype(np.int64)


CASES = [(key, M) for key, wl in workloads.WORKLOADS.items() for M in wl.token_counts]


@pytest.mark.parametrize("key,M", CASES, ids=[f"{k}-M{M}" for k, M in CASES])
def test_workload(torch, bl, orc, key, M):
    wl = workloads.WORKLOADS[key]
    mats = wl.matrices
    n = len(mats)
    # Weights: fp32 masters quantized in one grouped call, or pre-ternarized codes packed.
    if wl.weights == "fp32":
        W_host = [workloads.weight_fp32(wl, i) for i in range(n)]
        outs = bl.quantize_weights_grouped([dev(torch, w) for w in W_host])
        P = [o[0] for o in outs]
        G = [o[1] for o in outs]
    else:
        W_host = None
        codes = [workloads.weight_codes(wl, i) for i in range(n)]
        P = [bl.pack_codes(dev(torch, c)) for c in codes]
        G = [torch.full((1,), wl.code_gamma, dtype=torch.float32, device="cuda") for _ in mats]
    X_host = [workloads.activations(wl, i, M) for i in range(n)]
    g_host = [workloads.norm_weight(wl, i, kind="parity") if m.norm else None
              for i, m in enumerate(mats)]
    acts = bl.quantize_acts_grouped([dev(torch, x) for x in X_host],
                                    [None if g is None else dev(torch, g) for g in g_host], 1e-6)
    probs = []
    for i, m in enumerate(mats):
        probs.append(dict(X_q=acts[i][0], x_scale=acts[i][1], W_packed=P[i], gamma=G[i],
                          Y=torch.empty((M, m.N), dtype=torch.float32, device="cuda"),
                          acc=torch.empty((M, m.N), dtype=torch.int32, device="cuda")))
    bl.forward_grouped(probs)
    torch.cuda.synchronize()

    flips_total = 0
    for i, m in enumerate(mats):
        label = f"{key} M={M} {m.name}"
        Ph = host(P[i]).view(np.uint32)
        gamma = np.float32(host(G[i])[0])
        # Weights.
        if W_host is not None:
            W = W_host[i]
            g_orc, g64 = orc.gamma(W)
            assert rel_err(gamma, g_orc) <= REL, label
            assert np.array_equal(Ph, orc.pack(orc.ternary_codes(W, gamma))), label
            C = orc.unpack(Ph, m.K)
            flips = C != orc.ternary_codes(W, g_orc)
            if flips.any():
                t = np.abs(W.astype(np.float64) / g64)
                assert np.all(np.abs(t[flips] - 0.5) <= 1e-6), label
            flips_total += int(flips.sum())
        else:
            assert np.array_equal(Ph, orc.pack(codes[i])), label
            C = codes[i]
        # Activations.
        Xq = host(acts[i][0])
        sx = host(acts[i][1])
        q_ref, s_ref = orc.quantize_acts(X_host[i], g_host[i], 1e-6, bf16=(wl.x_dtype == "bf16"))
        assert np.array_equal(Xq, q_ref), label
        nz = s_ref != 0
        assert np.array_equal(sx == 0, ~nz) and rel_err(sx[nz], s_ref[nz]) <= REL, label
        # Accumulators and outputs.
        acc = host(probs[i]["acc"])
        Y = host(probs[i]["Y"])
        freivalds(acc, Xq, C, seed=i)
        mi, ni = sample_positions(M, m.N, i)
        ea, ey = orc.forward_entries(Xq, sx, Ph, gamma, mi, ni)
        assert np.array_equal(acc[mi, ni], ea), label
        assert rel_err(Y[mi, ni], ey) <= REL and np.array_equal(Y[mi, ni] == 0, ey == 0), label
        Y_ref = orc.epilogue(acc, sx, gamma)
        assert np.array_equal(Y == 0, Y_ref == 0), label
        assert rel_err(Y[Y_ref != 0], Y_ref[Y_ref != 0]) <= REL, label
    print(f"{key} M={M}: {n} matrices ok, code flips in the 1e-6 band: {flips_total}")


@pytest.mark.parametrize("key", sorted(workloads.WORKLOADS))
def test_workload_decode_leg(torch, bl, orc, key):
    """The benchmark's decode leg at full size: every matrix of the layer set in one grouped
    fused call at one token (activation quantization inside the product), on weights packed
    as the benchmark packs them (from the fp32 masters, or from the pre-ternarized codes) and
    the workload's own one-token activations and norm weights.  Codes bit-exact and scales
    within 1e-6 (through the call's optional outputs); Y equal to the oracle's product and
    epilogue on the oracle's own codes and scales, within 1e-6 relative, zeros exact."""
    wl = workloads.WORKLOADS[key]
    mats = wl.matrices
    calls, refs = [], []
    for i, m in enumerate(mats):
        if wl.weights == "fp32":
            P, g = bl.quantize_weights(dev(torch, workloads.weight_fp32(wl, i)))
        else:
            P = bl.pack_codes(dev(torch, workloads.weight_codes(wl, i)))
            g = torch.full((1,), wl.code_gamma, device="cuda")
        x = workloads.activations(wl, i, 1)
        nw = workloads.norm_weight(wl, i) if m.norm else None
        calls.append(dict(X=dev(torch, x), W_packed=P, gamma=g, norm_weight=None if nw is None else dev(torch, nw),
                          Y=torch.empty((1, m.N), device="cuda"),
                          X_q=torch.empty((1, m.K), dtype=torch.int8, device="cuda"),
                          x_scale=torch.empty(1, device="cuda"), eps=1e-6))
        refs.append((x, nw))
    assert all(bl.linear_fused(1, m.K) for m in mats)
    bl.linear_grouped(calls)
    torch.cuda.synchronize()
    bf16 = wl.x_dtype == "bf16"
    for i, m in enumerate(mats):
        x, nw = refs[i]
        c = calls[i]
        q_ref, s_ref = orc.quantize_acts(x, nw, 1e-6, bf16=bf16)
        q, s, Y = host(c["X_q"]), host(c["x_scale"]), host(c["Y"])
        assert np.array_equal(q, q_ref), (key, m.name)
        assert rel_err(s, s_ref) <= REL, (key, m.name)
        codes = orc.unpack(host(c["W_packed"]).view(np.uint32), m.K)
        gamma = np.float32(host(c["gamma"])[0])
        Y_ref = orc.epilogue(orc.matmul(q_ref, codes), s_ref, gamma)
        assert np.array_equal(Y == 0, Y_ref == 0), (key, m.name)
        nz = Y_ref != 0
        assert rel_err(Y[nz], Y_ref[nz]) <= REL, (key, m.name)
