"""The mixed batch (bitlinear_forward_mixed): prefill products and fused decode layer calls in
one call, one launch when both sets allow it.

Per case: every output (Y and the int32 sums of the prefill products; Y and the optional code
and scale outputs of the decode calls) equal bit for bit to the two calls it replaces,
bitlinear_forward_ex_grouped(prefill) then bitlinear_linear_grouped(decode), run on the same
inputs; and both sets checked against the CPU oracle: prefill entries sampled one by one
(int32 sums exact, Y within 1e-6), decode calls in full (codes exact, scales and Y within
1e-6).  Cases: the Distillix-125M layer set at 2048 prefill tokens with one decode token,
ragged sizes (K not a multiple of the 128-wide prefill stage or of the 256-wide decode step,
N not a multiple of the tile), bf16 decode activations with a norm, empty problems, and the
cases that take the two-launch path (a prefill product of at most 16 tokens, a decode call
past the fused size, mixed decode dtypes, a prefill set large enough for 128 x 256 tiles,
one set empty).
"""

import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu

REL = 1e-6
GAMMA = np.float32(0.021)
BL_OK, BL_ERR_NULL, BL_ERR_SHAPE, BL_ERR_COUNT = 0, -1, -2, -7


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


def rng(key):
    return np.random.Generator(np.random.PCG64([317] + list(key)))


def make_pre(torch, bl, M, N, K, key):
    """A prefill product on int8 codes and positive row scales; host copies for the oracle."""
    g = rng((0, M, N, K) + key)
    Xq = g.integers(-127, 128, size=(M, K), dtype=np.int8)
    sx = (np.abs(g.standard_normal(M)).astype(np.float32) + np.float32(0.01)) / np.float32(127)
    C = workloads.ternary((N, K), (318, N, K) + key)
    P = bl.pack_codes(dev(torch, C)) if N and K else torch.zeros((N, K // 16), dtype=torch.int32, device="cuda")
    p = dict(X_q=dev(torch, Xq), x_scale=dev(torch, sx), W_packed=P,
             gamma=dev(torch, np.array([GAMMA], np.float32)),
             Y=torch.empty((M, N), dtype=torch.float32, device="cuda"),
             acc=torch.empty((M, N), dtype=torch.int32, device="cuda"))
    return p, dict(Xq=Xq, sx=sx)


def make_dec(torch, bl, M, N, K, dtype, norm, key):
    X = workloads.gaussian((M, K), (319, M, N, K) + key, 1.0)
    gw = (np.float32(1) + workloads.gaussian((K,), (320, K) + key, 0.1)) if norm else None
    C = workloads.ternary((N, K), (321, N, K) + key)
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
                norm_weight=None if gw is None else dev(torch, gw), eps=1e-6)
    return call, dict(x=xin, g=gw, C=C, bf16=dtype == "bf16")


def fresh(torch, problems, keys):
    """Copies of the problem dicts with new output buffers (inputs shared)."""
    out = []
    for p in problems:
        q = dict(p)
        for k in keys:
            if q.get(k) is not None:
                q[k] = torch.full_like(q[k], -7)
        out.append(q)
    return out


def run_both(torch, bl, pre, dec):
    """The mixed call and the two calls it replaces, on separate outputs."""
    pre2 = fresh(torch, pre, ("Y", "acc"))
    dec2 = fresh(torch, dec, ("Y", "X_q", "x_scale"))
    # The same fill on both sides, so outputs that neither path writes (empty problems)
    # compare equal.
    for p in pre:
        for k in ("Y", "acc"):
            p[k].fill_(-7)
    for c in dec:
        for k in ("Y", "X_q", "x_scale"):
            c[k].fill_(-7)
    bl.forward_mixed(pre, dec)
    if pre2:
        bl.forward_ex_grouped(pre2)
    if dec2:
        bl.linear_grouped(dec2)
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(pre, pre2)):
        assert torch.equal(a["Y"], b["Y"]), ("prefill Y", i)
        assert torch.equal(a["acc"], b["acc"]), ("prefill acc", i)
    for i, (a, b) in enumerate(zip(dec, dec2)):
        assert torch.equal(a["Y"], b["Y"]), ("decode Y", i)
        assert torch.equal(a["X_q"], b["X_q"]), ("decode X_q", i)
        assert torch.equal(a["x_scale"], b["x_scale"]), ("decode x_scale", i)


def check_pre_oracle(orc, p, ref, label, samples=384):
    M, N = p["Y"].shape
    if M == 0 or N == 0:
        return
    g = rng((1,) + tuple(p["Y"].shape))
    m_idx = np.concatenate([g.integers(0, M, samples), [0, M - 1, M - 1]])
    n_idx = np.concatenate([g.integers(0, N, samples), [0, N - 1, 0]])
    acc_ref, y_ref = orc.forward_entries(ref["Xq"], ref["sx"], host(p["W_packed"]).view(np.uint32),
                                         GAMMA, m_idx, n_idx)
    acc, Y = host(p["acc"])[m_idx, n_idx], host(p["Y"])[m_idx, n_idx]
    assert np.array_equal(acc, acc_ref), label
    assert np.array_equal(Y == 0, y_ref == 0), label
    assert rel_err(Y[y_ref != 0], y_ref[y_ref != 0]) <= REL, label


def check_dec_oracle(orc, call, ref, label):
    q_ref, s_ref = orc.quantize_acts(ref["x"], ref["g"], 1e-6, bf16=ref["bf16"])
    q, s, Y = host(call["X_q"]), host(call["x_scale"]), host(call["Y"])
    assert np.array_equal(q, q_ref), label
    nz = s_ref != 0
    assert np.array_equal(s == 0, ~nz), label
    assert rel_err(s[nz], s_ref[nz]) <= REL, label
    Y_ref = orc.epilogue(orc.matmul(q_ref, ref["C"]), s_ref, GAMMA)
    assert np.array_equal(Y == 0, Y_ref == 0), label
    assert rel_err(Y[Y_ref != 0], Y_ref[Y_ref != 0]) <= REL, label


def build(torch, bl, pre_specs, dec_specs, key):
    pre, pre_ref, dec, dec_ref = [], [], [], []
    for i, (M, N, K) in enumerate(pre_specs):
        p, r = make_pre(torch, bl, M, N, K, key + (i,))
        pre.append(p)
        pre_ref.append(r)
    for i, (M, N, K, dt, nm) in enumerate(dec_specs):
        c, r = make_dec(torch, bl, M, N, K, dt, nm, key + (100 + i,))
        dec.append(c)
        dec_ref.append(r)
    return pre, pre_ref, dec, dec_ref


def check_all(torch, bl, orc, pre_specs, dec_specs, key):
    pre, pre_ref, dec, dec_ref = build(torch, bl, pre_specs, dec_specs, key)
    run_both(torch, bl, pre, dec)
    for i, (p, r) in enumerate(zip(pre, pre_ref)):
        check_pre_oracle(orc, p, r, ("prefill", key, pre_specs[i]))
    for i, (c, r) in enumerate(zip(dec, dec_ref)):
        if c["X"].shape[0] and c["Y"].shape[1]:
            check_dec_oracle(orc, c, r, ("decode", key, dec_specs[i]))


@pytest.mark.parametrize("norm", [False, True])
def test_mixed_distillix_layer(torch, bl, orc, norm):
    """The Distillix-125M layer set as the benchmark runs it: 2048 prefill tokens and one
    decode token per matrix, fp32 activations; and the same with a norm in front of the
    output and down projections' decode calls."""
    wl = workloads.WORKLOADS["c2_distillix125m_layer"]
    shapes = [(m.N, m.K) for m in wl.matrices]
    pre_specs = [(2048, N, K) for N, K in shapes]
    dec_specs = [(1, N, K, "f32", norm and i in (3, 6)) for i, (N, K) in enumerate(shapes)]
    check_all(torch, bl, orc, pre_specs, dec_specs, (1, int(norm)))


def test_mixed_edge_layer(torch, bl, orc):
    """The 1.4B edge layer set at 512 prefill tokens (pre-packed codes) with one decode token."""
    wl = workloads.WORKLOADS["c3_edge1p4b_prepacked"]
    shapes = [(m.N, m.K) for m in wl.matrices]
    check_all(torch, bl, orc, [(512, N, K) for N, K in shapes],
              [(1, N, K, "f32", False) for N, K in shapes], (6,))


@pytest.mark.parametrize("pre_ragged", [False, True])
@pytest.mark.parametrize("dec_ragged", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mixed_ragged(torch, bl, orc, pre_ragged, dec_ragged, dtype):
    """Whole and ragged K on each side (K = 272 and 1040 fill no whole 128-wide prefill stage
    or 256-wide decode step), N not a multiple of 128 or 16, M not a multiple of 128, fp32
    and bf16 decode activations, with and without a norm: every kernel form of the launch."""
    kp = (272, 1040) if pre_ragged else (256, 1024)
    kd = (272, 1040) if dec_ragged else (256, 1024)
    pre_specs = [(130, 300, kp[0]), (17, 129, kp[1]), (257, 64, 128)]
    dec_specs = [(3, 301, kd[0], dtype, True), (1, 17, kd[1], dtype, False),
                 (4, 1000, 768, dtype, True)]
    check_all(torch, bl, orc, pre_specs, dec_specs,
              (2, int(pre_ragged), int(dec_ragged), int(dtype == "bf16")))


def test_mixed_repeat_and_empty(torch, bl, orc):
    """Empty problems in either set are no-ops; a repeated call gives the same bits."""
    pre_specs = [(300, 0, 256), (0, 128, 256), (200, 200, 512)]
    dec_specs = [(1, 0, 768, "f32", False), (0, 64, 768, "f32", False), (2, 333, 512, "f32", True)]
    pre, pre_ref, dec, dec_ref = build(torch, bl, pre_specs, dec_specs, (3,))
    run_both(torch, bl, pre, dec)
    Y0 = [p["Y"].clone() for p in pre] + [c["Y"].clone() for c in dec]
    bl.forward_mixed(pre, dec)
    torch.cuda.synchronize()
    for a, b in zip(Y0, [p["Y"] for p in pre] + [c["Y"] for c in dec]):
        assert torch.equal(a, b)
    check_pre_oracle(orc, pre[2], pre_ref[2], "repeat prefill")
    check_dec_oracle(orc, dec[2], dec_ref[2], "repeat decode")


TWO_LAUNCH = ["small_prefill", "unfused_decode", "mixed_dtypes", "big_tiles", "prefill_only",
              "decode_only"]


@pytest.mark.parametrize("case", TWO_LAUNCH)
def test_mixed_two_launch_cases(torch, bl, orc, case):
    """Sets that do not share a launch still give the two calls' results."""
    pre_specs = [(256, 384, 768)]
    dec_specs = [(1, 512, 768, "f32", False)]
    if case == "small_prefill":
        pre_specs = pre_specs + [(16, 200, 512)]
    elif case == "unfused_decode":
        dec_specs = dec_specs + [(8, 100, 512, "f32", True)]
    elif case == "mixed_dtypes":
        dec_specs = dec_specs + [(2, 100, 512, "bf16", False)]
    elif case == "big_tiles":
        pre_specs = [(4096, 8192, 128)]          # 512 units of 256 x 256: 128 x 256 tiles
    elif case == "prefill_only":
        dec_specs = []
    elif case == "decode_only":
        pre_specs = []
    check_all(torch, bl, orc, pre_specs, dec_specs, (4, TWO_LAUNCH.index(case)))


def test_mixed_rejects(torch, bl):
    """Argument errors, checked on the host before anything is launched."""
    import ctypes
    L = bl.lib()
    pre, _, dec, _ = build(torch, bl, [(64, 64, 256)], [(1, 64, 256, "f32", False)], (5,))
    pt = bl.forward_ex_table(pre)
    dt = bl.linear_table(dec)
    a, b = ctypes.addressof(pt), ctypes.addressof(dt)
    assert L.bitlinear_forward_mixed(a, 0, b, 0, None) == BL_ERR_COUNT
    assert L.bitlinear_forward_mixed(a, -1, b, 1, None) == BL_ERR_COUNT
    assert L.bitlinear_forward_mixed(a, 1, b, 17, None) == BL_ERR_COUNT
    assert L.bitlinear_forward_mixed(None, 1, b, 1, None) == BL_ERR_NULL
    assert L.bitlinear_forward_mixed(a, 1, None, 1, None) == BL_ERR_NULL
    assert L.bitlinear_forward_mixed(None, 0, b, 1, None) == BL_OK
    # A bad decode problem rejects the whole call: the prefill output stays untouched.
    pre[0]["Y"].fill_(5.0)
    dt[0].K = 250
    assert L.bitlinear_forward_mixed(a, 1, b, 1, None) == BL_ERR_SHAPE
    torch.cuda.synchronize()
    assert bool((pre[0]["Y"] == 5.0).all())
