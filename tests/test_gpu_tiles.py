"""Decode tiles on the GPU: the packer bit-exact against the tile layout written out here from
the oracle's two-bit packing of the same codes, and the one-token call on tiles bit for bit
against the same call on the two-bit rows (codes, scales and outputs) and against the oracle
(codes bit-exact, scales and Y within 1e-6, as for the two-bit call)."""

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


def tile_layout(C, N, K):
    """The documented layout, written out from the codes C [N][K]: tile (rg, T) is 64 chunks of
    16 bytes; chunk 16 g + r holds row 16 rg + r as four dwords i, and field j (bits 8 b + 2 j)
    of byte b of dword i holds the code c of k = 256 T + 64 g + 16 j + 4 i + b, as c mod 4 for
    j = 3 and as c + 1 for j < 3; rows past N and k past K hold c = 0."""
    supers = (K // 16 + 15) // 16
    groups = (N + 15) // 16
    Cp = np.zeros((groups * 16, supers * 256), np.int64)
    Cp[:N, :K] = C
    c = Cp.reshape(groups, 16, supers, 4, 4, 4, 4)               # [rg][r][T][g][j][i][b]
    j = np.arange(4).reshape(4, 1, 1)
    b = np.arange(4).reshape(1, 1, 4)
    enc = np.where(j == 3, c & 3, (c + 1) & 3)
    dw = (enc << (8 * b + 2 * j)).sum(axis=(4, 6))             # [rg][r][T][g][i]
    return dw.transpose(0, 2, 3, 1, 4).reshape(-1).astype(np.uint32)


@pytest.mark.parametrize("N,K", [(1, 16), (16, 256), (17, 272), (300, 768), (129, 9728), (8, 12288),
                                 (40, 80)])
def test_pack_tiles(torch, bl, orc, N, K):
    C = workloads.ternary((N, K), (510, N, K))
    P = orc.pack(C)
    T = bl.pack_tiles(dev(torch, P.view(np.int32)), K)
    torch.cuda.synchronize()
    assert T.numel() * 4 == bl.tiles_bytes(N, K)
    assert np.array_equal(host(T).view(np.uint32), tile_layout(C, N, K))


SHAPES = [(1, 64), (37, 128), (300, 768), (768, 768), (129, 2048), (96, 9728), (40, 12288),
          (4100, 2560), (16400, 1024)]


def make(torch, bl, N, K, dtype, norm, key):
    X = workloads.gaussian((1, K), (511, N, K) + key, 1.0)
    g = (np.float32(1) + workloads.gaussian((K,), (512, K) + key, 0.1)) if norm else None
    C = workloads.ternary((N, K), (513, N, K) + key)
    P = bl.pack_codes(dev(torch, C))
    if dtype == "bf16":
        bits = workloads.f32_to_bf16_bits(X)
        Xt, xin = dev(torch, bits.view(np.int16)).view(torch.bfloat16), bits
    else:
        Xt, xin = dev(torch, X), X
    gt = dev(torch, np.array([GAMMA], np.float32))
    nt = None if g is None else dev(torch, g)

    def outs():
        return dict(Y=torch.empty((1, N), device="cuda"),
                    X_q=torch.empty((1, K), dtype=torch.int8, device="cuda"),
                    x_scale=torch.empty(1, device="cuda"))
    tiles = dict(X=Xt, W_tiles=bl.pack_tiles(P, K), gamma=gt, norm_weight=nt, eps=1e-6, **outs())
    two = dict(X=Xt, W_packed=P, gamma=gt, norm_weight=nt, eps=1e-6, **outs())
    return tiles, two, dict(x=xin, g=g, C=C, bf16=dtype == "bf16")


@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("norm", [False, True])
def test_linear_tiles(torch, bl, orc, N, K, dtype, norm):
    label = (N, K, dtype, norm)
    tiles, two, ref = make(torch, bl, N, K, dtype, norm, (0,))
    bl.linear_tiles_grouped([tiles])
    bl.linear_grouped([two])
    torch.cuda.synchronize()
    for k in ("Y", "X_q", "x_scale"):
        assert torch.equal(tiles[k], two[k]), (label, k)
    q_ref, s_ref = orc.quantize_acts(ref["x"], ref["g"], 1e-6, bf16=ref["bf16"])
    assert np.array_equal(host(tiles["X_q"]), q_ref), label
    s = host(tiles["x_scale"])
    nz = s_ref != 0
    assert rel_err(s[nz], s_ref[nz]) <= REL, label
    Y_ref = orc.epilogue(orc.matmul(q_ref, ref["C"]), s_ref, GAMMA)
    Y = host(tiles["Y"])
    assert np.array_equal(Y == 0, Y_ref == 0), label
    assert rel_err(Y[Y_ref != 0], Y_ref[Y_ref != 0]) <= REL, label


def extreme_case(kind, N, K):
    """Activations and codes at the ends of the ranges the offset planes and their correction
    must hold exactly: every activation code +-127 against weights all +1, all -1 or mixed,
    a one-hot row, and a row whose codes cancel within each plane."""
    k = np.arange(K)
    if kind == "all_plus":
        X, C = np.full((1, K), 3.0, np.float32), np.ones((N, K), np.int8)
    elif kind == "all_minus":
        X, C = np.full((1, K), -3.0, np.float32), -np.ones((N, K), np.int8)
    elif kind == "mixed_max":
        X = np.where(k % 3 == 0, 5.0, -5.0).astype(np.float32)[None, :]
        C = np.where((np.arange(N)[:, None] + k) % 2 == 0, 1, -1).astype(np.int8)
    elif kind == "one_hot":
        X = np.zeros((1, K), np.float32)
        X[0, K - 1] = -2.5
        C = workloads.ternary((N, K), (514, N, K))
    else:                                       # "cancel": +-x in neighbouring codes
        X = np.where(k % 2 == 0, 1.0, -1.0).astype(np.float32)[None, :]
        C = workloads.ternary((N, K), (515, N, K))
    return X, C


@pytest.mark.parametrize("kind", ["all_plus", "all_minus", "mixed_max", "one_hot", "cancel"])
@pytest.mark.parametrize("N,K", [(48, 12288), (33, 9728), (16, 64)])
def test_linear_tiles_extremes(torch, bl, orc, kind, N, K):
    X, C = extreme_case(kind, N, K)
    P = bl.pack_codes(dev(torch, C))
    gt = dev(torch, np.array([GAMMA], np.float32))

    def call(tiles):
        d = dict(X=dev(torch, X), gamma=gt, eps=1e-6, Y=torch.empty((1, N), device="cuda"),
                 X_q=torch.empty((1, K), dtype=torch.int8, device="cuda"),
                 x_scale=torch.empty(1, device="cuda"))
        if tiles:
            d["W_tiles"] = bl.pack_tiles(P, K)
            bl.linear_tiles_grouped([d])
        else:
            d["W_packed"] = P
            bl.linear_grouped([d])
        return d
    a, b = call(True), call(False)
    torch.cuda.synchronize()
    for key in ("Y", "X_q", "x_scale"):
        assert torch.equal(a[key], b[key]), (kind, N, K, key)
    q_ref, s_ref = orc.quantize_acts(X, None, 1e-6)
    assert np.array_equal(host(a["X_q"]), q_ref)
    acc = orc.matmul(q_ref, C)
    Y_ref = orc.epilogue(acc, s_ref, GAMMA)
    Y = host(a["Y"])
    assert np.array_equal(Y == 0, Y_ref == 0), (kind, N, K)
    nz = Y_ref != 0
    assert rel_err(Y[nz], Y_ref[nz]) <= REL, (kind, N, K)


def test_linear_tiles_layer_set(torch, bl, orc):
    """The Qwen3-4B decode layer set (one token) in one call, twice in a row: every output
    equals the two-bit call's, and the oracle's (codes exact, Y within 1e-6)."""
    mats = workloads.WORKLOADS["c5_qwen3_4b_layer"].matrices
    ts, twos, refs = [], [], []
    for i, m in enumerate(mats):
        t, two, ref = make(torch, bl, m.N, m.K, "f32", i % 2 == 0, (1, i))
        ts.append(t)
        twos.append(two)
        refs.append(ref)
    bl.linear_grouped(twos)
    for _ in range(2):
        for t in ts:
            t["Y"].fill_(float("nan"))
        bl.linear_tiles_grouped(ts)
        torch.cuda.synchronize()
        for a, b in zip(ts, twos):
            assert torch.equal(a["Y"], b["Y"])
    for t, ref, m in zip(ts, refs, mats):
        q_ref, s_ref = orc.quantize_acts(ref["x"], ref["g"], 1e-6)
        assert np.array_equal(host(t["X_q"]), q_ref), (m.N, m.K)
        Y_ref = orc.epilogue(orc.matmul(q_ref, ref["C"]), s_ref, GAMMA)
        Y = host(t["Y"])
        assert np.array_equal(Y == 0, Y_ref == 0)
        assert rel_err(Y[Y_ref != 0], Y_ref[Y_ref != 0]) <= REL, (m.N, m.K)


def test_linear_tiles_rejects_more_tokens(torch, bl):
    t, _, _ = make(torch, bl, 64, 256, "f32", False, (2,))
    t["X"] = torch.zeros((2, 256), device="cuda")
    t["Y"] = torch.empty((2, 64), device="cuda")
    with pytest.raises(bl.BitLinearError) as e:
        bl.linear_tiles_grouped([t])
    assert e.value.status == -2
