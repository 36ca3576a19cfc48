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


def tile_layout(P, N, K):
    """The documented layout: tile (rg, T) is 64 chunks of 16 bytes; chunk 16 g + r holds words
    16 T + 4 g .. + 3 of row 16 rg + r; rows past N and words past K / 16 are zero."""
    words = K // 16
    supers = (words + 15) // 16
    groups = (N + 15) // 16
    Pp = np.zeros((groups * 16, supers * 16), np.uint32)
    Pp[:N, :words] = P.view(np.uint32).reshape(N, words)
    t = Pp.reshape(groups, 16, supers, 4, 4)          # [rg][r][T][g][i]
    return t.transpose(0, 2, 3, 1, 4).reshape(-1)     # [rg][T][g][r][i]


@pytest.mark.parametrize("N,K", [(1, 16), (16, 256), (17, 272), (300, 768), (129, 9728), (8, 12288),
                                 (40, 80)])
def test_pack_tiles(torch, bl, orc, N, K):
    C = workloads.ternary((N, K), (510, N, K))
    P = orc.pack(C)
    T = bl.pack_tiles(dev(torch, P.view(np.int32)), K)
    torch.cuda.synchronize()
    assert T.numel() * 4 == bl.tiles_bytes(N, K)
    assert np.array_equal(host(T).view(np.uint32), tile_layout(P, N, K))


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


def test_linear_tiles_layer_set(torch, bl):
    """The Qwen3-4B decode layer set (one token) in one call, twice in a row: every output
    equals the two-bit call's."""
    mats = workloads.WORKLOADS["c5_qwen3_4b_layer"].matrices
    ts, twos = [], []
    for i, m in enumerate(mats):
        t, two, _ = make(torch, bl, m.N, m.K, "f32", i % 2 == 0, (1, i))
        ts.append(t)
        twos.append(two)
    bl.linear_grouped(twos)
    for _ in range(2):
        for t in ts:
            t["Y"].fill_(float("nan"))
        bl.linear_tiles_grouped(ts)
        torch.cuda.synchronize()
        for a, b in zip(ts, twos):
            assert torch.equal(a["Y"], b["Y"])


def test_linear_tiles_rejects_more_tokens(torch, bl):
    t, _, _ = make(torch, bl, 64, 256, "f32", False, (2,))
    t["X"] = torch.zeros((2, 256), device="cuda")
    t["Y"] = torch.empty((2, 64), device="cuda")
    with pytest.raises(bl.BitLinearError) as e:
        bl.linear_tiles_grouped([t])
    assert e.value.status == -2
