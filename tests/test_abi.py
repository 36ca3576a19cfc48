"""C ABI checks that need no GPU: the library loads, exports every declared entry point, and
rejects bad arguments on the host before launching anything.

Rejected calls never dereference their pointers, so small fake addresses stand in for device
buffers here.  Empty problems (M == 0) are accepted and launch nothing.
"""

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bitlinear.h")

BL_OK, BL_ERR_NULL, BL_ERR_SHAPE, BL_ERR_ALIGN, BL_ERR_DTYPE, BL_ERR_WORKSPACE, BL_ERR_HIP, \
    BL_ERR_COUNT = 0, -1, -2, -3, -4, -5, -6, -7

A = 0x10000  # fake, 16-byte aligned "device" addresses
B = 0x20000
C = 0x30000
D = 0x40000
E = 0x50000


@pytest.fixture(scope="module")
def bl():
    import bit_gemm_02_amd as m
    return m


@pytest.fixture(scope="module")
def L(bl):
    return bl.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bitlinear_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(bl):
    names = declared_functions()
    assert len(names) >= 11
    lib = ctypes.CDLL(bl.library_path())
    for name in names:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", bl.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\b(bitlinear_\w+)\b", out))
    assert set(names) <= exported


def test_library_is_gfx950(bl):
    data = open(bl.library_path(), "rb").read()
    assert b"gfx950" in data


def test_status_strings(L):
    for s in (BL_OK, BL_ERR_NULL, BL_ERR_SHAPE, BL_ERR_ALIGN, BL_ERR_DTYPE, BL_ERR_WORKSPACE,
              BL_ERR_HIP, BL_ERR_COUNT):
        assert L.bitlinear_status_string(s)
    assert L.bitlinear_status_string(12345) == b"unknown status"
    assert L.bitlinear_abi_version() == 104


def test_quantize_weights_noalloc_validation(L, bl):
    q = L.bitlinear_quantize_weights_grouped_noalloc
    arr = (bl._WeightProblem * 2)()
    arr[0] = bl._WeightProblem(A, B, C, 4, 64)
    arr[1] = bl._WeightProblem(A, B, C, 4, 64)
    assert q(None, 1, None) == BL_ERR_NULL
    assert q(ctypes.addressof(arr), 0, None) == BL_ERR_COUNT
    assert q(ctypes.addressof(arr), 17, None) == BL_ERR_COUNT
    arr[1] = bl._WeightProblem(A, B, C, 4, 24)
    assert q(ctypes.addressof(arr), 2, None) == BL_ERR_SHAPE
    arr[1] = bl._WeightProblem(A + 4, B, C, 4, 64)
    assert q(ctypes.addressof(arr), 2, None) == BL_ERR_ALIGN
    arr[1] = bl._WeightProblem(None, B, C, 4, 64)
    assert q(ctypes.addressof(arr), 2, None) == BL_ERR_NULL


def test_quantize_weights_validation(L):
    ws = L.bitlinear_quantize_weights_workspace(64, 64)
    assert ws >= 8
    assert L.bitlinear_workspace_bytes(64, 64) == ws == L.bitlinear_workspace_bytes(9728, 2560)
    q = L.bitlinear_quantize_weights
    assert q(None, 4, 64, B, C, D, ws, None) == BL_ERR_NULL
    assert q(A, 4, 64, None, C, D, ws, None) == BL_ERR_NULL
    assert q(A, 4, 64, B, None, D, ws, None) == BL_ERR_NULL
    assert q(A, 4, 64, B, C, None, ws, None) == BL_ERR_NULL
    assert q(A, 4, 24, B, C, D, ws, None) == BL_ERR_SHAPE
    assert q(A, 4, 0, B, C, D, ws, None) == BL_ERR_SHAPE
    assert q(A, -1, 64, B, C, D, ws, None) == BL_ERR_SHAPE
    assert q(A, 4, 262144 + 16, B, C, D, ws, None) == BL_ERR_SHAPE
    assert q(A + 4, 4, 64, B, C, D, ws, None) == BL_ERR_ALIGN
    assert q(A, 4, 64, B + 8, C, D, ws, None) == BL_ERR_ALIGN
    assert q(A, 4, 64, B, C + 2, D, ws, None) == BL_ERR_ALIGN
    assert q(A, 4, 64, B, C, D, ws - 1, None) == BL_ERR_WORKSPACE


def test_grouped_count_validation(L, bl):
    arr = (bl._WeightProblem * 1)()
    arr[0] = bl._WeightProblem(A, B, C, 4, 64)
    ws = L.bitlinear_quantize_weights_grouped_workspace(1)
    assert L.bitlinear_quantize_weights_grouped(ctypes.addressof(arr), 0, D, ws, None) == BL_ERR_COUNT
    assert L.bitlinear_quantize_weights_grouped(ctypes.addressof(arr), 17, D, ws, None) == BL_ERR_COUNT
    assert L.bitlinear_quantize_weights_grouped(None, 1, D, ws, None) == BL_ERR_NULL
    assert L.bitlinear_quantize_weights_grouped_workspace(0) == 0
    assert L.bitlinear_quantize_weights_grouped_workspace(2) == 2 * ws
    fa = (bl._ForwardProblem * 1)()
    assert L.bitlinear_forward_grouped(ctypes.addressof(fa), 0, None) == BL_ERR_COUNT
    aa = (bl._ActProblem * 1)()
    assert L.bitlinear_quantize_acts_grouped(ctypes.addressof(aa), 17, None) == BL_ERR_COUNT


def test_one_read_workspace_query(L, bl):
    """Invalid input gives 0; the size covers the two-read workspace and grows with the
    tensors (lists of one 20-byte entry per 16 four-weight chunks, plus 64 entries per wave:
    about 0.31 N K bytes and 1.3 MiB per tensor)."""
    q = L.bitlinear_quantize_weights_one_read_workspace
    arr = (bl._WeightProblem * 3)()
    arr[0] = bl._WeightProblem(A, B, C, 4096, 2560)
    arr[1] = bl._WeightProblem(A, B, C, 2560, 9728)
    arr[2] = bl._WeightProblem(A, B, C, 0, 64)
    assert q(None, 1) == 0
    assert q(ctypes.addressof(arr), 0) == 0
    assert q(ctypes.addressof(arr), 17) == 0
    one, two, three = (q(ctypes.addressof(arr), n) for n in (1, 2, 3))
    assert one >= L.bitlinear_quantize_weights_grouped_workspace(1)
    assert one < two < three
    assert 0.3125 * 4096 * 2560 <= one <= 0.3125 * 4096 * 2560 * 1.05 + (3 << 19)
    assert 0.3125 * 2560 * 9728 <= two - one <= 0.3125 * 2560 * 9728 * 1.05 + (3 << 19)
    arr[1] = bl._WeightProblem(A, B, C, 4, 24)
    assert q(ctypes.addressof(arr), 2) == 0
    arr[1] = bl._WeightProblem(A, B, C, -1, 64)
    assert q(ctypes.addressof(arr), 2) == 0


def test_forward_mixed_validation(L, bl):
    """Counts, NULL arrays and each problem's own checks; every case is rejected on the host
    (or is all empty), so nothing is launched."""
    m = L.bitlinear_forward_mixed
    pre = (bl._ForwardExProblem * 2)()
    pre[0] = bl._ForwardExProblem(A, B, C, D, E, None, None, 300, 64, 256)
    dec = (bl._LinearProblem * 2)()
    dec[0] = bl._LinearProblem(A, None, B, C, D, None, None, 1, 64, 256, 0, 1e-6)
    pa, da = ctypes.addressof(pre), ctypes.addressof(dec)
    assert m(pa, 0, da, 0, None) == BL_ERR_COUNT
    assert m(pa, -1, da, 1, None) == BL_ERR_COUNT
    assert m(pa, 1, da, -1, None) == BL_ERR_COUNT
    assert m(pa, 17, da, 1, None) == BL_ERR_COUNT
    assert m(pa, 1, da, 17, None) == BL_ERR_COUNT
    assert m(None, 1, da, 1, None) == BL_ERR_NULL
    assert m(pa, 1, None, 1, None) == BL_ERR_NULL
    # Problem errors on either side.
    pre[0].K = 250
    assert m(pa, 1, da, 1, None) == BL_ERR_SHAPE
    pre[0].K = 256
    pre[0].residual = 0x60002
    assert m(pa, 1, da, 1, None) == BL_ERR_ALIGN
    pre[0].residual = None
    dec[0].x_dtype = 5
    assert m(pa, 1, da, 1, None) == BL_ERR_DTYPE
    dec[0].x_dtype = 0
    dec[0].W_packed = None
    assert m(pa, 1, da, 1, None) == BL_ERR_NULL
    dec[0].W_packed = B
    dec[1] = bl._LinearProblem(A, None, B, C, D, None, None, 8, 64, 256, 0, 1e-6)
    assert m(pa, 1, da, 2, None) == BL_ERR_NULL     # past the fused size: needs X_q, x_scale
    # All-empty sets are accepted and launch nothing.
    pre[0].M = 0
    dec[0].N = 0
    assert m(pa, 1, da, 1, None) == BL_OK
    assert m(None, 0, da, 1, None) == BL_OK


def test_quantize_step_validation(L, bl):
    """Counts, NULL arrays, workspace and each problem's checks, all on the host."""
    q = L.bitlinear_quantize_step
    w = (bl._WeightProblem * 2)()
    w[0] = bl._WeightProblem(A, B, C, 4, 64)
    a = (bl._ActProblem * 2)()
    a[0] = bl._ActProblem(A, None, B, C, 2, 64, 0, 1e-6)
    wa, aa = ctypes.addressof(w), ctypes.addressof(a)
    ws = L.bitlinear_quantize_weights_grouped_workspace(1)
    assert q(wa, 0, D, ws, aa, 0, None) == BL_ERR_COUNT
    assert q(wa, -1, D, ws, aa, 1, None) == BL_ERR_COUNT
    assert q(wa, 17, D, ws, aa, 1, None) == BL_ERR_COUNT
    assert q(wa, 1, D, ws, aa, 17, None) == BL_ERR_COUNT
    assert q(None, 1, D, ws, aa, 1, None) == BL_ERR_NULL
    assert q(wa, 1, D, ws, None, 1, None) == BL_ERR_NULL
    assert q(wa, 1, None, ws, aa, 1, None) == BL_ERR_NULL
    assert q(wa, 1, D + 8, ws, aa, 1, None) == BL_ERR_ALIGN
    assert q(wa, 1, D, ws - 1, aa, 1, None) == BL_ERR_WORKSPACE
    w[0].K = 40
    assert q(wa, 1, D, ws, aa, 1, None) == BL_ERR_SHAPE
    w[0].K = 64
    a[0].x_dtype = 3
    assert q(wa, 1, D, ws, aa, 1, None) == BL_ERR_DTYPE
    a[0].x_dtype = 0
    a[0].X_q = B + 1
    assert q(wa, 1, D, ws, aa, 1, None) == BL_ERR_ALIGN
    # Activations only: no workspace needed; empty problems launch nothing.
    a[0].X_q = B
    a[0].M = 0
    assert q(None, 0, None, 0, aa, 1, None) == BL_OK


def test_pack_codes_validation(L):
    p = L.bitlinear_pack_codes
    assert p(None, 4, 64, B, None) == BL_ERR_NULL
    assert p(A, 4, 64, None, None) == BL_ERR_NULL
    assert p(A, 4, 40, B, None) == BL_ERR_SHAPE
    assert p(A + 1, 4, 64, B, None) == BL_ERR_ALIGN


def test_quantize_acts_validation(L):
    q = L.bitlinear_quantize_acts
    assert q(None, 0, 2, 64, None, 1e-6, B, C, None) == BL_ERR_NULL
    assert q(A, 0, 2, 64, None, 1e-6, None, C, None) == BL_ERR_NULL
    assert q(A, 0, 2, 64, None, 1e-6, B, None, None) == BL_ERR_NULL
    assert q(A, 2, 2, 64, None, 1e-6, B, C, None) == BL_ERR_DTYPE
    assert q(A, -1, 2, 64, None, 1e-6, B, C, None) == BL_ERR_DTYPE
    assert q(A, 0, -2, 64, None, 1e-6, B, C, None) == BL_ERR_SHAPE
    assert q(A, 0, 2, 65, None, 1e-6, B, C, None) == BL_ERR_SHAPE
    assert q(A, 0, 2, 64, D + 4, 1e-6, B, C, None) == BL_ERR_ALIGN
    assert q(A, 1, 2, 64, None, 1e-6, B + 2, C, None) == BL_ERR_ALIGN
    # M == 0 is a valid empty problem: accepted, nothing launched.
    assert q(A, 0, 0, 64, None, 1e-6, B, C, None) == BL_OK


def test_forward_validation(L):
    f = L.bitlinear_forward
    assert f(None, B, C, D, 1, 4, 64, E, None, None) == BL_ERR_NULL
    assert f(A, None, C, D, 1, 4, 64, E, None, None) == BL_ERR_NULL
    assert f(A, B, None, D, 1, 4, 64, E, None, None) == BL_ERR_NULL
    assert f(A, B, C, None, 1, 4, 64, E, None, None) == BL_ERR_NULL
    assert f(A, B, C, D, 1, 4, 64, None, None, None) == BL_ERR_NULL
    assert f(A, B, C, D, 1, 4, 8, E, None, None) == BL_ERR_SHAPE
    assert f(A, B, C, D, -1, 4, 64, E, None, None) == BL_ERR_SHAPE
    assert f(A, B, C, D, 1, -4, 64, E, None, None) == BL_ERR_SHAPE
    assert f(A + 8, B, C, D, 1, 4, 64, E, None, None) == BL_ERR_ALIGN
    assert f(A, B, C + 4, D, 1, 4, 64, E, None, None) == BL_ERR_ALIGN
    assert f(A, B, C, D, 1, 4, 64, E + 2, None, None) == BL_ERR_ALIGN
    assert f(A, B, C, D, 1, 4, 64, E, 0x60001, None) == BL_ERR_ALIGN
    # Empty problems are accepted and launch nothing.
    assert f(A, B, C, D, 0, 4, 64, E, None, None) == BL_OK
    assert f(A, B, C, D, 3, 0, 64, E, None, None) == BL_OK


def test_linear_grouped_validation(L, bl):
    g = L.bitlinear_linear_grouped

    def call(**kw):
        d = dict(X=A, norm_weight=None, W_packed=B, gamma=C, Y=D, X_q=None, x_scale=None,
                 M=1, N=4, K=64, x_dtype=0, eps=1e-6)
        d.update(kw)
        arr = (bl._LinearProblem * 1)()
        arr[0] = bl._LinearProblem(**d)
        return g(ctypes.addressof(arr), 1, None)

    arr = (bl._LinearProblem * 1)()
    assert g(None, 1, None) == BL_ERR_NULL
    assert g(ctypes.addressof(arr), 0, None) == BL_ERR_COUNT
    assert g(ctypes.addressof(arr), 17, None) == BL_ERR_COUNT
    assert call(X=None) == BL_ERR_NULL
    assert call(W_packed=None) == BL_ERR_NULL
    assert call(gamma=None) == BL_ERR_NULL
    assert call(Y=None) == BL_ERR_NULL
    assert call(x_dtype=2) == BL_ERR_DTYPE
    assert call(K=40) == BL_ERR_SHAPE
    assert call(M=-1) == BL_ERR_SHAPE
    assert call(X=A + 4) == BL_ERR_ALIGN
    assert call(norm_weight=E + 8) == BL_ERR_ALIGN
    assert call(X_q=E + 1) == BL_ERR_ALIGN
    # Beyond the fused form (M > 4, or M * K above its byte limit) the intermediate codes
    # and scales are required.
    assert call(M=5) == BL_ERR_NULL
    assert call(M=2, K=32768) == BL_ERR_NULL
    assert call(M=5, X_q=E) == BL_ERR_NULL
    # Empty problems are accepted and launch nothing.
    assert call(M=0) == BL_OK
    assert call(N=0) == BL_OK


def test_chain_entry_points_validation(L, bl):
    qa = L.bitlinear_quantize_acts_ex_grouped

    def act(**kw):
        d = dict(X=A, X2=B, norm_weight=None, X_q=C, x_scale=D, M=2, K=64, x_dtype=0, act=1, eps=1e-6)
        d.update(kw)
        arr = (bl._ActExProblem * 1)()
        arr[0] = bl._ActExProblem(**d)
        return qa(ctypes.addressof(arr), 1, None)

    assert qa(None, 1, None) == BL_ERR_NULL
    assert act(act=4) == BL_ERR_DTYPE
    assert act(act=-1) == BL_ERR_DTYPE
    assert act(x_dtype=1) == BL_ERR_DTYPE          # activations need fp32 inputs
    assert act(X2=None) == BL_ERR_NULL             # gated kinds need the up output
    assert act(act=2, X2=None) == BL_ERR_NULL
    assert act(X2=B + 4) == BL_ERR_ALIGN
    assert act(K=40) == BL_ERR_SHAPE
    assert act(X_q=None) == BL_ERR_NULL
    assert act(M=0) == BL_OK
    assert act(act=3, X2=None, M=0) == BL_OK
    fe = L.bitlinear_forward_ex_grouped

    def fwd(**kw):
        d = dict(X_q=A, x_scale=B, W_packed=C, gamma=D, Y=E, acc=None, residual=None, M=1, N=4, K=64)
        d.update(kw)
        arr = (bl._ForwardExProblem * 1)()
        arr[0] = bl._ForwardExProblem(**d)
        return fe(ctypes.addressof(arr), 1, None)

    assert fe(None, 1, None) == BL_ERR_NULL
    assert fwd(residual=0x60002) == BL_ERR_ALIGN
    assert fwd(W_packed=None) == BL_ERR_NULL
    assert fwd(K=8) == BL_ERR_SHAPE
    assert fwd(M=0, residual=0x60000) == BL_OK


def test_linear_ex_validation(L, bl):
    g = L.bitlinear_linear_ex_grouped

    def call(**kw):
        d = dict(X=A, norm_weight=None, W_packed=B, gamma=C, W2_packed=None, gamma2=None, Y=D,
                 residual=None, X_q=None, x_scale=None, M=1, N=4, K=64, x_dtype=0, act=0, eps=1e-6)
        d.update(kw)
        arr = (bl._LinearExProblem * 1)()
        arr[0] = bl._LinearExProblem(**d)
        return g(ctypes.addressof(arr), 1, None)

    arr = (bl._LinearExProblem * 1)()
    assert g(None, 1, None) == BL_ERR_NULL
    assert g(ctypes.addressof(arr), 0, None) == BL_ERR_COUNT
    assert g(ctypes.addressof(arr), 17, None) == BL_ERR_COUNT
    assert call(X=None) == BL_ERR_NULL
    assert call(Y=None) == BL_ERR_NULL
    assert call(act=5) == BL_ERR_DTYPE
    assert call(act=-1) == BL_ERR_DTYPE
    assert call(x_dtype=3) == BL_ERR_DTYPE
    # Gated kinds need the pair; single kinds refuse one.
    assert call(act=1) == BL_ERR_NULL
    assert call(act=2, W2_packed=E) == BL_ERR_NULL
    assert call(act=0, W2_packed=E, gamma2=C) == BL_ERR_DTYPE
    assert call(act=3, W2_packed=E, gamma2=C) == BL_ERR_DTYPE
    assert call(act=1, W2_packed=E + 4, gamma2=C) == BL_ERR_ALIGN
    assert call(act=1, W2_packed=E, gamma2=C + 2) == BL_ERR_ALIGN
    assert call(residual=E + 2) == BL_ERR_ALIGN
    # Only the fused form exists.
    assert call(M=5) == BL_ERR_SHAPE
    assert call(M=2, K=32768) == BL_ERR_SHAPE
    assert call(K=40) == BL_ERR_SHAPE
    assert call(M=-1) == BL_ERR_SHAPE
    assert call(M=0, act=1, gamma2=C) == BL_OK
    assert call(N=0) == BL_OK


def test_training_entry_points_validation(L, bl):
    fw = L.bitlinear_forward_wonly_grouped

    def wonly(**kw):
        d = dict(X=A, W_packed=B, gamma=C, Y=D, M=2, N=4, K=64, x_dtype=0)
        d.update(kw)
        arr = (bl._WonlyProblem * 1)()
        arr[0] = bl._WonlyProblem(**d)
        return fw(ctypes.addressof(arr), 1, None)

    assert fw(None, 1, None) == BL_ERR_NULL
    assert wonly(X=None) == BL_ERR_NULL
    assert wonly(gamma=None) == BL_ERR_NULL
    assert wonly(x_dtype=2) == BL_ERR_DTYPE
    assert wonly(K=40) == BL_ERR_SHAPE
    assert wonly(N=-1) == BL_ERR_SHAPE
    assert wonly(X=A + 8) == BL_ERR_ALIGN
    assert wonly(Y=D + 2) == BL_ERR_ALIGN
    assert wonly(M=0) == BL_OK and wonly(N=0, X=None) == BL_OK
    tp = L.bitlinear_transpose_packed
    assert tp(A, 40, 64, B, None) == BL_ERR_SHAPE          # N % 16 != 0
    assert tp(A, 32, 40, B, None) == BL_ERR_SHAPE          # K % 16 != 0
    assert tp(A, 16 * 20000, 64, B, None) == BL_ERR_SHAPE  # N above BL_MAX_K
    assert tp(None, 32, 64, B, None) == BL_ERR_NULL
    assert tp(A + 4, 32, 64, B, None) == BL_ERR_ALIGN
    assert tp(None, 0, 64, None, None) == BL_OK
    gi = L.bitlinear_grad_input_grouped

    def gin(**kw):
        d = dict(dY=A, Wt_packed=B, gamma=C, dX=D, M=2, N=64, K=32, dy_dtype=0)
        d.update(kw)
        arr = (bl._GradInputProblem * 1)()
        arr[0] = bl._GradInputProblem(**d)
        return gi(ctypes.addressof(arr), 1, None)

    assert gin(dY=None) == BL_ERR_NULL
    assert gin(N=40) == BL_ERR_SHAPE
    assert gin(K=0) == BL_ERR_SHAPE
    assert gin(dy_dtype=5) == BL_ERR_DTYPE
    assert gin(Wt_packed=B + 4) == BL_ERR_ALIGN
    assert gin(M=0, dY=None, dX=None) == BL_OK
    gw = L.bitlinear_grad_weight_grouped

    def gwt(**kw):
        d = dict(dY=A, X_q=B, x_scale=C, W=None, gamma=D, dW=E, M=2, N=4, K=64, ste=0, beta=2.0)
        d.update(kw)
        arr = (bl._GradWeightProblem * 1)()
        arr[0] = bl._GradWeightProblem(**d)
        return gw(ctypes.addressof(arr), 1, None)

    assert gw(None, 1, None) == BL_ERR_NULL
    assert gwt(ste=3) == BL_ERR_DTYPE
    assert gwt(ste=1) == BL_ERR_NULL                      # hard / soft need W
    assert gwt(ste=2, W=None) == BL_ERR_NULL
    assert gwt(dY=None) == BL_ERR_NULL
    assert gwt(K=40) == BL_ERR_SHAPE
    assert gwt(N=300000) == BL_ERR_SHAPE
    assert gwt(dY=A + 4) == BL_ERR_ALIGN
    assert gwt(ste=1, W=E + 8) == BL_ERR_ALIGN
    assert gwt(x_scale=C + 2) == BL_ERR_ALIGN
    assert gwt(N=0, dW=None) == BL_OK


def test_tiles_entry_points_validation(L, bl):
    assert L.bitlinear_tiles_bytes(16, 256) == 1024 and L.bitlinear_tiles_bytes(17, 256) == 2048
    assert L.bitlinear_tiles_bytes(16, 272) == 2048 and L.bitlinear_tiles_bytes(0, 256) == 0
    assert L.bitlinear_tiles_bytes(16, 40) == 0 and L.bitlinear_tiles_bytes(-1, 256) == 0
    pk = L.bitlinear_pack_tiles
    assert pk(None, 4, 64, B, None) == BL_ERR_NULL
    assert pk(A, 4, 40, B, None) == BL_ERR_SHAPE
    assert pk(A, -1, 64, B, None) == BL_ERR_SHAPE
    assert pk(A + 4, 4, 64, B, None) == BL_ERR_ALIGN
    assert pk(A, 4, 64, B + 8, None) == BL_ERR_ALIGN
    assert pk(None, 0, 64, None, None) == BL_OK
    g = L.bitlinear_linear_tiles_grouped

    def call(**kw):
        d = dict(X=A, norm_weight=None, W_packed=B, gamma=C, Y=D, X_q=None, x_scale=None,
                 M=1, N=4, K=64, x_dtype=0, eps=1e-6)
        d.update(kw)
        arr = (bl._LinearProblem * 1)()
        arr[0] = bl._LinearProblem(**d)
        return g(ctypes.addressof(arr), 1, None)

    assert g(None, 1, None) == BL_ERR_NULL
    assert call(X=None) == BL_ERR_NULL
    assert call(M=2) == BL_ERR_SHAPE              # one token only
    assert call(K=80) == BL_ERR_SHAPE             # K % 64 != 0
    assert call(K=12288 + 64) == BL_ERR_SHAPE     # past the one-token kernel's row length
    assert call(K=40) == BL_ERR_SHAPE
    assert call(x_dtype=2) == BL_ERR_DTYPE
    assert call(W_packed=B + 4) == BL_ERR_ALIGN
    assert call(M=0) == BL_OK


def test_quad_rows_entry_points_validation(L, bl):
    """The quad-row calls reject what the layout cannot hold (N % 4, K % 128), decode-sized
    products and the usual NULL / alignment cases on the host; nothing is launched."""
    pk = L.bitlinear_pack_quad_rows
    assert pk(None, 4, 128, B, None) == BL_ERR_NULL
    assert pk(A, 4, 128, None, None) == BL_ERR_NULL
    assert pk(A, 6, 128, B, None) == BL_ERR_SHAPE      # N % 4 != 0
    assert pk(A, 4, 192, B, None) == BL_ERR_SHAPE      # K % 128 != 0
    assert pk(A, 4, 40, B, None) == BL_ERR_SHAPE
    assert pk(A, -4, 128, B, None) == BL_ERR_SHAPE
    assert pk(A + 4, 4, 128, B, None) == BL_ERR_ALIGN
    assert pk(A, 4, 128, B + 8, None) == BL_ERR_ALIGN
    assert pk(None, 0, 128, None, None) == BL_OK
    f = L.bitlinear_forward_quad_rows_grouped
    fa = (bl._ForwardProblem * 2)()
    fa[0] = bl._ForwardProblem(A, B, C, D, E, None, 300, 64, 256)
    addr = ctypes.addressof(fa)
    assert f(None, 1, None) == BL_ERR_NULL
    assert f(addr, 0, None) == BL_ERR_COUNT and f(addr, 17, None) == BL_ERR_COUNT
    fa[0].M = 16
    assert f(addr, 1, None) == BL_ERR_SHAPE             # decode-sized products read rows
    fa[0].M = 300
    fa[0].N = 66
    assert f(addr, 1, None) == BL_ERR_SHAPE
    fa[0].N = 64
    fa[0].K = 320
    assert f(addr, 1, None) == BL_ERR_SHAPE
    fa[0].K = 256
    fa[0].W_packed = C + 4
    assert f(addr, 1, None) == BL_ERR_ALIGN
    fa[0].W_packed = C
    fa[1] = bl._ForwardProblem(None, None, None, D, None, None, 300, 64, 256)
    assert f(addr, 2, None) == BL_ERR_NULL              # the second problem's operands
    fa[1].M = 0
    fa[0].M = 0
    assert f(addr, 2, None) == BL_OK                    # all empty: nothing launched
    fx = L.bitlinear_forward_ex_quad_rows_grouped
    xa = (bl._ForwardExProblem * 1)()
    xa[0] = bl._ForwardExProblem(A, B, C, D, E, None, None, 300, 64, 256)
    xaddr = ctypes.addressof(xa)
    assert fx(None, 1, None) == BL_ERR_NULL and fx(xaddr, 0, None) == BL_ERR_COUNT
    xa[0].M = 8
    assert fx(xaddr, 1, None) == BL_ERR_SHAPE
    xa[0].M = 300
    xa[0].K = 320
    assert fx(xaddr, 1, None) == BL_ERR_SHAPE
    xa[0].K = 256
    xa[0].residual = 0x60002
    assert fx(xaddr, 1, None) == BL_ERR_ALIGN
    xa[0].residual = None
    xa[0].N = 0
    assert fx(xaddr, 1, None) == BL_OK
    q = L.bitlinear_quantize_step_quad_rows
    w = (bl._WeightProblem * 1)()
    w[0] = bl._WeightProblem(A, B, C, 6, 128)
    a = (bl._ActProblem * 1)()
    a[0] = bl._ActProblem(A, None, B, C, 2, 128, 0, 1e-6)
    ws = L.bitlinear_quantize_weights_grouped_workspace(1)
    wa, aa = ctypes.addressof(w), ctypes.addressof(a)
    assert q(wa, 1, D, ws, aa, 1, None) == BL_ERR_SHAPE     # N % 4 != 0
    w[0].N, w[0].K = 4, 192
    assert q(wa, 1, D, ws, aa, 1, None) == BL_ERR_SHAPE     # K % 128 != 0
    w[0].K = 128
    assert q(wa, 1, D, ws - 1, aa, 1, None) == BL_ERR_WORKSPACE
    assert q(wa, 0, D, ws, aa, 0, None) == BL_ERR_COUNT


def test_b3_entry_points_validation(L, bl):
    assert L.bitlinear_b3_row_bytes(80) == 16 and L.bitlinear_b3_row_bytes(96) == 32
    assert L.bitlinear_b3_row_bytes(2560) == 512 and L.bitlinear_b3_row_bytes(0) == 0
    pk = L.bitlinear_pack_b3
    assert pk(None, 4, 64, B, None) == BL_ERR_NULL
    assert pk(A, 4, 40, B, None) == BL_ERR_SHAPE
    assert pk(A, -1, 64, B, None) == BL_ERR_SHAPE
    assert pk(A + 4, 4, 64, B, None) == BL_ERR_ALIGN
    assert pk(None, 0, 64, None, None) == BL_OK
    g = L.bitlinear_linear_b3_grouped

    def call(**kw):
        d = dict(X=A, norm_weight=None, W_packed=B, gamma=C, Y=D, X_q=None, x_scale=None,
                 M=1, N=4, K=64, x_dtype=0, eps=1e-6)
        d.update(kw)
        arr = (bl._LinearProblem * 1)()
        arr[0] = bl._LinearProblem(**d)
        return g(ctypes.addressof(arr), 1, None)

    assert g(None, 1, None) == BL_ERR_NULL
    assert call(X=None) == BL_ERR_NULL
    assert call(M=5) == BL_ERR_SHAPE              # fused form only
    assert call(M=2, K=32768) == BL_ERR_SHAPE
    assert call(K=40) == BL_ERR_SHAPE
    assert call(x_dtype=2) == BL_ERR_DTYPE
    assert call(W_packed=B + 4) == BL_ERR_ALIGN
    assert call(M=0) == BL_OK


def test_calib_validation(L):
    cs, cm = L.bitlinear_calib_stream, L.bitlinear_calib_mfma
    assert cs(A, 40, B, None) == BL_ERR_SHAPE
    assert cs(A, -16, B, None) == BL_ERR_SHAPE
    assert cs(None, 16, B, None) == BL_ERR_NULL
    assert cs(A, 16, None, None) == BL_ERR_NULL
    assert cs(A + 4, 16, B, None) == BL_ERR_ALIGN
    assert cs(A, 16, B + 2, None) == BL_ERR_ALIGN
    assert cs(None, 0, B, None) == BL_OK
    assert cm(2, 10, 1, B, None) == BL_ERR_DTYPE
    assert cm(0, 0, 1, B, None) == BL_ERR_SHAPE
    assert cm(0, 10, 0, B, None) == BL_ERR_SHAPE
    assert cm(0, (1 << 21) + 1, 1, B, None) == BL_ERR_SHAPE
    assert cm(1, (1 << 16) + 1, 1, B, None) == BL_ERR_SHAPE
    assert cm(0, 10, 1, None, None) == BL_ERR_NULL
    assert cm(1, 10, 1, B + 2, None) == BL_ERR_ALIGN


def test_binding_refuses_host_tensors(bl):
    import torch
    with pytest.raises(TypeError):
        bl.quantize_weights(torch.zeros(4, 64))
    with pytest.raises(TypeError):
        bl.quantize_acts(torch.zeros(2, 64))


def test_package_has_no_oracle_dependency():
    """The product path never imports the oracle (only tests, smoke and the CPU baseline)."""
    pkg = os.path.join(ROOT, "bit_gemm_02_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower(), f
