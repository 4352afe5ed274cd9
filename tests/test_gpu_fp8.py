"""FP8 (OCP e4m3) slide path through the C ABI against the oracle: per-token FP8
quantisation fused with the 6:8 lift (codes and scales bit for bit), the FP8 x FP8
sparse product on plain 2:4 and slide-packed weights, and the whole online path.

Products of two e4m3 values are exact in f32, so integer-valued codes (every integer
up to 16 is an e4m3 value) keep every partial sum an exact integer and the product
must match the oracle bit for bit; random codes are held to the float-accumulation
bound |err| <= n u sum |x||w| with n the number of terms and u = 2^-24."""
import numpy as np
import pytest
import torch

import oracle as O
from tests._util import dev

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


@pytest.fixture(scope="module")
def nm():
    import semi_structured_sparsity_amd as m
    return m


def _bf16_dev(X):
    return torch.from_numpy(X.view(np.int16)).view(torch.bfloat16).to(dev())


def _fp8_dev(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).to(dev())


def _codes(t):
    return t.cpu().view(torch.uint8).numpy()


def _x(g, Mt, K):
    a = g.uniform(0.5, 2.0, (Mt, 1))
    X = O.f32_to_bf16((a * g.standard_normal((Mt, K))).astype(np.float32))
    if Mt > 2:
        X[1] = 0                                   # zero row: scale 0, codes 0
        X[2] = 0
        X[2, K // 2] = O.f32_to_bf16(np.array([-3.0], np.float32))[0]   # a single nonzero
    return X


def _weights(g, R, K, Ns, lim=None):
    """FP8 weight codes, their 6:8 (Ns = 4) or 2:4 mask by |w| and the oracle's packing."""
    if lim is None:
        Wc = O.e4m3_encode((g.standard_normal((R, K)) * 0.5).astype(np.float32))
    else:
        Wc = O.e4m3_encode(g.integers(-lim, lim + 1, (R, K)).astype(np.float32))
    # magnitude score with a random tie-break so the mask is unique
    S = np.abs(O.e4m3_decode(Wc)) + g.random((R, K)).astype(np.float32) * 1e-3
    if Ns:
        mask = O.topn_mask(S, 6, 8)
        vals, idx, bad = O.slide_decompose(Wc.view(np.int8), mask, Ns)
        assert bad == 0
    else:
        mask = O.topn_mask(S, 2, 4)
        vals, idx = O.pack(Wc.view(np.int8), mask, 2, 4)
    return Wc, mask, _fp8_dev(vals.view(np.uint8)), torch.from_numpy(idx.view(np.int32)).to(dev())


def _absdot(Xc, Wc, mask):
    Wm = np.where(O.mask_to_bool(mask, Wc.shape[1]), O.e4m3_decode(Wc), 0).astype(np.float64)
    return np.abs(O.e4m3_decode(Xc)).astype(np.float64) @ np.abs(Wm).T


@pytest.mark.parametrize("Mt,K", [(1, 64), (5, 8), (37, 2560), (300, 4096), (257, 1032), (2, 4104)])
@pytest.mark.parametrize("Ns", [0, 4])
def test_quant_lift_fp8_bit_exact(nm, Mt, K, Ns):
    g = np.random.default_rng(Mt * 17 + K + Ns)
    X = _x(g, Mt, K)
    Xq, sx = nm.nm_quant_lift(_bf16_dev(X), Ns, qdt=nm.NM_FP8)
    q_ref, s_ref = O.quant_lift(X, Ns, fp8=True)
    assert Xq.dtype == torch.float8_e4m3fn
    assert np.array_equal(sx.cpu().numpy(), s_ref)
    assert np.array_equal(_codes(Xq), q_ref)


def test_quant_fp8_saturation_and_ties(nm):
    """Rows whose quotients land on e4m3 rounding ties and on the largest code: the largest
    |x| maps to 448 exactly; values between codes round to the nearest, ties to even."""
    K = 64
    base = np.zeros((3, K), np.float32)
    base[:, 0] = 448.0                             # s_x = 1: quotients are the values themselves
    base[0, 1:9] = [1.0625, 1.1875, 17.0, 19.0, 0.0068359375, 240.0, 232.0, -416.0]   # ties and codes
    base[1, 1:5] = [-448.0, 447.0, 2 ** -9, 3 * 2 ** -10]                             # subnormals
    base[2, 1:] = np.linspace(-448, 448, K - 1, dtype=np.float32)
    X = O.f32_to_bf16(base)
    Xq, sx = nm.nm_quant_lift(_bf16_dev(X), 0, qdt=nm.NM_FP8)
    q_ref, s_ref = O.quant_fp8(X)
    assert np.array_equal(sx.cpu().numpy(), s_ref)
    assert np.array_equal(_codes(Xq), q_ref)
    assert (q_ref[:, 0] == 0x7E).all()             # 448 is the largest finite code


SHAPES = [(1, 70, 2560), (33, 96, 256), (256, 130, 512), (300, 64, 2560), (20, 100, 192), (70, 90, 128),
          (1100, 600, 512), (2100, 520, 1152)]


@pytest.mark.parametrize("Mt,R,K", SHAPES)
@pytest.mark.parametrize("Ns", [0, 4])
def test_spmm_fp8_integer_exact(nm, Mt, R, K, Ns):
    g = np.random.default_rng(Mt * 3 + R + K + Ns)
    lim = 8 if K <= 1024 else 4                    # every partial sum stays an integer below 2^24
    Wc, mask, v, i = _weights(g, R, K, Ns, lim=lim)
    Xc = O.e4m3_encode(g.integers(-lim, lim + 1, (Mt, K)).astype(np.float32))
    Y = nm.nm_spmm(_fp8_dev(Xc), v, i, R=R, Ns=Ns, ydt=nm.NM_F32).cpu().numpy()
    assert np.array_equal(Y.astype(np.float64), O.masked_matmul_fp8(Xc, Wc, mask))


@pytest.mark.parametrize("Mt,R,K", [(16, 300, 512), (200, 260, 1024), (5, 128, 4096), (1024, 512, 2560)])
@pytest.mark.parametrize("Ns", [0, 4])
def test_spmm_fp8_random_bound(nm, Mt, R, K, Ns):
    g = np.random.default_rng(Mt + R + K + 5 * Ns)
    Wc, mask, v, i = _weights(g, R, K, Ns)
    Xc = O.e4m3_encode((g.standard_normal((Mt, K)) * 4).astype(np.float32))
    Xd = _fp8_dev(Xc)
    Y32 = nm.nm_spmm(Xd, v, i, R=R, Ns=Ns, ydt=nm.NM_F32).cpu().numpy()
    ref = O.masked_matmul_fp8(Xc, Wc, mask)
    assert (np.abs(Y32.astype(np.float64) - ref) <= 1.01 * K * U * _absdot(Xc, Wc, mask) + 1e-30).all()
    # bf16 output is the f32 result rounded once
    Y16 = nm.nm_spmm(Xd, v, i, R=R, Ns=Ns, ydt=nm.NM_BF16).cpu()
    assert torch.equal(Y16, torch.from_numpy(Y32).to(torch.bfloat16))
    # scales: y = (w_scale * x_scale[m]) * acc in f32
    sx = g.uniform(0.5, 2.0, Mt).astype(np.float32) / 448
    ys = nm.nm_spmm(Xd, v, i, R=R, Ns=Ns, x_scale=torch.from_numpy(sx).to(dev()), w_scale=0.75,
                    ydt=nm.NM_F32).cpu().numpy()
    assert np.array_equal(ys, (np.float32(0.75) * sx)[:, None] * Y32)


@pytest.mark.parametrize("Mt,R,K", [(1, 70, 2560), (200, 300, 512), (600, 256, 4096)])
def test_online_fp8_slide_path(nm, Mt, R, K):
    """bf16 X -> FP8 quantise + lift -> FP8 sparse product over K' with the slide-packed FP8
    weight; the codes and scales must match the oracle bit for bit, the output within the
    accumulation bound of the oracle's product of the unlifted codes."""
    g = np.random.default_rng(Mt * 5 + R + K)
    Wc, mask, v, i = _weights(g, R, K, 4)
    X = _x(g, Mt, K)
    XL, sx = nm.nm_quant_lift(_bf16_dev(X), 4, qdt=nm.NM_FP8)
    Xc, s_ref = O.quant_fp8(X)
    assert np.array_equal(sx.cpu().numpy(), s_ref)
    assert np.array_equal(_codes(XL), O.lift(Xc.view(np.int8), 4).view(np.uint8))
    w_scale = 0.5
    acc = nm.nm_spmm(XL, v, i, R=R, Ns=0, ydt=nm.NM_F32).cpu().numpy().astype(np.float64)
    y = nm.nm_spmm(XL, v, i, R=R, Ns=0, x_scale=sx, w_scale=w_scale, ydt=nm.NM_F32).cpu().numpy()
    ref = O.masked_matmul_fp8(Xc, Wc, mask)
    bound = 1.01 * K * U * _absdot(Xc, Wc, mask) + 1e-30
    assert (np.abs(acc - ref) <= bound).all()
    scale = (np.float32(w_scale) * s_ref).astype(np.float64)[:, None]
    assert (np.abs(y - scale * ref) <= scale * bound + 2 * U * np.abs(scale * ref) + 1e-30).all()
    if Mt > 2:
        assert (y[1] == 0).all()                   # a zero row gives zero output
