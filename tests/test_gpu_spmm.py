"""GPU parity of the structured-sparse GEMM (nm_spmm) against the oracle's
dense masked matmul, through the C ABI.  The packed operands come from the
oracle (stage-wise check).  Integer-valued bf16 inputs make every float sum
exact, so those cases must match bit for bit -- any operand-layout or index
mistake shows up there; random bf16 inputs are held to the tolerance
2e-2 * ||x|| * ||w_hat|| per output and to the float-accumulation bound; int8
sums must be exact in int32."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests._util import dev, host, np_bf16, row_norms

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nm():
    import semi_structured_sparsity_amd as m
    return m


def _int_bf16(g, shape, lim):
    return O.f32_to_bf16(g.integers(-lim, lim + 1, shape).astype(np.float32))


def _pack_case(W_host, Ns, N=2, M=4, score=None):
    """Oracle mask + oracle packing (plain 2:4 or lifted slide)."""
    K = W_host.shape[1]
    S = score if score is not None else O.score(W_host, None, 0.0, O.SCORE_MAGNITUDE)
    if Ns:
        mask = O.topn_mask(S, 2 * Ns - 2, 2 * Ns)
        vals, idx, bad = O.slide_decompose(W_host, mask, Ns)
        assert bad == 0
    else:
        mask = O.topn_mask(S, N, M)
        vals, idx = O.pack(W_host, mask, N, M)
    return mask, vals, idx


def _to_dev(vals, idx):
    v = np_bf16(vals) if vals.dtype == np.uint16 else torch.from_numpy(vals)
    return v.to(dev()), torch.from_numpy(idx.view(np.int32)).to(dev())


SHAPES = [  # (tokens, R, K): few-token kernel (with and without a K split over blocks), many-token
    # LDS-ring kernel, the register-staged kernel (K not a multiple of the ring stage), ragged edges
    (1, 64, 256), (16, 100, 256), (37, 257, 128), (100, 300, 512), (129, 130, 256), (300, 200, 192), (64, 96, 4096),
    (260, 160, 4096), (300, 200, 640), (520, 260, 1152),   # ring stage counts that end mid index group
    (2048, 8192, 256), (2100, 8200, 256),
    (20, 100, 96), (50, 70, 64),   # K off the rings' stage grid: weight-streaming / register-staged kernels
]


@pytest.mark.parametrize("Mt,R,K,dt", [(4096, 8192, 128, "bf16"), (4000, 4000, 384, "bf16"), (4000, 4000, 768, "i8"),
                                       (4100, 8200, 384, "bf16"), (2100, 8200, 1152, "bf16"), (4100, 8200, 192, "bf16"),
                                       (2100, 8200, 768, "i8"), (2100, 8300, 1280, "fp8")])
def test_spmm_big_tile_integer_exact_sampled(nm, Mt, R, K, dt):
    """Many-token shapes whose tile plan uses 256 x 256 tiles (the split-ring kernel): all
    rows in them (the first three cases), or whole rounds of them over the first rows and
    256 x 128 tiles on the rest (the last four; K = 192 falls back to the register-staged
    kernel).  Stage counts of one value group, and ones that end mid index group (clamped
    index loads), ragged last tiles, all three operand types.
    Integer-valued inputs make every sum exact; outputs are compared on a random sample
    plus the whole ragged last row and column of tiles."""
    g = np.random.default_rng(Mt + R + K)
    if dt == "bf16":
        X, W = _int_bf16(g, (Mt, K), 8), _int_bf16(g, (R, K), 8)
        Xo, Wo = X, W
    elif dt == "i8":
        X, W = g.integers(-8, 9, (Mt, K)).astype(np.int8), g.integers(-8, 9, (R, K)).astype(np.int8)
        Xo, Wo = X, W
    else:
        X = O.e4m3_encode(g.integers(-8, 9, (Mt, K)).astype(np.float32))
        W = O.e4m3_encode(g.integers(-8, 9, (R, K)).astype(np.float32))
        Xo, Wo = O.e4m3_decode(X), O.e4m3_decode(W)
    S = np.abs(Wo.astype(np.float32) if dt != "bf16" else O.bf16_to_f32(W)) + g.random((R, K)).astype(np.float32)
    mask = O.topn_mask(S, 2, 4)
    vals, idx = O.pack(W.view(np.int8) if dt == "fp8" else W, mask, 2, 4)
    if dt == "bf16":
        v, Xd = np_bf16(vals).to(dev()), np_bf16(X).to(dev())
    elif dt == "i8":
        v, Xd = torch.from_numpy(vals).to(dev()), torch.from_numpy(X).to(dev())
    else:
        v = torch.from_numpy(vals.view(np.uint8)).view(torch.float8_e4m3fn).to(dev())
        Xd = torch.from_numpy(X).view(torch.float8_e4m3fn).to(dev())
    i = torch.from_numpy(idx.view(np.int32)).to(dev())
    Y = nm.nm_spmm(Xd, v, i, R=R, ydt=nm.NM_I32 if dt == "i8" else nm.NM_F32).cpu().numpy()
    tm = np.concatenate([g.integers(0, Mt, 20000), np.repeat(np.arange(Mt - 260, Mt), 8), g.integers(0, Mt, 4096)])
    ro = np.concatenate([g.integers(0, R, 20000), g.integers(0, R, 260 * 8), g.integers(R - 260, R, 4096)])
    ref = O.masked_matmul_at(Xo, Wo, mask, tm, ro)
    assert np.array_equal(Y[tm, ro].astype(np.float64), ref)


@pytest.mark.parametrize("Mt,R,K", SHAPES)
@pytest.mark.parametrize("Ns", [0, 4])
def test_spmm_bf16_integer_exact(nm, Mt, R, K, Ns):
    if Ns and K % 32:
        pytest.skip("lifted bf16 needs K % 32 == 0")
    g = np.random.default_rng(Mt * 7 + R + K + Ns)
    lim = 8 if K <= 256 else 2  # every partial sum stays an integer below 2^24
    X = _int_bf16(g, (Mt, K), lim)
    W = _int_bf16(g, (R, K), lim)
    mask, vals, idx = _pack_case(W, Ns, score=O.score(W, None, 0, O.SCORE_MAGNITUDE) + g.random((R, K)).astype(np.float32))
    v, i = _to_dev(vals, idx)
    Y = nm.nm_spmm(np_bf16(X).to(dev()), v, i, R=R, Ns=Ns, ydt=nm.NM_F32).cpu().numpy()
    ref = O.masked_matmul(X, W, mask)
    assert np.array_equal(Y.astype(np.float64), ref)


# 1 to 4 tokens: K of 16 or 48 columns (one or three 16-column chunks, an odd index
# word), K off the rings' stage grid, a K split over blocks, one row
FEW = [(1, 1, 16), (2, 300, 48), (3, 257, 4160), (4, 130, 32), (1, 513, 2560), (4, 64, 4096), (1, 1000, 96)]


@pytest.mark.parametrize("Mt,R,K", FEW)
@pytest.mark.parametrize("Ns", [0, 4])
def test_spmm_bf16_few_tokens_integer_exact(nm, Mt, R, K, Ns):
    test_spmm_bf16_integer_exact(nm, Mt, R, K, Ns)


@pytest.mark.parametrize("Mt,R,K", [(16, 300, 512), (200, 260, 1024), (5, 128, 4096), (1, 300, 4096), (4, 260, 1024),
                                    (3, 70, 2560)])
@pytest.mark.parametrize("Ns", [0, 4])
def test_spmm_bf16_random_tolerance(nm, Mt, R, K, Ns):
    g = np.random.default_rng(Mt + R + K + 11 * Ns)
    X = O.f32_to_bf16(g.standard_normal((Mt, K)))
    W = O.f32_to_bf16(g.standard_normal((R, K)) * 0.02)
    mask, vals, idx = _pack_case(W, Ns)
    v, i = _to_dev(vals, idx)
    Xd = np_bf16(X).to(dev())
    Y32 = nm.nm_spmm(Xd, v, i, R=R, Ns=Ns, ydt=nm.NM_F32).cpu().numpy().astype(np.float64)
    Y16 = nm.nm_spmm(Xd, v, i, R=R, Ns=Ns, ydt=nm.NM_BF16).float().cpu().numpy().astype(np.float64)
    ref = O.masked_matmul(X, W, mask)
    Wm = np.where(O.mask_to_bool(mask, K), O.bf16_to_f32(W), 0)
    xn, wn = row_norms(O.bf16_to_f32(X)), row_norms(Wm)
    tol = 2e-2 * xn[:, None] * wn[None, :]
    assert (np.abs(Y16 - ref) <= tol).all()
    assert (np.abs(Y32 - ref) <= tol).all()
    # float accumulation of K products in any order: |err| <= K u sum |x||w|
    absdot = np.abs(O.bf16_to_f32(X)).astype(np.float64) @ np.abs(Wm).astype(np.float64).T
    assert (np.abs(Y32 - ref) <= 1.01 * K * 2.0 ** -24 * absdot + 1e-30).all()
    # bf16 output is the float result rounded once
    assert torch.equal(nm.nm_spmm(Xd, v, i, R=R, Ns=Ns, ydt=nm.NM_BF16).cpu(),
                       torch.from_numpy(Y32.astype(np.float32)).to(torch.bfloat16))


@pytest.mark.parametrize("Mt,R,K", [(1, 70, 2560), (33, 96, 256), (256, 130, 512), (300, 64, 2560),
                                    (20, 100, 192), (70, 90, 128)])
@pytest.mark.parametrize("Ns", [0, 4])
def test_spmm_int8_exact(nm, Mt, R, K, Ns):
    g = np.random.default_rng(Mt + R + K + Ns)
    Wf, Wt = synth.ternary68_weights(R=R, K=K)
    Xq = g.integers(-127, 128, (Mt, K)).astype(np.int8)
    sx = g.uniform(0.5, 2.0, Mt).astype(np.float32) / 127
    alpha = np.float32(0.8)
    S = O.score(host(Wf), None, 0.0, O.SCORE_MAGNITUDE)
    if Ns:
        mask = O.topn_mask(S, 6, 8)
        vals, idx, _ = O.slide_decompose(Wt.numpy(), mask, Ns)
    else:
        mask = O.topn_mask(S, 2, 4)
        vals, idx = O.pack(Wt.numpy(), mask, 2, 4)
    v, i = _to_dev(vals, idx)
    Xd = torch.from_numpy(Xq).to(dev())
    acc = nm.nm_spmm(Xd, v, i, R=R, Ns=Ns, ydt=nm.NM_I32).cpu().numpy()
    y = nm.nm_spmm(Xd, v, i, R=R, Ns=Ns, x_scale=torch.from_numpy(sx).to(dev()), w_scale=float(alpha),
                   ydt=nm.NM_F32).cpu().numpy()
    acc_ref, y_ref = O.masked_matmul_i8(Xq, Wt.numpy(), mask, sx, float(alpha))
    assert np.array_equal(acc, acc_ref)
    assert np.array_equal(y, y_ref)


def test_spmm_strided_views(nm):
    """Leading dimensions larger than the logical width on X, vals, idx and Y."""
    g = np.random.default_rng(5)
    Mt, R, K = 40, 72, 256
    X = _int_bf16(g, (Mt, K), 4)
    W = _int_bf16(g, (R, K), 4)
    mask, vals, idx = _pack_case(W, 0)
    Xbig = torch.zeros((Mt, K + 64), dtype=torch.bfloat16)
    Xbig[:, :K] = np_bf16(X)
    vbig = torch.zeros((R, K // 2 + 16), dtype=torch.bfloat16)
    vbig[:, :K // 2] = np_bf16(vals)
    ibig = torch.zeros((R, K // 32 + 3), dtype=torch.int32)
    ibig[:, :K // 32] = torch.from_numpy(idx.view(np.int32))
    Xd, vd, idd = Xbig.to(dev()), vbig.to(dev()), ibig.to(dev())
    Ybig = torch.full((Mt, R + 8), -7.0, device=dev())
    nm.nm_spmm(Xd[:, :K], vd[:, :K // 2], idd[:, :K // 32], R=R, ydt=nm.NM_F32, out=Ybig[:, :R])
    Y = Ybig.cpu().numpy()
    assert np.array_equal(Y[:, :R].astype(np.float64), O.masked_matmul(X, W, mask))
    assert (Y[:, R:] == -7.0).all()


def test_spmm_deterministic(nm):
    g = np.random.default_rng(9)
    X = O.f32_to_bf16(g.standard_normal((16, 4096)))
    W = O.f32_to_bf16(g.standard_normal((256, 4096)))
    _, vals, idx = _pack_case(W, 0)
    v, i = _to_dev(vals, idx)
    Xd = np_bf16(X).to(dev())
    a = nm.nm_spmm(Xd, v, i, ydt=nm.NM_F32)
    b = nm.nm_spmm(Xd, v, i, ydt=nm.NM_F32)
    assert torch.equal(a, b)
