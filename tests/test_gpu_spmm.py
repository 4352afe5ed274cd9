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
    """Oracle mask + oracle packing (plain 2:4 or lifted slide of (2Ns-2):2Ns)."""
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


# 1 to 32 tokens: K of 16 or 48 columns (one or three 16-column chunks, an odd index
# word), K off the rings' stage grid, a K split over blocks, one row, the X range of a
# block held in LDS
FEW = [(1, 1, 16), (2, 300, 48), (3, 257, 4160), (4, 130, 32), (1, 513, 2560), (4, 64, 4096), (1, 1000, 96),
       (32, 200, 4096), (17, 130, 2048),   # X resident in LDS: a full 64 KB range, and 17 valid rows
       (1, 4096, 4096), (2, 4100, 4096),   # resident X rows of the whole K on many row tiles
       (1, 11008, 1024), (17, 9001, 512), (64, 10000, 256), (40, 14336, 768),   # row tiles of R / CUs rows
       (1, 5000, 1024), (16, 5120, 512)]   # 16-31 rows where the K split would not fill whole rounds


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
                                    (20, 100, 192), (70, 90, 128), (1, 4160, 2560)])
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


# One-byte codes at up to 64 tokens on weights whose 64-row tiles are too few for the CUs run
# the K-split ring on row tiles of R / CUs rows without splitting K (32-row tiles for shares of
# 16-32 rows, 64-row tiles above): lifted in the kernel (6:8) and plain 2:4, the resident-X
# form at one token, ragged row counts and every token row of a 32-token tile.
@pytest.mark.parametrize("dt,Ns,Mt,R,K", [("i8", 4, 1, 6912, 2560), ("i8", 0, 1, 6912, 2560), ("i8", 4, 17, 5200, 2560),
                                          ("i8", 0, 32, 8192, 1024), ("i8", 0, 5, 5150, 768), ("fp8", 4, 3, 5200, 2560),
                                          ("fp8", 0, 32, 6000, 512),
                                          ("i8", 0, 32, 5200, 2560), ("i8", 0, 3, 9000, 1024), ("fp8", 4, 1, 12000, 512),
                                          ("i8", 4, 64, 9000, 1024)])
def test_spmm_one_byte_32row_tiles_exact(nm, dt, Ns, Mt, R, K):
    g = np.random.default_rng(Mt + R + K + Ns + len(dt))
    if dt == "i8":
        X, W = g.integers(-127, 128, (Mt, K)).astype(np.int8), g.integers(-1, 2, (R, K)).astype(np.int8)
        S = W.astype(np.float32)
    else:
        X = O.e4m3_encode(g.integers(-8, 9, (Mt, K)).astype(np.float32))
        W = O.e4m3_encode(g.integers(-4, 5, (R, K)).astype(np.float32))
        S = O.e4m3_decode(W)
    Wc = W.view(np.int8) if dt == "fp8" else W
    if Ns:
        mask = O.topn_mask(np.abs(S) + g.random((R, K)).astype(np.float32), 6, 8)
        vals, idx, bad = O.slide_decompose(Wc, mask, Ns)
        assert bad == 0
    else:
        mask = O.topn_mask(np.abs(S) + g.random((R, K)).astype(np.float32), 2, 4)
        vals, idx = O.pack(Wc, mask, 2, 4)
    i = torch.from_numpy(idx.view(np.int32)).to(dev())
    if dt == "i8":
        v, Xd, ydt = torch.from_numpy(vals).to(dev()), torch.from_numpy(X).to(dev()), nm.NM_I32
        ref, _ = O.masked_matmul_i8(X, W, mask, np.ones(Mt, np.float32), 1.0)
    else:
        v = torch.from_numpy(vals.view(np.uint8)).view(torch.float8_e4m3fn).to(dev())
        Xd = torch.from_numpy(X).view(torch.float8_e4m3fn).to(dev())
        ydt = nm.NM_F32
        ref = O.masked_matmul_fp8(X, W, mask)
    if Ns == 0:
        # unsplit: the plan needs no split-K partials
        assert nm.raw.nm_spmm_workspace(Mt, K, R, 0, nm.dtype_code(Xd)) == 0
    Y = nm.nm_spmm(Xd, v, i, R=R, Ns=Ns, ydt=ydt).cpu().numpy()
    assert np.array_equal(Y.astype(np.float64), np.asarray(ref, np.float64))


# (2N-2):2N for other N: (tokens, rows, K) with K a multiple of 2N and the lifted width a
# multiple of 16 (bf16); few-token (K-split ring, or the weight-streaming kernel when the
# lifted width is off the ring's stage grid), many-token ring and register-staged shapes
GENERAL_NS = [(3, 1, 300, 384), (3, 40, 130, 96), (3, 300, 200, 768), (3, 2100, 600, 384),
              (5, 1, 257, 640), (5, 64, 300, 320), (5, 520, 260, 1280),
              (6, 16, 100, 384), (6, 300, 130, 768),
              (7, 3, 90, 224), (7, 260, 300, 448),
              (8, 1, 64, 512), (8, 129, 200, 256)]


@pytest.mark.parametrize("Ns,Mt,R,K", GENERAL_NS)
def test_spmm_general_slide_bf16_integer_exact(nm, Ns, Mt, R, K):
    """The lifted product of any (2N-2):2N weight (N-1 overlapping 2:4 windows per 2N
    group, activation lifted to (2 - 2/N) K) equals the oracle's masked product of the
    unlifted activation bit for bit on integer-valued inputs."""
    assert O.lifted_width(K, Ns) % 16 == 0
    g = np.random.default_rng(Ns * 1000 + Mt + R + K)
    X = _int_bf16(g, (Mt, K), 2)
    W = _int_bf16(g, (R, K), 2)
    mask, vals, idx = _pack_case(W, Ns, score=O.score(W, None, 0, O.SCORE_MAGNITUDE) + g.random((R, K)).astype(np.float32))
    v, i = _to_dev(vals, idx)
    Y = nm.nm_spmm(np_bf16(X).to(dev()), v, i, R=R, Ns=Ns, ydt=nm.NM_F32).cpu().numpy()
    assert np.array_equal(Y.astype(np.float64), O.masked_matmul(X, W, mask))


@pytest.mark.parametrize("Ns,Mt,R,K", [(3, 1, 70, 384), (3, 256, 130, 768), (3, 300, 64, 384),
                                       (5, 33, 96, 640), (5, 2048, 300, 640), (6, 5, 64, 1152)])
def test_spmm_general_slide_int8_exact(nm, Ns, Mt, R, K):
    """int8 x ternary under a (2N-2):2N mask from the latent weights, lifted: exact int32."""
    g = np.random.default_rng(Ns * 100 + Mt + R + K)
    Wf, Wt = synth.ternary68_weights(R=R, K=K)
    Xq = g.integers(-127, 128, (Mt, K)).astype(np.int8)
    sx = g.uniform(0.5, 2.0, Mt).astype(np.float32) / 127
    mask = O.topn_mask(O.score(host(Wf), None, 0.0, O.SCORE_MAGNITUDE), 2 * Ns - 2, 2 * Ns)
    vals, idx, bad = O.slide_decompose(Wt.numpy(), mask, Ns)
    assert bad == 0
    v, i = _to_dev(vals, idx)
    Xd = torch.from_numpy(Xq).to(dev())
    acc = nm.nm_spmm(Xd, v, i, R=R, Ns=Ns, ydt=nm.NM_I32).cpu().numpy()
    y = nm.nm_spmm(Xd, v, i, R=R, Ns=Ns, x_scale=torch.from_numpy(sx).to(dev()), w_scale=0.75,
                   ydt=nm.NM_F32).cpu().numpy()
    acc_ref, y_ref = O.masked_matmul_i8(Xq, Wt.numpy(), mask, sx, 0.75)
    assert np.array_equal(acc, acc_ref)
    assert np.array_equal(y, y_ref)


# 6:8 products of up to 256 tokens lift the activation inside the K-split ring kernel: token
# counts on each of its three tile sizes (32, 64, 128 tokens), stage counts with every
# phase of the 3-stage window pattern and K splits over blocks, rows of X with padding
# beyond K (the slot's chunks past the row end are clamped to it)
@pytest.mark.parametrize("dt", ["bf16", "i8", "fp8"])
@pytest.mark.parametrize("Mt,R,K,pad", [(1, 64, 256, 0), (1, 64, 1024, 16), (17, 130, 768, 16), (64, 96, 4096, 0), (100, 300, 512, 32),
                                       (200, 70, 1280, 0), (256, 64, 2560, 64), (3, 513, 2560, 0)])
def test_spmm_lift_in_kernel_exact(nm, dt, Mt, R, K, pad):
    g = np.random.default_rng(Mt + R + K + pad + len(dt))
    Kl = O.lifted_width(K, 4)
    if dt != "bf16" and Kl % 256:
        pytest.skip("one-byte lifted K-split ring needs K' % 256 == 0")
    if dt == "bf16":
        X, W = _int_bf16(g, (Mt, K), 2), _int_bf16(g, (R, K), 2)
        Xo, Wo = X, W
        S = O.bf16_to_f32(W)
    elif dt == "i8":
        X, W = g.integers(-127, 128, (Mt, K)).astype(np.int8), g.integers(-1, 2, (R, K)).astype(np.int8)
        Xo, Wo = X, W
        S = W.astype(np.float32)
    else:
        X = O.e4m3_encode(g.integers(-8, 9, (Mt, K)).astype(np.float32))
        W = O.e4m3_encode(g.integers(-4, 5, (R, K)).astype(np.float32))
        Xo, Wo = O.e4m3_decode(X), O.e4m3_decode(W)
        S = Wo
    mask = O.topn_mask(np.abs(S) + g.random((R, K)).astype(np.float32), 6, 8)
    vals, idx, bad = O.slide_decompose(W.view(np.int8) if dt == "fp8" else W, mask, 4)
    assert bad == 0
    i = torch.from_numpy(idx.view(np.int32)).to(dev())
    if dt == "bf16":
        v = np_bf16(vals).to(dev())
        Xbig = torch.zeros((Mt, K + pad), dtype=torch.bfloat16)
        Xbig[:, :K] = np_bf16(X)
    elif dt == "i8":
        v = torch.from_numpy(vals).to(dev())
        Xbig = torch.zeros((Mt, K + pad), dtype=torch.int8)
        Xbig[:, :K] = torch.from_numpy(X)
    else:
        v = torch.from_numpy(vals.view(np.uint8)).view(torch.float8_e4m3fn).to(dev())
        Xbig = torch.zeros((Mt, K + pad), dtype=torch.uint8)
        Xbig[:, :K] = torch.from_numpy(X)
        Xbig = Xbig.view(torch.float8_e4m3fn)
    Xd = Xbig.to(dev())[:, :K]
    ydt = nm.NM_I32 if dt == "i8" else nm.NM_F32
    Y = nm.nm_spmm(Xd, v, i, R=R, Ns=4, ydt=ydt).cpu().numpy()
    if dt == "fp8":
        ref = O.masked_matmul_fp8(X, W, mask)
    elif dt == "i8":
        ref, _ = O.masked_matmul_i8(X, W, mask, np.ones(Mt, np.float32), 1.0)
    else:
        ref = O.masked_matmul(Xo, Wo, mask)
    assert np.array_equal(Y.astype(np.float64), np.asarray(ref, np.float64))
    # the same product on the lifted activation (the plain kernel over K') agrees bit for bit
    if dt == "bf16":
        XL = np_bf16(O.lift(X, 4))
    elif dt == "i8":
        XL = torch.from_numpy(O.lift(X, 4))
    else:
        XL = torch.from_numpy(O.lift(X.view(np.int8), 4).view(np.uint8)).view(torch.float8_e4m3fn)
    Y2 = nm.nm_spmm(XL.to(dev()), v, i, R=R, Ns=0, ydt=ydt).cpu().numpy()
    assert np.array_equal(Y, Y2)


def test_spmm_workspace_query_covers_fallback_plan(nm):
    """An index view 4 bytes off 16-byte alignment with an odd row stride keeps the product
    off the DMA ring kernels; at one token on 11008 x 4096 the fallback splits K over two
    blocks.  The workspace from the query (which cannot see the pointer) must suffice, and
    the product must still equal the oracle exactly."""
    g = np.random.default_rng(21)
    Mt, R, K = 1, 11008, 4096
    X = _int_bf16(g, (Mt, K), 2)
    W = _int_bf16(g, (R, K), 2)
    mask, vals, idx = _pack_case(W, 0, score=O.score(W, None, 0, O.SCORE_MAGNITUDE) + g.random((R, K)).astype(np.float32))
    words = K // 32
    ibig = torch.zeros((R, words + 1), dtype=torch.int32)
    ibig[:, 1:] = torch.from_numpy(idx.view(np.int32))
    idd = ibig.to(dev())[:, 1:]                       # base + 4 bytes, ldi = 129
    assert idd.data_ptr() % 16 == 4 and idd.stride(0) == words + 1
    v = np_bf16(vals).to(dev())
    Xd = np_bf16(X).to(dev())
    need = nm.raw.nm_spmm_workspace(Mt, K, R, 0, nm.NM_BF16)
    assert need >= 2 * Mt * R * 4
    ws = torch.empty(need, dtype=torch.uint8, device=dev())
    Y = nm.nm_spmm(Xd, v, idd, R=R, ydt=nm.NM_F32, ws=ws).cpu().numpy()
    assert np.array_equal(Y.astype(np.float64), O.masked_matmul(X, W, mask))
    # the aligned index rows (ring plan) give the same product
    Y2 = nm.nm_spmm(Xd, v, torch.from_numpy(idx.view(np.int32)).to(dev()), R=R, ydt=nm.NM_F32, ws=ws).cpu().numpy()
    assert np.array_equal(Y, Y2)


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


# few-token shapes whose K is split over blocks (partials in the workspace, then a reduce)
SPLIT = [(4, 256, 4096, "bf16"), (1, 64, 4096, "bf16"), (64, 300, 4096, "i8"), (3, 130, 2560, "i8")]


def _split_case(nm, g, Mt, R, K, dt):
    if dt == "bf16":
        X, W = _int_bf16(g, (Mt, K), 2), _int_bf16(g, (R, K), 2)
        mask, vals, idx = _pack_case(W, 0, score=O.score(W, None, 0, O.SCORE_MAGNITUDE) + g.random((R, K)).astype(np.float32))
        Xd, ydt = np_bf16(X).to(dev()), nm.NM_F32
        ref = O.masked_matmul(X, W, mask)
    else:
        X, W = g.integers(-127, 128, (Mt, K)).astype(np.int8), g.integers(-127, 128, (R, K)).astype(np.int8)
        mask, vals, idx = _pack_case(W, 0, score=np.abs(W).astype(np.float32) + g.random((R, K)).astype(np.float32))
        Xd, ydt = torch.from_numpy(X).to(dev()), nm.NM_I32
        ref = O.masked_matmul_i8(X, W, mask, np.ones(Mt, np.float32), 1.0)[0]
    v, i = _to_dev(vals, idx)
    return Xd, v, i, ydt, ref


@pytest.mark.parametrize("Mt,R,K,dt", SPLIT)
def test_spmm_split_finish_any_workspace_contents(nm, Mt, R, K, dt):
    """The split-K partials live in the workspace: whatever it holds before the call
    (random bytes, all ones, what a previous call left), the product is exact, call after
    call on the same workspace, and after a call of another shape on it."""
    g = np.random.default_rng(Mt + R + K)
    Xd, v, i, ydt, ref = _split_case(nm, g, Mt, R, K, dt)
    xdt = nm.NM_BF16 if dt == "bf16" else nm.NM_I8
    need = nm.raw.nm_spmm_workspace(Mt, K, R, 0, xdt)
    assert need > 0, "the shape must split K over blocks"
    need = max(need, nm.raw.nm_spmm_workspace(2, 4096, 192, 0, nm.NM_BF16))   # the other shape below
    for fill in ("random", "ones", "reuse", "reuse"):
        ws = torch.empty(need + 4096, dtype=torch.uint8, device=dev()) if fill != "reuse" else ws
        if fill == "random":
            ws.copy_(torch.from_numpy(g.integers(0, 256, ws.numel(), dtype=np.uint8)).to(dev()))
        elif fill == "ones":
            ws.fill_(255)
        Y = nm.nm_spmm(Xd, v, i, R=R, ydt=ydt, ws=ws).cpu().numpy()
        assert np.array_equal(Y.astype(np.float64) if dt == "bf16" else Y, ref), fill
    # another split shape on the same workspace, then this one again
    Xo, vo, io, ydto, refo = _split_case(nm, g, 2, 192, 4096, "bf16")
    assert np.array_equal(nm.nm_spmm(Xo, vo, io, R=192, ydt=ydto, ws=ws).cpu().numpy().astype(np.float64), refo)
    Y = nm.nm_spmm(Xd, v, i, R=R, ydt=ydt, ws=ws).cpu().numpy()
    assert np.array_equal(Y.astype(np.float64) if dt == "bf16" else Y, ref)


def test_spmm_split_finish_graph_replays(nm):
    """A captured split-K product (two launches) replayed several times, with eager calls of
    another shape on the same workspace in between, gives the exact product on every replay."""
    g = np.random.default_rng(77)
    Mt, R, K = 4, 256, 4096
    Xd, v, i, ydt, ref = _split_case(nm, g, Mt, R, K, "bf16")
    Xo, vo, io, _, refo = _split_case(nm, g, 2, 192, 4096, "bf16")
    need = max(nm.raw.nm_spmm_workspace(Mt, K, R, 0, nm.NM_BF16), nm.raw.nm_spmm_workspace(2, K, 192, 0, nm.NM_BF16))
    ws = torch.empty(need, dtype=torch.uint8, device=dev())
    Y = torch.empty((Mt, R), dtype=torch.float32, device=dev())
    Yo = torch.empty((2, 192), dtype=torch.float32, device=dev())
    nm.nm_spmm(Xd, v, i, R=R, ydt=ydt, ws=ws, out=Y)   # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        nm.nm_spmm(Xd, v, i, R=R, ydt=ydt, ws=ws, out=Y)
    for rep in range(4):
        Y.fill_(-1.0)
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(Y.cpu().numpy().astype(np.float64), ref), rep
        if rep % 2 == 0:   # an eager call of another shape on the same workspace
            nm.nm_spmm(Xo, vo, io, R=192, ydt=ydt, ws=ws, out=Yo)
            torch.cuda.synchronize()
            assert np.array_equal(Yo.cpu().numpy().astype(np.float64), refo)


# 65-256 tokens on many rows (32- and 64-token tiles would need more than one round): bf16
# runs the 256 x 128 ring with its stages split over blocks (partials, then the reduce), or
# unsplit at two stages; int8 the K-split ring's 128-token tiles
RING_SPLIT = [(256, 4160, 512), (200, 4200, 1024), (130, 8300, 256)]


@pytest.mark.parametrize("Mt,R,K", RING_SPLIT)
def test_spmm_ring_split_bf16_integer_exact(nm, Mt, R, K):
    test_spmm_bf16_integer_exact(nm, Mt, R, K, 0)


@pytest.mark.parametrize("Mt,R,K", RING_SPLIT)
def test_spmm_ring_split_int8_exact(nm, Mt, R, K):
    test_spmm_int8_exact(nm, Mt, R, K, 0)
