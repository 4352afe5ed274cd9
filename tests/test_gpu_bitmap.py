"""GPU parity of the bitmap format ("SALR", section 4) through the C ABI: the encoder
(values and block table) bit for bit against the oracle, and the two-stage product
(decode into LDS, then dense MFMA) against the oracle's masked product -- bit for bit on
integer-valued inputs (every partial sum exact in f32), within 2e-2 ||x|| ||w_hat|| and
the float-accumulation bound on random ones -- for unstructured masks of several
densities, 2:4 and 6:8 masks, ragged edges, a K split over blocks, up to 4 tokens (the
row-streaming kernel), a full round of 256 x 256 tiles (the dense split ring on the
decoded weight) and rows whose kept count exceeds the value capacity."""
import numpy as np
import pytest
import torch

import oracle as O
from tests._util import dev, np_bf16, row_norms

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nm():
    import semi_structured_sparsity_amd as m
    return m


def _mask(g, W, kind):
    R, K = W.shape
    if kind == "2:4":
        return O.topn_mask(O.score(W, None, 0.0, O.SCORE_MAGNITUDE) + g.random((R, K)).astype(np.float32) * 1e-6, 2, 4)
    if kind == "6:8":
        return O.topn_mask(O.score(W, None, 0.0, O.SCORE_MAGNITUDE) + g.random((R, K)).astype(np.float32) * 1e-6, 6, 8)
    return O.bool_to_mask(g.random((R, K)) < float(kind))     # unstructured, density = kind


def _enc(nm, W, mask, ldv):
    return nm.nm_bitmap_encode(np_bf16(W).to(dev()), torch.from_numpy(mask).to(dev()), ldv=ldv)


@pytest.mark.parametrize("R,K,kind", [(37, 192, "0.5"), (130, 4096, "0.25"), (64, 8192, "0.75"), (100, 256, "2:4"),
                                      (33, 512, "6:8"), (5, 64, "0.0"), (7, 128, "1.0")])
def test_bitmap_encode_bit_exact(nm, R, K, kind):
    g = np.random.default_rng(R + K)
    W = O.f32_to_bf16(g.standard_normal((R, K)).astype(np.float32))
    mask = _mask(g, W, kind)
    vals_ref, offs_ref = O.bitmap_encode(W, mask)
    vals, offs = _enc(nm, W, mask, K)
    assert np.array_equal(offs.cpu().numpy(), offs_ref)
    assert np.array_equal(vals.cpu().view(torch.int16).numpy().view(np.uint16), vals_ref)


def test_bitmap_encode_capacity_drops_last_values(nm):
    g = np.random.default_rng(5)
    R, K, cap = 20, 256, 100
    W = O.f32_to_bf16(g.standard_normal((R, K)).astype(np.float32))
    mask = _mask(g, W, "0.6")                           # about 154 kept per row, 100 stored
    vals_ref, offs_ref = O.bitmap_encode(W, mask, ldv=cap)
    vals, offs = _enc(nm, W, mask, cap)
    assert np.array_equal(offs.cpu().numpy(), offs_ref)
    assert np.array_equal(vals.cpu().view(torch.int16).numpy().view(np.uint16), vals_ref)


# (tokens, rows, K, mask): K split over blocks (few tiles), many tokens, ragged edges
@pytest.mark.parametrize("Mt,R,K,kind", [(1, 200, 1024, "0.5"), (16, 130, 512, "2:4"), (100, 300, 2048, "6:8"),
                                         (300, 260, 512, "0.5"), (520, 130, 256, "0.3"), (2100, 1030, 1152, "0.5"),
                                         # a full round of 256 x 256 tiles: the dense split ring on the decoded
                                         # weight (exactly one round; ragged on both edges)
                                         (2048, 8192, 256, "6:8"), (2100, 8200, 192, "0.5")])
def test_spmm_bitmap_integer_exact(nm, Mt, R, K, kind):
    g = np.random.default_rng(Mt * 3 + R + K)
    X = O.f32_to_bf16(g.integers(-4, 5, (Mt, K)).astype(np.float32))
    W = O.f32_to_bf16(g.integers(-4, 5, (R, K)).astype(np.float32))
    mask = _mask(g, W, kind)
    vals, offs = O.bitmap_encode(W, mask)
    ref = O.masked_matmul(X, W, mask)
    md = torch.from_numpy(mask).to(dev())
    Xd, vd, od = np_bf16(X).to(dev()), np_bf16(vals).to(dev()), torch.from_numpy(offs).to(dev())
    Y = nm.nm_spmm_bitmap(Xd, vd, md, od, R=R, ydt=nm.NM_F32).cpu().numpy()
    assert np.array_equal(Y.astype(np.float64), ref)
    Y16 = nm.nm_spmm_bitmap(Xd, vd, md, od, R=R, ydt=nm.NM_BF16).cpu()
    assert torch.equal(Y16, torch.from_numpy(Y).to(torch.bfloat16))


# up to 4 tokens: the row-streaming kernel (one wave per weight row); K off a multiple of
# 512 columns leaves some lanes a group fewer, one row and K = 64 are the smallest cases
@pytest.mark.parametrize("Mt,R,K,kind", [(1, 300, 4160, "6:8"), (2, 257, 1024, "0.5"), (3, 64, 64, "0.3"),
                                         (4, 1000, 2048, "2:4"), (1, 1, 64, "0.5"), (4, 130, 8192, "0.9"),
                                         (1, 513, 1536, "0.05")])
def test_spmm_bitmap_few_tokens_integer_exact(nm, Mt, R, K, kind):
    test_spmm_bitmap_integer_exact(nm, Mt, R, K, kind)


@pytest.mark.parametrize("Mt,R,K,kind", [(8, 300, 2048, "0.5"), (400, 520, 1024, "6:8"), (1, 700, 4096, "6:8"),
                                         (4, 300, 2048, "0.5"), (2048, 8192, 320, "0.5")])
def test_spmm_bitmap_random_tolerance(nm, Mt, R, K, kind):
    g = np.random.default_rng(Mt + R + K + 1)
    X = O.f32_to_bf16(g.standard_normal((Mt, K)).astype(np.float32))
    W = O.f32_to_bf16((g.standard_normal((R, K)) * 0.02).astype(np.float32))
    mask = _mask(g, W, kind)
    vals, offs = O.bitmap_encode(W, mask)
    Y = nm.nm_spmm_bitmap(np_bf16(X).to(dev()), np_bf16(vals).to(dev()), torch.from_numpy(mask).to(dev()),
                          torch.from_numpy(offs).to(dev()), R=R, ydt=nm.NM_F32).cpu().numpy().astype(np.float64)
    ref = O.masked_matmul(X, W, mask)
    Wm = np.where(O.mask_to_bool(mask, K), O.bf16_to_f32(W), 0)
    xn, wn = row_norms(O.bf16_to_f32(X)), row_norms(Wm)
    assert (np.abs(Y - ref) <= 2e-2 * xn[:, None] * wn[None, :]).all()
    absdot = np.abs(O.bf16_to_f32(X)).astype(np.float64) @ np.abs(Wm).astype(np.float64).T
    assert (np.abs(Y - ref) <= 1.01 * K * 2.0 ** -24 * absdot + 1e-30).all()


@pytest.mark.parametrize("Mt", [64, 2])
def test_spmm_bitmap_values_past_capacity_read_as_zero(nm, Mt):
    g = np.random.default_rng(8 + Mt)
    R, K, cap = 96, 512, 200
    X = O.f32_to_bf16(g.integers(-3, 4, (Mt, K)).astype(np.float32))
    W = O.f32_to_bf16(g.integers(-3, 4, (R, K)).astype(np.float32))
    mask = _mask(g, W, "0.6")
    vals, offs = O.bitmap_encode(W, mask, ldv=cap)
    Wd = O.bitmap_decode(vals, mask, K)
    Y = nm.nm_spmm_bitmap(np_bf16(X).to(dev()), np_bf16(vals).to(dev()), torch.from_numpy(mask).to(dev()),
                          torch.from_numpy(offs).to(dev()), R=R, ydt=nm.NM_F32).cpu().numpy()
    assert np.array_equal(Y.astype(np.float64), O.masked_matmul(X, Wd, None))
