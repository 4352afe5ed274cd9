"""GPU parity of the sparse layer with stacked low-rank adapters (nm_spmm_lowrank,
"SALR" section 3) against the oracle, through the C ABI.  Integer-valued inputs with a
sparse A keep the adapter intermediate u an exact bf16 integer and every sum exact in f32,
so those cases match bit for bit on every kernel path (few-token kernels with the f32 add
pass, the 256 x 128 and 256 x 256 many-token kernels with the term in their accumulators);
random inputs are held to the sparse product's tolerance 2e-2 ||x|| ||w_hat|| plus 2^-6
sum_j |u_j| |b_j| (u is rounded to bf16 from an f32 sum on the GPU, from the exact sum in
the oracle: at most one bf16 unit apart)."""
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


def _int_bf16(g, shape, lim):
    return O.f32_to_bf16(g.integers(-lim, lim + 1, shape).astype(np.float32))


def _sparse_int_a(g, rank, K, nnz=8):
    """Adapter down-projection with nnz entries of +-1 per rank row: |u| <= nnz * max|x|."""
    A = np.zeros((rank, K), np.float32)
    for j in range(rank):
        A[j, g.choice(K, nnz, replace=False)] = g.choice([-1.0, 1.0], nnz)
    return O.f32_to_bf16(A)


def _case(g, Mt, R, K, Ns, rank, integer=True):
    if integer:
        X, W = _int_bf16(g, (Mt, K), 2), _int_bf16(g, (R, K), 2)
        A, B = _sparse_int_a(g, rank, K), _int_bf16(g, (R, rank), 3)
    else:
        X = O.f32_to_bf16(g.standard_normal((Mt, K)).astype(np.float32))
        W = O.f32_to_bf16((g.standard_normal((R, K)) * 0.02).astype(np.float32))
        A = O.f32_to_bf16((g.standard_normal((rank, K)) / np.sqrt(K)).astype(np.float32))
        B = O.f32_to_bf16((g.standard_normal((R, rank)) * 0.02).astype(np.float32))
    S = O.score(W, None, 0.0, O.SCORE_MAGNITUDE) + g.random((R, K)).astype(np.float32) * (1e-3 if integer else 1e-9)
    if Ns:
        mask = O.topn_mask(S, 2 * Ns - 2, 2 * Ns)
        vals, idx, bad = O.slide_decompose(W, mask, Ns)
        assert bad == 0
    else:
        mask = O.topn_mask(S, 2, 4)
        vals, idx = O.pack(W, mask, 2, 4)
    return X, W, A, B, mask, vals, idx


def _run(nm, X, vals, idx, A, B, R, Ns, ydt):
    return nm.nm_spmm_lowrank(np_bf16(X).to(dev()), np_bf16(vals).to(dev()),
                              torch.from_numpy(idx.view(np.int32)).to(dev()), np_bf16(A).to(dev()),
                              np_bf16(B).to(dev()), R=R, Ns=Ns, ydt=ydt)


# (tokens, rows, K, rank): few-token kernels with the add pass (1, 3, 4, 16, 100, 200), the
# 256 x 128 kernel (300, 520), ragged edges everywhere; ranks with a partial 16-wide step
@pytest.mark.parametrize("Mt,R,K,rank", [(1, 96, 256, 8), (3, 130, 512, 16), (4, 300, 1024, 64), (16, 130, 512, 16),
                                         (256, 4160, 512, 16),   # 256 x 128 tiles, K split: the term once
                                         (100, 200, 1024, 72), (200, 64, 256, 64),
                                         (300, 260, 512, 24), (520, 300, 1024, 128), (300, 200, 256, 256)])
@pytest.mark.parametrize("Ns", [0, 4])
def test_spmm_lowrank_integer_exact(nm, Mt, R, K, rank, Ns):
    g = np.random.default_rng(Mt * 3 + R + K + rank + Ns)
    X, W, A, B, mask, vals, idx = _case(g, Mt, R, K, Ns, rank)
    ref = O.sparse_lowrank(X, W, mask, A, B)
    Y = _run(nm, X, vals, idx, A, B, R, Ns, nm.NM_F32).cpu().numpy()
    assert np.array_equal(Y.astype(np.float64), ref)
    Y16 = _run(nm, X, vals, idx, A, B, R, Ns, nm.NM_BF16).cpu()
    assert torch.equal(Y16, torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16))


@pytest.mark.parametrize("Mt,R,K,rank,Ns", [(2100, 8200, 384, 64, 0), (4000, 4000, 256, 32, 0), (2100, 4100, 256, 16, 4)])
def test_spmm_lowrank_big_tiles_integer_exact_sampled(nm, Mt, R, K, rank, Ns):
    """Shapes planned on 256 x 256 tiles (whole, or whole rounds plus 256 x 128 on the rest);
    outputs compared on a random sample plus the ragged last tiles."""
    g = np.random.default_rng(Mt + R + K + rank)
    X, W, A, B, mask, vals, idx = _case(g, Mt, R, K, Ns, rank)
    Y = _run(nm, X, vals, idx, A, B, R, Ns, nm.NM_F32).cpu().numpy()
    tm = np.concatenate([g.integers(0, Mt, 12000), np.repeat(np.arange(Mt - 260, Mt), 4), g.integers(0, Mt, 2048)])
    ro = np.concatenate([g.integers(0, R, 12000), g.integers(0, R, 260 * 4), g.integers(R - 260, R, 2048)])
    rows, inv = np.unique(tm, return_inverse=True)
    u = O.lowrank_u(X[rows], A)
    assert np.abs(u).max() <= 256                      # exact in bf16
    lr = (u[inv] * O.bf16_to_f32(B)[ro].astype(np.float64)).sum(axis=1)
    ref = O.masked_matmul_at(X, W, mask, tm, ro) + lr
    assert np.array_equal(Y[tm, ro].astype(np.float64), ref)


@pytest.mark.parametrize("Mt,R,K,rank,Ns", [(8, 300, 1024, 64, 0), (333, 520, 2048, 32, 0), (700, 256, 1024, 48, 4),
                                            (40, 200, 768, 16, 3), (300, 260, 640, 32, 5)])
def test_spmm_lowrank_random_tolerance(nm, Mt, R, K, rank, Ns):
    g = np.random.default_rng(Mt + 7 * R + K + rank)
    X, W, A, B, mask, vals, idx = _case(g, Mt, R, K, Ns, rank, integer=False)
    ref = O.sparse_lowrank(X, W, mask, A, B)
    Y = _run(nm, X, vals, idx, A, B, R, Ns, nm.NM_F32).cpu().numpy().astype(np.float64)
    Wm = np.where(O.mask_to_bool(mask, K), O.bf16_to_f32(W), 0)
    xn, wn = row_norms(O.bf16_to_f32(X)), row_norms(Wm)
    u = O.lowrank_u(X, A)
    ub = np.abs(u) @ np.abs(O.bf16_to_f32(B).astype(np.float64)).T
    tol = 2e-2 * xn[:, None] * wn[None, :] + 2.0 ** -6 * ub
    assert (np.abs(Y - ref) <= tol).all()


@pytest.mark.parametrize("Mt,R,K,rank,Ns", [(3, 130, 384, 16, 3), (300, 200, 768, 32, 3), (64, 96, 640, 8, 5)])
def test_spmm_lowrank_general_slide_integer_exact(nm, Mt, R, K, rank, Ns):
    g = np.random.default_rng(Mt + R + K + rank + 13 * Ns)
    X, W, A, B, mask, vals, idx = _case(g, Mt, R, K, Ns, rank)
    ref = O.sparse_lowrank(X, W, mask, A, B)
    Y = _run(nm, X, vals, idx, A, B, R, Ns, nm.NM_F32).cpu().numpy()
    assert np.array_equal(Y.astype(np.float64), ref)


def test_spmm_lowrank_zero_adapter_equals_spmm(nm):
    """With B = 0 the layer is the plain sparse product, bit for bit, on the many-token path."""
    g = np.random.default_rng(3)
    Mt, R, K, rank = 600, 520, 1024, 32
    X, W, A, B, mask, vals, idx = _case(g, Mt, R, K, 0, rank, integer=False)
    Y = _run(nm, X, vals, idx, A, np.zeros_like(B), R, 0, nm.NM_F32)
    Y0 = nm.nm_spmm(np_bf16(X).to(dev()), np_bf16(vals).to(dev()), torch.from_numpy(idx.view(np.int32)).to(dev()),
                    R=R, ydt=nm.NM_F32)
    assert torch.equal(Y, Y0)
