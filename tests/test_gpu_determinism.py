"""Run-to-run bitwise determinism of every entry point beside the sparse product (whose own
run-twice check sits with its parity tests): each call is made twice on the same inputs with
a call on other shapes in between (so workspaces handed out again by the caching allocator
hold other contents), and the outputs must be equal bit for bit.  Every reduction in the
library sums in one fixed order, whatever the timing of its blocks."""
import numpy as np
import pytest
import torch

import oracle as O
from tests._util import dev, np_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nm():
    import semi_structured_sparsity_amd as m
    return m


def _bf16(g, shape, scale=1.0):
    return np_bf16(O.f32_to_bf16((g.standard_normal(shape) * scale).astype(np.float32))).to(dev())


def _same(a, b):
    if a is None or b is None:
        return a is None and b is None
    # bit patterns (NaN payloads included)
    return a.shape == b.shape and torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def _twice(f, other):
    a = f()
    other()
    b = f()
    a = a if isinstance(a, tuple) else (a,)
    b = b if isinstance(b, tuple) else (b,)
    for x, y in zip(a, b):
        assert _same(x, y)


def test_hessian_path_deterministic(nm):
    g = np.random.default_rng(3)
    X, W = _bf16(g, (256, 1024)), _bf16(g, (512, 1024), 0.015)
    X2, W2 = _bf16(g, (192, 512)), _bf16(g, (300, 512), 0.015)
    _twice(lambda: nm.nm_hdiag_colsumsq(X), lambda: nm.nm_hdiag_colsumsq(X2))
    _twice(lambda: nm.nm_hdiag_hutchinson(X, 512, 4, 17), lambda: nm.nm_hdiag_hutchinson(X2, 300, 3, 5))
    _twice(lambda: nm.nm_hutchinson_score(X, W, 4, 17, 1e-6), lambda: nm.nm_hutchinson_score(X2, W2, 3, 5, 1e-6))
    S, st = nm.nm_hutchinson_score(X, W, 4, 17, 1e-6)
    S2 = nm.nm_score(W2, nm.nm_hdiag_colsumsq(X2), 1e-6)
    _twice(lambda: nm.nm_score_stats(S), lambda: nm.nm_score_stats(S2))
    st2 = nm.nm_score_stats(S2)
    for steps, rho, t in ((8, 0.5, 2), (8, 0.8, 5), (5, 0.7, 1)):
        _twice(lambda: nm.nm_gate(S, st, 2, 4, 0.5, rho, steps, m_step=t),
               lambda: nm.nm_gate(S2, st2, 6, 8, 0.5, 0.6, 3, m_step=0))


def test_mask_pack_and_quant_deterministic(nm):
    g = np.random.default_rng(4)
    W, H = _bf16(g, (1000, 2048), 0.02), torch.rand(2048, device=dev()) + 0.1
    W2 = _bf16(g, (130, 480), 0.02)
    _twice(lambda: nm.nm_prune_pack(W, H, 1e-6, nm.NM_SCORE_HESSIAN, 2, 4),
           lambda: nm.nm_prune_pack(W2, None, 0.0, nm.NM_SCORE_MAGNITUDE, 2, 4))
    _twice(lambda: nm.nm_prune_slide(W, None, 0.0, nm.NM_SCORE_MAGNITUDE, 4),
           lambda: nm.nm_prune_slide(W2, None, 0.0, nm.NM_SCORE_MAGNITUDE, 3))
    _twice(lambda: nm.nm_absmean(W), lambda: nm.nm_absmean(W2))
    X = _bf16(g, (300, 2560))
    X2 = _bf16(g, (7, 512))
    _twice(lambda: nm.nm_quant_lift(X, 4), lambda: nm.nm_quant_lift(X2, 0))
    _twice(lambda: nm.nm_quant_lift(X, 4, nm.NM_FP8), lambda: nm.nm_quant_lift(X2, 4, nm.NM_FP8))


def test_bitmap_and_lowrank_deterministic(nm):
    g = np.random.default_rng(5)
    R, K = 512, 1024
    Wd = _bf16(g, (R, K), 0.02)
    mask = torch.from_numpy(O.bool_to_mask(g.random((R, K)) < 0.5)).to(dev())
    vals, offs = nm.nm_bitmap_encode(Wd, mask)
    W2 = _bf16(g, (64, 256), 0.02)
    m2 = torch.from_numpy(O.bool_to_mask(g.random((64, 256)) < 0.3)).to(dev())
    v2, o2 = nm.nm_bitmap_encode(W2, m2)
    _twice(lambda: nm.nm_bitmap_encode(Wd, mask), lambda: nm.nm_bitmap_encode(W2, m2))
    for M in (1, 40, 600):
        X, X2 = _bf16(g, (M, K)), _bf16(g, (3, 256))
        _twice(lambda: nm.nm_spmm_bitmap(X, vals, mask, offs, ydt=nm.NM_F32),
               lambda: nm.nm_spmm_bitmap(X2, v2, m2, o2, ydt=nm.NM_F32))
    vals24, idx24, _ = nm.nm_prune_pack(Wd, None, 0.0, nm.NM_SCORE_MAGNITUDE, 2, 4)
    A, B = _bf16(g, (64, K), 0.05), _bf16(g, (R, 64), 0.05)
    for M in (5, 300):
        X = _bf16(g, (M, K))
        _twice(lambda: nm.nm_spmm_lowrank(X, vals24, idx24, A, B, ydt=nm.NM_F32),
               lambda: nm.nm_hdiag_colsumsq(X))
