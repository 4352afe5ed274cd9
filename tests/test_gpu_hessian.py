"""GPU parity of the Hessian-aware soft-mask path: Hutchinson diagonal,
per-tensor standardisation statistics and the gate/anneal pass, through the C
ABI, against the oracle."""
import numpy as np
import pytest
import torch

import oracle as O
from tests._util import dev, host, np_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nm():
    import semi_structured_sparsity_amd as m
    return m


def test_hutchinson_exact_for_orthogonal_columns(nm):
    """X^T X diagonal: every probe gives V.*(2 V X^T X) = 2 diag(X^T X) exactly,
    and V X^T is exactly representable in bf16 here."""
    n, K, R, P = 128, 128, 200, 3
    X = np.zeros((n, K), np.float32)
    for k in range(K):
        X[k, k] = float((k % 7) + 1)
    Xb = O.f32_to_bf16(X)
    D = nm.nm_hdiag_hutchinson(np_bf16(Xb).to(dev()), R, P, 1234).cpu().numpy()
    assert np.array_equal(D, np.tile(2.0 * np.diag(X.T @ X).astype(np.float32), (R, 1)))


# one probe with one 64-column stage per probe (a sign flip at every stage boundary) and
# one 64-column block of signs; several probes over ragged tiles
@pytest.mark.parametrize("n,K,R,P", [(64, 128, 70, 2), (128, 256, 300, 8), (64, 64, 33, 1), (192, 320, 260, 3)])
def test_hutchinson_matches_oracle_rows(nm, n, K, R, P):
    g = np.random.default_rng(n + K + R)
    Xb = O.f32_to_bf16(g.standard_normal((n, K)))
    seed = 77
    D = nm.nm_hdiag_hutchinson(np_bf16(Xb).to(dev()), R, P, seed).cpu().numpy().astype(np.float64)
    rows = np.unique(np.r_[0, R - 1, g.integers(0, R, 24)])
    ref = O.hutchinson_rows(Xb, P, seed, rows)
    U = O.hutchinson_u_rows(Xb, P, seed, rows)  # [rows, P, n]
    xk = np.sqrt((O.bf16_to_f32(Xb).astype(np.float64) ** 2).sum(0))  # ||X[:, k]||
    unorm = np.sqrt((U ** 2).sum(-1))  # [rows, P]
    tol = 2e-2 * (2.0 / P) * unorm.sum(1)[:, None] * xk[None, :]
    assert (np.abs(D[rows] - ref) <= tol).all()
    # rounding V X^T to bf16 costs a relative 2^-8 per entry; the error is far below the bound
    assert np.abs(D[rows] - ref).max() < 0.1 * tol.min() + 1e-6


def test_hutchinson_unaligned_workspace_uses_tile_kernel(nm):
    """A workspace 8 bytes off 16-byte alignment sends the second product to the 128 x 128
    tile kernel instead of the split ring; on integer inputs both equal the oracle's rows
    and each other exactly."""
    n, K, R, P = 128, 256, 300, 4
    g = np.random.default_rng(5)
    Xb = O.f32_to_bf16(g.integers(-1, 2, (n, K)).astype(np.float32))
    Xd = np_bf16(Xb).to(dev())
    seed = 91
    D_ring = nm.nm_hdiag_hutchinson(Xd, R, P, seed).cpu().numpy()
    r = nm.raw
    need = r.nm_hutchinson_workspace(n, K, R, P)
    ws = torch.empty(need + 64, dtype=torch.uint8, device=dev())
    D = torch.empty((R, K), dtype=torch.float32, device=dev())
    st = r.nm_hdiag_hutchinson(Xd.data_ptr(), n, K, K, R, P, seed, D.data_ptr(), K, ws.data_ptr() + 8, need,
                               torch.cuda.current_stream().cuda_stream)
    assert st == 0, nm.last_error()
    torch.cuda.synchronize()
    D_tile = D.cpu().numpy()
    # |x| <= 1 and K = 256: every entry of V X^T is an integer of magnitude <= 256 (exact in
    # bf16) and every sum after it an integer below 2^24, so both kernels are exact whatever
    # their order
    assert np.array_equal(D_ring, D_tile)
    rows = np.unique(np.r_[0, R - 1, g.integers(0, R, 16)])
    assert np.array_equal(D_tile[rows].astype(np.float64), O.hutchinson_rows(Xb, P, seed, rows))


def test_stats_and_gate(nm):
    g = np.random.default_rng(8)
    R, K, steps = 96, 512, 8
    S = (g.standard_normal((R, K)) ** 2).astype(np.float32)
    Sd = torch.from_numpy(S).to(dev())
    st = nm.nm_score_stats(Sd).cpu().numpy()
    mu, sg = O.stats(S)
    assert abs(st[0] - mu) <= 1e-12 * abs(mu) and abs(st[1] - sg) <= 1e-12 * sg
    # the gate is fed the oracle's statistics: one stage at a time
    stats = torch.tensor([mu, sg], dtype=torch.float64, device=dev())
    mf, hm, lm = nm.nm_gate(Sd, stats, 2, 4, 0.5, 0.5, steps)
    m_ref, h_ref, l_ref = O.gate_anneal(S, mu, sg, 2, 4, 0.5, 0.5, steps)
    assert np.array_equal(hm.cpu().numpy(), h_ref)
    assert np.abs(mf.cpu().numpy() - m_ref).max() <= 1e-5
    lm = lm.cpu().numpy()
    assert np.allclose(lm, l_ref, rtol=1e-5, atol=1e-9)
    assert lm[-1] == 0.0


def test_gate_68_and_constant_scores(nm):
    R, K = 16, 64
    S = np.full((R, K), 0.25, np.float32)
    Sd = torch.from_numpy(S).to(dev())
    st = nm.nm_score_stats(Sd)
    assert float(st[1].cpu()) == 0.0
    mf, hm, lm = nm.nm_gate(Sd, st, 6, 8, 0.5, 0.5, 8)
    m_ref, h_ref, l_ref = O.gate_anneal(S, 0.25, 0.0, 6, 8, 0.5, 0.5, 8)
    assert np.array_equal(hm.cpu().numpy(), h_ref)
    assert np.allclose(lm.cpu().numpy(), l_ref, rtol=1e-5)
    assert np.array_equal(mf.cpu().numpy(), m_ref)
