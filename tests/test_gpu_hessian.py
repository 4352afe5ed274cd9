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


def test_hutchinson_long_rows_use_register_generating_kernel(nm):
    """A row stride past 2^23 elements puts the DMA offsets of a 256-row block beyond 32
    bits, so the first product runs on the tile kernel that generates the probe signs in
    registers.  Integer inputs (|x| <= 1, K = 128) keep V X^T exact in bf16 and every later
    sum an exact integer, and 4 probes make the 2/P scale exact: the result equals the
    packed-stride run and the oracle exactly."""
    n, K, R, P = 64, 128, 130, 4
    ldx = (1 << 23) + 64
    g = np.random.default_rng(6)
    Xb = O.f32_to_bf16(g.integers(-1, 2, (n, K)).astype(np.float32))
    seed = 5
    D_ref = nm.nm_hdiag_hutchinson(np_bf16(Xb).to(dev()), R, P, seed).cpu().numpy()
    big = torch.empty((n, ldx), dtype=torch.bfloat16, device=dev())   # about 1 GiB
    big[:, :K] = np_bf16(Xb).to(dev())
    assert (256 * ldx + K) * 2 >= 1 << 32
    D = nm.nm_hdiag_hutchinson(big[:, :K], R, P, seed).cpu().numpy()
    del big
    assert np.array_equal(D, D_ref)
    rows = np.unique(np.r_[0, R - 1, g.integers(0, R, 12)])
    assert np.array_equal(D[rows].astype(np.float64), O.hutchinson_rows(Xb, P, seed, rows))


# the fused diagonal -> score -> statistics call: K a multiple of 64 but not of the 256-column
# tile, rows past a tile, one and several probes
@pytest.mark.parametrize("n,K,R,P", [(64, 128, 70, 1), (128, 320, 300, 8), (192, 256, 520, 3)])
def test_hutchinson_score_fused_equals_separate_calls(nm, n, K, R, P):
    g = np.random.default_rng(n * 3 + K + R)
    Xb = O.f32_to_bf16(g.standard_normal((n, K)))
    Wb = O.f32_to_bf16(g.standard_normal((R, K)) * 0.02)
    Xd, Wd = np_bf16(Xb).to(dev()), np_bf16(Wb).to(dev())
    seed, eps = 19, 1e-6
    S, st = nm.nm_hutchinson_score(Xd, Wd, P, seed, eps)
    D = nm.nm_hdiag_hutchinson(Xd, R, P, seed)
    S2 = nm.nm_score(Wd, D, eps)
    assert torch.equal(S, S2)                       # same D, same score arithmetic
    st2 = nm.nm_score_stats(S2).cpu().numpy()
    mu, sg = O.stats(S.cpu().numpy())
    st = st.cpu().numpy()
    assert abs(st[0] - mu) <= 1e-12 * abs(mu) and abs(st[1] - sg) <= 1e-12 * sg
    assert abs(st[0] - st2[0]) <= 1e-13 * abs(mu) and abs(st[1] - st2[1]) <= 1e-13 * sg
    # and S against the oracle's score of the oracle's rows of D, to the Hutchinson bound
    rows = np.unique(np.r_[0, R - 1, g.integers(0, R, 8)])
    ref_d = O.hutchinson_rows(Xb, P, seed, rows)
    d_gpu = D[torch.from_numpy(rows).to(dev())].cpu().numpy()
    assert np.array_equal(S.cpu().numpy()[rows], O.score(Wb[rows], d_gpu, eps))
    U = O.hutchinson_u_rows(Xb, P, seed, rows)
    xk = np.sqrt((O.bf16_to_f32(Xb).astype(np.float64) ** 2).sum(0))
    tol = 2e-2 * (2.0 / P) * np.sqrt((U ** 2).sum(-1)).sum(1)[:, None] * xk[None, :]
    assert (np.abs(d_gpu - ref_d) <= tol).all()


def test_hutchinson_score_without_stats_and_rejections(nm):
    g = np.random.default_rng(2)
    n, K, R, P = 64, 128, 40, 2
    Xd = np_bf16(O.f32_to_bf16(g.standard_normal((n, K)))).to(dev())
    Wd = np_bf16(O.f32_to_bf16(g.standard_normal((R, K)))).to(dev())
    S, st = nm.nm_hutchinson_score(Xd, Wd, P, 7, 1e-6, want_stats=False)
    assert st is None
    assert torch.equal(S, nm.nm_score(Wd, nm.nm_hdiag_hutchinson(Xd, R, P, 7), 1e-6))
    with pytest.raises(nm.NMError):   # f32 weights are not taken
        nm.nm_hutchinson_score(Xd, Wd.float(), P, 7, 1e-6)


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
    for t in range(steps):
        # m_t element by element at every step: the sigmoid of z / T_t blended toward h
        mt, hm, lm = nm.nm_gate(Sd, stats, 2, 4, 0.5, 0.5, steps, m_step=t)
        m_ref, h_ref, l_ref = O.gate_anneal(S, mu, sg, 2, 4, 0.5, 0.5, steps, m_step=t)
        assert np.abs(mt.cpu().numpy() - m_ref).max() <= 1e-5, f"step {t}"
        assert np.array_equal(hm.cpu().numpy(), h_ref)
        lm = lm.cpu().numpy()
        assert np.allclose(lm, l_ref, rtol=1e-5, atol=1e-9)
        assert lm[-1] == 0.0
    # the early steps are far from binary: the comparison above sees the sigmoid itself
    m0, _, _ = O.gate_anneal(S, mu, sg, 2, 4, 0.5, 0.5, steps, m_step=0)
    assert ((m0 > 0.05) & (m0 < 0.95)).mean() > 0.3


@pytest.mark.parametrize("T0,rho,steps", [(0.5, 0.5, 8), (0.8, 0.6, 5), (2.0, 0.25, 4)])
def test_gate_two_valued_closed_form(nm, T0, rho, steps):
    """Scores 1 and 3, two of each per group: z = +-1 exactly, so at step t every kept
    entry is (1-b) expit(1/T_t) + b and every dropped one (1-b) expit(-1/T_t)."""
    from scipy.special import expit
    g = np.random.default_rng(17)
    R, K = 40, 256
    S = np.empty((R, K), np.float32)
    for r in range(R):
        for q in range(K // 4):
            S[r, 4 * q:4 * q + 4] = g.permutation([3.0, 1.0, 3.0, 1.0])
    Sd = torch.from_numpy(S).to(dev())
    assert np.allclose(nm.nm_score_stats(Sd).cpu().numpy(), [2.0, 1.0], rtol=1e-14)
    stats = torch.tensor([2.0, 1.0], dtype=torch.float64, device=dev())
    keep = S == 3.0
    for t in range(steps):
        T, b = T0 * rho ** t, t / (steps - 1)
        mt, hm, lm = nm.nm_gate(Sd, stats, 2, 4, T0, rho, steps, m_step=t)
        want = np.where(keep, (1 - b) * expit(1.0 / T) + b, (1 - b) * expit(-1.0 / T))
        assert np.abs(mt.cpu().numpy() - want).max() <= 1e-6
        assert np.array_equal(O.mask_to_bool(hm.cpu().numpy(), K), keep)


def test_gate_68_and_constant_scores(nm):
    R, K = 16, 64
    S = np.full((R, K), 0.25, np.float32)
    Sd = torch.from_numpy(S).to(dev())
    st = nm.nm_score_stats(Sd)
    assert float(st[1].cpu()) == 0.0
    for t in (0, 3, 7):
        mf, hm, lm = nm.nm_gate(Sd, st, 6, 8, 0.5, 0.5, 8, m_step=t)
        m_ref, h_ref, l_ref = O.gate_anneal(S, 0.25, 0.0, 6, 8, 0.5, 0.5, 8, m_step=t)
        assert np.array_equal(hm.cpu().numpy(), h_ref)
        assert np.allclose(lm.cpu().numpy(), l_ref, rtol=1e-5)
        # z = 0: m = (1 - beta) / 2 + beta h, one f32 rounding per operation on the GPU
        assert np.abs(mf.cpu().numpy() - m_ref).max() <= 1e-6


@pytest.mark.parametrize("N,M,K", [(6, 8, 200), (2, 4, 204)])   # K = 204: a last half-filled mask byte
def test_gate_random_every_step(nm, N, M, K):
    g = np.random.default_rng(18 + K)
    R, steps = 33, 6
    S = g.standard_normal((R, K)).astype(np.float32)
    Sd = torch.from_numpy(S).to(dev())
    mu, sg = O.stats(S)
    stats = torch.tensor([mu, sg], dtype=torch.float64, device=dev())
    for t in range(steps):
        mt, hm, lm = nm.nm_gate(Sd, stats, N, M, 0.7, 0.5, steps, m_step=t)
        m_ref, h_ref, l_ref = O.gate_anneal(S, mu, sg, N, M, 0.7, 0.5, steps, m_step=t)
        assert np.abs(mt.cpu().numpy() - m_ref).max() <= 1e-5
        assert np.array_equal(hm.cpu().numpy(), h_ref)
        assert np.allclose(lm.cpu().numpy(), l_ref, rtol=1e-5, atol=1e-9)


@pytest.mark.parametrize("steps,rho", [(24, 0.5), (24, 0.6)])
def test_gate_long_schedules_every_step(nm, steps, rho):
    """Many annealing steps: with rho = 1/2 the factor of a step is the previous one squared
    between exact 2^x evaluations, so its rounding must stay within the gate tolerance on the
    steps whose temperature puts the sigmoid of near-zero scores in its sensitive range."""
    g = np.random.default_rng(steps + int(rho * 10))
    R, K = 40, 512
    S = g.standard_normal((R, K)).astype(np.float32)
    S[:, :64] = (g.standard_normal((R, 64)) * 1e-3).astype(np.float32)   # scores near the mean
    Sd = torch.from_numpy(S).to(dev())
    mu, sg = O.stats(S)
    stats = torch.tensor([mu, sg], dtype=torch.float64, device=dev())
    for t in range(steps):
        mt, hm, lm = nm.nm_gate(Sd, stats, 2, 4, 4.0, rho, steps, m_step=t)
        m_ref, h_ref, l_ref = O.gate_anneal(S, mu, sg, 2, 4, 4.0, rho, steps, m_step=t)
        assert np.abs(mt.cpu().numpy() - m_ref).max() <= 1e-5, t
        assert np.array_equal(hm.cpu().numpy(), h_ref)
        assert np.allclose(lm.cpu().numpy(), l_ref, rtol=1e-5, atol=1e-9)


@pytest.mark.parametrize("N,M,rho", [(2, 4, 0.5), (2, 4, 0.6), (6, 8, 0.5), (6, 8, 0.6)])
def test_gate_default_schedule_kernels_agree(nm, N, M, rho):
    """The default 8-step schedule on whole 8-score units runs an unrolled kernel; a view
    with an odd leading dimension takes the general kernel.  Both do the same arithmetic,
    so every output agrees bit for bit; both are held to the oracle as well."""
    g = np.random.default_rng(31 + M + int(rho * 10))
    R, K, steps = 57, 512, 8
    S = (g.standard_normal((R, K)) * 1.3 + 0.2).astype(np.float32)
    S[:, :32] = 0.2   # ties inside groups and z = 0
    Sd = torch.from_numpy(S).to(dev())
    pad = torch.zeros((R, K + 1), dtype=torch.float32, device=dev())
    pad[:, :K] = Sd
    Sv = pad[:, :K]   # leading dimension K + 1: the general kernel
    mu, sg = O.stats(S)
    stats = torch.tensor([mu, sg], dtype=torch.float64, device=dev())
    for t in list(range(steps)) + [None]:
        a = nm.nm_gate(Sd, stats, N, M, 0.5, rho, steps, want_m=t is not None, m_step=t)
        b = nm.nm_gate(Sv, stats, N, M, 0.5, rho, steps, want_m=t is not None, m_step=t)
        assert torch.equal(a[1], b[1]) and torch.equal(a[2], b[2]), t
        if t is not None:
            assert torch.equal(a[0], b[0]), t
            m_ref, h_ref, l_ref = O.gate_anneal(S, mu, sg, N, M, 0.5, rho, steps, m_step=t)
            assert np.abs(a[0].cpu().numpy() - m_ref).max() <= 1e-5, t
            assert np.array_equal(a[1].cpu().numpy(), h_ref)
            assert np.allclose(a[2].cpu().numpy(), l_ref, rtol=1e-5, atol=1e-9)


# nm_gate_pack: the fused 2:4 pass (default 8 steps, K a multiple of 32, bf16), ragged row
# counts and both schedules of the fused kernel, and shapes that run the gate and then the
# pack (K not a multiple of 32, 6:8, other step counts, f32 weights packed to bf16)
@pytest.mark.parametrize("R,K,N,M,steps,rho,wdt", [(96, 512, 2, 4, 8, 0.5, "bf16"), (131, 1024, 2, 4, 8, 0.8, "bf16"),
                                                   (64, 520, 2, 4, 8, 0.5, "bf16"), (40, 512, 6, 8, 8, 0.5, "bf16"),
                                                   (50, 256, 2, 4, 5, 0.7, "bf16"), (33, 384, 2, 4, 8, 0.5, "f32")])
def test_gate_pack_equals_gate_then_pack(nm, R, K, N, M, steps, rho, wdt):
    g = np.random.default_rng(R + K + N + steps)
    # scores with ties (a coarse grid) so that the top-N tie rule is exercised as well
    S = np.round(g.standard_normal((R, K)) ** 2 * 8).astype(np.float32) / 8
    Sd = torch.from_numpy(S).to(dev())
    st = nm.nm_score_stats(Sd)
    Wf = (g.standard_normal((R, K)) * 0.02).astype(np.float32)
    W = np_bf16(O.f32_to_bf16(Wf)).to(dev()) if wdt == "bf16" else torch.from_numpy(Wf).to(dev())
    for m_step in (None, 2):
        mf, hm, lm = nm.nm_gate(Sd, st, N, M, 0.5, rho, steps, m_step=m_step)
        v_ref, i_ref = nm.nm_pack(W, hm, N, M, vdt=nm.NM_BF16)
        mf2, hm2, lm2, v, i = nm.nm_gate_pack(Sd, st, W, N, M, 0.5, rho, steps, m_step=m_step, vdt=nm.NM_BF16)
        assert torch.equal(hm2, hm) and torch.equal(lm2, lm)
        assert torch.equal(mf2.view(torch.int32), mf.view(torch.int32))
        assert torch.equal(v.view(torch.int16), v_ref.view(torch.int16)) and torch.equal(i, i_ref)
    # and against the oracle: the hard mask is the scores' top-N, the pack that of the weight under it
    m_or = O.topn_mask(S, N, M)
    assert np.array_equal(hm2.cpu().numpy(), m_or)
    Wh = O.f32_to_bf16(Wf) if wdt == "bf16" else Wf
    vo, io = O.pack(Wh, m_or, N, M, O.BF16)
    assert np.array_equal(v.cpu().view(torch.int16).numpy().view(np.uint16), vo)
    assert np.array_equal(i.cpu().numpy().view(np.uint32), io)
    # without the blend output
    _, hm3, lm3, v3, i3 = nm.nm_gate_pack(Sd, st, W, N, M, 0.5, rho, steps, want_m=False, vdt=nm.NM_BF16)
    assert torch.equal(hm3, hm) and torch.equal(lm3, lm) and torch.equal(v3.view(torch.int16), v.view(torch.int16))
    assert torch.equal(i3, i)
    # a weight view 4 bytes off 16-byte alignment (padded rows): the gate, then the pack
    Wp = torch.zeros((R, K + 8), dtype=W.dtype, device=dev())
    Wp[:, 2:K + 2] = W
    _, hm4, lm4, v4, i4 = nm.nm_gate_pack(Sd, st, Wp[:, 2:K + 2], N, M, 0.5, rho, steps, want_m=False, vdt=nm.NM_BF16)
    assert torch.equal(hm4, hm) and torch.equal(lm4, lm) and torch.equal(v4.view(torch.int16), v.view(torch.int16))
    assert torch.equal(i4, i)


def test_step_calls_graph_replays(nm):
    """The benchmark step's three calls (fused Hutchinson score, gate + pack, sparse product)
    captured in one HIP graph and replayed several times, outputs overwritten before each
    replay and eager calls of other shapes on the same workspaces in between: every replay
    reproduces the eager step bit for bit."""
    r = nm.raw
    g = np.random.default_rng(31)
    n, K, R, P, steps, Mt = 256, 1024, 512, 4, 8, 300
    X = np_bf16(O.f32_to_bf16(g.standard_normal((n, K)))).to(dev())
    W = np_bf16(O.f32_to_bf16(g.standard_normal((R, K)) * 0.015)).to(dev())
    X2 = np_bf16(O.f32_to_bf16(g.standard_normal((Mt, K)))).to(dev())
    S0, st0 = nm.nm_hutchinson_score(X, W, P, 5, 1e-6)
    _, hm0, lm0, v0, i0 = nm.nm_gate_pack(S0, st0, W, 2, 4, 0.5, 0.5, steps, want_m=False)
    Y0 = nm.nm_spmm(X2, v0, i0)
    refs = [t.clone() for t in (S0, st0, hm0, lm0, v0, i0, Y0)]
    u8 = torch.uint8
    S, st = torch.empty_like(S0), torch.empty_like(st0)
    hm, lm, v, i, Y = torch.empty_like(hm0), torch.empty_like(lm0), torch.empty_like(v0), torch.empty_like(i0), \
        torch.empty_like(Y0)
    wsh = torch.empty(r.nm_hutchinson_score_workspace(n, K, R, P), dtype=u8, device=dev())
    wsg = torch.empty(r.nm_gate_workspace(R, K, steps), dtype=u8, device=dev())
    wsy = torch.empty(max(1, r.nm_spmm_workspace(Mt, K, R, 0, nm.NM_BF16)), dtype=u8, device=dev())

    def chk(code):
        assert code == 0, nm.last_error()

    def step(sh):
        chk(r.nm_hutchinson_score(X.data_ptr(), n, K, K, R, P, 5, W.data_ptr(), nm.NM_BF16, K, 1e-6, S.data_ptr(), K,
                                  st.data_ptr(), wsh.data_ptr(), wsh.numel(), sh))
        chk(r.nm_gate_pack(S.data_ptr(), R, K, K, st.data_ptr(), 2, 4, 0.5, 0.5, steps, steps - 1, None, K,
                           hm.data_ptr(), K // 8, lm.data_ptr(), W.data_ptr(), nm.NM_BF16, K, nm.NM_BF16, v.data_ptr(),
                           K // 2, i.data_ptr(), K // 32, wsg.data_ptr(), wsg.numel(), sh))
        chk(r.nm_spmm(X2.data_ptr(), nm.NM_BF16, Mt, K, K, v.data_ptr(), nm.NM_BF16, i.data_ptr(), R, K // 2, K // 32,
                      0, None, 1.0, Y.data_ptr(), nm.NM_BF16, R, wsy.data_ptr(), wsy.numel(), sh))

    step(torch.cuda.current_stream().cuda_stream)   # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(torch.cuda.current_stream().cuda_stream)
    Xo = np_bf16(O.f32_to_bf16(g.standard_normal((128, K)))).to(dev())
    Wo = np_bf16(O.f32_to_bf16(g.standard_normal((256, K)) * 0.015)).to(dev())
    for rep in range(4):
        for t in (S, st, hm, lm, v, i, Y):
            t.view(torch.uint8).fill_(0xA5)
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip((S, st, hm, lm, v, i, Y), refs):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), rep
        if rep % 2 == 0:   # eager calls of other shapes on the same workspaces
            sh = torch.cuda.current_stream().cuda_stream
            So = torch.empty((256, K), dtype=torch.float32, device=dev())
            chk(r.nm_hutchinson_score(Xo.data_ptr(), 128, K, K, 256, 2, 9, Wo.data_ptr(), nm.NM_BF16, K, 1e-6,
                                      So.data_ptr(), K, st.data_ptr(), wsh.data_ptr(), wsh.numel(), sh))
            chk(r.nm_gate_pack(So.data_ptr(), 256, K, K, st.data_ptr(), 2, 4, 0.5, 0.8, steps, steps - 1, None, K,
                               hm.data_ptr(), K // 8, lm.data_ptr(), Wo.data_ptr(), nm.NM_BF16, K, nm.NM_BF16,
                               v.data_ptr(), K // 2, i.data_ptr(), K // 32, wsg.data_ptr(), wsg.numel(), sh))
            torch.cuda.synchronize()
