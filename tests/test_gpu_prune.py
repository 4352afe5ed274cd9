"""GPU parity of the weight-side kernels against the CPU oracle, called through
the C ABI: curvature column sums, scores, top-N masks, packing, the fused
score->mask->pack pass, the sliding-window decomposition and the ternary
scale.  Integer, mask and index outputs must match bit for bit."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests._util import bf16_np, dev, host, np_bf16, u32_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nm():
    import semi_structured_sparsity_amd as m
    return m


def _bf16(a):
    return np_bf16(O.f32_to_bf16(a))


# ------------------------------------------------------------------ A1
@pytest.mark.parametrize("n,K,dt", [(512, 4096, "bf16"), (100, 264, "bf16"), (37, 72, "f32"), (1, 8, "bf16")])
def test_colsumsq(nm, n, K, dt):
    g = np.random.default_rng(n + K)
    Xf = g.standard_normal((n, K)).astype(np.float32)
    X = _bf16(Xf) if dt == "bf16" else torch.from_numpy(Xf)
    H = nm.nm_hdiag_colsumsq(X.to(dev())).cpu().numpy().astype(np.float64)
    ref = O.colsumsq(host(X))
    # The GPU sums the (exact) squares in f64 over at most n/32 + 32 additions per column and
    # rounds once to f32; the oracle sums them in f64 in row order.  Both f64 sums are within
    # (additions) * 2^-53 of the exact sum (all terms are positive), so the two results differ
    # by at most the final f32 rounding, 2^-24 relative, plus those f64 errors.
    tol = (2.0 ** -24 + (n + n / 32 + 33) * 2.0 ** -53) * ref * (1 + 1e-12) + 1e-300
    assert (np.abs(H - ref) <= tol).all()
    # it is the f32 rounding of the oracle's sum except where that sum lies within the f64
    # errors of a rounding boundary
    assert (H == ref.astype(np.float32)).mean() > 0.999


# ------------------------------------------------------------------ A3
def test_score_tiny24_and_full_curvature(nm):
    W, H, _ = synth.tiny24_inputs()
    S = nm.nm_score(W.to(dev()), H.to(dev()), 1e-6).cpu().numpy()
    assert np.array_equal(S, O.score(W.numpy(), H.numpy(), 1e-6))
    g = np.random.default_rng(3)
    Wb = _bf16(g.standard_normal((96, 200)) * 0.02)
    Hf = g.uniform(-0.5, 2, (96, 200)).astype(np.float32)  # a Hutchinson diagonal may be negative
    S = nm.nm_score(Wb.to(dev()), torch.from_numpy(Hf).to(dev()), 1e-6).cpu().numpy()
    assert np.array_equal(S, O.score(host(Wb), Hf, 1e-6))
    S = nm.nm_score(Wb.to(dev()), None, 0.0, nm.NM_SCORE_MAGNITUDE).cpu().numpy()
    assert np.array_equal(S, O.score(host(Wb), None, 0.0, O.SCORE_MAGNITUDE))
    Hrow = g.uniform(0.1, 1.0, 200).astype(np.float32)  # one curvature per input column, shared by the rows
    S = nm.nm_score(Wb.to(dev()), torch.from_numpy(Hrow).to(dev()), 1e-6).cpu().numpy()
    assert np.array_equal(S, O.score(host(Wb), Hrow, 1e-6))


# ------------------------------------------------------------------ A7
@pytest.mark.parametrize("N,M", [(2, 4), (1, 4), (3, 4), (6, 8), (4, 8), (2, 8), (7, 8)])
def test_mask_with_ties_nan_signed_zero(nm, N, M):
    g = np.random.default_rng(N * 10 + M)
    R, K = 67, 8 * M + M  # ragged: not a multiple of 8 bytes when M = 4
    S = g.integers(0, 5, (R, K)).astype(np.float32)
    S[g.random((R, K)) < 0.05] = np.nan
    S[g.random((R, K)) < 0.05] = -0.0
    S[g.random((R, K)) < 0.02] = -np.inf
    mask = nm.nm_mask(torch.from_numpy(S).to(dev()), N, M).cpu().numpy()
    ref = O.topn_mask(S, N, M)
    assert np.array_equal(mask, ref)


# ------------------------------------------------------------------ A8
@pytest.mark.parametrize("N,M,dt", [(2, 4, "bf16"), (2, 4, "f32"), (6, 8, "bf16"), (1, 4, "i8"), (6, 8, "i8"),
                                    (3, 8, "bf16"), (7, 8, "i8")])
def test_pack_with_short_groups(nm, N, M, dt):
    g = np.random.default_rng(100 + N * 10 + M)
    R, K = 45, 40 * M
    Wf = g.standard_normal((R, K)).astype(np.float32)
    if dt == "bf16":
        W, vdt = _bf16(Wf), nm.NM_BF16
    elif dt == "f32":
        W, vdt = torch.from_numpy(Wf), nm.NM_BF16
    else:
        W, vdt = torch.from_numpy(g.integers(-1, 2, (R, K)).astype(np.int8)), nm.NM_I8
    bits = g.random((R, K)) < (N / M)  # any number of bits per group: short groups get padded
    mask = O.bool_to_mask(bits)
    vals, idx = nm.nm_pack(W.to(dev()), torch.from_numpy(mask).to(dev()), N, M, vdt)
    v_ref, i_ref = O.pack(host(W), mask, N, M, {nm.NM_BF16: O.BF16, nm.NM_I8: O.I8}[vdt])
    assert np.array_equal(host(vals), v_ref)
    assert np.array_equal(u32_np(idx), i_ref)


@pytest.mark.parametrize("N,M", [(2, 4), (6, 8), (3, 8)])
def test_pack_validate_flag(nm, N, M):
    """NM_FLAG_VALIDATE: a mask with over-full groups is refused with NM_ERR_PATTERN and the
    oracle's count of such groups, and nothing is written; a valid mask (N or fewer bits per
    group) packs exactly as without the flag."""
    g = np.random.default_rng(300 + N * 10 + M)
    R, K = 37, 24 * M
    W = _bf16(g.standard_normal((R, K)))
    Wd = W.to(dev())
    bits = g.random((R, K)) < (N + 0.5) / M
    mask = O.bool_to_mask(bits)
    bad = O.mask_overfull(mask, K, M, N)
    assert bad > 0
    slots = K // M * N
    words = nm.index_words(slots, M)
    vals = torch.full((R, slots), 7.0, dtype=torch.bfloat16, device=dev())
    idx = torch.full((R, words), -1, dtype=torch.int32, device=dev())
    md = torch.from_numpy(mask).to(dev())
    st = nm.raw.nm_pack(Wd.data_ptr(), nm.NM_BF16, R, K, K, md.data_ptr(), md.shape[1], N, M, nm.NM_BF16,
                        vals.data_ptr(), slots, idx.data_ptr(), words, nm.NM_FLAG_VALIDATE,
                        torch.cuda.current_stream().cuda_stream)
    assert nm.STATUS_NAMES[st] == "NM_ERR_PATTERN"
    assert f"{bad} groups" in nm.last_error()
    torch.cuda.synchronize()
    assert (vals == 7.0).all() and (idx == -1).all()
    with pytest.raises(nm.NMError):
        nm.nm_pack(Wd, md, N, M, flags=nm.NM_FLAG_VALIDATE)
    # valid: the top-N of a random score, minus a few bits (short groups are padded)
    keep = O.mask_to_bool(O.topn_mask(g.random((R, K)).astype(np.float32), N, M), K) & (g.random((R, K)) > 0.1)
    good = O.bool_to_mask(keep)
    assert O.mask_overfull(good, K, M, N) == 0
    gd = torch.from_numpy(good).to(dev())
    v1, i1 = nm.nm_pack(Wd, gd, N, M, flags=nm.NM_FLAG_VALIDATE)
    v0, i0 = nm.nm_pack(Wd, gd, N, M)
    v_ref, i_ref = O.pack(host(W), good, N, M)
    assert torch.equal(v1, v0) and torch.equal(i1, i0)
    assert np.array_equal(host(v1), v_ref) and np.array_equal(u32_np(i1), i_ref)


@pytest.mark.parametrize("Ns", [3, 4, 5])
def test_slide_validate_flag(nm, Ns):
    g = np.random.default_rng(400 + Ns)
    G = 2 * Ns
    R, K = 23, G * 17
    W = _bf16(g.standard_normal((R, K)))
    Wd = W.to(dev())
    bits = g.random((R, K)) < (G - 1.5) / G
    mask = O.bool_to_mask(bits)
    bad = O.mask_overfull(mask, K, G, G - 2)
    assert bad > 0
    with pytest.raises(nm.NMError) as e:
        nm.nm_slide_decompose(Wd, torch.from_numpy(mask).to(dev()), Ns, flags=nm.NM_FLAG_VALIDATE)
    assert e.value.status == nm.NM_ERR_PATTERN and f"{bad} groups" in str(e.value)
    keep = O.mask_to_bool(O.topn_mask(g.random((R, K)).astype(np.float32), G - 2, G), K) if G <= 8 else \
        np.stack([np.concatenate([g.permutation(np.r_[np.ones(G - 2), np.zeros(2)]) for _ in range(K // G)])
                  for _ in range(R)]).astype(bool)
    good = O.bool_to_mask(keep & (g.random((R, K)) > 0.1))
    vals, idx = nm.nm_slide_decompose(Wd, torch.from_numpy(good).to(dev()), Ns, flags=nm.NM_FLAG_VALIDATE)
    v_ref, i_ref, nb = O.slide_decompose(host(W), good, Ns)
    assert nb == 0
    assert np.array_equal(host(vals), v_ref) and np.array_equal(u32_np(idx), i_ref)


# ------------------------------------------------------------------ fused A3 + A7 + A8
@pytest.mark.parametrize("case", ["tiny24", "bf16_hess", "bf16_hess_full", "bf16_mag", "generic68", "generic14"])
def test_prune_pack_fused(nm, case):
    g = np.random.default_rng(7)
    if case == "tiny24":
        W, H, _ = synth.tiny24_inputs()
        N, M, mode, Hn = 2, 4, nm.NM_SCORE_HESSIAN, H.numpy()
    else:
        R, K = 131, 264  # ragged rows; K not a multiple of 32 (partial index word)
        W = _bf16(g.standard_normal((R, K)) * 0.02)
        N, M = {"generic68": (6, 8), "generic14": (1, 4)}.get(case, (2, 4))
        mode = nm.NM_SCORE_MAGNITUDE if case == "bf16_mag" else nm.NM_SCORE_HESSIAN
        if case == "bf16_hess_full":
            Hn = g.uniform(0.1, 1, (R, K)).astype(np.float32)
        else:
            Hn = g.uniform(0.1, 1, K).astype(np.float32)
        H = torch.from_numpy(Hn)
    Hd = None if mode == nm.NM_SCORE_MAGNITUDE else H.to(dev())
    vals, idx, mask = nm.nm_prune_pack(W.to(dev()), Hd, 1e-6, mode, N, M)
    Wn = host(W)
    S = O.score(Wn, None if mode == nm.NM_SCORE_MAGNITUDE else Hn, 1e-6,
                O.SCORE_MAGNITUDE if mode == nm.NM_SCORE_MAGNITUDE else O.SCORE_HESSIAN)
    m_ref = O.topn_mask(S, N, M)
    v_ref, i_ref = O.pack(Wn, m_ref, N, M, O.BF16)
    assert np.array_equal(mask.cpu().numpy(), m_ref)
    assert np.array_equal(host(vals), v_ref)
    assert np.array_equal(u32_np(idx), i_ref)


@pytest.mark.parametrize("kind,mode", [("pack24", "mag"), ("pack24", "hess"), ("slide68", "mag"), ("slide68", "hess")])
def test_fused_topn_ties_and_special_values(nm, kind, mode):
    """The fused 2-of-4 and 6-of-8 selections on weights drawn from a handful of values
    (ties in most groups), with NaN, infinities and signed zeros: masks, values and
    indices bit for bit against the oracle's counting rule."""
    g = np.random.default_rng(41 + (kind == "slide68") + 2 * (mode == "hess"))
    R, K = 53, 1024
    pool = np.array([0.0, -0.0, 1.0, -1.0, 2.0, -2.0, 0.5, np.nan, np.inf, -np.inf], np.float32)
    Wf = pool[g.choice(len(pool), (R, K), p=[0.2, 0.1, 0.15, 0.15, 0.1, 0.1, 0.1, 0.04, 0.03, 0.03])]
    W = _bf16(Wf)
    Hn = g.choice(np.array([0.25, 0.5, 1.0], np.float32), K) if mode == "hess" else None
    smode = nm.NM_SCORE_HESSIAN if mode == "hess" else nm.NM_SCORE_MAGNITUDE
    Hd = torch.from_numpy(Hn).to(dev()) if Hn is not None else None
    S = O.score(host(W), Hn, 1e-6, O.SCORE_HESSIAN if mode == "hess" else O.SCORE_MAGNITUDE)
    if kind == "pack24":
        vals, idx, mask = nm.nm_prune_pack(W.to(dev()), Hd, 1e-6, smode, 2, 4)
        m_ref = O.topn_mask(S, 2, 4)
        v_ref, i_ref = O.pack(host(W), m_ref, 2, 4, O.BF16)
    else:
        vals, idx, mask = nm.nm_prune_slide(W.to(dev()), Hd, 1e-6, smode, 4)
        m_ref = O.topn_mask(S, 6, 8)
        v_ref, i_ref, bad = O.slide_decompose(host(W), m_ref, 4)
        assert bad == 0
    assert np.array_equal(mask.cpu().numpy(), m_ref)
    assert np.array_equal(host(vals).view(np.uint16), v_ref.view(np.uint16))
    assert np.array_equal(u32_np(idx), i_ref)


def test_prune_pack_ternary_quant_then_mask(nm):
    """Mask from the bf16 master weights, values from the ternary code."""
    Wf, Wt = synth.ternary68_weights(R=70, K=256)
    vals, idx, mask = nm.nm_prune_pack(Wf.to(dev()), None, 0.0, nm.NM_SCORE_MAGNITUDE, 6, 8, Wv=Wt.to(dev()))
    m_ref = O.topn_mask(O.score(host(Wf), None, 0.0, O.SCORE_MAGNITUDE), 6, 8)
    v_ref, i_ref = O.pack(Wt.numpy(), m_ref, 6, 8, O.I8)
    assert np.array_equal(mask.cpu().numpy(), m_ref)
    assert np.array_equal(vals.cpu().numpy(), v_ref)
    assert np.array_equal(u32_np(idx), i_ref)


# ------------------------------------------------------------------ A9
@pytest.mark.parametrize("Ns", [2, 3, 4, 5, 6, 7, 8])
def test_slide_decompose_all_n(nm, Ns):
    g = np.random.default_rng(200 + Ns)
    M = 2 * Ns
    R, K = 29, M * 21
    W = _bf16(g.standard_normal((R, K)))
    # masks with at most 2N-2 bits per group (the (2N-2):2N family), some sparser
    keep = O.topn_mask(g.random((R, K)).astype(np.float32), M - 2, M) if M <= 8 else None
    if keep is None:
        bits = np.zeros((R, K), bool)
        for r in range(R):
            for gi in range(K // M):
                sel = g.choice(M, size=g.integers(0, M - 1), replace=False)
                bits[r, gi * M + sel] = True
        keep = O.bool_to_mask(bits)
    else:
        drop = g.random((R, K)) < 0.1
        keep = O.bool_to_mask(O.mask_to_bool(keep, K) & ~drop)
    vals, idx = nm.nm_slide_decompose(W.to(dev()), torch.from_numpy(keep).to(dev()), Ns)
    v_ref, i_ref, bad = O.slide_decompose(host(W), keep, Ns)
    assert bad == 0
    assert np.array_equal(host(vals), v_ref)
    assert np.array_equal(u32_np(idx), i_ref)


@pytest.mark.parametrize("kind", ["bf16", "ternary"])
def test_prune_slide_fused(nm, kind):
    if kind == "bf16":
        W = synth.slide68_weight(R=90, K=512)
        Wv = None
        v_host = host(W)
    else:
        W, Wt = synth.ternary68_weights(R=90, K=512)
        Wv = Wt.to(dev())
        v_host = Wt.numpy()
    vals, idx, mask = nm.nm_prune_slide(W.to(dev()), None, 0.0, nm.NM_SCORE_MAGNITUDE, 4, Wv=Wv)
    m_ref = O.topn_mask(O.score(host(W), None, 0.0, O.SCORE_MAGNITUDE), 6, 8)
    v_ref, i_ref, bad = O.slide_decompose(v_host, m_ref, 4)
    assert bad == 0
    assert np.array_equal(mask.cpu().numpy(), m_ref)
    assert np.array_equal(host(vals), v_ref)
    assert np.array_equal(u32_np(idx), i_ref)


# ------------------------------------------------------------------ A10
def test_absmean(nm):
    Wf, _ = synth.ternary68_weights(R=300, K=2560)
    a = float(nm.nm_absmean(Wf.to(dev())).cpu()[0])
    ref = np.float32(O.absmean(host(Wf)))
    # both reduce in double (different orders) and round once to float
    assert abs(a - ref) <= 2 * np.spacing(ref)
