"""Pins for the CPU oracle: each test ties an oracle function to something other
than itself -- a value printed on the pages, a closed form, an invariant, a
library routine that computes the same quantity independently, or brute force
over every case on tiny inputs.  CPU only."""
import itertools
import math
from pathlib import Path

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = Path(__file__).resolve().parent / "golden"


def _rng(seed):
    return np.random.default_rng(seed)


# ------------------------------------------------------------------ numerics
def test_bf16_rounding_matches_torch():
    g = _rng(0)
    x = np.concatenate([
        g.standard_normal(20000).astype(np.float32),
        (g.standard_normal(2000) * 1e-39).astype(np.float32),          # subnormals
        np.array([0.0, -0.0, np.inf, -np.inf, 1.0, -1.0, 3.0e38, -3.0e38], np.float32),
    ])
    # exact ties: mantissa ends in 0x8000 (round to even both ways)
    ties = (np.arange(1, 2001, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    ours = O.f32_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    nan = O.f32_to_bf16(np.array([np.nan], np.float32))
    assert np.isnan(O.bf16_to_f32(nan))[0]
    back = O.bf16_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


# ------------------------------------------------------------------ A1
def test_colsumsq_closed_forms():
    n, K = 7, 12
    X = np.full((n, K), 3.0, np.float32)
    assert np.array_equal(O.colsumsq(X), np.full(K, 9.0 * n))
    I = np.eye(K, dtype=np.float32)[:n]
    H = O.colsumsq(I)
    assert np.array_equal(H, np.r_[np.ones(n), np.zeros(K - n)])
    g = _rng(1)
    Xb = O.f32_to_bf16(g.standard_normal((33, 40)))
    Xf = O.bf16_to_f32(Xb).astype(np.float64)
    assert np.allclose(O.colsumsq(Xb), np.einsum("ik,ik->k", Xf, Xf), rtol=1e-14, atol=0)


def test_colsumsq_expectation():
    g = _rng(2)
    X = O.f32_to_bf16(g.standard_normal((512, 256)))
    H = O.colsumsq(X)
    # E[x^2] = 1 for N(0,1): mean over columns of H/n within 5 sigma (sd of chi2_n/n = sqrt(2/n))
    assert abs(H.mean() / 512 - 1.0) < 5 * math.sqrt(2 / 512) / math.sqrt(256)


# ------------------------------------------------------------------ A3
def test_score_exact_powers_of_two():
    K = 16
    w = np.array([2.0 ** (-e) for e in range(K)], np.float32)[None, :]
    h = np.full(K, 0.75, np.float32)
    S = O.score(w, h, 0.25)
    assert np.array_equal(S[0], (w[0].astype(np.float64) ** 2).astype(np.float32))  # (0.75+0.25) * w^2


def test_score_magnitude_mode_and_constant_curvature():
    g = _rng(3)
    W = O.f32_to_bf16(g.standard_normal((64, 64)) * 0.02)
    Wf = O.bf16_to_f32(W)
    assert np.array_equal(O.score(W, None, 0.0, O.SCORE_MAGNITUDE), np.abs(Wf))
    # constant curvature ranks exactly as magnitude: w^2 of a bf16 value is exact in float
    S = O.score(W, np.full(64, 0.3, np.float32), 1e-6)
    for N, M in ((2, 4), (6, 8)):
        assert np.array_equal(O.topn_mask(S, N, M), O.topn_mask(np.abs(Wf), N, M))


def test_score_against_float32_ops_and_broadcast():
    g = _rng(4)
    W = g.standard_normal((8, 32)).astype(np.float32) * 0.02
    H = g.uniform(0.1, 1, 32).astype(np.float32)
    eps = np.float32(1e-6)
    ref = (H + eps) * (W * W)  # numpy float32 ops, one rounding each
    assert np.array_equal(O.score(W, H, 1e-6), ref)
    Hfull = g.uniform(0.1, 1, (8, 32)).astype(np.float32)
    assert np.array_equal(O.score(W, Hfull, 1e-6), (Hfull + eps) * (W * W))


# ------------------------------------------------------------------ A7
def _brute_topn(vals, N):
    """The unique N-subset whose every member beats every non-member."""
    M = len(vals)

    def key(x):
        return -np.inf if np.isnan(x) else x + 0.0

    def beats(i, j):
        return key(vals[i]) > key(vals[j]) or (key(vals[i]) == key(vals[j]) and i < j)

    winners = [c for c in itertools.combinations(range(M), N)
               if all(beats(i, j) for i in c for j in range(M) if j not in c)]
    assert len(winners) == 1
    return set(winners[0])


@pytest.mark.parametrize("N,M", [(1, 4), (2, 4), (3, 4), (2, 8), (4, 8), (6, 8)])
def test_topn_bruteforce_and_stable_sort(N, M):
    g = _rng(10 + N * 10 + M)
    R, K = 40, 8 * M
    S = g.integers(0, 4, (R, K)).astype(np.float32)  # many ties
    S[g.random((R, K)) < 0.05] = np.nan
    S[g.random((R, K)) < 0.05] = -0.0
    mask = O.mask_to_bool(O.topn_mask(S, N, M), K)
    for r in range(R):
        for gi in range(K // M):
            grp = S[r, gi * M:(gi + 1) * M]
            kept = set(np.nonzero(mask[r, gi * M:(gi + 1) * M])[0])
            assert kept == _brute_topn(grp, N)
            keys = np.where(np.isnan(grp), -np.inf, grp + 0.0)
            order = np.argsort(-keys, kind="stable")
            assert kept == set(order[:N].tolist())
    assert (mask.reshape(R, K // M, M).sum(-1) == N).all()


def test_topn_crafted_ties():
    S = np.array([[1, 1, 1, 1, 5, 2, 5, 2, 0, 0, 7, 7]], np.float32)
    m = O.mask_to_bool(O.topn_mask(S, 2, 4), 12)[0]
    assert m.tolist() == [1, 1, 0, 0, 1, 0, 1, 0, 0, 0, 1, 1]
    S = np.array([[-0.0, 0.0, np.nan, -1.0]], np.float32)
    m = O.mask_to_bool(O.topn_mask(S, 2, 4), 4)[0]
    assert m.tolist() == [1, 1, 0, 0]
    m = O.mask_to_bool(O.topn_mask(S, 3, 4), 4)[0]
    assert m.tolist() == [1, 1, 0, 1]  # NaN ranks below -1


# ------------------------------------------------------------------ A8
@pytest.mark.parametrize("N,M,dt", [(2, 4, "bf16"), (2, 4, "f32in"), (6, 8, "bf16"), (1, 4, "i8"), (4, 8, "i8")])
def test_pack_roundtrip(N, M, dt):
    g = _rng(20 + N + M)
    R, K = 24, 16 * M
    Wf = g.standard_normal((R, K)).astype(np.float32)
    if dt == "bf16":
        W = O.f32_to_bf16(Wf)
        vdt = O.BF16
        expect = W
    elif dt == "f32in":
        W = Wf
        vdt = O.BF16
        expect = O.f32_to_bf16(Wf)
    else:
        W = g.integers(-1, 2, (R, K)).astype(np.int8)
        vdt = O.I8
        expect = W
    mask = O.topn_mask(np.abs(Wf), N, M)
    vals, idx = O.pack(W, mask, N, M, vdt)
    assert vals.shape == (R, K * N // M)
    b = math.ceil(math.log2(M))
    assert idx.shape == (R, (K * N // M * b + 31) // 32)
    dense = O.unpack(vals, idx, K, N, M)
    mb = O.mask_to_bool(mask, K)
    assert np.array_equal(dense, np.where(mb, expect, 0).astype(dense.dtype))
    # in-group indices strictly ascending, decoded by hand from the bitstream
    bits = np.unpackbits(idx.view(np.uint8), axis=1, bitorder="little")
    for r in range(0, R, 5):
        f = [int(sum(bits[r, j * b + t] << t for t in range(b))) for j in range(K * N // M)]
        for gi in range(K // M):
            pos = f[gi * N:(gi + 1) * N]
            assert all(pos[i] < pos[i + 1] for i in range(N - 1))
            assert set(pos) == set(np.nonzero(mb[r, gi * M:(gi + 1) * M])[0])


def test_pack_pads_short_groups():
    W = np.arange(1, 9, dtype=np.float32)[None, :]
    mask = O.bool_to_mask(np.array([[0, 0, 1, 0, 0, 0, 0, 0]], bool))  # group0: one bit, group1: none
    vals, idx = O.pack(W, mask, 2, 4, O.F32)
    assert vals.tolist() == [[0.0, 3.0, 0.0, 0.0]]
    # group0 positions {0 (pad), 2}, group1 positions {0, 1} (both pads): fields 0,2,0,1
    assert idx[0, 0] == (0 | 2 << 2 | 0 << 4 | 1 << 6)


# ------------------------------------------------------------------ A9 / A11
def test_slide_golden_windows_and_gamma():
    rows = [l.split() for l in (GOLDEN / "slide68_windows.txt").read_text().splitlines()
            if l.strip() and not l.startswith("#")]
    wins = [tuple(map(int, r)) for r in rows if r[0] != "gamma"]
    gam = [r for r in rows if r[0] == "gamma"][0]
    N = int(gam[1])
    assert O.lifted_width(8, N) / 8 == float(gam[2])
    assert 2 - 2 / N == float(gam[2]) and N / (N - 1) == pytest.approx(float(gam[3]))
    # a single 8-wide group of ones: lift shows which original column each lifted slot reads
    X = np.arange(1, 9, dtype=np.float32)[None, :]
    Xl = O.lift(X, N)[0]
    for (_, w, first, last) in wins:
        assert Xl[4 * (w - 1):4 * w].tolist() == list(range(first, last + 1))


@pytest.mark.parametrize("Ns", [2, 3, 4, 5, 6])
def test_slide_exhaustive_coverage(Ns):
    """Every 2N-bit mask with at most 2N-2 set bits fits N-1 windows; fold restores W."""
    M = 2 * Ns
    masks = [m for m in range(1 << M) if bin(m).count("1") <= M - 2]
    assert len(masks) == {2: 11, 3: 57, 4: 247, 5: 1013, 6: 4083}[Ns]
    R = len(masks)
    bits = np.array([[(m >> p) & 1 for p in range(M)] for m in masks], bool)
    W = np.arange(1, R * M + 1, dtype=np.float32).reshape(R, M)
    vals, idx, bad = O.slide_decompose(W, O.bool_to_mask(bits), Ns, O.F32)
    assert bad == 0
    assert vals.shape == (R, 2 * (Ns - 1))
    fold = O.slide_fold(vals, idx, M, Ns)
    assert np.array_equal(fold, np.where(bits, W, 0))
    # masks with exactly 2N-2 bits: every window holds two real entries (no zero padding)
    full = bits.sum(1) == M - 2
    assert (vals[full] != 0).all()
    # N-2 windows can never hold 2N-2 entries
    assert 2 * (Ns - 2) < M - 2


def test_slide_overfull_group_is_reported():
    bits = np.ones((1, 8), bool)  # 8 of 8 set: cannot fit 3 windows
    _, _, bad = O.slide_decompose(np.ones((1, 8), np.float32), O.bool_to_mask(bits), 4, O.F32)
    assert bad == 2


@pytest.mark.parametrize("G,cap", [(4, 2), (8, 6), (8, 4), (6, 4), (10, 8), (14, 12), (16, 14)])
def test_mask_overfull_counts_groups(G, cap):
    """The pattern check counts groups of G consecutive bits with more than cap set:
    against numpy's own bit unpacking and a per-group popcount, on random masks of a
    density that leaves some groups over and some under (and a ragged last byte)."""
    g = _rng(80 + G + cap)
    R, K = 9, G * 13
    p = (cap + 0.7) / G   # groups hover around the cap
    bits = g.random((R, K)) < p
    mask = np.zeros((R, (K + 7) // 8 + 3), np.uint8)   # row stride beyond ceil(K/8)
    packed = np.packbits(bits, axis=1, bitorder="little")
    mask[:, :packed.shape[1]] = packed
    want = int((bits.reshape(R, K // G, G).sum(-1) > cap).sum())
    assert 0 < want < R * K // G
    assert O.mask_overfull(mask, K, G, cap) == want
    # bits past K in the row's last byte and beyond never count
    mask[:, (K // 8):] |= np.uint8(0xFF) << np.uint8(K % 8) if K % 8 else 0
    mask[:, (K + 7) // 8:] = 0xFF
    assert O.mask_overfull(mask, K, G, cap) == want
    assert O.mask_overfull(O.bool_to_mask(np.ones((2, K), bool)), K, G, cap) == 2 * (K // G)
    assert O.mask_overfull(O.bool_to_mask(np.zeros((2, K), bool)), K, G, cap) == 0


@pytest.mark.parametrize("Ns", [3, 4])
def test_lifted_product_equals_dense_masked(Ns):
    g = _rng(30 + Ns)
    R, K, Mt = 12, 2 * Ns * 6, 5
    W = g.integers(-8, 9, (R, K)).astype(np.float32)
    X = g.integers(-8, 9, (Mt, K)).astype(np.float32)
    mask = O.topn_mask(np.abs(W) + g.random((R, K)).astype(np.float32) * 0.5, 2 * Ns - 2, 2 * Ns)
    vals, idx, bad = O.slide_decompose(W, mask, Ns, O.F32)
    assert bad == 0
    Wl = O.unpack(vals, idx, O.lifted_width(K, Ns), 2, 4).astype(np.float64)
    Xl = O.lift(X, Ns).astype(np.float64)
    Wm = np.where(O.mask_to_bool(mask, K), W, 0).astype(np.float64)
    assert np.array_equal(Xl @ Wl.T, X.astype(np.float64) @ Wm.T)
    assert np.array_equal(O.masked_matmul(X, W, mask), X.astype(np.float64) @ Wm.T)


# ------------------------------------------------------------------ per-token int8 quantisation (SlideSparse 2B/2C)
def test_quant_unit_scale_is_round_half_even():
    """A row whose absolute maximum is 127 has scale exactly 1, so the codes are the
    values rounded to the nearest integer with ties to even (numpy's rint)."""
    vals = np.array([127, -2.5, -1.5, -0.5, 0.5, 1.5, 2.5, 3.5, 0.25, -126.5, 63.75, 7.0], np.float32)
    X = O.f32_to_bf16(vals[None, :])
    xf = O.bf16_to_f32(X)[0]
    Xq, sx = O.quant_i8(X)
    assert sx[0] == 1.0
    assert np.array_equal(Xq[0], np.rint(xf).astype(np.int8))
    assert list(Xq[0, 1:8]) == [-2, -2, 0, 0, 2, 2, 4]


def test_quant_power_of_two_scales_and_zero_row():
    """max|x| = 127 * 2^e gives scale 2^e exactly: codes are rint(x / 2^e); a zero row has
    scale 0 and codes 0; the extreme element always maps to +-127."""
    g = _rng(70)
    rows = []
    for e in (-6, -1, 0, 3):
        r = g.integers(-126, 127, 16).astype(np.float32) * 2.0 ** e + 0.25 * 2.0 ** e
        r[5] = -127 * 2.0 ** e
        rows.append(r)
    X = O.f32_to_bf16(np.stack(rows + [np.zeros(16, np.float32)]))
    xf = O.bf16_to_f32(X).astype(np.float64)
    Xq, sx = O.quant_i8(X)
    for i, e in enumerate((-6, -1, 0, 3)):
        assert sx[i] == 2.0 ** e
        assert np.array_equal(Xq[i], np.rint(xf[i] / 2.0 ** e).astype(np.int8))
        assert Xq[i, 5] == -127
    assert sx[-1] == 0.0 and not Xq[-1].any()


def test_quant_error_bound_and_lift():
    """Random rows: |x - s q| <= s/2 (plus the float rounding of s and of x/s), |q| <= 127
    with the absmax element at +-127; the lifted codes are the codes remapped by the lift."""
    g = _rng(71)
    Mt, K = 9, 64
    a = g.uniform(0.5, 2.0, Mt)
    X = O.f32_to_bf16((a[:, None] * g.uniform(-1, 1, (Mt, K))).astype(np.float32))
    xf = O.bf16_to_f32(X).astype(np.float64)
    Xq, sx = O.quant_i8(X)
    s = sx.astype(np.float64)[:, None]
    assert (np.abs(xf - s * Xq) <= s * (0.5 + 1e-5)).all()
    assert (np.abs(Xq.astype(np.int32)) <= 127).all()
    assert (np.abs(Xq[np.arange(Mt), np.abs(xf).argmax(1)]) == 127).all()
    XL, sx2 = O.quant_lift(X, 4)
    assert np.array_equal(sx2, sx) and np.array_equal(XL, O.lift(Xq, 4))
    # lift by its definition: lifted column 12q + 4w + l holds column 8q + 2w + l
    for c in range(O.lifted_width(K, 4)):
        q, r = divmod(c, 12)
        w, l = divmod(r, 4)
        assert np.array_equal(XL[:, c], Xq[:, 8 * q + 2 * w + l])


# ------------------------------------------------------------------ FP8 e4m3 (SlideSparse: FP8 among the precisions)
def test_e4m3_decode_all_codes_matches_torch():
    c = np.arange(256, dtype=np.uint8)
    d = O.e4m3_decode(c)
    t = torch.from_numpy(c).view(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(np.isnan(d), np.isnan(t))
    assert np.array_equal(d[~np.isnan(d)], t[~np.isnan(t)])
    assert d[0x7e] == 448.0 and d[0x01] == 2.0 ** -9 and d[0x08] == 2.0 ** -6


def test_e4m3_encode_matches_torch_rounding_and_saturates():
    """Round-half-even against torch's float8_e4m3fn cast on every finite value, every
    midpoint between neighbouring codes, and random values; past 448 the oracle
    saturates (torch gives NaN there, so those are checked by value)."""
    fin = O.e4m3_decode(np.arange(127, dtype=np.uint8)).astype(np.float64)
    mids = ((fin[:-1] + fin[1:]) / 2).astype(np.float32)
    g = _rng(72)
    rnd = np.concatenate([g.uniform(-448, 448, 4000), g.uniform(-2.0 ** -5, 2.0 ** -5, 2000)]).astype(np.float32)
    for x in (fin.astype(np.float32), -fin.astype(np.float32), mids, -mids, rnd):
        ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(O.e4m3_encode(x), ref)
    assert list(O.e4m3_encode(np.array([448.0, 449.0, 1e6, -500.0], np.float32))) == [0x7e, 0x7e, 0x7e, 0xfe]


def test_quant_fp8_unit_scale_zero_row_and_error_bound():
    g = _rng(73)
    Mt, K = 6, 40
    a = g.uniform(0.5, 2.0, (Mt, 1))
    Xf = (a * g.uniform(-1, 1, (Mt, K))).astype(np.float32)
    Xf[0] = np.clip(Xf[0] * 300, -447, 447)
    Xf[0, 3] = 448.0                       # max|x| = 448: scale exactly 1
    Xf[1] = 0.0
    X = O.f32_to_bf16(Xf)
    xf = O.bf16_to_f32(X)
    Xq, sx = O.quant_fp8(X)
    assert sx[0] == 1.0
    assert np.array_equal(Xq[0], torch.from_numpy(xf[0]).to(torch.float8_e4m3fn).view(torch.uint8).numpy())
    assert sx[1] == 0.0 and not Xq[1].any()
    dq = O.e4m3_decode(Xq).astype(np.float64) * sx[:, None]
    # e4m3 keeps 4 significant bits: relative error <= 2^-4 for normals, absolute
    # <= 2^-10 * s in the subnormal range, plus the float rounding of s and x / s
    err = np.abs(dq - xf.astype(np.float64))
    bound = np.maximum(np.abs(xf) * 2.0 ** -4, 2.0 ** -10 * sx[:, None]) * (1 + 1e-5)
    assert (err <= bound).all()
    XL, sx2 = O.quant_lift(X, 4, fp8=True)
    assert np.array_equal(sx2, sx) and np.array_equal(XL, O.lift(Xq.view(np.int8), 4).view(np.uint8))


def test_masked_matmul_fp8_against_decoded_values():
    g = _rng(74)
    Mt, R, K = 3, 5, 24
    Xq = g.integers(0, 256, (Mt, K)).astype(np.uint8)
    Wq = g.integers(0, 256, (R, K)).astype(np.uint8)
    Xq[(Xq & 0x7f) == 0x7f] = 0x00          # no NaN codes
    Wq[(Wq & 0x7f) == 0x7f] = 0x38
    mask = O.topn_mask(g.random((R, K)).astype(np.float32), 6, 8)
    xd = torch.from_numpy(Xq).view(torch.float8_e4m3fn).double().numpy()
    wd = torch.from_numpy(Wq).view(torch.float8_e4m3fn).double().numpy()
    wm = np.where(O.mask_to_bool(mask, K), wd, 0.0)
    assert np.array_equal(O.masked_matmul_fp8(Xq, Wq, mask), xd @ wm.T)
    assert np.array_equal(O.masked_matmul_fp8(Xq, Wq), xd @ wd.T)


# ------------------------------------------------------------------ A12 / A13
def test_masked_matmul_bruteforce_tiny():
    g = _rng(40)
    for trial in range(20):
        Mt, R, K = g.integers(1, 9), g.integers(1, 9), 4 * g.integers(1, 9)
        X = g.standard_normal((Mt, K)).astype(np.float32)
        W = g.standard_normal((R, K)).astype(np.float32)
        mb = g.random((R, K)) < 0.5
        Y = O.masked_matmul(X, W, O.bool_to_mask(mb))
        ref = X.astype(np.float64) @ np.where(mb, W, 0).astype(np.float64).T
        assert np.allclose(Y, ref, rtol=1e-13, atol=1e-13)
    Xb = O.f32_to_bf16(g.standard_normal((3, 16)))
    Wb = O.f32_to_bf16(g.standard_normal((5, 16)))
    ref = O.bf16_to_f32(Xb).astype(np.float64) @ O.bf16_to_f32(Wb).astype(np.float64).T
    assert np.allclose(O.masked_matmul(Xb, Wb), ref, rtol=1e-13, atol=1e-13)
    ro, rm = np.array([4, 0, 2]), np.array([1, 2, 0])
    assert np.array_equal(O.masked_matmul_at(Xb, Wb, None, rm, ro), O.masked_matmul(Xb, Wb)[rm, ro])


def test_masked_matmul_i8_exact():
    g = _rng(41)
    Xq = g.integers(-127, 128, (6, 64)).astype(np.int8)
    Wt = g.integers(-1, 2, (9, 64)).astype(np.int8)
    mb = g.random((9, 64)) < 0.75
    sx = g.uniform(0.01, 0.02, 6).astype(np.float32)
    acc, y = O.masked_matmul_i8(Xq, Wt, O.bool_to_mask(mb), sx, 0.8)
    ref = Xq.astype(np.int64) @ np.where(mb, Wt, 0).astype(np.int64).T
    assert np.array_equal(acc, ref)
    assert np.array_equal(y, (np.float32(0.8) * sx)[:, None] * ref.astype(np.float32))


# ------------------------------------------------------------------ A10
def test_absmean_and_quant_then_mask():
    W = np.array([[-2.0, 1.0, 0.5, -0.5]], np.float32)
    assert O.absmean(W) == 1.0
    g = _rng(50)
    Wf = g.standard_normal((16, 64)).astype(np.float32)
    Wt = np.where(np.abs(Wf) > 0.55, np.sign(Wf), 0).astype(np.int8)
    mask = O.topn_mask(np.abs(Wf), 6, 8)
    Weff = O.apply_mask_i8(Wt, mask)
    # quantising zero gives zero, so masking before or after the code is the same
    assert np.array_equal(Weff, np.where(O.mask_to_bool(mask, 64), Wt, 0))
    assert O.absmean(Wf) == pytest.approx(np.abs(Wf.astype(np.float64)).mean(), rel=1e-15)


# ------------------------------------------------------------------ A2
def test_splitmix64_published_outputs():
    rows = [l.split() for l in (GOLDEN / "splitmix64_seed0.txt").read_text().splitlines()
            if l.strip() and not l.startswith("#")]
    for i, hx in rows:
        assert O.splitmix64_at(0, int(i)) == int(hx, 16)


def test_rademacher_balance_and_independence():
    K = 4096
    v = np.array([[O.rademacher(7, p, o, k, K) for k in range(0, K, 3)] for p in range(2) for o in range(4)])
    assert set(np.unique(v)) == {-1, 1}
    n = v.shape[1]
    assert abs(v.mean()) < 5 / math.sqrt(v.size)
    c = (v[0] * v[1]).mean()
    assert abs(c) < 5 / math.sqrt(n)


def test_hutchinson_matches_autograd_hessian():
    """Brute force: the full Hessian of ||X W^T||_F^2 from autograd, then the
    estimator (1/P) sum_p v_p * (Hess v_p) with the same probe signs."""
    g = _rng(60)
    n, K, R, P, seed = 5, 8, 3, 4, 11
    X = g.standard_normal((n, K))
    Xt = torch.from_numpy(X)

    def loss(w):
        return ((Xt @ w.reshape(R, K).T) ** 2).sum()

    Hs = torch.autograd.functional.hessian(loss, torch.zeros(R * K, dtype=torch.float64)).numpy()
    V = np.array([[[O.rademacher(seed, p, o, k, K) for k in range(K)] for o in range(R)] for p in range(P)], float)
    est = np.mean([V[p].ravel() * (Hs @ V[p].ravel()) for p in range(P)], axis=0).reshape(R, K)
    D = O.hutchinson_rows(X.astype(np.float32), P, seed, np.arange(R))
    assert np.allclose(D, est, rtol=1e-6, atol=1e-6 * np.abs(est).max())
    # and the exact diagonal is 2 * sum_i x_ik^2 for every row
    assert np.allclose(np.diag(Hs).reshape(R, K), 2 * (X ** 2).sum(0)[None, :])


def test_hutchinson_exact_for_orthogonal_columns():
    n, K = 12, 8
    X = np.zeros((n, K), np.float32)
    for k in range(K):
        X[k, k] = k + 1.0
    D = O.hutchinson_rows(X, 3, 5, np.arange(6))
    assert np.array_equal(D, np.tile(2.0 * np.arange(1, K + 1) ** 2, (6, 1)))


def test_hutchinson_unbiased():
    g = _rng(61)
    n, K, P = 16, 32, 2
    X = O.f32_to_bf16(g.standard_normal((n, K)))
    rows = np.arange(400)
    D = O.hutchinson_rows(X, P, 3, rows)
    target = 2 * O.colsumsq(X)
    Xf = O.bf16_to_f32(X).astype(np.float64)
    A = Xf.T @ Xf  # off-diagonal terms give the estimator's variance
    var = 4 * ((A ** 2).sum(1) - np.diag(A) ** 2) / P
    se = np.sqrt(var / rows.size)
    assert (np.abs(D.mean(0) - target) < 5 * se).all()


def test_hutchinson_u_rows_definition():
    g = _rng(62)
    X = g.standard_normal((6, 70)).astype(np.float32)
    U = O.hutchinson_u_rows(X, 2, 9, np.array([3, 1]))
    for q, o in enumerate([3, 1]):
        for p in range(2):
            v = np.array([O.rademacher(9, p, o, k, 70) for k in range(70)], float)
            assert np.allclose(U[q, p], X.astype(np.float64) @ v)


# ------------------------------------------------------------------ A4 - A6
def test_stats_match_numpy():
    g = _rng(70)
    S = (g.standard_normal((64, 128)) ** 2).astype(np.float32)
    mu, sg = O.stats(S)
    assert mu == pytest.approx(S.astype(np.float64).mean(), rel=1e-14)
    assert sg == pytest.approx(S.astype(np.float64).std(), rel=1e-12)
    z = (S.astype(np.float64) - mu) / sg
    assert abs(z.mean()) < 1e-12 and abs(z.std() - 1) < 1e-12


def test_gate_constant_scores_closed_form():
    """sigma = 0 -> z = 0 -> gate 0.5, so Lmid_t = n/4 (1 - beta_t^2)."""
    R, K, steps = 4, 16, 8
    S = np.full((R, K), 0.3, np.float32)
    mu, sg = O.stats(S)
    assert sg == 0.0
    m, hard, lm = O.gate_anneal(S, mu, sg, 2, 4, 0.5, 0.5, steps)
    beta = np.arange(steps) / (steps - 1)
    assert np.allclose(lm, R * K / 4 * (1 - beta ** 2), rtol=1e-14, atol=1e-12)
    assert O.gate_value(0.3, mu, sg, 0.5, 0.5, 0) == 0.5
    # ties everywhere: the hard mask keeps the first two of each group
    assert (O.mask_to_bool(hard, K).reshape(R, K // 4, 4) == [1, 1, 0, 0]).all()


def test_anneal_projection_invariants():
    g = _rng(71)
    R, K, steps = 32, 64, 8
    S = (g.standard_normal((R, K)) ** 2).astype(np.float32)
    mu, sg = O.stats(S)
    m, hard, lm = O.gate_anneal(S, mu, sg, 2, 4, 0.5, 0.5, steps)
    h = O.topn_mask(S, 2, 4)
    assert np.array_equal(hard, h)                        # beta = 1 at the end: projection = hard target
    assert np.array_equal(m, O.mask_to_bool(h, K).astype(np.float32))
    assert lm[-1] == 0.0
    assert ((lm >= 0) & (lm <= R * K / 4)).all()
    assert (np.diff(lm) <= 0).all()                       # separation grows as beta and 1/T grow
    # gate is monotone in the score and 1/2 at the mean
    s_sorted = np.sort(S.ravel())[:: max(1, S.size // 200)]
    gv = [O.gate_value(float(s), mu, sg, 0.5, 0.5, 2) for s in s_sorted]
    assert all(a <= b for a, b in zip(gv, gv[1:]))
    assert O.gate_value(np.float32(mu), mu, sg, 0.5, 0.5, 0) == pytest.approx(0.5, abs=1e-7)
    # for any step with beta > 0 the top-N of the blend is the hard target
    hb = O.mask_to_bool(h, K)
    for t in range(1, steps):
        beta = t / (steps - 1)
        gt = np.array([[O.gate_value(float(S[r, k]), mu, sg, 0.5, 0.5, t) for k in range(K)] for r in range(R)])
        mt = ((1 - beta) * gt + beta * hb).astype(np.float32)
        assert np.array_equal(O.topn_mask(mt, 2, 4), h)


def _two_valued_scores(R, K, g):
    """Scores 1 and 3, two of each in every group of 4 (positions shuffled per group):
    mean 2 and population standard deviation 1 exactly, so z = +-1 exactly and the
    hard target keeps the 3s."""
    S = np.empty((R, K), np.float32)
    for r in range(R):
        for q in range(K // 4):
            S[r, 4 * q:4 * q + 4] = g.permutation([3.0, 1.0, 3.0, 1.0])
    return S


@pytest.mark.parametrize("T0,rho,temps", [
    # T_t = T0 rho^t written out by hand for each schedule
    (0.5, 0.5, [0.5, 0.25, 0.125, 0.0625, 0.03125, 0.015625, 0.0078125, 0.00390625]),
    (0.8, 0.6, [0.8, 0.48, 0.288, 0.1728, 0.10368]),
    (2.0, 0.25, [2.0, 0.5, 0.125, 0.03125]),
])
def test_gate_schedule_closed_form(T0, rho, temps):
    """Two-valued scores with z = +-1 exactly: at step t the gate of a kept score is
    expit(1/T_t) and of a dropped one expit(-1/T_t) (scipy's logistic function, not the
    oracle's), beta_t = t/(S-1), so m_t and Lmid_t follow by hand for every step.  This
    fixes the temperature's place (z/T, not z*T), the geometric schedule's exponent (t,
    not t+1), the direction of the blend and the per-element output of any step."""
    from scipy.special import expit
    g = _rng(72)
    R, K, steps = 6, 32, len(temps)
    S = _two_valued_scores(R, K, g)
    mu, sg = O.stats(S)
    assert (mu, sg) == (2.0, 1.0)
    keep = S == 3.0
    n = R * K
    for t, T in enumerate(temps):
        beta = t / (steps - 1)
        m_keep = (1 - beta) * expit(1.0 / T) + beta
        m_drop = (1 - beta) * expit(-1.0 / T)
        m, hard, lm = O.gate_anneal(S, mu, sg, 2, 4, T0, rho, steps, m_step=t)
        want = np.where(keep, m_keep, m_drop).astype(np.float32)
        assert np.array_equal(m, want), f"step {t}"
        assert lm[t] == pytest.approx(n / 2 * (m_keep * (1 - m_keep) + m_drop * (1 - m_drop)), rel=1e-13)
        assert np.array_equal(O.mask_to_bool(hard, K), keep)   # projection keeps the 3s
        assert O.gate_value(3.0, mu, sg, T0, rho, t) == pytest.approx(expit(1.0 / T), rel=1e-14)
        assert O.gate_value(1.0, mu, sg, T0, rho, t) == pytest.approx(expit(-1.0 / T), rel=1e-14, abs=1e-300)


def test_gate_m_step_last_is_hard_target_and_default():
    """m_step = S-1 (the default) gives m_{S-1} = h; an earlier step is strictly between."""
    g = _rng(73)
    S = _two_valued_scores(4, 16, g)
    m_last, hard, _ = O.gate_anneal(S, 2.0, 1.0, 2, 4, 0.5, 0.5, 8)
    m7, _, _ = O.gate_anneal(S, 2.0, 1.0, 2, 4, 0.5, 0.5, 8, m_step=7)
    assert np.array_equal(m_last, m7) and np.array_equal(m_last, (S == 3.0).astype(np.float32))
    m0, _, _ = O.gate_anneal(S, 2.0, 1.0, 2, 4, 0.5, 0.5, 8, m_step=0)
    assert ((m0 > 0) & (m0 < 1)).all()


# ------------------------------------------------------------------ sparse + low-rank linear (SALR 2-3)
def _int_bf16(g, shape, lim):
    return O.f32_to_bf16(g.integers(-lim, lim + 1, shape).astype(np.float32))


def test_lowrank_u_matches_numpy():
    g = _rng(51)
    X, A = _int_bf16(g, (7, 40), 9), _int_bf16(g, (5, 40), 9)
    U = O.lowrank_u(X, A)
    assert np.array_equal(U, O.bf16_to_f32(X).astype(np.int64) @ O.bf16_to_f32(A).astype(np.int64).T)


def test_sparse_lowrank_reduces_to_masked_product_and_to_adapter():
    """A = 0 leaves the structured-sparse product; an empty mask leaves the adapter
    product u B^T, with u held in bf16 (integers up to 256 are exact there)."""
    g = _rng(52)
    Mt, R, K, r = 6, 9, 32, 4
    X, W = _int_bf16(g, (Mt, K), 3), _int_bf16(g, (R, K), 5)
    A, B = _int_bf16(g, (r, K), 2), _int_bf16(g, (R, r), 7)
    mask = O.topn_mask(O.score(W, None, 0.0, O.SCORE_MAGNITUDE) + g.random((R, K)).astype(np.float32), 2, 4)
    zeroA = np.zeros_like(A)
    assert np.array_equal(O.sparse_lowrank(X, W, mask, zeroA, B), O.masked_matmul(X, W, mask))
    empty = np.zeros_like(mask)
    Xi, Ai, Bi = (O.bf16_to_f32(t).astype(np.int64) for t in (X, A, B))
    u = Xi @ Ai.T
    assert np.abs(u).max() <= 256
    assert np.array_equal(O.sparse_lowrank(X, W, empty, A, B), (u @ Bi.T).astype(np.float64))


def test_sparse_lowrank_rounds_the_adapter_intermediate_to_bf16():
    """u = 257 is not a bf16 value: it rounds to 256 (tie to even) and 259 to 260."""
    K = 2
    X = O.f32_to_bf16(np.array([[1.0, 1.0], [1.0, 3.0]], np.float32))
    A = O.f32_to_bf16(np.array([[1.0, 256.0]], np.float32))          # u = 257, 769
    B = O.f32_to_bf16(np.array([[1.0]], np.float32))
    W = np.zeros((1, K), np.uint16)
    Y = O.sparse_lowrank(X, W, None, A, B)
    assert Y[0, 0] == 256.0 and Y[1, 0] == 768.0                       # 769 -> 768 (ulp 4, nearest)
    A2 = O.f32_to_bf16(np.array([[3.0, 256.0]], np.float32))         # u = 259 -> 260
    assert O.sparse_lowrank(X[:1], W, None, A2, B)[0, 0] == 260.0


def test_sparse_lowrank_full_rank_residual_restores_dense_product():
    """SALR section 2: the adapter carries the pruning residual E = W - mask*W.  At full
    rank (A = I, B = E) the layer computes the dense product X W^T exactly."""
    g = _rng(53)
    Mt, R, K = 5, 8, 16
    X, W = _int_bf16(g, (Mt, K), 4), _int_bf16(g, (R, K), 6)
    mask = O.topn_mask(O.score(W, None, 0.0, O.SCORE_MAGNITUDE) + g.random((R, K)).astype(np.float32), 2, 4)
    keep = O.mask_to_bool(mask, K)
    E = np.where(keep, 0, O.bf16_to_f32(W)).astype(np.float32)
    A = O.f32_to_bf16(np.eye(K, dtype=np.float32))
    Y = O.sparse_lowrank(X, W, mask, A, O.f32_to_bf16(E))
    dense = O.bf16_to_f32(X).astype(np.float64) @ O.bf16_to_f32(W).astype(np.float64).T
    assert np.array_equal(Y, dense)


def test_sparse_lowrank_concatenation_equals_separate_adapters():
    """SALR section 3: stacking two adapters along the rank gives the same layer output as
    applying them one after the other."""
    g = _rng(54)
    Mt, R, K = 6, 10, 24
    X, W = _int_bf16(g, (Mt, K), 3), _int_bf16(g, (R, K), 4)
    mask = O.topn_mask(O.score(W, None, 0.0, O.SCORE_MAGNITUDE) + g.random((R, K)).astype(np.float32), 2, 4)
    A1, B1 = _int_bf16(g, (3, K), 2), _int_bf16(g, (R, 3), 3)
    A2, B2 = _int_bf16(g, (5, K), 2), _int_bf16(g, (R, 5), 3)
    Ycat = O.sparse_lowrank(X, W, mask, np.concatenate([A1, A2]), np.concatenate([B1, B2], axis=1))
    base = O.masked_matmul(X, W, mask)
    assert np.array_equal(Ycat, O.sparse_lowrank(X, W, mask, A1, B1) + O.sparse_lowrank(X, W, mask, A2, B2) - base)


# ------------------------------------------------------------------ bitmap format (SALR 4)
def _unstructured_mask(W, density, g):
    """Magnitude mask keeping the given fraction of the whole tensor (ties broken at random)."""
    a = np.abs(O.bf16_to_f32(W)) + g.random(W.shape).astype(np.float32) * 1e-6
    thr = np.quantile(a, 1.0 - density)
    return O.bool_to_mask(a > thr)


def test_bitmap_encode_matches_numpy_selection():
    g = _rng(61)
    R, K = 9, 200                                     # K off the 64-column grid
    W = O.f32_to_bf16(g.standard_normal((R, K)).astype(np.float32))
    mask = _unstructured_mask(W, 0.5, g)
    keep = O.mask_to_bool(mask, K)
    vals, offs = O.bitmap_encode(W, mask)
    for r in range(R):
        sel = W[r][keep[r]]
        assert np.array_equal(vals[r, :sel.size], sel) and not vals[r, sel.size:].any()
        before = np.concatenate([[0], np.cumsum(keep[r])])
        assert np.array_equal(offs[r], before[np.minimum(np.arange(0, K + 64, 64), K)][: offs.shape[1]])
    assert np.array_equal(offs[:, -1], keep.sum(axis=1))


def test_bitmap_round_trip_and_product():
    g = _rng(62)
    R, K, Mt = 12, 256, 5
    W = O.f32_to_bf16(g.standard_normal((R, K)).astype(np.float32))
    X = O.f32_to_bf16(g.standard_normal((Mt, K)).astype(np.float32))
    for density in (0.5, 0.75, 0.3):
        mask = _unstructured_mask(W, density, g)
        vals, _ = O.bitmap_encode(W, mask)
        Wd = O.bitmap_decode(vals, mask, K)
        assert np.array_equal(Wd, np.where(O.mask_to_bool(mask, K), W, 0).astype(np.uint16))
        assert np.array_equal(O.masked_matmul(X, Wd, None), O.masked_matmul(X, W, mask))


def test_bitmap_of_a_24_mask_holds_the_24_packed_values():
    """For a 2:4 mask the compact values are exactly the 2:4 packed values (SALR's bitmap
    and the 2-bit index format carry the same information)."""
    g = _rng(63)
    R, K = 7, 128
    W = O.f32_to_bf16(g.standard_normal((R, K)).astype(np.float32))
    mask = O.topn_mask(O.score(W, None, 0.0, O.SCORE_MAGNITUDE), 2, 4)
    vals, offs = O.bitmap_encode(W, mask, ldv=K // 2)
    pvals, _ = O.pack(W, mask, 2, 4)
    assert np.array_equal(vals, pvals)
    assert (offs == np.arange(0, K // 64 + 1) * 32).all()


def test_bitmap_rows_beyond_capacity_drop_their_last_values():
    g = _rng(64)
    R, K, cap = 4, 64, 20
    W = O.f32_to_bf16(g.standard_normal((R, K)).astype(np.float32))
    keep = np.zeros((R, K), bool)
    keep[:, :30] = True                               # 30 kept per row, 20 stored
    mask = O.bool_to_mask(keep)
    vals, offs = O.bitmap_encode(W, mask, ldv=cap)
    assert (offs[:, -1] == 30).all()
    Wd = O.bitmap_decode(vals, mask, K)
    assert np.array_equal(Wd[:, :cap], W[:, :cap]) and not Wd[:, cap:].any()
