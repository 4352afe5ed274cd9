"""Per-token int8 quantisation fused with the 6:8 lift (SlideSparse 2B/2C online step),
through the C ABI, against the oracle: codes and scales bit for bit, then the whole int8
online path (quantise + lift, then the sparse product over the lifted width) exactly."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests._util import dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nm():
    import semi_structured_sparsity_amd as m
    return m


def _x(g, Mt, K):
    a = g.uniform(0.5, 2.0, (Mt, 1))
    X = O.f32_to_bf16((a * g.uniform(-1, 1, (Mt, K))).astype(np.float32))
    if Mt > 2:
        X[1] = 0                                   # zero row: scale 0, codes 0
        X[2] = 0
        X[2, K // 2] = O.f32_to_bf16(np.array([-3.0], np.float32))[0]   # a single nonzero
    return X


@pytest.mark.parametrize("Mt,K", [(1, 64), (5, 8), (37, 2560), (300, 4096), (257, 1032), (2, 4104)])
@pytest.mark.parametrize("Ns", [0, 4])
def test_quant_lift_bit_exact(nm, Mt, K, Ns):
    _quant_case(nm, Mt, K, Ns)


# other (2N-2):2N lifts: K a multiple of 8 and of 2N
@pytest.mark.parametrize("Ns,Mt,K", [(3, 1, 48), (3, 37, 2568), (5, 9, 640), (5, 300, 4000), (6, 4, 1152),
                                     (7, 3, 56), (8, 65, 4096)])
@pytest.mark.parametrize("fp8", [False, True])
def test_quant_lift_general_n_bit_exact(nm, Ns, Mt, K, fp8):
    _quant_case(nm, Mt, K, Ns, fp8)


def _quant_case(nm, Mt, K, Ns, fp8=False):
    g = np.random.default_rng(Mt * 31 + K + Ns)
    X = _x(g, Mt, K)
    Xq, sx = nm.nm_quant_lift(torch.from_numpy(X.view(np.int16)).view(torch.bfloat16).to(dev()), Ns,
                              nm.NM_FP8 if fp8 else nm.NM_I8)
    q_ref, s_ref = O.quant_lift(X, Ns, fp8=fp8)
    assert np.array_equal(sx.cpu().numpy(), s_ref)
    got = Xq.cpu().view(torch.uint8).numpy() if fp8 else Xq.cpu().numpy()
    assert np.array_equal(got, q_ref)


def test_quant_lift_strided_input(nm):
    g = np.random.default_rng(7)
    Mt, K = 9, 256
    X = _x(g, Mt, K)
    big = torch.zeros((Mt, K + 40), dtype=torch.bfloat16)
    big[:, :K] = torch.from_numpy(X.view(np.int16)).view(torch.bfloat16)
    Xq, sx = nm.nm_quant_lift(big.to(dev())[:, :K], 4)
    q_ref, s_ref = O.quant_lift(X, 4)
    assert np.array_equal(Xq.cpu().numpy(), q_ref) and np.array_equal(sx.cpu().numpy(), s_ref)


@pytest.mark.parametrize("Mt,R,K", [(1, 70, 2560), (200, 300, 512), (300, 64, 2560)])
def test_online_int8_slide_path_exact(nm, Mt, R, K):
    """bf16 X -> quantise + lift -> int8 sparse product over K' with the slide-packed ternary
    weight, against the oracle's masked product of the unlifted codes."""
    g = np.random.default_rng(Mt + R + K)
    Wf, Wt = synth.ternary68_weights(R=R, K=K)
    mask = O.topn_mask(O.score(host(Wf), None, 0.0, O.SCORE_MAGNITUDE), 6, 8)
    vals, idx, bad = O.slide_decompose(Wt.numpy(), mask, 4)
    assert bad == 0
    alpha = float(np.float32(O.absmean(host(Wf))))
    X = _x(g, Mt, K)
    Xd = torch.from_numpy(X.view(np.int16)).view(torch.bfloat16).to(dev())
    XL, sx = nm.nm_quant_lift(Xd, 4)
    v, i = torch.from_numpy(vals).to(dev()), torch.from_numpy(idx.view(np.int32)).to(dev())
    Kl = O.lifted_width(K, 4)
    acc = nm.nm_spmm(XL, v, i, R=R, Ns=0, ydt=nm.NM_I32).cpu().numpy()
    y = nm.nm_spmm(XL, v, i, R=R, Ns=0, x_scale=sx, w_scale=alpha, ydt=nm.NM_F32).cpu().numpy()
    Xq, s_ref = O.quant_i8(X)
    acc_ref, y_ref = O.masked_matmul_i8(Xq, Wt.numpy(), mask, s_ref, alpha)
    assert XL.shape[1] == Kl
    assert np.array_equal(acc, acc_ref)
    assert np.array_equal(y, y_ref)
