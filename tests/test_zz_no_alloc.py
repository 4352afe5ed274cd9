"""The no-allocation variant of the sparse product (nm_spmm_noalloc), through the C ABI:
its workspace is the library's static per-device scratch buffer.  Its outputs must equal
nm_spmm's (same kernels, same plan) bit for bit, on consecutive calls that reuse the buffer
with a smaller second input, and match the oracle exactly on integer-valued inputs."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests._util import dev, host, np_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nm():
    import semi_structured_sparsity_amd as m
    return m


def _int_bf16(g, shape, lim):
    return O.f32_to_bf16(g.integers(-lim, lim + 1, shape).astype(np.float32))


def _bf16_case(g, Mt, R, K, Ns):
    X, W = _int_bf16(g, (Mt, K), 2), _int_bf16(g, (R, K), 2)
    S = O.score(W, None, 0.0, O.SCORE_MAGNITUDE) + g.random((R, K)).astype(np.float32)
    if Ns:
        mask = O.topn_mask(S, 2 * Ns - 2, 2 * Ns)
        vals, idx, bad = O.slide_decompose(W, mask, Ns)
        assert bad == 0
    else:
        mask = O.topn_mask(S, 2, 4)
        vals, idx = O.pack(W, mask, 2, 4)
    return (np_bf16(X).to(dev()), np_bf16(vals).to(dev()), torch.from_numpy(idx.view(np.int32)).to(dev()),
            O.masked_matmul(X, W, mask))


def _raw_noalloc(nm, X, vals, idx, R, Ns, Y, ydt, xs=None, a=1.0):
    Mt, K = X.shape
    st = nm.raw.nm_spmm_noalloc(X.data_ptr(), nm.dtype_code(X), Mt, K, X.stride(0), vals.data_ptr(),
                                nm.dtype_code(vals), idx.data_ptr(), R, vals.stride(0), idx.stride(0), Ns,
                                None if xs is None else xs.data_ptr(), a, Y.data_ptr(), ydt, Y.stride(0),
                                torch.cuda.current_stream().cuda_stream)
    assert st == 0, nm.last_error()


def test_noalloc_equals_spmm_on_consecutive_calls(nm):
    g = np.random.default_rng(12)
    # first call: a lifted 6:8 product (the lifted activation lives in the scratch buffer)
    cases = [(64, 1024, 4096, 4), (1, 4096, 4096, 0), (3, 300, 384, 3)]   # then smaller ones reusing it
    for Mt, R, K, Ns in cases:
        assert nm.raw.nm_spmm_workspace(Mt, K, R, Ns, nm.NM_BF16) > 0
        X, v, i, ref = _bf16_case(g, Mt, R, K, Ns)
        Y = torch.full((Mt, R), -1.0, dtype=torch.float32, device=dev())
        _raw_noalloc(nm, X, v, i, R, Ns, Y, nm.NM_F32)
        Yw = nm.nm_spmm(X, v, i, R=R, Ns=Ns, ydt=nm.NM_F32)
        torch.cuda.synchronize()
        assert torch.equal(Y, Yw), (Mt, R, K, Ns)
        assert np.array_equal(Y.cpu().numpy().astype(np.float64), ref), (Mt, R, K, Ns)


def test_noalloc_int8_scaled_then_smaller(nm):
    g = np.random.default_rng(13)
    for Mt, R, K in [(256, 6912, 2560), (1, 700, 2560)]:
        Wf, Wt = synth.ternary68_weights(R=R, K=K)
        mask = O.topn_mask(O.score(host(Wf), None, 0.0, O.SCORE_MAGNITUDE), 6, 8)
        vals, idx, _ = O.slide_decompose(Wt.numpy(), mask, 4)
        v, i = torch.from_numpy(vals).to(dev()), torch.from_numpy(idx.view(np.int32)).to(dev())
        Xq = torch.from_numpy(g.integers(-127, 128, (Mt, K)).astype(np.int8)).to(dev())
        sx = torch.from_numpy((g.uniform(0.5, 2.0, Mt) / 127).astype(np.float32)).to(dev())
        Y = torch.empty((Mt, R), dtype=torch.float32, device=dev())
        _raw_noalloc(nm, Xq, v, i, R, 4, Y, nm.NM_F32, xs=sx, a=0.8)
        Yw = nm.nm_spmm(Xq, v, i, R=R, Ns=4, x_scale=sx, w_scale=0.8, ydt=nm.NM_F32)
        acc = torch.empty((Mt, R), dtype=torch.int32, device=dev())
        _raw_noalloc(nm, Xq, v, i, R, 4, acc, nm.NM_I32)
        torch.cuda.synchronize()
        assert torch.equal(Y, Yw)
        acc_ref, y_ref = O.masked_matmul_i8(Xq.cpu().numpy(), Wt.numpy(), mask, sx.cpu().numpy(), 0.8)
        assert np.array_equal(acc.cpu().numpy(), acc_ref) and np.array_equal(Y.cpu().numpy(), y_ref)


def test_noalloc_rejects_a_product_beyond_the_scratch(nm):
    """8192 tokens of a lifted 6:8 bf16 layer need ~100 MB of lifted activation."""
    Mt, R, K = 8192, 256, 4096
    assert nm.raw.nm_spmm_workspace(Mt, K, R, 4, nm.NM_BF16) > nm.NM_SPMM_SCRATCH_BYTES
    X = torch.zeros((Mt, K), dtype=torch.bfloat16, device=dev())
    v = torch.zeros((R, K // 8 * 12 // 2), dtype=torch.bfloat16, device=dev())
    i = torch.zeros((R, K // 8 * 12 // 32), dtype=torch.int32, device=dev())
    Y = torch.full((Mt, R), 3.0, dtype=torch.bfloat16, device=dev())
    with pytest.raises(nm.NMError) as e:
        nm.nm_spmm_noalloc(X, v, i, R=R, Ns=4, out=Y)
    assert e.value.status == nm.NM_ERR_WORKSPACE and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert (Y == 3.0).all()
