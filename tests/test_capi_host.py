"""Host-side checks of the C ABI: the library loads, exports every entry point
the header declares, and rejects bad arguments before touching the GPU (the
validation paths below return before any HIP call)."""
import ctypes
import re
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "nmsparse.h"


def declared_symbols():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nm_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def nm():
    import semi_structured_sparsity_amd as m
    return m


def test_library_exports_every_declared_symbol(nm):
    syms = declared_symbols()
    assert len(syms) >= 18
    for s in syms:
        assert hasattr(nm.raw, s), f"libnmsparse.so does not export {s}"
        assert s in nm.SIGNATURES, f"binding has no signature for {s}"
    assert nm.nm_abi_version() == 2


def test_binding_functions_have_c_names(nm):
    for s in declared_symbols():
        if s.endswith("_workspace") or s in ("nm_last_error",):
            continue
        assert callable(getattr(nm, s)), f"no Python wrapper named {s}"


def _st(nm, code):
    return nm.STATUS_NAMES[code]


def test_validation_errors_without_gpu(nm):
    r = nm.raw
    S = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first
    # unsupported N:M
    assert _st(nm, r.nm_mask(S, 4, 8, 8, 4, 6, S, 1, None)) == "NM_ERR_PATTERN"
    assert _st(nm, r.nm_mask(S, 4, 8, 8, 4, 4, S, 1, None)) == "NM_ERR_PATTERN"
    assert "M must be 4 or 8" in nm.last_error() or "N < M" in nm.last_error()
    # K not a multiple of M
    assert _st(nm, r.nm_mask(S, 4, 10, 10, 2, 4, S, 2, None)) == "NM_ERR_SHAPE"
    # NULL pointers
    assert _st(nm, r.nm_mask(None, 4, 8, 8, 2, 4, S, 1, None)) == "NM_ERR_NULL"
    # slide N out of range and K not a multiple of 2N
    assert _st(nm, r.nm_slide_decompose(S, 1, 4, 16, 16, S, 2, 9, 1, S, 8, S, 1, 0, None)) == "NM_ERR_PATTERN"
    assert _st(nm, r.nm_slide_decompose(S, 1, 4, 12, 12, S, 2, 4, 1, S, 8, S, 1, 0, None)) == "NM_ERR_SHAPE"
    # flags other than NM_FLAG_VALIDATE are rejected before anything runs
    assert _st(nm, r.nm_slide_decompose(S, 1, 4, 16, 16, S, 2, 4, 1, S, 12, S, 1, 2, None)) == "NM_ERR_SHAPE"
    assert "unknown flags" in nm.last_error()
    # sparse GEMM: unsupported slide N, bad dtype pairing, K multiple, int32 overflow bound
    Y = ctypes.c_void_p(0x100000)
    for bad_ns in (1, 2, 9):
        assert _st(nm, r.nm_spmm(S, 1, 4, 72, 72, S, 1, S, 8, 36, 4, bad_ns, None, 1.0, Y, 1, 8, None, 0,
                                 None)) == "NM_ERR_PATTERN"
    # (2N-2):2N for N = 3: K a multiple of 6, lifted width 4K/3 a multiple of 16 (bf16) / 32 (int8)
    assert _st(nm, r.nm_spmm(S, 1, 4, 64, 64, S, 1, S, 8, 64, 4, 3, None, 1.0, Y, 1, 8, None, 0, None)) == "NM_ERR_SHAPE"
    assert _st(nm, r.nm_spmm(S, 1, 4, 18, 24, S, 1, S, 8, 16, 4, 3, None, 1.0, Y, 1, 8, None, 0, None)) == "NM_ERR_SHAPE"
    assert _st(nm, r.nm_spmm(S, 2, 4, 36, 48, S, 2, S, 8, 24, 4, 3, None, 1.0, Y, 3, 8, None, 0, None)) == "NM_ERR_SHAPE"
    assert _st(nm, r.nm_spmm(S, 1, 4, 64, 64, S, 2, S, 8, 32, 4, 0, None, 1.0, Y, 1, 8, None, 0, None)) == "NM_ERR_DTYPE"
    assert _st(nm, r.nm_spmm(S, 2, 4, 64, 64, S, 2, S, 8, 32, 4, 0, None, 1.0, Y, 2, 8, None, 0, None)) == "NM_ERR_DTYPE"
    assert _st(nm, r.nm_spmm(S, 1, 4, 40, 40, S, 1, S, 8, 20, 4, 0, None, 1.0, Y, 1, 8, None, 0, None)) == "NM_ERR_SHAPE"
    big = 1 << 20
    assert _st(nm, r.nm_spmm(S, 2, 4, big, big, S, 2, S, 8, big, big, 0, None, 1.0, Y, 3, 8, None, 0, None)) == "NM_ERR_SHAPE"
    # 6:8 over K = 96: lifted width 144 -> 4.5 index words per row, so ldi = 4 is too small
    assert _st(nm, r.nm_spmm(S, 1, 4, 96, 96, S, 1, S, 8, 72, 4, 4, None, 1.0, Y, 1, 8, None, 0, None)) == "NM_ERR_SHAPE"
    # misaligned activation pointer
    assert _st(nm, r.nm_spmm(ctypes.c_void_p(0x1002), 1, 4, 64, 64, S, 1, S, 8, 32, 4, 0, None, 1.0, Y, 1, 8, None, 0,
                             None)) == "NM_ERR_ALIGN"
    # output aliasing an input
    assert _st(nm, r.nm_spmm(S, 1, 4, 64, 64, ctypes.c_void_p(0x8000), 1, ctypes.c_void_p(0x9000), 8, 32, 4, 0, None,
                             1.0, S, 1, 8, None, 0, None)) == "NM_ERR_ALIAS"
    # workspace missing
    assert _st(nm, r.nm_score_stats(S, 4, 8, 8, Y, None, 0, None)) == "NM_ERR_WORKSPACE"
    # gate: steps out of range, T0 not positive
    assert _st(nm, r.nm_gate(S, 4, 8, 8, S, 2, 4, 0.5, 0.5, 0, 0, S, 8, Y, 1, S, S, 1 << 20, None)) == "NM_ERR_SHAPE"
    assert _st(nm, r.nm_gate(S, 4, 8, 8, S, 2, 4, -1.0, 0.5, 8, 7, S, 8, Y, 1, S, S, 1 << 20, None)) == "NM_ERR_SHAPE"
    # the step whose blend is written must be one of the steps
    M_ = ctypes.c_void_p(0x200000)
    for bad_t in (-1, 8):
        assert _st(nm, r.nm_gate(S, 4, 8, 8, S, 2, 4, 0.5, 0.5, 8, bad_t, M_, 8, Y, 1, S, S, 1 << 20,
                                 None)) == "NM_ERR_SHAPE"
        assert "m_step" in nm.last_error()
    # gate + pack: the gate's rules, the pack's dtype rule, and no output over an input
    P_ = lambda a: ctypes.c_void_p(a)
    def gp(steps=8, W=P_(0x6000), vdt=1, vals=P_(0x7000)):
        return _st(nm, r.nm_gate_pack(S, 4, 8, 8, P_(0x3000), 2, 4, 0.5, 0.5, steps, 7, None, 8, P_(0x5000), 1,
                                      P_(0x4000), W, 1, 8, vdt, vals, 4, P_(0x8000), 1, P_(0x100000), 1 << 20, None))
    assert gp(steps=0) == "NM_ERR_SHAPE"
    assert gp(W=None) == "NM_ERR_NULL"
    assert gp(vdt=2) == "NM_ERR_DTYPE"
    assert gp(vals=P_(0x1040)) == "NM_ERR_ALIAS"
    # Hutchinson alignment rules
    assert _st(nm, r.nm_hdiag_hutchinson(S, 64, 100, 100, 8, 2, 1, Y, 100, S, 1 << 30, None)) == "NM_ERR_ALIGN"
    # pack dtype rule (bf16 weights cannot pack to int8)
    assert _st(nm, r.nm_pack(S, 1, 4, 8, 8, S, 1, 2, 4, 2, Y, 4, S, 1, 0, None)) == "NM_ERR_DTYPE"
    assert _st(nm, r.nm_pack(S, 1, 4, 8, 8, S, 1, 2, 4, 1, Y, 4, S, 1, 0x10, None)) == "NM_ERR_SHAPE"
    # FP8: only FP8 x FP8 -> f32/bf16 products, one-byte K multiples, codes from bf16 only, no FP8 absmean
    F8 = nm.NM_FP8
    assert _st(nm, r.nm_spmm(S, F8, 4, 64, 64, S, 2, S, 8, 32, 4, 0, None, 1.0, Y, 0, 8, None, 0, None)) == "NM_ERR_DTYPE"
    assert _st(nm, r.nm_spmm(S, F8, 4, 64, 64, S, F8, S, 8, 32, 4, 0, None, 1.0, Y, 3, 8, None, 0, None)) == "NM_ERR_DTYPE"
    assert _st(nm, r.nm_spmm(S, F8, 4, 48, 48, S, F8, S, 8, 24, 4, 0, None, 1.0, Y, 0, 8, None, 0, None)) == "NM_ERR_SHAPE"
    assert _st(nm, r.nm_spmm(S, F8, 4, 96, 96, S, F8, S, 8, 72, 8, 4, None, 1.0, Y, 0, 8, None, 0, None)) == "NM_ERR_SHAPE"
    assert _st(nm, r.nm_quant_lift(S, 1, 4, 64, 64, 4, 0, Y, 96, S, None)) == "NM_ERR_DTYPE"
    assert _st(nm, r.nm_quant_lift(S, 1, 4, 64, 64, 2, 2, Y, 96, S, None)) == "NM_ERR_PATTERN"
    assert _st(nm, r.nm_quant_lift(S, 1, 4, 64, 64, 3, 2, Y, 96, S, None)) == "NM_ERR_SHAPE"   # 64 % 6
    assert _st(nm, r.nm_quant_lift(S, F8, 4, 64, 64, 4, F8, Y, 96, S, None)) == "NM_ERR_DTYPE"
    assert _st(nm, r.nm_absmean(S, F8, 4, 8, 8, Y, S, 1 << 20, None)) == "NM_ERR_DTYPE"
    # sparse + low-rank: rank a multiple of 8 in [8, 256], bf16/f32 output, aligned A and B, enough workspace
    lr = r.nm_spmm_lowrank
    assert _st(nm, lr(S, 4, 64, 64, S, S, 8, 32, 4, 0, S, 64, S, 16, 12, Y, 1, 8, S, 1 << 30, None)) == "NM_ERR_SHAPE"
    assert _st(nm, lr(S, 4, 64, 64, S, S, 8, 32, 4, 0, S, 64, S, 512, 512, Y, 1, 8, S, 1 << 30, None)) == "NM_ERR_SHAPE"
    assert _st(nm, lr(S, 4, 64, 64, S, S, 8, 32, 4, 0, S, 64, S, 16, 16, Y, 3, 8, S, 1 << 30, None)) == "NM_ERR_DTYPE"
    assert _st(nm, lr(S, 4, 64, 64, S, S, 8, 32, 4, 0, ctypes.c_void_p(0x1008), 64, S, 16, 16, Y, 1, 8, S, 1 << 30,
                      None)) == "NM_ERR_ALIGN"
    assert _st(nm, lr(S, 4, 64, 64, S, S, 8, 32, 4, 0, S, 64, S, 16, 16, Y, 1, 8, S, 16, None)) == "NM_ERR_WORKSPACE"
    assert _st(nm, lr(S, 4, 64, 64, S, S, 8, 32, 4, 0, S, 64, S, 16, 16, Y, 1, 8, ctypes.c_void_p(0x40000008), 1 << 30,
                      None)) == "NM_ERR_ALIGN"
    # a product that needs a workspace (few tokens: K split over blocks) takes it 16-byte aligned
    need = r.nm_spmm_workspace(4, 4096, 256, 0, nm.NM_BF16)
    assert need > 0
    assert _st(nm, r.nm_spmm(S, 1, 4, 4096, 4096, ctypes.c_void_p(0x10000000), 1, ctypes.c_void_p(0x20000000), 256,
                             2048, 128, 0, None, 1.0, ctypes.c_void_p(0x30000000), 1, 256, ctypes.c_void_p(0x40000008),
                             need, None)) == "NM_ERR_ALIGN"
    # bitmap format: K a multiple of 64, bf16 weights, 8-byte aligned mask rows
    assert _st(nm, r.nm_bitmap_encode(S, 1, 4, 96, 96, S, 12, Y, 96, S, 3, None)) == "NM_ERR_SHAPE"
    assert _st(nm, r.nm_bitmap_encode(S, 0, 4, 64, 64, S, 8, Y, 64, S, 2, None)) == "NM_ERR_DTYPE"
    assert _st(nm, r.nm_bitmap_encode(S, 1, 4, 64, 64, ctypes.c_void_p(0x1004), 8, Y, 64, S, 2, None)) == "NM_ERR_ALIGN"
    assert _st(nm, r.nm_spmm_bitmap(S, 4, 64, 64, S, 64, S, 8, S, 1, 8, Y, 1, 8, None, 0, None)) == "NM_ERR_SHAPE"
    assert _st(nm, r.nm_spmm_bitmap(S, 4, 64, 64, S, 64, S, 8, S, 2, 8, Y, 3, 8, None, 0, None)) == "NM_ERR_DTYPE"
    # up to 4 tokens the bitmap product streams rows and needs no workspace; more tokens on
    # few rows split K over blocks (f32 partials)
    assert all(r.nm_spmm_bitmap_workspace(m, 4096, 14336) == 0 for m in (1, 2, 3, 4))
    assert r.nm_spmm_bitmap_workspace(8, 4096, 512) > 0


def test_empty_inputs_are_noops(nm):
    r = nm.raw
    assert r.nm_mask(None, 0, 8, 8, 2, 4, None, 1, None) == 0
    assert r.nm_spmm(None, 1, 0, 64, 64, None, 1, None, 8, 32, 4, 0, None, 1.0, None, 1, 8, None, 0, None) == 0
    assert r.nm_pack(None, 1, 0, 8, 8, None, 1, 2, 4, 1, None, 4, None, 1, 0, None) == 0


def test_spmm_noalloc_rejects_beyond_scratch_without_gpu(nm):
    """The size check of the no-allocation product precedes every HIP call."""
    r = nm.raw
    S, Y = ctypes.c_void_p(0x1000), ctypes.c_void_p(1 << 40)
    Mt, R, K = 8192, 256, 4096
    assert r.nm_spmm_workspace(Mt, K, R, 4, nm.NM_BF16) > nm.NM_SPMM_SCRATCH_BYTES
    st = r.nm_spmm_noalloc(S, 1, Mt, K, K, ctypes.c_void_p(1 << 36), 1, ctypes.c_void_p(1 << 38), R, 3072, 192, 4,
                           None, 1.0, Y, 1, R, None)
    assert _st(nm, st) == "NM_ERR_WORKSPACE" and "scratch" in nm.last_error()


def test_spmm_workspace_covers_every_plan(nm):
    """The workspace query does not know the index pointer or ldi, which decide whether the
    DMA ring kernels may run; it must cover the fallback plan too.  One token on the
    11008 x 4096 layer: the ring plan needs no workspace, the fallback (an index view
    that is only 4-byte aligned) splits K over two blocks and needs their f32 partials."""
    r = nm.raw
    need = r.nm_spmm_workspace(1, 4096, 11008, 0, nm.NM_BF16)
    assert need >= 2 * 1 * 11008 * 4
    # every plan of the lifted product includes the lifted activation
    assert r.nm_spmm_workspace(16, 4096, 14336, 4, nm.NM_BF16) >= 16 * 6144 * 2
    assert r.nm_spmm_workspace(16, 3072, 1024, 3, nm.NM_I8) >= 16 * 4096


def test_device_error_without_gpu(nm):
    """With no GPU, a call that passes validation reports NM_ERR_DEVICE from its launch (with
    the runtime's message), rather than failing silently.  Skipped where a GPU is visible:
    the call's pointers are fake."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible; this check launches on placeholder pointers")
    r = nm.raw
    S, mask = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x100000)
    assert _st(nm, r.nm_mask(S, 4, 8, 8, 2, 4, mask, 1, None)) == "NM_ERR_DEVICE"
    assert "nm_mask" in nm.last_error()
