"""ctypes binding of libnmsparse (the C ABI in include/nmsparse.h).

Argument marshalling only: torch tensors supply device memory and the current
HIP stream; every step runs in the library's HIP kernels.  There is no CPU
fallback -- importing this module without the built library raises.

Each C entry point is exposed twice:
  * ``raw.<name>`` -- the ctypes function with the exact C signature;
  * ``<name>(...)``  -- a wrapper with the same name that takes tensors,
    allocates outputs with ``torch.empty`` on the input's device, passes
    pointers, and raises ``NMError`` with the library's message on failure.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

import torch

_PKG = Path(__file__).resolve().parent
LIB_PATH = _PKG / "libnmsparse.so"

NM_OK, NM_ERR_NULL, NM_ERR_SHAPE, NM_ERR_PATTERN, NM_ERR_DTYPE, NM_ERR_ALIGN, NM_ERR_WORKSPACE, NM_ERR_DEVICE, NM_ERR_ALIAS = range(9)
STATUS_NAMES = ["NM_OK", "NM_ERR_NULL", "NM_ERR_SHAPE", "NM_ERR_PATTERN", "NM_ERR_DTYPE", "NM_ERR_ALIGN",
                "NM_ERR_WORKSPACE", "NM_ERR_DEVICE", "NM_ERR_ALIAS"]
NM_F32, NM_BF16, NM_I8, NM_I32, NM_FP8 = 0, 1, 2, 3, 4
NM_SCORE_HESSIAN, NM_SCORE_MAGNITUDE = 0, 1
NM_FLAG_VALIDATE = 1

# NM_FP8 travels as torch.float8_e4m3fn (OCP e4m3 codes, one byte each)
_DT = {torch.float32: NM_F32, torch.bfloat16: NM_BF16, torch.int8: NM_I8, torch.int32: NM_I32,
       torch.float8_e4m3fn: NM_FP8}
_TORCH = {v: k for k, v in _DT.items()}


class NMError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES[status] if 0 <= status < len(STATUS_NAMES) else status}: {msg}")
        self.status = status


if not LIB_PATH.exists():
    raise ImportError(f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
                      "(or semi_structured_sparsity_amd/build.py) first")

raw = ctypes.CDLL(str(LIB_PATH))

_P, _I64, _I, _F, _U64, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_uint64, ctypes.c_size_t
_U = ctypes.c_uint

SIGNATURES = {
    "nm_abi_version": (_I, []),
    "nm_last_error": (ctypes.c_char_p, []),
    "nm_colsumsq_workspace": (_SZ, [_I64, _I64]),
    "nm_hdiag_colsumsq": (_I, [_P, _I, _I64, _I64, _I64, _P, _P, _SZ, _P]),
    "nm_hutchinson_workspace": (_SZ, [_I64, _I64, _I64, _I]),
    "nm_hdiag_hutchinson": (_I, [_P, _I64, _I64, _I64, _I64, _I, _U64, _P, _I64, _P, _SZ, _P]),
    "nm_hutchinson_score_workspace": (_SZ, [_I64, _I64, _I64, _I]),
    "nm_hutchinson_score": (_I, [_P, _I64, _I64, _I64, _I64, _I, _U64, _P, _I, _I64, _F, _P, _I64, _P, _P, _SZ, _P]),
    "nm_score": (_I, [_P, _I, _I64, _I64, _I64, _P, _I64, _F, _I, _P, _I64, _P]),
    "nm_stats_workspace": (_SZ, [_I64, _I64]),
    "nm_score_stats": (_I, [_P, _I64, _I64, _I64, _P, _P, _SZ, _P]),
    "nm_gate_workspace": (_SZ, [_I64, _I64, _I]),
    "nm_gate": (_I, [_P, _I64, _I64, _I64, _P, _I, _I, _F, _F, _I, _I, _P, _I64, _P, _I64, _P, _P, _SZ, _P]),
    "nm_gate_pack": (_I, [_P, _I64, _I64, _I64, _P, _I, _I, _F, _F, _I, _I, _P, _I64, _P, _I64, _P,
                          _P, _I, _I64, _I, _P, _I64, _P, _I64, _P, _SZ, _P]),
    "nm_mask": (_I, [_P, _I64, _I64, _I64, _I, _I, _P, _I64, _P]),
    "nm_pack": (_I, [_P, _I, _I64, _I64, _I64, _P, _I64, _I, _I, _I, _P, _I64, _P, _I64, _U, _P]),
    "nm_prune_pack": (_I, [_P, _I, _I64, _P, _I64, _F, _I, _P, _I, _I64, _I64, _I64, _I, _I, _P, _I64, _I, _P, _I64,
                           _P, _I64, _P]),
    "nm_slide_decompose": (_I, [_P, _I, _I64, _I64, _I64, _P, _I64, _I, _I, _P, _I64, _P, _I64, _U, _P]),
    "nm_prune_slide": (_I, [_P, _I, _I64, _P, _I64, _F, _I, _P, _I, _I64, _I64, _I64, _I, _P, _I64, _I, _P, _I64, _P,
                            _I64, _P]),
    "nm_absmean": (_I, [_P, _I, _I64, _I64, _I64, _P, _P, _SZ, _P]),
    "nm_quant_lift": (_I, [_P, _I, _I64, _I64, _I64, _I, _I, _P, _I64, _P, _P]),
    "nm_spmm_workspace": (_SZ, [_I64, _I64, _I64, _I, _I]),
    "nm_spmm": (_I, [_P, _I, _I64, _I64, _I64, _P, _I, _P, _I64, _I64, _I64, _I, _P, _F, _P, _I, _I64, _P, _SZ, _P]),
    "nm_spmm_noalloc": (_I, [_P, _I, _I64, _I64, _I64, _P, _I, _P, _I64, _I64, _I64, _I, _P, _F, _P, _I, _I64, _P]),
    "nm_spmm_lowrank_workspace": (_SZ, [_I64, _I64, _I64, _I, _I]),
    "nm_bitmap_encode": (_I, [_P, _I, _I64, _I64, _I64, _P, _I64, _P, _I64, _P, _I64, _P]),
    "nm_spmm_bitmap_workspace": (_SZ, [_I64, _I64, _I64]),
    "nm_spmm_bitmap": (_I, [_P, _I64, _I64, _I64, _P, _I64, _P, _I64, _P, _I64, _I64, _P, _I, _I64, _P, _SZ, _P]),
    "nm_spmm_lowrank": (_I, [_P, _I64, _I64, _I64, _P, _P, _I64, _I64, _I64, _I, _P, _I64, _P, _I64, _I, _P, _I, _I64,
                             _P, _SZ, _P]),
}
for _name, (_res, _args) in SIGNATURES.items():
    _fn = getattr(raw, _name)
    _fn.restype = _res
    _fn.argtypes = _args


def last_error() -> str:
    m = raw.nm_last_error()
    return m.decode() if m else ""


def _check(st: int):
    if st != NM_OK:
        raise NMError(st, last_error())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _ld(t: torch.Tensor) -> int:
    """Leading dimension (elements) of a 2-D row-major view."""
    if t.dim() == 1:
        return t.shape[0]
    assert t.stride(1) == 1, "tensors must be row-major (unit stride along the last dimension)"
    return t.stride(0)


def _stream(t: torch.Tensor | None = None):
    dev = t.device if t is not None and t.is_cuda else None
    return torch.cuda.current_stream(dev).cuda_stream


def _ws(nbytes: int, device) -> torch.Tensor | None:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device) if nbytes else None


def dtype_code(t: torch.Tensor) -> int:
    return _DT[t.dtype]


def index_words(slots: int, M: int) -> int:
    b = (M - 1).bit_length()
    return (slots * b + 31) // 32


def lifted_width(K: int, Ns: int) -> int:
    return K // (2 * Ns) * 4 * (Ns - 1)


# ---------------------------------------------------------------- wrappers
def nm_abi_version() -> int:
    return raw.nm_abi_version()


def nm_hdiag_colsumsq(X: torch.Tensor) -> torch.Tensor:
    n, K = X.shape
    H = torch.empty(K, dtype=torch.float32, device=X.device)
    ws = _ws(raw.nm_colsumsq_workspace(n, K), X.device)
    _check(raw.nm_hdiag_colsumsq(_ptr(X), dtype_code(X), n, K, _ld(X), _ptr(H), _ptr(ws),
                                 0 if ws is None else ws.numel(), _stream(X)))
    return H


def nm_hdiag_hutchinson(X: torch.Tensor, R: int, probes: int, seed: int) -> torch.Tensor:
    n, K = X.shape
    D = torch.empty((R, K), dtype=torch.float32, device=X.device)
    ws = _ws(raw.nm_hutchinson_workspace(n, K, R, probes), X.device)
    _check(raw.nm_hdiag_hutchinson(_ptr(X), n, K, _ld(X), R, probes, seed, _ptr(D), K, _ptr(ws),
                                   0 if ws is None else ws.numel(), _stream(X)))
    return D


def nm_hutchinson_score(X: torch.Tensor, W: torch.Tensor, probes: int, seed: int, eps: float,
                        want_stats: bool = True):
    """S = (D + eps) W^2 with D the Hutchinson diagonal of ||X W^T||^2 (never stored), and
    the per-tensor (mean, std) of S: returns (S [R, K] f32, stats [2] f64 or None)."""
    n, K = X.shape
    R = W.shape[0]
    S = torch.empty((R, K), dtype=torch.float32, device=X.device)
    st = torch.empty(2, dtype=torch.float64, device=X.device) if want_stats else None
    ws = _ws(raw.nm_hutchinson_score_workspace(n, K, R, probes), X.device)
    _check(raw.nm_hutchinson_score(_ptr(X), n, K, _ld(X), R, probes, seed, _ptr(W), dtype_code(W), _ld(W), eps,
                                   _ptr(S), K, _ptr(st), _ptr(ws), 0 if ws is None else ws.numel(), _stream(X)))
    return S, st


def nm_score(W: torch.Tensor, H: torch.Tensor | None, eps: float, mode: int = NM_SCORE_HESSIAN) -> torch.Tensor:
    R, K = W.shape
    S = torch.empty((R, K), dtype=torch.float32, device=W.device)
    ldh = 0 if (H is None or H.dim() == 1) else _ld(H)
    _check(raw.nm_score(_ptr(W), dtype_code(W), R, K, _ld(W), _ptr(H), ldh, eps, mode, _ptr(S), K, _stream(W)))
    return S


def nm_score_stats(S: torch.Tensor) -> torch.Tensor:
    R, K = S.shape
    st = torch.empty(2, dtype=torch.float64, device=S.device)
    ws = _ws(raw.nm_stats_workspace(R, K), S.device)
    _check(raw.nm_score_stats(_ptr(S), R, K, _ld(S), _ptr(st), _ptr(ws), ws.numel(), _stream(S)))
    return st


def nm_gate(S: torch.Tensor, stats: torch.Tensor, N: int, M: int, T0: float, rho: float, steps: int,
            want_m: bool = True, m_step: int | None = None):
    """Returns (m_t [R, K] f32 of step m_step (default the last) or None, hard mask, lmid [steps])."""
    R, K = S.shape
    t = steps - 1 if m_step is None else m_step
    mf = torch.empty((R, K), dtype=torch.float32, device=S.device) if want_m else None
    hm = torch.empty((R, (K + 7) // 8), dtype=torch.uint8, device=S.device)
    lm = torch.empty(steps, dtype=torch.float64, device=S.device)
    ws = _ws(raw.nm_gate_workspace(R, K, steps), S.device)
    _check(raw.nm_gate(_ptr(S), R, K, _ld(S), _ptr(stats), N, M, T0, rho, steps, t, _ptr(mf), K, _ptr(hm),
                       hm.shape[1], _ptr(lm), _ptr(ws), ws.numel(), _stream(S)))
    return mf, hm, lm


def nm_gate_pack(S: torch.Tensor, stats: torch.Tensor, W: torch.Tensor, N: int, M: int, T0: float, rho: float,
                 steps: int, want_m: bool = True, m_step: int | None = None, vdt: int | None = None):
    """nm_gate and the pack of W under its hard mask in one call: returns (m_t or None,
    hard mask, lmid, vals, idx)."""
    R, K = S.shape
    t = steps - 1 if m_step is None else m_step
    vdt = dtype_code(W) if vdt is None else vdt
    mf = torch.empty((R, K), dtype=torch.float32, device=S.device) if want_m else None
    hm = torch.empty((R, (K + 7) // 8), dtype=torch.uint8, device=S.device)
    lm = torch.empty(steps, dtype=torch.float64, device=S.device)
    slots = K // M * N
    vals, idx = _pack_out(R, slots, index_words(slots, M), vdt, S.device)
    ws = _ws(raw.nm_gate_workspace(R, K, steps), S.device)
    _check(raw.nm_gate_pack(_ptr(S), R, K, _ld(S), _ptr(stats), N, M, T0, rho, steps, t, _ptr(mf), K, _ptr(hm),
                            hm.shape[1], _ptr(lm), _ptr(W), dtype_code(W), _ld(W), vdt, _ptr(vals), slots, _ptr(idx),
                            idx.shape[1], _ptr(ws), ws.numel(), _stream(S)))
    return mf, hm, lm, vals, idx


def nm_mask(S: torch.Tensor, N: int, M: int) -> torch.Tensor:
    R, K = S.shape
    mask = torch.empty((R, (K + 7) // 8), dtype=torch.uint8, device=S.device)
    _check(raw.nm_mask(_ptr(S), R, K, _ld(S), N, M, _ptr(mask), mask.shape[1], _stream(S)))
    return mask


def _pack_out(R, slots, words, vdt, device):
    vals = torch.empty((R, slots), dtype=_TORCH[vdt], device=device)
    idx = torch.empty((R, words), dtype=torch.int32, device=device)
    return vals, idx


def nm_pack(W: torch.Tensor, mask: torch.Tensor, N: int, M: int, vdt: int | None = None, flags: int = 0):
    R, K = W.shape
    vdt = dtype_code(W) if vdt is None else vdt
    slots = K // M * N
    vals, idx = _pack_out(R, slots, index_words(slots, M), vdt, W.device)
    _check(raw.nm_pack(_ptr(W), dtype_code(W), R, K, _ld(W), _ptr(mask), _ld(mask), N, M, vdt, _ptr(vals), slots,
                       _ptr(idx), idx.shape[1], flags, _stream(W)))
    return vals, idx


def nm_prune_pack(W: torch.Tensor, H: torch.Tensor | None, eps: float, mode: int, N: int, M: int,
                  Wv: torch.Tensor | None = None, vdt: int | None = None, want_mask: bool = True):
    """Fused score -> top-N -> pack.  Score from W, values from Wv (default W)."""
    R, K = W.shape
    Wv = W if Wv is None else Wv
    vdt = (NM_BF16 if Wv.dtype == torch.float32 else dtype_code(Wv)) if vdt is None else vdt
    slots = K // M * N
    vals, idx = _pack_out(R, slots, index_words(slots, M), vdt, W.device)
    mask = torch.empty((R, (K + 7) // 8), dtype=torch.uint8, device=W.device) if want_mask else None
    ldh = 0 if (H is None or H.dim() == 1) else _ld(H)
    _check(raw.nm_prune_pack(_ptr(W), dtype_code(W), _ld(W), _ptr(H), ldh, eps, mode, _ptr(Wv), dtype_code(Wv),
                             _ld(Wv), R, K, N, M, _ptr(mask), (K + 7) // 8, vdt, _ptr(vals), slots, _ptr(idx),
                             idx.shape[1], _stream(W)))
    return vals, idx, mask


def nm_slide_decompose(W: torch.Tensor, mask: torch.Tensor, Ns: int, vdt: int | None = None, flags: int = 0):
    R, K = W.shape
    vdt = dtype_code(W) if vdt is None else vdt
    Kl = lifted_width(K, Ns)
    vals, idx = _pack_out(R, Kl // 2, (Kl + 31) // 32, vdt, W.device)
    _check(raw.nm_slide_decompose(_ptr(W), dtype_code(W), R, K, _ld(W), _ptr(mask), _ld(mask), Ns, vdt, _ptr(vals),
                                  vals.shape[1], _ptr(idx), idx.shape[1], flags, _stream(W)))
    return vals, idx


def nm_prune_slide(W: torch.Tensor, H: torch.Tensor | None, eps: float, mode: int, Ns: int,
                   Wv: torch.Tensor | None = None, vdt: int | None = None, want_mask: bool = True):
    R, K = W.shape
    Wv = W if Wv is None else Wv
    vdt = dtype_code(Wv) if vdt is None else vdt
    Kl = lifted_width(K, Ns)
    vals, idx = _pack_out(R, Kl // 2, (Kl + 31) // 32, vdt, W.device)
    mask = torch.empty((R, (K + 7) // 8), dtype=torch.uint8, device=W.device) if want_mask else None
    ldh = 0 if (H is None or H.dim() == 1) else _ld(H)
    _check(raw.nm_prune_slide(_ptr(W), dtype_code(W), _ld(W), _ptr(H), ldh, eps, mode, _ptr(Wv), dtype_code(Wv),
                              _ld(Wv), R, K, Ns, _ptr(mask), (K + 7) // 8, vdt, _ptr(vals), vals.shape[1], _ptr(idx),
                              idx.shape[1], _stream(W)))
    return vals, idx, mask


def nm_absmean(W: torch.Tensor) -> torch.Tensor:
    R, K = W.shape
    a = torch.empty(1, dtype=torch.float32, device=W.device)
    ws = _ws(raw.nm_stats_workspace(R, K), W.device)
    _check(raw.nm_absmean(_ptr(W), dtype_code(W), R, K, _ld(W), _ptr(a), _ptr(ws), ws.numel(), _stream(W)))
    return a


def nm_quant_lift(X: torch.Tensor, Ns: int = 4, qdt: int = NM_I8) -> tuple[torch.Tensor, torch.Tensor]:
    """Per-token int8 or FP8 codes of bf16 X (lifted for Ns >= 3) and their scales."""
    Mtok, K = X.shape
    Kl = lifted_width(K, Ns) if Ns else K
    Xq = torch.empty((Mtok, Kl), dtype=_TORCH[qdt], device=X.device)
    sx = torch.empty(Mtok, dtype=torch.float32, device=X.device)
    _check(raw.nm_quant_lift(_ptr(X), dtype_code(X), Mtok, K, _ld(X), Ns, qdt, _ptr(Xq), Kl, _ptr(sx), _stream(X)))
    return Xq, sx


def nm_bitmap_encode(W: torch.Tensor, mask: torch.Tensor, ldv: int | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """Bitmap format of bf16 W under mask: (vals [R, ldv] bf16, offs [R, K/64 + 1] int32)."""
    R, K = W.shape
    ldv = K if ldv is None else ldv
    vals = torch.zeros((R, ldv), dtype=torch.bfloat16, device=W.device)
    offs = torch.empty((R, K // 64 + 1), dtype=torch.int32, device=W.device)
    _check(raw.nm_bitmap_encode(_ptr(W), dtype_code(W), R, K, _ld(W), _ptr(mask), _ld(mask), _ptr(vals), ldv,
                                _ptr(offs), _ld(offs), _stream(W)))
    return vals, offs


def nm_spmm_bitmap(X: torch.Tensor, vals: torch.Tensor, mask: torch.Tensor, offs: torch.Tensor, R: int | None = None,
                   ydt: int = NM_BF16, out: torch.Tensor | None = None, ws: torch.Tensor | None = None) -> torch.Tensor:
    """Y = X W_hat^T with W_hat in the bitmap format (decode into LDS, then dense MFMA)."""
    Mtok, K = X.shape
    R = vals.shape[0] if R is None else R
    Y = out if out is not None else torch.empty((Mtok, R), dtype=_TORCH[ydt], device=X.device)
    need = raw.nm_spmm_bitmap_workspace(Mtok, K, R)
    if need and (ws is None or ws.numel() < need):
        ws = _ws(need, X.device)
    _check(raw.nm_spmm_bitmap(_ptr(X), Mtok, K, _ld(X), _ptr(vals), _ld(vals), _ptr(mask), _ld(mask), _ptr(offs),
                              _ld(offs), R, _ptr(Y), ydt, _ld(Y), _ptr(ws), 0 if ws is None else ws.numel(),
                              _stream(X)))
    return Y


def nm_spmm_lowrank(X: torch.Tensor, vals: torch.Tensor, idx: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                    R: int | None = None, Ns: int = 0, ydt: int = NM_BF16, out: torch.Tensor | None = None,
                    ws: torch.Tensor | None = None) -> torch.Tensor:
    """Y = X W_hat^T + bf16(X A^T) B^T: sparse layer plus stacked low-rank adapters (bf16)."""
    Mtok, K = X.shape
    R = vals.shape[0] if R is None else R
    rank = A.shape[0]
    Y = out if out is not None else torch.empty((Mtok, R), dtype=_TORCH[ydt], device=X.device)
    need = raw.nm_spmm_lowrank_workspace(Mtok, K, R, Ns, rank)
    if need and (ws is None or ws.numel() < need):
        ws = _ws(need, X.device)
    _check(raw.nm_spmm_lowrank(_ptr(X), Mtok, K, _ld(X), _ptr(vals), _ptr(idx), R, _ld(vals), _ld(idx), Ns,
                               _ptr(A), _ld(A), _ptr(B), _ld(B), rank, _ptr(Y), ydt, _ld(Y), _ptr(ws),
                               0 if ws is None else ws.numel(), _stream(X)))
    return Y


def nm_spmm(X: torch.Tensor, vals: torch.Tensor, idx: torch.Tensor, R: int | None = None, Ns: int = 0,
            x_scale: torch.Tensor | None = None, w_scale: float = 1.0, ydt: int | None = None,
            out: torch.Tensor | None = None, ws: torch.Tensor | None = None) -> torch.Tensor:
    Mtok, K = X.shape
    R = vals.shape[0] if R is None else R
    xdt = dtype_code(X)
    if ydt is None:
        ydt = {NM_BF16: NM_BF16, NM_I8: NM_I32, NM_FP8: NM_F32}[xdt]
    Y = out if out is not None else torch.empty((Mtok, R), dtype=_TORCH[ydt], device=X.device)
    need = raw.nm_spmm_workspace(Mtok, K, R, Ns, xdt)
    if need and (ws is None or ws.numel() < need):
        ws = _ws(need, X.device)
    _check(raw.nm_spmm(_ptr(X), xdt, Mtok, K, _ld(X), _ptr(vals), dtype_code(vals), _ptr(idx), R, _ld(vals), _ld(idx),
                       Ns, _ptr(x_scale), w_scale, _ptr(Y), ydt, _ld(Y), _ptr(ws), 0 if ws is None else ws.numel(),
                       _stream(X)))
    return Y


NM_SPMM_SCRATCH_BYTES = 64 << 20


def nm_spmm_noalloc(X: torch.Tensor, vals: torch.Tensor, idx: torch.Tensor, R: int | None = None, Ns: int = 0,
                    x_scale: torch.Tensor | None = None, w_scale: float = 1.0, ydt: int | None = None,
                    out: torch.Tensor | None = None) -> torch.Tensor:
    """nm_spmm with the library's own per-device scratch buffer instead of a workspace (for
    callers that cannot allocate); give `out` to allocate nothing here either."""
    Mtok, K = X.shape
    R = vals.shape[0] if R is None else R
    xdt = dtype_code(X)
    if ydt is None:
        ydt = {NM_BF16: NM_BF16, NM_I8: NM_I32, NM_FP8: NM_F32}[xdt]
    Y = out if out is not None else torch.empty((Mtok, R), dtype=_TORCH[ydt], device=X.device)
    _check(raw.nm_spmm_noalloc(_ptr(X), xdt, Mtok, K, _ld(X), _ptr(vals), dtype_code(vals), _ptr(idx), R, _ld(vals),
                               _ld(idx), Ns, _ptr(x_scale), w_scale, _ptr(Y), ydt, _ld(Y), _stream(X)))
    return Y
