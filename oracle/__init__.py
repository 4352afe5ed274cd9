"""CPU oracle for the N:M sparsification hot path -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package.  The GPU library never does, and this package never imports the
GPU library: the two share no code.  The arithmetic lives in ``nm_oracle.c``
(plain scalar C, see its header for the passages each function follows); this
module compiles it with gcc on first use and wraps it with ctypes and numpy.

Every function takes and returns numpy arrays (bf16 is carried as uint16 bit
patterns).  Shapes: weights [R, K] row-major, activations [tokens, K],
mask bits uint8 [R, ceil(K/8)] LSB-first, packed values [R, K*N/M],
packed in-group indices uint32 [R, words] as an LSB-first bitstream of
ceil(log2 M)-bit fields.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "nm_oracle.c"
_LIB = _HERE / "libnmoracle.so"

F32, BF16, I8, I32 = 0, 1, 2, 3
SCORE_HESSIAN, SCORE_MAGNITUDE = 0, 1

_DT = {np.dtype(np.float32): F32, np.dtype(np.uint16): BF16, np.dtype(np.int8): I8, np.dtype(np.int32): I32}
_NP = {F32: np.float32, BF16: np.uint16, I8: np.int8, I32: np.int32}

CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-std=c11"]


def build(force: bool = False) -> Path:
    """Compile nm_oracle.c into libnmoracle.so (gcc)."""
    if force or not _LIB.exists() or _LIB.stat().st_mtime < _SRC.stat().st_mtime:
        tmp = _LIB.with_suffix(f".so.tmp{os.getpid()}")
        subprocess.check_call(["gcc", *CFLAGS, str(_SRC), "-o", str(tmp), "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


SANITIZE_FLAGS = ["-std=c11", "-O1", "-g", "-fopenmp", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                  "-fno-omit-frame-pointer"]


def build_sanitize_check(out: Path | None = None) -> Path:
    """Compile sanitize_check.c (every oracle routine over exactly sized buffers) with
    AddressSanitizer and UndefinedBehaviorSanitizer into a standalone program (gcc)."""
    out = Path(out) if out is not None else _HERE / "sanitize_check"
    tmp = out.with_name(out.name + f".tmp{os.getpid()}")
    subprocess.check_call(["gcc", *SANITIZE_FLAGS, "-I", str(_HERE), str(_HERE / "sanitize_check.c"), "-o", str(tmp),
                           "-lm"])
    os.replace(tmp, out)
    return out


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(str(build()))
        _declare(_lib)
    return _lib


def _declare(L):
    P, I64, I, F, D, U64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_double, ctypes.c_uint64
    sig = {
        "or_f32_to_bf16": (None, [P, I64, P]),
        "or_bf16_to_f32": (None, [P, I64, P]),
        "or_index_bits": (I, [I]),
        "or_colsumsq": (None, [P, I, I64, I64, P]),
        "or_score": (None, [P, I, I64, I64, P, I64, F, I, P]),
        "or_topn_mask": (None, [P, I64, I64, I64, I, I, P, I64]),
        "or_pack": (None, [P, I, I64, I64, I64, P, I64, I, I, I, P, I64, P, I64]),
        "or_unpack": (None, [P, I, I64, P, I64, I64, I64, I, I, P]),
        "or_slide_decompose": (I64, [P, I, I64, I64, I64, P, I64, I, I, P, I64, P, I64]),
        "or_slide_fold": (None, [P, I, I64, P, I64, I64, I64, I, P]),
        "or_lift": (None, [P, I, I64, I64, I, P]),
        "or_quant_i8": (None, [P, I64, I64, I64, P, P]),
        "or_e4m3_decode": (None, [P, I64, P]),
        "or_e4m3_encode": (None, [P, I64, P]),
        "or_quant_fp8": (None, [P, I64, I64, I64, P, P]),
        "or_masked_matmul_fp8": (None, [P, I64, I64, P, I64, P, I64, P]),
        "or_masked_matmul": (None, [P, I, I64, I64, I64, P, I, I64, I64, P, I64, P]),
        "or_masked_matmul_at": (None, [P, I, I64, I64, P, I, I64, P, I64, P, P, I64, P]),
        "or_masked_matmul_i8": (I64, [P, I64, I64, I64, P, I64, I64, P, I64, P, F, P, P]),
        "or_absmean": (D, [P, I, I64]),
        "or_lowrank_u": (None, [P, I, I64, I64, P, I, I64, P]),
        "or_bitmap_encode": (None, [P, I, I64, I64, P, I64, P, I, I64, P, I64]),
        "or_bitmap_decode": (None, [P, I, I64, P, I64, I64, I64, P, I]),
        "or_sparse_lowrank": (None, [P, I, I64, I64, P, I, I64, P, I64, P, I, P, I, I64, P]),
        "or_apply_mask_i8": (None, [P, I64, I64, P, I64, P]),
        "or_splitmix64_at": (U64, [U64, U64]),
        "or_rademacher": (I, [U64, I, I64, I64, I64]),
        "or_hutchinson_rows": (None, [P, I, I64, I64, I, U64, P, I64, P]),
        "or_hutchinson_u_rows": (None, [P, I, I64, I64, I, U64, P, I64, P]),
        "or_stats": (None, [P, I64, P, P]),
        "or_mask_overfull": (I64, [P, I64, I64, I64, I, I]),
        "or_gate_anneal": (None, [P, I64, I64, D, D, I, I, D, D, I, I, P, P, I64, P]),
        "or_gate_value": (D, [F, D, D, D, D, I]),
        "or_num_threads": (I, []),
        "or_set_threads": (None, [I]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args


def _p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _dt(a: np.ndarray) -> int:
    return _DT[a.dtype]


def _c(a, dtype=None):
    return np.ascontiguousarray(a if dtype is None else np.asarray(a, dtype=dtype))


def mask_bytes(K: int) -> int:
    return (K + 7) // 8


def index_words(slots: int, M: int) -> int:
    return (slots * lib().or_index_bits(M) + 31) // 32


# ---------------------------------------------------------------- numerics
def f32_to_bf16(x) -> np.ndarray:
    x = _c(x, np.float32)
    y = np.empty(x.shape, np.uint16)
    lib().or_f32_to_bf16(_p(x), x.size, _p(y))
    return y


def bf16_to_f32(x) -> np.ndarray:
    x = _c(x, np.uint16)
    y = np.empty(x.shape, np.float32)
    lib().or_bf16_to_f32(_p(x), x.size, _p(y))
    return y


# ---------------------------------------------------------------- A1
def colsumsq(X: np.ndarray) -> np.ndarray:
    """H_k = sum_i X_ik^2 in double.  X: [n, K] float32 or bf16 (uint16)."""
    X = _c(X)
    n, K = X.shape
    H = np.empty(K, np.float64)
    lib().or_colsumsq(_p(X), _dt(X), n, K, _p(H))
    return H


# ---------------------------------------------------------------- A3
def score(W: np.ndarray, H: np.ndarray | None, eps: float, mode: int = SCORE_HESSIAN) -> np.ndarray:
    """s = (H+eps) * W^2 (float, fixed op order) or |W|.  H: [K] (broadcast) or [R, K]."""
    W = _c(W)
    R, K = W.shape
    S = np.empty((R, K), np.float32)
    if mode == SCORE_MAGNITUDE:
        Hh, ldh = np.zeros(1, np.float32), 0
    else:
        Hh = _c(H, np.float32)
        ldh = 0 if Hh.ndim == 1 else K
    lib().or_score(_p(W), _dt(W), R, K, _p(Hh), ldh, ctypes.c_float(eps), mode, _p(S))
    return S


# ---------------------------------------------------------------- A7
def topn_mask(S: np.ndarray, N: int, M: int) -> np.ndarray:
    S = _c(S, np.float32)
    R, K = S.shape
    mask = np.zeros((R, mask_bytes(K)), np.uint8)
    lib().or_topn_mask(_p(S), R, K, K, N, M, _p(mask), mask.shape[1])
    return mask


def mask_to_bool(mask: np.ndarray, K: int) -> np.ndarray:
    return np.unpackbits(mask, axis=1, bitorder="little")[:, :K].astype(bool)


def bool_to_mask(b: np.ndarray) -> np.ndarray:
    return np.packbits(b.astype(np.uint8), axis=1, bitorder="little")


# ---------------------------------------------------------------- A8
def pack(W: np.ndarray, mask: np.ndarray, N: int, M: int, vdtype=None):
    """Returns (vals [R, K*N/M], idx uint32 [R, words])."""
    W = _c(W)
    R, K = W.shape
    vdt = _dt(W) if vdtype is None else vdtype
    slots = K // M * N
    vals = np.zeros((R, slots), _NP[vdt])
    words = index_words(slots, M)
    idx = np.zeros((R, words), np.uint32)
    mask = _c(mask, np.uint8)
    lib().or_pack(_p(W), _dt(W), R, K, K, _p(mask), mask.shape[1], N, M, vdt, _p(vals), slots, _p(idx), words)
    return vals, idx


def mask_overfull(mask: np.ndarray, K: int, G: int, cap: int) -> int:
    """Groups of G consecutive mask bits per row with more than cap set bits."""
    mask = _c(mask, np.uint8)
    return int(lib().or_mask_overfull(_p(mask), mask.shape[0], K, mask.shape[1], G, cap))


def unpack(vals: np.ndarray, idx: np.ndarray, K: int, N: int, M: int) -> np.ndarray:
    vals, idx = _c(vals), _c(idx, np.uint32)
    R = vals.shape[0]
    Wd = np.empty((R, K), vals.dtype)
    lib().or_unpack(_p(vals), _dt(vals), vals.shape[1], _p(idx), idx.shape[1], R, K, N, M, _p(Wd))
    return Wd


# ---------------------------------------------------------------- A9 / A11
def lifted_width(K: int, Ns: int) -> int:
    return K // (2 * Ns) * 4 * (Ns - 1)


def slide_decompose(W: np.ndarray, mask: np.ndarray, Ns: int, vdtype=None):
    """(2N-2):2N -> overlapping 2:4 over K' = (2-2/N)K.  Returns (vals, idx, unplaced)."""
    W = _c(W)
    R, K = W.shape
    vdt = _dt(W) if vdtype is None else vdtype
    Kl = lifted_width(K, Ns)
    vals = np.zeros((R, Kl // 2), _NP[vdt])
    words = (Kl // 2 * 2 + 31) // 32
    idx = np.zeros((R, words), np.uint32)
    mask = _c(mask, np.uint8)
    bad = lib().or_slide_decompose(_p(W), _dt(W), R, K, K, _p(mask), mask.shape[1], Ns, vdt,
                                   _p(vals), vals.shape[1], _p(idx), words)
    return vals, idx, int(bad)


def slide_fold(vals: np.ndarray, idx: np.ndarray, K: int, Ns: int) -> np.ndarray:
    vals, idx = _c(vals), _c(idx, np.uint32)
    R = vals.shape[0]
    Wd = np.empty((R, K), np.float64)
    lib().or_slide_fold(_p(vals), _dt(vals), vals.shape[1], _p(idx), idx.shape[1], R, K, Ns, _p(Wd))
    return Wd


def lift(X: np.ndarray, Ns: int) -> np.ndarray:
    X = _c(X)
    Mt, K = X.shape
    Xl = np.empty((Mt, lifted_width(K, Ns)), X.dtype)
    lib().or_lift(_p(X), _dt(X), Mt, K, Ns, _p(Xl))
    return Xl


def quant_i8(X: np.ndarray):
    """Per-token absmax int8 quantisation of bf16 X [Mt, K] (uint16 bits):
    returns (X_q int8 [Mt, K], s_x float32 [Mt]) with X ~= s_x[:, None] * X_q."""
    X = _c(X, np.uint16)
    Mt, K = X.shape
    Xq = np.empty((Mt, K), np.int8)
    sx = np.empty(Mt, np.float32)
    lib().or_quant_i8(_p(X), Mt, K, K, _p(Xq), _p(sx))
    return Xq, sx


def e4m3_decode(c: np.ndarray) -> np.ndarray:
    """OCP FP8 e4m3 codes (uint8) -> float32 values."""
    c = _c(c, np.uint8)
    y = np.empty(c.shape, np.float32)
    lib().or_e4m3_decode(_p(c), c.size, _p(y))
    return y


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest OCP FP8 e4m3 code, ties to even, saturating at 448."""
    x = _c(x, np.float32)
    c = np.empty(x.shape, np.uint8)
    lib().or_e4m3_encode(_p(x), x.size, _p(c))
    return c


def quant_fp8(X: np.ndarray):
    """Per-token FP8 quantisation of bf16 X: (codes uint8 [Mt, K], s_x float32 [Mt]),
    s_x = max|x| / 448, code = e4m3(x / s_x)."""
    X = _c(X, np.uint16)
    Mt, K = X.shape
    Xq = np.empty((Mt, K), np.uint8)
    sx = np.empty(Mt, np.float32)
    lib().or_quant_fp8(_p(X), Mt, K, K, _p(Xq), _p(sx))
    return Xq, sx


def quant_lift(X: np.ndarray, Ns: int, fp8: bool = False):
    """The online step of the slide path: quantise per token (int8, or FP8 e4m3 codes),
    then lift (Ns = 0: no lift).  Returns (codes lifted [Mt, K'], s_x float32 [Mt])."""
    Xq, sx = quant_fp8(X) if fp8 else quant_i8(X)
    if not Ns:
        return Xq, sx
    return (lift(Xq.view(np.int8), Ns).view(np.uint8) if fp8 else lift(Xq, Ns)), sx


def masked_matmul_fp8(Xq: np.ndarray, Wq: np.ndarray, mask: np.ndarray | None = None) -> np.ndarray:
    """Y = X (mask*W)^T over FP8 codes, in double."""
    Xq, Wq = _c(Xq, np.uint8), _c(Wq, np.uint8)
    Mt, K = Xq.shape
    R = Wq.shape[0]
    Y = np.empty((Mt, R), np.float64)
    m = None if mask is None else _c(mask, np.uint8)
    lib().or_masked_matmul_fp8(_p(Xq), Mt, K, _p(Wq), R, _p(m), 0 if m is None else m.shape[1], _p(Y))
    return Y


# ---------------------------------------------------------------- A12 / A13
def masked_matmul(X: np.ndarray, W: np.ndarray, mask: np.ndarray | None = None) -> np.ndarray:
    """Y = X (mask*W)^T in double.  X [Mt, K], W [R, K]."""
    X, W = _c(X), _c(W)
    Mt, K = X.shape
    R = W.shape[0]
    Y = np.empty((Mt, R), np.float64)
    m = None if mask is None else _c(mask, np.uint8)
    lib().or_masked_matmul(_p(X), _dt(X), Mt, K, K, _p(W), _dt(W), R, K, _p(m), 0 if m is None else m.shape[1], _p(Y))
    return Y


def masked_matmul_at(X, W, mask, rows_m, rows_o) -> np.ndarray:
    X, W = _c(X), _c(W)
    K = X.shape[1]
    rm, ro = _c(rows_m, np.int64), _c(rows_o, np.int64)
    Y = np.empty(rm.size, np.float64)
    m = None if mask is None else _c(mask, np.uint8)
    lib().or_masked_matmul_at(_p(X), _dt(X), K, K, _p(W), _dt(W), K, _p(m), 0 if m is None else m.shape[1],
                              _p(rm), _p(ro), rm.size, _p(Y))
    return Y


def lowrank_u(X: np.ndarray, A: np.ndarray) -> np.ndarray:
    """u = X A^T in double (exact value of the adapter's intermediate).  X [Mt, K], A [r, K]."""
    X, A = _c(X), _c(A)
    Mt, K = X.shape
    r = A.shape[0]
    U = np.empty((Mt, r), np.float64)
    lib().or_lowrank_u(_p(X), _dt(X), Mt, K, _p(A), _dt(A), r, _p(U))
    return U


def sparse_lowrank(X: np.ndarray, W: np.ndarray, mask: np.ndarray | None, A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """Y = X (mask*W)^T + bf16(X A^T) B^T in double (SALR section 3).  A [r, K], B [R, r]."""
    X, W, A, B = _c(X), _c(W), _c(A), _c(B)
    Mt, K = X.shape
    R = W.shape[0]
    r = A.shape[0]
    assert A.shape[1] == K and B.shape == (R, r)
    Y = np.empty((Mt, R), np.float64)
    m = None if mask is None else _c(mask, np.uint8)
    lib().or_sparse_lowrank(_p(X), _dt(X), Mt, K, _p(W), _dt(W), R, _p(m), 0 if m is None else m.shape[1],
                            _p(A), _dt(A), _p(B), _dt(B), r, _p(Y))
    return Y


def bitmap_encode(W: np.ndarray, mask: np.ndarray, ldv: int | None = None):
    """SALR bitmap format: (vals [R, ldv] kept values per row in column order, offs int32
    [R, ceil(K/64) + 1] kept values before each 64-column block, the last = row count).
    The bitmap is the mask itself."""
    W = _c(W)
    R, K = W.shape
    ldv = K if ldv is None else ldv
    vals = np.zeros((R, ldv), W.dtype)
    nb = (K + 63) // 64
    offs = np.zeros((R, nb + 1), np.int32)
    mask = _c(mask, np.uint8)
    lib().or_bitmap_encode(_p(W), _dt(W), R, K, _p(mask), mask.shape[1], _p(vals), _dt(W), ldv, _p(offs), nb + 1)
    return vals, offs


def bitmap_decode(vals: np.ndarray, mask: np.ndarray, K: int) -> np.ndarray:
    vals = _c(vals)
    R, ldv = vals.shape
    Wd = np.zeros((R, K), vals.dtype)
    mask = _c(mask, np.uint8)
    lib().or_bitmap_decode(_p(vals), _dt(vals), ldv, _p(mask), mask.shape[1], R, K, _p(Wd), _dt(vals))
    return Wd


def masked_matmul_i8(Xq, W, mask, sx, alpha):
    """Exact integer sum (int32 result, asserted in range) and y = (alpha*s_x)*acc in float."""
    Xq, W = _c(Xq, np.int8), _c(W, np.int8)
    Mt, K = Xq.shape
    R = W.shape[0]
    acc = np.empty((Mt, R), np.int32)
    y = np.empty((Mt, R), np.float32)
    m = None if mask is None else _c(mask, np.uint8)
    sx = _c(sx, np.float32)
    ovf = lib().or_masked_matmul_i8(_p(Xq), Mt, K, K, _p(W), R, K, _p(m), 0 if m is None else m.shape[1],
                                    _p(sx), ctypes.c_float(alpha), _p(acc), _p(y))
    assert ovf == 0, f"{ovf} outputs overflow int32"
    return acc, y


# ---------------------------------------------------------------- A10
def absmean(W: np.ndarray) -> float:
    W = _c(W)
    return float(lib().or_absmean(_p(W), _dt(W), W.size))


def apply_mask_i8(Wt: np.ndarray, mask: np.ndarray) -> np.ndarray:
    Wt = _c(Wt, np.int8)
    R, K = Wt.shape
    out = np.empty_like(Wt)
    mask = _c(mask, np.uint8)
    lib().or_apply_mask_i8(_p(Wt), R, K, _p(mask), mask.shape[1], _p(out))
    return out


# ---------------------------------------------------------------- A2
def splitmix64_at(seed: int, i: int) -> int:
    return int(lib().or_splitmix64_at(ctypes.c_uint64(seed), ctypes.c_uint64(i)))


def rademacher(seed: int, p: int, o: int, k: int, K: int) -> int:
    return int(lib().or_rademacher(ctypes.c_uint64(seed), p, o, k, K))


def hutchinson_rows(X: np.ndarray, probes: int, seed: int, rows) -> np.ndarray:
    """Hutchinson diagonal estimate rows D[rows, :] of ||X W^T||_F^2 (double)."""
    X = _c(X)
    n, K = X.shape
    rows = _c(rows, np.int64)
    D = np.empty((rows.size, K), np.float64)
    lib().or_hutchinson_rows(_p(X), _dt(X), n, K, probes, ctypes.c_uint64(seed), _p(rows), rows.size, _p(D))
    return D


def hutchinson_u_rows(X: np.ndarray, probes: int, seed: int, rows) -> np.ndarray:
    X = _c(X)
    n, K = X.shape
    rows = _c(rows, np.int64)
    U = np.empty((rows.size, probes, n), np.float64)
    lib().or_hutchinson_u_rows(_p(X), _dt(X), n, K, probes, ctypes.c_uint64(seed), _p(rows), rows.size, _p(U))
    return U


# ---------------------------------------------------------------- A4 - A6
def stats(S: np.ndarray):
    S = _c(S, np.float32)
    mu, sg = ctypes.c_double(), ctypes.c_double()
    lib().or_stats(_p(S), S.size, ctypes.byref(mu), ctypes.byref(sg))
    return mu.value, sg.value


def gate_anneal(S: np.ndarray, mu: float, sigma: float, N: int, M: int, T0: float, rho: float, steps: int,
                m_step: int | None = None):
    """Returns (m_t float32 [R,K] of step t = m_step (default the last), hard mask
    bits, Lmid [steps] double)."""
    S = _c(S, np.float32)
    R, K = S.shape
    t = steps - 1 if m_step is None else m_step
    mf = np.empty((R, K), np.float32)
    hm = np.zeros((R, mask_bytes(K)), np.uint8)
    lm = np.empty(steps, np.float64)
    lib().or_gate_anneal(_p(S), R, K, mu, sigma, N, M, T0, rho, steps, t, _p(mf), _p(hm), hm.shape[1], _p(lm))
    return mf, hm, lm


def num_threads() -> int:
    return int(lib().or_num_threads())


def set_threads(n: int) -> None:
    lib().or_set_threads(int(n))


def gate_value(s: float, mu: float, sigma: float, T0: float, rho: float, t: int) -> float:
    return float(lib().or_gate_value(ctypes.c_float(s), mu, sigma, T0, rho, t))
