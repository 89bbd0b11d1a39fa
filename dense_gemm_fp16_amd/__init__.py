"""Python binding of the MI355X fp16 TN GEMM library (libgemm_tn.so).

Argument marshalling only: every step of the GEMM runs in the HIP kernels
behind the C ABI declared in include/gemm_tn.h.  Torch supplies device
memory and the current HIP stream.  There is no fallback: if the compiled
library is missing, importing the package raises ImportError.

    D = gemm_tn(A, B, alpha=1.0, beta=0.0, C=None, out_dtype=torch.float16)

A: (M, K) or (batch, M, K) float16, B: (N, K) or (batch, N, K) float16,
C / D: (M, N) or (batch, M, N) of out_dtype, all on the GPU.  Row and
batch strides are taken from the tensors, so slices of wider arrays (and,
for A and B, a batch dimension made by expand) need no copy.  C and D must
have unit stride along N.  A and B may have unit stride along K (the TN
layout) or along M / N: a transposed view such as `At.t()` of a
contiguous (K, M) tensor is passed as an operand stored along M.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgemm_tn.so")

GEMM_TN_F16, GEMM_TN_F32 = 0, 1
GEMM_TN_ROW_K, GEMM_TN_ROW_MN = 0, 1
(OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_LAUNCH, ERR_WORKSPACE,
 ERR_SCRATCH) = range(6)
# fixed per-GPU split-K scratch of gemm_tn_ex_noalloc (GEMM_TN_NOALLOC_
# SCRATCH_BYTES in include/gemm_tn.h)
NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024

# torch bundles its own HIP runtime under the same soname as the system one
# (libamdhip64.so.7).  Whichever is loaded first serves the whole process, so
# torch is imported before the library: its streams and allocations and our
# launches then go through one runtime.
import torch  # noqa: E402,F401

EXPORTS = ("gemm_tn", "gemm_tn_strided_batched", "gemm_tn_ex",
           "gemm_tn_ex_noalloc", "gemm_tn_describe", "gemm_tn_status_string", "gemm_tn_version",
           "transpose_f32", "attention_fwd", "gemm_tn_f16acc")

_REBUILD = ("run `python dense_gemm_fp16_amd/build.py` "
            "(or __graft_entry__.build()) first")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; {_REBUILD}")

_lib = ctypes.CDLL(LIB_PATH)
_missing = [n for n in EXPORTS if not hasattr(_lib, n)]
if _missing:
    raise ImportError(f"{LIB_PATH} is stale (no {', '.join(_missing)}); "
                      f"{_REBUILD}")
_i64, _f32, _vp, _int = (ctypes.c_int64, ctypes.c_float, ctypes.c_void_p,
                         ctypes.c_int)
_lib.gemm_tn.restype = _int
_lib.gemm_tn.argtypes = [_i64, _i64, _i64, _f32, _vp, _vp, _f32, _vp, _vp,
                         _int, _vp]
_lib.gemm_tn_strided_batched.restype = _int
_lib.gemm_tn_strided_batched.argtypes = [_i64, _i64, _i64, _i64, _f32, _vp,
                                         _i64, _vp, _i64, _f32, _vp, _i64,
                                         _vp, _i64, _int, _vp]
_lib.gemm_tn_ex.restype = _int
_lib.gemm_tn_ex.argtypes = [_i64, _i64, _i64, _i64, _f32, _vp, _int, _i64,
                            _i64, _vp, _int, _i64, _i64, _f32, _vp, _i64, _i64,
                            _vp, _i64, _i64, _int, _vp]
_lib.gemm_tn_ex_noalloc.restype = _int
_lib.gemm_tn_ex_noalloc.argtypes = _lib.gemm_tn_ex.argtypes
_lib.gemm_tn_describe.restype = _int
_lib.gemm_tn_describe.argtypes = [_i64, _i64, _i64, _i64, _int, _i64, _int,
                                  _i64, _i64, _i64, _i64, _i64, _i64, _i64,
                                  _f32, _int, _int, ctypes.c_char_p, _i64]
_lib.transpose_f32.restype = _int
_lib.transpose_f32.argtypes = [_i64, _i64, _i64, _vp, _vp, _vp]
_lib.attention_fwd.restype = _int
_lib.attention_fwd.argtypes = [_i64, _i64, _i64, _i64, _f32, _vp, _vp, _vp,
                               _vp, _int, _vp, _vp]
_lib.gemm_tn_f16acc.restype = _int
_lib.gemm_tn_f16acc.argtypes = [_i64, _i64, _i64, _i64, _vp, _i64, _vp, _i64,
                                _vp, _i64, _vp]
_lib.gemm_tn_status_string.restype = ctypes.c_char_p
_lib.gemm_tn_status_string.argtypes = [_int]
_lib.gemm_tn_version.restype = _int
_lib.gemm_tn_version.argtypes = []

# The fast path of gemm_tn() (csrc/binding_fast.cpp): the same marshalling
# in C++ against torch's tensor API, calling this library's gemm_tn_ex
# through the pointer handed over here.  Without it (not built, or built
# for another torch) the calls are marshalled through ctypes.
_fast = None
_FAST_PATH = os.path.join(_HERE, "_gemm_tn_fast.so")
if os.path.exists(_FAST_PATH):
    import importlib.util as _ilu
    try:
        _spec = _ilu.spec_from_file_location(__name__ + "._gemm_tn_fast",
                                             _FAST_PATH)
        _fast = _ilu.module_from_spec(_spec)
        _spec.loader.exec_module(_fast)
        _fast.set_entry(ctypes.cast(_lib.gemm_tn_ex, ctypes.c_void_p).value)
    except ImportError:
        _fast = None



class GemmError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(f"gemm_tn failed: {status_string(status)} "
                         f"(status {status})")


def status_string(status: int) -> str:
    return _lib.gemm_tn_status_string(status).decode()


def version() -> tuple[int, int]:
    v = _lib.gemm_tn_version()
    return v >> 16, v & 0xFFFF


def lib() -> ctypes.CDLL:
    """The loaded C library (for callers that pass raw pointers)."""
    return _lib


def describe(batch, M, N, K, beta=0.0, out_dtype="f16", aligned16=True,
             strides=None, lds=None, layouts=(GEMM_TN_ROW_K, GEMM_TN_ROW_K)
             ) -> str:
    """Kernel configuration the library picks for this problem.
    lds = (lda, ldb, ldc, ldd), packed rows by default; layouts =
    (layout_a, layout_b)."""
    la, lb = layouts
    if lds is None:
        lds = (M if la else K, N if lb else K, N, N)
    if strides is None:
        strides = ((K if la else M) * lds[0], (K if lb else N) * lds[1],
                   M * lds[2], M * lds[3])
    buf = ctypes.create_string_buffer(256)
    _lib.gemm_tn_describe(batch, M, N, K, la, lds[0], lb, lds[1], lds[2],
                          lds[3], *strides, float(beta),
                          GEMM_TN_F16 if out_dtype == "f16" else GEMM_TN_F32,
                          1 if aligned16 else 0, buf, len(buf))
    return buf.value.decode()


_F16, _F32 = torch.float16, torch.float32


def _dtype_code(dt) -> int:
    if dt is _F16:
        return GEMM_TN_F16
    if dt is _F32:
        return GEMM_TN_F32
    raise TypeError("C / D must be float16 or float32")


# The current stream's raw handle without building a Stream object (which
# costs more than the rest of a small call's marshalling).
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_handle(stream, t):
    """Handle of `stream`, else of the current stream of tensor t's GPU."""
    if stream is not None:
        return stream.cuda_stream
    if _raw_stream is not None:
        return _raw_stream(t.get_device())
    return torch.cuda.current_stream(t.device).cuda_stream


# Each helper reads a tensor's shape and strides once: on small problems the
# Python attribute reads are a visible share of a call.

def _operand(t, name):
    """(layout, row stride, batch stride) of a 2-D operand or of each
    matrix of a 3-D batch: unit stride along K, else unit stride along
    M / N."""
    if t.dtype is not _F16:
        raise TypeError(f"{name} must be float16")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    sh, st = t.shape, t.stride()
    rows, k = sh[-2], sh[-1]
    bs = st[0] if len(sh) == 3 else 0
    if k <= 1 or st[-1] == 1:
        return GEMM_TN_ROW_K, (st[-2] if rows > 1 else max(k, 1)), bs
    if rows <= 1 or st[-2] == 1:
        return GEMM_TN_ROW_MN, st[-1], bs
    raise ValueError(f"{name} needs unit stride along its last or "
                     "second-to-last dimension")


def _matrix(t, name):
    """(row stride, batch stride) of a row-major C / D (unit element
    stride along N)."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    sh, st = t.shape, t.stride()
    if sh and sh[-1] > 1 and st[-1] != 1:
        raise ValueError(f"{name} must be row-major with unit element stride")
    return (st[-2] if sh[-2] > 1 else max(sh[-1], 1),
            st[0] if len(sh) == 3 else 0)


def _out_shape(A, B):
    ash, bsh = A.shape, B.shape
    if len(ash) != len(bsh) or len(ash) not in (2, 3):
        raise ValueError("A and B must both be 2-D or both 3-D")
    if len(ash) == 3:
        if bsh[0] != ash[0] or bsh[2] != ash[2]:
            raise ValueError("B must be (batch, N, K)")
        return (ash[0], ash[1], bsh[1])
    if bsh[1] != ash[1]:
        raise ValueError("B must be (N, K)")
    return (ash[0], bsh[0])


def gemm_tn(A, B, alpha: float = 1.0, beta: float = 0.0, C=None, out=None,
            out_dtype=None, stream=None):
    """D = alpha * A @ B^T + beta * C on the GPU (2-D or batched 3-D).

    `out` may be given (it is then D and is returned); otherwise D is
    allocated with `out_dtype` (default: C's dtype, else float16)."""
    if out is None:
        dt = out_dtype if out_dtype is not None else (
            C.dtype if C is not None else _F16)
        out = torch.empty(_out_shape(A, B), dtype=dt, device=A.device)
    if _fast is not None and out.is_cuda:
        try:
            st = _fast.gemm_tn_fast(A, B, out, alpha, beta,
                                    C if beta != 0.0 else None,
                                    _stream_handle(stream, out))
        except TypeError:      # not tensors / numbers: the checked path says
            st = -1
        if st == OK:
            return out
        if st > 0:
            raise GemmError(st)
    return _gemm_tn_checked(A, B, alpha, beta, C, out, stream)


def _gemm_tn_checked(A, B, alpha, beta, C, out, stream):
    """gemm_tn() with every argument checked in Python (the path for calls
    the fast path hands back, and without it)."""
    layout_a, lda, sa = _operand(A, "A")
    layout_b, ldb, sb = _operand(B, "B")
    ash, bsh = A.shape, B.shape
    if len(ash) != len(bsh) or len(ash) not in (2, 3):
        raise ValueError("A and B must both be 2-D or both 3-D")
    if len(ash) == 3:
        batch, M, K = ash
        if bsh[0] != batch or bsh[2] != K:
            raise ValueError("B must be (batch, N, K)")
        N = bsh[1]
        shape = (batch, M, N)
    else:
        M, K = ash
        if bsh[1] != K:
            raise ValueError("B must be (N, K)")
        N = bsh[0]
        batch, shape = 1, (M, N)
    if out.shape != shape:
        raise ValueError(f"out must have shape {shape}")
    ldd, sd = _matrix(out, "out")
    code = _dtype_code(out.dtype)
    c_ptr, ldc, sc = None, N, 0
    if beta != 0.0:
        if C is None:
            raise ValueError("beta != 0 needs C")
        if C.shape != shape or C.dtype is not out.dtype:
            raise ValueError("C must match D's shape and dtype")
        ldc, sc = _matrix(C, "C")
        c_ptr = C.data_ptr()
    st = _lib.gemm_tn_ex(
        batch, M, N, K, float(alpha), A.data_ptr(), layout_a, lda, sa,
        B.data_ptr(), layout_b, ldb, sb, float(beta), c_ptr, ldc, sc,
        out.data_ptr(), ldd, sd, code, _stream_handle(stream, out))
    if st != OK:
        raise GemmError(st)
    return out


def gemm_tn_strided_batched(batch, M, N, K, alpha, A_ptr, strideA, B_ptr,
                            strideB, beta, C_ptr, strideC, D_ptr, strideD,
                            d_dtype, stream_handle) -> int:
    """Raw-pointer call of the C entry point; returns the status code."""
    return _lib.gemm_tn_strided_batched(batch, M, N, K, float(alpha), A_ptr,
                                        strideA, B_ptr, strideB, float(beta),
                                        C_ptr, strideC, D_ptr, strideD,
                                        d_dtype, stream_handle)


def gemm_tn_raw(M, N, K, alpha, A_ptr, B_ptr, beta, C_ptr, D_ptr, d_dtype,
                stream_handle) -> int:
    """Raw-pointer call of gemm_tn(); returns the status code."""
    return _lib.gemm_tn(M, N, K, float(alpha), A_ptr, B_ptr, float(beta),
                        C_ptr, D_ptr, d_dtype, stream_handle)


def gemm_tn_ex(batch, M, N, K, alpha, A_ptr, lda, strideA, B_ptr, ldb,
               strideB, beta, C_ptr, ldc, strideC, D_ptr, ldd, strideD,
               d_dtype, stream_handle, layout_a=GEMM_TN_ROW_K,
               layout_b=GEMM_TN_ROW_K) -> int:
    """Raw-pointer call of gemm_tn_ex(); returns the status code."""
    return _lib.gemm_tn_ex(batch, M, N, K, float(alpha), A_ptr, layout_a, lda,
                           strideA, B_ptr, layout_b, ldb, strideB,
                           float(beta), C_ptr, ldc, strideC, D_ptr, ldd,
                           strideD, d_dtype, stream_handle)


def gemm_tn_ex_noalloc(batch, M, N, K, alpha, A_ptr, lda, strideA, B_ptr, ldb,
                       strideB, beta, C_ptr, ldc, strideC, D_ptr, ldd,
                       strideD, d_dtype, stream_handle, layout_a=GEMM_TN_ROW_K,
                       layout_b=GEMM_TN_ROW_K) -> int:
    """Raw-pointer call of gemm_tn_ex_noalloc() (split-K partials in the
    library's fixed per-GPU scratch, no allocation); returns the status
    code."""
    return _lib.gemm_tn_ex_noalloc(batch, M, N, K, float(alpha), A_ptr,
                                   layout_a, lda, strideA, B_ptr, layout_b,
                                   ldb, strideB, float(beta), C_ptr, ldc,
                                   strideC, D_ptr, ldd, strideD, d_dtype,
                                   stream_handle)


def transpose_f32(x, out=None, stream=None):
    """y = x^T for a contiguous float32 (M, N) or (batch, M, N) GPU tensor
    (include/transpose_f32.h); returns y of shape (N, M) or (batch, N, M)."""
    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous float32 GPU tensor")
    if x.dim() not in (2, 3):
        raise ValueError("x must be 2-D or 3-D")
    batch = x.shape[0] if x.dim() == 3 else 1
    M, N = x.shape[-2], x.shape[-1]
    shape = (N, M) if x.dim() == 2 else (batch, N, M)
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=x.device)
    if (tuple(out.shape) != shape or out.dtype != torch.float32
            or not out.is_contiguous() or not out.is_cuda):
        raise ValueError(f"out must be a contiguous float32 GPU tensor "
                         f"of shape {shape}")
    st = _lib.transpose_f32(batch, M, N, x.data_ptr(), out.data_ptr(),
                            _stream_handle(stream, out))
    if st != OK:
        raise GemmError(st)
    return out


def transpose_f32_raw(batch, M, N, x_ptr, y_ptr, stream_handle) -> int:
    """Raw-pointer call of transpose_f32(); returns the status code."""
    return _lib.transpose_f32(batch, M, N, x_ptr, y_ptr, stream_handle)


def attention_fwd(q, k, v, scale: float, out=None, out_dtype=None,
                  return_lse: bool = False, lse=None, stream=None):
    """O = softmax(scale * q k^T) v per head (include/attention_fwd.h).

    q: (Lq, d) or (batch, Lq, d), k and v: (Lk, d) or (batch, Lk, d), all
    contiguous float16 GPU tensors with d = 64.  out: optional contiguous
    tensor of q's shape, float16 (default) or float32.  With return_lse (or
    a float32 `lse` tensor of shape (batch, Lq) / (Lq,)), the natural
    log-sum-exp of each row of scale * q k^T is written too and (O, lse) is
    returned; otherwise O."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        if (t.dtype != torch.float16 or not t.is_cuda
                or not t.is_contiguous() or t.dim() not in (2, 3)):
            raise ValueError(f"{n} must be a contiguous 2-D or 3-D float16 "
                             f"GPU tensor")
    if not (q.dim() == k.dim() == v.dim()):
        raise ValueError("q, k and v need the same number of dimensions")
    batch = q.shape[0] if q.dim() == 3 else 1
    Lq, d = q.shape[-2], q.shape[-1]
    Lk = k.shape[-2]
    if (k.shape[-1] != d or tuple(v.shape) != tuple(k.shape)
            or (q.dim() == 3 and k.shape[0] != batch)):
        raise ValueError("k and v must be (batch, Lk, d) with q's batch and d")
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or torch.float16,
                          device=q.device)
    if (tuple(out.shape) != tuple(q.shape) or not out.is_cuda
            or not out.is_contiguous()):
        raise ValueError("out must be a contiguous GPU tensor of q's shape")
    lse_shape = tuple(q.shape[:-1])
    if lse is None and return_lse:
        lse = torch.empty(lse_shape, dtype=torch.float32, device=q.device)
    if lse is not None and (tuple(lse.shape) != lse_shape
                            or lse.dtype != torch.float32 or not lse.is_cuda
                            or not lse.is_contiguous()):
        raise ValueError(f"lse must be a contiguous float32 GPU tensor of "
                         f"shape {lse_shape}")
    st = _lib.attention_fwd(batch, Lq, Lk, d, float(scale), q.data_ptr(),
                            k.data_ptr(), v.data_ptr(), out.data_ptr(),
                            _dtype_code(out.dtype),
                            lse.data_ptr() if lse is not None else None,
                            _stream_handle(stream, out))
    if st != OK:
        raise GemmError(st)
    return (out, lse) if lse is not None else out


def attention_fwd_raw(batch, Lq, Lk, d, scale, q_ptr, k_ptr, v_ptr, o_ptr,
                      o_dtype, lse_ptr, stream_handle) -> int:
    """Raw-pointer call of attention_fwd(); returns the status code."""
    return _lib.attention_fwd(batch, Lq, Lk, d, float(scale), q_ptr, k_ptr,
                              v_ptr, o_ptr, o_dtype, lse_ptr, stream_handle)


def gemm_tn_f16acc(A, B, out=None, stream=None):
    """D = A @ B^T with the sum rounded to fp16 after every 16-deep step of
    K (include/gemm_f16acc.h).  A: (M, K) or (batch, M, K), B: (N, K) or
    (batch, N, K), contiguous float16 GPU tensors (a batch dimension made by
    expand, stride 0, broadcasts); returns D float16 (M, N) or (batch, M,
    N)."""
    for t, n in ((A, "A"), (B, "B")):
        if t.dtype != torch.float16 or not t.is_cuda or t.dim() not in (2, 3):
            raise ValueError(f"{n} must be a 2-D or 3-D float16 GPU tensor")
        if t.numel() > 0 and (t.stride(-1) != 1
                              or t.stride(-2) != t.shape[-1]):
            raise ValueError(f"{n} must have packed rows")
    if A.dim() != B.dim():
        raise ValueError("A and B need the same number of dimensions")
    batch = A.shape[0] if A.dim() == 3 else 1
    M, K = A.shape[-2], A.shape[-1]
    N = B.shape[-2]
    if B.shape[-1] != K or (A.dim() == 3 and B.shape[0] != batch):
        raise ValueError("B must be (batch, N, K) with A's batch and K")
    shape = (M, N) if A.dim() == 2 else (batch, M, N)
    if out is None:
        out = torch.empty(shape, dtype=torch.float16, device=A.device)
    if (tuple(out.shape) != shape or out.dtype != torch.float16
            or not out.is_contiguous() or not out.is_cuda):
        raise ValueError(f"out must be a contiguous float16 GPU tensor of "
                         f"shape {shape}")
    sA = A.stride(0) if A.dim() == 3 and A.numel() > 0 else M * K
    sB = B.stride(0) if B.dim() == 3 and B.numel() > 0 else N * K
    st = _lib.gemm_tn_f16acc(batch, M, N, K, A.data_ptr(), sA, B.data_ptr(),
                             sB, out.data_ptr(), M * N,
                             _stream_handle(stream, out))
    if st != OK:
        raise GemmError(st)
    return out


def gemm_tn_f16acc_raw(batch, M, N, K, A_ptr, strideA, B_ptr, strideB, D_ptr,
                       strideD, stream_handle) -> int:
    """Raw-pointer call of gemm_tn_f16acc(); returns the status code."""
    return _lib.gemm_tn_f16acc(batch, M, N, K, A_ptr, strideA, B_ptr, strideB,
                               D_ptr, strideD, stream_handle)
