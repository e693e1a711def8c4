"""Thin ctypes binding of libfq.so (include/fq.h).

Argument marshalling only: the functions below pass torch device pointers,
shapes and the current HIP stream to the C entry points of the same names and
raise FqError on a non-OK status. Every step of the quantization runs in the
library's HIP kernels; torch supplies device memory and streams.

The library is loaded on first use from this package directory; if it is
missing the binding raises (build it with __graft_entry__.build()). There is
no fallback.
"""
import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

# ---------------------------------------------------------------- enums (fq.h)
FQ_OK, FQ_E_INVALID, FQ_E_UNSUPPORTED, FQ_E_SHAPE, FQ_E_ALIGN, FQ_E_WORKSPACE, FQ_E_HIP = range(7)
FQ_IN_F32, FQ_IN_BF16 = 0, 1
FQ_E4M3, FQ_E5M2, FQ_E2M1 = 0, 1, 2
FQ_PER_TENSOR_CURRENT, FQ_PER_TENSOR_DELAYED, FQ_BLOCK_FP32, FQ_MX, FQ_NVFP4 = range(5)
FQ_ROWWISE, FQ_COLWISE = 1, 2
FQ_ROUND_NEAREST_EVEN, FQ_ROUND_STOCHASTIC = 0, 1
FQ_SCALE_DEFAULT, FQ_SCALE_POW2 = 0, 1
FQ_TRANSFORM_NONE, FQ_TRANSFORM_RHT16 = 0, 1

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfq.so")


class FqDesc(ctypes.Structure):
    _fields_ = [("recipe", ctypes.c_int32), ("in_dtype", ctypes.c_int32), ("format", ctypes.c_int32),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("block_rows", ctypes.c_int32),
                ("block_cols", ctypes.c_int32), ("outputs", ctypes.c_uint32), ("rounding", ctypes.c_int32),
                ("scale_mode", ctypes.c_int32), ("seed", ctypes.c_uint64), ("offset", ctypes.c_uint64),
                ("transform", ctypes.c_int32), ("rht_signs", ctypes.c_uint32)]


class FqPlane(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("scale", ctypes.c_void_p)]


class FqQuantized(ctypes.Structure):
    _fields_ = [("rowwise", FqPlane), ("colwise", FqPlane), ("tensor_scale", ctypes.c_void_p),
                ("amax", ctypes.c_void_p)]


FQ_DELAYED_PENDING_BYTES = 8256


class FqDelayedState(ctypes.Structure):
    _fields_ = [("amax_history", ctypes.c_void_p), ("history_len", ctypes.c_int32), ("scale", ctypes.c_void_p),
                ("scale_inv", ctypes.c_void_p), ("pending", ctypes.c_void_p), ("step", ctypes.c_int64)]


class FqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)}")


_lib = None
_P = ctypes.c_void_p
_SZ = ctypes.POINTER(ctypes.c_size_t)


def lib():
    """The loaded libfq.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    dp = ctypes.POINTER(FqDesc)
    qp = ctypes.POINTER(FqQuantized)
    sig = {
        "fq_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "fq_sizes": (ctypes.c_int, [dp, _SZ, _SZ, _SZ, _SZ, _SZ]),
        "fq_quantize": (ctypes.c_int, [dp, _P, qp, _P, ctypes.c_size_t, _P]),
        "fq_amax": (ctypes.c_int, [dp, _P, _P, _P, ctypes.c_size_t, _P]),
        "fq_quantize_with_amax": (ctypes.c_int, [dp, _P, _P, qp, _P, ctypes.c_size_t, _P]),
        "fq_quantize_delayed": (ctypes.c_int, [dp, _P, ctypes.POINTER(FqDelayedState), qp, _P, ctypes.c_size_t, _P]),
        "fq_delayed_flush": (ctypes.c_int, [dp, ctypes.POINTER(FqDelayedState), _P]),
        "fq_dequantize": (ctypes.c_int, [dp, qp, ctypes.c_int32, _P, ctypes.c_int32, _P]),
        "fq_requantize_transpose": (ctypes.c_int, [dp, qp, qp, _P]),
        "fq_quantize_noalloc": (ctypes.c_int, [dp, _P, qp, _P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def fq_status_str(status: int) -> str:
    return lib().fq_status_str(int(status)).decode()


status_str = fq_status_str


def _check(status: int, where: str):
    if status != FQ_OK:
        raise FqError(status, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


# ---------------------------------------------------------------- descriptors
def desc(recipe: int, in_dtype: int, fmt: int, rows: int, cols: int, block=(0, 0),
         outputs: int = FQ_ROWWISE, rounding: int = FQ_ROUND_NEAREST_EVEN, seed: int = 0, offset: int = 0,
         scale_mode: int = FQ_SCALE_DEFAULT, transform: int = FQ_TRANSFORM_NONE, rht_signs: int = 0) -> FqDesc:
    return FqDesc(recipe, in_dtype, fmt, rows, cols, block[0], block[1], outputs, rounding, scale_mode, seed,
                  offset, transform, rht_signs)


def in_dtype_of(x: torch.Tensor) -> int:
    if x.dtype == torch.bfloat16:
        return FQ_IN_BF16
    if x.dtype == torch.float32:
        return FQ_IN_F32
    raise TypeError("inputs are float32 or bfloat16")


@dataclass
class Sizes:
    row_data: int
    row_scale: int
    col_data: int
    col_scale: int
    workspace: int


def fq_sizes(d: FqDesc) -> Sizes:
    v = [ctypes.c_size_t() for _ in range(5)]
    _check(lib().fq_sizes(ctypes.byref(d), *[ctypes.byref(x) for x in v]), "fq_sizes")
    return Sizes(*[x.value for x in v])


# ---------------------------------------------------------------- output buffers
@dataclass
class Quantized:
    """Device buffers of one quantized tensor (uint8 codes, fp32 or uint8 scales)."""
    row_data: Optional[torch.Tensor] = None
    row_scale: Optional[torch.Tensor] = None
    col_data: Optional[torch.Tensor] = None
    col_scale: Optional[torch.Tensor] = None
    tensor_scale: Optional[torch.Tensor] = None
    amax: Optional[torch.Tensor] = None

    def c(self) -> FqQuantized:
        return FqQuantized(FqPlane(_ptr(self.row_data), _ptr(self.row_scale)),
                           FqPlane(_ptr(self.col_data), _ptr(self.col_scale)),
                           _ptr(self.tensor_scale), _ptr(self.amax))


def _scale_dtype(d: FqDesc):
    return torch.float32 if d.recipe == FQ_BLOCK_FP32 else torch.uint8


def alloc_quantized(d: FqDesc, device="cuda") -> Quantized:
    """Allocate every plane fq_sizes reports for d (shaped, on `device`)."""
    z = fq_sizes(d)
    R, C = d.rows, d.cols
    q = Quantized()
    sd = _scale_dtype(d)
    es = 4 if sd == torch.float32 else 1
    packed = d.format == FQ_E2M1
    if z.row_data:
        q.row_data = torch.empty((R, C // 2) if packed else (R, C), dtype=torch.uint8, device=device)
    if z.col_data:
        q.col_data = torch.empty((C, R // 2) if packed else (C, R), dtype=torch.uint8, device=device)
    if z.row_scale:
        q.row_scale = torch.empty(z.row_scale // es, dtype=sd, device=device)
    if z.col_scale:
        q.col_scale = torch.empty(z.col_scale // es, dtype=sd, device=device)
    q.tensor_scale = torch.empty(1, dtype=torch.float32, device=device)
    q.amax = torch.empty(1, dtype=torch.float32, device=device)
    return q


def alloc_workspace(d: FqDesc, device="cuda") -> Optional[torch.Tensor]:
    n = fq_sizes(d).workspace
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device) if n else None


# ---------------------------------------------------------------- entry points
def fq_quantize(d: FqDesc, x: torch.Tensor, out: Quantized, ws: Optional[torch.Tensor] = None, stream=None):
    q = out.c()
    _check(lib().fq_quantize(ctypes.byref(d), _ptr(x), ctypes.byref(q), _ptr(ws),
                             0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)), "fq_quantize")


def fq_quantize_noalloc(d: FqDesc, x: torch.Tensor, out: Quantized, stream=None):
    """fq_quantize with the library's own per-GPU scratch array (no workspace)."""
    q = out.c()
    _check(lib().fq_quantize_noalloc(ctypes.byref(d), _ptr(x), ctypes.byref(q), _stream(stream)),
           "fq_quantize_noalloc")


def fq_amax(d: FqDesc, x: torch.Tensor, amax_out: torch.Tensor, ws: torch.Tensor, stream=None):
    _check(lib().fq_amax(ctypes.byref(d), _ptr(x), _ptr(amax_out), _ptr(ws), ws.numel() * ws.element_size(),
                         _stream(stream)), "fq_amax")


def fq_quantize_with_amax(d: FqDesc, x: torch.Tensor, amax_in: torch.Tensor, out: Quantized,
                          ws: Optional[torch.Tensor] = None, stream=None):
    q = out.c()
    _check(lib().fq_quantize_with_amax(ctypes.byref(d), _ptr(x), _ptr(amax_in), ctypes.byref(q), _ptr(ws),
                                       0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)),
           "fq_quantize_with_amax")


class DelayedState:
    """Delayed-scaling state in device memory plus the host step counter."""

    def __init__(self, history_len: int = 1024, device="cuda"):
        self.amax_history = torch.zeros(history_len, dtype=torch.float32, device=device)
        self.scale = torch.ones(1, dtype=torch.float32, device=device)
        self.scale_inv = torch.ones(1, dtype=torch.float32, device=device)
        self.pending = torch.zeros(FQ_DELAYED_PENDING_BYTES // 4, dtype=torch.float32, device=device)
        self.step = 0

    def c(self) -> FqDelayedState:
        return FqDelayedState(_ptr(self.amax_history), self.amax_history.numel(), _ptr(self.scale),
                              _ptr(self.scale_inv), _ptr(self.pending), self.step)

    def state_dict(self):
        """The state as it stands (call fq_delayed_flush first to make the
        window and scales current and the pending records unnecessary)."""
        return {"amax_history": self.amax_history.clone(), "scale": self.scale.clone(),
                "scale_inv": self.scale_inv.clone(), "pending": self.pending.clone(), "step": self.step}

    def load_state_dict(self, sd):
        self.amax_history.copy_(sd["amax_history"])
        self.scale.copy_(sd["scale"])
        self.scale_inv.copy_(sd["scale_inv"])
        if "pending" in sd:
            self.pending.copy_(sd["pending"])
        else:
            self.pending.zero_()
        self.step = int(sd["step"])


def fq_quantize_delayed(d: FqDesc, x: torch.Tensor, state: DelayedState, out: Quantized,
                        ws: Optional[torch.Tensor] = None, stream=None, advance: bool = True):
    q = out.c()
    st = state.c()
    _check(lib().fq_quantize_delayed(ctypes.byref(d), _ptr(x), ctypes.byref(st), ctypes.byref(q), _ptr(ws),
                                     0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)),
           "fq_quantize_delayed")
    if advance:
        state.step += 1


def fq_delayed_flush(d: FqDesc, state: DelayedState, stream=None):
    """Bring state's window and scales up to date after its last step."""
    st = state.c()
    _check(lib().fq_delayed_flush(ctypes.byref(d), ctypes.byref(st), _stream(stream)), "fq_delayed_flush")


def fq_dequantize(d: FqDesc, qt: Quantized, which: int, y: torch.Tensor, stream=None):
    """y (float32 or bfloat16) = the values of plane `which` of qt."""
    q = qt.c()
    _check(lib().fq_dequantize(ctypes.byref(d), ctypes.byref(q), which, _ptr(y), in_dtype_of(y), _stream(stream)),
           "fq_dequantize")


def fq_requantize_transpose(d: FqDesc, src: Quantized, dst: Quantized, stream=None):
    """MXFP8, or blockwise 1x128 with power-of-two scales: dst's colwise planes
    from src's rowwise planes (no high-precision source)."""
    a, b = src.c(), dst.c()
    _check(lib().fq_requantize_transpose(ctypes.byref(d), ctypes.byref(a), ctypes.byref(b), _stream(stream)),
           "fq_requantize_transpose")
