"""The oracle: a plain CPU definition of every FP8/FP4 quantization recipe.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package. The GPU library does not import,
link or call it, and it shares no code with the GPU library.

The arithmetic lives in orc.c (built into liborc.so by oracle/build.py);
this module only marshals numpy arrays through ctypes.

Inputs are numpy arrays: float32 for fp32 tensors, uint16 holding the bit
patterns for bf16 tensors. Outputs are numpy arrays of uint8 codes and
float32 scales.

Sources (short labels used across the oracle):
  [MP] "混合精度训练：fp16 到 fp8" (garden.houmin.site)
  [CS] "FP8 Current Scaling：量化、缩放与精度边界" (notes.kuangjux.top)
  [LP] "从 BF16 到 FP8/FP4：大语言模型低精度训练与混合精度预训练" (r00kie-liu.github.io)

What pins each function (tests/test_oracle_*.py):
  decode / encode      all codes against the pages' format facts and against
                       torch's float8 casts; brute-force nearest search;
                       the E2M1 value list of [MP] "NVFP4".
  current / with_amax  the worked example, error and underflow examples and
                       the sharded all-gather example of [CS]; the
                       amax-to-Fmax invariant; the error bound.
  delayed              closed forms: a repeated input equals current scaling
                       on the next step; the window expiry step.
  block                per-tile amax-to-448 invariant, error bound, 2-D
                       transpose invariance, brute force on tiny tensors.
  mx                   closed form code = max(E(a)-8, 0) from the fp32 bits,
                       power-of-two scale, brute force on tiny tensors.
  nvfp4                structure (block holding the tensor amax gets the
                       E4M3 code of 448 and a +-6 element); brute force on
                       tiny tensors (both block shapes and planes, fp32 and
                       bf16, E4M3-subnormal and zero blocks) recomputing A,
                       S, every block code, d_B, r_B and nibble with the
                       test's own float32 arithmetic and nearest-value search
                       over torch-decoded E4M3 and the page's E2M1 list;
                       exact power-of-two cases whose bytes follow from the
                       construction; inputs on rounding boundaries showing
                       that a swapped fp32 association would fail. Which
                       association the pages mean is a reading (they fix the
                       structure only); the pins fix that the oracle computes
                       the stated one.
  variants             MX E5M2 / MXFP4 scale closed forms and brute force;
                       pow2 blockwise against closed forms, brute force and
                       MX blocks sharing the tile exponent.
  sr, rht              Philox against torch's engine; the rounding rule
                       (E2M1, and E4M3 / E5M2 for the per-tensor, blockwise
                       1x128 and MX recipes) against a bit-level
                       add-and-truncate on the fp32 significand and its
                       defining properties, each SR recipe's elements
                       recomputed by the test from their scaled values and
                       their plane's random bits; the
                       transform against a Hadamard matrix built by
                       Kronecker products, and its fp32 rounding against
                       those factors applied as float32 matrix products
                       in the stated stage order. The SR rule (which of the
                       two 16-bit discretizations of stochastic rounding)
                       and the butterfly's stage order are readings the
                       pages do not fix: parity unpinned at that level
                       (each is pinned to the stated reading).
  dequant              exact decode times scale; bf16 rounding against torch.
  requant (MX, pow2    brute force on tiny tensors in float64; exact
  blockwise 1x128)     transposition on grid values; equality with the
                       colwise copy quantized from the source wherever no
                       special value intervenes ([MP] "FP8 通信"); error bound.
"""
import ctypes
import os

import numpy as np

E4M3, E5M2, E2M1 = 0, 1, 2
IN_F32, IN_BF16 = 0, 1
ROWWISE, COLWISE = 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
# ORC_LIB names another build of orc.c (the pin-strength tests load copies
# with planted mistakes this way); by default the one built here.
_LIB_PATH = os.environ.get("ORC_LIB") or os.path.join(_HERE, "liborc.so")
_lib = None

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_u32 = ctypes.c_uint32
_f32 = ctypes.c_float
_fp = ctypes.POINTER(ctypes.c_float)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    sig = {
        "orc_max_code": (_u32, [ctypes.c_int]),
        "orc_decode": (ctypes.c_double, [ctypes.c_int, _u32]),
        "orc_decode_e8m0": (ctypes.c_double, [_u32]),
        "orc_fmax": (_f32, [ctypes.c_int]),
        "orc_encode": (_u32, [ctypes.c_int, _f32]),
        "orc_encode_array": (None, [ctypes.c_int, _p, _i64, _p]),
        "orc_amax": (_f32, [_p, ctypes.c_int, _i64]),
        "orc_tensor_scales": (None, [_f32, _f32, _fp, _fp]),
        "orc_mx_code": (_u32, [_f32]),
        "orc_transpose_u8": (None, [_p, _i64, _i64, _p]),
        "orc_quantize_with_amax": (ctypes.c_int, [_p, ctypes.c_int, _i64, _i64, ctypes.c_int, _u32, _f32,
                                                  _p, _p, _fp]),
        "orc_quantize_current": (ctypes.c_int, [_p, ctypes.c_int, _i64, _i64, ctypes.c_int, _u32,
                                                _p, _p, _fp, _fp]),
        "orc_quantize_delayed": (ctypes.c_int, [_p, ctypes.c_int, _i64, _i64, ctypes.c_int, _u32,
                                                _p, _i32, _fp, _fp, _i64, _p, _p, _fp]),
        "orc_quantize_block": (ctypes.c_int, [_p, ctypes.c_int, _i64, _i64, ctypes.c_int, ctypes.c_int, _u32,
                                              _p, _p, _p, _p]),
        "orc_quantize_mx": (ctypes.c_int, [_p, ctypes.c_int, _i64, _i64, _u32, _p, _p, _p, _p]),
        "orc_quantize_mx_fmt": (ctypes.c_int, [_p, ctypes.c_int, _i64, _i64, ctypes.c_int, _u32, _p, _p, _p, _p]),
        "orc_mx_code_fmt": (_u32, [_f32, ctypes.c_int]),
        "orc_quantize_block_mode": (ctypes.c_int, [_p, ctypes.c_int, _i64, _i64, ctypes.c_int, ctypes.c_int,
                                                   ctypes.c_int, _u32, _p, _p, _p, _p]),
        "orc_dequant_mx_fmt": (None, [_p, _p, _i64, _i64, ctypes.c_int, _p]),
        "orc_quantize_nvfp4": (ctypes.c_int, [_p, ctypes.c_int, _i64, _i64, ctypes.c_int, ctypes.c_int, _u32,
                                              _p, _p, _p, _p, _fp, _fp]),
        "orc_quantize_nvfp4_with_amax": (ctypes.c_int, [_p, ctypes.c_int, _i64, _i64, ctypes.c_int, ctypes.c_int,
                                                        _u32, _f32, _p, _p, _p, _p, _fp, _fp]),
        "orc_quantize_nvfp4_sr_with_amax": (ctypes.c_int, [_p, ctypes.c_int, _i64, _i64, _u32, _f32,
                                                           ctypes.c_uint64, ctypes.c_uint64, _p, _p, _p, _p,
                                                           _fp, _fp]),
        "orc_philox4x32_10": (None, [_p, _p, _p]),
        "orc_rht16_array": (None, [_p, _i64, _u32, _p]),
        "orc_quantize_nvfp4_rht": (ctypes.c_int, [_p, ctypes.c_int, _i64, _i64, _u32, ctypes.c_int, _f32,
                                                  ctypes.c_int, ctypes.c_uint64, ctypes.c_uint64, _p, _p, _fp, _fp]),
        "orc_sr_bits": (_u32, [ctypes.c_uint64, ctypes.c_uint64, _u32, _i64]),
        "orc_encode_e2m1_sr": (_u32, [_f32, _u32]),
        "orc_encode_e2m1_sr_array": (None, [_p, _p, _i64, _p]),
        "orc_encode_sr": (_u32, [ctypes.c_int, _f32, _u32]),
        "orc_encode_sr_array": (None, [ctypes.c_int, _p, _p, _i64, _p]),
        "orc_quantize_with_amax_sr": (ctypes.c_int, [_p, ctypes.c_int, _i64, _i64, ctypes.c_int, _u32, _f32,
                                                     ctypes.c_uint64, ctypes.c_uint64, _p, _p, _fp]),
        "orc_quantize_block_sr": (ctypes.c_int, [_p, ctypes.c_int, _i64, _i64, ctypes.c_int, _u32,
                                                 ctypes.c_uint64, ctypes.c_uint64, _p, _p, _p, _p]),
        "orc_quantize_mx_sr": (ctypes.c_int, [_p, ctypes.c_int, _i64, _i64, ctypes.c_int, _u32, ctypes.c_uint64,
                                              ctypes.c_uint64, _p, _p, _p, _p]),
        "orc_f32_to_bf16_array": (None, [_p, _i64, _p]),
        "orc_requant_mx_colwise": (ctypes.c_int, [_p, _p, _i64, _i64, _p, _p]),
        "orc_requant_block_colwise": (ctypes.c_int, [_p, _p, _i64, _i64, _p, _p]),
        "orc_dequant_tensor": (None, [_p, _i64, ctypes.c_int, _f32, _p]),
        "orc_dequant_block": (None, [_p, _p, _i64, _i64, ctypes.c_int, ctypes.c_int, _p]),
        "orc_dequant_mx": (None, [_p, _p, _i64, _i64, _p]),
        "orc_dequant_nvfp4": (None, [_p, _p, _f32, _i64, _i64, ctypes.c_int, ctypes.c_int, _p]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class OracleError(RuntimeError):
    pass


def _check(rc, what):
    if rc != 0:
        raise OracleError(f"{what}: oracle rejected the input (code {rc})")


def _in(x):
    """(pointer, dtype code, array kept alive) for an input array."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x.ctypes.data, IN_F32, x
    if x.dtype == np.uint16:
        return x.ctypes.data, IN_BF16, x
    raise TypeError("oracle inputs are float32 or uint16 (bf16 bits)")


def _ptr(a):
    return None if a is None else a.ctypes.data


def _shape2(x, shape):
    if shape is not None:
        return int(shape[0]), int(shape[1])
    if x.ndim == 1:
        return 1, int(x.shape[0])
    return int(x.shape[0]), int(x.shape[1])


# ---------------------------------------------------------------- codecs
def max_code(fmt):
    return int(_load().orc_max_code(fmt))


def decode(fmt, code):
    return float(_load().orc_decode(fmt, int(code)))


def decode_e8m0(code):
    return float(_load().orc_decode_e8m0(int(code)))


def fmax(fmt):
    return float(_load().orc_fmax(fmt))


def encode(fmt, y):
    return int(_load().orc_encode(fmt, float(np.float32(y))))


def encode_array(fmt, y):
    """Element-wise encode of a float32 array."""
    y = np.ascontiguousarray(y, dtype=np.float32)
    q = np.empty(y.shape, np.uint8)
    _load().orc_encode_array(fmt, y.ctypes.data, y.size, q.ctypes.data)
    return q


def mx_code(a, fmt=None):
    """E8M0 code of a block amax for MX elements of format fmt (default E4M3)."""
    if fmt is None:
        return int(_load().orc_mx_code(float(np.float32(a))))
    return int(_load().orc_mx_code_fmt(float(np.float32(a)), fmt))


def tensor_scales(a, fmax_value):
    al, s = ctypes.c_float(), ctypes.c_float()
    _load().orc_tensor_scales(float(np.float32(a)), float(np.float32(fmax_value)), ctypes.byref(al), ctypes.byref(s))
    return np.float32(al.value), np.float32(s.value)


def amax(x):
    p, dt, keep = _in(x)
    return np.float32(_load().orc_amax(p, dt, keep.size))


# ---------------------------------------------------------------- recipes
def quantize_current(x, fmt, outputs=ROWWISE, shape=None, sr=None):
    """Per-tensor current scaling. Returns dict(q_row, q_col, s, amax).
    `sr` = (seed, offset) rounds the elements stochastically."""
    p, dt, keep = _in(x)
    R, C = _shape2(keep, shape)
    if sr is not None:
        a = np.float32(_load().orc_amax(p, dt, R * C))
        out = quantize_with_amax(x, fmt, a, outputs=outputs, shape=shape, sr=sr)
        out["amax"] = a
        return out
    q_row = np.empty(R * C, np.uint8)
    q_col = np.empty(R * C, np.uint8) if outputs & COLWISE else None
    s, a = ctypes.c_float(), ctypes.c_float()
    _check(_load().orc_quantize_current(p, dt, R, C, fmt, outputs, _ptr(q_row), _ptr(q_col),
                                        ctypes.byref(s), ctypes.byref(a)), "quantize_current")
    return dict(q_row=q_row.reshape(R, C), q_col=None if q_col is None else q_col.reshape(C, R),
                s=np.float32(s.value), amax=np.float32(a.value))


def quantize_with_amax(x, fmt, amax_value, outputs=ROWWISE, shape=None, sr=None):
    """Per-tensor scaling with a given (e.g. all-reduced) amax.
    `sr` = (seed, offset) rounds the elements stochastically (each plane with
    its own random bits: the colwise copy is then not the rowwise one transposed)."""
    p, dt, keep = _in(x)
    R, C = _shape2(keep, shape)
    q_row = np.empty(R * C, np.uint8)
    q_col = np.empty(R * C, np.uint8) if outputs & COLWISE else None
    s = ctypes.c_float()
    if sr is None:
        rc = _load().orc_quantize_with_amax(p, dt, R, C, fmt, outputs, float(np.float32(amax_value)),
                                            _ptr(q_row), _ptr(q_col), ctypes.byref(s))
    else:
        rc = _load().orc_quantize_with_amax_sr(p, dt, R, C, fmt, outputs, float(np.float32(amax_value)),
                                               int(sr[0]), int(sr[1]), _ptr(q_row), _ptr(q_col), ctypes.byref(s))
    _check(rc, "quantize_with_amax")
    return dict(q_row=q_row.reshape(R, C), q_col=None if q_col is None else q_col.reshape(C, R),
                s=np.float32(s.value))


class DelayedState:
    """Delayed-scaling state: amax window, alpha and s (all fp32)."""

    def __init__(self, history_len=1024):
        self.hist = np.zeros(history_len, np.float32)
        self.alpha = np.float32(1.0)
        self.s = np.float32(1.0)
        self.step = 0

    def copy(self):
        c = DelayedState(len(self.hist))
        c.hist[:] = self.hist
        c.alpha, c.s, c.step = self.alpha, self.s, self.step
        return c


def quantize_delayed(x, fmt, state, outputs=ROWWISE, shape=None):
    """One delayed-scaling step; updates `state` (and advances its step)."""
    p, dt, keep = _in(x)
    R, C = _shape2(keep, shape)
    q_row = np.empty(R * C, np.uint8)
    q_col = np.empty(R * C, np.uint8) if outputs & COLWISE else None
    al, s, a = ctypes.c_float(float(state.alpha)), ctypes.c_float(float(state.s)), ctypes.c_float()
    _check(_load().orc_quantize_delayed(p, dt, R, C, fmt, outputs, state.hist.ctypes.data, len(state.hist),
                                        ctypes.byref(al), ctypes.byref(s), int(state.step),
                                        _ptr(q_row), _ptr(q_col), ctypes.byref(a)), "quantize_delayed")
    state.alpha, state.s = np.float32(al.value), np.float32(s.value)
    state.step += 1
    return dict(q_row=q_row.reshape(R, C), q_col=None if q_col is None else q_col.reshape(C, R),
                amax=np.float32(a.value))


def quantize_block(x, block, outputs=ROWWISE, shape=None, pow2=False, sr=None):
    """Blockwise E4M3 with fp32 tile scales; block is (1,128) or (128,128);
    pow2=True rounds each tile scale to the MX power of two;
    `sr` = (seed, offset) rounds the elements stochastically (1x128 only)."""
    p, dt, keep = _in(x)
    R, C = _shape2(keep, shape)
    br, bc = block
    out = {}
    q_row = np.empty(R * C, np.uint8) if outputs & ROWWISE else None
    s_row = np.empty((R // br) * (C // bc), np.float32) if outputs & ROWWISE else None
    q_col = np.empty(R * C, np.uint8) if outputs & COLWISE else None
    s_col = None
    if outputs & COLWISE:
        s_col = np.empty(C * (R // bc) if br == 1 else (C // bc) * (R // br), np.float32)
    if sr is None:
        rc = _load().orc_quantize_block_mode(p, dt, R, C, br, bc, 1 if pow2 else 0, outputs, _ptr(q_row),
                                             _ptr(s_row), _ptr(q_col), _ptr(s_col))
    else:
        if block != (1, 128):
            raise ValueError("stochastic rounding is offered for 1x128 tiles")
        rc = _load().orc_quantize_block_sr(p, dt, R, C, 1 if pow2 else 0, outputs, int(sr[0]), int(sr[1]),
                                           _ptr(q_row), _ptr(s_row), _ptr(q_col), _ptr(s_col))
    _check(rc, "quantize_block")
    out["q_row"] = None if q_row is None else q_row.reshape(R, C)
    out["s_row"] = None if s_row is None else s_row.reshape(R // br, C // bc)
    out["q_col"] = None if q_col is None else q_col.reshape(C, R)
    if s_col is not None:
        out["s_col"] = s_col.reshape(C, R // bc) if br == 1 else s_col.reshape(C // bc, R // br)
    else:
        out["s_col"] = None
    return out


def quantize_mx(x, outputs=ROWWISE | COLWISE, shape=None, fmt=None, sr=None):
    """MX with E8M0 codes; rowwise 1x32 and colwise 32x1 (transposed).
    fmt: E4M3 (default, MXFP8), E5M2, or E2M1 (MXFP4, codes packed two per byte);
    `sr` = (seed, offset) rounds E4M3 / E5M2 elements stochastically."""
    p, dt, keep = _in(x)
    R, C = _shape2(keep, shape)
    fmt = E4M3 if fmt is None else fmt
    k = 2 if fmt == E2M1 else 1
    q_row = np.empty(R * C // k, np.uint8) if outputs & ROWWISE else None
    e_row = np.empty(R * (C // 32), np.uint8) if outputs & ROWWISE else None
    q_col = np.empty(R * C // k, np.uint8) if outputs & COLWISE else None
    e_col = np.empty(C * (R // 32), np.uint8) if outputs & COLWISE else None
    if sr is None:
        rc = _load().orc_quantize_mx_fmt(p, dt, R, C, fmt, outputs, _ptr(q_row), _ptr(e_row), _ptr(q_col),
                                         _ptr(e_col))
    else:
        rc = _load().orc_quantize_mx_sr(p, dt, R, C, fmt, outputs, int(sr[0]), int(sr[1]), _ptr(q_row),
                                        _ptr(e_row), _ptr(q_col), _ptr(e_col))
    _check(rc, "quantize_mx")
    return dict(q_row=None if q_row is None else q_row.reshape(R, C // k),
                e_row=None if e_row is None else e_row.reshape(R, C // 32),
                q_col=None if q_col is None else q_col.reshape(C, R // k),
                e_col=None if e_col is None else e_col.reshape(C, R // 32))


def quantize_nvfp4(x, block, outputs=ROWWISE, shape=None, amax=None, sr=None):
    """NVFP4: packed E2M1 pairs, E4M3 block codes and the fp32 tensor scale S.
    `amax` gives the tensor amax A (default: this tensor's own).
    `sr` = (seed, offset) rounds the elements stochastically (1x16 blocks only)."""
    p, dt, keep = _in(x)
    R, C = _shape2(keep, shape)
    br, bc = block
    p_row = np.empty(R * C // 2, np.uint8) if outputs & ROWWISE else None
    c_row = np.empty((R // br) * (C // bc), np.uint8) if outputs & ROWWISE else None
    p_col = np.empty(R * C // 2, np.uint8) if outputs & COLWISE else None
    c_col = None
    if outputs & COLWISE:
        c_col = np.empty(C * (R // 16) if br == 1 else (C // 16) * (R // 16), np.uint8)
    S, A = ctypes.c_float(), ctypes.c_float()
    if sr is not None:
        if block != (1, 16):
            raise ValueError("stochastic rounding is offered for 1x16 blocks")
        a = _load().orc_amax(p, dt, R * C) if amax is None else amax
        rc = _load().orc_quantize_nvfp4_sr_with_amax(p, dt, R, C, outputs, float(np.float32(a)), int(sr[0]),
                                                     int(sr[1]), _ptr(p_row), _ptr(c_row), _ptr(p_col),
                                                     _ptr(c_col), ctypes.byref(S), ctypes.byref(A))
    elif amax is None:
        rc = _load().orc_quantize_nvfp4(p, dt, R, C, br, bc, outputs, _ptr(p_row), _ptr(c_row), _ptr(p_col),
                                        _ptr(c_col), ctypes.byref(S), ctypes.byref(A))
    else:
        rc = _load().orc_quantize_nvfp4_with_amax(p, dt, R, C, br, bc, outputs, float(np.float32(amax)),
                                                  _ptr(p_row), _ptr(c_row), _ptr(p_col), _ptr(c_col),
                                                  ctypes.byref(S), ctypes.byref(A))
    _check(rc, "quantize_nvfp4")
    out = dict(p_row=None if p_row is None else p_row.reshape(R, C // 2),
               c_row=None if c_row is None else c_row.reshape(R // br, C // bc),
               p_col=None if p_col is None else p_col.reshape(C, R // 2),
               S=np.float32(S.value), amax=np.float32(A.value))
    if c_col is not None:
        out["c_col"] = c_col.reshape(C, R // 16) if br == 1 else c_col.reshape(C // 16, R // 16)
    else:
        out["c_col"] = None
    return out


# ---------------------------------------------------------------- stochastic rounding
def philox4x32_10(counter, key):
    """Philox4x32-10 of a 4-word counter and a 2-word key (uint32 words)."""
    c = np.asarray(counter, np.uint32)
    k = np.asarray(key, np.uint32)
    out = np.empty(4, np.uint32)
    _load().orc_philox4x32_10(c.ctypes.data, k.ctypes.data, out.ctypes.data)
    return out


def sr_bits(seed, offset, plane, e):
    """The 16 random bits of element e of an output plane (0 rowwise, 1 colwise)."""
    return int(_load().orc_sr_bits(int(seed), int(offset), int(plane), int(e)))


def encode_e2m1_sr(y, u):
    """Stochastically rounded E2M1 codes of fp32 values y with 16-bit randoms u."""
    y = np.ascontiguousarray(y, dtype=np.float32)
    u = np.ascontiguousarray(u, dtype=np.uint16)
    assert y.shape == u.shape
    q = np.empty(y.size, np.uint8)
    _load().orc_encode_e2m1_sr_array(y.ctypes.data, u.ctypes.data, y.size, q.ctypes.data)
    return q.reshape(y.shape)


def encode_sr(fmt, y, u):
    """Stochastically rounded codes of format fmt (E4M3, E5M2 or E2M1) of fp32
    values y with 16-bit randoms u."""
    y = np.ascontiguousarray(y, dtype=np.float32)
    u = np.ascontiguousarray(u, dtype=np.uint16)
    assert y.shape == u.shape
    q = np.empty(y.size, np.uint8)
    _load().orc_encode_sr_array(int(fmt), y.ctypes.data, u.ctypes.data, y.size, q.ctypes.data)
    return q.reshape(y.shape)


# ---------------------------------------------------------------- random Hadamard transform
def rht16(x, signs):
    """The 16-point RHT of every consecutive 16-element chunk of x (fp32)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert x.size % 16 == 0
    y = np.empty_like(x)
    _load().orc_rht16_array(x.ctypes.data, x.size // 16, int(signs) & 0xFFFF, y.ctypes.data)
    return y


def quantize_nvfp4_rht(x, signs, amax=None, sr=None, shape=None):
    """NVFP4 1x16 colwise copy of the RHT-transformed X^T: dict(p_col [C, R/2],
    c_col [C, R/16], S, amax) with amax that of the transformed tensor."""
    p, dt, keep = _in(x)
    R, C = _shape2(keep, shape)
    p_col = np.empty(R * C // 2, np.uint8)
    c_col = np.empty(C * (R // 16), np.uint8)
    S, A = ctypes.c_float(), ctypes.c_float()
    seed, off = (0, 0) if sr is None else sr
    _check(_load().orc_quantize_nvfp4_rht(p, dt, R, C, int(signs) & 0xFFFF, 0 if amax is None else 1,
                                          0.0 if amax is None else float(np.float32(amax)),
                                          0 if sr is None else 1, int(seed), int(off), _ptr(p_col), _ptr(c_col),
                                          ctypes.byref(S), ctypes.byref(A)), "quantize_nvfp4_rht")
    return dict(p_col=p_col.reshape(C, R // 2), c_col=c_col.reshape(C, R // 16), S=np.float32(S.value),
                amax=np.float32(A.value))


# ---------------------------------------------------------------- dequantize
def dequant_tensor(q, fmt, s):
    q = np.ascontiguousarray(q, dtype=np.uint8)
    y = np.empty(q.size, np.float32)
    _load().orc_dequant_tensor(q.ctypes.data, q.size, fmt, float(np.float32(s)), y.ctypes.data)
    return y.reshape(q.shape)


def dequant_block(q, s, block):
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.float32)
    R, C = q.shape
    y = np.empty(R * C, np.float32)
    _load().orc_dequant_block(q.ctypes.data, s.ctypes.data, R, C, block[0], block[1], y.ctypes.data)
    return y.reshape(R, C)


def dequant_mx(q, codes, fmt=None):
    """MX values: element times 2^(code-127); E2M1 q is packed [R, C/2]."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    fmt = E4M3 if fmt is None else fmt
    R = q.shape[0]
    C = q.shape[1] * (2 if fmt == E2M1 else 1)
    y = np.empty(R * C, np.float32)
    _load().orc_dequant_mx_fmt(q.ctypes.data, codes.ctypes.data, R, C, fmt, y.ctypes.data)
    return y.reshape(R, C)


def dequant_nvfp4(p, codes, S, block):
    p = np.ascontiguousarray(p, dtype=np.uint8)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    R, C2 = p.shape
    y = np.empty(R * C2 * 2, np.float32)
    _load().orc_dequant_nvfp4(p.ctypes.data, codes.ctypes.data, float(np.float32(S)), R, C2 * 2, block[0], block[1],
                              y.ctypes.data)
    return y.reshape(R, C2 * 2)


def f32_to_bf16(y):
    """fp32 -> bf16 bit patterns (uint16), round to nearest even."""
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.shape, np.uint16)
    _load().orc_f32_to_bf16_array(y.ctypes.data, y.size, out.ctypes.data)
    return out


def requant_mx_colwise(q_row, e_row):
    """MXFP8 colwise copy (codes [C,R], E8M0 [C,R/32]) from the rowwise copy alone."""
    q_row = np.ascontiguousarray(q_row, dtype=np.uint8)
    e_row = np.ascontiguousarray(e_row, dtype=np.uint8)
    R, C = q_row.shape
    q_col = np.empty(R * C, np.uint8)
    e_col = np.empty(C * (R // 32), np.uint8)
    _check(_load().orc_requant_mx_colwise(q_row.ctypes.data, e_row.ctypes.data, R, C, q_col.ctypes.data,
                                          e_col.ctypes.data), "requant_mx_colwise")
    return dict(q_col=q_col.reshape(C, R), e_col=e_col.reshape(C, R // 32))


def requant_block_colwise(q_row, s_row):
    """Blockwise 1x128 with power-of-two scales: the colwise copy (codes
    [C,R], fp32 scales [C,R/128]) from the rowwise copy alone."""
    q_row = np.ascontiguousarray(q_row, dtype=np.uint8)
    s_row = np.ascontiguousarray(s_row, dtype=np.float32)
    R, C = q_row.shape
    q_col = np.empty(R * C, np.uint8)
    s_col = np.empty(C * (R // 128), np.float32)
    _check(_load().orc_requant_block_colwise(q_row.ctypes.data, s_row.ctypes.data, R, C, q_col.ctypes.data,
                                             s_col.ctypes.data), "requant_block_colwise")
    return dict(q_col=q_col.reshape(C, R), s_col=s_col.reshape(C, R // 128))
