"""libred: block-level parallel reductions on AMD Instinct MI355X (gfx950).

A thin ctypes binding over the C ABI of libred.so (include/libred.h,
include/libred_ablate.h, include/libred_probe.h). Each function here has the
name of the C entry point it calls and only marshals arguments: it takes
PyTorch tensors on a ROCm device (PyTorch supplies device memory and
streams), passes their data pointers, sizes and a hipStream_t, and raises
RedError on a non-zero status. Every step of every reduction runs in the HIP
kernels of libred.so; there is no other implementation behind this module.

The call is asynchronous on the stream (default: PyTorch's current stream of
the tensor's device); the output tensor is ready once that stream is.
"""
import ctypes
import os

import torch  # first: the HIP runtime PyTorch loads is the one libred.so binds to

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libred.so")

RED_OK = 0
RED_ERR_INVALID_ARG = 1
RED_ERR_NO_DEVICE = 2
RED_ERR_HIP = 3
RED_ERR_ALLOC = 4
RED_ERR_CAPTURE = 5
RED_ERR_SCRATCH = 6
RED_MAX_N = 1 << 40


class RedError(RuntimeError):
    """A red_* call returned a non-zero red_status."""

    def __init__(self, name, status, hip_error):
        self.status = status
        self.hip_error = hip_error
        msg = lib().red_status_string(status).decode()
        super().__init__(f"{name}: {msg} (hip error {hip_error})")


class FlatPolicy(ctypes.Structure):
    _fields_ = [("block", ctypes.c_int), ("blocks_per_cu", ctypes.c_int),
                ("unroll", ctypes.c_int), ("nontemporal", ctypes.c_int),
                ("layout", ctypes.c_int), ("prefetch", ctypes.c_int),
                ("combine", ctypes.c_int)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class RowsPolicy(ctypes.Structure):
    _fields_ = [("block", ctypes.c_int), ("unroll", ctypes.c_int),
                ("nontemporal", ctypes.c_int), ("max_blocks", ctypes.c_int),
                ("split", ctypes.c_int), ("prefetch", ctypes.c_int), ("short_rows", ctypes.c_int),
                ("cover", ctypes.c_int),
                ("defer", ctypes.c_int), ("lines", ctypes.c_int), ("xcd", ctypes.c_int),
                ("max_fold", ctypes.c_int)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class ColsPolicy(ctypes.Structure):
    _fields_ = [("unroll", ctypes.c_int), ("nontemporal", ctypes.c_int),
                ("target_waves", ctypes.c_int), ("vec", ctypes.c_int), ("width", ctypes.c_int),
                ("prefetch", ctypes.c_int), ("fold", ctypes.c_int), ("order", ctypes.c_int),
                ("xcd", ctypes.c_int)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class ReadShape(ctypes.Structure):
    _fields_ = [("block", ctypes.c_int), ("blocks_per_cu", ctypes.c_int), ("unroll", ctypes.c_int),
                ("nontemporal", ctypes.c_int), ("layout", ctypes.c_int)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


_P = ctypes.c_void_p
_Z = ctypes.c_size_t
_I = ctypes.c_int
_S = ctypes.c_int  # red_status

# name -> (restype, argtypes): every entry point declared in include/*.h.
SIGNATURES = {
    "red_sum_f32": (_S, [_P, _Z, _P, _P]),
    "red_sum_i32_i64": (_S, [_P, _Z, _P, _P]),
    "red_sum_f32_noalloc": (_S, [_P, _Z, _P, _P]),
    "red_max_f32": (_S, [_P, _Z, _P, _P]),
    "red_sum_max_f32": (_S, [_P, _Z, _P, _P]),
    "red_min_f32": (_S, [_P, _Z, _P, _P]),
    "red_argmax_f32": (_S, [_P, _Z, _P, _P]),
    "red_argmin_f32": (_S, [_P, _Z, _P, _P]),
    "red_sum_bf16_f32": (_S, [_P, _Z, _P, _P]),
    "red_sum_f16_f32": (_S, [_P, _Z, _P, _P]),
    "red_sum_f64": (_S, [_P, _Z, _P, _P]),
    "red_flat_with": (_S, [_I, _P, _Z, _P, ctypes.POINTER(FlatPolicy), _P]),
    "red_sum_max_f32_with": (_S, [_P, _Z, _P, ctypes.POINTER(FlatPolicy), _P]),
    "red_rows_sum_f32": (_S, [_P, _Z, _Z, _P, _P]),
    "red_rows_max_f32": (_S, [_P, _Z, _Z, _P, _P]),
    "red_rows_sum_f32_ld": (_S, [_P, _Z, _Z, _Z, _P, _P]),
    "red_cols_sum_f32": (_S, [_P, _Z, _Z, _Z, _P, _P]),
    "red_cols_max_f32": (_S, [_P, _Z, _Z, _Z, _P, _P]),
    "red_default_cols_policy": (None, [ctypes.POINTER(ColsPolicy)]),
    "red_cols_sum_f32_with": (_S, [_P, _Z, _Z, _Z, _P, ctypes.POINTER(ColsPolicy), _P]),
    "red_cols_max_f32_with": (_S, [_P, _Z, _Z, _Z, _P, ctypes.POINTER(ColsPolicy), _P]),
    "red_rows_max_f32_ld": (_S, [_P, _Z, _Z, _Z, _P, _P]),
    "red_status_string": (ctypes.c_char_p, [_S]),
    "red_last_hip_error": (_I, []),
    "red_version": (ctypes.c_char_p, []),
    "red_ablate_sum_f32": (_S, [_I, _P, _Z, _P, _Z, _P, _P]),
    "red_ablate_num_partials": (_Z, [_I, _Z]),
    "red_default_flat_policy": (None, [_Z, ctypes.POINTER(FlatPolicy)]),
    "red_sum_f32_partials": (_S, [_P, _Z, _P, _Z, ctypes.POINTER(FlatPolicy), ctypes.POINTER(_Z), _P]),
    "red_default_rows_policy": (None, [ctypes.POINTER(RowsPolicy)]),
    "red_flat_grid": (_Z, [_Z, ctypes.POINTER(FlatPolicy)]),
    "red_sum_f32_with": (_S, [_P, _Z, _P, ctypes.POINTER(FlatPolicy), _P]),
    "red_sum_i32_i64_with": (_S, [_P, _Z, _P, ctypes.POINTER(FlatPolicy), _P]),
    "red_max_f32_with": (_S, [_P, _Z, _P, ctypes.POINTER(FlatPolicy), _P]),
    "red_rows_sum_f32_with": (_S, [_P, _Z, _Z, _Z, _P, ctypes.POINTER(RowsPolicy), _P]),
    "red_rows_max_f32_with": (_S, [_P, _Z, _Z, _Z, _P, ctypes.POINTER(RowsPolicy), _P]),
    "red_probe_copy_f32": (_S, [_P, _P, _Z, _P]),
    "red_probe_read_f32": (_S, [_P, _Z, _P, _P]),
    "red_default_read_shape": (None, [ctypes.POINTER(ReadShape)]),
    "red_probe_read_ceiling": (_S, [_P, _Z, ctypes.POINTER(ReadShape), _P, _P]),
    "red_probe_fill_workspace": (_S, [ctypes.c_uint, _P]),
    "red_default_copy_shape": (None, [ctypes.POINTER(ReadShape)]),
    "red_probe_copy_ceiling": (_S, [_P, _P, _Z, ctypes.POINTER(ReadShape), _P]),
    "red_stream_new_workspace": (_S, [_P]),
    "red_device_info": (_S, [ctypes.POINTER(_I), ctypes.c_char_p, _Z]),
    "red_probe_lds_stride": (_S, [_I, _I, _P, _P]),
    "red_probe_wave_reduce": (_S, [_I, _P, _Z, _P, _P]),
    "red_probe_shfl_down_f32": (_S, [_P, _I, _P, _P]),
}

_lib = None


def lib():
    """The loaded libred.so with argument types set. Raises ImportError if the
    library has not been built (python -m reduction_libred_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run: python -m reduction_libred_amd.build")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(name, status):
    if status != RED_OK:
        raise RedError(name, status, lib().red_last_hip_error())


def _stream_handle(stream, device):
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _input(x, dtype, name):
    if not isinstance(x, torch.Tensor) or x.device.type != "cuda":
        raise TypeError(f"{name}: input must be a tensor on a ROCm device")
    if x.dtype != dtype:
        raise TypeError(f"{name}: input dtype must be {dtype}, got {x.dtype}")
    if not x.is_contiguous():
        raise ValueError(f"{name}: input must be contiguous")


def _output(out, shape, dtype, device, name):
    if out is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if out.dtype != dtype or out.device != device or out.numel() != int(torch.Size(shape).numel()):
        raise ValueError(f"{name}: out must be {dtype} with {torch.Size(shape).numel()} elements on {device}")
    if not out.is_contiguous():
        raise ValueError(f"{name}: out must be contiguous")
    return out


def _policy(cls, p, n=0):
    """A policy struct from None, a struct, or a dict of fields (fields not
    given take the library default for n elements)."""
    if p is None or isinstance(p, cls):
        return p
    if cls is FlatPolicy:
        base = red_default_flat_policy(n)
    elif cls is ColsPolicy:
        base = red_default_cols_policy()
    else:
        base = red_default_rows_policy()
    for k, v in p.items():
        if k not in base.as_dict():
            raise KeyError(f"unknown policy field {k!r}")
        setattr(base, k, int(v))
    return base


# Operation codes of red_flat_with (include/libred_ablate.h).
OPS = {"red_sum_f32": 0, "red_sum_i32_i64": 1, "red_max_f32": 2, "red_min_f32": 3,
       "red_argmax_f32": 4, "red_argmin_f32": 5, "red_sum_bf16_f32": 6, "red_sum_f16_f32": 7,
       "red_sum_f64": 8, "red_sum_max_f32": 9}


def _flat(name, cname, x, out, in_dtype, out_dtype, stream, policy=None, out_shape=()):
    _input(x, in_dtype, name)
    out = _output(out, out_shape, out_dtype, x.device, name)
    with torch.cuda.device(x.device):
        s = _stream_handle(stream, x.device)
        if policy is None:
            st = getattr(lib(), cname)(x.data_ptr(), x.numel(), out.data_ptr(), s)
        else:
            p = _policy(FlatPolicy, policy, x.numel())
            st = lib().red_flat_with(OPS[cname], x.data_ptr(), x.numel(), out.data_ptr(), ctypes.byref(p), s)
    _check(cname, st)
    return out


def red_sum_f32(x, out=None, stream=None, policy=None):
    """Sum of a float32 tensor into a 0-d float32 tensor (float64 inside)."""
    return _flat("red_sum_f32", "red_sum_f32", x, out, torch.float32, torch.float32, stream, policy)


def red_sum_f32_noalloc(x, out=None, stream=None):
    """red_sum_f32 with its block partials in a fixed device array: no
    device allocation. Calls that overlap in time on one device race."""
    return _flat("red_sum_f32_noalloc", "red_sum_f32_noalloc", x, out, torch.float32, torch.float32, stream)


def red_sum_i32_i64(x, out=None, stream=None, policy=None):
    """Exact sum of an int32 tensor into a 0-d int64 tensor."""
    return _flat("red_sum_i32_i64", "red_sum_i32_i64", x, out, torch.int32, torch.int64, stream, policy)


def red_max_f32(x, out=None, stream=None, policy=None):
    """Maximum of a float32 tensor (NaN never wins; empty gives -inf)."""
    return _flat("red_max_f32", "red_max_f32", x, out, torch.float32, torch.float32, stream, policy)


def red_min_f32(x, out=None, stream=None, policy=None):
    """Minimum of a float32 tensor (NaN never wins; empty gives +inf)."""
    return _flat("red_min_f32", "red_min_f32", x, out, torch.float32, torch.float32, stream, policy)


def red_argmax_f32(x, out=None, stream=None, policy=None):
    """Lowest index of the maximum of a float32 tensor (-1 if none) -> 0-d int64."""
    return _flat("red_argmax_f32", "red_argmax_f32", x, out, torch.float32, torch.int64, stream, policy)


def red_argmin_f32(x, out=None, stream=None, policy=None):
    """Lowest index of the minimum of a float32 tensor (-1 if none) -> 0-d int64."""
    return _flat("red_argmin_f32", "red_argmin_f32", x, out, torch.float32, torch.int64, stream, policy)


def _bits16(x, dtype, name):
    # A bfloat16 / float16 tensor is passed as its 16-bit patterns.
    if not isinstance(x, torch.Tensor) or x.dtype != dtype:
        raise TypeError(f"{name}: input must be a {dtype} tensor")
    return x.view(torch.int16)


def red_sum_bf16_f32(x, out=None, stream=None, policy=None):
    """Sum of a bfloat16 tensor into a 0-d float32 tensor (float64 inside)."""
    return _flat("red_sum_bf16_f32", "red_sum_bf16_f32", _bits16(x, torch.bfloat16, "red_sum_bf16_f32"), out,
                 torch.int16, torch.float32, stream, policy)


def red_sum_f16_f32(x, out=None, stream=None, policy=None):
    """Sum of a float16 tensor into a 0-d float32 tensor (float32 per 16-byte load, then float64)."""
    return _flat("red_sum_f16_f32", "red_sum_f16_f32", _bits16(x, torch.float16, "red_sum_f16_f32"), out,
                 torch.int16, torch.float32, stream, policy)


def red_sum_f64(x, out=None, stream=None, policy=None):
    """Sum of a float64 tensor into a 0-d float64 tensor."""
    return _flat("red_sum_f64", "red_sum_f64", x, out, torch.float64, torch.float64, stream, policy)


def red_sum_max_f32(x, out=None, stream=None, policy=None):
    """One pass: float32[3] = (sum, max, sum of |x|)."""
    return _flat("red_sum_max_f32", "red_sum_max_f32", x, out, torch.float32, torch.float32, stream, policy,
                 out_shape=(3,))


def _rows(cname, x, out, stream, policy):
    if not isinstance(x, torch.Tensor) or x.device.type != "cuda" or x.dtype != torch.float32:
        raise TypeError(f"{cname}: input must be a float32 tensor on a ROCm device")
    if x.dim() != 2:
        raise ValueError(f"{cname}: input must be 2-D (rows, cols)")
    rows, cols = x.shape
    # Rows may be spaced apart (a column slice of a wider matrix): the row
    # stride becomes the leading dimension; columns must be unit-stride.
    if rows > 1 and cols > 1 and x.stride(1) != 1:
        raise ValueError(f"{cname}: columns must be contiguous (stride 1)")
    ld = x.stride(0) if (rows > 1 and cols > 0) else cols
    if ld < cols:
        raise ValueError(f"{cname}: rows overlap (row stride {ld} < cols {cols})")
    out = _output(out, (rows,), torch.float32, x.device, cname)
    with torch.cuda.device(x.device):
        s = _stream_handle(stream, x.device)
        if policy is None:
            st = getattr(lib(), cname + "_ld")(x.data_ptr(), rows, cols, ld, out.data_ptr(), s)
        else:
            p = _policy(RowsPolicy, policy)
            st = getattr(lib(), cname + "_with")(x.data_ptr(), rows, cols, ld, out.data_ptr(),
                                                 ctypes.byref(p), s)
    _check(cname, st)
    return out


def red_rows_sum_f32(x, out=None, stream=None, policy=None):
    """Per-row sum of a 2-D float32 tensor with unit-stride columns (rows may
    be spaced apart, e.g. a column slice) -> float32[rows]."""
    return _rows("red_rows_sum_f32", x, out, stream, policy)


def red_rows_max_f32(x, out=None, stream=None, policy=None):
    """Per-row max of a 2-D row-major float32 tensor -> float32[rows]."""
    return _rows("red_rows_max_f32", x, out, stream, policy)


def _cols(cname, x, out, stream, policy):
    if not isinstance(x, torch.Tensor) or x.device.type != "cuda" or x.dtype != torch.float32:
        raise TypeError(f"{cname}: input must be a float32 tensor on a ROCm device")
    if x.dim() != 2:
        raise ValueError(f"{cname}: input must be 2-D (rows, cols)")
    rows, cols = x.shape
    if rows > 1 and cols > 1 and x.stride(1) != 1:
        raise ValueError(f"{cname}: columns must be contiguous (stride 1)")
    ld = x.stride(0) if (rows > 1 and cols > 0) else cols
    if ld < cols:
        raise ValueError(f"{cname}: rows overlap (row stride {ld} < cols {cols})")
    out = _output(out, (cols,), torch.float32, x.device, cname)
    with torch.cuda.device(x.device):
        s = _stream_handle(stream, x.device)
        ptr = x.data_ptr() if rows * cols else 0
        if policy is None:
            st = getattr(lib(), cname)(ptr, rows, cols, ld, out.data_ptr(), s)
        else:
            p = _policy(ColsPolicy, policy)
            st = getattr(lib(), cname + "_with")(ptr, rows, cols, ld, out.data_ptr(), ctypes.byref(p), s)
    _check(cname, st)
    return out


def red_cols_sum_f32(x, out=None, stream=None, policy=None):
    """Per-column sum of a 2-D float32 tensor with unit-stride columns -> float32[cols]."""
    return _cols("red_cols_sum_f32", x, out, stream, policy)


def red_cols_max_f32(x, out=None, stream=None, policy=None):
    """Per-column max of a 2-D float32 tensor with unit-stride columns -> float32[cols]."""
    return _cols("red_cols_max_f32", x, out, stream, policy)


def red_default_cols_policy():
    p = ColsPolicy()
    lib().red_default_cols_policy(ctypes.byref(p))
    return p


def red_ablate_num_partials(rung, n):
    return int(lib().red_ablate_num_partials(rung, n))


def red_ablate_sum_f32(rung, x, partials=None, out=None, stream=None, partials_only=False):
    """Ablation rung 1..6 of the f32 sum. Returns (out, partials); with
    partials_only=True only the rung's kernel runs and out is None."""
    _input(x, torch.float32, "red_ablate_sum_f32")
    n = x.numel()
    np_ = max(red_ablate_num_partials(rung, n), 1)
    if partials is None:
        partials = torch.empty(np_, dtype=torch.float32, device=x.device)
    if not partials_only:
        out = _output(out, (), torch.float32, x.device, "red_ablate_sum_f32")
    with torch.cuda.device(x.device):
        st = lib().red_ablate_sum_f32(rung, x.data_ptr(), n, partials.data_ptr(), partials.numel(),
                                      None if partials_only else out.data_ptr(),
                                      _stream_handle(stream, x.device))
    _check("red_ablate_sum_f32", st)
    return (None if partials_only else out), partials


def red_default_flat_policy(n):
    """The launch shape the single-value entry points use for n elements."""
    p = FlatPolicy()
    lib().red_default_flat_policy(n, ctypes.byref(p))
    return p


def red_default_rows_policy():
    p = RowsPolicy()
    lib().red_default_rows_policy(ctypes.byref(p))
    return p


def red_sum_f32_partials(x, partials=None, policy=None, stream=None):
    """Block partials (float64) of the f32 sum, no final combine. Returns the
    partials tensor trimmed to the number of blocks launched."""
    _input(x, torch.float32, "red_sum_f32_partials")
    p = _policy(FlatPolicy, policy, x.numel())
    cap = red_flat_grid(x.numel(), p)
    if partials is None:
        partials = torch.empty(max(cap, 1), dtype=torch.float64, device=x.device)
    count = ctypes.c_size_t()
    with torch.cuda.device(x.device):
        st = lib().red_sum_f32_partials(x.data_ptr(), x.numel(), partials.data_ptr(), partials.numel(),
                                        ctypes.byref(p) if p is not None else None, ctypes.byref(count),
                                        _stream_handle(stream, x.device))
    _check("red_sum_f32_partials", st)
    return partials[:count.value]


def red_flat_grid(n, policy=None):
    p = _policy(FlatPolicy, policy, n)
    return int(lib().red_flat_grid(n, ctypes.byref(p) if p is not None else None))


def red_probe_copy_f32(x, y, stream=None):
    _input(x, torch.float32, "red_probe_copy_f32")
    _input(y, torch.float32, "red_probe_copy_f32")
    if y.numel() != x.numel():
        raise ValueError("red_probe_copy_f32: x and y differ in size")
    with torch.cuda.device(x.device):
        st = lib().red_probe_copy_f32(x.data_ptr(), y.data_ptr(), x.numel(), _stream_handle(stream, x.device))
    _check("red_probe_copy_f32", st)
    return y


def red_probe_read_f32(x, sink=None, stream=None):
    _input(x, torch.float32, "red_probe_read_f32")
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=x.device)
    with torch.cuda.device(x.device):
        st = lib().red_probe_read_f32(x.data_ptr(), x.numel(), sink.data_ptr(), _stream_handle(stream, x.device))
    _check("red_probe_read_f32", st)
    return sink


def red_default_read_shape():
    """The read probe's default launch shape."""
    p = ReadShape()
    lib().red_default_read_shape(ctypes.byref(p))
    return p


def red_probe_read_ceiling(x, sink=None, shape=None, stream=None):
    """Load-only read of a contiguous tensor (16-byte aligned, a multiple of
    16 bytes) with the given launch shape (a ReadShape, a dict of its fields,
    or None for the default); sink[0] ^= the xor of all its 32-bit words."""
    if not isinstance(x, torch.Tensor) or x.device.type != "cuda" or not x.is_contiguous():
        raise TypeError("red_probe_read_ceiling: x must be a contiguous tensor on a ROCm device")
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=x.device)
    if isinstance(shape, dict):
        base = red_default_read_shape()
        for k, v in shape.items():
            if k not in base.as_dict():
                raise KeyError(f"unknown read shape field {k!r}")
            setattr(base, k, int(v))
        shape = base
    with torch.cuda.device(x.device):
        st = lib().red_probe_read_ceiling(x.data_ptr(), x.numel() * x.element_size(),
                                          ctypes.byref(shape) if shape is not None else None, sink.data_ptr(),
                                          _stream_handle(stream, x.device))
    _check("red_probe_read_ceiling", st)
    return sink


def red_default_copy_shape():
    """The copy probe's default launch shape."""
    p = ReadShape()
    lib().red_default_copy_shape(ctypes.byref(p))
    return p


def red_probe_copy_ceiling(x, y, shape=None, stream=None):
    """y = x (contiguous, 16-byte aligned, a multiple of 16 bytes, same size)
    with the copy probe's launch shape (a ReadShape, a dict of its fields, or
    None for the default)."""
    for t in (x, y):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or not t.is_contiguous():
            raise TypeError("red_probe_copy_ceiling: x and y must be contiguous tensors on a ROCm device")
    nbytes = x.numel() * x.element_size()
    if y.numel() * y.element_size() != nbytes:
        raise ValueError("red_probe_copy_ceiling: x and y differ in size")
    if isinstance(shape, dict):
        base = red_default_copy_shape()
        for k, v in shape.items():
            if k not in base.as_dict():
                raise KeyError(f"unknown copy shape field {k!r}")
            setattr(base, k, int(v))
        shape = base
    with torch.cuda.device(x.device):
        st = lib().red_probe_copy_ceiling(x.data_ptr(), y.data_ptr(), nbytes,
                                          ctypes.byref(shape) if shape is not None else None,
                                          _stream_handle(stream, x.device))
    _check("red_probe_copy_ceiling", st)
    return y


def red_probe_fill_workspace(word, stream=None, device=None):
    """Set every partial slot of the stream's workspace, and its column
    scratch, to the 32-bit `word` (a test of the poison rule)."""
    device = device or torch.device("cuda", torch.cuda.current_device())
    with torch.cuda.device(device):
        st = lib().red_probe_fill_workspace(word & 0xFFFFFFFF, _stream_handle(stream, device))
    _check("red_probe_fill_workspace", st)


def red_stream_new_workspace(stream=None, device=None):
    """Give the stream a fresh workspace (and column scratch), so that graphs
    captured on it from now on do not share buffers with earlier ones."""
    device = device or torch.device("cuda", torch.cuda.current_device())
    with torch.cuda.device(device):
        st = lib().red_stream_new_workspace(_stream_handle(stream, device))
    _check("red_stream_new_workspace", st)


def red_probe_lds_stride(stride, iters, sink, stream=None):
    """LDS bank probe: one wave reads word (lane*stride) mod 4160 (lane/2 for
    stride -1) `iters` times; the sum read is added to int32 tensor sink[0]."""
    with torch.cuda.device(sink.device):
        st = lib().red_probe_lds_stride(stride, iters, sink.data_ptr(), _stream_handle(stream, sink.device))
    _check("red_probe_lds_stride", st)
    return sink


_WAVE_OPS = {"sum_f64": (0, torch.float64), "sum_i64": (1, torch.int64), "max_f32": (2, torch.float32)}


def red_probe_wave_reduce(op, x, out=None, stream=None):
    """One 64-lane DPP wave reduce per group of 64 elements of x (op is
    'sum_f64', 'sum_i64' or 'max_f32'); returns a tensor of x.numel() / 64."""
    code, dt = _WAVE_OPS[op]
    _input(x, dt, "red_probe_wave_reduce")
    if x.numel() % 64:
        raise ValueError("red_probe_wave_reduce: x must hold a multiple of 64 elements")
    out = _output(out, (x.numel() // 64,), dt, x.device, "red_probe_wave_reduce")
    with torch.cuda.device(x.device):
        st = lib().red_probe_wave_reduce(code, x.data_ptr(), x.numel() // 64, out.data_ptr(),
                                         _stream_handle(stream, x.device))
    _check("red_probe_wave_reduce", st)
    return out


def red_probe_shfl_down_f32(x, offset, out=None, stream=None):
    """One 64-lane shuffle-down of the 64 floats in x."""
    _input(x, torch.float32, "red_probe_shfl_down_f32")
    if x.numel() != 64:
        raise ValueError("red_probe_shfl_down_f32: x must hold 64 floats")
    out = _output(out, (64,), torch.float32, x.device, "red_probe_shfl_down_f32")
    with torch.cuda.device(x.device):
        st = lib().red_probe_shfl_down_f32(x.data_ptr(), offset, out.data_ptr(), _stream_handle(stream, x.device))
    _check("red_probe_shfl_down_f32", st)
    return out


def red_device_info():
    """(compute-unit count, architecture name) of the current device."""
    cu = ctypes.c_int()
    buf = ctypes.create_string_buffer(64)
    _check("red_device_info", lib().red_device_info(ctypes.byref(cu), buf, 64))
    return cu.value, buf.value.decode()


def red_version():
    return lib().red_version().decode()
