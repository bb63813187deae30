"""ctypes binding of libmi_bitmask.so (include/mi_bitmask.h).

Argument marshalling only: tensors become device pointers, element strides
and torch's current HIP stream; every step of the apply runs in the
library's kernels.  There is no fallback -- without the built library every
entry point raises.
"""

from __future__ import annotations

import ctypes
import math
import pathlib
from typing import Optional, Sequence, Union

PKG = pathlib.Path(__file__).resolve().parent
LIBRARY = PKG / "libmi_bitmask.so"

MI_DTYPE = {"float32": 0, "float16": 1, "bfloat16": 2}
STATUS = ["MI_OK", "MI_ERR_NULL_POINTER", "MI_ERR_BAD_DTYPE", "MI_ERR_BAD_SHAPE", "MI_ERR_BAD_VOCAB",
          "MI_ERR_BAD_INDICES", "MI_ERR_ALIAS", "MI_ERR_HIP", "MI_ERR_MISALIGNED", "MI_ERR_BAD_VARIANT"]
VARIANT = {"auto": 0, "scalar": 1, "vec": 2, "wronly": 3, "vec_resident": 4}

# every symbol include/mi_bitmask.h declares
EXPORTS = ["mi_apply_bitmask_inplace", "mi_apply_bitmask_out", "mi_apply_bitmask_inplace_ex",
           "mi_apply_bitmask_out_ex", "mi_apply_bitmask_rows", "mi_apply_bitmask_sample",
           "mi_apply_bitmask_sample_ws", "mi_apply_bitmask_sample_noalloc", "mi_sample_workspace_bytes",
           "mi_apply_bitmask_inplace_host", "mi_apply_bitmask_out_host",
           "mi_resolve_vocab_size", "mi_fill_value_bits", "mi_status_string", "mi_last_error_message",
           "mi_host_isa"]

_i64, _p, _dbl = ctypes.c_int64, ctypes.c_void_p, ctypes.c_double
_INPLACE = [_p, ctypes.c_int, _i64, _i64, _i64, _p, _i64, _i64, _i64, _i64, _p, _i64, _dbl]
_OUT = [_p, _i64, _p, ctypes.c_int, _i64, _i64, _i64, _p, _i64, _i64, _i64, _i64, _p, _i64, _dbl]

_lib = None


class SampleParams(ctypes.Structure):
    """mi_sample_params_t."""
    _fields_ = [("temperature", ctypes.c_void_p), ("top_k", ctypes.c_void_p), ("top_p", ctypes.c_void_p),
                ("min_p", ctypes.c_void_p), ("temperature_all", ctypes.c_float), ("top_k_all", ctypes.c_int32),
                ("top_p_all", ctypes.c_float), ("min_p_all", ctypes.c_float), ("seed", ctypes.c_uint64),
                ("offset", ctypes.c_uint64)]


class BitmaskError(RuntimeError):
    """A non-OK status from the library (``status`` holds its name)."""

    def __init__(self, status: int, message: str):
        self.status = STATUS[status] if 0 <= status < len(STATUS) else f"status {status}"
        super().__init__(f"{self.status}: {message}")


def load_library(path: Union[str, pathlib.Path, None] = None) -> ctypes.CDLL:
    """Load (once) and return the C library; raises if it was never built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    so = pathlib.Path(path) if path else LIBRARY
    if not so.exists():
        raise ImportError(f"{so} is missing: build it with `python -m packed_logit_bitmask_amd.build` "
                          "(or __graft_entry__.build())")
    lib = ctypes.CDLL(str(so))
    lib.mi_apply_bitmask_inplace.argtypes = _INPLACE + [_p]
    lib.mi_apply_bitmask_inplace_ex.argtypes = _INPLACE + [ctypes.c_int, _p]
    lib.mi_apply_bitmask_out.argtypes = _OUT + [_p]
    lib.mi_apply_bitmask_out_ex.argtypes = _OUT + [ctypes.c_int, _p]
    lib.mi_apply_bitmask_rows.argtypes = [_p, ctypes.c_int, _i64, _i64, _i64, _p, _i64, _i64, _i64, _i64, _p, _p,
                                          _dbl, _p]
    lib.mi_apply_bitmask_sample.argtypes = [_p, ctypes.c_int, _i64, _i64, _i64, _p, _i64, _i64, _i64, _i64,
                                            ctypes.POINTER(SampleParams), _p, _p]
    lib.mi_apply_bitmask_sample_ws.argtypes = [_p, ctypes.c_int, _i64, _i64, _i64, _p, _i64, _i64, _i64, _i64,
                                               ctypes.POINTER(SampleParams), _p, _p, _i64, _p]
    lib.mi_apply_bitmask_sample_noalloc.argtypes = [_p, ctypes.c_int, _i64, _i64, _i64, _p, _i64, _i64, _i64,
                                                    _i64, ctypes.POINTER(SampleParams), _p, _p]
    lib.mi_sample_workspace_bytes.argtypes = [ctypes.c_int, _i64, _i64]
    lib.mi_sample_workspace_bytes.restype = _i64
    lib.mi_apply_bitmask_inplace_host.argtypes = _INPLACE + [ctypes.c_int]
    lib.mi_apply_bitmask_out_host.argtypes = _OUT + [ctypes.c_int]
    for f in ("mi_apply_bitmask_inplace", "mi_apply_bitmask_inplace_ex", "mi_apply_bitmask_out",
              "mi_apply_bitmask_out_ex", "mi_apply_bitmask_rows", "mi_apply_bitmask_sample",
              "mi_apply_bitmask_sample_ws", "mi_apply_bitmask_sample_noalloc", "mi_apply_bitmask_inplace_host", "mi_apply_bitmask_out_host",
              "mi_resolve_vocab_size", "mi_fill_value_bits"):
        getattr(lib, f).restype = ctypes.c_int
    lib.mi_resolve_vocab_size.argtypes = [_i64, _i64, _i64, ctypes.POINTER(_i64)]
    lib.mi_fill_value_bits.argtypes = [_dbl, ctypes.c_int, ctypes.POINTER(ctypes.c_uint32)]
    lib.mi_status_string.argtypes = [ctypes.c_int]
    lib.mi_status_string.restype = ctypes.c_char_p
    lib.mi_last_error_message.argtypes = []
    lib.mi_last_error_message.restype = ctypes.c_char_p
    lib.mi_host_isa.argtypes = []
    lib.mi_host_isa.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def check(status: int) -> None:
    if status != 0:
        msg = load_library().mi_last_error_message().decode(errors="replace")
        raise BitmaskError(status, msg)


# ----------------------------------------------------------------------------
# host helpers
# ----------------------------------------------------------------------------

def resolve_vocab_size(cols: int, mask_cols: int, vocab_size: Optional[int] = None) -> int:
    out = _i64()
    check(load_library().mi_resolve_vocab_size(cols, mask_cols, -1 if vocab_size is None else vocab_size,
                                               ctypes.byref(out)))
    return out.value


def host_isa() -> str:
    """The loop the host-memory entry points run: "avx512" or "portable"."""
    return load_library().mi_host_isa().decode()


def fill_value_bits(fill_value: float, dtype: str) -> int:
    out = ctypes.c_uint32()
    check(load_library().mi_fill_value_bits(float(fill_value), MI_DTYPE[dtype], ctypes.byref(out)))
    return out.value


# ----------------------------------------------------------------------------
# tensor marshalling
# ----------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_name(t) -> str:
    torch = _torch()
    names = {torch.float32: "float32", torch.float16: "float16", torch.bfloat16: "bfloat16"}
    if t.dtype not in names:
        raise TypeError(f"logits dtype {t.dtype} is not float32, float16 or bfloat16")
    return names[t.dtype]


def _as_rows(t, what: str):
    """A [rows, cols] view of ``t`` (leading dims flattened), last dim contiguous."""
    if t.dim() == 1:
        t = t.unsqueeze(0)
    if t.dim() > 2:
        try:
            t = t.view(-1, t.shape[-1])
        except RuntimeError as e:
            raise ValueError(f"{what}: leading dimensions cannot be flattened without a copy") from e
    if t.shape[-1] > 1 and t.stride(-1) != 1:
        raise ValueError(f"{what}: last dimension must be contiguous")
    return t


def _row_stride(t) -> int:
    return t.stride(0) if t.shape[0] > 1 else max(t.shape[1], 1)


def _stream_handle(device, stream) -> int:
    torch = _torch()
    s = torch.cuda.current_stream(device) if stream is None else stream
    return s.cuda_stream


def _on(stream):
    """The context every device entry point runs its marshalling in.

    With an explicit ``stream``, the helper tensors a call makes (index,
    gate and per-row parameter casts, the outputs and the workspace it
    allocates) are made on that stream: their copies are enqueued there,
    ahead of the library's kernels, and the allocator ties their memory to
    that stream, so it is never handed out again while the kernels may still
    use it.  The caller's own tensors must be ready on ``stream``, as for any
    call that takes one.
    """
    import contextlib
    return contextlib.nullcontext() if stream is None else _torch().cuda.stream(stream)


def _indices_arg(indices, device, limit: int):
    """(pointer, count, keepalive) for an index list or int tensor."""
    torch = _torch()
    if indices is None:
        return None, 0, None
    if isinstance(indices, torch.Tensor):
        t = indices
        if t.dim() != 1:
            raise ValueError("indices must be 1-D")
        if t.dtype != torch.int32 or t.device != device or (t.numel() > 1 and t.stride(0) != 1):
            t = t.to(device=device, dtype=torch.int32).contiguous()
    else:
        lst = [int(i) for i in indices]
        bad = [i for i in lst if not 0 <= i < limit]
        if bad:
            raise ValueError(f"indices {bad[:5]} outside [0, {limit})")
        t = torch.tensor(lst, dtype=torch.int32, device=device)
    # An empty list still needs a non-NULL pointer: NULL means "every row".
    # The library never dereferences it when the count is 0.
    ptr = t.data_ptr() if t.numel() else _EMPTY_LIST_PTR
    return ptr, t.numel(), t


_EMPTY_LIST_PTR = 256


def _check_mask(mask, device):
    torch = _torch()
    if not isinstance(mask, torch.Tensor) or mask.dtype != torch.int32:
        raise TypeError("bitmask must be an int32 tensor")
    if mask.device != device:
        raise ValueError(f"bitmask is on {mask.device}, logits on {device}: copy the bitmask to the GPU first")
    return _as_rows(mask, "bitmask")


def mi_apply_bitmask_inplace(logits, mask, vocab_size: Optional[int] = None,
                             indices: Union[None, Sequence[int], "torch.Tensor"] = None,
                             fill_value: float = -math.inf, *, variant: str = "auto", stream=None):
    """In-place apply on a GPU tensor; returns ``logits``.

    XGrammar "Bitmask Operations", apply_token_bitmask_inplace semantics with
    the Modular MAX fill_value: masked entries of the processed rows below
    the vocab size become ``fill_value`` (default -inf).
    """
    if not logits.is_cuda:
        raise ValueError("logits must be on the GPU (the library has no CPU path)")
    lib = load_library()
    L = _as_rows(logits, "logits")
    M = _check_mask(mask, logits.device)
    with _on(stream):
        ip, n, keep = _indices_arg(indices, logits.device, min(L.shape[0], M.shape[0]))
        args = (L.data_ptr(), MI_DTYPE[_dtype_name(L)], L.shape[0], L.shape[1], _row_stride(L),
                M.data_ptr(), M.shape[0], M.shape[1], _row_stride(M),
                -1 if vocab_size is None else int(vocab_size), ip, n, float(fill_value))
        st = _stream_handle(logits.device, stream)
        if variant == "auto":
            check(lib.mi_apply_bitmask_inplace(*args, st))
        else:
            check(lib.mi_apply_bitmask_inplace_ex(*args, VARIANT[variant], st))
    del keep
    return logits


def mi_apply_bitmask_rows(logits, mask, row_needs_mask=None, vocab_size: Optional[int] = None,
                          fill_value: float = -math.inf, *, report: bool = False, stream=None):
    """Gated in-place apply; returns the uint8 per-row report when ``report``.

    TensorRT-Edge-LLM "Guided Decoder": logits may be [activeBatchSize,
    rowsPerSlot, vocab] (leading dims are flattened into rows); a zero entry
    of ``row_needs_mask`` (int8/bool, one per row) leaves that row alone.  The
    report holds 1 where a row still admits one of its first V tokens, 0 for
    an unsatisfiable row.
    """
    torch = _torch()
    if not logits.is_cuda:
        raise ValueError("logits must be on the GPU (the library has no CPU path for this call)")
    lib = load_library()
    L = _as_rows(logits, "logits")
    M = _check_mask(mask, logits.device)
    with _on(stream):
        gate = None
        if row_needs_mask is not None:
            gate = row_needs_mask.reshape(-1)
            if gate.numel() != L.shape[0]:
                raise ValueError(f"row_needs_mask has {gate.numel()} entries for {L.shape[0]} rows")
            gate = gate.to(device=logits.device, dtype=torch.int8).contiguous()
        out = torch.empty(L.shape[0], dtype=torch.uint8, device=logits.device) if report else None
        check(lib.mi_apply_bitmask_rows(
            L.data_ptr(), MI_DTYPE[_dtype_name(L)], L.shape[0], L.shape[1], _row_stride(L),
            M.data_ptr(), M.shape[0], M.shape[1], _row_stride(M), -1 if vocab_size is None else int(vocab_size),
            None if gate is None else gate.data_ptr(), None if out is None else out.data_ptr(), float(fill_value),
            _stream_handle(logits.device, stream)))
    return out


def mi_apply_bitmask_sample(logits, mask=None, vocab_size: Optional[int] = None, *, temperature=1.0, top_k=0,
                            top_p=1.0, min_p=0.0, seed: int = 0, offset: int = 0, out=None, stream=None,
                            workspace="auto"):
    """One token per row (int64 [rows]) from the masked, filtered softmax.

    logits-processor page, "Ops: sample": per-row temperature (<= 0: argmax),
    top-k / top-p / min-p intersected as one keep threshold, Gumbel-max draw
    from a Philox stream keyed by (seed, row, offset).  Each of temperature,
    top_k, top_p and min_p is a scalar for every row or a length-rows tensor.
    With ``mask`` (int32 [rows, ceil(V/32)] on the same GPU) masked tokens
    take no part; the logits are not modified.  A row with no allowed token
    gets -1.

    ``workspace``: device memory that lets a small batch of filtered bf16 or
    fp16 rows spread over many compute units, and a large one hand out its
    dense rows first (``mi_apply_bitmask_sample_ws``; the tokens are the same
    either way).  "auto" allocates one when the call can use it, None uses
    none, and a device tensor is used as it is (at least
    ``sample_workspace_bytes`` bytes; calls sharing it must not overlap).
    """
    torch = _torch()
    lib = load_library()
    with _on(stream):
        c = _SampleCall(logits, mask, vocab_size, temperature, top_k, top_p, min_p, seed, offset, out)
        wp, wn = None, 0
        if isinstance(workspace, str):
            if workspace != "auto":
                raise ValueError('workspace must be "auto", None or a device tensor')
            need = lib.mi_sample_workspace_bytes(c.dt, c.rows, c.vocab)
            if need > 0 and c.may_filter:
                ws = torch.empty(need, dtype=torch.uint8, device=logits.device)
                c.keep.append(ws)
                wp, wn = ws.data_ptr(), need
        elif workspace is not None:
            if (not isinstance(workspace, torch.Tensor) or workspace.device != logits.device
                    or not workspace.is_contiguous()):
                raise ValueError("workspace must be a contiguous tensor on the logits' GPU")
            wp, wn = workspace.data_ptr(), workspace.numel() * workspace.element_size()
        check(lib.mi_apply_bitmask_sample_ws(*c.head(), wp, wn, _stream_handle(logits.device, stream)))
    return c.out


def mi_apply_bitmask_sample_noalloc(logits, mask=None, vocab_size: Optional[int] = None, *, temperature=1.0,
                                    top_k=0, top_p=1.0, min_p=0.0, seed: int = 0, offset: int = 0, out=None,
                                    stream=None):
    """As :func:`mi_apply_bitmask_sample`, through the entry point that
    allocates nothing: a small split batch uses the library's own device
    scratch instead of a workspace.  Calls that overlap on one GPU race on
    that scratch.  The binding itself allocates only what it must convert:
    pass ``out`` (int64, one per row) and per-row parameters already of the
    C types (float32, int32) on the GPU, or scalars, to allocate nothing.
    """
    lib = load_library()
    with _on(stream):
        c = _SampleCall(logits, mask, vocab_size, temperature, top_k, top_p, min_p, seed, offset, out)
        check(lib.mi_apply_bitmask_sample_noalloc(*c.head(), _stream_handle(logits.device, stream)))
    return c.out


class _SampleCall:
    """The marshalled arguments of one sampler call (run inside ``_on``)."""

    def __init__(self, logits, mask, vocab_size, temperature, top_k, top_p, min_p, seed, offset, out):
        torch = _torch()
        if not logits.is_cuda:
            raise ValueError("logits must be on the GPU")
        self.L = L = _as_rows(logits, "logits")
        self.rows = rows = L.shape[0]
        self.keep = []

        def per_row(v, dtype, name):
            """(device pointer, 0) for a per-row tensor, (None, v) for a scalar."""
            if isinstance(v, torch.Tensor):
                t = v.reshape(-1).to(device=logits.device, dtype=dtype).contiguous()
                if t.numel() != rows:
                    raise ValueError(f"{name} has {t.numel()} entries for {rows} rows")
                self.keep.append(t)
                return t.data_ptr(), 0
            return None, v

        prm = self.prm = SampleParams()
        prm.temperature, v = per_row(temperature, torch.float32, "temperature")
        prm.temperature_all = float(v)
        prm.top_k, v = per_row(top_k, torch.int32, "top_k")
        prm.top_k_all = int(v)
        prm.top_p, v = per_row(top_p, torch.float32, "top_p")
        prm.top_p_all = float(v)
        prm.min_p, v = per_row(min_p, torch.float32, "min_p")
        prm.min_p_all = float(v)
        prm.seed = int(seed) & 0xFFFFFFFFFFFFFFFF
        prm.offset = int(offset) & 0xFFFFFFFFFFFFFFFF
        self.may_filter = any(isinstance(v, torch.Tensor) for v in (top_k, top_p, min_p)) or (
            int(top_k) > 0 or float(top_p) < 1.0 or float(min_p) > 0.0)
        if out is None:
            out = torch.empty(rows, dtype=torch.int64, device=logits.device)
        if (out.dtype != torch.int64 or out.numel() != rows or not out.is_contiguous()
                or out.device != logits.device):
            raise ValueError("out must be a contiguous int64 tensor with one entry per row, on the logits' GPU")
        self.out = out
        self.vocab_arg = -1 if vocab_size is None else int(vocab_size)
        if mask is not None:
            M = _check_mask(mask, logits.device)
            self.m = (M.data_ptr(), M.shape[0], M.shape[1], _row_stride(M))
            # the apply's vocab-size rule, from the library
            self.vocab = resolve_vocab_size(L.shape[1], M.shape[1], vocab_size)
        else:
            self.m = (None, 0, 0, 0)
            # without a mask every token below the given vocab size (else the
            # row width) takes part; the call itself rejects a bad value
            self.vocab = L.shape[1] if vocab_size is None else max(int(vocab_size), 0)
        self.dt = MI_DTYPE[_dtype_name(L)]

    def head(self):
        """The arguments every sampler entry point starts with, up to ``tokens``."""
        L = self.L
        return (L.data_ptr(), self.dt, self.rows, L.shape[1], _row_stride(L), *self.m, self.vocab_arg,
                ctypes.byref(self.prm), self.out.data_ptr())


def sample_workspace_bytes(dtype, rows: int, vocab: int) -> int:
    """Bytes of workspace ``mi_apply_bitmask_sample`` can use for ``rows`` rows of
    ``vocab`` tokens of a torch ``dtype`` (0: none is used)."""
    torch = _torch()
    names = {torch.float32: "float32", torch.float16: "float16", torch.bfloat16: "bfloat16"}
    if dtype not in names:
        raise TypeError(f"unsupported dtype {dtype}")
    return int(load_library().mi_sample_workspace_bytes(MI_DTYPE[names[dtype]], int(rows), int(vocab)))


def mi_apply_bitmask_out(logits, mask, out=None, vocab_size: Optional[int] = None,
                         indices: Union[None, Sequence[int], "torch.Tensor"] = None,
                         fill_value: float = -math.inf, *, variant: str = "auto", stream=None):
    """Out-of-place apply (Modular MAX "apply_packed_bitmask"); returns ``out``.

    ``out`` defaults to a new tensor shaped like ``logits``.  Elements outside
    the processed region are copies of ``logits``.
    """
    torch = _torch()
    if not logits.is_cuda:
        raise ValueError("logits must be on the GPU (the library has no CPU path)")
    lib = load_library()
    with _on(stream):
        if out is None:
            out = torch.empty_like(logits, memory_format=torch.contiguous_format)
        if out.dtype != logits.dtype or out.shape != logits.shape or out.device != logits.device:
            raise ValueError("out must match logits in dtype, shape and device")
        L = _as_rows(logits, "logits")
        O = _as_rows(out, "out")
        M = _check_mask(mask, logits.device)
        ip, n, keep = _indices_arg(indices, logits.device, min(L.shape[0], M.shape[0]))
        args = (O.data_ptr(), _row_stride(O), L.data_ptr(), MI_DTYPE[_dtype_name(L)], L.shape[0], L.shape[1],
                _row_stride(L), M.data_ptr(), M.shape[0], M.shape[1], _row_stride(M),
                -1 if vocab_size is None else int(vocab_size), ip, n, float(fill_value))
        st = _stream_handle(logits.device, stream)
        if variant == "auto":
            check(lib.mi_apply_bitmask_out(*args, st))
        else:
            check(lib.mi_apply_bitmask_out_ex(*args, VARIANT[variant], st))
    del keep
    return out


# ----------------------------------------------------------------------------
# host-memory (CPU tensor) entry points
# ----------------------------------------------------------------------------

def _check_host_mask(mask):
    torch = _torch()
    if not isinstance(mask, torch.Tensor) or mask.dtype != torch.int32:
        raise TypeError("bitmask must be an int32 tensor")
    return _as_rows(mask, "bitmask")


def _host_indices(indices):
    torch = _torch()
    if indices is None:
        return None, 0, None
    t = torch.as_tensor(indices if isinstance(indices, torch.Tensor) else list(indices), dtype=torch.int32)
    t = t.to("cpu").contiguous().reshape(-1)
    return (t.data_ptr() if t.numel() else _EMPTY_LIST_PTR), t.numel(), t


def mi_apply_bitmask_inplace_host(logits, mask, vocab_size: Optional[int] = None, indices=None,
                                  fill_value: float = -math.inf, *, num_threads: int = 0):
    """In-place apply on CPU tensors (native host code, not the GPU kernels)."""
    if logits.is_cuda or mask.is_cuda:
        raise ValueError("the host entry point takes CPU tensors only")
    lib = load_library()
    L = _as_rows(logits, "logits")
    M = _check_host_mask(mask)
    ip, n, keep = _host_indices(indices)
    check(lib.mi_apply_bitmask_inplace_host(
        L.data_ptr(), MI_DTYPE[_dtype_name(L)], L.shape[0], L.shape[1], _row_stride(L),
        M.data_ptr(), M.shape[0], M.shape[1], _row_stride(M),
        -1 if vocab_size is None else int(vocab_size), ip, n, float(fill_value), int(num_threads)))
    del keep
    return logits


def mi_apply_bitmask_out_host(logits, mask, out=None, vocab_size: Optional[int] = None, indices=None,
                              fill_value: float = -math.inf, *, num_threads: int = 0):
    """Out-of-place apply on CPU tensors (native host code)."""
    torch = _torch()
    if logits.is_cuda or mask.is_cuda or (out is not None and out.is_cuda):
        raise ValueError("the host entry point takes CPU tensors only")
    lib = load_library()
    if out is None:
        out = torch.empty_like(logits, memory_format=torch.contiguous_format)
    if out.dtype != logits.dtype or out.shape != logits.shape:
        raise ValueError("out must match logits in dtype and shape")
    L = _as_rows(logits, "logits")
    O = _as_rows(out, "out")
    M = _check_host_mask(mask)
    ip, n, keep = _host_indices(indices)
    check(lib.mi_apply_bitmask_out_host(
        O.data_ptr(), _row_stride(O), L.data_ptr(), MI_DTYPE[_dtype_name(L)], L.shape[0], L.shape[1],
        _row_stride(L), M.data_ptr(), M.shape[0], M.shape[1], _row_stride(M),
        -1 if vocab_size is None else int(vocab_size), ip, n, float(fill_value), int(num_threads)))
    del keep
    return out
