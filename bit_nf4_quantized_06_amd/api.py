"""Python binding of the C ABI, one function per entry point, same names.

Argument marshalling only: torch tensors supply device memory and the
current HIP stream; every step of the computation runs in the library's
kernels.  bf16 tensors are passed as their bit patterns.
"""
from __future__ import annotations

import ctypes
import functools
import inspect
from dataclasses import dataclass

import torch

from . import _lib


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _as_torch_stream(stream):
    if isinstance(stream, torch.cuda.Stream):
        return stream
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return torch.cuda.ExternalStream(handle)


def _stream_scoped(fn):
    """Run `fn` with the caller's `stream` as torch's current stream.

    Every output and workspace the binding allocates for a call is then taken
    from the caching allocator's pool of the stream the kernels run on: a
    workspace released when the call returns can only be handed to a later
    allocation on that same stream, whose work is ordered after these kernels.
    (Allocated on another stream, the block could be reused by that stream
    while the kernels still read and write it.)"""
    sig = inspect.signature(fn)
    pos = list(sig.parameters).index("stream")

    @functools.wraps(fn)
    def wrapper(*args, **kw):
        # fast path (no signature binding): no stream given
        stream = args[pos] if len(args) > pos else kw.get("stream")
        if stream is None:
            return fn(*args, **kw)
        ba = sig.bind(*args, **kw)
        ba.arguments["stream"] = None
        with torch.cuda.stream(_as_torch_stream(stream)):
            return fn(*ba.args, **ba.kwargs)
    return wrapper


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, shape: tuple, device) -> None:
    if t.dtype == dtype and t.shape == shape and t.device == device and t.is_contiguous():
        return
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name}: expected device {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


@dataclass
class NF4Weight:
    """Packed 4-bit weight: the four device buffers of qlora_nf4_weight and
    its format (quant_type "nf4" or "int4", double_quant, compute_dtype
    "bf16" or "fp16").  Without double quantisation absmax_scale holds the
    float32 block constants and absmax_code, absmax_offset are empty."""
    rows: int
    cols: int
    codes: torch.Tensor          # uint8 [rows * cols / 2]
    absmax_code: torch.Tensor    # uint8 [n_b]     (E4M3 bit patterns)
    absmax_scale: torch.Tensor   # float32 [n_g]   ([n_b] without double quantisation)
    absmax_offset: torch.Tensor  # float32 [1]
    quant_type: str = "nf4"
    double_quant: bool = True
    compute_dtype: str = "bf16"

    @staticmethod
    def _init(d, rows, cols, quant_type, double_quant, compute_dtype):
        lib = _lib.load()
        _lib.check("qlora_nf4_weight_init_ex",
                   lib.qlora_nf4_weight_init_ex(ctypes.byref(d), rows, cols,
                                                _lib.QUANT_TYPES[quant_type], int(bool(double_quant)),
                                                _lib.COMPUTE_DTYPES[compute_dtype]))

    @staticmethod
    def empty(rows: int, cols: int, device=None, quant_type: str = "nf4",
              double_quant: bool = True, compute_dtype: str = "bf16") -> "NF4Weight":
        lib = _lib.load()
        d = _lib.Nf4WeightDesc()
        NF4Weight._init(d, rows, cols, quant_type, double_quant, compute_dtype)
        sizes = [ctypes.c_size_t() for _ in range(4)]
        _lib.check("qlora_nf4_weight_buffer_sizes",
                   lib.qlora_nf4_weight_buffer_sizes(ctypes.byref(d),
                                                     *[ctypes.byref(s) for s in sizes]))
        device = torch.device("cuda", torch.cuda.current_device()) if device is None else device
        return NF4Weight(
            rows, cols,
            torch.empty(sizes[0].value, dtype=torch.uint8, device=device),
            torch.empty(sizes[1].value, dtype=torch.uint8, device=device),
            torch.empty(sizes[2].value // 4, dtype=torch.float32, device=device),
            torch.empty(sizes[3].value // 4, dtype=torch.float32, device=device),
            quant_type, bool(double_quant), compute_dtype,
        )

    @property
    def device(self):
        return self.codes.device

    @property
    def dtype16(self) -> torch.dtype:
        """torch dtype of the 16-bit tensors that go with this weight."""
        return torch.float16 if self.compute_dtype == "fp16" else torch.bfloat16

    def descriptor(self) -> _lib.Nf4WeightDesc:
        """The C descriptor of this weight, built once and rebuilt only when a
        field changes (a call's host work stays small next to its kernels)."""
        key = (self.rows, self.cols, self.quant_type, self.double_quant, self.compute_dtype,
               self.codes.data_ptr(), self.absmax_code.data_ptr(),
               self.absmax_scale.data_ptr(), self.absmax_offset.data_ptr())
        cached = self.__dict__.get("_desc")
        if cached is not None and cached[0] == key:
            return cached[1]
        d = _lib.Nf4WeightDesc()
        NF4Weight._init(d, self.rows, self.cols, self.quant_type, self.double_quant,
                        self.compute_dtype)
        d.codes, d.absmax_code, d.absmax_scale, d.absmax_offset = key[5:]
        self.__dict__["_desc"] = (key, d)
        return d


def _bits(t: torch.Tensor) -> torch.Tensor:
    """bf16 tensor -> same storage viewed as int16 bit patterns."""
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


@_stream_scoped
def qlora_nf4_quantize(W: torch.Tensor, out: NF4Weight | None = None,
                       workspace: torch.Tensor | None = None, stream=None,
                       quant_type: str = "nf4", double_quant: bool = True,
                       compute_dtype: str = "bf16") -> NF4Weight:
    """Blockwise 4-bit quantisation of a float32 [rows, cols] weight
    (qlora_nf4_quantize): NF4 + double quantisation by default; the format
    arguments apply when `out` is not given (else out's format is used)."""
    lib = _lib.load()
    rows, cols = W.shape
    if out is None:
        out = NF4Weight.empty(rows, cols, W.device, quant_type, double_quant, compute_dtype)
    _need(W, "W", torch.float32, (rows, cols), out.device)
    ws_bytes = lib.qlora_nf4_quantize_workspace(rows, cols)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=W.device)
    desc = out.descriptor()
    _lib.check("qlora_nf4_quantize",
               lib.qlora_nf4_quantize(W.data_ptr(), ctypes.byref(desc), workspace.data_ptr(),
                                      workspace.numel(), _stream(stream)))
    return out


@_stream_scoped
def qlora_nf4_dequantize(w: NF4Weight, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """[rows, cols] dequantised weight in the weight's compute dtype
    (qlora_nf4_dequantize)."""
    lib = _lib.load()
    if out is None:
        out = torch.empty(w.rows, w.cols, dtype=w.dtype16, device=w.device)
    _need(out, "out", w.dtype16, (w.rows, w.cols), w.device)
    desc = w.descriptor()
    _lib.check("qlora_nf4_dequantize",
               lib.qlora_nf4_dequantize(ctypes.byref(desc), out.data_ptr(), _stream(stream)))
    return out


@_stream_scoped
def qlora_nf4_merge(w: NF4Weight, A: torch.Tensor, B: torch.Tensor, alpha: float,
                    out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """[rows, cols] weight with the adapter folded in (qlora_nf4_merge):
    round16(dequant(W) + (alpha/r) B A) in the weight's compute dtype."""
    lib = _lib.load()
    r = A.shape[0]
    dt = w.dtype16
    _need(A, "A", dt, (r, w.cols), w.device)
    _need(B, "B", dt, (w.rows, r), w.device)
    if out is None:
        out = torch.empty(w.rows, w.cols, dtype=dt, device=w.device)
    _need(out, "out", dt, (w.rows, w.cols), w.device)
    desc = w.descriptor()
    _lib.check("qlora_nf4_merge",
               lib.qlora_nf4_merge(ctypes.byref(desc), A.data_ptr(), B.data_ptr(), int(r),
                                   float(alpha), out.data_ptr(), _stream(stream)))
    return out


def qlora_adamw_step(param: torch.Tensor, exp_avg: torch.Tensor, exp_avg_sq: torch.Tensor,
                     grad: torch.Tensor, step: int, lr: float, beta1: float = 0.9,
                     beta2: float = 0.999, eps: float = 1e-8, weight_decay: float = 0.0,
                     param_bf16: torch.Tensor | None = None, stream=None) -> None:
    """One AdamW step in place on float32 param / exp_avg / exp_avg_sq
    (qlora_adamw_step); param_bf16, if given, receives the bf16 copy."""
    lib = _lib.load()
    n = param.numel()
    dev = param.device
    for t, name in ((param, "param"), (exp_avg, "exp_avg"), (exp_avg_sq, "exp_avg_sq"),
                    (grad, "grad")):
        _need(t, name, torch.float32, tuple(param.shape), dev)
    if param_bf16 is not None:
        _need(param_bf16, "param_bf16", torch.bfloat16, tuple(param.shape), dev)
    _lib.check("qlora_adamw_step",
               lib.qlora_adamw_step(param.data_ptr(), exp_avg.data_ptr(), exp_avg_sq.data_ptr(),
                                    grad.data_ptr(),
                                    param_bf16.data_ptr() if param_bf16 is not None else None,
                                    int(n), int(step), float(lr), float(beta1), float(beta2),
                                    float(eps), float(weight_decay), _stream(stream)))


def qlora_adamw_step16(param: torch.Tensor, exp_avg: torch.Tensor, exp_avg_sq: torch.Tensor,
                       grad: torch.Tensor, step: int, lr: float, param16: torch.Tensor,
                       beta1: float = 0.9, beta2: float = 0.999, eps: float = 1e-8,
                       weight_decay: float = 0.0, stream=None) -> None:
    """qlora_adamw_step16: the AdamW step with the 16-bit copy written in
    param16's dtype (torch.bfloat16 or torch.float16, the compute dtype)."""
    lib = _lib.load()
    n = param.numel()
    dev = param.device
    for t, name in ((param, "param"), (exp_avg, "exp_avg"), (exp_avg_sq, "exp_avg_sq"),
                    (grad, "grad")):
        _need(t, name, torch.float32, tuple(param.shape), dev)
    if param16.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError(f"param16: expected bfloat16 or float16, got {param16.dtype}")
    _need(param16, "param16", param16.dtype, tuple(param.shape), dev)
    cd = _lib.COMPUTE_DTYPES["fp16" if param16.dtype == torch.float16 else "bf16"]
    _lib.check("qlora_adamw_step16",
               lib.qlora_adamw_step16(param.data_ptr(), exp_avg.data_ptr(), exp_avg_sq.data_ptr(),
                                      grad.data_ptr(), param16.data_ptr(), cd, int(n), int(step),
                                      float(lr), float(beta1), float(beta2), float(eps),
                                      float(weight_decay), _stream(stream)))


@functools.lru_cache(maxsize=256)
def qlora_linear_workspace(T: int, rows: int, cols: int, r: int, is_bwd: bool) -> int:
    return int(_lib.load().qlora_linear_workspace(T, rows, cols, r, int(bool(is_bwd))))


def qlora_set_pre_dequant_min_tokens(min_tokens: int) -> int:
    """Token count from which qlora_linear_* dequantise the weight once per
    call into their workspace (process-wide; returns the previous value)."""
    prev = int(_lib.load().qlora_set_pre_dequant_min_tokens(int(min_tokens)))
    if prev < 0:
        raise ValueError("min_tokens must be >= 0")
    return prev


def qlora_pre_dequant_min_tokens() -> int:
    return int(_lib.load().qlora_pre_dequant_min_tokens())


@_stream_scoped
def qlora_linear_fwd(w: NF4Weight, X: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                     alpha: float, Y: torch.Tensor | None = None,
                     U_save: torch.Tensor | None = None, save_u: bool = True,
                     workspace: torch.Tensor | None = None, stream=None):
    """Y = X dequant(W)^T + (alpha/r) (X A^T) B^T (qlora_linear_fwd).

    Returns (Y, U) with U = X A^T in bf16 (None when save_u is False and no
    U_save buffer is given).
    """
    lib = _lib.load()
    T, K = X.shape
    r = A.shape[0]
    dev = w.device
    _need(X, "X", w.dtype16, (T, w.cols), dev)
    _need(A, "A", w.dtype16, (r, w.cols), dev)
    _need(B, "B", w.dtype16, (w.rows, r), dev)
    if Y is None:
        Y = torch.empty(T, w.rows, dtype=w.dtype16, device=dev)
    _need(Y, "Y", w.dtype16, (T, w.rows), dev)
    if U_save is None and save_u:
        U_save = torch.empty(T, r, dtype=w.dtype16, device=dev)
    if U_save is not None:
        _need(U_save, "U_save", w.dtype16, (T, r), dev)
    if workspace is None:
        ws_bytes = qlora_linear_workspace(T, w.rows, w.cols, r, False)
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    desc = w.descriptor()
    _lib.check("qlora_linear_fwd",
               lib.qlora_linear_fwd(ctypes.byref(desc), X.data_ptr(), T, A.data_ptr(),
                                    B.data_ptr(), r, float(alpha), Y.data_ptr(), _ptr(U_save),
                                    workspace.data_ptr(), workspace.numel(), _stream(stream)))
    return Y, U_save


def qlora_linear_fwd_noalloc(w: NF4Weight, X: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                             alpha: float, Y: torch.Tensor, U_save: torch.Tensor | None = None,
                             stream=None):
    """qlora_linear_fwd_noalloc: the forward with the library's fixed device
    array as workspace (for callers that cannot allocate, e.g. under graph
    capture).  Y (and U_save, if wanted) must be given; nothing is allocated."""
    lib = _lib.load()
    T = X.shape[0]
    r = A.shape[0]
    dev = w.device
    _need(X, "X", w.dtype16, (T, w.cols), dev)
    _need(A, "A", w.dtype16, (r, w.cols), dev)
    _need(B, "B", w.dtype16, (w.rows, r), dev)
    _need(Y, "Y", w.dtype16, (T, w.rows), dev)
    if U_save is not None:
        _need(U_save, "U_save", w.dtype16, (T, r), dev)
    desc = w.descriptor()
    _lib.check("qlora_linear_fwd_noalloc",
               lib.qlora_linear_fwd_noalloc(ctypes.byref(desc), X.data_ptr(), T, A.data_ptr(),
                                            B.data_ptr(), r, float(alpha), Y.data_ptr(),
                                            _ptr(U_save), _stream(stream)))
    return Y, U_save


@_stream_scoped
def qlora_linear_bwd(w: NF4Weight, X: torch.Tensor, dY: torch.Tensor, A: torch.Tensor,
                     B: torch.Tensor, alpha: float, U_saved: torch.Tensor | None = None,
                     dX: torch.Tensor | None = None, dA: torch.Tensor | None = None,
                     dB: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                     stream=None):
    """dX (bf16), dA and dB (float32) of the layer; no dW (qlora_linear_bwd)."""
    lib = _lib.load()
    T = X.shape[0]
    r = A.shape[0]
    dev = w.device
    _need(X, "X", w.dtype16, (T, w.cols), dev)
    _need(dY, "dY", w.dtype16, (T, w.rows), dev)
    _need(A, "A", w.dtype16, (r, w.cols), dev)
    _need(B, "B", w.dtype16, (w.rows, r), dev)
    if U_saved is not None:
        _need(U_saved, "U_saved", w.dtype16, (T, r), dev)
    if dX is None:
        dX = torch.empty(T, w.cols, dtype=w.dtype16, device=dev)
    if dA is None:
        dA = torch.empty(r, w.cols, dtype=torch.float32, device=dev)
    if dB is None:
        dB = torch.empty(w.rows, r, dtype=torch.float32, device=dev)
    _need(dX, "dX", w.dtype16, (T, w.cols), dev)
    _need(dA, "dA", torch.float32, (r, w.cols), dev)
    _need(dB, "dB", torch.float32, (w.rows, r), dev)
    if workspace is None:
        ws_bytes = qlora_linear_workspace(T, w.rows, w.cols, r, True)
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    desc = w.descriptor()
    _lib.check("qlora_linear_bwd",
               lib.qlora_linear_bwd(ctypes.byref(desc), X.data_ptr(), dY.data_ptr(), T,
                                    A.data_ptr(), B.data_ptr(), r, float(alpha), _ptr(U_saved),
                                    dX.data_ptr(), dA.data_ptr(), dB.data_ptr(),
                                    workspace.data_ptr(), workspace.numel(), _stream(stream)))
    return dX, dA, dB


# --------------------------------------------------------------------------
# lora_dropout
# --------------------------------------------------------------------------
def _dropout_desc(p: float, seed: int, offset: int) -> _lib.DropoutDesc:
    return _lib.DropoutDesc(float(p), int(seed) & 0xFFFFFFFFFFFFFFFF,
                            int(offset) & 0xFFFFFFFFFFFFFFFF)


def qlora_dropout_mask_bytes(T: int, cols: int) -> int:
    return int(_lib.load().qlora_dropout_mask_bytes(T, cols))


@_stream_scoped
def qlora_dropout_mask(T: int, cols: int, p: float, seed: int, offset: int,
                       X: torch.Tensor | None = None, X_dropped: torch.Tensor | None = None,
                       keep: torch.Tensor | None = None, device=None, stream=None):
    """Packed keep mask (uint8 [ceil(T/4), cols/2]) of lora_dropout and, when
    X is given, the dropped input (x where kept, +0 elsewhere; the
    1 / (1 - p) scale not applied) (qlora_dropout_mask).  Returns
    (keep, X_dropped)."""
    lib = _lib.load()
    dev = X.device if X is not None else (device or torch.device("cuda"))
    quads = (T + 3) // 4
    if keep is None:
        keep = torch.empty(quads, cols // 2, dtype=torch.uint8, device=dev)
    _need(keep, "keep", torch.uint8, (quads, cols // 2), dev)
    if X is not None:
        # the mask only moves 16-bit patterns: bf16 or fp16
        _need(X, "X", X.dtype if X.dtype == torch.float16 else torch.bfloat16, (T, cols), dev)
        if X_dropped is None:
            X_dropped = torch.empty_like(X)
        _need(X_dropped, "X_dropped", X.dtype, (T, cols), dev)
    d = _dropout_desc(p, seed, offset)
    _lib.check("qlora_dropout_mask",
               lib.qlora_dropout_mask(ctypes.byref(d), T, cols, _ptr(X), _ptr(X_dropped),
                                      keep.data_ptr(), _stream(stream)))
    return keep, X_dropped


def qlora_linear_workspace_dropout(T: int, rows: int, cols: int, r: int, is_bwd: bool) -> int:
    return int(_lib.load().qlora_linear_workspace_dropout(T, rows, cols, r, int(bool(is_bwd))))


@_stream_scoped
def qlora_linear_fwd_dropout(w: NF4Weight, X: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                             alpha: float, p: float, seed: int, offset: int,
                             Y: torch.Tensor | None = None, U_save: torch.Tensor | None = None,
                             save_u: bool = True, keep_save: torch.Tensor | None = None,
                             save_keep: bool = True, workspace: torch.Tensor | None = None,
                             X_dropped_save: torch.Tensor | None = None, stream=None):
    """Forward with lora_dropout on the adapter input (qlora_linear_fwd_dropout):
    Y = X dequant(W)^T + (alpha/r) (D(X) A^T) B^T, D(X) = keep X / (1 - p).
    Returns (Y, U, keep) with U = D(X) A^T in bf16 and the packed keep mask
    (each None when not saved).  X_dropped_save, when given ([T, cols] in
    the compute dtype), receives the dropped input (x where kept, +0
    elsewhere) for the backward's X_dropped_saved."""
    lib = _lib.load()
    T = X.shape[0]
    r = A.shape[0]
    dev = w.device
    _need(X, "X", w.dtype16, (T, w.cols), dev)
    _need(A, "A", w.dtype16, (r, w.cols), dev)
    _need(B, "B", w.dtype16, (w.rows, r), dev)
    if Y is None:
        Y = torch.empty(T, w.rows, dtype=w.dtype16, device=dev)
    _need(Y, "Y", w.dtype16, (T, w.rows), dev)
    if U_save is None and save_u:
        U_save = torch.empty(T, r, dtype=w.dtype16, device=dev)
    if U_save is not None:
        _need(U_save, "U_save", w.dtype16, (T, r), dev)
    quads = (T + 3) // 4
    if keep_save is None and save_keep:
        keep_save = torch.empty(quads, w.cols // 2, dtype=torch.uint8, device=dev)
    if keep_save is not None:
        _need(keep_save, "keep_save", torch.uint8, (quads, w.cols // 2), dev)
    if X_dropped_save is not None:
        _need(X_dropped_save, "X_dropped_save", w.dtype16, (T, w.cols), dev)
    ws_bytes = lib.qlora_linear_workspace_dropout(T, w.rows, w.cols, r, 0)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    desc = w.descriptor()
    d = _dropout_desc(p, seed, offset)
    _lib.check("qlora_linear_fwd_dropout",
               lib.qlora_linear_fwd_dropout(ctypes.byref(desc), X.data_ptr(), T, A.data_ptr(),
                                            B.data_ptr(), r, float(alpha), ctypes.byref(d),
                                            Y.data_ptr(), _ptr(U_save), _ptr(keep_save),
                                            _ptr(X_dropped_save), workspace.data_ptr(),
                                            workspace.numel(),
                                            _stream(stream)))
    return Y, U_save, keep_save


@_stream_scoped
def qlora_linear_bwd_dropout(w: NF4Weight, X: torch.Tensor | None, dY: torch.Tensor,
                             A: torch.Tensor, B: torch.Tensor, alpha: float, p: float, seed: int,
                             offset: int, keep_saved: torch.Tensor | None = None,
                             U_saved: torch.Tensor | None = None,
                             dX: torch.Tensor | None = None, dA: torch.Tensor | None = None,
                             dB: torch.Tensor | None = None,
                             workspace: torch.Tensor | None = None,
                             X_dropped_saved: torch.Tensor | None = None, stream=None):
    """Backward with lora_dropout (qlora_linear_bwd_dropout): dX (bf16), dA and
    dB (float32); no dW.  keep_saved / U_saved / X_dropped_saved from the
    forward, or None to redraw / recompute them; with X_dropped_saved, X is
    not read and may be None."""
    lib = _lib.load()
    if X is None and X_dropped_saved is None:
        raise ValueError("X: needed unless X_dropped_saved is given")
    T = (X if X is not None else X_dropped_saved).shape[0]
    r = A.shape[0]
    dev = w.device
    if X is not None:
        _need(X, "X", w.dtype16, (T, w.cols), dev)
    if X_dropped_saved is not None:
        _need(X_dropped_saved, "X_dropped_saved", w.dtype16, (T, w.cols), dev)
    _need(dY, "dY", w.dtype16, (T, w.rows), dev)
    _need(A, "A", w.dtype16, (r, w.cols), dev)
    _need(B, "B", w.dtype16, (w.rows, r), dev)
    if U_saved is not None:
        _need(U_saved, "U_saved", w.dtype16, (T, r), dev)
    if keep_saved is not None:
        _need(keep_saved, "keep_saved", torch.uint8, ((T + 3) // 4, w.cols // 2), dev)
    if dX is None:
        dX = torch.empty(T, w.cols, dtype=w.dtype16, device=dev)
    if dA is None:
        dA = torch.empty(r, w.cols, dtype=torch.float32, device=dev)
    if dB is None:
        dB = torch.empty(w.rows, r, dtype=torch.float32, device=dev)
    _need(dX, "dX", w.dtype16, (T, w.cols), dev)
    _need(dA, "dA", torch.float32, (r, w.cols), dev)
    _need(dB, "dB", torch.float32, (w.rows, r), dev)
    ws_bytes = lib.qlora_linear_workspace_dropout(T, w.rows, w.cols, r, 1)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    desc = w.descriptor()
    d = _dropout_desc(p, seed, offset)
    _lib.check("qlora_linear_bwd_dropout",
               lib.qlora_linear_bwd_dropout(ctypes.byref(desc), _ptr(X), dY.data_ptr(), T,
                                            A.data_ptr(), B.data_ptr(), r, float(alpha),
                                            ctypes.byref(d), _ptr(keep_saved),
                                            _ptr(X_dropped_saved), _ptr(U_saved),
                                            dX.data_ptr(), dA.data_ptr(), dB.data_ptr(),
                                            workspace.data_ptr(), workspace.numel(),
                                            _stream(stream)))
    return dX, dA, dB
