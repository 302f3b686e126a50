"""Python binding of ``libfa_fwd.so``, the MI355X (gfx950) FlashAttention
forward library whose C ABI is ``include/fa_fwd.h``.

The functions named like the C entry points (``fa_fwd_bf16``, ``fa_fwd_f16``,
``fa_fwd_f32``, ``fa_fwd``, ``fa_fwd_ex``, ``fa_fwd_split``, ``fa_fwd_tile_shape``,
``fa_strerror``, ``fa_build_info``, ``fa_standard_fwd`` of
``include/fa_standard.h``, the materialising baseline, and ``fa_bwd_bf16``,
``fa_bwd_f16``, ``fa_bwd_f32``, ``fa_bwd`` of ``include/fa_bwd.h``, the backward with
recomputation) only marshal arguments: pointers are
plain integers (device addresses), the stream an integer ``hipStream_t``
handle, and the C status code is returned unchanged.

``attention(q, k, v, ...)`` is a convenience on top for torch tensors: it
allocates the outputs with torch (device memory only), passes torch's current
stream, and raises on a non-zero status.  Every step of the computation runs
in the HIP kernels; there is no fallback.  If the library has not been built
the import of this package still succeeds but every call raises
``FaLibraryMissing`` (build with ``python -m tiled_exact_attention_fwd_amd.build``).
"""

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa_fwd.so")

FA_OK, FA_ERR_INVALID, FA_ERR_UNSUPPORTED, FA_ERR_HIP = 0, 1, 2, 3
FA_DTYPE_F32, FA_DTYPE_F16, FA_DTYPE_BF16 = 0, 1, 2
COUNTER_NAMES = ("computed", "full", "causal_masked", "ragged", "skipped")

# entry point name -> (restype, argtypes)
_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_FWD12 = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P]
_BWD17 = [_P] * 10 + [_I, _I, _I, _I, _F, _I, _P]


class FaArgs(ctypes.Structure):
    """Mirror of ``fa_fwd_args``."""
    _fields_ = [("q", _P), ("k", _P), ("v", _P), ("o", _P), ("lse", _P),
                ("B", _I), ("H", _I), ("N", _I), ("d", _I),
                ("scale", _F), ("causal", _I), ("stream", _P),
                ("dtype", _I), ("out_dtype", _I), ("tile_q", _I), ("tile_k", _I),
                ("counters", _P)]


SIGNATURES = {
    "fa_fwd_bf16": (_I, _FWD12),
    "fa_fwd_f16": (_I, _FWD12),
    "fa_fwd_f32": (_I, _FWD12),
    "fa_fwd": (_I, _FWD12 + [_I]),
    "fa_fwd_ex": (_I, [ctypes.POINTER(FaArgs)]),
    "fa_fwd_tile_shape": (_I, [_I, _I, _I, ctypes.POINTER(_I), ctypes.POINTER(_I)]),
    "fa_fwd_launch_tile": (_I, [ctypes.POINTER(FaArgs), ctypes.POINTER(_I), ctypes.POINTER(_I)]),
    "fa_strerror": (ctypes.c_char_p, [_I]),
    "fa_build_info": (ctypes.c_char_p, []),
    "fa_standard_fwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P, _I]),
    "fa_fwd_split": (_I, [_P] * 7 + [_I, _I, _I, _I, _F, _I, _I, _P, _I]),
    "fa_fwd_split_count": (_I, [_I, _I, _I, _I, _I, _I, ctypes.POINTER(_I)]),
    "fa_bwd_bf16": (_I, _BWD17),
    "fa_bwd_f16": (_I, _BWD17),
    "fa_bwd_f32": (_I, _BWD17),
    "fa_bwd": (_I, _BWD17 + [_I]),
    "fa_bwd_o32": (_I, _BWD17 + [_I]),
    "fa_bwd_noalloc": (_I, [_P] * 9 + [_I, _I, _I, _I, _F, _I, _P, _I]),
    "fa_clock_probe": (_I, [_P, ctypes.c_uint, _P]),
    "fa_issue_probe": (_I, [_I, _I, _P, ctypes.c_longlong, _P]),
}
FA_ERR_SCRATCH = 4
BWD_NOALLOC_MAX_ROWS = 1 << 22


class FaLibraryMissing(ImportError):
    pass


class FaError(RuntimeError):
    def __init__(self, status, what=""):
        self.status = status
        super().__init__(f"{what}: status {status} ({fa_strerror(status)})")


_lib = None


def lib(path=None):
    """Load (once) and return the ctypes handle of libfa_fwd.so."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise FaLibraryMissing(
            f"{p} not found: build it with `python -m tiled_exact_attention_fwd_amd.build`")
    handle = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(handle, name)
        fn.restype, fn.argtypes = res, args
    if path is None:
        _lib = handle
    return handle


# --- thin wrappers with the C names -----------------------------------------

def fa_fwd_bf16(q, k, v, o, lse, B, H, N, d, scale, causal, stream):
    return lib().fa_fwd_bf16(q, k, v, o, lse, B, H, N, d, scale, causal, stream)


def fa_fwd_f16(q, k, v, o, lse, B, H, N, d, scale, causal, stream):
    return lib().fa_fwd_f16(q, k, v, o, lse, B, H, N, d, scale, causal, stream)


def fa_fwd_f32(q, k, v, o, lse, B, H, N, d, scale, causal, stream):
    return lib().fa_fwd_f32(q, k, v, o, lse, B, H, N, d, scale, causal, stream)


def fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, stream, dtype):
    return lib().fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, stream, dtype)


def fa_fwd_ex(q, k, v, o, lse, B, H, N, d, scale, causal, stream, dtype,
              out_dtype=0, tile_q=0, tile_k=0, counters=None):
    a = FaArgs(q, k, v, o, lse, B, H, N, d, scale, causal, stream, dtype,
               out_dtype, tile_q, tile_k, counters)
    return lib().fa_fwd_ex(ctypes.byref(a))


def fa_standard_fwd(q, k, v, o, lse, s, p, B, H, N, d, scale, causal, stream, dtype):
    return lib().fa_standard_fwd(q, k, v, o, lse, s, p, B, H, N, d, scale, causal, stream, dtype)


def standard_attention(q, k, v, causal=False, scale=None):
    """The standard (materialising) forward of include/fa_standard.h on the
    device: returns ``(o, lse, s, p)`` with the N x N score and probability
    matrices it wrote (16-bit inputs only)."""
    import math
    import torch
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    s = torch.empty((B, H, N, N), dtype=q.dtype, device=q.device)
    p = torch.empty_like(s)
    st = fa_standard_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), s.data_ptr(),
                         p.data_ptr(), B, H, N, d, float(scale), int(bool(causal)),
                         torch.cuda.current_stream(q.device).cuda_stream, dtype_code(q.dtype))
    if st == FA_ERR_INVALID:
        raise ValueError(f"fa_standard_fwd: {fa_strerror(st)}")
    if st != FA_OK:
        raise FaError(st, "fa_standard_fwd")
    return o, lse, s, p


def fa_fwd_split(q, k, v, o, lse, o_part, lse_part, B, H, N, d, scale, causal, splits, stream, dtype):
    return lib().fa_fwd_split(q, k, v, o, lse, o_part, lse_part, B, H, N, d, scale, causal, splits, stream, dtype)


def fa_fwd_split_count(B, H, N, d, causal, dtype):
    """Returns ``(status, splits)``: the key-range count the library suggests
    for ``fa_fwd_split`` on the current device (1: the plain call is faster)."""
    n = _I(0)
    st = lib().fa_fwd_split_count(B, H, N, d, causal, dtype, ctypes.byref(n))
    return st, n.value


def attention_split(q, k, v, splits=None, causal=False, scale=None, stream=None):
    """Split-KV forward (include/fa_fwd.h ``fa_fwd_split``):
    returns ``(o, lse, o_part, lse_part)``, the merged outputs and the fp32
    per-range partials ([splits, B, H, N, d] and [splits, B, H, N]; only the
    ranges the library used are written).  ``splits=None`` takes the count
    ``fa_fwd_split_count`` suggests."""
    import math
    import torch
    for t in (q, k, v):
        if not t.is_contiguous() or not t.is_cuda or t.dtype != q.dtype or t.shape != q.shape or t.dim() != 4:
            raise ValueError("q, k, v must be contiguous device tensors of one [B, H, N, d] shape and dtype")
    B, H, N, d = q.shape
    if splits is None:
        st, splits = fa_fwd_split_count(B, H, N, d, int(bool(causal)), dtype_code(q.dtype))
        if st != FA_OK:
            raise FaError(st, "fa_fwd_split_count")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    o_part = torch.empty((max(splits, 1), B, H, N, d), dtype=torch.float32, device=q.device)
    lse_part = torch.empty((max(splits, 1), B, H, N), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    st = fa_fwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), o_part.data_ptr(),
                      lse_part.data_ptr(), B, H, N, d, float(scale), int(bool(causal)), int(splits), stream,
                      dtype_code(q.dtype))
    if st == FA_ERR_INVALID:
        raise ValueError(f"fa_fwd_split: {fa_strerror(st)}")
    if st != FA_OK:
        raise FaError(st, "fa_fwd_split")
    return o, lse, o_part, lse_part


def split_ranges(N, splits, tile_k=64):
    """The key ranges fa_fwd_split uses: whole 64-key tiles, at most one range
    per key tile (mirrors the host layer's rule; the GPU test checks the
    partials it wrote against this)."""
    nk = (N + tile_k - 1) // tile_k
    want = min(splits, nk)
    per = (nk + want - 1) // want
    used = (nk + per - 1) // per
    return [(s * per * tile_k, min(N, (s + 1) * per * tile_k)) for s in range(used)]


def fa_bwd_bf16(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, d, scale, causal, stream):
    return lib().fa_bwd_bf16(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, d, scale, causal, stream)


def fa_bwd_f16(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, d, scale, causal, stream):
    return lib().fa_bwd_f16(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, d, scale, causal, stream)


def fa_bwd_f32(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, d, scale, causal, stream):
    return lib().fa_bwd_f32(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, d, scale, causal, stream)


def fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, d, scale, causal, stream, dtype):
    return lib().fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, d, scale, causal, stream, dtype)


def fa_bwd_o32(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, d, scale, causal, stream, dtype):
    return lib().fa_bwd_o32(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, d, scale, causal, stream, dtype)


def fa_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale, causal, stream, dtype):
    return lib().fa_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, scale, causal, stream, dtype)


def attention_backward(q, k, v, o, lse, dout, causal=False, scale=None, stream=None):
    """Gradients ``(dq, dk, dv)`` of the attention forward on the device
    (include/fa_bwd.h), from the forward's ``o`` and ``lse`` for the same
    inputs and the output gradient ``dout`` ([B, H, N, d] tensors of one
    type, bf16, fp16 or fp32; lse [B, H, N] fp32).  ``o`` may also be the
    forward's fp32 output (``attention(..., out_f32=True)``) for 16-bit
    inputs: D = rowsum(dout * o) is then taken from it (``fa_bwd_o32``).
    Also returns the ``delta`` work array the call wrote (D, fp32)."""
    import math
    import torch
    ts = (q, k, v, o, dout)
    o32 = o.dtype == torch.float32 and q.dtype != torch.float32
    if not all(t.dtype == q.dtype for t in (q, k, v, dout)) or not (o32 or o.dtype == q.dtype):
        raise ValueError("q, k, v, dout must share one dtype, and o that one or fp32")
    if q.dim() != 4 or not all(t.shape == q.shape for t in ts):
        raise ValueError("q, k, v, o, dout must all be [B, H, N, d]")
    for t in ts + (lse,):
        if not t.is_contiguous() or not t.is_cuda:
            raise ValueError("inputs must be contiguous device tensors")
    B, H, N, d = q.shape
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N):
        raise ValueError("lse must be fp32 [B, H, N]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    entry = fa_bwd_o32 if o32 else fa_bwd
    st = entry(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
               dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(), B, H, N, d, float(scale),
               int(bool(causal)), stream, dtype_code(q.dtype))
    name = "fa_bwd_o32" if o32 else "fa_bwd"
    if st == FA_ERR_INVALID:
        raise ValueError(f"{name}: {fa_strerror(st)}")
    if st != FA_OK:
        raise FaError(st, name)
    return dq, dk, dv, delta


def fa_clock_probe(out, ticks, stream):
    return lib().fa_clock_probe(out, ticks, stream)


def fa_issue_probe(mode, iters, out, out_len, stream):
    return lib().fa_issue_probe(mode, iters, out, out_len, stream)


def fa_fwd_tile_shape(dtype, d, causal):
    """Returns ``(status, tile_q, tile_k)``."""
    tq, tk = _I(0), _I(0)
    st = lib().fa_fwd_tile_shape(dtype, d, causal, ctypes.byref(tq), ctypes.byref(tk))
    return st, tq.value, tk.value


def fa_fwd_launch_tile(q, k, v, o, lse, B, H, N, d, scale, causal, stream, dtype,
                       out_dtype=0, tile_q=0, tile_k=0, counters=None):
    """Returns ``(status, tile_q, tile_k)``: the tile of the kernel that
    ``fa_fwd_ex`` with these arguments runs."""
    a = FaArgs(q, k, v, o, lse, B, H, N, d, scale, causal, stream, dtype,
               out_dtype, tile_q, tile_k, counters)
    tq, tk = _I(0), _I(0)
    st = lib().fa_fwd_launch_tile(ctypes.byref(a), ctypes.byref(tq), ctypes.byref(tk))
    return st, tq.value, tk.value


def fa_strerror(status):
    return lib().fa_strerror(status).decode()


def fa_build_info():
    return lib().fa_build_info().decode()


# --- torch convenience (device memory and streams only) ---------------------

def dtype_code(torch_dtype):
    import torch
    codes = {torch.float32: FA_DTYPE_F32, torch.float16: FA_DTYPE_F16,
             torch.bfloat16: FA_DTYPE_BF16}
    if torch_dtype not in codes:
        raise ValueError(f"unsupported element type {torch_dtype}")
    return codes[torch_dtype]


def check_outputs(q, o=None, lse=None, out_f32=False):
    """Raises ValueError unless caller-supplied output buffers fit the launch
    for ``q``: the kernel writes B*H*N*d elements of O (fp32 when ``out_f32``,
    else q's type) and B*H*N fp32 LSE values through raw pointers, so a
    smaller, strided, mistyped or foreign-device buffer would be overrun."""
    import torch
    B, H, N, _ = q.shape
    o_dtype = torch.float32 if out_f32 else q.dtype
    if o is not None and (o.dtype != o_dtype or o.shape != q.shape or not o.is_contiguous()
                          or o.device != q.device):
        raise ValueError(f"o must be a contiguous {o_dtype} tensor of shape {tuple(q.shape)} on {q.device}")
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N)
                            or not lse.is_contiguous() or lse.device != q.device):
        raise ValueError(f"lse must be a contiguous float32 tensor of shape {(B, H, N)} on {q.device}")


def attention(q, k, v, causal=False, scale=None, out_f32=False, counters=False,
              o=None, lse=None, stream=None, tile=None):
    """Exact attention forward on the device.

    q, k, v: contiguous [B, H, N, d] CUDA(HIP) tensors of one dtype (fp32, fp16
    or bf16).  Returns ``(o, lse)``, or ``(o, lse, counts)`` with ``counts`` a
    dict of tile counts when ``counters`` is set (that launch uses the
    instrumented kernel).  ``o`` / ``lse`` may be passed in preallocated.
    ``tile`` = (query rows, keys) asks for a tile shape other than the
    default (bf16, d = 128, no mask: {64, 128, 256} x {32, 64, 128}).
    """
    import math
    import torch
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share one dtype")
    if not (q.shape == k.shape == v.shape) or q.dim() != 4:
        raise ValueError("q, k, v must all be [B, H, N, d]")
    for t in (q, k, v):
        if not t.is_contiguous() or not t.is_cuda:
            raise ValueError("q, k, v must be contiguous device tensors")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dt = dtype_code(q.dtype)
    check_outputs(q, o, lse, out_f32)
    if o is None:
        o = torch.empty(q.shape, dtype=torch.float32 if out_f32 else q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    cnt = torch.zeros(len(COUNTER_NAMES), dtype=torch.int64, device=q.device) if counters else None
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    st = fa_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                   B, H, N, d, float(scale), int(bool(causal)), stream, dt,
                   out_dtype=1 if out_f32 else 0,
                   tile_q=tile[0] if tile else 0, tile_k=tile[1] if tile else 0,
                   counters=cnt.data_ptr() if cnt is not None else None)
    if st == FA_ERR_INVALID:
        raise ValueError(f"fa_fwd: {fa_strerror(st)}")
    if st != FA_OK:
        raise FaError(st, "fa_fwd")
    if counters:
        vals = cnt.cpu().tolist()
        return o, lse, dict(zip(COUNTER_NAMES, vals))
    return o, lse
