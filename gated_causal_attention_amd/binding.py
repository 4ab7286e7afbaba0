"""ctypes binding of libresolvent.so -- argument marshalling only.

Every function here has the name of the C entry point it calls (declared in
``include/resolvent.h``).  PyTorch supplies device memory and the stream; all
of the computation happens in the library's HIP kernels.  There is no other
path: a missing library is an error, never a fallback.
"""
import ctypes
import enum
import os

PKG = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(PKG, "libresolvent.so")

BF16, F32 = 0, 1


class Status(enum.IntEnum):
    OK = 0
    NONFINITE = 1
    BAD_SHAPE = 2
    BAD_ARG = 3
    UNSUPPORTED = 4
    DEVICE_ERROR = 5
    TOO_LARGE = 6


class ResolventError(RuntimeError):
    def __init__(self, status):
        self.status = Status(status) if status in Status._value2member_map_ else status
        super().__init__(f"resolvent: {resolvent_status_str(int(status))} ({int(status)})")


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise RuntimeError(
            f"{library_path} is missing: build it first (python -c 'import __graft_entry__ as g; "
            "g.build()'); there is no fallback implementation")
    # torch ships its own HIP runtime (libamdhip64) and HSA runtime.  Loading
    # torch first lets the library's libamdhip64.so.7 dependency resolve to
    # that same runtime by soname; loaded the other way round the process
    # holds two HIP runtimes, torch's streams and device state are not the
    # library's, and its HIP calls can fail (hipErrorNoDevice) or misbehave.
    import torch  # noqa: F401

    lib = ctypes.CDLL(library_path)
    i64, i32, vp, dbl = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_double
    lib.resolvent_workspace_bytes.argtypes = [i64, i64, i64, i64, i32, i32]
    lib.resolvent_workspace_bytes.restype = ctypes.c_size_t
    lib.resolvent_forward.argtypes = [vp, vp, vp, vp, vp, dbl, dbl, dbl, i64, i64, i64, i64, i32,
                                      i32, vp, vp, vp, ctypes.c_size_t, vp, vp]
    lib.resolvent_forward.restype = i32
    lib.resolvent_forward_marked.argtypes = lib.resolvent_forward.argtypes + [vp]
    lib.resolvent_forward_marked.restype = i32
    lib.resolvent_forward_noalloc.argtypes = [vp, vp, vp, vp, vp, dbl, dbl, dbl, i64, i64, i64,
                                              i64, i32, i32, vp, vp, vp, vp]
    lib.resolvent_forward_noalloc.restype = i32
    lib.resolvent_noalloc_scratch_bytes.argtypes = []
    lib.resolvent_noalloc_scratch_bytes.restype = ctypes.c_size_t
    lib.resolvent_counters_offset.argtypes = [i64, i64, i64, i64, i32, i32]
    lib.resolvent_counters_offset.restype = ctypes.c_size_t
    lib.resolvent_tile_shape.argtypes = [ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.resolvent_tile_shape.restype = None
    lib.resolvent_workspace_bytes_grouped.argtypes = [i64, i64, i64, i64, i64, i64, i32, i32]
    lib.resolvent_workspace_bytes_grouped.restype = ctypes.c_size_t
    lib.resolvent_forward_grouped.argtypes = [vp, vp, vp, vp, vp, dbl, dbl, dbl, i64, i64, i64,
                                              i64, i64, i64, i32, i32, vp, vp, vp,
                                              ctypes.c_size_t, vp, vp]
    lib.resolvent_forward_grouped.restype = i32
    lib.resolvent_chain_workspace_bytes.argtypes = [i64, i64, i64, i64]
    lib.resolvent_chain_workspace_bytes.restype = ctypes.c_size_t
    lib.resolvent_chain.argtypes = [vp, vp, vp, dbl, i64, i64, i64, i64, i32, vp, vp, vp,
                                    ctypes.c_size_t, vp, vp]
    lib.resolvent_chain.restype = i32
    lib.resolvent_decode_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i64, i32, i32]
    lib.resolvent_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.resolvent_decode.argtypes = [vp, vp, vp, vp, vp, dbl, dbl, dbl, i64, i64, i64, i64, i64,
                                     i64, i64, i32, i32, vp, vp, vp, ctypes.c_size_t, vp, vp]
    lib.resolvent_decode.restype = i32
    lib.resolvent_chain_step.argtypes = [vp, vp, vp, vp, vp, dbl, i64, i64, i64, i32, vp, vp]
    lib.resolvent_chain_step.restype = i32
    lib.resolvent_operator_workspace_bytes.argtypes = [i64, i64, i64, i64, i32]
    lib.resolvent_operator_workspace_bytes.restype = ctypes.c_size_t
    lib.resolvent_operator.argtypes = [vp, vp, vp, vp, dbl, dbl, dbl, i64, i64, i64, i64, i32,
                                       vp, vp, vp, ctypes.c_size_t, vp, vp]
    lib.resolvent_operator.restype = i32
    lib.resolvent_path_product.argtypes = [vp, vp, i64, i64, vp, vp, vp]
    lib.resolvent_path_product.restype = i32
    lib.resolvent_status_str.argtypes = [i32]
    lib.resolvent_status_str.restype = ctypes.c_char_p
    _lib = lib
    return lib


def resolvent_status_str(status: int) -> str:
    return _load().resolvent_status_str(int(status)).decode()


def resolvent_workspace_bytes(B, H, n, d, qk_dtype=BF16, v_dtype=BF16) -> int:
    return int(_load().resolvent_workspace_bytes(B, H, n, d, qk_dtype, v_dtype))


def resolvent_counters_offset(B, H, n, d, qk_dtype=BF16, v_dtype=BF16) -> int:
    return int(_load().resolvent_counters_offset(B, H, n, d, qk_dtype, v_dtype))


def resolvent_tile_shape() -> tuple:
    """(query rows per query tile, keys per key tile) of the library's tiling."""
    bq, bk = ctypes.c_int32(), ctypes.c_int32()
    _load().resolvent_tile_shape(ctypes.byref(bq), ctypes.byref(bk))
    return bq.value, bk.value


def _dtype_code(t):
    import torch

    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def resolvent_forward(q, k, u, theta, v, beta, qk, g, *, o_re=None, o_im=None, workspace=None,
                      status=None, stream=None, check=True, marks=None):
    """O = readout of the resolvent head: (o_re, o_im), each [B, H, n, d] fp32.

    q, k, v: contiguous [B, H, n, d] device tensors (bf16 or fp32); u, theta:
    [B, H, n] fp32.  Buffers not given are allocated with torch.  With
    ``check`` the stream is synchronised and a non-OK device status raises
    ResolventError; otherwise the caller reads ``status`` itself.  ``marks``
    (four HIP event handles) selects resolvent_forward_marked."""
    import torch

    B, H, n, d = q.shape
    for t in (q, k, v, u, theta):
        if not t.is_contiguous():
            raise ValueError("inputs must be contiguous")
    dev = q.device
    qk_dt, v_dt = _dtype_code(q), _dtype_code(v)
    if o_re is None:
        o_re = torch.empty((B, H, n, d), device=dev, dtype=torch.float32)
    if o_im is None:
        o_im = torch.empty((B, H, n, d), device=dev, dtype=torch.float32)
    ws_bytes = resolvent_workspace_bytes(B, H, n, d, qk_dt, v_dt)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), device=dev, dtype=torch.uint8)
    if status is None:
        status = torch.zeros(1, device=dev, dtype=torch.int32)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    args = (q.data_ptr(), k.data_ptr(), u.data_ptr(), theta.data_ptr(), v.data_ptr(),
            float(beta), float(qk), float(g), B, H, n, d, qk_dt, v_dt, o_re.data_ptr(),
            o_im.data_ptr(), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
            status.data_ptr(), handle)
    if marks is None:
        rc = _load().resolvent_forward(*args)
    else:
        arr = (ctypes.c_void_p * 4)(*marks)
        rc = _load().resolvent_forward_marked(*args, arr)
    if rc != Status.OK:
        raise ResolventError(rc)
    if check and n > 0 and B > 0 and H > 0:
        if hasattr(stream, "synchronize"):
            stream.synchronize()
        else:
            torch.cuda.synchronize(dev)
        st = int(status.item())
        if st != Status.OK:
            raise ResolventError(st)
    return o_re, o_im


def resolvent_noalloc_scratch_bytes() -> int:
    return int(_load().resolvent_noalloc_scratch_bytes())


def resolvent_forward_noalloc(q, k, u, theta, v, beta, qk, g, *, o_re, o_im, status,
                              stream=None, check=True):
    """resolvent_forward with the library's fixed device scratch as workspace:
    the caller passes every buffer (outputs and status included) and nothing
    is allocated.  Raises ResolventError(TOO_LARGE) beyond the scratch size."""
    import torch

    B, H, n, d = q.shape
    for t in (q, k, v, u, theta, o_re, o_im):
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    dev = q.device
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    rc = _load().resolvent_forward_noalloc(
        q.data_ptr(), k.data_ptr(), u.data_ptr(), theta.data_ptr(), v.data_ptr(), float(beta),
        float(qk), float(g), B, H, n, d, _dtype_code(q), _dtype_code(v), o_re.data_ptr(),
        o_im.data_ptr(), status.data_ptr(), handle)
    if rc != Status.OK:
        raise ResolventError(rc)
    if check and n > 0 and B > 0 and H > 0:
        if hasattr(stream, "synchronize"):
            stream.synchronize()
        else:
            torch.cuda.synchronize(dev)
        st = int(status.item())
        if st != Status.OK:
            raise ResolventError(st)
    return o_re, o_im


def resolvent_workspace_bytes_grouped(B, H, Hkv, n, d, dv, qk_dtype=BF16, v_dtype=BF16) -> int:
    return int(_load().resolvent_workspace_bytes_grouped(B, H, Hkv, n, d, dv, qk_dtype, v_dtype))


def resolvent_forward_grouped(q, k, u, theta, v, beta, qk, g, *, o_re=None, o_im=None,
                              workspace=None, status=None, stream=None, check=True):
    """Grouped k/v heads and free value width: q [B, H, n, d]; k [B, Hkv, n, d];
    v [B, Hkv, n, dv]; u, theta [B, H, n].  Returns (o_re, o_im), each
    [B, H, n, dv] fp32."""
    import torch

    B, H, n, d = q.shape
    Hkv, dv = k.shape[1], v.shape[-1]
    for t in (q, k, v, u, theta):
        if not t.is_contiguous():
            raise ValueError("inputs must be contiguous")
    dev = q.device
    qk_dt, v_dt = _dtype_code(q), _dtype_code(v)
    if o_re is None:
        o_re = torch.empty((B, H, n, dv), device=dev, dtype=torch.float32)
    if o_im is None:
        o_im = torch.empty((B, H, n, dv), device=dev, dtype=torch.float32)
    ws_bytes = resolvent_workspace_bytes_grouped(B, H, Hkv, n, d, dv, qk_dt, v_dt)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), device=dev, dtype=torch.uint8)
    if status is None:
        status = torch.zeros(1, device=dev, dtype=torch.int32)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    rc = _load().resolvent_forward_grouped(
        q.data_ptr(), k.data_ptr(), u.data_ptr(), theta.data_ptr(), v.data_ptr(), float(beta),
        float(qk), float(g), B, H, Hkv, n, d, dv, qk_dt, v_dt, o_re.data_ptr(), o_im.data_ptr(),
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), status.data_ptr(),
        handle)
    if rc != Status.OK:
        raise ResolventError(rc)
    if check and n > 0 and B > 0 and H > 0:
        if hasattr(stream, "synchronize"):
            stream.synchronize()
        else:
            torch.cuda.synchronize(dev)
        st = int(status.item())
        if st != Status.OK:
            raise ResolventError(st)
    return o_re, o_im


def resolvent_chain_workspace_bytes(B, H, n, dv) -> int:
    return int(_load().resolvent_chain_workspace_bytes(B, H, n, dv))


def resolvent_chain(u, theta, v, g, *, o_re=None, o_im=None, workspace=None, status=None,
                    stream=None, check=True):
    """The path-product corner: O_i = sum_{j<=i} G_ij V_j as the gated chain,
    (o_re, o_im) each [B, H, n, dv] fp32.  u, theta: [B, H, n] fp32 device
    tensors; v: [B, H, n, dv] bf16 or fp32.  Buffers not given are allocated
    with torch; ``check`` synchronises and raises on a non-OK device status."""
    import torch

    B, H, n, dv = v.shape
    for t in (u, theta, v):
        if not t.is_contiguous():
            raise ValueError("inputs must be contiguous")
    dev = v.device
    if o_re is None:
        o_re = torch.empty((B, H, n, dv), device=dev, dtype=torch.float32)
    if o_im is None:
        o_im = torch.empty((B, H, n, dv), device=dev, dtype=torch.float32)
    ws_bytes = resolvent_chain_workspace_bytes(B, H, n, dv)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), device=dev, dtype=torch.uint8)
    if status is None:
        status = torch.zeros(1, device=dev, dtype=torch.int32)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    rc = _load().resolvent_chain(u.data_ptr(), theta.data_ptr(), v.data_ptr(), float(g), B, H,
                                 n, dv, _dtype_code(v), o_re.data_ptr(), o_im.data_ptr(),
                                 workspace.data_ptr(),
                                 workspace.numel() * workspace.element_size(), status.data_ptr(),
                                 handle)
    if rc != Status.OK:
        raise ResolventError(rc)
    if check and n > 0 and B > 0 and H > 0:
        if hasattr(stream, "synchronize"):
            stream.synchronize()
        else:
            torch.cuda.synchronize(dev)
        st = int(status.item())
        if st != Status.OK:
            raise ResolventError(st)
    return o_re, o_im


def _stream_handle(stream, dev):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(dev)
    return stream, (stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _finish(rc, stream, dev, status, check):
    """Raise on a refused call; with ``check``, wait and raise on a refused
    device status."""
    import torch

    if rc != Status.OK:
        raise ResolventError(rc)
    if check:
        if hasattr(stream, "synchronize"):
            stream.synchronize()
        else:
            torch.cuda.synchronize(dev)
        st = int(status.item())
        if st != Status.OK:
            raise ResolventError(st)


def resolvent_decode_workspace_bytes(B, H, Hkv, n, d, dv, qk_dtype=BF16, v_dtype=BF16) -> int:
    return int(_load().resolvent_decode_workspace_bytes(B, H, Hkv, n, d, dv, qk_dtype, v_dtype))


def resolvent_decode(q, k, u, theta, v, beta, qk, g, *, n=None, o_re=None, o_im=None,
                     workspace=None, status=None, stream=None, check=True):
    """One decode step: the readout of position n-1 for the query q [B, H, d]
    against the caches k [B, Hkv, cap, d], v [B, Hkv, cap, dv] and the gate
    inputs u, theta [B, H, cap], of which positions 0..n-1 are read (n
    defaults to cap).  Returns (o_re, o_im), each [B, H, dv] fp32."""
    import torch

    B, H, d = q.shape
    Hkv, cap, dv = k.shape[1], k.shape[2], v.shape[-1]
    n = cap if n is None else int(n)
    for t in (q, k, v, u, theta):
        if not t.is_contiguous():
            raise ValueError("inputs must be contiguous")
    dev = q.device
    qk_dt, v_dt = _dtype_code(q), _dtype_code(v)
    if o_re is None:
        o_re = torch.empty((B, H, dv), device=dev, dtype=torch.float32)
    if o_im is None:
        o_im = torch.empty((B, H, dv), device=dev, dtype=torch.float32)
    ws_bytes = resolvent_decode_workspace_bytes(B, H, Hkv, n, d, dv, qk_dt, v_dt)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), device=dev, dtype=torch.uint8)
    if status is None:
        status = torch.zeros(1, device=dev, dtype=torch.int32)
    stream, handle = _stream_handle(stream, dev)
    rc = _load().resolvent_decode(
        q.data_ptr(), k.data_ptr(), u.data_ptr(), theta.data_ptr(), v.data_ptr(), float(beta),
        float(qk), float(g), B, H, Hkv, n, cap, d, dv, qk_dt, v_dt, o_re.data_ptr(),
        o_im.data_ptr(),
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), status.data_ptr(),
        handle)
    _finish(rc, stream, dev, status, check and n > 0 and B > 0 and H > 0)
    return o_re, o_im


def resolvent_chain_step(y_re, y_im, u, theta, v, g, *, status=None, stream=None, check=True):
    """One step of the chain corner, in place: y <- a y + v with
    a = gate(u, theta, g); y_re, y_im [B, H, dv] fp32, u, theta [B, H] fp32,
    v [B, H, dv] bf16 or fp32.  Returns (y_re, y_im)."""
    import torch

    B, H, dv = v.shape
    for t in (y_re, y_im, u, theta, v):
        if not t.is_contiguous():
            raise ValueError("inputs must be contiguous")
    dev = v.device
    if status is None:
        status = torch.zeros(1, device=dev, dtype=torch.int32)
    stream, handle = _stream_handle(stream, dev)
    rc = _load().resolvent_chain_step(y_re.data_ptr(), y_im.data_ptr(), u.data_ptr(),
                                      theta.data_ptr(), v.data_ptr(), float(g), B, H, dv,
                                      _dtype_code(v), status.data_ptr(), handle)
    _finish(rc, stream, dev, status, check and B > 0 and H > 0 and dv > 0)
    return y_re, y_im


def resolvent_operator_workspace_bytes(B, H, n, d, qk_dtype=BF16) -> int:
    return int(_load().resolvent_operator_workspace_bytes(B, H, n, d, qk_dtype))


def resolvent_operator(q, k, u, theta, beta, qk, g, *, w_re=None, w_im=None, workspace=None,
                       status=None, stream=None, check=True):
    """The operator W of every head: q, k [B, H, n, d]; u, theta [B, H, n].
    Returns (w_re, w_im), each [B, H, n, n] fp32."""
    import torch

    B, H, n, d = q.shape
    for t in (q, k, u, theta):
        if not t.is_contiguous():
            raise ValueError("inputs must be contiguous")
    dev = q.device
    qk_dt = _dtype_code(q)
    if w_re is None:
        w_re = torch.empty((B, H, n, n), device=dev, dtype=torch.float32)
    if w_im is None:
        w_im = torch.empty((B, H, n, n), device=dev, dtype=torch.float32)
    ws_bytes = resolvent_operator_workspace_bytes(B, H, n, d, qk_dt)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), device=dev, dtype=torch.uint8)
    if status is None:
        status = torch.zeros(1, device=dev, dtype=torch.int32)
    stream, handle = _stream_handle(stream, dev)
    rc = _load().resolvent_operator(
        q.data_ptr(), k.data_ptr(), u.data_ptr(), theta.data_ptr(), float(beta), float(qk),
        float(g), B, H, n, d, qk_dt, w_re.data_ptr(), w_im.data_ptr(), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), status.data_ptr(), handle)
    _finish(rc, stream, dev, status, check and n > 0 and B > 0 and H > 0)
    return w_re, w_im


def resolvent_path_product(a_re, a_im, *, g_re=None, g_im=None, stream=None):
    """G = path_product(a) of each gate sequence: a_re, a_im [..., n] fp64
    device tensors; returns (g_re, g_im), each [..., n, n] fp64."""
    import torch

    if a_re.dtype != torch.float64 or a_im.dtype != torch.float64:
        raise TypeError("gates are float64")
    if not (a_re.is_contiguous() and a_im.is_contiguous()) or a_re.shape != a_im.shape:
        raise ValueError("a_re, a_im: contiguous, one shape")
    n = a_re.shape[-1] if a_re.dim() else 0
    batch = a_re.numel() // n if n else 0
    dev = a_re.device
    shape = tuple(a_re.shape) + (n,)
    if g_re is None:
        g_re = torch.empty(shape, device=dev, dtype=torch.float64)
    if g_im is None:
        g_im = torch.empty(shape, device=dev, dtype=torch.float64)
    stream, handle = _stream_handle(stream, dev)
    rc = _load().resolvent_path_product(a_re.data_ptr(), a_im.data_ptr(), batch, n,
                                        g_re.data_ptr(), g_im.data_ptr(), handle)
    if rc != Status.OK:
        raise ResolventError(rc)
    return g_re, g_im


def forward(q, k, u, theta, v, beta, qk, g, **kw):
    """resolvent_forward returning one complex tensor (o_re + i o_im)."""
    import torch

    o_re, o_im = resolvent_forward(q, k, u, theta, v, beta, qk, g, **kw)
    return torch.complex(o_re, o_im)
