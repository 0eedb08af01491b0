"""ctypes binding of the C ABI in include/fa.h (argument marshalling only)."""

import ctypes
import math
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libfa.so")

FA_F32, FA_F16, FA_BF16 = 0, 1, 2

STATUS_NAMES = {
    0: "FA_OK",
    -1: "FA_ERR_NULL",
    -2: "FA_ERR_DIM",
    -3: "FA_ERR_UNSUPPORTED_D",
    -4: "FA_ERR_DTYPE",
    -5: "FA_ERR_ALIGN",
    -6: "FA_ERR_ALIAS",
    -7: "FA_ERR_LAUNCH",
    -8: "FA_ERR_SCALE",
    -9: "FA_ERR_TOO_LARGE",
    -10: "FA_ERR_DEVICE",
    -11: "FA_ERR_WORKSPACE",
    -12: "FA_ERR_SPLITS",
    -13: "FA_ERR_STRIDE",
    -14: "FA_ERR_SCRATCH",
}

# Every symbol include/fa.h declares.
EXPORTS = ("fa_device_info", "fa_forward", "fa_forward_ex", "fa_forward_ex_noalloc",
           "fa_forward_ex_workspace_bytes",
           "fa_forward_strided", "fa_key_groups_suggest", "fa_naive_forward", "fa_naive_workspace_bytes",
           "fa_splitkv_suggest", "fa_status_string", "fa_version", "fa_workgroup_shape")

_lib = None


class FAError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {fa_status_string(status)}")


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libfa.so (built in-tree by __graft_entry__.build() or
    tiled_attention_fa_amd/build.py).  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; "
                          f"g.build()'` or `python tiled_attention_fa_amd/build.py` first")
    lib = ctypes.CDLL(_LIB_PATH)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.fa_forward.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_float, ctypes.c_int,
                               ctypes.c_int, vp]
    lib.fa_forward.restype = ctypes.c_int
    lib.fa_forward_strided.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                       ctypes.c_float, ctypes.c_int, ctypes.c_int, vp]
    lib.fa_forward_strided.restype = ctypes.c_int
    lib.fa_forward_ex.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_float, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_int, vp, i64, vp]
    lib.fa_forward_ex.restype = ctypes.c_int
    lib.fa_forward_ex_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_float,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
    lib.fa_forward_ex_noalloc.restype = ctypes.c_int
    lib.fa_forward_ex_workspace_bytes.argtypes = [i64, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                                  ctypes.c_int]
    lib.fa_forward_ex_workspace_bytes.restype = i64
    lib.fa_splitkv_suggest.argtypes = [i64, i64, i64, i64, ctypes.c_int, ctypes.c_int]
    lib.fa_splitkv_suggest.restype = ctypes.c_int
    lib.fa_key_groups_suggest.argtypes = [i64, i64, i64, i64, ctypes.c_int, ctypes.c_int]
    lib.fa_key_groups_suggest.restype = ctypes.c_int
    ip = ctypes.POINTER(ctypes.c_int)
    lib.fa_workgroup_shape.argtypes = [i64, i64, i64, i64, ctypes.c_int, ctypes.c_int, ip, ip, ip]
    lib.fa_workgroup_shape.restype = ctypes.c_int
    lib.fa_naive_forward.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_float, ctypes.c_int,
                                     ctypes.c_int, vp, i64, vp]
    lib.fa_naive_forward.restype = ctypes.c_int
    lib.fa_naive_workspace_bytes.argtypes = [i64, i64, i64, ctypes.c_int]
    lib.fa_naive_workspace_bytes.restype = i64
    lib.fa_device_info.argtypes = [ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)]
    lib.fa_device_info.restype = ctypes.c_int
    lib.fa_status_string.argtypes = [ctypes.c_int]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_version.argtypes = []
    lib.fa_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def fa_status_string(status: int) -> str:
    return load_library().fa_status_string(int(status)).decode()


def fa_version() -> str:
    return load_library().fa_version().decode()


def fa_device_info():
    """(compute units, peak shader clock in kHz) of the current device."""
    cus, clk = ctypes.c_int(0), ctypes.c_int(0)
    st = load_library().fa_device_info(ctypes.byref(cus), ctypes.byref(clk))
    if st != 0:
        raise FAError(st)
    return cus.value, clk.value


def fa_forward_raw(q: int, k: int, v: int, o: int, B: int, H: int, N: int, D: int, scale: float,
                   causal: bool, dtype: int, stream: int = 0) -> int:
    """Direct call of the C entry point with integer addresses; returns the
    status code (no exception)."""
    return load_library().fa_forward(q or None, k or None, v or None, o or None, int(B), int(H),
                                     int(N), int(D), float(scale), int(bool(causal)), int(dtype),
                                     stream or None)


def fa_forward_strided_raw(q: int, q_strides, k: int, k_strides, v: int, v_strides, o: int, o_strides,
                           B: int, H: int, H_kv: int, N: int, D: int, scale: float, causal: bool,
                           dtype: int, stream: int = 0) -> int:
    """Direct call of fa_forward_strided with integer addresses and stride
    triples (or None); returns the status code."""
    def arr(s):
        return None if s is None else (ctypes.c_int64 * 3)(*[int(x) for x in s])
    return load_library().fa_forward_strided(q or None, arr(q_strides), k or None, arr(k_strides),
                                             v or None, arr(v_strides), o or None, arr(o_strides),
                                             int(B), int(H), int(H_kv), int(N), int(D), float(scale),
                                             int(bool(causal)), int(dtype), stream or None)


def fa_forward_ex_raw(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, N: int, D: int,
                      scale: float, causal: bool, dtype: int, num_splits: int, workspace: int,
                      workspace_bytes: int, stream: int = 0) -> int:
    """Direct call of fa_forward_ex with integer addresses; returns the
    status code."""
    return load_library().fa_forward_ex(q or None, k or None, v or None, o or None, lse or None,
                                        int(B), int(H), int(N), int(D), float(scale),
                                        int(bool(causal)), int(dtype), int(num_splits),
                                        workspace or None, int(workspace_bytes), stream or None)


def fa_forward_ex_noalloc_raw(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, N: int, D: int,
                              scale: float, causal: bool, dtype: int, num_splits: int,
                              stream: int = 0) -> int:
    """Direct call of fa_forward_ex_noalloc (split-KV partials in the
    library's fixed per-device scratch); returns the status code."""
    return load_library().fa_forward_ex_noalloc(q or None, k or None, v or None, o or None, lse or None,
                                                int(B), int(H), int(N), int(D), float(scale),
                                                int(bool(causal)), int(dtype), int(num_splits),
                                                stream or None)


def fa_forward_ex_workspace_bytes(B: int, H: int, N: int, D: int, dtype: int, causal: bool,
                                  num_splits: int) -> int:
    return int(load_library().fa_forward_ex_workspace_bytes(int(B), int(H), int(N), int(D), int(dtype),
                                                            int(bool(causal)), int(num_splits)))


def fa_splitkv_suggest(B: int, H: int, N: int, D: int, dtype: int, causal: bool) -> int:
    return int(load_library().fa_splitkv_suggest(int(B), int(H), int(N), int(D), int(dtype),
                                                 int(bool(causal))))


def fa_key_groups_suggest(B: int, H: int, N: int, D: int, dtype: int, causal: bool) -> int:
    """Key groups (1, 2 or 4) the forward kernel uses for these sizes on the
    current device, or a negative status."""
    return int(load_library().fa_key_groups_suggest(int(B), int(H), int(N), int(D), int(dtype),
                                                    int(bool(causal))))


def fa_workgroup_shape(B: int, H: int, N: int, D: int, dtype: int, causal: bool):
    """(waves, key_groups, block_n) of the forward kernel for these sizes
    on the current device, or a negative status (an int)."""
    w, g, bn = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(0)
    st = int(load_library().fa_workgroup_shape(int(B), int(H), int(N), int(D), int(dtype), int(bool(causal)),
                                               ctypes.byref(w), ctypes.byref(g), ctypes.byref(bn)))
    if st != 0:
        return st
    return (w.value, g.value, bn.value)


def fa_naive_workspace_bytes(B: int, H: int, N: int, dtype: int) -> int:
    """Workspace bytes of the three-pass path (negative status on bad
    arguments)."""
    return int(load_library().fa_naive_workspace_bytes(int(B), int(H), int(N), int(dtype)))


def fa_naive_forward_raw(q: int, k: int, v: int, o: int, B: int, H: int, N: int, D: int,
                         scale: float, causal: bool, dtype: int, workspace: int, workspace_bytes: int,
                         stream: int = 0) -> int:
    """Direct call of the three-pass entry point; returns the status code."""
    return load_library().fa_naive_forward(q or None, k or None, v or None, o or None, int(B), int(H),
                                           int(N), int(D), float(scale), int(bool(causal)),
                                           int(dtype), workspace or None, int(workspace_bytes),
                                           stream or None)


def _dtype_code(t):
    import torch
    codes = {torch.float32: FA_F32, torch.float16: FA_F16, torch.bfloat16: FA_BF16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported tensor dtype {t.dtype}")
    return codes[t.dtype]


def _check_qkvo(q, k, v, o):
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, N, D], got shape {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device:
            raise ValueError(f"{name} must match q in shape, dtype and device")
    if q.device.type != "cuda":
        raise ValueError("tensors must be on a HIP device")


def _stream_handle(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _used_on(stream, device, *tensors):
    """Tensors allocated here on torch's current stream and written by
    kernels enqueued on `stream`: when that is another stream, record it on
    them, so that the caching allocator does not hand their memory out again
    (to work on the current stream) before `stream` has finished with it."""
    import torch
    if stream is None:
        return
    s = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(int(stream), device=device)
    if s == torch.cuda.current_stream(device):
        return
    for t in tensors:
        if t is not None:
            t.record_stream(s)


def fa_forward(q, k, v, o, scale=None, causal=False, stream=None) -> None:
    """o <- softmax(scale * q k^T [+ causal mask]) v for torch tensors of shape
    [B, H, N, D] on the current HIP device (contiguous, one dtype).
    scale defaults to 1/sqrt(D); stream defaults to torch's current stream.
    Enqueues the kernel and returns; raises FAError on a rejected call."""
    import torch
    _check_qkvo(q, k, v, o)
    B, H, N, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    handle = _stream_handle(stream, q.device)
    with torch.cuda.device(q.device):
        st = fa_forward_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), B, H, N, D,
                            scale, causal, _dtype_code(q), handle)
    if st != 0:
        raise FAError(st)


def forward(q, k, v, scale=None, causal=False, stream=None):
    """Allocate o like q and run fa_forward; returns o.  With a stream other
    than torch's current one, o is recorded as in use by that stream."""
    import torch
    o = torch.empty_like(q)
    fa_forward(q, k, v, o, scale=scale, causal=causal, stream=stream)
    _used_on(stream, q.device, o)
    return o


def naive_workspace(q):
    """A uint8 device tensor big enough for the three-pass path on tensors
    shaped and typed like q (torch's allocator returns 256-byte aligned
    blocks)."""
    import torch
    B, H, N, _ = q.shape
    n = fa_naive_workspace_bytes(B, H, N, _dtype_code(q))
    if n < 0:
        raise FAError(n)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)


def fa_naive_forward(q, k, v, o, workspace, scale=None, causal=False, stream=None) -> None:
    """The three-pass attention (S and P through `workspace`, a uint8 device
    tensor from naive_workspace); same result as fa_forward.  Enqueues and
    returns; raises FAError on a rejected call."""
    import torch
    _check_qkvo(q, k, v, o)
    if workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on q's device")
    B, H, N, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    handle = _stream_handle(stream, q.device)
    with torch.cuda.device(q.device):
        st = fa_naive_forward_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), B, H, N, D,
                                  scale, causal, _dtype_code(q), workspace.data_ptr(),
                                  workspace.numel() * workspace.element_size(), handle)
    if st != 0:
        raise FAError(st)


def naive_forward(q, k, v, scale=None, causal=False, stream=None, workspace=None):
    """Allocate o (and the workspace unless given) and run the three-pass
    path; returns o.  With a stream other than torch's current one, what was
    allocated here is recorded as in use by that stream."""
    import torch
    o = torch.empty_like(q)
    ws = workspace if workspace is not None else naive_workspace(q)
    fa_naive_forward(q, k, v, o, ws, scale=scale, causal=causal, stream=stream)
    _used_on(stream, q.device, o, ws if workspace is None else None)
    return o


def splitkv_workspace(q, num_splits=0, causal=False):
    """A uint8 device tensor big enough for fa_forward_ex on tensors shaped
    and typed like q with this split count (0: the suggestion)."""
    import torch
    B, H, N, D = q.shape
    n = fa_forward_ex_workspace_bytes(B, H, N, D, _dtype_code(q), causal, num_splits)
    if n < 0:
        raise FAError(n)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)


def fa_forward_ex(q, k, v, o, lse=None, scale=None, causal=False, num_splits=1, workspace=None,
                  stream=None) -> None:
    """fa_forward_ex on torch tensors: o <- attention, lse (optional float32
    [B, H, N] tensor) <- each row's log-sum-exp; num_splits key ranges per
    query block (0: the suggestion), workspace a uint8 device tensor from
    splitkv_workspace (needed unless the split count resolves to 1).
    Enqueues and returns; raises FAError on a rejected call."""
    import torch
    _check_qkvo(q, k, v, o)
    B, H, N, D = q.shape
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N)
                            or not lse.is_contiguous() or lse.device != q.device):
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor on q's device")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    handle = _stream_handle(stream, q.device)
    ws_ptr, ws_bytes = (workspace.data_ptr(), workspace.numel() * workspace.element_size()) \
        if workspace is not None else (0, 0)
    with torch.cuda.device(q.device):
        st = fa_forward_ex_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                               lse.data_ptr() if lse is not None else 0, B, H, N, D, scale, causal,
                               _dtype_code(q), num_splits, ws_ptr, ws_bytes, handle)
    if st != 0:
        raise FAError(st)


def fa_forward_ex_noalloc(q, k, v, o, lse=None, scale=None, causal=False, num_splits=1,
                          stream=None) -> None:
    """fa_forward_ex_noalloc on torch tensors: as fa_forward_ex without a
    workspace (the library's fixed scratch holds the split-KV partials; the
    call allocates nothing).  Calls that overlap in time on one device race.
    Enqueues and returns; raises FAError on a rejected call (FA_ERR_SCRATCH
    when the partials exceed the scratch)."""
    import torch
    _check_qkvo(q, k, v, o)
    B, H, N, D = q.shape
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N)
                            or not lse.is_contiguous() or lse.device != q.device):
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor on q's device")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    handle = _stream_handle(stream, q.device)
    with torch.cuda.device(q.device):
        st = fa_forward_ex_noalloc_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                       lse.data_ptr() if lse is not None else 0, B, H, N, D, scale,
                                       causal, _dtype_code(q), num_splits, handle)
    if st != 0:
        raise FAError(st)


def forward_ex(q, k, v, scale=None, causal=False, num_splits=1, lse=False, workspace=None,
               stream=None):
    """O (and, with lse=True, the [B, H, N] float32 log-sum-exp) through
    fa_forward_ex; num_splits 0 takes the suggestion.  Allocates o, the lse
    tensor and (unless given) the workspace with torch; returns o or
    (o, lse).  With a stream other than torch's current one, what was
    allocated here is recorded as in use by that stream."""
    import torch
    o = torch.empty_like(q)
    B, H, N, _ = q.shape
    lse_t = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse else None
    with torch.cuda.device(q.device):
        ws = workspace if workspace is not None else splitkv_workspace(q, num_splits, causal)
    fa_forward_ex(q, k, v, o, lse_t, scale=scale, causal=causal, num_splits=num_splits, workspace=ws,
                  stream=stream)
    _used_on(stream, q.device, o, lse_t, ws if workspace is None else None)
    return (o, lse_t) if lse else o


def fa_forward_strided(q, k, v, o, scale=None, causal=False, stream=None) -> None:
    """o <- attention for torch tensors of any strides with a contiguous last
    dimension: q and o [B, H, N, D], k and v [B, H_kv, N, D] with H_kv
    dividing H (grouped / multi-query heads).  A [B, N, H, D] tensor x is
    passed as x.transpose(1, 2).  Enqueues and returns; raises FAError on a
    rejected call."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-d, got shape {tuple(t.shape)}")
        if t.stride(3) != 1:
            raise ValueError(f"{name} must have a contiguous last dimension")
        if t.dtype != q.dtype or t.device != q.device:
            raise ValueError(f"{name} must match q in dtype and device")
    B, H, N, D = q.shape
    Hk = k.shape[1]
    if tuple(o.shape) != (B, H, N, D) or tuple(k.shape) != (B, Hk, N, D) or tuple(v.shape) != (B, Hk, N, D):
        raise ValueError("shapes must be q, o: [B, H, N, D] and k, v: [B, H_kv, N, D]")
    if q.device.type != "cuda":
        raise ValueError("tensors must be on a HIP device")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    handle = _stream_handle(stream, q.device)
    st = lambda t: t.stride()[:3]
    with torch.cuda.device(q.device):
        r = fa_forward_strided_raw(q.data_ptr(), st(q), k.data_ptr(), st(k), v.data_ptr(), st(v),
                                   o.data_ptr(), st(o), B, H, Hk, N, D, scale, causal, _dtype_code(q),
                                   handle)
    if r != 0:
        raise FAError(r)
