"""ctypes binding of libnf4.so.  Argument marshalling only: shapes and dtypes are
checked here so that errors name the Python argument; everything else (the
library's own checks, every kernel) happens behind the C ABI."""
import ctypes
import os

import torch  # loaded first so libnf4 binds to the HIP runtime torch already uses

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libnf4.so")

GROUP = 64
MAX_M = 32
MAX_K = 32768
PACK_NONFINITE = 1
PACK_SCALE_OVERFLOW = 2
EMBED_BAD_ID = 1

_STATUS = {0: "NF4_OK", -1: "NF4_EINVAL", -2: "NF4_EALIGN", -3: "NF4_ERANGE",
           -4: "NF4_EDEVICE", -5: "NF4_ELAUNCH"}

_lib = None


class NF4Error(RuntimeError):
    def __init__(self, func, status, msg):
        super().__init__(f"{func}: {_STATUS.get(status, status)} ({msg})")
        self.status = status


def lib_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built; run __graft_entry__.build() "
                          "or python dequant_gemv_nf4_amd/build.py")
    L = ctypes.CDLL(_LIB_PATH)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    L.nf4_pack.argtypes = [vp, i64, i64, vp, vp, vp, vp]
    L.nf4_unpack.argtypes = [vp, vp, i64, i64, vp, vp]
    L.nf4_gemv.argtypes = [vp, vp, i64, i64, vp, vp, vp]
    L.nf4_gemm_smallm.argtypes = [vp, vp, i64, i64, vp, i64, vp, vp]
    L.nf4_gemm_prefill.argtypes = [vp, vp, i64, i64, vp, i64, vp, vp]
    L.nf4_gemm_smallm_ws.argtypes = [vp, vp, i64, i64, vp, i64, vp, vp, i64, vp]
    L.nf4_gemm_smallm_workspace_bytes.argtypes = [i64, i64, i64]
    L.nf4_gemm_smallm_workspace_bytes.restype = ctypes.c_int64
    L.nf4_gemm_smallm_noalloc.argtypes = [vp, vp, i64, i64, vp, i64, vp, vp]
    L.nf4_gemm_smallm_noalloc.restype = ctypes.c_int
    L.nf4_gemm_smallm_noalloc_max_bytes.argtypes = []
    L.nf4_gemm_smallm_noalloc_max_bytes.restype = ctypes.c_int64
    L.nf4_gemm_prefill_ws.argtypes = [vp, vp, i64, i64, vp, i64, vp, vp, i64, vp]
    L.nf4_gemm_prefill_workspace_bytes.argtypes = [i64, i64, i64]
    L.nf4_gemm_prefill_workspace_bytes.restype = ctypes.c_int64
    L.nf4_embed.argtypes = [vp, vp, i64, i64, vp, i64, vp, vp, vp]
    L.nf4_ring_create.argtypes = [ctypes.POINTER(ctypes.c_void_p), vp, vp, i64, vp, vp]
    L.nf4_ring_gemm.argtypes = [vp, vp, vp, i64, i64, vp, i64, vp]
    L.nf4_ring_destroy.argtypes = [vp]
    L.nf4_ring_slot_bytes.argtypes = [i64, i64]
    L.nf4_ring_slot_bytes.restype = ctypes.c_int64
    for f in (L.nf4_ring_create, L.nf4_ring_gemm, L.nf4_ring_destroy):
        f.restype = ctypes.c_int
    for f in (L.nf4_pack, L.nf4_unpack, L.nf4_gemv, L.nf4_gemm_smallm, L.nf4_gemm_smallm_ws,
              L.nf4_gemm_prefill, L.nf4_gemm_prefill_ws, L.nf4_embed):
        f.restype = ctypes.c_int
    L.nf4_codebook.argtypes = [ctypes.POINTER(ctypes.c_float)]
    L.nf4_codebook.restype = None
    L.nf4_strerror.argtypes = [ctypes.c_int]
    L.nf4_strerror.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(func, status):
    if status != 0:
        raise NF4Error(func, status, _load().nf4_strerror(status).decode())


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(device, stream):
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtypes, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() not in ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, has {t.dim()}")


_U16 = (torch.int16, torch.uint16)
_BF16 = (torch.bfloat16, torch.int16, torch.uint16)


def nf4_pack(W, codes, scales, dev_status=None, stream=None):
    """Quantize fp32 W [N][K] into codes uint8 [N][K/2] and scales (fp16 bits) [N][K/64]."""
    _need(W, "W", (torch.float32,), (2,))
    N, K = W.shape
    _need(codes, "codes", (torch.uint8,))
    _need(scales, "scales", _U16 + (torch.float16,))
    if dev_status is not None:
        _need(dev_status, "dev_status", (torch.int32,))
    with torch.cuda.device(W.device):
        _check("nf4_pack", _load().nf4_pack(_ptr(W), N, K, _ptr(codes), _ptr(scales),
                                            _ptr(dev_status), _stream(W.device, stream)))


def nf4_unpack(codes, scales, W_out, stream=None):
    """Dequantize to fp32 W_out [N][K] = fp32(L[c] * s)."""
    _need(W_out, "W_out", (torch.float32,), (2,))
    N, K = W_out.shape
    _need(codes, "codes", (torch.uint8,))
    _need(scales, "scales", _U16 + (torch.float16,))
    with torch.cuda.device(W_out.device):
        _check("nf4_unpack", _load().nf4_unpack(_ptr(codes), _ptr(scales), N, K, _ptr(W_out),
                                                _stream(W_out.device, stream)))


def _nk(codes, scales, K):
    N = codes.shape[0]
    if codes.numel() != N * K // 2:
        raise ValueError(f"codes has {codes.numel()} bytes, expected N*K/2 = {N * K // 2}")
    if scales.numel() != N * (K // GROUP):
        raise ValueError(f"scales has {scales.numel()} entries, expected N*K/64")
    return N


def nf4_gemv(codes, scales, x, y, stream=None):
    """y [N] (fp32) = dequant(codes, scales) . x, x bf16 [K]."""
    _need(codes, "codes", (torch.uint8,), (2,))
    _need(scales, "scales", _U16 + (torch.float16,))
    _need(x, "x", _BF16)
    _need(y, "y", (torch.float32,))
    K = x.numel()
    N = _nk(codes, scales, K)
    if y.numel() != N:
        raise ValueError("y must have N elements")
    with torch.cuda.device(x.device):
        _check("nf4_gemv", _load().nf4_gemv(_ptr(codes), _ptr(scales), N, K, _ptr(x), _ptr(y),
                                            _stream(x.device, stream)))


def nf4_gemm_smallm(codes, scales, X, Y, stream=None):
    """Y [M][N] (fp32) = X . dequant(codes, scales)^T, X bf16 [M][K], 1 <= M <= 32."""
    _need(codes, "codes", (torch.uint8,), (2,))
    _need(scales, "scales", _U16 + (torch.float16,))
    _need(X, "X", _BF16, (1, 2))
    _need(Y, "Y", (torch.float32,))
    M, K = (1, X.shape[0]) if X.dim() == 1 else X.shape
    N = _nk(codes, scales, K)
    if Y.numel() != M * N:
        raise ValueError("Y must have M*N elements")
    with torch.cuda.device(X.device):
        _check("nf4_gemm_smallm", _load().nf4_gemm_smallm(_ptr(codes), _ptr(scales), N, K,
                                                          _ptr(X), M, _ptr(Y),
                                                          _stream(X.device, stream)))


def smallm_workspace_bytes(N, K, M):
    """Bytes of workspace nf4_gemm_smallm_ws needs for (N, K, M); 0 = no split."""
    n = _load().nf4_gemm_smallm_workspace_bytes(int(N), int(K), int(M))
    if n < 0:
        raise ValueError(f"invalid shape N={N} K={K} M={M}")
    return int(n)


def nf4_gemm_smallm_ws(codes, scales, X, Y, workspace, stream=None):
    """nf4_gemm_smallm with a device workspace (uint8 tensor, counters zeroed
    before its first use; or None when smallm_workspace_bytes is 0)."""
    _need(codes, "codes", (torch.uint8,), (2,))
    _need(scales, "scales", _U16 + (torch.float16,))
    _need(X, "X", _BF16, (1, 2))
    _need(Y, "Y", (torch.float32,))
    M, K = (1, X.shape[0]) if X.dim() == 1 else X.shape
    N = _nk(codes, scales, K)
    if Y.numel() != M * N:
        raise ValueError("Y must have M*N elements")
    nbytes = 0
    if workspace is not None:
        _need(workspace, "workspace", (torch.uint8,))
        nbytes = workspace.numel()
    with torch.cuda.device(X.device):
        _check("nf4_gemm_smallm_ws", _load().nf4_gemm_smallm_ws(
            _ptr(codes), _ptr(scales), N, K, _ptr(X), M, _ptr(Y), _ptr(workspace), nbytes,
            _stream(X.device, stream)))


def noalloc_max_bytes():
    """Size of the library-owned scratch behind nf4_gemm_smallm_noalloc."""
    return int(_load().nf4_gemm_smallm_noalloc_max_bytes())


def nf4_gemm_smallm_noalloc(codes, scales, X, Y, stream=None):
    """nf4_gemm_smallm_ws with the library's own per-device scratch instead of a
    workspace: no allocation anywhere in the call.  Calls that overlap on one GPU
    race on that scratch."""
    _need(codes, "codes", (torch.uint8,), (2,))
    _need(scales, "scales", _U16 + (torch.float16,))
    _need(X, "X", _BF16, (1, 2))
    _need(Y, "Y", (torch.float32,))
    M, K = (1, X.shape[0]) if X.dim() == 1 else X.shape
    N = _nk(codes, scales, K)
    if Y.numel() != M * N:
        raise ValueError("Y must have M*N elements")
    with torch.cuda.device(X.device):
        _check("nf4_gemm_smallm_noalloc", _load().nf4_gemm_smallm_noalloc(
            _ptr(codes), _ptr(scales), N, K, _ptr(X), M, _ptr(Y), _stream(X.device, stream)))


# one workspace per (device, stream): calls sharing one must not overlap, and
# calls on one stream never do
_workspaces = {}
# Workspaces replaced by a larger one stay allocated for the life of the
# process: a HIP graph captured earlier still holds their address, and work
# already enqueued may still use them.  (Each replacement at least doubles the
# size, so the kept ones add up to less than the current one.)
_retired = []


def workspace_for(device, nbytes, stream=None):
    """A zero-initialised workspace of at least nbytes for calls on `stream`
    (default: the current stream) of `device`, kept and reused.  A new one is
    allocated and zeroed on that stream, so the zeroing is ordered before the
    call that receives it."""
    device = torch.device(device)
    if device.index is None:
        device = torch.device("cuda", torch.cuda.current_device())
    handle = _stream(device, stream).value
    key = (device.index, handle)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        size = max(nbytes, 1 << 16, 2 * ws.numel() if ws is not None else 0)
        if isinstance(stream, torch.cuda.Stream):
            ts = stream
        elif stream is None:
            ts = torch.cuda.current_stream(device)
        else:
            ts = torch.cuda.ExternalStream(handle, device=device)
        with torch.cuda.device(device), torch.cuda.stream(ts):
            new = torch.zeros(size, dtype=torch.uint8, device=device)
        if ws is not None:
            _retired.append(ws)
        _workspaces[key] = ws = new
    return ws


def nf4_gemm_prefill(codes, scales, X, Y, stream=None):
    """Y [M][N] (fp32) = X . dequant(codes, scales)^T, X bf16 [M][K], any M >= 1
    (M * K < 2^30), on the large-tile MFMA kernel."""
    _need(codes, "codes", (torch.uint8,), (2,))
    _need(scales, "scales", _U16 + (torch.float16,))
    _need(X, "X", _BF16, (1, 2))
    _need(Y, "Y", (torch.float32,))
    M, K = (1, X.shape[0]) if X.dim() == 1 else X.shape
    N = _nk(codes, scales, K)
    if Y.numel() != M * N:
        raise ValueError("Y must have M*N elements")
    with torch.cuda.device(X.device):
        _check("nf4_gemm_prefill", _load().nf4_gemm_prefill(_ptr(codes), _ptr(scales), N, K,
                                                            _ptr(X), M, _ptr(Y),
                                                            _stream(X.device, stream)))


def prefill_workspace_bytes(N, K, M):
    """Bytes of workspace nf4_gemm_prefill_ws needs for (N, K, M); 0 = no split."""
    n = _load().nf4_gemm_prefill_workspace_bytes(int(N), int(K), int(M))
    if n < 0:
        raise ValueError(f"invalid shape N={N} K={K} M={M}")
    return int(n)


def nf4_gemm_prefill_ws(codes, scales, X, Y, workspace, stream=None):
    """nf4_gemm_prefill with a device workspace (uint8 tensor, counters zeroed
    before its first use; or None when prefill_workspace_bytes is 0)."""
    _need(codes, "codes", (torch.uint8,), (2,))
    _need(scales, "scales", _U16 + (torch.float16,))
    _need(X, "X", _BF16, (1, 2))
    _need(Y, "Y", (torch.float32,))
    M, K = (1, X.shape[0]) if X.dim() == 1 else X.shape
    N = _nk(codes, scales, K)
    if Y.numel() != M * N:
        raise ValueError("Y must have M*N elements")
    nbytes = 0
    if workspace is not None:
        _need(workspace, "workspace", (torch.uint8,))
        nbytes = workspace.numel()
    with torch.cuda.device(X.device):
        _check("nf4_gemm_prefill_ws", _load().nf4_gemm_prefill_ws(
            _ptr(codes), _ptr(scales), N, K, _ptr(X), M, _ptr(Y), _ptr(workspace), nbytes,
            _stream(X.device, stream)))


def nf4_embed(codes, scales, K, ids, out, dev_status=None, stream=None):
    """out bf16 [T][K] = rows ids (int64 [T]) of dequant(codes, scales), rounded once."""
    _need(codes, "codes", (torch.uint8,), (2,))
    _need(scales, "scales", _U16 + (torch.float16,))
    _need(ids, "ids", (torch.int64,), (1,))
    _need(out, "out", _BF16, (2,))
    N = _nk(codes, scales, K)
    T = ids.numel()
    if tuple(out.shape) != (T, K):
        raise ValueError(f"out must be [T={T}][K={K}]")
    if dev_status is not None:
        _need(dev_status, "dev_status", (torch.int32,))
    with torch.cuda.device(codes.device):
        _check("nf4_embed", _load().nf4_embed(_ptr(codes), _ptr(scales), N, K, _ptr(ids), T,
                                              _ptr(out), _ptr(dev_status),
                                              _stream(codes.device, stream)))


def ring_slot_bytes(N, K):
    """Device bytes one CopyRing slot needs for an N x K packed matrix."""
    return int(_load().nf4_ring_slot_bytes(N, K))


class Ring:
    """CopyRing (nf4_ring_*): products over packed matrices in pinned host memory,
    streamed through two device slots of `slot_bytes` each.  Copies run on their
    own stream, products on `compute_stream` (default: the current stream)."""

    def __init__(self, slot_bytes, device, compute_stream=None, copy_stream=None):
        self.device = torch.device(device)
        self.slots = [torch.empty(slot_bytes, dtype=torch.uint8, device=self.device)
                      for _ in range(2)]
        self.compute_stream = compute_stream or torch.cuda.current_stream(self.device)
        self.copy_stream = copy_stream or torch.cuda.Stream(self.device)
        self._ring = ctypes.c_void_p()
        with torch.cuda.device(self.device):
            _check("nf4_ring_create", _load().nf4_ring_create(
                ctypes.byref(self._ring), _ptr(self.slots[0]), _ptr(self.slots[1]), slot_bytes,
                ctypes.c_void_p(self.compute_stream.cuda_stream),
                ctypes.c_void_p(self.copy_stream.cuda_stream)))
        self._keep = []  # host buffers of enqueued copies, held until close()

    def gemm(self, host_codes, host_scales, X, Y):
        """Y [M][N] fp32 = X bf16 [M][K] . dequant(host_codes, host_scales)^T."""
        for t, n in ((host_codes, "host_codes"), (host_scales, "host_scales")):
            if t.device.type != "cpu" or not t.is_pinned() or not t.is_contiguous():
                raise ValueError(f"{n} must be a contiguous pinned host tensor")
        _need(X, "X", _BF16, (1, 2))
        _need(Y, "Y", (torch.float32,))
        M, K = (1, X.shape[0]) if X.dim() == 1 else X.shape
        N = _nk(host_codes, host_scales, K)
        if Y.numel() != M * N:
            raise ValueError("Y must have M*N elements")
        self._keep.append((host_codes, host_scales))
        with torch.cuda.device(self.device):
            _check("nf4_ring_gemm", _load().nf4_ring_gemm(
                self._ring, _ptr(host_codes), _ptr(host_scales), N, K, _ptr(X), M, _ptr(Y)))

    def close(self):
        if self._ring:
            with torch.cuda.device(self.device):
                st = _load().nf4_ring_destroy(self._ring)
            self._ring = ctypes.c_void_p()
            self._keep.clear()
            _check("nf4_ring_destroy", st)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def nf4_codebook():
    """The library's 16 fp32 NF4 levels (host call, no GPU needed)."""
    out = (ctypes.c_float * 16)()
    _load().nf4_codebook(out)
    return [float(v) for v in out]


# ---- allocation conveniences (torch allocates; the library is then called) ----
def empty_packed(N, K, device):
    codes = torch.empty((N, K // 2), dtype=torch.uint8, device=device)
    scales = torch.empty((N, K // GROUP), dtype=torch.int16, device=device)
    return codes, scales


def pack(W, stream=None, check=True):
    """Allocate and fill (codes, scales) for W; with check=True raise on flagged groups."""
    N, K = W.shape
    codes, scales = empty_packed(N, K, W.device)
    status = torch.zeros(1, dtype=torch.int32, device=W.device) if check else None
    nf4_pack(W, codes, scales, status, stream)
    if check:
        st = int(status.item())
        if st:
            raise ValueError(f"nf4_pack flagged groups: status bits {st:#x}")
    return codes, scales


def unpack(codes, scales, K, stream=None):
    W = torch.empty((codes.shape[0], K), dtype=torch.float32, device=codes.device)
    nf4_unpack(codes, scales, W, stream)
    return W


def gemv(codes, scales, x, stream=None):
    y = torch.empty(codes.shape[0], dtype=torch.float32, device=x.device)
    nf4_gemv(codes, scales, x, y, stream)
    return y


def embed(codes, scales, K, ids, stream=None):
    out = torch.empty((ids.numel(), K), dtype=torch.bfloat16, device=codes.device)
    nf4_embed(codes, scales, K, ids, out, None, stream)
    return out


def gemm(codes, scales, X, stream=None):
    """Y = X . dequant(codes, scales)^T for any M: up to MAX_M rows on the
    small-batch kernels (with a kept workspace where K splits over workgroups),
    beyond that on the prefill tiles."""
    M = 1 if X.dim() == 1 else X.shape[0]
    Y = torch.empty((M, codes.shape[0]), dtype=torch.float32, device=X.device)
    if M <= MAX_M:
        need = smallm_workspace_bytes(codes.shape[0], X.shape[-1], M)
        if need:
            nf4_gemm_smallm_ws(codes, scales, X, Y, workspace_for(X.device, need, stream), stream)
        else:
            nf4_gemm_smallm(codes, scales, X, Y, stream)
    else:
        need = prefill_workspace_bytes(codes.shape[0], X.shape[-1], M)
        if need:
            nf4_gemm_prefill_ws(codes, scales, X, Y, workspace_for(X.device, need, stream), stream)
        else:
            nf4_gemm_prefill(codes, scales, X, Y, stream)
    return Y
