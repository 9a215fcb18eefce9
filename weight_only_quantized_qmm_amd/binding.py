"""ctypes binding of libqmm.so (include/qmm.h), same names as the C ABI.

Argument marshalling only: torch tensors are passed as device pointers and
torch's current HIP stream is passed as the stream; every step of the matmul
runs in the library's kernels. PyTorch is used for device memory and streams.
The library must be built (``python -m weight_only_quantized_qmm_amd.build``);
if it is missing, every call raises -- there is no fallback implementation.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqmm.so")

QMM_OK = 0
QMM_ERR_ARG = -1
QMM_ERR_SHAPE = -2
QMM_ERR_ALIGN = -3
QMM_ERR_WORKSPACE = -4
QMM_ERR_HIP = -5
QMM_ERR_SIZE = -6
QMM_ERR_SCRATCH = -7
QMM_NOALLOC_SCRATCH_BYTES = 64 << 20
QMM_PARTIAL_BF16 = 0
QMM_PARTIAL_F32 = 1

# Every symbol include/qmm.h declares.
EXPORTED_FUNCTIONS = ("qmm_splitk_plan", "qmm_w4a16_g128", "qmm_splitk_reduce", "qmm_bf16_splitk",
                      "qmm_status_string", "qmm_w4a16_gemv", "qmm_gemv_min_split", "qmm_w4a16_g128_f32p",
                      "qmm_wna16", "qmm_wna16_plan", "qmm_attn_decode", "qmm_attn_decode_split",
                      "qmm_attn_decode_workspace_bytes", "qmm_w4a16_g128_streamk", "qmm_streamk_workspace_bytes",
                      "qmm_w4a16_g128_pass1", "qmm_splitk_reduce_cols", "qmm_w4a16_g128_noalloc")
EXPORTED_DATA = ("QMM_POLICY_PAGE", "QMM_POLICY_MI355X")


class QmmError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__("%s returned %d (%s)" % (where, status, qmm_status_string(status)))


class qmm_policy(ctypes.Structure):
    _fields_ = [("tile_m", ctypes.c_int), ("tile_n", ctypes.c_int), ("target_blocks", ctypes.c_int),
                ("cap", ctypes.c_int), ("min_k_per_split", ctypes.c_int)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class qmm_plan(ctypes.Structure):
    _fields_ = [("s", ctypes.c_int), ("base_tiles", ctypes.c_int), ("tile_m", ctypes.c_int),
                ("tile_n", ctypes.c_int), ("grid_x", ctypes.c_int), ("grid_y", ctypes.c_int),
                ("grid_z", ctypes.c_int), ("block_m", ctypes.c_int), ("block_n", ctypes.c_int),
                ("workspace_bytes", ctypes.c_size_t), ("full_tiles", ctypes.c_int)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


_LIB = None


def lib():
    """The loaded libqmm.so; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libqmm.so is not built (%s); run python -m weight_only_quantized_qmm_amd.build"
                               % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        I, P, S = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
        L.qmm_splitk_plan.argtypes = [I, I, I, I, ctypes.POINTER(qmm_policy), ctypes.POINTER(qmm_plan)]
        L.qmm_splitk_plan.restype = I
        L.qmm_w4a16_g128.argtypes = [P, P, P, P, P, I, I, I, I, P, S, P]
        L.qmm_w4a16_g128.restype = I
        L.qmm_w4a16_g128_noalloc.argtypes = [P, P, P, P, P, I, I, I, I, P]
        L.qmm_w4a16_g128_noalloc.restype = I
        L.qmm_w4a16_g128_f32p.argtypes = [P, P, P, P, P, I, I, I, I, P, S, P]
        L.qmm_w4a16_g128_f32p.restype = I
        L.qmm_w4a16_g128_streamk.argtypes = [P, P, P, P, P, I, I, I, I, P, S, P]
        L.qmm_w4a16_g128_streamk.restype = I
        L.qmm_streamk_workspace_bytes.argtypes = [I, I, I, I]
        L.qmm_streamk_workspace_bytes.restype = S
        L.qmm_wna16.argtypes = [I, I, I, P, P, P, P, P, I, I, I, I, P, S, P]
        L.qmm_wna16.restype = I
        L.qmm_wna16_plan.argtypes = [I, I, I, I, I, ctypes.POINTER(qmm_policy), ctypes.POINTER(qmm_plan)]
        L.qmm_wna16_plan.restype = I
        L.qmm_splitk_reduce.argtypes = [P, I, I, I, I, P, P]
        L.qmm_splitk_reduce.restype = I
        L.qmm_w4a16_g128_pass1.argtypes = [P, P, P, P, P, I, I, I, I, P, S, ctypes.POINTER(I), ctypes.POINTER(I), P]
        L.qmm_w4a16_g128_pass1.restype = I
        L.qmm_splitk_reduce_cols.argtypes = [P, I, I, I, I, I, P, P]
        L.qmm_splitk_reduce_cols.restype = I
        L.qmm_bf16_splitk.argtypes = [P, P, P, I, I, I, I, P, S, P]
        L.qmm_bf16_splitk.restype = I
        L.qmm_w4a16_gemv.argtypes = [P, P, P, P, P, I, I, I, I, P, S, P]
        L.qmm_w4a16_gemv.restype = I
        L.qmm_attn_decode.argtypes = [P, P, P, P, P, I, I, I, I, I, I, ctypes.c_float, I, P, S, P]
        L.qmm_attn_decode.restype = I
        L.qmm_attn_decode_split.argtypes = [I, I, I]
        L.qmm_attn_decode_split.restype = I
        L.qmm_attn_decode_workspace_bytes.argtypes = [I, I, I, I]
        L.qmm_attn_decode_workspace_bytes.restype = S
        L.qmm_gemv_min_split.argtypes = [I, I]
        L.qmm_gemv_min_split.restype = I
        L.qmm_status_string.argtypes = [I]
        L.qmm_status_string.restype = ctypes.c_char_p
        _LIB = L
    return _LIB


def qmm_status_string(status):
    return lib().qmm_status_string(int(status)).decode()


def policy_preset(name):
    """QMM_POLICY_PAGE or QMM_POLICY_MI355X as a qmm_policy value."""
    if name not in EXPORTED_DATA:
        raise KeyError(name)
    p = qmm_policy.in_dll(lib(), name)
    return qmm_policy(p.tile_m, p.tile_n, p.target_blocks, p.cap, p.min_k_per_split)


def qmm_splitk_plan(M, N, K, group_size=128, policy=None):
    """Host-only plan (no device); returns a qmm_plan, raises QmmError on a bad shape."""
    out = qmm_plan()
    pol = ctypes.byref(policy) if policy is not None else None
    rc = lib().qmm_splitk_plan(int(M), int(N), int(K), int(group_size), pol, ctypes.byref(out))
    if rc != QMM_OK:
        raise QmmError(rc, "qmm_splitk_plan")
    return out


def qmm_wna16_plan(bits, group_size, M, N, K, policy=None):
    """Host-only plan for a (bits, group_size) weight format; returns a qmm_plan."""
    out = qmm_plan()
    pol = ctypes.byref(policy) if policy is not None else None
    rc = lib().qmm_wna16_plan(int(bits), int(group_size), int(M), int(N), int(K), pol, ctypes.byref(out))
    if rc != QMM_OK:
        raise QmmError(rc, "qmm_wna16_plan")
    return out


def _ptr(x):
    """Device pointer of a tensor (or an int address / None)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _nbytes(t):
    if t is None:
        return 0
    return t.numel() * t.element_size()


def qmm_w4a16_g128(A, Wq, scale, bias, C, M, N, K, s=0, workspace=None, workspace_bytes=None,
                   stream=None, check=True):
    """C = A . dequant(W)^T on `stream` (torch's current stream by default); returns the status."""
    if workspace_bytes is None:
        workspace_bytes = _nbytes(workspace) if not isinstance(workspace, int) else 0
    rc = lib().qmm_w4a16_g128(_ptr(A), _ptr(Wq), _ptr(scale), _ptr(bias), _ptr(C), int(M), int(N), int(K),
                              int(s), _ptr(workspace), int(workspace_bytes), _stream(stream))
    if check and rc != QMM_OK:
        raise QmmError(rc, "qmm_w4a16_g128")
    return rc


def qmm_w4a16_g128_noalloc(A, Wq, scale, bias, C, M, N, K, s=0, stream=None, check=True):
    """qmm_w4a16_g128 with the split's planes in the library's static device scratch (no
    workspace argument, nothing allocated); returns the status."""
    rc = lib().qmm_w4a16_g128_noalloc(_ptr(A), _ptr(Wq), _ptr(scale), _ptr(bias), _ptr(C), int(M), int(N), int(K),
                                      int(s), _stream(stream))
    if check and rc != QMM_OK:
        raise QmmError(rc, "qmm_w4a16_g128_noalloc")
    return rc


def qmm_w4a16_g128_pass1(A, Wq, scale, bias, C, M, N, K, s=0, workspace=None, workspace_bytes=None,
                         stream=None, check=True):
    """The matmul launch of qmm_w4a16_g128 alone; returns (status, s, n_lo): the effective split
    and the first column whose outputs are left in the workspace planes."""
    if workspace_bytes is None:
        workspace_bytes = _nbytes(workspace) if not isinstance(workspace, int) else 0
    s_out, n_lo = ctypes.c_int(0), ctypes.c_int(0)
    rc = lib().qmm_w4a16_g128_pass1(_ptr(A), _ptr(Wq), _ptr(scale), _ptr(bias), _ptr(C), int(M), int(N), int(K),
                                    int(s), _ptr(workspace), int(workspace_bytes), ctypes.byref(s_out),
                                    ctypes.byref(n_lo), _stream(stream))
    if check and rc != QMM_OK:
        raise QmmError(rc, "qmm_w4a16_g128_pass1")
    return rc, s_out.value, n_lo.value


def qmm_w4a16_g128_f32p(A, Wq, scale, bias, C, M, N, K, s=0, workspace=None, workspace_bytes=None,
                        stream=None, check=True):
    """qmm_w4a16_g128 with fp32 partial planes (workspace >= 4*s*M*N bytes); returns the status."""
    if workspace_bytes is None:
        workspace_bytes = _nbytes(workspace) if not isinstance(workspace, int) else 0
    rc = lib().qmm_w4a16_g128_f32p(_ptr(A), _ptr(Wq), _ptr(scale), _ptr(bias), _ptr(C), int(M), int(N), int(K),
                                   int(s), _ptr(workspace), int(workspace_bytes), _stream(stream))
    if check and rc != QMM_OK:
        raise QmmError(rc, "qmm_w4a16_g128_f32p")
    return rc


def qmm_w4a16_g128_streamk(A, Wq, scale, bias, C, M, N, K, workgroups=0, workspace=None, workspace_bytes=None,
                           stream=None, check=True):
    """C = A . dequant(W)^T with the stream-K decomposition (M > 64); returns the status."""
    if workspace_bytes is None:
        workspace_bytes = _nbytes(workspace) if not isinstance(workspace, int) else 0
    rc = lib().qmm_w4a16_g128_streamk(_ptr(A), _ptr(Wq), _ptr(scale), _ptr(bias), _ptr(C), int(M), int(N), int(K),
                                      int(workgroups), _ptr(workspace), int(workspace_bytes), _stream(stream))
    if check and rc != QMM_OK:
        raise QmmError(rc, "qmm_w4a16_g128_streamk")
    return rc


def qmm_streamk_workspace_bytes(M, N, K, workgroups=0):
    return int(lib().qmm_streamk_workspace_bytes(int(M), int(N), int(K), int(workgroups)))


def qmm_wna16(bits, group_size, partial_dtype, A, Wq, scale, bias, C, M, N, K, s=0, workspace=None,
              workspace_bytes=None, stream=None, check=True):
    """C = A . dequant(W)^T for `bits`-wide codes and scale/bias groups of group_size; returns the status."""
    if workspace_bytes is None:
        workspace_bytes = _nbytes(workspace) if not isinstance(workspace, int) else 0
    rc = lib().qmm_wna16(int(bits), int(group_size), int(partial_dtype), _ptr(A), _ptr(Wq), _ptr(scale),
                         _ptr(bias), _ptr(C), int(M), int(N), int(K), int(s), _ptr(workspace),
                         int(workspace_bytes), _stream(stream))
    if check and rc != QMM_OK:
        raise QmmError(rc, "qmm_wna16")
    return rc


def qmm_w4a16_gemv(A, Wq, scale, bias, C, M, N, K, s=0, workspace=None, workspace_bytes=None,
                   stream=None, check=True):
    """C = A . dequant(W)^T for M <= 8 on the matrix-vector kernel; returns the status."""
    if workspace_bytes is None:
        workspace_bytes = _nbytes(workspace) if not isinstance(workspace, int) else 0
    rc = lib().qmm_w4a16_gemv(_ptr(A), _ptr(Wq), _ptr(scale), _ptr(bias), _ptr(C), int(M), int(N), int(K),
                              int(s), _ptr(workspace), int(workspace_bytes), _stream(stream))
    if check and rc != QMM_OK:
        raise QmmError(rc, "qmm_w4a16_gemv")
    return rc


def qmm_attn_decode(Q, K, V, lengths, O, B, Mq, Hq, Hkv, Lmax, head_dim, scale, s=0, workspace=None,
                    workspace_bytes=None, stream=None, check=True):
    """Split-KV decode attention through the C ABI; returns the status."""
    if workspace_bytes is None:
        workspace_bytes = _nbytes(workspace) if not isinstance(workspace, int) else 0
    rc = lib().qmm_attn_decode(_ptr(Q), _ptr(K), _ptr(V), _ptr(lengths), _ptr(O), int(B), int(Mq), int(Hq), int(Hkv),
                               int(Lmax), int(head_dim), float(scale), int(s), _ptr(workspace), int(workspace_bytes),
                               _stream(stream))
    if check and rc != QMM_OK:
        raise QmmError(rc, "qmm_attn_decode")
    return rc


def qmm_attn_decode_split(B, Hkv, Lmax):
    rc = lib().qmm_attn_decode_split(int(B), int(Hkv), int(Lmax))
    if rc < 0:
        raise QmmError(rc, "qmm_attn_decode_split")
    return rc


def qmm_attn_decode_workspace_bytes(B, Mq, Hq, s):
    return int(lib().qmm_attn_decode_workspace_bytes(int(B), int(Mq), int(Hq), int(s)))


def qmm_gemv_min_split(M, K):
    """The split qmm_w4a16_gemv uses for s = 0; raises on an invalid shape."""
    rc = lib().qmm_gemv_min_split(int(M), int(K))
    if rc < 0:
        raise QmmError(rc, "qmm_gemv_min_split")
    return rc


def qmm_splitk_reduce(partials, partial_dtype, s, M, N, C, stream=None, check=True):
    rc = lib().qmm_splitk_reduce(_ptr(partials), int(partial_dtype), int(s), int(M), int(N), _ptr(C),
                                 _stream(stream))
    if check and rc != QMM_OK:
        raise QmmError(rc, "qmm_splitk_reduce")
    return rc


def qmm_splitk_reduce_cols(partials, partial_dtype, s, M, N, n_lo, C, stream=None, check=True):
    rc = lib().qmm_splitk_reduce_cols(_ptr(partials), int(partial_dtype), int(s), int(M), int(N), int(n_lo), _ptr(C),
                                      _stream(stream))
    if check and rc != QMM_OK:
        raise QmmError(rc, "qmm_splitk_reduce_cols")
    return rc


def qmm_bf16_splitk(A, B, C, M, N, K, s=0, workspace=None, workspace_bytes=None, stream=None, check=True):
    if workspace_bytes is None:
        workspace_bytes = _nbytes(workspace) if not isinstance(workspace, int) else 0
    rc = lib().qmm_bf16_splitk(_ptr(A), _ptr(B), _ptr(C), int(M), int(N), int(K), int(s), _ptr(workspace),
                               int(workspace_bytes), _stream(stream))
    if check and rc != QMM_OK:
        raise QmmError(rc, "qmm_bf16_splitk")
    return rc


# ---------------------------------------------------------------- conveniences

def w4a16_workspace_bytes(M, N, s, f32_partials=False):
    return (4 if f32_partials else 2) * s * M * N if s > 1 else 0


def effective_split(M, N, K, s=0):
    return qmm_splitk_plan(M, N, K).s if s == 0 else s


def wna16(bits, group_size, A, Wq, scale, bias, s=0, out=None, workspace=None, f32_partials=False):
    """Allocating wrapper for qmm_wna16: A bf16[M,K], Wq int32/uint32[N, K*bits/32],
    scale/bias bf16[N, K/group_size] -> C bf16[M,N]."""
    import torch
    M, K = A.shape
    N = Wq.shape[0]
    s_eff = qmm_wna16_plan(bits, group_size, M, N, K).s if s == 0 else s
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    if s_eff > 1 and workspace is None:
        workspace = torch.empty(w4a16_workspace_bytes(M, N, s_eff, f32_partials), dtype=torch.uint8,
                                device=A.device)
    qmm_wna16(bits, group_size, QMM_PARTIAL_F32 if f32_partials else QMM_PARTIAL_BF16, A, Wq, scale, bias, out,
              M, N, K, s, workspace)
    return out


def w4a16(A, Wq, scale, bias, s=0, out=None, workspace=None, f32_partials=False):
    """Allocating wrapper: A bf16[M,K], Wq int32/uint32[N,K/8], scale/bias bf16[N,K/128] -> C bf16[M,N].

    f32_partials selects qmm_w4a16_g128_f32p (fp32 partial planes)."""
    import torch
    M, K = A.shape
    N = Wq.shape[0]
    s_eff = effective_split(M, N, K, s)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    if s_eff > 1 and workspace is None:
        workspace = torch.empty(w4a16_workspace_bytes(M, N, s_eff, f32_partials), dtype=torch.uint8,
                                device=A.device)
    # s = 0 goes to the library as is: its plan may also run part of the tiles unsplit
    fn = qmm_w4a16_g128_f32p if f32_partials else qmm_w4a16_g128
    fn(A, Wq, scale, bias, out, M, N, K, s, workspace)
    return out


def bf16_splitk(A, B, s=1, out=None, workspace=None):
    import torch
    M, K = A.shape
    N = B.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    if s > 1 and workspace is None:
        workspace = torch.empty(4 * s * M * N, dtype=torch.uint8, device=A.device)
    qmm_bf16_splitk(A, B, out, M, N, K, s, workspace)
    return out
