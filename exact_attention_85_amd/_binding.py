"""ctypes binding of libfa2.so (names as in include/fa2.h).

Argument marshalling only: dtype/device/contiguity checks, output and
workspace allocation with torch, and the raw stream handle.  Every step of the
attention computation runs in the library's kernels.
"""
import contextlib
import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libfa2.so")
# the race-check build (LDS slots filled with NaN before each asynchronous load)
_POISON_LIB_PATH = os.path.join(_PKG, "libfa2_poison.so")
FA2_MAX_SPLITS = 256

_lib = None


class Fa2Error(RuntimeError):
    """A non-zero fa2_status returned by the library."""

    def __init__(self, status: int, text: str):
        super().__init__(text)
        self.status = status


def lib_path() -> str:
    return _LIB_PATH


def poison_lib_path() -> str:
    return _POISON_LIB_PATH


def load_library():
    """Loads libfa2.so (built by exact_attention_85_amd/build.py).
    Raises if it is missing: there is no fallback path."""
    global _lib
    if _lib is not None:
        return _lib
    _lib = open_library(_LIB_PATH)
    return _lib


@contextlib.contextmanager
def library_at(path: str):
    """Routes this module's calls to the build at `path` (such as the race-check
    build) inside the block; the default library is used again afterwards.  It
    swaps one module-wide handle, so it is for single-threaded use (tests and
    measurements), not for code that calls the library from several threads."""
    global _lib
    saved = load_library()
    _lib = open_library(path)
    try:
        yield _lib
    finally:
        _lib = saved


def open_library(path: str):
    """A handle on the build at `path` with the C signatures of include/fa2.h declared."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run exact_attention_85_amd/build.py first")
    lib = ctypes.CDLL(path)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.fa2_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    lib.fa2_fwd.restype = i
    lib.fa2_fwd_splitkv_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
    lib.fa2_fwd_splitkv_noalloc.restype = i
    lib.fa2_splitkv_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.fa2_splitkv_workspace_bytes.restype = ctypes.c_size_t
    lib.fa2_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, ctypes.c_size_t, vp]
    lib.fa2_fwd_splitkv.restype = i
    lib.fa2_fwd_window.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp]
    lib.fa2_fwd_window.restype = i
    lib.fa2_bwd_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.fa2_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.fa2_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp, ctypes.c_size_t, vp]
    lib.fa2_bwd.restype = i
    lib.fa2_num_splits.argtypes = [i, i, i, i, i, i]
    lib.fa2_num_splits.restype = i
    lib.fa2_fp8_vt_stride.argtypes = [i]
    lib.fa2_fp8_vt_stride.restype = i
    lib.fa2_quantize_fp8.argtypes = [vp, vp, vp, i, i, i, i, i, vp]
    lib.fa2_quantize_fp8.restype = i
    lib.fa2_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    lib.fa2_fwd_fp8.restype = i
    lib.fa2_decode_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, vp]
    lib.fa2_decode_fp8.restype = i
    lib.fa2_fwd_blocksparse.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, vp, i, i, i, i, f, vp]
    lib.fa2_fwd_blocksparse.restype = i
    lib.fa2_fwd_config.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, vp]
    lib.fa2_fwd_config.restype = i
    lib.fa2_fwd_num_configs.argtypes = []
    lib.fa2_fwd_num_configs.restype = i
    lib.fa2_fwd_config_name.argtypes = [i]
    lib.fa2_fwd_config_name.restype = ctypes.c_char_p
    lib.fa2_fwd_default_config.argtypes = [i, i, i, i, i]
    lib.fa2_fwd_default_config.restype = i
    lib.fa2_probe_xcc.argtypes = [vp, i, vp]
    lib.fa2_probe_xcc.restype = i
    lib.fa2_status_string.argtypes = [i]
    lib.fa2_status_string.restype = ctypes.c_char_p
    return lib


def status_string(status: int) -> str:
    return load_library().fa2_status_string(int(status)).decode()


def _check(rc: int):
    if rc != 0:
        raise Fa2Error(rc, status_string(rc))


def _check_inputs(q, k, v):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be a bfloat16 torch tensor")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must live on the GPU")
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [B, H, N, d] tensor")
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k, v must be on the same device")
    B, H, n_q, d = q.shape
    n_k = k.shape[2]
    if tuple(k.shape) != (B, H, n_k, d) or tuple(v.shape) != (B, H, n_k, d):
        raise ValueError("k and v must be [B, H, N_k, d] with q's B, H, d")
    return B, H, n_q, n_k, d


def _check_out(t, name, shape, dtype, device):
    """A caller-supplied output: exactly `shape` and `dtype`, contiguous, on `device`.  The
    library sizes every write from the shape arguments, so anything else would be written out
    of bounds or read back wrongly."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous() or t.device != device:
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} on {device}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}"
                         f"{'' if t.is_contiguous() else ' (not contiguous)'}")
    return t


def _outputs(out, lse, B, H, n_q, d, device):
    """O and LSE buffers: the caller's (validated) or new ones."""
    if out is None:
        out = torch.empty((B, H, n_q, d), dtype=torch.bfloat16, device=device)
    else:
        _check_out(out, "out", (B, H, n_q, d), torch.bfloat16, device)
    if lse is None:
        lse = torch.empty((B, H, n_q), dtype=torch.float32, device=device)
    else:
        _check_out(lse, "lse", (B, H, n_q), torch.float32, device)
    return out, lse


def _scale(scale, d):
    return float(1.0 / math.sqrt(d)) if scale is None else float(scale)


def _stream_handle(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def forward(q, k, v, causal: bool = False, scale=None, out=None, lse=None):
    """O = softmax(scale * Q K^T [+ causal mask]) V and LSE, via fa2_fwd.

    q: [B, H, N_q, d], k, v: [B, H, N_k, d] bf16 contiguous on the GPU.
    Returns (o [B, H, N_q, d] bf16, lse [B, H, N_q] fp32).  The work is
    enqueued on torch's current stream of q's device."""
    lib = load_library()
    B, H, n_q, n_k, d = _check_inputs(q, k, v)
    out, lse = _outputs(out, lse, B, H, n_q, d, q.device)
    rc = lib.fa2_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                     B, H, n_q, n_k, d, int(bool(causal)), _scale(scale, d), _stream_handle(q.device))
    _check(rc)
    return out, lse


def forward_window(q, k, v, window_left: int, window_right: int, scale=None, out=None, lse=None):
    """Sliding-window attention via fa2_fwd_window: key j visible to query i iff
    (window_left < 0 or j >= i - window_left) and (window_right < 0 or j <= i + window_right).
    Returns (o, lse); rows that see no key get O = 0 and LSE = -inf."""
    lib = load_library()
    B, H, n_q, n_k, d = _check_inputs(q, k, v)
    out, lse = _outputs(out, lse, B, H, n_q, d, q.device)
    rc = lib.fa2_fwd_window(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                            B, H, n_q, n_k, d, int(window_left), int(window_right), _scale(scale, d),
                            _stream_handle(q.device))
    _check(rc)
    return out, lse


MASK_BLOCK_Q, MASK_BLOCK_K = 128, 64  # FA2_MASK_BLOCK_Q, FA2_MASK_BLOCK_K


def forward_blocksparse(q, k, v, block_mask, window_left: int = -1, window_right: int = -1, scale=None, out=None,
                        lse=None):
    """Attention under a block mask via fa2_fwd_blocksparse.

    block_mask: uint8 tensor on q's device, [n_qb, n_kb], [Mh, n_qb, n_kb] or [Mb, Mh, n_qb, n_kb]
    with n_qb = ceil(N_q / 128), n_kb = ceil(N_k / 64), Mb in {1, B}, Mh in {1, H}; a non-zero
    entry makes its (128-row query block, 64-key block) visible, further limited by the band
    (window_left, window_right) as forward_window.  Returns (o, lse); rows that see no key get
    O = 0 and LSE = -inf."""
    lib = load_library()
    B, H, n_q, n_k, d = _check_inputs(q, k, v)
    if not isinstance(block_mask, torch.Tensor) or block_mask.dtype != torch.uint8:
        raise TypeError("block_mask must be a uint8 torch tensor")
    n_qb, n_kb = -(-n_q // MASK_BLOCK_Q), -(-n_k // MASK_BLOCK_K)
    m = block_mask
    while m.dim() < 4:
        m = m.unsqueeze(0)
    if (m.dim() != 4 or tuple(m.shape[2:]) != (n_qb, n_kb) or m.shape[0] not in (1, B) or m.shape[1] not in (1, H)
            or not m.is_contiguous() or m.device != q.device):
        raise ValueError(f"block_mask must be a contiguous uint8 [Mb, Mh, {n_qb}, {n_kb}] tensor on q's device "
                         f"(Mb in {{1, {B}}}, Mh in {{1, {H}}}), got {tuple(block_mask.shape)} on {block_mask.device}")
    out, lse = _outputs(out, lse, B, H, n_q, d, q.device)
    rc = lib.fa2_fwd_blocksparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                 B, H, n_q, n_k, d, m.data_ptr(), int(m.shape[0]), int(m.shape[1]),
                                 int(window_left), int(window_right), _scale(scale, d), _stream_handle(q.device))
    _check(rc)
    return out, lse


def num_configs() -> int:
    """Number of forward configurations (kernel x workgroup order) fa2_fwd_config accepts."""
    return int(load_library().fa2_fwd_num_configs())


def config_name(config: int) -> str:
    name = load_library().fa2_fwd_config_name(int(config))
    if name is None:
        raise ValueError(f"no forward configuration {config}")
    return name.decode()


def default_config(d: int, banded: bool, n_q: int, B: int = 1, H: int = 1) -> int:
    """The configuration fa2_fwd / fa2_fwd_window take for the shape (the tuned table)."""
    rc = int(load_library().fa2_fwd_default_config(int(d), int(bool(banded)), int(n_q), int(B), int(H)))
    if rc < 0:
        _check(rc)
    return rc


def forward_config(q, k, v, config: int, window_left: int = -1, window_right: int = -1, scale=None, out=None,
                   lse=None):
    """fa2_fwd_window with an explicit forward configuration (see config_name); causal is the
    window (-1, 0).  Returns (o, lse)."""
    lib = load_library()
    B, H, n_q, n_k, d = _check_inputs(q, k, v)
    out, lse = _outputs(out, lse, B, H, n_q, d, q.device)
    rc = lib.fa2_fwd_config(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                            B, H, n_q, n_k, d, int(window_left), int(window_right), _scale(scale, d), int(config),
                            _stream_handle(q.device))
    _check(rc)
    return out, lse


def probe_xcc(n_workgroups: int, device="cuda"):
    """fa2_probe_xcc: (xcd [n], hw_id [n]) int32 tensors on the host, for workgroups 0 .. n-1
    of one launch."""
    lib = load_library()
    dev = torch.device(device)
    out = torch.full((n_workgroups, 2), -1, dtype=torch.int32, device=dev)
    _check(lib.fa2_probe_xcc(out.data_ptr(), int(n_workgroups), _stream_handle(dev)))
    out = out.cpu()
    return out[:, 0], out[:, 1]


def splitkv_workspace_bytes(B, H, n_q, d, num_splits) -> int:
    return int(load_library().fa2_splitkv_workspace_bytes(B, H, n_q, d, num_splits))


def forward_splitkv(q, k, v, num_splits: int = 16, causal: bool = False, scale=None, workspace=None,
                    out=None, lse=None):
    """Same result as forward(), with the key sequence split into num_splits chunks
    (fp32 partials in a workspace, then a merge pass), via fa2_fwd_splitkv.

    Returns (o, lse).  A caller-supplied workspace (fp32, contiguous, on q's device, at least
    splitkv_workspace_bytes() bytes) holds the per-chunk partials afterwards: acc [S][R][d],
    then m and l, each [S][R] (R = B*H*N_q), with acc / l the chunk's output and m + log(l)
    its log-sum-exp."""
    lib = load_library()
    B, H, n_q, n_k, d = _check_inputs(q, k, v)
    need = lib.fa2_splitkv_workspace_bytes(B, H, n_q, d, int(num_splits))
    if workspace is None:
        workspace = torch.empty((max(need, 4) + 3) // 4, dtype=torch.float32, device=q.device)
    elif (not isinstance(workspace, torch.Tensor) or workspace.dtype != torch.float32
          or not workspace.is_contiguous() or workspace.device != q.device):
        raise ValueError("workspace must be a contiguous fp32 tensor on q's device")
    out, lse = _outputs(out, lse, B, H, n_q, d, q.device)
    rc = lib.fa2_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                             B, H, n_q, n_k, d, int(bool(causal)), _scale(scale, d), int(num_splits),
                             workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                             _stream_handle(q.device))
    _check(rc)
    return out, lse


NOALLOC_SCRATCH_BYTES = 32 << 20  # FA2_NOALLOC_SCRATCH_BYTES


def forward_splitkv_noalloc(q, k, v, num_splits: int = 16, causal: bool = False, scale=None, out=None, lse=None):
    """forward_splitkv() with the partials in the library's own fixed device array
    (fa2_fwd_splitkv_noalloc): no workspace, nothing allocated by the library.  Pass out and
    lse to allocate nothing at all.  Calls that overlap on one GPU share that array and race.
    Returns (o, lse); raises Fa2Error (FA2_ERR_SCRATCH) when the partials would exceed
    NOALLOC_SCRATCH_BYTES."""
    lib = load_library()
    B, H, n_q, n_k, d = _check_inputs(q, k, v)
    out, lse = _outputs(out, lse, B, H, n_q, d, q.device)
    rc = lib.fa2_fwd_splitkv_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                     B, H, n_q, n_k, d, int(bool(causal)), _scale(scale, d), int(num_splits),
                                     _stream_handle(q.device))
    _check(rc)
    return out, lse


def num_splits(B, H, n_q, n_k, d, num_cus: int = 0) -> int:
    """fa2_num_splits: the key-chunk count that fills num_cus compute units
    (0 = ask the current HIP device).  Raises Fa2Error on bad arguments."""
    rc = int(load_library().fa2_num_splits(int(B), int(H), int(n_q), int(n_k), int(d), int(num_cus)))
    if rc < 0:
        _check(rc)
    return rc


def attention(q, k, v, causal: bool = False, scale=None):
    """forward() or forward_splitkv(), whichever fa2_num_splits picks for q's
    device: a split count of 1 (or a single query row) takes fa2_fwd, otherwise
    the split path with a workspace from torch's allocator.  Returns (o, lse)."""
    B, H, n_q, n_k, d = _check_inputs(q, k, v)
    with torch.cuda.device(q.device):
        s = num_splits(B, H, n_q, n_k, d, 0)
    if s == 1:
        return forward(q, k, v, causal=causal, scale=scale)
    return forward_splitkv(q, k, v, num_splits=s, causal=causal, scale=scale)


def bwd_workspace_bytes(B, H, n_q, n_k, d) -> int:
    return int(load_library().fa2_bwd_workspace_bytes(B, H, n_q, n_k, d))


def backward(q, k, v, o, lse, do, causal: bool = False, scale=None, workspace=None, dq=None, dk=None, dv=None):
    """Gradients (dq, dk, dv) of O = forward(q, k, v, causal, scale) for upstream
    gradient do, from that forward's o and lse, via fa2_bwd (deterministic)."""
    lib = load_library()
    B, H, n_q, n_k, d = _check_inputs(q, k, v)
    for name, t, shape in (("o", o, (B, H, n_q, d)), ("do", do, (B, H, n_q, d))):
        if t.dtype != torch.bfloat16 or tuple(t.shape) != shape or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous bf16 {shape} tensor on q's device")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, n_q) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 [B, H, N_q] tensor")
    if lse.device != q.device:
        raise ValueError("lse must be on q's device")
    need = lib.fa2_bwd_workspace_bytes(B, H, n_q, n_k, d)
    if workspace is None:
        workspace = torch.empty((max(need, 4) + 3) // 4, dtype=torch.float32, device=q.device)
    elif (not isinstance(workspace, torch.Tensor) or workspace.dtype != torch.float32
          or not workspace.is_contiguous() or workspace.device != q.device):
        raise ValueError("workspace must be a contiguous fp32 tensor on q's device")
    dq = torch.empty_like(q) if dq is None else _check_out(dq, "dq", q.shape, torch.bfloat16, q.device)
    dk = torch.empty_like(k) if dk is None else _check_out(dk, "dk", k.shape, torch.bfloat16, q.device)
    dv = torch.empty_like(v) if dv is None else _check_out(dv, "dv", v.shape, torch.bfloat16, q.device)
    rc = lib.fa2_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                     dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, n_q, n_k, d, int(bool(causal)),
                     _scale(scale, d), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                     _stream_handle(q.device))
    _check(rc)
    return dq, dk, dv


def fp8_vt_stride(n_k: int) -> int:
    """Row stride (keys) of a transposed V code tensor: n_k rounded up to a multiple of 16."""
    rc = int(load_library().fa2_fp8_vt_stride(int(n_k)))
    if rc < 0:
        _check(rc)
    return rc


def quantize_fp8(x, transposed: bool = False):
    """Per-(batch, head) e4m3 quantisation of bf16 x [B, H, N, d] via fa2_quantize_fp8.

    Returns (codes, descale): codes uint8 [B, H, N, d], or [B, H, d, fp8_vt_stride(N)] when
    transposed (the V layout fa2_fwd_fp8 takes); descale fp32 [B, H] = amax / 448."""
    lib = load_library()
    if not isinstance(x, torch.Tensor) or x.dtype != torch.bfloat16 or x.device.type != "cuda":
        raise TypeError("x must be a bfloat16 tensor on the GPU")
    if x.dim() != 4 or not x.is_contiguous():
        raise ValueError("x must be a contiguous [B, H, N, d] tensor")
    B, H, n, d = x.shape
    if transposed:
        codes = torch.empty((B, H, d, fp8_vt_stride(n)), dtype=torch.uint8, device=x.device)
    else:
        codes = torch.empty((B, H, n, d), dtype=torch.uint8, device=x.device)
    descale = torch.empty((B, H), dtype=torch.float32, device=x.device)
    rc = lib.fa2_quantize_fp8(x.data_ptr(), codes.data_ptr(), descale.data_ptr(), B, H, n, d,
                              int(bool(transposed)), _stream_handle(x.device))
    _check(rc)
    return codes, descale


def forward_fp8(qc, kc, vt, descale_q, descale_k, descale_v, causal: bool = False, scale=None, out=None,
                lse=None):
    """Attention forward on e4m3 codes via fa2_fwd_fp8.

    qc [B, H, N_q, d], kc [B, H, N_k, d] uint8 codes; vt [B, H, d, fp8_vt_stride(N_k)] codes of V
    transposed; descales fp32 [B, H].  Returns (o bf16 [B, H, N_q, d], lse fp32 [B, H, N_q])."""
    lib = load_library()
    for name, t in (("qc", qc), ("kc", kc), ("vt", vt)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.uint8 or t.device.type != "cuda":
            raise TypeError(f"{name} must be a uint8 tensor on the GPU")
        if t.dim() != 4 or not t.is_contiguous() or t.device != qc.device:
            raise ValueError(f"{name} must be a contiguous 4-d tensor on qc's device")
    B, H, n_q, d = qc.shape
    n_k = kc.shape[2]
    if tuple(kc.shape) != (B, H, n_k, d) or tuple(vt.shape) != (B, H, d, fp8_vt_stride(n_k)):
        raise ValueError("kc must be [B, H, N_k, d] and vt [B, H, d, fp8_vt_stride(N_k)]")
    for name, t in (("descale_q", descale_q), ("descale_k", descale_k), ("descale_v", descale_v)):
        if t.dtype != torch.float32 or tuple(t.shape) != (B, H) or not t.is_contiguous() or t.device != qc.device:
            raise ValueError(f"{name} must be a contiguous fp32 [B, H] tensor on qc's device")
    out, lse = _outputs(out, lse, B, H, n_q, d, qc.device)
    rc = lib.fa2_fwd_fp8(qc.data_ptr(), kc.data_ptr(), vt.data_ptr(), descale_q.data_ptr(), descale_k.data_ptr(),
                         descale_v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, n_q, n_k, d,
                         int(bool(causal)), _scale(scale, d), _stream_handle(qc.device))
    _check(rc)
    return out, lse


def decode_fp8(qc, kc, vc, descale_q, descale_k, descale_v, scale=None, out=None, lse=None):
    """One decode step over an FP8 K/V cache via fa2_decode_fp8.

    qc [B, H, 1, d], kc and vc [B, H, N_k, d] uint8 codes in row layout; descales fp32 [B, H].
    Returns (o bf16 [B, H, 1, d], lse fp32 [B, H, 1])."""
    lib = load_library()
    for name, t in (("qc", qc), ("kc", kc), ("vc", vc)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.uint8 or t.device.type != "cuda":
            raise TypeError(f"{name} must be a uint8 tensor on the GPU")
        if t.dim() != 4 or not t.is_contiguous() or t.device != qc.device:
            raise ValueError(f"{name} must be a contiguous 4-d tensor on qc's device")
    B, H, n_q, d = qc.shape
    n_k = kc.shape[2]
    if n_q != 1 or tuple(kc.shape) != (B, H, n_k, d) or tuple(vc.shape) != (B, H, n_k, d):
        raise ValueError("qc must be [B, H, 1, d] and kc, vc [B, H, N_k, d]")
    for name, t in (("descale_q", descale_q), ("descale_k", descale_k), ("descale_v", descale_v)):
        if t.dtype != torch.float32 or tuple(t.shape) != (B, H) or not t.is_contiguous() or t.device != qc.device:
            raise ValueError(f"{name} must be a contiguous fp32 [B, H] tensor on qc's device")
    out, lse = _outputs(out, lse, B, H, 1, d, qc.device)
    rc = lib.fa2_decode_fp8(qc.data_ptr(), kc.data_ptr(), vc.data_ptr(), descale_q.data_ptr(),
                            descale_k.data_ptr(), descale_v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                            B, H, n_k, d, _scale(scale, d), _stream_handle(qc.device))
    _check(rc)
    return out, lse
