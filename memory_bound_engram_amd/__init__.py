"""libengram: the four-stream Engram saved-state gate on AMD MI355X (gfx950).

A thin ctypes binding over the C ABI declared in ``include/engram.h``.  It only
marshals arguments (device pointers, N, the current stream) after checking
that each tensor has the element type, size and device the call will touch;
every step of the computation runs in the HIP kernels of ``libengram.so``.  There is no
fallback: if the library is missing, importing this package raises.

PyTorch is used only as a source of device memory and streams.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libengram.so")

STREAMS = 4
HIDDEN = 5120
KV_COLS = 25600
N_MAX = 4194240
BWD_N_MAX = 8192
BWD_N_MULTIPLE = 64

OK, ERR_NULL, ERR_N_RANGE, ERR_N_MULT64, ERR_ALIGN, ERR_OVERLAP, ERR_LAUNCH = range(7)

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libengram.so is not built ({LIB_PATH}); run __graft_entry__.build() "
                      "or python memory_bound_engram_amd/build.py")


def _hip_runtimes():
    """Paths of every libamdhip64 mapped into this process."""
    try:
        with open("/proc/self/maps") as f:
            return sorted({line.split()[-1] for line in f if "libamdhip64" in line})
    except OSError:  # pragma: no cover
        return []


# Streams and device memory come from PyTorch, which ships its own copy of the
# HIP runtime (same soname as /opt/rocm's).  libengram must bind to that copy:
# load torch first so the dynamic loader resolves libamdhip64.so.7 to it.
try:
    import torch as _torch  # noqa: F401
except ImportError:  # the C ABI alone (no torch) binds to the system runtime
    _torch = None

lib = ctypes.CDLL(LIB_PATH)
if len(_hip_runtimes()) > 1:
    raise ImportError("two HIP runtimes are loaded in this process " + str(_hip_runtimes()) +
                      "; libengram would not see torch's streams and memory")
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
lib.engram_gate_fwd.argtypes = [_P, _P, _P, _P, _P, _P, _I64, _P]
lib.engram_gate_fwd.restype = ctypes.c_int
lib.engram_gate_bwd.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _P]
lib.engram_gate_bwd.restype = ctypes.c_int
lib.engram_gate_bwd_with_norm_weights.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _P]
lib.engram_gate_bwd_with_norm_weights.restype = ctypes.c_int
lib.engram_gate_bwd_noalloc.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _I64, _P]
lib.engram_gate_bwd_noalloc.restype = ctypes.c_int
lib.engram_fused_weight.argtypes = [_P, _P, _P, _P]
lib.engram_fused_weight.restype = ctypes.c_int
lib.engram_gate_bwd_workspace_bytes.argtypes = [_I64]
lib.engram_gate_bwd_workspace_bytes.restype = ctypes.c_size_t
lib.engram_gateconv_fwd.argtypes = [_P] * 12 + [_I64, _I64, _I64, ctypes.c_float, _P]
lib.engram_gateconv_fwd.restype = ctypes.c_int
lib.engram_gateconv_bwd.argtypes = [_P] * 19 + [_I64, _I64, _I64, _P]
lib.engram_gateconv_bwd.restype = ctypes.c_int
lib.engram_gateconv_bwd_workspace_bytes.argtypes = [_I64, _I64, _I64]
lib.engram_gateconv_bwd_workspace_bytes.restype = ctypes.c_size_t
lib.engram_status_string.argtypes = [ctypes.c_int]
lib.engram_status_string.restype = ctypes.c_char_p
lib.engram_last_hip_error.argtypes = []
lib.engram_last_hip_error.restype = ctypes.c_int


class EngramError(RuntimeError):
    def __init__(self, status: int):
        msg = lib.engram_status_string(status).decode()
        if status == ERR_LAUNCH:
            msg += f" (hipError {lib.engram_last_hip_error()})"
        super().__init__(f"libengram status {status}: {msg}")
        self.status = status


def _check(status: int) -> None:
    if status != OK:
        raise EngramError(status)


def _ptr(t):
    """Device address of a tensor (or a raw int address); None stays NULL."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("libengram needs contiguous tensors")
    return t.data_ptr()


# Host-side checks of tensor arguments against the sizes a call will touch.
# The C ABI sees raw pointers only, so a tensor shorter than N rows, of the
# wrong element type or on another device would become out-of-bounds device
# accesses; these checks turn every such call into a ValueError before
# anything reaches the library.  A raw integer address is passed through
# unchecked: the caller then vouches for its size.
_BF16, _F32 = "bfloat16", "float32"
_BYTE_DTYPES = ("bool", "uint8", "int8")


def _dtype_name(t):
    return str(t.dtype).replace("torch.", "")


def _check_tensors(specs):
    """specs: (name, tensor or None or int, allowed dtype names, minimum element
    count).  Every tensor must have one of its dtypes, hold at least that many
    elements, be contiguous and live on the same CUDA/HIP device."""
    specs = [sp for sp in specs if sp[1] is not None and not isinstance(sp[1], int)]
    for name, t, dtypes, need in specs:
        if _dtype_name(t) not in dtypes:
            raise ValueError(f"{name}: dtype {_dtype_name(t)}, expected {' or '.join(dtypes)}")
        if t.numel() < need:
            raise ValueError(f"{name}: {t.numel()} elements, the call needs at least {need}")
        if not t.is_contiguous():
            raise ValueError(f"{name}: libengram needs contiguous tensors")
    device = None
    for name, t, _, _ in specs:
        if t.device.type != "cuda":
            raise ValueError(f"{name}: on {t.device}, libengram needs GPU (HIP) tensors")
        if device is None:
            device = t.device
        elif t.device != device:
            raise ValueError(f"{name}: on {t.device}, other arguments on {device}")


def _check_n(N, lo, hi):
    if not isinstance(N, int) or isinstance(N, bool):
        raise ValueError(f"N must be an int, got {type(N).__name__}")
    # sizes outside the accepted range are left to the library, which
    # rejects them with its own status (nothing would be touched)
    return lo <= N <= hi


def _gate_specs(N, x=None, kv=None, weight=None, mask=None, saved=None, grad_out=None, grad_x=None,
                grad_kv=None, grad_weight=None, workspace=None, out=None):
    row, kvrow = STREAMS * HIDDEN, KV_COLS
    return [("x", x, (_BF16,), N * row), ("kv", kv, (_BF16,), N * kvrow),
            ("weight", weight, (_F32,), STREAMS * HIDDEN), ("mask", mask, _BYTE_DTYPES, N),
            ("out", out, (_BF16,), N * row), ("saved", saved, (_F32,), N * STREAMS * 4),
            ("grad_out", grad_out, (_BF16,), N * row), ("grad_x", grad_x, (_BF16,), N * row),
            ("grad_kv", grad_kv, (_BF16,), N * kvrow), ("grad_weight", grad_weight, (_F32,), STREAMS * HIDDEN),
            ("workspace", workspace, _BYTE_DTYPES + (_F32,), 0)]


def _check_workspace(workspace, need_bytes):
    if workspace is None or isinstance(workspace, int):
        return
    have = workspace.numel() * workspace.element_size()
    if have < need_bytes:
        raise ValueError(f"workspace: {have} bytes, the call needs {need_bytes}")


def _stream(stream, *tensors):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    for t in tensors:
        if t is not None and not isinstance(t, int):
            return torch.cuda.current_stream(t.device).cuda_stream
    return torch.cuda.current_stream().cuda_stream


def engram_gate_bwd_workspace_bytes(N: int) -> int:
    """Backward scratch size in bytes: 4 * (16N + 4*5120*(N//64))."""
    return int(lib.engram_gate_bwd_workspace_bytes(N))


def engram_gate_fwd(x, kv, weight, mask, out, saved, N=None, stream=None) -> None:
    """Enqueue the forward on `stream` (default: the current torch stream).

    x [N,4,5120] bf16, kv [N,25600] bf16, weight [4,5120] fp32, mask [N]
    bool/uint8, out [N,4,5120] bf16 (written), saved [N,4,4] fp32 (written),
    or saved=None for the inference forward.
    """
    if N is None:
        N = x.shape[0]
    if _check_n(N, 1, N_MAX):
        _check_tensors(_gate_specs(N, x=x, kv=kv, weight=weight, mask=mask, out=out, saved=saved))
    _check(lib.engram_gate_fwd(_ptr(x), _ptr(kv), _ptr(weight), _ptr(mask), _ptr(out), _ptr(saved), N,
                               _stream(stream, x)))


def engram_gate_bwd(x, kv, weight, saved, grad_out, grad_x, grad_kv, grad_weight, workspace, N=None,
                    stream=None) -> None:
    """Enqueue the backward on `stream` (default: the current torch stream).

    grad_x [N,4,5120] bf16, grad_kv [N,25600] bf16 and grad_weight [4,5120]
    fp32 are written in full; workspace holds
    engram_gate_bwd_workspace_bytes(N) bytes of scratch.
    """
    if N is None:
        N = x.shape[0]
    _check_bwd_args(N, x, kv, weight, saved, grad_out, grad_x, grad_kv, grad_weight, workspace)
    _check(lib.engram_gate_bwd(_ptr(x), _ptr(kv), _ptr(weight), _ptr(saved), _ptr(grad_out), _ptr(grad_x),
                               _ptr(grad_kv), _ptr(grad_weight), _ptr(workspace), N, _stream(stream, x)))


def _check_bwd_args(N, x, kv, weight, saved, grad_out, grad_x, grad_kv, grad_weight, workspace, extra=()):
    if _check_n(N, 1, BWD_N_MAX):
        _check_workspace(workspace, engram_gate_bwd_workspace_bytes(N))
        _check_tensors(_gate_specs(N, x=x, kv=kv, weight=weight, saved=saved, grad_out=grad_out, grad_x=grad_x,
                                   grad_kv=grad_kv, grad_weight=grad_weight, workspace=workspace) + list(extra))


def engram_gate_bwd_with_norm_weights(x, kv, weight, saved, grad_out, grad_x, grad_kv, grad_weight, wh, we,
                                      grad_wh, grad_we, workspace, N=None, stream=None) -> None:
    """engram_gate_bwd plus grad_wh = grad_weight * we and grad_we = grad_weight * wh
    for weight = wh * we (wh, we [4,5120] bf16; grad_wh, grad_we [4,5120] fp32)."""
    if N is None:
        N = x.shape[0]
    w = STREAMS * HIDDEN
    _check_bwd_args(N, x, kv, weight, saved, grad_out, grad_x, grad_kv, grad_weight, workspace,
                    [("wh", wh, (_BF16,), w), ("we", we, (_BF16,), w), ("grad_wh", grad_wh, (_F32,), w),
                     ("grad_we", grad_we, (_F32,), w)])
    _check(lib.engram_gate_bwd_with_norm_weights(
        _ptr(x), _ptr(kv), _ptr(weight), _ptr(saved), _ptr(grad_out), _ptr(grad_x), _ptr(grad_kv),
        _ptr(grad_weight), _ptr(wh), _ptr(we), _ptr(grad_wh), _ptr(grad_we), _ptr(workspace), N,
        _stream(stream, x)))


NOALLOC_N_MAX = 8192


def engram_gate_bwd_noalloc(x, kv, weight, saved, grad_out, grad_x, grad_kv, grad_weight, N=None,
                            stream=None) -> None:
    """engram_gate_bwd without a workspace, for callers that cannot allocate:
    the partial rows live in the library's own per-GPU array (N <= 8192).
    Calls that overlap in time on one GPU race on that array."""
    if N is None:
        N = x.shape[0]
    if _check_n(N, 1, NOALLOC_N_MAX):
        _check_tensors(_gate_specs(N, x=x, kv=kv, weight=weight, saved=saved, grad_out=grad_out, grad_x=grad_x,
                                   grad_kv=grad_kv, grad_weight=grad_weight))
    _check(lib.engram_gate_bwd_noalloc(_ptr(x), _ptr(kv), _ptr(weight), _ptr(saved), _ptr(grad_out), _ptr(grad_x),
                                       _ptr(grad_kv), _ptr(grad_weight), N, _stream(stream, x)))


def engram_fused_weight(wh, we, weight, stream=None) -> None:
    """weight [4,5120] fp32 = float(wh) * float(we), wh and we [4,5120] bf16 (exact)."""
    w = STREAMS * HIDDEN
    _check_tensors([("wh", wh, (_BF16,), w), ("we", we, (_BF16,), w), ("weight", weight, (_F32,), w)])
    _check(lib.engram_fused_weight(_ptr(wh), _ptr(we), _ptr(weight), _stream(stream, wh)))


GATECONV_D_MAX = 5120
GATECONV_ROWS_MAX = 4194304


def engram_gateconv_bwd_workspace_bytes(M: int, T: int, d: int) -> int:
    """GateConv backward scratch size in bytes (0 for sizes the call rejects)."""
    return int(lib.engram_gateconv_bwd_workspace_bytes(M, T, d))


def engram_gateconv_fwd(H, k, v, rms_w_h, rms_w_v, conv_w, Y, vhat, alpha, rrms_h, rrms_k, rrms_v, eps=1e-6,
                        stream=None) -> None:
    """Enqueue the GateConv forward.  H, k, v, Y, vhat [M,T,d] bf16; rms_w_h,
    rms_w_v [d] fp32; conv_w [4,d] fp32; alpha, rrms_* [M,T] fp32 (written)."""
    M, T, d = H.shape
    rows = M * T
    _check_tensors([(n_, t_, (_BF16,), rows * d) for n_, t_ in (("H", H), ("k", k), ("v", v), ("Y", Y), ("vhat", vhat))]
                   + [(n_, t_, (_F32,), rows) for n_, t_ in (("alpha", alpha), ("rrms_h", rrms_h), ("rrms_k", rrms_k),
                                                             ("rrms_v", rrms_v))]
                   + [("rms_w_h", rms_w_h, (_F32,), d), ("rms_w_v", rms_w_v, (_F32,), d),
                      ("conv_w", conv_w, (_F32,), 4 * d)])
    _check(lib.engram_gateconv_fwd(_ptr(H), _ptr(k), _ptr(v), _ptr(rms_w_h), _ptr(rms_w_v), _ptr(conv_w), _ptr(Y),
                                   _ptr(vhat), _ptr(alpha), _ptr(rrms_h), _ptr(rrms_k), _ptr(rrms_v), M, T, d, eps,
                                   _stream(stream, H)))


def engram_gateconv_bwd(dY, H, k, v, rms_w_h, rms_w_v, conv_w, vhat, alpha, rrms_h, rrms_k, rrms_v, dH, dk, dv,
                        drms_w_h, drms_w_v, dconv_w, workspace, stream=None) -> None:
    """Enqueue the GateConv backward from the forward's saved tensors; dH, dk,
    dv [M,T,d] bf16 and drms_w_h, drms_w_v [d], dconv_w [4,d] fp32 are written
    in full; workspace holds engram_gateconv_bwd_workspace_bytes(M, T, d) bytes."""
    M, T, d = H.shape
    rows = M * T
    _check_workspace(workspace, engram_gateconv_bwd_workspace_bytes(M, T, d))
    _check_tensors([(n_, t_, (_BF16,), rows * d)
                    for n_, t_ in (("dY", dY), ("H", H), ("k", k), ("v", v), ("vhat", vhat), ("dH", dH), ("dk", dk),
                                   ("dv", dv))]
                   + [(n_, t_, (_F32,), rows) for n_, t_ in (("alpha", alpha), ("rrms_h", rrms_h), ("rrms_k", rrms_k),
                                                             ("rrms_v", rrms_v))]
                   + [(n_, t_, (_F32,), d) for n_, t_ in (("rms_w_h", rms_w_h), ("rms_w_v", rms_w_v),
                                                          ("drms_w_h", drms_w_h), ("drms_w_v", drms_w_v))]
                   + [("conv_w", conv_w, (_F32,), 4 * d), ("dconv_w", dconv_w, (_F32,), 4 * d),
                      ("workspace", workspace, _BYTE_DTYPES + (_F32,), 0)])
    _check(lib.engram_gateconv_bwd(_ptr(dY), _ptr(H), _ptr(k), _ptr(v), _ptr(rms_w_h), _ptr(rms_w_v), _ptr(conv_w),
                                   _ptr(vhat), _ptr(alpha), _ptr(rrms_h), _ptr(rrms_k), _ptr(rrms_v), _ptr(dH),
                                   _ptr(dk), _ptr(dv), _ptr(drms_w_h), _ptr(drms_w_v), _ptr(dconv_w),
                                   _ptr(workspace), M, T, d, _stream(stream, H)))


__all__ = ["engram_gate_bwd_noalloc", "engram_gateconv_fwd", "engram_gateconv_bwd", "engram_gateconv_bwd_workspace_bytes", "engram_gate_bwd_with_norm_weights", "engram_fused_weight", "engram_gate_fwd", "engram_gate_bwd", "engram_gate_bwd_workspace_bytes", "EngramError", "lib",
           "LIB_PATH"]
