"""Python binding of libnvfp4.so: the batched T-token NVFP4 W4A4 MLP on MI355X.

Argument marshalling only.  Every step of the path runs in the library's HIP
kernels; torch provides device memory and the current stream.  The functions
carry the C entry points' names (see include/nvfp4.h for the contract).

Importing this module loads the built library and fails loudly when it is
missing; there is no fallback implementation.
"""
import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built (python -m mlp_prefill_amd.build)")

_lib = ctypes.CDLL(LIB_PATH)

# ---- C types -------------------------------------------------------------------
_vp = ctypes.c_void_p
_i64 = ctypes.c_int64


class nvfp4_tensor(ctypes.Structure):
    _fields_ = [("codes", _vp), ("scales", _vp), ("gscale", _vp), ("tiled", _vp)]


OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_WORKSPACE, ERR_ARG, ERR_DEVICE, ERR_LAUNCH = range(8)
F32, BF16 = 0, 1
GS_COMPUTE, GS_GIVEN, GS_FROM_AMAX = 0, 1, 2
AMAX_SLOTS = 1024     # partial maxima written by an output-amax epilogue
EPI_STORE, EPI_SILU_MUL_REQUANT, EPI_SILU_MUL_QUANT_GIVEN = 0, 1, 2
KC_QUANTIZE, KC_EXPAND, KC_GEMM_GLU, KC_GEMM_STORE, KC_REDUCE, KC_ROUTE, KC_COMBINE = range(7)

_sig = {
    "nvfp4_quantize_act": [_vp, ctypes.c_int, _i64, _i64, _i64, nvfp4_tensor, ctypes.c_int, _vp,
                           ctypes.POINTER(ctypes.c_size_t), _vp],
    "nvfp4_quantize_act_noalloc": [_vp, ctypes.c_int, _i64, _i64, _i64, nvfp4_tensor, ctypes.c_int, _vp],
    "nvfp4_gemm": [nvfp4_tensor, nvfp4_tensor, _i64, _i64, _i64, _vp, ctypes.c_int, _i64, _vp, _vp,
                   ctypes.POINTER(ctypes.c_size_t), _vp],
    "nvfp4_mlp_gu_act": [nvfp4_tensor, nvfp4_tensor, nvfp4_tensor, _i64, _i64, _i64, nvfp4_tensor, _vp,
                         ctypes.POINTER(ctypes.c_size_t), _vp],
    "nvfp4_mlp_down": [nvfp4_tensor, nvfp4_tensor, _i64, _i64, _i64, _vp, ctypes.c_int, _i64, _vp, _vp,
                       ctypes.POINTER(ctypes.c_size_t), _vp],
    "nvfp4_mlp": [_vp, ctypes.c_int, _i64, _vp, _i64, _i64, _i64, nvfp4_tensor, nvfp4_tensor, nvfp4_tensor,
                  nvfp4_tensor, nvfp4_tensor, _vp, ctypes.c_int, _i64, _vp, _vp, ctypes.POINTER(ctypes.c_size_t), _vp],
    "nvfp4_mlp_gu_act_static": [nvfp4_tensor, nvfp4_tensor, nvfp4_tensor, _i64, _i64, _i64, nvfp4_tensor, _vp,
                                ctypes.POINTER(ctypes.c_size_t), _vp],
    "nvfp4_mlp_down_quant": [nvfp4_tensor, nvfp4_tensor, _i64, _i64, _i64, nvfp4_tensor, _vp,
                             ctypes.POINTER(ctypes.c_size_t), _vp],
    "nvfp4_grouped_gemm": [nvfp4_tensor, _vp, _vp, ctypes.c_int, _i64, nvfp4_tensor, nvfp4_tensor, _i64, _i64,
                           ctypes.c_int, _vp, ctypes.c_int, _i64, nvfp4_tensor, _vp,
                           ctypes.POINTER(ctypes.c_size_t), _vp],
    "nvfp4_rmsnorm_quantize_act": [_vp, ctypes.c_int, _i64, _i64, _i64, _vp, ctypes.c_float, nvfp4_tensor, _vp,
                                   ctypes.POINTER(ctypes.c_size_t), _vp],
    "nvfp4_moe_route": [_vp, _i64, ctypes.c_int, ctypes.c_int, _i64, _vp, _vp, _vp, _vp, _vp,
                        ctypes.POINTER(ctypes.c_size_t), _vp],
    "nvfp4_moe_combine": [_vp, ctypes.c_int, _i64, _vp, _vp, _i64, ctypes.c_int, _i64, _vp, ctypes.c_int, _i64,
                          _vp],
    "nvfp4_tile_weight": [nvfp4_tensor, _i64, _i64, _i64, _vp, ctypes.POINTER(ctypes.c_size_t), _vp],
    "nvfp4_moe_mlp": [_vp, ctypes.c_int, _i64, _i64, _i64, _i64, ctypes.c_int, _vp, _vp, _i64, nvfp4_tensor,
                      nvfp4_tensor, nvfp4_tensor, nvfp4_tensor, nvfp4_tensor, _vp, ctypes.c_int, _i64, _vp,
                      ctypes.POINTER(ctypes.c_size_t), _vp],
    "nvfp4_moe_mlp_static": [_vp, ctypes.c_int, _i64, _i64, _i64, _i64, ctypes.c_int, _vp, _vp, _i64, nvfp4_tensor,
                             nvfp4_tensor, nvfp4_tensor, nvfp4_tensor, nvfp4_tensor, _vp, ctypes.c_int, _i64, _vp,
                             ctypes.POINTER(ctypes.c_size_t), _vp],
}
for _name, _args in _sig.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = ctypes.c_int
_lib.nvfp4_strerror.argtypes = [ctypes.c_int]
_lib.nvfp4_strerror.restype = ctypes.c_char_p
_lib.nvfp4_launch_count.argtypes = []
_lib.nvfp4_launch_count.restype = ctypes.c_uint64
_lib.nvfp4_timing_begin.argtypes = [ctypes.c_int, _i64]
_lib.nvfp4_timing_begin.restype = ctypes.c_int
_lib.nvfp4_timing_end.argtypes = [ctypes.POINTER(_i64), ctypes.POINTER(_i64), ctypes.POINTER(ctypes.c_double)]
_lib.nvfp4_timing_end.restype = ctypes.c_int

lib = _lib


class Nvfp4Error(RuntimeError):
    def __init__(self, status, where):
        super().__init__(f"{where}: {_lib.nvfp4_strerror(status).decode()} (status {status})")
        self.status = status


def _check(status, where):
    if status != OK:
        raise Nvfp4Error(status, where)


def launch_count():
    """Kernel launches this library has enqueued in this process."""
    return int(_lib.nvfp4_launch_count())


def nvfp4_timing_begin(kernel_class, max_launches):
    """Open a timing window for one kernel class (see include/nvfp4.h)."""
    _check(_lib.nvfp4_timing_begin(kernel_class, max_launches), "nvfp4_timing_begin")


def nvfp4_timing_end():
    """Close the timing window: (launches timed, launches dropped, summed milliseconds)."""
    n, d, ms = _i64(0), _i64(0), ctypes.c_double(0.0)
    _check(_lib.nvfp4_timing_end(ctypes.byref(n), ctypes.byref(d), ctypes.byref(ms)), "nvfp4_timing_end")
    return n.value, d.value, ms.value


def _stream(stream=None):
    if stream is not None:
        return _vp(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))
    return _vp(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return _vp(t.data_ptr()) if t is not None else _vp(0)


# ---- device NVFP4 matrices --------------------------------------------------------
@dataclass
class NVFP4:
    """Device NVFP4 matrix [rows][cols] (or an expert stack [experts][rows][cols])."""
    codes: torch.Tensor     # uint8 [..., rows, cols // 2]
    scales: torch.Tensor    # uint8 [..., rows, cols // 16]
    gscale: torch.Tensor    # float32 [1] or [experts]
    rows: int
    cols: int
    tiled: torch.Tensor = None   # uint8: tile-contiguous copy of a weight (nvfp4_tile_weight), or None

    @staticmethod
    def empty(rows, cols, device="cuda", experts=None):
        lead = () if experts is None else (experts,)
        return NVFP4(torch.empty(lead + (rows, cols // 2), dtype=torch.uint8, device=device),
                     torch.empty(lead + (rows, cols // 16), dtype=torch.uint8, device=device),
                     torch.empty((experts or 1,), dtype=torch.float32, device=device),
                     rows, cols)

    @staticmethod
    def stack(mats):
        """Stack per-expert matrices into one [experts][rows][cols] operand."""
        return NVFP4(torch.stack([m.codes for m in mats]), torch.stack([m.scales for m in mats]),
                     torch.cat([m.gscale for m in mats]), mats[0].rows, mats[0].cols)

    def c(self):
        return nvfp4_tensor(self.codes.data_ptr(), self.scales.data_ptr(), self.gscale.data_ptr(),
                            self.tiled.data_ptr() if self.tiled is not None else 0)

    def tile(self, stream=None):
        """Write (or rewrite) this weight's tile-contiguous copy; returns self."""
        nvfp4_tile_weight(self, stream=stream)
        return self


def _null_tensor():
    return nvfp4_tensor(0, 0, 0, 0)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _foreign_stream(stream):
    """torch's handle of `stream` when it is not torch's current stream, else None."""
    if stream is None:
        return None
    ptr = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    if ptr == torch.cuda.current_stream().cuda_stream:
        return None
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(ptr)


def _scratch(need, ws, device, stream):
    """The workspace of one call: the caller's `ws`, or a new one.  A new one is
    allocated on torch's current stream and dropped when the call returns; when
    the call runs on another stream, that stream is recorded on it, so the
    caching allocator does not hand the memory to a later allocation before the
    call's kernels on that stream are done with it."""
    if ws is not None:
        return ws
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    other = _foreign_stream(stream)
    if other is not None:
        ws.record_stream(other)
    return ws


def _workspace(query, ws, device, stream=None):
    """Query the required size, allocate (or take) a byte workspace."""
    size = ctypes.c_size_t(0)
    _check(query(_vp(0), ctypes.byref(size)), "workspace query")
    ws = _scratch(size.value, ws, device, stream)
    return ws, ctypes.c_size_t(ws.numel())


# ---- entry points ----------------------------------------------------------------
def amax_buffer(device="cuda"):
    """Device float32 [AMAX_SLOTS]: the output-amax argument of nvfp4_gemm / nvfp4_mlp_down."""
    return torch.empty(AMAX_SLOTS, dtype=torch.float32, device=device)


def nvfp4_quantize_act(x, out, gs_mode=GS_COMPUTE, ws=None, stream=None):
    """Quantise x [rows, cols] (bf16 or float32, device) into `out` (NVFP4).
    With gs_mode=GS_FROM_AMAX, `ws` is the amax buffer an earlier
    nvfp4_mlp_down(..., amax=) or nvfp4_gemm(..., amax=) filled for x."""
    rows, cols = x.shape
    ld = x.stride(0)
    if x.stride(1) != 1:
        raise ValueError("x must be row-major")
    dt = _dtype_code(x)
    if gs_mode == GS_FROM_AMAX:
        if ws is None or ws.dtype != torch.float32 or ws.numel() < AMAX_SLOTS:
            raise ValueError("GS_FROM_AMAX takes the partial maxima as ws (float32 device tensor of AMAX_SLOTS)")
        sz = ctypes.c_size_t(ws.numel() * 4)
        _check(_lib.nvfp4_quantize_act(_ptr(x), dt, rows, cols, ld, out.c(), gs_mode, _ptr(ws), ctypes.byref(sz),
                                       _stream(stream)), "nvfp4_quantize_act")
        return out

    def q(wsp, szp):
        return _lib.nvfp4_quantize_act(_vp(0), dt, rows, cols, ld, _null_tensor(), gs_mode, wsp, szp, _vp(0))
    ws, sz = _workspace(q, ws, x.device, stream)
    _check(_lib.nvfp4_quantize_act(_ptr(x), dt, rows, cols, ld, out.c(), gs_mode, _ptr(ws), ctypes.byref(sz),
                                   _stream(stream)), "nvfp4_quantize_act")
    return out


def nvfp4_quantize_act_noalloc(x, out, gs_mode=GS_COMPUTE, stream=None):
    """nvfp4_quantize_act with the library's per-GPU scratch array instead of a workspace."""
    rows, cols = x.shape
    if x.stride(1) != 1:
        raise ValueError("x must be row-major")
    _check(_lib.nvfp4_quantize_act_noalloc(_ptr(x), _dtype_code(x), rows, cols, x.stride(0), out.c(), gs_mode,
                                           _stream(stream)), "nvfp4_quantize_act_noalloc")
    return out


def gemm_ws_bytes(m, n, k):
    """Workspace bytes nvfp4_gemm needs for C [m, n] with K = k."""
    size = ctypes.c_size_t(0)
    _check(_lib.nvfp4_gemm(_null_tensor(), _null_tensor(), m, n, k, _vp(0), F32, max(n, 1), _vp(0), _vp(0),
                           ctypes.byref(size), _vp(0)), "workspace query")
    return size.value


def nvfp4_gemm(a, b, c, ws=None, stream=None, amax=None):
    """c [M, N] (float32 or bf16) = A~ . B~^T * gs_a * gs_b; amax (optional, see
    amax_buffer) receives partial maxima of |c| as stored."""
    m, n = c.shape
    need = gemm_ws_bytes(m, n, a.cols)
    ws = _scratch(need, ws, c.device, stream)
    sz = ctypes.c_size_t(ws.numel())
    _check(_lib.nvfp4_gemm(a.c(), b.c(), m, n, a.cols, _ptr(c), _dtype_code(c), c.stride(0), _ptr(amax), _ptr(ws),
                           ctypes.byref(sz), _stream(stream)), "nvfp4_gemm")
    return c


def ws_bytes_quantize(rows, cols, gs_mode=GS_COMPUTE):
    """Workspace bytes nvfp4_quantize_act needs (at least 256 so a buffer can always be allocated)."""
    size = ctypes.c_size_t(0)
    _check(_lib.nvfp4_quantize_act(_vp(0), BF16, rows, cols, cols, _null_tensor(), gs_mode, _vp(0),
                                   ctypes.byref(size), _vp(0)), "workspace query")
    return max(size.value, 256)


def mlp_gu_act_ws_bytes(t, k, i):
    size = ctypes.c_size_t(0)
    _check(_lib.nvfp4_mlp_gu_act(_null_tensor(), _null_tensor(), _null_tensor(), t, k, i, _null_tensor(),
                                 _vp(0), ctypes.byref(size), _vp(0)), "workspace query")
    return size.value


def nvfp4_mlp_gu_act(x, w_gate, w_up, h_out, ws=None, stream=None):
    """h_out (NVFP4 [T, I]) = requant(SiLU(x~ . Wg~^T) * (x~ . Wu~^T)); ws keeps float32 H."""
    t, k, i = x.rows, x.cols, w_gate.rows
    need = mlp_gu_act_ws_bytes(t, k, i)
    ws = _scratch(need, ws, x.codes.device, stream)
    sz = ctypes.c_size_t(ws.numel())
    _check(_lib.nvfp4_mlp_gu_act(x.c(), w_gate.c(), w_up.c(), t, k, i, h_out.c(), _ptr(ws), ctypes.byref(sz),
                                 _stream(stream)), "nvfp4_mlp_gu_act")
    return ws


def mlp_ws_bytes(t, k, i):
    """Workspace bytes nvfp4_mlp needs for T tokens, hidden k, intermediate i."""
    size = ctypes.c_size_t(0)
    z = _null_tensor()
    _check(_lib.nvfp4_mlp(_vp(0), BF16, k, _vp(0), t, k, i, z, z, z, z, z, _vp(0), F32, k, _vp(0), _vp(0),
                          ctypes.byref(size), _vp(0)), "workspace query")
    return size.value


def nvfp4_mlp(x, w_gate, w_up, w_down, x_q, h_q, y, x_amax=None, y_amax=None, ws=None, stream=None):
    """One whole MLP call (see include/nvfp4.h): x [T, K] (bf16 or float32) -> y [T, K]
    (float32 or bf16); x_q and h_q receive x~ and H~; x_amax / y_amax are amax buffers."""
    t, k = x.shape
    i = w_gate.rows
    if x.stride(1) != 1 or y.stride(1) != 1:
        raise ValueError("x and y must be row-major")
    need = mlp_ws_bytes(t, k, i)
    ws = _scratch(need, ws, x.device, stream)
    sz = ctypes.c_size_t(ws.numel())
    _check(_lib.nvfp4_mlp(_ptr(x), _dtype_code(x), x.stride(0), _ptr(x_amax), t, k, i, w_gate.c(), w_up.c(),
                          w_down.c(), x_q.c(), h_q.c(), _ptr(y), _dtype_code(y), y.stride(0), _ptr(y_amax), _ptr(ws),
                          ctypes.byref(sz), _stream(stream)), "nvfp4_mlp")
    return y


def mlp_gu_act_static_ws_bytes(t, k, i):
    """Workspace bytes nvfp4_mlp_gu_act_static needs."""
    size = ctypes.c_size_t(0)
    _check(_lib.nvfp4_mlp_gu_act_static(_null_tensor(), _null_tensor(), _null_tensor(), t, k, i, _null_tensor(),
                                        _vp(0), ctypes.byref(size), _vp(0)), "workspace query")
    return size.value


def nvfp4_mlp_gu_act_static(x, w_gate, w_up, h_out, ws=None, stream=None):
    """h_out (NVFP4 [T, I]) = NVFP4(SiLU(x~ . Wg~^T) * (x~ . Wu~^T)) with the global
    scale already stored in h_out.gscale (read on the device)."""
    t, k, i = x.rows, x.cols, w_gate.rows
    need = mlp_gu_act_static_ws_bytes(t, k, i)
    ws = _scratch(need, ws, x.codes.device, stream)
    sz = ctypes.c_size_t(ws.numel())
    _check(_lib.nvfp4_mlp_gu_act_static(x.c(), w_gate.c(), w_up.c(), t, k, i, h_out.c(), _ptr(ws),
                                        ctypes.byref(sz), _stream(stream)), "nvfp4_mlp_gu_act_static")
    return h_out


def mlp_down_quant_ws_bytes(t, i, k):
    """Workspace bytes nvfp4_mlp_down_quant needs."""
    size = ctypes.c_size_t(0)
    _check(_lib.nvfp4_mlp_down_quant(_null_tensor(), _null_tensor(), t, i, k, _null_tensor(), _vp(0),
                                     ctypes.byref(size), _vp(0)), "workspace query")
    return size.value


def nvfp4_mlp_down_quant(h, w_down, y_out, ws=None, stream=None):
    """y_out (NVFP4 [T, K]) = NVFP4(H~ . Wd~^T * gs_h * gs_wd) with the global scale
    already stored in y_out.gscale (read on the device)."""
    t, i, kk = h.rows, h.cols, w_down.rows
    need = mlp_down_quant_ws_bytes(t, i, kk)
    ws = _scratch(need, ws, h.codes.device, stream)
    sz = ctypes.c_size_t(ws.numel())
    _check(_lib.nvfp4_mlp_down_quant(h.c(), w_down.c(), t, i, kk, y_out.c(), _ptr(ws), ctypes.byref(sz),
                                     _stream(stream)), "nvfp4_mlp_down_quant")
    return y_out


def mlp_down_ws_bytes(t, i, k):
    """Workspace bytes nvfp4_mlp_down needs for T tokens, intermediate i, hidden k."""
    size = ctypes.c_size_t(0)
    _check(_lib.nvfp4_mlp_down(_null_tensor(), _null_tensor(), t, i, k, _vp(0), F32, k, _vp(0), _vp(0),
                               ctypes.byref(size), _vp(0)), "workspace query")
    return size.value


def nvfp4_mlp_down(h, w_down, y, ws=None, stream=None, amax=None):
    """y [T, K] (float32 or bf16) = H~ . Wd~^T * gs_h * gs_wd; amax (optional, see
    amax_buffer) receives partial maxima of |y| as stored -- the next layer's input amax."""
    t, kk = y.shape
    need = mlp_down_ws_bytes(t, h.cols, kk)
    ws = _scratch(need, ws, y.device, stream)
    sz = ctypes.c_size_t(ws.numel())
    _check(_lib.nvfp4_mlp_down(h.c(), w_down.c(), t, h.cols, kk, _ptr(y), _dtype_code(y), y.stride(0), _ptr(amax),
                               _ptr(ws), ctypes.byref(sz), _stream(stream)), "nvfp4_mlp_down")
    return y


def grouped_ws_bytes(m, n, k, e, epilogue):
    size = ctypes.c_size_t(0)
    _check(_lib.nvfp4_grouped_gemm(_null_tensor(), _vp(0), _vp(0), e, m, _null_tensor(), _null_tensor(), n, k,
                                   epilogue, _vp(0), F32, n, _null_tensor(), _vp(0), ctypes.byref(size), _vp(0)),
           "workspace query")
    return size.value


def nvfp4_grouped_gemm(a, a_rows, group_offsets, w0, w1=None, out=None, out_q=None,
                       epilogue=EPI_STORE, m=None, ws=None, stream=None):
    """Expert-grouped GEMM; see include/nvfp4.h.  Returns the workspace used (GLU epilogue)."""
    e = w0.gscale.numel()
    n, k = w0.rows, w0.cols
    if m is None:
        m = out.shape[0] if out is not None else out_q.rows
    need = grouped_ws_bytes(m, n, k, e, epilogue)
    if need:
        ws = _scratch(need, ws, w0.codes.device, stream)
    sz = ctypes.c_size_t(ws.numel() if ws is not None else 0)
    out_dt = _dtype_code(out) if out is not None else F32
    ld = out.stride(0) if out is not None else n
    _check(_lib.nvfp4_grouped_gemm(a.c(), _ptr(a_rows), _ptr(group_offsets), e, m, w0.c(),
                                   w1.c() if w1 is not None else _null_tensor(), n, k, epilogue, _ptr(out), out_dt,
                                   ld, out_q.c() if out_q is not None else _null_tensor(), _ptr(ws),
                                   ctypes.byref(sz), _stream(stream)), "nvfp4_grouped_gemm")
    return ws


def rmsnorm_quantize_ws_bytes(rows, cols):
    size = ctypes.c_size_t(0)
    _check(_lib.nvfp4_rmsnorm_quantize_act(_vp(0), BF16, rows, cols, cols, _vp(0), 1e-6, _null_tensor(), _vp(0),
                                           ctypes.byref(size), _vp(0)), "workspace query")
    return size.value


def nvfp4_rmsnorm_quantize_act(x, gamma, eps, out, ws=None, stream=None):
    """NVFP4 of RMSNorm(x) = x * gamma / sqrt(mean(x^2) + eps), fused; see include/nvfp4.h.
    Returns the workspace (its first rows floats hold 1/rms)."""
    rows, cols = x.shape
    need = rmsnorm_quantize_ws_bytes(rows, cols)
    ws = _scratch(need, ws, x.device, stream)
    sz = ctypes.c_size_t(ws.numel())
    _check(_lib.nvfp4_rmsnorm_quantize_act(_ptr(x), _dtype_code(x), rows, cols, x.stride(0), _ptr(gamma), float(eps),
                                           out.c(), _ptr(ws), ctypes.byref(sz), _stream(stream)),
           "nvfp4_rmsnorm_quantize_act")
    return ws


def moe_route_ws_bytes(t, e, k):
    size = ctypes.c_size_t(0)
    _check(_lib.nvfp4_moe_route(_vp(0), t, e, k, e, _vp(0), _vp(0), _vp(0), _vp(0), _vp(0), ctypes.byref(size),
                                _vp(0)), "workspace query")
    return size.value


def nvfp4_moe_route(logits, k, group_offsets, a_rows, slot_of, weights, ws=None, stream=None):
    """Top-k routing on the device; see include/nvfp4.h.  logits: float32 [T][E] device tensor."""
    t, e = logits.shape
    need = moe_route_ws_bytes(t, e, k)
    ws = _scratch(need, ws, logits.device, stream)
    sz = ctypes.c_size_t(ws.numel())
    _check(_lib.nvfp4_moe_route(_ptr(logits), t, e, k, logits.stride(0), _ptr(group_offsets), _ptr(a_rows),
                                _ptr(slot_of), _ptr(weights), _ptr(ws), ctypes.byref(sz), _stream(stream)),
           "nvfp4_moe_route")
    return ws


def nvfp4_moe_combine(y_slots, slot_of, weights, y, stream=None):
    """y[t] = sum_j weights[t, j] * y_slots[slot_of[t, j]] on the device; see include/nvfp4.h."""
    t, k = slot_of.shape
    n = y.shape[1]
    _check(_lib.nvfp4_moe_combine(_ptr(y_slots), _dtype_code(y_slots), y_slots.stride(0), _ptr(slot_of),
                                  _ptr(weights), t, k, n, _ptr(y), _dtype_code(y), y.stride(0), _stream(stream)),
           "nvfp4_moe_combine")


def moe_mlp_ws_bytes(t, k, i, e, m, static=False):
    size = ctypes.c_size_t(0)
    fn = _lib.nvfp4_moe_mlp_static if static else _lib.nvfp4_moe_mlp
    _check(fn(_vp(0), BF16, k, t, k, i, e, _vp(0), _vp(0), m, _null_tensor(), _null_tensor(),
              _null_tensor(), _null_tensor(), _null_tensor(), _vp(0), F32, k, _vp(0),
              ctypes.byref(size), _vp(0)), "workspace query")
    return size.value


def nvfp4_moe_mlp(x, a_rows, group_offsets, w_gate, w_up, w_down, x_q, h_q, y_slots, ws=None, stream=None):
    """The expert MLP over routed slots in one call; see include/nvfp4.h."""
    t, k = x.shape
    m = y_slots.shape[0]
    e = w_gate.gscale.numel()
    i = w_gate.rows
    need = moe_mlp_ws_bytes(t, k, i, e, m)
    if need:
        ws = _scratch(need, ws, x.device, stream)
    sz = ctypes.c_size_t(ws.numel() if ws is not None else 0)
    _check(_lib.nvfp4_moe_mlp(_ptr(x), _dtype_code(x), x.stride(0), t, k, i, e, _ptr(a_rows), _ptr(group_offsets), m,
                              w_gate.c(), w_up.c(), w_down.c(), x_q.c(), h_q.c(), _ptr(y_slots),
                              _dtype_code(y_slots), y_slots.stride(0), _ptr(ws), ctypes.byref(sz), _stream(stream)),
           "nvfp4_moe_mlp")
    return ws


def nvfp4_moe_mlp_static(x, a_rows, group_offsets, w_gate, w_up, w_down, x_q, h_q, y_slots, ws=None, stream=None):
    """The expert MLP over routed slots in one call with the given global
    scales x_q.gscale and h_q.gscale; see include/nvfp4.h."""
    t, k = x.shape
    m = y_slots.shape[0]
    e = w_gate.gscale.numel()
    i = w_gate.rows
    need = moe_mlp_ws_bytes(t, k, i, e, m, static=True)
    if need:
        ws = _scratch(need, ws, x.device, stream)
    sz = ctypes.c_size_t(ws.numel() if ws is not None else 0)
    _check(_lib.nvfp4_moe_mlp_static(_ptr(x), _dtype_code(x), x.stride(0), t, k, i, e, _ptr(a_rows),
                                     _ptr(group_offsets), m, w_gate.c(), w_up.c(), w_down.c(), x_q.c(), h_q.c(),
                                     _ptr(y_slots), _dtype_code(y_slots), y_slots.stride(0), _ptr(ws),
                                     ctypes.byref(sz), _stream(stream)),
           "nvfp4_moe_mlp_static")
    return ws


def tile_weight_bytes(n, k, experts=1):
    need = ctypes.c_size_t(0)
    _check(_lib.nvfp4_tile_weight(_null_tensor(), experts, n, k, None, ctypes.byref(need), None), "nvfp4_tile_weight")
    return need.value


def nvfp4_tile_weight(w, stream=None):
    """Tile-contiguous copy of weight `w` (or an expert stack) into w.tiled,
    allocated here when absent; the large-batch contractions then stage the
    weight from it (bit-identical results)."""
    experts = w.codes.shape[0] if w.codes.dim() == 3 else 1
    need = tile_weight_bytes(w.rows, w.cols, experts)
    if w.tiled is None or w.tiled.numel() < need:
        w.tiled = torch.empty(max(need, 1), dtype=torch.uint8, device=w.codes.device)
    have = ctypes.c_size_t(w.tiled.numel())
    _check(_lib.nvfp4_tile_weight(w.c(), experts, w.rows, w.cols, _ptr(w.tiled), ctypes.byref(have), _stream(stream)),
           "nvfp4_tile_weight")


# ---- convenience: host <-> device NVFP4 (test and setup plumbing) -------------------
def to_device(q_codes, q_scales, gs, rows, cols, device="cuda"):
    """NVFP4 from host arrays (numpy uint8 codes/scales, float32 gs)."""
    return NVFP4(torch.from_numpy(q_codes).to(device), torch.from_numpy(q_scales).to(device),
                 torch.tensor([float(gs)], dtype=torch.float32, device=device), rows, cols)


def bf16_from_bits(bits_u16, device="cuda"):
    """bf16 device tensor from a numpy uint16 array of bf16 bit patterns."""
    return torch.from_numpy(bits_u16.view("int16")).to(device).view(torch.bfloat16)
