"""Python binding of libfp8q.so -- W8A8 block-scaled FP8 projection on MI355X.

Argument marshalling only: every function takes torch tensors that already
live on the current GPU, passes their device pointers and the current torch
stream to the C ABI (include/fp8q.h) and raises on a non-OK status.  Every
step of the computation runs in the library's HIP kernels; there is no CPU
or PyTorch fallback: the first call raises if the library has not been built
(``python -m w8a8_fp8_block_amd.build``).

Names match the C entry points:

  fp8q_quant_act(x, q, scale_rm, variant=0)
  fp8q_quant_act_kmajor(x, q, scale_rm, scale_km, variant=0)
  fp8q_scale_to_kmajor(scale_rm, scale_km)
  fp8q_gemm_blockscaled(a, a_scale_km, w, w_scale, out, kernel=0)
  fp8q_proj(x, w, w_scale, out, act_q, act_scale, act_scale_km)
  fp8q_silu_mul_quant(gate, up, h, h_scale_km)
  fp8q_ffn_gate_up(x_q, x_scale_km, w_gate, w_gate_scale, w_up, w_up_scale, h, h_scale_km)
  fp8q_ffn(x, w_gate, w_gate_scale, w_up, w_up_scale, w_down, w_down_scale, out,
           workspace, variant=0)
  fp8q_m_pad(m), fp8q_quant_select(M, K, cu_count), ...

Dtypes: bf16 tensors may be torch.bfloat16 or torch.uint16/int16 views;
e4m3 codes may be torch.uint8 or torch.float8_e4m3fn; scales float32.
"""
from __future__ import annotations

import ctypes
import os

# torch first: its libtorch_hip.so asks for "libamdhip64.so" while this
# library asks for "libamdhip64.so.7"; loading torch's runtime first lets the
# dynamic linker satisfy ours with the same object (matching soname), so one
# HIP runtime serves both.  The other order would load a second runtime.
import torch  # noqa: F401  (device memory and streams)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8q.so")

_P = ctypes.c_void_p
_U = ctypes.c_uint32
_I = ctypes.c_int
_SZ = ctypes.c_size_t


class SelectParams(ctypes.Structure):
    _fields_ = [("cu_count", ctypes.c_uint32), ("min_wg_per_cu", ctypes.c_uint32),
                ("b_groups_per_wg", ctypes.c_uint32), ("a_groups_per_wg", ctypes.c_uint32),
                ("requested", ctypes.c_int), ("b_present", ctypes.c_int),
                ("a_present", ctypes.c_int)]


_SIGS = {
    "fp8q_m_pad": (_U, [_U]),
    "fp8q_last_error": (ctypes.c_char_p, []),
    "fp8q_version": (ctypes.c_char_p, []),
    "fp8q_quant_act": (_I, [_P, _P, _P, _U, _U, _P]),
    "fp8q_quant_act_ex": (_I, [_P, _P, _P, _U, _U, _I, _P]),
    "fp8q_quant_act_kmajor": (_I, [_P, _P, _P, _P, _U, _U, _P]),
    "fp8q_quant_act_kmajor_ex": (_I, [_P, _P, _P, _P, _U, _U, _I, _P]),
    "fp8q_default_select_params": (SelectParams, [_U]),
    "fp8q_quant_select_with": (_I, [_U, _U, ctypes.POINTER(SelectParams),
                                    ctypes.POINTER(_U * 3), ctypes.POINTER(ctypes.c_char_p)]),
    "fp8q_quant_select": (_I, [_U, _U, _U, ctypes.POINTER(_U * 3),
                               ctypes.POINTER(ctypes.c_char_p)]),
    "fp8q_quant_b_min_m": (_U, [_U, ctypes.POINTER(SelectParams)]),
    "fp8q_quant_log_slot": (_I, [_I, ctypes.c_char_p, _I]),
    "fp8q_scale_to_kmajor": (_I, [_P, _P, _U, _U, _P]),
    "fp8q_gemm_select": (_I, [_U, _U, _U]),
    "fp8q_gemm_select_cus": (_I, [_U, _U, _U, _U]),
    "fp8q_proj_quant_fused": (_I, [_U, _U]),
    "fp8q_gemm_blockscaled": (_I, [_P, _P, _P, _P, _P, _U, _U, _U, _P]),
    "fp8q_gemm_blockscaled_ex": (_I, [_P, _P, _P, _P, _P, _U, _U, _U, _I, _P]),
    "fp8q_gemm_blockscaled_splitk": (_I, [_P, _P, _P, _P, _P, _P, _SZ, _U, _U, _U, _U, _P]),
    "fp8q_gemm_splitk_select": (_U, [_U, _U, _U]),
    "fp8q_gemm_splitk_select_cus": (_U, [_U, _U, _U, _U]),
    "fp8q_gemm_streamk_select": (_I, [_U, _U, _U]),
    "fp8q_gemm_streamk_select_cus": (_I, [_U, _U, _U, _U]),
    "fp8q_gemm_splitk_workspace_bytes": (_SZ, [_U, _U, _U, _U]),
    "fp8q_gemm_blockscaled_streamk": (_I, [_P, _P, _P, _P, _P, _P, _SZ, _U, _U, _U, _U, _P]),
    "fp8q_gemm_kernel_name": (ctypes.c_char_p, [_U, _U, _U, _I]),
    "fp8q_gemm_streamk_workspace_bytes": (_SZ, [_U]),
    "fp8q_gemm_blockscaled_splitk_noalloc": (_I, [_P, _P, _P, _P, _P, _U, _U, _U, _U, _P]),
    "fp8q_clock_stamp": (_I, [_P, _U, _P]),
    "fp8q_proj": (_I, [_P, _P, _P, _P, _P, _P, _P, _U, _U, _U, _P]),
    "fp8q_proj_splitk": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _SZ, _U, _U, _U, _P]),
    "fp8q_gemm_rowscaled": (_I, [_P, _P, _P, _P, _P, _U, _U, _U, _P]),
    "fp8q_gemm_rowscaled_ex": (_I, [_P, _P, _P, _P, _P, _U, _U, _U, _I, _P]),
    "fp8q_proj_rowscaled": (_I, [_P, _P, _P, _P, _P, _P, _P, _U, _U, _U, _P]),
    "fp8q_dequant_fp8_bf16": (_I, [_P, _P, _P, _U, _U, _I, _P]),
    "fp8q_gemm_bf16": (_I, [_P, _P, _P, _U, _U, _U, _P]),
    "fp8q_silu_mul_quant": (_I, [_P, _P, _P, _P, _U, _U, _P]),
    "fp8q_ffn_gate_up": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _U, _U, _U, _P]),
    "fp8q_ffn_select": (_I, [_U, _U, _U]),
    "fp8q_ffn_workspace_bytes": (ctypes.c_size_t, [_U, _U, _U, _I]),
    "fp8q_ffn": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _U, _U, _U, _I, _P]),
}

_lib = None


def lib():
    """The ctypes handle of libfp8q.so (raw C ABI), loaded on first use.
    Raises if the library has not been built: there is no fallback path."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m w8a8_fp8_block_amd.build` "
                "(the projection has no fallback path)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


STATUS = {0: "FP8Q_OK", 1: "FP8Q_ERR_NULL", 2: "FP8Q_ERR_SHAPE", 3: "FP8Q_ERR_ALIGN",
          4: "FP8Q_ERR_DEVICE", 5: "FP8Q_ERR_LAUNCH", 6: "FP8Q_ERR_VARIANT"}


class Fp8qError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


def _check(st: int):
    if st != 0:
        raise Fp8qError(st, lib().fp8q_last_error().decode())


def _ptr(t) -> int:
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _optr(t) -> int:
    return 0 if t is None else _ptr(t)


_raw_stream = None


def _stream(stream=None) -> int:
    """The HIP stream handle to launch on: `stream`'s, else torch's current
    stream on the current device (read through torch's raw-handle query
    where the build has it: ~0.4 us against ~2.7 us for building a Stream
    object, per call, on the host)."""
    global _raw_stream
    import torch
    if stream is not None:
        return stream.cuda_stream
    if _raw_stream is None:
        q = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        _raw_stream = ((lambda: q(torch.cuda.current_device())) if q is not None
                       else (lambda: torch.cuda.current_stream().cuda_stream))
    return _raw_stream()


def _dims(t, nd):
    shape = t.shape
    if len(shape) != nd:
        raise ValueError(f"expected a {nd}-d tensor, got shape {tuple(shape)}")
    return shape


# ------------------------------------------------------------------ API
def fp8q_m_pad(m: int) -> int:
    return int(lib().fp8q_m_pad(m))


def fp8q_version() -> str:
    return lib().fp8q_version().decode()


def fp8q_quant_act(x, q, scale_rm, variant: int = 0, stream=None):
    M, K = _dims(x, 2)
    _check(lib().fp8q_quant_act_ex(_ptr(x), _ptr(q), _ptr(scale_rm), M, K, variant,
                                  _stream(stream)))


def fp8q_quant_act_kmajor(x, q, scale_rm, scale_km, variant: int = 0, stream=None):
    M, K = _dims(x, 2)
    _check(lib().fp8q_quant_act_kmajor_ex(_ptr(x), _ptr(q), _optr(scale_rm), _ptr(scale_km), M,
                                         K, variant, _stream(stream)))


def fp8q_scale_to_kmajor(scale_rm, scale_km, stream=None):
    M, G = _dims(scale_rm, 2)
    _check(lib().fp8q_scale_to_kmajor(_ptr(scale_rm), _ptr(scale_km), M, G * 128,
                                     _stream(stream)))


def fp8q_gemm_blockscaled(a, a_scale_km, w, w_scale, out, kernel: int = 0, stream=None):
    M, K = _dims(a, 2)
    N, K2 = _dims(w, 2)
    if K2 != K:
        raise ValueError("a and w disagree on K")
    _check(lib().fp8q_gemm_blockscaled_ex(_ptr(a), _ptr(a_scale_km), _ptr(w), _ptr(w_scale),
                                         _ptr(out), M, N, K, kernel, _stream(stream)))


def fp8q_gemm_splitk_select(M: int, N: int, K: int, cu_count: int = None) -> int:
    """Split count fp8q_gemm_blockscaled_splitk takes with splits=0 (1 = no split)
    on the current device, or on a device with cu_count compute units."""
    if cu_count is not None:
        return int(lib().fp8q_gemm_splitk_select_cus(M, N, K, cu_count))
    return int(lib().fp8q_gemm_splitk_select(M, N, K))


def fp8q_gemm_streamk_select(M: int, N: int, K: int, cu_count: int = None) -> int:
    """1 if fp8q_gemm_blockscaled_splitk with splits=0 runs the stream-K form
    (on the current device, or one with cu_count compute units)."""
    if cu_count is not None:
        return int(lib().fp8q_gemm_streamk_select_cus(M, N, K, cu_count))
    return int(lib().fp8q_gemm_streamk_select(M, N, K))


def fp8q_gemm_splitk_workspace_bytes(M: int, N: int, K: int, splits: int = 0) -> int:
    return int(lib().fp8q_gemm_splitk_workspace_bytes(M, N, K, splits))


def fp8q_gemm_blockscaled_splitk(a, a_scale_km, w, w_scale, out, workspace, splits: int = 0,
                                 stream=None):
    """fp8q_gemm_blockscaled with the K blocks split over `splits` workgroups
    per tile (0 = automatic); workspace: a device tensor of at least
    fp8q_gemm_splitk_workspace_bytes(M, N, K, splits) bytes, or None when that is 0."""
    M, K = _dims(a, 2)
    N, K2 = _dims(w, 2)
    if K2 != K:
        raise ValueError("a and w disagree on K")
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().fp8q_gemm_blockscaled_splitk(_ptr(a), _ptr(a_scale_km), _ptr(w), _ptr(w_scale),
                                             _ptr(out), _optr(workspace), nbytes, M, N, K,
                                             splits, _stream(stream)))


def fp8q_gemm_streamk_workspace_bytes(workgroups: int = 0) -> int:
    return int(lib().fp8q_gemm_streamk_workspace_bytes(workgroups))


def fp8q_gemm_blockscaled_streamk(a, a_scale_km, w, w_scale, out, workspace, workgroups: int = 0,
                                  stream=None):
    """fp8q_gemm_blockscaled in its stream-K form on `workgroups` persistent
    workgroups (0 = the device's CU count); workspace: a device tensor of at
    least fp8q_gemm_streamk_workspace_bytes(workgroups) bytes."""
    M, K = _dims(a, 2)
    N, K2 = _dims(w, 2)
    if K2 != K:
        raise ValueError("a and w disagree on K")
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().fp8q_gemm_blockscaled_streamk(_ptr(a), _ptr(a_scale_km), _ptr(w), _ptr(w_scale),
                                              _ptr(out), _optr(workspace), nbytes, M, N, K,
                                              workgroups, _stream(stream)))


NOALLOC_SCRATCH_BYTES = 32 << 20  # FP8Q_NOALLOC_SCRATCH_BYTES


def fp8q_gemm_blockscaled_splitk_noalloc(a, a_scale_km, w, w_scale, out, splits: int = 0,
                                         stream=None):
    """fp8q_gemm_blockscaled_splitk with the partials in the library's static
    device scratch (no workspace; splits * M * N * 4 <= NOALLOC_SCRATCH_BYTES)."""
    M, K = _dims(a, 2)
    N, K2 = _dims(w, 2)
    if K2 != K:
        raise ValueError("a and w disagree on K")
    _check(lib().fp8q_gemm_blockscaled_splitk_noalloc(_ptr(a), _ptr(a_scale_km), _ptr(w),
                                                     _ptr(w_scale), _ptr(out), M, N, K, splits,
                                                     _stream(stream)))


def fp8q_proj(x, w, w_scale, out, act_q, act_scale, act_scale_km, stream=None):
    M, K = _dims(x, 2)
    N, K2 = _dims(w, 2)
    if K2 != K:
        raise ValueError("x and w disagree on K")
    _check(lib().fp8q_proj(_ptr(x), _ptr(w), _ptr(w_scale), _ptr(out), _ptr(act_q),
                          _ptr(act_scale), _ptr(act_scale_km), M, N, K, _stream(stream)))


def fp8q_proj_splitk(x, w, w_scale, out, act_q, act_scale, act_scale_km, workspace, stream=None):
    """fp8q_proj with the GEMM split over K where fp8q_gemm_splitk_select says
    so; workspace: a device tensor of at least
    fp8q_gemm_splitk_workspace_bytes(M, N, K) bytes, or None when that is 0."""
    M, K = _dims(x, 2)
    N, K2 = _dims(w, 2)
    if K2 != K:
        raise ValueError("x and w disagree on K")
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().fp8q_proj_splitk(_ptr(x), _ptr(w), _ptr(w_scale), _ptr(out), _ptr(act_q),
                                 _ptr(act_scale), _ptr(act_scale_km), _optr(workspace), nbytes,
                                 M, N, K, _stream(stream)))


def fp8q_gemm_rowscaled(a, a_scale_km, w, w_scale_row, out, kernel: int = 0, stream=None):
    """As fp8q_gemm_blockscaled with one fp32 weight scale per row, w_scale_row [N]."""
    M, K = _dims(a, 2)
    N, K2 = _dims(w, 2)
    if K2 != K:
        raise ValueError("a and w disagree on K")
    _check(lib().fp8q_gemm_rowscaled_ex(_ptr(a), _ptr(a_scale_km), _ptr(w), _ptr(w_scale_row),
                                       _ptr(out), M, N, K, kernel, _stream(stream)))


def fp8q_proj_rowscaled(x, w, w_scale_row, out, act_q, act_scale, act_scale_km, stream=None):
    M, K = _dims(x, 2)
    N, K2 = _dims(w, 2)
    if K2 != K:
        raise ValueError("x and w disagree on K")
    _check(lib().fp8q_proj_rowscaled(_ptr(x), _ptr(w), _ptr(w_scale_row), _ptr(out), _ptr(act_q),
                                    _ptr(act_scale), _ptr(act_scale_km), M, N, K, _stream(stream)))


def fp8q_dequant_fp8_bf16(w, scale, dst, per_row: bool, stream=None):
    """FP8 weights [N,K] -> bf16 [N,K] (dst), block-scaled or per-row scales."""
    N, K = _dims(w, 2)
    _check(lib().fp8q_dequant_fp8_bf16(_ptr(w), _ptr(scale), _ptr(dst), N, K, 1 if per_row else 0,
                                      _stream(stream)))


def fp8q_gemm_bf16(x, w, out, stream=None):
    """bf16 comparator GEMM: out[M,N] = bf16(x[M,K] . w[N,K]^T)."""
    M, K = _dims(x, 2)
    N, K2 = _dims(w, 2)
    if K2 != K:
        raise ValueError("x and w disagree on K")
    _check(lib().fp8q_gemm_bf16(_ptr(x), _ptr(w), _ptr(out), M, N, K, _stream(stream)))


def fp8q_silu_mul_quant(gate, up, h, h_scale_km, stream=None):
    """FFN intermediate h = bf16(silu(gate) * up) of bf16 gate/up [M,I],
    quantized: codes h [M,I], K-major scales h_scale_km [I/128, ceil16(M)]."""
    M, I = _dims(gate, 2)
    if _dims(up, 2) != (M, I):
        raise ValueError("gate and up differ in shape")
    _check(lib().fp8q_silu_mul_quant(_ptr(gate), _ptr(up), _ptr(h), _ptr(h_scale_km), M, I,
                                    _stream(stream)))


def fp8q_ffn_gate_up(x_q, x_scale_km, w_gate, w_gate_scale, w_up, w_up_scale, h, h_scale_km,
                     stream=None):
    """Fused gate/up projection of quantized x [M,H] with weights [I,H] to the
    quantized intermediate h [M,I] and its K-major scales."""
    M, H = _dims(x_q, 2)
    I, H2 = _dims(w_gate, 2)
    if H2 != H or _dims(w_up, 2) != (I, H):
        raise ValueError("x, w_gate and w_up disagree in shape")
    _check(lib().fp8q_ffn_gate_up(_ptr(x_q), _ptr(x_scale_km), _ptr(w_gate), _ptr(w_gate_scale),
                                 _ptr(w_up), _ptr(w_up_scale), _ptr(h), _ptr(h_scale_km), M, H, I,
                                 _stream(stream)))


def fp8q_ffn_select(M: int, H: int, I: int) -> int:
    """Variant fp8q_ffn runs with variant=0: 1 fused gate/up, 2 separate."""
    return int(lib().fp8q_ffn_select(M, H, I))


def fp8q_ffn_workspace_bytes(M: int, H: int, I: int, variant: int = 0) -> int:
    return int(lib().fp8q_ffn_workspace_bytes(M, H, I, variant))


def fp8q_ffn(x, w_gate, w_gate_scale, w_up, w_up_scale, w_down, w_down_scale, out, workspace,
             variant: int = 0, stream=None):
    """The dense FFN: out [M,H] = down(quant(bf16(silu(gate) * up))) of x [M,H];
    workspace: a device byte tensor of fp8q_ffn_workspace_bytes(M, H, I, variant)."""
    M, H = _dims(x, 2)
    I, H2 = _dims(w_gate, 2)
    if H2 != H or _dims(w_up, 2) != (I, H) or _dims(w_down, 2) != (H, I):
        raise ValueError("x and the weights disagree in shape")
    _check(lib().fp8q_ffn(_ptr(x), _ptr(w_gate), _ptr(w_gate_scale), _ptr(w_up), _ptr(w_up_scale),
                         _ptr(w_down), _ptr(w_down_scale), _ptr(out), _ptr(workspace),
                         workspace.numel() * workspace.element_size(), M, H, I, variant,
                         _stream(stream)))


def fp8q_default_select_params(cu_count: int) -> SelectParams:
    return lib().fp8q_default_select_params(cu_count)


def fp8q_quant_select_with(M: int, K: int, params: SelectParams):
    """-> (variant, grid tuple, reject reason or None); variant -1 on bad args."""
    grid = (_U * 3)()
    why = ctypes.c_char_p()
    v = lib().fp8q_quant_select_with(M, K, ctypes.byref(params), ctypes.byref(grid),
                                    ctypes.byref(why))
    return v, tuple(grid), (why.value.decode() if why.value else None)


def fp8q_quant_select(M: int, K: int, cu_count: int):
    grid = (_U * 3)()
    why = ctypes.c_char_p()
    v = lib().fp8q_quant_select(M, K, cu_count, ctypes.byref(grid), ctypes.byref(why))
    return v, tuple(grid), (why.value.decode() if why.value else None)


def fp8q_gemm_select(M: int, N: int, K: int, cu_count: int = None) -> int:
    """Kernel id the auto GEMM runs for this shape (see fp8q_gemm_blockscaled_ex)
    on the current device, or on a device with cu_count compute units."""
    if cu_count is not None:
        return int(lib().fp8q_gemm_select_cus(M, N, K, cu_count))
    return int(lib().fp8q_gemm_select(M, N, K))


def fp8q_proj_quant_fused(M: int, K: int) -> bool:
    """True if fp8q_proj writes the K-major scales from the quantizer itself."""
    return bool(lib().fp8q_proj_quant_fused(M, K))


def fp8q_gemm_kernel_name(M: int, N: int, K: int, kernel: int = 0) -> str:
    """Name (as a kernel trace shows it) of the kernel fp8q_gemm_blockscaled
    runs for this shape and kernel id (0 = automatic) on the current device."""
    return lib().fp8q_gemm_kernel_name(M, N, K, kernel).decode()


FFN_GATE_UP_KERNEL_NAME = "gemm_pp_kernel<3, false, true>"
SPLITK_KERNEL_NAMES = ("gemm_tiled_kernel<128, 128, 2, 2, 2, false, true>", "splitk_reduce_kernel")
STREAMK_KERNEL_NAME = "gemm_pp_sk_kernel<3>"


def fp8q_quant_b_min_m(K: int, params: SelectParams) -> int:
    return int(lib().fp8q_quant_b_min_m(K, ctypes.byref(params)))


def fp8q_quant_log_slot(variant: int, reject, requested: bool) -> int:
    r = None if reject is None else reject.encode()
    return int(lib().fp8q_quant_log_slot(variant, r, int(bool(requested))))


def fp8q_clock_stamp(stamps, stream=None):
    """Clock stamp into stamps (int64 device tensor [n, 4]): per one-wave
    workgroup {XCD id, HW_ID, shader clock counter, 100 MHz counter}."""
    n, four = _dims(stamps, 2)
    if four != 4:
        raise ValueError("stamps must be [n, 4]")
    _check(lib().fp8q_clock_stamp(_ptr(stamps), n, _stream(stream)))


def shader_clock_ghz(before, after):
    """Average shader clock per XCD between two clock stamps (host arrays
    [n, 4] from fp8q_clock_stamp), pairing the stamps of the same CU:
    ({xcd: median GHz over its CU pairs}, number of pairs)."""
    first = {}
    for r in before:
        first.setdefault((int(r[0]), (int(r[1]) >> 8) & 0xFF), r)
    per = {}
    for r in after:
        b = first.get((int(r[0]), (int(r[1]) >> 8) & 0xFF))
        if b is None or int(r[3]) <= int(b[3]):
            continue
        per.setdefault(int(r[0]), []).append((int(r[2]) - int(b[2])) / (int(r[3]) - int(b[3])) * 0.1)
    import statistics
    return {x: statistics.median(v) for x, v in per.items()}, sum(len(v) for v in per.values())


# ------------------------------------------------------- allocation helpers
def alloc_proj_scratch(M: int, K: int, device="cuda"):
    """(act_q [M,K] u8, act_scale [M,K/128] f32, act_scale_km [K/128, ceil16(M)] f32)."""
    import torch
    G = K // 128
    return (torch.empty((M, K), dtype=torch.uint8, device=device),
            torch.empty((M, G), dtype=torch.float32, device=device),
            torch.empty((G, fp8q_m_pad(M)), dtype=torch.float32, device=device))


def alloc_ffn_workspace(M: int, H: int, I: int, variant: int = 0, device="cuda"):
    """Device byte tensor sized for fp8q_ffn(M, H, I, variant)."""
    import torch
    n = fp8q_ffn_workspace_bytes(M, H, I, variant)
    if n == 0:
        raise ValueError("invalid FFN shape or variant")
    return torch.empty((n,), dtype=torch.uint8, device=device)
