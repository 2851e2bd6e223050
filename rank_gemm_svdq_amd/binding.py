"""ctypes binding of libsvdq (include/svdq.h).

Argument marshalling only: every step of the layer runs in the C++ host code
or the HIP kernels of the library.  Host arrays are numpy arrays; device
buffers are torch CUDA tensors (torch supplies memory and streams).  A
missing library raises ImportError-like RuntimeError on first use; there is
no fallback.
"""

import ctypes as C
import os

import numpy as np

__all__ = [
    "INT4", "MXFP4", "W8A8", "MXFP4_OCP", "SvdqError", "lib", "status_str", "abi_version", "device_check",
    "layer_sizes", "workspace_layout", "workspace_bytes", "calib_absmax", "pack_host",
    "prepare", "attach_lora", "kernel_layout", "unpack_activations", "DeviceLayer",
    "quantize_lora_down", "gemm_lora_up", "linear_forward", "linear_forward_unfused", "linear_forward_noalloc",
    "NOALLOC_MAX_WORKSPACE", "fmt_code", "LIB_PATH",
    "ABI_VERSION", "mfma_rate_probe", "reservoir_select", "smooth_candidates", "search_workspace_bytes", "smooth_search", "SearchOpts", "SearchResult",
]

INT4 = 0
MXFP4 = 1
W8A8 = 2
MXFP4_OCP = 3   # MXFP4 with the OCP shared-exponent rule (floor(log2 amax) - 2, saturated elements)
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libsvdq.so")


def fmt_code(fmt):
    if fmt in (INT4, "int4"):
        return INT4
    if fmt in (MXFP4, "mxfp4"):
        return MXFP4
    if fmt in (W8A8, "w8a8"):
        return W8A8
    if fmt in (MXFP4_OCP, "mxfp4_ocp"):
        return MXFP4_OCP
    raise ValueError(f"unknown format {fmt!r}")


def _canon(rows, K, f):
    """Empty canonical code and scale arrays of `rows` rows in format f."""
    if f == W8A8:
        return np.empty((rows, K), np.uint8), np.empty((rows, 4), np.uint8)
    return np.empty((rows, K // 2), np.uint8), np.empty((rows, (K // 64) * 2 if f == INT4 else K // 32), np.uint8)


def _scales_view(a, f):
    """Canonical scale bytes as fp16 bits (INT4), E8M0 bytes (MXFP4) or fp32 [rows] (W8A8)."""
    if f == INT4:
        return a.view(np.uint16)
    if f == W8A8:
        return a.view(np.float32).reshape(-1)
    return a


class SvdqError(RuntimeError):
    def __init__(self, status, where):
        try:
            text = status_str(status)
        except Exception:           # the library itself may be what failed to load
            text = "error"
        super().__init__(f"{where}: {text} (status {status})")
        self.status = status


class Layer(C.Structure):
    _fields_ = [("K", C.c_int32), ("N", C.c_int32), ("rank", C.c_int32), ("fmt", C.c_int32),
                ("smooth_inv", C.c_void_p), ("wq", C.c_void_p), ("ws", C.c_void_p),
                ("l1k", C.c_void_p), ("l2k", C.c_void_p), ("bias", C.c_void_p)]


class Sizes(C.Structure):
    _fields_ = [(n, C.c_size_t) for n in ("wq_bytes", "ws_bytes", "l1k_bytes", "l2k_bytes",
                                           "wq_canon_bytes", "ws_canon_bytes")]


class WsLayout(C.Structure):
    _fields_ = [(n, C.c_size_t) for n in ("xq_off", "xq_bytes", "xs_off", "xs_bytes", "z_off",
                                           "z_bytes", "total")] + [("zsplit", C.c_int32)]


class PrepareOpts(C.Structure):
    _fields_ = [("lora_rank", C.c_int32), ("lora_a", C.c_void_p), ("lora_b", C.c_void_p),
                ("lora_strength", C.c_float), ("threads", C.c_int32), ("max_iters", C.c_int32),
                ("residual_iters", C.c_int32), ("residual_early_stop", C.c_int32),
                ("has_beta", C.c_int32), ("beta", C.c_double)]


class Prepared(C.Structure):
    _fields_ = [("lambda_", C.c_void_p), ("smooth_inv", C.c_void_p), ("l1", C.c_void_p),
                ("l2", C.c_void_p), ("residual", C.c_void_p), ("sigma", C.c_void_p),
                ("wq", C.c_void_p), ("ws", C.c_void_p), ("iter_errors", C.c_void_p),
                ("best_iter", C.c_void_p)]


class SearchOpts(C.Structure):
    _fields_ = [("grids", C.c_int32), ("residual_iters", C.c_int32), ("residual_early_stop", C.c_int32),
                ("threads", C.c_int32)]


class SearchResult(C.Structure):
    _fields_ = [("count", C.c_int32), ("best", C.c_int32), ("alpha", C.c_double), ("beta", C.c_double),
                ("errors", C.c_void_p), ("best_iter", C.c_int32)]


_lib = None
ABI_VERSION = 8   # SVDQ_ABI_VERSION of include/svdq.h that these structures mirror


def lib():
    """Load libsvdq.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libsvdq.so not built ({LIB_PATH}); run __graft_entry__.build()")
    L = C.CDLL(LIB_PATH)
    i32, sz, vp = C.c_int32, C.c_size_t, C.c_void_p
    L.svdq_status_str.restype = C.c_char_p
    L.svdq_status_str.argtypes = [C.c_int]
    L.svdq_abi_version.restype = i32
    if L.svdq_abi_version() != ABI_VERSION:
        raise RuntimeError(f"libsvdq.so ABI {L.svdq_abi_version()} != {ABI_VERSION}: rebuild the library")
    L.svdq_device_check.argtypes = [i32]
    L.svdq_mfma_rate_probe.argtypes = [i32, i32, i32, i32, vp, vp, vp]
    L.svdq_layer_sizes.argtypes = [i32, i32, i32, i32, C.POINTER(Sizes)]
    L.svdq_workspace_layout.argtypes = [i32, i32, i32, i32, C.POINTER(WsLayout)]
    L.svdq_workspace_bytes.restype = sz
    L.svdq_workspace_bytes.argtypes = [i32, i32, i32, i32]
    L.svdq_calib_absmax.argtypes = [vp, C.c_int64, i32, vp]
    L.svdq_pack_host.argtypes = [vp, i32, i32, i32, vp, vp]
    L.svdq_prepare.argtypes = [vp, vp, i32, i32, C.c_double, i32, i32, C.POINTER(PrepareOpts), C.POINTER(Prepared)]
    L.svdq_attach_lora.argtypes = [vp, vp, vp, i32, i32, i32, vp, vp, i32, C.c_float, vp, vp]
    L.svdq_kernel_layout.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.svdq_unpack_activations.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp]
    L.svdq_quantize_lora_down.argtypes = [C.POINTER(Layer), vp, i32, vp, sz, vp]
    L.svdq_gemm_lora_up.argtypes = [C.POINTER(Layer), vp, sz, i32, vp, vp]
    L.svdq_linear_forward.argtypes = [C.POINTER(Layer), vp, i32, vp, vp, sz, vp]
    L.svdq_linear_forward_unfused.argtypes = [C.POINTER(Layer), vp, i32, vp, vp, sz, vp]
    L.svdq_linear_forward_noalloc.argtypes = [C.POINTER(Layer), vp, i32, vp, vp]
    L.svdq_reservoir_select.restype = C.c_int64
    L.svdq_reservoir_select.argtypes = [C.c_int64, C.c_int64, C.c_uint64, vp]
    L.svdq_smooth_candidates.restype = i32
    L.svdq_smooth_candidates.argtypes = [i32, vp, vp]
    L.svdq_search_workspace_bytes.restype = sz
    L.svdq_search_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    L.svdq_smooth_search.argtypes = [vp, i32, i32, i32, i32, vp, i32, C.POINTER(SearchOpts), vp, sz, vp,
                                     C.POINTER(SearchResult), C.POINTER(Prepared)]
    for name in ("svdq_device_check", "svdq_layer_sizes", "svdq_workspace_layout", "svdq_calib_absmax",
                 "svdq_pack_host", "svdq_prepare", "svdq_attach_lora", "svdq_kernel_layout",
                 "svdq_unpack_activations", "svdq_quantize_lora_down", "svdq_gemm_lora_up",
                 "svdq_linear_forward", "svdq_linear_forward_unfused", "svdq_linear_forward_noalloc",
                 "svdq_smooth_search"):
        getattr(L, name).restype = C.c_int
    _lib = L
    return L


def status_str(s):
    return lib().svdq_status_str(int(s)).decode()


def _check(s, where):
    if s != 0:
        raise SvdqError(s, where)


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def abi_version():
    return lib().svdq_abi_version()


def device_check(device=0):
    return lib().svdq_device_check(device)


def layer_sizes(K, N, rank, fmt):
    s = Sizes()
    _check(lib().svdq_layer_sizes(K, N, rank, fmt_code(fmt), C.byref(s)), "svdq_layer_sizes")
    return {f: getattr(s, f) for f, _ in Sizes._fields_}


def workspace_layout(M, K, rank, fmt):
    w = WsLayout()
    _check(lib().svdq_workspace_layout(M, K, rank, fmt_code(fmt), C.byref(w)), "svdq_workspace_layout")
    return {f: getattr(w, f) for f, _ in WsLayout._fields_}


def workspace_bytes(M, K, rank, fmt):
    return lib().svdq_workspace_bytes(M, K, rank, fmt_code(fmt))


def calib_absmax(x_bits, amax=None):
    """Running per-channel max |x| of bf16 bit patterns [rows, K]."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    rows, K = x_bits.shape
    amax = np.zeros(K, np.float32) if amax is None else np.ascontiguousarray(amax, np.float32).copy()
    _check(lib().svdq_calib_absmax(_p(x_bits), rows, K, _p(amax)), "svdq_calib_absmax")
    return amax


def pack_host(x, fmt):
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, K = x.shape
    f = fmt_code(fmt)
    codes, scales = _canon(rows, K, f)
    _check(lib().svdq_pack_host(_p(x), rows, K, f, _p(codes), _p(scales)), "svdq_pack_host")
    return codes, _scales_view(scales, f)


def prepare(W, act_amax, alpha, rank, fmt, lora=None, threads=0, want_residual=False, max_iters=0,
            residual_iters=1, early_stop=False, beta=None):
    """Offline prepare (svdq_prepare).  Returns canonical host arrays, the
    per-iteration reconstruction errors and the index of the kept one."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    act_amax = np.ascontiguousarray(act_amax, dtype=np.float32)
    K, N = W.shape
    f = fmt_code(fmt)
    k = 0 if lora is None else lora["A"].shape[1]
    rt = rank + k
    T = max(1, int(residual_iters))
    out = {
        "lambda": np.empty(K, np.float32), "smooth_inv": np.empty(K, np.float32),
        "l1": np.empty((K, rt), np.uint16), "l2": np.empty((rt, N), np.uint16),
        "sigma": np.empty(max(rank, 1), np.float64),
        "iter_errors": np.empty(T, np.float64), "best_iter": np.zeros(1, np.int32),
    }
    out["wq"], out["ws"] = _canon(N, K, f)
    if want_residual:
        out["residual"] = np.empty((K, N), np.float32)
    opts = PrepareOpts(0, None, None, 1.0, threads, max_iters, int(residual_iters), int(bool(early_stop)),
                       0 if beta is None else 1, 0.0 if beta is None else float(beta))
    keep = []
    if lora is not None:
        a = np.ascontiguousarray(lora["A"], np.float32)
        b = np.ascontiguousarray(lora["B"], np.float32)
        keep += [a, b]
        opts.lora_rank, opts.lora_a, opts.lora_b = k, _p(a).value, _p(b).value
        opts.lora_strength = float(lora.get("strength", 1.0))
    pr = Prepared(_p(out["lambda"]).value, _p(out["smooth_inv"]).value,
                  _p(out["l1"]).value if rt else None, _p(out["l2"]).value if rt else None,
                  _p(out["residual"]).value if want_residual else None, _p(out["sigma"]).value,
                  _p(out["wq"]).value, _p(out["ws"]).value, _p(out["iter_errors"]).value,
                  _p(out["best_iter"]).value)
    _check(lib().svdq_prepare(_p(W), _p(act_amax), K, N, float(alpha), rank, f, C.byref(opts), C.byref(pr)),
           "svdq_prepare")
    out["ws"] = _scales_view(out["ws"], f)
    out["sigma"] = out["sigma"][:rank]
    out["best_iter"] = int(out["best_iter"][0])
    out.update(K=K, N=N, rank=rt, fmt=f)
    return out


def attach_lora(lam, l1, l2, A, B, strength=1.0):
    lam = np.ascontiguousarray(lam, np.float32)
    l1 = np.ascontiguousarray(l1, np.uint16)
    l2 = np.ascontiguousarray(l2, np.uint16)
    A = np.ascontiguousarray(A, np.float32)
    B = np.ascontiguousarray(B, np.float32)
    K, rank = l1.shape
    N = l2.shape[1]
    k = A.shape[1]
    l1o = np.empty((K, rank + k), np.uint16)
    l2o = np.empty((rank + k, N), np.uint16)
    _check(lib().svdq_attach_lora(_p(lam), _p(l1), _p(l2), K, N, rank, _p(A), _p(B), k, float(strength),
                                  _p(l1o), _p(l2o)), "svdq_attach_lora")
    return l1o, l2o


def kernel_layout(prep):
    """Canonical prepare outputs -> kernel-layout host arrays."""
    K, N, rank, f = prep["K"], prep["N"], prep["rank"], prep["fmt"]
    s = layer_sizes(K, N, rank, f)
    out = {"wq_k": np.empty(s["wq_bytes"], np.uint8), "ws_k": np.empty(s["ws_bytes"], np.uint8),
           "l1k": np.empty(max(s["l1k_bytes"] // 2, 8), np.uint16),
           "l2k": np.empty(max(s["l2k_bytes"] // 2, 8), np.uint16)}
    sinv = np.ascontiguousarray(prep["smooth_inv"], np.float32)
    wq = np.ascontiguousarray(prep["wq"], np.uint8)
    ws = np.ascontiguousarray(prep["ws"]).view(np.uint8)
    l1 = np.ascontiguousarray(prep["l1"], np.uint16) if rank else None
    l2 = np.ascontiguousarray(prep["l2"], np.uint16) if rank else None
    _check(lib().svdq_kernel_layout(K, N, rank, f, _p(sinv), _p(wq), _p(ws), _p(l1), _p(l2),
                                    _p(out["wq_k"]), _p(out["ws_k"]), _p(out["l1k"]), _p(out["l2k"])),
           "svdq_kernel_layout")
    return out


def unpack_activations(ws_host, M, K, rank, fmt):
    """Host copy of a workspace -> canonical (xq [M, K/2] u8, xs, z [M, rank] fp32)."""
    f = fmt_code(fmt)
    ws_host = np.ascontiguousarray(ws_host).view(np.uint8)
    xq, xs = _canon(M, K, f)
    z = np.empty((M, max(rank, 1)), np.float32)
    _check(lib().svdq_unpack_activations(_p(ws_host), M, K, rank, f, _p(xq), _p(xs), _p(z) if rank else None),
           "svdq_unpack_activations")
    return xq, _scales_view(xs, f), z[:, :rank]


# ------------------------------------------------------------ device side

def _torch():
    import torch
    return torch


class DeviceLayer:
    """Kernel-layout buffers of one layer in device memory (torch tensors)."""

    def __init__(self, prep, bias_bits=None, device="cuda"):
        torch = _torch()
        kl = kernel_layout(prep)
        self.K, self.N, self.rank, self.fmt = prep["K"], prep["N"], prep["rank"], prep["fmt"]
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
        self.smooth_inv = t(prep["smooth_inv"].astype(np.float32))
        self.wq = t(kl["wq_k"])
        self.ws = t(kl["ws_k"])
        self.l1k = t(kl["l1k"].view(np.int16))
        self.l2k = t(kl["l2k"].view(np.int16))
        self.bias = None if bias_bits is None else t(np.asarray(bias_bits, np.uint16).view(np.int16))
        self.struct = Layer(self.K, self.N, self.rank, self.fmt, self.smooth_inv.data_ptr(),
                            self.wq.data_ptr(), self.ws.data_ptr(), self.l1k.data_ptr(), self.l2k.data_ptr(),
                            None if self.bias is None else self.bias.data_ptr())

    def workspace(self, M):
        torch = _torch()
        return torch.empty(workspace_bytes(M, self.K, self.rank, self.fmt), dtype=torch.uint8,
                           device=self.wq.device)


_TWO_BYTE = ("torch.int16", "torch.bfloat16")


def _check_tensor(t, what, where, layer, dtypes, shape=None):
    """Reject a tensor the kernels cannot take: wrong dtype or shape, a
    strided view, or memory that is not on the layer's GPU.  The C ABI gets
    bare pointers and cannot see any of these."""
    if str(t.dtype) not in dtypes:
        raise SvdqError(1, f"{where}: {what} has dtype {t.dtype}, expected one of {', '.join(dtypes)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise SvdqError(2, f"{where}: {what} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise SvdqError(1, f"{where}: {what} is not contiguous")


def _check_device(layer, where, **tensors):
    for what, t in tensors.items():
        if not t.is_cuda:
            raise SvdqError(1, f"{where}: {what} is not in GPU memory")
        if t.device != layer.wq.device:
            raise SvdqError(1, f"{where}: {what} is on {t.device}, the layer on {layer.wq.device}")


def _check_x(layer, X, where):
    if X.dim() != 2 or X.shape[1] != layer.K:
        raise SvdqError(2, f"{where}: X has shape {tuple(X.shape)}, expected (M, {layer.K})")
    _check_tensor(X, "X", where, layer, _TWO_BYTE)
    return X.shape[0]


def _check_y(layer, Y, M, where):
    _check_tensor(Y, "Y", where, layer, _TWO_BYTE, (M, layer.N))


def _check_ws(layer, ws, where):
    _check_tensor(ws, "workspace", where, layer, ("torch.uint8",))


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def mfma_rate_probe(kind, zero_operands, blocks, iters, sink, marks=None, stream=None):
    """svdq_mfma_rate_probe (a diagnostic, not part of the layer): sink a
    contiguous float32 CUDA tensor of at least blocks * 512 elements, marks
    None or a contiguous int64 CUDA tensor of at least blocks * 16."""
    torch = _torch()
    where = "svdq_mfma_rate_probe"
    if not (isinstance(sink, torch.Tensor) and sink.is_cuda and sink.dtype == torch.float32 and sink.is_contiguous()
            and sink.numel() >= blocks * 512):
        raise SvdqError(1, f"{where}: sink must be a contiguous float32 CUDA tensor of >= blocks * 512 elements")
    if marks is not None and not (isinstance(marks, torch.Tensor) and marks.is_cuda and marks.dtype == torch.int64
                                  and marks.is_contiguous() and marks.numel() >= blocks * 16
                                  and marks.device == sink.device):
        raise SvdqError(1, f"{where}: marks must be None or a contiguous int64 CUDA tensor of >= blocks * 16 "
                           "elements on the sink's device")
    _check(lib().svdq_mfma_rate_probe(kind, zero_operands, blocks, iters, sink.data_ptr(),
                                      None if marks is None else marks.data_ptr(), _stream(stream)), where)


def quantize_lora_down(layer, X, ws, stream=None):
    M = _check_x(layer, X, "svdq_quantize_lora_down")
    _check_ws(layer, ws, "svdq_quantize_lora_down")
    _check_device(layer, "svdq_quantize_lora_down", X=X, workspace=ws)
    _check(lib().svdq_quantize_lora_down(C.byref(layer.struct), X.data_ptr(), M, ws.data_ptr(), ws.numel(),
                                         _stream(stream)), "svdq_quantize_lora_down")


def gemm_lora_up(layer, ws, M, Y, stream=None):
    _check_ws(layer, ws, "svdq_gemm_lora_up")
    _check_y(layer, Y, M, "svdq_gemm_lora_up")
    _check_device(layer, "svdq_gemm_lora_up", workspace=ws, Y=Y)
    _check(lib().svdq_gemm_lora_up(C.byref(layer.struct), ws.data_ptr(), ws.numel(), M, Y.data_ptr(),
                                   _stream(stream)), "svdq_gemm_lora_up")


def linear_forward(layer, X, Y, ws, stream=None):
    M = _check_x(layer, X, "svdq_linear_forward")
    _check_y(layer, Y, M, "svdq_linear_forward")
    _check_ws(layer, ws, "svdq_linear_forward")
    _check_device(layer, "svdq_linear_forward", X=X, Y=Y, workspace=ws)
    _check(lib().svdq_linear_forward(C.byref(layer.struct), X.data_ptr(), M, Y.data_ptr(), ws.data_ptr(),
                                     ws.numel(), _stream(stream)), "svdq_linear_forward")


NOALLOC_MAX_WORKSPACE = 32 << 20   # SVDQ_NOALLOC_MAX_WORKSPACE


def linear_forward_noalloc(layer, X, Y, stream=None):
    """svdq_linear_forward with the library's own per-GPU scratch array as
    the workspace (no allocation; calls overlapping on one GPU race)."""
    M = _check_x(layer, X, "svdq_linear_forward_noalloc")
    _check_y(layer, Y, M, "svdq_linear_forward_noalloc")
    _check_device(layer, "svdq_linear_forward_noalloc", X=X, Y=Y)
    _check(lib().svdq_linear_forward_noalloc(C.byref(layer.struct), X.data_ptr(), M, Y.data_ptr(), _stream(stream)),
           "svdq_linear_forward_noalloc")


def linear_forward_unfused(layer, X, Y, ws, stream=None):
    """The same layer as four separate kernels (svdq_linear_forward_unfused)."""
    M = _check_x(layer, X, "svdq_linear_forward_unfused")
    _check_y(layer, Y, M, "svdq_linear_forward_unfused")
    _check_ws(layer, ws, "svdq_linear_forward_unfused")
    _check_device(layer, "svdq_linear_forward_unfused", X=X, Y=Y, workspace=ws)
    _check(lib().svdq_linear_forward_unfused(C.byref(layer.struct), X.data_ptr(), M, Y.data_ptr(), ws.data_ptr(),
                                             ws.numel(), _stream(stream)), "svdq_linear_forward_unfused")


def smooth_candidates(grids=20):
    """(alpha, beta) pairs of the smooth search, in scoring order."""
    n = lib().svdq_smooth_candidates(int(grids), None, None)
    if n == 0:
        raise SvdqError(1, "svdq_smooth_candidates")
    a, b = np.empty(n, np.float64), np.empty(n, np.float64)
    lib().svdq_smooth_candidates(int(grids), _p(a), _p(b))
    return list(zip(a.tolist(), b.tolist()))


def search_workspace_bytes(M, K, N, rank, fmt):
    return lib().svdq_search_workspace_bytes(M, K, N, rank, fmt_code(fmt))


def smooth_search(W, X_cal, rank, fmt, grids=20, residual_iters=1, early_stop=False, threads=0, stream=None):
    """Smooth-factor grid search (svdq_smooth_search).  W: host [K, N] fp32;
    X_cal: device [M, K] bf16 bits (int16 tensor).  Returns the winner's
    index and exponents, every candidate's score and the winner's canonical
    prepared arrays (as prepare() returns them)."""
    torch = _torch()
    W = np.ascontiguousarray(W, dtype=np.float32)
    K, N = W.shape
    if X_cal.dim() != 2 or X_cal.shape[1] != K:
        raise SvdqError(2, f"svdq_smooth_search: X_cal has shape {tuple(X_cal.shape)}, expected (M, {K})")
    if str(X_cal.dtype) not in _TWO_BYTE or not X_cal.is_contiguous() or not X_cal.is_cuda:
        raise SvdqError(1, "svdq_smooth_search: X_cal must be a contiguous int16/bfloat16 GPU tensor")
    M = X_cal.shape[0]
    f = fmt_code(fmt)
    n = lib().svdq_smooth_candidates(int(grids), None, None)
    if n == 0:
        raise SvdqError(1, "svdq_smooth_search")
    wsb = search_workspace_bytes(M, K, N, rank, f)
    if wsb == 0:
        raise SvdqError(2, "svdq_smooth_search")
    ws = torch.empty(wsb, dtype=torch.uint8, device=X_cal.device)
    errors = np.empty(n, np.float64)
    out = {
        "lambda": np.empty(K, np.float32), "smooth_inv": np.empty(K, np.float32),
        "l1": np.empty((K, rank), np.uint16), "l2": np.empty((rank, N), np.uint16),
    }
    out["wq"], out["ws"] = _canon(N, K, f)
    pr = Prepared(_p(out["lambda"]).value, _p(out["smooth_inv"]).value,
                  _p(out["l1"]).value if rank else None, _p(out["l2"]).value if rank else None,
                  None, None, _p(out["wq"]).value, _p(out["ws"]).value, None, None)
    res = SearchResult(0, -1, 0.0, 0.0, _p(errors).value, -1)
    opts = SearchOpts(int(grids), int(residual_iters), int(bool(early_stop)), int(threads))
    _check(lib().svdq_smooth_search(_p(W), K, N, rank, f, X_cal.data_ptr(), M, C.byref(opts), ws.data_ptr(),
                                    ws.numel(), _stream(stream), C.byref(res), C.byref(pr)), "svdq_smooth_search")
    out["ws"] = _scales_view(out["ws"], f)
    out.update(K=K, N=N, rank=rank, fmt=f)
    return {"best": res.best, "alpha": res.alpha, "beta": res.beta, "errors": errors, "prepared": out,
            "best_iter": res.best_iter}


def reservoir_select(n_calls, k, seed):
    """Indices of the calibration calls a reservoir of size k keeps
    (svdq_reservoir_select), in increasing order."""
    out = np.empty(max(1, min(int(n_calls), int(k))), np.int64)
    n = lib().svdq_reservoir_select(int(n_calls), int(k), int(seed) & ((1 << 64) - 1), _p(out))
    if n < 0:
        raise SvdqError(1, "svdq_reservoir_select")
    return out[:n].tolist()
