"""Python binding of libvla.so (include/vla.h): argument marshalling only.

Every function here has the name of the C entry point it calls and takes torch
tensors (device memory and streams come from PyTorch); the computation runs in
the library's HIP kernels.  There is no fallback: if libvla.so is missing or
fails to load, `lib()` raises.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import List, Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# VLA_LIBRARY selects another build of the same library (the sanitized host build of the tests)
LIB_PATH = os.environ.get("VLA_LIBRARY") or os.path.join(HERE, "libvla.so")

VLA_OK = 0
STATUS = {0: "VLA_OK", 1: "VLA_ERR_INVALID_ARGUMENT", 2: "VLA_ERR_SHAPE_MISMATCH", 3: "VLA_ERR_INVALID_HANDLE",
          4: "VLA_ERR_UNSUPPORTED", 5: "VLA_ERR_OUT_OF_MEMORY", 6: "VLA_ERR_DEVICE"}
PRECISION = {"f32": 0, "bf16": 1, "w2a8": 2}
VLA_OUT_F32, VLA_OUT_BF16 = 0, 1
VLA_GEMM_STORE, VLA_GEMM_GEGLU, VLA_GEMM_RESIDUAL = 0, 1, 2
ABI_VERSION = 2
ATTN_MODE = {"cross": 0, "joint": 1}

# every symbol include/vla.h declares
EXPORTS = (
    "vla_status_string", "vla_last_error", "vla_n_tensors", "vla_tensor_info", "vla_model_create",
    "vla_model_destroy", "vla_kv_cache_bytes", "vla_prefix_encode", "vla_denoise_chunk",
    "vla_kv_cache_release", "vla_kv_cache_info", "vla_quantize_rows_i8", "vla_w2a8_gemm",
    "vla_ternary_pack", "vla_ternary_unpack", "vla_probe_arm", "vla_probe_arm_ex", "vla_probe_read", "vla_gemm_bf16", "vla_w2a8_gemm_ex",
    "vla_w2a8_gemm_noalloc", "vla_prefix_encode_masked", "vla_prefix_encode_ex",
)
W2A8_MFMA, W2A8_DOT4 = 0, 1
PROBE_PREFIX_GATEUP, PROBE_PREFIX_DOWN, PROBE_PREFIX_QKV, PROBE_PREFIX_ATTN, PROBE_PREFIX_O, PROBE_CACHE = range(1, 7)
PROBE_EXPERT_SELF_ATTN, PROBE_EXPERT_CROSS_ATTN, PROBE_EXPERT_SCORES, PROBE_EXPERT_GATEUP = 7, 8, 9, 10


class VlaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class vla_model_config(C.Structure):
    _fields_ = [("abi_version", C.c_int32), ("precision", C.c_int32),
                ("d_p", C.c_int32), ("L_p", C.c_int32), ("Hq", C.c_int32), ("Hkv", C.c_int32),
                ("hd", C.c_int32), ("F_p", C.c_int32),
                ("d_e", C.c_int32), ("L_e", C.c_int32), ("Hq_e", C.c_int32), ("Hkv_e", C.c_int32),
                ("hd_e", C.c_int32), ("F_e", C.c_int32),
                ("H", C.c_int32), ("d_a", C.c_int32), ("rms_eps", C.c_float), ("attn_mode", C.c_int32)]


class vla_weights(C.Structure):
    _fields_ = [("tensors", C.POINTER(C.c_void_p)), ("n_tensors", C.c_int32),
                ("ternary_beta", C.POINTER(C.c_float))]


class vla_solver(C.Structure):
    _fields_ = [("tau_start", C.c_float), ("tau_end", C.c_float), ("schedule", C.POINTER(C.c_float))]


class vla_timing(C.Structure):
    _fields_ = [("prefix_ms", C.c_float), ("denoise_ms", C.c_float), ("step_ms", C.c_float),
                ("graph_replayed", C.c_int32)]


_LIB = None


def lib():
    """Load libvla.so (once).  Raises if it is missing: there is no other path."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with prefix_cache_flow_amd/build.py")
    L = C.CDLL(LIB_PATH)
    P, I, S = C.c_void_p, C.c_int32, C.c_size_t
    sig = {
        "vla_status_string": (C.c_char_p, [I]),
        "vla_last_error": (C.c_char_p, []),
        "vla_n_tensors": (I, [C.POINTER(vla_model_config)]),
        "vla_tensor_info": (I, [C.POINTER(vla_model_config), I, C.POINTER(C.c_int64), C.POINTER(C.c_int64),
                                C.POINTER(I)]),
        "vla_model_create": (I, [C.POINTER(vla_model_config), C.POINTER(vla_weights), P, C.POINTER(P)]),
        "vla_model_destroy": (I, [P]),
        "vla_kv_cache_bytes": (S, [P, I, I]),
        "vla_prefix_encode": (I, [P, P, I, I, P, S, P, C.POINTER(P), C.POINTER(vla_timing)]),
        "vla_prefix_encode_masked": (I, [P, P, I, I, C.POINTER(C.c_int32), P, S, P, C.POINTER(P),
                                         C.POINTER(vla_timing)]),
        "vla_prefix_encode_ex": (I, [P, P, I, I, I, C.POINTER(C.c_int32), P, S, P, C.POINTER(P),
                                     C.POINTER(vla_timing)]),
        "vla_denoise_chunk": (I, [P, P, P, I, C.POINTER(vla_solver), P, I, P, C.POINTER(vla_timing)]),
        "vla_kv_cache_release": (I, [P]),
        "vla_kv_cache_info": (I, [P, C.POINTER(I), C.POINTER(I)]),
        "vla_quantize_rows_i8": (I, [P, I, I, P, P, P]),
        "vla_w2a8_gemm": (I, [P, P, P, C.c_float, I, I, I, P, P, P]),
        "vla_w2a8_gemm_noalloc": (I, [P, P, P, C.c_float, I, I, I, P, P, P]),
        "vla_w2a8_gemm_ex": (I, [P, P, P, C.POINTER(C.c_float), I, I, I, I, I, P, P, P, C.POINTER(C.c_float)]),
        "vla_ternary_pack": (I, [P, I, I, P]),
        "vla_ternary_unpack": (I, [P, I, I, P]),
        "vla_probe_arm": (I, [P, I, I]),
        "vla_probe_arm_ex": (I, [P, I, I, I]),
        "vla_gemm_bf16": (I, [P, P, I, I, I, I, P, P]),
        "vla_probe_read": (I, [P, C.POINTER(C.c_float), C.POINTER(I)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _LIB = L
    return L


def _check(status: int):
    if status != VLA_OK:
        raise VlaError(status, lib().vla_last_error().decode())


def _stream(stream=None) -> C.c_void_p:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _ptr(t) -> C.c_void_p:
    return C.c_void_p(t.data_ptr())


def make_config(cfg) -> vla_model_config:
    """A vla_model_config from a mapping or object with the model fields."""
    get = (lambda k: cfg[k]) if isinstance(cfg, dict) else (lambda k: getattr(cfg, k))
    prec = get("precision")
    prec = PRECISION[prec] if isinstance(prec, str) else int(prec)
    c = vla_model_config()
    c.abi_version = ABI_VERSION
    c.precision = prec
    for k in ("d_p", "L_p", "Hq", "Hkv", "hd", "F_p", "d_e", "L_e", "Hq_e", "Hkv_e", "hd_e", "F_e", "H", "d_a"):
        setattr(c, k, int(get(k)))
    c.rms_eps = float(get("rms_eps"))
    try:
        attn = get("attn")
    except (KeyError, AttributeError):
        attn = "cross"
    c.attn_mode = ATTN_MODE[attn] if isinstance(attn, str) else int(attn)
    return c


# ---------------------------------------------------------------- C entry points

def vla_status_string(status: int) -> str:
    return lib().vla_status_string(status).decode()


def vla_last_error() -> str:
    return lib().vla_last_error().decode()


def vla_n_tensors(cfg) -> int:
    return lib().vla_n_tensors(C.byref(make_config(cfg)))


def vla_tensor_info(cfg, index: int):
    r, c, k = C.c_int64(), C.c_int64(), C.c_int32()
    _check(lib().vla_tensor_info(C.byref(make_config(cfg)), index, C.byref(r), C.byref(c), C.byref(k)))
    return r.value, c.value, k.value


def vla_ternary_pack(q: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.int8)
    n, k = q.shape
    out = np.empty((n, k // 4), dtype=np.uint8)
    _check(lib().vla_ternary_pack(q.ctypes.data_as(C.c_void_p), n, k, out.ctypes.data_as(C.c_void_p)))
    return out


def vla_ternary_unpack(packed: np.ndarray, k: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    n = packed.shape[0]
    out = np.empty((n, k), dtype=np.int8)
    _check(lib().vla_ternary_unpack(packed.ctypes.data_as(C.c_void_p), n, k, out.ctypes.data_as(C.c_void_p)))
    return out


class Model:
    """Owner of a vla_model handle (destroyed with the object)."""

    def __init__(self, handle: C.c_void_p, cfg: vla_model_config):
        self.handle = handle
        self.cfg = cfg

    def close(self):
        if self.handle:
            _check(lib().vla_model_destroy(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class KVCache:
    """A vla_kv_cache handle plus the torch tensor that owns its storage."""

    def __init__(self, handle: C.c_void_p, storage, batch: int, n_prefix: int):
        self.handle = handle
        self.storage = storage
        self.batch = batch
        self.n_prefix = n_prefix

    def close(self):
        if self.handle:
            _check(lib().vla_kv_cache_release(self.handle))
            self.handle = None


def upload_weights(cfg, arrays: Sequence[np.ndarray], device="cuda"):
    """Tensors in boundary order from host arrays in the same order, on `device` ("cpu" keeps them in host
    memory: vla_model_create reads host tensors directly).

    Gains and fp32 linears become float32 tensors, bf16 linears bfloat16
    tensors, ternary codes ({-1, 0, 1} int8) packed uint8 tensors (packed by
    vla_ternary_pack).
    """
    import torch
    ccfg = make_config(cfg)
    n = lib().vla_n_tensors(C.byref(ccfg))
    if n < 0:
        raise VlaError(1, vla_last_error())
    if len(arrays) != n:
        raise ValueError(f"expected {n} tensors, got {len(arrays)}")
    out = []
    for i, a in enumerate(arrays):
        rows, cols, kind = vla_tensor_info(cfg, i)
        a = np.asarray(a)
        if kind == 2:
            t = torch.from_numpy(vla_ternary_pack(a))
        elif kind == 0:
            t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32).reshape(rows))
        else:
            t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32).reshape(rows, cols))
            if ccfg.precision != PRECISION["f32"]:
                t = t.to(torch.bfloat16)
        out.append(t.to(device))
    return out


def vla_model_create(cfg, tensors: List, betas: Optional[Sequence[float]] = None, stream=None) -> Model:
    ccfg = make_config(cfg)
    ptrs = (C.c_void_p * len(tensors))(*[t.data_ptr() for t in tensors])
    w = vla_weights()
    w.tensors = C.cast(ptrs, C.POINTER(C.c_void_p))
    w.n_tensors = len(tensors)
    beta_arr = None
    if betas is not None:
        beta_arr = (C.c_float * len(betas))(*betas)
        w.ternary_beta = C.cast(beta_arr, C.POINTER(C.c_float))
    h = C.c_void_p()
    _check(lib().vla_model_create(C.byref(ccfg), C.byref(w), _stream(stream), C.byref(h)))
    return Model(h, ccfg)


def vla_kv_cache_bytes(model: Model, batch: int, n_prefix: int) -> int:
    return lib().vla_kv_cache_bytes(model.handle, batch, n_prefix)


IN_F32, IN_BF16 = 0, 1


def vla_prefix_encode(model: Model, prefix_hidden, kv_storage=None, stream=None, timing: bool = False, lengths=None):
    """prefix_hidden: float32 (or bfloat16: vla_prefix_encode_ex) cuda tensor [B, N, d_p]; returns a
    KVCache (and a timing dict when asked).  lengths (optional, B ints in 1..N) calls
    vla_prefix_encode_masked: observation b fills its first lengths[b] rows."""
    import torch
    assert prefix_hidden.dtype in (torch.float32, torch.bfloat16) and prefix_hidden.is_contiguous()
    B, N, _ = prefix_hidden.shape
    nbytes = vla_kv_cache_bytes(model, B, N)
    if kv_storage is None:
        kv_storage = torch.empty(nbytes, dtype=torch.uint8, device=prefix_hidden.device)
    h = C.c_void_p()
    tm = vla_timing() if timing else None
    nb = kv_storage.numel() * kv_storage.element_size()
    tmp = C.byref(tm) if tm is not None else None
    if prefix_hidden.dtype == torch.bfloat16:
        lens = (C.c_int32 * B)(*[int(x) for x in lengths]) if lengths is not None else None
        _check(lib().vla_prefix_encode_ex(model.handle, _ptr(prefix_hidden), IN_BF16, B, N, lens, _ptr(kv_storage),
                                          nb, _stream(stream), C.byref(h), tmp))
    elif lengths is None:
        _check(lib().vla_prefix_encode(model.handle, _ptr(prefix_hidden), B, N, _ptr(kv_storage), nb,
                                       _stream(stream), C.byref(h), tmp))
    else:
        lens = (C.c_int32 * B)(*[int(x) for x in lengths])
        _check(lib().vla_prefix_encode_masked(model.handle, _ptr(prefix_hidden), B, N, lens, _ptr(kv_storage), nb,
                                              _stream(stream), C.byref(h), tmp))
    kv = KVCache(h, kv_storage, B, N)
    if timing:
        return kv, {"prefix_ms": tm.prefix_ms}
    return kv


def vla_gemm_bf16(a, w, geglu: bool = False, stream=None, residual=None):
    """a: cuda bfloat16 [M, K], w: cuda bfloat16 [N, K] -> float32 [M, N] (or [M, N / 2] with the GeGLU of
    gate/up rows interleaved in blocks of 16), on the prefix's product kernels.  With `residual` (cuda float32
    [M, N], updated in place and returned): residual += a w^T, the prefix's O-projection form."""
    import torch
    assert a.dtype == torch.bfloat16 and w.dtype == torch.bfloat16 and a.is_contiguous() and w.is_contiguous()
    M, K = a.shape
    N = w.shape[0]
    if residual is not None:
        assert not geglu and residual.dtype == torch.float32 and residual.is_contiguous()
        assert tuple(residual.shape) == (M, N)
        out, epilogue = residual, VLA_GEMM_RESIDUAL
    else:
        out = torch.empty((M, N // 2 if geglu else N), dtype=torch.float32, device=a.device)
        epilogue = VLA_GEMM_GEGLU if geglu else VLA_GEMM_STORE
    _check(lib().vla_gemm_bf16(C.c_void_p(a.data_ptr()), C.c_void_p(w.data_ptr()), M, N, K, epilogue,
                               C.c_void_p(out.data_ptr()), _stream(stream)))
    return out


def vla_probe_arm(model: Model, kind: int, max_launches: int = 4096, repeat: int = 1):
    _check(lib().vla_probe_arm_ex(model.handle, int(kind), int(max_launches), int(repeat)))


def vla_probe_read(model: Model):
    ms, n = C.c_float(), C.c_int32()
    _check(lib().vla_probe_read(model.handle, C.byref(ms), C.byref(n)))
    return ms.value, n.value


class Probe:
    """Arms a kernel probe on construction; collect() reads and disarms it."""

    def __init__(self, model: Model, kind: int, max_launches: int = 4096, repeat: int = 1):
        self.model = model
        vla_probe_arm(model, kind, max_launches, repeat)

    def collect(self):
        r = vla_probe_read(self.model)
        vla_probe_arm(self.model, 0, 0)
        return r


def vla_denoise_chunk(model: Model, kv: KVCache, noise, steps: int, schedule=None, tau=None, out_dtype=None,
                      out=None, stream=None, timing: bool = False):
    """noise: float32 cuda tensor [B, H, d_a]; returns X^T (and a timing dict when asked)."""
    import torch
    assert noise.dtype == torch.float32 and noise.is_contiguous()
    out_dtype = out_dtype or torch.float32
    if out is None:
        out = torch.empty(noise.shape, dtype=out_dtype, device=noise.device)
    code = VLA_OUT_BF16 if out.dtype == torch.bfloat16 else VLA_OUT_F32
    solver = None
    keep = None
    if schedule is not None or tau is not None:
        solver = vla_solver()
        if tau is not None:
            solver.tau_start, solver.tau_end = float(tau[0]), float(tau[1])
        else:
            solver.tau_start, solver.tau_end = 0.0, 1.0
        if schedule is not None:
            keep = (C.c_float * len(schedule))(*[float(x) for x in schedule])
            solver.schedule = C.cast(keep, C.POINTER(C.c_float))
    tm = vla_timing() if timing else None
    _check(lib().vla_denoise_chunk(model.handle, kv.handle, _ptr(noise), int(steps),
                                   C.byref(solver) if solver is not None else None, _ptr(out), code,
                                   _stream(stream), C.byref(tm) if tm is not None else None))
    if timing:
        return out, {"denoise_ms": tm.denoise_ms, "step_ms": tm.step_ms, "graph_replayed": tm.graph_replayed}
    return out


def vla_kv_cache_release(kv: KVCache):
    kv.close()


def vla_kv_cache_info(kv: KVCache):
    b, n = C.c_int32(), C.c_int32()
    _check(lib().vla_kv_cache_info(kv.handle, C.byref(b), C.byref(n)))
    return b.value, n.value


def vla_model_destroy(model: Model):
    model.close()


def vla_quantize_rows_i8(x, stream=None):
    """x: float32 cuda [M, K] -> (int8 codes [M, K], float32 alpha [M])."""
    import torch
    x = x.contiguous()
    M, K = x.shape
    a = torch.empty((M, K), dtype=torch.int8, device=x.device)
    alpha = torch.empty((M,), dtype=torch.float32, device=x.device)
    _check(lib().vla_quantize_rows_i8(_ptr(x), M, K, _ptr(a), _ptr(alpha), _stream(stream)))
    return a, alpha


def vla_w2a8_gemm_ex(a, alpha, q_packed, beta, group: int, path: int = W2A8_MFMA, want_acc: bool = True,
                     want_y: bool = True, stream=None, timing: bool = False):
    """As vla_w2a8_gemm with group-wise scales beta [N / group] (host floats) and a kernel choice;
    returns (acc, y) or, with timing, (acc, y, kernel_ms)."""
    import torch
    M, K = a.shape
    N = q_packed.shape[0]
    b = (C.c_float * len(beta))(*[float(x) for x in beta])
    acc = torch.empty((M, N), dtype=torch.int32, device=a.device) if want_acc else None
    y = torch.empty((M, N), dtype=torch.bfloat16, device=a.device) if want_y else None
    ms = C.c_float()
    _check(lib().vla_w2a8_gemm_ex(_ptr(a), _ptr(alpha), _ptr(q_packed), b, int(group), int(path), M, N, K,
                                  _ptr(acc) if acc is not None else None, _ptr(y) if y is not None else None,
                                  _stream(stream), C.byref(ms) if timing else None))
    return (acc, y, ms.value) if timing else (acc, y)


def vla_w2a8_gemm(a, alpha, q_packed, beta: float, want_acc: bool = True, want_y: bool = True, stream=None):
    """a int8 [M, K], alpha f32 [M], q_packed uint8 [N, K/4] (cuda) -> (acc int32 [M, N], y bf16 [M, N])."""
    import torch
    M, K = a.shape
    N = q_packed.shape[0]
    acc = torch.empty((M, N), dtype=torch.int32, device=a.device) if want_acc else None
    y = torch.empty((M, N), dtype=torch.bfloat16, device=a.device) if want_y else None
    _check(lib().vla_w2a8_gemm(_ptr(a), _ptr(alpha), _ptr(q_packed), float(beta), M, N, K,
                               _ptr(acc) if acc is not None else None, _ptr(y) if y is not None else None,
                               _stream(stream)))
    return acc, y


def vla_w2a8_gemm_noalloc(a, alpha, q_packed, beta: float, acc_out=None, y_out=None, stream=None):
    """As vla_w2a8_gemm, writing into caller-provided outputs (acc int32 [M, N] and/or y bf16 [M, N],
    either may be None); the library allocates nothing for the call."""
    M, K = a.shape
    N = q_packed.shape[0]
    _check(lib().vla_w2a8_gemm_noalloc(_ptr(a), _ptr(alpha), _ptr(q_packed), float(beta), M, N, K,
                                       _ptr(acc_out) if acc_out is not None else None,
                                       _ptr(y_out) if y_out is not None else None, _stream(stream)))
    return acc_out, y_out
