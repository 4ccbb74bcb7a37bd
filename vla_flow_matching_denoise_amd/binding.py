"""ctypes binding of ``libvla_expert.so`` (argument marshalling only).

The functions keep the C names.  Every step of the denoise loop runs in the
HIP library; PyTorch is used here only to place tensors in device memory and
to hand over a stream.  There is no CPU path: if the library is missing the
import of this module raises.
"""
from __future__ import annotations

import atexit
import ctypes
import os
from typing import Callable, Dict, Optional

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libvla_expert.so")

VLA_BF16 = 0
VLA_FP8_E4M3 = 1
VLA_FP8_E4M3_MXFP4_GU = 2
VLA_OK = 0
VLA_ERR_ARG = -1
VLA_ERR_SHAPE = -2
VLA_ERR_OOM = -3
VLA_ERR_HIP = -4
VLA_OPT_USE_GRAPH = 1
VLA_OPT_PERSISTENT = 2
VLA_OPT_PERSISTENT_ACTIVE = 3
VLA_OPT_PERSISTENT_STATUS = 4
VLA_OPT_GEMM_TILE = 5
VLA_OPT_L2_PREFETCH = 6
VLA_OPT_SPLIT_BATCH = 8
VLA_OPT_WEIGHT_NT = 9

# every symbol include/vla_expert.h declares
EXPORTED = (
    "vla_expert_create", "vla_denoise", "vla_denoise_varlen", "vla_denoise_static", "vla_set_stream", "vla_set_option", "vla_get_option",
    "vla_expert_destroy",
    "vla_last_error", "vla_device_bytes", "vla_test_modulation", "vla_test_layer",
    "vla_test_attention", "vla_profile_kernel",
    "vla_prefill_create", "vla_prefill", "vla_prefill_set_stream", "vla_prefill_set_option", "vla_prefill_destroy",
    "vla_prefill_device_bytes",
)
VLA_KERNEL_QKV, VLA_KERNEL_ATTN, VLA_KERNEL_O, VLA_KERNEL_GATE_UP, VLA_KERNEL_DOWN = range(5)


class VlaDims(ctypes.Structure):
    _fields_ = [
        ("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("intermediate", ctypes.c_int32),
        ("action_dim", ctypes.c_int32), ("horizon", ctypes.c_int32), ("prefix_len", ctypes.c_int32),
        ("batch", ctypes.c_int32), ("time_emb_dim", ctypes.c_int32), ("rope_theta", ctypes.c_float),
        ("rms_eps", ctypes.c_float), ("time_scale", ctypes.c_float), ("weight_dtype", ctypes.c_int32),
    ]


_P = ctypes.c_void_p
_PP = ctypes.POINTER(ctypes.c_void_p)


class VlaWeights(ctypes.Structure):
    _fields_ = [
        ("in_w", _P), ("in_b", _P), ("out_w", _P), ("out_b", _P),
        ("t1_w", _P), ("t1_b", _P), ("t2_w", _P), ("t2_b", _P),
        ("mod_w", _PP), ("mod_b", _PP), ("modf_w", _P), ("modf_b", _P),
        ("wq", _PP), ("wk", _PP), ("wv", _PP), ("wo", _PP), ("wg", _PP), ("wu", _PP), ("wd", _PP),
        ("sq", _PP), ("sk", _PP), ("sv", _PP), ("so", _PP), ("sg", _PP), ("su", _PP), ("sd", _PP),
    ]


class VlaBackboneDims(ctypes.Structure):
    _fields_ = [
        ("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("intermediate", ctypes.c_int32),
        ("prefix_len", ctypes.c_int32), ("batch", ctypes.c_int32), ("rope_theta", ctypes.c_float),
        ("rms_eps", ctypes.c_float), ("weight_dtype", ctypes.c_int32),
    ]


class VlaBackboneWeights(ctypes.Structure):
    _fields_ = [
        ("norm1", _PP), ("norm2", _PP), ("wq", _PP), ("wk", _PP), ("wv", _PP), ("wo", _PP), ("wg", _PP),
        ("wu", _PP), ("wd", _PP),
        ("sq", _PP), ("sk", _PP), ("sv", _PP), ("so", _PP), ("sg", _PP), ("su", _PP), ("sd", _PP),
    ]


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run vla_flow_matching_denoise_amd.build.build()")
    # torch ships its own HIP runtime under the same soname. Loading torch first
    # makes the library bind to that one runtime, so the device pointers and
    # streams torch hands over belong to the runtime the library calls; loading
    # the library first would put a second HIP runtime into the process.
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    lib.vla_expert_create.restype = ctypes.c_void_p
    lib.vla_expert_create.argtypes = [ctypes.POINTER(VlaWeights), ctypes.POINTER(VlaDims)]
    lib.vla_denoise.restype = ctypes.c_int
    lib.vla_denoise.argtypes = [_P, _P, _P, _P, _P, ctypes.c_int, _P]
    lib.vla_denoise_static.restype = ctypes.c_int
    lib.vla_denoise_static.argtypes = [_P, _P, _P, _P, _P, ctypes.c_int, _P]
    lib.vla_denoise_varlen.restype = ctypes.c_int
    lib.vla_denoise_varlen.argtypes = [_P, _P, _P, _P, _P, _P, ctypes.c_int, _P]
    lib.vla_set_stream.restype = ctypes.c_int
    lib.vla_set_stream.argtypes = [_P, _P]
    lib.vla_set_option.restype = ctypes.c_int
    lib.vla_set_option.argtypes = [_P, ctypes.c_int, ctypes.c_int]
    lib.vla_get_option.argtypes = [_P, ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
    lib.vla_get_option.restype = ctypes.c_int
    lib.vla_expert_destroy.restype = None
    lib.vla_expert_destroy.argtypes = [_P]
    lib.vla_last_error.restype = ctypes.c_char_p
    lib.vla_last_error.argtypes = []
    lib.vla_device_bytes.restype = ctypes.c_int64
    lib.vla_device_bytes.argtypes = [_P]
    lib.vla_test_modulation.restype = ctypes.c_int
    lib.vla_test_modulation.argtypes = [_P, _P, ctypes.c_int, _P]
    lib.vla_test_layer.restype = ctypes.c_int
    lib.vla_test_layer.argtypes = [_P, _P, _P, _P, ctypes.c_int, ctypes.c_int, ctypes.c_int, _P, _P]
    lib.vla_test_attention.restype = ctypes.c_int
    lib.vla_test_attention.argtypes = [_P, _P, _P, ctypes.c_int, _P, _P, _P, _P]
    lib.vla_profile_kernel.restype = ctypes.c_int
    lib.vla_profile_kernel.argtypes = [_P, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
    lib.vla_prefill_create.restype = ctypes.c_void_p
    lib.vla_prefill_create.argtypes = [ctypes.POINTER(VlaBackboneWeights), ctypes.POINTER(VlaBackboneDims)]
    lib.vla_prefill.restype = ctypes.c_int
    lib.vla_prefill.argtypes = [_P, _P, _P, _P]
    lib.vla_prefill_set_stream.restype = ctypes.c_int
    lib.vla_prefill_set_stream.argtypes = [_P, _P]
    lib.vla_prefill_set_option.restype = ctypes.c_int
    lib.vla_prefill_set_option.argtypes = [_P, ctypes.c_int, ctypes.c_int]
    lib.vla_prefill_destroy.restype = None
    lib.vla_prefill_destroy.argtypes = [_P]
    lib.vla_prefill_device_bytes.restype = ctypes.c_int64
    lib.vla_prefill_device_bytes.argtypes = [_P]
    return lib


_LIB: Optional[ctypes.CDLL] = None

# Contexts created through this module and not yet destroyed, handle -> the
# destroy function.  They are destroyed at interpreter exit by an atexit hook
# registered right after the library (and with it torch's HIP runtime) is
# loaded: Python runs its atexit hooks in reverse order of registration and
# before the C-level exit handlers, so the contexts' graphs, streams, events
# and allocations are released while the HIP runtime (and a profiler that
# intercepts it) is still fully up, instead of being left for the runtime's
# own exit-time teardown or for a finalizer that runs after it.
_LIVE: Dict[int, Callable[[int], None]] = {}


def close_all() -> int:
    """Destroy every context still open (in creation order reversed).
    Returns how many were destroyed."""
    n = 0
    for h in reversed(list(_LIVE)):
        destroy = _LIVE.pop(h, None)
        if destroy is not None:
            destroy(h)
            n += 1
    return n


def lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        _LIB = load_library()
        atexit.register(close_all)
    return _LIB


class VlaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"vla error {code}: {msg}")
        self.code = code


def _check(rc: int) -> int:
    if rc != VLA_OK:
        raise VlaError(rc, vla_last_error())
    return rc


# ---- thin wrappers with the C names ---------------------------------------

def vla_last_error() -> str:
    return (lib().vla_last_error() or b"").decode()


def vla_expert_create(weights: VlaWeights, dims: VlaDims) -> int:
    h = lib().vla_expert_create(ctypes.byref(weights), ctypes.byref(dims))
    if not h:
        raise VlaError(-1, vla_last_error())
    _LIVE[h] = lib().vla_expert_destroy
    return h


def vla_denoise(ctx: int, prefix_k: int, prefix_v: int, noise: int, t_schedule: int, n_steps: int,
                out_actions: int, check: bool = True) -> int:
    rc = lib().vla_denoise(ctx, prefix_k, prefix_v, noise, t_schedule, int(n_steps), out_actions)
    return _check(rc) if check else rc


VLA_STATIC_SCRATCH_BYTES = 64 << 20


def vla_denoise_static(ctx: int, prefix_k: int, prefix_v: int, noise: int, t_schedule: int, n_steps: int,
                       out_actions: int, check: bool = True) -> int:
    rc = lib().vla_denoise_static(ctx, prefix_k, prefix_v, noise, t_schedule, int(n_steps), out_actions)
    return _check(rc) if check else rc


def vla_denoise_varlen(ctx: int, prefix_k: int, prefix_v: int, prefix_valid: Optional[int], noise: int,
                       t_schedule: int, n_steps: int, out_actions: int, check: bool = True) -> int:
    rc = lib().vla_denoise_varlen(ctx, prefix_k, prefix_v, prefix_valid, noise, t_schedule, int(n_steps),
                                  out_actions)
    return _check(rc) if check else rc


def vla_set_stream(ctx: int, stream: Optional[int]) -> int:
    return _check(lib().vla_set_stream(ctx, stream))


def vla_set_option(ctx: int, option: int, value: int) -> int:
    return _check(lib().vla_set_option(ctx, option, value))


def vla_get_option(ctx: int, option: int) -> int:
    v = ctypes.c_int(0)
    _check(lib().vla_get_option(ctx, option, ctypes.byref(v)))
    return int(v.value)


def vla_expert_destroy(ctx: Optional[int]) -> None:
    if ctx:
        _LIVE.pop(ctx, None)
    lib().vla_expert_destroy(ctx)


def vla_device_bytes(ctx: int) -> int:
    return int(lib().vla_device_bytes(ctx))


def vla_test_modulation(ctx: int, t_schedule: int, n_steps: int, mod_out: int) -> int:
    return _check(lib().vla_test_modulation(ctx, t_schedule, int(n_steps), mod_out))


def vla_test_layer(ctx: int, prefix_k: int, prefix_v: int, t_schedule: int, n_steps: int, step: int,
                   layer: int, h_in: int, h_out: int) -> int:
    return _check(lib().vla_test_layer(ctx, prefix_k, prefix_v, t_schedule, int(n_steps), int(step),
                                       int(layer), h_in, h_out))


def vla_test_attention(ctx: int, prefix_k: int, prefix_v: int, layer: int, q: int, k_new: int, v_new: int,
                       o_out: int) -> int:
    return _check(lib().vla_test_attention(ctx, prefix_k, prefix_v, int(layer), q, k_new, v_new, o_out))


def vla_profile_kernel(ctx: int, kernel: int, iters: int):
    """Returns (mean launch microseconds, algorithmic bytes, algorithmic flops) of one launch."""
    us, by, fl = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    _check(lib().vla_profile_kernel(ctx, int(kernel), int(iters), ctypes.byref(us), ctypes.byref(by),
                                    ctypes.byref(fl)))
    return us.value, by.value, fl.value


def vla_prefill_create(weights: VlaBackboneWeights, dims: VlaBackboneDims) -> int:
    h = lib().vla_prefill_create(ctypes.byref(weights), ctypes.byref(dims))
    if not h:
        raise VlaError(-1, vla_last_error())
    _LIVE[h] = lib().vla_prefill_destroy
    return h


def vla_prefill(ctx: int, embeddings: int, prefix_k: int, prefix_v: int, check: bool = True) -> int:
    rc = lib().vla_prefill(ctx, embeddings, prefix_k, prefix_v)
    return _check(rc) if check else rc


def vla_prefill_set_stream(ctx: int, stream: Optional[int]) -> int:
    return _check(lib().vla_prefill_set_stream(ctx, stream))


def vla_prefill_set_option(ctx: int, option: int, value: int) -> int:
    return _check(lib().vla_prefill_set_option(ctx, option, value))


def vla_prefill_destroy(ctx: Optional[int]) -> None:
    if ctx:
        _LIVE.pop(ctx, None)
    lib().vla_prefill_destroy(ctx)


def vla_prefill_device_bytes(ctx: int) -> int:
    return int(lib().vla_prefill_device_bytes(ctx))
