"""ctypes binding of libvaep.so (argument marshalling only).

The library is built in-tree by ``spatially_sharded_conv_amd.build``.  Loading
fails loudly when it is missing: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# VAEP_LIB selects another build of the same library (the host-sanitized one of
# build_sanitized.py); there is no other implementation to fall back to.
LIB_PATH = os.environ.get("VAEP_LIB") or os.path.join(HERE, "libvaep.so")

VAEP_OK = 0
VAEP_WARN_FELL_BACK = 1
VAEP_ERR_INVALID_ARG = -1
VAEP_ERR_UNSUPPORTED = -2
VAEP_ERR_WORKSPACE = -3
VAEP_ERR_HIP = -4
VAEP_ERR_NOT_READY = -5

FAMILY_KL2D = 1
FAMILY_WAN3D = 2
DTYPE_F32 = 1
DTYPE_BF16 = 2
MAX_STAGES = 6
MAX_BANDS = 64
AXIS_AUTO, AXIS_HEIGHT, AXIS_WIDTH, AXIS_DENSE, AXIS_TILE = 0, 1, 2, 3, 4

# every symbol the public headers declare
EXPORTS = [
    "vaep_last_error", "vaep_version", "vaep_config_preset", "vaep_param_count",
    "vaep_param_info", "vaep_model_create", "vaep_model_destroy", "vaep_model_set_norm_fold",
    "vaep_model_set_halo_poison",
    "vaep_workspace_bytes",
    "vaep_decode_full", "vaep_decode_bands", "vaep_select_axis", "vaep_decode_sharded",
    "vaep_sharded_workspace_bytes", "vaep_noalloc_scratch_bytes", "vaep_decode_bands_noalloc",
    "vaep_tiled_workspace_bytes", "vaep_decode_tiled",
    "vaep_encoder_param_count", "vaep_encoder_param_info", "vaep_encoder_create", "vaep_encoder_destroy",
    "vaep_encode_tiled_workspace_bytes", "vaep_encode_tiled",
    "vaep_groupnorm_merge",
    "vaep_step_conv", "vaep_step_groupnorm", "vaep_step_rmsnorm", "vaep_step_attention",
    "vaep_step_temporal_upsample", "vaep_profile_begin", "vaep_profile_end",
]

STEP_CONV, STEP_GROUPNORM, STEP_RMSNORM, STEP_ATTENTION, STEP_MOVE = 1, 2, 3, 4, 5
(KERNEL_OTHER, KERNEL_CONV_TILE128, KERNEL_CONV_WIDE256, KERNEL_CONV_WIDE128, KERNEL_CONV_NARROW,
 KERNEL_CONV_F32, KERNEL_CONV_WIDE128X512, KERNEL_CONV_HALO, KERNEL_CONV_HALO_X2) = 0, 1, 2, 3, 4, 5, 6, 7, 8


class VaepConfig(C.Structure):
    _fields_ = [
        ("family", C.c_int32), ("dtype", C.c_int32), ("z_channels", C.c_int32),
        ("n_stages", C.c_int32), ("stage_channels", C.c_int32 * MAX_STAGES),
        ("resnets_per_stage", C.c_int32), ("norm_groups", C.c_int32),
        ("temporal_up_stages", C.c_int32), ("eps", C.c_float),
    ]


class VaepDecodeInfo(C.Structure):
    _fields_ = [
        ("bands_used", C.c_int32), ("fell_back", C.c_int32), ("n_launches", C.c_int32),
        ("axis", C.c_int32), ("workspace_bytes", C.c_uint64),
    ]


class VaepProfileEntry(C.Structure):
    _fields_ = [
        ("step", C.c_int32), ("n_kernels", C.c_int32), ("kt", C.c_int32), ("ks", C.c_int32),
        ("cin", C.c_int32), ("cout", C.c_int32), ("ups", C.c_int32), ("mode", C.c_int32),
        ("pixels", C.c_int64), ("flops", C.c_double), ("bytes", C.c_double), ("ms", C.c_float),
        ("kernel", C.c_int32),
    ]


class VaepError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"vaep error {code}: {msg}")
        self.code = code


_lib = None

P = C.c_void_p
I = C.c_int
SZ = C.c_size_t


def _proto(lib):
    def f(name, res, *args):
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = list(args)

    f("vaep_last_error", C.c_char_p)
    f("vaep_version", C.c_char_p)
    f("vaep_config_preset", I, I, C.POINTER(VaepConfig))
    f("vaep_param_count", I, C.POINTER(VaepConfig))
    f("vaep_param_info", I, C.POINTER(VaepConfig), I, C.c_char_p, I, C.POINTER(C.c_int64),
      C.POINTER(C.c_int))
    f("vaep_model_create", I, C.POINTER(VaepConfig), C.POINTER(P), I, P, C.POINTER(P))
    f("vaep_model_destroy", I, P)
    f("vaep_model_set_norm_fold", I, P, I)
    f("vaep_model_set_halo_poison", I, P, I)
    f("vaep_workspace_bytes", I, P, I, I, I, I, I, C.POINTER(SZ))
    f("vaep_decode_full", I, P, P, I, I, I, I, P, P, SZ, P)
    f("vaep_decode_bands", I, P, P, I, I, I, I, C.POINTER(C.c_int32), I, P, P, SZ, P,
      C.POINTER(VaepDecodeInfo))
    f("vaep_select_axis", I, I, I, I, C.POINTER(C.c_int32))
    f("vaep_noalloc_scratch_bytes", SZ)
    f("vaep_decode_bands_noalloc", I, P, P, I, I, I, I, C.POINTER(C.c_int32), I, P, P,
      C.POINTER(VaepDecodeInfo))
    f("vaep_tiled_workspace_bytes", I, P, I, I, I, I, I, I, C.POINTER(SZ))
    f("vaep_decode_tiled", I, P, P, I, I, I, I, I, I, P, P, SZ, P)
    f("vaep_encoder_param_count", I, C.POINTER(VaepConfig))
    f("vaep_encoder_param_info", I, C.POINTER(VaepConfig), I, C.c_char_p, I, C.POINTER(C.c_int64),
      C.POINTER(C.c_int))
    f("vaep_encoder_create", I, C.POINTER(VaepConfig), C.POINTER(P), I, P, C.POINTER(P))
    f("vaep_encoder_destroy", I, P)
    f("vaep_encode_tiled_workspace_bytes", I, P, I, I, I, I, I, C.POINTER(SZ))
    f("vaep_encode_tiled", I, P, P, I, I, I, I, I, P, P, SZ, P, C.POINTER(VaepDecodeInfo))
    f("vaep_decode_sharded", I, P, P, I, I, I, I, I, C.POINTER(C.c_int32), I, P, P, SZ, P,
      C.POINTER(VaepDecodeInfo))
    f("vaep_sharded_workspace_bytes", I, P, I, I, I, I, I, C.POINTER(SZ))
    f("vaep_groupnorm_merge", I, I, I, P, P, P, P, P, P)
    f("vaep_profile_begin", I, P, I)
    f("vaep_profile_end", I, P, C.POINTER(VaepProfileEntry), I, C.POINTER(C.c_int))
    f("vaep_step_conv", I, I, I, P, I, I, I, I, I, P, P, I, I, I, I, I, I, P,
      C.POINTER(C.c_int32), I, P, P, SZ, C.POINTER(SZ), P)
    f("vaep_step_groupnorm", I, I, P, I, I, I, I, I, I, C.c_float, P, P, I,
      C.POINTER(C.c_int32), I, P, P, P, P, SZ, C.POINTER(SZ), P)
    f("vaep_step_rmsnorm", I, I, P, I, I, I, I, I, C.c_float, P, I, C.POINTER(C.c_int32), I,
      P, P, SZ, C.POINTER(SZ), P)
    f("vaep_step_attention", I, I, P, I, I, I, I, I, I, C.c_float, P, P, P, P, P, P, P, P, P, P,
      C.POINTER(C.c_int32), I, P, P, SZ, C.POINTER(SZ), P)
    f("vaep_step_temporal_upsample", I, I, P, I, I, I, I, I, P, P, C.POINTER(C.c_int32), I, P,
      P, SZ, C.POINTER(SZ), P)


def load(path: str = LIB_PATH):
    """Load libvaep.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with "
                               "`python -m spatially_sharded_conv_amd.build` (no fallback exists)")
        lib = C.CDLL(path)
        _proto(lib)
        _lib = lib
    return _lib


def last_error() -> str:
    return load().vaep_last_error().decode()


def check(code: int, allow_warning: bool = True) -> int:
    if code < 0 or (code > 0 and not allow_warning):
        raise VaepError(code, last_error())
    return code
