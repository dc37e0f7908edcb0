"""ctypes declarations of libskinny.so (the C ABI in include/skinny.h). No arithmetic here."""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# SKINNY_LIB may name another build of the same C ABI (e.g. a build with different
# compiled configurations); by default the in-tree library is used.
LIB_PATH = os.environ.get("SKINNY_LIB") or os.path.join(PKG, "libskinny.so")

STATUS = {0: "SKINNY_OK", 1: "SKINNY_EINVAL", 2: "SKINNY_EALIGN", 3: "SKINNY_ENOTSUP", 4: "SKINNY_EHIP"}
PATH_GEMV = 0
PATH_MFMA = 1
PATH_MFMA_LDS = 2
PATH_GEMM = 3
PATH_SIMT = 4
PATH_GEMM_DMA = 5
PATH_GEMM_RING = 6
PATH_GEMM_WS = 7
FLAG_ROUND_PRODUCT = 1  # shard epilogue: round the product sum to bf16, add R, round again
FLAG_NO_NEG_ZERO = 2    # shard epilogue: write +0 for a -0 result
CONFIG_FIELDS = ("path", "block_size", "outputs_per_block", "k_unroll", "vector_width", "m_tile", "k_split",
                 "k_stage")

EXPORTED = ("skinny_addmm_bf16", "skinny_select_config", "skinny_addmm_bf16_with_config",
            "skinny_addmm_bf16_acc_f32", "skinny_addmm_bf16_shard", "skinny_addmm_bf16_shard_acc_f32",
            "skinny_kbit_gemv_bf16", "skinny_kbit_gemv_bf16_acc_f32", "skinny_kda_verify_bf16",
            "skinny_num_configs", "skinny_get_config",
            "skinny_config_resources", "skinny_status_string", "skinny_last_hip_error",
            "skinny_version", "skinny_probe_null", "skinny_probe_read", "skinny_probe_copy",
            "skinny_probe_read_rows", "skinny_probe_spin", "skinny_config_kernel_name")


class SkinnyConfig(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int32) for f in CONFIG_FIELDS]

    def as_dict(self) -> dict:
        return {f: int(getattr(self, f)) for f in CONFIG_FIELDS}


class SkinnyResources(ctypes.Structure):
    _fields_ = [("num_vgprs", ctypes.c_int32), ("spill_bytes", ctypes.c_int32),
                ("lds_bytes_static", ctypes.c_int32), ("max_threads", ctypes.c_int32)]


class SkinnyKdaArgs(ctypes.Structure):
    """skinny_kda_args of include/skinny.h (pointers as integers, sizes, scale)."""
    _fields_ = ([(f, ctypes.c_void_p) for f in ("mixed", "conv_w", "conv_b", "conv_pool", "cache_idx", "inter_idx",
                                                "a", "b", "A_log", "dt_bias", "ssm", "conv_win", "snap", "ring_v",
                                                "ring_k", "ring_g", "ring_beta", "out")]
                + [(f, ctypes.c_int64) for f in ("B", "T", "H", "HV", "K", "V", "lines", "slots", "ring_len")]
                + [("scale", ctypes.c_float)])


class SkinnyError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s: %s (%s)" % (what, STATUS.get(status, status), _status_text(status)))


_lib = None


def _status_text(status: int) -> str:
    try:
        return lib().skinny_status_string(status).decode()
    except Exception:  # noqa: BLE001
        return "?"


def lib() -> ctypes.CDLL:
    """Load libskinny.so; raise if it has not been built (there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libskinny.so is not built (%s); run `python -m decode_skinny_addmm_amd.build` "
                           "or __graft_entry__.build()" % LIB_PATH)
    # Load torch first so the library binds to the HIP runtime torch already uses
    # (same soname), and device pointers/streams from torch are valid for it.
    import torch  # noqa: F401
    L = ctypes.CDLL(LIB_PATH)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    cfgp = ctypes.POINTER(SkinnyConfig)
    L.skinny_addmm_bf16.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp]
    L.skinny_addmm_bf16_with_config.argtypes = [vp, vp, vp, vp, i64, i64, i64, cfgp, vp]
    L.skinny_addmm_bf16_acc_f32.argtypes = [vp, vp, vp, vp, i64, i64, i64, cfgp, vp]
    L.skinny_addmm_bf16_shard.argtypes = [vp, vp, vp, i64, vp, i64, i64, i64, i64, ctypes.c_uint32, cfgp, vp]
    L.skinny_addmm_bf16_shard_acc_f32.argtypes = [vp, vp, vp, i64, vp, i64, i64, i64, i64, ctypes.c_uint32,
                                                  cfgp, vp]
    L.skinny_kbit_gemv_bf16.argtypes = [vp, vp, vp, vp, ctypes.c_int32, vp, vp, i64, i64, i64, vp]
    L.skinny_kbit_gemv_bf16_acc_f32.argtypes = [vp, vp, vp, vp, ctypes.c_int32, vp, vp, i64, i64, i64, vp]
    L.skinny_kda_verify_bf16.argtypes = [ctypes.POINTER(SkinnyKdaArgs), vp]
    L.skinny_select_config.argtypes = [i64, i64, i64, cfgp]
    L.skinny_get_config.argtypes = [ctypes.c_int32, cfgp]
    L.skinny_config_resources.argtypes = [cfgp, ctypes.POINTER(SkinnyResources)]
    L.skinny_config_kernel_name.argtypes = [cfgp, ctypes.c_char_p, ctypes.c_int32]
    L.skinny_config_kernel_name.restype = ctypes.c_int
    L.skinny_status_string.argtypes = [ctypes.c_int]
    L.skinny_status_string.restype = ctypes.c_char_p
    L.skinny_version.restype = ctypes.c_char_p
    L.skinny_probe_null.argtypes = [vp]
    L.skinny_probe_read.argtypes = [vp, i64, vp, ctypes.c_int32, ctypes.c_int32, vp]
    L.skinny_probe_copy.argtypes = [vp, vp, i64, vp]
    L.skinny_probe_read_rows.argtypes = [vp, i64, ctypes.c_int32, vp, vp]
    L.skinny_probe_spin.argtypes = [i64, ctypes.c_int32, ctypes.c_int32, vp]
    for f in ("skinny_probe_null", "skinny_probe_read", "skinny_probe_copy", "skinny_probe_read_rows",
              "skinny_probe_spin"):
        getattr(L, f).restype = ctypes.c_int
    for f in ("skinny_addmm_bf16", "skinny_addmm_bf16_with_config", "skinny_addmm_bf16_acc_f32",
              "skinny_addmm_bf16_shard", "skinny_addmm_bf16_shard_acc_f32",
              "skinny_kbit_gemv_bf16", "skinny_kbit_gemv_bf16_acc_f32", "skinny_kda_verify_bf16",
              "skinny_select_config", "skinny_get_config", "skinny_config_resources",
              "skinny_num_configs", "skinny_last_hip_error"):
        getattr(L, f).restype = ctypes.c_int
    _lib = L
    return L


def check(status: int, what: str) -> None:
    if status != 0:
        raise SkinnyError(status, what)
