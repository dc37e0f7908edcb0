"""MI355X-native skinny residual GEMM  Y = X * W^T + R  (bf16 in, fp32 accumulate, bf16 out).

The compute runs in hand-written HIP kernels for gfx950 behind the C ABI in
``include/skinny.h`` (library ``libskinny.so``); this package only marshals
arguments to it. Importing the package does not load the library; the first
call into it does, and raises if the library has not been built.
"""
from . import synth  # noqa: F401  (input generators; no arithmetic of the operation)

__all__ = ["synth", "addmm", "addmm_default", "addmm_acc_f32", "addmm_shard", "addmm_shard_acc_f32",
           "kbit_gemv", "kbit_gemv_acc_f32", "kda_verify", "select_config", "configs", "config_resources", "version",
           "config_kernel"]


def __getattr__(name):
    if name == "ops":
        import importlib
        return importlib.import_module(".ops", __name__)
    if name in ("addmm", "addmm_default", "addmm_acc_f32", "addmm_shard", "addmm_shard_acc_f32",
                "kbit_gemv", "kbit_gemv_acc_f32", "kda_verify", "select_config", "configs", "config_resources", "version",
                "config_kernel"):
        from . import ops
        return getattr(ops, name)
    raise AttributeError(name)
