"""Looped normalized-GPT forward pass on gfx950 (MI355X).

The implementation is the HIP library libdory.so (include/dory.h); this
package is its thin Python binding. The binding loads on first use of any
name below and raises ImportError if the library is not built: there is no
CPU fallback. (`looped_ngpt_amd.build` imports without the library.)
"""
_NAMES = (
    "DoryError", "Session", "make_config", "validate_config", "kv_bytes", "workspace_bytes", "kv_slot",
    "upload_weights", "op_linear", "op_argmax", "op_argmax_noalloc", "argmax_scratch_bytes", "lib", "EXPORTS",
    "quantize_weights_mxfp8", "op_quant_mxfp8", "op_linear_mx", "WEIGHTS_DTYPE", "WEIGHTS_MXFP8", "PROJECTIONS",
    "WEIGHTS_NVFP4", "quantize_weights_nvfp4", "op_quant_nvfp4", "op_linear_fp4", "backward_workspace_bytes", "backward_workspace_min_bytes",
    "DORY_OK", "DORY_E_ARG", "DORY_E_CAPACITY", "DORY_E_LOOPS", "DORY_E_KV_MODE", "DORY_E_STATE", "DORY_E_HIP",
    "DORY_F32", "DORY_BF16", "DORY_KV_PER_LOOP", "DORY_KV_LAST_LOOP", "KV_MODES",
)
__all__ = list(_NAMES)


def __getattr__(name):
    if name in _NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
