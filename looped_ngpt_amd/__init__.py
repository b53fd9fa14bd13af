"""Looped normalized-GPT forward pass on gfx950 (MI355X).

The implementation is the HIP library libdory.so (include/dory.h); this
package is its thin Python binding. Importing it without the built library
raises: there is no CPU fallback.
"""
from .binding import (  # noqa: F401
    DoryError, Session, make_config, validate_config, kv_bytes, workspace_bytes, kv_slot,
    upload_weights, op_linear, op_argmax, argmax_scratch_bytes, lib, EXPORTS,
    DORY_OK, DORY_E_ARG, DORY_E_CAPACITY, DORY_E_LOOPS, DORY_E_KV_MODE, DORY_E_STATE, DORY_E_HIP,
    DORY_F32, DORY_BF16, DORY_KV_PER_LOOP, DORY_KV_LAST_LOOP, KV_MODES,
)
