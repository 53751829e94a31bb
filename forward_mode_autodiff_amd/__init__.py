"""MI355X-native fused attention forward with tangents (JVP) and its reverse pass, behind a C ABI.

The computation lives in libjvpattn.so (HIP, gfx950); ``jvpattn`` is the
ctypes binding with the C names. Build with
``python -m forward_mode_autodiff_amd.build``.
"""
from .jvpattn import (JVPATTN_BF16, JVPATTN_F16, JVPATTN_F32, JVPATTN_MASK_ADDITIVE, JVPATTN_MASK_BOOL,
                      JVPATTN_MASK_NONE, JvpattnError, jvpattn_bwd, jvpattn_bwd_workspace_bytes,
                      jvpattn_check_bwd, jvpattn_check_fwd, jvpattn_fwd, jvpattn_params, jvpattn_strerror,
                      load_library)

__all__ = ["jvpattn_fwd", "jvpattn_check_fwd", "jvpattn_bwd", "jvpattn_check_bwd", "jvpattn_bwd_workspace_bytes",
           "jvpattn_strerror", "jvpattn_params", "JvpattnError",
           "load_library", "JVPATTN_F32", "JVPATTN_F16", "JVPATTN_BF16", "JVPATTN_MASK_NONE",
           "JVPATTN_MASK_BOOL", "JVPATTN_MASK_ADDITIVE"]
