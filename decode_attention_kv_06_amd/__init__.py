"""MI355X (gfx950) decode attention: IncreFlashAttention and SparseFlashAttention.

The compute lives in libifadecode.so (hand-written HIP kernels behind the C ABI
in include/ifa_decode.h); this package holds the ctypes binding, the seeded
workload generators and the build script.
"""
from .binding import (IFA_ERR_PARAM_INVALID, IFA_ERR_PARAM_NULLPTR, IFA_ERR_RUNTIME, IFA_OK, IfaError,
                      ifa_decode, ifa_decode_paged, sfa_decode_mla, status_string)

__all__ = ["ifa_decode", "ifa_decode_paged", "sfa_decode_mla", "IfaError", "status_string", "IFA_OK",
           "IFA_ERR_PARAM_NULLPTR", "IFA_ERR_PARAM_INVALID", "IFA_ERR_RUNTIME"]
