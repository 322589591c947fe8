"""MI355X-native batched speculative-decoding verification.

The verification runs in hand-written HIP kernels for gfx950 behind a C ABI
(include/spec_verify.h, built into libspecverify.so).  This package holds the
ctypes binding (``binding``), the build step (``_build``) and the seeded
synthetic workload generator (``workloads``).
"""
from .binding import (  # noqa: F401
    SpecVerifyError,
    load,
    profile_events,
    release_workspace,
    rng_uniforms,
    spec_verify,
    spec_verify_greedy,
    spec_verify_stats,
)
