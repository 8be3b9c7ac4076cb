"""MI355X-native chunked gated linear attention (GLA): prefill forward, backward
and decode, and the gated delta rule forward.

The computation lives in libgla.so (hand-written HIP kernels for gfx950 behind
the C ABI in include/gla.h, include/gla_scalar.h, include/gla_bwd.h,
include/gla_gdn.h and include/gla_decode.h); this package is its thin Python binding.  Build
the library with ``python -m chunked_state_recurrence_amd.build``.
"""

from ._binding import (  # noqa: F401
    EXPORTED,
    GLAError,
    GLALibraryMissing,
    LIB_PATH,
    gla_gdn_fwd,
    gla_bwd,
    gla_bwd_f32,
    gla_decode,
    gla_decode_f32,
    gla_fwd,
    gla_fwd_f32,
    gla_fwd_noalloc,
    gla_fwd_scalar,
    gla_fwd_scalar_f32,
    gla_stage_cumsum,
    gla_stage_intra,
    gla_stage_states,
    load_library,
    profile_start,
    profile_stop,
    release,
    set_tuning,
    gdn_set_path,
    strerror,
    version,
    workspace_bytes,
)
