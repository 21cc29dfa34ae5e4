"""lossless_verify_tv_amd -- speculative-sampling verify and E2E-TV loss on
AMD MI355X (gfx950).

The work runs in hand-written HIP kernels behind a C ABI (``include/lvtv.h``,
``liblvtv.so``). This package holds the kernels and the ABI
(``csrc/``), the build script (``build``), a thin ctypes binding
(``spec_verify``, ``spec_verify_packed``, ``spec_verify_topkp``,
``e2e_tv_loss_fwd_bwd``, ``draft_loss_fwd_bwd``, ``dspark_schedule``) and the
seeded synthetic input generators (``synth``).

The binding loads the library lazily, on first call, and raises if it is
missing; there is no CPU fallback.
"""

from ._binding import (  # noqa: F401
    EXPORTS,
    LVTV_BF16,
    LVTV_F32,
    STATUS_BAD_K,
    STATUS_BAD_TRUNCATION,
    STATUS_BAD_TEMPERATURE,
    STATUS_BAD_TOKEN,
    STATUS_NONFINITE,
    OBJECTIVES,
    LvtvError,
    NOALLOC_SCRATCH_BYTES,
    PATHS,
    debug_draft_loss,
    draft_loss_fwd_bwd,
    draft_loss_logits_fwd_bwd,
    draft_loss_logits_workspace_bytes,
    draft_loss_workspace_bytes,
    dspark_schedule,
    e2e_tv_loss_fwd_bwd,
    e2e_tv_loss_workspace_bytes,
    load_library,
    new_workspace,
    spec_verify,
    spec_verify_noalloc,
    spec_verify_packed,
    spec_verify_packed_workspace_bytes,
    spec_verify_topkp,
    spec_verify_topkp_workspace_bytes,
    spec_verify_workspace_bytes,
    strerror,
)
