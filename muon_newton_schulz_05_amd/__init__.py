"""Shape-fused Muon optimizer step for AMD MI355X (gfx950).

The computation lives in hand-written HIP kernels behind the C ABI of
``include/muon.h`` (``libmuon.so``); this package only loads that library and
marshals arguments.  Importing does not load the library; ``MuonPlan`` and the
``muon_*`` functions do, and fail loudly if it has not been built.
"""

from .binding import (  # noqa: F401
    EXPORTED,
    KERNEL_CLASSES,
    LIB_PATH,
    MUON_BF16,
    MUON_F32,
    MUON_MODE_BF16_MFMA,
    MUON_MODE_FP32,
    MuonError,
    MuonPlan,
    PlanInfo,
    info_dict,
    load_library,
    make_descs,
    make_opts,
    muon_default_opts,
    muon_last_error,
    muon_plan_create,
    muon_plan_describe,
    muon_plan_destroy,
    muon_plan_query,
    muon_plan_status,
    muon_plan_timings,
    muon_step,
    muon_step_noalloc,
    MUON_NOALLOC_SCRATCH_BYTES,
)
