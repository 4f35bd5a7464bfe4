"""MI355X-native Mamba-2 SSD chunked scan (forward and backward).

The compute runs in ``libssd.so`` (HIP kernels for gfx950 behind the C ABI
of ``include/ssd.h``); this package is its Python binding.  Functions carry
the C names: ``ssd_fwd``, ``ssd_fwd_workspace_bytes``, ``ssd_status_string``,
``ssd_abi_version``, ``ssd_fwd_plan``, ``ssd_fwd_ex`` (as
``prepare(..., tuning=...).run(stages)``), ``ssd_bwd``, ``ssd_bwd_ex``,
``ssd_bwd_workspace_bytes`` (``prepare_bwd(...).run()`` re-launches);
``ssd_fwd_bidir`` (``prepare_bidir(...).run()`` re-launches) runs both
directions of the bidirectional mode.
"""
from ._binding import (  # noqa: F401
    CHUNK, SSD_BF16, SSD_F32, STAGE_ALL, STAGE_PASS, STAGE_SCAN, STAGE_STATE, STAGE_TABLE,
    TUNING_FIELDS, PreparedBidir, PreparedBwd, PreparedCall, SsdDims, SsdError, SsdLayout, SsdPlanInfo,
    SsdTuning, dims_for, layout_of, library, make_dims, make_tuning, prepare, prepare_bidir, prepare_bwd,
    ssd_abi_version, ssd_bwd, ssd_bwd_workspace_bytes, ssd_fwd, ssd_fwd_bidir, ssd_fwd_noalloc,
    ssd_fwd_noalloc_max_bytes, ssd_fwd_plan,
    ssd_fwd_workspace_bytes, ssd_status_string,
)
