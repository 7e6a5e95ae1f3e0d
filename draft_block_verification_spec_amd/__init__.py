"""MI355X-native draft-block verification for speculative decoding.

The work runs in ``libspecverify.so`` (HIP kernels for gfx950 behind the C ABI in
``include/spec_verify.h``); :mod:`.binding` marshals torch tensors into it and
:mod:`.workload` draws the seeded synthetic inputs.  Importing the package does
not load the library; the first call does, and fails if it has not been built.
"""
from .binding import (  # noqa: F401
    SpecVerifyError, Weights, Outputs, make_outputs, workspace, sv_workspace_bytes, spec_verify_greedy,
    spec_verify_sample, spec_verify_scheduled, spec_draft_propose, version, load,
    SV_MODE_GREEDY, SV_MODE_SAMPLE, SV_MODE_SCHEDULED, SV_MODE_PROPOSE, SV_DIAG_COLS,
    SV_DEV_OK, SV_DEV_BAD_TOKEN, SV_DEV_NONFINITE,
)
