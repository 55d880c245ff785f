"""P-EAGLE parallel drafting + greedy verify on AMD Instinct MI355X (gfx950).

The compute path is libpe.so (HIP kernels behind the C ABI in include/pe.h); `binding` marshals
arguments to it. PyTorch is only used by callers for device memory and streams.
"""

from .binding import (  # noqa: F401
    PE_BF16,
    PE_ERR_INVALID,
    PE_ERR_UNSUPPORTED,
    PE_F32,
    PE_PROF_ATTENTION,
    PE_PROF_COUNT,
    PE_PROF_DOWN,
    PE_PROF_GATE_UP,
    PE_PROF_LM_HEAD,
    PE_PROF_O_PROJ,
    PE_PROF_QKV,
    PE_PROF_ROWS,
    PE_PROF_VERIFY_SCAN,
    PeError,
    load_library,
    make_config,
    make_kv,
    make_weights,
    pe_config,
    pe_config_validate,
    pe_destroy,
    pe_device_flags,
    pe_draft_ar,
    pe_draft_catchup,
    pe_draft_rows,
    pe_draft_step,
    pe_init,
    pe_kv,
    pe_last_error,
    pe_profile_enable,
    pe_profile_read,
    pe_status_string,
    pe_verify,
    pe_verify_sampled,
    pe_verify_static,
    pe_weights,
)
