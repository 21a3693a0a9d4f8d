"""liboscar_kv: the OSCAR INT2 KV-cache hot path for AMD Instinct MI355X (gfx950).

The compute runs in hand-written HIP kernels behind a C ABI (include/oscar_kv.h); this
package is the thin Python binding over it (argument marshalling only) plus the host
utilities a caller needs to build the per-head rotations. PyTorch supplies device memory
and streams.
"""

from ._lib import (  # noqa: F401
    LIB_PATH,
    OSCAR_ERR_HIP,
    OSCAR_ERR_INVALID_ARG,
    OSCAR_ERR_UNSUPPORTED,
    OSCAR_ERR_WORKSPACE,
    OSCAR_OK,
    LayerDesc,
    OscarError,
    layer_desc,
    lib,
    oscar_attend,
    oscar_attend_codebook,
    oscar_calib_covariances,
    oscar_calib_workspace_bytes,
    oscar_check_desc,
    oscar_decode,
    oscar_decode_codebook,
    oscar_decode_dense_bf16,
    oscar_dense_workspace_bytes,
    oscar_decode_multi,
    oscar_decode_multi_codebook,
    oscar_decode_bf16,
    oscar_decode_int2,
    oscar_decode_int2_grouped,
    oscar_decode_step_grouped,
    oscar_decode_step,
    oscar_decode_step_codebook,
    oscar_decode_workspace_bytes,
    oscar_default_splits,
    oscar_demote,
    oscar_demote_grouped,
    oscar_demote_codebook,
    oscar_last_error,
    oscar_merge,
    oscar_page_bytes,
    oscar_partials_bytes,
    oscar_prepare,
    oscar_prepare_codebook,
    oscar_read_probe,
    oscar_status_string,
    oscar_version,
    oscar_window_splits,
    oscar_window_tokens,
)
