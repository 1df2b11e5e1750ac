"""MI355X (gfx950) decode-time sparse attention: RTPurbo's retrieval-head indexer with
exact block top-p, block-sparse split attention with a log-sum-exp reduce, and
window + sink attention for local heads, as hand-written HIP kernels behind the C
ABI in include/rtp.h (librtp.so).  This package is the thin Python binding."""
from .abi import (  # noqa: F401
    RTPError, lib, rtp_index_topp, rtp_index_topp_workspace_size, rtp_local_window_attn,
    rtp_local_window_workspace_size, rtp_sparse_attn_split, rtp_split_reduce, status_string, version,
)
from .step import DecodeStep, StepShape  # noqa: F401
