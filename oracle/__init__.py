"""fp64 CPU oracle for the sparse decode path.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.
"""
from .rtp_oracle import (  # noqa: F401
    HEAD_DIM, INDEX_DIM, HeadResult, Selection, attend, bf16_to_f64, block_masses,
    block_tokens, decode_step, dense_head, index_query, index_scores, local_head,
    local_tokens, merge_partials, retrieval_head, retrieval_masses, select_top_p,
    token_softmax,
)
from .accept import (  # noqa: F401
    EPS_MASS, TOL_MAX_ABS, TOL_MEAN_REL, accept_selection, output_errors, outputs_ok,
)
