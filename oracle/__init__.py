"""CPU oracle for the Mixture-of-Experts router.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
CPU-baseline leg of the benchmark; never by the product package. It shares no
code with the HIP library. The arithmetic lives in ``moero.c`` (plain C,
fp64); this package only builds it and marshals numpy arrays.
"""
from .api import (  # noqa: F401
    PROPORTIONAL,
    SIGN,
    SIGMOID,
    SOFTMAX,
    affinities,
    agg_entropy,
    balance_step,
    balanced_indices,
    bias_update,
    build_oracle,
    capacity_route,
    combine,
    dispatch,
    hotspot_accumulate,
    layout,
    load_stats,
    logit_bias,
    num_threads,
    route,
    scores,
    select,
    set_num_threads,
)
