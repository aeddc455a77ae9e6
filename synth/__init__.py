"""Seeded synthetic inputs for the tile-overlap workloads.

This package only draws numbers: it holds none of the arithmetic of the
all-gather, the matrix products, the reduction or the all-to-all.  Both the
CPU oracle and the HIP path read the bits it produces, so the tests, the
smoke check and the benchmark all start from the same stored inputs.
"""

from .gen import (  # noqa: F401
    stream_key,
    raw_u64,
    uniform,
    normal_f32,
    bf16_rne,
    normal_bf16,
    small_int_bf16,
    small_int_f32,
    permutation,
    zipf_top2_routing,
    zipf_topk_gates,
)
from .configs import (  # noqa: F401
    CONFIGS, AgGemmCfg, GemmRsCfg, DispatchCfg, RingCfg,
    ag_inputs, rs_inputs, dispatch_inputs, combine_inputs, ring_inputs, producer_order,
)
