"""CPU oracle for the tile-overlap hot path.

TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the library under
`communication_overlap_amd/` never does, and this package imports nothing
from it.  It computes, slowly and plainly, what the overlapped kernels must
produce: overlap changes only *when* work happens, never the result, so each
function here is the plain definition of its result, in float64.

Parity pins (tests/test_oracle_*.py) tie every function to facts outside this
package: brute-force loops, exact (math.fsum) sums, closed forms (identity
operands, small-integer inputs), two independent constructions of the
all-to-all layout, and the invariants the pages state.  No function is
"parity unpinned".
"""

from .bf16 import bf16_to_f64, bf16_to_f32  # noqa: F401
from .ag_gemm import all_gather, ag_gemm, gemm, gemm_entries, ag_flag_units, expected_flags  # noqa: F401
from .gemm_rs import gemm_rs, rs_expected_flags  # noqa: F401
from .dispatch import dispatch_layout, dispatch, grouped_gemm, grouped_gemm_rows  # noqa: F401
from .combine import combine, combine_positions  # noqa: F401
from .ring import ring_allreduce, allreduce_sum, ring_chunk_bounds  # noqa: F401
from .fp8 import e4m3_decode, e4m3_encode, quantize_rows, dispatch_fp8, grouped_gemm_fp8  # noqa: F401
