"""CPU oracle for the Flash-Cache per-layer denoising step and the decode-side
reductions that follow it.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or run
anything in this package: only the test suite, the smoke check of the graft
entry point and the cpu_baseline leg of bench.py use it.  It shares no code with
the HIP library (no kernels, headers, helpers, tables or constants) and does not
import it; the two meet only through the seeded inputs of
io_aware_kv_amd.workloads, which hold none of the method's arithmetic.

Every function is the plain definition of one step, in float64, pinned by the
closed-form, invariant and brute-force tests in tests/test_oracle_*.py.
"""
from .flashcache import (  # noqa: F401
    OracleError,
    build_block_table,
    row_slots,
    project,
    rope,
    round_bf16,
    scatter,
    attention,
    column_mass,
    layer_range_score,
    topk,
    layer_step,
)
from .lowbit import E4M3_MAX, e4m3_decode, e4m3_encode, e4m3_round  # noqa: F401
from .decode import confidence_argmax, confidence_commit, verify_accept  # noqa: F401
