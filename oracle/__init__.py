"""CPU oracle of one DeepSeekMoE layer forward with bias-based balancing.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  This package is a plain, slow, obviously
correct numpy statement of what the layer computes.  Only the tests, the smoke
check and the benchmark's CPU-baseline leg may import it.  It shares no code,
table or helper with the HIP library, and the library never calls it.

Floating point is fp64 except where the method itself fixes fp32: the affinity
that routing sees is rounded once to fp32, and the biased score, the group
score and the bias update are fp32 adds with round-to-nearest-even, because
that is the arithmetic the GPU must reproduce bit for bit.

Pins: every function is checked in tests/ against something other than itself
(brute-force enumeration, closed forms, library routines on special cases,
hand-derived fixtures in tests/golden/, central finite differences of an
independent forward for every gradient).  Parity unpinned by the pages: the
group-score rule (sum of the top-r biased scores of a group), the balance
trajectory values and the form of the sequence-wise balance loss; all are
readings, not page facts.
"""
from .route import affinity, route, route_diagnostics  # noqa: F401
from .dispatch import dispatch, permute_rows  # noqa: F401
from .ffn import swiglu, routed_ffn, shared_ffn  # noqa: F401
from .combine import combine  # noqa: F401
from .balance import update_bias  # noqa: F401
from .fp8 import e4m3_decode, e4m3_encode, quantize_rows_1x128, quantize_blocks_128x128, fp8_matmul  # noqa: F401
from .layer import decode_act, forward_from_routing, layer_forward, sampled_forward  # noqa: F401
from .backward import backward_from_routing, gate_backward, seq_balance_loss, swiglu_backward  # noqa: F401
