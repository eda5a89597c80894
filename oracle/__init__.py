"""Float64 CPU oracle for Nystrom attention.  Test infrastructure only: the
test suite, the smoke check and the benchmark's CPU-baseline leg may import
it; the HIP library never does."""
from .nystrom_oracle import (  # noqa: F401
    INIT_EXACT, INIT_ORIGINAL, depthwise_conv_same, exact_attention, init_scale,
    newton_schulz_pinv, nystrom_attention, nystrom_kernels, scale_qk,
    segment_means, softmax_rows)
