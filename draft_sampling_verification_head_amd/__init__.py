"""DSpark draft / verify / confidence hot path for MI355X (gfx950).

The compute lives in libdspark.so (hand-written HIP kernels behind the C ABI of
include/dspark.h); this package only builds it and binds it for torch tensors.
"""
from .binding import (markov_draft, markov_draft_one_launch, markov_draft_path,  # noqa: F401
                      markov_draft_plan, markov_draft_noalloc, draft_gave_up, rnn_draft,
                      markov_draft_schedule, markov_draft_schedule_fused,
                      rnn_draft_path, verify,
                      verify_markov, tv_labels, schedule, schedule_lagged, ConfRing, sts_fit, load,
                      DsparkError, F32, BF16, GLOBAL, EARLY_STOP, STS_NLL, STS_ECE)
