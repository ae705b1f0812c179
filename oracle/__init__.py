"""fp64 CPU oracle for the DSpark draft / verify / confidence path.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or link this
package; only the tests, the package smoke check and the benchmark's CPU-baseline leg
use it. It shares no code with the HIP library: the two meet only in the seeded input
generators of ``synth``.

Everything is plain numpy in float64, request by request and row by row, with no
blocking, fusion or reordering beyond the definitions it follows. bf16 inputs are
decoded exactly (bits << 16) and fp32 inputs are widened exactly.

Pages cited (titles as published):

* [P1] "大模型推理加速的系统级工程：DeepSeek V4-Pro DSpark 推测解码方案深度解析与开源工具链
  DeepSpec" (Best Partners TV, 2026-06-30).
* [P2] "DeepSeek 开源 DSpark，一个可将大语言模型推理速度提升高达 85% 的新框架"
  (VentureBeat article, Chinese translation).
* [P3] "DSpark Speculative Decoding" (concept note).

Functions and what pins them (all pins live in ``tests/test_oracle_*.py``):

* ``inverse_cdf``, ``clamp_uniform`` - the one-uniform draw from a law in token-id order
  (the reading for how [P3] "Semi-Autoregressive Generation"'s sample is drawn) and the
  clamp of a host uniform into [0, 1 - 2^-24] (NaN counts as 0). Pinned by laws with exact
  dyadic cumulative sums (boundaries, zero-mass tokens, the past-the-end fallback, an empty
  law), a brute force in exact rationals, fixed clamp values, and planted mistakes that
  those pins catch.

* ``markov_draft`` - [P3] "Semi-Autoregressive Generation" (p_k formula, Markov bias
  B = W1[x_{k-1}] W2). Pinned by rational-weight distributions with integer CDFs, a
  one-hot Markov bias with exact expected tokens, a permutation chain, a dominant logit,
  logsumexp against scipy and a chi-squared test of the sampler. Its ``forced`` option
  (the conditional laws along a given block) is pinned by the permutation chain on an
  arbitrary block and by equality with the plain draft on its own draws.
* ``rnn_draft`` - [P3] "Semi-Autoregressive Generation" (the RNN head: a recurrent state
  inside the block) and [P1] "DSpark 架构设计：半自回归生成与马尔可夫修正" (its paragraph), with
  the reading h_1 = W1[x_0], h_k = A h_{k-1} + W1[x_{k-1}], B_k = h_k W2. Pinned by A = 0
  reproducing ``markov_draft`` bit for bit, a permutation-matrix A with one-hot W1 and
  log-integer W2 (an integer law of the whole prefix, exact tokens and states), the A = 2I
  chain whose context token keeps the largest weight, and forcing on its own draws.
* ``verify`` - [P1] "大模型推理的显存瓶颈与推测解码的演进逻辑" (rejection sampling) and [P3]
  intro (longest prefix + bonus). Pinned by p_d = p_t, zero target mass on a draft token,
  len = 0, and chi-squared losslessness (single position and multi-round joint). Its
  ``n_forced`` option and ``ratio`` output are pinned by two-point laws with exact ratios,
  residuals and bonus draws.
* ``tv_labels`` - [P3] "Confidence-Scheduled Verification" (c* = 1 - 1/2 ||p_d - p_t||_1).
  Pinned by exact rational arithmetic, the two-point closed form, identical and disjoint
  rows, and the Monte-Carlo acceptance rate of ``verify``.
* ``temperature_scale``, ``prefix_survival``, ``schedule``, ``brute_force_schedule`` -
  [P1] "硬件感知与置信度自适应调度机制" and [P3] "Confidence-Scheduled Verification"
  (a_{r,j} = prod c, Theta = tau * SPS(B)). Pinned by brute-force enumeration, the
  constant-SPS and zero-SPS closed forms, early-stop = global for a smooth curve, a
  step-shaped curve with known answers, and exact temperature values.
* ``lagged_confidences``, ``lagged_schedule`` - [P1] same section (the asynchronous
  adaptation: step t is scheduled from the confidences of step t - 2) and [P3] same section.
  Pinned by the no-history closed form (all ones: lengths from the SPS curve alone) and by
  round t's schedule ignoring rounds t and t - 1 while following round t - 2.
* ``outcomes``, ``scale``, ``nll``, ``ece``, ``sts_fit`` - [P1] "硬件感知与置信度自适应调度机制"
  (sequential temperature scaling: a per-position 1-D grid search, order preserving, judged
  by the expected calibration error) and [P3] "Confidence-Scheduled Verification" (c_k is
  the acceptance probability given the prefix). Pinned by the outcome pattern of verify's
  results, a hand-computed ECE, the closed-form NLL optimum logit(c)/logit(p) for a single
  score, recovery of the temperature that generated Bernoulli outcomes, T = 1 leaving the
  ECE unchanged, and order preservation.
"""
from .numerics import decode_factor, clamp_uniform, softmax_row, inverse_cdf
from .draft import markov_draft
from .rnn import rnn_draft
from .verify import verify, accept_test
from .tv import tv_labels, tv_row_pair
from .schedule import (temperature_scale, prefix_survival, schedule, brute_force_schedule,
                       theta_curve, lagged_confidences, lagged_schedule, GLOBAL, EARLY_STOP)
from . import sts

__all__ = [
    "decode_factor", "clamp_uniform", "softmax_row", "inverse_cdf", "markov_draft", "rnn_draft",
    "verify", "accept_test", "tv_labels", "tv_row_pair", "temperature_scale",
    "prefix_survival", "schedule", "brute_force_schedule", "theta_curve", "lagged_confidences",
    "lagged_schedule", "GLOBAL",
    "EARLY_STOP",
]
