"""CPU oracle for the DSpark per-step draft/verify path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library.

It is a plain, slow and deliberately unoptimised restatement of what the
method computes, in float64 over the decoded fp32/bf16 inputs.  Every function
cites the passage of the pages it follows.  The pages are cited by title and
section:

  [blog]      "DSpark：半自回归生成与置信度调度的投机解码" (DSpark: semi-autoregressive
              generation and confidence-scheduled speculative decoding),
              pinghaoyang.com.cn/aigc/posts/dspark/
  [teardown]  "拒绝盲猜与算力空转：深度拆解 DeepSeek 开源投机采样方案 DeepSpec & DSpark",
              val213.github.io/2026/06/28/DSpark&DSpec/
  [summary]   "DeepSeek-AI与北京大学联手破局：AI聊天机器人'慢速打字'的终极解决方案",
              techwalker.com/2026/0716/3193540.shtml

Pins (tests/test_oracle_*.py) tie each function to something other than
itself: published RNG test vectors, closed forms, the P3 one-hot matrix form of
the bias, exact enumeration of the lossless law, Monte-Carlo chi-square
against softmax / target laws, brute-force scheduling, scikit-learn's reliability curve (for the
calibration error), recovery of known temperatures, and hand-worked
fixtures under tests/golden/.
"""
from .rng import (DRAFT, ACCEPT, RESID, BONUS, mix64, splitmix64_next, fmix32, row_key,
                  uniforms, uniform_at, gumbels)
from .sampling import gumbel_draw, gumbel_keys
from .markov import decode_weights, markov_bias, draft_markov, DraftResult
from .rnn import gru_cell, draft_rnn
from .confidence import confidence, ConfidenceResult
from .schedule import schedule, schedule_async, ScheduleResult
from .verify import verify, VerifyResult, target_logprobs, accept_ratio, residual_weights, accept_prob
from .step import run_step, step_lengths, StepResult
from .sts_fit import ece, labels, candidate_scores, sts_fit, StsFit

__all__ = [
    "DRAFT", "ACCEPT", "RESID", "BONUS", "mix64", "splitmix64_next", "fmix32", "row_key",
    "uniforms", "uniform_at", "gumbels", "gumbel_draw", "gumbel_keys", "decode_weights", "markov_bias", "draft_markov", "gru_cell", "draft_rnn",
    "DraftResult", "confidence", "ConfidenceResult", "schedule", "schedule_async", "ScheduleResult", "verify",
    "VerifyResult", "target_logprobs", "accept_ratio", "residual_weights", "accept_prob", "run_step", "step_lengths",
    "StepResult", "ece", "labels", "candidate_scores", "sts_fit", "StsFit",
]
