"""TEST INFRASTRUCTURE ONLY -- the fp64 CPU oracle of the gated delta rule.

Nothing in the product package imports this; only tests, the smoke check
and the CPU-baseline leg of the benchmark may.  It shares no code with the
HIP path.

  recurrent_forward / recurrent_step : the definition, token by token
      (C, fp64; gdn_recurrence.c)
  chunked_forward  : the chunked UT form with its intermediates (numpy fp64)
  brute_force_forward, wy_ungated : explicit transition products and WY
      recursions, used to pin the two above on tiny inputs.
  activation.log_gate / beta_from_logits : the gate and beta activations
      from raw logits (the in-kernel activation's reference);
      activation.l2_normalize : q, k scaled to unit L2 norm per token and head.
  backward.recurrent_backward : gradients (dq, dk, dv, dbeta, dg, dh0) by
      autograd through the fp64 token recurrence (PyTorch CPU)
  backward.chunked_backward : the chunkwise backward steps with the gate
      terms (numpy fp64), pinned to the former.
  backward.activation_backward, l2_normalize_backward : the chain rules of
      the input activation and of the L2 normalisation.
"""
from .recurrence import recurrent_forward, recurrent_step, as_f64  # noqa: F401
from .chunked import chunked_forward  # noqa: F401
from .brute import brute_force_forward, wy_ungated, transition  # noqa: F401
from . import activation  # noqa: F401
from . import backward  # noqa: F401
