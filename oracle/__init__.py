"""CPU oracle for the PRISM rank-L gated delta-rule forward.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this package.  The product path (the
HIP library and its Python binding) never calls it, and it shares no code
with that path.

The oracle is plain float64 numpy that steps the recurrence token by token
and runs the residual chain one refinement step at a time.  See
``oracle.prism`` for the definitions and the passages each one follows,
``oracle.prism_grad`` for the float64 gradients of the same forward, and
``oracle.prism_nl`` for the nonlinear refinement variant (the GELU of the
gain-modulated residual in the chain) and its absorbed per-channel factors, and
``oracle.prism_delta`` for the written-correction form (each layer writes its
GELU correction along its own key with its own gate) and the predictor front end
(gains, keys and gates from the anchor).
"""
from .prism import (shortconv_anchor, residual_chain, token_step, forward,
                    forward_pairs, conv_tail, decode_step)

__all__ = ["shortconv_anchor", "residual_chain", "token_step", "forward",
           "forward_pairs", "conv_tail", "decode_step"]
