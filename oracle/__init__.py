"""fp64 CPU oracle for fused multi-head softmax attention, forward and backward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this
package: only the tests, the smoke check and the benchmark's CPU-baseline leg
call it.  It shares no code with the HIP library (no kernels, headers,
helpers or constants); both sides are fed by the seeded input generator, which
holds none of the method's arithmetic.

The oracle is the plain definition of attention written out in float64 with
no tiling and no online rescaling:

  * ``attention.visible``     -- the visibility predicate of the four mask modes
  * ``attention.oracle_fwd``  -- O and the per-row natural-log logsumexp
  * ``attention.oracle_bwd``  -- dQ, dK, dV of L = <O, dO>
  * ``premix.premix_fwd``     -- IHA pseudo-token construction
                                 Out[h, p] = sum_s W[h, p, s] X[s]
  * ``premix.premix_bwd``     -- its dX = W^T dOut and dW = sum dOut X^T
  * ``brute``                 -- scalar loops with math.fsum for tiny inputs,
                                 used only to pin the vectorised functions

Every function is pinned by tests that do not retype its formula: scalar brute
force, torch's own fp64 ``scaled_dot_product_attention`` with autograd,
central finite differences, closed forms and invariants.
"""
from .attention import MASKS, visible, oracle_fwd, oracle_bwd
from .premix import premix_bwd, premix_fwd, pseudo_tokens

__all__ = ["MASKS", "visible", "oracle_fwd", "oracle_bwd", "premix_fwd", "premix_bwd",
           "pseudo_tokens"]
