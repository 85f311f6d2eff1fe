"""Plain CPU oracle of the serial draft walk -- TEST INFRASTRUCTURE ONLY.

Follows "Weights That Stay: On-Chip Megakernels for Serial Heads in Speculative
Decoding" (arXiv 2611.00506): abstract, Fig. 2 (serial refinement through one
shared vocabulary projection), Fig. 7 (two int8 vectors for the latent, scaled
results summed, base logits added, one rounding to bf16), Fig. 8 (selection of
one common winner across all workers), Fig. 10 (T=0 and T=1), Fig. 13
(Markov and recurrent heads; the fixed-latent probe of Fig. 13b).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or runs anything from here, and this
package imports nothing from the product path.

Arithmetic contract: every float32 operation on the bit-exact path is one
numpy float32 element-wise operation (IEEE-754 binary32, round to nearest
even, no fused multiply-add).  Integer dot products are exact (int64).
Parity status of each function is stated in its docstring; the Philox
stream is pinned by one published known-answer vector and by statistics.
"""
from .fp import bf16_rne, bf16_to_f32, log_p, exp_p, tanh_p  # noqa: F401
from .quant import quant_hilo  # noqa: F401
from .philox import philox4x32_10, uniform24, gumbel_noise  # noqa: F401
from .walk import (  # noqa: F401
    order_key, select_token, project_int8, epilogue_int8, project_bf16,
    recurrent_preact, recurrent_update, log_normaliser, walk,
)
