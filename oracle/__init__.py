"""CPU oracle for the AWQ W4A16 hot path.  TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct reference that the HIP
library is checked against.  Only the test suite, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it.  The product path
(``bit_weight_only_quantize_amd``) never imports, calls or links anything here,
and this package imports nothing from the product path.

Sources (the pages this follows, cited by title and section):

* "AWQ Advanced Usage Guide" (skillselion.com awq-quantization skill, page
  "Awq Quantization"): section "How AWQ Works" gives the objective
  L(s) = ||Q(W*s)(s^-1*X) - W*X||; sections "Group Size Configuration" and
  "Zero-Point Quantization" give w_bit=4, q_group_size=128 and the meaning of
  zero_point (an offset for asymmetric weight distributions).
* ai.lansai.wang AWQ explainer, section "AWQ 的四步链路" (the four-stage
  chain): the equivalence Y = XW = (X/s)(sW) with a positive per-input-channel
  s, and the pipeline statistics -> salient channels -> scale search -> pack;
  its checkpoint-field table defines a group as consecutive weights that share
  quantization parameters and zero_point as an asymmetric mapping with a zero
  point.

Precision: every decision that produces an integer (a code, a zero point, the
chosen alpha index) is taken in IEEE fp32 exactly as the kernels take it
(correctly rounded division, round-half-to-even); dequantisation, the matmul
and the search loss are fp64.

Parity status per function is listed in each module header.
"""

from .quant import (  # noqa: F401
    ORDER,
    SYM_ZERO,
    QuantConfig,
    quantize_groups,
    pack_codes,
    unpack_codes,
    dequantize,
    quantize_pack,
)
from .linear import gate_up_silu64, linear64, linear_naive, silu64  # noqa: F401
from .search import (  # noqa: F401
    CLIP_GRID,
    DEFAULT_ALPHAS,
    activation_mean_abs,
    clip_search,
    group_gram,
    quantize_group_clipped,
    weight_mean_abs,
    scale_vector,
    scale_table,
    scaled_activation,
    reference_output,
    search_loss,
    scale_search,
)
from .bf16 import bf16_bits_to_f32  # noqa: F401
