"""Plain CPU reference (the oracle) for the OSCAR INT2 decode path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package.  The product path (the HIP library and its Python binding) never
imports it, and this package imports nothing from the product path.  The two
share no code; only the seeded input generator (``synthetic/``) serves both.

What it computes, and where the pages say so:
  * write path, per token and KV head (``quant``): rotate by R, clip to +-tau,
    per-group asymmetric INT2 quantization with bf16 scale and zero, 4 codes
    per byte (MarkTechPost article, "The Serving System"; ModelScope/CSDN page,
    section on OSCAR's design, three-segment pool and packing paragraphs);
  * the logical three-segment pool with demotion of the oldest recent token
    (``pool``; ModelScope/CSDN page, same section);
  * decode attention as one softmax over the dequantized, inverse-rotated,
    concatenated pool in fp64 (``attention``), and the log-sum-exp merge of
    partial attentions (``merge``; ModelScope/CSDN page, decode paragraph on
    the split INT2/BF16 kernels and the online-softmax merge);
  * offline calibration (query and score-weighted value covariances, their
    eigenbases, R = U H P_br, clip thresholds) and the synthetic error chain
    that compares rotations by logit error, score KL and output MSE
    (``calibration``; MarkTechPost article, "What OSCAR Does Differently";
    ModelScope/CSDN page, motivation section, Figure 1);
  * the four-level Lloyd-Max codebook variant of the history quantizer
    (``codebook``; ModelScope/CSDN page, closing section).

Floating point: fp64 except where the method's encoding fixes an fp32 or bf16
rounding (the quantizer's scale, zero and code decisions), which are done in
IEEE fp32 / bf16 round-to-nearest-even exactly as stated in each function.

Every function is pinned by ``tests/test_oracle_*.py`` against brute force,
closed forms, invariants and special cases that reduce to textbook attention.
"""

from .numerics import round_bf16, f32  # noqa: F401
from .quant import (  # noqa: F401
    quantize_token, quantize_tokens, dequantize, pack_codes, unpack_codes,
)
from .pool import SeqPool  # noqa: F401
from .attention import decode_attention, bf16_decode_attention, attention_one_head  # noqa: F401
from .merge import merge_partials  # noqa: F401
from . import calibration  # noqa: F401
from . import codebook  # noqa: F401
from .calibration import calibrate  # noqa: F401
