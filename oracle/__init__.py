"""CPU oracle for the ROCS shared-forward stack -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call anything in this package.  The product path
(``request_candidate_sharing_amd``) never does: it has no CPU fallback.

What it computes
----------------
The dense, early-fused model with explicitly masked weights and a
materialized broadcast, evaluated candidate by candidate in float64.  The
shared (request-once) execution of the HIP path is a re-association of the
same arithmetic, so this plain definition is the expected result up to
rounding order.

Citations name the web pages by title:

* [R]  "ROCS：面向请求的大规模推荐计算共享" (liuzhao09.github.io review of the
  ROCS paper).  §2.1 Generalized Layer Masking (GLM invariance, two-group
  form, dependency mask, masked-weight linear equation, two-group block
  matrix, masked FM, request-output equality), §2.2 Deep Cross Attention
  (request-only encoder, query generator, grouped cross-attention), §2.4
  In-Kernel Broadcast Optimization (decomposed LCB equation).
* [D]  "Meta推出ROCS：推荐系统推理效率提升3倍，零质量损失" (longzhangge.com
  PaperDaily digest), section on the three mechanisms.

* [U]  "Compute Only Once: UG-Separation for Efficient Large Recommendation
  Models" (xllm-io review), §3 (TokenMixer layer, separation mask,
  information compensation): ``oracle/ugsep.py``; stage 4 and the W8A16
  configuration (8-bit float weights, bf16 activations): ``oracle/w8a16.py``.

Pins of every function are listed in the ``oracle/ops.py``,
``oracle/stack.py``, ``oracle/ugsep.py`` and ``oracle/w8a16.py`` headers.  The
stack compositions are readings of the workload descriptions (the pages fix
their operators only); each composition is pinned by special-weight closed
forms computed with library routines.
"""

from .ops import (  # noqa: F401
    glm_mask,
    glm_linear,
    group_norm,
    relu,
    masked_fm,
    token_lcb,
    attention,
    mha,
    encoder_layer,
    decomposed_linear,
)
from .stack import oracle_forward, oracle_encoder  # noqa: F401
from . import ugsep, w8a16  # noqa: F401
