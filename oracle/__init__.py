"""CPU oracle for the DFlash draft-and-accept hot path.

TEST INFRASTRUCTURE ONLY.  Only tests, the smoke check and the benchmark's CPU
baseline leg may import this package; the product path never does.  It is a
plain, slow, fp64 numpy restatement of what the pages define:

* "Inside SGLang: DFlash and DFlash 2 Implementation" (himanshu-arora.com):
  Step 1 (context materialisation), Step 3 (block preparation), Step 4 (the
  draft backbone pass and lm_head selection), Step 6 (acceptance), Step 7
  (commit of the live verification rows).
* The CSDN DFlash article (devpress.csdn.net): the z-lab reference loop (target
  prefill, draft predict, target verify), the fused K/V materialisation
  section, the Kimi-K2.6-DFlash config sample and SGLang flow steps 7-9.

It shares no code with the HIP library.  Every function states the passage it
follows.  Pinned by the CPU tests (worked examples, closed forms, invariants,
library cross-checks, brute force); see each function for its pins.
"""
from .formats import round_bf16, round_e4m3, e4m3_decode, e4m3_encode, round_kv  # noqa: F401
from .primitives import rms_norm, rope_neox, silu, softmax, block_attention  # noqa: F401
from .dflash import (block_prep, project_context, draft_block, accept,  # noqa: F401
                     greedy_posterior, accept_logits, OracleCache, speculative_decode,
                     select_draft_tokens)
from .sampling import accept_sampling  # noqa: F401
from . import selector  # noqa: F401
from . import relay  # noqa: F401
