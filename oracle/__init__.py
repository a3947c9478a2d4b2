"""Oracle for the chunked gated-delta-rule prefill.  TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously correct CPU implementation in float64
of what the GPU library computes.  Only the test-suite, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it.  The product package
(``linear_attention_ssm_chunk_amd``) never imports it, and it imports nothing
from the product package: the two share no code.

Modules
-------
``recurrence``  the definition: the gated delta rule token by token (the
                method the page "spark_model/layers/ops/ssm_gdn_a3.rs" runs
                as its GDN prefill, kernels gated_delta_rule_chunk_*; the
                recurrence for S_t and o_t), entry states recorded at every
                64-token chunk boundary.
``normalize``   the per-token L2 normalisation of queries and keys that
                the method applies before the recurrence (``l2_normalize``).
``chunked``     the same result reached in 64-token chunks, in the three
                stages the page "spark_model/layers/ops/ssm_gdn_a3.rs"
                lists in the doc comment of ``gdn_prefill_fla`` (cumulative
                log-gate and WY/UT solve; serial state spine emitting
                per-chunk entry states; per-chunk output).  Used to check the
                GPU path's intermediates (gc, W, U, entry states, corrected
                values) stage by stage.

Conventions shared with the GPU library only through documentation:

* state orientation: ``h[dk][dv]`` as the page's ``h_state`` comment gives it
  (one state per request, key dimension before value dimension), i.e. the
  transpose of the recurrence's S;
* GQA grouping (the pages are silent): v-head ``h`` reads k-head
  ``(h * nk) // nv`` -- parity unpinned, it is a convention;
* no query scale (the recurrence's ``o_t = S_t q_t`` has none).
"""

from .recurrence import gdn_recurrence, kv_head_map  # noqa: F401
from .normalize import l2_normalize  # noqa: F401
from .chunked import (  # noqa: F401
    chunk_cumsum,
    gram_strict_lower,
    wy_solve,
    ut_transform,
    spine_step,
    chunk_output,
    gdn_chunked,
)
