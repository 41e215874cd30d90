"""CPU oracle for causal grouped-query attention with a per-head sink logit and
an optional sliding window.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library and imports nothing from it.

``oracle.attention`` is the plain fp64 NumPy definition; ``oracle.brute`` is an
independent pure-Python scalar enumeration of the same definition;
``oracle.ring`` is the W-slot ring cache of windowed layers (append by position,
decode through the windowed definition); ``oracle.rope`` is the rotary position
encoding of new tokens and their KV-cache append; ``oracle.backward`` is the
gradient of the prefill (dq, dk, dv and the sink logits), the chain rule
applied to the forward definition.

Sources (the web pages this method is taken from):

* "GPT-OSS-20B : Architecture MoE & Résumé du Model Card" (papasega.github.io),
  §3.3 "Attention par Requêtes Groupées (GQA)": 64 query heads share 8 key/value
  heads, each KV head serving 8 query heads.
* "GPT-OSS vs Qwen3 : comparaison détaillée de l'évolution de l'architecture des
  LLM depuis GPT-2" (fr.news.hada.io), section "Utilisation de Sliding Window
  Attention": some layers attend only to the most recent 128 tokens; section
  "Attention Bias et Sinks": the sink is a learned bias logit per head that
  leaves the input tokens unchanged; section "Introduction de Grouped Query
  Attention (GQA)": keys/values are shared between query heads.
* "gpt-oss Deep Dive with Xiaoli Alex Shen" (postsingularityinstitute.com),
  "Key Moments" / "Critical Evaluation": dense and sliding-window layers
  alternate; "Pour aller plus loin": off-by-one attention.
* "OpenAI lance gpt-oss-20b, qui tient sur 16 Go" (orderchaos.eu), opening
  section: the models are autoregressive decoder-only transformers, hence
  causal attention.

Readings taken where the pages are silent (each also listed in the design notes):
sink = an extra zero-value logit in the softmax denominator, compared with the
*scaled* logits; one sink per query head; query head h uses KV head
h // (Hq/Hkv); a window W > 0 keeps exactly the W most recent keys including
the query's own position; queries of a chunk are the newest positions of their
sequence (bottom-right causal alignment); scale defaults to 1/sqrt(D).

Parity pins: every function here is pinned by tests in ``tests/test_oracle_pins.py``
and the ``tests/test_oracle_*_pins.py`` files of the other modules (brute force,
closed forms, library routines, finite differences, invariants).  No function is
"parity unpinned".
"""
from .attention import (  # noqa: F401
    attend,
    decode_ref,
    gather_paged,
    kv_head,
    prefill_ref,
    prefill_rows_ref,
    probabilities,
    varlen_ref,
    visible_mask,
)
from .backward import (  # noqa: F401
    dout_dot_out,
    prefill_grad_ref,
    row_grads,
)
from .rope import (  # noqa: F401
    default_inv_freq,
    new_positions,
    rope_append_ref,
    rope_ref,
)
from .ring import (  # noqa: F401
    decode_ring_ref,
    ring_append_ref,
    ring_from_history,
    ring_positions,
    ring_slot,
)
