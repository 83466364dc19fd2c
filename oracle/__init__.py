"""CPU oracle for tiled exact attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package.  The product path (the HIP
library and its Python binding) never imports, calls or links it, and the
oracle never imports the product package: the two share no code.

Everything here is plain numpy in float64.  Inputs of any float dtype are
upcast exactly to float64 before any arithmetic.

Modules
-------
attention
    The plain definition softmax(scale * Q K^T, masked) V, its natural-log
    log-sum-exp, and the analytic gradient of that definition.
online
    The block-by-block online-softmax recurrence, in both loop orders the
    pages print.  Used only to check ``attention`` against an independent
    formulation of the method.
philox
    Philox4x32-10 from its published definition (Salmon et al., SC 2011)
    and the dropout keep-mask built from it.  The attention dropout is
    defined by this mask; the HIP library implements the same published
    generator separately.

Sources (cited by page title and section):
  [tonho] "FlashAttention: Fast and Memory-Efficient Exact Attention with
          IO-Awareness", digest on tonho.wtf -- sections "o problema",
          "como funciona".
  [mm]    "Um contexto de dia inteiro supera um contexto de dez minutos?
          Atencao Flash e a questao do comprimento da sequencia",
          marketmaker.cc -- "O algoritmo de atencao do Flash", "A recorrencia
          do softmax online", "O mascaramento causal ...", "Uma verificacao
          de exatidao".
  [ldl]   "Atencao Eficiente em Escala", living-dl-book -- section 8
          (FlashAttention v1).
  [agi]   "FlashAttention: Fast and Memory-Efficient Exact Attention with
          IO-Awareness", agihunt.info summary -- algorithm, IO and
          block-sparse paragraphs.
  [lynx]  "02 -- FlashAttention como una optimizacion de roofline",
          lynx-cortex -- "El algoritmo naive de attention", "El algoritmo
          Flash (forward)", "Por que Flash es exacto", "Una nota sobre
          Flash 1 vs Flash 2", "Problemas de practica".

Parity status: every function is pinned by CPU tests (closed forms,
invariants, finite differences, library routines, the tiled recurrence,
the generator's published known-answer vectors, binomial bounds);
see tests/test_oracle_*.py.  No function here is "parity unpinned".
"""

from .attention import (  # noqa: F401
    visibility,
    attention_forward,
    attention_backward,
    attention_probs,
)
from .philox import dropout_keep, philox4x32_10  # noqa: F401
from .online import tiled_forward_kv_outer, tiled_forward_q_outer  # noqa: F401
