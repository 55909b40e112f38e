"""Oracle for MLA decode with weight absorption — TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct fp64 CPU implementation (NumPy) of what the
GPU hot path computes. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it. The product path (the HIP
library and its Python binding) never imports, links or executes anything in
this package, and this package imports nothing from the product path.

Sources (the pages' text, cited by page title and section):

* "02 — Multi-Latent Attention (MLA)" (lynx-cortex course notes), sections
  "Multi-head attention estándar", "La compresión de MLA", "Truco de
  codificación posicional", "Coste de memoria", "Coste de cómputo",
  "Lo que MLA no es".
* "Multi-head Latent Attention (MLA) și arhitectura DeepSeekMoE" (dexblog),
  opening paragraph and "Exemplul 1" / "Exemplul 2".
* "DeepSeek MLA" (llm-engineer card), sections on the content/positional
  score split and on decode reading the KV cache.
* "Atención latente de múltiples cabezas" (aiunderstanding), "Información
  técnica" (absorption of the up-projections into query and output sides).

Modules:

* :mod:`oracle.codecs`     storage codecs (fp32, bf16, OCP fp8 e4m3fn) decoded
                           exactly to fp64 and encoded with round-to-nearest-even.
* :mod:`oracle.rope`       rotary position embedding, interleaved pairs.
* :mod:`oracle.mla`        append (down-projection + RoPE + storage rounding),
                           non-absorbed decode (the definition), absorbed decode
                           (self-check), log-sum-exp merge of split partials.
* :mod:`oracle.cache_size` the pages' per-token cache-size closed forms.
* :mod:`oracle.merged`     precomputed absorbed weights (W_UK^T W_Q per head,
                           W_O W_UV) and the decode that consumes them.

Every function is pinned by ``tests/test_oracle_*.py`` against something other
than itself (brute force, a library routine, closed forms, printed values).
Parity unpinned: none of the functions here; the pages' 93.3 %, "~1/4 HBM",
"1/8 SSD" and "~5 % parameters" figures are not functions of this package.
"""

from . import codecs, rope, mla, cache_size, merged  # noqa: F401
