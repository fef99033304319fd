"""CPU oracle of the TurboQuant KV-cache path (TEST INFRASTRUCTURE ONLY).

This package is a plain, slow, float64 reference written from the public
descriptions of the method. It exists to check the GPU library. Only the
test suite (``tests/``), the smoke check in ``__graft_entry__`` and the
``cpu_baseline`` leg of ``bench.py`` may import it. The product path
(``kv_cache_vector_rotation_amd``) never imports, calls or links it, and
the oracle never imports the product path: they share no code. Their only
common dependency is the seeded input generator module ``synth``.

Sources, cited by title and section (the pages are web articles):

[ZB]  zubnet.ai news, "Google's TurboQuant quantizes LLM KV cache 3.5 bits
      per channel, near ..." (Spanish, Portuguese and French editions of
      one article), paragraph 2: a random rotation makes each coordinate
      follow a Beta law, an optimal per-coordinate scalar quantizer is then
      applied (stage one); an MSE quantizer followed by a 1-bit quantized
      Johnson-Lindenstrauss transform of the residual (stage two); the
      per-token storage is quantization indices, sign bits and an L2 norm;
      3.5 and 2.5 bits per channel are named.
[WD]  winningdata.io blog, "TurboQuant: Google comprime KV cache para 3 bits
      sem perder acuracia ...", sections "Como o TurboQuant funciona"
      (sub-sections "1. PolarQuant": multiply by a random orthogonal matrix,
      then quantize; "2. QJL Residual": one extra bit per value removes the
      inner-product bias; distortion within a constant factor of the
      Shannon bound), "Os numeros que importam" (memory/speed table) and
      "O problema" (KV-cache sizing example).
[UB]  usedby.ai blog, "TurboQuant: Compresion de KV Cache a 3 bits y
      aceleracion de inferencia en H100", section "Bajo el capo" (two
      stages, the second being a 1-bit QJL correction).

Where the pages are silent the oracle takes a stated reading; each reading
is stated in the module header and cited in the function that relies on
it.

Pins: every public function here is checked by ``tests/test_oracle_*.py``
against closed forms, textbook limits, invariants, statistics or brute
force, never against the GPU library.
"""
from .codebook import (
    coordinate_pdf, coordinate_cdf, coordinate_ppf, cell_first_moment,
    lloyd_max, Codebook,
)
from .quantize import Quantizer, QuantizedVectors, quantize, legal_variants
from .estimate import dequantize, estimate_logits, attention_decode, attention_prefill, softmax
from .records import (
    pack_token_major, pack_block32, record_words, record_bytes,
)
from .search import top_k, estimated_scores, search, exact_search, recall_at_k

__all__ = [
    "coordinate_pdf", "coordinate_cdf", "coordinate_ppf", "cell_first_moment",
    "lloyd_max", "Codebook",
    "Quantizer", "QuantizedVectors", "quantize", "legal_variants",
    "dequantize", "estimate_logits", "attention_decode", "attention_prefill", "softmax",
    "pack_token_major", "pack_block32", "record_words", "record_bytes",
    "top_k", "estimated_scores", "search", "exact_search", "recall_at_k",
]
