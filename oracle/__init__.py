"""Float64 CPU oracle for TurboQuant KV encode and compressed decode attention.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import or run anything in this package.  The
product path (the HIP library and its Python binding) never imports it, and this
package imports nothing from the product path: the two share no code.  Inputs
come from the seeded generators in ``compressed_kv_decode_tq_amd.workloads``,
which hold no arithmetic of the method.

The oracle is deliberately plain: numpy/scipy in float64, one step after the
other in the order the pages give them, no blocking or fusion.  Sources, cited
in every function by page title and section:

* [audit]  page "turboquant/audit_claims.py" (git.saillant.cc, electron-rare/
  turboquant): the store/quantizer API, the byte accounting (AUDIT 1), the
  dequantize-then-attend decode (AUDIT 2, AUDIT 4), the distortion bound
  (AUDIT 5) and the unbiasedness check (AUDIT 6).
* [explainer]  page "TurboQuant — Random rotation trước khi quantize, 3-bit KV
  cache không mất accuracy" (troisinh.com): sections "Ý tưởng cốt lõi" (core
  idea: fixed random rotation, one MSE-optimal scalar quantizer for every
  coordinate, 1-bit QJL residual) and "Tại sao nó hoạt động" (why it works,
  with the pseudo-code: rotate the query at run time).
* [results]  page "03. Results & Benchmarks" (devtechjr turboquant_cutile):
  sections "Compression" (3-bit K and V, 5.02x) and "Latency Benchmarks"
  (one fused pass: scores, QJL correction, online softmax, V accumulation).

Every function is pinned by ``tests/test_oracle_*.py`` against something other
than itself (closed forms, textbook special cases, brute force, Monte Carlo,
the pages' printed byte counts).  Where the pages leave a step open, the
function that takes it states the reading it follows.
"""
from .codebook import Codebook, lloyd_max, coord_density, coord_cdf  # noqa: F401
from .quantize import (  # noqa: F401
    KeyCode, ValueMinMax, ValueMSE,
    encode_keys, encode_values_minmax, encode_values_mse,
    dequantize_keys, dequantize_values_minmax, dequantize_values_mse,
    score_estimate, round_scalar, half_bit_coordinates,
)
from .attention import decode_attention, decode_attention_bruteforce, decode_attention_multi  # noqa: F401
from .layout import (  # noqa: F401
    Layout, pack_key_planes, unpack_key_planes, pack_value_planes, unpack_value_planes,
    pack_value_codes, unpack_value_codes, pack_value_words, unpack_value_words, value_words_packed,
    memory_bytes, bytes_per_token_head, half_plane_position,
    key_record_planes, key_block_positions, key_records_to_blocks, key_blocks_to_records,
)
