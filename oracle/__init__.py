"""Plain, slow fp64 CPU oracle for the TurboQuant encode and compressed-key score path.

This package is TEST INFRASTRUCTURE. Only the test suite, the package smoke check
(``__graft_entry__.smoke``) and the ``cpu_baseline`` leg of ``bench.py`` may import it.
The product path (the HIP library and its Python binding) never imports, links or runs
anything here, and nothing here imports the product.

Every step follows the method as the source pages state it, in their order and notation,
computed in float64 with numpy (a library QR, sort or matmul serves as a single step where
one is used).  Pages cited in docstrings:

* "TurboQuant 详解" (wnma3mz blog) -- the tutorial with the worked examples,
  TurboQuant_mse / TurboQuant_prod and the KV prefill/decode flow.
* "TurboQuant first-principles walkthrough" (blog.hotdry.top) -- coordinate density,
  centroids, distortion bound, 2/pi shrinkage, QJL constant.
* "TurboQuant 和 RotorQuant 的真相" (zhichai.net) -- community kernels, attention formula,
  MSE-only vs QJL.
* "Sub-byte KV cache quantization with TurboQuant" (blog2.hotdry.top) -- codebook recipe,
  fused score kernel, GQA head mapping, deployment checklist.

Parity status of each function is stated in its module header.  Functions whose exact
values no page fixes (the seeded generator streams and the randomized Hadamard sign draw)
are marked "parity unpinned"; they are pinned only by structural and statistical checks.
"""

from .rng import splitmix64, uniform53, gaussian, rademacher
from .rotation import (dense_rotation, wht_rotation, block_wht_rotation, sylvester_hadamard,
                       rotation_from_matrix)
from .codebook import (Codebook, lloyd_max_points, coordinate_weights, codebook,
                       codebook_from_values)
from .quantizer import (nearest_index, pack_bits, unpack_bits, pack_token_blocked,
                        unpack_token_blocked, encode_mse, decode_mse,
                        encode_prod, decode_prod, qjl_matrix, qjl_encode, qjl_correction, scores_mse, scores_prod,
                        quantize_rotated, EncodedMSE, EncodedProd, QJL_CONST)
from .attention import decode_attention, prefill_attention, topk
from .kv_cache import (cache_rows, append_rows_mse, append_rows_prod, assign_token_blocked,
                       append_token_blocked_mse, live_rows)
from .split import (channel_order, encode_split, decode_split, scores_split, decode_attention_split,
                    EncodedSplit)
from .outlier8 import (int8_absmax, rest_mask, encode_outlier8, decode_outlier8, scores_outlier8,
                       decode_attention_outlier8, EncodedOutlier8)

__all__ = [
    "int8_absmax", "rest_mask", "encode_outlier8", "decode_outlier8", "scores_outlier8", "EncodedOutlier8",
    "decode_attention_outlier8",
    "channel_order", "encode_split", "decode_split", "scores_split", "decode_attention_split", "EncodedSplit",
    "splitmix64", "uniform53", "gaussian", "rademacher",
    "dense_rotation", "wht_rotation", "block_wht_rotation", "sylvester_hadamard", "rotation_from_matrix",
    "Codebook", "lloyd_max_points", "coordinate_weights", "codebook", "codebook_from_values",
    "nearest_index", "pack_bits", "unpack_bits", "pack_token_blocked", "unpack_token_blocked", "encode_mse", "decode_mse", "encode_prod",
    "decode_prod", "qjl_matrix", "qjl_encode", "qjl_correction", "scores_mse", "scores_prod", "quantize_rotated",
    "EncodedMSE", "EncodedProd", "QJL_CONST",
    "decode_attention", "prefill_attention", "topk",
    "cache_rows", "append_rows_mse", "append_rows_prod", "assign_token_blocked",
    "append_token_blocked_mse", "live_rows",
]
