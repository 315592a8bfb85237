"""Plain CPU oracle of the DeepSeek Sparse Attention (DSA) forward path.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import or run anything in this package. The GPU library neither imports nor links it, and it
shares no code with the GPU library (no kernels, tables, headers or helpers).

What it computes (DeepSeek-V3.2 paper digest, "Key claims", paper section 2.1, Eq. 1-2, and
"Method"): for each query token t and each preceding key s (s <= t),

    I[t, s] = sum_j w[t, j] * ReLU(qI[t, j] . kI[s]),

the top-k keys of I[t, :] are selected, and every one of the H query heads of token t attends
(softmax) only to the selected rows of one latent vector per key that is shared by all heads
(MLA in MQA mode). Everything is evaluated in float64 after decoding the stored FP8 / bf16 /
fp32 inputs with the oracle's own tables.

Modules:
  numerics  decoding of OCP FP8 e4m3fn codes and bf16 bit patterns (own tables)
  dsa       the vectorised float64 oracle (indexer, top-k, attention, composition, and the
            indexer-alignment target with its KL divergence)
  brute     pure-Python loop versions for tiny inputs (cross-check of `dsa`)
"""
from .numerics import decode, fp8_e4m3fn_table, bf16_bits_to_f64  # noqa: F401
from .dsa import (Seqs, indexer_scores_row, indexer_scores, topk_row, topk, attn_row,  # noqa: F401
                  sparse_mla_attn, forward_rows, alignment_row)
