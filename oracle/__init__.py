"""Float64 CPU oracle - TEST INFRASTRUCTURE ONLY.

Imported by the tests, the smoke check and the benchmark's CPU-baseline leg,
never by the library.  It shares no code with the GPU kernels; see
oracle.kvzip for the definitions it follows and oracle.brute for the scalar
brute force that pins it; oracle.epikv holds the attention-free EpiKV token
score and oracle.selkv the SelKV soft cosine gate.
"""
from .kvzip import (attention_rows, bf16_to_f64, chunk_bounds,
                    chunked_head_scores, compact, head_level_scores,
                    head_scores, head_scores_parallel, keep_count, row_lse, select,
                    topk_ascending, visible_keys, workload_head_inputs)
from . import epikv
from . import selkv
