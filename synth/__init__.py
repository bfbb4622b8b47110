"""Seeded synthetic inputs shared by the oracle tests and the GPU path.

Holds workload shapes and the random recipe only; no part of the scoring,
selection or compaction arithmetic lives here.
"""
from .configs import (ALL, BY_NAME, GEMMA12B_16K, LLAMA8B_128K, LLAMA8B_8K,
                      QWEN14B_32K, TINY, Workload)
from .generate import (bf16_bits_to_f32, chunk_rows, default_workers,
                       f64_to_bf16_bits, generate_chunked_head,
                       generate_chunked_workload, generate_head,
                       generate_workload)
from .epikv import (EPI_ALL, EPI_BY_NAME, EPIKV_R1_8B_64K, EPIKV_TINY, EpiWorkload,
                    generate_hidden, generate_hidden_layer, generate_kv)
from .routing import nearest_position_routes
from .extreme import PROFILES as EXTREME_PROFILES, generate_extreme_workload
