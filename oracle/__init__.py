"""fp64 CPU oracle of MLA decode.  Test infrastructure only: imported by tests/,
__graft_entry__.smoke() and bench.py's cpu_baseline leg, never by the product."""
from .mla_oracle import (absorbed_decode_seq, bf16_to_f64, cache_rows_from_hidden,  # noqa: F401
                         causal_prefill_seq, causal_prefill_workload,
                         decode_workload, gather_rows, lse_merge, multi_decode_seq,
                         multi_decode_workload, naive_decode_seq,
                         query_from_hidden, query_from_latent, rope, rope_matrix, rope_theta, softmax_scale,
                         to_f64)
