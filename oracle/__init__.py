"""fp64 CPU oracle for attention-guided KV eviction and paged compaction.

Test infrastructure only: imported by tests/, by __graft_entry__.smoke() and by
the CPU-baseline leg of bench.py, never by the product library.
"""
from .kvs_oracle import (  # noqa: F401
    PAGE, bf16_bits_to_f64, slot_location, gather_stream_rows, observer_rows,
    score_stream, score, fixed_point_mass, mass_cut, lrfu_decay, fma_f32, lrfu_update,
    select_top_b, ratchet, RATCHET_INITIAL, RATCHET_NUM, RATCHET_DEN, RATCHET_CAP,
    plan_stream, plan_sequence, compact_stream, eviction_round, round_fraction_to_f32,
)
from . import confidence_oracle as confidence  # noqa: F401
from . import decode_oracle as decode  # noqa: F401
from . import stepkv_oracle as stepkv  # noqa: F401
from . import kmeans_oracle as kmeans  # noqa: F401
