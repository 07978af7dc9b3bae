"""CPU oracle for the paged-KV attention path -- test infrastructure only.

Imported only by the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``; the product library never uses it.
"""

from .paged_kv import (  # noqa: F401
    bf16_bits_to_float,
    float_to_bf16_bits,
    gather_kv,
    paged_attention,
    paged_attention_blocked,
    paged_decode,
    store_kv,
    token_slots,
)
from .alloc import alloc_pages  # noqa: F401
from .rope import f64_to_bf16_bits, rope, rope_f64, rope_store_kv, rope_table  # noqa: F401
