"""CPU oracle for jagged flash attention (float64 NumPy).

TEST INFRASTRUCTURE ONLY. The tests, the smoke check and the benchmark's
CPU-baseline leg may import it; the library (variable_length_flash_jaggedfa_amd)
never imports, links or runs anything in here, and the oracle imports nothing
from the library. The two share only the seeded input generator (jfa_inputs),
which holds no attention arithmetic.

  attention.py     exact softmax attention and its gradients, per sequence
  schedule_ref.py  the KV-work-sorted zigzag tile deal, in plain integers
  rotary.py        block-diagonal attention of rotary-embedded queries and keys
  pool.py          the oracle over a whole workload in worker processes (sub-batches of
                   sequences; comparison with stored results)
"""
from . import attention, rotary, schedule_ref  # noqa: F401
