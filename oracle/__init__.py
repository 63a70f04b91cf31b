"""CPU oracle for the segmented multi-LoRA linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP path (the only common module is the seeded input generator in
``workloads``, which holds none of the method's arithmetic).

Every function is pinned by CPU tests against facts the pages or the
mathematics fix (printed metadata examples, the merged closed form,
base-only reductions, invariants, exact small-integer cases, fingerprint
adapters); see ``tests/test_oracle_pins.py``.
"""
from .lora_oracle import (  # noqa: F401
    decode,
    validate_rows,
    segment_metadata,
    lora_forward,
    gather_bmm_forward,
    per_adapter_forward,
    merged_forward,
    stacked_forward,
    decode_fp8_e4m3,
    lora_forward_fp8w,
    dora_column_scale,
    dora_forward,
    dora_factored_forward,
    lora_param_count,
    full_param_count,
)
