"""CPU oracle for the SwiftKV prefill -- test infrastructure, not product code.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package.  It shares no code with the HIP library and never calls
it.  See swiftkv_oracle.py for the computation and its citations.
"""
from .swiftkv_oracle import *  # noqa: F401,F403
from .swiftkv_oracle import (Dims, DictWeights, LazyWeights, OracleResult, swiftkv_prefill,  # noqa: F401
                             standard_incremental_decode, prefill_flops, per_token_breakdown, kv_slots,
                             kv_memory_fraction, slot_of_layer, representative, n_groups)
