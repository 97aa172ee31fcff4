"""Float64 CPU oracle (test infrastructure only; see oracle.py)."""
from .oracle import *  # noqa: F401,F403
from .oracle import (E2M1_TABLE, E4M3_TABLE, E8M0_TABLE, Problem, attend, bf16_to_f64, decode,  # noqa: F401
                     decode_partials, default_scale, dequant, merge, q_to_f64, slab_kv, split_ranges)
from . import cache  # noqa: F401,E402
from . import passq  # noqa: F401,E402
