"""fp64 CPU oracle for the routed-expert MoE forward over 4-bit codebook experts.

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg
may import it. The GPU library never imports it, and it imports nothing from the library.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import dequant_f64_exact, layer_forward  # noqa: F401
