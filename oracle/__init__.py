"""CPU oracle for the RaggedShard flat-buffer hot path.

TEST INFRASTRUCTURE ONLY.  Plain, slow, obviously correct definitions of
what the planner and the grouped buffer operations compute, written from the
pages (veScale-FSDP: Flexible and High-Performance FSDP at Scale; PyTorch
FSDP: Experiences on Scaling Fully Sharded Data Parallel; veScale 深度技术分析).
Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg may
import it.  It shares no code with the HIP path; both take inputs from the
seeded generators in workloads.py.
"""
from . import casts, ops, plan  # noqa: F401
from . import optim  # noqa: F401,E402
