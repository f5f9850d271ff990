"""CPU oracle for the ReduceScatter + AllGather AllReduce over N virtual ranks.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
statement of what the collectives compute, used to check the HIP library.
Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  The product path (``collective_reduction_amd``)
never imports, links or runs anything here, and this package imports nothing
from the product: the two share no code.  Inputs reach the oracle as NumPy
arrays; the seeded generators that produce them hold none of the method's
arithmetic.

Pages cited throughout (the oracle restates their definitions; it copies no
listing):

* [DECOMP]  "NCCL 专家课程 07：AllReduce 等价分解、显存生命周期与 Kernel 证据"
  (blog.cptz.space, nccl-collective-decomposition).
* [WHY-EQ]  "为什么说 AllReduce = ReduceScatter + AllGather？——结合 NCCL Ring
  AllReduce" (loosp.cn).
* [RING]    "Ring AllReduce 核心流程：梯度是怎么聚合的" (llmnex.top).
* [RS-PAGE] "ReduceScatter" (tier6-model.pages.dev, 集合通信).
* [PRIMS]   "通信与互联（01）：集合通信原语与代价模型——α-β 模型与 ring
  all-reduce" (arganzheng.life).

Modules
-------
``reduction``   identity elements, the combine operator ⊕ per dtype, bf16
                rounding (round-to-nearest-even) and the fp64 reference.
``collectives`` direct AllReduce, rank-major ReduceScatter, source-ordered
                AllGather, identity padding and trim (NumPy, vectorised over
                elements, explicit loops over ranks).
``ring``        the ring schedule stepped literally rank by rank, with its
                routing table and per-step state.
``scalar``      a pure-Python scalar twin of the above for tiny inputs.
``recursive``   recursive-halving ReduceScatter and recursive-doubling
                AllGather (N a power of two), stepped rank by rank.

Every function is pinned by ``tests/test_oracle_*.py`` against values the
pages print, closed forms, brute force and invariants; nothing here is
"parity unpinned".
"""

from . import reduction, collectives, ring, scalar, recursive  # noqa: F401

__all__ = ["reduction", "collectives", "ring", "scalar", "recursive"]
