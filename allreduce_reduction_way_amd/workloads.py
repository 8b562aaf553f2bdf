"""The named workloads the library is measured and checked on.

Shapes come from the pages: 440x5120, 512x7168 and 680x5120 are the bf16
allreduce shapes of aiter PR #1910 "optimize allreduce write mode by
broadcast output ptr" (Test Result tables); 4096 elements is the smallest
one-shot size of Helion PR #245 "One shot all reduce Example" (benchmark
table, "(4k)").  The 64 Mi-element, 4-rank two-shot case is the large-message
end where the share is purely HBM-bound.
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    op: str            # oneshot_sum | write_bcast | packet_fused | twoshot_share
    P: int
    n: int
    dist: str          # uniform | normal
    ranks: tuple = (0,)  # two-shot owners run in this order; packet path: all ranks
    calls: int = 1     # packet path: consecutive calls, flag = call + 1, seed = call
    note: str = field(default="", compare=False)


ONESHOT_4K = Workload("oneshot_4096_p8", "oneshot_sum", 8, 4096, "uniform")
WRITE_BCAST_440x5120 = Workload("write_bcast_440x5120_p8", "write_bcast", 8, 440 * 5120, "uniform")
PACKET_512x7168 = Workload("packet_fused_512x7168_p8", "packet_fused", 8, 512 * 7168, "uniform",
                           ranks=tuple(range(8)), calls=3)
TWOSHOT_680x5120_R3 = Workload("twoshot_680x5120_p8_rank3", "twoshot_share", 8, 680 * 5120,
                               "uniform", ranks=(3,))
TWOSHOT_64Mi_P4 = Workload("twoshot_64Mi_p4_all_owners", "twoshot_share", 4, 64 * 1024 * 1024,
                           "normal", ranks=(0, 1, 2, 3))

# Widened rows: the unfused three-operation packet decomposition, the fused
# packet kernel with its flag on the device replayed from a HIP graph, and the
# one-shot reduce-scatter sibling (rank 3's block of 440x5120 x 8).
PACKET_3OP_512x7168 = Workload("packet_3op_512x7168_p8", "packet_3op", 8, 512 * 7168, "uniform",
                               ranks=tuple(range(8)), calls=3)
PACKET_EPOCH_GRAPH_512x7168 = Workload("packet_epoch_graph_512x7168_p8", "packet_epoch", 8,
                                       512 * 7168, "uniform", ranks=tuple(range(8)), calls=3)
REDUCE_SCATTER_440x5120_R3 = Workload("reduce_scatter_440x5120_p8_rank3", "reduce_scatter", 8,
                                      440 * 5120, "uniform", ranks=(3,))

# One rank's share of the packet path on its own: rank 3 of 8 against peer
# packets already in place; and the LL codec alone on one rank's 512x7168.
PACKET_RANK3_512x7168 = Workload("packet_rank3_share_512x7168_p8", "packet_rank", 8, 512 * 7168,
                                 "uniform", ranks=(3,))
LL_ENCODE_512x7168 = Workload("ll_encode_512x7168", "ll_encode", 1, 512 * 7168, "uniform")
LL_DECODE_512x7168 = Workload("ll_decode_512x7168", "ll_decode", 1, 512 * 7168, "uniform")

ALL = (ONESHOT_4K, WRITE_BCAST_440x5120, PACKET_512x7168, TWOSHOT_680x5120_R3, TWOSHOT_64Mi_P4,
       PACKET_3OP_512x7168, PACKET_EPOCH_GRAPH_512x7168, REDUCE_SCATTER_440x5120_R3,
       PACKET_RANK3_512x7168, LL_ENCODE_512x7168, LL_DECODE_512x7168)
BY_NAME = {w.name: w for w in ALL}
