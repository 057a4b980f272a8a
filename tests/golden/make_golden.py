"""Writes the stored expected values under tests/golden that come from the oracle.

Calls only ``oracle`` (and the seeded input generators); nothing here touches
the HIP library.  Run: ``python tests/golden/make_golden.py``.
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from ulysses_inputs import WORKLOADS, make_inputs, seq_shards  # noqa: E402


def segments_packed():
    case = WORKLOADS[3]
    inp = make_inputs(case, with_dout=False)
    cu, n, mx = oracle.segments(oracle.gather_positions(seq_shards(inp.positions, case.P)))
    return {
        "source": ("cu_seqlens / max_len rebuilt by the oracle from the gathered position_ids of "
                   "the packed workload (S=32768, P=4 contiguous shards, document lengths uniform "
                   "in [512, 8192] drawn from seed 3, last one cut to fit); rebuild rule from the "
                   "accelerate PR 'Add an FSDP2-native Ulysses sequence parallelism backend', "
                   "comment on the flash-attention kwargs"),
        "doc_lengths": inp.doc_lengths,
        "cu_seqlens": cu.tolist(),
        "n_seqs": n,
        "max_len": mx,
    }


if __name__ == "__main__":
    with open(os.path.join(HERE, "segments_packed_s32768.json"), "w") as f:
        json.dump(segments_packed(), f, indent=1)
        f.write("\n")
