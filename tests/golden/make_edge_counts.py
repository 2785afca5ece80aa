"""Writes tests/golden/edge_counts.json: per-KV-head visible (row, key) counts counted by
the oracle's element-wise mask (oracle.edge_counts) at the 1024-, 4096- and 32768-token
shapes of the workloads (windows: sink/near as given, gap 0, bands of width
ceil((L - near) / Hkv); modes complementary / duplicated / dense).

Run from the repository root:  python tests/golden/make_edge_counts.py
"""
import json
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
import oracle  # noqa: E402

CASES = [
    # (Lq, Lk, Hkv, sink, near)
    (1024, 1024, 2, 64, 128),
    (4096, 4096, 8, 128, 512),
    (32768, 32768, 8, 128, 2048),
]


def main():
    out = {"source": "oracle.edge_counts (element-wise mask), written by make_edge_counts.py",
           "cases": []}
    for Lq, Lk, Hkv, sink, near in CASES:
        for mode in oracle.MODES:
            win = oracle.Window.for_length(Lk, Hkv, sink, near, 0, mode=mode)
            per_head = oracle.edge_counts(Lq, Lk, Hkv, win, row_chunk=512)
            out["cases"].append(dict(Lq=Lq, Lk=Lk, Hkv=Hkv, sink=sink, near=near, gap=0,
                                     lr=win.lr, mode=mode, per_head=per_head))
            print(Lq, mode, per_head, sum(per_head), flush=True)
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "edge_counts.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
