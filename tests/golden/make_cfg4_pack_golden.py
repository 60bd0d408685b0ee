#!/usr/bin/env python3
"""Write cfg4_pack_sha256.txt: the oracle's packed FP8 weights of the whole
28-layer, 7-projection 7B-class sweep (196 weights), one line per weight.

Calls only ``oracle/`` (the packing) and ``workloads/`` (the seeded block
generators); nothing from the HIP path.  Each line holds the layer, the
projection, the GGML type id, n, k, the SHA-256 of the n*k E4M3 codes
(row-major bytes), and the fp32 bit patterns of the weight's absmax and of
its dequantisation scale RN(absmax'/448), as the oracle computes them from
the pages' steps (gemm.rs page, get_or_cache_fp8_weight).

Usage:  python tests/golden/make_cfg4_pack_golden.py [--jobs J]
(about 30 s of CPU per layer and 4 GB of memory per job).
"""
from __future__ import annotations

import argparse
import hashlib
import os
import sys
from concurrent.futures import ProcessPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "cfg4_pack_sha256.txt")
ORDER = ("q", "k", "v", "o", "gate", "up", "down")


def layer_lines(layer: int) -> list[str]:
    import workloads as W
    from oracle import fp8_path

    gemms = {gm.name: gm for grp in W.config_groups(4, layer=layer) for gm in grp.gemms}
    lines = []
    for name in ORDER:
        gm = gemms[name]
        blocks = W.weight_blocks(gm.qtype, gm.w_seed, gm.n, gm.k)
        w8, dq, a = fp8_path.pack_weight(gm.qtype, blocks, gm.n, gm.k)
        digest = hashlib.sha256(np.ascontiguousarray(w8).tobytes()).hexdigest()
        a_bits = int(np.array([a], np.float32).view(np.uint32)[0])
        dq_bits = int(np.array([dq], np.float32).view(np.uint32)[0])
        lines.append(f"{layer} {name} {gm.qtype} {gm.n} {gm.k} {digest} {a_bits:08x} {dq_bits:08x}")
    return lines


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    args = ap.parse_args()
    import workloads as W

    with ProcessPoolExecutor(max_workers=args.jobs) as ex:
        per_layer = list(ex.map(layer_lines, range(W.CFG4_LAYERS)))
    with open(OUT, "w") as fh:
        fh.write("# Oracle-packed FP8 weights of the 28-layer sweep (M=4096 configuration), written by\n")
        fh.write("# make_cfg4_pack_golden.py from oracle/ and the seeded generators in workloads/ only.\n")
        fh.write("# layer proj qtype n k sha256(codes) absmax_bits dq_bits\n")
        for lines in per_layer:
            for ln in lines:
                fh.write(ln + "\n")
    print(OUT)
    return 0


if __name__ == "__main__":
    sys.exit(main())
