"""Write exhaustive_digests.txt: SHA-256 digests of the CPU oracle's codes
and scales over the whole (x, amax) bf16 domain (1,065,402,238 pairs), in
the chunk layout of synth.exhaustive_*_chunk.  Calls only oracle/ and the
input generator; the GPU tests compare the kernels' outputs chunk by chunk.

    python tests/golden/make_exhaustive_digests.py [--procs 8]
"""
import argparse
import hashlib
import os
import sys
from multiprocessing import Pool

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from oracle import quant  # noqa: E402

NCHUNKS = 16
OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "exhaustive_digests.txt")


def digest(q, s):
    h = hashlib.sha256()
    h.update(q.tobytes())
    h.update(s.tobytes())
    return h.hexdigest()


def work(job):
    kind, c, lo, hi = job
    if kind == "act":
        q, s = quant.act_quant_group(synth.exhaustive_act_chunk(lo, hi))
    else:
        q, s = quant.weight_block_quant(synth.exhaustive_weight_chunk(lo, hi))
    return f"{kind} {c} {lo:#06x} {hi:#06x} {digest(q, s)}"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--procs", type=int, default=8)
    a = ap.parse_args()
    jobs = [(k, c, lo, hi) for k in ("act", "weight")
            for c, (lo, hi) in enumerate(synth.exhaustive_chunk_bounds(NCHUNKS))]
    with Pool(a.procs) as p:
        lines = p.map(work, jobs)
    with open(OUT, "w") as f:
        f.write("# kind chunk amax_lo amax_hi sha256(codes || scales)  -- written by "
                "make_exhaustive_digests.py from the CPU oracle\n")
        f.write("\n".join(lines) + "\n")
    print(OUT)


if __name__ == "__main__":
    main()
