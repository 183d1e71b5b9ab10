"""Write exhaustive_digests.txt: SHA-256 digests of the CPU oracle's codes
and scales over the whole (x, amax) bf16 domain (1,065,402,238 pairs), in
the chunk layout of synth.exhaustive_*_chunk, for both quantizers with fp32
scales (kinds act, weight) and with E8M0 scales (act_ue8m0, weight_ue8m0).
Calls only oracle/ and the input generator; the GPU tests compare the
kernels' outputs chunk by chunk.  Lines of kinds not regenerated are kept.

    python tests/golden/make_exhaustive_digests.py [--procs 4] [--kinds act,weight,...]
"""
import argparse
import hashlib
import os
import sys
from multiprocessing import Pool

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from oracle import quant, ue8m0  # noqa: E402

NCHUNKS = 16
KINDS = ("act", "weight", "act_ue8m0", "weight_ue8m0")
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
    elif kind == "weight":
        q, s = quant.weight_block_quant(synth.exhaustive_weight_chunk(lo, hi))
    elif kind == "act_ue8m0":
        q, s = ue8m0.act_quant_group_ue8m0(synth.exhaustive_act_chunk(lo, hi))
    else:
        q, s = ue8m0.weight_block_quant_ue8m0(synth.exhaustive_weight_chunk(lo, hi))
    return f"{kind} {c} {lo:#06x} {hi:#06x} {digest(q, s)}"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--procs", type=int, default=4)
    ap.add_argument("--kinds", default=",".join(KINDS))
    a = ap.parse_args()
    kinds = a.kinds.split(",")
    assert all(k in KINDS for k in kinds), kinds
    jobs = [(k, c, lo, hi) for k in kinds
            for c, (lo, hi) in enumerate(synth.exhaustive_chunk_bounds(NCHUNKS))]
    kept = []
    if os.path.exists(OUT):
        kept = [ln.rstrip("\n") for ln in open(OUT)
                if ln.strip() and not ln.startswith("#") and ln.split()[0] not in kinds]
    with Pool(a.procs) as p:
        lines = p.map(work, jobs)
    order = {k: i for i, k in enumerate(KINDS)}
    lines = sorted(kept + lines, key=lambda ln: (order[ln.split()[0]], int(ln.split()[1])))
    with open(OUT, "w") as f:
        f.write("# kind chunk amax_lo amax_hi sha256(codes || scales)  -- written by "
                "make_exhaustive_digests.py from the CPU oracle\n")
        f.write("\n".join(lines) + "\n")
    print(OUT)


if __name__ == "__main__":
    main()
