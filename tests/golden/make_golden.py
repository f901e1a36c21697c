"""Writes tests/golden/brute_tiny.json: 40-digit reference outputs for tiny cases.

The values come only from ``oracle.brute`` (decimal arithmetic) over inputs drawn
by ``synth``; the pages print no worked numeric example for this method, so the
fixture pins the C oracle to an independent high-precision evaluation of the same
definition.  Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from oracle import brute  # noqa: E402

CASES = [
    (synth.Case(2, 4, 2, 4, 2, 6, priv_len=1, dtype="bf16", name="decode bf16 with suffix"), 21,
     dict(b_sigma=0.5)),
    (synth.Case(2, 2, 2, 4, 2, 5, page_size=2, n_phys_pages=4, dtype="f32", name="paged f32"), 22,
     dict(b_sigma=0.5, q_scale=2.0)),
    (synth.Case(3, 2, 1, 3, 2, 4, priv_len=2, q_len=2, mode="prefill", shared_lr=True, dtype="bf16",
                name="causal chunk, shared low-rank"), 23, dict(b_sigma=0.5)),
]


def main():
    out = []
    for case, seed, kw in CASES:
        x = synth.make_inputs(case, seed, **kw)
        o, l = brute.attend(case, x)
        flat_o = [str(v) for a in o for t in a for h in t for v in h]
        flat_l = [str(v) for a in l for t in a for v in t]
        fields = {k: getattr(case, k) for k in case.__dataclass_fields__}
        out.append(dict(case=fields, seed=seed, kwargs=kw, out=flat_o, lse=flat_l))
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "brute_tiny.json")
    with open(path, "w") as f:
        json.dump(dict(source="oracle.brute (decimal, 40 digits)", cases=out), f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
