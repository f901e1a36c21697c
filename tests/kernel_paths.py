"""One small workload per kernel instantiation of librattn that a call can run.

Each entry names the instantiation (as ``shared_base_residual_amd.kernel_of``
reports it from the library's own planner) and a shape that reaches it, with
a ragged prefix (several 16-token groups, a partial last tile) and, for
decode, a ragged private suffix.  ``tests/test_kernel_paths.py`` checks on the
host that every shape still lands on its instantiation and that together they
cover every instantiation the library builds; ``tests/test_gpu_parity.py``
runs each one against the oracle.
"""
import synth

C = synth.Case


def _dec(N, HQ, HK, D, r, L, S=37, ql=1, dtype="bf16", shared=False, name=""):
    return C(N, HQ, HK, D, r, L, priv_len=S, q_len=ql, dtype=dtype, shared_lr=shared, name=name)


def _pre(N, HQ, HK, D, r, L, S, dtype="bf16", shared=False, ps=0, nphys=0, name=""):
    return C(N, HQ, HK, D, r, L, priv_len=S, q_len=S, dtype=dtype, shared_lr=shared, page_size=ps,
             n_phys_pages=nphys, mode="prefill", name=name)


# (instantiation, workload)
PATHS = [
    # prefill kernel: (dtype, d, residual columns); 256-row workgroups at d = 128
    # with r <= 32 (two 256-row blocks per (agent, head) with q_len * g = 512),
    # 128-row ones for wider residuals
    (("prefill", "bf16", 128, 0), _pre(2, 8, 2, 128, 0, 0, 130, name="prefill d128 r0 private only, 2 q-blocks")),
    (("prefill", "bf16", 128, 0), _pre(1, 8, 2, 128, 0, 700, 90, name="prefill d128 r0 with prefix, 2 q-blocks")),
    (("prefill", "bf16", 128, 32), _pre(2, 16, 4, 128, 16, 1000, 128, name="prefill d128 r16, 2 q-blocks")),
    (("prefill", "bf16", 128, 64), _pre(2, 8, 2, 128, 64, 1000, 70, name="prefill d128 r64, 128-row blocks")),
    (("prefill", "bf16", 128, 128), _pre(2, 8, 2, 128, 128, 600, 40, name="prefill d128 r128, 128-row blocks")),
    (("prefill", "bf16", 64, 0), _pre(2, 8, 2, 64, 0, 500, 70, name="prefill d64 r0")),
    (("prefill", "bf16", 64, 32), _pre(3, 8, 2, 64, 32, 1000, 90, shared=True, name="prefill d64 shared r32")),
    (("prefill", "bf16", 64, 64), _pre(2, 8, 2, 64, 64, 800, 70, name="prefill d64 r64")),
    (("prefill", "bf16", 64, 128), _pre(2, 8, 2, 64, 128, 600, 40, name="prefill d64 r128, 128-row blocks")),
    # prefill on the split kernel: a paged prefix of more than 2048 pages (bf16), and fp32
    (("split", "bf16", 64, 32, False, True),
     _pre(1, 2, 2, 64, 8, 33000, 20, ps=16, nphys=2070, name="prefill bf16 paged prefix over 2048 pages")),
    (("split", "f32", 128, 32, False, False), _pre(2, 4, 2, 128, 16, 500, 30, dtype="f32",
                                                   name="prefill fp32 d128 r16")),
    # split kernel, bf16: (d, residual columns, masked, twelve-wave form)
    (("split", "bf16", 128, 0, False, False), _dec(2, 4, 2, 128, 0, 1000, name="d128 r0")),
    (("split", "bf16", 128, 0, False, True), _dec(1, 16, 2, 128, 0, 0, 400, ql=3, name="d128 r0 12 waves")),
    (("split", "bf16", 128, 32, False, False), _dec(2, 4, 2, 128, 8, 1000, name="d128 r8")),
    (("split", "bf16", 128, 32, False, True), _dec(5, 4, 1, 128, 8, 1000, name="d128 r8 12 waves")),
    (("split", "bf16", 128, 64, False, False), _dec(1, 2, 2, 128, 64, 1000, name="d128 r64")),
    (("split", "bf16", 128, 128, False, False), _dec(1, 2, 2, 128, 128, 1000, name="d128 r128")),
    (("split", "bf16", 128, 32, True, False), _dec(2, 2, 2, 128, 32, 1000, name="d128 r32 masked")),
    (("split", "bf16", 128, 32, True, True), _dec(5, 4, 1, 128, 32, 1000, name="d128 r32 masked 12 waves")),
    (("split", "bf16", 128, 64, True, False), _dec(2, 2, 2, 128, 64, 1000, name="d128 r64 masked")),
    (("split", "bf16", 128, 128, True, False), _dec(2, 4, 4, 128, 128, 1000, name="d128 r128 masked")),
    (("split", "bf16", 64, 0, False, False), _dec(2, 4, 2, 64, 0, 1000, name="d64 r0")),
    (("split", "bf16", 64, 0, False, True), _dec(1, 16, 2, 64, 0, 0, 400, ql=3, name="d64 r0 12 waves")),
    (("split", "bf16", 64, 32, False, False), _dec(1, 4, 1, 64, 8, 1000, name="d64 r8")),
    (("split", "bf16", 64, 32, False, True), _dec(1, 2, 2, 64, 8, 1000, name="d64 r8 12 waves")),
    (("split", "bf16", 64, 64, False, False), _dec(1, 4, 1, 64, 64, 1000, name="d64 r64")),
    (("split", "bf16", 64, 64, False, True), _dec(1, 2, 2, 64, 64, 1000, name="d64 r64 12 waves")),
    (("split", "bf16", 64, 128, False, False), _dec(1, 2, 2, 64, 128, 1000, name="d64 r128")),
    (("split", "bf16", 64, 32, True, False), _dec(3, 2, 2, 64, 32, 1000, name="d64 r32 masked")),
    (("split", "bf16", 64, 32, True, True), _dec(2, 2, 2, 64, 32, 1000, name="d64 r32 masked 12 waves")),
    (("split", "bf16", 64, 64, True, False), _dec(2, 2, 2, 64, 64, 1000, name="d64 r64 masked")),
    (("split", "bf16", 64, 64, True, True), _dec(2, 4, 4, 64, 64, 1000, name="d64 r64 masked 12 waves")),
    (("split", "bf16", 64, 128, True, False), _dec(2, 2, 2, 64, 128, 1000, name="d64 r128 masked")),
    # split kernel, fp32
    (("split", "f32", 128, 0, False, False), _dec(2, 4, 2, 128, 0, 1000, dtype="f32", name="fp32 d128 r0")),
    (("split", "f32", 128, 0, False, True), _dec(1, 16, 2, 128, 0, 0, 400, ql=3, dtype="f32",
                                                 name="fp32 d128 r0 12 waves")),
    (("split", "f32", 128, 32, False, False), _dec(1, 2, 2, 128, 8, 1000, dtype="f32", name="fp32 d128 r8")),
    (("split", "f32", 128, 64, False, False), _dec(2, 2, 2, 128, 64, 1000, dtype="f32", name="fp32 d128 r64")),
    (("split", "f32", 64, 0, False, False), _dec(2, 4, 2, 64, 0, 1000, dtype="f32", name="fp32 d64 r0")),
    (("split", "f32", 64, 0, False, True), _dec(1, 16, 2, 64, 0, 0, 400, ql=3, dtype="f32",
                                                name="fp32 d64 r0 12 waves")),
    (("split", "f32", 64, 32, False, False), _dec(1, 2, 2, 64, 8, 1000, dtype="f32", name="fp32 d64 r8")),
    (("split", "f32", 64, 32, False, True), _dec(2, 2, 2, 64, 32, 1000, dtype="f32", name="fp32 d64 r32 12 waves")),
    (("split", "f32", 64, 64, False, False), _dec(1, 2, 2, 64, 64, 1000, dtype="f32", name="fp32 d64 r64")),
    (("split", "f32", 64, 64, False, True), _dec(3, 2, 2, 64, 64, 1000, dtype="f32", name="fp32 d64 r64 12 waves")),
    (("split", "f32", 64, 128, False, False), _dec(1, 4, 4, 64, 128, 1000, dtype="f32", name="fp32 d64 r128")),
]


def _k8(N, HQ, HK, r, L, shared=False, name=""):
    """Decode over int8 base keys (d = 128, no private tokens)."""
    return C(N, HQ, HK, 128, r, L, dtype="bf16", shared_lr=shared, name=name)


# split kernel over int8 base keys (d = 128): (residual columns, masked, twelve-wave form)
PATHS_K8 = [
    (("split", "bf16-k8", 128, 0, False, False), _k8(2, 4, 2, 0, 1000, name="int8 keys r0")),
    (("split", "bf16-k8", 128, 0, False, True), _k8(2, 16, 1, 0, 1000, name="int8 keys r0 12 waves")),
    (("split", "bf16-k8", 128, 32, False, False), _k8(1, 2, 2, 32, 1000, name="int8 keys r32 one agent")),
    (("split", "bf16-k8", 128, 32, False, True), _k8(5, 4, 1, 8, 1000, name="int8 keys r8 12 waves")),
    (("split", "bf16-k8", 128, 64, False, False), _k8(1, 2, 2, 64, 1000, name="int8 keys r64")),
    (("split", "bf16-k8", 128, 128, False, False), _k8(1, 2, 2, 128, 1000, name="int8 keys r128")),
    (("split", "bf16-k8", 128, 32, True, False), _k8(2, 2, 2, 32, 1000, name="int8 keys r32 masked")),
    (("split", "bf16-k8", 128, 32, True, True), _k8(5, 4, 1, 32, 1000, name="int8 keys r32 masked 12 waves")),
    (("split", "bf16-k8", 128, 64, True, False), _k8(2, 2, 2, 64, 1000, name="int8 keys r64 masked")),
    (("split", "bf16-k8", 128, 128, True, False), _k8(3, 16, 2, 128, 1000, name="int8 keys r128 masked")),
]


def built_instantiations():
    """Every kernel instantiation librattn builds (the rules the launchers
    follow: which split widths fit in registers in the eight- and twelve-wave
    forms, masked mode for bf16 ranks of 32 or more)."""
    keys = set()
    for dt in ("bf16", "f32"):
        for d in (64, 128):
            for cp in (0, 32, 64, 128):
                for masked in (False, True):
                    if masked and (dt != "bf16" or cp == 0):
                        continue
                    ok = dt == "bf16" or d == 64 or cp <= 64
                    wide = cp <= (64 if d == 64 else 32) if dt == "bf16" else cp <= (64 if d == 64 else 0)
                    if ok:
                        keys.add(("split", dt, d, cp, masked, False))
                    if ok and wide:
                        keys.add(("split", dt, d, cp, masked, True))
                if dt == "bf16":
                    keys.add(("prefill", dt, d, cp))
                    if d == 128:  # int8 keys: the d = 128 split kernels
                        for masked in (False, True):
                            if masked and cp == 0:
                                continue
                            keys.add(("split", "bf16-k8", d, cp, masked, False))
                            if cp <= 32:
                                keys.add(("split", "bf16-k8", d, cp, masked, True))
    return keys
