"""Parity bars shared by the GPU tests (and exercised on the CPU by negative controls).

Contract bar, per output element over one call (all layers of a multi-layer call):
max |o - o_ref| <= 2e-2 and mean |o - o_ref| <= 2e-3.  Because the synthetic
workloads have flat attention and tiny outputs, the contract bar alone does not
detect a dropped residual term at every shape; two supplementary bars do:
  * relative RMS error  ||o - o_ref|| / ||o_ref||  <= 1e-2 (bf16) or 1e-4 (fp32);
  * residual sensitivity ||o - o_ref|| <= 0.05 ||o_ref - o_ref(B = 0)||, i.e. the
    error is small against what the residual terms contribute.
"""
import numpy as np

MAX_ABS = 2e-2
MEAN_ABS = 2e-3
REL_RMS = {"bf16": 1e-2, "f32": 1e-4}
RESID_FRAC = 0.05


def stats(got, ref, ref_b0=None):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    mask = ~np.isnan(ref)
    err = np.abs(got[mask] - ref[mask])
    s = dict(max_abs=float(err.max()) if err.size else 0.0,
             mean_abs=float(err.mean()) if err.size else 0.0,
             rel_rms=float(np.linalg.norm(err) / max(np.linalg.norm(ref[mask]), 1e-300)),
             finite=bool(np.all(np.isfinite(got[mask]))))
    if ref_b0 is not None:
        ref_b0 = np.asarray(ref_b0, dtype=np.float64)
        resid = np.linalg.norm(ref[mask] - ref_b0[mask])
        s["resid_ratio"] = float(np.linalg.norm(err) / max(resid, 1e-300))
    return s


def failures(s, dtype):
    bad = []
    if not s["finite"]:
        bad.append("non-finite output")
    if s["max_abs"] > MAX_ABS:
        bad.append(f"max_abs {s['max_abs']:.3e} > {MAX_ABS}")
    if s["mean_abs"] > MEAN_ABS:
        bad.append(f"mean_abs {s['mean_abs']:.3e} > {MEAN_ABS}")
    if s["rel_rms"] > REL_RMS[dtype]:
        bad.append(f"rel_rms {s['rel_rms']:.3e} > {REL_RMS[dtype]}")
    if "resid_ratio" in s and s["resid_ratio"] > RESID_FRAC:
        bad.append(f"resid_ratio {s['resid_ratio']:.3e} > {RESID_FRAC}")
    return bad


def check(got, ref, dtype, ref_b0=None, what=""):
    s = stats(got, ref, ref_b0)
    bad = failures(s, dtype)
    assert not bad, f"{what}: {'; '.join(bad)} ({s})"
    return s
