"""Parity helpers shared by the GPU tests: moving seeded inputs to the device
and comparing the HIP path with the CPU oracle.

Criteria (the score definition is exact; only rounding differs):
  * scores: |S_gpu - S_ref| <= TOL * A_s, where A_s = sum_h |w_h| |x_h| is the
    oracle's magnitude of the terms that make up S_s (>= |S_s|); a plain
    |S|-relative bound is impossible because S can cancel to ~0;
  * selection given the scores: the GPU's index row must equal, bit for bit,
    the oracle's top-k of the GPU's own fp32 scores (same precision on both
    sides, so ties and the lower-position rule are checked exactly);
  * selection against the oracle's own: equal sizes, no duplicates, nothing
    invisible, and every position in the symmetric difference scores within
    TOL * (A_s + A_theta) of the oracle's k-th score theta.
"""
import numpy as np
import torch

import oracle

TOL = 2e-3


def dev(a, dtype=None):
    """numpy -> CUDA tensor; raw bf16 (uint16) / fp8 (uint8) bits keep their bits."""
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "bf16":
        t = t.view(torch.int16).view(torch.bfloat16)
    elif dtype == "fp8_e4m3":
        t = t.view(torch.float8_e4m3fn)
    return t.cuda()


def check_scores(gpu, ref, mag, tol=TOL, exact=False, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if exact:
        assert np.array_equal(gpu + 0.0, ref + 0.0), f"{what}: scores not bit-exact"
        return 0.0
    err = np.abs(gpu - ref)
    bound = tol * np.asarray(mag, dtype=np.float64)
    bad = err > bound
    assert not bad.any(), (f"{what}: {bad.sum()} scores outside {tol}*A "
                           f"(worst err {err[bad].max():.3g} vs bound {bound[bad][np.argmax(err[bad])]:.3g})")
    m = np.asarray(mag, dtype=np.float64)
    return float((err / np.where(m > 0, m, 1)).max()) if err.size else 0.0


def check_topk_of_own_scores(idx_rows, score_rows, lens, k, what=""):
    """Each GPU index row equals the oracle's top-k of the GPU scores of that row."""
    for r, (idx, s, n) in enumerate(zip(idx_rows, score_rows, lens)):
        want = oracle.topk(np.asarray(s[:n], dtype=np.float64)[None, :], [n], k)[0]
        assert np.array_equal(np.asarray(idx), want), f"{what}: row {r} selection differs from top-k of its scores"


def check_sets(gpu_idx, ref_idx, ref_s, ref_a, n, tol=TOL, what=""):
    """Compare one row's selection with the oracle's (ref_s / ref_a indexed by position)."""
    g = np.asarray(gpu_idx)
    r = np.asarray(ref_idx)
    gv, rv = g[g >= 0], r[r >= 0]
    assert len(gv) == len(rv) == min(n, len(g)), f"{what}: sizes {len(gv)} vs {len(rv)}"
    assert len(np.unique(gv)) == len(gv), f"{what}: duplicates"
    assert np.all(np.diff(gv) > 0), f"{what}: not ascending"
    assert gv.min(initial=0) >= 0 and gv.max(initial=-1) < n, f"{what}: out of range"
    diff = np.setxor1d(gv, rv)
    if diff.size == 0:
        return 0
    theta_pos = rv[np.argmin(ref_s[rv])]
    theta, a_theta = ref_s[theta_pos], ref_a[theta_pos]
    ok = np.abs(ref_s[diff] - theta) <= tol * (ref_a[diff] + a_theta)
    assert ok.all(), f"{what}: {np.sum(~ok)} set differences beyond the tolerance band"
    return int(diff.size)
