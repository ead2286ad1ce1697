"""Comparison helpers shared by the GPU parity tests: bit-exact checks for
integer, index and bit-copy results, and the LayerNorm tolerance (max-abs 2e-3,
mean-abs 1e-4 against the oracle, equal NaN positions) for normalised rows.

Normalised rows are also held to a mismatch count, 0 by default: the kernels
round the binary64 LayerNorm once to binary16, so an output can differ from the
oracle's only when the exact value lies within ~2^-43 (relative) of a rounding
midpoint, which none of the seeded inputs here comes close to. The kernels are
deterministic (fixed reduction order, no atomics), so a count above 0 on these
inputs is a regression in the rounding, reported as a failure rather than as
a printed number."""
import numpy as np

MAX_ABS, MEAN_ABS = 2e-3, 1e-4


def to_dev(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def bits(a):
    return np.asarray(a, dtype=np.float16).view(np.uint16)


def assert_bit_exact(got, ref, label=""):
    g, r = bits(got), bits(ref)
    assert g.shape == r.shape, label
    bad = np.flatnonzero(g.reshape(-1) != r.reshape(-1))
    assert bad.size == 0, f"{label}: {bad.size} elements differ, first at flat index {bad[:5]}"


def assert_ln_close(got, ref, label="", max_mismatches=0):
    g = np.asarray(got, np.float16).astype(np.float64)
    r = np.asarray(ref, np.float16).astype(np.float64)
    assert g.shape == r.shape, label
    nan_r = np.isnan(r)
    assert np.array_equal(np.isnan(g), nan_r), f"{label}: NaN positions differ"
    d = np.abs(g[~nan_r] - r[~nan_r])
    if d.size == 0:
        return 0
    mismatches = int((d > 0).sum())
    print(f"[{label}] max_abs={d.max():.3e} mean_abs={d.mean():.3e} "
          f"mismatches={mismatches}/{d.size}", flush=True)
    assert d.max() <= MAX_ABS, f"{label}: max-abs {d.max()}"
    assert d.mean() <= MEAN_ABS, f"{label}: mean-abs {d.mean()}"
    assert mismatches <= max_mismatches, f"{label}: {mismatches} outputs differ from the oracle"
    return mismatches


