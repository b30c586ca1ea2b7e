"""Helpers for the GPU parity tests (tolerance check, device transfer)."""
import numpy as np
import torch

# |y - y_ref| <= 2e-3 * sum_k |x w| + 1e-5, elementwise (the stated bound)
REL, ABS = 2e-3, 1e-5


def err_ratio(y, y_ref, abs_ref):
    y = np.asarray(y, dtype=np.float64)
    assert np.all(np.isfinite(y)), "non-finite output"
    return np.abs(y - y_ref) / (REL * abs_ref + ABS)


def assert_within_bound(y, y_ref, abs_ref, what=""):
    r = err_ratio(y, y_ref, abs_ref)
    if r.size == 0:
        return 0.0
    worst = np.unravel_index(np.argmax(r), r.shape)
    assert r.max() <= 1.0, f"{what}: max err/bound {r.max():.3g} at {worst}"
    return float(r.max())


def dev(case):
    return case.to("cuda")


def cpu(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def sample_points(M, N, count, seed):
    """Output coordinates to check one by one: corners, tile edges and random."""
    rng = np.random.default_rng(seed)
    ms = list(rng.integers(0, M, count))
    ns = list(rng.integers(0, N, count))
    for m in {0, M - 1}:
        for n in {0, N - 1, min(63, N - 1), min(64, N - 1), N // 2}:
            ms.append(m)
            ns.append(n)
    return np.array(ms, np.int32), np.array(ns, np.int32)
