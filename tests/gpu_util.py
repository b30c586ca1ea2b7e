"""Helpers for the GPU parity tests (tolerance check, device transfer, the
oracle's full result for the full-size workloads, a parity log)."""
import json
import os

import numpy as np
import torch

import oracle
import synth_inputs as si

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


_FULL = {}


def full_reference(name):
    """The oracle's (y_ref, abs_ref) over EVERY output of a full-size workload
    (threaded over columns, bit-identical to the single-threaded oracle).
    Results are kept for the session (under 2 GB for every workload), so tests
    of one workload share one oracle run."""
    if name not in _FULL:
        case = si.workload(name)
        _FULL[name] = oracle.qmm_mt(*case.oracle_args())
    return _FULL[name]


def full_reference_i8t2(name):
    """The oracle's exact int32 product over every output of a ternary workload."""
    key = ("i8t2", name)
    if key not in _FULL:
        case = si.workload(name)
        _FULL[key] = oracle.i8t2_mm_mt(case.A.numpy(), case.Wp.numpy(), case.M, case.N, case.K)
    return _FULL[key]


def log_parity(what, **fields):
    """Print a parity figure and, if QMM_PARITY_LOG names a file, append it
    there as one JSON line."""
    rec = dict(case=what, **fields)
    print(json.dumps(rec), flush=True)
    path = os.environ.get("QMM_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(rec) + "\n")
