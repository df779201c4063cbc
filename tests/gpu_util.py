"""Helpers for the GPU parity tests: device transfer and tolerance checks."""
import os

import numpy as np


def dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host(t) -> np.ndarray:
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def empty(shape, dtype):
    import torch
    return torch.empty(shape, dtype=dtype, device="cuda")


def sentinel(shape, dtype, value=-7):
    import torch
    return torch.full(shape, value, dtype=dtype, device="cuda")


def oracle_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def assert_within_bound(y_gpu: np.ndarray, y_ref: np.ndarray, bound: np.ndarray, rel: float = 1e-5, what: str = ""):
    """|y_gpu - y_ref| <= rel * bound per element (bound = sum |w_i x_i| from the oracle);
    an all-zero row (bound 0) must give exactly 0."""
    y_gpu = np.asarray(y_gpu, np.float64)
    err = np.abs(y_gpu - y_ref)
    lim = rel * bound
    bad = err > lim
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError("%s: %d of %d outputs exceed %.1e*bound; first %s: gpu=%r ref=%r bound=%r" % (
            what, int(bad.sum()), bad.size, rel, idx.tolist(), y_gpu[tuple(idx[0])], y_ref[tuple(idx[0])],
            bound[tuple(idx[0])]))
    return float((err / np.maximum(bound, 1e-300)).max()) if err.size else 0.0


def progress(msg: str):
    print("[gpu-test] " + msg, flush=True)
