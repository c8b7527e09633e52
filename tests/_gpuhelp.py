"""Helpers for the GPU parity tests: move the generator's storage arrays to
the device and back.  No arithmetic of the method lives here."""
import numpy as np
import torch

import oracle


def dev(x):
    """numpy storage array -> torch tensor on cuda:0 (bf16 bits as int16)."""
    if isinstance(x, tuple):
        return tuple(dev(e) for e in x)
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        x = x.view(np.int16)
    return torch.from_numpy(x).to("cuda:0")


def host(t):
    return t.detach().to("cpu").numpy()


def bf16_out_to_f64(t):
    """bf16 torch output -> float64 numpy."""
    return oracle.bf16_bits_to_f64(t.detach().view(torch.int16).cpu().numpy().view(np.uint16))


def out_f64(t):
    if t.dtype == torch.bfloat16:
        return bf16_out_to_f64(t)
    return t.detach().cpu().numpy().astype(np.float64)


def check_topk_threshold_rule(gpu_idx, ref_scores, top_k, rel=1e-3):
    """Index sets may differ only at positions whose reference score lies
    within rel*|k-th score| of the reference threshold.  Also checks the
    list is ascending, in range, -1 padded, of the right length."""
    n = ref_scores.size
    m = min(top_k, n)
    g = np.asarray(gpu_idx)
    assert np.all(g[m:] == -1), "padding"
    v = g[:m]
    assert np.all(v >= 0) and np.all(v < n), "range"
    assert np.all(np.diff(v) > 0), "ascending, unique"
    ref = oracle.topk_row(ref_scores, top_k)[:m]
    t = oracle.topk_threshold(ref_scores, top_k)
    diff = np.setxor1d(v, ref)
    tol = rel * abs(t)
    bad = diff[np.abs(ref_scores[diff] - t) > tol]
    assert bad.size == 0, f"{bad.size} selections differ away from the threshold (t={t})"
    return diff.size
