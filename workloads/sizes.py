"""Gradient-tensor size lists for the two tensor-fusion workloads.

``python -m workloads.sizes`` rewrites the frozen JSON lists next to this
file; everything else reads the JSON, so the lists never drift.

c4: 161 fp32 gradient tensors whose sizes are log-uniform between 256 and
    2,400,000 elements and sum to exactly 25,600,000 elements.  159 sizes
    are drawn by seed, one tensor is pinned at each end point, and the 159
    drawn sizes are scaled by one common factor (found by bisection, then
    clamped to the end points and rounded) so that the total is exact; the
    rounding residual goes to the largest unpinned tensor.  The list is then
    shuffled by seed.  The pages state both ">50% of tensors under 1 MB" and
    a ~25.6M total; a log-uniform population with these end points cannot
    hold both with the count fixed, so the count, end points, shape and the
    total are kept and the realised under-1-MiB share is reported.

c5: the gradients of a 12-layer Transformer encoder with hidden size 1024
    and FFN size 4096, in backward (production) order: the final LayerNorm's
    gamma/beta first, then layers 11..0, each as b2, W2, b1, W1, LN2 beta,
    LN2 gamma, bo, Wo, bv, Wv, bk, Wk, bq, Wq, LN1 beta, LN1 gamma.
"""
from __future__ import annotations

import json
import os

import numpy as np

from . import rng

HERE = os.path.dirname(os.path.abspath(__file__))
C4_PATH = os.path.join(HERE, "c4_sizes.json")
C5_PATH = os.path.join(HERE, "c5_sizes.json")

C4_COUNT, C4_LO, C4_HI, C4_TOTAL, C4_SEED = 161, 256, 2_400_000, 25_600_000, 4


def _c4_scaled(base: np.ndarray, k: float) -> np.ndarray:
    return np.clip(np.rint(base * k), C4_LO, C4_HI).astype(np.int64)


def make_c4() -> list:
    n_free = C4_COUNT - 2
    u = rng.uniform(C4_SEED, 0, n_free)
    base = np.exp(np.log(C4_LO) + u * (np.log(C4_HI) - np.log(C4_LO)))
    target = C4_TOTAL - C4_LO - C4_HI
    lo, hi = 1e-6, 1e3
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if _c4_scaled(base, mid).sum() > target:
            hi = mid
        else:
            lo = mid
    sizes = _c4_scaled(base, lo)
    resid = target - int(sizes.sum())
    j = int(np.argmax(sizes))
    sizes[j] += resid
    assert C4_LO <= sizes[j] <= C4_HI, "residual pushed a size out of range"
    allsz = np.concatenate([sizes, [C4_LO, C4_HI]])
    order = np.argsort(rng.uniform(C4_SEED, 1, C4_COUNT), kind="stable")
    out = [int(s) for s in allsz[order]]
    assert len(out) == C4_COUNT and sum(out) == C4_TOTAL
    return out


def make_c5() -> list:
    H, F, L = 1024, 4096, 12
    per_layer = [("b2", H), ("W2", H * F), ("b1", F), ("W1", F * H),
                 ("ln2_beta", H), ("ln2_gamma", H), ("bo", H), ("Wo", H * H),
                 ("bv", H), ("Wv", H * H), ("bk", H), ("Wk", H * H),
                 ("bq", H), ("Wq", H * H), ("ln1_beta", H), ("ln1_gamma", H)]
    out = [{"name": "lnf_gamma", "numel": H}, {"name": "lnf_beta", "numel": H}]
    for layer in range(L - 1, -1, -1):
        for name, n in per_layer:
            out.append({"name": f"l{layer}.{name}", "numel": n})
    return out


def c4_sizes() -> list:
    with open(C4_PATH) as f:
        return json.load(f)["numel"]


def c5_sizes() -> list:
    with open(C5_PATH) as f:
        return [t["numel"] for t in json.load(f)["tensors"]]


def main() -> None:
    c4 = make_c4()
    under = sum(1 for s in c4 if 4 * s < (1 << 20))
    with open(C4_PATH, "w") as f:
        json.dump({"recipe": "workloads/sizes.py make_c4", "count": len(c4),
                   "total_numel": sum(c4), "under_1MiB_share": under / len(c4),
                   "numel": c4}, f, indent=0)
        f.write("\n")
    c5 = make_c5()
    with open(C5_PATH, "w") as f:
        json.dump({"recipe": "workloads/sizes.py make_c5", "count": len(c5),
                   "total_numel": sum(t["numel"] for t in c5), "tensors": c5}, f, indent=0)
        f.write("\n")
    print("c4", len(c4), sum(c4), "under 1 MiB:", under / len(c4))
    print("c5", len(c5), sum(t["numel"] for t in c5))


if __name__ == "__main__":
    main()
