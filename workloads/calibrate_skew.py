"""Find the logit-offset scale of the skewed workload (v3-skew-loop).

The offsets are alpha * ln(p_rank) for Zipf(1.2) rank probabilities.  alpha is
chosen so that, at step 0 with zero bias, the 16 most-used experts receive about
half of all routings.  Bisection runs on an approximate router (float64 logits via
numpy plus the offset, selection by the CPU oracle); the final alpha is checked with
the oracle's own routing and written to skew_alpha.json next to this file.

Run:  python -m workloads.calibrate_skew
"""
import json
import os

import numpy as np

import oracle
import workloads


def main():
    w = workloads.get("v3-skew-loop", skew=False)
    w_router, _ = workloads.make_router(w)
    x = workloads.make_x(workloads.get("v3-skew-loop", skew=False)).float().numpy()
    x[:, 0] = 1.0
    wr = w_router.numpy().astype(np.float64)
    base = x[:, 1:].astype(np.float64) @ wr[:, 1:].T
    zero = np.zeros(w.E, np.float32)

    def share(alpha):
        off = workloads.zipf_offsets(w, alpha).astype(np.float64)
        z = (base + off).astype(np.float32)
        _, _, counts = oracle.select(z, zero, w.G, w.M, w.K, w.J)
        return workloads.zipf_top16_share(counts)

    lo, hi = 0.0, 4.0
    for _ in range(30):
        mid = (lo + hi) / 2
        if share(mid) < 0.5:
            lo = mid
        else:
            hi = mid
    alpha = round((lo + hi) / 2, 4)
    # exact check with the oracle's routing of the real inputs
    wr32 = w_router.numpy().copy()
    wr32[:, 0] = workloads.zipf_offsets(w, alpha)
    xb = workloads.make_x(workloads.get("v3-skew-loop", skew=False))
    xb[:, 0] = 1.0
    _, _, counts, _ = oracle.route(workloads.to_numpy(xb), wr32, zero, w.G, w.M, w.K, w.J)
    exact = workloads.zipf_top16_share(counts)
    out = dict(alpha=alpha, top16_share_at_step0=round(exact, 4), zipf_s=workloads.ZIPF_S,
               note="written by workloads/calibrate_skew.py (CPU oracle routing)")
    with open(os.path.join(os.path.dirname(__file__), "skew_alpha.json"), "w") as f:
        json.dump(out, f, indent=1)
    print(out)


if __name__ == "__main__":
    main()
