"""Writes the stored expected values for the full-size parity tests.

For each full-size workload (forward only for the N=2048 one), the fp64
oracle computes O, LSE and dQ at sampled query rows and dK, dV at sampled key
columns of selected heads (every row of the head still enters through the
logsumexp and D terms). The inputs are regenerated from the seeded recipe of
the `workloads` module; a SHA-256 of each stored input tensor is saved so a
test can tell that it regenerated the same bytes.

The block-sparse workload ("local_global") is written the same way, with
its block mask, to sampled_sparse_local_global.npz.

Only `oracle` and `workloads` are used. Run from the repository root:
    python tests/golden/make_golden.py [config ... | local_global]
"""
import hashlib
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from workloads import SPARSE_WORKLOADS, WORKLOADS, block_mask_local_global, make_inputs  # noqa: E402

OUT = os.path.dirname(os.path.abspath(__file__))


def sample_indices(N, seed):
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, 255, N // 2 - 1, N // 2, N - 129, N - 128, N - 2, N - 1]
    rng = np.random.default_rng(seed)
    extra = rng.choice(N, size=9, replace=False)
    return np.unique(np.clip(np.array(fixed + list(extra)), 0, N - 1))


def heads_for(w):
    if w.config_id == 5:
        return [(0, 5)]
    return [(0, 0), (w.B - 1, w.H - 1)]


def main(cfgs):
    for cfg in cfgs:
        if cfg in SPARSE_WORKLOADS:
            sparse(cfg)
            continue
        w = WORKLOADS[cfg]
        t0 = time.time()
        inp = make_inputs(w)
        sha = {k: hashlib.sha256(np.ascontiguousarray(v[0]).tobytes()).hexdigest() for k, v in inp.items()}
        vals = {k: v[1] for k, v in inp.items()}
        rows = sample_indices(w.N, 100 + cfg)
        cols = sample_indices(w.N, 200 + cfg)
        out = {"rows": rows, "cols": cols, "heads": np.array(heads_for(w), np.int64)}
        for name, digest in sha.items():
            out[f"sha256_{name}"] = np.array(digest)
        for hi, (b, h) in enumerate(heads_for(w)):
            s = oracle.sampled_head(vals["q"], vals["k"], vals["v"], vals.get("do"), w.scale, w.causal,
                                    w.dropout_p, w.dropout_seed, b, h, rows, cols)
            for key, arr in s.items():
                out[f"h{hi}_{key}"] = arr
        path = os.path.join(OUT, f"sampled_cfg{cfg}.npz")
        np.savez_compressed(path, **out)
        print(f"config {cfg}: wrote {path} in {time.time() - t0:.1f} s", flush=True)


def sparse(name):
    w, kw = SPARSE_WORKLOADS[name]
    t0 = time.time()
    inp = make_inputs(w)
    mask = block_mask_local_global(w.N, **kw)
    vals = {k: v[1] for k, v in inp.items()}
    rows = sample_indices(w.N, 300)
    cols = sample_indices(w.N, 400)
    heads = [(0, 0), (0, w.H - 1)]
    out = {"rows": rows, "cols": cols, "heads": np.array(heads, np.int64), "mask": mask}
    for k, v in inp.items():
        out[f"sha256_{k}"] = np.array(hashlib.sha256(np.ascontiguousarray(v[0]).tobytes()).hexdigest())
    for hi, (b, h) in enumerate(heads):
        s = oracle.sampled_head(vals["q"], vals["k"], vals["v"], vals["do"], w.scale, w.causal,
                                w.dropout_p, w.dropout_seed, b, h, rows, cols, bmask=mask)
        for key, arr in s.items():
            out[f"h{hi}_{key}"] = arr
    path = os.path.join(OUT, f"sampled_sparse_{name}.npz")
    np.savez_compressed(path, **out)
    print(f"{name}: wrote {path} in {time.time() - t0:.1f} s", flush=True)


if __name__ == "__main__":
    main([a if a in SPARSE_WORKLOADS else int(a) for a in sys.argv[1:]] or [2, 3, 4, 5, "local_global"])
