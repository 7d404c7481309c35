"""Fit the constants of the forward's sequence-split cost model on the current GPU.

The model (page "Qwen Team Releases FlashQLA for High-Performance Linear
Attention", section "Core Technical Principles", with a fixed cost per call):
a split into segments of L chunks, whose work items fit one wave, takes
    lambda_1 L + lambda_2 segments + lambda_0
and the unsplit call over N chunks, with w waves of its 64-column work items,
    mu_1 N w + mu_0
(microseconds).  This script times gla_chunk_fwd (unsplit) and
gla_chunk_fwd_segments over a grid of (units = B x H, T, segment count) on
seeded synthetic bf16 inputs (d_k = d_v = 128, weak gates), fits both lines by
least squares, and prints the constants for csrc/split_model.h with the fit's
relative residuals.  It needs a GPU:

    python -m sub_quadratic_sequence_amd.fit_split [--out fit.json]
"""
import argparse
import json
import math

import numpy as np
import torch

from . import gla

DK = DV = 128
UNITS = (1, 2, 4, 8, 16, 32, 64)
TOKENS = (1024, 4096, 16384, 65536)
MAX_TOKENS = 1 << 21          # units x T per shape (memory and run time)
SEGMENTS = (2, 3, 4, 6, 8, 12, 16, 24, 32, 48, 64, 96, 128, 192, 256)


def _inputs(units, T, seed):
    gen = torch.Generator(device="cuda").manual_seed(seed)
    shape = (1, units, T, DK)
    q = (torch.randn(shape, generator=gen, device="cuda") / math.sqrt(DK)).to(torch.bfloat16)
    k = (torch.randn(shape, generator=gen, device="cuda") / math.sqrt(DK)).to(torch.bfloat16)
    v = torch.randn((1, units, T, DV), generator=gen, device="cuda").to(torch.bfloat16)
    g = (torch.nn.functional.logsigmoid(torch.randn(shape, generator=gen, device="cuda") + 4) / 16
         ).to(torch.bfloat16)
    return q, k, v, g


def _time_us(fn, reps=15, warm=3):
    for _ in range(warm):
        fn()
    ts = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        b.synchronize()
        ts.append(a.elapsed_time(b) * 1e3)
    ts.sort()
    return ts[len(ts) // 2]


def measure(num_cus):
    rows = []
    for units in UNITS:
        for T in TOKENS:
            if units * T > MAX_TOKENS:
                continue
            q, k, v, g = _inputs(units, T, seed=units * 100003 + T)
            o = torch.empty((1, units, T, DV), dtype=torch.bfloat16, device="cuda")
            nch = (T + 63) // 64
            t = _time_us(lambda: gla.gla_chunk_fwd(q, k, v, g, out=o, split=False))
            waves = -(-units * (DV // 64) // num_cus)
            rows.append({"units": units, "T": T, "segments": 1, "L": nch, "waves": waves, "us": t})
            for n in SEGMENTS:
                if n > nch or units * (DV // 128) * n > num_cus:
                    continue
                L = -(-nch // n)
                ns = -(-nch // L)
                if any(r["units"] == units and r["T"] == T and r["segments"] == ns for r in rows):
                    continue
                ws = torch.empty(gla.load_library().gla_chunk_fwd_segments_workspace_size(
                    1, units, T, DK, DV, ns) + 256, dtype=torch.uint8, device="cuda")
                t = _time_us(lambda: gla.gla_chunk_fwd_segments(q, k, v, g, ns, out=o, workspace=ws))
                rows.append({"units": units, "T": T, "segments": ns, "L": L, "waves": 1, "us": t})
            print(f"[fit] units={units} T={T}: {sum(1 for r in rows if r['units'] == units and r['T'] == T)}"
                  " timings", flush=True)
    return rows


def fit(rows):
    sp = [r for r in rows if r["segments"] > 1]
    un = [r for r in rows if r["segments"] == 1]
    A = np.array([[r["L"], r["segments"], 1.0] for r in sp])
    y = np.array([r["us"] for r in sp])
    lam, *_ = np.linalg.lstsq(A, y, rcond=None)
    Au = np.array([[r["L"] * r["waves"], 1.0] for r in un])
    yu = np.array([r["us"] for r in un])
    mu, *_ = np.linalg.lstsq(Au, yu, rcond=None)
    rel_sp = np.abs(A @ lam - y) / y
    rel_un = np.abs(Au @ mu - yu) / yu
    return {"lambda1": lam[0], "lambda2": lam[1], "lambda0": lam[2], "mu1": mu[0], "mu0": mu[1],
            "split_samples": len(sp), "unsplit_samples": len(un),
            "split_rel_residual_median": float(np.median(rel_sp)), "split_rel_residual_max": float(rel_sp.max()),
            "unsplit_rel_residual_median": float(np.median(rel_un)),
            "unsplit_rel_residual_max": float(rel_un.max())}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--out", help="write the timings and the fit as JSON")
    args = ap.parse_args()
    if not torch.cuda.is_available():
        raise SystemExit("fit_split needs a GPU")
    num_cus = torch.cuda.get_device_properties(0).multi_processor_count
    rows = measure(num_cus)
    f = fit(rows)
    f["num_cus"] = num_cus
    f["device"] = torch.cuda.get_device_name(0)
    print(json.dumps(f, indent=1))
    if args.out:
        with open(args.out, "w") as fh:
            json.dump({"fit": f, "rows": rows}, fh, indent=1)


if __name__ == "__main__":
    main()
