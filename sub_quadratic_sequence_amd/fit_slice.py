"""Choose the constants of the forward's d_v slice-width model on the current GPU.

The model (csrc/split_model.h, namespace slice_model): a call runs its work
items in rounds of num_cus; a last partial round with a fraction f of the
compute units busy costs kPartial + (1 - kPartial) f of a full round, and a
round of 128-column items kWide rounds of 64-column items.  The 128-column slice
is taken when kWide x rounds(items at 128) < rounds(items at 64).

This script times gla_chunk_fwd_sliced at both widths over a grid of
(units = B x H, T, d_v) on seeded synthetic bf16 inputs (d_k = 128, weak gates),
then searches a 0.05 grid of (kWide, kPartial) for the pairs whose choices lose
the least time against the faster width, on average over the grid.  It prints
those pairs, their mean and largest loss, and the same figures for the rule
"128 columns once their work items fill the device".  It needs a GPU:

    python -m sub_quadratic_sequence_amd.fit_slice [--out fit.json]
"""
import argparse
import json
import math

import numpy as np
import torch

from . import gla

DK = 128
GRID = ([(T, dv, u) for T in (512, 2048, 8192) for dv in (128, 256) for u in range(32, 513, 32)] +
        [(T, dv, u) for T in (1024, 4096) for dv in (128, 256)
         for u in (40, 100, 150, 200, 270, 300, 350, 400, 460, 540, 600, 700, 800)])
MAX_ELEMS = 1 << 28    # units x T x dv per shape (memory and run time)


def _time_us(fn, reps=12, warm=3):
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


def measure():
    rows = []
    gen = torch.Generator(device="cuda").manual_seed(7)
    for T, dv, units in GRID:
        if units * T * dv > MAX_ELEMS:
            continue
        shape = (1, units, T, DK)
        q = (torch.randn(shape, generator=gen, device="cuda") / math.sqrt(DK)).to(torch.bfloat16)
        k = (torch.randn(shape, generator=gen, device="cuda") / math.sqrt(DK)).to(torch.bfloat16)
        v = torch.randn((1, units, T, dv), generator=gen, device="cuda").to(torch.bfloat16)
        g = (torch.nn.functional.logsigmoid(torch.randn(shape, generator=gen, device="cuda")) / 16
             ).to(torch.bfloat16)
        o = torch.empty((1, units, T, dv), dtype=torch.bfloat16, device="cuda")
        r = {"T": T, "dv": dv, "units": units}
        for w in (64, 128):
            r[f"us{w}"] = _time_us(lambda: gla.gla_chunk_fwd(q, k, v, g, out=o, dv_slice=w))
        print("[fit] " + json.dumps(r), flush=True)
        rows.append(r)
        del q, k, v, g, o
    return rows


def rounds(items, num_cus, partial):
    full, rem = divmod(items, num_cus)
    return full + (partial + (1.0 - partial) * rem / num_cus if rem else 0.0)


def choices(rows, num_cus, wide, partial):
    out = []
    for r in rows:
        i128 = r["units"] * r["dv"] // 128
        out.append(128 if wide * rounds(i128, num_cus, partial) < rounds(2 * i128, num_cus, partial)
                   else 64)
    return out


def losses(rows, picks):
    """Mean and largest time lost against the faster width, as fractions."""
    lost = [r[f"us{w}"] / min(r["us64"], r["us128"]) - 1.0 for r, w in zip(rows, picks)]
    return float(np.mean(lost)), float(np.max(lost))


def choose(rows, num_cus):
    grid = {}
    for partial in np.round(np.arange(0.0, 1.0001, 0.05), 2):
        for wide in np.round(np.arange(1.0, 2.5001, 0.05), 2):
            grid[(float(wide), float(partial))] = losses(rows, choices(rows, num_cus, wide, partial))
    best = min(v[0] for v in grid.values())
    optimal = sorted(k for k, v in grid.items() if v[0] <= best + 1e-12)
    threshold = [128 if r["units"] * r["dv"] // 128 >= num_cus else 64 for r in rows]
    return {"optimal_pairs_kWide_kPartial": optimal, "mean_loss": best,
            "max_loss": grid[optimal[0]][1], "samples": len(rows),
            "threshold_rule_losses_mean_max": losses(rows, threshold)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--out", help="write the timings and the result as JSON")
    args = ap.parse_args()
    if not torch.cuda.is_available():
        raise SystemExit("fit_slice needs a GPU")
    num_cus = torch.cuda.get_device_properties(0).multi_processor_count
    rows = measure()
    f = choose(rows, num_cus)
    f["num_cus"] = num_cus
    f["device"] = torch.cuda.get_device_name(0)
    print(json.dumps(f, indent=1))
    if args.out:
        with open(args.out, "w") as fh:
            json.dump({"result": f, "rows": rows}, fh, indent=1)


if __name__ == "__main__":
    main()
