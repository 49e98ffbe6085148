"""Measure both attention kernels over a grid of masks and shapes and fit
the coefficients of the kernel-choice cost model (csrc/select_model.h).

    python -m sparse_masked_head_amd.calibrate --out sweep.json   # on a GPU
    python -m sparse_masked_head_amd.calibrate --fit sweep.json   # anywhere

Each point times the forced row-wise and block-wise kernels with HIP events
over back-to-back launches (inputs resident, mask encoded once) and records
the encoding statistics the model sees.  The block-wise kernel is timed as
SMH_AUTO runs it: with the per-tile dispatch of sparse partial tiles to its
gather path.
"""
import argparse
import json
import sys
import time

import numpy as np

MASKS = [("random", {"p": 0.001}), ("random", {"p": 0.01}),
         ("random", {"p": 0.05}), ("random", {"p": 0.3}),
         ("window", {"w": 4}), ("window", {"w": 64}), ("window", {"w": 256}),
         ("causal", {}), ("full", {}), ("bigbird", {})]
SIZES = [256, 512, 1024, 2048, 4096]
HEADS = [1, 8, 64]
DIMS = [64, 128]
# long sequences: fewer heads, and no dense mask (its row-wise time alone
# would dominate the sweep)
MASKS_LONG = [("random", {"p": 0.001}), ("random", {"p": 0.01}),
              ("far_random", {"p": 0.02}), ("long_random", {}),
              ("window", {"w": 64}), ("causal", {})]
SIZES_LONG = [8192, 16384]
HEADS_LONG = [1, 8, 32]
# the decision rule of select_model: row-wise when t_row < ROW_MARGIN * t_blk
ROW_MARGIN = 1.0
# weight of the row/block time ratio's log error in the fit
RATIO_WEIGHT = 2.0


def _time(fn, reps, tries=3):
    """Microseconds per launch: the best of `tries` runs of `reps`
    back-to-back launches (a single stalled run does not decide a point)."""
    import torch
    fn()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    best = float("inf")
    for _ in range(tries):
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        best = min(best, a.elapsed_time(b) * 1e3 / reps)
    return best


def sweep(out_path, quick=False):
    import torch
    import sparse_masked_head_amd as smh
    from workloads import mask_family
    dev = torch.device("cuda:0")
    points = []
    sizes = SIZES[:3] if quick else SIZES
    grid = [(fam, kw, S, HEADS) for fam, kw in MASKS for S in sizes]
    if not quick:
        grid += [(fam, kw, S, HEADS_LONG) for fam, kw in MASKS_LONG
                 for S in SIZES_LONG]
    t0 = time.time()
    for fam, kw, S, heads in grid:
        if fam == "bigbird" and S < 1024:
            continue    # needs enough 64-wide blocks for 3 random picks
        mask = mask_family(fam, S, seed=S, **kw)
        m = torch.from_numpy(mask).to(dev)
        del mask
        enc = smh.encode_mask(m)
        st = smh.mask_stats_get(enc)
        for d in DIMS:
            for BH in heads:
                if BH * S * d * 2 * 4 > (1 << 31):
                    continue
                q = torch.randn(1, BH, S, d, device=dev).half()
                k = torch.randn_like(q)
                v = torch.randn_like(q)
                o = torch.empty_like(q)
                reps = 50 if S * BH < 65536 else 5
                t = {}
                for kern in ("rowwise", "blockwise"):
                    t[kern] = _time(lambda: smh.sparse_mha_fwd(
                        q, k, v, enc, kernel=kern, out=o), reps)
                points.append(dict(family=fam, kw=kw, S=S, d=d, BH=BH,
                                   stats=st, t_row_us=t["rowwise"],
                                   t_blk_us=t["blockwise"]))
                print(f"{fam:8s} {str(kw):14s} S={S:5d} d={d:3d} "
                      f"BH={BH:3d} row {t['rowwise']:9.1f} us  blk "
                      f"{t['blockwise']:9.1f} us  [{time.time()-t0:.0f}s]",
                      flush=True)
    with open(out_path, "w") as f:
        json.dump(points, f)
    return points


def model(coef, p):
    """Python restatement of select_costs_us for fitting (same formula)."""
    launch, bt, bp, bs, rg, rk, rsg, rsk, be, bsp, bes, launch_r = coef
    st = p["stats"]
    n = -(-p["S"] // 64)
    tiles = st["n_full"] + st["n_partial"]
    ents = st.get("row_entries", 0)
    nsp = st.get("n_sparse", 0) if ents > 0 else 0
    w_blk = p["BH"] * ((tiles - nsp) * bt + (st["n_partial"] - nsp) * bp +
                       ents * be + nsp * bsp)
    # heaviest row: its tiles split like the mask's, the sparse ones costing
    # their entries per wavefront (4 wavefronts, one group of 16 rows each)
    f = nsp / tiles if tiles else 0.0
    ept = ents / (4.0 * nsp) if nsp else 0.0
    crit = st["max_row_tiles"] * ((1.0 - f) * bs + f * ept * bes)
    t_blk = launch + max(w_blk, crit)
    live = 64.0 * st["n_full"]
    if st["n_partial"] > 0:
        rho = (st["nnz"] - 4096.0 * st["n_full"]) / (4096.0 * st["n_partial"])
        rho = min(max(rho, 0.0), 1.0)
        live += st["n_partial"] * 64.0 * (1.0 - (1.0 - rho) ** 8)
    chunks = live / 64.0 + n
    w_row = p["BH"] * (tiles * rg + 8.0 * chunks * rk)
    live_max = live / tiles * st["max_row_tiles"] if tiles else 0.0
    s_row = st["max_row_tiles"] / 8.0 * rsg + (live_max / 64.0 + 1.0) * rsk
    t_row = launch_r + max(w_row, s_row)
    return t_row, t_blk


def fit(points):
    from scipy.optimize import least_squares
    out = {}
    for d in DIMS:
        pts = [p for p in points if p["d"] == d and
               p["stats"]["n_full"] + p["stats"]["n_partial"] > 0]

        # log errors of both times, and (weighted) of their ratio, the
        # quantity the choice depends on
        def resid(c):
            r = []
            for p in pts:
                tr, tb = model(np.abs(c), p)
                r.append(np.log(tr / p["t_row_us"]))
                r.append(np.log(tb / p["t_blk_us"]))
                r.append(RATIO_WEIGHT * (np.log(tr / tb) -
                                         np.log(p["t_row_us"] / p["t_blk_us"])))
            return np.array(r)
        c0 = np.array([4.0, 1e-3, 2e-4, 0.5, 1e-4, 1e-3, 1.0, 1.0, 5e-5, 1e-4, 0.02, 4.0])
        res = least_squares(resid, c0, x_scale=c0)
        c = np.abs(res.x)
        agree = tie = regret = best_sum = 0
        for p in pts:
            tr, tb = model(c, p)
            best = min(p["t_row_us"], p["t_blk_us"])
            row = tr < ROW_MARGIN * tb
            got = p["t_row_us"] if row else p["t_blk_us"]
            agree += row == (p["t_row_us"] < p["t_blk_us"])
            tie += got <= 1.03 * best
            regret += got - best
            best_sum += best
        out[d] = dict(coef=c.tolist(), rms_log=float(np.sqrt(np.mean(
            res.fun ** 2))), agree=agree, tie=tie, n=len(pts),
            regret=regret / best_sum)
        print(f"d={d}: coef {', '.join('%.5g' % x for x in c)}  rms log "
              f"{out[d]['rms_log']:.3f}  choice agrees {agree}/{len(pts)} "
              f"({tie} within 3% of the faster)  time lost to wrong picks "
              f"{100 * regret / best_sum:.2f}%")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", help="run the sweep on the GPU, write JSON")
    ap.add_argument("--fit", help="fit coefficients from a sweep JSON")
    ap.add_argument("--quick", action="store_true")
    a = ap.parse_args()
    if a.out:
        pts = sweep(a.out, a.quick)
        fit(pts)
    elif a.fit:
        fit(json.load(open(a.fit)))
    else:
        ap.print_help()
        sys.exit(2)


if __name__ == "__main__":
    main()
