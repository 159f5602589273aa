"""Measure the tile configurations and fit the time model used to choose one.

    python -m tiled_fp32_gemm_sgemm_amd.calibrate [--out calib.json]
    python -m tiled_fp32_gemm_sgemm_amd.calibrate --fit calib.json

For every configuration it times shapes whose tile count fills the GPU with
one workgroup per CU (256 tiles) and with as many as a CU holds (256 * w
tiles, w from the configuration's waves and LDS footprint, at least 2), each
at K = 128, 256, 1024 and 4096, and fits, per unit of tile area,

    one round of 256 tiles:      BM*BN * (one_a + one_b * K)  microseconds
    one round of 256 * w tiles:  BM*BN * (two_a + two_b * K)  microseconds

A configuration counts as holding w workgroups per CU when the full round runs
clearly faster per tile than 256 tiles do (the workgroups overlap).
`--configs` restricts the run to some configurations (control and
experimental builds included).  The fitted rows are
printed in the form the configuration table in csrc/sgemm.hip takes.  Tile
size is a per-shape trade-off that libraries tune per GPU ("Tiling
Strategies", section 4; "CMU DLSys Lecture 12", section 6); this is that
tuning, stored as a model rather than as a per-shape table.
"""
from __future__ import annotations

import argparse
import json
import sys
import time

K_POINTS = (128, 256, 1024, 4096)
CUS = 256


def _slots(w: int):
    return (CUS, min(4, max(2, w)) * CUS)


def measure(out_path: str | None, configs=None) -> dict:
    import torch
    from . import api
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev).cuda_stream
    data = {}
    for c in range(api.num_configs()):
        info = api.config_info(c)
        if configs is None and not api.config_selectable(c):
            continue
        if configs is not None and c not in configs:
            continue
        w = api.workgroups_per_cu(c)
        data["_w_" + info["name"]] = w
        for slots in _slots(w):
            M = info["bm"] * 16
            N = info["bn"] * slots // 16
            for K in K_POINTS:
                A = torch.randn(M * K, device=dev)
                B = torch.randn(K * N, device=dev)
                C = torch.empty(M * N, device=dev)

                def run():
                    st = api.sgemm_strided_batched_raw(M, N, K, A.data_ptr(), K, 0,
                                                       B.data_ptr(), N, 0, C.data_ptr(), N, 0,
                                                       1, stream, "mfma", c)
                    if st != 0:
                        raise RuntimeError("config %d failed: %d" % (c, st))

                run()
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                run()
                torch.cuda.synchronize()
                n = max(5, min(200, int(0.25 / max(time.perf_counter() - t0, 1e-6))))
                for _ in range(3):
                    run()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(n):
                    run()
                e1.record()
                torch.cuda.synchronize()
                ms = e0.elapsed_time(e1) / n
                data.setdefault(info["name"], []).append(
                    (slots, K, 2.0 * M * N * K / ms / 1e9))
        print(info["name"], data[info["name"]], flush=True)
    if out_path:
        with open(out_path, "w") as f:
            json.dump(data, f)
    return data


def fit(data: dict) -> dict:
    """name -> (per_cu, one_a, one_b, two_a, two_b), least squares of time per
    unit tile area against K."""
    import numpy as np
    rows = {}
    for name, pts in data.items():
        if name.startswith("_w_"):
            continue
        w = min(4, max(2, int(data.get("_w_" + name, 2))))
        coef = []
        top = {}
        for slots in _slots(w):
            K = np.array([k for s, k, _ in pts if s == slots], float)
            tf = np.array([t for s, _, t in pts if s == slots], float)
            t_us = 2.0 * slots * K / (tf * 1e12) * 1e6
            A = np.vstack([np.ones_like(K), K]).T
            (a, b), *_ = np.linalg.lstsq(A, t_us, rcond=None)
            coef += [max(float(a), 0.0), float(b)]  # a fixed cost is never negative
            top[slots] = tf[np.argmax(K)]
        per_cu = w if top[w * CUS] > 1.06 * top[CUS] else 1
        rows[name] = (per_cu, *coef)
    return rows


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--out", help="write the measurements here (JSON)")
    ap.add_argument("--fit", help="fit measurements read from this JSON instead of measuring")
    ap.add_argument("--configs", help="comma-separated configuration indices to measure")
    args = ap.parse_args(argv)
    configs = [int(c) for c in args.configs.split(",")] if args.configs else None
    data = json.load(open(args.fit)) if args.fit else measure(args.out, configs)
    for name, (per_cu, a1, b1, a2, b2) in fit(data).items():
        print('    "%s": %d, %.4e, %.4e, %.4e, %.4e' % (name, per_cu, a1, b1, a2, b2))
    return 0


if __name__ == "__main__":
    sys.exit(main())
