"""Microbenchmarks of single library kernels, for profiling (rocprofv3) and tuning.

    python -m fp8_precision_transformer_amd.microbench gemm --m 15872 --n 12288 --k 4096
    python -m fp8_precision_transformer_amd.microbench cast --rows 15872 --cols 16384

Operands are random bytes / values drawn on the GPU (timing only; parity lives in
tests/).  Each launch is timed with HIP events on the launch stream; the report
is one JSON line with the median launch time and the algorithmic rate.
"""

from __future__ import annotations

import argparse
import json

import torch

from . import binding as B


def _time(fn, iters, warmup):
    for _ in range(warmup):
        fn()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in ev)
    return t[len(t) // 2]


def gemm(args):
    dev = "cuda:0"
    m, n, k = args.m, args.n, args.k
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    if args.kind == "bf16":
        a = (torch.randn((m, k), device=dev, generator=g)).to(torch.bfloat16)
        b = (torch.randn((n, k), device=dev, generator=g) * 0.02).to(torch.bfloat16)
        sa = sb = None
        fa = fb = "BF16"
        gran = B.TE_GRAN_TENSOR
    else:
        # finite mid-range codes with random signs
        a = (torch.randint(0x18, 0x48, (m, k), device=dev, generator=g, dtype=torch.int32) |
             (torch.randint(0, 2, (m, k), device=dev, generator=g, dtype=torch.int32) << 7)).to(torch.uint8)
        b = (torch.randint(0x18, 0x48, (n, k), device=dev, generator=g, dtype=torch.int32) |
             (torch.randint(0, 2, (n, k), device=dev, generator=g, dtype=torch.int32) << 7)).to(torch.uint8)
        fa, fb = args.fa, args.fb
        if args.kind == "mx":
            sa = torch.full((m, k // 32), 127, dtype=torch.uint8, device=dev)
            sb = torch.full((n, k // 32), 127, dtype=torch.uint8, device=dev)
            gran = B.TE_GRAN_MX_BLOCK32
        else:
            sa = torch.ones(1, dtype=torch.float32, device=dev)
            sb = torch.ones(1, dtype=torch.float32, device=dev)
            gran = B.TE_GRAN_TENSOR
    d = torch.empty((m, n), dtype=torch.bfloat16 if args.out == "bf16" else torch.float32, device=dev)
    ms = _time(lambda: B.te_fp8_gemm(a, fa, sa, b, fb, sb, d, gran=gran), args.iters, args.warmup)
    fl = 2.0 * m * n * k
    print(json.dumps({"kernel": f"gemm_{args.kind}", "m": m, "n": n, "k": k, "ms": round(ms, 5),
                      "tflops": round(fl / ms / 1e9, 1)}), flush=True)


def cast(args):
    dev = "cuda:0"
    x = torch.randn((args.rows, args.cols), device=dev).to(torch.bfloat16)
    R, C = args.rows, args.cols
    scale = torch.ones(1, device=dev)
    si = torch.empty(1, device=dev)
    am = torch.empty(1, device=dev)
    mode = B.TE_SCALE_CURRENT if args.mode == "current" else B.TE_SCALE_DELAYED
    if args.op == "cast":
        out = torch.empty((R, C), dtype=torch.uint8, device=dev)
        fn = lambda: B.te_amax_cast(x, "E4M3", mode, 0, scale, si, am, out)  # noqa: E731
        nbytes = R * C * (5 if mode == B.TE_SCALE_CURRENT else 3)
    elif args.op == "transpose":
        out = torch.empty((C, R), dtype=torch.uint8, device=dev)
        fn = lambda: B.te_cast_transpose(x, "E4M3", mode, 0, scale, si, am, None, out)  # noqa: E731
        nbytes = R * C * (5 if mode == B.TE_SCALE_CURRENT else 3)
    elif args.op == "both":
        o1 = torch.empty((R, C), dtype=torch.uint8, device=dev)
        o2 = torch.empty((C, R), dtype=torch.uint8, device=dev)
        fn = lambda: B.te_cast_transpose(x, "E4M3", mode, 0, scale, si, am, o1, o2)  # noqa: E731
        nbytes = R * C * (6 if mode == B.TE_SCALE_CURRENT else 4)
    else:  # mx
        o1 = torch.empty((R, C), dtype=torch.uint8, device=dev)
        s1 = torch.empty((R, C // 32), dtype=torch.uint8, device=dev)
        fn = lambda: B.te_mxfp8_quantize(x, "E4M3", o1, s1)  # noqa: E731
        nbytes = R * C * 3 + R * C // 32
    ms = _time(fn, args.iters, args.warmup)
    print(json.dumps({"kernel": f"{args.op}_{args.mode}", "rows": R, "cols": C, "ms": round(ms, 5),
                      "gbs": round(nbytes / ms / 1e6, 1)}), flush=True)


def peak(args):
    """Sustained MFMA rate with register operands only (the clocks the device really runs)."""
    import ctypes
    import os
    from .build import PEAK_LIB

    if not os.path.exists(PEAK_LIB):
        raise RuntimeError(f"{PEAK_LIB} missing: run __graft_entry__.build()")
    L = ctypes.CDLL(PEAK_LIB)
    L.te_peak_launch.argtypes = [ctypes.c_int] * 3 + [ctypes.c_void_p] * 3
    dev = "cuda:0"
    seed = torch.zeros(1, dtype=torch.int32, device=dev)
    blocks = 256 * args.waves_per_cu  # one 4-wave block per CU per wave slot
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for kind in ("fp8", "bf16"):
        bf = 1 if kind == "bf16" else 0
        fn = lambda: L.te_peak_launch(bf, blocks, args.iters, ctypes.c_void_p(seed.data_ptr()),  # noqa: E731
                                      ctypes.c_void_p(out.data_ptr()), st)
        ms = _time(fn, 5, 2)
        flop_per_mfma = 2 * 32 * 32 * (16 if bf else 64)
        fl = float(blocks) * 4 * args.iters * 16 * flop_per_mfma
        print(json.dumps({"kernel": f"mfma_peak_{kind}", "ms": round(ms, 4), "tflops": round(fl / ms / 1e9, 1)}),
              flush=True)


def main():
    p = argparse.ArgumentParser()
    sub = p.add_subparsers(dest="cmd", required=True)
    g = sub.add_parser("gemm")
    g.add_argument("--m", type=int, default=15872)
    g.add_argument("--n", type=int, default=12288)
    g.add_argument("--k", type=int, default=4096)
    g.add_argument("--kind", choices=["fp8", "mx", "bf16"], default="fp8")
    g.add_argument("--fa", default="E4M3")
    g.add_argument("--fb", default="E4M3")
    g.add_argument("--out", choices=["bf16", "f32"], default="bf16")
    g.add_argument("--iters", type=int, default=20)
    g.add_argument("--warmup", type=int, default=3)
    c = sub.add_parser("cast")
    c.add_argument("--rows", type=int, default=15872)
    c.add_argument("--cols", type=int, default=16384)
    c.add_argument("--op", choices=["cast", "transpose", "both", "mx"], default="cast")
    c.add_argument("--mode", choices=["delayed", "current"], default="delayed")
    c.add_argument("--iters", type=int, default=20)
    c.add_argument("--warmup", type=int, default=3)
    k = sub.add_parser("peak")
    k.add_argument("--iters", type=int, default=4096)
    k.add_argument("--waves-per-cu", type=int, default=1)
    args = p.parse_args()
    torch.cuda.set_device(0)
    {"gemm": gemm, "cast": cast, "peak": peak}[args.cmd](args)


if __name__ == "__main__":
    main()
