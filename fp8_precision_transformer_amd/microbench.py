"""Microbenchmarks of single library kernels, for profiling (rocprofv3) and tuning.

    python -m fp8_precision_transformer_amd.microbench gemm --m 15872 --n 12288 --k 4096
    python -m fp8_precision_transformer_amd.microbench cast --rows 15872 --cols 16384
    python -m fp8_precision_transformer_amd.microbench layer --kind fp8
    python -m fp8_precision_transformer_amd.microbench copy --mib 1024

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
        if args.kind == "mx4":  # packed E2M1 pairs: every byte is a valid pair of codes
            a = torch.randint(0, 256, (m, k // 2), device=dev, generator=g, dtype=torch.int32).to(torch.uint8)
            b = torch.randint(0, 256, (n, k // 2), device=dev, generator=g, dtype=torch.int32).to(torch.uint8)
            fa = fb = "E2M1"
        if args.kind in ("mx", "mx4"):
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


def _operands(kind, m, n, k, g, dev, fa="E4M3", fb="E4M3"):
    """Random operands of one GEMM drawn on the GPU: finite mid-range FP8 codes with
    random signs (unit MX scales), or bf16 normals."""
    if kind == "bf16":
        a = torch.randn((m, k), device=dev, generator=g).to(torch.bfloat16)
        b = (torch.randn((n, k), device=dev, generator=g) * 0.02).to(torch.bfloat16)
        return a, "BF16", None, b, "BF16", None, B.TE_GRAN_TENSOR

    def codes(r, c):
        return (torch.randint(0x18, 0x48, (r, c), device=dev, generator=g, dtype=torch.int32) |
                (torch.randint(0, 2, (r, c), device=dev, generator=g, dtype=torch.int32) << 7)).to(torch.uint8)
    def unit_scales(rows, panel):  # E8M0 127 in the row-major or the panel layout
        if panel:
            return torch.full((B.te_mx_scale_panel_bytes(rows, k),), 127, dtype=torch.uint8, device=dev)
        return torch.full((rows, k // 32), 127, dtype=torch.uint8, device=dev)
    panel = kind in ("mxp", "mx4p")
    gran = B.TE_GRAN_MX_BLOCK32_PANEL if panel else B.TE_GRAN_MX_BLOCK32
    if kind in ("mx4", "mx4p"):  # packed E2M1 pairs: every byte is a valid pair of codes
        a = torch.randint(0, 256, (m, k // 2), device=dev, generator=g, dtype=torch.int32).to(torch.uint8)
        b = torch.randint(0, 256, (n, k // 2), device=dev, generator=g, dtype=torch.int32).to(torch.uint8)
        return a, "E2M1", unit_scales(m, panel), b, "E2M1", unit_scales(n, panel), gran
    a, b = codes(m, k), codes(n, k)
    if kind in ("mx", "mxp"):
        return a, fa, unit_scales(m, panel), b, fb, unit_scales(n, panel), gran
    one = torch.ones(1, dtype=torch.float32, device=dev)
    return a, fa, one, b, fb, one, B.TE_GRAN_TENSOR


def layer(args):
    """The 12 GEMMs of the CodonFM-5B-shaped layer (Fprop E4M3 x E4M3, Dgrad and Wgrad
    E5M2 x E4M3 for the per-tensor kind), each launched --iters times; one JSON line per
    GEMM and one for the layer (sum of medians)."""
    from .shapes import CODONFM_5B, layer_gemms
    dev = "cuda:0"
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    total_ms, total_fl = 0.0, 0.0
    for gm in layer_gemms(CODONFM_5B):
        fa = "E4M3" if (gm.stage == "fprop" or args.kind != "fp8") else "E5M2"
        a, fa, sa, b, fb, sb, gran = _operands(args.kind, gm.m, gm.n, gm.k, g, dev, fa, "E4M3")
        d = torch.empty((gm.m, gm.n), dtype=torch.bfloat16, device=dev)
        ms = _time(lambda: B.te_fp8_gemm(a, fa, sa, b, fb, sb, d, gran=gran), args.iters, args.warmup)
        total_ms += ms
        total_fl += gm.flops
        print(json.dumps({"kernel": f"gemm_{args.kind}", "gemm": f"{gm.weight}.{gm.stage}", "m": gm.m, "n": gm.n,
                          "k": gm.k, "ms": round(ms, 5), "tflops": round(gm.flops / ms / 1e9, 1)}), flush=True)
        del a, b, d
    print(json.dumps({"kernel": f"gemm_{args.kind}", "gemm": "layer", "ms": round(total_ms, 4),
                      "tflops": round(total_fl / total_ms / 1e9, 1)}), flush=True)


def lib(args):
    """The same 12 layer GEMMs through the vendor library (torch._scaled_mm -> hipBLASLt
    for FP8, torch.matmul for BF16): a timing reference beside this library's kernels,
    not part of its path."""
    from .shapes import CODONFM_5B, layer_gemms
    dev = "cuda:0"
    total_ms, total_fl = 0.0, 0.0
    one = torch.ones((), dtype=torch.float32, device=dev)
    for gm in layer_gemms(CODONFM_5B):
        a = torch.randn((gm.m, gm.k), device=dev).to(torch.bfloat16)
        b = (torch.randn((gm.n, gm.k), device=dev) * 0.02).to(torch.bfloat16)
        if args.kind == "fp8":
            fa = torch.float8_e4m3fn if (gm.stage == "fprop" or not args.hybrid) else torch.float8_e5m2
            a8, b8 = a.to(fa), b.to(torch.float8_e4m3fn)
            fn = lambda: torch._scaled_mm(a8, b8.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16)  # noqa: E731
        else:
            bt = b.t()
            fn = lambda: torch.matmul(a, bt)  # noqa: E731
        ms = _time(fn, args.iters, args.warmup)
        total_ms += ms
        total_fl += gm.flops
        print(json.dumps({"kernel": f"lib_{args.kind}", "gemm": f"{gm.weight}.{gm.stage}", "ms": round(ms, 5),
                          "tflops": round(gm.flops / ms / 1e9, 1)}), flush=True)
    print(json.dumps({"kernel": f"lib_{args.kind}", "gemm": "layer", "ms": round(total_ms, 4),
                      "tflops": round(total_fl / total_ms / 1e9, 1)}), flush=True)


def _peak_lib():
    import ctypes
    import os
    from .build import PEAK_LIB

    if not os.path.exists(PEAK_LIB):
        raise RuntimeError(f"{PEAK_LIB} missing: run __graft_entry__.build()")
    L = ctypes.CDLL(PEAK_LIB)
    L.te_peak_launch.argtypes = [ctypes.c_int] * 3 + [ctypes.c_void_p] * 3
    L.te_copy_launch.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    L.te_read_launch.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    L.te_stream_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    return L


def stream(args):
    """The streaming ceiling study (k_stream): copy, cast-shaped (read 2 : write 1, the
    bf16 -> FP8 ratio), read-only and write-only streams of --mib MiB of input, with 1, 2,
    4 or 8 chunks of 16 bytes per lane in flight, cached or nontemporal loads and
    stores (nt bit 0: loads, bit 1: stores), over grid sizes of 1 to 16 blocks of 256
    lanes per CU.  One JSON line per run, then the
    best configuration of each kind."""
    import ctypes
    L = _peak_lib()
    dev = "cuda:0"
    n = args.mib * (1 << 20)
    src = torch.ones(n // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ps, pd = ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr())
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    moved = {0: 2 * n, 1: n + n // 2, 2: n, 3: n}
    names = {0: "copy", 1: "cast_shaped", 2: "read", 3: "write"}
    best = {}
    for kind in (0, 1, 2, 3):
        for u in (1, 2, 4, 8):
            for nt in ((0, 1, 2, 3) if kind < 2 else (0, 3)):
                for per_cu in (1, 2, 4, 8, 16):
                    grid = per_cu * cus

                    def fn():
                        if L.te_stream_launch(kind, u, nt, ps, pd, n // 16, grid, st):
                            raise RuntimeError("te_stream_launch failed")
                    ms = _time(fn, args.iters, args.warmup)
                    rec = {"kernel": "k_stream", "kind": names[kind], "u": u, "nt": nt, "grid": grid,
                           "bytes": moved[kind], "ms": round(ms, 5), "gbs": round(moved[kind] / ms / 1e6, 1)}
                    print(json.dumps(rec), flush=True)
                    if rec["gbs"] > best.get(names[kind], {"gbs": 0})["gbs"]:
                        best[names[kind]] = rec
    print(json.dumps({"best": best}), flush=True)


def copy(args):
    """A plain device copy (k_copy, 16 bytes per lane) of --mib MiB: the known-size
    reference that HBM byte counters are calibrated against.  With --sweep it also
    times the copy and a read-only stream (k_read) over several grid sizes: the
    practical streaming rates a memory-bound kernel on this chip can reach."""
    import ctypes
    L = _peak_lib()
    dev = "cuda:0"
    n = args.mib * (1 << 20)
    src = torch.ones(n // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ps, pd = ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr())
    for grid in ([0] + ([1024, 2048, 4096, 8192] if args.sweep else [])):
        ms = _time(lambda: L.te_copy_launch(ps, pd, n // 16, grid, st), args.iters, args.warmup)
        print(json.dumps({"kernel": "k_copy", "grid": grid or min(4096, n // 4096), "bytes_read": n,
                          "bytes_written": n, "ms": round(ms, 5), "gbs": round(2 * n / ms / 1e6, 1)}), flush=True)
    assert torch.equal(src, dst)
    if args.sweep:
        for grid in (1024, 2048, 4096, 8192):
            ms = _time(lambda: L.te_read_launch(ps, pd, n // 16, grid, st), args.iters, args.warmup)
            print(json.dumps({"kernel": "k_read", "grid": grid, "bytes_read": n, "bytes_written": 0,
                              "ms": round(ms, 5), "gbs": round(n / ms / 1e6, 1)}), flush=True)


def cast(args):
    dev = "cuda:0"
    x = torch.randn((args.rows, args.cols), device=dev).to(torch.bfloat16)
    R, C = args.rows, args.cols
    scale = torch.ones(1, device=dev)
    si = torch.empty(1, device=dev)
    am = torch.empty(1, device=dev)
    mode = B.TE_SCALE_CURRENT if args.mode == "current" else B.TE_SCALE_DELAYED
    wsa = B.amax_workspace(torch.device(dev))
    if args.op == "cast":
        out = torch.empty((R, C), dtype=torch.uint8, device=dev)
        fn = lambda: B.te_amax_cast(x, "E4M3", mode, 0, scale, si, am, out, workspace=wsa)  # noqa: E731
        nbytes = R * C * (5 if mode == B.TE_SCALE_CURRENT else 3)
    elif args.op == "transpose":
        out = torch.empty((C, R), dtype=torch.uint8, device=dev)
        fn = lambda: B.te_cast_transpose(x, "E4M3", mode, 0, scale, si, am, None, out, workspace=wsa)  # noqa: E731
        nbytes = R * C * (5 if mode == B.TE_SCALE_CURRENT else 3)
    elif args.op == "both":
        o1 = torch.empty((R, C), dtype=torch.uint8, device=dev)
        o2 = torch.empty((C, R), dtype=torch.uint8, device=dev)
        fn = lambda: B.te_cast_transpose(x, "E4M3", mode, 0, scale, si, am, o1, o2, workspace=wsa)  # noqa: E731
        nbytes = R * C * (6 if mode == B.TE_SCALE_CURRENT else 4)
    elif args.op == "bothdbias":  # both copies plus the bias gradient (column sums) of x
        o1 = torch.empty((R, C), dtype=torch.uint8, device=dev)
        o2 = torch.empty((C, R), dtype=torch.uint8, device=dev)
        db = torch.empty(C, dtype=torch.float32, device=dev)
        ws = B.dbias_workspace(R, C, torch.device(dev))
        fn = lambda: B.te_cast_transpose_dbias(x, "E5M2", mode, 0, scale, si, am, db, ws, o1, o2)  # noqa: E731
        nbytes = R * C * (6 if mode == B.TE_SCALE_CURRENT else 4) + C * 4
    elif args.op == "ln":  # LayerNorm over the rows, written as FP8 codes
        out = torch.empty((R, C), dtype=torch.uint8, device=dev)
        g = torch.ones(C, device=dev)
        b = torch.zeros(C, device=dev)
        fn = lambda: B.te_layernorm_fp8(x, g, b, 1e-5, "E4M3", mode, 0, scale, si, am, out, workspace=wsa)  # noqa: E731
        nbytes = R * C * (5 if mode == B.TE_SCALE_CURRENT else 3)
    elif args.op == "mx":  # row-wise copy
        o1 = torch.empty((R, C), dtype=torch.uint8, device=dev)
        s1 = torch.empty((R, C // 32), dtype=torch.uint8, device=dev)
        fn = lambda: B.te_mxfp8_quantize(x, "E4M3", o1, s1)  # noqa: E731
        nbytes = R * C * 3 + R * C // 32
    elif args.op == "mxcol":  # column-wise copy
        o2 = torch.empty((C, R), dtype=torch.uint8, device=dev)
        s2 = torch.empty((C, R // 32), dtype=torch.uint8, device=dev)
        fn = lambda: B.te_mxfp8_quantize(x, "E4M3", None, None, o2, s2)  # noqa: E731
        nbytes = R * C * 3 + R * C // 32
    elif args.op in ("mx4", "mx4col", "mx4both"):  # MXFP4: row-wise, column-wise or both copies
        row, col = args.op in ("mx4", "mx4both"), args.op in ("mx4col", "mx4both")
        o1 = torch.empty((R, C // 2), dtype=torch.uint8, device=dev) if row else None
        s1 = torch.empty((R, C // 32), dtype=torch.uint8, device=dev) if row else None
        o2 = torch.empty((C, R // 2), dtype=torch.uint8, device=dev) if col else None
        s2 = torch.empty((C, R // 32), dtype=torch.uint8, device=dev) if col else None
        fn = lambda: B.te_mxfp4_quantize(x, o1, s1, o2, s2)  # noqa: E731
        nbytes = R * C * 2 + (int(row) + int(col)) * (R * C // 2 + R * C // 32)
    elif args.op.startswith("mxp") or args.op.startswith("mx4p"):  # panel-layout scales: row, col or both
        fp4 = args.op.startswith("mx4p")
        kind = args.op[4:] if fp4 else args.op[3:]
        row, col = kind in ("", "both"), kind in ("col", "both")
        eb = 2 if fp4 else 1
        o1 = torch.empty((R, C // eb), dtype=torch.uint8, device=dev) if row else None
        s1 = torch.empty(B.te_mx_scale_panel_bytes(R, C), dtype=torch.uint8, device=dev) if row else None
        o2 = torch.empty((C, R // eb), dtype=torch.uint8, device=dev) if col else None
        s2 = torch.empty(B.te_mx_scale_panel_bytes(C, R), dtype=torch.uint8, device=dev) if col else None
        if fp4:
            fn = lambda: B.te_mxfp4_quantize_panel(x, o1, s1, o2, s2)  # noqa: E731
        else:
            fn = lambda: B.te_mxfp8_quantize_panel(x, "E4M3", o1, s1, o2, s2)  # noqa: E731
        nbytes = R * C * 2 + (int(row) + int(col)) * (R * C // eb + R * C // 32)
    else:  # mxboth
        o1 = torch.empty((R, C), dtype=torch.uint8, device=dev)
        s1 = torch.empty((R, C // 32), dtype=torch.uint8, device=dev)
        o2 = torch.empty((C, R), dtype=torch.uint8, device=dev)
        s2 = torch.empty((C, R // 32), dtype=torch.uint8, device=dev)
        fn = lambda: B.te_mxfp8_quantize(x, "E4M3", o1, s1, o2, s2)  # noqa: E731
        nbytes = R * C * 4 + 2 * (R * C // 32)
    ms = _time(fn, args.iters, args.warmup)
    print(json.dumps({"kernel": f"{args.op}_{args.mode}", "rows": R, "cols": C, "ms": round(ms, 5),
                      "gbs": round(nbytes / ms / 1e6, 1)}), flush=True)


def peak(args):
    """Sustained MFMA rate with register operands only (the clocks the device really runs)."""
    import ctypes
    L = _peak_lib()
    dev = "cuda:0"
    seed = torch.zeros(1, dtype=torch.int32, device=dev)
    blocks = 256 * args.waves_per_cu  # one 4-wave block per CU per wave slot
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    kinds = ((0, "fp8"), (1, "bf16"), (2, "mxfp8"), (3, "mxfp4"), (4, "fp8_32x32x64_changing_operands"),
             (5, "fp8_16x16x128_changing_operands"))
    for code, kind in kinds * args.repeat:  # later passes run at the clocks the first settled
        bf = code == 1
        fn = lambda: L.te_peak_launch(code, blocks, args.iters, ctypes.c_void_p(seed.data_ptr()),  # noqa: E731
                                      ctypes.c_void_p(out.data_ptr()), st)
        ms = _time(fn, 5, 2)
        flop_per_mfma = 2 * 32 * 32 * (16 if bf else 64)
        # k_peak: 16 instructions per iteration; k_peak_rand: 8 x 16 of 32x32x64 or the same
        # FLOP in 8 x 32 of 16x16x128
        fl = float(blocks) * 4 * args.iters * (128 if code >= 4 else 16) * flop_per_mfma
        print(json.dumps({"kernel": f"mfma_peak_{kind}", "ms": round(ms, 4), "tflops": round(fl / ms / 1e9, 1)}),
              flush=True)


def main():
    p = argparse.ArgumentParser()
    sub = p.add_subparsers(dest="cmd", required=True)
    g = sub.add_parser("gemm")
    g.add_argument("--m", type=int, default=15872)
    g.add_argument("--n", type=int, default=12288)
    g.add_argument("--k", type=int, default=4096)
    g.add_argument("--kind", choices=["fp8", "mx", "mx4", "bf16"], default="fp8")
    g.add_argument("--fa", default="E4M3")
    g.add_argument("--fb", default="E4M3")
    g.add_argument("--out", choices=["bf16", "f32"], default="bf16")
    g.add_argument("--iters", type=int, default=20)
    g.add_argument("--warmup", type=int, default=3)
    c = sub.add_parser("cast")
    c.add_argument("--rows", type=int, default=15872)
    c.add_argument("--cols", type=int, default=16384)
    c.add_argument("--op", choices=["cast", "transpose", "both", "bothdbias", "ln", "mx", "mxcol", "mxboth", "mx4",
                                    "mx4col", "mx4both", "mxp", "mxpcol", "mxpboth", "mx4p", "mx4pcol", "mx4pboth"],
                   default="cast")
    c.add_argument("--mode", choices=["delayed", "current"], default="delayed")
    c.add_argument("--iters", type=int, default=20)
    c.add_argument("--warmup", type=int, default=3)
    ly = sub.add_parser("layer")
    ly.add_argument("--kind", choices=["fp8", "mx", "mxp", "mx4", "mx4p", "bf16"], default="fp8")
    ly.add_argument("--iters", type=int, default=10)
    ly.add_argument("--warmup", type=int, default=2)
    lb = sub.add_parser("lib")
    lb.add_argument("--kind", choices=["fp8", "bf16"], default="fp8")
    lb.add_argument("--hybrid", action="store_true", help="E5M2 left operand for Dgrad/Wgrad")
    lb.add_argument("--iters", type=int, default=10)
    lb.add_argument("--warmup", type=int, default=2)
    cp = sub.add_parser("copy")
    cp.add_argument("--mib", type=int, default=1024)
    cp.add_argument("--iters", type=int, default=10)
    cp.add_argument("--warmup", type=int, default=2)
    cp.add_argument("--sweep", action="store_true", help="also time copy and read-only streams over grid sizes")
    sm = sub.add_parser("stream")
    sm.add_argument("--mib", type=int, default=2048)
    sm.add_argument("--iters", type=int, default=5)
    sm.add_argument("--warmup", type=int, default=1)
    k = sub.add_parser("peak")
    k.add_argument("--iters", type=int, default=4096)
    k.add_argument("--waves-per-cu", type=int, default=1)
    k.add_argument("--repeat", type=int, default=2)
    args = p.parse_args()
    torch.cuda.set_device(0)
    {"gemm": gemm, "cast": cast, "peak": peak, "layer": layer, "copy": copy, "lib": lib, "stream": stream}[args.cmd](args)


if __name__ == "__main__":
    main()
