"""Shape ablations of gemm_bf16_nt on the GPU (measurement tool, not a test).

    python -m dense_gemm_14_amd.ablation instances [--csv FILE]
    python -m dense_gemm_14_amd.ablation supergroup [--csv FILE]
    python -m dense_gemm_14_amd.ablation streams [--csv FILE]
    python -m dense_gemm_14_amd.ablation mx_supergroup [--csv FILE]

``instances`` times the three BF16 instances (forced through
gemm355_force_instance) and the automatic choice on the shape grid
M, N, K in {1024, 2048, 4096, 8192, 16384} that the NVFP4 page ablates its
configurations over ("NVFP4 GEMM on Blackwell", "Production Kernel"),
restricted to shapes with fewer 256 x 256 tiles than 256, plus skinny and mid
shapes. ``supergroup`` times the band width of the visiting order
(gemm355_force_supergroup; the page's "Supergroup Size" ablation) on the
large shapes M, N in {4096, 8192, 16384}, K in {1024, 4096, 16384}.
``streams`` times independent back-to-back products issued on one stream
against the same products alternating over two streams, which lets one
product's workgroups start on units the other's tail leaves idle (the
question of "Kernel 6", "The Gap Between Grids", without programmatic
dependent launch). ``mx_supergroup`` times the band width for the
microscaled FP4 product (gemm_mxfp4_nt; same 256 x 256 tiles, a quarter of
the operand bytes per tile) at 8192^3 and 16384 x 16384 x 8192.

Every configuration of a shape is timed in three round-robin passes and the
minimum kept (the first configuration timed on fresh buffers runs slow).
Operands are standard-normal values rounded to BF16, rotated over enough sets
to exceed 512 MiB so that they come from HBM, not the last-level cache.
"""
from __future__ import annotations

import argparse
import sys

import torch

import dense_gemm_14_amd as g

GRID = [1024, 2048, 4096, 8192, 16384]
EXTRA = [(64, 4096, 8192), (128, 2048, 8192), (256, 1024, 8192), (512, 4096, 8192), (128, 8192, 8192),
         (128, 8192, 2048), (256, 256, 256), (1992, 2040, 2056), (3072, 3072, 3072), (2560, 2560, 4096),
         (1536, 1536, 8192)]
WIDTHS = [1, 2, 4, 8, 16, 32, 64]


def _sets(M, N, K):
    per = 2 * (M * K + N * K + M * N)
    n = max(1, -(-(600 << 20) // per))
    return [(torch.randn(M, K, device="cuda").to(torch.bfloat16), torch.randn(N, K, device="cuda").to(torch.bfloat16),
             torch.empty(M, N, device="cuda", dtype=torch.bfloat16)) for _ in range(n)]


def _time_us(M, N, K, sets, target_ms=20.0):
    n = len(sets)
    for i in range(2):
        A, B, C = sets[i % n]
        g.gemm_bf16_nt(M, N, K, A, B, C)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    A, B, C = sets[0]
    g.gemm_bf16_nt(M, N, K, A, B, C)
    e1.record()
    torch.cuda.synchronize()
    reps = max(3, min(100, int(target_ms / max(e0.elapsed_time(e1), 1e-3))))
    e0.record()
    for i in range(reps):
        A, B, C = sets[i % n]
        g.gemm_bf16_nt(M, N, K, A, B, C)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps * 1e3


def _run(shape, configs):
    """Min over three round-robin passes of each (instance, width) config."""
    M, N, K = shape
    sets = _sets(M, N, K)
    best = {}
    try:
        for _ in range(3):
            for inst, width in configs:
                g.force_instance(inst)
                g.force_supergroup(width)
                t = _time_us(M, N, K, sets)
                best[(inst, width)] = min(best.get((inst, width), float("inf")), t)
    finally:
        g.force_instance(g.INSTANCE_AUTO)
        g.force_supergroup(0)
    del sets
    torch.cuda.empty_cache()
    return best


def instances(csv):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    shapes = [(M, N, K) for M in GRID for N in GRID for K in GRID if -(-M // 256) * -(-N // 256) < 256] + EXTRA
    worst = 1.0
    print("#     M      N      K  plan(inst,splits)   auto  i1(256)  i2(64)  i3(128/split)  auto/best   [us]")
    for shp in shapes:
        r = _run(shp, [(g.INSTANCE_LARGE, 0), (g.INSTANCE_SMALL, 0), (g.INSTANCE_SPLITK, 0), (g.INSTANCE_AUTO, 0)])
        best = min(r.values())
        ratio = r[(0, 0)] / best
        worst = max(worst, ratio)
        print("%7d %6d %6d  %-17s %7.1f %8.1f %7.1f %14.1f  %9.3f" % (
            *shp, g.bf16_plan(*shp, cus), r[(0, 0)], r[(1, 0)], r[(2, 0)], r[(3, 0)], ratio), flush=True)
        if csv:
            for (inst, _), us in r.items():
                csv.write("%d,%d,%d,%d,%.2f\n" % (*shp, inst, us))
    print("# worst automatic choice / fastest instance: %.3f over %d shapes" % (worst, len(shapes)))


def supergroup(csv):
    L = [4096, 8192, 16384]
    print("#     M      N      K  " + " ".join("%8s" % ("w=%d" % w) for w in WIDTHS) + "   best  best/w8   [us]")
    for shp in [(M, N, K) for M in L for N in L for K in (1024, 4096, 16384)]:
        r = _run(shp, [(g.INSTANCE_LARGE, w) for w in WIDTHS])
        b = min(r, key=r.get)
        print("%7d %6d %6d  " % shp + " ".join("%8.1f" % r[(1, w)] for w in WIDTHS) +
              "  %5d  %7.3f" % (b[1], r[b] / r[(1, 8)]), flush=True)
        if csv:
            for (_, w), us in r.items():
                csv.write("%d,%d,%d,%d,%.2f\n" % (*shp, w, us))


STREAM_SHAPES = [(8192, 8192, 8192), (4096, 4096, 4096), (3072, 3072, 3072), (2048, 2048, 2048),
                 (128, 8192, 8192), (8192, 8192, 1024)]


def streams(csv):
    s0 = torch.cuda.current_stream()
    s1 = torch.cuda.Stream()
    print("#     M      N      K   one stream   two streams   gain   [us per product, min of 3 passes]")
    for M, N, K in STREAM_SHAPES:
        sets = _sets(M, N, K)
        n = len(sets)
        reps = 200 if M * N * K < 1e11 else 100
        best = {}
        for _ in range(3):
            for mode in ("one", "two"):
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(s0)
                s1.wait_event(e0)
                for i in range(reps):
                    A, B, C = sets[i % n]
                    g.gemm_bf16_nt(M, N, K, A, B, C, stream=s1 if (mode == "two" and i % 2) else s0)
                done = torch.cuda.Event()
                done.record(s1)
                s0.wait_event(done)
                e1.record(s0)
                torch.cuda.synchronize()
                best[mode] = min(best.get(mode, float("inf")), e0.elapsed_time(e1) / reps * 1e3)
        print("%7d %6d %6d  %10.1f  %12.1f  %+5.1f%%" % (M, N, K, best["one"], best["two"],
                                                        100 * (best["one"] / best["two"] - 1)), flush=True)
        if csv:
            csv.write("%d,%d,%d,%.2f,%.2f\n" % (M, N, K, best["one"], best["two"]))
        del sets
        torch.cuda.empty_cache()


def _mx_sets(M, N, K):
    import synthetic as syn
    per = M * K // 2 + M * K // 32 + N * K // 2 + N * K // 32 + 2 * M * N
    n = max(2, -(-(600 << 20) // per))
    sets = []
    for s in range(n):
        Aq, SA = syn.mxfp4_operand(M, K, 10 + s)
        Bq, SB = syn.mxfp4_operand(N, K, 20 + s)
        sets.append([torch.from_numpy(x).cuda() for x in (Aq, SA, Bq, SB)] +
                    [torch.empty(M * N, dtype=torch.int16, device="cuda")])
    return sets


def mx_supergroup(csv):
    widths = [2, 4, 8, 16, 32]
    print("#     M      N      K  " + " ".join("%8s" % ("w=%d" % w) for w in widths) + "   best  best/w8   [us]")
    for M, N, K in [(8192, 8192, 8192), (16384, 16384, 8192)]:
        sets = _mx_sets(M, N, K)
        n = len(sets)
        best = {}
        try:
            for _ in range(3):
                for w in widths:
                    g.force_supergroup(w)
                    for i in range(4):
                        g.gemm_mxfp4_nt(M, N, K, *sets[i % n])
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    reps = 100 if M * N < 1e8 else 30
                    e0.record()
                    for i in range(reps):
                        g.gemm_mxfp4_nt(M, N, K, *sets[i % n])
                    e1.record()
                    torch.cuda.synchronize()
                    best[w] = min(best.get(w, float("inf")), e0.elapsed_time(e1) / reps * 1e3)
        finally:
            g.force_supergroup(0)
        b = min(best, key=best.get)
        print("%7d %6d %6d  " % (M, N, K) + " ".join("%8.1f" % best[w] for w in widths) +
              "  %5d  %7.3f" % (b, best[b] / best[8]), flush=True)
        if csv:
            for w, us in best.items():
                csv.write("%d,%d,%d,%d,%.2f\n" % (M, N, K, w, us))
        del sets
        torch.cuda.empty_cache()


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("what", choices=["instances", "supergroup", "streams", "mx_supergroup"])
    ap.add_argument("--csv", default=None, help="also write M,N,K,config,us rows here")
    args = ap.parse_args(argv)
    if not torch.cuda.is_available():
        sys.exit("the ablation needs a GPU")
    csv = open(args.csv, "w") if args.csv else None
    try:
        {"instances": instances, "supergroup": supergroup, "streams": streams,
         "mx_supergroup": mx_supergroup}[args.what](csv)
    finally:
        if csv:
            csv.close()


if __name__ == "__main__":
    main()
