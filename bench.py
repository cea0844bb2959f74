#!/usr/bin/env python3
"""Throughput of libgemm355 on one MI355X: TFLOP/s of C = A * B^T.

Default workload: BF16 M = N = K = 8192 (inputs i.i.d. uniform[-1, 1] rounded
to BF16, FP32 accumulation, BF16 output), rotating between enough input sets
that the footprint exceeds twice the 256 MiB last-level cache (the
measurement method of "NVFP4 GEMM on Blackwell", section "Benchmarking":
separate warm-up and timed iterations, buffer rotation, uniform data).

A step is one call of the library's entry point on one input set that is
already resident in device memory. W warm-up steps run first; if they took
less than --warm-seconds of wall time, more untimed steps follow until they
have (the board's clock and power settle within about a second of sustained
load; the extra steps are reported in their own field and `warmup` stays W).
Then exactly K timed steps run, bracketed by device synchronisation; HIP
events recorded on the launch stream time them. A second pass times each of
--launch-samples launches with its own event pair, for the spread. The GPU
clock and socket power are sampled (amdsmi gpu_metrics) during both passes.
One JSON line goes to stdout:
  value      TFLOP/s over the K timed steps (2 M N K per step);
  roofline   the kernel's achieved TFLOP/s (algorithmic FLOPs per launch over
             the mean launch duration of the timed steps) against the dense
             peak of its operand type, plus the L2-egress traffic per launch
             (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy) from the
             committed rocprofv3 counter summary when it was taken from the
             current kernel source;
  launch_ms  mean, p10, p50, p90, min, max of the per-launch pass;
  clock      mean GPU clock (MHz, over the XCDs) and socket power (W) sampled
             during the timed steps and during the per-launch pass;
  cpu_baseline  the plain CPU oracle timed on a bounded sample of the same
             workload's output elements on this host's cores.

--parity-full compares every element of set 0's C with the oracle (minutes of
CPU time at 8192^3) and adds the result to the line.

Other workloads (--workload): bf16_4096, bf16_8000, bf16_skinny (128 x 8192 x
8192, HBM roofline), bf16_256, fp4_8192 (E2M1 + E4M3 per 16, decoded to FP16),
bf16_gelu_8192 (bias + GELU fused), mx_8192 (E2M1 + E8M0 per 32 on the scaled
FP4 matrix instructions, against the FP4 peak), fp4_ws_8192 (the NVFP4 product
through gemm_nvfp4_nt_ws: decoded once into a BF16 workspace allocated before
the timing, then the BF16 kernels).

Only one GPU is used; --gpus above 1 exits with a message.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

LLC_BYTES = 256 << 20                  # MI355X Infinity Cache (last-level cache)
# Dense matrix-core peaks of MI355X (the datasheet's 2.5 PFLOP/s BF16/FP16 and
# 10.1 PFLOP/s FP4, exactly: 256 CUs x 2.4 GHz x 4096 BF16 FLOP per clock, and
# four times that for FP4)
PEAK_TFLOPS = {"bf16": 2516.58, "fp16": 2516.58, "fp4": 10066.33}
HBM_PEAK_GBS = 8000.0

WORKLOADS = {
    # name: (kind, M, N, K)
    "bf16_8192": ("bf16", 8192, 8192, 8192),
    "bf16_4096": ("bf16", 4096, 4096, 4096),
    "bf16_8000": ("bf16", 8000, 8000, 8000),
    "bf16_skinny": ("bf16", 128, 8192, 8192),
    "bf16_256": ("bf16", 256, 256, 256),
    "fp4_8192": ("fp4", 8192, 8192, 8192),
    # the same product with the fused epilogue: C = gelu(A B^T + bias)
    "bf16_gelu_8192": ("bf16_gelu", 8192, 8192, 8192),
    # microscaled FP4 (E2M1 codes, E8M0 scale per 32) on the scaled matrix instructions
    "mx_8192": ("mx", 8192, 8192, 8192),
    # the NVFP4 product through gemm_nvfp4_nt_ws: decoded once into a BF16
    # workspace (allocated before timing), then the BF16 kernels
    "fp4_ws_8192": ("fp4_ws", 8192, 8192, 8192),
}
CONFIG_INDEX = {"bf16_256": 0, "bf16_4096": 1, "bf16_8192": 2, "bf16_8000": 3, "bf16_skinny": 3,
                "fp4_8192": 4, "bf16_gelu_8192": 2, "mx_8192": 4, "fp4_ws_8192": 4}
# BF16 kernels are templates over the epilogue: -1 plain, 2 bias + tanh-form GELU
# (the 256 x 256 kernel also over whether K has a tail past a multiple of 64)
KERNEL_NAME = {"bf16": "gemm355::bf16::gemm_bf16_nt_kernel<%d, %s>", "fp4": "gemm355::fp4::gemm_nvfp4_nt_kernel",
               "mx": "gemm355::mx::gemm_mxfp4_nt_kernel<-1>",
               "bf16_small": "gemm355::bf16_small::gemm_bf16_nt_small_kernel<%d>",
               "bf16_small_long": "gemm355::bf16_small_long::gemm_bf16_nt_small_long_kernel<%d, 4>",
               "bf16_splitk": "gemm355::bf16_splitk::gemm_bf16_nt_splitk_kernel<%d>",
               "bf16_splitk_reduce": "gemm355::bf16_splitk::splitk_reduce_kernel<%d>",
               "fp4_decode": "gemm355::fp4::decode_nvfp4_bf16_kernel"}
EPILOGUE = {"bf16": -1, "bf16_gelu": 2}


def kernels_for(kind: str, M: int, N: int, K: int, compute_units: int = 256) -> list:
    """The kernels gemm_bf16_nt / gemm_bf16_nt_bias_act / gemm_nvfp4_nt launch
    for this shape, in launch order (the library's own choice, gemm355_bf16_plan)."""
    if kind in ("fp4", "mx"):
        return [KERNEL_NAME[kind]]
    import dense_gemm_14_amd as g
    if kind == "fp4_ws":
        if not g.nvfp4_plan(M, N, K, compute_units)[0]:
            return [KERNEL_NAME["fp4"]]
        return [KERNEL_NAME["fp4_decode"]] + kernels_for("bf16", M, N, K, compute_units)
    instance, splits = g.bf16_plan(M, N, K, compute_units)
    epi = EPILOGUE[kind]
    if instance == 3:
        names = [KERNEL_NAME["bf16_splitk"] % epi]
        return names + [KERNEL_NAME["bf16_splitk_reduce"] % epi] if splits > 1 else names
    if instance == 2:   # the 64 x 64 instance's long-K staging (same rule as the library's)
        long_k = K >= 4096 and 2 * -(-M // 64) * -(-N // 64) >= compute_units
        return [KERNEL_NAME["bf16_small_long" if long_k else "bf16_small"] % epi]
    return [KERNEL_NAME["bf16"] % (epi, "true" if K % 64 else "false")]
PROFILE_DIR = os.path.join(ROOT, "profiles")


# the source file of each kernel family; a family's counters also depend on
# the shared helpers and the tile order
KERNEL_SOURCE = {"bf16": "gemm_bf16.hpp", "bf16_small": "gemm_bf16_small.hpp",
                 "bf16_small_long": "gemm_bf16_small_long.hpp", "bf16_splitk": "gemm_bf16_splitk.hpp",
                 "fp4": "gemm_fp4.hpp", "mx": "gemm_mxfp4.hpp"}
SHARED_SOURCES = ("common.hpp", "schedule.hpp")


def dominant_family(workload: str) -> str:
    """Kernel family (KERNEL_SOURCE key) of the first kernel the workload launches."""
    kind, M, N, K = WORKLOADS[workload]
    first = kernels_for(kind, M, N, K)[0]
    for fam in ("bf16_small_long", "bf16_small", "bf16_splitk", "fp4", "mx"):
        if KERNEL_NAME[fam].split("<")[0] in first:
            return fam
    return "bf16"


def kernel_source_hash(workload: str) -> str:
    """SHA-256 over the dominant kernel's source and the shared headers;
    counter figures are used only if it matches."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "dense_gemm_14_amd", "csrc")
    for name in (KERNEL_SOURCE[dominant_family(workload)],) + SHARED_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def launch_supergroup(workload: str) -> int:
    """Band width of the tile order the library uses for the workload's kernel."""
    import dense_gemm_14_amd as g
    kind, M, N, K = WORKLOADS[workload]
    fam = dominant_family(workload)
    tile = {"bf16_small": 64, "bf16_small_long": 64, "bf16_splitk": 128}.get(fam, 256)
    kernel = {"fp4": g.KERNEL_NVFP4, "mx": g.KERNEL_MXFP4, "bf16_small": g.KERNEL_BF16_SMALL,
              "bf16_small_long": g.KERNEL_BF16_SMALL}.get(fam, g.KERNEL_BF16)
    return g.supergroup(-(-N // tile), K, kernel)


def set_bytes(kind, M, N, K):
    if kind == "bf16":
        return 2 * (M * K + N * K + M * N)
    if kind == "bf16_gelu":
        return 2 * (M * K + N * K + M * N + N)   # plus the bias
    if kind == "mx":
        return M * K // 2 + M * K // 32 + N * K // 2 + N * K // 32 + 2 * M * N
    return M * K // 2 + M * K // 16 + N * K // 2 + N * K // 16 + 2 * M * N


def algorithmic_bytes(kind, M, N, K):
    """Compulsory traffic of one product: read the operands once, write C once."""
    return set_bytes(kind, M, N, K)


def make_sets(kind, M, N, K, n_sets, cfg):
    import numpy as np
    import torch
    import synthetic as syn
    sets = []
    for s in range(n_sets):
        seed = syn.seed_for(cfg, s)
        if kind in ("bf16", "bf16_gelu"):
            A = torch.from_numpy(syn.bf16_uniform(M, K, seed).view(np.int16)).cuda()
            B = torch.from_numpy(syn.bf16_uniform(N, K, seed + 500).view(np.int16)).cuda()
            ops = (A, B)
            if kind == "bf16_gelu":   # bias on the scale of the sums (sqrt(K / 9) = 30)
                bias = syn.bf16_uniform(1, N, seed + 900, lo=-32.0, hi=32.0)[0]
                ops = (A, B, torch.from_numpy(bias.view(np.int16)).cuda())
        else:
            operand = syn.mxfp4_operand if kind == "mx" else syn.fp4_operand   # fp4 and fp4_ws
            Aq, SFA = operand(M, K, seed)
            Bq, SFB = operand(N, K, seed + 500)
            ops = tuple(torch.from_numpy(x).cuda() for x in (Aq, SFA, Bq, SFB))
        C = torch.empty(M * N, dtype=torch.int16, device="cuda")
        sets.append((ops, C))
    return sets


def launcher(kind, M, N, K, stream):
    import dense_gemm_14_amd as g
    if kind == "bf16":
        return lambda ops, C: g.gemm_bf16_nt(M, N, K, ops[0], ops[1], C, stream=stream)
    if kind == "bf16_gelu":
        return lambda ops, C: g.gemm_bf16_nt_bias_act(M, N, K, ops[0], ops[1], ops[2], g.ACT_GELU_TANH, C,
                                                      stream=stream)
    if kind == "mx":
        return lambda ops, C: g.gemm_mxfp4_nt(M, N, K, *ops, C, stream=stream)
    if kind == "fp4_ws":
        import torch
        nbytes = g.nvfp4_workspace_size(M, N, K)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda") if nbytes else None
        return lambda ops, C: g.gemm_nvfp4_nt_ws(M, N, K, *ops, C, ws, nbytes, stream=stream)
    return lambda ops, C: g.gemm_nvfp4_nt(M, N, K, *ops, C, stream=stream)


def read_traffic(workload: str):
    """L2-egress bytes per launch (FETCH_SIZE + WRITE_SIZE, each scaled by a
    plain copy of known size) from the committed counter summary, or None when
    it was taken from another version of the kernel's source or with another
    tile-order band width. These counters count the bytes L2 requests from the
    fabric, which include hits in the 256 MiB last-level cache, so they bound
    the HBM bytes from above."""
    path = os.path.join(PROFILE_DIR, "traffic_%s.txt" % workload)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256") != kernel_source_hash(workload):
        return None
    if fields.get("supergroup") != str(launch_supergroup(workload)):
        return None
    try:
        return float(fields["l2_egress_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class ClockSampler:
    """Samples the GPU clock (mean over the XCDs' current gfx clocks) and the
    socket power from the driver's gpu_metrics table in a background thread,
    through the amdsmi Python module (read-only queries; no HIP calls)."""

    def __init__(self, period_s: float = 0.005):
        import threading
        self.period = period_s
        self.samples = []   # (time.perf_counter(), mhz, watts)
        self.error = None
        self._stop = threading.Event()
        self._thread = None
        self._handle = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            self._handle = self._match(amdsmi, handles)
            self._amdsmi = amdsmi
        except Exception as e:   # no driver access: the line then says why
            self.error = "%s: %s" % (type(e).__name__, e)

    @staticmethod
    def _match(amdsmi, handles):
        """The handle of torch's device 0 (by PCI bus), else the only one."""
        import torch
        if len(handles) == 1:
            return handles[0]
        props = torch.cuda.get_device_properties(0)
        bus = getattr(props, "pci_bus_id", None)
        for h in handles:
            bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)
            if bus is not None and int(bdf.split(":")[1], 16) == bus:
                return h
        return handles[0]

    def _read(self):
        m = self._amdsmi.amdsmi_get_gpu_metrics_info(self._handle)
        clks = m.get("current_gfxclks")
        vals = [c for c in clks if isinstance(c, (int, float)) and 0 < c < 10000] if isinstance(clks, list) else []
        if not vals and isinstance(m.get("current_gfxclk"), (int, float)):
            vals = [m["current_gfxclk"]]
        mhz = sum(vals) / len(vals) if vals else None
        w = m.get("current_socket_power")
        if not isinstance(w, (int, float)) or not 0 < w < 10000:
            w = m.get("average_socket_power")
        watts = w if isinstance(w, (int, float)) and 0 < w < 10000 else None
        return mhz, watts

    def _run(self):
        while not self._stop.is_set():
            try:
                mhz, watts = self._read()
                self.samples.append((time.perf_counter(), mhz, watts))
            except Exception as e:
                self.error = "%s: %s" % (type(e).__name__, e)
                return
            self._stop.wait(self.period)

    def start(self):
        import threading
        if self._handle is not None:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def stop(self):
        self._stop.set()
        if self._thread is not None:
            self._thread.join()

    def window(self, t0: float, t1: float):
        """Mean, min and max clock and mean power of the samples in [t0, t1]."""
        s = [x for x in self.samples if t0 <= x[0] <= t1]
        mhz = [x[1] for x in s if x[1] is not None]
        w = [x[2] for x in s if x[2] is not None]
        # the driver refreshes the table at a coarse interval: count the
        # distinct readings so a stale window shows as one
        out = {"samples": len(s), "distinct": len(set((x[1], x[2]) for x in s))}
        if mhz:
            out.update({"gfx_mhz_mean": round(sum(mhz) / len(mhz), 1), "gfx_mhz_min": round(min(mhz), 1),
                        "gfx_mhz_max": round(max(mhz), 1)})
        if w:
            out["socket_w_mean"] = round(sum(w) / len(w), 1)
        return out


def percentiles(xs):
    import numpy as np
    a = np.asarray(xs, dtype=np.float64)
    return {"n": int(a.size), "mean": round(float(a.mean()), 5),
            **{"p%d" % q: round(float(np.percentile(a, q)), 5) for q in (10, 50, 90)},
            "min": round(float(a.min()), 5), "max": round(float(a.max()), 5)}


def host_operands(kind, ops):
    """Set 0's operands as numpy arrays of raw bits (BF16 as uint16)."""
    import numpy as np
    host = [o.cpu().numpy() for o in ops]
    if kind in ("bf16", "bf16_gelu"):
        host = [h.view(np.uint16) for h in host]
    return host


def parity_sigma(kind, host, K):
    """sigma_A * sigma_B of the decoded operands (from their first 256 rows)
    for the FP4 bound; 1 for BF16 inputs in [-1, 1]."""
    import numpy as np
    import oracle
    from tests import tolerance
    if kind in ("fp4", "fp4_ws"):
        sub = slice(0, 256)
        return (tolerance.sigma_of(oracle.decode_nvfp4(host[0][sub], host[1][sub], K)) *
                tolerance.sigma_of(oracle.decode_nvfp4(host[2][sub], host[3][sub], K)))
    if kind == "mx":
        e2 = np.array([oracle.e2m1_to_double(c) for c in range(16)])
        e8 = np.array([oracle.e8m0_to_double(b) if b != 0xFF else np.nan for b in range(256)])

        def dec(Q, S):
            Q, S = Q[:256], S[:256]
            return e2[np.stack([Q & 15, Q >> 4], -1).reshape(Q.shape[0], -1)] * np.repeat(e8[S], 32, axis=1)
        return tolerance.sigma_of(dec(host[0], host[1])) * tolerance.sigma_of(dec(host[2], host[3]))
    return 1.0


def parity_full(kind, M, N, K, sets):
    """Every element of set 0's C against the oracle (run after the timing)."""
    import numpy as np
    import oracle
    from tests import tolerance
    (ops, C) = sets[0]
    host = host_operands(kind, ops)
    got = C.cpu().numpy().view(np.uint16).reshape(M, N)
    t0 = time.perf_counter()
    if kind == "bf16":
        chk = tolerance.check(got, oracle.gemm_bf16_nt(host[0], host[1]), K)
    elif kind == "bf16_gelu":
        ms, ns = (x.ravel().astype(np.int32) for x in np.meshgrid(np.arange(M), np.arange(N), indexing="ij"))
        ref, z = oracle.gemm_bf16_nt_bias_act_at(host[0], host[1], host[2], oracle.ACT_GELU_TANH, ms, ns,
                                                 with_z=True)
        chk = tolerance.check_fused(got, ref.reshape(M, N), z.reshape(M, N), K, oracle.ACT_GELU_TANH)
    elif kind == "mx":
        chk = tolerance.check(got, oracle.gemm_mxfp4_nt(*host, K), K, parity_sigma(kind, host, K))
    else:
        chk = tolerance.check(got, oracle.gemm_nvfp4_nt(*host, K), K, parity_sigma(kind, host, K))
    return {"elements": M * N, "within_tolerance": bool(chk), "worst_ratio": round(float(chk.worst_ratio), 4),
            "failures": int(chk.n_bad), "oracle_seconds": round(time.perf_counter() - t0, 1),
            "cores": oracle.max_threads()}


def cpu_baseline(kind, M, N, K, sets, seconds_target, seed=0):
    """The oracle, as it stands, on a bounded sample of output elements."""
    import numpy as np
    import oracle
    import synthetic as syn
    from tests import tolerance
    (ops, C) = sets[0]
    host = host_operands(kind, ops)
    if kind == "bf16":
        A, B = host
        fn = lambda ms, ns: oracle.gemm_bf16_nt_at(A, B, ms, ns)
    elif kind == "bf16_gelu":
        A, B, bias = host
        fn = lambda ms, ns: oracle.gemm_bf16_nt_bias_act_at(A, B, bias, oracle.ACT_GELU_TANH, ms, ns, with_z=True)
    elif kind == "mx":
        Aq, SA, Bq, SB = host
        fn = lambda ms, ns: oracle.gemm_mxfp4_nt_at(Aq, SA, Bq, SB, K, ms, ns)
    else:
        Aq, SFA, Bq, SFB = host
        fn = lambda ms, ns: oracle.gemm_nvfp4_nt_at(Aq, SFA, Bq, SFB, K, ms, ns)
    g = np.random.Generator(np.random.PCG64(seed))
    cores = oracle.max_threads()
    # calibrate on a small batch, then size the timed sample to the target
    n0 = max(256, cores * 64)
    t0 = time.perf_counter()
    fn(g.integers(0, M, n0).astype(np.int32), g.integers(0, N, n0).astype(np.int32))
    rate = n0 / max(time.perf_counter() - t0, 1e-6)
    n = int(min(max(rate * seconds_target, n0), M * N))
    ms = g.integers(0, M, n).astype(np.int32)
    ns = g.integers(0, N, n).astype(np.int32)
    t0 = time.perf_counter()
    ref = fn(ms, ns)
    dt = time.perf_counter() - t0
    if kind == "bf16_gelu":
        ref, z = ref
    # the same sample doubles as a spot check of the GPU output of set 0
    got = C.cpu().numpy().view(np.uint16).reshape(M, N)[ms, ns]
    sigma = parity_sigma(kind, host, K)
    if kind == "bf16_gelu":
        chk = tolerance.check_fused(got, ref, z, K, oracle.ACT_GELU_TANH)
    else:
        chk = tolerance.check(got, ref, K, sigma)
    return {
        "value": 2.0 * n * K / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": "%d random output elements of the %dx%dx%d product (full K each), "
                  "binary64 sums, %.1f s" % (n, M, N, K, dt),
        "seconds": dt,
        "spot_check": {"elements": n, "within_tolerance": bool(chk), "worst_ratio": chk.worst_ratio},
    }


def copy_calibration(nbytes: int, reps: int):
    """A plain device copy of known size, for scaling FETCH_SIZE / WRITE_SIZE."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.bitwise_not(src, out=dst)  # one elementwise kernel: reads and writes nbytes
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps}))


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--warm-seconds", type=float, default=1.5,
                    help="least wall time of untimed warm-up; steps beyond --warmup are reported apart")
    ap.add_argument("--launch-samples", type=int, default=300,
                    help="launches timed one by one (own event pair each) for the spread")
    ap.add_argument("--workload", default="bf16_8192", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle leg (used for profiler runs)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target duration of the oracle's timed sample")
    ap.add_argument("--parity-full", action="store_true",
                    help="also compare every element of set 0's C with the oracle")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes (counter calibration)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        return 1
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, 5)
        return 0

    import dense_gemm_14_amd as g
    g.load()  # fails loudly if the HIP library is missing

    kind, M, N, K = WORKLOADS[args.workload]
    per_set = set_bytes(kind, M, N, K)
    n_sets = 2 * LLC_BYTES // per_set + 1
    sets = make_sets(kind, M, N, K, n_sets, CONFIG_INDEX[args.workload])
    stream = torch.cuda.current_stream()
    run = launcher(kind, M, N, K, stream)
    clock = ClockSampler().start()

    # warm-up: W steps, then more until --warm-seconds of sustained work
    t_warm = time.perf_counter()
    i = 0
    for i in range(args.warmup):
        run(*sets[i % n_sets])
    torch.cuda.synchronize()
    extra = 0
    while time.perf_counter() - t_warm < args.warm_seconds:
        for _ in range(16):
            run(*sets[(args.warmup + extra) % n_sets])
            extra += 1
        torch.cuda.synchronize()
    warm_s = time.perf_counter() - t_warm
    first = args.warmup + extra   # the timed steps continue the rotation

    # timed region: exactly K steps between two events on the launch stream
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        run(*sets[(first + i) % n_sets])
    stop.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_total = start.elapsed_time(stop)
    ms_step = ms_total / max(args.steps, 1)
    flops = 2.0 * M * N * K
    tflops = flops / (ms_step * 1e-3) / 1e12

    # per-launch pass: each launch between its own pair of events
    P = max(args.launch_samples, 0)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(P)]
    t2 = time.perf_counter()
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        run(*sets[(first + args.steps + i) % n_sets])
        b.record(stream)
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    clock.stop()
    launch_ms = percentiles([a.elapsed_time(b) for a, b in evs]) if P else None

    # output of set 0 for the spot checks: recomputed last
    run(*sets[0])
    torch.cuda.synchronize()

    # NVFP4 operands are decoded to FP16 for the MFMA; MX operands enter it as FP4
    dtype = {"fp4": "fp16", "mx": "fp4"}.get(kind, "bf16")   # fp4_ws: BF16 matrix instructions
    traffic = read_traffic(args.workload)
    alg_bytes = algorithmic_bytes(kind, M, N, K)
    ridge = PEAK_TFLOPS[dtype] * 1e12 / (HBM_PEAK_GBS * 1e9)   # FLOP per byte
    if flops / alg_bytes >= ridge:
        roofline = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_TFLOPS[dtype], "unit": "TFLOP/s",
                    "frac": round(tflops / PEAK_TFLOPS[dtype], 4)}
    else:  # below the ridge the kernel is bound by HBM: algorithmic bytes per launch time
        gbs = alg_bytes / (ms_step * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(gbs / HBM_PEAK_GBS, 4)}
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    roofline.update({"traffic": traffic,
                     "traffic_kind": "l2_egress_bytes_per_launch (FETCH_SIZE + WRITE_SIZE scaled by a plain copy; "
                                     "includes last-level-cache hits, so an upper bound on HBM bytes)",
                     "kernel": " + ".join(kernels_for(kind, M, N, K, cus)),
                     "algorithmic_bytes": alg_bytes, "mean_launch_ms": round(ms_step, 5)})
    clk = {"source": "amdsmi gpu_metrics (current gfx clock, mean over XCDs; socket power)",
           "timed": clock.window(t0, t1), "per_launch_pass": clock.window(t2, t3)}
    if clock.error:
        clk["error"] = clock.error
    out = {
        "metric": "TFLOP/s for BF16 C=A·B^T at M=N=K=8192; % of MI355X dense BF16 peak"
        if args.workload == "bf16_8192" else
        "TFLOP/s for bf16 C=gelu_tanh(A·B^T+bias) at %dx%dx%d" % (M, N, K) if kind == "bf16_gelu" else
        "TFLOP/s for %s C=A·B^T at %dx%dx%d" % (kind, M, N, K),
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp4": "fp4(e2m1+e4m3)->fp16", "mx": "fp4(e2m1+e8m0)",
                  "fp4_ws": "fp4(e2m1+e4m3)->bf16 (decoded once)"}.get(kind, "bf16"),
        "data": "synthetic",
        "config": {"workload": "%s_nt_%dx%dx%d" % (kind, M, N, K), "M": M, "N": N, "K": K,
                   "rotation_sets": n_sets, "footprint_MiB": round(n_sets * per_set / 2 ** 20, 1),
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "percent_of_peak": round(100.0 * tflops / PEAK_TFLOPS[dtype], 2),
        "warmup_extra": {"steps": extra, "seconds_total": round(warm_s, 3), "floor_seconds": args.warm_seconds},
        "launch_ms": launch_ms,
        "launch_tflops_p50": round(flops / (launch_ms["p50"] * 1e-3) / 1e12, 2) if launch_ms else None,
        "clock": clk,
        "device": {"name": torch.cuda.get_device_properties(0).name, "compute_units": cus},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(kind, M, N, K, sets, args.cpu_seconds)
    if args.parity_full:
        out["parity_full"] = parity_full(kind, M, N, K, sets)
    print(json.dumps(out), flush=True)
    if args.parity_full and not out["parity_full"]["within_tolerance"]:
        return 3
    return 0


if __name__ == "__main__":
    sys.exit(main())
