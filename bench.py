"""Benchmark of the Flash EQ-Linear hot path on one MI355X.

One step = one training pass of the layer over one batch of synthetic input:
weight spectrum (Wt changes every step) + forward + weight gradient + input
gradient, all through the C ABI of libeqlinear.so on torch's current stream.
Inputs are resident in HBM before the timed region starts.  Before the W
warmup steps, the same step runs untimed for --device-warmup-ms (60 ms), so
that the GPU's clocks are at the steady state of this load (reported in the
config as "device_warmup").

Default workload: the ViT-B-like FFN fc1 layer, p4 (T=4), N = 64 images x 197
tokens = 12608 rows, C = 768 -> D = 3072, fp16 I/O with fp32 accumulation.

Prints ONE JSON line:
  value       tokens/s of the whole step (N rows per step)
  roofline    the dominant kernel against its bound (HBM or MFMA), achieved =
              algorithmic bytes (or FLOPs) per launch / mean launch time
              measured with HIP events on the launch stream
  cpu_baseline  the float64 oracle timed on the host cores on the first rows
              of the same batch (a bounded sample)
  dense       the dense GEMMs of the assembled C x D matrix (rocBLAS gemm_ex,
              and torch's F.linear / matmul) on the same data, same protocol

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
                       [--workload NAME] [--dtype f16|f32]
                       [--no-cpu] [--no-dense] [--sets R] [--sweep]
                       [--device-warmup-ms MS]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "EQ-Linear fwd+bwd tokens/s & MFMA util at T=4, C=768→D=3072 vs dense GEMM"

# MI355X published peaks.
PEAK_HBM_GBS = 8000.0
PEAK_MFMA_TFLOPS = {"f16": 2516.6, "f32": 157.3}

KERNEL_SRC = os.path.join(ROOT, "group_wise_dft_amd", "csrc", "eqlinear_kernels.hip")
PROFILES = os.path.join(ROOT, "profiles")


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


# ---------------------------------------------------------------- analytics
def freq_flops(N, C_T, D_T, T, octic=False):
    """Real multiply-adds x2 of the per-frequency contractions (4-mult
    complex products): one real GEMM at k=0 and one at k=T/2 (even T), 4 per
    complex frequency.  Octic group: four character GEMMs and the 2x2 E-block
    product (8 real GEMMs)."""
    g = 12 if octic else 1 + (1 - T % 2) + 4 * ((T - 1) // 2)
    return 2.0 * g * N * C_T * D_T


def pass_bytes(N, C_T, D_T, T, esz):
    """Algorithmic HBM bytes of one forward (or dX, or dWt) launch: read the
    activation once, write the output once, read the T weight planes once."""
    C, D = C_T * T, D_T * T
    return float(N * C + N * D + C * D // T) * esz


def dense_flops(N, C, D):
    return 2.0 * N * C * D


# ---------------------------------------------------------------- rocBLAS
class RocBlas:
    """Minimal ctypes front end of rocblas_gemm_ex (column-major GEMM)."""
    OP_N, OP_T = 111, 112
    DT = {"f16": 150, "f32": 151}
    F32 = 151

    def __init__(self, stream_ptr):
        self.lib = ctypes.CDLL("/opt/rocm/lib/librocblas.so")
        self.h = ctypes.c_void_p()
        st = self.lib.rocblas_create_handle(ctypes.byref(self.h))
        if st != 0:
            raise RuntimeError("rocblas_create_handle: %d" % st)
        self.lib.rocblas_set_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        st = self.lib.rocblas_set_stream(self.h, ctypes.c_void_p(stream_ptr))
        if st != 0:
            raise RuntimeError("rocblas_set_stream: %d" % st)
        i32, vp, u32 = ctypes.c_int32, ctypes.c_void_p, ctypes.c_uint32
        self.lib.rocblas_gemm_ex.argtypes = [
            vp, i32, i32, i32, i32, i32, vp, vp, i32, i32, vp, i32, i32, vp, vp, i32, i32,
            vp, i32, i32, i32, i32, i32, u32]
        self.alpha = ctypes.c_float(1.0)
        self.beta = ctypes.c_float(0.0)

    def gemm(self, ta, tb, m, n, k, a, lda, b, ldb, c, ldc, dt):
        t = self.DT[dt]
        st = self.lib.rocblas_gemm_ex(
            self.h, ta, tb, m, n, k, ctypes.byref(self.alpha), a, t, lda, b, t, ldb,
            ctypes.byref(self.beta), c, t, ldc, c, t, ldc, self.F32, 0, 0, 0)
        if st != 0:
            raise RuntimeError("rocblas_gemm_ex: status %d" % st)


# ---------------------------------------------------------------- timing
SPIN_CYCLES = 20_000_000      # GPU clock cycles; about 10 ms


def time_loop(torch, fn, iters, warmup):
    """Mean and median per-call milliseconds, HIP events on the current stream.

    A GPU spin of a few milliseconds is queued first, so the host has queued
    every call before the GPU reaches them: the events then time the kernels
    back to back, not the host's call overhead (which exceeds the run time of
    the small kernels)."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(iters)]
    torch.cuda._sleep(SPIN_CYCLES)
    for i in range(iters):
        ev[i][0].record()
        fn(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) for a, b in ev)
    return sum(ts) / len(ts), ts[len(ts) // 2]


def read_traffic(kernel_tag):
    """HBM traffic per launch from a committed rocprofv3 counter summary, or
    None when the summary is absent or the kernel source changed since."""
    path = os.path.join(PROFILES, "traffic_%s.txt" % kernel_tag)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    sha = hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()
    if kv.get("kernel_source_sha256") != sha:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def assemble_dense(torch, wt, T, dev):
    """The naive EQ-Linear weight: the dense block-circulant [D, C] matrix
    W[d*T + g, c*T + h] = Wt[d, c, (g - h) mod T] assembled from Wt [D_T, C_T, T]."""
    D_T, C_T, _ = wt.shape
    idx = (torch.arange(T).view(T, 1) - torch.arange(T).view(1, T)) % T  # [g, h]
    wd = wt[:, :, idx.to(dev)]                                           # [D_T, C_T, g, h]
    return wd.permute(0, 2, 1, 3).reshape(D_T * T, C_T * T).contiguous()


def octic_index(torch, dev):
    """[g, h] -> h^-1 g in the octic group (element a + 4 b = r^a s^b, with
    r^a s^b . r^c s^d = r^(a + (-1)^b c) s^(b + d))."""
    def mul(g, h):
        a, b, c, d = g % 4, g // 4, h % 4, h // 4
        return (a - c if b else a + c) % 4 + 4 * (b ^ d)

    def inv(g):
        return g if g >= 4 else (-g) % 4
    return torch.tensor([[mul(inv(h), g) for h in range(8)] for g in range(8)], device=dev)


def assemble_dense_octic(torch, wt, dev):
    """The dense [D, C] matrix of the octic layer, W[d*8 + g, c*8 + h] = Wt[d, c, h^-1 g]."""
    D_T, C_T, _ = wt.shape
    wd = wt[:, :, octic_index(torch, dev)]                              # [D_T, C_T, g, h]
    return wd.permute(0, 2, 1, 3).reshape(D_T * 8, C_T * 8).contiguous()


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ---------------------------------------------------------------- sweep
def sweep(torch, E, dev, iters=20):
    """Every configured workload: the three passes of the library and the
    dense GEMMs (torch, i.e. hipBLASLt) of the assembled block-circulant
    C x D matrix, two rotating buffer sets, the same event timing as the main
    measurement."""
    from group_wise_dft_amd.workloads import OCTIC_WORKLOADS, SCALING_WORKLOADS, WORKLOADS, inputs
    rows = []
    log("sweep (us; dense = torch GEMMs of the assembled matrix):")
    log("%-16s %-4s %8s %8s %8s %8s %8s %8s %6s   %s" % (
        "workload", "dt", "fwd", "dx", "dw", "d_fwd", "d_dx", "d_dw", "x_fwd", "bound, frac of peak fwd dx dw"))
    runs = [(name, wl, False) for name, wl in WORKLOADS.items()] + \
        [(name, wl, True) for name, wl in OCTIC_WORKLOADS.items()] + \
        [(name, wl, False) for name, wl in SCALING_WORKLOADS.items()]
    for name, wl, octic in runs:
        if octic:
            spec, fwd_, bwd_x, bwd_w, wsz = (E.eqlinear_octic_weight_spectrum, E.eqlinear_octic_forward,
                                            E.eqlinear_octic_backward_input, E.eqlinear_octic_backward_weight,
                                            lambda N, C_T, D_T, T, tdt: E.eqlinear_octic_workspace_size(
                                                N, C_T, D_T, tdt))
        else:
            spec, fwd_, bwd_x, bwd_w, wsz = (E.eqlinear_weight_spectrum, E.eqlinear_forward,
                                            E.eqlinear_backward_input, E.eqlinear_backward_weight,
                                            E.eqlinear_workspace_size)
        for dt in wl.dtypes:
            tdt = {"f16": torch.float16, "f32": torch.float32}[dt]
            N, C_T, D_T, T, C, D = wl.N, wl.C_T, wl.D_T, wl.T, wl.C, wl.D
            x_np, w_np, dy_np = inputs(wl, dt)
            x0, w0, dy0 = (torch.from_numpy(a).to(dev) for a in (x_np, w_np, dy_np))
            sets = [dict(x=x0.clone(), dy=dy0.clone(),
                         y=torch.empty((N, D_T, T), dtype=tdt, device=dev),
                         dx=torch.empty((N, C_T, T), dtype=tdt, device=dev),
                         dw=torch.empty((D_T, C_T, T), dtype=tdt, device=dev)) for _ in range(2)]
            what = spec(w0)
            ws = torch.empty(max(wsz(N, C_T, D_T, T, tdt), 16), dtype=torch.uint8, device=dev)
            t_f = time_loop(torch, lambda i: fwd_(sets[i % 2]["x"], what, sets[i % 2]["y"]), iters, 3)[0] * 1e3
            t_x = time_loop(torch, lambda i: bwd_x(sets[i % 2]["dy"], what, sets[i % 2]["dx"]), iters, 3)[0] * 1e3
            t_w = time_loop(torch, lambda i: bwd_w(sets[i % 2]["x"], sets[i % 2]["dy"], sets[i % 2]["dw"], ws),
                            iters, 3)[0] * 1e3
            wd = assemble_dense_octic(torch, w0, dev) if octic else assemble_dense(torch, w0, T, dev)
            xs = [s_["x"].view(N, C) for s_ in sets]
            dys = [s_["dy"].view(N, D) for s_ in sets]
            d_f = time_loop(torch, lambda i: torch.matmul(xs[i % 2], wd.t()), iters, 3)[0] * 1e3
            d_x = time_loop(torch, lambda i: torch.matmul(dys[i % 2], wd), iters, 3)[0] * 1e3
            d_w = time_loop(torch, lambda i: torch.matmul(dys[i % 2].t(), xs[i % 2]), iters, 3)[0] * 1e3
            esz = 2 if dt == "f16" else 4
            by, fl = pass_bytes(N, C_T, D_T, T, esz), freq_flops(N, C_T, D_T, T, octic)
            ridge = PEAK_MFMA_TFLOPS[dt] * 1e12 / (PEAK_HBM_GBS * 1e9)
            roof = {}
            for pn, t_us in (("forward", t_f), ("backward_input", t_x), ("backward_weight", t_w)):
                if fl / by < ridge:
                    roof[pn] = {"bound": "hbm", "frac": round(by / (t_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
                else:
                    roof[pn] = {"bound": "mfma", "frac": round(fl / (t_us * 1e-6) / 1e12 / PEAK_MFMA_TFLOPS[dt], 4)}
            row = {"workload": name, "group": "octic" if octic else "cyclic", "dtype": dt, "N": N, "C": C,
                   "D": D, "T": T, "roofline": roof,
                   "forward_us": round(t_f, 2), "backward_input_us": round(t_x, 2),
                   "backward_weight_us": round(t_w, 2), "dense_forward_us": round(d_f, 2),
                   "dense_backward_input_us": round(d_x, 2), "dense_backward_weight_us": round(d_w, 2)}
            rows.append(row)
            log("%-16s %-4s %8.2f %8.2f %8.2f %8.2f %8.2f %8.2f %6.2f   %s %.3f %.3f %.3f" % (
                name, dt, t_f, t_x, t_w, d_f, d_x, d_w, d_f / t_f, roof["forward"]["bound"],
                roof["forward"]["frac"], roof["backward_input"]["frac"], roof["backward_weight"]["frac"]))
            del sets, what, ws, wd, xs, dys, x0, w0, dy0
            torch.cuda.empty_cache()
    return rows


# ---------------------------------------------------------------- peaks
def peaks(torch, dev):
    """Achievable rates on this GPU (libeqlinear_peaks.so): matrix-core
    FLOP/s in a register loop, HBM copy bandwidth, and the per-CU rates of
    LDS reads, LDS writes, buffer -> LDS copies and L2 -> VGPR loads, each
    with the shader clock measured during the loop."""
    lib = ctypes.CDLL(os.path.join(ROOT, "group_wise_dft_amd", "libeqlinear_peaks.so"))
    vp = ctypes.c_void_p
    lib.peaks_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, ctypes.c_uint32, vp, vp]
    lib.peaks_copy.argtypes = [vp, vp, ctypes.c_size_t, ctypes.c_int, vp]
    st = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    clk = torch.zeros(4, dtype=torch.int64, device=dev)
    src = torch.ones(1 << 21, dtype=torch.uint8, device=dev)        # 2 MiB: L2-resident
    res = {}

    def run(kind, grid, iters):
        out = torch.empty(grid * 256, dtype=torch.float32, device=dev)
        for _ in range(2):
            e = lib.peaks_run(kind, grid, iters, out.data_ptr(), src.data_ptr(), src.numel(), clk.data_ptr(), st)
            if e != 0:
                raise RuntimeError("peaks_run %d: hip error %d" % (kind, e))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        lib.peaks_run(kind, grid, iters, out.data_ptr(), src.data_ptr(), src.numel(), clk.data_ptr(), st)
        e1.record()
        torch.cuda.synchronize()
        c = clk.cpu().tolist()
        ghz = (c[2] - c[0]) / max(1, (c[3] - c[1])) * 0.1            # s_memrealtime runs at 100 MHz
        return e0.elapsed_time(e1) * 1e-3, ghz

    for kind, name, fl in ((0, "mfma_f16_32x32x16", 32768), (1, "mfma_f32_32x32x2", 4096)):
        grid, iters = 4 * cus, 4000 if kind == 0 else 1000
        t, ghz = run(kind, grid, iters)
        tf = grid * 4 * iters * 4 * fl / t / 1e12
        res[name] = {"TFLOP_s": round(tf, 1), "clock_GHz": round(ghz, 2),
                     "per_CU_clock_FLOP": round(tf * 1e12 / cus / (ghz * 1e9), 1)}
    for kind, name in ((2, "lds_read_b128"), (3, "lds_write_b128"), (4, "buffer_to_lds_16B"),
                       (5, "l2_to_vgpr_16B")):
        grid, iters = 2 * cus, 1000 if kind < 4 else 200
        t, ghz = run(kind, grid, iters)
        nbytes = grid * 256 * iters * 8 * 16
        res[name] = {"TB_s": round(nbytes / t / 1e12, 2), "clock_GHz": round(ghz, 2),
                     "bytes_per_CU_clock": round(nbytes / t / cus / (ghz * 1e9), 1)}
    n = 1 << 27                                                       # 2 GiB of 16-byte elements
    a = torch.empty(n * 16, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    for _ in range(2):
        lib.peaks_copy(a.data_ptr(), b.data_ptr(), n, 8 * cus, st)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    lib.peaks_copy(a.data_ptr(), b.data_ptr(), n, 8 * cus, st)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3
    res["hbm_copy"] = {"TB_s": round(2 * n * 16 / t / 1e12, 2), "bytes": 2 * n * 16}
    del a, b
    for k, v in res.items():
        log("peak %-20s %s" % (k, v))
    return res


# ---------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--dtype", default=None)
    ap.add_argument("--sets", type=int, default=0,
                    help="rotating buffer sets (0: enough to exceed 512 MiB)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--device-warmup-ms", type=float, default=60.0,
                    help="untimed steps before the warmup steps, so that the GPU clocks reach their "
                         "steady state for this load (0 to skip)")
    ap.add_argument("--sweep", action="store_true",
                    help="also time every configured workload (table on stderr, 'sweep' in the JSON)")
    ap.add_argument("--peaks", action="store_true",
                    help="only measure achievable MFMA / HBM / LDS / L2 rates (libeqlinear_peaks.so)")
    ap.add_argument("--overlap-backward", action="store_true",
                    help="run dW on a second stream beside dX (measured slower at ViT-B size)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the layer's hot path runs on a single "
              "MI355X and the library has no multi-GPU path (asked for --gpus %d, "
              "WORLD_SIZE %d)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import torch

    from group_wise_dft_amd.workloads import HEADLINE, OCTIC_WORKLOADS, SCALING_WORKLOADS, WORKLOADS, inputs

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    if args.peaks:
        torch.cuda.set_device(0)
        res = peaks(torch, torch.device("cuda:0"))
        print(json.dumps({"peaks": res, "device": torch.cuda.get_device_name(0),
                          "published": {"mfma_f16_TFLOP_s": PEAK_MFMA_TFLOPS["f16"],
                                        "mfma_f32_TFLOP_s": PEAK_MFMA_TFLOPS["f32"],
                                        "hbm_TB_s": PEAK_HBM_GBS / 1e3}}), flush=True)
        return
    from group_wise_dft_amd import eqlinear as E  # raises if the library is missing

    name = args.workload or HEADLINE
    octic = name in OCTIC_WORKLOADS
    wl = OCTIC_WORKLOADS[name] if octic else SCALING_WORKLOADS.get(name) or WORKLOADS[name]
    if octic:   # the octic group's entry points, same signatures
        new_spec = lambda C_T, D_T, T, tdt, dev: E.new_octic_weight_spectrum(C_T, D_T, tdt, dev)  # noqa: E731
        ws_size = lambda N, C_T, D_T, T, tdt: E.eqlinear_octic_workspace_size(N, C_T, D_T, tdt)  # noqa: E731
        spec_size = lambda C_T, D_T, T, tdt: E.eqlinear_octic_spectrum_size(C_T, D_T, tdt)  # noqa: E731
        f_spec, f_fwd, f_dx, f_dw = (E.eqlinear_octic_weight_spectrum, E.eqlinear_octic_forward,
                                     E.eqlinear_octic_backward_input, E.eqlinear_octic_backward_weight)
    else:
        new_spec, ws_size, spec_size = E.new_weight_spectrum, E.eqlinear_workspace_size, E.eqlinear_spectrum_size
        f_spec, f_fwd, f_dx, f_dw = (E.eqlinear_weight_spectrum, E.eqlinear_forward,
                                     E.eqlinear_backward_input, E.eqlinear_backward_weight)
    dt = args.dtype or ("f16" if "f16" in wl.dtypes else wl.dtypes[0])
    tdt = {"f16": torch.float16, "f32": torch.float32}[dt]
    esz = 2 if dt == "f16" else 4
    N, C_T, D_T, T = wl.N, wl.C_T, wl.D_T, wl.T
    C, D = wl.C, wl.D
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("workload %s %s N=%d C_T=%d D_T=%d T=%d on %s" % (
        wl.name, dt, N, C_T, D_T, T, torch.cuda.get_device_name(dev)))

    x_np, w_np, dy_np = inputs(wl, dt)
    x0 = torch.from_numpy(x_np).to(dev)
    w0 = torch.from_numpy(w_np).to(dev)
    dy0 = torch.from_numpy(dy_np).to(dev)

    set_bytes = (2 * N * C + 2 * N * D + 3 * C * D) * esz
    R = args.sets or max(2, -(-(512 << 20) // set_bytes))
    sets = []
    for r in range(R):
        sets.append(dict(
            x=x0.clone(), w=w0.clone(), dy=dy0.clone(),
            what=new_spec(C_T, D_T, T, tdt, dev),
            y=torch.empty((N, D_T, T), dtype=tdt, device=dev),
            dx=torch.empty((N, C_T, T), dtype=tdt, device=dev),
            dw=torch.empty((D_T, C_T, T), dtype=tdt, device=dev)))
    ws_bytes = ws_size(N, C_T, D_T, T, tdt)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    log("%d rotating buffer sets of %.1f MiB; dW workspace %.1f MiB" % (
        R, set_bytes / 2**20, ws_bytes / 2**20))

    def spectrum(i):
        s = sets[i % R]
        f_spec(s["w"], s["what"])

    def forward(i):
        s = sets[i % R]
        f_fwd(s["x"], s["what"], s["y"])

    def backward_input(i):
        s = sets[i % R]
        f_dx(s["dy"], s["what"], s["dx"])

    def backward_weight(i):
        s = sets[i % R]
        f_dw(s["x"], s["dy"], s["dw"], ws)

    main_stream = torch.cuda.current_stream(dev)
    side_stream = torch.cuda.Stream(device=dev)    # default priority

    def step_serial(i):
        # the weight gradient first: it meets dY cold and leaves it in the
        # Infinity Cache for the input gradient, which loses more to a cold
        # read (ViT-B fc1 on MI355X in the steady state: 146.9 us a step
        # against 152.5 the other way round).  The octic layer measured the
        # other way round (137.3 against 141.2 us at ViT-B width).
        spectrum(i)
        forward(i)
        if octic:
            backward_input(i)
            backward_weight(i)
        else:
            backward_weight(i)
            backward_input(i)

    def step_overlap(i):
        # the two gradient products are independent: dW on a side stream while
        # dX runs on the main stream (measured slower than the serial order)
        spectrum(i)
        forward(i)
        side_stream.wait_stream(main_stream)
        with torch.cuda.stream(side_stream):
            backward_weight(i)
        backward_input(i)
        main_stream.wait_stream(side_stream)

    step = step_overlap if args.overlap_backward else step_serial

    # ---- device warm-up: from idle, the GPU needs tens of milliseconds of
    # this load before its clocks settle (measured at ViT-B fc1 on MI355X,
    # each after 3 s idle, 5 warmup steps, 20 timed: no warm-up 162-169 us a
    # step; 100 / 300 ms of GPU spin 167-170; 300 steps of this step first
    # 148; dense GEMMs and large copies for 0.1-1 s first 166-178).  A
    # training job runs in that steady state, so before the W warmup steps
    # the same step runs untimed for --device-warmup-ms (reported as
    # "device_warmup"). ----
    dev_warm = None
    if args.device_warmup_ms > 0:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        n_warm = 0
        while (time.perf_counter() - t0) * 1e3 < args.device_warmup_ms:
            for _ in range(10):
                step_serial(n_warm)
                n_warm += 1
            torch.cuda.synchronize()
        dev_warm = {"what": "untimed steps, the same as the timed ones, before the W warmup steps, so that "
                            "the GPU clocks are at their steady state for this load",
                    "steps": n_warm, "ms": round((time.perf_counter() - t0) * 1e3, 1)}
        log("device warm-up: %d untimed steps in %.1f ms" % (n_warm, dev_warm["ms"]))

    # ---- the timed region: K whole steps ----
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record()
    for i in range(args.steps):
        step(i)
    t_end.record()
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps
    tokens_s = N / (ms_step * 1e-3)
    log("step %.4f ms  -> %.4g tokens/s (%s backward)" % (
        ms_step, tokens_s, "overlapped" if args.overlap_backward else "serial"))
    other = step_serial if args.overlap_backward else step_overlap
    ms_other, _ = time_loop(torch, other, args.steps, 2)
    log("step with %s backward: %.4f ms" % (
        "serial" if args.overlap_backward else "overlapped", ms_other))

    # ---- per-pass launch times (each entry point timed alone) ----
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    torch.cuda._sleep(SPIN_CYCLES)
    e1.record()
    torch.cuda.synchronize()
    log("GPU spin ahead of each timing loop: %.2f ms" % e0.elapsed_time(e1))
    iters = max(args.steps, 20)
    passes = {}
    fl = freq_flops(N, C_T, D_T, T, octic)
    by = pass_bytes(N, C_T, D_T, T, esz)
    for name, fn in (("spectrum", spectrum), ("forward", forward),
                     ("backward_input", backward_input), ("backward_weight", backward_weight)):
        mean, med = time_loop(torch, fn, iters, 3)
        rec = {"us_mean": round(mean * 1e3, 3), "us_median": round(med * 1e3, 3)}
        if name != "spectrum":
            rec["GB_s"] = round(by / (mean * 1e-3) / 1e9, 1)
            rec["hbm_frac"] = round(by / (mean * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
            rec["freq_TFLOP_s"] = round(fl / (mean * 1e-3) / 1e12, 2)
            rec["mfma_frac"] = round(fl / (mean * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS[dt], 4)
            rec["dense_equiv_TFLOP_s"] = round(dense_flops(N, C, D) / (mean * 1e-3) / 1e12, 2)
        else:   # read Wt once, write the cached spectrum (both orientations)
            sb = float(C * D // T * esz + spec_size(C_T, D_T, T, tdt))
            rec["GB_s"] = round(sb / (mean * 1e-3) / 1e9, 1)
        passes[name] = rec
        log("%-16s %s" % (name, rec))

    # ---- the group-shared bias (not part of the step: the layer above has
    # none); forward with the bias in the epilogue, and the bias gradient ----
    bias = torch.randn((D_T,), device=dev).to(tdt)
    db = torch.empty((D_T,), dtype=tdt, device=dev)
    bws = torch.empty(max(E.eqlinear_bias_workspace_size(N, D_T, T, tdt), 16), dtype=torch.uint8,
                      device=dev)

    def forward_bias(i):
        s = sets[i % R]
        f_fwd(s["x"], s["what"], s["y"], bias=bias)

    def backward_bias(i):
        E.eqlinear_backward_bias(sets[i % R]["dy"], db, bws)

    mean, med = time_loop(torch, forward_bias, iters, 3)
    passes["forward_with_bias"] = {"us_mean": round(mean * 1e3, 3), "us_median": round(med * 1e3, 3)}
    mean, med = time_loop(torch, backward_bias, iters, 3)
    bb = float(N * D * esz + D_T * esz)
    passes["backward_bias"] = {"us_mean": round(mean * 1e3, 3), "us_median": round(med * 1e3, 3),
                               "GB_s": round(bb / (mean * 1e-3) / 1e9, 1),
                               "hbm_frac": round(bb / (mean * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    for name in ("forward_with_bias", "backward_bias"):
        log("%-16s %s" % (name, passes[name]))

    # ---- dominant kernel and its roofline ----
    main_passes = ("forward", "backward_input", "backward_weight")
    dom = max(main_passes, key=lambda p: passes[p]["us_mean"])
    t_dom = passes[dom]["us_mean"] * 1e-6
    ai = fl / by
    ridge = PEAK_MFMA_TFLOPS[dt] * 1e12 / (PEAK_HBM_GBS * 1e9)
    tag = "%s_%s_%s" % (dom, wl.name, dt)
    if ai < ridge:
        roof = {"bound": "hbm", "achieved": round(by / t_dom / 1e9, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": round(fl / t_dom / 1e12, 2),
                "peak": PEAK_MFMA_TFLOPS[dt], "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = read_traffic(tag)
    roof["kernel"] = {"forward": "row_kernel (forward)",
                      "backward_input": "row_kernel (input gradient)",
                      "backward_weight": "weight-gradient kernel (dw_kernel or dwp_kernel, by the "
                                         "shape's plan) + dw_finalize"}[dom]
    roof["algorithmic_per_launch"] = by if roof["bound"] == "hbm" else fl
    roof["launch_us"] = passes[dom]["us_mean"]

    # ---- dense baseline: GEMMs of the assembled C x D matrix ----
    dense = None
    if not args.no_dense:
        wd = assemble_dense_octic(torch, w0, dev) if octic else assemble_dense(torch, w0, T, dev)
        xs = [s["x"].view(N, C) for s in sets]
        dys = [s["dy"].view(N, D) for s in sets]
        ys = [torch.empty((N, D), dtype=tdt, device=dev) for _ in range(R)]
        dxs = [torch.empty((N, C), dtype=tdt, device=dev) for _ in range(R)]
        dws = [torch.empty((D, C), dtype=tdt, device=dev) for _ in range(R)]
        dense = {}
        try:
            rb = RocBlas(torch.cuda.current_stream(dev).cuda_stream)
            OPN, OPT = RocBlas.OP_N, RocBlas.OP_T

            # Row-major [R, S] buffers are column-major [S, R] to rocBLAS.
            def rb_fwd(i):   # Y^T (D x N) = W (D x C) . X^T (C x N)
                r = i % R
                rb.gemm(OPT, OPN, D, N, C, wd.data_ptr(), C, xs[r].data_ptr(), C,
                        ys[r].data_ptr(), D, dt)

            def rb_dx(i):    # dX^T (C x N) = W^T (C x D) . dY^T (D x N)
                r = i % R
                rb.gemm(OPN, OPN, C, N, D, wd.data_ptr(), C, dys[r].data_ptr(), D,
                        dxs[r].data_ptr(), C, dt)

            def rb_dw(i):    # dW^T (C x D) = X^T (C x N) . dY (N x D)
                r = i % R
                rb.gemm(OPN, OPT, C, D, N, xs[r].data_ptr(), C, dys[r].data_ptr(), D,
                        dws[r].data_ptr(), C, dt)

            # correctness of the baseline itself against torch on set 0
            rb_fwd(0); rb_dx(0); rb_dw(0)
            torch.cuda.synchronize()
            ref_y = (xs[0].float() @ wd.float().t())
            err = ((ys[0].float() - ref_y).norm() / ref_y.norm()).item()
            if not err < 5e-3:
                raise RuntimeError("rocBLAS baseline disagrees with torch: %.3e" % err)
            tot = 0.0
            rec = {}
            for nm, fn in (("forward", rb_fwd), ("backward_input", rb_dx),
                           ("backward_weight", rb_dw)):
                mean, _ = time_loop(torch, fn, iters, 3)
                rec[nm + "_us"] = round(mean * 1e3, 3)
                rec[nm + "_TFLOP_s"] = round(dense_flops(N, C, D) / (mean * 1e-3) / 1e12, 1)
                tot += mean
            rec["tokens_s"] = N / (tot * 1e-3)
            dense["rocblas"] = rec
        except (OSError, RuntimeError, AttributeError) as e:
            dense["rocblas_error"] = str(e)[:200]

        def tl_fwd(i):
            r = i % R
            torch.nn.functional.linear(xs[r], wd, out=ys[r])

        def tl_dx(i):
            r = i % R
            torch.matmul(dys[r], wd, out=dxs[r])

        def tl_dw(i):
            r = i % R
            torch.matmul(dys[r].t(), xs[r], out=dws[r])

        tot = 0.0
        rec = {}
        for nm, fn in (("forward", tl_fwd), ("backward_input", tl_dx),
                       ("backward_weight", tl_dw)):
            mean, _ = time_loop(torch, fn, iters, 3)
            rec[nm + "_us"] = round(mean * 1e3, 3)
            tot += mean
        rec["tokens_s"] = N / (tot * 1e-3)
        dense["torch_linear"] = rec
        best = max(v["tokens_s"] for k, v in dense.items() if isinstance(v, dict))
        dense["speedup_fwd_bwd"] = round(tokens_s / best, 3)
        best_fwd = min(v["forward_us"] for k, v in dense.items() if isinstance(v, dict))
        dense["speedup_forward"] = round(best_fwd / passes["forward"]["us_mean"], 3)
        log("dense %s" % dense)

    # ---- a plain copy of known size, for counter calibration under rocprofv3 ----
    cal_src = torch.ones(1 << 29, dtype=torch.uint8, device=dev)   # 512 MiB
    cal_dst = torch.empty_like(cal_src)
    for _ in range(2):
        cal_dst.copy_(cal_src)
    torch.cuda.synchronize()
    del cal_src, cal_dst

    # ---- CPU baseline: the float64 oracle on the first rows of the batch ----
    cpu = None
    if not args.no_cpu:
        import oracle
        thr = oracle.num_threads()

        def run_oracle(ns):
            t0 = time.perf_counter()
            if octic:
                oracle.octic_forward(x_np[:ns], w_np)
                oracle.octic_backward_input(dy_np[:ns], w_np)
                oracle.octic_backward_weight(x_np[:ns], dy_np[:ns])
            else:
                oracle.forward(x_np[:ns], w_np)
                oracle.backward_input(dy_np[:ns], w_np)
                oracle.backward_weight(x_np[:ns], dy_np[:ns])
            return time.perf_counter() - t0

        probe = min(N, 16)
        tp = run_oracle(probe)
        ns = int(max(probe, min(N, args.cpu_seconds / max(tp / probe, 1e-9))))
        tc = run_oracle(ns)
        cpu = {"value": round(ns / tc, 2), "unit": "tokens/s", "cores": thr, "cpu_model": cpu_model(),
               "kind": "oracle",
               "sample": "float64 direct-sum forward + input gradient + weight gradient over "
                         "the first %d of %d rows (full C=%d -> D=%d), %.1f s" % (
                             ns, N, C, D, tc)}
        log("cpu baseline %s" % cpu)

    sweep_rows = sweep(torch, E, dev) if args.sweep else None

    out = {
        "metric": METRIC, "value": round(tokens_s, 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": dt, "data": "synthetic",
        "config": {"workload": "%s: %s" % (wl.name, wl.what), "group": "octic" if octic else "cyclic",
                   "N": N, "C": C, "D": D, "T": T,
                   "io_dtype": dt, "accumulate": "f32",
                   "step": ("weight spectrum + forward + input grad + weight grad" if octic else
                            "weight spectrum + forward + weight grad + input grad") + (
                       " (weight grad on a second stream, overlapping the input grad)"
                       if args.overlap_backward else ""),
                   "rotating_sets": R, "device_warmup": dev_warm},
        "roofline": roof,
        "cpu_baseline": cpu,
        "mfma_frac_step": round(3 * fl / (ms_step * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS[dt], 4),
        "dense_equiv_TFLOP_s_step": round(3 * dense_flops(N, C, D) / (ms_step * 1e-3) / 1e12, 2),
        "passes": passes,
        "dense": dense,
        "device": torch.cuda.get_device_name(dev),
    }
    if sweep_rows is not None:
        out["sweep"] = sweep_rows
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
