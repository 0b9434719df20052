#!/usr/bin/env python3
"""Throughput of the Whisper-style encoder block forward on one MI355X.

A step is one call of the C ABI over the whole workload (every step of the block: LN1, QKV
projection, attention, out-projection + residual, LN2, fc1 + GELU, fc2 + residual; for a stack
every block and the final LayerNorm).  The default workload is the batched large-v3 block:
16 windows x 1500 positions, d_model 1280, 20 heads, ffn 5120, bf16-valued weights, 5 % of the
input rows scaled by 20.  Inputs are seeded synthetic data resident in HBM before timing starts.

Prints ONE JSON line: frames/s (frames = encoder positions), the per-kernel breakdown timed with
HIP events on the launch stream, the roofline entry of the dominant kernel, and the CPU oracle
timed on a bounded sample of the same workload on the host cores.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "encoder frames/sec per 1500-frame window + attention/GEMM TFLOP/s (% MFMA peak)"
# Dense MFMA peaks of the operand types (MXFP8 runs at the fp8 rate; BF16X2 / X3 at bf16's).
PEAK_TFLOPS = {"bf16": 2500.0, "fp16": 2500.0, "fp32": 157.3, "bf16x2": 2500.0, "bf16x3": 2500.0,
               "q8": 2500.0, "q4": 2500.0, "mxfp8": 5000.0}
PEAK_HBM_GBS = 8000.0
COLD_FLUSH_BYTES = 512 << 20  # twice the 256 MB Infinity Cache
COUNTERS = os.path.join(ROOT, "profiles", "hbm_traffic.json")
CSRC = os.path.join(ROOT, "speech_transformer_encoder_amd", "csrc")


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="before the warm-up steps, run the step this long (wall time) so that the "
                         "GPU clocks leave their idle state; reported as settle_ms")
    ap.add_argument("--config", default="large_v3_batch16_block")
    ap.add_argument("--path", default="fp16", choices=["bf16", "fp16", "fp32", "mxfp8"],
                    help="operand path of the timed step (mxfp8: its own numerical method, with "
                         "attention and the out-projection on fp16)")
    ap.add_argument("--compare-paths", default="bf16,bf16x3,mxfp8",
                    help="comma-separated other paths timed the same way (reported, not value): "
                         "bf16, bf16x2, bf16x3, mxfp8, fp32")
    ap.add_argument("--kernel-reps", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-windows", type=int, default=16)
    ap.add_argument("--cpu-sample-layers", type=int, default=2)
    ap.add_argument("--pmc-run", action="store_true",
                    help="launch each block kernel once plus a calibration copy (for rocprofv3 --pmc)")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/hbm_traffic.json from two rocprofv3 counter CSVs")
    ap.add_argument("--pmc-command", default="", help="command line recorded with --ingest-pmc")
    ap.add_argument("--no-next-steps", action="store_true",
                    help="skip timing the adjacent steps (front end, cross K/V, ragged, q8/q4)")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip timing the other workloads and the fp32 path")
    return ap.parse_args()


def source_hash(files):
    h = hashlib.sha256()
    for f in sorted(files):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def time_events(fn, reps, stream):
    """Average duration of fn() over reps launches, from HIP events on `stream`."""
    import torch
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    fn()
    torch.cuda.synchronize()
    s.record(stream)
    for _ in range(reps):
        fn()
    e.record(stream)
    e.synchronize()
    return s.elapsed_time(e) / reps  # ms


def time_events_cold(fn, reps, stream, flush_bytes=COLD_FLUSH_BYTES):
    """Median duration of fn() with the caches cold: before each launch a buffer twice the size
    of the 256 MB Infinity Cache is read (a read, so that no dirty lines are left to be written
    back during fn()), and only fn() lies between the events."""
    import torch
    buf = torch.ones(flush_bytes // 4, device="cuda")
    sink = torch.empty((), device="cuda")
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    times = []
    for _ in range(reps):
        torch.amax(buf, dim=0, out=sink)
        s.record(stream)
        fn()
        e.record(stream)
        e.synchronize()
        times.append(s.elapsed_time(e))
    del buf
    times.sort()
    return times[len(times) // 2]  # ms


KERNEL_SOURCES = {
    "ln": ["layernorm.hip", "wenc_device.h"],
    "gemm_qkv": ["gemm.hip", "wenc_device.h"],
    "attention": ["attention.hip", "wenc_device.h"],
    "gemm_out_residual": ["gemm.hip", "wenc_device.h"],
    "gemm_fc1_gelu": ["gemm.hip", "wenc_device.h"],
    "gemm_fc2_residual": ["gemm.hip", "wenc_device.h"],
}
KERNEL_ORDER = list(KERNEL_SOURCES)
COPY_BYTES = 1 << 30  # plain device copy used to scale the HBM byte counters


def make_kernels(cfg, path_name):
    """Each kernel of one block at the workload's shapes, as (launch, bound, work) on buffers
    chained in the block's order (LN writes the projections' input, QKV the attention's, attention
    the out-projection's, fc1 fc2's): LN, the QKV projection, attention, out-projection +
    residual, fc1 + GELU, fc2 + residual.  Work is algorithmic flops (MFMA-bound) or bytes
    (HBM-bound) per launch."""
    import torch
    from speech_transformer_encoder_amd import binding as B
    path = B.PATHS[path_name]
    dt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[path_name]
    es = 4 if path_name == "fp32" else 2
    M, d, f, H = cfg.batch * cfg.t, cfg.d_model, cfg.ffn_dim, cfg.heads
    dev = "cuda"
    g = torch.Generator(device=dev).manual_seed(0)
    rnd = lambda *s: torch.randn(*s, device=dev, generator=g)  # noqa: E731
    x = rnd(M, d)
    y = x.clone()
    a = torch.empty(M, d, device=dev, dtype=dt)
    o = torch.empty(M, d, device=dev, dtype=dt)
    hid = torch.empty(M, f, device=dev, dtype=dt)
    qkv_out = torch.empty(M, 3 * d, device=dev, dtype=dt)
    wqkv, wo = (rnd(3 * d, d) * 0.02).to(dt), (rnd(d, d) * 0.02).to(dt)
    w1, w2 = (rnd(f, d) * 0.02).to(dt), (rnd(d, f) * 0.02).to(dt)
    ones, zeros = torch.ones(d, device=dev), torch.zeros(d, device=dev)
    b3, bf = torch.zeros(3 * d, device=dev), torch.zeros(f, device=dev)
    ln_dt = {"bf16": B.WENC_DTYPE_BF16, "fp16": B.WENC_DTYPE_F16, "fp32": B.WENC_DTYPE_F32}[path_name]
    qp = qkv_out.data_ptr()  # the buffers are chained in the block's order
    return {
        "ln": (lambda: B.whisper_enc_layernorm(x, ones, zeros, a, M, d, ln_dt),
               "hbm", M * d * (4 + es) + 2 * d * 4),
        "gemm_qkv": (lambda: B.whisper_enc_linear(a, wqkv, b3, None, qkv_out, M, 3 * d, d, path,
                                                  B.WENC_EPI_BIAS), "mfma", 2.0 * M * 3 * d * d),
        "attention": (lambda: B.whisper_enc_attention(qp, qp + d * es, qp + 2 * d * es, o,
                                                      cfg.batch, cfg.t, H, 3 * d, d, path),
                      "mfma", 4.0 * cfg.batch * cfg.t * cfg.t * d),
        "gemm_out_residual": (lambda: B.whisper_enc_linear(o, wo, zeros, y, y, M, d, d, path,
                                                           B.WENC_EPI_BIAS_RESIDUAL), "mfma",
                              2.0 * M * d * d),
        "gemm_fc1_gelu": (lambda: B.whisper_enc_linear(a, w1, bf, None, hid, M, f, d, path,
                                                       B.WENC_EPI_BIAS_GELU), "mfma", 2.0 * M * f * d),
        "gemm_fc2_residual": (lambda: B.whisper_enc_linear(hid, w2, zeros, y, y, M, d, f, path,
                                                           B.WENC_EPI_BIAS_RESIDUAL), "mfma",
                              2.0 * M * d * f),
    }


def mx_kernel_breakdown(cfg, reps):
    """The MXFP8 path's own kernels at the workload's shapes: the LayerNorm writing MXFP8, and
    the QKV, fc1 + GELU (MXFP8 out) and fc2 + residual projections on MXFP8 operands (weights
    quantised on the GPU from random fp32; the LayerNorm writes the projections' input and fc1
    fc2's).  Attention and the out-projection are the fp16 kernels.  Rates against the dense
    fp8 MFMA peak."""
    import torch
    from speech_transformer_encoder_amd import binding as B
    M, d, f = cfg.batch * cfg.t, cfg.d_model, cfg.ffn_dim
    g = torch.Generator(device="cuda").manual_seed(0)
    rnd = lambda *s: torch.randn(*s, device="cuda", generator=g)  # noqa: E731

    def mx(rows, k, scale=1.0):
        out = torch.empty(B.whisper_enc_mx_bytes(rows, k), dtype=torch.uint8, device="cuda")
        B.whisper_enc_mx_quantize(rnd(rows, k) * scale, out, rows, k)
        return out
    wqkv, w1, w2 = mx(3 * d, d, 0.02), mx(f, d, 0.02), mx(d, f, 0.02)
    x = rnd(M, d)
    y = x.clone()
    ones, zeros = torch.ones(d, device="cuda"), torch.zeros(d, device="cuda")
    b3, bf = torch.zeros(3 * d, device="cuda"), torch.zeros(f, device="cuda")
    qkv = torch.empty(M, 3 * d, dtype=torch.float16, device="cuda")
    hid = torch.empty(B.whisper_enc_mx_bytes(M, f), dtype=torch.uint8, device="cuda")
    ln_out = torch.empty(B.whisper_enc_mx_bytes(M, d), dtype=torch.uint8, device="cuda")
    P = B.WENC_PATH_MXFP8
    kernels = {
        "ln": (lambda: B.whisper_enc_layernorm(x, ones, zeros, ln_out, M, d, B.WENC_DTYPE_MXFP8),
               "hbm", M * d * 4 + B.whisper_enc_mx_bytes(M, d) + 2 * d * 4),
        "gemm_qkv": (lambda: B.whisper_enc_linear(ln_out, wqkv, b3, None, qkv, M, 3 * d, d, P,
                                                  B.WENC_EPI_BIAS), "mfma", 2.0 * M * 3 * d * d),
        "gemm_fc1_gelu": (lambda: B.whisper_enc_linear(ln_out, w1, bf, None, hid, M, f, d, P,
                                                       B.WENC_EPI_BIAS_GELU), "mfma", 2.0 * M * f * d),
        "gemm_fc2_residual": (lambda: B.whisper_enc_linear(hid, w2, zeros, y, y, M, d, f, P,
                                                           B.WENC_EPI_BIAS_RESIDUAL), "mfma",
                              2.0 * M * d * f),
    }
    st = torch.cuda.current_stream()
    out = {}
    for fn, _, _ in kernels.values():  # one pass in the block's order fills the chained buffers
        fn()
    for name, (fn, bound, work) in kernels.items():
        ms = time_events(fn, reps, st)
        if bound == "hbm":
            ach, peak, unit = work / (ms * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s"
        else:
            ach, peak, unit = work / (ms * 1e-3) / 1e12, PEAK_TFLOPS["mxfp8"], "TFLOP/s"
        out[name] = {"ms": round(ms, 5), "bound": bound, "achieved": round(ach, 1), "unit": unit,
                     "peak": peak, "frac": round(ach / peak, 4), "work": work,
                     "launches_per_block": 2 if name == "ln" else 1}
    del wqkv, w1, w2, hid, ln_out, qkv
    torch.cuda.empty_cache()
    return out


def mfma_peak(path_name):
    """Dense 16-bit (or MXFP8) MFMA rate this GPU sustains on register operands (the probe
    library beside the encoder library), with the shader clock while it runs; None on the fp32
    path."""
    import ctypes
    import torch
    if path_name == "fp32":
        return None
    lib = ctypes.CDLL(os.path.join(ROOT, "speech_transformer_encoder_amd", "libwenc_probe.so"))
    lib.wenc_probe_mfma.restype = ctypes.c_int
    lib.wenc_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p]
    lib.wenc_probe_mfma_flops.restype = ctypes.c_longlong
    lib.wenc_probe_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    dtype = {"fp16": 2, "bf16": 1, "mxfp8": 8}[path_name]
    blocks, iters = 256 * 2, 100000  # two wavefronts per SIMD; ~20 ms per launch
    clocks = torch.zeros(2, dtype=torch.int64, device="cuda")
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream()
    fn = lambda: lib.wenc_probe_mfma(dtype, blocks, iters, clocks.data_ptr(),  # noqa: E731
                                     sink.data_ptr(), st.cuda_stream)
    assert fn() == 0
    torch.cuda.synchronize()
    best, clk = None, None
    for _ in range(3):
        ms = time_events(fn, 1, st)
        c = clocks.cpu().tolist()
        if best is None or ms < best:
            best, clk = ms, (c[0] / c[1] * 0.1 if c[1] > 0 else None)  # GHz (100 MHz reference)
    tf = lib.wenc_probe_mfma_flops(dtype, blocks, iters) / (best * 1e-3) / 1e12
    return {"dtype": path_name, "tflops": round(tf, 1), "shader_clock_ghz": round(clk, 3) if clk else None,
            "rated_tflops": PEAK_TFLOPS[path_name], "rated_clock_ghz": 2.4,
            "probe": ("v_mfma_scale_f32_32x32x64_f8f6f4" if path_name == "mxfp8" else
                      "v_mfma_f32_32x32x16") + " on register operands, 4 chains x 2 wavefronts per SIMD"}


def kernel_breakdown(cfg, path_name, reps):
    """Each kernel of one block at the workload's shapes, timed on the current stream as `reps`
    launches back to back between two events (one launch per event pair would add the events'
    own cost, ~10 % of a 0.3 ms kernel, to every launch)."""
    import torch
    st = torch.cuda.current_stream()
    per_block = {"ln": 2}  # LN1 and LN2
    out = {}
    kernels = make_kernels(cfg, path_name)
    for fn, _, _ in kernels.values():  # one pass in the block's order fills the chained buffers
        fn()
    for name, (fn, bound, work) in kernels.items():
        ms = time_events(fn, reps, st)
        if bound == "hbm":
            ach = work / (ms * 1e-3) / 1e9
            peak = PEAK_HBM_GBS
            unit = "GB/s"
        else:
            ach = work / (ms * 1e-3) / 1e12
            peak = PEAK_TFLOPS[path_name]
            unit = "TFLOP/s"
        out[name] = {"ms": round(ms, 5), "bound": bound, "achieved": round(ach, 2), "unit": unit,
                     "peak": peak, "frac": round(ach / peak, 4), "work": work,
                     "launches_per_block": per_block.get(name, 1)}
        if bound == "hbm":
            # The LayerNorm's tensors fit in the Infinity Cache, so the rate above is an
            # effective one; the same launch after a cache flush gives the HBM rate.
            # A plain device copy of as many bytes, timed the same way, shows the rate such a
            # single launch can reach from HBM.
            ms_cold = time_events_cold(fn, max(reps, 5), st)
            ach_cold = work / (ms_cold * 1e-3) / 1e9
            src = torch.empty(work // 8, device="cuda", dtype=torch.float32).fill_(1.0)
            dst = torch.empty_like(src)
            ms_copy = time_events_cold(lambda: dst.copy_(src), max(reps, 5), st)
            del src, dst
            out[name].update({"ms_cold": round(ms_cold, 5), "achieved_cold": round(ach_cold, 2),
                              "frac_cold": round(ach_cold / peak, 4),
                              "copy_cold_gbs": round(work / (ms_copy * 1e-3) / 1e9, 2)})
    return out


def pmc_run(cfg, path_name):
    """For `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE`: two passes of one launch of each
    block kernel (in KERNEL_ORDER; a step may be more than one dispatch, e.g. a GEMM whose last
    partial round runs as half tiles), each step followed by a small fill that separates it from
    the next, and each pass by a plain device copy of COPY_BYTES that scales the counters (the
    last pass is the one read)."""
    import torch
    kern = make_kernels(cfg, path_name)
    src = torch.zeros(COPY_BYTES // 4, device="cuda")
    dst = torch.empty_like(src)
    sep = torch.empty(64, device="cuda")
    for _ in range(2):
        for name in KERNEL_ORDER:
            kern[name][0]()
            torch.cuda.synchronize()
            sep.fill_(1.0)
            torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
    print("pmc run done: " + ", ".join(KERNEL_ORDER) + f", copy of {COPY_BYTES} bytes", flush=True)


def _counter_rows(path):
    import csv
    with open(path) as fh:
        rows = list(csv.DictReader(fh))
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    return rows


def _last_pass(rows, counter):
    """(per-step KiB in KERNEL_ORDER, copy KiB, kernel names) of the last pmc pass in a counter
    CSV.  A step's dispatches are the library's kernels between two separating fills; their
    readings are added."""
    rows = [r for r in rows if r["Counter_Name"] == counter]
    copy_idx = max(i for i, r in enumerate(rows) if "opy" in r["Kernel_Name"]
                   and "wenc" not in r["Kernel_Name"])
    groups, cur = [], []
    for r in rows[:copy_idx]:
        if "wenc::" in r["Kernel_Name"]:
            cur.append(r)
        elif cur:
            groups.append(cur)
            cur = []
    if cur:
        groups.append(cur)
    ours = groups[-len(KERNEL_ORDER):]
    return [sum(float(r["Counter_Value"]) for r in g) for g in ours], \
        float(rows[copy_idx]["Counter_Value"]), \
        [" + ".join(r["Kernel_Name"].split("(")[0] for r in g) for g in ours]


def ingest_pmc(cfg, path_name, fetch_csv, write_csv, command):
    """Scale the FETCH_SIZE / WRITE_SIZE readings (KiB per dispatch) by the copy's known bytes and
    store bytes per launch per kernel, with the hash of the sources they were taken on."""
    fetch, fcopy, names = _last_pass(_counter_rows(fetch_csv), "FETCH_SIZE")
    write, wcopy, _ = _last_pass(_counter_rows(write_csv), "WRITE_SIZE")
    f_fetch = COPY_BYTES / (fcopy * 1024.0)
    f_write = COPY_BYTES / (wcopy * 1024.0)
    out = {"command": command, "copy_bytes": COPY_BYTES,
           "copy_fetch_kib": fcopy, "copy_write_kib": wcopy,
           "scale_fetch": f_fetch, "scale_write": f_write, "kernels": {}}
    for i, name in enumerate(KERNEL_ORDER):
        srcs = KERNEL_SOURCES[name]
        out["kernels"][name] = {
            "kernel_name": names[i], "fetch_kib": fetch[i], "write_kib": write[i],
            "bytes_per_launch": round(fetch[i] * 1024 * f_fetch + write[i] * 1024 * f_write),
            "config": cfg.name, "path": path_name, "sources": srcs,
            "source_hash": source_hash(srcs)}
    with open(COUNTERS, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


DECODER_LAYERS = {384: 4, 512: 6, 768: 12, 1280: 32}  # Whisper tiny / base / small / large-v3


def time_cross_kv(cfg, path_name, reps):
    """The step after the encoder: cross-attention keys and values of every decoder layer of the
    matching Whisper size from the workload's encoder output, one C ABI call."""
    import torch
    from speech_transformer_encoder_amd import binding as B
    from speech_transformer_encoder_amd import synth
    path = B.PATHS[path_name]
    d, L = cfg.d_model, DECODER_LAYERS.get(cfg.d_model, 4)
    M = cfg.batch * cfg.t
    layers = synth.make_cross_layers(cfg.seed, L, d, bf16=cfg.bf16_weights)
    dev = lambda a: torch.from_numpy(a).cuda()  # noqa: E731
    blob = torch.empty(B.whisper_enc_cross_kv_bytes(d, L, path), dtype=torch.uint8, device="cuda")
    B.whisper_enc_pack_cross_kv([dev(q["wk"]) for q in layers], [dev(q["wv"]) for q in layers],
                                [dev(q["bv"]) for q in layers], L, d, path, blob)
    ws_bytes = B.whisper_enc_cross_kv_workspace_bytes(cfg.batch, cfg.t, d, path)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
    es = 4 if path_name == "fp32" else 2
    kv = torch.empty(cfg.batch * L * 2 * cfg.t * d * es, dtype=torch.uint8, device="cuda")
    y = torch.randn(cfg.batch, cfg.t, d, device="cuda")
    fn = lambda: B.whisper_enc_cross_kv(y, kv, blob, L, cfg.batch, cfg.t, d, cfg.heads, path,  # noqa: E731
                                        ws, ws.numel())
    ms = time_events(fn, reps, torch.cuda.current_stream())
    flops = 2.0 * M * (2 * L * d) * d
    tf = flops / (ms * 1e-3) / 1e12
    out = {"decoder_layers": L, "ms": round(ms, 4), "achieved": round(tf, 1), "unit": "TFLOP/s",
           "peak": PEAK_TFLOPS[path_name], "frac": round(tf / PEAK_TFLOPS[path_name], 4),
           "work": flops}
    del kv, blob, ws
    torch.cuda.empty_cache()
    return out


def time_stem(cfg, path_name, reps):
    """The step before the first block: the conv front end from 2 t mel frames (the matching
    Whisper size's mel bins) to the workload's t rows, one C ABI call (unfold, conv1 GEMM + GELU,
    stride-2 unfold + positions, conv2 GEMM + GELU + positions)."""
    import torch
    from speech_transformer_encoder_amd import binding as B
    from speech_transformer_encoder_amd import synth
    path = B.PATHS[path_name]
    d, t2 = cfg.d_model, cfg.t
    t_mel, n_mels = 2 * t2, synth.N_MELS.get(d, 80)
    p = synth.make_stem(cfg.seed, n_mels, d, bf16=cfg.bf16_weights, n_pos=t2)
    dev = lambda a: torch.from_numpy(a).cuda()  # noqa: E731
    blob = torch.empty(B.whisper_enc_stem_bytes(n_mels, d, t2, path), dtype=torch.uint8,
                       device="cuda")
    B.whisper_enc_pack_stem(dev(p["conv1_w"]), dev(p["conv1_b"]), dev(p["conv2_w"]),
                            dev(p["conv2_b"]), dev(p["pos"]), n_mels, d, t2, path, blob)
    ws_bytes = B.whisper_enc_stem_workspace_bytes(cfg.batch, t_mel, n_mels, d, path)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
    mel = torch.randn(cfg.batch, t_mel, n_mels, device="cuda")
    x = torch.empty(cfg.batch, t2, d, device="cuda")
    fn = lambda: B.whisper_enc_stem_forward(mel, x, blob, cfg.batch, t_mel, n_mels, d, t2, path,  # noqa: E731
                                            ws, ws.numel())
    ms = time_events(fn, reps, torch.cuda.current_stream())
    flops = 2.0 * cfg.batch * (t_mel * d * 3 * n_mels + t2 * d * 3 * d)
    tf = flops / (ms * 1e-3) / 1e12
    out = {"n_mels": n_mels, "mel_frames": t_mel, "ms": round(ms, 4), "achieved": round(tf, 1),
           "unit": "TFLOP/s", "peak": PEAK_TFLOPS[path_name],
           "frac": round(tf / PEAK_TFLOPS[path_name], 4), "work": flops}
    del blob, ws, mel, x
    torch.cuda.empty_cache()
    return out


def time_varlen(cfg, path_name, reps, enc, padded_ms):
    """The same stack over a ragged batch: as many windows, of 150 .. t rows (seeded uniform
    lengths), packed back to back with no padding; throughput counts real frames only.  Beside
    it, the real frames per second of the padded call (every window padded to t rows)."""
    import numpy as np
    import torch
    from speech_transformer_encoder_amd import binding as B
    from speech_transformer_encoder_amd import synth
    lens = synth.ragged_lengths(cfg.seed, cfg.batch, max_t=cfg.t)
    total, max_t = int(lens.sum()), int(lens.max())
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32), device="cuda")
    x = torch.randn(total, cfg.d_model, device="cuda")
    y = torch.empty_like(x)
    ws_bytes = B.whisper_enc_varlen_workspace_bytes(cfg.batch, total, max_t, cfg.d_model,
                                                    cfg.heads, cfg.ffn_dim, enc.path)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
    g, b = enc.ln_post if enc.ln_post is not None else (None, None)
    fn = lambda: B.whisper_enc_stack_forward_varlen(  # noqa: E731
        x, y, enc.blob, enc.n_layers, g, b, cu, cfg.batch, total, max_t, cfg.d_model, cfg.heads,
        cfg.ffn_dim, enc.path, ws, ws.numel())
    ms = time_events(fn, reps, torch.cuda.current_stream())
    out = {"windows": cfg.batch, "frames": total, "min_t": int(lens.min()), "max_t": max_t,
           "ms": round(ms, 4), "frames_per_s": round(total / (ms * 1e-3), 1),
           "padded_ms": round(padded_ms, 4),
           "padded_frames_per_s": round(total / (padded_ms * 1e-3), 1)}
    del x, y, ws
    torch.cuda.empty_cache()
    return out


def time_quantized(cfg, w, x, y, reps, bits):
    """The same block step with the weights stored as q8 / q4 blocks of 32 (expanded to fp16 by
    each block call); real frames per second and weight bytes at rest per layer."""
    import torch
    from speech_transformer_encoder_amd import binding as B
    from speech_transformer_encoder_amd.encoder import build_from_workload
    path = B.WENC_PATH_Q8 if bits == 8 else B.WENC_PATH_Q4
    ref = build_from_workload(w, B.WENC_PATH_FP16)
    enc = build_from_workload(w, path)
    ref.workspace(cfg.batch, cfg.t)
    enc.workspace(cfg.batch, cfg.t)
    st = torch.cuda.current_stream()
    # fp16 weights timed before and after, in the same loop, against order effects
    ms16a = time_events(lambda: ref.forward(x, y), reps, st)
    ms = time_events(lambda: enc.forward(x, y), reps, st)
    ms16 = 0.5 * (ms16a + time_events(lambda: ref.forward(x, y), reps, st))
    out = {"ms": round(ms, 4), "fp16_ms_same_loop": round(ms16, 4),
           "value": round(cfg.batch * cfg.t / (ms * 1e-3), 1), "unit": "frames/s",
           "layer_bytes": B.whisper_enc_layer_bytes(cfg.d_model, cfg.ffn_dim, path),
           "fp16_layer_bytes": B.whisper_enc_layer_bytes(cfg.d_model, cfg.ffn_dim,
                                                         B.WENC_PATH_FP16)}
    del enc, ref
    torch.cuda.empty_cache()
    return out


def time_graph(path_name, reps):
    """A launch-bound call: the base stack (6 blocks + final LayerNorm, one 1500-position window),
    called eagerly (7 launches per block from the host) and replayed from a HIP graph captured
    from the same C ABI call."""
    import torch
    from speech_transformer_encoder_amd import binding as B
    from speech_transformer_encoder_amd import synth
    from speech_transformer_encoder_amd.encoder import build_from_workload, to_device_input
    cfg = synth.CONFIGS["base_stack"]
    w = synth.make_workload(cfg)
    enc = build_from_workload(w, B.PATHS[path_name])
    x = to_device_input(w.x)
    y = torch.empty_like(x)
    enc.workspace(cfg.batch, cfg.t)
    st = torch.cuda.current_stream()
    eager = time_events(lambda: enc.forward(x, y), reps, st)
    s = torch.cuda.Stream()
    s.wait_stream(st)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            enc.forward(x, y, stream=s.cuda_stream)
    torch.cuda.synchronize()
    replay = time_events(graph.replay, reps, st)
    frames = cfg.batch * cfg.t
    out = {"workload": cfg.name, "blocks": cfg.n_layers, "eager_ms": round(eager, 4),
           "graph_ms": round(replay, 4), "eager_frames_per_s": round(frames / (eager * 1e-3), 1),
           "graph_frames_per_s": round(frames / (replay * 1e-3), 1)}
    del graph, enc
    torch.cuda.empty_cache()
    return out


def time_config(name, path_name, reps, peak, mpeak):
    """One whole workload as the C ABI call its name says (a block, or a stack of all its blocks
    plus the final LayerNorm), timed with HIP events on the launch stream: ms per call, frames/s
    and the algorithmic TFLOP/s of the call."""
    import torch
    from speech_transformer_encoder_amd import binding as B
    from speech_transformer_encoder_amd import synth
    from speech_transformer_encoder_amd.encoder import build_from_workload, to_device_input
    cfg = synth.CONFIGS[name]
    w = synth.make_workload(cfg)
    enc = build_from_workload(w, B.PATHS[path_name])
    x = to_device_input(w.x)
    y = torch.empty_like(x)
    enc.workspace(cfg.batch, cfg.t)
    del w
    ms = time_events(lambda: enc.forward(x, y), reps, torch.cuda.current_stream())
    fl = cfg.flops()
    tf = fl["total"] / (ms * 1e-3) / 1e12
    pk = PEAK_TFLOPS[path_name]
    out = {"path": path_name, "blocks": cfg.n_layers, "batch_windows": cfg.batch,
           "final_layernorm": cfg.ln_post, "ms": round(ms, 4),
           "ms_per_block": round(ms / cfg.n_layers, 4),
           "frames_per_s": round(cfg.batch * cfg.t / (ms * 1e-3), 1),
           "tflops": round(tf, 1), "frac_peak": round(tf / pk, 4),
           "frac_measured_peak": round(tf / mpeak, 4) if (mpeak and path_name != "fp32") else None}
    del enc, x, y
    torch.cuda.empty_cache()
    return out


def cpu_baseline(cfg, windows, layers):
    """The oracle as it stands, on a bounded sample of the workload (first windows / layers)."""
    import numpy as np
    import oracle
    from speech_transformer_encoder_amd import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as fh:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")),
                             None)
    except OSError:
        pass
    nw = min(windows, cfg.batch)
    nl = min(layers, cfg.n_layers)
    sub = cfg.with_(batch=nw, n_layers=nl)
    w = synth.make_workload(sub)
    t0 = time.perf_counter()
    y = oracle.encoder_stack(w.x, w.layers, cfg.heads, w.ln_post if nl == cfg.n_layers else None)
    dt = time.perf_counter() - t0
    assert np.isfinite(y).all()
    # frames/s of the full workload: the sample did nw/batch of the windows and nl/n_layers of
    # the blocks, so the full call would take dt * (batch/nw) * (n_layers/nl).
    full_s = dt * (cfg.batch / nw) * (cfg.n_layers / nl)
    return {"value": round(cfg.batch * cfg.t / full_s, 2), "unit": "frames/s", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model, "nproc": os.cpu_count(),
            "sample": f"{nw} of {cfg.batch} windows x {nl} of {cfg.n_layers} blocks "
                      f"({dt:.1f} s float64 numpy, scaled to the full workload)"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(windows shard by data parallelism with no exchange between GPUs). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np  # noqa: F401
    import torch
    from speech_transformer_encoder_amd import binding as B
    from speech_transformer_encoder_amd import synth
    from speech_transformer_encoder_amd.encoder import build_from_workload, to_device_input

    cfg = synth.CONFIGS[args.config]
    if args.ingest_pmc:
        ingest_pmc(cfg, args.path, args.ingest_pmc[0], args.ingest_pmc[1], args.pmc_command)
        return
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    B.load()
    if args.pmc_run:
        if args.path == "mxfp8":
            sys.exit("--pmc-run times the 16-bit block kernels: use --path fp16 or bf16")
        pmc_run(cfg, args.path)
        return
    path = B.PATHS[args.path]
    w = synth.make_workload(cfg)
    x = to_device_input(w.x)
    y = torch.empty_like(x)
    st = torch.cuda.current_stream()

    def time_forward(enc):
        enc.workspace(cfg.batch, cfg.t)
        # Clock settling: from idle, the first few milliseconds of steps run at lower clocks (a
        # 5-step warm-up then measures ~4 % slow); a few hundred ms of steps, in synchronized
        # chunks so that the queue stays short, reach the sustained rate.
        t_settle = time.perf_counter() + args.settle_ms * 1e-3
        while time.perf_counter() < t_settle:
            for _ in range(10):
                enc.forward(x, y)
            torch.cuda.synchronize()
        for _ in range(args.warmup):
            enc.forward(x, y)
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        s.record(st)
        for _ in range(args.steps):
            enc.forward(x, y)
        e.record(st)
        torch.cuda.synchronize()
        return s.elapsed_time(e) / args.steps, time.perf_counter() - t0

    enc_main = build_from_workload(w, path)
    ms, wall = time_forward(enc_main)
    others = {}
    for pn in [p for p in args.compare_paths.split(",") if p and p != args.path]:
        oms, _ = time_forward(build_from_workload(w, B.PATHS[pn]))
        others[pn] = {"value": round(cfg.batch * cfg.t / (oms * 1e-3), 1), "ms_per_step": round(oms, 4)}
        if pn == "mxfp8":
            others[pn]["kernels"] = mx_kernel_breakdown(cfg, args.kernel_reps)
            if not args.no_other_configs and cfg.name != "large_v3_stack":
                others[pn]["large_v3_stack"] = time_config("large_v3_stack", "mxfp8",
                                                           args.kernel_reps, PEAK_TFLOPS["mxfp8"],
                                                           None)
    frames = cfg.batch * cfg.t
    flops = cfg.flops()

    if args.path == "mxfp8":
        # The MXFP8 step's own kernels (LN with MXFP8 output, QKV / fc1 / fc2 on MXFP8 operands)
        # and the fp16 attention and out-projection it keeps.
        kern16 = kernel_breakdown(cfg, "fp16", args.kernel_reps)
        kern = mx_kernel_breakdown(cfg, args.kernel_reps)
        kern["attention"] = kern16["attention"]
        kern["gemm_out_residual"] = kern16["gemm_out_residual"]
    else:
        kern = kernel_breakdown(cfg, args.path, args.kernel_reps)
    # Kernel time per step: every kernel runs once per block (LN twice), n_layers blocks.
    for k in kern.values():
        k["ms_per_step"] = round(k["ms"] * k["launches_per_block"] * cfg.n_layers, 4)
    dom_name = max(kern, key=lambda n: kern[n]["ms_per_step"])
    dom = kern[dom_name]
    traffic = None
    if os.path.exists(COUNTERS):
        with open(COUNTERS) as fh:
            c = json.load(fh)
        ent = c.get("kernels", {}).get(dom_name)
        if ent and ent.get("source_hash") == source_hash(ent.get("sources", [])) \
                and ent.get("config") == args.config and ent.get("path") == args.path:
            traffic = ent.get("bytes_per_launch")
    roof = {"kernel": dom_name, "bound": dom["bound"], "achieved": dom["achieved"],
            "peak": dom["peak"], "unit": dom["unit"], "frac": dom["frac"], "traffic": traffic,
            "work_per_launch": dom["work"], "ms_per_launch": dom["ms"]}

    gemm_ms = sum(v["ms_per_step"] for n, v in kern.items() if n.startswith("gemm"))
    attn_ms = kern["attention"]["ms_per_step"]
    gemm_tf = flops["gemm"] / (gemm_ms * 1e-3) / 1e12
    attn_tf = flops["attention"] / (attn_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[args.path]
    measured = mfma_peak(args.path)
    mpeak = measured["tflops"] if measured else None
    # On the MXFP8 path attention and the out-projection run fp16 MFMAs: their peaks are fp16's.
    attn_peak, attn_mpeak = peak, mpeak
    if args.path == "mxfp8":
        m16 = mfma_peak("fp16")
        attn_peak, attn_mpeak = PEAK_TFLOPS["fp16"], m16["tflops"]
        measured = {"mxfp8": measured, "fp16": m16}
    if mpeak and roof["unit"] == "TFLOP/s":
        rm = attn_mpeak if dom_name in ("attention", "gemm_out_residual") else mpeak
        roof["measured_peak"] = rm
        roof["frac_measured_peak"] = round(roof["achieved"] / rm, 4)

    # Every other workload, timed whole (the 32-block large-v3 stack as one call), on the same
    # operand type; and the fp32 fallback path on the bench workload itself.
    configs = {}
    if not args.no_other_configs:
        for name in synth.CONFIGS:
            if name != cfg.name:
                configs[name] = time_config(name, args.path, args.kernel_reps, peak, mpeak)
        if args.path != "fp32":
            configs[cfg.name + "/fp32"] = time_config(cfg.name, "fp32", max(3, args.kernel_reps // 3),
                                                      PEAK_TFLOPS["fp32"], None)

    next_steps = {}
    if not args.no_next_steps and args.path != "mxfp8":  # the adjacent steps have no MXFP8 form
        next_steps["stem"] = time_stem(cfg, args.path, args.kernel_reps)
        next_steps["cross_kv"] = time_cross_kv(cfg, args.path, args.kernel_reps)
        next_steps["varlen"] = time_varlen(cfg, args.path, args.kernel_reps, enc_main, ms)
        next_steps["graph"] = time_graph(args.path, args.kernel_reps)
        if args.path == "fp16":
            next_steps["q8_weights"] = time_quantized(cfg, w, x, y, args.kernel_reps, 8)
            next_steps["q4_weights"] = time_quantized(cfg, w, x, y, args.kernel_reps, 4)
            # One window, where the weights are a larger share of each block's bytes: four
            # large-v3 blocks and the final norm.
            c1 = synth.CONFIGS["large_v3_stack"].with_(n_layers=4)
            w1 = synth.make_workload(c1)
            x1 = to_device_input(w1.x)
            y1 = torch.empty_like(x1)
            for bits in (8, 4):
                q = time_quantized(c1, w1, x1, y1, args.kernel_reps, bits)
                q["blocks"] = c1.n_layers
                next_steps[f"q{bits}_weights_one_window"] = q
            del w1, x1, y1

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, args.cpu_sample_windows, args.cpu_sample_layers)

    out = {
        "metric": METRIC, "value": round(frames / (ms * 1e-3), 1), "unit": "frames/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "settle_ms": args.settle_ms,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": args.path,
        "data": "synthetic (seeded N(0,1) inputs, N(0,0.02^2) weights; no checkpoint)",
        "config": {"workload": cfg.name, "batch_windows": cfg.batch, "t": cfg.t,
                   "d_model": cfg.d_model, "heads": cfg.heads, "ffn_dim": cfg.ffn_dim,
                   "n_layers": cfg.n_layers, "final_layernorm": cfg.ln_post,
                   "weights": "bf16-valued" if cfg.bf16_weights else "fp32",
                   "operands": args.path, "parallelism": "single GPU"},
        "tflops": {"total": round(flops["total"] / (ms * 1e-3) / 1e12, 1),
                   "gemm": round(gemm_tf, 1), "gemm_frac_peak": round(gemm_tf / peak, 4),
                   "attention": round(attn_tf, 1), "attention_frac_peak": round(attn_tf / attn_peak, 4),
                   "peak": peak, "measured_peak": mpeak,
                   "gemm_frac_measured_peak": round(gemm_tf / mpeak, 4) if mpeak else None,
                   "attention_frac_measured_peak": (round(attn_tf / attn_mpeak, 4)
                                                    if attn_mpeak else None),
                   "gemm_peak_note": ("the out-projection (fp16) is counted in the GEMM rate, "
                                      "priced at the fp8 peak" if args.path == "mxfp8" else None)},
        "mfma_peak_measured": measured,
        "configs": configs,
        "roofline": roof,
        "kernels": kern,
        "wall_s_timed": round(wall, 4),
        "cpu_baseline": cpu,
        "other_paths": others,
        "next_steps": next_steps,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
