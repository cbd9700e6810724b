"""Benchmark of the NVFP4 quantized-linear hot path on one MI355X.

One step = forward + backward of the dense linear layer
X [8192 x 4096] (BF16), W [14336 x 4096] (BF16), dY [8192 x 14336] (BF16):
  1 quantize X   row-wise 1x16 RTN + column-wise 1x16 RHT SR   (one read of X)
  2 quantize W   16x16 RTN
  3 fprop        Y  = Xq Wq^T       NVFP4 GEMM, BF16 out
  4 quantize dY  column-wise 1x16 RHT SR + row-wise MXFP8 SR  (one read of dY)
  5 requantize   Wq -> MXFP8 of Wq^T, SR
  6 dgrad        dX = dY W          MXFP8 GEMM, BF16 out
  7 wgrad        dW = dY^T X        NVFP4 GEMM over the RHT'd copies, FP32 out
Inputs are seeded synthetic tensors resident in HBM before timing starts.
Prints one JSON line (value = whole-step GEMM TFLOP/s including every
quantize pass), with per-kernel times, a roofline entry for the fprop GEMM,
the CPU oracle timed on a bounded sample and, from the same oracle, parity
counts for the outputs of the timed kernels.

Per-kernel times: 10 warm-up calls, then 100 back-to-back calls with a HIP
event after every 10; "ms" is the median of the ten 10-call means and
"ms_mean" the mean of a second batch of 100 calls timed by two events only
(the average launch duration, comparable with a rocprofv3 kernel trace).
Every timed call, in the step and in the sections after it, cycles through
ROTATE buffer sets so that its inputs are not resident in the 256 MB MALL.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

M, K, N = 8192, 4096, 14336
GEMM_FLOP = 2.0 * M * N * K                     # 962.07 GFLOP per GEMM
PEAK_HBM_GBPS = 8000.0
PEAK_FP16_TFLOPS = 2500.0                      # MFMA class the NVFP4 GEMM issues (fp16)
PEAK_FP8_TFLOPS = 5000.0
PEAK_FP4_TFLOPS = 10100.0
COPY_BYTES = 1 << 29                            # counter calibration copy (512 MiB)

ROTATE = 8                                     # buffer sets the timed runs cycle through
# HBM bytes per launch of the fprop GEMM, from rocprofv3 FETCH_SIZE and
# WRITE_SIZE runs scaled by what the same counters read for the 512 MiB copy
# (profiles/sq_hbm_counters_step_kernels_8192x4096x14336.md), valid only for the kernel
# sources they were taken on: reported as null once those sources change.
FPROP_TRAFFIC = {"bytes": 626723567, "sources_sha256_16": "9210d85e89b17c03"}
FPROP_SOURCES = ["bit_block_scaled_amd/csrc/gemm_nvfp4.hip", "bit_block_scaled_amd/csrc/bbs_device.hpp",
                 "bit_block_scaled_amd/csrc/bbs_kernels.hpp", "bit_block_scaled_amd/build.py"]


def fprop_traffic():
    import hashlib
    h = hashlib.sha256()
    for f in FPROP_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return FPROP_TRAFFIC["bytes"] if h.hexdigest()[:16] == FPROP_TRAFFIC["sources_sha256_16"] else None


def nvfp4_bytes(r, c):
    return r * c // 2 + r * c // 16


def time_calls(torch, calls, n=100, warm=10, group=10):
    """calls: callables cycled through in order (one per buffer set).  After
    `warm` calls, n back-to-back calls in groups of `group` with a HIP event
    between groups (an event between every two calls adds about 3 us to each
    interval on this GPU).  Returns (median of the group means, mean over a
    separate batch of n calls between two events)."""
    k = len(calls)
    group = max(1, min(group, n))
    for i in range(warm):
        calls[i % k]()
    ng = n // group
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(ng + 1)]
    ev[0].record()
    for gi in range(ng):
        for j in range(group):
            calls[(warm + gi * group + j) % k]()
        ev[gi + 1].record()
    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    b0.record()
    for i in range(n):
        calls[(warm + n + i) % k]()
    b1.record()
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) / group for i in range(ng)]
    return float(np.median(per)), b0.elapsed_time(b1) / n


def gemm_entry(t_med, t_mean, flop, own_peak, own_name, issued_peak=None):
    tf = flop / (t_med * 1e-3) / 1e12
    e = {"ms": round(t_med, 4), "ms_mean": round(t_mean, 4), "TFLOP/s": round(tf, 1),
         f"frac_{own_name}_peak": round(tf / own_peak, 4)}
    if issued_peak is not None:
        e["frac_fp16_mfma_peak"] = round(tf / issued_peak, 4)
    return e


def bytes_entry(t_med, t_mean, b):
    gbps = b / (t_med * 1e-3) / 1e9
    return {"ms": round(t_med, 4), "ms_mean": round(t_mean, 4), "GB/s": round(gbps, 1),
            "hbm_frac": round(gbps / PEAK_HBM_GBPS, 4), "bytes": b}


def two_pass_bytes():
    """Bytes each quantize op moves through HBM: the amax pass's read of the
    source, then the encode's read and its outputs (the requantize is one
    pass)."""
    ab = algorithmic_bytes()
    return {"quant_x": ab["quant_x"] + 2 * M * K, "quant_w": ab["quant_w"] + 2 * N * K,
            "quant_dy": ab["quant_dy"] + 2 * M * N, "requant_w": ab["requant_w"]}


def algorithmic_bytes():
    """Bytes each memory-bound pass must move (one read of its input + its outputs)."""
    x_in, w_in, dy_in = 2 * M * K, 2 * N * K, 2 * M * N
    return {
        "quant_x": x_in + nvfp4_bytes(M, K) + nvfp4_bytes(K, M),
        "quant_w": w_in + (N * K // 2 + (N // 16) * (K // 16)),
        "quant_dy": dy_in + nvfp4_bytes(N, M) + (M * N + M * N // 32),
        "requant_w": (N * K // 2 + (N // 16) * (K // 16)) + (K * N + K * N // 32),
    }


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-moe", action="store_true",
                    help="skip the grouped-GEMM (MoE expert forward) measurement")
    ap.add_argument("--only", default=None,
                    help="time one op of the step in isolation (quant_x, quant_w, fprop, "
                         "quant_dy, requant_w, dgrad, wgrad), 'moe' (the grouped-GEMM "
                         "expert forward alone) or 'copy' (a plain 512 MiB device copy); used "
                         "for counter and trace runs")
    return ap.parse_args()


def cpu_baseline(full_quant=None):
    """The oracle, as it stands, on a bounded sample of the same step: the
    quantize parts at full size when the parity leg has timed them
    (full_quant), else on the slices below; the FP64 GEMMs on slices, each
    scaled to the full size by the share of work sampled."""
    import oracle as O
    from workloads import synth
    ms, ns = 512, 2048                    # sampled token rows / weight rows
    x = synth.normal_with_outliers(ms, K, 301)
    w = synth.normal(ns, K, 302, 0.02)
    dy = synth.laplace(ms, N, 401, 1e-3)
    s = synth.rht_signs(402)
    t = {}
    t0 = time.perf_counter()
    xq = O.nvfp4_quantize(x)
    xc = O.nvfp4_quantize(x, transpose=True, rht=True, signs=s, mode=O.SR, seed=405)
    t["quant_x"] = (time.perf_counter() - t0) * (M / ms)
    t0 = time.perf_counter()
    wq = O.nvfp4_quantize(w, tile2d=True)
    t["quant_w"] = (time.perf_counter() - t0) * (N / ns)
    t0 = time.perf_counter()
    gc = O.nvfp4_quantize(dy, transpose=True, rht=True, signs=s, mode=O.SR, seed=403)
    gm = O.mxfp8_quantize(dy, mode=O.SR, seed=404)
    t["quant_dy"] = (time.perf_counter() - t0) * (M / ms)
    t0 = time.perf_counter()
    wt = O.mxfp8_requantize_t(wq, mode=O.SR, seed=406)
    t["requant_w"] = (time.perf_counter() - t0) * (N / ns)
    if full_quant:
        t.update(full_quant)
    # GEMMs: FP64 over dequantized operands, on ms x ns outputs
    t0 = time.perf_counter()
    O.gemm_f64(xq.dequant_f64(), wq.dequant_f64())
    t["fprop"] = (time.perf_counter() - t0) * (M / ms) * (N / ns)
    t0 = time.perf_counter()
    # dX sample: ms x K outputs over an ns-wide slice of the contraction dim N
    O.gemm_f64(np.ascontiguousarray(gm.dequant_f64()[:, :ns]), wt.dequant_f64())
    t["dgrad"] = (time.perf_counter() - t0) * (M / ms) * (N / ns)
    t0 = time.perf_counter()
    O.gemm_f64(gc.dequant_f64()[:ns], xc.dequant_f64()[:ns])
    t["wgrad"] = (time.perf_counter() - t0) * (N / ns) * (K / ns) * (M / ms)
    total = sum(t.values())
    return {
        "value": round(3 * GEMM_FLOP / total / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": O.num_threads(),
        "kind": "oracle",
        "sample": ((("quantize passes (X, W, dY, W requantize) at full size; " if full_quant else
                     f"quantize passes on X/dY slices of {ms} token rows and a W slice of {ns} "
                     f"rows; ") +
                    f"FP64 GEMMs on slices: fprop on {ms}x{ns} outputs, dgrad on {ms}x{K} outputs "
                    f"over {ns} of N, wgrad on {ns}x{ns} outputs over {ms} tokens; each sliced "
                    f"part's time scaled to the full step by its work ratio")),
        "extrapolated_step_s": round(total, 2),
        "parts_s": {k: round(v, 2) for k, v in t.items()},
    }


def sample_positions(rows, cols, per_tile, seed, tile=256):
    """per_tile random outputs inside every tile x tile output tile, plus the
    last row's first and last 64 columns (the ragged edge of any tiling)."""
    rng = np.random.default_rng(seed)
    tm, tn = -(-rows // tile), -(-cols // tile)
    ti = np.repeat(np.arange(tm), tn * per_tile)
    tj = np.tile(np.repeat(np.arange(tn), per_tile), tm)
    r = np.minimum(ti * tile + rng.integers(0, tile, ti.size), rows - 1)
    c = np.minimum(tj * tile + rng.integers(0, tile, tj.size), cols - 1)
    edge = np.concatenate([np.arange(64), np.arange(cols - 64, cols)])
    r = np.concatenate([r, np.full(edge.size, rows - 1)])
    c = np.concatenate([c, edge])
    return r.astype(np.int64), c.astype(np.int64)


GEMM_SAMPLES = {"fprop": (M, N, 1), "dgrad": (M, K, 2), "wgrad": (N, K, 2)}


def capture_outputs(torch, b):
    """Host copies of one step's outputs: every quantized copy whole, the GEMM
    outputs at sampled positions (2 per 256 x 256 tile of dX and dW, 1 of Y,
    and the ragged edge)."""
    def nv(q):
        return (q.codes.cpu().numpy(), q.scales.cpu().numpy(), float(q.s_dec[0]))

    def mx(q):
        return (q.codes.cpu().numpy(), q.scales.cpu().numpy())

    cap = {"xq": nv(b["xq"]), "xc": nv(b["xc"]), "wq": nv(b["wq"]), "gc": nv(b["gc"]),
           "gm": mx(b["gm"]), "wt": mx(b["wt"])}
    for name, key in (("fprop", "y"), ("dgrad", "dx"), ("wgrad", "dw")):
        R, Cn, per_tile = GEMM_SAMPLES[name]
        r, c = sample_positions(R, Cn, per_tile, 900 + len(name))
        out = b[key]
        g = out[torch.from_numpy(r).to(out.device), torch.from_numpy(c).to(out.device)].cpu()
        if key == "dw":
            v = g.numpy().astype(np.float64)
        else:
            v = ((g.numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32)
                 .astype(np.float64))
        cap[name] = (r, c, v)
    return cap


def parity(cap, host_in, signs, seeds):
    """The timed kernels' outputs of one step against the oracle run on the
    same inputs: equal bytes of every quantized copy (codes, scales and the
    FP32 decode scale), and for each GEMM the sampled outputs against the
    FP64 product of the oracle's own copies, with the rigorous FP32
    accumulation bound (K + 4) 2^-24 sum|a b| plus the output rounding."""
    import oracle as O
    t0 = time.perf_counter()
    x, w, dy = host_in["x"], host_in["w"], host_in["dy"]
    ref, op_s = {}, {}

    def timed(op, fn):
        t1 = time.perf_counter()
        fn()
        op_s[op] = time.perf_counter() - t1

    timed("quant_x", lambda: ref.update(
        xq=O.nvfp4_quantize(x),
        xc=O.nvfp4_quantize(x, transpose=True, rht=True, signs=signs, mode=O.SR,
                            seed=seeds["x_col"], stream=0)))
    timed("quant_w", lambda: ref.update(wq=O.nvfp4_quantize(w, tile2d=True)))
    timed("quant_dy", lambda: ref.update(
        gc=O.nvfp4_quantize(dy, transpose=True, rht=True, signs=signs, mode=O.SR,
                            seed=seeds["dy_col"], stream=0),
        gm=O.mxfp8_quantize(dy, mode=O.SR, seed=seeds["dy_mx8"], stream=0)))
    timed("requant_w", lambda: ref.update(
        wt=O.mxfp8_requantize_t(ref["wq"], mode=O.SR, seed=seeds["w_req"], stream=0)))
    t_quant = time.perf_counter() - t0
    res = {}
    for key in ("xq", "xc", "wq", "gc", "gm", "wt"):
        o, g = ref[key], cap[key]
        total = o.codes.size + o.scales.size
        equal = int((g[0] == o.codes).sum()) + int((g[1] == o.scales).sum())
        e = {"bytes": total, "equal": equal}
        if len(g) == 3:
            e["s_dec_equal"] = bool(np.float32(g[2]) == np.float32(o.s_dec))
        res[key] = e
    gemms = {"fprop": (ref["xq"], ref["wq"], K, "bf16"),
             "dgrad": (ref["gm"], ref["wt"], N, "bf16"),
             "wgrad": (ref["gc"], ref["xc"], M, "f32")}
    for name, (qa, qb, kc, out_t) in gemms.items():
        r, c, v = cap[name]
        A, B = qa.dequant_f64(), qb.dequant_f64()
        y = O.gemm_f64_sampled(A, B, r, c)
        a_abs = O.gemm_f64_sampled(np.abs(A), np.abs(B), r, c)
        del A, B
        acc = (kc + 4) * 2.0 ** -24 * a_abs
        rnd = 2.0 ** -8 if out_t == "bf16" else 2.0 ** -24
        bound = acc + rnd * (np.abs(y) + acc)
        err = np.abs(v - y)
        ratio = err / np.where(bound > 0, bound, np.inf)
        res[name] = {"samples": int(v.size), "within_bound": int((err <= bound).sum()),
                     "max_err_over_bound": float(ratio.max()),
                     "rel_fro": O.rel_fro(v, y),
                     "max_abs_err": float(err.max())}
    res["oracle_s"] = round(time.perf_counter() - t0, 2)
    res["oracle_quantize_full_size_s"] = round(t_quant, 2)
    return res, op_s


def moe_bench(torch, bbs, dev, reps):
    """The MoE expert forward (grouped NVFP4 GEMMs) at its full shape: 65536
    tokens x hidden 4096, 64 experts, top-8 Zipf(1.1) routing with 4 empty
    experts; up-projection 4096 -> 1536 over the gathered routed rows, then
    the up output is quantized (1x16, RTN) and projected 1536 -> 4096.  Each
    expert's weight is its own NVFP4 tensor (16x16 scales, own s_dec).  The
    down output then goes through the combine wire format (RHT-32 + S2F6
    encode; weighted sum of each token's 8 rows + inverse RHT)."""
    from workloads import synth
    T_, H_, F_, E_, K_ = 65536, 4096, 1536, 64, 8
    d = synth.moe_forward(T_, H_, F_, E_, K_, with_weights=False)
    rows = int(d["group_offsets"][-1])
    x = torch.from_numpy(d["x"].view(np.int16)).to(dev)
    ri = torch.from_numpy(d["row_index"]).to(dev)
    off = torch.from_numpy(d["group_offsets"]).to(dev)
    # the combine: each token's K rows of the down output (expert order)
    src = torch.from_numpy(np.argsort(d["row_index"], kind="stable").astype(np.int32)
                           .reshape(T_, K_)).to(dev)
    gate = torch.softmax(torch.randn((T_, K_), generator=torch.Generator().manual_seed(702)),
                         dim=1).to(dev)
    del d
    ws = bbs.amax_workspace(dev)
    N4 = bbs.NVFP4Tensor

    def stacked(n, k, seed0):
        st = N4.empty(E_ * n, k, tile2d=True, n_scales=E_, device=dev)
        for g in range(E_):
            w = torch.from_numpy(synth.normal(n, k, seed0 + g, 0.02).view(np.int16)).to(dev)
            view = N4(st.codes[g * n:(g + 1) * n], st.scales[g * n // 16:(g + 1) * n // 16],
                      st.s_dec[g:g + 1], n, k, True)
            bbs.nvfp4_quantize(w, view, tile2d=True, amax_ws=ws)
        return st

    w_up = stacked(F_, H_, 503)
    w_dn = stacked(H_, F_, 503 + E_)
    xq = N4.empty(T_, H_, device=dev)
    bbs.nvfp4_quantize(x, xq, amax_ws=ws)
    h = torch.empty((rows, F_), dtype=torch.int16, device=dev)
    hq = N4.empty(rows, F_, device=dev)
    y = torch.empty((rows, H_), dtype=torch.int16, device=dev)
    yq = bbs.S2F6Tensor.empty(rows, H_, device=dev)
    yq2 = bbs.S2F6Tensor.empty(rows, H_, device=dev)
    hq2 = N4.empty(rows, F_, device=dev)
    amax_h = torch.zeros(1, dtype=torch.float32, device=dev)
    s_h = torch.ones(1, dtype=torch.float32, device=dev)
    bbs.grouped_nvfp4_gemm_quant(xq, ri, off, E_, rows, w_up, F_, s_h, hq2, amax=amax_h)
    torch.cuda.synchronize()
    s_h.fill_(2688.0 / max(float(amax_h[0]), 1e-30))
    comb = torch.empty((T_, H_), dtype=torch.int16, device=dev)
    signs = 0xB5297A4D
    ops = {
        "moe_up": lambda: bbs.grouped_nvfp4_gemm(xq, ri, off, E_, rows, w_up, F_, h, bbs.OUT_BF16),
        "moe_quant_h": lambda: bbs.nvfp4_quantize(h, hq, amax_ws=ws),
        "moe_down": lambda: bbs.grouped_nvfp4_gemm(hq, None, off, E_, rows, w_dn, H_, y,
                                                   bbs.OUT_BF16),
        # the up-projection with the quantize in its epilogue (scale from the
        # first call's amax), in place of moe_up + moe_quant_h
        "moe_up_quant": lambda: bbs.grouped_nvfp4_gemm_quant(xq, ri, off, E_, rows, w_up, F_,
                                                             s_h, hq2, amax=amax_h),
        # combine wire format: RHT-32 + S2F6 encode of the down output, then
        # the receiver's weighted sum over each token's K rows + inverse RHT
        "combine_encode": lambda: bbs.s2f6_quantize(y, yq, rht=True, signs=signs),
        # the down projection with that encode in its epilogue, in place of
        # moe_down + combine_encode (the BF16 output never goes to memory)
        "moe_down_s2f6": lambda: bbs.grouped_nvfp4_gemm_s2f6(hq, None, off, E_, rows, w_dn, H_, yq2,
                                                             rht=True, signs=signs),
        "combine_decode": lambda: bbs.s2f6_combine(yq, src, comb, gate, rht=True, signs=signs),
    }
    codec_bytes = {"combine_encode": rows * H_ * 2 + rows * H_ + rows * H_ // 32,
                   "combine_decode": rows * (H_ + H_ // 32) + rows * 8 + T_ * H_ * 2}
    # The working set (1.6 GB up output, 0.4 GB weights) is far above the
    # MALL, so the ops run on one buffer set.
    out = {}
    flop = 2.0 * rows * F_ * H_
    hq_bytes = rows * F_ * 2 + rows * F_ // 2 + rows * F_ // 16
    for name, f in ops.items():
        t_med, t_mean = time_calls(torch, [f], n=reps, warm=min(10, reps))
        if name in codec_bytes:
            e = bytes_entry(t_med, t_mean, codec_bytes[name])
        elif name == "moe_quant_h":
            e = bytes_entry(t_med, t_mean, hq_bytes)
        else:
            e = gemm_entry(t_med, t_mean, flop, PEAK_FP4_TFLOPS, "fp4", PEAK_FP16_TFLOPS)
        out[name] = e
    out["routed_rows"] = rows
    out["flop_per_projection"] = 2.0 * rows * F_ * H_
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    dev = torch.device("cuda:0")
    if args.only == "copy":
        # a plain copy of known size: calibrates the HBM byte counters
        src = torch.ones(COPY_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"only": "copy", "bytes": COPY_BYTES}), flush=True)
        return
    import bit_block_scaled_amd as bbs
    from workloads import synth
    if args.only == "moe":
        res = moe_bench(torch, bbs, dev, max(3, args.steps // 4))
        print(json.dumps({"only": "moe", **res}), flush=True)
        return

    fw = synth.dense_forward(M, K, N)
    bw = synth.backward(M, N)
    signs, seeds = bw["rht_signs"], bw["seeds"]
    want_oracle = not args.no_cpu_baseline

    def up(a):
        return torch.from_numpy(a.view(np.int16)).to(dev)

    x0, w0, dy0 = up(fw["x"]), up(fw["w"]), up(bw["dy"])
    host_in = {"x": fw["x"], "w": fw["w"], "dy": bw["dy"]} if want_oracle else None
    del fw, bw
    T = bbs.NVFP4Tensor
    ws = bbs.amax_workspace(dev)

    def make_set(x, w, dy):
        """One complete set of the step's buffers (inputs, copies, outputs)."""
        xq, xc = T.empty(M, K, device=dev), T.empty(K, M, device=dev)
        wq = T.empty(N, K, tile2d=True, device=dev)
        gc = T.empty(N, M, device=dev)
        gm = bbs.MXFP8Tensor.empty(M, N, device=dev)
        wt = bbs.MXFP8Tensor.empty(K, N, device=dev)
        y = torch.empty((M, N), dtype=torch.int16, device=dev)
        dx = torch.empty((M, K), dtype=torch.int16, device=dev)
        dw = torch.empty((N, K), dtype=torch.float32, device=dev)
        bufs = {"x": x, "w": w, "dy": dy, "xq": xq, "xc": xc, "wq": wq, "gc": gc, "gm": gm,
                "wt": wt, "y": y, "dx": dx, "dw": dw}
        return bufs, {
            "quant_x": lambda: bbs.nvfp4_quantize(x, xq, xc, col_round=bbs.SR,
                                                  col_rng=(seeds["x_col"], 0), col_rht=True,
                                                  rht_signs=signs, amax_ws=ws),
            "quant_w": lambda: bbs.nvfp4_quantize(w, wq, tile2d=True, amax_ws=ws),
            "fprop": lambda: bbs.nvfp4_gemm(bbs.FMT_NVFP4, xq, wq, y, bbs.OUT_BF16),
            "quant_dy": lambda: bbs.nvfp4_quantize(dy, None, gc, gm, col_round=bbs.SR,
                                                   col_rng=(seeds["dy_col"], 0), col_rht=True,
                                                   rht_signs=signs, mx8_round=bbs.SR,
                                                   mx8_rng=(seeds["dy_mx8"], 0), amax_ws=ws),
            "requant_w": lambda: bbs.mxfp8_requantize_t(wq, wt, bbs.SR, (seeds["w_req"], 0)),
            "dgrad": lambda: bbs.nvfp4_gemm(bbs.FMT_MXFP8, gm, wt, dx, bbs.OUT_BF16),
            "wgrad": lambda: bbs.nvfp4_gemm(bbs.FMT_NVFP4, gc, xc, dw, bbs.OUT_F32),
        }

    # Timed runs rotate over ROTATE complete buffer sets (about 1.3 GB each,
    # the same values in every set), so no kernel finds its inputs in the
    # 256 MB MALL from the previous launch; --only (the counter runs) uses one.
    n_sets = 1 if args.only else ROTATE
    sets_b, sets_o = [], []
    for i in range(n_sets):
        bset, oset = make_set(x0, w0, dy0) if i == 0 else make_set(x0.clone(), w0.clone(),
                                                                   dy0.clone())
        sets_b.append(bset)
        sets_o.append(oset)
    ops = sets_o[0]

    def step(i=0):
        for f in sets_o[i % n_sets].values():
            f()

    if args.only:
        # inputs of the op come from one untimed step
        step()
        torch.cuda.synchronize()
        f = ops[args.only]
        for _ in range(args.warmup):
            f()
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record()
        for _ in range(args.steps):
            f()
        s1.record()
        torch.cuda.synchronize()
        print(json.dumps({"only": args.only, "ms": s0.elapsed_time(s1) / args.steps}), flush=True)
        return

    for i in range(max(args.warmup, n_sets)):
        step(i)
    torch.cuda.synchronize()
    print(f"[bench] warmup {args.warmup} steps done ({n_sets} buffer sets)", file=sys.stderr,
          flush=True)

    # whole-step timing
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record()
    for i in range(args.steps):
        step(i)
    end.record()
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t_wall
    ms_per_step = start.elapsed_time(end) / args.steps
    print(f"[bench] {args.steps} steps: {ms_per_step:.3f} ms/step", file=sys.stderr, flush=True)

    # per-kernel timing: each op alone, cycling over the buffer sets
    per, per_mean = {}, {}
    for name in ops:
        per[name], per_mean[name] = time_calls(torch, [o[name] for o in sets_o])
    ab = algorithmic_bytes()
    kernels = {}
    for name in ops:
        if name in ab:
            kernels[name] = bytes_entry(per[name], per_mean[name], ab[name])
        elif name == "dgrad":
            kernels[name] = gemm_entry(per[name], per_mean[name], GEMM_FLOP, PEAK_FP8_TFLOPS,
                                       "fp8")
        else:
            kernels[name] = gemm_entry(per[name], per_mean[name], GEMM_FLOP, PEAK_FP4_TFLOPS,
                                       "fp4", PEAK_FP16_TFLOPS)
    print(f"[bench] per-kernel: {json.dumps(kernels)}", file=sys.stderr, flush=True)

    # The streaming ceiling on this GPU: a plain 512 MiB device copy (read +
    # write), against which the bytes each quantize op moves are set.
    src = torch.ones(COPY_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    c_med, c_mean = time_calls(torch, [lambda: dst.copy_(src)], n=20, warm=3)
    copy_gbps = 2 * COPY_BYTES / (c_med * 1e-3) / 1e9
    del src, dst
    moved = two_pass_bytes()
    vs_copy = {"copy_GBps": round(copy_gbps, 1)}
    for name, b in moved.items():
        gbps = b / (per[name] * 1e-3) / 1e9
        vs_copy[name] = {"moved_bytes": b, "moved_GBps": round(gbps, 1),
                         "frac_of_copy": round(gbps / copy_gbps, 4)}
    print(f"[bench] quantize ops against a device copy: {json.dumps(vs_copy)}", file=sys.stderr,
          flush=True)

    # Outputs of one more step on set 0, kept on the host for the oracle
    # parity check at the end (whole quantized copies; sampled GEMM outputs).
    captured = None
    if want_oracle:
        step(0)
        torch.cuda.synchronize()
        captured = capture_outputs(torch, sets_b[0])

    # Activation copy of X with a per-token outer scale and Four Over Six
    # (the first NEXT row; not part of the step) and the fprop GEMM over it.
    xa = [T.empty(M, K, device=dev, sdec_per_row=True) for _ in sets_b]
    act = {}
    t_med, t_mean = time_calls(torch, [
        (lambda b=b, a=a: bbs.nvfp4_quantize(b["x"], a, row_per_token=True, row_four_six=True))
        for b, a in zip(sets_b, xa)])
    act["quant_x_act"] = bytes_entry(t_med, t_mean, 2 * M * K + nvfp4_bytes(M, K) + 4 * M)
    t_med, t_mean = time_calls(torch, [
        (lambda b=b, a=a: bbs.nvfp4_gemm(bbs.FMT_NVFP4, a, b["wq"], b["y"], bbs.OUT_BF16))
        for b, a in zip(sets_b, xa)])
    act["fprop_act"] = gemm_entry(t_med, t_mean, GEMM_FLOP, PEAK_FP4_TFLOPS, "fp4",
                                  PEAK_FP16_TFLOPS)
    del xa
    print(f"[bench] per-token + 4/6 activation path: {json.dumps(act)}", file=sys.stderr, flush=True)

    # The activation quantize with both copies stochastic (4096 x 4096
    # Student-t(3), row and column NVFP4 SR, no RHT), amax pass included,
    # over ROTATE input buffers: 33.55 MB read + 18.87 MB written.
    d2 = synth.activation_sr()
    x2 = [up(d2["x"])]
    for _ in range(ROTATE - 1):
        x2.append(x2[0].clone())
    R2 = d2["x"].shape[0]
    o2 = [(T.empty(R2, R2, device=dev), T.empty(R2, R2, device=dev)) for _ in range(ROTATE)]
    t_med, t_mean = time_calls(torch, [
        (lambda xi=xi, o=o: bbs.nvfp4_quantize(xi, o[0], o[1], row_round=bbs.SR,
                                               row_rng=(d2["seed"], d2["row_stream"]),
                                               col_round=bbs.SR,
                                               col_rng=(d2["seed"], d2["col_stream"]),
                                               amax_ws=ws))
        for xi, o in zip(x2, o2)])
    act_sr = bytes_entry(t_med, t_mean, 2 * R2 * R2 + 2 * nvfp4_bytes(R2, R2))
    del x2, o2
    print(f"[bench] activation SR row + col 4096x4096: {json.dumps(act_sr)}", file=sys.stderr,
          flush=True)

    # Fused GELU + quantize of the MLP hidden tensor H [M x N] (between the
    # layer's two projections): the NVFP4 copy of GELU(H) alone, with its
    # MXFP8 SR copy for the backward pass, and as the per-token + 4/6
    # activation copy.  Each op is the amax pass plus the encode pass.
    hs = [up(synth.mlp_hidden(M, N)["h"])]
    for _ in range(ROTATE - 1):
        hs.append(hs[0].clone())
    hq = [T.empty(M, N, device=dev) for _ in hs]
    hm = [bbs.MXFP8Tensor.empty(M, N, device=dev) for _ in hs]
    ha = [T.empty(M, N, device=dev, sdec_per_row=True) for _ in hs]
    mx_rng = (synth.MLP_SEEDS["mx8"], 0)
    gelu_ops = {
        "gelu_quant_row": (
            [(lambda i=i: bbs.nvfp4_quantize(hs[i], hq[i], gelu=True, amax_ws=ws))
             for i in range(ROTATE)],
            2 * M * N + nvfp4_bytes(M, N)),
        "gelu_quant_row_mx8": (
            [(lambda i=i: bbs.nvfp4_quantize(hs[i], hq[i], None, hm[i], mx8_round=bbs.SR,
                                             mx8_rng=mx_rng, gelu=True, amax_ws=ws))
             for i in range(ROTATE)],
            2 * M * N + nvfp4_bytes(M, N) + M * N + M * N // 32),
        "gelu_quant_act": (
            [(lambda i=i: bbs.nvfp4_quantize(hs[i], ha[i], row_per_token=True,
                                             row_four_six=True, gelu=True, amax_ws=ws))
             for i in range(ROTATE)],
            2 * M * N + nvfp4_bytes(M, N) + 4 * M),
    }
    gelu = {}
    for name, (fs, b) in gelu_ops.items():
        t_med, t_mean = time_calls(torch, fs)
        gelu[name] = bytes_entry(t_med, t_mean, b)
        gelu[name]["Gelem/s"] = round(M * N / (t_med * 1e-3) / 1e9, 1)
    del hs, hq, hm, ha
    # The forward GEMM with the quantize (and GELU) in its epilogue, against
    # the same output through BF16 and a separate quantize pass.  The encode
    # scale is 2688 / the output's amax, taken from a first call.
    yq = [T.empty(M, N, device=dev) for _ in sets_b]
    amax_y = torch.zeros(1, dtype=torch.float32, device=dev)
    s_y = torch.ones(1, dtype=torch.float32, device=dev)
    epi = {}
    for g in (False, True):
        bbs.nvfp4_gemm_quant(sets_b[0]["xq"], sets_b[0]["wq"], s_y, yq[0], gelu=g, amax=amax_y)
        torch.cuda.synchronize()
        s_y.fill_(2688.0 / max(float(amax_y[0]), 1e-30))
        name = "fprop_gelu_quant" if g else "fprop_quant"
        t_med, t_mean = time_calls(torch, [
            (lambda b=b, o=o, g=g: bbs.nvfp4_gemm_quant(b["xq"], b["wq"], s_y, o, gelu=g,
                                                        amax=amax_y))
            for b, o in zip(sets_b, yq)])
        epi[name] = gemm_entry(t_med, t_mean, GEMM_FLOP, PEAK_FP4_TFLOPS, "fp4", PEAK_FP16_TFLOPS)
    q_med, _ = time_calls(torch, [(lambda b=b, o=o: bbs.nvfp4_quantize(b["y"], o, amax_ws=ws))
                                  for b, o in zip(sets_b, yq)])
    epi["unfused_fprop_bf16_then_quant"] = {"ms": round(per["fprop"] + q_med, 4)}
    epi["unfused_fprop_bf16_then_gelu_quant"] = {
        "ms": round(per["fprop"] + gelu["gelu_quant_row"]["ms"], 4)}
    del yq
    print(f"[bench] fused GELU + quantize of H {M}x{N}: {json.dumps(gelu)}", file=sys.stderr,
          flush=True)
    print(f"[bench] quantize in the GEMM epilogue: {json.dumps(epi)}", file=sys.stderr, flush=True)

    # The layer as a user calls it: the autograd function over the C ABI,
    # forward alone and forward + backward (allocations and dispatch
    # included), one layer (own weight) per buffer set.
    from bit_block_scaled_amd.layer import QLinear
    layers = []
    for b in sets_b:
        lay = QLinear(K, N, seed=seeds["x_col"], rht_signs=signs, device=dev)
        with torch.no_grad():
            lay.weight.copy_(b["w"].view(torch.bfloat16))
        xin = b["x"].view(torch.bfloat16).detach().requires_grad_(True)
        layers.append((lay, xin, b["dy"].view(torch.bfloat16)))

    def layer_fwd(i):
        lay, xin, _ = layers[i]
        lay(xin)

    def layer_fwd_bwd(i):
        lay, xin, gin = layers[i]
        lay(xin).backward(gin)
        xin.grad = None
        lay.weight.grad = None

    layer_t = {}
    for name, f in (("forward", layer_fwd), ("forward_backward", layer_fwd_bwd)):
        t_med, t_mean = time_calls(torch, [(lambda i=i: f(i)) for i in range(len(layers))])
        flop = GEMM_FLOP * (1 if name == "forward" else 3)
        layer_t[name] = {"ms": round(t_med, 4), "ms_mean": round(t_mean, 4),
                         "TFLOP/s": round(flop / (t_med * 1e-3) / 1e12, 1)}
    del layers
    print(f"[bench] QLinear layer (autograd): {json.dumps(layer_t)}", file=sys.stderr, flush=True)

    # The MXFP4 comparison format: X and W as MXFP4 (E2M1, E8M0 per 32; RTN)
    # and the same forward GEMM on the block-scaled MFMA with E2M1 operands.
    x4 = [bbs.MXFP4Tensor.empty(M, K, device=dev) for _ in sets_b]
    w4 = [bbs.MXFP4Tensor.empty(N, K, device=dev) for _ in sets_b]
    mx4 = {}
    t_med, t_mean = time_calls(torch, [(lambda b=b, o=o: bbs.mxfp4_quantize(b["x"], o))
                                       for b, o in zip(sets_b, x4)])
    mx4["mxfp4_quant_x"] = bytes_entry(t_med, t_mean, 2 * M * K + M * K // 2 + M * K // 32)
    t_med, t_mean = time_calls(torch, [(lambda b=b, o=o: bbs.mxfp4_quantize(b["w"], o))
                                       for b, o in zip(sets_b, w4)])
    mx4["mxfp4_quant_w"] = bytes_entry(t_med, t_mean, 2 * N * K + N * K // 2 + N * K // 32)
    t_med, t_mean = time_calls(torch, [
        (lambda b=b, a=a, c=c: bbs.nvfp4_gemm(bbs.FMT_MXFP4, a, c, b["y"], bbs.OUT_BF16))
        for b, a, c in zip(sets_b, x4, w4)])
    mx4["mxfp4_fprop"] = gemm_entry(t_med, t_mean, GEMM_FLOP, PEAK_FP4_TFLOPS, "fp4")
    del x4, w4
    print(f"[bench] MXFP4 forward: {json.dumps(mx4)}", file=sys.stderr, flush=True)

    fprop_tf = GEMM_FLOP / (per["fprop"] * 1e-3) / 1e12
    fprop_tf_avg = GEMM_FLOP / (per_mean["fprop"] * 1e-3) / 1e12
    qbytes = ab["quant_x"] + ab["quant_w"]
    q_gbps = qbytes / ((per["quant_x"] + per["quant_w"]) * 1e-3) / 1e9
    q_all = sum(ab.values()) / (sum(per[k] for k in ab) * 1e-3) / 1e9
    value = 3 * GEMM_FLOP / (ms_per_step * 1e-3) / 1e12
    out = {
        "metric": "NVFP4 quantize GB/s + NVFP4 GEMM TFLOPS (8192x4096x14336), % of roofline",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4/mxfp8 operands, fp16+fp8 MFMA, fp32 accumulate",
        "data": "synthetic (seeded)",
        "config": {"workload": "dense NVFP4 linear fwd+bwd, X 8192x4096, W 14336x4096, "
                               "dY 8192x14336", "M": M, "K": K, "N": N,
                   "step_gemm_flop": 3 * GEMM_FLOP},
        "quantize_GBps": round(q_gbps, 1),
        "quantize_GBps_all_passes": round(q_all, 1),
        "quantize_vs_copy": vs_copy,
        "gemm_TFLOPs": round(fprop_tf, 1),
        "kernels": kernels,
        "roofline": {"bound": "mfma", "achieved": round(fprop_tf_avg, 1),
                     "peak": PEAK_FP4_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(fprop_tf_avg / PEAK_FP4_TFLOPS, 4),
                     "traffic": fprop_traffic(), "traffic_unit": "bytes per launch",
                     "kernel": "nvfp4_gemm_big_kernel<true> (fprop, 8192x14336x4096, BF16 out)",
                     "peak_dtype": "fp4 (the operands' own format)",
                     "issued_mfma": "v_mfma_f32_32x32x16_f16",
                     "peak_issued_class": PEAK_FP16_TFLOPS,
                     "frac_issued_class": round(fprop_tf_avg / PEAK_FP16_TFLOPS, 4)},
        "activation_per_token_4over6": act,
        "activation_sr_row_col_4096x4096": act_sr,
        "gelu_quantize_mlp_hidden_8192x14336": gelu,
        "gemm_epilogue_quantize_8192x14336x4096": epi,
        "mxfp4_forward_8192x14336x4096": mx4,
        "qlinear_layer_autograd": layer_t,
        "wall_s_timed": round(wall_s, 3),
    }
    if not args.no_moe:
        del x0, w0, dy0, sets_b, sets_o, ops
        torch.cuda.empty_cache()
        print("[bench] MoE grouped GEMMs (65536 tokens, 64 experts, top-8)", file=sys.stderr,
              flush=True)
        out["moe"] = moe_bench(torch, bbs, dev, 100)
        print(f"[bench] moe: {json.dumps(out['moe'])}", file=sys.stderr, flush=True)
    if want_oracle:
        print("[bench] parity of the timed kernels' outputs against the oracle", file=sys.stderr,
              flush=True)
        out["parity"], full_quant = parity(captured, host_in, signs, seeds)
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(full_quant)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
