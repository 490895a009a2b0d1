"""Benchmark of the AWQ W4A16 hot path on one MI355X.

One step is one pass of the whole path over one batch of synthetic input:

  producer  for layer L = step % layers of a Llama-3-8B-shaped stack:
            awq_calib_stats on the layer's 4 distinct inputs (512 calibration
            tokens each), awq_search_scale (20-point alpha grid, g = 128) and
            awq_pack_int4 for its 7 linears, written back into the stack;
  decode    the whole 32-layer stack (7 linears per layer: q, k and v in one
            awq_linear_w4a16_group call; o; gate and up in one group call;
            down; 128 calls, replayed as one HIP graph each) at M = 1, 8, 32
            and 128 tokens with g = 128, and at M = 1 and 32 with g = 64;
  shared s  the same stack at M = 1 with one s for q/k/v and one for gate/up
            (searched on their weights stacked along N), each packed and run
            as one linear on activations that already carry 1/s, and down's
            s folded into the rows of up (down also runs without 1/s);
  prefill   the 7 linears of layer L at M = 2048 tokens (GEMM), grouped as
            in the decode (4 calls, each one activation-prep launch and one
            GEMM launch over the tiles of its linears);
  bf16      the M = 1 decode of the stack and the layer's M = 2048 prefill
            with bf16 activations and outputs (awq_linear_w4a16_group_bf16);
  mixed     the mixed-precision baseline (1 % of channels by mean |x| kept in
            fp16, the rest RTN): the M = 1 decode of the stack with
            awq_linear_mixed (224 calls as one graph); untimed, its output-
            error loss beside the RTN and searched losses of layer 0's 7
            linears over the 512 calibration tokens (the ablation);
  3/8-bit   the stack searched at 3 and at 8 bits (per-linear alpha, 128
            calibration tokens) and packed in those layouts: all 224 linears
            at M = 1 (one awq_linear_wbit call each, replayed as one HIP
            graph) and the 7 linears of layer L at M = 2048;
  70B rows  the four Llama-3-70B-shaped linears (8192<-8192, 1024<-8192,
            28672<-8192, 8192<-28672) at M = 1 and 16, each call on its own
            copy of the packed weights (>= 512 MB of copies per shape), so
            every call streams its weights from HBM.

Inputs are resident in HBM before the timed region.  The reported value is
the M = 1 decode: algorithmic bytes of the 224 linears (packed nibbles +
fp16 scales + packed zeros + activations in/out) divided by the time of the
graph replays (128 decode-GEMV launches per stack), measured with HIP events on the stream the kernels run
on.  The stack is 3.6 GB, far beyond the 256 MB Infinity Cache, so every
weight byte comes from HBM.

    python bench.py [--steps K] [--warmup W] [--layers 32] [--no-cpu] [--no-sclk]
    python bench.py --copy-calibration      (counter calibration only)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
F16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA
METRIC = "W4A16 GEMV achieved HBM GB/s (% of peak) at M=1; GEMM TFLOP/s at M=2048"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def gemv_bytes(m, n, k, g, inv=True):
    """Algorithmic bytes of one W4A16 linear call: packed weights, fp16 scales,
    packed zero points, the fp16 activation and inv_s (when given) read once,
    the fp16 output written once."""
    return (n * k // 2 + 2 * n * (k // g) + 4 * n * (-(-k // (8 * g))) + 2 * m * k + (2 * k if inv else 0)
            + 2 * m * n)


def wbit_bytes(m, n, k, g, w_bit):
    """gemv_bytes for the 3- and 8-bit layouts (codes, fp16 scales, zero-point
    words, activation, inv_s and output)."""
    zpw = 4 if w_bit == 8 else 8
    return (n * k * w_bit // 8 + 2 * n * (k // g) + 4 * n * (-(-(k // g) // zpw)) + 2 * m * k + 2 * k
            + 2 * m * n)


# Child process that samples the shader (GFX) clock of the GPU whose PCI bus
# id it is given, through amdsmi's gpu_metrics, every ~2 ms for argv[2]
# seconds after printing "ready"; it prints one JSON line with two series in
# MHz: the current clock (mean over the XCDs that report one) and the
# firmware's activity-averaged clock.
_SCLK_SAMPLER = r"""
import json, sys, time
import amdsmi
want, dur = sys.argv[1].lower(), float(sys.argv[2])
amdsmi.amdsmi_init()
handle = None
for h in amdsmi.amdsmi_get_processor_handles():
    bdf = str(amdsmi.amdsmi_get_gpu_device_bdf(h)).lower()
    if bdf.endswith(want) or want.endswith(bdf):
        handle = h
print("ready" if handle is not None else "nomatch", flush=True)
out = {"current_gfxclks": [], "average_gfxclk_frequency": []}
t_end = time.time() + dur
while handle is not None and time.time() < t_end:
    m = amdsmi.amdsmi_get_gpu_metrics_info(handle)
    for key in out:
        v = m.get(key)
        vals = [float(x) for x in (v if isinstance(v, (list, tuple)) else [v])
                if isinstance(x, (int, float)) and 0 < x < 10000]
        if vals:
            out[key].append(sum(vals) / len(vals))
    time.sleep(0.002)
amdsmi.amdsmi_shut_down()
print(json.dumps(out), flush=True)
"""


def sample_sclk(work, seconds=0.6):
    """Mean shader clock (MHz) while `work()` runs back to back on the GPU for
    about `seconds`, sampled by a child process; None where the clock cannot
    be read (no amdsmi, the device not found, a timeout)."""
    import select
    import subprocess
    import torch
    try:
        props = torch.cuda.get_device_properties(0)
        bdf = "%02x:%02x.0" % (int(props.pci_bus_id), int(props.pci_device_id))
    except Exception:
        return None
    try:
        child = subprocess.Popen([sys.executable, "-c", _SCLK_SAMPLER, bdf, str(seconds)],
                                 stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True)
    except Exception:
        return None
    try:
        ready, _, _ = select.select([child.stdout], [], [], 30.0)
        if not ready or child.stdout.readline().strip() != "ready":
            child.kill()
            child.wait(timeout=10)
            return None
        t_end = time.perf_counter() + seconds
        while time.perf_counter() < t_end:
            work()
            torch.cuda.synchronize()
        out, _ = child.communicate(timeout=30)
        series = json.loads(out.strip().splitlines()[-1])
    except Exception:
        child.kill()
        child.wait(timeout=10)
        return None
    res = {key: {"mean": round(sum(v) / len(v), 1), "min": round(min(v), 1), "max": round(max(v), 1),
                 "samples": len(v)}
           for key, v in series.items() if v}
    return res or None


def measured_traffic(root):
    """HBM bytes per decode-GEMV launch from the committed counter summary, if it
    was taken on the current kernel source (else None)."""
    import hashlib
    import pathlib
    import re
    root = pathlib.Path(root)
    md = root / "profiles" / "gemv_w4a16_m1_g128_llama3_8b_stack.md"
    src = root / "weight_only_int4_awq_amd" / "csrc" / "linear.hip"
    try:
        text = md.read_text()
        sha = hashlib.sha256(src.read_bytes()).hexdigest()[:16]
    except OSError:
        return None
    m_t = re.search(r"^traffic_bytes_per_launch:\s*(\d+)", text, flags=re.M)
    m_s = re.search(r"^source_sha256_prefix:\s*([0-9a-f]+)", text, flags=re.M)
    if not m_t or not m_s or m_s.group(1) != sha:
        return None
    return int(m_t.group(1))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-sclk", action="store_true", help="skip the shader-clock sampling")
    ap.add_argument("--cpu-seconds", type=float, default=30.0,
                    help="time of the M=1 oracle leg (one thread plus all cores); the other legs are fixed samples")
    ap.add_argument("--cpu-only", action="store_true", help="only the CPU oracle baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run 10 plain device-to-device copies of 256 MiB (the reference "
                         "for scaling the FETCH_SIZE / WRITE_SIZE counters to bytes) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    cpu = None
    if not args.no_cpu:
        t_cpu = time.time()
        cpu = cpu_baseline(args.cpu_seconds)
        log(f"CPU oracle baseline in {time.time() - t_cpu:.1f}s")
    if args.cpu_only:
        print(json.dumps({"cpu_baseline": cpu}), flush=True)
        return

    import torch
    import synthetic as S
    import weight_only_int4_awq_amd as P

    P.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    L = args.layers
    shapes = S.LLAMA3_8B_LINEARS
    inputs = ("attn_in", "o", "mlp_in", "down_in")
    kin = {"attn_in": 4096, "o": 4096, "mlp_in": 4096, "down_in": 14336}
    m_cal = 512
    n_grid = 20

    # ------------------------------------------------------------ set-up (untimed)
    t_setup = time.time()
    W = []      # [layer][linear] fp16 weights
    XC = []     # [layer][input] fp16 calibration tokens
    for layer in range(L):
        W.append([S.torch_weights(n, k, 0.02, S.seed_of(5, layer, S.SLOTS[nm], 0), dev)
                  for nm, n, k in shapes])
        xc = {}
        for inp in inputs:
            slot = S.SLOTS.get(inp, S.SLOTS.get("o"))
            ch = S.outlier_channels(kin[inp], 0.01, S.seed_of(5, layer, slot, 3))
            xc[inp] = S.torch_activations(m_cal, kin[inp], S.seed_of(5, layer, slot, 1), ch, 20.0, dev)
        XC.append(xc)
    log(f"generated {L} layers of weights in {time.time() - t_setup:.1f}s")

    def produce(layer, g, dst, m_tokens, ws):
        """calib -> search -> pack for one layer; packed tensors written into dst[layer]."""
        stats = {inp: P.awq_calib_stats(XC[layer][inp][:m_tokens].contiguous() if m_tokens < m_cal
                                        else XC[layer][inp]) for inp in inputs}
        for li, (nm, n, k) in enumerate(shapes):
            inp = S.INPUT_OF[nm]
            x = XC[layer][inp] if m_tokens == m_cal else XC[layer][inp][:m_tokens].contiguous()
            so = dst[layer][li + len(shapes)]          # persistent (best, s16, inv_s16, losses)
            P.awq_search_scale(W[layer][li], x, stats[inp], g=g, n_grid=n_grid,
                               workspace=ws[li], out=so)
            qw, sc, qz, bad = dst[layer][li]
            P.awq_pack_int4(W[layer][li], so[1], g=g, out=(qw, sc, qz, bad))

    def alloc_stack(g):
        st = []
        for layer in range(L):
            row = []
            for nm, n, k in shapes:
                row.append((torch.empty((n, k // 8), dtype=torch.int32, device=dev),
                            torch.empty((n, k // g), dtype=torch.float16, device=dev),
                            torch.empty((n, -(-k // (8 * g))), dtype=torch.int32, device=dev),
                            torch.empty(1, dtype=torch.int32, device=dev)))
            for nm, n, k in shapes:
                row.append((torch.empty(1, dtype=torch.int32, device=dev),
                            torch.empty(k, dtype=torch.float16, device=dev),
                            torch.empty(k, dtype=torch.float16, device=dev),
                            torch.empty(n_grid, dtype=torch.float64, device=dev)))
            st.append(row)
        return st

    def alloc_ws(g, m_tokens):
        return [torch.empty(P.awq_search_workspace_size(n, k, m_tokens, g, n_grid), dtype=torch.uint8,
                            device=dev) for nm, n, k in shapes]

    stacks = {128: alloc_stack(128), 64: alloc_stack(64)}
    ws_setup = {g: alloc_ws(g, 128) for g in (128, 64)}
    ws_step = alloc_ws(128, m_cal)
    t0 = time.time()
    for g in (128, 64):
        for layer in range(L):
            produce(layer, g, stacks[g], 128, ws_setup[g])   # whole-stack search over 128 tokens
    torch.cuda.synchronize()
    log(f"searched + packed the {L}-layer stack at g=128 and g=64 in {time.time() - t0:.1f}s")

    # decode inputs: one token batch per distinct input per layer
    XR = {}
    for m in (1, 8, 32, 128):
        XR[m] = []
        for layer in range(L):
            d = {}
            for inp in inputs:
                slot = S.SLOTS.get(inp, S.SLOTS.get("o"))
                ch = S.outlier_channels(kin[inp], 0.01, S.seed_of(5, layer, slot, 3))
                d[inp] = S.torch_activations(m, kin[inp], S.seed_of(5, layer, slot, 2) + 7 * m, ch, 20.0, dev)
            XR[m].append(d)
    YR = {m: [[torch.empty((m, n), dtype=torch.float16, device=dev) for nm, n, k in shapes]
              for _ in range(L)] for m in (1, 8, 32, 128)}

    # a decode step: the linears that read the same input (q, k, v; gate,
    # up) are independent and run as one group call; o and down alone
    groups = []
    for li, (nm, n, k) in enumerate(shapes):
        if groups and S.INPUT_OF[shapes[groups[-1][0]][0]] == S.INPUT_OF[nm] and nm not in ("o", "down"):
            groups[-1].append(li)
        else:
            groups.append([li])

    def decode(g, m):
        st = stacks[g]
        for layer in range(L):
            for grp in groups:
                items = []
                for li in grp:
                    nm = shapes[li][0]
                    qw, sc, qz, _ = st[layer][li]
                    items.append((XR[m][layer][S.INPUT_OF[nm]], qw, sc, qz,
                                  st[layer][li + len(shapes)][2], YR[m][layer][li]))
                P.awq_linear_w4a16_group(items, g=g)

    # the stack with one shared s for q/k/v and one for gate/up (searched on
    # their weights stacked along N, 128 calibration tokens), packed as one
    # linear each and run on activations that already carry 1/s (folded into
    # the producing operation's weight): inv_s16 absent for those two.  The
    # down projection's s is searched first and folded into the rows of the up
    # projection (awq_fold_inv_scale_rows) before the gate/up search, so down
    # runs without inv_s16 too; o keeps its inv_s16 (v's outputs feed several
    # of o's input channels under grouped-query attention)
    def shared_search(wst, xc):
        ws = torch.empty(P.awq_search_workspace_size(wst.shape[0], wst.shape[1], 128, 128, n_grid),
                         dtype=torch.uint8, device=dev)
        return P.awq_search_scale(wst, xc, P.awq_calib_stats(xc), g=128, n_grid=n_grid, workspace=ws)[1]

    li_o = [li for li, (nm, n, k) in enumerate(shapes) if nm == "o"][0]
    li_d = [li for li, (nm, n, k) in enumerate(shapes) if nm == "down"][0]
    li_u = [li for li, (nm, n, k) in enumerate(shapes) if nm == "up"][0]
    fused = []
    for layer in range(L):
        xd = XC[layer][S.INPUT_OF["down"]][:128].contiguous()
        s16d = shared_search(W[layer][li_d], xd)
        w_up_f = P.awq_fold_inv_scale_rows(W[layer][li_u], s16d)
        row = []
        for grp_names in (("q", "k", "v"), ("gate", "up")):
            wst = torch.cat([w_up_f if li == li_u else W[layer][li]
                             for li, (nm, n, k) in enumerate(shapes) if nm in grp_names], 0)
            inp = S.INPUT_OF[grp_names[0]]
            s16f = shared_search(wst, XC[layer][inp][:128].contiguous())
            qwf, scf, qzf, _ = P.awq_pack_int4(wst, s16f, g=128)
            row.append((inp, qwf, scf, qzf))
            del wst
        qwd, scd, qzd, _ = P.awq_pack_int4(W[layer][li_d], s16d, g=128)
        row.append((S.INPUT_OF["down"], qwd, scd, qzd))
        fused.append(row)
        del w_up_f
    torch.cuda.synchronize()
    YF = [[torch.empty((1, 6144), dtype=torch.float16, device=dev),
           torch.empty((1, 28672), dtype=torch.float16, device=dev),
           YR[1][layer][li_d]] for layer in range(L)]

    def decode_fused():
        st = stacks[128]
        for layer in range(L):
            for fi, (inp, qwf, scf, qzf) in enumerate(fused[layer]):
                P.awq_linear_w4a16(XR[1][layer][inp], qwf, scf, qzf, None, g=128, out=YF[layer][fi])
                if fi == 0:
                    qw, sc, qz, _ = st[layer][li_o]
                    P.awq_linear_w4a16(XR[1][layer][S.INPUT_OF["o"]], qw, sc, qz,
                                       st[layer][li_o + len(shapes)][2], g=128, out=YR[1][layer][li_o])

    decode_cases = [(128, 1), (128, 8), (128, 32), (128, 128), (64, 1), (64, 32)]
    for g, m in decode_cases:        # eager runs first (the binding sizes each call's workspace)
        decode(g, m)
    torch.cuda.synchronize()
    decode_fused()
    torch.cuda.synchronize()
    graphs = {}
    for g, m in decode_cases:
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            decode(g, m)
        graphs[(g, m)] = gr
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        decode_fused()
    graphs["fused"] = gr
    torch.cuda.synchronize()
    log("captured the decode graphs")

    # prefill inputs
    XP = {}
    for inp in inputs:
        slot = S.SLOTS.get(inp, S.SLOTS.get("o"))
        ch = S.outlier_channels(kin[inp], 0.01, S.seed_of(3, 0, slot, 3))
        XP[inp] = S.torch_activations(2048, kin[inp], S.seed_of(3, 0, slot, 2), ch, 20.0, dev)
    YP = [torch.empty((2048, n), dtype=torch.float16, device=dev) for nm, n, k in shapes]

    def prefill(layer):
        st = stacks[128]
        for grp in groups:
            items = []
            for li in grp:
                nm = shapes[li][0]
                qw, sc, qz, _ = st[layer][li]
                items.append((XP[S.INPUT_OF[nm]], qw, sc, qz, st[layer][li + len(shapes)][2], YP[li]))
            P.awq_linear_w4a16_group(items, g=128)

    # Llama-3-70B-shaped single linears at M = 1 and 16, searched and packed
    # like the stack (128 calibration tokens); timed cold: every call reads its
    # own copy of the packed weights, the copies of one shape >= 512 MB, all
    # calls of one (shape, M) replayed as one HIP graph
    big = []
    for nm, n, k in S.LLAMA3_70B_LINEARS:
        slot = S.SLOTS[nm]
        ch = S.outlier_channels(k, 0.005, S.seed_of(4, 0, slot, 3))
        w = S.torch_weights(n, k, 0.015, S.seed_of(4, 0, slot, 0), dev)
        xc = S.torch_activations(128, k, S.seed_of(4, 0, slot, 1), ch, 30.0, dev)
        ws = torch.empty(P.awq_search_workspace_size(n, k, 128, 128, n_grid), dtype=torch.uint8, device=dev)
        _, s16, inv, _ = P.awq_search_scale(w, xc, P.awq_calib_stats(xc), g=128, n_grid=n_grid, workspace=ws)
        qw, sc, qz, _ = P.awq_pack_int4(w, s16, g=128)
        del w, ws
        copies = max(2, -(-(512 << 20) // (n * k // 2)))
        packs = [(qw, sc, qz)] + [(qw.clone(), sc.clone(), qz.clone()) for _ in range(copies - 1)]
        xr = {m: S.torch_activations(m, k, S.seed_of(4, 0, slot, 2) + m, ch, 30.0, dev) for m in (1, 16)}
        yb = {m: torch.empty((m, n), dtype=torch.float16, device=dev) for m in (1, 16)}
        big.append((nm, n, k, packs, inv, xr, yb))
    big_cases = [(bi, m) for bi in range(len(big)) for m in (1, 16)]

    # 3- and 8-bit stacks: searched per linear at that width (128 calibration
    # tokens of the stack's calibration set) and packed in its layout
    wbits = (3, 8)
    wstacks = {}
    for wb in wbits:
        st = []
        for layer in range(L):
            stats = {inp: P.awq_calib_stats(XC[layer][inp][:128].contiguous()) for inp in inputs}
            row = []
            for li, (nm, n, k) in enumerate(shapes):
                inp = S.INPUT_OF[nm]
                _, s16, inv, _ = P.awq_search_scale_wbit(W[layer][li], XC[layer][inp][:128].contiguous(),
                                                         stats[inp], g=128, n_grid=n_grid, w_bit=wb,
                                                         workspace=ws_setup[128][li])
                qw, sc, qz, _ = P.awq_pack_wbit(W[layer][li], s16, g=128, w_bit=wb)
                row.append((qw, sc, qz, inv))
            st.append(row)
        wstacks[wb] = st

    def decode_wbit(wb):
        for layer in range(L):
            for li, (nm, n, k) in enumerate(shapes):
                qw, sc, qz, inv = wstacks[wb][layer][li]
                P.awq_linear_wbit(XR[1][layer][S.INPUT_OF[nm]], qw, sc, qz, inv, g=128, w_bit=wb,
                                  out=YR[1][layer][li])

    def prefill_wbit(wb, layer):
        for li, (nm, n, k) in enumerate(shapes):
            qw, sc, qz, inv = wstacks[wb][layer][li]
            P.awq_linear_wbit(XP[S.INPUT_OF[nm]], qw, sc, qz, inv, g=128, w_bit=wb, out=YP[li])

    # bf16 activations: the same inputs rounded to bf16, bf16 outputs
    XRb = [{inp: XR[1][layer][inp].to(torch.bfloat16) for inp in inputs} for layer in range(L)]
    YRb = [[torch.empty((1, n), dtype=torch.bfloat16, device=dev) for nm, n, k in shapes] for _ in range(L)]
    XPb = {inp: XP[inp].to(torch.bfloat16) for inp in inputs}
    YPb = [torch.empty((2048, n), dtype=torch.bfloat16, device=dev) for nm, n, k in shapes]

    def decode_bf16():
        st = stacks[128]
        for layer in range(L):
            for grp in groups:
                items = []
                for li in grp:
                    nm = shapes[li][0]
                    qw, sc, qz, _ = st[layer][li]
                    items.append((XRb[layer][S.INPUT_OF[nm]], qw, sc, qz, st[layer][li + len(shapes)][2],
                                  YRb[layer][li]))
                P.awq_linear_w4a16_group_bf16(items, g=128)

    def prefill_bf16(layer):
        st = stacks[128]
        for grp in groups:
            items = []
            for li in grp:
                nm = shapes[li][0]
                qw, sc, qz, _ = st[layer][li]
                items.append((XPb[S.INPUT_OF[nm]], qw, sc, qz, st[layer][li + len(shapes)][2], YPb[li]))
            P.awq_linear_w4a16_group_bf16(items, g=128)

    decode_bf16()
    prefill_bf16(0)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        decode_bf16()
    graphs["bf16"] = gr

    # mixed-precision baseline: RTN packs, the 1 % protected channels of each
    # linear (by mean |x| over 128 calibration tokens) and their fp16 columns
    mixed = []
    for layer in range(L):
        stats = {inp: P.awq_calib_stats(XC[layer][inp][:128].contiguous()) for inp in inputs}
        row = []
        for li, (nm, n, k) in enumerate(shapes):
            idx = P.awq_salient_channels(stats[S.INPUT_OF[nm]], int(np.floor(0.01 * k + 0.5)))
            qw, sc, qz, _ = P.awq_pack_int4(W[layer][li], None, g=128)
            row.append((qw, sc, qz, P.awq_channel_mask(idx, k), P.awq_gather_channels(W[layer][li], idx), idx))
        mixed.append(row)

    def decode_mixed():
        for layer in range(L):
            for li, (nm, n, k) in enumerate(shapes):
                qw, sc, qz, keep, ws_, idx = mixed[layer][li]
                P.awq_linear_mixed(XR[1][layer][S.INPUT_OF[nm]], qw, sc, qz, keep, ws_, idx, g=128,
                                   out=YR[1][layer][li])

    decode_mixed()
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        decode_mixed()
    graphs["mixed"] = gr

    # the ablation on layer 0 (512 calibration tokens): plain RTN (alpha = 0),
    # the searched scale and the mixed-precision weight at 1 % and 0.1 %
    ablation = {}
    stats0 = {inp: P.awq_calib_stats(XC[0][inp]) for inp in inputs}
    for li, (nm, n, k) in enumerate(shapes):
        inp = S.INPUT_OF[nm]
        ws_a = torch.empty(P.awq_search_workspace_size(n, k, m_cal, 128, n_grid), dtype=torch.uint8, device=dev)
        best, _, _, losses = P.awq_search_scale(W[0][li], XC[0][inp], stats0[inp], g=128, n_grid=n_grid,
                                                workspace=ws_a)
        lm = {}
        for frac in (0.01, 0.001):
            idx = P.awq_salient_channels(stats0[inp], int(np.floor(frac * k + 0.5)))
            lm[frac] = P.awq_mixed_loss(W[0][li], XC[0][inp], P.awq_channel_mask(idx, k), g=128)
        torch.cuda.synchronize()
        lo = losses.cpu().numpy()
        b = int(best.item())
        ablation[nm] = {"loss_rtn": float(lo[0]), "loss_awq": float(lo[b]), "alpha": b / n_grid,
                        "loss_mixed_1pct": float(lm[0.01].item()), "loss_mixed_0.1pct": float(lm[0.001].item())}
        del ws_a
    log("built the mixed-precision stack and the layer-0 ablation")

    for wb in wbits:                  # eager runs first
        decode_wbit(wb)
        prefill_wbit(wb, 0)
    torch.cuda.synchronize()
    for wb in wbits:
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            decode_wbit(wb)
        graphs[f"w{wb}"] = gr
    torch.cuda.synchronize()
    log("searched, packed and captured the 3- and 8-bit stacks")

    def big_calls(bi, m):
        nm, n, k, packs, inv, xr, yb = big[bi]
        for qw, sc, qz in packs:
            P.awq_linear_w4a16(xr[m], qw, sc, qz, inv, g=128, out=yb[m])

    for bi, m in big_cases:
        big_calls(bi, m)
    torch.cuda.synchronize()
    big_graphs = {}
    for bi, m in big_cases:
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            big_calls(bi, m)
        big_graphs[(bi, m)] = gr
    torch.cuda.synchronize()
    log("packed and captured the 70B-shaped linears")

    phases = (["producer"] + [f"decode_g{g}_m{m}" for g, m in decode_cases] + ["decode_fused"] + ["prefill"] +
              [f"big_{big[bi][0]}_m{m}" for bi, m in big_cases] +
              [f"decode_w{wb}_m1" for wb in wbits] + [f"prefill_w{wb}" for wb in wbits] +
              ["decode_bf16_m1", "prefill_bf16", "decode_mixed_m1"])
    acc = {p: 0.0 for p in phases}

    def step(i, timed):
        layer = i % L
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(phases) + 1)]
        ev[0].record(stream)
        produce(layer, 128, stacks[128], m_cal, ws_step)
        ev[1].record(stream)
        for pi, (g, m) in enumerate(decode_cases):
            graphs[(g, m)].replay()
            ev[2 + pi].record(stream)
        graphs["fused"].replay()
        ev[2 + len(decode_cases)].record(stream)
        prefill(layer)
        ev[3 + len(decode_cases)].record(stream)
        for ci, key in enumerate(big_cases):
            big_graphs[key].replay()
            ev[4 + len(decode_cases) + ci].record(stream)
        e0 = 4 + len(decode_cases) + len(big_cases)
        for wi, wb in enumerate(wbits):
            graphs[f"w{wb}"].replay()
            ev[e0 + wi].record(stream)
        for wi, wb in enumerate(wbits):
            prefill_wbit(wb, layer)
            ev[e0 + len(wbits) + wi].record(stream)
        graphs["bf16"].replay()
        ev[e0 + 2 * len(wbits)].record(stream)
        prefill_bf16(layer)
        ev[e0 + 2 * len(wbits) + 1].record(stream)
        graphs["mixed"].replay()
        ev[e0 + 2 * len(wbits) + 2].record(stream)
        if timed:
            return ev
        return None

    for i in range(args.warmup):
        step(i, False)
        torch.cuda.synchronize()
        log(f"warmup step {i + 1}/{args.warmup} done")

    torch.cuda.synchronize()
    events = []
    t_start = time.perf_counter()
    for i in range(args.steps):
        events.append(step(args.warmup + i, True))
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_start
    for ev in events:
        for pi, p in enumerate(phases):
            acc[p] += ev[pi].elapsed_time(ev[pi + 1]) * 1e-3     # seconds
    log(f"timed {args.steps} steps in {t_total:.3f}s")

    # shader clock under the two headline loads, after the timed region
    sclk = None
    if not args.no_sclk:
        sclk = {"prefill_m2048": sample_sclk(lambda: prefill(0)),
                "decode_g128_m1": sample_sclk(lambda: graphs[(128, 1)].replay()),
                "source": "amdsmi gpu_metrics, sampled every ~2 ms while the load runs back to back "
                          "after the timed region: current_gfxclks (mean over XCDs), and "
                          "average_gfxclk_frequency where the firmware reports it"}
        log(f"shader clock: {sclk['prefill_m2048']} (prefill), {sclk['decode_g128_m1']} (decode)")

    K = args.steps
    nlin = L * len(shapes)
    bytes_by = {}
    for g, m in decode_cases:
        bytes_by[(g, m)] = L * sum(gemv_bytes(m, n, k, g) for nm, n, k in shapes)
    rows = {}
    for g, m in decode_cases:
        t = acc[f"decode_g{g}_m{m}"] / K
        rows[f"decode_g{g}_m{m}"] = {"us_per_stack": t * 1e6, "us_per_linear": t * 1e6 / nlin,
                                     "GBps": bytes_by[(g, m)] / t / 1e9,
                                     "frac_hbm_peak": bytes_by[(g, m)] / t / 1e9 / HBM_PEAK_GBS}
    t_f = acc["decode_fused"] / K
    by_f = L * (gemv_bytes(1, 6144, 4096, 128, inv=False) + gemv_bytes(1, 28672, 4096, 128, inv=False)
                + gemv_bytes(1, 4096, 4096, 128) + gemv_bytes(1, 4096, 14336, 128, inv=False))
    rows["decode_shared_s_g128_m1"] = {"us_per_stack": t_f * 1e6, "GBps": by_f / t_f / 1e9,
                                       "frac_hbm_peak": by_f / t_f / 1e9 / HBM_PEAK_GBS,
                                       "launches_per_stack": 4 * L}
    prefill_flops = sum(2 * 2048 * n * k for nm, n, k in shapes)
    t_pf = acc["prefill"] / K
    rows["prefill_m2048"] = {"us_per_layer": t_pf * 1e6, "TFLOPs": prefill_flops / t_pf / 1e12,
                             "frac_mfma_peak": prefill_flops / t_pf / 1e12 / F16_MFMA_PEAK_TFLOPS}
    search_flops = n_grid * sum(2 * n * k * m_cal for nm, n, k in shapes)
    t_pr = acc["producer"] / K
    rows["producer_m512"] = {"us_per_layer": t_pr * 1e6,
                             "search_TFLOPs_algorithmic": search_flops / t_pr / 1e12}

    for bi, m in big_cases:
        nm, n, k, packs, inv, xr, yb = big[bi]
        t = acc[f"big_{nm}_m{m}"] / K / len(packs)
        by = gemv_bytes(m, n, k, 128)
        rows[f"llama3_70b_{nm}_m{m}"] = {"us_per_call": t * 1e6, "GBps": by / t / 1e9,
                                         "frac_hbm_peak": by / t / 1e9 / HBM_PEAK_GBS,
                                         "n": n, "k": k, "cold_copies": len(packs)}
    for wb in wbits:
        t = acc[f"decode_w{wb}_m1"] / K
        by = L * sum(wbit_bytes(1, n, k, 128, wb) for nm, n, k in shapes)
        rows[f"decode_w{wb}_g128_m1"] = {"us_per_stack": t * 1e6, "us_per_linear": t * 1e6 / nlin,
                                         "GBps": by / t / 1e9, "frac_hbm_peak": by / t / 1e9 / HBM_PEAK_GBS,
                                         "stack_bytes": by}
        t = acc[f"prefill_w{wb}"] / K
        rows[f"prefill_w{wb}_m2048"] = {"us_per_layer": t * 1e6, "TFLOPs": prefill_flops / t / 1e12,
                                        "frac_mfma_peak": prefill_flops / t / 1e12 / F16_MFMA_PEAK_TFLOPS}
    t = acc["decode_bf16_m1"] / K
    rows["decode_bf16_g128_m1"] = {"us_per_stack": t * 1e6, "us_per_linear": t * 1e6 / nlin,
                                   "GBps": bytes_by[(128, 1)] / t / 1e9,
                                   "frac_hbm_peak": bytes_by[(128, 1)] / t / 1e9 / HBM_PEAK_GBS}
    t = acc["prefill_bf16"] / K
    rows["prefill_bf16_m2048"] = {"us_per_layer": t * 1e6, "TFLOPs": prefill_flops / t / 1e12,
                                  "frac_mfma_peak": prefill_flops / t / 1e12 / F16_MFMA_PEAK_TFLOPS}
    t = acc["decode_mixed_m1"] / K
    cnt_of = {k: int(np.floor(0.01 * k + 0.5)) for nm, n, k in shapes}
    # 4-bit bytes (keep16 read as inv_s) + protected fp16 columns and indices +
    # the add pass's read and write of y
    by_mx = L * sum(gemv_bytes(1, n, k, 128) + 2 * n * cnt_of[k] + 4 * cnt_of[k] + 4 * n for nm, n, k in shapes)
    rows["decode_mixed_g128_m1"] = {"us_per_stack": t * 1e6, "us_per_linear": t * 1e6 / nlin,
                                    "GBps": by_mx / t / 1e9, "frac_hbm_peak": by_mx / t / 1e9 / HBM_PEAK_GBS,
                                    "launches_per_stack": 2 * nlin, "protected_frac": 0.01}
    tot = {key: sum(v[key] for v in ablation.values()) for key in ("loss_rtn", "loss_awq", "loss_mixed_1pct",
                                                                  "loss_mixed_0.1pct")}
    rows["ablation_layer0_m512"] = {
        "per_linear": {nm: {key: (round(v, 6) if key == "alpha" else float(f"{v:.6g}")) for key, v in d.items()}
                       for nm, d in ablation.items()},
        "sum": {key: float(f"{v:.6g}") for key, v in tot.items()},
        "awq_over_rtn": round(tot["loss_awq"] / tot["loss_rtn"], 4),
        "mixed_1pct_over_rtn": round(tot["loss_mixed_1pct"] / tot["loss_rtn"], 4),
        "mixed_0.1pct_over_rtn": round(tot["loss_mixed_0.1pct"] / tot["loss_rtn"], 4)}
    # the two 122 MB shapes (28672<-8192, 8192<-28672) at M = 1 together
    bp = [rows[f"llama3_70b_{nm}_m1"] for nm in ("gate_up", "down")]
    bp_bytes = sum(gemv_bytes(1, r["n"], r["k"], 128) for r in bp)
    bp_us = sum(r["us_per_call"] for r in bp)
    big_pair = {"GBps": round(bp_bytes / bp_us / 1e3, 2),
                "frac_hbm_peak": round(bp_bytes / bp_us / 1e3 / HBM_PEAK_GBS, 4),
                "us_per_call": [round(r["us_per_call"], 2) for r in bp]}
    value = rows["decode_g128_m1"]["GBps"]
    t1 = acc["decode_g128_m1"] / K
    n_launch = L * len(groups)               # one decode-GEMV launch per group call at M = 1
    avg_launch = t1 / n_launch
    bytes_per_launch = bytes_by[(128, 1)] / n_launch
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(t_total / K * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) activations with 1% x20 outlier channels)",
        "config": {"workload": "llama3-8b-shaped linear stack: producer (calib 512 tok, 20-pt alpha "
                               "search, int4 g128 pack) on one layer + 32-layer decode at M=1/8/32/128 "
                               "(g128) and M=1/32 (g64) + 7-linear prefill at M=2048 + llama3-70b-"
                               "shaped linears at M=1/16 (cold copies) + the stack at 3 and 8 bits "
                               "(M=1 decode, M=2048 prefill of one layer) + bf16 activations (M=1 "
                               "decode, M=2048 prefill) + the mixed-precision baseline (M=1 decode; "
                               "layer-0 loss ablation, untimed)",
                   "layers": L, "linears_per_layer": len(shapes), "m_decode": [1, 8, 32, 128],
                   "m_prefill": 2048, "m_calib": m_cal, "n_grid": n_grid, "group_size": [128, 64]},
        "gemm_tflops_m2048": round(rows["prefill_m2048"]["TFLOPs"], 2),
        "gemv_70b_big_pair_m1": big_pair,
        "roofline": {"bound": "hbm", "achieved": round(bytes_per_launch / avg_launch / 1e9, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(bytes_per_launch / avg_launch / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(os.path.dirname(os.path.abspath(__file__))),
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                     "kernel": "W4A16 decode GEMV (M=1, g=128)",
                     "bytes_per_launch": bytes_per_launch, "avg_launch_us": avg_launch * 1e6,
                     "launches_per_stack": n_launch},
        "roofline_gemm": {"bound": "mfma", "achieved": round(rows["prefill_m2048"]["TFLOPs"], 2),
                          "peak": F16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                          "frac": round(rows["prefill_m2048"]["frac_mfma_peak"], 4)},
        "rows": rows,
    }
    if sclk is not None:
        out["sclk_mhz"] = sclk
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


def copy_calibration():
    """Ten device-to-device copies of 256 MiB (read 256 MiB, write 256 MiB
    each): a known byte count against which the HBM traffic counters are scaled."""
    import torch
    nbytes = 256 * 1024 * 1024
    a = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(10):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read_per_copy": nbytes,
                                           "bytes_written_per_copy": nbytes, "copies": 10}}),
          flush=True)


# ---------------------------------------------------------------- CPU baseline
# The float64 oracle timed on this host's cores beside the GPU numbers, on
# bounded samples of the same workloads.  Runs before the GPU is touched, so
# the worker processes of the all-cores mode are plain forks.

def _host_info():
    info = {"cores": len(os.sched_getaffinity(0)), "cpu_model": None, "numpy": np.__version__, "blas": None}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        info["blas"] = [{"api": d.get("internal_api"), "threads": d.get("num_threads"),
                         "version": d.get("version")} for d in threadpool_info()]
    except Exception:  # pragma: no cover
        pass
    return info


def _one_thread():
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(1)
    except Exception:  # pragma: no cover
        import contextlib
        return contextlib.nullcontext()


_SHARED = {}          # inputs prepared by the parent, inherited by the forked workers


def _run_workers(fn, args_list):
    """Run fn(args) in one forked single-thread process per args (inputs come
    from _SHARED), all starting together after a barrier.  Returns (results,
    wall seconds from the first start to the last end)."""
    import multiprocessing as mp
    ctx = mp.get_context("fork")
    barrier = ctx.Barrier(len(args_list))
    q = ctx.Queue()

    def body(i, args):
        with _one_thread():
            barrier.wait()
            t0 = time.time()
            res = fn(args)
            q.put((i, res, t0, time.time()))

    procs = [ctx.Process(target=body, args=(i, a)) for i, a in enumerate(args_list)]
    for pr in procs:
        pr.start()
    out = [q.get() for _ in procs]
    for pr in procs:
        pr.join()
    out.sort(key=lambda r: r[0])
    return [r[1] for r in out], max(r[3] for r in out) - min(r[2] for r in out)


def _decode_work(seconds):
    """float64 oracle W4A16 linears at M = 1 over the prepared linears for
    about `seconds`; returns algorithmic bytes."""
    from oracle import awq_oracle as O
    done, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for n, k, qw, sc, qz, x in _SHARED["decode"]:
            O.linear_ref(x, qw, sc, qz, None, k, 128)
            done += gemv_bytes(1, n, k, 128)
            if time.perf_counter() - t0 >= seconds:
                break
    return done


def _search_work(key):
    """The oracle's 20-alpha losses on the prepared rows of each linear (the
    loss is a sum over rows); returns the per-linear loss vectors."""
    from oracle import awq_oracle as O
    out = []
    for w, x_cal in _SHARED[key]:
        a = O.calib_stats(x_cal)
        out.append(np.array([O.search_loss(w, x_cal, O.scale_candidate(a, al), 128) for al in O.alpha_grid(20)]))
    return out


def _gemm_work(key):
    """The oracle's linear reference at M = 2048 on the prepared columns; returns flops."""
    from oracle import awq_oracle as O
    flops = 0
    for x, qw, sc, qz, inv, k in _SHARED[key]:
        O.linear_ref(x, qw, sc, qz, inv, k, 128)
        flops += 2 * x.shape[0] * qw.shape[0] * k
    return flops


def cpu_baseline(budget_s):
    """The float64 oracle (oracle/awq_oracle.py, as it stands) on bounded
    samples of the benchmark's workloads, on one thread and on all cores (one
    single-thread process per core over independent linears or row chunks,
    started together; the search's per-alpha losses summed in fixed chunk
    order).  Set-up (drawing and packing the inputs) is not timed.  `value` is
    the headline leg: the M = 1 W4A16 linear in the metric's unit
    (algorithmic GB/s) on all cores.  Legs marked extrapolated scale a timed
    sample by its share of the full work (the search loss and the products are
    sums over rows and columns, so their cost is linear in them)."""
    import synthetic as S
    from oracle import awq_oracle as O
    info = _host_info()
    cores = info["cores"]
    legs = {}
    per = max(budget_s / 2.0, 1.0)
    L8 = S.LLAMA3_8B_LINEARS

    # decode, M = 1: the 7 Llama-3-8B-shaped linears (packed once here)
    with _one_thread():
        dec = []
        for nm, n, k in L8:
            w = S.weights(n, k, 0.02, S.seed_of(2, 0, S.SLOTS[nm], 0))
            qw, sc, qz, _ = O.pack_int4(w, None, 128)
            del w
            dec.append((n, k, qw, sc, qz, S.activations(1, k, S.seed_of(2, 0, S.SLOTS[nm], 2))))
    _SHARED["decode"] = dec
    (b1,), t1 = _run_workers(_decode_work, [per])
    ball, wall = _run_workers(_decode_work, [per] * cores)
    legs["decode_m1_llama3_8b_linears"] = {
        "unit": "GB/s", "one_thread": round(b1 / t1 / 1e9, 4), "all_cores": round(sum(ball) / wall / 1e9, 4),
        "sample": "float64 oracle W4A16 linears at M=1 (g=128) cycling over the 7 Llama-3-8B-shaped linears "
                  f"for {per:.0f}s, on one thread and in {cores} processes"}
    del _SHARED["decode"], dec

    # the search (20 alpha) and pack of the single 4096 x 4096 linear at 128
    # calibration tokens: the whole layer on all cores (row chunks), every 4th
    # row on one thread (x4); the pack is timed on the whole layer
    n1, k1 = 4096, 4096
    w1, xc1, _, _ = S.config_layer(1, "q", n1, k1, 128, 0, 0.02, 0.01, 20.0)
    for c in range(cores):
        _SHARED[f"s1_{c}"] = [(np.ascontiguousarray(w1[c::cores]), xc1)]
    parts, wall_all = _run_workers(_search_work, [f"s1_{c}" for c in range(cores)])
    losses = np.zeros(20)
    for lp in parts:                        # fixed chunk order
        losses = losses + lp[0]
    best = O.select_best(losses)
    _SHARED["s1_one"] = [(np.ascontiguousarray(w1[::4]), xc1)]
    _, t_one = _run_workers(_search_work, ["s1_one"])
    with _one_thread():
        t0 = time.perf_counter()
        a1 = O.calib_stats(xc1)
        O.pack_int4(w1, O.scale_candidate(a1, O.alpha_grid(20)[best]), 128)
        t_pack = time.perf_counter() - t0
    for key in [kk for kk in _SHARED if kk.startswith("s1_")]:
        del _SHARED[key]
    del w1
    flops1 = 20 * 2 * n1 * k1 * 128
    legs["producer_4096x4096_m128"] = {
        "unit": "s per layer", "one_thread": round(4 * t_one + t_pack, 2), "all_cores": round(wall_all + t_pack, 2),
        "alpha_index": int(best), "extrapolated": "one thread: search on every 4th row, x4",
        "search_TFLOPs_algorithmic_all_cores": round(flops1 / wall_all / 1e12, 5),
        "sample": f"calib stats + 20-alpha search (whole layer in {cores} row chunks on all cores) + pack "
                  "(one thread, whole layer)"}

    # the search of one Llama-3-8B-shaped layer (7 linears, 512 calibration
    # tokens) and of the 32-layer stack (128 tokens per layer): sampled rows
    # of every linear, scaled to all rows (and x32 layers)
    for key, cfg, m_cal, layers in (("search_llama3_8b_layer_m512", 3, 512, 1),
                                    ("search_llama3_8b_32_layers_m128", 5, 128, 32)):
        rows_per = 32
        for c in range(cores):
            _SHARED[f"{key}_{c}"] = [
                (S.weights(rows_per, k, 0.02, S.seed_of(cfg, 0, S.SLOTS[nm], 0) + 7919 * (c + 1)),
                 S.config_layer(cfg, nm, 1, k, m_cal, 0, 0.02, 0.01, 20.0)[1]) for nm, n, k in L8]
        _, wall = _run_workers(_search_work, [f"{key}_{c}" for c in range(cores)])
        _, t_one = _run_workers(_search_work, [f"{key}_0"])
        for c in range(cores):
            del _SHARED[f"{key}_{c}"]
        rows_full = sum(n for _, n, _ in L8)
        share_one = rows_per * len(L8) / rows_full
        share_all = cores * share_one
        flops = layers * 20 * sum(2 * n * k * m_cal for _, n, k in L8)
        legs[key] = {"unit": "s", "one_thread": round(layers * t_one / share_one, 1),
                     "all_cores": round(layers * wall / share_all, 1),
                     "extrapolated": f"{rows_per} rows per linear per process, scaled to all rows"
                                     + (" and 32 layers" if layers > 1 else ""),
                     "search_TFLOPs_algorithmic_all_cores": round(flops / (layers * wall / share_all) / 1e12, 5),
                     "sample": f"20-alpha search losses of the 7 linears ({m_cal} calibration tokens)"}

    # the prefill GEMM reference at M = 2048 on sampled output columns
    cols_per = 4
    x2 = {}
    for c in range(cores):
        items = []
        for nm, n, k in L8:
            if k not in x2:
                _, x_cal, x_run, _ = S.config_layer(3, nm, 1, k, 64, 2048, 0.02, 0.01, 20.0)
                s16 = O.scale_candidate(O.calib_stats(x_cal), 0.35)
                x2[k] = (x_run, O.fp16_rn(1.0 / s16.astype(np.float64)), s16)
            x_run, inv, s16 = x2[k]
            w = S.weights(cols_per, k, 0.02, S.seed_of(3, 0, S.SLOTS[nm], 0) + 7919 * (c + 1))
            qw, sc, qz, _ = O.pack_int4(w, s16, 128)
            items.append((x_run, qw, sc, qz, inv, k))
        _SHARED[f"g_{c}"] = items
    fall, wall = _run_workers(_gemm_work, [f"g_{c}" for c in range(cores)])
    (f1,), t1 = _run_workers(_gemm_work, ["g_0"])
    for c in range(cores):
        del _SHARED[f"g_{c}"]
    legs["prefill_m2048_llama3_8b_layer"] = {
        "unit": "TFLOP/s", "one_thread": round(f1 / t1 / 1e12, 5), "all_cores": round(sum(fall) / wall / 1e12, 5),
        "sample": f"float64 oracle linear reference of the 7 linears at M=2048 on {cols_per} output columns "
                  "each per process"}

    head = legs["decode_m1_llama3_8b_linears"]
    return {"value": head["all_cores"], "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": head["sample"], "one_thread_value": head["one_thread"],
            "host": info, "legs": legs}


if __name__ == "__main__":
    main()
