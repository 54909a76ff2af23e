"""Benchmark of the MoE layer on one MI355X.

A step is one pass of the whole layer -- moe_route -> moe_permute ->
moe_grouped_ffn -> moe_combine, with route and permute as one moe_route_plan
call (a single launch) at T <= 32 -- over one batch of seeded synthetic input,
inputs already resident in HBM.  The headline workload is the T=4096 prefill
(int4 group-32 routed experts, int8 per-row shared expert, bf16 activations,
d=2560, E=512, top-10 + 1 shared, expert width 1024); the T=16 decode/verify
batch of the same layer is measured in the same run and reported beside it.

Prints ONE JSON line.  Per-call times come from HIP events recorded on the
stream the calls are launched on, inside the timed region.  The routed expert
blobs are rotated over several identical copies so no step can be served from
the 256 MB last-level cache left warm by the previous one.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s
FP4_PEAK_TFLOPS = 10100.0    # MI355X dense fp4 (MXFP4) MFMA, TFLOP/s
N_ROT = 4                    # routed-blob copies rotated across steps


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--decode-steps", type=int, default=200)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-tokens", type=int, default=4096)
    p.add_argument("--calib-copy", action="store_true",
                   help="also run one 1 GiB device-to-device copy (reference for HBM byte counters)")
    p.add_argument("--workload", choices=("both", "prefill", "decode", "bits", "mxfp4", "configs"),
                   default="both",
                   help="limit the run to one workload (for per-workload profiles); the default "
                        "runs the T=4096 prefill (headline), the T=16/32 decode and the other "
                        "layer configurations")
    p.add_argument("--no-configs", action="store_true",
                   help="default run without the bf16 T=512, bf16-weight T=4096 and Zipf "
                        "T=16384 layers")
    return p.parse_args()


class Setup:
    """One layer's weights on the GPU (N_ROT copies of the routed blob)."""

    def __init__(self, cfg, T, torch):
        import workloads as W
        from expert_grouped_quantized_amd import make_desc
        from expert_grouped_quantized_amd.layer import MoELayer, blobs_from_inputs
        self.cfg, self.T, self.torch = cfg, T, torch
        t0 = time.time()
        self.inputs = W.generate(cfg, T=T)
        self.desc = make_desc(cfg.d, cfg.E, cfg.F, cfg.n_shared, cfg.Fs, act=cfg.act,
                              expert_w=cfg.expert, shared_w=cfg.shared)
        routed, shared = blobs_from_inputs(self.desc, self.inputs)
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        self.routed = [dev(routed)]
        for _ in range(N_ROT - 1):
            self.routed.append(self.routed[0].clone())
        self.shared = dev(shared) if shared is not None else None
        self.wr = dev(self.inputs["wr"].view(np.int16)).view(torch.bfloat16)
        self.bias = None if self.inputs.get("bias") is None else dev(self.inputs["bias"])
        self.x = dev(self.inputs["x"].view(np.int16)).view(torch.bfloat16)
        self.layer = MoELayer(self.desc, cfg.k, T)
        self.layer.set_weights(self.wr, self.routed[0], self.shared, self.bias)
        self.routed_bytes = routed.nbytes
        print(f"[bench] {cfg.name} T={T}: inputs ready in {time.time() - t0:.1f}s", file=sys.stderr,
              flush=True)

    def step(self, i, ev=None):
        L = self.layer
        L.routed_blob = self.routed[i % N_ROT]
        if ev is not None:
            ev[0].record()
        if self.T <= 32:  # the layer's small-call front end: one launch
            L.route_plan(self.x, self.T)
        else:
            L.route(self.x, self.T)
        if ev is not None:
            ev[1].record()
        if self.T > 32:
            L.permute(self.x, self.T)
        if ev is not None:
            ev[2].record()
        L.grouped_ffn(self.x, self.T)
        if ev is not None:
            ev[3].record()
        L.combine(self.T)
        if ev is not None:
            ev[4].record()


def time_steps(S: Setup, steps: int, warmup: int):
    torch = S.torch
    for i in range(warmup):
        S.step(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        S.step(i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_call = np.zeros(4)
    for e in evs:
        per_call += [e[j].elapsed_time(e[j + 1]) for j in range(4)]
    per_call /= steps
    layer_ms = np.mean([e[0].elapsed_time(e[4]) for e in evs])
    return wall, layer_ms, per_call


def call_ms(per, T):
    """Per-call HIP-event times of one step (route and permute are one
    moe_route_plan call at T <= 32)."""
    if T <= 32:
        return dict(route_plan=per[0] + per[1], grouped_ffn=per[2], combine=per[3])
    return dict(route=per[0], permute=per[1], grouped_ffn=per[2], combine=per[3])


def time_graph(S: Setup, steps: int):
    """The layer's calls captured as one HIP graph per routed-blob copy, replayed
    back to back; wall clock and HIP-event time per replay."""
    torch = S.torch
    graphs = []
    for i in range(N_ROT):
        S.layer.routed_blob = S.routed[i]
        graphs.append(S.layer.capture(S.x, S.T))
    for i in range(2 * N_ROT):
        graphs[i % N_ROT].replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        graphs[i % N_ROT].replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    del graphs
    return wall * 1e3 / steps, e0.elapsed_time(e1) / steps


def measured_peaks(torch):
    """Secondary denominators measured on this GPU: a large bf16 GEMM
    (torch.mm, 8192^3, hipBLASLt) and a 2 GiB device-to-device copy (bytes
    read + written per second)."""
    n = 8192
    a = torch.randn(n, n, dtype=torch.bfloat16, device="cuda")
    b = torch.randn(n, n, dtype=torch.bfloat16, device="cuda")
    for _ in range(3):
        torch.mm(a, b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        torch.mm(a, b)
    e1.record()
    torch.cuda.synchronize()
    tflops = 2.0 * n ** 3 * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del a, b
    src = torch.ones(1 << 31, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2 * src.numel() * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del dst
    # stream read: a bf16 matrix-vector product over the same 2 GiB (the
    # vendor GEMV; the fastest plain read of the torch operations tried --
    # reductions such as sum or amax read at 2-4 TB/s)
    m = src.view(torch.bfloat16).view(32768, -1)
    vec = torch.ones(m.shape[1], dtype=torch.bfloat16, device="cuda")
    for _ in range(2):
        torch.mv(m, vec)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        torch.mv(m, vec)
    e1.record()
    torch.cuda.synchronize()
    rgbs = src.numel() * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, m, vec
    torch.cuda.empty_cache()
    return {"mfma_bf16_tflops": round(tflops, 1), "hbm_copy_gbs": round(gbs, 1),
            "hbm_read_gbs": round(rgbs, 1),
            "how": "torch.mm bf16 8192^3; 2 GiB device-to-device copy, read + write bytes; "
                   "torch.mv bf16 over a 2 GiB matrix, bytes read"}


def algorithmic(cfg, T, n_active):
    """Flops and bytes of one layer call (the definition, not what the kernels move)."""
    d, F, Fs, k, E = cfg.d, cfg.F, cfg.Fs, cfg.k, cfg.E
    import workloads as W
    wbytes = {"i4g32": 0.5 + 2 / 32, "bf16": 2.0, "i8row": 1.0, "mxfp4": 0.5 + 1 / 32}
    wbytes.update({name: b / 8 + 2 / 32 for b, name in W.IG32.items()})
    ffn_flops = 6.0 * T * k * d * F + 6.0 * T * d * Fs
    router_flops = 2.0 * T * E * d
    per_expert = 3 * d * F * wbytes[cfg.expert]
    shared = 3 * d * Fs * wbytes[cfg.shared] + (2 * Fs + d) * 2 * (cfg.shared == "i8row")
    weight_bytes = n_active * per_expert + shared
    act = T * d * 2 * 2 + E * d * 2                     # x in, y out, router weights
    # h written and read back (bf16; MXFP4 layers: e2m1 codes + E8M0 scales,
    # and x's codes written and read once); per-assignment and shared outputs
    # (fp32) written by the down products and read by the combine
    mx = cfg.expert == W.MXFP4
    hb = 0.5 + 1 / 32 if mx else 2.0
    inter = (T * k * F * hb * 2 + T * Fs * 2 * 2 + T * k * d * 4 * 2 + T * d * 4 * 2
             + (T * d * hb * 2 if mx else 0))
    return dict(ffn_flops=ffn_flops, router_flops=router_flops, weight_bytes=weight_bytes,
                ffn_bytes=weight_bytes + T * d * 2 + inter - T * d * 4 - T * k * d * 4,
                layer_bytes=weight_bytes + act + inter)


def cpu_baseline(cfg, inp: dict, T: int, n_tok: int):
    """The fp64 oracle (never tuned) on a bounded token sample of the same workload."""
    import oracle
    fm = {"f32": oracle.F32, "bf16": oracle.BF16, "i4g32": oracle.I4G32, "i8row": oracle.I8ROW}
    rng = np.random.default_rng(123)
    tok = np.sort(rng.choice(T, size=min(n_tok, T), replace=False))
    spec = dict(d=cfg.d, E=cfg.E, k=cfg.k, F=cfg.F, n_shared=cfg.n_shared, Fs=cfg.Fs,
                x_fmt=fm[cfg.act], expert_fmt=fm[cfg.expert], shared_fmt=fm[cfg.shared])
    t0 = time.perf_counter()
    L = oracle.router_logits(inp["x"], fm[cfg.act], inp["wr"], fm[cfg.act], cfg.d, cfg.E,
                             bias=inp.get("bias"), tokens=tok)
    ids, w = oracle.topk_softmax(L, cfg.k)
    oracle.moe_experts(spec, inp, ids, w, tokens=tok, want_parts=False)
    dt = time.perf_counter() - t0
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": round(len(tok) / dt, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{len(tok)} of the {T} tokens of the same seeded workload, whole layer "
                      f"(fp64 router, top-k, per-expert SwiGLU, shared expert, sum); {dt:.1f} s"}


GEMM_SOURCES = ("ffn.hip", "ffn_kernels.h", "wave_tile.h", "moe_internal.h", "device_common.h")
MX_SOURCES = ("ffn_mx.hip", "ffn_kernels.h", "wave_tile.h", "moe_internal.h", "device_common.h")


def sources_sha(files) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "expert_grouped_quantized_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def counted_traffic(workload: str):
    """HBM bytes per moe_grouped_ffn launch from the committed rocprofv3 counter
    runs (profiles/hbm_traffic.json: FETCH_SIZE and WRITE_SIZE, each scaled by
    what it reads for a 1 GiB copy), or None once the sources of the kernels
    that launch runs have changed since those counters were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if workload not in rec:
        return None
    files = MX_SOURCES if workload.startswith("mxfp4") else GEMM_SOURCES
    key = "mx_src_sha256" if workload.startswith("mxfp4") else "src_sha256"
    if rec.get(key) != sources_sha(files):
        return None
    return rec[workload]["grouped_ffn_bytes_per_launch"]


def run_prefill(args, torch, W):
    """The T=4096 prefill workload; returns (result dict, roofline dict, host inputs)."""
    cfg = W.CONFIGS["int4_T4096"]
    S = Setup(cfg, cfg.T, torch)
    wall, layer_ms, per_call = time_steps(S, args.steps, args.warmup)
    ms_per_step = wall * 1e3 / args.steps
    n_active = int((np.diff(S.layer.offsets.cpu().numpy()) > 0).sum())
    A = algorithmic(cfg, cfg.T, n_active)
    ffn_ms = per_call[2]
    ffn_tflops = A["ffn_flops"] / (ffn_ms * 1e-3) / 1e12
    layer_tflops = (A["ffn_flops"] + A["router_flops"]) / (ms_per_step * 1e-3) / 1e12
    res = dict(T=cfg.T, tokens_per_s=cfg.T / (ms_per_step * 1e-3), ms_per_step=ms_per_step,
               layer_event_ms=layer_ms,
               call_ms=call_ms(per_call, cfg.T),
               layer_tflops=layer_tflops, layer_mfma_frac=layer_tflops / BF16_PEAK_TFLOPS,
               layer_gbs=A["layer_bytes"] / (ms_per_step * 1e-3) / 1e9)
    roof = {"bound": "mfma", "kernel": "moe_grouped_ffn (gate/up + down GEMMs)",
            "achieved": round(ffn_tflops, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(ffn_tflops / BF16_PEAK_TFLOPS, 4), "traffic": counted_traffic("prefill"),
            "algorithmic_flops_per_launch": A["ffn_flops"], "avg_launch_ms": round(ffn_ms, 4)}
    inputs = S.inputs
    del S
    torch.cuda.empty_cache()
    return res, roof, inputs


def run_decode(args, torch, W):
    """The T=16 decode / verify workload; returns (result dict, roofline dict)."""
    dcfg = W.CONFIGS["int4_decode"]
    D = Setup(dcfg, 16, torch)
    dwall, dlayer_ms, dper = time_steps(D, args.decode_steps, 10)
    d_ms = dwall * 1e3 / args.decode_steps
    d_active = int((np.diff(D.layer.offsets.cpu().numpy()) > 0).sum())
    DA = algorithmic(dcfg, 16, d_active)
    ffn_gbs = DA["weight_bytes"] / (dper[2] * 1e-3) / 1e9
    res = dict(T=16, tokens_per_s=16 / (d_ms * 1e-3), ms_per_step=d_ms, active_experts=d_active,
               layer_event_ms=dlayer_ms,
               call_ms=call_ms(dper, 16),
               weight_bytes=DA["weight_bytes"],
               layer_hbm_frac=DA["layer_bytes"] / (d_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
               ffn_weight_gbs=ffn_gbs)
    roof = {"bound": "hbm", "kernel": "moe_grouped_ffn (gate/up + down weight streams)",
            "achieved": round(ffn_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ffn_gbs / HBM_PEAK_GBS, 4), "traffic": counted_traffic("decode"),
            "algorithmic_bytes_per_launch": DA["weight_bytes"], "avg_launch_ms": round(dper[2], 4)}
    # the same layer as one HIP graph per step, at 16 rows and at 32 rows (a
    # verify batch): the 32-row call's cost against its byte ratio
    g_ms, g_ev = time_graph(D, args.decode_steps)
    res["graph"] = dict(ms_per_step=g_ms, event_ms_per_step=g_ev, tokens_per_s=16 / (g_ms * 1e-3),
                        layer_hbm_frac=DA["layer_bytes"] / (g_ms * 1e-3) / 1e9 / HBM_PEAK_GBS)
    del D
    torch.cuda.empty_cache()
    D32 = Setup(dcfg, 32, torch)
    D32.step(0)
    torch.cuda.synchronize()
    a32 = int((np.diff(D32.layer.offsets.cpu().numpy()) > 0).sum())
    g32_ms, g32_ev = time_graph(D32, args.decode_steps)
    A32 = algorithmic(dcfg, 32, a32)
    res["graph_T32"] = dict(ms_per_step=g32_ms, event_ms_per_step=g32_ev, active_experts=a32,
                            tokens_per_s=32 / (g32_ms * 1e-3),
                            layer_hbm_frac=A32["layer_bytes"] / (g32_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                            time_ratio_to_T16=g32_ms / g_ms,
                            byte_ratio_to_T16=A32["layer_bytes"] / DA["layer_bytes"])
    del D32
    torch.cuda.empty_cache()
    return res, roof


class _View:
    """A second call size on a Setup's weights (its first T rows of x)."""

    def __init__(self, S, T):
        from expert_grouped_quantized_amd.layer import MoELayer
        self.torch, self.T, self.routed = S.torch, T, S.routed
        self.x = S.x[:T].contiguous()
        self.layer = MoELayer(S.desc, S.cfg.k, T)
        self.layer.set_weights(S.wr, S.routed[0], S.shared, S.bias)

    step = Setup.step


def run_bits(args, torch, W):
    """Every routed code width (2..8 bits, group-32 fp16 scales) on the prefill
    layer shape: T=4096 eager steps and T=16 as one HIP graph per step."""
    import dataclasses
    out = {}
    for b in (2, 3, 4, 5, 6, 7, 8):
        fmt = W.I4G32 if b == 4 else W.IG32[b]
        cfg = dataclasses.replace(W.CONFIGS["int4_T4096"], name=f"bits{b}_T4096", expert=fmt)
        S = Setup(cfg, cfg.T, torch)
        wall, layer_ms, per = time_steps(S, args.steps, args.warmup)
        ms = wall * 1e3 / args.steps
        act = int((np.diff(S.layer.offsets.cpu().numpy()) > 0).sum())
        A = algorithmic(cfg, cfg.T, act)
        D = _View(S, 16)
        D.step(0)
        torch.cuda.synchronize()
        d_act = int((np.diff(D.layer.offsets.cpu().numpy()) > 0).sum())
        DA = algorithmic(cfg, 16, d_act)
        g_ms, _ = time_graph(D, args.decode_steps)
        out[f"{b}bit"] = dict(
            prefill_tokens_per_s=cfg.T / (ms * 1e-3), prefill_ms=ms, prefill_ffn_ms=per[2],
            prefill_ffn_tflops=A["ffn_flops"] / (per[2] * 1e-3) / 1e12,
            decode_graph_tokens_per_s=16 / (g_ms * 1e-3), decode_graph_ms=g_ms,
            decode_weight_bytes=DA["weight_bytes"],
            decode_layer_hbm_frac=DA["layer_bytes"] / (g_ms * 1e-3) / 1e9 / HBM_PEAK_GBS)
        print(f"[bench] {b}-bit: prefill {ms:.3f} ms (ffn {per[2]:.3f}), decode graph "
              f"{g_ms * 1e3:.1f} us", file=sys.stderr, flush=True)
        del S, D
        torch.cuda.empty_cache()
    return out


def run_mxfp4(args, torch, W):
    """MXFP4 W4A4 routed experts (scaled FP4 MFMA) on the prefill layer shape:
    T=4096 eager steps; its first 16 rows as eager steps and as one HIP graph
    per step; its first 32 rows as a graph."""
    import dataclasses
    cfg = dataclasses.replace(W.CONFIGS["int4_T4096"], name="mxfp4_T4096", expert=W.MXFP4)
    S = Setup(cfg, cfg.T, torch)
    wall, layer_ms, per = time_steps(S, args.steps, args.warmup)
    ms = wall * 1e3 / args.steps
    act = int((np.diff(S.layer.offsets.cpu().numpy()) > 0).sum())
    A = algorithmic(cfg, cfg.T, act)
    ffn_s = per[2] * 1e-3
    pre = dict(T=cfg.T, tokens_per_s=cfg.T / (ms * 1e-3), ms_per_step=ms, layer_event_ms=layer_ms,
               call_ms=call_ms(per, cfg.T),
               active_experts=act,
               ffn_tflops=A["ffn_flops"] / ffn_s / 1e12,
               ffn_fp4_mfma_frac=A["ffn_flops"] / ffn_s / 1e12 / FP4_PEAK_TFLOPS,
               ffn_algorithmic_bytes=A["ffn_bytes"],
               ffn_gbs=A["ffn_bytes"] / ffn_s / 1e9,
               ffn_hbm_frac=A["ffn_bytes"] / ffn_s / 1e9 / HBM_PEAK_GBS)
    out = {"prefill": pre}
    out["roofline"] = {
        "bound": "hbm", "kernel": "moe_grouped_ffn (x -> MXFP4, FP4 gate/up + h -> MXFP4, FP4 down)",
        "achieved": round(pre["ffn_gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(pre["ffn_hbm_frac"], 4), "traffic": counted_traffic("mxfp4_prefill"),
        "algorithmic_bytes_per_launch": A["ffn_bytes"], "avg_launch_ms": round(per[2], 4),
        "fp4_mfma_frac": round(pre["ffn_fp4_mfma_frac"], 4)}
    for T in (16, 32):
        D = _View(S, T)
        D.step(0)
        torch.cuda.synchronize()
        d_act = int((np.diff(D.layer.offsets.cpu().numpy()) > 0).sum())
        DA = algorithmic(cfg, T, d_act)
        rec = dict(T=T, active_experts=d_act, weight_bytes=DA["weight_bytes"])
        if T == 16:
            dwall, dlayer, dper = time_steps(D, args.decode_steps, 10)
            d_ms = dwall * 1e3 / args.decode_steps
            rec.update(tokens_per_s=T / (d_ms * 1e-3), ms_per_step=d_ms, layer_event_ms=dlayer,
                       call_ms=call_ms(dper, T),
                       ffn_weight_gbs=DA["weight_bytes"] / (dper[2] * 1e-3) / 1e9,
                       ffn_weight_hbm_frac=DA["weight_bytes"] / (dper[2] * 1e-3) / 1e9 / HBM_PEAK_GBS)
            out["decode_roofline"] = {
                "bound": "hbm", "kernel": "moe_grouped_ffn at T=16 (weight streams)",
                "achieved": round(rec["ffn_weight_gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(rec["ffn_weight_hbm_frac"], 4),
                "traffic": counted_traffic("mxfp4_decode"),
                "algorithmic_bytes_per_launch": DA["weight_bytes"], "avg_launch_ms": round(dper[2], 4)}
        g_ms, g_ev = time_graph(D, args.decode_steps)
        rec["graph"] = dict(ms_per_step=g_ms, event_ms_per_step=g_ev, tokens_per_s=T / (g_ms * 1e-3),
                            layer_hbm_frac=DA["layer_bytes"] / (g_ms * 1e-3) / 1e9 / HBM_PEAK_GBS)
        out[f"decode_T{T}"] = rec
        print(f"[bench] mxfp4 T={T}: graph {g_ms * 1e3:.1f} us", file=sys.stderr, flush=True)
        del D
        torch.cuda.empty_cache()
    print(f"[bench] mxfp4 T=4096: {ms:.3f} ms (ffn {per[2]:.3f} ms)", file=sys.stderr, flush=True)
    del S
    torch.cuda.empty_cache()
    return out


CPU_SAMPLE = {"bf16_T512": 512, "bf16w_T4096": 1024, "zipf_T16384": 2048}


def run_configs(args, torch, W, with_cpu=False):
    """The layer configurations measured beside the headline ones, each as
    eager steps with the roofline its shape sits under: the bf16 layer at
    T=512 (weight bound: every expert's bf16 weights read once), the T=4096
    layer with bf16 routed weights (also weight bound), and T=16384 with int4
    routed experts and Zipf-skewed routing (MFMA bound).  with_cpu: the oracle
    timed on a token sample of each (CPU_SAMPLE tokens)."""
    import dataclasses
    cases = [("bf16_T512", W.CONFIGS["bf16_T512"], "hbm"),
             ("bf16w_T4096", dataclasses.replace(W.CONFIGS["int4_T4096"], name="bf16w_T4096",
                                                 expert=W.BF16), "hbm"),
             ("zipf_T16384", W.CONFIGS["zipf_T16384"], "mfma")]
    out = {}
    for name, cfg, bound in cases:
        S = Setup(cfg, cfg.T, torch)
        steps = max(5, args.steps // (4 if cfg.T > 4096 else 1))
        wall, layer_ms, per = time_steps(S, steps, args.warmup)
        ms = wall * 1e3 / steps
        counts = np.diff(S.layer.offsets.cpu().numpy())
        act = int((counts > 0).sum())
        A = algorithmic(cfg, cfg.T, act)
        ffn_s = per[2] * 1e-3
        rec = dict(T=cfg.T, routed_w=cfg.expert, shared_w=cfg.shared, bound=bound,
                   tokens_per_s=cfg.T / (ms * 1e-3), ms_per_step=ms, layer_event_ms=layer_ms,
                   call_ms=call_ms(per, cfg.T),
                   active_experts=act, max_over_mean_load=float(counts.max() / counts.mean()),
                   ffn_tflops=A["ffn_flops"] / ffn_s / 1e12,
                   ffn_mfma_frac=A["ffn_flops"] / ffn_s / 1e12 / BF16_PEAK_TFLOPS,
                   ffn_algorithmic_bytes=A["ffn_bytes"],
                   ffn_gbs=A["ffn_bytes"] / ffn_s / 1e9,
                   ffn_hbm_frac=A["ffn_bytes"] / ffn_s / 1e9 / HBM_PEAK_GBS,
                   layer_hbm_frac=A["layer_bytes"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS)
        if with_cpu:
            rec["cpu_baseline"] = cpu_baseline(cfg, S.inputs, cfg.T, CPU_SAMPLE[name])
        out[name] = rec
        print(f"[bench] {name}: {ms:.3f} ms/step (ffn {per[2]:.3f} ms, "
              f"{rec['ffn_tflops']:.0f} TFLOP/s, {rec['ffn_gbs']:.0f} GB/s)", file=sys.stderr,
              flush=True)
        del S
        torch.cuda.empty_cache()
    return out


def _r(d):
    return {k: (round(v, 4) if isinstance(v, float) else _r(v) if isinstance(v, dict) else v)
            for k, v in d.items()}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the library runs the "
              "layer on one GPU and has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    import torch
    import workloads as W
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)

    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.workload == "bits":
        bits = run_bits(args, torch, W)
        print(json.dumps({"metric": "MoE-layer tokens/s across routed code widths (T=4096 "
                                    "prefill; T=16 decode as one HIP graph)",
                          "unit": "tokens/s", "n_gpus": 1, "data": "synthetic",
                          "config": {"d": 2560, "E": 512, "k": 10, "F": 1024, "n_shared": 1,
                                     "routed_w": "b-bit symmetric codes, fp16 scale per 32",
                                     "shared_w": "int8 per-row fp16 scales"},
                          "bit_widths": _r(bits)}), flush=True)
        return
    if args.workload == "configs":
        cf = run_configs(args, torch, W)
        print(json.dumps({"metric": "MoE-layer tokens/s and roofline fraction of the other layer "
                                    "configurations (bf16 T=512, bf16 routed weights at T=4096, "
                                    "Zipf-skewed T=16384)",
                          "unit": "tokens/s", "n_gpus": 1, "data": "synthetic",
                          "peaks": {"bf16_mfma_tflops": BF16_PEAK_TFLOPS,
                                    "hbm_gbs": HBM_PEAK_GBS},
                          "configs": _r(cf)}), flush=True)
        return
    if args.workload == "mxfp4":
        mx = run_mxfp4(args, torch, W)
        peaks = measured_peaks(torch)
        mx["decode_roofline"]["frac_of_measured_peak"] = round(
            mx["decode_roofline"]["achieved"] / peaks["hbm_read_gbs"], 4)
        print(json.dumps({"metric": "MoE-layer tokens/s with MXFP4 W4A4 routed experts (T=4096 "
                                    "prefill; T=16 and T=32 decode)",
                          "unit": "tokens/s", "n_gpus": 1, "data": "synthetic", "dtype": "fp4",
                          "config": {"workload": "moe_layer_mxfp4_w4a4", "d": 2560, "E": 512,
                                     "k": 10, "F": 1024, "n_shared": 1,
                                     "routed_w": "MXFP4 (e2m1 + E8M0 per 32), activations "
                                                 "MXFP4-quantized per 32",
                                     "shared_w": "int8 per-row fp16 scales, bf16 activations"},
                          "peaks": {"fp4_mfma_tflops": FP4_PEAK_TFLOPS, "hbm_gbs": HBM_PEAK_GBS},
                          "measured_peaks": peaks,
                          "mxfp4": _r(mx)}), flush=True)
        return
    prefill = decode = roof_p = roof_d = pre_inputs = configs = None
    if args.workload in ("both", "prefill"):
        prefill, roof_p, pre_inputs = run_prefill(args, torch, W)
    if args.workload in ("both", "decode"):
        decode, roof_d = run_decode(args, torch, W)
    cpu = None
    if not args.no_cpu_baseline and pre_inputs is not None:
        cfg = W.CONFIGS["int4_T4096"]
        cpu = cpu_baseline(cfg, pre_inputs, cfg.T, args.cpu_sample_tokens)
        del pre_inputs
    if args.workload == "both" and not args.no_configs:
        configs = run_configs(args, torch, W, with_cpu=not args.no_cpu_baseline)
    peaks = measured_peaks(torch)

    cfg = W.CONFIGS["int4_T4096"]
    common = {"d": cfg.d, "E": cfg.E, "k": cfg.k, "n_shared": cfg.n_shared, "F": cfg.F,
              "routed_w": "int4 g32 fp16 scales", "shared_w": "int8 per-row fp16 scales",
              "activations": "bf16"}
    if prefill is not None:
        head, roof, steps = prefill, roof_p, args.steps
        metric = "MoE-layer tokens/s at T=4096 prefill (int4 g32 experts, int8 shared)"
        workload = "moe_layer_int4_T4096_prefill"
        warm = args.warmup
    else:
        head, roof, steps = decode, roof_d, args.decode_steps
        metric = "MoE-layer tokens/s at T=16 decode (int4 g32 experts, int8 shared)"
        workload = "moe_layer_int4_T16_decode"
        warm = 10
    line = {
        "metric": metric,
        "value": round(head["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": round(head["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": dict({"workload": workload, "T": head["T"]}, **common),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    line["measured_peaks"] = peaks
    if roof_p is not None:
        roof_p["frac_of_measured_peak"] = round(roof_p["achieved"] / peaks["mfma_bf16_tflops"], 4)
    if roof_d is not None:
        roof_d["frac_of_measured_peak"] = round(roof_d["achieved"] / peaks["hbm_read_gbs"], 4)
    if prefill is not None:
        line["prefill"] = _r(prefill)
    if decode is not None:
        line["decode"] = _r(decode)
        line["decode_roofline"] = roof_d
    if configs is not None:
        line["configs"] = _r(configs)
    print(json.dumps(line, default=float), flush=True)


if __name__ == "__main__":
    main()
