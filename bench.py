#!/usr/bin/env python3
"""Throughput of the RMM hot path on one MI355X.

One step = one pass of every reduced product of a layer over one batch of
synthetic input already resident in HBM: for each projection, column scores ->
top-k -> reduced GEMM (q/k/v share one selection, up/gate share one, since
the scores depend on A only); then the feature-reduced Q K^T and the
token-reduced P V over all heads, both in their causal form (the layer is a
causal decoder: S above the diagonal is not needed and P is zero there).  The
attention probabilities P are a precomputed input (a causal softmax of the
layer's logits), like X.

Prints one JSON line.  `value` is effective TFLOP/s: the dense-equivalent
flops of the step (2 m d n per projection, 2 dh per causal query-key pair,
per head, for each attention product) divided by the measured step time.

`fused_attention` times, beside the step, the fused reduced attention
(rmm_attention: Q, K, V -> O with the softmax, the token scores and both
selections inside, S and P never written) on the same Q, K and V, at the
layer's ratio and at rho = 1.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
DEFAULT_WORKLOAD = "llama3.1-8b-layer-16k"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--rho", type=float, default=None, help="projection ratio filter (multi-ratio workloads)")
    ap.add_argument("--m", type=int, default=None, help="token-count filter (multi-m workloads)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true", help="skip the rho = 1 pass")
    ap.add_argument("--no-fuse", action="store_true",
                    help="one reduced product per weight instead of one per shared activation")
    ap.add_argument("--graph", action="store_true",
                    help="replay the step from a captured HIP graph (launch-bound shapes such as decode batches)")
    ap.add_argument("--no-fused-attention", action="store_true",
                    help="skip the separate timing of the fused reduced attention (rmm_attention)")
    ap.add_argument("--no-producers", action="store_true",
                    help="skip the separate timing of the producer-fused scoring kernels")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the compact timings of the other workloads (default workload only)")
    ap.add_argument("--cpu-ops", action="store_true",
                    help="only time the CPU oracle per op on every workload (baseline table) and exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for HBM counters)")
    return ap.parse_args()


# ------------------------------------------------------------------ workload
def build_layer(wl, args, dev, cache=None):
    """The projections and attention of the run's workload, as build_layer_for builds them."""
    return build_layer_for(wl, _selected(wl, args), dev, args.no_fuse, _has_attention(wl, args), cache)


def build_layer_for(wl, lins, dev, no_fuse=False, with_attention=True, cache=None):
    """Device tensors of the given projections (and the workload's attention):
    seeded synthetic activations and weights, resident in HBM.  `cache` (a dict)
    keeps generated tensors for later layers of the same workload (other
    ratios reuse the same activations and weights)."""
    import torch

    import synth

    cache = {} if cache is None else cache
    dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    layer = {"linears": [], "attention": None, "dtype": dt}
    for lin in lins:
        key = synth.activation_key(wl, lin)
        if ("A", key) not in cache:
            cache[("A", key)] = torch.from_numpy(synth.linear_activation(wl, lin)).to(dev, dt)
        bkey = ("B", lin.tensor_b, lin.d, lin.n)
        if bkey not in cache:
            cache[bkey] = torch.from_numpy(synth.linear_weight(wl, lin)).to(dev, dt)
        B = cache[bkey]
        prev = [e for e in layer["linears"] if e["akey"] == key and e["rho"] == lin.rho]
        if prev and not no_fuse:
            # Same activation and ratio: the selection is the same, so the
            # products are one reduced product over the weights side by side
            # ([d][n1 + n2 ...]), as a fused q|k|v or up|gate projection.
            e = prev[0]
            e["B"] = torch.cat([e["B"], B], dim=1).contiguous()
            e["n"] += lin.n
            e["name"] = e["name"].split("@")[0] + "+" + lin.name
            continue
        layer["linears"].append({
            "name": lin.name, "m": lin.m, "d": lin.d, "n": lin.n, "rho": lin.rho,
            "A": cache[("A", key)], "akey": key, "B": B,
        })
    if wl.attention is not None and with_attention:
        at = wl.attention
        if "attention" not in cache:
            Q, Kt, V = synth.attention_operands(wl)
            Qd = torch.from_numpy(Q).to(dev, torch.bfloat16)
            Ktd = torch.from_numpy(Kt).to(dev, torch.bfloat16)
            Vd = torch.from_numpy(V).to(dev, torch.bfloat16)
            del Q, Kt, V
            P = synth.causal_probs(Qd, Ktd, 1.0 / math.sqrt(at.dh), device=dev)
            cache["attention"] = (Qd, Ktd, Vd, P)
        Qd, Ktd, Vd, P = cache["attention"]
        layer["attention"] = {"Q": Qd, "Kt": Ktd, "V": Vd, "P": P, "L": at.L, "Hq": at.Hq, "Hkv": at.Hkv,
                              "dh": at.dh, "rho": at.rho}
    return layer


class Runner:
    """Holds outputs/workspaces for one ratio setting and runs a step."""

    def __init__(self, R, layer, dev, rho_scale_one=False):
        import torch

        self.R, self.layer, self.dev = R, layer, dev
        dt = layer["dtype"]
        self.plan = []
        self.sel = {}
        ws_cn = ws_g = 0
        for lin in layer["linears"]:
            k = lin["d"] if rho_scale_one else R.rmm_k_from_rho(lin["rho"], lin["d"])
            skey = (lin["akey"], k)
            if skey not in self.sel:
                self.sel[skey] = {
                    "scores": torch.empty(lin["d"], dtype=torch.float32, device=dev),
                    "idx": torch.empty(R.rmm_k_pad(k), dtype=torch.int32, device=dev),
                    "owner": lin["name"],
                }
                ws_cn = max(ws_cn, R.rmm_colnorm_workspace_bytes(dt, lin["m"], lin["d"], 1))
            ws_g = max(ws_g, R.rmm_gemm_workspace_bytes(dt, lin["m"], lin["n"], k))
            self.plan.append({**lin, "k": k, "skey": skey,
                              "Y": torch.empty((lin["m"], lin["n"]), dtype=dt, device=dev)})
        self.ws_cn = torch.empty(max(ws_cn, 1), dtype=torch.uint8, device=dev)
        self.ws_g = torch.empty(max(ws_g, 1), dtype=torch.uint8, device=dev)
        at = layer["attention"]
        self.att = None
        if at is not None:
            kf = at["dh"] if rho_scale_one else R.rmm_k_from_rho(at["rho"], at["dh"])
            kt = at["L"] if rho_scale_one else R.rmm_k_from_rho(at["rho"], at["L"])
            self.att = {
                "kf": kf, "kt": kt,
                "S": torch.empty((at["Hq"], at["L"], at["L"]), dtype=torch.float32, device=dev),
                "O": torch.empty((at["L"], at["Hq"], at["dh"]), dtype=torch.bfloat16, device=dev),
                "iq": torch.empty((at["Hq"], R.rmm_k_pad(kf)), dtype=torch.int32, device=dev),
                "ip": torch.empty((at["Hq"], R.rmm_k_pad(kt)), dtype=torch.int32, device=dev),
                "wq": torch.empty(R.rmm_qk_workspace_bytes(at["L"], at["Hq"], at["dh"], kf), dtype=torch.uint8,
                                  device=dev),
                "wp": torch.empty(R.rmm_pv_workspace_bytes(at["Hq"], at["L"], at["L"], kt), dtype=torch.uint8,
                                  device=dev),
            }

    def free(self):
        self.plan = self.sel = self.att = None
        self.ws_cn = self.ws_g = None

    def step(self, tagged=False):
        R = self.R
        T = R.timing
        done = set()
        for p in self.plan:
            s = self.sel[p["skey"]]
            if p["skey"] not in done:
                if tagged:
                    T.tag(p["name"].split("@")[0])
                R.rmm_colnorm(p["A"], out=s["scores"], ws=self.ws_cn)
                R.rmm_topk(s["scores"], p["k"], out=s["idx"])
                done.add(p["skey"])
            if tagged:
                T.tag(p["name"].split("@")[0])
            R.rmm_gemm(p["A"], p["B"], s["idx"], p["k"], out=p["Y"], ws=self.ws_g)
        if self.att is not None:
            at, a = self.layer["attention"], self.att
            if tagged:
                T.tag("qk")
            R.rmm_qk(at["Q"], at["Kt"], a["kf"], S=a["S"], idx=a["iq"], ws=a["wq"], causal=True)
            if tagged:
                T.tag("pv")
            R.rmm_pv(at["P"], at["V"], a["kt"], O=a["O"], idx=a["ip"], ws=a["wp"], causal=True)
        if tagged:
            T.tag(None)


def causal_pairs(L):
    """(query, key) pairs a causal layer of L tokens uses: L (L + 1) / 2."""
    return L * (L + 1) / 2.0


def dense_flops(layer):
    """Dense-equivalent flops of the step: 2 m d n per projection; for the causal
    attention products, 2 dh per used (query, key) pair, per head, for each of
    Q K^T and P V."""
    f = sum(2.0 * l["m"] * l["d"] * l["n"] for l in layer["linears"])
    at = layer["attention"]
    if at is not None:
        f += 2 * (2.0 * causal_pairs(at["L"]) * at["dh"] * at["Hq"])
    return f


class GraphStep:
    """One step of a runner captured into a HIP graph (torch.cuda.CUDAGraph); the
    library launches on torch's current stream, which the capture redirects."""

    def __init__(self, runner):
        import torch

        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            runner.step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        self.g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.g):
            runner.step()
        torch.cuda.synchronize()

    def step(self, tagged=False):
        self.g.replay()


def time_steps(runner, steps, warmup):
    import torch

    for _ in range(warmup):
        runner.step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        runner.step()
    e1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    return e0.elapsed_time(e1) / steps, wall


def step_distribution(runner, steps, flush_buf=None):
    """Per-step times (HIP events around each step): median, p10 and p90 in ms.
    With `flush_buf` (>= 1 GiB), the buffer is overwritten before every step,
    outside the timed span, so the 256 MB Infinity Cache holds none of the
    step's operands when it starts (cold cache)."""
    import numpy as np
    import torch

    ts = []
    for _ in range(steps):
        if flush_buf is not None:
            flush_buf.fill_(1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        runner.step()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    a = np.asarray(ts)
    return {"median_ms": round(float(np.median(a)), 4), "p10_ms": round(float(np.percentile(a, 10)), 4),
            "p90_ms": round(float(np.percentile(a, 90)), 4), "steps": steps}


def torch_matmul_context(layer, steps, warmup):
    """Context only: the step's projections as dense torch.matmul (hipBLASLt) on
    the same A and B, with no selection (ms per step)."""
    import torch

    outs = [torch.empty((l["m"], l["n"]), dtype=layer["dtype"], device=l["A"].device) for l in layer["linears"]]

    class _D:
        def step(self, tagged=False):
            for l, o in zip(layer["linears"], outs):
                torch.matmul(l["A"], l["B"], out=o)

    ms, _ = time_steps(_D(), steps, warmup)
    del outs
    return round(ms, 4)


def kernel_breakdown(runner, steps):
    """Per tag/kernel average launch durations (HIP events recorded by the library)."""
    import torch

    R = runner.R
    R.timing.reset()
    R.timing.enable(True)
    for _ in range(steps):
        runner.step(tagged=True)
    torch.cuda.synchronize()
    R.timing.enable(False)
    tot = R.timing.collect()
    R.timing.reset()
    return {k: {"avg_ms": v[0] / v[1], "launches_per_step": v[1] / steps} for k, v in tot.items()}


def algorithmic_work(runner, key):
    """(bound, amount per launch, unit) for a tag/kernel entry of the step."""
    tag, kern = key.split("/", 1) if "/" in key else ("", key)
    at = runner.layer["attention"]
    a = runner.att
    if tag == "qk" and "gemm" in kern:
        # A_I and B_I read once, the causal part of S written (fp32)
        per_head = at["L"] * a["kf"] * 2 + a["kf"] * at["L"] * 2 + causal_pairs(at["L"]) * 4
        return "hbm", per_head * at["Hq"], "bytes"
    if tag == "pv" and "gemm" in kern:
        per_head = at["L"] * a["kt"] * 2 + a["kt"] * at["dh"] * 2 + at["L"] * at["dh"] * 2
        return "hbm", per_head * at["Hq"], "bytes"
    if tag == "pv" and kern == "colnorm":
        # the causal part of P read once
        return "hbm", at["Hq"] * (causal_pairs(at["L"]) * 2 + 4 * at["L"]), "bytes"
    if tag == "pv" and kern == "pack":
        return "hbm", at["Hq"] * at["L"] * a["kt"] * 2 * 2, "bytes"
    if tag == "qk" and kern == "colnorm":
        return "hbm", at["Hq"] * (at["L"] * at["dh"] * 2 + 4 * at["dh"]), "bytes"
    if tag == "qk" and kern == "pack":
        return "hbm", at["Hq"] * at["L"] * a["kf"] * 2 * 2, "bytes"
    plans = [p for p in runner.plan if p["name"].split("@")[0] == tag]
    if not plans:
        return None, 0, None
    p = plans[0]
    e = 4 if runner.layer["dtype"].itemsize == 4 else 2
    if kern.startswith("gemm"):
        # MFMA-bound unless reading the operands once takes longer at peak
        # bandwidth than the kept flops at peak rate (few rows: decode batches).
        flops = 2.0 * p["m"] * p["k"] * p["n"]
        byts = float(p["m"] * p["k"] * e + p["k"] * p["n"] * e + p["m"] * p["n"] * e)
        peak_f = (PEAK_F32_TFLOPS if e == 4 else PEAK_BF16_TFLOPS) * 1e12
        if byts / (PEAK_HBM_GBS * 1e9) > flops / peak_f:
            return "hbm", byts, "bytes"
        return "mfma", flops, "flops"
    if kern == "bt_pack":
        # kept weight rows read, their transposed copy written
        return "hbm", 2.0 * p["k"] * p["n"] * e, "bytes"
    if kern == "colnorm":
        return "hbm", p["m"] * p["d"] * e + 4 * p["d"], "bytes"
    if kern == "pack":
        return "hbm", p["m"] * p["k"] * e * 2, "bytes"
    return None, 0, None


def fused_attention(R, layer, steps, warmup, dense=True):
    """Time rmm_attention on the layer's Q, K and V: the whole reduced chain
    (feature selection, Q K^T, causal softmax, token scores, token selection,
    P V) in one call that never writes S or P, at the layer's ratio and at
    rho = 1 (every feature and token kept).  Effective TFLOP/s counts the same
    dense-equivalent attention flops as the step."""
    import numpy as np
    import torch

    at = layer["attention"]
    L, Hq, dh = at["L"], at["Hq"], at["dh"]
    fl = 2 * (2.0 * causal_pairs(L) * dh * Hq)
    res = {}
    ratios = [("rho", R.rmm_k_from_rho(at["rho"], dh), R.rmm_k_from_rho(at["rho"], L))]
    if dense:
        ratios.append(("rho1", dh, L))
    for name, kf, kt in ratios:
        dev = at["Q"].device
        O = torch.empty((L, Hq, dh), dtype=torch.bfloat16, device=dev)
        If = torch.empty((Hq, R.rmm_k_pad(kf)), dtype=torch.int32, device=dev)
        It = torch.empty((Hq, R.rmm_k_pad(kt)), dtype=torch.int32, device=dev)
        ws = torch.empty(R.rmm_attention_workspace_bytes(L, L, Hq, dh, kf, kt), dtype=torch.uint8, device=dev)

        class _One:
            def step(self, tagged=False):
                R.rmm_attention(at["Q"], at["Kt"], at["V"], kf, kt, O=O, idx_feat=If, idx_tok=It, ws=ws,
                                causal=True)

        ms, _ = time_steps(_One(), steps, warmup)
        res[name] = {"k_feat": kf, "k_tok": kt, "ms": round(ms, 4), "effective_tflops": round(fl / (ms * 1e-3) / 1e12, 1)}
        if name == "rho":
            R.timing.reset()
            R.timing.enable(True)
            n = max(2, min(steps, 5))
            for _ in range(n):
                _One().step()
            torch.cuda.synchronize()
            R.timing.enable(False)
            tot = R.timing.collect()
            R.timing.reset()
            # exponentials per pass: every visible (query, key) pair in the two
            # statistics passes, every visible (query, kept token) pair in the output pass
            J = It[:, :kt].cpu().numpy().astype(np.float64)
            n_exp = {"attn_stats": Hq * causal_pairs(L), "attn_colsq": Hq * causal_pairs(L),
                     "attn_out": float((L - J).sum())}
            kern = {}
            for key, v in tot.items():
                e = {"avg_ms": round(v[0] / v[1], 4)}
                if key in n_exp:
                    e["gexp_per_s"] = round(n_exp[key] / (v[0] / v[1] * 1e-3) / 1e9, 1)
                kern[key] = e
            res[name]["kernels"] = kern
        del O, If, It, ws
        torch.cuda.empty_cache()
    if "rho1" in res:
        res["speedup_vs_rho1"] = round(res["rho1"]["ms"] / res["rho"]["ms"], 3)
    res["decode"] = decode_attention(R, layer, steps, warmup, dense)
    return res


def decode_attention(R, layer, steps, warmup, dense=True):
    """One new token after the layer's full context (a decode step): rmm_attention
    with Lq = 1 on the last query row and every key, replayed from a HIP graph
    (the call is a handful of short launches)."""
    import torch

    at = layer["attention"]
    L, Hq, dh = at["L"], at["Hq"], at["dh"]
    Q1 = at["Q"][L - 1:]
    out = {"Lq": 1, "context": L, "launch": "hip graph replay"}
    ratios = [("rho", R.rmm_k_from_rho(at["rho"], dh), R.rmm_k_from_rho(at["rho"], L))]
    if dense:
        ratios.append(("rho1", dh, L))
    for name, kf, kt in ratios:
        dev = Q1.device
        O = torch.empty((1, Hq, dh), dtype=torch.bfloat16, device=dev)
        If = torch.empty((Hq, R.rmm_k_pad(kf)), dtype=torch.int32, device=dev)
        It = torch.empty((Hq, R.rmm_k_pad(kt)), dtype=torch.int32, device=dev)
        ws = torch.empty(R.rmm_attention_workspace_bytes(1, L, Hq, dh, kf, kt), dtype=torch.uint8, device=dev)

        class _One:
            def step(self, tagged=False):
                R.rmm_attention(Q1, at["Kt"], at["V"], kf, kt, O=O, idx_feat=If, idx_tok=It, ws=ws, causal=True)

        ms, _ = time_steps(GraphStep(_One()), max(steps, 20), warmup)
        out[name + "_us"] = round(ms * 1e3, 1)
        del O, If, It, ws
    out["batch"] = decode_batch(R, layer, steps, warmup, dense)
    return out


def decode_batch(R, layer, steps, warmup, dense=True, nseq=16):
    """One decode step of `nseq` sequences with their own caches (rmm_attention_decode_batch):
    context lengths drawn uniformly from [L/4, L] (seeded), the layer's heads and ratio, caches
    of seeded normal draws; HIP graph replay."""
    import numpy as np
    import torch

    at = layer["attention"]
    L, Hq, Hkv, dh = at["L"], at["Hq"], at["Hkv"], at["dh"]
    dev = at["Q"].device
    rng = np.random.default_rng([0, 91, nseq])
    lens = np.sort(rng.integers(L // 4, L + 1, size=nseq)).astype(np.int32)
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    Q = torch.randn((nseq, Hq, dh), generator=g, device=dev).to(torch.bfloat16)
    Kt = torch.randn((nseq, Hkv, dh, L), generator=g, device=dev).to(torch.bfloat16)
    V = torch.randn((nseq, L, Hkv, dh), generator=g, device=dev).to(torch.bfloat16)
    ld = torch.from_numpy(lens).to(dev)
    out = {"sequences": nseq, "context_min": int(lens.min()), "context_max": int(lens.max()),
           "launch": "hip graph replay"}
    ratios = [("rho", R.rmm_k_from_rho(at["rho"], dh), [R.rmm_k_from_rho(at["rho"], int(x)) for x in lens])]
    if dense:
        ratios.append(("rho1", dh, [int(x) for x in lens]))
    for name, kf, kts in ratios:
        kd = torch.tensor(kts, dtype=torch.int32, device=dev)
        ktm = max(kts)
        O = torch.empty((nseq, Hq, dh), dtype=torch.bfloat16, device=dev)
        If = torch.empty((nseq * Hq, R.rmm_k_pad(kf)), dtype=torch.int32, device=dev)
        It = torch.empty((nseq * Hq, R.rmm_k_pad(ktm)), dtype=torch.int32, device=dev)
        ws = torch.empty(R.rmm_attention_decode_batch_workspace_bytes(nseq, Hq, dh, L, ktm), dtype=torch.uint8,
                         device=dev)

        class _B:
            def step(self, tagged=False):
                R.rmm_attention_decode_batch(Q, Kt, V, ld, kd, kf, ktm, O=O, idx_feat=If, idx_tok=It, ws=ws)

        ms, _ = time_steps(GraphStep(_B()), max(steps, 20), warmup)
        out[name + "_us"] = round(ms * 1e3, 1)
        del O, If, It, ws
    del Q, Kt, V
    torch.cuda.empty_cache()
    return out


def producer_fused(R, wl, args, steps, warmup, dev):
    """Time the producers that write a projection's A together with its column
    scores, on the layer's shapes: rmm_rmsnorm_scored (the q/k/v/gate/up input,
    m x hidden) and rmm_swiglu_scored (the down input, m x mlp), each beside the
    separate rmm_colnorm pass over the same output that it makes unnecessary.
    Bytes are the algorithmic ones (rmsnorm: read X, write Y; swiglu: read G
    and U, write H); inputs are seeded normal draws resident in HBM."""
    import torch

    sel = _selected(wl, args)
    q = next((l for l in sel if l.name == "q"), None)
    dn = next((l for l in sel if l.name == "down"), None)
    if wl.dtype != "bf16" or (q is None and dn is None):
        return None
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    bf = torch.bfloat16
    res = {}

    def timed(fn):
        class _S:
            def step(self, tagged=False):
                fn()
        return time_steps(_S(), steps, warmup)[0]

    def entry(shape, ms, nbytes, ms_colnorm):
        rate = nbytes / (ms * 1e-3) / 1e9
        return {"shape": list(shape), "ms": round(ms, 4), "gbs": round(rate, 1),
                "frac": round(rate / PEAK_HBM_GBS, 4), "colnorm_ms": round(ms_colnorm, 4)}

    if q is not None and q.d % 512 == 0 and q.d <= 8192:
        m, d = q.m, q.d
        X = torch.randn((m, d), generator=g, device=dev).mul_(
            torch.rand((m, 1), generator=g, device=dev).mul_(20.0).add_(0.05)).to(bf)
        w = torch.rand(d, generator=g, device=dev).mul_(1.3).add_(0.2).to(bf)
        Y = torch.empty((m, d), dtype=bf, device=dev)
        s = torch.empty(d, dtype=torch.float32, device=dev)
        ws = torch.empty(max(R.rmm_rmsnorm_scored_workspace_bytes(m, d), 256), dtype=torch.uint8, device=dev)
        wsc = torch.empty(max(R.rmm_colnorm_workspace_bytes(torch.bfloat16, m, d, 1), 256), dtype=torch.uint8,
                          device=dev)
        ms = timed(lambda: R.rmm_rmsnorm_scored(X, w, 1e-5, Y=Y, scores=s, ws=ws))
        ms_c = timed(lambda: R.rmm_colnorm(Y, out=s, ws=wsc))
        res["rmsnorm_scored"] = entry((m, d), ms, 2 * m * d * 2, ms_c)
        del X, w, Y, s, ws, wsc
    if dn is not None and dn.d % 8 == 0:
        m, n = dn.m, dn.d
        G = torch.randn((m, n), generator=g, device=dev).to(bf)
        U = torch.randn((m, n), generator=g, device=dev).to(bf)
        H = torch.empty((m, n), dtype=bf, device=dev)
        s = torch.empty(n, dtype=torch.float32, device=dev)
        ws = torch.empty(max(R.rmm_swiglu_scored_workspace_bytes(m, n), 256), dtype=torch.uint8, device=dev)
        wsc = torch.empty(max(R.rmm_colnorm_workspace_bytes(torch.bfloat16, m, n, 1), 256), dtype=torch.uint8,
                          device=dev)
        ms = timed(lambda: R.rmm_swiglu_scored(G, U, H=H, scores=s, ws=ws))
        ms_c = timed(lambda: R.rmm_colnorm(H, out=s, ws=wsc))
        res["swiglu_scored"] = entry((m, n), ms, 3 * m * n * 2, ms_c)
        del G, U, H, s, ws, wsc
    torch.cuda.empty_cache()
    return res


def fused_layer(R, layer, steps, warmup, dense=True):
    """A LLaMA-style layer built from the fused entry points: RMS norm with its
    column scores -> top-k -> q|k|v reduced GEMM -> fused reduced attention
    (with the column scores of O) -> top-k -> o reduced GEMM -> residual ->
    RMS norm with scores -> top-k -> up|gate reduced GEMM -> SiLU gate with
    scores -> top-k -> down reduced GEMM -> residual.  No separate column-norm
    pass and no S or P in memory.  Glue that a model would fuse elsewhere
    runs in torch inside the timed step: the transposed copy of K that the
    attention reads (feature-major) and the two residual adds.  RoPE is left
    out.  Timed at the layer's ratios and with every index kept (k = d)."""
    import torch

    at = layer["attention"]
    lin = {l["name"].split("@")[0]: l for l in layer["linears"]}
    need = ("q+k+v", "o", "up+gate", "down")
    if at is None or any(n not in lin for n in need):
        return None
    m, hid = lin["q+k+v"]["m"], lin["q+k+v"]["d"]
    mlp = lin["down"]["d"]
    Hq, Hkv, dh, L = at["Hq"], at["Hkv"], at["dh"], at["L"]
    if m != L or lin["q+k+v"]["n"] != (Hq + 2 * Hkv) * dh:
        return None
    dev = lin["o"]["A"].device
    bf = torch.bfloat16
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    X = torch.randn((m, hid), generator=g, device=dev).to(bf)
    w1 = (torch.rand(hid, generator=g, device=dev) * 1.3 + 0.2).to(bf)
    w2 = (torch.rand(hid, generator=g, device=dev) * 1.3 + 0.2).to(bf)
    Wqkv, Wo, Wug, Wd = lin["q+k+v"]["B"], lin["o"]["B"], lin["up+gate"]["B"], lin["down"]["B"]
    nq, nkv = Hq * dh, Hkv * dh
    buf = {
        "Xn": torch.empty((m, hid), dtype=bf, device=dev), "s": torch.empty(mlp, dtype=torch.float32, device=dev),
        "QKV": torch.empty((m, nq + 2 * nkv), dtype=bf, device=dev), "Kt": torch.empty((Hkv, dh, m), dtype=bf, device=dev),
        "O": torch.empty((m, Hq, dh), dtype=bf, device=dev), "os": torch.empty(nq, dtype=torch.float32, device=dev),
        "Yo": torch.empty((m, hid), dtype=bf, device=dev), "X2": torch.empty((m, hid), dtype=bf, device=dev),
        "UG": torch.empty((m, Wug.shape[1]), dtype=bf, device=dev), "H": torch.empty((m, mlp), dtype=bf, device=dev),
        "Yd": torch.empty((m, hid), dtype=bf, device=dev), "X3": torch.empty((m, hid), dtype=bf, device=dev),
    }
    ws_n = torch.empty(max(R.rmm_rmsnorm_scored_workspace_bytes(m, hid), 256), dtype=torch.uint8, device=dev)
    ws_h = torch.empty(max(R.rmm_swiglu_scored_workspace_bytes(m, mlp), 256), dtype=torch.uint8, device=dev)
    out = {"model": "llama3.1-8b layer", "tokens": m,
           "glue": "torch: K transposed for the attention, residual adds; RoPE left out"}
    for name, scale_one in [("rho", False)] + ([("rho1", True)] if dense else []):
        def kk(l, d):
            return d if scale_one else R.rmm_k_from_rho(l["rho"], d)
        k1, ko, k2, kd = kk(lin["q+k+v"], hid), kk(lin["o"], nq), kk(lin["up+gate"], hid), kk(lin["down"], mlp)
        kf = dh if scale_one else R.rmm_k_from_rho(at["rho"], dh)
        kt = L if scale_one else R.rmm_k_from_rho(at["rho"], L)
        ix = {n: torch.empty(R.rmm_k_pad(k), dtype=torch.int32, device=dev)
              for n, k in (("qkv", k1), ("o", ko), ("ug", k2), ("d", kd))}
        If = torch.empty((Hq, R.rmm_k_pad(kf)), dtype=torch.int32, device=dev)
        It = torch.empty((Hq, R.rmm_k_pad(kt)), dtype=torch.int32, device=dev)
        wsg = torch.empty(max(R.rmm_gemm_workspace_bytes(bf, m, n, k) for n, k in
                              ((nq + 2 * nkv, k1), (hid, ko), (Wug.shape[1], k2), (hid, kd))), dtype=torch.uint8,
                          device=dev)
        wsa = torch.empty(R.rmm_attention_workspace_bytes(m, m, Hq, dh, kf, kt), dtype=torch.uint8, device=dev)
        b = buf
        half = Wug.shape[1] // 2

        class _Layer:
            def step(self, tagged=False):
                s1 = b["s"][:hid]
                R.rmm_rmsnorm_scored(X, w1, 1e-5, Y=b["Xn"], scores=s1, ws=ws_n)
                R.rmm_topk(s1, k1, out=ix["qkv"])
                R.rmm_gemm(b["Xn"], Wqkv, ix["qkv"], k1, out=b["QKV"], ws=wsg)
                Q = b["QKV"][:, :nq].view(m, Hq, dh)
                b["Kt"].copy_(b["QKV"][:, nq:nq + nkv].view(m, Hkv, dh).permute(1, 2, 0))
                V = b["QKV"][:, nq + nkv:].view(m, Hkv, dh)
                R.rmm_attention(Q, b["Kt"], V, kf, kt, O=b["O"], idx_feat=If, idx_tok=It, ws=wsa, causal=True,
                                o_scores=b["os"])
                R.rmm_topk(b["os"], ko, out=ix["o"])
                R.rmm_gemm(b["O"].view(m, nq), Wo, ix["o"], ko, out=b["Yo"], ws=wsg)
                torch.add(X, b["Yo"], out=b["X2"])
                R.rmm_rmsnorm_scored(b["X2"], w2, 1e-5, Y=b["Xn"], scores=s1, ws=ws_n)
                R.rmm_topk(s1, k2, out=ix["ug"])
                R.rmm_gemm(b["Xn"], Wug, ix["ug"], k2, out=b["UG"], ws=wsg)
                R.rmm_swiglu_scored(b["UG"][:, half:], b["UG"][:, :half], H=b["H"], scores=b["s"], ws=ws_h)
                R.rmm_topk(b["s"], kd, out=ix["d"])
                R.rmm_gemm(b["H"], Wd, ix["d"], kd, out=b["Yd"], ws=wsg)
                torch.add(b["X2"], b["Yd"], out=b["X3"])

        ms, _ = time_steps(_Layer(), steps, warmup)
        out[name + "_ms"] = round(ms, 4)
        del ix, If, It, wsg, wsa
        torch.cuda.empty_cache()
    if "rho1_ms" in out:
        out["speedup_vs_rho1"] = round(out["rho1_ms"] / out["rho_ms"], 3)
    return out


def system_info(dev):
    """The device the line was measured on (name, compute units, HIP runtime) and the host's cores."""
    import torch

    p = torch.cuda.get_device_properties(dev)
    return {"gpu": p.name, "arch": getattr(p, "gcnArchName", None), "compute_units": p.multi_processor_count,
            "memory_gib": round(p.total_memory / 2 ** 30, 1), "hip": torch.version.hip,
            "host_cores": os.cpu_count()}


def csrc_sha256():
    import glob
    import hashlib

    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "input_adaptive_reduced_rmm_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode())
        h.update(open(f, "rb").read())
    return h.hexdigest()


def measured_traffic(workload, tag):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE runs, or None
    when they were taken on other kernel sources or another kernel."""
    path = os.path.join(ROOT, "profiles", f"{workload}_traffic.json")
    try:
        t = json.load(open(path))
    except (OSError, ValueError):
        return None
    if t.get("tag") != tag or t.get("csrc_sha256") != csrc_sha256():
        return None
    return int(round(t["read_bytes"] + t["write_bytes"]))


def cpu_baseline(wl, layer_meta):
    """Time the CPU oracle on a bounded sample of the same workload."""
    import numpy as np

    import oracle
    import synth

    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        cores = max(i["num_threads"] for i in blas) if blas else os.cpu_count()
    except Exception:
        cores = os.cpu_count()
    lins = layer_meta["linears"]
    m_s = min(8192, min(l.m for l in lins)) if lins else 0
    parts = []
    flops = 0.0
    t_total = 0.0
    for lin in lins:
        A, B = synth.linear_operands(wl, lin, m=m_s)
        t0 = time.perf_counter()
        oracle.rmm(A, B, lin.rho)
        t_total += time.perf_counter() - t0
        flops += 2.0 * m_s * lin.d * lin.n
    if lins:
        parts.append(f"{len(lins)} projections on the first {m_s} tokens")
    at = layer_meta["attention"]
    if at is not None:
        Ls = min(8192, at.L)
        Q, Kt, V = synth.attention_operands(wl, L=Ls, Hq=1, Hkv=1)
        t0 = time.perf_counter()
        oracle.attention_chain(Q, Kt, V, at.rho)
        t_total += time.perf_counter() - t0
        flops += 2 * 2.0 * Ls * Ls * at.dh
        parts.append(f"reduced attention (QK^T, softmax, PV) of 1 head at {Ls} tokens")
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": "; ".join(parts) + f" (float64 NumPy oracle, {t_total:.1f} s)", "seconds": round(t_total, 2)}


def cpu_ops_table(max_single_s=20.0):
    """The float64 oracle timed per op on this host's cores (median of 3 runs,
    or one run when a run takes longer than `max_single_s`), for the CPU
    baseline table: column scores, top-k and the reduced product of every
    distinct projection shape of the five workloads at their ratios, and per
    attention head the reduced Q K^T (scores, selection and product), the
    causal softmax and the reduced P V (scores, selection and product) -
    attention times are for one head and are multiplied by the head count in
    `total_s`.  Seeded synthetic inputs as the GPU runs use."""
    import numpy as np

    import oracle
    import synth

    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        cores = max(i["num_threads"] for i in blas) if blas else os.cpu_count()
    except Exception:
        cores = os.cpu_count()

    def timed(fn):
        t0 = time.perf_counter()
        out = fn()
        t = time.perf_counter() - t0
        if t > max_single_s:
            return out, t, 1
        ts = [t]
        for _ in range(2):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return out, float(np.median(ts)), 3

    rows = []
    for key in ("xw-fp32-64x512", "llama3.2-1b-proj-2k", "llama3.1-8b-layer-16k", "llama3.1-70b-layer"):
        wl = synth.WORKLOADS[key]
        seen = set()
        for lin in wl.linears:
            shape = (lin.m, lin.d, lin.n, lin.rho, synth.activation_key(wl, lin))
            if shape in seen or lin.name.split("@")[0] in ("k", "v", "gate"):
                continue
            seen.add(shape)
            A, B = synth.linear_operands(wl, lin)
            k = oracle.retained_count(lin.rho, lin.d)
            sc, t_s, n_s = timed(lambda: oracle.column_scores(A))
            I, t_k, n_k = timed(lambda: oracle.select_top(sc, k))
            _, t_g, n_g = timed(lambda: oracle.reduced_product(A, B, I))
            name = lin.name.split("@")[0]
            for op, t, n in (("colnorm", t_s, n_s), ("topk", t_k, n_k), ("gemm", t_g, n_g)):
                rows.append({"workload": key, "product": f"{name} {lin.m}x{lin.d}x{lin.n}", "rho": lin.rho, "op": op,
                             "seconds": round(t, 4), "runs": n, "total_s": round(t, 4)})
            del A, B
            print(f"[cpu-ops] {key} {lin.name} done", file=sys.stderr, flush=True)
    for key in ("attn-32h-4k", "llama3.1-8b-layer-16k", "llama3.1-70b-layer"):
        wl = synth.WORKLOADS[key]
        at = wl.attention
        Q, Kt, V = synth.attention_operands(wl, Hq=1, Hkv=1)
        kf = oracle.retained_count(at.rho, at.dh)
        kt = oracle.retained_count(at.rho, at.L)
        (S, _, _), t_qk, n_qk = timed(lambda: oracle.reduced_qk(Q, Kt, kf))
        P, t_sm, n_sm = timed(lambda: oracle.causal_softmax(S, 1.0 / math.sqrt(at.dh)))
        _, t_pv, n_pv = timed(lambda: oracle.reduced_pv(P, V, kt))
        for op, t, n in (("qk (1 head)", t_qk, n_qk), ("causal softmax (1 head)", t_sm, n_sm),
                         ("pv (1 head)", t_pv, n_pv)):
            rows.append({"workload": key, "product": f"L={at.L} Hq={at.Hq} Hkv={at.Hkv} dh={at.dh}", "rho": at.rho,
                         "op": op, "seconds": round(t, 4), "runs": n, "total_s": round(t * at.Hq, 3)})
        del Q, Kt, V, S, P
        print(f"[cpu-ops] {key} attention done", file=sys.stderr, flush=True)
    return {"cores": int(cores), "host_cores": os.cpu_count(), "rows": rows}


def copy_calibration(dev):
    import torch

    a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()


def summarize(run, kern, dtype):
    """Per-kernel detail of a step, the roofline of its dominant kernel and the
    kept-work MFMA fraction of its projection GEMMs.  The dominant kernel is the
    one with the largest GPU time per step summed over every launch of it (the
    four projections' GEMMs are one kernel); its achieved rate is the algorithmic
    work of those launches over their time, i.e. the average work per launch over
    the average launch time."""
    import torch

    detail = {}
    groups = {}
    for key, v in kern.items():
        bound, amount, unit = algorithmic_work(run, key)
        tot = v["avg_ms"] * v["launches_per_step"]
        ent = {"avg_ms": round(v["avg_ms"], 4), "per_step": v["launches_per_step"]}
        if bound:
            rate = amount / (v["avg_ms"] * 1e-3)
            if unit == "flops":
                peak = PEAK_F32_TFLOPS if dtype == torch.float32 else PEAK_BF16_TFLOPS
                ent["tflops"] = round(rate / 1e12, 1)
                ent["frac"] = round(rate / 1e12 / peak, 4)
            else:
                ent["gbs"] = round(rate / 1e9, 1)
                ent["frac"] = round(rate / 1e9 / PEAK_HBM_GBS, 4)
            tag, name = key.split("/", 1) if "/" in key else ("", key)
            g = groups.setdefault((name, bound, unit), {"ms": 0.0, "amount": 0.0, "launches": 0.0, "tags": []})
            g["ms"] += tot
            g["amount"] += amount * v["launches_per_step"]
            g["launches"] += v["launches_per_step"]
            g["tags"].append(tag)
        detail[key] = ent
    roof = None
    if groups:
        (name, bound, unit), g = max(groups.items(), key=lambda kv: kv[1]["ms"])
        per_launch, avg = g["amount"] / g["launches"], g["ms"] / g["launches"]
        kernel = name if len(g["tags"]) > 1 else f"{g['tags'][0]}/{name}"
        if unit == "flops":
            peak = PEAK_F32_TFLOPS if dtype == torch.float32 else PEAK_BF16_TFLOPS
            ach = per_launch / (avg * 1e-3) / 1e12
            roof = {"bound": bound, "achieved": round(ach, 1), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(ach / peak, 4), "kernel": kernel, "per_launch": f"{per_launch:.4g} flops",
                    "avg_launch_ms": round(avg, 4), "launches_per_step": g["launches"]}
        else:
            ach = per_launch / (avg * 1e-3) / 1e9
            roof = {"bound": bound, "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(ach / PEAK_HBM_GBS, 4), "kernel": kernel, "per_launch": f"{per_launch:.4g} bytes",
                    "avg_launch_ms": round(avg, 4), "launches_per_step": g["launches"]}
        if len(g["tags"]) > 1:
            roof["tags"] = g["tags"]
    g_fl = g_ms = 0.0
    for key, v in kern.items():
        bound, amount, unit = algorithmic_work(run, key)
        if unit == "flops":
            g_fl += amount * v["launches_per_step"]
            g_ms += v["avg_ms"] * v["launches_per_step"]
    peak = PEAK_F32_TFLOPS if dtype == torch.float32 else PEAK_BF16_TFLOPS
    mfma_frac = (g_fl / (g_ms * 1e-3) / 1e12 / peak) if g_ms > 0 else None
    return detail, roof, mfma_frac


def other_workloads(R, dev, steps, warmup):
    """Compact timings of the other synthetic workloads, each at its ratios and at
    rho = 1 (the same pipeline keeping every index): ms per step (mean of `steps`
    back-to-back steps after `warmup`), effective TFLOP/s, speedup, and the
    dominant kernel with its roofline fraction.  Launch-bound shapes (the fp32
    64 x 512 product, the 16-row decode batch) replay the step from a HIP graph."""
    import torch

    import synth

    out = {}
    plans = [
        ("xw-fp32-64x512", [(0.5, None)], True),
        ("llama3.2-1b-proj-2k", [(0.5, None), (0.7, None), (0.8, None)], False),
        ("attn-32h-4k", [(None, None)], False),
        ("llama3.1-70b-layer", [(r, 8192) for r in (0.3, 0.5, 0.7, 0.8, 1.0)] + [(0.5, 16)], None),
    ]
    for key, cases, graph in plans:
        wl = synth.WORKLOADS[key]
        cache = {}
        t0 = time.perf_counter()
        for rho, m in cases:
            lins = list(wl.linears)
            if rho is not None:
                lins = [l for l in lins if abs(l.rho - rho) < 1e-12]
            if m is not None:
                lins = [l for l in lins if l.m == m]
            with_att = wl.attention is not None and (m is None or m == wl.attention.L)
            layer = build_layer_for(wl, lins, dev, False, with_att, cache)
            use_graph = graph if graph is not None else (m is not None and m <= 32)
            run = Runner(R, layer, dev)
            stepper = GraphStep(run) if use_graph else run
            ms, _ = time_steps(stepper, steps, warmup)
            kern = kernel_breakdown(run, max(2, min(steps, 5)))
            _, roof, mfma = summarize(run, kern, layer["dtype"])
            run.free()
            del run, stepper
            all_kept = all(l.rho == 1.0 for l in lins) and (not with_att or wl.attention.rho == 1.0)
            if all_kept:
                ms1 = ms
            else:
                run1 = Runner(R, layer, dev, rho_scale_one=True)
                ms1, _ = time_steps(GraphStep(run1) if use_graph else run1, steps, warmup)
                run1.free()
                del run1
            name = key
            if rho is not None:
                name += f"@rho{rho}"
            if m is not None:
                name += f"@m{m}"
            ent = {"ms": round(ms, 4), "effective_tflops": round(dense_flops(layer) / (ms * 1e-3) / 1e12, 2),
                   "rho1_ms": round(ms1, 4), "speedup_vs_rho1": round(ms1 / ms, 3),
                   "launch": "hip graph replay" if use_graph else "eager"}
            if roof:
                ent["dominant"] = {"kernel": roof["kernel"], "bound": roof["bound"], "frac": roof["frac"]}
            if mfma is not None:
                ent["gemm_kept_mfma_frac"] = round(mfma, 4)
            out[name] = ent
            del layer
            torch.cuda.empty_cache()
        cache.clear()
        torch.cuda.empty_cache()
        print(f"[bench] {key}: {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    return out


def main():
    args = parse()
    if args.cpu_ops:
        print(json.dumps(cpu_ops_table()), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import input_adaptive_reduced_rmm_amd as R
    import synth

    R.load()
    if not torch.cuda.is_available():
        print("no HIP device visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    wl = synth.WORKLOADS[args.workload]
    t_gen = time.perf_counter()
    layer = build_layer(wl, args, dev)
    torch.cuda.synchronize()
    print(f"[bench] inputs ready in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)
    if args.copy_calibration:
        copy_calibration(dev)

    run = Runner(R, layer, dev)
    stepper = GraphStep(run) if args.graph else run
    # Headline: exactly `steps` steps after `warmup`, each with the 256 MB
    # memory-side cache flushed first (untimed), each bracketed by HIP events
    # with a device synchronisation after it; the median step.
    for _ in range(args.warmup):
        stepper.step()
    torch.cuda.synchronize()
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cold = step_distribution(stepper, args.steps, flush)
    ms = cold["median_ms"]
    print(f"[bench] rho step {ms:.3f} ms (cold-cache median of {args.steps})", file=sys.stderr, flush=True)
    hot_ms, wall = time_steps(stepper, args.steps, args.warmup)
    hot = step_distribution(stepper, args.steps)
    hot["mean_ms"] = round(hot_ms, 4)
    del flush, stepper
    kern = kernel_breakdown(run, max(2, min(args.steps, 5)))
    flops = dense_flops(layer)
    detail, roof, mfma_frac = summarize(run, kern, layer["dtype"])
    if roof:
        roof["traffic"] = measured_traffic(wl.key, roof["kernel"])
    # the step's own Q K^T and P V (P an input), for comparison with the fused call
    qkpv_ms = sum(v["avg_ms"] * v["launches_per_step"] for k, v in kern.items() if k.split("/")[0] in ("qk", "pv"))
    proj_ms = sum(v["avg_ms"] * v["launches_per_step"] for k, v in kern.items()
                  if k.split("/")[0] not in ("qk", "pv"))
    torch_proj_ms = torch_matmul_context(layer, args.steps, args.warmup) if layer["linears"] else None
    run.free()
    del run
    torch.cuda.empty_cache()

    fused = None
    if layer["attention"] is not None and not args.no_fused_attention:
        fused = fused_attention(R, layer, args.steps, args.warmup, dense=not args.no_dense)
        fused["step_qk_pv_ms"] = round(qkpv_ms, 4)
        print(f"[bench] fused attention {fused['rho']['ms']:.3f} ms", file=sys.stderr, flush=True)

    producers = None
    if not args.no_producers:
        producers = producer_fused(R, wl, args, args.steps, args.warmup, dev)
    layer_fused = None
    if not args.no_fused_attention and not args.no_producers:
        layer_fused = fused_layer(R, layer, args.steps, args.warmup, dense=not args.no_dense)
        if layer_fused:
            print(f"[bench] fused layer {layer_fused['rho_ms']:.3f} ms", file=sys.stderr, flush=True)

    speedup = dense_ms = None
    if not args.no_dense:
        run1 = Runner(R, layer, dev, rho_scale_one=True)
        st1 = GraphStep(run1) if args.graph else run1
        for _ in range(args.warmup):
            st1.step()
        torch.cuda.synchronize()
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dense_ms = step_distribution(st1, args.steps, flush)["median_ms"]
        speedup = dense_ms / ms
        print(f"[bench] rho=1 step {dense_ms:.3f} ms", file=sys.stderr, flush=True)
        del flush, st1
        run1.free()
        del run1
        torch.cuda.empty_cache()
    del layer
    torch.cuda.empty_cache()

    others = None
    if not args.no_other_workloads and args.workload == DEFAULT_WORKLOAD:
        others = other_workloads(R, dev, args.steps, args.warmup)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, {"linears": [l for l in wl.linears if l in _selected(wl, args)],
                                "attention": wl.attention if _has_attention(wl, args) else None})

    value = flops / (ms * 1e-3) / 1e12
    cfg = {"workload": wl.key, "dtype": wl.dtype, "rho": _rho_desc(wl, args),
           "products": _products_desc(wl, args), "launch": "hip graph replay" if args.graph else "eager",
           "timing": "median step, memory-side cache flushed before each step"}
    out = {
        "metric": "effective TFLOP/s (dense-equivalent flops / RMM step time)",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32", "data": "synthetic (seeded; shapes and value "
        "distributions of the pages' model families)", "config": cfg,
        "speedup_vs_rho1": round(speedup, 3) if speedup else None,
        "rho1_ms_per_step": round(dense_ms, 4) if dense_ms else None,
        "gemm_kept_mfma_frac": round(mfma_frac, 4) if mfma_frac is not None else None,
        "roofline": roof, "cpu_baseline": cpu, "kernels": detail, "fused_attention": fused,
        "producer_fused": producers, "fused_layer": layer_fused,
        "step_times": {"hot": hot, "cold_cache": cold},
        "workloads": others,
        "system": system_info(dev),
        "context": {"rmm_projections_ms": round(proj_ms, 4), "torch_matmul_projections_ms": torch_proj_ms},
    }
    print(json.dumps(out), flush=True)


def _selected(wl, args):
    lins = list(wl.linears)
    if wl.key == "llama3.1-70b-layer":
        m = args.m if args.m is not None else 8192
        rho = args.rho if args.rho is not None else 0.5
        return [l for l in lins if l.m == m and abs(l.rho - rho) < 1e-12]
    if args.rho is not None:
        return [l for l in lins if abs(l.rho - args.rho) < 1e-12]
    if wl.key == "llama3.2-1b-proj-2k":
        return [l for l in lins if l.rho == 0.5]
    return lins


def _has_attention(wl, args):
    return wl.attention is not None and (wl.key != "llama3.1-70b-layer" or args.m in (None, 8192))


def _rho_desc(wl, args):
    rs = sorted({l.rho for l in _selected(wl, args)})
    d = {"projections": rs}
    if _has_attention(wl, args):
        d["attention"] = wl.attention.rho
    return d


def _products_desc(wl, args):
    import synth

    groups = []
    for l in _selected(wl, args):
        key = (synth.activation_key(wl, l), l.rho)
        g = None if args.no_fuse else next((g for g in groups if g["key"] == key), None)
        if g is None:
            groups.append({"key": key, "names": [l.name.split("@")[0]], "m": l.m, "d": l.d, "n": l.n})
        else:
            g["names"].append(l.name.split("@")[0])
            g["n"] += l.n
    out = [f"{'|'.join(g['names'])} {g['m']}x{g['d']}x{g['n']}" for g in groups]
    if _has_attention(wl, args):
        at = wl.attention
        out.append(f"QK^T+PV L={at.L} Hq={at.Hq} Hkv={at.Hkv} dh={at.dh}")
    return out


if __name__ == "__main__":
    main()
