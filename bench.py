"""Benchmark: one training step of a stack of pre-norm decoder blocks
(forward + backward of every layer, inputs resident in HBM) on one MI355X.

Default workload: the Llama-style GQA stack -- 4 layers, B=8, T=2048, C=2048,
NH=32, NKV=8, head 64, SwiGLU H=5632, RMSNorm gamma, NeoX RoPE base 1e4, bf16
storage / fp32 accumulation, seeded N(0, 0.02) weights, x_in = embedding rows
of seeded uniform token ids, seeded N(0, 1) upstream gradient.

Prints ONE JSON line.  value = tokens/s per block = B*T*L / (time of one
forward+backward of the L-block stack).  The roofline object reports the
dominant kernel class (the MFMA GEMMs) from HIP events recorded around every
launch on its stream during the timed region; cpu_baseline times the oracle
(plain fp64 C) on a bounded sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"bf16": 2500.0, "f32": 157.3}   # dense MFMA TFLOP/s (MI355X datasheet)
HBM_PEAK = 8000.0                        # GB/s
# the bf16 forward-projection GEMM: one main loop, two epilogues (MODE 0: bias /
# residual / RoPE for QKV, O and down; MODE 5: SwiGLU for the MLP up projection)
GEMM_FWD_KERNEL = "gemm_k64m16_kernel<0|5>"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_fwd_llama_gqa_traffic.md")
GEMM_SOURCES = [os.path.join(ROOT, "decoder_only_transformer_block_amd", "csrc", f) for f in ("gemm.hip", "common.h")]


def gemm_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str):
    """HBM bytes per launch of the forward-projection GEMM from the committed
    counter summary, or None when it is missing or was taken on other kernel
    sources or another workload."""
    import re
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if not m:
        return None
    d = json.loads(m.group(1))
    if d.get("source_hash") != gemm_source_hash() or d.get("workload") != workload:
        return None
    return d


def traffic_summary(root: str, cmds: dict) -> str:
    """Markdown summary of four rocprofv3 --pmc runs under root/{fetch,write,copy_fetch,copy_write}:
    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the forward-projection GEMM
    dispatches, each scaled by the ratio of known bytes to what the same counter
    reads for a plain copy of known size."""
    import glob
    import sqlite3

    def per_dispatch(sub, counter, match):
        vals = {}
        for db in glob.glob(os.path.join(root, sub, "**", "*.db"), recursive=True):
            c = sqlite3.connect(db)
            for name, disp, v in c.execute("select kernel_name, dispatch_id, value from counters_collection "
                                           "where counter_name = ?", (counter,)):
                if match(name):
                    vals[disp] = vals.get(disp, 0.0) + v
        return vals

    is_gemm = lambda n: any(k in n for k in ("gemm_k64m16_kernel<0>", "gemm_k64m16_kernel<5>",
                                             "gemm_k64m16_kernelILi0E", "gemm_k64m16_kernelILi5E"))
    is_copy = lambda n: "copy" in n.lower()
    f = per_dispatch("fetch", "FETCH_SIZE", is_gemm)
    w = per_dispatch("write", "WRITE_SIZE", is_gemm)
    cf = per_dispatch("copy_fetch", "FETCH_SIZE", is_copy)
    cw = per_dispatch("copy_write", "WRITE_SIZE", is_copy)
    known = cmds["copy_bytes"]
    fs = known / (1024.0 * max(cf.values()))
    ws = known / (1024.0 * max(cw.values()))
    fk = sum(f.values()) / len(f)
    wk = sum(w.values()) / len(w)
    traffic = (fk * fs + wk * ws) * 1024.0
    d = {"workload": cmds["workload"], "kernel": GEMM_FWD_KERNEL, "source_hash": gemm_source_hash(),
         "dispatches": len(f), "fetch_kib_per_dispatch": round(fk, 1), "write_kib_per_dispatch": round(wk, 1),
         "copy_fetch_kib": round(max(cf.values()), 1), "copy_write_kib": round(max(cw.values()), 1),
         "copy_bytes": known, "fetch_scale": round(fs, 4), "write_scale": round(ws, 4),
         "traffic_bytes_per_launch": round(traffic)}
    lines = ["# HBM traffic of the forward-projection GEMM (%s, Llama-GQA 4-layer stack)" % GEMM_FWD_KERNEL, "",
             "Counter runs (from the repository root on an MI355X, one counter per run):", "", "```"]
    lines += cmds["commands"] + ["```", "",
              "FETCH_SIZE / WRITE_SIZE are read in KiB per dispatch and averaged over the kernel's dispatches "
              "(QKV, O, MLP up and MLP down projections of every layer).  Each is scaled by known bytes / "
              "counter reading of the plain copy kernel in the copy-probe run.  `source_hash` is the SHA-256 "
              "prefix of gemm.hip + common.h when the counters were taken; bench.py reports the traffic only "
              "while the sources still match.", "", "```json", json.dumps(d), "```", ""]
    return "\n".join(lines)


COUNTER_PASSES = {
    "a": "SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_SALU SQ_INSTS_LDS SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES "
         "SQ_WAVE_CYCLES SQ_ACTIVE_INST_VALU GRBM_GUI_ACTIVE",
    "b": "SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_WAIT_INST_LDS SQ_WAIT_INST_ANY "
         "SQ_ACTIVE_INST_LDS GRBM_GUI_ACTIVE",
}
COUNTER_KERNELS = [("attention forward", "fwd_bf16_kernel"), ("attention backward dQ", "dq_bf16_kernel"),
                   ("attention backward dK/dV", "dkv_bf16_kernel"), ("GEMM forward", "gemm_k64m16_kernel"),
                   ("GEMM input gradient", "gemm_k64_kernel"), ("GEMM weight gradient", "gemm_dma_kernel"),
                   ("norm forward", "norm_fwd_kernel"), ("norm backward", "norm_bwd_kernel"),
                   ("activation backward", "act_bwd_kernel")]


def counter_summary(root: str, cmds: list) -> str:
    """Markdown table of the instruction counters of two rocprofv3 --pmc runs
    (root/a, root/b: COUNTER_PASSES) per kernel family, per dispatch."""
    import glob
    import sqlite3
    tot = {}  # family -> counter -> [sum, dispatches]
    for sub in COUNTER_PASSES:
        seen = {}
        for db in glob.glob(os.path.join(root, sub, "**", "*.db"), recursive=True):
            c = sqlite3.connect(db)
            for name, disp, ctr, v in c.execute("select kernel_name, dispatch_id, counter_name, value "
                                                "from counters_collection"):
                fam = next((f for f, key in COUNTER_KERNELS if key in name), None)
                if fam is None:
                    continue
                t = tot.setdefault(fam, {}).setdefault(ctr, [0.0, set()])
                t[0] += v
                t[1].add((sub, disp))
    lines = ["# Instruction counters per kernel family (Llama-GQA 4-layer stack, bf16)", "",
             "Two counter runs over the same bench command (one kernel at a time: `--no-overlap`), from the "
             "repository root on an MI355X:", "", "```"] + cmds + ["```", "",
             "Per dispatch, averaged over the family's dispatches.  `VALU instr`: SQ_INSTS_VALU, which counts "
             "the MFMA instructions too; `other VALU / MFMA`: (SQ_INSTS_VALU - SQ_INSTS_MFMA) / SQ_INSTS_MFMA; "
             "`SALU`, `LDS`: SQ_INSTS_SALU, SQ_INSTS_LDS per MFMA instruction.  `MFMA busy`: SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 1024 SIMDs), "
             "the fraction of the kernel's active cycles in which a SIMD's matrix unit is busy.  `VALU active`: "
             "SQ_ACTIVE_INST_VALU / SQ_WAVE_CYCLES, the share of a wave's cycles spent issuing VALU work.  "
             "`MFMA TFLOP per dispatch`: 512 x SQ_INSTS_VALU_MFMA_MOPS_BF16, the matrix work one launch "
             "executed (recomputed products and padding included).  `LDS conflict`: SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE.", "",
             "| kernel family | dispatches | MFMA instr | VALU instr | other VALU / MFMA | SALU / MFMA | "
             "LDS / MFMA | MFMA busy | VALU active | MFMA TFLOP per dispatch | LDS conflict |",
             "|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
    out = {}
    for fam, _ in COUNTER_KERNELS:
        t = tot.get(fam)
        if not t:
            continue
        avg = {k: v[0] / max(len(v[1]), 1) for k, v in t.items()}
        g = lambda k: avg.get(k, 0.0)
        n = len(t.get("SQ_INSTS_MFMA", [0, set()])[1])
        mf = g("SQ_INSTS_MFMA")
        busy = g("SQ_VALU_MFMA_BUSY_CYCLES") / max(g("GRBM_GUI_ACTIVE") / 8 * 1024, 1.0)
        per = lambda k: g(k) / mf if mf > 0 else None
        row = {"dispatches": n, "mfma": mf, "valu": g("SQ_INSTS_VALU"),
               "other_valu_per_mfma": (g("SQ_INSTS_VALU") - mf) / mf if mf > 0 else None,
               "salu_per_mfma": per("SQ_INSTS_SALU"), "lds_per_mfma": per("SQ_INSTS_LDS"),
               "mfma_busy": busy, "valu_active": g("SQ_ACTIVE_INST_VALU") / max(g("SQ_WAVE_CYCLES"), 1.0),
               "mfma_tflop": 512 * g("SQ_INSTS_VALU_MFMA_MOPS_BF16") / 1e12,
               "lds_conflict": g("SQ_LDS_BANK_CONFLICT") / max(g("SQ_LDS_IDX_ACTIVE"), 1.0)}
        out[fam] = {k: (round(v, 4) if v is not None else None) for k, v in row.items()}
        f2 = lambda v: "—" if v is None else f"{v:.2f}"
        lines.append(f"| {fam} | {n} | {mf:.4g} | {row['valu']:.4g} | {f2(row['other_valu_per_mfma'])} | "
                     f"{f2(row['salu_per_mfma'])} | {f2(row['lds_per_mfma'])} | {busy:.3f} | "
                     f"{row['valu_active']:.3f} | {row['mfma_tflop']:.4f} | {row['lds_conflict']:.3f} |")
    lines += ["", "```json", json.dumps(out), "```", ""]
    return "\n".join(lines)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama_gqa",
                    choices=["llama_gqa", "gpt2_small", "mini_qwen2", "microgpt", "attn_long", "adamw",
                             "head_ce", "decode", "mtp_head", "hbm_cold", "oracle_table"])
    ap.add_argument("--no-overlap", action="store_true",
                    help="block backward on one stream (block_backward): no weight-gradient GEMM runs beside "
                         "another kernel, so per-kernel profiles isolate them")
    ap.add_argument("--attn-long-tokens", type=int, default=4096,
                    help="oracle_table: sequence length of the long-context attention sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-layout", choices=["position", "head"], default="position",
                    help="decode workload: position-major caches [B][Tmax][NKV*hd] (attn_decode) or head-major "
                         "[B][NKV][Tmax][hd] (attn_decode_strided)")
    ap.add_argument("--no-timing", action="store_true", help="skip the per-kernel HIP events")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB three times (the known-size "
                         "reference kernel that scales the FETCH_SIZE / WRITE_SIZE counters) and exit")
    ap.add_argument("--traffic-summary", default="",
                    help="only write the forward-GEMM traffic summary from the rocprofv3 runs under this "
                         "directory (subdirectories fetch, write, copy_fetch, copy_write) and exit")
    ap.add_argument("--counter-summary", default="",
                    help="only write the per-kernel instruction-counter summary from the two rocprofv3 runs "
                         "under this directory (subdirectories a and b) and exit")
    ap.add_argument("--cpu-tokens", type=int, default=0,
                    help="tokens of the oracle's bounded sample (one sequence, one layer); 0: the workload's T")
    return ap.parse_args()


def cpu_baseline(cfg, tokens):
    import numpy as np
    import oracle
    from decoder_only_transformer_block_amd import configs
    oracle.build(force=False)
    sub = cfg.replace(L=1, B=1, T=tokens)
    w = configs.block_weights(sub, 0)
    x = configs.block_input(sub)
    dy = configs.block_dout(sub)
    t0 = time.perf_counter()
    y, sv = oracle.block_forward(sub, w, x)
    oracle.block_backward(sub, w, x, sv, dy)
    dt = time.perf_counter() - t0
    return {"value": round(tokens / dt, 3), "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"one {cfg.name} block (C={cfg.C}, NH={cfg.NH}, NKV={cfg.NKV}, H={cfg.H}) forward+backward "
                      f"on B=1, T={tokens} in fp64, {dt:.2f} s"}


def cpu_baseline_attn(cfg, tokens):
    import oracle
    from decoder_only_transformer_block_amd import configs
    oracle.build(force=False)
    sub = cfg.replace(T=tokens)
    qkv, dout = configs.attn_inputs(sub)
    t0 = time.perf_counter()
    oracle.attn_forward(qkv, sub.B, sub.T, sub.C, sub.NH, sub.NKV)
    oracle.attn_backward(qkv, dout, sub.B, sub.T, sub.C, sub.NH, sub.NKV)
    dt = time.perf_counter() - t0
    return {"value": round(tokens / dt, 3), "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"attention forward+backward B=1, T={tokens}, NH={cfg.NH}, NKV={cfg.NKV}, hd={cfg.hd} "
                      f"in fp64, {dt:.2f} s"}


def oracle_table(args):
    """The oracle timed on the host cores, per configuration: the whole block
    stack forward + backward (microgpt, mini-Qwen2, GPT-2-small) on every
    thread and on one thread (GPT-2-small on one thread: one of its twelve
    layers), one Llama-GQA block on one sequence at the full T = 2048, and
    long-context attention forward + backward at --attn-long-tokens.  Progress
    lines go to stderr; a markdown table and one JSON line to stdout."""
    import numpy as np
    import oracle
    from decoder_only_transformer_block_amd import configs
    oracle.build(force=False)
    allt = oracle.num_threads()
    rows = []

    def log(msg):
        print(msg, file=sys.stderr, flush=True)

    def stack(cfg, layers, threads):
        oracle.set_num_threads(threads)
        x = configs.block_input(cfg)
        dy = configs.block_dout(cfg)
        ws = [configs.block_weights(cfg, l) for l in range(layers)]
        t0 = time.perf_counter()
        h, saved, xs = x, [], []
        for l in range(layers):
            xs.append(h)
            h, sv = oracle.block_forward(cfg, ws[l], h)
            saved.append(sv)
            log(f"  {cfg.name}: layer {l} forward done ({time.perf_counter() - t0:.1f} s, {threads} threads)")
        g = dy
        for l in reversed(range(layers)):
            g, _ = oracle.block_backward(cfg, ws[l], xs[l], saved[l], g)
            log(f"  {cfg.name}: layer {l} backward done ({time.perf_counter() - t0:.1f} s, {threads} threads)")
        return time.perf_counter() - t0

    for name in ("microgpt", "mini_qwen2", "gpt2_small"):
        cfg = configs.BLOCK_CONFIGS[name]
        tok = cfg.B * cfg.T
        for threads in (allt, 1):
            layers = cfg.L if (threads == allt or cfg.L <= 2) else 1
            dt = stack(cfg, layers, threads)
            rows.append({"config": name, "shape": f"L={layers} B={cfg.B} T={cfg.T}", "threads": threads,
                         "seconds": round(dt, 3), "tokens_per_s_per_block": round(tok * layers / dt, 2),
                         "gflop": round((cfg.gemm_flops_per_layer() + cfg.attn_flops_per_layer()) * layers / 1e9, 4)})
            log(json.dumps(rows[-1]))
    cfg = configs.LLAMA_GQA.replace(B=1, L=1)
    dt = stack(cfg, 1, allt)
    rows.append({"config": "llama_gqa", "shape": f"L=1 B=1 T={cfg.T} (one of the B=8 sequences of one layer)",
                 "threads": allt, "seconds": round(dt, 3), "tokens_per_s_per_block": round(cfg.T / dt, 2),
                 "gflop": round((cfg.gemm_flops_per_layer() + cfg.attn_flops_per_layer()) / 1e9, 4)})
    log(json.dumps(rows[-1]))
    oracle.set_num_threads(allt)
    cfg = configs.ATTN_LONG.replace(T=args.attn_long_tokens)
    qkv, dout = configs.attn_inputs(cfg)
    t0 = time.perf_counter()
    oracle.attn_forward(qkv, cfg.B, cfg.T, cfg.C, cfg.NH, cfg.NKV)
    log(f"  attn_long T={cfg.T}: forward done ({time.perf_counter() - t0:.1f} s)")
    oracle.attn_backward(qkv, dout, cfg.B, cfg.T, cfg.C, cfg.NH, cfg.NKV)
    dt = time.perf_counter() - t0
    rows.append({"config": "attn_long", "shape": f"B=1 T={cfg.T} NH=32 NKV=8 hd=128 (attention forward+backward)",
                 "threads": allt, "seconds": round(dt, 3), "tokens_per_s_per_block": round(cfg.T / dt, 2),
                 "gflop": round(cfg.fwd_flops() * 3.5 / 1e9, 4)})
    log(json.dumps(rows[-1]))
    print("| config | oracle run | threads | seconds | tokens/s per block | GFLOP |")
    print("|---|---|---:|---:|---:|---:|")
    for r in rows:
        print(f"| {r['config']} | {r['shape']} | {r['threads']} | {r['seconds']} | {r['tokens_per_s_per_block']} | "
              f"{r['gflop']} |")
    print(json.dumps({"oracle_table": rows, "host_threads": allt}))


def bench_hbm_cold(args):
    """The bandwidth-bound kernels of the Llama-GQA layer (RMSNorm forward and
    backward with the residual gradient, the SwiGLU forward and backward) and
    of the GPT-2-small layer (LayerNorm forward and backward, GELU forward and
    backward, the bias gradient), each launched alone through the C ABI on its
    full-size tensors: hot (the same buffers every launch, so what fits stays
    in the 256 MB last-level cache) and cold (launches rotate over buffer sets
    of more than 1.5 GB in all, so every launch reads tensors that left the
    cache).  GB/s from the algorithmic bytes the library records per launch
    and the HIP events on each kernel."""
    import torch
    from decoder_only_transformer_block_amd import binding, configs
    out = []
    for cname in ("llama_gqa", "gpt2_small"):
        cfg = configs.BLOCK_CONFIGS[cname]
        R, C, H, dt = cfg.B * cfg.T, cfg.C, cfg.H, cfg.dtype
        td = torch.bfloat16 if dt == "bf16" else torch.float32
        es = 2 if dt == "bf16" else 4
        W = 2 * H if cfg.mlp == "swiglu" else H
        norm, mlp = cfg.norm, cfg.mlp
        g = torch.Generator(device="cuda").manual_seed(7)

        def rnd(*shape):
            return torch.randn(*shape, device="cuda", generator=g).to(td)

        gam, bet = rnd(C), rnd(C)
        nws = torch.empty(binding.norm_workspace_bytes(R, C), dtype=torch.uint8, device="cuda")
        lws = torch.empty(binding.linear_workspace_bytes(R, 8, W, dt), dtype=torch.uint8, device="cuda")
        kernels = {
            "norm_forward": (lambda b: binding.norm_forward(b["o"], b["rs"], b["mu"], b["x"], gam, bet, R, C, norm,
                                                            1e-5, dt), ("x", "o"), C),
            "norm_backward (+ residual)": (
                lambda b: binding.norm_backward(b["o"], b["dg"], b["db"], b["dy"], b["x"], gam, b["rs"], b["mu"],
                                                b["r"], R, C, norm, dt, nws), ("x", "o", "dy", "r"), C),
            f"{mlp} forward": (lambda b: binding.activation_forward(b["h"], b["up"], R, H, mlp, dt), ("up", "h"), 0),
            f"{mlp} backward": (lambda b: binding.activation_backward(b["dup"], b["h"], b["up"], R, H, mlp, dt),
                                ("up", "h", "dup"), 0),
        }
        if cfg.mlp_bias:
            kernels["bias gradient (MLP up)"] = (
                lambda b: binding.linear_backward(None, None, b["db2"], b["up"], None, None, R, 8, W, dt, lws),
                ("up",), 0)
        shapes = {"x": (R, C), "o": (R, C), "dy": (R, C), "r": (R, C), "up": (R, W), "h": (R, H), "dup": (R, W)}
        for kname, (fn, used, _) in kernels.items():
            set_elems = sum(R * shapes[u][1] for u in used)
            nsets = max(2, -(-int(1.6e9) // (set_elems * es)))
            # every set is a view of one allocation (one contiguous range of
            # device memory), filled with N(0, 1) values
            flat = torch.empty(nsets * set_elems, dtype=td, device="cuda")
            for i in range(nsets):
                flat[i * set_elems:(i + 1) * set_elems].copy_(
                    torch.randn(set_elems, device="cuda", generator=g))
            sets = []
            for i in range(nsets):
                b, off = {}, i * set_elems
                for u in used:
                    n = R * shapes[u][1]
                    b[u] = flat[off:off + n].view(*shapes[u])
                    off += n
                b.update(rs=torch.rand(R, device="cuda", generator=g) + 0.5,
                         mu=torch.zeros(R, device="cuda"), dg=torch.zeros(C, device="cuda"),
                         db=torch.zeros(C, device="cuda"), db2=torch.zeros(W, device="cuda"))
                if "o" not in b:
                    b["o"] = None
                sets.append(b)
            res = {}
            for mode in ("hot", "cold"):
                for i in range(3):
                    fn(sets[0] if mode == "hot" else sets[i % nsets])
                torch.cuda.synchronize()
                binding.timing_enable(classes=["elementwise"])
                binding.timing_collect()
                n = 4 * nsets if mode == "cold" else 20
                for i in range(n):
                    fn(sets[0] if mode == "hot" else sets[(i + 3) % nsets])
                t = binding.timing_collect()["elementwise"]
                binding.timing_enable(False)
                gbps = t["bytes"] / (t["ms"] * 1e-3) / 1e9
                res[mode] = {"gbps": round(gbps, 1), "frac_hbm_peak": round(gbps / HBM_PEAK, 4),
                             "us_per_launch": round(t["ms"] * 1e3 / t["launches"], 2)}
            row = {"workload": cname, "kernel": kname, "dtype": dt,
                   "bytes_per_launch": round(t["bytes"] / t["launches"]), "buffer_sets": nsets, **res}
            out.append(row)
            print(json.dumps(row), file=sys.stderr, flush=True)
            del sets, flat
            torch.cuda.empty_cache()
    return out


def timed_steps(args, step, roof_classes):
    """Time args.steps steps.  Inside the timed region only the roofline
    kernel's class carries HIP events (on the kernels' own dispatch packets);
    a second, untimed pass of the same steps with every class enabled gives
    the per-class breakdown (the library then runs the block backward on one
    stream, so the classes' times do not overlap).  Returns (seconds, timings), where timings maps
    each class to its event totals and the roofline classes' entries come
    from the timed region."""
    import torch
    from decoder_only_transformer_block_amd import binding
    torch.cuda.synchronize()
    if not args.no_timing:
        binding.timing_enable(classes=roof_classes)
        binding.timing_collect()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    ev[0].record()
    for i in range(args.steps):
        step()
        ev[i + 1].record()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    # per-step GPU times between the events at the step boundaries (on the
    # stream the steps are issued to): their median next to the mean above
    per_step = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
    args.step_median_ms = per_step[len(per_step) // 2] if len(per_step) % 2 else \
        0.5 * (per_step[len(per_step) // 2 - 1] + per_step[len(per_step) // 2])
    tim = {}
    if not args.no_timing:
        roof = binding.timing_collect()
        binding.timing_enable(True)
        for _ in range(args.steps):
            step()
        tim = binding.timing_collect()
        binding.timing_enable(False)
        for c in roof_classes:
            tim[c] = roof[c]
    return dt, tim


def bench_block(args, cfg):
    import torch
    from decoder_only_transformer_block_amd import binding, configs
    from decoder_only_transformer_block_amd.runtime import BlockStack, to_device

    ws = [configs.block_weights(cfg, l) for l in range(cfg.L)]
    x = to_device(configs.block_input(cfg), cfg.dtype)
    dy = to_device(configs.block_dout(cfg), cfg.dtype)
    st = BlockStack(cfg, ws, overlap=not args.no_overlap)
    del ws

    def step():
        st.forward(x)
        st.backward(dy)

    for _ in range(args.warmup):
        step()
    dt, tim = timed_steps(args, step, ["gemm_fwd"])
    ms = dt * 1e3 / args.steps
    tokens = cfg.B * cfg.T
    value = tokens * cfg.L / (dt / args.steps)
    return ms, value, tim


def bench_attn(args, cfg):
    import torch
    from decoder_only_transformer_block_amd import binding, configs
    from decoder_only_transformer_block_amd.runtime import to_device
    qkv_np, dout_np = configs.attn_inputs(cfg)
    q, d = to_device(qkv_np, cfg.dtype), to_device(dout_np, cfg.dtype)
    del qkv_np, dout_np
    B, T, C = cfg.B, cfg.T, cfg.C
    out = torch.empty((B, T, C), dtype=q.dtype, device="cuda")
    lse = torch.empty((B, cfg.NH, T), dtype=torch.float32, device="cuda")
    dq = torch.empty_like(q)
    wsb = torch.empty(binding.attn_workspace_bytes(B, T, cfg.NH), dtype=torch.uint8, device="cuda")

    def step():
        binding.attn_forward(out, lse, q, B, T, C, cfg.NH, cfg.NKV, cfg.dtype)
        binding.attn_backward(dq, q, out, d, lse, B, T, C, cfg.NH, cfg.NKV, cfg.dtype, wsb)

    for _ in range(args.warmup):
        step()
    dt, tim = timed_steps(args, step, ["attn_bwd"])
    return dt * 1e3 / args.steps, B * T / (dt / args.steps), tim


def bench_adamw(args):
    """One AdamW step over every parameter of the Llama-GQA model (4 blocks,
    token table and untied head: fp32 master values, moments and gradients,
    the bf16 storage copy refreshed and the gradient cleared) as one launch."""
    import numpy as np
    import torch
    from decoder_only_transformer_block_amd import binding, configs
    cfg = configs.LLAMA_GQA
    per_layer = sum(int(np.prod(s)) for s in configs.weight_shapes(cfg).values())
    n = cfg.L * per_layer + 2 * cfg.vocab * cfg.C
    g = torch.Generator(device="cuda").manual_seed(3)
    p = torch.randn(n, device="cuda", generator=g) * 0.02
    m = torch.zeros(n, device="cuda")
    v = torch.zeros(n, device="cuda")
    grads = torch.randn(n, device="cuda", generator=g) * 1e-3
    lowp = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    step = [0]

    def one():
        step[0] += 1
        binding.adamw_update(p, grads, m, v, lowp, n, 3e-4, 0.9, 0.95, 1e-8, 0.1, step[0], "bf16", False)

    for _ in range(args.warmup):
        one()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        one()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    nbytes = n * 30.0  # read p, g, m, v; write p, m, v; write the bf16 copy
    return dt * 1e3, n, nbytes


def bench_head_ce(args):
    """The Llama-GQA LM head + cross-entropy forward and backward (R = 16384
    positions, C = 2048, V = 32000, bf16): the fused vocabulary-chunked path
    (lm_head_ce, 4096-row chunks) and, for context, the unfused one."""
    import torch
    from decoder_only_transformer_block_amd import binding, configs
    cfg = configs.LLAMA_GQA
    R, C, V = cfg.B * cfg.T, cfg.C, cfg.vocab
    g = torch.Generator(device="cuda").manual_seed(4)
    inp = torch.randn(R, C, device="cuda", generator=g).bfloat16()
    w = (torch.randn(V, C, device="cuda", generator=g) * 0.02).bfloat16()
    tgt = torch.randint(0, V, (R,), device="cuda", generator=g, dtype=torch.int32)
    loss = torch.empty(1, device="cuda")
    rows = torch.empty(R, device="cuda")
    dinp = torch.empty(R, C, device="cuda", dtype=torch.bfloat16)
    dw = torch.zeros(V, C, device="cuda")
    ws = torch.empty(binding.lm_head_ce_workspace_bytes(R, C, V, 4096, "bf16"), dtype=torch.uint8, device="cuda")
    ldl = (V + 7) // 8 * 8
    logits = torch.empty(R, ldl, device="cuda", dtype=torch.bfloat16)
    ws2 = torch.empty(binding.lm_head_workspace_bytes(R, C, V, "bf16"), dtype=torch.uint8, device="cuda")

    def fused():
        binding.lm_head_ce(loss, rows, dinp, dw, inp, w, tgt, R, C, V, 4096, 1.0 / R, "bf16", ws)

    def unfused():
        binding.lm_head_forward(logits, ldl, inp, w, R, C, V, "bf16")
        binding.softmax_ce(loss, rows, logits, logits, ldl, tgt, R, V, 1.0 / R, "bf16")
        binding.lm_head_backward(dinp, dw, logits, ldl, inp, w, R, C, V, "bf16", ws2)

    out = {}
    for name, fn in (("fused", fused), ("unfused", unfused)):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        out[name] = (time.perf_counter() - t0) / args.steps * 1e3
    return out, R, C, V, ws.numel(), logits.numel() * 2


def bench_mtp_head(args, K=4):
    """Four prediction heads on the Llama-GQA head (R = 16384 positions,
    C = 2048, V = 32000 per head, bf16) through the fused, vocabulary-chunked
    head + cross-entropy (4096-row chunks): loss, dinp and the head gradient."""
    import torch
    from decoder_only_transformer_block_amd import binding, configs
    cfg = configs.LLAMA_GQA
    R, C, V = cfg.B * cfg.T, cfg.C, cfg.vocab
    g = torch.Generator(device="cuda").manual_seed(5)
    inp = torch.randn(R, C, device="cuda", generator=g).bfloat16()
    w = (torch.randn(K * V, C, device="cuda", generator=g) * 0.02).bfloat16()
    tgt = torch.randint(0, V, (R, K), device="cuda", generator=g, dtype=torch.int32)
    loss = torch.empty(1, device="cuda")
    rows = torch.empty(R * K, device="cuda")
    dinp = torch.empty(R, C, device="cuda", dtype=torch.bfloat16)
    dw = torch.zeros(K * V, C, device="cuda")
    ws = torch.empty(binding.lm_head_ce_workspace_bytes(R, C, V, 4096, "bf16"), dtype=torch.uint8, device="cuda")

    def one():
        binding.lm_head_mtp_ce(loss, rows, dinp, dw, inp, w, tgt, R, C, V, K, 4096, 1.0 / (R * K), "bf16", ws)

    for _ in range(args.warmup):
        one()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        one()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / args.steps * 1e3, R, C, V, K, ws.numel()


def bench_decode(args):
    """Decode attention over the Llama-GQA heads: 256 sequences, cache lengths
    uniform in [1, 4096] (capacity 4096), one new query per sequence, bf16.
    The caches stay resident; a step is one attn_decode call (the chunked
    attention kernel and its merge), or with --decode-layout head one
    attn_decode_strided call on head-major caches holding the same values."""
    import numpy as np
    import torch
    from decoder_only_transformer_block_amd import binding, configs
    from decoder_only_transformer_block_amd.runtime import DecodeAttention, to_device
    cfg = configs.DECODE_LLAMA_GQA
    q, kc, vc, lens = configs.decode_inputs(cfg)
    dq, dk, dv = to_device(q, cfg.dtype), to_device(kc, cfg.dtype), to_device(vc, cfg.dtype)
    if args.decode_layout == "head":   # [B][Tmax][NKV][hd] -> [B][NKV][Tmax][hd]
        shape = (cfg.B, cfg.Tmax, cfg.NKV, cfg.hd)
        dk = dk.view(shape).permute(0, 2, 1, 3).contiguous()
        dv = dv.view(shape).permute(0, 2, 1, 3).contiguous()
    dl = torch.from_numpy(lens).cuda()
    dec = DecodeAttention(cfg.B, cfg.NH, cfg.NKV, cfg.hd, cfg.Tmax, cfg.dtype, layout=args.decode_layout)
    for _ in range(args.warmup):
        dec(dq, dk, dv, dl)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dec(dq, dk, dv, dl)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / args.steps * 1e3
    tim = None
    if not args.no_timing:
        binding.timing_enable(True)
        binding.timing_collect()
        for _ in range(args.steps):
            dec(dq, dk, dv, dl)
        tim = binding.timing_collect()
        binding.timing_enable(False)
    es = 2
    kv_bytes = float(lens.astype(np.int64).sum()) * cfg.NKV * cfg.hd * es * 2
    q_bytes = cfg.B * cfg.NH * cfg.hd * es
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        oracle.build(force=False)
        t0 = time.perf_counter()
        oracle.attn_decode(q, kc, vc, lens, cfg.NH, cfg.NKV, cfg.hd)
        dt = time.perf_counter() - t0
        cpu = {"value": round(cfg.B / dt, 2), "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
               "sample": f"the whole workload ({cfg.B} sequences) in fp64, {dt:.2f} s"}
    return cfg, ms, tim, kv_bytes, q_bytes, int(lens.sum()), dec.ws.numel(), cpu


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for --gpus {args.gpus}); this library has no multi-GPU "
              "path: the block shards over sequences with one gradient all-reduce per layer, described in the "
              "design notes but not built.", file=sys.stderr)
        sys.exit(2)
    if args.traffic_summary:
        n = 256 * (1 << 20)
        root = args.traffic_summary
        bench = "python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-timing"
        cmds = ["export TMPDIR=/tmp"]
        for sub, ctr, prog in (("fetch", "FETCH_SIZE", bench), ("write", "WRITE_SIZE", bench),
                               ("copy_fetch", "FETCH_SIZE", "python3 bench.py --copy-probe-mib 256"),
                               ("copy_write", "WRITE_SIZE", "python3 bench.py --copy-probe-mib 256")):
            cmds.append(f"timeout -s KILL 120 rocprofv3 --pmc {ctr} -d {root}/{sub} -o p -- {prog}")
        cmds.append(f"python3 bench.py --traffic-summary {root} > profiles/gemm_fwd_llama_gqa_traffic.md")
        print(traffic_summary(root, {"workload": "llama_gqa", "copy_bytes": n, "commands": cmds}))
        return
    if args.counter_summary:
        root = args.counter_summary
        bench = "python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-timing --no-overlap"
        cmds = ["cd /tmp && export TMPDIR=/tmp"]
        for sub, ctrs in COUNTER_PASSES.items():
            cmds.append(f"timeout -s KILL 150 rocprofv3 --pmc {ctrs} -d {root}/{sub} -o p -- "
                        f"{bench.replace('bench.py', '/root/repo/bench.py')}")
        cmds.append(f"cd /root/repo && python3 bench.py --counter-summary {root} > "
                    "profiles/llama_gqa_instruction_counters.md")
        print(counter_summary(root, cmds))
        return
    if args.workload == "oracle_table":
        oracle_table(args)
        return
    import torch
    from decoder_only_transformer_block_amd import configs
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4, "repeats": 3}))
        return
    if args.workload == "hbm_cold":
        rows = bench_hbm_cold(args)
        print("| workload | kernel | dtype | bytes per launch | hot GB/s (frac) | cold GB/s (frac) | cold us |")
        print("|---|---|---|---:|---:|---:|---:|")
        for r in rows:
            print(f"| {r['workload']} | {r['kernel']} | {r['dtype']} | {r['bytes_per_launch']} | "
                  f"{r['hot']['gbps']} ({r['hot']['frac_hbm_peak']}) | {r['cold']['gbps']} "
                  f"({r['cold']['frac_hbm_peak']}) | {r['cold']['us_per_launch']} |")
        print(json.dumps({"hbm_cold": rows}))
        return
    if args.workload == "adamw":
        ms, n, nbytes = bench_adamw(args)
        gbps = nbytes / (ms * 1e-3) / 1e9
        print(json.dumps({
            "metric": "AdamW parameter updates/s (fused, flat fp32 master buffer + bf16 copy)",
            "value": round(n / (ms * 1e-3), 1), "unit": "params/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": "adamw over the Llama-GQA model (4 blocks + token table + head)", "params": n},
            "roofline": {"kernel": "adamw_kernel", "bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK,
                         "unit": "GB/s", "frac": round(gbps / HBM_PEAK, 4), "traffic": None,
                         "algorithmic_bytes_per_launch": nbytes},
            "cpu_baseline": None}), flush=True)
        return
    if args.workload == "head_ce":
        t, R, C, V, ws_bytes, logit_bytes = bench_head_ce(args)
        fl = 2.0 * R * C * V
        tf = 4 * fl / (t["fused"] * 1e-3) / 1e12
        print(json.dumps({
            "metric": "LM head + cross-entropy forward and backward tokens/s (fused, vocabulary-chunked)",
            "value": round(R / (t["fused"] * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(t["fused"], 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "Llama-GQA head: R=16384 positions, C=2048, V=32000, chunk 4096"},
            "roofline": {"kernel": "lm_head_ce (four GEMMs of the head's size)", "bound": "mfma",
                         "achieved": round(tf, 2), "peak": 2500.0, "unit": "TFLOP/s", "frac": round(tf / 2500.0, 4),
                         "traffic": None},
            "unfused_ms": round(t["unfused"], 4),
            "unfused_tflops_3gemm": round(3 * fl / (t["unfused"] * 1e-3) / 1e12, 2),
            "workspace_bytes_fused": ws_bytes, "logits_bytes_unfused": logit_bytes,
            "cpu_baseline": None}), flush=True)
        return
    if args.workload == "mtp_head":
        ms, R, C, V, K, ws_bytes = bench_mtp_head(args)
        fl = 4 * 2.0 * R * C * V * K  # four head-sized GEMMs per head (two passes, dinp, dW)
        tf = fl / (ms * 1e-3) / 1e12
        print(json.dumps({
            "metric": "multi-token-prediction head + cross-entropy forward and backward tokens/s (fused, chunked)",
            "value": round(R / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": f"Llama-GQA head with K={K} prediction heads: R=16384 positions, C=2048, "
                                   "V=32000 per head, chunk 4096"},
            "roofline": {"kernel": "lm_head_mtp_ce (four GEMMs of one head's size per head)", "bound": "mfma",
                         "achieved": round(tf, 2), "peak": 2500.0, "unit": "TFLOP/s", "frac": round(tf / 2500.0, 4),
                         "traffic": None},
            "workspace_bytes": ws_bytes, "cpu_baseline": None}), flush=True)
        return
    if args.workload == "decode":
        cfg, ms, tim, kv_bytes, q_bytes, ntok, ws_bytes, cpu = bench_decode(args)
        roof = None
        brk = {}
        if tim:
            for k in ("attn_decode", "decode_merge"):
                v = tim.get(k)
                if v and v["launches"]:
                    brk[k] = {"ms_per_step": round(v["ms"] / args.steps, 4),
                              "launches_per_step": v["launches"] // args.steps}
            d = tim.get("attn_decode")
            if d and d["launches"]:
                avg = d["ms"] / d["launches"]
                per = kv_bytes + q_bytes
                gb = per / (avg * 1e-3) / 1e9
                inst = "decode_bf16_kernel<64, 2, 1>" if args.decode_layout == "head" else "decode_bf16_kernel<64, 2, 8>"
                roof = {"kernel": f"{inst} (chunked decode attention)", "bound": "hbm",
                        "achieved": round(gb, 1), "peak": HBM_PEAK, "unit": "GB/s", "frac": round(gb / HBM_PEAK, 4),
                        "traffic": None, "avg_launch_ms": round(avg, 4), "algorithmic_bytes_per_launch": per}
        print(json.dumps({
            "metric": "decode attention tokens/s (one new query per sequence against its KV cache)",
            "value": round(cfg.B / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic (seeded N(0,1) q / caches, uniform lengths)",
            "config": {"workload": "decode attention, Llama-GQA heads: B=256 sequences, cache lengths uniform "
                                   "in [1, 4096], NH=32, NKV=8, hd=64", "cache_layout": args.decode_layout,
                       "cached_positions": ntok,
                       "kv_bytes": kv_bytes, "workspace_bytes": ws_bytes},
            "roofline": roof, "breakdown": brk, "cpu_baseline": cpu}), flush=True)
        return
    cfg = configs.ALL_CONFIGS[args.workload]

    if args.workload == "attn_long":
        ms, value, tim = bench_attn(args, cfg)
        flops_step = cfg.fwd_flops() * 3.5
        config = {"workload": cfg.name, "B": cfg.B, "T": cfg.T, "NH": cfg.NH, "NKV": cfg.NKV, "hd": cfg.hd,
                  "global_batch": cfg.B, "seq_len": cfg.T, "parallelism": "none (1 GPU)"}
    else:
        ms, value, tim = bench_block(args, cfg)
        flops_step = (cfg.gemm_flops_per_layer() + cfg.attn_flops_per_layer()) * cfg.L
        config = {"workload": cfg.name, "layers": cfg.L, "B": cfg.B, "T": cfg.T, "C": cfg.C, "NH": cfg.NH,
                  "NKV": cfg.NKV, "head_dim": cfg.hd, "H": cfg.H, "norm": cfg.norm, "mlp": cfg.mlp,
                  "rope": cfg.rope, "global_batch": cfg.B, "seq_len": cfg.T, "parallelism": "none (1 GPU)"}

    peak = PEAK[cfg.dtype]
    breakdown = {}
    for k, v in tim.items():
        if v["launches"] == 0:
            continue
        e = {"ms_per_step": round(v["ms"] / args.steps, 4), "launches_per_step": v["launches"] // args.steps}
        if v["flops"] > 0:
            tf = v["flops"] / (v["ms"] * 1e-3) / 1e12
            e["tflops"] = round(tf, 2)
            e["frac_mfma_peak"] = round(tf / peak, 4)
        if v["bytes"] > 0 and v["flops"] == 0:
            gb = v["bytes"] / (v["ms"] * 1e-3) / 1e9
            e["gbps"] = round(gb, 1)
            e["frac_hbm_peak"] = round(gb / HBM_PEAK, 4)
        breakdown[k] = e
    gem = [tim[k] for k in ("gemm_fwd", "gemm_dinp", "gemm_dw") if k in tim and tim[k]["launches"]]
    if gem:
        ms_g = sum(v["ms"] for v in gem)
        fl_g = sum(v["flops"] for v in gem)
        tf = fl_g / (ms_g * 1e-3) / 1e12
        breakdown["gemm"] = {"ms_per_step": round(ms_g / args.steps, 4),
                             "launches_per_step": sum(v["launches"] for v in gem) // args.steps,
                             "tflops": round(tf, 2), "frac_mfma_peak": round(tf / peak, 4)}
    dom = "attn_bwd" if args.workload == "attn_long" else "gemm_fwd"
    roof = None
    if dom in tim and tim[dom]["launches"]:
        d = tim[dom]
        ach = d["flops"] / (d["ms"] * 1e-3) / 1e12
        traffic = None
        if dom == "gemm_fwd":
            st = stored_traffic(args.workload) if cfg.dtype == "bf16" else None
            traffic = st["traffic_bytes_per_launch"] if st else None
        gemm_name = GEMM_FWD_KERNEL if cfg.dtype == "bf16" else "gemm_kernel<float, 64, 128|64, true, true>"
        roof = {"kernel": "attention backward (dq + dk/dv kernels)" if dom == "attn_bwd" else
                f"forward-projection GEMM {gemm_name} (QKV, O, MLP up, MLP down)",
                "bound": "mfma", "achieved": round(ach, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(ach / peak, 4), "traffic": traffic,
                "avg_launch_ms": round(d["ms"] / d["launches"], 4),
                "flops_per_launch": d["flops"] / d["launches"],
                "algorithmic_bytes_per_launch": round(d["bytes"] / d["launches"])}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_attn(cfg, 1024) if args.workload == "attn_long" else \
            cpu_baseline(cfg, args.cpu_tokens or cfg.T)

    line = {
        "metric": "train tokens/s per block fwd+bwd; attn+GEMM TFLOP/s as % MFMA peak",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "ms_per_step_median": round(getattr(args, "step_median_ms", ms), 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.dtype, "data": "synthetic (seeded N(0,0.02) weights, uniform token ids, random init)",
        "config": config,
        "algorithmic_tflops_per_step": round(flops_step / 1e12, 4),
        "achieved_tflops": round(flops_step / (ms * 1e-3) / 1e12, 2),
        "roofline": roof, "breakdown": breakdown, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
