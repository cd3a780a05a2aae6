#!/usr/bin/env python3
"""EntropyCache denoising-step benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Workload: the 8B-shaped bf16 model (32 layers, d=4096, 32x128 heads, SwiGLU
12288, V=126464, RoPE) decoding L = 1024 = 768 prompt + 256 masked positions
in blocks of 32, one token per step, k = 16, tau = 1.0 (the middle of the
{0.25, 0.5, 1, 2} sweep). Weights are seeded N(0, 0.02) and prompts uniform
random ids (synthetic stand-ins for trained weights and benchmark prompts).

A step is one call of ec_step: forward (refresh or skip), entropy/argmax/
confidence reduction, decode/decide/plan, and the one host readback of E.
Prints ONE JSON line on stdout; progress goes to stderr.
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

METRIC = "denoising steps/s and gen tokens/s at L=1024,k=16 (1 GPU); % HBM/MFMA peak"
# kernel the library launches for each timed group at M = 1024 (must match the profile's tag)
KERNEL_TAGS = {"gateup": "gemm_bf16_kernel<256,192,64,96,2,false,EPI_SWIGLU,false,64,4>"}
DOMINANT = "gateup"  # the SwiGLU GEMM: the largest kernel group of a refresh step
PROFILE_DIR = os.path.join(ROOT, "profiles")
HBM_PEAK = 8.0e12          # bytes/s, MI355X HBM3E
MFMA_BF16_PEAK = 2.5e15    # flop/s, dense bf16


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ algorithmic work per step
def step_work(m, L: int, r: int, n_cand: int):
    """(flops, bytes) the method must do for one step that recomputes r rows.

    flops: every projection over the r rows, attention of r queries over L keys,
    except in the last layer, whose K/V projection covers the r rows and whose
    attention, O-proj and MLP only the candidate rows (the only final states the LM
    head reads); the LM head over the candidate rows. bytes: every weight once, the
    K/V cache read once (L rows) and the r recomputed rows written, the candidate
    logits written and read by the reduction.
    """
    d, F, V, nl = m.d_model, m.ffn_dim, m.vocab, m.n_layers
    per_layer_w = 4 * d * d + 3 * d * F
    c = min(n_cand, r)
    last = 2 * r * 3 * d * d + 2 * c * (d * d + 3 * d * F) + 4 * c * L * d
    flops = (nl - 1) * (2 * r * per_layer_w + 4 * r * L * d) + last + 2 * n_cand * V * d
    bytes_ = 2 * (nl * per_layer_w + V * d) + nl * (2 * L * d * 2 + 2 * r * d * 2) + 2 * 2 * n_cand * V
    return float(flops), float(bytes_)


def measured_traffic(group: str):
    """HBM bytes per launch from the committed PMC summary, if it covers the kernel in use."""
    import re
    tag = KERNEL_TAGS.get(group)
    if tag is None or not os.path.isdir(PROFILE_DIR):
        return None
    for f in sorted(os.listdir(PROFILE_DIR)):
        if not f.endswith((".md", ".txt")):
            continue
        for line in open(os.path.join(PROFILE_DIR, f)):
            m = re.match(r"traffic_bytes_per_launch: (\d+) kernel: (\S+)", line.strip())
            if m and m.group(2) == tag:
                return int(m.group(1))
    return None


def t_roof(flops: float, bytes_: float) -> float:
    return max(flops / MFMA_BF16_PEAK, bytes_ / HBM_PEAK)


# ------------------------------------------------------------------ model upload
def upload_model(cfg, keep_layers: int, device="cuda"):
    """Generate seeded weights layer by layer on the host and upload them.

    Returns (DeviceModel, host copy of embed / the first keep_layers layers / lm_head).
    """
    import numpy as np
    import torch
    from concurrent.futures import ThreadPoolExecutor
    import synth
    from entropy_guided_kv_amd import api

    m = cfg.model
    threads = min(16, len(os.sched_getaffinity(0)))
    to_dev = lambda a: api._to_device(a, m.dtype, device)
    host = {"layers": []}
    t0 = time.time()
    with ThreadPoolExecutor(threads) as pool:
        emb = synth.make_embed(m, cfg.seed, pool)
        head = synth.make_lm_head(m, cfg.seed, pool)
        d_emb, d_head = to_dev(emb), to_dev(head)
        host["embed"], host["lm_head"] = emb, head
        layers = []
        for i in range(m.n_layers):
            lw = synth.make_layer(m, i, cfg.seed, pool)
            layers.append({k: to_dev(v) for k, v in lw.items()})
            if i < keep_layers:
                host["layers"].append(lw)
            if i % 8 == 7:
                log(f"[bench] weights: {i + 1}/{m.n_layers} layers on device ({time.time() - t0:.1f}s)")
    fn = synth.make_final_norm(m)
    host["final_norm"] = fn
    rope_max = max(cfg.seq_len, synth.CONFIGS["long"].seq_len)  # the long-context batch reuses the model
    dm = api.DeviceModel(m, d_emb, layers, to_dev(fn), d_head, rope_max_pos=rope_max, device=device)
    torch.cuda.synchronize()
    return dm, host


# ------------------------------------------------------------------ GPU runs
def run_trajectory(dec, prompt, steps=None):
    """Run one trajectory from reset; returns (outs, wall seconds, event ms)."""
    import torch
    dec.reset(prompt)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    outs = dec.run(max_steps=steps)
    ev1.record()
    torch.cuda.synchronize()
    return outs, time.perf_counter() - t0, ev0.elapsed_time(ev1)


def timed_steps(dec, prompt, K, time_group=None):
    """Exactly K ec_step calls (restarting the trajectory when it completes).

    With time_group, the library brackets every launch of that kernel group with a
    pair of HIP events on its stream during these K steps (two event records per
    launch, no other group is timed); the group's totals are returned as well."""
    import torch
    from entropy_guided_kv_amd import api
    dec.reset(prompt)
    outs = []
    torch.cuda.synchronize()
    if time_group:
        api.ec_timing_read(reset=True)
        api.ec_timing_select([time_group])
        api.ec_timing_enable(True)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(K):
        if dec.done:
            dec.reset(prompt)
        outs.append(dec.step())
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    group = None
    if time_group:
        api.ec_timing_enable(False)
        group = api.ec_timing_read(reset=True)[time_group]
        api.ec_timing_select(None)
    return outs, wall, ev0.elapsed_time(ev1), group


def batch_step_work(m, L: int, rows, cands):
    """(flops, bytes) of one batched step: per-sequence work summed, weights read once."""
    f = b = 0.0
    w_bytes = 2.0 * (m.n_layers * (4 * m.d_model ** 2 + 3 * m.d_model * m.ffn_dim) + m.vocab * m.d_model)
    for r, c in zip(rows, cands):
        fi, bi = step_work(m, L, r, c)
        f += fi
        b += bi - w_bytes
    return f, b + w_bytes


def long_batch_bench(dm, steps: int, warmup: int = 2):
    """The long-context workload: 4 sequences of 3584 prompt + 512 masked positions,
    k = 32, stepped together by ec_step_batch (one forward over all their rows per step).
    tau = 1.0 as configured (every step refreshes with random weights), then tau = +inf
    (one refresh per sequence, then skip steps)."""
    import torch
    import synth
    from entropy_guided_kv_amd import api
    cfg = synth.CONFIGS["long"]
    m = cfg.model
    prompts = [torch.from_numpy(synth.make_prompt(cfg, seq=i)) for i in range(cfg.batch)]
    bd = api.BatchDecoder(dm, cfg.batch, cfg.seq_len, cfg.prompt_len, cfg.tokens_per_step,
                          cfg.block_len, cfg.k_recent, 1.0)
    res = {"workload": f"{cfg.batch} sequences x (L={cfg.seq_len} = {cfg.prompt_len} prompt + "
                       f"{cfg.n_masked} masked), k={cfg.k_recent}, 1 token/step, blocks of {cfg.block_len}",
           "workspace_MiB": bd.workspace.numel() / 2 ** 20}
    for tau in (1.0, math.inf):
        bd.set_tau(tau)
        bd.reset(prompts)
        n_warm = warmup if tau == 1.0 else 1  # at +inf the first (refresh) step is the warmup
        for _ in range(n_warm):
            bd.step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        outs = [bd.step() for _ in range(steps)]
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        roof = 0.0
        ntok = nref = nseq = 0
        for st in outs:
            live = [o for o in st if o is not None]
            f, b = batch_step_work(m, cfg.seq_len, [o.rows for o in live], [o.n_cand for o in live])
            roof += t_roof(f, b)
            ntok += sum(len(o.positions) for o in live)
            nref += sum(o.refreshed for o in live)
            nseq += len(live)
        first = n_warm if tau == 1.0 else 1
        res[f"tau={tau}"] = {"window": f"steps {first}..{first + steps - 1} of the {cfg.steps}-step trajectory "
                                       f"(not a whole trajectory)",
                             "steps": steps, "steps_per_s": steps / wall,
                             "gen_tokens_per_s": ntok / wall, "ms_per_step": wall * 1e3 / steps,
                             "refresh_rate": nref / max(nseq, 1),
                             "mean_rows_per_seq": sum(o.rows for st in outs for o in st if o) / max(nseq, 1),
                             "roofline_frac": roof / wall}
        log(f"[bench] long batch-4 tau={tau}: {steps / wall:.2f} steps/s, {ntok / wall:.1f} tokens/s, "
            f"roofline {roof / wall:.3f}")
    del bd
    torch.cuda.empty_cache()
    return res


def drift_probe_bench(dec, prompt, steps: int):
    """ec_step_probe on the headline workload: the probe's cost per step, and E of step t
    against the mean (over layers) V drift that step t+1 measures on the rows it recomputes
    (every row on a refresh step: the pages' step-to-step KV drift)."""
    import numpy as np
    import torch
    nl = len(dec.model.layers)
    drift = torch.zeros(4 * nl, dtype=torch.float32, device="cuda")
    res = {}
    for probe in (False, True):
        dec.reset(prompt)
        dec.step(drift=drift if probe else None)  # first step: cache never written (NaN drift)
        torch.cuda.synchronize()
        es, dv, dk = [], [], []
        t0 = time.perf_counter()
        for _ in range(steps):
            if dec.done:
                break
            o = dec.step(drift=drift if probe else None)
            if probe:
                d = drift.cpu().numpy().reshape(nl, 4)
                dk.append(float(np.nanmean(d[:, 0])))
                dv.append(float(np.nanmean(d[:, 2])))
            es.append(o.emax)
        torch.cuda.synchronize()
        res["probe" if probe else "plain"] = (time.perf_counter() - t0) / max(len(es), 1)
    e = np.array(es[:-1])
    v = np.array(dv[1:])
    out = {"steps": len(es), "ms_per_step_plain": res["plain"] * 1e3, "ms_per_step_probe": res["probe"] * 1e3,
           "probe_overhead_ms": (res["probe"] - res["plain"]) * 1e3,
           "mean_V_drift": float(np.mean(dv)) if dv else None, "mean_K_drift": float(np.mean(dk)) if dk else None,
           "corr_E_t_vs_V_drift_t1": float(np.corrcoef(e, v)[0, 1]) if len(e) > 2 and np.std(e) > 0 else None}
    log(f"[bench] KV-drift probe: +{out['probe_overhead_ms']:.2f} ms/step, mean V drift {out['mean_V_drift']}, "
        f"corr(E_t, V drift t+1) {out['corr_E_t_vs_V_drift_t1']}")
    return out


def kernel_breakdown(dec, prompt, n_refresh=4, n_skip=8):
    """Per-kernel-group event timing for refresh steps and for skip steps."""
    import math as _m
    from entropy_guided_kv_amd import api
    res = {}
    tau0 = dec.params.tau
    for label, tau, n in (("refresh", -_m.inf, n_refresh), ("skip", _m.inf, n_skip + 1)):
        if n <= 1 and label == "skip":
            continue
        dec.set_tau(tau)
        dec.reset(prompt)
        if label == "skip":
            dec.step()                  # the first step always refreshes
        api.ec_timing_read(reset=True)
        api.ec_timing_enable(True)
        outs = [dec.step() for _ in range(n if label == "refresh" else n - 1)]
        api.ec_timing_enable(False)
        t = api.ec_timing_read(reset=True)
        res[label] = {"steps": len(outs), "rows_mean": sum(o.rows for o in outs) / len(outs),
                      "kernels": t}
    dec.set_tau(tau0)
    return res


def _entropy_kernel_bench(iters=50):
    """ec_entropy_max on 64 x 126464 bf16 logits: warm (one buffer) and cold (40 rotating buffers).

    A device-side sleep is queued first, so the host has enqueued all the calls by the
    time the GPU reaches them: they run back to back, and one HIP event pair around the
    batch gives the device time per call (its three kernels and the gaps between them)
    without host issue cost.
    """
    import torch
    import synth
    from entropy_guided_kv_amd import api
    bits, _ = synth.make_entropy_logits()
    import numpy as np
    base = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    rows, V = base.shape
    nbuf = 40  # 40 x 16.2 MB = 647 MB > 256 MB Infinity Cache
    bufs = [base] + [base.roll(i * 7919, dims=1).contiguous() for i in range(1, nbuf)]
    ws = torch.empty(api.load().ec_entropy_max_workspace_size(rows, V), dtype=torch.uint8, device="cuda")
    outs = (torch.empty(rows, dtype=torch.float32, device="cuda"), torch.empty(rows, dtype=torch.int32, device="cuda"),
            torch.empty(rows, dtype=torch.float32, device="cuda"), torch.empty(1, dtype=torch.float32, device="cuda"))
    for b in bufs[:4]:
        api.ec_entropy_max(b, workspace=ws, out=outs)
    torch.cuda.synchronize()
    out = {}
    for mode in ("warm", "cold"):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(20_000_000)
        ev0.record()
        for i in range(iters):
            api.ec_entropy_max(bufs[0] if mode == "warm" else bufs[i % nbuf], workspace=ws, out=outs)
        ev1.record()
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1) / iters
        out[mode] = {"us_per_call": ms * 1e3, "bytes": rows * V * 2,
                     "GBps_call": rows * V * 2 / (ms * 1e-3) / 1e9, "calls": iters}
    return out


# ------------------------------------------------------------------ CPU oracle baseline
def _host_cores():
    threads = None
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max((i.get("num_threads", 0) for i in info), default=None)
    except Exception:
        pass
    return threads or len(os.sched_getaffinity(0))


def cpu_baseline(cfg, host, prompt):
    """The oracle as it stands, on the host cores, over a bounded window of the 8B workload:
    one refresh step (all L rows, 32 layers) and the two skip steps that follow it at
    tau = +inf (r = 256 recomputed rows each), float64 numpy. `value` is the refresh-step
    rate, the step the headline workload takes every time (its E exceeds tau); the skip
    steps' times are reported beside it."""
    import numpy as np
    import synth
    from oracle import loop as ol
    from oracle import model as om

    w = synth.ModelWeights(cfg.model, host["embed"], host["layers"], host["final_norm"], host["lm_head"])
    mdl = om.OracleModel(w, keep_f64=False)
    st = ol.init_state(cfg, prompt)
    cache = om.new_cache(mdl, cfg.seq_len)
    times = []
    for _ in range(3):
        t0 = time.perf_counter()
        r = ol.step(mdl, cfg, st, cache, math.inf)
        times.append((time.perf_counter() - t0, len(r.rows), bool(r.refreshed)))
        log(f"[bench] oracle step: {times[-1][0]:.1f}s, {times[-1][1]} rows, refresh={times[-1][2]}")
    t_full = times[0][0]
    t_skip = sum(t for t, _, _ in times[1:]) / 2
    return {
        "value": 1.0 / t_full, "unit": "steps/s", "cores": _host_cores(), "kind": "oracle",
        "precision": "float64 (numpy, bf16 rounding points mirrored)",
        "sample": (f"8B-shaped model, all 32 layers: 1 refresh step (L={cfg.seq_len} rows, {t_full:.1f}s) "
                   f"and the 2 skip steps after it at tau=+inf ({times[1][1]} and {times[2][1]} rows, "
                   f"{times[1][0]:.1f}s and {times[2][0]:.1f}s); value = refresh steps/s"),
        "refresh_step_s": t_full, "skip_step_s": t_skip, "skip_steps_per_s": 1.0 / t_skip,
        "host_cpus": len(os.sched_getaffinity(0)),
    }


# ------------------------------------------------------------------ small configurations
def small_configs_bench(with_oracle: bool):
    """The tiny (fp32) and small (bf16) configurations: one whole decode each at the
    configured tau (after a warmup decode), and the oracle's whole decode of the same
    inputs timed on the host beside it."""
    import torch
    import synth
    from entropy_guided_kv_amd import api
    from oracle import loop as ol
    from oracle import model as om
    res = {}
    for name in ("tiny", "small"):
        cfg = synth.CONFIGS[name]
        w = synth.make_model(cfg.model)
        dm = api.DeviceModel.from_host(w, rope_max_pos=cfg.seq_len)
        dec = api.Decoder(dm, cfg.seq_len, cfg.prompt_len, cfg.tokens_per_step, cfg.block_len,
                          cfg.k_recent, cfg.tau)
        prompt_np = synth.make_prompt(cfg)
        prompt = torch.from_numpy(prompt_np)
        run_trajectory(dec, prompt)
        outs, wall, _ = run_trajectory(dec, prompt)
        r = {"workload": f"{name}: {cfg.model.n_layers} layers, d={cfg.model.d_model}, V={cfg.model.vocab}, "
                         f"{cfg.model.dtype}, L={cfg.seq_len} = {cfg.prompt_len} + {cfg.n_masked}, "
                         f"{cfg.tokens_per_step} token(s)/step, k={cfg.k_recent}, tau={cfg.tau}",
             "steps": len(outs), "steps_per_s": len(outs) / wall,
             "gen_tokens_per_s": sum(len(o.positions) for o in outs) / wall,
             "refresh_rate": sum(o.refreshed for o in outs) / len(outs)}
        if with_oracle:
            t0 = time.perf_counter()
            recs, _, _ = ol.run_entropycache(om.OracleModel(w), cfg, prompt_np, cfg.tau)
            t = time.perf_counter() - t0
            r["oracle"] = {"steps": len(recs), "seconds": t, "steps_per_s": len(recs) / t,
                           "cores": _host_cores(), "precision": "float64 numpy"}
        log(f"[bench] {name}: {r['steps_per_s']:.1f} steps/s" +
            (f", oracle {r['oracle']['steps_per_s']:.2f} steps/s" if with_oracle else ""))
        res[name] = r
        del dec, dm
        torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------------ mixed refresh rate
def _model_with_head(dm, head):
    """The same device model with another LM head (the layers are shared)."""
    import ctypes as C
    from types import SimpleNamespace
    desc = type(dm.desc).from_buffer_copy(dm.desc)
    desc.lm_head = head.data_ptr()
    return SimpleNamespace(desc=desc, device=dm.device, shape=dm.shape, layers=dm.layers,
                           torch_dtype=dm.torch_dtype, _keep=(dm, head, C))


def mixed_refresh_bench(dm, cfg, host, prompt, t_full_s, t_skip_s, taus=(1.0, 2.0)):
    """The 8B workload on the hot-token LM head (synth.make_hot_token_model's head: a few
    token ids' rows scaled up, every other weight as configured): decoded rows' entropies
    then spread from near 0 to near ln V, so at tau = 1 and 2 the refresh rate rho lies
    strictly between 0 and 1. Reported with the rate the refresh and skip step times of the
    plain runs predict, 1 / (rho T_full + (1 - rho) T_skip)."""
    import numpy as np
    import torch
    import synth
    from entropy_guided_kv_amd import api
    m = cfg.model
    hot = np.random.default_rng(0).choice(m.vocab - 1, 8, replace=False)
    head_np = host["lm_head"].copy()
    head_np[hot] = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(head_np[hot]) * np.float32(10.0))
    head = api._to_device(head_np, m.dtype, "cuda")
    view = _model_with_head(dm, head)
    res = {"workload": "8B-shaped bf16, L=1024 = 768 + 256, blocks of 32, 1 token/step, k=16; LM head with "
                       "8 hot token rows x10 (other weights as configured)"}
    for tau in taus:
        dec = api.Decoder(view, cfg.seq_len, cfg.prompt_len, cfg.tokens_per_step, cfg.block_len, cfg.k_recent, tau)
        run_trajectory(dec, prompt, steps=8)
        outs, wall, _ = run_trajectory(dec, prompt)
        rho = sum(o.refreshed for o in outs) / len(outs)
        pred = 1.0 / (rho * t_full_s + (1 - rho) * t_skip_s)
        res[f"tau={tau}"] = {"steps": len(outs), "steps_per_s": len(outs) / wall, "refresh_rate": rho,
                             "mean_rows": sum(o.rows for o in outs) / len(outs),
                             "predicted_steps_per_s": pred, "T_full_ms": t_full_s * 1e3, "T_skip_ms": t_skip_s * 1e3}
        log(f"[bench] hot-token head tau={tau}: {len(outs) / wall:.1f} steps/s at refresh rate {rho:.3f} "
            f"(predicted {pred:.1f})")
        del dec
    del view, head
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------------ main
def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256, help="timed denoising steps")
    ap.add_argument("--warmup", type=int, default=16, help="untimed steps before timing")
    ap.add_argument("--no-sweep", action="store_true", help="skip the tau sweep")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-small", action="store_true", help="skip the tiny / small configuration runs")
    ap.add_argument("--no-breakdown", action="store_true",
                    help="skip the per-kernel event timing (and the roofline object)")
    ap.add_argument("--breakdown", choices=("refresh", "both"), default="both",
                    help="which step kinds the per-kernel event timing covers")
    ap.add_argument("--no-entropy", action="store_true", help="skip the 64x126464 entropy kernel run")
    ap.add_argument("--entropy-only", action="store_true",
                    help="only the 64x126464 entropy kernel run (no model)")
    ap.add_argument("--no-drift", action="store_true", help="skip the KV-drift probe run")
    ap.add_argument("--no-long", action="store_true",
                    help="skip the long-context batch-of-4 workload (ec_step_batch)")
    ap.add_argument("--long-steps", type=int, default=8, help="timed steps of the long-context batch")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 256 MiB device copy (a known-size reference for HBM counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the EntropyCache step of one sequence runs on one "
              "MI355X with no sharding (see the design notes for how it would shard); run with "
              "--gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import synth
    from entropy_guided_kv_amd import api

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    api.load()
    if args.calib_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.entropy_only:
        ent = _entropy_kernel_bench()
        print(json.dumps({"entropy_kernel_64x126464": ent}), flush=True)
        return
    cfg = synth.CONFIGS["8b"]
    m = cfg.model
    tau = 1.0
    prompt_np = synth.make_prompt(cfg)
    prompt = torch.from_numpy(prompt_np)
    keep = 0 if args.no_cpu else m.n_layers
    dm, host = upload_model(cfg, keep)
    dec = api.Decoder(dm, cfg.seq_len, cfg.prompt_len, cfg.tokens_per_step, cfg.block_len,
                      cfg.k_recent, tau)
    log(f"[bench] model on device; workspace {dec.workspace.numel() / 2**20:.0f} MiB")

    # warmup
    dec.reset(prompt)
    for _ in range(args.warmup):
        if dec.done:
            dec.reset(prompt)
        dec.step()
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} steps done")

    # headline: exactly K steps of the configured trajectory; the dominant kernel of a refresh
    # step (the SwiGLU GEMM) is timed with HIP events on the library's stream inside this region
    outs, wall, ev_ms, dom_live = timed_steps(dec, prompt, args.steps, time_group=DOMINANT)
    steps_s = args.steps / wall
    tokens = sum(len(o.positions) for o in outs)
    refresh_rate = sum(o.refreshed for o in outs) / len(outs)
    roof_s = 0.0
    for o in outs:
        f, b = step_work(m, cfg.seq_len, o.rows, o.n_cand)
        roof_s += t_roof(f, b)
    log(f"[bench] timed {args.steps} steps: {steps_s:.2f} steps/s, refresh rate {refresh_rate:.3f}, "
        f"events {ev_ms:.1f} ms vs wall {wall * 1e3:.1f} ms")

    # tau sweep (whole trajectories) + tau = +inf (one refresh, then skip steps)
    sweep = {}
    if not args.no_sweep:
        for tv in (0.25, 0.5, 1.0, 2.0, math.inf):
            dec.set_tau(tv)
            o2, w2, _ = run_trajectory(dec, prompt)
            f_roof = sum(t_roof(*step_work(m, cfg.seq_len, o.rows, o.n_cand)) for o in o2)
            sweep[str(tv)] = {
                "steps": len(o2), "steps_per_s": len(o2) / w2,
                "gen_tokens_per_s": sum(len(o.positions) for o in o2) / w2,
                "refresh_rate": sum(o.refreshed for o in o2) / len(o2),
                "mean_rows": sum(o.rows for o in o2) / len(o2),
                "roofline_frac": f_roof / w2,
                "emax_mean": float(np.mean([o.emax for o in o2])),
            }
            log(f"[bench] tau={tv}: {sweep[str(tv)]['steps_per_s']:.2f} steps/s, "
                f"refresh {sweep[str(tv)]['refresh_rate']:.3f}")
        dec.set_tau(tau)

    # sliding-window decoding (candidates from a window at the lowest masked position)
    window = {}
    if not args.no_sweep:
        wdec = api.Decoder(dm, cfg.seq_len, cfg.prompt_len, cfg.tokens_per_step, cfg.block_len,
                           cfg.k_recent, tau, window=True)
        for tv in (1.0, math.inf):
            wdec.set_tau(tv)
            o2, w2, _ = run_trajectory(wdec, prompt)
            f_roof = sum(t_roof(*step_work(m, cfg.seq_len, o.rows, o.n_cand)) for o in o2)
            window[str(tv)] = {"steps": len(o2), "steps_per_s": len(o2) / w2,
                               "gen_tokens_per_s": sum(len(o.positions) for o in o2) / w2,
                               "refresh_rate": sum(o.refreshed for o in o2) / len(o2),
                               "mean_rows": sum(o.rows for o in o2) / len(o2), "roofline_frac": f_roof / w2}
            log(f"[bench] sliding window tau={tv}: {window[str(tv)]['steps_per_s']:.2f} steps/s")
        del wdec
        sweep["sliding_window"] = window

    # roofline object of the dominant kernel, from the timed region's events
    roofline = roofline_object(DOMINANT, dom_live)
    # per-kernel event timing (refresh steps and skip steps)
    kernels = {}
    if not args.no_breakdown:
        kernels = breakdown_report(dec, prompt, args.breakdown == "both")
        if args.breakdown == "both":
            kernels["skip_rows_profile"] = skip_rows_profile(dm, dec.cache)

    drift_res = None
    if not args.no_drift:
        drift_res = drift_probe_bench(dec, prompt, 32)

    long_res = None
    if not args.no_long:
        long_res = long_batch_bench(dm, args.long_steps)

    ent = None
    if not args.no_entropy:
        ent = _entropy_kernel_bench()
        log(f"[bench] entropy kernel 64x126464: warm {ent['warm']['us_per_call']:.1f} us, "
            f"cold {ent['cold']['us_per_call']:.1f} us")

    mixed = None
    if not args.no_sweep and "inf" in sweep:
        t_full = wall / args.steps  # every headline step refreshes
        inf = sweep["inf"]
        t_skip = (inf["steps"] / inf["steps_per_s"] - t_full) / max(inf["steps"] - 1, 1)
        mixed = mixed_refresh_bench(dm, cfg, host, prompt, t_full, t_skip)

    small = None
    if not args.no_small:
        small = small_configs_bench(with_oracle=not args.no_cpu)

    cpu = None
    if not args.no_cpu:
        log("[bench] CPU oracle baseline (1 refresh + 2 skip steps of the 8B model) ...")
        cpu = cpu_baseline(cfg, host, prompt_np)
        log(f"[bench] CPU oracle: {cpu['value']:.4f} refresh steps/s, {cpu['skip_steps_per_s']:.4f} skip steps/s "
            f"on {cpu['cores']} threads")
    emit(args, cfg, tau, steps_s, wall, tokens, refresh_rate, roof_s, ev_ms, sweep, roofline, kernels,
         ent, cpu, long_res, drift_res, mixed, small)


def roofline_object(dom, dk):
    """`roofline` of the dominant kernel group from its event totals (timed region)."""
    if not dk or not dk["launches"]:
        return None
    avg_ms = dk["ms"] / dk["launches"]
    flops_launch = dk["flops"] / dk["launches"]
    bytes_launch = dk["bytes"] / dk["launches"]
    if flops_launch > 0:
        achieved = flops_launch / (avg_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "kernel": dom, "achieved": achieved, "peak": MFMA_BF16_PEAK / 1e12,
                    "unit": "TFLOP/s", "frac": achieved / (MFMA_BF16_PEAK / 1e12),
                    "traffic": measured_traffic(dom),
                    "avg_launch_us": avg_ms * 1e3, "launches": dk["launches"],
                    "flops_per_launch": flops_launch, "bytes_per_launch": bytes_launch}
    else:
        achieved = bytes_launch / (avg_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK / 1e9,
                    "unit": "GB/s", "frac": achieved / (HBM_PEAK / 1e9),
                    "traffic": measured_traffic(dom),
                    "avg_launch_us": avg_ms * 1e3, "launches": dk["launches"], "bytes_per_launch": bytes_launch}
    log(f"[bench] dominant kernel {dom}: {avg_ms * 1e3:.1f} us/launch over the timed region "
        f"({dk['launches']} launches), {roofline['frac']:.3f} of peak")
    return roofline


def skip_rows_profile(dm, cache, rs=(17, 32, 64, 96, 128, 192, 256), reps=5):
    """Partial forwards of a skip step at several row counts r, on the decoder's cache.

    rows = the last r positions, outputs = the first min(32, max(1, r - 16)) of them (a skip
    step recomputes its masked positions plus the k = 16 most recent ones; the candidates are
    masked). Per r: the device time per forward (HIP events around `reps` back-to-back calls,
    untimed groups), the time per kernel group (a second pass with every group event-timed) and
    the fraction of the step's roof, max(flops / MFMA peak, bytes / HBM peak), with the LM head's
    stored logits in place of the fused entropy epilogue of ec_step.
    """
    import torch
    from entropy_guided_kv_amd import api
    m = dm.shape
    L = cache.seq_len
    tokens = torch.randint(0, m.vocab - 1, (L,), dtype=torch.int32, generator=torch.Generator().manual_seed(5)).cuda()
    ws = None
    out = {}
    for r in rs:
        n_out = min(32, max(1, r - 16))
        rows = torch.arange(L - r, L, dtype=torch.int32, device="cuda")
        oidx = torch.arange(n_out, dtype=torch.int32, device="cuda")
        need = api.load().ec_forward_workspace_size(api.C.byref(dm.desc), r, n_out, L)
        if ws is None or ws.numel() < need:
            ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        for _ in range(2):
            api.ec_forward(dm, cache, tokens, rows, oidx, workspace=ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            api.ec_forward(dm, cache, tokens, rows, oidx, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        api.ec_timing_read(reset=True)
        api.ec_timing_enable(True)
        for _ in range(reps):
            api.ec_forward(dm, cache, tokens, rows, oidx, workspace=ws)
        api.ec_timing_enable(False)
        t = api.ec_timing_read(reset=True)
        fl, by = step_work(m, L, r, n_out)
        out[str(r)] = {"outputs": n_out, "ms": ms, "roofline_frac": t_roof(fl, by) * 1e3 / ms,
                       "groups_ms": {k: x["ms"] / reps for k, x in t.items() if x["launches"]}}
        log(f"[bench] skip forward r={r}: {ms:.3f} ms, {t_roof(fl, by) * 1e3 / ms:.3f} of its roof")
    return out


def breakdown_report(dec, prompt, with_skip=True):
    """Per-kernel-group timing of refresh and skip steps (every group timed, so slower than
    the headline run); checks that the SwiGLU GEMM is the dominant group of a refresh step."""
    kb = kernel_breakdown(dec, prompt, n_skip=8 if with_skip else 0)
    ref = kb["refresh"]["kernels"]
    dom = max(ref, key=lambda k: ref[k]["ms"])
    if dom != DOMINANT:
        log(f"[bench] warning: the largest group of a refresh step is {dom}, not {DOMINANT}")
    kernels = {}
    for label, v in kb.items():
        tot = sum(x["ms"] for x in v["kernels"].values())
        kernels[label] = {
            "rows_mean": v["rows_mean"],
            "ms_per_step": tot / v["steps"],
            "groups": {k: {"ms_per_step": x["ms"] / v["steps"],
                           "TFLOPs": (x["flops"] / (x["ms"] * 1e-3) / 1e12) if x["ms"] > 0 else 0.0,
                           "GBps": (x["bytes"] / (x["ms"] * 1e-3) / 1e9) if x["ms"] > 0 else 0.0}
                       for k, x in v["kernels"].items() if x["launches"]},
        }
        dec_ms = v["kernels"]["entropy"]["ms"] + v["kernels"]["select"]["ms"]
        kernels[label]["decision_overhead_frac"] = dec_ms / tot if tot > 0 else None
    return kernels


def emit(args, cfg, tau, steps_s, wall, tokens, refresh_rate, roof_s, ev_ms, sweep, roofline,
         kernels, ent, cpu, long_res=None, drift_res=None, mixed=None, small=None):
    res = {
        "metric": METRIC,
        "value": steps_s,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) weights, uniform random prompt ids)",
        "config": {"workload": "EntropyCache decode, 8B-shaped bf16 model (32 layers, d=4096, 32x128 "
                               "heads, SwiGLU 12288, V=126464), L=1024 = 768 prompt + 256 masked, "
                               "blocks of 32, 1 token/step, k=16, tau=1.0",
                   "seq_len": cfg.seq_len, "k_recent": cfg.k_recent, "tau": tau, "global_batch": 1},
        "gen_tokens_per_s": tokens / wall,
        "refresh_rate": refresh_rate,
        "step_roofline_frac": roof_s / wall,
        "event_ms_timed_region": ev_ms,
        "tau_sweep": sweep,
        "roofline": roofline,
        "kernels": kernels,
        "entropy_kernel_64x126464": ent,
        "long_context_batch4": long_res,
        "kv_drift_probe": drift_res,
        "mixed_refresh_rate": mixed,
        "small_configs": small,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
