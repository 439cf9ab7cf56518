"""Throughput of the speculative-sampling verifier on one MI355X.

One step = one call of the verifier over the whole batch (every logit row
read, every request verified).  The timed region holds only the K steps;
per-kernel durations come from a second pass of the same K steps with HIP
events around every launch.  Default workload: 1024 requests, gamma 8,
vocabulary 256000, bf16 logits, temperature 0.7 then top-64 on p and q,
probabilistic draft (spec_verify_prob).  Inputs are seeded synthetic logits
generated on the GPU and resident in HBM before the timed region.

Prints one JSON line: verified draft positions per second (value), plus
rows/s, algorithmic GB/s, the roofline of the dominant kernel (the row pass,
timed with HIP events on the launch stream) and the fp64 CPU oracle timed on
a bounded sample of the same workload on the host cores, with the oracle's
check of the GPU's outputs on the first requests, and the method's outcome on
the batch (law of the accepted length, tokens per round, beta per position
and Eq. 1's prediction from it).
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

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, vendor figure
MALL_BYTES = 256 << 20  # MI355X last-level (Infinity) cache


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "speculative_decoding_rejection_amd", "csrc")
    for fn in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, fn), "rb") as f:
            h.update(fn.encode() + f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, per_launch_alg: float):
    """HBM bytes per launch of the row pass from committed rocprofv3 counter
    runs, if they were taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "rows_topk_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_hash") != kernel_source_hash() or t.get("workload") != workload:
        return None
    return t.get("bytes_per_launch")


def read_ceiling(sv, dev, stream, nbytes: int = 4 << 30, reps: int = 10) -> float:
    """Measured streaming-read ceiling (GB/s): the best of three timings of
    `reps` reads of an nbytes device buffer with the row passes' 16-byte
    nontemporal loads and nothing else (sv_stream_read), HIP events on the
    launch stream."""
    import torch

    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.zeros(256, dtype=torch.int32, device=dev)
    for _ in range(2):
        sv.sv_stream_read(buf, sink, stream)
    best = 0.0
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            sv.sv_stream_read(buf, sink, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        best = max(best, nbytes * reps / (e0.elapsed_time(e1) / 1e3) / 1e9)
    del buf
    torch.cuda.empty_cache()
    return best


def cpu_baseline(wl, inp, target_seconds: float, got: dict | None = None, check_requests: int | None = None) -> dict:
    """The fp64 oracle timed on the first requests of the workload (sized to
    about target_seconds of host time).  With got (the GPU's outputs of the
    same call, per request, host arrays), an untimed diagnostics pass over
    the first check_requests of them (default: every request) compares the
    two: largest |dp| and |dq| of the gathered probabilities, near-tie rows
    against the 0.01% bar, and requests that differ (outside near-ties, and
    within them)."""
    import oracle
    import workloads
    from oracle.parity import compare, compare_batch, near_tie_rows

    modes = {"prob": oracle.MODE_PROB, "onehot": oracle.MODE_ONEHOT, "greedy": oracle.MODE_GREEDY}

    def run(n, diagnostics=False):
        sub = slice(0, n)
        lt = workloads.to_host_arrays(inp["target_logits"][sub])
        ld = workloads.to_host_arrays(inp["draft_logits"][sub]) if wl.has_draft_logits else None
        x = workloads.to_host_arrays(inp["draft_tokens"][sub])
        if wl.has_settings:
            probs = inp["draft_probs"][sub].cpu().numpy() if wl.draft_probs else None
            lens = inp["lengths"][sub].cpu().numpy() if wl.lengths else None
            par = inp["parents"][sub].cpu().numpy() if inp.get("parents") is not None else None
            tt, kk, pp = (inp[k][sub].cpu().numpy() for k in ("temperature", "top_k", "top_p"))
        t0 = time.perf_counter()
        if wl.has_settings:
            ref = oracle.verify_batch(lt, None if wl.draft_probs else ld, x, tt, kk, pp,
                                      max_top_k=max(k for _, k, _ in wl.mix), seed=wl.verify_seed,
                                      draft_probs=probs, lengths=lens, match=wl.entry == "match", parents=par,
                                      diagnostics=diagnostics)
        else:
            ref = oracle.verify(modes[wl.entry], lt, ld, x, temperature=wl.temperature, top_k=wl.top_k,
                                seed=wl.verify_seed, diagnostics=diagnostics and wl.entry != "greedy")
        return time.perf_counter() - t0, ref

    threads = oracle.max_threads()
    n = min(wl.B, max(4, threads))
    t, _ = run(n)
    if t < target_seconds / 3 and n < wl.B:
        n = int(min(wl.B, max(n + 1, n * target_seconds / max(t, 1e-3))))
        t, _ = run(n)
    reps = 1
    if t < target_seconds / 3 and n == wl.B:
        # The whole workload is a short sample: time it repeated (the same
        # call, every request each time) for a bounded total.
        reps = int(min(10000, max(2, target_seconds / 2 / max(t, 1e-4))))
        t = sum(run(n)[0] for _ in range(reps)) / reps  # oracle time only, per call
    check = None
    if got is not None:
        m = wl.B if check_requests is None else min(wl.B, check_requests)
        t_check, ref = run(m, diagnostics=True)
        sub = {k: v[:m] for k, v in got.items()}
        rep = compare_batch(sub, ref) if wl.has_settings else compare(wl.entry, sub, ref)
        rows = int(wl.draft_lengths[:m].sum()) + m if wl.has_settings else m * (wl.G + 1)
        ties = near_tie_rows(ref)
        check = {"requests": m, "rows": rows, "max_dp": rep["max_dp"], "max_dq": rep["max_dq"],
                 "near_tie_rows": ties, "near_tie_fraction": ties / rows, "near_tie_bar": 1e-4,
                 "near_tie_requests": rep["near_tie_requests"],
                 "mismatch_non_tie": rep["mismatch_non_tie"], "mismatch_tie": rep["mismatch_tie"],
                 "seconds": round(t_check, 2)}
        if "near_cut_requests" in rep:
            check["near_cut_requests"] = rep["near_cut_requests"]
            check["mismatch_cut"] = rep["mismatch_cut"]
    return {
        "value": int(wl.draft_lengths[:n].sum()) / t,
        "unit": "verified draft positions/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"first {n} of {wl.B} requests of the same workload (fp64 oracle, OpenMP over requests), "
                   f"{t:.2f} s wall" if reps == 1 else
                   f"all {n} requests of the same workload (fp64 oracle, OpenMP over requests), the call timed "
                   f"{reps} times, {t * 1e3:.2f} ms wall per call"),
        "check": check,
    }


def rounds_driver(sv, wl, rounds: int, device, seed_offset: int = 1000) -> dict:
    """Multi-round synthetic driver: `rounds` verification rounds of the
    workload, each on fresh seeded rows, with the per-position acceptance
    probability beta and the per-request counters (+= draft positions,
    accepted drafts, 1 per round) kept on the GPU.  Returns the method's
    statistics: tokens per round, the acceptance rate of each position
    measured from n (P(n > j | n >= j)), the mean beta of each position, the
    expected tokens per round from those betas by Eq. 1 of the draft-model
    page generalised to per-position rates (sum over i of the product of the
    first i rates), and the counters' totals."""
    import numpy as np
    import torch

    import workloads

    G, B = wl.G, wl.B
    counters = torch.zeros((B, 3), dtype=torch.int64, device=device)
    ns, betas, ms_stats, ms_plain = [], [], [], []
    stream = torch.cuda.current_stream()
    for r in range(rounds):
        inp = workloads.generate(wl.scaled(data_seed=wl.data_seed + seed_offset + r), device=device)
        ld = inp["draft_logits"] if wl.entry == "prob" else None
        kw = dict(single_temperature=wl.temperature, single_top_k=wl.top_k, seed=wl.verify_seed + r)
        # The same call without statistics, timed for comparison.
        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        e0.record(stream)
        sv.verify_batch(inp["target_logits"], inp["draft_tokens"], ld, **kw)
        e1.record(stream)
        res = sv.verify_batch(inp["target_logits"], inp["draft_tokens"], ld, beta=True, counters=counters, **kw)
        e2.record(stream)
        torch.cuda.synchronize()
        if r > 0:  # the first round warms up
            ms_plain.append(e0.elapsed_time(e1))
            ms_stats.append(e1.elapsed_time(e2))
        ns.append(res["num_accepted"].cpu().numpy())
        betas.append(res["beta"].cpu().numpy())
    n = np.concatenate(ns)
    beta = np.concatenate(betas)
    reach = np.array([(n >= j).sum() for j in range(G + 1)], dtype=np.float64)
    acc = [float((n > j).sum() / reach[j]) if reach[j] else float("nan") for j in range(G)]
    bmean = beta.mean(axis=0)
    eq1 = float(sum(np.prod(bmean[:i]) for i in range(G + 1)))
    c = counters.cpu().numpy().sum(axis=0)
    return {"rounds": rounds, "requests": B, "gamma": G, "tokens_per_round": float((n + 1).mean()),
            "tokens_per_round_eq1": eq1, "acceptance_by_position": acc,
            "beta_by_position": [float(v) for v in bmean],
            "counters": {"draft_n": int(c[0]), "draft_n_accepted": int(c[1]), "draft_rounds": int(c[2])},
            "mean_accepted_per_round": float(c[1] / c[2]) if c[2] else 0.0,
            "ms_per_call": float(np.mean(ms_plain)) if ms_plain else None,
            "ms_per_call_with_beta_and_counters": float(np.mean(ms_stats)) if ms_stats else None,
            "_n": n, "_counters": counters.cpu().numpy()}


def outcome_stats(sv, wl, params, sampling, layout, lt, ld, x, out, nacc, pd, qd, ta, pn, ws, stream):
    """What the method did on the batch (untimed, after the timed region):
    the law of n from the last timed call, and beta = sum min(p, q) per
    position from one more call of the same inputs with beta requested (a
    uniform batch call is bit-identical to the single-setting entry points).
    Returns (outcome, got): the statistics, and the timed call's outputs per
    request as host arrays for the oracle check."""
    import numpy as np
    import torch

    B, G, dev = wl.B, wl.G, out.device
    n_gpu = nacc.cpu().numpy()

    g_req = wl.draft_lengths if wl.has_settings else np.full(B, G)
    beta_t = torch.empty(x.shape, dtype=torch.float32, device=dev)
    o2 = [torch.empty_like(out), torch.empty_like(nacc), torch.empty_like(pd), torch.empty_like(qd)]
    if wl.has_settings:
        pn2 = torch.empty_like(pn) if pn is not None else None
        sv.spec_verify_batch(params, sampling, layout, lt, ld, x,
                             sv.make_outputs(*o2, beta=beta_t, path_nodes=pn2), ws, stream)
    else:
        bparams = sv.make_params(B, G, wl.V, wl.torch_dtype, wl.temperature if wl.entry != "greedy" else 0.0,
                                 wl.top_k, wl.verify_seed)
        bws = torch.empty(sv.sv_workspace_bytes_batch(bparams, None), dtype=torch.uint8, device=dev)
        bdraft = ld if wl.entry == "prob" else None
        blay = sv.SvLayout(sv.SV_DRAFT_LOGITS if bdraft is not None else sv.SV_DRAFT_ONEHOT, 0, wl.V,
                           wl.V if bdraft is not None else 0, None, None)
        sv.spec_verify_batch(bparams, None, blay, lt, bdraft, x, sv.make_outputs(*o2, beta=beta_t), bws, stream)
    torch.cuda.synchronize()
    beta_flat = beta_t.cpu().numpy()
    beta_pad = np.full((B, G), np.nan)
    if wl.lengths or beta_flat.ndim == 1:
        off = 0
        for b in range(B):
            beta_pad[b, :g_req[b]] = beta_flat[off:off + g_req[b]]
            off += g_req[b]
    else:
        beta_pad[:] = beta_flat
    bmean = np.nanmean(beta_pad, axis=0)
    reach = np.array([(n_gpu >= j).sum() for j in range(G + 1)], dtype=np.float64)
    outcome = {"n_histogram": np.bincount(n_gpu, minlength=G + 1).tolist(),
               "tokens_per_round": float((n_gpu + 1).mean()),
               "acceptance_by_position": [float((n_gpu > j).sum() / reach[j]) if reach[j] else None
                                          for j in range(G)],
               "beta_by_position": [float(v) for v in bmean],
               "mean_beta": float(np.nanmean(beta_pad)),
               "beta_call_same_n": bool((o2[1].cpu().numpy() == n_gpu).all())}
    if not wl.parents:
        # Eq. 1 of the draft-model page with each request's own per-position
        # rates: given its rows, position j of request b accepts with
        # probability beta[b, j], independently of the others, so
        # E[n_b + 1] = sum over i <= g_b of prod_{j < i} beta[b, j].  (The
        # same sum over the batch-mean rates is lower whenever a request's
        # rates rise and fall together, as they do with a per-request draft
        # noise.)
        cp = np.cumprod(np.nan_to_num(beta_pad, nan=0.0), axis=1)
        per_req = 1.0 + np.array([cp[b, :g_req[b]].sum() for b in range(B)])
        outcome["tokens_per_round_eq1"] = float(per_req.mean())

    # The GPU's outputs per request, for the oracle check of the CPU leg.
    got = {"out_tokens": out.cpu().numpy(), "num_accepted": n_gpu}
    if wl.entry == "greedy" and not wl.has_settings:
        got["target_argmax"] = ta.cpu().numpy()
    elif wl.entry != "greedy":
        for key, t in (("p_draft", pd), ("q_draft", qd)):
            if key == "q_draft" and wl.entry == "onehot" and not wl.has_settings:
                continue
            flat = t.cpu().numpy()
            if flat.ndim == 1:  # packed ragged rows back to [B, G]
                dense, off = np.full((B, G), np.nan, np.float32), 0
                for b in range(B):
                    dense[b, :g_req[b]] = flat[off:off + g_req[b]]
                    off += g_req[b]
                flat = dense
            got[key] = flat

    return outcome, got


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--rounds", type=int, default=0,
                    help="also run the multi-round driver for this many rounds and report its statistics")
    ap.add_argument("--no-outcome", action="store_true",
                    help="skip the untimed outcome statistics and the oracle check (profiling runs: only the "
                         "warm-up and timed calls run)")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the measured streaming-read ceiling (sv_stream_read over 4 GiB)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for HBM counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (the verifier shards by request "
              f"with no exchange; run one process per GPU on its share)", file=sys.stderr)
        sys.exit(2)

    import torch

    import speculative_decoding_rejection_amd as sv
    import workloads

    name = args.workload or workloads.HEADLINE
    wl = workloads.ALL_WORKLOADS[name]
    dev = torch.device("cuda:0")
    sv.load_library()
    log(f"[bench] {name}: generating inputs on {torch.cuda.get_device_name(0)}")
    inp = workloads.generate(wl, device=dev)
    torch.cuda.synchronize()

    params = sv.make_params(wl.B, wl.G, wl.V, wl.torch_dtype, wl.temperature or 1.0, wl.top_k, wl.verify_seed)
    sampling = layout = None
    dense_inp = inp
    if wl.has_settings:
        sampling = sv.make_sampling(inp["temperature"], inp["top_k"], inp["top_p"], max(k for _, k, _ in wl.mix))
        ws = torch.empty(sv.sv_workspace_bytes_batch(params, sampling), dtype=torch.uint8, device=dev)
        if wl.entry == "match":
            # Token-only drafts (chains or trees), packed before the timed
            # region if ragged.
            src = workloads.pack_ragged(inp, inp["lengths"].cpu()) if wl.lengths else inp
            layout = sv.SvLayout(sv.SV_DRAFT_MATCH, 0, wl.V, 0, sv._ptr(src.get("cu_draft")),
                                 sv._ptr(src.get("parents")))
            inp = dict(inp, target_logits=src["target_logits"], draft_tokens=src["draft_tokens"],
                       cu_draft=src.get("cu_draft"), parents=src.get("parents"))
            torch.cuda.synchronize()
        elif wl.lengths or wl.draft_probs:
            # Packed ragged rows and / or the drafter's probabilities, laid
            # out before the timed region.
            src = inp
            if wl.lengths:
                src = workloads.pack_ragged(inp, inp["lengths"].cpu())
            draft = src["draft_probs"] if wl.draft_probs else src["draft_logits"]
            layout = sv.SvLayout(sv.SV_DRAFT_PROBS if wl.draft_probs else sv.SV_DRAFT_LOGITS, 0, wl.V, wl.V,
                                 sv._ptr(src["cu_draft"]) if wl.lengths else None)
            dense_inp = inp
            inp = dict(inp, target_logits=src["target_logits"], draft_logits=draft,
                       draft_tokens=src["draft_tokens"], cu_draft=src.get("cu_draft"))
            torch.cuda.synchronize()
    else:
        ws = sv.alloc_workspace(params, dev)
    B, G = wl.B, wl.G
    out = torch.empty((B, G + 1), dtype=torch.int32, device=dev)
    nacc = torch.empty((B,), dtype=torch.int32, device=dev)
    pd = torch.empty(inp["draft_tokens"].shape, dtype=torch.float32, device=dev)
    qd = torch.empty(inp["draft_tokens"].shape, dtype=torch.float32, device=dev)
    ta = torch.empty((B, G + 1), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    pn = torch.empty((B, G + 1), dtype=torch.int32, device=dev) if wl.entry == "match" else None
    outputs = sv.make_outputs(out, nacc, pd, qd, path_nodes=pn)
    lt, ld, x = inp["target_logits"], inp["draft_logits"], inp["draft_tokens"]
    # A workload whose logits fit twice in the 256 MB MALL would be read from
    # that cache, not HBM, when called back to back: such calls rotate
    # through enough copies of the inputs (at least 768 MB in all) that each
    # call's rows were evicted since their last use.
    ring = [(lt, ld, x)]
    if wl.logit_bytes < 2 * MALL_BYTES and not wl.has_settings:
        copies = -(-3 * MALL_BYTES // wl.logit_bytes)
        ring += [(lt.clone(), ld.clone() if ld is not None else None, x.clone()) for _ in range(copies - 1)]
        torch.cuda.synchronize()
        log(f"[bench] inputs rotated through {copies} copies ({copies * wl.logit_bytes / 1e6:.0f} MB)")
    n_copies = len(ring)
    it = [0]

    def step():
        lt_, ld_, x_ = ring[it[0] % len(ring)]
        it[0] += 1
        if wl.entry == "prob":
            sv.spec_verify_prob(params, lt_, ld_, x_, out, nacc, pd, qd, ws, stream)
        elif wl.entry == "onehot":
            sv.spec_verify_onehot(params, lt_, x_, out, nacc, pd, ws, stream)
        elif wl.has_settings:
            sv.spec_verify_batch(params, sampling, layout, lt_, ld_, x_, outputs, ws, stream)
        else:
            sv.spec_verify_greedy(params, lt_, x_, out, nacc, ta, ws, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup} steps); timing {args.steps} steps")

    # Timed region: K steps, nothing else enqueued (no per-kernel events: an
    # event record costs host time comparable to a whole small call).
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dev_ms = ev0.elapsed_time(ev1)
    # Kernel durations: the same K steps again, with a pair of HIP events
    # around every launch of the library on its launch stream.
    sv.sv_kernel_timing_reset()
    sv.sv_kernel_timing_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    sv.sv_kernel_timing_enable(False)
    rows_ms, rows_n = sv.sv_kernel_timing_read(sv.FAMILY_ROWS)
    acc_ms, acc_n = sv.sv_kernel_timing_read(sv.FAMILY_ACCEPT)
    race_ms, race_n = sv.sv_kernel_timing_read(sv.FAMILY_RACE)
    log(f"[bench] timed: wall {wall * 1e3:.2f} ms, device {dev_ms:.2f} ms; kernels (second pass) rows "
        f"{rows_ms:.2f} ms/{rows_n}, accept {acc_ms:.2f} ms/{acc_n}, race {race_ms:.2f} ms/{race_n}")

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log("[bench] copy calibration: 3 copies of 1 GiB done")

    ceiling = None
    if not args.no_ceiling:
        del ring[1:]
        torch.cuda.empty_cache()
        ceiling = read_ceiling(sv, dev, stream)
        log(f"[bench] measured streaming-read ceiling {ceiling:.0f} GB/s")

    outcome = got = None
    if not args.no_outcome:
        outcome, got = outcome_stats(sv, wl, params, sampling, layout, lt, ld, x, out, nacc, pd, qd, ta, pn, ws,
                                     stream)

    sec = wall / args.steps
    positions = int(wl.draft_lengths.sum()) if wl.has_settings else B * G
    rows = positions + B  # (request, position) rows: B (G + 1) for a dense call
    logit_rows = wl.target_rows + wl.draft_rows
    bytes_alg = wl.logit_bytes
    # Row-pass time per step: one launch for the single-setting entries; the
    # batch entry's row family (classify, top-k, softmax, argmax, nucleus
    # kernels) is taken as a whole.
    row_step_s = rows_ms / args.steps / 1e3
    achieved = bytes_alg / row_step_s / 1e9
    traffic = load_traffic(name, bytes_alg)
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(wl, dense_inp, args.cpu_seconds, got=got)
    res = {
        "metric": "verified draft positions/sec and HBM GB/s (% of peak) at B=1024,gamma=8,V=256k",
        "value": positions / sec,
        "unit": "verified draft positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": sec * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded, generated on the GPU; no dataset)",
        "config": {"workload": name, "entry": f"spec_verify_{wl.entry}", "batch": B, "gamma": G, "vocab": wl.V,
                   "logits": wl.dtype, "temperature": wl.temperature, "top_k": wl.top_k,
                   "parallelism": "single GPU",
                   **({"mix (T, top_k, top_p)": [list(m) for m in wl.mix]} if wl.has_settings else {}),
                   **({"draft": "tokens only (sampler-match)"} if wl.entry == "match" else {}),
                   **({"tree parents": list(wl.parents)} if wl.parents else {}),
                   **({"draft lengths": list(wl.lengths)} if wl.lengths else {}),
                   **({"draft": "fp32 probabilities"} if wl.draft_probs else {})},
        "rows_per_s": rows / sec,
        "logit_rows_per_s": logit_rows / sec,
        "requests_per_s": B / sec,
        "input_copies_rotated": n_copies if n_copies > 1 else None,
        "algorithmic_gbps": bytes_alg / sec / 1e9,
        "hbm_fraction": bytes_alg / sec / 1e9 / HBM_PEAK_GBPS,
        "kernels_ms_per_step": {"rows": rows_ms / args.steps, "accept": acc_ms / args.steps,
                                "race": race_ms / args.steps},
        "roofline": {"bound": "hbm", "kernel": ("row pass (rows_topk_kernel)" if wl.top_k else
                                                "row family (all row kernels of a step)" if wl.has_settings
                                                else "row pass"),
                     "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": traffic, "measured_read_ceiling": ceiling,
                     "frac_of_measured_ceiling": achieved / ceiling if ceiling else None},
        "cpu_baseline": cpu,
        "outcome": outcome,
    }
    if args.rounds:
        log(f"[bench] multi-round driver: {args.rounds} rounds")
        st = rounds_driver(sv, wl, args.rounds, dev)
        res["rounds"] = {k: v for k, v in st.items() if not k.startswith("_")}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
