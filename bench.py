#!/usr/bin/env python3
"""Throughput of the MI355X WFST beam-search decoder on one GPU.

A step is one whole decode (wfst_decode) of the synthetic HLG-scale batch: 32
utterances of 300-500 frames (fp16 log-probs [32, 500, 5000]) over a 2M-state,
21M-arc power-law graph, beam 20, max_active 10000. Inputs are resident in HBM
before the timed region; a decode's host work (one 24-byte descriptor copy in,
one result copy out) is inside it.

Prints one JSON line: decoded frames/s (value), arcs expanded/s, the achieved
fraction of the HBM roofline for the dominant kernel (algorithmic bytes per
launch over its average launch time, from hipEvents recorded between the
decoder's launches in a second, instrumented pass of the same K decodes), and
the CPU oracle's frames/s on a bounded sample of lanes (test infrastructure,
single thread). The line's ``configs`` object repeats the measurement for every
other synthetic workload at full size (frames/s, arcs/s, the method's bytes per
second against the HBM peak, the oracle on one core beside it).
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

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
PROFILES = os.path.join(ROOT, "profiles")


# kernels of the epsilon closure, timed and charged as one group
CLOSURE_KERNELS = ("eps_expand", "eps_apply", "eps_apply_expand")


def algorithmic_bytes(st, elem_bytes, vocab):
    """Bytes the method must move per decode, from the device step counters.

    Per-unit figures (what the method itself reads or writes once, single pass):
    n tokens expanded, S candidate arcs, C admitted candidates, D distinct
    admitted destinations (the winners), n' survivors (next-frontier tokens the
    compaction writes; n' = D), F lane-frames, e*V one log-prob row; on graphs
    with epsilon arcs E epsilon arcs relaxed, Ce admitted, De distinct, Ne tokens
    appended or replaced by the closure.

      max       20 n + 6 S + 12 C + e V F   (token state / score / entry 12 B and its arc
                                             range 8 B; ilabel u16 + weight f32 per arc;
                                             dest i32 + one u64 recombination atomic per
                                             admitted candidate; one row per lane-frame)
      finalize  28 D + 20 n'                (per destination: key 4 B, payload read-back
                                             12 B, targeted clear 12 B; per survivor the
                                             token 12 B + winners-log entry 8 B)
      closure   8 E + 12 Ce + 28 De + 20 Ne (weight + dest per epsilon arc; the same
                                             per-candidate, per-destination and per-token
                                             terms as a real step)

    The path figure is their sum. ``design`` counts what this implementation's
    own choices add on top (the 16-byte candidate record written by the slot
    pass for every listed candidate and read back by the compaction, the
    compaction's 128-byte state record per new token, the 16-byte token record
    the slot pass reads): reported beside the method's bytes, never in them.
    """
    n, S, C, D, F = st["tokens"], st["arcs"], st["admitted"], st["distinct"], st["lane_frames"]
    E, Ce, De, Ne = st["eps_arcs"], st["eps_admitted"], st["eps_distinct"], st["eps_changed"]
    row = elem_bytes * vocab * F
    per = {
        "max": 20 * n + 6 * S + 12 * C + row,
        "finalize": 28 * D + 20 * D,
        # the closure's kernels (a pass's relaxation, its resolution, and the
        # launches that resolve pass k while they relax pass k + 1) as one group
        "closure": 8 * E + 12 * Ce + 28 * De + 20 * Ne,
    }
    path = sum(per.values())
    design = {"candidate_records": 32 * st["listed"], "state_records": 128 * D, "token_records": 16 * n}
    return per, path, design


def graph_kind(wl):
    """What the synthetic graph of workload ``wl`` stands for."""
    if wl.epsilon:
        return "synthetic TLG-style graph with epsilon arcs"
    return "synthetic HLG-scale graph" if wl.num_states >= 1_000_000 else "synthetic HLG-style graph"


def degree_kind(wl):
    kind = wl.degree[0]
    if kind == "power":
        return f"power-law out-degree (alpha {wl.degree[1]}, {wl.degree[2]}-{wl.degree[3]})"
    if kind == "geom":
        return f"geometric out-degree (p {wl.degree[1]}, cap {wl.degree[2]})"
    return f"uniform out-degree {wl.degree[1]}-{wl.degree[2]}"


def measure_copy_gbps(dev, mib=1024, reps=5):
    """Bandwidth of a plain device-to-device copy on this GPU (bytes read plus
    bytes written per second), the measured companion of the 8 TB/s peak."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    s = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(s)
    for _ in range(reps):
        dst.copy_(src)
    b.record(s)
    b.synchronize()
    ms = a.elapsed_time(b) / reps
    del src, dst
    return round(2 * n / (ms * 1e-3) / 1e9, 1)


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("wfst_kernels.hip", "wfst_internal.h"):
        with open(os.path.join(ROOT, "wfst_beam_search_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel, workload_name):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary,
    when it was taken on the current kernel source; else None."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get(workload_name, {}).get(kernel)
    if not ent or ent.get("kernel_source") != kernel_source_hash():
        return None
    return ent.get("bytes_per_launch")


def cpu_baseline(graph, lp, lengths, wl, seconds, gpu=None, allow_partial=False):
    """The oracle on one pinned core over the batch's first lanes for about
    ``seconds``; with ``gpu`` (the timed run's last result) each of those lanes
    is also compared with it: arcs and words equal, score bits equal."""
    import numpy as np

    import oracle
    cpus = os.sched_getaffinity(0)
    os.sched_setaffinity(0, {sorted(cpus)[0]})
    og = oracle.OracleGraph(graph)
    frames = arcs = 0
    lanes = same = 0
    t0 = time.perf_counter()
    for b in range(lp.shape[0]):
        r = oracle.decode_lane(og, lp[b], int(lengths[b]), wl.beam, wl.max_active,
                               allow_partial=allow_partial, eps_iterations=wl.eps_iterations)
        frames += int(lengths[b])
        arcs += int(r["steps"][:, 4].sum() + r["steps"][:, 7].sum())
        lanes += 1
        if gpu is not None:
            same += int(np.array_equal(gpu.arcs[b], r["arcs"]) and np.array_equal(gpu.words[b], r["words"]) and
                        np.float32(gpu.scores[b]).tobytes() == np.float32(r["score"]).tobytes() and
                        int(gpu.meta[b, 1]) == int(r["reached_final"]))
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    os.sched_setaffinity(0, cpus)
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": frames / dt, "unit": "frames/s", "cores": 1, "kind": "oracle",
            "arcs_per_s": arcs / dt,
            **({} if gpu is None else {"gpu_lanes_identical": f"{same}/{lanes}"}),
            "sample": f"lanes 0..{lanes - 1} of the {wl.name} batch ({frames} frames, {dt:.1f} s, "
                      f"single-threaded C oracle pinned to one core; host nproc {os.cpu_count()}, {model})"}


def cpu_baseline_all_cores(graph, lp, lengths, wl, allow_partial=False, threads=16):
    """The oracle over every lane of the batch, one lane per thread at a time on
    up to ``threads`` of the host's cores (the oracle is plain C called through
    ctypes, which releases the interpreter lock, and keeps no global state):
    the host's throughput with lanes in parallel, beside the one-core figure."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    og = oracle.OracleGraph(graph)
    n = max(1, min(threads, len(os.sched_getaffinity(0))))

    def one(b):
        oracle.decode_lane(og, lp[b], int(lengths[b]), wl.beam, wl.max_active,
                           allow_partial=allow_partial, eps_iterations=wl.eps_iterations)
        return int(lengths[b])

    one(0)   # (loads the library before the threads start)
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=n) as ex:
        frames = sum(ex.map(one, range(lp.shape[0])))
    dt = time.perf_counter() - t0
    return {"value": frames / dt, "unit": "frames/s", "cores": n, "kind": "oracle",
            "sample": f"all {lp.shape[0]} lanes of the {wl.name} batch ({frames} frames, {dt:.1f} s), "
                      f"{n} threads, lanes in parallel"}


def stream_bench(args, wl, graph, lp, lengths, dev):
    """Streams the workload's utterances (one stream per lane, all lanes advanced
    together chunk by chunk, then finalized): a step is the whole batch streamed.
    The chunks are packed on the device before the timed region."""
    import numpy as np
    import torch

    import wfst_beam_search_amd as wb

    B, T, V = lp.shape
    N = args.stream_chunk
    P = wl.eps_iterations if graph.epsilon_id >= 0 else 0
    arena = min(max(1 << 20, 4 * wl.max_active * (T + 2) * (1 + P)), ((1 << 31) - 1) // B)
    dg = wb.Graph(graph, device=0)
    if args.arena:
        arena = args.arena
    dec = wb.Decoder(dg, wl.beam, wl.max_active, max_lanes=B, max_frames=N, lp_dtype=wl.dtype,
                     eps_iterations=wl.eps_iterations, use_graphs=not args.eager, grid_blocks=args.grid,
                     path_cap=(T + 2) * (1 + P), arena_entries=arena, gc_interval=args.gc_interval)
    x = torch.from_numpy(lp).to(dev)
    chunks = []
    for s in range(0, T, N):
        lens = np.clip(np.asarray(lengths) - s, 0, N).astype(np.int32)
        if lens.max() == 0:
            break
        live = [b for b in range(B) if lens[b] > 0]
        xc = x[live, s:s + N].contiguous()
        if xc.shape[1] < N:
            xc = torch.cat([xc, torch.zeros((len(live), N - xc.shape[1], V), dtype=xc.dtype, device=dev)], 1)
        chunks.append((live, xc, lens[live]))
    torch.cuda.synchronize()

    phase = [0.0, 0.0, 0.0]   # seconds in create, advance, finalize + release calls

    def one():
        ta = time.perf_counter()
        ch = dec.create_streams(B) if args.stream_together else [dec.create_stream() for _ in range(B)]
        tb = time.perf_counter()
        for live, xc, lens in chunks:
            dec.advance_chunk([ch[b] for b in live], xc, lens, want_partial=args.stream_partial)
        tc = time.perf_counter()
        if args.stream_together:
            r = dec.finalize_streams(ch)
            res = [r.meta[j:j + 1] for j in range(len(ch))]
        else:
            res = [dec.finalize_stream(c).meta for c in ch]
        for c in ch:
            dec.release_stream(c)
        td = time.perf_counter()
        phase[0] += tb - ta
        phase[1] += tc - tb
        phase[2] += td - tc
        return res

    for _ in range(args.warmup):
        one()
    torch.cuda.synchronize()
    phase[:] = [0.0, 0.0, 0.0]
    t0 = time.perf_counter()
    for _ in range(args.steps):
        res = one()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    frames = int(np.asarray(lengths).sum())
    ok = all(int(m[0, 0]) == 1 and int(m[0, 2]) == 0 for m in res)
    ktimes = {}
    if not args.no_profile_pass:
        dec.profile(True)
        acc = {}
        ch = [dec.create_stream() for _ in range(B)]
        for live, xc, lens in chunks:
            dec.advance_chunk([ch[b] for b in live], xc, lens, want_partial=args.stream_partial)
            for k, (ms, cnt) in dec.kernel_times().items():
                a = acc.setdefault(k, [0.0, 0])
                a[0] += ms
                a[1] += cnt
        for c in ch:
            dec.finalize_stream(c)
            dec.release_stream(c)
        dec.profile(False)
        ktimes = {k: {"total_ms_per_decode": v[0], "launches_per_decode": v[1],
                      "avg_launch_us": (v[0] / v[1] * 1e3) if v[1] else 0.0} for k, v in acc.items() if v[1]}
    line = {
        "metric": "streamed frames/sec at 1 GPU (every lane a stream, advanced chunk by chunk)",
        "value": round(frames * args.steps / dt, 2), "unit": "frames/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(dt / args.steps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{wl.name} streamed in chunks of {N} frames"
                               f"{' with partial hypotheses after each chunk' if args.stream_partial else ''}"
                               f"{', all opened by one call and ended by one' if args.stream_together else ''}: "
                               f"{graph.num_states - 1} states, {graph.num_arcs} arcs, log_prob {wl.dtype} "
                               f"[{B},{T},{V}], lengths {wl.lengths[0]}-{wl.lengths[1]}",
                   "batch": B, "frames": T, "vocab": V, "chunk": N, "chunk_calls_per_step": len(chunks),
                   "beam": wl.beam, "max_active": wl.max_active,
                   "execution": "per-phase kernels, " + ("eager" if args.eager else "hipGraph replay per chunk")},
        "ms_per_chunk_call": round(phase[1] / args.steps / max(len(chunks), 1) * 1e3, 4),
        "ms_per_step_by_call": {"create": round(phase[0] / args.steps * 1e3, 3),
                                "advance": round(phase[1] / args.steps * 1e3, 3),
                                "finalize_release": round(phase[2] / args.steps * 1e3, 3)},
        "parity_meta_ok": ok,
        "roofline": None,
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)
    if args.report:
        with open(args.report, "w") as f:
            json.dump({"line": line, "kernels": ktimes, "kernel_source": kernel_source_hash()}, f, indent=1)
    dec.close()
    dg.release()


def blank_skip_bench(args, wl, graph, lp, lengths, dev):
    """Blank-skip pre-slicing of the whole batch per timed step: the blank column
    read for every frame, kept rows copied, the rest of the output zeroed."""
    import numpy as np
    import torch

    import wfst_beam_search_amd as wb
    B, T, V = lp.shape
    dg = wb.Graph(graph, device=0)
    dec = wb.Decoder(dg, wl.beam, wl.max_active, max_lanes=B, max_frames=T, lp_dtype=wl.dtype,
                     eps_iterations=wl.eps_iterations, arena_entries=1 << 16, arena_commit=-1)
    x = torch.from_numpy(lp).to(dev)
    blank = 0
    for _ in range(args.warmup):
        dec.blank_skip(x, lengths, blank, args.blank_skip)
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(s)
        _, kept = dec.blank_skip(x, lengths, blank, args.blank_skip)   # returns after its stream finished
        b.record(s)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    gpu_ms = sum(a.elapsed_time(b) for a, b in ev) / args.steps
    elem = 2 if wl.dtype == "f16" else 4
    frames = int(np.asarray(lengths).sum())
    nk = int(np.asarray(kept).sum())
    # blank value of every frame, kept rows read and written, the other rows zeroed
    nbytes = frames * elem + 2 * nk * V * elem + (B * T - nk) * V * elem
    achieved = nbytes / (gpu_ms * 1e-3) / 1e9
    line = {
        "metric": "blank-skip pre-slicing throughput at 1 GPU (frames in per second)",
        "value": round(frames * args.steps / dt, 1), "unit": "frames/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(dt / args.steps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": f"{wl.name} log_prob {wl.dtype} [{B},{T},{V}], lengths "
                               f"{wl.lengths[0]}-{wl.lengths[1]}, blank id {blank}, threshold {args.blank_skip}",
                   "batch": B, "frames": T, "vocab": V},
        "kept_frames": nk, "input_frames": frames,
        "gpu_ms_per_call": round(gpu_ms, 4),
        "roofline": {"bound": "hbm", "kernel": "blank_scan + blank_copy (one call)", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None, "bytes_per_launch": int(nbytes)},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)
    dec.close()
    dg.release()


def config_summary(wid, steps, warmup, cpu_seconds, dev):
    """One of the five workloads at full size: decode throughput (captured graph,
    inputs resident), the method's algorithmic bytes per second against the HBM
    peak, and the oracle on one core over the batch's first lanes, each of which
    is compared with the GPU's result."""
    import numpy as np
    import torch

    import synth
    import wfst_beam_search_amd as wb

    wl = synth.WORKLOADS[wid]
    graph, lp, lengths = synth.workload_inputs(wid)
    B, T, V = lp.shape
    dg = wb.Graph(graph, device=0)
    dec = wb.Decoder(dg, wl.beam, wl.max_active, max_lanes=B, max_frames=T, lp_dtype=wl.dtype,
                     eps_iterations=wl.eps_iterations, arena_commit=-1)
    x = torch.from_numpy(lp).to(dev)
    torch.cuda.synchronize()
    for _ in range(warmup):
        dec.decode(x, lengths)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        res = dec.decode(x, lengths)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    st = dec.stats()
    frames = int(np.asarray(lengths).sum())
    elem = 2 if wl.dtype == "f16" else 4
    _, path_bytes, _ = algorithmic_bytes(st, elem, V)
    ok = bool((res.meta[:, 0] == 1).all() and (res.meta[:, 2] == 0).all())
    dec.close()
    dg.release()
    del x
    torch.cuda.empty_cache()
    out = {"workload": f"{wl.name}: {graph.num_states - 1} states, {graph.num_arcs} arcs, log_prob {wl.dtype} "
                       f"[{B},{T},{V}], lengths {wl.lengths[0]}-{wl.lengths[1]}, beam {wl.beam}, "
                       f"max_active {wl.max_active}" + (f", {wl.eps_iterations} closure passes" if wl.epsilon else ""),
           "frames_per_s": round(frames * steps / dt, 1),
           "arcs_expanded_per_s": round((st["arcs"] + st["eps_arcs"]) * steps / dt, 1),
           "ms_per_decode": round(dt / steps * 1e3, 4),
           "path_algorithmic_GBps": round(path_bytes * steps / dt / 1e9, 2),
           "path_hbm_frac": round(path_bytes * steps / dt / 1e9 / HBM_PEAK_GBS, 5),
           "parity_meta_ok": ok, "steps": steps, "warmup": warmup}
    if cpu_seconds > 0:
        cb = cpu_baseline(graph, lp, lengths, wl, cpu_seconds, gpu=res)
        out["oracle_1core_frames_per_s"] = round(cb["value"], 1)
        out["oracle_gpu_lanes_identical"] = cb["gpu_lanes_identical"]
    return out


def run_probes() -> dict:
    """Machine probes (libwfst_probe.so, built with the decoder): the random-line
    rate, the latency of a dependent load, posted 64-bit atomics, the launch
    floor, and returning atomics on few hot counters on this GPU."""
    import ctypes
    import torch
    torch.cuda.init()
    lib = ctypes.CDLL(os.path.join(ROOT, "wfst_beam_search_amd", "libwfst_probe.so"))
    out = (ctypes.c_double * 32)()
    rc = lib.wfst_probe_run(out, 32)
    if rc != 0:
        raise RuntimeError(f"wfst_probe_run failed ({rc})")
    v = list(out)
    res = {"gather": [], "atomic_max_u64": []}
    for j, mb in enumerate((4, 32, 128, 512, 1024, 4096)):
        us, glines, lvl = v[3 * j: 3 * j + 3]
        res["gather"].append({"footprint_mib": mb, "us_per_launch": round(us, 2),
                              "random_lines_per_s_G": round(glines, 2), "dependent_level_us": round(lvl, 3),
                              "loads_per_launch": 1024 * 256 * 4})
    for j, mb in enumerate((8, 512)):
        us, gat = v[18 + 2 * j: 20 + 2 * j]
        res["atomic_max_u64"].append({"table_mib": mb, "us_per_launch": round(us, 2),
                                      "atomics_per_s_G": round(gat, 2), "atomics_per_launch": 1024 * 256})
    res["launch_floor_us"] = {"eager": round(v[22], 3), "graph_replay": round(v[23], 3)}
    res["hot_counter_atomic_us"] = [{"counters": nc, "wavefronts": 4096, "mean": round(v[24 + 2 * j], 3),
                                     "max": round(v[25 + 2 * j], 3)} for j, nc in enumerate((1, 8, 32, 4096))]
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", type=int, default=3, help="synthetic workload id (1-5); 3 = HLG-scale")
    ap.add_argument("--eager", action="store_true", help="plain launches instead of the captured graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--cpu-all-cores", type=int, default=1,
                    help="1: also time the oracle over every lane with lanes in parallel on up to 16 cores")
    ap.add_argument("--grid", type=int, default=0, help="workgroups per frame-loop launch (0: derive)")
    ap.add_argument("--no-profile-pass", action="store_true")
    ap.add_argument("--report", default="", help="also write a detailed JSON report here")
    ap.add_argument("--lattice", type=float, default=None, metavar="OUTPUT_BEAM",
                    help="lattice mode: keep every admitted arc and prune with this output beam")
    ap.add_argument("--lat-prune-interval", type=int, default=0, metavar="N",
                    help="with --lattice: the interval prune every N steps")
    ap.add_argument("--sparse-finals", type=float, default=None, metavar="KEEP",
                    help="keep each state's final arc with probability KEEP (allow_partial on: lanes "
                         "without a final arc at their end redirect to their best token)")
    ap.add_argument("--recomb-slots", type=int, default=0, metavar="SLOTS",
                    help="recombination through a per-lane open-addressing hash of SLOTS slots "
                         "(power of 2) instead of the direct-mapped per-state table")
    ap.add_argument("--gc-interval", type=int, default=0, metavar="N",
                    help="compact the winners log every N steps (and per stream chunk)")
    ap.add_argument("--arena", type=int, default=0, metavar="ENTRIES",
                    help="winners-log entries per lane (0: the decoder's default)")
    ap.add_argument("--arena-commit", type=int, default=-1, metavar="ENTRIES",
                    help="winners-log entries per lane committed at creation (-1, the default "
                         "here: the whole region, so no warm-up decode is cut short and run again "
                         "and every counted dispatch belongs to a whole decode; 0: the decoder's "
                         "lazy default)")
    ap.add_argument("--stream-chunk", type=int, default=0, metavar="N",
                    help="stream every lane in chunks of N frames (create / advance / finalize / "
                         "release per timed step) instead of one batch decode")
    ap.add_argument("--stream-together", action="store_true",
                    help="with --stream-chunk: open every stream of the batch with one wfst_create_streams call "
                         "and end them with one wfst_finalize_streams call")
    ap.add_argument("--stream-partial", action="store_true",
                    help="with --stream-chunk: ask for every lane's partial hypothesis after each chunk")
    ap.add_argument("--blank-skip", type=float, default=None, metavar="THRESHOLD",
                    help="time blank-skip pre-slicing of the workload's log_prob (frames whose blank "
                         "probability exceeds THRESHOLD dropped) instead of a decode")
    ap.add_argument("--configs", default="1,2,4,5", metavar="IDS",
                    help="also run these workloads at full size after the headline one (comma list; "
                         "empty: none) and report them in the line's `configs` object")
    ap.add_argument("--config-steps", type=int, default=5, help="timed decodes per extra workload")
    ap.add_argument("--probe", action="store_true",
                    help="only run the machine probes (random gathers over 4 MiB - 4 GiB, dependent "
                         "load chains, posted 64-bit atomics, the launch floor) and print them as JSON")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB three times (scales rocprofv3 "
                         "FETCH_SIZE / WRITE_SIZE readings to bytes)")
    args = ap.parse_args()
    if args.probe:
        print(json.dumps(run_probes()))
        return
    if args.calibrate_copy:
        import torch
        n = args.calibrate_copy << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 3}))
        return
    if args.gpus != 1:
        print("bench.py: this decoder runs on one GPU; utterances shard across GPUs with no "
              "exchange, so there is no multi-GPU step to time (use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import wfst_beam_search_amd as wb

    wl = synth.WORKLOADS[args.workload]
    graph, lp, lengths = synth.workload_inputs(args.workload)
    if args.sparse_finals is not None:
        # keep each state's final arc with this probability; lanes that end
        # without one redirect to their best token (allow_partial)
        graph = synth.drop_finals(graph, 4000 + args.workload, args.sparse_finals)
    B, T, V = lp.shape
    dev = torch.device("cuda:0")
    if args.stream_chunk > 0:
        stream_bench(args, wl, graph, lp, lengths, dev)
        return
    if args.blank_skip is not None:
        blank_skip_bench(args, wl, graph, lp, lengths, dev)
        return
    dg = wb.Graph(graph, device=0)
    lat = {} if args.lattice is None else dict(lattice=True, output_beam=args.lattice,
                                               lat_prune_interval=args.lat_prune_interval)
    lat.update(gc_interval=args.gc_interval, arena_entries=args.arena, arena_commit=args.arena_commit)
    dec = wb.Decoder(dg, wl.beam, wl.max_active, max_lanes=B, max_frames=T, lp_dtype=wl.dtype,
                     eps_iterations=wl.eps_iterations, use_graphs=not args.eager,
                     grid_blocks=args.grid, allow_partial=args.sparse_finals is not None,
                     recomb_slots=args.recomb_slots, **lat)
    x = torch.from_numpy(lp).to(dev)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        dec.decode(x, lengths)
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    per_decode = []
    for _ in range(args.steps):
        ta = time.perf_counter()
        res = dec.decode(x, lengths)      # returns after its stream has finished
        per_decode.append(time.perf_counter() - ta)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    st = dec.stats()
    copy_gbps = measure_copy_gbps(dev)

    frames = int(np.asarray(lengths).sum())
    ms_per_step = dt / args.steps * 1e3
    fps = frames * args.steps / dt
    arcs_ps = (st["arcs"] + st["eps_arcs"]) * args.steps / dt
    ok = bool((res.meta[:, 0] == 1).all() and (res.meta[:, 2] == 0).all())
    elem = 2 if wl.dtype == "f16" else 4
    per_kernel_bytes, path_bytes, design_bytes = algorithmic_bytes(st, elem, V)

    roofline = None
    ktimes = {}
    prof_ms = None
    if not args.no_profile_pass:
        dec.profile(True)
        dec.decode(x, lengths)            # capture the instrumented graph
        torch.cuda.synchronize()
        acc = {}
        tp = time.perf_counter()
        for _ in range(args.steps):
            dec.decode(x, lengths)
            for k, (ms, cnt) in dec.kernel_times().items():
                a = acc.setdefault(k, [0.0, 0])
                a[0] += ms
                a[1] += cnt
        torch.cuda.synchronize()
        prof_ms = (time.perf_counter() - tp) / args.steps * 1e3
        dec.profile(False)
        ktimes = {k: {"total_ms_per_decode": v[0] / args.steps, "launches_per_decode": v[1] // args.steps,
                      "avg_launch_us": (v[0] / v[1] * 1e3) if v[1] else 0.0} for k, v in acc.items()}
        cl = [ktimes[k] for k in CLOSURE_KERNELS if k in ktimes and ktimes[k]["launches_per_decode"]]
        if cl:
            tot = sum(x["total_ms_per_decode"] for x in cl)
            nl = sum(x["launches_per_decode"] for x in cl)
            ktimes["closure"] = {"total_ms_per_decode": tot, "launches_per_decode": nl,
                                 "avg_launch_us": tot / nl * 1e3 if nl else 0.0}
        dom = max((k for k in ktimes if k in per_kernel_bytes), key=lambda k: ktimes[k]["total_ms_per_decode"])
        launches = ktimes[dom]["launches_per_decode"]
        avg_s = ktimes[dom]["avg_launch_us"] * 1e-6
        bpl = per_kernel_bytes[dom] / max(launches, 1)
        achieved = bpl / avg_s / 1e9 if avg_s > 0 else 0.0
        roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 5),
                    "traffic": traffic_from_profiles(dom, wl.name),
                    "bytes_per_launch": int(bpl), "avg_launch_us": round(ktimes[dom]["avg_launch_us"], 3)}

    cpu = cpu_all = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(graph, lp, lengths, wl, args.cpu_seconds, gpu=res,
                           allow_partial=args.sparse_finals is not None)
        if args.cpu_all_cores:
            cpu_all = cpu_baseline_all_cores(graph, lp, lengths, wl, allow_partial=args.sparse_finals is not None)

    configs = {}
    others = [int(c) for c in args.configs.split(",") if c.strip()] if args.configs else []
    others = [c for c in others if c != args.workload and c in synth.WORKLOADS]
    if (others and args.lattice is None and not args.gc_interval and not args.eager and args.sparse_finals is None
            and not args.recomb_slots):
        # the other workloads (each its own decoder, released before the next)
        dec.close()
        dg.release()
        del x
        torch.cuda.empty_cache()
        dec = dg = None
        cpu_s = {1: 2.0, 2: 3.0, 3: 10.0, 4: 6.0, 5: 4.0}
        for c in others:
            configs[str(c)] = config_summary(c, args.config_steps, min(args.warmup, 2),
                                             0.0 if args.no_cpu_baseline else cpu_s.get(c, 3.0), dev)
            print(f"bench.py: workload {c} done", file=sys.stderr, flush=True)
        # the headline workload's own entry, from the run above
        configs[str(args.workload)] = {
            "workload": wl.name, "frames_per_s": round(fps, 1), "arcs_expanded_per_s": round(arcs_ps, 1),
            "ms_per_decode": round(ms_per_step, 4),
            "path_algorithmic_GBps": round(path_bytes * args.steps / dt / 1e9, 2),
            "path_hbm_frac": round(path_bytes * args.steps / dt / 1e9 / HBM_PEAK_GBS, 5),
            "parity_meta_ok": ok, "steps": args.steps, "warmup": args.warmup,
            **({} if cpu is None else {"oracle_1core_frames_per_s": round(cpu["value"], 1),
                                       "oracle_gpu_lanes_identical": cpu["gpu_lanes_identical"]})}
        configs = {k: configs[k] for k in sorted(configs, key=int)}

    line = {
        "metric": "decoded frames/sec and arcs expanded/sec at 1 GPU; % of HBM peak",
        "value": round(fps, 2), "unit": "frames/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": f"{wl.name}: {graph_kind(wl)} ({graph.num_states - 1} states, "
                               f"{graph.num_arcs} arcs, {degree_kind(wl)}), log_prob {wl.dtype} "
                               f"[{B},{T},{V}], lengths {wl.lengths[0]}-{wl.lengths[1]}",
                   "batch": B, "frames": T, "vocab": V, "beam": wl.beam, "max_active": wl.max_active,
                   "log_prob_dtype": wl.dtype, "score_dtype": "f32",
                   "execution": "per-phase kernels, eager" if args.eager else "per-phase kernels, hipGraph replay",
                   **({} if args.lattice is None else {"lattice_output_beam": args.lattice}),
                   **({} if not args.lat_prune_interval else {"lat_prune_interval": args.lat_prune_interval}),
                   **({} if args.sparse_finals is None else {"final_arc_keep": args.sparse_finals,
                                                             "allow_partial": True}),
                   **({} if not args.recomb_slots else {"recombination": f"hash, {args.recomb_slots} slots per lane"}),
                   **({} if not args.gc_interval else {"gc_interval": args.gc_interval}),
                   **({} if not args.arena else {"arena_entries": args.arena})},
        "arcs_expanded_per_s": round(arcs_ps, 1),
        "ms_per_decode_median_min_max": [round(float(np.median(per_decode)) * 1e3, 4),
                                         round(min(per_decode) * 1e3, 4), round(max(per_decode) * 1e3, 4)],
        "hbm_copy_GBps_measured": copy_gbps,
        "path_algorithmic_GBps": round(path_bytes * args.steps / dt / 1e9, 2),
        "path_hbm_frac": round(path_bytes * args.steps / dt / 1e9 / HBM_PEAK_GBS, 5),
        "path_bytes_per_decode": int(path_bytes),
        "design_bytes_per_decode": {k: int(v) for k, v in design_bytes.items()},
        "parity_meta_ok": ok,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if cpu_all is not None:
        line["cpu_baseline_all_cores"] = cpu_all
    if configs:
        line["configs"] = configs
    line["log_entries_at_end"] = int(st["log_entries"])
    line["log_bytes_committed"] = int(st["log_committed_bytes"])
    line["log_bytes_reserved"] = int(st["log_reserved_bytes"])
    if args.lattice is not None:
        line["lattice_kept_arcs"] = int(sum(dec.lattice(b).shape[0] for b in range(B)))
        line["lattice_arcs"] = int(st["admitted"])
    print(json.dumps(line), flush=True)
    if args.report:
        with open(args.report, "w") as f:
            json.dump({"line": line, "stats": st, "kernels": ktimes, "per_kernel_bytes": per_kernel_bytes,
                       "path_bytes": path_bytes, "profiled_ms_per_step": prof_ms,
                       "kernel_source": kernel_source_hash()}, f, indent=1)
    if dec is not None:
        dec.close()
        dg.release()


if __name__ == "__main__":
    main()
