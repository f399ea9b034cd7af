"""Benchmark: batched spec-verify + SAM-draft steps on one MI355X.

One step = verify the current drafts, extend every automaton with the
emitted tokens and draft for the next step, over the whole batch (one
spec_step call: the HBM stream pass, then the per-sequence finish pass), on
the workload B=256, V=151936, K=3, T=1.0 with one-hot SAM drafts and 8,192-
token histories (copy process, p_copy 0.6, span mean 8). Target logits are
fp32 N(0, 2) noise from a ring of 4 device-resident slots (2.5 GB, far beyond
the 256 MB Infinity Cache) with +4 on the true next token; a tiny harness
kernel applies that boost before each verify (it is the stand-in for the
target model and sits inside the timed loop, so the reported rate is
conservative). Inputs are resident in HBM when timing starts.

Prints one JSON line (see the keys below). `roofline` is for the dominant
kernel (the stream pass): algorithmic bytes = rows verified x V x 4, timed
with HIP events recorded on the launch stream in a second pass that issues
the same steps as spec_stream + spec_finish, around back-to-back batches of
stream launches (per-launch time = event interval / batch size).
`cpu_baseline` is the oracle (C++, double precision, std::map automata) on the
host cores, on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("spec-verify+SAM-draft steps/s at B=256,V=152k,K=3; "
          "achieved HBM GB/s")
PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E, AMD's published figure
INFINITY_CACHE_BYTES = 256 << 20
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "spec_stream_c3_traffic.json")


STREAM_SOURCES = ("stream.hip", "stream_row.h", "verify_common.h", "internal.h")


def stream_source_hash() -> str:
    """Digest of the sources the stream kernel is written in; a traffic
    record taken on other sources is stale."""
    h = hashlib.sha256()
    for name in STREAM_SOURCES:
        p = os.path.join(ROOT, "sam_drafting_lossless_amd", "csrc", name)
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def _traffic_from_profile(rows_per_launch: float):
    """HBM bytes per stream launch from the committed rocprofv3 counter
    record, scaled from the rows of the profiled launches to the rows of this
    run's launches; None if the record was taken on other stream sources."""
    try:
        rec = json.load(open(PROFILE_TRAFFIC))
    except (OSError, ValueError):
        return None
    if rec.get("stream_sources_sha256_16") != stream_source_hash():
        return None
    return rec["hbm_bytes_per_row"] * rows_per_launch


def cpu_baseline(slot_host, gt, cfg, nthreads: int, budget_s: float = 10.0):
    """Times the oracle's whole step (draft, verify, extend) over all B
    sequences on one host copy of a boosted logit slot, with `nthreads`
    threads over sequences for about budget_s seconds; then a shorter
    single-thread run, and a split of one step's time between verification
    and the automata. Returns (baseline line, detail)."""
    import numpy as np

    import oracle
    import synth
    H = cfg.hist_len
    T = np.full(cfg.B, cfg.T, np.float32)

    def run(nthreads, budget, cap):
        sams = [oracle.SAM(gt[b, :H]) for b in range(cfg.B)]
        steps = 0
        t0 = time.perf_counter()
        while True:
            u = synth.uniforms(cfg, 10_000 + steps)
            oracle.step(sams, slot_host, T, u, nthreads=nthreads)
            steps += 1
            el = time.perf_counter() - t0
            if el >= budget or steps >= cap:
                return steps, el, sams

    steps, el, sams = run(nthreads, budget_s, 5000)
    steps1, el1, _ = run(1, budget_s / 4, 5000)
    # Split: drafts from the automata, verification, then the extension, on
    # the automata the main run left behind.
    t_sam = t_ver = 0.0
    nsplit = 10
    for i in range(nsplit):
        t0 = time.perf_counter()
        dr = [s.draft(cfg.K) for s in sams]
        t1 = time.perf_counter()
        d = np.stack([x[0] for x in dr]).astype(np.int32)
        dl = np.array([x[1] for x in dr], np.int32)
        u = synth.uniforms(cfg, 20_000 + i)
        r = oracle.verify(slot_host, d, dl, T, u, nthreads=nthreads)
        t2 = time.perf_counter()
        for b, s in enumerate(sams):
            s.extend(r.out_tokens[b, :r.num_emitted[b]])
        t3 = time.perf_counter()
        t_sam += (t1 - t0) + (t3 - t2)
        t_ver += t2 - t1
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = None
    line = {"value": steps / el, "unit": "steps/s", "cores": nthreads,
            "kind": "oracle",
            "sample": (f"{steps} whole steps (draft, verify and extend each over "
                       f"{nthreads} threads, sequences split between them) of "
                       f"all {cfg.B} sequences on one host copy of a boosted "
                       f"logit slot [{cfg.B},{cfg.K + 1},{cfg.V}] fp32, "
                       f"{el:.1f} s")}
    detail = {"threads_used": nthreads,
              "host_logical_cpus": os.cpu_count(),
              "host_cpus_available_to_process": affinity,
              "single_thread_steps_per_s": steps1 / el1,
              "single_thread_sample": f"{steps1} steps, {el1:.1f} s",
              "verify_ms_per_step": 1e3 * t_ver / nsplit,
              "verify_threads": nthreads,
              "automata_ms_per_step": 1e3 * t_sam / nsplit,
              "automata_threads": 1,
              "split_sample": (f"{nsplit} steps: drafts and extends through the "
                               f"oracle's per-sequence calls on one thread, "
                               f"verification over all sequences on "
                               f"{nthreads} threads")}
    return line, detail


def hbm_read_probe(torch, harness, nbytes=4 << 30, iters=5):
    """Achievable read bandwidth: non-temporal 16-byte loads over 4 GiB."""
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    harness.read_bw(buf, sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = 0.0
    for _ in range(iters):
        e0.record()
        harness.read_bw(buf, sink)
        e1.record()
        e1.synchronize()
        best = max(best, nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del buf
    return best


def same_size_read_probe(torch, harness, ring, nbytes, reps=20, batch=8):
    """The plain read kernel on exactly one stream launch's bytes: 8
    back-to-back launches between events over the ring slots in turn (the
    same way the stream kernel is timed), for a grid-stride grid of 4096
    workgroups and for one workgroup per 32 KiB; the faster is reported."""
    import numpy as np
    nbytes = int(nbytes) // 16 * 16
    views = [r.view(-1).view(torch.uint8)[:nbytes] for r in ring]
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    best = None
    for grid in (4096, max(1, nbytes // 32768)):
        for i in range(batch):
            harness.read_bw(views[i % len(views)], sink, grid)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        for k in range(reps):
            evs[k][0].record()
            for i in range(batch):
                harness.read_bw(views[(k * batch + i) % len(views)], sink, grid)
            evs[k][1].record()
        torch.cuda.synchronize()
        us = float(np.median([a.elapsed_time(b) for a, b in evs])) * 1e3 / batch
        if best is None or us < best["us_per_launch"]:
            best = {"bytes_per_launch": nbytes, "grid": grid, "us_per_launch": round(us, 2),
                    "GBps": round(nbytes / us / 1e3, 1)}
    return best


def sam_stats_report(steps: int):
    """Automaton work per appended token (hash lookups, 128-byte bucket reads,
    suffix-link steps, clones) and time per extend call, for prefill and for
    the per-step append, on the c2 (1,024 tokens), c3 (8,192) and c4
    (32,768) histories and on a c3-shaped run with a +12 boost (long accepted
    drafts)."""
    import numpy as np
    import torch

    import sam_drafting_lossless_amd as ssl
    import synth
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    for c, over in [(2, {}), (3, {}), (4, {}), (3, {"boost": 12.0, "B": 256})]:
        cfg = synth.config(c, **over)
        gt_h = synth.token_streams(cfg, steps)
        gt = torch.as_tensor(gt_h, device=dev)
        H = cfg.hist_len
        st = ssl.SamState(cfg.B, cfg.stream_len(steps), cfg.V, dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        pre = st.extend_stats(gt[:, :H].contiguous(),
                              torch.full((cfg.B,), H, dtype=torch.int32, device=dev))
        e1.record()
        torch.cuda.synchronize()
        prefill_ms = e0.elapsed_time(e1)
        pre = pre.cpu().numpy()
        # Per-step appends: the tokens the verifier emits, from the real step.
        T = torch.full((cfg.B,), cfg.T, dtype=torch.float32, device=dev)
        ws = ssl.verify_workspace(cfg.B, cfg.K, cfg.V, dev)
        stats = torch.zeros(len(ssl.SAM_STATS), dtype=torch.int64, device=dev)
        n = np.full(cfg.B, H, np.int32)
        ext_us = []
        for s in range(steps):
            d, dl, ml = st.draft(cfg.K)
            x = synth.target_logits(cfg, s, gt_h, n, device=dev)
            u = torch.as_tensor(synth.uniforms(cfg, s), device=dev)
            out, nem, _, _ = ssl.spec_verify(x, d, dl, T, u, workspace=ws)
            e0.record()
            st.extend_stats(out, nem, stats)
            e1.record()
            torch.cuda.synchronize()
            ext_us.append(1e3 * e0.elapsed_time(e1))
            n = n + nem.cpu().numpy()
        per = stats.cpu().numpy()
        names = ssl.SAM_STATS

        def norm(v):
            return {k: round(float(v[i]) / max(float(v[0]), 1.0), 4)
                    for i, k in enumerate(names) if i > 0}
        print(json.dumps({
            "workload": cfg.name + ("" if not over else "_boost12"),
            "B": cfg.B, "history": H,
            "prefill": {"tokens": int(pre[0]), "ms": round(prefill_ms, 3),
                        "tokens_per_s": round(float(pre[0]) / (prefill_ms * 1e-3)),
                        "per_token": norm(pre)},
            "steps": {"steps": steps, "tokens": int(per[0]),
                      "tokens_per_step_per_seq": round(float(per[0]) / (steps * cfg.B), 3),
                      "extend_us_median": round(float(np.median(ext_us)), 2),
                      "per_token": norm(per)},
            "status_ok": bool(int(st.status().abs().sum()) == 0)}), flush=True)


def copy_probe(nbytes: int, iters: int = 5):
    """A copy kernel of known size (the reference for hardware byte
    counters): reads and writes `nbytes` per launch."""
    import torch

    from sam_drafting_lossless_amd import harness
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(iters):
        harness.copy(dst, src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "launches": iters}), flush=True)


def measure_sam_workload(cfg, steps: int, warmup: int):
    """Runs the one-call step (harness boost, then spec_step) over `steps`
    timed steps after `warmup`, then the event, separate-call and per-step
    passes described in the module docstring. Inputs are resident before
    timing starts."""
    import numpy as np
    import torch

    import sam_drafting_lossless_amd as ssl
    import synth
    from sam_drafting_lossless_amd import harness

    dev = torch.device("cuda:0")
    B, K, V, R = cfg.B, cfg.K, cfg.V, cfg.K + 1
    dt = ssl.DTYPE_BF16 if cfg.dtype == "bf16" else ssl.DTYPE_F32
    # Ring slots: at least 4, and together at least twice the 256 MB
    # Infinity Cache, so that re-reading a slot comes from HBM (at most 64:
    # a launch-bound workload such as B=1, V=32 is cache-resident anyway).
    RING = max(4, min(64, -(-(2 * INFINITY_CACHE_BYTES) // (B * R * V * cfg.elem_bytes))))
    total = warmup + 4 * steps
    t_setup = time.perf_counter()
    gt_h = synth.token_streams(cfg, total)
    gt = torch.as_tensor(gt_h, device=dev)
    H = cfg.hist_len
    max_len = cfg.stream_len(total)

    # Resident inputs: noise ring, uniforms for every step, automata.
    ring = [synth.noise(cfg, s, dev) for s in range(RING)]
    if dt == ssl.DTYPE_BF16:
        ring = [x.to(torch.bfloat16) for x in ring]
    u_all = torch.as_tensor(
        np.stack([synth.uniforms(cfg, s) for s in range(total)]), device=dev)
    temp = torch.full((B,), cfg.T, dtype=torch.float32, device=dev)
    # Truncation of the target (top-k / top-p), when the workload asks for it.
    trunc = cfg.top_k != 0 or cfg.top_p < 1.0
    tk = torch.full((B,), cfg.top_k, dtype=torch.int32, device=dev) if trunc else None
    tp = torch.full((B,), cfg.top_p, dtype=torch.float32, device=dev) if trunc else None
    tk_p = tk.data_ptr() if trunc else None
    tp_p = tp.data_ptr() if trunc else None
    st = ssl.SamState(B, max_len, V, dev)
    st.extend(gt[:, :H].contiguous(),
              torch.full((B,), H, dtype=torch.int32, device=dev))
    booster = harness.Booster(gt, np.full(B, H, np.int32), R, V, RING,
                              cfg.boost, dt)
    # Rows that get the boost (all of them unless the workload boosts a
    # share, as B=1, V=32 does), one [B, R] mask per step.
    mask = None
    if cfg.boost_prob < 1.0:
        mask = torch.as_tensor(np.stack([synth.boost_mask(cfg, s) for s in range(total)])
                               .astype(np.uint8), device=dev)
    ws = ssl.verify_workspace(B, K, V, dev, truncation=trunc)
    drafts = [torch.empty((B, K), dtype=torch.int32, device=dev) for _ in range(2)]
    mlen = torch.empty(B, dtype=torch.int32, device=dev)
    dl_hist = torch.zeros((total + 1, B), dtype=torch.int32, device=dev)
    nem_hist = torch.zeros((total, B), dtype=torch.int32, device=dev)
    out = torch.empty((B, R), dtype=torch.int32, device=dev)
    pd = torch.empty((B, K), dtype=torch.float32, device=dev)
    status = torch.zeros(B, dtype=torch.int32, device=dev)
    st.draft(K, drafts[0], dl_hist[0], mlen)
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup

    # Direct C calls with precomputed device addresses: the timed loop does
    # argument marshalling only (the checked wrappers cost as much host time
    # as a whole GPU step).
    L = ssl.lib()
    H_ = harness.lib()
    stream = torch.cuda.current_stream().cuda_stream
    ring_p = [t.data_ptr() for t in ring]
    draft_p = [t.data_ptr() for t in drafts]
    dl0, nem0, u0 = dl_hist.data_ptr(), nem_hist.data_ptr(), u_all.data_ptr()
    rowB, rowU = B * 4, B * R * 4
    temp_p, st_p, out_p, pd_p = temp.data_ptr(), st.buf.data_ptr(), out.data_ptr(), pd.data_ptr()
    status_p, mlen_p, ws_p, ws_n = status.data_ptr(), mlen.data_ptr(), ws.data_ptr(), ws.numel()
    gt_p, gt_ld = booster.gt.data_ptr(), booster.gt.shape[1]
    nc_p = [t.data_ptr() for t in booster.ncommit]
    sp_p = [booster.saved_pos[i].data_ptr() for i in range(RING)]
    sv_p = [booster.saved_val[i].data_ptr() for i in range(RING)]
    mask_p = None if mask is None else mask.data_ptr()

    def boost(s):
        slot = s % RING
        rc = H_.hs_boost_step(ring_p[slot], dt, B, R, V, gt_p, gt_ld, nc_p[s % 2],
                              nc_p[(s + 1) % 2], nem0 + (s - 1) * rowB if s else None,
                              sp_p[slot], sv_p[slot],
                              None if mask_p is None else mask_p + s * B * R,
                              float(cfg.boost), stream)
        if rc:
            raise RuntimeError("hs_boost_step failed")

    def fused(s):
        rc = L.spec_step(ring_p[s % RING], dt, B, K, V, draft_p[s % 2], dl0 + s * rowB,
                         temp_p, u0 + s * rowU, tk_p, tp_p, st_p, max_len, out_p,
                         nem0 + s * rowB,
                         pd_p, None, status_p, draft_p[(s + 1) % 2], dl0 + (s + 1) * rowB,
                         mlen_p, ws_p, ws_n, stream)
        if rc:
            raise RuntimeError("spec_step failed: " + L.ss_last_error_string().decode())

    def separate(s):
        # The same step as three calls: verify, extend + next draft.
        rc = L.spec_verify(ring_p[s % RING], dt, B, K, V, draft_p[s % 2], dl0 + s * rowB,
                           None, temp_p, u0 + s * rowU, tk_p, tp_p, out_p,
                           nem0 + s * rowB, pd_p, None, status_p, ws_p, ws_n, stream)
        rc |= L.sam_extend_draft(st_p, B, max_len, out_p, R, nem0 + s * rowB, K,
                                 draft_p[(s + 1) % 2], dl0 + (s + 1) * rowB, mlen_p,
                                 stream)
        if rc:
            raise RuntimeError("separate step failed: " + L.ss_last_error_string().decode())

    STREAM_BATCH = 2 * RING

    def timed_step(s, evs):
        # The same step as spec_stream + spec_finish. The stream pass is
        # launched STREAM_BATCH times back to back between two events, over
        # every ring slot in turn (650 MB of distinct rows per cycle, so the
        # re-reads do not come from the 256 MB Infinity Cache), ending with
        # this step's slot so the workspace holds its statistics; one event
        # pair per launch would add the event's own dispatch gap to each.
        boost(s)
        evs[0].record()
        rc = 0
        for r in range(STREAM_BATCH):
            slot = (s + 1 + r) % RING
            rc |= L.spec_stream(ring_p[slot], dt, B, K, V, draft_p[s % 2],
                                dl0 + s * rowB, temp_p, u0 + s * rowU, tk_p, tp_p,
                                ws_p, ws_n, stream)
        evs[1].record()
        rc |= L.spec_finish(ring_p[s % RING], dt, B, K, V, draft_p[s % 2],
                            dl0 + s * rowB, None, temp_p, u0 + s * rowU, tk_p, tp_p,
                            out_p, nem0 + s * rowB, pd_p, None, status_p, st_p, max_len,
                            draft_p[(s + 1) % 2], dl0 + (s + 1) * rowB, mlen_p,
                            ws_p, ws_n, stream)
        evs[2].record()
        if rc:
            raise RuntimeError("two-pass step failed: " + L.ss_last_error_string().decode())

    def step(s, path=fused):
        boost(s)
        path(s)

    for s in range(warmup):
        step(s)
    torch.cuda.synchronize()
    # Timed region: exactly `steps` steps, synchronised on both sides.
    t0 = time.perf_counter()
    for i in range(steps):
        step(warmup + i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # Per-call durations from HIP events recorded on the launch stream (a
    # second pass over the next `steps` steps; events add small gaps, so this
    # pass is not the one `value` comes from).
    first_ev = warmup + steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
           for _ in range(steps)]
    for i in range(steps):
        timed_step(first_ev + i, evs[i])
    torch.cuda.synchronize()
    dur = np.array([[e[k].elapsed_time(e[k + 1]) for k in range(2)] for e in evs])
    stream_us = 1e3 * dur[:, 0].mean() / STREAM_BATCH
    finish_us = 1e3 * dur[:, 1].mean()

    # The same steps issued as separate library calls (verify, then extend +
    # draft), for comparison.
    first_sep = first_ev + steps
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(steps):
        step(first_sep + i, path=separate)
    torch.cuda.synchronize()
    separate_steps_s = steps / (time.perf_counter() - t1)

    # Per-step library time (harness excluded): events around each spec_step
    # call of a fourth pass. The event pair adds its own dispatch gap to each
    # sample, so these are upper bounds.
    first_ps = first_sep + steps
    evp = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for i in range(steps):
        boost(first_ps + i)
        evp[i][0].record()
        fused(first_ps + i)
        evp[i][1].record()
    torch.cuda.synchronize()
    step_us = np.array([1e3 * a.elapsed_time(b) for a, b in evp])

    ms_per_step = elapsed * 1e3 / steps
    dl = dl_hist[first_ev:first_ev + steps].cpu().numpy()
    nem = nem_hist[warmup:first_ev].cpu().numpy()
    accept_hist = np.bincount(nem.ravel() - 1, minlength=R)[:R]
    needed_bytes = float(nem.sum(axis=1).mean()) * V * cfg.elem_bytes
    rows_per_launch = float((dl + 1).sum(axis=1).mean())
    # Rows of every stream launch this run made (warmup, timed pass, event
    # pass x STREAM_BATCH, separate-call pass), for the traffic record.
    rows_all = (dl_hist[:total].cpu().numpy() + 1).sum(axis=1).astype(np.float64)
    w = np.ones(total)
    w[first_ev:first_ev + steps] = STREAM_BATCH
    stream_launch_rows_mean = float((rows_all * w).sum() / w.sum())
    bytes_per_launch = rows_per_launch * V * cfg.elem_bytes
    achieved = bytes_per_launch / (stream_us * 1e-6) / 1e9
    if int(status.cpu().abs().sum()) != 0 or int(st.status().abs().sum()) != 0:
        raise RuntimeError("status words are non-zero: the run is invalid")
    # The harness alone: the same boost calls as the per-step pass, back to
    # back (last, after the status check: it moves the harness state past the
    # verified steps). Library time per step = the timed loop's step minus
    # this.
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for i in range(steps):
        boost(first_ps + i)
    torch.cuda.synchronize()
    harness_us = (time.perf_counter() - t2) * 1e6 / steps
    library_us = ms_per_step * 1e3 - harness_us
    return {
        "elapsed": elapsed, "setup_s": setup_s, "ring": ring, "gt_h": gt_h,
        "total": total, "RING": RING, "STREAM_BATCH": STREAM_BATCH,
        "stream_us": stream_us, "finish_us": finish_us, "step_us": step_us,
        "harness_us": harness_us, "library_us": library_us,
        "separate_steps_s": separate_steps_s, "rows_per_launch": rows_per_launch,
        "stream_launch_rows_mean": stream_launch_rows_mean,
        "bytes_per_launch": bytes_per_launch, "achieved": achieved, "nem": nem,
        "accept_hist": accept_hist, "needed_bytes": needed_bytes,
    }



def stream_timing(cfg, ring, dl_host, reps: int = 20, batch: int = 8) -> dict:
    """Per-launch time of the stream pass alone for given draft lengths
    (seeded random draft tokens, the workload's temperature): about 50 ms of
    settling launches, then `reps` event pairs around `batch` back-to-back
    launches over the ring slots (as the headline stream timing); the
    median."""
    import numpy as np
    import torch

    import sam_drafting_lossless_amd as ssl
    dev = ring[0].device
    B, K, V = cfg.B, cfg.K, cfg.V
    rng = np.random.default_rng(cfg.seed + 17)
    draft = torch.as_tensor(rng.integers(0, V, (B, K)).astype(np.int32), device=dev)
    dl = torch.as_tensor(np.asarray(dl_host, np.int32), device=dev)
    temp = torch.full((B,), cfg.T, dtype=torch.float32, device=dev)
    u = torch.as_tensor(rng.random((B, K + 1)).astype(np.float32), device=dev)
    ws = ssl.verify_workspace(B, K, V, dev)
    L = ssl.lib()
    stream = torch.cuda.current_stream().cuda_stream
    dt = ssl.DTYPE_BF16 if ring[0].dtype == torch.bfloat16 else ssl.DTYPE_F32

    def launch(i):
        rc = L.spec_stream(ring[i % len(ring)].data_ptr(), dt, B, K, V, draft.data_ptr(),
                           dl.data_ptr(), temp.data_ptr(), u.data_ptr(), None, None,
                           ws.data_ptr(), ws.numel(), stream)
        if rc:
            raise RuntimeError("spec_stream failed: " + L.ss_last_error_string().decode())

    # About 50 ms of launches first: after host-side work the GPU's clocks
    # are still ramping, and the first 30 ms or so of a long launch sequence
    # read up to 9 % slower.
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < 0.05:
        for _ in range(batch):
            launch(i)
            i += 1
        torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for r in range(reps):
        evs[r][0].record()
        for i in range(batch):
            launch(r * batch + i)
        evs[r][1].record()
    torch.cuda.synchronize()
    us = float(np.median([a.elapsed_time(b) for a, b in evs])) * 1e3 / batch
    rows = int((np.clip(np.asarray(dl_host), 0, K) + 1).sum())
    nbytes = rows * V * cfg.elem_bytes
    gbps = nbytes / (us * 1e-6) / 1e9
    return {"rows": rows, "bytes_per_launch": nbytes, "us_per_launch": round(us, 2),
            "GBps": round(gbps, 1), "frac_of_8TBps": round(gbps / PEAK_HBM_GBPS, 4),
            "launches_per_event_pair": batch}


def all_rows_stream(cfg, ring, reps: int = 20, batch: int = 8) -> dict:
    """The stream pass with every sequence's draft of length K, so that all
    B x (K+1) rows are verified (B = 256, K = 3: 1,024 rows, 622 MB)."""
    import numpy as np
    return stream_timing(cfg, ring, np.full(cfg.B, cfg.K, np.int32), reps, batch)


def stream_sweep(reps: int = 20):
    """The stream pass alone at the headline shape (B = 256, V = 151936,
    fp32, T = 1) for draft-length mixes from none to all, at K = 3 and
    K = 16: one JSON line each."""
    import numpy as np

    import synth
    for K in (3, 16):
        cfg = synth.config(3, K=K)
        ring = [synth.noise(cfg, s, "cuda") for s in range(4)]
        rng = np.random.default_rng(5 + K)
        c3like = np.zeros(cfg.B, np.int32)
        c3like[:5], c3like[5:7], c3like[7:9] = K, min(2, K), 1
        mixes = {"none": np.zeros(cfg.B, np.int32),
                 "c3-like (5 x K, 2 x 2, 2 x 1, rest 0)": rng.permutation(c3like),
                 f"uniform 0..{K}": rng.integers(0, K + 1, cfg.B).astype(np.int32),
                 "all K": np.full(cfg.B, K, np.int32)}
        for name, dl in mixes.items():
            line = {"workload": f"stream pass B={cfg.B} V={cfg.V} K={K} fp32 T={cfg.T}",
                    "draft_lengths": name, **stream_timing(cfg, ring, dl, reps)}
            print(json.dumps(line), flush=True)
        del ring


def _sam_workload_line(cfg, m, steps: int) -> dict:
    import numpy as np
    line = {
        "workload": cfg.name, "dtype": cfg.dtype, "B": cfg.B, "V": cfg.V,
        "K": cfg.K, "T": cfg.T, "steps": steps,
        "steps_per_s": steps / m["elapsed"],
        "us_per_step": m["elapsed"] * 1e6 / steps,
        "stream_pass_avg_us": m["stream_us"],
        "verified_rows_per_launch": m["rows_per_launch"],
        "stream_bytes_per_launch": m["bytes_per_launch"],
        "stream_GBps": m["achieved"],
        "stream_frac_of_8TBps": m["achieved"] / PEAK_HBM_GBPS,
        "finish_pass_event_us": m["finish_us"],
        "mean_tokens_per_step": float(m["nem"].mean()),
        "accepted_drafts_histogram": {str(k): int(c) for k, c in
                                      enumerate(m["accept_hist"])},
        "step_event_us_p10_p50_p90": [round(float(x), 2) for x in
                                      np.percentile(m["step_us"], [10, 50, 90])],
        "harness_us_per_step": m["harness_us"],
        "library_steps_per_s": 1e6 / m["library_us"],
        "ring_slots": m["RING"],
    }
    if cfg.top_k != 0 or cfg.top_p < 1.0:
        line["top_k"], line["top_p"] = cfg.top_k, cfg.top_p
        line["finish_pass_contents"] = ("truncation select (plan, candidates from the "
                                        "chunks' band segments, selection); finalize")
    return line


def measure_draft_model_workload(cfg, steps: int, warmup: int) -> dict:
    """Verification with given draft probabilities q (no automaton): each
    step is one spec_verify call (stream pass, finish pass, residual chunk
    sums over the rejected row, residual draw), all drafts of length K, on
    two resident slots of target logits, q and drafts (1.7 GB). The stream
    pass is timed as in the main bench (events around back-to-back batches
    alternating the two slots)."""
    import numpy as np
    import torch

    import sam_drafting_lossless_amd as ssl
    import synth
    dev = torch.device("cuda:0")
    B, K, V, R = cfg.B, cfg.K, cfg.V, cfg.K + 1
    nslots = 2
    slots = []
    for i in range(nslots):
        x = synth.noise(cfg, i, dev)
        q, draft = synth.draft_model_inputs(cfg, i, x, dev)
        slots.append((x, q, torch.as_tensor(draft, device=dev)))
    total = warmup + 2 * steps
    u_all = torch.as_tensor(
        np.stack([synth.uniforms(cfg, s) for s in range(total)]), device=dev)
    temp = torch.full((B,), cfg.T, dtype=torch.float32, device=dev)
    dl = torch.full((B,), K, dtype=torch.int32, device=dev)
    out = torch.empty((B, R), dtype=torch.int32, device=dev)
    nem_hist = torch.zeros((total, B), dtype=torch.int32, device=dev)
    pd = torch.empty((B, K), dtype=torch.float32, device=dev)
    status = torch.zeros(B, dtype=torch.int32, device=dev)
    ws = ssl.verify_workspace(B, K, V, dev)
    torch.cuda.synchronize()
    L = ssl.lib()
    stream = torch.cuda.current_stream().cuda_stream
    xp = [t[0].data_ptr() for t in slots]
    qp = [t[1].data_ptr() for t in slots]
    dp = [t[2].data_ptr() for t in slots]
    u0, nem0, rowU, rowB = u_all.data_ptr(), nem_hist.data_ptr(), B * R * 4, B * 4

    def call(s):
        k = s % nslots
        rc = L.spec_verify(xp[k], 0, B, K, V, dp[k], dl.data_ptr(), qp[k],
                           temp.data_ptr(), u0 + s * rowU, None, None, out.data_ptr(),
                           nem0 + s * rowB, pd.data_ptr(), None, status.data_ptr(),
                           ws.data_ptr(), ws.numel(), stream)
        if rc:
            raise RuntimeError("spec_verify failed: " + L.ss_last_error_string().decode())

    for s in range(warmup):
        call(s)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        call(warmup + i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    batch = 2 * nslots
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
           for _ in range(steps)]
    for i in range(steps):
        s = warmup + steps + i
        k = s % nslots
        evs[i][0].record()
        rc = 0
        for r in range(batch):
            kk = (s + 1 + r) % nslots
            rc |= L.spec_stream(xp[kk], 0, B, K, V, dp[k], dl.data_ptr(),
                                temp.data_ptr(), u0 + s * rowU, None, None,
                                ws.data_ptr(), ws.numel(), stream)
        evs[i][1].record()
        rc |= L.spec_finish(xp[k], 0, B, K, V, dp[k], dl.data_ptr(), qp[k],
                            temp.data_ptr(), u0 + s * rowU, None, None, out.data_ptr(),
                            nem0 + s * rowB, pd.data_ptr(), None, status.data_ptr(),
                            None, 0, None, None, None, ws.data_ptr(), ws.numel(), stream)
        evs[i][2].record()
        if rc:
            raise RuntimeError("two-pass call failed: " + L.ss_last_error_string().decode())
    torch.cuda.synchronize()
    if int(status.cpu().abs().sum()) != 0:
        raise RuntimeError("status words are non-zero: the run is invalid")
    dur = np.array([[e[k].elapsed_time(e[k + 1]) for k in range(2)] for e in evs])
    stream_us = 1e3 * dur[:, 0].mean() / batch
    finish_us = 1e3 * dur[:, 1].mean()
    nem = nem_hist[warmup:warmup + steps].cpu().numpy()
    stream_bytes = B * R * V * 4
    rejected = float((nem <= K).sum(axis=1).mean())
    return {
        "workload": cfg.name, "dtype": cfg.dtype, "B": B, "V": V, "K": K, "T": cfg.T,
        "steps": steps, "steps_per_s": steps / elapsed,
        "us_per_step": elapsed * 1e6 / steps,
        "stream_pass_avg_us": stream_us,
        "verified_rows_per_launch": B * R,
        "stream_bytes_per_launch": stream_bytes,
        "stream_GBps": stream_bytes / (stream_us * 1e-6) / 1e9,
        "stream_frac_of_8TBps": stream_bytes / (stream_us * 1e-6) / 1e9 / PEAK_HBM_GBPS,
        "finish_pass_event_us": finish_us,
        "finish_pass_contents": "finish kernel, residual chunk sums, residual draw",
        "rejected_sequences_per_step": rejected,
        "residual_bytes_per_step": rejected * V * 8,
        "mean_tokens_per_step": float(nem.mean()),
        "accepted_drafts_histogram": {str(k): int(c) for k, c in
                                      enumerate(np.bincount(nem.ravel() - 1,
                                                            minlength=R)[:R])},
        "slots": nslots,
    }


def measure_tree_workload(cfg, steps: int, warmup: int) -> dict:
    """Draft-tree verification (spec_verify_tree): every sequence carries an
    8-node tree (the root with three candidate continuations, one of them
    four deep); the stream pass reads all 8 rows of every sequence, the tree
    kernel walks it. Two resident slots of target logits [B, 8, V] (2.5 GB at
    c3's B and V), the nodes of the first candidate's path raised by cfg.boost
    in their parents' rows so that walks go deep."""
    import numpy as np
    import torch

    import sam_drafting_lossless_amd as ssl
    import synth
    dev = torch.device("cuda:0")
    B, V = cfg.B, cfg.V
    N = len(synth.TREE8_PARENTS)
    nslots = 2
    slots = []
    for i in range(nslots):
        x = synth.noise(cfg, i, dev, rows_per_seq=N)
        tok, par, chain = synth.draft_trees(cfg, i)
        bi, ni = np.nonzero(chain)
        x[torch.as_tensor(bi, device=dev), torch.as_tensor(par[bi, ni], device=dev),
          torch.as_tensor(tok[bi, ni].astype(np.int64), device=dev)] += cfg.boost
        slots.append((x, torch.as_tensor(tok, device=dev), torch.as_tensor(par, device=dev)))
    total = warmup + 2 * steps
    u_all = torch.as_tensor(
        np.stack([synth.tree_uniforms(cfg, s, N) for s in range(total)]), device=dev)
    temp = torch.full((B,), cfg.T, dtype=torch.float32, device=dev)
    nn = torch.full((B,), N, dtype=torch.int32, device=dev)
    out = torch.empty((B, N), dtype=torch.int32, device=dev)
    onode = torch.empty((B, N), dtype=torch.int32, device=dev)
    nem_hist = torch.zeros((total, B), dtype=torch.int32, device=dev)
    status = torch.zeros(B, dtype=torch.int32, device=dev)
    ws = ssl.tree_workspace(B, N, V, dev)
    torch.cuda.synchronize()
    L = ssl.lib()
    stream = torch.cuda.current_stream().cuda_stream
    u0, nem0, rowU, rowB = u_all.data_ptr(), nem_hist.data_ptr(), B * N * 4, B * 4

    def call(s):
        x, tk, pr = slots[s % nslots]
        rc = L.spec_verify_tree(x.data_ptr(), 0, B, N, V, tk.data_ptr(), pr.data_ptr(),
                                nn.data_ptr(), temp.data_ptr(), u0 + s * rowU,
                                out.data_ptr(), onode.data_ptr(), nem0 + s * rowB,
                                status.data_ptr(), ws.data_ptr(), ws.numel(), stream)
        if rc:
            raise RuntimeError("spec_verify_tree failed: " + L.ss_last_error_string().decode())

    for s in range(warmup):
        call(s)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        call(warmup + i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for i in range(steps):
        evs[i][0].record()
        call(warmup + steps + i)
        evs[i][1].record()
    torch.cuda.synchronize()
    if int(status.cpu().abs().sum()) != 0:
        raise RuntimeError("status words are non-zero: the run is invalid")
    call_us = np.array([1e3 * a.elapsed_time(b) for a, b in evs])
    nem = nem_hist[warmup:warmup + steps].cpu().numpy()
    stream_bytes = B * N * V * 4
    return {
        "workload": cfg.name, "dtype": cfg.dtype, "B": B, "V": V, "tree_nodes": N,
        "tree_parents": list(synth.TREE8_PARENTS), "T": cfg.T, "steps": steps,
        "steps_per_s": steps / elapsed, "us_per_step": elapsed * 1e6 / steps,
        "call_event_us_p10_p50_p90": [round(float(v), 2) for v in
                                      np.percentile(call_us, [10, 50, 90])],
        "rows_per_step": B * N, "stream_bytes_per_step": stream_bytes,
        "whole_call_GBps": stream_bytes / (elapsed / steps) / 1e9,
        "mean_tokens_per_step": float(nem.mean()),
        "emitted_histogram": {str(k): int(c) for k, c in
                              enumerate(np.bincount(nem.ravel(), minlength=N + 1)[1:], 1)},
        "slots": nslots,
    }


# Workloads beside the headline one. c3 with truncation takes the pages'
# sampling setting for their end-to-end throughput figure (T = 0.7,
# top_p = 0.9), with and without top_k = 50.
def _workload_configs():
    import synth
    return {
        "c1": synth.config(1),
        "c2": synth.config(2),
        "c4": synth.config(4),
        "c5": synth.config(5),
        "c3_drafted": synth.config(3, name="c3_b256_v151936_k3_t1_onehot_boost12",
                                   boost=12.0),
        "c3_topp": synth.config(3, name="c3_b256_v151936_k3_t0.7_topp0.9_onehot",
                                T=0.7, top_p=0.9),
        "c3_topk_topp": synth.config(3, name="c3_b256_v151936_k3_t0.7_topk50_topp0.9_onehot",
                                     T=0.7, top_k=50, top_p=0.9),
        "c3_tree8": synth.config(3, name="c3_b256_v151936_t1_tree8", q_mode="tree",
                                 boost=12.0),
    }


def _measure_workload(cfg, steps: int, warmup: int) -> dict:
    if cfg.q_mode == "model":
        return measure_draft_model_workload(cfg, steps, warmup)
    if cfg.q_mode == "tree":
        return measure_tree_workload(cfg, steps, warmup)
    return _sam_workload_line(cfg, measure_sam_workload(cfg, steps, warmup), steps)


def workloads_report(steps: int, warmup: int, names: str = "all"):
    """One JSON line per workload: c2 (greedy), c4 (bf16 logits, long
    histories) and the truncated c3 variants through the automaton step, c5
    through given q."""
    cfgs = _workload_configs()
    pick = list(cfgs) if names == "all" else names.split(",")
    for n in pick:
        print(json.dumps(_measure_workload(cfgs[n], steps, warmup)), flush=True)


# The measures of each workload's own line kept in the headline line.
SUMMARY_KEYS = ("steps", "steps_per_s", "us_per_step", "library_steps_per_s",
                "stream_pass_avg_us", "verified_rows_per_launch",
                "stream_frac_of_8TBps", "finish_pass_event_us", "mean_tokens_per_step",
                "rows_per_step", "whole_call_GBps")


def workloads_summary(warmup: int) -> dict:
    """Every other workload measured in the headline run too, in compact
    form (C1 over its 500 steps, the others over 200; `--workloads` prints
    their full lines)."""
    out = {}
    for n, cfg in _workload_configs().items():
        line = _measure_workload(cfg, 500 if n == "c1" else 200, warmup)
        out[line["workload"]] = {k: line[k] for k in SUMMARY_KEYS if k in line}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle work for cpu_baseline (0 = skip)")
    ap.add_argument("--no-probe", action="store_true")
    ap.add_argument("--sam-stats", action="store_true",
                    help="report automaton work per token instead")
    ap.add_argument("--workloads", nargs="?", const="all", default=None,
                    help="measure other workloads instead: all, or a comma "
                         "list of c1, c2, c4, c5, c3_drafted, c3_topp, "
                         "c3_topk_topp, c3_tree8")
    ap.add_argument("--stream-sweep", action="store_true",
                    help="time only the stream pass at the headline shape for "
                         "draft-length mixes from none to all, K = 3 and 16")
    ap.add_argument("--all-rows", action="store_true",
                    help="time only the stream pass over all B x (K+1) rows "
                         "of the headline shape (every draft full)")
    ap.add_argument("--no-extras", action="store_true",
                    help="headline line without the all-rows, drafted and "
                         "other workloads' measurements (for profiling the "
                         "headline alone)")
    ap.add_argument("--copy-probe", type=int, default=0,
                    help="run a copy kernel of this many bytes instead")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path "
              "(the step would shard by sequence, with no exchange between "
              "GPUs). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.sam_stats:
        sam_stats_report(args.steps)
        return
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return

    import numpy as np
    import torch

    import synth
    from sam_drafting_lossless_amd import harness

    torch.cuda.set_device(torch.device("cuda:0"))
    if args.workloads:
        workloads_report(args.steps, args.warmup, args.workloads)
        return
    cfg = synth.config(3)
    if args.stream_sweep:
        stream_sweep()
        return
    if args.all_rows:
        ring = [synth.noise(cfg, s, "cuda") for s in range(4)]
        print(json.dumps({"workload": cfg.name + "_all_rows",
                          **all_rows_stream(cfg, ring, reps=args.steps)}), flush=True)
        return
    B, K, V = cfg.B, cfg.K, cfg.V
    m = measure_sam_workload(cfg, args.steps, args.warmup)
    elapsed, ring, total, RING = m["elapsed"], m["ring"], m["total"], m["RING"]
    ms_per_step = elapsed * 1e3 / args.steps
    rows_per_launch, achieved = m["rows_per_launch"], m["achieved"]
    nem, step_us, H = m["nem"], m["step_us"], cfg.hist_len
    gt_h = m["gt_h"]

    # The same shape with every draft full (all 1,024 rows verified), and with
    # the true next token boosted by +12, so that drafts are accepted and
    # the automaton grows by several tokens per step.
    all_rows = drafted = None
    if not args.no_extras:
        all_rows = all_rows_stream(cfg, ring)
        dcfg = _workload_configs()["c3_drafted"]
        dsteps = max(1, min(args.steps, 200))
        drafted = _sam_workload_line(
            dcfg, measure_sam_workload(dcfg, dsteps, args.warmup), dsteps)
        drafted["boost"] = dcfg.boost

    others = None if args.no_extras else workloads_summary(min(args.warmup, 20))
    probe = None if args.no_probe else hbm_read_probe(torch, harness)
    probe_same = (None if args.no_probe else
                  same_size_read_probe(torch, harness, ring, m["bytes_per_launch"]))
    cpu = cpu_detail = None
    if args.cpu_budget > 0:
        slot_h = ring[(total - 1) % RING].cpu().numpy()
        try:
            ncpu = len(os.sched_getaffinity(0))
        except AttributeError:
            ncpu = os.cpu_count() or 1
        # at most 16 threads: the share of the host's cores that one GPU's
        # process is given on an 8-GPU MI355X node
        cpu, cpu_detail = cpu_baseline(slot_h, gt_h, cfg, min(ncpu, 16),
                                       args.cpu_budget)

    res = {
        "metric": METRIC,
        "value": args.steps / elapsed,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": B, "V": V, "K": K, "T": cfg.T,
                   "logits": "fp32 [B,K+1,V]", "drafts": "one-hot SAM",
                   "history": H, "p_copy": cfg.p_copy, "span_mean": cfg.span_mean,
                   "noise_sigma": round(cfg.sigma, 6), "boost": cfg.boost,
                   "ring_slots": RING},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": achieved / PEAK_HBM_GBPS,
                     "traffic": _traffic_from_profile(rows_per_launch)},
        "cpu_baseline": cpu,
        "cpu_baseline_detail": cpu_detail,
        "path": "spec_step (stream pass, then finish pass: decisions, draws, "
                "SAM extend, next draft)",
        "stream_pass_avg_us": m["stream_us"],
        "finish_pass_event_us": m["finish_us"],
        "stream_launches_per_event_pair": m["STREAM_BATCH"],
        "separate_calls_steps_per_s": m["separate_steps_s"],
        "verified_rows_per_launch": rows_per_launch,
        "stream_launch_rows_mean": m["stream_launch_rows_mean"],
        "verify_bytes_per_launch": m["bytes_per_launch"],
        "mean_tokens_per_step": float(nem.mean()),
        "accepted_drafts_histogram": {str(k): int(c) for k, c in enumerate(m["accept_hist"])},
        "needed_rows_bytes_per_step": m["needed_bytes"],
        "step_event_us_p10_p50_p90": [round(float(x), 2) for x in
                                      np.percentile(step_us, [10, 50, 90])],
        "harness_us_per_step": m["harness_us"],
        "library_steps_per_s": 1e6 / m["library_us"],
        "library_steps_note": ("the timed loop's time per step minus the harness "
                               "boost kernel's (the same boost calls timed back to "
                               "back in a last pass): the library calls alone, as "
                               "the metric defines the step; value keeps the "
                               "harness in"),
        "verify_all_rows": all_rows,
        "c3_drafted": drafted,
        "workloads": others,
        "hbm_read_probe_GBps": probe,
        "hbm_read_probe_same_bytes": probe_same,
        "setup_s": m["setup_s"],
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
