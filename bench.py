"""Benchmark: BPE training on one MI355X, one JSON line on stdout.

A step is one whole training job on device-resident bytes: tag + count
into the global pair table (bpe_init), every merge iteration (one launch:
selection of the merge from the candidate list, or by a sweep of the
table, then merge + compaction + count update of the new sequence), and
the copy-out of merges and tokens. The default workload is the 256 MiB
ASCII corpus with 32,000 merges and a 2^22-slot pair table. Warm-up steps
run without events; timed steps run with a HIP event after each
iteration's launch on the library's stream (one host wait per step), which
gives both the wall-clock value and the per-iteration times behind the
roofline figures.

Algorithmic bytes of iteration k (n_k symbols before it, n_{k+1} after,
T table slots of 8 bytes):
  2 n_k + 2 n_{k+1}: the merge pass reads the symbols (16-bit ids; a word
  start is a change of byte class between neighbours, so no tag is stored)
  once and writes the compacted result once (the roofline figure of
  k_merge);
  + 16 T in an iteration that sweeps the table (for the maximum, then for
  the candidates; "table_sweeps" counts them). The table is never reset
  (its counts are updated in place), so no reset write is credited. Count
  updates, candidate-list reads and look-back status words are
  implementation overhead: timed, not credited.

After training, the line also reports inference ("inference"): greedy
longest-match tokenization of the same corpus with the trie of the merges
just learned (walk, scan, copy), timed per kernel with HIP events on the
trie's stream. Its algorithmic bytes are the text read once (1 byte per
input byte) plus the token ids written once (4 bytes per token); trie nodes
are read from cache, and the per-tile slices are implementation traffic:
timed, not credited.

"encoding" reports encoding of the same corpus with the same merges (a
learned list applied to new text, word by word, each distinct word encoded
once), with the same accounting.

"chunked" reports training over the corpus's distinct words
(bpe_train_chunked: each distinct word once with its frequency, the same
merges and tokens by another route), whole jobs timed by the wall clock and
compared with the full-array result; the headline stays the full-array
path, whose merge pass is the HBM-bound kernel of the roofline figures.

"configs" reports the other four workloads (64 KiB, 16 MiB, 128 MiB and
1 GiB corpora, each with its own merge count and table size): one timed
job each, merges/s, the merge pass's GB/s and fraction of peak, whether
the result is bit-identical to the chunk-multiset CPU oracle on the same
bytes (timed beside it, one core), and the distinct-word training's job.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E


def log(msg: str) -> None:
    print("[bench] " + msg, file=sys.stderr, flush=True)


def kernel_sources_sha256(files=None) -> str:
    """SHA-256 of the kernel sources: the given files of bpe_merge_amd/csrc,
    or every header plus bpe.hip."""
    import glob
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bpe_merge_amd", "csrc")
    paths = ([os.path.join(csrc, f) for f in files] if files else
             sorted(glob.glob(os.path.join(csrc, "*.hpp"))) + [os.path.join(csrc, "bpe.hip")])
    for f in paths:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary, only if it was taken on the kernel's sources as they are now."""
    path = os.path.join(ROOT, "profiles", "traffic_%s_%s.json" % (kernel, workload))
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("kernel_sources_sha256") != kernel_sources_sha256(t.get("kernel_sources")):
        return None
    return t


def cpu_facts() -> dict:
    """The host CPU model and core count, for the CPU baseline."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "host_cores": os.cpu_count()}


class one_core:
    """Pin this process to one core while the oracle is timed (it is
    single-threaded), and restore the previous affinity afterwards."""

    def __enter__(self):
        self.prev = None
        if hasattr(os, "sched_getaffinity"):
            self.prev = os.sched_getaffinity(0)
            os.sched_setaffinity(0, {min(self.prev)})
        return self

    def __exit__(self, *exc):
        if self.prev is not None:
            os.sched_setaffinity(0, self.prev)


def pct(a, q):
    import numpy as np
    return float(np.percentile(a, q)) if len(a) else 0.0


def inference_leg(args, bpe, spec, data, d, m, np, torch, time, log, source="learned above"):
    """Greedy longest-match inference of the corpus (device-resident) with
    the trie of merges m, timed per kernel; returns the report object."""
    k = int(m.shape[0])
    log("inference: trie of the %d learned merges over the same corpus, %d launches"
        % (k, args.inference_reps))
    with bpe.Trie(m) as tr:
        slots, longest = tr.info()
        n_tok, ms = tr.profile(d, args.inference_reps)
        sample_n = min(spec.n_bytes, 16 << 20)
        gpu_sample = None
        if not args.no_cpu_baseline:
            gpu_sample = tr.encode(d[:sample_n]).cpu().numpy().astype(np.uint32)
    ms = ms.astype(np.float64)
    per_kernel = ms.mean(axis=0)
    ms = ms.sum(axis=1)
    avg_ms = float(ms.mean())
    inf_bytes = float(spec.n_bytes) + 4.0 * n_tok
    inf_gbps = inf_bytes / (avg_ms / 1e3) / 1e9
    inf_traffic = measured_traffic(spec.name, "trie")
    inf_cpu = None
    if gpu_sample is not None:
        import oracle
        mh = m.cpu().numpy()
        with one_core():
            t0 = time.perf_counter()
            ot = oracle.trie_encode(data[:sample_n], mh)
            cpu_s = time.perf_counter() - t0
        inf_cpu = {"value": round(sample_n / cpu_s, 1), "unit": "bytes/s", "cores": 1, "kind": "oracle",
                   "sample": "the first %d bytes of the corpus through the C oracle (oracle/bpe_oracle.c, "
                             "trie_encode, pointer trie), one thread, %.2f s; GPU tokens of the same bytes "
                             "identical: %s" % (sample_n, cpu_s, bool(np.array_equal(ot, gpu_sample))),
                   "pinned": "one core (sched_setaffinity)", **cpu_facts()}
        log("inference oracle: %.2f s on %d bytes, identical: %s"
            % (cpu_s, sample_n, np.array_equal(ot, gpu_sample)))
    inference = {
        "metric": "trie greedy longest-match tokenization, input bytes/s",
        "value": round(spec.n_bytes / (avg_ms / 1e3), 1),
        "unit": "bytes/s",
        "workload": "%s corpus (%d bytes), vocabulary of the %d merges %s (trie %d slots, "
                    "longest string %d bytes)" % (spec.name, spec.n_bytes, k, source, slots, longest),
        "tokens": int(n_tok),
        "runs": len(ms),
        "ms_per_run": {"mean": round(avg_ms, 4), "min": round(float(ms.min()), 4),
                       "max": round(float(ms.max()), 4)},
        "kernels_ms_per_run": {"k_trie_walk": round(float(per_kernel[0]), 4),
                               "k_trie_scan": round(float(per_kernel[1]), 4),
                               "k_trie_copy": round(float(per_kernel[2]), 4)},
        "roofline": {"bound": "hbm", "kernel": "all three passes", "achieved": round(inf_gbps, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(inf_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": (round(inf_traffic["fetch_bytes_per_launch"] + inf_traffic["write_bytes_per_launch"])
                                 if inf_traffic else None),
                     "bytes_per_launch": round(inf_bytes), "avg_launch_ms": round(avg_ms, 5)},
        "cpu_baseline": inf_cpu,
    }
    log("inference: %.3f ms per run (walk %.3f, scan %.3f, copy %.3f), %.1f GB/s algorithmic, %d tokens"
        % (avg_ms, per_kernel[0], per_kernel[1], per_kernel[2], inf_gbps, n_tok))

    return inference


def encode_leg(args, bpe, spec, data, d, m, np, time, log, source="learned above", train_tokens=None):
    """Encoding of the corpus (device-resident) with merges m, word by word,
    timed per kernel; returns the report object. With the training run's
    tokens given, the whole encoding is compared with them (encoding a
    training corpus with its own merges must give its training tokens)."""
    k = int(m.shape[0])
    log("encoding: the %d merges over the same corpus, %d runs" % (k, args.inference_reps))
    same_as_training = None
    with bpe.Encoder(m) as enc:
        n_tok, ms = enc.profile(d, args.inference_reps)
        if train_tokens is not None:
            whole = enc.encode(d)
            same_as_training = bool(whole.shape == train_tokens.shape and bool((whole == train_tokens).all()))
            del whole
            log("encoding: whole corpus identical to the training tokens: %s" % same_as_training)
        sample_n = min(spec.n_bytes, 128 << 10)
        gpu_sample = None
        if not args.no_cpu_baseline:
            gpu_sample = enc.encode(d[:sample_n]).cpu().numpy().astype(np.uint32)
    ms = ms.astype(np.float64)
    per_kernel = ms.mean(axis=0)
    ms = ms.sum(axis=1)
    avg_ms = float(ms.mean())
    enc_bytes = float(spec.n_bytes) + 4.0 * n_tok
    enc_gbps = enc_bytes / (avg_ms / 1e3) / 1e9
    enc_traffic = measured_traffic(spec.name, "encode")
    cpu = None
    if gpu_sample is not None:
        import oracle
        mh = m.cpu().numpy()
        with one_core():
            t0 = time.perf_counter()
            _, ot = oracle.encode(data[:sample_n], mh)
            cpu_s = time.perf_counter() - t0
        cpu = {"value": round(sample_n / cpu_s, 1), "unit": "bytes/s", "cores": 1, "kind": "oracle",
               "sample": "the first %d bytes of the corpus through the C oracle (oracle/bpe_oracle.c, encode: "
                         "every merge applied over the whole text in order), one thread, %.2f s; GPU tokens of "
                         "the same bytes identical: %s" % (sample_n, cpu_s, bool(np.array_equal(ot, gpu_sample))),
               "pinned": "one core (sched_setaffinity)", **cpu_facts()}
        log("encoding oracle: %.2f s on %d bytes, identical: %s" % (cpu_s, sample_n, np.array_equal(ot, gpu_sample)))
    log("encoding: %.3f ms per run (word cache %.3f, walk %.3f, scan %.3f, copy %.3f), %.1f GB/s algorithmic, "
        "%d tokens" % (avg_ms, per_kernel[0], per_kernel[1], per_kernel[2], per_kernel[3], enc_gbps, n_tok))
    return {
        "metric": "BPE encoding of new text with a merge list, input bytes/s",
        "value": round(spec.n_bytes / (avg_ms / 1e3), 1),
        "unit": "bytes/s",
        "workload": "%s corpus (%d bytes), the %d merges %s" % (spec.name, spec.n_bytes, k, source),
        "tokens": int(n_tok),
        "identical_to_training_tokens": same_as_training,
        "runs": len(ms),
        "ms_per_run": {"mean": round(avg_ms, 4), "min": round(float(ms.min()), 4), "max": round(float(ms.max()), 4)},
        "kernels_ms_per_run": {"word_cache": round(float(per_kernel[0]), 4),
                               "k_enc_walk": round(float(per_kernel[1]), 4),
                               "k_enc_gscan": round(float(per_kernel[2]), 4),
                               "k_enc_copy": round(float(per_kernel[3]), 4)},
        "roofline": {"bound": "hbm", "kernel": "all passes", "achieved": round(enc_gbps, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(enc_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": (round(enc_traffic["fetch_bytes_per_launch"] + enc_traffic["write_bytes_per_launch"])
                                 if enc_traffic else None),
                     "traffic_source": "profiles/traffic_encode_%s.json" % spec.name if enc_traffic else None,
                     "bytes_per_launch": round(enc_bytes), "avg_launch_ms": round(avg_ms, 5)},
        "cpu_baseline": cpu,
    }


def traffic_windows(workload: str, kernel: str):
    """Measured HBM bytes of a kernel from the committed rocprofv3
    FETCH_SIZE/WRITE_SIZE summary (one or more windows of launches), only if
    it was taken on the kernel sources as they are now."""
    t = measured_traffic(workload, kernel)
    if t is None:
        return None
    wins = t.get("windows") or [t]
    out = []
    for w in wins:
        meas = w["fetch_bytes_per_launch"] + w["write_bytes_per_launch"]
        alg = w["algorithmic_bytes_per_launch"]
        out.append({"launches": w.get("launches"), "iterations": w.get("iterations"),
                    "read": round(w["fetch_bytes_per_launch"]), "write": round(w["write_bytes_per_launch"]),
                    "measured": round(meas), "algorithmic_same_launches": round(alg),
                    "ratio": round(meas / alg, 4)})
    return out


def train_leg(bpe, corpus, spec, steps, warmup, np, torch, time, log, cpu_reps=0, events=True, chunk=0):
    """Train spec's workload: warmup unprofiled jobs, then `steps` jobs with
    a HIP event after each iteration's launch (without events: timed by the
    wall clock only, for runs under a profiler). Returns the measurements,
    the last job's merges and tokens, and (cpu_reps > 0) the CPU oracle's
    timing on the same bytes with the bit-identity check."""
    log("generating %s (%d bytes)" % (spec.name, spec.n_bytes))
    data = corpus.generate(spec)
    sha = corpus.sha256(data)
    d = torch.from_numpy(data).to("cuda:0")
    torch.cuda.synchronize()
    n_merges, tlog2 = spec.n_merges, spec.table_log2

    usage = [0, 0, 0]

    def step(profiled: bool):
        t0 = time.perf_counter()
        st = bpe.State(d, table_log2=tlog2)
        prof = None
        if profiled:
            prof = st.profile(n_merges, per_iteration=True)
        elif chunk:
            # at most `chunk` launches in flight (a profiler that serialises
            # dispatches keeps one record per queued launch)
            for i in range(0, n_merges, chunk):
                st.run(min(chunk, n_merges - i))
                st.sync()
        else:
            st.run(n_merges)
            st.sync()
        merges = st.merges()
        tokens = st.tokens()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        lengths = st.lengths().cpu().numpy().astype(np.int64)
        usage[:] = st.table_usage()
        st.free()
        return t1 - t0, merges, tokens, lengths, prof

    warm_s = []
    for i in range(warmup):
        dt, m, t, _, _ = step(False)
        warm_s.append(dt)
        log("%s warmup step %d: %.3f s, %d merges, %d tokens" % (spec.name, i + 1, dt, m.shape[0], t.shape[0]))
    wall, last, ref = [], None, None
    for i in range(steps):
        torch.cuda.synchronize()
        dt, m, t, lengths, prof = step(events)
        wall.append(dt)
        last = (m, t, lengths, prof)
        sig = (m.cpu().numpy().tobytes(), t.shape[0])
        if ref is None:
            ref = sig
        elif sig != ref:
            raise RuntimeError("timed steps of %s disagree" % spec.name)
        log("%s timed step %d: %.3f s, %d merges" % (spec.name, i + 1, dt, m.shape[0]))
    m, t, lengths, prof = last
    k = m.shape[0]
    if prof is None:  # no per-iteration events: the job's wall time stands in
        r = type("NoEvents", (), {"sweeps": -1})()
        m_ms = np.full(k, 1e3 * wall[-1] / max(k, 1))
    else:
        r, m_ms = prof
    n_k = lengths[:k].astype(np.float64)
    n_k1 = lengths[1: k + 1].astype(np.float64)
    m_ms = m_ms[:k].astype(np.float64)
    merge_bytes = 2.0 * n_k + 2.0 * n_k1
    total_wall = float(sum(wall))
    res = {"spec": spec, "data": data, "d": d, "sha": sha, "merges": m, "tokens": t, "lengths": lengths,
           "k": int(k), "wall": wall, "warm_s": warm_s, "value": k * len(wall) / total_wall,
           "ms_per_step": 1e3 * total_wall / len(wall), "m_ms": m_ms, "n_k": n_k, "merge_bytes": merge_bytes,
           "sweeps": int(r.sweeps), "merge_ms_sum": float(m_ms.sum()), "table_usage": list(usage),
           "merge_gbps": float(merge_bytes.sum() / (m_ms.sum() / 1e3) / 1e9) if k else 0.0}
    if cpu_reps:
        import oracle
        log("timing the CPU oracle (chunk-multiset, single thread) on %s, %d run(s)" % (spec.name, cpu_reps))
        times = []
        for _ in range(cpu_reps):
            with one_core():
                t0 = time.perf_counter()
                om, ot, _ = oracle.train_chunks(data, n_merges)
                times.append(time.perf_counter() - t0)
        cpu_s = float(np.median(times))
        same = bool(np.array_equal(om, m.cpu().numpy().astype(np.int64)) and
                    np.array_equal(ot, t.cpu().numpy().astype(np.uint32)))
        res.update({"cpu_s": cpu_s, "cpu_merges_s": len(om) / cpu_s, "cpu_reps": cpu_reps, "identical": same})
        log("%s oracle: %.2f s, bit-identical to the GPU result: %s" % (spec.name, cpu_s, same))
    return res


def chunked_leg(bpe, spec, d, ref_m, ref_t, ref_oracle, steps, warmup, np, torch, time, log):
    """Training over the corpus's distinct words (bpe_train_chunked): each
    distinct word once with its frequency, the tokens through the encoder.
    Whole jobs on the device-resident corpus, timed by the wall clock (word
    passes, merges, tokens and the copy-out included); the result is
    compared with the full-array path's (ref_m, ref_t), and so with the
    oracle where that was (ref_oracle). Timed twice: as called (where the
    distinct words would not save work the call runs the full-array path)
    and with BPE_FLAG_ALWAYS_CHUNKS."""
    out = {}
    for always in (False, True):
        def job():
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            m, t = bpe.train_chunked(d, spec.n_merges, spec.table_log2, always_chunks=always)
            torch.cuda.synchronize()
            return time.perf_counter() - t0, m, t
        for _ in range(warmup):
            job()
        walls, m, t = [], None, None
        for _ in range(steps):
            dt, m, t = job()
            walls.append(dt)
        same = bool(torch.equal(m, ref_m) and torch.equal(t, ref_t))
        k = int(m.shape[0])
        rate = k * len(walls) / sum(walls)
        key = "over_chunks" if always else "as_called"
        out[key] = {"merges_per_s": round(rate, 1), "s_per_job": round(float(np.median(walls)), 4),
                    "jobs": steps, "identical_to_full_array_path": same,
                    "bit_identical_to_oracle": (same and ref_oracle) if ref_oracle is not None else None}
        log("%s chunked (%s): %.1f merges/s, %.3f s per job, identical to the full-array path: %s"
            % (spec.name, key, rate, float(np.median(walls)), same))
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", type=int, default=3, help="workload 1..5 (default 3: 256 MiB, 32k merges)")
    ap.add_argument("--merges", type=int, default=None, help="override the merge count")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other four workloads (one job each, with the oracle check)")
    ap.add_argument("--report", default=None, help="write per-iteration details to this JSON file")
    ap.add_argument("--no-inference", action="store_true", help="skip the inference and encoding legs")
    ap.add_argument("--save-merges", default=None, metavar="PATH", help="write the learned merges (.npy)")
    ap.add_argument("--inference-only", default=None, metavar="PATH",
                    help="skip training: time inference and encoding with the merges saved in PATH (.npy) "
                         "by --save-merges")
    ap.add_argument("--inference-reps", type=int, default=20)
    ap.add_argument("--no-iteration-events", action="store_true",
                    help="time whole jobs only (no HIP event per iteration; for runs under a profiler)")
    ap.add_argument("--run-chunk", type=int, default=0, metavar="K",
                    help="with --no-iteration-events: enqueue K iterations at a time, waiting in between")
    ap.add_argument("--no-chunked", action="store_true",
                    help="skip the legs that train over the distinct words (bpe_train_chunked)")
    ap.add_argument("--chunked-only", action="store_true",
                    help="only time training over the distinct words on the workload (for profiles)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="first run a plain device-to-device copy of BYTES bytes (hardware-counter reference)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the training path here is single-GPU and --gpus %d is not "
              "supported (multi-GPU sharding is a design note, not built)" % max(args.gpus, world),
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import bpe_merge_amd as bpe
    import corpus

    if args.copy_calibration:
        nb = args.copy_calibration // 16 * 16
        src = torch.ones(nb // 4, dtype=torch.int32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: %d bytes read + %d bytes written per copy, 2 copies" % (nb, nb))
        del src, dst

    spec = corpus.CONFIGS[args.config]
    if args.merges is not None:
        spec = spec.scaled(spec.n_bytes, n_merges=args.merges)
    n_merges, tlog2 = spec.n_merges, spec.table_log2
    T = 1 << tlog2

    if args.chunked_only:
        log("generating %s (%d bytes)" % (spec.name, spec.n_bytes))
        data = corpus.generate(spec)
        d = torch.from_numpy(data).to("cuda:0")
        walls, k = [], 0
        for i in range(args.warmup + args.steps):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            m, t = bpe.train_chunked(d, n_merges, tlog2)
            torch.cuda.synchronize()
            if i >= args.warmup:
                walls.append(time.perf_counter() - t0)
            k = int(m.shape[0])
            log("%s chunked job %d: %.3f s, %d merges" % (spec.name, i + 1, time.perf_counter() - t0, k))
        out = {"metric": "BPE train merges/sec over the distinct words", "value": round(k * len(walls) / sum(walls), 1),
               "unit": "merges/s", "n_gpus": 1, "steps": len(walls), "warmup": args.warmup,
               "ms_per_step": round(1e3 * sum(walls) / len(walls), 3), "higher_is_better": True, "scaling": "weak",
               "vs_baseline": None, "dtype": "u16", "data": "synthetic",
               "config": {"workload": "%s: %d-byte seeded corpus (%s), %d merges, pair table 2^%d"
                                      % (spec.name, spec.n_bytes, spec.kind, n_merges, tlog2)}}
        print(json.dumps(out), flush=True)
        return 0

    if args.inference_only:
        log("generating %s (%d bytes)" % (spec.name, spec.n_bytes))
        data = corpus.generate(spec)
        d = torch.from_numpy(data).to("cuda:0")
        m = torch.from_numpy(np.load(args.inference_only, allow_pickle=False)).to("cuda:0")
        inf = inference_leg(args, bpe, spec, data, d, m, np, torch, time, log,
                            source="learned by an earlier run on the same corpus")
        enc = encode_leg(args, bpe, spec, data, d, m, np, time, log,
                         source="learned by an earlier run on the same corpus")
        out = dict(inf)
        out["encoding"] = enc
        out.update({"n_gpus": 1, "steps": inf["runs"], "warmup": 1, "higher_is_better": True, "scaling": "weak",
                    "vs_baseline": None, "dtype": "u8", "data": "synthetic",
                    "config": {"workload": inf["workload"], "corpus_bytes": spec.n_bytes}})
        print(json.dumps(out), flush=True)
        return 0

    # the large workloads once, the others three times (median)
    cpu_reps = 0 if args.no_cpu_baseline else (1 if spec.n_bytes >= (256 << 20) else 3)
    res = train_leg(bpe, corpus, spec, args.steps, args.warmup, np, torch, time, log, cpu_reps,
                    events=not args.no_iteration_events, chunk=args.run_chunk)
    m, t, lengths, k = res["merges"], res["tokens"], res["lengths"], res["k"]
    m_ms, n_k, merge_bytes = res["m_ms"], res["n_k"], res["merge_bytes"]
    data, d, sha = res["data"], res["d"], res["sha"]
    it_s = m_ms / 1e3
    # an iteration that sweeps the pair table reads it twice (maximum, then
    # candidates); the others read only the candidate list's slots (not
    # credited). Per-iteration figures leave the sweeps out.
    sweep_bytes = 2 * 8.0 * T * res["sweeps"]
    sym_per_s_agg = float(n_k.sum() / it_s.sum())
    hbm_agg = float((merge_bytes.sum() + sweep_bytes) / it_s.sum() / 1e9)
    merge_gbps = res["merge_gbps"]
    per_it_sym = n_k / it_s
    per_it_gbps = merge_bytes / it_s / 1e9
    dominant = "k_merge"  # the merge pass takes >95% of the time (see kernels_ms_per_step)
    achieved, avg_bytes, avg_ms = merge_gbps, float(merge_bytes.mean()), float(m_ms.mean())
    windows = traffic_windows(spec.name, dominant)

    cpu = None
    if cpu_reps:
        cpu = {"value": round(res["cpu_merges_s"], 3), "unit": "merges/s", "cores": 1, "kind": "oracle",
               "sample": "the whole workload (%d bytes, %d merges) through the chunk-multiset C oracle "
                         "(oracle/bpe_oracle.c, train_chunks), one thread, %.2f s including chunking (median "
                         "of %d); GPU result bit-identical: %s"
                         % (spec.n_bytes, n_merges, res["cpu_s"], cpu_reps, res["identical"]),
               "pinned": "one core (sched_setaffinity)", **cpu_facts()}
        if spec.n_bytes <= (1 << 20):
            # the literal definition (a full recount every iteration) is
            # feasible only on the smallest workload
            import oracle
            with one_core():
                t0 = time.perf_counter()
                lm, lt, _ = oracle.train_literal(data, n_merges)
                lit_s = time.perf_counter() - t0
            om, ot, _ = oracle.train_chunks(data, n_merges)
            cpu["literal"] = {"value": round(len(lm) / lit_s, 3), "unit": "merges/s",
                              "sample": "the literal C oracle (train_literal: full recount each iteration), "
                                        "one thread, %.2f s; equal to the chunk oracle: %s"
                                        % (lit_s, bool(np.array_equal(lm, om) and np.array_equal(lt, ot)))}

    chunked = None
    if not args.no_chunked:
        chunked = chunked_leg(bpe, spec, d, m, t, res.get("identical"), 3, 1, np, torch, time, log)

    if args.save_merges:
        np.save(args.save_merges, m.cpu().numpy())
    inference = None
    encoding = None
    if not args.no_inference:
        inference = inference_leg(args, bpe, spec, data, d, m, np, torch, time, log)
        encoding = encode_leg(args, bpe, spec, data, d, m, np, time, log, train_tokens=t)

    # the other workloads: one timed job each (after one unprofiled job on
    # the small ones), with the oracle's result on the same bytes
    configs = None
    if not args.no_configs and args.merges is None:
        configs = {}
        del d, res["d"]
        for c in sorted(corpus.CONFIGS):
            if c == args.config:
                continue
            cs = corpus.CONFIGS[c]
            small = cs.n_bytes < (256 << 20)
            r = train_leg(bpe, corpus, cs, 1, 1 if small else 0, np, torch, time, log,
                          0 if args.no_cpu_baseline else 1)
            frac = r["merge_gbps"] / HBM_PEAK_GBPS
            ck = None
            if not args.no_chunked:
                ck = chunked_leg(bpe, cs, r["d"], r["merges"], r["tokens"], r.get("identical"), 1,
                                 1 if small else 0, np, torch, time, log)
            configs[cs.name] = {
                "workload": "%d-byte seeded corpus (%s), %d merges, pair table 2^%d, sha256 %s"
                            % (cs.n_bytes, cs.kind, cs.n_merges, cs.table_log2, r["sha"][:16]),
                "merges_done": r["k"], "merges_per_s": round(r["value"], 1), "s_per_job": round(r["ms_per_step"] / 1e3, 4),
                "k_merge_ms": round(r["merge_ms_sum"], 3), "k_merge_gbps": round(r["merge_gbps"], 1),
                "k_merge_frac_of_peak": round(frac, 4), "table_sweeps": r["sweeps"],
                "table_slots_claimed": r["table_usage"][1], "table_claim_limit": r["table_usage"][2],
                "final_tokens": int(r["tokens"].shape[0]),
                "cpu_oracle_merges_per_s": round(r["cpu_merges_s"], 1) if "cpu_merges_s" in r else None,
                "bit_identical_to_oracle": r.get("identical"),
                "chunked": ck,
                "note": ("launch- and latency-bound: the roofline fraction is not meaningful"
                         if cs.n_bytes <= (1 << 20) else
                         "the 64 MiB symbol array and 16 MiB table fit the 256 MB last-level cache; GB/s is "
                         "effective" if cs.n_bytes <= (16 << 20) else "HBM-bound"),
            }
            log("%s: %.1f merges/s, k_merge %.1f GB/s (%.1f%% of peak), bit-identical: %s"
                % (cs.name, r["value"], r["merge_gbps"], 100 * frac, r.get("identical")))
            del r

    out = {
        "metric": "BPE train merges/sec + symbols/sec per merge, 256 MiB/32k merges; HBM GB/s",
        "value": round(res["value"], 3),
        "unit": "merges/s",
        "n_gpus": 1,
        "steps": len(res["wall"]),
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u16",
        "data": "synthetic",
        "config": {
            "workload": "%s: %d-byte seeded corpus (%s), %d merges, pair table 2^%d, sha256 %s"
                        % (spec.name, spec.n_bytes, spec.kind, n_merges, tlog2, sha[:16]),
            "corpus_bytes": spec.n_bytes,
            "n_merges": n_merges,
            "merges_done": int(k),
            "table_slots": T,
            "table_slots_claimed": res["table_usage"][1],
            "final_tokens": int(t.shape[0]),
        },
        "symbols_per_s_per_merge": {"aggregate": sym_per_s_agg, "p10": pct(per_it_sym, 10),
                                    "p50": pct(per_it_sym, 50), "p90": pct(per_it_sym, 90)},
        "hbm_gbps_per_iteration": {"aggregate": round(hbm_agg, 1), "frac_of_peak": round(hbm_agg / HBM_PEAK_GBPS, 4),
                                   "p10": round(pct(per_it_gbps, 10), 1), "p50": round(pct(per_it_gbps, 50), 1),
                                   "p90": round(pct(per_it_gbps, 90), 1)},
        "kernels_ms_per_step": {"k_merge": round(res["merge_ms_sum"], 3), "k_merge_gbps": round(merge_gbps, 1),
                                "table_sweeps": res["sweeps"]},
        "warmup_unprofiled_s": [round(x, 3) for x in res["warm_s"]],
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     # measured bytes per launch over the whole run (committed
                     # rocprofv3 counters), beside the windows it was taken in
                     "traffic": (next((w["measured"] for w in windows if w["launches"] == k), windows[-1]["measured"])
                                 if windows else None),
                     "traffic_windows": windows,
                     "traffic_source": ("profiles/traffic_%s_%s.json" % (dominant, spec.name)) if windows else None,
                     "bytes_per_launch": round(avg_bytes), "avg_launch_ms": round(avg_ms, 5)},
        "cpu_baseline": cpu,
        "chunked": chunked,
        "configs": configs,
        "inference": inference,
        "encoding": encoding,
    }
    if args.report:
        with open(args.report, "w") as fh:
            json.dump({"summary": out, "lengths": lengths.tolist(), "merge_ms": m_ms.tolist()}, fh)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
