"""Benchmark of the TurboQuant hot path on one MI355X.

One step = the whole path on one batch of the TurboQuant_prod workload (16 sequences x 8 KV heads x
16384 tokens x d = 128, bf16 keys with outlier channels and a log-normal per-token scale):
TurboQuant_prod b = 4 encode of all 2,097,152 keys (norm, dense rotation on MFMA, 3-bit Lloyd-Max
bucketize, bit-pack, residual, 1-bit QJL sketch of the residual with S' on MFMA, residual norm),
then the query prologue and the unbiased scores of 32 query heads per sequence (GQA 4) over the
packed keys.  Inputs are resident in HBM before timing; the step rotates through several input and
output buffer sets whose total exceeds the last-level cache.  The single-layer KV-key step (1 x 8 x
32768 keys, MSE b = 3) is reported beside it as a nested secondary line.

Prints ONE JSON line.  `--gpus N` with N > 1 is refused: this path runs on one GPU.
"""

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
CACHE_DEFEAT_BYTES = 1.5e9


# Sources of each timed kernel: its counters stay valid while these files are unchanged.
KERNEL_SOURCES = {
    "encode": ("tq_device.h", "tq_internal.h", "tq_encode_mse32.hip"),
    "prod_encode": ("tq_device.h", "tq_internal.h", "tq_encode_prod128.hip"),
    "scores": ("tq_device.h", "tq_internal.h", "tq_decode.h", "tq_cache.h", "tq_score128.hip"),
}
# (encode kernel, score kernel) of each step workload, as the profiler names them
HEADLINE_KERNELS = {
    "c3": ("k_encode_prod_d128<3, true, 2> (prod b=4, dense R, bf16 keys)",
           "k_scores_d128<3, true, false, 0> (prod, GQA 4)"),
    "c2": ("k_encode_mse32_d128<3, true, 2> (MSE b=3, dense R, bf16 keys)",
           "k_scores_d128<3, false, false, 0> (MSE, GQA 4)"),
}
# name prefixes of those kernels in a rocprofv3 database (for the counter summary)
PMC_KERNELS = {
    "c3:prod_encode": "k_encode_prod_d128<3, true, 2>",
    "c3:scores": "k_scores_d128<3, true, false, 0>",
    "c2:encode": "k_encode_mse32_d128<3, true, 2>",
    "c2:scores": "k_scores_d128<3, false, false, 0>",
}


def kernel_source_hash(kind):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        h.update(open(os.path.join(ROOT, "kv_cache_compression_turboquant_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profile(key):
    """HBM bytes per launch of kernel `key` ("c3:encode", ...) from the committed counter summary,
    if it was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
    except Exception:
        return None
    ent = data.get(key)
    if not ent or ent.get("source_hash") != kernel_source_hash(key.split(":")[1]):
        return None
    return ent.get("hbm_bytes_per_launch")


COPY_PROBE_BYTES = 512 << 20


def copy_probe(torch, dev, reps=3):
    """Plain device-to-device copies of a known size: what FETCH_SIZE / WRITE_SIZE read for
    them calibrates the counters against algorithmic bytes."""
    src = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()


def _pmc_rows(db, counter):
    import sqlite3
    con = sqlite3.connect(db)
    q = ("select k.name, p.value from counters_collection p join kernels k "
         "on p.dispatch_id = k.dispatch_id where p.counter_name = ?")
    out = {}
    for name, v in con.execute(q, (counter,)).fetchall():
        out.setdefault(name, []).append(float(v))
    return out


def _short(name):
    return name.replace("void ", "").replace("tq::(anonymous namespace)::", "").split("(")[0]


def pmc_summary(fetch_db, write_db):
    """HBM bytes per dispatch from FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled
    by bytes / counted for the copy probe of the same run."""
    fetch = _pmc_rows(fetch_db, "FETCH_SIZE")
    write = _pmc_rows(write_db, "WRITE_SIZE")
    probe_kib = COPY_PROBE_BYTES / 1024.0

    def probe_factor(rows):
        vals = [v for name, vs in rows.items() if "copy" in name.lower() for v in vs
                if 0.5 * probe_kib < v < 2.0 * probe_kib]
        if not vals:
            raise SystemExit("pmc-summary: no copy-probe dispatch found (run bench.py with --copy-probe)")
        return probe_kib / float(np.median(vals)), len(vals)

    ff, nf = probe_factor(fetch)
    fw, nw = probe_factor(write)
    lines = [f"copy probe {COPY_PROBE_BYTES} B: FETCH_SIZE scale {ff:.4f} ({nf} dispatches), "
             f"WRITE_SIZE scale {fw:.4f} ({nw} dispatches)",
             f"{'kernel':60s} {'dispatches':>10s} {'fetch MB':>10s} {'write MB':>10s} {'HBM MB':>10s}"]
    table = {}
    for name in sorted(set(fetch) & set(write)):
        if "copy" in name.lower() or "elementwise" in name.lower() or "fill" in name.lower():
            continue
        fb = float(np.mean(fetch[name])) * 1024.0 * ff
        wb = float(np.mean(write[name])) * 1024.0 * fw
        table[_short(name)] = (name, len(fetch[name]), fb, wb)
        lines.append(f"{_short(name)[:60]:60s} {len(fetch[name]):10d} {fb / 1e6:10.2f} {wb / 1e6:10.2f} "
                     f"{(fb + wb) / 1e6:10.2f}")
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        out = json.load(open(path))
    except Exception:
        out = {}
    out["_note"] = ("HBM bytes per dispatch = FETCH_SIZE and WRITE_SIZE (KiB per dispatch) x 1024, each scaled "
                    "by the copy-probe factor; valid only for the kernel sources of source_hash")
    for key, prefix in PMC_KERNELS.items():
        hit = [v for k, v in table.items() if v[0].startswith("void tq::(anonymous namespace)::" + prefix)]
        if not hit:
            continue
        name, nd, fb, wb = hit[0]
        out[key] = {"kernel": name[:120], "dispatches": nd, "fetch_bytes": fb, "write_bytes": wb,
                    "hbm_bytes_per_launch": fb + wb, "fetch_scale": ff, "write_scale": fw,
                    "source_hash": kernel_source_hash(key.split(":")[1])}
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("\n".join(lines))


def trace_summary(db):
    """Markdown table of a rocprofv3 --kernel-trace database: calls and mean / min / max duration
    per kernel, longest total first."""
    import sqlite3
    con = sqlite3.connect(db)
    rows = {}
    for name, dur in con.execute("select name, duration from kernels"):
        rows.setdefault(_short(name), []).append(float(dur) / 1e3)
    lines = ["| kernel | calls | mean us | min us | max us | total us |", "|---|---|---|---|---|---|"]
    for name, v in sorted(rows.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{name[:90]}` | {len(v)} | {np.mean(v):.2f} | {np.min(v):.2f} | {np.max(v):.2f} | "
                     f"{np.sum(v):.1f} |")
    print("\n".join(lines))


def pmc_table(db):
    """Markdown table of a rocprofv3 --pmc database: per kernel, the mean over dispatches of every
    counter collected (values as the profiler reports them, summed over the device per dispatch)."""
    import sqlite3
    con = sqlite3.connect(db)
    q = ("select k.name, p.counter_name, p.value from counters_collection p join kernels k "
         "on p.dispatch_id = k.dispatch_id")
    acc = {}
    for name, cn, v in con.execute(q):
        acc.setdefault(_short(name), {}).setdefault(cn, []).append(float(v))
    counters = sorted({c for d in acc.values() for c in d})
    lines = ["| kernel | dispatches | " + " | ".join(counters) + " |", "|---|---|" + "---|" * len(counters)]
    for name, d in sorted(acc.items()):
        nd = max(len(v) for v in d.values())
        lines.append(f"| `{name[:70]}` | {nd} | " + " | ".join(
            f"{np.mean(d[c]):.4g}" if c in d else "" for c in counters) + " |")
    print("\n".join(lines))


def cpu_baseline(cfg, keys_bits, q, budget_s=12.0):
    """The oracle, as it stands, on a bounded sample of the same workload: one KV head slab of
    keys encoded and scored by the 4 query heads that share it (the full step is 8 such slabs of
    32768 tokens)."""
    import oracle
    from kv_cache_compression_turboquant_amd import workloads as wl
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    rot = oracle.dense_rotation(cfg.d, cfg.rot_seed)
    cb = oracle.codebook(cfg.d, cfg.bits)
    ratio = cfg.hq // cfg.hkv
    tokens = 0
    scores = 0
    t0 = time.perf_counter()
    chunk = 4096
    head = 0
    while True:
        x = wl.bf16_bits_to_f32(keys_bits[0, head % cfg.hkv, (tokens % cfg.T):(tokens % cfg.T) + chunk])
        enc = oracle.encode_mse(x.astype(np.float64), rot, cb)
        qs = q[0, (head % cfg.hkv) * ratio:((head % cfg.hkv) + 1) * ratio].astype(np.float64)
        s = oracle.scores_mse(qs, enc.idx, enc.norms, rot, cb)
        tokens += x.shape[0]
        scores += s.size
        if time.perf_counter() - t0 > budget_s:
            break
        if tokens % cfg.T == 0:
            head += 1
    dt = time.perf_counter() - t0
    cpu = platform.processor() or platform.machine()
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except Exception:
        pass
    return {"value": scores / dt, "unit": "scores/s (encode + score of the sampled keys)",
            "cores": int(threads), "kind": "oracle",
            "sample": f"{tokens} keys of the workload (4096-key chunks of one KV head slab) encoded "
                      f"and scored by their {ratio} query heads in {dt:.1f} s; numpy fp64; {cpu}"}


def _cpu_info():
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    cpu = platform.processor() or platform.machine()
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except Exception:
        pass
    return int(threads), cpu


def cpu_baseline_decode(cfg, b, t_cap, budget_s=10.0):
    """The oracle on a bounded sample of the decode loop: one decode step of one (sequence, KV
    head) group (append the new key and value, then attention of its query heads over a prefix of
    the cache), repeated on growing prefixes until the budget is spent; scaled to decode tokens/s
    of the full step (every group at the full context length)."""
    import oracle
    from kv_cache_compression_turboquant_amd import workloads as wl
    threads, cpu = _cpu_info()
    rot = oracle.dense_rotation(cfg.d, cfg.rot_seed)
    cb = oracle.codebook(cfg.d, b)
    ratio = cfg.hq // cfg.hkv
    T = 8192
    kx = wl.bf16_bits_to_f32(wl.kv_keys(cfg, T=T, B=1)[0, 0]).astype(np.float64)
    vx = wl.bf16_bits_to_f32(wl.kv_values(cfg, T=T, B=1)[0, 0]).astype(np.float64)
    q = wl.kv_queries(cfg)[0:1, :ratio].astype(np.float64)
    ke, ve = oracle.encode_mse(kx, rot, cb), oracle.encode_mse(vx, rot, cb)
    tokens = 0
    t0 = time.perf_counter()
    steps = 0
    while True:
        n = T - 1 - (steps % 64)
        new_k = oracle.encode_mse(kx[n:n + 1], rot, cb)
        new_v = oracle.encode_mse(vx[n:n + 1], rot, cb)
        kidx = np.concatenate([ke.idx[:n], new_k.idx])[None, None]
        vidx = np.concatenate([ve.idx[:n], new_v.idx])[None, None]
        kn = np.concatenate([ke.norms[:n], new_k.norms])[None, None]
        vn = np.concatenate([ve.norms[:n], new_v.norms])[None, None]
        oracle.decode_attention(q, kidx, kn, vidx, vn, rot, rot, cb, cb, 1 / np.sqrt(cfg.d))
        tokens += n + 1
        steps += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    per_token_group = dt / tokens                       # seconds per cached token of one group
    step_s = per_token_group * t_cap * cfg.B * cfg.hkv  # one full decode step, every group
    return {"value": cfg.B / step_s, "unit": "decode tokens/s (4 sequences per step)", "cores": threads,
            "kind": "oracle",
            "sample": f"{steps} single-token decode steps of one (sequence, KV head) group over prefixes of "
                      f"{T - 64}..{T} tokens (append key and value, attention of its {ratio} query heads) in "
                      f"{dt:.1f} s, scaled to {cfg.B} x {cfg.hkv} groups x {t_cap} tokens; numpy fp64; {cpu}"}


def cpu_baseline_prod(cfg, kind, budget_s=10.0):
    """The oracle on a bounded sample of the prod workload: 4096-key chunks of one KV head slab
    encoded (TurboQuant_prod b = 4) and scored by their query heads; keys/s and scores/s."""
    import oracle
    from kv_cache_compression_turboquant_amd import workloads as wl
    threads, cpu = _cpu_info()
    rot = {"dense": oracle.dense_rotation(cfg.d, 1), "wht": oracle.wht_rotation(cfg.d, 1),
           "block_wht": oracle.block_wht_rotation(cfg.d, 1, 32)}[kind]
    smat = oracle.qjl_matrix(cfg.d, 2)
    cb = oracle.codebook(cfg.d, cfg.bits - 1)
    ratio = cfg.hq // cfg.hkv
    x = wl.bf16_bits_to_f32(wl.kv_keys(cfg, T=4096, B=1)[0, 0]).astype(np.float64)
    q = wl.kv_queries(cfg)[0, :ratio].astype(np.float64)
    keys = scores = 0
    t0 = time.perf_counter()
    while True:
        encp = oracle.encode_prod(x, rot, cb, smat)
        s = oracle.scores_prod(q, encp, rot, cb, smat)
        keys += x.shape[0]
        scores += s.size
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": scores / dt, "unit": "scores/s (prod encode + score of the sampled keys)", "cores": threads,
            "kind": "oracle", "encode_vectors_per_s": keys / dt,
            "sample": f"{keys} keys (4096-key chunks of one KV head slab, {kind} rotation) encoded and scored by "
                      f"their {ratio} query heads in {dt:.1f} s; numpy fp64; {cpu}"}


def cpu_baseline_headdim(d, kb, vb, ratio, budget_s=10.0):
    """The oracle on a bounded sample of the head-dim workload: one (sequence, KV head) group of
    4096 tokens, keys (MSE kb bits) and values (MSE vb bits) encoded, then the scores and the decode
    attention of its query heads over them, repeated until the budget is spent.  Reports
    attention KV positions/s (the GPU line's kv_positions_per_s) and the encode and score rates."""
    import oracle
    from kv_cache_compression_turboquant_amd import workloads as wl
    threads, cpu = _cpu_info()
    rot = oracle.dense_rotation(d, 1)
    cbk, cbv = oracle.codebook(d, kb), oracle.codebook(d, vb)
    T = 4096
    kx = wl.bf16_bits_to_f32(wl.kv_tensor_bf16(1, 1, T, d, seed=1, outlier_seed=2, scale_seed=3)[0, 0]).astype(np.float64)
    vx = wl.bf16_bits_to_f32(wl.kv_tensor_bf16(1, 1, T, d, seed=4, outlier_seed=5, scale_seed=None)[0, 0]).astype(np.float64)
    q = wl.gaussian((1, ratio, d), 6).astype(np.float64)
    t_enc = t_sc = t_at = 0.0
    reps = 0
    t0 = time.perf_counter()
    while True:
        a = time.perf_counter()
        ke, ve = oracle.encode_mse(kx, rot, cbk), oracle.encode_mse(vx, rot, cbv)
        b = time.perf_counter()
        oracle.scores_mse(q[0], ke.idx, ke.norms, rot, cbk)
        c = time.perf_counter()
        oracle.decode_attention(q, ke.idx[None, None], ke.norms[None, None], ve.idx[None, None], ve.norms[None, None],
                                rot, rot, cbk, cbv, 1 / np.sqrt(d))
        e = time.perf_counter()
        t_enc += b - a
        t_sc += c - b
        t_at += e - c
        reps += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": reps * T / t_at, "unit": "KV positions/s (decode attention over packed K and V)",
            "cores": threads, "kind": "oracle", "encode_vectors_per_s": 2 * reps * T / t_enc,
            "scores_per_s": reps * T * ratio / t_sc,
            "sample": f"{reps} rounds of one group of {T} tokens at d = {d}: keys ({kb} bits) and values ({vb} bits) "
                      f"encoded, scored and attended by {ratio} query heads, {dt:.1f} s; numpy fp64; {cpu}"}


def cpu_baseline_mse(cfg, kind, b, budget_s=10.0):
    """The oracle on a bounded sample of the MSE-key workload: 4096-key chunks of one KV head slab
    encoded (TurboQuant_mse, b bits, the given rotation as an explicit matrix) and scored by their
    query heads; scores/s and encoded keys/s."""
    import oracle
    from kv_cache_compression_turboquant_amd import workloads as wl
    threads, cpu = _cpu_info()
    rot = {"dense": oracle.dense_rotation(cfg.d, 1), "wht": oracle.wht_rotation(cfg.d, 1),
           "block_wht": oracle.block_wht_rotation(cfg.d, 1, 32)}[kind]
    cb = oracle.codebook(cfg.d, b)
    ratio = cfg.hq // cfg.hkv
    x = wl.bf16_bits_to_f32(wl.kv_keys(cfg, T=4096, B=1)[0, 0]).astype(np.float64)
    q = wl.kv_queries(cfg)[0, :ratio].astype(np.float64)
    keys = scores = 0
    t_enc = 0.0
    t0 = time.perf_counter()
    while True:
        a = time.perf_counter()
        enc = oracle.encode_mse(x, rot, cb)
        t_enc += time.perf_counter() - a
        s = oracle.scores_mse(q, enc.idx, enc.norms, rot, cb)
        keys += x.shape[0]
        scores += s.size
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": scores / dt, "unit": "scores/s (MSE encode + score of the sampled keys)", "cores": threads,
            "kind": "oracle", "encode_vectors_per_s": keys / t_enc,
            "sample": f"{keys} keys (4096-key chunks of one KV head slab, {kind} rotation, b = {b}) encoded and "
                      f"scored by their {ratio} query heads in {dt:.1f} s; numpy fp64; {cpu}"}


def cpu_baseline_split(cfg, bo, br, budget_s=10.0):
    """The oracle on a bounded sample of the split-code workload: 4096-key chunks of one KV head
    split-encoded (outlier half b_o bits, rest b_r) and scored by their query heads; scores/s."""
    import oracle
    from kv_cache_compression_turboquant_amd import workloads as wl
    threads, cpu = _cpu_info()
    r_o, r_r = oracle.dense_rotation(64, 3), oracle.dense_rotation(64, 4)
    cb_o, cb_r = oracle.codebook(64, bo), oracle.codebook(64, br)
    ratio = cfg.hq // cfg.hkv
    x = wl.bf16_bits_to_f32(wl.kv_keys(cfg, T=4096, B=1)[:, :1]).astype(np.float64)
    out = np.argsort(-np.mean(x * x, axis=(0, 2)), axis=1, kind="stable")[:, :64]
    q = wl.kv_queries(cfg)[:, :ratio].astype(np.float64)
    keys = scores = 0
    t0 = time.perf_counter()
    while True:
        enc = oracle.encode_split(x, out, r_o, r_r, cb_o, cb_r)
        s = oracle.scores_split(q, enc, r_o, r_r, cb_o, cb_r)
        keys += x.shape[2]
        scores += s.size
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": scores / dt, "unit": "scores/s (split encode + score of the sampled keys)", "cores": threads,
            "kind": "oracle", "encode_vectors_per_s": keys / dt,
            "sample": f"{keys} keys (4096-key chunks of one KV head, outlier half {bo} bits, rest {br}) encoded and "
                      f"scored by their {ratio} query heads in {dt:.1f} s; numpy fp64; {cpu}"}


def _timed(fn, steps, warmup):
    """Mean ms of fn() over `steps` calls, HIP events on the current stream."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record()
        fn(warmup + i)
        ev[i][1].record()
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in ev]))


def bench_other(name, steps, warmup, cpu_budget=0.0):
    """Per-kernel timing of the other workloads (prod scores, decode attention): not the
    headline line; reports algorithmic GB/s against the HBM peak."""
    import torch
    import kv_cache_compression_turboquant_amd as tq
    from kv_cache_compression_turboquant_amd import workloads as wl
    dev = torch.device("cuda:0")
    res = {"config": name}
    if name in ("c3", "c3wht", "c3bwht"):
        cfg = wl.CONFIGS["c3"]
        kind = {"c3": "dense", "c3wht": "wht", "c3bwht": "block_wht"}[name]
        n = cfg.B * cfg.hkv * cfg.T
        keys = torch.from_numpy(wl.kv_keys(cfg).reshape(n, cfg.d).view(np.int16)).to(dev).view(torch.bfloat16)
        q = torch.from_numpy(wl.kv_queries(cfg)).to(dev)
        rot = tq.make_rotation(cfg.d, 1, kind)
        qjl = tq.make_qjl(cfg.d, 2, rot)
        cb = tq.codebook(cfg.d, cfg.bits - 1)
        nbuf = 3
        packs = [tq.alloc_packed(n, cfg.d, cfg.bits - 1, "prod", device=dev) for _ in range(nbuf)]
        outs = [torch.empty((cfg.B, cfg.hq, cfg.T), device=dev) for _ in range(nbuf)]
        ws = torch.empty(tq.scores_workspace(cfg.B, cfg.hq, cfg.d), dtype=torch.uint8, device=dev)
        enc_ms = _timed(lambda i: tq.encode(keys, cfg.bits, "prod", cb, rot, qjl, out=packs[i % nbuf]), steps, warmup)
        sc_ms = _timed(lambda i: tq.scores(q, packs[i % nbuf], cfg.hkv, cb, rot, qjl, out=outs[i % nbuf], ws=ws),
                       steps, warmup)
        enc_bytes = n * (cfg.d * 2 + 48 + 16 + 8)
        sc_bytes = n * 72 + q.numel() * 4 + outs[0].numel() * 4
        res.update({"rotation": kind, "encode_ms": enc_ms, "encode_gbs": enc_bytes / enc_ms / 1e6,
                    "encode_vectors_per_s": n / enc_ms * 1e3,
                    "scores_ms": sc_ms, "scores_gbs": sc_bytes / sc_ms / 1e6,
                    "scores_hbm_frac": sc_bytes / sc_ms / 1e6 / HBM_PEAK_GBS,
                    "scores_per_s": outs[0].numel() / sc_ms * 1e3})
        if cpu_budget > 0:
            res["cpu_baseline"] = cpu_baseline_prod(cfg, kind, cpu_budget)
    elif name in ("c3mse", "c3msewht", "c3msebwht"):
        # TurboQuant_mse (b = 3) of the C3 keys: dense R on the matrix cores against the randomized
        # Hadamard rotations as the in-register butterfly transform
        cfg = wl.CONFIGS["c3"]
        kind = {"c3mse": "dense", "c3msewht": "wht", "c3msebwht": "block_wht"}[name]
        b = cfg.bits - 1
        n = cfg.B * cfg.hkv * cfg.T
        keys = torch.from_numpy(wl.kv_keys(cfg).reshape(n, cfg.d).view(np.int16)).to(dev).view(torch.bfloat16)
        q = torch.from_numpy(wl.kv_queries(cfg)).to(dev)
        rot = tq.make_rotation(cfg.d, 1, kind)
        cb = tq.codebook(cfg.d, b)
        nbuf = 3
        packs = [tq.alloc_packed(n, cfg.d, b, "mse", device=dev) for _ in range(nbuf)]
        outs = [torch.empty((cfg.B, cfg.hq, cfg.T), device=dev) for _ in range(nbuf)]
        ws = torch.empty(tq.scores_workspace(cfg.B, cfg.hq, cfg.d), dtype=torch.uint8, device=dev)
        enc_ms = _timed(lambda i: tq.encode(keys, b, "mse", cb, rot, out=packs[i % nbuf]), steps, warmup)
        sc_ms = _timed(lambda i: tq.scores(q, packs[i % nbuf], cfg.hkv, cb, rot, out=outs[i % nbuf], ws=ws),
                       steps, warmup)
        enc_bytes = n * (cfg.d * 2 + cfg.d * b // 8 + 4)
        sc_bytes = n * (cfg.d * b // 8 + 4) + q.numel() * 4 + outs[0].numel() * 4
        res.update({"rotation": kind, "encode_ms": enc_ms, "encode_gbs": enc_bytes / enc_ms / 1e6,
                    "encode_hbm_frac": enc_bytes / enc_ms / 1e6 / HBM_PEAK_GBS,
                    "encode_vectors_per_s": n / enc_ms * 1e3,
                    "scores_ms": sc_ms, "scores_gbs": sc_bytes / sc_ms / 1e6,
                    "scores_hbm_frac": sc_bytes / sc_ms / 1e6 / HBM_PEAK_GBS,
                    "scores_per_s": outs[0].numel() / sc_ms * 1e3})
        if cpu_budget > 0:
            res["cpu_baseline"] = cpu_baseline_mse(cfg, kind, b, cpu_budget)
    elif name in ("hd64", "hd256"):
        # head dims 64 and 256: scores and decode attention of 32 query heads over 4 x 8 x 32768 keys
        # and values (MSE, 4-bit keys, 2-bit values, dense R, bf16 inputs from the KV generator); the
        # value encode and the keys' encode as TurboQuant_prod (4 bits) are timed too
        d = 64 if name == "hd64" else 256
        B, hkv, hq, T, kb, vb = 4, 8, 32, 32768, 4, 2
        n = B * hkv * T
        rot = tq.make_rotation(d, 1)
        cbk, cbv = tq.codebook(d, kb), tq.codebook(d, vb)
        kx = torch.from_numpy(wl.kv_tensor_bf16(B, hkv, T, d, seed=1, outlier_seed=2, scale_seed=3)
                              .reshape(n, d).view(np.int16)).to(dev).view(torch.bfloat16)
        K = tq.encode(kx, kb, "mse", cbk, rot)
        # the same keys as TurboQuant_prod (kb bits: a (kb - 1)-bit stage and the QJL sketch)
        qjl = tq.make_qjl(d, 2, rot)
        cbp = tq.codebook(d, kb - 1)
        pwsb = tq.encode_workspace(n, d, kb, "prod")
        pws = torch.empty((pwsb,), dtype=torch.uint8, device=dev) if pwsb else None
        Kp = tq.encode(kx, kb, "prod", cbp, rot, qjl, ws=pws)
        prod_ms = _timed(lambda i: tq.encode(kx, kb, "prod", cbp, rot, qjl, out=Kp, ws=pws), steps, warmup)
        del Kp, pws, kx
        vx = torch.from_numpy(wl.kv_tensor_bf16(B, hkv, T, d, seed=4, outlier_seed=5, scale_seed=None)
                              .reshape(n, d).view(np.int16)).to(dev).view(torch.bfloat16)
        V = tq.encode(vx, vb, "mse", cbv, rot)
        enc_ms = _timed(lambda i: tq.encode(vx, vb, "mse", cbv, rot, out=V), steps, warmup)
        del vx
        q = torch.from_numpy(wl.gaussian((B, hq, d), 6)).to(dev)
        sc = torch.empty((B, hq, T), device=dev)
        sws = torch.empty((tq.scores_workspace(B, hq, d),), dtype=torch.uint8, device=dev)
        sc_ms = _timed(lambda i: tq.scores(q, K, hkv, cbk, rot, out=sc, ws=sws), steps, warmup)
        out = torch.empty((B, hq, d), device=dev)
        aws = torch.empty((tq.decode_attn_workspace(B, hq, hkv, T, d),), dtype=torch.uint8, device=dev)
        at_ms = _timed(lambda i: tq.decode_attn(q, K, V, hkv, cbk, cbv, rot, rot, out=out, ws=aws), steps, warmup)
        kbytes = n * (d * kb // 8 + 4)
        vbytes = n * (d * vb // 8 + 4)
        sc_bytes = kbytes + sc.numel() * 4
        res.update({"head_dim": d, "keys": [B, hkv, T], "query_heads": hq, "k_bits": kb, "v_bits": vb,
                    "value_encode_ms": enc_ms, "value_encode_frac_hbm": n * (2 * d + d * vb // 8 + 4) / enc_ms / 1e6
                    / HBM_PEAK_GBS,
                    "key_prod_encode_ms": prod_ms,
                    "key_prod_encode_frac_hbm": n * (2 * d + d * (kb - 1) // 8 + d // 8 + 8) / prod_ms / 1e6
                    / HBM_PEAK_GBS,
                    "scores_ms": sc_ms, "scores_gbs": sc_bytes / sc_ms / 1e6,
                    "scores_frac_hbm": sc_bytes / sc_ms / 1e6 / HBM_PEAK_GBS,
                    "attention_ms": at_ms, "attention_gbs": (kbytes + vbytes) / at_ms / 1e6,
                    "attention_frac_hbm": (kbytes + vbytes) / at_ms / 1e6 / HBM_PEAK_GBS,
                    "kv_positions_per_s": n / at_ms * 1e3})
        if cpu_budget > 0:
            res["cpu_baseline"] = cpu_baseline_headdim(d, kb, vb, hq // hkv, cpu_budget)
    elif name in ("c4b2", "c4b4"):
        cfg = wl.CONFIGS["c4"]
        b = 2 if name == "c4b2" else 4
        n = cfg.B * cfg.hkv * cfg.T
        rot = tq.make_rotation(cfg.d, 1)
        cb = tq.codebook(cfg.d, b)
        kx = torch.from_numpy(wl.kv_keys(cfg).reshape(n, cfg.d).view(np.int16)).to(dev).view(torch.bfloat16)
        nbuf = 2
        Ks = [tq.encode(kx, b, "mse", cb, rot)]
        Ks.append(tq.alloc_packed(n, cfg.d, b, "mse", device=dev))
        Ks[1].idx.copy_(Ks[0].idx); Ks[1].norms.copy_(Ks[0].norms)
        del kx
        vx = torch.from_numpy(wl.kv_values(cfg).reshape(n, cfg.d).view(np.int16)).to(dev).view(torch.bfloat16)
        enc_v_ms = _timed(lambda i: tq.encode(vx, b, "mse", cb, rot, layout="blocked"), 3, 1)
        Vs = [tq.encode(vx, b, "mse", cb, rot, layout="blocked")]
        Vs.append(tq.alloc_packed(n, cfg.d, b, "mse", device=dev, layout="blocked"))
        Vs[1].idx.copy_(Vs[0].idx); Vs[1].norms.copy_(Vs[0].norms)
        del vx
        q = torch.from_numpy(wl.kv_queries(cfg)).to(dev)
        out = torch.empty((cfg.B, cfg.hq, cfg.d), device=dev)
        ws = torch.empty(tq.decode_attn_workspace(cfg.B, cfg.hq, cfg.hkv, cfg.T, cfg.d), dtype=torch.uint8, device=dev)
        at_ms = _timed(lambda i: tq.decode_attn(q, Ks[i % nbuf], Vs[i % nbuf], cfg.hkv, cb, cb, rot, rot, out=out, ws=ws),
                       steps, warmup)
        words = cfg.d * b // 32
        bytes_ = 2 * n * (words * 4 + 4) + q.numel() * 4 + out.numel() * 4
        res.update({"bits": b, "encode_v_blocked_ms": enc_v_ms, "attn_ms": at_ms, "attn_gbs": bytes_ / at_ms / 1e6,
                    "attn_hbm_frac": bytes_ / at_ms / 1e6 / HBM_PEAK_GBS,
                    "kv_positions_per_s": n / at_ms * 1e3})
    elif name == "c4o8":
        # Decode attention with outlier-8 keys on the attention workload (4 x 131072 tokens x 8 KV
        # heads, 32 query heads): keys with their 8 outlier channels per head (largest mean square
        # over the first 4096 tokens) as int8 and the rest at 3 bits, values at 2 bits.
        cfg = wl.CONFIGS["c4"]
        kbits, vbits, n_o = 3, 2, 8
        n = cfg.B * cfg.hkv * cfg.T
        rot = tq.make_rotation(cfg.d, 1)
        cbk, cbv = tq.codebook(cfg.d, kbits), tq.codebook(cfg.d, vbits)
        kb = wl.kv_keys(cfg)
        xs = wl.bf16_bits_to_f32(kb[0, :, :4096]).astype(np.float64)
        outl = np.argsort(-np.mean(xs * xs, axis=1), axis=1, kind="stable")[:, :n_o]
        del xs
        o = tq.make_outlier8(outl)
        kx = torch.from_numpy(kb.view(np.int16)).to(dev).view(torch.bfloat16)
        del kb
        enc_k_ms = _timed(lambda i: tq.encode_outlier8(kx, o, cbk, rot), 3, 1)
        K = tq.encode_outlier8(kx, o, cbk, rot)
        del kx
        vx = torch.from_numpy(wl.kv_values(cfg).reshape(n, cfg.d).view(np.int16)).to(dev).view(torch.bfloat16)
        V = tq.encode(vx, vbits, "mse", cbv, rot, layout="blocked")
        del vx
        q = torch.from_numpy(wl.kv_queries(cfg)).to(dev)
        out = torch.empty((cfg.B, cfg.hq, cfg.d), device=dev)
        ws = torch.empty(tq.decode_attn_outlier8_workspace(cfg.B, cfg.hq, cfg.hkv, cfg.T), dtype=torch.uint8,
                         device=dev)
        at_ms = _timed(lambda i: tq.decode_attn_outlier8(q, K, V, cfg.hkv, o, cbk, cbv, rot, rot, out=out, ws=ws),
                       steps, warmup)
        bytes_ = n * (cfg.d * kbits // 8 + 4 + n_o + 4) + n * (cfg.d * vbits // 8 + 4) + q.numel() * 4 + out.numel() * 4
        res.update({"bits_k_rest": kbits, "outliers_per_head": n_o, "bits_v": vbits, "encode_k_ms": enc_k_ms,
                    "attn_ms": at_ms, "attn_gbs": bytes_ / at_ms / 1e6, "attn_hbm_frac": bytes_ / at_ms / 1e6 / HBM_PEAK_GBS,
                    "kv_positions_per_s": n / at_ms * 1e3})
    elif name == "c4split":
        # Decode attention with split keys on the attention workload (4 x 131072 tokens x 8 KV heads,
        # 32 query heads): keys at 2.5 bits per channel (outlier half 3 bits, rest 2; the 64 channels
        # of largest mean square over the first 4096 tokens), values at 2 bits.
        cfg = wl.CONFIGS["c4"]
        bo, br, vbits = 3, 2, 2
        n = cfg.B * cfg.hkv * cfg.T
        kb = wl.kv_keys(cfg)
        xs = wl.bf16_bits_to_f32(kb[:1, :, :4096]).astype(np.float64)
        outl = np.argsort(-np.mean(xs * xs, axis=(0, 2)), axis=1, kind="stable")[:, :64]
        del xs
        sp = tq.make_split(outl)
        rot_o, rot_r, rot_v = tq.make_rotation(64, 3), tq.make_rotation(64, 4), tq.make_rotation(cfg.d, 1)
        cbo, cbr, cbv = tq.codebook(64, bo), tq.codebook(64, br), tq.codebook(cfg.d, vbits)
        kx = torch.from_numpy(kb.view(np.int16)).to(dev).view(torch.bfloat16)
        del kb
        K = tq.encode_split(kx, sp, cbo, cbr, rot_o, rot_r)
        del kx
        vx = torch.from_numpy(wl.kv_values(cfg).reshape(n, cfg.d).view(np.int16)).to(dev).view(torch.bfloat16)
        V = tq.encode(vx, vbits, "mse", cbv, rot_v, layout="blocked")
        del vx
        q = torch.from_numpy(wl.kv_queries(cfg)).to(dev)
        out = torch.empty((cfg.B, cfg.hq, cfg.d), device=dev)
        ws = torch.empty(tq.decode_attn_split_workspace(cfg.B, cfg.hq, cfg.hkv, cfg.T), dtype=torch.uint8, device=dev)
        at_ms = _timed(lambda i: tq.decode_attn_split(q, K, V, cfg.hkv, sp, cbo, cbr, cbv, rot_o, rot_r, rot_v, out=out,
                                                      ws=ws), steps, warmup)
        bytes_ = n * (8 * (bo + br) + 8) + n * (cfg.d * vbits // 8 + 4) + q.numel() * 4 + out.numel() * 4
        res.update({"bits_outlier": bo, "bits_rest": br, "bits_v": vbits, "attn_ms": at_ms,
                    "attn_gbs": bytes_ / at_ms / 1e6, "attn_hbm_frac": bytes_ / at_ms / 1e6 / HBM_PEAK_GBS,
                    "kv_positions_per_s": n / at_ms * 1e3})
    elif name in ("decode", "decodeb4"):
        # Streaming decode over the long-context cache (batch 4, 8 KV heads, d = 128, GQA 4, K and V
        # MSE at b bits): prefill the cache up to T0 tokens per sequence, then per step append one
        # token's key and value per sequence and attend over the whole prefix.
        cfg = wl.CONFIGS["c4"]
        b = 2 if name == "decode" else 4
        t_cap = cfg.T
        t0 = t_cap - warmup - steps
        rot = tq.make_rotation(cfg.d, 1)
        cb = tq.codebook(cfg.d, b)
        kc = tq.alloc_cache(cfg.B, cfg.hkv, t_cap, cfg.d, b, "mse", device=dev)
        vc = tq.alloc_cache(cfg.B, cfg.hkv, t_cap, cfg.d, b, "mse", layout="blocked", device=dev)
        kx = torch.from_numpy(wl.kv_keys(cfg).view(np.int16)).view(torch.bfloat16)
        vx = torch.from_numpy(wl.kv_values(cfg).view(np.int16)).view(torch.bfloat16)
        knew = kx[:, :, t0:].permute(2, 0, 1, 3).contiguous().to(dev)   # [steps, B, Hkv, d]
        vnew = vx[:, :, t0:].permute(2, 0, 1, 3).contiguous().to(dev)
        kpre = kx[:, :, :t0].contiguous().to(dev)
        vpre = vx[:, :, :t0].contiguous().to(dev)
        del kx, vx
        pre_ms = _timed(lambda i: tq.kv_append(kc, vc, kpre, vpre, 0, cb, cb, rot, rot), 2, 1)
        del kpre, vpre
        q = torch.from_numpy(wl.kv_queries(cfg)).to(dev)
        out = torch.empty((cfg.B, cfg.hq, cfg.d), device=dev)
        ws = torch.empty(tq.decode_attn_workspace(cfg.B, cfg.hq, cfg.hkv, t_cap, cfg.d), dtype=torch.uint8, device=dev)

        def append(i):
            tq.kv_append(kc, vc, knew[i].unsqueeze(2), vnew[i].unsqueeze(2), t0 + i, cb, cb, rot, rot)

        def step(i):
            append(i)
            tq.decode_attn_cache(q, kc, vc, t0 + i + 1, cb, cb, rot, rot, out=out, ws=ws)

        step_ms = _timed(step, steps, warmup)
        # the parts alone: appends rewrite the same positions; attention over the full cache
        app_ms = _timed(append, steps, 0)
        at_ms = _timed(lambda i: tq.decode_attn_cache(q, kc, vc, t_cap, cb, cb, rot, rot, out=out, ws=ws), 20, 2)
        n = cfg.B * cfg.hkv * t_cap
        words = cfg.d * b // 32
        at_bytes = 2 * n * (words * 4 + 4) + q.numel() * 4 + out.numel() * 4
        pre_tokens = 2 * cfg.B * cfg.hkv * t0
        res.update({"bits": b, "cache": [cfg.B, cfg.hkv, t_cap, cfg.d], "prefill_tokens": t0,
                    "prefill_ms": pre_ms, "prefill_kv_vectors_per_s": pre_tokens / pre_ms * 1e3,
                    "step_ms": step_ms, "decode_tokens_per_s": cfg.B / step_ms * 1e3,
                    "append_ms": app_ms, "attn_full_ms": at_ms, "attn_gbs": at_bytes / at_ms / 1e6,
                    "attn_hbm_frac": at_bytes / at_ms / 1e6 / HBM_PEAK_GBS})
        if cpu_budget > 0:
            res["cpu_baseline"] = cpu_baseline_decode(cfg, b, t_cap, cpu_budget)
    elif name in ("c2split", "c2split35", "c3split"):
        # Outlier-channel split codes on the KV-key workload (1 x 8 KV heads x 32768 tokens, 32 query
        # heads): 2.5 bits per channel (outlier half 3 bits, rest 2) or 3.5 (4 and 3); c3split: 2.5
        # bits on the prod workload's keys (16 x 8 KV heads x 16384 tokens).  The 64 outlier channels
        # per head are those of largest mean square over the first 4096 tokens.
        cfg = wl.CONFIGS["c3" if name == "c3split" else "c2"]
        bo, br = (4, 3) if name == "c2split35" else (3, 2)
        n = cfg.B * cfg.hkv * cfg.T
        kb = wl.kv_keys(cfg)
        xs = wl.bf16_bits_to_f32(kb[:1, :, :4096]).astype(np.float64)
        outl = np.argsort(-np.mean(xs * xs, axis=(0, 2)), axis=1, kind="stable")[:, :64]
        del xs
        keys = torch.from_numpy(kb.view(np.int16)).to(dev).view(torch.bfloat16)
        q = torch.from_numpy(wl.kv_queries(cfg)).to(dev)
        sp = tq.make_split(outl)
        rot_o, rot_r = tq.make_rotation(64, 3), tq.make_rotation(64, 4)
        cb_o, cb_r = tq.codebook(64, bo), tq.codebook(64, br)
        nbuf = 3
        packs = [(tq.alloc_packed(n, 64, bo, device=dev), tq.alloc_packed(n, 64, br, device=dev)) for _ in range(nbuf)]
        outs = [torch.empty((cfg.B, cfg.hq, cfg.T), device=dev) for _ in range(nbuf)]
        ws = torch.empty(tq.scores_split_workspace(cfg.B, cfg.hq), dtype=torch.uint8, device=dev)
        enc = lambda i: tq.encode_split(keys, sp, cb_o, cb_r, rot_o, rot_r, out=packs[i % nbuf])
        sco = lambda i: tq.scores_split(q, packs[i % nbuf], cfg.hkv, sp, cb_o, cb_r, rot_o, rot_r, out=outs[i % nbuf],
                                        ws=ws)
        enc_ms = _timed(enc, steps, warmup)
        sc_ms = _timed(sco, steps, warmup)
        step_ms = _timed(lambda i: (enc(i), sco(i)), steps, warmup)
        words = 2 * (bo + br)
        enc_bytes = n * (cfg.d * 2 + 4 * words + 8)
        enc_flop = n * 2 * 2 * 64 * 64
        sc_bytes = n * (4 * words + 8) + q.numel() * 4 + outs[0].numel() * 4
        res.update({"bits_outlier": bo, "bits_rest": br, "bits_per_channel": (bo + br) / 2,
                    "step_ms": step_ms, "scores_per_s_step": outs[0].numel() / step_ms * 1e3,
                    "encode_ms": enc_ms, "encode_gbs": enc_bytes / enc_ms / 1e6,
                    "encode_tflops": enc_flop / enc_ms / 1e9, "encode_hbm_frac": enc_bytes / enc_ms / 1e6 / HBM_PEAK_GBS,
                    "scores_ms": sc_ms, "scores_gbs": sc_bytes / sc_ms / 1e6,
                    "scores_hbm_frac": sc_bytes / sc_ms / 1e6 / HBM_PEAK_GBS,
                    "scores_per_s": outs[0].numel() / sc_ms * 1e3})
        if cpu_budget > 0:
            res["cpu_baseline"] = cpu_baseline_split(cfg, bo, br, cpu_budget)
    elif name == "c2o8":
        # Outlier-8 keys on the KV-key workload (1 x 8 KV heads x 32768 tokens, 32 query heads): per
        # KV head the 8 channels of largest mean square over the first 4096 tokens as int8 with a
        # per-key scale, the other 120 channels TurboQuant_mse at 3 bits (d = 128).
        cfg = wl.CONFIGS["c2"]
        b, n_o = 3, 8
        n = cfg.B * cfg.hkv * cfg.T
        kb = wl.kv_keys(cfg)
        xs = wl.bf16_bits_to_f32(kb[:, :, :4096]).astype(np.float64)
        outl = np.argsort(-np.mean(xs * xs, axis=(0, 2)), axis=1, kind="stable")[:, :n_o]
        del xs
        keys = torch.from_numpy(kb.view(np.int16)).to(dev).view(torch.bfloat16)
        q = torch.from_numpy(wl.kv_queries(cfg)).to(dev)
        o = tq.make_outlier8(outl)
        rot = tq.make_rotation(cfg.d, cfg.rot_seed)
        cb = tq.codebook(cfg.d, b)
        nbuf = 3
        packs = [(tq.alloc_packed(n, cfg.d, b, device=dev), torch.empty((n, n_o), dtype=torch.int8, device=dev),
                  torch.empty((n,), device=dev)) for _ in range(nbuf)]
        outs = [torch.empty((cfg.B, cfg.hq, cfg.T), device=dev) for _ in range(nbuf)]
        ws = torch.empty(tq.scores_outlier8_workspace(cfg.B, cfg.hq), dtype=torch.uint8, device=dev)
        enc = lambda i: tq.encode_outlier8(keys, o, cb, rot, out=packs[i % nbuf])
        sco = lambda i: tq.scores_outlier8(q, packs[i % nbuf], cfg.hkv, o, cb, rot, out=outs[i % nbuf], ws=ws)
        enc_ms = _timed(enc, steps, warmup)
        sc_ms = _timed(sco, steps, warmup)
        step_ms = _timed(lambda i: (enc(i), sco(i)), steps, warmup)
        code = 4 * (cfg.d * b // 32) + 4 + n_o + 4      # rest words, rest norm, int8 values, scale
        enc_bytes = n * (cfg.d * 2 + code)
        sc_bytes = n * code + q.numel() * 4 + outs[0].numel() * 4
        res.update({"bits_rest": b, "outliers_per_head": n_o,
                    "bits_per_channel": (b * (cfg.d - n_o) + 8 * n_o) / cfg.d,
                    "step_ms": step_ms, "scores_per_s_step": outs[0].numel() / step_ms * 1e3,
                    "encode_ms": enc_ms, "encode_gbs": enc_bytes / enc_ms / 1e6,
                    "encode_hbm_frac": enc_bytes / enc_ms / 1e6 / HBM_PEAK_GBS,
                    "scores_ms": sc_ms, "scores_gbs": sc_bytes / sc_ms / 1e6,
                    "scores_hbm_frac": sc_bytes / sc_ms / 1e6 / HBM_PEAK_GBS,
                    "scores_per_s": outs[0].numel() / sc_ms * 1e3})
    elif name == "c2splitdecode":
        # Split keys as a streaming key cache on the KV-key workload (1 x 8 KV heads x 32768 tokens,
        # 32 query heads, 2.5 bits per channel): prefill to T0 tokens in one append, then per step
        # append one key per sequence and score the prefix.
        cfg = wl.CONFIGS["c2"]
        bo, br = 3, 2
        t_cap = cfg.T
        t0 = t_cap - warmup - steps
        kb = wl.kv_keys(cfg)
        xs = wl.bf16_bits_to_f32(kb[:, :, :4096]).astype(np.float64)
        outl = np.argsort(-np.mean(xs * xs, axis=(0, 2)), axis=1, kind="stable")[:, :64]
        del xs
        keys = torch.from_numpy(kb.view(np.int16)).to(dev).view(torch.bfloat16)
        knew = keys[:, :, t0:].permute(2, 0, 1, 3).contiguous()        # [steps, B, Hkv, d]
        kpre = keys[:, :, :t0].contiguous()
        q = torch.from_numpy(wl.kv_queries(cfg)).to(dev)
        sp = tq.make_split(outl)
        rot_o, rot_r = tq.make_rotation(64, 3), tq.make_rotation(64, 4)
        cb_o, cb_r = tq.codebook(64, bo), tq.codebook(64, br)
        K = tq.alloc_split_cache(cfg.B, cfg.hkv, t_cap, bo, br, device=dev)
        out = torch.empty((cfg.B * cfg.hq * t_cap,), device=dev)
        ws = torch.empty(tq.scores_split_workspace(cfg.B, cfg.hq), dtype=torch.uint8, device=dev)
        pre_ms = _timed(lambda i: tq.cache_append_split(K, kpre, 0, t_cap, sp, cb_o, cb_r, rot_o, rot_r), 2, 1)

        def append(i):
            tq.cache_append_split(K, knew[i].unsqueeze(2), t0 + i, t_cap, sp, cb_o, cb_r, rot_o, rot_r)

        def step(i):
            append(i)
            T = t0 + i + 1
            tq.scores_split_cache(q, K, cfg.hkv, T, t_cap, sp, cb_o, cb_r, rot_o, rot_r,
                                  out=out[:cfg.B * cfg.hq * T].view(cfg.B, cfg.hq, T), ws=ws)

        step_ms = _timed(step, steps, warmup)
        app_ms = _timed(append, steps, 0)
        res.update({"bits_outlier": bo, "bits_rest": br, "cache": [cfg.B, cfg.hkv, t_cap, cfg.d], "prefill_tokens": t0,
                    "prefill_ms": pre_ms, "step_ms": step_ms, "append_ms": app_ms,
                    "decode_scores_per_s": cfg.hq * t_cap / step_ms * 1e3})
    elif name in ("prefill", "prefillb4"):
        # Prefill fused with attention: a 16384-token prompt of one sequence (8 KV heads, 32 query
        # heads, d = 128, bf16 K and V) appended to empty compressed caches (MSE, b = 2 or 4) in one
        # chunk, and its causal attention over the packed caches.
        b = 2 if name == "prefill" else 4
        B, hkv, hq, T, d = 1, 8, 32, 16384, 128
        rot = tq.make_rotation(d, 1)
        cb = tq.codebook(d, b)
        kc = tq.alloc_cache(B, hkv, T, d, b, "mse", device=dev)
        vc = tq.alloc_cache(B, hkv, T, d, b, "mse", layout="blocked", device=dev)
        k = torch.from_numpy(wl.kv_tensor_bf16(B, hkv, T, d, seed=0, outlier_seed=10, scale_seed=11).view(np.int16)).to(
            dev).view(torch.bfloat16)
        v = torch.from_numpy(wl.kv_tensor_bf16(B, hkv, T, d, seed=20, outlier_seed=21, scale_seed=None).view(np.int16)).to(
            dev).view(torch.bfloat16)
        q = torch.from_numpy(wl.gaussian((B, hq, T, d), 12)).to(dev)
        out = torch.empty((B, hq, T, d), device=dev)
        ws = torch.empty(tq.prefill_attn_workspace(B, hq, T, d), dtype=torch.uint8, device=dev)
        pf_ms = _timed(lambda i: tq.prefill_attn(q, kc, vc, k, v, 0, cb, cb, rot, rot, out=out, ws=ws), steps, warmup)
        app_ms = _timed(lambda i: tq.kv_append(kc, vc, k, v, 0, cb, cb, rot, rot), steps, warmup)
        pairs = hq * T * (T + 1) / 2                       # visible (query, key) pairs, causal
        alg = 4.0 * d * pairs                              # q.k and p.v per pair
        # issued fp16 MFMA work: per 32-key step and 16 queries, 24 instructions for the scores (Khi Qhi,
        # Klo Qhi, Khi Qlo) and 16 for P V (weights hi and lo), 16 x 16 x 32 x 2 flops each
        steps32 = sum((16 * (t + 1) + 31) // 32 for t in range(T // 16))
        issued = hq * steps32 * 40 * 16384.0
        att_ms = pf_ms - app_ms
        res.update({"bits": b, "prompt": [B, hkv, T, d], "query_heads": hq, "prefill_ms": pf_ms,
                    "prefill_tokens_per_s": B * T / pf_ms * 1e3, "append_ms": app_ms,
                    "attention_ms_est": att_ms, "alg_tflops": alg / att_ms / 1e9,
                    "issued_f16_tflops": issued / att_ms / 1e9, "issued_frac_f16_peak": issued / att_ms / 1e9 / 2500.0})
    elif name == "peaks":
        # Achievable ceilings on this machine, from the library's own measurement kernels: a streaming
        # read and a streaming copy of 1 GiB (far larger than the last-level cache), swept over
        # grid sizes; and independent MFMA chains of each operand type, swept over waves per SIMD.
        nbytes = 1 << 30
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        reads, copies = {}, {}
        for per_cu in (2, 4, 8, 16):
            blocks = cus * per_cu
            reads[per_cu] = _timed(lambda i: tq.peak_read(src, blocks), steps, warmup)
            copies[per_cu] = _timed(lambda i: tq.peak_copy(dst, src, blocks), steps, warmup)
        br = min(reads, key=reads.get)
        bc = min(copies, key=copies.get)
        res.update({"bytes": nbytes, "cus": cus,
                    "read_gbs_by_blocks_per_cu": {k: nbytes / v / 1e6 for k, v in reads.items()},
                    "copy_gbs_by_blocks_per_cu": {k: 2 * nbytes / v / 1e6 for k, v in copies.items()},
                    "read_gbs": nbytes / reads[br] / 1e6, "read_frac": nbytes / reads[br] / 1e6 / HBM_PEAK_GBS,
                    "copy_gbs": 2 * nbytes / copies[bc] / 1e6,
                    "copy_frac": 2 * nbytes / copies[bc] / 1e6 / HBM_PEAK_GBS})
        del src, dst
        mf = {}
        for kind in tq.PEAK_MFMA_KINDS:
            best = 0.0
            for per_simd in (1, 2, 4):
                blocks = cus * per_simd          # 4 waves per block: per_simd waves on each SIMD
                out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
                flops = [0.0]

                def run(i):
                    flops[0] = tq.peak_mfma(kind, 2000, blocks, out)
                ms = _timed(run, max(3, steps // 10), 1)
                best = max(best, flops[0] / ms / 1e9)
            mf[kind] = {"tflops": best, "frac_of_2500": best / 2500.0}
        res["mfma"] = mf
    elif name == "c5":
        cfg = wl.CONFIGS["c5"]
        n, d = cfg.n, cfg.d
        nq, k = cfg.extra["queries"], cfg.extra["k"]
        x = torch.empty((n, d), dtype=torch.float32, device=dev)
        for lo, xc in wl.index_vectors(cfg):
            x[lo:lo + xc.shape[0]].copy_(torch.from_numpy(xc))
        q = torch.from_numpy(wl.index_queries(cfg)).to(dev)
        rot = tq.make_rotation(d, cfg.rot_seed, "dense")
        qjl = tq.make_qjl(d, cfg.qjl_seed, rot)
        cb = tq.codebook(d, cfg.bits - 1)
        p = tq.alloc_packed(n, d, cfg.bits - 1, "prod", device=dev)
        ews = torch.empty((tq.encode_workspace(n, d, cfg.bits, "prod"),), dtype=torch.uint8, device=dev)
        enc_ms = _timed(lambda i: tq.encode(x, cfg.bits, "prod", cb, rot, qjl, out=p, ws=ews), steps, warmup)
        del x
        sws = torch.empty((tq.search_workspace(nq, n, d, k),), dtype=torch.uint8, device=dev)
        outs = (torch.empty((nq, k), device=dev), torch.empty((nq, k), dtype=torch.int64, device=dev))
        se_ms = _timed(lambda i: tq.search_topk(q, p, k, cb, rot, qjl, ws=sws, out=outs), steps, warmup)
        enc_flops = 4.0 * n * d * d            # R x and S' r, fp32-accurate (three bf16 passes each)
        search_flops = 4.0 * nq * n * d        # <q_rot, c> and <q_s, z> per pair, fp16 operands
        res.update({"encode_ms": enc_ms, "encode_vectors_per_s": n / enc_ms * 1e3,
                    "encode_tflops_fp32_accurate": enc_flops / enc_ms / 1e9,
                    "encode_bf16_passes_issued": 3,
                    "encode_frac_bf16_issued": 3 * enc_flops / enc_ms / 1e9 / 2500.0,
                    "search_ms": se_ms, "search_scores_per_s": nq * n / se_ms * 1e3,
                    "search_tflops": search_flops / se_ms / 1e9,
                    "search_frac_fp16_mfma": search_flops / se_ms / 1e9 / 2500.0})
    print(json.dumps(res), flush=True)


def step_bench(name, steps, warmup, copy_probe_after=False, cpu_budget=0.0, event_every=4):
    """One step = encode every key of the workload, then the query prologue and the scores of every
    query head over the packed keys.  c3: TurboQuant_prod b = 4 (3-bit Lloyd-Max + 1-bit QJL) of
    16 x 8 x 16384 bf16 keys, dense R; c2: TurboQuant_mse b = 3 of 1 x 8 x 32768 bf16 keys.
    Returns the result dict (the bench line's fields)."""
    import torch
    import kv_cache_compression_turboquant_amd as tq
    from kv_cache_compression_turboquant_amd import workloads as wl
    dev = torch.device("cuda:0")
    cfg = wl.CONFIGS[name]
    prod = cfg.mode == "prod"
    stage = cfg.bits - 1 if prod else cfg.bits
    n = cfg.B * cfg.hkv * cfg.T
    keys_bits = wl.kv_keys(cfg)
    q_np = wl.kv_queries(cfg)

    cb = tq.codebook(cfg.d, stage)
    rot = tq.make_rotation(cfg.d, cfg.rot_seed, "dense")
    qjl = tq.make_qjl(cfg.d, cfg.qjl_seed, rot) if prod else None
    words = cfg.d * stage // 32
    in_bytes = n * cfg.d * 2
    row_bytes = words * 4 + 4 + ((cfg.d // 8 + 4) if prod else 0)   # indices + norm (+ signs + gamma)
    out_bytes = n * row_bytes
    score_bytes_out = cfg.B * cfg.hq * cfg.T * 4
    per_set = in_bytes + out_bytes + score_bytes_out
    nbuf = max(2, int(np.ceil(CACHE_DEFEAT_BYTES / per_set)))
    base = torch.from_numpy(keys_bits.reshape(n, cfg.d).view(np.int16)).to(dev).view(torch.bfloat16)
    del keys_bits
    xs = [base] + [base.clone() for _ in range(nbuf - 1)]
    packs = [tq.alloc_packed(n, cfg.d, stage, cfg.mode, device=dev) for _ in range(nbuf)]
    q = torch.from_numpy(q_np).to(dev)
    outs = [torch.empty((cfg.B, cfg.hq, cfg.T), dtype=torch.float32, device=dev) for _ in range(nbuf)]
    ws = torch.empty(tq.scores_workspace(cfg.B, cfg.hq, cfg.d), dtype=torch.uint8, device=dev)

    def step(i, timers=None):
        j = i % nbuf
        if timers is not None:
            timers[0].append(tq.timer_arm("encode"))
            timers[1].append(tq.timer_arm("scores"))
        tq.encode(xs[j], cfg.bits, cfg.mode, cb, rot, qjl, out=packs[j])
        tq.scores(q, packs[j], cfg.hkv, cb, rot, qjl, out=outs[j], ws=ws)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region: exactly `steps` steps.  The encode and score kernels' durations are taken live,
    # on every event_every-th step, with HIP events that the library attaches to those kernels'
    # dispatches (hipExtLaunchKernel): they bracket each kernel alone, on the stream it runs on.
    timers = ([], [])
    tq.timer_reset()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(warmup + i, timers if i % event_every == 0 else None)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_s = (t1 - t0) / steps
    enc_ms = float(np.mean([tq.timer_read(t) for t in timers[0]]))
    sc_ms = float(np.mean([tq.timer_read(t) for t in timers[1]]))
    tq.timer_reset()

    scores_per_step = cfg.B * cfg.hq * cfg.T
    enc_alg_bytes = in_bytes + out_bytes
    score_alg_bytes = out_bytes + cfg.B * cfg.hq * cfg.d * 4 + score_bytes_out
    enc_gbs = enc_alg_bytes / (enc_ms * 1e-3) / 1e9
    sc_gbs = score_alg_bytes / (sc_ms * 1e-3) / 1e9
    # bf16 MFMA passes the encode issues per d x d product: R as hi + lo (x is exact in bf16);
    # S' r as S'hi rhi + S'hi rlo + S'lo rhi
    passes = 2 + (3 if prod else 0)
    issued_flops = passes * 2.0 * cfg.d * cfg.d * n
    enc_kernel, sc_kernel = HEADLINE_KERNELS[name]
    res = {
        "workload": cfg.workload, "keys": [cfg.B, cfg.hkv, cfg.T, cfg.d], "bits": cfg.bits,
        "mode": cfg.mode, "query_heads": cfg.hq, "rotation": "dense QR (seed 1)" + (", S seed 2" if prod else ""),
        "ms_per_step": step_s * 1e3, "scores_per_s": scores_per_step / step_s,
        "encode_vectors_per_s": n / step_s, "encode_kernel_ms": enc_ms, "score_kernel_ms": sc_ms,
        "buffer_sets": nbuf,
        "roofline": {"bound": "hbm", "kernel": enc_kernel,
                     "timing": f"HIP events attached to the kernel's dispatch on every {event_every}th timed step",
                     "achieved": enc_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": enc_gbs / HBM_PEAK_GBS,
                     "traffic": traffic_from_profile(name + (":prod_encode" if prod else ":encode")),
                     "alg_bytes_per_launch": enc_alg_bytes,
                     "mfma_issued": {"passes": passes, "tflops": issued_flops / (enc_ms * 1e-3) / 1e12,
                                     "peak": 2500.0, "frac": issued_flops / (enc_ms * 1e-3) / 1e12 / 2500.0}},
        "roofline_score": {"bound": "hbm", "kernel": sc_kernel,
                           "timing": f"HIP events attached to the kernel's dispatch on every {event_every}th timed step",
                           "achieved": sc_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": sc_gbs / HBM_PEAK_GBS,
                           "traffic": traffic_from_profile(name + ":scores"),
                           "alg_bytes_per_launch": score_alg_bytes},
    }
    if copy_probe_after:
        copy_probe(torch, dev)
    if cpu_budget > 0:
        if prod:
            res["cpu_baseline"] = cpu_baseline_prod(cfg, "dense", cpu_budget)
        else:
            res["cpu_baseline"] = cpu_baseline(cfg, wl.kv_keys(cfg), q_np, cpu_budget)
    del xs, packs, outs, base
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true", help="skip the nested KV-key (c2) step line")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--config", default="c3", choices=["c3", "c2", "c3wht", "c3bwht", "c3mse", "c3msewht", "c3msebwht", "hd64", "hd256", "c4b2", "c4b4", "c5", "decode",
                                                        "decodeb4", "peaks", "c2split", "c2split35", "c3split", "c2splitdecode", "c2o8", "c4o8", "c4split",
                                                        "prefill", "prefillb4"],
                    help="c3 = the headline step (c2 is its nested secondary line); the others print "
                         "per-kernel timings only")
    ap.add_argument("--copy-probe", action="store_true",
                    help="after the timed steps, run plain device copies of COPY_PROBE_BYTES "
                         "(the calibration for the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--trace-summary", metavar="DB",
                    help="print the per-kernel table of a rocprofv3 --kernel-trace database; no GPU needed")
    ap.add_argument("--pmc-table", metavar="DB",
                    help="print the per-kernel means of every counter in a rocprofv3 --pmc database; no GPU needed")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                    help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) made with "
                         "--copy-probe into profiles/traffic.json and print the table; no GPU needed")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary)
        return
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.pmc_table:
        pmc_table(args.pmc_table)
        return
    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} is not supported "
              "(the multi-GPU sharding is described in the design notes, not built)", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no HIP device", file=sys.stderr)
        sys.exit(1)
    cpu_budget = 0.0 if args.no_cpu_baseline else args.cpu_budget
    if args.config not in ("c3", "c2"):
        bench_other(args.config, args.steps, args.warmup, cpu_budget)
        return
    print(f"bench.py: {args.config} step, {args.warmup} warmup + {args.steps} timed steps", file=sys.stderr, flush=True)
    main_res = step_bench(args.config, args.steps, args.warmup, args.copy_probe, cpu_budget)
    secondary = None
    if args.config == "c3" and not args.no_secondary:
        print("bench.py: secondary c2 step", file=sys.stderr, flush=True)
        secondary = step_bench("c2", max(20, args.steps // 2), min(args.warmup, 5), False, 0.0)
    r = main_res
    result = {
        "metric": "Q·K^T scores/s over packed keys + encode vectors/s; % of HBM roofline",
        "value": r["scores_per_s"],
        "unit": "scores/s (each step encodes all keys, then scores every query head)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {k: r[k] for k in ("workload", "keys", "bits", "mode", "query_heads", "rotation",
                                     "encode_vectors_per_s", "encode_kernel_ms", "score_kernel_ms", "buffer_sets")},
        "roofline": r["roofline"],
        "roofline_score": r["roofline_score"],
    }
    if secondary is not None:
        result["secondary"] = {"kv_keys_c2": {k: secondary[k] for k in (
            "workload", "ms_per_step", "scores_per_s", "encode_vectors_per_s", "encode_kernel_ms",
            "score_kernel_ms")}}
        result["secondary"]["kv_keys_c2"]["encode_frac_hbm"] = secondary["roofline"]["frac"]
        result["secondary"]["kv_keys_c2"]["score_frac_hbm"] = secondary["roofline_score"]["frac"]
    if "cpu_baseline" in r:
        result["cpu_baseline"] = r["cpu_baseline"]
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
