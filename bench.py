"""Benchmark of the dasc checkpoint hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
pack n checkpoints into pool slots, unpack them with zero-fill, and refresh
n_req requests over their suffix windows with the decays given directly
(Eq. 1 as written).  The static plan is built once, before timing, as the
pages build it offline; its host time is reported.

Headline workload, the largest configuration: "mixed", 27 layers
alternating GDN and KDA (32 heads, d = 128, per-layer retention 20-80%,
W_max = 64), 512 checkpoints in a random slot order, 64 requests with
suffixes of U{64..1024} tokens.  The same JSON line carries two
sub-objects with the same measurements: "gdn" (36 GDN layers x 32 heads,
64 checkpoints, 64 x 256 tokens over the omitted heads) and "kda" (20 KDA
layers x 32 heads with conv state, 64 checkpoints, 64 x 256 tokens).
`--workload mixed|gdn|kda` runs one of them alone (the profiling runs).

Prints ONE JSON line.  value = pack+unpack GB/s of the headline workload
(algorithmic bytes / time); its refresh request-tokens/s and every
kernel's roofline ride along.  Timed after the steps, on their own: INT8
checkpoint pack and unpack (Eq. 10), the refresh from bf16 gate logits
(the fused gate, Eq. 2 in the kernel), per-head Eq. 7 windows for both,
the dasc-wr load (unpack then refresh against the fused load), TP8
storage balancing (gdn, kda) and the token-by-token vector form of the
refresh (kda).  A cpu_baseline times the fp64 oracle on a bounded sample
of the headline workload: pack and unpack in one process, the refresh
over a pool of one worker per host core.
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

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP32_MFMA_PEAK_TF = 157.3      # MI355X dense fp32 matrix (MFMA), TFLOP/s
FP32_VALU_UNPACKED_TF = 78.6   # fp32 vector FMA rate without packed (2-wide) FMA, TFLOP/s

# Kernel sources whose hash a traffic summary under profiles/ records: the
# counters it holds describe these exact kernels and piece lists.
KERNEL_SOURCES = ["recurrent_state_cache_amd/csrc/dasc_kernels.hip",
                  "recurrent_state_cache_amd/csrc/dasc_internal.h",
                  "recurrent_state_cache_amd/csrc/dasc_host.cpp"]
# rounds of the rocprofv3 kernel-statistics run (--warmup, --steps)
PROFILE_WARMUP, PROFILE_STEPS = 3, 10

# kernel name pattern -> role.  refresh_kernel<D, gate mode, windowed, fused,
# one chunk>: gate modes 0-2 read bf16 gate logits, 3-5 fp32 decays.
KERNEL_ROLES = {r"qmove_kernel<true(, (true|false))?>": "pack_int8",
                r"qmove_kernel<false(, false)?>": "unpack_int8",
                r"(?<!q)move_kernel<true, \d+, \d+, false>": "pack",
                r"(?<!q)move_kernel<false, \d+, \d+, false>": "unpack",
                r"(?<!q)move_kernel<true, \d+, \d+, true>": "pack_tp",
                r"(?<!q)move_kernel<false, \d+, \d+, true>": "unpack_tp",
                r"refresh_kernel<\d+, [345], false, false, false>": "refresh",
                r"refresh_kernel<\d+, [012], false, false, false>": "refresh_gate",
                r"refresh_kernel<\d+, [345], true, false, (true|false)>": "refresh_windowed",
                r"refresh_kernel<\d+, [012], true, false, (true|false)>": "refresh_windowed_gate",
                r"refresh_kernel<\d+, \d+, (true|false), true, (true|false)>": "refresh_fused",
                r"recurrent_kernel<": "refresh_recurrent"}
ROLE_ORDER = ("pack", "unpack", "refresh", "refresh_gate", "pack_int8", "unpack_int8", "pack_tp",
              "unpack_tp", "refresh_windowed", "refresh_windowed_gate", "refresh_fused",
              "refresh_recurrent")
WORKLOADS = ("mixed", "gdn", "kda")


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300,
                    help="timed steps of every workload's pack + unpack + refresh")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--side-steps", type=int, default=20,
                    help="timed rounds of each section after the steps (INT8, windows, ...)")
    ap.add_argument("--workload", choices=("all",) + WORKLOADS, default="all",
                    help="all: the mixed headline with gdn and kda sub-objects")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--skip-wr-load", action="store_true",
                    help="skip the dasc-wr load section (its unpack launches would share the "
                         "unpack kernel's name in a profile)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--summarize", nargs=5, metavar=("STATS", "FETCH", "WRITE", "FETCH_COPY",
                                                     "WRITE_COPY"),
                    help="print a markdown summary of rocprofv3 csv output directories "
                         "(kernel stats; FETCH_SIZE and WRITE_SIZE of this bench and of "
                         "--calibrate-copy) and exit")
    ap.add_argument("--counters", nargs="+", metavar="DIR",
                    help="print the mean per-dispatch value of every counter in these "
                         "rocprofv3 csv output directories, per kernel of the library, and exit")
    return ap.parse_args()


def _workload(name):
    import workloads as W
    if name == "kda":
        cfg = W.kda(n_ckpt=64, n_req=64, window=256)
        desc = "KDA 20x32 heads d=128: pack+unpack 64 ckpts, refresh 64 req x 256 tok"
    elif name == "gdn":
        cfg = W.gdn(n_ckpt=64)
        cfg.n_req, cfg.window = 64, (256, 256)
        desc = "GDN 36x32 heads d=128: pack+unpack 64 ckpts, refresh 64 req x 256 tok"
    else:
        cfg = W.mixed(n_ckpt=512, n_req=64)
        desc = ("mixed 27 layers GDN/KDA 32 heads d=128: pack+unpack 512 ckpts, "
                "refresh 64 req x U{64..1024} tok")
    return cfg, desc


def _algorithmic_bytes(P):
    """Bytes pack and unpack must move, from the plan: pack reads each GDN
    retained head in full and, of a KDA head, every 32-channel column block
    (d = 128; the whole head for other widths) with a retained channel (a
    strided column forces whole 128-byte row segments), writes the ragged
    payload, and copies the conv bytes; unpack reads the payload and the conv
    bytes and writes the whole dense checkpoint.  INT8 pack reads the same
    (a column's scale spans the rows of its block, and a d = 128 head's
    block without a retained channel is not read) and writes the int8
    payload, the scales and the conv bytes."""
    info = P.info()
    read_pack = read_pack_q = 0
    for l in range(info["n_layers"]):
        L = P.layer(l)
        ret = P.units(l)[0]
        if L["kind"] == 0:
            read_pack += int(ret.sum()) * L["unit_bytes"]
            read_pack_q += int(ret.sum()) * L["unit_bytes"]
        else:
            per_head = ret.reshape(L["n_heads"], L["d_k"]).any(axis=1)
            if L["d_k"] == 128 and L["d_v"] == 128:
                # both packs read the 32-channel column blocks with a retained channel
                per_block = ret.reshape(L["n_heads"], 4, 32).any(axis=2)
                read_pack += int(per_block.sum()) * L["d_v"] * 32 * 4
                read_pack_q += int(per_block.sum()) * L["d_v"] * 32 * 4
            else:
                read_pack += int(per_head.sum()) * L["d_v"] * L["d_k"] * 4
                read_pack_q += int(per_head.sum()) * L["d_v"] * L["d_k"] * 4
    pack = read_pack + info["temporal_rag_bytes"] + 2 * info["conv_bytes"]
    unpack = info["temporal_rag_bytes"] + info["temporal_dense_bytes"] + 2 * info["conv_bytes"]
    q = info["int8_payload_bytes"] + info["int8_scale_bytes"]
    pack_q = read_pack_q + q + 2 * info["conv_bytes"]
    unpack_q = q + info["temporal_dense_bytes"] + 2 * info["conv_bytes"]
    return pack, unpack, pack_q, unpack_q


BF16_MFMA_PEAK_TF = 2500.0  # MI355X dense bf16 matrix peak


def _refresh_mfma_flops(P, Wn):
    """Matrix flops the refresh kernel issues (not algorithmic): per replayed
    head of width d and 16-token chunk, with d >= 64 the readout S Q as three
    bf16 products (hi hi, hi lo, lo hi) of 16 x d x d, the update W C as two
    16x16x32 bf16 products per 16 x 16 state tile, and C = T R as fp32
    16x16x4 products; with d <= 32 all three on fp32 MFMA.  Returns (bf16,
    fp32) flops for one launch."""
    import numpy as np
    chunks = int(np.sum((np.asarray(Wn) + 15) // 16))
    bf16 = f32 = 0
    for l in range(P.info()["n_layers"]):
        L = P.layer(l)
        d, h = L["d_k"], L["n_refresh_heads"]
        tiles = (d // 16) ** 2
        if d >= 64:
            per = 3 * (d // 32) * (d // 16) * 16384 + 2 * tiles * 16384
            bf16 += h * chunks * per
            f32 += h * chunks * (d // 16) * 4 * 2048
        else:
            f32 += h * chunks * (2 * tiles * 4 + (d // 16) * 4) * 2048
    return bf16, f32


def _windowed_work(P, Wn):
    """(flops, head-token replays) of the refresh with per-head Eq. 7
    windows: head (l, h) replays min(W_lh, n_r) tokens of request r, W_lh
    being the largest window over the head's local units."""
    import numpy as np
    flops = head_tokens = 0
    for l in range(P.info()["n_layers"]):
        L = P.layer(l)
        ret, _, win = P.units(l)
        per = 1 if L["kind"] == 0 else L["d_k"]
        local = ~ret.reshape(L["n_heads"], per).astype(bool)
        w = np.where(local, win.reshape(L["n_heads"], per), 0).max(axis=1)[local.any(axis=1)]
        ht = int(np.minimum(w[:, None], np.asarray(Wn)[None, :]).sum())
        head_tokens += ht
        flops += 5 * L["d_v"] * L["d_k"] * ht
    return flops, head_tokens


def _windowed_bytes(P, Wn, decay_bytes=2):
    """Algorithmic HBM bytes of the refresh with per-head Eq. 7 windows: the
    token inputs each replayed head reads for min(W_lh, n_r) tokens (k and
    v bf16, the decays as bf16 gate logits (decay_bytes = 2) or fp32
    (decay_bytes = 4), beta fp32), and the write-back of the local columns,
    counted by the whole 32-channel row segments (128-byte lines at d_k =
    128) that hold a local channel: a column is strided in the row-major
    state, and a line it touches is written whole.  Every request writes
    every replayed head."""
    import numpy as np
    total = 0
    for l in range(P.info()["n_layers"]):
        L = P.layer(l)
        ret, _, win = P.units(l)
        kda = L["kind"] != 0
        dk, dv = L["d_k"], L["d_v"]
        per = dk if kda else 1
        local = ~ret.reshape(L["n_heads"], per).astype(bool)
        heads = local.any(axis=1)
        w = np.where(local, win.reshape(L["n_heads"], per), 0).max(axis=1)[heads]
        ht = int(np.minimum(w[:, None], np.asarray(Wn)[None, :]).sum())
        per_token = 2 * dk + 2 * dv + (dk if kda else 1) * decay_bytes + 4
        nseg = (dk + 31) // 32
        seg_w = np.minimum(32, dk - 32 * np.arange(nseg))       # channels per segment
        if kda:
            lc = np.zeros((int(heads.sum()), nseg * 32), bool)
            lc[:, :dk] = local[heads]
            cols = int((lc.reshape(-1, nseg, 32).any(axis=2) * seg_w).sum())
        else:
            cols = int(heads.sum()) * dk
        total += ht * per_token + cols * dv * 4 * len(Wn)
    return total


def _windowed_sector_reads(P, Wn):
    """HBM bytes the windowed refresh's write-back must also read: a store
    that covers part of a 32-byte sector (8 fp32 channels of a row) costs
    the memory a read of the sector, so every sector of a replayed head
    that holds both local and retained channels is read once per row and
    request (all-local heads, such as GDN heads, have none)."""
    import numpy as np
    total = 0
    for l in range(P.info()["n_layers"]):
        L = P.layer(l)
        if L["kind"] == 0:
            continue
        ret, _, _ = P.units(l)
        dk, dv = L["d_k"], L["d_v"]
        local = ~ret.reshape(L["n_heads"], dk).astype(bool)
        heads = local.any(axis=1)
        nsec = (dk + 7) // 8
        lc = np.zeros((int(heads.sum()), nsec * 8), bool)
        rc = np.zeros_like(lc)
        lc[:, :dk] = local[heads]
        rc[:, :dk] = ~local[heads]
        mixed = int((lc.reshape(-1, nsec, 8).any(axis=2) & rc.reshape(-1, nsec, 8).any(axis=2)).sum())
        total += mixed * 32 * dv * len(Wn)
    return total


def _calibrate_copy(steps):
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(steps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_per_dispatch_read": n,
                      "bytes_per_dispatch_write": n, "dispatches": steps}), flush=True)


# ---------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on a bounded sample of the workload.
# ---------------------------------------------------------------------------

def _cpu_worker_init():
    os.environ["OMP_NUM_THREADS"] = "1"
    os.environ["OPENBLAS_NUM_THREADS"] = "1"
    os.environ["MKL_NUM_THREADS"] = "1"


def _cpu_warm(i):
    time.sleep(0.25)   # long enough that every worker takes one
    return os.getpid()


def _cpu_refresh_task(task):
    """One request's refresh over a few layers with the oracle, in a worker:
    the layers' own plan (a unit's retention depends on its own parameters
    only, so their heads are the ones the full plan replays) and their
    slices of the token rows.  Returns (head-token replays, flops, seconds)."""
    from threadpoolctl import threadpool_limits
    import numpy as np
    import oracle
    layers, a_s, eps, w_max, k, v, alpha, beta, head_windows = task
    with threadpool_limits(limits=1):
        t = time.perf_counter()
        O = oracle.build_plan(layers, a_s, eps, w_max)
        n = k.shape[0]
        out = oracle.refresh_expected(O, k, v, None, beta, np.array([0, n]), alpha=alpha,
                                      head_windows=head_windows)
        secs = time.perf_counter() - t
    ht = flops = 0
    for (_, li, h) in out:
        L = O.layers[li]
        w = min(O.head_window(li, h), n) if head_windows else n
        ht += w
        flops += 5 * L.d_v * L.d_k * w
    return ht, flops, secs, os.getpid()


def _cpu_pool():
    """One worker process per host core, started before the GPU is touched
    (spawned interpreters that import nothing of the GPU path)."""
    import multiprocessing
    from concurrent.futures import ProcessPoolExecutor
    n = os.cpu_count() or 1
    ex = ProcessPoolExecutor(max_workers=n, mp_context=multiprocessing.get_context("spawn"),
                             initializer=_cpu_worker_init)
    list(ex.map(_cpu_warm, range(n)))   # every submission spawns a worker until n exist
    return ex, n


def _cpu_baseline(cfg, P, ex, n_workers, dense_cpu, pack_bytes_per_ckpt, unpack_bytes_per_ckpt,
                  rows, Wn, int8_bytes_per_ckpt):
    """The fp64 NumPy oracle on a bounded sample of the workload, on this
    host's cores: pack and unpack of a few checkpoints in one process
    (memory-bound, single-threaded); the refresh with the decays given
    directly, one task per (request, pair of layers), over the pool of
    n_workers processes (one per core); the same with per-head Eq. 7
    windows; INT8 pack and unpack of a few checkpoints in one process."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    with threadpool_limits(limits=1):
        O = oracle.build_plan(cfg.layers, cfg.a_s, cfg.eps, cfg.w_max)
        n = dense_cpu.shape[0]
        pool = np.zeros((n, O.slot_bytes), np.uint8)
        out = np.zeros((n, O.dense_bytes), np.uint8)
        t = time.perf_counter()
        oracle.pack(O, dense_cpu, list(range(n)), pool, list(range(n)))
        oracle.unpack_zero_fill(O, pool, list(range(n)), out, list(range(n)))
        t_move = time.perf_counter() - t
        m = min(4, n)
        lo = oracle.Int8Layout(O)
        pool_q = np.zeros((m, lo.slot_bytes), np.uint8)
        out_q = np.zeros((m, O.dense_bytes), np.uint8)
        t = time.perf_counter()
        oracle.pack_int8(O, dense_cpu[:m], list(range(m)), pool_q, list(range(m)))
        oracle.unpack_int8_zero_fill(O, pool_q, list(range(m)), out_q, list(range(m)))
        t_q = time.perf_counter() - t

    # refresh tasks: request r_i = i mod n_req over layers (2j, 2j + 1), j = i mod
    # (L / 2), so the sample covers every layer and many window lengths
    k_all, v_all, alpha_all, beta_all, tok = rows
    ko = vo = go = bo = 0
    offs = []
    for L in cfg.layers:
        offs.append((ko, vo, go, bo))
        ko += L.n_heads * L.d_k
        vo += L.n_heads * L.d_v
        go += L.gate_width
        bo += L.n_heads
    pairs = [(2 * j, 2 * j + 1) for j in range(len(cfg.layers) // 2)] or [(0,)]
    n_tasks = 4 * n_workers

    def task(i, head_windows):
        r = i % cfg.n_req
        ls = pairs[i % len(pairs)]
        t0, t1 = int(tok[r]), int(tok[r + 1])
        sl = lambda a, o, w: np.concatenate([a[t0:t1, offs[l][o]:offs[l][o] + w(cfg.layers[l])]
                                             for l in ls], axis=1)
        return ([cfg.layers[l] for l in ls], cfg.a_s, cfg.eps, cfg.w_max,
                sl(k_all, 0, lambda L: L.n_heads * L.d_k), sl(v_all, 1, lambda L: L.n_heads * L.d_v),
                sl(alpha_all, 2, lambda L: L.gate_width), sl(beta_all, 3, lambda L: L.n_heads),
                head_windows)

    def run(head_windows):
        tasks = [task(i, head_windows) for i in range(n_tasks)]
        t = time.perf_counter()
        res = list(ex.map(_cpu_refresh_task, tasks))
        wall = time.perf_counter() - t
        return (sum(r[0] for r in res), sum(r[1] for r in res), wall, len(tasks),
                len({r[3] for r in res}))

    ht, fl, t_ref, nt, used = run(False)
    ht_w, fl_w, t_win, _, _ = run(True)
    heads_all = sum(len(O.refreshed_heads(l)) for l in range(len(O.layers)))
    gbs = n * (pack_bytes_per_ckpt + unpack_bytes_per_ckpt) / t_move / 1e9
    return {
        "value": round(gbs, 4), "unit": "GB/s pack+unpack",
        "cores": used, "kind": "oracle", "blas_threads_per_worker": 1,
        "refresh_request_tokens_per_s": round(ht / t_ref / heads_all, 3),
        "refresh_gflops": round(fl / t_ref / 1e9, 3),
        "refresh_eq7_windows_head_tokens_per_s": round(ht_w / t_win, 1),
        "int8_pack_unpack_gbs": round(m * int8_bytes_per_ckpt / t_q / 1e9, 4),
        "sample": (f"pack+unpack of {n} checkpoints in one process ({t_move:.2f} s); refresh "
                   f"with the decays given: {nt} tasks (request i mod {cfg.n_req}, a pair of "
                   f"layers) over {n_workers} worker processes ({used} of them took tasks), "
                   f"one thread each, {ht} head-token replays "
                   f"({t_ref:.2f} s wall), converted to request-tokens at {heads_all} replayed "
                   f"heads per token; the same with per-head Eq. 7 windows ({ht_w} head-token "
                   f"replays, {t_win:.2f} s); INT8 pack+unpack of {m} checkpoints in one "
                   f"process ({t_q:.2f} s)"),
        "host_cpus": os.cpu_count(),
    }


def _bench_tp(cfg, args, stream):
    """Store and load with TP storage balancing at TP = 8, all eight ranks'
    shares on this GPU (one launch per rank and direction): pack / partition
    of the checkpoints into slot and send rows, and the gather / zero-fill
    unpack from slot and receive rows.  The exchange between ranks is not
    timed (one GPU); its volume is reported."""
    import numpy as np
    import torch
    import recurrent_state_cache_amd as R
    import workloads as W
    tp, n = 8, cfg.n_ckpt
    plans = [R.Plan(cfg.layers, cfg.a_s, cfg.eps, cfg.w_max, tp=tp, rank=r).upload()
             for r in range(tp)]
    infos = [p.tp_info() for p in plans]
    g = torch.Generator(device="cuda")
    g.manual_seed(cfg.seed + 101)
    dense = [torch.randint(0, 256, (n, p.info()["dense_bytes"]), generator=g, dtype=torch.uint8,
                           device="cuda") for p in plans]
    pools = [torch.empty((n, i["slot_bytes"]), dtype=torch.uint8, device="cuda") for i in infos]
    rows = [torch.empty((n, max(16, i["send_bytes"])), dtype=torch.uint8, device="cuda")
            for i in infos]
    out = [torch.empty_like(d) for d in dense]
    idx = torch.arange(n, dtype=torch.int32, device="cuda")
    rounds, warm = max(1, min(args.steps, args.side_steps)), args.warmup
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(rounds)]
    for i in range(warm + rounds):
        e = ev[i - warm] if i >= warm else None
        if e: e[0].record(stream)
        for r, p in enumerate(plans):
            R.ckpt_pack_tp(p, dense[r], idx, pools[r], idx, rows[r], idx, stream)
        if e: e[1].record(stream)
        for r, p in enumerate(plans):
            R.ckpt_unpack_tp_zero_fill(p, pools[r], idx, rows[r], idx, out[r], idx, stream)
        if e: e[2].record(stream)
    torch.cuda.synchronize()
    assert all(p.status() == 0 for p in plans)
    t_pack = np.median([e[0].elapsed_time(e[1]) for e in ev]) * 1e-3
    t_unpack = np.median([e[1].elapsed_time(e[2]) for e in ev]) * 1e-3
    moved = 0
    for p in plans:
        pk, upk, _, _ = _algorithmic_bytes(p)
        moved += n * (pk + upk)
    ub, conv = infos[0]["unit_bytes"], plans[0].info()["conv_bytes"]
    slot_off = infos[0]["max_local"] * ub + conv      # worst rank's slot without balancing
    slot_on = infos[0]["slot_units"] * ub + conv
    return {
        "tp": tp,
        "n_local": [i["n_local"] for i in infos],
        "slot_units": infos[0]["slot_units"],
        "m_remote_units": infos[0]["m_remote"],
        "exchange_bytes_per_checkpoint": infos[0]["m_remote"] * ub,
        "worst_rank_slot_bytes_off": slot_off,
        "worst_rank_slot_bytes_balanced": slot_on,
        "slot_capacity_gain": round(slot_off / slot_on, 4),
        "pack_tp_ms": round(t_pack * 1e3, 4),
        "unpack_tp_ms": round(t_unpack * 1e3, 4),
        "pack_unpack_gbs": round(moved / (t_pack + t_unpack) / 1e9, 2),
        "frac_of_hbm_peak": round(moved / (t_pack + t_unpack) / 1e9 / HBM_PEAK_GBS, 4),
        "kernel": (f"move_kernel<*, kAlt> ({sum(p.launches('pack_tp', n)[0] for p in plans)} "
                   f"pack and {sum(p.launches('unpack_tp', n)[0] for p in plans)} unpack "
                   f"launches over the {len(plans)} ranks)"),
        "rank0_pack_unpack_bytes_per_checkpoint": int(sum(_algorithmic_bytes(plans[0])[:2])),
    }


def _sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _role(kernel_name):
    import re
    for key, role in KERNEL_ROLES.items():
        if re.search(key, kernel_name):
            return role
    return None


def _csv_rows(directory, suffix):
    import csv
    import glob
    files = glob.glob(os.path.join(directory, f"*{suffix}"))
    if len(files) != 1:
        raise SystemExit(f"expected one *{suffix} under {directory}, found {files}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def _counter_means(directory, counter, match):
    """Mean counter value (KiB) per dispatch of each kernel that `match` names."""
    acc = {}
    for r in _csv_rows(directory, "_counter_collection.csv"):
        if r["Counter_Name"] != counter:
            continue
        key = match(r["Kernel_Name"])
        if key:
            acc.setdefault(key, []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def _summarize(dirs, workload):
    """Markdown summary of the rocprofv3 runs: kernel durations, and HBM
    traffic per dispatch from FETCH_SIZE / WRITE_SIZE, each scaled by what the
    same counter reads for a plain 1 GiB device copy.  A role that several
    kernel instantiations serve in one run (the refresh of a workload with
    both GDN and KDA layers) gets one row per instantiation, and no
    machine-readable traffic: its launches are not alike."""
    import re
    stats_d, fetch_d, write_d, fetch_c, write_c = dirs
    trace = sorted(_csv_rows(stats_d, "_kernel_trace.csv"), key=lambda r: int(r["Dispatch_Id"]))
    names = {}
    for r in trace:
        role = _role(r["Kernel_Name"])
        if role:
            names.setdefault(role, set()).add(r["Kernel_Name"])

    def key(name):
        role = _role(name)
        if not role:
            return None
        if len(names.get(role, ())) <= 1:
            return role
        m = re.search(r"<([^<>]*)>", name)
        return f"{role} <{m.group(1) if m else name}>"

    stats = {}
    for r in _csv_rows(stats_d, "_kernel_stats.csv"):
        k = key(r["Name"])
        if k:
            stats[k] = (int(r["Calls"]), float(r["AverageNs"]), float(r["MinNs"]), float(r["MaxNs"]))
    # The timed launches alone: the stats run makes PROFILE_WARMUP + PROFILE_STEPS
    # rounds of every section, and the first round's launches (cold buffers)
    # are left out, as the bench's own clock leaves out its warm-up.
    runs = {}
    for r in trace:
        k = key(r["Kernel_Name"])
        if k:
            runs.setdefault(k, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    timed = {}
    for k, d in runs.items():
        skip = len(d) // (PROFILE_WARMUP + PROFILE_STEPS) * PROFILE_WARMUP
        timed[k] = sum(d[skip:]) / max(1, len(d) - skip)
    copy = lambda name: "copy" if "copyBuffer" in name or "copy_kernel" in name else None
    cal_f = _counter_means(fetch_c, "FETCH_SIZE", copy).get("copy")
    cal_w = _counter_means(write_c, "WRITE_SIZE", copy).get("copy")
    if not cal_f or not cal_w:
        raise SystemExit("no device-copy dispatch in the calibration runs")
    kib = (1 << 30) / 1024.0
    f_scale, w_scale = kib / cal_f, kib / cal_w
    fetch = _counter_means(fetch_d, "FETCH_SIZE", key)
    write = _counter_means(write_d, "WRITE_SIZE", key)
    traffic = {k: int(round(fetch[k] * 1024 * f_scale + write[k] * 1024 * w_scale))
               for k in fetch if k in write}
    lines = [f"| kernel | calls | average (us) | timed launches: average (us) | min (us) | "
             f"max (us) | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | HBM bytes per launch (calibrated) |",
             "|---|---|---|---|---|---|---|---|---|"]
    order = ROLE_ORDER
    for k in sorted(stats, key=lambda k: (order.index(k.split(" ")[0]), k)):
        c, avg, mn, mx = stats[k]
        lines.append(f"| {k} | {c} | {avg / 1e3:.1f} | {timed.get(k, float('nan')) / 1e3:.1f} | "
                     f"{mn / 1e3:.1f} | {mx / 1e3:.1f} | "
                     f"{fetch.get(k, float('nan')):.0f} | {write.get(k, float('nan')):.0f} | "
                     f"{traffic.get(k, 'n/a')} |")
    out = "\n".join(lines)
    out += (f"\n\nCalibration: a 1 GiB device copy reads FETCH_SIZE {cal_f:.1f} KiB and "
            f"WRITE_SIZE {cal_w:.1f} KiB per dispatch, so FETCH_SIZE is scaled by "
            f"{f_scale:.4f} and WRITE_SIZE by {w_scale:.4f}.\n\n")
    out += "Machine-readable (bench.py reads these lines):\n\n"
    out += f"    workload: {workload}\n"
    out += f"    kernel_sources_sha256: {_sources_sha256()}\n"
    machine = {k: v for k, v in traffic.items() if k in order}
    # A role served by several instantiations, each launched once per call
    # (the refresh of a model with GDN and KDA layers): its bytes per call.
    for role, kernels in names.items():
        keys = [key(nm) for nm in kernels]
        if len(keys) > 1 and all(k in traffic for k in keys) and \
                len({stats[k][0] for k in keys if k in stats}) == 1:
            machine[role] = sum(traffic[k] for k in keys)
    out += f"    traffic_bytes: {json.dumps(machine, sort_keys=True)}\n"
    return out


def _counter_table(dirs):
    table = {}
    for d in dirs:
        for r in _csv_rows(d, "_counter_collection.csv"):
            role = _role(r["Kernel_Name"])
            if role:
                table.setdefault(r["Counter_Name"], {}).setdefault(role, []).append(
                    float(r["Counter_Value"]))
    roles = [r for r in ROLE_ORDER if any(r in v for v in table.values())]
    lines = ["| counter | " + " | ".join(roles) + " |", "|" + "---|" * (len(roles) + 1)]
    for c in sorted(table):
        vals = [table[c].get(r) for r in roles]
        lines.append(f"| {c} | " + " | ".join(f"{sum(v) / len(v):.4g}" if v else "" for v in vals)
                     + " |")
    return "\n".join(lines)


def _recorded_traffic(workload):
    """HBM bytes per launch recorded under profiles/ for this workload, or {}
    when there is none or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.md")
    if not os.path.exists(path):
        return {}
    rec = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            for key in ("workload:", "kernel_sources_sha256:", "traffic_bytes:"):
                if line.startswith(key):
                    rec[key[:-1]] = line[len(key):].strip()
    if rec.get("workload") != workload or rec.get("kernel_sources_sha256") != _sources_sha256():
        return {}
    return json.loads(rec.get("traffic_bytes", "{}"))


def _timed(stream, rounds, warmup, *fns):
    """Median seconds of each of fns over `rounds` timed rounds (after
    warm-up rounds), with HIP events recorded on `stream` around every call."""
    import numpy as np
    import torch
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)]
          for _ in range(rounds)]
    for i in range(warmup + rounds):
        e = ev[i - warmup] if i >= warmup else None
        if e: e[0].record(stream)
        for j, fn in enumerate(fns):
            fn()
            if e: e[j + 1].record(stream)
    torch.cuda.synchronize()
    return [float(np.median([e[j].elapsed_time(e[j + 1]) for e in ev])) * 1e-3
            for j in range(len(fns))]


def _run_workload(name, args, stream, ex=None, n_workers=0):
    """Every measurement of one workload; the cpu_baseline when ex is given."""
    import numpy as np
    import torch

    import recurrent_state_cache_amd as R
    import workloads as W

    cfg, desc = _workload(name)
    t = time.perf_counter()
    P = R.Plan(cfg.layers, cfg.a_s, cfg.eps, cfg.w_max)
    plan_ms = (time.perf_counter() - t) * 1e3
    P.upload()
    info = P.info()
    n = cfg.n_ckpt
    dense = W.dense_states(cfg, n, device="cuda")
    pool = torch.empty((n, info["slot_bytes"]), dtype=torch.uint8, device="cuda")
    out = torch.empty((n, info["dense_bytes"]), dtype=torch.uint8, device="cuda")
    perm = np.random.default_rng(cfg.seed).permutation(n).astype(np.int32)
    src = torch.arange(n, dtype=torch.int32, device="cuda")
    slot = torch.from_numpy(perm).cuda()
    Wn = W.windows(cfg)
    T = int(Wn.sum())
    inp = W.refresh_inputs(cfg, Wn, device="cuda")
    alpha = W.refresh_decays(cfg, T, device="cuda")
    dst = torch.arange(cfg.n_req, dtype=torch.int32, device="cuda") % n
    pack_b, unpack_b, pack_qb, unpack_qb = _algorithmic_bytes(P)
    # Eq. 1 per token and replayed head: decay (1), readout (2), rank-1 write (2) flops per element
    flops = T * sum(5 * P.layer(l)["d_v"] * P.layer(l)["d_k"] * P.layer(l)["n_refresh_heads"]
                    for l in range(info["n_layers"]))
    head_steps = T * sum(P.layer(l)["n_refresh_heads"] for l in range(info["n_layers"]))
    n_groups = len({(P.layer(l)["kind"], P.layer(l)["d_k"]) for l in range(info["n_layers"])
                    if P.layer(l)["n_refresh_heads"]})
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]

    def step(e=None):
        if e: e[0].record(stream)
        R.ckpt_pack(P, dense, src, pool, slot, stream)
        if e: e[1].record(stream)
        R.ckpt_unpack_zero_fill(P, pool, slot, out, src, stream)
        if e: e[2].record(stream)
        R.ckpt_refresh_suffix_alpha(P, inp.k, inp.v, alpha, inp.beta, inp.tok_off, out, dst,
                                    stream)
        if e: e[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert P.status() == 0, "kernels flagged bad arguments"
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert P.status() == 0
    # per section: the median over the timed steps (HIP events on the stream)
    t_pack = float(np.median([e[0].elapsed_time(e[1]) for e in ev])) * 1e-3
    t_unpack = float(np.median([e[1].elapsed_time(e[2]) for e in ev])) * 1e-3
    t_ref = float(np.median([e[2].elapsed_time(e[3]) for e in ev])) * 1e-3

    rounds, warm = max(1, min(args.steps, args.side_steps)), args.warmup
    # INT8 checkpoints (Eq. 10): pack and unpack of the same checkpoints.
    pool_q = torch.empty((n, info["int8_slot_bytes"]), dtype=torch.uint8, device="cuda")
    t_pack_q, t_unpack_q = _timed(
        stream, rounds, warm,
        lambda: R.ckpt_pack_int8(P, dense, src, pool_q, slot, stream),
        lambda: R.ckpt_unpack_int8_zero_fill(P, pool_q, slot, out, src, stream))
    del pool_q
    # The same suffixes with the decays made in the kernel from bf16 gate
    # logits (Eq. 2), and both forms with per-head Eq. 7 windows.
    t_gate, = _timed(stream, rounds, warm,
                     lambda: R.ckpt_refresh_suffix(P, inp.k, inp.v, inp.a, inp.beta, inp.tok_off,
                                                   out, dst, stream))
    t_win, t_win_gate = _timed(
        stream, rounds, warm,
        lambda: R.ckpt_refresh_suffix_alpha_windowed(P, inp.k, inp.v, alpha, inp.beta,
                                                     inp.tok_off, out, dst, stream),
        lambda: R.ckpt_refresh_suffix_windowed(P, inp.k, inp.v, inp.a, inp.beta, inp.tok_off,
                                               out, dst, stream))
    assert P.status() == 0
    win_flops, win_head_tokens = _windowed_work(P, Wn)
    win_bytes = _windowed_bytes(P, Wn, decay_bytes=4)
    win_bytes_gate = _windowed_bytes(P, Wn, decay_bytes=2)
    win_sector_reads = _windowed_sector_reads(P, Wn)

    # dasc-wr load of the refreshed requests: unpack then refresh, against
    # the fused load (gate logits), with the full suffixes and with windows.
    wr = {}
    if not args.skip_wr_load:
        src_slot = slot[:cfg.n_req].contiguous()
        req_out = torch.arange(cfg.n_req, dtype=torch.int32, device="cuda")
        for hw, key in ((False, "full_suffix"), (True, "eq7_windows")):
            refresh = R.ckpt_refresh_suffix_windowed if hw else R.ckpt_refresh_suffix

            def two_step():
                R.ckpt_unpack_zero_fill(P, pool, src_slot, out, req_out, stream)
                refresh(P, inp.k, inp.v, inp.a, inp.beta, inp.tok_off, out, req_out, stream)

            def fused():
                R.ckpt_unpack_refresh(P, pool, src_slot, inp.k, inp.v, inp.a, inp.beta,
                                      inp.tok_off, out, req_out, head_windows=hw, stream=stream)
            t2, = _timed(stream, rounds, warm, two_step)
            t1, = _timed(stream, rounds, warm, fused)
            wr[key] = {"unpack_then_refresh_ms": round(t2 * 1e3, 4), "fused_ms": round(t1 * 1e3, 4),
                       "speedup": round(t2 / t1, 3)}
        assert P.status() == 0

    # The recurrence's own form (token by token on the vector units): the
    # reference point for the chunked kernel, on the KDA workload.
    t_rec = None
    if name == "kda":
        t_rec, = _timed(stream, rounds, warm,
                        lambda: R.ckpt_refresh_suffix_recurrent(P, inp.k, inp.v, inp.a, inp.beta,
                                                                inp.tok_off, out, dst, stream))
        assert P.status() == 0

    tp8 = _bench_tp(cfg, args, stream) if name in ("kda", "gdn") else None

    traffic = _recorded_traffic(name)
    mm_bf16, mm_f32 = _refresh_mfma_flops(P, Wn)

    def hbm(role, bytes_, secs, launches, kernel):
        a = bytes_ / secs / 1e9
        per_launch = int(bytes_ // launches)
        tr = traffic.get(role)
        return {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(a / HBM_PEAK_GBS, 4), "traffic": tr,
                # measured HBM bytes over the algorithmic bytes (a guard: <= 1.05)
                "traffic_over_algorithmic": round(tr / per_launch, 4) if tr else None,
                "kernel": kernel, "ms": round(secs * 1e3, 4), "bytes": int(bytes_),
                "launches": launches, "bytes_per_launch": per_launch}

    def mfma(role, fl, secs, kernel, extra=None):
        a = fl / secs / 1e12
        return {"bound": "mfma", "achieved": round(a, 3), "peak": FP32_MFMA_PEAK_TF,
                "unit": "TFLOP/s", "frac": round(a / FP32_MFMA_PEAK_TF, 4),
                "traffic": traffic.get(role), "kernel": kernel, "ms": round(secs * 1e3, 4),
                "flops": int(fl), "launches": n_groups, **(extra or {})}

    mover_gbs = (pack_b + unpack_b) * n / (t_pack + t_unpack) / 1e9
    res = {
        "workload": desc,
        "checkpoints": n, "requests": cfg.n_req, "refresh_tokens": T, "w_max": cfg.w_max,
        "dense_bytes": info["dense_bytes"], "slot_bytes": info["slot_bytes"],
        "c_ckpt": round(info["c_ckpt"], 4),
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "pack_unpack_gbs": round(mover_gbs, 2),
        "pack_unpack_frac_of_hbm_peak": round(mover_gbs / HBM_PEAK_GBS, 4),
        "refresh_request_tokens_per_s": round(T / t_ref, 1),
        "plan_build_ms": round(plan_ms, 3),
        "roofline": mfma("refresh", flops, t_ref,
                         "refresh_kernel<128, fp32 decays, false, false, false>",
                         {"note": "algorithmic fp32 flops (5 d^2 per token-head) against the fp32 "
                                  "matrix peak; the big products run as bf16 hi/lo splits on the "
                                  "bf16 matrix cores, whose issued rate is below",
                          "token_head_steps_per_s": round(head_steps / t_ref, 1),
                          "bf16_mfma_issued_tflops": round(mm_bf16 / t_ref / 1e12, 2),
                          "bf16_mfma_peak": BF16_MFMA_PEAK_TF,
                          "fp32_mfma_issued_tflops": round(mm_f32 / t_ref / 1e12, 2)}),
        "roofline_pack": hbm("pack", pack_b * n, t_pack, P.launches("pack", n)[0],
                             f"move_kernel<true> ({P.launches('pack', n)[1]} pairs per launch)"),
        "roofline_unpack": hbm("unpack", unpack_b * n, t_unpack, P.launches("unpack", n)[0],
                               f"move_kernel<false> ({P.launches('unpack', n)[1]} pairs per "
                               "launch)"),
        "int8": {
            "c_ckpt_int8": round(info["c_ckpt_int8"], 4),
            "pack_unpack_gbs": round(n * (pack_qb + unpack_qb) / (t_pack_q + t_unpack_q) / 1e9, 2),
            "pack": hbm("pack_int8", n * pack_qb, t_pack_q, P.launches("pack_int8", n)[0],
                        f"qmove_kernel<true, *> ({P.launches('pack_int8', n)[1]} pairs per "
                        "launch)"),
            "unpack": hbm("unpack_int8", n * unpack_qb, t_unpack_q, P.launches("unpack_int8", n)[0],
                          f"qmove_kernel<false> ({P.launches('unpack_int8', n)[1]} pairs per "
                          "launch)"),
        },
        "refresh_fused_gate": mfma("refresh_gate", flops, t_gate,
                                   "refresh_kernel<128, gate logits, false, false, false>",
                                   {"note": "the same suffixes with the decays made in the kernel "
                                            "from bf16 gate logits by Eq. 2"}),
        "refresh_eq7_windows": {
            "kernel": "refresh_kernel<128, fp32 decays, true, false, one_chunk> (per-head "
                      "windows; the one-chunk kernel when every window is at most 16 tokens)",
            "ms": round(t_win * 1e3, 4),
            "head_tokens": int(win_head_tokens),
            "head_tokens_per_s": round(win_head_tokens / t_win, 1),
            "speedup_vs_full_suffix": round(t_ref / t_win, 3),
            "roofline": {**mfma("refresh_windowed", win_flops, t_win, "refresh_kernel<.., true, ..>"),
                         "hbm_bytes": int(win_bytes),
                         "hbm_achieved_gbs": round(win_bytes / t_win / 1e9, 1),
                         "hbm_frac": round(win_bytes / t_win / 1e9 / HBM_PEAK_GBS, 4),
                         "sector_read_bytes": int(win_sector_reads),
                         "hbm_frac_with_sector_reads":
                             round((win_bytes + win_sector_reads) / t_win / 1e9 / HBM_PEAK_GBS, 4)},
            "fused_gate_ms": round(t_win_gate * 1e3, 4),
            "fused_gate_hbm_frac": round(win_bytes_gate / t_win_gate / 1e9 / HBM_PEAK_GBS, 4),
            "fused_gate_traffic": traffic.get("refresh_windowed_gate"),
        },
    }
    if wr:
        res["dasc_wr_load"] = dict(wr, requests=cfg.n_req)
    if tp8:
        res["tp8_storage_balancing"] = tp8
    if t_rec is not None:
        res["refresh_recurrent_form"] = {
            "kernel": "recurrent_kernel<128, gate> (token by token, fp32 vector units)",
            "ms": round(t_rec * 1e3, 4),
            "achieved_tflops": round(flops / t_rec / 1e12, 3),
            "fp32_vector_peak_unpacked": FP32_VALU_UNPACKED_TF,
            "frac_of_unpacked_peak": round(flops / t_rec / 1e12 / FP32_VALU_UNPACKED_TF, 4),
            "chunked_fused_gate_speedup": round(t_rec / t_gate, 3),
            "note": "same suffixes, output and tolerance as the chunked refresh from gate logits; "
                    "the vector units' fp32 rate without packed FMA (the library is compiled "
                    "without packed fp32 instructions) is half the 157.3 TF/s datasheet figure",
        }
    if ex is not None:
        m = min(32, n)
        dense_cpu = dense[:m].cpu().numpy()
        bits = lambda x: x.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
        rows = (bits(inp.k), bits(inp.v), alpha.cpu().numpy(), inp.beta.cpu().numpy(),
                inp.tok_off.cpu().numpy())
        res["cpu_baseline"] = _cpu_baseline(cfg, P, ex, n_workers, dense_cpu, pack_b, unpack_b,
                                            rows, Wn, pack_qb + unpack_qb)
    del dense, pool, out, inp, alpha
    torch.cuda.empty_cache()
    return res


def main():
    args = _args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the library has no "
              f"multi-GPU path", file=sys.stderr)
        sys.exit(2)
    if args.summarize:
        print(_summarize(args.summarize, args.workload))
        return
    if args.counters:
        print(_counter_table(args.counters))
        return
    # The oracle's worker pool starts before anything touches the GPU.
    ex = n_workers = None
    if not args.no_cpu_baseline and not args.calibrate_copy:
        ex, n_workers = _cpu_pool()
    import torch
    if args.calibrate_copy:
        _calibrate_copy(args.steps)
        return
    stream = torch.cuda.current_stream()
    names = WORKLOADS if args.workload == "all" else (args.workload,)
    results = {}
    for i, name in enumerate(names):
        results[name] = _run_workload(name, args, stream, ex if i == 0 else None, n_workers)
    if ex is not None:
        ex.shutdown()
    head = results[names[0]]
    cpu = head.pop("cpu_baseline", None)
    line = {
        "metric": "checkpoint pack+unpack GB/s (% HBM peak); suffix-refresh tokens/s, 1 MI355X",
        "value": head["pack_unpack_gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32 copy (pack/unpack), f32 (refresh: fp32 state and accumulation, "
                 "products on bf16 hi/lo splits)",
        "data": "synthetic",
        "config": {k: head[k] for k in ("workload", "checkpoints", "requests", "refresh_tokens",
                                        "w_max", "dense_bytes", "slot_bytes", "c_ckpt")},
        "pack_unpack_frac_of_hbm_peak": head["pack_unpack_frac_of_hbm_peak"],
        "refresh_request_tokens_per_s": head["refresh_request_tokens_per_s"],
        "roofline": head["roofline"],
        "roofline_pack": head["roofline_pack"],
        "roofline_unpack": head["roofline_unpack"],
        **{k: v for k, v in head.items()
           if k not in ("workload", "checkpoints", "requests", "refresh_tokens", "w_max",
                        "dense_bytes", "slot_bytes", "c_ckpt", "ms_per_step", "pack_unpack_gbs",
                        "pack_unpack_frac_of_hbm_peak", "refresh_request_tokens_per_s",
                        "roofline", "roofline_pack", "roofline_unpack")},
        **{name: results[name] for name in names[1:]},
    }
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
