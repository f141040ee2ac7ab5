"""Benchmark of the 4-bit KV-cache hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
quantize-and-append the batch's tokens into the paged cache, then decode
attention over a cache (the longprefix workload appends one token per sequence
before each of its 64 decodes).  The step decodes the pool quantized two steps
earlier.  Inputs and pools rotate over enough copies that each kernel's
distinct data spans at least twice the 256 MB Infinity Cache, so every launch
reads from HBM.  Inputs are resident in HBM before any timed region starts.

Timing (HIP events on the launch stream, the host queue filled first):
  * ms_per_step: K whole steps between two events;
  * per-kernel launch time: K back-to-back launches of the kernel alone over
    the rotating copies between two events (the decode launch includes its
    split merge), so that event markers add nothing to each kernel.

Output: one JSON line.  ``value`` is the decode's effective KV bandwidth
(logical 4-bit KV bytes read / decode time); ``quantize_tokens_per_s`` the
quantize rate; ``roofline`` the kernel that takes most of the step time
against the 8 TB/s HBM peak; ``cpu_baseline`` the CPU oracle timed on this
host on a bounded sample.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--config agentic]
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", default="cascade",
                   choices=["llama8b", "agentic", "longprefix", "fp4", "tq4v2", "calib", "verify", "prefill",
                            "verify_fp4", "prefill_fp4", "agentic_fp4", "cascade_fp4",
                            "cascade"],
                   help="cascade (the default): the agentic workload, decoded with its shared prefix blocks read "
                        "once per group of sequences (the per-sequence decode is timed beside it); agentic: the same "
                        "workload with the per-sequence decode; calib: the calibrated key-table fit of a 32-layer "
                        "stack; verify / prefill: multi-token attention over the cache; tq4v2: the llama8b shape "
                        "with 2-bit values; *_fp4: the same workload over an MX-FP4 cache (each its own JSON line)")
    p.add_argument("--copies", type=int, default=0, help="rotating input/pool copies (0 = automatic)")
    p.add_argument("--cascade-group-blocks", type=int, default=48,
                   help="cascade: shared ranges are cut into groups of at most this many blocks")
    p.add_argument("--cascade-group-members", type=int, default=0,
                   help="cascade: groups are cut into groups of at most this many sequences "
                        "(default: 32 rows' worth, the direct kernel's tile)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--ceilings", action="store_true",
                   help="print the measured bandwidth ceilings of this GPU (stream read, record gather, copy, fill) "
                        "and exit")
    p.add_argument("--no-ceilings", action="store_true",
                   help="leave the measured bandwidth ceilings out of the line")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain device copy of known size (for counter calibration)")
    return p.parse_args()


def payload_row_bytes(fmt, d):
    """Bytes of the record sections per (token, kv-head), the padding of a
    record to whole 128-byte lines excluded (algorithmic bytes)."""
    g = d // 32
    if fmt == 1:
        return d // 2 + d // 2 + g + g           # MX-FP4: codes, exponent bytes
    vcode = d // 2 if fmt == 0 else d // 4       # TQ4/4 or TQ4/2 value codes
    return d // 2 + vcode + 4 * g + 2            # key codes, value codes, (scale, min), key scale


def kernel_source_hash():
    """Hash of the native sources with comments and whitespace taken out, so
    that stored counters stay valid across edits of comments only."""
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bit_quantized_kv_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(name.encode())
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def ceilings():
    import torch
    print(json.dumps({"ceilings": measure_ceilings(), "device": torch.cuda.get_device_name(0)}))


def measure_ceilings():
    """Bandwidth ceilings of this GPU for the path's access patterns, from the
    probe kernels of libtqprobe.so (no arithmetic on the data): a streaming
    read of 4 GiB, a gather of whole TQ4/4 records (2336 of every 2432 bytes,
    D = 128) of a 2 GiB pool in random order, the decode's pattern,
    and the quantize's mix of traffic (7 words read, 2 written per item; 1.1 GB
    read per launch), its output written in order or as 2 KB pieces at
    scattered places; each the best over a few grid sizes of the median of
    five launches.  A torch device copy and fill of 1 GiB are given beside
    them."""
    import ctypes

    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "bit_quantized_kv_amd", "libtqprobe.so"))
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.tqprobe_stream_read.argtypes = [P, I64, P, I32, P]
    lib.tqprobe_record_gather.argtypes = [P, P, I64, I64, I32, P, I32, P]
    lib.tqprobe_mixed_stream.argtypes = [P, P, P, I64, I32, P]
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")

    def med(fn, reps=5):
        assert fn() == 0
        torch.cuda.synchronize()
        out = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            rc = fn()
            b.record(stream)
            torch.cuda.synchronize()
            assert rc == 0
            out.append(a.elapsed_time(b) * 1e-3)
        return sorted(out)[reps // 2]

    res = {}
    n = 4 << 30
    buf = torch.ones(n // 4, dtype=torch.float32, device="cuda")   # equal words: every fold is 0
    rates = {g: n / med(lambda g=g: lib.tqprobe_stream_read(buf.data_ptr(), n, sink.data_ptr(), g, sp)) / 1e9
             for g in (2048, 4096, 8192, 16384, 32768)}
    g_best = max(rates, key=rates.get)
    res["stream_read_GBps"], res["stream_read_grid"] = round(rates[g_best], 1), g_best
    del buf
    from bit_quantized_kv_amd import Cache
    stride = Cache(0, 128, 1, 1).record_bytes
    rec = 16 * payload_row_bytes(0, 128)
    nrec = (2 << 30) // stride
    pool = torch.ones(nrec * stride // 4, dtype=torch.float32, device="cuda")
    ids = torch.from_numpy(np.random.default_rng(7).permutation(nrec).astype(np.int32)).cuda()
    rates = {g: nrec * rec / med(lambda g=g: lib.tqprobe_record_gather(pool.data_ptr(), ids.data_ptr(), nrec, stride,
                                                                       rec, sink.data_ptr(), g, sp)) / 1e9
             for g in (1024, 2048, 4096, 8192, 16384)}
    g_best = max(rates, key=rates.get)
    res["record_gather_GBps"], res["record_gather_grid"] = round(rates[g_best], 1), g_best
    res["record_bytes"], res["record_stride"], res["records"] = rec, stride, nrec
    del pool, ids
    # the quantize's 7 : 2 mix: 1.1 GB read and 0.31 GB written per launch
    chunks = (1100 << 20) // (7 * 1024)
    src = torch.ones(chunks * 7 * 256, dtype=torch.float32, device="cuda")
    dst = torch.empty(chunks * 2 * 256, dtype=torch.float32, device="cuda")
    moved = chunks * 9 * 1024
    perm = torch.from_numpy(np.random.default_rng(8).permutation(chunks).astype(np.int32)).cuda()
    for key, pp in (("mixed_7r2w", None), ("mixed_7r2w_scattered", perm)):
        pptr = pp.data_ptr() if pp is not None else None
        rates = {g: moved / med(lambda g=g: lib.tqprobe_mixed_stream(src.data_ptr(), dst.data_ptr(), pptr, chunks, g,
                                                                     sp)) / 1e9
                 for g in (2048, 4096, 8192, 16384)}
        g_best = max(rates, key=rates.get)
        res[key + "_GBps"], res[key + "_grid"] = round(rates[g_best], 1), g_best
    res["mixed_7r2w_bytes"] = moved
    del src, dst, perm
    m = 1 << 30
    a = torch.ones(m // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    res["torch_copy_GBps"] = round(2 * m / med(lambda: (b.copy_(a), 0)[1]) / 1e9, 1)
    res["torch_fill_GBps"] = round(m / med(lambda: (b.fill_(2.0), 0)[1]) / 1e9, 1)
    res["peak_GBps"] = HBM_PEAK_GBPS
    del a, b, sink
    torch.cuda.empty_cache()
    return res


def copy_calibration():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_launch": n, "launches": 5}))


class Bench:
    def __init__(self, cfg, copies, cascade=False, group_blocks=48, group_members=None):
        import torch

        import workloads
        from bit_quantized_kv_amd import Cache
        self.torch = torch
        self.w = workloads.make(cfg)
        self.cfg = self.w.cfg
        c, w = self.cfg, self.w
        dev = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
        i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
        plan = w.write_plan()
        ks, vs, ss = [], [], []
        for b, t0, t1 in plan:
            k, v = w.sequence_kv(b)
            ks.append(k[t0:t1])
            vs.append(v[t0:t1])
            ss.append(w.slots(b, t0, t1))
        self.n_tokens = int(sum(t1 - t0 for _, t0, t1 in plan))
        k0, v0, s0 = dev(np.concatenate(ks)), dev(np.concatenate(vs)), i32(np.concatenate(ss))
        # appended tokens (one per sequence per decode step), if any
        self.appends = []
        if c.appended:
            kvs = [w.sequence_kv(b) for b in range(c.batch)]
            for step in range(c.decode_steps):
                t = w.prompt_lens + step
                ka = np.stack([kvs[b][0][int(t[b])] for b in range(c.batch)])
                va = np.stack([kvs[b][1][int(t[b])] for b in range(c.batch)])
                sa = np.array([w.slots(b, int(t[b]), int(t[b]) + 1)[0] for b in range(c.batch)])
                self.appends.append((dev(ka), dev(va), i32(sa)))
        rec_bytes = Cache(c.fmt, c.head_dim, c.num_kv_heads, 1).record_bytes
        self.row_bytes = payload_row_bytes(c.fmt, c.head_dim)
        pool_bytes = rec_bytes * c.num_kv_heads * w.num_blocks
        in_bytes = k0.numel() * 4
        # rotating copies so that no launch finds its data in the 256 MB
        # Infinity Cache: every kernel's distinct data spans >= 2x its size
        mall2 = 2 * 256 * 2 ** 20
        self.in_copies = copies if copies > 0 else max(3, -(-mall2 // in_bytes))
        self.pool_copies = copies if copies > 0 else max(3, -(-mall2 // pool_bytes))
        self.kv = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(self.in_copies - 1)]
        self.slots = s0
        self.caches = [Cache(c.fmt, c.head_dim, c.num_kv_heads, w.num_blocks) for _ in range(self.pool_copies)]
        self.table = i32(w.block_table)
        self.q = [dev(w.query_bits(s)) for s in range(c.decode_steps)]
        self.ctx = [i32(w.context_lens_at(s)) for s in range(c.decode_steps)]
        self.max_ctx = [int(w.context_lens_at(s).max()) for s in range(c.decode_steps)]
        self.out = torch.empty((c.batch, c.num_q_heads, c.head_dim), dtype=torch.float32, device="cuda")
        for cache in self.caches:   # size the decode workspace outside the timed region
            cache.workspace(c.batch, c.num_q_heads, max(self.max_ctx))
        self.cascade = None
        if cascade:
            from bit_quantized_kv_amd import CascadeGroups
            g = c.num_q_heads // c.num_kv_heads
            self.cascade = CascadeGroups(c.batch, w.shared_block_groups(w.context_lens_at(0)), max_blocks=group_blocks,
                                         max_members=group_members if group_members else max(1, 32 // g))
            for cache in self.caches:
                cache.cascade_decode(self.q[0], self.table, self.ctx[0], self.max_ctx[0], c.scale, self.cascade,
                                     out=self.out)
        self.stream = torch.cuda.current_stream()

    # algorithmic bytes ---------------------------------------------------------
    def quantize_bytes(self):
        c = self.cfg
        per_tok = c.num_kv_heads * (2 * 2 * c.head_dim + self.row_bytes) + 4
        n = self.n_tokens
        return n * per_tok

    def append_bytes(self):
        c = self.cfg
        return c.batch * (c.num_kv_heads * (2 * 2 * c.head_dim + self.row_bytes) + 4)

    def decode_bytes(self, step, unique=False):
        c, w = self.cfg, self.w
        lens = w.context_lens_at(step).astype(np.int64)
        kv = int(lens.sum()) * c.num_kv_heads * self.row_bytes
        if unique and c.shared_seqs:
            ids = set()
            toks = 0
            for b in range(c.batch):
                nb = -(-int(lens[b]) // 16)
                for j, bid in enumerate(w.block_table[b, :nb].tolist()):
                    if bid not in ids:
                        ids.add(bid)
                        toks += min(16, int(lens[b]) - 16 * j)
            kv = toks * c.num_kv_heads * self.row_bytes
        other = c.batch * c.num_q_heads * c.head_dim * (2 + 4) + int((-(-lens // 16)).sum()) * 4 + c.batch * 4
        return kv, kv + other

    # launches --------------------------------------------------------------------
    def quantize(self, i):
        k, v = self.kv[i % self.in_copies]
        self.caches[i % self.pool_copies].quantize_append(k, v, self.slots)

    def decode(self, i, s, plain=False):
        c = self.cfg
        if self.cascade is not None and not plain:
            self.caches[i % self.pool_copies].cascade_decode(self.q[s], self.table, self.ctx[s], self.max_ctx[s],
                                                             c.scale, self.cascade, out=self.out)
            return
        self.caches[i % self.pool_copies].decode(self.q[s], self.table, self.ctx[s], self.max_ctx[s], c.scale,
                                                 out=self.out)

    def append(self, i, s):
        """The single-token append of decode step s (one token per sequence)
        into pool copy i."""
        ka, va, sa = self.appends[s]
        self.caches[i % self.pool_copies].quantize_append(ka, va, sa)

    def step(self, i):
        """One pass of the whole path: quantize-append batch i into pool copy
        i, then (append one token per sequence and) decode over pool copy i-2."""
        c = self.cfg
        self.quantize(i)
        dc = (i - 2) % self.pool_copies
        for s in range(c.decode_steps):
            if self.appends:
                ka, va, sa = self.appends[s]
                self.caches[dc].quantize_append(ka, va, sa)
            self.decode(dc, s)


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cpu_worker(cfg, unit_q, deadline_s, barrier, out_q):
    """One oracle worker process: after the start barrier, take (sequence,
    kv-head) units from the shared queue and quantize them until the deadline
    (seconds after the start); wait for every worker; decode the units it
    quantized; wait again; then count the near-ties of its rows and report."""
    try:
        from threadpoolctl import threadpool_limits
        _limits = threadpool_limits(limits=1)  # noqa: F841  (kept for the worker's life)
    except ImportError:
        pass
    import queue

    import workloads
    from oracle import attention, paged, tq4
    w = workloads.make(cfg)
    c = w.cfg
    g = c.num_q_heads // c.num_kv_heads
    lens = w.context_lens_at(0)
    q_all = workloads.bf16_bits_to_f32(w.query_bits(0))
    res = {"tq": 0.0, "td": 0.0, "toks": 0, "units": 0, "kel": 0, "kties": 0, "kdiff": 0, "kfree": 0,
           "vel": 0, "vties": 0, "vdiff": 0, "vfree": 0}
    done = []
    barrier.wait()
    start = time.perf_counter()
    while time.perf_counter() - start < deadline_s:
        try:
            b, h = unit_q.get_nowait()
        except queue.Empty:
            break
        T = int(lens[b])
        k, v = w.sequence_kv(b)
        kf, vf = workloads.bf16_bits_to_f32(k[:T, h:h + 1]), workloads.bf16_bits_to_f32(v[:T, h:h + 1])
        pool = paged.PagedPool(c.fmt, w.num_blocks, 1, c.head_dim)
        pool.append(kf, vf, w.slots(b, 0, T))
        done.append((b, h, pool, kf[:, 0], vf[:, 0]))
        res["toks"] += T
        res["units"] += 1
    barrier.wait()
    for b, h, pool, _, _ in done:
        attention.decode(pool, q_all[:, h * g:(h + 1) * g], w.block_table, lens, c.scale,
                         rows=[(b, j) for j in range(g)])
    barrier.wait()
    # near-ties of the sampled rows (after the timed phases): the fp32
    # decision rule (the kernels' rule) against the exact fp64 rule and its
    # near-tie flags; a difference away from a flagged near-tie would be a
    # fault of the rules
    if c.fmt in (0, 2):
        levels = 15 if c.fmt == 0 else 3
        for _, _, pool, kf, vf in done:
            s = tq4.key_scale(kf)
            kc = tq4.key_codes(kf, s, pool.table)
            kx, knear = tq4.key_codes_exact(kf, s, pool.table)
            vc, sc, mn = tq4.value_encode(vf, levels)
            vx, vnear = tq4.value_codes_exact(vf, sc, mn, levels=levels)
            res["kel"] += kc.size
            res["kties"] += int(knear.sum())
            res["kdiff"] += int((kc != kx).sum())
            res["kfree"] += int(((kc != kx) & ~knear).sum())
            res["vel"] += vc.size
            res["vties"] += int(vnear.sum())
            res["vdiff"] += int((vc != vx).sum())
            res["vfree"] += int(((vc != vx) & ~vnear).sum())
    out_q.put(res)


def cpu_baseline(cfg, deadline_s=10.0):
    """The CPU oracle, as it stands, on a bounded sample of the workload, run
    in worker processes over this host's cores (at most 16; BLAS limited to
    one thread each).  Phase 1: the workers take (sequence, kv-head) units in
    order from a shared queue and quantize each unit's tokens, until
    ``deadline_s`` seconds have passed; phase 2: each worker decodes the g
    query heads of its units.  Each phase is timed on the wall clock between
    barriers.  Run before the GPU is initialised (the workers are forked).
    Also returns the near-tie counts of the sampled rows."""
    import multiprocessing as mp

    import workloads
    c = cfg
    units = [(b, h) for b in range(c.batch) for h in range(c.num_kv_heads)]
    ncores = max(1, min(len(os.sched_getaffinity(0)), 16, len(units)))
    ctx = mp.get_context("fork")
    unit_q = ctx.Queue()
    for u in units:
        unit_q.put(u)
    time.sleep(0.2)                      # the queue's feeder thread has flushed
    barrier = ctx.Barrier(ncores + 1)
    out_q = ctx.Queue()
    procs = [ctx.Process(target=_cpu_worker, args=(cfg, unit_q, deadline_s, barrier, out_q)) for _ in range(ncores)]
    for p in procs:
        p.start()
    barrier.wait()                       # workers ready: phase 1 starts
    t0 = time.perf_counter()
    barrier.wait()                       # phase 1 (quantize) done
    t1 = time.perf_counter()
    barrier.wait()                       # phase 2 (decode) done
    t2 = time.perf_counter()
    parts = [out_q.get() for _ in procs]
    for p in procs:
        p.join()
    tot = {k: sum(r[k] for r in parts) for k in parts[0]}
    d = c.head_dim
    row = {0: d + 2 + d // 8, 1: d + d // 16, 2: 3 * d // 4 + 2 + d // 8}[c.fmt]   # bytes per token-head
    toks = tot["toks"]
    g = c.num_q_heads // c.num_kv_heads
    res = {
        "value": toks * row / (t2 - t1) / 1e9,
        "unit": "GB/s",
        "cores": ncores,
        "kind": "oracle",
        "cpu_model": _cpu_model(),
        "sample": f"{c.name}: the first {tot['units']} of {len(units)} (sequence, kv-head) units, {toks} token-heads, "
                  f"on {ncores} worker processes: quantize {t1 - t0:.2f} s, decode of their {g} query heads each "
                  f"{t2 - t1:.2f} s wall (numpy fp64, BLAS limited to 1 thread per worker)",
        "quantize_tokens_per_s": toks / (t1 - t0) / c.num_kv_heads,
    }
    if c.fmt in (0, 2):
        res["near_ties"] = {
            "key_codes": tot["kel"], "key_near_ties": tot["kties"], "key_rule_differences": tot["kdiff"],
            "key_differences_not_flagged": tot["kfree"],
            "value_codes": tot["vel"], "value_near_ties": tot["vties"], "value_rule_differences": tot["vdiff"],
            "value_differences_not_flagged": tot["vfree"],
            "rule": "codes of the sampled rows by the fp32 decision rule (the kernels' rule; the GPU's codes are "
                    "bit-identical to it) against the exact fp64 rule; near-tie = gap below 1e-5 code units",
        }
    return res


def traffic_from_profiles(cfg_name, kernel):
    """HBM bytes per launch of ``kernel`` ("quantize": the bulk quantize
    dispatch; "decode": the decode kernel plus its merge) from the committed
    FETCH_SIZE / WRITE_SIZE counter runs, each scaled by what the counter
    reads for a plain copy of known size.  None unless the counters were
    taken on the current kernel sources."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
        if d.get("kernel_source_hash") != kernel_source_hash():
            return None
        ents = d["workloads"][cfg_name]
        def hbm(e):
            return (e["fetch_kib_per_dispatch"] * d["fetch_scale"] + e["write_kib_per_dispatch"] * d["write_scale"]) * 1024
        if kernel == "quantize":
            cands = [(int(k.split("|")[1]), e) for k, e in ents.items() if "quantize_kernel" in k]
            return round(hbm(max(cands, key=lambda x: x[0])[1])) if cands else None
        if kernel == "multitoken":
            # the attention launch: the direct or staged kernel and its merge
            parts = [e for k, e in ents.items() if "multitoken" in k or "mt_direct" in k]
        elif cfg_name.startswith("cascade"):
            # the cascade launch: the own-token pass, the shared-block pass and
            # their merge (not the per-sequence decode timed beside it)
            parts = [e for k, e in ents.items()
                     if "quantize_kernel" not in k and ("cascade_merge" in k or "true" in k.split("|")[0])]
        else:
            # the decode launch: decode kernel and merge
            parts = [e for k, e in ents.items() if "quantize_kernel" not in k]
        return round(sum(hbm(e) for e in parts)) if parts else None
    except Exception:
        return None


def mfma_busy_from_profiles(cfg_name, kernel_prefix):
    """SQ_VALU_MFMA_BUSY_CYCLES per SIMD-cycle of the kernel whose name starts
    with ``kernel_prefix``, from the committed counter run; None unless it was
    taken on the current kernel sources."""
    path = os.path.join(PROFILES, "mfma_busy.json")
    try:
        d = json.load(open(path))
        if d.get("kernel_source_hash") != kernel_source_hash():
            return None
        for k, e in d["workloads"].get(cfg_name, {}).items():
            if k.startswith(kernel_prefix):
                return e["mfma_busy"]
    except Exception:
        return None
    return None


_SPIN_CYCLES_PER_MS = None


def gpu_spin(ms):
    """Occupy the stream for about ``ms`` milliseconds (torch's spin kernel)."""
    import torch
    global _SPIN_CYCLES_PER_MS
    if _SPIN_CYCLES_PER_MS is None:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        torch.cuda._sleep(1_000_000)
        b.record()
        torch.cuda.synchronize()
        _SPIN_CYCLES_PER_MS = 1_000_000 / max(a.elapsed_time(b), 1e-3)
    torch.cuda._sleep(int(ms * _SPIN_CYCLES_PER_MS))


def timed(torch, stream, launches, enqueue):
    """Average GPU time of `launches` calls of enqueue(j), measured with two HIP
    events on the launch stream around them.  A GPU spin placed first lets the
    host queue every launch before the first one runs, so host enqueue time
    does not show up as gaps between kernels."""
    t0 = time.perf_counter()
    enqueue(0)
    torch.cuda.synchronize()
    per = time.perf_counter() - t0
    gpu_spin(1.5 * per * launches * 1e3 + 2.0)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for j in range(launches):
        enqueue(j)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / launches


def timed_median(torch, stream, launches, enqueue, regions=3):
    """Median over ``regions`` timed regions of ``launches`` launches each
    (the per-kernel figures; the whole-step figure is one region of exactly
    the requested steps)."""
    return sorted(timed(torch, stream, launches, enqueue) for _ in range(regions))[regions // 2]


FP64_VALU_PEAK_TFLOPS = 78.6


def calib_cpu_baseline(kbits, max_iters, budget_s=10.0):
    """The oracle's fit of as many layers as fit in about ``budget_s``."""
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:
        threadpool_limits = None
    import workloads
    from oracle import calibrate, lloyd_max
    k = workloads.bf16_bits_to_f32(kbits)
    init = lloyd_max.default_key_table_f16()
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    if ctx:
        ctx.__enter__()
    try:
        t0 = time.perf_counter()
        n = 0
        for layer in range(k.shape[0]):
            calibrate.fit_table(k[layer], init, max_iters)
            calibrate.key_mse(k[layer], init)
            n += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        dt = time.perf_counter() - t0
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    return {"value": n / dt, "unit": "layers/s", "cores": 1, "kind": "oracle",
            "sample": f"calib: {n} of {k.shape[0]} layers fitted ({max_iters} updates at most) with the "
                      f"initial-table MSE, {dt:.2f} s (numpy fp64, BLAS limited to 1 thread)"}


def bench_calib(args):
    """Calibrated key-table fit: 32 layers x 20 tokens x 8 kv-heads x D 128,
    at most 100 Lloyd updates, one launch per stack."""
    import torch

    import workloads
    from bit_quantized_kv_amd import calibrate_key_tables
    torch.cuda.set_device(0)
    kbits = workloads.calibration_keys()
    layers, rows, d = kbits.shape
    max_iters = 100
    k = torch.from_numpy(np.ascontiguousarray(kbits).view(np.int16)).view(torch.bfloat16).cuda()
    stream = torch.cuda.current_stream()
    out = calibrate_key_tables(k, None, max_iters)
    for _ in range(args.warmup):
        calibrate_key_tables(k, None, max_iters)
    torch.cuda.synchronize()
    updates = out[3].cpu().numpy()
    ms = timed(torch, stream, args.steps, lambda j: calibrate_key_tables(k, None, max_iters))
    # algorithmic fp64 work: per sample and Lloyd pass, a 4-compare search of
    # the 15 midpoints and one add into its cell's sum; passes = updates + 1
    samples = rows * d
    ops = float(np.sum(updates + 1)) * samples * 5
    achieved = ops / (ms * 1e-3) / 1e12
    res = {
        "metric": "calibrated key-table fit: layers per second",
        "value": round(layers / (ms * 1e-3), 1),
        "unit": "layers/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "data": "synthetic (seeded; Student-t keys with per-layer outlier channels)",
        "config": {"workload": f"calib: {layers} layers x {rows} rows (20 tokens x 8 kv-heads) x head_dim {d}, "
                               f"at most {max_iters} Lloyd updates",
                   "updates_mean": float(np.mean(updates))},
        "roofline": {"bound": "alu", "achieved": round(achieved, 4), "peak": FP64_VALU_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / FP64_VALU_PEAK_TFLOPS, 6), "traffic": None,
                     "kernel": "calibrate", "avg_launch_us": round(ms * 1e3, 2)},
        "kernel_source_hash": kernel_source_hash(),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = calib_cpu_baseline(kbits, max_iters)
    print(json.dumps(res))


MFMA_F16_PEAK_TFLOPS = 2500.0


class MtBench:
    """Multi-token attention: each sequence's last M tokens are the query
    tokens.  A step appends their keys and values (quantize) and runs the
    causal multi-token attention over the whole cached context."""

    def __init__(self, name, copies):
        import torch

        import workloads
        from bit_quantized_kv_amd import Cache
        self.torch = torch
        cfg = workloads.MT_CONFIGS[name]
        self.m = workloads.MT_QUERY_TOKENS[name]
        self.w = w = workloads.make(cfg)
        self.cfg = c = w.cfg
        dev = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
        i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
        qbits, q_start = w.multi_queries(self.m)
        self.q = dev(qbits)
        self.q_start_np = q_start
        self.q_start = i32(q_start)
        self.ctx_np = w.total_lens.astype(np.int32)
        self.ctx = i32(self.ctx_np)
        self.max_q = int(np.max(np.diff(q_start)))
        self.max_ctx = int(self.ctx_np.max())
        self.table = i32(w.block_table)
        rec = Cache(c.fmt, c.head_dim, c.num_kv_heads, 1).record_bytes
        self.row_bytes = payload_row_bytes(c.fmt, c.head_dim)
        pool_bytes = rec * c.num_kv_heads * w.num_blocks
        self.copies = copies if copies > 0 else max(3, -(-2 * 256 * 2 ** 20 // pool_bytes))
        self.caches = [Cache(c.fmt, c.head_dim, c.num_kv_heads, w.num_blocks) for _ in range(self.copies)]
        # the whole context quantized once into every copy (set-up, untimed)
        plan = w.write_plan(w.total_lens)
        ks, vs, ss, ka, va, sa = [], [], [], [], [], []
        for b, t0, t1 in plan:
            k, v = w.sequence_kv(b)
            ks.append(k[t0:t1])
            vs.append(v[t0:t1])
            ss.append(w.slots(b, t0, t1))
        for b in range(c.batch):
            k, v = w.sequence_kv(b)
            t1 = int(w.total_lens[b])
            t0 = t1 - int(q_start[b + 1] - q_start[b])
            ka.append(k[t0:t1])
            va.append(v[t0:t1])
            sa.append(w.slots(b, t0, t1))
        k0, v0, s0 = dev(np.concatenate(ks)), dev(np.concatenate(vs)), i32(np.concatenate(ss))
        for cache in self.caches:
            cache.quantize_append(k0, v0, s0)
        del k0, v0, s0
        self.ka, self.va, self.sa = dev(np.concatenate(ka)), dev(np.concatenate(va)), i32(np.concatenate(sa))
        self.n_new = int(self.sa.numel())
        self.out = torch.empty(self.q.shape, dtype=torch.float32, device="cuda")
        for cache in self.caches:
            self.attend(cache)
        torch.cuda.synchronize()
        self.stream = torch.cuda.current_stream()

    def attend(self, cache):
        c = self.cfg
        cache.multitoken(self.q, self.q_start, self.max_q, self.table, self.ctx, self.max_ctx, c.scale, out=self.out)

    def append(self, i):
        self.caches[i % self.copies].quantize_append(self.ka, self.va, self.sa)

    def attention(self, i):
        self.attend(self.caches[i % self.copies])

    def step(self, i):
        self.append(i)
        self.attention(i)

    def work(self):
        """Algorithmic bytes and flops of one attention call: every cached
        token-head read once (shared blocks once), q read, out written; 4 D
        flops (QK and PV multiply-adds) per visible key of every row."""
        c, w = self.cfg, self.w
        ids = {}
        for b in range(c.batch):
            n = -(-int(self.ctx_np[b]) // 16)
            for j, bid in enumerate(w.block_table[b, :n].tolist()):
                ids[bid] = max(ids.get(bid, 0), min(16, int(self.ctx_np[b]) - 16 * j))
        kv = sum(ids.values()) * c.num_kv_heads * self.row_bytes
        nq = int(self.q.shape[0])
        byts = kv + nq * c.num_q_heads * c.head_dim * (2 + 4) + (c.batch + 1) * 4 * 2
        flops = 0
        for b in range(c.batch):
            mb = int(self.q_start_np[b + 1] - self.q_start_np[b])
            t = int(self.ctx_np[b])
            vis = sum(t - mb + i + 1 for i in range(mb))
            flops += 4 * c.head_dim * vis * c.num_q_heads
        return byts, flops, kv


def bench_multitoken(args):
    import torch
    torch.cuda.set_device(0)
    mb = MtBench(args.config, args.copies)
    c = mb.cfg
    for i in range(args.warmup + mb.copies):
        mb.step(i)
    torch.cuda.synchronize()
    base = args.warmup + mb.copies
    step_ms = timed(torch, mb.stream, args.steps, lambda j: mb.step(base + j))
    a_ms = timed_median(torch, mb.stream, args.steps, lambda j: mb.attention(base + j))
    q_ms = timed_median(torch, mb.stream, args.steps, lambda j: mb.append(base + j))
    byts, flops, kv = mb.work()
    t_hbm = byts / (HBM_PEAK_GBPS * 1e9)
    t_mfma = flops / (MFMA_F16_PEAK_TFLOPS * 1e12)
    if t_mfma >= t_hbm:
        ach = flops / (a_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / MFMA_F16_PEAK_TFLOPS, 4)}
    else:
        ach = byts / (a_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBPS, 4)}
    roof.update({"traffic": traffic_from_profiles(args.config, "multitoken"), "kernel": "multitoken",
                 "bytes_per_launch": byts, "flops_per_launch": flops,
                 "avg_launch_us": round(a_ms * 1e3, 2)})
    nq = int(mb.q.shape[0])
    res = {
        "metric": "multi-token attention over the 4-bit cache: query tokens per second",
        "value": round(nq / (a_ms * 1e-3), 1),
        "unit": "query tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("e2m1 codes; fp8 x fp4 scaled MFMA (QK), bf16 MFMA (PV), f32 softmax" if c.fmt == 1
                  else "u4 codes; f16 MFMA, f32 softmax"),
        "data": "synthetic (seeded; shapes of the pages' agentic workloads)",
        "config": {"workload": f"{c.name}: batch {c.batch}, {mb.m} query tokens per sequence, "
                               f"{c.num_q_heads}/{c.num_kv_heads} heads, head_dim {c.head_dim}, "
                               f"context up to {mb.max_ctx}, format {['TQ4/4', 'MX-FP4', 'TQ4/2'][c.fmt]}",
                   "pool_copies": mb.copies},
        "attention_us": round(a_ms * 1e3, 2),
        "append_us": round(q_ms * 1e3, 2),
        "effective_kv_GBps": round(kv / (a_ms * 1e-3) / 1e9, 1),
        # the attention kernel's matrix-unit use (committed counters)
        "attention_mfma_busy": (mfma_busy_from_profiles(args.config, "tq::tq4_mt_direct_kernel")
                                or mfma_busy_from_profiles(args.config, "tq::tq4_multitoken_kernel")
                                or mfma_busy_from_profiles(args.config, "tq::mxfp4_mt_kernel")),
        "roofline": roof,
        "kernel_source_hash": kernel_source_hash(),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = mt_cpu_baseline(mb)
    print(json.dumps(res))


def mt_cpu_baseline(mb, budget_s=10.0):
    """The oracle on a bounded sample: sequence 0's cache (one kv-head) built
    by the oracle, then its query rows of that kv-head until ~budget_s."""
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:
        threadpool_limits = None
    import workloads
    from oracle import attention, paged
    c, w = mb.cfg, mb.w
    g = c.num_q_heads // c.num_kv_heads
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    if ctx:
        ctx.__enter__()
    try:
        T = int(mb.ctx_np[0])
        k, v = w.sequence_kv(0)
        pool = paged.PagedPool(c.fmt, w.num_blocks, 1, c.head_dim)
        pool.append(workloads.bf16_bits_to_f32(k[:T, :1]), workloads.bf16_bits_to_f32(v[:T, :1]), w.slots(0, 0, T))
        q = workloads.bf16_bits_to_f32(mb.q.view(torch_int16()).cpu().numpy().view(np.uint16))
        t0 = time.perf_counter()
        n = 0
        m0 = int(mb.q_start_np[1])
        for i in range(m0):
            attention.multi_token(pool, q[:, :g], mb.q_start_np, w.block_table, mb.ctx_np, c.scale,
                                  rows=[(i, h) for h in range(g)])
            n += g
            if time.perf_counter() - t0 >= budget_s:
                break
        dt = time.perf_counter() - t0
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    return {"value": n / g / dt, "unit": "query tokens/s (one kv-head's g heads each)", "cores": 1, "kind": "oracle",
            "sample": f"{c.name}: sequence 0, kv-head 0: {n} query rows ({n // g} tokens x {g} heads) over a "
                      f"{T}-token context, {dt:.2f} s (numpy fp64, BLAS limited to 1 thread)"}


def torch_int16():
    import torch
    return torch.int16


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path "
              "(the decode shards by sequence or kv-head with no exchange).", file=sys.stderr)
        sys.exit(2)
    if args.ceilings:
        ceilings()
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.config == "calib":
        bench_calib(args)
        return
    if args.config in ("verify", "prefill", "verify_fp4", "prefill_fp4"):
        bench_multitoken(args)
        return
    import workloads
    cascade = args.config in ("cascade", "cascade_fp4")
    cfg_name = "agentic" if cascade else args.config
    import dataclasses
    if args.config == "tq4v2":
        cfg = dataclasses.replace(workloads.CONFIGS["llama8b"], name="tq4v2", fmt=2)
    elif args.config in ("agentic_fp4", "cascade_fp4"):
        # the agentic workload over an MX-FP4 cache
        cfg = dataclasses.replace(workloads.CONFIGS["agentic"], name="agentic_fp4", fmt=1)
    else:
        cfg = workloads.CONFIGS[cfg_name]
    # the CPU oracle first: its worker processes are forked before any GPU use
    cpu = None if args.no_cpu_baseline else cpu_baseline(cfg)
    import torch
    torch.cuda.set_device(0)
    bench = Bench(cfg, args.copies, cascade=cascade, group_blocks=args.cascade_group_blocks,
                  group_members=args.cascade_group_members)
    c = bench.cfg
    stream = bench.stream
    for i in range(args.warmup + bench.pool_copies):
        bench.step(i)
    torch.cuda.synchronize()

    # 1. the whole path: K steps between two events
    base = args.warmup + bench.pool_copies
    step_ms = timed(torch, stream, args.steps, lambda j: bench.step(base + j))
    # 2. each kernel alone, back to back over the rotating copies (the decode
    #    launch includes its split merge)
    q_ms = timed_median(torch, stream, args.steps, lambda j: bench.quantize(base + j))
    nd = args.steps * c.decode_steps
    d_ms = timed_median(torch, stream, nd, lambda j: bench.decode(j, j % c.decode_steps))
    # cascade: the per-sequence decode of the same pools, for comparison
    p_ms = (timed_median(torch, stream, nd, lambda j: bench.decode(j, j % c.decode_steps, plain=True))
            if cascade else None)
    # the single-token appends of the decode steps (one token per sequence), alone
    a_ms = (timed_median(torch, stream, nd, lambda j: bench.append(j, j % c.decode_steps)) if bench.appends else None)

    kv_logical = sum(bench.decode_bytes(s)[0] for s in range(c.decode_steps)) / c.decode_steps
    kv_unique = sum(bench.decode_bytes(s, unique=True)[0] for s in range(c.decode_steps)) / c.decode_steps
    dec_alg = sum(bench.decode_bytes(s, unique=True)[1] for s in range(c.decode_steps)) / c.decode_steps
    decode_gbps = kv_logical / (d_ms * 1e-3) / 1e9
    q_alg = bench.quantize_bytes()
    quant_gbps = q_alg / (q_ms * 1e-3) / 1e9
    kernels = {
        "quantize": {"avg_us": q_ms * 1e3, "bytes": q_alg, "GBps": quant_gbps},
        "decode": {"avg_us": d_ms * 1e3, "bytes": dec_alg, "GBps": dec_alg / (d_ms * 1e-3) / 1e9},
    }
    dominant = "quantize" if q_ms >= d_ms * c.decode_steps else "decode"

    def roof(name):
        k = kernels[name]
        return {"bound": "hbm", "achieved": round(k["GBps"], 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(k["GBps"] / HBM_PEAK_GBPS, 4),
                "traffic": traffic_from_profiles(args.config, name),
                "kernel": name, "bytes_per_launch": k["bytes"], "avg_launch_us": round(k["avg_us"], 2)}

    res = {
        "metric": "4-bit KV decode attn: effective KV GB/s & % HBM peak; quantize tokens/s",
        "value": round(decode_gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("e2m1 codes; fp8 x fp4 scaled MFMA (QK), bf16 MFMA (PV), f32 softmax" if c.fmt == 1
                  else "u4 codes; f16 MFMA, f32 softmax"),
        "data": "synthetic (seeded; shapes of the pages' agentic workloads)",
        "config": {"workload": f"{c.name}: batch {c.batch}, {c.num_q_heads}/{c.num_kv_heads} heads, "
                               f"head_dim {c.head_dim}, context {int(bench.w.context_lens_at(0).max())}, "
                               f"format {['TQ4/4', 'MX-FP4', 'TQ4/2'][c.fmt]}"
                               + (f", cascade decode over {bench.cascade.num_groups} nested groups of shared blocks"
                                  if cascade else ""),
                   "tokens_quantized_per_step": bench.n_tokens, "decode_steps_per_step": c.decode_steps,
                   "input_copies": bench.in_copies, "pool_copies": bench.pool_copies},
        "decode_hbm_frac": round(kv_unique / (d_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "decode_us": round(d_ms * 1e3, 2),
        "quantize_us": round(q_ms * 1e3, 2),
        "quantize_tokens_per_s": round(bench.n_tokens / (q_ms * 1e-3), 1),
        "roofline": roof(dominant),
        "roofline_other": roof("decode" if dominant == "quantize" else "quantize"),
        "kernel_source_hash": kernel_source_hash(),
    }
    if p_ms is not None:
        # the per-sequence decode over the same cache (every sharer reads the
        # shared blocks itself)
        res["plain_decode_us"] = round(p_ms * 1e3, 2)
        res["plain_value"] = round(kv_logical / (p_ms * 1e-3) / 1e9, 1)
    if c.fmt == 1:
        # the FP4 decode's matrix-unit use (committed counters)
        res["decode_mfma_busy"] = mfma_busy_from_profiles(args.config, "tq::mxfp4_decode_kernel")
    if a_ms is not None:
        res["append_1tok_us"] = round(a_ms * 1e3, 2)
        res["append_1tok_GBps"] = round(bench.append_bytes() / (a_ms * 1e-3) / 1e9, 1)
    if not args.no_ceilings and os.path.exists(os.path.join(ROOT, "bit_quantized_kv_amd", "libtqprobe.so")):
        # this GPU's measured ceilings for the two kernels' access patterns,
        # taken after the timed regions, and where the kernels stand against them
        try:
            ceil = measure_ceilings()
            q_rate = bench.quantize_bytes() / (q_ms * 1e-3) / 1e9
            d_rate = kv_unique / (d_ms * 1e-3) / 1e9
            ceil["quantize_frac_of_mixed_scattered"] = round(q_rate / ceil["mixed_7r2w_scattered_GBps"], 4)
            ceil["decode_unique_frac_of_record_gather"] = round(d_rate / ceil["record_gather_GBps"], 4)
            res["ceilings"] = ceil
        except Exception as e:  # the probes are context, not the measurement
            res["ceilings"] = {"error": str(e)[:200]}
    if cpu is not None:
        res["cpu_baseline"] = cpu
        if "near_ties" in cpu:
            res["near_ties"] = cpu["near_ties"]
    print(json.dumps(res))


if __name__ == "__main__":
    main()
