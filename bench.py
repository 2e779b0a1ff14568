"""Benchmark of the paged-KV attention hot path on one MI355X.

A step is one pass of the whole path over the mixed continuous-batching
workload (4 chunked-prefill sequences of 512 new tokens at offsets up to 8192,
200 decode sequences with contexts of 1024..32768 tokens, 50 of them sharing a
4096-token prefix, 32/8 heads, head_dim 128, block 256, bf16):

    kv_store of all 2248 new tokens -> causal paged prefill -> split-K decode (+ reduce)

on one stream, inputs resident in HBM.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload 5] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


def _pin_blas_threads() -> int:
    """BLAS / OpenMP threads of the oracle = the cores this process may run on (or a
    smaller cap the environment already sets), fixed before numpy is first imported."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ.setdefault(var, str(n))
    return n


BLAS_THREADS = _pin_blas_threads()


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 matrix peak, TFLOP/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_split_traffic.md")


# What the decode split pass is built and launched from: its kernel sources whole,
# the argument struct, and the host functions that size its grid and workspace.
DECODE_FILES = ("common.hpp", "row_attn.hip", "row_attn.hpp")
DECODE_PARTS = (("kernels.hpp", "struct RowAttnArgs {"), ("api.cpp", "int32_t auto_split("),
                ("api.cpp", "int64_t state_bytes("), ("api.cpp", "int prepare_decode("))


def _block(text: str, start: str) -> str:
    """The text from the line holding `start` to the first line that closes it at column 0."""
    i = text.index(start)
    i = text.rindex("\n", 0, i) + 1
    j = text.index("\n}", i)
    return text[i:text.index("\n", j + 1) + 1]


def kernel_source_hash() -> str:
    """sha256 over what defines the decode split pass (file names and bytes, in order)."""
    import hashlib

    h = hashlib.sha256()
    d = os.path.join(ROOT, "paged_kv_gqa_mapping_amd", "csrc")
    for name in DECODE_FILES:
        h.update(name.encode())
        h.update(open(os.path.join(d, name), "rb").read())
    for name, start in DECODE_PARTS:
        h.update(f"{name}:{start}".encode())
        h.update(_block(open(os.path.join(d, name)).read(), start).encode())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per decode-split launch from the committed counter summary, or None when
    the kernel sources changed since the counters were taken (or no summary exists)."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    fields = dict(line.strip("- `").split(": ", 1) for line in text.splitlines()
                  if line.startswith("- `") and ": " in line)
    try:
        if fields.get("kernel_source_sha256", "").strip("`") != kernel_source_hash():
            return None
        return int(fields["hbm_bytes_per_launch"].strip("`"))
    except (KeyError, ValueError):
        return None


def calibrate_copy(mib: int) -> None:
    """A plain device-to-device copy of a known size, for scaling FETCH_SIZE / WRITE_SIZE."""
    import torch

    n = mib << 20
    x = torch.empty(n, dtype=torch.uint8, device="cuda")
    x.fill_(3)
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes": n, "launches": 3}), flush=True)


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def cpu_baseline(w, decode_budget_s: float = 12.0, prefill_budget_s: float = 6.0):
    """The fp64 oracle, as it stands, timed on the host on bounded samples of the same
    workload, with the GPU figures' algorithmic numerators:

    * kv_store: the whole step's new tokens (the oracle returns new caches, so its time
      includes copying the pool; GB/s over the store's algorithmic bytes);
    * decode (the metric): whole sequences in order until the budget is spent, KV GB/s;
    * prefill: query rows of the chunks, the longest sequence first, until the budget is
      spent, TFLOP/s over 4 * Hq * D per (query, key) pair.

    Returns the cpu_baseline record (value = decode GB/s) and the caches after the store."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle

    t0 = time.perf_counter()
    kc, vc = oracle.kv_store(w.k_cache, w.v_cache, w.new_k, w.new_v, w.slot_mapping, w.block_size)
    t_store = time.perf_counter() - t0

    t0 = time.perf_counter()
    done_bytes = 0
    n = 0
    row = 2 * w.num_kv_heads * w.head_dim * w.elt_bytes
    while n < len(w.dec_context_lens) and time.perf_counter() - t0 < decode_budget_s:
        oracle.decode(w.dec_q[n:n + 1], kc, vc, w.dec_block_tables[n:n + 1], w.dec_context_lens[n:n + 1], w.scale,
                      w.dtype, w.block_size)
        done_bytes += int(w.dec_context_lens[n]) * row
        n += 1
    t_dec = time.perf_counter() - t0

    pre = None
    if w.pre_q is not None:
        lq = np.diff(w.cu_seqlens_q)
        lk = np.diff(w.cu_seqlens_k)
        s = int(np.argmax(lk))
        q0, Lq, Lk = int(w.cu_seqlens_q[s]), int(lq[s]), int(lk[s])
        t0 = time.perf_counter()
        pairs = rows = 0
        for i in range(Lq - 1, -1, -1):
            if time.perf_counter() - t0 >= prefill_budget_s:
                break
            p = Lk - Lq + i
            oracle.prefill(w.pre_q[q0 + i:q0 + i + 1], kc, vc, np.array([0, 1], np.int32),
                           np.array([0, p + 1], np.int32), w.pre_block_tables[s:s + 1], w.scale, w.dtype,
                           w.block_size)
            pairs += p + 1
            rows += 1
        t_pre = time.perf_counter() - t0
        pre = {"TFLOP/s": round(4 * w.num_q_heads * w.head_dim * pairs / t_pre / 1e12, 6), "rows": rows,
               "seconds": round(t_pre, 2)}
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    rec = {
        "value": round(done_bytes / t_dec / 1e9, 4),
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "cpu": cpu_model(),
        "sample": f"fp64 numpy oracle on the host: decode of the first {n} of {len(w.dec_context_lens)} decode "
                  f"sequences ({done_bytes / 1e9:.3f} GB of K/V, {t_dec:.1f} s; value, same algorithmic bytes per "
                  f"token as the GPU figure)"
                  + (f"; prefill of {pre['rows']} query rows of the longest chunk ({pre['seconds']} s)" if pre else "")
                  + f"; kv_store of all {len(w.slot_mapping)} new tokens ({t_store:.1f} s, includes copying the pool)",
        "kv_store_GB/s": round(w.store_bytes() / t_store / 1e9, 6),
        "decode_GB/s": round(done_bytes / t_dec / 1e9, 4),
    }
    if pre:
        rec["prefill_TFLOP/s"] = pre["TFLOP/s"]
    return rec


def measure_rope_kv_store(w, torch, pkv, dev, pq, dq, nk, nv, kc, vc, slots, bf, iters=20):
    """Fused rotary embedding + cache write over the step's new tokens (chunk
    tokens, then decode tokens, at their own positions), timed on its own after
    the step: a 512 MiB read between launches evicts the inputs from the caches."""
    q = torch.cat([pq, dq], dim=0).contiguous()
    pos = dev(w.store_positions)
    N, Hq, D = q.shape
    elt = 2 if bf else 4
    algo = 2 * N * (Hq + 2 * w.num_kv_heads) * D * elt + 8 * N
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    ts = []
    for i in range(iters + 2):
        flush.sum()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        pkv.rope_kv_store(q, nk, nv, pos, kc, vc, slots, 1e6, False)
        b.record()
        torch.cuda.synchronize()
        if i >= 2:
            ts.append(a.elapsed_time(b))
    ms = sum(ts) / len(ts)
    gbs = algo / (ms * 1e-3) / 1e9
    return {"ms": round(ms, 5), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
            "tokens": int(N), "algorithmic_bytes": int(algo), "rope_theta": 1e6,
            "note": "next-row kernel, timed separately after the step (not part of value)"}


def measure_cascade(w, torch, cascade_decode, out, plain_ms, iters=20):
    """Shared-prefix decode of the step's decode batch (group pass, split pass and
    merge), timed on its own after the step, against the step's plain decode."""
    for _ in range(3):
        cascade_decode(out)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for a, b in ev:
        a.record()
        cascade_decode(out)
        b.record()
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in ev) / iters
    logical, unique = w.decode_kv_bytes(), w.decode_kv_bytes_unique()
    return {"ms": round(ms, 5), "plain_decode_ms": round(plain_ms, 5),
            "logical_GB/s": round(logical / (ms * 1e-3) / 1e9, 1),
            "unique_GB/s": round(unique / (ms * 1e-3) / 1e9, 1),
            "frac_hbm_unique": round(unique / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "unique_kv_gb": round(unique / 1e9, 4),
            "note": "next-row path (group pass + split pass + merge), timed separately after the step"}


def report(iters: int = 7) -> None:
    """Per-workload figures (workloads 1-5): median kernel times after a 1 GiB read that evicts
    the caches, throughput against the roofline, max-abs error of sampled outputs against the
    oracle, the stored rows bit for bit, and the oracle's own speed on those samples.  One JSON
    line per workload."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info

    import oracle
    import paged_kv_gqa_mapping_amd as pkv
    import workloads as W

    torch.cuda.set_device(0)
    pkv.lib()
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])

    def dev(a, bf):
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16) if bf else \
            torch.from_numpy(np.ascontiguousarray(a))
        return t.cuda()

    def timed(fn):
        fn()
        ts = []
        for _ in range(iters):
            flush.sum()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts))

    for i in range(1, 6):
        w = W.make_config(i)
        bf = w.dtype == W.BF16
        kc, vc = dev(w.k_cache, bf), dev(w.v_cache, bf)
        nk, nv, slots = dev(w.new_k, bf), dev(w.new_v, bf), dev(w.slot_mapping, False)
        rec = {"workload": w.name, "dtype": w.dtype}
        t_store = timed(lambda: pkv.kv_store(nk, nv, kc, vc, slots))
        rec["kv_store_us"] = round(t_store * 1e3, 2)
        rec["kv_store_GB/s"] = round(w.store_bytes() / (t_store * 1e-3) / 1e9, 1)
        # the stored rows, bit for bit
        hkv, d = w.num_kv_heads, w.head_dim
        rows = kc.view(-1, hkv, d)[slots.long()]
        rec["kv_store_bitwise"] = bool(torch.equal(rows.view(torch.int16) if bf else rows.view(torch.int32),
                                                   nk.view(torch.int16) if bf else nk.view(torch.int32)))
        # host caches after the store (in place: the workload is not used again)
        for cache, new in ((w.k_cache, w.new_k), (w.v_cache, w.new_v)):
            cache.reshape(-1, hkv, d)[w.slot_mapping] = new
        if w.dec_q is not None:
            dq, dbt, dcl = dev(w.dec_q, bf), dev(w.dec_block_tables, False), dev(w.dec_context_lens, False)
            out = torch.empty_like(dq)
            B, Hq, _ = dq.shape
            split = pkv.decode_split_tokens(B, Hq, hkv, d, w.max_context_len, w.block_size, 1 if bf else 0)
            ws = torch.empty(max(pkv.decode_workspace_bytes(B, Hq, d, w.max_context_len, split), 16),
                             dtype=torch.uint8, device="cuda")
            t_dec = timed(lambda: pkv.paged_decode_attn(dq, kc, vc, dbt, dcl, w.scale, out,
                                                        max_context_len=w.max_context_len, split_tokens=split,
                                                        workspace=ws))
            byts = w.decode_kv_bytes() + w.decode_io_bytes()
            rec["decode_us"] = round(t_dec * 1e3, 2)
            rec["decode_GB/s"] = round(byts / (t_dec * 1e-3) / 1e9, 1)
            rec["decode_frac_hbm"] = round(byts / (t_dec * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
            rec["split_tokens"] = int(split)
            lens = w.dec_context_lens
            pick = sorted(set(int(x) for x in np.linspace(0, len(lens) - 1, 6).round()) |
                          {int(np.argmax(lens)), int(np.argmin(lens))})
            got = out.cpu().view(torch.int16).numpy().view(np.uint16) if bf else out.cpu().numpy()
            t0 = time.perf_counter()
            ref = oracle.decode(w.dec_q[pick], w.k_cache, w.v_cache, w.dec_block_tables[pick], lens[pick], w.scale,
                                w.dtype, w.block_size)
            t_or = time.perf_counter() - t0
            rec["decode_max_abs_err"] = float(np.max(np.abs(W.to_float32(got[pick], w.dtype) - ref)))
            rec["decode_rows_checked"] = len(pick)
            sample_bytes = int(lens[pick].astype(np.int64).sum()) * 2 * hkv * d * w.elt_bytes
            rec["oracle_decode_GB/s"] = round(sample_bytes / t_or / 1e9, 4)
        if w.pre_q is not None:
            pq = dev(w.pre_q, bf)
            pbt, cuq, cuk = dev(w.pre_block_tables, False), dev(w.cu_seqlens_q, False), dev(w.cu_seqlens_k, False)
            pout = torch.empty_like(pq)
            # the library's default prefill path (the one-launch kernel), as in the timed step
            t_pre = timed(lambda: pkv.paged_prefill_attn(pq, kc, vc, cuq, cuk, pbt, pout, max_seqlen_q=w.max_seqlen_q,
                                                         max_seqlen_k=w.max_seqlen_k, scale=w.scale))
            fl = w.prefill_flops()
            rec["prefill_us"] = round(t_pre * 1e3, 2)
            rec["prefill_TFLOP/s"] = round(fl / (t_pre * 1e-3) / 1e12, 1)
            rec["prefill_frac_mfma"] = round(fl / (t_pre * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS, 4)
            got = pout.cpu().view(torch.int16).numpy().view(np.uint16)
            worst, n_rows, t_or, pairs = 0.0, 0, 0.0, 0
            for sq in range(len(w.cu_seqlens_q) - 1):
                q0, q1 = int(w.cu_seqlens_q[sq]), int(w.cu_seqlens_q[sq + 1])
                lk = int(w.cu_seqlens_k[sq + 1] - w.cu_seqlens_k[sq])
                for r in sorted({0, (q1 - q0) // 2, q1 - q0 - 1}):
                    p_ = lk - (q1 - q0) + r
                    t0 = time.perf_counter()
                    ref = oracle.decode(w.pre_q[q0 + r:q0 + r + 1], w.k_cache, w.v_cache,
                                        w.pre_block_tables[sq:sq + 1], np.array([p_ + 1], np.int32), w.scale,
                                        w.dtype, w.block_size)
                    t_or += time.perf_counter() - t0
                    pairs += p_ + 1
                    worst = max(worst, float(np.max(np.abs(W.to_float32(got[q0 + r], w.dtype) - ref[0]))))
                    n_rows += 1
            rec["prefill_max_abs_err"] = worst
            rec["prefill_rows_checked"] = n_rows
            rec["oracle_prefill_TFLOP/s"] = round(4 * w.num_q_heads * d * pairs / t_or / 1e12, 6)
        rec["oracle_cores"] = int(threads)
        print(json.dumps(rec), flush=True)
        del kc, vc
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=5, help="workload number (5 = the mixed step)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flush", action="store_true",
                    help="no cache-evicting read between timed steps (ms_per_step is then still the step events' mean)")
    ap.add_argument("--split-tokens", type=int, default=0)
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the separately timed next-row measurements (fused rope + kv_store, cascade decode)")
    ap.add_argument("--fused-store", action="store_true",
                    help="write the decode tokens' K/V inside the decode launch (kv_store then covers prefill tokens only)")
    ap.add_argument("--cascade", action="store_true",
                    help="decode with shared-prefix (cascade) decode inside the step instead of plain split-K decode")
    ap.add_argument("--overlap-prefill", action="store_true",
                    help="run prefill on a second stream concurrently with decode (after kv_store); the decode "
                         "kernel then shares the GPU, so its event time is not the kernel's own")
    ap.add_argument("--prefill-planned", action="store_true",
                    help="prefill through a workspace: the device-side plan (query tiles with long key ranges cut "
                         "into pieces) run as one workgroup per planned item, instead of the one-launch kernel")
    ap.add_argument("--graph", action="store_true",
                    help="capture the step in a HIP graph and time graph replays (per-kernel events are not recorded)")
    ap.add_argument("--report", action="store_true",
                    help="per-workload figures of workloads 1-5 (one JSON line each) instead of the step benchmark")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain copy of MIB MiB (counter calibration) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import paged_kv_gqa_mapping_amd as pkv
    import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.report:
        report()
        return
    pkv.lib()  # fail loudly if the library is missing

    t_build = time.perf_counter()
    w = W.make_config(args.workload)
    log(f"built workload {w.name} on the host in {time.perf_counter() - t_build:.1f} s")

    def dev(a, bf=False):
        if a is None:
            return None
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16) if bf else torch.from_numpy(
            np.ascontiguousarray(a))
        return t.cuda()

    bf = w.dtype == W.BF16
    kc, vc = dev(w.k_cache, bf), dev(w.v_cache, bf)
    nk, nv, slots = dev(w.new_k, bf), dev(w.new_v, bf), dev(w.slot_mapping)
    has_dec, has_pre = w.dec_q is not None, w.pre_q is not None
    if has_dec:
        dq, dbt, dcl = dev(w.dec_q, bf), dev(w.dec_block_tables), dev(w.dec_context_lens)
        dout = torch.empty_like(dq)
        B, Hq, D = dq.shape
        split = args.split_tokens or pkv.decode_split_tokens(B, Hq, w.num_kv_heads, D, w.max_context_len,
                                                             w.block_size, 1 if bf else 0)
        ws_bytes = pkv.decode_workspace_bytes(B, Hq, D, w.max_context_len, split)
        ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
        shared, goff, gseq, gmax, smax, gown = w.cascade_groups()
        has_groups = len(goff) > 1
        if has_groups:
            csh, cgo, cgs = dev(shared), dev(goff), dev(gseq)
            cws = torch.empty(max(pkv.cascade_workspace_bytes(B, Hq, w.num_kv_heads, D, w.max_context_len, gown, 0,
                                                              len(goff) - 1, gmax, smax), 16),
                              dtype=torch.uint8, device="cuda")
            cout = torch.empty_like(dq)
        if args.cascade and not has_groups:
            print("--cascade needs a workload with shared prefixes", file=sys.stderr)
            sys.exit(2)

        def cascade_decode(o):
            pkv.cascade_decode_attn(dq, kc, vc, dbt, dcl, csh, cgo, cgs, w.scale, o, max_context_len=w.max_context_len,
                                    max_group_size=gmax, max_shared_len=smax, max_own_len=gown, workspace=cws)
    if has_pre:
        pq, pbt, cuq, cuk = dev(w.pre_q, bf), dev(w.pre_block_tables), dev(w.cu_seqlens_q), dev(w.cu_seqlens_k)
        pout = torch.empty_like(pq)
        pws = None
        if args.prefill_planned:
            need = pkv.prefill_workspace_bytes(int(len(w.cu_seqlens_q) - 1), w.max_seqlen_q, w.num_q_heads,
                                               w.num_kv_heads, w.head_dim, 1 if bf else 0)
            pws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")

        def prefill():
            pkv.paged_prefill_attn(pq, kc, vc, cuq, cuk, pbt, pout, max_seqlen_q=w.max_seqlen_q,
                                   max_seqlen_k=w.max_seqlen_k, scale=w.scale, workspace=pws,
                                   planned=args.prefill_planned)
    torch.cuda.synchronize()
    log("inputs resident on the GPU")

    n_pre_tok = int(w.cu_seqlens_q[-1]) if has_pre else 0  # the chunk tokens come first in slot_mapping
    if args.fused_store and (not has_dec or args.cascade):
        print("--fused-store needs decode sequences and plain decode", file=sys.stderr)
        sys.exit(2)
    n_ev = 8
    overlap = args.overlap_prefill and has_pre and has_dec
    s_pre = torch.cuda.Stream() if overlap else None

    def step(events=None):
        def rec(i):
            if events is not None:
                events[i].record()
        rec(0)
        if not args.fused_store:
            pkv.kv_store(nk, nv, kc, vc, slots)
        elif n_pre_tok:
            pkv.kv_store(nk[:n_pre_tok], nv[:n_pre_tok], kc, vc, slots[:n_pre_tok])
        rec(1)
        if overlap:
            # prefill on its own stream after kv_store, decode meanwhile on the current stream
            s_pre.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s_pre):
                rec(5)
                prefill()
                rec(6)
        elif has_pre:
            prefill()
        rec(2)
        if has_dec and args.cascade:
            cascade_decode(dout)
            rec(3)
        elif has_dec and args.fused_store:
            pkv.paged_decode_store_attn(dq, nk[n_pre_tok:], nv[n_pre_tok:], kc, vc, dbt, dcl, w.scale, dout,
                                        max_context_len=w.max_context_len, split_tokens=split, workspace=ws)
            rec(3)
        elif has_dec:
            pkv.paged_decode_split(dq, kc, vc, dbt, dcl, w.scale, dout, max_context_len=w.max_context_len,
                                   split_tokens=split, workspace=ws)
            rec(3)
            pkv.paged_decode_reduce(dq, kc, vc, dbt, dcl, w.scale, dout, max_context_len=w.max_context_len,
                                    split_tokens=split, workspace=ws)
        else:
            rec(3)
        rec(4)
        if overlap:
            torch.cuda.current_stream().wait_stream(s_pre)
        rec(7)  # end of the step (after prefill too, when it ran on its own stream)

    if args.graph:
        # capture once (after a warm-up on the capture stream), then time replays
        cs = torch.cuda.Stream()
        cs.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cs):
            step()
        torch.cuda.current_stream().wait_stream(cs)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / args.steps
        print(json.dumps({"workload": w.name, "graph_ms_per_step": round(ms, 5), "steps": args.steps}), flush=True)
        return
    # between timed steps a 512 MiB read (twice the last-level cache) evicts what the
    # previous step left in the caches; it is outside the step's events, so
    # ms_per_step is the mean event time of the steps themselves
    flush = None if args.no_flush else torch.empty(512 << 20, dtype=torch.uint8, device="cuda")

    def evict():
        if flush is not None:
            flush.view(torch.int32).sum()

    for _ in range(args.warmup):
        evict()
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        evict()
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = float(np.mean([e[0].elapsed_time(e[7]) for e in evs]))

    def avg(i, j):
        return float(np.mean([e[i].elapsed_time(e[j]) for e in evs]))  # ms

    t_store, t_pre, t_split, t_red = avg(0, 1), avg(5, 6) if overlap else avg(1, 2), avg(2, 3), avg(3, 4)
    kv_bytes = w.decode_kv_bytes()
    dec_io = w.decode_io_bytes()
    flops = w.prefill_flops()
    stored_tokens = n_pre_tok if args.fused_store else int(len(w.slot_mapping))
    store_bytes = w.store_bytes() * stored_tokens // max(len(w.slot_mapping), 1)
    # with --cascade the timed decode is the whole shared-prefix call, which reads the unique bytes
    split_bytes = (w.decode_kv_bytes_unique() if args.cascade else kv_bytes) + dec_io
    achieved_gbs = split_bytes / (t_split * 1e-3) / 1e9 if has_dec else 0.0

    kernels = {
        "kv_store": {"ms": round(t_store, 5), "GB/s": round(store_bytes / (t_store * 1e-3) / 1e9, 1) if t_store else None,
                     "tokens": stored_tokens},
        "decode_split": {"ms": round(t_split, 5), "GB/s": round(achieved_gbs, 1),
                         "frac_hbm": round(achieved_gbs / HBM_PEAK_GBS, 4),
                         "split_tokens": (None if args.cascade else int(split)) if has_dec else 0},
        "decode_reduce": {"ms": round(t_red, 5)},
    }
    if has_pre:
        tfs = flops / (t_pre * 1e-3) / 1e12
        kernels["prefill"] = {"ms": round(t_pre, 5), "TFLOP/s": round(tfs, 2),
                              "frac_mfma": round(tfs / MFMA_BF16_PEAK_TFS, 4), "tflop": round(flops / 1e12, 5)}
    if has_dec:
        value = kv_bytes / (ms_per_step * 1e-3) / 1e9
        traffic = measured_traffic() if args.workload == 5 and not args.split_tokens and not args.cascade else None
        roofline = {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                    "kernel": ("shared-prefix decode call (group pass + split pass + merge)" if args.cascade
                               else "row_attn_kernel (decode split pass)"),
                    "algorithmic_bytes_per_launch": int(split_bytes)}
    else:
        value = flops / (ms_per_step * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(kernels["prefill"]["TFLOP/s"], 2), "peak": MFMA_BF16_PEAK_TFS,
                    "unit": "TFLOP/s", "frac": kernels["prefill"]["frac_mfma"], "traffic": None,
                    "kernel": "prefill_mfma_kernel"}

    if has_dec and has_groups and not args.cascade and not args.no_extras:
        kernels["cascade_decode"] = measure_cascade(w, torch, cascade_decode, cout, t_split + t_red)
    if has_dec and has_pre and not args.no_extras:
        kernels["rope_kv_store"] = measure_rope_kv_store(w, torch, pkv, dev, pq, dq, nk, nv, kc, vc, slots, bf)

    cpu = None
    if not args.no_cpu_baseline and has_dec:
        log("timing the oracle on a bounded sample")
        cpu = cpu_baseline(w)

    out = {
        "metric": "paged decode attn KV GB/s & % HBM peak; prefill attn TFLOP/s & % MFMA peak",
        "value": round(value, 2),
        "unit": "GB/s" if has_dec else "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "wall_ms_per_step_incl_eviction": round(wall * 1e3 / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf else "f32",
        "data": "synthetic (seeded N(0,1) values, seeded lengths and block tables)",
        "config": {
            "workload": w.name,
            "decode_seqs": int(len(w.dec_context_lens)) if has_dec else 0,
            "prefill_seqs": int(len(w.cu_seqlens_q) - 1) if has_pre else 0,
            "new_tokens": int(len(w.slot_mapping)),
            "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
            "block_size": w.block_size, "num_blocks": w.num_blocks,
            "value_definition": "decode algorithmic K/V bytes (logical, each sequence's context read once per KV "
                                "head) per step time (HIP events from the step's first kernel to its last)" if has_dec else "prefill flops per step time",
            "decode_kv_gb": round(kv_bytes / 1e9, 4),
            "parallelism": "single-gpu",
            "prefill_overlapped_with_decode": bool(overlap),
        },
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
