#!/usr/bin/env python3
"""Paged decode attention benchmark on one MI355X.

A step is one decode step of one layer over the whole batch, every kernel of
the path on the GPU with all inputs resident in HBM: paged_decode_append_attn,
i.e. the new token of every sequence written to its slot (found through its
block table) and attention over the cache that holds it -- for 16-bit pools one
persistent attention kernel that also stores the token, then the log-sum-exp
merge; for 8-bit pools the quantising append kernel first.
Default workload: the Llama-3-8B-shaped layer (64 sequences, lengths U{512..8192},
32 q / 8 KV heads, head_dim 128, bf16 KV, shuffled 16-token blocks).

Printed: one JSON line.  `value` is KV bytes read per step / step time (GB/s);
`roofline` describes the attention kernel (its algorithmic KV bytes per launch
over its own average duration, timed with HIP events on its stream);
`cpu_baseline` is the fp64 CPU oracle timed on the host's cores over a bounded
sample of the same workload.

    python bench.py [--steps 50] [--warmup 5] [--workload llama3] [--no-cpu-baseline]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attn: KV GB/s read (% of HBM peak) and decode tokens/s, 1 GPU"
HBM_PEAK_GBS = 8000.0
_CSRC = "paged_kv_cache_283_amd/csrc/"
_COMMON = ("device_common.hpp", "geometry.hpp", "launch.hpp", "../build.py")
# Sources each operation's kernels are built from: a profile summary carries the hash of its set,
# so a summary taken before a kernel change is recognisably stale.
OP_SOURCES = {
    "decode": ("decode_attn.hip", "mfma_ops.hpp", "kv_codec.hpp", "fp8_e4m3.hpp"),
    "prefill": ("prefill_attn.hip", "mfma_ops.hpp"),
    "evict": ("keep_select.hip", "kv_compact.hip", "decode_attn.hip", "mfma_ops.hpp", "kv_codec.hpp", "fp8_e4m3.hpp"),
    "fill": ("kv_write.hip", "kv_codec.hpp", "fp8_e4m3.hpp"),
    "swap": ("kv_swap.hip",),
}
KERNEL_SOURCES = tuple(_CSRC + f for f in OP_SOURCES["decode"] + _COMMON)
WORKLOAD_NAMES = {"llama3": "llama3-8b-layer-decode", "fp8long": "fp8-kv-32k-shared-prefix",
                  "int8long": "int8-kv-32k", "fp8chlong": "fp8-per-channel-kv-32k",
                  "streaming": "streamingllm-131k-sinks4-window4096", "h2o": "h2o-8k-mass",
                  "llama2": "llama2-70b-80-layer-decode", "tiny": "tiny-paged-decode"}


def kernel_hash(op: str = "decode") -> str:
    """sha256 prefix of the sources (and build flags) the operation's kernels are built from."""
    h = hashlib.sha256()
    for f in OP_SOURCES[op] + _COMMON:
        h.update(open(os.path.join(ROOT, _CSRC + f), "rb").read())
    return h.hexdigest()[:16]


def traffic_file(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"attn_wave_{workload}_traffic.txt")


def read_traffic(workload):
    """HBM traffic of the attention kernel from the committed counter summary, if it is current."""
    path = traffic_file(workload)
    if not os.path.exists(path):
        return None, None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_hash") != kernel_hash():
        return None, "kernel changed since the counters were taken"
    try:
        return float(kv["traffic_bytes_per_launch"]), kv.get("note")
    except (KeyError, ValueError):
        return None, None


ELEM_BYTES = {"f32": 4, "bf16": 2, "f16": 2, "fp8": 1, "int8": 1, "fp8_ch": 1, "int8_ch": 1}


def kv_bytes_per_token(w):
    """K + V bytes of one token, all KV heads, with per-token scales (static per-channel scales are
    read once per segment, not per token)."""
    per = w.num_kv_heads * 2 * w.head_dim * ELEM_BYTES[w.kv_dtype]
    if w.kv_dtype in ("fp8", "int8"):
        per += w.num_kv_heads * 2 * 4
    return per


def attended_tokens(w, lay):
    """Positions decode attention reads per layer: the whole context, or sinks + window."""
    n = 0
    for L in lay.lens:
        L = int(L)
        n += w.num_sinks + w.window if (w.window > 0 and L > w.num_sinks + w.window) else L
    return int(n)


def cpu_baseline(w, lay, ksrc, vsrc, q, seconds):
    """Time the fp64 oracle on host cores over the workload's sequences (cycled), bounded in time."""
    import math

    import numpy as np
    import torch

    from oracle import attention, policies
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [1])
        blas = ", ".join(f"{i.get('internal_api')} {i.get('version')}" for i in info if i.get("user_api") == "blas")
    except Exception:  # noqa: BLE001
        threads = len(os.sched_getaffinity(0))
    per_tok = kv_bytes_per_token(w)
    # host copies of the sample's source rows (not timed): the oracle decodes and attends
    sample, budget_rows = [], 600_000
    for s in range(w.num_seqs):
        L = int(lay.lens[s])
        keep = policies.streaming_keep(L, w.num_sinks, w.window)
        pos = np.nonzero(keep)[0]
        i = np.searchsorted(lay.data_pos[s], pos)
        rows = torch.from_numpy(lay.data_row[s][i]).to(ksrc.device)
        sample.append((s, keep, ksrc.index_select(0, rows).cpu(), vsrc.index_select(0, rows).cpu()))
        budget_rows -= pos.size
        if budget_rows <= 0:
            break
    qh = q.cpu()
    scale = 1.0 / math.sqrt(w.head_dim)
    done_bytes, n_seq = 0, 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for s, keep, k, v in sample:
            K = k.to(torch.float64).numpy()
            V = v.to(torch.float64).numpy()
            attention.decode_attention(qh[s].to(torch.float64).numpy(), K, V, scale)
            done_bytes += K.shape[0] * per_tok
            n_seq += 1
            if time.perf_counter() - t0 >= seconds:
                break
    dt = time.perf_counter() - t0
    return {"value": round(done_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle", "blas": blas,
            "sample": f"{n_seq} sequence-decodes of the {w.name} workload ({len(sample)} distinct sequences, "
                      f"{done_bytes / 1e9:.2f} GB of KV) in {dt:.1f} s, numpy float64, bf16->f64 decode included",
            "seconds": round(dt, 2)}


def bench_evict(args, dev, stream, read_gbs, copy_gbs):
    """Eviction step on the h2o workload: kv_keep_select (H2OEviction.select: budget 2048, recent 512)
    then kv_compact of every sequence's kept tokens into fresh blocks.  The scores come from one
    untimed decode step with the H2O mass.  Bytes: compaction reads and writes each kept token's K and
    V (all KV heads); the select reads the score rows and writes the keep lists.  Also timed: the next
    decode step applying the same keep-set itself (paged_decode_attn_compact, with the H2O mass)
    against the H2O decode step over the same cache; their difference is the eviction's cost when
    fused."""
    import dataclasses

    import numpy as np
    import torch

    import workloads as W
    from workloads import device as H
    from paged_kv_cache_283_amd import ops

    base = W.WORKLOADS["h2o"]
    per_seq = -(-base.budget // 16)
    w = dataclasses.replace(base, extra_blocks=base.num_seqs * per_seq)
    lay = W.make_layout(w)
    tables = torch.from_numpy(lay.tables).to(dev)
    lens = torch.from_numpy(lay.lens).to(dev)
    pools = H.make_pools(w, lay.num_blocks)
    ksrc, vsrc = W.kv_source(w, lay, device=dev)
    H.fill(w, lay, pools, ksrc, vsrc, tables)
    del ksrc, vsrc
    k, v, ks, vs = pools
    q = W.queries(w, device=dev)
    L = lay.max_len
    scores = torch.zeros((w.num_seqs, L), dtype=torch.float32, device=dev)
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    ops.paged_decode_attn(out, q, k, v, tables, lens, L, k_scale=ks, v_scale=vs, attn_mass=scores)
    free = np.asarray(lay.unused_blocks, dtype=np.int32)[: w.num_seqs * per_seq]
    dst = torch.from_numpy(free.reshape(w.num_seqs, per_seq).copy()).to(dev)
    keep_idx = torch.empty((w.num_seqs, w.budget), dtype=torch.int32, device=dev)
    keep_count = torch.empty(w.num_seqs, dtype=torch.int32, device=dev)
    rule = (0, w.recent, w.budget - w.recent, "rest")

    def step(ev):
        ev[0].record(stream)
        ops.keep_select(scores, lens, L, *rule, keep_idx=keep_idx, keep_count=keep_count, stream=stream)
        ev[1].record(stream)
        ops.kv_compact(k, v, tables, dst, keep_idx, keep_count, ks, vs, stream=stream)
        ev[2].record(stream)

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.warmup):
        step(evs[0])
    torch.cuda.synchronize()
    ops.probe_read(torch.empty(1 << 30, dtype=torch.uint8, device=dev), torch.zeros(1024, device=dev))
    for ev in evs:                  # enqueued behind a 1 GiB read so no launch gap enters the events
        step(ev)
    torch.cuda.synchronize()
    sel_ms = [ev[0].elapsed_time(ev[1]) for ev in evs]
    cmp_ms = [ev[1].elapsed_time(ev[2]) for ev in evs]

    # The same keep-set applied by the next decode step instead (paged_decode_attn_compact: attention
    # over the kept tokens, which it also stores into the destination blocks, and the H2O scores of the
    # kept tokens moved to their new positions with this step's mass added), against the H2O decode step
    # over the same cache (paged_decode_attn with the mass): the difference is what eviction adds.
    scores2 = torch.zeros_like(scores)
    plain = ops.paged_decode_attn(out, q, k, v, tables, lens, L, attn_mass=scores, workspace=ops.alloc_workspace(
        w.num_seqs, w.num_q_heads, w.head_dim, L, want_mass=True, device=dev), stream=stream, prepare=True)
    fused = ops.paged_decode_attn_compact(out, q, k, v, tables, lens, L, keep_idx, keep_count, dst,
                                          attn_mass_src=scores, attn_mass=scores2, stream=stream, prepare=True)
    pev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for _ in range(args.warmup):
        plain()
        fused()
    torch.cuda.synchronize()
    ops.probe_read(torch.empty(1 << 30, dtype=torch.uint8, device=dev), torch.zeros(1024, device=dev))
    for ev in pev:
        ev[0].record(stream)
        plain()
        ev[1].record(stream)
        fused()
        ev[2].record(stream)
    torch.cuda.synchronize()
    t_plain = float(np.median([ev[0].elapsed_time(ev[1]) for ev in pev]))
    t_fused = float(np.median([ev[1].elapsed_time(ev[2]) for ev in pev]))
    kept = int(keep_count.sum().item())
    tok_bytes = kv_bytes_per_token(w)
    moved = 2 * kept * tok_bytes                          # read + write of every kept token
    sel_bytes = int(lens.sum().item()) * 4 + w.num_seqs * w.budget * 4
    t_sel, t_cmp = float(np.median(sel_ms)), float(np.median(cmp_ms))
    achieved = moved / (t_cmp * 1e-3) / 1e9
    print(json.dumps({
        "metric": "eviction step: H2O keep-set + compaction into fresh blocks, GB/s moved",
        "value": round(moved / ((t_sel + t_cmp) * 1e-3) / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(t_sel + t_cmp, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.kv_dtype, "data": "synthetic",
        "config": {"workload": "h2o-8k-evict", "batch": w.num_seqs, "context": L, "budget": w.budget,
                   "recent": w.recent, "kept_tokens": kept, "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None},
        "keep_select_us": round(1e3 * t_sel, 2), "keep_select_bytes": sel_bytes,
        "compact_us": round(1e3 * t_cmp, 2), "compact_bytes": moved,
        "decode_step_us": round(1e3 * t_plain, 2), "compacting_decode_step_us": round(1e3 * t_fused, 2),
        "eviction_added_to_decode_us": round(1e3 * (t_fused - t_plain), 2),
        "probe_read_gbs": round(read_gbs, 1), "probe_copy_gbs": round(copy_gbs, 1),
        "kernel_hash": kernel_hash("evict")}), flush=True)


MFMA_PEAK_BF16_TFLOPS = 2500.0


def bench_prefill(args, dev, stream):
    """Chunked prefill on the prefill workload: 4 sequences whose last 2048 tokens (after a 6144-token
    cached prefix, 8192 batched tokens in all) attend causally over the paged cache.  Algorithmic work:
    4 * D flops per (query token, attended key, query head) -- 2 D for q.k and 2 D for p.v."""
    import numpy as np
    import torch

    import workloads as W
    from workloads import device as H
    from paged_kv_cache_283_amd import ops

    w = W.WORKLOADS["prefill"]
    lay = W.make_layout(w)
    tables = torch.from_numpy(lay.tables).to(dev)
    lens = torch.from_numpy(lay.lens).to(dev)
    pools = H.make_pools(w, lay.num_blocks)
    ksrc, vsrc = W.kv_source(w, lay, device=dev)
    H.fill(w, lay, pools, ksrc, vsrc, tables)
    del ksrc, vsrc
    k, v, ks, vs = pools
    q, start = W.chunk_queries(w, device=dev)
    qs = torch.from_numpy(start).to(dev)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    call = ops.paged_prefill_attn(out, q, k, v, tables, lens, qs, lay.max_len, w.chunk, k_scale=ks, v_scale=vs,
                                  stream=stream, prepare=True)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for ev in evs:
        ev[0].record(stream)
        call()
        ev[1].record(stream)
    torch.cuda.synchronize()
    ms = np.array([ev[0].elapsed_time(ev[1]) for ev in evs])
    pairs = 0
    for L in lay.lens:
        pre = int(L) - w.chunk
        pairs += w.chunk * pre + w.chunk * (w.chunk + 1) // 2      # keys attended by the chunk's rows
    flops = 4 * w.head_dim * w.num_q_heads * pairs
    t = float(np.median(ms))
    tflops = flops / (t * 1e-3) / 1e12
    kv_bytes = int(lay.lens.sum()) * w.num_kv_heads * 2 * w.head_dim * 2
    print(json.dumps({
        "metric": "chunked prefill over the paged cache: causal multi-query attention TFLOP/s",
        "value": round(tflops, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(t, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.kv_dtype, "data": "synthetic",
        "config": {"workload": "prefill-4x2048-after-6144", "batch": w.num_seqs, "chunk": w.chunk,
                   "context": int(lay.max_len), "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "batched_tokens": w.num_seqs * w.chunk},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_PEAK_BF16_TFLOPS, 4), "traffic": None},
        "flops_per_step": flops, "prefill_kernel_avg_us": round(1e3 * float(np.mean(ms)), 2),
        "prefill_kernel_min_us": round(1e3 * float(ms.min()), 2), "kv_bytes_in_context": kv_bytes,
        "tokens_per_s": round(w.num_seqs * w.chunk / (t * 1e-3), 1), "kernel_hash": kernel_hash("prefill")}),
          flush=True)


def bench_fill(args, dev, stream, copy_gbs):
    """Bulk cache write (a prefill's or a whole prompt's K/V): every position of the workload's layout
    in one paged_kv_write call with precomputed slots.  Algorithmic bytes per token: the source rows
    read plus the stored rows (and per-token scales) written, K and V."""
    import numpy as np
    import torch

    import workloads as W
    from workloads import device as H
    from paged_kv_cache_283_amd import ops

    w = W.WORKLOADS[args.workload]
    lay = W.make_layout(w)
    tables = torch.from_numpy(lay.tables).to(dev)
    pools = H.make_pools(w, lay.num_blocks)
    ksrc, vsrc = W.kv_source(w, lay, device=dev)
    seq, pos, rows = lay.fill_tokens()
    r = torch.from_numpy(rows).to(dev)
    k_rows, v_rows = ksrc.index_select(0, r).contiguous(), vsrc.index_select(0, r).contiguous()
    del ksrc, vsrc
    slots = ops.paged_token_slots(tables, torch.from_numpy(seq).to(dev), torch.from_numpy(pos).to(dev),
                                  lay.num_blocks)
    k, v, ks, vs = pools
    call = ops.paged_kv_write(k_rows, v_rows, k, v, slots, ks, vs, stream=stream, prepare=True)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for ev in evs:
        ev[0].record(stream)
        call()
        ev[1].record(stream)
    torch.cuda.synchronize()
    ms = np.array([ev[0].elapsed_time(ev[1]) for ev in evs])
    t = float(np.median(ms))
    n_tok = int(seq.size)
    src_eb = k_rows.element_size()
    per_tok = w.num_kv_heads * w.head_dim * 2 * src_eb + kv_bytes_per_token(w)
    gbs = n_tok * per_tok / (t * 1e-3) / 1e9
    print(json.dumps({
        "metric": "bulk paged KV write (slot mapping precomputed): GB/s of source read + cache written",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(t, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.kv_dtype, "data": "synthetic",
        "config": {"workload": f"fill-{WORKLOAD_NAMES[args.workload]}", "tokens": n_tok,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "src_dtype": w.src_dtype,
                   "kv_dtype": w.kv_dtype},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
        "bytes_per_token": per_tok, "write_kernel_avg_us": round(1e3 * float(np.mean(ms)), 2),
        "probe_copy_gbs": round(copy_gbs, 1), "frac_of_probe_copy": round(gbs / copy_gbs, 4),
        "kernel_hash": kernel_hash("fill")}), flush=True)


HOST_LINK_PEAK_GBS = 64.0   # PCIe 5.0 x16, one direction


def bench_swap(args, dev, stream):
    """Block swap over the host link: 4096 blocks of the Llama-3-8B layer shape (8 KV heads, head_dim 128,
    bf16: 64 KiB per block, 256 MiB in all) from scattered pool blocks to a pinned host arena and back."""
    import numpy as np
    import torch

    from paged_kv_cache_283_amd import ops

    n, nb, hkv, d = 4096, 8192, 8, 128
    pools = ops.allocate_pools(nb, hkv, d, torch.bfloat16, dev, fill_byte=0x3C)
    arena = ops.allocate_host_arena(n, hkv, d, torch.bfloat16)
    rng = np.random.default_rng(2838)
    blocks = rng.permutation(nb)[:n].astype(np.int32)
    pairs = torch.from_numpy(np.stack([blocks, np.arange(n, dtype=np.int32)], 1)).to(dev)
    out_call = ops.kv_swap(pools, arena, pairs, True, stream=stream, prepare=True)
    in_call = ops.kv_swap(pools, arena, pairs, False, stream=stream, prepare=True)
    for _ in range(args.warmup):
        out_call()
        in_call()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for ev in evs:
        ev[0].record(stream)
        out_call()
        ev[1].record(stream)
        in_call()
        ev[2].record(stream)
    torch.cuda.synchronize()
    t_out = float(np.median([ev[0].elapsed_time(ev[1]) for ev in evs]))
    t_in = float(np.median([ev[1].elapsed_time(ev[2]) for ev in evs]))
    nbytes = n * hkv * 16 * d * 2 * 2
    out_gbs, in_gbs = nbytes / (t_out * 1e-3) / 1e9, nbytes / (t_in * 1e-3) / 1e9
    print(json.dumps({
        "metric": "KV block swap over the host link: GB/s out (pool -> pinned host) and in",
        "value": round(2 * nbytes / ((t_out + t_in) * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(t_out + t_in, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "swap-4096-blocks-llama3-layer", "blocks": n, "bytes_each_way": nbytes},
        "roofline": {"bound": "link", "achieved": round(max(out_gbs, in_gbs), 2), "peak": HOST_LINK_PEAK_GBS,
                     "unit": "GB/s", "frac": round(max(out_gbs, in_gbs) / HOST_LINK_PEAK_GBS, 4), "traffic": None},
        "swap_out_gbs": round(out_gbs, 2), "swap_in_gbs": round(in_gbs, 2),
        "swap_out_ms": round(t_out, 4), "swap_in_ms": round(t_in, 4), "kernel_hash": kernel_hash("swap")}),
          flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama3", choices=sorted(WORKLOAD_NAMES))
    ap.add_argument("--rotate", type=int, default=2, help="disjoint pool replicas cycled so that the 256 MB "
                    "Infinity Cache cannot serve repeated steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--probe-only", action="store_true", help="run only the HBM read/copy probes")
    ap.add_argument("--contiguous-blocks", action="store_true", help="hand out physical blocks in order "
                    "instead of the shuffled placement (comparison only)")
    ap.add_argument("--op", default="decode", choices=("decode", "evict", "prefill", "swap", "fill"),
                    help="decode: the decode step (default); evict: H2O keep-set + compaction on the h2o "
                         "workload; prefill: causal multi-query attention on the prefill workload; swap: "
                         "4096 blocks to pinned host memory and back; fill: bulk cache write of --workload")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by sequence or KV head with no exchange; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import workloads as W
    from paged_kv_cache_283_amd import ops

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    # ---- HBM probes: practical read and copy ceilings on this machine
    probe_n = 4 << 30
    buf = torch.empty(probe_n, dtype=torch.uint8, device=dev)
    buf2 = torch.empty(probe_n // 4, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1024, dtype=torch.float32, device=dev)
    ops.probe_read(buf, sink)
    ops.probe_copy(buf2, buf[: probe_n // 4])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        ops.probe_read(buf, sink)
    e1.record()
    torch.cuda.synchronize()
    read_gbs = 5 * probe_n / (e0.elapsed_time(e1) * 1e-3) / 1e9
    e0.record()
    for _ in range(5):
        ops.probe_copy(buf2, buf[: probe_n // 4])
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 5 * 2 * (probe_n // 4) / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del buf, buf2
    if args.probe_only:
        print(json.dumps({"probe_read_gbs": round(read_gbs, 1), "probe_copy_gbs": round(copy_gbs, 1),
                          "copy_bytes_per_launch": 2 * (probe_n // 4)}))
        return

    if args.op == "evict":
        bench_evict(args, dev, stream, read_gbs, copy_gbs)
        return
    if args.op == "prefill":
        bench_prefill(args, dev, stream)
        return
    if args.op == "swap":
        bench_swap(args, dev, stream)
        return
    if args.op == "fill":
        bench_fill(args, dev, stream, copy_gbs)
        return

    # ---- workload: pools filled through the library's own write path (untimed prefill)
    w = W.WORKLOADS[args.workload]
    lay = W.make_layout(w, shuffle=not args.contiguous_blocks)
    tables = torch.from_numpy(lay.tables).to(dev)
    lens = torch.from_numpy(lay.lens).to(dev)
    layers = w.num_layers
    replicas = 1 if layers > 1 else max(1, args.rotate)
    from workloads import device as H   # pool construction + fill through the library's write path
    pools = []
    for layer in range(max(layers, replicas)):
        p = H.make_pools(w, lay.num_blocks)
        ksrc, vsrc = W.kv_source(w, lay, layer=layer if layers > 1 else 0, device=dev)
        H.fill(w, lay, p, ksrc, vsrc, tables, hold_last=True)
        pools.append(p)
        if layer + 1 < max(layers, replicas):
            del ksrc, vsrc
    # the new token of every sequence (this step's K/V rows) and the queries
    r = torch.from_numpy(H.newest_rows(lay)).to(dev)
    k_new, v_new = ksrc.index_select(0, r).contiguous(), vsrc.index_select(0, r).contiguous()
    q = W.queries(w, device=dev)
    out = torch.empty(q.shape, dtype=torch.bfloat16 if w.q_dtype == "bf16" else torch.float32, device=dev)
    # H2O workloads: the step also emits the per-position attention mass (accumulated into a score row)
    scores = torch.zeros((w.num_seqs, lay.max_len), dtype=torch.float32, device=dev) if w.mass else None
    ws = ops.alloc_workspace(w.num_seqs, w.num_q_heads, w.head_dim, lay.max_len, w.num_sinks, w.window,
                             w.mass, dev)
    torch.cuda.synchronize()

    launches = []
    for p in pools:
        k, v, ks, vs = p
        launches.append((
            ops.paged_decode_append_attn(out, q, k_new, v_new, k, v, tables, lens, lay.max_len, k_scale=ks,
                                         v_scale=vs, num_sinks=w.num_sinks, window=w.window, attn_mass=scores,
                                         workspace=ws, stream=stream, prepare=True),))

    def step(i):
        if layers > 1:
            for la in launches:
                for f in la:
                    f()
        else:
            for f in launches[i % replicas]:
                f()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # The attention kernel's dispatches of the first fifth of the timed steps
    # (at least 10) stamp HIP events (its own start and end); each stamped
    # dispatch costs its step a few us, so the rest run without them.
    n_attn = min(args.steps * layers, max(10, (args.steps * layers) // 5))
    ops.timing_begin(n_attn)
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    kernel_ms = ops.timing_end(n_attn)
    step_ms = t_start.elapsed_time(t_end) / args.steps

    # Per-iteration step times (an event pair around each step, in a pass of its own after the
    # back-to-back timed steps above, which give ms_per_step).
    it_evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    for i, (a, b) in enumerate(it_evs):
        a.record(stream)
        step(i)
        b.record(stream)
    torch.cuda.synchronize()
    it_ms = np.array([a.elapsed_time(b) for a, b in it_evs])

    n_tok = attended_tokens(w, lay)
    per_tok = kv_bytes_per_token(w)
    kv_bytes_layer = n_tok * per_tok
    kv_bytes_step = kv_bytes_layer * layers
    value = kv_bytes_step / (step_ms * 1e-3) / 1e9
    k_avg_ms = float(np.mean(kernel_ms))
    achieved = kv_bytes_layer / (k_avg_ms * 1e-3) / 1e9
    traffic, traffic_note = read_traffic(args.workload)
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.kv_dtype,
        "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES[args.workload], "batch": w.num_seqs, "layers": layers,
                   "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "kv_dtype": w.kv_dtype, "block_size": 16, "max_context_len": lay.max_len,
                   "attended_tokens_per_layer": n_tok, "num_sinks": w.num_sinks, "window": w.window,
                   "h2o_mass": bool(w.mass),
                   "pool_replicas_rotated": replicas,
                   "block_placement": "contiguous" if args.contiguous_blocks else "shuffled"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic},
        "tokens_per_s": round(w.num_seqs / (step_ms * 1e-3), 1),
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "kv_bytes_per_step": kv_bytes_step,
        "attn_kernel_avg_us": round(1e3 * k_avg_ms, 2),
        "attn_kernel_median_us": round(1e3 * float(np.median(kernel_ms)), 2),
        "attn_kernel_min_us": round(1e3 * float(np.min(kernel_ms)), 2),
        "attn_kernel_timed_launches": len(kernel_ms),
        "step_ms_median": round(float(np.median(it_ms)), 4),
        "step_ms_min": round(float(np.min(it_ms)), 4),
        "traffic_source": (f"profiles/attn_wave_{args.workload}_traffic.txt: rocprofv3 --pmc FETCH_SIZE and "
                           "WRITE_SIZE of this kernel build (kernel_hash matches), scaled by the copy-probe "
                           "calibration" if traffic is not None else None),
        "probe_read_gbs": round(read_gbs, 1),
        "probe_copy_gbs": round(copy_gbs, 1),
        "frac_of_probe_read": round(achieved / read_gbs, 4),
        "wall_s": round(wall, 3),
        "kernel_hash": kernel_hash(),
    }
    if traffic_note:
        result["traffic_note"] = traffic_note
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, lay, ksrc, vsrc, q, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
