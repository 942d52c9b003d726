#!/usr/bin/env python3
"""Benchmark of one block-sparse decode step on one MI355X.

Workload: 8 requests x 1 query token, 4 KV heads x 16 query heads, head_dim 128,
32768 cached tokens each + 1 appended token, NVFP4 KV in shuffled P128 pages, index
keys E4M3, top-16 blocks. A step is the whole path: append -> index score -> select
-> sparse decode -> combine.

Timing. All inputs are resident in HBM before timing. The pool is replicated R times
and step i uses replica i % R; R is chosen so that at least 512 MiB of other data
(about 64 x 9 MB of decode reads at the default workload) pass between two uses of a
replica even by one kernel alone, which evicts the 256 MB Infinity Cache and the L2s.
Steps are captured in HIP graphs: one of the R replicas in turn, one of the W warm-up
steps and one of exactly the K timed steps. Before timing, the timed graph and the
replica cycle each run once (whatever W is), then the W warm-up steps, ordered so
that every replica's last use lies R - 1 steps before its next one; then the timed
graph runs once between two events (behind a short GPU spin, so that the host's
submission of the graph does not fall inside the timed region).

Per-kernel durations are measured live with HIP events on the step's stream: each
kernel is captured R times in a graph of its own (once per replica), and at least 8
replays of that graph are timed, so the mean includes the dispatch gap between
back-to-back launches. (The fused scorer's figure is the step time minus the decode
kernel's mean: launched alone back to back it shows gaps between launches that the
step does not have.) The roofline entry uses the decode kernel's mean duration and its
algorithmic bytes (selected visible K/V bytes + Q + O + selection/block-table reads).
HBM traffic comes from rocprofv3 FETCH_SIZE / WRITE_SIZE counters recorded in
profiles/ and is reported only while the kernel source is unchanged since then. Each
duration also carries p10 / p50 / p90 over the replays (each a mean over R launches).

Read references measured in the same run: `read_floor`, a plain kernel that reads the
step's own selected K/V bytes (each selected block of each KV head once, through the
page list, in the same replica rotation), and `box_read_gbs`, a streaming read of
1 GiB. The decode's time is stated as a fraction of both.

The CPU baseline is the float64 oracle on a bounded sample of the same workload, timed
with numpy's BLAS at one thread (`cpu_baseline`) and at up to 16 (`cpu_baseline_all_cores`).
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

HBM_PEAK_GBS = 8000.0
WORKLOAD_CFG = 1
MIN_REUSE_BYTES = 512 << 20     # other data moved between two uses of a replica
MIN_REPLAYS = 8                 # replays behind every percentile


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--num-splits", type=int, default=0, help="0 = library default for k and the number of (row, KV head) pairs")
    ap.add_argument("--replicas", type=int, default=0,
                    help="pool replicas (0: enough for 512 MiB between reuses, within a 48 GiB budget)")
    ap.add_argument("--replays", type=int, default=MIN_REPLAYS,
                    help=f"replays of each per-kernel graph for the durations (at least {MIN_REPLAYS})")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--config", type=int, default=WORKLOAD_CFG, choices=[0, 1, 2, 3, 4],
                    help="workload (1, the default, is the one the metric is quoted on)")
    ap.add_argument("--index-fmt", choices=["e4m3", "nvfp4"], default="e4m3",
                    help="index-key format (the workload specifies e4m3; nvfp4 is the option)")
    ap.add_argument("--select-in", choices=["decode", "score"], default="decode",
                    help="fused step: select inside the decode launch (default) or at the end of "
                         "the scoring launch")
    ap.add_argument("--per-kv-head", action="store_true",
                    help="one selection per (row, KV head), each from its share of the index heads")
    ap.add_argument("--launches", type=int, choices=[1, 2], default=2,
                    help="fused step: 1 = the whole step in one msa_decode_step launch (where its shape "
                         "allows), 2 = append + score, then select + decode + combine")
    ap.add_argument("--separate", action="store_true",
                    help="five launches per step (one per stage) instead of the two fused ones")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="oracle time budget, for each of the two thread counts")
    ap.add_argument("--no-read-probe", action="store_true",
                    help="skip the 1 GiB streaming-read reference measurement")
    ap.add_argument("--no-pairing", action="store_true",
                    help="skip the query-pairing comparison (workloads with several rows per request)")
    ap.add_argument("--counters-pass", action="store_true",
                    help="rocprofv3 --pmc runs: only the replica cycle and the timed steps (then the "
                         "calibration copy); pool replicas for 64 MiB between reuses unless --replicas")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after timing, run one device copy of this size (counter calibration)")
    return ap.parse_args()


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for f in ("sparse_decode.hip", "decode_device.h", "msa_device.h", "select_device.h"):
        with open(os.path.join(ROOT, "sparse_attention_decode_fp8_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stream_read_gbs(torch, dev, gib=1, launches=10):
    """Read bandwidth the part sustains: a plain streaming-read kernel (libmsaprobe) over
    a 1 GiB buffer, median of `launches` timed launches after one warm-up launch."""
    import ctypes

    import numpy as np
    lib = ctypes.CDLL(os.path.join(ROOT, "sparse_attention_decode_fp8_amd", "libmsaprobe.so"))
    lib.msa_probe_stream_read.restype = ctypes.c_int
    lib.msa_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                          ctypes.c_int32, ctypes.c_void_p]
    nbytes = gib << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    buf.fill_(3)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    wgs = nbytes // (16 * 4 * 256)   # one pass: four 16-byte loads per lane (the fastest grid)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(launches + 1)]
    assert lib.msa_probe_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), wgs, stream) == 0
    ev[0].record()
    for i in range(launches):
        assert lib.msa_probe_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), wgs, stream) == 0
        ev[i + 1].record()
    torch.cuda.synchronize()
    t = np.median([ev[i].elapsed_time(ev[i + 1]) * 1e-3 for i in range(launches)])
    del buf
    return nbytes / t / 1e9


def decode_algorithmic_bytes(wl, sel, bytes_per_token):
    """Selected visible tokens (union over a request's rows) x KV heads x bytes per
    token, + Q and O (bf16), + selection table and block-table entries read. With
    per-KV-head tables (sel [rows][H_kv][k]) each KV head counts its own union."""
    import numpy as np
    tables = sel.shape[1] if sel.ndim == 3 else 1
    tok_heads = 0
    for t in range(tables):
        st = sel[:, t] if sel.ndim == 3 else sel
        for s in range(len(wl.ctx_lens)):
            rows = np.nonzero(wl.row_seq == s)[0]
            vis = set()
            for r in rows:
                for b in st[r]:
                    if b >= 0:
                        hi = min(128 * (int(b) + 1), int(wl.row_pos[r]) + 1)
                        vis.update(range(128 * int(b), hi))
            tok_heads += len(vis)
    tok = tok_heads // tables if tables > 1 else tok_heads
    kv = tok_heads * (wl.num_kv_heads // tables) * bytes_per_token
    qo = 2 * wl.num_rows * wl.num_heads * 128 * 2
    meta = sel.size * 4 + int((sel >= 0).sum()) * 4
    return kv + qo + meta, tok


def selected_units(wl, sel):
    """The step's selected K/V as read units (physical page, KV head, visible tokens):
    each selected block of each KV head once per request, with the most tokens any of
    the request's rows sees in it (the union decode_algorithmic_bytes counts)."""
    import numpy as np
    tables = sel.shape[1] if sel.ndim == 3 else 1
    units = []
    for s in range(len(wl.ctx_lens)):
        rows = np.nonzero(wl.row_seq == s)[0]
        for g in range(wl.num_kv_heads):
            st = sel[:, g] if tables > 1 else sel
            vis = {}
            for r in rows:
                for b in st[r]:
                    if b >= 0:
                        n = min(128, int(wl.row_pos[r]) - 128 * int(b) + 1)
                        vis[int(b)] = max(vis.get(int(b), 0), n)
            units += [(int(wl.block_table[s][b]), g, n) for b, n in sorted(vis.items()) if n > 0]
    return np.asarray(units, dtype=np.int32).reshape(-1, 3)


def auto_replicas(wl, pool_bytes, budget=48 << 30, reuse=MIN_REUSE_BYTES):
    """Pool replicas so that at least `reuse` bytes of decode reads alone pass between
    two uses of a replica (the decode moves the fewest bytes of the step's kernels):
    1 + reuse / (bytes of k selected blocks per row and KV head), a multiple of 8, at
    most 512 and within `budget` bytes of device memory."""
    bpt = 144 if wl.fmt == 2 else 256
    est = sum(min(int(p) // 128 + 1, wl.k) * 128 for p in wl.row_pos) * wl.num_kv_heads * bpt
    r = 1 + -(-reuse // max(est, 1))
    r = -(-r // 8) * 8
    return int(max(8, min(r, 512, budget // max(pool_bytes, 1))))


def page_read_probe(torch, pools, units, stream):
    """Launcher of the read-floor probe (libmsaprobe msa_probe_page_read) on one pool."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "sparse_attention_decode_fp8_amd", "libmsaprobe.so"))
    f = lib.msa_probe_page_read
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32] + [ctypes.c_void_p] * 4 + \
        [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    dev_units = torch.from_numpy(units).to(pools[0].k_codes.device)
    sink = torch.zeros(1, dtype=torch.int32, device=dev_units.device)

    def launch(p):
        st = f(dev_units.data_ptr(), len(units), p.fmt, p.k_codes.data_ptr(), p.v_codes.data_ptr(),
               p.k_scales.data_ptr(), p.v_scales.data_ptr(), p.num_kv_heads, sink.data_ptr(),
               torch.cuda.current_stream().cuda_stream)
        assert st == 0, f"msa_probe_page_read returned {st}"
    launch.keep = (dev_units, sink)
    return launch


def calibration_copy(torch, dev, mib):
    """One device copy of `mib` MiB (a kernel of known traffic for the counter scale)."""
    if not mib:
        return
    a = torch.empty(mib << 20, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the decode path has no multi-GPU part in this library)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import sparse_attention_decode_fp8_amd as M
    from sparse_attention_decode_fp8_amd.pipeline import FUSED_APPEND_MAX, default_num_splits
    from synth import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    wl = W.config(args.config, index_fmt=W.IDX_NVFP4 if args.index_fmt == "nvfp4" else W.IDX_E4M3)
    ns = args.num_splits or default_num_splits(wl.k, wl.num_rows * wl.num_kv_heads)
    print(f"[bench] workload {wl.name} generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    def bf16(bits):
        a = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16)).view(np.int16)
        return torch.from_numpy(a).to(dev).view(torch.bfloat16)

    pool0 = M.KVPool(wl.fmt, wl.num_pages, wl.num_kv_heads, k_tensor_scale=wl.k_tensor_scale,
                     v_tensor_scale=wl.v_tensor_scale, k_page_scale=wl.k_page_scale,
                     v_page_scale=wl.v_page_scale, index_fmt=wl.index_fmt,
                     index_tensor_scale=wl.index_tensor_scale)
    for s in range(len(wl.ctx_lens)):
        L = int(wl.ctx_lens[s])
        M.msa_kv_append(pool0, torch.from_numpy(wl.slots(s, np.arange(L))).to(dev),
                        bf16(wl.k_src[s][:L]), bf16(wl.v_src[s][:L]), bf16(wl.idx_src[s][:L]))
    torch.cuda.synchronize()
    pool_bytes = sum(a.numel() * a.element_size() for a in pool0.arrays().values())
    R = args.replicas or auto_replicas(wl, pool_bytes, reuse=(64 << 20) if args.counters_pass else MIN_REUSE_BYTES)
    pools = [pool0] + [pool0.clone() for _ in range(R - 1)]
    tables = wl.num_kv_heads if args.per_kv_head else 1
    step = M.Step(wl.block_table, wl.row_seq, wl.row_pos, sel_tables=tables)
    q, q_idx = bf16(wl.q), bf16(wl.q_idx)
    w = torch.from_numpy(wl.w).to(dev)
    sl, kb, vb, ib = wl.step_tokens()
    slot, k_new, v_new, idx_new = torch.from_numpy(sl).to(dev), bf16(kb), bf16(vb), bf16(ib)
    bufs = M.DecodeBuffers(wl.num_rows, wl.num_heads, wl.max_blocks, wl.k, ns, sel_tables=tables)
    print(f"[bench] {R} pool replicas ready, splits {ns}", file=sys.stderr, flush=True)

    select_in = args.select_in

    def step_call(p, stream=None):
        """The single launch (msa_decode_step); False if the shape is outside it."""
        return M.msa_decode_step(p, step, q_idx, w, q, wl.k, wl.n_init, wl.n_local, wl.softmax_scale, ns,
                                 bufs.score_x, bufs.score_words, bufs.merge_o, bufs.merge_ml, bufs.counters,
                                 bufs.out, block_scores=bufs.block_scores, sel=bufs.sel, sel_pages=bufs.sel_pages,
                                 slot=slot, k_new=k_new, v_new=v_new, idx_k_new=idx_new, stream=stream,
                                 unsupported_ok=True)

    single = (args.launches == 1 and not args.separate and select_in == "decode" and tables == 1
              and step_call(pools[0]))
    if args.launches == 1 and not single:
        print("[bench] the single launch does not cover this shape: two launches", file=sys.stderr, flush=True)
    # run_step appends in a launch of its own when a step has this many new tokens
    app_sep = not args.separate and not single and select_in == "decode" and len(sl) > FUSED_APPEND_MAX

    def one_step(p, stream=None):
        M.run_step(p, step, bufs, q, q_idx, w, wl.softmax_scale, slot=slot, k_new=k_new,
                   v_new=v_new, idx_k_new=idx_new, n_init=wl.n_init, n_local=wl.n_local,
                   fused=not args.separate, stream=stream, select_in=select_in, single_launch=single)

    # ---- capture: the replica cycle, the warm-up steps and exactly the K timed steps.
    # Warm-up step i uses replica (R - W + i) % R, so that it ends right before replica
    # 0 and every replica's last use before the timed graph lies R - 1 steps back.
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for p in pools:
            one_step(p)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    def capture(seq):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in seq:
                one_step(pools[i])
        return g

    g_cycle = capture(range(R))
    g_warm = capture([(R - args.warmup + i) % R for i in range(args.warmup)]) if args.warmup else None
    g_timed = capture([i % R for i in range(args.steps)])
    torch.cuda.synchronize()

    g_timed.replay()           # every graph runs once before timing, whatever --warmup is
    g_cycle.replay()
    if g_warm is not None:
        g_warm.replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # A short spin on the GPU in front of the start event (untimed) keeps the GPU busy
    # while the host submits the timed graph, so no submission gap lands in the timed
    # region (at small K it would otherwise add its ~15 us to every step's mean).
    torch.cuda._sleep(1 << 20)
    ev0.record()
    g_timed.replay()
    ev1.record()
    torch.cuda.synchronize()
    ms_total = ev0.elapsed_time(ev1)
    ms_per_step = ms_total / args.steps
    print(f"[bench] timed {args.steps} steps: {ms_per_step * 1e3:.2f} us/step", file=sys.stderr, flush=True)
    if args.counters_pass:
        calibration_copy(torch, dev, args.calib_copy_mib)
        print(json.dumps({"counters_pass": wl.name, "replicas": R, "num_splits": ns, "steps": args.steps,
                          "us_per_step": ms_per_step * 1e3}), flush=True)
        return
    reps = max(MIN_REPLAYS, args.replays)

    def time_replays(g, per_replay):
        """Mean duration of one of the `per_replay` launches (or steps) a graph holds,
        over `reps` back-to-back replays after one untimed replay, and p10 / p50 / p90
        of the per-replay means."""
        g.replay()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        torch.cuda._sleep(1 << 20)   # (as for the timed steps: no submission gap inside)
        ev[0].record()
        for i in range(reps):
            g.replay()
            ev[i + 1].record()
        torch.cuda.synchronize()
        per = np.array([ev[i].elapsed_time(ev[i + 1]) * 1e3 / per_replay for i in range(reps)])
        return {"mean": ev[0].elapsed_time(ev[reps]) * 1e3 / (reps * per_replay),
                "p10": float(np.percentile(per, 10)), "p50": float(np.percentile(per, 50)),
                "p90": float(np.percentile(per, 90)), "launches": reps * per_replay}

    step_us = time_replays(g_cycle, R)   # the spread of the step time over replays

    # ---- per-kernel durations: events around each launch, queued behind a GPU sleep
    if args.separate:
        names = ["msa_kv_append", "msa_index_score", "msa_select_topk", "msa_sparse_decode", "msa_combine"]
        calls = [
            lambda p: M.msa_kv_append(p, slot, k_new, v_new, idx_new),
            lambda p: M.msa_index_score(p, step, q_idx, w, bufs.block_scores),
            lambda p: M.msa_select_topk(step, bufs.block_scores, wl.k, wl.n_init, wl.n_local, bufs.sel,
                                        bufs.sel_pages),
            lambda p: M.msa_sparse_decode(p, step, q, bufs.sel, wl.k, wl.softmax_scale, ns, bufs.part_o,
                                          bufs.part_ml, sel_pages=bufs.sel_pages),
            lambda p: M.msa_combine(wl.num_rows, wl.num_heads, 128, ns, bufs.part_o, bufs.part_ml, bufs.out),
        ]
        decode_kernels = ["msa_sparse_decode", "msa_combine"]
    elif single:
        names = ["msa_decode_step"]
        calls = [lambda p: step_call(p)]
        decode_kernels = ["msa_decode_step"]
    elif select_in == "decode":
        names = ["msa_append_score_select", "msa_select_decode_combine"]
        calls = [
            lambda p: M.msa_append_score_select(p, step, q_idx, w, wl.k, wl.n_init, wl.n_local,
                                                bufs.block_scores, slot=slot, k_new=k_new,
                                                v_new=v_new, idx_k_new=idx_new),
            lambda p: M.msa_select_decode_combine(p, step, q, bufs.block_scores, wl.k, wl.n_init,
                                                  wl.n_local, wl.softmax_scale, ns, bufs.merge_o,
                                                  bufs.merge_ml, bufs.counters, bufs.out,
                                                  sel=bufs.sel, sel_pages=bufs.sel_pages),
        ]
        decode_kernels = ["msa_select_decode_combine"]
        if app_sep:   # (as run_step does for this many new tokens)
            names = ["msa_kv_append", "msa_index_score"] + names[1:]
            calls = [lambda p: M.msa_kv_append(p, slot, k_new, v_new, idx_new),
                     lambda p: M.msa_index_score(p, step, q_idx, w, bufs.block_scores)] + calls[1:]
    else:
        names = ["msa_append_score_select", "msa_sparse_decode_combine"]
        calls = [
            lambda p: M.msa_append_score_select(p, step, q_idx, w, wl.k, wl.n_init, wl.n_local,
                                                bufs.block_scores, sel=bufs.sel, sel_pages=bufs.sel_pages,
                                                counters=bufs.score_counters, slot=slot, k_new=k_new,
                                                v_new=v_new, idx_k_new=idx_new),
            lambda p: M.msa_sparse_decode_combine(p, step, q, bufs.sel, wl.k, wl.softmax_scale, ns,
                                                  bufs.merge_o, bufs.merge_ml, bufs.counters, bufs.out,
                                                  sel_pages=bufs.sel_pages),
        ]
        decode_kernels = ["msa_sparse_decode_combine"]
    # One graph per kernel that launches it once on every pool replica (inputs as the step
    # leaves them); events around replays of it give the mean launch duration, the
    # dispatch gap between back-to-back launches included.
    kgraphs = []
    for call in calls:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for p in pools:
                call(p)
        kgraphs.append(g)
    torch.cuda.synchronize()
    per_kernel_us = {nm: time_replays(g, R) for nm, g in zip(names, kgraphs)}

    # The table-driven decode entry alone (msa_sparse_decode on the selection the fused
    # step wrote; partials only), timed the same way: the kernel the decode target names.
    sd_us = None
    if not args.separate:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for p in pools:
                M.msa_sparse_decode(p, step, q, bufs.sel, wl.k, wl.softmax_scale, ns, bufs.part_o,
                                    bufs.part_ml, sel_pages=bufs.sel_pages)
        sd = time_replays(g, R)
        sd_us = sd["mean"]

    sel = bufs.sel.cpu().numpy()
    bpt = 144 if wl.fmt == W.FMT_NVFP4 else 256
    dec_bytes, dec_tokens = decode_algorithmic_bytes(wl, sel, bpt)

    # Query pairing (several verify rows per request): the rows of a request decoded
    # together over the union of their tables (msa_sparse_decode_union, one split, bf16
    # out) against the one-row decode with the same output (msa_sparse_decode_combine, one
    # split), on the step's selection and on full-overlap tables (every row of a request
    # takes its first row's table: the most sharing the rows can have).
    pairing = None
    if wl.rows_per_req > 1 and tables == 1 and not args.no_pairing:
        groups = torch.from_numpy(M.group_rows_of(wl.row_seq, 4)).to(dev)
        first = {}
        for r in range(wl.num_rows):
            first.setdefault(int(wl.row_seq[r]), r)
        sel_full = np.stack([sel[first[int(x)]] for x in wl.row_seq]).astype(np.int32)
        pair_out = torch.empty_like(bufs.out)
        ws = M.DecodeBuffers(wl.num_rows, wl.num_heads, wl.max_blocks, wl.k, 1)
        pairing = {"group_rows": 4, "num_splits": 1}
        for tag, tab in (("step_selection", sel), ("full_overlap", sel_full)):
            tab_d = torch.from_numpy(np.ascontiguousarray(tab, dtype=np.int32)).to(dev)
            ub, _ = decode_algorithmic_bytes(wl, tab, bpt)
            per_row = sum(min(int(wl.row_pos[r]) - 128 * int(b) + 1, 128) for r in range(wl.num_rows)
                          for b in tab[r] if b >= 0) * wl.num_kv_heads * bpt
            res = {"union_bytes": ub, "per_row_bytes": per_row}
            for nm, call in (
                    ("msa_sparse_decode_union", lambda p: M.msa_sparse_decode_union(
                        p, step, q, tab_d, wl.k, groups, 4, wl.softmax_scale, 1, out=pair_out)),
                    ("msa_sparse_decode_combine", lambda p: M.msa_sparse_decode_combine(
                        p, step, q, tab_d, wl.k, wl.softmax_scale, 1, ws.merge_o, ws.merge_ml, ws.counters,
                        pair_out))):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for p in pools:
                        call(p)
                t = time_replays(g, R)
                res[nm] = {"mean_us": t["mean"], "p50_us": t["p50"],
                           "union_gbs": ub / (t["mean"] * 1e-6) / 1e9}
            pairing[tag] = res

    # The read floor: the same selected K/V bytes read by a plain kernel through the page
    # list, one launch per replica in the same rotation, timed like the kernels above.
    units = selected_units(wl, sel)
    probe = page_read_probe(torch, pools, units, None)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for p in pools:
            probe(p)
    floor = time_replays(g, R)
    floor_bytes = int(units[:, 2].sum()) * bpt + (8 * len(units) if wl.fmt == W.FMT_FP8 else 0)
    key_bytes = 64 if wl.index_fmt == W.IDX_E4M3 else 32 + 4        # per token: codes (+ scales)
    # every visible index key once per request (its rows are scored together)
    last = {}
    for r in range(wl.num_rows):
        last[int(wl.row_seq[r])] = max(last.get(int(wl.row_seq[r]), -1), int(wl.row_pos[r]))
    idx_bytes = int(sum(p + 1 for p in last.values()) * key_bytes)
    t_dec = sum(per_kernel_us[k]["mean"] for k in decode_kernels) * 1e-6
    if single:
        t_idx = None   # (the scoring runs inside the one launch)
        idx_method = None
    elif args.separate or app_sep:
        t_idx = per_kernel_us["msa_index_score"]["mean"] * 1e-6
        idx_method = "events around replays of a graph of this kernel alone"
    else:
        # Back-to-back launches of the scorer alone leave gaps between them that the
        # step does not have; within the step it takes what the decode leaves of it.
        t_idx = ms_per_step * 1e-3 - per_kernel_us[decode_kernels[0]]["mean"] * 1e-6
        idx_method = "step time minus the decode kernel's mean"
    # The single launch is the whole step: its algorithmic bytes are the index keys' and
    # the decode's together.
    roof_bytes = dec_bytes + (idx_bytes if single else 0)
    achieved = roof_bytes / t_dec / 1e9

    traffic = None
    # HBM bytes per launch of the decode kernel from the committed rocprofv3 counter
    # digest of this workload, if it was taken from the current kernel sources
    prof = os.path.join(ROOT, "profiles", f"{decode_kernels[0]}_{wl.name}.counters.json")
    if os.path.exists(prof):
        with open(prof) as fh:
            pc = json.load(fh)
        if (pc.get("source_digest") == kernel_source_digest() and pc.get("num_splits") == ns
                and pc.get("workload") == wl.name and tables == 1 and not args.separate
                and select_in == "decode"):
            traffic = pc.get("hbm_bytes_per_launch")

    box_read = None if args.no_read_probe else stream_read_gbs(torch, dev)

    calibration_copy(torch, dev, args.calib_copy_mib)

    cpu = cpu_all = None
    if not args.no_cpu_baseline:
        cpu, cpu_all = cpu_baseline(wl, args.cpu_seconds, [1, min(16, len(os.sched_getaffinity(0)))], tables)

    rows = wl.num_rows
    line = {
        "metric": "sparse-decode query tokens/s + achieved HBM GB/s (% of peak), B=8 ctx 32k",
        "value": rows / (ms_per_step * 1e-3),
        "unit": "q-tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4/e4m3 storage, fp16 MFMA operands, fp32 accumulate, bf16 out",
        "data": "synthetic (seeded N(0,1) K/V/Q, shuffled page table)",
        "config": {"workload": wl.name, "batch": len(wl.ctx_lens), "query_rows": rows,
                   "kv_heads": wl.num_kv_heads,
                   "index_keys": args.index_fmt,
                   "q_heads": wl.num_heads, "head_dim": 128, "cached_tokens": int(wl.ctx_lens[0]) if len(set(wl.ctx_lens.tolist())) == 1 else
                   f"{int(wl.ctx_lens.min())}..{int(wl.ctx_lens.max())} (mean {float(wl.ctx_lens.mean()):.0f})",
                   "appended_tokens": wl.n_append, "top_k": wl.k, "kv_format": "nvfp4" if wl.fmt == W.FMT_NVFP4 else "fp8",
                   "num_splits": ns, "selection": "per KV head" if tables > 1 else "per query row",
                   "select_in": "separate launch" if args.separate else select_in,
                   "launches": "separate" if args.separate else 1 if single else 2,
                   "pool_replicas": R, "reuse_distance_decode_bytes": (R - 1) * dec_bytes,
                   "parallelism": "single GPU"},
        "step_us": step_us,
        "roofline": {"kernel": "+".join(decode_kernels), "bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "algorithmic_bytes": roof_bytes,
                     "visible_selected_tokens": dec_tokens, "mean_us": t_dec * 1e6,
                     **({f"{q}_us": per_kernel_us[decode_kernels[0]][q] for q in ("p10", "p50", "p90")}
                        if len(decode_kernels) == 1 else {}),
                     "frac_of_box_read": None if box_read is None else achieved / box_read,
                     "frac_of_read_floor": None if single else floor["mean"] / (t_dec * 1e6)},
        "index_score_roofline": None if single else {"kernel": "msa_index_score" if args.separate or app_sep else names[0],
                                 "bound": "hbm", "achieved": idx_bytes / t_idx / 1e9,
                                 "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                 "frac": idx_bytes / t_idx / 1e9 / HBM_PEAK_GBS,
                                 "algorithmic_bytes": idx_bytes, "mean_us": t_idx * 1e6,
                                 "method": idx_method},
        "sparse_decode_roofline": None if sd_us is None else {
            "kernel": "msa_sparse_decode", "bound": "hbm", "achieved": dec_bytes / (sd_us * 1e-6) / 1e9,
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": dec_bytes / (sd_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "algorithmic_bytes": dec_bytes, "mean_us": sd_us,
            "p10_us": sd["p10"], "p50_us": sd["p50"], "p90_us": sd["p90"],
            "frac_of_box_read": None if box_read is None else dec_bytes / (sd_us * 1e-6) / 1e9 / box_read,
            "frac_of_read_floor": floor["mean"] / sd_us,
            "method": "the table-driven entry alone on the step's selection (partials, no merge)"},
        "read_floor": {"kernel": "msa_probe_page_read", "bytes": floor_bytes, "units": int(len(units)),
                       "mean_us": floor["mean"], "p10_us": floor["p10"], "p50_us": floor["p50"],
                       "p90_us": floor["p90"], "gbs": floor_bytes / (floor["mean"] * 1e-6) / 1e9,
                       "frac_of_peak": floor_bytes / (floor["mean"] * 1e-6) / 1e9 / HBM_PEAK_GBS,
                       "method": "the step's selected K/V bytes (each selected block of each KV head "
                                 "once, its visible tokens) read cold through the page list by a plain "
                                 "kernel, one workgroup per block, one launch per replica in the step's "
                                 "rotation; frac_of_read_floor = its mean time / the decode's"},
        "query_pairing": pairing,
        "box_read_gbs": box_read,
        "kernel_us": per_kernel_us,
        "cpu_baseline": cpu,
        "cpu_baseline_all_cores": cpu_all,
    }
    print(json.dumps(line), flush=True)


def cpu_model() -> str:
    """The host CPU as /proc/cpuinfo names it (model name, family / model / stepping,
    max MHz from lscpu's source where present) and the logical CPUs this process may use."""
    info = {}
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ":" in ln:
                    k, v = ln.split(":", 1)
                    info.setdefault(k.strip(), v.strip())
    except OSError:
        pass
    name = info.get("model name", "unknown")
    fam = f"family {info.get('cpu family', '?')} model {info.get('model', '?')} stepping {info.get('stepping', '?')}"
    usable = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return f"{name} ({fam}; {os.cpu_count()} logical CPUs, {usable} usable by this process)"


def cpu_baseline(wl, budget_s, thread_counts, tables=1):
    """The float64 oracle, unchanged, timed on host cores for a bounded sample of the
    same workload: whole steps (append, index score, select, attention) of the 8
    requests, round robin, until the time budget is spent; once per entry of
    thread_counts, with numpy's BLAS limited to that many threads."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import msa_oracle as O

    cases = []
    with threadpool_limits(1):
        for s in range(len(wl.ctx_lens)):
            rows = np.nonzero(wl.row_seq == s)[0]
            L = int(wl.ctx_lens[s])
            pool = O.new_pool(wl.fmt, wl.num_pages, wl.num_kv_heads, k_tensor_scale=wl.k_tensor_scale,
                              v_tensor_scale=wl.v_tensor_scale, index_fmt=wl.index_fmt,
                              index_tensor_scale=wl.index_tensor_scale)
            O.kv_append(pool, wl.slots(s, np.arange(L)), None, None, wl.idx_src[s][:L])
            sl, kb, vb, ib = wl.prefill_slices(s, np.arange(L, L + wl.n_append))
            args = (wl.block_table, wl.row_seq[rows], wl.row_pos[rows], sl, kb, vb, ib,
                    wl.q_idx[rows], wl.w[rows], wl.q[rows], wl.k, wl.softmax_scale, wl.max_blocks)
            # untimed: learn which pages the step attends and give the pool their K/V
            S = O.index_score(pool, *args[:3], args[7], args[8], wl.max_blocks, tables)
            sel = O.select_topk(S, args[2], wl.k, wl.n_init, wl.n_local)
            pos = np.concatenate([np.arange(128 * b, min(128 * (b + 1), L)) for b in sel.ravel() if b >= 0])
            pos = np.unique(pos[pos < L])
            O.kv_append(pool, wl.slots(s, pos), wl.k_src[s][pos], wl.v_src[s][pos], None)
            cases.append((pool, args, len(rows)))
    out = []
    for threads in thread_counts:
        with threadpool_limits(threads):
            done, steps, t_total = 0, 0, 0.0
            while t_total < budget_s:
                pool, args, nrows = cases[steps % len(cases)]
                t = time.perf_counter()
                O.decode_step(pool, *args, tables=tables)
                t_total += time.perf_counter() - t
                done += nrows
                steps += 1
        out.append({"value": done / t_total, "unit": "q-tok/s", "cores": threads, "kind": "oracle",
                    "cpu": cpu_model(),
                    "sample": f"{steps} oracle steps of single requests of the same workload, round robin "
                              f"(each: append {wl.n_append} token(s), index score over the request's "
                              f"tokens, top-{wl.k} select, attention over the selected pages for "
                              f"{wl.num_heads} heads), {done} query rows in {t_total:.1f} s, "
                              f"numpy/BLAS limited to {threads} thread(s)"})
    return out


if __name__ == "__main__":
    main()
