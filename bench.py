"""Benchmark of the codec's hot path on one MI355X.

One step = the whole path over one batch: tq_encode_kv of every key and value
of the workload into a compressed paged cache, and one tq_decode_attend of
every sequence's query over a full cache.  Default workload: the
Llama-3.1-70B-shaped layer, 4 sequences x 131072 tokens, 8 KV heads, 64 query
heads (GQA 8), head_dim 128, bf16 K/V with outlier-channel keys, 3-bit keys
and values, 16-token pages.

Cold caches: C sets of inputs and caches rotate (C >= 2, and C - 1 sets hold
at least 1 GiB).  Step i encodes set i mod C and decodes set (i + 1) mod C,
which was encoded C - 1 steps earlier: at least 1 GiB of other traffic (four
times the 256 MB Infinity Cache) separates a cache's encode from its decode,
so the decode reads HBM.  All sets are encoded once before timing.  Inputs
are resident on the GPU before timing starts.

Printed: one JSON line (rank 0).  `value` is decode-attend GB/s of compressed
KV read (algorithmic bytes / mean decode time: split kernel + merge kernel);
encoded vectors/s and the encode GB/s are reported beside it, each with its
fraction of the 8 TB/s HBM peak.  Kernel times are HIP events on the stream
the kernels run on.  `other_workloads` repeats the step on the 1 x 32768 and
16 x 8192 decode configurations (4-bit codes).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "decode-attend GB/s of compressed KV read (% HBM peak) + encoded vectors/s"
KERNEL_SOURCES = ["kv_cache_vector_encode_amd/csrc/tq_encode.hip", "kv_cache_vector_encode_amd/csrc/tq_encode_row.h",
                  "kv_cache_vector_encode_amd/csrc/tq_decode.hip",
                  "kv_cache_vector_encode_amd/csrc/tq_decode_mfma.hip", "kv_cache_vector_encode_amd/csrc/tq_merge.hip",
                  "kv_cache_vector_encode_amd/csrc/tq_device.h", "kv_cache_vector_encode_amd/csrc/tq_internal.h"]


def kernel_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def bytes_per_vector(bits: int, in_bytes: int = 2, qjl: bool = False) -> tuple[int, int]:
    """(input bytes, compressed bytes) of one 128-d vector."""
    return 128 * in_bytes, 128 * bits // 8 + 2 + ((16 + 2) if qjl else 0)


def host_cpu() -> dict:
    """Model name and core counts of the host (lscpu's model name line)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"model": model, "logical_cpus": os.cpu_count(), "usable_cpus": usable}


def _oracle_sample(w, sample_tokens: int):
    """One timed pass of the oracle over the sample: encode of every key and
    value, then original-frame decode-attend of every query head.  Returns
    (encode seconds, decode seconds, vectors)."""
    from kv_cache_vector_encode_amd import workloads as W
    from oracle import tq_oracle as O

    c32, _ = O.codebook_fp32(128, w.bits_k)
    _, k64 = W.keys(w, 0, sample_tokens)
    _, v64 = W.values(w, 0, sample_tokens)
    x = np.concatenate([k64.reshape(-1, 128), v64.reshape(-1, 128)])
    t0 = time.perf_counter()
    encs = [O.encode(x[i:i + 32768], w.rot_seed, c32) for i in range(0, len(x), 32768)]
    t_enc = time.perf_counter() - t0
    nk = sample_tokens * w.num_kv_heads
    idx = np.concatenate([e["idx"] for e in encs])
    g16 = np.concatenate([e["gamma16"] for e in encs])
    kidx, vidx = idx[:nk].reshape(sample_tokens, w.num_kv_heads, 128), idx[nk:].reshape(sample_tokens, w.num_kv_heads, 128)
    kg, vg = g16[:nk].reshape(sample_tokens, w.num_kv_heads), g16[nk:].reshape(sample_tokens, w.num_kv_heads)
    _, q64 = W.queries(w)
    G = w.num_q_heads // w.num_kv_heads
    t0 = time.perf_counter()
    for h in range(w.num_kv_heads):
        khat = O.reconstruct(kidx[:, h], kg[:, h], w.rot_seed, c32)
        vhat = O.reconstruct(vidx[:, h], vg[:, h], w.rot_seed, c32)
        for g in range(G):
            O.attention(q64[0, h * G + g], khat, vhat)
    t_dec = time.perf_counter() - t0
    return t_enc, t_dec, len(x)


def cpu_baseline(w, sample_tokens: int):
    """The oracle (float64 numpy), as it stands, on a bounded sample of the
    same workload: once with the BLAS threads numpy starts with and once on
    one thread."""
    from threadpoolctl import threadpool_info, threadpool_limits

    _, comp = bytes_per_vector(w.bits_k)
    dec_bytes = sample_tokens * w.num_kv_heads * 2 * comp
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    t_enc, t_dec, nvec = _oracle_sample(w, sample_tokens)
    with threadpool_limits(limits=1):
        t_enc1, t_dec1, _ = _oracle_sample(w, sample_tokens)
    return {
        "value": round(dec_bytes / t_dec / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"{sample_tokens} tokens x {w.num_kv_heads} KV heads of the workload: float64 numpy oracle "
                   f"encode of {nvec} vectors and original-frame decode-attend of {w.num_q_heads} query heads "
                   f"over them; value = the decode's algorithmic bytes / its time on {threads} BLAS threads"),
        "encode_vectors_per_s": round(nvec / t_enc, 1),
        "seconds": round(t_enc + t_dec, 2),
        "one_core": {"value": round(dec_bytes / t_dec1 / 1e9, 4), "unit": "GB/s",
                     "encode_vectors_per_s": round(nvec / t_enc1, 1), "seconds": round(t_enc1 + t_dec1, 2)},
        "host": host_cpu(),
    }


def measure_step(w, dev, stream, steps: int, warmup: int, only: str = "both", sets_arg: int = 0) -> dict:
    """Time `steps` steps of workload w (after `warmup`), cold: step i encodes
    set i mod C and decodes set (i + 1) mod C, encoded C - 1 steps before."""
    import torch

    from kv_cache_vector_encode_amd import tq
    from kv_cache_vector_encode_amd import workloads as W

    print(f"# workload {w.name}: generating inputs", file=sys.stderr, flush=True)
    kb, _ = W.keys(w)
    vb, _ = W.values(w)
    qb, _ = W.queries(w)
    K0 = torch.from_numpy(kb.view(np.int16)).view(torch.bfloat16).to(dev)
    V0 = torch.from_numpy(vb.view(np.int16)).view(torch.bfloat16).to(dev)
    q = torch.from_numpy(qb.view(np.int16)).view(torch.bfloat16).to(dev)
    slots = torch.from_numpy(W.slot_mapping(w)).to(dev)
    bt = torch.from_numpy(W.block_tables(w)).to(dev)
    lens = torch.from_numpy(W.seq_lens(w)).to(dev)
    del kb, vb

    rot = tq.tq_make_rotation(w.rot_seed, 128)
    cfg = tq.make_config(w.num_kv_heads, w.num_blocks, w.bits_k, w.bits_v, rot)
    pool_bytes = tq.tq_cache_bytes(cfg)
    set_bytes = 2 * K0.numel() * 2 + pool_bytes
    nsets = sets_arg or max(2, math.ceil((1 << 30) / set_bytes) + 1)
    sets = []
    for i in range(nsets):
        pool = torch.zeros(pool_bytes, dtype=torch.uint8, device=dev)
        cache = tq.tq_cache_create(cfg, pool)
        ws = tq.new_workspace(cache, w.num_seqs, w.num_q_heads, bt.shape[1], device=dev)
        sets.append(dict(K=K0.clone() if i else K0, V=V0.clone() if i else V0, cache=cache, ws=ws,
                         out=torch.empty((w.num_seqs, w.num_q_heads, 128), device=dev)))
    # every cache holds the workload's codes before any timed decode
    for s_ in sets:
        tq.tq_encode_kv(s_["K"], s_["V"], slots, w.bits_k, s_["cache"], stream)
    torch.cuda.synchronize()

    def step(i, ev=None):
        if only != "decode":
            s_ = sets[i % nsets]
            if ev is not None:
                ev[0].record(stream)
            tq.tq_encode_kv(s_["K"], s_["V"], slots, w.bits_k, s_["cache"], stream)
            if ev is not None:
                ev[1].record(stream)
        if only != "encode":
            s_ = sets[(i + 1) % nsets]
            if ev is not None:
                ev[2].record(stream)
            tq.tq_decode_attend(q, s_["cache"], bt, lens, s_["out"], s_["ws"], stream=stream)
            if ev is not None:
                ev[3].record(stream)

    print(f"# {nsets} rotating sets of {set_bytes / 1e6:.1f} MB; warmup {warmup}", file=sys.stderr, flush=True)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        step(warmup + i, evs[i])
    stop.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    return {
        "enc_ms": [e[0].elapsed_time(e[1]) for e in evs] if only != "decode" else [float("nan")],
        "dec_ms": [e[2].elapsed_time(e[3]) for e in evs] if only != "encode" else [float("nan")],
        "total_ms": start.elapsed_time(stop), "wall_s": t_wall, "nsets": nsets, "set_bytes": set_bytes,
        "K0": K0, "V0": V0, "q": q, "slots": slots, "bt": bt, "lens": lens, "sets": sets,
    }


def step_summary(w, r) -> dict:
    """Per-workload line: decode and encode rates of a measure_step result."""
    nvec = 2 * w.tokens * w.num_kv_heads
    in_b, comp_b = bytes_per_vector(w.bits_k)
    enc_s, dec_s = float(np.mean(r["enc_ms"])) / 1e3, float(np.mean(r["dec_ms"])) / 1e3
    dec_b = w.tokens * w.num_kv_heads * 2 * comp_b
    return {"decode_gbps": round(dec_b / dec_s / 1e9, 1), "decode_frac_hbm": round(dec_b / dec_s / 1e9 / HBM_PEAK_GBPS, 4),
            "decode_us": round(dec_s * 1e6, 2), "encode_vectors_per_s": round(nvec / enc_s, 1),
            "encode_gbps": round(nvec * (in_b + comp_b) / enc_s / 1e9, 1),
            "encode_frac_hbm": round(nvec * (in_b + comp_b) / enc_s / 1e9 / HBM_PEAK_GBPS, 4),
            "encode_us": round(enc_s * 1e6, 2), "rotating_sets": r["nsets"], "bits": w.bits_k}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama70b_4x131072_h8_gqa8_b3")
    ap.add_argument("--sets", type=int, default=0, help="rotating input/cache sets (0: >= 2 and enough that 1 GiB separates a cache's encode from its decode)")
    ap.add_argument("--no-other-workloads", action="store_true", help="skip the 1 x 32768 and 16 x 8192 workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the decompress and decode-step measurements after the step (profiling aid: their "
                         "launches would mix into the per-kernel statistics)")
    ap.add_argument("--cpu-sample-tokens", type=int, default=32768)
    ap.add_argument("--only", choices=["encode", "decode", "both"], default="both",
                    help="profiling aid: time only one of the two kernels")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (steps times), to scale HBM counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this path has no multi-GPU mode.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from kv_cache_vector_encode_amd import tq
    from kv_cache_vector_encode_amd import workloads as W

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": args.steps}), flush=True)
        return
    w = W.CONFIGS[args.workload]
    tq.lib()
    stream = torch.cuda.current_stream()
    mres = measure_step(w, dev, stream, args.steps, args.warmup, args.only, args.sets)
    enc_ms, dec_ms, total_ms, t_wall = mres["enc_ms"], mres["dec_ms"], mres["total_ms"], mres["wall_s"]
    nsets, set_bytes = mres["nsets"], mres["set_bytes"]
    K0, V0, q, slots, bt, lens, sets = mres["K0"], mres["V0"], mres["q"], mres["slots"], mres["bt"], mres["lens"], mres["sets"]
    nvec = 2 * w.tokens * w.num_kv_heads
    in_b, comp_b = bytes_per_vector(w.bits_k)
    enc_bytes = nvec * (in_b + comp_b)
    dec_bytes = w.tokens * w.num_kv_heads * 2 * comp_b     # K and V records + norms
    enc_s = float(np.mean(enc_ms)) / 1e3
    dec_s = float(np.mean(dec_ms)) / 1e3
    dec_gbps = dec_bytes / dec_s / 1e9
    enc_gbps = enc_bytes / enc_s / 1e9
    enc_vps = nvec / enc_s

    # ---- decompression of every cached key and value to bf16 (attention over
    # a compressed prefix): outside the step, reported beside it
    dq_ms = []
    if args.only == "both" and not args.no_extras:
        Ko = torch.empty((w.tokens, w.num_kv_heads, 128), dtype=torch.bfloat16, device=dev)
        Vo = torch.empty_like(Ko)
        for i in range(3):
            tq.tq_decompress_kv(sets[i % nsets]["cache"], slots, Ko, Vo, stream=stream)
        reps = max(5, args.steps // 4)
        dq_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
        for i in range(reps):
            dq_ev[i][0].record(stream)
            tq.tq_decompress_kv(sets[(i + 3) % nsets]["cache"], slots, Ko, Vo, stream=stream)
            dq_ev[i][1].record(stream)
        torch.cuda.synchronize()
        dq_ms = [e[0].elapsed_time(e[1]) for e in dq_ev]
        del Ko, Vo

    # ---- one decode step with append (each sequence's last token arrives
    # with the step) against the same work as two calls: encode of the new
    # tokens, then decode-attend.  Outside the timed step, reported beside it.
    st_ms, un_ms = [], []
    if args.only == "both" and not args.no_extras:
        S = w.seq_len
        Kn = K0.view(w.num_seqs, S, w.num_kv_heads, 128)[:, S - 1].contiguous()
        Vn = V0.view(w.num_seqs, S, w.num_kv_heads, 128)[:, S - 1].contiguous()
        new_slots = slots.view(w.num_seqs, S)[:, S - 1].contiguous()
        reps = max(5, args.steps // 4)

        def fused(i):
            s = sets[i % nsets]
            tq.tq_decode_step(q, Kn, Vn, s["cache"], bt, lens, s["out"], s["ws"], stream=stream)

        def unfused(i):
            s = sets[i % nsets]
            tq.tq_encode_kv(Kn, Vn, new_slots, w.bits_k, s["cache"], stream)
            tq.tq_decode_attend(q, s["cache"], bt, lens, s["out"], s["ws"], stream=stream)

        for fn, acc in ((fused, st_ms), (unfused, un_ms)):
            for i in range(3):
                fn(i)
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
            for i in range(reps):
                ev[i][0].record(stream)
                fn(i + 3)
                ev[i][1].record(stream)
            torch.cuda.synchronize()
            acc.extend(e[0].elapsed_time(e[1]) for e in ev)

    # ---- caches with the QJL residual sketch on the keys (E6): encode every
    # key and value into them (the vector-unit encoder), and decode-attend
    # over them; two caches used in turn
    qe_ms, qd_ms = [], []
    if args.only == "both" and not args.no_extras:
        qrot = tq.tq_make_rotation(w.rot_seed, 128)
        qrot2 = tq.tq_make_rotation(w.rot_seed + 1, 128)
        qcfg = tq.make_config(w.num_kv_heads, w.num_blocks, w.bits_k, w.bits_v, qrot, True, qrot2)
        qsets = []
        for i in range(2):
            qpool = torch.zeros(tq.tq_cache_bytes(qcfg), dtype=torch.uint8, device=dev)
            qc = tq.tq_cache_create(qcfg, qpool)
            qsets.append(dict(cache=qc, ws=tq.new_workspace(qc, w.num_seqs, w.num_q_heads, bt.shape[1], device=dev),
                              out=torch.empty((w.num_seqs, w.num_q_heads, 128), device=dev)))
        reps = max(5, args.steps // 4)

        def q_enc(i):
            s, c = sets[i % nsets], qsets[i % 2]
            tq.tq_encode_kv(s["K"], s["V"], slots, w.bits_k, c["cache"], stream)

        def q_dec(i):
            c = qsets[(i + 1) % 2]
            tq.tq_decode_attend(q, c["cache"], bt, lens, c["out"], c["ws"], stream=stream)

        for fn, acc in ((q_enc, qe_ms), (q_dec, qd_ms)):
            for i in range(3):
                fn(i)
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
            for i in range(reps):
                ev[i][0].record(stream)
                fn(i + 3)
                ev[i][1].record(stream)
            torch.cuda.synchronize()
            acc.extend(e[0].elapsed_time(e[1]) for e in ev)
        del qsets

    # ---- the min/max comparison codec on the same keys and values
    mm_enc_ms, mm_dec_ms = [], []
    if args.only == "both" and not args.no_extras:
        mrot = tq.tq_make_rotation(w.rot_seed, 128)
        nv = w.tokens * w.num_kv_heads
        mcodes = [torch.empty((nv, 16 * w.bits_k), dtype=torch.uint8, device=dev) for _ in range(2)]
        mparams = [torch.empty((nv, 2), dtype=torch.int16, device=dev) for _ in range(2)]
        mout = torch.empty((nv, 128), dtype=torch.bfloat16, device=dev)
        reps = max(5, args.steps // 4)

        def mm_enc(i):
            s = sets[i % nsets]
            tq.tq_minmax_encode(s["K"].view(-1, 128), w.bits_k, mrot, mcodes[0], mparams[0], stream)
            tq.tq_minmax_encode(s["V"].view(-1, 128), w.bits_k, mrot, mcodes[1], mparams[1], stream)

        def mm_dec(i):
            for j in range(2):
                tq.tq_minmax_decode(mcodes[j], mparams[j], w.bits_k, mrot, mout, stream)

        for fn, acc in ((mm_enc, mm_enc_ms), (mm_dec, mm_dec_ms)):
            for i in range(3):
                fn(i)
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
            for i in range(reps):
                ev[i][0].record(stream)
                fn(i + 3)
                ev[i][1].record(stream)
            torch.cuda.synchronize()
            acc.extend(e[0].elapsed_time(e[1]) for e in ev)
        del mcodes, mparams, mout

    # ---- the octahedral triplet codec: encode every key (head-major, so
    # that each head's records are contiguous), then the logits of sequence
    # 0's query group against every key of its KV head straight from the
    # records.  Outside the timed step, reported beside it.
    oc_enc_ms, oc_log_ms, oq_enc_ms, oq_log_ms, oa_ms = [], [], [], [], []
    if args.only == "both" and not args.no_extras:
        orot = tq.tq_make_rotation(w.rot_seed, 128)
        otb = torch.empty(tq.tq_octo_table_bytes(w.bits_k), dtype=torch.uint8, device=dev)
        tq.tq_octo_tables(w.bits_k, otb, stream)
        orb = tq.tq_octo_record_bytes(128, w.bits_k)
        H, G, T = w.num_kv_heads, w.num_q_heads // w.num_kv_heads, w.tokens
        okh = [s["K"].view(T, H, 128).transpose(0, 1).contiguous() for s in sets]
        ocodes = [torch.empty((H, T, orb), dtype=torch.uint8, device=dev) for _ in sets]
        ogam = [torch.empty((H, T), dtype=torch.int16, device=dev) for _ in sets]
        oq = q[0].float().view(H, G, 128).contiguous()
        olog = torch.empty((H, G, T), dtype=torch.float32, device=dev)
        # OCTOPUS-QJL: the same codes plus the residual sketch (16 sign bytes
        # and an fp16 norm per key)
        orot2 = tq.tq_make_rotation(w.rot_seed + 1, 128)
        osig = [torch.empty((H, T, 16), dtype=torch.uint8, device=dev) for _ in sets]
        orho = [torch.empty((H, T), dtype=torch.int16, device=dev) for _ in sets]
        # decode-attend over triplet-coded keys and values: every sequence's
        # query group against its own keys; a "head" of the call is one
        # (KV head, sequence), whose keys are contiguous in the [H][T] layout
        NS, S = w.num_seqs, w.seq_len
        ovh = [s["V"].view(T, H, 128).transpose(0, 1).contiguous() for s in sets]
        ovcodes = [torch.empty((H, T, orb), dtype=torch.uint8, device=dev) for _ in sets]
        ovgam = [torch.empty((H, T), dtype=torch.int16, device=dev) for _ in sets]
        for j in range(nsets):
            tq.tq_octo_encode(ovh[j].view(-1, 128), w.bits_k, orot, otb, ovcodes[j].view(-1, orb), ovgam[j].view(-1),
                              stream)
        del ovh
        oqa = q.float().view(NS, H, G, 128).transpose(0, 1).reshape(H * NS, G, 128).contiguous()
        oout = torch.empty((H * NS, G, 128), dtype=torch.float32, device=dev)
        ows = torch.empty(tq.tq_octo_attend_workspace_bytes(H * NS, G, S), dtype=torch.uint8, device=dev)
        reps = max(5, args.steps // 4)

        def oc_enc(i):
            j = i % nsets
            tq.tq_octo_encode(okh[j].view(-1, 128), w.bits_k, orot, otb, ocodes[j].view(-1, orb), ogam[j].view(-1),
                              stream)

        def oc_log(i):
            j = i % nsets
            tq.tq_octo_logits(oq, ocodes[j], ogam[j], w.bits_k, orot, otb, olog, stream=stream)

        def oq_enc(i):
            j = i % nsets
            tq.tq_octo_encode_qjl(okh[j].view(-1, 128), w.bits_k, orot, orot2, otb, ocodes[j].view(-1, orb),
                                  ogam[j].view(-1), osig[j].view(-1, 16), orho[j].view(-1), stream)

        def oq_log(i):
            j = i % nsets
            tq.tq_octo_logits_qjl(oq, ocodes[j], ogam[j], osig[j], orho[j], w.bits_k, orot, orot2, otb, olog,
                                  stream=stream)

        def oa_att(i):
            j = i % nsets
            tq.tq_octo_attend(oqa, ocodes[j].view(H * NS, S, orb), ogam[j].view(H * NS, S),
                              ovcodes[j].view(H * NS, S, orb), ovgam[j].view(H * NS, S), w.bits_k, orot, otb, oout,
                              ows, stream=stream)

        for fn, acc in ((oc_enc, oc_enc_ms), (oc_log, oc_log_ms), (oq_enc, oq_enc_ms), (oq_log, oq_log_ms),
                        (oa_att, oa_ms)):
            for i in range(max(3, nsets)):
                fn(i)
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
            for i in range(reps):
                ev[i][0].record(stream)
                fn(i + 3)
                ev[i][1].record(stream)
            torch.cuda.synchronize()
            acc.extend(e[0].elapsed_time(e[1]) for e in ev)
        del okh, ocodes, ogam, olog, osig, orho, ovcodes, ovgam, oout, ows

    # ---- on-box ceilings: a plain stream read (the library's measurement
    # aid) and a device copy, each over 2 GiB
    onbox = None
    if args.only == "both" and not args.no_extras:
        buf = torch.empty(1 << 31, dtype=torch.uint8, device=dev)
        buf2 = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        sink = torch.zeros(4, dtype=torch.int32, device=dev)
        for _ in range(3):
            tq.tq_stream_read(buf, sink, stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(10):
            tq.tq_stream_read(buf, sink, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        read_gbps = 10 * buf.numel() / (e0.elapsed_time(e1) / 1e3) / 1e9
        src = buf[: 1 << 30]
        for _ in range(3):
            buf2.copy_(src)
        e0.record(stream)
        for _ in range(10):
            buf2.copy_(src)
        e1.record(stream)
        torch.cuda.synchronize()
        copy_gbps = 10 * 2 * buf2.numel() / (e0.elapsed_time(e1) / 1e3) / 1e9
        del buf, buf2, src
        onbox = {"read_gbps": round(read_gbps, 1), "copy_gbps": round(copy_gbps, 1),
                 "read_kernel": "tq_stream_read, 2 GiB, non-temporal 16-byte loads",
                 "copy_kernel": "torch copy_, 1 GiB (read + write counted)"}

    kernels = {
        "tq_encode": {"bound": "hbm", "achieved": round(enc_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                      "frac": round(enc_gbps / HBM_PEAK_GBPS, 4), "bytes_per_launch": enc_bytes,
                      "us_per_launch": round(enc_s * 1e6, 2), "median_us": round(float(np.median(enc_ms)) * 1e3, 2)},
        "tq_decode_attend": {"bound": "hbm", "achieved": round(dec_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                             "frac": round(dec_gbps / HBM_PEAK_GBPS, 4), "bytes_per_launch": dec_bytes,
                             "us_per_launch": round(dec_s * 1e6, 2), "median_us": round(float(np.median(dec_ms)) * 1e3, 2)},
    }
    if dq_ms:
        dq_s = float(np.mean(dq_ms)) / 1e3
        dq_bytes = w.tokens * w.num_kv_heads * 2 * (comp_b + 2 * 128)   # codes + norms in, bf16 out
        kernels["tq_decompress_kv"] = {
            "bound": "hbm", "achieved": round(dq_bytes / dq_s / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(dq_bytes / dq_s / 1e9 / HBM_PEAK_GBPS, 4), "bytes_per_launch": dq_bytes,
            "us_per_launch": round(dq_s * 1e6, 2), "median_us": round(float(np.median(dq_ms)) * 1e3, 2),
            "note": "every cached key and value to bf16; not part of the timed step"}
    if st_ms:
        st_s, un_s = float(np.mean(st_ms)) / 1e3, float(np.mean(un_ms)) / 1e3
        kernels["tq_decode_step"] = {
            "bound": "hbm", "achieved": round(dec_bytes / st_s / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(dec_bytes / st_s / 1e9 / HBM_PEAK_GBPS, 4), "bytes_per_launch": dec_bytes,
            "us_per_launch": round(st_s * 1e6, 2), "median_us": round(float(np.median(st_ms)) * 1e3, 2),
            "unfused_us": round(un_s * 1e6, 2),
            "note": "append each sequence's new token + decode-attend in one call; unfused_us = tq_encode_kv of "
                    "the new tokens + tq_decode_attend; not part of the timed step"}
    if qe_ms:
        # keys carry 16 sign bytes and an fp16 residual norm more
        qkb = 128 * w.bits_k // 8 + 2 + 16 + 2
        qvb = 128 * w.bits_v // 8 + 2
        th = w.tokens * w.num_kv_heads
        qeb = th * (2 * in_b + qkb + qvb)
        qe_s = float(np.mean(qe_ms)) / 1e3
        kernels["tq_encode_kv_qjl"] = {
            "bound": "hbm", "achieved": round(qeb / qe_s / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(qeb / qe_s / 1e9 / HBM_PEAK_GBPS, 4), "bytes_per_launch": qeb,
            "us_per_launch": round(qe_s * 1e6, 2), "vectors_per_s": round(2 * th / qe_s, 1),
            "note": "encode into a cache with the QJL residual sketch on the keys (matrix-core encoder, sketch product in split f16); "
                    "not part of the timed step"}
        qdb = th * (qkb + qvb)
        qd_s = float(np.mean(qd_ms)) / 1e3
        kernels["tq_decode_attend_qjl"] = {
            "bound": "hbm", "achieved": round(qdb / qd_s / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(qdb / qd_s / 1e9 / HBM_PEAK_GBPS, 4), "bytes_per_launch": qdb,
            "us_per_launch": round(qd_s * 1e6, 2),
            "note": "decode-attend over a cache with the QJL residual sketch (matrix-core split kernel + merge); "
                    "not part of the timed step"}
    if mm_enc_ms:
        mb = nvec * (in_b + 128 * w.bits_k // 8 + 4)            # bf16 in, codes + fp16 scale and zero out
        me_s = float(np.mean(mm_enc_ms)) / 1e3
        kernels["tq_minmax_encode"] = {
            "bound": "hbm", "achieved": round(mb / me_s / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(mb / me_s / 1e9 / HBM_PEAK_GBPS, 4), "bytes_per_launch": mb,
            "us_per_launch": round(me_s * 1e6, 2), "vectors_per_s": round(nvec / me_s, 1),
            "note": "min/max comparison codec, every key and value (two launches); not part of the timed step"}
        db = nvec * (128 * w.bits_k // 8 + 4 + 256)
        md_s = float(np.mean(mm_dec_ms)) / 1e3
        kernels["tq_minmax_decode"] = {
            "bound": "hbm", "achieved": round(db / md_s / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(db / md_s / 1e9 / HBM_PEAK_GBPS, 4), "bytes_per_launch": db,
            "us_per_launch": round(md_s * 1e6, 2),
            "note": "min/max comparison codec back to bf16, every key and value (two launches)"}
    if oc_enc_ms:
        orb = tq.tq_octo_record_bytes(128, w.bits_k)
        nk = w.tokens * w.num_kv_heads
        ob = nk * (in_b + orb + 2)                               # bf16 in, record + fp16 norm out
        oe_s = float(np.mean(oc_enc_ms)) / 1e3
        kernels["tq_octo_encode"] = {
            "bound": "hbm", "achieved": round(ob / oe_s / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(ob / oe_s / 1e9 / HBM_PEAK_GBPS, 4), "bytes_per_launch": ob,
            "us_per_launch": round(oe_s * 1e6, 2), "vectors_per_s": round(nk / oe_s, 1),
            "note": "octahedral triplet codec, every key (bits_dir = b+1, bits_norm = b-1); "
                    "not part of the timed step"}
        G = w.num_q_heads // w.num_kv_heads
        lb = nk * (orb + 2) + nk * G * 4 + w.num_q_heads * 128 * 4   # records + norms in, logits out
        ol_s = float(np.mean(oc_log_ms)) / 1e3
        kernels["tq_octo_logits"] = {
            "bound": "hbm", "achieved": round(lb / ol_s / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(lb / ol_s / 1e9 / HBM_PEAK_GBPS, 4), "bytes_per_launch": lb,
            "us_per_launch": round(ol_s * 1e6, 2), "keys_per_s": round(nk / ol_s, 1),
            "note": f"sequence 0's {G} queries per KV head against every key of that head, fp32 logits out"}
    if oq_enc_ms:
        qb = nk * (in_b + orb + 2 + 16 + 2)                      # plus 16 sign bytes and an fp16 norm out
        qe_s = float(np.mean(oq_enc_ms)) / 1e3
        kernels["tq_octo_encode_qjl"] = {
            "bound": "hbm", "achieved": round(qb / qe_s / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(qb / qe_s / 1e9 / HBM_PEAK_GBPS, 4), "bytes_per_launch": qb,
            "us_per_launch": round(qe_s * 1e6, 2), "vectors_per_s": round(nk / qe_s, 1),
            "note": "OCTOPUS-QJL: the triplet codes of every key plus the one-bit sketch of their residual"}
        qlb = nk * (orb + 2 + 16 + 2) + nk * G * 4 + w.num_q_heads * 128 * 4
        ql_s = float(np.mean(oq_log_ms)) / 1e3
        kernels["tq_octo_logits_qjl"] = {
            "bound": "hbm", "achieved": round(qlb / ql_s / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(qlb / ql_s / 1e9 / HBM_PEAK_GBPS, 4), "bytes_per_launch": qlb,
            "us_per_launch": round(ql_s * 1e6, 2), "keys_per_s": round(nk / ql_s, 1),
            "note": f"OCTOPUS-QJL logits: {G} queries per KV head against every key, with the residual estimate"}
    if oa_ms:
        ab = 2 * nk * (orb + 2) + 2 * w.num_seqs * w.num_q_heads * 128 * 4   # key and value records + norms in
        oa_s = float(np.mean(oa_ms)) / 1e3
        kernels["tq_octo_attend"] = {
            "bound": "hbm", "achieved": round(ab / oa_s / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(ab / oa_s / 1e9 / HBM_PEAK_GBPS, 4), "bytes_per_launch": ab,
            "us_per_launch": round(oa_s * 1e6, 2),
            "note": "decode-attend over triplet-coded keys and values, every sequence's query group "
                    "(split kernel + merge); not part of the timed step"}
    dom = "tq_encode" if enc_s >= dec_s else "tq_decode_attend"
    traffic = None
    tf = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tf):
        with open(tf) as f:
            tj = json.load(f)
        ent = tj.get(w.name, {}).get(dom)
        if ent and ent.get("kernel_hash") == kernel_hash():
            traffic = ent.get("hbm_bytes_per_launch")
    roof = dict(kernels[dom])
    roof["kernel"] = dom
    roof["traffic"] = traffic
    for k in ("bytes_per_launch", "us_per_launch", "median_us"):
        roof.pop(k, None)

    res = {
        "metric": METRIC,
        "value": round(dec_gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "dtype_detail": ("decode: matrix-core products with f16 operands and f32 accumulation (2/3-bit keys and all "
                         "values: codebooks as scaled f16, queries as f16 high + low parts, p*gamma_v as f16; "
                         "4-bit keys: 16-bit integer centroids and queries as 8-bit planes, exact int32 sums), "
                         "online softmax and merge in f32; encode: bf16 input, Hadamard product on bf16 matrix "
                         "cores with f32 accumulation, f32 threshold search, fp16 norms"),
        "data": "synthetic",
        "config": {"workload": w.name, "num_seqs": w.num_seqs, "seq_len": w.seq_len,
                   "num_kv_heads": w.num_kv_heads, "num_q_heads": w.num_q_heads, "head_dim": 128,
                   "bits_k": w.bits_k, "bits_v": w.bits_v, "block_tokens": 16, "input": "bf16",
                   "rotating_sets": nsets},
        "decode_frac_hbm": round(dec_gbps / HBM_PEAK_GBPS, 4),
        "encode_vectors_per_s": round(enc_vps, 1),
        "encode_gbps": round(enc_gbps, 1),
        "encode_frac_hbm": round(enc_gbps / HBM_PEAK_GBPS, 4),
        "kernels": kernels,
        "roofline": roof,
        "wall_s_timed": round(t_wall, 4),
    }
    if onbox:
        onbox["decode_frac_of_read"] = round(dec_gbps / onbox["read_gbps"], 4)
        onbox["encode_frac_of_copy"] = round(enc_gbps / onbox["copy_gbps"], 4)
        res["onbox_ceiling"] = onbox
    if args.only != "both":
        res["only"] = args.only
    if not args.no_other_workloads and args.only == "both":
        # the other decode configurations, the same cold step on each
        mres.clear()
        del K0, V0, q, slots, bt, lens, sets
        torch.cuda.empty_cache()
        other = {}
        for name in ("decode_1x32768_h8_gqa8_b4", "prefill_16x8192_h8_gqa8_b4"):
            if name == w.name:
                continue
            wo = W.CONFIGS[name]
            r = measure_step(wo, dev, stream, min(args.steps, 50), min(args.warmup, 5))
            other[name] = step_summary(wo, r)
            r.clear()
            torch.cuda.empty_cache()
        res["other_workloads"] = other
    if not args.no_cpu_baseline:
        print("# cpu baseline (oracle)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_sample_tokens)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
