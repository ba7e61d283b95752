"""GPU parity at the full sizes of the benchmark configurations.

* decode_1x32768_h8_gqa8_b4 and prefill_16x8192_h8_gqa8_b4: one
  tq_encode_kv of every key and value, then tq_decode_attend without
  logits (the launch configuration bench.py times) and with logits; codes
  and norms of sampled token windows, and outputs / logits of sampled
  (sequence, query head) pairs, against the oracle computed one by one.
* llama70b_4x131072_h8_gqa8_b3: the same, with the encode split into one
  call per sequence (host memory), decode as in bench.py.
* decode_1x32768_h8_gqa8_b4 as a generation step: every token but the last
  through tq_encode_kv, the last through tq_decode_step (the launch
  configuration bench.py times); the appended codes and norms and sampled
  outputs against the oracle; then tq_decompress_kv of every key and value
  to bf16, checked on sampled vectors.
* sweep_16h_65536_keys: keys-only caches for b = 2, 3, 4 with and without
  the QJL residual; tq_decode_logits for one query per head; parity of codes
  and logits on exactly 10^5 seeded (head, token) pairs, plus the logit bias
  and MSE against the unquantised keys (reported; the QJL variant must lower
  the MSE).
"""

import functools
import math

import numpy as np
import pytest
import torch

from kv_cache_vector_encode_amd import tq
from kv_cache_vector_encode_amd import workloads as W
from oracle import tq_oracle as O

from gpu_common import (LOGIT_RTOL, OUT_RTOL, check_codes, check_norms, check_octo_codes, cs_scale, make_cache,
                        to_device)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _say(*a):
    print(*a, flush=True)


def _chunks(cache, w, blocks, head=None):
    """Pool bytes of the given physical blocks (all heads, or one head) and an
    oracle layout describing exactly that sub-pool."""
    lay_full = O.LayoutV1(128, w.num_kv_heads, w.bits_k, w.bits_v, w.qjl, w.num_blocks)
    view = cache.pool.view(w.num_blocks, w.num_kv_heads, lay_full.block_bytes)
    idx = torch.from_numpy(np.asarray(blocks, dtype=np.int64)).to(cache.pool.device)
    sub = view.index_select(0, idx)
    if head is not None:
        sub = sub[:, head:head + 1]
    arr = sub.contiguous().cpu().numpy()
    lay = O.LayoutV1(128, arr.shape[1], w.bits_k, w.bits_v, w.qjl, arr.shape[0])
    return arr, lay


def _encode_all(w, device, per_call_tokens=None, slots=None):
    cache = make_cache(w, device)
    slots = W.slot_mapping(w) if slots is None else slots
    n = w.tokens if per_call_tokens is None else per_call_tokens
    for t0 in range(0, w.tokens, n):
        cnt = min(n, w.tokens - t0)
        kb, _ = W.keys(w, t0, cnt)
        vb, _ = W.values(w, t0, cnt)
        K, V = to_device(kb, w.in_dtype, device), to_device(vb, w.in_dtype, device)
        del kb, vb
        sm = torch.from_numpy(np.ascontiguousarray(slots[t0:t0 + cnt])).to(device)
        tq.tq_encode_kv(K, V, sm, w.bits_k, cache)
        torch.cuda.synchronize()
        del K, V
    return cache, slots


def _check_encode_windows(w, cache, slots, rng, windows=4, width=256):
    c32, t32 = O.codebook_fp32(128, w.bits_k)
    starts = rng.choice(w.tokens // width, windows, replace=False) * width
    worst = 0
    for t0 in starts:
        k64 = W.keys(w, int(t0), width)[1]
        v64 = W.values(w, int(t0), width)[1]
        s = slots[t0:t0 + width]
        blocks, inv = np.unique(s // 16, return_inverse=True)
        arr, lay = _chunks(cache, w, blocks)
        up = O.unpack_pool(arr, lay)
        for name, x64, ki, kg in (("K", k64, "k_idx", "k_g16"), ("V", v64, "v_idx", "v_g16")):
            enc = O.encode(x64.reshape(-1, 128), w.rot_seed, c32)
            gidx = up[ki][inv, :, s % 16].reshape(-1, 128)
            g16 = up[kg][inv, :, s % 16].reshape(-1)
            worst = max(worst, check_codes(gidx, enc["idx"], enc["y"], t32, what=f"{name} window {t0}"))
            check_norms(g16, enc["gamma"], what=f"{name} norms window {t0}")
    return worst


def _check_decode_pairs(w, cache, pairs, out, logits=None):
    c32k, _ = O.codebook_fp32(128, w.bits_k)
    c32v, _ = O.codebook_fp32(128, w.bits_v)
    bt = W.block_tables(w)
    _, q64 = W.queries(w)
    group = w.num_q_heads // w.num_kv_heads
    R = O.rotation_matrix(w.rot_seed, 128)
    tau = 1 / math.sqrt(128)
    go = out.cpu().numpy().astype(np.float64)
    gl = logits.cpu().numpy() if logits is not None else None
    worst_o = worst_l = 0.0
    for n, hq in pairs:
        h = hq // group
        L = w.seq_len
        arr, lay = _chunks(cache, w, bt[n, :w.blocks_per_seq], head=h)
        up = O.unpack_pool(arr, lay)
        kidx = up["k_idx"][:, 0].reshape(-1, 128)[:L]
        kg = up["k_g16"][:, 0].reshape(-1)[:L]
        khat = O.reconstruct(kidx, kg, w.rot_seed, c32k)
        vhat = O.reconstruct(up["v_idx"][:, 0].reshape(-1, 128)[:L], up["v_g16"][:, 0].reshape(-1)[:L],
                             w.rot_seed, c32v)
        o, s = O.attention(q64[n, hq], khat, vhat)
        e = np.linalg.norm(go[n, hq] - o) / np.linalg.norm(o)
        assert e <= OUT_RTOL, (n, hq, e)
        worst_o = max(worst_o, e)
        if gl is not None:
            scl = cs_scale(tau, kg, np.linalg.norm(R @ q64[n, hq]), np.linalg.norm(c32k[kidx], axis=1))
            err = np.abs(gl[n, hq, :L].astype(np.float64) - s)
            assert np.all(err <= LOGIT_RTOL * scl), (n, hq, float((err / scl).max()))
            worst_l = max(worst_l, float((err / scl).max()))
    return worst_o, worst_l


def _decode(w, cache, device, want_logits):
    bt = torch.from_numpy(W.block_tables(w)).to(device)
    lens = torch.from_numpy(W.seq_lens(w)).to(device)
    qb, _ = W.queries(w)
    q = to_device(qb, "bf16", device)
    out = torch.full((w.num_seqs, w.num_q_heads, 128), float("nan"), device=device)
    logits = None
    if want_logits:
        logits = torch.full((w.num_seqs, w.num_q_heads, bt.shape[1] * 16), float("nan"), device=device)
    ws = tq.new_workspace(cache, w.num_seqs, w.num_q_heads, bt.shape[1], device=device)
    tq.tq_decode_attend(q, cache, bt, lens, out, ws, logits_out=logits)
    torch.cuda.synchronize()
    return out, logits


@pytest.mark.parametrize("name,npairs", [("decode_1x32768_h8_gqa8_b4", 8), ("prefill_16x8192_h8_gqa8_b4", 8)])
def test_fullsize_encode_and_decode(device, name, npairs):
    w = W.CONFIGS[name]
    rng = np.random.default_rng(11)
    _say(f"{name}: encode {2 * w.tokens * w.num_kv_heads} vectors")
    cache, slots = _encode_all(w, device)
    nb = _check_encode_windows(w, cache, slots, rng)
    pairs = [(int(rng.integers(w.num_seqs)), int(hq)) for hq in rng.choice(w.num_q_heads, npairs, replace=False)]
    out, _ = _decode(w, cache, device, want_logits=False)
    wo, _ = _check_decode_pairs(w, cache, pairs, out)
    out2, logits = _decode(w, cache, device, want_logits=True)
    wo2, wl = _check_decode_pairs(w, cache, pairs, out2, logits)
    _say(f"{name}: band mismatches {nb}; worst out {max(wo, wo2):.2e}; worst logit {wl:.2e} (bars 2e-3, 1e-4)")


def test_fullsize_decode_step_and_decompress(device):
    w = W.DECODE_32K
    rng = np.random.default_rng(14)
    S = w.seq_len
    full = W.slot_mapping(w)
    slots = full.copy()
    slots[S - 1::S] = -1                       # each sequence's last token arrives with the step
    _say(f"{w.name}: encode {2 * (w.tokens - w.num_seqs) * w.num_kv_heads} vectors, then one decode step")
    cache, _ = _encode_all(w, device, slots=slots)
    kb, k64 = W.keys(w, S - 1, 1)
    vb, v64 = W.values(w, S - 1, 1)
    Kn, Vn = to_device(kb, w.in_dtype, device), to_device(vb, w.in_dtype, device)
    bt = torch.from_numpy(W.block_tables(w)).to(device)
    lens = torch.from_numpy(W.seq_lens(w)).to(device)
    q = to_device(W.queries(w)[0], "bf16", device)
    out = torch.full((w.num_seqs, w.num_q_heads, 128), float("nan"), device=device)
    ws = tq.new_workspace(cache, w.num_seqs, w.num_q_heads, bt.shape[1], device=device)
    tq.tq_decode_step(q, Kn, Vn, cache, bt, lens, out, ws)
    torch.cuda.synchronize()
    # appended token: codes and norms against the oracle encode
    c32, t32 = O.codebook_fp32(128, w.bits_k)
    s_new = full[S - 1]
    arr, lay = _chunks(cache, w, [s_new // 16])
    up = O.unpack_pool(arr, lay)
    for x64, ki, kg in ((k64, "k_idx", "k_g16"), (v64, "v_idx", "v_g16")):
        enc = O.encode(x64.reshape(-1, 128), w.rot_seed, c32)
        check_codes(up[ki][0, :, s_new % 16], enc["idx"], enc["y"], t32, what="appended codes")
        check_norms(up[kg][0, :, s_new % 16], enc["gamma"], what="appended norms")
    pairs = [(0, int(hq)) for hq in rng.choice(w.num_q_heads, 6, replace=False)]
    wo, _ = _check_decode_pairs(w, cache, pairs, out)
    # every key and value back to bf16; sampled vectors against the oracle
    Ko = torch.empty((w.tokens, w.num_kv_heads, 128), dtype=torch.bfloat16, device=device)
    Vo = torch.empty_like(Ko)
    tq.tq_decompress_kv(cache, torch.from_numpy(full).to(device), Ko, Vo)
    torch.cuda.synchronize()
    toks = np.sort(rng.choice(w.tokens, 64, replace=False))
    arr, lay = _chunks(cache, w, full[toks] // 16)
    up = O.unpack_pool(arr, lay)
    r = full[toks] % 16
    worst = 0.0
    for out16, ki, kg in ((Ko, "k_idx", "k_g16"), (Vo, "v_idx", "v_g16")):
        got = out16[torch.from_numpy(toks).to(device)].float().cpu().numpy().astype(np.float64)
        idx = up[ki][np.arange(len(toks)), :, r]
        g16 = up[kg][np.arange(len(toks)), :, r]
        want = O.reconstruct(idx, g16, w.rot_seed, c32)
        scale = np.abs(g16.astype(np.float64))[..., None] * np.max(np.abs(c32))
        err = np.abs(got - want) - (2.0 ** -8) * np.abs(want)
        assert np.all(err <= 1e-5 * scale + 2.0 ** -24)
        worst = max(worst, float(np.max(np.abs(got - want) / (scale + 1e-30))))
    _say(f"{w.name} step: worst out {wo:.2e} (bar 2e-3); decompress worst |err|/scale {worst:.2e}")


def test_fullsize_llama70b_b3(device):
    w = W.LLAMA70B_128K
    rng = np.random.default_rng(12)
    _say(f"{w.name}: encode {2 * w.tokens * w.num_kv_heads} vectors, one call per sequence")
    cache, slots = _encode_all(w, device, per_call_tokens=w.seq_len)
    nb = _check_encode_windows(w, cache, slots, rng)
    pairs = [(int(rng.integers(w.num_seqs)), int(rng.integers(w.num_q_heads))) for _ in range(4)]
    out, _ = _decode(w, cache, device, want_logits=False)
    wo, _ = _check_decode_pairs(w, cache, pairs, out)
    out2, logits = _decode(w, cache, device, want_logits=True)
    wo2, wl = _check_decode_pairs(w, cache, pairs[:2], out2, logits)
    _say(f"{w.name}: band mismatches {nb}; worst out {max(wo, wo2):.2e}; worst logit {wl:.2e}")


# ------------------------------------------------------------ sweep config --

@functools.lru_cache(maxsize=1)
def _sweep_keys():
    w = W.SWEEP_64K
    kb, k64 = W.keys(w)
    return kb, k64


def _sample_records(arr, lay, blocks, heads, rows):
    """Oracle-unpacked records for the sampled (block, head, row) triples,
    unpacking the pool a slice of blocks at a time."""
    n = len(blocks)
    out = {}
    step = 256
    for b0 in range(0, lay.num_blocks, step):
        sel = np.nonzero((blocks >= b0) & (blocks < b0 + step))[0]
        if len(sel) == 0:
            continue
        nb = min(step, lay.num_blocks - b0)
        sub = arr[b0:b0 + nb]
        up = O.unpack_pool(sub, O.LayoutV1(128, lay.hkv, lay.bk, lay.bv, lay.qjl, nb))
        for k, v in up.items():
            if k not in out:
                out[k] = np.zeros((n,) + v.shape[3:], dtype=v.dtype)
            out[k][sel] = v[blocks[sel] - b0, heads[sel], rows[sel]]
    return out


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_sweep_logits_1e5_pairs(device, bits):
    base = W.SWEEP_64K
    kb, k64 = _sweep_keys()
    K = to_device(kb, base.in_dtype, device)
    rng = np.random.default_rng(2024 + bits)
    NP = 100_000
    heads = rng.integers(0, base.num_kv_heads, NP)
    toks = rng.integers(0, base.tokens, NP)
    qb, q64 = W.queries(base)             # one query per head (16 query heads)
    q = to_device(qb, "bf16", device)
    c32, t32 = O.codebook_fp32(128, bits)
    R = O.rotation_matrix(base.rot_seed, 128)
    tau = 1 / math.sqrt(128)
    xs = k64[toks, heads]                 # the sampled exact keys
    enc = O.encode(xs, base.rot_seed, c32)
    s_exact = tau * np.einsum("nd,nd->n", xs, q64[0, heads])
    mse = {}
    for qjl in (False, True):
        w = base.with_(bits_k=bits, qjl=qjl)
        cache = make_cache(w, device)
        slots = torch.from_numpy(W.slot_mapping(w)).to(device)
        tq.tq_encode_kv(K, None, slots, bits, cache)
        bt = torch.from_numpy(W.block_tables(w)).to(device)
        lens = torch.from_numpy(W.seq_lens(w)).to(device)
        logits = torch.full((1, w.num_q_heads, bt.shape[1] * 16), float("nan"), device=device)
        tq.tq_decode_logits(q, cache, bt, lens, logits)
        torch.cuda.synchronize()
        lay = O.LayoutV1(128, w.num_kv_heads, bits, 0, qjl, w.num_blocks)
        arr = cache.pool.cpu().numpy().reshape(w.num_blocks, w.num_kv_heads, lay.block_bytes)
        s_map = W.slot_mapping(w)[toks]
        rec = _sample_records(arr, lay, s_map // 16, heads, s_map % 16)
        # codes and norms of the sampled keys
        check_codes(rec["k_idx"], enc["idx"], enc["y"], t32, what=f"b{bits} qjl={qjl} codes")
        check_norms(rec["k_g16"], enc["gamma"], what=f"b{bits} qjl={qjl} norms")
        # logits: oracle from the GPU's codes, original frame
        khat = O.reconstruct(rec["k_idx"], rec["k_g16"], base.rot_seed, c32)
        s_or = tau * np.einsum("nd,nd->n", khat, q64[0, heads])
        rho = None
        if qjl:
            qrot = q64[0, heads] @ R.T
            est = O.qjl_dot_estimate(rec["qjl_bits"], rec["rho16"], qrot, base.qjl_seed)
            s_or = s_or + tau * rec["k_g16"].astype(np.float64) * est
            rho = rec["rho16"]
        gl = logits.cpu().numpy()[0, heads, toks].astype(np.float64)
        qn = np.linalg.norm(q64[0, heads] @ R.T, axis=1)
        scl = cs_scale(tau, rec["k_g16"], qn, np.linalg.norm(c32[rec["k_idx"]], axis=1), rho)
        err = np.abs(gl - s_or)
        assert np.all(err <= LOGIT_RTOL * scl), f"b{bits} qjl={qjl}: worst {float((err / scl).max()):.3g}"
        e = gl - s_exact
        mse[qjl] = float(np.mean(e * e))
        se = float(np.std(e) / math.sqrt(NP))
        _say(f"sweep b={bits} qjl={qjl}: logit parity worst {float((err / scl).max()):.2e} of the bar; "
             f"vs unquantised keys: bias {float(np.mean(e)):+.3e} (SE {se:.1e}), MSE {mse[qjl]:.3e}, "
             f"normalised MSE {mse[qjl] / float(np.mean(s_exact ** 2)):.3e}")
        del cache
    assert mse[True] < 0.85 * mse[False], f"b{bits}: QJL did not lower the logit MSE ({mse})"


def test_fullsize_octo_decode_workload(device):
    w = W.DECODE_32K
    H, T, G, bits = w.num_kv_heads, w.tokens, w.num_q_heads // w.num_kv_heads, w.bits_k
    kb, k64 = W.keys(w)                                    # [T][H][128]
    Kh = to_device(np.ascontiguousarray(np.swapaxes(kb, 0, 1)).reshape(H * T, 128), "bf16", device)
    rot = tq.tq_make_rotation(w.rot_seed, 128)
    tb = torch.empty(tq.tq_octo_table_bytes(bits), dtype=torch.uint8, device=device)
    tq.tq_octo_tables(bits, tb)
    rb = tq.tq_octo_record_bytes(128, bits)
    codes = torch.zeros((H, T, rb), dtype=torch.uint8, device=device)
    gamma = torch.zeros((H, T), dtype=torch.int16, device=device)
    _say("octo full size: encode", H * T, "keys")
    tq.tq_octo_encode(Kh, bits, rot, tb, codes.view(-1, rb), gamma.view(-1))
    _, q64 = W.queries(w)
    q = torch.from_numpy(q64[0].astype(np.float32).reshape(H, G, 128)).to(device)
    out = torch.empty((H, G, T), device=device)
    scale = 1.0 / math.sqrt(128)
    tq.tq_octo_logits(q, codes, gamma, bits, rot, tb, out, scale=scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(2024)
    hs, ts = rng.integers(0, H, 4096), rng.integers(0, T, 4096)
    rec = codes.cpu().numpy()[hs, ts]
    g16 = gamma.cpu().numpy().view(np.float16)[hs, ts]
    nmis = check_octo_codes(rec, g16, k64[ts, hs], bits, w.rot_seed)
    dirs, crho = O.octo_codebooks(128, bits)
    a, c, k = O.octo_unpack(rec, bits, 128)
    xh = O.octo_decode(a, c, k, g16, w.rot_seed, 128, dirs, crho)           # [4096][128]
    qf = q.cpu().numpy().astype(np.float64)[hs]                              # [4096][G][128]
    want = scale * np.einsum("sgd,sd->sg", qf, xh)
    got = out.cpu().numpy().astype(np.float64)[hs, :, ts]                    # [4096][G]
    csn = scale * np.linalg.norm(qf, axis=-1) * np.linalg.norm(xh, axis=-1)[:, None]
    assert np.all(np.abs(got - want) <= LOGIT_RTOL * csn + 1e-30)
    _say("  sampled codes off the oracle's pick (near ties):", nmis)


@pytest.mark.parametrize("qjl", [False, True])
def test_longest_sequence_at_the_split_limit(device, qjl):
    """The longest sequence decode-attend takes: 4096 splits of the largest
    split size, i.e. 4,194,304 blocks (67,108,859 tokens, a ragged last block;
    a 6.7 GB pool) without the QJL sidecar, and 262,144 blocks (4,194,299
    tokens) with it (the same matrix-core kernel, a shorter sequence: the
    vector kernel's old limit); one KV head with
    3-bit codes, 8 query heads; the merge folds 4096 partials per head in 32
    rounds.  Every key but five points against the queries (logits near
    -20), the five hot ones along them (near +20), so the other tokens carry
    a total softmax weight below 1e-8 and the output is the oracle's
    attention over the hot tokens.  Checked: the hot tokens' logits and the
    output against the oracle, and every other logit at least 30 below the
    hot ones."""
    bits, nblk = 3, 4096 * (64 if qjl else 1024)
    T = nblk * 16 - 5
    rng = np.random.default_rng(4096)
    e = rng.standard_normal(128)
    e /= np.linalg.norm(e)
    q64 = 15.0 * (e[None, :] + 0.05 * rng.standard_normal((8, 128)))
    q64 = (torch.from_numpy(q64.astype(np.float32)).double().numpy())[None]        # [1][8][128], f32 values
    split_tokens = 16 * nblk // 4096
    hot = np.array([0, T // 13 + 3, split_tokens * 2048, T // 5 * 3 + 17, T - 1], dtype=np.int64)   # one at a split's first token
    cold_k = torch.from_numpy((-15.0 * e).astype(np.float32)).to(device).to(torch.bfloat16)
    hot_k = torch.from_numpy((15.0 * e).astype(np.float32)).to(device).to(torch.bfloat16)
    vbank = torch.from_numpy(rng.standard_normal((1024, 128)).astype(np.float32)).to(device).to(torch.bfloat16)
    rot = tq.tq_make_rotation(42, 128)
    rot2 = tq.tq_make_rotation(43, 128) if qjl else None
    cfg = tq.make_config(1, nblk, bits, bits, rot, qjl, rot2)
    cache = tq.tq_cache_create(cfg, torch.zeros(tq.tq_cache_bytes(cfg), dtype=torch.uint8, device=device))
    cache._rots = (rot, rot2)
    _say("longest sequence:", T, "tokens,", tq.tq_cache_bytes(cfg), "pool bytes")
    step = 1 << 23
    for t0 in range(0, T, step):
        cnt = min(step, T - t0)
        idx = torch.arange(t0, t0 + cnt, device=device)
        K = cold_k.expand(cnt, 1, 128).contiguous()
        sel = hot[(hot >= t0) & (hot < t0 + cnt)] - t0
        if sel.size:
            K[torch.from_numpy(sel).to(device), 0] = hot_k
        V = vbank.index_select(0, idx % 1024).view(cnt, 1, 128)
        tq.tq_encode_kv(K, V, idx.to(torch.int32), bits, cache)
        torch.cuda.synchronize()
        del K, V, idx
    bt = torch.arange(nblk, dtype=torch.int32, device=device).view(1, nblk)
    lens = torch.tensor([T], dtype=torch.int32, device=device)
    q = torch.from_numpy(q64.astype(np.float32)).to(device)
    out = torch.full((1, 8, 128), float("nan"), device=device)
    logits = torch.empty((1, 8, nblk * 16), device=device)
    ws = tq.new_workspace(cache, 1, 8, nblk, device=device)
    tq.tq_decode_attend(q, cache, bt, lens, out, ws, logits_out=logits)
    torch.cuda.synchronize()
    # the hot tokens' codes from their blocks, and the oracle over them
    lay_full = O.LayoutV1(128, 1, bits, bits, qjl, nblk)
    view = cache.pool.view(nblk, 1, lay_full.block_bytes)
    arr = view.index_select(0, torch.from_numpy(hot // 16).to(device)).cpu().numpy()
    up = O.unpack_pool(arr, O.LayoutV1(128, 1, bits, bits, qjl, hot.size))
    r = hot % 16
    c32, _ = O.codebook_fp32(128, bits)
    khat = O.reconstruct(up["k_idx"][np.arange(hot.size), 0, r], up["k_g16"][np.arange(hot.size), 0, r], 42, c32)
    vhat = O.reconstruct(up["v_idx"][np.arange(hot.size), 0, r], up["v_g16"][np.arange(hot.size), 0, r], 42, c32)
    R = O.rotation_matrix(42, 128)
    tau = 1 / math.sqrt(128)
    hot_d = torch.from_numpy(hot).to(device)
    mask = torch.ones(nblk * 16, dtype=torch.bool, device=device)
    mask[hot_d] = False
    mask[T:] = False
    go = out.cpu().numpy().astype(np.float64)
    kg = up["k_g16"][np.arange(hot.size), 0, r]
    kidx = up["k_idx"][np.arange(hot.size), 0, r]
    qj = None
    if qjl:
        qj = dict(bits=up["qjl_bits"][np.arange(hot.size), 0, r], rho16=up["rho16"][np.arange(hot.size), 0, r],
                  gamma16=kg, seed=42, seed_qjl=43)
    for hq in range(8):
        s = O.logits(q64[0, hq], khat, qjl=qj)
        p = np.exp(s - s.max())
        o = (p / p.sum()) @ vhat
        scl = cs_scale(tau, kg, np.linalg.norm(R @ q64[0, hq]), np.linalg.norm(c32[kidx], axis=1),
                       qj["rho16"] if qj else None)
        gl_hot = logits[0, hq].index_select(0, hot_d).cpu().numpy().astype(np.float64)
        assert np.all(np.abs(gl_hot - s) <= LOGIT_RTOL * scl), hq
        cold_max = float(logits[0, hq][mask].max())
        assert cold_max <= float(s.min()) - 30.0, (hq, cold_max, float(s.min()))
        e_o = np.linalg.norm(go[0, hq] - o) / np.linalg.norm(o)
        assert e_o <= OUT_RTOL, (hq, e_o)
    _say("  hot logits", np.round(s, 2), "cold max", round(cold_max, 2))
    del cache, logits, ws, mask
    torch.cuda.empty_cache()
