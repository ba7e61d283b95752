"""tq_decode_attend_noalloc (the split partials in the library's fixed
per-GPU scratch) against tq_decode_attend with a caller workspace: the same
kernels, so outputs and logits must be bit-identical.  Two calls in a row,
the second on a smaller input, so the second call meets the first one's
partials still in the scratch."""

import numpy as np
import pytest
import torch

from gpu_common import encode_gpu, to_device
from kv_cache_vector_encode_amd import tq
from kv_cache_vector_encode_amd import workloads as W


def _both(device, bits, hkv, group, lens, dtype="bf16"):
    w = W.DECODE_32K.with_(seed=9, num_seqs=len(lens), seq_len=max(lens), num_kv_heads=hkv,
                           num_q_heads=hkv * group, bits_k=bits, bits_v=bits)
    cache, _, _, _ = encode_gpu(w, device)
    bt = torch.from_numpy(W.block_tables(w)).to(device)
    qb, _ = W.queries(w)
    q = to_device(qb, "bf16", device)
    if dtype == "f32":
        q = q.float()
    lens_d = torch.tensor(lens, dtype=torch.int32, device=device)
    shape = (len(lens), w.num_q_heads)
    out_ws = torch.full(shape + (128,), float("nan"), device=device)
    out_na = torch.full_like(out_ws, float("nan"))
    lg_ws = torch.full(shape + (bt.shape[1] * 16,), float("nan"), device=device)
    lg_na = torch.full_like(lg_ws, float("nan"))
    ws = tq.new_workspace(cache, len(lens), w.num_q_heads, bt.shape[1], device=device)
    tq.tq_decode_attend(q, cache, bt, lens_d, out_ws, ws, logits_out=lg_ws)
    tq.tq_decode_attend_noalloc(q, cache, bt, lens_d, out_na, logits_out=lg_na)
    torch.cuda.synchronize()
    assert torch.isfinite(out_na).all()
    assert torch.equal(out_ws, out_na)
    for n, L in enumerate(lens):
        assert torch.equal(lg_ws[n, :, :L], lg_na[n, :, :L])
    return tq.tq_decode_workspace_bytes(cache, len(lens), w.num_q_heads, bt.shape[1])


@pytest.mark.gpu
def test_noalloc_decode_equals_workspace_decode_on_two_calls(device):
    print("noalloc: 3-bit, 3 sequences (1500, 700, 2100 tokens), then 4-bit, 2 sequences (300, 40)", flush=True)
    big = _both(device, 3, 2, 8, [1500, 700, 2100])
    small = _both(device, 4, 1, 8, [300, 40], dtype="f32")
    assert small < big <= tq.NOALLOC_SCRATCH_BYTES


@pytest.mark.gpu
def test_noalloc_rejects_partials_past_the_scratch(device):
    # 64 sequences of 131072 tokens, 8 KV heads: more partials than 16 MiB
    cache = tq.new_cache(8, 4, 4, 4, device=device)
    need = tq.tq_decode_workspace_bytes(cache, 64, 64, 8192)
    assert need > tq.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((64, 64, 128), dtype=torch.bfloat16, device=device)
    bt = torch.zeros((64, 8192), dtype=torch.int32, device=device)
    sl = torch.zeros(64, dtype=torch.int32, device=device)
    out = torch.zeros((64, 64, 128), device=device)
    with pytest.raises(tq.TQError) as e:
        tq.tq_decode_attend_noalloc(q, cache, bt, sl, out)
    assert e.value.status == tq.TQ_ERR_WORKSPACE
    assert "fixed scratch" in str(e.value)
