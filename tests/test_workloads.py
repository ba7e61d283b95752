"""Seeded input generators: shapes, determinism, bf16 rounding, paging."""

import numpy as np
import torch

from kv_cache_vector_encode_amd import workloads as W


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 37
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0]   # ties to even
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(W.bf16_bits(x), want)
    np.testing.assert_array_equal(W.bf16_to_f64(W.bf16_bits(x)),
                                  torch.from_numpy(x).to(torch.bfloat16).double().numpy())


def test_generators_are_deterministic_and_sliceable():
    w = W.DECODE_32K.with_(seq_len=300)
    a, a64 = W.keys(w)
    b, b64 = W.keys(w, 100, 50)
    assert a.shape == (300, 8, 128) and a.dtype == np.uint16
    assert np.array_equal(a[100:150], b)
    assert np.array_equal(a64[100:150], b64)
    v, _ = W.values(w)
    q, _ = W.queries(w)
    assert q.shape == (1, 64, 128)
    assert not np.array_equal(a, v)


def test_outlier_channels_and_tiny_case():
    w = W.DECODE_32K.with_(seq_len=4096)
    m = W.key_channel_scales(w)
    _, k = W.keys(w)
    for h in range(w.num_kv_heads):
        top2 = np.argsort(np.std(k[:, h], axis=0))[-2:]
        assert set(top2) == set(np.argsort(m[h])[-2:])
    t, t64 = W.keys(W.TINY)
    assert t.dtype == np.float32 and t.shape == (4096, 1, 128)
    big = np.std(t64[:, 0], axis=0) > 10
    assert big.sum() == 2


def test_paging_is_a_permutation_and_slots_agree():
    w = W.PREFILL_16x8K.with_(num_seqs=3, seq_len=100)
    bt = W.block_tables(w)
    assert bt.shape == (3, 7)
    assert sorted(bt.ravel().tolist()) == list(range(21))
    sm = W.slot_mapping(w)
    assert sm.shape == (300,)
    assert len(set(sm.tolist())) == 300
    for s in range(3):
        for t in (0, 15, 16, 99):
            assert sm[s * 100 + t] == bt[s, t // 16] * 16 + t % 16
