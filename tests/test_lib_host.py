"""Host side of libtq (no GPU needed): exported symbols, seeded signs,
codebooks against the oracle, layout sizes, argument validation."""

import ctypes

import numpy as np
import pytest

from kv_cache_vector_encode_amd import tq
from oracle import tq_oracle as O


def test_library_exports_every_declared_symbol():
    L = tq.lib()
    names = tq.declared_functions()
    assert len(names) >= 17
    for n in names:
        assert hasattr(L, n), n
    assert L.tq_layout_version() == tq.LAYOUT_VERSION


def test_status_strings():
    assert tq.status_string(0) == "TQ_OK"
    assert tq.status_string(-3) == "TQ_ERR_BITS_MISMATCH"
    assert tq.status_string(-99) == "TQ_ERR_UNKNOWN"


@pytest.mark.parametrize("seed", [0, 1, 42, 43, 2 ** 63 + 5, 2 ** 64 - 1])
@pytest.mark.parametrize("d", [2, 16, 128, 1024])
def test_rotation_signs_match_oracle(seed, d):
    r = tq.tq_make_rotation(seed, d)
    assert np.array_equal(tq.tq_rotation_signs(r), O.rotation_signs(seed, d))


def test_rotation_rejects_bad_dimensions():
    for d in (0, 1, 3, 100, 8192):
        with pytest.raises(tq.TQError) as e:
            tq.tq_make_rotation(1, d)
        assert e.value.status == tq.TQ_ERR_INVALID_ARG


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_codebook_bitwise_equal_to_oracle(d, bits):
    # the library's float64 Lloyd-Max (trig-substitution CDF) and the oracle's
    # (scipy incomplete beta) are independent; their fp32 roundings must agree
    c, t = tq.tq_codebook(d, bits)
    oc, ot = O.codebook_fp32(d, bits)
    assert np.array_equal(c.astype(np.float64), oc)
    assert np.array_equal(t.astype(np.float64), ot)


def test_codebook_rejects_bad_bits():
    for b in (0, 5):
        with pytest.raises(tq.TQError) as e:
            tq.tq_codebook(128, b)
        assert e.value.status == tq.TQ_ERR_UNSUPPORTED


@pytest.mark.parametrize("hkv,bk,bv,qjl", [(8, 4, 4, False), (8, 3, 3, False), (16, 2, 0, True),
                                           (1, 4, 0, False), (3, 2, 2, True)])
def test_layout_matches_oracle_spec(hkv, bk, bv, qjl):
    r = tq.tq_make_rotation(42, 128)
    rq = tq.tq_make_rotation(43, 128)
    cfg = tq.make_config(hkv, 37, bk, bv, r, qjl, rq if qjl else None)
    lay = tq.tq_cache_layout_query(cfg)
    ol = O.LayoutV1(128, hkv, bk, bv, qjl, 37)
    assert lay.block_bytes == ol.block_bytes
    assert (lay.off_k, lay.off_v, lay.off_gamma_k) == (ol.off_k, ol.off_v, ol.off_gk)
    if bv:
        assert lay.off_gamma_v == ol.off_gv
    if qjl:
        assert (lay.off_rho, lay.off_sign) == (ol.off_rho, ol.off_sig)
    assert tq.tq_cache_bytes(cfg) == ol.pool_bytes
    # the pages' bit budget per token-head
    assert 8 * (lay.k_rec_bytes + 2) == O.bits_per_vector(128, bk)


def test_config_validation():
    r = tq.tq_make_rotation(42, 128)
    bad = [
        (dict(bits_k=5), tq.TQ_ERR_UNSUPPORTED), (dict(bits_k=1), tq.TQ_ERR_UNSUPPORTED),
        (dict(bits_v=1), tq.TQ_ERR_UNSUPPORTED), (dict(bits_v=3), tq.TQ_ERR_UNSUPPORTED),
        (dict(d=64), tq.TQ_ERR_UNSUPPORTED), (dict(block_size=32), tq.TQ_ERR_UNSUPPORTED),
        (dict(num_kv_heads=0), tq.TQ_ERR_INVALID_ARG), (dict(num_blocks=0), tq.TQ_ERR_INVALID_ARG),
        (dict(num_blocks=2 ** 62), tq.TQ_ERR_INVALID_ARG), (dict(layout_version=2), tq.TQ_ERR_UNSUPPORTED),
        (dict(qjl=2), tq.TQ_ERR_INVALID_ARG),
    ]
    for kw, want in bad:
        cfg = tq.make_config(8, 4, 4, 4, r)
        for k, v in kw.items():
            setattr(cfg, k, v)
        assert tq.lib().tq_cache_bytes(ctypes.byref(cfg)) == want, kw


def _fake_cache(**kw):
    # a descriptor bound to a fake (never dereferenced) 16-byte aligned pool
    r = tq.tq_make_rotation(42, 128)
    args = dict(num_kv_heads=8, num_blocks=4, bits_k=4, bits_v=4)
    args.update(kw)
    cfg = tq.make_config(args["num_kv_heads"], args["num_blocks"], args["bits_k"], args["bits_v"], r)
    c = tq.tq_cache_create(cfg, 0x100000)
    c._rots = (r,)
    return c


def test_cache_create_validation():
    r = tq.tq_make_rotation(42, 128)
    cfg = tq.make_config(8, 4, 4, 4, r)
    h = ctypes.c_void_p()
    assert tq.lib().tq_cache_create(ctypes.byref(cfg), None, ctypes.byref(h)) == tq.TQ_ERR_INVALID_ARG
    assert tq.lib().tq_cache_create(ctypes.byref(cfg), 0x100004, ctypes.byref(h)) == tq.TQ_ERR_INVALID_ARG
    cfg.rot = None
    assert tq.lib().tq_cache_create(ctypes.byref(cfg), 0x100000, ctypes.byref(h)) == tq.TQ_ERR_INVALID_ARG
    cfg = tq.make_config(8, 4, 4, 0, r, qjl=True, rot_qjl=None)
    assert tq.lib().tq_cache_create(ctypes.byref(cfg), 0x100000, ctypes.byref(h)) == tq.TQ_ERR_INVALID_ARG
    # rotations may be destroyed after create: the descriptor copies the signs
    r2 = tq.tq_make_rotation(42, 128)
    cfg = tq.make_config(8, 4, 4, 4, r2)
    c = tq.tq_cache_create(cfg, 0x100000)
    del r2
    assert c.handle


def test_encode_argument_checks_happen_before_the_device():
    c = _fake_cache()
    L = tq.lib()
    K, V, sm = 0x200000, 0x300000, 0x400000
    assert L.tq_encode_kv(K, V, 2, 10, sm, 3, c.handle, None) == tq.TQ_ERR_BITS_MISMATCH
    assert L.tq_encode_kv(K, None, 2, 10, sm, 4, c.handle, None) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_encode_kv(K, V, 7, 10, sm, 4, c.handle, None) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_encode_kv(K, V, 2, -1, sm, 4, c.handle, None) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_encode_kv(K, V, 2, 0, sm, 4, c.handle, None) == tq.TQ_OK      # nothing to do
    assert L.tq_encode_kv(None, V, 2, 10, sm, 4, c.handle, None) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_encode_kv(K, V, 2, 10, sm, 4, None, None) == tq.TQ_ERR_INVALID_ARG
    ko = _fake_cache(bits_v=0)
    assert L.tq_encode_kv(K, V, 2, 10, sm, 4, ko.handle, None) == tq.TQ_ERR_INVALID_ARG
    assert "keys-only" in L.tq_last_error().decode()


def test_decode_argument_checks_and_workspace_size():
    c = _fake_cache()
    L = tq.lib()
    q, bt, sl, out, ws = 0x200000, 0x300000, 0x400000, 0x500000, 0x600000
    need = L.tq_decode_workspace_bytes(c.handle, 2, 64, 100)
    assert need > 0
    # group 64/8 = 8: splits of 4..64 blocks, 130 floats per (split, head)
    assert L.tq_decode_workspace_bytes(c.handle, 2, 60, 100) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_decode_attend(q, 2, c.handle, bt, sl, 2, 60, 100, 0.0, out, None, ws, need, None) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_decode_attend(q, 2, c.handle, bt, sl, 2, 64 * 3, 100, 0.0, out, None, ws, need, None) == tq.TQ_ERR_UNSUPPORTED
    assert L.tq_decode_attend(q, 2, c.handle, bt, sl, 2, 64, 100, 0.0, out, None, ws, need - 1, None) == tq.TQ_ERR_WORKSPACE
    assert L.tq_decode_attend(q, 2, c.handle, bt, sl, 2, 64, 100, 0.0, out, None, None, need, None) == tq.TQ_ERR_WORKSPACE
    assert L.tq_decode_attend(q, 9, c.handle, bt, sl, 2, 64, 100, 0.0, out, None, ws, need, None) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_decode_attend(q, 2, c.handle, bt, sl, 0, 64, 100, 0.0, out, None, ws, need, None) == tq.TQ_OK
    ko = _fake_cache(bits_v=0)
    assert L.tq_decode_attend(q, 2, ko.handle, bt, sl, 2, 64, 100, 0.0, out, None, ws, need, None) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_decode_logits(q, 2, c.handle, bt, sl, 2, 64, 100, 0.0, None, None) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_reconstruct(c.handle, bt, 5, 2, out, None) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_reconstruct(ko.handle, bt, 5, 1, out, None) == tq.TQ_ERR_INVALID_ARG


def test_no_device_is_reported_without_touching_memory():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    c = _fake_cache()
    st = tq.lib().tq_encode_kv(0x200000, 0x300000, 2, 10, 0x400000, 4, c.handle, None)
    assert st == tq.TQ_ERR_NO_DEVICE


def test_qjl_attend_split_sizes_for_long_sequences():
    # Caches with the QJL sidecar take the matrix-core decode-attend kernel
    # at every width, so their splits are those of the caches without it
    # (at most 1024 blocks, up to 4096 splits per sequence and KV head)
    r, rq = tq.tq_make_rotation(42, 128), tq.tq_make_rotation(43, 128)
    L = tq.lib()
    for bits in (2, 3, 4):
        c = tq.tq_cache_create(tq.make_config(8, 4, bits, bits, r, qjl=True, rot_qjl=rq), 0x100000)
        p = tq.tq_cache_create(tq.make_config(8, 4, bits, bits, r), 0x100000)
        c._rots = p._rots = (r, rq)
        for ns, mb in ((4, 8192), (1, 2048), (16, 512), (1, 1024 * 4096)):
            n = L.tq_decode_workspace_bytes(c.handle, ns, 64, mb)
            assert n > 0 and n == L.tq_decode_workspace_bytes(p.handle, ns, 64, mb), (bits, ns, mb)
        assert L.tq_decode_workspace_bytes(c.handle, 1, 64, 1024 * 4096 + 1) == tq.TQ_ERR_UNSUPPORTED


def test_matrix_core_attend_split_sizes():
    # Splits of the matrix-core decode-attend kernel (values, no QJL): aim
    # at one round of workgroups, two 8-wave ones per CU (512); when that
    # leaves splits of at most 32 blocks, aim at half as many with whole
    # block pairs per wave (multiples of 16 blocks); never more than 64
    # block pairs per wave (a wave keeps its pairs' block-table entries one
    # per lane): 1024 blocks.
    r = tq.tq_make_rotation(42, 128)
    c = tq.tq_cache_create(tq.make_config(8, 4, 4, 4, r), 0x100000)
    c._rots = (r,)
    c3 = tq.tq_cache_create(tq.make_config(8, 4, 3, 3, r), 0x100000)
    c3._rots = (r,)
    L = tq.lib()
    per = 8 * 132 * 4   # 8 query heads of the group, 132 floats each
    # 1 x 32768 tokens: 2048 blocks, 8 units -> 32 blocks -> short: 64 blocks -> 32 splits
    assert L.tq_decode_workspace_bytes(c.handle, 1, 64, 2048) == 1 * 8 * 32 * per
    # 16 x 8192 tokens: 512 blocks, 128 units -> 128 blocks -> 4 splits
    assert L.tq_decode_workspace_bytes(c.handle, 16, 64, 512) == 16 * 8 * 4 * per
    # 4 x 131072 tokens: 8192 blocks, 32 units -> 512 blocks -> 16 splits
    assert L.tq_decode_workspace_bytes(c.handle, 4, 64, 8192) == 4 * 8 * 16 * per
    # 3-bit codes: 512 workgroups -> 512 blocks -> 16 splits
    assert L.tq_decode_workspace_bytes(c3.handle, 4, 64, 8192) == 4 * 8 * 16 * per
    # 3-bit, 1 x 32768 tokens: 2048 blocks, 8 units -> 32 blocks -> short: 64 blocks -> 32 splits
    assert L.tq_decode_workspace_bytes(c3.handle, 1, 64, 2048) == 1 * 8 * 32 * per
    assert L.tq_decode_workspace_bytes(c3.handle, 1, 64, 1024 * 4096) == 1 * 8 * 4096 * per
    assert L.tq_decode_workspace_bytes(c3.handle, 1, 64, 1024 * 4096 + 1) == tq.TQ_ERR_UNSUPPORTED
    # the 1024-block cap and the 4096-split limit
    assert L.tq_decode_workspace_bytes(c.handle, 1, 64, 1024 * 4096) == 1 * 8 * 4096 * per
    assert L.tq_decode_workspace_bytes(c.handle, 1, 64, 1024 * 4096 + 1) == tq.TQ_ERR_UNSUPPORTED


def test_decompress_argument_checks_happen_before_the_device():
    c = _fake_cache()
    L = tq.lib()
    sl, Ko, Vo = 0x200000, 0x300000, 0x400000
    assert L.tq_decompress_kv(None, sl, 10, tq.TQ_BF16, Ko, Vo, None) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_decompress_kv(c.handle, sl, -1, tq.TQ_BF16, Ko, Vo, None) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_decompress_kv(c.handle, sl, 10, tq.TQ_F32, Ko, Vo, None) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_decompress_kv(c.handle, sl, 10, tq.TQ_BF16, Ko + 8, Vo, None) == tq.TQ_ERR_INVALID_ARG
    assert "aligned" in L.tq_last_error().decode()
    assert L.tq_decompress_kv(c.handle, None, 10, tq.TQ_F16, Ko, Vo, None) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_decompress_kv(c.handle, sl, 0, tq.TQ_BF16, Ko, Vo, None) == tq.TQ_OK       # nothing to do
    assert L.tq_decompress_kv(c.handle, sl, 10, tq.TQ_BF16, None, None, None) == tq.TQ_OK  # no outputs
    ko = _fake_cache(bits_v=0)
    assert L.tq_decompress_kv(ko.handle, sl, 10, tq.TQ_BF16, Ko, Vo, None) == tq.TQ_ERR_INVALID_ARG
    assert "keys-only" in L.tq_last_error().decode()


def test_decode_step_argument_checks_happen_before_the_device():
    c = _fake_cache()
    L = tq.lib()
    q, K, V, bt, sl, out, ws = 0x200000, 0x300000, 0x400000, 0x500000, 0x600000, 0x700000, 0x800000

    def step(cache, kv_dtype=tq.TQ_BF16, Kp=K, Vp=V, ns=2, wsb=1 << 30):
        return L.tq_decode_step(q, tq.TQ_BF16, Kp, Vp, kv_dtype, cache, bt, sl, ns, 64, 8, 0.0, out, None, ws, wsb,
                                None)

    assert step(None) == tq.TQ_ERR_INVALID_ARG
    assert step(c.handle, kv_dtype=7) == tq.TQ_ERR_INVALID_ARG
    assert step(c.handle, Kp=None) == tq.TQ_ERR_INVALID_ARG
    assert step(c.handle, Vp=V + 4) == tq.TQ_ERR_INVALID_ARG
    assert "aligned" in L.tq_last_error().decode()
    assert step(c.handle, wsb=16) == tq.TQ_ERR_WORKSPACE
    assert step(c.handle, ns=0) == tq.TQ_OK   # nothing to do
    assert step(_fake_cache(bits_v=0).handle) == tq.TQ_ERR_INVALID_ARG
    r, r2 = tq.tq_make_rotation(42, 128), tq.tq_make_rotation(43, 128)
    qc = tq.tq_cache_create(tq.make_config(8, 4, 4, 4, r, True, r2), 0x100000)
    assert step(qc.handle) == tq.TQ_ERR_UNSUPPORTED


def test_minmax_argument_checks_happen_before_the_device():
    L = tq.lib()
    r = tq.tq_make_rotation(42, 128)
    r64 = tq.tq_make_rotation(42, 64)
    X, cd, pr, out = 0x200000, 0x300000, 0x400000, 0x500000
    assert L.tq_minmax_encode(X, tq.TQ_BF16, 10, 4, None, cd, pr, None) == tq.TQ_ERR_UNSUPPORTED
    assert L.tq_minmax_encode(X, tq.TQ_BF16, 10, 4, r64.handle, cd, pr, None) == tq.TQ_ERR_UNSUPPORTED
    assert L.tq_minmax_encode(X, tq.TQ_BF16, 10, 5, r.handle, cd, pr, None) == tq.TQ_ERR_UNSUPPORTED
    assert L.tq_minmax_encode(X, 9, 10, 4, r.handle, cd, pr, None) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_minmax_encode(X, tq.TQ_BF16, -1, 4, r.handle, cd, pr, None) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_minmax_encode(X + 8, tq.TQ_BF16, 10, 4, r.handle, cd, pr, None) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_minmax_encode(X, tq.TQ_BF16, 10, 4, r.handle, None, pr, None) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_minmax_encode(X, tq.TQ_BF16, 0, 4, r.handle, cd, pr, None) == tq.TQ_OK      # nothing to do
    assert L.tq_minmax_decode(cd, pr, 10, 3, r.handle, 9, out, None) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_minmax_decode(cd, pr + 2, 10, 3, r.handle, tq.TQ_F32, out, None) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_minmax_decode(cd, pr, 10, 1, r.handle, tq.TQ_F32, out, None) == tq.TQ_ERR_UNSUPPORTED
    assert L.tq_minmax_decode(cd, pr, 0, 3, r.handle, tq.TQ_F32, out, None) == tq.TQ_OK


# --------------------------------------------------------- triplet codec ----

@pytest.mark.parametrize("bits", [2, 3, 4])
def test_octo_tables_match_oracle(bits):
    # C++ (double trig and a trig-substitution CDF for rho) against the
    # oracle (numpy trig, scipy incomplete beta): the fp32 tables agree to
    # the last bit except where two float64 paths round apart (one ulp)
    dirs, rho = tq.tq_octo_codebook(128, bits)
    od, orho = O.octo_codebooks(128, bits)
    nd = 1 << (bits + 1)
    assert dirs.shape == (nd * nd, 4) and np.all(dirs[:, 3] == 0)
    got = dirs[:, :3].reshape(nd, nd, 3)
    want = od.astype(np.float32)
    ulp = np.spacing(np.abs(want))
    assert np.all(np.abs(got - want) <= ulp)
    assert np.mean(got == want) > 0.99
    assert np.all(np.abs(rho - orho.astype(np.float32)) <= np.spacing(orho.astype(np.float32)))


def test_octo_sizes_and_argument_checks_happen_before_the_device():
    assert [tq.tq_octo_record_bytes(128, b) for b in (2, 3, 4)] == [40, 56, 72]
    assert [tq.tq_octo_record_bytes(128, b) for b in (2, 3, 4)] == [O.octo_record_bytes(128, b) for b in (2, 3, 4)]
    assert [tq.tq_octo_table_bytes(b) for b in (2, 3, 4)] == [1024, 4096, 16384]
    L = tq.lib()
    assert L.tq_octo_record_bytes(64, 4) == tq.TQ_ERR_UNSUPPORTED
    assert L.tq_octo_table_bytes(5) == tq.TQ_ERR_UNSUPPORTED
    r = tq.tq_make_rotation(42, 128)
    r64 = tq.tq_make_rotation(42, 64)
    X, cd, g, tb, q, out = 0x200000, 0x300000, 0x400000, 0x500000, 0x600000, 0x700000
    assert L.tq_octo_encode(X, tq.TQ_BF16, 10, 4, r64.handle, tb, 16384, cd, g, None) == tq.TQ_ERR_UNSUPPORTED
    assert L.tq_octo_encode(X, tq.TQ_BF16, 10, 1, r.handle, tb, 16384, cd, g, None) == tq.TQ_ERR_UNSUPPORTED
    assert L.tq_octo_encode(X, tq.TQ_BF16, 10, 4, r.handle, None, 16384, cd, g, None) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_octo_encode(X, tq.TQ_BF16, 10, 4, r.handle, tb + 4, 16384, cd, g, None) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_octo_encode(X, 7, 10, 4, r.handle, tb, 16384, cd, g, None) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_octo_encode(X + 8, tq.TQ_BF16, 10, 4, r.handle, tb, 16384, cd, g, None) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_octo_encode(X, tq.TQ_BF16, 10, 4, r.handle, tb, 16384, cd + 4, g, None) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_octo_encode(X, tq.TQ_BF16, 0, 4, r.handle, tb, 16384, cd, g, None) == tq.TQ_OK
    assert L.tq_octo_logits(q, cd, g, 8, 17, 100, 4, r.handle, tb, 16384, 0.1, out, None) == tq.TQ_ERR_UNSUPPORTED
    assert L.tq_octo_logits(q, cd, g, 0, 8, 100, 4, r.handle, tb, 16384, 0.1, out, None) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_octo_logits(q, cd, g, 8, 8, 100, 4, r.handle, tb, 16384, float("nan"), out, None) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_octo_logits(q + 4, cd, g, 8, 8, 100, 4, r.handle, tb, 16384, 0.1, out, None) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_octo_logits(q, cd, g, 8, 8, 0, 4, r.handle, tb, 16384, 0.1, out, None) == tq.TQ_OK
    assert L.tq_octo_logits(q, cd, g, 8, 8, -1, 4, r.handle, tb, 16384, 0.1, out, None) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_octo_tables(4, None, None) == tq.TQ_ERR_INVALID_ARG
    # a table filled for fewer bits is too small for b = 4
    assert L.tq_octo_encode(X, tq.TQ_BF16, 10, 4, r.handle, tb, 4096, cd, g, None) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_octo_logits(q, cd, g, 8, 8, 100, 4, r.handle, tb, 1024, 0.1, out, None) == tq.TQ_ERR_INVALID_ARG


def test_octo_qjl_argument_checks_happen_before_the_device():
    L = tq.lib()
    r = tq.tq_make_rotation(42, 128)
    r2 = tq.tq_make_rotation(43, 128)
    r64 = tq.tq_make_rotation(42, 64)
    X, cd, g, tb, q, out, sg, rh = 0x200000, 0x300000, 0x400000, 0x500000, 0x600000, 0x700000, 0x800000, 0x900000
    enc = L.tq_octo_encode_qjl
    assert enc(X, tq.TQ_BF16, 10, 4, r.handle, None, tb, 16384, cd, g, sg, rh, None) == tq.TQ_ERR_UNSUPPORTED
    assert enc(X, tq.TQ_BF16, 10, 4, r.handle, r64.handle, tb, 16384, cd, g, sg, rh, None) == tq.TQ_ERR_UNSUPPORTED
    assert enc(X, tq.TQ_BF16, 10, 4, r.handle, r2.handle, tb, 16384, cd, g, None, rh, None) == tq.TQ_ERR_INVALID_ARG
    assert enc(X, tq.TQ_BF16, 10, 4, r.handle, r2.handle, tb, 16384, cd, g, sg, None, None) == tq.TQ_ERR_INVALID_ARG
    assert enc(X, tq.TQ_BF16, 10, 4, r.handle, r2.handle, tb, 16384, cd, g, sg + 8, rh, None) == tq.TQ_ERR_INVALID_ARG
    assert enc(X, tq.TQ_BF16, 10, 4, r.handle, r2.handle, tb, 16384, cd, g, sg, rh + 1, None) == tq.TQ_ERR_INVALID_ARG
    assert enc(X, tq.TQ_BF16, 0, 4, r.handle, r2.handle, tb, 16384, cd, g, sg, rh, None) == tq.TQ_OK
    lg = L.tq_octo_logits_qjl
    assert lg(q, cd, g, sg, rh, 8, 8, 100, 4, r.handle, None, tb, 16384, 0.1, out, None) == tq.TQ_ERR_UNSUPPORTED
    assert lg(q, cd, g, None, rh, 8, 8, 100, 4, r.handle, r2.handle, tb, 16384, 0.1, out, None) == tq.TQ_ERR_INVALID_ARG
    assert lg(q, cd, g, sg + 4, rh, 8, 8, 100, 4, r.handle, r2.handle, tb, 16384, 0.1, out, None) == tq.TQ_ERR_INVALID_ARG
    assert lg(q, cd, g, sg, rh, 8, 17, 100, 4, r.handle, r2.handle, tb, 16384, 0.1, out, None) == tq.TQ_ERR_UNSUPPORTED
    assert lg(q, cd, g, sg, rh, 8, 8, 0, 4, r.handle, r2.handle, tb, 16384, 0.1, out, None) == tq.TQ_OK


def test_octo_attend_argument_checks_happen_before_the_device():
    L = tq.lib()
    r = tq.tq_make_rotation(42, 128)
    q, kc, kg, vc, vg, tb, out, ws = (0x200000 + 0x100000 * i for i in range(8))
    need = L.tq_octo_attend_workspace_bytes(8, 8, 100)
    # 100 keys of 8 heads: one 128-key split per head, one partial of 8 queries
    assert need == 8 * 1 * 8 * 132 * 4
    assert L.tq_octo_attend_workspace_bytes(0, 8, 100) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_octo_attend_workspace_bytes(8, 17, 100) == tq.TQ_ERR_INVALID_ARG
    at = L.tq_octo_attend
    assert at(q, kc, kg, vc, vg, 8, 8, 100, 4, r.handle, tb, 16384, 0.1, out, ws, need - 1, None) == tq.TQ_ERR_WORKSPACE
    assert at(q, kc, kg, vc, vg, 8, 17, 100, 4, r.handle, tb, 16384, 0.1, out, ws, need, None) == tq.TQ_ERR_UNSUPPORTED
    assert at(q, kc, kg, vc, vg, 8, 8, 100, 5, r.handle, tb, 16384, 0.1, out, ws, need, None) == tq.TQ_ERR_UNSUPPORTED
    assert at(q, kc, kg, None, vg, 8, 8, 100, 4, r.handle, tb, 16384, 0.1, out, ws, need, None) == tq.TQ_ERR_INVALID_ARG
    assert at(q, kc, kg, vc, vg, 8, 8, 100, 4, r.handle, tb, 16384, 0.1, out + 4, ws, need, None) == tq.TQ_ERR_INVALID_ARG
    assert at(q, kc, kg, vc, vg, 8, 8, 100, 4, r.handle, tb, 16384, float("inf"), out, ws, need, None) == tq.TQ_ERR_INVALID_ARG
    # splits stay whole 128-key chunks and at most 1024 per head
    for heads, n in ((1, 1), (8, 32768), (1, 1 << 24), (64, 131072)):
        b = L.tq_octo_attend_workspace_bytes(heads, 1, n)
        nsplit = b // (heads * 132 * 4)
        assert 1 <= nsplit <= 1024 and nsplit * heads * 132 * 4 == b


def test_noalloc_decode_checks_happen_before_the_device():
    # the allocation-free decode takes tq_decode_attend's arguments minus the
    # workspace; a call whose split partials would not fit the fixed 16 MiB
    # scratch is refused before any device call
    c = _fake_cache()
    L = tq.lib()
    q, bt, sl, out = 0x200000, 0x300000, 0x400000, 0x500000
    need = L.tq_decode_workspace_bytes(c.handle, 64, 64, 8192)
    assert need > tq.NOALLOC_SCRATCH_BYTES == 16 << 20
    assert L.tq_decode_attend_noalloc(q, 2, c.handle, bt, sl, 64, 64, 8192, 0.0, out, None, None) == tq.TQ_ERR_WORKSPACE
    assert "fixed scratch" in L.tq_last_error().decode()
    assert L.tq_decode_attend_noalloc(q, 9, c.handle, bt, sl, 2, 64, 100, 0.0, out, None, None) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_decode_attend_noalloc(q, 2, c.handle, bt, sl, 2, 60, 100, 0.0, out, None, None) == tq.TQ_ERR_INVALID_ARG
    assert L.tq_decode_attend_noalloc(q, 2, c.handle, bt, sl, 0, 64, 100, 0.0, out, None, None) == tq.TQ_OK
    ko = _fake_cache(bits_v=0)
    assert L.tq_decode_attend_noalloc(q, 2, ko.handle, bt, sl, 2, 64, 100, 0.0, out, None, None) == tq.TQ_ERR_INVALID_ARG
