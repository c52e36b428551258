"""The seeded input generator: determinism, shapes, padding, bf16 rounding."""
import numpy as np
import pytest

from long_context_decode_fd_amd import workloads as wl


def test_bf16_rounding_is_nearest_even_like_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e30).astype(np.float32),
        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.4e38, -3.4e38,
                  1e-40, np.inf, -np.inf], np.float32)])
    ours = wl.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy()
    np.testing.assert_array_equal(ours, ref.view(np.uint16))
    nan = wl.bf16_bits(np.array([np.nan], np.float32))
    assert np.isnan(wl.bf16_to_f32(nan)).all()


def test_generation_is_deterministic_and_slab_local():
    w = wl.WORKLOADS["b4_mha_h32_d128_l32768_peaked"].with_(Lmax=256, B=2,
                                                             Hq=2, Hkv=2)
    q1, k1, v1, _ = wl.gen_all(w)
    q2 = wl.gen_q(w)
    k2, v2 = wl.gen_slab(w, 1, 1)
    np.testing.assert_array_equal(q1, q2)
    np.testing.assert_array_equal(k1[1, 1], k2)
    np.testing.assert_array_equal(v1[1, 1], v2)
    assert not np.array_equal(k1[0, 0], k1[0, 1])


def test_peaked_rows_are_exactly_scaled():
    w = wl.WORKLOADS["b4_mha_h32_d128_l32768_peaked"].with_(Lmax=1000)
    rows = wl.peak_rows(w, 0, 3, 1000)
    assert rows.size == 10 and np.unique(rows).size == 10
    plain = w.with_(peak_frac=0.0)
    kp, _ = wl.gen_slab(w, 0, 3)
    k0, _ = wl.gen_slab(plain, 0, 3)
    f = wl.bf16_to_f32
    np.testing.assert_array_equal(f(kp[rows]), f(k0[rows]) * 8)
    mask = np.ones(1000, bool); mask[rows] = False
    np.testing.assert_array_equal(kp[mask], k0[mask])


def test_varlen_seqlens_and_nan_padding():
    w = wl.WORKLOADS["varlen_b16_gqa8_h64_d128_lmax131072"]
    s = wl.gen_seqlens(w)
    assert s.dtype == np.int32 and s.shape == (16,)
    assert s.min() >= 1024 and s.max() <= 131072
    small = w.with_(Lmax=64, B=2, Hq=2, Hkv=1, varlen=(8, 64))
    sl = wl.gen_seqlens(small)
    k, v = wl.gen_slab(small, 0, 0, sl)
    L = int(sl[0])
    assert np.all(k[L:] == 0xFFFF) and np.all(v[L:] == 0xFFFF)
    assert np.isfinite(wl.bf16_to_f32(k[:L])).all()


def test_algorithmic_bytes_of_batch1_64k():
    w = wl.WORKLOADS["b1_gqa8_h64_d128_l65536"]
    assert wl.algorithmic_bytes(w) == 268_468_480
    assert wl.flops(w) == 4 * 65536 * 64 * 128


def test_first_batch_entries_are_the_smaller_workload():
    # bench.py's CPU baseline times the first entries of a large batch as
    # the same workload with a smaller B: that must give identical inputs.
    w = wl.WORKLOADS["varlen_b16_gqa8_h64_d128_lmax131072"].with_(
        Lmax=512, Hq=8, varlen=(8, 512))
    ws = w.with_(B=3)
    np.testing.assert_array_equal(wl.gen_seqlens(w)[:3], wl.gen_seqlens(ws))
    np.testing.assert_array_equal(wl.gen_q(w)[:3], wl.gen_q(ws))
    sl = wl.gen_seqlens(w)
    for b in range(3):
        k1, v1 = wl.gen_slab(w, b, 1, sl)
        k2, v2 = wl.gen_slab(ws, b, 1, wl.gen_seqlens(ws))
        np.testing.assert_array_equal(k1, k2)
        np.testing.assert_array_equal(v1, v2)


@pytest.mark.parametrize("hm", [False, True])
@pytest.mark.parametrize("P,sls", [(16, [100, 0, 37]), (64, [200, 200, 65]),
                                   (48, [1, 144, 150])])
def test_page_pools_hold_each_row_once_and_nan_elsewhere(P, sls, hm):
    torch = pytest.importorskip("torch")
    w = wl.Workload("pages", B=3, Hq=4, Hkv=2, D=64, Lmax=200,
                    dtype="bf16", seed=9, page_size=P, head_major=hm)
    sl = np.array(sls, np.int32)
    bt = wl.gen_block_table(w)
    assert bt.shape == (3, w.max_pages)
    assert np.unique(bt).size == bt.size and bt.min() >= 0
    assert bt.max() < w.num_pages and w.num_pages > bt.size
    q, k, v, _ = wl.gen_all(w.with_(varlen=None))
    for b in range(3):              # rows past the length are NaN bits
        k[b, :, sl[b]:] = wl.BF16_NAN
        v[b, :, sl[b]:] = wl.BF16_NAN
    kp, vp = wl.scatter_pages(w, k, v, bt, sl)
    owned = np.zeros(w.num_pages * P * 2, bool)
    for b in range(3):
        for j in range(int(sl[b])):
            pg, t = bt[b, j // P], j % P
            for g in range(2):
                r = (pg * 2 + g) * P + t if hm else (pg * P + t) * 2 + g
                np.testing.assert_array_equal(kp.reshape(-1, 64)[r],
                                              k[b, g, j])
                np.testing.assert_array_equal(vp.reshape(-1, 64)[r],
                                              v[b, g, j])
                owned[r] = True
    assert np.all(kp.reshape(-1, 64)[~owned] == wl.BF16_NAN)
    assert np.all(vp.reshape(-1, 64)[~owned] == wl.BF16_NAN)
    # the torch scatter (used on the device for large pools) agrees
    qd, kd, vd, btd, sld, sl2, bt2 = wl.device_paged_inputs(w, sl,
                                                            device="cpu")
    np.testing.assert_array_equal(bt2, bt)
    np.testing.assert_array_equal(btd.numpy(), bt)
    np.testing.assert_array_equal(sld.numpy(), sl)
    np.testing.assert_array_equal(
        kd.view(torch.int16).numpy().view(np.uint16), kp)
    np.testing.assert_array_equal(
        vd.view(torch.int16).numpy().view(np.uint16), vp)
    np.testing.assert_array_equal(
        qd.view(torch.int16).numpy().view(np.uint16), q)


def test_multi_token_queries_extend_the_q_stream():
    w = wl.EXTRA_WORKLOADS["mq4_b64_gqa4_h32_d128_l4096"]
    q = wl.gen_q(w)
    assert q.shape == (64, 4, 32, 128)
    one = wl.gen_q(w.with_(Tq=1))
    assert one.shape == (64, 32, 128)
    # the first B*Hq*D draws are the single-token q
    np.testing.assert_array_equal(q.reshape(-1)[:one.size], one.reshape(-1))
    base = wl.WORKLOADS["b64_gqa4_h32_d128_l4096"]
    assert wl.algorithmic_bytes(w) - wl.algorithmic_bytes(base) == \
        3 * (2 * 64 * 32 * 128 * 2 + 4 * 64 * 32)


def test_threaded_generation_matches_one_slab_at_a_time():
    w = wl.WORKLOADS["varlen_b16_gqa8_h64_d128_lmax131072"].with_(
        B=3, Hq=8, Hkv=4, Lmax=300, varlen=(20, 300))
    seqlens = np.array([300, 0, 77], np.int32)
    q, k, v, _ = wl.gen_all(w, seqlens=seqlens, threads=4)
    slabs = list(wl.iter_slabs(w, seqlens, threads=3))
    assert [(b, g) for b, g, *_ in slabs] == [(b, g) for b in range(3)
                                              for g in range(4)]
    for b, g, L, kr, vr in slabs:
        assert L == int(seqlens[b])
        k1, v1 = wl.gen_slab(w, b, g, seqlens)
        np.testing.assert_array_equal(k[b, g], k1)
        np.testing.assert_array_equal(v[b, g], v1)
        np.testing.assert_array_equal(kr, k1[:L])
        np.testing.assert_array_equal(vr, v1[:L])
    k_serial = wl.gen_all(w, seqlens=seqlens, threads=1)[1]
    np.testing.assert_array_equal(k, k_serial)


def test_fp16_inputs_are_the_same_draws_rounded_to_fp16():
    torch = pytest.importorskip("torch")
    w = wl.WORKLOADS["varlen_b16_gqa8_h64_d128_lmax131072"].with_(
        B=3, Hq=4, Hkv=2, Lmax=300, varlen=(1, 300))
    wh = w.with_(dtype="f16")
    q, k, v, sl = wl.gen_all(w)
    qh, kh, vh, slh = wl.gen_all(wh)
    np.testing.assert_array_equal(sl, slh)
    assert qh.dtype == np.float16 and kh.dtype == np.float16
    assert wh.elem_bytes == 2
    # the same float32 draws, rounded to nearest even as torch rounds them
    x = _f32_of_generator(w)
    np.testing.assert_array_equal(
        qh.view(np.uint16),
        torch.from_numpy(x).to(torch.float16).numpy().view(np.uint16))
    for b in range(w.B):
        L = int(sl[b])
        for arr_h, arr_b in ((kh, k), (vh, v)):
            # valid rows: fp16 of the value whose bf16 rounding the bf16
            # workload holds; padding: NaN
            assert np.all(np.isnan(arr_h[b, :, L:]))
            assert not np.isnan(arr_h[b, :, :L]).any()
            near = np.abs(arr_h[b, :, :L].astype(np.float32)
                          - wl.bf16_to_f32(arr_b[b, :, :L]))
            assert near.max() <= 2.0 ** -7 * max(
                1.0, float(np.abs(arr_h[b, :, :L].astype(np.float32)).max()))


def _f32_of_generator(w):
    """q's float32 draws, from the generator's own stream."""
    shape = (w.B, w.Hq, w.D)
    return wl._rng(w.seed, 0).standard_normal(shape, dtype=np.float32)
