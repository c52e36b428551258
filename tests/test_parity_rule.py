"""The comparison rule itself (tests/parity.py), on the CPU: what it must
accept and what it must refuse."""
import numpy as np

from long_context_decode_fd_amd import workloads as wl
from parity import check_lse, check_out


def _bf(x):
    return wl.bf16_bits(np.asarray(x, np.float32))


def _far_neighbour(ref):
    """The bf16 value on the other side of ref from its nearest one."""
    near = wl.bf16_to_f32(_bf(ref)).astype(np.float64)
    # step a whole bf16 ulp: move the float32 bit pattern by 0x10000
    u = near.astype(np.float32).view(np.uint32)
    toward = np.where((ref > near) == (near > 0), u + 0x10000, u - 0x10000)
    return toward.astype(np.uint32).view(np.float32).astype(np.float64)


def test_nearest_bf16_always_passes():
    rng = np.random.default_rng(0)
    ref = np.concatenate([rng.uniform(-8, 8, 20000), [0.0, 4.0, -7.99]])
    ok, rep = check_out(_bf(ref), ref, "bf16")
    assert ok, rep


def test_far_neighbour_fails_where_half_an_ulp_exceeds_the_bound():
    rng = np.random.default_rng(1)
    ref = rng.uniform(4.0, 8.0, 5000) * rng.choice([-1, 1], 5000)
    far = _far_neighbour(ref)
    assert np.all(np.abs(far - ref) > 1e-2)
    for r, f in zip(ref[:200], far[:200]):
        assert not check_out(_bf([f]), np.array([r]), "bf16")[0], (r, f)


def test_below_four_the_bound_is_the_plain_max_abs():
    rng = np.random.default_rng(2)
    ref = rng.uniform(-3.99, 3.99, 5000)
    off = ref + rng.choice([-1, 1], 5000) * 1.2e-2
    # a bf16 value more than 1e-2 away fails even if it brackets ref
    g = _bf(off)
    gf = wl.bf16_to_f32(g).astype(np.float64)
    bad = np.abs(gf - ref) > 1e-2
    assert bad.any()
    for r, gi in zip(ref[bad][:200], g[bad][:200]):
        assert not check_out(np.array([gi]), np.array([r]), "bf16")[0]


def test_fp32_and_special_values():
    ref = np.array([1.0, np.nan, -np.inf, 0.25])
    assert check_out(np.array([1.009, np.nan, -np.inf, 0.25], np.float32),
                     ref, "f32")[0]
    assert not check_out(np.array([1.011, np.nan, -np.inf, 0.25],
                                  np.float32), ref, "f32")[0]
    assert not check_out(np.array([1.0, 0.0, -np.inf, 0.25], np.float32),
                         ref, "f32")[0]
    assert not check_out(np.array([1.0, np.nan, np.inf, 0.25], np.float32),
                         ref, "f32")[0]
    assert check_lse(np.array([2.0009, -np.inf]), np.array([2.0, -np.inf]))[0]
    assert not check_lse(np.array([2.0011]), np.array([2.0]))[0]
    assert not check_lse(np.array([-np.inf]), np.array([-50.0]))[0]


def test_fp16_nearest_value_passes_and_far_ones_fail():
    rng = np.random.default_rng(3)
    # numpy's float64 -> float16 conversion rounds to nearest even
    ref = np.concatenate([rng.uniform(-60, 60, 20000), [0.0, 32.0, -63.9]])
    ok, rep = check_out(ref.astype(np.float16), ref, "f16")
    assert ok, rep
    # below 32 the bound is the plain 1e-2: 0.012 away fails
    small = rng.uniform(-31.9, 31.9, 2000)
    off = (small + 0.012 * np.sign(small)).astype(np.float16)
    bad = np.abs(off.astype(np.float64) - small) > 1e-2
    assert bad.any()
    for r, g in zip(small[bad][:200], off[bad][:200]):
        assert not check_out(np.array([g]), np.array([r]), "f16")[0], (r, g)
    # from 32 on (ulp 2^-5) correct rounding is the bound: the nearest
    # fp16 value passes, the next one beyond it fails
    big = rng.uniform(32.0, 64.0, 2000)
    near = big.astype(np.float16)
    far = np.where(near.astype(np.float64) < big,
                   np.nextafter(near, np.float16(np.inf)),
                   np.nextafter(near, np.float16(-np.inf)))
    assert check_out(near, big, "f16")[0]
    assert np.all(np.abs(far.astype(np.float64) - big) > 1e-2)
    for r, f in zip(big[:200], far[:200]):
        assert not check_out(np.array([f]), np.array([r]), "f16")[0], (r, f)


def test_fp16_rule_needs_fp16_results():
    import pytest
    with pytest.raises(AssertionError):
        check_out(np.array([1.0], np.float32), np.array([1.0]), "f16")
