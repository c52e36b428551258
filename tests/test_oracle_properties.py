"""Property tests of the fp64 oracle over random shapes, lengths and
chunkings (hypothesis), beside the fixed pins of test_oracle_pins.py.

* the split/merge twin equals the exact definition for any chunk length
  ([FD], *A faster attention for decoding: Flash-Decoding*: the chunks'
  outputs rescaled by their log-sum-exp give the exact attention);
* a joint permutation of a sequence's key/value rows changes nothing (the
  softmax is a sum over keys);
* rows past a sequence's length never matter, whatever they hold (NaN
  included);
* with scale 0 every key weighs the same: out = mean of the valid value
  rows, lse = ln L (empty sequences: out 0, lse -inf).
"""
import math

import numpy as np
import pytest

hyp = pytest.importorskip("hypothesis")
from hypothesis import HealthCheck, given, settings  # noqa: E402
from hypothesis import strategies as st  # noqa: E402

from long_context_decode_fd_amd import workloads as wl  # noqa: E402

SETTINGS = settings(max_examples=60, deadline=None,
                    suppress_health_check=[HealthCheck.function_scoped_fixture])


def rand_bf16(rng, shape, scale=1.0):
    return wl.bf16_bits((rng.standard_normal(shape) * scale).astype(
        np.float32))


@st.composite
def problems(draw):
    B = draw(st.integers(1, 3))
    Hkv = draw(st.integers(1, 3))
    G = draw(st.integers(1, 4))
    D = draw(st.sampled_from([8, 16, 64]))
    Lmax = draw(st.integers(1, 48))
    seqlens = np.array(draw(st.lists(st.integers(0, Lmax), min_size=B,
                                     max_size=B)), np.int32)
    seed = draw(st.integers(0, 2**32 - 1))
    rng = np.random.default_rng(seed)
    q = rand_bf16(rng, (B, Hkv * G, D))
    k = rand_bf16(rng, (B, Hkv, Lmax, D), 2.0)
    v = rand_bf16(rng, (B, Hkv, Lmax, D))
    scale = draw(st.sampled_from([0.05, 0.125, 0.3, 1.0]))
    return q, k, v, seqlens, scale, rng


def _close(o1, l1, o2, l2):
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-13)
    fin = np.isfinite(l1)
    assert np.array_equal(fin, np.isfinite(l2))
    assert np.all(l1[~fin] == l2[~fin])
    np.testing.assert_allclose(l2[fin], l1[fin], rtol=0, atol=1e-12)


@SETTINGS
@given(p=problems(), data=st.data())
def test_split_merge_equals_exact(oracle_mod, p, data):
    q, k, v, seqlens, scale, _ = p
    chunk = data.draw(st.integers(1, k.shape[2] + 5))
    o1, l1 = oracle_mod.decode(q, k, v, seqlens, scale)
    o2, l2 = oracle_mod.decode_split(q, k, v, seqlens, scale, chunk)
    _close(o1, l1, o2, l2)


@SETTINGS
@given(p=problems())
def test_joint_row_permutation_is_invisible(oracle_mod, p):
    q, k, v, seqlens, scale, rng = p
    k2, v2 = k.copy(), v.copy()
    for b, L in enumerate(seqlens):
        for g in range(k.shape[1]):
            perm = rng.permutation(int(L))
            k2[b, g, :L] = k[b, g, perm]
            v2[b, g, :L] = v[b, g, perm]
    o1, l1 = oracle_mod.decode(q, k, v, seqlens, scale)
    o2, l2 = oracle_mod.decode(q, k2, v2, seqlens, scale)
    _close(o1, l1, o2, l2)


@SETTINGS
@given(p=problems())
def test_rows_past_the_length_never_matter(oracle_mod, p):
    q, k, v, seqlens, scale, rng = p
    k2, v2 = k.copy(), v.copy()
    for b, L in enumerate(seqlens):
        junk = rng.integers(0, 1 << 16, size=k2[b, :, L:].shape,
                            dtype=np.uint16)
        junk.flat[::3] = 0xFFFF                 # NaN bits among them
        k2[b, :, L:] = junk
        v2[b, :, L:] = junk[..., ::-1]
    o1, l1 = oracle_mod.decode(q, k, v, seqlens, scale)
    o2, l2 = oracle_mod.decode(q, k2, v2, seqlens, scale)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@SETTINGS
@given(p=problems())
def test_scale_zero_gives_mean_of_values_and_ln_length(oracle_mod, p):
    q, k, v, seqlens, _, _ = p
    out, lse = oracle_mod.decode(q, k, v, seqlens, 0.0)
    G = q.shape[1] // k.shape[1]
    vf = wl.bf16_to_f32(v).astype(np.float64)
    for b, L in enumerate(seqlens):
        for h in range(q.shape[1]):
            if L == 0:
                assert np.all(out[b, h] == 0) and lse[b, h] == -np.inf
                continue
            mean = vf[b, h // G, :L].mean(axis=0)
            np.testing.assert_allclose(out[b, h], mean, rtol=1e-12,
                                       atol=1e-13)
            assert abs(lse[b, h] - math.log(L)) < 1e-12
