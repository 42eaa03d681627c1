"""Pins of oracle.rope against what the mathematics fixes (the pages print no RoPE formula or
worked example): the complex-multiplication form of a plane rotation, the relative-position
property that defines rotary embeddings, identity at position 0, inversion by the negative
angle, norm preservation, the fixed permutation between the two pair layouts, the dtype
rounding against torch's own conversion, and ring positions that follow chunk chronology."""
import numpy as np
import pytest
import torch

from oracle import cache as Cc
from oracle import rope as R

RNG = np.random.default_rng(1234)


def freqs(D, base=10000.0):
    return base ** (-np.arange(D // 2) * 2.0 / D)


def rand_x(T, H, D):
    return RNG.standard_normal((T, H, D))


@pytest.mark.parametrize("layout", [R.LAYOUT_HALF, R.LAYOUT_INTERLEAVED])
def test_complex_multiplication_form(layout):
    T, H, D = 7, 3, 16
    x = rand_x(T, H, D)
    pos = RNG.integers(0, 50000, T)
    f = freqs(D)
    first, second = R.pair_indices(D, layout)
    z = x[..., first] + 1j * x[..., second]
    w = z * np.exp(1j * (pos[:, None, None].astype(np.float64) * f[None, None, :]))
    got = R.rope_rotate(x, pos, f, layout)
    assert np.allclose(got[..., first], w.real, rtol=0, atol=1e-12)
    assert np.allclose(got[..., second], w.imag, rtol=0, atol=1e-12)


@pytest.mark.parametrize("layout", [R.LAYOUT_HALF, R.LAYOUT_INTERLEAVED])
def test_scores_depend_only_on_relative_position(layout):
    D = 64
    f = freqs(D)
    q = rand_x(1, 1, D)
    k = rand_x(1, 1, D)
    for m, n in [(5, 2), (1000, 997), (40000, 39997), (3, 0)]:
        a = np.dot(R.rope_rotate(q, [m], f, layout).ravel(), R.rope_rotate(k, [n], f, layout).ravel())
        b = np.dot(R.rope_rotate(q, [m - n], f, layout).ravel(), k.ravel())
        assert abs(a - b) < 1e-9, (m, n, a, b)


@pytest.mark.parametrize("layout", [R.LAYOUT_HALF, R.LAYOUT_INTERLEAVED])
def test_identity_at_zero_inverse_and_norms(layout):
    T, H, D = 5, 2, 32
    x = rand_x(T, H, D)
    f = freqs(D)
    assert np.array_equal(R.rope_rotate(x, np.zeros(T, dtype=np.int64), f, layout), x)
    pos = RNG.integers(0, 60000, T)
    y = R.rope_rotate(x, pos, f, layout)
    back = R.rope_rotate(y, -pos, f, layout)
    assert np.allclose(back, x, rtol=0, atol=1e-12)
    first, second = R.pair_indices(D, layout)
    assert np.allclose(x[..., first] ** 2 + x[..., second] ** 2,
                       y[..., first] ** 2 + y[..., second] ** 2, rtol=1e-13, atol=0)
    # a pair with frequency 0 is left alone; the other coordinates are rotated
    f0 = f.copy()
    f0[3] = 0.0
    y0 = R.rope_rotate(x, pos, f0, layout)
    assert np.array_equal(y0[..., first[3]], x[..., first[3]])
    assert not np.allclose(y0[..., first[4]], x[..., first[4]])


def test_layouts_related_by_a_fixed_permutation():
    T, H, D = 4, 2, 16
    x = rand_x(T, H, D)
    pos = RNG.integers(0, 9000, T)
    f = freqs(D)
    # perm moves coordinate pair (i, i + D/2) to (2i, 2i + 1)
    perm = np.empty(D, dtype=np.int64)
    perm[0::2] = np.arange(D // 2)
    perm[1::2] = np.arange(D // 2) + D // 2
    half = R.rope_rotate(x, pos, f, R.LAYOUT_HALF)
    inter = R.rope_rotate(x[..., perm], pos, f, R.LAYOUT_INTERLEAVED)
    assert np.array_equal(inter, half[..., perm])


@pytest.mark.parametrize("dtype,tdt", [("bf16", torch.bfloat16), ("f16", torch.float16)])
def test_rounding_matches_torch_conversion(dtype, tdt):
    x = np.concatenate([RNG.standard_normal(20000) * s for s in (1e-3, 1.0, 300.0)])
    # exact ties of the fp32 -> bf16 step, both parities
    ties = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 2.0 + 2 ** -7])
    x = np.concatenate([x, ties])
    want = torch.from_numpy(x.astype(np.float32)).to(tdt).to(torch.float64).numpy()
    assert np.array_equal(R.round_cache(x, dtype), want)
    # the fp64 -> fp32 step rounds first (double rounding is part of the reading)
    y = np.array([1.0 + 2 ** -8 + 2 ** -30])
    assert R.round_cache(y, "bf16")[0] == torch.tensor(np.float32(y[0])).to(torch.bfloat16).item()


def test_ring_positions_follow_chronology_not_slots():
    """Keys carry the position of their chunk in time since reset; after wraparound the slot
    no longer tells it (the planted variant, positions by slot, must differ)."""
    n_slots, sink, C, H, D = 4, 1, 3, 2, 8
    f = freqs(D)
    ring = Cc.RingPhysical(n_slots, sink, C, (H, D))
    raw = {}
    for cid in range(7):
        ring.reserve()
        raw[cid] = rand_x(C, H, D)
        ring.write(R.rope_keys(raw[cid], R.ring_positions(cid, C), f, R.LAYOUT_HALF, "f32"))
    retained = sorted(c for c in ring.slot_chunk if c is not None)
    assert retained == [0, 4, 5, 6]
    for s, cid in enumerate(ring.slot_chunk):
        stored = ring.storage[s * C:(s + 1) * C]
        assert np.array_equal(stored, R.rope_keys(raw[cid], R.ring_positions(cid, C), f,
                                                  R.LAYOUT_HALF, "f32"))
        planted = R.rope_keys(raw[cid], R.ring_positions(s, C), f, R.LAYOUT_HALF, "f32")
        assert (s == cid) == np.array_equal(stored, planted)
