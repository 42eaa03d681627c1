"""Pins for oracle/ragged.py (packing of ragged K/V for variable-length cross-attention)."""
import numpy as np
import pytest

from oracle import attention as A
from oracle import ragged as R

rng = np.random.default_rng(1812)


def test_metadata_fixture():
    cu, mx = R.ragged_metadata([512, 448])
    assert cu.tolist() == [0, 512, 960] and mx == 512
    cu, mx = R.ragged_metadata([3, 0, 2])
    assert cu.tolist() == [0, 3, 3, 5] and mx == 3
    with pytest.raises(ValueError):
        R.ragged_metadata([2, -1])


def test_pack_fixture():
    """Rows labelled 100*b + t: the packed buffer lists branch 0's valid rows, then branch 1's."""
    B, L = 2, 4
    padded = (100 * np.arange(B)[:, None] + np.arange(L)[None, :]).astype(np.float64)[:, :, None]
    packed, cu = R.pack_ragged(padded, [3, 2])
    assert packed[:, 0].tolist() == [0, 1, 2, 100, 101]
    assert cu.tolist() == [0, 3, 5]
    with pytest.raises(ValueError):
        R.pack_ragged(padded, [5, 1])


@pytest.mark.parametrize("lens", [(512, 448), (512, 256), (512, 51), (7, 1), (1, 7, 3)])
def test_pack_then_packed_attention_equals_padded_prefix_attention(lens):
    """The three arms of the page agree: packed (cu_seqlens) attention over pack(padded) equals
    per-branch prefix attention over the padded buffer (seqused) and the padded-and-masked
    full-capacity attention -- different code paths of the oracle."""
    lens = [min(x, 64) for x in lens]  # keep the CPU case small
    B, L, Tq, Hq, Hkv, D = len(lens), 64, 5, 4, 2, 16
    q = rng.standard_normal((B, Tq, Hq, D))
    k = rng.standard_normal((B, L, Hkv, D))
    v = rng.standard_normal((B, L, Hkv, D))
    kp, cu = R.pack_ragged(k, lens)
    vp, cu2 = R.pack_ragged(v, lens)
    assert np.array_equal(cu, cu2) and kp.shape[0] == sum(lens)
    for b in range(B):
        np.testing.assert_array_equal(kp[cu[b]:cu[b + 1]], k[b, :lens[b]])
    o_p, l_p = A.attend_packed(q, kp, vp, cu)
    o_s, l_s = A.attend_batch_prefix(q, k, v, lens)
    assert np.max(np.abs(o_p - o_s)) <= 1e-13 and np.max(np.abs(l_p - l_s)) <= 1e-13
    for b in range(B):
        o_m, _ = A.attend_full_capacity_masked(q[b], k[b], v[b], lens[b])
        assert np.max(np.abs(o_m - o_p[b])) <= 1e-12


def test_planted_off_by_one_pack_is_caught(monkeypatch):
    real = R.pack_ragged

    def shifted(padded, lens):
        packed, cu = real(padded, lens)
        return np.roll(packed, 1, axis=0), cu
    monkeypatch.setattr(R, "pack_ragged", shifted)
    with pytest.raises(AssertionError):
        test_pack_then_packed_attention_equals_padded_prefix_attention((7, 1))
