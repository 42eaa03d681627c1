"""Margin of the bf16/fp16 argmax bar, predicted on the CPU for every low-precision workload.

The GPU kernels compute scores in fp32, take exponentials in fp32 against the row's running
maximum, round P to bf16 before the P V product on bf16 inputs with bf16 output (fp16 for
fp16 inputs), sum the rounded P in fp32, accumulate P V in fp32, divide, and round the output
to the input dtype. This test emulates exactly that rounding in numpy on the workloads' own
shapes and value distributions -- queries of the decode job at its prefixes (inputs scaled by
1/sqrt(128)), the saturated ring step (32760 keys), the multi-user chunk 15 (16384 keys,
causal in the chunk) and the three ragged skews -- and compares with the fp64 oracle under
the parity bar (max-abs <= 2e-2 and tie-aware argmax agreement >= 99.9%, ties counted as
agreement when the GPU's row maximum sits at the reference's argmax). It asserts that the predicted agreement clears 99.9% with room to spare
(>= 99.93% over >= 4000 rows), so that a GPU pass is not a coin flip. The emulation is test
code, not the oracle: the oracle never rounds."""
import numpy as np
import pytest
import torch

import seeded_inputs as SI
from oracle import attention as A
from tests.helpers import ARGMAX_MIN, LOWP_ATOL, argmax_agreement

LOG2E = 1.4426950408889634
MARGIN_RATE = 0.9993


def _round(x: np.ndarray, dtype: str) -> np.ndarray:
    t = {"bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(t).to(torch.float32).numpy()


def emulate(q, k, v, allowed, p_dtype, out_dtype):
    """What the kernels compute, in fp32: q [n, D], k/v [L, D] hold values exact in the input
    dtype; allowed [n, L]."""
    D = q.shape[1]
    c2 = np.float32(LOG2E / np.sqrt(D))
    s = q.astype(np.float32) @ k.astype(np.float32).T
    s = np.where(allowed, s, np.float32(-np.inf))
    m = s.max(axis=1, keepdims=True)
    p = np.exp2(s * c2 - m * c2).astype(np.float32)
    pr = _round(p, p_dtype)
    l = pr.sum(axis=1, keepdims=True, dtype=np.float32)
    o = (pr @ v.astype(np.float32)) / l
    return _round(o, out_dtype)


def _rows(q, k, v, allowed, p_dtype, out_dtype, block=256):
    got, want = [], []
    for r0 in range(0, q.shape[0], block):
        r1 = min(q.shape[0], r0 + block)
        got.append(emulate(q[r0:r1], k, v, allowed[r0:r1], p_dtype, out_dtype))
        ref, _ = A.attend_keys(q[r0:r1, None].astype(np.float64), k[:, None].astype(np.float64),
                               v[:, None].astype(np.float64), allowed[r0:r1])
        want.append(ref[:, 0])
    return np.concatenate(got), np.concatenate(want)


def _check(got, want, what):
    err = float(np.max(np.abs(got - want)))
    tie, strict = argmax_agreement(got, want)
    print(f"{what}: rows {len(got)} max_abs {err:.3g} tie-aware {tie:.5f} strict {strict:.5f}")
    assert len(got) >= 4000
    assert err <= LOWP_ATOL, (what, err)
    assert tie >= MARGIN_RATE > ARGMAX_MIN, (what, tie)
    return tie


def _key(workload, tensor, chunk=0):
    return SI.seed_key(workload, tensor, 0, 100 + chunk)


def _inputs(workload, n, L, dtype, std=1.0, chunk=0):
    q = SI.round_to(SI.normal_f32((n, 128), _key(workload, "q", chunk), std), dtype).float().numpy()
    k = SI.round_to(SI.normal_f32((L, 128), _key(workload, "k", chunk), std), dtype).float().numpy()
    v = SI.round_to(SI.normal_f32((L, 128), _key(workload, "v", chunk), std), dtype).float().numpy()
    return q, k, v


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_decode_job_margin(dtype):
    """Single queries over the decode job's prefixes (235 .. 1258 keys), inputs N(0,1)/sqrt(128):
    32 prefixes x 128 queries (the 4 query heads of a group share keys)."""
    W = SI.Decode()
    rates = []
    for j, L in enumerate(np.linspace(W.prompt + 1, W.prompt + W.steps, 32).astype(int)):
        q, k, v = _inputs("decode", 128, int(L), dtype, W.std, chunk=j)
        allowed = np.ones((128, int(L)), dtype=bool)
        got, want = _rows(q, k, v, allowed, dtype, dtype)
        rates.append((got, want))
    _check(np.concatenate([g for g, _ in rates]), np.concatenate([w for _, w in rates]), f"decode {dtype}")


def test_ring_saturated_margin():
    L = SI.Ring().n_slots * SI.Ring().C
    q, k, v = _inputs("ring", 4000, L, "bf16")
    got, want = _rows(q, k, v, np.ones((4000, L), dtype=bool), "bf16", "bf16")
    _check(got, want, "ring saturated (32760 keys)")


def test_multiuser_chunk15_margin():
    M = SI.MultiUser()
    # 4000 query rows of the last chunk (positions spread over it), causal inside the chunk
    t = np.linspace(0, M.chunk - 1, 4000).astype(int)
    q, k, v = _inputs("multiuser", 4000, M.cap, "bf16")
    allowed = np.stack([A.visible_keys(int(ti), M.chunk, M.cap, A.MASK_BLOCK_CAUSAL, M.block) for ti in t])
    got, want = _rows(q, k, v, allowed, "bf16", "bf16")
    _check(got, want, "multi-user chunk 15 (16384 keys, causal in chunk)")


@pytest.mark.parametrize("L", [512, 448, 256, 51])
def test_ragged_margin(L):
    q, k, v = _inputs("ragged", 8000, L, "bf16", chunk=L)
    got, want = _rows(q, k, v, np.ones((8000, L), dtype=bool), "bf16", "bf16")
    _check(got, want, f"ragged branch of {L} keys")


def test_a_planted_coarser_rounding_is_caught():
    """The emulation is sensitive: rounding P to 4 mantissa bits instead of bf16's 8 drops the
    predicted agreement below the margin on the ragged shape."""
    q, k, v = _inputs("ragged", 4000, 512, "bf16", chunk=7)
    D = q.shape[1]
    c2 = np.float32(LOG2E / np.sqrt(D))
    s = q @ k.T
    p = np.exp2(s * c2 - s.max(axis=1, keepdims=True) * c2).astype(np.float32)
    bits = p.view(np.uint32)
    p4 = ((bits + 0x40000) & 0xFFF80000).view(np.float32)  # 4 explicit mantissa bits
    o = _round((p4 @ v) / p4.sum(axis=1, keepdims=True), "bf16")
    ref, _ = A.attend_keys(q[:, None].astype(np.float64), k[:, None].astype(np.float64),
                           v[:, None].astype(np.float64), np.ones((4000, 512), dtype=bool))
    tie, _ = argmax_agreement(o, ref[:, 0])
    assert tie < MARGIN_RATE
