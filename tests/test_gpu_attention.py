"""Fused attention forward against the fp64 oracle (oracle/attention.c):
every element on small, ragged and causal shapes that span several query and
key tiles, sampled rows of the full 16k-token workload in the launch the
benchmark times, the exact case of identical keys, and the edge cases (no
keys, queries beyond the keys under the causal mask, one row, one key).

Acceptance is the oracle's ``check_attention`` bound: the probabilities'
bf16 rounding, the fp32 score error through exp, fp32 sums, and for bf16
output half a bf16 ulp ("B200 TMEM Lifecycle Planner", section A2 trigger 2
and section E: the S, P and O tiles of attention on the matrix cores)."""
import sys

import numpy as np
import pytest
import torch

import matrix_core_engineering_amd as mce
import oracle
from matrix_core_engineering_amd.inputs import (ATTENTION_WORKLOADS, OUT_BF16, OUT_F32,
                                                attention_inputs)
from helpers import bf16_bits_to_f64, f64_to_bf16_bits

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
GUARD = 64                   # sentinel elements on each side of O
SENTINEL_F32 = 0x7F8ABCDE
SENTINEL_BF16 = 0x7F8B
NAN_F32 = 0x7FC00000
NAN_BF16 = 0x7FC0


def announce(msg):
    sys.__stderr__.write(f"[gpu] {msg}\n")
    sys.__stderr__.flush()


def dev16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV)


class AttnRun:
    """Q, K, V on the device; O inside a buffer with sentinel guard bands and
    NaN in every logical element, so an unwritten element is caught."""

    def __init__(self, shape, q, k, v, o_dtype):
        B, H, S, T, D = shape
        self.shape, self.o_dtype = shape, o_dtype
        self.n = B * H * S * D
        self.Q, self.K, self.V = dev16(q), dev16(k), dev16(v)
        if o_dtype == OUT_F32:
            host = np.full(self.n + 2 * GUARD, SENTINEL_F32, np.uint32)
            host[GUARD:GUARD + self.n] = NAN_F32
            self.O = torch.from_numpy(host.view(np.int32)).to(DEV)
            self.esize = 4
        else:
            host = np.full(self.n + 2 * GUARD, SENTINEL_BF16, np.uint16)
            host[GUARD:GUARD + self.n] = NAN_BF16
            self.O = torch.from_numpy(host.view(np.int16)).to(DEV)
            self.esize = 2

    def run(self, scale, causal):
        B, H, S, T, D = self.shape
        return mce.attention_bf16(B, H, S, T, D, self.Q.data_ptr(), self.K.data_ptr(),
                                  self.V.data_ptr(), self.O.data_ptr() + GUARD * self.esize,
                                  self.o_dtype, scale, causal, raise_on_error=False)

    def result(self):
        torch.cuda.synchronize()
        raw = self.O.cpu().numpy()
        B, H, S, T, D = self.shape
        if self.o_dtype == OUT_F32:
            raw = raw.view(np.uint32)
            sent = SENTINEL_F32
            vals = raw[GUARD:GUARD + self.n].view(np.float32).astype(np.float64)
        else:
            raw = raw.view(np.uint16)
            sent = SENTINEL_BF16
            vals = bf16_bits_to_f64(raw[GUARD:GUARD + self.n])
        guards_ok = bool(np.all(raw[:GUARD] == sent) and np.all(raw[GUARD + self.n:] == sent))
        return vals.reshape(B * H * S, D), raw[GUARD:GUARD + self.n], guards_ok


def run_and_check(shape, causal, o_dtype, seed=0, std=1.0, scale=None, rows=None):
    B, H, S, T, D = shape
    q, k, v = attention_inputs(B, H, S, T, D, seed=seed, std=std)
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    r = AttnRun(shape, q, k, v, o_dtype)
    st = r.run(scale, causal)
    assert st == mce.MCE_OK, mce.gemm_status_string(st)
    vals, _, guards_ok = r.result()
    assert guards_ok, "a write landed outside O"
    assert not np.any(np.isnan(vals)), "an element of O was left unwritten (or is NaN)"
    ranges = rows if rows is not None else [(0, B * H * S)]
    worst = 0.0
    for r0, r1 in ranges:
        oref, pv, smax = oracle.attention(B, H, S, T, D, q, k, v, np.float32(scale), causal, r0, r1)
        ok, w, bad = oracle.check_attention(vals[r0:r1], oref, pv, smax, T, o_dtype == OUT_BF16)
        if not ok:
            err = np.abs(vals[r0:r1] - oref)
            i, d = np.unravel_index(np.argmax(err), err.shape)
            pytest.fail(f"{shape} causal={causal} rows {r0}..{r1 - 1}: {bad} out of bound, worst "
                        f"{w:.3g}; e.g. O[{r0 + i},{d}]={vals[r0 + i, d]!r} ref={oref[i, d]!r}")
        worst = max(worst, w)
    return worst, vals


SHAPES = [
    (1, 1, 1, 1, 64),           # one query, one key
    (1, 1, 1, 1, 128),
    (1, 2, 130, 70, 64),        # ragged query and key tails
    (2, 3, 200, 333, 128),
    (1, 1, 257, 513, 128),      # three query tiles, nine key tiles
    (1, 1, 64, 64, 64),
    (2, 1, 128, 1000, 64),      # long keys, one query tile
    (1, 2, 700, 130, 128),      # queries beyond the keys
]


@pytest.mark.parametrize("o_dtype", [OUT_F32, OUT_BF16])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_every_element(shape, causal, o_dtype):
    announce(f"attention {shape} causal={causal} out={o_dtype}")
    run_and_check(shape, causal, o_dtype, seed=sum(shape) + causal)


def test_no_keys_gives_zeros():
    announce("attention without keys")
    shape = (1, 2, 150, 0, 128)
    B, H, S, T, D = shape
    q, _, _ = attention_inputs(B, H, S, 1, D, seed=3)
    r = AttnRun(shape, q, np.zeros(8, np.uint16), np.zeros(8, np.uint16), OUT_F32)
    assert r.run(0.1, False) == mce.MCE_OK
    vals, _, guards_ok = r.result()
    assert guards_ok and np.all(vals == 0.0)


def test_causal_rows_without_keys_are_zero():
    """seq_q > seq_k under the causal mask: the first seq_q - seq_k rows see
    no key and are written as zeros; row seq_q - seq_k sees key 0 only and
    is exactly its value row."""
    announce("attention causal rows without keys")
    shape = (1, 1, 300, 100, 64)
    B, H, S, T, D = shape
    q, k, v = attention_inputs(B, H, S, T, D, seed=4)
    r = AttnRun(shape, q, k, v, OUT_F32)
    assert r.run(0.125, True) == mce.MCE_OK
    vals, _, guards_ok = r.result()
    assert guards_ok
    assert np.all(vals[:S - T] == 0.0)
    assert np.array_equal(vals[S - T], bf16_bits_to_f64(v.reshape(T, D)[0]))


@pytest.mark.parametrize("o_dtype", [OUT_F32, OUT_BF16])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("zero_q", [True, False])
def test_identical_keys_average_the_values(D, o_dtype, zero_q):
    """Every key the same: every score of a row is the same number, so every
    probability is the same and o is the mean of the value rows (integer
    values, 256 keys, 300 queries: a ragged query tail).  With zero queries
    the scores are exactly 0, every probability exactly 1 and o exact in
    fp32.  With random queries the kernel subtracts the row maximum inside
    one fma of the unrounded scaled score, so the probabilities are
    exp2(delta) with delta the rounding error of the scaled score (below
    2^-24 of it): o is the mean within a few fp32 ulps."""
    announce(f"attention identical keys D={D} zero_q={zero_q}")
    S, T = 300, 256
    g = torch.Generator().manual_seed(5)
    q = torch.zeros(1, 1, S, D) if zero_q else torch.randn(1, 1, S, D, generator=g)
    k = torch.randn(1, 1, 1, D, generator=g).expand(1, 1, T, D).contiguous()
    v = torch.randint(-8, 9, (1, 1, T, D), generator=g).float()
    qb, kb, vb = (f64_to_bf16_bits(x.double().numpy()) for x in (q, k, v))
    r = AttnRun((1, 1, S, T, D), qb, kb, vb, o_dtype)
    assert r.run(0.3, False) == mce.MCE_OK
    vals, raw, guards_ok = r.result()
    assert guards_ok
    mean = np.broadcast_to(v.numpy().reshape(T, D).astype(np.float64).mean(0), (S, D))
    if zero_q and o_dtype == OUT_F32:
        assert np.array_equal(vals, mean)
    elif zero_q:
        assert np.array_equal(raw.reshape(S, D), f64_to_bf16_bits(mean))
    elif o_dtype == OUT_F32:
        assert np.all(np.abs(vals - mean) <= 4 * 2.0 ** -24 * np.abs(mean))
    else:
        assert np.all(np.abs(vals - mean) <= 2.0 ** -8 * np.abs(mean) * (1 + 2.0 ** -16))


@pytest.mark.parametrize("scale", [0.0, -0.2, 1.0])
def test_scales(scale):
    """Zero scale (uniform probabilities), a negative scale, and scores of
    tens (std 2 inputs, unit scale): the running maximum keeps exp in
    range."""
    announce(f"attention scale {scale}")
    run_and_check((1, 2, 200, 300, 128), False, OUT_F32, seed=6,
                  std=2.0 if scale == 1.0 else 1.0, scale=scale)


@pytest.mark.parametrize("name", sorted(ATTENTION_WORKLOADS))
def test_full_workload_sampled_rows(name):
    """The 16k-token workload in the benchmark's launch (bf16 out): every
    element written, no NaN; against the oracle on the first, middle and
    last query tiles of the first and last (batch, head)."""
    w = ATTENTION_WORKLOADS[name]
    shape = (w["batch"], w["heads"], w["seq_q"], w["seq_k"], w["dim"])
    announce(f"attention workload {name} {shape}")
    S = w["seq_q"]
    last = (w["batch"] * w["heads"] - 1) * S
    rows = [(0, 128), (S // 2 - 64, S // 2 + 64), (S - 128, S), (last, last + 64),
            (last + S - 64, last + S)]
    run_and_check(shape, w["causal"], OUT_BF16, seed=7, rows=rows)


def test_unsupported_on_device():
    announce("attention unsupported cases")
    q = torch.zeros(4096, dtype=torch.int16, device=DEV)
    o = torch.zeros(4096, dtype=torch.int16, device=DEV)
    p = q.data_ptr()
    args = (1, 1, 4, 4)
    assert mce.attention_bf16(*args, 96, p, p, p, o.data_ptr(), OUT_BF16, 0.1, 0,
                              raise_on_error=False) == mce.MCE_EUNSUPPORTED
    assert mce.attention_bf16(*args, 64, p + 8, p, p, o.data_ptr(), OUT_BF16, 0.1, 0,
                              raise_on_error=False) == mce.MCE_EUNSUPPORTED
    assert mce.attention_bf16(*args, 64, p, p, p, o.data_ptr() + 4, OUT_BF16, 0.1, 0,
                              raise_on_error=False) == mce.MCE_EUNSUPPORTED
