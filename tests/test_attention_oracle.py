"""Pins of the fp64 attention oracle (oracle/attention.c) against closed
forms, invariances and an independent float64 computation, and of its
acceptance bound from both sides.  CPU only."""
import numpy as np
import pytest
import torch

import oracle


def bits(x):
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def vals(b):
    return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).double()


def run(q, k, v, scale, causal=False):
    B, H, S, D = q.shape
    T = k.shape[2]
    return oracle.attention(B, H, S, T, D, bits(q), bits(k), bits(v), scale, causal)


def reference(q, k, v, scale, causal):
    """The definition in float64 by torch (bf16-rounded inputs)."""
    qd, kd, vd = q.to(torch.bfloat16).double(), k.to(torch.bfloat16).double(), v.to(torch.bfloat16).double()
    s = (qd @ kd.transpose(-1, -2)) * float(np.float32(scale))
    S, T = s.shape[-2:]
    if causal:
        i = torch.arange(S)[:, None]
        j = torch.arange(T)[None, :]
        s = s.masked_fill(j > i + T - S, float("-inf"))
    p = torch.softmax(s, -1)
    p = torch.nan_to_num(p, nan=0.0)      # rows with no visible key
    o = p @ vd
    return o.reshape(-1, q.shape[-1]).numpy(), (p @ vd.abs()).reshape(-1, q.shape[-1]).numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 1, 1, 1, 8), (2, 3, 7, 7, 16), (1, 2, 5, 9, 64),
                                   (1, 1, 9, 5, 32), (2, 1, 33, 65, 128)])
def test_matches_float64_definition(shape, causal):
    B, H, S, T, D = shape
    g = torch.Generator().manual_seed(sum(shape) + causal)
    q = torch.randn(B, H, S, D, generator=g)
    k = torch.randn(B, H, T, D, generator=g)
    v = torch.randn(B, H, T, D, generator=g)
    scale = 1.0 / np.sqrt(D)
    o, pv, smax = run(q, k, v, scale, causal)
    ro, rpv = reference(q, k, v, scale, causal)
    assert np.allclose(o, ro, rtol=1e-12, atol=1e-13)
    assert np.allclose(pv, rpv, rtol=1e-12, atol=1e-13)


def test_single_key_returns_its_value():
    g = torch.Generator().manual_seed(1)
    q = torch.randn(1, 2, 4, 16, generator=g)
    k = torch.randn(1, 2, 1, 16, generator=g)
    v = torch.randn(1, 2, 1, 16, generator=g)
    o, pv, _ = run(q, k, v, 0.7)
    want = np.repeat(vals(bits(v)).numpy().reshape(2, 16), 4, axis=0)
    assert np.array_equal(o, want)
    assert np.array_equal(pv, np.abs(want))


def test_equal_keys_average_the_values():
    """Identical keys: every probability is 1/T, so o is the mean of the
    value rows (exact here: integer values, T a power of two)."""
    T, D = 16, 8
    g = torch.Generator().manual_seed(2)
    q = torch.randn(1, 1, 3, D, generator=g)
    k = torch.randn(1, 1, 1, D, generator=g).expand(1, 1, T, D).contiguous()
    v = torch.randint(-8, 9, (1, 1, T, D), generator=g).float()
    o, _, _ = run(q, k, v, 0.5)
    assert np.array_equal(o, np.repeat(v.numpy().reshape(T, D).mean(0)[None], 3, axis=0))


def test_key_permutation_invariance():
    g = torch.Generator().manual_seed(3)
    q = torch.randn(1, 1, 6, 32, generator=g)
    k = torch.randn(1, 1, 20, 32, generator=g)
    v = torch.randn(1, 1, 20, 32, generator=g)
    perm = torch.randperm(20, generator=g)
    o1, _, s1 = run(q, k, v, 0.2)
    o2, _, s2 = run(q, k[:, :, perm], v[:, :, perm], 0.2)
    assert np.allclose(o1, o2, rtol=1e-13, atol=1e-14)
    assert np.array_equal(s1, s2)


def test_softmax_shift_invariance():
    """A key component constant over keys shifts every score of a row by the
    same amount: changing the query's matching component leaves o."""
    g = torch.Generator().manual_seed(4)
    q = torch.randn(1, 1, 5, 16, generator=g)
    k = torch.randn(1, 1, 12, 16, generator=g)
    v = torch.randn(1, 1, 12, 16, generator=g)
    k[..., 3] = 2.0
    q2 = q.clone()
    q2[..., 3] += 8.0
    o1, _, _ = run(q, k, v, 0.3)
    o2, _, _ = run(q2, k, v, 0.3)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-13)


def test_max_subtraction_keeps_large_scores_finite():
    """Scores near 1e4: exp without the row maximum subtracted overflows;
    the oracle's result is the one-hot pick of the largest score's value."""
    D = 8
    q = torch.full((1, 1, 1, D), 64.0)
    k = torch.zeros(1, 1, 3, D)
    k[0, 0, 0] = 20.0
    k[0, 0, 1] = 19.0
    v = torch.randn(1, 1, 3, D, generator=torch.Generator().manual_seed(5))
    o, _, smax = run(q, k, v, 1.0)
    assert np.all(np.isfinite(o))
    assert np.allclose(o[0], vals(bits(v))[0, 0, 0].numpy(), atol=1e-12)
    assert smax[0] == 64.0 * 20.0 * D


def test_causal_mask_edges():
    """seq_q == seq_k: row 0 sees key 0 only; seq_q < seq_k: the last row
    sees every key; seq_q > seq_k: the first seq_q - seq_k rows see none
    and are zero."""
    g = torch.Generator().manual_seed(6)
    D = 16
    q = torch.randn(1, 1, 6, D, generator=g)
    k = torch.randn(1, 1, 6, D, generator=g)
    v = torch.randn(1, 1, 6, D, generator=g)
    o, _, _ = run(q, k, v, 0.25, causal=True)
    assert np.array_equal(o[0], vals(bits(v))[0, 0, 0].numpy())
    k9 = torch.randn(1, 1, 9, D, generator=g)
    v9 = torch.randn(1, 1, 9, D, generator=g)
    oc, _, _ = run(q, k9, v9, 0.25, causal=True)
    of, _, _ = run(q, k9, v9, 0.25, causal=False)
    assert np.array_equal(oc[-1], of[-1]) and not np.allclose(oc[0], of[0])
    k3, v3 = k[:, :, :3], v[:, :, :3]
    o3, pv3, _ = run(q, k3, v3, 0.25, causal=True)
    assert np.all(o3[:3] == 0.0) and np.all(pv3[:3] == 0.0)
    assert np.array_equal(o3[3], vals(bits(v3))[0, 0, 0].numpy())


def test_bad_arguments_rejected():
    z = np.zeros(8, np.uint16)
    with pytest.raises(ValueError):
        oracle.attention(1, 1, 1, 1, 0, z, z, z, 1.0)
    with pytest.raises(ValueError):
        oracle.attention(-1, 1, 1, 1, 8, z, z, z, 1.0)


# ------------------------------------------------------- the attention bound

def test_attention_bound_failing_side():
    rng = np.random.default_rng(7)
    n, D, T = 200, 16, 300
    oref = rng.normal(size=(n, D))
    pv = np.abs(oref) + rng.uniform(0, 1, (n, D))
    smax = rng.uniform(0, 40, n)
    for bf16 in (False, True):
        tol = oracle.attention_tolerance(oref, pv, smax, T, bf16)
        sign = rng.choice([-1.0, 1.0], (n, D))
        ok, worst, _ = oracle.check_attention(oref + 0.99 * sign * tol, oref, pv, smax, T, bf16)
        assert ok and worst <= 0.99 + 1e-9
        ok, _, bad = oracle.check_attention(oref + 1.01 * sign * tol, oref, pv, smax, T, bf16)
        assert bad == n * D


def test_attention_bound_covers_bf16_probabilities_only_once():
    """The computation the kernel does (probabilities rounded to bf16 before
    the P V product, everything else in float64 here) stays inside the
    bound; doubling that rounding error (probabilities off by a whole bf16
    ulp) leaves it for some entries: the 2^-8 pv term is half an ulp, not
    more.  (Small scores, so that the score term expm1(2 delta) of the bound
    is far below the bf16 term and the latter decides.)"""
    g = torch.Generator().manual_seed(8)
    S, T, D = 64, 256, 32
    q = torch.randn(1, 1, S, D, generator=g)
    k = torch.randn(1, 1, T, D, generator=g)
    v = torch.randn(1, 1, T, D, generator=g)
    scale = 0.01
    oref, pv, smax = run(q, k, v, scale)
    qd, kd, vd = (x.to(torch.bfloat16).double()[0, 0] for x in (q, k, v))
    s = qd @ kd.T * float(np.float32(scale))
    w = torch.exp(s - s.max(-1, keepdim=True).values)
    l = w.sum(-1, keepdim=True)
    wb = w.to(torch.bfloat16).double()
    o_kernel = ((wb @ vd) / l).numpy()
    assert float(np.expm1(2 * 2.1e-4 * smax).max()) < 2.0 ** -12
    ok, worst, _ = oracle.check_attention(o_kernel, oref, pv, smax, T, False)
    assert ok, worst
    doubled = oref + 2.0 * (o_kernel - oref) + 2.0 ** -8 * pv * np.sign(o_kernel - oref)
    ok, _, bad = oracle.check_attention(doubled, oref, pv, smax, T, False)
    assert bad > 0
