"""Pins of the oracle's causal paged prefill: torch's scaled_dot_product_attention
with the causal-offset mask on dense K/V, reduction to the decode oracle
with one new token, closed forms (a prompt's first token returns V_0; equal
keys give prefix means), causality, chunked prefill equal to one prefill,
physical-id permutation, and a scalar brute force on tiny inputs."""

import math

import numpy as np
import pytest
import torch

from oracle import paged_attention_decode, paged_attention_prefill
from tests.test_oracle_attention import _as_f64, _draw, _paged_from_dense


def _qsl(news):
    return np.concatenate([[0], np.cumsum(news)]).astype(np.int32)


CASES = [  # (lens, new tokens per seq, Hq, Hkv, D, B, dtype)
    ([1, 16, 17, 40], [1, 16, 5, 33], 4, 4, 64, 16, "f32"),
    ([5, 33, 64], [5, 1, 20], 8, 2, 16, 8, "bf16"),
    ([31, 32, 2, 100], [0, 32, 2, 7], 8, 1, 8, 4, "bf16"),
]


@pytest.mark.parametrize("case", CASES)
def test_equals_sdpa_with_causal_offset_mask(case):
    lens, news, hq, hkv, d, B, dtype = case
    rng = np.random.default_rng(21)
    kc, vc, bt, ctx, dk, dv = _paged_from_dense(rng, lens, hkv, d, B, dtype)
    T = sum(news)
    q = _draw(rng, (T, hq, d), dtype)
    qsl = _qsl(news)
    scale = 1.0 / math.sqrt(d)
    got = paged_attention_prefill(q, kc, vc, bt, ctx, qsl, scale, dtype)
    G = hq // hkv
    for s, (n, m) in enumerate(zip(lens, news)):
        if m == 0:
            continue
        qs = torch.from_numpy(_as_f64(q[qsl[s]:qsl[s + 1]], dtype)).permute(1, 0, 2)   # [Hq, m, d]
        K = torch.from_numpy(_as_f64(dk[s], dtype)).permute(1, 0, 2).repeat_interleave(G, 0)
        V = torch.from_numpy(_as_f64(dv[s], dtype)).permute(1, 0, 2).repeat_interleave(G, 0)
        pos = torch.arange(n - m, n)[:, None]
        mask = torch.arange(n)[None, :] <= pos                                       # [m, n]
        ref = torch.nn.functional.scaled_dot_product_attention(qs, K, V, attn_mask=mask, scale=scale)
        np.testing.assert_allclose(got[qsl[s]:qsl[s + 1]], ref.permute(1, 0, 2).numpy(), rtol=1e-10,
                                   atol=1e-12)


def test_one_new_token_is_decode():
    rng = np.random.default_rng(22)
    lens = [3, 17, 64, 1]
    kc, vc, bt, ctx, _, _ = _paged_from_dense(rng, lens, 2, 32, 8, "bf16")
    q = _draw(rng, (len(lens), 8, 32), "bf16")
    a = paged_attention_prefill(q, kc, vc, bt, ctx, _qsl([1] * len(lens)), 0.2, "bf16")
    b = paged_attention_decode(q, kc, vc, bt, ctx, 0.2, "bf16")
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-14)


def test_first_prompt_token_returns_v0_and_equal_keys_give_prefix_means():
    rng = np.random.default_rng(23)
    n, d, B = 12, 16, 4
    kc, vc, bt, ctx, dk, dv = _paged_from_dense(rng, [n], 1, d, B, "f32")
    q = _draw(rng, (n, 2, d), "f32")
    out = paged_attention_prefill(q, kc, vc, bt, ctx, _qsl([n]), 0.3, "f32")
    np.testing.assert_array_equal(out[0, 0], dv[0][0, 0].astype(np.float64))
    # equal keys: every row attends uniformly to its prefix
    kc2 = kc.copy()
    kc2[:] = kc[bt[0][0], :, 0:1, :]
    out2 = paged_attention_prefill(q, kc2, vc, bt, ctx, _qsl([n]), 0.3, "f32")
    V = dv[0][:, 0].astype(np.float64)
    for j in range(n):
        np.testing.assert_allclose(out2[j, 1], V[: j + 1].mean(0), rtol=1e-12, atol=1e-13)


def test_causality_later_positions_never_matter():
    rng = np.random.default_rng(24)
    lens, news = [40], [25]
    kc, vc, bt, ctx, _, _ = _paged_from_dense(rng, lens, 2, 16, 8, "f32")
    q = _draw(rng, (25, 4, 16), "f32")
    base = paged_attention_prefill(q, kc, vc, bt, ctx, _qsl(news), 0.25, "f32")
    first = lens[0] - news[0]
    for p in (first, first + 7, lens[0] - 2):
        k2, v2 = kc.copy(), vc.copy()
        for t in range(p + 1, lens[0]):          # change every position after p
            k2[bt[0][t // 8], :, t % 8] += 1.0
            v2[bt[0][t // 8], :, t % 8] -= 2.0
        out = paged_attention_prefill(q, k2, v2, bt, ctx, _qsl(news), 0.25, "f32")
        j = p - first
        np.testing.assert_array_equal(out[: j + 1], base[: j + 1])
        assert not np.allclose(out[j + 1:], base[j + 1:])


def test_chunked_prefill_equals_one_prefill():
    """Prefill of a prompt in two chunks (the second sees the first through the
    table) gives the rows of one prefill of the whole prompt."""
    rng = np.random.default_rng(25)
    n, split = 37, 13
    kc, vc, bt, ctx, _, _ = _paged_from_dense(rng, [n], 2, 16, 4, "bf16")
    q = _draw(rng, (n, 4, 16), "bf16")
    whole = paged_attention_prefill(q, kc, vc, bt, ctx, _qsl([n]), 0.25, "bf16")
    c1 = paged_attention_prefill(q[:split], kc, vc, bt, np.array([split], np.int32), _qsl([split]), 0.25,
                                 "bf16")
    c2 = paged_attention_prefill(q[split:], kc, vc, bt, ctx, _qsl([n - split]), 0.25, "bf16")
    np.testing.assert_array_equal(np.concatenate([c1, c2]), whole)


def test_physical_permutation_is_invisible():
    rng = np.random.default_rng(26)
    lens, news = [9, 30], [9, 11]
    kc, vc, bt, ctx, _, _ = _paged_from_dense(rng, lens, 2, 16, 4, "bf16")
    q = _draw(rng, (20, 4, 16), "bf16")
    base = paged_attention_prefill(q, kc, vc, bt, ctx, _qsl(news), 0.25, "bf16")
    perm = rng.permutation(kc.shape[0])
    inv = np.argsort(perm)
    out = paged_attention_prefill(q, kc[perm], vc[perm], inv[bt].astype(np.int32), ctx, _qsl(news), 0.25,
                                  "bf16")
    np.testing.assert_array_equal(out, base)


def test_brute_force_tiny():
    rng = np.random.default_rng(27)
    lens, news = [3, 5], [2, 5]
    kc, vc, bt, ctx, dk, dv = _paged_from_dense(rng, lens, 1, 2, 2, "f32")
    q = _draw(rng, (7, 2, 2), "f32")
    got = paged_attention_prefill(q, kc, vc, bt, ctx, _qsl(news), 0.7, "f32")
    row = 0
    for s, (n, m) in enumerate(zip(lens, news)):
        for j in range(m):
            p = n - m + j
            for h in range(2):
                ls = [0.7 * sum(float(q[row, h, e]) * float(dk[s][t, 0, e]) for e in range(2))
                      for t in range(p + 1)]
                mx = max(ls)
                ws = [math.exp(x - mx) for x in ls]
                for e in range(2):
                    want = sum(w * float(dv[s][t, 0, e]) for t, w in enumerate(ws)) / sum(ws)
                    assert abs(got[row, h, e] - want) < 1e-12
            row += 1


def test_rejects_more_new_tokens_than_context():
    rng = np.random.default_rng(28)
    kc, vc, bt, ctx, _, _ = _paged_from_dense(rng, [4], 1, 4, 4, "f32")
    q = _draw(rng, (5, 1, 4), "f32")
    with pytest.raises(ValueError):
        paged_attention_prefill(q, kc, vc, bt, ctx, _qsl([5]), 1.0, "f32")
