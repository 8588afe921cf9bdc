"""Pins of the oracle's decode attention.

The attention is pinned to things the oracle does not compute itself: torch's
scaled_dot_product_attention on dense, contiguous K/V (the pages: paged
attention is ordinary attention plus a gather), closed forms, a pure-Python
brute force on tiny inputs, and invariances (physical-id permutation, poison
in slots no sequence reads)."""

import math

import numpy as np
import pytest
import torch

from datagen import bf16_from_f32, bf16_to_f32, poison_unused
from oracle import BlockAllocatorModel, paged_attention_decode, paged_kv_write


def _draw(rng, shape, dtype):
    x = rng.standard_normal(shape).astype(np.float32)
    return bf16_from_f32(x) if dtype == "bf16" else x


def _as_f64(x, dtype):
    return (bf16_to_f32(x) if dtype == "bf16" else x).astype(np.float64)


def _paged_from_dense(rng, lens, hkv, d, B, dtype, extra_blocks=3):
    """Dense per-sequence K/V -> a scattered pool, through the allocator's slots."""
    need = sum(-(-n // B) for n in lens)
    nb = need + extra_blocks
    m = BlockAllocatorModel(nb, B, list(rng.permutation(nb)))
    kc = _draw(rng, (nb, hkv, B, d), dtype)
    vc = _draw(rng, (nb, hkv, B, d), dtype)
    dense_k, dense_v = [], []
    for s, n in enumerate(lens):
        k = _draw(rng, (n, hkv, d), dtype)
        v = _draw(rng, (n, hkv, d), dtype)
        kc, vc = paged_kv_write(k, v, m.add(s, n), kc, vc)
        dense_k.append(k)
        dense_v.append(v)
    width = max(1, max(-(-n // B) for n in lens))
    tables, ctx = m.build_tables(list(range(len(lens))), width)
    return kc, vc, np.array(tables, np.int32), np.array(ctx, np.int32), dense_k, dense_v


CASES = [  # (lens, Hq, Hkv, D, B, dtype)
    ([1, 16, 17, 40], 4, 4, 64, 16, "f32"),
    ([5, 33, 64], 8, 2, 16, 8, "bf16"),
    ([31, 32, 2, 100], 8, 1, 8, 4, "bf16"),
    ([70, 9], 6, 3, 32, 32, "f32"),
]


@pytest.mark.parametrize("case", CASES)
def test_equals_sdpa_on_dense_kv(case):
    lens, hq, hkv, d, B, dtype = case
    rng = np.random.default_rng(11)
    kc, vc, bt, ctx, dk, dv = _paged_from_dense(rng, lens, hkv, d, B, dtype)
    q = _draw(rng, (len(lens), hq, d), dtype)
    scale = 1.0 / math.sqrt(d)
    out = paged_attention_decode(q, kc, vc, bt, ctx, scale, dtype)
    G = hq // hkv
    for s, n in enumerate(lens):
        qt = torch.from_numpy(_as_f64(q[s], dtype))[None, :, None, :]          # [1,Hq,1,D]
        kt = torch.from_numpy(_as_f64(dk[s], dtype)).permute(1, 0, 2)        # [Hkv,n,D]
        vt = torch.from_numpy(_as_f64(dv[s], dtype)).permute(1, 0, 2)
        kt = kt.repeat_interleave(G, dim=0)[None]                            # [1,Hq,n,D]
        vt = vt.repeat_interleave(G, dim=0)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
        np.testing.assert_allclose(out[s], ref[0, :, 0, :].numpy(), rtol=1e-12, atol=1e-12)


def _brute(q, kc, vc, bt, ctx, scale):
    """Pure-Python loops with math.exp, no numpy arithmetic (tiny inputs)."""
    S, Hq, D = len(q), len(q[0]), len(q[0][0])
    Hkv, B = len(kc[0]), len(kc[0][0])
    G = Hq // Hkv
    out = [[[0.0] * D for _ in range(Hq)] for _ in range(S)]
    for s in range(S):
        n = ctx[s]
        for h in range(Hq):
            rows = [(bt[s][t // B], t % B) for t in range(n)]
            logit = []
            for (b, o) in rows:
                acc = 0.0
                for i in range(D):
                    acc += q[s][h][i] * kc[b][h // G][o][i]
                logit.append(acc * scale)
            if not logit:
                continue
            mx = max(logit)
            w = [math.exp(x - mx) for x in logit]
            z = sum(w)
            for i in range(D):
                out[s][h][i] = sum(w[j] * vc[rows[j][0]][h // G][rows[j][1]][i] for j in range(n)) / z
    return out


def test_brute_force_tiny():
    rng = np.random.default_rng(5)
    lens = [0, 1, 3, 7, 9]
    kc, vc, bt, ctx, _, _ = _paged_from_dense(rng, lens, 2, 4, 2, "f32")
    q = _draw(rng, (len(lens), 4, 4), "f32")
    out = paged_attention_decode(q, kc, vc, bt, ctx, 0.7, "f32")
    ref = _brute(q.astype(np.float64).tolist(), kc.astype(np.float64).tolist(),
                 vc.astype(np.float64).tolist(), bt.tolist(), ctx.tolist(), 0.7)
    np.testing.assert_allclose(out, np.array(ref), rtol=1e-13, atol=1e-13)
    assert np.all(out[0] == 0.0), "an empty context gives zeros"


def test_single_token_returns_its_value_exactly():
    rng = np.random.default_rng(6)
    kc, vc, bt, ctx, _, dv = _paged_from_dense(rng, [1, 1], 2, 16, 16, "bf16")
    q = _draw(rng, (2, 4, 16), "bf16")
    out = paged_attention_decode(q, kc, vc, bt, ctx, 0.25, "bf16")
    for s in range(2):
        for h in range(4):
            assert np.array_equal(out[s, h], _as_f64(dv[s][0, h // 2], "bf16"))


def test_zero_query_and_equal_keys_give_mean_of_values():
    rng = np.random.default_rng(9)
    kc, vc, bt, ctx, dk, dv = _paged_from_dense(rng, [13, 40], 1, 8, 4, "f32")
    q = np.zeros((2, 1, 8), np.float32)
    out = paged_attention_decode(q, kc, vc, bt, ctx, 1.0, "f32")
    for s in range(2):
        np.testing.assert_allclose(out[s, 0], dv[s][:, 0].astype(np.float64).mean(0), rtol=1e-12, atol=1e-13)
    # all keys equal -> uniform weights whatever q is
    same = np.ones((40, 1, 8), np.float32) * 0.5
    kc2, vc2 = paged_kv_write(same, dv[1], [int(bt[1][t // 4]) * 4 + t % 4 for t in range(40)], kc, vc)
    q2 = rng.standard_normal((2, 1, 8)).astype(np.float32)
    out2 = paged_attention_decode(q2, kc2, vc2, bt, ctx, 3.0, "f32")
    np.testing.assert_allclose(out2[1, 0], dv[1][:, 0].astype(np.float64).mean(0), rtol=1e-12, atol=1e-13)


def test_two_token_closed_form_fixes_scale_and_sign():
    """K_0 = 0, K_1 = e_0, q = c e_0: weights 1 : exp(scale c)."""
    D, B = 4, 2
    kc = np.zeros((3, 1, B, D), np.float32)
    vc = np.zeros((3, 1, B, D), np.float32)
    kc[2, 0, 1, 0] = 1.0
    vc[2, 0, 0] = [1.0, 0.0, 0.0, 0.0]
    vc[2, 0, 1] = [0.0, 1.0, 0.0, 0.0]
    bt = np.array([[2]], np.int32)
    for c, scale in [(2.0, 0.5), (-3.0, 0.25), (1.0, 2.0)]:
        q = np.array([[[c, 0, 0, 0]]], np.float32)
        out = paged_attention_decode(q, kc, vc, bt, np.array([2]), scale, "f32")
        w1 = math.exp(scale * c) / (1.0 + math.exp(scale * c))
        np.testing.assert_allclose(out[0, 0], [1.0 - w1, w1, 0.0, 0.0], rtol=1e-14, atol=1e-15)


def test_grouped_heads_read_floor_h_over_g():
    """V of KV head g is the constant g + 1, so query head h must return
    h // G + 1 (and not h % Hkv + 1)."""
    rng = np.random.default_rng(10)
    hkv, G, D, B = 4, 3, 8, 4
    kc, vc, bt, ctx, _, _ = _paged_from_dense(rng, [6, 11], hkv, D, B, "f32")
    for g in range(hkv):
        vc[:, g] = g + 1.0
    q = _draw(rng, (2, hkv * G, D), "f32")
    out = paged_attention_decode(q, kc, vc, bt, ctx, 0.3, "f32")
    for h in range(hkv * G):
        np.testing.assert_allclose(out[:, h], h // G + 1.0, rtol=1e-14)


def test_physical_permutation_is_bit_identical():
    rng = np.random.default_rng(12)
    kc, vc, bt, ctx, _, _ = _paged_from_dense(rng, [20, 3, 47], 2, 16, 8, "bf16")
    q = _draw(rng, (3, 4, 16), "bf16")
    out = paged_attention_decode(q, kc, vc, bt, ctx, 0.25, "bf16")
    nb = kc.shape[0]
    perm = rng.permutation(nb)            # old id b lives at new id perm[b]
    kc2 = np.empty_like(kc)
    vc2 = np.empty_like(vc)
    kc2[perm] = kc
    vc2[perm] = vc
    out2 = paged_attention_decode(q, kc2, vc2, perm[bt], ctx, 0.25, "bf16")
    assert np.array_equal(out, out2)


def test_poison_in_unread_slots_changes_nothing():
    rng = np.random.default_rng(13)
    kc, vc, bt, ctx, _, _ = _paged_from_dense(rng, [20, 3, 47, 16], 2, 16, 8, "bf16", extra_blocks=5)
    q = _draw(rng, (4, 4, 16), "bf16")
    out = paged_attention_decode(q, kc, vc, bt, ctx, 0.25, "bf16")
    kp, vp = kc.copy(), vc.copy()
    poison_unused(kp, vp, bt, ctx, 8, "bf16")
    assert np.isnan(bf16_to_f32(kp)).sum() > 0
    out2 = paged_attention_decode(q, kp, vp, bt, ctx, 0.25, "bf16")
    assert np.array_equal(out, out2) and np.isfinite(out2).all()
