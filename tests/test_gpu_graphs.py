"""The device calls record into a HIP graph (torch.cuda.CUDAGraph) and the
replays give the eager results: no call allocates, clears memory with a
memset or synchronises with the host.  Each graph is replayed several times
with eager work and synchronisations in between, new inputs copied into its
static tensors before each replay, and every replay is compared bit for bit
with an eager run of the same calls on the same inputs (the kernels are
deterministic), and once with the oracle."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import datagen  # noqa: E402
import paged_kv_cache_377_amd as pkv  # noqa: E402
from oracle import BlockAllocatorModel, paged_attention_decode, paged_attention_prefill  # noqa: E402
from tests.gpu_util import check_close, dev, host  # noqa: E402


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _pool(rng, lens, hkv, D, B, extra=8):
    need = sum(-(-n // B) for n in lens)
    nb = need + extra
    m = BlockAllocatorModel(nb, B, rng.permutation(nb).astype(np.int32))
    for s, n in enumerate(lens):
        m.add(s, n)
    width = max(1, max(-(-n // B) for n in lens))
    t, ctx = m.build_tables(list(range(len(lens))), width)
    tables = np.array(t, np.int32)
    used = sorted({int(b) for s, n in enumerate(lens) for b in tables[s][:-(-n // B)]})
    free = sorted(set(range(nb)) - set(used))
    kc = datagen.normal(rng, (nb, hkv, B, D), "bf16")
    vc = datagen.normal(rng, (nb, hkv, B, D), "bf16")
    return kc, vc, tables, np.array(ctx, np.int32), used, free


def _capture(fn):
    fn()  # eager warm-up on the same static tensors
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_decode_step_graph_replays_match_eager():
    """copy_blocks + fused append/decode (balanced split), as one step."""
    rng = np.random.default_rng(71)
    lens = [33, 1, 700, 129, 2048, 16, 17, 500]
    hq, hkv, D, B = 32, 8, 128, 16
    print(f"graph decode step lens={lens}", flush=True)
    kc, vc, tables, ctx, used, free = _pool(rng, lens, hkv, D, B)
    pairs = np.array([[used[0], free[0]], [used[3], free[1]], [used[-1], free[2]]], np.int32)
    S = len(lens)
    scale = 1.0 / np.sqrt(D)
    mx = int(ctx.max())
    desc = pkv.CacheDesc(kc.shape[0], hkv, B, D, pkv.PKV_BF16)
    ws_bytes = pkv.decode_workspace_bytes(desc, S, hq, mx)

    # static tensors of the graph
    s_kc, s_vc = dev(kc), dev(vc)
    s_q = dev(datagen.normal(rng, (S, hq, D), "bf16"))
    s_kn = dev(datagen.normal(rng, (S, hkv, D), "bf16"))
    s_vn = dev(datagen.normal(rng, (S, hkv, D), "bf16"))
    s_out = torch.empty_like(s_q)
    s_tab, s_ctx, s_pairs = dev(tables), dev(ctx), dev(pairs)
    s_ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")

    def step(out, q, kn, vn, kcache, vcache, ws):
        pkv.copy_blocks(kcache, vcache, s_pairs)
        pkv.paged_attention_decode_append(out, q, kn, vn, kcache, vcache, s_tab, s_ctx, scale, mx,
                                          workspace=ws)

    g = _capture(lambda: step(s_out, s_q, s_kn, s_vn, s_kc, s_vc, s_ws))
    e_ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    for rep in range(3):
        q = datagen.normal(rng, (S, hq, D), "bf16")
        kn = datagen.normal(rng, (S, hkv, D), "bf16")
        vn = datagen.normal(rng, (S, hkv, D), "bf16")
        s_q.copy_(dev(q)); s_kn.copy_(dev(kn)); s_vn.copy_(dev(vn))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        # eager run of the same calls on fresh copies of the same inputs
        e_kc, e_vc = s_kc.clone(), s_vc.clone()
        e_out = torch.empty_like(s_q)
        step(e_out, dev(q), dev(kn), dev(vn), e_kc, e_vc, e_ws)
        torch.cuda.synchronize()
        assert np.array_equal(host(s_out), host(e_out)), f"replay {rep}: output differs from eager"
        assert np.array_equal(host(s_kc), host(e_kc)) and np.array_equal(host(s_vc), host(e_vc))
        if rep == 2:
            k_after, v_after = host(s_kc), host(s_vc)
            ref = paged_attention_decode(q, k_after, v_after, tables, ctx, scale, "bf16")
            check_close(host(s_out), ref, "bf16")
            # the copied blocks hold their sources, the new rows their slots
            for s_, d_ in pairs:
                assert np.array_equal(k_after[d_], k_after[s_])
            for s, n in enumerate(lens):
                t = n - 1
                blk = tables[s][t // B]
                assert np.array_equal(k_after[blk, :, t % B], kn[s])
                assert np.array_equal(v_after[blk, :, t % B], vn[s])


@pytest.mark.parametrize("partition_size", [pkv.PKV_PARTITION_AUTO, 128])
def test_noalloc_decode_graph_replays_match_eager(partition_size):
    """The allocation-free decode (its workspace is the library's scratch
    array) recorded into a graph: every replay, with new queries and eager
    calls of both entry points in between, matches the workspace entry point
    bit for bit."""
    rng = np.random.default_rng(74 + max(partition_size, 0))
    lens = [900, 33, 2048, 1, 500, 129]
    hq, hkv, D, B = 32, 8, 128, 16
    print(f"graph noalloc decode lens={lens} partition_size={partition_size}", flush=True)
    kc, vc, tables, ctx, used, free = _pool(rng, lens, hkv, D, B)
    S = len(lens)
    scale = 1.0 / np.sqrt(D)
    mx = int(ctx.max())
    s_kc, s_vc, s_tab, s_ctx = dev(kc), dev(vc), dev(tables), dev(ctx)
    s_q = dev(datagen.normal(rng, (S, hq, D), "bf16"))
    s_out = torch.empty_like(s_q)

    g = _capture(lambda: pkv.paged_attention_decode_noalloc(s_out, s_q, s_kc, s_vc, s_tab, s_ctx,
                                                            scale, mx, partition_size))
    for rep in range(3):
        q = datagen.normal(rng, (S, hq, D), "bf16")
        s_q.copy_(dev(q))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        e_out = torch.empty_like(s_q)
        pkv.paged_attention_decode(e_out, dev(q), s_kc, s_vc, s_tab, s_ctx, scale, mx,
                                   partition_size)
        n_out = torch.empty_like(s_q)
        pkv.paged_attention_decode_noalloc(n_out, dev(q), s_kc, s_vc, s_tab, s_ctx, scale, mx,
                                           partition_size)
        torch.cuda.synchronize()
        assert np.array_equal(host(s_out), host(e_out)), f"replay {rep}: differs from eager"
        assert np.array_equal(host(n_out), host(e_out))
        if rep == 2:
            ref = paged_attention_decode(q, kc, vc, tables, ctx, scale, "bf16")
            check_close(host(s_out), ref, "bf16")


@pytest.mark.parametrize("partition_size", [pkv.PKV_PARTITION_AUTO, 256])
def test_write_then_decode_graph_replays_match_eager(partition_size):
    """paged_kv_write of new tokens + decode (balanced split or split-context)."""
    rng = np.random.default_rng(72 + max(partition_size, 0))
    lens = [300, 5, 1030, 64]
    hq, hkv, D, B = 16, 4, 128, 16
    print(f"graph write+decode lens={lens} partition_size={partition_size}", flush=True)
    kc, vc, tables, ctx, used, free = _pool(rng, lens, hkv, D, B)
    S = len(lens)
    scale = 1.0 / np.sqrt(D)
    mx = int(ctx.max())
    # each step rewrites the last two positions of every sequence
    slots = np.array([tables[s][t // B] * B + t % B for s, n in enumerate(lens)
                      for t in (n - 2, n - 1)], np.int64)
    desc = pkv.CacheDesc(kc.shape[0], hkv, B, D, pkv.PKV_BF16)
    ws_bytes = max(16, pkv.decode_workspace_bytes(desc, S, hq, mx, partition_size))
    s_kc, s_vc = dev(kc), dev(vc)
    s_q = dev(datagen.normal(rng, (S, hq, D), "bf16"))
    s_k = dev(datagen.normal(rng, (len(slots), hkv, D), "bf16"))
    s_v = dev(datagen.normal(rng, (len(slots), hkv, D), "bf16"))
    s_out = torch.empty_like(s_q)
    s_slots, s_tab, s_ctx = dev(slots), dev(tables), dev(ctx)
    s_ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")

    def step(out, q, k, v, kcache, vcache, ws):
        pkv.paged_kv_write(k, v, s_slots, kcache, vcache)
        pkv.paged_attention_decode(out, q, kcache, vcache, s_tab, s_ctx, scale, mx,
                                   partition_size, workspace=ws)

    g = _capture(lambda: step(s_out, s_q, s_k, s_v, s_kc, s_vc, s_ws))
    e_ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    for rep in range(3):
        q = datagen.normal(rng, (S, hq, D), "bf16")
        k = datagen.normal(rng, (len(slots), hkv, D), "bf16")
        v = datagen.normal(rng, (len(slots), hkv, D), "bf16")
        s_q.copy_(dev(q)); s_k.copy_(dev(k)); s_v.copy_(dev(v))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        e_kc, e_vc = s_kc.clone(), s_vc.clone()
        e_out = torch.empty_like(s_q)
        step(e_out, dev(q), dev(k), dev(v), e_kc, e_vc, e_ws)
        torch.cuda.synchronize()
        assert np.array_equal(host(s_out), host(e_out)), f"replay {rep}: output differs from eager"
        if rep == 1:
            ref = paged_attention_decode(q, host(s_kc), host(s_vc), tables, ctx, scale, "bf16")
            check_close(host(s_out), ref, "bf16")


def test_prefill_graph_replays_match_eager():
    rng = np.random.default_rng(73)
    lens, news = [600, 130, 77], [200, 130, 1]
    hq, hkv, D, B = 32, 8, 128, 16
    print(f"graph prefill lens={lens} news={news}", flush=True)
    kc, vc, tables, ctx, used, free = _pool(rng, lens, hkv, D, B)
    qsl = np.concatenate([[0], np.cumsum(news)]).astype(np.int32)
    T = int(qsl[-1])
    scale = 1.0 / np.sqrt(D)
    s_kc, s_vc = dev(kc), dev(vc)
    s_q = dev(datagen.normal(rng, (T, hq, D), "bf16"))
    s_out = torch.empty_like(s_q)
    s_tab, s_ctx, s_qsl = dev(tables), dev(ctx), dev(qsl)

    def step(out, q):
        pkv.paged_attention_prefill(out, q, s_kc, s_vc, s_tab, s_ctx, s_qsl, scale, max(news),
                                    int(ctx.max()))

    g = _capture(lambda: step(s_out, s_q))
    for rep in range(3):
        q = datagen.normal(rng, (T, hq, D), "bf16")
        s_q.copy_(dev(q))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        e_out = torch.empty_like(s_q)
        step(e_out, dev(q))
        torch.cuda.synchronize()
        assert np.array_equal(host(s_out), host(e_out)), f"replay {rep}: output differs from eager"
        if rep == 0:
            ref = paged_attention_prefill(q, kc, vc, tables, ctx, qsl, scale, "bf16")
            check_close(host(s_out), ref, "bf16")
