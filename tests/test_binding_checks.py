"""The Python binding refuses tensors the kernels cannot reach (host memory
that is not pinned, tensors on another device) before anything is launched:
a host address handed to a kernel would fault the GPU.  Runs on the CPU: the
library is loaded, no device call is made."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import paged_kv_cache_377_amd as pkv  # noqa: E402


def _host_cache(nb=4, hkv=2, b=16, d=64):
    return torch.zeros((nb, hkv, b, d), dtype=torch.bfloat16)


def _refused(fn):
    with pytest.raises(pkv.PagedKVError) as e:
        fn()
    assert e.value.code == pkv.PKV_EINVAL
    assert "GPU memory" in e.value.message


def test_write_refuses_host_tensors():
    kc = _host_cache()
    k = torch.zeros((3, 2, 64), dtype=torch.bfloat16)
    slots = torch.tensor([0, 1, 2], dtype=torch.int64)
    _refused(lambda: pkv.paged_kv_write(k, k, slots, kc, kc))


def test_copy_refuses_host_tensors():
    kc = _host_cache()
    pairs = torch.tensor([[0, 1]], dtype=torch.int32)
    _refused(lambda: pkv.copy_blocks(kc, kc, pairs))


def test_decode_refuses_host_tensors():
    kc = _host_cache()
    q = torch.zeros((2, 4, 64), dtype=torch.bfloat16)
    tables = torch.zeros((2, 2), dtype=torch.int32)
    ctx = torch.tensor([5, 9], dtype=torch.int32)
    ws = torch.zeros(1 << 16, dtype=torch.uint8)
    _refused(lambda: pkv.paged_attention_decode(q.clone(), q, kc, kc, tables, ctx, 0.125, 9,
                                                workspace=ws))
    kn = torch.zeros((2, 2, 64), dtype=torch.bfloat16)
    _refused(lambda: pkv.paged_attention_decode_append(q.clone(), q, kn, kn, kc, kc, tables, ctx,
                                                       0.125, 9, workspace=ws))


def test_prefill_refuses_host_tensors():
    kc = _host_cache()
    q = torch.zeros((5, 4, 64), dtype=torch.bfloat16)
    tables = torch.zeros((1, 2), dtype=torch.int32)
    ctx = torch.tensor([5], dtype=torch.int32)
    qsl = torch.tensor([0, 5], dtype=torch.int32)
    _refused(lambda: pkv.paged_attention_prefill(q.clone(), q, kc, kc, tables, ctx, qsl, 0.125, 5, 5))


def test_swap_refuses_unpinned_host_pools():
    kc = _host_cache()
    pairs = torch.from_numpy(np.array([[0, 1]], np.int32))
    with pytest.raises(pkv.PagedKVError) as e:
        pkv.swap_blocks(kc, kc, kc, kc, pairs)
    assert e.value.code == pkv.PKV_EINVAL and "pinned" in e.value.message


def test_empty_host_tensors_pass_the_check():
    # nothing is read from an empty tensor, so its placement does not matter
    # (the call itself is not made here: this only exercises the check)
    from paged_kv_cache_377_amd import _lib
    assert _lib._ptr(torch.zeros((0, 2), dtype=torch.int32)) is not None


# Shape and dtype mismatches the C side cannot see (it sizes every pointer from
# the one descriptor built from the K pool) are refused by the binding, before
# the placement check and before any launch.

def _mismatch(fn, words):
    with pytest.raises(pkv.PagedKVError) as e:
        fn()
    assert e.value.code == pkv.PKV_EINVAL
    assert "GPU memory" not in e.value.message, "the mismatch must be caught first"
    assert any(w in e.value.message for w in words), e.value.message


def test_decode_refuses_head_dim_and_pool_mismatches():
    kc = _host_cache(nb=4, hkv=2, b=16, d=64)
    small_v = _host_cache(nb=3, hkv=2, b=16, d=64)
    q = torch.zeros((2, 4, 64), dtype=torch.bfloat16)
    q32 = torch.zeros((2, 4, 32), dtype=torch.bfloat16)
    q3 = torch.zeros((2, 3, 64), dtype=torch.bfloat16)
    tables = torch.zeros((2, 2), dtype=torch.int32)
    ctx = torch.tensor([5, 9], dtype=torch.int32)
    _mismatch(lambda: pkv.paged_attention_decode(q32.clone(), q32, kc, kc, tables, ctx, 0.1, 9),
              ["head_dim"])
    _mismatch(lambda: pkv.paged_attention_decode(q3.clone(), q3, kc, kc, tables, ctx, 0.1, 9),
              ["multiple"])
    _mismatch(lambda: pkv.paged_attention_decode(q.clone(), q, kc, small_v, tables, ctx, 0.1, 9),
              ["differ"])
    _mismatch(lambda: pkv.paged_attention_decode(q.clone(), q, kc, kc.float(), tables, ctx, 0.1, 9),
              ["differ"])
    kn = torch.zeros((2, 2, 64), dtype=torch.bfloat16)
    _mismatch(lambda: pkv.paged_attention_decode_append(q32.clone(), q32, kn, kn, kc, kc, tables,
                                                        ctx, 0.1, 9), ["head_dim"])
    _mismatch(lambda: pkv.paged_attention_decode_append(q.clone(), q, kn, kn, kc, small_v, tables,
                                                        ctx, 0.1, 9), ["differ"])
    kn32 = torch.zeros((2, 2, 32), dtype=torch.bfloat16)
    _mismatch(lambda: pkv.paged_attention_decode_append(q.clone(), q, kn32, kn32, kc, kc, tables,
                                                        ctx, 0.1, 9), ["k_new"])


def test_prefill_refuses_head_dim_and_pool_mismatches():
    kc = _host_cache(nb=4, hkv=2, b=16, d=64)
    q32 = torch.zeros((5, 4, 32), dtype=torch.bfloat16)
    q = torch.zeros((5, 4, 64), dtype=torch.bfloat16)
    tables = torch.zeros((1, 2), dtype=torch.int32)
    ctx = torch.tensor([5], dtype=torch.int32)
    qsl = torch.tensor([0, 5], dtype=torch.int32)
    _mismatch(lambda: pkv.paged_attention_prefill(q32.clone(), q32, kc, kc, tables, ctx, qsl,
                                                  0.1, 5, 5), ["head_dim"])
    _mismatch(lambda: pkv.paged_attention_prefill(q.clone(), q, kc, _host_cache(nb=2), tables, ctx,
                                                  qsl, 0.1, 5, 5), ["differ"])


def test_write_and_copy_refuse_pool_mismatches():
    kc = _host_cache(nb=4)
    k = torch.zeros((3, 2, 64), dtype=torch.bfloat16)
    slots = torch.tensor([0, 1, 2], dtype=torch.int64)
    _mismatch(lambda: pkv.paged_kv_write(k, k, slots, kc, _host_cache(nb=2)), ["differ"])
    _mismatch(lambda: pkv.paged_kv_write(k, k, slots, kc, kc.float()), ["differ"])
    pairs = torch.tensor([[0, 1]], dtype=torch.int32)
    _mismatch(lambda: pkv.copy_blocks(kc, _host_cache(nb=2), pairs), ["differ"])


def test_swap_refuses_v_pools_of_another_shape():
    dev_k = _host_cache(nb=4)
    host_k = _host_cache(nb=8)
    pairs = torch.from_numpy(np.array([[0, 1]], np.int32))
    _mismatch(lambda: pkv.swap_blocks(dev_k, _host_cache(nb=2), host_k, host_k, pairs),
              ["dst_k and dst_v"])
    _mismatch(lambda: pkv.swap_blocks(dev_k, dev_k, host_k, _host_cache(nb=3), pairs),
              ["src_k and src_v"])
    _mismatch(lambda: pkv.swap_blocks(dev_k, dev_k, host_k, host_k.float(), pairs),
              ["src_k and src_v"])
