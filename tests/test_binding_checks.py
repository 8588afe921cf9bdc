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
