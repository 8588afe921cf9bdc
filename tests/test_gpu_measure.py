"""The gather probe (pkv_measure_gather) reads exactly the runs it is given.

Each wave XORs every 32-bit word of the K and V runs of its share (runs
[w n / W, (w + 1) n / W) of the list, ids outside the pool read run 0) and
stores the result; the expected values are the same XORs taken with numpy over
the pools' bytes.  This is the check behind the gather-ceiling figures: a
probe that skipped or repeated runs would be timed on other bytes."""

import zlib

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import paged_kv_cache_377_amd as pkv  # noqa: E402
from datagen import normal  # noqa: E402
from tests.gpu_util import dev  # noqa: E402


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _expected(kc, vc, runs, workers):
    nb, hkv = kc.shape[0], kc.shape[1]
    kw = kc.reshape(nb * hkv, -1).view(np.uint32)
    vw = vc.reshape(nb * hkv, -1).view(np.uint32)
    ids = np.where((runs >= 0) & (runs < nb * hkv), runs, 0)
    n = len(runs)
    out = np.zeros(workers, np.uint32)
    for w in range(workers):
        a, b = w * n // workers, (w + 1) * n // workers
        if b > a:
            out[w] = np.bitwise_xor.reduce(np.concatenate([kw[ids[a:b]].ravel(), vw[ids[a:b]].ravel()]))
    return out


SHAPES = [  # (NB, Hkv, B, D, dtype): runs of 4, 1, 8 and 4 KiB
    (64, 8, 16, 128, "bf16"),
    (40, 4, 8, 64, "bf16"),
    (30, 2, 32, 128, "bf16"),
    (50, 4, 16, 64, "f32"),
]


@pytest.mark.parametrize("in_flight", [1, 2, 3])
@pytest.mark.parametrize("shape", SHAPES)
def test_probe_reads_exactly_its_runs(shape, in_flight):
    nb, hkv, B, D, dtype = shape
    print(f"gather probe {shape} in_flight={in_flight}", flush=True)
    rng = np.random.default_rng(zlib.crc32(repr((shape, in_flight)).encode()))
    kc = normal(rng, (nb, hkv, B, D), dtype)
    vc = normal(rng, (nb, hkv, B, D), dtype)
    n, workers = 1000, 37
    runs = rng.integers(-3, nb * hkv + 3, size=n).astype(np.int32)  # a few ids outside the pool
    sink = torch.zeros(workers + 3, dtype=torch.int32, device="cuda")
    pkv.measure_gather(dev(kc), dev(vc), dev(runs), workers, in_flight, sink)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    np.testing.assert_array_equal(got[:workers], _expected(kc, vc, runs, workers))
    assert not got[workers:].any()  # nothing written past the workers


def test_more_workers_than_runs_and_the_share_limit():
    rng = np.random.default_rng(5)
    kc = normal(rng, (16, 2, 16, 128), "bf16")
    vc = normal(rng, (16, 2, 16, 128), "bf16")
    runs = rng.integers(0, 32, size=10).astype(np.int32)
    sink = torch.zeros(64, dtype=torch.int32, device="cuda")
    pkv.measure_gather(dev(kc), dev(vc), dev(runs), 64, 2, sink)  # 54 empty shares
    torch.cuda.synchronize()
    np.testing.assert_array_equal(sink.cpu().numpy().view(np.uint32), _expected(kc, vc, runs, 64))
    many = dev(np.zeros(4097, np.int32))
    with pytest.raises(pkv.PagedKVError):
        pkv.measure_gather(dev(kc), dev(vc), many, 1, 1, sink)  # 4097 runs for one wave
    with pytest.raises(pkv.PagedKVError):
        pkv.measure_gather(dev(kc), dev(vc), dev(runs), 4, 4, sink)  # at most 3 in flight
