"""GPU routing bookkeeping vs the oracle's counting sort: bit-exact."""

import numpy as np
import pytest
import torch

import mixture_experts_routed_topk_amd as m
import synth
from oracle.moe import route as oracle_route

pytestmark = pytest.mark.gpu


def _gpu_route(idx: np.ndarray, E: int, flags: int = 0):
    t = torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).cuda()
    c, o, p, i = m.route(t, E, flags=flags)
    torch.cuda.synchronize()
    return c.cpu().numpy(), o.cpu().numpy(), p.cpu().numpy(), i.cpu().numpy()


def _check(idx, E):
    got = _gpu_route(idx, E)
    ref = oracle_route(idx, E)
    for name, g, r in zip(("counts", "offsets", "perm", "inv"), got, ref):
        assert np.array_equal(g, r), f"{name} differs"


@pytest.mark.parametrize("name", ["tiny_fp32", "qwen_prefill_bf16", "qwen_decode_bf16",
                                  "dsv3_prefill_bf16", "dsv3_fp8_f32scale"])
def test_route_configs(name):
    spec = synth.spec_for(name)
    idx, _ = synth.routing(spec)
    _check(idx, spec.E)


@pytest.mark.parametrize("T,k,E,kind", [
    (1, 1, 1, "uniform"), (1, 8, 256, "uniform"), (5, 4, 4, "uniform"),   # k == E
    (1000, 1, 1, "uniform"), (777, 3, 1024, "uniform"), (4096, 4, 60, "one"),
    (3000, 8, 256, "few"), (65, 2, 8, "uniform"), (64, 2, 8, "uniform"),
    # chunked routing (more than 4096 slots): a short last chunk, E = 1024, 64 chunks
    (1025, 4, 8, "uniform"), (1500, 3, 1024, "uniform"), (70000, 4, 4, "uniform"),
    (16384, 4, 60, "one"),
])
def test_route_edge_cases(T, k, E, kind):
    rng = np.random.default_rng(T * 31 + k * 7 + E)
    if kind == "one":
        idx = np.full((T, k), E - 1, dtype=np.int32)
    elif kind == "few":
        idx = rng.choice([3, 17, 200], size=(T, k)).astype(np.int32)
    else:
        idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
    _check(idx, E)


@pytest.mark.parametrize("T", [200, 3000])   # one workgroup / chunked routing
def test_route_out_of_range_ids(T):
    rng = np.random.default_rng(5)
    idx = rng.integers(0, 16, size=(T, 4)).astype(np.int32)
    bad = np.zeros_like(idx, dtype=bool)
    bad[3, 1] = bad[50, 0] = bad[T - 1, 3] = bad[T // 2, 2] = True
    idx_bad = idx.copy()
    idx_bad[3, 1], idx_bad[50, 0], idx_bad[T - 1, 3], idx_bad[T // 2, 2] = 16, -1, 1 << 20, -7
    c, o, p, i = _gpu_route(idx_bad, 16)
    # the valid slots are sorted exactly as the oracle sorts them on their own
    flat = idx_bad.reshape(-1)
    valid = np.nonzero(~bad.reshape(-1))[0]
    ref_perm = valid[np.argsort(flat[valid], kind="stable")]
    assert np.array_equal(c, np.bincount(flat[valid], minlength=16))
    assert o[-1] == valid.size
    assert np.array_equal(p[: valid.size], ref_perm)
    assert (i[bad.reshape(-1)] == -1).all()
    assert np.array_equal(i[ref_perm], np.arange(valid.size))
    with pytest.raises(IndexError):
        _gpu_route(idx_bad, 16, flags=m.FLAG_CHECK_INDICES)
    _gpu_route(idx, 16, flags=m.FLAG_CHECK_INDICES)  # valid ids: no error
