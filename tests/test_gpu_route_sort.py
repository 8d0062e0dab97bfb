"""GPU parity: moe_route and moe_sort against the CPU oracle (bit-exact ids,
offsets and permutations; routing weights within 2e-6)."""
import numpy as np
import pytest
import torch

import mixture_experts_expert_softmax_amd as M
import moe_synth as S
import oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _route_case(T, E, seed, bias_var=0.0, integer=False):
    g = np.random.default_rng(seed)
    if integer:  # many exact ties, including -0.0 against +0.0
        lg = g.integers(-2, 3, size=(T, E)).astype(np.float32)
        lg[lg == 0] = np.where(g.random(np.count_nonzero(lg == 0)) < 0.5, -0.0, 0.0)
        return lg
    return S.route_logits(g, T, E, bias_var)


ROUTE_CASES = [
    # (T, E, k, bias_var, integer) -- tiny, Mixtral, expert shard, W4A8 sweep, edges
    (32, 8, 2, 0.0, False), (4096, 8, 2, 0.5, False), (8192, 256, 8, 0.0, False),
    (1024, 64, 8, 0.0, False), (1, 64, 8, 0.0, False), (777, 8, 2, 0.0, True),
    (513, 256, 8, 0.0, True), (300, 1, 1, 0.0, False), (100, 1024, 16, 0.0, False),
    (65, 16, 16, 0.0, False), (129, 100, 5, 0.0, True), (40, 32, 3, 0.0, False),
    (257, 128, 4, 0.0, False), (50, 200, 6, 0.0, True), (70, 512, 8, 0.0, True),
]


@pytest.mark.parametrize("T,E,k,bias,integer", ROUTE_CASES)
def test_route_parity(T, E, k, bias, integer):
    lg = _route_case(T, E, T + E + k, bias, integer)
    ids, w = M.moe_route(torch.from_numpy(lg).to(DEV), k)
    ref_ids, ref_w = O.route(lg, k)
    np.testing.assert_array_equal(ids.cpu().numpy(), ref_ids)
    np.testing.assert_allclose(w.cpu().numpy().astype(np.float64), ref_w, rtol=0, atol=2e-6)


def test_route_empty_is_noop():
    ids, w = M.moe_route(torch.empty((0, 8), dtype=torch.float32, device=DEV), 2)
    assert ids.shape == (0, 2) and w.shape == (0, 2)


SORT_CASES = [
    # (T, k, E, L, off)
    (32, 2, 8, 8, 0), (4096, 2, 8, 8, 0), (8192, 8, 256, 32, 64), (8192, 8, 64, 64, 0),
    (1, 8, 64, 64, 0), (1, 1, 4, 4, 0), (1000, 3, 10, 3, 7), (65536, 8, 256, 256, 0),
    (3000, 16, 1024, 1000, 24),
    # one-workgroup path at its limit (n = 16384) and just past it (chunked path)
    (1024, 16, 900, 900, 0), (2049, 8, 64, 64, 0), (4096, 4, 256, 128, 64),
    # chunked path with many experts and a partial last chunk
    (4000, 16, 900, 900, 0), (8193, 8, 64, 64, 0),
]


@pytest.mark.parametrize("T,k,E,L,off", SORT_CASES)
def test_sort_parity(T, k, E, L, off):
    g = np.random.default_rng(T * 7 + k)
    ids = g.integers(-2, E + 3, size=(T, k)).astype(np.int32)  # includes invalid ids
    r = M.moe_sort(torch.from_numpy(ids).to(DEV), E, L, off)
    ref = O.sort_routes(ids, E, L, off)
    n = int(r["n_local"].item())
    assert n == ref["n_local"]
    np.testing.assert_array_equal(r["offs"].cpu().numpy(), ref["offs"])
    np.testing.assert_array_equal(r["m_indptr"].cpu().numpy(), ref["m_indptr"])
    np.testing.assert_array_equal(r["e2p"].cpu().numpy(), ref["e2p"])
    np.testing.assert_array_equal(r["p2e"][:n].cpu().numpy(), ref["p2e"])


def test_sort_of_routed_ids_expert_shard():
    c = S.expert_shard_moe(T=8192, with_weights=False)
    ids, _ = M.moe_route(torch.from_numpy(c.logits).to(DEV), c.top_k)
    r = M.moe_sort(ids, c.num_experts, c.num_local, c.local_offset)
    ref = O.sort_routes(ids.cpu().numpy(), c.num_experts, c.num_local, c.local_offset)
    np.testing.assert_array_equal(r["e2p"].cpu().numpy(), ref["e2p"])
    np.testing.assert_array_equal(r["offs"].cpu().numpy(), ref["offs"])


def test_sort_empty_and_all_foreign():
    r = M.moe_sort(torch.empty((0, 8), dtype=torch.int32, device=DEV), 64, 16, 0)
    assert int(r["n_local"].item()) == 0 and torch.all(r["offs"] == 0) and torch.all(r["m_indptr"] == 0)
    ids = torch.full((100, 4), 3, dtype=torch.int32, device=DEV)
    r = M.moe_sort(ids, 64, 16, 32)
    assert int(r["n_local"].item()) == 0
    assert torch.all(r["e2p"] == -1) and torch.all(r["offs"] == 0)


def test_sort_all_routes_on_one_expert():
    ids = torch.full((5000, 2), 5, dtype=torch.int32, device=DEV)
    r = M.moe_sort(ids, 8)
    ref = O.sort_routes(ids.cpu().numpy(), 8, 8, 0)
    np.testing.assert_array_equal(r["offs"].cpu().numpy(), ref["offs"])
    np.testing.assert_array_equal(r["p2e"][:10000].cpu().numpy(), np.arange(10000))


def test_sort_into_preallocated_outputs():
    """Outputs passed back in are overwritten completely: a second sort of different ids
    into the first call's tensors matches a fresh sort of those ids."""
    g = np.random.default_rng(5)
    a = torch.from_numpy(g.integers(0, 64, size=(3000, 8)).astype(np.int32)).to(DEV)
    b = torch.from_numpy(g.integers(0, 64, size=(3000, 8)).astype(np.int32)).to(DEV)
    r1 = M.moe_sort(a, 64, 16, 8)
    r2 = M.moe_sort(b, 64, 16, 8, out=r1)
    assert r2["e2p"].data_ptr() == r1["e2p"].data_ptr()
    ref = O.sort_routes(b.cpu().numpy(), 64, 16, 8)
    n = int(r2["n_local"].item())
    assert n == ref["n_local"]
    np.testing.assert_array_equal(r2["offs"].cpu().numpy(), ref["offs"])
    np.testing.assert_array_equal(r2["m_indptr"].cpu().numpy(), ref["m_indptr"])
    np.testing.assert_array_equal(r2["e2p"].cpu().numpy(), ref["e2p"])
    np.testing.assert_array_equal(r2["p2e"][:n].cpu().numpy(), ref["p2e"])
    with pytest.raises(ValueError):
        M.moe_sort(b, 64, 16, 8, out=dict(r1, e2p=r1["e2p"][:10]))
