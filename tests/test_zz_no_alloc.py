"""moe_count_index_noalloc (block tables in the library's static per-GPU
scratch instead of a caller workspace) against moe_count_index, through the
C ABI: bit-identical counts, offsets, dest and src on two calls in a row, the
second with a smaller input (the scratch keeps the first call's contents),
and again after a plain moe_count_index call; sizes beyond the scratch are
refused on the host."""
import numpy as np
import pytest
import torch

from moe_inputs import random_topk_ids
from tests._gpu import DEV, dev, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _native_lib():
    global L
    import mixture_experts_layer_gating_amd._lib as lib
    L = lib


def _outs(E, Tk):
    i32 = torch.int32
    return (torch.full((E,), -1, dtype=i32, device=DEV),
            torch.full((E + 1,), -1, dtype=i32, device=DEV),
            torch.full((Tk,), -1, dtype=i32, device=DEV),
            torch.full((Tk,), -1, dtype=i32, device=DEV))


def _with_workspace(ids, T, k, E):
    c, o, d, s = _outs(E, T * k)
    nb = L.moe_count_index_workspace_size(T, k, E)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    L.moe_count_index(ids, T, k, E, c, o, d, s, ws, nb)
    torch.cuda.synchronize()
    return [host(t) for t in (c, o, d, s)]


def _no_alloc(ids, T, k, E):
    c, o, d, s = _outs(E, T * k)
    L.moe_count_index_noalloc(ids, T, k, E, c, o, d, s)
    torch.cuda.synchronize()
    return [host(t) for t in (c, o, d, s)]


# (T, k, E): the first large enough to use most of the scratch (and the
# separate scan launch), the second smaller (fused scan + scatter).
CASES = [((131072, 8, 256), (8192, 8, 64)), ((16384, 8, 128), (512, 8, 256)),
         ((65536, 4, 1024), (1000, 2, 3))]


@pytest.mark.parametrize("big,small", CASES)
def test_noalloc_matches_workspace_call(big, small):
    for (T, k, E), seed in ((big, 1), (small, 2), (big, 3)):
        say(f"count_index_noalloc T={T} k={k} E={E}")
        assert L.moe_count_index_workspace_size(T, k, E) <= L.MOE_NOALLOC_SCRATCH_BYTES
        ids = dev(random_topk_ids(T, k, E, seed=seed + T))
        want = _with_workspace(ids, T, k, E)
        got = _no_alloc(ids, T, k, E)
        for name, g, w in zip(("counts", "offsets", "dest", "src"), got, want):
            np.testing.assert_array_equal(g, w, err_msg=name)
        assert int(got[0].sum()) == T * k


def test_noalloc_refuses_sizes_beyond_scratch():
    T, k, E = 262656, 1, 1024
    assert L.moe_count_index_workspace_size(T, k, E) > L.MOE_NOALLOC_SCRATCH_BYTES
    with pytest.raises(L.MoEError) as ei:
        L.moe_count_index_noalloc(0x1000, T, k, E, 0x1000, 0x1000, 0x1000, 0x1000)
    assert ei.value.status == L.MOE_ERR_UNSUPPORTED
