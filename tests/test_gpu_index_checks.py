"""Range checks on indices read from device buffers.

Out-of-range expert ids, row-map entries and group offsets are caller errors.
Each kernel that reads one keeps every access inside its buffer, applies the
documented stand-in and records the event in the record that
moe_index_errors() returns.  Valid calls record nothing.

Every case below feeds bad indices that the kernels' own checks handle:
  * clamped ids;
  * rows that are skipped or read as zeros;
  * groups that are dropped.
Guard rows past each output show that nothing is written outside it."""
import numpy as np
import pytest
import torch

import oracle as O
from moe_inputs import WORKLOADS, Workload, make_inputs, random_topk_ids, round_to_bf16
from tests._gpu import DEV, TOL_F32, TOL_ONE_ROUNDING, bits, dev, host, rel, say

pytestmark = pytest.mark.gpu

L = None


@pytest.fixture(autouse=True)
def _native_lib():
    """The HIP library (raises if not built); each test starts from an empty
    record."""
    global L
    import mixture_experts_layer_gating_amd._lib as lib
    L = lib
    torch.cuda.synchronize()
    lib.moe_index_errors(clear=True)


def _normal(shape, seed, scale=1.0):
    a = (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)
    return round_to_bf16(a)


@pytest.mark.parametrize("wl", [WORKLOADS["tiny"],
                                Workload("idx_bf16", T=1024, d=512, E=8, k=2, F=384,
                                         dtype="bf16", w_std=0.02, seed=1100)],
                         ids=lambda w: w.name)
def test_valid_layer_records_nothing(wl):
    from mixture_experts_layer_gating_amd.layer import MoELayer
    say(f"index record stays empty: layer {wl.name}")
    inp = make_inputs(wl)
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    layer = MoELayer(wl.T, wl.d, wl.E, wl.k, wl.F, dtype=tdt, device=DEV)
    x, wr, w1, w2, dy = (dev(a, tdt) for a in (inp.x, inp.wr, inp.w1, inp.w2, inp.dy))
    layer.forward(x, wr, w1, w2)
    layer.backward(dy)
    torch.cuda.synchronize()
    assert L.moe_index_errors() == 0


def test_expert_ids_clamped_and_recorded():
    T, E, k = 96, 16, 4
    say("index record: expert ids")
    logits = np.random.default_rng(1).standard_normal((T, E)).astype(np.float32)
    forced = random_topk_ids(T, k, E, seed=2).astype(np.int32)
    forced[3, 1] = E + 5
    ld = dev(logits)
    idx = torch.empty(T, k, dtype=torch.int32, device=DEV)
    w = torch.empty(T, k, dtype=torch.float32, device=DEV)
    probs = torch.empty(T, E, dtype=torch.float32, device=DEV)
    L.moe_route_topk(ld, None, T, E, k, 0, dev(forced), idx, w, probs)
    assert L.moe_index_errors() == L.MOE_IDXERR_EXPERT
    assert host(idx)[3, 1] == E - 1
    assert L.moe_index_errors() == 0  # cleared by the previous read

    # routing backward: a bad topk_idx gives the result of the clamped id
    good = host(idx).astype(np.int32)
    bad = good.copy()
    bad[7, 2] = -1
    clamped = bad.copy()
    clamped[7, 2] = 0
    dtw = dev(np.random.default_rng(3).standard_normal((T, k)).astype(np.float32))
    z_bad = torch.empty(T, E, dtype=torch.float32, device=DEV)
    z_ref = torch.empty_like(z_bad)
    L.moe_route_topk_bwd(probs, dev(bad), dtw, T, E, k, 0, z_bad, L.MOE_F32)
    assert L.moe_index_errors() == L.MOE_IDXERR_EXPERT
    L.moe_route_topk_bwd(probs, dev(clamped), dtw, T, E, k, 0, z_ref, L.MOE_F32)
    assert L.moe_index_errors() == 0
    np.testing.assert_array_equal(host(z_bad), host(z_ref))

    # counting
    ids = random_topk_ids(T, k, E, seed=4).astype(np.int32)
    ids[0, 0] = -9
    counts = torch.empty(E, dtype=torch.int32, device=DEV)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    dest = torch.empty(T * k, dtype=torch.int32, device=DEV)
    src = torch.empty(T * k, dtype=torch.int32, device=DEV)
    nb = L.moe_count_index_workspace_size(T, k, E)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    L.moe_count_index(dev(ids), T, k, E, counts, offsets, dest, src, ws, nb)
    assert L.moe_index_errors() == L.MOE_IDXERR_EXPERT
    np.testing.assert_array_equal(host(counts), O.count_tokens(np.clip(ids, 0, E - 1), E))


def test_row_maps_skip_bad_rows():
    """permute: a bad dest entry writes nothing; combine: it contributes
    nothing; combine backward: it writes nothing and its dw is 0."""
    T, k, E, d = 40, 4, 6, 64
    M, G = T * k, 8  # rows, guard rows past the end
    say("index record: dest rows")
    bf, code = torch.bfloat16, L.MOE_BF16
    ids = random_topk_ids(T, k, E, seed=5)
    _, _, dest, src = O.build_index(ids, E)
    dest = np.asarray(dest, dtype=np.int32)
    badslots = [5, 11, 20]
    bad = dest.copy()
    bad[5], bad[11], bad[20] = M + 3, -1, 1 << 30
    x = _normal((T, d), 6)
    sentinel = 7.0
    xp_full = torch.full((M + G, d), sentinel, dtype=bf, device=DEV)
    L.moe_permute(dev(x, bf), dev(bad), T, k, d, code, xp_full[:M])
    assert L.moe_index_errors() == L.MOE_IDXERR_ROW
    got = host(xp_full)
    want = np.full((M + G, d), sentinel)
    for s in range(M):
        if s not in badslots:
            want[dest[s]] = x[s // k]
    np.testing.assert_array_equal(got, want)

    yp = _normal((M, d), 7)
    w = np.random.default_rng(8).random((T, k)).astype(np.float32)
    w_masked = w.copy().reshape(-1)
    w_masked[badslots] = 0.0
    w_masked = w_masked.reshape(T, k)
    y = torch.empty(T, d, dtype=bf, device=DEV)
    L.moe_unpermute(dev(yp, bf), dev(bad), dev(w), T, k, d, code, y)
    assert L.moe_index_errors() == L.MOE_IDXERR_ROW
    assert rel(host(y), O.combine(yp, dest, w_masked, k)) <= TOL_ONE_ROUNDING

    dy = _normal((T, d), 9)
    dyp_full = torch.full((M + G, d), sentinel, dtype=bf, device=DEV)
    dw = torch.full((T, k), 5.0, dtype=torch.float32, device=DEV)
    L.moe_unpermute_bwd(dev(dy, bf), dev(yp, bf), dev(bad), dev(w), T, k, d, code,
                        dyp_full[:M], dw)
    assert L.moe_index_errors() == L.MOE_IDXERR_ROW
    rdyp, rdw = O.combine_backward(dy, yp, dest, w, k)
    got = host(dyp_full)
    keep = np.ones(M, dtype=bool)
    keep[dest[badslots]] = False
    assert (got[:M][~keep] == sentinel).all() and (got[M:] == sentinel).all()
    assert rel(got[:M][keep], rdyp[keep]) <= TOL_ONE_ROUNDING
    gdw = host(dw).reshape(-1)
    assert (gdw[badslots] == 0).all()
    ok = np.setdiff1d(np.arange(M), badslots)
    assert rel(gdw[ok], rdw.reshape(-1)[ok]) <= TOL_F32


@pytest.mark.parametrize("offsets", [[0, 100, 300, 100, 100],   # group 2 reversed
                                     [0, 100, 400, 400, 300]])  # groups 1-3 leave [0, M]
def test_bad_group_offsets_skip_the_group(offsets):
    M, K, N, E = 300, 64, 128, 4
    say(f"index record: group offsets {offsets}")
    bf, code = torch.bfloat16, L.MOE_BF16
    off = np.asarray(offsets, dtype=np.int32)
    good = [e for e in range(E) if 0 <= off[e] <= off[e + 1] <= M]
    a, b, dc = _normal((M, K), 10), _normal((E, K, N), 11, 0.05), _normal((M, N), 12)
    ad, bd, dcd, offd = dev(a, bf), dev(b, bf), dev(dc, bf), dev(off)
    sentinel = 3.0
    c = torch.full((M, N), sentinel, dtype=torch.float32, device=DEV)
    L.moe_grouped_gemm_fwd(ad, bd, offd, M, K, N, E, code, c, L.MOE_F32)
    assert L.moe_index_errors() == L.MOE_IDXERR_GROUP
    # the valid groups against the oracle, on offsets holding only them
    covered = np.zeros(M, dtype=bool)
    for e in good:
        covered[off[e]:off[e + 1]] = True
    ref = np.zeros((M, N))
    for e in good:  # each valid group as a one-group oracle call
        r = slice(off[e], off[e + 1])
        n = int(off[e + 1] - off[e])
        ref[r] = O.grouped_matmul(a[r], b[e:e + 1], np.array([0, n]))
    got = host(c)
    assert (got[~covered] == sentinel).all()
    if covered.any():
        assert rel(got[covered], ref[covered]) <= TOL_F32
    # weight gradient: zero for the skipped groups
    nb = L.moe_grouped_gemm_workspace_size(M, K, N, E, code)
    ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=DEV)
    db = torch.full((E, K, N), sentinel, dtype=torch.float32, device=DEV)
    L.moe_grouped_gemm_bwd(ad, bd, dcd, offd, M, K, N, E, code, None, None, db, ws, nb)
    assert L.moe_index_errors() == L.MOE_IDXERR_GROUP
    gdb = host(db)
    for e in range(E):
        if e in good:
            r = slice(off[e], off[e + 1])
            n = int(off[e + 1] - off[e])
            want = O.grouped_matmul_backward(a[r], b[e:e + 1], dc[r], np.array([0, n]))[1][0]
            if n > 0:
                assert rel(gdb[e], want) <= TOL_F32
            else:
                assert not gdb[e].any()
        else:
            assert not gdb[e].any(), e


def test_gather_rows_out_of_range_read_zeros():
    """A row-map entry outside [0, x_phys * x_div) reads a zero row: the
    gathered calls then equal the plain calls on the permuted copy with that
    row zeroed, bit for bit."""
    T, k, d, F, E = 256, 2, 128, 64, 4
    M = T * k
    say("index record: gathered rows")
    bf, code = torch.bfloat16, L.MOE_BF16
    off = np.array([0, 100, 260, 400, M], dtype=np.int32)
    src = np.random.default_rng(13).permutation(M).astype(np.int32)
    badrows = [7, 130, 301]
    bad = src.copy()
    bad[7], bad[130], bad[301] = M + 5, -3, 1 << 29
    x = _normal((T, d), 14)
    w1 = _normal((E, d, 2 * F), 15, 0.05)
    dh = _normal((M, 2 * F), 16)
    xp = x[src // k]
    xp[badrows] = 0.0
    xd, badd, w1d, offd, dhd, xpd = dev(x, bf), dev(bad), dev(w1, bf), dev(off), dev(dh, bf), dev(xp, bf)
    h0 = torch.zeros(M, 2 * F, dtype=bf, device=DEV)
    a0 = torch.zeros(M, F, dtype=bf, device=DEV)
    L.moe_grouped_gemm_swiglu_fwd(xpd, w1d, offd, M, d, F, E, code, h0, a0)
    assert L.moe_index_errors() == 0
    h1, a1 = torch.zeros_like(h0), torch.zeros_like(a0)
    L.moe_grouped_gemm_swiglu_fwd_gather(xd, badd, k, T, w1d, offd, M, d, F, E, code, h1, a1)
    assert L.moe_index_errors() == L.MOE_IDXERR_GATHER
    np.testing.assert_array_equal(bits(h1), bits(h0))
    np.testing.assert_array_equal(bits(a1), bits(a0))
    nb = L.moe_grouped_gemm_workspace_size(M, d, 2 * F, E, code)
    ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=DEV)
    db0 = torch.full((E, d, 2 * F), 7.0, dtype=torch.float32, device=DEV)
    db1 = torch.full_like(db0, -7.0)
    L.moe_grouped_gemm_bwd(xpd, w1d, dhd, offd, M, d, 2 * F, E, code, None, None, db0, ws, nb)
    assert L.moe_index_errors() == 0
    L.moe_grouped_gemm_bwd_gather(xd, badd, k, T, w1d, dhd, offd, M, d, 2 * F, E, code, None,
                                  None, db1, ws, nb)
    assert L.moe_index_errors() == L.MOE_IDXERR_GATHER
    np.testing.assert_array_equal(host(db1), host(db0))
