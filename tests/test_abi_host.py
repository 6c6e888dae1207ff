"""The C-ABI library loads, exports every symbol the header declares, and its
host-side validation returns the documented status codes (CPU only: no call
here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

L = pytest.importorskip("mixture_experts_layer_gating_amd._lib",
                        reason="libmoe.so not built")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


def test_header_symbols_exported():
    names = _declared()
    assert len(names) >= 14
    lib = ctypes.CDLL(L.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L.SYMBOLS)


def test_version_and_error_string():
    assert L.moe_version().startswith("moe-mi355x")
    assert isinstance(L.moe_last_error(), str)


def test_index_error_bits_match_header():
    text = open(HEADER).read()
    bits = {m.group(1): int(m.group(2)) for m in
            re.finditer(r"#define (MOE_IDXERR_[A-Z]+) (\d+)u", text)}
    assert bits == {n: getattr(L, n) for n in
                    ("MOE_IDXERR_EXPERT", "MOE_IDXERR_ROW", "MOE_IDXERR_GROUP", "MOE_IDXERR_GATHER")}
    assert len(set(bits.values())) == 4 and all(v & (v - 1) == 0 for v in bits.values())
    # A null mask is refused on the host, before any device work.
    assert _rc("moe_index_errors", None, 1, None) == L.MOE_ERR_INVALID_ARG
    assert "mask" in L.moe_last_error()


def _rc(name, *args):
    return getattr(L.lib(), name)(*args)


FAKE = 0x1000  # never dereferenced: validation fails before any device work


def test_route_validation():
    assert _rc("moe_route_topk", FAKE, None, 0, 8, 2, 0, None, FAKE, FAKE, None, None) == L.MOE_ERR_INVALID_ARG
    assert _rc("moe_route_topk", FAKE, None, 4, 8, 9, 0, None, FAKE, FAKE, None, None) == L.MOE_ERR_INVALID_ARG
    assert "k" in L.moe_last_error()
    assert _rc("moe_route_topk", FAKE, None, 4, 2048, 2, 0, None, FAKE, FAKE, None, None) == L.MOE_ERR_UNSUPPORTED
    assert _rc("moe_route_topk", FAKE, None, 4, 64, 33, 0, None, FAKE, FAKE, None, None) == L.MOE_ERR_UNSUPPORTED
    assert _rc("moe_route_topk", None, None, 4, 8, 2, 0, None, FAKE, FAKE, None, None) == L.MOE_ERR_INVALID_ARG
    assert _rc("moe_route_topk_bwd", FAKE, FAKE, FAKE, 4, 8, 2, 0, FAKE, 5, None) == L.MOE_ERR_UNSUPPORTED


def test_count_index_validation_and_workspace():
    ws = L.moe_count_index_workspace_size(8192, 8, 64)
    assert ws >= 2 * 64 * 2 * 4 and ws % 256 == 0
    assert L.moe_count_index_workspace_size(0, 8, 64) == 0
    assert _rc("moe_count_index", FAKE, 16, 2, 4, FAKE, FAKE, FAKE, FAKE, None, 0, None) == L.MOE_ERR_WORKSPACE
    need = L.moe_count_index_workspace_size(16, 2, 4)
    assert _rc("moe_count_index", FAKE, 16, 2, 4, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, None) == L.MOE_ERR_WORKSPACE
    assert _rc("moe_count_index", FAKE, 16, 5, 4, FAKE, FAKE, FAKE, FAKE, FAKE, need, None) == L.MOE_ERR_INVALID_ARG
    assert _rc("moe_count_index", FAKE + 4, 16, 2, 4, FAKE, FAKE, FAKE, None, FAKE, need, None) == L.MOE_ERR_INVALID_ARG


def test_move_and_act_validation():
    assert _rc("moe_permute", FAKE, FAKE, 4, 2, 12, L.MOE_BF16, FAKE, None) == L.MOE_ERR_UNSUPPORTED
    assert _rc("moe_permute", FAKE, FAKE, 4, 2, 16, 9, FAKE, None) == L.MOE_ERR_UNSUPPORTED
    assert _rc("moe_unpermute", None, FAKE, FAKE, 4, 2, 16, L.MOE_BF16, FAKE, None) == L.MOE_ERR_INVALID_ARG
    assert _rc("moe_unpermute_bwd", FAKE, FAKE, FAKE, None, 4, 2, 16, L.MOE_BF16, FAKE, FAKE, None) == L.MOE_ERR_INVALID_ARG
    assert _rc("moe_act_fwd", FAKE, 4, 12, L.MOE_BF16, FAKE, None) == L.MOE_ERR_UNSUPPORTED
    assert _rc("moe_act_bwd", FAKE, FAKE, 0, 16, L.MOE_BF16, FAKE, None) == L.MOE_ERR_INVALID_ARG


def test_gemm_validation_and_workspace():
    # Router-like weight gradient (one group, few output tiles) uses split partials.
    ws = L.moe_grouped_gemm_workspace_size(8192, 2048, 64, 1, L.MOE_BF16)
    assert ws > 0 and ws % (2048 * 64 * 4) == 0
    # Expert weight gradients of a large layer need none; float32 never does.
    assert L.moe_grouped_gemm_workspace_size(65536, 2048, 2048, 64, L.MOE_BF16) == 0
    assert L.moe_grouped_gemm_workspace_size(8192, 2048, 64, 1, L.MOE_F32) == 0
    assert _rc("moe_grouped_gemm_fwd", FAKE, FAKE, None, 4, 8, 8, 1, L.MOE_BF16, FAKE, L.MOE_BF16, None, 0, None) == L.MOE_ERR_INVALID_ARG
    assert _rc("moe_grouped_gemm_fwd", FAKE, FAKE, FAKE, 4, 8, 8, 1, L.MOE_F32, FAKE, L.MOE_BF16, None, 0, None) == L.MOE_ERR_UNSUPPORTED
    assert _rc("moe_grouped_gemm_fwd", FAKE, FAKE, FAKE, 0, 8, 8, 1, L.MOE_BF16, FAKE, L.MOE_BF16, None, 0, None) == L.MOE_ERR_INVALID_ARG
    assert _rc("moe_grouped_gemm_bwd", FAKE, FAKE, FAKE, FAKE, 8192, 2048, 64, 1, L.MOE_BF16, None, None, FAKE, None, 0, None) == L.MOE_ERR_WORKSPACE
    assert _rc("moe_grouped_gemm_bwd", FAKE, None, FAKE, FAKE, 16, 8, 8, 1, L.MOE_BF16, FAKE, None, None, None, 0, None) == L.MOE_ERR_INVALID_ARG
    # fused GEMM 1 + SwiGLU
    assert _rc("moe_grouped_gemm_swiglu_fwd", FAKE, FAKE, FAKE, 16, 8, 12, 1, L.MOE_BF16, FAKE, FAKE, None) == L.MOE_ERR_UNSUPPORTED
    assert _rc("moe_grouped_gemm_swiglu_fwd", FAKE, FAKE, FAKE, 16, 8, 16, 1, L.MOE_BF16, None, FAKE, None) == L.MOE_ERR_INVALID_ARG
    assert _rc("moe_grouped_gemm_swiglu_fwd", FAKE, FAKE, None, 16, 8, 16, 1, L.MOE_BF16, FAKE, FAKE, None) == L.MOE_ERR_INVALID_ARG
    assert _rc("moe_grouped_gemm_swiglu_fwd", FAKE, FAKE, FAKE, 16, 8, 0, 1, L.MOE_BF16, FAKE, FAKE, None) == L.MOE_ERR_INVALID_ARG
    assert _rc("moe_grouped_gemm_swiglu_fwd", FAKE, FAKE, FAKE, 16, 8, 16, 1, L.MOE_BF16, FAKE, FAKE + 8, None) == L.MOE_ERR_INVALID_ARG
    assert L.moe_grouped_gemm_plan(3, 65536, 2048, 2048, 64, L.MOE_BF16)["tile_n"] == 256
    assert L.moe_grouped_gemm_plan(3, 2048, 512, 64, 1, L.MOE_BF16)["tile_n"] == 128
    # the MFMA path moves 16-byte vectors: misaligned operands are rejected
    odd = FAKE + 8
    assert _rc("moe_grouped_gemm_fwd", odd, FAKE, FAKE, 4, 8, 8, 1, L.MOE_BF16, FAKE, L.MOE_BF16, None, 0, None) == L.MOE_ERR_INVALID_ARG
    assert _rc("moe_grouped_gemm_fwd", FAKE, FAKE, FAKE, 4, 8, 8, 1, L.MOE_BF16, odd, L.MOE_F32, None, 0, None) == L.MOE_ERR_INVALID_ARG
    assert _rc("moe_grouped_gemm_bwd", FAKE, FAKE, FAKE, FAKE, 16, 8, 8, 1, L.MOE_BF16, odd, None, None, None, 0, None) == L.MOE_ERR_INVALID_ARG
    assert _rc("moe_grouped_gemm_bwd", FAKE, FAKE, FAKE, FAKE, 16, 8, 8, 1, L.MOE_BF16, FAKE, odd, None, None, 0, None) == L.MOE_ERR_INVALID_ARG


def test_gathered_gemm_validation():
    # swiglu_fwd_gather(x, x_rows, x_div, x_phys, b, offsets, M, K, F, E, dtype, h, act, stream)
    ok = (FAKE, FAKE, 8, 64, FAKE, FAKE, 512, 64, 32, 4, L.MOE_BF16, FAKE, FAKE, None)
    def sw(**kw):
        args = list(ok)
        for i, v in kw.items():
            args[int(i[1:])] = v
        return _rc("moe_grouped_gemm_swiglu_fwd_gather", *args)
    assert sw(a1=None) == L.MOE_ERR_INVALID_ARG          # null row map
    assert sw(a2=0) == L.MOE_ERR_INVALID_ARG             # divisor < 1
    assert sw(a3=0) == L.MOE_ERR_INVALID_ARG             # no physical rows
    assert sw(a3=1 << 24) == L.MOE_ERR_UNSUPPORTED       # rows past 24 bits
    assert sw(a8=36) == L.MOE_ERR_UNSUPPORTED            # F not a multiple of 8
    assert sw(a10=L.MOE_F32) == L.MOE_ERR_UNSUPPORTED    # float32: no MFMA path
    assert sw(a0=FAKE + 8) == L.MOE_ERR_INVALID_ARG      # misaligned x
    assert sw(a0=None) == L.MOE_ERR_INVALID_ARG
    # bwd_gather(a, a_rows, a_div, a_phys, b, dc, offsets, M, K, N, E, dtype, da, da_add, db,
    #            ws, ws_bytes, stream)
    okb = (FAKE, FAKE, 8, 64, FAKE, FAKE, FAKE, 512, 64, 64, 4, L.MOE_BF16, None, None, FAKE,
           None, 0, None)
    def bw(**kw):
        args = list(okb)
        for i, v in kw.items():
            args[int(i[1:])] = v
        return _rc("moe_grouped_gemm_bwd_gather", *args)
    assert bw(a1=None) == L.MOE_ERR_INVALID_ARG
    assert bw(a2=-1) == L.MOE_ERR_INVALID_ARG
    assert bw(a3=1 << 20, a8=2048) == L.MOE_ERR_UNSUPPORTED  # physical rows * K >= 2^30
    assert bw(a8=12) == L.MOE_ERR_UNSUPPORTED            # K not a multiple of 8
    assert bw(a11=L.MOE_F32) == L.MOE_ERR_UNSUPPORTED
    assert bw(a14=FAKE + 4) == L.MOE_ERR_INVALID_ARG     # misaligned db


def test_count_index_noalloc_validation():
    """The allocation-free variant validates like moe_count_index and refuses
    shapes whose block tables exceed its static scratch, all before any
    device call."""
    assert L.MOE_NOALLOC_SCRATCH_BYTES == 4 << 20
    assert _rc("moe_count_index_noalloc", FAKE, 0, 2, 4, FAKE, FAKE, FAKE, FAKE, None) == L.MOE_ERR_INVALID_ARG
    assert _rc("moe_count_index_noalloc", FAKE, 16, 5, 4, FAKE, FAKE, FAKE, FAKE, None) == L.MOE_ERR_INVALID_ARG
    assert _rc("moe_count_index_noalloc", None, 16, 2, 4, FAKE, FAKE, FAKE, FAKE, None) == L.MOE_ERR_INVALID_ARG
    T, k, E = 262656, 1, 1024
    assert L.moe_count_index_workspace_size(T, k, E) > L.MOE_NOALLOC_SCRATCH_BYTES
    assert _rc("moe_count_index_noalloc", FAKE, T, k, E, FAKE, FAKE, FAKE, FAKE, None) == L.MOE_ERR_UNSUPPORTED
    assert "scratch" in L.moe_last_error()


def test_layer_refuses_mismatched_inputs():
    """MoELayer checks every input against its shape, dtype and device before
    any library call (the kernels size buffer ranges from the layer's shape,
    not from the tensors).  Built on the host: no call reaches the library."""
    import torch

    from mixture_experts_layer_gating_amd.layer import MoELayer
    T, d, E, k, F = 16, 64, 8, 2, 32
    bf = torch.bfloat16
    lay = MoELayer(T, d, E, k, F, dtype=bf, device="cpu", gather_dy=False)
    x, wr = torch.zeros(T, d, dtype=bf), torch.zeros(d, E, dtype=bf)
    w1, w2 = torch.zeros(E, d, 2 * F, dtype=bf), torch.zeros(E, F, d, dtype=bf)
    bad = [
        dict(x=torch.zeros(T + 1, d, dtype=bf)),
        dict(x=torch.zeros(T, d, dtype=torch.float32)),
        dict(wr=torch.zeros(E, d, dtype=bf)),
        dict(w1=torch.zeros(E, d, F, dtype=bf)),
        dict(w2=torch.zeros(E, d, F, dtype=bf)),
        dict(bias=torch.zeros(E, dtype=torch.float64)),
        dict(bias=torch.zeros(E + 1, dtype=torch.float32)),
        dict(forced_idx=torch.zeros(T, k, dtype=torch.int64)),
        dict(x=torch.zeros(d, T, dtype=bf).t()),
    ]
    for kw in bad:
        args = dict(x=x, wr=wr, w1=w1, w2=w2)
        args.update(kw)
        with pytest.raises(ValueError):
            lay.forward(**args)
    assert lay.xp is None  # the gathered path keeps no permuted copy of x
    # what each recompute mode keeps between the passes
    Tk = T * k
    full = lay.saved_bytes("none")
    assert full["h"] == Tk * 2 * F * 2 and full["a"] == Tk * F * 2 and full["yp"] == Tk * d * 2
    assert full["dest"] == full["src"] == Tk * 4 and full["probs"] == T * E * 4
    act = lay.saved_bytes("act")
    assert set(full) - set(act) == {"a"} and sum(full.values()) - sum(act.values()) == Tk * F * 2
    assert lay.saved_bytes("layer") == {}
    # reading dy through the row map in GEMM 2's backward, the backward pass
    # never reads `a`: no mode keeps it, and dyp is not allocated
    lay2 = MoELayer(T, d, E, k, F, dtype=bf, device="cpu")
    assert lay2.gather_dy and lay2.dyp is None and not lay.gather_dy and lay.dyp is not None
    assert lay2.saved_bytes("none") == lay2.saved_bytes("act") == act
    with pytest.raises(ValueError):
        MoELayer(T, d, E, k, F, dtype=bf, device="cpu", recompute="all")
    with pytest.raises(RuntimeError):
        lay.backward(torch.zeros(T, d, dtype=bf))
