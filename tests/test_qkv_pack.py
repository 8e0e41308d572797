"""The fused QKV path's weight packing (host logic, CPU): the tile order that qi_gemm_qkv_tiles reads
(include/qi.h) -- for each head h the 128 rows of K_h, then the rows of V_h dims 0..63; then the rows
of V_h dims 64..127 for each head; then the Q rows -- checked row by row against that definition, and
the unpacking that undoes it."""
import pytest

torch = pytest.importorskip("torch")

from image_generation_qi_amd import runtime as rt  # noqa: E402


@pytest.mark.parametrize("H", [1, 2, 3, 24])
def test_pack_qkv_tiles_row_order(H):
    D = 128 * H
    w = torch.arange(3 * D, dtype=torch.float64)[:, None] * torch.ones(1, 5, dtype=torch.float64)
    p = rt.pack_qkv_tiles(w, H)
    assert p.shape == w.shape and p.is_contiguous()
    src = p[:, 0].long().tolist()
    want = []
    for h in range(H):
        want += [D + 128 * h + d for d in range(128)]           # K_h
        want += [2 * D + 128 * h + d for d in range(64)]        # V_h dims 0..63
    for h in range(H):
        want += [2 * D + 128 * h + 64 + d for d in range(64)]   # V_h dims 64..127
    want += list(range(D))                                      # Q
    assert src == want
    # 192-row tile h (h < H) holds the whole K of head h in its first 128 rows
    for h in range(H):
        assert src[192 * h] == D + 128 * h and src[192 * h + 127] == D + 128 * h + 127
    assert torch.equal(rt.unpack_qkv_tiles(p, H), w)


def test_pack_qkv_tiles_bias_follows_rows():
    # a bias table computed from the packed weights is the packed bias: (s W^T)[perm] = s (W[perm])^T
    H, Din = 2, 16
    g = torch.Generator().manual_seed(5)
    w = torch.randn((3 * 128 * H, Din), generator=g, dtype=torch.float64)
    s = torch.randn((3, Din), generator=g, dtype=torch.float64)
    perm = rt.pack_qkv_tiles(torch.arange(w.shape[0], dtype=torch.float64)[:, None], H)[:, 0].long()
    assert torch.equal(s @ rt.pack_qkv_tiles(w, H).T, (s @ w.T)[:, perm])
