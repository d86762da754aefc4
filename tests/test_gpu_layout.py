"""GPU: the slot layout step (moe_pack_expert) against the permutation it is
documented to be. K-quant: in each matrix, block s of row r moves from
(r * nsb + s) * B to ((r / 8) * nsb + s) * 8 * B + (r % 8) * B. MXFP4: each
matrix's codes and scales are cut into tiles of 64 rows x 128 columns, tiles in
row-major tile order, each tile's rows in order (codes first, then scales)."""
import pytest
import torch

import mixture_experts_ffn_gemv_amd as moe
import synthetic as S

pytestmark = pytest.mark.gpu


def panel_order(mat, rows, nsb, B):
    """Plain row order [rows * nsb * B] -> panel order, by reshaping."""
    return mat.reshape(rows // 8, 8, nsb, B).permute(0, 2, 1, 3).reshape(-1)


@pytest.mark.parametrize("dim,inter", [(256, 256), (512, 768)])
def test_pack_expert_is_the_panel_permutation(dim, inter):
    shape = S.LayerShape(dim, inter, 4, 2)
    cfg = moe.make_cfg(dim, inter, 4, 2)
    size, o1, o3, o2 = S.expert_layout(shape)
    src = S.make_expert_slot(shape, 7, 1).cuda()
    dst = torch.full_like(src, 0xAB)
    moe.moe_pack_expert(cfg, src, dst)
    torch.cuda.synchronize()
    ref = torch.cat([
        panel_order(src[o1:o3], inter, dim // 256, 84),
        panel_order(src[o3:o2], inter, dim // 256, 84),
        panel_order(src[o2:], dim, inter // 256, 110),
    ])
    assert torch.equal(dst, ref)


def test_pack_expert_rejects_overlap():
    cfg = moe.make_cfg(256, 256, 4, 2)
    buf = torch.zeros(2 * S.expert_layout(S.LayerShape(256, 256, 4, 2))[0], dtype=torch.uint8, device="cuda")
    with pytest.raises(moe.MoeError):
        moe.moe_pack_expert(cfg, buf, buf[16:])


@pytest.mark.parametrize("dim,inter", [(256, 256), (512, 768)])
def test_pack_expert_mxfp4_is_the_tile_permutation(dim, inter):
    shape = S.LayerShape(dim, inter, 4, 2)
    cfg = moe.make_cfg(dim, inter, 4, 2, expert_fmt=moe.MOE_EXPERT_MXFP4)
    size, o1, o3, o2 = S.expert_layout(shape, "fp4")
    src = S.make_expert_slot(shape, 7, 1, fmt="fp4").cuda()
    dst = torch.full_like(src, 0xAB)
    moe.moe_pack_expert(cfg, src, dst)
    torch.cuda.synchronize()

    def tiled(mat, rows, cols):
        cb = rows * cols // 2
        codes = mat[:cb].reshape(rows // 64, 64, cols // 128, 64).permute(0, 2, 1, 3).reshape(-1)
        scales = mat[cb:].reshape(rows // 64, 64, cols // 128, 4).permute(0, 2, 1, 3).reshape(-1)
        return torch.cat([codes, scales])

    ref = torch.cat([tiled(src[o1:o3], inter, dim), tiled(src[o3:o2], inter, dim), tiled(src[o2:], dim, inter)])
    assert torch.equal(dst, ref)
    # a probe: the scale of row 70, columns 160..191 of W2 (tile 1 * inter/128 + 1, row 6, block 1)
    cb2 = dim * inter // 2
    t = 1 * (inter // 128) + 1
    assert dst[o2 + cb2 + 256 * t + 6 * 4 + 1] == src[o2 + cb2 + 70 * (inter // 32) + 5]
