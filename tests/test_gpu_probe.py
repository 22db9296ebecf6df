"""fgb_hbm_probe: the reference access patterns move exactly the bytes they
document (they calibrate the bandwidth figures, so they must not skip work)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def _strided_layout(x):
    """Expected FGB_PROBE_STRIDED_READ output of x [rows, cols], from the header's map."""
    rows, cols = x.shape
    ntb = rows // 128
    out = np.empty(rows * cols, dtype=np.uint8)
    for b in range(ntb * (cols // 128)):
        tb, cb = b % ntb, b // ntb
        for lane in range(64):
            tsub, csub = lane & 7, lane >> 3
            for j in range(16):
                r = tb * 128 + tsub * 16 + j
                c = cb * 128 + csub * 16
                o = b * 16384 + j * 1024 + lane * 16
                out[o:o + 16] = x[r, c:c + 16]
    return out.reshape(rows, cols)


@pytest.mark.parametrize("rows,cols", [(128, 128), (256, 384)])
def test_hbm_probe_patterns(rows, cols):
    import torch
    import fine_grained_blockwise_amd as fgb
    g = torch.Generator().manual_seed(rows + cols)
    x = torch.randint(0, 256, (rows, cols), dtype=torch.uint8, generator=g)
    xd = x.cuda()
    xn = x.numpy()

    d = torch.full_like(xd, 7)
    fgb.fgb_hbm_probe(xd, d, fgb.PROBE_COPY)
    assert torch.equal(d.cpu(), x)

    fgb.fgb_hbm_probe(None, d, fgb.PROBE_FILL)
    assert int(d.count_nonzero()) == 0

    r = torch.empty(rows * cols // 256, dtype=torch.uint8, device="cuda")
    fgb.fgb_hbm_probe(xd, r, fgb.PROBE_READ)
    words = xn.reshape(-1, 4096 // 16, 16)  # 4 KB blocks of 16-byte words
    expect = np.bitwise_xor.reduce(words, axis=1).reshape(-1)
    assert np.array_equal(r.cpu().numpy(), expect)

    s = torch.empty_like(xd)
    fgb.fgb_hbm_probe(xd, s, fgb.PROBE_STRIDED_READ)
    assert np.array_equal(s.cpu().numpy(), _strided_layout(xn))

    back = torch.empty_like(xd)
    fgb.fgb_hbm_probe(s, back, fgb.PROBE_STRIDED_WRITE)
    assert torch.equal(back.cpu(), x)
