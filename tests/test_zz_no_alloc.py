"""permute_pad_noalloc (the entry point for callers that cannot allocate)
against permute_pad with a caller workspace: bit for bit on every output, on
two calls in a row, the second with a smaller input (fewer tokens, experts
and columns), so the second call runs on scratch contents the first call left
behind.  The small case is also checked against the oracle."""
import sys

import numpy as np
import pytest
import torch

import oracle as O
import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _inputs(T, H, G, topk, seed):
    idx, _ = synth.routing(T, G, topk, 1.1, seed)
    g = torch.Generator().manual_seed(seed + 100)
    xq = torch.randint(0, 256, (T, H), generator=g, dtype=torch.int32).to(torch.uint8)
    xq[(xq & 0x7F) == 0x7F] ^= 1
    xs = torch.randint(107, 132, (T, H // 128), generator=g, dtype=torch.int32).to(torch.uint8)
    return xq, xs, torch.from_numpy(np.ascontiguousarray(idx)).to(torch.int32)


def test_permute_pad_noalloc_matches_workspace_form_on_two_calls():
    import fine_grained_blockwise_amd as fgb
    for T, H, G, topk, seed in [(16384, 7168, 32, 8, 0), (700, 512, 6, 4, 1)]:
        say(f"permute_pad_noalloc T={T} H={H} G={G} topk={topk}")
        xq, xs, idx = _inputs(T, H, G, topk, seed)
        xq_d, xs_d, idx_d = xq.to(DEV), xs.to(DEV), idx.to(DEV)
        ref = fgb.permute_pad(xq_d, xs_d, idx_d, G, 16)
        M_cap = ref[0].shape[0]
        # outputs allocated by the caller beforehand, filled with other bytes
        out = (torch.full((M_cap, H), 0xAB, dtype=torch.uint8, device=DEV),
               torch.full((M_cap, H // 128), 0xCD, dtype=torch.uint8, device=DEV),
               torch.full((T, topk), -7, dtype=torch.int32, device=DEV),
               torch.full((G + 1,), -7, dtype=torch.int32, device=DEV))
        got = fgb.permute_pad_noalloc(xq_d, xs_d, idx_d, G, out, 16)
        torch.cuda.synchronize()
        assert all(g is o for g, o in zip(got, out))
        off = ref[3].cpu().numpy()
        used = int(off[G])
        assert np.array_equal(got[3].cpu().numpy(), off)
        assert np.array_equal(got[2].cpu().numpy(), ref[2].cpu().numpy())
        assert np.array_equal(got[1][:used].cpu().numpy(), ref[1][:used].cpu().numpy())
        assert np.array_equal(got[0][:used].cpu().numpy(), ref[0][:used].cpu().numpy())
        # rows past off[G] are left as the caller wrote them
        assert bool((got[0][used:] == 0xAB).all()) and bool((got[1][used:] == 0xCD).all())
        if T <= 1024:
            oq, os_, orm, ooff, oused = O.permute_pad(xq.numpy(), xs.numpy(), idx.numpy(), G, 16)
            assert oused == used and np.array_equal(ooff, off)
            assert np.array_equal(got[2].cpu().numpy(), orm)
            assert np.array_equal(got[0][:used].cpu().numpy(), oq[:used])
            assert np.array_equal(got[1][:used].cpu().numpy(), os_[:used])
