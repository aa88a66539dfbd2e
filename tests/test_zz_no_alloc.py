"""gae_scan_noalloc (the allocation-free form of gae_scan) against gae_scan
through the C ABI: bit-identical results on two calls in a row, the second
with a smaller input, then a scan of at most 512 steps (which needs no
scratch) of more episodes than the scratch holds carries, one that fills
the scratch exactly, and a refused oversized scan; each result also within
the fp32 tolerance of the oracle (on a spread of episodes at the largest
size)."""
import numpy as np
import pytest

import oracle
import synthdata
from parity import close_mask, gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X")]


def _scan(r, v, d, lv, noalloc):
    import torch
    import rl_experience_collection_amd as rx
    R, V, D = (torch.from_numpy(x).cuda() for x in (r, v, d))
    LV = None if lv is None else torch.from_numpy(lv).cuda()
    A, Rt = torch.empty_like(R), torch.empty_like(R)
    rx.gae_scan(R, V, D, LV, 0.99, 0.95, A, Rt, noalloc=noalloc)
    torch.cuda.synchronize()
    return A.cpu().numpy(), Rt.cpu().numpy()


def _check(N, L, seed, last=False):
    r, v, d = synthdata.gae_inputs(N, L, seed)
    lv = (0.5 * np.random.default_rng(seed).standard_normal(N)).astype(np.float32) if last else None
    a0, r0 = _scan(r, v, d, lv, noalloc=True)
    a1, r1 = _scan(r, v, d, lv, noalloc=False)
    assert a0.tobytes() == a1.tobytes() and r0.tobytes() == r1.tobytes()
    Ao, Ro = oracle.gae(r, v, d, 0.99, 0.95, last_values=lv)
    assert close_mask(a0, Ao).all() and close_mask(r0, Ro).all()


def test_noalloc_matches_gae_scan_two_calls_second_smaller():
    _check(4096, 3000, 2)                # 6 chunks x 4096 episodes: 24,576 carries
    _check(1000, 1100, 3, last=True)     # smaller, another layout of the scratch


def test_noalloc_short_scan_needs_no_scratch():
    _check(600_000, 7, 4)                # one chunk: no carry, no limit on N


def test_noalloc_scan_that_fills_the_scratch():
    """8 chunks x 65,536 episodes: exactly the scratch's 524,288 carries.  The
    inputs repeat a block of 8191 episodes on the device (8191 is prime, so
    repeats land at other places in the 64-episode columns); the oracle
    recomputes a spread of episodes from the block."""
    import torch
    import rl_experience_collection_amd as rx
    N, L, B = 65_536, 4096, 8191
    blk = synthdata.gae_inputs(B, L, 5)
    R, V, D = (torch.from_numpy(x).cuda().repeat(1, -(-N // B))[:, :N].contiguous() for x in blk)
    out = []
    for noalloc in (True, False):
        A, Rt = torch.empty_like(R), torch.empty_like(R)
        rx.gae_scan(R, V, D, None, 0.99, 0.95, A, Rt, noalloc=noalloc)
        torch.cuda.synchronize()
        out.append((A, Rt))
    assert torch.equal(out[0][0], out[1][0]) and torch.equal(out[0][1], out[1][1])
    cols = np.unique(np.concatenate([np.arange(0, N, N // 29), [N - 1]]))
    Ao, Ro = oracle.gae(*(np.ascontiguousarray(x[:, cols % B]) for x in blk), 0.99, 0.95)
    idx = torch.from_numpy(cols).cuda()
    assert close_mask(out[0][0][:, idx].cpu().numpy(), Ao).all()
    assert close_mask(out[0][1][:, idx].cpu().numpy(), Ro).all()


def test_noalloc_refuses_a_scan_beyond_its_scratch():
    import torch
    import rl_experience_collection_amd as rx
    R = torch.zeros((4096, 65_537), device="cuda")
    D = torch.zeros((4096, 65_537), dtype=torch.uint8, device="cuda")
    with pytest.raises(rx.RolloutError, match="524288"):
        rx.gae_scan(R, R, D, None, 0.99, 0.95, R, R, noalloc=True)
