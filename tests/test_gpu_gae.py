"""GPU parity of the standalone GAE scan (PPO CUDA Pipeline Design, Kernel
Phases, Phase B) against the oracle, through the C ABI."""
import numpy as np
import pytest

import oracle
import synthdata
from parity import close_mask, gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X")]


def run(r, v, d, gamma=0.99, lam=0.95, last=None, offset=0):
    import torch
    import rl_experience_collection_amd as rx
    L, N = r.shape

    def dev(a):
        if offset == 0:
            return torch.from_numpy(np.ascontiguousarray(a)).cuda()
        # misaligned view: `offset` elements into a larger buffer
        flat = torch.zeros(a.size + offset, dtype=torch.from_numpy(a[:0]).dtype, device="cuda")
        flat[offset:] = torch.from_numpy(np.ascontiguousarray(a).ravel()).cuda()
        return flat[offset:].view(a.shape)

    R, V, D = dev(r), dev(v), dev(d)
    A = torch.empty_like(R)
    Rt = torch.empty_like(R)
    lv = None if last is None else dev(last)
    rx.gae_scan(R, V, D, lv, gamma, lam, A, Rt)
    torch.cuda.synchronize()
    return A.cpu().numpy(), Rt.cpu().numpy()


def check(r, v, d, gamma=0.99, lam=0.95, last=None, offset=0):
    A, R = run(r, v, d, gamma, lam, last, offset)
    Ao, Ro = oracle.gae(r, v, d, gamma, lam, last_values=last)
    assert close_mask(A, Ao).all(), np.abs(A - Ao).max()
    assert close_mask(R, Ro).all(), np.abs(R - Ro).max()
    assert np.array_equal(R, (A + v).astype(np.float32))
    return A, R


@pytest.mark.parametrize("L,N", [(1, 1), (2, 3), (17, 5), (16, 1024), (100, 16), (37, 1000),
                                 (33, 2049), (500, 8192), (129, 4100), (512, 96), (513, 31),
                                 (700, 33), (1025, 100), (1537, 40), (2048, 17),
                                 (2049, 20), (2600, 70)])
def test_gae_matches_oracle(L, N):
    r, v, d = synthdata.gae_inputs(N, L, seed=L * 7 + N)
    check(r, v, d)


def test_gae_full_size_4096x2048():
    spec = synthdata.WORKLOADS["gae_n4096_l2048"]
    r, v, d = synthdata.gae_inputs(spec["N"], spec["L"], spec["seed"])
    check(r, v, d)


@pytest.mark.parametrize("N", [6, 7, 1030])
def test_gae_last_values_and_vector_widths(N):
    L = 45
    r, v, d = synthdata.gae_inputs(N, L, seed=N)
    last = np.linspace(-1, 1, N).astype(np.float32)
    check(r, v, d, last=last)


@pytest.mark.parametrize("offset", [1, 2])
def test_gae_misaligned_views(offset):
    r, v, d = synthdata.gae_inputs(256, 40, seed=offset)
    check(r, v, d, offset=offset)


def test_gae_dense_dones_and_extreme_params():
    r, v, d = synthdata.gae_inputs(300, 64, seed=9, p_done=0.5)
    check(r, v, d, gamma=1.0, lam=1.0)
    check(r, v, d, gamma=0.5, lam=0.0)
    d1 = np.ones_like(d)
    A, _ = check(r, v, d1)
    assert np.array_equal(A, r - v)


@pytest.mark.parametrize("L,N", [(512, 4096), (2048, 1024), (2600, 1024)])
def test_gae_deterministic_across_calls(L, N):
    r, v, d = synthdata.gae_inputs(N, L, seed=3)
    A1, R1 = run(r, v, d)
    A2, R2 = run(r, v, d)
    assert np.array_equal(A1, A2) and np.array_equal(R1, R2)


@pytest.mark.parametrize("p_done", [0.0, 0.0005])
def test_gae_long_chains(p_done):
    """Rollouts of many super-chunks: carries cross more super-chunks than a
    reader folds before it waits on an inclusive value."""
    r, v, d = synthdata.gae_inputs(64, 5000, seed=11, p_done=p_done)
    check(r, v, d)


def test_gae_empty_is_noop():
    import torch
    import rl_experience_collection_amd as rx
    z = torch.zeros((0, 5), device="cuda")
    rx.gae_scan(z, z, torch.zeros((0, 5), dtype=torch.uint8, device="cuda"), None, 0.99, 0.95, z, z)


@pytest.mark.parametrize("L,N", [(500, 65536), (2048, 16384), (16384, 2048)])
def test_gae_large_sizes_sampled_episodes(L, N):
    """Large launches (33.5 M elements, 570 MB moved): 2048 columns of the
    single-super-chunk path, 256 columns of 4 chained super-chunks, and 32
    chained super-chunks per column; the oracle recomputes a spread of
    episodes (episodes are independent), and every return is A + V."""
    r, v, d = synthdata.gae_inputs(N, L, seed=N + L)
    A, R = run(r, v, d)
    cols = np.unique(np.concatenate([np.arange(0, N, N // 37), [N - 1, N // 2 + 1]]))
    Ao, Ro = oracle.gae(np.ascontiguousarray(r[:, cols]), np.ascontiguousarray(v[:, cols]),
                        np.ascontiguousarray(d[:, cols]), 0.99, 0.95)
    assert close_mask(A[:, cols], Ao).all(), np.abs(A[:, cols] - Ao).max()
    assert close_mask(R[:, cols], Ro).all()
    assert np.array_equal(R, (A + v).astype(np.float32))
    assert np.isfinite(A).all()


@pytest.mark.parametrize("L,N", [(513, 524288), (513, 2097157), (300, 2097157)])
def test_gae_many_episodes_both_address_widths(L, N):
    """Scans of very many episodes: 524,288 episodes address a 512-step
    super-chunk with 32-bit offsets, 2,097,157 (over 2^21, so a super-chunk
    spans more than 4 GiB of floats) with 64-bit addresses, chained (513
    steps) or in one super-chunk (300 steps).  The inputs
    repeat a block of 8191 episodes on the device (8191 is prime, so every
    repeat lands at another place in the 64-episode columns), which keeps
    the host's work small; the oracle recomputes a spread of episodes from
    the block, and every return is A + V."""
    import torch
    import rl_experience_collection_amd as rx
    B = 8191
    blk = synthdata.gae_inputs(B, L, seed=N + L)
    reps = -(-N // B)
    R, V, D = (torch.from_numpy(x).cuda().repeat(1, reps)[:, :N].contiguous() for x in blk)
    A, Rt = torch.empty_like(R), torch.empty_like(R)
    rx.gae_scan(R, V, D, None, 0.99, 0.95, A, Rt)
    torch.cuda.synchronize()
    assert torch.equal(Rt, A + V)
    assert bool(torch.isfinite(A).all())
    cols = np.unique(np.concatenate([np.arange(0, N, N // 41), [N - 1, N // 2 + 1, 2 ** 21]]))
    cols = cols[cols < N]
    Ao, Ro = oracle.gae(*(np.ascontiguousarray(x[:, cols % B]) for x in blk), 0.99, 0.95)
    Ag = A[:, torch.from_numpy(cols).cuda()].cpu().numpy()
    Rg = Rt[:, torch.from_numpy(cols).cuda()].cpu().numpy()
    assert close_mask(Ag, Ao).all(), np.abs(Ag - Ao).max()
    assert close_mask(Rg, Ro).all()
