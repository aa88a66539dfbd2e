"""Pins for the oracle's counter-based generator (Philox4x32-10, SC'11).

The pages draw with an LCG; the method here keys one Philox4x32-10 block per
(seed, episode, step, stream) instead.  The oracle's implementation is pinned
to an independent one: the Philox4x32-10 of the installed rocRAND headers
(host-side inline functions), whose (seed, subsequence, offset) state maps to
key = seed and counter = (offset/4, subsequence) as 64-bit halves.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle

HELPERS = os.path.join(os.path.dirname(os.path.abspath(__file__)), "helpers")


@pytest.fixture(scope="module")
def philox_ref():
    exe = os.path.join(HELPERS, "philox_ref")
    if not os.path.exists(exe):
        import importlib.util
        spec = importlib.util.spec_from_file_location("helpers_build", os.path.join(HELPERS, "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        try:
            mod.build_philox_ref()
        except Exception as e:  # pragma: no cover - only without a ROCm toolchain
            pytest.skip(f"cannot build the rocRAND reference helper: {e}")

    def run(triples):
        txt = "".join(f"{s} {b} {o}\n" for s, b, o in triples)
        out = subprocess.run([exe], input=txt, capture_output=True, text=True, check=True).stdout
        return [[int(w, 16) for w in line.split()] for line in out.strip().splitlines()]

    return run


def test_philox_matches_rocrand(philox_ref):
    rng = np.random.default_rng(123)
    triples = [(0, 0, 0), (0, 0, 4), (2**64 - 1, 2**64 - 1, 4 * (2**62 - 1))]
    for _ in range(300):
        seed = int(rng.integers(0, 2**63)) * 2 + int(rng.integers(0, 2))
        sub = int(rng.integers(0, 2**63))
        off = 4 * int(rng.integers(0, 2**61))
        triples.append((seed, sub, off))
    ref = philox_ref(triples)
    for (seed, sub, off), r in zip(triples, ref):
        blk = off // 4
        ctr = [blk & 0xFFFFFFFF, blk >> 32, sub & 0xFFFFFFFF, sub >> 32]
        key = [seed & 0xFFFFFFFF, seed >> 32]
        assert list(oracle.philox(ctr, key)) == r, (seed, sub, off)


def test_uniform_is_24bit_grid_in_unit_interval():
    n = 200_000
    e = np.arange(n) % 977
    t = np.arange(n) // 977
    u = oracle.uniform(0xDEADBEEF12345, e, t)
    assert u.min() >= 0.0 and u.max() < 1.0
    k = u.astype(np.float64) * 2**24
    assert np.all(k == np.floor(k))


def test_uniform_equals_top_bits_of_block():
    seed = 0x0123456789ABCDEF
    for (e, t, s) in [(0, 0, 0), (5, 17, 0), (8191, 499, 0), (3, 4, 2)]:
        blk = oracle.philox([e, t, s, 0], [seed & 0xFFFFFFFF, seed >> 32])
        assert oracle.uniform(seed, [e], [t], s)[0] == np.float32((blk[0] >> 8) / 2**24)


def test_uniform_statistics():
    """Mean 1/2, variance 1/12 and no lag-1 correlation along episodes and steps."""
    E, T = 1000, 1000
    e, t = np.meshgrid(np.arange(E), np.arange(T), indexing="ij")
    u = oracle.uniform(42, e.ravel(), t.ravel()).astype(np.float64).reshape(E, T)
    n = u.size
    assert abs(u.mean() - 0.5) < 5 * np.sqrt(1 / 12 / n)
    assert abs(u.var() - 1 / 12) < 5 * np.sqrt(1 / 180 / n)
    c = u - 0.5
    for a, b in [(c[1:, :], c[:-1, :]), (c[:, 1:], c[:, :-1])]:
        r = (a * b).mean() / (1 / 12)
        assert abs(r) < 5 / np.sqrt(a.size)
    # streams are independent draws
    u1 = oracle.uniform(42, e.ravel()[:100000], t.ravel()[:100000], 1).astype(np.float64)
    r = ((u.ravel()[:100000] - 0.5) * (u1 - 0.5)).mean() * 12
    assert abs(r) < 5 / np.sqrt(100000)
