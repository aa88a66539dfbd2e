"""The C-ABI library loads and exports every symbol include/*.h declares;
host-side argument checks answer without touching a GPU."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("rollout.h", "dqn.h", "per.h")]


def declared_functions():
    names = []
    for header in HEADERS:
        txt = open(header).read()
        txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
        names += re.findall(r"^\s*(?:int|void|const char \*)\s*\*?\s*(\w+)\s*\(", txt,
                            flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def rx():
    import rl_experience_collection_amd as rx
    rx.load_library()
    return rx


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(
        ["rollout_config_default", "rollout_create", "rollout_set_weights", "rollout_collect",
         "rollout_phase_cycles",
         "gae_scan", "gae_scan_noalloc", "rollout_destroy", "rollout_last_error",
         "dqn_config_default", "dqn_create", "dqn_set_weights", "dqn_set_epsilon",
         "dqn_collect", "dqn_destroy", "per_create", "per_sample", "per_gather", "per_update", "per_destroy"])


def test_library_exports_every_declared_symbol(rx):
    lib = rx.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(rx.EXPORTED) == set(declared_functions())


def test_config_default_values(rx):
    cfg = rx.rollout_config_default(128, 500)
    assert (cfg.n_episodes, cfg.n_steps, cfg.n_features, cfg.state_dim, cfg.n_actions) == \
        (128, 500, 51, 54, 45)
    assert list(cfg.actor_dims) == [54, 128, 64, 45]
    assert list(cfg.critic_dims) == [54, 512, 384, 256, 128, 64, 1]
    assert list(cfg.cur_dims) == [99, 128, 51]
    assert cfg.max_hold == 50 and cfg.div_window == 20
    assert abs(cfg.gamma - 0.99) < 1e-7 and abs(cfg.lam - 0.95) < 1e-7


def test_config_struct_size_matches_header(rx):
    # 5 + 4 + 7 + 3 + 1 ints, 2 + 2 floats, 1 int, 1 int + 2 floats, 4 floats, 5 + 3 + 1 floats
    assert C.sizeof(rx.RolloutConfig) == 4 * (5 + 4 + 7 + 3 + 1 + 2 + 2 + 1 + 1 + 2 + 4 + 9 + 1 + 1)


def test_host_side_errors_without_gpu(rx):
    lib = rx.load_library()
    h = C.c_void_p()
    assert lib.rollout_create(None, None, None, None, None, None, 0, None, C.byref(h)) == rx.ROLLOUT_EINVAL
    assert "config" in rx.rollout_last_error()
    cfg = rx.rollout_config_default(16, 100)
    cfg.critic_dims[2] = 383
    arr = (C.c_void_p * 12)(*([1] * 12))
    assert lib.rollout_create(C.byref(cfg), arr, arr, arr, C.c_void_p(1), C.c_void_p(1), 20000,
                              None, C.byref(h)) == rx.ROLLOUT_EINVAL
    assert "critic dims" in rx.rollout_last_error()
    cfg = rx.rollout_config_default(0, 100)
    assert lib.rollout_create(C.byref(cfg), arr, arr, arr, C.c_void_p(1), C.c_void_p(1), 20000,
                              None, C.byref(h)) == rx.ROLLOUT_EINVAL
    cfg = rx.rollout_config_default(16, 100)
    cfg.div_window = 33
    assert lib.rollout_create(C.byref(cfg), arr, arr, arr, C.c_void_p(1), C.c_void_p(1), 20000,
                              None, C.byref(h)) == rx.ROLLOUT_EINVAL
    cfg = rx.rollout_config_default(16, 100)
    assert lib.rollout_create(C.byref(cfg), arr, arr, arr, C.c_void_p(1), C.c_void_p(1), 100,
                              None, C.byref(h)) == rx.ROLLOUT_EINVAL
    assert "n_bars" in rx.rollout_last_error()
    cfg = rx.rollout_config_default(16, 100)
    assert cfg.overlap == -1
    cfg.overlap = 2
    assert lib.rollout_create(C.byref(cfg), arr, arr, arr, C.c_void_p(1), C.c_void_p(1), 20000,
                              None, C.byref(h)) == rx.ROLLOUT_EINVAL
    assert "overlap" in rx.rollout_last_error()
    assert lib.rollout_collect(None, None, 0, None, None) == rx.ROLLOUT_EINVAL
    assert lib.gae_scan(None, None, None, None, 0, 5, 0.99, 0.95, None, None, None) == rx.ROLLOUT_OK
    assert lib.gae_scan(None, None, None, None, 3, 5, 0.99, 0.95, None, None, None) == rx.ROLLOUT_EINVAL
    assert lib.gae_scan(None, None, None, None, -1, 5, 0.99, 0.95, None, None, None) == rx.ROLLOUT_EINVAL
    lib.rollout_destroy(None)


def test_gae_scan_noalloc_rejects_scans_beyond_its_scratch(rx):
    """The allocation-free scan holds 524,288 chunk carries: a scan longer
    than 512 steps needing more is refused on the host, before any device
    call; short scans need none."""
    lib = rx.load_library()
    d = C.c_void_p(1)
    assert lib.gae_scan_noalloc(d, d, d, None, 2304, 104858, 0.99, 0.95, d, d, None) == \
        rx.ROLLOUT_EINVAL
    msg = rx.rollout_last_error()
    assert "524288" in msg and "5 chunks" in msg and "104858" in msg
    assert lib.gae_scan_noalloc(None, None, None, None, 0, 5, 0.99, 0.95, None, None, None) == \
        rx.ROLLOUT_OK
    assert lib.gae_scan_noalloc(None, None, None, None, 3, 5, 0.99, 0.95, None, None, None) == \
        rx.ROLLOUT_EINVAL
    assert lib.gae_scan_noalloc(None, None, None, None, 3, -5, 0.99, 0.95, None, None, None) == \
        rx.ROLLOUT_EINVAL


def test_rollout_phase_cycles_rejects_a_null_handle(rx):
    lib = rx.load_library()
    n = C.c_int64(7)
    assert lib.rollout_phase_cycles(None, 1, None, 0, C.byref(n)) == rx.ROLLOUT_EINVAL
    assert "handle" in rx.rollout_last_error()


def test_dqn_config_default_values(rx):
    cfg = rx.dqn_config_default(16384, 500)
    assert (cfg.n_episodes, cfg.n_steps, cfg.n_features, cfg.state_dim, cfg.n_actions) == \
        (16384, 500, 51, 54, 45)
    assert list(cfg.trunk_dims) == [54, 256, 128]
    assert list(cfg.value_dims) == [128, 64, 1]
    assert list(cfg.advantage_dims) == [128, 64, 45]
    assert list(cfg.cur_dims) == [99, 128, 51]
    assert abs(cfg.epsilon - 0.1) < 1e-7 and abs(cfg.gamma - 0.99) < 1e-7
    assert abs(cfg.priority_alpha - 0.6) < 1e-7
    assert cfg.max_hold == 50 and cfg.div_window == 20


def test_dqn_config_struct_size_matches_header(rx):
    # 5 ints, 4 x 3 dims, 3 floats, 2 floats, 2 ints, 2 + 4 floats, 5 + 3 + 1 floats, 1 int
    assert C.sizeof(rx.DqnConfig) == 4 * (5 + 12 + 3 + 2 + 2 + 6 + 9 + 1)
    assert C.sizeof(rx.DqnOutputs) == 8 * 14


def test_dqn_host_side_errors_without_gpu(rx):
    lib = rx.load_library()
    h = C.c_void_p()
    assert lib.dqn_create(None, None, None, None, None, None, 0, None, C.byref(h)) == rx.ROLLOUT_EINVAL
    assert "config" in rx.rollout_last_error()
    cfg = rx.dqn_config_default(16, 10)
    cfg.epsilon = 1.5
    assert lib.dqn_create(C.byref(cfg), None, None, None, None, None, 0, None, C.byref(h)) == \
        rx.ROLLOUT_EINVAL
    assert "epsilon" in rx.rollout_last_error()
    cfg = rx.dqn_config_default(16, 10)
    cfg.trunk_dims[1] = 512
    assert lib.dqn_create(C.byref(cfg), None, None, None, None, None, 0, None, C.byref(h)) == \
        rx.ROLLOUT_EINVAL
    assert "trunk" in rx.rollout_last_error()
    assert lib.dqn_collect(None, None, 0, None, None) == rx.ROLLOUT_EINVAL
    lib.dqn_destroy(None)


def test_dqn_set_epsilon_rejects_values_outside_unit_interval(rx):
    """Epsilon Decay ("GPU Pipeline Phase 2b", Concerns and Mitigations): a
    per-launch probability; the value is checked before the handle."""
    lib = rx.load_library()
    for bad in (-0.01, 1.0001, float("nan"), float("inf"), -float("inf")):
        assert lib.dqn_set_epsilon(None, bad) == rx.ROLLOUT_EINVAL
        assert "epsilon" in rx.rollout_last_error()
    for ok in (0.0, 0.05, 1.0):
        assert lib.dqn_set_epsilon(None, ok) == rx.ROLLOUT_EINVAL
        assert "handle" in rx.rollout_last_error()


def test_per_host_side_errors_without_gpu(rx):
    lib = rx.load_library()
    h = C.c_void_p()
    assert lib.per_create(0, 16, C.byref(h)) == rx.ROLLOUT_EINVAL
    assert "capacity" in rx.rollout_last_error()
    assert lib.per_create(100, 0, C.byref(h)) == rx.ROLLOUT_EINVAL
    assert lib.per_sample(None, None, 10, 1, 0, 0.4, None, None, None) == rx.ROLLOUT_EINVAL
    assert lib.per_update(None, 10, None, None, 1, 0.6, 0.01, 1.0, None) == rx.ROLLOUT_EINVAL
    assert lib.per_update(None, 10, None, None, 0, 0.6, 0.01, 1.0, None) == rx.ROLLOUT_OK
    assert lib.per_gather(None, 2, 10, None, None, None, None, None, None, None, None, None, None,
                          None) == rx.ROLLOUT_EINVAL
    lib.per_destroy(None)
