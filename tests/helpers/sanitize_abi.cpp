// Drives the host-side argument checks of every C-ABI entry point of
// librollout.so (include/rollout.h, dqn.h, per.h) for an AddressSanitizer +
// UndefinedBehaviorSanitizer build of the library's host code: each call is
// given arguments the library must reject before touching a device, and the
// error text is read back.  No GPU is needed or used: on a machine without
// one, the calls that pass the checks fail at their first HIP call with
// ROLLOUT_EHIP, which exercises that error path too.  Exit status 0 means
// every call returned the expected code with no sanitizer report.
// Built and run by tests/test_sanitizers.py.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/dqn.h"
#include "../../include/per.h"
#include "../../include/rollout.h"

static int fails = 0;
static void expect(int got, int want, const char* what, const char* text = nullptr) {
  const std::string err = rollout_last_error();
  if (got != want || (text && err.find(text) == std::string::npos)) {
    std::fprintf(stderr, "%s: got %d (want %d), error \"%s\"\n", what, got, want, err.c_str());
    ++fails;
  }
}

int main() {
  float dummy[64] = {0};
  const float* w12[12];
  for (auto& p : w12) p = dummy;
  rollout_handle h = nullptr;

  expect(rollout_config_default(nullptr, 1, 1), ROLLOUT_EINVAL, "config_default(NULL)", "NULL");
  rollout_config cfg;
  expect(rollout_config_default(&cfg, 16, 100), ROLLOUT_OK, "config_default");
  expect(rollout_create(nullptr, w12, w12, w12, dummy, dummy, 1000, nullptr, &h), ROLLOUT_EINVAL,
         "create(NULL config)", "config");
  expect(rollout_create(&cfg, w12, w12, w12, dummy, dummy, 1000, nullptr, nullptr),
         ROLLOUT_EINVAL, "create(NULL out)", "out");
  rollout_config c2 = cfg;
  c2.critic_dims[3] = 255;
  expect(rollout_create(&c2, w12, w12, w12, dummy, dummy, 1000, nullptr, &h), ROLLOUT_EINVAL,
         "create(critic dims)", "critic dims");
  c2 = cfg;
  c2.n_episodes = 0;
  expect(rollout_create(&c2, w12, w12, w12, dummy, dummy, 1000, nullptr, &h), ROLLOUT_EINVAL,
         "create(N = 0)", "n_episodes");
  c2 = cfg;
  c2.div_window = 0;
  expect(rollout_create(&c2, w12, w12, w12, dummy, dummy, 1000, nullptr, &h), ROLLOUT_EINVAL,
         "create(div_window)", "div_window");
  c2 = cfg;
  c2.precision = 7;
  expect(rollout_create(&c2, w12, w12, w12, dummy, dummy, 1000, nullptr, &h), ROLLOUT_EINVAL,
         "create(precision)", "precision");
  c2 = cfg;
  c2.recycle = 2;
  expect(rollout_create(&c2, w12, w12, w12, dummy, dummy, 1000, nullptr, &h), ROLLOUT_EINVAL,
         "create(recycle)", "recycle");
  const float* w_null[12];
  std::memcpy(w_null, w12, sizeof(w12));
  w_null[5] = nullptr;
  expect(rollout_create(&cfg, w12, w_null, w12, dummy, dummy, 1000, nullptr, &h), ROLLOUT_EINVAL,
         "create(NULL critic tensor)", "critic tensor 5");
  expect(rollout_create(&cfg, w12, w12, w12, nullptr, dummy, 1000, nullptr, &h), ROLLOUT_EINVAL,
         "create(NULL features)", "features");
  expect(rollout_create(&cfg, w12, w12, w12, dummy, dummy, 100, nullptr, &h), ROLLOUT_EINVAL,
         "create(n_bars = L)", "n_bars");
  expect(rollout_create(&cfg, w12, w12, w12, dummy, dummy, (int64_t)1 << 40, nullptr, &h),
         ROLLOUT_EINVAL, "create(n_bars huge)", "n_bars");
  // valid arguments: on a machine without a GPU the first HIP call fails
  const int rc = rollout_create(&cfg, w12, w12, w12, dummy, dummy, 1000, nullptr, &h);
  if (rc == ROLLOUT_OK) rollout_destroy(h);
  else expect(rc, ROLLOUT_EHIP, "create(valid, no device)");
  expect(rollout_set_weights(nullptr, w12, w12, w12, nullptr), ROLLOUT_EINVAL, "set_weights(NULL)",
         "handle");
  expect(rollout_collect(nullptr, nullptr, 0, nullptr, nullptr), ROLLOUT_EINVAL, "collect(NULL)",
         "handle");
  expect(rollout_phase_cycles(nullptr, 1, nullptr, 0, nullptr), ROLLOUT_EINVAL,
         "phase_cycles(NULL)", "handle");
  expect(gae_scan(nullptr, nullptr, nullptr, nullptr, 0, 5, 0.99f, 0.95f, nullptr, nullptr,
                  nullptr),
         ROLLOUT_OK, "gae_scan(L = 0)");
  expect(gae_scan(nullptr, nullptr, nullptr, nullptr, 3, 5, 0.99f, 0.95f, nullptr, nullptr,
                  nullptr),
         ROLLOUT_EINVAL, "gae_scan(NULL)", "NULL");
  expect(gae_scan(nullptr, nullptr, nullptr, nullptr, -1, 5, 0.99f, 0.95f, nullptr, nullptr,
                  nullptr),
         ROLLOUT_EINVAL, "gae_scan(L < 0)", "negative");
  expect(gae_scan(dummy, dummy, reinterpret_cast<const uint8_t*>(dummy), nullptr, 1 << 21,
                  1 << 20, 0.99f, 0.95f, dummy, dummy, nullptr),
         ROLLOUT_EINVAL, "gae_scan(too large)", "too large");
  expect(gae_scan_noalloc(nullptr, nullptr, nullptr, nullptr, 0, 5, 0.99f, 0.95f, nullptr,
                          nullptr, nullptr),
         ROLLOUT_OK, "gae_scan_noalloc(L = 0)");
  expect(gae_scan_noalloc(nullptr, nullptr, nullptr, nullptr, 3, 5, 0.99f, 0.95f, nullptr,
                          nullptr, nullptr),
         ROLLOUT_EINVAL, "gae_scan_noalloc(NULL)", "NULL");
  expect(gae_scan_noalloc(nullptr, nullptr, nullptr, nullptr, 3, -5, 0.99f, 0.95f, nullptr,
                          nullptr, nullptr),
         ROLLOUT_EINVAL, "gae_scan_noalloc(N < 0)", "negative");
  // 5 chunks of 512 steps x 104858 episodes: more carries than the fixed scratch holds
  expect(gae_scan_noalloc(dummy, dummy, reinterpret_cast<const uint8_t*>(dummy), nullptr, 2304,
                          104858, 0.99f, 0.95f, dummy, dummy, nullptr),
         ROLLOUT_EINVAL, "gae_scan_noalloc(beyond scratch)", "524288");
  rollout_destroy(nullptr);

  dqn_config dc;
  dqn_handle dh = nullptr;
  expect(dqn_config_default(&dc, 16, 10), ROLLOUT_OK, "dqn_config_default");
  dqn_config d2 = dc;
  d2.epsilon = NAN;
  expect(dqn_create(&d2, w12, w12, w12, dummy, dummy, 100, nullptr, &dh), ROLLOUT_EINVAL,
         "dqn_create(epsilon NaN)", "epsilon");
  d2 = dc;
  d2.advantage_dims[2] = 44;
  expect(dqn_create(&d2, w12, w12, w12, dummy, dummy, 100, nullptr, &dh), ROLLOUT_EINVAL,
         "dqn_create(advantage dims)", "advantage");
  expect(dqn_create(&dc, w12, nullptr, w12, dummy, dummy, 100, nullptr, &dh), ROLLOUT_EINVAL,
         "dqn_create(NULL target)", "NULL");
  expect(dqn_set_epsilon(nullptr, 1.5f), ROLLOUT_EINVAL, "dqn_set_epsilon(1.5)", "epsilon");
  expect(dqn_set_epsilon(nullptr, 0.5f), ROLLOUT_EINVAL, "dqn_set_epsilon(NULL)", "handle");
  expect(dqn_set_weights(nullptr, w12, nullptr, nullptr, nullptr), ROLLOUT_EINVAL,
         "dqn_set_weights(NULL)", "handle");
  expect(dqn_collect(nullptr, nullptr, 0, nullptr, nullptr), ROLLOUT_EINVAL, "dqn_collect(NULL)",
         "handle");
  dqn_destroy(nullptr);

  per_handle ph = nullptr;
  expect(per_create(0, 16, &ph), ROLLOUT_EINVAL, "per_create(capacity 0)", "capacity");
  expect(per_create(100, 0, &ph), ROLLOUT_EINVAL, "per_create(batch 0)", "max_batch");
  expect(per_create(100, 16, nullptr), ROLLOUT_EINVAL, "per_create(NULL out)", "out");
  expect(per_sample(nullptr, dummy, 10, 1, 0, 0.4f, nullptr, nullptr, nullptr), ROLLOUT_EINVAL,
         "per_sample(NULL)", "handle");
  expect(per_update(dummy, 10, nullptr, nullptr, 1, 0.6f, 0.01f, 1.0f, nullptr), ROLLOUT_EINVAL,
         "per_update(NULL)", "NULL");
  expect(per_update(dummy, 10, nullptr, nullptr, 1, 0.6f, 2.0f, 1.0f, nullptr), ROLLOUT_EINVAL,
         "per_update(NULL first)", "NULL");
  expect(per_update(nullptr, 10, nullptr, nullptr, -1, 0.6f, 0.01f, 1.0f, nullptr),
         ROLLOUT_EINVAL, "per_update(batch < 0)", "batch");
  expect(per_gather(nullptr, 2, 10, dummy, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                    nullptr, nullptr, nullptr, nullptr),
         ROLLOUT_EINVAL, "per_gather(NULL indices)", "NULL");
  const int32_t idx[2] = {0, 1};
  expect(per_gather(idx, 2, 10, dummy, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                    nullptr, nullptr, nullptr, nullptr),
         ROLLOUT_EINVAL, "per_gather(source without output)", "output");
  per_destroy(nullptr);

  if (fails) {
    std::fprintf(stderr, "%d calls returned the wrong code\n", fails);
    return 1;
  }
  std::printf("ABI sanitizer run: clean\n");
  return 0;
}
