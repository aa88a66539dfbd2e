// C ABI of librollout.so (declared in include/rollout.h): argument checks,
// device memory of collectors, weight packing and the launch sequence
//   actor rollout -> batched critic/curiosity/reward -> GAE scan
// on the caller's stream.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "../../include/dqn.h"
#include "../../include/per.h"
#include "../../include/rollout.h"
#include "collect.hpp"
#include "per.hpp"
#include "gae.hpp"
#include "pack.hpp"

// The fixed scratch of gae_scan_noalloc (see NoAllocDevice below): 4 MiB +
// 256 bytes per device.
static __device__ __align__(256) unsigned char scratch[256 + ((size_t)1 << 19) * 8];

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(ROLLOUT_EHIP, "%s: %s", what, hipGetErrorString(e));
}

#define RL_HIP(call, what)                        \
  do {                                            \
    hipError_t _e = (call);                       \
    if (_e != hipSuccess) return hip_fail(_e, what); \
  } while (0)

// Carry scratch of the GAE scan (flags at a fixed offset, epoch-tagged).
struct GaeScratch {
  char* mem = nullptr;
  size_t bytes = 0;
  bool fixed = false;  // memory not owned by the scratch: never reallocated
  int32_t nk = 0, nc = 0, n = 0;
  uint32_t ticket_base = 0;
  uint32_t epoch = 0;
};

int gae_prepare(GaeScratch& s, const rl::GaeShape& shape, int32_t N, hipStream_t st,
                rl::GaeScratchView* view) {
  const size_t need = rl::gae_scratch_bytes(shape.nk, N);
  bool relayout = (shape.nk != s.nk || N != s.n);
  if (s.bytes < need && s.fixed)
    return fail(ROLLOUT_EINVAL, "gae scratch: %zu bytes needed, %zu available", need, s.bytes);
  if (s.bytes < need) {
    if (s.mem) {
      hipError_t e = hipFree(s.mem);
      s.mem = nullptr;
      s.bytes = 0;
      if (e != hipSuccess) return hip_fail(e, "hipFree(gae scratch)");
    }
    void* p = nullptr;
    if (hipMalloc(&p, need) != hipSuccess) {
      (void)hipGetLastError();
      return fail(ROLLOUT_ENOMEM, "gae scratch: cannot allocate %zu bytes", need);
    }
    s.mem = static_cast<char*>(p);
    s.bytes = need;
    RL_HIP(rl::zero_words(reinterpret_cast<uint32_t*>(s.mem), 64, st), "clear gae ticket");
    s.ticket_base = 0;
    relayout = true;
  }
  // The words are epoch-tagged; they are cleared only when their layout
  // changes (or the epoch wraps), so that stale words never carry the
  // current epoch.
  if (relayout || s.epoch >= (1u << 28)) {
    RL_HIP(rl::zero_words(reinterpret_cast<uint32_t*>(s.mem + 256),
                          rl::gae_words_bytes(shape.nk, N) / 4, st),
           "clear gae words");
    s.epoch = 0;
    s.nk = shape.nk;
    s.nc = shape.nc;
    s.n = N;
  }
  s.epoch += 1;
  view->ticket = reinterpret_cast<uint32_t*>(s.mem);
  view->words = reinterpret_cast<uint64_t*>(s.mem + 256);
  view->ticket_base = s.ticket_base;
  view->epoch = s.epoch;
  return ROLLOUT_OK;
}

// Polls of a GAE look-back before it gives up: the built-in limit, unless
// the environment variable ROLLOUT_GAE_SPIN_LIMIT sets another (a test of the
// give-up path lowers it; it never needs raising).
uint32_t gae_spin_limit() {
  const char* v = std::getenv("ROLLOUT_GAE_SPIN_LIMIT");
  if (!v || !*v) return rl::kGaeSpinLimit;
  char* end = nullptr;
  const unsigned long x = std::strtoul(v, &end, 10);
  if (end == v || *end) return rl::kGaeSpinLimit;
  return x > rl::kGaeSpinLimit ? rl::kGaeSpinLimit : (uint32_t)x;
}

// Whether a collector may keep the actor's first-layer feature table: yes,
// unless the environment variable ROLLOUT_FEATURE_TABLE, read at
// rollout_create, is "0" (the step then always computes that part itself).
bool feature_table_enabled() {
  const char* v = std::getenv("ROLLOUT_FEATURE_TABLE");
  return !(v && v[0] == '0' && v[1] == 0);
}

int gae_run(GaeScratch& s, rl::GaeArgs a, hipStream_t st) {
  if (a.L == 0 || a.N == 0) return ROLLOUT_OK;
  a.spin_limit = gae_spin_limit();
  const rl::GaeShape shape = rl::gae_shape(a.L, a.N);
  if (shape.tiles() >= (int64_t)1 << 31) return fail(ROLLOUT_EINVAL, "gae_scan: too many tiles");
  // a single chunk per episode passes no carry: no scratch
  rl::GaeScratchView view{};
  if (shape.nk > 1) {
    const int rc = gae_prepare(s, shape, a.N, st, &view);
    if (rc) return rc;
  }
  hipError_t e = rl::gae_launch(a, shape, view, st);
  if (e != hipSuccess) return hip_fail(e, "gae_scan launch");
  if (shape.nk > 1) s.ticket_base += (uint32_t)shape.tiles();  // tickets are taken only then
  return ROLLOUT_OK;
}

// Reserve the scratch for the largest tile grid an (L, N) scan can use.
int gae_reserve(GaeScratch& s, int32_t L, int32_t N, hipStream_t st) {
  const rl::GaeShape shape = rl::gae_shape(L, N);
  if (shape.nk == 1) return ROLLOUT_OK;  // no carries to keep
  rl::GaeScratchView view;
  const int rc = gae_prepare(s, shape, N, st, &view);
  s.epoch -= 1;  // nothing was launched with this epoch
  return rc;
}

// Scratch of gae_scan_noalloc, for callers that cannot allocate: the
// inter-chunk carries of one scan (a 256-byte header holding the ticket
// counter, then 8 bytes per episode and 512-step chunk), at most
// kNoAllocCarries of them.  Each device holds its own copy until the process
// ends; host code reaches it only through the address hipGetSymbolAddress
// returns for the current device.
constexpr size_t kNoAllocCarries = (size_t)1 << 19;
constexpr size_t kNoAllocBytes = 256 + kNoAllocCarries * 8;
constexpr int kMaxDevices = 64;

struct NoAllocDevice {
  bool ready = false;
  GaeScratch s;  // s.mem: this device's address of `scratch`
};
std::mutex g_noalloc_mu;
NoAllocDevice g_noalloc[kMaxDevices];

std::mutex g_gae_mu;
std::map<std::pair<int, hipStream_t>, GaeScratch>& gae_cache() {
  static auto* m = new std::map<std::pair<int, hipStream_t>, GaeScratch>();
  return *m;
}

const int32_t kActorDims[4] = {54, 128, 64, 45};
const int32_t kCriticDims[7] = {54, 512, 384, 256, 128, 64, 1};
const int32_t kCurDims[3] = {99, 128, 51};

template <class Config>
rl::EnvParams env_params(const Config& c) {
  rl::EnvParams p;
  p.ex0 = c.exposure[0]; p.ex1 = c.exposure[1]; p.ex2 = c.exposure[2];
  p.ex3 = c.exposure[3]; p.ex4 = c.exposure[4];
  p.cost0 = c.cost[0]; p.cost1 = c.cost[1]; p.cost2 = c.cost[2];
  p.urgency_mult = c.urgency_mult;
  // fp32 threshold multipliers; the barrier compares P[bar+1] with entry * these
  p.up_pt = 1.0f + c.profit_take;
  p.dn_sl = 1.0f - c.stop_loss;
  p.dn_pt = 1.0f - c.profit_take;
  p.up_sl = 1.0f + c.stop_loss;
  p.max_hold = c.max_hold;
  p.div_window = c.div_window;
  p.div_threshold = c.div_threshold;
  p.div_penalty = c.div_penalty;
  p.barrier_scale = c.barrier_scale;
  p.spread = c.spread;
  p.risk_coef = c.risk_coef;
  p.curiosity_coef = c.curiosity_coef;
  return p;
}

int check_config(const rollout_config* c) {
  if (!c) return fail(ROLLOUT_EINVAL, "config is NULL");
  if (c->n_episodes < 1 || c->n_steps < 1)
    return fail(ROLLOUT_EINVAL, "n_episodes and n_steps must be >= 1 (got %d, %d)", c->n_episodes,
                c->n_steps);
  if ((int64_t)c->n_episodes * c->n_steps >= (int64_t)1 << 40)
    return fail(ROLLOUT_EINVAL, "n_episodes * n_steps too large");
  if (c->n_features != 51 || c->state_dim != 54 || c->n_actions != 45)
    return fail(ROLLOUT_EINVAL, "features/state/actions must be 51/54/45");
  for (int i = 0; i < 4; ++i)
    if (c->actor_dims[i] != kActorDims[i]) return fail(ROLLOUT_EINVAL, "actor dims must be 54,128,64,45");
  for (int i = 0; i < 7; ++i)
    if (c->critic_dims[i] != kCriticDims[i])
      return fail(ROLLOUT_EINVAL, "critic dims must be 54,512,384,256,128,64,1");
  for (int i = 0; i < 3; ++i)
    if (c->cur_dims[i] != kCurDims[i]) return fail(ROLLOUT_EINVAL, "curiosity dims must be 99,128,51");
  if (c->precision != ROLLOUT_FP32 && c->precision != ROLLOUT_BF16)
    return fail(ROLLOUT_EINVAL, "unknown precision %d", c->precision);
  if (c->div_window < 1 || c->div_window > 32)
    return fail(ROLLOUT_EINVAL, "div_window must be in 1..32 (got %d)", c->div_window);
  if (c->max_hold < 1) return fail(ROLLOUT_EINVAL, "max_hold must be >= 1");
  if (c->recycle != 0 && c->recycle != 1) return fail(ROLLOUT_EINVAL, "recycle must be 0 or 1");
  if (c->overlap < -1 || c->overlap > 1) return fail(ROLLOUT_EINVAL, "overlap must be -1, 0 or 1");
  return ROLLOUT_OK;
}

// Launches the rollout of one collection is split into, so that the value
// pass over each finished part runs on another stream while the rollout
// continues.  By default only where it pays: fp32 (the bf16 value pass is
// too short to repay the extra launches) with the rollout's workgroups (16
// episodes each) leaving at least three quarters of the CUs idle; `overlap`
// 1 forces it, 0 turns it off.
// How many: the last part is kept to at most one value work item per CU (its
// pass runs after the rollout, see rollout_create); each earlier part's pass,
// on the CUs the rollout leaves free, should end within the part after it,
// so a part holds at most the rows those CUs finish in the rounds of work
// items that fit in the last part's duration.  A work item takes about as
// long as kItemSteps rollout steps (measured at N=128: ~55 us against
// ~2.7 us).  Fewer parts mean fewer launch and event gaps (~7 us each):
// N=128 L=500 fp32 runs as 4 parts, 1.43 -> 1.41 ms against 7.
constexpr int64_t kItemSteps = 20;
int overlap_parts(const rollout_config& c, int cus) {
  if (c.overlap == 0 || c.n_steps < 2) return 1;
  const bool bf16 = c.precision != ROLLOUT_FP32;
  const int64_t blocks = ((int64_t)c.n_episodes + 15) / 16;
  if (c.overlap < 0 && (bf16 || blocks * 4 > (int64_t)cus)) return 1;
  const int64_t item_rows = bf16 ? 128 : 32;
  const int64_t fit = (int64_t)cus * item_rows / c.n_episodes;
  const int64_t half = (c.n_steps + 1) / 2;
  const int64_t last = fit < 1 ? 1 : (fit < half ? fit : half);
  const int64_t free_cus = (int64_t)cus - blocks > 0 ? (int64_t)cus - blocks : 1;
  const int64_t rounds = last / kItemSteps > 1 ? last / kItemSteps : 1;
  int64_t per_part = rounds * free_cus * item_rows / c.n_episodes;
  per_part = per_part < 1 ? 1 : per_part;
  const int64_t k = 1 + (c.n_steps - last + per_part - 1) / per_part;
  return (int)(k < 2 ? 2 : (k > 8 ? 8 : k));
}

int check_weights(const float* const actor[6], const float* const critic[12],
                  const float* const cur[4]) {
  if (!actor || !critic || !cur) return fail(ROLLOUT_EINVAL, "weight array is NULL");
  for (int i = 0; i < 6; ++i)
    if (!actor[i]) return fail(ROLLOUT_EINVAL, "actor tensor %d is NULL", i);
  for (int i = 0; i < 12; ++i)
    if (!critic[i]) return fail(ROLLOUT_EINVAL, "critic tensor %d is NULL", i);
  for (int i = 0; i < 4; ++i)
    if (!cur[i]) return fail(ROLLOUT_EINVAL, "curiosity tensor %d is NULL", i);
  return ROLLOUT_OK;
}

const int32_t kTrunkDims[3] = {54, 256, 128};
const int32_t kValueDims[3] = {128, 64, 1};
const int32_t kAdvDims[3] = {128, 64, 45};

int check_dqn_config(const dqn_config* c) {
  if (!c) return fail(ROLLOUT_EINVAL, "config is NULL");
  if (c->n_episodes < 1 || c->n_steps < 1)
    return fail(ROLLOUT_EINVAL, "n_episodes and n_steps must be >= 1 (got %d, %d)", c->n_episodes,
                c->n_steps);
  if ((int64_t)c->n_episodes * c->n_steps >= (int64_t)1 << 40)
    return fail(ROLLOUT_EINVAL, "n_episodes * n_steps too large");
  if (c->n_features != 51 || c->state_dim != 54 || c->n_actions != 45)
    return fail(ROLLOUT_EINVAL, "features/state/actions must be 51/54/45");
  for (int i = 0; i < 3; ++i) {
    if (c->trunk_dims[i] != kTrunkDims[i]) return fail(ROLLOUT_EINVAL, "trunk dims must be 54,256,128");
    if (c->value_dims[i] != kValueDims[i]) return fail(ROLLOUT_EINVAL, "value head dims must be 128,64,1");
    if (c->advantage_dims[i] != kAdvDims[i])
      return fail(ROLLOUT_EINVAL, "advantage head dims must be 128,64,45");
    if (c->cur_dims[i] != kCurDims[i]) return fail(ROLLOUT_EINVAL, "curiosity dims must be 99,128,51");
  }
  if (!(c->epsilon >= 0.0f && c->epsilon <= 1.0f))
    return fail(ROLLOUT_EINVAL, "epsilon must be in [0, 1]");
  if (c->div_window < 1 || c->div_window > 32)
    return fail(ROLLOUT_EINVAL, "div_window must be in 1..32 (got %d)", c->div_window);
  if (c->max_hold < 1) return fail(ROLLOUT_EINVAL, "max_hold must be >= 1");
  if (c->recycle != 0 && c->recycle != 1) return fail(ROLLOUT_EINVAL, "recycle must be 0 or 1");
  return ROLLOUT_OK;
}

int check_tensors(const float* const* w, int count, const char* what) {
  if (!w) return ROLLOUT_OK;
  for (int i = 0; i < count; ++i)
    if (!w[i]) return fail(ROLLOUT_EINVAL, "%s tensor %d is NULL", what, i);
  return ROLLOUT_OK;
}

}  // namespace

struct per_s {
  int device = 0;
  int64_t capacity = 0;
  int32_t max_batch = 0;
  double* prefix = nullptr;  // block prefix sums, per_blocks(capacity)
  double* lanes = nullptr;   // in-block lane prefixes, 64 per block
  double* raw = nullptr;     // unnormalised weights, max_batch
};

struct dqn_s {
  int device = 0;
  dqn_config cfg;
  rl::EnvParams ep;
  const float* features = nullptr;
  const float* prices = nullptr;
  int64_t n_bars = 0;
  float* weights = nullptr;  // packed block (dqn_packed_offsets layout)
  float* heads = nullptr;    // assembly scratch of the head layers
};

struct rollout_s {
  int device = 0;
  rollout_config cfg;
  rl::EnvParams ep;
  const float* features = nullptr;
  const float* prices = nullptr;
  int64_t n_bars = 0;
  float* weights = nullptr;      // packed block
  int32_t* start_used = nullptr; // [N]
  unsigned long long* value_sched = nullptr;  // work counter of the value kernel
  int32_t* bars = nullptr;       // [L][N] bar of every step (recycling only)
  float* ftable = nullptr;       // [L][N][128] actor first-layer feature part, or null
  int32_t cus = 0;               // compute units of the device
  GaeScratch gae;
  // the rollout split into `parts` launches, the value pass of each part on
  // `side` (only when parts > 1)
  int parts = 1;
  int32_t* carry = nullptr;      // [N][kCarryWords] episode state between parts
  hipStream_t side = nullptr;
  std::vector<hipEvent_t> part_done;  // [parts] rollout part finished
  hipEvent_t values_done = nullptr;   // last value pass finished
  hipEvent_t table_go = nullptr;      // the caller's stream reached the feature table
  hipEvent_t table_done = nullptr;    // the table rows of the later parts are written
  int32_t ov_grid = 0;  // value workgroups while a rollout part runs
  int32_t ov_pad = 0;   // their LDS reservation
  int32_t tab_pad = 0;  // the same for the feature table's later rows
  int32_t last_steps = 0;  // steps of the final part (its pass is not overlapped)
  // per-wave phase cycle totals of the instrumented step kernel
  uint64_t* stamps = nullptr;
  size_t stamp_words = 0;
  bool stamping = false;
};

extern "C" {

int rollout_config_default(rollout_config* cfg, int32_t n_episodes, int32_t n_steps) {
  if (!cfg) return fail(ROLLOUT_EINVAL, "config is NULL");
  std::memset(cfg, 0, sizeof(*cfg));
  cfg->n_episodes = n_episodes;
  cfg->n_steps = n_steps;
  cfg->n_features = 51;
  cfg->state_dim = 54;
  cfg->n_actions = 45;
  std::memcpy(cfg->actor_dims, kActorDims, sizeof(kActorDims));
  std::memcpy(cfg->critic_dims, kCriticDims, sizeof(kCriticDims));
  std::memcpy(cfg->cur_dims, kCurDims, sizeof(kCurDims));
  cfg->precision = ROLLOUT_FP32;
  cfg->gamma = 0.99f;
  cfg->lambda = 0.95f;
  cfg->profit_take = 0.02f;
  cfg->stop_loss = 0.01f;
  cfg->max_hold = 50;
  cfg->div_window = 20;
  cfg->div_threshold = 1.0f;
  cfg->div_penalty = -0.1f;
  cfg->curiosity_coef = 0.01f;
  cfg->risk_coef = 0.01f;
  cfg->spread = 0.0005f;
  cfg->barrier_scale = 0.5f;
  const float ex[5] = {-1.0f, -0.5f, 0.0f, 0.5f, 1.0f};
  const float co[3] = {0.0002f, 0.0005f, 0.001f};
  std::memcpy(cfg->exposure, ex, sizeof(ex));
  std::memcpy(cfg->cost, co, sizeof(co));
  cfg->urgency_mult = 0.5f;
  cfg->overlap = -1;
  return ROLLOUT_OK;
}

int rollout_create(const rollout_config* cfg, const float* const actor[6],
                   const float* const critic[12], const float* const curiosity[4],
                   const float* features, const float* prices, int64_t n_bars, void* hip_stream,
                   rollout_handle* out) {
  if (!out) return fail(ROLLOUT_EINVAL, "out handle pointer is NULL");
  *out = nullptr;
  int rc = check_config(cfg);
  if (rc) return rc;
  rc = check_weights(actor, critic, curiosity);
  if (rc) return rc;
  if (!features || !prices) return fail(ROLLOUT_EINVAL, "features/prices are NULL");
  if (n_bars < (int64_t)cfg->n_steps + 1)
    return fail(ROLLOUT_EINVAL, "n_bars (%lld) must be >= n_steps + 1", (long long)n_bars);
  if (n_bars > ((int64_t)1 << 31) - 2) return fail(ROLLOUT_EINVAL, "n_bars too large");
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  auto* h = new (std::nothrow) rollout_s();
  if (!h) return fail(ROLLOUT_ENOMEM, "host allocation failed");
  h->cfg = *cfg;
  h->ep = env_params(*cfg);
  h->features = features;
  h->prices = prices;
  h->n_bars = n_bars;
  hipError_t e = hipGetDevice(&h->device);
  if (e != hipSuccess) {
    delete h;
    return hip_fail(e, "hipGetDevice");
  }
  const rl::PackedOffsets P = rl::packed_offsets();
  void* p = nullptr;
  if (hipMalloc(&p, (size_t)P.total * sizeof(float)) != hipSuccess) {
    (void)hipGetLastError();
    delete h;
    return fail(ROLLOUT_ENOMEM, "cannot allocate packed weights");
  }
  h->weights = static_cast<float*>(p);
  if (hipMalloc(&p, (size_t)cfg->n_episodes * sizeof(int32_t)) != hipSuccess) {
    (void)hipGetLastError();
    rollout_destroy(h);
    return fail(ROLLOUT_ENOMEM, "cannot allocate start buffer");
  }
  h->start_used = static_cast<int32_t*>(p);
  if (hipMalloc(&p, 256) != hipSuccess) {
    (void)hipGetLastError();
    rollout_destroy(h);
    return fail(ROLLOUT_ENOMEM, "cannot allocate scheduler counter");
  }
  h->value_sched = static_cast<unsigned long long*>(p);
  if (cfg->recycle) {
    if (hipMalloc(&p, (size_t)cfg->n_episodes * cfg->n_steps * sizeof(int32_t)) != hipSuccess) {
      (void)hipGetLastError();
      rollout_destroy(h);
      return fail(ROLLOUT_ENOMEM, "cannot allocate the bar record");
    }
    h->bars = static_cast<int32_t*>(p);
  }
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, h->device);
  if (e != hipSuccess) {
    rollout_destroy(h);
    return hip_fail(e, "hipDeviceGetAttribute");
  }
  h->parts = overlap_parts(*cfg, cus);
  h->cus = cus;
  // The feature table pays where the rollout's chain is latency-bound: fewer
  // workgroups (16 episodes each) than compute units.  Recycled episodes
  // leave their start + t bar sequence, so they compute the part in the step.
  const size_t table_bytes =
      (size_t)cfg->n_episodes * (size_t)cfg->n_steps * rl::kActorOut1 * sizeof(float);
  if (feature_table_enabled() && !cfg->recycle &&
      (cfg->n_episodes + rl::kRowsPerWave - 1) / rl::kRowsPerWave < cus &&
      table_bytes <= ((size_t)1 << 28)) {
    if (hipMalloc(&p, table_bytes) != hipSuccess) {
      (void)hipGetLastError();
      rollout_destroy(h);
      return fail(ROLLOUT_ENOMEM, "cannot allocate the feature table (%zu bytes)", table_bytes);
    }
    h->ftable = static_cast<float*>(p);
  }
  if (h->parts > 1) {
    if (hipMalloc(&p, (size_t)cfg->n_episodes * rl::kCarryWords * sizeof(int32_t)) != hipSuccess) {
      (void)hipGetLastError();
      rollout_destroy(h);
      return fail(ROLLOUT_ENOMEM, "cannot allocate the episode carry");
    }
    h->carry = static_cast<int32_t*>(p);
    // non-blocking: the caller's stream may be the null stream, which a
    // blocking stream would serialise against
    e = hipStreamCreateWithFlags(&h->side, hipStreamNonBlocking);
    for (int i = 0; e == hipSuccess && i <= h->parts + 2; ++i) {
      hipEvent_t ev = nullptr;
      e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
      if (e != hipSuccess) break;
      if (i < h->parts)
        h->part_done.push_back(ev);
      else if (i == h->parts)
        h->values_done = ev;
      else if (i == h->parts + 1)
        h->table_go = ev;
      else
        h->table_done = ev;
    }
    if (e != hipSuccess) {
      rollout_destroy(h);
      return hip_fail(e, "side stream and events");
    }
    // While a rollout part runs, its workgroups must keep their CUs to
    // themselves (a value workgroup beside one slows the sequential chain):
    // the value passes reserve enough LDS that none fits beside a rollout
    // workgroup, and leave as many CUs free as the rollout has workgroups.
    const bool bf16 = cfg->precision == ROLLOUT_BF16;
    int lds_cu = 0;
    e = hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor,
                              h->device);
    const int a_lds = rl::actor_lds_bytes(bf16, cfg->recycle != 0);
    const int v_lds = rl::value_lds_bytes(bf16);
    const int t_lds = rl::feature_table_lds_bytes(bf16);
    if (e != hipSuccess || a_lds < 0 || v_lds < 0 || t_lds < 0) {
      rollout_destroy(h);
      return fail(ROLLOUT_EHIP, "kernel LDS sizes");
    }
    const int need = lds_cu - a_lds - v_lds + 256;  // value + pad + rollout > lds_cu
    const int need_t = lds_cu - a_lds - t_lds + 256;
    const int64_t blocks = ((int64_t)cfg->n_episodes + 15) / 16;
    if (blocks < cus) {  // (otherwise the rollout holds every CU: no limit)
      h->ov_pad = need > 0 ? need : 0;
      h->tab_pad = need_t > 0 ? need_t : 0;
      h->ov_grid = (int32_t)(cus - blocks);
    }
    // The final part's value pass runs after the rollout: keep it to at most
    // one work item (32 fp32 / 128 bf16 rows) per CU, which takes one item's
    // time, by making that part shorter than the others.
    const int64_t item_rows = bf16 ? 128 : 32;
    const int64_t fit = (int64_t)cus * item_rows / cfg->n_episodes;
    const int64_t even = ((int64_t)cfg->n_steps + h->parts - 1) / h->parts;
    h->last_steps = (int32_t)(fit < 1 ? 1 : (fit < even ? fit : even));
  }
  rc = gae_reserve(h->gae, cfg->n_steps, cfg->n_episodes, st);
  if (rc) {
    rollout_destroy(h);
    return rc;
  }
  e = rl::pack_weights(actor, critic, curiosity, h->weights, st);
  if (e != hipSuccess) {
    rollout_destroy(h);
    return hip_fail(e, "weight packing");
  }
  *out = h;
  return ROLLOUT_OK;
}

int rollout_set_weights(rollout_handle h, const float* const actor[6], const float* const critic[12],
                        const float* const curiosity[4], void* hip_stream) {
  if (!h) return fail(ROLLOUT_EINVAL, "handle is NULL");
  int rc = check_weights(actor, critic, curiosity);
  if (rc) return rc;
  hipError_t e = rl::pack_weights(actor, critic, curiosity, h->weights,
                                  static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return hip_fail(e, "weight packing");
  return ROLLOUT_OK;
}

int rollout_collect(rollout_handle h, const int32_t* episode_starts, uint64_t seed,
                    const rollout_outputs* out, void* hip_stream) {
  if (!h) return fail(ROLLOUT_EINVAL, "handle is NULL");
  if (!episode_starts) return fail(ROLLOUT_EINVAL, "episode_starts is NULL");
  if (!out) return fail(ROLLOUT_EINVAL, "outputs struct is NULL");
  if (!out->states || !out->actions || !out->log_probs || !out->values || !out->rewards ||
      !out->dones || !out->barrier || !out->advantages || !out->returns)
    return fail(ROLLOUT_EINVAL, "a required output buffer is NULL");
  int dev = -1;
  RL_HIP(hipGetDevice(&dev), "hipGetDevice");
  if (dev != h->device)
    return fail(ROLLOUT_EINVAL, "handle was created on device %d, current device is %d", h->device, dev);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const int32_t N = h->cfg.n_episodes, L = h->cfg.n_steps;
  int rc = ROLLOUT_OK;
  if (out->counters) RL_HIP(rl::zero_words(out->counters, 3, st), "clear counters");
  auto mark = [&](int i) -> hipError_t {
    if (!out->phase_events || !out->phase_events[i]) return hipSuccess;
    return hipEventRecord(static_cast<hipEvent_t>(out->phase_events[i]), st);
  };
  RL_HIP(mark(0), "hipEventRecord(phase 0)");

  rl::RolloutArgs ra;
  ra.weights = h->weights;
  ra.features = h->features;
  ra.prices = h->prices;
  ra.n_bars = h->n_bars;
  ra.starts = episode_starts;
  ra.seed = seed;
  ra.N = N;
  ra.L = L;
  ra.ep = h->ep;
  ra.start_used = h->start_used;
  ra.states = out->states;
  ra.actions = out->actions;
  ra.log_probs = out->log_probs;
  ra.rewards = out->rewards;
  ra.dones = out->dones;
  ra.barrier = out->barrier;
  ra.logits = out->logits;
  ra.counters = out->counters;
  ra.bf16 = h->cfg.precision == ROLLOUT_BF16;
  ra.bars = h->bars;
  ra.t_begin = 0;
  ra.t_end = L;
  ra.carry = h->carry;
  ra.stamps = h->stamping ? h->stamps : nullptr;
  ra.ftable = h->ftable;
  // The feature part of every step for the current weights and features.
  // A split rollout needs only its first part's rows (and the next step's)
  // before it starts: the rest are written on the handle's second stream
  // while that part runs, and the second part waits for them.
  const int64_t rows_all = (int64_t)L * N;
  const int64_t head = L - h->last_steps;  // steps of the parts before the last
  if (h->ftable) {
    int64_t rows_first = rows_all;
    if (h->parts > 1) {
      const int64_t t1 = head / (h->parts - 1);  // first step of the second part
      rows_first = (t1 + 1) * N < rows_all ? (t1 + 1) * N : rows_all;
    }
    RL_HIP(rl::launch_feature_table(h->weights, h->features, episode_starts, h->n_bars, N, L,
                                    ra.bf16 != 0, h->ftable, 0, rows_first, 4 * h->cus, 0, st),
           "feature table launch");
    if (rows_first < rows_all) {
      RL_HIP(hipEventRecord(h->table_go, st), "hipEventRecord(table)");
      RL_HIP(hipStreamWaitEvent(h->side, h->table_go, 0), "hipStreamWaitEvent(table)");
      // (one workgroup per CU the rollout leaves free, none beside a rollout
      // workgroup: see the value passes below)
      RL_HIP(rl::launch_feature_table(h->weights, h->features, episode_starts, h->n_bars, N, L,
                                      ra.bf16 != 0, h->ftable, rows_first, rows_all,
                                      h->ov_grid > 0 ? h->ov_grid : h->cus, h->tab_pad, h->side),
             "feature table launch");
      RL_HIP(hipEventRecord(h->table_done, h->side), "hipEventRecord(table)");
    }
  }

  rl::ValueArgs va;
  va.weights = h->weights;
  va.features = h->features;
  va.states = out->states;
  va.actions = out->actions;
  va.start_used = h->start_used;
  va.bars = h->bars;
  va.N = N;
  va.L = L;
  va.ep = h->ep;
  va.values = out->values;
  va.rewards = out->rewards;
  va.counters = out->counters;
  va.sched = h->value_sched;
  va.bf16 = h->cfg.precision == ROLLOUT_BF16;
  va.t_off = 0;
  va.max_grid = 0;
  va.lds_pad = 0;

  if (h->parts == 1) {
    RL_HIP(rl::launch_actor_rollout(ra, st), "actor rollout launch");
    RL_HIP(mark(1), "hipEventRecord(phase 1)");
    RL_HIP(rl::launch_value(va, st), "value launch");
  } else {
    // part k of the rollout, then (on the side stream, once it is done) the
    // value pass over its rows, while part k + 1 runs; the rows of a part
    // are a contiguous block of the [L][N] outputs
    for (int k = 0; k < h->parts; ++k) {
      const bool last = k + 1 == h->parts;
      const int32_t t0 = (int32_t)(head * k / (h->parts - 1));
      const int32_t t1 = last ? L : (int32_t)(head * (k + 1) / (h->parts - 1));
      ra.t_begin = t0;
      ra.t_end = t1;
      if (k == 1 && h->ftable)
        RL_HIP(hipStreamWaitEvent(st, h->table_done, 0), "hipStreamWaitEvent(table)");
      RL_HIP(rl::launch_actor_rollout(ra, st), "actor rollout launch");
      RL_HIP(hipEventRecord(h->part_done[k], st), "hipEventRecord(part)");
      RL_HIP(hipStreamWaitEvent(h->side, h->part_done[k], 0), "hipStreamWaitEvent(side)");
      const int64_t r0 = (int64_t)t0 * N;
      rl::ValueArgs vk = va;
      vk.states = out->states + r0 * 54;
      vk.actions = out->actions + r0;
      vk.bars = h->bars ? h->bars + r0 : nullptr;
      vk.values = out->values + r0;
      vk.rewards = out->rewards + r0;
      vk.L = t1 - t0;
      vk.t_off = t0;
      if (k + 1 < h->parts) {  // the last pass runs after the rollout, on the whole device
        vk.max_grid = h->ov_grid;
        vk.lds_pad = h->ov_pad;
      }
      RL_HIP(rl::launch_value(vk, h->side), "value launch");
    }
    RL_HIP(mark(1), "hipEventRecord(phase 1)");
    RL_HIP(hipEventRecord(h->values_done, h->side), "hipEventRecord(values)");
    RL_HIP(hipStreamWaitEvent(st, h->values_done, 0), "hipStreamWaitEvent(values)");
  }
  RL_HIP(mark(2), "hipEventRecord(phase 2)");

  rl::GaeArgs ga;
  ga.rewards = out->rewards;
  ga.values = out->values;
  ga.dones = out->dones;
  ga.last_values = nullptr;
  ga.L = L;
  ga.N = N;
  ga.gamma = h->cfg.gamma;
  ga.lambda = h->cfg.lambda;
  ga.advantages = out->advantages;
  ga.returns = out->returns;
  ga.status = out->counters ? out->counters + 2 : nullptr;
  ga.spin_limit = rl::kGaeSpinLimit;
  rc = gae_run(h->gae, ga, st);
  if (rc) return rc;
  RL_HIP(mark(3), "hipEventRecord(phase 3)");
  return ROLLOUT_OK;
}

int gae_scan(const float* rewards, const float* values, const uint8_t* dones,
             const float* last_values, int32_t L, int32_t N, float gamma, float lambda,
             float* advantages, float* returns, void* hip_stream) {
  if (L < 0 || N < 0) return fail(ROLLOUT_EINVAL, "gae_scan: negative size (L=%d, N=%d)", L, N);
  if (L == 0 || N == 0) return ROLLOUT_OK;
  if (!rewards || !values || !dones || !advantages || !returns)
    return fail(ROLLOUT_EINVAL, "gae_scan: NULL buffer");
  if ((int64_t)L * N >= (int64_t)1 << 40) return fail(ROLLOUT_EINVAL, "gae_scan: too large");
  int dev = -1;
  RL_HIP(hipGetDevice(&dev), "hipGetDevice");
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  rl::GaeArgs ga{rewards, values,     dones,   last_values, L,
                 N,       gamma,      lambda,  advantages,  returns,
                 nullptr, rl::kGaeSpinLimit};
  std::lock_guard<std::mutex> lock(g_gae_mu);
  return gae_run(gae_cache()[std::make_pair(dev, st)], ga, st);
}

int gae_scan_noalloc(const float* rewards, const float* values, const uint8_t* dones,
                     const float* last_values, int32_t L, int32_t N, float gamma, float lambda,
                     float* advantages, float* returns, void* hip_stream) {
  static_assert(sizeof(scratch) == kNoAllocBytes, "scratch size");
  if (L < 0 || N < 0)
    return fail(ROLLOUT_EINVAL, "gae_scan_noalloc: negative size (L=%d, N=%d)", L, N);
  if (L == 0 || N == 0) return ROLLOUT_OK;
  if (!rewards || !values || !dones || !advantages || !returns)
    return fail(ROLLOUT_EINVAL, "gae_scan_noalloc: NULL buffer");
  if ((int64_t)L * N >= (int64_t)1 << 40) return fail(ROLLOUT_EINVAL, "gae_scan_noalloc: too large");
  const rl::GaeShape shape = rl::gae_shape(L, N);
  if (shape.nk > 1 && (size_t)shape.nk * (size_t)N > kNoAllocCarries)
    return fail(ROLLOUT_EINVAL,
                "gae_scan_noalloc: %d chunks of 512 steps x %d episodes need %zu carries, more "
                "than the %zu of its fixed scratch (rollouts of at most 512 steps need none)",
                shape.nk, N, (size_t)shape.nk * (size_t)N, kNoAllocCarries);
  int dev = -1;
  RL_HIP(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(ROLLOUT_EINVAL, "gae_scan_noalloc: device %d beyond %d", dev, kMaxDevices);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  std::lock_guard<std::mutex> lock(g_noalloc_mu);
  NoAllocDevice& d = g_noalloc[dev];
  if (!d.ready) {
    // once per device, with it current: this device's copy of the array
    void* ptr = nullptr;
    RL_HIP(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(ROLLOUT_EHIP, "hipGetSymbolAddress(scratch) returned NULL");
    // the ticket counter starts at zero (the carries are cleared on first
    // use of each layout, in gae_prepare)
    RL_HIP(rl::zero_words(static_cast<uint32_t*>(ptr), 64, st), "clear noalloc ticket");
    d.s.mem = static_cast<char*>(ptr);
    d.s.bytes = kNoAllocBytes;
    d.s.fixed = true;
    d.ready = true;
  }
  rl::GaeArgs ga{rewards, values,     dones,   last_values, L,
                 N,       gamma,      lambda,  advantages,  returns,
                 nullptr, rl::kGaeSpinLimit};
  return gae_run(d.s, ga, st);
}

int rollout_phase_cycles(rollout_handle h, int32_t enable, uint64_t* out, int64_t out_len,
                         int64_t* n_written) {
  static_assert(ROLLOUT_STAMP_WORDS == rl::kStampWords, "stamp layout");
  static_assert(rl::kSplit == 4 && rl::kRowsPerWave == 16, "stamp layout");
  if (!h) return fail(ROLLOUT_EINVAL, "handle is NULL");
  int dev = -1;
  RL_HIP(hipGetDevice(&dev), "hipGetDevice");
  if (dev != h->device)
    return fail(ROLLOUT_EINVAL, "handle was created on device %d, current device is %d", h->device, dev);
  const size_t words = (size_t)rl::kStampWords * rl::kSplit *
                       (size_t)((h->cfg.n_episodes + rl::kRowsPerWave - 1) / rl::kRowsPerWave);
  if (out && out_len < (int64_t)words)
    return fail(ROLLOUT_EINVAL, "rollout_phase_cycles: out_len %lld < %zu words",
                (long long)out_len, words);
  if (n_written) *n_written = 0;
  if (out) {
    RL_HIP(hipDeviceSynchronize(), "hipDeviceSynchronize");
    if (h->stamps) {
      RL_HIP(hipMemcpy(out, h->stamps, words * 8, hipMemcpyDeviceToHost), "copy stamps");
      RL_HIP(rl::zero_words(reinterpret_cast<uint32_t*>(h->stamps), words * 2, nullptr),
             "clear stamps");
      RL_HIP(hipDeviceSynchronize(), "hipDeviceSynchronize");
    } else {
      std::memset(out, 0, words * 8);
    }
    if (n_written) *n_written = (int64_t)words;
  }
  if (enable && !h->stamps) {
    void* p = nullptr;
    if (hipMalloc(&p, words * 8) != hipSuccess) {
      (void)hipGetLastError();
      return fail(ROLLOUT_ENOMEM, "stamps: cannot allocate %zu bytes", words * 8);
    }
    h->stamps = static_cast<uint64_t*>(p);
    h->stamp_words = words;
    RL_HIP(rl::zero_words(reinterpret_cast<uint32_t*>(h->stamps), words * 2, nullptr),
           "clear stamps");
    RL_HIP(hipDeviceSynchronize(), "hipDeviceSynchronize");
  }
  h->stamping = enable != 0;
  return ROLLOUT_OK;
}

void rollout_destroy(rollout_handle h) {
  if (!h) return;
  // value passes of a split rollout may still run on the handle's own
  // stream, reading the packed weights and the scratch freed below
  if (h->side) (void)hipStreamSynchronize(h->side);
  if (h->weights) (void)hipFree(h->weights);
  if (h->start_used) (void)hipFree(h->start_used);
  if (h->value_sched) (void)hipFree(h->value_sched);
  if (h->bars) (void)hipFree(h->bars);
  if (h->gae.mem) (void)hipFree(h->gae.mem);
  for (hipEvent_t ev : h->part_done) (void)hipEventDestroy(ev);
  if (h->values_done) (void)hipEventDestroy(h->values_done);
  if (h->table_go) (void)hipEventDestroy(h->table_go);
  if (h->table_done) (void)hipEventDestroy(h->table_done);
  if (h->side) (void)hipStreamDestroy(h->side);
  if (h->carry) (void)hipFree(h->carry);
  if (h->stamps) (void)hipFree(h->stamps);
  if (h->ftable) (void)hipFree(h->ftable);
  delete h;
}

const char* rollout_last_error(void) { return g_last_error.c_str(); }

int dqn_config_default(dqn_config* cfg, int32_t n_episodes, int32_t n_steps) {
  if (!cfg) return fail(ROLLOUT_EINVAL, "config is NULL");
  rollout_config base;
  rollout_config_default(&base, n_episodes, n_steps);
  std::memset(cfg, 0, sizeof(*cfg));
  cfg->n_episodes = n_episodes;
  cfg->n_steps = n_steps;
  cfg->n_features = 51;
  cfg->state_dim = 54;
  cfg->n_actions = 45;
  std::memcpy(cfg->trunk_dims, kTrunkDims, sizeof(kTrunkDims));
  std::memcpy(cfg->value_dims, kValueDims, sizeof(kValueDims));
  std::memcpy(cfg->advantage_dims, kAdvDims, sizeof(kAdvDims));
  std::memcpy(cfg->cur_dims, kCurDims, sizeof(kCurDims));
  cfg->epsilon = 0.1f;
  cfg->gamma = 0.99f;
  cfg->priority_alpha = 0.6f;
  cfg->profit_take = base.profit_take;
  cfg->stop_loss = base.stop_loss;
  cfg->max_hold = base.max_hold;
  cfg->div_window = base.div_window;
  cfg->div_threshold = base.div_threshold;
  cfg->div_penalty = base.div_penalty;
  cfg->curiosity_coef = base.curiosity_coef;
  cfg->risk_coef = base.risk_coef;
  cfg->spread = base.spread;
  cfg->barrier_scale = base.barrier_scale;
  std::memcpy(cfg->exposure, base.exposure, sizeof(base.exposure));
  std::memcpy(cfg->cost, base.cost, sizeof(base.cost));
  cfg->urgency_mult = base.urgency_mult;
  return ROLLOUT_OK;
}

int dqn_create(const dqn_config* cfg, const float* const online[12], const float* const target[12],
               const float* const curiosity[4], const float* features, const float* prices,
               int64_t n_bars, void* hip_stream, dqn_handle* out) {
  if (!out) return fail(ROLLOUT_EINVAL, "out handle pointer is NULL");
  *out = nullptr;
  int rc = check_dqn_config(cfg);
  if (rc) return rc;
  if (!online || !target || !curiosity) return fail(ROLLOUT_EINVAL, "weight array is NULL");
  if ((rc = check_tensors(online, 12, "online")) || (rc = check_tensors(target, 12, "target")) ||
      (rc = check_tensors(curiosity, 4, "curiosity")))
    return rc;
  if (!features || !prices) return fail(ROLLOUT_EINVAL, "features/prices are NULL");
  if (n_bars < (int64_t)cfg->n_steps + 1)
    return fail(ROLLOUT_EINVAL, "n_bars (%lld) must be >= n_steps + 1", (long long)n_bars);
  if (n_bars > ((int64_t)1 << 31) - 2) return fail(ROLLOUT_EINVAL, "n_bars too large");
  auto* h = new (std::nothrow) dqn_s();
  if (!h) return fail(ROLLOUT_ENOMEM, "host allocation failed");
  h->cfg = *cfg;
  h->ep = env_params(*cfg);
  h->features = features;
  h->prices = prices;
  h->n_bars = n_bars;
  hipError_t e = hipGetDevice(&h->device);
  if (e != hipSuccess) {
    delete h;
    return hip_fail(e, "hipGetDevice");
  }
  void* p = nullptr;
  if (hipMalloc(&p, (size_t)rl::dqn_packed_offsets().total * sizeof(float)) != hipSuccess) {
    (void)hipGetLastError();
    delete h;
    return fail(ROLLOUT_ENOMEM, "cannot allocate packed weights");
  }
  h->weights = static_cast<float*>(p);
  if (hipMalloc(&p, rl::dqn_pack_scratch_floats() * sizeof(float)) != hipSuccess) {
    (void)hipGetLastError();
    dqn_destroy(h);
    return fail(ROLLOUT_ENOMEM, "cannot allocate head scratch");
  }
  h->heads = static_cast<float*>(p);
  e = rl::pack_dqn_weights(online, target, curiosity, h->weights, h->heads,
                           static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) {
    dqn_destroy(h);
    return hip_fail(e, "weight packing");
  }
  *out = h;
  return ROLLOUT_OK;
}

int dqn_set_weights(dqn_handle h, const float* const online[12], const float* const target[12],
                    const float* const curiosity[4], void* hip_stream) {
  if (!h) return fail(ROLLOUT_EINVAL, "handle is NULL");
  int rc;
  if ((rc = check_tensors(online, 12, "online")) || (rc = check_tensors(target, 12, "target")) ||
      (rc = check_tensors(curiosity, 4, "curiosity")))
    return rc;
  hipError_t e = rl::pack_dqn_weights(online, target, curiosity, h->weights, h->heads,
                                      static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return hip_fail(e, "weight packing");
  return ROLLOUT_OK;
}

int dqn_set_epsilon(dqn_handle h, float epsilon) {
  if (!(epsilon >= 0.0f && epsilon <= 1.0f))
    return fail(ROLLOUT_EINVAL, "epsilon must be in [0, 1]");
  if (!h) return fail(ROLLOUT_EINVAL, "handle is NULL");
  h->cfg.epsilon = epsilon;
  return ROLLOUT_OK;
}

int dqn_collect(dqn_handle h, const int32_t* episode_starts, uint64_t seed, const dqn_outputs* out,
                void* hip_stream) {
  if (!h) return fail(ROLLOUT_EINVAL, "handle is NULL");
  if (!episode_starts) return fail(ROLLOUT_EINVAL, "episode_starts is NULL");
  if (!out) return fail(ROLLOUT_EINVAL, "outputs struct is NULL");
  if (!out->states || !out->actions || !out->q_taken || !out->q_next_max || !out->rewards ||
      !out->dones || !out->barrier || !out->td || !out->priorities)
    return fail(ROLLOUT_EINVAL, "a required output buffer is NULL");
  int dev = -1;
  RL_HIP(hipGetDevice(&dev), "hipGetDevice");
  if (dev != h->device)
    return fail(ROLLOUT_EINVAL, "handle was created on device %d, current device is %d", h->device, dev);
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  if (out->counters) RL_HIP(rl::zero_words(out->counters, 2, st), "clear counters");
  auto mark = [&](int i) -> hipError_t {
    if (!out->phase_events || !out->phase_events[i]) return hipSuccess;
    return hipEventRecord(static_cast<hipEvent_t>(out->phase_events[i]), st);
  };
  RL_HIP(mark(0), "hipEventRecord(phase 0)");
  rl::DqnArgs da;
  da.weights = h->weights;
  da.features = h->features;
  da.prices = h->prices;
  da.n_bars = h->n_bars;
  da.starts = episode_starts;
  da.seed = seed;
  da.N = h->cfg.n_episodes;
  da.L = h->cfg.n_steps;
  da.ep = h->ep;
  da.epsilon = h->cfg.epsilon;
  da.gamma = h->cfg.gamma;
  da.alpha = h->cfg.priority_alpha;
  da.recycle = h->cfg.recycle;
  da.states = out->states;
  da.next_states = out->next_states;
  da.q_values = out->q_values;
  da.actions = out->actions;
  da.explored = out->explored;
  da.q_taken = out->q_taken;
  da.q_next_max = out->q_next_max;
  da.rewards = out->rewards;
  da.dones = out->dones;
  da.barrier = out->barrier;
  da.td = out->td;
  da.priority = out->priorities;
  da.counters = out->counters;
  RL_HIP(rl::launch_dqn(da, st), "dqn launch");
  RL_HIP(mark(1), "hipEventRecord(phase 1)");
  return ROLLOUT_OK;
}

constexpr int32_t kPerMaxBatch = 1 << 20;

int per_create(int64_t capacity, int32_t max_batch, per_handle* out) {
  if (!out) return fail(ROLLOUT_EINVAL, "out handle pointer is NULL");
  *out = nullptr;
  if (capacity < 1 || capacity > ((int64_t)1 << 31) - 1)
    return fail(ROLLOUT_EINVAL, "capacity must be in 1 .. 2^31 - 1 (got %lld)", (long long)capacity);
  if (max_batch < 1 || max_batch > kPerMaxBatch)
    return fail(ROLLOUT_EINVAL, "max_batch must be in 1 .. %d (got %d)", kPerMaxBatch, max_batch);
  auto* h = new (std::nothrow) per_s();
  if (!h) return fail(ROLLOUT_ENOMEM, "host allocation failed");
  h->capacity = capacity;
  h->max_batch = max_batch;
  hipError_t e = hipGetDevice(&h->device);
  if (e != hipSuccess) {
    delete h;
    return hip_fail(e, "hipGetDevice");
  }
  void* p = nullptr;
  if (hipMalloc(&p, (size_t)rl::per_blocks(capacity) * sizeof(double)) != hipSuccess) {
    (void)hipGetLastError();
    delete h;
    return fail(ROLLOUT_ENOMEM, "cannot allocate block prefixes");
  }
  h->prefix = static_cast<double*>(p);
  if (hipMalloc(&p, (size_t)rl::per_blocks(capacity) * 64 * sizeof(double)) != hipSuccess) {
    (void)hipGetLastError();
    per_destroy(h);
    return fail(ROLLOUT_ENOMEM, "cannot allocate lane prefixes");
  }
  h->lanes = static_cast<double*>(p);
  if (hipMalloc(&p, (size_t)max_batch * sizeof(double)) != hipSuccess) {
    (void)hipGetLastError();
    per_destroy(h);
    return fail(ROLLOUT_ENOMEM, "cannot allocate weight scratch");
  }
  h->raw = static_cast<double*>(p);
  *out = h;
  return ROLLOUT_OK;
}

int per_sample(per_handle h, const float* priorities, int64_t n, int32_t batch, uint64_t seed,
               float beta, int32_t* indices, float* weights, void* hip_stream) {
  if (!h) return fail(ROLLOUT_EINVAL, "handle is NULL");
  if (!priorities || (batch > 0 && (!indices || !weights)))
    return fail(ROLLOUT_EINVAL, "per_sample: NULL buffer");
  if (n < 1 || n > h->capacity)
    return fail(ROLLOUT_EINVAL, "per_sample: n must be in 1 .. capacity (%lld), got %lld",
                (long long)h->capacity, (long long)n);
  if (batch < 0 || batch > h->max_batch)
    return fail(ROLLOUT_EINVAL, "per_sample: batch must be in 0 .. %d, got %d", h->max_batch, batch);
  int dev = -1;
  RL_HIP(hipGetDevice(&dev), "hipGetDevice");
  if (dev != h->device)
    return fail(ROLLOUT_EINVAL, "handle was created on device %d, current device is %d", h->device, dev);
  RL_HIP(rl::per_sample_launch(priorities, n, batch, seed, beta, indices, weights, h->prefix,
                               h->lanes, h->raw, static_cast<hipStream_t>(hip_stream)),
         "per_sample launch");
  return ROLLOUT_OK;
}

int per_gather(const int32_t* indices, int32_t batch, int64_t n, const float* states,
               const float* next_states, const int32_t* actions, const float* rewards,
               const uint8_t* dones, float* out_states, float* out_next_states,
               int32_t* out_actions, float* out_rewards, uint8_t* out_dones, void* hip_stream) {
  if (batch < 0 || batch > kPerMaxBatch) return fail(ROLLOUT_EINVAL, "per_gather: bad batch %d", batch);
  if (batch == 0) return ROLLOUT_OK;
  if (!indices || n < 1) return fail(ROLLOUT_EINVAL, "per_gather: NULL indices or n < 1");
  if ((states && !out_states) || (next_states && !out_next_states) || (actions && !out_actions) ||
      (rewards && !out_rewards) || (dones && !out_dones))
    return fail(ROLLOUT_EINVAL, "per_gather: a source without its output buffer");
  rl::PerGatherArgs a{indices, batch, n, states, next_states, actions, rewards, dones,
                      out_states, out_next_states, out_actions, out_rewards, out_dones};
  RL_HIP(rl::per_gather_launch(a, static_cast<hipStream_t>(hip_stream)), "per_gather launch");
  return ROLLOUT_OK;
}

int per_update(float* priorities, int64_t n, const int32_t* indices, const float* td, int32_t batch,
               float alpha, float epsilon, float max_priority, void* hip_stream) {
  if (batch < 0 || batch > kPerMaxBatch) return fail(ROLLOUT_EINVAL, "per_update: bad batch %d", batch);
  if (batch == 0) return ROLLOUT_OK;
  if (!priorities || !indices || !td) return fail(ROLLOUT_EINVAL, "per_update: NULL buffer");
  if (!(epsilon >= 0.0f && epsilon <= max_priority))
    return fail(ROLLOUT_EINVAL, "per_update: need 0 <= epsilon <= max_priority");
  RL_HIP(rl::per_update_launch(priorities, n, indices, td, batch, alpha, epsilon, max_priority,
                               static_cast<hipStream_t>(hip_stream)),
         "per_update launch");
  return ROLLOUT_OK;
}

void per_destroy(per_handle h) {
  if (!h) return;
  if (h->prefix) (void)hipFree(h->prefix);
  if (h->lanes) (void)hipFree(h->lanes);
  if (h->raw) (void)hipFree(h->raw);
  delete h;
}

void dqn_destroy(dqn_handle h) {
  if (!h) return;
  if (h->weights) (void)hipFree(h->weights);
  if (h->heads) (void)hipFree(h->heads);
  delete h;
}

}  // extern "C"
