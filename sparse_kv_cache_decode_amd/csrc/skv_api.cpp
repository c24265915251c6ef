// C ABI of the skv library: argument validation, handle lifecycle, the build
// sequence (pre-fill) and the stream-ordered decode step.  No host
// synchronisation inside skv_decode_step; the build is host-synchronous.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "skv_internal.h"

using namespace skv;

namespace {

// The side stream the handles of one device share for the host-value gather
// (default priority, created once and kept until the process ends), so that the
// number of streams, and of hardware queues in use, stays fixed however many
// layers are built.
struct DeviceStreams {
  hipStream_t side = nullptr;
};

constexpr int kMaxDevices = 64;
std::mutex g_streams_mu;
DeviceStreams g_streams[kMaxDevices];   // by device ordinal

hipError_t device_streams(DeviceStreams** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_streams_mu);
  if (!g_streams[dev].side) {
    e = hipStreamCreateWithFlags(&g_streams[dev].side, hipStreamNonBlocking);
    if (e != hipSuccess) {
      g_streams[dev].side = nullptr;
      return e;
    }
  }
  *out = &g_streams[dev];
  return hipSuccess;
}

// Failure injection for the tests of the error paths.  SKV_INJECT_FAIL="alloc:N"
// makes the N-th device allocation of each skv_build report failure (as if
// memory were exhausted); "hip:N" makes the N-th HIP call of a built handle's
// decode steps and appends report failure instead of being issued.  Only return
// codes are injected: the work before stays valid, nothing after is enqueued.
struct Injection {
  int alloc = 0, hip = 0;
};

Injection read_injection() {
  Injection j;
  const char* e = std::getenv("SKV_INJECT_FAIL");
  int n = 0;
  if (e && std::sscanf(e, "alloc:%d", &n) == 1) j.alloc = n;
  else if (e && std::sscanf(e, "hip:%d", &n) == 1) j.hip = n;
  return j;
}

// SKV_POISON_SLOTS=1: skv_build fills the key (and host-value) slot caches with
// bf16 NaN, so that a read of a slot no step has written shows as NaN output.
bool poison_slots() {
  const char* e = std::getenv("SKV_POISON_SLOTS");
  return e && e[0] == '1';
}

}  // namespace

struct skv_layer {
  skv_config cfg;
  int G = 0, n_c = 0, n_win = 0, P = 0, HD = 0, U = 0;
  int n_cand0 = 0;                   // candidates of the pre-filled context
  int n_cand = 0;                    // candidates now (n_cand0 + n_fold)
  int cand_cap = 0;                  // candidate rows per pair (n_cand0 + folds possible)
  int n_new = 0;                     // generated tokens appended so far
  int n_fold = 0;                    // appended chunks folded into the candidates (low rank)
  int64_t a_rows = 0;                // rows of A per batch element
  int upw = 0, res_words = 0;
  int n_part_att = 0;                // attention partial rows per pair
  int rebuild = SKV_REBUILD_SEPARATE; // resolved rebuild mode (FUSED, SEPARATE or OVERLAP)
  bool poisoned = false;
  bool need_reset = false;
  int inject_hip = 0;                // failure injection: the HIP call that reports failure (0: none)
  const uint16_t* v_dev = nullptr;   // device-visible address of the value store
  void* pool = nullptr;
  // carved from pool
  uint16_t* Bst = nullptr;   // B^T in the rebuild's stage order (bf16; widened from FP8 B)
  uint16_t *A = nullptr, *Bt = nullptr, *L = nullptr, *k_out = nullptr, *v_out = nullptr,
           *k_win = nullptr, *v_win = nullptr, *key_slots = nullptr, *val_slots = nullptr,
           *key_new = nullptr, *val_new = nullptr;
  int32_t *cand_map = nullptr, *outlier_ids = nullptr, *slot_cand = nullptr, *slot_chunk = nullptr,
          *miss_slot = nullptr, *miss_chunk = nullptr, *miss_cand = nullptr, *free_slot = nullptr,
          *hit_slot = nullptr, *hit_chunk = nullptr,
          *n_miss = nullptr, *hits_last = nullptr;
  uint32_t *resident = nullptr, *keys = nullptr;
  long long *hits_total = nullptr, *miss_total = nullptr;
  float* min_cos = nullptr;
  // per-step transient scratch (logits, LSE partials, selection lists, attention
  // partials): the handle's own region of the pool, laid out by `xs_layout`
  TransientLayout xs_layout;
  char* xs = nullptr;
  double* inv_freq = nullptr;
  std::vector<double> eig;
  hipStream_t side = nullptr;        // the device's shared side stream: host-value gather
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
  hipStream_t last_stream = nullptr;
  int64_t steps = 0;
  // per-phase timing: kEv events per recorded step
  std::vector<hipEvent_t> tev;
  int t_cap = 0, t_n = 0;
};

namespace {

constexpr size_t kAlign = 256;
constexpr int kEv = 7;   // score | select | rebuild | attention on the stream, gather on the side

struct Carver {
  size_t off = 0;
  template <class T>
  size_t take(size_t count) {
    size_t o = (off + kAlign - 1) / kAlign * kAlign;
    off = o + std::max<size_t>(count * sizeof(T), 1);
    return o;
  }
};

// FP8 E5M2 byte -> bf16 bits (exact: 2 mantissa bits, exponents inside bf16's).
uint16_t e5m2_to_bf16(uint8_t v) {
  const int e = (v >> 2) & 31, m = v & 3;
  float x;
  if (e == 31) x = m ? NAN : INFINITY;
  else if (e == 0) x = std::ldexp((float)m, -16);
  else x = std::ldexp(1.0f + m * 0.25f, e - 15);
  uint32_t u;
  std::memcpy(&u, &x, 4);
  u = (u >> 16) | ((uint32_t)(v & 0x80) << 8);
  return (uint16_t)u;
}

skv_status validate(const skv_config* c) {
  if (!c) return SKV_ERR_INVALID_ARG;
  if (c->landmark_format != SKV_FORMAT_BF16 && c->landmark_format != SKV_FORMAT_FP8_E5M2)
    return SKV_ERR_INVALID_ARG;
  if (c->a_format != SKV_FORMAT_BF16 && c->a_format != SKV_FORMAT_FP8_E5M2) return SKV_ERR_INVALID_ARG;
  if (c->b_format != SKV_FORMAT_BF16 && c->b_format != SKV_FORMAT_FP8_E5M2) return SKV_ERR_INVALID_ARG;
  if (c->value_placement != SKV_VALUES_DEVICE && c->value_placement != SKV_VALUES_HOST)
    return SKV_ERR_INVALID_ARG;
  if (c->temporal_cache != 0 && c->temporal_cache != 1) return SKV_ERR_INVALID_ARG;
  if (c->batch < 1 || c->n_q_heads < 1 || c->n_kv_heads < 1 || c->seq_len < 1) return SKV_ERR_SHAPE;
  if (c->head_dim != kHeadDim) return SKV_ERR_UNSUPPORTED;
  if (c->n_q_heads % c->n_kv_heads != 0) return SKV_ERR_SHAPE;
  const int G = c->n_q_heads / c->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return SKV_ERR_UNSUPPORTED;
  if (c->chunk != 4 && c->chunk != 8 && c->chunk != 16) return SKV_ERR_UNSUPPORTED;
  if (c->seq_len % c->chunk != 0) return SKV_ERR_SHAPE;
  if (c->seq_len / c->chunk > (int64_t)INT32_MAX / 64) return SKV_ERR_UNSUPPORTED;
  if (c->window < 0 || c->window % c->chunk != 0 || c->window >= c->seq_len) return SKV_ERR_SHAPE;
  if (c->n_outlier < 0) return SKV_ERR_SHAPE;
  const int64_t n_c = c->seq_len / c->chunk;
  const int64_t n_cand = n_c - c->n_outlier - c->window / c->chunk;
  if (n_cand < 1) return SKV_ERR_SHAPE;
  if (c->top_k < 1 || c->top_k > n_cand) return SKV_ERR_SHAPE;
  if (c->top_k > kMaxTopK) return SKV_ERR_UNSUPPORTED;
  const int64_t HD = (int64_t)c->n_kv_heads * c->head_dim;
  if (HD > 2048) return SKV_ERR_UNSUPPORTED;
  if (c->rank < 1 || c->rank > std::min<int64_t>(c->seq_len, HD)) return SKV_ERR_SHAPE;
  if (c->rank % 16 != 0) return SKV_ERR_UNSUPPORTED;
  if (!(c->rope_theta > 0.0) || !std::isfinite(c->rope_theta)) return SKV_ERR_SHAPE;
  if (c->max_new_tokens < 0) return SKV_ERR_SHAPE;
  if (c->new_token_mode != SKV_NEW_EXACT && c->new_token_mode != SKV_NEW_LOWRANK) return SKV_ERR_INVALID_ARG;
  if (c->rebuild_mode != SKV_REBUILD_AUTO && c->rebuild_mode != SKV_REBUILD_FUSED &&
      c->rebuild_mode != SKV_REBUILD_SEPARATE && c->rebuild_mode != SKV_REBUILD_OVERLAP)
    return SKV_ERR_INVALID_ARG;
  if ((c->rebuild_mode == SKV_REBUILD_FUSED || c->rebuild_mode == SKV_REBUILD_OVERLAP) &&
      c->value_placement == SKV_VALUES_HOST)
    return SKV_ERR_UNSUPPORTED;
  if (c->select_mode != SKV_SELECT_AUTO && c->select_mode != SKV_SELECT_FULL) return SKV_ERR_INVALID_ARG;
  // attention splits: at most kMaxSplits per pair with every appended token present
  const int64_t units = c->n_outlier + c->top_k + c->window / c->chunk +
                        ((int64_t)c->max_new_tokens + c->chunk - 1) / c->chunk;
  const int64_t per_wg = 4 * attn_units_per_wave(c->chunk);
  if ((units + per_wg - 1) / per_wg > kMaxSplits) return SKV_ERR_UNSUPPORTED;
  return SKV_OK;
}

// Kernels move bf16 and float data in 16-byte pieces.
bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; }

bool is_device_ptr(const void* p) {
  hipPointerAttribute_t at;
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return at.type == hipMemoryTypeDevice;
}

const void* host_device_ptr(const void* p) {
  hipPointerAttribute_t at;
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (at.type != hipMemoryTypeHost) return nullptr;
  void* dp = nullptr;
  if (hipHostGetDevicePointer(&dp, const_cast<void*>(p), 0) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  return dp;
}

void drop_timing(skv_layer* h) {
  for (hipEvent_t e : h->tev)
    if (e) (void)hipEventDestroy(e);
  h->tev.clear();
  h->t_cap = h->t_n = 0;
}

void release(skv_layer* h) {
  if (!h) return;
  drop_timing(h);
  if (h->pool) (void)hipFree(h->pool);
  if (h->ev_fork) (void)hipEventDestroy(h->ev_fork);
  if (h->ev_join) (void)hipEventDestroy(h->ev_join);

  delete h;
}

DecodeArgs decode_args(skv_layer* h) {
  const skv_config& c = h->cfg;
  DecodeArgs a;
  std::memset(&a, 0, sizeof(a));
  a.batch = c.batch;
  a.n_kv = c.n_kv_heads;
  a.group = h->G;
  a.chunk = c.chunk;
  a.top_k = c.top_k;
  a.n_outlier = c.n_outlier;
  a.n_win_units = h->n_win;
  a.n_new_tokens = h->n_new;
  a.n_new_units = (h->n_new + c.chunk - 1) / c.chunk;
  a.max_new = c.max_new_tokens;
  a.n_fold = h->n_fold;
  a.key_new = h->key_new;
  a.val_new = h->val_new;
  a.n_cand = h->n_cand;
  a.cand_stride = h->cand_cap;
  a.n_c = h->n_c;
  a.seq_len = c.seq_len;
  a.a_rows = h->a_rows;
  // score: a 32 KB block of landmarks per workgroup (kScoreRows bf16 rows or
  // kScoreRows8 FP8 rows; a larger grid beats longer per-workgroup loops);
  // logits rows padded to 16 bytes
  a.landmark_format = c.landmark_format;
  a.a_format = c.a_format;
  a.b_format = c.b_format;
  a.cpb = c.landmark_format == SKV_FORMAT_FP8_E5M2 ? kScoreRows8 : kScoreRows;
  a.nb_score = (h->n_cand + a.cpb - 1) / a.cpb;
  a.ncp = (h->n_cand + 3) / 4 * 4;
  // attention splits grow with the exact region (window + appended, not folded)
  a.n_split = (h->U + a.n_new_units - h->n_fold + h->upw - 1) / h->upw;
  a.upw = h->upw;
  a.n_part_att = h->n_part_att;
  a.rebuild_fused = h->rebuild != SKV_REBUILD_SEPARATE;
  a.miss_part_units = h->rebuild == SKV_REBUILD_FUSED ? kRebuildRows / c.chunk : h->upw;
  a.temporal = c.temporal_cache;
  a.host_values = c.value_placement == SKV_VALUES_HOST;
  a.scale = 1.0f / std::sqrt((float)c.head_dim);
  a.inv_freq = h->inv_freq;
  a.L = h->L;
  a.cand_map = h->cand_map;
  a.A = h->A;
  a.Bt = h->Bt;
  a.Bst = h->Bst;
  a.n_kq = (c.rank + 31) / 32;
  a.rank = c.rank;
  a.k_out = h->k_out;
  a.v_out = h->v_out;
  a.k_win = h->k_win;
  a.v_win = h->v_win;
  a.v_store = h->v_dev;
  a.key_slots = h->key_slots;
  a.val_slots = h->val_slots;
  a.slot_cand = h->slot_cand;
  a.slot_chunk = h->slot_chunk;
  a.resident = h->resident;
  a.res_words = h->res_words;
  a.miss_slot = h->miss_slot;
  a.miss_chunk = h->miss_chunk;
  a.miss_cand = h->miss_cand;
  a.free_slot = h->free_slot;
  a.hit_slot = h->hit_slot;
  a.hit_chunk = h->hit_chunk;
  a.n_miss = h->n_miss;
  a.hits_last = h->hits_last;
  a.hits_total = h->hits_total;
  a.miss_total = h->miss_total;
  a.keys = h->keys;
  select_partition(h->n_cand, c.top_k, h->G, h->P, &a.n_part, &a.part_size);
  a.n_ctiles = (h->n_cand + 15) / 16;
  a.n_ctiles_cap = (h->cand_cap + 15) / 16;
  a.sel_two_level = c.select_mode != SKV_SELECT_FULL &&
                    select2_shape(a.n_ctiles_cap, c.top_k, h->res_words, &a.sel_nt, &a.sel_tpt, &a.sel_ipt);
  // fused rebuild with the two-level selection: the units that do not depend on
  // the selection (outliers, exact region) are attended inside the selection's
  // launch, on the CUs its one workgroup per pair leaves idle
  a.n_static = 0;
  a.tile_row0 = a.n_split;
  if (h->rebuild == SKV_REBUILD_FUSED && a.sel_two_level) {
    const int static_units = c.n_outlier + a.n_win_units + a.n_new_units - h->n_fold;
    const int per_wg = kStaticWaves * attn_units_per_wave(c.chunk);
    a.n_static = (static_units + per_wg - 1) / per_wg;
    // n_static + ceil(hits / upw) <= n_split + 1 (n_static <= ceil(static_units / upw))
    if (a.n_static > 0) a.tile_row0 = a.n_split + 1;
  }
  apply_transient(a, h->xs_layout, h->xs);
  return a;
}

#define HIP_TRY(expr)                  \
  do {                                 \
    hipError_t e_ = (expr);            \
    if (e_ != hipSuccess) goto hip_fail; \
  } while (0)

// HIP_TRY for a built handle's decode and append calls, with failure injection
#define HIP_TRY_H(expr)                                              \
  do {                                                               \
    if (h->inject_hip > 0 && --h->inject_hip == 0) goto hip_fail;     \
    HIP_TRY(expr);                                                   \
  } while (0)

}  // namespace

namespace skv {

size_t transient_bytes(const skv_layer* h) { return h->xs_layout.bytes; }

skv_status decode_enqueue(skv_layer* h, const uint16_t* q, float* out, int32_t* chunk_ids, void* stream,
                          char* xs) {
  if (!h) return SKV_ERR_INVALID_ARG;
  if (h->poisoned) return SKV_ERR_STATE;
  if (!q || !out || !chunk_ids) return SKV_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(chunk_ids, 4)) return SKV_ERR_INVALID_ARG;
  // a host pointer here would fault the kernels: refuse it before any launch
  if (!is_device_ptr(q) || !is_device_ptr(out) || !is_device_ptr(chunk_ids)) return SKV_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  DecodeArgs a = decode_args(h);
  apply_transient(a, h->xs_layout, xs);
  a.q = q;
  a.out = out;
  a.chunk_ids = chunk_ids;
  {
    hipEvent_t* ev = h->t_n < h->t_cap ? &h->tev[(size_t)h->t_n * kEv] : nullptr;
    if (h->need_reset) {
      HIP_TRY_H(launch_reset_cache(a, s));
      h->need_reset = false;
    }
    // the score phase is the kernel's own start and end (recorded by its launch)
    HIP_TRY_H(launch_score(a, s, ev ? ev[0] : nullptr, ev ? ev[1] : nullptr));
    HIP_TRY_H(launch_select(a, s));
    if (ev) HIP_TRY_H(hipEventRecord(ev[2], s));
    if (h->rebuild != SKV_REBUILD_SEPARATE) {
      HIP_TRY_H(launch_tail(a, h->rebuild == SKV_REBUILD_FUSED, s));
      if (h->rebuild == SKV_REBUILD_OVERLAP) HIP_TRY_H(launch_attention_misses(a, s));
      if (ev) HIP_TRY_H(hipEventRecord(ev[3], s));
      HIP_TRY_H(launch_combine(a, s));
      if (ev) {
        HIP_TRY_H(hipEventRecord(ev[4], s));
        h->t_n++;
      }
      h->steps++;
      h->last_stream = s;
      return SKV_OK;
    }
    if (a.host_values) {
      HIP_TRY_H(hipEventRecord(h->ev_fork, s));
      HIP_TRY_H(hipStreamWaitEvent(h->side, h->ev_fork, 0));
      if (ev) HIP_TRY_H(hipEventRecord(ev[5], h->side));
      HIP_TRY_H(launch_value_gather(a, h->side));
      if (ev) HIP_TRY_H(hipEventRecord(ev[6], h->side));
      HIP_TRY_H(hipEventRecord(h->ev_join, h->side));
      HIP_TRY_H(launch_rebuild(a, s));
      if (ev) HIP_TRY_H(hipEventRecord(ev[3], s));
      HIP_TRY_H(hipStreamWaitEvent(s, h->ev_join, 0));
    } else {
      HIP_TRY_H(launch_rebuild(a, s));
      if (ev) HIP_TRY_H(hipEventRecord(ev[3], s));
    }
    HIP_TRY_H(launch_attention(a, s));
    HIP_TRY_H(launch_combine(a, s));
    if (ev) {
      HIP_TRY_H(hipEventRecord(ev[4], s));
      h->t_n++;
    }
  }
  h->steps++;
  h->last_stream = s;
  return SKV_OK;
hip_fail:
  (void)hipGetLastError();
  h->poisoned = true;
  return SKV_ERR_HIP;
}

}  // namespace skv

extern "C" {

int32_t skv_abi_version(void) { return SKV_ABI_VERSION; }

const char* skv_status_string(skv_status s) {
  switch (s) {
    case SKV_OK: return "ok";
    case SKV_ERR_INVALID_ARG: return "invalid argument";
    case SKV_ERR_SHAPE: return "shape violates the method's constraints";
    case SKV_ERR_UNSUPPORTED: return "unsupported configuration";
    case SKV_ERR_OOM: return "out of memory";
    case SKV_ERR_HIP: return "HIP runtime error";
    case SKV_ERR_STATE: return "handle poisoned by an earlier HIP error";
    case SKV_ERR_INTERNAL: return "internal error (eigensolver did not converge)";
    case SKV_ERR_SCRATCH: return "transient scratch larger than the static array of skv_decode_step_noalloc";
    default: return "unknown status";
  }
}

skv_status skv_build(const skv_config* cfg, const uint16_t* k_pre, const uint16_t* v, void* stream,
                     skv_layer** out) {
  if (out) *out = nullptr;
  skv_status st = validate(cfg);
  if (st != SKV_OK) return st;
  if (!k_pre || !v || !out) return SKV_ERR_INVALID_ARG;
  if (!aligned(k_pre, 16) || !aligned(v, 16)) return SKV_ERR_INVALID_ARG;
  if (!is_device_ptr(k_pre)) return SKV_ERR_INVALID_ARG;
  const uint16_t* v_dev = nullptr;
  if (cfg->value_placement == SKV_VALUES_DEVICE) {
    if (!is_device_ptr(v)) return SKV_ERR_INVALID_ARG;
    v_dev = v;
  } else {
    v_dev = static_cast<const uint16_t*>(host_device_ptr(v));
    if (!v_dev) return SKV_ERR_INVALID_ARG;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);

  skv_layer* h = new (std::nothrow) skv_layer();
  if (!h) return SKV_ERR_OOM;
  h->cfg = *cfg;
  const skv_config& c = *cfg;
  const int b = c.batch, H = c.n_kv_heads, C = c.chunk, K = c.top_k, O = c.n_outlier, r = c.rank;
  const int64_t S = c.seq_len;
  h->G = c.n_q_heads / H;
  h->n_c = (int)(S / C);
  h->n_win = c.window / C;
  const bool lowrank = c.new_token_mode == SKV_NEW_LOWRANK;
  h->n_cand0 = h->n_cand = h->n_c - O - h->n_win;
  // low rank: every completed chunk of appended tokens adds one candidate
  h->cand_cap = h->n_cand0 + (lowrank ? c.max_new_tokens / C : 0);
  h->a_rows = (S + (lowrank ? c.max_new_tokens : 0) + C - 1) / C * C;   // whole chunks (A is chunk-tiled)
  h->P = b * H;
  h->HD = H * kHeadDim;
  h->U = O + K + h->n_win;
  h->res_words = (h->cand_cap + 31) / 32;
  h->rebuild = c.rebuild_mode != SKV_REBUILD_AUTO ? c.rebuild_mode
              : c.value_placement == SKV_VALUES_DEVICE ? SKV_REBUILD_FUSED : SKV_REBUILD_SEPARATE;
  h->v_dev = v_dev;
  const int P = h->P, G = h->G, n_c = h->n_c, cap = h->cand_cap, HD = h->HD;
  // scratch sized for the largest candidate count the handle can reach (the
  // bf16 score block is the smaller one, so its count bounds both formats)
  const int nb_cap = (cap + kScoreRows - 1) / kScoreRows, ncp_cap = (cap + 3) / 4 * 4;
  const bool fp8 = c.landmark_format == SKV_FORMAT_FP8_E5M2;
  const int lrow = fp8 ? kHeadDim : kHeadDim * 2;   // bytes per landmark
  int n_part_cap = 1;
  for (int n = h->n_cand0; n <= cap; n++) {
    int np, ps;
    select_partition(n, K, G, P, &np, &ps);
    n_part_cap = std::max(n_part_cap, np);
  }
  {
    // attention: each wave owns at most attn_units_per_wave units (all loads issued
    // at once); split so that there are about 8 waves per CU
    const int nuw = attn_units_per_wave(C);
    const int waves_target = 2048;
    const int64_t wave_units = (int64_t)P * h->U;
    int upw_wave = (int)((wave_units + waves_target - 1) / waves_target);
    upw_wave = std::max(1, std::min(upw_wave, nuw));
    h->upw = 4 * upw_wave;
    const int64_t u_max = h->U + ((int64_t)c.max_new_tokens + C - 1) / C;   // with every appended token
    if ((int64_t)h->upw * kMaxSplits < u_max) h->upw = 4 * nuw;
  }

  // persistent state, one allocation
  Carver cv;
  const bool a8 = c.a_format == SKV_FORMAT_FP8_E5M2;
  const size_t oA = cv.take<uint8_t>((size_t)b * h->a_rows * ((r + 31) / 32 * 32) * (a8 ? 1 : 2));
  const bool b8 = c.b_format == SKV_FORMAT_FP8_E5M2;
  const size_t oBt = cv.take<uint8_t>((size_t)b * HD * r * (b8 ? 1 : 2));
  const int n_kq = (r + 31) / 32;
  const size_t oBst = cv.take<uint16_t>((size_t)P * n_kq * kHeadDim * 32);
  const size_t oL = cv.take<uint8_t>((size_t)P * cap * lrow);
  const size_t oKo = cv.take<uint16_t>((size_t)P * O * C * kHeadDim);
  const size_t oVo = cv.take<uint16_t>((size_t)P * O * C * kHeadDim);
  const size_t oKw = cv.take<uint16_t>((size_t)P * c.window * kHeadDim);
  const size_t oVw = cv.take<uint16_t>((size_t)P * c.window * kHeadDim);
  const size_t oKs = cv.take<uint16_t>((size_t)P * K * C * kHeadDim);
  const size_t oVs = cv.take<uint16_t>(c.value_placement == SKV_VALUES_HOST ? (size_t)P * K * C * kHeadDim : 0);
  const size_t oCm = cv.take<int32_t>((size_t)P * cap);
  const size_t oOi = cv.take<int32_t>((size_t)P * O);
  const size_t oSc = cv.take<int32_t>((size_t)P * K);
  const size_t oSch = cv.take<int32_t>((size_t)P * K);
  const size_t oMs = cv.take<int32_t>((size_t)P * K);
  const size_t oMch = cv.take<int32_t>((size_t)P * K);
  const size_t oMca = cv.take<int32_t>((size_t)P * K);
  const size_t oFs = cv.take<int32_t>((size_t)P * K);
  const size_t oHs = cv.take<int32_t>((size_t)P * K);
  const size_t oHc = cv.take<int32_t>((size_t)P * K);
  const size_t oNm = cv.take<int32_t>(P);
  const size_t oHl = cv.take<int32_t>(P);
  const size_t oRes = cv.take<uint32_t>((size_t)P * h->res_words);
  const size_t oKeys = cv.take<uint32_t>((size_t)P * n_c);
  const size_t oHt = cv.take<long long>(P);
  const size_t oMt = cv.take<long long>(P);
  {
    // transient scratch, laid out from offset 0 so that any 256-byte aligned base serves
    Carver tc;
    TransientLayout& t = h->xs_layout;
    t.part_keys = tc.take<uint32_t>((size_t)P * n_part_cap * K);
    t.part_idx = tc.take<int32_t>((size_t)P * n_part_cap * K);
    const int n_merge_cap = n_part_cap > 1 ? (n_part_cap + 1) / 2 : 0;   // first tree level's lists
    t.merge_keys = tc.take<uint32_t>((size_t)P * n_merge_cap * K);
    t.merge_idx = tc.take<int32_t>((size_t)P * n_merge_cap * K);
    t.logits = tc.take<float>((size_t)P * G * ncp_cap);
    t.lse_part = tc.take<float>((size_t)P * nb_cap * G * 2);
    t.tile_max = tc.take<float>((size_t)P * ((cap + 15) / 16) * G);
    const int n_split_max = (h->U + (c.max_new_tokens + C - 1) / C + h->upw - 1) / h->upw;
    // fused rebuild: one more partial per tile of kRebuildRows rows of misses
    const int mpb = kRebuildRows / C;
    // (fused: one more row, for the selection launch's static partials; see decode_args)
    h->n_part_att = n_split_max + (h->rebuild == SKV_REBUILD_FUSED     ? 1 + (K + mpb - 1) / mpb
                                   : h->rebuild == SKV_REBUILD_OVERLAP ? (K + h->upw - 1) / h->upw
                                                                       : 0);
    t.attn_part = tc.take<float>((size_t)P * h->n_part_att * G * kPartStride);
    t.bytes = (tc.off + kAlign - 1) / kAlign * kAlign;
  }
  const size_t oXs = cv.take<uint8_t>(h->xs_layout.bytes);
  const size_t oKn = cv.take<uint16_t>((size_t)P * c.max_new_tokens * kHeadDim);
  const size_t oVn = cv.take<uint16_t>((size_t)P * c.max_new_tokens * kHeadDim);
  const size_t oMc = cv.take<float>((size_t)P * n_c);
  const size_t oIf = cv.take<double>(kHeadDim / 2);
  const size_t pool_bytes = cv.off;

  // build temporaries
  const int nseg = gram_segments(b, S, HD);
  void* L_full = nullptr;
  double *gpart = nullptr, *gram = nullptr;
  std::vector<double> psi((size_t)b * HD * r);
  std::vector<double> invf(kHeadDim / 2);
  int rc;
  hipError_t herr = hipSuccess;

  // device allocations of this build, the injected one reporting failure
  const Injection inj = read_injection();
  int n_alloc = 0;
  auto dev_alloc = [&](void** ptr, size_t bytes) {
    if (inj.alloc > 0 && ++n_alloc == inj.alloc) {
      *ptr = nullptr;
      return false;
    }
    return hipMalloc(ptr, bytes) == hipSuccess;
  };
  h->inject_hip = inj.hip;
  if (!dev_alloc(&h->pool, pool_bytes)) {
    (void)hipGetLastError();
    h->pool = nullptr;
    release(h);
    return SKV_ERR_OOM;
  }
  if (!dev_alloc(&L_full, (size_t)P * n_c * lrow) || !dev_alloc((void**)&gpart, (size_t)b * nseg * HD * HD * 8) ||
      !dev_alloc((void**)&gram, (size_t)b * HD * HD * 8)) {
    (void)hipGetLastError();
    if (L_full) (void)hipFree(L_full);
    if (gpart) (void)hipFree(gpart);
    if (gram) (void)hipFree(gram);
    release(h);
    return SKV_ERR_OOM;
  }
  {
    char* base = static_cast<char*>(h->pool);
    h->A = (uint16_t*)(base + oA);
    h->Bt = (uint16_t*)(base + oBt);
    h->Bst = (uint16_t*)(base + oBst);
    h->L = (uint16_t*)(base + oL);
    h->k_out = (uint16_t*)(base + oKo);
    h->v_out = (uint16_t*)(base + oVo);
    h->k_win = (uint16_t*)(base + oKw);
    h->v_win = (uint16_t*)(base + oVw);
    h->key_slots = (uint16_t*)(base + oKs);
    h->val_slots = c.value_placement == SKV_VALUES_HOST ? (uint16_t*)(base + oVs) : nullptr;
    h->cand_map = (int32_t*)(base + oCm);
    h->outlier_ids = (int32_t*)(base + oOi);
    h->slot_cand = (int32_t*)(base + oSc);
    h->slot_chunk = (int32_t*)(base + oSch);
    h->miss_slot = (int32_t*)(base + oMs);
    h->miss_chunk = (int32_t*)(base + oMch);
    h->miss_cand = (int32_t*)(base + oMca);
    h->free_slot = (int32_t*)(base + oFs);
    h->hit_slot = (int32_t*)(base + oHs);
    h->hit_chunk = (int32_t*)(base + oHc);
    h->n_miss = (int32_t*)(base + oNm);
    h->hits_last = (int32_t*)(base + oHl);
    h->resident = (uint32_t*)(base + oRes);
    h->keys = (uint32_t*)(base + oKeys);
    h->hits_total = (long long*)(base + oHt);
    h->miss_total = (long long*)(base + oMt);
    h->xs = base + oXs;
    h->key_new = (uint16_t*)(base + oKn);
    h->val_new = (uint16_t*)(base + oVn);
    h->min_cos = (float*)(base + oMc);
    h->inv_freq = (double*)(base + oIf);
  }
  for (int i = 0; i < kHeadDim / 2; i++) invf[i] = std::pow(c.rope_theta, -2.0 * i / kHeadDim);

  {
    DeviceStreams* ds = nullptr;
    HIP_TRY(device_streams(&ds));
    h->side = ds->side;
  }
  HIP_TRY(hipEventCreateWithFlags(&h->ev_fork, hipEventDisableTiming));
  HIP_TRY(hipEventCreateWithFlags(&h->ev_join, hipEventDisableTiming));
  HIP_TRY(hipMemsetAsync(h->pool, 0, pool_bytes, s));
  if (poison_slots()) {
    HIP_TRY(launch_fill_u16(h->key_slots, (size_t)P * K * C * kHeadDim, 0x7fc0u, s));   // bf16 NaN
    if (h->val_slots) HIP_TRY(launch_fill_u16(h->val_slots, (size_t)P * K * C * kHeadDim, 0x7fc0u, s));
  }
  HIP_TRY(hipMemcpyAsync(h->inv_freq, invf.data(), invf.size() * 8, hipMemcpyHostToDevice, s));
  // post-RoPE keys -> landmarks and min-cos; outliers; candidates; exact caches
  HIP_TRY(launch_rope_landmark(k_pre, b, S, H, C, h->inv_freq, fp8, L_full, h->min_cos, s));
  HIP_TRY(launch_outliers(h->min_cos, P, n_c, n_c - h->n_win, O, h->keys, h->outlier_ids, s));
  HIP_TRY(launch_candidates(L_full, h->outlier_ids, P, n_c, n_c - h->n_win, O, cap, lrow, h->L, h->cand_map, s));
  HIP_TRY(launch_static_gather(k_pre, v_dev, h->outlier_ids, b, S, H, C, O, c.window, h->inv_freq,
                               h->k_out, h->v_out, h->k_win, h->v_win, s));
  // low-rank factors
  HIP_TRY(launch_gram(k_pre, b, S, HD, nseg, gpart, gram, s));
  HIP_TRY(hipStreamSynchronize(s));
  h->eig.resize((size_t)b * r);
  rc = top_eigvecs(gram, b, HD, r, s, psi.data(), h->eig.data(), &herr);
  if (rc == 2) goto hip_fail;
  if (rc != 0) {
    (void)hipFree(L_full);
    (void)hipFree(gpart);
    (void)hipFree(gram);
    release(h);
    return SKV_ERR_INTERNAL;
  }
  // Psi in fp64 through the (now free) Gram partials buffer, b*nseg*HD*HD >= b*HD*r
  // doubles; B^T is rounded from it and A = K Psi projected from it in float64
  HIP_TRY(hipMemcpyAsync(gpart, psi.data(), psi.size() * 8, hipMemcpyHostToDevice, s));
  HIP_TRY(launch_round_psi(gpart, b, HD, r, b8, h->Bt, s));
  HIP_TRY(launch_stage_bt(h->Bt, P, r, n_kq, b8, h->Bst, s));
  HIP_TRY(launch_project(k_pre, gpart, b, S, HD, r, C, h->a_rows, a8, h->A, s));
  HIP_TRY(launch_reset_cache(decode_args(h), s));
  HIP_TRY(hipStreamSynchronize(s));
  (void)hipFree(L_full);
  (void)hipFree(gpart);
  (void)hipFree(gram);
  h->last_stream = s;
  *out = h;
  return SKV_OK;

hip_fail:
  (void)hipGetLastError();
  (void)hipStreamSynchronize(s);
  (void)hipFree(L_full);
  (void)hipFree(gpart);
  (void)hipFree(gram);
  release(h);
  return SKV_ERR_HIP;
}

skv_status skv_decode_step(skv_layer* h, const uint16_t* q, float* out, int32_t* chunk_ids,
                           void* stream) {
  if (!h) return SKV_ERR_INVALID_ARG;
  return skv::decode_enqueue(h, q, out, chunk_ids, stream, h->xs);
}

skv_status skv_append_token(skv_layer* h, const uint16_t* k_new, const uint16_t* v_new, void* stream) {
  if (!h || !k_new || !v_new) return SKV_ERR_INVALID_ARG;
  if (h->poisoned) return SKV_ERR_STATE;
  if (!aligned(k_new, 16) || !aligned(v_new, 16)) return SKV_ERR_INVALID_ARG;
  if (!is_device_ptr(k_new) || !is_device_ptr(v_new)) return SKV_ERR_INVALID_ARG;
  if (h->n_new >= h->cfg.max_new_tokens) return SKV_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  {
    const bool lowrank = h->cfg.new_token_mode == SKV_NEW_LOWRANK;
    HIP_TRY_H(launch_append(decode_args(h), k_new, v_new, h->n_new, lowrank, s));
    h->n_new++;
    h->last_stream = s;
    if (lowrank && h->n_new % h->cfg.chunk == 0) {
      // the chunk just completed pushes the oldest exact chunk into the candidates
      HIP_TRY_H(launch_fold(decode_args(h), s));
      h->n_cand++;
      h->n_fold++;
    }
  }
  return SKV_OK;
hip_fail:
  (void)hipGetLastError();
  h->poisoned = true;
  return SKV_ERR_HIP;
}

skv_status skv_reset_temporal_cache(skv_layer* h) {
  if (!h) return SKV_ERR_INVALID_ARG;
  if (h->poisoned) return SKV_ERR_STATE;
  h->need_reset = true;
  h->steps = 0;
  return SKV_OK;
}

skv_status skv_get_stats(const skv_layer* hc, skv_stats* out) {
  if (!hc || !out) return SKV_ERR_INVALID_ARG;
  skv_layer* h = const_cast<skv_layer*>(hc);
  if (h->poisoned) return SKV_ERR_STATE;
  std::memset(out, 0, sizeof(*out));
  out->steps = h->steps;
  out->new_tokens = h->n_new;
  if (h->need_reset) return SKV_OK;   // counters are cleared by the next step
  const int P = h->P;
  std::vector<int32_t> nm(P), hl(P);
  std::vector<long long> ht(P), mt(P);
  HIP_TRY(hipStreamSynchronize(h->last_stream));
  HIP_TRY(hipStreamSynchronize(h->side));
  HIP_TRY(hipMemcpy(nm.data(), h->n_miss, P * 4, hipMemcpyDeviceToHost));
  HIP_TRY(hipMemcpy(hl.data(), h->hits_last, P * 4, hipMemcpyDeviceToHost));
  HIP_TRY(hipMemcpy(ht.data(), h->hits_total, P * 8, hipMemcpyDeviceToHost));
  HIP_TRY(hipMemcpy(mt.data(), h->miss_total, P * 8, hipMemcpyDeviceToHost));
  if (h->steps > 0) {
    for (int p = 0; p < P; p++) {
      out->last_hits += hl[p];
      out->last_misses += nm[p];
      out->total_hits += ht[p];
      out->total_misses += mt[p];
    }
    const double denom = (double)P * h->cfg.top_k;
    out->last_alpha = h->steps > 1 ? out->last_hits / denom : 0.0;
    out->mean_alpha = h->steps > 1 ? out->total_hits / (denom * (double)(h->steps - 1)) : 0.0;
    if (h->cfg.value_placement == SKV_VALUES_HOST)
      out->last_host_bytes = out->last_misses * (int64_t)h->cfg.chunk * kHeadDim * 2;
  }
  return SKV_OK;
hip_fail:
  (void)hipGetLastError();
  h->poisoned = true;
  return SKV_ERR_HIP;
}

skv_status skv_export_state(const skv_layer* hc, const skv_state_host* d) {
  if (!hc || !d) return SKV_ERR_INVALID_ARG;
  skv_layer* h = const_cast<skv_layer*>(hc);
  if (h->poisoned) return SKV_ERR_STATE;
  const skv_config& c = h->cfg;
  const int b = c.batch, H = c.n_kv_heads, C = c.chunk, O = c.n_outlier, r = c.rank;
  const int64_t S = c.seq_len;
  const int P = h->P, HD = h->HD;
  HIP_TRY(hipStreamSynchronize(h->last_stream));
  if (d->A) {   // rows 0..S-1 out of the chunk-tiled layout
    const int r_pad = (r + 31) / 32 * 32;
    const bool a8 = c.a_format == SKV_FORMAT_FP8_E5M2;
    const size_t n = (size_t)b * h->a_rows * r_pad;
    std::vector<uint8_t> raw(n * (a8 ? 1 : 2));
    HIP_TRY(hipMemcpy(raw.data(), h->A, raw.size(), hipMemcpyDeviceToHost));
    const uint16_t* r16 = reinterpret_cast<const uint16_t*>(raw.data());
    for (int bi = 0; bi < b; bi++)
      for (int64_t row = 0; row < S; row++)
        for (int k = 0; k < r; k++) {
          const int64_t at = a_tiled(bi, h->a_rows, r_pad, C, row, k);
          d->A[((size_t)bi * S + row) * r + k] = a8 ? e5m2_to_bf16(raw[at]) : r16[at];
        }
  }
  if (d->B) {
    std::vector<uint16_t> bt((size_t)b * HD * r);
    if (c.b_format == SKV_FORMAT_FP8_E5M2) {   // FP8 bytes widened to bf16
      std::vector<uint8_t> b8((size_t)b * HD * r);
      HIP_TRY(hipMemcpy(b8.data(), h->Bt, b8.size(), hipMemcpyDeviceToHost));
      for (size_t i = 0; i < b8.size(); i++) bt[i] = e5m2_to_bf16(b8[i]);
    } else {
      HIP_TRY(hipMemcpy(bt.data(), h->Bt, bt.size() * 2, hipMemcpyDeviceToHost));
    }
    for (int bi = 0; bi < b; bi++)
      for (int hh = 0; hh < H; hh++)
        for (int k = 0; k < r; k++)
          for (int dd = 0; dd < kHeadDim; dd++)
            d->B[(((size_t)bi * H + hh) * r + k) * kHeadDim + dd] =
                bt[((size_t)bi * HD + hh * kHeadDim + dd) * r + k];
  }
  if (d->landmarks && c.landmark_format == SKV_FORMAT_FP8_E5M2) {
    // FP8 bytes widened to bf16 (every E5M2 value is a bf16 value)
    std::vector<uint8_t> l8((size_t)P * h->n_cand0 * kHeadDim);
    HIP_TRY(hipMemcpy2D(l8.data(), (size_t)h->n_cand0 * kHeadDim, h->L, (size_t)h->cand_cap * kHeadDim,
                        (size_t)h->n_cand0 * kHeadDim, P, hipMemcpyDeviceToHost));
    for (size_t i = 0; i < l8.size(); i++) d->landmarks[i] = e5m2_to_bf16(l8[i]);
  } else if (d->landmarks) {
    HIP_TRY(hipMemcpy2D(d->landmarks, (size_t)h->n_cand0 * kHeadDim * 2, h->L, (size_t)h->cand_cap * kHeadDim * 2,
                        (size_t)h->n_cand0 * kHeadDim * 2, P, hipMemcpyDeviceToHost));
  }
  if (d->cand_ids)
    HIP_TRY(hipMemcpy2D(d->cand_ids, (size_t)h->n_cand0 * 4, h->cand_map, (size_t)h->cand_cap * 4,
                        (size_t)h->n_cand0 * 4, P, hipMemcpyDeviceToHost));
  if (d->outlier_ids && O) HIP_TRY(hipMemcpy(d->outlier_ids, h->outlier_ids, (size_t)P * O * 4, hipMemcpyDeviceToHost));
  if (d->k_outlier && O) HIP_TRY(hipMemcpy(d->k_outlier, h->k_out, (size_t)P * O * C * kHeadDim * 2, hipMemcpyDeviceToHost));
  if (d->v_outlier && O) HIP_TRY(hipMemcpy(d->v_outlier, h->v_out, (size_t)P * O * C * kHeadDim * 2, hipMemcpyDeviceToHost));
  if (d->k_window && c.window) HIP_TRY(hipMemcpy(d->k_window, h->k_win, (size_t)P * c.window * kHeadDim * 2, hipMemcpyDeviceToHost));
  if (d->v_window && c.window) HIP_TRY(hipMemcpy(d->v_window, h->v_win, (size_t)P * c.window * kHeadDim * 2, hipMemcpyDeviceToHost));
  if (d->min_cos) HIP_TRY(hipMemcpy(d->min_cos, h->min_cos, (size_t)P * h->n_c * 4, hipMemcpyDeviceToHost));
  if (d->eigvals) std::memcpy(d->eigvals, h->eig.data(), h->eig.size() * 8);
  return SKV_OK;
hip_fail:
  (void)hipGetLastError();
  h->poisoned = true;
  return SKV_ERR_HIP;
}

skv_status skv_set_timing(skv_layer* h, int32_t capacity) {
  if (!h || capacity < 0) return SKV_ERR_INVALID_ARG;
  if (h->poisoned) return SKV_ERR_STATE;
  (void)hipStreamSynchronize(h->last_stream);
  if (h->side) (void)hipStreamSynchronize(h->side);
  drop_timing(h);
  if (capacity == 0) return SKV_OK;
  h->tev.assign((size_t)capacity * kEv, nullptr);
  for (auto& e : h->tev) {
    if (hipEventCreate(&e) != hipSuccess) {
      (void)hipGetLastError();
      drop_timing(h);
      return SKV_ERR_OOM;
    }
  }
  h->t_cap = capacity;
  return SKV_OK;
}

skv_status skv_get_timing(const skv_layer* hc, double* phase_ms, int64_t* steps) {
  if (!hc || !phase_ms || !steps) return SKV_ERR_INVALID_ARG;
  skv_layer* h = const_cast<skv_layer*>(hc);
  if (h->poisoned) return SKV_ERR_STATE;
  for (int i = 0; i < SKV_NUM_PHASES; i++) phase_ms[i] = 0.0;
  *steps = h->t_n;
  const bool host = h->cfg.value_placement == SKV_VALUES_HOST;
  for (int i = 0; i < h->t_n; i++) {
    hipEvent_t* ev = &h->tev[(size_t)i * kEv];
    float ms;
    HIP_TRY(hipEventSynchronize(ev[4]));
    HIP_TRY(hipEventElapsedTime(&ms, ev[0], ev[1]));
    phase_ms[SKV_PHASE_SCORE] += ms;
    HIP_TRY(hipEventElapsedTime(&ms, ev[1], ev[2]));
    phase_ms[SKV_PHASE_SELECT] += ms;
    HIP_TRY(hipEventElapsedTime(&ms, ev[2], ev[3]));
    phase_ms[SKV_PHASE_REBUILD] += ms;
    HIP_TRY(hipEventElapsedTime(&ms, ev[3], ev[4]));
    phase_ms[SKV_PHASE_ATTENTION] += ms;
    if (host) {
      HIP_TRY(hipEventSynchronize(ev[6]));
      HIP_TRY(hipEventElapsedTime(&ms, ev[5], ev[6]));
      phase_ms[SKV_PHASE_VALUE_GATHER] += ms;
    }
  }
  return SKV_OK;
hip_fail:
  (void)hipGetLastError();
  h->poisoned = true;
  return SKV_ERR_HIP;
}

void skv_destroy(skv_layer* h) {
  if (!h) return;
  (void)hipStreamSynchronize(h->last_stream);
  if (h->side) (void)hipStreamSynchronize(h->side);
  release(h);
}

}  // extern "C"
