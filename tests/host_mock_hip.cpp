// Host-only driver of the library's C ABI (skv_api.cpp + eig_host.cpp) for
// sanitizer builds on a machine without a GPU.
//
// The HIP runtime is replaced by a small mock in which "device" memory is host
// memory with a registry of live allocations; streams and events are plain
// host objects.  The kernel launchers are replaced by stubs that do no work but
// check that every buffer the host side hands them lies inside one live
// allocation, at the extent the kernels index (so a wrong size in the host-side
// layout arithmetic shows here as a failed check, not as a GPU fault).  The
// Gram kernel writes a diagonal matrix with well separated eigenvalues and the fp64
// products run on the host, so that the eigensolver takes its real path.
//
// The driver runs every entry point: validation, builds in each mode, decode
// steps, appends, statistics, timing, export, reset and destroy, the failure
// injection switches (allocation failure, HIP-call failure) and the slot
// poisoning switch, and checks after each scenario that every mock allocation
// has been returned.  Exit status 0 means every check passed; AddressSanitizer,
// LeakSanitizer and UBSan report on their own.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <vector>

#include "skv_internal.h"

// ---------------------------------------------------------------------------
// mock runtime

namespace {

struct Block {
  size_t bytes;
  hipMemoryType type;
};
std::map<const char*, Block> g_blocks;   // live allocations by base address
int g_streams = 0, g_events = 0;
int g_failures = 0;

#define CHECK(cond)                                                          \
  do {                                                                       \
    if (!(cond)) {                                                           \
      std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++g_failures;                                                          \
    }                                                                        \
  } while (0)

const Block* find_block(const void* p, const char** base) {
  const char* c = static_cast<const char*>(p);
  auto it = g_blocks.upper_bound(c);
  if (it == g_blocks.begin()) return nullptr;
  --it;
  if (c >= it->first + it->second.bytes) return nullptr;
  *base = it->first;
  return &it->second;
}

// [p, p + bytes) inside one live allocation
bool inside(const void* p, size_t bytes) {
  if (bytes == 0) return true;
  const char* base;
  const Block* b = find_block(p, &base);
  return b && static_cast<const char*>(p) + bytes <= base + b->bytes;
}

void* mock_alloc(size_t bytes, hipMemoryType type) {
  void* p = std::malloc(bytes ? bytes : 1);
  if (p) g_blocks[static_cast<char*>(p)] = {bytes, type};
  return p;
}

hipError_t mock_free(void* p) {
  if (!p) return hipSuccess;
  auto it = g_blocks.find(static_cast<char*>(p));
  if (it == g_blocks.end()) return hipErrorInvalidValue;
  g_blocks.erase(it);
  std::free(p);
  return hipSuccess;
}

}  // namespace

struct ihipStream_t { int id; };
struct ihipEvent_t { double t; };

extern "C" {

hipError_t hipGetDevice(int* d) { *d = 0; return hipSuccess; }
hipError_t hipGetLastError(void) { return hipSuccess; }
hipError_t hipPeekAtLastError(void) { return hipSuccess; }
hipError_t hipMalloc(void** p, size_t n) {
  *p = mock_alloc(n, hipMemoryTypeDevice);
  return *p ? hipSuccess : hipErrorOutOfMemory;
}
hipError_t hipHostMalloc(void** p, size_t n, unsigned int) {
  *p = mock_alloc(n, hipMemoryTypeHost);
  return *p ? hipSuccess : hipErrorOutOfMemory;
}
hipError_t hipFree(void* p) { return mock_free(p); }
hipError_t hipHostFree(void* p) { return mock_free(p); }
hipError_t hipPointerGetAttributes(hipPointerAttribute_t* at, const void* p) {
  const char* base;
  const Block* b = find_block(p, &base);
  if (!b) return hipErrorInvalidValue;
  std::memset(at, 0, sizeof(*at));
  at->type = b->type;
  at->devicePointer = const_cast<void*>(p);
  at->hostPointer = b->type == hipMemoryTypeHost ? const_cast<void*>(p) : nullptr;
  return hipSuccess;
}
hipError_t hipHostGetDevicePointer(void** d, void* h, unsigned int) {
  const char* base;
  const Block* b = find_block(h, &base);
  if (!b || b->type != hipMemoryTypeHost) return hipErrorInvalidValue;
  *d = h;
  return hipSuccess;
}
hipError_t hipMemcpy(void* dst, const void* src, size_t n, hipMemcpyKind kind) {
  if (kind == hipMemcpyDeviceToHost) CHECK(inside(src, n));
  if (kind == hipMemcpyHostToDevice) CHECK(inside(dst, n));
  std::memmove(dst, src, n);
  return hipSuccess;
}
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t n, hipMemcpyKind kind, hipStream_t) {
  return hipMemcpy(dst, src, n, kind);
}
hipError_t hipMemcpy2D(void* dst, size_t dpitch, const void* src, size_t spitch, size_t width, size_t height,
                       hipMemcpyKind kind) {
  if (height == 0) return hipSuccess;
  if (kind == hipMemcpyDeviceToHost) CHECK(inside(src, spitch * (height - 1) + width));
  for (size_t i = 0; i < height; i++)
    std::memmove(static_cast<char*>(dst) + i * dpitch, static_cast<const char*>(src) + i * spitch, width);
  return hipSuccess;
}
hipError_t hipMemsetAsync(void* dst, int v, size_t n, hipStream_t) {
  CHECK(inside(dst, n));
  std::memset(dst, v, n);
  return hipSuccess;
}
hipError_t hipStreamCreateWithFlags(hipStream_t* s, unsigned int) {
  *s = new ihipStream_t{++g_streams};
  return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
hipError_t hipStreamWaitEvent(hipStream_t, hipEvent_t e, unsigned int) {
  return e ? hipSuccess : hipErrorInvalidHandle;
}
hipError_t hipEventCreate(hipEvent_t* e) {
  *e = new ihipEvent_t{0.0};
  ++g_events;
  return hipSuccess;
}
hipError_t hipEventCreateWithFlags(hipEvent_t* e, unsigned) { return hipEventCreate(e); }
hipError_t hipEventDestroy(hipEvent_t e) {
  if (!e) return hipErrorInvalidHandle;
  delete e;
  --g_events;
  return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t e, hipStream_t) {
  static double clock = 0.0;
  if (!e) return hipErrorInvalidHandle;
  e->t = (clock += 0.25);
  return hipSuccess;
}
hipError_t hipEventSynchronize(hipEvent_t e) { return e ? hipSuccess : hipErrorInvalidHandle; }
hipError_t hipEventElapsedTime(float* ms, hipEvent_t a, hipEvent_t b) {
  if (!a || !b) return hipErrorInvalidHandle;
  *ms = (float)(b->t - a->t);
  return hipSuccess;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// kernel launcher stubs: extent checks only (the Gram matrix and the fp64
// products excepted)

namespace skv {

int g_static_steps = 0;   // launches that saw static-unit attention in the selection launch

void check_decode(const DecodeArgs& a, bool step_io = true) {
  const size_t P = (size_t)a.batch * a.n_kv, K = a.top_k, G = a.group, C = a.chunk, d = kHeadDim;
  const size_t lbytes = a.landmark_format == SKV_FORMAT_FP8_E5M2 ? 1 : 2;
  if (step_io) CHECK(inside(a.q, (size_t)a.batch * a.n_kv * G * d * 2));
  CHECK(inside(a.L, P * a.cand_stride * d * lbytes));
  CHECK(inside(a.cand_map, P * a.cand_stride * 4));
  CHECK(a.n_cand <= a.cand_stride);
  CHECK(inside(a.key_slots, P * K * C * d * 2));
  CHECK(inside(a.slot_cand, P * K * 4) && inside(a.slot_chunk, P * K * 4));
  CHECK(inside(a.miss_slot, P * K * 4) && inside(a.miss_chunk, P * K * 4) && inside(a.miss_cand, P * K * 4));
  CHECK(inside(a.hit_slot, P * K * 4) && inside(a.hit_chunk, P * K * 4) && inside(a.free_slot, P * K * 4));
  CHECK(inside(a.n_miss, P * 4) && inside(a.hits_last, P * 4));
  CHECK(inside(a.hits_total, P * 8) && inside(a.miss_total, P * 8));
  CHECK(inside(a.resident, P * a.res_words * 4));
  CHECK((size_t)a.res_words * 32 >= (size_t)a.cand_stride);
  CHECK(inside(a.keys, P * a.cand_stride * 4));
  CHECK(inside(a.logits, P * G * a.ncp * 4));
  CHECK((size_t)a.ncp >= (size_t)a.n_cand);
  CHECK(inside(a.lse_part, P * a.nb_score * G * 2 * 4));
  CHECK(inside(a.tile_max, P * a.n_ctiles_cap * G * 4));
  CHECK(a.n_ctiles <= a.n_ctiles_cap && (size_t)a.n_ctiles * 16 >= (size_t)a.n_cand);
  CHECK(inside(a.part_keys, P * a.n_part * K * 4) && inside(a.part_idx, P * a.n_part * K * 4));
  CHECK(a.n_part_att >= a.n_split && a.tile_row0 >= a.n_split);
  if (a.n_static > 0) {   // static rows, then the hit splits' rows, below the first miss row
    g_static_steps++;
    CHECK(a.rebuild_fused && a.sel_two_level);
    CHECK(a.n_static + (K + a.upw - 1) / a.upw <= a.tile_row0);
    const int static_units = a.n_outlier + a.n_win_units + a.n_new_units - a.n_fold;
    CHECK(static_units > 0 && a.n_static * kStaticWaves * (32 / C) >= static_units);
  }
  if (a.rebuild_fused) CHECK(a.tile_row0 + (K + a.miss_part_units - 1) / a.miss_part_units <= a.n_part_att);
  CHECK(inside(a.attn_part, P * a.n_part_att * G * kPartStride * 4));
  if (step_io) CHECK(inside(a.out, (size_t)a.batch * a.n_kv * G * d * 4) && inside(a.chunk_ids, P * K * 4));
  CHECK(inside(a.k_out, P * a.n_outlier * C * d * 2) || a.n_outlier == 0);
  CHECK(inside(a.k_win, P * a.n_win_units * C * d * 2) || a.n_win_units == 0);
  CHECK(inside(a.v_store, (size_t)a.batch * a.n_kv * a.seq_len * d * 2));
  if (a.host_values) CHECK(inside(a.val_slots, P * K * C * d * 2));
  if (a.max_new) CHECK(inside(a.key_new, P * a.max_new * d * 2) && inside(a.val_new, P * a.max_new * d * 2));
  const size_t abytes = a.a_format == SKV_FORMAT_FP8_E5M2 ? 1 : 2;
  CHECK(a.a_rows % C == 0 && a.n_kq * 32 >= a.rank);   // chunk-tiled A, whole chunks and k-steps
  CHECK(inside(a.A, (size_t)a.batch * a.a_rows * a.n_kq * 32 * abytes));
  CHECK(a.n_kq * 32 >= a.rank && (a.n_kq - 1) * 32 < a.rank);   // the rebuild's stage-order copy of B^T
  CHECK(inside(a.Bst, P * a.n_kq * kHeadDim * 32 * 2));
  CHECK(inside(a.inv_freq, kHeadDim / 2 * 8));
}

int g_launches = 0;
hipError_t decode_stub(const DecodeArgs& a, bool step_io = true) {
  ++g_launches;
  check_decode(a, step_io);
  return hipSuccess;
}

hipError_t launch_rope_landmark(const uint16_t* k, int b, int64_t S, int H, int C, const double* invf, bool fp8,
                                void* L, float* min_cos, hipStream_t) {
  CHECK(inside(k, (size_t)b * S * H * kHeadDim * 2));
  CHECK(inside(L, (size_t)b * H * (S / C) * kHeadDim * (fp8 ? 1 : 2)));
  CHECK(inside(min_cos, (size_t)b * H * (S / C) * 4));
  CHECK(inside(invf, kHeadDim / 2 * 8));
  return hipSuccess;
}
hipError_t launch_outliers(const float* min_cos, int P, int n_c, int n_sel, int O, uint32_t* keys, int32_t* ids,
                           hipStream_t) {
  CHECK(n_sel <= n_c && O <= n_sel);
  CHECK(inside(min_cos, (size_t)P * n_c * 4));
  CHECK(inside(keys, (size_t)P * n_sel * 4));
  CHECK(inside(ids, (size_t)P * O * 4) || O == 0);
  // outliers: the first O chunks of every pair
  for (int p = 0; p < P; p++)
    for (int i = 0; i < O; i++) ids[(size_t)p * O + i] = i;
  return hipSuccess;
}
hipError_t launch_candidates(const void* L_full, const int32_t* outlier_ids, int P, int n_c, int n_sel, int O,
                             int cap, int lrow, void* L, int32_t* cand_map, hipStream_t) {
  CHECK(inside(L_full, (size_t)P * n_c * lrow));
  CHECK(inside(L, (size_t)P * cap * lrow));
  CHECK(inside(cand_map, (size_t)P * cap * 4));
  CHECK(n_sel - O <= cap);
  (void)outlier_ids;
  return hipSuccess;
}
hipError_t launch_static_gather(const uint16_t* k, const uint16_t* v, const int32_t*, int b, int64_t S, int H, int C,
                                int O, int W, const double*, uint16_t* ko, uint16_t* vo, uint16_t* kw, uint16_t* vw,
                                hipStream_t) {
  const size_t P = (size_t)b * H, d = kHeadDim;
  CHECK(inside(k, (size_t)b * S * H * d * 2));
  CHECK(inside(v, (size_t)b * H * S * d * 2));
  CHECK(O == 0 || (inside(ko, P * O * C * d * 2) && inside(vo, P * O * C * d * 2)));
  CHECK(W == 0 || (inside(kw, P * W * d * 2) && inside(vw, P * W * d * 2)));
  return hipSuccess;
}
int gram_segments(int, int64_t, int) { return 2; }
hipError_t launch_gram(const uint16_t* k, int b, int64_t S, int HD, int nseg, double* partial, double* gram,
                       hipStream_t) {
  CHECK(inside(k, (size_t)b * S * HD * 2));
  CHECK(inside(partial, (size_t)b * nseg * HD * HD * 8));
  CHECK(inside(gram, (size_t)b * HD * HD * 8));
  for (int bi = 0; bi < b; bi++)
    for (int i = 0; i < HD; i++)
      for (int j = 0; j < HD; j++) gram[((size_t)bi * HD + i) * HD + j] = i == j ? std::pow(0.8, i) : 0.0;
  return hipSuccess;
}
hipError_t launch_gemm_f64(const double* A, const double* B, double* C, int batch, int M, int N, int K,
                           hipStream_t) {
  CHECK(inside(A, (size_t)batch * M * K * 8) && inside(B, (size_t)batch * K * N * 8) &&
        inside(C, (size_t)batch * M * N * 8));
  for (int bi = 0; bi < batch; bi++)
    for (int m = 0; m < M; m++)
      for (int n = 0; n < N; n++) {
        double s = 0;
        for (int k = 0; k < K; k++) s += A[((size_t)bi * M + m) * K + k] * B[((size_t)bi * K + k) * N + n];
        C[((size_t)bi * M + m) * N + n] = s;
      }
  return hipSuccess;
}
hipError_t launch_gemm_f64_tn(const double* A, const double* B, double* C, int batch, int M, int N, int K,
                              hipStream_t) {
  CHECK(inside(A, (size_t)batch * K * M * 8) && inside(B, (size_t)batch * K * N * 8) &&
        inside(C, (size_t)batch * M * N * 8));
  for (int bi = 0; bi < batch; bi++)
    for (int m = 0; m < M; m++)
      for (int n = 0; n < N; n++) {
        double s = 0;
        for (int k = 0; k < K; k++) s += A[((size_t)bi * K + k) * M + m] * B[((size_t)bi * K + k) * N + n];
        C[((size_t)bi * M + m) * N + n] = s;
      }
  return hipSuccess;
}
hipError_t launch_round_psi(const double* psi, int b, int HD, int r, bool b8, void* bt, hipStream_t) {
  CHECK(inside(psi, (size_t)b * HD * r * 8) && inside(bt, (size_t)b * HD * r * (b8 ? 1 : 2)));
  return hipSuccess;
}
hipError_t launch_stage_bt(const void* bt, int P, int r, int n_kq, bool b8, uint16_t* bst, hipStream_t) {
  CHECK(n_kq * 32 >= r && (n_kq - 1) * 32 < r);
  CHECK(inside(bt, (size_t)P * kHeadDim * r * (b8 ? 1 : 2)) && inside(bst, (size_t)P * n_kq * kHeadDim * 32 * 2));
  return hipSuccess;
}
hipError_t launch_project(const uint16_t* k, const double* psi, int b, int64_t S, int HD, int r, int C,
                          int64_t a_rows, bool a8, void* A, hipStream_t) {
  CHECK(a_rows >= S && a_rows % C == 0 && S % C == 0);
  CHECK(inside(k, (size_t)b * S * HD * 2) && inside(psi, (size_t)b * HD * r * 8));
  CHECK(inside(A, (size_t)b * a_rows * ((r + 31) / 32 * 32) * (a8 ? 1 : 2)));
  return hipSuccess;
}
hipError_t launch_fill_u16(uint16_t* p, size_t n, uint16_t value, hipStream_t) {
  CHECK(inside(p, n * 2));
  for (size_t i = 0; i < n; i++) p[i] = value;
  return hipSuccess;
}
void select_partition(int n_cand, int, int, int, int* n_part, int* part_size) {
  *n_part = 1;
  *part_size = n_cand;
}
int select2_shape(int, int top_k, int, int* nt, int* tpt, int* ipt) {
  // the kernels' rule on the budget (two levels up to K = 512); the shape values only size launches
  *nt = 1024;
  *tpt = *ipt = 1;
  return top_k <= 512;
}
int attn_units_per_wave(int chunk) { return 32 / chunk; }   // two 16-token tiles per wave
hipError_t launch_reset_cache(const DecodeArgs& a, hipStream_t) { return decode_stub(a, false); }
hipError_t launch_score(const DecodeArgs& a, hipStream_t, hipEvent_t t0, hipEvent_t t1) {
  if (t0) (void)hipEventRecord(t0, nullptr);
  if (t1) (void)hipEventRecord(t1, nullptr);
  return decode_stub(a);
}
hipError_t launch_select(const DecodeArgs& a, hipStream_t) { return decode_stub(a); }
hipError_t launch_rebuild(const DecodeArgs& a, hipStream_t) { return decode_stub(a); }
hipError_t launch_value_gather(const DecodeArgs& a, hipStream_t) { return decode_stub(a); }
hipError_t launch_attention(const DecodeArgs& a, hipStream_t) { return decode_stub(a); }
hipError_t launch_attention_misses(const DecodeArgs& a, hipStream_t) { return decode_stub(a); }
hipError_t launch_tail(const DecodeArgs& a, bool, hipStream_t) { return decode_stub(a); }
hipError_t launch_combine(const DecodeArgs& a, hipStream_t) { return decode_stub(a); }
hipError_t launch_fold(const DecodeArgs& a, hipStream_t) { return decode_stub(a, false); }
hipError_t launch_append(const DecodeArgs& a, const uint16_t* k, const uint16_t* v, int, bool, hipStream_t) {
  CHECK(inside(k, (size_t)a.batch * a.n_kv * kHeadDim * 2) && inside(v, (size_t)a.batch * a.n_kv * kHeadDim * 2));
  return decode_stub(a, false);
}

}  // namespace skv

// ---------------------------------------------------------------------------
// scenarios

namespace {

skv_config tiny() {
  skv_config c{};
  c.batch = 2;
  c.n_q_heads = 8;
  c.n_kv_heads = 2;
  c.head_dim = 128;
  c.seq_len = 1024;
  c.rank = 32;
  c.chunk = 8;
  c.top_k = 12;
  c.n_outlier = 4;
  c.window = 32;
  c.value_placement = SKV_VALUES_DEVICE;
  c.rope_theta = 500000.0;
  c.temporal_cache = 1;
  return c;
}

struct Inputs {
  void *k = nullptr, *v = nullptr, *q = nullptr, *out = nullptr, *ids = nullptr, *kn = nullptr, *vn = nullptr;
  explicit Inputs(const skv_config& c) {
    const size_t d = c.head_dim, H = c.n_kv_heads;
    (void)hipMalloc(&k, (size_t)c.batch * c.seq_len * H * d * 2);
    if (c.value_placement == SKV_VALUES_HOST)
      (void)hipHostMalloc(&v, (size_t)c.batch * H * c.seq_len * d * 2, 0);
    else
      (void)hipMalloc(&v, (size_t)c.batch * H * c.seq_len * d * 2);
    (void)hipMalloc(&q, (size_t)c.batch * c.n_q_heads * d * 2);
    (void)hipMalloc(&out, (size_t)c.batch * c.n_q_heads * d * 4);
    (void)hipMalloc(&ids, (size_t)c.batch * H * c.top_k * 4);
    (void)hipMalloc(&kn, (size_t)c.batch * H * d * 2);
    (void)hipMalloc(&vn, (size_t)c.batch * H * d * 2);
    std::memset(k, 0, (size_t)c.batch * c.seq_len * H * d * 2);
    std::memset(v, 0, (size_t)c.batch * H * c.seq_len * d * 2);
  }
  ~Inputs() {
    (void)hipFree(k);
    (void)hipFree(v);
    (void)hipFree(q);
    (void)hipFree(out);
    (void)hipFree(ids);
    (void)hipFree(kn);
    (void)hipFree(vn);
  }
};

skv_status build(const skv_config& c, const Inputs& in, skv_layer** h) {
  return skv_build(&c, (const uint16_t*)in.k, (const uint16_t*)in.v, nullptr, h);
}

skv_status step(skv_layer* h, const Inputs& in) {
  return skv_decode_step(h, (const uint16_t*)in.q, (float*)in.out, (int32_t*)in.ids, nullptr);
}

// every entry point on a built handle, in the order a caller would use them
void exercise(const skv_config& c) {
  const size_t live = g_blocks.size();
  {
    Inputs in(c);
    skv_layer* h = nullptr;
    { const skv_status got = build(c, in, &h); if (got) std::fprintf(stderr, "build: %d\n", got); CHECK(got == SKV_OK && h); }
    if (!h) return;
    CHECK(skv_set_timing(h, 4) == SKV_OK);
    for (int t = 0; t < 3; t++) {
      CHECK(step(h, in) == SKV_OK);
      if (c.max_new_tokens > t)
        CHECK(skv_append_token(h, (const uint16_t*)in.kn, (const uint16_t*)in.vn, nullptr) == SKV_OK);
    }
    skv_stats st{};
    CHECK(skv_get_stats(h, &st) == SKV_OK && st.steps == 3);
    CHECK(st.new_tokens == (c.max_new_tokens < 3 ? c.max_new_tokens : 3));
    double ms[SKV_NUM_PHASES];
    int64_t n = 0;
    CHECK(skv_get_timing(h, ms, &n) == SKV_OK && n == 3);
    // misaligned or wrong-kind pointers are rejected before any launch
    const int before = skv::g_launches;
    CHECK(skv_decode_step(h, (const uint16_t*)((char*)in.q + 2), (float*)in.out, (int32_t*)in.ids, nullptr) ==
          SKV_ERR_INVALID_ARG);
    std::vector<uint16_t> host_q((size_t)c.batch * c.n_q_heads * c.head_dim);
    CHECK(skv_decode_step(h, host_q.data(), (float*)in.out, (int32_t*)in.ids, nullptr) == SKV_ERR_INVALID_ARG);
    CHECK(skv::g_launches == before);
    // export of everything
    const size_t b = c.batch, H = c.n_kv_heads, d = c.head_dim, C = c.chunk, S = c.seq_len;
    const size_t n_c = S / C, n_cand = n_c - c.n_outlier - c.window / C;
    std::vector<uint16_t> A(b * S * c.rank), B(b * H * c.rank * d), L(b * H * n_cand * d), ko(b * H * c.n_outlier * C * d),
        vo(ko.size()), kw(b * H * c.window * d), vw(kw.size());
    std::vector<int32_t> cand(b * H * n_cand), oi(b * H * c.n_outlier);
    std::vector<float> mc(b * H * n_c);
    std::vector<double> ev(b * c.rank);
    skv_state_host sh{A.data(), B.data(), L.data(), cand.data(), oi.data(), ko.data(), vo.data(),
                      kw.data(), vw.data(), mc.data(), ev.data()};
    CHECK(skv_export_state(h, &sh) == SKV_OK);
    for (size_t i = 0; i + 1 < (size_t)c.rank; i++) CHECK(ev[i] > ev[i + 1]);   // diagonal mock Gram
    CHECK(skv_reset_temporal_cache(h) == SKV_OK);
    CHECK(step(h, in) == SKV_OK);
    CHECK(skv_set_timing(h, 0) == SKV_OK);
    skv_destroy(h);
  }
  CHECK(g_blocks.size() == live);
}

void validation() {
  const size_t live = g_blocks.size();
  skv_config c = tiny();
  Inputs in(c);
  skv_layer* h = reinterpret_cast<skv_layer*>(0x1);
  struct Case {
    void (*edit)(skv_config&);
    skv_status expect;
  } cases[] = {
      {[](skv_config& x) { x.head_dim = 64; }, SKV_ERR_UNSUPPORTED},
      {[](skv_config& x) { x.n_q_heads = 7; }, SKV_ERR_SHAPE},
      {[](skv_config& x) { x.n_q_heads = 30; }, SKV_ERR_UNSUPPORTED},   // G = 15
      {[](skv_config& x) { x.seq_len = 1020; }, SKV_ERR_SHAPE},
      {[](skv_config& x) { x.chunk = 6; }, SKV_ERR_UNSUPPORTED},
      {[](skv_config& x) { x.top_k = 0; }, SKV_ERR_SHAPE},
      {[](skv_config& x) { x.top_k = 200; }, SKV_ERR_SHAPE},
      {[](skv_config& x) { x.rank = 20; }, SKV_ERR_UNSUPPORTED},
      {[](skv_config& x) { x.value_placement = 5; }, SKV_ERR_INVALID_ARG},
      {[](skv_config& x) { x.rebuild_mode = 9; }, SKV_ERR_INVALID_ARG},
      {[](skv_config& x) { x.select_mode = -1; }, SKV_ERR_INVALID_ARG},
      {[](skv_config& x) { x.max_new_tokens = -2; }, SKV_ERR_SHAPE},
  };
  for (const Case& cs : cases) {
    skv_config x = tiny();
    cs.edit(x);
    h = reinterpret_cast<skv_layer*>(0x1);
    { const skv_status got = build(x, in, &h); if (got != cs.expect) std::fprintf(stderr, "case %d: %d\n", (int)(&cs - cases), got); CHECK(got == cs.expect); }
    CHECK(h == nullptr);
  }
  // host memory where device memory is required
  std::vector<uint16_t> host_k((size_t)c.batch * c.seq_len * c.n_kv_heads * c.head_dim);
  CHECK(skv_build(&c, host_k.data(), (const uint16_t*)in.v, nullptr, &h) == SKV_ERR_INVALID_ARG);
  CHECK(skv_build(nullptr, (const uint16_t*)in.k, (const uint16_t*)in.v, nullptr, &h) == SKV_ERR_INVALID_ARG);
  CHECK(skv_decode_step(nullptr, (const uint16_t*)in.q, (float*)in.out, (int32_t*)in.ids, nullptr) ==
        SKV_ERR_INVALID_ARG);
  CHECK(std::strcmp(skv_status_string(99), "unknown status") == 0);
  CHECK(g_blocks.size() == live + 7);
}

// SKV_INJECT_FAIL=alloc:N: the N-th device allocation of a build fails
void allocation_failures() {
  skv_config c = tiny();
  Inputs in(c);
  const size_t live = g_blocks.size();
  int n_ok = 0;
  for (int n = 1; n <= 8; n++) {
    char v[32];
    std::snprintf(v, sizeof v, "alloc:%d", n);
    setenv("SKV_INJECT_FAIL", v, 1);
    skv_layer* h = nullptr;
    const skv_status s = build(c, in, &h);
    CHECK(s == SKV_OK || s == SKV_ERR_OOM);
    if (s == SKV_OK) {
      ++n_ok;
      CHECK(h != nullptr);
      CHECK(step(h, in) == SKV_OK);
      skv_destroy(h);
    } else {
      CHECK(h == nullptr);
      CHECK(n_ok == 0);   // failures at every allocation, then none
    }
    CHECK(g_blocks.size() == live);
  }
  CHECK(n_ok > 0 && n_ok < 8);
  unsetenv("SKV_INJECT_FAIL");
}

// SKV_INJECT_FAIL=hip:N: the N-th HIP call of the decode steps and appends fails
void hip_failures(skv_config c) {
  Inputs in(c);
  const size_t live = g_blocks.size();
  const int events = g_events;
  for (int n = 1; n <= 40; n += 3) {
    char v[32];
    std::snprintf(v, sizeof v, "hip:%d", n);
    setenv("SKV_INJECT_FAIL", v, 1);
    skv_layer* h = nullptr;
    CHECK(build(c, in, &h) == SKV_OK);
    unsetenv("SKV_INJECT_FAIL");
    if (!h) continue;
    skv_status s = SKV_OK;
    int t = 0;
    for (; t < 12 && s == SKV_OK; t++) {
      s = step(h, in);
      if (s == SKV_OK && c.max_new_tokens > t)
        s = skv_append_token(h, (const uint16_t*)in.kn, (const uint16_t*)in.vn, nullptr);
    }
    CHECK(s == SKV_ERR_HIP);
    CHECK(step(h, in) == SKV_ERR_STATE);
    CHECK(skv_append_token(h, (const uint16_t*)in.kn, (const uint16_t*)in.vn, nullptr) == SKV_ERR_STATE);
    skv_stats st{};
    CHECK(skv_get_stats(h, &st) == SKV_ERR_STATE);
    CHECK(skv_reset_temporal_cache(h) == SKV_ERR_STATE);
    CHECK(skv_set_timing(h, 2) == SKV_ERR_STATE);
    skv_destroy(h);
    CHECK(g_blocks.size() == live);
    CHECK(g_events == events);
  }
}

}  // namespace

int main() {
  validation();
  skv_config c = tiny();
  for (int mode : {SKV_REBUILD_AUTO, SKV_REBUILD_FUSED, SKV_REBUILD_SEPARATE, SKV_REBUILD_OVERLAP}) {
    c.rebuild_mode = mode;
    exercise(c);
  }
  c = tiny();
  c.value_placement = SKV_VALUES_HOST;
  exercise(c);
  c = tiny();
  c.max_new_tokens = 20;
  exercise(c);
  c.new_token_mode = SKV_NEW_LOWRANK;
  c.a_format = SKV_FORMAT_FP8_E5M2;
  c.b_format = SKV_FORMAT_FP8_E5M2;
  c.landmark_format = SKV_FORMAT_FP8_E5M2;
  exercise(c);
  c = tiny();
  c.temporal_cache = 0;
  c.select_mode = SKV_SELECT_FULL;
  exercise(c);
  setenv("SKV_POISON_SLOTS", "1", 1);
  c = tiny();
  c.value_placement = SKV_VALUES_HOST;
  exercise(c);
  unsetenv("SKV_POISON_SLOTS");
  allocation_failures();
  c = tiny();
  hip_failures(c);
  c.value_placement = SKV_VALUES_HOST;
  hip_failures(c);
  c = tiny();
  c.max_new_tokens = 8;
  c.new_token_mode = SKV_NEW_LOWRANK;
  hip_failures(c);
  std::printf("launches %d failures %d live blocks %zu static-split launches %d\n", skv::g_launches, g_failures,
              g_blocks.size(), skv::g_static_steps);
  return g_failures == 0 ? 0 : 1;
}
