// Decode-step kernels for gfx950, following the decode algorithm of "ShadowKV ..."
// (papercache deep notes, section A2; paper-graph-ui summary, section 3.4,
// "Decoding-Time KV Selection via Landmark-Guided Approximate Attention" and
// "Sparse KV Reconstruction and Overlapping Strategy").
//
//  score        : landmark GEMV: every 256-B landmark row is read once and dotted
//                 with the G query heads of its KV head; the d = 128 contraction
//                 runs on MFMA 16x16x32 bf16 (16 landmarks x 16 head columns per
//                 tile, fp32 accumulation) so the vector ALUs only run the softmax
//                 epilogue.  Writes fp32 logits, per-head log-sum-exp partials
//                 and the largest logit of every 16-candidate tile and head.
//  select       : one workgroup per (batch, KV head) pair combines the LSE, forms
//                 the chunk score max_g(l_g - LSE_g) (log of the group max of the
//                 softmax probabilities), selects the top-K chunks with radix
//                 selects in LDS (first over the tiles' maxima, then over the
//                 chunks of the tiles that can hold a selected chunk; or over
//                 every chunk, in parts for long contexts) and runs the
//                 temporal-cache index scan (hits, misses, slot assignment).
//  tail         : one launch that rebuilds the keys of the missed chunks,
//                 RoPE(Gather(A, I_miss) B), as bf16 MFMA 16x16x32 tiles with the
//                 rotation in the epilogue, and attends them from LDS, while its
//                 other workgroups attend the outliers, the slots that hit and
//                 the window (rebuild and attention are also separate kernels).
//  value_gather : missed chunks' values from pinned host memory (side stream).
//  attention    : split-K flash-decode over [outliers; selected; window] with an
//                 online softmax in fp32, then a per-(pair, head) merge of splits.
// Workgroups never wait on one another inside a kernel: device-scope fences on
// gfx950 write back and invalidate the whole L2, so every cross-workgroup
// hand-off goes through a kernel boundary instead.
#include <hip/hip_ext.h>

#include <algorithm>
#include <type_traits>

#include "skv_internal.h"
#include "skv_select.h"

namespace skv {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;

// ---------------------------------------------------------------------------
__global__ void reset_cache_kernel(DecodeArgs a) {
  const int p = blockIdx.x;
  for (int i = threadIdx.x; i < a.top_k; i += blockDim.x) {
    a.slot_cand[(int64_t)p * a.top_k + i] = -1;
    a.slot_chunk[(int64_t)p * a.top_k + i] = -1;
  }
  for (int i = threadIdx.x; i < a.res_words; i += blockDim.x) a.resident[(int64_t)p * a.res_words + i] = 0u;
  if (threadIdx.x == 0) {
    a.n_miss[p] = 0;
    a.hits_last[p] = 0;
    a.hits_total[p] = 0;
    a.miss_total[p] = 0;
  }
}

hipError_t launch_reset_cache(const DecodeArgs& a, hipStream_t st) {
  reset_cache_kernel<<<a.batch * a.n_kv, 256, 0, st>>>(a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Score epilogue, shared by both landmark formats: one 16-landmark tile's MFMA
// output (lane (head col, kq) holds landmarks cb .. cb+3 of head col) scaled to
// logits, stored, folded into the lane's running (max, sum) of exp, and the
// tile's largest logit of each head stored for the two-level selection (tile
// (cb - 4kq) / 16 of the pair; a tile past the candidates writes nothing).
// Called by every lane of the wave.
template <int G>
__device__ __forceinline__ void score_tile_out(const DecodeArgs& a, float* lg, float* tmax, int col, int kq, int cb,
                                               int c1, f32x4 acc, float& m_run, float& s_run) {
  float v[4];
#pragma unroll
  for (int i = 0; i < 4; i++) v[i] = acc[i] * a.scale;
  float mx = kNegBig;
#pragma unroll
  for (int i = 0; i < 4; i++)
    if (cb + i < c1) mx = fmaxf(mx, v[i]);
  if (col < G && cb < c1) {
    if (cb + 4 <= c1) {
      *reinterpret_cast<f32x4*>(lg + cb) = (f32x4){v[0], v[1], v[2], v[3]};
    } else {
      for (int i = 0; i < 4 && cb + i < c1; i++) lg[cb + i] = v[i];
    }
    const float mn = fmaxf(m_run, mx);
    float add = 0.f;
#pragma unroll
    for (int i = 0; i < 4; i++)
      if (cb + i < c1) add += __expf(v[i] - mn);
    s_run = s_run * __expf(m_run - mn) + add;
    m_run = mn;
  }
  // the tile's maximum of head col: lanes col, col + 16, col + 32, col + 48
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const int tb = cb - 4 * kq;   // first candidate of the tile
  if (kq == 0 && col < G && tb < c1) tmax[(tb >> 4) * G + col] = mx;
}

// The workgroup's per-head (max, sum) partial from its 16 lanes per head.
template <int G>
__device__ __forceinline__ void score_lse_out(const DecodeArgs& a, int p, int blk, int w, int col, int kq,
                                              float m_run, float s_run, float (&red)[2][16][16]) {
  if (col < G) {
    red[0][w * 4 + kq][col] = m_run;
    red[1][w * 4 + kq][col] = s_run;
  }
  __syncthreads();
  if (threadIdx.x < G) {
    float M = kNegBig;
    for (int k = 0; k < 16; k++) M = fmaxf(M, red[0][k][threadIdx.x]);
    float S = 0.f;
    for (int k = 0; k < 16; k++) S += red[1][k][threadIdx.x] * __expf(red[0][k][threadIdx.x] - M);
    float* dst = a.lse_part + (((int64_t)p * a.nb_score + blk) * G + threadIdx.x) * 2;
    dst[0] = M;
    dst[1] = S;
  }
}

// Cache policy of the landmark stream (read once per step): sc0 nt, the
// non-temporal hint, so that the stream does not displace what stays cached.
// At the Llama-3.1-8B shape the bf16 score kernel takes 46.2 instead of 50.1 us
// (event-timed); the same hint on the select's logits reads (written just
// before) or on the attention's K/V reads is neutral or slower, and on the FP8
// score kernel's direct loads slower.
constexpr int kStreamPolicy = 3;

// Score.  A workgroup takes a block of kScoreRows candidate landmarks (32 KB).
// The block is copied into LDS with direct global->LDS loads, each wave
// instruction reading 1 KB of contiguous rows (full 128-byte lines; reading
// the MFMA operand layout straight from memory touches only 64 bytes of a row
// per instruction, and streamed about 5 % slower).  The 16-byte pieces of row r
// sit at position piece ^ (r & 15), so the operand reads of 16 rows hit 16
// distinct LDS bank groups.  Wave w then takes tiles w*2, w*2+1 of 16
// landmarks.  MFMA operands (16x16x32): A = landmarks, lane (row r = lane%16,
// kq = lane/16) holds dims j*32 + kq*8 .. +7 of landmark r; B = q^T, lane
// (col g = lane%16, kq) holds the same dims of head g.  Output lane (g, kq)
// holds landmarks kq*4 .. kq*4+3 of head g.

template <int G>
__global__ __launch_bounds__(256) void score_kernel(DecodeArgs a) {
  __shared__ u32x4 stage[kScoreRows * 16];
  __shared__ float red[2][16][16];   // (m, s) per (wave, kq) and head
  const int p = blockIdx.y, blk = blockIdx.x;
  const int b = p / a.n_kv, h = p % a.n_kv;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = lane & 15, kq = lane >> 4;
  const int hq = a.n_kv * G;
  const int c0 = blk * kScoreRows, c1 = min(a.n_cand, c0 + kScoreRows), nr = c1 - c0;
  const uint16_t* Lp = a.L + ((int64_t)p * a.cand_stride + c0) * kHeadDim;
  // rows past a ragged block's end repeat its last row; their outputs are not used
#pragma unroll
  for (int i = w; i < kScoreRows / 4; i += 4) {
    const int s = i * 64 + lane;
    const int row = s >> 4, c = (s & 15) ^ (row & 15);
    __builtin_amdgcn_global_load_lds(Lp + (int64_t)min(row, nr - 1) * kHeadDim + c * 8,
                                     (__attribute__((address_space(3))) void*)(stage + i * 64), 16, 0,
                                     kStreamPolicy);
  }
  // head columns past G repeat head G-1; their outputs are not used
  bf16x8 bq[4];
  const uint16_t* qp = a.q + ((int64_t)b * hq + h * G + min(col, G - 1)) * kHeadDim + kq * 8;
#pragma unroll
  for (int j = 0; j < 4; j++) bq[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qp + j * 32));
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  float* lg = a.logits + ((int64_t)p * G + (col < G ? col : 0)) * a.ncp;
  float* tmax = a.tile_max + (int64_t)p * a.n_ctiles * G;
  float m_run = kNegBig, s_run = 0.f;
  constexpr int kTiles = kScoreRows / 64;   // 16-row tiles per wave
#pragma unroll
  for (int t = 0; t < kTiles; t++) {
    const int row = w * (kScoreRows / 4) + t * 16 + col;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const u32x4 av = stage[row * 16 + ((j * 4 + kq) ^ (row & 15))];
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), bq[j], acc, 0, 0, 0);
    }
    score_tile_out<G>(a, lg, tmax, col, kq, c0 + w * (kScoreRows / 4) + t * 16 + kq * 4, c1, acc, m_run, s_run);
  }
  score_lse_out<G>(a, p, blk, w, col, kq, m_run, s_run, red);
}

// Score over FP8 (E5M2) landmarks: 128-byte rows, kScoreRows8 per workgroup (the
// same 32 KB block).  Lane (row r, kq) loads dims kq*32 .. kq*32+31 of its row
// with two 16-byte loads per tile, all tiles' loads issued first; MFMA j
// (16x16x32 fp16) takes dims kq*32 + j*8 .. +7, and q's operand follows the same
// assignment (a dot product does not depend on the order of the dims).  An E5M2
// byte is the high byte of the fp16 with the same value, so widening is a shift;
// q's bf16 values convert to fp16 exactly in fp16's normal range; beyond it they
// saturate at +-65504 (no inf, so no NaN logits), below 2^-14 they lose bits.

__device__ __forceinline__ u32x4 e5m2x8_to_f16x8(uint32_t lo, uint32_t hi) {
  return (u32x4){((lo & 0xffu) << 8) | ((lo & 0xff00u) << 16), ((lo >> 8) & 0xff00u) | (lo & 0xff000000u),
                 ((hi & 0xffu) << 8) | ((hi & 0xff00u) << 16), ((hi >> 8) & 0xff00u) | (hi & 0xff000000u)};
}

template <int G>
__global__ __launch_bounds__(256) void score_fp8_kernel(DecodeArgs a) {
  __shared__ float red[2][16][16];   // (m, s) per (wave, kq) and head
  typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
  const int p = blockIdx.y, blk = blockIdx.x;
  const int b = p / a.n_kv, h = p % a.n_kv;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = lane & 15, kq = lane >> 4;
  const int hq = a.n_kv * G;
  const int c0 = blk * kScoreRows8, c1 = min(a.n_cand, c0 + kScoreRows8), nr = c1 - c0;
  const uint8_t* Lp = reinterpret_cast<const uint8_t*>(a.L) + ((int64_t)p * a.cand_stride + c0) * kHeadDim;
  constexpr int kTiles = kScoreRows8 / 64;   // 16-row tiles per wave
  // rows past a ragged block's end repeat its last row; their outputs are not used
  u32x4 lf[kTiles][2];
#pragma unroll
  for (int t = 0; t < kTiles; t++) {
    const uint8_t* rp = Lp + (int64_t)min(w * (kScoreRows8 / 4) + t * 16 + col, nr - 1) * kHeadDim + kq * 32;
    lf[t][0] = *reinterpret_cast<const u32x4*>(rp);
    lf[t][1] = *reinterpret_cast<const u32x4*>(rp + 16);
  }
  // head columns past G repeat head G-1; their outputs are not used
  f16x8 bq[4];
  const uint16_t* qp = a.q + ((int64_t)b * hq + h * G + min(col, G - 1)) * kHeadDim + kq * 32;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    float x[8];
    unpack8(*reinterpret_cast<const u32x4*>(qp + j * 8), x);
#pragma unroll
    for (int k = 0; k < 8; k++) bq[j][k] = (_Float16)fminf(fmaxf(x[k], -65504.0f), 65504.0f);   // saturate
  }
  float* lg = a.logits + ((int64_t)p * G + (col < G ? col : 0)) * a.ncp;
  float* tmax = a.tile_max + (int64_t)p * a.n_ctiles * G;
  float m_run = kNegBig, s_run = 0.f;
#pragma unroll
  for (int t = 0; t < kTiles; t++) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const u32x4 half = lf[t][j / 2];
      const u32x4 av = e5m2x8_to_f16x8(half[(j % 2) * 2], half[(j % 2) * 2 + 1]);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, av), bq[j], acc, 0, 0, 0);
    }
    score_tile_out<G>(a, lg, tmax, col, kq, c0 + w * (kScoreRows8 / 4) + t * 16 + kq * 4, c1, acc, m_run, s_run);
  }
  score_lse_out<G>(a, p, blk, w, col, kq, m_run, s_run, red);
}

// With t0 / t1, the launch itself records the kernel's start and end in those
// events (hipExtLaunchKernel: the dispatch's own timestamps, not event packets
// around it, whose barriers add a few microseconds to the measured span).
template <int G>
static void launch_score_g(const DecodeArgs& a, dim3 grid, hipStream_t st, hipEvent_t t0, hipEvent_t t1) {
  const bool fp8 = a.landmark_format == SKV_FORMAT_FP8_E5M2;
  if (t0 || t1) {
    if (fp8) hipExtLaunchKernelGGL(score_fp8_kernel<G>, grid, dim3(256), 0, st, t0, t1, 0u, a);
    else hipExtLaunchKernelGGL(score_kernel<G>, grid, dim3(256), 0, st, t0, t1, 0u, a);
  } else if (fp8) {
    score_fp8_kernel<G><<<grid, 256, 0, st>>>(a);
  } else {
    score_kernel<G><<<grid, 256, 0, st>>>(a);
  }
}

hipError_t launch_score(const DecodeArgs& a, hipStream_t st, hipEvent_t t0, hipEvent_t t1) {
  const dim3 grid(a.nb_score, a.batch * a.n_kv);
  switch (a.group) {
    case 1: launch_score_g<1>(a, grid, st, t0, t1); break;
    case 2: launch_score_g<2>(a, grid, st, t0, t1); break;
    case 4: launch_score_g<4>(a, grid, st, t0, t1); break;
    case 8: launch_score_g<8>(a, grid, st, t0, t1); break;
    case 16: launch_score_g<16>(a, grid, st, t0, t1); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Selection, workgroups of kSelThreads.  The chunk key of a candidate is
// max_g(l_g - LSE_g), the log of the group max of the softmax probabilities,
// with LSE_g combined from the score workgroups' partials; keys are compared as
// order-preserving uint32.
//  select_kernel, one workgroup per pair while the pair's logits are at most
//    256 KB: thread t forms the keys of candidates [t*PT, t*PT + PT) in
//    registers straight from the logits, the top-K is found by a radix select whose histogram lives in LDS
//    (ascending candidate order, ties to the lower index), then the temporal-
//    cache index scan runs.  All per-pair state the scan touches (slot map,
//    resident bitmap, miss / free lists) is staged in LDS.
//  With more logits per pair the candidates are cut into n_part parts whose
//    top-K are taken the same way by separate workgroups (part_topk_kernel,
//    grid (n_part, P)); merged_select_kernel then selects from the merged part
//    lists.  The pair's top-K is
//    contained in that union: an element beaten by K others inside its part is
//    beaten by them overall.
// LDS layout of both per-pair kernels (ints): hist[2048 + kTopkSmall] | sh[32] |
// sel[K] | selch[K] | freel[K] | missp[K] | scl[K] | resl[res_words], followed in
// merged_select_kernel by keys[m] | idx[m] (m the merged length) when they fit.

constexpr int kSelThreads = 1024;
constexpr int kHist = 2048 + kTopkSmall;

// position of x in the ascending v[0, n), or -1
__device__ __forceinline__ int sorted_find(const int* v, int n, int x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (v[mid] < x) lo = mid + 1; else hi = mid;
  }
  return lo < n && v[lo] == x ? lo : -1;
}

void select_partition(int n_cand, int top_k, int group, int pairs, int* n_part, int* part_size) {
  // One workgroup per pair while its logits are at most 256 KB (one CU pulls that
  // in about as fast as a second kernel launch would cost).  Beyond, about one
  // stage-1 workgroup per CU, parts at least 2K long (a part's top-K keeps at most
  // half of it) and at most 16K (register keys); the part lists are then merged
  // in a tree (merge_groups).
  int np = 1;
  if ((int64_t)group * n_cand > 65536 || n_cand > kSelThreads * 16) {
    np = std::min({(256 + pairs - 1) / pairs, n_cand / (2 * top_k), 64});
    np = std::max({np, 2, (n_cand + kSelThreads * 16 - 1) / (kSelThreads * 16)});
    // a part just past 4 or 8 keys per thread would double every thread's
    // registers and loads: take a few more, smaller parts instead
    for (int tier : {kSelThreads * 4, kSelThreads * 8}) {
      const int ps = (n_cand + np - 1) / np;
      if (ps > tier && ps <= tier + tier / 8) np = (n_cand + tier - 1) / tier;
    }
  }
  const int ps = np == 1 ? n_cand : ((n_cand + np - 1) / np + 15) / 16 * 16;   // 16-B aligned parts
  *part_size = ps;
  *n_part = (n_cand + ps - 1) / ps;
}

// keys per thread of the register-resident selection for n candidates
static int keys_per_thread(int n) { return n <= kSelThreads * 4 ? 4 : (n <= kSelThreads * 8 ? 8 : 16); }

// Lists merged by one workgroup of the merge tree: their entries (at most K each)
// fit 16 per thread in registers.
int merge_groups(int top_k) { return std::max(2, kSelThreads * 16 / top_k); }

static size_t select_lds_bytes(const DecodeArgs& a) {
  return (size_t)(kHist + 32 + 5 * a.top_k + a.res_words) * sizeof(int);
}

// LSE_g of the pair's G heads from the score workgroups' (max, sum) partials, by
// the NT / 64 waves of the workgroup, head g by wave g mod (NT / 64): one pass,
// each lane folding its blocks into a running (max, sum) with four independent
// 8-byte loads in flight, then across the wave.
template <int G, int NT = kSelThreads>
__device__ __forceinline__ void pair_lse(const DecodeArgs& a, int p, float* lse) {
  const int lane = threadIdx.x & 63;
  for (int w = threadIdx.x >> 6; w < G; w += NT / 64) {
    const float* src = a.lse_part + (int64_t)p * a.nb_score * G * 2;
    float M = kNegBig, S = 0.f;
    for (int k0 = lane; k0 < a.nb_score; k0 += 4 * 64) {
      float2 ms[4];
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const int k = k0 + u * 64;
        ms[u] = k < a.nb_score ? *reinterpret_cast<const float2*>(src + (k * G + w) * 2) : make_float2(kNegBig, 0.f);
      }
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const float Mn = fmaxf(M, ms[u].x);
        S = S * __expf(M - Mn) + ms[u].y * __expf(ms[u].x - Mn);
        M = Mn;
      }
    }
    // fold the lanes: DPP within each row of 16, then the four rows as scalars
    auto fold = [&](float Mo, float So) {
      const float Mn = fmaxf(M, Mo);
      S = S * __expf(M - Mn) + So * __expf(Mo - Mn);
      M = Mn;
    };
    fold(dpp<SKV_DPP_QP_XOR1>(M), dpp<SKV_DPP_QP_XOR1>(S));
    fold(dpp<SKV_DPP_QP_XOR2>(M), dpp<SKV_DPP_QP_XOR2>(S));
    fold(dpp<SKV_DPP_ROW_HALF_MIRROR>(M), dpp<SKV_DPP_ROW_HALF_MIRROR>(S));
    fold(dpp<SKV_DPP_ROW_MIRROR>(M), dpp<SKV_DPP_ROW_MIRROR>(S));
    float Mr[4], Sr[4];
#pragma unroll
    for (int r = 0; r < 4; r++) {
      Mr[r] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(M), 16 * r));
      Sr[r] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(S), 16 * r));
    }
    float Mt = fmaxf(fmaxf(Mr[0], Mr[1]), fmaxf(Mr[2], Mr[3])), St = 0.f;
#pragma unroll
    for (int r = 0; r < 4; r++) St += Sr[r] * __expf(Mr[r] - Mt);
    if (lane == 0) lse[w] = Mt + __logf(St);
  }
}

// Index scan of pair p against the chunks its slots hold, given the selection
// sel[0, K) (ascending candidate indices): chunk ids out, hits / misses, slot
// reassignment, miss list, list of the slots that hit, counters.
template <int NT = kSelThreads>
__device__ void index_scan(const DecodeArgs& a, int p, int* sh, int* sel, int* selch, int* freel, int* missp,
                           int* scl, uint32_t* resl, const uint32_t* selbits = nullptr) {
  const int K = a.top_k, RW = a.res_words;
  int32_t* sc = a.slot_cand + (int64_t)p * K;
  int32_t* sch = a.slot_chunk + (int64_t)p * K;
  uint32_t* res = a.resident + (int64_t)p * RW;
  const int32_t* cmap = a.cand_map + (int64_t)p * a.cand_stride;
  // chunk ids of this thread's selected candidates and of its slots' chunks (the
  // ones they keep if they hit), loaded before the scan and used after it, so
  // that their latency hides behind it; K <= 4 * NT
  constexpr int kPer = 4;
  static_assert(kMaxTopK <= kPer * NT, "selection entries per thread");
  int my_sel[kPer], my_slot[kPer];
  // the running hit / miss totals, read now and written at the end, so the end
  // waits for no load
  long long hits_run = 0, miss_run = 0;
  if (threadIdx.x == 0) {
    hits_run = a.hits_total[p];
    miss_run = a.miss_total[p];
  }
  // after the step the slots hold exactly the selection: with its bitmap at hand
  // the resident bitmap is written now, off the end of the launch
  if (selbits)
    for (int i = threadIdx.x; i < RW; i += NT) res[i] = selbits[i];
#pragma unroll
  for (int j = 0; j < kPer; j++) {
    const int i = threadIdx.x + j * NT;
    if (i < K) {
      my_sel[j] = cmap[sel[i]];
      my_slot[j] = sch[i];
    }
  }
  const bool has_prev = a.temporal && scl[0] >= 0;
  int n_free = 0, n_miss = 0;
#pragma unroll
  for (int j = 0; j < kPer; j++) {
    if (j * NT >= K) break;      // block-uniform
    const int s = j * NT + threadIdx.x;
    int fr = 0, ms = 0;
    if (s < K) {
      const int old = scl[s];
      // is the slot's chunk still selected: the selection's bitmap when the
      // caller built one (one LDS read), else a binary search of sel
      const bool kept = has_prev && old >= 0 &&
                        (selbits ? ((selbits[old >> 5] >> (old & 31)) & 1u) != 0u : sorted_find(sel, K, old) >= 0);
      fr = !kept;
      const int ci = sel[s];
      ms = !(has_prev && ((resl[ci >> 5] >> (ci & 31)) & 1u));
    }
    int tot;
    // closing barrier only where another round of the scan follows (the last
    // round's reads of sh are ordered by the barrier after the loop)
    const int ex = block_exclusive_scan<NT, false>(fr | (ms << 16), sh, &tot);
    if ((j + 1) * NT < K) __syncthreads();   // block-uniform
    if (fr) freel[n_free + (ex & 0xffff)] = s;
    if (ms) missp[n_miss + (ex >> 16)] = s;
    // a slot that keeps its chunk is a hit: listed in ascending slot order, with
    // the chunk id it holds (slot_chunk[s] is the chunk of slot_cand[s])
    if (s < K && !fr) {
      const int64_t hi = (int64_t)p * K + s - n_free - (ex & 0xffff);
      a.hit_slot[hi] = s;
      a.hit_chunk[hi] = my_slot[j];
    }
    n_free += tot & 0xffff;
    n_miss += tot >> 16;
  }
#pragma unroll
  for (int j = 0; j < kPer; j++) {
    const int i = threadIdx.x + j * NT;
    if (i < K) {
      selch[i] = my_sel[j];
      a.chunk_ids[(int64_t)p * K + i] = my_sel[j];
    }
  }
  __syncthreads();
  // n_free == n_miss: every missed chunk takes the next evicted slot.  The miss
  // list is written in full, -1 past n_miss, so its readers need not load n_miss.
  for (int j = threadIdx.x; j < K; j += NT) {
    int slot = -1, ch = -1;
    if (j < n_miss) {
      slot = freel[j];
      const int ci = sel[missp[j]];
      ch = selch[missp[j]];
      if (!selbits) {   // the resident bitmap follows the slots' changes
        const int old = scl[slot];
        if (old >= 0) atomicAnd(&resl[old >> 5], ~(1u << (old & 31)));
        atomicOr(&resl[ci >> 5], 1u << (ci & 31));
      }
      sc[slot] = ci;
      sch[slot] = ch;
    }
    a.miss_slot[(int64_t)p * K + j] = slot;
    a.miss_chunk[(int64_t)p * K + j] = ch;
  }
  if (!selbits) {
    __syncthreads();
    for (int i = threadIdx.x; i < RW; i += NT) res[i] = resl[i];
  }
  if (threadIdx.x == 0) {
    a.n_miss[p] = n_miss;
    a.hits_last[p] = has_prev ? K - n_miss : 0;
    if (has_prev) {
      a.hits_total[p] = hits_run + (K - n_miss);
      a.miss_total[p] = miss_run + n_miss;
    }
  }
}

// Keys of candidates [c0 + PT*t, c0 + PT*t + nv) of pair p for thread t, in
// registers, with the thread's min / max; returns nv.  The G logits of those
// candidates are loaded with 16-byte loads (GB heads in flight at once) before
// the LSE of every head is reduced; `stage` issues the caller's other staging
// work before the barrier, and hist[0, 2048) is cleared in the same window.
// The key is the order-preserving uint32 of score - 1 (score = the log of the
// group max of probabilities, <= 0): in [-1, -30] fp32 values are spaced nearly
// evenly, so the radix select's first 11-bit digit over the key range resolves
// the top of the distribution.  On the score itself a pair with one dominant
// chunk (score 0) stretched the range over every tiny negative value, and its
// selection took three digit passes instead of one (11.5 against 6.3 us).
// The pair's slot map (K entries) and resident bitmap (RW words), read by the
// index scan, copied to LDS in two halves: issue() loads this thread's first
// kSlotRegs entries of each into registers, so that their latency overlaps
// whatever the caller loads next; finish() writes them (and loads and writes any
// further entries) to LDS; a later barrier publishes them.
constexpr int kSlotRegs = 4;   // K <= kMaxTopK = 4 * kSelThreads
struct SlotStage {
  int sc[kSlotRegs];
  uint32_t rs[kSlotRegs];
  __device__ __forceinline__ void issue(const DecodeArgs& a, int p) {
    const int K = a.top_k, RW = a.res_words;
#pragma unroll
    for (int j = 0; j < kSlotRegs; j++) {
      const int i = threadIdx.x + j * kSelThreads;
      sc[j] = i < K ? a.slot_cand[(int64_t)p * K + i] : 0;
      rs[j] = i < RW ? a.resident[(int64_t)p * RW + i] : 0u;
    }
  }
  __device__ __forceinline__ void finish(const DecodeArgs& a, int p, int* scl, uint32_t* resl) const {
    const int K = a.top_k, RW = a.res_words;
#pragma unroll
    for (int j = 0; j < kSlotRegs; j++) {
      const int i = threadIdx.x + j * kSelThreads;
      if (i < K) scl[i] = sc[j];
      if (i < RW) resl[i] = rs[j];
    }
    for (int i = threadIdx.x + kSlotRegs * kSelThreads; i < RW; i += kSelThreads)
      resl[i] = a.resident[(int64_t)p * RW + i];
  }
};
static_assert(kMaxTopK <= kSlotRegs * kSelThreads, "slot map entries per thread");

template <int G, int PT, class Stage>
__device__ __forceinline__ int reg_keys(const DecodeArgs& a, int p, int c0, int n, float* lse, int* hist,
                                        uint32_t (&key)[PT], uint32_t& lo, uint32_t& hi, Stage stage) {
  const int i0 = threadIdx.x * PT;
  const int nv = max(0, min(PT, n - i0));
  const int cb = c0 + i0;                        // a multiple of 4: 16-byte aligned rows
  const float* lg = a.logits + (int64_t)p * G * a.ncp + cb;
  // all heads at once when their logits fit in 64 registers, else groups of 64
  // logits (32 at 16 keys per thread, which hold more registers themselves)
  constexpr int GB = G * PT <= 64 ? G : (PT <= 8 ? 64 : 32) / PT;
  f32x4 lv[GB][PT / 4];
  auto load_heads = [&](int g0) {
#pragma unroll
    for (int gb = 0; gb < GB; gb++)
#pragma unroll
      for (int j = 0; j < PT / 4; j++)
        lv[gb][j] = *reinterpret_cast<const f32x4*>(   // unconditional: entries past nv are unused
            lg + (int64_t)(g0 + gb) * a.ncp + (min(cb + 4 * j, a.ncp - 4) - cb));
  };
  load_heads(0);
  stage();
  for (int i = threadIdx.x; i < 2048; i += kSelThreads) hist[i] = 0;
  pair_lse<G>(a, p, lse);
  __syncthreads();
  float best[PT];
  auto fold_heads = [&](int g0) {
#pragma unroll
    for (int gb = 0; gb < GB; gb++) {
      const float l = lse[g0 + gb];
#pragma unroll
      for (int j = 0; j < PT / 4; j++)
#pragma unroll
        for (int c = 0; c < 4; c++) {
          const float v = lv[gb][j][c] - l;
          best[4 * j + c] = (g0 + gb == 0) ? v : fmaxf(best[4 * j + c], v);
        }
    }
  };
  fold_heads(0);
#pragma unroll 1
  for (int g0 = GB; g0 < G; g0 += GB) {   // one group of heads in registers at a time
    load_heads(g0);
    fold_heads(g0);
  }
  lo = 0xffffffffu;
  hi = 0u;
#pragma unroll
  for (int e = 0; e < PT; e++) {
    key[e] = float_key(best[e] - 1.0f);
    if (e < nv) {
      lo = min(lo, key[e]);
      hi = max(hi, key[e]);
    }
  }
  return nv;
}

template <int G, int PT>
__global__ __launch_bounds__(kSelThreads) void select_kernel(DecodeArgs a) {
  extern __shared__ int smem[];
  const int K = a.top_k, RW = a.res_words;
  int* hist = smem;
  int* sh = smem + kHist;
  int* sel = sh + 32;        // selected candidate indices, ascending
  int* selch = sel + K;      // their chunk ids
  int* freel = selch + K;    // evicted slots, ascending
  int* missp = freel + K;    // positions in sel of the missed chunks, ascending
  int* scl = missp + K;      // slot -> candidate index (copy of the pair's slot map)
  uint32_t* resl = reinterpret_cast<uint32_t*>(scl + K);   // resident bitmap copy
  __shared__ float lse[16];
  const int p = blockIdx.x;
  uint32_t key[PT], lo, hi;
  int nv;
  if constexpr (G * PT <= 64) {
    SlotStage ss;   // loads issued beside the logits', stored to LDS after the LSE
    nv = reg_keys<G, PT>(a, p, 0, a.n_cand, lse, hist, key, lo, hi, [&] { ss.issue(a, p); });
    ss.finish(a, p, scl, resl);   // published by the barriers below
  } else {          // the logits fill the registers: load and store in place
    nv = reg_keys<G, PT>(a, p, 0, a.n_cand, lse, hist, key, lo, hi, [&] {
      for (int i = threadIdx.x; i < K; i += kSelThreads) scl[i] = a.slot_cand[(int64_t)p * K + i];
      for (int i = threadIdx.x; i < RW; i += kSelThreads) resl[i] = a.resident[(int64_t)p * RW + i];
    });
  }
  block_range<kSelThreads>(lo, hi, sh);
  const int i0 = threadIdx.x * PT;
  block_topk_reg<kSelThreads, PT>(key, prefix_mask(nv), K, lo, hi, hist, sh, true,
                                  [&](int pos, int e) { sel[pos] = i0 + e; });
  index_scan(a, p, sh, sel, selch, freel, missp, scl, resl);
}

template <int G, int PT>
__global__ __launch_bounds__(kSelThreads) void part_topk_kernel(DecodeArgs a) {
  extern __shared__ int smem[];
  int* hist = smem;
  int* sh = smem + kHist;
  __shared__ float lse[16];
  const int part = blockIdx.x, p = blockIdx.y;
  const int K = a.top_k;
  const int c0 = part * a.part_size, n = min(a.part_size, a.n_cand - c0);
  uint32_t key[PT], lo, hi;
  const int nv = reg_keys<G, PT>(a, p, c0, n, lse, hist, key, lo, hi, [] {});
  block_range<kSelThreads>(lo, hi, sh);
  uint32_t* ok = a.part_keys + ((int64_t)p * a.n_part + part) * K;
  int32_t* oi = a.part_idx + ((int64_t)p * a.n_part + part) * K;
  const int ci = c0 + threadIdx.x * PT;
  block_topk_reg<kSelThreads, PT>(key, prefix_mask(nv), min(K, n), lo, hi, hist, sh, true, [&](int pos, int e) {
    ok[pos] = key[e];
    oi[pos] = ci + e;
  });
}

// Lists of (key, candidate index) per pair, each in ascending candidate order and
// covering consecutive candidate ranges in list order: list j of pair p starts at
// element p * pair_stride + j * K; every list but the last holds len0 entries, all
// lists of a pair m entries.  Entry i of a pair is entry i % len0 of list i / len0.
struct ListSet {
  const uint32_t* keys;
  const int32_t* idx;
  int64_t pair_stride;
  int len0, n_lists, m;
};

// Entries [e0, e0 + n) of pair p's lists, thread t holding [e0 + t*PT, e0 + t*PT + PT)
// in registers (n <= kSelThreads * PT; entries past n re-read entry n - 1 and are
// not counted), with the thread's key range; returns the thread's count.
template <int PT>
__device__ __forceinline__ int load_entries(const ListSet& ls, int K, int p, int e0, int n, uint32_t (&key)[PT],
                                            int (&idx)[PT], uint32_t& lo, uint32_t& hi) {
  const int i0 = threadIdx.x * PT, nv = max(0, min(PT, n - i0));
  const uint32_t* gk = ls.keys + (int64_t)p * ls.pair_stride;
  const int32_t* gi = ls.idx + (int64_t)p * ls.pair_stride;
  if (ls.len0 % PT == 0 && K % 4 == 0 && e0 % PT == 0 && nv == PT) {
    // the PT entries lie in one list, 16-byte aligned: PT / 4 loads of each
    const int i = e0 + i0, off = (i / ls.len0) * K + i % ls.len0;
#pragma unroll
    for (int j = 0; j < PT / 4; j++) {
      const u32x4 kw = *reinterpret_cast<const u32x4*>(gk + off + 4 * j);
      const u32x4 iw = *reinterpret_cast<const u32x4*>(gi + off + 4 * j);
#pragma unroll
      for (int c = 0; c < 4; c++) {
        key[4 * j + c] = kw[c];
        idx[4 * j + c] = (int)iw[c];
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < PT; e++) {
      const int i = e0 + min(i0 + e, n - 1);
      const int off = (i / ls.len0) * K + i % ls.len0;
      key[e] = gk[off];
      idx[e] = gi[off];
    }
  }
  lo = 0xffffffffu;
  hi = 0u;
#pragma unroll
  for (int e = 0; e < PT; e++) {
    if (e < nv) {
      lo = min(lo, key[e]);
      hi = max(hi, key[e]);
    }
  }
  return nv;
}

// One level of the merge tree: workgroup (gi, p) takes lists [gi*grp, gi*grp + grp)
// of pair p and writes their top-K (in ascending candidate order, so ties still
// go to the lower candidate) as list gi of `out` (pair stride out_stride).  The
// pair's top-K is contained in the union of the groups' top-K.
__global__ __launch_bounds__(kSelThreads) void merge_level_kernel(DecodeArgs a, ListSet ls, int grp,
                                                                  uint32_t* out_keys, int32_t* out_idx,
                                                                  int64_t out_stride) {
  __shared__ int hist[kHist];
  __shared__ int sh[32];
  constexpr int PT = 16;
  const int gi = blockIdx.x, p = blockIdx.y, K = a.top_k;
  const int e0 = gi * grp * ls.len0, n = min(ls.m - e0, grp * ls.len0);
  uint32_t key[PT], lo, hi;
  int idx[PT];
  const int nv = load_entries<PT>(ls, K, p, e0, n, key, idx, lo, hi);
  for (int i = threadIdx.x; i < 2048; i += kSelThreads) hist[i] = 0;
  block_range<kSelThreads>(lo, hi, sh);   // its barriers also publish the cleared histogram
  uint32_t* ok = out_keys + (int64_t)p * out_stride + (int64_t)gi * K;
  int32_t* oi = out_idx + (int64_t)p * out_stride + (int64_t)gi * K;
  block_topk_reg<kSelThreads, PT>(key, prefix_mask(nv), min(K, n), lo, hi, hist, sh, true, [&](int pos, int e) {
    ok[pos] = key[e];
    oi[pos] = idx[e];
  });
}

// Last level: the top-K of all of pair p's lists (at most kSelThreads * 16 entries,
// in registers), then the temporal-cache index scan.
__global__ __launch_bounds__(kSelThreads) void merged_select_kernel(DecodeArgs a, ListSet ls) {
  extern __shared__ int smem[];
  constexpr int PT = 16;
  const int K = a.top_k, RW = a.res_words;
  int* hist = smem;
  int* sh = smem + kHist;
  int* sel = sh + 32;
  int* selch = sel + K;
  int* freel = selch + K;
  int* missp = freel + K;
  int* scl = missp + K;
  uint32_t* resl = reinterpret_cast<uint32_t*>(scl + K);
  const int p = blockIdx.x;
  uint32_t key[PT], lo, hi;
  int idx[PT];
  SlotStage ss;   // loads issued before the lists', stored to LDS after them
  ss.issue(a, p);
  const int nv = load_entries<PT>(ls, K, p, 0, ls.m, key, idx, lo, hi);
  ss.finish(a, p, scl, resl);
  for (int i = threadIdx.x; i < 2048; i += kSelThreads) hist[i] = 0;
  block_range<kSelThreads>(lo, hi, sh);   // its barriers also publish the cleared histogram
  block_topk_reg<kSelThreads, PT>(key, prefix_mask(nv), K, lo, hi, hist, sh, true, [&](int pos, int e) { sel[pos] = idx[e]; });
  index_scan(a, p, sh, sel, selch, freel, missp, scl, resl);
}

template <class F>
static hipError_t allow_lds(F* kernel) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                             kSelLdsMax);
}

// ---------------------------------------------------------------------------
// Two-level selection, one workgroup per pair.  The key of a 16-candidate tile
// is the largest key in it, and it follows from the score kernel's per-tile
// maxima of each head's logits: max_g(M_g - LSE_g) is the same fp32 arithmetic
// as each candidate's max_g(l_g - LSE_g) applied to the tile's largest logits,
// and every later step (- 1, the order-preserving map) is monotone.
//  1. beta = a lower bound of the K-th largest tile key (the lower edge of its
//     radix bucket).  At least K tiles hold a candidate whose key is >= beta,
//     so the pair's K-th largest key is >= beta: every selected candidate has
//     key >= beta and lies in a tile whose key is >= beta ("hot").
//  2. The candidates of the hot tiles (4 per item, items in ascending candidate
//     order) form the keys; those below beta are left out, which changes
//     nothing, since every candidate left out is smaller than every selected one
//     (ties included).  The top-K among them is the pair's top-K, with ties to
//     the lower candidate index as over all candidates.
// With K above the tile count every tile is hot and no key is left out.  The
// tile maxima of a pair are about 1/16 of its logits and the hot tiles' logits
// about K/n_tiles of them, so the selection reads a small fraction of what a
// full pass over the logits reads (at the Llama-3.1-8B shape 15 KB + 61 KB of
// 245 KB per pair; about 400 keys pass beta).  If the hot tiles outnumber the
// register budget (IPT items of 4 candidates per thread; only with many equal
// tile keys), the second level runs over them from memory instead.
// LDS layout (ints): hist[2048 + kTopkSmall] | sh[32] | sel[K] | selch[K] |
// freel[K] | missp[K] | scl[K] | resl[res_words] | hot tile list[n_ctiles] |
// selbits[res_words] (the selection as a bitmap over candidate indices, for the
// index scan's "is the slot's chunk still selected").

// key of candidate c (< n_cand) of pair p from its G logits
template <int G>
__device__ __forceinline__ uint32_t cand_key(const DecodeArgs& a, int p, int c, const float* lse) {
  const float* lg = a.logits + (int64_t)p * G * a.ncp + c;
  float best = lg[0] - lse[0];
#pragma unroll
  for (int g = 1; g < G; g++) best = fmaxf(best, lg[(int64_t)g * a.ncp] - lse[g]);
  return float_key(best - 1.0f);
}

template <int G, int C>
__device__ void attend_static(const DecodeArgs& a, int p, int s, float* lds);

// Workgroups P .. P + P * n_static - 1 of the launch attend to the units that do
// not depend on the selection (attend_static), on CUs the selection leaves idle.
template <int G, int NT, int TPT, int IPT>
__global__ __launch_bounds__(NT) void select2_kernel(DecodeArgs a) {
  extern __shared__ int smem[];
  if ((int)blockIdx.x >= a.batch * a.n_kv) {   // workgroup-uniform
    static_assert(NT == kStaticWaves * 64, "one wave per static attention wave");
    const int P = a.batch * a.n_kv, x = blockIdx.x - P;
    float* lds = reinterpret_cast<float*>(smem);
    switch (a.chunk) {
      case 4: attend_static<G, 4>(a, x % P, x / P, lds); break;
      case 8: attend_static<G, 8>(a, x % P, x / P, lds); break;
      default: attend_static<G, 16>(a, x % P, x / P, lds); break;
    }
    return;
  }
  const int K = a.top_k, RW = a.res_words, n_tiles = a.n_ctiles, n = a.n_cand;
  int* hist = smem;
  int* sh = smem + kHist;
  int* sel = sh + 32;        // selected candidate indices, ascending
  int* selch = sel + K;      // their chunk ids
  int* freel = selch + K;    // evicted slots, ascending
  int* missp = freel + K;    // positions in sel of the missed chunks, ascending
  int* scl = missp + K;      // slot -> candidate index (copy of the pair's slot map)
  uint32_t* resl = reinterpret_cast<uint32_t*>(scl + K);   // resident bitmap copy
  int* hot = reinterpret_cast<int*>(resl + RW);            // hot tiles, ascending
  uint32_t* selbits = reinterpret_cast<uint32_t*>(hot + a.n_ctiles_cap);   // the selection as a bitmap
  __shared__ float lse[16];
  const int p = blockIdx.x;
  // ---- level 1: tile keys of tiles [t*TPT, t*TPT + TPT); their maxima are
  // loaded before the LSE is reduced when they fit in 32 registers, else after
  const int t0 = threadIdx.x * TPT;
  const int ntv = max(0, min(TPT, n_tiles - t0));   // this thread's tiles
  const float* tm = a.tile_max + (int64_t)p * n_tiles * G;
  constexpr bool kPrefetch = TPT * G <= 32;
  float mg[kPrefetch ? TPT : 1][G];
  auto load_tile = [&](int e, float (&m)[G]) {
    const int tile = min(t0 + e, n_tiles - 1);   // past the tiles: re-read the last, not counted
    if constexpr (G % 4 == 0) {
#pragma unroll
      for (int g = 0; g < G; g += 4) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(tm + (int64_t)tile * G + g);
#pragma unroll
        for (int j = 0; j < 4; j++) m[g + j] = v[j];
      }
    } else {
#pragma unroll
      for (int g = 0; g < G; g++) m[g] = tm[(int64_t)tile * G + g];
    }
  };
  if constexpr (kPrefetch) {
#pragma unroll
    for (int e = 0; e < TPT; e++) load_tile(e, mg[e]);
  }
  // the slot map and the resident bitmap (read by the index scan) are loaded
  // now and written to LDS after the LSE, so their latency overlaps the LSE
  // partials' (the first NT entries through registers)
  const int32_t* sc = a.slot_cand + (int64_t)p * K;
  const uint32_t* res = a.resident + (int64_t)p * RW;
  const int i0 = threadIdx.x;
  const int sc0 = i0 < K ? sc[i0] : 0;
  const uint32_t rs0 = i0 < RW ? res[i0] : 0u;
  for (int i = threadIdx.x; i < 2048; i += NT) hist[i] = 0;
  pair_lse<G, NT>(a, p, lse);
  if (i0 < K) scl[i0] = sc0;
  if (i0 < RW) resl[i0] = rs0;
  for (int i = i0 + NT; i < K; i += NT) scl[i] = sc[i];
  for (int i = i0 + NT; i < RW; i += NT) resl[i] = res[i];
  __syncthreads();
  uint32_t tk[TPT];
  uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
  for (int e = 0; e < TPT; e++) {
    float m1[G];
    if constexpr (kPrefetch) {
#pragma unroll
      for (int g = 0; g < G; g++) m1[g] = mg[e][g];
    } else {
      load_tile(e, m1);
    }
    float best = m1[0] - lse[0];
#pragma unroll
    for (int g = 1; g < G; g++) best = fmaxf(best, m1[g] - lse[g]);
    tk[e] = float_key(best - 1.0f);
    if (e < ntv) {
      lo = min(lo, tk[e]);
      hi = max(hi, tk[e]);
    }
  }
  // (no barrier before: nothing has touched sh yet; none after: the selection's
  // histogram barrier, or the one below, comes before the next write to sh)
  block_range<NT, false, false>(lo, hi, sh);
  const uint32_t hi1 = hi;   // the pair's largest key
  uint32_t beta = 0u;   // every key passes when K exceeds the tile count
  if (K <= n_tiles) {   // block-uniform
    int kk;
    // lean: its last reads of sh[0, 16) and of hist precede a barrier inside; the
    // hot-tile scan below writes only sh[0, 16), and hist after a barrier.
    // beta need only be a lower bound of the K-th largest tile key (a lower one
    // adds hot tiles, never drops a selected chunk): the edge of the first digit
    // pass's boundary bucket, without the passes that would pin it exactly
    beta = block_kth_reg<NT, TPT, true, true>(tk, prefix_mask(ntv), K, lo, hi, hist, sh, true, &kk);
  } else {
    __syncthreads();
  }
  // hot tiles, compacted in ascending order
  int nh = 0;
#pragma unroll
  for (int e = 0; e < TPT; e++) nh += (e < ntv && tk[e] >= beta);
  int n_hot;
  // (no closing barrier: the one after the histogram clear below comes first)
  int off = block_exclusive_scan<NT, false>(nh, sh, &n_hot);
#pragma unroll
  for (int e = 0; e < TPT; e++)
    if (e < ntv && tk[e] >= beta) hot[off++] = t0 + e;
  for (int i = threadIdx.x; i < 2048; i += NT) hist[i] = 0;
  for (int i = threadIdx.x; i < RW; i += NT) selbits[i] = 0u;
  __syncthreads();
  // ---- level 2: the candidates of the hot tiles, items of 4 candidates
  const int n_items = n_hot * 4;
  if (n_items <= NT * IPT) {
    const int i0 = threadIdx.x * IPT;
    uint32_t key[IPT * 4];
    int cbs[IPT];   // first candidate of each item (kept for the emission)
    uint64_t vmask = 0;
#pragma unroll
    for (int it = 0; it < IPT; it++) {
      const int item = min(i0 + it, n_items - 1);
      const int cb = hot[item >> 2] * 16 + (item & 3) * 4;
      cbs[it] = cb;
      const int cl = min(cb, a.ncp - 4);     // past the candidates: re-read the last row's end, not counted
      // the G heads in groups of (at most) 4 loads
      constexpr int GB = G < 4 ? G : 4;
      float best[4];
#pragma unroll
      for (int g0 = 0; g0 < G; g0 += GB) {
        f32x4 lv[GB];
#pragma unroll
        for (int g = 0; g < GB; g++)
          lv[g] = *reinterpret_cast<const f32x4*>(a.logits + ((int64_t)p * G + g0 + g) * a.ncp + cl);
#pragma unroll
        for (int g = 0; g < GB; g++)
#pragma unroll
          for (int c = 0; c < 4; c++) {
            const float v = lv[g][c] - lse[g0 + g];
            best[c] = (g0 + g == 0) ? v : fmaxf(best[c], v);
          }
      }
#pragma unroll
      for (int c = 0; c < 4; c++) {
        const uint32_t kv = float_key(best[c] - 1.0f);
        key[it * 4 + c] = kv;
        if (i0 + it < n_items && cb + c < n && kv >= beta) vmask |= 1ull << (it * 4 + c);
      }
    }
    // the keys that pass lie in [beta, the largest tile key]; a version that
    // ranked each passing key against all others (one per thread, from LDS)
    // took 18.7 us per pair at the Llama-3.1-8B shape against 3.6 us for this.
    // Loading the hot candidates' chunk ids here (so that the index scan need
    // not look up the selected ones) made the launch slower, 18.9 against 16.8 us.
    // lean: it ends with the barrier that publishes sel, before the index scan
    // writes sh again
    block_topk_reg<NT, IPT * 4, true>(key, vmask, K, beta, hi1, hist, sh, true, [&](int pos, int e) {
      const int c = cbs[e / 4] + (e & 3);
      sel[pos] = c;
      atomicOr(&selbits[c >> 5], 1u << (c & 31));
    });
  } else {
    // many equal tile keys: the hot tiles' candidates from memory (candidates
    // past n_cand get key 0, below every real key, and are never taken)
    const int m = n_hot * 16;
    block_topk<NT>(
        [&](int i) {
          const int c = hot[i >> 4] * 16 + (i & 15);
          return c < n ? cand_key<G>(a, p, c, lse) : 0u;
        },
        m, K, hist, sh, [&](int pos, int i) {
          const int c = hot[i >> 4] * 16 + (i & 15);
          sel[pos] = c;
          atomicOr(&selbits[c >> 5], 1u << (c & 31));
        });
  }
  index_scan<NT>(a, p, sh, sel, selch, freel, missp, scl, resl, selbits);
}

static size_t select2_lds_bytes(const DecodeArgs& a) {
  return (size_t)(kHist + 32 + 5 * a.top_k + 2 * a.res_words + a.n_ctiles_cap) * sizeof(int);
}

// LDS of a static attention workgroup: every wave's o[G][d], m[G] and l[G]
static size_t static_lds_bytes(int G) { return (size_t)kStaticWaves * G * (kHeadDim + 2) * sizeof(float); }

// Workgroup size, tiles and level-2 items per thread of the two-level selection,
// or 0 when it does not apply (a budget above kSelect2MaxTopK, more tiles per
// thread than 16, or LDS that would not fit).  1024 threads: 256 (one wave per
// SIMD) made every block-wide step cheaper but the per-thread loops longer, 20.8
// against 15.2 us per pair at the Llama-3.1-8B shape (phase stamps).  The budget
// bound: one workgroup per pair takes about 5 K hot candidates through level 2,
// which at K = 1024 and 2048 (few pairs, long contexts) was three times slower
// than the selection in parts over all candidates (182 against 60 us per layer
// at the GLM-4-9B-1M shape); at K = 240 and 400 it was faster (17 against 20,
// 22 against 27 us).
constexpr int kSelect2MaxTopK = 512;

int select2_shape(int n_ctiles_cap, int top_k, int res_words, int* nt, int* tpt, int* ipt) {
  if (top_k > kSelect2MaxTopK) return 0;
  if ((size_t)(kHist + 32 + 5 * top_k + 2 * res_words + n_ctiles_cap) * sizeof(int) > (size_t)kSelLdsMax) return 0;
  const int threads = kSelThreads;
  const int t = (n_ctiles_cap + threads - 1) / threads;
  // hot tiles are about K (more only on equal tile keys): room for 1.25 K, 4
  // candidates per item, at most 4 items per thread (K <= 512)
  const int need = (5 * top_k + threads - 1) / threads;
  if (t > 16 || need > 4) return 0;
  *nt = threads;
  *tpt = t <= 1 ? 1 : t <= 2 ? 2 : t <= 4 ? 4 : t <= 8 ? 8 : 16;
  *ipt = need <= 1 ? 1 : need <= 2 ? 2 : 4;
  return 1;
}

template <int G, int NT, int TPT, int IPT>
static hipError_t launch_select2_i(const DecodeArgs& a, hipStream_t st) {
  static bool attr = false;
  if (!attr) {
    hipError_t e = allow_lds(&select2_kernel<G, NT, TPT, IPT>);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const size_t lds = std::max(select2_lds_bytes(a), a.n_static > 0 ? static_lds_bytes(G) : (size_t)0);
  select2_kernel<G, NT, TPT, IPT><<<a.batch * a.n_kv * (1 + a.n_static), NT, lds, st>>>(a);
  return hipGetLastError();
}

template <int G, int NT, int TPT>
static hipError_t launch_select2_t(const DecodeArgs& a, hipStream_t st) {
  switch (a.sel_ipt) {
    case 1: return launch_select2_i<G, NT, TPT, 1>(a, st);
    case 2: return launch_select2_i<G, NT, TPT, 2>(a, st);
    default: return launch_select2_i<G, NT, TPT, 4>(a, st);
  }
}

template <int G, int NT>
static hipError_t launch_select2_n(const DecodeArgs& a, hipStream_t st) {
  switch (a.sel_tpt) {
    case 1: return launch_select2_t<G, NT, 1>(a, st);
    case 2: return launch_select2_t<G, NT, 2>(a, st);
    case 4: return launch_select2_t<G, NT, 4>(a, st);
    case 8: return launch_select2_t<G, NT, 8>(a, st);
    default: return launch_select2_t<G, NT, 16>(a, st);
  }
}

template <int G>
static hipError_t launch_select2_g(const DecodeArgs& a, hipStream_t st) {
  return launch_select2_n<G, kSelThreads>(a, st);
}

template <int G, int PT>
static hipError_t launch_select_pt(const DecodeArgs& a, hipStream_t st) {
  const int P = a.batch * a.n_kv, K = a.top_k;
  static bool attr = false;
  if (!attr) {
    hipError_t e = allow_lds(&select_kernel<G, PT>);
    if (e == hipSuccess) e = allow_lds(&merged_select_kernel);
    if (e != hipSuccess) return e;
    attr = true;
  }
  if (a.n_part == 1) {
    select_kernel<G, PT><<<P, kSelThreads, select_lds_bytes(a), st>>>(a);
    return hipGetLastError();
  }
  part_topk_kernel<G, PT><<<dim3(a.n_part, P), kSelThreads, (kHist + 32) * sizeof(int), st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // merge tree: the part lists, then each level's lists alternately in the merge
  // buffers and back in the part buffers, until one workgroup holds them all
  const int len0 = std::min(K, a.part_size);
  ListSet ls{a.part_keys, a.part_idx, (int64_t)a.n_part * K, len0, a.n_part,
             (a.n_part - 1) * len0 + std::min(K, a.n_cand - (a.n_part - 1) * a.part_size)};
  const int grp = merge_groups(K);
  bool to_merge = true;
  while (ls.n_lists > grp) {
    const int n_out = (ls.n_lists + grp - 1) / grp;
    uint32_t* ok = to_merge ? a.merge_keys : a.part_keys;
    int32_t* oi = to_merge ? a.merge_idx : a.part_idx;
    const int64_t out_stride = (int64_t)n_out * K;
    merge_level_kernel<<<dim3(n_out, P), kSelThreads, 0, st>>>(a, ls, grp, ok, oi, out_stride);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int last = ls.m - (n_out - 1) * grp * ls.len0;   // entries of the last group
    ls = ListSet{ok, oi, out_stride, K, n_out, (n_out - 1) * K + std::min(K, last)};
    to_merge = !to_merge;
  }
  merged_select_kernel<<<P, kSelThreads, select_lds_bytes(a), st>>>(a, ls);
  return hipGetLastError();
}

template <int G>
static hipError_t launch_select_g(const DecodeArgs& a, hipStream_t st) {
  switch (keys_per_thread(a.part_size)) {
    case 4: return launch_select_pt<G, 4>(a, st);
    case 8: return launch_select_pt<G, 8>(a, st);
    default: return launch_select_pt<G, 16>(a, st);
  }
}

hipError_t launch_select(const DecodeArgs& a, hipStream_t st) {
  if (a.sel_two_level) {
    switch (a.group) {
      case 1: return launch_select2_g<1>(a, st);
      case 2: return launch_select2_g<2>(a, st);
      case 4: return launch_select2_g<4>(a, st);
      case 8: return launch_select2_g<8>(a, st);
      case 16: return launch_select2_g<16>(a, st);
      default: return hipErrorInvalidValue;
    }
  }
  switch (a.group) {
    case 1: return launch_select_g<1>(a, st);
    case 2: return launch_select_g<2>(a, st);
    case 4: return launch_select_g<4>(a, st);
    case 8: return launch_select_g<8>(a, st);
    case 16: return launch_select_g<16>(a, st);
    default: return hipErrorInvalidValue;
  }
}

// ---------------------------------------------------------------------------
// Key rebuild: 128 rows (MPB = 128/C missed chunks) per workgroup, 4 waves x 32
// rows, N = d = 128 as 8 MFMA column tiles, k in steps of 32.  Every k-step is
// one load group per wave (two direct global->LDS loads of B^T, two A-row
// fragment loads), all groups issued up front; the MFMAs of step q start as soon
// as groups 0..q have landed, while the later groups are still in flight.

constexpr int kMaxSteps = 5;                  // k-steps per staged slice (160 k)
constexpr int kOutW = kHeadDim + 8;           // staged output row pitch (bf16)
constexpr int kStepPieces = kRebuildRows * 4; // 16-byte pieces of B^T per k-step

// Piece c (0..3) of B^T row n within a k-step: XOR-swizzled so that the 16 rows
// one MFMA operand read touches fall in 16 distinct LDS bank groups.
__device__ __forceinline__ int bt_slot(int n, int c) { return n * 4 + (c ^ ((n >> 2) & 3)); }

// s_waitcnt immediate: vector-memory count n, other counters left alone (gfx9 layout)
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Wait until at most g load groups of 4 vector-memory instructions are outstanding
// (g is a constant once the k-step loop is unrolled).
__device__ __forceinline__ void wait_load_groups(int g) {
  switch (g) {
    case 0: __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); break;
    case 1: __builtin_amdgcn_s_waitcnt(vmcnt_imm(4)); break;
    case 2: __builtin_amdgcn_s_waitcnt(vmcnt_imm(8)); break;
    case 3: __builtin_amdgcn_s_waitcnt(vmcnt_imm(12)); break;
    case 4: __builtin_amdgcn_s_waitcnt(vmcnt_imm(16)); break;
    default: __builtin_amdgcn_s_waitcnt(vmcnt_imm(20)); break;
  }
}

// Four B^T operand pieces (column tiles H*4 .. H*4+3) of k-step Q, read from LDS
// in one asm block that ends with lgkmcnt(0), so the values exist only once they
// have arrived.  A read the compiler can see would make it wait for every direct
// global->LDS load still in flight (all k-steps at once); this one is ordered by
// the explicit waits and barrier in mfma_steps.
template <int Q, int H>
__device__ __forceinline__ void stage_reads(uint32_t addr, u32x4 (&bw)[4]) {
  constexpr int T = 16 * 4 * 16;                              // column-tile stride
  constexpr int O = Q * kStepPieces * 16 + H * 4 * T;         // step and half offset
  asm volatile(
      "ds_read_b128 %0, %4 offset:%5\n"
      "ds_read_b128 %1, %4 offset:%6\n"
      "ds_read_b128 %2, %4 offset:%7\n"
      "ds_read_b128 %3, %4 offset:%8\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(bw[0]), "=&v"(bw[1]), "=&v"(bw[2]), "=&v"(bw[3])
      : "v"(addr), "i"(O), "i"(O + T), "i"(O + 2 * T), "i"(O + 3 * T));
}

// 8 FP8 E5M2 values (bytes of lo, then hi) -> 8 bf16, exactly: the byte is the
// high byte of the equal fp16, widened to fp32 and cut to its high half.
__device__ __forceinline__ u32x4 e5m2x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  const u32x4 h = e5m2x8_to_f16x8(lo, hi);
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const float f0 = (float)__builtin_bit_cast(_Float16, (uint16_t)(h[i] & 0xffffu));
    const float f1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(h[i] >> 16));
    o[i] = (__float_as_uint(f0) >> 16) | (__float_as_uint(f1) & 0xffff0000u);
  }
  return o;
}

// An A fragment as the MFMA takes it: 8 bf16 as loaded, or widened from 8 FP8
// bytes.  The empty volatile asm pins the widening after the explicit load waits
// (without it the compiler hoists it next to the loads and waits for all of them).
__device__ __forceinline__ u32x4 a_operand(const u32x4& v) { return v; }
__device__ __forceinline__ u32x4 a_operand(const uint2& v) {
  uint32_t lo = v.x, hi = v.y;
  asm volatile("" : "+v"(lo), "+v"(hi));
  return e5m2x8_to_bf16x8(lo, hi);
}

template <int Q, int H, class AF>
__device__ __forceinline__ void mfma_half(const AF (&a)[2], bool kin, uint32_t baddr, f32x4 (&acc)[2][8]) {
  u32x4 bw[4];
  stage_reads<Q, H>(baddr, bw);
  u32x4 av[2];
#pragma unroll
  for (int mt = 0; mt < 2; mt++) av[mt] = a_operand(a[mt]);
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const bf16x8 bfr = __builtin_bit_cast(bf16x8, kin ? bw[i] : (u32x4){0u, 0u, 0u, 0u});
#pragma unroll
    for (int mt = 0; mt < 2; mt++)
      acc[mt][H * 4 + i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av[mt]), bfr,
                                                                   acc[mt][H * 4 + i], 0, 0, 0);
  }
}

// k-step Q of a slice: wait for load groups 0..Q of every wave, then 16 MFMAs.
// A fragments are used as loaded (rows past the misses hold finite data and are
// never stored); B^T pieces past kn are zeroed, which cancels the k-padding.
template <int NSTEP, int Q, class AF>
__device__ __forceinline__ void mfma_steps(const AF (&af)[NSTEP][2], int kn, int lk, uint32_t baddr,
                                           f32x4 (&acc)[2][8]) {
  __builtin_amdgcn_sched_barrier(0);             // step Q-1's MFMAs stay ahead of this wait
  wait_load_groups(NSTEP - 1 - Q);               // this wave's groups 0..Q have landed
  __builtin_amdgcn_s_barrier();                  // ... and every other wave's
  __builtin_amdgcn_sched_barrier(0);             // nothing that reads them moves above the waits
  const bool kin = Q * 32 + lk * 8 < kn;
  mfma_half<Q, 0>(af[Q], kin, baddr, acc);
  mfma_half<Q, 1>(af[Q], kin, baddr, acc);
  if constexpr (Q + 1 < NSTEP) mfma_steps<NSTEP, Q + 1, AF>(af, kn, lk, baddr, acc);
}

// Staging buffer of one rebuild tile: B^T pieces of NSTEP k-steps, later the
// tile's bf16 output rows.
template <int NSTEP>
constexpr int rebuild_stage_bytes() {
  return NSTEP * kStepPieces * 16 > kRebuildRows * kOutW * 2 ? NSTEP * kStepPieces * 16 : kRebuildRows * kOutW * 2;
}

// One tile of kRebuildRows rows of pair p: the keys of the missed chunks
// mchunk[0, 128/C) (-1: none), rotated and rounded to bf16, left in `stage` as
// rows of kOutW bf16 (row m = token m % C of miss m / C); store_tile writes them
// into their slots.  Called by all 256 threads of a workgroup with mchunk in LDS
// (written before a barrier) and `stage` an LDS buffer of
// rebuild_stage_bytes<NSTEP>(); returns after a barrier, with the rows in place.
// With `park` (an LDS buffer of kParkFloats floats), the RoPE angles are parked
// there across the MFMAs instead of held in 12 registers per lane (the fused
// tail's attention state otherwise costs it its single k-step slice).
// A8: rows of A stored as FP8 E5M2 (r bytes per row) instead of bf16, widened to
// bf16 exactly after the loads.  B^T is always read from its bf16 stage-order copy
// (with B stored as FP8 E5M2, the build widens it into that copy exactly, so the
// MFMA inputs are the FP8 values either way).
constexpr int kParkFloats = 12 * 256;

template <int C, int NSTEP, bool A8, bool PARK = false>
__device__ __forceinline__ void rebuild_tile(const DecodeArgs& a, int p, const int* mchunk, u32x4* stage,
                                             float* park = nullptr) {
  const int b = p / a.n_kv;
  const int r = a.rank;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int lr = lane & 15, lk = lane >> 4;
  double ffreq[4];
#pragma unroll
  for (int nt = 0; nt < 4; nt++) ffreq[nt] = a.inv_freq[nt * 16 + lr];
  const int r_pad = a.n_kq * 32;
  // A operand rows of this lane: row m = w*32 + mt*16 + lr, element offset of its
  // k-step 0 in the chunk-tiled A (k-step q adds q * C * 32); rows past the
  // misses read chunk 0 of the batch element, their outputs not stored
  int64_t arow[2];
  int64_t pos0[2];   // position of this lane's first output row of each tile
#pragma unroll
  for (int mt = 0; mt < 2; mt++) {
    const int m = w * 32 + mt * 16 + lr;
    const int ch = mchunk[m / C];
    arow[mt] = a_tiled(b, a.a_rows, r_pad, C, (int64_t)max(ch, 0) * C + (m % C), 0);
    const int m0 = w * 32 + mt * 16 + lk * 4;
    pos0[mt] = (int64_t)max(mchunk[m0 / C], 0) * C + (m0 % C);
  }
  // LDS byte address of this lane's B^T operand piece in k-step 0, column tile 0:
  // row lr, piece lk swizzled; the swizzle depends on lr only, so every (step,
  // column tile) is a constant offset from it.
  const uint32_t baddr = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) u32x4*)stage +
                         (uint32_t)bt_slot(lr, lk) * 16u;
  // RoPE angles: a lane's four output rows lk*4 .. lk*4+3 of a tile are
  // consecutive positions of one chunk, so the float64 reduction runs once per
  // (tile, column) and the rows add j * f.
  float ang[2][4], ff[4];
#pragma unroll
  for (int nt = 0; nt < 4; nt++) {
    ff[nt] = (float)ffreq[nt];
#pragma unroll
    for (int mt = 0; mt < 2; mt++) ang[mt][nt] = rope_angle(pos0[mt], ffreq[nt]);
  }
  if constexpr (PARK) {
#pragma unroll
    for (int nt = 0; nt < 4; nt++) {
      park[nt * 256 + threadIdx.x] = ff[nt];
#pragma unroll
      for (int mt = 0; mt < 2; mt++) park[(4 + mt * 4 + nt) * 256 + threadIdx.x] = ang[mt][nt];
    }
  }
  f32x4 acc[2][8];
#pragma unroll
  for (int mt = 0; mt < 2; mt++)
#pragma unroll
    for (int nt = 0; nt < 8; nt++) acc[mt][nt] = (f32x4){0.f, 0.f, 0.f, 0.f};

  for (int ks = 0; ks < r; ks += NSTEP * 32) {
    const int kn = min(NSTEP * 32, r - ks);
    if (ks > 0) __syncthreads();                 // previous slice fully consumed
    using AFrag = typename std::conditional<A8, uint2, u32x4>::type;
    AFrag af[NSTEP][2];
#pragma unroll
    for (int q = 0; q < NSTEP; q++) {
#pragma unroll
      for (int u = 0; u < 2; u++) {
        const int i = w * 2 + u;                 // instruction 0..7 of the step
        const int e = i * 64 + lane;
        // B^T pre-arranged in stage order (the pieces already swizzled, zero past
        // r): one contiguous 1 KB per instruction; a k-step past the rank (the
        // last slice of a split contraction) re-reads the last one, masked below
        const int qg = min(ks / 32 + q, a.n_kq - 1);
        __builtin_amdgcn_global_load_lds(a.Bst + ((int64_t)(p * a.n_kq + qg) * kStepPieces + e) * 8,
            (__attribute__((address_space(3))) void*)(stage + q * kStepPieces + i * 64), 16, 0, 0);
      }
#pragma unroll
      for (int mt = 0; mt < 2; mt++) {
        // the chunk's block of k-step qg: its C rows' 32 columns contiguous (zero
        // past r); a k-step past the rank re-reads the last one (B is masked there)
        const int qg = min(ks / 32 + q, a.n_kq - 1);
        const int64_t at = arow[mt] + (int64_t)qg * (C * 32) + lk * 8;
        if constexpr (A8)
          af[q][mt] = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(a.A) + at);
        else
          af[q][mt] = *reinterpret_cast<const u32x4*>(a.A + at);
      }
      __builtin_amdgcn_sched_barrier(0);         // keep the groups in issue order
    }
    mfma_steps<NSTEP, 0, AFrag>(af, kn, lk, baddr, acc);
  }
  __syncthreads();
  if constexpr (PARK) {
#pragma unroll
    for (int nt = 0; nt < 4; nt++) {
      ff[nt] = park[nt * 256 + threadIdx.x];
#pragma unroll
      for (int mt = 0; mt < 2; mt++) ang[mt][nt] = park[(4 + mt * 4 + nt) * 256 + threadIdx.x];
    }
  }
  // epilogue: RoPE on (col, col + 64) pairs, bf16 rows staged in LDS
  uint16_t* otile = reinterpret_cast<uint16_t*>(stage);
#pragma unroll
  for (int mt = 0; mt < 2; mt++) {
    const int m0 = w * 32 + mt * 16 + lk * 4;
#pragma unroll
    for (int nt = 0; nt < 4; nt++) {
      const int col = nt * 16 + lr;
#pragma unroll
      for (int jj = 0; jj < 4; jj++) {
        float c, s;
        __sincosf(ang[mt][nt] + jj * ff[nt], &s, &c);
        const float x1 = acc[mt][nt][jj], x2 = acc[mt][nt + 4][jj];
        const uint32_t pk = pack_bf16x2(x1 * c - x2 * s, x2 * c + x1 * s);
        otile[(m0 + jj) * kOutW + col] = (uint16_t)pk;
        otile[(m0 + jj) * kOutW + col + 64] = (uint16_t)(pk >> 16);
      }
    }
  }
  __syncthreads();
}

// The rebuilt rows of a tile (in LDS, as rebuild_tile left them) into the key
// slots mslot[] of their chunks (-1: none).  The caller orders the stores against
// later readers.  NT: non-temporal stores, for keys read at the earliest by the
// next step (the fused tail attends them from LDS), long after these lines would
// have left the L2 (tail 29.4 -> 29.0 us at the Llama-3.1-8B shape); keys that
// the next launch attends keep plain stores (non-temporal ones cost the separate
// and overlapped modes 3 % and 1.5 % of the step).
template <int C, bool NT = false>
__device__ __forceinline__ void store_tile(const DecodeArgs& a, int p, const int* mslot, const uint16_t* otile) {
  for (int e = threadIdx.x; e < kRebuildRows * 16; e += 256) {
    const int m = e >> 4, piece = e & 15;
    const int slot = mslot[m / C];
    if (slot < 0) continue;
    uint16_t* dst = a.key_slots + (((int64_t)p * a.top_k + slot) * C + (m % C)) * kHeadDim + piece * 8;
    const u32x4 v = *reinterpret_cast<const u32x4*>(&otile[m * kOutW + piece * 8]);
    if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst));
    else *reinterpret_cast<u32x4*>(dst) = v;
  }
}

template <int C, int NSTEP, bool A8>
__global__ __launch_bounds__(256, 3) void rebuild_kernel(DecodeArgs a) {
  constexpr int MPB = kRebuildRows / C;
  static_assert(MPB <= 256, "one miss entry per thread");
  __shared__ u32x4 stage[rebuild_stage_bytes<NSTEP>() / 16];
  __shared__ int mchunk[MPB], mslot[MPB];
  const int P = a.batch * a.n_kv;
  // Workgroup L serves pair L % P and tile T - 1 - L / P of its T tiles:
  // a pair's misses form a prefix of its list, so the empty tiles (all of them
  // past the misses) are dispatched first and leave at once, and the tiles with
  // work start right after them instead of waiting behind them for a slot.
  // Workgroups go to the 8 XCDs round-robin by linear id; with P a multiple of 8
  // all tiles of a pair run on one XCD and share one L2 copy of the pair's B^T.
  const int n_tiles = (a.top_k + MPB - 1) / MPB;
  const int p = blockIdx.x % P, j0 = (n_tiles - 1 - (int)(blockIdx.x / P)) * MPB;
  const int K = a.top_k;
  // The tile's first miss says whether it has work (the misses are a prefix of
  // the list, which is written in full): every thread reads it beside its own
  // entry, so an empty tile leaves before the barrier and a working one waits for
  // no extra load.  MPB <= 32 entries, one per thread.
  const int64_t l0 = (int64_t)p * K + j0;   // j0 < K: the tiles cover [0, K)
  int mc = -1, ms = -1;
  if ((int)threadIdx.x < MPB && j0 + (int)threadIdx.x < K) {
    mc = a.miss_chunk[l0 + threadIdx.x];
    ms = a.miss_slot[l0 + threadIdx.x];
  }
  if (a.miss_chunk[l0] < 0) return;   // workgroup-uniform: nothing here
  if ((int)threadIdx.x < MPB) {
    mchunk[threadIdx.x] = mc;
    mslot[threadIdx.x] = ms;
  }
  __syncthreads();
  rebuild_tile<C, NSTEP, A8>(a, p, mchunk, stage);
  store_tile<C>(a, p, mslot, reinterpret_cast<const uint16_t*>(stage));
}

template <int C, bool A8>
static hipError_t launch_rebuild_c(const DecodeArgs& a, dim3 grid, hipStream_t st) {
  switch (min(kMaxSteps, (a.rank + 31) / 32)) {
    case 1: rebuild_kernel<C, 1, A8><<<grid, 256, 0, st>>>(a); break;
    case 2: rebuild_kernel<C, 2, A8><<<grid, 256, 0, st>>>(a); break;
    case 3: rebuild_kernel<C, 3, A8><<<grid, 256, 0, st>>>(a); break;
    case 4: rebuild_kernel<C, 4, A8><<<grid, 256, 0, st>>>(a); break;
    case 5: rebuild_kernel<C, 5, A8><<<grid, 256, 0, st>>>(a); break;
    default: rebuild_kernel<C, kMaxSteps, A8><<<grid, 256, 0, st>>>(a); break;
  }
  return hipGetLastError();
}

template <bool A8>
static hipError_t launch_rebuild_a(const DecodeArgs& a, dim3 grid, hipStream_t st) {
  switch (a.chunk) {
    case 4: return launch_rebuild_c<4, A8>(a, grid, st);
    case 8: return launch_rebuild_c<8, A8>(a, grid, st);
    case 16: return launch_rebuild_c<16, A8>(a, grid, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_rebuild(const DecodeArgs& a, hipStream_t st) {
  const int mpb = kRebuildRows / a.chunk;
  dim3 grid(((a.top_k + mpb - 1) / mpb) * a.batch * a.n_kv);
  return a.a_format == SKV_FORMAT_FP8_E5M2 ? launch_rebuild_a<true>(a, grid, st)
                                            : launch_rebuild_a<false>(a, grid, st);
}

// ---------------------------------------------------------------------------
// Append one generated token (position S + t) for every batch element.
//  append_exact_kernel, one workgroup per (batch element, KV head): the exact
//    post-RoPE key RoPE(k') and the value into key_new / val_new.  In both modes
//    an appended token is first held exactly (the summary's assembly keeps the
//    recent tokens' K_new exact; ShadowKV+ keeps them there until their chunk
//    leaves the local window).
//  append_project_kernel, low rank only (paper-graph-ui summary, section 3.4,
//    ShadowKV+ paragraph), one workgroup per batch element: a' = k' Psi with
//    Psi^T the stored B (float64 accumulation of the exact bf16 products,
//    rounded once to the format of A), written as row S + t of the batch
//    element's A, from where the key rebuild reads it once the token's chunk
//    has been folded into the candidates.  1024 threads keep about 20 row loads
//    of B^T per thread, issued eight at a time.
//  fold_kernel, low rank only, after the append that completes a chunk: the
//    oldest exact chunk (combined index n_fold over [window units; appended
//    units]) becomes the pair's last candidate, its landmark the mean of its
//    stored exact keys (rounded once to the landmark format) and its chunk id
//    n_c - W/C + n_fold.  Chunk ids of the
//    candidates stay ascending.

constexpr int kMaxHD = 2048;
constexpr int kAppendThreads = 1024;

__global__ __launch_bounds__(128) void append_exact_kernel(DecodeArgs a, const uint16_t* k_new,
                                                           const uint16_t* v_new, int t) {
  const int b = blockIdx.x % a.batch, h = blockIdx.x / a.batch, tid = threadIdx.x;
  const uint16_t* kp = k_new + (int64_t)b * a.n_kv * kHeadDim + h * kHeadDim;
  const int64_t row = ((int64_t)(b * a.n_kv + h) * a.max_new + t) * kHeadDim;
  if (tid < kHeadDim / 2) {   // rotated in float64, rounded once to bf16
    const double x1 = bf16_to_f32(kp[tid]), x2 = bf16_to_f32(kp[tid + kHeadDim / 2]);
    double cs, sn;
    rope_cs64(a.seq_len + t, a.inv_freq[tid], &cs, &sn);
    a.key_new[row + tid] = f64_to_bf16_rne(x1 * cs - x2 * sn);
    a.key_new[row + tid + kHeadDim / 2] = f64_to_bf16_rne(x2 * cs + x1 * sn);
  } else if (tid < kHeadDim / 2 + kHeadDim / 8) {
    const int c = tid - kHeadDim / 2;
    *reinterpret_cast<u32x4*>(a.val_new + row + c * 8) =
        *reinterpret_cast<const u32x4*>(v_new + ((int64_t)b * a.n_kv + h) * kHeadDim + c * 8);
  }
}

__global__ __launch_bounds__(kAppendThreads) void append_project_kernel(DecodeArgs a, const uint16_t* k_new,
                                                                        int t, uint16_t* A) {
  __shared__ float ks[kMaxHD];                  // k' of the batch element
  __shared__ double red[kAppendThreads * 4];    // per-row-group partials, half of the columns at a time
  __shared__ double red2[kAppendThreads];       // second-level partials
  const int b = blockIdx.x;
  const int HD = a.n_kv * kHeadDim, r = a.rank, tid = threadIdx.x;
  const uint16_t* kp = k_new + (int64_t)b * HD;
  const bool b8 = a.b_format == SKV_FORMAT_FP8_E5M2;
  // B^T of the batch element: bf16, or FP8 bytes (element offsets the same)
  const uint16_t* Bt = b8 ? reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(a.Bt) + (int64_t)b * HD * r)
                          : a.Bt + (int64_t)b * HD * r;
  for (int i = tid; i < HD; i += kAppendThreads) ks[i] = bf16_to_f32(kp[i]);
  __syncthreads();
  // thread (row group g, column piece c) sums rows g, g + ng, ... of B^T over its
  // 8 columns in float64 (every bf16 product is exact there); rows past HD
  // re-read the last row with weight 0
  const int nch = r / 8, ng = kAppendThreads / nch;   // r <= 2048 keeps ng >= 4
  const int c = tid % nch, g = tid / nch;
  double acc[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
  if (g < ng) {
    for (int i0 = g; i0 < HD; i0 += 8 * ng) {
      u32x4 w[8];
#pragma unroll
      for (int m = 0; m < 8; m++) {
        const int64_t at = (int64_t)min(i0 + m * ng, HD - 1) * r + c * 8;
        if (b8) {
          const uint2 w8 = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(Bt) + at);
          w[m] = e5m2x8_to_bf16x8(w8.x, w8.y);
        } else {
          w[m] = *reinterpret_cast<const u32x4*>(Bt + at);
        }
      }
#pragma unroll
      for (int m = 0; m < 8; m++) {
        const int i = i0 + m * ng;
        const double x = i < HD ? (double)ks[min(i, HD - 1)] : 0.0;
        float y[8];
        unpack8(w[m], y);
#pragma unroll
        for (int k = 0; k < 8; k++) acc[k] = fma(x, (double)y[k], acc[k]);
      }
    }
  }
  // sum the ng groups, four of each thread's eight columns per round: parts of
  // the groups first, then the parts.  Column j = 8c + 4hf + k sits at index
  // jj = 4c + k of the round's r/2 columns.
  const int R2 = r / 2, parts = kAppendThreads / R2;   // r <= 2048 keeps parts >= 1
  for (int hf = 0; hf < 2; hf++) {
    if (g < ng) {
#pragma unroll
      for (int k = 0; k < 4; k++) red[g * R2 + c * 4 + k] = acc[hf * 4 + k];
    }
    __syncthreads();
    if (tid < parts * R2) {
      const int jj = tid % R2, pt = tid / R2;
      double sum = 0.0;
      for (int gg = pt; gg < ng; gg += parts) sum += red[gg * R2 + jj];
      red2[pt * R2 + jj] = sum;
    }
    __syncthreads();
    for (int jj = tid; jj < R2; jj += kAppendThreads) {
      double sum = 0.0;
      for (int pt = 0; pt < parts; pt++) sum += red2[pt * R2 + jj];
      const int j = (jj >> 2) * 8 + hf * 4 + (jj & 3);
      const int64_t at = a_tiled(b, a.a_rows, a.n_kq * 32, a.chunk, a.seq_len + t, j);
      if (a.a_format == SKV_FORMAT_FP8_E5M2)
        reinterpret_cast<uint8_t*>(A)[at] = f64_to_e5m2_rne(sum);
      else
        A[at] = f64_to_bf16_rne(sum);
    }
    __syncthreads();   // red and red2 are rewritten by the next round
  }
  for (int j = r + tid; j < a.n_kq * 32; j += kAppendThreads) {   // the row's columns past r stay zero
    const int64_t at = a_tiled(b, a.a_rows, a.n_kq * 32, a.chunk, a.seq_len + t, j);
    if (a.a_format == SKV_FORMAT_FP8_E5M2)
      reinterpret_cast<uint8_t*>(A)[at] = 0;
    else
      A[at] = 0;
  }
}

hipError_t launch_append(const DecodeArgs& a, const uint16_t* k_new, const uint16_t* v_new, int t, bool lowrank,
                         hipStream_t st) {
  append_exact_kernel<<<a.batch * a.n_kv, 128, 0, st>>>(a, k_new, v_new, t);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !lowrank) return e;
  append_project_kernel<<<a.batch, kAppendThreads, 0, st>>>(a, k_new, t, const_cast<uint16_t*>(a.A));
  return hipGetLastError();
}

__global__ __launch_bounds__(kHeadDim) void fold_kernel(DecodeArgs a, uint16_t* L, int32_t* cand_map) {
  const int p = blockIdx.x, dim = threadIdx.x, C = a.chunk, Wu = a.n_win_units, x = a.n_fold;
  const uint16_t* src = x < Wu ? a.k_win + ((int64_t)p * Wu + x) * C * kHeadDim
                               : a.key_new + ((int64_t)p * a.max_new + (int64_t)(x - Wu) * C) * kHeadDim;
  float sum = 0.f;
  for (int i = 0; i < C; i++) sum += bf16_to_f32(src[i * kHeadDim + dim]);
  const int64_t at = ((int64_t)p * a.cand_stride + a.n_cand) * kHeadDim + dim;
  if (a.landmark_format == SKV_FORMAT_FP8_E5M2)
    reinterpret_cast<uint8_t*>(L)[at] = f32_to_e5m2(sum * (1.0f / C));
  else
    L[at] = f32_to_bf16(sum * (1.0f / C));
  if (dim == 0) cand_map[(int64_t)p * a.cand_stride + a.n_cand] = a.n_c - Wu + x;
}

hipError_t launch_fold(const DecodeArgs& a, hipStream_t st) {
  fold_kernel<<<a.batch * a.n_kv, kHeadDim, 0, st>>>(a, const_cast<uint16_t*>(a.L), const_cast<int32_t*>(a.cand_map));
  return hipGetLastError();
}

// Values of chunk ch of pair p: context chunks from the value store, chunks of
// appended tokens (folded into the candidates in low-rank mode) from val_new.
__device__ __forceinline__ const uint16_t* chunk_values(const DecodeArgs& a, int p, int b, int h, int ch) {
  if (ch < a.n_c) return a.v_store + (((int64_t)b * a.n_kv + h) * a.seq_len + (int64_t)ch * a.chunk) * kHeadDim;
  return a.val_new + ((int64_t)p * a.max_new + (int64_t)(ch - a.n_c) * a.chunk) * kHeadDim;
}

// ---------------------------------------------------------------------------
// Value gather from pinned host memory (zero-copy reads over PCIe).

constexpr int kGatherMisses = 16;

__global__ __launch_bounds__(256) void value_gather_kernel(DecodeArgs a) {
  const int p = blockIdx.y;
  const int j0 = blockIdx.x * kGatherMisses;
  const int n = a.n_miss[p];
  if (j0 >= n) return;
  const int b = p / a.n_kv, h = p % a.n_kv;
  const int C = a.chunk, K = a.top_k;
  const int per_miss = C * 16;   // 16-byte pieces
  for (int e = threadIdx.x; e < kGatherMisses * per_miss; e += 256) {
    const int jm = j0 + e / per_miss;
    if (jm >= n) break;
    const int piece = e % per_miss;
    const int slot = a.miss_slot[(int64_t)p * K + jm];
    const int ch = a.miss_chunk[(int64_t)p * K + jm];
    const uint16_t* src = chunk_values(a, p, b, h, ch) + piece * 8;
    uint16_t* dst = a.val_slots + ((int64_t)p * K + slot) * C * kHeadDim + piece * 8;
    *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
  }
}

hipError_t launch_value_gather(const DecodeArgs& a, hipStream_t st) {
  dim3 grid((a.top_k + kGatherMisses - 1) / kGatherMisses, a.batch * a.n_kv);
  value_gather_kernel<<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Split-K flash-decode.  Work unit = one chunk of C tokens: unit u < O is an
// outlier chunk, the next ns units are selected chunks held in key slots, the
// rest the window and the appended tokens.  One workgroup per (pair, split)
// serves all G <= 16 query heads of its KV head, so every key and value is read
// once.  Each wave owns up to NT*16 consecutive tokens (NT tiles of 16) and
// issues all of their K/V loads before computing.  Per tile, both products run
// on MFMA:
//  * S = K q^T (16x16x32 bf16): lane (row r, kq) feeds dims j*32+kq*8.. of token
//    r; the output lane (head n = lane%16, kq) holds tokens 4kq..4kq+3.
//  * softmax in that layout, base 2: one running max and sum per head.
//  * O^T += V^T P (16x16x16 bf16).  The scores' output layout is already the
//    B operand (tokens 4kq..4kq+3 of head n), so P stays in registers; it goes
//    in as bf16 hi + lo parts, which keeps 16 bits of every weight.  The A
//    operand (four tokens of one dim per lane) comes from the value loads by a
//    4x4 dword transpose within each lane quad and one byte permute.
// The four waves of a workgroup merge through LDS into one partial (m, l, o).
//
// Two ways to meet the missed chunks (rebuild_fused):
//  * separate: rebuild_kernel refreshes the missed slots first, then every slot
//    is an attention unit (ns = K);
//  * fused (the summary's reconstruction overlapped with the fetch, section 3.4
//    "Sparse KV Reconstruction and Overlapping Strategy", as one launch): the
//    workgroup that rebuilds a tile of missed chunks attends to those keys
//    straight from LDS (and stores them to their slots for later hits), while
//    the attention workgroups of the same launch take the outliers, the slots
//    that hit (ns = K - misses, listed by the selection) and the exact region.
//    One partial per split and one per tile of misses; combine_kernel merges
//    the ones that hold tokens.

// 16-token tiles per wave.  Two measured fastest (17.6 us per launch at
// b = 8, S = 122 880, G = 4 against 17.9 with three and 20.6 with four; at
// b = 4, S = 1M, G = 16 the same order): the kernel then holds 94 VGPRs + 36
// AGPRs, three waves per SIMD, and a long context splits into more, shorter
// workgroups.
constexpr int kAttnTiles = 2;
constexpr int kAttnMaxHeads = 16;   // query heads per KV head (the MFMA's N)

int attn_units_per_wave(int chunk) { return kAttnTiles * 16 / chunk; }

// Selected-chunk units of pair p: every slot (separate rebuild), or the slots
// that hit (fused rebuild: the misses are attended where they are rebuilt).
__device__ __forceinline__ int slot_units(const DecodeArgs& a, int p) {
  return a.rebuild_fused ? a.top_k - a.n_miss[p] : a.top_k;
}

// Key / value rows of unit u of pair p: O outlier units, then ns selected-chunk
// units, then the exact region; `slot` and `ch` the slot and chunk id of u when it
// is a selected chunk.
template <int C>
__device__ __forceinline__ const uint16_t* unit_key(const DecodeArgs& a, int p, int u, int O, int ns, int slot) {
  const int K = a.top_k, Wu = a.n_win_units;
  if (u < O) return a.k_out + ((int64_t)p * O + u) * C * kHeadDim;
  if (u < O + ns) return a.key_slots + ((int64_t)p * K + slot) * C * kHeadDim;
  const int x = u - O - ns + a.n_fold;
  if (x < Wu) return a.k_win + ((int64_t)p * Wu + x) * C * kHeadDim;
  return a.key_new + ((int64_t)p * a.max_new + (int64_t)(x - Wu) * C) * kHeadDim;
}

template <int C>
__device__ __forceinline__ const uint16_t* unit_value(const DecodeArgs& a, int p, int b, int h, int u, int O, int ns,
                                                      int slot, int ch) {
  const int K = a.top_k;
  if (u < O) return a.v_out + ((int64_t)p * O + u) * C * kHeadDim;
  if (u < O + ns)
    return a.host_values ? a.val_slots + ((int64_t)p * K + slot) * C * kHeadDim : chunk_values(a, p, b, h, ch);
  const int Wu = a.n_win_units, x = u - O - ns + a.n_fold;
  if (x < Wu) return a.v_win + ((int64_t)p * Wu + x) * C * kHeadDim;
  return a.val_new + ((int64_t)p * a.max_new + (int64_t)(x - Wu) * C) * kHeadDim;
}

// Lane j of each quad holds dword w = element (j, w) of a 4x4 block; afterwards
// it holds element (w, j).  Two rounds of 2x2 swaps: lanes one apart exchange
// dwords one apart, then lanes two apart exchange dwords two apart.
__device__ __forceinline__ u32x4 quad_transpose(u32x4 x, int lane) {
  const bool odd = lane & 1, hi = lane & 2;
  constexpr int kSwap1 = 0xB1;   // quad_perm [1,0,3,2]
  constexpr int kSwap2 = 0x4E;   // quad_perm [2,3,0,1]
  uint32_t r = __builtin_amdgcn_mov_dpp((int)(odd ? x[0] : x[1]), kSwap1, 0xF, 0xF, false);
  x[0] = odd ? r : x[0];
  x[1] = odd ? x[1] : r;
  r = __builtin_amdgcn_mov_dpp((int)(odd ? x[2] : x[3]), kSwap1, 0xF, 0xF, false);
  x[2] = odd ? r : x[2];
  x[3] = odd ? x[3] : r;
  r = __builtin_amdgcn_mov_dpp((int)(hi ? x[0] : x[2]), kSwap2, 0xF, 0xF, false);
  x[0] = hi ? r : x[0];
  x[2] = hi ? x[2] : r;
  r = __builtin_amdgcn_mov_dpp((int)(hi ? x[1] : x[3]), kSwap2, 0xF, 0xF, false);
  x[1] = hi ? r : x[1];
  x[3] = hi ? x[3] : r;
  return x;
}

// q^T of pair p in the MFMA B layout: head lr, dims j*32 + lq*8 (zero for heads >= G).
__device__ __forceinline__ void load_q(const DecodeArgs& a, int p, int lr, int lq, bf16x8 (&bq)[4]) {
  const int b = p / a.n_kv, h = p % a.n_kv, G = a.group;
  const int64_t row = (int64_t)b * a.n_kv * G + h * G + lr;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    u32x4 wq = {0u, 0u, 0u, 0u};
    if (lr < G) wq = *reinterpret_cast<const u32x4*>(a.q + row * kHeadDim + j * 32 + lq * 8);
    bq[j] = __builtin_bit_cast(bf16x8, wq);
  }
}

// Merge buffers of one workgroup's four waves (fp32 partial o per wave and head,
// and the running max / sum).
struct AttnMerge {
  float wo[4][kAttnMaxHeads][kHeadDim];
  float wm[4][kAttnMaxHeads], wl[4][kAttnMaxHeads];
};

// Online-softmax attention of one wave over NT tiles of 16 tokens, ntok of them
// valid (the rest weigh 0): keys kf in the MFMA A layout (token t*16 + lr, dims
// j*32 + lq*8), values vf as loaded (token t*16 + 4lq + lr%4, dims c*32 + 8(lr/4)).
// Accumulates the running max m and sum l of head lr and o[c][e][i] = head lr,
// dim c*32 + 8lq + 2i + e.
template <int NT>
__device__ __forceinline__ void wave_attend(const u32x4 (&kf)[NT][4], const u32x4 (&vf)[NT][4], const bf16x8 (&bq)[4],
                                            int ntok, float qscale, int lane, float& m, float& l,
                                            f32x4 (&o)[4][2]) {
  typedef short bf16x4 __attribute__((ext_vector_type(4)));
  constexpr uint32_t kLoHalves = 0x05040100u, kHiHalves = 0x07060302u;   // v_perm selectors
  const int lq = (lane & 63) >> 4;
#pragma unroll
  for (int t = 0; t < NT; t++) {
    if (t * 16 < ntok) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; j++)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[t][j]), bq[j], acc, 0, 0, 0);
      float sv[4];
      float tmax = kNegBig;
#pragma unroll
      for (int i = 0; i < 4; i++) {
        sv[i] = (t * 16 + lq * 4 + i < ntok) ? acc[i] * qscale : kNegBig;
        tmax = fmaxf(tmax, sv[i]);
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float mn = fmaxf(m, tmax);
      const float corr = __builtin_amdgcn_exp2f(m - mn);
      m = mn;
      uint32_t ph[4], pl[4];
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const float pv = __builtin_amdgcn_exp2f(sv[i] - mn);
        psum += pv;
        ph[i] = __builtin_bit_cast(uint32_t, pv);
        pl[i] = __builtin_bit_cast(uint32_t, pv - __builtin_bit_cast(float, ph[i] & 0xffff0000u));
      }
      psum += __shfl_xor(psum, 16);
      psum += __shfl_xor(psum, 32);
      l = l * corr + psum;
      // weights of tokens 4lq..4lq+3 for head lr, truncated to bf16: hi, then the remainder
      const bf16x4 bh = __builtin_bit_cast(bf16x4, (uint32_t __attribute__((ext_vector_type(2)))){
          __builtin_amdgcn_perm(ph[1], ph[0], kHiHalves), __builtin_amdgcn_perm(ph[3], ph[2], kHiHalves)});
      const bf16x4 bl = __builtin_bit_cast(bf16x4, (uint32_t __attribute__((ext_vector_type(2)))){
          __builtin_amdgcn_perm(pl[1], pl[0], kHiHalves), __builtin_amdgcn_perm(pl[3], pl[2], kHiHalves)});
#pragma unroll
      for (int c = 0; c < 4; c++) {
        const u32x4 x = quad_transpose(vf[t][c], lane);   // x[i]: dims (c*32 + 2lr, +1) of token 4lq + i
        const bf16x4 ve = __builtin_bit_cast(bf16x4, (uint32_t __attribute__((ext_vector_type(2)))){
            __builtin_amdgcn_perm(x[1], x[0], kLoHalves), __builtin_amdgcn_perm(x[3], x[2], kLoHalves)});
        const bf16x4 vo = __builtin_bit_cast(bf16x4, (uint32_t __attribute__((ext_vector_type(2)))){
            __builtin_amdgcn_perm(x[1], x[0], kHiHalves), __builtin_amdgcn_perm(x[3], x[2], kHiHalves)});
#pragma unroll
        for (int e = 0; e < 2; e++) o[c][e] *= corr;
        o[c][0] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ve, bh, o[c][0], 0, 0, 0);
        o[c][0] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ve, bl, o[c][0], 0, 0, 0);
        o[c][1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vo, bh, o[c][1], 0, 0, 0);
        o[c][1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vo, bl, o[c][1], 0, 0, 0);
      }
    }
  }
}

// The four waves' (m, l, o) through LDS into one partial row per head at `part`
// (G rows of kPartStride: o[d], m, l).  Called by all 256 threads; `mg` may alias
// memory the waves have finished reading before the call.
__device__ __forceinline__ void merge_waves(int G, int lane, float m, float l, const f32x4 (&o)[4][2],
                                            AttnMerge& mg, float* part) {
  const int w = threadIdx.x >> 6, lr = lane & 15, lq = lane >> 4;
  __syncthreads();   // the waves are done with what `mg` may alias
  if (lr < G) {
#pragma unroll
    for (int c = 0; c < 4; c++) {
      float* dst = &mg.wo[w][lr][c * 32 + 8 * lq];
      *reinterpret_cast<f32x4*>(dst) = f32x4{o[c][0][0], o[c][1][0], o[c][0][1], o[c][1][1]};
      *reinterpret_cast<f32x4*>(dst + 4) = f32x4{o[c][0][2], o[c][1][2], o[c][0][3], o[c][1][3]};
    }
    if (lq == 0) {
      mg.wm[w][lr] = m;
      mg.wl[w][lr] = l;
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * kHeadDim; idx += 256) {
    const int g = idx / kHeadDim, dim = idx % kHeadDim;
    float M = kNegBig;
#pragma unroll
    for (int ww = 0; ww < 4; ww++) M = fmaxf(M, mg.wm[ww][g]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ww++) {
      const float c = __builtin_amdgcn_exp2f(mg.wm[ww][g] - M);
      num += mg.wo[ww][g][dim] * c;
      den += mg.wl[ww][g] * c;
    }
    part[g * kPartStride + dim] = num;
    if (dim == 0) {
      part[g * kPartStride + kHeadDim] = M;
      part[g * kPartStride + kHeadDim + 1] = den;
    }
  }
}

// Attention workgroup (pair p, split): units [split*upw, split*upw + upw) of the
// pair's [outliers; selected-chunk units; exact region] (the exact region being
// the window units and appended units not yet folded into the candidates; its
// last unit may be partly filled: tokens past it are masked like a wave's tail).
// With a.n_static > 0 (the outliers and the exact region attended in the
// selection launch) the splits cover the selected-chunk units alone, and split s
// writes row n_static + s.  With MISSES, the units are the slots of the step's
// misses alone (the overlapped rebuild attends to them after their keys are
// stored) and the partial goes to row tile_row0 + split.  A split past the
// pair's units writes nothing (the merge skips it).
template <int NT, int C, bool MISSES = false>
__device__ __forceinline__ void attend_split(const DecodeArgs& a, int p, int split, AttnMerge& mg) {
  const int b = p / a.n_kv, h = p % a.n_kv;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int lr = lane & 15, lq = lane >> 4;   // (row|head|dim, kq)
  const int K = a.top_k;
  const int O = MISSES ? 0 : a.n_outlier;
  const int ns = MISSES ? a.n_miss[p] : slot_units(a, p);
  const bool hits_only = !MISSES && a.n_static > 0;
  const int u_lo = hits_only ? O : 0;        // first unit of split 0
  const int U = O + ns + (MISSES || hits_only ? 0 : a.n_win_units + a.n_new_units - a.n_fold);
  if (u_lo + split * a.upw >= U) return;     // workgroup-uniform
  const int per_wave = (a.upw + 3) / 4;
  const int uw0 = min(U, u_lo + split * a.upw + w * per_wave);
  const int uw1 = min(min(U, u_lo + split * a.upw + a.upw), uw0 + per_wave);
  // tokens in units [0, U)
  const int valid = MISSES || hits_only ? (O + ns) * C : (O + ns + a.n_win_units - a.n_fold) * C + a.n_new_tokens;
  const int ntok = max(0, min((uw1 - uw0) * C, valid - uw0 * C));

  float m = kNegBig, l = 0.f;   // head lr
  f32x4 o[4][2];
#pragma unroll
  for (int c = 0; c < 4; c++)
#pragma unroll
    for (int e = 0; e < 2; e++) o[c][e] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (ntok > 0) {   // wave-uniform
    // slot and chunk id of each selected-chunk unit of the wave, one per lane
    int my_slot = 0, my_ch = 0;
    if (lane < uw1 - uw0) {
      const int sidx = uw0 + lane - O;
      if (sidx >= 0 && sidx < ns) {
        // the chunk id comes from the list that gives the slot (not through it),
        // so the value loads wait for one dependent load, not two
        const int64_t li = (int64_t)p * K + sidx;
        my_slot = MISSES ? a.miss_slot[li] : (a.rebuild_fused ? a.hit_slot[li] : sidx);
        my_ch = max(MISSES ? a.miss_chunk[li] : (a.rebuild_fused ? a.hit_chunk[li] : a.slot_chunk[li]), 0);
      }
    }
    // q first (every tile needs it; vector-memory loads complete in issue order),
    // then tile by tile, keys then values, so that tile 0 can start as soon as its
    // own loads are in.  Values: lane (lr = 4q + jj, lq) reads token tile*16 + 4lq
    // + jj, dims c*32 + 8q .. +8 for c = 0..3; the quad transpose then leaves it
    // dims c*32 + 2lr and c*32 + 2lr + 1 of tokens 4lq .. 4lq+3.  The loads are
    // unconditional (branch-free code keeps the compiler's per-tile wait counts
    // exact): tokens past the wave's range re-read its last token, whose scores
    // are masked to -inf, so they weigh 0.
    bf16x8 bq[4];
    load_q(a, p, lr, lq, bq);
    const int tlast = ntok - 1;
    u32x4 kf[NT][4], vf[NT][4];
#pragma unroll
    for (int t = 0; t < NT; t++) {
      const int tk = min(t * 16 + lr, tlast);
      const int ks = __shfl(my_slot, tk / C);
      const uint16_t* kp = unit_key<C>(a, p, uw0 + tk / C, O, ns, ks) + (tk % C) * kHeadDim + lq * 8;
#pragma unroll
      for (int j = 0; j < 4; j++) kf[t][j] = *reinterpret_cast<const u32x4*>(kp + j * 32);
      const int tv = min(t * 16 + 4 * lq + (lr & 3), tlast);
      const int vs = __shfl(my_slot, tv / C), vc = __shfl(my_ch, tv / C);
      const uint16_t* vp =
          unit_value<C>(a, p, b, h, uw0 + tv / C, O, ns, vs, vc) + (tv % C) * kHeadDim + (lr >> 2) * 8;
#pragma unroll
      for (int c = 0; c < 4; c++) vf[t][c] = *reinterpret_cast<const u32x4*>(vp + c * 32);
    }
    wave_attend<NT>(kf, vf, bq, ntok, a.scale * kLog2e, lane, m, l, o);
  }
  const int row = MISSES ? a.tile_row0 + split : hits_only ? a.n_static + split : split;
  merge_waves(a.group, lane, m, l, o, mg, a.attn_part + ((int64_t)p * a.n_part_att + row) * a.group * kPartStride);
}

// Static-unit attention workgroup s of pair p (kStaticWaves waves, in the
// two-level selection launch): the pair's outlier units and exact region, which
// do not depend on the step's selection, kStaticWaves * 32 / C units per
// workgroup, 32 / C per wave; the waves' (m, l, o) merge through `lds`
// (static_lds_bytes(G)) into partial row s.
static_assert((size_t)kStaticWaves * kAttnMaxHeads * (kHeadDim + 2) * sizeof(float) <= (size_t)kSelLdsMax,
              "static attention LDS");

template <int G, int C>
__device__ void attend_static(const DecodeArgs& a, int p, int s, float* lds) {
  constexpr int NUW = kAttnTiles * 16 / C;
  const int b = p / a.n_kv, h = p % a.n_kv;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  const int O = a.n_outlier;
  const int U = O + a.n_win_units + a.n_new_units - a.n_fold;   // the static units (none selected)
  const int valid = (O + a.n_win_units - a.n_fold) * C + a.n_new_tokens;
  const int u0 = min(U, (s * kStaticWaves + w) * NUW), u1 = min(U, u0 + NUW);
  const int ntok = max(0, min((u1 - u0) * C, valid - u0 * C));
  float m = kNegBig, l = 0.f;
  f32x4 o[4][2];
#pragma unroll
  for (int c = 0; c < 4; c++)
#pragma unroll
    for (int e = 0; e < 2; e++) o[c][e] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (ntok > 0) {   // wave-uniform; loads as in attend_split (no slot units: ns = 0)
    bf16x8 bq[4];
    load_q(a, p, lr, lq, bq);
    const int tlast = ntok - 1;
    u32x4 kf[kAttnTiles][4], vf[kAttnTiles][4];
#pragma unroll
    for (int t = 0; t < kAttnTiles; t++) {
      const int tk = min(t * 16 + lr, tlast);
      const uint16_t* kp = unit_key<C>(a, p, u0 + tk / C, O, 0, 0) + (tk % C) * kHeadDim + lq * 8;
#pragma unroll
      for (int j = 0; j < 4; j++) kf[t][j] = *reinterpret_cast<const u32x4*>(kp + j * 32);
      const int tv = min(t * 16 + 4 * lq + (lr & 3), tlast);
      const uint16_t* vp = unit_value<C>(a, p, b, h, u0 + tv / C, O, 0, 0, 0) + (tv % C) * kHeadDim + (lr >> 2) * 8;
#pragma unroll
      for (int c = 0; c < 4; c++) vf[t][c] = *reinterpret_cast<const u32x4*>(vp + c * 32);
    }
    wave_attend<kAttnTiles>(kf, vf, bq, ntok, a.scale * kLog2e, lane, m, l, o);
  }
  // merge: wo[wave][head][d], then wm[wave][head], wl[wave][head]
  float* wo = lds;
  float* wm = lds + kStaticWaves * G * kHeadDim;
  float* wl = wm + kStaticWaves * G;
  if (lr < G) {
#pragma unroll
    for (int c = 0; c < 4; c++) {
      float* dst = wo + (w * G + lr) * kHeadDim + c * 32 + 8 * lq;
      *reinterpret_cast<f32x4*>(dst) = f32x4{o[c][0][0], o[c][1][0], o[c][0][1], o[c][1][1]};
      *reinterpret_cast<f32x4*>(dst + 4) = f32x4{o[c][0][2], o[c][1][2], o[c][0][3], o[c][1][3]};
    }
    if (lq == 0) {
      wm[w * G + lr] = m;
      wl[w * G + lr] = l;
    }
  }
  __syncthreads();
  float* part = a.attn_part + ((int64_t)p * a.n_part_att + s) * G * kPartStride;
  for (int idx = threadIdx.x; idx < G * kHeadDim; idx += kStaticWaves * 64) {
    const int g = idx / kHeadDim, dim = idx % kHeadDim;
    float M = kNegBig;
#pragma unroll
    for (int ww = 0; ww < kStaticWaves; ww++) M = fmaxf(M, wm[ww * G + g]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int ww = 0; ww < kStaticWaves; ww++) {
      const float c = __builtin_amdgcn_exp2f(wm[ww * G + g] - M);
      num += wo[(ww * G + g) * kHeadDim + dim] * c;
      den += wl[ww * G + g] * c;
    }
    part[g * kPartStride + dim] = num;
    if (dim == 0) {
      part[g * kPartStride + kHeadDim] = M;
      part[g * kPartStride + kHeadDim + 1] = den;
    }
  }
}

template <int NT, int C, bool MISSES>
__global__ __launch_bounds__(256) void attn_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) AttnMerge mg;
  // pairs fastest: workgroups go to the 8 XCDs round-robin by linear id, so each
  // XCD gets whole pairs (all splits of pairs p = x mod 8) and equal work even
  // when the last split of a pair is short
  attend_split<NT, C, MISSES>(a, blockIdx.x, blockIdx.y, mg);
}

// Merge the partials of one (pair, head) that hold tokens: the attention splits
// [0, ns) and, when the misses are attended on their own (fused or overlapped
// rebuild), the partials of their miss_part_units-unit groups [0, nt) (rows
// tile_row0 + t):  out = sum_s o_s 2^(m_s - M) / sum_s l_s 2^(m_s - M).
// 512 threads: 32 lanes cover one partial row (4 dims each, 16-byte loads) and
// the 16 row groups take every 16th partial, then sum their rows through LDS, so
// a long list is read 16 rows at a time.
constexpr int kCombineThreads = 512;
constexpr int kCombineGroups = kCombineThreads / (kHeadDim / 4);

template <int G>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(DecodeArgs a) {
  __shared__ float cw[kMaxPartials];
  __shared__ __attribute__((aligned(16))) float rows[kCombineGroups][kHeadDim];
  __shared__ float den_sh;
  const int g = blockIdx.x, p = blockIdx.y;
  const int b = p / a.n_kv, h = p % a.n_kv;
  int ns = a.n_split, nt = 0;
  if (a.rebuild_fused) {
    const int nm = a.n_miss[p];
    if (a.n_static > 0) {   // static rows, then the splits over the hits
      ns = a.n_static + (a.top_k - nm + a.upw - 1) / a.upw;
    } else {
      const int units = a.n_outlier + (a.top_k - nm) + a.n_win_units + a.n_new_units - a.n_fold;
      ns = (units + a.upw - 1) / a.upw;
    }
    nt = (nm + a.miss_part_units - 1) / a.miss_part_units;
  }
  const int n = ns + nt;
  const int64_t stride = (int64_t)G * kPartStride;
  const float* base = a.attn_part + (int64_t)p * a.n_part_att * stride + g * kPartStride;
  auto row = [&](int s) { return base + (int64_t)(s < ns ? s : a.tile_row0 + (s - ns)) * stride; };
  for (int s = threadIdx.x; s < n; s += kCombineThreads) cw[s] = row(s)[kHeadDim];
  __syncthreads();
  if (threadIdx.x < 64) {   // wave 0: partial weights 2^(m_s - M) and the denominator
    float M = kNegBig;
    for (int s = threadIdx.x; s < n; s += 64) M = fmaxf(M, cw[s]);
    M = wave_max(M);
    float den = 0.f;
    for (int s = threadIdx.x; s < n; s += 64) {
      const float c = __builtin_amdgcn_exp2f(cw[s] - M);
      den += row(s)[kHeadDim + 1] * c;
      cw[s] = c;
    }
    den = wave_sum(den);
    if (threadIdx.x == 0) den_sh = den;
  }
  __syncthreads();
  const int c4 = threadIdx.x % (kHeadDim / 4), grp = threadIdx.x / (kHeadDim / 4);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = grp; s < n; s += kCombineGroups) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(row(s) + c4 * 4);
    const float c = cw[s];
#pragma unroll
    for (int k = 0; k < 4; k++) acc[k] = fmaf(x[k], c, acc[k]);
  }
  *reinterpret_cast<f32x4*>(&rows[grp][c4 * 4]) = acc;
  __syncthreads();
  if (threadIdx.x < kHeadDim) {
    const int dim = threadIdx.x;
    float num = 0.f;
#pragma unroll
    for (int r = 0; r < kCombineGroups; r++) num += rows[r][dim];
    a.out[((int64_t)b * a.n_kv * G + h * G + g) * kHeadDim + dim] = num / den_sh;
  }
}

template <int G>
static hipError_t launch_combine_g(const DecodeArgs& a, hipStream_t st) {
  combine_kernel<G><<<dim3(G, a.batch * a.n_kv), kCombineThreads, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_combine(const DecodeArgs& a, hipStream_t st) {
  switch (a.group) {
    case 1: return launch_combine_g<1>(a, st);
    case 2: return launch_combine_g<2>(a, st);
    case 4: return launch_combine_g<4>(a, st);
    case 8: return launch_combine_g<8>(a, st);
    case 16: return launch_combine_g<16>(a, st);
    default: return hipErrorInvalidValue;
  }
}

template <bool MISSES>
static hipError_t launch_attention_m(const DecodeArgs& a, hipStream_t st) {
  if (a.group < 1 || a.group > kAttnMaxHeads) return hipErrorInvalidValue;
  const dim3 grid(a.batch * a.n_kv, MISSES ? (a.top_k + a.upw - 1) / a.upw : a.n_split);
  switch (a.chunk) {
    case 4: attn_kernel<kAttnTiles, 4, MISSES><<<grid, 256, 0, st>>>(a); break;
    case 8: attn_kernel<kAttnTiles, 8, MISSES><<<grid, 256, 0, st>>>(a); break;
    case 16: attn_kernel<kAttnTiles, 16, MISSES><<<grid, 256, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attention(const DecodeArgs& a, hipStream_t st) { return launch_attention_m<false>(a, st); }
hipError_t launch_attention_misses(const DecodeArgs& a, hipStream_t st) { return launch_attention_m<true>(a, st); }

// ---------------------------------------------------------------------------
// Fused tail of a decode step: one launch whose first P * n_tiles workgroups
// each rebuild one tile of a pair's missed chunks (rebuild_tile), store the keys
// to their slots (when the temporal cache keeps them) and attend to them from
// LDS, with the tile's values loaded from the value store before the rebuild
// starts, and whose other P * n_split workgroups attend to the outliers, the
// slots that hit and the exact region (attend_split).  Miss tiles go first, the
// empty ones (past a pair's misses) first of all, so the tiles with work start
// at once and the attention workgroups fill in behind them.
// Three workgroups per CU: the tile's values and query are loaded after the
// rebuild, not beside it, and the RoPE angles wait in LDS across the MFMAs.

// Attention of a miss tile: its n_rows rebuilt keys in LDS (rows of kOutW bf16),
// values vf loaded by this wave (rows w*32 + t*16 + 4lq + lr%4, clamped to the
// wave's last row), q in bq; one partial at `part`.
template <int C>
__device__ __forceinline__ void attend_tile(const DecodeArgs& a, int n_rows, const uint16_t* otile,
                                            const u32x4 (&vf)[2][4], const bf16x8 (&bq)[4], float* part,
                                            AttnMerge& mg) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  const int ntok = max(0, min(32, n_rows - w * 32));
  float m = kNegBig, l = 0.f;
  f32x4 o[4][2];
#pragma unroll
  for (int c = 0; c < 4; c++)
#pragma unroll
    for (int e = 0; e < 2; e++) o[c][e] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (ntok > 0) {   // wave-uniform
    u32x4 kf[2][4];
#pragma unroll
    for (int t = 0; t < 2; t++) {
      const int row = w * 32 + min(t * 16 + lr, ntok - 1);
#pragma unroll
      for (int j = 0; j < 4; j++)
        kf[t][j] = *reinterpret_cast<const u32x4*>(otile + row * kOutW + j * 32 + lq * 8);
    }
    wave_attend<2>(kf, vf, bq, ntok, a.scale * kLog2e, lane, m, l, o);
  }
  merge_waves(a.group, lane, m, l, o, mg, part);
}

template <int C, int NSTEP, bool A8, bool ATTEND>
__global__ __launch_bounds__(256, 3) void tail_kernel(DecodeArgs a) {
  constexpr int MPB = kRebuildRows / C;
  static_assert(MPB <= 256, "one miss entry per thread");
  constexpr int kStage = rebuild_stage_bytes<NSTEP>() > (int)sizeof(AttnMerge) ? rebuild_stage_bytes<NSTEP>()
                                                                                : (int)sizeof(AttnMerge);
  __shared__ u32x4 stage[kStage / 16];
  __shared__ float park[ATTEND ? kParkFloats : 1];
  __shared__ int mchunk[MPB], mslot[MPB];
  AttnMerge& mg = *reinterpret_cast<AttnMerge*>(stage);   // used once the stage is read
  const int P = a.batch * a.n_kv;
  const int n_tiles = (a.top_k + MPB - 1) / MPB;
  // Miss tiles first, the empty ones (past a pair's misses: the misses are a
  // prefix of its list) first of all, so they leave at once and the tiles with
  // work start right behind them; the attention splits follow.  Dispatching the
  // two kinds interleaved (tile s and split s of every pair, stage by stage) was
  // slower, 34 against 31 us per launch at the Llama-3.1-8B shape: the tiles
  // still held the slots and the splits waited behind them; dispatching every
  // split first, so that the tiles start behind them, took 37.5 against 32 us.
  const int bid = blockIdx.x;
  if (bid >= P * n_tiles) {
    const int x = bid - P * n_tiles;
    attend_split<kAttnTiles, C>(a, x % P, x / P, mg);
    return;
  }
  const int p = bid % P, idx = n_tiles - 1 - bid / P;
  // miss tile T of pair p: misses [T*MPB, T*MPB + MPB) of the pair's list
  const int T = idx;
  const int j0 = T * MPB, K = a.top_k;
  // The tile's first miss says whether it has work (the misses are a prefix of
  // the list, which is written in full): every thread reads it beside its own
  // entry, so an empty tile leaves before the barrier and a working one waits for
  // no extra load.  MPB <= 32 entries, one per thread.
  const int64_t l0 = (int64_t)p * K + j0;   // j0 < K: the tiles cover [0, K)
  int mc = -1, ms = -1;
  if ((int)threadIdx.x < MPB && j0 + (int)threadIdx.x < K) {
    mc = a.miss_chunk[l0 + threadIdx.x];
    ms = a.miss_slot[l0 + threadIdx.x];
  }
  if (a.miss_chunk[l0] < 0) return;   // workgroup-uniform: nothing here
  if ((int)threadIdx.x < MPB) {
    mchunk[threadIdx.x] = mc;
    mslot[threadIdx.x] = ms;
  }
  __syncthreads();
  if constexpr (!ATTEND) {     // overlapped rebuild: the keys only, attended by the next launch
    rebuild_tile<C, NSTEP, A8>(a, p, mchunk, stage);
    store_tile<C>(a, p, mslot, reinterpret_cast<const uint16_t*>(stage));
    return;
  }
  int nmiss = 0;               // misses in this tile (a prefix of mchunk)
  for (int i = 0; i < MPB; i++) nmiss += mchunk[i] >= 0;
  const int n_rows = nmiss * C;
  const int b = p / a.n_kv, h = p % a.n_kv;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  rebuild_tile<C, NSTEP, A8, true>(a, p, mchunk, stage, park);
  // q and this wave's values go out once the rebuild's accumulators are dead (held
  // across the rebuild they cost the third workgroup per CU), and arrive while the
  // keys are stored to their slots
  bf16x8 bq[4];
  u32x4 vf[2][4];
  const int ntok = max(0, min(32, n_rows - w * 32));
  load_q(a, p, lr, lq, bq);
  if (ntok > 0) {   // wave-uniform
#pragma unroll
    for (int t = 0; t < 2; t++) {
      const int row = w * 32 + min(t * 16 + 4 * lq + (lr & 3), ntok - 1);
      const uint16_t* vp = chunk_values(a, p, b, h, mchunk[row / C]) + (row % C) * kHeadDim + (lr >> 2) * 8;
#pragma unroll
      for (int c = 0; c < 4; c++) vf[t][c] = *reinterpret_cast<const u32x4*>(vp + c * 32);
    }
  } else {
#pragma unroll
    for (int t = 0; t < 2; t++)
#pragma unroll
      for (int c = 0; c < 4; c++) vf[t][c] = (u32x4){0u, 0u, 0u, 0u};
  }
  const uint16_t* otile = reinterpret_cast<const uint16_t*>(stage);
  if (a.temporal) store_tile<C, true>(a, p, mslot, otile);   // kept for the next steps' hits
  attend_tile<C>(a, n_rows, otile, vf, bq,
                 a.attn_part + ((int64_t)p * a.n_part_att + a.tile_row0 + T) * a.group * kPartStride, mg);
}

// k-steps per staged slice of the bf16 path: the whole of r = 160 in one slice
// (one round of operand loads) where three workgroups per CU (168 registers)
// still hold without spills.  With the RoPE angles parked in LDS that is every
// chunk size but C = 4 with the tile attended, which takes slices of 3.  At the
// Llama-3.1-8B shape: slices of 4 (two load rounds), 32.0 us per launch; one
// slice, 30.4 us; two workgroups per CU (all operands in registers), 34.2 us.
template <int C, bool ATTEND>
constexpr int tail_max_steps() {
  return ATTEND && C == 4 ? 3 : kMaxSteps;
}

template <int C, int NS, bool A8, bool ATTEND>
static void launch_tail_s(const DecodeArgs& a, dim3 grid, int want, hipStream_t st) {
  if constexpr (NS < tail_max_steps<C, ATTEND>()) {
    if (want > NS) return launch_tail_s<C, NS + 1, A8, ATTEND>(a, grid, want, st);
  }
  tail_kernel<C, NS, A8, ATTEND><<<grid, 256, 0, st>>>(a);
}

template <int C, bool A8, bool ATTEND>
static hipError_t launch_tail_c(const DecodeArgs& a, dim3 grid, hipStream_t st) {
  launch_tail_s<C, 1, A8, ATTEND>(a, grid, (a.rank + 31) / 32, st);
  return hipGetLastError();
}

template <bool A8, bool ATTEND>
static hipError_t launch_tail_a(const DecodeArgs& a, dim3 grid, hipStream_t st) {
  switch (a.chunk) {
    case 4: return launch_tail_c<4, A8, ATTEND>(a, grid, st);
    case 8: return launch_tail_c<8, A8, ATTEND>(a, grid, st);
    case 16: return launch_tail_c<16, A8, ATTEND>(a, grid, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_tail(const DecodeArgs& a, bool attend_tiles, hipStream_t st) {
  if (a.group < 1 || a.group > kAttnMaxHeads) return hipErrorInvalidValue;
  const int P = a.batch * a.n_kv, mpb = kRebuildRows / a.chunk;
  // with the static units attended in the selection launch, the splits cover at
  // most the K selected chunks
  const int n_split = a.n_static > 0 ? (a.top_k + a.upw - 1) / a.upw : a.n_split;
  const dim3 grid(P * ((a.top_k + mpb - 1) / mpb) + P * n_split);
  const bool a8 = a.a_format == SKV_FORMAT_FP8_E5M2;
  if (attend_tiles) return a8 ? launch_tail_a<true, true>(a, grid, st) : launch_tail_a<false, true>(a, grid, st);
  return a8 ? launch_tail_a<true, false>(a, grid, st) : launch_tail_a<false, false>(a, grid, st);
}

}  // namespace skv
