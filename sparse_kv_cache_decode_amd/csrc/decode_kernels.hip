// Decode-step kernels for gfx950, following the decode algorithm of "ShadowKV ..."
// (papercache deep notes, section A2; paper-graph-ui summary, section 3.4,
// "Decoding-Time KV Selection via Landmark-Guided Approximate Attention" and
// "Sparse KV Reconstruction and Overlapping Strategy").
//
//  score        : landmark GEMV (one 256-B landmark row feeds the G heads of its
//                 KV head), fp32 logits and per-head log-sum-exp partials.
//  select       : one workgroup per pair combines the LSE, forms the chunk score
//                 max_g(l_g - LSE_g) (log of the group max of softmax
//                 probabilities), selects the top-K chunks and runs the
//                 temporal-cache index scan (hits, misses, slot assignment).
//  rebuild      : keys of the missed chunks, RoPE(Gather(A, I_miss) B), as bf16
//                 MFMA 16x16x32 tiles with the rotation fused into the epilogue.
//  value_gather : missed chunks' values from pinned host memory (side stream).
//  attention    : split-K flash-decode over [outliers; selected; window] with an
//                 online softmax in fp32, then a per-pair merge of the splits.
// Workgroups never wait on one another inside a kernel: device-scope fences on
// gfx950 write back and invalidate the whole L2, so every cross-workgroup
// hand-off goes through a kernel boundary instead.
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
// Score + select + index scan.

__device__ __forceinline__ bool sorted_contains(const int* v, int n, int x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (v[mid] < x) lo = mid + 1; else hi = mid;
  }
  return lo < n && v[lo] == x;
}

template <int G>
__device__ __forceinline__ float pick(const float (&v)[G], int i) {
  float r = v[0];
#pragma unroll
  for (int g = 1; g < G; g++) r = (i == g) ? v[g] : r;
  return r;
}

constexpr int kScoreUnroll = 4;

template <int G>
__global__ __launch_bounds__(256) void score_kernel(DecodeArgs a) {
  __shared__ float red[2][16][16];   // (m, s) per (wave, row) and head
  const int p = blockIdx.y, blk = blockIdx.x;
  const int b = p / a.n_kv, h = p % a.n_kv;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, ds = lane & 15, tg = lane >> 4;
  const int n_cand = a.n_cand;
  const int hq = a.n_kv * G;

  float qv[G][8];
#pragma unroll
  for (int g = 0; g < G; g++) {
    const u32x4 wq = *reinterpret_cast<const u32x4*>(a.q + ((int64_t)b * hq + h * G + g) * kHeadDim + ds * 8);
    unpack8(wq, qv[g]);
#pragma unroll
    for (int i = 0; i < 8; i++) qv[g][i] *= a.scale;
  }
  const int c0 = blk * a.cpb, c1 = min(n_cand, c0 + a.cpb);
  const uint16_t* Lp = a.L + (int64_t)p * n_cand * kHeadDim;
  float* lg = a.logits + (int64_t)p * n_cand * G;
  float m_run = kNegBig, s_run = 0.f;

  for (int base = c0; base < c1; base += 16 * kScoreUnroll) {
    u32x4 wl[kScoreUnroll];
#pragma unroll
    for (int u = 0; u < kScoreUnroll; u++) {
      const int c = base + u * 16 + w * 4 + tg;
      wl[u] = (u32x4){0u, 0u, 0u, 0u};
      if (c < c1) wl[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Lp + (int64_t)c * kHeadDim + ds * 8));
    }
#pragma unroll
    for (int u = 0; u < kScoreUnroll; u++) {
      const int c = base + u * 16 + w * 4 + tg;
      float x[8];
      unpack8(wl[u], x);
      float l[G];
#pragma unroll
      for (int g = 0; g < G; g++) {
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < 8; i++) part = fmaf(qv[g][i], x[i], part);
        l[g] = row16_sum(part);
      }
      if (c < c1 && ds < G) {
        const float v = pick<G>(l, ds);
        lg[(int64_t)c * G + ds] = v;
        const float mn = fmaxf(m_run, v);
        s_run = s_run * __expf(m_run - mn) + __expf(v - mn);
        m_run = mn;
      }
    }
  }
  // per-workgroup (max, sum exp) of every head
  if (ds < G) {
    red[0][w * 4 + tg][ds] = m_run;
    red[1][w * 4 + tg][ds] = s_run;
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

// One workgroup per pair: log-sum-exp of every head over all candidates, chunk
// scores, top-K selection, then the temporal-cache index scan.
constexpr int kSelThreads = 512;

template <int G>
__global__ __launch_bounds__(kSelThreads) void select_kernel(DecodeArgs a) {
  extern __shared__ int smem[];
  int* hist = smem;                 // 2048
  int* sh = smem + 2048;            // 16
  int* sel = smem + 2064;           // top_k
  __shared__ float lse[16];
  const int p = blockIdx.x;
  const int n_cand = a.n_cand;
  const float* lg = a.logits + (int64_t)p * n_cand * G;
  if (threadIdx.x < G) {
    const float* src = a.lse_part + (int64_t)p * a.nb_score * G * 2;
    float M = kNegBig;
    for (int k = 0; k < a.nb_score; k++) M = fmaxf(M, src[(k * G + threadIdx.x) * 2]);
    float S = 0.f;
    for (int k = 0; k < a.nb_score; k++)
      S += src[(k * G + threadIdx.x) * 2 + 1] * __expf(src[(k * G + threadIdx.x) * 2] - M);
    lse[threadIdx.x] = M + __logf(S);
  }
  __syncthreads();
  uint32_t* kp = a.keys + (int64_t)p * n_cand;
  for (int c = threadIdx.x; c < n_cand; c += kSelThreads) {
    float best = -3.0e38f;
#pragma unroll
    for (int g = 0; g < G; g++) best = fmaxf(best, lg[(int64_t)c * G + g] - lse[g]);
    kp[c] = float_key(best);
  }
  __syncthreads();
  const int K = a.top_k;
  block_topk<kSelThreads>([&](int i) { return kp[i]; }, n_cand, K, hist, sh,
                          [&](int pos, int i) { if (pos < K) sel[pos] = i; });
  const int32_t* cmap = a.cand_map + (int64_t)p * n_cand;
  for (int i = threadIdx.x; i < K; i += kSelThreads) a.chunk_ids[(int64_t)p * K + i] = cmap[sel[i]];

  // ---- temporal-cache index scan against the chunks held by the slots
  int32_t* sc = a.slot_cand + (int64_t)p * K;
  int32_t* sch = a.slot_chunk + (int64_t)p * K;
  uint32_t* res = a.resident + (int64_t)p * a.res_words;
  const bool has_prev = a.temporal && sc[0] >= 0;
  int n_free = 0, n_miss = 0;
  for (int t0 = 0; t0 < K; t0 += kSelThreads) {
    const int s = t0 + threadIdx.x;
    int fr = 0, ms = 0, ci = -1;
    if (s < K) {
      const int old = sc[s];
      fr = !(has_prev && old >= 0 && sorted_contains(sel, K, old));
      ci = sel[s];
      ms = !(has_prev && ((res[ci >> 5] >> (ci & 31)) & 1u));
    }
    int tot;
    const int ex = block_exclusive_scan<kSelThreads>(fr | (ms << 16), sh, &tot);
    if (fr) a.free_slot[(int64_t)p * K + n_free + (ex & 0xffff)] = s;
    if (ms) a.miss_cand[(int64_t)p * K + n_miss + (ex >> 16)] = ci;
    n_free += tot & 0xffff;
    n_miss += tot >> 16;
  }
  __syncthreads();
  // n_free == n_miss: every missed chunk takes the next evicted slot
  for (int j = threadIdx.x; j < n_miss; j += kSelThreads) {
    const int slot = a.free_slot[(int64_t)p * K + j];
    const int ci = a.miss_cand[(int64_t)p * K + j];
    const int old = sc[slot];
    if (old >= 0) atomicAnd(&res[old >> 5], ~(1u << (old & 31)));
    atomicOr(&res[ci >> 5], 1u << (ci & 31));
    const int ch = cmap[ci];
    sc[slot] = ci;
    sch[slot] = ch;
    a.miss_slot[(int64_t)p * K + j] = slot;
    a.miss_chunk[(int64_t)p * K + j] = ch;
  }
  if (threadIdx.x == 0) {
    a.n_miss[p] = n_miss;
    a.hits_last[p] = has_prev ? K - n_miss : 0;
    if (has_prev) {
      a.hits_total[p] += K - n_miss;
      a.miss_total[p] += n_miss;
    }
  }
}

hipError_t launch_score(const DecodeArgs& a, hipStream_t st) {
  dim3 grid(a.nb_score, a.batch * a.n_kv);
  switch (a.group) {
    case 1: score_kernel<1><<<grid, 256, 0, st>>>(a); break;
    case 2: score_kernel<2><<<grid, 256, 0, st>>>(a); break;
    case 4: score_kernel<4><<<grid, 256, 0, st>>>(a); break;
    case 8: score_kernel<8><<<grid, 256, 0, st>>>(a); break;
    case 16: score_kernel<16><<<grid, 256, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_select(const DecodeArgs& a, hipStream_t st) {
  const size_t lds = (size_t)(2064 + a.top_k) * sizeof(int);
  const int P = a.batch * a.n_kv;
  switch (a.group) {
    case 1: select_kernel<1><<<P, kSelThreads, lds, st>>>(a); break;
    case 2: select_kernel<2><<<P, kSelThreads, lds, st>>>(a); break;
    case 4: select_kernel<4><<<P, kSelThreads, lds, st>>>(a); break;
    case 8: select_kernel<8><<<P, kSelThreads, lds, st>>>(a); break;
    case 16: select_kernel<16><<<P, kSelThreads, lds, st>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Key rebuild: 128 rows (MPB = 128/C missed chunks) per workgroup, 4 waves x 32
// rows, N = d = 128 as 8 MFMA column tiles; B^T slices of 128 k staged in LDS.

constexpr int kRebuildRows = 128;
constexpr int kKSlice = 128;
constexpr int kLdsW = kKSlice + 8;

template <int C>
__global__ __launch_bounds__(256) void rebuild_kernel(DecodeArgs a) {
  constexpr int MPB = kRebuildRows / C;
  __shared__ __attribute__((aligned(16))) uint16_t tile[128 * kLdsW];
  const int p = blockIdx.y;
  const int j0 = blockIdx.x * MPB;
  const int n = a.n_miss[p];
  if (j0 >= n) return;
  const int b = p / a.n_kv, h = p % a.n_kv;
  const int K = a.top_k, r = a.rank;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int lr = lane & 15, lk = lane >> 4;
  const uint16_t* Bt = a.Bt + ((int64_t)b * a.n_kv * kHeadDim + (int64_t)h * kHeadDim) * r;

  // A operand rows of this lane: row m = w*32 + mt*16 + lr
  const uint16_t* arow[2];
#pragma unroll
  for (int mt = 0; mt < 2; mt++) {
    const int m = w * 32 + mt * 16 + lr;
    const int jm = j0 + m / C;
    arow[mt] = nullptr;
    if (jm < n) {
      const int ch = a.miss_chunk[(int64_t)p * K + jm];
      const int64_t pos = (int64_t)ch * C + (m % C);
      arow[mt] = a.A + ((int64_t)b * a.seq_len + pos) * r;
    }
  }
  f32x4 acc[2][8];
#pragma unroll
  for (int mt = 0; mt < 2; mt++)
#pragma unroll
    for (int nt = 0; nt < 8; nt++) acc[mt][nt] = (f32x4){0.f, 0.f, 0.f, 0.f};

  for (int ks = 0; ks < r; ks += kKSlice) {
    const int kn = min(kKSlice, r - ks);
    __syncthreads();
    const int per_row = kn / 8;
    for (int e = threadIdx.x; e < 128 * per_row; e += 256) {
      const int nr = e / per_row, k8 = (e % per_row) * 8;
      *reinterpret_cast<u32x4*>(&tile[nr * kLdsW + k8]) =
          *reinterpret_cast<const u32x4*>(Bt + (int64_t)nr * r + ks + k8);
    }
    __syncthreads();
    for (int kk = 0; kk < kn; kk += 32) {
      const int kof = kk + lk * 8;
      const bool kin = kof < kn;
      bf16x8 af[2];
#pragma unroll
      for (int mt = 0; mt < 2; mt++) {
        u32x4 wv = {0u, 0u, 0u, 0u};
        if (kin && arow[mt]) wv = *reinterpret_cast<const u32x4*>(arow[mt] + ks + kof);
        af[mt] = __builtin_bit_cast(bf16x8, wv);
      }
#pragma unroll
      for (int nt = 0; nt < 8; nt++) {
        u32x4 wb = {0u, 0u, 0u, 0u};
        if (kin) wb = *reinterpret_cast<const u32x4*>(&tile[(nt * 16 + lr) * kLdsW + kof]);
        const bf16x8 bfr = __builtin_bit_cast(bf16x8, wb);
#pragma unroll
        for (int mt = 0; mt < 2; mt++)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mt], bfr, acc[mt][nt], 0, 0, 0);
      }
    }
  }
  __syncthreads();
  // epilogue: RoPE on (col, col + 64) pairs, stage bf16 rows in LDS
#pragma unroll
  for (int mt = 0; mt < 2; mt++) {
#pragma unroll
    for (int jj = 0; jj < 4; jj++) {
      const int m = w * 32 + mt * 16 + lk * 4 + jj;
      const int jm = j0 + m / C;
      const int ch = jm < n ? a.miss_chunk[(int64_t)p * K + jm] : 0;
      const int64_t pos = (int64_t)ch * C + (m % C);
#pragma unroll
      for (int nt = 0; nt < 4; nt++) {
        const int col = nt * 16 + lr;
        float c, s;
        rope_cs(pos, a.inv_freq[col], &c, &s);
        const float x1 = acc[mt][nt][jj], x2 = acc[mt][nt + 4][jj];
        tile[m * kLdsW + col] = f32_to_bf16(x1 * c - x2 * s);
        tile[m * kLdsW + col + 64] = f32_to_bf16(x2 * c + x1 * s);
      }
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < kRebuildRows * 16; e += 256) {
    const int m = e >> 4, piece = e & 15;
    const int jm = j0 + m / C;
    if (jm >= n) continue;
    const int slot = a.miss_slot[(int64_t)p * K + jm];
    uint16_t* dst = a.key_slots + (((int64_t)p * K + slot) * C + (m % C)) * kHeadDim + piece * 8;
    *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(&tile[m * kLdsW + piece * 8]);
  }
}

hipError_t launch_rebuild(const DecodeArgs& a, hipStream_t st) {
  const int mpb = kRebuildRows / a.chunk;
  dim3 grid((a.top_k + mpb - 1) / mpb, a.batch * a.n_kv);
  switch (a.chunk) {
    case 4: rebuild_kernel<4><<<grid, 256, 0, st>>>(a); break;
    case 8: rebuild_kernel<8><<<grid, 256, 0, st>>>(a); break;
    case 16: rebuild_kernel<16><<<grid, 256, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
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
    const uint16_t* src = a.v_store + (((int64_t)b * a.n_kv + h) * a.seq_len + (int64_t)ch * C) * kHeadDim + piece * 8;
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
// outlier chunk, O <= u < O+K the chunk held by slot u-O, the rest the window.
// Lane (ds, tg): dims 8*ds..8*ds+7 of the tokens tg, tg+4, ... of a unit.

template <int C>
__device__ __forceinline__ void unit_ptrs(const DecodeArgs& a, int p, int b, int h, int u,
                                          const uint16_t** kp, const uint16_t** vp) {
  const int O = a.n_outlier, K = a.top_k;
  if (u < O) {
    const int64_t off = ((int64_t)p * O + u) * C * kHeadDim;
    *kp = a.k_out + off;
    *vp = a.v_out + off;
  } else if (u < O + K) {
    const int s = u - O;
    const int64_t off = ((int64_t)p * K + s) * C * kHeadDim;
    *kp = a.key_slots + off;
    if (a.host_values) {
      *vp = a.val_slots + off;
    } else {
      const int ch = max(a.slot_chunk[(int64_t)p * K + s], 0);
      *vp = a.v_store + (((int64_t)b * a.n_kv + h) * a.seq_len + (int64_t)ch * C) * kHeadDim;
    }
  } else {
    const int wu = u - O - K;
    const int64_t off = ((int64_t)p * a.n_win_units + wu) * C * kHeadDim;
    *kp = a.k_win + off;
    *vp = a.v_win + off;
  }
}

template <int G, int C>
__global__ __launch_bounds__(256) void attn_kernel(DecodeArgs a) {
  constexpr int TPR = C / 4;   // tokens of a unit per lane row
  __shared__ float wo[4][G][kHeadDim];
  __shared__ float wm[4][G], wl[4][G];
  const int p = blockIdx.y, split = blockIdx.x;
  const int b = p / a.n_kv, h = p % a.n_kv;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, ds = lane & 15, tg = lane >> 4;
  const int U = a.n_outlier + a.top_k + a.n_win_units;
  const int u0 = split * a.upw, u1 = min(U, u0 + a.upw);
  const int hq = a.n_kv * G;

  float qv[G][8];
#pragma unroll
  for (int g = 0; g < G; g++) {
    const u32x4 wq = *reinterpret_cast<const u32x4*>(a.q + ((int64_t)b * hq + h * G + g) * kHeadDim + ds * 8);
    unpack8(wq, qv[g]);
#pragma unroll
    for (int i = 0; i < 8; i++) qv[g][i] *= a.scale * kLog2e;
  }
  float m[G], l[G], o[G][8];
#pragma unroll
  for (int g = 0; g < G; g++) {
    m[g] = kNegBig;
    l[g] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; i++) o[g][i] = 0.f;
  }
  u32x4 kw[TPR], vw[TPR];
  int u = u0 + w;
  auto load = [&](int uu, u32x4* kd, u32x4* vd) {
    const uint16_t *kp, *vp;
    unit_ptrs<C>(a, p, b, h, uu, &kp, &vp);
#pragma unroll
    for (int i = 0; i < TPR; i++) {
      const int t = tg + 4 * i;
      kd[i] = *reinterpret_cast<const u32x4*>(kp + t * kHeadDim + ds * 8);
      vd[i] = *reinterpret_cast<const u32x4*>(vp + t * kHeadDim + ds * 8);
    }
  };
  if (u < u1) load(u, kw, vw);
  while (u < u1) {
    const int un = u + 4;
    u32x4 nk[TPR], nv[TPR];
    if (un < u1) load(un, nk, nv);
    float s[TPR][G];
#pragma unroll
    for (int i = 0; i < TPR; i++) {
      float x[8];
      unpack8(kw[i], x);
#pragma unroll
      for (int g = 0; g < G; g++) {
        float part = 0.f;
#pragma unroll
        for (int k = 0; k < 8; k++) part = fmaf(qv[g][k], x[k], part);
        s[i][g] = row16_sum(part);
      }
    }
#pragma unroll
    for (int g = 0; g < G; g++) {
      float mx = s[0][g];
#pragma unroll
      for (int i = 1; i < TPR; i++) mx = fmaxf(mx, s[i][g]);
      const float mn = fmaxf(m[g], mx);
      const float corr = exp2f(m[g] - mn);
      m[g] = mn;
      l[g] *= corr;
#pragma unroll
      for (int k = 0; k < 8; k++) o[g][k] *= corr;
    }
#pragma unroll
    for (int i = 0; i < TPR; i++) {
      float y[8];
      unpack8(vw[i], y);
#pragma unroll
      for (int g = 0; g < G; g++) {
        const float pr = exp2f(s[i][g] - m[g]);
        l[g] += pr;
#pragma unroll
        for (int k = 0; k < 8; k++) o[g][k] = fmaf(pr, y[k], o[g][k]);
      }
    }
#pragma unroll
    for (int i = 0; i < TPR; i++) {
      kw[i] = nk[i];
      vw[i] = nv[i];
    }
    u = un;
  }
  // merge the four token rows of the wave (lanes ds, ds+16, ds+32, ds+48)
#pragma unroll
  for (int off = 16; off <= 32; off <<= 1) {
#pragma unroll
    for (int g = 0; g < G; g++) {
      const float mo = __shfl_xor(m[g], off), lo = __shfl_xor(l[g], off);
      const float mn = fmaxf(m[g], mo);
      const float c1 = exp2f(m[g] - mn), c2 = exp2f(mo - mn);
      l[g] = l[g] * c1 + lo * c2;
#pragma unroll
      for (int k = 0; k < 8; k++) {
        const float oo = __shfl_xor(o[g][k], off);
        o[g][k] = o[g][k] * c1 + oo * c2;
      }
      m[g] = mn;
    }
  }
  if (tg == 0) {
#pragma unroll
    for (int g = 0; g < G; g++) {
#pragma unroll
      for (int k = 0; k < 8; k++) wo[w][g][ds * 8 + k] = o[g][k];
      if (ds == 0) {
        wm[w][g] = m[g];
        wl[w][g] = l[g];
      }
    }
  }
  __syncthreads();
  float* part = a.attn_part + ((int64_t)p * a.n_split + split) * G * (kHeadDim + 2);
  for (int idx = threadIdx.x; idx < G * kHeadDim; idx += 256) {
    const int g = idx / kHeadDim, dim = idx % kHeadDim;
    float M = kNegBig;
#pragma unroll
    for (int ww = 0; ww < 4; ww++) M = fmaxf(M, wm[ww][g]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ww++) {
      const float c = exp2f(wm[ww][g] - M);
      num += wo[ww][g][dim] * c;
      den += wl[ww][g] * c;
    }
    part[g * (kHeadDim + 2) + dim] = num;
    if (dim == 0) {
      part[g * (kHeadDim + 2) + kHeadDim] = M;
      part[g * (kHeadDim + 2) + kHeadDim + 1] = den;
    }
  }
}

// Merge the split partials of one pair: out = sum_s o_s 2^(m_s - M) / sum_s l_s 2^(m_s - M).
template <int G>
__global__ __launch_bounds__(256) void combine_kernel(DecodeArgs a) {
  const int p = blockIdx.x;
  const int b = p / a.n_kv, h = p % a.n_kv;
  const int hq = a.n_kv * G;
  const float* allp = a.attn_part + (int64_t)p * a.n_split * G * (kHeadDim + 2);
  for (int idx = threadIdx.x; idx < G * kHeadDim; idx += 256) {
    const int g = idx / kHeadDim, dim = idx % kHeadDim;
    float M = kNegBig;
    for (int sp = 0; sp < a.n_split; sp++) M = fmaxf(M, allp[(sp * G + g) * (kHeadDim + 2) + kHeadDim]);
    float num = 0.f, den = 0.f;
    for (int sp = 0; sp < a.n_split; sp++) {
      const float* ps = allp + (sp * G + g) * (kHeadDim + 2);
      const float c = exp2f(ps[kHeadDim] - M);
      num += ps[dim] * c;
      den += ps[kHeadDim + 1] * c;
    }
    a.out[((int64_t)b * hq + h * G + g) * kHeadDim + dim] = num / den;
  }
}

template <int G>
static hipError_t launch_attn_g(const DecodeArgs& a, hipStream_t st) {
  dim3 grid(a.n_split, a.batch * a.n_kv);
  switch (a.chunk) {
    case 4: attn_kernel<G, 4><<<grid, 256, 0, st>>>(a); break;
    case 8: attn_kernel<G, 8><<<grid, 256, 0, st>>>(a); break;
    case 16: attn_kernel<G, 16><<<grid, 256, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  combine_kernel<G><<<a.batch * a.n_kv, 256, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_attention(const DecodeArgs& a, hipStream_t st) {
  switch (a.group) {
    case 1: return launch_attn_g<1>(a, st);
    case 2: return launch_attn_g<2>(a, st);
    case 4: return launch_attn_g<4>(a, st);
    case 8: return launch_attn_g<8>(a, st);
    case 16: return launch_attn_g<16>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace skv
