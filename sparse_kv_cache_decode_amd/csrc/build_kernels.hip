// Pre-fill (build) kernels for gfx950: post-RoPE keys, chunk-mean landmarks and
// in-chunk minimum cosine, outlier choice, candidate compaction, exact outlier /
// window caches, fp64 Gram matrices, fp64 products for the subspace iteration
// and the projection A = K Psi.  The method's pre-fill is described in
// "ShadowKV ..." (papercache deep notes, section A2, pre-fill algorithm; the
// paper-graph-ui summary, section 3.4, "Landmark Construction and Outlier
// Detection" and "Low-Rank Key Cache Compression via Online SVD").
#include <algorithm>

#include "skv_internal.h"
#include "skv_select.h"

namespace skv {

// ---------------------------------------------------------------------------
// RoPE + landmark + min-cos: one wave per (b, h, chunk); lane l holds dims l, l+64
// (the rotate-half pair).  The rotation, the chunk mean and the cosines run in
// float64, and the landmark is rounded once from the float64 mean to its storage
// format (bf16, or FP8 E5M2 with fp8): the stored landmark is then the rounding of
// the exact chunk mean up to float64 error, which only a mean within ~1e-15 of a
// rounding boundary could change.

template <int C>
__global__ __launch_bounds__(256) void rope_landmark_kernel(const uint16_t* __restrict__ k_pre,
                                                            int64_t S, int H, int n_c,
                                                            const double* __restrict__ inv_freq, bool fp8,
                                                            void* __restrict__ L_full,
                                                            float* __restrict__ min_cos) {
  const int lane = threadIdx.x & 63;
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int h = blockIdx.y, b = blockIdx.z;
  if (j >= n_c) return;
  const double f = inv_freq[lane];
  double y1[C], y2[C];
  double m1 = 0.0, m2 = 0.0;
#pragma unroll
  for (int i = 0; i < C; i++) {
    const int64_t pos = (int64_t)j * C + i;
    const uint16_t* row = k_pre + ((int64_t)b * S + pos) * (int64_t)(H * kHeadDim) + h * kHeadDim;
    const double x1 = bf16_to_f32(row[lane]), x2 = bf16_to_f32(row[lane + 64]);
    double c, s;
    rope_cs64(pos, f, &c, &s);
    y1[i] = x1 * c - x2 * s;
    y2[i] = x2 * c + x1 * s;
    m1 += y1[i];
    m2 += y2[i];
  }
  m1 *= 1.0 / C;
  m2 *= 1.0 / C;
  const double mm = wave_sum64(m1 * m1 + m2 * m2);
  double mc = 3.0;
#pragma unroll
  for (int i = 0; i < C; i++) {
    const double dot = wave_sum64(y1[i] * m1 + y2[i] * m2);
    const double kk = wave_sum64(y1[i] * y1[i] + y2[i] * y2[i]);
    const double cs = dot / fmax(sqrt(kk) * sqrt(mm), 1e-8);
    mc = fmin(mc, cs);
  }
  const int64_t pr = (int64_t)b * H + h;
  if (fp8) {
    uint8_t* lrow = static_cast<uint8_t*>(L_full) + (pr * n_c + j) * kHeadDim;
    lrow[lane] = f64_to_e5m2_rne(m1);
    lrow[lane + 64] = f64_to_e5m2_rne(m2);
  } else {
    uint16_t* lrow = static_cast<uint16_t*>(L_full) + (pr * n_c + j) * kHeadDim;
    lrow[lane] = f64_to_bf16_rne(m1);
    lrow[lane + 64] = f64_to_bf16_rne(m2);
  }
  if (lane == 0) min_cos[pr * n_c + j] = (float)mc;
}

hipError_t launch_rope_landmark(const uint16_t* k_pre, int b, int64_t S, int H, int C,
                                const double* inv_freq, bool fp8, void* L_full, float* min_cos,
                                hipStream_t st) {
  const int n_c = (int)(S / C);
  dim3 grid((n_c + 3) / 4, H, b);
  switch (C) {
    case 4: rope_landmark_kernel<4><<<grid, 256, 0, st>>>(k_pre, S, H, n_c, inv_freq, fp8, L_full, min_cos); break;
    case 8: rope_landmark_kernel<8><<<grid, 256, 0, st>>>(k_pre, S, H, n_c, inv_freq, fp8, L_full, min_cos); break;
    case 16: rope_landmark_kernel<16><<<grid, 256, 0, st>>>(k_pre, S, H, n_c, inv_freq, fp8, L_full, min_cos); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Outliers: per pair, the O eligible chunks with the lowest min-cos (lower id on
// ties), ascending.  Key = order-preserving bits of -min_cos.

__global__ __launch_bounds__(256) void outlier_kernel(const float* __restrict__ min_cos, int n_c,
                                                      int n_elig, int O, uint32_t* __restrict__ keys,
                                                      int32_t* __restrict__ outlier_ids) {
  __shared__ int hist[2048 + kTopkSmall];
  __shared__ int sh[32];
  const int p = blockIdx.x;
  const float* mc = min_cos + (int64_t)p * n_c;
  uint32_t* kp = keys + (int64_t)p * n_c;
  for (int i = threadIdx.x; i < n_elig; i += 256) kp[i] = float_key(-mc[i]);
  __syncthreads();
  int32_t* out = outlier_ids + (int64_t)p * O;
  block_topk<256>([&](int i) { return kp[i]; }, n_elig, O, hist, sh,
                  [&](int pos, int i) { if (pos < O) out[pos] = i; });
}

hipError_t launch_outliers(const float* min_cos, int P, int n_c, int n_elig, int O,
                           uint32_t* key_scratch, int32_t* outlier_ids, hipStream_t st) {
  if (O == 0) return hipSuccess;
  outlier_kernel<<<P, 256, 0, st>>>(min_cos, n_c, n_elig, O, key_scratch, outlier_ids);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Candidates: every eligible chunk that is not an outlier, in ascending order;
// landmarks are compacted to those rows.  One wave per chunk.

__global__ __launch_bounds__(256) void candidates_kernel(const uint32_t* __restrict__ L_full,
                                                         const int32_t* __restrict__ outlier_ids,
                                                         int n_c, int n_elig, int O, int stride, int row_words,
                                                         uint32_t* __restrict__ L,
                                                         int32_t* __restrict__ cand_map) {
  const int lane = threadIdx.x & 63;
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int p = blockIdx.y;
  if (j >= n_elig) return;
  const int32_t* oid = outlier_ids + (int64_t)p * O;
  // number of outliers below j (binary search over the ascending list)
  int lo = 0, hi = O;
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (oid[mid] < j) lo = mid + 1; else hi = mid;
  }
  if (lo < O && oid[lo] == j) return;
  const int ci = j - lo;
  const uint32_t* src = L_full + ((int64_t)p * n_c + j) * row_words;
  uint32_t* dst = L + ((int64_t)p * stride + ci) * row_words;
  if (lane < row_words) dst[lane] = src[lane];
  if (lane == 0) cand_map[(int64_t)p * stride + ci] = j;
}

hipError_t launch_candidates(const void* L_full, const int32_t* outlier_ids, int P, int n_c,
                             int n_elig, int O, int stride, int row_bytes, void* L, int32_t* cand_map,
                             hipStream_t st) {
  dim3 grid((n_elig + 3) / 4, P);
  candidates_kernel<<<grid, 256, 0, st>>>(static_cast<const uint32_t*>(L_full), outlier_ids, n_c, n_elig, O,
                                          stride, row_bytes / 4, static_cast<uint32_t*>(L), cand_map);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Exact static caches: post-RoPE keys (rotated in float64, rounded once to bf16)
// and values of the outlier chunks and of the last W tokens.  One wave per
// (pair, token); `v` may be a mapped host pointer.

__global__ __launch_bounds__(256) void static_gather_kernel(
    const uint16_t* __restrict__ k_pre, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ outlier_ids, int64_t S, int H, int C, int O, int W,
    const double* __restrict__ inv_freq, uint16_t* __restrict__ k_out, uint16_t* __restrict__ v_out,
    uint16_t* __restrict__ k_win, uint16_t* __restrict__ v_win) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int p = blockIdx.y;
  const int b = p / H, h = p % H;
  const int n_tok = O * C + W;
  if (t >= n_tok) return;
  int64_t pos;
  uint16_t *kd, *vd;
  if (t < O * C) {
    pos = (int64_t)outlier_ids[(int64_t)p * O + t / C] * C + (t % C);
    kd = k_out + ((int64_t)p * O * C + t) * kHeadDim;
    vd = v_out + ((int64_t)p * O * C + t) * kHeadDim;
  } else {
    const int w = t - O * C;
    pos = S - W + w;
    kd = k_win + ((int64_t)p * W + w) * kHeadDim;
    vd = v_win + ((int64_t)p * W + w) * kHeadDim;
  }
  const uint16_t* row = k_pre + ((int64_t)b * S + pos) * (int64_t)(H * kHeadDim) + h * kHeadDim;
  const double x1 = bf16_to_f32(row[lane]), x2 = bf16_to_f32(row[lane + 64]);
  double c, s;
  rope_cs64(pos, inv_freq[lane], &c, &s);   // rotated in float64, rounded once
  kd[lane] = f64_to_bf16_rne(x1 * c - x2 * s);
  kd[lane + 64] = f64_to_bf16_rne(x2 * c + x1 * s);
  const uint32_t* vs = reinterpret_cast<const uint32_t*>(v + (((int64_t)b * H + h) * S + pos) * kHeadDim);
  reinterpret_cast<uint32_t*>(vd)[lane] = vs[lane];
}

hipError_t launch_static_gather(const uint16_t* k_pre, const uint16_t* v, const int32_t* outlier_ids,
                                int b, int64_t S, int H, int C, int O, int W, const double* inv_freq,
                                uint16_t* k_out, uint16_t* v_out, uint16_t* k_win, uint16_t* v_win,
                                hipStream_t st) {
  const int n_tok = O * C + W;
  if (n_tok == 0) return hipSuccess;
  dim3 grid((n_tok + 3) / 4, b * H);
  static_gather_kernel<<<grid, 256, 0, st>>>(k_pre, v, outlier_ids, S, H, C, O, W, inv_freq, k_out,
                                             v_out, k_win, v_win);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Gram matrices G_b = K_b^T K_b on MFMA.  A bf16 x bf16 product is exact in
// fp32; every v_mfma_f32_32x32x8_bf16 sums the products of 8 rows into fp32 from
// zero, and its result is added to fp64 accumulators at once, so each fp32
// rounding touches a sum of 8 terms only (relative error of the eigenvalues
// about 1e-9 against an fp64 Gram).  Upper-triangle 128 x 128 tiles; a
// workgroup's 4 waves own its 64 x 64 quadrants (2 x 2 MFMA tiles each).  Rows of
// K are split into `nseg` segments whose partial Grams are added in a fixed
// order afterwards (deterministic).

constexpr int GM = 128;          // output tile edge
constexpr int GR = 64;           // rows of K staged per step
constexpr int GP = GR + 4;       // LDS pitch (bf16) of one staged column: 136 B

__global__ __launch_bounds__(256, 2) void gram_kernel(const uint16_t* __restrict__ k_pre, int64_t S, int HD,
                                                      int nseg, double* __restrict__ partial) {
  typedef short bf16x4 __attribute__((ext_vector_type(4)));
  typedef float f32x16 __attribute__((ext_vector_type(16)));
  // staged rows, transposed: column c (0..127 the i-block, 128..255 the j-block)
  // holds its GR rows contiguously, so an MFMA operand (4 consecutive rows of one
  // column) is one 8-byte read; the 136-B pitch spreads 32 columns over all banks
  __shared__ __attribute__((aligned(16))) uint16_t st[2 * GM * GP];
  const int nt = HD / GM;
  int t = blockIdx.x, a = 0;
  while (t >= nt - a) { t -= nt - a; a++; }
  const int i0 = a * GM, j0 = (a + t) * GM;
  const int seg = blockIdx.y, b = blockIdx.z;
  const int64_t seg_len = (S + nseg - 1) / nseg;
  const int64_t s0 = seg * seg_len, s1 = min(S, s0 + seg_len);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wi = w >> 1, wj = w & 1;             // the wave's quadrant
  const int lc = lane & 31, lk = lane >> 5;      // operand column, k group (rows 4lk .. 4lk+3)
  const uint16_t* kb = k_pre + (int64_t)b * S * HD;
  double acc[2][2][16];
#pragma unroll
  for (int mi = 0; mi < 2; mi++)
#pragma unroll
    for (int nj = 0; nj < 2; nj++)
#pragma unroll
      for (int x = 0; x < 16; x++) acc[mi][nj][x] = 0.0;
  for (int64_t s = s0; s < s1; s += GR) {
    __syncthreads();                             // the previous step's reads are done
    for (int e = threadIdx.x; e < GR * 32; e += 256) {
      const int row = e >> 5, c0 = (e & 31) * 8;
      const int gcol = c0 < GM ? i0 + c0 : j0 + c0 - GM;
      u32x4 v = {0u, 0u, 0u, 0u};                // rows past the segment add nothing
      if (s + row < s1) v = *reinterpret_cast<const u32x4*>(kb + (s + row) * HD + gcol);
#pragma unroll
      for (int q = 0; q < 4; q++) {
        st[(c0 + 2 * q) * GP + row] = (uint16_t)(v[q] & 0xffffu);
        st[(c0 + 2 * q + 1) * GP + row] = (uint16_t)(v[q] >> 16);
      }
    }
    __syncthreads();
#pragma unroll 2
    for (int ks = 0; ks < GR / 8; ks++) {
      bf16x4 af[2], bfr[2];
#pragma unroll
      for (int m = 0; m < 2; m++) {
        af[m] = *reinterpret_cast<const bf16x4*>(&st[(wi * 64 + m * 32 + lc) * GP + ks * 8 + lk * 4]);
        bfr[m] = *reinterpret_cast<const bf16x4*>(&st[(GM + wj * 64 + m * 32 + lc) * GP + ks * 8 + lk * 4]);
      }
#pragma unroll
      for (int mi = 0; mi < 2; mi++)
#pragma unroll
        for (int nj = 0; nj < 2; nj++) {
          const f32x16 zero = {};
          const f32x16 c = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(af[mi], bfr[nj], zero, 0, 0, 0);
#pragma unroll
          for (int x = 0; x < 16; x++) acc[mi][nj][x] += (double)c[x];
        }
    }
  }
  // output lane (column lc of the 32 x 32 tile) holds rows 8(x/4) + 4lk + x%4
  double* out = partial + ((int64_t)b * nseg + seg) * HD * HD;
#pragma unroll
  for (int mi = 0; mi < 2; mi++)
#pragma unroll
    for (int nj = 0; nj < 2; nj++)
#pragma unroll
      for (int x = 0; x < 16; x++) {
        const int row = i0 + wi * 64 + mi * 32 + 8 * (x >> 2) + 4 * lk + (x & 3);
        const int col = j0 + wj * 64 + nj * 32 + lc;
        out[(int64_t)row * HD + col] = acc[mi][nj][x];
      }
}

// Sum the segments in order and mirror the upper triangle.
__global__ void gram_reduce_kernel(const double* __restrict__ partial, int HD, int nseg,
                                   double* __restrict__ gram) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int b = blockIdx.y;
  if (idx >= (int64_t)HD * HD) return;
  const int i = (int)(idx / HD), j = (int)(idx % HD);
  const int ti = i / GM, tj = j / GM;
  const int64_t src = ti <= tj ? idx : (int64_t)j * HD + i;
  double s = 0.0;
  for (int g = 0; g < nseg; g++) s += partial[((int64_t)b * nseg + g) * HD * HD + src];
  gram[(int64_t)b * HD * HD + idx] = s;
}

int gram_segments(int b, int64_t S, int HD) {
  const int nt = HD / GM;
  const int tiles = nt * (nt + 1) / 2 * b;
  int nseg = (1024 + tiles - 1) / tiles;        // about 1024 workgroups
  const int64_t max_seg = (S + 4 * GR - 1) / (4 * GR);   // at least 4 staging steps each
  if (nseg > max_seg) nseg = (int)max_seg;
  if (nseg < 1) nseg = 1;
  if (nseg > 64) nseg = 64;
  return nseg;
}

hipError_t launch_gram(const uint16_t* k_pre, int b, int64_t S, int HD, int nseg, double* partial,
                       double* gram, hipStream_t st) {
  const int nt = HD / GM;
  dim3 grid(nt * (nt + 1) / 2, nseg, b);
  gram_kernel<<<grid, 256, 0, st>>>(k_pre, S, HD, nseg, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2((unsigned)(((int64_t)HD * HD + 255) / 256), b);
  gram_reduce_kernel<<<g2, 256, 0, st>>>(partial, HD, nseg, gram);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Batched fp64 C[bi] = op(A[bi]) * B[bi], all row-major: op(A) = A (M x K), or
// with TA the transpose of a K x M array.

template <bool TA>
__global__ __launch_bounds__(256) void gemm_f64_kernel(const double* __restrict__ A,
                                                       const double* __restrict__ B,
                                                       double* __restrict__ C, int M, int N, int K) {
  __shared__ double ta[16][64 + 1];
  __shared__ double tb[16][64 + 1];
  const int bi = blockIdx.z;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  A += (int64_t)bi * M * K;
  B += (int64_t)bi * K * N;
  C += (int64_t)bi * M * N;
  double acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
    for (int e = threadIdx.x; e < 16 * 64; e += 256) {
      const int kk = e / 64, mm = e % 64;
      const int gm = m0 + mm, gk = k0 + kk, gn = n0 + mm;
      ta[kk][mm] = (gm < M && gk < K) ? A[TA ? (int64_t)gk * M + gm : (int64_t)gm * K + gk] : 0.0;
      tb[kk][mm] = (gk < K && gn < N) ? B[(int64_t)gk * N + gn] : 0.0;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; kk++) {
      double x[4], y[4];
#pragma unroll
      for (int q = 0; q < 4; q++) {
        x[q] = ta[kk][ty * 4 + q];
        y[q] = tb[kk][tx * 4 + q];
      }
#pragma unroll
      for (int p = 0; p < 4; p++)
#pragma unroll
        for (int q = 0; q < 4; q++) acc[p][q] = fma(x[p], y[q], acc[p][q]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int p = 0; p < 4; p++)
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const int gm = m0 + ty * 4 + p, gn = n0 + tx * 4 + q;
      if (gm < M && gn < N) C[(int64_t)gm * N + gn] = acc[p][q];
    }
}

hipError_t launch_gemm_f64(const double* A, const double* B, double* C, int batch, int M, int N,
                           int K, hipStream_t st) {
  dim3 grid((N + 63) / 64, (M + 63) / 64, batch);
  gemm_f64_kernel<false><<<grid, 256, 0, st>>>(A, B, C, M, N, K);
  return hipGetLastError();
}

hipError_t launch_gemm_f64_tn(const double* A, const double* B, double* C, int batch, int M, int N,
                              int K, hipStream_t st) {
  dim3 grid((N + 63) / 64, (M + 63) / 64, batch);
  gemm_f64_kernel<true><<<grid, 256, 0, st>>>(A, B, C, M, N, K);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// B^T: psi [b][HD][r] (float64) rounded once to bf16, or to FP8 E5M2 bytes with b8,
// in the same layout.

__global__ void round_psi_kernel(const double* __restrict__ psi, int64_t n, bool b8, void* __restrict__ bt) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  if (b8)
    static_cast<uint8_t*>(bt)[idx] = f64_to_e5m2_rne(psi[idx]);
  else
    static_cast<uint16_t*>(bt)[idx] = f64_to_bf16_rne(psi[idx]);
}

hipError_t launch_round_psi(const double* psi, int b, int HD, int r, bool b8, void* bt, hipStream_t st) {
  const int64_t n = (int64_t)b * HD * r;
  round_psi_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(psi, n, b8, bt);
  return hipGetLastError();
}

// B^T of pair p (rows p*128 .. p*128 + 127 of bt, r each) in the rebuild's stage
// order: element ((p*n_kq + q)*128 + n)*32 + s*8 + j is k = q*32 + (s ^ ((n >> 2) &
// 3))*8 + j of row n, or 0 past r; FP8 E5M2 values (b8) widened to bf16 exactly
// (the byte is the high byte of the equal fp16).  One thread per element.
__global__ void stage_bt_kernel(const void* __restrict__ bt, int64_t n_el, int r, int n_kq, bool b8,
                                uint16_t* __restrict__ bst) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n_el) return;
  const int j = (int)(idx & 7), sl = (int)((idx >> 3) & 3), n = (int)((idx >> 5) & 127);
  const int64_t pq = idx >> 12;   // p * n_kq + q
  const int q = (int)(pq % n_kq);
  const int64_t p = pq / n_kq;
  const int k = q * 32 + ((sl ^ ((n >> 2) & 3)) * 8) + j;
  uint16_t v = 0;
  if (k < r) {
    const int64_t at = (p * 128 + n) * r + k;
    if (b8) {
      const float f = (float)__builtin_bit_cast(_Float16, (uint16_t)(static_cast<const uint8_t*>(bt)[at] << 8));
      v = (uint16_t)(__float_as_uint(f) >> 16);
    } else {
      v = static_cast<const uint16_t*>(bt)[at];
    }
  }
  bst[idx] = v;
}

hipError_t launch_stage_bt(const void* bt, int P, int r, int n_kq, bool b8, uint16_t* bst, hipStream_t st) {
  const int64_t n = (int64_t)P * n_kq * 4096;
  stage_bt_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(bt, n, r, n_kq, b8, bst);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Projection A[b] = K_b Psi_b (S x HD times HD x r) in float64: K's bf16 values are
// exact in float64, Psi is the eigensolver's float64 basis, and every product is
// accumulated with float64 FMAs, so the stored A is the rounding (once, to bf16 or
// FP8 E5M2) of K Psi up to float64 error.  Tiles of 64 rows x 64 columns, k-steps
// of 16 staged in LDS; each of the 256 threads owns 4 x 4 outputs.  The build is
// untimed; at b = 8, S = 122 880, HD = 1024, r = 160 this is about 0.4 TFLOP.

__global__ __launch_bounds__(256) void project_f64_kernel(const uint16_t* __restrict__ k_pre,
                                                          const double* __restrict__ psi, int64_t S, int HD,
                                                          int r, int C, int64_t a_rows, bool fp8,
                                                          void* __restrict__ A) {
  __shared__ double ta[16][64 + 1];   // K tile, [k][row]
  __shared__ double tb[16][64 + 1];   // Psi tile, [k][column]
  const int b = blockIdx.z;
  const int64_t m0 = (int64_t)blockIdx.y * 64;
  const int n0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const uint16_t* kb = k_pre + (int64_t)b * S * HD;
  const double* pb = psi + (int64_t)b * HD * r;
  double acc[4][4] = {};
  for (int k0 = 0; k0 < HD; k0 += 16) {   // HD is a multiple of 128
    for (int e = threadIdx.x; e < 16 * 64; e += 256) {
      const int mm = e >> 4, kk = e & 15;          // 16 consecutive k of one row of K
      const int64_t gm = m0 + mm;
      ta[kk][mm] = gm < S ? (double)bf16_to_f32(kb[gm * HD + k0 + kk]) : 0.0;
      const int kp = e >> 6, nn = e & 63;          // 64 consecutive columns of one row of Psi
      const int gn = n0 + nn;
      tb[kp][nn] = gn < r ? pb[(int64_t)(k0 + kp) * r + gn] : 0.0;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; kk++) {
      double x[4], y[4];
#pragma unroll
      for (int i = 0; i < 4; i++) {
        x[i] = ta[kk][ty * 4 + i];
        y[i] = tb[kk][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = fma(x[i], y[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int64_t row = m0 + ty * 4 + i;
    if (row >= S) continue;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int col = n0 + tx * 4 + j;
      const int r_pad = (r + 31) / 32 * 32;   // the grid's columns cover it: 64-column tiles
      if (col >= r_pad) continue;
      const int64_t at = a_tiled(b, a_rows, r_pad, C, row, col);
      const double v = col < r ? acc[i][j] : 0.0;   // columns past r stay zero
      if (fp8)
        static_cast<uint8_t*>(A)[at] = f64_to_e5m2_rne(v);
      else
        static_cast<uint16_t*>(A)[at] = f64_to_bf16_rne(v);
    }
  }
}

hipError_t launch_project(const uint16_t* k_pre, const double* psi, int b, int64_t S, int HD, int r, int C,
                          int64_t a_rows, bool fp8, void* A, hipStream_t st) {
  if (a_rows % C != 0 || S % C != 0) return hipErrorInvalidValue;
  dim3 grid((r + 63) / 64, (unsigned)((S + 63) / 64), b);
  project_f64_kernel<<<grid, 256, 0, st>>>(k_pre, psi, S, HD, r, C, a_rows, fp8, A);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Fill of a 16-bit array (the optional NaN poisoning of the slot caches).

__global__ void fill_u16_kernel(uint16_t* __restrict__ p, size_t n, uint16_t value) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = value;
}

hipError_t launch_fill_u16(uint16_t* p, size_t n, uint16_t value, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const size_t blocks = std::min<size_t>((n + 255) / 256, 65536);
  fill_u16_kernel<<<(unsigned)blocks, 256, 0, st>>>(p, n, value);
  return hipGetLastError();
}

}  // namespace skv
