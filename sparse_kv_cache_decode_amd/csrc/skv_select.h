// Block-wide top-k selection over uint32 keys (radix select, digits 11/11/10),
// deterministic: larger key first, lower index on equal keys, indices emitted in
// ascending order.  Used for the outlier test at build time and for the per-KV-head
// chunk selection at decode time.
#pragma once
#include "skv_device.h"

namespace skv {

// LDS needed: hist[2048] ints and sh[NT/64 + 8] ints.
// get(i) -> uint32 key of element i (0 <= i < n); emit(pos, i) is called once for
// each selected element with its rank pos in ascending index order (0..k-1).
// Every thread of the block must call it.  Requires 1 <= k <= n.
template <int NT, class Get, class Emit>
__device__ void block_topk(Get get, int n, int k, int* hist, int* sh, Emit emit) {
  static_assert(NT % 64 == 0 && 2048 % NT == 0, "block size");
  constexpr int PER = 2048 / NT;
  uint32_t prefix = 0, mask = 0;
  int kk = k;
  for (int pass = 0; pass < 3; pass++) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const uint32_t dmask = pass < 2 ? 2047u : 1023u;
    for (int i = threadIdx.x; i < 2048; i += NT) hist[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += NT) {
      uint32_t u = get(i);
      if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & dmask], 1);
    }
    __syncthreads();
    // bins in descending order; thread t owns bins 2047 - PER*t - (0..PER-1)
    int local = 0;
    const int top = 2047 - PER * threadIdx.x;
#pragma unroll
    for (int j = 0; j < PER; j++) local += hist[top - j];
    int tot;
    int above = block_exclusive_scan<NT>(local, sh, &tot);
#pragma unroll
    for (int j = 0; j < PER; j++) {
      int h = hist[top - j];
      if (above < kk && kk <= above + h) {
        sh[NT / 64] = top - j;
        sh[NT / 64 + 1] = kk - above;
      }
      above += h;
    }
    __syncthreads();
    const uint32_t dv = (uint32_t)sh[NT / 64];
    kk = sh[NT / 64 + 1];
    prefix |= dv << shift;
    mask |= dmask << shift;
    __syncthreads();
  }
  // prefix is the k-th largest key; kk elements equal to it are taken, lowest index first
  const uint32_t T = prefix;
  int out_base = 0, eq_run = 0;
  for (int t0 = 0; t0 < n; t0 += NT) {
    const int i = t0 + threadIdx.x;
    uint32_t u = i < n ? get(i) : 0u;
    const int gt = (i < n) && (u > T);
    const int eq = (i < n) && (u == T);
    int tot;
    const int ex = block_exclusive_scan<NT>(gt | (eq << 16), sh, &tot);
    const int gt_ex = ex & 0xffff, eq_ex = ex >> 16;
    const int gt_tot = tot & 0xffff, eq_tot = tot >> 16;
    const int taken_before = min(eq_run + eq_ex, kk) - min(eq_run, kk);
    if (gt || (eq && eq_run + eq_ex < kk)) emit(out_base + gt_ex + taken_before, i);
    out_base += gt_tot + min(eq_run + eq_tot, kk) - min(eq_run, kk);
    eq_run += eq_tot;
  }
  __syncthreads();
}

}  // namespace skv
