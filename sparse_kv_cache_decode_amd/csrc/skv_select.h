// Block-wide top-k selection over uint32 keys (radix select on 11-bit digits of key - min),
// deterministic: larger key first, lower index on equal keys, indices emitted in
// ascending order.  Used for the outlier test at build time and for the per-KV-head
// chunk selection at decode time.
#pragma once
#include "skv_device.h"

namespace skv {

// LDS needed: hist[2048] ints and sh[32] ints.  Requires n < 2^19, k <= 4096.
// get(i) -> uint32 key of element i (0 <= i < n); emit(pos, i) is called once for
// each selected element with its rank pos in ascending index order (0..k-1).
// Every thread of the block must call it.  Requires 1 <= k <= n.
template <int NT, class Get, class Emit>
__device__ void block_topk(Get get, int n, int k, int* hist, int* sh, Emit emit) {
  static_assert(NT % 64 == 0 && 2048 % NT == 0 && NT / 64 + 8 <= 32, "block size");
  constexpr int PER = 2048 / NT;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  // Digits are taken from key - min(key), starting at its most significant bit, so the
  // first histogram spreads over the keys' actual range (scores share a few exponents).
  uint32_t lo = 0xffffffffu, hi = 0u;
  for (int i = threadIdx.x; i < n; i += NT) {
    const uint32_t u = get(i);
    lo = min(lo, u);
    hi = max(hi, u);
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    lo = min(lo, (uint32_t)__shfl_xor((int)lo, o));
    hi = max(hi, (uint32_t)__shfl_xor((int)hi, o));
  }
  if (lane == 0) {
    hist[wid] = (int)lo;
    hist[64 + wid] = (int)hi;
  }
  __syncthreads();
  lo = 0xffffffffu;
  hi = 0u;
#pragma unroll
  for (int w = 0; w < NT / 64; w++) {
    lo = min(lo, (uint32_t)hist[w]);
    hi = max(hi, (uint32_t)hist[64 + w]);
  }
  __syncthreads();
  const uint32_t kmin = lo, range = hi - lo;
  const int nbits = range == 0u ? 1 : 32 - __clz(range);
  uint32_t prefix = 0, mask = 0;   // on key - kmin
  int kk = k;
  for (int top = nbits; top > 0; top -= 11) {
    const int shift = max(0, top - 11);
    const uint32_t dmask = (1u << (top - shift)) - 1u;
    for (int i = threadIdx.x; i < 2048; i += NT) hist[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += NT) {
      const uint32_t rel = get(i) - kmin;
      if ((rel & mask) == prefix) atomicAdd(&hist[(rel >> shift) & dmask], 1);
    }
    __syncthreads();
    // bins in descending order; thread t owns bins 2047 - PER*t - (0..PER-1)
    int local = 0;
    const int tb = 2047 - PER * threadIdx.x;
#pragma unroll
    for (int j = 0; j < PER; j++) local += hist[tb - j];
    int tot;
    int above = block_exclusive_scan<NT>(local, sh, &tot);
#pragma unroll
    for (int j = 0; j < PER; j++) {
      const int hcount = hist[tb - j];
      if (above < kk && kk <= above + hcount) {
        sh[NT / 64] = tb - j;
        sh[NT / 64 + 1] = kk - above;
      }
      above += hcount;
    }
    __syncthreads();
    const uint32_t dv = (uint32_t)sh[NT / 64];
    kk = sh[NT / 64 + 1];
    prefix |= dv << shift;
    mask |= dmask << shift;
    __syncthreads();
  }
  prefix += kmin;
  // prefix is the k-th largest key T; every key > T is taken plus the kk lowest-index
  // keys equal to T.  Each thread owns a contiguous index range, so one block scan of
  // its (greater, equal) counts places its selections in ascending index order.
  const uint32_t T = prefix;
  const int per = (n + NT - 1) / NT;
  const int i0 = min(n, (int)threadIdx.x * per), i1 = min(n, i0 + per);
  int gt = 0, eq = 0;
  for (int i = i0; i < i1; i++) {
    const uint32_t u = get(i);
    gt += u > T;
    eq += u == T;
  }
  int tot;
  // greater counts sum to < k <= 4096 (13 bits); equal counts to <= n < 2^19
  const int ex = block_exclusive_scan<NT>(gt | (eq << 13), sh, &tot);
  int pos = (ex & 0x1fff) + min(ex >> 13, kk);
  int eq_seen = ex >> 13;
  for (int i = i0; i < i1; i++) {
    const uint32_t u = get(i);
    if (u > T) {
      emit(pos++, i);
    } else if (u == T) {
      if (eq_seen < kk) emit(pos++, i);
      eq_seen++;
    }
  }
  __syncthreads();
}

}  // namespace skv
