// Block-wide top-k selection over uint32 keys (radix select on 11-bit digits of key - min),
// deterministic: larger key first, lower index on equal keys, indices emitted in
// ascending order.  Used for the outlier test at build time and for the per-KV-head
// chunk selection at decode time.
#pragma once
#include "skv_device.h"

namespace skv {

// Largest key range start: every thread passes its own partial min / max of the
// keys it produced; block_range combines them (needs sh[32]).  SH_BUSY: sh may
// still be read by another thread (wait for it before writing).  TRAIL = false:
// no closing barrier; the caller passes one before anything writes sh again.
template <int NT, bool SH_BUSY = true, bool TRAIL = true>
__device__ __forceinline__ void block_range(uint32_t& lo, uint32_t& hi, int* sh) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  lo = wave_umin(lo);
  hi = wave_umax(hi);
  if constexpr (SH_BUSY) __syncthreads();
  if (lane == 0) {
    sh[wid] = (int)lo;
    sh[16 + wid] = (int)hi;
  }
  __syncthreads();
  lo = 0xffffffffu;
  hi = 0u;
#pragma unroll
  for (int w = 0; w < NT / 64; w++) {
    lo = min(lo, (uint32_t)sh[w]);
    hi = max(hi, (uint32_t)sh[16 + w]);
  }
  if constexpr (TRAIL) __syncthreads();
}

// Boundary buckets at most this large are finished by counting ranks directly.
constexpr int kTopkSmall = 256;

// LDS needed: hist[2048 + kTopkSmall] ints and sh[32] ints.  Requires n < 2^19,
// k <= 4096 and 1 <= k <= n.  get(i) -> uint32 key of element i (0 <= i < n);
// emit(pos, i) is called once for each selected element with its rank pos in
// ascending index order (0..k-1).  [kmin, kmax] must bound the keys (block_range).
// Every thread of the block must call it.
template <int NT, class Get, class Emit>
__device__ void block_topk(Get get, int n, int k, uint32_t kmin, uint32_t kmax, int* hist, int* sh,
                           Emit emit) {
  static_assert(NT % 64 == 0 && 2048 % NT == 0 && NT / 64 + 8 <= 32 && NT >= kTopkSmall, "block size");
  constexpr int PER = 2048 / NT;
  // Digits are taken from key - kmin, starting at its most significant bit, so the
  // first histogram spreads over the keys' actual range (scores share a few exponents).
  const uint32_t range = kmax - kmin;
  const int nbits = range == 0u ? 1 : 32 - __clz(range);
  uint32_t prefix = 0, mask = 0;   // on key - kmin
  int kk = k;
  int* small = hist + 2048;
  bool done = false;
  for (int top = nbits; top > 0 && !done; top -= 11) {
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
        sh[NT / 64 + 2] = hcount;
      }
      above += hcount;
    }
    __syncthreads();
    const uint32_t dv = (uint32_t)sh[NT / 64];
    kk = sh[NT / 64 + 1];
    const int bcount = sh[NT / 64 + 2];
    prefix |= dv << shift;
    mask |= dmask << shift;
    __syncthreads();
    if (shift > 0 && bcount <= kTopkSmall) {
      // few keys share the boundary bucket: gather them and find the kk-th
      // largest of them by counting, instead of more histogram passes
      if (threadIdx.x == 0) sh[NT / 64 + 3] = 0;
      __syncthreads();
      for (int i = threadIdx.x; i < n; i += NT) {
        const uint32_t rel = get(i) - kmin;
        if ((rel & mask) == prefix) small[atomicAdd(&sh[NT / 64 + 3], 1)] = (int)rel;
      }
      __syncthreads();
      if ((int)threadIdx.x < bcount) {
        const uint32_t v = (uint32_t)small[threadIdx.x];
        int gt = 0, eq = 0;
        for (int j = 0; j < bcount; j++) {
          const uint32_t u = (uint32_t)small[j];
          gt += u > v;
          eq += u == v;
        }
        if (gt < kk && kk <= gt + eq) {   // v is the kk-th largest; all such threads agree
          sh[NT / 64 + 4] = (int)v;
          sh[NT / 64 + 5] = kk - gt;
        }
      }
      __syncthreads();
      prefix = (uint32_t)sh[NT / 64 + 4];
      kk = sh[NT / 64 + 5];
      __syncthreads();
      done = true;
    }
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

// The range sweep folded in: min / max over all keys, then block_topk.
template <int NT, class Get, class Emit>
__device__ void block_topk(Get get, int n, int k, int* hist, int* sh, Emit emit) {
  uint32_t lo = 0xffffffffu, hi = 0u;
  for (int i = threadIdx.x; i < n; i += NT) {
    const uint32_t u = get(i);
    lo = min(lo, u);
    hi = max(hi, u);
  }
  block_range<NT>(lo, hi, sh);
  block_topk<NT>(get, n, k, lo, hi, hist, sh, emit);
}

// The k-th largest of keys held in registers (radix select on 11-bit digits of
// key - kmin; element e of a thread counts when bit e of vmask is set; [kmin, kmax]
// bound the counted keys, as block_range gives them).  Returns the k-th largest
// key T and, in *kk_eq, how many of the keys equal to T are among the k largest.
// If hist_cleared, hist[0, 2048) is already zero and visible to every thread.
// LEAN: no barrier that only guards sh[0, NT/64) or hist against the caller's next
// writes (the last reads of sh[0, NT/64) and of hist end before a barrier inside;
// sh[NT/64, NT/64 + 6) may still be read on return): for a caller whose next
// write to sh[NT/64, ...) or to small (hist + 2048) follows a barrier of its own.
// BOUND: stop after the first digit pass and return the lower edge of the bucket
// that holds the k-th largest key (its key - kmin with the digits below zero): a
// value <= the k-th largest key with at least k keys >= it (*kk_eq is then not
// meaningful).  Exact when one digit covers the range.
template <int NT, int PT, bool LEAN = false, bool BOUND = false>
__device__ uint32_t block_kth_reg(const uint32_t (&key)[PT], uint64_t vmask, int k, uint32_t kmin, uint32_t kmax,
                                  int* hist, int* sh, bool hist_cleared, int* kk_eq) {
  static_assert(NT % 64 == 0 && 2048 % NT == 0 && NT / 64 + 8 <= 32 && NT >= kTopkSmall, "block size");
  static_assert(PT <= 64, "validity mask");
  constexpr int PER = 2048 / NT;
  const uint32_t range = kmax - kmin;
  const int nbits = range == 0u ? 1 : 32 - __clz(range);
  uint32_t prefix = 0, mask = 0;   // on key - kmin
  int kk = k;
  int* small = hist + 2048;
  bool done = false, cleared = hist_cleared;
  for (int top = nbits; top > 0 && !done; top -= 11) {
    const int shift = max(0, top - 11);
    const uint32_t dmask = (1u << (top - shift)) - 1u;
    if (!cleared) {
      for (int i = threadIdx.x; i < 2048; i += NT) hist[i] = 0;
      __syncthreads();
    }
    cleared = false;
#pragma unroll
    for (int e = 0; e < PT; e++) {
      const uint32_t rel = key[e] - kmin;
      if (((vmask >> e) & 1) && (rel & mask) == prefix) atomicAdd(&hist[(rel >> shift) & dmask], 1);
    }
    __syncthreads();
    // bins in descending order; thread t owns bins 2047 - PER*t - (0..PER-1)
    int local = 0;
    const int tb = 2047 - PER * threadIdx.x;
#pragma unroll
    for (int j = 0; j < PER; j++) local += hist[tb - j];
    int tot;   // (the barrier after `find` below orders the scan's reads before later writes)
    int above = block_exclusive_scan<NT, !LEAN>(local, sh, &tot);
#pragma unroll
    for (int j = 0; j < PER; j++) {
      const int hcount = hist[tb - j];
      if (above < kk && kk <= above + hcount) {
        sh[NT / 64] = tb - j;
        sh[NT / 64 + 1] = kk - above;
        sh[NT / 64 + 2] = hcount;
        sh[NT / 64 + 3] = 0;     // gather counter of the small path
      }
      above += hcount;
    }
    __syncthreads();
    const uint32_t dv = (uint32_t)sh[NT / 64];
    kk = sh[NT / 64 + 1];
    const int bcount = sh[NT / 64 + 2];
    prefix |= dv << shift;
    mask |= dmask << shift;
    if constexpr (BOUND) {
      done = true;   // (loop exit; the lower digits of prefix stay zero)
      continue;
    }
    if (shift > 0 && bcount <= kTopkSmall) {
      // few keys share the boundary bucket: gather them and find the kk-th
      // largest of them by counting, instead of more histogram passes
#pragma unroll
      for (int e = 0; e < PT; e++) {
        const uint32_t rel = key[e] - kmin;
        if (((vmask >> e) & 1) && (rel & mask) == prefix) small[atomicAdd(&sh[NT / 64 + 3], 1)] = (int)rel;
      }
      __syncthreads();
      if ((int)threadIdx.x < bcount) {
        const uint32_t v = (uint32_t)small[threadIdx.x];
        int gt = 0, eq = 0;
        for (int j = 0; j < bcount; j++) {
          const uint32_t u = (uint32_t)small[j];
          gt += u > v;
          eq += u == v;
        }
        if (gt < kk && kk <= gt + eq) {   // v is the kk-th largest; all such threads agree
          sh[NT / 64 + 4] = (int)v;
          sh[NT / 64 + 5] = kk - gt;
        }
      }
      __syncthreads();
      prefix = (uint32_t)sh[NT / 64 + 4];
      kk = sh[NT / 64 + 5];
      done = true;
    }
  }
  if constexpr (!LEAN) __syncthreads();   // sh and hist are free for the caller
  *kk_eq = kk;
  return prefix + kmin;
}

// block_topk over keys held in registers: thread t owns elements [t*PT, t*PT + PT)
// of the array, element e counting when bit e of vmask is set, so the sweeps touch
// no memory.  emit(pos, e) receives the thread's local element index e.  If
// hist_cleared, hist[0, 2048) is already zero and visible to every thread.
template <int NT, int PT, bool LEAN = false, class Emit>
__device__ void block_topk_reg(const uint32_t (&key)[PT], uint64_t vmask, int k, uint32_t kmin, uint32_t kmax,
                               int* hist, int* sh, bool hist_cleared, Emit emit) {
  int kk;
  const uint32_t T = block_kth_reg<NT, PT, LEAN>(key, vmask, k, kmin, kmax, hist, sh, hist_cleared, &kk);
  // every key > T is taken plus the kk lowest-index keys equal to T; one block
  // scan of the (greater, equal) counts places the selections in index order
  int gt = 0, eq = 0;
#pragma unroll
  for (int e = 0; e < PT; e++) {
    if ((vmask >> e) & 1) {
      gt += key[e] > T;
      eq += key[e] == T;
    }
  }
  int tot;   // (LEAN: the closing barrier below orders the scan's reads before later writes)
  const int ex = block_exclusive_scan<NT, !LEAN>(gt | (eq << 13), sh, &tot);
  int pos = (ex & 0x1fff) + min(ex >> 13, kk);
  int eq_seen = ex >> 13;
#pragma unroll
  for (int e = 0; e < PT; e++) {
    if ((vmask >> e) & 1) {
      if (key[e] > T) {
        emit(pos++, e);
      } else if (key[e] == T) {
        if (eq_seen < kk) emit(pos++, e);
        eq_seen++;
      }
    }
  }
  __syncthreads();
}

// The first nv elements valid.
__device__ __forceinline__ uint64_t prefix_mask(int nv) { return nv >= 64 ? ~0ull : ((1ull << nv) - 1ull); }

}  // namespace skv
