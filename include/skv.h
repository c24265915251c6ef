/*
 * skv.h -- C ABI of the ShadowKV sparse-KV decode step for AMD MI355X (gfx950).
 *
 * The method is the one described in "ShadowKV: KV Cache in Shadows for
 * High-Throughput Long-Context LLM Inference":
 *   - pre-fill (papercache deep notes, section A2, pre-fill algorithm; paper-graph-ui
 *     summary, section 3.4 "Low-Rank Key Cache Compression via Online SVD" and
 *     "Landmark Construction and Outlier Detection"): a rank-r SVD of the
 *     pre-RoPE keys K ~ A x3 B with A shared by the KV heads, chunk-mean landmarks of
 *     the post-RoPE keys, the O chunks with the lowest in-chunk minimum cosine to
 *     their landmark kept exactly as a static outlier cache;
 *   - decode (papercache deep notes, section A2, decode algorithm; paper-graph-ui
 *     summary, section 3.4 "Decoding-Time KV Selection" and "Sparse KV
 *     Reconstruction and Overlapping Strategy"): softmax(Q L^T / sqrt(d)) per query
 *     head, maximum over each GQA group, top-K chunks per KV head, an index scan
 *     against the previous step's chunks so only misses are rebuilt
 *     (RoPE(Gather(A, I_miss) B)) and fetched, then exact attention over
 *     [outliers; selected chunks; local window; generated tokens];
 *   - generated tokens (paper-graph-ui summary, section 3.4 "Sparse KV
 *     Reconstruction and Overlapping Strategy": the assembly
 *     [K_outlier; RoPE(K_sparse); K_new] and the paragraph on the ShadowKV+
 *     extension): appended one per step, either kept exact and always attended
 *     (ShadowKV) or, once their chunk has left the local window, kept only as
 *     their projection onto the pre-fill subspace and selected and
 *     reconstructed like the context's chunks (ShadowKV+).
 *
 * Conventions shared by every entry point
 *   - Every call returns an skv_status; SKV_OK is 0.  No C++ exception crosses
 *     the ABI.  Arguments are validated before anything is enqueued; a call that
 *     fails validation leaves the handle unchanged.  A HIP failure inside a call
 *     poisons the handle: later calls on it return SKV_ERR_STATE until
 *     skv_destroy.
 *   - bf16 tensors are passed as uint16_t bit patterns, row-major, with the
 *     layouts given per argument.  "device" pointers are HIP device memory on the
 *     current device; "pinned host" pointers come from hipHostMalloc.  bf16 and
 *     float tensors start on a 16-byte boundary, int32 ones on a 4-byte boundary
 *     (every HIP allocation is 256-byte aligned); otherwise SKV_ERR_INVALID_ARG.
 *   - Query head hq uses KV head hq / G with G = n_q_heads / n_kv_heads.
 *   - Streams are passed as void* holding a hipStream_t (NULL = default stream).
 *   - A handle (one model layer) is not thread-safe; distinct handles are
 *     independent.
 *   - Environment switches read by skv_build, for tests and debugging:
 *     SKV_INJECT_FAIL="alloc:N" makes the N-th device allocation of the build
 *     report failure (SKV_ERR_OOM, everything allocated before it freed);
 *     SKV_INJECT_FAIL="hip:N" makes the N-th HIP call of the handle's later
 *     decode steps and appends report failure without being issued
 *     (SKV_ERR_HIP, then SKV_ERR_STATE); SKV_POISON_SLOTS=1 fills the slot
 *     caches with bf16 NaN at build, so that a read of a slot no step wrote
 *     shows in the output.
 */
#ifndef SKV_H
#define SKV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SKV_ABI_VERSION 8

typedef int32_t skv_status;
#define SKV_OK 0
#define SKV_ERR_INVALID_ARG 1  /* null pointer, bad enum value, wrong pointer kind */
#define SKV_ERR_SHAPE 2        /* sizes that violate the method's constraints     */
#define SKV_ERR_UNSUPPORTED 3  /* valid for the method, not implemented here      */
#define SKV_ERR_OOM 4          /* device or host allocation failed                */
#define SKV_ERR_HIP 5          /* a HIP runtime call failed                       */
#define SKV_ERR_STATE 6        /* handle poisoned by an earlier HIP failure       */
#define SKV_ERR_INTERNAL 7     /* internal invariant broken (e.g. no convergence)  */
#define SKV_ERR_SCRATCH 8      /* a decode step's transient scratch exceeds the
                                  static array of skv_decode_step_noalloc          */

/* Value placement (the value store V_CPU of the pages). */
#define SKV_VALUES_DEVICE 0    /* values stay in HBM and are read by chunk id      */
#define SKV_VALUES_HOST 1      /* values in pinned host memory, missed chunks are
                                  gathered over PCIe on a side stream that overlaps
                                  the key rebuild                                   */

/* Storage formats of the landmarks (chunk means), of the rows of A and of B.
 * FP8 follows the precision study of the paper-graph-ui summary of ShadowKV
 * (section 5, Tables 9 and 10), which runs the method in torch.float8_e5m2.
 * The landmarks are the stream that dominates a decode step's bytes and A the
 * largest store (S x r per batch element); B is about 1/100 of A's size and
 * enters every rebuilt key (the summary's section 7 expects it to need more
 * precision than A), so each format is chosen on its own. */
#define SKV_FORMAT_BF16 0      /* bfloat16                                           */
#define SKV_FORMAT_FP8_E5M2 1  /* FP8 E5M2 (1 sign, 5 exponent bits with bias 15, 2
                                  mantissa bits, the torch.float8_e5m2 format), each
                                  value rounded once to nearest even from fp32.
                                  Landmarks (128 bytes each) are widened to fp16
                                  exactly and scored with q in fp16 (q's bf16 values
                                  are exact there in fp16's normal range,
                                  2^-14 <= |q| <= 65504; larger ones saturate at
                                  +-65504, smaller ones lose bits down to fp16's
                                  subnormal step 2^-24); rows of A (r bytes each) and B are
                                  widened to bf16 exactly for the key rebuild and
                                  the low-rank append                              */

/* How appended (generated) tokens keep their keys. */
#define SKV_NEW_EXACT 0        /* post-RoPE key kept exactly (ShadowKV)             */
#define SKV_NEW_LOWRANK 1      /* ShadowKV+: a' = k' Psi (Psi^T = the stored B) joins
                                  A; the token stays exact while it is in the local
                                  window, then its chunk becomes a candidate that is
                                  reconstructed as RoPE(a' Psi^T) when selected      */

/* How a decode step meets the chunks that missed the temporal cache (the summary's
 * "Sparse KV Reconstruction and Overlapping Strategy", section 3.4: the key
 * reconstruction of the selected chunks overlapped with the rest of the step). */
#define SKV_REBUILD_AUTO 0     /* FUSED with values in HBM, SEPARATE with host values  */
#define SKV_REBUILD_FUSED 1    /* one launch: each tile of missed chunks is rebuilt and
                                  attended from on-chip memory by one workgroup (and
                                  stored to the key slots for later hits, with the
                                  temporal cache on), while the other workgroups of
                                  the launch attend to the slots that hit; the
                                  outliers and the window are attended there too, or,
                                  with the two-level selection, by extra workgroups
                                  of the selection launch; values in HBM only       */
#define SKV_REBUILD_SEPARATE 2 /* a rebuild launch refreshes the missed key slots, then
                                  an attention launch reads every slot               */
#define SKV_REBUILD_OVERLAP 3  /* one launch rebuilds the missed chunks into their
                                  slots beside the attention over the outliers, the
                                  slots that hit and the window; a second attends to
                                  the missed slots; values in HBM only              */

/* How the top-K of the chunk scores is found (the same chunks either way). */
#define SKV_SELECT_AUTO 0      /* two levels where they fit: the largest score of every
                                  16-chunk tile first (from per-tile maxima of the
                                  logits), the K-th largest of those as a threshold,
                                  then the top-K among the chunks of the tiles that
                                  reach it (one workgroup per KV head and batch
                                  element, for K <= 512); a full pass otherwise     */
#define SKV_SELECT_FULL 1      /* a pass over every candidate's score                */

/*
 * Shape and budget of one layer.
 *   head_dim must be 128.  seq_len % chunk == 0, chunk in {4, 8, 16},
 *   window % chunk == 0, G in {1, 2, 4, 8, 16}, rank % 16 == 0,
 *   1 <= rank <= min(seq_len, n_kv_heads * head_dim), n_kv_heads * head_dim <= 2048,
 *   n_cand = seq_len/chunk - n_outlier - window/chunk, 1 <= top_k <= n_cand, top_k <= 4096.
 *   max_new_tokens >= 0 is the capacity for appended tokens (skv_append_token);
 *   new_token_mode is SKV_NEW_EXACT or SKV_NEW_LOWRANK; landmark_format, a_format
 *   and b_format are SKV_FORMAT_BF16 or SKV_FORMAT_FP8_E5M2; rebuild_mode is one of
 *   the SKV_REBUILD_* values, select_mode one of the SKV_SELECT_* values.  An unknown
 *   enum value gives SKV_ERR_INVALID_ARG.
 */
typedef struct skv_config {
  int32_t batch;           /* b                                                   */
  int32_t n_q_heads;       /* H_q                                                 */
  int32_t n_kv_heads;      /* H_kv                                                */
  int32_t head_dim;        /* d (128)                                             */
  int64_t seq_len;         /* S: context tokens held by the cache                 */
  int32_t rank;            /* r: SVD rank of the pre-RoPE keys                    */
  int32_t chunk;           /* C: tokens per chunk / landmark                      */
  int32_t top_k;           /* K: chunks selected per KV head and step             */
  int32_t n_outlier;       /* O: outlier chunks per KV head                       */
  int32_t window;          /* W: last W context tokens kept exact (local window)  */
  int32_t value_placement; /* SKV_VALUES_DEVICE or SKV_VALUES_HOST                */
  double rope_theta;       /* RoPE base (rotate-half pairing (i, i + d/2))        */
  int32_t temporal_cache;  /* 1: rebuild/fetch only chunks missed vs the previous
                              step; 0: rebuild every selected chunk every step     */
  int32_t landmark_format; /* SKV_FORMAT_BF16 or SKV_FORMAT_FP8_E5M2              */
  int32_t max_new_tokens;  /* capacity for generated tokens (0: none)             */
  int32_t new_token_mode;  /* SKV_NEW_EXACT or SKV_NEW_LOWRANK                     */
  int32_t a_format;        /* SKV_FORMAT_BF16 or SKV_FORMAT_FP8_E5M2 (rows of A,
                              also those appended in SKV_NEW_LOWRANK mode)        */
  int32_t b_format;        /* SKV_FORMAT_BF16 or SKV_FORMAT_FP8_E5M2 (B = Psi^T)   */
  int32_t rebuild_mode;    /* SKV_REBUILD_AUTO, _FUSED, _SEPARATE or _OVERLAP; FUSED
                              or OVERLAP with SKV_VALUES_HOST gives
                              SKV_ERR_UNSUPPORTED                                  */
  int32_t select_mode;     /* SKV_SELECT_AUTO or SKV_SELECT_FULL                   */
} skv_config;

typedef struct skv_layer skv_layer;   /* opaque; owns all derived state */

/* Temporal-cache counters (summed over the b * n_kv_heads pairs). */
typedef struct skv_stats {
  int64_t steps;          /* decode steps since build or the last reset             */
  int64_t last_hits;      /* |I_t & I_{t-1}| of the last step                       */
  int64_t last_misses;    /* chunks rebuilt (and, for host values, fetched) last step */
  int64_t total_hits;     /* hits over steps 1.. since build/reset                  */
  int64_t total_misses;   /* misses over steps 1.. since build/reset                */
  double last_alpha;      /* last_hits / (pairs * top_k); 0 for the first step      */
  double mean_alpha;      /* total_hits / (pairs * top_k * (steps - 1))             */
  int64_t last_host_bytes;/* value bytes gathered from pinned host memory last step */
  int64_t new_tokens;     /* generated tokens appended since build                  */
} skv_stats;

/*
 * Host copies of the built state, for inspection and parity checks.  Any
 * pointer may be NULL to skip that tensor.  Sizes (elements):
 *   A          bf16 [b][S][r]             (bf16 values also with FP8 storage)
 *   B          bf16 [b][H_kv][r][d]       (the per-head right factor; bf16 values
 *                                          also with FP8 storage)
 *   landmarks  bf16 [b][H_kv][n_cand][d]  (bf16 values also with FP8 storage, which
 *                                          they hold exactly; candidate chunks of the pre-filled
 *                                          context, ascending chunk id; chunks
 *                                          folded in by skv_append_token are not
 *                                          exported)
 *   cand_ids   int32 [b][H_kv][n_cand]    (chunk id of each landmark row)
 *   outlier_ids int32 [b][H_kv][O]        (ascending)
 *   k_outlier, v_outlier bf16 [b][H_kv][O*C][d]   (post-RoPE keys, values)
 *   k_window,  v_window  bf16 [b][H_kv][W][d]
 *   min_cos    float [b][H_kv][S/C]       (in-chunk minimum cosine, every chunk)
 *   eigvals    double [b][r]              (largest eigenvalues of K_b^T K_b, i.e.
 *                                          squared singular values, descending)
 */
typedef struct skv_state_host {
  uint16_t* A;
  uint16_t* B;
  uint16_t* landmarks;
  int32_t* cand_ids;
  int32_t* outlier_ids;
  uint16_t* k_outlier;
  uint16_t* v_outlier;
  uint16_t* k_window;
  uint16_t* v_window;
  float* min_cos;
  double* eigvals;
} skv_state_host;

/*
 * skv_build -- pre-fill of one layer (pre-fill algorithm of the papercache notes,
 * section A2; paper-graph-ui summary, section 3.4).
 *   k_pre : device, bf16 [b][S][H_kv*d]; row t holds the pre-RoPE keys of token
 *           position t, heads concatenated.  Only read during the call.
 *   v     : bf16 [b][H_kv][S][d]; device memory for SKV_VALUES_DEVICE, pinned host
 *           memory for SKV_VALUES_HOST.  BORROWED: it must stay valid and unchanged
 *           until skv_destroy (the value store is never copied whole).
 *   stream: work is enqueued there; the call returns after it has completed
 *           (host-synchronous).
 *   out   : receives the new handle; set to NULL on any failure.
 * Computes post-RoPE keys (angles in float64), landmarks, per-chunk min-cosine,
 * outliers among the non-window chunks (lowest min-cos, lower id on ties), the
 * exact outlier and window K/V, and the rank-r factors from the top-r
 * eigenvectors of K_b^T K_b (fp64 Gram on the GPU, subspace iteration with
 * Rayleigh-Ritz in fp64), with each right singular vector's largest-magnitude
 * entry made positive.  Stored state is bf16 (round-to-nearest-even).
 * Errors: INVALID_ARG, SHAPE, UNSUPPORTED, OOM, HIP, INTERNAL (eigensolver did
 * not converge).
 */
skv_status skv_build(const skv_config* cfg, const uint16_t* k_pre, const uint16_t* v,
                     void* stream, skv_layer** out);

/*
 * skv_decode_step -- one decode step of one layer (decode algorithm of the
 * papercache notes, section A2; paper-graph-ui summary, section 3.4).
 *   q         : device, bf16 [b][H_q][d], post-RoPE queries of one new token.
 *   out       : device, float [b][H_q][d], attention output.
 *   chunk_ids : device, int32 [b][H_kv][K]: the selected chunk ids, ascending.
 *   stream    : every kernel is enqueued on it (plus an internal side stream
 *               joined back into it for host values); no host synchronisation,
 *               so the call can be captured in a HIP graph.  Outputs are valid
 *               once the stream has completed.
 * Selection uses fp32 scores; a chunk's score is max_g(logit_g/sqrt(d) - LSE_g),
 * the log of the pages' max over the group of softmax probabilities, compared as
 * the fp32 value score - 1 (scores within one fp32 spacing of it, about 1e-7,
 * tie); ties go to the lower chunk id.  The attention accumulates in fp32 with
 * the softmax weights carried at 16 bits of precision (bf16 hi + lo parts).
 * Errors: INVALID_ARG (null, misaligned or non-device pointer; checked before
 * any launch), STATE, HIP.
 */
skv_status skv_decode_step(skv_layer* h, const uint16_t* q, float* out, int32_t* chunk_ids,
                           void* stream);

/*
 * skv_append_token -- append one generated token to the layer (paper-graph-ui
 * summary, section 3.4 "Sparse KV Reconstruction and Overlapping Strategy": the
 * generated tokens' K_new, V_new close the assembled cache; its ShadowKV+
 * paragraph: a new pre-RoPE key k' is kept as k' Psi and reconstructed as
 * (k' Psi) Psi^T when needed).
 *   k_new : device, bf16 [b][H_kv*d], the new token's pre-RoPE keys, heads
 *           concatenated; its position is seq_len + (tokens appended so far).
 *   v_new : device, bf16 [b][H_kv][d], its values.
 *   stream: enqueued, no host synchronisation.  Both inputs are only read by the
 *           enqueued work (they may be reused once the stream has passed it).
 * SKV_NEW_EXACT: the key RoPE(k') (bf16) and the value are kept, and every later
 * decode step attends to all appended tokens after the local window; landmarks,
 * outliers and the selection cover the pre-filled context only.
 * SKV_NEW_LOWRANK (ShadowKV+): a' = k' Psi (fp32 accumulation over the stored
 * bf16 Psi^T, rounded to the format of A) becomes row seq_len + t of A, and RoPE(k') is kept
 * exactly while the token is in the exact region: the last `window` tokens of the
 * completed chunks plus the chunk being filled.  When an append completes a chunk,
 * the oldest exact chunk leaves that region and becomes the last candidate of
 * every pair (never an outlier): its landmark is the mean of its stored exact
 * keys rounded to the landmark format, its chunk id (seq_len - window)/chunk + (chunks completed so far)
 * - 1; from the next decode step it is scored, selected, rebuilt from A and its
 * values read (from the value store, or from the appended values) like a
 * context chunk.
 * Errors: INVALID_ARG (null, misaligned or non-device pointer), SHAPE (capacity
 * max_new_tokens reached), STATE, HIP.
 */
skv_status skv_append_token(skv_layer* h, const uint16_t* k_new, const uint16_t* v_new, void* stream);

/*
 * skv_decode_step_noalloc -- for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The same step, arguments, outputs and errors as skv_decode_step,
 * but the step's transient scratch (logits, log-sum-exp partials, selection
 * lists, attention partials) lives in a static device array of the library,
 * SKV_NOALLOC_SCRATCH_BYTES per device, held until the process ends, instead of
 * the handle's own region.  The call allocates nothing.
 *   - A handle whose transient scratch is larger gives SKV_ERR_SCRATCH before
 *     anything is enqueued (the transient scratch is about
 *     4 * b * n_q_heads * (n_cand + 4) bytes of logits plus lists and attention
 *     partials: 18 MB for a layer of batch 8, 32 query heads, 15 310 candidates).
 *   - Every call on one device uses that device's one array: calls whose work
 *     overlaps on a device (other streams, other threads) race on it and must be
 *     ordered by the caller.  Nothing in the array needs clearing between calls.
 *   - Errors: as skv_decode_step, plus SCRATCH; HIP if the array's address
 *     cannot be looked up.
 */
#define SKV_NOALLOC_SCRATCH_BYTES (64 << 20)
skv_status skv_decode_step_noalloc(skv_layer* h, const uint16_t* q, float* out, int32_t* chunk_ids,
                                   void* stream);

/* Temporal-cache counters; synchronises with the last stream used. */
skv_status skv_get_stats(const skv_layer* h, skv_stats* stats);

/* Forget the previous selection: the next step rebuilds every selected chunk. */
skv_status skv_reset_temporal_cache(skv_layer* h);

/* Synchronous copy of the built state into caller-owned host buffers. */
skv_status skv_export_state(const skv_layer* h, const skv_state_host* dst);

/*
 * Per-phase device timing.  With capacity > 0 the next `capacity` decode steps
 * record HIP events on the decode stream (and on the side stream around the host
 * value gather); capacity 0 stops recording.  The score phase is the score
 * kernel's own start and end, recorded by its launch (hipExtLaunchKernel); the
 * other phases run from one event to the next, each recorded after its kernels.
 * No host synchronisation.
 */
#define SKV_PHASE_SCORE 0         /* landmark GEMV: logits + per-head LSE partials */
#define SKV_PHASE_SELECT 1        /* LSE, chunk scores, top-K, index scan          */
#define SKV_PHASE_REBUILD 2       /* key rebuild + RoPE of the missed chunks; with
                                     the fused rebuild, the whole fused launch
                                     (rebuild and attention of the misses, and
                                     the attention over everything else)          */
#define SKV_PHASE_VALUE_GATHER 3  /* host-value gather (side stream, overlapped)   */
#define SKV_PHASE_ATTENTION 4     /* split-K attention + merge of the partials; with
                                     the fused rebuild, the merge alone           */
#define SKV_NUM_PHASES 5
skv_status skv_set_timing(skv_layer* h, int32_t capacity);

/* Sums of the recorded phase durations in milliseconds (phase_ms[SKV_NUM_PHASES])
 * and the number of recorded steps; synchronises with the recorded streams. */
skv_status skv_get_timing(const skv_layer* h, double* phase_ms, int64_t* steps);

/* Release everything the handle owns (never the borrowed value store). NULL is ok. */
void skv_destroy(skv_layer* h);

/* Static description of a status code. */
const char* skv_status_string(skv_status s);

/* SKV_ABI_VERSION of the loaded library. */
int32_t skv_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SKV_H */
