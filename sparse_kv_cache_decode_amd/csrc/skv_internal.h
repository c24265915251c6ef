// Internal declarations of the skv library: the layer handle and kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/skv.h"

namespace skv {

constexpr int kHeadDim = 128;
constexpr int kMaxTopK = 4096;
constexpr int kSelLdsMax = 150 * 1024;   // dynamic LDS of the select kernel
constexpr int kMaxSplits = 4096;         // attention workgroups per pair
constexpr int kMaxPartials = kMaxSplits + 512;   // attention partials per pair (splits + miss tiles)
constexpr int kScoreRows = 128;          // candidate landmarks per score workgroup (bf16)
constexpr int kScoreRows8 = 256;         // the same for FP8 landmarks (the same 32 KB)
constexpr int kPartStride = kHeadDim + 4; // floats per attention partial row: o[d], m, l, 2 pad (16-B rows)
constexpr int kStaticWaves = 16;          // waves of a static-unit attention workgroup (selection launch)
constexpr int kRebuildRows = 128;        // key rows rebuilt per workgroup (128 / C missed chunks)

// Element offset of column k of row `row` of A (batch element b) in its chunk-tiled
// layout: every chunk of C rows is one run of n_kq = r_pad / 32 blocks of C x 32
// elements (k-step, then row, then the step's 32 columns), columns r .. r_pad - 1
// zero.  The rebuild's load of one k-step of a chunk's rows then reads C * 32
// contiguous elements instead of C pieces 2r bytes apart.  a_rows is a multiple of C.
constexpr int64_t a_tiled(int64_t b, int64_t a_rows, int r_pad, int C, int64_t row, int k) {
  return b * a_rows * r_pad + (row / C) * ((int64_t)C * r_pad) + (int64_t)(k >> 5) * (C * 32) + (row % C) * 32 +
         (k & 31);
}

// Everything a decode step touches, by value into the kernels.
struct DecodeArgs {
  int batch, n_kv, group, chunk, top_k, n_outlier, n_win_units, n_cand;
  int cand_stride;            // rows per pair of L and cand_map (candidate capacity)
  int n_c;                    // chunks of the pre-filled context (S / C)
  int landmark_format;        // SKV_FORMAT_BF16 or SKV_FORMAT_FP8_E5M2
  int a_format;               // the same for the rows of A
  int b_format;               // the same for B^T
  int n_new_tokens, n_new_units, max_new;   // appended tokens, their units, capacity
  int n_fold;                 // appended chunks folded into the candidates (low-rank mode)
  int64_t seq_len;
  int64_t a_rows;             // rows of A per batch element (S, plus max_new in low-rank mode, rounded
                              // up to a multiple of C)
  int nb_score, cpb;          // score workgroups per pair, candidates per workgroup
  int ncp;                    // logits row stride (n_cand rounded up to 4)
  int n_split, upw;           // attention workgroups per pair, units per workgroup
  int n_part_att;             // attention partial rows per pair (splits, then miss tiles when fused)
  int n_static;               // >0: the outliers and the exact region are attended by n_static extra
                              // workgroups per pair of the two-level selection launch (partial rows
                              // [0, n_static)); the splits then cover the slots that hit alone
  int tile_row0;              // partial row of miss tile (or miss split) 0
  int rebuild_fused;          // 1: misses attended apart from the hits (fused or overlapped rebuild)
  int miss_part_units;        // missed chunks per partial of theirs (a tile, or a split's units)
  int temporal, host_values;
  float scale;                // 1/sqrt(d)
  const double* inv_freq;     // [64]
  // inputs / state
  const uint16_t* q;          // [b][Hq][d]
  const uint16_t* L;          // [P][cand_stride][d] bf16 (bytes for FP8), first n_cand rows in use
  const int32_t* cand_map;    // [P][cand_stride]
  const uint16_t* A;          // bf16 (bytes for FP8), chunk-tiled: element a_tiled(b, a_rows, 32 n_kq, C, row, k)
  const uint16_t* Bt;         // [b][HD][r] bf16 (bytes for FP8)         // [b][Hkv*d][r]
  const uint16_t* Bst;        // [P][n_kq][128][32] bf16 B^T (widened from FP8 B) in the rebuild's stage order
  int n_kq;                   // k-steps of 32 over the rank: ceil(r / 32)
  int rank;
  const uint16_t* k_out;      // [P][O*C][d]
  const uint16_t* v_out;
  const uint16_t* k_win;      // [P][W][d]
  const uint16_t* v_win;
  const uint16_t* v_store;    // [b][Hkv][S][d] (device pointer, may map host memory)
  uint16_t* key_slots;        // [P][K][C][d]
  uint16_t* key_new;          // [P][max_new][d] post-RoPE keys of appended tokens
  uint16_t* val_new;          // [P][max_new][d] their values
  uint16_t* val_slots;        // [P][K][C][d] (host placement only)
  // temporal cache
  int32_t* slot_cand;         // [P][K]
  int32_t* slot_chunk;        // [P][K]
  uint32_t* resident;         // [P][res_words] bitmap over candidate indices
  int res_words;
  int32_t* miss_slot;         // [P][K]
  int32_t* miss_chunk;        // [P][K]
  int32_t* miss_cand;         // [P][K]
  int32_t* hit_slot;          // [P][K] slots that kept their chunk this step, ascending (K - n_miss)
  int32_t* hit_chunk;         // [P][K] the chunk id each of those slots holds
  int32_t* free_slot;         // [P][K]
  int32_t* n_miss;            // [P]
  int32_t* hits_last;         // [P]
  long long* hits_total;      // [P]
  long long* miss_total;      // [P]
  // scratch
  float* logits;              // [P][G][ncp]
  float* lse_part;            // [P][nb_score][G][2]
  float* tile_max;            // [P][n_ctiles][G] largest logit of each 16-candidate tile and head
  int n_ctiles;               // 16-candidate tiles per pair: ceil(n_cand / 16)
  int n_ctiles_cap;           // tile rows per pair of tile_max (candidate capacity / 16)
  int sel_two_level;          // 1: select2_kernel (tile keys, then the candidates of the hot tiles)
  int sel_nt, sel_tpt, sel_ipt;   // its workgroup size, tiles and level-2 items (4 candidates) per thread
  uint32_t* keys;             // [P][n_cand]
  int n_part, part_size;      // selection stage 1: candidate parts per pair and their size
  uint32_t* part_keys;        // [P][n_part][K] each part's top-K keys, ascending candidate index
  int32_t* part_idx;          // [P][n_part][K] their candidate indices
  uint32_t* merge_keys;       // [P][<= n_part / 2][K] lists of a merge-tree level
  int32_t* merge_idx;
  float* attn_part;           // [P][n_part_att][G][kPartStride]
  // outputs
  float* out;                 // [b][Hq][d]
  int32_t* chunk_ids;         // [P][K]
};

// Byte offsets of a decode step's transient scratch from a 256-byte aligned base
// (nothing in it has to start at zero: every step writes each part before it
// reads it).  Computed at build for the handle's largest candidate count.
struct TransientLayout {
  size_t logits = 0, lse_part = 0, tile_max = 0, part_keys = 0, part_idx = 0, merge_keys = 0, merge_idx = 0,
         attn_part = 0, bytes = 0;
};

inline void apply_transient(DecodeArgs& a, const TransientLayout& t, char* base) {
  a.logits = reinterpret_cast<float*>(base + t.logits);
  a.lse_part = reinterpret_cast<float*>(base + t.lse_part);
  a.tile_max = reinterpret_cast<float*>(base + t.tile_max);
  a.part_keys = reinterpret_cast<uint32_t*>(base + t.part_keys);
  a.part_idx = reinterpret_cast<int32_t*>(base + t.part_idx);
  a.merge_keys = reinterpret_cast<uint32_t*>(base + t.merge_keys);
  a.merge_idx = reinterpret_cast<int32_t*>(base + t.merge_idx);
  a.attn_part = reinterpret_cast<float*>(base + t.attn_part);
}

// One decode step of `h` (validation, then every launch on `stream`), with the
// transient scratch at `xs`: a 256-byte aligned device region of at least
// transient_bytes(h) bytes.  skv_decode_step passes the handle's own region, the
// no-allocation entry point the library's static device array.
skv_status decode_enqueue(skv_layer* h, const uint16_t* q, float* out, int32_t* chunk_ids, void* stream,
                          char* xs);
size_t transient_bytes(const skv_layer* h);

// ---- build launchers (build_kernels.hip); all enqueue on `st`
// L_full: [P][n_c][d] bf16, or bytes with fp8 (FP8 E5M2)
hipError_t launch_rope_landmark(const uint16_t* k_pre, int b, int64_t S, int H, int C,
                                const double* inv_freq, bool fp8, void* L_full, float* min_cos,
                                hipStream_t st);
hipError_t launch_outliers(const float* min_cos, int P, int n_c, int n_elig, int O,
                           uint32_t* key_scratch, int32_t* outlier_ids, hipStream_t st);
// rows of row_bytes (256 bf16, 128 FP8)
hipError_t launch_candidates(const void* L_full, const int32_t* outlier_ids, int P, int n_c,
                             int n_elig, int O, int stride, int row_bytes, void* L, int32_t* cand_map,
                             hipStream_t st);
hipError_t launch_static_gather(const uint16_t* k_pre, const uint16_t* v, const int32_t* outlier_ids,
                                int b, int64_t S, int H, int C, int O, int W, const double* inv_freq,
                                uint16_t* k_out, uint16_t* v_out, uint16_t* k_win, uint16_t* v_win,
                                hipStream_t st);
hipError_t launch_gram(const uint16_t* k_pre, int b, int64_t S, int HD, int nseg, double* partial,
                       double* gram, hipStream_t st);
int gram_segments(int b, int64_t S, int HD);
hipError_t launch_gemm_f64(const double* A, const double* B, double* C, int batch, int M, int N,
                           int K, hipStream_t st);
// C[bi] (M x N) = A[bi]^T B[bi] with A[bi] stored K x M, B[bi] K x N
hipError_t launch_gemm_f64_tn(const double* A, const double* B, double* C, int batch, int M, int N,
                              int K, hipStream_t st);
// psi [b][HD][r] fp64 -> bt = bf16(psi), or FP8 E5M2 bytes with b8 (same layout),
// each value rounded once to nearest even from the fp64 value
hipError_t launch_round_psi(const double* psi, int b, int HD, int r, bool b8, void* bt, hipStream_t st);
// bst [P][n_kq][128][32] bf16 from bt [P*128][r] (bf16, or FP8 E5M2 bytes with b8,
// widened exactly): for each k-step of 32, row n's four 8-element pieces in the
// slots the rebuild stages them to in LDS (piece s ^ ((n >> 2) & 3) in slot s),
// zero past r, so that a stage load reads 1 KB contiguous
hipError_t launch_stage_bt(const void* bt, int P, int r, int n_kq, bool b8, uint16_t* bst, hipStream_t st);
// Rows 0..S-1 of A (chunk-tiled, a_tiled with chunk C and r_pad columns, those past
// r zero) = K_b Psi_b in float64, each rounded once to
// bf16, or FP8 E5M2 bytes with fp8; psi [b][HD][r] float64
hipError_t launch_project(const uint16_t* k_pre, const double* psi, int b, int64_t S, int HD, int r, int C,
                          int64_t a_rows, bool fp8, void* A, hipStream_t st);

// n 16-bit words at p set to `value` (debug poisoning of the slot caches)
hipError_t launch_fill_u16(uint16_t* p, size_t n, uint16_t value, hipStream_t st);

// ---- decode launchers (decode_kernels.hip)
hipError_t launch_reset_cache(const DecodeArgs& a, hipStream_t st);
// t0 / t1 (optional): events that receive the kernel's own start and end
hipError_t launch_score(const DecodeArgs& a, hipStream_t st, hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr);
hipError_t launch_select(const DecodeArgs& a, hipStream_t st);
// Two-stage top-K: the candidates of a pair are cut into n_part parts whose
// top-K are taken by separate workgroups (stage 1), then merged per pair (stage 2).
void select_partition(int n_cand, int top_k, int group, int pairs, int* n_part, int* part_size);
int merge_groups(int top_k);   // part lists merged per workgroup of the merge tree
// Two-level selection: workgroup size, tiles and level-2 items per thread, or 0
// where it does not apply.
int select2_shape(int n_ctiles_cap, int top_k, int res_words, int* nt, int* tpt, int* ipt);
hipError_t launch_rebuild(const DecodeArgs& a, hipStream_t st);
// Append token t (position S + t) of every batch element: exact post-RoPE key
// and value into key_new / val_new; lowrank: also its row a' = k' Psi of A.
hipError_t launch_append(const DecodeArgs& a, const uint16_t* k_new, const uint16_t* v_new, int t, bool lowrank,
                         hipStream_t st);
// Low-rank mode, after an append that completes a chunk: the oldest exact chunk
// (combined window/appended index a.n_fold) becomes candidate a.n_cand of every
// pair, its landmark the bf16 mean of its stored keys.
hipError_t launch_fold(const DecodeArgs& a, hipStream_t st);
hipError_t launch_value_gather(const DecodeArgs& a, hipStream_t st);
hipError_t launch_attention(const DecodeArgs& a, hipStream_t st);   // separate rebuild: every slot
// One launch: tiles of missed chunks rebuilt (and, with attend_tiles, attended
// from LDS) beside the attention splits over outliers, hits and window.
hipError_t launch_tail(const DecodeArgs& a, bool attend_tiles, hipStream_t st);
// The attention over the missed chunks' slots alone (after an overlapped rebuild).
hipError_t launch_attention_misses(const DecodeArgs& a, hipStream_t st);
hipError_t launch_combine(const DecodeArgs& a, hipStream_t st);     // merge of the partials
int attn_units_per_wave(int chunk);   // 16-token tiles per wave * 16 / C

// ---- host eigensolver (eig_host.cpp)
// Top-r eigenpairs of each symmetric n x n matrix gram[bi] (row-major fp64, on the
// device), by block subspace iteration with Rayleigh-Ritz.  Every n x p product
// runs on the GPU in fp64 (launch_gemm_f64 / _tn); the host does the p x p work
// (Cholesky factors, the Rayleigh-Ritz eigenproblem).  psi receives [b][n][r] (columns =
// eigenvectors, eigenvalues descending, largest-|.| entry positive), eig [b][r].
// Returns 0 on success, 1 on non-convergence, 2 on a HIP error (err set).
int top_eigvecs(const double* gram_dev, int b, int n, int r, hipStream_t st, double* psi,
                double* eig, hipError_t* err);

}  // namespace skv
