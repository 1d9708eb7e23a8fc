// Internal interface between the C-ABI layer (kd_api.cpp) and the kernels.
// Every launcher enqueues on the given stream and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kd {

constexpr int kTileN = 256;      // vocabulary columns per tile (top-K kernels, dW)
constexpr int kTileNFull = 128;  // vocabulary columns per tile (dual-accumulator kernels)
constexpr int kTileM = 256;      // token rows per tile

// The direct-load path addresses each operand with 32-bit offsets.
inline bool fits32(int64_t bytes) { return bytes < (int64_t(1) << 32) - 65536; }

// Per-row teacher data of the top-K loss, written by the prep kernel for
// every valid row t (row-major [T][KE], sorted by vocabulary index; KE is K,
// or K + 1 when the label of a cross-entropy term is one more entry).
struct TopkRowData {
  int2* pair;       // (vocabulary index, weight bits), ascending index
  uint16_t* perm;   // original position k of each sorted entry (K: the label)
  float* ent;       // [T] sum_k w_k log p_k (the teacher-entropy term)
  float4* rowc;     // [T] (log2(e) / tau_t, 1 / tau_t, mass, log2(mass)) of row t
  float* zpair;     // nullable: the forward's logit at each sorted entry (zeroed by the prep), for z_topk
};

// Optional parts of the top-K loss, as the prep kernel applies them.
struct TopkPrepOpts {
  const float* tau_rows;     // nullable [T]: per-row temperature
  const float* teacher_lse;  // nullable [T]: partial mass, p = exp(A / tau - teacher_lse)
  const int32_t* labels;     // nullable [T]: labels of the cross-entropy term
  float beta;                // weight of the cross-entropy term (labels set)
  float rev;                 // weight r of the reverse KL: the forward-KL weights are scaled by 1 - r
  float c2, inv_tau;         // log2(e) / tau and 1 / tau of the scalar temperature
  int32_t v0, vs;            // columns [v0, v0 + vs) of a vocabulary shard of W (vs = 0: the whole head)
  int32_t* bad;              // nullable: counts the cached indices and labels of valid rows outside [0, V)
  int32_t V;                 // the vocabulary size the check uses
};

struct Compact {
  int32_t* rows;   // [T] original row of each valid row, in order
  int32_t* count;  // [1] number of valid rows
};

// Elementwise passes that write a dZ chunk: a block of 256 threads covers
// kEwRows rows and one of at most kEwRanges ranges of the rows' column tiles,
// a tile being 1 KB of dZ per row (512 bf16 or 256 fp32 columns).  Each wave
// reads 4 of the rows, 16 bytes of dZ's columns per lane (one coalesced access
// per row and operand); the tile goes through LDS so that each wave then
// writes 16 rows of one 64-byte piece: a contiguous kilobyte of the panels.
constexpr int kEwRows = 16;
constexpr int kEwRanges = 16;
inline int ew_ranges(int elem, int64_t V) {
  const int64_t tiles = (V * elem + 1023) / 1024;
  return (int)(tiles < kEwRanges ? tiles : kEwRanges);
}

// ---------------------------------------------------------------- small kernels
hipError_t launch_compact(const uint8_t* mask, int64_t T, Compact c, hipStream_t st);
hipError_t launch_topk_prep(const float* logits, const int32_t* idx, const uint8_t* mask, int64_t T, int64_t K,
                            int64_t KE, const TopkPrepOpts& o, TopkRowData rd, float* z_topk, hipStream_t st);
// z_topk of compacted rows [jb, je) from the logits the forward gathered at
// the sorted entries (rd.zpair): entry i of row t goes to z_topk[t][perm[i]]
// (the label entry, perm == Kz, nowhere).
hipError_t launch_topk_zpermute(const TopkRowData& rd, Compact c, int64_t T, int64_t KE, int64_t Kz, float* z_topk,
                                int64_t jb, int64_t je, hipStream_t st);
// KL mixing on the cached entries, for compacted rows [jb, je): each row's
// reverse KL between the student and the teacher restricted to the K entries
// and renormalised there, from z_topk [T,K] and the cached logits.  kl
// (nullable) gains wr * RKL; with upd, the row's support weights become
// w - wr * q~_k (log q~_k - log p^_k - RKL), so that a dZ pass scattering
// them adds the reverse gradient.  Needs the prep's per-row constants.
hipError_t launch_topk_reverse(const float* z_topk, const float* logits, Compact c, int64_t T, int64_t K,
                               int64_t KE, float wr, TopkRowData rd, float* kl, bool upd, int64_t jb, int64_t je,
                               hipStream_t st);
// Merges the split partials of compacted rows [jb, je) (partial row p holds
// compacted row jb + p) into kl and lse; with zero_masked, also zeroes kl and
// lse of every masked row.
hipError_t launch_topk_combine(const float* part, int S, int64_t part_stride, Compact c, const uint8_t* mask,
                               TopkRowData rd, int64_t T, float* kl, float* lse, int64_t jb, int64_t je,
                               bool zero_masked, hipStream_t st);
// A vocabulary shard's forward: merges the split partials like
// launch_topk_combine but writes the row's exchange record instead of kl and
// lse: rec[t] = (m2, l, x / tau_t, 0) (base-2 max and sum over the shard's
// columns, the shard's cross term) and trow[t] = (entropy term, mass); with
// zero_masked, both are zero on masked rows.
hipError_t launch_topk_shard_record(const float* part, int S, int64_t part_stride, Compact c, const uint8_t* mask,
                                    TopkRowData rd, int64_t T, float4* rec, float2* trow, int64_t jb, int64_t je,
                                    bool zero_masked, hipStream_t st);
// kl and lse of every row from R shards' records rec [R][T] and trow [T].
hipError_t launch_topk_shard_combine(const float4* rec, int R, int64_t T, const float2* trow, const uint8_t* mask,
                                     float* kl, float* lse, hipStream_t st);
// A full-vocabulary shard's forward: row t's split partials merged into its
// record rec[2t], rec[2t + 1] = (ms, ls, mt, lt), (R, R2, 0, 0).
hipError_t launch_full_shard_record(const float* part, int S, int64_t part_stride, Compact c, const uint8_t* mask,
                                    int64_t T, float4* rec, int64_t jb, int64_t je, bool zero_masked,
                                    hipStream_t st);
// kl, both log-normalisers and kl_rev of every row from R shards' records
// rec [R][T][2] (float4 pairs).
hipError_t launch_full_shard_combine(const float4* rec, int R, int64_t T, const uint8_t* mask, float r, float* kl,
                                     float* lse_s, float* lse_t, float* kl_rev, hipStream_t st);
// kl = (1 - r) KL(p||q) + r KL(q||p); kl_rev (nullable) gets KL(q||p).
hipError_t launch_full_combine(const float* part, int S, int64_t part_stride, Compact c, const uint8_t* mask,
                               int64_t T, float r, float* kl, float* lse_s, float* lse_t, float* kl_rev, int64_t jb,
                               int64_t je, bool zero_masked, hipStream_t st);
// H^T of one chunk of compacted rows: out[j][i] = H[rows[c0 + i]][j] for
// i < valid rows of the chunk, 0 up to C; out is [d][C] in panels of d rows
// (piece p of row j at (p d + j) * 64 bytes).
hipError_t launch_gather_transpose(const void* H, int elem, int64_t d, Compact c, int64_t c0, int64_t C, void* out,
                                   hipStream_t st);
// The rows of one chunk of compacted rows (row_bytes each, a multiple of 16)
// in panels of C rows: byte b of row rows[c0 + i] at (b / 64 * C + i) * 64 +
// b % 64, for i < valid rows of the chunk.  The tiles read their
// k-contiguous operand from these panels.
hipError_t launch_gather_panels(const void* H, int64_t row_bytes, Compact c, int64_t c0, int64_t C, void* out,
                                hipStream_t st);
// dH[rows[c0 + i]] = sum_s part[s][i] (converted to the element type)
// dH's vocabulary contraction takes the direct-load ring for bf16 when V is a
// multiple of 32 (whole 64-byte stages of W's rows); for V not a multiple of
// 128 the ring runs over V rounded up to 128, so the dZ chunk's columns from V
// to ldz must hold zeros (dz_tail_bytes of them, in whole panel pieces, at
// dz_tail_offset).
inline bool dh_direct(int elem, int64_t V) { return elem == 2 && V % 32 == 0; }
inline int64_t dz_tail_offset(int64_t C, int64_t V) { return V / 32 * C * 64; }
inline int64_t dz_tail_bytes(int64_t C, int64_t V, int64_t ldz) { return (ldz - V) / 32 * C * 64; }
hipError_t launch_reduce_dh(const float* part, int S, int64_t C, int64_t d, Compact c, int64_t c0, void* dH,
                            int elem, hipStream_t st);
hipError_t launch_zero_masked_rows(const uint8_t* mask, int64_t T, int64_t row_bytes, void* out, hipStream_t st);
// Zeroes `bytes` bytes at p in whole 16-byte units (a remainder below 16 is
// left as it is): p 16-byte aligned, bytes normally a multiple of 16.
hipError_t launch_fill_zero(void* p, int64_t bytes, hipStream_t st);

// ---------------------------------------------------------------- top-K tiles
struct TopkFwdArgs {
  const char* Hp;  // rows [c0, c0 + C) of H in panels of C rows (launch_gather_panels)
  const char* W;  // [d][V]
  Compact c;
  TopkRowData rd;
  float* z_topk;  // nullable
  float* part;    // [S][part_stride][4], row p of a split is compacted row part_row0 + p
  int64_t part_stride, part_row0;
  int64_t c0, C;  // compacted rows [c0, c0 + C) (all rows: 0, T)
  float* zout;    // nullable: the logits of those rows, fp32 [C][ldz]
  int64_t ldz;
  int64_t T, d, V;
  int64_t K;      // entries per row of the pair arrays
  int64_t Kz;     // width of z_topk (the cached entries; a label entry has perm == Kz)
  int nrb, S, ntiles;
  int group;  // row blocks per raster group (grouped_coords)
};
hipError_t launch_topk_fwd(int elem, const TopkFwdArgs& a, hipStream_t st);

struct TopkDzArgs {
  const char* Hp;  // rows [c0, c0 + C) of H in panels of C rows
  const char* W;
  Compact c;
  TopkRowData rd;
  const float* lse;
  const float* g;
  char* dz;        // [C][ldz] chunk of dZ, in panels of C rows (panel_off)
  int64_t ldz;     // padded vocabulary (multiple of the tile width)
  int64_t c0, C;   // first compacted row of the chunk, chunk capacity
  int64_t T, d, V, K;  // K: entries per row of the pair arrays
  int nrb, S, ntiles;
  int group;  // row blocks per raster group (grouped_coords)
};
hipError_t launch_topk_dz(int elem, const TopkDzArgs& a, hipStream_t st);

// dZ of a chunk from its stored fp32 logits (no recompute):
// dz[i][v] = (g/tau) (mass 2^(z c2 - L2) - sum of w over hits) for the
// chunk's valid rows i and v < V; zero for the chunk's other rows.
struct TopkDzFromZArgs {
  const float* z;    // [C][ldz]
  char* dz;          // [C][ldz], element type, in panels of C rows
  int64_t ldz;
  Compact c;
  int64_t c0, C, V, K;  // K: entries per row of the pair arrays
  TopkRowData rd;
  const float* lse;
  const float* g;
};
hipError_t launch_topk_dz_from_z(int elem, const TopkDzFromZArgs& a, hipStream_t st);

// ---------------------------------------------------------------- full-vocabulary tiles
struct FullFwdArgs {
  const char* Hp;   // rows [c0, c0 + C) of H in panels of C rows
  const char* Ws;   // [d][V]
  const char* Htp;  // rows [c0, c0 + C) of Ht in panels of C rows
  const char* Wt;  // [dt][V]
  Compact c;
  float* part;     // [S][part_stride][8], row p of a split is compacted row part_row0 + p
  int64_t part_stride, part_row0;
  int64_t c0, C;   // compacted rows [c0, c0 + C) (all rows: 0, T)
  int64_t T, d, dt, V;
  int nrb, S, ntiles;
  int group;  // row blocks per raster group (grouped_coords)
  float c2;               // log2(e) / tau
  const float* tau_rows;  // nullable [T]: per-row temperature, replaces tau
};
hipError_t launch_full_fwd(int elem, const FullFwdArgs& a, hipStream_t st);

// Per-row mixing of the backward: dZ = (g/tau) [(1 - r)(q - p) + r q (log q - log p - KLr)].
struct FullMix {
  const float* tau_rows;  // nullable [T]
  const float* kl_rev;    // [T] KL(q||p) of each row (read when r > 0)
  float r;                // weight of the reverse KL
};

struct FullDzArgs {
  const char* Hp;   // rows [c0, c0 + C) of H in panels of C rows
  const char* Ws;
  const char* Htp;  // rows [c0, c0 + C) of Ht in panels of C rows
  const char* Wt;
  Compact c;
  const float* lse_s;
  const float* lse_t;
  const float* g;
  char* dz;  // [C][ldz] chunk of dZ, in panels of C rows
  int64_t ldz, c0, C;
  int64_t T, d, dt, V;
  int nrb, S, ntiles;
  int group;  // row blocks per raster group (grouped_coords)
  float c2, inv_tau;
  FullMix mix;
};
hipError_t launch_full_dz(int elem, const FullDzArgs& a, hipStream_t st);

// ---------------------------------------------------------------- full vocabulary, single call
// The single call runs each head through the top-K forward tiles (no cached
// entries, logits kept) and then one elementwise pass over the chunk's two
// stored logit arrays.  Per-row constants of those tiles: rowc[t] =
// (log2(e) / tau_t, 1 / tau_t, 1, 0) for every valid row.
hipError_t launch_full_rowc(Compact c, int64_t T, const float* tau_rows, float c2, float inv_tau, float4* rowc,
                            hipStream_t st);
// lse_s, lse_t of compacted rows [jb, je) from the student's and teacher's
// split partials (m2, l, -, -), partial row p = compacted row jb + p; with
// zero_masked, also zeroes kl, lse_s, lse_t and kl_rev (nullable) of masked rows.
hipError_t launch_full_lse_combine(const float* part_s, const float* part_t, int S, int64_t part_stride, Compact c,
                                   const uint8_t* mask, int64_t T, float* kl, float* lse_s, float* lse_t,
                                   float* kl_rev, int64_t jb, int64_t je, bool zero_masked, hipStream_t st);

// Elementwise pass over a chunk's stored fp32 logits (both heads): per chunk
// row i and column range b (ew_ranges), terms[i][b] = (sum p (yt - ys),
// sum q (ys - yt)) in base 2 with the final log-normalisers, and (dz set) dZ
// as the recomputing tile's epilogue writes it; dZ is zero on rows past the
// chunk's valid rows.
struct FullFromZArgs {
  const float* zs;   // [C][ldz]
  const float* zt;   // [C][ldz]
  int64_t ldz;
  char* dz;          // nullable: [C][ldz], element type, in panels of C rows
  float2* terms;     // nullable: [C][nblk]
  int nblk;
  Compact c;
  int64_t c0, C, V;
  const float* lse_s;
  const float* lse_t;
  const float* g;
  float c2, inv_tau;
  FullMix mix;
};
int full_from_z_blocks(int elem, int64_t V);
hipError_t launch_full_from_z(int elem, const FullFromZArgs& a, hipStream_t st);
// kl (and kl_rev, nullable) of compacted rows [jb, je) from the pass's terms.
hipError_t launch_full_kl_from_terms(const float2* terms, int nblk, Compact c, const float* lse_s,
                                     const float* lse_t, float r, float* kl, float* kl_rev, int64_t jb, int64_t je,
                                     hipStream_t st);

// ---------------------------------------------------------------- gradient contractions
// part[s][i][j] = sum over the s-th vocabulary range of dz[i][v] * W[j][v]
struct DhArgs {
  const char* dz;  // [C][ldz] in panels of C rows
  const char* W;   // [d][V]
  float* part;     // [S][C][d]
  const int32_t* count;
  int64_t c0, C, ldz, d, V;
  int nrb, ncb, S;
  int group;
};
hipError_t launch_dh(int elem, const DhArgs& a, hipStream_t st);

// dW[j][v] (+)= sum_i hT[j][i] * dz[i][v]
struct DwArgs {
  const char* hT;  // [d][C] in panels of d rows
  const char* dz;  // [C][ldz] in panels of C rows
  float* dW;       // [d][V]
  const int32_t* count;
  int64_t c0, C, ldz, d, V;
  int nrb, ncb;
  int group;
  int accumulate;
};
hipError_t launch_dw(int elem, const DwArgs& a, hipStream_t st);

}  // namespace kd
