// Top-K KL tiles: forward (log Z + gather) and backward dZ (recompute).
//
// "Efficient Knowledge Distillation for LLMs: Offline Top-K Logits and a Fused
// Chunked KL Loss", §3 "Offline distillation": with a cached top-K teacher only
// log Z needs the whole vocabulary; the teacher terms and the cross term use
// the K cached entries.  §3 "Fused chunked KL": the output projection is part
// of the loss, logit tiles are discarded after use, and the backward pass
// recomputes them.
//
// Grid: (valid-row block of 256) x (vocabulary split).  A workgroup walks the
// 256-wide vocabulary tiles of its split in ascending order; each tile is
// Z = H_rows . W[:, tile] on matrix cores.  The tile is then staged through LDS
// in four rounds of 2 x 32 columns (one 32-column block from each wave column
// half) and read back one row per thread:
//   forward  : running base-2 max / sum per row, plus the index-match gather.
//              The row's cached indices are sorted, so two cursors (one per
//              128-column half of the tile) walk them in step with the rounds
//              and pick the hits out of LDS.
//   backward : dZ = (g/tau) (2^(y - L2) - sum of p over hits), written in the
//              input dtype to the chunk's dZ buffer.
#include <climits>

#include "kd_gemm.h"
#include "kd_launch.h"
#include "kd_main.h"

namespace kd {

namespace {

constexpr int kBN = kTileN;

// First sorted position at or after `from` whose index is >= v.
__device__ inline int seek(const int32_t* idx, int K, int from, long v) {
  int lo = from, hi = K;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if ((long)idx[mid] < v) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// Per-thread row state shared by the forward and backward epilogues.
struct RowCursor {
  const int32_t* idx;
  const float* p;
  int K;
  int cur[2];   // sorted positions for the lower / upper 128 columns of a tile
  long nxt[2];  // index at cur (LONG_MAX past the end)

  __device__ inline long at(int c) const { return c < K ? (long)idx[c] : LONG_MAX; }
  // entering tile [n0, n0 + 256): cur[0] already points at the first index >= n0
  __device__ inline void enter_tile(long n0) {
    cur[1] = seek(idx, K, cur[0], n0 + 128);
    nxt[0] = at(cur[0]);
    nxt[1] = at(cur[1]);
  }
  __device__ inline void leave_tile() { cur[0] = cur[1]; }
};

struct FwdRow {
  RowCursor rc;
  const uint16_t* perm;
  float* ztk;  // z_topk row (nullable)
  float m2, l, x;
  bool rv;

  // 32 columns [cb, cb + 32) of this row, staged in st; V bounds the valid ones
  __device__ inline void consume(StPair st, long cb, long V, int half, float c2) {
    if (!rv) return;
    const int nv = (int)max(0L, min(32L, V - cb));
    if (nv == 0) return;
    const int r = threadIdx.x;
    // two passes over the staged row: block maximum, then the scaled sum
    float cm = -INFINITY;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (4 * j < nv) {
        const float4 f = st_read4(st, r, j);
        cm = fmaxf(cm, fmaxf(fmaxf(f.x, f.y), fmaxf(f.z, f.w)));
      }
    }
    const float cmy = cm * c2;
    if (cmy > m2) {
      l *= fast_exp2(m2 - cmy);
      m2 = cmy;
    }
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (4 * j < nv) {
        const float4 f = st_read4(st, r, j);
        sum += fast_exp2(fmaf(f.x, c2, -m2)) + fast_exp2(fmaf(f.y, c2, -m2)) + fast_exp2(fmaf(f.z, c2, -m2)) +
               fast_exp2(fmaf(f.w, c2, -m2));
      }
    }
    l += sum;
    // index-match gather: cached indices that fall in this block
    while (rc.nxt[half] < cb + nv) {
      const int c = rc.cur[half];
      const float z = st_row(st, r)[st_pos(r, (int)(rc.nxt[half] - cb))];
      x = fmaf(rc.p[c], z, x);
      if (ztk) ztk[perm[c]] = z;
      rc.cur[half] = c + 1;
      rc.nxt[half] = rc.at(c + 1);
    }
  }
};

struct DzRow {
  RowCursor rc;
  float L2, gs;
  bool rv;

  // replace the staged logits of this row by dZ (zero outside the valid rows
  // and columns)
  __device__ inline void consume(StPair st, long cb, long V, int half, float c2) {
    const int r = threadIdx.x;
    const int nv = rv ? (int)max(0L, min(32L, V - cb)) : 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float4 f = st_read4(st, r, j);
      f.x = 4 * j + 0 < nv ? gs * fast_exp2(fmaf(f.x, c2, -L2)) : 0.f;
      f.y = 4 * j + 1 < nv ? gs * fast_exp2(fmaf(f.y, c2, -L2)) : 0.f;
      f.z = 4 * j + 2 < nv ? gs * fast_exp2(fmaf(f.z, c2, -L2)) : 0.f;
      f.w = 4 * j + 3 < nv ? gs * fast_exp2(fmaf(f.w, c2, -L2)) : 0.f;
      st_write4(st, r, j, f);
    }
    while (rc.nxt[half] < cb + nv) {  // scatter-add of the teacher mass
      const int c = rc.cur[half];
      st_row(st, r)[st_pos(r, (int)(rc.nxt[half] - cb))] -= gs * rc.p[c];
      rc.cur[half] = c + 1;
      rc.nxt[half] = rc.at(c + 1);
    }
  }
};

template <int NBI>
__device__ inline void fwd_round(const Slots& sl, const f32x16_t (&acc)[4][4], long n0, FwdRow& R,
                                 const TopkFwdArgs& a) {
  const StPair s0 = st_pair<0>(sl), s1 = st_pair<1>(sl);
  stage_block<NBI, 4>(s0, s1, acc);
  __syncthreads();
  R.consume(s0, n0 + NBI * 32, a.V, 0, a.c2);
  R.consume(s1, n0 + 128 + NBI * 32, a.V, 1, a.c2);
  __syncthreads();
}

template <class E, int NBI>
__device__ inline void dz_round(const Slots& sl, const f32x16_t (&acc)[4][4], long n0, long row0, DzRow& R,
                                const TopkDzArgs& a) {
  const StPair s0 = st_pair<0>(sl), s1 = st_pair<1>(sl);
  stage_block<NBI, 4>(s0, s1, acc);
  __syncthreads();
  R.consume(s0, n0 + NBI * 32, a.V, 0, a.c2);
  R.consume(s1, n0 + 128 + NBI * 32, a.V, 1, a.c2);
  __syncthreads();
  store_block<E>(s0, a.dz, a.ldz, row0, n0 + NBI * 32, LONG_MAX, a.ldz);
  store_block<E>(s1, a.dz, a.ldz, row0, n0 + 128 + NBI * 32, LONG_MAX, a.ldz);
  __syncthreads();
}

}  // namespace

template <class Main, class E>
__global__ __launch_bounds__(kThreads, 1) void topk_fwd_kernel(TopkFwdArgs a) {
  KD_DECLARE_SLOTS(sl);

  const int count = *a.c.count;
  int rb, sp;
  grouped_coords(xcd_remap(blockIdx.x, gridDim.x), a.nrb, a.S, 4, rb, sp);
  const int row0 = rb * kBM;
  if (row0 >= count) return;
  const int tb = (int)((long)a.ntiles * sp / a.S);
  const int te = (int)((long)a.ntiles * (sp + 1) / a.S);

  Main mainloop;
  mainloop.init(
      a.H,
      [&](int r) -> const char* {
        const int i = row0 + r;
        return i < count ? a.H + (long)a.c.rows[i] * a.d * E::kElem : nullptr;
      },
      a.W, a.V * E::kElem, a.V, a.d);

  const int ti = row0 + (int)threadIdx.x;
  FwdRow R;
  R.rv = ti < count;
  const long t = R.rv ? a.c.rows[ti] : 0;
  R.rc.idx = a.rd.idx + t * a.K;
  R.rc.p = a.rd.p + t * a.K;
  R.rc.K = R.rv ? (int)a.K : 0;
  R.rc.cur[0] = seek(R.rc.idx, R.rc.K, 0, (long)tb * kBN);
  R.perm = a.rd.perm + t * a.K;
  R.ztk = a.z_topk ? a.z_topk + t * a.K : nullptr;
  R.m2 = -INFINITY;
  R.l = 0.f;
  R.x = 0.f;

  f32x16_t acc[4][kBN / 64];
  for (int vt = tb; vt < te; ++vt) {
    const long n0 = (long)vt * kBN;
    mainloop.tile(sl, n0, acc);
    R.rc.enter_tile(n0);
    fwd_round<0>(sl, acc, n0, R, a);
    fwd_round<1>(sl, acc, n0, R, a);
    fwd_round<2>(sl, acc, n0, R, a);
    fwd_round<3>(sl, acc, n0, R, a);
    R.rc.leave_tile();
  }
  if (R.rv) {
    float4* o = reinterpret_cast<float4*>(a.part) + (long)sp * a.part_stride + ti;
    *o = make_float4(R.m2, R.l, R.x, 0.f);
  }
}

template <class Main, class E>
__global__ __launch_bounds__(kThreads, 1) void topk_dz_kernel(TopkDzArgs a) {
  KD_DECLARE_SLOTS(sl);

  const long count = *a.c.count;
  const long M = min(a.C, count - a.c0);  // valid rows in this chunk
  if (M <= 0) return;
  int rb, sp;
  grouped_coords(xcd_remap(blockIdx.x, gridDim.x), a.nrb, a.S, 4, rb, sp);
  const int row0 = rb * kBM;
  if (row0 >= M) return;
  const int tb = (int)((long)a.ntiles * sp / a.S);
  const int te = (int)((long)a.ntiles * (sp + 1) / a.S);
  const int32_t* rows = a.c.rows + a.c0;

  Main mainloop;
  mainloop.init(
      a.H,
      [&](int r) -> const char* {
        const long i = row0 + r;
        return i < M ? a.H + (long)rows[i] * a.d * E::kElem : nullptr;
      },
      a.W, a.V * E::kElem, a.V, a.d);

  const int ti = row0 + (int)threadIdx.x;
  DzRow R;
  R.rv = ti < M;
  const long t = R.rv ? rows[ti] : 0;
  R.rc.idx = a.rd.idx + t * a.K;
  R.rc.p = a.rd.p + t * a.K;
  R.rc.K = R.rv ? (int)a.K : 0;
  R.rc.cur[0] = seek(R.rc.idx, R.rc.K, 0, (long)tb * kBN);
  R.L2 = R.rv ? a.lse[t] * kLog2e : 0.f;
  R.gs = R.rv ? a.g[t] * a.inv_tau : 0.f;

  f32x16_t acc[4][kBN / 64];
  for (int vt = tb; vt < te; ++vt) {
    const long n0 = (long)vt * kBN;
    mainloop.tile(sl, n0, acc);
    R.rc.enter_tile(n0);
    dz_round<E, 0>(sl, acc, n0, row0, R, a);
    dz_round<E, 1>(sl, acc, n0, row0, R, a);
    dz_round<E, 2>(sl, acc, n0, row0, R, a);
    dz_round<E, 3>(sl, acc, n0, row0, R, a);
    R.rc.leave_tile();
  }
}

// The direct-load ring needs bf16 and a hidden width that is a multiple of 32.
hipError_t launch_topk_fwd(int elem, const TopkFwdArgs& a, hipStream_t st) {
  const dim3 grid(a.nrb * a.S), block(kThreads);
  if (elem == 2 && a.d % kDmaKs == 0 && fits32(a.part_stride * a.d * 2) && fits32(a.d * a.V * 2))
    hipLaunchKernelGGL((topk_fwd_kernel<DmaNN<kBN>, Bf16>), grid, block, 0, st, a);
  else if (elem == 2)
    hipLaunchKernelGGL((topk_fwd_kernel<GenNN<Bf16, kBN>, Bf16>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((topk_fwd_kernel<GenNN<F32, kBN>, F32>), grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_topk_dz(int elem, const TopkDzArgs& a, hipStream_t st) {
  const dim3 grid(a.nrb * a.S), block(kThreads);
  if (elem == 2 && a.d % kDmaKs == 0 && fits32(a.T * a.d * 2) && fits32(a.d * a.V * 2))
    hipLaunchKernelGGL((topk_dz_kernel<DmaNN<kBN>, Bf16>), grid, block, 0, st, a);
  else if (elem == 2)
    hipLaunchKernelGGL((topk_dz_kernel<GenNN<Bf16, kBN>, Bf16>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((topk_dz_kernel<GenNN<F32, kBN>, F32>), grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace kd
