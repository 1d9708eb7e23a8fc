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
// Z = H_rows . W[:, tile] on matrix cores, staged through LDS half by half,
// and read back one row per thread.
//   forward  : running base-2 max / sum per row, plus the index-match gather:
//              the row's cached indices are sorted, so one cursor per row walks
//              them in step with the tiles and picks the hits out of LDS.
//   backward : dZ = (g/tau) (2^(y - L2) - sum of p over hits) written in the
//              input dtype to the chunk's dZ buffer.
#include <climits>

#include "kd_gemm.h"
#include "kd_launch.h"

namespace kd {

namespace {

// First sorted position whose index is >= v (binary search over K entries).
__device__ inline int lower_bound_idx(const int32_t* idx, int K, long v) {
  int lo = 0, hi = K;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if ((long)idx[mid] < v) lo = mid + 1; else hi = mid;
  }
  return lo;
}

template <class E, int BN>
struct TopkTile {
  using S = TileShape<BN>;
  using SG = Stage<BN>;
  static constexpr int kLds = S::kLds > SG::kBytes ? S::kLds : SG::kBytes;
  static constexpr int kKs = kStageBytes / E::kElem;
};

}  // namespace

template <class E>
__global__ __launch_bounds__(kThreads, 1) void topk_fwd_kernel(TopkFwdArgs a) {
  constexpr int BN = kTileN;
  using TT = TopkTile<E, BN>;
  using SG = Stage<BN>;
  __shared__ __attribute__((aligned(16))) char lds[TT::kLds];

  const int count = *a.c.count;
  int rb, sp;
  grouped_coords(xcd_remap(blockIdx.x, gridDim.x), a.nrb, a.S, 4, rb, sp);
  const int row0 = rb * kBM;
  if (row0 >= count) return;
  const int tb = (int)((long)a.ntiles * sp / a.S);
  const int te = (int)((long)a.ntiles * (sp + 1) / a.S);

  KRowLoader<kBM> al;
  al.init_q();
#pragma unroll
  for (int j = 0; j < KRowLoader<kBM>::kPer; ++j) {
    const int i = row0 + al.row_of(j);
    al.rp[j] = (i < count) ? a.H + (long)a.c.rows[i] * a.d * E::kElem : nullptr;
  }
  NColLoader<E, BN> bl;
  bl.ld = a.V * E::kElem;
  bl.N = a.V;
  bl.K = a.d;
  const long kbytes = a.d * E::kElem;
  const long nst = (kbytes + kStageBytes - 1) / kStageBytes;

  // this thread's row in the epilogue
  const int ti = row0 + (int)threadIdx.x;
  const bool rv = ti < count;
  const long t = rv ? a.c.rows[ti] : 0;
  const int32_t* idx = a.rd.idx + t * a.K;
  const float* pp = a.rd.p + t * a.K;
  const uint16_t* perm = a.rd.perm + t * a.K;
  int cur = rv ? lower_bound_idx(idx, (int)a.K, (long)tb * BN) : 0;
  long nxt = (rv && cur < a.K) ? (long)idx[cur] : LONG_MAX;
  float m2 = -INFINITY, l = 0.f, x = 0.f;

  f32x16_t acc[4][BN / 64];
  float* st = reinterpret_cast<float*>(lds);

  for (int vt = tb; vt < te; ++vt) {
    const long n0 = (long)vt * BN;
    bl.base = a.W + n0 * E::kElem;
    bl.n0 = n0;
    zero_acc<BN>(acc);
    contract<E, BN>(
        lds, 0, nst, acc,
        [&](long s) {
          al.load(s * kStageBytes, kbytes);
          bl.load(s * TT::kKs);
        },
        [&](char* buf) {
          al.store(buf);
          bl.store(buf + TileShape<BN>::kABytes);
        });
#pragma unroll 1
    for (int half = 0; half < 2; ++half) {
      stage_acc<BN>(st, acc, half);
      __syncthreads();
      const long cb = n0 + half * SG::kWN;
      const int nv = (int)max(0L, min((long)SG::kWN, a.V - cb));
      if (rv && nv > 0) {
        const float* rowp = st + threadIdx.x * SG::kSP;
#pragma unroll 1
        for (int c = 0; c < nv; c += 32) {
          float v[32];
          float cm = -INFINITY;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float4 f = *reinterpret_cast<const float4*>(rowp + c + 4 * j);
            const bool ok = c + 4 * j < nv;
            v[4 * j + 0] = ok ? f.x : -INFINITY;
            v[4 * j + 1] = ok ? f.y : -INFINITY;
            v[4 * j + 2] = ok ? f.z : -INFINITY;
            v[4 * j + 3] = ok ? f.w : -INFINITY;
            cm = fmaxf(cm, fmaxf(fmaxf(v[4 * j], v[4 * j + 1]), fmaxf(v[4 * j + 2], v[4 * j + 3])));
          }
          const float cmy = cm * a.c2;
          if (cmy > m2) {
            l *= fast_exp2(m2 - cmy);
            m2 = cmy;
          }
          float sum = 0.f;
#pragma unroll
          for (int j = 0; j < 32; ++j) sum += fast_exp2(fmaf(v[j], a.c2, -m2));
          l += sum;
        }
        // index-match gather: the cursor's next cached index lies in this slice
        while (nxt < cb + nv) {
          const float z = rowp[nxt - cb];
          x = fmaf(pp[cur], z, x);
          if (a.z_topk) a.z_topk[t * a.K + perm[cur]] = z;
          ++cur;
          nxt = cur < a.K ? (long)idx[cur] : LONG_MAX;
        }
      }
      __syncthreads();
    }
  }
  if (rv) {
    float4* o = reinterpret_cast<float4*>(a.part) + (long)sp * a.part_stride + ti;
    *o = make_float4(m2, l, x, 0.f);
  }
}

template <class E>
__global__ __launch_bounds__(kThreads, 1) void topk_dz_kernel(TopkDzArgs a) {
  constexpr int BN = kTileN;
  using TT = TopkTile<E, BN>;
  using SG = Stage<BN>;
  __shared__ __attribute__((aligned(16))) char lds[TT::kLds];

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

  KRowLoader<kBM> al;
  al.init_q();
#pragma unroll
  for (int j = 0; j < KRowLoader<kBM>::kPer; ++j) {
    const int i = row0 + al.row_of(j);
    al.rp[j] = (i < M) ? a.H + (long)rows[i] * a.d * E::kElem : nullptr;
  }
  NColLoader<E, BN> bl;
  bl.ld = a.V * E::kElem;
  bl.N = a.V;
  bl.K = a.d;
  const long kbytes = a.d * E::kElem;
  const long nst = (kbytes + kStageBytes - 1) / kStageBytes;

  const int ti = row0 + (int)threadIdx.x;
  const bool rv = ti < M;
  const long t = rv ? rows[ti] : 0;
  const int32_t* idx = a.rd.idx + t * a.K;
  const float* pp = a.rd.p + t * a.K;
  int cur = rv ? lower_bound_idx(idx, (int)a.K, (long)tb * BN) : 0;
  long nxt = (rv && cur < a.K) ? (long)idx[cur] : LONG_MAX;
  const float L2 = rv ? a.lse[t] * kLog2e : 0.f;
  const float gs = rv ? a.g[t] * a.inv_tau : 0.f;

  f32x16_t acc[4][BN / 64];
  float* st = reinterpret_cast<float*>(lds);

  for (int vt = tb; vt < te; ++vt) {
    const long n0 = (long)vt * BN;
    bl.base = a.W + n0 * E::kElem;
    bl.n0 = n0;
    zero_acc<BN>(acc);
    contract<E, BN>(
        lds, 0, nst, acc,
        [&](long s) {
          al.load(s * kStageBytes, kbytes);
          bl.load(s * TT::kKs);
        },
        [&](char* buf) {
          al.store(buf);
          bl.store(buf + TileShape<BN>::kABytes);
        });
#pragma unroll 1
    for (int half = 0; half < 2; ++half) {
      stage_acc<BN>(st, acc, half);
      __syncthreads();
      const long cb = n0 + half * SG::kWN;
      const int nv = (int)max(0L, min((long)SG::kWN, a.V - cb));
      float* rowp = st + threadIdx.x * SG::kSP;
      if (rv) {
#pragma unroll 4
        for (int c = 0; c < SG::kWN; c += 4) {
          float4 f = *reinterpret_cast<float4*>(rowp + c);
          const bool ok = c < nv;
          f.x = ok ? gs * fast_exp2(fmaf(f.x, a.c2, -L2)) : 0.f;
          f.y = ok ? gs * fast_exp2(fmaf(f.y, a.c2, -L2)) : 0.f;
          f.z = ok ? gs * fast_exp2(fmaf(f.z, a.c2, -L2)) : 0.f;
          f.w = ok ? gs * fast_exp2(fmaf(f.w, a.c2, -L2)) : 0.f;
          *reinterpret_cast<float4*>(rowp + c) = f;
        }
        while (nxt < cb + nv) {  // scatter-add of the teacher mass
          rowp[nxt - cb] -= gs * pp[cur];
          ++cur;
          nxt = cur < a.K ? (long)idx[cur] : LONG_MAX;
        }
      } else {
#pragma unroll 4
        for (int c = 0; c < SG::kWN; c += 4) *reinterpret_cast<float4*>(rowp + c) = make_float4(0.f, 0.f, 0.f, 0.f);
      }
      __syncthreads();
      store_slice<E, SG::kWN>(st, a.dz, a.ldz, row0, cb, LONG_MAX);
      __syncthreads();
    }
  }
}

hipError_t launch_topk_fwd(int elem, const TopkFwdArgs& a, hipStream_t st) {
  const dim3 grid(a.nrb * a.S), block(kThreads);
  if (elem == 2)
    hipLaunchKernelGGL(topk_fwd_kernel<Bf16>, grid, block, 0, st, a);
  else
    hipLaunchKernelGGL(topk_fwd_kernel<F32>, grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_topk_dz(int elem, const TopkDzArgs& a, hipStream_t st) {
  const dim3 grid(a.nrb * a.S), block(kThreads);
  if (elem == 2)
    hipLaunchKernelGGL(topk_dz_kernel<Bf16>, grid, block, 0, st, a);
  else
    hipLaunchKernelGGL(topk_dz_kernel<F32>, grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace kd
