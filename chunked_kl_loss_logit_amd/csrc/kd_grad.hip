// Gradient contractions of one backward chunk (the dZ chunk is written by the
// top-K or full-vocabulary dZ kernel):
//   dH_chunk = dZ . W^T   [C, V] x [V, d]: both operands are contiguous along
//                         the vocabulary, which is the contraction; the
//                         vocabulary is split S ways and each split writes
//                         its own float32 partial (summed in a fixed order by
//                         the reduce kernel, so results are deterministic).
//   dW      += H^T . dZ   [d, C] x [C, V]: H^T of the chunk is a gathered,
//                         transposed copy (contiguous along the chunk's rows);
//                         dZ is [rows][V] and goes through the transposing
//                         column loader.  The first chunk stores, later chunks
//                         add in place, so chunks act as a fixed-order split
//                         over tokens.
// "Efficient Knowledge Distillation for LLMs: Offline Top-K Logits and a Fused
// Chunked KL Loss", §3 "Fused chunked KL": per chunk, the backward pass costs
// the recomputed projection plus these two products.
#include "kd_gemm.h"
#include "kd_launch.h"

namespace kd {

template <class E>
__global__ __launch_bounds__(kThreads, 1) void dh_kernel(DhArgs a) {
  constexpr int BN = 256;
  using S = TileShape<BN>;
  static_assert(Stage<BN>::kBytes <= S::kLds, "epilogue slice must fit the operand buffers");
  __shared__ __attribute__((aligned(16))) char lds[S::kLds];

  const long count = *a.count;
  const long M = min(a.C, count - a.c0);
  if (M <= 0) return;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int per_split = a.nrb * a.ncb;
  const int sp = logical / per_split;
  int rb, cb;
  grouped_coords(logical - sp * per_split, a.nrb, a.ncb, 4, rb, cb);
  const long row0 = (long)rb * kBM, n0 = (long)cb * BN;
  if (row0 >= M) return;

  // contraction over the vocabulary, split in S contiguous ranges; columns
  // past V are never read from either operand (V is a whole number of chunks)
  const long kza = a.V * E::kElem;
  const long kwb = a.V * E::kElem;
  const long nst = (kza + kStageBytes - 1) / kStageBytes;
  const long s0 = nst * sp / a.S, s1 = nst * (sp + 1) / a.S;

  KRowLoader<kBM> al, bl;
  al.init_q();
  bl.init_q();
#pragma unroll
  for (int j = 0; j < KRowLoader<kBM>::kPer; ++j) {
    const long i = row0 + al.row_of(j);
    al.rp[j] = (i < M) ? a.dz + i * a.ldz * E::kElem : nullptr;
    const long n = n0 + bl.row_of(j);
    bl.rp[j] = (n < a.d) ? a.W + n * a.V * E::kElem : nullptr;
  }

  f32x16_t acc[4][BN / 64];
  zero_acc<BN>(acc);
  contract<E, BN>(
      lds, s0, s1, acc,
      [&](long s) {
        al.load(s * kStageBytes, kza);
        bl.load(s * kStageBytes, kwb);
      },
      [&](char* buf) {
        al.store(buf);
        bl.store(buf + S::kABytes);
      });

  float* out = a.part + (long)sp * a.C * a.d;
  float* st = reinterpret_cast<float*>(lds);
#pragma unroll 1
  for (int half = 0; half < 2; ++half) {
    stage_acc<BN>(st, acc, half);
    __syncthreads();
    rmw_slice_f32<BN / 2>(st, out, a.d, row0, n0 + half * (BN / 2), M, a.d, false);
    __syncthreads();
  }
}

template <class E>
__global__ __launch_bounds__(kThreads, 1) void dw_kernel(DwArgs a) {
  constexpr int BN = 256;
  using S = TileShape<BN>;
  static_assert(Stage<BN>::kBytes <= S::kLds, "epilogue slice must fit the operand buffers");
  __shared__ __attribute__((aligned(16))) char lds[S::kLds];

  const long count = *a.count;
  const long M = max(0L, min(a.C, count - a.c0));  // contraction length: valid rows of the chunk
  if (M == 0 && a.accumulate) return;              // nothing to add
  int rb, cb;
  grouped_coords(xcd_remap(blockIdx.x, gridDim.x), a.nrb, a.ncb, 4, rb, cb);
  const long row0 = (long)rb * kBM, n0 = (long)cb * BN;

  const long kb = M * E::kElem;
  const long nst = (kb + kStageBytes - 1) / kStageBytes;

  KRowLoader<kBM> al;
  al.init_q();
#pragma unroll
  for (int j = 0; j < KRowLoader<kBM>::kPer; ++j) {
    const long r = row0 + al.row_of(j);
    al.rp[j] = (r < a.d) ? a.hT + r * a.C * E::kElem : nullptr;
  }
  NColLoader<E, BN> bl;
  bl.base = a.dz + n0 * E::kElem;
  bl.ld = a.ldz * E::kElem;
  bl.N = a.V;
  bl.n0 = n0;
  bl.K = M;
  constexpr int KS = kStageBytes / E::kElem;

  f32x16_t acc[4][BN / 64];
  zero_acc<BN>(acc);
  contract<E, BN>(
      lds, 0, nst, acc,
      [&](long s) {
        al.load(s * kStageBytes, kb);
        bl.load(s * KS);
      },
      [&](char* buf) {
        al.store(buf);
        bl.store(buf + S::kABytes);
      });

  float* st = reinterpret_cast<float*>(lds);
#pragma unroll 1
  for (int half = 0; half < 2; ++half) {
    stage_acc<BN>(st, acc, half);
    __syncthreads();
    rmw_slice_f32<BN / 2>(st, a.dW, a.V, row0, n0 + half * (BN / 2), a.d, a.V, a.accumulate != 0);
    __syncthreads();
  }
}

hipError_t launch_dh(int elem, const DhArgs& a, hipStream_t st) {
  const dim3 grid(a.nrb * a.ncb * a.S), block(kThreads);
  if (elem == 2)
    hipLaunchKernelGGL(dh_kernel<Bf16>, grid, block, 0, st, a);
  else
    hipLaunchKernelGGL(dh_kernel<F32>, grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_dw(int elem, const DwArgs& a, hipStream_t st) {
  const dim3 grid(a.nrb * a.ncb), block(kThreads);
  if (elem == 2)
    hipLaunchKernelGGL(dw_kernel<Bf16>, grid, block, 0, st, a);
  else
    hipLaunchKernelGGL(dw_kernel<F32>, grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace kd
