// Gradient contractions of one backward chunk (the dZ chunk is written by the
// top-K or full-vocabulary dZ kernel):
//   dH_chunk = dZ . W^T   [C, V] x [V, d]: both operands are contiguous along
//                         the vocabulary, which is the contraction (dZ in
//                         panels of C rows, W row-major); the vocabulary is
//                         split S ways and each split writes its own float32
//                         partial (summed in a fixed order by the reduce
//                         kernel, so results are deterministic).
//   dW      += H^T . dZ   [d, C] x [C, V]: H^T of the chunk is a gathered,
//                         transposed copy in panels of d rows (contiguous along
//                         the chunk's rows); dZ is n-contiguous here, read
//                         from its panels.  The first chunk stores, later
//                         chunks add in place, so chunks act as a fixed-order
//                         split over tokens.
// "Efficient Knowledge Distillation for LLMs: Offline Top-K Logits and a Fused
// Chunked KL Loss", §3 "Fused chunked KL": per chunk, the backward pass costs
// the recomputed projection plus these two products.
#include "kd_gemm.h"
#include "kd_launch.h"
#include "kd_main.h"

namespace kd {

namespace {

template <int NBI>
__device__ inline void f32_round(const Slots& sl, const f32x16_t (&acc)[4][4], float* dst, long ld, long row0,
                                 long n0, long nrows, long ncols, bool accumulate) {
  const StPair s0 = st_pair<0>(sl), s1 = st_pair<1>(sl);
  stage_block<NBI, 4>(s0, s1, acc);
  __syncthreads();
  rmw_pair_f32(s0, s1, dst, ld, row0, n0 + NBI * 32, n0 + 128 + NBI * 32, nrows, ncols, accumulate);
  __syncthreads();
}

__device__ inline void store_tile_f32(const Slots& sl, const f32x16_t (&acc)[4][4], float* dst, long ld, long row0,
                                      long n0, long nrows, long ncols, bool accumulate) {
  f32_round<0>(sl, acc, dst, ld, row0, n0, nrows, ncols, accumulate);
  f32_round<1>(sl, acc, dst, ld, row0, n0, nrows, ncols, accumulate);
  f32_round<2>(sl, acc, dst, ld, row0, n0, nrows, ncols, accumulate);
  f32_round<3>(sl, acc, dst, ld, row0, n0, nrows, ncols, accumulate);
}

}  // namespace

template <class Main, class E>
__global__ __launch_bounds__(kThreads, 1) void dh_kernel(DhArgs a) {
  constexpr int BN = 256;
  KD_DECLARE_SLOTS(sl);

  const long count = *a.count;
  const long M = min(a.C, count - a.c0);
  if (M <= 0) return;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int per_split = a.nrb * a.ncb;
  const int sp = logical / per_split;
  int rb, cb;
  grouped_coords(logical - sp * per_split, a.nrb, a.ncb, a.group, rb, cb);
  const long row0 = (long)rb * kBM, n0 = (long)cb * BN;
  if (row0 >= M) return;

  // contraction over the first V columns of both operands, split in S
  // ranges (the direct-load ring rounds it up to whole turns: the dZ chunk
  // holds zeros from V to ldz)
  Main mainloop;
  // dz in panels of C rows, W row-major
  mainloop.init(a.dz, [&](int r) -> const char* { return row0 + r < M ? a.dz + (row0 + r) * kRowB : nullptr; },
                a.W, [&](int r) -> const char* { return n0 + r < a.d ? a.W + (n0 + r) * a.V * E::kElem : nullptr; },
                a.V, a.C * kRowB);
  // split boundaries on whole groups of Main::kStageGroup stages
  const long ng = mainloop.nst / Main::kStageGroup;
  const long s0 = ng * sp / a.S * Main::kStageGroup, s1 = ng * (sp + 1) / a.S * Main::kStageGroup;
  f32x16_t acc[4][BN / 64];
  mainloop.tile(sl, s0, s1, acc);
  store_tile_f32(sl, acc, a.part + (long)sp * a.C * a.d, a.d, row0, n0, M, a.d, false);
}

template <class Main, class E>
__global__ __launch_bounds__(kThreads, 1) void dw_kernel(DwArgs a) {
  constexpr int BN = 256;
  KD_DECLARE_SLOTS(sl);

  const long count = *a.count;
  const long M = max(0L, min(a.C, count - a.c0));  // valid rows of the chunk
  if (M == 0 && a.accumulate) return;              // nothing to add
  int rb, cb;
  grouped_coords(xcd_remap(blockIdx.x, gridDim.x), a.nrb, a.ncb, a.group, rb, cb);
  const long row0 = (long)rb * kBM, n0 = (long)cb * BN;

  // contraction over the chunk's rows, rounded up to Main::kKMult (at most
  // 256): both buffers hold zeros between M and the end of their last
  // 256-row tile
  const long K = (M + Main::kKMult - 1) / Main::kKMult * Main::kKMult;
  Main mainloop;
  // hT in panels of d rows, dz in panels of C rows
  mainloop.init(a.hT, [&](int r) -> const char* { return row0 + r < a.d ? a.hT + (row0 + r) * kRowB : nullptr; },
                a.dz, 0, a.V, K, a.d * kRowB, a.C);
  f32x16_t acc[4][BN / 64];
  mainloop.tile(sl, n0, acc);
  store_tile_f32(sl, acc, a.dW, a.V, row0, n0, a.d, a.V, a.accumulate != 0);
}

hipError_t launch_dh(int elem, const DhArgs& a, hipStream_t st) {
  const dim3 grid(a.nrb * a.ncb * a.S), block(kThreads);
  if (dh_direct(elem, a.V) && fits32(a.C * a.ldz * 2) && fits32(a.d * a.V * 2))
    hipLaunchKernelGGL((dh_kernel<DmaNT<256>, Bf16>), grid, block, 0, st, a);
  else if (elem == 2)
    hipLaunchKernelGGL((dh_kernel<GenNT<Bf16, 256>, Bf16>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((dh_kernel<GenNT<F32, 256>, F32>), grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_dw(int elem, const DwArgs& a, hipStream_t st) {
  const dim3 grid(a.nrb * a.ncb), block(kThreads);
  if (elem == 2 && fits32(a.C * a.ldz * 2) && fits32(a.d * a.C * 2))
    hipLaunchKernelGGL((dw_kernel<DmaNN<256>, Bf16>), grid, block, 0, st, a);
  else if (elem == 2)
    hipLaunchKernelGGL((dw_kernel<GenNN<Bf16, 256>, Bf16>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((dw_kernel<GenNN<F32, 256>, F32>), grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace kd
