// Full-vocabulary KL tiles: forward and backward dZ.
//
// Teacher logits are recomputed from the teacher's final hidden states through
// a frozen copy of its output head (KDFlow abstract,
// thelatestinai.com/papers/2606.20005), so every vocabulary tile needs two
// contractions: u = Ht . Wt (teacher, width dt) and s = H . Ws (student,
// width d).  Both accumulator sets stay in registers (a 256 x 128 tile each),
// then both are staged through LDS and read back one row per thread.
//
// Forward, per row and in base 2 (y = z log2(e) / tau): running maxima and
// sums of 2^(ys - ms) and 2^(yt - mt), plus R = sum 2^(yt - mt) (yt - ys),
// rescaled whenever mt grows.  This is the one-pass online form of the
// coupled two-distribution KL (the idea of StreamKL's abstract, same page as
// the KDFlow abstract, applied to vocabulary tiles instead of attention):
//   KL = ln2 (R / lt - (mt + log2 lt) + (ms + log2 ls)).
// Backward: dZ = (g / tau) (2^(ys - Ls2) - 2^(yt - Lt2)).
#include "kd_gemm.h"
#include "kd_launch.h"

namespace kd {

namespace {

template <class E>
struct FullTile {
  static constexpr int BN = kTileNFull;
  using S = TileShape<BN>;
  using SG = Stage<BN>;
  static constexpr int kStaged = 2 * SG::kBytes;  // student and teacher slices
  static constexpr int kLds = S::kLds > kStaged ? S::kLds : kStaged;
  static constexpr int kKs = kStageBytes / E::kElem;
};

// Both contractions of one vocabulary tile: acc_t = Ht . Wt, acc_s = H . Ws.
template <class E>
__device__ inline void dual_tile(char* lds, KRowLoader<kBM>& alt, KRowLoader<kBM>& als,
                                 NColLoader<E, kTileNFull>& blt, NColLoader<E, kTileNFull>& bls, long kbt,
                                 long kbs, f32x16_t (&acc_t)[4][2], f32x16_t (&acc_s)[4][2]) {
  constexpr int BN = kTileNFull;
  using FT = FullTile<E>;
  zero_acc<BN>(acc_t);
  zero_acc<BN>(acc_s);
  contract<E, BN>(
      lds, 0, (kbt + kStageBytes - 1) / kStageBytes, acc_t,
      [&](long s) {
        alt.load(s * kStageBytes, kbt);
        blt.load(s * FT::kKs);
      },
      [&](char* buf) {
        alt.store(buf);
        blt.store(buf + TileShape<BN>::kABytes);
      });
  contract<E, BN>(
      lds, 0, (kbs + kStageBytes - 1) / kStageBytes, acc_s,
      [&](long s) {
        als.load(s * kStageBytes, kbs);
        bls.load(s * FT::kKs);
      },
      [&](char* buf) {
        als.store(buf);
        bls.store(buf + TileShape<BN>::kABytes);
      });
}

}  // namespace

template <class E>
__global__ __launch_bounds__(kThreads, 1) void full_fwd_kernel(FullFwdArgs a) {
  constexpr int BN = kTileNFull;
  using FT = FullTile<E>;
  using SG = Stage<BN>;
  __shared__ __attribute__((aligned(16))) char lds[FT::kLds];

  const int count = *a.c.count;
  int rb, sp;
  grouped_coords(xcd_remap(blockIdx.x, gridDim.x), a.nrb, a.S, 4, rb, sp);
  const int row0 = rb * kBM;
  if (row0 >= count) return;
  const int tb = (int)((long)a.ntiles * sp / a.S);
  const int te = (int)((long)a.ntiles * (sp + 1) / a.S);

  KRowLoader<kBM> als, alt;
  als.init_q();
  alt.init_q();
#pragma unroll
  for (int j = 0; j < KRowLoader<kBM>::kPer; ++j) {
    const int i = row0 + als.row_of(j);
    const long r = (i < count) ? (long)a.c.rows[i] : -1;
    als.rp[j] = r >= 0 ? a.H + r * a.d * E::kElem : nullptr;
    alt.rp[j] = r >= 0 ? a.Ht + r * a.dt * E::kElem : nullptr;
  }
  NColLoader<E, BN> bls, blt;
  bls.ld = blt.ld = a.V * E::kElem;
  bls.N = blt.N = a.V;
  bls.K = a.d;
  blt.K = a.dt;
  const long kbs = a.d * E::kElem, kbt = a.dt * E::kElem;

  const int ti = row0 + (int)threadIdx.x;
  const bool rv = ti < count;
  float ms = -INFINITY, ls = 0.f, mt = -INFINITY, lt = 0.f, R = 0.f;

  f32x16_t acc_s[4][2], acc_t[4][2];
  float* sts = reinterpret_cast<float*>(lds);
  float* stt = sts + kBM * SG::kSP;

  for (int vt = tb; vt < te; ++vt) {
    const long n0 = (long)vt * BN;
    bls.base = a.Ws + n0 * E::kElem;
    blt.base = a.Wt + n0 * E::kElem;
    bls.n0 = blt.n0 = n0;
    dual_tile<E>(lds, alt, als, blt, bls, kbt, kbs, acc_t, acc_s);
#pragma unroll 1
    for (int half = 0; half < 2; ++half) {
      stage_acc<BN>(sts, acc_s, half);
      stage_acc<BN>(stt, acc_t, half);
      __syncthreads();
      const long cb = n0 + half * SG::kWN;
      const int nv = (int)max(0L, min((long)SG::kWN, a.V - cb));
      if (rv && nv > 0) {
        const float* rs = sts + threadIdx.x * SG::kSP;
        const float* rt = stt + threadIdx.x * SG::kSP;
#pragma unroll 1
        for (int c = 0; c < nv; c += 32) {
          float vs[32], vt2[32];
          float cms = -INFINITY, cmt = -INFINITY;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float4 fs = *reinterpret_cast<const float4*>(rs + c + 4 * j);
            const float4 ft = *reinterpret_cast<const float4*>(rt + c + 4 * j);
            const bool ok = c + 4 * j < nv;
            vs[4 * j + 0] = ok ? fs.x : -INFINITY;
            vs[4 * j + 1] = ok ? fs.y : -INFINITY;
            vs[4 * j + 2] = ok ? fs.z : -INFINITY;
            vs[4 * j + 3] = ok ? fs.w : -INFINITY;
            vt2[4 * j + 0] = ok ? ft.x : -INFINITY;
            vt2[4 * j + 1] = ok ? ft.y : -INFINITY;
            vt2[4 * j + 2] = ok ? ft.z : -INFINITY;
            vt2[4 * j + 3] = ok ? ft.w : -INFINITY;
            cms = fmaxf(cms, fmaxf(fmaxf(vs[4 * j], vs[4 * j + 1]), fmaxf(vs[4 * j + 2], vs[4 * j + 3])));
            cmt = fmaxf(cmt, fmaxf(fmaxf(vt2[4 * j], vt2[4 * j + 1]), fmaxf(vt2[4 * j + 2], vt2[4 * j + 3])));
          }
          const float cys = cms * a.c2, cyt = cmt * a.c2;
          if (cys > ms) {
            ls *= fast_exp2(ms - cys);
            ms = cys;
          }
          if (cyt > mt) {
            const float f = fast_exp2(mt - cyt);
            lt *= f;
            R *= f;
            mt = cyt;
          }
          float sum_s = 0.f, sum_t = 0.f, r = 0.f;
#pragma unroll
          for (int j = 0; j < 32; ++j) {
            if (c + j < nv) {
              const float ys = vs[j] * a.c2, yt = vt2[j] * a.c2;
              const float et = fast_exp2(yt - mt);
              sum_s += fast_exp2(ys - ms);
              sum_t += et;
              r = fmaf(et, yt - ys, r);
            }
          }
          ls += sum_s;
          lt += sum_t;
          R += r;
        }
      }
      __syncthreads();
    }
  }
  if (rv) {
    float4* o = reinterpret_cast<float4*>(a.part) + 2 * ((long)sp * a.part_stride + ti);
    o[0] = make_float4(ms, ls, mt, lt);
    o[1] = make_float4(R, 0.f, 0.f, 0.f);
  }
}

template <class E>
__global__ __launch_bounds__(kThreads, 1) void full_dz_kernel(FullDzArgs a) {
  constexpr int BN = kTileNFull;
  using FT = FullTile<E>;
  using SG = Stage<BN>;
  __shared__ __attribute__((aligned(16))) char lds[FT::kLds];

  const long count = *a.c.count;
  const long M = min(a.C, count - a.c0);
  if (M <= 0) return;
  int rb, sp;
  grouped_coords(xcd_remap(blockIdx.x, gridDim.x), a.nrb, a.S, 4, rb, sp);
  const int row0 = rb * kBM;
  if (row0 >= M) return;
  const int tb = (int)((long)a.ntiles * sp / a.S);
  const int te = (int)((long)a.ntiles * (sp + 1) / a.S);
  const int32_t* rows = a.c.rows + a.c0;

  KRowLoader<kBM> als, alt;
  als.init_q();
  alt.init_q();
#pragma unroll
  for (int j = 0; j < KRowLoader<kBM>::kPer; ++j) {
    const int i = row0 + als.row_of(j);
    const long r = (i < M) ? (long)rows[i] : -1;
    als.rp[j] = r >= 0 ? a.H + r * a.d * E::kElem : nullptr;
    alt.rp[j] = r >= 0 ? a.Ht + r * a.dt * E::kElem : nullptr;
  }
  NColLoader<E, BN> bls, blt;
  bls.ld = blt.ld = a.V * E::kElem;
  bls.N = blt.N = a.V;
  bls.K = a.d;
  blt.K = a.dt;
  const long kbs = a.d * E::kElem, kbt = a.dt * E::kElem;

  const int ti = row0 + (int)threadIdx.x;
  const bool rv = ti < M;
  const long t = rv ? rows[ti] : 0;
  const float Ls2 = rv ? a.lse_s[t] * kLog2e : 0.f;
  const float Lt2 = rv ? a.lse_t[t] * kLog2e : 0.f;
  const float gs = rv ? a.g[t] * a.inv_tau : 0.f;

  f32x16_t acc_s[4][2], acc_t[4][2];
  float* sts = reinterpret_cast<float*>(lds);
  float* stt = sts + kBM * SG::kSP;

  for (int vt = tb; vt < te; ++vt) {
    const long n0 = (long)vt * BN;
    bls.base = a.Ws + n0 * E::kElem;
    blt.base = a.Wt + n0 * E::kElem;
    bls.n0 = blt.n0 = n0;
    dual_tile<E>(lds, alt, als, blt, bls, kbt, kbs, acc_t, acc_s);
#pragma unroll 1
    for (int half = 0; half < 2; ++half) {
      stage_acc<BN>(sts, acc_s, half);
      stage_acc<BN>(stt, acc_t, half);
      __syncthreads();
      const long cb = n0 + half * SG::kWN;
      const int nv = (int)max(0L, min((long)SG::kWN, a.V - cb));
      float* rs = sts + threadIdx.x * SG::kSP;
      const float* rt = stt + threadIdx.x * SG::kSP;
#pragma unroll 4
      for (int c = 0; c < SG::kWN; c += 4) {
        float4 fs = *reinterpret_cast<float4*>(rs + c);
        const float4 ft = *reinterpret_cast<const float4*>(rt + c);
        const bool ok = rv && c < nv;
        fs.x = ok ? gs * (fast_exp2(fmaf(fs.x, a.c2, -Ls2)) - fast_exp2(fmaf(ft.x, a.c2, -Lt2))) : 0.f;
        fs.y = ok ? gs * (fast_exp2(fmaf(fs.y, a.c2, -Ls2)) - fast_exp2(fmaf(ft.y, a.c2, -Lt2))) : 0.f;
        fs.z = ok ? gs * (fast_exp2(fmaf(fs.z, a.c2, -Ls2)) - fast_exp2(fmaf(ft.z, a.c2, -Lt2))) : 0.f;
        fs.w = ok ? gs * (fast_exp2(fmaf(fs.w, a.c2, -Ls2)) - fast_exp2(fmaf(ft.w, a.c2, -Lt2))) : 0.f;
        *reinterpret_cast<float4*>(rs + c) = fs;
      }
      __syncthreads();
      store_slice<E, SG::kWN>(sts, a.dz, a.ldz, row0, cb, LONG_MAX);
      __syncthreads();
    }
  }
}

hipError_t launch_full_fwd(int elem, const FullFwdArgs& a, hipStream_t st) {
  const dim3 grid(a.nrb * a.S), block(kThreads);
  if (elem == 2)
    hipLaunchKernelGGL(full_fwd_kernel<Bf16>, grid, block, 0, st, a);
  else
    hipLaunchKernelGGL(full_fwd_kernel<F32>, grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_full_dz(int elem, const FullDzArgs& a, hipStream_t st) {
  const dim3 grid(a.nrb * a.S), block(kThreads);
  if (elem == 2)
    hipLaunchKernelGGL(full_dz_kernel<Bf16>, grid, block, 0, st, a);
  else
    hipLaunchKernelGGL(full_dz_kernel<F32>, grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace kd
