// Full-vocabulary KL tiles: forward and backward dZ.
//
// Teacher logits are recomputed from the teacher's final hidden states through
// a frozen copy of its output head (KDFlow abstract,
// thelatestinai.com/papers/2606.20005), so every vocabulary tile needs two
// contractions: u = Ht . Wt (teacher, width dt) and s = H . Ws (student,
// width d), with H and Ht read from the chunk's panel copies.  Both
// accumulator sets stay in registers (a 256 x 128 tile each).  On the
// direct-load path (bf16) both are accumulated transposed and the epilogues
// work on each lane's own columns in registers (full_fwd_t_kernel,
// full_dz_t_kernel); otherwise each of two epilogue rounds stages one
// 32-column block of each wave column half of both sets (all four LDS slots)
// and reads it back one row per thread.
//
// Forward, per row and in base 2 (y = z log2(e) / tau): running maxima and
// sums of 2^(ys - ms) and 2^(yt - mt), plus R = sum 2^(yt - mt) (yt - ys),
// rescaled whenever mt grows, and R2 = sum 2^(ys - ms) (ys - yt), rescaled
// whenever ms grows.  This is the one-pass online form of the coupled
// two-distribution KL (the idea in StreamKL's abstract, on the same page as
// the KDFlow abstract, here over vocabulary tiles), in both directions:
//   KL(p||q) = ln2 (R / lt - (mt + log2 lt) + (ms + log2 ls)),
//   KL(q||p) = ln2 (R2 / ls - (ms + log2 ls) + (mt + log2 lt)).
// Backward: dZ = (g / tau) (2^(ys - Ls2) - 2^(yt - Lt2)), or with KL mixing
// (the KL-direction abstract on the same page) weight r on the reverse KL:
//   dZ = (g / tau) [(1 - r)(q - p) + r q (ln q - ln p - KL(q||p))].
// A per-row temperature (tau_rows) gives each row its own log2(e) / tau.
#include <climits>

#include "kd_gemm.h"
#include "kd_launch.h"
#include "kd_main.h"

namespace kd {

namespace {

constexpr int kBN = kTileNFull;

struct FullFwdRow {
  float ms, ls, mt, lt, R, R2, c2;
  bool rv;

  __device__ inline void consume(StPair ss, StPair su, long cb, long V) {
    if (!rv) return;
    const int nv = (int)max(0L, min(32L, V - cb));
    if (nv == 0) return;
    const int r = threadIdx.x;
    // two online updates of 16 columns each: half the live temporaries of one
    // 32-column update, so the epilogue needs no scratch
    half<0>(ss, su, r, nv);
    if (nv > 16) half<4>(ss, su, r, nv);
  }

  // columns [4 J0, 4 J0 + 16) of the staged blocks, those below nv valid
  template <int J0>
  __device__ inline void half(StPair ss, StPair su, int r, int nv) {
    float vs[16], vu[16];
    float cms = -INFINITY, cmt = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 fs = st_read4(ss, r, J0 + j), fu = st_read4(su, r, J0 + j);
      const bool ok = 4 * (J0 + j) < nv;
      vs[4 * j + 0] = ok ? fs.x : -INFINITY;
      vs[4 * j + 1] = ok ? fs.y : -INFINITY;
      vs[4 * j + 2] = ok ? fs.z : -INFINITY;
      vs[4 * j + 3] = ok ? fs.w : -INFINITY;
      vu[4 * j + 0] = ok ? fu.x : -INFINITY;
      vu[4 * j + 1] = ok ? fu.y : -INFINITY;
      vu[4 * j + 2] = ok ? fu.z : -INFINITY;
      vu[4 * j + 3] = ok ? fu.w : -INFINITY;
      cms = fmaxf(cms, fmaxf(fmaxf(vs[4 * j], vs[4 * j + 1]), fmaxf(vs[4 * j + 2], vs[4 * j + 3])));
      cmt = fmaxf(cmt, fmaxf(fmaxf(vu[4 * j], vu[4 * j + 1]), fmaxf(vu[4 * j + 2], vu[4 * j + 3])));
    }
    const float cys = cms * c2, cyt = cmt * c2;
    if (cys > ms) {
      const float f = fast_exp2(ms - cys);
      ls *= f;
      R2 *= f;
      ms = cys;
    }
    if (cyt > mt) {
      const float f = fast_exp2(mt - cyt);
      lt *= f;
      R *= f;
      mt = cyt;
    }
    float sum_s = 0.f, sum_t = 0.f, rr = 0.f, rr2 = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (4 * J0 + j < nv) {
        const float ys = vs[j] * c2, yt = vu[j] * c2;
        const float et = fast_exp2(yt - mt), es = fast_exp2(ys - ms);
        sum_s += es;
        sum_t += et;
        rr = fmaf(et, yt - ys, rr);
        rr2 = fmaf(es, ys - yt, rr2);
      }
    }
    ls += sum_s;
    lt += sum_t;
    R += rr;
    R2 += rr2;
  }
};

// dZ of one element from its two logits and the row's constants.
struct FullDzConst {
  float Ls2, Lt2, gs, c2;
  float a, b, kr;  // KL mixing: weights of the forward and reverse terms, the row's KL(q||p)
  bool mix;

  __device__ inline float operator()(float zs, float zt) const {
    const float ds = fmaf(zs, c2, -Ls2), dt = fmaf(zt, c2, -Lt2);
    const float qs = fast_exp2(ds), pt = fast_exp2(dt);
    if (!mix) return gs * (qs - pt);
    return gs * fmaf(a, qs - pt, b * qs * fmaf(kLn2, ds - dt, -kr));
  }
};

// The row's constants for the backward, from the forward's outputs.
__device__ inline FullDzConst full_dz_const(bool rv, long t, const float* lse_s, const float* lse_t, const float* g,
                                            float c2, float inv_tau, const FullMix& mx) {
  FullDzConst k{};
  if (!rv) return k;
  if (mx.tau_rows) {
    const float tt = mx.tau_rows[t];
    c2 = (float)(1.4426950408889634 / (double)tt);
    inv_tau = 1.0f / tt;
  }
  k.c2 = c2;
  k.Ls2 = lse_s[t] * kLog2e;
  k.Lt2 = lse_t[t] * kLog2e;
  k.gs = g[t] * inv_tau;
  k.mix = mx.r != 0.f;
  k.a = 1.f - mx.r;
  k.b = mx.r;
  k.kr = k.mix ? mx.kl_rev[t] : 0.f;
  return k;
}

struct FullDzRow {
  FullDzConst k;
  bool rv;

  __device__ inline void consume(StPair ss, StPair su, long cb, long V) {
    const int r = threadIdx.x;
    const int nv = rv ? (int)max(0L, min(32L, V - cb)) : 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float4 fs = st_read4(ss, r, j);
      const float4 fu = st_read4(su, r, j);
      fs.x = 4 * j + 0 < nv ? k(fs.x, fu.x) : 0.f;
      fs.y = 4 * j + 1 < nv ? k(fs.y, fu.y) : 0.f;
      fs.z = 4 * j + 2 < nv ? k(fs.z, fu.z) : 0.f;
      fs.w = 4 * j + 3 < nv ? k(fs.w, fu.w) : 0.f;
      st_write4(ss, r, j, fs);
    }
  }
};

template <int NBI>
__device__ inline void stage_pair(const Slots& sl, const f32x16_t (&acc_s)[4][2], const f32x16_t (&acc_t)[4][2]) {
  stage_block<NBI, 2>(st_pair<0>(sl), st_pair<1>(sl), acc_s);
  stage_block<NBI, 2>(st_pair<2>(sl), st_pair<3>(sl), acc_t);
}

template <int NBI>
__device__ inline void full_fwd_round(const Slots& sl, const f32x16_t (&acc_s)[4][2],
                                      const f32x16_t (&acc_t)[4][2], long n0, FullFwdRow& R, const FullFwdArgs& a) {
  stage_pair<NBI>(sl, acc_s, acc_t);
  __syncthreads();
  R.consume(st_pair<0>(sl), st_pair<2>(sl), n0 + NBI * 32, a.V);
  R.consume(st_pair<1>(sl), st_pair<3>(sl), n0 + 64 + NBI * 32, a.V);
  __syncthreads();
}

template <class E, int NBI>
__device__ inline void full_dz_round(const Slots& sl, const f32x16_t (&acc_s)[4][2], const f32x16_t (&acc_t)[4][2],
                                     long n0, long row0, FullDzRow& R, const FullDzArgs& a) {
  stage_pair<NBI>(sl, acc_s, acc_t);
  __syncthreads();
  R.consume(st_pair<0>(sl), st_pair<2>(sl), n0 + NBI * 32, a.V);
  R.consume(st_pair<1>(sl), st_pair<3>(sl), n0 + 64 + NBI * 32, a.V);
  __syncthreads();
  store_block<E>(st_pair<0>(sl), a.dz, a.ldz, row0, n0 + NBI * 32, LONG_MAX, a.ldz, 0, a.C);
  store_block<E>(st_pair<1>(sl), a.dz, a.ldz, row0, n0 + 64 + NBI * 32, LONG_MAX, a.ldz, 0, a.C);
  __syncthreads();
}

}  // namespace

// Rows: the compacted valid rows [c0, c0 + C) (the plain forward takes them
// all); partials are indexed by compacted position.
template <class Main, class E>
__global__ __launch_bounds__(kThreads, 1) void full_fwd_kernel(FullFwdArgs a) {
  KD_DECLARE_SLOTS(sl);

  const long count = *a.c.count;
  const long M = min(a.C, count - a.c0);  // rows of this launch
  if (M <= 0) return;
  int rb, sp;
  grouped_coords(xcd_remap(blockIdx.x, gridDim.x), a.nrb, a.S, a.group, rb, sp);
  const int row0 = rb * kBM;
  if (row0 >= M) return;
  const int tb = (int)((long)a.ntiles * sp / a.S);
  const int te = (int)((long)a.ntiles * (sp + 1) / a.S);
  const int32_t* rows = a.c.rows + a.c0;

  Main ms, mt;
  // rows past the valid ones read the last valid row: they only feed
  // accumulator rows that the epilogue discards
  ms.init(a.Hp, [&](int r) -> const char* { return a.Hp + min((long)row0 + r, M - 1) * kRowB; }, a.Ws,
          a.V * E::kElem, a.V, a.d, a.C * kRowB);
  mt.init(a.Htp, [&](int r) -> const char* { return a.Htp + min((long)row0 + r, M - 1) * kRowB; }, a.Wt,
          a.V * E::kElem, a.V, a.dt, a.C * kRowB);

  const int ti = row0 + (int)threadIdx.x;
  FullFwdRow R{-INFINITY, 0.f, -INFINITY, 0.f, 0.f, 0.f, a.c2, ti < M};
  if (R.rv && a.tau_rows) R.c2 = (float)(1.4426950408889634 / (double)a.tau_rows[rows[ti]]);

  f32x16_t acc_s[4][2], acc_t[4][2];
  for (int vt = tb; vt < te; ++vt) {
    const long n0 = (long)vt * kBN;
    mt.tile(sl, n0, acc_t);
    ms.tile(sl, n0, acc_s);
    full_fwd_round<0>(sl, acc_s, acc_t, n0, R, a);
    full_fwd_round<1>(sl, acc_s, acc_t, n0, R, a);
  }
  if (R.rv) {
    float4* o = reinterpret_cast<float4*>(a.part) + 2 * ((long)sp * a.part_stride + (a.c0 - a.part_row0) + ti);
    o[0] = make_float4(R.ms, R.ls, R.mt, R.lt);
    o[1] = make_float4(R.R, R.R2, 0.f, 0.f);
  }
}

template <class Main, class E>
__global__ __launch_bounds__(kThreads, 1) void full_dz_kernel(FullDzArgs a) {
  KD_DECLARE_SLOTS(sl);

  const long count = *a.c.count;
  const long M = min(a.C, count - a.c0);
  if (M <= 0) return;
  int rb, sp;
  grouped_coords(xcd_remap(blockIdx.x, gridDim.x), a.nrb, a.S, a.group, rb, sp);
  const int row0 = rb * kBM;
  if (row0 >= M) return;
  const int tb = (int)((long)a.ntiles * sp / a.S);
  const int te = (int)((long)a.ntiles * (sp + 1) / a.S);
  const int32_t* rows = a.c.rows + a.c0;

  Main ms, mt;
  // rows past the valid ones read the last valid row: they only feed
  // accumulator rows that the epilogue discards
  ms.init(a.Hp, [&](int r) -> const char* { return a.Hp + min((long)row0 + r, M - 1) * kRowB; }, a.Ws,
          a.V * E::kElem, a.V, a.d, a.C * kRowB);
  mt.init(a.Htp, [&](int r) -> const char* { return a.Htp + min((long)row0 + r, M - 1) * kRowB; }, a.Wt,
          a.V * E::kElem, a.V, a.dt, a.C * kRowB);

  const int ti = row0 + (int)threadIdx.x;
  FullDzRow R;
  R.rv = ti < M;
  const long t = R.rv ? rows[ti] : 0;
  R.k = full_dz_const(R.rv, t, a.lse_s, a.lse_t, a.g, a.c2, a.inv_tau, a.mix);

  f32x16_t acc_s[4][2], acc_t[4][2];
  for (int vt = tb; vt < te; ++vt) {
    const long n0 = (long)vt * kBN;
    mt.tile(sl, n0, acc_t);
    ms.tile(sl, n0, acc_s);
    full_dz_round<E, 0>(sl, acc_s, acc_t, n0, row0, R, a);
    full_dz_round<E, 1>(sl, acc_s, acc_t, n0, row0, R, a);
  }
}

// ---------------------------------------------------------------- dual tiles, accumulators transposed
// The direct-load (bf16) forms of the two kernels above.  Both heads' tiles
// are accumulated transposed (mma_frags_t): lane l of wave (wm, wn) owns row
// wm 128 + 32 mb + l % 32 of the tile in block row mb and, in register i of
// block (mb, nb), column wn 64 + 32 nb + 8 (i / 4) + 4 (l / 32) + i % 4, for
// the student and the teacher alike.  The epilogues then work on each
// register pair in place: the forward keeps, per lane and row, the running
// state of the online form over its own 32 columns (in LDS between tiles;
// the two lanes and the two waves of a row merge it at the end of the
// split), and the backward turns each pair into dZ, rounds it and writes it
// through a wave-private 2 KB LDS region as whole-kilobyte panel stores.
namespace {

constexpr int kFStF = 6 * 4 * 64;  // floats per wave: (ms, ls, mt, lt, R, R2) of 4 rows x 64 lanes

// One row's update from its 32 columns per head in the lane; columns at or
// past V do not count (a group of four is in or out as a whole: V, base are
// multiples of 8).
template <bool kFull>
__device__ inline void full_row_t(const f32x16_t (&as)[2], const f32x16_t (&at)[2], float c2, float* st, int base,
                                  int V) {
  const int h4 = 4 * ((opaque((int)threadIdx.x) >> 5) & 1);
  float ms = st[0], ls = st[64], mt = st[128], lt = st[192], R = st[256], R2 = st[320];
  float pen[8];
#pragma unroll
  for (int g = 0; g < 8; ++g) pen[g] = kFull || base + 32 * (g >> 2) + 8 * (g & 3) + h4 < V ? 0.f : -INFINITY;
  float cms = -INFINITY, cmt = -INFINITY;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      cms = fmaxf(cms, as[nb][i] + pen[4 * nb + (i >> 2)]);
      cmt = fmaxf(cmt, at[nb][i] + pen[4 * nb + (i >> 2)]);
    }
  const float cys = cms * c2, cyt = cmt * c2;
  if (cys > ms) {
    const float f = fast_exp2(ms - cys);
    ls *= f;
    R2 *= f;
    ms = cys;
  }
  if (cyt > mt) {
    const float f = fast_exp2(mt - cyt);
    lt *= f;
    R *= f;
    mt = cyt;
  }
  float ss = 0.f, st_ = 0.f, rr = 0.f, rr2 = 0.f;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float pg = pen[4 * nb + (i >> 2)];
      const float es = fast_exp2(fmaf(as[nb][i], c2, -ms) + pg), et = fast_exp2(fmaf(at[nb][i], c2, -mt) + pg);
      const float dy = (at[nb][i] - as[nb][i]) * c2;  // yt - ys, finite on every column
      ss += es;
      st_ += et;
      rr = fmaf(et, dy, rr);
      rr2 = fmaf(es, -dy, rr2);
    }
  // a lane whose columns are all past V adds nothing (its maxima may still
  // be -inf, and 2^(-inf - -inf) would be NaN)
  if (cms != -INFINITY) {
    ls += ss;
    R2 += rr2;
  }
  if (cmt != -INFINITY) {
    lt += st_;
    R += rr;
  }
  st[0] = ms;
  st[64] = ls;
  st[128] = mt;
  st[192] = lt;
  st[256] = R;
  st[320] = R2;
}

// the online state of one row over two column sets, merged
struct FullPart {
  float ms, ls, mt, lt, R, R2;
};
__device__ inline FullPart full_merge(const FullPart& a, const FullPart& b) {
  FullPart o;
  o.ms = fmaxf(a.ms, b.ms);
  o.mt = fmaxf(a.mt, b.mt);
  const float fas = a.ms == -INFINITY ? 0.f : fast_exp2(a.ms - o.ms);
  const float fbs = b.ms == -INFINITY ? 0.f : fast_exp2(b.ms - o.ms);
  const float fat = a.mt == -INFINITY ? 0.f : fast_exp2(a.mt - o.mt);
  const float fbt = b.mt == -INFINITY ? 0.f : fast_exp2(b.mt - o.mt);
  o.ls = a.ls * fas + b.ls * fbs;
  o.R2 = a.R2 * fas + b.R2 * fbs;
  o.lt = a.lt * fat + b.lt * fbt;
  o.R = a.R * fat + b.R * fbt;
  return o;
}

}  // namespace

__global__ __launch_bounds__(kThreads, 1) void full_fwd_t_kernel(FullFwdArgs a) {
  KD_DECLARE_SLOTS(sl);

  const long count = *a.c.count;
  const long M = min(a.C, count - a.c0);  // rows of this launch
  if (M <= 0) return;
  int rb, sp;
  grouped_coords(xcd_remap(blockIdx.x, gridDim.x), a.nrb, a.S, a.group, rb, sp);
  const int row0 = rb * kBM;
  if (row0 >= M) return;
  const int tb = (int)((long)a.ntiles * sp / a.S);
  const int te = (int)((long)a.ntiles * (sp + 1) / a.S);
  const int32_t* rows = a.c.rows + a.c0;

  DmaNN<kBN> ms, mt;
  // rows past the valid ones read the last valid row: they only feed
  // accumulator rows that the epilogue discards
  ms.init(a.Hp, [&](int r) -> const char* { return a.Hp + min((long)row0 + r, M - 1) * kRowB; }, a.Ws, a.V * 2, a.V,
          a.d, a.C * kRowB);
  mt.init(a.Htp, [&](int r) -> const char* { return a.Htp + min((long)row0 + r, M - 1) * kRowB; }, a.Wt, a.V * 2,
          a.V, a.dt, a.C * kRowB);

  const int w = wave_id(), wm = w >> 1, wn = w & 1;
  const int lane = (int)threadIdx.x & 63;
  const int trow0 = wm * 128;
  float* fst = sl.ep + w * kFStF;
  float* c2k = sl.ep + 4 * kFStF;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int ti = row0 + trow0 + mb * 32 + (lane & 31);
    if (wn == 0 && lane < 32)
      c2k[trow0 + mb * 32 + lane] =
          ti < M && a.tau_rows ? (float)(1.4426950408889634 / (double)a.tau_rows[rows[ti]]) : a.c2;
#pragma unroll
    for (int q = 0; q < 6; ++q) fst[mb * 384 + q * 64 + lane] = (q == 0 || q == 2) ? -INFINITY : 0.f;
  }
  const int V = (int)a.V;

  f32x16_t acc_s[4][2], acc_t[4][2];
  for (int vt = tb; vt < te; ++vt) {
    const long n0 = (long)vt * kBN;
    mt.template tile<true>(sl, n0, acc_t);
    ms.template tile<true>(sl, n0, acc_s);
    // (tile() ends with a barrier: the row constants written before the
    // first tile are visible)
    const int base = (int)n0 + wn * 64;
    const int ln = opaque((int)threadIdx.x) & 63;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const float c2 = c2k[trow0 + mb * 32 + (ln & 31)];
      float* st = fst + mb * 384 + ln;
      if (base + 64 <= V)
        full_row_t<true>(acc_s[mb], acc_t[mb], c2, st, base, V);
      else
        full_row_t<false>(acc_s[mb], acc_t[mb], c2, st, base, V);
    }
  }

  // the split's partial per row: lane halves, then column halves (wave wn = 1
  // hands its state to wave wn = 0 through slot 0, free after the last tile)
  float* xch = reinterpret_cast<float*>(sl.s0);
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const float* st = fst + mb * 384 + lane;
    FullPart p{st[0], st[64], st[128], st[192], st[256], st[320]};
    const FullPart o{__shfl_xor(p.ms, 32), __shfl_xor(p.ls, 32), __shfl_xor(p.mt, 32),
                     __shfl_xor(p.lt, 32), __shfl_xor(p.R, 32),  __shfl_xor(p.R2, 32)};
    p = full_merge(p, o);
    if (wn == 1 && lane < 32) {
      float* x = xch + (trow0 + mb * 32 + lane) * 8;
      x[0] = p.ms;
      x[1] = p.ls;
      x[2] = p.mt;
      x[3] = p.lt;
      x[4] = p.R;
      x[5] = p.R2;
    }
    float* sw = fst + mb * 384 + lane;
    sw[0] = p.ms;
    sw[64] = p.ls;
    sw[128] = p.mt;
    sw[192] = p.lt;
    sw[256] = p.R;
    sw[320] = p.R2;
  }
  __syncthreads();
  if (wn == 0 && lane < 32) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int ti = row0 + trow0 + mb * 32 + lane;
      if (ti >= M) continue;
      const float* st = fst + mb * 384 + lane;
      const float* x = xch + (trow0 + mb * 32 + lane) * 8;
      const FullPart p = full_merge(FullPart{st[0], st[64], st[128], st[192], st[256], st[320]},
                                    FullPart{x[0], x[1], x[2], x[3], x[4], x[5]});
      float4* o = reinterpret_cast<float4*>(a.part) + 2 * ((long)sp * a.part_stride + (a.c0 - a.part_row0) + ti);
      o[0] = make_float4(p.ms, p.ls, p.mt, p.lt);
      o[1] = make_float4(p.R, p.R2, 0.f, 0.f);
    }
  }
}

namespace {

// Byte position of 8 bytes (half hh of 16-byte chunk j) of row r in a
// wave's [32][64 B] staging region, swizzled so that the 32 rows a half-wave
// writes, and the 4 rows x 4 chunks a quarter-wave reads back, hit distinct
// banks.
__device__ inline int fstg8(int r, int j, int hh) {
  return r * 64 + ((j ^ ((r >> 2) & 3)) << 4) + ((hh ^ ((r >> 4) & 1)) << 3);
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ inline uint32_t fpk_bf16(float lo, float hi) {  // round to nearest even
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// dZ of block (mb, nb) of the lane's row: columns at or past V are zero
template <bool kFull>
__device__ inline void full_dz_block_t(const f32x16_t& vs, const f32x16_t& vu, const FullDzConst& k, int cb, int V,
                                       char* stg, char* dz, long C, long brow0) {
  const int lane = opaque((int)threadIdx.x) & 63, h = lane >> 5, cl = lane & 31;
  float o[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float e = k(vs[i], vu[i]);
    o[i] = kFull || cb + 8 * (i >> 2) + 4 * h < V ? e : 0.f;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j)
    *reinterpret_cast<uint2*>(stg + fstg8(cl, j, h)) =
        make_uint2(fpk_bf16(o[4 * j], o[4 * j + 1]), fpk_bf16(o[4 * j + 2], o[4 * j + 3]));
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int r = kk * 16 + (lane >> 2), j = lane & 3;
    const uint4 q = *reinterpret_cast<const uint4*>(stg + r * 64 + ((j ^ ((r >> 2) & 3)) << 4));
    const uint4 wv = ((r >> 4) & 1) ? make_uint4(q.z, q.w, q.x, q.y) : q;
    *reinterpret_cast<uint4*>(dz + panel_off(C, brow0 + r, (long)(cb + 8 * j) * 2)) = wv;
  }
}

}  // namespace

__global__ __launch_bounds__(kThreads, 1) void full_dz_t_kernel(FullDzArgs a) {
  KD_DECLARE_SLOTS(sl);

  const long count = *a.c.count;
  const long M = min(a.C, count - a.c0);
  if (M <= 0) return;
  int rb, sp;
  grouped_coords(xcd_remap(blockIdx.x, gridDim.x), a.nrb, a.S, a.group, rb, sp);
  const int row0 = rb * kBM;
  if (row0 >= M) return;
  const int tb = (int)((long)a.ntiles * sp / a.S);
  const int te = (int)((long)a.ntiles * (sp + 1) / a.S);
  const int32_t* rows = a.c.rows + a.c0;

  DmaNN<kBN> ms, mt;
  ms.init(a.Hp, [&](int r) -> const char* { return a.Hp + min((long)row0 + r, M - 1) * kRowB; }, a.Ws, a.V * 2, a.V,
          a.d, a.C * kRowB);
  mt.init(a.Htp, [&](int r) -> const char* { return a.Htp + min((long)row0 + r, M - 1) * kRowB; }, a.Wt, a.V * 2,
          a.V, a.dt, a.C * kRowB);

  const int w = wave_id(), wm = w >> 1, wn = w & 1;
  const int lane = (int)threadIdx.x & 63;
  const int trow0 = wm * 128;
  FullDzConst* rowk = reinterpret_cast<FullDzConst*>(sl.ep);  // [256] row constants
  char* stg = reinterpret_cast<char*>(sl.ep) + kBM * sizeof(FullDzConst) + w * 2048;
  if (wn == 0 && lane < 32) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int ti = row0 + trow0 + mb * 32 + lane;
      const bool rv = ti < M;
      rowk[trow0 + mb * 32 + lane] =
          full_dz_const(rv, rv ? rows[ti] : 0, a.lse_s, a.lse_t, a.g, a.c2, a.inv_tau, a.mix);
    }
  }
  const int V = (int)a.V;

  f32x16_t acc_s[4][2], acc_t[4][2];
  for (int vt = tb; vt < te; ++vt) {
    const long n0 = (long)vt * kBN;
    mt.template tile<true>(sl, n0, acc_t);
    ms.template tile<true>(sl, n0, acc_s);
    const int base = (int)n0 + wn * 64;
    const int ln = opaque((int)threadIdx.x) & 63;
    const bool full = base + 64 <= V;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const FullDzConst k = rowk[trow0 + mb * 32 + (ln & 31)];
      const long brow0 = row0 + trow0 + mb * 32;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        if (full)
          full_dz_block_t<true>(acc_s[mb][nb], acc_t[mb][nb], k, base + 32 * nb, V, stg, a.dz, a.C, brow0);
        else
          full_dz_block_t<false>(acc_s[mb][nb], acc_t[mb][nb], k, base + 32 * nb, V, stg, a.dz, a.C, brow0);
      }
    }
  }
}

// ---------------------------------------------------------------- single call
__global__ void full_rowc_kernel(Compact c, long T, const float* tau_rows, float c2, float inv_tau, float4* rowc) {
  const long j = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= T || j >= *c.count) return;
  const long t = c.rows[j];
  if (tau_rows) {
    const float tt = tau_rows[t];
    c2 = (float)(1.4426950408889634 / (double)tt);
    inv_tau = 1.0f / tt;
  }
  rowc[t] = make_float4(c2, inv_tau, 1.f, 0.f);
}

hipError_t launch_full_rowc(Compact c, int64_t T, const float* tau_rows, float c2, float inv_tau, float4* rowc,
                            hipStream_t st) {
  hipLaunchKernelGGL(full_rowc_kernel, dim3((unsigned)((T + 255) / 256)), dim3(256), 0, st, c, (long)T, tau_rows, c2,
                     inv_tau, rowc);
  return hipGetLastError();
}

// Block geometry as kEwRows / kEwRanges say, with 8 waves of 2 rows each.  A
// lane handles EPT consecutive columns (16 bytes of dZ) of its wave's 2 rows
// per tile and sums the rows' two KL terms over them; at the end each row's
// sums are added over the wave's lanes in a fixed order, for the terms array.
// Without dz (the terms pass of the KL mixture) nothing is staged.  The rows'
// constants sit in LDS and a wave has two rows, which keeps the kernel's
// registers low: it is bound by HBM and needs the occupancy.
template <class E>
__global__ __launch_bounds__(512) void full_from_z_kernel(FullFromZArgs a) {
  constexpr int EPT = E::kEpc;
  constexpr int NT = 64 * EPT;   // columns per tile
  constexpr int RS = 1024 + 16;  // LDS row stride, bytes
  __shared__ __attribute__((aligned(16))) char tile[kEwRows * RS];
  __shared__ FullDzConst kc[kEwRows];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const long M = min(a.C, (long)*a.c.count - a.c0);
  const long i0 = (long)blockIdx.y * kEwRows;
  const long nt = (a.V + NT - 1) / NT;
  const long jb = nt * blockIdx.x / gridDim.x, je = nt * (blockIdx.x + 1) / gridDim.x;
  if (threadIdx.x < kEwRows) {
    const long i = i0 + threadIdx.x;
    const bool v = i < M;
    kc[threadIdx.x] = full_dz_const(v, v ? a.c.rows[a.c0 + i] : 0, a.lse_s, a.lse_t, a.g, a.c2, a.inv_tau, a.mix);
  }
  __syncthreads();
  float tp[2] = {0.f, 0.f}, tq[2] = {0.f, 0.f};  // sum p (yt - ys), sum q (ys - yt), base 2
  for (long j = jb; j < je; ++j) {
    const long v0 = j * NT + lane * EPT;
    const bool in = v0 < a.V;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int row = 2 * w + r;
      const long i = i0 + row;
      float o[EPT];
      if (i < M && in) {
        const FullDzConst k = kc[row];
        const float* sr = a.zs + i * a.ldz + v0;
        const float* ur = a.zt + i * a.ldz + v0;
#pragma unroll
        for (int e = 0; e < EPT; e += 4) {
          const float4 fs = *reinterpret_cast<const float4*>(sr + e);
          const float4 fu = *reinterpret_cast<const float4*>(ur + e);
          const float s4[4] = {fs.x, fs.y, fs.z, fs.w}, u4[4] = {fu.x, fu.y, fu.z, fu.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            o[e + q] = k(s4[q], u4[q]);
            const float ds = fmaf(s4[q], k.c2, -k.Ls2), dt = fmaf(u4[q], k.c2, -k.Lt2);
            const float dy = (u4[q] - s4[q]) * k.c2;  // yt - ys
            tp[r] = fmaf(fast_exp2(dt), dy, tp[r]);
            tq[r] = fmaf(fast_exp2(ds), -dy, tq[r]);
          }
        }
      } else {
#pragma unroll
        for (int q = 0; q < EPT; ++q) o[q] = 0.f;
      }
      if (a.dz) *reinterpret_cast<u32x4_t*>(tile + row * RS + lane * 16) = pack16<E>(o);
    }
    if (a.dz) {  // uniform
      __syncthreads();
      ew_store_tile<8>(tile, RS, a.dz, a.C, i0, j * 1024, a.V * E::kElem);
      __syncthreads();
    }
  }
  if (a.terms == nullptr) return;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      tp[r] += __shfl_xor(tp[r], off);
      tq[r] += __shfl_xor(tq[r], off);
    }
    if (lane == 0 && i0 + 2 * w + r < M) a.terms[(i0 + 2 * w + r) * a.nblk + blockIdx.x] = make_float2(tp[r], tq[r]);
  }
}

int full_from_z_blocks(int elem, int64_t V) { return ew_ranges(elem, V); }

hipError_t launch_full_from_z(int elem, const FullFromZArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)full_from_z_blocks(elem, a.V), (unsigned)(a.C / kEwRows)), block(512);
  if (elem == 2)
    hipLaunchKernelGGL(full_from_z_kernel<Bf16>, grid, block, 0, st, a);
  else
    hipLaunchKernelGGL(full_from_z_kernel<F32>, grid, block, 0, st, a);
  return hipGetLastError();
}

// The direct-load ring needs bf16 and both hidden widths multiples of 128.
// C: rows of the launch's panel buffers
static bool full_dma_ok(int64_t C, int64_t d, int64_t dt, int64_t V) {
  return d % kDmaKMult == 0 && dt % kDmaKMult == 0 && fits32(C * d * 2) && fits32(C * dt * 2) && fits32(d * V * 2) &&
         fits32(dt * V * 2);
}

hipError_t launch_full_fwd(int elem, const FullFwdArgs& a, hipStream_t st) {
  const dim3 grid(a.nrb * a.S), block(kThreads);
  if (elem == 2 && full_dma_ok(a.C, a.d, a.dt, a.V))
    hipLaunchKernelGGL(full_fwd_t_kernel, grid, block, 0, st, a);
  else if (elem == 2)
    hipLaunchKernelGGL((full_fwd_kernel<GenNN<Bf16, kBN>, Bf16>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((full_fwd_kernel<GenNN<F32, kBN>, F32>), grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_full_dz(int elem, const FullDzArgs& a, hipStream_t st) {
  const dim3 grid(a.nrb * a.S), block(kThreads);
  if (elem == 2 && full_dma_ok(a.C, a.d, a.dt, a.V))
    hipLaunchKernelGGL(full_dz_t_kernel, grid, block, 0, st, a);
  else if (elem == 2)
    hipLaunchKernelGGL((full_dz_kernel<GenNN<Bf16, kBN>, Bf16>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((full_dz_kernel<GenNN<F32, kBN>, F32>), grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace kd
