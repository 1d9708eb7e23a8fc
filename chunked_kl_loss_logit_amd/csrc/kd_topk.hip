// Top-K KL tiles: forward (log Z + gather) and backward dZ (recompute).
//
// "Efficient Knowledge Distillation for LLMs: Offline Top-K Logits and a Fused
// Chunked KL Loss", §3 "Offline distillation": with a cached top-K teacher only
// log Z needs the whole vocabulary; the teacher terms and the cross term use
// the K cached entries.  §3 "Fused chunked KL": the output projection is part
// of the loss, logit tiles are discarded after use, and the backward pass
// recomputes them.
//
// Grid: (valid-row block of 256) x (vocabulary split), per chunk of rows.  A
// workgroup walks the 256-wide vocabulary tiles of its split in ascending
// order; each tile is Z = H_rows . W[:, tile] on matrix cores, with H_rows
// read from the chunk's panel copy (launch_gather_panels), and the operand
// loads of the next tile run while the epilogue of this one works.  The epilogue stages the
// tile through LDS one 256 x 32 block at a time and reads it back one row per
// thread:
//   forward  : running base-2 max / sum per row, plus the index-match gather.
//              The row's cached indices are sorted, so one cursor walks them
//              in step with the column blocks and picks the hits out of LDS.
//   backward : dZ = (g/tau) (mass 2^(y - L2) - sum of w over hits), written in
//              the input dtype to the chunk's dZ buffer (panels of C rows).
// Each row carries its own constants (log2(e)/tau, 1/tau, mass) from the prep
// kernel: per-token temperature, a partial-mass teacher and a cross-entropy
// entry change those and the weights w, not the tiles.
#include <climits>

#include "kd_gemm.h"
#include "kd_launch.h"
#include "kd_main.h"

namespace kd {

namespace {

constexpr int kBN = kTileN;

// First sorted position of row entries [b, e) whose index is >= v.
__device__ inline int lower_bound(const int2* pair, int b, int e, long v) {
  while (b < e) {
    const int mid = (b + e) >> 1;
    if ((long)pair[mid].x < v) b = mid + 1; else e = mid;
  }
  return b;
}

// A row's cached entries, sorted by vocabulary index, walked in step with the
// epilogue's column blocks (ascending across the tiles of a split).
//
// No epilogue may wait on a load it issues itself: vector-memory counters
// complete in order, so that wait would also wait for the operand loads of
// the next tile that the ring issued just before the epilogue.  The cursor
// therefore keeps a window of the two entries at its position, loaded at the
// end of the previous tile's epilogue (refill) and complete long before they
// are used.  A third hit inside one tile (rare) loads synchronously and waits
// on the spot, so no load is ever pending where code paths merge.
// Positions are offsets into the [T][K] pair array (32-bit, which the
// argument checks guarantee).
struct Cursor {
  const int2* pair;  // uniform base
  int c, end;        // next position, end of the row (= its start for a row that is not valid)
  int cw;            // position of e0
  int2 e0, e1;       // entries cw and cw + 1 (meaningful below end)

  // load the window at c; every lane loads, from a valid address
  __device__ inline void refill() {
    cw = c;
    e0 = pair[c < end ? c : 0];
    e1 = pair[c + 1 < end ? c + 1 : 0];
  }
  // entry at c (c < end)
  __device__ inline int2 entry() const {
    if (c == cw) return e0;
    if (c == cw + 1) return e1;
    const int2 x = pair[c];
    wait_vm<0>();
    return x;
  }
  // calls f(index, p, position) for every entry below `lim`, moving past them
  template <class F>
  __device__ inline void take_below(int lim, F&& f) {
    while (c < end) {
      const int2 x = entry();
      if (x.x >= lim) break;
      f(x.x, __int_as_float(x.y), c);
      ++c;
    }
  }
};

// valid columns of the 32-column block at cb: [lo, hi) relative to cb, both
// multiples of 4.  Column arithmetic is 32-bit (V < 2^30): 64-bit compares
// would need vector registers.
__device__ inline void block_range(int cb, int clo, int chi, int& lo, int& hi) {
  lo = min(32, max(0, clo - cb));
  hi = max(0, min(32, chi - cb));
}

// kZ: the caller asked for z_topk.  Without it the gather keeps no output
// state, which leaves the epilogue enough registers that nothing spills (a
// spilled cursor word reloaded in the hit path made every round wait for all
// vector memory, the next tile's operand loads and earlier stores included).
template <bool kZ>
struct FwdRow {
  Cursor cur;
  const uint16_t* perm;  // uniform bases, indexed by pair position
  float* ztk;            // z_topk, indexed by row_k + original position (kZ)
  long row_k;            // t * Kz
  int kz;                // cached entries per row (a label entry has perm == kz)
  float m2, l, x, c2;
  bool rv;

  // 32 columns [cb, cb + 32) of this row, staged in st; [clo, chi) are the
  // columns this tile accounts for.  Blocks arrive in ascending column order.
  __device__ inline void consume(StPair st, int cb, int clo, int chi, float c2) {
    int lo, hi;
    block_range(cb, clo, chi, lo, hi);
    if (lo >= hi || !rv) return;
    const int r = opaque((int)threadIdx.x);
    float4 f[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = st_read4(st, r, j);
    // block maximum over the valid chunks, then the scaled sum
    float cm = -INFINITY;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float b = fmaxf(fmaxf(f[j].x, f[j].y), fmaxf(f[j].z, f[j].w));
      cm = (4 * j >= lo && 4 * j < hi) ? fmaxf(cm, b) : cm;
    }
    const float cmy = cm * c2;
    l = cmy > m2 ? l * fast_exp2(m2 - cmy) : l;  // 2^(-inf) = 0 while l is still 0
    m2 = fmaxf(m2, cmy);
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float e = fast_exp2(fmaf(f[j].x, c2, -m2)) + fast_exp2(fmaf(f[j].y, c2, -m2)) +
                      fast_exp2(fmaf(f[j].z, c2, -m2)) + fast_exp2(fmaf(f[j].w, c2, -m2));
      sum += (4 * j >= lo && 4 * j < hi) ? e : 0.f;
    }
    l += sum;
    // index-match gather: cached indices that fall in this block
    cur.take_below(cb + hi, [&](int v, float pv, int c) {
      const float z = st_row(st, r)[st_pos(r, v - cb)];
      x = fmaf(pv, z, x);
      if constexpr (kZ) {
        const int k = perm[c];
        if (k < kz) ztk[row_k + k] = z;
      }
    });
  }
};

struct DzRow {
  Cursor cur;
  float L2, gs, c2;  // L2: base-2 log Z less log2(mass), so 2^(y - L2) = mass q
  bool rv;

  // replace the staged logits of this row by dZ (zero outside the valid rows
  // and the columns [clo, chi))
  __device__ inline void consume(StPair st, int cb, int clo, int chi, float c2) {
    const int r = opaque((int)threadIdx.x);
    int lo, hi;
    block_range(cb, clo, chi, lo, hi);
    if (!rv) hi = 0;
    float4 f[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = st_read4(st, r, j);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool v = 4 * j >= lo && 4 * j < hi;
      float4 o;
      o.x = v ? gs * fast_exp2(fmaf(f[j].x, c2, -L2)) : 0.f;
      o.y = v ? gs * fast_exp2(fmaf(f[j].y, c2, -L2)) : 0.f;
      o.z = v ? gs * fast_exp2(fmaf(f[j].z, c2, -L2)) : 0.f;
      o.w = v ? gs * fast_exp2(fmaf(f[j].w, c2, -L2)) : 0.f;
      st_write4(st, r, j, o);
    }
    cur.take_below(cb + hi, [&](int v, float pv, int) {  // scatter-add of the teacher mass
      st_row(st, r)[st_pos(r, v - cb)] -= gs * pv;
    });
  }
};

// Vocabulary tile vt of a split is staged from column n0 = min(256 vt, V - 256)
// and accounts for columns [256 vt, min(256 vt + 256, V)): a last partial
// tile is shifted left so that every operand load stays inside W (its first
// columns were the previous tile's).  Vocabularies under 256 columns take one
// tile at 0 whose loads are bounded by the general mainloop.
__device__ inline int tile_n0(int vt, int V) { return V >= kBN ? min(vt * kBN, V - kBN) : 0; }

// The epilogue walks the 256 x 256 tile in eight rounds of one 32-column
// block (wave column half h, block NBI) staged in the epilogue array, in
// ascending column order: half 0 blocks 0..3, then half 1.
template <int H, int NBI, class Row>
__device__ inline void fwd_round(const Slots& sl, const f32x16_t (&acc)[4][4], int n0, int lo, int hi, Row& R,
                                 const TopkFwdArgs& a, long row0, long M) {
  const int cb = n0 + H * 128 + NBI * 32;
  stage_half<NBI, 4>(sl.ep, H, acc);
  ring_barrier();
  R.consume(sl.ep, cb, lo, hi, R.c2);
  // both only read the staged block: the logits go out as they are
  if (a.zout) store_block<F32>(sl.ep, reinterpret_cast<char*>(a.zout), a.ldz, row0, cb, M, a.ldz, lo);
  ring_barrier();
}

template <class E, int H, int NBI>
__device__ inline void dz_round(const Slots& sl, const f32x16_t (&acc)[4][4], int n0, int lo, int hi, long row0,
                                DzRow& R, const TopkDzArgs& a) {
  const int cb = n0 + H * 128 + NBI * 32;
  stage_half<NBI, 4>(sl.ep, H, acc);
  ring_barrier();
  R.consume(sl.ep, cb, lo, hi, R.c2);
  ring_barrier();
  store_block<E>(sl.ep, a.dz, a.ldz, row0, cb, LONG_MAX, a.ldz, lo, a.C);
  ring_barrier();
}

}  // namespace

// Rows: the compacted valid rows [c0, c0 + C) (the plain forward takes them
// all); partials are indexed by compacted position, and with zout set the
// tile's logits are also written out, fp32, one row per compacted row.
template <class Main, class E, bool kZ>
__global__ __launch_bounds__(kThreads, 1) void topk_fwd_kernel(TopkFwdArgs a) {
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
  const int V = (int)a.V;
  const int32_t* rows = a.c.rows + a.c0;

  Main mainloop;
  mainloop.init(
      a.Hp, [&](int r) -> const char* { return row0 + r < M ? a.Hp + (row0 + r) * kRowB : nullptr; }, a.W,
      a.V * E::kElem, a.V, a.d, a.C * kRowB);

  const int ti = row0 + (int)threadIdx.x;
  FwdRow<kZ> R;
  R.rv = ti < M;
  const long t = R.rv ? rows[ti] : 0;
  R.cur.pair = a.rd.pair;
  R.cur.end = (int)(t * a.K + (R.rv ? a.K : 0));
  R.cur.c = lower_bound(a.rd.pair, (int)(t * a.K), R.cur.end, (long)tb * kBN);
  R.cur.refill();
  R.perm = a.rd.perm;
  R.ztk = a.z_topk;
  R.row_k = t * a.Kz;
  R.kz = (int)a.Kz;
  R.m2 = -INFINITY;
  R.l = 0.f;
  R.x = 0.f;
  R.c2 = R.rv ? a.rd.rowc[t].x : 0.f;

  mainloop.run(
      sl, te - tb, [&](int i) { return TileAt{0, tile_n0(tb + i, V)}; },
      [&](int i, const f32x16_t (&acc)[4][4]) {
        const int vt = tb + i, n0 = tile_n0(vt, V), lo = vt * kBN, hi = min(lo + kBN, V);
        fwd_round<0, 0>(sl, acc, n0, lo, hi, R, a, row0, M);
        fwd_round<0, 1>(sl, acc, n0, lo, hi, R, a, row0, M);
        fwd_round<0, 2>(sl, acc, n0, lo, hi, R, a, row0, M);
        fwd_round<0, 3>(sl, acc, n0, lo, hi, R, a, row0, M);
        fwd_round<1, 0>(sl, acc, n0, lo, hi, R, a, row0, M);
        fwd_round<1, 1>(sl, acc, n0, lo, hi, R, a, row0, M);
        fwd_round<1, 2>(sl, acc, n0, lo, hi, R, a, row0, M);
        fwd_round<1, 3>(sl, acc, n0, lo, hi, R, a, row0, M);
        R.cur.refill();
      });
  if (R.rv) {
    float4* o = reinterpret_cast<float4*>(a.part) + (long)sp * a.part_stride + (a.c0 - a.part_row0) + ti;
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
  grouped_coords(xcd_remap(blockIdx.x, gridDim.x), a.nrb, a.S, a.group, rb, sp);
  const int row0 = rb * kBM;
  if (row0 >= M) return;
  const int tb = (int)((long)a.ntiles * sp / a.S);
  const int te = (int)((long)a.ntiles * (sp + 1) / a.S);
  const int V = (int)a.V;
  const int32_t* rows = a.c.rows + a.c0;

  Main mainloop;
  mainloop.init(
      a.Hp, [&](int r) -> const char* { return row0 + r < M ? a.Hp + (row0 + r) * kRowB : nullptr; }, a.W,
      a.V * E::kElem, a.V, a.d, a.C * kRowB);

  const int ti = row0 + (int)threadIdx.x;
  DzRow R;
  R.rv = ti < M;
  const long t = R.rv ? rows[ti] : 0;
  R.cur.pair = a.rd.pair;
  R.cur.end = (int)(t * a.K + (R.rv ? a.K : 0));
  R.cur.c = lower_bound(a.rd.pair, (int)(t * a.K), R.cur.end, (long)tb * kBN);
  R.cur.refill();
  const float4 rc = R.rv ? a.rd.rowc[t] : make_float4(0.f, 0.f, 1.f, 0.f);
  R.L2 = R.rv ? a.lse[t] * kLog2e - rc.w : 0.f;
  R.gs = R.rv ? a.g[t] * rc.y : 0.f;
  R.c2 = rc.x;

  mainloop.run(
      sl, te - tb, [&](int i) { return TileAt{0, tile_n0(tb + i, V)}; },
      [&](int i, const f32x16_t (&acc)[4][4]) {
        const int vt = tb + i, n0 = tile_n0(vt, V), lo = vt * kBN, hi = min(lo + kBN, V);
        dz_round<E, 0, 0>(sl, acc, n0, lo, hi, row0, R, a);
        dz_round<E, 0, 1>(sl, acc, n0, lo, hi, row0, R, a);
        dz_round<E, 0, 2>(sl, acc, n0, lo, hi, row0, R, a);
        dz_round<E, 0, 3>(sl, acc, n0, lo, hi, row0, R, a);
        dz_round<E, 1, 0>(sl, acc, n0, lo, hi, row0, R, a);
        dz_round<E, 1, 1>(sl, acc, n0, lo, hi, row0, R, a);
        dz_round<E, 1, 2>(sl, acc, n0, lo, hi, row0, R, a);
        dz_round<E, 1, 3>(sl, acc, n0, lo, hi, row0, R, a);
        R.cur.refill();
      });
}

// ---------------------------------------------------------------- dZ from stored logits
constexpr int kDzzRows = 64;    // rows per block of the top-K elementwise dZ pass
constexpr int kDzzRanges = 64;  // column ranges per block row

// A block covers kDzzRows rows and one of at most kDzzRanges ranges of the
// rows' 64-byte dZ pieces, four threads per piece, so each wave writes 16
// consecutive rows of a piece: a contiguous kilobyte of the panels (staging
// through LDS, as the full pass does, measured slower here).  A thread handles
// EPT consecutive columns (16 bytes of dZ) of its row in each piece of the
// block's range, with the recomputing tile's epilogue formula.  The row's
// entries are sorted and the thread's columns ascend, so one cursor walks the
// hits in order; they are subtracted before the one rounding to the element
// type.
template <class E>
__global__ __launch_bounds__(256) void topk_dz_from_z_kernel(TopkDzFromZArgs a) {
  constexpr int EPT = E::kEpc;
  constexpr int PC = kRowB / E::kElem;  // columns per piece
  const long i = (long)blockIdx.y * kDzzRows + (threadIdx.x >> 2);  // row of the chunk
  const int sub = threadIdx.x & 3;
  const long np = (a.V * E::kElem + kRowB - 1) / kRowB;
  const long pb = np * blockIdx.x / gridDim.x, pe = np * (blockIdx.x + 1) / gridDim.x;
  const long M = min(a.C, (long)*a.c.count - a.c0);
  const bool rv = i < M;
  float L2 = 0.f, gs = 0.f, c2 = 0.f;
  int c = 0, ce = 0;
  if (rv) {
    const long t = a.c.rows[a.c0 + i];
    const float4 rc = a.rd.rowc[t];
    L2 = a.lse[t] * kLog2e - rc.w;
    gs = a.g[t] * rc.y;
    c2 = rc.x;
    ce = (int)(t * a.K + a.K);
    c = lower_bound(a.rd.pair, (int)(t * a.K), ce, pb * PC);
  }
  const float* zr = a.z + i * a.ldz;
  for (long p = pb; p < pe; ++p) {
    const long v0 = p * PC + sub * EPT;
    if (v0 >= a.V) break;
    float o[EPT];
    if (rv) {
#pragma unroll
      for (int e = 0; e < EPT; e += 4) {
        const float4 z4 = *reinterpret_cast<const float4*>(zr + v0 + e);
        o[e + 0] = gs * fast_exp2(fmaf(z4.x, c2, -L2));
        o[e + 1] = gs * fast_exp2(fmaf(z4.y, c2, -L2));
        o[e + 2] = gs * fast_exp2(fmaf(z4.z, c2, -L2));
        o[e + 3] = gs * fast_exp2(fmaf(z4.w, c2, -L2));
      }
      for (; c < ce; ++c) {
        const int2 pr = a.rd.pair[c];
        if ((long)pr.x >= v0 + EPT) break;
        if ((long)pr.x < v0) continue;  // another thread's columns
#pragma unroll
        for (int q = 0; q < EPT; ++q) o[q] = (long)pr.x == v0 + q ? o[q] - gs * __int_as_float(pr.y) : o[q];
      }
    } else {
#pragma unroll
      for (int q = 0; q < EPT; ++q) o[q] = 0.f;
    }
    *reinterpret_cast<u32x4_t*>(a.dz + panel_off(a.C, i, v0 * E::kElem)) = pack16<E>(o);
  }
}

hipError_t launch_topk_dz_from_z(int elem, const TopkDzFromZArgs& a, hipStream_t st) {
  const int64_t pieces = (a.V * elem + kRowB - 1) / kRowB;
  const dim3 grid((unsigned)std::min<int64_t>(kDzzRanges, pieces), (unsigned)(a.C / kDzzRows)), block(256);
  if (elem == 2)
    hipLaunchKernelGGL(topk_dz_from_z_kernel<Bf16>, grid, block, 0, st, a);
  else
    hipLaunchKernelGGL(topk_dz_from_z_kernel<F32>, grid, block, 0, st, a);
  return hipGetLastError();
}

// The direct-load ring needs bf16, a hidden width that is a multiple of 128
// and at least one whole 256-column tile of vocabulary.
template <bool kZ>
static void launch_topk_fwd_z(int elem, const TopkFwdArgs& a, hipStream_t st) {
  const dim3 grid(a.nrb * a.S), block(kThreads);
  if (elem == 2 && a.d % kDmaKMult == 0 && a.V >= kBN && fits32(a.C * a.d * 2) && fits32(a.d * a.V * 2))
    hipLaunchKernelGGL((topk_fwd_kernel<DmaNN<kBN>, Bf16, kZ>), grid, block, 0, st, a);
  else if (elem == 2)
    hipLaunchKernelGGL((topk_fwd_kernel<GenNN<Bf16, kBN>, Bf16, kZ>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((topk_fwd_kernel<GenNN<F32, kBN>, F32, kZ>), grid, block, 0, st, a);
}

hipError_t launch_topk_fwd(int elem, const TopkFwdArgs& a, hipStream_t st) {
  if (a.z_topk)
    launch_topk_fwd_z<true>(elem, a, st);
  else
    launch_topk_fwd_z<false>(elem, a, st);
  return hipGetLastError();
}

hipError_t launch_topk_dz(int elem, const TopkDzArgs& a, hipStream_t st) {
  const dim3 grid(a.nrb * a.S), block(kThreads);
  if (elem == 2 && a.d % kDmaKMult == 0 && a.V >= kBN && fits32(a.C * a.d * 2) && fits32(a.d * a.V * 2))
    hipLaunchKernelGGL((topk_dz_kernel<DmaNN<kBN>, Bf16>), grid, block, 0, st, a);
  else if (elem == 2)
    hipLaunchKernelGGL((topk_dz_kernel<GenNN<Bf16, kBN>, Bf16>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((topk_dz_kernel<GenNN<F32, kBN>, F32>), grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace kd
