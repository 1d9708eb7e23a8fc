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
// On the direct-load path (bf16) both are accumulated transposed instead,
// each lane holding 16 columns of one row per 32 x 32 block, and the
// epilogues work in registers (topk_fwd_t_kernel, topk_dz_t_kernel): the
// forward keeps per-lane running maxima and sums that two lane exchanges
// merge at the end of a split, the backward turns each register into dZ.
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
  // moves past every entry below `lim` without using it
  __device__ inline void skip_below(int lim) {
    while (c < end && entry().x < lim) ++c;
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

// kZ: the caller asked for z_topk.  A hit then stores its logit at the
// entry's sorted position (rd.zpair, one address from the cursor), and a
// small kernel puts them in z_topk's order afterwards: mapping to the
// original position in the hit path (the permutation load and the row's
// offset) cost registers, and a spilled cursor word reloaded there made
// every round wait for all vector memory, the next tile's operand loads and
// earlier stores included.
template <bool kZ>
struct FwdRow {
  Cursor cur;
  float* zp;  // rd.zpair, indexed by pair position (kZ)
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
      if constexpr (kZ) zp[c] = z;
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
  R.zp = a.rd.zpair;
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

// ---------------------------------------------------------------- dZ tiles, accumulators transposed
// The direct-load (bf16) form of topk_dz_kernel.  The tile's products are
// accumulated transposed (mma_frags_t): lane l of wave (wm, wn) owns chunk
// row wm 128 + 32 mb + l % 32 of the tile in block row mb, and register i of
// block (mb, nb) holds vocabulary column wn 128 + 32 nb + 8 (i / 4) +
// 4 (l / 32) + i % 4 of it.  dZ of a register is then a function of that
// register and its row's constants alone, so the epilogue needs neither
// staged fp32 blocks nor workgroup barriers: each lane turns its values into
// dZ, subtracts the teacher weights at the cached entries of its rows that
// fall in its columns (one cursor per row, ascending), rounds to bf16, and
// each 32 x 32 block goes through a wave-private 2 KB LDS region so that the
// stores to the dZ panels are whole kilobytes.
//
// The main loop leaves few registers free, so only each row's cursor
// position and end stay in registers.  The rows' constants sit in LDS for
// the whole kernel, and the two entries at each cursor are brought in by
// direct-to-LDS loads issued at the end of the previous tile's epilogue:
// they land while the next tile is contracted, no register waits for them,
// and no epilogue waits on a load of its own (a third entry of one row in
// one tile's half, rare, is loaded on the spot as in Cursor::entry).
constexpr int kStgBytes = 2048;            // per wave: 32 rows x 64 bytes
constexpr int kWinBytes = 4 * 4 * 64 * 4;  // per wave: 4 rows x 4 words x 64 lanes

// Byte position of 8 bytes (half hh of 16-byte chunk j) of row r in a
// wave's [32][64 B] staging region.  The chunk is XOR-swizzled with
// (r / 4) % 4 and the half with (r / 16) % 2: the 32 rows a half-wave writes
// at once land in 32 distinct 8-byte bank groups, and the 4 chunks of the
// 4 rows a quarter-wave reads back in 16 distinct 16-byte ones.
__device__ inline int stg8(int r, int j, int hh) {
  return r * 64 + ((j ^ ((r >> 2) & 3)) << 4) + ((hh ^ ((r >> 4) & 1)) << 3);
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// two floats to bf16 bits, round to nearest even (v_cvt_pk_bf16_f32)
__device__ inline uint32_t pk_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// A row's cached entries as the transposed epilogues walk them: the position
// and end live in registers; the window (the entries at the position when
// the epilogue starts) was loaded into LDS by refill().
struct TCursor {
  int c, end;
  int c0;       // position of the window (the cursor at the epilogue's start)
  int2 e0, e1;  // window entries c0, c0 + 1 (meaningful below end)
  __device__ inline int2 entry(const int2* pair) const {
    if (c == c0) return e0;
    if (c == c0 + 1) return e1;
    const int2 x = pair[c];
    wait_vm<0>();
    return x;
  }
  __device__ inline void skip_below(const int2* pair, int lim) {
    while (c < end && entry(pair).x < lim) ++c;
  }
  template <class F>
  __device__ inline void take_below(const int2* pair, int lim, F&& f) {
    while (c < end) {
      const int2 x = entry(pair);
      if (x.x >= lim) break;
      f(x.x, __int_as_float(x.y), c);
      ++c;
    }
  }
};

// Direct-to-LDS loads of the window of each of a lane's four rows: word q of
// row mb at win + (4 mb + q) * 256 + 4 lane.
__device__ inline void twin_refill(__amdgpu_buffer_rsrc_t rs, const int (&c)[4], const int (&end)[4], char* win) {
  win = reinterpret_cast<char*>(opaque_ptr(win));
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int pos = c[mb] + (q >> 1);
      const uint32_t off = (uint32_t)(pos < end[mb] ? pos : 0) * 8u + 4u * (q & 1);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (KD_LDS void*)(win + (4 * mb + q) * 256), 4, (int)off, 0, 0, 0);
    }
}
__device__ inline void twin_read(const char* win, int mb, TCursor& t) {
  const int lane = opaque((int)threadIdx.x) & 63;
  const int* w = reinterpret_cast<const int*>(win + 1024 * mb) + lane;
  t.e0 = make_int2(w[0 * 64], w[1 * 64]);
  t.e1 = make_int2(w[2 * 64], w[3 * 64]);
}

// One 32 x 32 block (mb, nb) of the wave's share of a tile: dZ of the lane's
// row mb at its 16 columns, staged as bf16 and written to the chunk's panels.
// Columns [lo, hi) are the tile's own (a shifted last tile starts before lo;
// columns at or past V read as zero), stored from lo on.  rk = (L2, gs, c2)
// of the row; gs = 0 on rows past the chunk's valid rows (dZ = 0 there).
template <bool kFull>
__device__ inline void dz_block_t(const f32x16_t& v, const float4 rk, TCursor& cur, const int2* pair, int cb,
                                  int lo, int hi, char* stg, char* dz, long C, long brow0) {
  // lane quantities recomputed per block (opaque), not hoisted out of the
  // tile loop where they would hold registers through the main loop
  const int lane = opaque((int)threadIdx.x) & 63, h = lane >> 5, cl = lane & 31;
  float o[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float e = rk.y * fast_exp2(fmaf(v[i], rk.z, -rk.x));
    if constexpr (kFull)
      o[i] = e;
    else
      o[i] = cb + 8 * (i >> 2) + 4 * h + (i & 3) < hi ? e : 0.f;
  }
  // scatter-add of the teacher weights at the row's cached entries in the
  // block (each lane takes those in its own columns)
  cur.take_below(pair, min(cb + 32, hi), [&](int idx, float p, int) {
    const int dcol = idx - cb;
    if (((dcol >> 2) & 1) == h) {
      const int at = ((dcol >> 3) << 2) | (dcol & 3);
      const float gp = rk.y * p;
#pragma unroll
      for (int i = 0; i < 16; ++i) o[i] = i == at ? o[i] - gp : o[i];
    }
  });
#pragma unroll
  for (int j = 0; j < 4; ++j)
    *reinterpret_cast<uint2*>(stg + stg8(cl, j, h)) =
        make_uint2(pk_bf16(o[4 * j], o[4 * j + 1]), pk_bf16(o[4 * j + 2], o[4 * j + 3]));
  // back out of LDS (the same wave: its LDS accesses complete in order, no
  // barrier), 16 bytes per lane, 16 consecutive rows of one 64-byte panel
  // piece per store instruction
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int r = k * 16 + (lane >> 2), j = lane & 3;
    const uint4 q = *reinterpret_cast<const uint4*>(stg + r * 64 + ((j ^ ((r >> 2) & 3)) << 4));
    const uint4 w = ((r >> 4) & 1) ? make_uint4(q.z, q.w, q.x, q.y) : q;  // halves stored exchanged
    const int col = cb + 8 * j;
    if (kFull || col >= lo) *reinterpret_cast<uint4*>(dz + panel_off(C, brow0 + r, (long)col * 2)) = w;
  }
}

template <bool kFull>
__device__ inline void dz_tile_t(const f32x16_t (&acc)[4][4], const float4* rowk, TCursor (&R)[4], const int2* pair,
                                 int base, int lo, int hi, char* stg, char* dz, long C, int wrow0, int trow0) {
  const int lane = opaque((int)threadIdx.x) & 63;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const float4 rk = rowk[trow0 + mb * 32 + (lane & 31)];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
      dz_block_t<kFull>(acc[mb][nb], rk, R[mb], pair, base + 32 * nb, lo, hi, stg, dz, C, wrow0 + mb * 32);
  }
}

__global__ __launch_bounds__(kThreads, 1) void topk_dz_t_kernel(TopkDzArgs a) {
  __shared__ __attribute__((aligned(16))) char sl_0[kSlotBytes];
  __shared__ __attribute__((aligned(16))) char sl_1[kSlotBytes];
  __shared__ __attribute__((aligned(16))) char sl_2[kSlotBytes];
  __shared__ __attribute__((aligned(16))) char sl_3[kSlotBytes];
  __shared__ __attribute__((aligned(16))) char stg_all[4 * kStgBytes];
  __shared__ __attribute__((aligned(16))) float4 rowk[kBM];
  __shared__ __attribute__((aligned(16))) char win_all[4 * kWinBytes];
  const Slots sl{sl_0, sl_1, sl_2, sl_3, nullptr};

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
  const int2* pair = a.rd.pair;

  DmaNN<kBN> mainloop;
  mainloop.init(
      a.Hp, [&](int r) -> const char* { return row0 + r < M ? a.Hp + (row0 + r) * kRowB : nullptr; }, a.W,
      a.V * 2, a.V, a.d, a.C * kRowB);

  const int w = wave_id(), wm = w >> 1, wn = w & 1;
  const int lane = (int)threadIdx.x & 63;
  const int trow0 = wm * 128;        // the wave's first row of the tile
  const int wrow0 = row0 + trow0;    // ... of the chunk
  char* stg = stg_all + w * kStgBytes;
  char* win = win_all + w * kWinBytes;
  const __amdgpu_buffer_rsrc_t prs = make_rsrc(reinterpret_cast<const char*>(pair));
  int cpos[4], cend[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int ti = wrow0 + mb * 32 + (lane & 31);
    const bool rv = ti < M;
    const long t = rv ? rows[ti] : 0;
    cend[mb] = (int)(t * a.K + (rv ? a.K : 0));
    cpos[mb] = lower_bound(pair, (int)(t * a.K), cend[mb], (long)tb * kBN);
    if (wn == 0 && lane < 32) {
      const float4 rc = rv ? a.rd.rowc[t] : make_float4(0.f, 0.f, 1.f, 0.f);
      rowk[trow0 + mb * 32 + lane] = make_float4(rv ? a.lse[t] * kLog2e - rc.w : 0.f, rv ? a.g[t] * rc.y : 0.f,
                                                 rc.x, 0.f);
    }
  }
  twin_refill(prs, cpos, cend, win);  // lands before the ring's first wait

  mainloop.template run<true>(
      sl, te - tb, [&](int i) { return TileAt{0, tile_n0(tb + i, V)}; },
      [&](int i, const f32x16_t (&acc)[4][4]) {
        const int vt = tb + i, n0 = tile_n0(vt, V), lo = vt * kBN, hi = min(lo + kBN, V);
        const int base = n0 + wn * 128;
        TCursor R[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          R[mb].c = R[mb].c0 = cpos[mb];
          R[mb].end = cend[mb];
          twin_read(win, mb, R[mb]);
          // entries before this wave's columns (the other wave's half of the
          // previous tile) are passed over
          R[mb].skip_below(pair, max(base, lo));
        }
        if (n0 == lo && lo + kBN <= hi)
          dz_tile_t<true>(acc, rowk, R, pair, base, lo, hi, stg, a.dz, a.C, wrow0, trow0);
        else
          dz_tile_t<false>(acc, rowk, R, pair, base, lo, hi, stg, a.dz, a.C, wrow0, trow0);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) cpos[mb] = R[mb].c;
        twin_refill(prs, cpos, cend, win);
      });
}

// ---------------------------------------------------------------- forward tiles, accumulators transposed
// The direct-load (bf16) form of topk_fwd_kernel, with the tile accumulated
// transposed as in topk_dz_t_kernel.  Each lane keeps, for each of its four
// rows, a running base-2 maximum and scaled sum over its own columns (16 per
// block, 64 per tile) and its part of the gather, Σ w z over the cached
// entries that fall in its columns; these live in LDS between tiles (the
// main loop leaves no registers for them).  After the split's last tile the
// two lanes of a row and then the two waves of a row (its column halves)
// merge their parts in a fixed order into the split's partial (m2, l, x).
// With zout set the raw logits also go out, fp32, 16 bytes per lane.
constexpr int kFstBytes = 3 * 4 * 64 * 4;  // per wave: (m2, l, x) of 4 rows x 64 lanes

// One row's update from its 64 values in the lane (val(nb, i): column
// base + 32 nb + 8 (i / 4) + 4 (l / 32) + i % 4, -inf where the column is not
// the tile's own): running maximum and scaled sum, then the gather of the
// cached entries in the lane's columns.
template <bool kZ, class Val>
__device__ inline void fwd_row_t(Val&& val, float c2, float* st, TCursor& cur, const int2* pair, int base, int hi,
                                 const TopkFwdArgs& a) {
  const int lane = opaque((int)threadIdx.x) & 63, h = lane >> 5;
  float m2 = st[0], l = st[64], x = st[128];
  float cm = -INFINITY;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int i = 0; i < 16; ++i) cm = fmaxf(cm, val(nb, i));
  const float cmy = cm * c2;
  l = cmy > m2 ? l * fast_exp2(m2 - cmy) : l;  // 2^(-inf) = 0 while l is still 0
  m2 = fmaxf(m2, cmy);
  float sum = 0.f;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int i = 0; i < 16; ++i) sum += fast_exp2(fmaf(val(nb, i), c2, -m2));  // -inf columns add 0
  // a lane whose columns are all outside the tile keeps m2 = -inf and adds
  // nothing (2^(-inf - -inf) would be NaN)
  l += cm == -INFINITY ? 0.f : sum;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int cb = base + 32 * nb;
    cur.take_below(pair, min(cb + 32, hi), [&](int idx, float p, int c) {
      const int dcol = idx - cb;
      if (((dcol >> 2) & 1) == h) {
        const int at = ((dcol >> 3) << 2) | (dcol & 3);
        float z = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) z = i == at ? val(nb, i) : z;
        x = fmaf(p, z, x);
        if constexpr (kZ) a.rd.zpair[c] = z;
      }
    });
  }
  st[0] = m2;
  st[64] = l;
  st[128] = x;
}

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// The tile's raw logits of one row (the columns from lo on), fp32, 16 bytes
// per lane: four consecutive accumulator registers per store, taken as they
// are (gfx950 stores take accumulator registers as data).
template <int NB, int J>
__device__ inline void zout4(const f32x16_t (&acc)[4], float* zr, int base, int lo, int h) {
  const int col = base + 32 * NB + 8 * J + 4 * h;
  if (col >= lo)
    *reinterpret_cast<f32x4_t*>(zr + col) =
        __builtin_shufflevector(acc[NB], acc[NB], 4 * J, 4 * J + 1, 4 * J + 2, 4 * J + 3);
}
template <int NB>
__device__ inline void zout_nb(const f32x16_t (&acc)[4], float* zr, int base, int lo, int h) {
  zout4<NB, 0>(acc, zr, base, lo, h);
  zout4<NB, 1>(acc, zr, base, lo, h);
  zout4<NB, 2>(acc, zr, base, lo, h);
  zout4<NB, 3>(acc, zr, base, lo, h);
}
__device__ inline void fwd_zout_t(const f32x16_t (&acc)[4], float* zr, int base, int lo) {
  const int h = (opaque((int)threadIdx.x) >> 5) & 1;
  zout_nb<0>(acc, zr, base, lo, h);
  zout_nb<1>(acc, zr, base, lo, h);
  zout_nb<2>(acc, zr, base, lo, h);
  zout_nb<3>(acc, zr, base, lo, h);
}

// base-2 (max, sum, cross) parts of one row over two column sets, merged
__device__ inline void merge_part(float& m2, float& l, float& x, float om2, float ol, float ox) {
  const float m = fmaxf(m2, om2);
  l = (m2 == -INFINITY ? 0.f : l * fast_exp2(m2 - m)) + (om2 == -INFINITY ? 0.f : ol * fast_exp2(om2 - m));
  m2 = m;
  x += ox;
}

template <bool kZ, bool kOut>
__global__ __launch_bounds__(kThreads, 1) void topk_fwd_t_kernel(TopkFwdArgs a) {
  __shared__ __attribute__((aligned(16))) char sl_0[kSlotBytes];
  __shared__ __attribute__((aligned(16))) char sl_1[kSlotBytes];
  __shared__ __attribute__((aligned(16))) char sl_2[kSlotBytes];
  __shared__ __attribute__((aligned(16))) char sl_3[kSlotBytes];
  __shared__ __attribute__((aligned(16))) char win_all[4 * kWinBytes];
  __shared__ __attribute__((aligned(16))) float fst_all[4 * kFstBytes / 4];
  __shared__ float c2k[kBM];
  const Slots sl{sl_0, sl_1, sl_2, sl_3, nullptr};

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
  const int2* pair = a.rd.pair;

  DmaNN<kBN> mainloop;
  mainloop.init(
      a.Hp, [&](int r) -> const char* { return row0 + r < M ? a.Hp + (row0 + r) * kRowB : nullptr; }, a.W,
      a.V * 2, a.V, a.d, a.C * kRowB);

  const int w = wave_id(), wm = w >> 1, wn = w & 1;
  const int lane = (int)threadIdx.x & 63;
  const int trow0 = wm * 128;
  char* win = win_all + w * kWinBytes;
  float* fst = fst_all + w * (kFstBytes / 4);
  const __amdgpu_buffer_rsrc_t prs = make_rsrc(reinterpret_cast<const char*>(pair));
  int cpos[4], cend[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int ti = row0 + trow0 + mb * 32 + (lane & 31);
    const bool rv = ti < M;
    const long t = rv ? rows[ti] : 0;
    cend[mb] = (int)(t * a.K + (rv ? a.K : 0));
    cpos[mb] = lower_bound(pair, (int)(t * a.K), cend[mb], (long)tb * kBN);
    if (wn == 0 && lane < 32) c2k[trow0 + mb * 32 + lane] = rv ? a.rd.rowc[t].x : 1.f;
    fst[mb * 192 + lane] = -INFINITY;
    fst[mb * 192 + 64 + lane] = 0.f;
    fst[mb * 192 + 128 + lane] = 0.f;
  }
  twin_refill(prs, cpos, cend, win);  // lands before the ring's first wait

  mainloop.template run<true>(
      sl, te - tb, [&](int i) { return TileAt{0, tile_n0(tb + i, V)}; },
      [&](int i, const f32x16_t (&acc)[4][4]) {
        const int vt = tb + i, n0 = tile_n0(vt, V), lo = vt * kBN, hi = min(lo + kBN, V);
        const int base = n0 + wn * 128;
        const bool full = n0 == lo && lo + kBN <= hi;
        const int ln = opaque((int)threadIdx.x) & 63;
        if constexpr (kOut) {  // the logits first, straight from the accumulators
          const int zr0 = opaque(row0 + trow0 + (ln & 31));  // the lane's row of block row 0
          float* zp = a.zout + (long)zr0 * a.ldz;
#pragma unroll
          for (int mb = 0; mb < 4; ++mb)
            if (zr0 + mb * 32 < M) fwd_zout_t(acc[mb], zp + (long)mb * 32 * a.ldz, base, lo);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          TCursor R;
          R.c = R.c0 = cpos[mb];
          R.end = cend[mb];
          twin_read(win, mb, R);
          R.skip_below(pair, max(base, lo));
          const float c2 = c2k[trow0 + mb * 32 + (ln & 31)];
          float* st = fst + mb * 192 + ln;
          if (full) {
            fwd_row_t<kZ>([&](int nb, int i) { return acc[mb][nb][i]; }, c2, st, R, pair, base, hi, a);
          } else {
            // only the tile's own columns [lo, hi) count: a group of four
            // (lo, hi and base are multiples of 8) outside them gets -inf
            // added, which drops it from the maximum and the sum
            float pen[16];
            const int h4 = 4 * (ln >> 5);
#pragma unroll
            for (int g = 0; g < 16; ++g) {
              const int col = base + 32 * (g >> 2) + 8 * (g & 3) + h4;
              pen[g] = col >= lo && col < hi ? 0.f : -INFINITY;
            }
            fwd_row_t<kZ>([&](int nb, int i) { return acc[mb][nb][i] + pen[4 * nb + (i >> 2)]; }, c2, st, R, pair,
                          base, hi, a);
          }
          cpos[mb] = R.c;
        }
        twin_refill(prs, cpos, cend, win);
      });

  // the split's partial per row: lane halves, then column halves (wave wn = 1
  // hands its parts to wave wn = 0 through slot 0, free after the ring)
  float4* xch = reinterpret_cast<float4*>(sl_0);
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    float m2 = fst[mb * 192 + lane], l = fst[mb * 192 + 64 + lane], x = fst[mb * 192 + 128 + lane];
    const float om2 = __shfl_xor(m2, 32), ol = __shfl_xor(l, 32), ox = __shfl_xor(x, 32);
    if (lane < 32) merge_part(m2, l, x, om2, ol, ox);
    if (wn == 1 && lane < 32) xch[trow0 + mb * 32 + lane] = make_float4(m2, l, x, 0.f);
    fst[mb * 192 + lane] = m2;
    fst[mb * 192 + 64 + lane] = l;
    fst[mb * 192 + 128 + lane] = x;
  }
  __syncthreads();
  if (wn == 0 && lane < 32) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int ti = row0 + trow0 + mb * 32 + lane;
      if (ti >= M) continue;
      float m2 = fst[mb * 192 + lane], l = fst[mb * 192 + 64 + lane], x = fst[mb * 192 + 128 + lane];
      const float4 o = xch[trow0 + mb * 32 + lane];
      merge_part(m2, l, x, o.x, o.y, o.z);
      float4* dst = reinterpret_cast<float4*>(a.part) + (long)sp * a.part_stride + (a.c0 - a.part_row0) + ti;
      *dst = make_float4(m2, l, x, 0.f);
    }
  }
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
  // the row's next cached entry, kept in registers between pieces (most
  // pieces hold none of the row's K entries)
  int2 nx = rv && c < ce ? a.rd.pair[c] : make_int2(INT_MAX, 0);
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
      while ((long)nx.x < v0 + EPT) {  // entries below v0 are another thread's columns
        if ((long)nx.x >= v0) {
#pragma unroll
          for (int q = 0; q < EPT; ++q) o[q] = (long)nx.x == v0 + q ? o[q] - gs * __int_as_float(nx.y) : o[q];
        }
        ++c;
        nx = c < ce ? a.rd.pair[c] : make_int2(INT_MAX, 0);
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
  if (elem == 2 && a.d % kDmaKMult == 0 && a.V >= kBN && fits32(a.C * a.d * 2) && fits32(a.d * a.V * 2) &&
      fits32((a.T * a.K + 2) * 8))
    if (a.zout)
      hipLaunchKernelGGL((topk_fwd_t_kernel<kZ, true>), grid, block, 0, st, a);
    else
      hipLaunchKernelGGL((topk_fwd_t_kernel<kZ, false>), grid, block, 0, st, a);
  else if (elem == 2 && a.d % kDmaKMult == 0 && a.V >= kBN && fits32(a.C * a.d * 2) && fits32(a.d * a.V * 2))
    hipLaunchKernelGGL((topk_fwd_kernel<DmaNN<kBN>, Bf16, kZ>), grid, block, 0, st, a);
  else if (elem == 2)
    hipLaunchKernelGGL((topk_fwd_kernel<GenNN<Bf16, kBN>, Bf16, kZ>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((topk_fwd_kernel<GenNN<F32, kBN>, F32, kZ>), grid, block, 0, st, a);
}

hipError_t launch_topk_fwd(int elem, const TopkFwdArgs& a, hipStream_t st) {
  if (a.z_topk && !a.rd.zpair) return hipErrorInvalidValue;  // the gather writes the sorted entries' logits there
  if (a.z_topk)
    launch_topk_fwd_z<true>(elem, a, st);
  else
    launch_topk_fwd_z<false>(elem, a, st);
  return hipGetLastError();
}

hipError_t launch_topk_dz(int elem, const TopkDzArgs& a, hipStream_t st) {
  const dim3 grid(a.nrb * a.S), block(kThreads);
  if (elem == 2 && a.d % kDmaKMult == 0 && a.V >= kBN && fits32(a.C * a.d * 2) && fits32(a.d * a.V * 2))
    hipLaunchKernelGGL((fits32((a.T * a.K + 2) * 8) ? topk_dz_t_kernel : topk_dz_kernel<DmaNN<kBN>, Bf16>), grid,
                       block, 0, st, a);
  else if (elem == 2)
    hipLaunchKernelGGL((topk_dz_kernel<GenNN<Bf16, kBN>, Bf16>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((topk_dz_kernel<GenNN<F32, kBN>, F32>), grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace kd
