// Mainloop policies: a 256-row tile A times a BN-column panel of B, into
// f32x16_t acc[4][BN / 64] per wave.  All of them stage operands in the LDS
// slot layout of kd_gemm.h and leave the slots free when tile() returns.
//
//   NN (B is n-contiguous: W as [d][V], or the dZ chunk in panels)
//     DmaNN<BN>      bf16, contraction a multiple of 128: direct-load ring,
//                    transposing LDS reads for B
//     GenNN<E, BN>   any shape or dtype: register-staged loads, B transposed
//                    in registers, double buffer in slots 0 and 1
//   NT (B is k-contiguous: W as [d][V] when V is the contraction)
//     DmaNT<BN>      bf16, contraction K a multiple of 32, run over K rounded
//                    up to 128 (whole ring turns): A must hold readable zeros
//                    in the rounding, and B's stages past K re-read its last
//                    one (finite data times those zeros adds nothing)
//     GenNT<E, BN>   any shape or dtype
//
// init(row_ptr, ...) takes row_ptr(r) -> address of the first stage of A row
// r of the tile (row-major: the row itself; panels: the row's first 64-byte
// piece), or nullptr outside the operand, and the stage stride that leads to
// the row's next stage; NT policies take the same for B rows.
#pragma once

#include <climits>

#include "kd_dma.h"
#include "kd_gemm.h"

namespace kd {

// One output tile of a persistent run: A is the operand's rows `a_off` bytes
// after the rows init() saw, B is the panel at column n0.
struct TileAt {
  long a_off;
  long n0;
};

// ------------------------------------------------------------------ shared stage product
// Both operands k-contiguous rows.
template <class E, int BN>
__device__ inline void mma_stage_rows(const char* As, const char* Bs, f32x16_t (&acc)[4][BN / 64]) {
  constexpr int NB = BN / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
#pragma unroll
  for (int kg = 0; kg < 2; ++kg) {
    const int c = 2 * kg + (lane >> 5);
    u32x4_t a[4], b[NB];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) a[mb] = row_frag(As, wm * 128 + mb * 32 + (lane & 31), c);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) b[nb] = row_frag(Bs, wn * (BN / 2) + nb * 32 + (lane & 31), c);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) E::mma(acc[mb][nb], a[mb], b[nb]);
  }
}

// ------------------------------------------------------------------ register-staged loaders
// k-contiguous operand with NR rows; thread t loads chunk t % 4 of rows
// t / 4 + 64 j.  Rows without a pointer and bytes past kbytes read as zero.
// rp[j] is the address of a row's first stage; stage s is s * sst bytes
// further (row-major: 64; panels of R rows: 64 R).
template <int NR>
struct GRows {
  static constexpr int kPer = NR / 64;
  const char* rp[kPer];
  u32x4_t r[kPer];
  long sst;
  __device__ inline static int row_of(int j) { return (threadIdx.x >> 2) + 64 * j; }
  // kbyte0: the stage's first byte along the rows, a multiple of 64
  __device__ inline void load(long kbyte0, long kbytes, long extra = 0) {
    const long off = kbyte0 + 16 * (threadIdx.x & 3);
    const long pos = kbyte0 / kRowB * sst + 16 * (threadIdx.x & 3);
    const bool kv = off < kbytes;
#pragma unroll
    for (int j = 0; j < kPer; ++j) r[j] = (kv && rp[j]) ? ld16(rp[j] + extra + pos) : zero4();
  }
  __device__ inline void store(char* dst) const {
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      *reinterpret_cast<u32x4_t*>(dst + row_pos(row_of(j), threadIdx.x & 3)) = r[j];
  }
};

// n-contiguous operand ([K][N], row-major or in panels of prows rows) stored
// as BN k-contiguous rows: each thread loads an EPC x EPC block (EPC k-rows of
// one 16-byte column chunk), transposes it in registers and writes EPC
// 16-byte row chunks.
template <class E, int BN>
struct GCols {
  static constexpr int kKs = kRowB / E::kElem;  // k-rows per stage
  static constexpr int kNkb = kKs / E::kEpc;    // 4
  static constexpr int kNnc = BN / E::kEpc;
  static constexpr int kNblk = kNkb * kNnc;
  static constexpr int kPer = (kNblk + kThreads - 1) / kThreads;
  u32x4_t r[kPer][E::kEpc];
  const char* mat;   // element (0, 0)
  const char* base;  // element (0, n0)
  long ld;           // row-major: row stride, bytes
  long prows;        // panels: rows per panel (0: row-major)
  long N, n0, K;

  __device__ inline void load(long k0) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int b = threadIdx.x + kThreads * i;
      const int kb = b % kNkb, nc = b / kNkb;
      const bool nv = (b < kNblk) && (n0 + nc * E::kEpc < N);
#pragma unroll
      for (int e = 0; e < E::kEpc; ++e) {
        const long k = k0 + kb * E::kEpc + e;
        const long byte = (n0 + (long)nc * E::kEpc) * E::kElem;
        const char* p = prows ? mat + panel_off(prows, k, byte) : base + k * ld + (long)nc * 16;
        r[i][e] = (nv && k < K) ? ld16(p) : zero4();
      }
    }
  }
  __device__ inline void store(char* dst) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int b = threadIdx.x + kThreads * i;
      if (b >= kNblk) continue;
      const int kb = b % kNkb, nc = b / kNkb;
      if constexpr (E::kEpc == 8) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
          u32x4_t o;
#pragma unroll
          for (int w = 0; w < 4; ++w) o[w] = __builtin_amdgcn_perm(r[i][2 * w + 1][j >> 1], r[i][2 * w][j >> 1], sel);
          *reinterpret_cast<u32x4_t*>(dst + row_pos(nc * 8 + j, kb)) = o;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32x4_t o{r[i][0][j], r[i][1][j], r[i][2][j], r[i][3][j]};
          *reinterpret_cast<u32x4_t*>(dst + row_pos(nc * 4 + j, kb)) = o;
        }
      }
    }
  }
};

// Double-buffered contraction over slots 0 and 1 for the general policies.
template <class Load, class Store, class Mma>
__device__ inline void gen_contract(const Slots& sl, long nst, Load&& load, Store&& store, Mma&& mma) {
  __syncthreads();
  if (nst <= 0) return;
  char* bufa[2] = {sl.A<0>(), sl.A<1>()};
  char* bufb[2] = {sl.B<0>(), sl.B<1>()};
  load(0);
  store(bufa[0], bufb[0]);
  __syncthreads();
  for (long s = 0; s < nst; ++s) {
    const int cur = (int)(s & 1);
    if (s + 1 < nst) load(s + 1);
    mma(static_cast<const char*>(bufa[cur]), static_cast<const char*>(bufb[cur]));
    if (s + 1 < nst) store(bufa[cur ^ 1], bufb[cur ^ 1]);
    __syncthreads();
  }
}

// ------------------------------------------------------------------ NN policies
template <class E, int BN>
struct GenNN {
  static constexpr int kKMult = 1;
  GRows<kBM> al;
  GCols<E, BN> bl;
  const char* B;
  long kbytes, nst;

  // a_sst: stage stride of A (see GRows); b_prows: B in panels of that many
  // rows (0: row-major with stride ldb)
  template <class RowPtr>
  __device__ inline void init(const char*, RowPtr&& row_ptr, const char* Bm, long ldb, long N, long K,
                              long a_sst = kRowB, long b_prows = 0) {
#pragma unroll
    for (int j = 0; j < GRows<kBM>::kPer; ++j) al.rp[j] = row_ptr(GRows<kBM>::row_of(j));
    al.sst = a_sst;
    B = Bm;
    bl.mat = Bm;
    bl.prows = b_prows;
    bl.ld = ldb;
    bl.N = N;
    bl.K = K;
    kbytes = K * E::kElem;
    nst = (kbytes + kRowB - 1) / kRowB;
  }

  // tiles t = 0 .. ntiles-1 described by at(t); done(t, acc) after each
  template <class At, class Done>
  __device__ inline void run(const Slots& sl, int ntiles, At&& at, Done&& done) {
    f32x16_t acc[4][BN / 64];
    for (int t = 0; t < ntiles; ++t) {
      const TileAt ta = at(t);
      tile(sl, ta.n0, acc, ta.a_off);
      done(t, acc);
    }
  }

  __device__ inline void tile(const Slots& sl, long n0, f32x16_t (&acc)[4][BN / 64], long a_off = 0) {
    constexpr int KS = kRowB / E::kElem;
    bl.base = B + n0 * E::kElem;
    bl.n0 = n0;
    zero_acc<BN / 64>(acc);
    gen_contract(
        sl, nst,
        [&](long s) {
          al.load(s * kRowB, kbytes, a_off);
          bl.load(s * KS);
        },
        [&](char* da, char* db) {
          al.store(da);
          bl.store(db);
        },
        [&](const char* as, const char* bs) { mma_stage_rows<E, BN>(as, bs, acc); });
  }
};

// A rows are addressed relative to `abase` (the start of the A operand) and
// must lie within 4 GiB of it; so must the B panel's rows.
template <int BN>
struct DmaNN {
  static constexpr int kKMult = kDmaKMult;
  static constexpr int kLpw = DmaRows<kBM>::kPer + DmaCols<BN>::kPer;
  static_assert(DmaRows<kBM>::kBytes <= kHalfBytes && DmaCols<BN>::kBytes <= kHalfBytes, "stage must fit a slot");
  DmaRows<kBM> a;
  DmaCols<BN> b;
  FragReader<BN> rd;
  const char* B;
  long N;
  long b_prows;
  int nst;

  // a_sst: stage stride of A (see DmaRows); b_prows: B in panels of that many
  // rows (0: row-major with stride ldb; run() takes row-major B only)
  template <class RowPtr>
  __device__ inline void init(const char* abase, RowPtr&& row_ptr, const char* Bm, long ldb, long Nn, long K,
                              uint32_t a_sst = kRowB, long bp = 0) {
    const char* safe = row_ptr(0);  // row 0 of a launched tile is always inside the operand
    a.init(
        abase,
        [&](int i) {
          const char* p = row_ptr(DmaRows<kBM>::row_of(i));
          return p ? p : safe;
        },
        a_sst);
    B = Bm;
    b_prows = bp;
    b.ld = ldb;
    N = Nn;
    nst = (int)(K / kDmaKs);
    rd.init_nn();
  }

  // Tiles t = 0 .. ntiles-1 described by at(t), through one ring; done(t,
  // acc) after each (see ring_run for what it may do).  Every tile must lie
  // inside both operands: no row or column is clamped.  kT: the
  // accumulators hold the transposed tile (mma_frags_t).
  template <bool kT = false, class At, class Done>
  __device__ inline void run(const Slots& sl, int ntiles, At&& at, Done&& done) {
    b.init(B, LONG_MAX);
    f32x16_t acc[4][BN / 64];
    ring_run<kLpw, FragsNN<BN>>(
        sl, ntiles, nst,
        [&](long t, int s, char* da, char* db) {
          const TileAt ta = at((int)t);
          a.issue(s, ta.a_off, da);
          b.issue(s, ta.n0, db);
        },
        [&](const char* slot, FragsNN<BN>& f) { rd.read_nn(slot, f); },
        [&](const FragsNN<BN>& f) {
          if constexpr (kT)
            mma_frags_t(f, acc);
          else
            mma_frags(f, acc);
        },
        [&](const FragsNN<BN>& f) { mma_frags_first<kT>(f, acc); }, [&](int t) { done(t, acc); });
  }

  // kT: the accumulators hold the transposed tile (mma_frags_t)
  template <bool kT = false>
  __device__ inline void tile(const Slots& sl, long n0, f32x16_t (&acc)[4][BN / 64]) {
    if (b_prows)
      b.init_panels(B, n0, N - n0, b_prows);
    else
      b.init(B + n0 * 2, N - n0);
    zero_acc<BN / 64>(acc);
    ring_contract<kLpw, FragsNN<BN>>(
        sl, nst,
        [&](long s, char* da, char* db) {
          a.issue(s, da);
          b.issue(s, db);
        },
        [&](const char* slot, FragsNN<BN>& f) { rd.read_nn(slot, f); },
        [&](const FragsNN<BN>& f) {
          if constexpr (kT)
            mma_frags_t(f, acc);
          else
            mma_frags(f, acc);
        });
  }
};

// ------------------------------------------------------------------ NT policies
template <class E, int BN>
struct GenNT {
  static constexpr int kStageGroup = 1;
  GRows<kBM> al;
  GRows<BN> bl;
  long kbytes, nst;

  // a_sst, b_sst: stage strides of the operands (see GRows)
  template <class RowPtrA, class RowPtrB>
  __device__ inline void init(const char*, RowPtrA&& row_a, const char*, RowPtrB&& row_b, long K, long a_sst = kRowB,
                              long b_sst = kRowB) {
#pragma unroll
    for (int j = 0; j < GRows<kBM>::kPer; ++j) al.rp[j] = row_a(GRows<kBM>::row_of(j));
#pragma unroll
    for (int j = 0; j < GRows<BN>::kPer; ++j) bl.rp[j] = row_b(GRows<BN>::row_of(j));
    al.sst = a_sst;
    bl.sst = b_sst;
    kbytes = K * E::kElem;
    nst = (kbytes + kRowB - 1) / kRowB;
  }

  // contraction stages [s0, s1)
  __device__ inline void tile(const Slots& sl, long s0, long s1, f32x16_t (&acc)[4][BN / 64]) {
    zero_acc<BN / 64>(acc);
    gen_contract(
        sl, s1 - s0,
        [&](long s) {
          al.load((s0 + s) * kRowB, kbytes);
          bl.load((s0 + s) * kRowB, kbytes);
        },
        [&](char* da, char* db) {
          al.store(da);
          bl.store(db);
        },
        [&](const char* as, const char* bs) { mma_stage_rows<E, BN>(as, bs, acc); });
  }
};

template <int BN>
struct DmaNT {
  static constexpr int kStageGroup = kRing;
  static constexpr int kLpw = DmaRows<kBM>::kPer + DmaRows<BN>::kPer;
  static_assert(DmaRows<kBM>::kBytes <= kHalfBytes && DmaRows<BN>::kBytes <= kHalfBytes, "stage must fit a slot");
  DmaRows<kBM> a;
  DmaRows<BN> b;
  FragReader<BN> rd;
  long nst, b_last;  // stages contracted; B's last stage

  // a_sst, b_sst: stage strides of the operands (see DmaRows)
  template <class RowPtrA, class RowPtrB>
  __device__ inline void init(const char* abase, RowPtrA&& row_a, const char* bbase, RowPtrB&& row_b, long K,
                              uint32_t a_sst = kRowB, uint32_t b_sst = kRowB) {
    const char* sa = row_a(0);
    const char* sb = row_b(0);
    a.init(
        abase,
        [&](int i) {
          const char* p = row_a(DmaRows<kBM>::row_of(i));
          return p ? p : sa;
        },
        a_sst);
    b.init(
        bbase,
        [&](int i) {
          const char* p = row_b(DmaRows<BN>::row_of(i));
          return p ? p : sb;
        },
        b_sst);
    nst = (K + kDmaKMult - 1) / kDmaKMult * kRing;
    b_last = K / kDmaKs - 1;
    rd.init_rows();
  }

  __device__ inline void tile(const Slots& sl, long s0, long s1, f32x16_t (&acc)[4][BN / 64]) {
    zero_acc<BN / 64>(acc);
    ring_contract<kLpw, FragsRows<BN>>(
        sl, (int)(s1 - s0),
        [&](long s, char* da, char* db) {
          a.issue(s0 + s, da);
          b.issue(min(s0 + s, b_last), db);
        },
        [&](const char* slot, FragsRows<BN>& f) { rd.read_rows(slot, f); },
        [&](const FragsRows<BN>& f) { mma_frags(f, acc); });
  }
};

}  // namespace kd
