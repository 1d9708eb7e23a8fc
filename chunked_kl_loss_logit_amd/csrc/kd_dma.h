// bf16 contraction mainloop with direct global->LDS loads (gfx950).
//
// Operands go from HBM/L2 straight into a ring of four LDS slots
// (global_load_lds, 16 bytes per lane, no VGPR staging), three stages ahead of
// the stage the matrix cores are working on.  A stage holds 32 k of
//   A: 256 rows, k-contiguous                     [row][4 chunks of 16 B]
//   B: BN rows, k-contiguous (NT)                 [row][4 chunks]
//      or 32 k-rows of BN columns, n-contiguous   [k][BN/8 chunks]   (NN)
// NN fragments of B come out of LDS with the transposing read
// ds_read_b64_tr_b16: within each 16-lane group, lane j addresses 8 bytes at
// k-row k0 + j/4, columns c0 + 4 (j % 4), and lane i receives column c0 + i,
// rows k0..k0+3; a 32x32x16 B fragment takes two of them.
//
// Bank conflicts are avoided by XOR swizzles on 16-byte chunk positions:
//   k-contiguous rows:  chunk c of row m sits at c ^ ((m >> 2) & 3)
//   n-contiguous rows:  chunk c of k-row k sits at c ^ (4 (k & 3))
// A direct load writes its wave's 64 x 16 bytes contiguously in lane order,
// so each lane fetches the global chunk that belongs at its LDS position.
//
// The slots are separate __shared__ arrays addressed with compile-time slot
// numbers, so the compiler can tell a read of the current slot from direct
// loads still landing in the other three and does not wait for them; the ring
// waits on its own loads with explicit vmcnt counts.
//
// Operands come in two layouts.  Row-major: row r at r * ld bytes.  Panels
// (the library's own workspace buffers): a matrix of R rows is cut into
// 64-byte pieces along its rows, and piece p of row r sits at (p R + r) * 64,
// so the 64-byte pieces of one stage of consecutive rows are contiguous: a
// stage of a 256-row operand is one 16 KB run instead of 256 pieces of 64
// bytes in 256 cache lines, which halves the cache-line requests of its loads.
//
// Requirements (the launchers fall back to the general path otherwise): bf16
// and a contraction length that is a multiple of 128 (whole ring turns)
// whose data is readable (real data or zero padding).  Rows or columns outside the operand are
// loaded from a clamped valid address; they only feed accumulator rows or
// columns that the epilogues discard.
#pragma once

#include "kd_gemm.h"

namespace kd {

#define KD_LDS __attribute__((address_space(3)))

typedef short s16x4_t __attribute__((ext_vector_type(4)));

constexpr int kRing = 4;                   // slots
constexpr int kDmaKs = 32;                 // k per stage
constexpr int kDmaKMult = kRing * kDmaKs;  // the contraction length must be a multiple of this

// Direct loads are buffer loads: a resource descriptor (scalar registers) for
// the operand, a per-lane 32-bit offset that stays in the same register for
// the whole tile, and a scalar per-stage offset.  An instruction that reads
// its address from registers that are rewritten while it is in flight makes
// the compiler wait for every outstanding load first; loop-invariant offset
// registers avoid that.  Operands must therefore span less than 4 GiB.
// `base` must be the same in every lane.  It is read from the first active
// lane, so the compiler keeps the descriptor in scalar registers even where
// it cannot prove the pointer uniform; otherwise it wraps every load that
// uses the descriptor in a loop over the distinct values.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const char* base) {
  // the builtin takes and returns int: widen through uint32_t, or a low
  // half with bit 31 set would be sign-extended over the high half
  const uint64_t v = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  const uint64_t u = (uint64_t)lo | ((uint64_t)hi << 32);
  // raw buffer, no stride, full 32-bit range, gfx9 data format dword
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<char*>(u), (short)0, (int)0xffffffff, 0x00020000);
}

__device__ inline void dma16(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff, char* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (KD_LDS void*)(lds_wave_base), 16, (int)voff, (int)soff, 0, 0);
}

// 16 bytes of LDS at a byte offset from a slot array (one offset, so the
// compiler keeps the array's alias information)
__device__ inline u32x4_t ld_lds16(const char* slot, int off) {
  return *reinterpret_cast<const u32x4_t*>(slot + off);
}

// k-contiguous operand with NR rows: NR / 16 direct loads per stage, NR / 64
// per wave.  Lane L of load q covers row 16 q + L / 4 at chunk position L % 4.
// row_ptr gives the address of a row's first stage; stage s is s * sst bytes
// further (row-major: 64; panels of R rows: 64 R).
template <int NR>
struct DmaRows {
  static constexpr int kPer = NR / 64;
  static constexpr int kBytes = NR * kRowB;  // per stage
  __amdgpu_buffer_rsrc_t rs;
  uint32_t off[kPer];  // this lane's row offset from the operand base, plus its swizzled chunk
  uint32_t sst;        // bytes from one stage of a row to the next

  __device__ inline static int row_of(int i) {
    const int q = wave_id() * kPer + i;
    return 16 * q + ((threadIdx.x & 63) >> 2);
  }
  // row_ptr(i) for i < kPer: address of row row_of(i) (clamped to a valid row)
  template <class RowAddr>
  __device__ inline void init(const char* b, RowAddr&& row_ptr, uint32_t stage_stride = kRowB) {
    rs = make_rsrc(b);
    sst = stage_stride;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int m = row_of(i);
      off[i] = (uint32_t)(row_ptr(i) - b) + 16u * ((threadIdx.x & 3) ^ ((m >> 2) & 3));
    }
  }
  // stage s of the rows `extra` bytes further on (a uniform offset, such as
  // another row block of the same operand)
  __device__ inline void issue(long s, long extra, char* dst) const {
    const int w = wave_id();
    const uint32_t soff = (uint32_t)(s * sst + extra);
#pragma unroll
    for (int i = 0; i < kPer; ++i) dma16(rs, off[i], soff, dst + (w * kPer + i) * 1024);
  }
  __device__ inline void issue(long s, char* dst) const { issue(s, 0L, dst); }
};

// n-contiguous operand ([K][N]), BN columns per tile, row-major or in panels
// of K rows (each 64-byte piece of a k-row is one 16-byte-chunk group).
template <int BN>
struct DmaCols {
  static constexpr int kRowBytes = BN * 2;
  static constexpr int kChunks = BN / 8;                // 16-byte chunks per k-row
  static constexpr int kRowsPerLoad = 1024 / kRowBytes;  // 2 (BN 256) or 4 (BN 128)
  static constexpr int kLoads = kDmaKs / kRowsPerLoad;   // per stage
  static constexpr int kPer = kLoads / 4;                // per wave
  static constexpr int kBytes = kDmaKs * kRowBytes;      // per stage
  __amdgpu_buffer_rsrc_t rs;
  long ld;       // row-major: global row stride, bytes
  uint32_t sst;  // bytes from one stage to the next
  uint32_t off[kPer];

  // this lane's k-row and column of load i; columns at or past ncols are
  // clamped to the last whole chunk
  __device__ inline static void lane_pos(int i, long ncols, int& k, long& col) {
    const int w = wave_id(), L = threadIdx.x & 63;
    const int q = w * kPer + i;
    k = q * kRowsPerLoad + L / kChunks;
    col = 8L * ((L % kChunks) ^ (4 * (k & 3)));
    if (col + 8 > ncols) col = ncols - 8;
  }

  // row-major panel at b (element (0, n0)), ncols valid columns from it
  __device__ inline void init(const char* b, long ncols) {
    rs = make_rsrc(b);
    sst = (uint32_t)(kDmaKs * ld);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      int k;
      long col;
      lane_pos(i, ncols, k, col);
      off[i] = (uint32_t)(k * ld + col * 2);
    }
  }
  // columns [n0, n0 + BN) of a matrix at b stored in panels of prows rows,
  // ncols valid columns from n0
  __device__ inline void init_panels(const char* b, long n0, long ncols, long prows) {
    rs = make_rsrc(b);
    sst = (uint32_t)(kDmaKs * kRowB);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      int k;
      long col;
      lane_pos(i, ncols, k, col);
      off[i] = (uint32_t)panel_off(prows, k, (n0 + col) * 2);
    }
  }
  __device__ inline void issue(long s, char* dst) const {
    const int w = wave_id();
#pragma unroll
    for (int i = 0; i < kPer; ++i) dma16(rs, off[i], (uint32_t)(s * sst), dst + (w * kPer + i) * 1024);
  }
  // stage s of the panel that starts col0 columns after the one init() saw
  // (row-major only)
  __device__ inline void issue(long s, long col0, char* dst) const {
    const int w = wave_id();
    const uint32_t soff = (uint32_t)(s * kDmaKs * ld + col0 * 2);
#pragma unroll
    for (int i = 0; i < kPer; ++i) dma16(rs, off[i], soff, dst + (w * kPer + i) * 1024);
  }
};

// ------------------------------------------------------------------ register fragments
// One stage's operand fragments for one wave: for each of the two k-groups,
// 4 A fragments (rows wm*128 + 32 mb + lane % 32) and NB B fragments.
template <int NB, int NDS>
struct Frags {
  static constexpr int kMma = 2 * 4 * NB;  // matrix instructions per stage
  static constexpr int kDs = NDS;          // LDS read instructions per stage
  u32x4_t a[2][4];
  u32x4_t b[2][NB];
};

template <int NB, int NDS>
__device__ inline void mma_frags(const Frags<NB, NDS>& f, f32x16_t (&acc)[4][NB]) {
#pragma unroll
  for (int kg = 0; kg < 2; ++kg)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) Bf16::mma(acc[mb][nb], f.a[kg][mb], f.b[kg][nb]);
}

// The same products with the operands exchanged: block (mb, nb) then holds
// B's block nb times A's block mb transposed, so lane l owns A row
// 32 mb + l % 32 and, in register i, B column 32 nb + 8 (i / 4) + 4 (l / 32)
// + i % 4 (the A and B operand layouts of the matrix instruction are the
// same, so exchanging them transposes the product).  Epilogues that reduce
// along B's columns per A row then find 16 of a row's values in each lane.
template <int NB, int NDS>
__device__ inline void mma_frags_t(const Frags<NB, NDS>& f, f32x16_t (&acc)[4][NB]) {
#pragma unroll
  for (int kg = 0; kg < 2; ++kg)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) Bf16::mma(acc[mb][nb], f.b[kg][nb], f.a[kg][mb]);
}

// The first stage of a tile: k-group 0 starts every accumulator afresh.
template <bool kT, int NB, int NDS>
__device__ inline void mma_frags_first(const Frags<NB, NDS>& f, f32x16_t (&acc)[4][NB]) {
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      if constexpr (kT)
        Bf16::mma0(acc[mb][nb], f.b[0][nb], f.a[0][mb]);
      else
        Bf16::mma0(acc[mb][nb], f.a[0][mb], f.b[0][nb]);
    }
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      if constexpr (kT)
        Bf16::mma(acc[mb][nb], f.b[1][nb], f.a[1][mb]);
      else
        Bf16::mma(acc[mb][nb], f.a[1][mb], f.b[1][nb]);
    }
}

template <int BN>
using FragsNN = Frags<BN / 64, 2 * (4 + 2 * (BN / 64))>;  // b128 A reads, two transposing reads per B

template <int BN>
using FragsRows = Frags<BN / 64, 2 * (4 + BN / 64)>;

// Per-lane byte offsets of this wave's fragments inside a stage slot,
// computed once.  Every fragment read is then one of these registers plus an
// immediate, and the compiler keeps a handful of address registers instead of
// re-deriving the swizzled address of each read.
//   k-contiguous rows (A, and B of NT): row m = base + 32 mb + lane % 32 with
//     base a multiple of 128; chunk 2 kg + lane / 32 sits at position
//     c ^ ((m >> 2) & 3) = c ^ ((lane >> 2) & 3): offset a_off[kg] + 2048 mb.
//   n-contiguous B (NN): lane j of a 16-lane group reads k-row kl + 16 kg + 4 q
//     (kl = 8 (lane / 32) + j / 4) at column col0 + 16 ((lane >> 4) & 1) +
//     4 (j % 4); the swizzle key 4 (k & 3) only depends on kl, so the read is
//     b_off[nb] + (16 kg + 4 q) * row bytes.
template <int BN>
struct FragReader {
  static constexpr int NB = BN / 64;
  static constexpr int kRowBytes = BN * 2;  // one k-row of an n-contiguous B stage
  int a_off[2];
  int b_off[NB];  // NN: per column block; NT: entries 0 and 1 per k-group

  __device__ inline void init_nn() {
    const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int wm = w >> 1, wn = w & 1;
    const int h = l >> 5, x = (l >> 2) & 3;
#pragma unroll
    for (int kg = 0; kg < 2; ++kg) a_off[kg] = (wm * 128 + (l & 31)) * kRowB + 16 * ((2 * kg + h) ^ x);
    const int j = l & 15;
    const int kl = 8 * h + (j >> 2);
    const int cl = 2 * ((l >> 4) & 1) + ((j & 3) >> 1);
    const int hb = ((4 * (j & 3)) & 7) * 2;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int c = (wn * (BN / 2) + nb * 32) / 8 + cl;
      b_off[nb] = kHalfBytes + kl * kRowBytes + 16 * (c ^ (4 * (kl & 3))) + hb;
    }
  }

  __device__ inline void init_rows() {
    const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int wm = w >> 1, wn = w & 1;
    const int h = l >> 5, x = (l >> 2) & 3;
#pragma unroll
    for (int kg = 0; kg < 2; ++kg) {
      a_off[kg] = (wm * 128 + (l & 31)) * kRowB + 16 * ((2 * kg + h) ^ x);
      b_off[kg] = kHalfBytes + (wn * (BN / 2) + (l & 31)) * kRowB + 16 * ((2 * kg + h) ^ x);
    }
  }

  // A (256 rows, k-contiguous) and B (BN columns, n-contiguous) of the stage
  // in `slot` into this wave's fragments.
  __device__ inline void read_nn(const char* slot, FragsNN<BN>& f) const {
#pragma unroll
    for (int kg = 0; kg < 2; ++kg) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) f.a[kg][mb] = ld_lds16(slot, a_off[kg] + mb * 32 * kRowB);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        u32x4_t o;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int off = b_off[nb] + (16 * kg + 4 * q) * kRowBytes;
          const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((KD_LDS s16x4_t*)(const_cast<char*>(slot) + off));
          const uint2 u = __builtin_bit_cast(uint2, v);
          o[2 * q] = u.x;
          o[2 * q + 1] = u.y;
        }
        f.b[kg][nb] = o;
      }
    }
  }

  // A (256 rows) and B (BN rows), both k-contiguous.
  __device__ inline void read_rows(const char* slot, FragsRows<BN>& f) const {
#pragma unroll
    for (int kg = 0; kg < 2; ++kg) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) f.a[kg][mb] = ld_lds16(slot, a_off[kg] + mb * 32 * kRowB);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) f.b[kg][nb] = ld_lds16(slot, b_off[kg] + nb * 32 * kRowB);
    }
  }
};

// Instruction interleave of one ring step: each matrix instruction is
// followed by one LDS read (the next stage's fragments) while reads remain,
// then by one direct load.  Without it the scheduler issues each fragment
// read just before its first use, and the matrix pipe waits on LDS latency.
template <int NMMA, int NDS, int NVM>
__device__ inline void ring_sched() {
#pragma unroll
  for (int m = 0; m < NMMA; ++m) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    if (m < NDS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
    else if (m - NDS < NVM) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
  }
}

// ------------------------------------------------------------------ the ring
// Stages move HBM -> LDS slot (direct loads, issued kRing stages ahead of the
// matrix cores) -> registers (read one stage ahead) -> matrix cores.  Step i
// (stage i sits in slot J = i % 4 and already in registers `cur`):
//   wait until stage i + 1 has landed and every wave passed the barrier (so
//   every wave has also finished reading slot J into registers);
//   issue stage i + 4 into slot J (past the end: the last stage again, which
//   nobody reads, so every step issues the same number of loads and the
//   compiler's bookkeeping of in-flight loads stays exact);
//   read stage i + 1 from slot J + 1 into `nxt` while multiplying `cur`.
template <int J, int LPW, class Frag, class Issue, class Read, class Mma>
__device__ inline void ring_step(const Slots& sl, int i, int nst, Frag& cur, Frag& nxt, Issue& issue, Read& read,
                                 Mma& mma) {
  constexpr int JN = (J + 1) % kRing;
  wait_vm<(kRing - 2) * LPW>();
  ring_barrier();
  issue((long)min(i + kRing, nst - 1), sl.template A<J>(), sl.template B<J>());
  read(static_cast<const char*>(sl.template A<JN>()), nxt);
  mma(cur);
  ring_sched<Frag::kMma, Frag::kDs, LPW>();
}

// One tile's contraction over stages [0, nst), nst a multiple of 4 (the
// launchers choose this path only then).  `issue(s, A, B)` enqueues
// stage s into a slot's halves (LPW direct loads per wave), `read(slot, f)`
// loads one stage's fragments, `mma(f)` multiplies them.  Drains vector
// memory on entry (so the counts it waits on are its own) and on exit, then
// ends with a barrier, after which the caller may use the slots.
template <int LPW, class Frag, class Issue, class Read, class Mma>
__device__ inline void ring_contract(const Slots& sl, int nst, Issue&& issue, Read&& read, Mma&& mma) {
  static_assert(LPW * kRing < 64, "vmcnt range");
  wait_vm<0>();
  __syncthreads();
  if (nst > 0) {
    Frag f0, f1;
    issue(0L, sl.A<0>(), sl.B<0>());
    issue((long)min(1, nst - 1), sl.A<1>(), sl.B<1>());
    issue((long)min(2, nst - 1), sl.A<2>(), sl.B<2>());
    issue((long)min(3, nst - 1), sl.A<3>(), sl.B<3>());
    wait_vm<(kRing - 1) * LPW>();
    ring_barrier();
    read(static_cast<const char*>(sl.A<0>()), f0);
    for (int i = 0; i < nst; i += kRing) {
      ring_step<0, LPW>(sl, i, nst, f0, f1, issue, read, mma);
      ring_step<1, LPW>(sl, i + 1, nst, f1, f0, issue, read, mma);
      ring_step<2, LPW>(sl, i + 2, nst, f0, f1, issue, read, mma);
      ring_step<3, LPW>(sl, i + 3, nst, f1, f0, issue, read, mma);
    }
    wait_vm<0>();
  }
  __syncthreads();
}

// ------------------------------------------------------------------ the ring across tiles
// One step of ring_run: like ring_step, but the stage to issue is given as
// (tile, stage), and the read of the next stage can be left out (kRead).
template <int J, int LPW, bool kRead, class Frag, class Issue, class Read, class Mma>
__device__ inline void run_step(const Slots& sl, long it, int is, Frag& cur, Frag& nxt, Issue& issue, Read& read,
                                Mma& mma) {
  constexpr int JN = (J + 1) % kRing;
  wait_vm<(kRing - 2) * LPW>();
  ring_barrier();
  issue(it, is, sl.template A<J>(), sl.template B<J>());
  if constexpr (kRead) read(static_cast<const char*>(sl.template A<JN>()), nxt);
  mma(cur);
  ring_sched<Frag::kMma, kRead ? Frag::kDs : 0, LPW>();
}

// ntiles contractions of nst stages each (nst a multiple of 4, at least 4)
// through one ring that never drains between tiles: the last four steps of
// tile t issue the first four stages of tile t + 1, and while `done(t)`
// consumes the accumulators the loads keep landing.  `issue(t, s, A, B)`,
// `read` and `mma` are as in ring_contract; `mma0` multiplies a tile's first
// stage into fresh accumulators (so they need no clearing between tiles).
// done(t) runs after the last multiply of tile t, on every wave; it may use
// the epilogue array and ring_barrier(), but not the slots, and must not
// wait for vector memory (__syncthreads would).  Loads and stores it issues
// only make the next step's wait longer.
template <int LPW, class Frag, class Issue, class Read, class Mma, class Mma0, class Done>
__device__ inline void ring_run(const Slots& sl, int ntiles, int nst, Issue&& issue, Read&& read, Mma&& mma,
                                Mma0&& mma0, Done&& done) {
  static_assert(LPW * kRing < 64, "vmcnt range");
  wait_vm<0>();
  __syncthreads();
  if (ntiles > 0) {
    Frag f0, f1;
    issue(0L, 0, sl.A<0>(), sl.B<0>());
    issue(0L, 1, sl.A<1>(), sl.B<1>());
    issue(0L, 2, sl.A<2>(), sl.B<2>());
    issue(0L, 3, sl.A<3>(), sl.B<3>());
    wait_vm<(kRing - 1) * LPW>();
    ring_barrier();
    read(static_cast<const char*>(sl.A<0>()), f0);
    for (int t = 0; t < ntiles; ++t) {
      const bool more = t + 1 < ntiles;
      const long tn = more ? t + 1 : t;
      if (nst > kRing) {
        run_step<0, LPW, true>(sl, t, 4, f0, f1, issue, read, mma0);
        run_step<1, LPW, true>(sl, t, 5, f1, f0, issue, read, mma);
        run_step<2, LPW, true>(sl, t, 6, f0, f1, issue, read, mma);
        run_step<3, LPW, true>(sl, t, 7, f1, f0, issue, read, mma);
        for (int s = kRing; s + kRing < nst; s += kRing) {
          run_step<0, LPW, true>(sl, t, s + 4, f0, f1, issue, read, mma);
          run_step<1, LPW, true>(sl, t, s + 5, f1, f0, issue, read, mma);
          run_step<2, LPW, true>(sl, t, s + 6, f0, f1, issue, read, mma);
          run_step<3, LPW, true>(sl, t, s + 7, f1, f0, issue, read, mma);
        }
        // last four stages: issue the next tile's first four (after the last
        // tile, this tile's last stage again, into slots nobody reads)
        run_step<0, LPW, true>(sl, tn, more ? 0 : nst - 1, f0, f1, issue, read, mma);
      } else {
        run_step<0, LPW, true>(sl, tn, more ? 0 : nst - 1, f0, f1, issue, read, mma0);
      }
      run_step<1, LPW, true>(sl, tn, more ? 1 : nst - 1, f1, f0, issue, read, mma);
      run_step<2, LPW, true>(sl, tn, more ? 2 : nst - 1, f0, f1, issue, read, mma);
      run_step<3, LPW, false>(sl, tn, more ? 3 : nst - 1, f1, f0, issue, read, mma);
      done(t);
      // stage 0 of the next tile landed before the last step's barrier
      read(static_cast<const char*>(sl.A<0>()), f0);
    }
    wait_vm<0>();
  }
  __syncthreads();
}

}  // namespace kd
