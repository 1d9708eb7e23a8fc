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
// Requirements (the launchers fall back to the general path otherwise): bf16
// and a contraction length that is a multiple of 32 whose data is readable
// (real data or zero padding).  Rows or columns outside the operand are
// loaded from a clamped valid address; they only feed accumulator rows or
// columns that the epilogues discard.
#pragma once

#include "kd_gemm.h"

namespace kd {

#define KD_LDS __attribute__((address_space(3)))

typedef short s16x4_t __attribute__((ext_vector_type(4)));

constexpr int kRing = 4;    // slots
constexpr int kDmaKs = 32;  // k per stage

// Direct loads are buffer loads: a resource descriptor (scalar registers) for
// the operand, a per-lane 32-bit offset that stays in the same register for
// the whole tile, and a scalar per-stage offset.  An instruction that reads
// its address from registers that are rewritten while it is in flight makes
// the compiler wait for every outstanding load first; loop-invariant offset
// registers avoid that.  Operands must therefore span less than 4 GiB.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const char* base) {
  // raw buffer, no stride, full 32-bit range, gfx9 data format dword
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, (int)0xffffffff, 0x00020000);
}

__device__ inline void dma16(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff, char* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (KD_LDS void*)(lds_wave_base), 16, (int)voff, (int)soff, 0, 0);
}

// k-contiguous operand with NR rows: NR / 16 direct loads per stage, NR / 64
// per wave.  Lane L of load q covers row 16 q + L / 4 at chunk position L % 4.
template <int NR>
struct DmaRows {
  static constexpr int kPer = NR / 64;
  static constexpr int kBytes = NR * kRowB;  // per stage
  __amdgpu_buffer_rsrc_t rs;
  uint32_t off[kPer];  // this lane's row offset from the operand base, plus its swizzled chunk

  __device__ inline static int row_of(int i) {
    const int q = wave_id() * kPer + i;
    return 16 * q + ((threadIdx.x & 63) >> 2);
  }
  // row_ptr(i) for i < kPer: address of row row_of(i) (clamped to a valid row)
  template <class RowAddr>
  __device__ inline void init(const char* b, RowAddr&& row_ptr) {
    rs = make_rsrc(b);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int m = row_of(i);
      off[i] = (uint32_t)(row_ptr(i) - b) + 16u * ((threadIdx.x & 3) ^ ((m >> 2) & 3));
    }
  }
  __device__ inline void issue(long s, char* dst) const {
    const int w = wave_id();
#pragma unroll
    for (int i = 0; i < kPer; ++i) dma16(rs, off[i], (uint32_t)(s * kRowB), dst + (w * kPer + i) * 1024);
  }
};

// n-contiguous operand ([K][N] row-major), BN columns per tile.
template <int BN>
struct DmaCols {
  static constexpr int kRowBytes = BN * 2;
  static constexpr int kChunks = BN / 8;                // 16-byte chunks per k-row
  static constexpr int kRowsPerLoad = 1024 / kRowBytes;  // 2 (BN 256) or 4 (BN 128)
  static constexpr int kLoads = kDmaKs / kRowsPerLoad;   // per stage
  static constexpr int kPer = kLoads / 4;                // per wave
  static constexpr int kBytes = kDmaKs * kRowBytes;      // per stage
  __amdgpu_buffer_rsrc_t rs;
  long ld;  // global row stride, bytes
  uint32_t off[kPer];

  // panel at b (element (0, n0)), ncols valid columns from it (clamped beyond)
  __device__ inline void init(const char* b, long ncols) {
    rs = make_rsrc(b);
    const int w = wave_id(), L = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int q = w * kPer + i;
      const int k = q * kRowsPerLoad + L / kChunks;
      const int c = (L % kChunks) ^ (4 * (k & 3));
      long col = 8L * c;
      if (col + 8 > ncols) col = ncols - 8;
      off[i] = (uint32_t)(k * ld + col * 2);
    }
  }
  __device__ inline void issue(long s, char* dst) const {
    const int w = wave_id();
#pragma unroll
    for (int i = 0; i < kPer; ++i) dma16(rs, off[i], (uint32_t)(s * kDmaKs * ld), dst + (w * kPer + i) * 1024);
  }
  // B fragment of a 32x32x16 MFMA out of the slot starting at `slot` (B half
  // at boff): columns col0 .. col0 + 31 (col0 % 32 == 0), k = 16 kg +
  // 8 (lane / 32) + 0..7 of the stage.  Each address is one integer offset
  // from the slot array: a deeper chain of pointer arithmetic loses the
  // alias information that keeps the compiler from waiting on in-flight
  // direct loads.
  __device__ inline static u32x4_t frag(const char* slot, int boff, int col0, int kg) {
    const int l = threadIdx.x & 63;
    const int j = l & 15;
    const int col = col0 + 16 * ((l >> 4) & 1) + 4 * (j & 3);
    const int c = col >> 3;
    const int hb = (col & 7) * 2;
    u32x4_t out;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int k = 16 * kg + 8 * (l >> 5) + 4 * q + (j >> 2);
      const int off = boff + k * kRowBytes + 16 * (c ^ (4 * (k & 3))) + hb;
      const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((KD_LDS s16x4_t*)(const_cast<char*>(slot) + off));
      const uint2 u = __builtin_bit_cast(uint2, v);
      out[2 * q] = u.x;
      out[2 * q + 1] = u.y;
    }
    return out;
  }
};

// One step of the ring: stage i sits in slot J.  The step always issues a
// stage into slot (J + 3) % 4 (which every wave finished reading before this
// step's barrier): stage i + 3, or past the end a repeat of the last stage,
// which lands in a slot nobody reads.  Steps past the last stage still wait,
// meet at the barrier and issue; they only skip the multiply.  Keeping every
// direct load unconditional keeps the compiler's bookkeeping of in-flight
// loads identical on all paths; with a conditional one it makes every LDS
// read wait for all outstanding loads.
template <int J, int LPW, class Issue, class Mma>
__device__ inline void ring_step(const Slots& sl, int i, int nst, Issue& issue, Mma& mma) {
  constexpr int JN = (J + kRing - 1) % kRing;
  wait_vm<(kRing - 2) * LPW>();  // this wave's loads of stage i have landed
  ring_barrier();                // ... and every other wave's; slot JN is free
  issue((long)min(i + kRing - 1, nst - 1), sl.template A<JN>(), sl.template B<JN>());
  if (i < nst) mma(static_cast<const char*>(sl.template A<J>()), static_cast<const char*>(sl.template B<J>()));
}

// One tile's contraction over stages [0, nst): kRing - 1 stages are issued
// ahead.  `issue(s, A, B)` enqueues stage s into a slot's halves, `mma(A, B)`
// multiplies one stage out of LDS.  Each wave issues LPW direct loads per
// stage.  Drains vector memory on entry (so the counts it waits on are its
// own) and on exit, then ends with a barrier, after which the caller may use
// the slots.
template <int LPW, class Issue, class Mma>
__device__ inline void ring_contract(const Slots& sl, int nst, Issue&& issue, Mma&& mma) {
  static_assert(LPW * (kRing - 2) < 64, "vmcnt range");
  wait_vm<0>();
  __syncthreads();
  if (nst > 0) {
    issue(0L, sl.A<0>(), sl.B<0>());
    issue((long)min(1, nst - 1), sl.A<1>(), sl.B<1>());
    issue((long)min(2, nst - 1), sl.A<2>(), sl.B<2>());
    for (int i = 0; i < nst; i += kRing) {
      ring_step<0, LPW>(sl, i, nst, issue, mma);
      ring_step<1, LPW>(sl, i + 1, nst, issue, mma);
      ring_step<2, LPW>(sl, i + 2, nst, issue, mma);
      ring_step<3, LPW>(sl, i + 3, nst, issue, mma);
    }
    wait_vm<0>();
  }
  __syncthreads();
}

// A (256 rows, k-contiguous) x B (n-contiguous) stage product into a
// 128 x (BN/2) wave tile.
template <int BN>
__device__ inline void mma_stage_nn(const char* As, const char* /*Bs = As + kHalfBytes*/, f32x16_t (&acc)[4][BN / 64]) {
  constexpr int NB = BN / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
#pragma unroll
  for (int kg = 0; kg < 2; ++kg) {
    u32x4_t a[4], b[NB];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) a[mb] = row_frag(As, wm * 128 + mb * 32 + (lane & 31), 2 * kg + (lane >> 5));
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) b[nb] = DmaCols<BN>::frag(As, kHalfBytes, wn * (BN / 2) + nb * 32, kg);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) Bf16::mma(acc[mb][nb], a[mb], b[nb]);
  }
}

}  // namespace kd
