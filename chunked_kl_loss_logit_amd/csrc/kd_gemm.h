// Device building blocks shared by every contraction of the loss.
//
// Geometry: a workgroup of 4 waves (2 x 2) computes a 256-row x BN-column tile
// (BN = 256, or 128 where two accumulator sets live side by side) on gfx950
// matrix cores; each wave owns 128 rows x BN/2 columns = 4 x (BN/64) blocks of
// 32 x 32 (bf16: v_mfma_f32_32x32x16_bf16; fp32: v_mfma_f32_32x32x2_f32).
//
// LDS is four stage "slots" of 32 KB, separate __shared__ arrays (see
// kd_dma.h for why).  During a contraction they hold operand stages;
// afterwards the epilogues use them to stage accumulator columns.
//
// Slot layout of a k-contiguous operand stage: 64 bytes of the contraction
// per row (32 bf16 or 16 fp32), 16-byte chunk c of row m stored at chunk
// position c ^ ((m >> 2) & 3), so the 16-byte fragment reads of 16
// consecutive rows hit 64 distinct banks.
//
// A "k-group" is 32 bytes of contraction of one row: 16 bf16 (one MFMA) or 8
// fp32 (four MFMAs).  Lane half h = lane / 32 takes chunk 2 kg + h of every
// row of both operands, so the two operands always pair the same k.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kd {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kBM = 256;             // rows per workgroup tile
constexpr int kRowB = 64;            // contraction bytes per row and stage
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ------------------------------------------------------------------ element types
struct Bf16 {
  static constexpr int kElem = 2;  // bytes per element
  static constexpr int kEpc = 8;   // elements per 16-byte chunk
  __device__ static inline void mma(f32x16_t& acc, u32x4_t a, u32x4_t b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
  }
  // the same product into a fresh accumulator (the instruction's C operand
  // is the constant 0, so nothing has to clear the accumulator first)
  __device__ static inline void mma0(f32x16_t& acc, u32x4_t a, u32x4_t b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), f32x16_t{}, 0, 0, 0);
  }
  // float -> bf16 bits, round to nearest even (NaN stays NaN)
  __device__ static inline uint32_t pack2(float lo, float hi) { return cvt(lo) | (cvt(hi) << 16); }
  __device__ static inline uint32_t cvt(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  }
};

struct F32 {
  static constexpr int kElem = 4;
  static constexpr int kEpc = 4;
  __device__ static inline void mma(f32x16_t& acc, u32x4_t a, u32x4_t b) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[s]), __uint_as_float(b[s]), acc, 0, 0, 0);
  }
};

__device__ inline u32x4_t zero4() { return u32x4_t{0u, 0u, 0u, 0u}; }
__device__ inline u32x4_t ld16(const char* p) { return *reinterpret_cast<const u32x4_t*>(p); }

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// wave index within the workgroup, known to the compiler to be wave-uniform
__device__ inline int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// A copy of x the compiler cannot see through: values derived from it are
// recomputed after each call instead of being hoisted out of enclosing loops
// (where they would hold registers across the matrix-core loop).
__device__ inline int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}
// the same for a uniform pointer (kept in scalar registers)
template <class T>
__device__ inline T* opaque_ptr(T* p) {
  asm volatile("" : "+s"(p));
  return p;
}

// ------------------------------------------------------------------ synchronisation
// s_waitcnt vmcnt(n) leaving the other counters alone (gfx9 encoding)
template <int N>
__device__ inline void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier that orders this wave's LDS accesses but, unlike
// __syncthreads(), does not wait for outstanding vector memory operations.
__device__ inline void ring_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ------------------------------------------------------------------ LDS slots
// Four stage slots of 32 KB, separate __shared__ arrays: the A half of a
// stage at offset 0, the B half at offset 16 KB.  Addressing every slot by a
// compile-time slot number lets the compiler tell the slots apart (kd_dma.h).
// A fifth 32 KB array stages epilogue blocks while the slots keep receiving
// the next tile's operands: 160 KB, the whole LDS of a CU.
constexpr int kHalfBytes = 16384;
constexpr int kSlotBytes = 2 * kHalfBytes;
constexpr int kEpBytes = 32768;

struct Slots {
  char* s0;
  char* s1;
  char* s2;
  char* s3;
  float* ep;  // epilogue staging, [256][32] floats
  template <int J>
  __device__ inline char* at() const {
    static_assert(J >= 0 && J < 4, "slot");
    if constexpr (J == 0) return s0;
    if constexpr (J == 1) return s1;
    if constexpr (J == 2) return s2;
    return s3;
  }
  template <int J>
  __device__ inline char* A() const { return at<J>(); }
  template <int J>
  __device__ inline char* B() const { return at<J>() + kHalfBytes; }
};

#define KD_DECLARE_SLOTS(name)                                       \
  __shared__ __attribute__((aligned(16))) char name##_0[kSlotBytes]; \
  __shared__ __attribute__((aligned(16))) char name##_1[kSlotBytes]; \
  __shared__ __attribute__((aligned(16))) char name##_2[kSlotBytes]; \
  __shared__ __attribute__((aligned(16))) char name##_3[kSlotBytes]; \
  __shared__ __attribute__((aligned(16))) float name##_e[kEpBytes / 4]; \
  const Slots name{name##_0, name##_1, name##_2, name##_3, name##_e}

// 16-byte fragment of a k-contiguous stage: row m, logical chunk c (0..3)
__device__ inline u32x4_t row_frag(const char* st, int m, int c) {
  return *reinterpret_cast<const u32x4_t*>(st + m * kRowB + 16 * (c ^ ((m >> 2) & 3)));
}
__device__ inline int row_pos(int m, int c) { return m * kRowB + 16 * (c ^ ((m >> 2) & 3)); }

// ------------------------------------------------------------------ workgroup placement
// Workgroups are handed to the 8 XCDs round-robin by id.  Renumber them so that
// consecutive logical ids share an XCD (and its L2): XCD x runs one contiguous
// range of logical ids, of n/8 (rounded up for the first n%8 XCDs) ids.
__device__ inline int xcd_remap(int id, int n) {
  const int q = n >> 3, r = n & 7, x = id & 7, j = id >> 3;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + j;
}

// Grouped raster over an nrb x ncb grid: G row-blocks form a group; inside a
// group the row-block moves fastest, so a run of consecutive logical ids
// covers a compact G x k block of tiles (shared operand slabs stay in L2).
__device__ inline void grouped_coords(int logical, int nrb, int ncb, int G, int& rb, int& cb) {
  const int per_group = G * ncb;
  const int grp = logical / per_group;
  const int first = grp * G;
  const int gsz = min(G, nrb - first);
  const int rem = logical - grp * per_group;
  rb = first + rem % gsz;
  cb = rem / gsz;
}

template <int NB>
__device__ inline void zero_acc(f32x16_t (&acc)[4][NB]) {
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.f;
}

// ------------------------------------------------------------------ epilogue staging
// A round stages one 32-column block of every wave's accumulators as [256
// rows][32 floats] into one slot.  Float4 chunk c of row r sits at chunk
// c ^ ((r >> 1) & 7), so 16 consecutive rows read at the same column hit 64
// distinct banks.
//
// Accumulator layout of the 32 x 32 MFMA output: lane l holds column l % 32
// and, in register i, row 8 (i / 4) + 4 (l / 32) + i % 4 of its block.
typedef float* StPair;  // one slot viewed as [256][32] floats

template <int J>
__device__ inline StPair st_pair(const Slots& sl) {
  return reinterpret_cast<float*>(sl.template at<J>());
}

__device__ inline int st_pos(int r, int col) { return ((((col >> 2) ^ ((r >> 1) & 7))) << 2) + (col & 3); }
__device__ inline float* st_row(StPair st, int r) { return st + r * 32; }

__device__ inline float4 st_read4(StPair st, int r, int c4) {
  return *reinterpret_cast<const float4*>(st + r * 32 + ((c4 ^ ((r >> 1) & 7)) << 2));
}
__device__ inline void st_write4(StPair st, int r, int c4, float4 v) {
  *reinterpret_cast<float4*>(st + r * 32 + ((c4 ^ ((r >> 1) & 7)) << 2)) = v;
}

// Where a wave's accumulators go in a staged [256][32] block: element i of
// row block mb of a lane belongs to row wm 128 + 32 mb + 8 (i / 4) + 4 (lane
// / 32) + i % 4 and column lane % 32, i.e. float row * 32 + st_pos(row, col).
// The swizzle key (row / 2) % 8 is the lane's bit (lane / 32) at position 1
// plus compile-time bits of i, so the offset is one of four per-lane values
// plus a constant: o[q(i)] + 1024 mb + 256 (i / 4) + 32 (i % 4), with
// q(i) = (i % 4) / 2 + 2 ((i / 4) % 2).  Each write is then one LDS store with
// an immediate offset instead of a rebuilt address.
struct StageOff {
  int o[4];
};
__device__ inline StageOff stage_offsets(int wm, int lane) {
  const int h = lane >> 5, col = lane & 31;
  const int base = wm * 4096 + h * 128 + (col & 3);
  const int g = ((col >> 2) ^ (h << 1)) << 2;
  return StageOff{{base + g, base + (g ^ 4), base + (g ^ 16), base + (g ^ 20)}};
}
// Each block passes through an empty asm statement that takes and returns it
// in accumulator registers, so no copy of it can be made before its round:
// otherwise the compiler copies later rounds' accumulators out early, spills
// them, and the reloads wait on all vector memory (the next tile's operand
// loads included).
template <int NBI, int NB>
__device__ inline void stage_acc(float* st, const StageOff& so, const f32x16_t (&acc)[4][NB]) {
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    f32x16_t v = acc[mb][NBI];
    asm volatile("" : "+a"(v));
#pragma unroll
    for (int i = 0; i < 16; ++i)
      st[so.o[((i & 3) >> 1) + 2 * ((i >> 2) & 1)] + mb * 1024 + (i >> 2) * 256 + (i & 3) * 32] = v[i];
  }
}

// Block NBI (0 .. NB-1) of the waves of column half 0 goes to st0, of column
// half 1 to st1.
template <int NBI, int NB>
__device__ inline void stage_block(StPair st0, StPair st1, const f32x16_t (&acc)[4][NB]) {
  const int w = wave_id();
  const int lane = opaque((int)threadIdx.x) & 63;
  stage_acc<NBI, NB>((w & 1) ? st1 : st0, stage_offsets(w >> 1, lane), acc);
}

// Block NBI of the waves of column half h (wave index & 1 == h) into st; the
// other two waves write nothing.
template <int NBI, int NB>
__device__ inline void stage_half(StPair st, int h, const f32x16_t (&acc)[4][NB]) {
  const int w = wave_id();
  if ((w & 1) != h) return;
  const int lane = opaque((int)threadIdx.x) & 63;
  stage_acc<NBI, NB>(st, stage_offsets(w >> 1, lane), acc);
}

// Panels: a matrix of prows rows cut into 64-byte pieces along its rows,
// piece p of row r at (p prows + r) * 64 bytes.  Offset of byte `byte` of
// row `row`:
__device__ inline long panel_off(long prows, long row, long byte) {
  return ((byte >> 6) * prows + row) * kRowB + (byte & 63);
}

// ------------------------------------------------------------------ elementwise dZ passes
// Pack EPT floats as 16 bytes of the element type.
template <class E>
__device__ inline u32x4_t pack16(const float* o) {
  if constexpr (E::kEpc == 8)
    return u32x4_t{Bf16::pack2(o[0], o[1]), Bf16::pack2(o[2], o[3]), Bf16::pack2(o[4], o[5]), Bf16::pack2(o[6], o[7])};
  else
    return u32x4_t{__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]), __float_as_uint(o[3])};
}

// Write a staged [16][1 KB] tile of dZ (LDS row stride rs) to the panels
// of C rows with NW waves: wave w writes 16 / NW consecutive 64-byte pieces,
// lane l row l / 4 and 16-byte chunk l % 4 of each, so every store of a wave
// is a contiguous kilobyte.  byte0: the tile's first byte along the rows.
template <int NW>
__device__ inline void ew_store_tile(const char* tile, int rs, char* dz, long C, long i0, long byte0, long rowbytes) {
  constexpr int PPW = 16 / NW;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int row = lane >> 2, sub = lane & 3;
#pragma unroll
  for (int q = 0; q < PPW; ++q) {
    const int pc = PPW * w + q;
    const long byte = byte0 + pc * kRowB + 16 * sub;
    if (byte < rowbytes)
      *reinterpret_cast<u32x4_t*>(dz + panel_off(C, i0 + row, byte)) =
          *reinterpret_cast<const u32x4_t*>(tile + row * rs + pc * kRowB + 16 * sub);
  }
}

// Store a staged [256][32] float block as the element type: rows [row0,
// row0 + 256) clipped to nrows, columns [col0, col0 + 32) clipped to
// [clo, ncols) (both multiples of 4/8).  The destination is row-major (`ld`
// elements per row) or, with prows set, in panels of prows rows.
template <class E>
__device__ inline void store_block(StPair st, char* dst, long ld, long row0, long col0, long nrows,
                                   long ncols, long clo = 0, long prows = 0) {
  constexpr int CPR = 32 * E::kElem / 16;  // 16-byte chunks per row
  constexpr int RPP = kThreads / CPR;
  const int tid = opaque((int)threadIdx.x);
  const int q = tid % CPR;
  const long col = col0 + (long)q * E::kEpc;
  if (col >= ncols || col < clo) return;
  // unrolled, so the LDS reads of all of a thread's rows go out before the
  // first store waits on them
#pragma unroll
  for (int k = 0; k < kBM / RPP; ++k) {
    const int r = tid / CPR + k * RPP;
    if (row0 + r >= nrows) break;
    u32x4_t o;
    if constexpr (E::kEpc == 8) {
      const float4 a = st_read4(st, r, 2 * q), b = st_read4(st, r, 2 * q + 1);
      o[0] = Bf16::pack2(a.x, a.y);
      o[1] = Bf16::pack2(a.z, a.w);
      o[2] = Bf16::pack2(b.x, b.y);
      o[3] = Bf16::pack2(b.z, b.w);
    } else {
      const float4 a = st_read4(st, r, q);
      o = u32x4_t{__float_as_uint(a.x), __float_as_uint(a.y), __float_as_uint(a.z), __float_as_uint(a.w)};
    }
    // a plain store: the next kernels read the block back soon (dH and dW the
    // dZ chunk, the elementwise pass a chunk's logits), and measured against
    // evict-first stores it was as fast for dZ and 1-2% faster for the logits
    const long byte = col * E::kElem;
    char* p = dst + (prows ? panel_off(prows, row0 + r, byte) : (row0 + r) * ld * E::kElem + byte);
    *reinterpret_cast<u32x4_t*>(p) = o;
  }
}

// Float32 destination: store (or add to) two staged [256][32] blocks, st0 at
// columns [col0, col0 + 32) and st1 at [col1, col1 + 32), rows [row0,
// min(row0 + 256, nrows)).  A thread owns one float4 chunk of every 32nd
// row.  Adding issues all of the thread's loads of both blocks first and
// waits once, so the read-modify-write costs one memory round trip per
// round instead of one per row (vector-memory counters complete in order,
// so a wait for a load also waits for every earlier store).
__device__ inline void rmw_pair_f32(StPair st0, StPair st1, float* dst, long ld, long row0, long col0, long col1,
                                    long nrows, long ncols, bool accumulate) {
  constexpr int kRowsPer = kBM / (kThreads / 8);  // rows per thread and block
  const int tid = opaque((int)threadIdx.x);
  const int q = tid & 7;  // float4 chunk of the row
  const int rt = tid >> 3;
  const long ca = col0 + 4 * q, cb = col1 + 4 * q;
  const bool oka = ca < ncols, okb = cb < ncols;
  if (!accumulate) {  // one block after the other
    if (oka)
      for (int r = rt; r < kBM; r += kThreads / 8) {
        if (row0 + r >= nrows) break;
        *reinterpret_cast<float4*>(dst + (row0 + r) * ld + ca) = st_read4(st0, r, q);
      }
    if (okb)
      for (int r = rt; r < kBM; r += kThreads / 8) {
        if (row0 + r >= nrows) break;
        *reinterpret_cast<float4*>(dst + (row0 + r) * ld + cb) = st_read4(st1, r, q);
      }
    return;
  }
  float4 oa[kRowsPer], ob[kRowsPer];
#pragma unroll
  for (int it = 0; it < kRowsPer; ++it) {
    const long r = row0 + rt + it * (kThreads / 8);
    const bool rv = r < nrows;
    oa[it] = rv && oka ? *reinterpret_cast<const float4*>(dst + r * ld + ca) : make_float4(0.f, 0.f, 0.f, 0.f);
    ob[it] = rv && okb ? *reinterpret_cast<const float4*>(dst + r * ld + cb) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int it = 0; it < kRowsPer; ++it) {
    const int r = rt + it * (kThreads / 8);
    if (row0 + r >= nrows) break;
    if (oka) {
      float4 v = st_read4(st0, r, q);
      v.x += oa[it].x;
      v.y += oa[it].y;
      v.z += oa[it].z;
      v.w += oa[it].w;
      *reinterpret_cast<float4*>(dst + (row0 + r) * ld + ca) = v;
    }
    if (okb) {
      float4 v = st_read4(st1, r, q);
      v.x += ob[it].x;
      v.y += ob[it].y;
      v.z += ob[it].z;
      v.w += ob[it].w;
      *reinterpret_cast<float4*>(dst + (row0 + r) * ld + cb) = v;
    }
  }
}

}  // namespace kd
