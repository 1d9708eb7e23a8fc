// Device building blocks shared by every contraction of the loss: a 256-row
// workgroup tile computed with gfx950 matrix cores, operands staged through
// LDS in double-buffered 128-byte slabs of the contraction dimension.
//
// Geometry (one workgroup = 4 waves of 64 lanes, 2 x 2):
//   tile        256 rows x BN columns (BN = 256, or 128 where two
//               accumulator sets must live side by side)
//   wave tile   128 rows x BN/2 columns = 4 x (BN/64) blocks of 32 x 32
//   MFMA        bf16: v_mfma_f32_32x32x16_bf16 (16 k per instruction)
//               fp32: v_mfma_f32_32x32x2_f32   (2 k per instruction)
//   LDS         both operands stored k-contiguous per row/column, row pitch
//               144 bytes (128 + 16 padding), so that the 16-byte fragment
//               reads of 16 consecutive lanes touch 64 distinct banks.
//
// A "k-group" is 32 bytes of the contraction dimension of one row: 16 bf16
// (one MFMA) or 8 fp32 (four MFMAs).  Lane half h = lane / 32 reads bytes
// [16h, 16h + 16) of each k-group for both operands, so the pairing of lane
// halves to physical k is the same on both sides and the products sum the
// right terms whatever order the instruction uses internally.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kd {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kBM = 256;                    // rows per workgroup tile
constexpr int kStageBytes = 128;            // contraction bytes per stage and row
constexpr int kPitch = kStageBytes + 16;    // LDS row pitch in bytes
constexpr int kKGroups = kStageBytes / 32;  // k-groups per stage
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

// ------------------------------------------------------------------ workgroup placement
// Workgroups are handed to the 8 XCDs round-robin by id.  Renumber them so that
// consecutive logical ids share an XCD (and its L2): XCD x runs logical ids
// [x*n/8, (x+1)*n/8).  Only done when n divides evenly.
__device__ inline int xcd_remap(int id, int n) {
  if (n % 8) return id;
  return (id % 8) * (n / 8) + id / 8;
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

// ------------------------------------------------------------------ operand loaders
// Operand stored k-contiguous in memory, NROWS rows per tile (rows of H, of
// dZ, of H^T, or of W seen as [d][V] when V is the contraction).  Thread t
// loads 16-byte chunk (t % 8) of rows (t / 8) + 32 j.
template <int NROWS>
struct KRowLoader {
  static constexpr int kPer = NROWS * 8 / kThreads;
  const char* rp[kPer];  // row base pointers (nullptr: row outside the operand)
  u32x4_t r[kPer];
  int q;

  __device__ inline void init_q() { q = threadIdx.x & 7; }
  __device__ inline int row_of(int j) const { return (threadIdx.x >> 3) + 32 * j; }

  // kbyte0: first contraction byte of the stage; kbytes: valid contraction bytes
  __device__ inline void load(long kbyte0, long kbytes) {
    const long off = kbyte0 + 16 * q;
    const bool kv = off < kbytes;
#pragma unroll
    for (int j = 0; j < kPer; ++j) r[j] = (kv && rp[j]) ? ld16(rp[j] + off) : zero4();
  }
  __device__ inline void store(char* s) const {
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      *reinterpret_cast<u32x4_t*>(s + row_of(j) * kPitch + 16 * q) = r[j];
  }
};

// Operand stored n-contiguous in memory ([K][N] row-major: W as [d][V], or dZ
// as [rows][V] when rows are the contraction).  Each thread loads an
// EPC x EPC block (EPC k-rows of one 16-byte column chunk), transposes it in
// registers and writes EPC k-contiguous 16-byte runs, one per column.
template <class E, int BN>
struct NColLoader {
  static constexpr int kKs = kStageBytes / E::kElem;  // k rows per stage
  static constexpr int kNkb = kKs / E::kEpc;          // k-blocks per stage (8)
  static constexpr int kNnc = BN / E::kEpc;           // column chunks
  static constexpr int kNblk = kNkb * kNnc;
  static constexpr int kPer = (kNblk + kThreads - 1) / kThreads;
  u32x4_t r[kPer][E::kEpc];
  const char* base;  // element (0, n0) of the tile's column panel
  long ld;           // row stride in bytes
  long N, n0, K;     // columns, first column, valid contraction rows

  __device__ inline void load(long k0) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int b = threadIdx.x + kThreads * i;
      const int kb = b % kNkb, nc = b / kNkb;
      const bool nv = (b < kNblk) && (n0 + nc * E::kEpc < N);
#pragma unroll
      for (int e = 0; e < E::kEpc; ++e) {
        const long k = k0 + kb * E::kEpc + e;
        r[i][e] = (nv && k < K) ? ld16(base + k * ld + (long)nc * 16) : zero4();
      }
    }
  }

  __device__ inline void store(char* s) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int b = threadIdx.x + kThreads * i;
      if (b >= kNblk) continue;
      const int kb = b % kNkb, nc = b / kNkb;
      if constexpr (E::kEpc == 8) {
        // 8 x 8 bf16 transpose: out[j] holds column j, k = 0..7
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
          u32x4_t o;
#pragma unroll
          for (int w = 0; w < 4; ++w)
            o[w] = __builtin_amdgcn_perm(r[i][2 * w + 1][j >> 1], r[i][2 * w][j >> 1], sel);
          *reinterpret_cast<u32x4_t*>(s + (nc * 8 + j) * kPitch + kb * 16) = o;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          u32x4_t o{r[i][0][j], r[i][1][j], r[i][2][j], r[i][3][j]};
          *reinterpret_cast<u32x4_t*>(s + (nc * 4 + j) * kPitch + kb * 16) = o;
        }
      }
    }
  }
};

// ------------------------------------------------------------------ tile compute
template <int BN>
struct TileShape {
  static constexpr int kWN = BN / 2;      // columns per wave
  static constexpr int kNB = kWN / 32;    // 32-wide blocks per wave
  static constexpr int kMB = 4;           // 32-high blocks per wave (128 rows)
  static constexpr int kABytes = kBM * kPitch;
  static constexpr int kBBytes = BN * kPitch;
  static constexpr int kStage = kABytes + kBBytes;
  static constexpr int kLds = 2 * kStage;
};

template <class E, int BN>
__device__ inline void mma_stage(const char* As, const char* Bs, f32x16_t (&acc)[4][BN / 64], int wm, int wn,
                                 int lane) {
  constexpr int NB = BN / 64;
  constexpr int WN = BN / 2;
  const char* ap = As + (wm * 128 + (lane & 31)) * kPitch + (lane >> 5) * 16;
  const char* bp = Bs + (wn * WN + (lane & 31)) * kPitch + (lane >> 5) * 16;
#pragma unroll
  for (int kg = 0; kg < kKGroups; ++kg) {
    u32x4_t a[4], b[NB];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) a[mb] = *reinterpret_cast<const u32x4_t*>(ap + mb * 32 * kPitch + kg * 32);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) b[nb] = *reinterpret_cast<const u32x4_t*>(bp + nb * 32 * kPitch + kg * 32);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) E::mma(acc[mb][nb], a[mb], b[nb]);
  }
}

template <int BN>
__device__ inline void zero_acc(f32x16_t (&acc)[4][BN / 64]) {
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < BN / 64; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.f;
}

// Software-pipelined contraction over stages [s0, s1): global loads of stage
// s+1 are in flight while stage s is multiplied out of LDS.  ALoad/BLoad
// expose load(stage) into registers and store(lds) of those registers.
// Ends with a barrier, so the caller may reuse the LDS right away.
template <class E, int BN, class LoadFn, class StoreFn>
__device__ inline void contract(char* lds, long s0, long s1, f32x16_t (&acc)[4][BN / 64], LoadFn&& load,
                                StoreFn&& store) {
  using S = TileShape<BN>;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
  if (s0 >= s1) return;
  load(s0);
  store(lds);
  __syncthreads();
  for (long s = s0; s < s1; ++s) {
    const int buf = (int)((s - s0) & 1);
    char* cur = lds + buf * S::kStage;
    if (s + 1 < s1) load(s + 1);
    mma_stage<E, BN>(cur, cur + S::kABytes, acc, wm, wn, lane);
    if (s + 1 < s1) store(lds + (buf ^ 1) * S::kStage);
    __syncthreads();
  }
}

// ------------------------------------------------------------------ epilogue staging
// Row stride (floats) of one staged column slice of the tile.
template <int BN>
struct Stage {
  static constexpr int kWN = BN / 2;
  static constexpr int kSP = kWN + 4;
  static constexpr int kBytes = kBM * kSP * 4;
};

// Copy the accumulators of the waves whose column half is `half` into LDS as
// [256 rows][BN/2 columns] floats (pitch BN/2 + 4).  Accumulator layout of
// the 32 x 32 MFMA output: lane l holds column l % 32 and, in register r,
// row 8 (r / 4) + 4 (l / 32) + r % 4 of its block.
template <int BN>
__device__ inline void stage_acc(float* st, const f32x16_t (&acc)[4][BN / 64], int half) {
  constexpr int NB = BN / 64;
  constexpr int SP = Stage<BN>::kSP;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
  if (wn != half) return;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 128 + mb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        st[row * SP + nb * 32 + (lane & 31)] = acc[mb][nb][r];
      }
}

// Store a staged [256][WN] float slice (rows [row0, row0 + 256) of a
// row-major destination with `ld` elements per row, columns [col0, col0+WN))
// converted to the element type, 16 bytes per lane.  Rows >= nrows are
// skipped.
template <class E, int WN>
__device__ inline void store_slice(const float* st, char* dst, long ld, long row0, long col0, long nrows) {
  constexpr int SP = WN + 4;
  constexpr int CPR = WN * E::kElem / 16;  // 16-byte chunks per row
  constexpr int RPP = kThreads / CPR;      // rows per pass
  const int q = threadIdx.x % CPR;
  for (int r = threadIdx.x / CPR; r < kBM; r += RPP) {
    if (row0 + r >= nrows) continue;
    const float* s = st + r * SP + q * E::kEpc;
    u32x4_t o;
    if constexpr (E::kEpc == 8) {
#pragma unroll
      for (int w = 0; w < 4; ++w) o[w] = Bf16::pack2(s[2 * w], s[2 * w + 1]);
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w) o[w] = __float_as_uint(s[w]);
    }
    *reinterpret_cast<u32x4_t*>(dst + ((row0 + r) * ld + col0) * E::kElem + q * 16) = o;
  }
}

// Float32 destination, row-major with `ld` floats per row: store (or add to)
// a staged [256][WN] slice at rows [row0, row0 + 256) x columns
// [col0, col0 + WN), clipped to nrows x ncols.  16 bytes per lane; a row's
// WN floats are covered by consecutive lanes.  ncols and ld must be
// multiples of 4.
template <int WN>
__device__ inline void rmw_slice_f32(const float* st, float* dst, long ld, long row0, long col0, long nrows,
                                     long ncols, bool accumulate) {
  constexpr int SP = WN + 4;
  constexpr int CPR = WN / 4;
  constexpr int RPP = kThreads / CPR;
  const int q = threadIdx.x % CPR;
  const long col = col0 + 4 * q;
  if (col >= ncols) return;
  for (int r = threadIdx.x / CPR; r < kBM; r += RPP) {
    const long row = row0 + r;
    if (row >= nrows) break;
    float4 v = *reinterpret_cast<const float4*>(st + r * SP + 4 * q);
    float4* p = reinterpret_cast<float4*>(dst + row * ld + col);
    if (accumulate) {
      const float4 o = *p;
      v.x += o.x;
      v.y += o.y;
      v.z += o.z;
      v.w += o.w;
    }
    *p = v;
  }
}

// ------------------------------------------------------------------ small helpers
__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ inline float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

}  // namespace kd
