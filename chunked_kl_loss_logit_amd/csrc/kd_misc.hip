// Per-row and elementwise kernels around the tile contractions.
//
//   compact        valid-row list from the mask, in row order (masked rows
//                  skip all contraction work and are never read)
//   topk_prep      teacher side of each valid row, from "Efficient Knowledge
//                  Distillation for LLMs: Offline Top-K Logits and a Fused
//                  Chunked KL Loss", §3 "Offline distillation": the teacher
//                  terms need the K cached entries only.  p = softmax(A / tau),
//                  sum p log p, and the (index, p, position) triples sorted by
//                  index so the tile epilogue can gather with one cursor.
//   *_combine      merge the per-split running max / sum partials into the
//                  row's log Z and KL (§3: each row keeps a scalar log Z)
//   topk_shard_*   the same merge for a vocabulary shard of W: a row record
//                  (max, sum, cross term) per shard, then one merge of the
//                  shards' records (the timing at the largest tensor-parallel
//                  rank of App. B; sharding the head by vocabulary columns is
//                  the usual tensor-parallel layout of an output head)
//   gather_transpose, reduce_dh, zero_masked_rows, fill_zero: chunk plumbing
//                  of the backward pass
#include <stdint.h>

#include "kd_gemm.h"
#include "kd_launch.h"

namespace kd {

namespace {

constexpr int kCompactThreads = 1024;

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

template <int NT>
__device__ inline float block_max(float v, float* red) {
  v = wave_max(v);
  if constexpr (NT > 64) {
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    v = red[0];
#pragma unroll
    for (int i = 1; i < NT / 64; ++i) v = fmaxf(v, red[i]);
  }
  return v;
}
template <int NT>
__device__ inline float block_sum(float v, float* red) {
  v = wave_sum(v);
  if constexpr (NT > 64) {
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    v = red[0];
#pragma unroll
    for (int i = 1; i < NT / 64; ++i) v += red[i];
  }
  return v;
}

}  // namespace

// ------------------------------------------------------------------ compaction
__global__ __launch_bounds__(kCompactThreads) void compact_kernel(const uint8_t* mask, long T, int32_t* rows,
                                                                  int32_t* count) {
  __shared__ int sums[kCompactThreads];
  const long per = (T + kCompactThreads - 1) / kCompactThreads;
  const long b = (long)threadIdx.x * per, e = min(T, b + per);
  int n = 0;
  for (long t = b; t < e; ++t) n += (mask == nullptr || mask[t] != 0);
  sums[threadIdx.x] = n;
  __syncthreads();
  for (int off = 1; off < kCompactThreads; off <<= 1) {
    const int v = threadIdx.x >= off ? sums[threadIdx.x - off] : 0;
    __syncthreads();
    sums[threadIdx.x] += v;
    __syncthreads();
  }
  int pos = sums[threadIdx.x] - n;
  for (long t = b; t < e; ++t)
    if (mask == nullptr || mask[t] != 0) rows[pos++] = (int32_t)t;
  if (threadIdx.x == kCompactThreads - 1) *count = sums[kCompactThreads - 1];
}

hipError_t launch_compact(const uint8_t* mask, int64_t T, Compact c, hipStream_t st) {
  hipLaunchKernelGGL(compact_kernel, dim3(1), dim3(kCompactThreads), 0, st, mask, (long)T, c.rows, c.count);
  return hipGetLastError();
}

// ------------------------------------------------------------------ teacher prep
// One workgroup per row.  Dynamic LDS: KP sort keys (64-bit: biased index in
// the high word, position k in the low word) and K probabilities.
//
// Row t's temperature is tau_rows[t] when given (per-token temperature, the
// adaptive-distillation abstract on the WASD page), else the scalar one.
// The teacher probabilities are softmax(A_t / tau) over the K cached entries,
// or, with a teacher log-normaliser, the cached probabilities
// exp(A_t / tau - teacher_lse[t]) of the full teacher softmax, which keep
// their partial mass m = sum_k p_k ("Efficient Knowledge Distillation for
// LLMs ...", §3 "Offline distillation").  A cross-entropy term with weight
// beta on label y is one more entry (y, beta), the others weigh (1 - beta) p,
// so the loss keeps the support form sum w log p - sum w s + mass L with
// mass = (1 - beta) m + beta.
//
// For a shard holding columns [v0, v0 + vs) of W, indices (the label too) are
// shifted to the shard's columns and those outside it become INT32_MAX, which
// sorts after every column and is never matched; the teacher terms stay those
// of all K entries.
template <int NT>
__global__ __launch_bounds__(NT) void topk_prep_kernel(const float* logits, const int32_t* idx, const uint8_t* mask,
                                                       int K, int KE, int KP, TopkPrepOpts o, TopkRowData rd,
                                                       float* z_topk) {
  extern __shared__ __attribute__((aligned(16))) char sm[];
  __shared__ float red[NT / 64 > 0 ? NT / 64 : 1];
  uint64_t* key = reinterpret_cast<uint64_t*>(sm);
  float* p = reinterpret_cast<float*>(key + KP);
  const long t = blockIdx.x;
  const long base = t * K, pbase = t * KE;
  if (z_topk)
    for (int k = threadIdx.x; k < K; k += NT) z_topk[base + k] = 0.f;
  if (mask != nullptr && mask[t] == 0) return;

  float inv_tau = o.inv_tau, c2 = o.c2;
  if (o.tau_rows) {
    const float tt = o.tau_rows[t];
    inv_tau = 1.0f / tt;
    c2 = (float)(1.4426950408889634 / (double)tt);
  }
  // log p = A_t / tau - log-normaliser (of the K entries, or the given one)
  for (int k = threadIdx.x; k < K; k += NT) p[k] = logits[base + k] * inv_tau;
  float lz;
  if (o.teacher_lse) {
    lz = o.teacher_lse[t];
    __syncthreads();
  } else {
    float mx = -INFINITY;
    for (int k = threadIdx.x; k < K; k += NT) mx = fmaxf(mx, p[k]);
    mx = block_max<NT>(mx, red);
    float s = 0.f;
    for (int k = threadIdx.x; k < K; k += NT) s += expf(p[k] - mx);
    s = block_sum<NT>(s, red);
    lz = mx + logf(s);
  }
  float ent = 0.f, m = 0.f;
  for (int k = threadIdx.x; k < K; k += NT) {
    const float lp = p[k] - lz;
    const float pk = expf(lp);
    p[k] = pk;
    ent = fmaf(pk, lp, ent);
    m += pk;
  }
  ent = block_sum<NT>(ent, red);
  float mass = 1.f;  // renormalised: exactly one
  if (o.teacher_lse) mass = block_sum<NT>(m, red);
  const bool ce = KE > K;
  // weight of the forward-KL part: 1 - beta with a CE label, times 1 - r
  // under KL mixing (the reverse part comes from topk_reverse_kernel)
  const float wk = (ce ? 1.f - o.beta : 1.f) * (1.f - o.rev);
  if (ce || o.rev != 0.f) {
    ent *= wk;
    mass = fmaf(wk, mass, ce ? o.beta : 0.f);
  }

  // sort (index, position) pairs by index; ties keep position order
  for (int j = threadIdx.x; j < KP; j += NT) {
    int32_t v = j < K ? idx[base + j] : (j < KE ? o.labels[t] : 0);
    if (o.bad && j < KE && (uint32_t)v >= (uint32_t)o.V) atomicAdd(o.bad, 1);  // the check on request
    if (o.vs > 0) {  // a vocabulary shard: local column, or a sentinel past every column
      v -= o.v0;
      v = (uint32_t)v < (uint32_t)o.vs ? v : INT32_MAX;
    }
    key[j] = j < KE ? ((uint64_t)((uint32_t)v ^ 0x80000000u) << 32) | (uint32_t)j : ~0ull;
  }
  for (int size = 2; size <= KP; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      __syncthreads();
      for (int i = threadIdx.x; i < (KP >> 1); i += NT) {
        const int lo = 2 * stride * (i / stride) + (i % stride);
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const uint64_t x = key[lo], y = key[hi];
        if ((x > y) == up) {
          key[lo] = y;
          key[hi] = x;
        }
      }
    }
  }
  __syncthreads();
  for (int j = threadIdx.x; j < KE; j += NT) {
    const uint64_t kv = key[j];
    const uint32_t k = (uint32_t)(kv & 0xffffffffu);
    const float w = k < (uint32_t)K ? wk * p[k] : o.beta;
    rd.pair[pbase + j] = make_int2((int32_t)((uint32_t)(kv >> 32) ^ 0x80000000u), __float_as_int(w));
    rd.perm[pbase + j] = (uint16_t)k;
    if (rd.zpair) rd.zpair[pbase + j] = 0.f;  // an entry no tile matches reads as 0
  }
  if (threadIdx.x == 0) {
    rd.ent[t] = ent;
    rd.rowc[t] = make_float4(c2, inv_tau, mass, log2f(mass));
  }
}

hipError_t launch_topk_prep(const float* logits, const int32_t* idx, const uint8_t* mask, int64_t T, int64_t K,
                            int64_t KE, const TopkPrepOpts& o, TopkRowData rd, float* z_topk, hipStream_t st) {
  int KP = 1;
  while (KP < KE) KP <<= 1;
  const size_t shm = (size_t)KP * 8 + (size_t)K * 4;
  const dim3 grid((unsigned)T);
  if (shm > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(topk_prep_kernel<256>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
    if (e != hipSuccess) return e;
  }
  if (KE <= 64)
    hipLaunchKernelGGL(topk_prep_kernel<64>, grid, dim3(64), shm, st, logits, idx, mask, (int)K, (int)KE, KP, o, rd,
                       z_topk);
  else
    hipLaunchKernelGGL(topk_prep_kernel<256>, grid, dim3(256), shm, st, logits, idx, mask, (int)K, (int)KE, KP, o,
                       rd, z_topk);
  return hipGetLastError();
}

// ------------------------------------------------------------------ z_topk from the sorted entries
// One block of 64 threads per compacted row.
__global__ __launch_bounds__(64) void topk_zpermute_kernel(TopkRowData rd, Compact c, int KE, int Kz, float* z_topk,
                                                           long jb, long je) {
  const long j = jb + blockIdx.x;
  if (j >= je || j >= (long)*c.count) return;
  const long t = c.rows[j];
  const long pb = t * KE;
  for (int i = threadIdx.x; i < KE; i += 64) {
    const int k = rd.perm[pb + i];
    if (k < Kz) z_topk[t * Kz + k] = rd.zpair[pb + i];
  }
}

hipError_t launch_topk_zpermute(const TopkRowData& rd, Compact c, int64_t T, int64_t KE, int64_t Kz, float* z_topk,
                                int64_t jb, int64_t je, hipStream_t st) {
  if (je > T) je = T;
  if (je <= jb) return hipSuccess;
  hipLaunchKernelGGL(topk_zpermute_kernel, dim3((unsigned)(je - jb)), dim3(64), 0, st, rd, c, (int)KE, (int)Kz,
                     z_topk, (long)jb, (long)je);
  return hipGetLastError();
}

// ------------------------------------------------------------------ KL mixing on the cached entries
// One block per compacted row: a = z_topk / tau_t and b = A / tau_t over the
// K entries, q~ = softmax(a), p^ = softmax(b), RKL = sum q~ (log q~ - log p^).
// The entries are read from global memory once per pass (K floats each).
template <int NT>
__global__ __launch_bounds__(NT) void topk_reverse_kernel(const float* z_topk, const float* logits, Compact c,
                                                          int K, int KE, float wr, TopkRowData rd, float* kl,
                                                          int upd, long jb, long je) {
  __shared__ float red[NT / 64 > 0 ? NT / 64 : 1];
  const long j = jb + blockIdx.x;
  if (j >= je || j >= (long)*c.count) return;
  const long t = c.rows[j];
  const float it = rd.rowc[t].y;  // 1 / tau_t
  const float* za = z_topk + t * K;
  const float* zb = logits + t * K;
  float ma = -INFINITY, mb = -INFINITY;
  for (int k = threadIdx.x; k < K; k += NT) {
    ma = fmaxf(ma, za[k] * it);
    mb = fmaxf(mb, zb[k] * it);
  }
  ma = block_max<NT>(ma, red);
  mb = block_max<NT>(mb, red);
  float sa = 0.f, sb = 0.f;
  for (int k = threadIdx.x; k < K; k += NT) {
    sa += expf(za[k] * it - ma);
    sb += expf(zb[k] * it - mb);
  }
  sa = block_sum<NT>(sa, red);
  sb = block_sum<NT>(sb, red);
  const float la = ma + logf(sa), lb = mb + logf(sb);
  float rk = 0.f;
  for (int k = threadIdx.x; k < K; k += NT) {
    const float lq = za[k] * it - la;
    rk = fmaf(expf(lq), lq - (zb[k] * it - lb), rk);
  }
  rk = block_sum<NT>(rk, red);
  if (kl != nullptr && threadIdx.x == 0) kl[t] = fmaf(wr, rk, kl[t]);
  if (upd) {
    const long pb = t * KE;
    for (int i = threadIdx.x; i < KE; i += NT) {
      const int k = rd.perm[pb + i];
      if (k >= K) continue;  // the CE label's entry
      const float lq = za[k] * it - la;
      const float v = expf(lq) * (lq - (zb[k] * it - lb) - rk);
      int2 e = rd.pair[pb + i];
      e.y = __float_as_int(fmaf(-wr, v, __int_as_float(e.y)));
      rd.pair[pb + i] = e;
    }
  }
}

hipError_t launch_topk_reverse(const float* z_topk, const float* logits, Compact c, int64_t T, int64_t K,
                               int64_t KE, float wr, TopkRowData rd, float* kl, bool upd, int64_t jb, int64_t je,
                               hipStream_t st) {
  if (je > T) je = T;
  if (je <= jb) return hipSuccess;
  const dim3 grid((unsigned)(je - jb));
  if (K <= 64)
    hipLaunchKernelGGL(topk_reverse_kernel<64>, grid, dim3(64), 0, st, z_topk, logits, c, (int)K, (int)KE, wr, rd,
                       kl, upd ? 1 : 0, (long)jb, (long)je);
  else
    hipLaunchKernelGGL(topk_reverse_kernel<256>, grid, dim3(256), 0, st, z_topk, logits, c, (int)K, (int)KE, wr,
                       rd, kl, upd ? 1 : 0, (long)jb, (long)je);
  return hipGetLastError();
}

// ------------------------------------------------------------------ combines
// Thread j: (a) zero kl/lse of row j if it is masked, (b) if j is a valid
// compacted row, merge its S partials (m2, l, x) in split order:
// kl = sum w log p - x / tau + mass L.
// (m2, l, x) of S partials at stride `stride` (float4 units), in split order
__device__ inline float3 merge_splits(const float4* pp, int S, long stride) {
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, pp[(long)s * stride].x);
  float l = 0.f, x = 0.f;
  for (int s = 0; s < S; ++s) {
    const float4 q = pp[(long)s * stride];
    l += q.y * exp2f(q.x - M);
    x += q.z;
  }
  return make_float3(M, l, x);
}

__global__ void topk_combine_kernel(const float* part, int S, long stride, Compact c, const uint8_t* mask,
                                    TopkRowData rd, long T, float* kl, float* lse, long jb, long je,
                                    int zero_masked) {
  const long j = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= T) return;
  if (zero_masked && mask != nullptr && mask[j] == 0) {
    kl[j] = 0.f;
    lse[j] = 0.f;
  }
  if (j < jb || j >= je || j >= *c.count) return;
  const float3 q = merge_splits(reinterpret_cast<const float4*>(part) + (j - jb), S, stride);
  const float M = q.x, l = q.y, x = q.z;
  const long t = c.rows[j];
  const float4 rc = rd.rowc[t];
  const float L = (M + log2f(l)) * kLn2;
  lse[t] = L;
  kl[t] = rd.ent[t] - x * rc.y + rc.z * L;
}

hipError_t launch_topk_combine(const float* part, int S, int64_t part_stride, Compact c, const uint8_t* mask,
                               TopkRowData rd, int64_t T, float* kl, float* lse, int64_t jb, int64_t je,
                               bool zero_masked, hipStream_t st) {
  const dim3 grid((unsigned)((T + 255) / 256));
  hipLaunchKernelGGL(topk_combine_kernel, grid, dim3(256), 0, st, part, S, (long)part_stride, c, mask, rd, (long)T,
                     kl, lse, (long)jb, (long)je, zero_masked ? 1 : 0);
  return hipGetLastError();
}

__global__ void topk_shard_record_kernel(const float* part, int S, long stride, Compact c, const uint8_t* mask,
                                         TopkRowData rd, long T, float4* rec, float2* trow, long jb, long je,
                                         int zero_masked) {
  const long j = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= T) return;
  if (zero_masked && mask != nullptr && mask[j] == 0) {
    rec[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    trow[j] = make_float2(0.f, 0.f);
  }
  if (j < jb || j >= je || j >= *c.count) return;
  const float3 q = merge_splits(reinterpret_cast<const float4*>(part) + (j - jb), S, stride);
  const long t = c.rows[j];
  const float4 rc = rd.rowc[t];
  rec[t] = make_float4(q.x, q.y, q.z * rc.y, 0.f);
  trow[t] = make_float2(rd.ent[t], rc.z);
}

hipError_t launch_topk_shard_record(const float* part, int S, int64_t part_stride, Compact c, const uint8_t* mask,
                                    TopkRowData rd, int64_t T, float4* rec, float2* trow, int64_t jb, int64_t je,
                                    bool zero_masked, hipStream_t st) {
  const dim3 grid((unsigned)((T + 255) / 256));
  hipLaunchKernelGGL(topk_shard_record_kernel, grid, dim3(256), 0, st, part, S, (long)part_stride, c, mask, rd,
                     (long)T, rec, trow, (long)jb, (long)je, zero_masked ? 1 : 0);
  return hipGetLastError();
}

// Row t: the R shards' (m2, l) give the log-normaliser over all columns,
// their cross terms add: kl = entropy term - sum of cross terms + mass L.
__global__ void topk_shard_combine_kernel(const float4* rec, int R, long T, const float2* trow,
                                          const uint8_t* mask, float* kl, float* lse) {
  const long t = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  if (mask != nullptr && mask[t] == 0) {
    kl[t] = 0.f;
    lse[t] = 0.f;
    return;
  }
  const float3 q = merge_splits(rec + t, R, T);
  const float2 tr = trow[t];
  const float L = (q.x + log2f(q.y)) * kLn2;
  lse[t] = L;
  kl[t] = tr.x - q.z + tr.y * L;
}

hipError_t launch_topk_shard_combine(const float4* rec, int R, int64_t T, const float2* trow, const uint8_t* mask,
                                     float* kl, float* lse, hipStream_t st) {
  const dim3 grid((unsigned)((T + 255) / 256));
  hipLaunchKernelGGL(topk_shard_combine_kernel, grid, dim3(256), 0, st, rec, R, (long)T, trow, mask, kl, lse);
  return hipGetLastError();
}

// Partials per (split, row): (ms, ls, mt, lt), (R, R2, -, -) in base 2, with
// R = sum 2^(yt - mt) (yt - ys) and R2 = sum 2^(ys - ms) (ys - yt); the
// partial row p holds compacted row jb + p.
// The pair of float4 (ms, ls, mt, lt), (R, R2, -, -) of row p merged over S
// partials at stride `stride` rows, in order.
struct FullMerged {
  float4 q, x;
};

__device__ inline FullMerged merge_full(const float4* pp, int S, long stride, long p) {
  float Ms = -INFINITY, Mt = -INFINITY;
  for (int s = 0; s < S; ++s) {
    const float4 q = pp[2 * ((long)s * stride + p)];
    Ms = fmaxf(Ms, q.x);
    Mt = fmaxf(Mt, q.z);
  }
  float ls = 0.f, lt = 0.f, R = 0.f, R2 = 0.f;
  for (int s = 0; s < S; ++s) {
    const float4 q = pp[2 * ((long)s * stride + p)];
    const float4 x = pp[2 * ((long)s * stride + p) + 1];
    const float fs = exp2f(q.x - Ms);
    ls += q.y * fs;
    R2 += x.y * fs;
    const float f = exp2f(q.z - Mt);
    lt += q.w * f;
    R += x.x * f;
  }
  return FullMerged{make_float4(Ms, ls, Mt, lt), make_float4(R, R2, 0.f, 0.f)};
}

// Row t's outputs from its merged partials.
__device__ inline void full_finish(const FullMerged& m, long t, float r, float* kl, float* lse_s, float* lse_t,
                                   float* kl_rev) {
  const float Ls2 = m.q.x + log2f(m.q.y), Lt2 = m.q.z + log2f(m.q.w);
  lse_s[t] = Ls2 * kLn2;
  lse_t[t] = Lt2 * kLn2;
  const float fwd = (m.x.x / m.q.w - Lt2 + Ls2) * kLn2;
  const float rev = (m.x.y / m.q.y - Ls2 + Lt2) * kLn2;
  kl[t] = r == 0.f ? fwd : (1.f - r) * fwd + r * rev;
  if (kl_rev) kl_rev[t] = rev;
}

__device__ inline void full_zero(long t, float* kl, float* lse_s, float* lse_t, float* kl_rev) {
  kl[t] = 0.f;
  lse_s[t] = 0.f;
  lse_t[t] = 0.f;
  if (kl_rev) kl_rev[t] = 0.f;
}

__global__ void full_combine_kernel(const float* part, int S, long stride, Compact c, const uint8_t* mask, long T,
                                    float r, float* kl, float* lse_s, float* lse_t, float* kl_rev, long jb, long je,
                                    int zero_masked) {
  const long j = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= T) return;
  if (zero_masked && mask != nullptr && mask[j] == 0) full_zero(j, kl, lse_s, lse_t, kl_rev);
  if (j < jb || j >= je || j >= *c.count) return;
  const FullMerged m = merge_full(reinterpret_cast<const float4*>(part), S, stride, j - jb);
  full_finish(m, c.rows[j], r, kl, lse_s, lse_t, kl_rev);
}

// A vocabulary shard's forward: row t's merged partials are its record,
// rec[t] = the pair above (zero on masked rows with zero_masked).
__global__ void full_shard_record_kernel(const float* part, int S, long stride, Compact c, const uint8_t* mask,
                                         long T, float4* rec, long jb, long je, int zero_masked) {
  const long j = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= T) return;
  if (zero_masked && mask != nullptr && mask[j] == 0) {
    rec[2 * j] = make_float4(0.f, 0.f, 0.f, 0.f);
    rec[2 * j + 1] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  if (j < jb || j >= je || j >= *c.count) return;
  const FullMerged m = merge_full(reinterpret_cast<const float4*>(part), S, stride, j - jb);
  const long t = c.rows[j];
  rec[2 * t] = m.q;
  rec[2 * t + 1] = m.x;
}

hipError_t launch_full_shard_record(const float* part, int S, int64_t part_stride, Compact c, const uint8_t* mask,
                                    int64_t T, float4* rec, int64_t jb, int64_t je, bool zero_masked,
                                    hipStream_t st) {
  const dim3 grid((unsigned)((T + 255) / 256));
  hipLaunchKernelGGL(full_shard_record_kernel, grid, dim3(256), 0, st, part, S, (long)part_stride, c, mask, (long)T,
                     rec, (long)jb, (long)je, zero_masked ? 1 : 0);
  return hipGetLastError();
}

// Row t from the R shards' records rec [R][T] (pairs of float4).
__global__ void full_shard_combine_kernel(const float4* rec, int R, long T, const uint8_t* mask, float r, float* kl,
                                          float* lse_s, float* lse_t, float* kl_rev) {
  const long t = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  if (mask != nullptr && mask[t] == 0) {
    full_zero(t, kl, lse_s, lse_t, kl_rev);
    return;
  }
  full_finish(merge_full(rec, R, T, t), t, r, kl, lse_s, lse_t, kl_rev);
}

hipError_t launch_full_shard_combine(const float4* rec, int R, int64_t T, const uint8_t* mask, float r, float* kl,
                                     float* lse_s, float* lse_t, float* kl_rev, hipStream_t st) {
  const dim3 grid((unsigned)((T + 255) / 256));
  hipLaunchKernelGGL(full_shard_combine_kernel, grid, dim3(256), 0, st, rec, R, (long)T, mask, r, kl, lse_s, lse_t,
                     kl_rev);
  return hipGetLastError();
}

hipError_t launch_full_combine(const float* part, int S, int64_t part_stride, Compact c, const uint8_t* mask,
                               int64_t T, float r, float* kl, float* lse_s, float* lse_t, float* kl_rev, int64_t jb,
                               int64_t je, bool zero_masked, hipStream_t st) {
  const dim3 grid((unsigned)((T + 255) / 256));
  hipLaunchKernelGGL(full_combine_kernel, grid, dim3(256), 0, st, part, S, (long)part_stride, c, mask, (long)T, r,
                     kl, lse_s, lse_t, kl_rev, (long)jb, (long)je, zero_masked ? 1 : 0);
  return hipGetLastError();
}

// Single call, full vocabulary: the two heads' log-normalisers from the
// top-K tiles' split partials (m2, l, -, -) of each head.
__global__ void full_lse_combine_kernel(const float* part_s, const float* part_t, int S, long stride, Compact c,
                                        const uint8_t* mask, long T, float* kl, float* lse_s, float* lse_t,
                                        float* kl_rev, long jb, long je, int zero_masked) {
  const long j = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= T) return;
  if (zero_masked && mask != nullptr && mask[j] == 0) {
    kl[j] = 0.f;
    lse_s[j] = 0.f;
    lse_t[j] = 0.f;
    if (kl_rev) kl_rev[j] = 0.f;
  }
  if (j < jb || j >= je || j >= *c.count) return;
  const float4* ps = reinterpret_cast<const float4*>(part_s) + (j - jb);
  const float4* pt = reinterpret_cast<const float4*>(part_t) + (j - jb);
  float Ms = -INFINITY, Mt = -INFINITY;
  for (int s = 0; s < S; ++s) {
    Ms = fmaxf(Ms, ps[(long)s * stride].x);
    Mt = fmaxf(Mt, pt[(long)s * stride].x);
  }
  float ls = 0.f, lt = 0.f;
  for (int s = 0; s < S; ++s) {
    const float4 a = ps[(long)s * stride], b = pt[(long)s * stride];
    ls += a.y * exp2f(a.x - Ms);
    lt += b.y * exp2f(b.x - Mt);
  }
  const long t = c.rows[j];
  lse_s[t] = (Ms + log2f(ls)) * kLn2;
  lse_t[t] = (Mt + log2f(lt)) * kLn2;
}

hipError_t launch_full_lse_combine(const float* part_s, const float* part_t, int S, int64_t part_stride, Compact c,
                                   const uint8_t* mask, int64_t T, float* kl, float* lse_s, float* lse_t,
                                   float* kl_rev, int64_t jb, int64_t je, bool zero_masked, hipStream_t st) {
  hipLaunchKernelGGL(full_lse_combine_kernel, dim3((unsigned)((T + 255) / 256)), dim3(256), 0, st, part_s, part_t, S,
                     (long)part_stride, c, mask, (long)T, kl, lse_s, lse_t, kl_rev, (long)jb, (long)je,
                     zero_masked ? 1 : 0);
  return hipGetLastError();
}

// KL(p||q) = ln2 sum p (yt - ys) - Lt + Ls and KL(q||p) = ln2 sum q (ys - yt) - Ls + Lt
// per valid row, the sums taken over the terms' column blocks in order.
__global__ void full_kl_from_terms_kernel(const float2* terms, int nblk, Compact c, const float* lse_s,
                                          const float* lse_t, float r, float* kl, float* kl_rev, long jb, long je) {
  const long j = jb + (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= je || j >= *c.count) return;
  const float2* tr = terms + (j - jb) * nblk;
  float a = 0.f, b = 0.f;
  for (int k = 0; k < nblk; ++k) {
    a += tr[k].x;
    b += tr[k].y;
  }
  const long t = c.rows[j];
  const float d = lse_s[t] - lse_t[t];
  const float fwd = a * kLn2 + d, rev = b * kLn2 - d;
  kl[t] = r == 0.f ? fwd : (1.f - r) * fwd + r * rev;
  if (kl_rev) kl_rev[t] = rev;
}

hipError_t launch_full_kl_from_terms(const float2* terms, int nblk, Compact c, const float* lse_s,
                                     const float* lse_t, float r, float* kl, float* kl_rev, int64_t jb, int64_t je,
                                     hipStream_t st) {
  const int64_t n = je - jb;
  hipLaunchKernelGGL(full_kl_from_terms_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, terms, nblk, c,
                     lse_s, lse_t, r, kl, kl_rev, (long)jb, (long)je);
  return hipGetLastError();
}

// ------------------------------------------------------------------ chunk plumbing
// out[j][i] = H[rows[c0 + i]][j] for i < M (valid rows of the chunk), 0 for
// M <= i < C.  64 x 64 tiles through LDS.
template <typename U>
__global__ __launch_bounds__(256) void gather_transpose_kernel(const U* H, long d, Compact c, long c0, long C,
                                                               U* out) {
  __shared__ U tile[64][65];
  const long M = min(C, (long)*c.count - c0);
  const long i0 = (long)blockIdx.x * 64, j0 = (long)blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int ii = ty; ii < 64; ii += 4) {
    const long i = i0 + ii, j = j0 + tx;
    U v = 0;
    if (i < M && j < d) v = H[(long)c.rows[c0 + i] * d + j];
    tile[ii][tx] = v;
  }
  __syncthreads();
  for (int jj = ty; jj < 64; jj += 4) {
    const long j = j0 + jj, i = i0 + tx;
    if (j < d && i < C) *reinterpret_cast<U*>(reinterpret_cast<char*>(out) + panel_off(d, j, i * (long)sizeof(U))) = tile[tx][jj];
  }
}

// The same for bf16 when d and C are multiples of 64, 16 bytes per access:
// a thread loads 8 consecutive hidden values of a row and stores 8
// consecutive rows of one hidden index (16 bytes of one 64-byte piece), so a
// wave's store covers two contiguous 512-byte runs of the panels.
__global__ __launch_bounds__(256) void gather_transpose16_kernel(const uint16_t* H, long d, Compact c, long c0, long C,
                                                                uint16_t* out) {
  constexpr int kLd = 72;  // row stride of the LDS tile in elements (16-byte aligned rows)
  __shared__ __attribute__((aligned(16))) uint16_t tile[64 * kLd];
  const long M = min(C, (long)*c.count - c0);
  const long i0 = (long)blockIdx.x * 64, j0 = (long)blockIdx.y * 64;
  const int t = threadIdx.x, q = t & 7;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int ii = (t >> 3) + 32 * r;
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (i0 + ii < M) v = *reinterpret_cast<const u32x4_t*>(H + (long)c.rows[c0 + i0 + ii] * d + j0 + 8 * q);
    *reinterpret_cast<u32x4_t*>(tile + ii * kLd + 8 * q) = v;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int jj = (t >> 3) + 32 * r;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = (uint32_t)tile[(8 * q + 2 * e) * kLd + jj] | ((uint32_t)tile[(8 * q + 2 * e + 1) * kLd + jj] << 16);
    *reinterpret_cast<u32x4_t*>(reinterpret_cast<char*>(out) + panel_off(d, j0 + jj, (i0 + 8 * q) * 2)) =
        u32x4_t{w[0], w[1], w[2], w[3]};
  }
}

hipError_t launch_gather_transpose(const void* H, int elem, int64_t d, Compact c, int64_t c0, int64_t C, void* out,
                                   hipStream_t st) {
  const dim3 grid((unsigned)((C + 63) / 64), (unsigned)((d + 63) / 64));
  if (elem == 2 && d % 64 == 0 && C % 64 == 0)
    hipLaunchKernelGGL(gather_transpose16_kernel, grid, dim3(256), 0, st, (const uint16_t*)H, (long)d, c, (long)c0,
                       (long)C, (uint16_t*)out);
  else if (elem == 2)
    hipLaunchKernelGGL(gather_transpose_kernel<uint16_t>, grid, dim3(256), 0, st, (const uint16_t*)H, (long)d, c,
                       (long)c0, (long)C, (uint16_t*)out);
  else
    hipLaunchKernelGGL(gather_transpose_kernel<uint32_t>, grid, dim3(256), 0, st, (const uint32_t*)H, (long)d, c,
                       (long)c0, (long)C, (uint32_t*)out);
  return hipGetLastError();
}

// Rows of one chunk of compacted rows in panels of C rows: byte b of H row
// rows[c0 + i] goes to panel_off(C, i, b).  A block covers 64 rows of one
// 64-byte piece, four threads per piece, so a wave writes 16 consecutive
// rows of the piece: one contiguous kilobyte.  Rows past the chunk's valid
// rows are not written (the tiles never read them).
__global__ __launch_bounds__(256) void gather_panels_kernel(const char* H, long rowb, Compact c, long c0, long C,
                                                            char* out) {
  const long M = min(C, (long)*c.count - c0);
  const long i = (long)blockIdx.y * 64 + (threadIdx.x >> 2);
  const long b = (long)blockIdx.x * kRowB + 16 * (threadIdx.x & 3);
  if (i >= M || b >= rowb) return;
  const u32x4_t v = *reinterpret_cast<const u32x4_t*>(H + (long)c.rows[c0 + i] * rowb + b);
  *reinterpret_cast<u32x4_t*>(out + panel_off(C, i, b)) = v;
}

hipError_t launch_gather_panels(const void* H, int64_t row_bytes, Compact c, int64_t c0, int64_t C, void* out,
                                hipStream_t st) {
  const dim3 grid((unsigned)((row_bytes + kRowB - 1) / kRowB), (unsigned)((C + 63) / 64));
  hipLaunchKernelGGL(gather_panels_kernel, grid, dim3(256), 0, st, static_cast<const char*>(H), (long)row_bytes, c,
                     (long)c0, (long)C, static_cast<char*>(out));
  return hipGetLastError();
}

// dH[rows[c0 + i]][j..j+3] = sum over s of part[s][i][j..j+3], in split order.
template <int ELEM>
__global__ void reduce_dh_kernel(const float* part, int S, long C, long d, Compact c, long c0, void* dH) {
  const long q = (long)blockIdx.x * blockDim.x + threadIdx.x;  // float4 index within [C][d]
  const long d4 = d / 4;
  const long i = q / d4, j = (q % d4) * 4;
  const long M = min(C, (long)*c.count - c0);
  if (i >= M) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < S; ++s) {
    const float4 v = *reinterpret_cast<const float4*>(part + ((long)s * C + i) * d + j);
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  const long t = c.rows[c0 + i];
  if constexpr (ELEM == 2) {
    uint2 o;
    o.x = Bf16::pack2(acc.x, acc.y);
    o.y = Bf16::pack2(acc.z, acc.w);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(dH) + t * d + j) = o;
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(dH) + t * d + j) = acc;
  }
}

hipError_t launch_reduce_dh(const float* part, int S, int64_t C, int64_t d, Compact c, int64_t c0, void* dH,
                            int elem, hipStream_t st) {
  const long n = C * (d / 4);
  const dim3 grid((unsigned)((n + 255) / 256));
  if (elem == 2)
    hipLaunchKernelGGL(reduce_dh_kernel<2>, grid, dim3(256), 0, st, part, S, (long)C, (long)d, c, (long)c0, dH);
  else
    hipLaunchKernelGGL(reduce_dh_kernel<4>, grid, dim3(256), 0, st, part, S, (long)C, (long)d, c, (long)c0, dH);
  return hipGetLastError();
}

__global__ void zero_masked_rows_kernel(const uint8_t* mask, long T, long row16, u32x4_t* out) {
  const long q = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long t = q / row16;
  if (t >= T || mask[t] != 0) return;
  out[q] = zero4();
}

hipError_t launch_zero_masked_rows(const uint8_t* mask, int64_t T, int64_t row_bytes, void* out, hipStream_t st) {
  if (mask == nullptr || T == 0) return hipSuccess;
  const long row16 = row_bytes / 16;
  const long n = T * row16;
  const dim3 grid((unsigned)((n + 255) / 256));
  hipLaunchKernelGGL(zero_masked_rows_kernel, grid, dim3(256), 0, st, mask, (long)T, row16, (u32x4_t*)out);
  return hipGetLastError();
}

__global__ void fill_zero_kernel(u32x4_t* p, long n16) {
  for (long q = (long)blockIdx.x * blockDim.x + threadIdx.x; q < n16; q += (long)gridDim.x * blockDim.x)
    p[q] = zero4();
}

hipError_t launch_fill_zero(void* p, int64_t bytes, hipStream_t st) {
  const long n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const long blocks = min(4096L, (n16 + 255) / 256);
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (u32x4_t*)p, n16);
  return hipGetLastError();
}

}  // namespace kd
