// C-ABI entry points of libkdloss: argument checks, workspace planning and the
// launch sequence of each call.  Every argument check runs on the host before
// any HIP call, so a rejected call enqueues nothing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "kd_launch.h"
#include "kdloss.h"

namespace {

thread_local std::string g_err;

kd_status fail(kd_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

// ------------------------------------------------------------------ profiling
struct ProfEvent {
  const char* name;
  hipEvent_t a, b;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfEvent> g_prof_pending;
std::vector<std::string> g_prof_names;
std::map<std::string, std::pair<int64_t, double>> g_prof_tot;

// Set while a call that may not allocate runs on this thread: its launches
// are not bracketed by events (hipEventCreate allocates).
thread_local bool g_no_alloc = false;

// Runs one launcher; while profiling, brackets it with events on `st`.
template <class F>
hipError_t run(const char* name, hipStream_t st, F&& launch) {
  if (!g_prof_on || g_no_alloc) return launch();
  hipEvent_t a = nullptr, b = nullptr;
  if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) return launch();
  (void)hipEventRecord(a, st);
  const hipError_t e = launch();
  (void)hipEventRecord(b, st);
  std::lock_guard<std::mutex> g(g_prof_mu);
  g_prof_pending.push_back({name, a, b});
  return e;
}

void prof_fold() {
  std::lock_guard<std::mutex> g(g_prof_mu);
  for (auto& p : g_prof_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(p.b) == hipSuccess && hipEventElapsedTime(&ms, p.a, p.b) == hipSuccess) {
      auto it = g_prof_tot.find(p.name);
      if (it == g_prof_tot.end()) {
        g_prof_names.push_back(p.name);
        it = g_prof_tot.emplace(p.name, std::make_pair(int64_t(0), 0.0)).first;
      }
      it->second.first += 1;
      it->second.second += ms;
    }
    (void)hipEventDestroy(p.a);
    (void)hipEventDestroy(p.b);
  }
  g_prof_pending.clear();
}

// ------------------------------------------------------------------ shapes and checks
constexpr size_t kAlign = 256;
inline size_t up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

int elem_of(kd_dtype dt) { return dt == KD_BF16 ? 2 : 4; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

kd_status check_common(int64_t T, int64_t d, int64_t V, kd_dtype dt, float tau) {
  if (dt != KD_F32 && dt != KD_BF16) return fail(KD_ERR_INVALID_ARG, "dtype must be KD_F32 or KD_BF16");
  if (T < 0) return fail(KD_ERR_INVALID_ARG, "T must be >= 0");
  if (d < 1) return fail(KD_ERR_INVALID_ARG, "d must be >= 1");
  if (V < 1) return fail(KD_ERR_INVALID_ARG, "V must be >= 1");
  if (!(tau > 0.f) || !std::isfinite(tau)) return fail(KD_ERR_INVALID_ARG, "tau must be finite and > 0");
  const int64_t epc = dt == KD_BF16 ? 8 : 4;
  if (d % epc) return fail(KD_ERR_UNSUPPORTED, "d must be a multiple of 8 (bf16) or 4 (fp32)");
  if (V % epc) return fail(KD_ERR_UNSUPPORTED, "V must be a multiple of 8 (bf16) or 4 (fp32)");
  if (T > INT32_MAX / 2 || V > INT32_MAX / 2 || d > INT32_MAX / 2)
    return fail(KD_ERR_UNSUPPORTED, "T, d and V must be below 2^30");
  return KD_OK;
}

kd_status check_k(int64_t T, int64_t K, int64_t V, bool k_le_v = true) {
  if (K < 1) return fail(KD_ERR_INVALID_ARG, "K must be >= 1");
  if (k_le_v && K > V) return fail(KD_ERR_INVALID_ARG, "K must be <= V");
  if (K > KD_MAX_K) return fail(KD_ERR_UNSUPPORTED, "K above KD_MAX_K");
  if (T * (K + 1) >= INT32_MAX) return fail(KD_ERR_UNSUPPORTED, "T * (K + 1) must be below 2^31");
  return KD_OK;
}

kd_status need(const void* p, const char* name) {
  if (p == nullptr) return fail(KD_ERR_INVALID_ARG, std::string(name) + " is NULL");
  return KD_OK;
}

kd_status need_align(const void* p, size_t a, const char* name) {
  if (p != nullptr && !aligned(p, a))
    return fail(KD_ERR_ALIGNMENT, std::string(name) + " must be " + std::to_string(a) + "-byte aligned");
  return KD_OK;
}

#define KD_TRY(x)                   \
  do {                              \
    const kd_status _s = (x);       \
    if (_s != KD_OK) return _s;     \
  } while (0)

#define KD_LAUNCH(name, st, call)                                                              \
  do {                                                                                         \
    const hipError_t _e = run(name, st, [&]() { return (call); });                             \
    if (_e != hipSuccess) return fail(KD_ERR_HIP, std::string(name) + ": " + hipGetErrorString(_e)); \
  } while (0)

// Row blocks per raster group of the tile kernels: consecutive workgroups of
// one XCD share a row block's operand across this many row blocks (grouped_coords).
// Sweeping 1..16 at the 4096 x 3072 x 128256 head moved each kernel by under 4%.
// (dW over all its row blocks in one group ran 1% faster but fetched 60% more
// from HBM, 10.8 instead of 6.8 GB per launch.)
constexpr int kRasterGroup = 4;

// Vocabulary splits of the tile kernels: enough workgroups to fill the CUs,
// and at least 8 so that at large T the workgroups running together read
// several W panels instead of all hammering one.
// Splits of `work` units (vocabulary tiles or stage groups) for `units`
// independent tile rows, at most max_s: the tile kernels run one workgroup
// per CU, so the launch takes ceil(units * S / 256) rounds of ceil(work / S)
// units each, plus about two units per workgroup of fixed cost (ring fill,
// partials); the S with the lowest total wins, ties going to fewer splits.  A
// rule such as ceil(256 / units) overshoots 256 workgroups by a few whenever
// units does not divide 256 (15 row blocks: 270 workgroups, a second round
// for 14 of them).
int balanced_splits(int64_t units, int64_t work, int64_t max_s) {
  units = std::max<int64_t>(1, units);
  int best = 1;
  int64_t cost = INT64_MAX;
  for (int64_t s = 1; s <= std::max<int64_t>(1, std::min(max_s, work)); ++s) {
    const int64_t c = cdiv(units * s, 256) * (cdiv(work, s) + 2);
    if (c < cost) {
      cost = c;
      best = (int)s;
    }
  }
  return best;
}

int splits_for(int64_t nrb, int64_t ntiles) { return balanced_splits(nrb, ntiles, ntiles); }

// Launch shape of the tile kernels for the chunk of C rows at c0: row blocks
// of the rows it can hold (a last partial chunk gets fewer, and more splits),
// and the splits that fill the GPU with them.  S never exceeds
// max_splits(ntiles), which sizes the per-chunk partial buffers.
struct ChunkShape {
  int nrb, S;
};
ChunkShape chunk_shape(int64_t T, int64_t c0, int64_t C, int64_t ntiles) {
  const int nrb = (int)cdiv(std::min(C, T - c0), kd::kTileM);
  return {nrb, splits_for(nrb, ntiles)};
}
int64_t max_splits(int64_t ntiles) { return splits_for(1, ntiles); }

// Rows per backward chunk: the request (or the default) rounded up to whole
// 256-row tiles, at most the rows present, and for bf16 at most what keeps
// the chunk's dZ buffer within the 32-bit offsets of the direct-to-LDS loads
// that dH and dW read it with, rounded down to a multiple of the default
// chunk when that is possible (16384 rows at V = 128256: a cap of 65 row
// blocks would launch the tiles in poorly filled rounds).
int64_t chunk_of(int64_t T, int64_t V, int elem, int64_t chunk_rows) {
  int64_t C = chunk_rows <= 0 ? KD_DEFAULT_CHUNK_ROWS : chunk_rows;
  C = (int64_t)up((size_t)C, 256);
  C = std::min<int64_t>(C, (int64_t)up((size_t)std::max<int64_t>(T, 1), 256));
  if (elem == 2) {
    const int64_t ldz = cdiv(V, kd::kTileN) * kd::kTileN;
    int64_t cmax = ((int64_t(1) << 32) - 65537) / (ldz * 2) / 256 * 256;
    if (cmax >= KD_DEFAULT_CHUNK_ROWS) cmax = cmax / KD_DEFAULT_CHUNK_ROWS * KD_DEFAULT_CHUNK_ROWS;
    C = std::min<int64_t>(C, std::max<int64_t>(cmax, 256));
  }
  return C;
}

struct Carver {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t o = off;
    off = up(off + bytes, kAlign);
    return o;
  }
};

// Bytes of `rows` rows of row_bytes each in 64-byte panels (a last partial
// piece takes a whole slot).
size_t panel_bytes(int64_t rows, int64_t row_bytes) { return (size_t)rows * (size_t)cdiv(row_bytes, 64) * 64; }

// Backward chunk buffers shared by both variants.
struct ChunkPlan {
  int64_t C, ldz;
  int nrb_c, nrb_dh, ncb_dh, S_dh, nrb_dw, ncb_dw;
  size_t o_dz, o_hT, o_dhp, o_hp;  // o_hp: the chunk's rows of H in panels
};

ChunkPlan plan_chunk(int64_t T, int64_t d, int64_t V, int elem, int64_t chunk_rows, Carver& cv) {
  ChunkPlan p{};
  p.C = chunk_of(T, V, elem, chunk_rows);
  p.ldz = cdiv(V, kd::kTileN) * kd::kTileN;
  p.nrb_c = (int)(p.C / kd::kTileM);
  p.nrb_dh = p.nrb_c;
  p.ncb_dh = (int)cdiv(d, 256);
  // dH splits the vocabulary (whole groups of four 64-byte stages); at most
  // enough splits for four rounds, which bounds the fp32 partials
  const int64_t units = (int64_t)p.nrb_dh * p.ncb_dh;
  p.S_dh = balanced_splits(units, cdiv(V * elem, 256), std::max<int64_t>(1, cdiv(1024, units)));
  p.nrb_dw = (int)cdiv(d, 256);
  p.ncb_dw = (int)cdiv(V, 256);
  p.o_dz = cv.take((size_t)p.C * p.ldz * elem);
  p.o_hT = cv.take((size_t)d * p.C * elem);
  p.o_dhp = cv.take((size_t)p.S_dh * p.C * d * 4);
  p.o_hp = cv.take(panel_bytes(p.C, d * elem));
  return p;
}

struct TopkPlan {
  // the forward call: chunks of Cf rows (the default chunk size, whatever the
  // backward's), each with its own launch shape and combine, so the partials
  // hold one chunk; the chunk's rows of H in panels
  int ntiles;
  int64_t Cf;
  size_t o_pair, o_perm, o_ent, o_rowc, o_rows, o_count, o_bad, o_part, o_hp_f;
  size_t o_zpair;  // the forward's logits at the sorted entries, when z_topk is asked for
  ChunkPlan ch;
  // bytes the forward call needs without and with z_topk; bytes both calls need
  size_t fwd_total, fwd_total_z, total;
  // single-call forward + backward: per-chunk partials, the chunk's fp32
  // logits and the backward chunk buffers all live at once
  ChunkPlan ch_f;
  size_t o_part_c, o_z, o_zpair_f, fused_total;
};

TopkPlan plan_topk(int64_t T, int64_t d, int64_t V, int64_t K, int elem, int64_t chunk_rows) {
  TopkPlan p{};
  p.ntiles = (int)cdiv(V, kd::kTileN);
  p.Cf = chunk_of(T, V, elem, 0);
  Carver cv;
  // room for K + 1 entries per row: a cross-entropy label is one more
  p.o_pair = cv.take((size_t)T * (K + 1) * 8);
  p.o_perm = cv.take((size_t)T * (K + 1) * 2);
  p.o_ent = cv.take((size_t)T * 4);
  p.o_rowc = cv.take((size_t)T * 16);
  p.o_rows = cv.take((size_t)T * 4);
  p.o_count = cv.take(16);
  p.o_bad = cv.take(16);  // the index check's counter
  Carver fw = cv, bw = cv;  // forward partials and backward chunk buffers overlap
  p.o_part = fw.take((size_t)max_splits(p.ntiles) * p.Cf * 16);
  p.o_hp_f = fw.take(panel_bytes(p.Cf, d * elem));
  p.fwd_total = fw.off;
  p.o_zpair = fw.take((size_t)T * (K + 1) * 4);  // last, so the forward without z_topk needs no room for it
  p.fwd_total_z = fw.off;
  p.ch = plan_chunk(T, d, V, elem, chunk_rows, bw);
  p.total = std::max(fw.off, bw.off);
  Carver fu = cv;
  p.o_part_c = fu.take((size_t)max_splits(p.ntiles) * chunk_of(T, V, elem, chunk_rows) * 16);
  p.ch_f = plan_chunk(T, d, V, elem, chunk_rows, fu);
  p.o_z = fu.take((size_t)p.ch.C * p.ch.ldz * 4);
  p.o_zpair_f = fu.take((size_t)T * (K + 1) * 4);
  p.fused_total = fu.off;
  return p;
}

struct FullPlan {
  // the forward call as the top-K one, with the chunk's rows of both H and Ht
  // in panels; the backward and the single call add Ht's panels to their
  // chunk buffers
  int ntiles;
  int64_t Cf;
  size_t o_rows, o_count, o_part, o_hp_f, o_htp_f, o_htp_b, o_htp_u;
  ChunkPlan ch;
  size_t fwd_total, total;
  // single-call forward + backward: each head through the 256-wide top-K
  // tiles (per-chunk split partials of both, per-row constants, a dummy
  // entry list), the chunk's fp32 logits of both heads, the elementwise
  // pass's per-row terms, per-row reverse KL, and the backward chunk buffers
  int nblk;
  ChunkPlan ch_f;
  size_t o_part_s, o_part_t, o_rowc, o_pair0, o_zs, o_zt, o_terms, o_krev, fused_total;
};

FullPlan plan_full(int64_t T, int64_t d, int64_t dt, int64_t V, int elem, int64_t chunk_rows) {
  FullPlan p{};
  p.ntiles = (int)cdiv(V, kd::kTileNFull);
  p.Cf = chunk_of(T, V, elem, 0);
  Carver cv;
  p.o_rows = cv.take((size_t)T * 4);
  p.o_count = cv.take(16);
  Carver fw = cv, bw = cv;
  p.o_part = fw.take((size_t)max_splits(p.ntiles) * p.Cf * 32);
  p.o_hp_f = fw.take(panel_bytes(p.Cf, d * elem));
  p.o_htp_f = fw.take(panel_bytes(p.Cf, dt * elem));
  p.ch = plan_chunk(T, d, V, elem, chunk_rows, bw);
  p.o_htp_b = bw.take(panel_bytes(p.ch.C, dt * elem));
  p.fwd_total = fw.off;
  p.total = std::max(fw.off, bw.off);
  Carver fu = cv;
  const int64_t C = chunk_of(T, V, elem, chunk_rows);
  p.nblk = kd::full_from_z_blocks(elem, V);
  p.o_part_s = fu.take((size_t)max_splits(cdiv(V, kd::kTileN)) * C * 16);
  p.o_part_t = fu.take((size_t)max_splits(cdiv(V, kd::kTileN)) * C * 16);
  p.o_rowc = fu.take((size_t)T * 16);
  p.o_pair0 = fu.take(16);
  p.ch_f = plan_chunk(T, d, V, elem, chunk_rows, fu);
  p.o_htp_u = fu.take(panel_bytes(p.ch.C, dt * elem));
  p.o_zs = fu.take((size_t)p.ch.C * p.ch.ldz * 4);
  p.o_zt = fu.take((size_t)p.ch.C * p.ch.ldz * 4);
  p.o_terms = fu.take((size_t)C * p.nblk * 8);
  p.o_krev = fu.take((size_t)T * 4);
  p.fused_total = fu.off;
  return p;
}

template <class T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

kd_status check_workspace(const void* ws, size_t have, size_t want) {
  if (want > 0) KD_TRY(need(ws, "workspace"));
  KD_TRY(need_align(ws, kAlign, "workspace"));
  if (have < want)
    return fail(KD_ERR_WORKSPACE_TOO_SMALL,
                "workspace has " + std::to_string(have) + " bytes, needs " + std::to_string(want));
  return KD_OK;
}

// dH and dW of one backward chunk whose dZ sits in the chunk buffer:
// H^T of the chunk's rows, dH split over the vocabulary and reduced in a
// fixed order (into dH's element size dh_elem, 0 = the inputs'), dW stored
// (first chunk) or added in place.
kd_status grad_chunk(const void* H, const void* W, void* dH, float* dW, int elem, int64_t d, int64_t V,
                     const kd::Compact& c, const ChunkPlan& ch, char* dz, char* hT, float* dhp, int64_t c0,
                     bool accumulate, hipStream_t st, int dh_elem = 0) {
  KD_LAUNCH("gather_transpose", st, kd::launch_gather_transpose(H, elem, d, c, c0, ch.C, hT, st));
  if (c0 == 0 && kd::dh_direct(elem, V) && V % 128 != 0)  // the dH ring reads the chunk's columns up to ldz
    KD_LAUNCH("fill_zero", st,
              kd::launch_fill_zero(dz + kd::dz_tail_offset(ch.C, V), kd::dz_tail_bytes(ch.C, V, ch.ldz), st));
  kd::DhArgs ha{};
  ha.dz = dz;
  ha.W = static_cast<const char*>(W);
  ha.part = dhp;
  ha.count = c.count;
  ha.c0 = c0;
  ha.C = ch.C;
  ha.ldz = ch.ldz;
  ha.d = d;
  ha.V = V;
  ha.nrb = ch.nrb_dh;
  ha.ncb = ch.ncb_dh;
  ha.group = kRasterGroup;
  ha.S = ch.S_dh;
  KD_LAUNCH("dh_tile", st, kd::launch_dh(elem, ha, st));
  KD_LAUNCH("reduce_dh", st, kd::launch_reduce_dh(dhp, ch.S_dh, ch.C, d, c, c0, dH, dh_elem ? dh_elem : elem, st));
  kd::DwArgs wa{};
  wa.hT = hT;
  wa.dz = dz;
  wa.dW = dW;
  wa.count = c.count;
  wa.c0 = c0;
  wa.C = ch.C;
  wa.ldz = ch.ldz;
  wa.d = d;
  wa.V = V;
  wa.nrb = ch.nrb_dw;
  wa.ncb = ch.ncb_dw;
  wa.group = kRasterGroup;
  wa.accumulate = accumulate;
  KD_LAUNCH("dw_tile", st, kd::launch_dw(elem, wa, st));
  return KD_OK;
}

}  // namespace

// ====================================================================== C ABI
extern "C" {

const char* kd_status_string(kd_status s) {
  switch (s) {
    case KD_OK: return "KD_OK";
    case KD_ERR_INVALID_ARG: return "KD_ERR_INVALID_ARG";
    case KD_ERR_UNSUPPORTED: return "KD_ERR_UNSUPPORTED";
    case KD_ERR_ALIGNMENT: return "KD_ERR_ALIGNMENT";
    case KD_ERR_WORKSPACE_TOO_SMALL: return "KD_ERR_WORKSPACE_TOO_SMALL";
    case KD_ERR_INDEX_OUT_OF_RANGE: return "KD_ERR_INDEX_OUT_OF_RANGE";
    case KD_ERR_HIP: return "KD_ERR_HIP";
  }
  return "KD_ERR_UNKNOWN";
}

const char* kd_last_error(void) { return g_err.c_str(); }

int kd_version(void) { return 10400; }

kd_status kd_profile_enable(int on) {
  g_prof_on = on != 0;
  return KD_OK;
}

int kd_profile_count(void) {
  prof_fold();
  std::lock_guard<std::mutex> g(g_prof_mu);
  return (int)g_prof_names.size();
}

kd_status kd_profile_get(int i, const char** name, int64_t* launches, double* total_ms) {
  std::lock_guard<std::mutex> g(g_prof_mu);
  if (i < 0 || i >= (int)g_prof_names.size()) return fail(KD_ERR_INVALID_ARG, "profile index out of range");
  const auto& e = g_prof_tot[g_prof_names[i]];
  if (name) *name = g_prof_names[i].c_str();
  if (launches) *launches = e.first;
  if (total_ms) *total_ms = e.second;
  return KD_OK;
}

kd_status kd_profile_reset(void) {
  prof_fold();
  std::lock_guard<std::mutex> g(g_prof_mu);
  g_prof_names.clear();
  g_prof_tot.clear();
  return KD_OK;
}

// ---------------------------------------------------------------- top-K
}  // extern "C"

namespace {

// The options of a top-K call as the kernels take them; KE is the number of
// support entries per row (K, or K + 1 with a cross-entropy label).
struct TopkOpts {
  kd::TopkPrepOpts prep;
  int64_t KE;
  bool check;          // the index check on request
  float wr;            // weight of the reverse KL on the cached entries: r (1 - beta with a CE label)
  const float* z_in;   // the forward's z_topk, for the backward's reverse part
};

kd_status resolve_opts(const kd_topk_opts* o, float tau, int64_t K, TopkOpts& r) {
  r.prep = kd::TopkPrepOpts{};
  r.prep.c2 = (float)(1.4426950408889634 / (double)tau);
  r.prep.inv_tau = 1.0f / tau;
  r.KE = K;
  r.check = false;
  r.wr = 0.f;
  r.z_in = nullptr;
  if (o == nullptr) return KD_OK;
  r.check = o->check_indices != 0;
  if (!std::isfinite(o->ce_weight) || o->ce_weight < 0.f || o->ce_weight > 1.f)
    return fail(KD_ERR_INVALID_ARG, "ce_weight must be finite and in [0, 1]");
  if (!std::isfinite(o->rev_weight) || o->rev_weight < 0.f || o->rev_weight > 1.f)
    return fail(KD_ERR_INVALID_ARG, "rev_weight must be finite and in [0, 1]");
  if (o->ce_weight > 0.f && o->labels == nullptr) return fail(KD_ERR_INVALID_ARG, "ce_weight > 0 needs labels");
  KD_TRY(need_align(o->tau_rows, 4, "tau_rows"));
  KD_TRY(need_align(o->teacher_lse, 4, "teacher_lse"));
  KD_TRY(need_align(o->labels, 4, "labels"));
  KD_TRY(need_align(o->z_topk, 4, "opts.z_topk"));
  r.prep.tau_rows = o->tau_rows;
  r.prep.teacher_lse = o->teacher_lse;
  if (o->ce_weight > 0.f) {
    if (K + 1 > KD_MAX_K) return fail(KD_ERR_UNSUPPORTED, "a CE label needs K < KD_MAX_K");
    r.prep.labels = o->labels;
    r.prep.beta = o->ce_weight;
    r.KE = K + 1;
  }
  r.prep.rev = o->rev_weight;
  r.wr = o->rev_weight * (o->ce_weight > 0.f ? 1.f - o->ce_weight : 1.f);
  r.z_in = o->z_topk;
  return KD_OK;
}

kd_status resolve_full_opts(const kd_full_opts* o, kd::FullMix& mx) {
  mx = kd::FullMix{};
  if (o == nullptr) return KD_OK;
  if (!std::isfinite(o->rev_weight) || o->rev_weight < 0.f || o->rev_weight > 1.f)
    return fail(KD_ERR_INVALID_ARG, "rev_weight must be finite and in [0, 1]");
  KD_TRY(need_align(o->tau_rows, 4, "tau_rows"));
  mx.tau_rows = o->tau_rows;
  mx.r = o->rev_weight;
  return KD_OK;
}

// The index check on request: the counter is cleared before the prep kernel
// counts into it, and read back (one synchronisation of the stream) after.
kd_status start_index_check(TopkOpts& op, void* ws, const TopkPlan& p, int64_t V, hipStream_t st) {
  if (!op.check) return KD_OK;
  int32_t* bad = at<int32_t>(ws, p.o_bad);
  KD_LAUNCH("fill_zero", st, kd::launch_fill_zero(bad, 16, st));  // the counter's whole 16-byte region
  op.prep.bad = bad;
  op.prep.V = (int32_t)V;
  return KD_OK;
}

kd_status finish_index_check(const TopkOpts& op, hipStream_t st) {
  if (!op.check) return KD_OK;
  int32_t n = 0;
  hipError_t e = hipMemcpyAsync(&n, op.prep.bad, sizeof n, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(KD_ERR_HIP, std::string("index check: ") + hipGetErrorString(e));
  if (n > 0)
    return fail(KD_ERR_INDEX_OUT_OF_RANGE,
                std::to_string(n) + " cached indices or labels of valid rows lie outside [0, V)");
  return KD_OK;
}

// The per-row data of the prep; with a zpair offset, also the array in
// which the forward's gather leaves the logits of the sorted entries for
// z_topk.
kd::TopkRowData row_data(void* ws, const TopkPlan& p, const size_t* o_zpair = nullptr) {
  return kd::TopkRowData{at<int2>(ws, p.o_pair), at<uint16_t>(ws, p.o_perm), at<float>(ws, p.o_ent),
                         at<float4>(ws, p.o_rowc), o_zpair ? at<float>(ws, *o_zpair) : nullptr};
}

// A vocabulary shard of the head: W holds its columns [v0, v0 + V).  The
// forward then writes each row's record (rec [T,4]) and teacher terms
// (trow [T,2]) in place of kl and lse; the backward takes the whole head's
// lse and writes an fp32 partial of dH.
struct Shard {
  int64_t v0;
  float* rec;
  float* trow;
};

kd_status check_shard(int64_t T, int64_t K, int64_t V, int64_t v0, const kd_topk_opts* o = nullptr) {
  KD_TRY(check_k(T, K, V, false));
  if (o != nullptr && o->check_indices != 0)
    return fail(KD_ERR_UNSUPPORTED, "check_indices: a shard does not know the whole head's width");
  if (o != nullptr && o->rev_weight != 0.f)
    return fail(KD_ERR_UNSUPPORTED, "rev_weight: the reverse KL needs the student's logits at all K entries, "
                                    "which no one shard holds");
  if (v0 < 0) return fail(KD_ERR_INVALID_ARG, "v0 must be >= 0");
  if (v0 + V > INT32_MAX / 2) return fail(KD_ERR_UNSUPPORTED, "v0 + V must be below 2^30");
  return KD_OK;
}

}  // namespace

extern "C" {

kd_status kd_topk_kl_workspace_size(int64_t T, int64_t d, int64_t V, int64_t K, kd_dtype dt, int64_t chunk_rows,
                                    size_t* bytes) {
  g_err.clear();
  KD_TRY(need(bytes, "bytes"));
  KD_TRY(check_common(T, d, V, dt, 1.0f));
  KD_TRY(check_k(T, K, V));
  *bytes = T == 0 ? 0 : plan_topk(T, d, V, K, elem_of(dt), chunk_rows).total;
  return KD_OK;
}

kd_status kd_topk_kl_fwd(const void* H, const void* W, const int32_t* topk_idx, const float* topk_logits,
                         const uint8_t* mask, float tau, int64_t T, int64_t d, int64_t V, int64_t K, kd_dtype dt,
                         float* kl, float* lse, float* z_topk, void* workspace, size_t workspace_bytes,
                         void* stream) {
  return kd_topk_kl_fwd_ex(H, W, topk_idx, topk_logits, mask, tau, nullptr, T, d, V, K, dt, kl, lse, z_topk,
                           workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// The top-K forward; with a shard, the row records replace kl and lse.
kd_status topk_fwd(const void* H, const void* W, const int32_t* topk_idx, const float* topk_logits,
                   const uint8_t* mask, float tau, const kd_topk_opts* opts, int64_t T, int64_t d, int64_t V,
                   int64_t K, kd_dtype dt, float* kl, float* lse, float* z_topk, const Shard* shard, void* workspace,
                   size_t workspace_bytes, void* stream) {
  g_err.clear();
  KD_TRY(check_common(T, d, V, dt, tau));
  KD_TRY(shard ? check_shard(T, K, V, shard->v0, opts) : check_k(T, K, V));
  TopkOpts op;
  KD_TRY(resolve_opts(opts, tau, K, op));
  if (shard) {
    op.prep.v0 = (int32_t)shard->v0;
    op.prep.vs = (int32_t)V;
  }
  if (T == 0) return KD_OK;
  KD_TRY(need(H, "H"));
  KD_TRY(need(W, "W"));
  KD_TRY(need(topk_idx, "topk_idx"));
  KD_TRY(need(topk_logits, "topk_logits"));
  if (shard) {
    KD_TRY(need(shard->rec, "rec"));
    KD_TRY(need(shard->trow, "trow"));
    KD_TRY(need_align(shard->rec, 16, "rec"));
    KD_TRY(need_align(shard->trow, 8, "trow"));
  } else {
    KD_TRY(need(kl, "kl"));
    KD_TRY(need(lse, "lse"));
    KD_TRY(need_align(kl, 4, "kl"));
    KD_TRY(need_align(lse, 4, "lse"));
  }
  KD_TRY(need_align(H, 16, "H"));
  KD_TRY(need_align(W, 16, "W"));
  KD_TRY(need_align(topk_idx, 4, "topk_idx"));
  KD_TRY(need_align(topk_logits, 4, "topk_logits"));
  KD_TRY(need_align(z_topk, 4, "z_topk"));
  if (op.prep.rev > 0.f) KD_TRY(need(z_topk, "z_topk (rev_weight > 0 reads it)"));
  const int elem = elem_of(dt);
  const TopkPlan p = plan_topk(T, d, V, K, elem, 0);
  KD_TRY(check_workspace(workspace, workspace_bytes, z_topk ? p.fwd_total_z : p.fwd_total));

  hipStream_t st = static_cast<hipStream_t>(stream);
  kd::Compact c{at<int32_t>(workspace, p.o_rows), at<int32_t>(workspace, p.o_count)};
  const kd::TopkRowData rd = row_data(workspace, p, z_topk ? &p.o_zpair : nullptr);
  float* part = at<float>(workspace, p.o_part);

  KD_LAUNCH("compact", st, kd::launch_compact(mask, T, c, st));
  KD_TRY(start_index_check(op, workspace, p, V, st));
  KD_LAUNCH("topk_prep", st, kd::launch_topk_prep(topk_logits, topk_idx, mask, T, K, op.KE, op.prep, rd, z_topk, st));
  KD_TRY(finish_index_check(op, st));
  char* hp = at<char>(workspace, p.o_hp_f);
  kd::TopkFwdArgs a{};
  a.Hp = hp;
  a.W = static_cast<const char*>(W);
  a.c = c;
  a.rd = rd;
  a.z_topk = z_topk;
  a.part = part;
  a.part_stride = p.Cf;
  a.C = p.Cf;
  a.T = T;
  a.d = d;
  a.V = V;
  a.K = op.KE;
  a.Kz = K;
  a.ntiles = p.ntiles;
  a.group = kRasterGroup;
  for (int64_t c0 = 0; c0 < T; c0 += p.Cf) {
    const ChunkShape sh = chunk_shape(T, c0, p.Cf, p.ntiles);
    KD_LAUNCH("gather_panels", st, kd::launch_gather_panels(H, d * elem, c, c0, p.Cf, hp, st));
    a.c0 = a.part_row0 = c0;
    a.nrb = sh.nrb;
    a.S = sh.S;
    KD_LAUNCH("topk_fwd_tile", st, kd::launch_topk_fwd(elem, a, st));
    if (z_topk)
      KD_LAUNCH("topk_zpermute", st, kd::launch_topk_zpermute(rd, c, T, op.KE, K, z_topk, c0, c0 + p.Cf, st));
    if (shard)
      KD_LAUNCH("topk_shard_record", st,
                kd::launch_topk_shard_record(part, sh.S, p.Cf, c, mask, rd, T, reinterpret_cast<float4*>(shard->rec),
                                             reinterpret_cast<float2*>(shard->trow), c0, c0 + p.Cf, c0 == 0, st));
    else
      KD_LAUNCH("topk_combine", st,
                kd::launch_topk_combine(part, sh.S, p.Cf, c, mask, rd, T, kl, lse, c0, c0 + p.Cf, c0 == 0, st));
    if (op.prep.rev > 0.f)
      KD_LAUNCH("topk_reverse", st,
                kd::launch_topk_reverse(z_topk, topk_logits, c, T, K, op.KE, op.wr, rd, kl, false, c0, c0 + p.Cf,
                                        st));
  }
  return KD_OK;
}

}  // namespace

extern "C" {

kd_status kd_topk_kl_fwd_ex(const void* H, const void* W, const int32_t* topk_idx, const float* topk_logits,
                            const uint8_t* mask, float tau, const kd_topk_opts* opts, int64_t T, int64_t d,
                            int64_t V, int64_t K, kd_dtype dt, float* kl, float* lse, float* z_topk,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return topk_fwd(H, W, topk_idx, topk_logits, mask, tau, opts, T, d, V, K, dt, kl, lse, z_topk, nullptr, workspace,
                  workspace_bytes, stream);
}

}  // extern "C"

namespace {

// ---------------------------------------------------------------- the forward's fixed scratch
// The scratch of kd_topk_kl_fwd_noalloc: one array per GPU, loaded with the
// library's code object.  Host code never uses its name as an address (on
// the host it is only a stand-in); the device address comes from
// hipGetSymbolAddress, read once per device with that device current, and is
// what the kernels get.
static __device__ __align__(256) char scratch[KD_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_ptr;  // device ordinal -> the array's device address there

kd_status scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(KD_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  std::lock_guard<std::mutex> g(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it == g_scratch_ptr.end()) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return fail(KD_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    it = g_scratch_ptr.emplace(dev, ptr).first;
  }
  *out = it->second;
  return KD_OK;
}

}  // namespace

extern "C" {

kd_status kd_topk_kl_fwd_noalloc(const void* H, const void* W, const int32_t* topk_idx, const float* topk_logits,
                                 const uint8_t* mask, float tau, int64_t T, int64_t d, int64_t V, int64_t K,
                                 kd_dtype dt, float* kl, float* lse, float* z_topk, void* stream) {
  g_err.clear();
  KD_TRY(check_common(T, d, V, dt, tau));
  KD_TRY(check_k(T, K, V));
  if (T == 0) return KD_OK;
  const TopkPlan plan = plan_topk(T, d, V, K, elem_of(dt), 0);
  const size_t want = z_topk ? plan.fwd_total_z : plan.fwd_total;
  if (want > KD_NOALLOC_SCRATCH_BYTES)
    return fail(KD_ERR_UNSUPPORTED, "this forward needs " + std::to_string(want) +
                                        " bytes of scratch, above KD_NOALLOC_SCRATCH_BYTES (" +
                                        std::to_string((size_t)KD_NOALLOC_SCRATCH_BYTES) +
                                        "); use kd_topk_kl_fwd with a workspace");
  void* ptr = nullptr;
  KD_TRY(scratch_on_current_device(&ptr));
  g_no_alloc = true;
  const kd_status s = topk_fwd(H, W, topk_idx, topk_logits, mask, tau, nullptr, T, d, V, K, dt, kl, lse, z_topk,
                               nullptr, ptr, KD_NOALLOC_SCRATCH_BYTES, stream);
  g_no_alloc = false;
  return s;
}

kd_status kd_topk_kl_bwd(const void* H, const void* W, const int32_t* topk_idx, const float* topk_logits,
                         const uint8_t* mask, float tau, int64_t T, int64_t d, int64_t V, int64_t K, kd_dtype dt,
                         const float* lse, const float* grad_kl, void* dH, float* dW, int64_t chunk_rows,
                         void* workspace, size_t workspace_bytes, void* stream) {
  return kd_topk_kl_bwd_ex(H, W, topk_idx, topk_logits, mask, tau, nullptr, T, d, V, K, dt, lse, grad_kl, dH, dW,
                           chunk_rows, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// The top-K backward; with a shard (v0 used), dH is an fp32 partial.
kd_status topk_bwd(const void* H, const void* W, const int32_t* topk_idx, const float* topk_logits,
                   const uint8_t* mask, float tau, const kd_topk_opts* opts, int64_t T, int64_t d, int64_t V,
                   int64_t K, kd_dtype dt, const float* lse, const float* grad_kl, void* dH, float* dW,
                   int64_t chunk_rows, const Shard* shard, void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  KD_TRY(check_common(T, d, V, dt, tau));
  KD_TRY(shard ? check_shard(T, K, V, shard->v0, opts) : check_k(T, K, V));
  TopkOpts op;
  KD_TRY(resolve_opts(opts, tau, K, op));
  if (shard) {
    op.prep.v0 = (int32_t)shard->v0;
    op.prep.vs = (int32_t)V;
  }
  KD_TRY(need(dW, "dW"));
  KD_TRY(need_align(dW, 16, "dW"));
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (T == 0) {
    KD_LAUNCH("fill_zero", st, kd::launch_fill_zero(dW, d * V * 4, st));
    return KD_OK;
  }
  KD_TRY(need(H, "H"));
  KD_TRY(need(W, "W"));
  KD_TRY(need(topk_idx, "topk_idx"));
  KD_TRY(need(topk_logits, "topk_logits"));
  KD_TRY(need(lse, "lse"));
  KD_TRY(need(grad_kl, "grad_kl"));
  KD_TRY(need(dH, "dH"));
  KD_TRY(need_align(H, 16, "H"));
  KD_TRY(need_align(W, 16, "W"));
  KD_TRY(need_align(dH, 16, "dH"));
  KD_TRY(need_align(topk_idx, 4, "topk_idx"));
  KD_TRY(need_align(topk_logits, 4, "topk_logits"));
  KD_TRY(need_align(lse, 4, "lse"));
  KD_TRY(need_align(grad_kl, 4, "grad_kl"));
  if (chunk_rows < 0) return fail(KD_ERR_INVALID_ARG, "chunk_rows must be >= 0");
  if (op.prep.rev > 0.f) KD_TRY(need(op.z_in, "opts.z_topk (rev_weight > 0 reads it)"));
  const int elem = elem_of(dt);
  const TopkPlan p = plan_topk(T, d, V, K, elem, chunk_rows);
  KD_TRY(check_workspace(workspace, workspace_bytes, p.total));

  kd::Compact c{at<int32_t>(workspace, p.o_rows), at<int32_t>(workspace, p.o_count)};
  const kd::TopkRowData rd = row_data(workspace, p);
  KD_LAUNCH("compact", st, kd::launch_compact(mask, T, c, st));
  KD_TRY(start_index_check(op, workspace, p, V, st));
  KD_LAUNCH("topk_prep", st, kd::launch_topk_prep(topk_logits, topk_idx, mask, T, K, op.KE, op.prep, rd, nullptr, st));
  KD_TRY(finish_index_check(op, st));
  if (op.prep.rev > 0.f)  // the reverse part's gradient folded into the support weights
    KD_LAUNCH("topk_reverse", st,
              kd::launch_topk_reverse(op.z_in, topk_logits, c, T, K, op.KE, op.wr, rd, nullptr, true, 0, T, st));
  const int dh_elem = shard ? 4 : elem;
  KD_LAUNCH("zero_masked_rows", st, kd::launch_zero_masked_rows(mask, T, d * dh_elem, dH, st));

  const ChunkPlan& ch = p.ch;
  char* dz = at<char>(workspace, ch.o_dz);
  char* hT = at<char>(workspace, ch.o_hT);
  float* dhp = at<float>(workspace, ch.o_dhp);
  const int64_t nchunks = cdiv(T, ch.C);
  for (int64_t k = 0; k < nchunks; ++k) {
    const int64_t c0 = k * ch.C;
    char* hp = at<char>(workspace, ch.o_hp);
    KD_LAUNCH("gather_panels", st, kd::launch_gather_panels(H, d * elem, c, c0, ch.C, hp, st));
    kd::TopkDzArgs za{};
    za.Hp = hp;
    za.W = static_cast<const char*>(W);
    za.c = c;
    za.rd = rd;
    za.lse = lse;
    za.g = grad_kl;
    za.dz = dz;
    za.ldz = ch.ldz;
    za.c0 = c0;
    za.C = ch.C;
    za.T = T;
    za.d = d;
    za.V = V;
    za.K = op.KE;
    const ChunkShape sh = chunk_shape(T, c0, ch.C, p.ntiles);
    za.nrb = sh.nrb;
    za.ntiles = p.ntiles;
    za.group = kRasterGroup;
    za.S = sh.S;
    KD_LAUNCH("topk_dz_tile", st, kd::launch_topk_dz(elem, za, st));
    KD_TRY(grad_chunk(H, W, dH, dW, elem, d, V, c, ch, dz, hT, dhp, c0, k > 0, st, dh_elem));
  }
  return KD_OK;
}

}  // namespace

extern "C" {

kd_status kd_topk_kl_bwd_ex(const void* H, const void* W, const int32_t* topk_idx, const float* topk_logits,
                            const uint8_t* mask, float tau, const kd_topk_opts* opts, int64_t T, int64_t d,
                            int64_t V, int64_t K, kd_dtype dt, const float* lse, const float* grad_kl, void* dH,
                            float* dW, int64_t chunk_rows, void* workspace, size_t workspace_bytes, void* stream) {
  return topk_bwd(H, W, topk_idx, topk_logits, mask, tau, opts, T, d, V, K, dt, lse, grad_kl, dH, dW, chunk_rows,
                  nullptr, workspace, workspace_bytes, stream);
}

// ---------------------------------------------------------------- top-K, one vocabulary shard
kd_status kd_topk_kl_shard_workspace_size(int64_t T, int64_t d, int64_t V, int64_t v0, int64_t K, kd_dtype dt,
                                          int64_t chunk_rows, size_t* bytes) {
  g_err.clear();
  KD_TRY(need(bytes, "bytes"));
  KD_TRY(check_common(T, d, V, dt, 1.0f));
  KD_TRY(check_shard(T, K, V, v0));
  *bytes = T == 0 ? 0 : plan_topk(T, d, V, K, elem_of(dt), chunk_rows).total;
  return KD_OK;
}

kd_status kd_topk_kl_fwd_shard(const void* H, const void* W, const int32_t* topk_idx, const float* topk_logits,
                               const uint8_t* mask, float tau, const kd_topk_opts* opts, int64_t T, int64_t d,
                               int64_t V, int64_t v0, int64_t K, kd_dtype dt, float* rec, float* trow,
                               float* z_topk, void* workspace, size_t workspace_bytes, void* stream) {
  const Shard sh{v0, rec, trow};
  return topk_fwd(H, W, topk_idx, topk_logits, mask, tau, opts, T, d, V, K, dt, nullptr, nullptr, z_topk, &sh,
                  workspace, workspace_bytes, stream);
}

kd_status kd_topk_kl_shard_combine(const float* rec, int64_t R, const float* trow, const uint8_t* mask, int64_t T,
                                   float* kl, float* lse, void* stream) {
  g_err.clear();
  if (T < 0) return fail(KD_ERR_INVALID_ARG, "T must be >= 0");
  if (R < 1) return fail(KD_ERR_INVALID_ARG, "R must be >= 1");
  if (T > INT32_MAX / 2 || R * T > INT32_MAX) return fail(KD_ERR_UNSUPPORTED, "R * T must be below 2^31");
  if (T == 0) return KD_OK;
  KD_TRY(need(rec, "rec"));
  KD_TRY(need(trow, "trow"));
  KD_TRY(need(kl, "kl"));
  KD_TRY(need(lse, "lse"));
  KD_TRY(need_align(rec, 16, "rec"));
  KD_TRY(need_align(trow, 8, "trow"));
  KD_TRY(need_align(kl, 4, "kl"));
  KD_TRY(need_align(lse, 4, "lse"));
  hipStream_t st = static_cast<hipStream_t>(stream);
  KD_LAUNCH("topk_shard_combine", st,
            kd::launch_topk_shard_combine(reinterpret_cast<const float4*>(rec), (int)R, T,
                                          reinterpret_cast<const float2*>(trow), mask, kl, lse, st));
  return KD_OK;
}

kd_status kd_topk_kl_bwd_shard(const void* H, const void* W, const int32_t* topk_idx, const float* topk_logits,
                               const uint8_t* mask, float tau, const kd_topk_opts* opts, int64_t T, int64_t d,
                               int64_t V, int64_t v0, int64_t K, kd_dtype dt, const float* lse, const float* grad_kl,
                               float* dH, float* dW, int64_t chunk_rows, void* workspace, size_t workspace_bytes,
                               void* stream) {
  const Shard sh{v0, nullptr, nullptr};
  return topk_bwd(H, W, topk_idx, topk_logits, mask, tau, opts, T, d, V, K, dt, lse, grad_kl, dH, dW, chunk_rows,
                  &sh, workspace, workspace_bytes, stream);
}


// ---------------------------------------------------------------- full vocabulary
kd_status kd_full_kl_workspace_size(int64_t T, int64_t d, int64_t dt_hidden, int64_t V, kd_dtype dt,
                                    int64_t chunk_rows, size_t* bytes) {
  g_err.clear();
  KD_TRY(need(bytes, "bytes"));
  KD_TRY(check_common(T, d, V, dt, 1.0f));
  KD_TRY(check_common(T, dt_hidden, V, dt, 1.0f));
  *bytes = T == 0 ? 0 : plan_full(T, d, dt_hidden, V, elem_of(dt), chunk_rows).total;
  return KD_OK;
}

kd_status kd_full_kl_fwd(const void* H, const void* Ws, const void* Ht, const void* Wt, const uint8_t* mask, float tau,
                         int64_t T, int64_t d, int64_t dt_hidden, int64_t V, kd_dtype dt, float* kl, float* lse_s,
                         float* lse_t, void* workspace, size_t workspace_bytes, void* stream) {
  return kd_full_kl_fwd_ex(H, Ws, Ht, Wt, mask, tau, nullptr, T, d, dt_hidden, V, dt, kl, lse_s, lse_t, nullptr,
                           workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// The full-vocabulary forward; with rec (a vocabulary shard's record [T,8])
// the merged partials replace kl and the log-normalisers.
kd_status full_fwd(const void* H, const void* Ws, const void* Ht, const void* Wt, const uint8_t* mask, float tau,
                   const kd_full_opts* opts, int64_t T, int64_t d, int64_t dt_hidden, int64_t V, kd_dtype dt,
                   float* kl, float* lse_s, float* lse_t, float* kl_rev, float* rec, void* workspace,
                   size_t workspace_bytes, void* stream) {
  g_err.clear();
  KD_TRY(check_common(T, d, V, dt, tau));
  KD_TRY(check_common(T, dt_hidden, V, dt, tau));
  kd::FullMix mx;
  KD_TRY(resolve_full_opts(opts, mx));
  KD_TRY(need_align(kl_rev, 4, "kl_rev"));
  if (T == 0) return KD_OK;
  KD_TRY(need(H, "H"));
  KD_TRY(need(Ws, "Ws"));
  KD_TRY(need(Ht, "Ht"));
  KD_TRY(need(Wt, "Wt"));
  if (rec) {
    KD_TRY(need_align(rec, 16, "rec"));
  } else {
    KD_TRY(need(kl, "kl"));
    KD_TRY(need(lse_s, "lse_s"));
    KD_TRY(need(lse_t, "lse_t"));
    KD_TRY(need_align(kl, 4, "kl"));
    KD_TRY(need_align(lse_s, 4, "lse_s"));
    KD_TRY(need_align(lse_t, 4, "lse_t"));
  }
  KD_TRY(need_align(H, 16, "H"));
  KD_TRY(need_align(Ws, 16, "Ws"));
  KD_TRY(need_align(Ht, 16, "Ht"));
  KD_TRY(need_align(Wt, 16, "Wt"));
  const int elem = elem_of(dt);
  const FullPlan p = plan_full(T, d, dt_hidden, V, elem, 0);
  KD_TRY(check_workspace(workspace, workspace_bytes, p.fwd_total));

  hipStream_t st = static_cast<hipStream_t>(stream);
  kd::Compact c{at<int32_t>(workspace, p.o_rows), at<int32_t>(workspace, p.o_count)};
  float* part = at<float>(workspace, p.o_part);
  KD_LAUNCH("compact", st, kd::launch_compact(mask, T, c, st));
  char* hp = at<char>(workspace, p.o_hp_f);
  char* htp = at<char>(workspace, p.o_htp_f);
  kd::FullFwdArgs a{};
  a.Hp = hp;
  a.Ws = static_cast<const char*>(Ws);
  a.Htp = htp;
  a.Wt = static_cast<const char*>(Wt);
  a.c = c;
  a.part = part;
  a.part_stride = p.Cf;
  a.C = p.Cf;
  a.T = T;
  a.d = d;
  a.dt = dt_hidden;
  a.V = V;
  a.ntiles = p.ntiles;
  a.group = kRasterGroup;
  a.c2 = (float)(1.4426950408889634 / (double)tau);
  a.tau_rows = mx.tau_rows;
  for (int64_t c0 = 0; c0 < T; c0 += p.Cf) {
    const ChunkShape sh = chunk_shape(T, c0, p.Cf, p.ntiles);
    KD_LAUNCH("gather_panels", st, kd::launch_gather_panels(H, d * elem, c, c0, p.Cf, hp, st));
    KD_LAUNCH("gather_panels", st, kd::launch_gather_panels(Ht, dt_hidden * elem, c, c0, p.Cf, htp, st));
    a.c0 = a.part_row0 = c0;
    a.nrb = sh.nrb;
    a.S = sh.S;
    KD_LAUNCH("full_fwd_tile", st, kd::launch_full_fwd(elem, a, st));
    if (rec)
      KD_LAUNCH("full_shard_record", st,
                kd::launch_full_shard_record(part, sh.S, p.Cf, c, mask, T, reinterpret_cast<float4*>(rec), c0,
                                             c0 + p.Cf, c0 == 0, st));
    else
      KD_LAUNCH("full_combine", st,
                kd::launch_full_combine(part, sh.S, p.Cf, c, mask, T, mx.r, kl, lse_s, lse_t, kl_rev, c0, c0 + p.Cf,
                                        c0 == 0, st));
  }
  return KD_OK;
}

}  // namespace

extern "C" {

kd_status kd_full_kl_fwd_ex(const void* H, const void* Ws, const void* Ht, const void* Wt, const uint8_t* mask,
                            float tau, const kd_full_opts* opts, int64_t T, int64_t d, int64_t dt_hidden, int64_t V,
                            kd_dtype dt, float* kl, float* lse_s, float* lse_t, float* kl_rev, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return full_fwd(H, Ws, Ht, Wt, mask, tau, opts, T, d, dt_hidden, V, dt, kl, lse_s, lse_t, kl_rev, nullptr,
                  workspace, workspace_bytes, stream);
}

kd_status kd_full_kl_bwd(const void* H, const void* Ws, const void* Ht, const void* Wt, const uint8_t* mask, float tau,
                         int64_t T, int64_t d, int64_t dt_hidden, int64_t V, kd_dtype dt, const float* lse_s,
                         const float* lse_t, const float* grad_kl, void* dH, float* dWs, int64_t chunk_rows,
                         void* workspace, size_t workspace_bytes, void* stream) {
  return kd_full_kl_bwd_ex(H, Ws, Ht, Wt, mask, tau, nullptr, T, d, dt_hidden, V, dt, lse_s, lse_t, nullptr, grad_kl,
                           dH, dWs, chunk_rows, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// The full-vocabulary backward; dh_elem 4 gives an fp32 dH (a shard's partial).
kd_status full_bwd(const void* H, const void* Ws, const void* Ht, const void* Wt, const uint8_t* mask, float tau,
                   const kd_full_opts* opts, int64_t T, int64_t d, int64_t dt_hidden, int64_t V, kd_dtype dt,
                   const float* lse_s, const float* lse_t, const float* kl_rev, const float* grad_kl, void* dH,
                   float* dWs, int64_t chunk_rows, int dh_elem, void* workspace, size_t workspace_bytes,
                   void* stream) {
  g_err.clear();
  KD_TRY(check_common(T, d, V, dt, tau));
  KD_TRY(check_common(T, dt_hidden, V, dt, tau));
  kd::FullMix mx;
  KD_TRY(resolve_full_opts(opts, mx));
  KD_TRY(need_align(kl_rev, 4, "kl_rev"));
  mx.kl_rev = kl_rev;
  KD_TRY(need(dWs, "dWs"));
  KD_TRY(need_align(dWs, 16, "dWs"));
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (T == 0) {
    KD_LAUNCH("fill_zero", st, kd::launch_fill_zero(dWs, d * V * 4, st));
    return KD_OK;
  }
  KD_TRY(need(H, "H"));
  KD_TRY(need(Ws, "Ws"));
  KD_TRY(need(Ht, "Ht"));
  KD_TRY(need(Wt, "Wt"));
  KD_TRY(need(lse_s, "lse_s"));
  KD_TRY(need(lse_t, "lse_t"));
  KD_TRY(need(grad_kl, "grad_kl"));
  KD_TRY(need(dH, "dH"));
  if (mx.r != 0.f) KD_TRY(need(kl_rev, "kl_rev (rev_weight > 0)"));
  KD_TRY(need_align(H, 16, "H"));
  KD_TRY(need_align(Ws, 16, "Ws"));
  KD_TRY(need_align(Ht, 16, "Ht"));
  KD_TRY(need_align(Wt, 16, "Wt"));
  KD_TRY(need_align(dH, 16, "dH"));
  KD_TRY(need_align(lse_s, 4, "lse_s"));
  KD_TRY(need_align(lse_t, 4, "lse_t"));
  KD_TRY(need_align(grad_kl, 4, "grad_kl"));
  if (chunk_rows < 0) return fail(KD_ERR_INVALID_ARG, "chunk_rows must be >= 0");
  const int elem = elem_of(dt);
  const FullPlan p = plan_full(T, d, dt_hidden, V, elem, chunk_rows);
  KD_TRY(check_workspace(workspace, workspace_bytes, p.total));

  kd::Compact c{at<int32_t>(workspace, p.o_rows), at<int32_t>(workspace, p.o_count)};
  KD_LAUNCH("compact", st, kd::launch_compact(mask, T, c, st));
  if (dh_elem == 0) dh_elem = elem;
  KD_LAUNCH("zero_masked_rows", st, kd::launch_zero_masked_rows(mask, T, d * dh_elem, dH, st));

  const ChunkPlan& ch = p.ch;
  char* dz = at<char>(workspace, ch.o_dz);
  char* hT = at<char>(workspace, ch.o_hT);
  float* dhp = at<float>(workspace, ch.o_dhp);
  const int64_t nchunks = cdiv(T, ch.C);
  for (int64_t k = 0; k < nchunks; ++k) {
    const int64_t c0 = k * ch.C;
    char* hp = at<char>(workspace, ch.o_hp);
    char* htp = at<char>(workspace, p.o_htp_b);
    KD_LAUNCH("gather_panels", st, kd::launch_gather_panels(H, d * elem, c, c0, ch.C, hp, st));
    KD_LAUNCH("gather_panels", st, kd::launch_gather_panels(Ht, dt_hidden * elem, c, c0, ch.C, htp, st));
    kd::FullDzArgs za{};
    za.Hp = hp;
    za.Ws = static_cast<const char*>(Ws);
    za.Htp = htp;
    za.Wt = static_cast<const char*>(Wt);
    za.c = c;
    za.lse_s = lse_s;
    za.lse_t = lse_t;
    za.g = grad_kl;
    za.dz = dz;
    za.ldz = ch.ldz;
    za.c0 = c0;
    za.C = ch.C;
    za.T = T;
    za.d = d;
    za.dt = dt_hidden;
    za.V = V;
    const ChunkShape sh = chunk_shape(T, c0, ch.C, p.ntiles);
    za.nrb = sh.nrb;
    za.ntiles = p.ntiles;
    za.group = kRasterGroup;
    za.S = sh.S;
    za.c2 = (float)(1.4426950408889634 / (double)tau);
    za.inv_tau = 1.0f / tau;
    za.mix = mx;
    KD_LAUNCH("full_dz_tile", st, kd::launch_full_dz(elem, za, st));
    KD_TRY(grad_chunk(H, Ws, dH, dWs, elem, d, V, c, ch, dz, hT, dhp, c0, k > 0, st, dh_elem));
  }
  return KD_OK;
}

}  // namespace

extern "C" {

kd_status kd_full_kl_bwd_ex(const void* H, const void* Ws, const void* Ht, const void* Wt, const uint8_t* mask,
                            float tau, const kd_full_opts* opts, int64_t T, int64_t d, int64_t dt_hidden, int64_t V,
                            kd_dtype dt, const float* lse_s, const float* lse_t, const float* kl_rev,
                            const float* grad_kl, void* dH, float* dWs, int64_t chunk_rows, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return full_bwd(H, Ws, Ht, Wt, mask, tau, opts, T, d, dt_hidden, V, dt, lse_s, lse_t, kl_rev, grad_kl, dH, dWs,
                  chunk_rows, 0, workspace, workspace_bytes, stream);
}

// ---------------------------------------------------------------- full vocabulary, one vocabulary shard
kd_status kd_full_kl_fwd_shard(const void* H, const void* Ws, const void* Ht, const void* Wt, const uint8_t* mask,
                               float tau, const kd_full_opts* opts, int64_t T, int64_t d, int64_t dt_hidden,
                               int64_t V, kd_dtype dt, float* rec, void* workspace, size_t workspace_bytes,
                               void* stream) {
  if (T > 0 && rec == nullptr) {
    g_err.clear();
    return fail(KD_ERR_INVALID_ARG, "rec is NULL");
  }
  return full_fwd(H, Ws, Ht, Wt, mask, tau, opts, T, d, dt_hidden, V, dt, nullptr, nullptr, nullptr, nullptr, rec,
                  workspace, workspace_bytes, stream);
}

kd_status kd_full_kl_shard_combine(const float* rec, int64_t R, const uint8_t* mask, int64_t T, float rev_weight,
                                   float* kl, float* lse_s, float* lse_t, float* kl_rev, void* stream) {
  g_err.clear();
  if (T < 0) return fail(KD_ERR_INVALID_ARG, "T must be >= 0");
  if (R < 1) return fail(KD_ERR_INVALID_ARG, "R must be >= 1");
  if (!std::isfinite(rev_weight) || rev_weight < 0.f || rev_weight > 1.f)
    return fail(KD_ERR_INVALID_ARG, "rev_weight must be finite and in [0, 1]");
  if (T > INT32_MAX / 2 || R * T > INT32_MAX / 2) return fail(KD_ERR_UNSUPPORTED, "R * T must be below 2^30");
  if (T == 0) return KD_OK;
  KD_TRY(need(rec, "rec"));
  KD_TRY(need(kl, "kl"));
  KD_TRY(need(lse_s, "lse_s"));
  KD_TRY(need(lse_t, "lse_t"));
  KD_TRY(need_align(rec, 16, "rec"));
  KD_TRY(need_align(kl, 4, "kl"));
  KD_TRY(need_align(lse_s, 4, "lse_s"));
  KD_TRY(need_align(lse_t, 4, "lse_t"));
  KD_TRY(need_align(kl_rev, 4, "kl_rev"));
  hipStream_t st = static_cast<hipStream_t>(stream);
  KD_LAUNCH("full_shard_combine", st,
            kd::launch_full_shard_combine(reinterpret_cast<const float4*>(rec), (int)R, T, mask, rev_weight, kl,
                                          lse_s, lse_t, kl_rev, st));
  return KD_OK;
}

kd_status kd_full_kl_bwd_shard(const void* H, const void* Ws, const void* Ht, const void* Wt, const uint8_t* mask,
                               float tau, const kd_full_opts* opts, int64_t T, int64_t d, int64_t dt_hidden,
                               int64_t V, kd_dtype dt, const float* lse_s, const float* lse_t, const float* kl_rev,
                               const float* grad_kl, float* dH, float* dWs, int64_t chunk_rows, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return full_bwd(H, Ws, Ht, Wt, mask, tau, opts, T, d, dt_hidden, V, dt, lse_s, lse_t, kl_rev, grad_kl, dH, dWs,
                  chunk_rows, 4, workspace, workspace_bytes, stream);
}


// ---------------------------------------------------------------- full vocabulary, forward and backward in one call
kd_status kd_full_kl_fwd_bwd_workspace_size(int64_t T, int64_t d, int64_t dt_hidden, int64_t V, kd_dtype dt,
                                            int64_t chunk_rows, size_t* bytes) {
  g_err.clear();
  KD_TRY(need(bytes, "bytes"));
  KD_TRY(check_common(T, d, V, dt, 1.0f));
  KD_TRY(check_common(T, dt_hidden, V, dt, 1.0f));
  if (chunk_rows < 0) return fail(KD_ERR_INVALID_ARG, "chunk_rows must be >= 0");
  *bytes = T == 0 ? 0 : plan_full(T, d, dt_hidden, V, elem_of(dt), chunk_rows).fused_total;
  return KD_OK;
}

kd_status kd_full_kl_fwd_bwd(const void* H, const void* Ws, const void* Ht, const void* Wt, const uint8_t* mask,
                             float tau, int64_t T, int64_t d, int64_t dt_hidden, int64_t V, kd_dtype dt,
                             const float* grad_kl, float* kl, float* lse_s, float* lse_t, void* dH, float* dWs,
                             int64_t chunk_rows, void* workspace, size_t workspace_bytes, void* stream) {
  return kd_full_kl_fwd_bwd_ex(H, Ws, Ht, Wt, mask, tau, nullptr, T, d, dt_hidden, V, dt, grad_kl, kl, lse_s, lse_t,
                               nullptr, dH, dWs, chunk_rows, workspace, workspace_bytes, stream);
}

kd_status kd_full_kl_fwd_bwd_ex(const void* H, const void* Ws, const void* Ht, const void* Wt, const uint8_t* mask,
                                float tau, const kd_full_opts* opts, int64_t T, int64_t d, int64_t dt_hidden,
                                int64_t V, kd_dtype dt, const float* grad_kl, float* kl, float* lse_s, float* lse_t,
                                float* kl_rev, void* dH, float* dWs, int64_t chunk_rows, void* workspace,
                                size_t workspace_bytes, void* stream) {
  g_err.clear();
  KD_TRY(check_common(T, d, V, dt, tau));
  KD_TRY(check_common(T, dt_hidden, V, dt, tau));
  kd::FullMix mx;
  KD_TRY(resolve_full_opts(opts, mx));
  KD_TRY(need_align(kl_rev, 4, "kl_rev"));
  KD_TRY(need(dWs, "dWs"));
  KD_TRY(need_align(dWs, 16, "dWs"));
  if (chunk_rows < 0) return fail(KD_ERR_INVALID_ARG, "chunk_rows must be >= 0");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (T == 0) {
    KD_LAUNCH("fill_zero", st, kd::launch_fill_zero(dWs, d * V * 4, st));
    return KD_OK;
  }
  KD_TRY(need(H, "H"));
  KD_TRY(need(Ws, "Ws"));
  KD_TRY(need(Ht, "Ht"));
  KD_TRY(need(Wt, "Wt"));
  KD_TRY(need(grad_kl, "grad_kl"));
  KD_TRY(need(kl, "kl"));
  KD_TRY(need(lse_s, "lse_s"));
  KD_TRY(need(lse_t, "lse_t"));
  KD_TRY(need(dH, "dH"));
  KD_TRY(need_align(H, 16, "H"));
  KD_TRY(need_align(Ws, 16, "Ws"));
  KD_TRY(need_align(Ht, 16, "Ht"));
  KD_TRY(need_align(Wt, 16, "Wt"));
  KD_TRY(need_align(dH, 16, "dH"));
  KD_TRY(need_align(grad_kl, 4, "grad_kl"));
  KD_TRY(need_align(kl, 4, "kl"));
  KD_TRY(need_align(lse_s, 4, "lse_s"));
  KD_TRY(need_align(lse_t, 4, "lse_t"));
  const int elem = elem_of(dt);
  const FullPlan p = plan_full(T, d, dt_hidden, V, elem, chunk_rows);
  KD_TRY(check_workspace(workspace, workspace_bytes, p.fused_total));

  kd::Compact c{at<int32_t>(workspace, p.o_rows), at<int32_t>(workspace, p.o_count)};
  float* part_s = at<float>(workspace, p.o_part_s);
  float* part_t = at<float>(workspace, p.o_part_t);
  float* zs = at<float>(workspace, p.o_zs);
  float* zt = at<float>(workspace, p.o_zt);
  float2* terms = at<float2>(workspace, p.o_terms);
  // the reverse KL of each row feeds its dZ when mixing: the caller's array, else the workspace's
  float* krev = kl_rev ? kl_rev : at<float>(workspace, p.o_krev);
  mx.kl_rev = krev;
  const ChunkPlan& ch = p.ch_f;
  char* dz = at<char>(workspace, ch.o_dz);
  char* hT = at<char>(workspace, ch.o_hT);
  float* dhp = at<float>(workspace, ch.o_dhp);
  const float c2 = (float)(1.4426950408889634 / (double)tau);
  // each head goes through the top-K forward tiles with no cached entries:
  // the per-row constants are the temperatures', the entry list is empty
  const kd::TopkRowData rd{at<int2>(workspace, p.o_pair0), nullptr, nullptr, at<float4>(workspace, p.o_rowc)};

  KD_LAUNCH("compact", st, kd::launch_compact(mask, T, c, st));
  KD_LAUNCH("zero_masked_rows", st, kd::launch_zero_masked_rows(mask, T, d * elem, dH, st));
  KD_LAUNCH("fill_zero", st, kd::launch_fill_zero(rd.pair, 16, st));
  KD_LAUNCH("full_rowc", st, kd::launch_full_rowc(c, T, mx.tau_rows, c2, 1.0f / tau, rd.rowc, st));
  const int64_t nchunks = cdiv(T, ch.C);
  for (int64_t k = 0; k < nchunks; ++k) {
    const int64_t c0 = k * ch.C;
    // the chunk's logits of each head, kept in fp32, and each head's log Z partials
    char* hp = at<char>(workspace, ch.o_hp);
    char* htp = at<char>(workspace, p.o_htp_u);
    KD_LAUNCH("gather_panels", st, kd::launch_gather_panels(H, d * elem, c, c0, ch.C, hp, st));
    KD_LAUNCH("gather_panels", st, kd::launch_gather_panels(Ht, dt_hidden * elem, c, c0, ch.C, htp, st));
    const ChunkShape sh = chunk_shape(T, c0, ch.C, cdiv(V, kd::kTileN));
    for (int head = 0; head < 2; ++head) {
      kd::TopkFwdArgs a{};
      a.Hp = head ? htp : hp;
      a.W = static_cast<const char*>(head ? Wt : Ws);
      a.c = c;
      a.rd = rd;
      a.part = head ? part_t : part_s;
      a.part_stride = ch.C;
      a.part_row0 = c0;
      a.c0 = c0;
      a.C = ch.C;
      a.zout = head ? zt : zs;
      a.ldz = ch.ldz;
      a.T = T;
      a.d = head ? dt_hidden : d;
      a.V = V;
      a.K = 0;
      a.Kz = 0;
      a.nrb = sh.nrb;
      a.S = sh.S;
      a.ntiles = (int)cdiv(V, kd::kTileN);
      a.group = kRasterGroup;
      KD_LAUNCH(head ? "full_teacher_tile" : "full_student_tile", st, kd::launch_topk_fwd(elem, a, st));
    }
    KD_LAUNCH("full_lse_combine", st,
              kd::launch_full_lse_combine(part_s, part_t, sh.S, ch.C, c, mask, T, kl, lse_s, lse_t, kl_rev, c0,
                                          c0 + ch.C, k == 0, st));
    // one pass over the kept logits: both KL terms with the final
    // normalisers and dZ (no second pair of projections); with the reverse
    // KL in the mix, dZ needs the row's reverse KL first, so the terms come
    // from a pass of their own
    kd::FullFromZArgs za{};
    za.zs = zs;
    za.zt = zt;
    za.ldz = ch.ldz;
    za.nblk = p.nblk;
    za.c = c;
    za.c0 = c0;
    za.C = ch.C;
    za.V = V;
    za.lse_s = lse_s;
    za.lse_t = lse_t;
    za.g = grad_kl;
    za.c2 = c2;
    za.inv_tau = 1.0f / tau;
    za.mix = mx;
    za.terms = terms;
    za.dz = mx.r != 0.f ? nullptr : dz;
    KD_LAUNCH("full_from_z", st, kd::launch_full_from_z(elem, za, st));
    KD_LAUNCH("full_kl_from_terms", st,
              kd::launch_full_kl_from_terms(terms, p.nblk, c, lse_s, lse_t, mx.r, kl, krev, c0, c0 + ch.C, st));
    if (mx.r != 0.f) {
      za.terms = nullptr;
      za.dz = dz;
      KD_LAUNCH("full_from_z", st, kd::launch_full_from_z(elem, za, st));
    }
    KD_TRY(grad_chunk(H, Ws, dH, dWs, elem, d, V, c, ch, dz, hT, dhp, c0, k > 0, st));
  }
  return KD_OK;
}

// ---------------------------------------------------------------- top-K, forward and backward in one call
kd_status kd_topk_kl_fwd_bwd_workspace_size(int64_t T, int64_t d, int64_t V, int64_t K, kd_dtype dt,
                                            int64_t chunk_rows, size_t* bytes) {
  g_err.clear();
  KD_TRY(need(bytes, "bytes"));
  KD_TRY(check_common(T, d, V, dt, 1.0f));
  KD_TRY(check_k(T, K, V));
  if (chunk_rows < 0) return fail(KD_ERR_INVALID_ARG, "chunk_rows must be >= 0");
  *bytes = T == 0 ? 0 : plan_topk(T, d, V, K, elem_of(dt), chunk_rows).fused_total;
  return KD_OK;
}

kd_status kd_topk_kl_fwd_bwd(const void* H, const void* W, const int32_t* topk_idx, const float* topk_logits,
                             const uint8_t* mask, float tau, int64_t T, int64_t d, int64_t V, int64_t K,
                             kd_dtype dt, const float* grad_kl, float* kl, float* lse, float* z_topk, void* dH,
                             float* dW, int64_t chunk_rows, void* workspace, size_t workspace_bytes, void* stream) {
  return kd_topk_kl_fwd_bwd_ex(H, W, topk_idx, topk_logits, mask, tau, nullptr, T, d, V, K, dt, grad_kl, kl, lse,
                               z_topk, dH, dW, chunk_rows, workspace, workspace_bytes, stream);
}

kd_status kd_topk_kl_fwd_bwd_ex(const void* H, const void* W, const int32_t* topk_idx, const float* topk_logits,
                                const uint8_t* mask, float tau, const kd_topk_opts* opts, int64_t T, int64_t d,
                                int64_t V, int64_t K, kd_dtype dt, const float* grad_kl, float* kl, float* lse,
                                float* z_topk, void* dH, float* dW, int64_t chunk_rows, void* workspace,
                                size_t workspace_bytes, void* stream) {
  g_err.clear();
  KD_TRY(check_common(T, d, V, dt, tau));
  KD_TRY(check_k(T, K, V));
  TopkOpts op;
  KD_TRY(resolve_opts(opts, tau, K, op));
  KD_TRY(need(dW, "dW"));
  KD_TRY(need_align(dW, 16, "dW"));
  if (chunk_rows < 0) return fail(KD_ERR_INVALID_ARG, "chunk_rows must be >= 0");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (T == 0) {
    KD_LAUNCH("fill_zero", st, kd::launch_fill_zero(dW, d * V * 4, st));
    return KD_OK;
  }
  KD_TRY(need(H, "H"));
  KD_TRY(need(W, "W"));
  KD_TRY(need(topk_idx, "topk_idx"));
  KD_TRY(need(topk_logits, "topk_logits"));
  KD_TRY(need(grad_kl, "grad_kl"));
  KD_TRY(need(kl, "kl"));
  KD_TRY(need(lse, "lse"));
  KD_TRY(need(dH, "dH"));
  KD_TRY(need_align(H, 16, "H"));
  KD_TRY(need_align(W, 16, "W"));
  KD_TRY(need_align(dH, 16, "dH"));
  KD_TRY(need_align(topk_idx, 4, "topk_idx"));
  KD_TRY(need_align(topk_logits, 4, "topk_logits"));
  KD_TRY(need_align(grad_kl, 4, "grad_kl"));
  KD_TRY(need_align(kl, 4, "kl"));
  KD_TRY(need_align(lse, 4, "lse"));
  KD_TRY(need_align(z_topk, 4, "z_topk"));
  if (op.prep.rev > 0.f) KD_TRY(need(z_topk, "z_topk (rev_weight > 0 reads it)"));
  const int elem = elem_of(dt);
  const TopkPlan p = plan_topk(T, d, V, K, elem, chunk_rows);
  KD_TRY(check_workspace(workspace, workspace_bytes, p.fused_total));

  kd::Compact c{at<int32_t>(workspace, p.o_rows), at<int32_t>(workspace, p.o_count)};
  const kd::TopkRowData rd = row_data(workspace, p, z_topk ? &p.o_zpair_f : nullptr);
  float* part = at<float>(workspace, p.o_part_c);
  float* z = at<float>(workspace, p.o_z);
  const ChunkPlan& ch = p.ch_f;
  char* dz = at<char>(workspace, ch.o_dz);
  char* hT = at<char>(workspace, ch.o_hT);
  float* dhp = at<float>(workspace, ch.o_dhp);

  KD_LAUNCH("compact", st, kd::launch_compact(mask, T, c, st));
  KD_TRY(start_index_check(op, workspace, p, V, st));
  KD_LAUNCH("topk_prep", st, kd::launch_topk_prep(topk_logits, topk_idx, mask, T, K, op.KE, op.prep, rd, z_topk, st));
  KD_TRY(finish_index_check(op, st));
  KD_LAUNCH("zero_masked_rows", st, kd::launch_zero_masked_rows(mask, T, d * elem, dH, st));
  const int64_t nchunks = cdiv(T, ch.C);
  for (int64_t k = 0; k < nchunks; ++k) {
    const int64_t c0 = k * ch.C;
    // the chunk's logits: log Z partials, the top-K gather, and z kept in fp32
    char* hp = at<char>(workspace, ch.o_hp);
    KD_LAUNCH("gather_panels", st, kd::launch_gather_panels(H, d * elem, c, c0, ch.C, hp, st));
    const ChunkShape sh = chunk_shape(T, c0, ch.C, p.ntiles);
    kd::TopkFwdArgs a{};
    a.Hp = hp;
    a.W = static_cast<const char*>(W);
    a.c = c;
    a.rd = rd;
    a.z_topk = z_topk;
    a.part = part;
    a.part_stride = ch.C;
    a.part_row0 = c0;
    a.c0 = c0;
    a.C = ch.C;
    a.zout = z;
    a.ldz = ch.ldz;
    a.T = T;
    a.d = d;
    a.V = V;
    a.K = op.KE;
    a.Kz = K;
    a.nrb = sh.nrb;
    a.S = sh.S;
    a.ntiles = p.ntiles;
    a.group = kRasterGroup;
    KD_LAUNCH("topk_fwd_tile", st, kd::launch_topk_fwd(elem, a, st));
    if (z_topk)
      KD_LAUNCH("topk_zpermute", st, kd::launch_topk_zpermute(rd, c, T, op.KE, K, z_topk, c0, c0 + ch.C, st));
    KD_LAUNCH("topk_combine", st,
              kd::launch_topk_combine(part, sh.S, ch.C, c, mask, rd, T, kl, lse, c0, c0 + ch.C, k == 0, st));
    if (op.prep.rev > 0.f)  // the reverse part: into kl, and into the weights the dZ pass scatters
      KD_LAUNCH("topk_reverse", st,
                kd::launch_topk_reverse(z_topk, topk_logits, c, T, K, op.KE, op.wr, rd, kl, true, c0, c0 + ch.C,
                                        st));
    // dZ from the kept logits: no second projection
    kd::TopkDzFromZArgs za{};
    za.z = z;
    za.dz = dz;
    za.ldz = ch.ldz;
    za.c = c;
    za.c0 = c0;
    za.C = ch.C;
    za.V = V;
    za.K = op.KE;
    za.rd = rd;
    za.lse = lse;
    za.g = grad_kl;
    KD_LAUNCH("topk_dz_from_z", st, kd::launch_topk_dz_from_z(elem, za, st));
    KD_TRY(grad_chunk(H, W, dH, dW, elem, d, V, c, ch, dz, hT, dhp, c0, k > 0, st));
  }
  return KD_OK;
}

}  // extern "C"
