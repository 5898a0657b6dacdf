// api.cpp -- host side of libcsa2.so: argument checks, workspace layout and
// the launch sequence of each entry point declared in include/csa2.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <utility>
#include <vector>

#include "../../include/csa2.h"
#include "csa2_internal.hpp"

using namespace csa2;

namespace csa2 {
LaunchTiming& launch_timing() {
  static thread_local LaunchTiming t;
  return t;
}
std::atomic<int32_t> g_topk_forced{kTopkAuto};
std::atomic<uint32_t> g_wait_limit{1u << 20};
std::atomic<uint32_t> g_generation{0};
thread_local int32_t g_topk_last = -1;
int32_t topk_variant_forced() { return g_topk_forced.load(std::memory_order_relaxed); }
void set_topk_last(int32_t v) { g_topk_last = v; }
uint32_t wait_limit() { return g_wait_limit.load(std::memory_order_relaxed); }
uint32_t next_generation() { return g_generation.fetch_add(1, std::memory_order_relaxed) + 1; }
}  // namespace csa2

namespace {

thread_local std::string g_last_error;

csa2_status fail(csa2_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
csa2_status fail(csa2_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

csa2_status hip_check(hipError_t e, const char* what) {
  if (e == hipSuccess) return CSA2_OK;
  return fail(CSA2_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define CSA2_TRY(expr, what)                         \
  do {                                               \
    csa2_status _s = hip_check((expr), (what));      \
    if (_s != CSA2_OK) return _s;                    \
  } while (0)

#define CSA2_REQUIRE(cond, status, ...)              \
  do {                                               \
    if (!(cond)) return fail((status), __VA_ARGS__); \
  } while (0)


// ---- optional launch timing (csa2_profile_begin / csa2_profile_end)
struct Profiler {
  bool on = false;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> ev[CSA2_PROFILE_KERNELS];
  std::vector<hipEvent_t> pool;
  size_t next = 0;
  hipEvent_t get() {
    if (next == pool.size()) {
      hipEvent_t e = nullptr;
      if (hipEventCreate(&e) != hipSuccess) return nullptr;
      pool.push_back(e);
    }
    return pool[next++];
  }
};
Profiler g_prof;

// While profiling is on, hands a start/stop event pair to the launcher of
// one call; the launcher attaches them to its kernels, so the pair times the
// kernels themselves.
struct ProfScope {
  int id;
  hipEvent_t b = nullptr, e = nullptr;
  ProfScope(int id_, hipStream_t) : id(id_) {
    if (g_prof.on && (b = g_prof.get()) && (e = g_prof.get())) launch_timing() = {b, e, false, false};
  }
  ~ProfScope() {
    LaunchTiming& t = launch_timing();
    if (b && e && t.started && t.stopped) g_prof.ev[id].push_back({b, e});
    t = LaunchTiming{};
  }
};

// Every entry point names its stream argument `stream`.
#define PROF_STREAM reinterpret_cast<hipStream_t>(stream)
#define CSA2_LAUNCH(id, st, expr, what)        \
  do {                                          \
    ProfScope _ps((id), (st));                  \
    csa2_status _s = hip_check((expr), (what)); \
    if (_s != CSA2_OK) return _s;               \
  } while (0)

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

constexpr int32_t kRowChunk = CSA2_PASS_ROWS;  // query rows scored / selected / attended per pass
// Passes of a prefill step that selects without a score matrix: its
// per-row buffers are small (samples, a candidate list, the exact path's
// score row), and passes this long fill the device in every launch.
constexpr int32_t kPrefillPassRows = CSA2_PREFILL_PASS_ROWS;
// Rows per attention launch within a pass: a 1024-row launch's partials
// (about 170 MB with 5 splits per row) fit the 256 MB last-level cache.
constexpr int32_t kAttnPassRows = 1024;

// A bump allocator over the caller's workspace.  The per-row control block
// (kCtlWordsPerRow words) always comes first, so every kind of call finds
// its control words at the same offsets.
struct Carve {
  char* base;
  size_t off = 0;
  explicit Carve(void* ws) : base((char*)ws) {}
  template <typename T>
  T* take(size_t count) {
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off = align_up(off + count * sizeof(T));
    return p;
  }
};

// Control block of row r: the kHistWords histogram copies, then the Top-K
// counters.
void carve_ctl(Carve& c, int32_t rows, TopkWs* tw) {
  uint32_t* ctl = c.take<uint32_t>((size_t)rows * kCtlWordsPerRow);
  if (tw) {
    tw->hist = ctl;
    tw->hist_stride = kCtlWordsPerRow;
    tw->ctr = ctl ? ctl + kHistWords : nullptr;
    tw->ctr_stride = kCtlWordsPerRow;
    tw->cut = ctl ? ctl + kHistWords + 1 : nullptr;
    // Copies spread the histogram atomics of a row's many scoring blocks,
    // but every select block reads all of them: two balance the two (measured
    // at 256K positions x 4 rows); with many rows per pass, one.
    tw->hist_copies = rows <= 32 ? 2 : 1;
  }
}

// Kept-position and candidate regions: one kTopkChunk region of each per
// select block of a row, and the blocks' counts.
void carve_topk(Carve& c, int32_t rows, int64_t n, int32_t k, TopkWs* tw) {
  (void)k;
  const int64_t nblk = std::max<int64_t>(1, (n + kTopkChunk - 1) / kTopkChunk);
  // regions cover whole blocks of either chunk size
  const int64_t span = std::max<int64_t>(1, (n + kTopkChunkLarge - 1) / kTopkChunkLarge) * kTopkChunkLarge;
  tw->above_stride = span;
  tw->above = c.take<uint32_t>((size_t)rows * tw->above_stride);
  tw->cand_stride = span;
  tw->cand = c.take<uint64_t>((size_t)rows * tw->cand_stride);
  tw->counts_stride = 2 * nblk;
  tw->counts = c.take<uint32_t>((size_t)rows * tw->counts_stride);
}

// Attention partials of passes of rc rows over `rows` rows.  exact: the
// passes' own split counts (attn_rounds of each pass's rows, FP4 cache);
// otherwise room for one round per split, which serves either cache.
void carve_attn(Carve& c, int32_t rows, int32_t rc, int32_t K, int32_t W, int32_t dv, AttnWs* aw,
                bool exact = false) {
  int64_t units = (int64_t)rc * attn_split(K, W).nsplit;
  if (exact) {
    const int32_t last = rows % rc;
    units = (int64_t)rc * attn_split(K, W, attn_rounds(rc, K, W, false)).nsplit;
    if (last > 0)
      units = std::max<int64_t>(units, (int64_t)last * attn_split(K, W, attn_rounds(last, K, W, false)).nsplit);
  }
  aw->part = c.take<float>((size_t)units * (16 * (size_t)dv + 32));
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

bool attn_shape_ok(int32_t D, int32_t dv) { return (D == 576 && dv == 512) || (D == 128 && dv == 128); }

}  // namespace

// ------------------------------------------------------------ static scratch
// Workspace of csa2_layer_step_static: one copy of this array per GPU,
// held until the process ends.  Host code never uses the array's name as a
// device address: the address comes from hipGetSymbolAddress, once per
// device, with that device current.
namespace {
constexpr size_t kStaticScratchBytes = CSA2_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

struct StaticScratch {
  void* ptr = nullptr;  // device address of this GPU's copy
  bool clean = false;   // control words known to be zero
};
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
StaticScratch g_scratch[kMaxDevices];

// This device's scratch address; on first use (and after a call that failed
// part-way) the whole array is zero-filled by a kernel on `st`.
csa2_status static_scratch(hipStream_t st, int* dev_out, void** ptr_out) {
  int dev = -1;
  CSA2_TRY(hipGetDevice(&dev), "current device");
  CSA2_REQUIRE(dev >= 0 && dev < kMaxDevices, CSA2_ERR_UNSUPPORTED, "device %d beyond %d", dev,
               kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  StaticScratch& sc = g_scratch[dev];
  if (!sc.ptr) {
    void* p = nullptr;
    CSA2_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "static scratch address");
    CSA2_REQUIRE(p, CSA2_ERR_HIP, "static scratch address is NULL");
    sc.ptr = p;
  }
  if (!sc.clean) {
    CSA2_TRY(launch_fill_zero(sc.ptr, kStaticScratchBytes, st), "static scratch clear");
    sc.clean = true;
  }
  *dev_out = dev;
  *ptr_out = sc.ptr;
  return CSA2_OK;
}
}  // namespace

extern "C" {

const char* csa2_status_string(csa2_status s) {
  switch (s) {
    case CSA2_OK: return "ok";
    case CSA2_ERR_NULL: return "null pointer";
    case CSA2_ERR_SHAPE: return "bad shape";
    case CSA2_ERR_DTYPE: return "bad dtype";
    case CSA2_ERR_WORKSPACE: return "workspace too small";
    case CSA2_ERR_UNSUPPORTED: return "unsupported";
    case CSA2_ERR_HIP: return "hip error";
    case CSA2_ERR_INCOMPLETE: return "a one-wait launch gave up waiting";
  }
  return "unknown status";
}

const char* csa2_last_error(void) { return g_last_error.c_str(); }

const char* csa2_version(void) { return "csa2-mi355x 0.1 (gfx950)"; }

size_t csa2_layer_args_size(void) { return sizeof(csa2_layer_args); }

csa2_status csa2_profile_begin(void) {
  g_last_error.clear();
  for (auto& v : g_prof.ev) v.clear();
  g_prof.next = 0;
  g_prof.on = true;
  return CSA2_OK;
}

csa2_status csa2_profile_end(int32_t* counts, double* total_ms) {
  g_last_error.clear();
  g_prof.on = false;
  for (int k = 0; k < CSA2_PROFILE_KERNELS; ++k) {
    double tot = 0.0;
    for (auto& pr : g_prof.ev[k]) {
      CSA2_TRY(hipEventSynchronize(pr.second), "profile event wait");
      float ms = 0.0f;
      CSA2_TRY(hipEventElapsedTime(&ms, pr.first, pr.second), "profile event time");
      tot += ms;
    }
    if (counts) counts[k] = (int32_t)g_prof.ev[k].size();
    if (total_ms) total_ms[k] = tot;
    g_prof.ev[k].clear();
  }
  g_prof.next = 0;
  return CSA2_OK;
}
size_t csa2_fp4_cache_size(void) { return sizeof(csa2_fp4_cache); }

size_t csa2_workspace_control_bytes(int32_t rows) {
  if (rows < 1) return 0;
  return (size_t)std::min(rows, kRowChunk) * kCtlWordsPerRow * sizeof(uint32_t);
}

int64_t csa2_fp4_bytes_per_token(int32_t dim) {
  if (dim <= 0 || dim % 16) return -1;
  return dim / 2 + dim / 16;
}

csa2_status csa2_workspace_check(void* ws, size_t ws_bytes, int32_t rows, void* stream) {
  g_last_error.clear();
  CSA2_REQUIRE(ws, CSA2_ERR_NULL, "workspace is NULL");
  CSA2_REQUIRE(rows >= 1, CSA2_ERR_SHAPE, "rows must be >= 1");
  const size_t ctl = csa2_workspace_control_bytes(rows);
  CSA2_REQUIRE(ws_bytes >= ctl, CSA2_ERR_WORKSPACE, "workspace needs %zu control bytes (got %zu)",
               ctl, ws_bytes);
  const int32_t rc = std::min(rows, kRowChunk);
  const hipStream_t st = as_stream(stream);
  CSA2_TRY(hipStreamSynchronize(st), "stream wait");
  // per row: 16 words after the histogram copies; word 2 is the Top-K
  // one-wait flag, word kAttnCtlWord - kHistWords + 2 the one-launch
  // attention's
  constexpr int kSpan = 16;
  static_assert(kAttnCtlWord - kHistWords + 2 < kSpan, "flags inside the words read");
  std::vector<uint32_t> words((size_t)rc * kSpan);
  CSA2_TRY(hipMemcpy2D(words.data(), kSpan * sizeof(uint32_t),
                       static_cast<char*>(ws) + kHistWords * sizeof(uint32_t),
                       kCtlWordsPerRow * sizeof(uint32_t), kSpan * sizeof(uint32_t), (size_t)rc,
                       hipMemcpyDeviceToHost),
           "control word read");
  int32_t first = -1, nbad = 0;
  for (int32_t r = 0; r < rc; ++r) {
    const uint32_t* w = words.data() + (size_t)r * kSpan;
    if (w[2] != 0u || w[kAttnCtlWord - kHistWords + 2] != 0u) {
      if (first < 0) first = r;
      ++nbad;
    }
  }
  if (nbad == 0) return CSA2_OK;
  CSA2_TRY(launch_fill_zero(ws, ctl, st), "control block clear");
  CSA2_TRY(hipStreamSynchronize(st), "stream wait");
  return fail(CSA2_ERR_INCOMPLETE,
              "a one-wait launch gave up waiting for another block (%d row slot(s), first %d): "
              "the outputs of the calls since the last check are incomplete",
              nbad, first);
}

csa2_status csa2_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t blocks,
                             void* stream) {
  g_last_error.clear();
  CSA2_REQUIRE(src && sink, CSA2_ERR_NULL, "src and sink are required");
  CSA2_REQUIRE(bytes >= 16 && bytes % 16 == 0, CSA2_ERR_SHAPE, "bytes must be a positive multiple of 16");
  CSA2_REQUIRE(blocks >= 1 && blocks <= (1 << 20), CSA2_ERR_SHAPE, "blocks must be in [1, 2^20]");
  CSA2_TRY(launch_stream_read(src, (int64_t)bytes, sink, blocks, as_stream(stream)), "stream read launch");
  return CSA2_OK;
}

int32_t csa2_set_topk_variant(int32_t variant) {
  if (variant < kTopkAuto || variant >= kTopkVariants) variant = kTopkAuto;
  return g_topk_forced.exchange(variant);
}

int32_t csa2_topk_last_variant(void) { return g_topk_last; }

uint32_t csa2_set_wait_limit(uint32_t polls) { return g_wait_limit.exchange(polls); }

csa2_status csa2_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  if (ws_bytes == 0) return CSA2_OK;
  CSA2_REQUIRE(ws, CSA2_ERR_NULL, "workspace is NULL");
  CSA2_TRY(launch_fill_zero(ws, ws_bytes, as_stream(stream)), "workspace fill");
  return CSA2_OK;
}

// ------------------------------------------------------------ quantize
csa2_status csa2_quantize_kv(const void* x, csa2_dtype dtype, int64_t rows, int32_t dim,
                             int64_t x_row_stride, const int64_t* dst_rows, uint8_t* codes,
                             uint8_t* scales, void* stream) {
  g_last_error.clear();
  CSA2_REQUIRE(dtype == CSA2_F32 || dtype == CSA2_BF16, CSA2_ERR_DTYPE, "unknown dtype %d", (int)dtype);
  CSA2_REQUIRE(rows >= 0, CSA2_ERR_SHAPE, "rows < 0");
  CSA2_REQUIRE(dim > 0 && dim % 16 == 0 && dim <= 4096, CSA2_ERR_SHAPE,
               "dim must be a positive multiple of 16 <= 4096 (got %d)", dim);
  CSA2_REQUIRE(x_row_stride >= dim, CSA2_ERR_SHAPE, "row stride %lld < dim %d",
               (long long)x_row_stride, dim);
  if (rows == 0) return CSA2_OK;
  CSA2_REQUIRE(x && codes && scales, CSA2_ERR_NULL, "x, codes and scales are required");
  CSA2_LAUNCH(0, PROF_STREAM, launch_quantize(x, dtype == CSA2_BF16, rows, dim, x_row_stride, dst_rows, codes, scales,
                           as_stream(stream)),
           "quantize launch");
  return CSA2_OK;
}

csa2_status csa2_rope_quantize_kv(const void* x, csa2_dtype dtype, int64_t rows, int32_t dim,
                                  int64_t x_row_stride, int32_t rope_dim, const float* cos_sin,
                                  const int64_t* dst_rows, uint8_t* codes, uint8_t* scales,
                                  void* stream) {
  g_last_error.clear();
  CSA2_REQUIRE(dtype == CSA2_F32 || dtype == CSA2_BF16, CSA2_ERR_DTYPE, "unknown dtype %d", (int)dtype);
  CSA2_REQUIRE(rows >= 0, CSA2_ERR_SHAPE, "rows < 0");
  CSA2_REQUIRE(dim > 0 && dim % 16 == 0 && dim <= 4096, CSA2_ERR_SHAPE,
               "dim must be a positive multiple of 16 <= 4096 (got %d)", dim);
  CSA2_REQUIRE(rope_dim >= 0 && rope_dim % 16 == 0 && rope_dim <= dim, CSA2_ERR_SHAPE,
               "rope_dim must be a multiple of 16 in [0, dim] (got %d)", rope_dim);
  CSA2_REQUIRE(x_row_stride >= dim, CSA2_ERR_SHAPE, "row stride %lld < dim %d",
               (long long)x_row_stride, dim);
  if (rows == 0) return CSA2_OK;
  CSA2_REQUIRE(x && codes && scales, CSA2_ERR_NULL, "x, codes and scales are required");
  CSA2_REQUIRE(rope_dim == 0 || cos_sin, CSA2_ERR_NULL, "cos_sin is required when rope_dim > 0");
  CSA2_LAUNCH(0, PROF_STREAM, launch_rope_quantize(x, dtype == CSA2_BF16, rows, dim, x_row_stride, rope_dim,
                                                   cos_sin, dst_rows, codes, scales, as_stream(stream)),
              "rope quantize launch");
  return CSA2_OK;
}

// ------------------------------------------------------------ index score
static csa2_status check_icache(const csa2_fp4_cache* c, const char* name) {
  CSA2_REQUIRE(c, CSA2_ERR_NULL, "%s cache descriptor is NULL", name);
  CSA2_REQUIRE(c->codes && c->scales, CSA2_ERR_NULL, "%s cache planes are NULL", name);
  CSA2_REQUIRE(c->cap >= 1, CSA2_ERR_SHAPE, "%s cache capacity < 1", name);
  return CSA2_OK;
}

csa2_status csa2_index_score(const csa2_fp4_cache* icache, int32_t B, int32_t T,
                             const uint16_t* q_idx, const float* w, int32_t H_I,
                             const int32_t* n_valid, const int32_t* pool, int32_t P,
                             int64_t n_out, float* scores, void* stream) {
  g_last_error.clear();
  csa2_status s = check_icache(icache, "index");
  if (s) return s;
  CSA2_REQUIRE(B >= 1 && T >= 1, CSA2_ERR_SHAPE, "B and T must be >= 1");
  CSA2_REQUIRE(H_I >= 1 && H_I <= CSA2_MAX_INDEX_HEADS, CSA2_ERR_SHAPE, "H_I must be in [1,16]");
  CSA2_REQUIRE(icache->dim % 128 == 0 && icache->dim >= 128 && icache->dim <= 512,
               CSA2_ERR_UNSUPPORTED, "index dim must be 128, 256, 384 or 512 (got %d)",
               icache->dim);
  CSA2_REQUIRE(q_idx && w && n_valid && scores, CSA2_ERR_NULL,
               "q_idx, w, n_valid and scores are required");
  CSA2_REQUIRE(n_out >= 1, CSA2_ERR_SHAPE, "n_out < 1");
  CSA2_REQUIRE(!pool || P >= 1, CSA2_ERR_SHAPE, "pool given with P < 1");
  CSA2_REQUIRE((int64_t)B * T <= 65535, CSA2_ERR_SHAPE, "B*T must be <= 65535");
  const int64_t n_max = pool ? std::min<int64_t>(P, n_out) : std::min<int64_t>(icache->cap, n_out);
  CSA2_LAUNCH(1, PROF_STREAM, launch_index_score(icache->codes, icache->scales, icache->dim, icache->cap, B * T, T,
                              q_idx, w, H_I, n_valid, 0, pool, pool ? P : 0, n_max, scores, n_out,
                              nullptr, 0, 1, as_stream(stream)),
           "index score launch");
  return CSA2_OK;
}

// ------------------------------------------------------------ top-k
size_t csa2_topk_workspace_bytes(int32_t rows, int64_t n, int32_t k) {
  if (rows < 1 || n < 1 || k < 1) return 0;
  const int32_t rc = std::min(rows, kRowChunk);
  Carve c(nullptr);
  TopkWs tw;
  carve_ctl(c, rc, &tw);
  carve_topk(c, rc, n, k, &tw);
  return c.off;
}

csa2_status csa2_topk(const float* scores, int32_t rows, int64_t n, const int32_t* n_valid,
                      const int32_t* slot_pos, int32_t k, int32_t* idx_out, int32_t* count_out,
                      void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  CSA2_REQUIRE(rows >= 1 && rows <= 65535, CSA2_ERR_SHAPE, "rows must be in [1,65535]");
  CSA2_REQUIRE(n >= 1 && n <= kMaxTopkN, CSA2_ERR_SHAPE, "n must be in [1, 2^25]");
  CSA2_REQUIRE(k >= 1 && k <= CSA2_MAX_K, CSA2_ERR_SHAPE, "k must be in [1,%d]", CSA2_MAX_K);
  CSA2_REQUIRE(scores && n_valid && idx_out, CSA2_ERR_NULL, "scores, n_valid and idx_out are required");
  const size_t need = csa2_topk_workspace_bytes(rows, n, k);
  CSA2_REQUIRE(ws && ws_bytes >= need, CSA2_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)",
               need, ws_bytes);
  const int32_t rc = std::min(rows, kRowChunk);
  Carve c(ws);
  TopkWs tw;
  carve_ctl(c, rc, &tw);
  carve_topk(c, rc, n, k, &tw);
  const hipStream_t st = as_stream(stream);
  for (int32_t r0 = 0; r0 < rows; r0 += rc) {
    const int32_t nr = std::min(rc, rows - r0);
    const float* sc = scores + (size_t)r0 * n;
    const int32_t* nv = n_valid + r0;
    const int32_t* sp = slot_pos ? slot_pos + (size_t)r0 * n : nullptr;
    const bool row = topk_row_pass(nr, n);  // one block per row: no histogram
    if (!row)
      CSA2_LAUNCH(2, PROF_STREAM, launch_topk_hist(sc, nr, n, nv, 0, n, tw.hist, tw.hist_stride, tw.hist_copies, st),
                  "top-k histogram launch");
    CSA2_LAUNCH(2, PROF_STREAM,
                launch_topk_select(sc, nr, n, nv, 0, n, sp, k, idx_out + (size_t)r0 * k,
                                   count_out ? count_out + r0 : nullptr, tw, st, row),
                "top-k select launch");
  }
  return CSA2_OK;
}

// ------------------------------------------------------------ attention
size_t csa2_sparse_attn_workspace_bytes(int32_t rows, int32_t K, int32_t W, int32_t dv) {
  if (rows < 1 || K < 0 || W < 0 || dv < 1) return 0;
  const int32_t rc = std::min(rows, kRowChunk);
  Carve c(nullptr);
  AttnWs aw;
  carve_ctl(c, rc, nullptr);
  carve_attn(c, rows, rc, K, W, dv, &aw);
  return c.off;
}

static csa2_status check_attn(const uint16_t* q, int32_t B, int32_t T, int32_t H,
                              const csa2_fp4_cache* kv, const int32_t* idx, int32_t K,
                              const uint8_t* swa, const float* swa_scale,
                              const int32_t* swa_pos0, int32_t S, int32_t W,
                              const int32_t* q_pos, int32_t dv, const float* out) {
  csa2_status s = check_icache(kv, "main");
  if (s) return s;
  CSA2_REQUIRE(B >= 1 && T >= 1, CSA2_ERR_SHAPE, "B and T must be >= 1");
  CSA2_REQUIRE((int64_t)B * T <= 65535, CSA2_ERR_SHAPE, "B*T must be <= 65535");
  CSA2_REQUIRE(H == CSA2_HEADS, CSA2_ERR_UNSUPPORTED, "H must be %d (got %d)", CSA2_HEADS, H);
  CSA2_REQUIRE(attn_shape_ok(kv->dim, dv), CSA2_ERR_UNSUPPORTED,
               "(D, dv) must be (576, 512) or (128, 128) (got (%d, %d))", kv->dim, dv);
  CSA2_REQUIRE(K >= 0 && K <= CSA2_MAX_K, CSA2_ERR_SHAPE, "K must be in [0,%d]", CSA2_MAX_K);
  CSA2_REQUIRE(W >= 0 && W <= CSA2_MAX_W && S >= 0, CSA2_ERR_SHAPE,
               "W must be in [0,%d] and S >= 0", CSA2_MAX_W);
  CSA2_REQUIRE(q && q_pos && out, CSA2_ERR_NULL, "q, q_pos and out are required");
  CSA2_REQUIRE(K == 0 || idx, CSA2_ERR_NULL, "idx is required when K > 0");
  CSA2_REQUIRE(W == 0 || S == 0 || (swa && swa_scale && swa_pos0), CSA2_ERR_NULL,
               "swa, swa_scale and swa_pos0 are required when W > 0 and S > 0");
  return CSA2_OK;
}

static csa2_status sparse_attn_impl(const uint16_t* q, int32_t B, int32_t T, int32_t H,
                                    const csa2_fp4_cache* kv, const int32_t* idx, int32_t K,
                                    const uint8_t* swa, const float* swa_scale,
                                    const int32_t* swa_pos0, int32_t S, int32_t W,
                                    const int32_t* q_pos, float sm_scale, int32_t dv, float* out,
                                    float* lse, void* ws, size_t ws_bytes, void* stream,
                                    bool one_launch) {
  g_last_error.clear();
  csa2_status s = check_attn(q, B, T, H, kv, idx, K, swa, swa_scale, swa_pos0, S, W, q_pos, dv, out);
  if (s) return s;
  const int32_t rows = B * T;
  const int32_t Weff = (S > 0) ? W : 0;
  const size_t need = csa2_sparse_attn_workspace_bytes(rows, K, Weff, dv);
  CSA2_REQUIRE(ws && ws_bytes >= need, CSA2_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)",
               need, ws_bytes);
  const int32_t rc = std::min(rows, kRowChunk);
  Carve c(ws);
  AttnWs aw;
  carve_ctl(c, rc, nullptr);
  carve_attn(c, rows, rc, K, Weff, dv, &aw);
  const int32_t D = kv->dim;
  for (int32_t r0 = 0; r0 < rows; r0 += rc) {
    const int32_t nr = std::min(rc, rows - r0);
    CSA2_LAUNCH(3, PROF_STREAM,
                launch_sparse_attn(q + (size_t)r0 * H * D, nr, T, D, dv, kv->codes, kv->scales,
                                   kv->cap, idx ? idx + (size_t)r0 * K : nullptr, K, swa,
                                   swa_scale, swa_pos0, S, Weff, q_pos + r0, sm_scale,
                                   out + (size_t)r0 * H * dv, lse ? lse + (size_t)r0 * H : nullptr,
                                   aw, as_stream(stream), r0, nullptr,
                                   one_launch ? static_cast<uint32_t*>(ws) + kAttnCtlWord : nullptr),
                "sparse attention launch");
  }
  return CSA2_OK;
}

csa2_status csa2_sparse_attn(const uint16_t* q, int32_t B, int32_t T, int32_t H,
                             const csa2_fp4_cache* kv, const int32_t* idx, int32_t K,
                             const uint8_t* swa, const float* swa_scale, const int32_t* swa_pos0,
                             int32_t S, int32_t W, const int32_t* q_pos, float sm_scale,
                             int32_t dv, float* out, float* lse, void* ws, size_t ws_bytes,
                             void* stream) {
  return sparse_attn_impl(q, B, T, H, kv, idx, K, swa, swa_scale, swa_pos0, S, W, q_pos, sm_scale,
                          dv, out, lse, ws, ws_bytes, stream, false);
}

csa2_status csa2_sparse_attn_one_launch(const uint16_t* q, int32_t B, int32_t T, int32_t H,
                                        const csa2_fp4_cache* kv, const int32_t* idx, int32_t K,
                                        const uint8_t* swa, const float* swa_scale,
                                        const int32_t* swa_pos0, int32_t S, int32_t W,
                                        const int32_t* q_pos, float sm_scale, int32_t dv,
                                        float* out, float* lse, void* ws, size_t ws_bytes,
                                        void* stream) {
  return sparse_attn_impl(q, B, T, H, kv, idx, K, swa, swa_scale, swa_pos0, S, W, q_pos, sm_scale,
                          dv, out, lse, ws, ws_bytes, stream, true);
}

csa2_status csa2_quantize_kv_fp8(const void* x, csa2_dtype dtype, int64_t rows, int32_t dim,
                                 int64_t x_row_stride, const int64_t* dst_rows, uint8_t* codes,
                                 float* scales, void* stream) {
  g_last_error.clear();
  CSA2_REQUIRE(dtype == CSA2_F32 || dtype == CSA2_BF16, CSA2_ERR_DTYPE, "unknown dtype %d", (int)dtype);
  CSA2_REQUIRE(rows >= 0, CSA2_ERR_SHAPE, "rows < 0");
  CSA2_REQUIRE(dim > 0 && dim % 16 == 0 && dim <= 4096, CSA2_ERR_SHAPE,
               "dim must be a positive multiple of 16 <= 4096 (got %d)", dim);
  CSA2_REQUIRE(x_row_stride >= dim, CSA2_ERR_SHAPE, "row stride %lld < dim %d",
               (long long)x_row_stride, dim);
  if (rows == 0) return CSA2_OK;
  CSA2_REQUIRE(x && codes && scales, CSA2_ERR_NULL, "x, codes and scales are required");
  CSA2_LAUNCH(0, PROF_STREAM, launch_quantize_fp8(x, dtype == CSA2_BF16, rows, dim, x_row_stride,
                                                  dst_rows, codes, scales, as_stream(stream)),
              "fp8 quantize launch");
  return CSA2_OK;
}

csa2_status csa2_sparse_attn_fp8(const uint16_t* q, int32_t B, int32_t T, int32_t H,
                                 const csa2_fp8_cache* kv, const int32_t* idx, int32_t K,
                                 const uint8_t* swa, const float* swa_scale,
                                 const int32_t* swa_pos0, int32_t S, int32_t W,
                                 const int32_t* q_pos, float sm_scale, int32_t dv, float* out,
                                 float* lse, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  CSA2_REQUIRE(kv, CSA2_ERR_NULL, "kv cache descriptor is NULL");
  // the shared checks see the FP8 planes through an FP4 descriptor of the same shape
  const csa2_fp4_cache shape{kv->codes, reinterpret_cast<uint8_t*>(kv->scales), kv->dim, kv->cap};
  csa2_status s = check_attn(q, B, T, H, &shape, idx, K, swa, swa_scale, swa_pos0, S, W, q_pos, dv, out);
  if (s) return s;
  const int32_t rows = B * T;
  const int32_t Weff = (S > 0) ? W : 0;
  const size_t need = csa2_sparse_attn_workspace_bytes(rows, K, Weff, dv);
  CSA2_REQUIRE(ws && ws_bytes >= need, CSA2_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)",
               need, ws_bytes);
  const int32_t rc = std::min(rows, kRowChunk);
  Carve c(ws);
  AttnWs aw;
  carve_ctl(c, rc, nullptr);
  carve_attn(c, rows, rc, K, Weff, dv, &aw);
  const int32_t D = kv->dim;
  for (int32_t r0 = 0; r0 < rows; r0 += rc) {
    const int32_t nr = std::min(rc, rows - r0);
    CSA2_LAUNCH(3, PROF_STREAM,
                launch_sparse_attn(q + (size_t)r0 * H * D, nr, T, D, dv, kv->codes, nullptr,
                                   kv->cap, idx ? idx + (size_t)r0 * K : nullptr, K, swa,
                                   swa_scale, swa_pos0, S, Weff, q_pos + r0, sm_scale,
                                   out + (size_t)r0 * H * dv, lse ? lse + (size_t)r0 * H : nullptr,
                                   aw, as_stream(stream), r0, kv->scales),
                "fp8 sparse attention launch");
  }
  return CSA2_OK;
}

// ------------------------------------------------------------ layer step
namespace {

struct StepLayout {
  int32_t rc;         // rows per pass
  bool sampled;       // a prefill step selecting without a score matrix
  int64_t n_out;      // score row length
  TopkWs tw;
  AttnWs aw;
  float* scores;
  float* pscores;     // FULL with a pool: pool members' scores
  size_t bytes;
};

// Whether a step's passes select without a score matrix (its shapes, and
// unless shapes_only the forced Top-K variant; every pass of such a step
// qualifies, since passes start at multiples of 32 rows).
bool sampled_step(csa2_mode mode, const csa2_layer_args* a, bool shapes_only) {
  if (mode == CSA2_MODE_REUSE || (mode == CSA2_MODE_FULL && a->P > 0) ||
      (mode == CSA2_MODE_REINDEX && a->pool_in))
    return false;
  return shapes_only ? sampled_select_shapes(1, a->T, a->H_I, a->D_I, 0, a->K, a->icache.cap)
                     : sampled_select_pass(1, a->T, a->H_I, a->D_I, 0, a->K, a->icache.cap);
}

// sampled: -1 from the step and the forced Top-K variant now, else 0 / 1.
StepLayout step_layout(csa2_mode mode, const csa2_layer_args* a, void* ws, int sampled = -1) {
  StepLayout L{};
  const int32_t rows = a->B * a->T;
  L.sampled = sampled < 0 ? sampled_step(mode, a, false) : sampled == 1;
  L.rc = std::min(rows, L.sampled ? kPrefillPassRows : kRowChunk);
  const bool pooled_in = (mode == CSA2_MODE_REINDEX && a->pool_in);
  L.n_out = (mode == CSA2_MODE_REUSE) ? 1 : (pooled_in ? a->P_in : a->icache.cap);
  const int32_t Weff = (a->S > 0) ? a->W : 0;
  Carve c(ws);
  // the control block always covers min(rows, kRowChunk) rows (the sampled
  // selection uses none of its words)
  carve_ctl(c, std::min(L.rc, kRowChunk), &L.tw);
  if (L.sampled) {
    // the exact path's score rows, then the position samples, the
    // candidate lists and the per-row threshold, count and fail words
    L.scores = c.take<float>((size_t)L.rc * L.n_out);
    L.tw.above_stride = (L.n_out + kSampleStride - 1) / kSampleStride;
    L.tw.above = c.take<uint32_t>((size_t)L.rc * L.tw.above_stride);
    L.tw.cand_stride = kCandCap;
    L.tw.cand = c.take<uint64_t>((size_t)L.rc * kCandCap);
    L.tw.counts_stride = 3;
    L.tw.counts = c.take<uint32_t>((size_t)L.rc * 3);
  } else if (mode != CSA2_MODE_REUSE) {
    L.scores = c.take<float>((size_t)L.rc * L.n_out);
    const int32_t kmax = (mode == CSA2_MODE_FULL && a->P > 0) ? std::max(a->P, a->K) : a->K;
    if (mode == CSA2_MODE_FULL && a->P > 0) L.pscores = c.take<float>((size_t)L.rc * a->P);
    carve_topk(c, L.rc, std::max<int64_t>(L.n_out, a->P), kmax, &L.tw);
  }
  carve_attn(c, rows, std::min(L.rc, kAttnPassRows), a->K, Weff, a->dv, &L.aw, true);
  L.bytes = c.off;
  return L;
}

// Workspace bytes of a step: the larger of the layouts it can take (a
// prefill step's passes select without a score matrix unless a forced Top-K
// variant says otherwise, so a workspace sized once serves every variant).
size_t step_bytes(csa2_mode mode, const csa2_layer_args* a) {
  size_t b = step_layout(mode, a, nullptr, 0).bytes;
  if (sampled_step(mode, a, true)) b = std::max(b, step_layout(mode, a, nullptr, 1).bytes);
  return b;
}

csa2_status check_step(csa2_mode mode, const csa2_layer_args* a) {
  CSA2_REQUIRE(a, CSA2_ERR_NULL, "layer args are NULL");
  CSA2_REQUIRE(mode == CSA2_MODE_FULL || mode == CSA2_MODE_REINDEX || mode == CSA2_MODE_REUSE,
               CSA2_ERR_SHAPE, "unknown mode %d", (int)mode);
  csa2_status s = check_attn(a->q, a->B, a->T, a->H, &a->kv,
                             mode == CSA2_MODE_REUSE ? a->idx_in : a->idx_out, a->K, a->swa,
                             a->swa_scale, a->swa_pos0, a->S, a->W, a->q_pos, a->dv, a->out);
  if (s) return s;
  CSA2_REQUIRE(a->D == a->kv.dim, CSA2_ERR_SHAPE, "D (%d) != kv.dim (%d)", a->D, a->kv.dim);
  if (mode == CSA2_MODE_REUSE) {
    CSA2_REQUIRE(a->K == 0 || a->idx_in, CSA2_ERR_NULL, "REUSE needs idx_in");
    return CSA2_OK;
  }
  s = check_icache(&a->icache, "index");
  if (s) return s;
  CSA2_REQUIRE(a->K >= 1, CSA2_ERR_SHAPE, "FULL/REINDEX need K >= 1");
  CSA2_REQUIRE(a->D_I == a->icache.dim, CSA2_ERR_SHAPE, "D_I (%d) != icache.dim (%d)", a->D_I,
               a->icache.dim);
  CSA2_REQUIRE(a->D_I % 128 == 0 && a->D_I >= 128 && a->D_I <= 512, CSA2_ERR_UNSUPPORTED,
               "index dim must be 128, 256, 384 or 512");
  CSA2_REQUIRE(a->H_I >= 1 && a->H_I <= CSA2_MAX_INDEX_HEADS, CSA2_ERR_SHAPE, "H_I must be in [1,16]");
  CSA2_REQUIRE(a->q_idx && a->w_idx && a->idx_out, CSA2_ERR_NULL,
               "q_idx, w_idx and idx_out are required");
  CSA2_REQUIRE(a->icache.cap <= kMaxTopkN, CSA2_ERR_SHAPE, "index cache capacity above 2^25");
  if (mode == CSA2_MODE_FULL) {
    CSA2_REQUIRE(a->new_kv && a->new_ikey, CSA2_ERR_NULL, "FULL needs new_kv and new_ikey");
    CSA2_REQUIRE(a->new_dtype == CSA2_F32 || a->new_dtype == CSA2_BF16, CSA2_ERR_DTYPE,
                 "unknown dtype %d", (int)a->new_dtype);
    CSA2_REQUIRE(a->P >= 0 && a->P <= CSA2_MAX_K, CSA2_ERR_SHAPE, "P must be in [0,%d]", CSA2_MAX_K);
    CSA2_REQUIRE(a->P == 0 || a->P >= a->K, CSA2_ERR_SHAPE, "P must be >= K");
    CSA2_REQUIRE(a->P == 0 || (a->pool_out && a->pool_count_out), CSA2_ERR_NULL,
                 "FULL with P > 0 needs pool_out and pool_count_out");
  } else {
    CSA2_REQUIRE(!a->pool_in || (a->pool_count_in && a->P_in >= 1), CSA2_ERR_SHAPE,
                 "pool_in needs pool_count_in and P_in >= 1");
  }
  return CSA2_OK;
}

}  // namespace

size_t csa2_workspace_bytes(csa2_mode mode, const csa2_layer_args* a) {
  if (check_step(mode, a) != CSA2_OK) return 0;
  return step_bytes(mode, a);
}

csa2_status csa2_layer_step(csa2_mode mode, const csa2_layer_args* a, void* ws, size_t ws_bytes,
                            void* stream) {
  g_last_error.clear();
  csa2_status s = check_step(mode, a);
  if (s) return s;
  const size_t need = step_bytes(mode, a);
  CSA2_REQUIRE(ws && ws_bytes >= need, CSA2_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)",
               need, ws_bytes);
  const StepLayout L = step_layout(mode, a, ws);
  const hipStream_t st = as_stream(stream);
  const int32_t rows = a->B * a->T;
  const int32_t Weff = (a->S > 0) ? a->W : 0;

  // A decode step (one token per sequence, 1, 2 or 4 indexer heads) writes
  // its new rows inside the scan launch; otherwise they are quantized first.
  const bool fresh_in_scan =
      mode == CSA2_MODE_FULL && fresh_rows_supported(false, a->T, a->H_I, a->D_I, a->D);
  if (mode == CSA2_MODE_FULL && !fresh_in_scan)
    CSA2_LAUNCH(0, PROF_STREAM, launch_quantize_step(a->new_kv, a->new_ikey, a->new_dtype == CSA2_BF16, rows, a->T,
                                  a->q_pos, a->D, a->kv.cap, a->kv.codes, a->kv.scales, a->D_I,
                                  a->icache.cap, a->icache.codes, a->icache.scales, st),
             "quantize-on-write launch");

  for (int32_t r0 = 0; r0 < rows; r0 += L.rc) {
    const int32_t nr = std::min(L.rc, rows - r0);
    // Row r0+j of this pass is row j of every per-pass buffer; the kernels
    // see the pass as B' = nr / T' sequences only when T divides it, so the
    // sequence index is recovered from the absolute row below.
    const int32_t* qpos = a->q_pos + r0;
    if (mode != CSA2_MODE_REUSE) {
      const bool pooled_in = (mode == CSA2_MODE_REINDEX && a->pool_in);
      const uint16_t* qi = a->q_idx + (size_t)r0 * a->H_I * a->D_I;
      const float* wi = a->w_idx + (size_t)r0 * a->H_I;
      const int32_t* nvp = pooled_in ? a->pool_count_in + r0 : qpos;
      const int32_t nv_add = pooled_in ? 0 : 1;
      const int32_t* pool = pooled_in ? a->pool_in + (size_t)r0 * a->P_in : nullptr;
      const int64_t n_max = pooled_in ? a->P_in : a->icache.cap;
      // one Top-K block per row (many rows, no pool kept): no score histogram
      const bool row = !(mode == CSA2_MODE_FULL && a->P > 0) && topk_row_pass(nr, n_max);
      NewRows fresh;
      if (fresh_in_scan) {
        const size_t esz = a->new_dtype == CSA2_BF16 ? 2 : 4;
        fresh.kv = static_cast<const char*>(a->new_kv) + (size_t)r0 * a->D * esz;
        fresh.ikey = static_cast<const char*>(a->new_ikey) + (size_t)r0 * a->D_I * esz;
        fresh.bf16 = a->new_dtype == CSA2_BF16;
        fresh.q_pos = qpos;
        fresh.kv_codes = a->kv.codes;
        fresh.kv_scales = a->kv.scales;
        fresh.kv_cap = a->kv.cap;
        fresh.kv_dim = a->D;
      }
      int32_t* idx = a->idx_out + (size_t)r0 * a->K;
      // Prefill passes over long contexts select without a score matrix: a
      // sampled threshold, the candidates above it, the exact Top-K among
      // them, and the exact path for any row that needs it (the sample
      // lives in the kept-position region, the candidates in the candidate
      // region and the per-row words in the count region of the Top-K
      // workspace, none of which the exact path of these passes touches).
      if (L.sampled) {
        SampledSel sel;
        sel.samp = reinterpret_cast<float*>(L.tw.above);
        sel.ns_stride = L.tw.above_stride;
        sel.cand = reinterpret_cast<uint2*>(L.tw.cand);
        sel.thr = L.tw.counts;
        sel.count = L.tw.counts + nr;
        sel.fail = L.tw.counts + 2 * (size_t)nr;
        const bool force_fail = topk_variant_forced() == kTopkSampledFallback;
        const uint8_t* ic = a->icache.codes;
        const uint8_t* isc = a->icache.scales;
        CSA2_LAUNCH(1, PROF_STREAM, launch_index_sample(ic, isc, a->D_I, a->icache.cap, nr, a->T, qi, wi,
                                                        a->H_I, nvp, nv_add, n_max, sel, st, r0),
                    "index sample launch");
        CSA2_LAUNCH(2, PROF_STREAM, launch_sample_threshold(nr, nvp, nv_add, n_max, a->K, sel, force_fail, st),
                    "sample threshold launch");
        CSA2_LAUNCH(1, PROF_STREAM, launch_index_candidates(ic, isc, a->D_I, a->icache.cap, nr, a->T, qi, wi,
                                                            a->H_I, nvp, nv_add, n_max, sel, st, r0),
                    "index candidates launch");
        CSA2_LAUNCH(2, PROF_STREAM, launch_sampled_final(nr, nvp, nv_add, n_max, a->K, idx, sel, st),
                    "candidate select launch");
        CSA2_LAUNCH(1, PROF_STREAM, launch_index_score_failed(ic, isc, a->D_I, a->icache.cap, nr, a->T, qi, wi,
                                                              a->H_I, nvp, nv_add, n_max, L.scores,
                                                              L.n_out, sel.fail, st, r0),
                    "index score launch (exact path)");
        CSA2_LAUNCH(2, PROF_STREAM, launch_topk_row_failed(L.scores, nr, L.n_out, nvp, nv_add, a->K, idx,
                                                           sel.fail, st),
                    "top-k select launch (exact path)");
        set_topk_last(force_fail ? kTopkSampledFallback : kTopkSampled);
      } else {
      CSA2_LAUNCH(1, PROF_STREAM, launch_index_score(a->icache.codes, a->icache.scales, a->D_I, a->icache.cap, nr, a->T,
                                  qi, wi, a->H_I, nvp, nv_add, pool, pooled_in ? a->P_in : 0, n_max,
                                  L.scores, L.n_out, row ? nullptr : L.tw.hist, L.tw.hist_stride,
                                  L.tw.hist_copies, st, r0, fresh_in_scan ? &fresh : nullptr),
               "index score launch");
      if (mode == CSA2_MODE_FULL && a->P > 0) {
        int32_t* pool_out = a->pool_out + (size_t)r0 * a->P;
        int32_t* pcount = a->pool_count_out + r0;
        // the pool's scores gathered into a dense row (with the histogram its
        // selection starts from, unless it takes one block per row): by the
        // one-wait selection itself as it writes the pool, else by a kernel
        const bool prow = topk_row_pass(nr, a->P);
        bool gathered = false;
        CSA2_LAUNCH(2, PROF_STREAM, launch_topk_select(L.scores, nr, L.n_out, qpos, 1, n_max, nullptr, a->P, pool_out,
                                    pcount, L.tw, st, false, prow ? L.pscores : nullptr, &gathered),
                 "pool select launch");
        if (!gathered)
          CSA2_LAUNCH(4, PROF_STREAM, launch_gather_scores(L.scores, L.n_out, pool_out, a->P, pcount, nr, L.pscores,
                                        prow ? nullptr : L.tw.hist, L.tw.hist_stride, L.tw.hist_copies, st),
                   "pool gather launch");
        CSA2_LAUNCH(2, PROF_STREAM, launch_topk_select(L.pscores, nr, a->P, pcount, 0, a->P, pool_out, a->K, idx,
                                    nullptr, L.tw, st, prow),
                 "top-k select launch");
      } else {
        CSA2_LAUNCH(2, PROF_STREAM, launch_topk_select(L.scores, nr, L.n_out, nvp, nv_add, n_max,
                                    pooled_in ? pool : nullptr, a->K, idx, nullptr, L.tw, st, row),
                 "top-k select launch");
      }
      }
    }
    // attention in sub-passes of at most kAttnPassRows rows, so a long
    // pass's partials stay within the last-level cache for the merge
    for (int32_t a0 = r0; a0 < r0 + nr; a0 += kAttnPassRows) {
      const int32_t na = std::min(kAttnPassRows, r0 + nr - a0);
      const int32_t* idx_att = (mode == CSA2_MODE_REUSE ? a->idx_in : a->idx_out) + (size_t)a0 * a->K;
      CSA2_LAUNCH(3, PROF_STREAM, launch_sparse_attn(a->q + (size_t)a0 * a->H * a->D, na, a->T, a->D, a->dv, a->kv.codes,
                                  a->kv.scales, a->kv.cap, idx_att, a->K, a->swa, a->swa_scale,
                                  a->swa_pos0, a->S, Weff, a->q_pos + a0, a->sm_scale,
                                  a->out + (size_t)a0 * a->H * a->dv,
                                  a->lse ? a->lse + (size_t)a0 * a->H : nullptr, L.aw, st, a0),
               "sparse attention launch");
    }
  }
  return CSA2_OK;
}

csa2_status csa2_layer_step_static(csa2_mode mode, const csa2_layer_args* a, void* stream) {
  g_last_error.clear();
  csa2_status s = check_step(mode, a);
  if (s) return s;
  const size_t need = step_bytes(mode, a);
  CSA2_REQUIRE(need <= kStaticScratchBytes, CSA2_ERR_WORKSPACE,
               "this step needs %zu bytes of scratch, more than the static scratch's %zu; "
               "call csa2_layer_step with a workspace instead",
               need, kStaticScratchBytes);
  int dev = -1;
  void* ws = nullptr;
  s = static_scratch(as_stream(stream), &dev, &ws);
  if (s) return s;
  s = csa2_layer_step(mode, a, ws, kStaticScratchBytes, stream);
  if (s == CSA2_ERR_HIP) {  // launches may have stopped part-way: clear before the next use
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    g_scratch[dev].clean = false;
  }
  return s;
}

}  // extern "C"
