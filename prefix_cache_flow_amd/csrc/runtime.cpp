// C ABI of the policy step (include/vla.h): handles, validation, weight layout,
// workspace planning, the prefix and solver sequences, and the per-shape HIP
// graph cache of the solver loop.
//
// The paper (vla.cpp, arXiv 2606.08094, §III-B) keeps the observation's cached
// conditioning for the solver steps of one request, refreshes it on each new
// observation, and keeps graphs and buffers for unchanged shapes across
// requests; here a K/V cache handle is the conditioning of one encode call, the
// model owns a workspace that grows to the largest shape seen, and the solver
// loop is captured once per (cache storage, batch, prefix length, steps) and
// replayed.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <set>
#include <string>
#include <tuple>
#include <vector>

#include "../../include/vla.h"
#include "../../include/vla_probe.h"
#include "kernels.h"

using namespace vla;

// ============================================================== errors
static thread_local std::string g_last_error;

static vla_status fail(vla_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

#define HIP_TRY(expr)                                                                                   \
  do {                                                                                                  \
    hipError_t e_ = (expr);                                                                             \
    if (e_ != hipSuccess)                                                                               \
      return fail(e_ == hipErrorOutOfMemory ? VLA_ERR_OUT_OF_MEMORY : VLA_ERR_DEVICE,                    \
                  std::string(#expr) + ": " + hipGetErrorString(e_));                                   \
  } while (0)

extern "C" const char* vla_status_string(vla_status s) {
  switch (s) {
    case VLA_OK: return "VLA_OK";
    case VLA_ERR_INVALID_ARGUMENT: return "VLA_ERR_INVALID_ARGUMENT";
    case VLA_ERR_SHAPE_MISMATCH: return "VLA_ERR_SHAPE_MISMATCH";
    case VLA_ERR_INVALID_HANDLE: return "VLA_ERR_INVALID_HANDLE";
    case VLA_ERR_UNSUPPORTED: return "VLA_ERR_UNSUPPORTED";
    case VLA_ERR_OUT_OF_MEMORY: return "VLA_ERR_OUT_OF_MEMORY";
    case VLA_ERR_DEVICE: return "VLA_ERR_DEVICE";
  }
  return "VLA_ERR_UNKNOWN";
}

extern "C" const char* vla_last_error(void) { return g_last_error.c_str(); }

// ============================================================== allocation fault injection
// Every device and pinned-host allocation of the library goes through
// lib_malloc / lib_host_malloc.  With VLA_FAIL_ALLOC=n in the environment the
// n-th allocation after the variable was (re)set fails as if memory were
// exhausted (n <= 0 or unset: none fails), so tests can walk every
// out-of-memory path.  The variable is read at every allocation; a changed
// value restarts the count.
static std::mutex g_inject_mu;
static std::string g_inject_env;
static long g_inject_count = 0;

static bool inject_failure() {
  const char* v = getenv("VLA_FAIL_ALLOC");
  std::lock_guard<std::mutex> g(g_inject_mu);
  const std::string cur = v ? v : "";
  if (cur != g_inject_env) {
    g_inject_env = cur;
    g_inject_count = 0;
  }
  if (cur.empty()) return false;
  const long n = strtol(cur.c_str(), nullptr, 10);
  return n > 0 && ++g_inject_count == n;
}

static hipError_t lib_malloc(void** p, size_t bytes) {
  *p = nullptr;
  if (inject_failure()) return hipErrorOutOfMemory;
  return hipMalloc(p, bytes);
}

static hipError_t lib_host_malloc(void** p, size_t bytes) {
  *p = nullptr;
  if (inject_failure()) return hipErrorOutOfMemory;
  return hipHostMalloc(p, bytes);
}

// ============================================================== config
static bool pos(int v) { return v > 0; }

static vla_status check_config(const vla_model_config* c) {
  if (!c) return fail(VLA_ERR_INVALID_ARGUMENT, "config is NULL");
  if (c->abi_version != VLA_ABI_VERSION) return fail(VLA_ERR_UNSUPPORTED, "abi_version mismatch");
  if (c->precision < VLA_F32 || c->precision > VLA_W2A8_BF16) return fail(VLA_ERR_INVALID_ARGUMENT, "bad precision");
  const int v[] = {c->d_p, c->L_p, c->Hq, c->Hkv, c->hd, c->F_p, c->d_e, c->L_e, c->Hq_e, c->Hkv_e, c->hd_e, c->F_e, c->H, c->d_a};
  for (int x : v)
    if (!pos(x)) return fail(VLA_ERR_INVALID_ARGUMENT, "every model dimension must be positive");
  if (!(c->rms_eps >= 0.f) || !std::isfinite(c->rms_eps)) return fail(VLA_ERR_INVALID_ARGUMENT, "rms_eps must be >= 0");
  if (c->Hq % c->Hkv || c->Hq_e % c->Hkv_e) return fail(VLA_ERR_UNSUPPORTED, "query heads must be a multiple of kv heads");
  if (c->d_a > 256) return fail(VLA_ERR_UNSUPPORTED, "d_a > 256");
  if (c->precision == VLA_F32) {
    if ((c->hd != 32 && c->hd != 64) || (c->hd_e != 32 && c->hd_e != 64))
      return fail(VLA_ERR_UNSUPPORTED, "fp32 models need head widths 32 or 64");
    if (c->d_p % 16 || c->d_e % 16 || c->F_p % 16 || c->F_e % 16 || (c->Hq * c->hd) % 16 || (c->Hq_e * c->hd_e) % 16)
      return fail(VLA_ERR_UNSUPPORTED, "fp32 model widths must be multiples of 16");
  } else {
    auto hd_ok = [](int h) { return h == 64 || h == 128 || h == 256; };
    if (!hd_ok(c->hd) || !hd_ok(c->hd_e)) return fail(VLA_ERR_UNSUPPORTED, "head widths must be 64, 128 or 256");
    if (c->d_p % 64 || c->d_e % 64 || c->F_p % 64 || c->F_e % 64)
      return fail(VLA_ERR_UNSUPPORTED, "model widths must be multiples of 64");
    if (c->d_e > 4096) return fail(VLA_ERR_UNSUPPORTED, "d_e > 4096");
    if (c->precision == VLA_W2A8_BF16 && (c->d_p % 128 || c->F_p % 128 || (c->Hq * c->hd) % 128))
      return fail(VLA_ERR_UNSUPPORTED, "ternary prefix widths must be multiples of 128");
  }
  // the residual + RMSNorm row kernel holds rows of up to 4096 columns and sums
  // up to 16 split-K partials; the chunk-sized GEMM splits K in 1024-wide
  // chunks, so the inputs of its partial products stay at 16384 or below
  if (c->d_p > 4096) return fail(VLA_ERR_UNSUPPORTED, "d_p > 4096");
  if (c->F_p > 16384 || c->F_e > 16384 || (int64_t)c->Hq * c->hd > 16384 || (int64_t)c->Hq_e * c->hd_e > 16384)
    return fail(VLA_ERR_UNSUPPORTED, "F_p, F_e, Hq*hd and Hq_e*hd_e must be at most 16384");
  if (c->attn_mode != VLA_ATTN_CROSS && c->attn_mode != VLA_ATTN_JOINT)
    return fail(VLA_ERR_INVALID_ARGUMENT, "bad attn_mode");
  if (c->attn_mode == VLA_ATTN_JOINT) {
    if (c->L_e != c->L_p || c->Hkv_e != c->Hkv || c->hd_e != c->hd)
      return fail(VLA_ERR_SHAPE_MISMATCH, "joint attention needs L_e == L_p, Hkv_e == Hkv and hd_e == hd");
    if (c->precision == VLA_W2A8_BF16) return fail(VLA_ERR_UNSUPPORTED, "joint attention with a ternary prefix");
  }
  return VLA_OK;
}

// Tensor order of the boundary: (rows, cols, kind) with kind 0 gain, 1 linear, 2 ternary.
struct Spec {
  int64_t rows, cols;
  int kind;
};

static std::vector<Spec> specs(const vla_model_config* c) {
  std::vector<Spec> s;
  const int lp = c->precision == VLA_W2A8_BF16 ? 2 : 1;
  auto lin_p = [&](int64_t r, int64_t k) { s.push_back({r, lp == 2 ? k / 4 : k, lp}); };
  const int64_t qw = (int64_t)c->Hq * c->hd, kvw = (int64_t)c->Hkv * c->hd;
  const int64_t qe = (int64_t)c->Hq_e * c->hd_e, kve = (int64_t)c->Hkv_e * c->hd_e;
  for (int l = 0; l < c->L_p; ++l) {
    s.push_back({c->d_p, 1, 0});
    lin_p(qw, c->d_p);
    lin_p(kvw, c->d_p);
    lin_p(kvw, c->d_p);
    lin_p(c->d_p, qw);
    s.push_back({c->d_p, 1, 0});
    lin_p(c->F_p, c->d_p);
    lin_p(c->F_p, c->d_p);
    lin_p(c->d_p, c->F_p);
  }
  const bool joint = c->attn_mode == VLA_ATTN_JOINT;
  if (!joint) {
    s.push_back({c->d_p, 1, 0});
    for (int e = 0; e < c->L_e; ++e) {
      s.push_back({kve, c->d_p, 1});
      s.push_back({kve, c->d_p, 1});
    }
  }
  s.push_back({c->d_e, c->d_a, 1});
  for (int e = 0; e < c->L_e; ++e) {
    s.push_back({c->d_e, 1, 0});
    s.push_back({qe, c->d_e, 1});
    s.push_back({kve, c->d_e, 1});
    s.push_back({kve, c->d_e, 1});
    s.push_back({c->d_e, qe, 1});
    if (!joint) {
      s.push_back({c->d_e, 1, 0});
      s.push_back({qe, c->d_e, 1});
      s.push_back({c->d_e, qe, 1});
    }
    s.push_back({c->d_e, 1, 0});
    s.push_back({c->F_e, c->d_e, 1});
    s.push_back({c->F_e, c->d_e, 1});
    s.push_back({c->d_e, c->F_e, 1});
  }
  s.push_back({c->d_e, 1, 0});
  s.push_back({c->d_a, c->d_e, 1});
  return s;
}

extern "C" int32_t vla_n_tensors(const vla_model_config* cfg) {
  if (check_config(cfg) != VLA_OK) return -1;
  return (int32_t)specs(cfg).size();
}

extern "C" vla_status vla_tensor_info(const vla_model_config* cfg, int32_t index, int64_t* rows, int64_t* cols,
                                      int32_t* kind) {
  vla_status st = check_config(cfg);
  if (st != VLA_OK) return st;
  auto s = specs(cfg);
  if (index < 0 || index >= (int32_t)s.size()) return fail(VLA_ERR_INVALID_ARGUMENT, "tensor index out of range");
  if (rows) *rows = s[index].rows;
  if (cols) *cols = s[index].cols;
  if (kind) *kind = s[index].kind;
  return VLA_OK;
}

// ============================================================== model
static const uint32_t MODEL_MAGIC = 0x564c414du;  // "VLAM"
static const uint32_t CACHE_MAGIC = 0x564c414bu;  // "VLAK"

struct PrefixLayer {
  float* w1 = nullptr;
  float* w2 = nullptr;
  void* wqkv = nullptr;  // [(Hq + 2 Hkv) hd][d_p]   bf16 / fp32 / packed words
  void* wo = nullptr;    // [d_p][Hq hd]
  void* wgu = nullptr;   // [2 F_p][d_p], gate/up interleaved in blocks of 16 rows
  void* wd = nullptr;    // [d_p][F_p]
  float *bqkv = nullptr, *bo = nullptr, *bgu = nullptr, *bd = nullptr;  // ternary scales per output row
};

struct ExpertLayer {
  float *a1 = nullptr, *a2 = nullptr, *a3 = nullptr;
  void* wqkv = nullptr;  // [(Hq_e + 2 Hkv_e) hd_e][d_e]
  void* wos = nullptr;   // [d_e][Hq_e hd_e]
  void* wqc = nullptr;   // [Hq_e hd_e][d_e]
  void* woc = nullptr;   // [d_e][Hq_e hd_e]
  void* wgu = nullptr;   // [2 F_e][d_e] interleaved
  void* wd = nullptr;    // [d_e][F_e]
};

// A captured solver loop bakes in the cache storage and its lengths array, so
// those are part of its key.  The model keeps the kMaxGraphs most recently
// used graphs and destroys older ones (a caller that encodes every observation
// into fresh storage would otherwise grow the set without bound).
struct GraphKey {
  const void* kv;
  const int* lens;
  int B, N, steps;
  bool operator<(const GraphKey& o) const {
    return std::tie(kv, lens, B, N, steps) < std::tie(o.kv, o.lens, o.B, o.N, o.steps);
  }
};
static const size_t kMaxGraphs = 8;
struct GraphEntry {
  hipGraphExec_t exec;
  uint64_t last_use;
};

struct vla_model {
  uint32_t magic = MODEL_MAGIC;
  vla_model_config cfg{};
  int device = 0;
  bool f32 = false, w2a8 = false, joint = false;
  std::vector<void*> allocs;  // every device allocation of weights
  std::vector<PrefixLayer> pl;
  std::vector<ExpertLayer> el;
  float* w_pf = nullptr;
  void* wcache = nullptr;  // [L_e 2 Hkv_e hd_e][d_p]
  void* w_in = nullptr;
  float* w_ef = nullptr;
  void* w_out = nullptr;
  // workspace
  char* ws = nullptr;
  size_t ws_bytes = 0;
  float* sched_dev = nullptr;  // [max_steps + 1]
  float* sched_host = nullptr; // pinned staging
  int sched_cap = 0;
  std::vector<float> sched_last;     // what sched_dev holds (empty: unknown)
  hipStream_t sched_stream = nullptr;  // the stream that wrote it
  hipStream_t cap_stream = nullptr;
  // expert weights of all layers in one allocation, layer e at ew + e * ew_layer
  char* ew = nullptr;
  size_t ew_layer = 0;
  std::map<GraphKey, GraphEntry> graphs;
  uint64_t graph_clock = 0;
  std::set<vla_kv_cache*> caches;
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  int64_t plan_rows = 0, plan_erows = 0;  // largest prefix / chunk row counts seen
  int64_t plan_kvrows = 0;                 // largest batch x padded prefix length seen
  // persistent solver step (fused.hip): per-layer gains in one array, barrier words, error word
  bool fused = false;
  // The chunk-sized chain folds the expert's norms into its products unless the
  // model was created with VLA_FOLD=0 in the environment (then it runs them as
  // row kernels, in the persistent step's summation order)
  bool fold = true;
  // Absorbed cross attention (batch-1 encodes): the encode also forms each
  // layer's Wq^T K^T and V Wo^T, and the solver runs each cross sublayer as two
  // products; off with VLA_ABSORB=0 in the environment at creation.  wqT holds
  // every layer's cross-query weights transposed, [L_e][d_e][Hq_e hd_e].
  bool absorb = false;
  uint16_t* wqT = nullptr;
  float* egains = nullptr;
  unsigned* fbar = nullptr;
  unsigned* ferr = nullptr;
  int ncu = 0;
  std::map<int, int> fused_occ;  // occupancy per (hd_e, row blocks)
  // kernel probe
  int probe_kind = 0, probe_max = 0, probe_used = 0, probe_repeat = 1;
  std::vector<hipEvent_t> probe_ev;
  hipStream_t probe_stream = nullptr;
};

struct vla_kv_cache {
  uint32_t magic = CACHE_MAGIC;
  vla_model* model = nullptr;
  int B = 0, N = 0;
  void* storage = nullptr;
  int* lens = nullptr;  // per-observation prefix lengths, in the storage's tail
  // absorbed cross-attention products after the lengths (null: none), layer l
  // at + l * ab_ls elements: Wqk [Hq_e Np][d_e] and Wvo [d_e][Hq_e Np]
  uint16_t* wqk = nullptr;
  uint16_t* wvo = nullptr;
  long ab_ls = 0;
};

static std::mutex g_mu;
static std::set<vla_model*> g_models;

static bool live_model(const vla_model* m) {
  std::lock_guard<std::mutex> g(g_mu);
  return m && g_models.count(const_cast<vla_model*>(m)) && m->magic == MODEL_MAGIC;
}

static bool live_cache(const vla_kv_cache* k) {
  if (!k) return false;
  std::lock_guard<std::mutex> g(g_mu);
  for (vla_model* m : g_models)
    if (m->caches.count(const_cast<vla_kv_cache*>(k))) return k->magic == CACHE_MAGIC;
  return false;
}

static vla_status check_device() {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    return fail(VLA_ERR_DEVICE, "no HIP device");
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(VLA_ERR_DEVICE, "hipGetDevice failed");
  hipDeviceProp_t p;
  if (hipGetDeviceProperties(&p, dev) != hipSuccess) return fail(VLA_ERR_DEVICE, "hipGetDeviceProperties failed");
  if (strncmp(p.gcnArchName, "gfx950", 6) != 0)
    return fail(VLA_ERR_DEVICE, std::string("this library is built for gfx950, device is ") + p.gcnArchName);
  return VLA_OK;
}

static size_t elt(const vla_model* m) { return m->f32 ? 4 : 2; }

static vla_status dev_alloc(vla_model* m, void** p, size_t bytes) {
  *p = nullptr;
  if (bytes == 0) bytes = 16;
  hipError_t e = lib_malloc(p, bytes);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(VLA_ERR_OUT_OF_MEMORY, "hipMalloc of " + std::to_string(bytes) + " bytes failed");
  }
  m->allocs.push_back(*p);
  return VLA_OK;
}

static void free_model(vla_model* m) {
  for (auto& kv : m->graphs) (void)hipGraphExecDestroy(kv.second.exec);
  m->graphs.clear();
  for (void* p : m->allocs) (void)hipFree(p);
  m->allocs.clear();
  if (m->ws) (void)hipFree(m->ws);
  if (m->sched_dev) (void)hipFree(m->sched_dev);
  if (m->sched_host) (void)hipHostFree(m->sched_host);
  if (m->egains) (void)hipFree(m->egains);
  if (m->fbar) (void)hipFree(m->fbar);
  if (m->ferr) (void)hipFree(m->ferr);
  if (m->cap_stream) (void)hipStreamDestroy(m->cap_stream);
  if (m->ev0) (void)hipEventDestroy(m->ev0);
  if (m->ev1) (void)hipEventDestroy(m->ev1);
  for (hipEvent_t e : m->probe_ev) (void)hipEventDestroy(e);
  m->magic = 0;
  delete m;
}

// ---- weight copy helpers (all on `s`)
struct Src {
  const void* const* t;
  int i = 0;
  const float* beta;
  int bi = 0;
};

// Source tensors may live in device memory or in host memory (pageable or
// pinned): every copy below names no direction (hipMemcpyDefault), and the one
// kernel that reads a source directly (the ternary repack) gets a device copy
// of a host tensor first.
static bool on_device(const void* p) {
  hipPointerAttribute_t a{};
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();  // unknown to HIP: plain host memory
    return false;
  }
  return a.type == hipMemoryTypeDevice || a.type == hipMemoryTypeManaged;
}

// copy rows of a linear weight, converting fp32 -> bf16 is never needed (the
// caller gives the precision's own type), into dst at row offset `row0`
static vla_status put_rows(vla_model* m, void* dst, int64_t row0, const void* src, int64_t rows, int64_t cols,
                           hipStream_t s) {
  const size_t es = elt(m);
  HIP_TRY(hipMemcpyAsync((char*)dst + row0 * cols * es, src, rows * cols * es, hipMemcpyDefault, s));
  return VLA_OK;
}

// interleave gate and up [F][cols] into [2F][cols] in blocks of 16 rows
static vla_status put_interleaved(void* dst, const void* g, const void* u, int64_t F, size_t row_bytes, hipStream_t s) {
  const size_t blk = 16 * row_bytes;
  HIP_TRY(hipMemcpy2DAsync(dst, 2 * blk, g, blk, blk, F / 16, hipMemcpyDefault, s));
  HIP_TRY(hipMemcpy2DAsync((char*)dst + blk, 2 * blk, u, blk, blk, F / 16, hipMemcpyDefault, s));
  return VLA_OK;
}

static vla_status put_gain(vla_model* m, float** dst, const void* src, int64_t n, hipStream_t s) {
  vla_status st = dev_alloc(m, (void**)dst, n * 4);
  if (st != VLA_OK) return st;
  HIP_TRY(hipMemcpyAsync(*dst, src, n * 4, hipMemcpyDefault, s));
  return VLA_OK;
}

// ternary: canonical bytes -> library words at row offset (rows of K/16 words)
static vla_status put_ternary(uint32_t* dst, int64_t row0, const void* src, int64_t rows, int64_t K, int* flags,
                              hipStream_t s) {
  if (on_device(src)) {
    HIP_TRY(ternary_repack((const uint8_t*)src, (int)rows, (int)K, dst + row0 * (K / 16), flags, s));
    return VLA_OK;
  }
  // host tensor: through a device copy, freed once the repack has run
  void* d = nullptr;
  const size_t bytes = (size_t)rows * K / 4;
  if (lib_malloc(&d, bytes) != hipSuccess) {
    (void)hipGetLastError();
    return fail(VLA_ERR_OUT_OF_MEMORY, "ternary source staging");
  }
  hipError_t e = hipMemcpyAsync(d, src, bytes, hipMemcpyDefault, s);
  if (e == hipSuccess) e = ternary_repack((const uint8_t*)d, (int)rows, (int)K, dst + row0 * (K / 16), flags, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  (void)hipFree(d);
  if (e != hipSuccess) return fail(VLA_ERR_DEVICE, std::string("ternary upload: ") + hipGetErrorString(e));
  return VLA_OK;
}

static vla_status build_weights(vla_model* m, const vla_weights* w, hipStream_t s) {
  const vla_model_config& c = m->cfg;
  Src src{w->tensors, 0, w->ternary_beta, 0};
  const size_t es = elt(m);
  const int64_t qw = (int64_t)c.Hq * c.hd, kvw = (int64_t)c.Hkv * c.hd, qkvw = qw + 2 * kvw;
  const int64_t qe = (int64_t)c.Hq_e * c.hd_e, kve = (int64_t)c.Hkv_e * c.hd_e, qkve = qe + 2 * kve;
  vla_status st;
  int* flags = nullptr;
  std::vector<void*> temps;
  auto cleanup = [&]() {
    for (void* p : temps) (void)hipFree(p);
  };
  if (m->w2a8) {
    if (lib_malloc((void**)&flags, 64) != hipSuccess) return fail(VLA_ERR_OUT_OF_MEMORY, "flags");
    temps.push_back(flags);
    if (hipMemsetAsync(flags, 0, 64, s) != hipSuccess) { cleanup(); return fail(VLA_ERR_DEVICE, "memset"); }
  }
#define TRY(x)           \
  do {                   \
    st = (x);            \
    if (st != VLA_OK) {  \
      cleanup();         \
      return st;         \
    }                    \
  } while (0)
  // Every bf16 projection is assembled row-major in a staging buffer and stored
  // in the MFMA fragment layout (kernels.h, frag_pack): every weight load of a
  // wave is then one contiguous 1 KB.
  const int64_t ncache = m->joint ? 0 : (int64_t)c.L_e * 2 * kve;
  void* stage = nullptr;
  if (!m->f32) {
    int64_t big = std::max<int64_t>(std::max<int64_t>(qkve, 2 * (int64_t)c.F_e) * c.d_e, (int64_t)c.d_e * std::max<int64_t>(qe, c.F_e));
    big = std::max<int64_t>(big, ncache * c.d_p);
    if (!m->w2a8)
      big = std::max<int64_t>(big, std::max<int64_t>(std::max<int64_t>(qkvw, 2 * (int64_t)c.F_p) * c.d_p,
                                                     (int64_t)c.d_p * std::max<int64_t>(qw, c.F_p)));
    if (lib_malloc(&stage, big * es) != hipSuccess) {
      (void)hipGetLastError();
      cleanup();
      return fail(VLA_ERR_OUT_OF_MEMORY, "staging");
    }
    temps.push_back(stage);
  }
  // rows x cols assembled by `fill` (row-major) into a new allocation, fragment layout in bf16
  auto packed_weight = [&](void** dst, int64_t rows, int64_t cols, auto fill) -> vla_status {
    vla_status r = dev_alloc(m, dst, rows * cols * es);
    if (r != VLA_OK) return r;
    if (m->f32) return fill(*dst);
    r = fill(stage);
    if (r != VLA_OK) return r;
    HIP_TRY(frag_pack((const uint16_t*)stage, (int)rows, (int)cols, (uint16_t*)*dst, s));
    return VLA_OK;
  };
  m->pl.resize(c.L_p);
  for (int l = 0; l < c.L_p; ++l) {
    PrefixLayer& P = m->pl[l];
    TRY(put_gain(m, &P.w1, src.t[src.i++], c.d_p, s));
    const void* wq = src.t[src.i++];
    const void* wk = src.t[src.i++];
    const void* wv = src.t[src.i++];
    const void* wo = src.t[src.i++];
    TRY(put_gain(m, &P.w2, src.t[src.i++], c.d_p, s));
    const void* wg = src.t[src.i++];
    const void* wu = src.t[src.i++];
    const void* wd = src.t[src.i++];
    if (!m->w2a8) {
      TRY(packed_weight(&P.wqkv, qkvw, c.d_p, [&](void* d) {
        vla_status r = put_rows(m, d, 0, wq, qw, c.d_p, s);
        if (r == VLA_OK) r = put_rows(m, d, qw, wk, kvw, c.d_p, s);
        if (r == VLA_OK) r = put_rows(m, d, qw + kvw, wv, kvw, c.d_p, s);
        return r;
      }));
      TRY(packed_weight(&P.wo, c.d_p, qw, [&](void* d) { return put_rows(m, d, 0, wo, c.d_p, qw, s); }));
      TRY(packed_weight(&P.wgu, 2 * (int64_t)c.F_p, c.d_p,
                        [&](void* d) { return put_interleaved(d, wg, wu, c.F_p, c.d_p * es, s); }));
      TRY(packed_weight(&P.wd, c.d_p, c.F_p, [&](void* d) { return put_rows(m, d, 0, wd, c.d_p, c.F_p, s); }));
    } else {
      const float bq = src.beta[src.bi++], bk = src.beta[src.bi++], bv = src.beta[src.bi++], bo = src.beta[src.bi++];
      const float bg = src.beta[src.bi++], bu = src.beta[src.bi++], bdn = src.beta[src.bi++];
      TRY(dev_alloc(m, &P.wqkv, qkvw * c.d_p / 4));
      TRY(put_ternary((uint32_t*)P.wqkv, 0, wq, qw, c.d_p, flags, s));
      TRY(put_ternary((uint32_t*)P.wqkv, qw, wk, kvw, c.d_p, flags, s));
      TRY(put_ternary((uint32_t*)P.wqkv, qw + kvw, wv, kvw, c.d_p, flags, s));
      TRY(dev_alloc(m, &P.wo, (int64_t)c.d_p * qw / 4));
      TRY(put_ternary((uint32_t*)P.wo, 0, wo, c.d_p, qw, flags, s));
      // gate/up: repack each, then interleave the word rows
      void *tg = nullptr, *tu = nullptr;
      const int64_t gbytes = (int64_t)c.F_p * c.d_p / 4;
      if (lib_malloc(&tg, gbytes) != hipSuccess || lib_malloc(&tu, gbytes) != hipSuccess) {
        if (tg) (void)hipFree(tg);
        cleanup();
        return fail(VLA_ERR_OUT_OF_MEMORY, "ternary staging");
      }
      temps.push_back(tg);
      temps.push_back(tu);
      TRY(put_ternary((uint32_t*)tg, 0, wg, c.F_p, c.d_p, flags, s));
      TRY(put_ternary((uint32_t*)tu, 0, wu, c.F_p, c.d_p, flags, s));
      TRY(dev_alloc(m, &P.wgu, 2 * gbytes));
      TRY(put_interleaved(P.wgu, tg, tu, c.F_p, c.d_p / 4, s));
      TRY(dev_alloc(m, &P.wd, (int64_t)c.d_p * c.F_p / 4));
      TRY(put_ternary((uint32_t*)P.wd, 0, wd, c.d_p, c.F_p, flags, s));
      // per-output-row scales
      std::vector<float> h;
      auto put_beta = [&](float** dst, const std::vector<float>& v) -> vla_status {
        vla_status r = dev_alloc(m, (void**)dst, v.size() * 4);
        if (r != VLA_OK) return r;
        if (hipMemcpy(*dst, v.data(), v.size() * 4, hipMemcpyHostToDevice) != hipSuccess)
          return fail(VLA_ERR_DEVICE, "beta upload");
        return VLA_OK;
      };
      h.assign(qkvw, bq);
      std::fill(h.begin() + qw, h.begin() + qw + kvw, bk);
      std::fill(h.begin() + qw + kvw, h.end(), bv);
      TRY(put_beta(&P.bqkv, h));
      h.assign(c.d_p, bo);
      TRY(put_beta(&P.bo, h));
      h.assign(2 * (int64_t)c.F_p, bg);
      for (int64_t r = 0; r < 2 * (int64_t)c.F_p; ++r) h[r] = ((r / 16) & 1) ? bu : bg;
      TRY(put_beta(&P.bgu, h));
      h.assign(c.d_p, bdn);
      TRY(put_beta(&P.bd, h));
    }
  }
  if (!m->joint) {
    TRY(put_gain(m, &m->w_pf, src.t[src.i++], c.d_p, s));
    // expert prefix-side projections, concatenated in boundary order: [l][k|v][h][d]
    TRY(packed_weight(&m->wcache, ncache, c.d_p, [&](void* d) {
      vla_status r = VLA_OK;
      for (int e = 0; e < c.L_e && r == VLA_OK; ++e) {
        r = put_rows(m, d, (int64_t)(2 * e) * kve, src.t[src.i++], kve, c.d_p, s);
        if (r == VLA_OK) r = put_rows(m, d, (int64_t)(2 * e + 1) * kve, src.t[src.i++], kve, c.d_p, s);
      }
      return r;
    }));
  }
  TRY(dev_alloc(m, &m->w_in, (int64_t)c.d_e * c.d_a * es));
  TRY(put_rows(m, m->w_in, 0, src.t[src.i++], c.d_e, c.d_a, s));
  // Expert projections (fragment layout in bf16, like the prefix): the chunk
  // has few rows, so these GEMMs are weight streams.
  // all expert projections in one allocation, layer by layer
  auto rnd = [](int64_t b) { return (b + 255) / 256 * 256; };
  // (joint attention has no cross-attention projections: slots 2 and 3 are empty)
  const int64_t njoint = m->joint ? 0 : 1;
  const int64_t shapes[6][2] = {{qkve, c.d_e}, {c.d_e, qe}, {qe * njoint, c.d_e}, {c.d_e * njoint, qe},
                                {2 * (int64_t)c.F_e, c.d_e}, {c.d_e, c.F_e}};
  m->ew_layer = 0;
  for (auto& sh : shapes) m->ew_layer += rnd(sh[0] * sh[1] * (int64_t)es);
  TRY(dev_alloc(m, (void**)&m->ew, m->ew_layer * c.L_e));
  size_t ew_off = 0;
  // rows x cols assembled by `fill` (row-major) into the next slot, fragment layout in bf16
  auto expert_weight = [&](void** dst, int64_t rows, int64_t cols, auto fill) -> vla_status {
    *dst = m->ew + ew_off;
    ew_off += rnd(rows * cols * (int64_t)es);
    vla_status r = VLA_OK;
    if (m->f32) return fill(*dst);
    r = fill(stage);
    if (r != VLA_OK) return r;
    HIP_TRY(frag_pack((const uint16_t*)stage, (int)rows, (int)cols, (uint16_t*)*dst, s));
    return VLA_OK;
  };
  m->el.resize(c.L_e);
  for (int e = 0; e < c.L_e; ++e) {
    ExpertLayer& E = m->el[e];
    TRY(put_gain(m, &E.a1, src.t[src.i++], c.d_e, s));
    const void* wqs = src.t[src.i++];
    const void* wks = src.t[src.i++];
    const void* wvs = src.t[src.i++];
    TRY(expert_weight(&E.wqkv, qkve, c.d_e, [&](void* d) {
      vla_status r = put_rows(m, d, 0, wqs, qe, c.d_e, s);
      if (r == VLA_OK) r = put_rows(m, d, qe, wks, kve, c.d_e, s);
      if (r == VLA_OK) r = put_rows(m, d, qe + kve, wvs, kve, c.d_e, s);
      return r;
    }));
    const void* wos = src.t[src.i++];
    TRY(expert_weight(&E.wos, c.d_e, qe, [&](void* d) { return put_rows(m, d, 0, wos, c.d_e, qe, s); }));
    if (!m->joint) {
      TRY(put_gain(m, &E.a2, src.t[src.i++], c.d_e, s));
      const void* wqc = src.t[src.i++];
      TRY(expert_weight(&E.wqc, qe, c.d_e, [&](void* d) { return put_rows(m, d, 0, wqc, qe, c.d_e, s); }));
      if (m->absorb) {
        // the staging buffer still holds the row-major cross-query weights
        if (!m->wqT) TRY(dev_alloc(m, (void**)&m->wqT, (size_t)c.L_e * c.d_e * qe * 2));
        TRY([&]() -> vla_status {
          HIP_TRY(frag_pack_t((const uint16_t*)stage, (int)qe, c.d_e, m->wqT + (size_t)e * c.d_e * qe, s));
          return VLA_OK;
        }());
      }
      const void* woc = src.t[src.i++];
      TRY(expert_weight(&E.woc, c.d_e, qe, [&](void* d) { return put_rows(m, d, 0, woc, c.d_e, qe, s); }));
    }
    TRY(put_gain(m, &E.a3, src.t[src.i++], c.d_e, s));
    const void* wg = src.t[src.i++];
    const void* wu = src.t[src.i++];
    TRY(expert_weight(&E.wgu, 2 * (int64_t)c.F_e, c.d_e,
                      [&](void* d) { return put_interleaved(d, wg, wu, c.F_e, c.d_e * es, s); }));
    const void* wd = src.t[src.i++];
    TRY(expert_weight(&E.wd, c.d_e, c.F_e, [&](void* d) { return put_rows(m, d, 0, wd, c.d_e, c.F_e, s); }));
  }
  TRY(put_gain(m, &m->w_ef, src.t[src.i++], c.d_e, s));
  TRY(dev_alloc(m, &m->w_out, (int64_t)c.d_a * c.d_e * es));
  TRY(put_rows(m, m->w_out, 0, src.t[src.i++], c.d_a, c.d_e, s));
#undef TRY
  hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    cleanup();
    return fail(VLA_ERR_DEVICE, std::string("weight copy: ") + hipGetErrorString(e));
  }
  if (flags) {
    int hf = 0;
    e = hipMemcpy(&hf, flags, 4, hipMemcpyDeviceToHost);
    if (e != hipSuccess || hf) {
      cleanup();
      return fail(e != hipSuccess ? VLA_ERR_DEVICE : VLA_ERR_INVALID_ARGUMENT,
                  e != hipSuccess ? "flag readback failed" : "ternary weights contain the invalid code 3");
    }
  }
  cleanup();
  return VLA_OK;
}

// The persistent solver step (fused.hip) is opt-in: a model created with
// VLA_FUSED=1 in the environment runs it for bf16 cross-attention experts whose
// chunk-sized GEMMs over d_e take one K chunk (d_e <= 1024); everything else
// runs the kernel chain.  On the single-camera workload the chain is faster
// (0.99 vs 1.23 ms per step): a grid barrier costs about 1.8 us, more than a
// graph kernel boundary, whose launch overlaps the previous kernel's tail.
static vla_status setup_fused(vla_model* m, hipStream_t s) {
  const vla_model_config& c = m->cfg;
  const char* env = getenv("VLA_FUSED");
  // one K chunk for the products over d_e, at most four for those over Hq_e hd_e and F_e
  if (!env || env[0] != '1' || m->f32 || m->joint || c.d_e > 1024 || gemm_chunk_splits(c.Hq_e * c.hd_e, 4) > 4 ||
      gemm_chunk_splits(c.F_e, 4) > 4)
    return VLA_OK;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, m->device) != hipSuccess) return fail(VLA_ERR_DEVICE, "hipGetDeviceProperties");
  m->ncu = prop.multiProcessorCount;
  const size_t gb = (size_t)c.L_e * 3 * c.d_e * 4;
  if (lib_malloc((void**)&m->egains, gb) != hipSuccess ||
      lib_malloc((void**)&m->fbar, fused_barrier_words(c.L_e) * 4) != hipSuccess ||
      lib_malloc((void**)&m->ferr, 256) != hipSuccess) {
    (void)hipGetLastError();
    return fail(VLA_ERR_OUT_OF_MEMORY, "persistent step buffers");
  }
  for (int e = 0; e < c.L_e; ++e) {
    const float* g[3] = {m->el[e].a1, m->el[e].a2, m->el[e].a3};
    for (int i = 0; i < 3; ++i)
      HIP_TRY(hipMemcpyAsync(m->egains + ((size_t)e * 3 + i) * c.d_e, g[i], (size_t)c.d_e * 4, hipMemcpyDeviceToDevice, s));
  }
  HIP_TRY(hipMemsetAsync(m->ferr, 0, 256, s));
  HIP_TRY(hipStreamSynchronize(s));
  m->fused = true;
  return VLA_OK;
}

// Whether the model's batch-1 solver can run the absorbed cross sublayer: bf16
// cross attention with the chunk chain's folded norms (the same shape limits),
// at most 32 query heads, unless VLA_ABSORB=0 is set at creation.
static bool absorb_capable(const vla_model* m) {
  const vla_model_config& c = m->cfg;
  const char* env = getenv("VLA_ABSORB");
  if ((env && env[0] == '0') || m->f32 || m->joint || !m->fold || c.H > 64 || c.Hq_e > 32) return false;
  int used = 0, kc = 0;
  gemm_chunk_plan(c.d_e, 1, &used, &kc);
  const int d8 = c.d_e / 128, qe = c.Hq_e * c.hd_e;
  return used == 1 && c.d_e % 128 == 0 && (d8 == 1 || d8 == 2 || d8 == 4 || d8 == 8) && qe % 32 == 0 &&
         qe <= 4096 && c.F_e % 32 == 0 && c.F_e <= 4096 && (c.hd_e == 64 || c.hd_e == 128 || c.hd_e == 256);
}

extern "C" vla_status vla_model_create(const vla_model_config* cfg, const vla_weights* weights, void* stream,
                                       vla_model** out) {
  if (!out) return fail(VLA_ERR_INVALID_ARGUMENT, "out is NULL");
  *out = nullptr;
  vla_status st = check_config(cfg);
  if (st != VLA_OK) return st;
  if (!weights || !weights->tensors) return fail(VLA_ERR_INVALID_ARGUMENT, "weights are NULL");
  const int n = (int)specs(cfg).size();
  if (weights->n_tensors != n)
    return fail(VLA_ERR_SHAPE_MISMATCH, "expected " + std::to_string(n) + " weight tensors, got " +
                                            std::to_string(weights->n_tensors));
  for (int i = 0; i < n; ++i)
    if (!weights->tensors[i]) return fail(VLA_ERR_INVALID_ARGUMENT, "weight tensor " + std::to_string(i) + " is NULL");
  if (cfg->precision == VLA_W2A8_BF16) {
    if (!weights->ternary_beta) return fail(VLA_ERR_INVALID_ARGUMENT, "ternary_beta is NULL");
    for (int i = 0; i < 7 * cfg->L_p; ++i)
      if (!std::isfinite(weights->ternary_beta[i])) return fail(VLA_ERR_INVALID_ARGUMENT, "non-finite ternary beta");
  }
  st = check_device();
  if (st != VLA_OK) return st;
  vla_model* m = new vla_model();
  m->cfg = *cfg;
  m->f32 = cfg->precision == VLA_F32;
  {
    const char* fe = getenv("VLA_FOLD");
    m->fold = !(fe && fe[0] == '0');
  }
  m->w2a8 = cfg->precision == VLA_W2A8_BF16;
  m->joint = cfg->attn_mode == VLA_ATTN_JOINT;
  m->absorb = absorb_capable(m);
  (void)hipGetDevice(&m->device);
  hipStream_t s = (hipStream_t)stream;
  st = build_weights(m, weights, s);
  if (st == VLA_OK) st = setup_fused(m, s);
  if (m->fused) m->absorb = false;  // the persistent step reads the cached keys and values
  if (st == VLA_OK && (hipStreamCreateWithFlags(&m->cap_stream, hipStreamNonBlocking) != hipSuccess ||
                       hipEventCreate(&m->ev0) != hipSuccess || hipEventCreate(&m->ev1) != hipSuccess))
    st = fail(VLA_ERR_DEVICE, "stream/event creation failed");
  if (st != VLA_OK) {
    free_model(m);
    return st;
  }
  {
    std::lock_guard<std::mutex> g(g_mu);
    g_models.insert(m);
  }
  *out = m;
  return VLA_OK;
}

extern "C" vla_status vla_model_destroy(vla_model* m) {
  {
    std::lock_guard<std::mutex> g(g_mu);
    if (!m || !g_models.count(m) || m->magic != MODEL_MAGIC) return fail(VLA_ERR_INVALID_HANDLE, "unknown model");
    g_models.erase(m);
  }
  (void)hipDeviceSynchronize();
  for (vla_kv_cache* k : m->caches) {
    k->magic = 0;
    delete k;
  }
  m->caches.clear();
  free_model(m);
  return VLA_OK;
}

// Key rows of one K or V block: bf16 blocks hold whole 32-key tiles in the MFMA
// operand orders (padding rows zero), fp32 blocks are plain rows.
static int64_t key_rows(const vla_model* m, int64_t n) { return m->f32 ? n : (n + 31) / 32 * 32; }

// Padded keys per head of the absorbed products an encode of B observations of
// N tokens forms (0: none): one observation, at most 16 key tiles per head and
// 4096 score columns in all, and a chunk of more than one 16-row block (with
// one block the two products take about as long as the three kernels they
// replace, so the encode's extra work would not pay).
static int64_t absorb_np(const vla_model* m, int64_t B, int64_t N) {
  if (!m->absorb || B != 1 || m->cfg.H <= 16) return 0;
  const int64_t np = key_rows(m, N);
  return np / 32 <= 16 && m->cfg.Hq_e * np <= 4096 ? np : 0;
}
// Bytes of those products: per layer Wqk and Wvo (bf16), then every layer's
// values in frag_idx order (the operand the Wvo product reads)
static size_t absorb_bytes(const vla_model* m, int64_t B, int64_t N) {
  const int64_t np = absorb_np(m, B, N);
  const vla_model_config& c = m->cfg;
  return np ? (size_t)c.L_e * (2 * (size_t)c.Hq_e * np * c.d_e + (size_t)c.Hkv_e * np * c.hd_e) * 2 : 0;
}

// ============================================================== workspace
// Byte layout of the model workspace for `rows` prefix tokens and `erows` chunk rows.
struct WS {
  float* h;         // prefix residual [rows][d_p]
  void* u;          // normalized activations [rows][max(d_p, d_e)]
  void* qkv;        // [rows][(Hq + 2 Hkv) hd]; bf16 above 64 rows: queries only, [rows][Hq hd]
  void* pk;         // bf16 prefix keys   [B][Hkv][Np][hd], frag_idx order (Np = N rounded up to 32)
  void* pv;         // bf16 prefix values [B][Hkv][Np][hd], vfrag_idx order
  void* attn;       // [rows][Hq hd]       (fp32 for the ternary prefix)
  void* mlp;        // [rows][F_p]         (fp32 for the ternary prefix)
  int8_t* qa;       // ternary: int8 codes [rows][max(d_p, Hq hd, F_p)]
  float* alpha;     // ternary: [rows]
  W2A8Work w2;      // ternary: K-split partial sums and per-tile counters (zeroed once, left zero)
  float* part;      // split-K partials
  // expert
  float* X;         // [erows][d_a]
  float* E;         // [erows][d_e]
  void* eu;         // [erows][d_e]
  void* eqkv;       // [erows][(Hq_e + 2 Hkv_e) hd_e] (bf16: queries only, [erows][Hq_e hd_e])
  void* ek;         // bf16 chunk keys   [B][Hkv_e][Hp][hd_e], frag_idx order, Hp = H rounded up to 32
  void* ev;         // bf16 chunk values [B][Hkv_e][Hp][hd_e], vfrag_idx order
  void* eq;         // [erows][Hq_e hd_e]
  void* eattn;      // [erows][Hq_e hd_e]
  void* emlp;       // [erows][F_e]
  float* epart;     // split-K partials of the expert
  float* ess;       // folded norms: partial sums of squares of the residual [d_e / 16][64]
  void* esc;        // absorbed cross attention: score weights, bf16 fragment layout [64][<= 4096]
  float* est;       // absorbed cross attention: {max, sum} per row and 32-key block [64][<= 128][2]
  unsigned* sink;   // 64 words for the prefetch kernel
  size_t total;
  // byte sizes of the chunk buffers (bounds of the persistent step's accesses)
  size_t n_E, n_X, n_eu, n_eqkv, n_ekv, n_eattn, n_eq, n_emlp, n_epart;
};

static const int kExpertSplits = 4;

// Split-K counts: the one place that fixes them for a GEMM and for the row
// kernel (or reduction) that sums its partials.
static const int kPrefixChunkSplits = 4;  // split request of the chunk-sized kernel
// kind: the product's epilogue (its split count, and so its workspace, depends on it)
static int prefix_splits(int64_t M, int N, int K, int kind = EPI_PARTIAL) {
  return M <= 64 ? gemm_chunk_splits(K, kPrefixChunkSplits) : gemm_frag_splits((int)M, N, K, 0, kind);
}
static int expert_splits(int64_t M, int N, int K, int kind = EPI_PARTIAL) {
  // chunk-sized kernel up to 64 rows, the 288-row-tile kernel (its own split choice) above
  return M <= 64 ? gemm_chunk_splits(K, kExpertSplits) : gemm_frag_splits((int)M, N, K, 0, kind);
}
// bf16 product with both operands in the fragment layout: the chunk-sized
// kernel up to 64 rows, 288-row tiles above; split counts as prefix_splits
static hipError_t mm_frag(const void* A, const void* W, int64_t M, int N, int K, const Epilogue& e, float* ws,
                          hipStream_t s) {
  if (M <= 64) return gemm_chunk((const uint16_t*)A, (const uint16_t*)W, (int)M, N, K, e, kPrefixChunkSplits, ws, s);
  return gemm_frag((const uint16_t*)A, (const uint16_t*)W, (int)M, N, K, e, 0, ws, s);
}
// floats of split-K partials the prefix (rows tokens) and the expert (erows chunk rows) need
static int64_t prefix_part_floats(const vla_model_config& c, int64_t rows) {
  if (rows <= 0) return 0;
  const int qw = c.Hq * c.hd, qkvw = (c.Hq + 2 * c.Hkv) * c.hd, ncache = c.L_e * 2 * c.Hkv_e * c.hd_e;
  int64_t f = (int64_t)prefix_splits(rows, ncache, c.d_p, EPI_CACHE) * ncache;
  if (c.precision != VLA_W2A8_BF16) {
    f = std::max<int64_t>(f, (int64_t)prefix_splits(rows, qkvw, c.d_p, EPI_QKV) * qkvw);
    f = std::max<int64_t>(f, (int64_t)prefix_splits(rows, c.d_p, qw) * c.d_p);
    f = std::max<int64_t>(f, (int64_t)prefix_splits(rows, c.d_p, c.F_p) * c.d_p);
    f = std::max<int64_t>(f, (int64_t)prefix_splits(rows, 2 * c.F_p, c.d_p, EPI_GEGLU) * 2 * c.F_p);
  }
  return f * rows;
}
static int64_t expert_part_floats(const vla_model_config& c, int64_t erows) {
  if (erows <= 0) return 0;
  const int qe = c.Hq_e * c.hd_e, qkve = (c.Hq_e + 2 * c.Hkv_e) * c.hd_e;
  int64_t f = (int64_t)expert_splits(erows, c.d_e, qe) * c.d_e;
  f = std::max<int64_t>(f, (int64_t)expert_splits(erows, c.d_e, c.F_e) * c.d_e);
  f = std::max<int64_t>(f, (int64_t)expert_splits(erows, qkve, c.d_e, EPI_QKV) * qkve);
  f = std::max<int64_t>(f, (int64_t)expert_splits(erows, qe, c.d_e, EPI_STORE) * qe);
  f = std::max<int64_t>(f, (int64_t)expert_splits(erows, 2 * c.F_e, c.d_e, EPI_GEGLU) * 2 * c.F_e);
  return f * erows;
}

static WS plan(const vla_model* m, int64_t rows, int64_t erows, int64_t kvrows, char* base) {
  const vla_model_config& c = m->cfg;
  const size_t es = elt(m);
  size_t off = 0;
  auto take = [&](size_t bytes) -> char* {
    char* p = base ? base + off : nullptr;
    off += (bytes + 255) / 256 * 256;
    return p;
  };
  WS w{};
  const int64_t qkvw = (int64_t)(c.Hq + 2 * c.Hkv) * c.hd, qw = (int64_t)c.Hq * c.hd;
  const int64_t act_es = m->w2a8 ? 4 : es;  // ternary: fp32 attention / GeGLU outputs feed the quantizer
  // bf16 GEMM inputs are in the fragment layout, whole 16-row blocks (at
  // least 64 rows for the chunk-sized kernel); the ternary prefix keeps fp32 rows
  const int64_t prow = m->f32 ? rows : std::max<int64_t>(64, (rows + 15) / 16 * 16);
  const int64_t arow = m->w2a8 ? rows : prow;
  w.h = (float*)take(rows * c.d_p * 4);
  w.u = take(prow * std::max<int64_t>(c.d_p, c.d_e) * es);
  w.qkv = take(rows * qkvw * es);
  w.pk = take(kvrows * c.Hkv * c.hd * es);
  w.pv = take(kvrows * c.Hkv * c.hd * es);
  w.attn = take(arow * qw * act_es);
  w.mlp = take(arow * (int64_t)c.F_p * act_es);
  if (m->w2a8) {
    w.qa = (int8_t*)take(rows * std::max<int64_t>(std::max<int64_t>(c.d_p, qw), c.F_p));
    w.alpha = (float*)take(rows * 4);
    const int M = (int)rows, Ns[3] = {(int)qkvw, c.d_p, 2 * c.F_p};
    for (int N : Ns) {
      w.w2.ws_bytes = std::max(w.w2.ws_bytes, w2a8_part_bytes(M, N));
      w.w2.ncnt = std::max(w.w2.ncnt, w2a8_counters(M, N));
    }
    w.w2.ws = (int*)take(w.w2.ws_bytes);
    w.w2.cnt = (unsigned*)take((size_t)w.w2.ncnt * 4);
  }
  w.part = (float*)take((size_t)prefix_part_floats(c, rows) * 4);
  const int64_t qe = (int64_t)c.Hq_e * c.hd_e, qkve = (int64_t)(c.Hq_e + 2 * c.Hkv_e) * c.hd_e;
  w.n_X = erows * c.d_a * 4;
  w.n_E = erows * c.d_e * 4;
  w.X = (float*)take(w.n_X);
  w.E = (float*)take(w.n_E);
  // GEMM inputs of the chunk (bf16: fragment layout, whole 16-row blocks, and
  // the chunk-sized kernel reads 1, 2 or 4 of them: at least 64 rows)
  const int64_t frows = m->f32 ? std::max<int64_t>(64, erows) : std::max<int64_t>(64, (erows + 15) / 16 * 16);
  w.n_eu = frows * c.d_e * es;
  w.eu = take(w.n_eu);
  w.n_eqkv = erows * qkve * es;
  w.eqkv = take(w.n_eqkv);
  const int64_t kvblk = c.H > 0 ? erows / c.H * c.Hkv_e * key_rows(m, c.H) * c.hd_e : 0;
  w.n_ekv = kvblk * es;
  w.ek = take(w.n_ekv);
  w.ev = take(w.n_ekv);
  w.n_eq = erows * qe * es;
  w.eq = take(w.n_eq);
  w.n_eattn = frows * qe * es;
  w.eattn = take(w.n_eattn);
  w.n_emlp = frows * (int64_t)c.F_e * es;
  w.emlp = take(w.n_emlp);
  // split partials [S][erows][N] of the expert GEMMs
  w.n_epart = (size_t)expert_part_floats(c, erows) * 4;
  w.epart = (float*)take(w.n_epart);
  w.ess = (float*)take((size_t)std::max(1, c.d_e / 16) * 64 * 4);
  if (m->absorb) {
    // rows past the chunk are never written: zero weights and statistics
    w.esc = take((size_t)64 * 4096 * 2);
    w.est = (float*)take((size_t)64 * 128 * 2 * 4);
  }
  w.sink = (unsigned*)take(256);
  w.total = off;
  return w;
}

static vla_status ensure_ws(vla_model* m, int64_t rows, int64_t erows, int64_t kvrows, WS* out) {
  WS need = plan(m, rows, erows, kvrows, nullptr);
  if (need.total > m->ws_bytes) {
    if (m->ws) {
      hipError_t e = hipDeviceSynchronize();
      if (e != hipSuccess) return fail(VLA_ERR_DEVICE, std::string("sync: ") + hipGetErrorString(e));
      (void)hipFree(m->ws);
      m->ws = nullptr;
      m->ws_bytes = 0;
      for (auto& kv : m->graphs) (void)hipGraphExecDestroy(kv.second.exec);
      m->graphs.clear();
    }
    void* p = nullptr;
    if (lib_malloc(&p, need.total) != hipSuccess) {
      (void)hipGetLastError();
      return fail(VLA_ERR_OUT_OF_MEMORY, "workspace allocation of " + std::to_string(need.total) + " bytes failed");
    }
    // zeroed once, so the padding rows of fragment-layout buffers hold finite values
    if (hipMemset(p, 0, need.total) != hipSuccess) {
      (void)hipGetLastError();
      (void)hipFree(p);
      return fail(VLA_ERR_DEVICE, "workspace clear failed");
    }
    m->ws = (char*)p;
    m->ws_bytes = need.total;
  }
  *out = plan(m, rows, erows, kvrows, m->ws);
  return VLA_OK;
}

// Encode plans prefix rows (and padded key rows), denoise chunk rows; all share
// one arena sized for the largest of each seen so far.
static vla_status get_ws(vla_model* m, int64_t rows, int64_t erows, WS* out, int64_t kvrows = 0) {
  m->plan_rows = std::max(m->plan_rows, rows);
  m->plan_erows = std::max(m->plan_erows, erows);
  m->plan_kvrows = std::max(m->plan_kvrows, kvrows);
  return ensure_ws(m, m->plan_rows, m->plan_erows, m->plan_kvrows, out);
}

// ============================================================== prefix
static vla_status hip_ok(hipError_t e, const char* what) {
  if (e == hipSuccess) return VLA_OK;
  return fail(e == hipErrorOutOfMemory ? VLA_ERR_OUT_OF_MEMORY : VLA_ERR_DEVICE,
              std::string(what) + ": " + hipGetErrorString(e));
}
#define K_TRY(expr, what)                          \
  do {                                             \
    vla_status st_ = hip_ok((expr), what);         \
    if (st_ != VLA_OK) return st_;                 \
  } while (0)

// Bracket one launch of kernel class `kind` with probe events when armed for it.
struct ProbeScope {
  vla_model* m;
  bool on;
  hipStream_t s;
  ProbeScope(vla_model* m_, int kind, hipStream_t s_) : m(m_), on(false), s(s_) {
    if (m->probe_kind == kind && m->probe_used < m->probe_max) {
      on = hipEventRecord(m->probe_ev[2 * m->probe_used], s) == hipSuccess;
    }
  }
  ~ProbeScope() {
    if (on && hipEventRecord(m->probe_ev[2 * m->probe_used + 1], s) == hipSuccess) ++m->probe_used;
  }
  // times the bracketed launch is issued: the probe's repeat count when armed for it, else once
  int reps() const { return on ? m->probe_repeat : 1; }
};

extern "C" vla_status vla_probe_arm(vla_model* m, int32_t kind, int32_t max_launches) {
  return vla_probe_arm_ex(m, kind, max_launches, 1);
}

extern "C" vla_status vla_probe_arm_ex(vla_model* m, int32_t kind, int32_t max_launches, int32_t repeat) {
  if (!live_model(m)) return fail(VLA_ERR_INVALID_HANDLE, "unknown model");
  if (kind < VLA_PROBE_NONE || kind > VLA_PROBE_EXPERT_GATEUP) return fail(VLA_ERR_INVALID_ARGUMENT, "bad probe kind");
  if (max_launches < 0 || max_launches > 100000) return fail(VLA_ERR_INVALID_ARGUMENT, "bad max_launches");
  if (repeat < 1 || repeat > 1000) return fail(VLA_ERR_INVALID_ARGUMENT, "repeat must be in 1..1000");
  m->probe_repeat = repeat;
  while ((int)m->probe_ev.size() < 2 * max_launches) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return fail(VLA_ERR_DEVICE, "event creation failed");
    m->probe_ev.push_back(e);
  }
  m->probe_kind = kind;
  m->probe_max = kind ? max_launches : 0;
  m->probe_used = 0;
  return VLA_OK;
}

extern "C" vla_status vla_probe_read(vla_model* m, float* total_ms, int32_t* launches) {
  if (!live_model(m)) return fail(VLA_ERR_INVALID_HANDLE, "unknown model");
  if (!total_ms || !launches) return fail(VLA_ERR_INVALID_ARGUMENT, "NULL pointer");
  double sum = 0.0;
  for (int i = 0; i < m->probe_used; ++i) {
    K_TRY(hipEventSynchronize(m->probe_ev[2 * i + 1]), "probe sync");
    float ms = 0.f;
    K_TRY(hipEventElapsedTime(&ms, m->probe_ev[2 * i], m->probe_ev[2 * i + 1]), "probe elapsed");
    sum += ms;
  }
  *total_ms = (float)sum;
  *launches = m->probe_used * m->probe_repeat;
  return VLA_OK;
}

static Epilogue epi_store(void* out, int ldo, int out_f32) {
  Epilogue e;
  e.kind = EPI_STORE;
  e.out = out;
  e.ldo = ldo;
  e.out_f32 = out_f32;
  return e;
}

// lens: per-observation prefix lengths on the device (null: every observation
// fills all N positions).  Rows past an observation's length are zeroed on the
// way in, and their keys are masked in the prefix attention.
static vla_status run_prefix(vla_model* m, const void* x, int x_bf16, int B, int N, const int* lens, void* kv,
                             const WS& w, hipStream_t s, uint16_t* ab = nullptr) {
  const vla_model_config& c = m->cfg;
  const int M = B * N;
  const int qw = c.Hq * c.hd, qkvw = (c.Hq + 2 * c.Hkv) * c.hd;
  const float eps = c.rms_eps;
  const int uf = m->f32 ? 1 : 0;
  if (lens || x_bf16) K_TRY(copy_prefix_rows(x, x_bf16, w.h, B, N, c.d_p, lens, s), "copy prefix");
  else K_TRY(copy_f32((const float*)x, w.h, (long)M * c.d_p, s), "copy prefix");
  AttnArgs aa{};
  aa.klen = lens;
  aa.q = w.qkv; aa.q_bs = (long)N * qkvw; aa.q_hs = c.hd; aa.q_rs = qkvw;
  aa.k = (const char*)w.qkv + (size_t)qw * elt(m); aa.k_bs = aa.q_bs; aa.k_hs = c.hd; aa.k_rs = qkvw;
  aa.v = (const char*)w.qkv + (size_t)(qw + c.Hkv * c.hd) * elt(m); aa.v_bs = aa.q_bs; aa.v_hs = c.hd; aa.v_rs = qkvw;
  aa.o = w.attn; aa.o_bs = (long)N * qw; aa.o_rs = qw;
  aa.B = B; aa.Nq = N; aa.Nk = N; aa.Hq = c.Hq; aa.Hkv = c.Hkv; aa.hd = c.hd;
  aa.o_f32 = (m->f32 || m->w2a8) ? 1 : 0;
  // bf16: the fused projection writes query rows and the keys and values in the
  // MFMA operand orders, read by the chunk-style attention kernel, which writes
  // its output in the fragment layout for the O projection
  const bool kvfrag = !m->f32 && !m->w2a8;
  const int Np = (int)key_rows(m, N);
  Epilogue qkv_e = epi_store(w.qkv, qkvw, 0);
  if (kvfrag) {
    qkv_e.kind = EPI_QKV; qkv_e.ldo = qw; qkv_e.nq = qw;
    qkv_e.kout = w.pk; qkv_e.vout = w.pv; qkv_e.hkv = c.Hkv; qkv_e.hd = c.hd; qkv_e.npre = N; qkv_e.npad = Np;
    aa.q_bs = (long)N * qw; aa.q_rs = qw;
    aa.k = w.pk; aa.k_bs = (long)c.Hkv * Np * c.hd; aa.k_hs = (long)Np * c.hd;
    aa.v = w.pv; aa.v_bs = aa.k_bs; aa.v_hs = aa.k_hs;
    aa.o_frag = 1;
    if (Np > N && !m->joint) {  // padding key rows: finite values (zero weights times values)
      K_TRY(zero_tails(w.pk, (long)B * c.Hkv, (long)Np * c.hd, 32 * c.hd, s), "key padding");
      K_TRY(zero_tails(w.pv, (long)B * c.Hkv, (long)Np * c.hd, 32 * c.hd, s), "value padding");
    }
  }
  // Joint attention (the pi0 form): layer l's keys and values are the cache,
  // so the fused projection writes them straight into cache block l (K and V
  // of every KV head, per observation jbs elements apart) and the layer's
  // attention reads them there.  fp32 keeps plain rows.
  const long jbs = (long)c.L_p * 2 * c.Hkv * Np * c.hd;
  if (m->joint) {
    if (m->f32) {
      qkv_e.kind = EPI_QKV; qkv_e.ldo = qw; qkv_e.nq = qw; qkv_e.out_f32 = 1;
      qkv_e.hkv = c.Hkv; qkv_e.hd = c.hd; qkv_e.npre = N; qkv_e.npad = Np;
      aa.q_bs = (long)N * qw; aa.q_rs = qw;
    } else if (Np > N) {
      K_TRY(zero_tails(kv, (long)B * c.L_p * 2 * c.Hkv, (long)Np * c.hd, 32 * c.hd, s), "cache padding");
    }
    qkv_e.kv_bs = jbs;
    aa.k_bs = aa.v_bs = jbs;
    aa.k_hs = aa.v_hs = (long)Np * c.hd;
    aa.k_rs = aa.v_rs = c.hd;
  }
  auto joint_layer = [&](int l) {
    char* kb = (char*)kv + (size_t)l * 2 * c.Hkv * Np * c.hd * elt(m);
    char* vb = kb + (size_t)c.Hkv * Np * c.hd * elt(m);
    qkv_e.kout = kb; qkv_e.vout = vb;
    aa.k = kb; aa.v = vb;
  };

  if (m->w2a8) {
    K_TRY(resid_norm(w.h, c.d_p, nullptr, 0, M, c.d_p, m->pl[0].w1, eps, nullptr, 0, 0, w.qa, w.alpha, s), "norm");
    for (int l = 0; l < c.L_p; ++l) {
      const PrefixLayer& P = m->pl[l];
      Epilogue e = epi_store(w.qkv, qkvw, 0);
      e.alpha = w.alpha; e.beta = P.bqkv;
      {
        ProbeScope ps(m, VLA_PROBE_PREFIX_QKV, s);
        for (int rep = 0; rep < ps.reps(); ++rep)
          K_TRY(gemm_w2a8(w.qa, c.d_p, (const uint32_t*)P.wqkv, M, qkvw, c.d_p, e, s, &w.w2), "qkv");
      }
      K_TRY(attention_bf16(aa, s), "attention");
      K_TRY(quantize_rows((const float*)w.attn, qw, M, qw, w.qa, w.alpha, s), "quantize attn");
      Epilogue r;
      r.kind = EPI_RESID; r.resid = w.h; r.ldr = c.d_p; r.alpha = w.alpha; r.beta = P.bo;
      {
        ProbeScope ps(m, VLA_PROBE_PREFIX_O, s);
        for (int rep = 0; rep < ps.reps(); ++rep)
          K_TRY(gemm_w2a8(w.qa, qw, (const uint32_t*)P.wo, M, c.d_p, qw, r, s, &w.w2), "o proj");
      }
      K_TRY(resid_norm(w.h, c.d_p, nullptr, 0, M, c.d_p, P.w2, eps, nullptr, 0, 0, w.qa, w.alpha, s), "norm");
      Epilogue g;
      g.kind = EPI_GEGLU; g.out = w.mlp; g.ldo = c.F_p; g.out_f32 = 1; g.alpha = w.alpha; g.beta = P.bgu;
      {
        ProbeScope ps(m, VLA_PROBE_PREFIX_GATEUP, s);
        for (int rep = 0; rep < ps.reps(); ++rep)
          K_TRY(gemm_w2a8(w.qa, c.d_p, (const uint32_t*)P.wgu, M, 2 * c.F_p, c.d_p, g, s, &w.w2), "gate/up");
      }
      K_TRY(quantize_rows((const float*)w.mlp, c.F_p, M, c.F_p, w.qa, w.alpha, s), "quantize mlp");
      r.beta = P.bd;
      {
        ProbeScope ps(m, VLA_PROBE_PREFIX_DOWN, s);
        for (int rep = 0; rep < ps.reps(); ++rep)
          K_TRY(gemm_w2a8(w.qa, c.F_p, (const uint32_t*)P.wd, M, c.d_p, c.F_p, r, s, &w.w2), "down");
      }
      if (l + 1 < c.L_p)
        K_TRY(resid_norm(w.h, c.d_p, nullptr, 0, M, c.d_p, m->pl[l + 1].w1, eps, nullptr, 0, 0, w.qa, w.alpha, s),
              "norm");
      else
        K_TRY(resid_norm(w.h, c.d_p, nullptr, 0, M, c.d_p, m->w_pf, eps, w.u, 0, c.d_p, nullptr, nullptr, s, 1), "norm");
    }
  } else {
    K_TRY(resid_norm(w.h, c.d_p, nullptr, 0, M, c.d_p, m->pl[0].w1, eps, w.u, uf, c.d_p, nullptr, nullptr, s, uf ? 0 : 1),
          "norm");
    for (int l = 0; l < c.L_p; ++l) {
      const PrefixLayer& P = m->pl[l];
      const float* next_gain = l + 1 < c.L_p ? m->pl[l + 1].w1 : m->w_pf;
      if (m->joint) joint_layer(l);
      // joint: the last layer's output is never read, only its keys and values
      const bool kv_only = m->joint && l + 1 == c.L_p;
      if (m->f32) {
        K_TRY(gemm_f32((const float*)w.u, c.d_p, (const float*)P.wqkv, c.d_p, M, qkvw, c.d_p,
                       m->joint ? qkv_e : epi_store(w.qkv, qkvw, 1), s), "qkv");
        if (kv_only) break;
        K_TRY(attention_f32(aa, s), "attention");
        Epilogue r;
        r.kind = EPI_RESID; r.resid = w.h; r.ldr = c.d_p;
        K_TRY(gemm_f32((const float*)w.attn, qw, (const float*)P.wo, qw, M, c.d_p, qw, r, s), "o proj");
        K_TRY(resid_norm(w.h, c.d_p, nullptr, 0, M, c.d_p, P.w2, eps, w.u, 1, c.d_p, nullptr, nullptr, s), "norm");
        Epilogue g = epi_store(w.mlp, c.F_p, 1);
        g.kind = EPI_GEGLU;
        K_TRY(gemm_f32((const float*)w.u, c.d_p, (const float*)P.wgu, c.d_p, M, 2 * c.F_p, c.d_p, g, s), "gate/up");
        K_TRY(gemm_f32((const float*)w.mlp, c.F_p, (const float*)P.wd, c.F_p, M, c.d_p, c.F_p, r, s), "down");
        K_TRY(resid_norm(w.h, c.d_p, nullptr, 0, M, c.d_p, next_gain, eps, w.u, 1, c.d_p, nullptr, nullptr, s), "norm");
      } else {
        // every GEMM input in the fragment layout: u from the row kernels, the
        // attention output, the GeGLU output
        {
          ProbeScope ps(m, VLA_PROBE_PREFIX_QKV, s);
          for (int rep = 0; rep < ps.reps(); ++rep)
            K_TRY(mm_frag(w.u, P.wqkv, M, qkvw, c.d_p, qkv_e, w.part, s), "qkv");
        }
        if (kv_only) break;
        {
          ProbeScope ps(m, VLA_PROBE_PREFIX_ATTN, s);
          for (int rep = 0; rep < ps.reps(); ++rep)
            K_TRY(attention_chunk(aa, s), "attention");
        }
        Epilogue pe;
        pe.kind = EPI_PARTIAL;
        // at a few hundred rows the O projection adds into the residual itself (whole-K row tiles), and the
        // norm reads the residual alone; otherwise it leaves split-K partials for the norm to add
        const bool o_in_place = M > 64 && gemm_frag_rowtile(M, c.d_p, qw, EPI_RESID);
        Epilogue oe;
        oe.kind = EPI_RESID; oe.resid = w.h; oe.ldr = c.d_p;
        {
          ProbeScope ps(m, VLA_PROBE_PREFIX_O, s);
          for (int rep = 0; rep < ps.reps(); ++rep)
            K_TRY(mm_frag(w.attn, P.wo, M, c.d_p, qw, o_in_place ? oe : pe, w.part, s), "o proj");
        }
        K_TRY(resid_norm(w.h, c.d_p, w.part, o_in_place ? 0 : prefix_splits(M, c.d_p, qw), M, c.d_p, P.w2, eps, w.u, 0,
                         c.d_p, nullptr, nullptr, s, 1), "norm");
        Epilogue g = epi_store(w.mlp, c.F_p, 0);
        g.kind = EPI_GEGLU;
        g.out_frag = 1;
        {
          ProbeScope ps(m, VLA_PROBE_PREFIX_GATEUP, s);
          for (int rep = 0; rep < ps.reps(); ++rep)
            K_TRY(mm_frag(w.u, P.wgu, M, 2 * c.F_p, c.d_p, g, w.part, s), "gate/up");
        }
        {
          ProbeScope ps(m, VLA_PROBE_PREFIX_DOWN, s);
          for (int rep = 0; rep < ps.reps(); ++rep)
            K_TRY(mm_frag(w.mlp, P.wd, M, c.d_p, c.F_p, pe, w.part, s), "down");
        }
        K_TRY(resid_norm(w.h, c.d_p, w.part, prefix_splits(M, c.d_p, c.F_p), M, c.d_p, next_gain, eps, w.u, 0, c.d_p,
                         nullptr, nullptr, s, 1), "norm");
      }
    }
  }
  if (m->joint) return VLA_OK;
  // Z = RMS(h; w_final) is in w.u; project into every expert layer's K and V
  Epilogue ce;
  ce.kind = EPI_CACHE; ce.out = kv; ce.out_f32 = m->f32 ? 1 : 0;
  ce.npre = N; ce.L = c.L_e; ce.hkv = c.Hkv_e; ce.hd = c.hd_e;
  ce.npad = (int)key_rows(m, N);
  ce.out_frag = m->f32 ? 0 : 1;
  const int ncache = c.L_e * 2 * c.Hkv_e * c.hd_e;
  // absorbed products (one observation): the values are also written in frag_idx order for them
  const int64_t anp = ab ? absorb_np(m, B, N) : 0;
  uint16_t* vcopy = anp ? ab + (size_t)c.L_e * 2 * c.Hq_e * anp * c.d_e : nullptr;
  ce.vcopy = vcopy;
  // padding key rows of the last tile must hold finite values (zero weight times value)
  if (ce.npad > N) {
    K_TRY(zero_tails(kv, (long)B * c.L_e * 2 * c.Hkv_e, (long)ce.npad * c.hd_e, 32 * c.hd_e, s), "cache padding");
    if (vcopy) K_TRY(zero_tails(vcopy, (long)c.L_e * c.Hkv_e, (long)ce.npad * c.hd_e, 32 * c.hd_e, s), "value padding");
  }
  {
    ProbeScope ps(m, VLA_PROBE_CACHE, s);
    for (int rep = 0; rep < ps.reps(); ++rep) {
      if (m->f32)
        K_TRY(gemm_f32((const float*)w.u, c.d_p, (const float*)m->wcache, c.d_p, M, ncache, c.d_p, ce, s), "cache");
      else
        K_TRY(mm_frag(w.u, m->wcache, M, ncache, c.d_p, ce, w.part, s), "cache");
    }
  }
  if (anp) {
    // each layer's Wq^T K^T (scaled to log2 units) and V Wo^T from the cache just written
    AbsorbP ap{};
    const int qe = c.Hq_e * c.hd_e;
    ap.k = (const uint16_t*)kv;
    ap.v = vcopy;
    ap.wqT = m->wqT;
    ap.wo = (const uint16_t*)m->el[0].woc;
    ap.wqk = ab;
    ap.wvo = ab + (size_t)c.Hq_e * anp * c.d_e;
    ap.k_ls = 2L * c.Hkv_e * anp * c.hd_e;
    ap.v_ls = (long)c.Hkv_e * anp * c.hd_e;
    ap.wq_ls = (long)c.d_e * qe;
    ap.wo_ls = c.L_e > 1 ? (long)(((const char*)m->el[1].woc - (const char*)m->el[0].woc) / 2) : 0;
    ap.out_ls = 2L * c.Hq_e * anp * c.d_e;
    ap.L = c.L_e; ap.Hq = c.Hq_e; ap.Hkv = c.Hkv_e; ap.hd = c.hd_e; ap.Np = (int)anp; ap.d_e = c.d_e;
    ap.sl2 = 1.4426950408889634f / sqrtf((float)c.hd_e);
    K_TRY(absorb_products(ap, s), "absorbed products");
  }
  return VLA_OK;
}

// K/V blocks of a cache; the per-observation prefix lengths follow them
static size_t kv_core_bytes(const vla_model* m, int32_t batch, int32_t n_prefix) {
  const vla_model_config& c = m->cfg;
  return (size_t)batch * c.L_e * 2 * c.Hkv_e * (size_t)key_rows(m, n_prefix) * c.hd_e * elt(m);
}

extern "C" size_t vla_kv_cache_bytes(const vla_model* m, int32_t batch, int32_t n_prefix) {
  if (!live_model(m) || batch <= 0 || n_prefix <= 0) return 0;
  return (kv_core_bytes(m, batch, n_prefix) + 255) / 256 * 256 + ((size_t)batch * 4 + 255) / 256 * 256 +
         absorb_bytes(m, batch, n_prefix);
}

extern "C" vla_status vla_prefix_encode_ex(vla_model* m, const void* x, int32_t x_dtype, int32_t batch,
                                           int32_t n_prefix, const int32_t* lengths, void* kv_storage, size_t kv_bytes,
                                           void* stream, vla_kv_cache** out, vla_timing* timing) {
  if (!out) return fail(VLA_ERR_INVALID_ARGUMENT, "out is NULL");
  *out = nullptr;
  if (!live_model(m)) return fail(VLA_ERR_INVALID_HANDLE, "unknown model");
  if (!x || !kv_storage) return fail(VLA_ERR_INVALID_ARGUMENT, "prefix_hidden or kv_storage is NULL");
  if (x_dtype != VLA_IN_F32 && x_dtype != VLA_IN_BF16) return fail(VLA_ERR_INVALID_ARGUMENT, "bad prefix_hidden dtype");
  if (batch <= 0 || n_prefix <= 0) return fail(VLA_ERR_INVALID_ARGUMENT, "batch and n_prefix must be positive");
  if ((int64_t)batch * n_prefix > (1 << 22)) return fail(VLA_ERR_UNSUPPORTED, "too many prefix tokens");
  if (lengths)
    for (int b = 0; b < batch; ++b)
      if (lengths[b] < 1 || lengths[b] > n_prefix)
        return fail(VLA_ERR_INVALID_ARGUMENT, "lengths[" + std::to_string(b) + "] = " + std::to_string(lengths[b]) +
                                                  " is outside 1.." + std::to_string(n_prefix));
  const size_t need = vla_kv_cache_bytes(m, batch, n_prefix);
  if (kv_bytes < need)
    return fail(VLA_ERR_SHAPE_MISMATCH, "kv_bytes " + std::to_string(kv_bytes) + " < required " + std::to_string(need));
  hipStream_t s = (hipStream_t)stream;
  WS w;
  vla_status st = get_ws(m, (int64_t)batch * n_prefix, 0, &w, (int64_t)batch * key_rows(m, n_prefix));
  if (st != VLA_OK) return st;
  int* lens = (int*)((char*)kv_storage + (kv_core_bytes(m, batch, n_prefix) + 255) / 256 * 256);
  uint16_t* ab = absorb_bytes(m, batch, n_prefix) ? (uint16_t*)((char*)lens + ((size_t)batch * 4 + 255) / 256 * 256)
                                                   : nullptr;
  if (timing) K_TRY(hipEventRecord(m->ev0, s), "event");
  if (lengths) K_TRY(set_lengths(lens, lengths, batch, n_prefix, s), "prefix lengths");
  st = run_prefix(m, x, x_dtype == VLA_IN_BF16, batch, n_prefix, lengths ? lens : nullptr, kv_storage, w, s, ab);
  if (st != VLA_OK) return st;
  if (timing) {
    K_TRY(hipEventRecord(m->ev1, s), "event");
    K_TRY(hipEventSynchronize(m->ev1), "event sync");
    float ms = 0.f;
    K_TRY(hipEventElapsedTime(&ms, m->ev0, m->ev1), "elapsed");
    timing->prefix_ms = ms;
    timing->denoise_ms = 0.f;
    timing->step_ms = 0.f;
    timing->graph_replayed = 0;
  }
  vla_kv_cache* k = new vla_kv_cache();
  k->model = m;
  k->B = batch;
  k->N = n_prefix;
  k->storage = kv_storage;
  k->lens = lengths ? lens : nullptr;
  if (ab) {
    const int64_t np = absorb_np(m, batch, n_prefix);
    k->ab_ls = 2L * m->cfg.Hq_e * np * m->cfg.d_e;
    k->wqk = ab;
    k->wvo = ab + (size_t)m->cfg.Hq_e * np * m->cfg.d_e;
  }
  {
    std::lock_guard<std::mutex> g(g_mu);
    m->caches.insert(k);
  }
  *out = k;
  return VLA_OK;
}

extern "C" vla_status vla_prefix_encode_masked(vla_model* m, const float* x, int32_t batch, int32_t n_prefix,
                                               const int32_t* lengths, void* kv_storage, size_t kv_bytes, void* stream,
                                               vla_kv_cache** out, vla_timing* timing) {
  return vla_prefix_encode_ex(m, x, VLA_IN_F32, batch, n_prefix, lengths, kv_storage, kv_bytes, stream, out, timing);
}

extern "C" vla_status vla_prefix_encode(vla_model* m, const float* x, int32_t batch, int32_t n_prefix, void* kv_storage,
                                        size_t kv_bytes, void* stream, vla_kv_cache** out, vla_timing* timing) {
  return vla_prefix_encode_ex(m, x, VLA_IN_F32, batch, n_prefix, nullptr, kv_storage, kv_bytes, stream, out, timing);
}

extern "C" vla_status vla_kv_cache_release(vla_kv_cache* k) {
  std::lock_guard<std::mutex> g(g_mu);
  for (vla_model* m : g_models) {
    if (m->caches.count(k)) {
      m->caches.erase(k);
      k->magic = 0;
      delete k;
      return VLA_OK;
    }
  }
  return fail(VLA_ERR_INVALID_HANDLE, "unknown or released cache");
}

extern "C" vla_status vla_kv_cache_info(const vla_kv_cache* k, int32_t* batch, int32_t* n_prefix) {
  if (!live_cache(k)) return fail(VLA_ERR_INVALID_HANDLE, "unknown or released cache");
  if (batch) *batch = k->B;
  if (n_prefix) *n_prefix = k->N;
  return VLA_OK;
}

// ============================================================== solver
// Workgroups of the persistent step for this call, or 0 when the kernel chain runs.
static int fused_wgs(vla_model* m, const vla_kv_cache* kv, int* shadows) {
  const vla_model_config& c = m->cfg;
  const int64_t M = (int64_t)kv->B * c.H;
  if (!m->fused || M > 64 || vla_kv_cache_bytes(m, kv->B, kv->N) >= ((size_t)1 << 31)) return 0;
  const int mb = M <= 16 ? 1 : M <= 32 ? 2 : 4;
  const int key = c.hd_e * 8 + mb;
  auto it = m->fused_occ.find(key);
  if (it == m->fused_occ.end()) it = m->fused_occ.emplace(key, fused_occupancy(c.hd_e, (int)M)).first;
  const int occ = it->second;
  if (occ < 1) return 0;
  const int nwg = std::min(m->ncu, 256);
  // a shadow workgroup shares its compute workgroup's XCD (linear id mod 8) and needs a second slot per CU
  *shadows = occ >= 2 && nwg % 8 == 0 ? 1 : 0;
  return nwg;
}

static vla_status run_steps_fused(vla_model* m, const vla_kv_cache* kv, int steps, const WS& w, int nwg, int shadows,
                                  hipStream_t s) {
  const vla_model_config& c = m->cfg;
  FusedStepP p{};
  p.B = kv->B; p.H = c.H; p.M = kv->B * c.H; p.Hp = (int)key_rows(m, c.H); p.N = kv->N; p.Np = (int)key_rows(m, kv->N);
  p.d_e = c.d_e; p.d_a = c.d_a; p.F = c.F_e; p.L = c.L_e; p.Hq = c.Hq_e; p.Hkv = c.Hkv_e; p.D = c.hd_e;
  p.qe = c.Hq_e * c.hd_e; p.qkve = (c.Hq_e + 2 * c.Hkv_e) * c.hd_e;
  p.nrb = (c.Hq_e / c.Hkv_e * c.H + 15) / 16;
  p.eps = c.rms_eps;
  int used = 0;
  gemm_chunk_plan(c.d_e, 1, &used, &p.kc_qkv);
  if (used != 1) return fail(VLA_ERR_UNSUPPORTED, "persistent step: d_e needs one K chunk");
  p.kc_q = p.kc_gu = p.kc_qkv;
  gemm_chunk_plan(p.qe, expert_splits(p.M, c.d_e, p.qe), &p.s_o, &p.kc_o);
  gemm_chunk_plan(c.F_e, expert_splits(p.M, c.d_e, c.F_e), &p.s_d, &p.kc_d);
  if (p.s_o > 4 || p.s_d > 4) return fail(VLA_ERR_UNSUPPORTED, "persistent step: more than 4 K splits");
  p.spw_qkv = p.spw_q = p.spw_gu = p.kc_qkv >> 7;
  p.spw_o = p.kc_o >> 7;
  p.spw_d = p.kc_d >> 7;
  const ExpertLayer& L0 = m->el[0];
  p.ew = m->ew; p.ew_layer = (long)m->ew_layer;
  p.off_qkv = (const char*)L0.wqkv - m->ew; p.off_os = (const char*)L0.wos - m->ew;
  p.off_qc = (const char*)L0.wqc - m->ew; p.off_oc = (const char*)L0.woc - m->ew;
  p.off_gu = (const char*)L0.wgu - m->ew; p.off_d = (const char*)L0.wd - m->ew;
  p.egains = m->egains; p.w_ef = m->w_ef;
  p.w_out = (const uint16_t*)m->w_out; p.w_in = (const uint16_t*)m->w_in; p.sched = m->sched_dev;
  p.cache = (const uint16_t*)kv->storage;
  p.klen = kv->lens;
  p.bytes_cache = (uint32_t)vla_kv_cache_bytes(m, kv->B, kv->N);
  p.E = w.E; p.X = w.X; p.u = (uint16_t*)w.eu; p.q = (uint16_t*)w.eqkv; p.kc = (uint16_t*)w.ek; p.vc = (uint16_t*)w.ev;
  p.attn = (uint16_t*)w.eattn; p.eq = (uint16_t*)w.eq; p.g = (uint16_t*)w.emlp; p.part = w.epart;
  p.bytes_E = (uint32_t)w.n_E; p.bytes_X = (uint32_t)w.n_X; p.bytes_u = (uint32_t)w.n_eu; p.bytes_q = (uint32_t)w.n_eq;
  p.bytes_kv = (uint32_t)w.n_ekv; p.bytes_attn = (uint32_t)w.n_eattn; p.bytes_g = (uint32_t)w.n_emlp;
  p.bytes_part = (uint32_t)w.n_epart;
  p.bar = m->fbar; p.err = m->ferr; p.nwg = nwg;
  p.gen_tail = 1;
  K_TRY(fused_zero(m->fbar, fused_barrier_words(c.L_e), s), "barrier clear");
  for (int k = 0; k < steps; ++k) {
    p.k_head = k - 1;
    p.k_embed = k;
    p.trailing_head = k + 1 == steps;
    p.k_tail = k;
    p.gen = (unsigned)(k + 1);
    K_TRY(fused_step(p, shadows, s), "persistent step");
  }
  return VLA_OK;
}

static vla_status run_steps(vla_model* m, const vla_kv_cache* kv, int steps, const WS& w, hipStream_t s) {
  const vla_model_config& c = m->cfg;
  {
    int shadows = 0;
    const int nwg = fused_wgs(m, kv, &shadows);
    if (nwg > 0) return run_steps_fused(m, kv, steps, w, nwg, shadows, s);
  }
  const int B = kv->B, N = kv->N, H = c.H, M = B * H;
  const int qe = c.Hq_e * c.hd_e, qkve = (c.Hq_e + 2 * c.Hkv_e) * c.hd_e;
  const float eps = c.rms_eps;
  const bool f32 = m->f32;
  const size_t es = elt(m);
  // self-attention over the H chunk tokens of each observation
  AttnArgs sa{};
  const int Hp = (int)key_rows(m, H), Np = (int)key_rows(m, N);
  if (f32) {  // plain rows of the fused projection output
    sa.q = w.eqkv; sa.q_bs = (long)H * qkve; sa.q_hs = c.hd_e; sa.q_rs = qkve;
    sa.k = (const char*)w.eqkv + (size_t)qe * es; sa.k_bs = sa.q_bs; sa.k_hs = c.hd_e; sa.k_rs = qkve;
    sa.v = (const char*)w.eqkv + (size_t)(qe + c.Hkv_e * c.hd_e) * es; sa.v_bs = sa.q_bs; sa.v_hs = c.hd_e; sa.v_rs = qkve;
  } else {  // query rows, keys and values in the MFMA operand orders (EPI_QKV)
    sa.q = w.eqkv; sa.q_bs = (long)H * qe; sa.q_hs = c.hd_e; sa.q_rs = qe;
    sa.k = w.ek; sa.k_bs = (long)c.Hkv_e * Hp * c.hd_e; sa.k_hs = (long)Hp * c.hd_e;
    sa.v = w.ev; sa.v_bs = sa.k_bs; sa.v_hs = sa.k_hs;
  }
  sa.o = w.eattn; sa.o_bs = (long)H * qe; sa.o_rs = qe;
  sa.B = B; sa.Nq = H; sa.Nk = H; sa.Hq = c.Hq_e; sa.Hkv = c.Hkv_e; sa.hd = c.hd_e; sa.o_f32 = f32 ? 1 : 0;
  Epilogue qkv_e;  // bf16 fused self-attention projection
  qkv_e.kind = EPI_QKV; qkv_e.out = w.eqkv; qkv_e.ldo = qe; qkv_e.nq = qe;
  qkv_e.kout = w.ek; qkv_e.vout = w.ev; qkv_e.hkv = c.Hkv_e; qkv_e.hd = c.hd_e; qkv_e.npre = H; qkv_e.npad = Hp;
  // bf16: every GEMM input in the fragment layout (weights always are); up to
  // 64 chunk rows the chunk-sized kernel with weight prefetch, above that the
  // 288-row-tile kernel of the prefix
  const int fr = f32 ? 0 : 1;
  const bool small = fr && M <= 64;
  sa.o_frag = fr;
  // cross-attention into the cache [B][L_e][2][Hkv_e][N][hd_e]
  AttnArgs ca = sa;
  const long layer_stride = 2L * c.Hkv_e * Np * c.hd_e;
  ca.q = w.eq; ca.q_bs = (long)H * qe; ca.q_hs = c.hd_e; ca.q_rs = qe;
  ca.k_bs = c.L_e * layer_stride; ca.k_hs = (long)Np * c.hd_e; ca.k_rs = c.hd_e;
  ca.v_bs = ca.k_bs; ca.v_hs = ca.k_hs; ca.v_rs = c.hd_e;
  ca.Nk = N;
  ca.klen = kv->lens;   // key padding of the cached prefix
  sa.klen2 = kv->lens;  // joint attention: the prefix keys are the second source
  Epilogue pe;
  pe.kind = EPI_PARTIAL;
  const int S_o = expert_splits(M, c.d_e, qe), S_d = expert_splits(M, c.d_e, c.F_e);
  // Kernels of the chain get extra workgroups that read the weights of the
  // GEMMs ahead once, so those GEMMs find them in cache: a weight load then
  // costs an L2 hit instead of an HBM round trip, while the carrier's own work
  // hides the read.  The attention kernels run longest with the fewest
  // workgroups of their own, so they carry most of it: self attention reads
  // the O and cross-query weights, cross attention the cross O and gate/up
  // weights.  The gate/up GEMM reads the down weights, and the norms the
  // layer's cache block and the next layer's QKV weights; with the norms folded
  // into the products, the cross query reads the cache block and the gate/up
  // GEMM the next layer's QKV weights too.  With the absorbed cross sublayer
  // the self attention reads the O weights and both absorbed products, and the
  // gate/up weights are not read ahead.  Only for the fragment path (batch-1
  // sized chunks).
  const size_t b_qkv = (size_t)qkve * c.d_e * es, b_o = (size_t)c.d_e * qe * es, b_q = (size_t)qe * c.d_e * es;
  const size_t b_gu = (size_t)2 * c.F_e * c.d_e * es, b_d = (size_t)c.d_e * c.F_e * es;
  const size_t layer_kv = (size_t)layer_stride * es;
  // Weight ranges are read XCD by XCD, in the column groups of the GEMM that
  // consumes them, so each lands in the L2 its consumer's workgroups read from.
  const size_t g_qkv = gemm_chunk_group_bytes(M, qkve, c.d_e, EPI_QKV, 1);
  const size_t g_o0 = gemm_chunk_group_bytes(M, c.d_e, qe, EPI_PARTIAL, S_o);
  const size_t g_q = gemm_chunk_group_bytes(M, qe, c.d_e, EPI_STORE, 1);
  const size_t g_gu = gemm_chunk_group_bytes(M, 2 * c.F_e, c.d_e, EPI_GEGLU, 1);
  const size_t g_d0 = gemm_chunk_group_bytes(M, c.d_e, c.F_e, EPI_PARTIAL, S_d);
  // Folded norms (chunk path): the O, cross O and down products add their sums
  // to the residual themselves and write the next product's input unnormalised,
  // bf16(h (1 + g)), with each row's sums of squares over 16-column blocks; the
  // next product scales its output rows by the norm factor those sums give.
  // Three row kernels and their launch gaps less per layer.
  int d_used = 0, d_chunk = 0;
  gemm_chunk_plan(c.d_e, 1, &d_used, &d_chunk);
  auto res_k = [](int K) { return K % 32 == 0 && K <= 4096; };
  const int d8 = c.d_e / 128;  // column groups of 16 per XCD in the residual products
  const bool fold = m->fold && small && d_used == 1 && c.d_e % 128 == 0 && (d8 == 1 || d8 == 2 || d8 == 4 || d8 == 8) &&
                    res_k(qe) && res_k(c.F_e);
  const size_t g_o = fold ? gemm_chunk_resnorm_group_bytes(c.d_e, qe) : g_o0;
  const size_t g_d = fold ? gemm_chunk_resnorm_group_bytes(c.d_e, c.F_e) : g_d0;
  // absorbed cross sublayer (the encode formed the products): score columns, their weights and statistics
  const bool absorbed = kv->wqk && fold && B == 1;
  const int np_ab = absorbed ? (int)(kv->ab_ls / (2L * c.Hq_e * c.d_e)) : 0, ns_ab = c.Hq_e * np_ab;
  const size_t b_ab = (size_t)ns_ab * c.d_e * es;
  const size_t g_sc = absorbed ? gemm_chunk_group_bytes(M, ns_ab, c.d_e, EPI_SCORES, 1) : 0;
  const size_t g_vo = absorbed ? gemm_chunk_resnorm_group_bytes(c.d_e, ns_ab) : 0;
  Epilogue sc_e;
  sc_e.kind = EPI_SCORES; sc_e.out = w.esc; sc_e.ldo = ns_ab; sc_e.stats = w.est;
  sc_e.npad = np_ab; sc_e.npre = N; sc_e.klen = kv->lens;
  auto scaled = [&](Epilogue ep) {
    ep.rss = w.ess; ep.nss = c.d_e / 16; ep.rdim = c.d_e; ep.reps = eps;
    return ep;
  };
  auto pfr = [&](const void* p, size_t bytes, size_t group, const void* p2, size_t bytes2, size_t group2, int blocks) {
    Prefetch f;
    if (!small) return f;
    f.p = p; f.bytes = bytes; f.group = group;
    f.p2 = p2; f.bytes2 = p2 ? bytes2 : 0; f.group2 = p2 ? group2 : 0;
    f.sink = w.sink; f.blocks = blocks;
    return f;
  };
  // row kernel between steps: head of step k - 1 (if any) fused with the embedding of step k (if any)
  auto rows = [&](int k_head, int k_embed) {
    StepRows a;
    a.E = w.E; a.Eout = w.E; a.X = w.X; a.M = M; a.d_e = c.d_e; a.d_a = c.d_a; a.eps = eps;
    a.gain_f = m->w_ef; a.w_out = m->w_out; a.w_in = m->w_in; a.gain_1 = m->el[0].a1;
    a.u = w.eu; a.u_f32 = f32 ? 1 : 0; a.u_frag = fr; a.sched = m->sched_dev;
    a.k_head = k_head; a.k_embed = k_embed;
    if (k_embed >= 0)
      a.pf = pfr(m->el[0].wqkv, b_qkv, g_qkv, m->joint && B == 1 ? kv->storage : nullptr, layer_kv, 0, 64);
    return step_rows(a, f32 ? 1 : 0, s);
  };
  for (int k = 0; k < steps; ++k) {
    if (k == 0) K_TRY(rows(-1, 0), "embed");
    for (int e = 0; e < c.L_e; ++e) {
      const ExpertLayer& L = m->el[e];
      ca.k = (const char*)kv->storage + (size_t)e * layer_stride * es;
      ca.v = (const char*)ca.k + (size_t)c.Hkv_e * Np * c.hd_e * es;
      if (m->joint) {
        // joint attention: the chunk's own keys, then prefix layer e's (cache block e)
        sa.k2 = ca.k; sa.k2_bs = ca.k_bs; sa.k2_hs = ca.k_hs; sa.k2_rs = ca.k_rs;
        sa.v2 = ca.v; sa.v2_bs = ca.v_bs; sa.v2_hs = ca.v_hs; sa.v2_rs = ca.v_rs;
        sa.Nk2 = N;
      }
      if (f32 && m->joint) {
        K_TRY(gemm_f32((const float*)w.eu, c.d_e, (const float*)L.wqkv, c.d_e, M, qkve, c.d_e, epi_store(w.eqkv, qkve, 1), s), "qkv_s");
        K_TRY(attention_f32(sa, s), "joint attn");
        Epilogue r;
        r.kind = EPI_RESID; r.resid = w.E; r.ldr = c.d_e;
        K_TRY(gemm_f32((const float*)w.eattn, qe, (const float*)L.wos, qe, M, c.d_e, qe, r, s), "o_s");
        K_TRY(resid_norm(w.E, c.d_e, nullptr, 0, M, c.d_e, L.a3, eps, w.eu, 1, c.d_e, nullptr, nullptr, s), "norm");
        Epilogue g = epi_store(w.emlp, c.F_e, 1);
        g.kind = EPI_GEGLU;
        K_TRY(gemm_f32((const float*)w.eu, c.d_e, (const float*)L.wgu, c.d_e, M, 2 * c.F_e, c.d_e, g, s), "gate/up");
        K_TRY(gemm_f32((const float*)w.emlp, c.F_e, (const float*)L.wd, c.F_e, M, c.d_e, c.F_e, r, s), "down");
        if (e + 1 < c.L_e)
          K_TRY(resid_norm(w.E, c.d_e, nullptr, 0, M, c.d_e, m->el[e + 1].a1, eps, w.eu, 1, c.d_e, nullptr, nullptr, s), "norm");
      } else if (f32) {
        K_TRY(gemm_f32((const float*)w.eu, c.d_e, (const float*)L.wqkv, c.d_e, M, qkve, c.d_e, epi_store(w.eqkv, qkve, 1), s), "qkv_s");
        K_TRY(attention_f32(sa, s), "self attn");
        Epilogue r;
        r.kind = EPI_RESID; r.resid = w.E; r.ldr = c.d_e;
        K_TRY(gemm_f32((const float*)w.eattn, qe, (const float*)L.wos, qe, M, c.d_e, qe, r, s), "o_s");
        K_TRY(resid_norm(w.E, c.d_e, nullptr, 0, M, c.d_e, L.a2, eps, w.eu, 1, c.d_e, nullptr, nullptr, s), "norm");
        K_TRY(gemm_f32((const float*)w.eu, c.d_e, (const float*)L.wqc, c.d_e, M, qe, c.d_e, epi_store(w.eq, qe, 1), s), "q_c");
        K_TRY(attention_f32(ca, s), "cross attn");
        K_TRY(gemm_f32((const float*)w.eattn, qe, (const float*)L.woc, qe, M, c.d_e, qe, r, s), "o_c");
        K_TRY(resid_norm(w.E, c.d_e, nullptr, 0, M, c.d_e, L.a3, eps, w.eu, 1, c.d_e, nullptr, nullptr, s), "norm");
        Epilogue g = epi_store(w.emlp, c.F_e, 1);
        g.kind = EPI_GEGLU;
        K_TRY(gemm_f32((const float*)w.eu, c.d_e, (const float*)L.wgu, c.d_e, M, 2 * c.F_e, c.d_e, g, s), "gate/up");
        K_TRY(gemm_f32((const float*)w.emlp, c.F_e, (const float*)L.wd, c.F_e, M, c.d_e, c.F_e, r, s), "down");
        if (e + 1 < c.L_e)
          K_TRY(resid_norm(w.E, c.d_e, nullptr, 0, M, c.d_e, m->el[e + 1].a1, eps, w.eu, 1, c.d_e, nullptr, nullptr, s), "norm");
      } else {
        const uint16_t* u = (const uint16_t*)w.eu;
        // C = A W^T on the chunk: fragment-layout operands up to 64 rows, else the tiled kernel
        // (splits: the chunk kernel's request; the wide kernel picks its own, as expert_splits says)
        auto mm = [&](const void* A, int lda, const void* W, int N, int K, const Epilogue& ep, int splits,
                      const Prefetch* pf = nullptr) {
          (void)lda;
          if (small) return gemm_chunk((const uint16_t*)A, (const uint16_t*)W, M, N, K, ep, splits, w.epart, s, pf);
          return gemm_frag((const uint16_t*)A, (const uint16_t*)W, M, N, K, ep, 0, w.epart, s);
        };
        // layer 0 reads the normalised rows of the step kernel, later layers the folded input
        K_TRY(mm(u, c.d_e, L.wqkv, qkve, c.d_e, fold && e > 0 ? scaled(qkv_e) : qkv_e, 1), "qkv_s");
        if (m->joint) {
          // one attention over the chunk and prefix layer e, then the MLP
          sa.pf = pfr(L.wos, b_o, g_o, L.wgu, b_gu, g_gu, 192);
          {
            ProbeScope ps(m, VLA_PROBE_EXPERT_SELF_ATTN, s);
            for (int rep = 0; rep < ps.reps(); ++rep)
              K_TRY(attention_chunk(sa, s), "joint attn");
          }
          if (fold) {
            K_TRY(gemm_chunk_resnorm((const uint16_t*)w.eattn, (const uint16_t*)L.wos, M, c.d_e, qe, w.E, c.d_e, L.a3,
                                     (uint16_t*)w.eu, w.ess, s, nullptr), "o_s");
          } else {
            K_TRY(mm(w.eattn, qe, L.wos, c.d_e, qe, pe, S_o), "o_s");
            K_TRY(resid_norm(w.E, c.d_e, w.epart, S_o, M, c.d_e, L.a3, eps, w.eu, 0, c.d_e, nullptr, nullptr, s, fr), "norm");
          }
        } else {
          sa.pf = absorbed ? pfr(L.wos, b_o, g_o, kv->wqk + (size_t)e * kv->ab_ls, b_ab, g_sc, 192)
                           : pfr(L.wos, b_o, g_o, L.wqc, b_q, g_q, 192);
          if (absorbed) {
            // absorbed: the self attention also reads Wvo; the score product carries no prefetch (the
            // gate/up weights read by its extra workgroups cost the product more than gate/up saved)
            sa.pf.p3 = kv->wvo + (size_t)e * kv->ab_ls;
            sa.pf.bytes3 = b_ab;
            sa.pf.group3 = g_vo;
          }
          {
            ProbeScope ps(m, VLA_PROBE_EXPERT_SELF_ATTN, s);
            for (int rep = 0; rep < ps.reps(); ++rep)
              K_TRY(attention_chunk(sa, s), "self attn");
          }
          if (absorbed) {
            // cross sublayer as two products: the scores from the normalised rows (with each
            // 32-key block's max and weight sum), then the weights times Wvo into the residual
            const uint16_t* wqk = kv->wqk + (size_t)e * kv->ab_ls;
            const uint16_t* wvo = kv->wvo + (size_t)e * kv->ab_ls;
            K_TRY(gemm_chunk_resnorm((const uint16_t*)w.eattn, (const uint16_t*)L.wos, M, c.d_e, qe, w.E, c.d_e, L.a2,
                                     (uint16_t*)w.eu, w.ess, s, nullptr), "o_s");
            {
              ProbeScope ps(m, VLA_PROBE_EXPERT_SCORES, s);
              for (int rep = 0; rep < ps.reps(); ++rep)
                K_TRY(mm(u, c.d_e, wqk, ns_ab, c.d_e, scaled(sc_e), 1, nullptr), "scores");
            }
            K_TRY(gemm_chunk_probres((const uint16_t*)w.esc, w.est, np_ab / 32, wvo, M, c.d_e, ns_ab, w.E, c.d_e, L.a3,
                                     (uint16_t*)w.eu, w.ess, s, nullptr), "cross out");
          } else {
            const Prefetch pf_kv = pfr(B == 1 ? ca.k : nullptr, B == 1 ? layer_kv : 0, 0, nullptr, 0, 0, 64);
            if (fold) {
              // the cache block goes with the cross query below: workgroups of this product hold too many
              // registers for a prefetch workgroup to share their CU, so one would run after them
              K_TRY(gemm_chunk_resnorm((const uint16_t*)w.eattn, (const uint16_t*)L.wos, M, c.d_e, qe, w.E, c.d_e, L.a2,
                                       (uint16_t*)w.eu, w.ess, s, nullptr), "o_s");
            } else {
              K_TRY(mm(w.eattn, qe, L.wos, c.d_e, qe, pe, S_o), "o_s");
              K_TRY(resid_norm(w.E, c.d_e, w.epart, S_o, M, c.d_e, L.a2, eps, w.eu, 0, c.d_e, nullptr, nullptr, s, fr,
                               &pf_kv), "norm");
            }
            const Epilogue qc_e = epi_store(w.eq, qe, 0);
            K_TRY(mm(u, c.d_e, L.wqc, qe, c.d_e, fold ? scaled(qc_e) : qc_e, 1, fold ? &pf_kv : nullptr), "q_c");
            ca.pf = pfr(L.woc, b_o, g_o, L.wgu, b_gu, g_gu, 192);
            {
              ProbeScope ps(m, VLA_PROBE_EXPERT_CROSS_ATTN, s);
              for (int rep = 0; rep < ps.reps(); ++rep)
                K_TRY(attention_chunk(ca, s), "cross attn");
            }
            if (fold) {
              K_TRY(gemm_chunk_resnorm((const uint16_t*)w.eattn, (const uint16_t*)L.woc, M, c.d_e, qe, w.E, c.d_e, L.a3,
                                       (uint16_t*)w.eu, w.ess, s, nullptr), "o_c");
            } else {
              K_TRY(mm(w.eattn, qe, L.woc, c.d_e, qe, pe, S_o), "o_c");
              K_TRY(resid_norm(w.E, c.d_e, w.epart, S_o, M, c.d_e, L.a3, eps, w.eu, 0, c.d_e, nullptr, nullptr, s, fr), "norm");
            }
          }
        }
        Epilogue g = epi_store(w.emlp, c.F_e, 0);
        g.kind = EPI_GEGLU;
        g.out_frag = fr;
        // next layer's QKV weights (and, joint, its cache block)
        const void* next_kv = m->joint && B == 1 ? (const char*)ca.k + (size_t)layer_stride * es : nullptr;
        const Prefetch pf_next =
            e + 1 < c.L_e ? pfr(m->el[e + 1].wqkv, b_qkv, g_qkv, next_kv, layer_kv, 0, 192) : Prefetch{};
        Prefetch pf_d = pfr(L.wd, b_d, g_d, nullptr, 0, 0, 192);
        if (fold && e + 1 < c.L_e) {
          // folded: the gate/up product also reads what the down product would (see the cross query above)
          pf_d.p2 = pf_next.p; pf_d.bytes2 = pf_next.bytes; pf_d.group2 = pf_next.group;
          pf_d.p3 = pf_next.p2; pf_d.bytes3 = pf_next.bytes2; pf_d.group3 = pf_next.group2;
        }
        {
          ProbeScope ps(m, VLA_PROBE_EXPERT_GATEUP, s);
          for (int rep = 0; rep < ps.reps(); ++rep)
            K_TRY(mm(u, c.d_e, L.wgu, 2 * c.F_e, c.d_e, fold ? scaled(g) : g, 1, &pf_d), "gate/up");
        }
        if (fold) {
          // after the last layer only the residual: the step kernel applies the final norm
          K_TRY(gemm_chunk_resnorm((const uint16_t*)w.emlp, (const uint16_t*)L.wd, M, c.d_e, c.F_e, w.E, c.d_e,
                                   e + 1 < c.L_e ? m->el[e + 1].a1 : nullptr, (uint16_t*)w.eu, w.ess, s, nullptr),
                "down");
        } else {
          K_TRY(mm(w.emlp, c.F_e, L.wd, c.d_e, c.F_e, pe, S_d), "down");
          K_TRY(resid_norm(w.E, c.d_e, w.epart, S_d, M, c.d_e, e + 1 < c.L_e ? m->el[e + 1].a1 : m->w_ef, eps,
                           e + 1 < c.L_e ? w.eu : nullptr, 0, c.d_e, nullptr, nullptr, s, fr, &pf_next), "norm");
        }
      }
    }
    K_TRY(rows(k, k + 1 < steps ? k + 1 : -1), "head");
  }
  return VLA_OK;
}

static bool use_graphs() {
  const char* v = getenv("VLA_NO_GRAPH");
  return !(v && v[0] == '1');
}

extern "C" vla_status vla_denoise_chunk(vla_model* m, const vla_kv_cache* kv, const float* noise, int32_t steps,
                                        const vla_solver* solver, void* actions_out, int32_t out_dtype, void* stream,
                                        vla_timing* timing) {
  if (!live_model(m)) return fail(VLA_ERR_INVALID_HANDLE, "unknown model");
  if (!live_cache(kv)) return fail(VLA_ERR_INVALID_HANDLE, "unknown or released cache");
  if (kv->model != m) return fail(VLA_ERR_INVALID_HANDLE, "cache belongs to another model");
  if (!noise || !actions_out) return fail(VLA_ERR_INVALID_ARGUMENT, "noise or actions_out is NULL");
  if (steps <= 0 || steps > 4096) return fail(VLA_ERR_INVALID_ARGUMENT, "steps must be in 1..4096");
  if (out_dtype != VLA_OUT_F32 && out_dtype != VLA_OUT_BF16) return fail(VLA_ERR_INVALID_ARGUMENT, "bad out_dtype");
  std::vector<float> sched(steps + 1);
  if (solver && solver->schedule) {
    for (int k = 0; k <= steps; ++k) {
      sched[k] = solver->schedule[k];
      if (!std::isfinite(sched[k])) return fail(VLA_ERR_INVALID_ARGUMENT, "non-finite schedule");
    }
  } else {
    const double t0 = solver ? solver->tau_start : 0.0, t1 = solver ? solver->tau_end : 1.0;
    if (!std::isfinite(t0) || !std::isfinite(t1)) return fail(VLA_ERR_INVALID_ARGUMENT, "non-finite tau");
    for (int k = 0; k <= steps; ++k) sched[k] = (float)(t0 + k * (t1 - t0) / steps);
  }
  const vla_model_config& c = m->cfg;
  hipStream_t s = (hipStream_t)stream;
  WS w;
  vla_status st = get_ws(m, 0, (int64_t)kv->B * c.H, &w);
  if (st != VLA_OK) return st;
  if (steps + 1 > m->sched_cap) {
    if (m->sched_dev) {
      (void)hipDeviceSynchronize();
      (void)hipFree(m->sched_dev);
      (void)hipHostFree(m->sched_host);
      m->sched_dev = nullptr;
      m->sched_host = nullptr;
      m->sched_last.clear();
      for (auto& g : m->graphs) (void)hipGraphExecDestroy(g.second.exec);
      m->graphs.clear();
    }
    const int cap = std::max(64, steps + 1);
    if (lib_malloc((void**)&m->sched_dev, cap * 4) != hipSuccess || lib_host_malloc((void**)&m->sched_host, cap * 4) != hipSuccess) {
      (void)hipGetLastError();
      return fail(VLA_ERR_OUT_OF_MEMORY, "schedule buffers");
    }
    m->sched_cap = cap;
  }
  // The device schedule is uploaded only when it changes (or comes from
  // another stream), so a repeated call neither waits on the host nor copies.
  const bool upload = m->sched_stream != s || m->sched_last != sched;
  if (upload) {
    // the pinned staging buffer may still feed an earlier copy on this stream
    K_TRY(hipStreamSynchronize(s), "sync");
    memcpy(m->sched_host, sched.data(), (steps + 1) * 4);
  }
  if (timing) K_TRY(hipEventRecord(m->ev0, s), "event");
  if (upload) {
    K_TRY(hipMemcpyAsync(m->sched_dev, m->sched_host, (steps + 1) * 4, hipMemcpyHostToDevice, s), "schedule upload");
    m->sched_last = sched;
    m->sched_stream = s;
  }
  const long nx = (long)kv->B * c.H * c.d_a;
  K_TRY(copy_f32(noise, w.X, nx, s), "noise in");
  int replayed = 0;
  if (use_graphs()) {
    GraphKey key{kv->storage, kv->lens, kv->B, kv->N, steps};
    auto it = m->graphs.find(key);
    hipGraphExec_t exec = nullptr;
    if (it == m->graphs.end()) {
      if (m->graphs.size() >= kMaxGraphs) {
        // evict the least recently used graph, once nothing can still be running it
        auto lru = m->graphs.begin();
        for (auto g = m->graphs.begin(); g != m->graphs.end(); ++g)
          if (g->second.last_use < lru->second.last_use) lru = g;
        K_TRY(hipDeviceSynchronize(), "sync before graph eviction");
        (void)hipGraphExecDestroy(lru->second.exec);
        m->graphs.erase(lru);
      }
      K_TRY(hipStreamBeginCapture(m->cap_stream, hipStreamCaptureModeThreadLocal), "begin capture");
      vla_status rs = run_steps(m, kv, steps, w, m->cap_stream);
      hipGraph_t graph = nullptr;
      hipError_t ce = hipStreamEndCapture(m->cap_stream, &graph);
      if (rs != VLA_OK) {
        if (graph) (void)hipGraphDestroy(graph);
        return rs;
      }
      K_TRY(ce, "end capture");
      hipError_t ie = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
      (void)hipGraphDestroy(graph);
      K_TRY(ie, "graph instantiate");
      m->graphs[key] = GraphEntry{exec, ++m->graph_clock};
    } else {
      exec = it->second.exec;
      it->second.last_use = ++m->graph_clock;
      replayed = 1;
    }
    K_TRY(hipGraphLaunch(exec, s), "graph launch");
  } else {
    st = run_steps(m, kv, steps, w, s);
    if (st != VLA_OK) return st;
  }
  K_TRY(copy_out(w.X, actions_out, nx, out_dtype == VLA_OUT_BF16, s), "actions out");
  if (timing) {
    K_TRY(hipEventRecord(m->ev1, s), "event");
    K_TRY(hipEventSynchronize(m->ev1), "event sync");
    float ms = 0.f;
    K_TRY(hipEventElapsedTime(&ms, m->ev0, m->ev1), "elapsed");
    timing->prefix_ms = 0.f;
    timing->denoise_ms = ms;
    timing->step_ms = ms / steps;
    timing->graph_replayed = replayed;
    if (m->ferr) {
      unsigned err = 0;
      K_TRY(hipMemcpy(&err, m->ferr, 4, hipMemcpyDeviceToHost), "error word");
      if (err) {
        K_TRY(hipMemset(m->ferr, 0, 4), "error word");
        return fail(VLA_ERR_DEVICE, "persistent solver step: a grid barrier wait gave up (workgroups not co-resident?)");
      }
    }
  }
  return VLA_OK;
}

// ============================================================== bf16 product unit entry point
extern "C" vla_status vla_gemm_bf16(const uint16_t* a, const uint16_t* w, int32_t M, int32_t N, int32_t K,
                                    int32_t epilogue, float* out, void* stream) {
  if (!a || !w || !out) return fail(VLA_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (epilogue != VLA_GEMM_STORE && epilogue != VLA_GEMM_GEGLU && epilogue != VLA_GEMM_RESIDUAL)
    return fail(VLA_ERR_INVALID_ARGUMENT, "epilogue must be VLA_GEMM_STORE, VLA_GEMM_GEGLU or VLA_GEMM_RESIDUAL");
  const bool geglu = epilogue == VLA_GEMM_GEGLU;
  if (M <= 0 || N <= 0 || K <= 0) return fail(VLA_ERR_INVALID_ARGUMENT, "M, N and K must be positive");
  if (K % 64 || N % 32) return fail(VLA_ERR_UNSUPPORTED, "need K % 64 == 0 and N % 32 == 0");
  if ((int64_t)M * K > ((int64_t)1 << 31) || (int64_t)N * K > ((int64_t)1 << 31) || (int64_t)M * N > ((int64_t)1 << 29))
    return fail(VLA_ERR_UNSUPPORTED, "operands too large for the unit entry point");
  vla_status st = check_device();
  if (st != VLA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  // fragment-layout operands: A rows padded to whole 16-row blocks, at least 64 (zero rows)
  const int64_t rows = std::max<int64_t>(64, ((int64_t)M + 15) / 16 * 16);
  uint16_t *ap = nullptr, *af = nullptr, *wf = nullptr;
  float* ws = nullptr;
  auto done = [&](vla_status r) {
    for (void* p : {(void*)ap, (void*)af, (void*)wf, (void*)ws})
      if (p) (void)hipFree(p);
    return r;
  };
  const size_t ws_bytes = (size_t)4 * M * N * 4;  // at most four K splits for a finishing epilogue
  if (lib_malloc((void**)&ap, (size_t)rows * K * 2) != hipSuccess || lib_malloc((void**)&af, (size_t)rows * K * 2) != hipSuccess ||
      lib_malloc((void**)&wf, (size_t)N * K * 2) != hipSuccess || lib_malloc((void**)&ws, ws_bytes) != hipSuccess) {
    (void)hipGetLastError();
    return done(fail(VLA_ERR_OUT_OF_MEMORY, "staging"));
  }
  if (hipMemsetAsync(ap, 0, (size_t)rows * K * 2, s) != hipSuccess ||
      hipMemcpyAsync(ap, a, (size_t)M * K * 2, hipMemcpyDeviceToDevice, s) != hipSuccess ||
      frag_pack(ap, (int)rows, K, af, s) != hipSuccess || frag_pack(w, N, K, wf, s) != hipSuccess)
    return done(fail(VLA_ERR_DEVICE, "operand repack"));
  Epilogue e = epi_store(out, geglu ? N / 2 : N, 1);
  if (geglu) e.kind = EPI_GEGLU;
  hipError_t le = hipSuccess;
  if (epilogue == VLA_GEMM_RESIDUAL) {
    // as the prefix's O projection added into the residual: whole-K row tiles where the prefix uses them,
    // else the tile kernels whose K splits the fixed-order reduction adds into out
    e.kind = EPI_RESID; e.resid = out; e.ldr = N;
    le = gemm_frag(af, wf, M, N, K, e, 0, ws, s);
  } else {
    le = M <= 64 ? gemm_chunk(af, wf, M, N, K, e, kPrefixChunkSplits, ws, s) : gemm_frag(af, wf, M, N, K, e, 0, ws, s);
  }
  if (le != hipSuccess) return done(fail(VLA_ERR_DEVICE, std::string("gemm launch: ") + hipGetErrorString(le)));
  if (hipStreamSynchronize(s) != hipSuccess) return done(fail(VLA_ERR_DEVICE, "gemm sync"));
  return done(VLA_OK);
}

// ============================================================== ternary unit entry points
extern "C" vla_status vla_quantize_rows_i8(const float* x, int32_t M, int32_t K, int8_t* a, float* alpha, void* stream) {
  if (!x || !a || !alpha) return fail(VLA_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (M <= 0 || K <= 0) return fail(VLA_ERR_INVALID_ARGUMENT, "M and K must be positive");
  vla_status st = check_device();
  if (st != VLA_OK) return st;
  K_TRY(quantize_rows(x, K, M, K, a, alpha, (hipStream_t)stream), "quantize");
  return VLA_OK;
}

// Partial sums and counters of one ternary GEMM's K splits, allocated for the
// call (the counters cleared on the stream); freed with free_w2work.
static bool alloc_w2work(int M, int N, W2A8Work& w, hipStream_t s) {
  w.ws_bytes = w2a8_part_bytes(M, N);
  w.ncnt = w2a8_counters(M, N);
  if (lib_malloc((void**)&w.ws, w.ws_bytes) != hipSuccess || lib_malloc((void**)&w.cnt, (size_t)w.ncnt * 4) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return hipMemsetAsync(w.cnt, 0, (size_t)w.ncnt * 4, s) == hipSuccess;
}
static void free_w2work(W2A8Work& w) {
  if (w.ws) (void)hipFree(w.ws);
  if (w.cnt) (void)hipFree(w.cnt);
  w = W2A8Work{};
}

extern "C" vla_status vla_w2a8_gemm(const int8_t* a, const float* alpha, const uint8_t* q_packed, float beta, int32_t M,
                                    int32_t N, int32_t K, int32_t* acc_out, uint16_t* y_bf16, void* stream) {
  if (!a || !alpha || !q_packed) return fail(VLA_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (M <= 0 || N <= 0 || K <= 0) return fail(VLA_ERR_INVALID_ARGUMENT, "M, N and K must be positive");
  if (K % 128 || N % 32) return fail(VLA_ERR_UNSUPPORTED, "need K % 128 == 0 and N % 32 == 0");
  if (!std::isfinite(beta)) return fail(VLA_ERR_INVALID_ARGUMENT, "non-finite beta");
  vla_status st = check_device();
  if (st != VLA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  uint32_t* words = nullptr;
  int* flags = nullptr;
  W2A8Work work;
  auto done = [&](vla_status r) {
    if (words) (void)hipFree(words);
    if (flags) (void)hipFree(flags);
    free_w2work(work);
    return r;
  };
  if (lib_malloc((void**)&words, (size_t)N * K / 4) != hipSuccess || lib_malloc((void**)&flags, 64) != hipSuccess) {
    (void)hipGetLastError();
    return done(fail(VLA_ERR_OUT_OF_MEMORY, "staging"));
  }
  if (!alloc_w2work(M, N, work, s)) return done(fail(VLA_ERR_OUT_OF_MEMORY, "partial sums"));
  if (hipMemsetAsync(flags, 0, 64, s) != hipSuccess) return done(fail(VLA_ERR_DEVICE, "memset"));
  if (ternary_repack(q_packed, N, K, words, flags, s) != hipSuccess) return done(fail(VLA_ERR_DEVICE, "repack"));
  int hf = 0;
  if (hipMemcpyAsync(&hf, flags, 4, hipMemcpyDeviceToHost, s) != hipSuccess || hipStreamSynchronize(s) != hipSuccess)
    return done(fail(VLA_ERR_DEVICE, "flag readback"));
  if (hf) return done(fail(VLA_ERR_INVALID_ARGUMENT, "packed weights contain the invalid code 3"));
  Epilogue e = epi_store(y_bf16, N, 0);
  e.alpha = alpha;
  e.acc_out = acc_out;
  if (gemm_w2a8_scalar(a, K, words, M, N, K, e, beta, s, &work) != hipSuccess)
    return done(fail(VLA_ERR_DEVICE, "w2a8 launch"));
  if (hipStreamSynchronize(s) != hipSuccess) return done(fail(VLA_ERR_DEVICE, "w2a8 sync"));
  return done(VLA_OK);
}

// The same GEMM for callers that cannot allocate: the repacked weight words and
// the invalid-code flag go to the library's fixed per-device scratch array
// (kernels.h, w2a8_scratch) instead of fresh device allocations.  No
// hipMalloc, hipFree or other allocating call is made; calls on one device
// share the array, so calls that overlap on one device race.
extern "C" vla_status vla_w2a8_gemm_noalloc(const int8_t* a, const float* alpha, const uint8_t* q_packed, float beta,
                                            int32_t M, int32_t N, int32_t K, int32_t* acc_out, uint16_t* y_bf16,
                                            void* stream) {
  if (!a || !alpha || !q_packed) return fail(VLA_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (M <= 0 || N <= 0 || K <= 0) return fail(VLA_ERR_INVALID_ARGUMENT, "M, N and K must be positive");
  if (K % 128 || N % 32) return fail(VLA_ERR_UNSUPPORTED, "need K % 128 == 0 and N % 32 == 0");
  if (!std::isfinite(beta)) return fail(VLA_ERR_INVALID_ARGUMENT, "non-finite beta");
  const size_t words_bytes = (size_t)N * (size_t)K / 4;
  if (words_bytes > kW2A8ScratchBytes - kW2A8FlagBytes)
    return fail(VLA_ERR_UNSUPPORTED, "N * K / 4 = " + std::to_string(words_bytes) + " bytes exceeds the fixed scratch of " +
                                         std::to_string(kW2A8ScratchBytes - kW2A8FlagBytes) + " bytes");
  vla_status st = check_device();
  if (st != VLA_OK) return st;
  void* base = nullptr;
  hipError_t e = w2a8_scratch(&base);
  if (e != hipSuccess) return fail(VLA_ERR_DEVICE, std::string("scratch lookup: ") + hipGetErrorString(e));
  hipStream_t s = (hipStream_t)stream;
  uint32_t* words = (uint32_t*)base;
  int* flags = (int*)((char*)base + kW2A8ScratchBytes - kW2A8FlagBytes);
  // the flag keeps the previous call's value: clear it first
  if (hipMemsetAsync(flags, 0, kW2A8FlagBytes, s) != hipSuccess) return fail(VLA_ERR_DEVICE, "flag clear");
  if (ternary_repack(q_packed, N, K, words, flags, s) != hipSuccess) return fail(VLA_ERR_DEVICE, "repack");
  int hf = 0;
  if (hipMemcpyAsync(&hf, flags, 4, hipMemcpyDeviceToHost, s) != hipSuccess || hipStreamSynchronize(s) != hipSuccess)
    return fail(VLA_ERR_DEVICE, "flag readback");
  if (hf) return fail(VLA_ERR_INVALID_ARGUMENT, "packed weights contain the invalid code 3");
  Epilogue ep = epi_store(y_bf16, N, 0);
  ep.alpha = alpha;
  ep.acc_out = acc_out;
  if (gemm_w2a8_scalar(a, K, words, M, N, K, ep, beta, s) != hipSuccess) return fail(VLA_ERR_DEVICE, "w2a8 launch");
  if (hipStreamSynchronize(s) != hipSuccess) return fail(VLA_ERR_DEVICE, "w2a8 sync");
  return VLA_OK;
}

extern "C" vla_status vla_w2a8_gemm_ex(const int8_t* a, const float* alpha, const uint8_t* q_packed, const float* beta,
                                       int32_t group, int32_t path, int32_t M, int32_t N, int32_t K, int32_t* acc_out,
                                       uint16_t* y_bf16, void* stream, float* kernel_ms) {
  if (!a || !alpha || !q_packed || !beta) return fail(VLA_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (M <= 0 || N <= 0 || K <= 0) return fail(VLA_ERR_INVALID_ARGUMENT, "M, N and K must be positive");
  if (group <= 0 || N % group) return fail(VLA_ERR_INVALID_ARGUMENT, "group must be positive and divide N");
  if (path != VLA_W2A8_MFMA && path != VLA_W2A8_DOT4) return fail(VLA_ERR_INVALID_ARGUMENT, "bad path");
  if (path == VLA_W2A8_MFMA && (K % 128 || N % 32)) return fail(VLA_ERR_UNSUPPORTED, "need K % 128 == 0 and N % 32 == 0");
  if (path == VLA_W2A8_DOT4 && K % 64) return fail(VLA_ERR_UNSUPPORTED, "need K % 64 == 0");
  std::vector<float> bn(N);
  for (int n = 0; n < N; ++n) {
    bn[n] = beta[n / group];
    if (!std::isfinite(bn[n])) return fail(VLA_ERR_INVALID_ARGUMENT, "non-finite beta");
  }
  vla_status st = check_device();
  if (st != VLA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  uint32_t* words = nullptr;
  int* flags = nullptr;
  float* bdev = nullptr;
  W2A8Work work;
  hipEvent_t ev[2] = {nullptr, nullptr};
  auto done = [&](vla_status r) {
    if (words) (void)hipFree(words);
    if (flags) (void)hipFree(flags);
    if (bdev) (void)hipFree(bdev);
    free_w2work(work);
    for (hipEvent_t e : ev)
      if (e) (void)hipEventDestroy(e);
    return r;
  };
  if (lib_malloc((void**)&words, (size_t)N * K / 4) != hipSuccess || lib_malloc((void**)&flags, 64) != hipSuccess ||
      lib_malloc((void**)&bdev, (size_t)N * 4) != hipSuccess) {
    (void)hipGetLastError();
    return done(fail(VLA_ERR_OUT_OF_MEMORY, "staging"));
  }
  if (path == VLA_W2A8_MFMA && !alloc_w2work(M, N, work, s)) return done(fail(VLA_ERR_OUT_OF_MEMORY, "partial sums"));
  if (kernel_ms && (hipEventCreate(&ev[0]) != hipSuccess || hipEventCreate(&ev[1]) != hipSuccess))
    return done(fail(VLA_ERR_DEVICE, "events"));
  if (hipMemsetAsync(flags, 0, 64, s) != hipSuccess) return done(fail(VLA_ERR_DEVICE, "memset"));
  if (ternary_repack(q_packed, N, K, words, flags, s) != hipSuccess) return done(fail(VLA_ERR_DEVICE, "repack"));
  int hf = 0;
  if (hipMemcpyAsync(&hf, flags, 4, hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipMemcpyAsync(bdev, bn.data(), (size_t)N * 4, hipMemcpyHostToDevice, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return done(fail(VLA_ERR_DEVICE, "flag readback"));
  if (hf) return done(fail(VLA_ERR_INVALID_ARGUMENT, "packed weights contain the invalid code 3"));
  Epilogue e = epi_store(y_bf16, N, 0);
  e.alpha = alpha;
  e.beta = bdev;
  e.acc_out = acc_out;
  if (kernel_ms && hipEventRecord(ev[0], s) != hipSuccess) return done(fail(VLA_ERR_DEVICE, "event"));
  const hipError_t le = path == VLA_W2A8_MFMA ? gemm_w2a8(a, K, words, M, N, K, e, s, &work)
                                               : gemm_w2a8_dot4(a, K, words, M, N, K, e, 0.f, s);
  if (le != hipSuccess) return done(fail(VLA_ERR_DEVICE, "w2a8 launch"));
  if (kernel_ms && hipEventRecord(ev[1], s) != hipSuccess) return done(fail(VLA_ERR_DEVICE, "event"));
  if (hipStreamSynchronize(s) != hipSuccess) return done(fail(VLA_ERR_DEVICE, "w2a8 sync"));
  if (kernel_ms && hipEventElapsedTime(kernel_ms, ev[0], ev[1]) != hipSuccess)
    return done(fail(VLA_ERR_DEVICE, "elapsed"));
  return done(VLA_OK);
}

extern "C" vla_status vla_ternary_pack(const int8_t* q, int32_t N, int32_t K, uint8_t* packed) {
  if (!q || !packed) return fail(VLA_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (N <= 0 || K <= 0 || K % 4) return fail(VLA_ERR_INVALID_ARGUMENT, "need N, K > 0 and K % 4 == 0");
  for (int64_t i = 0; i < (int64_t)N * K; ++i)
    if (q[i] < -1 || q[i] > 1) return fail(VLA_ERR_INVALID_ARGUMENT, "ternary values must be -1, 0 or +1");
  for (int64_t r = 0; r < N; ++r)
    for (int64_t j = 0; j < K / 4; ++j) {
      uint8_t b = 0;
      for (int i = 0; i < 4; ++i) b |= (uint8_t)((q[r * K + 4 * j + i] + 1) << (2 * i));
      packed[r * (K / 4) + j] = b;
    }
  return VLA_OK;
}

extern "C" vla_status vla_ternary_unpack(const uint8_t* packed, int32_t N, int32_t K, int8_t* q) {
  if (!q || !packed) return fail(VLA_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (N <= 0 || K <= 0 || K % 4) return fail(VLA_ERR_INVALID_ARGUMENT, "need N, K > 0 and K % 4 == 0");
  for (int64_t i = 0; i < (int64_t)N * K / 4; ++i)
    for (int t = 0; t < 4; ++t)
      if (((packed[i] >> (2 * t)) & 3) == 3) return fail(VLA_ERR_INVALID_ARGUMENT, "invalid ternary code 3");
  for (int64_t i = 0; i < (int64_t)N * K / 4; ++i)
    for (int t = 0; t < 4; ++t) q[4 * i + t] = (int8_t)(((packed[i] >> (2 * t)) & 3) - 1);
  return VLA_OK;
}
