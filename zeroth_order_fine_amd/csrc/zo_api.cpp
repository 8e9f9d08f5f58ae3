// Host runtime of libzo: the C-ABI declared in include/zo.h.
//
// Plans, packing and the bank's keys are host objects; every step of the path
// runs in the HIP kernels of this library, launched on the caller's stream.
// The query process follows the arXiv abstract of "Inference-Native
// Zeroth-Order Optimization" (ProbePlan -> candidate evaluation -> estimation ->
// update) and the estimator and lazy update of "Zeroth-Order Fine-Tuning Was an
// Inference Workload All Along" (sections "Why ZO Fine-Tuning Is Really
// Scoring" and "The System Reorganization").
#include "../../include/zo.h"
#include "common.h"
#include <rocprofiler-sdk-roctx/roctx.h>

#include <algorithm>
#include <array>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <deque>
#include <vector>

// Device scratch of zo_score_noalloc: the workspace of a score call, held in the code
// object so that the call allocates nothing.  Each device that loads the library holds its
// own copy for the life of the process.  In host code `scratch` names a host-side stand-in:
// its device address comes from hipGetSymbolAddress, once per device (scratch_init).
static __device__ __align__(256) unsigned char scratch[ZO_NOALLOC_SCRATCH_BYTES];

// A roctx range over one public call (shown by rocprofv3 --marker-trace; free otherwise)
struct CallRange {
  explicit CallRange(const char* name) { roctxRangePushA(name); }
  ~CallRange() { roctxRangePop(); }
  CallRange(const CallRange&) = delete;
  CallRange& operator=(const CallRange&) = delete;
};

namespace {

thread_local std::string g_err;

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
bool g_scratch_tried[kMaxDevices] = {};

// Looks up the scratch array's address on `device`, which must be the current device;
// once per device (later calls return the recorded result).
void* scratch_init(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_tried[device]) {
    g_scratch_tried[device] = true;
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) == hipSuccess) g_scratch_ptr[device] = ptr;
    else (void)hipGetLastError();        // no device here (host-only use): the entry point refuses
  }
  return g_scratch_ptr[device];
}

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

#define ZO_HIP(expr)                                                                             \
  do {                                                                                           \
    hipError_t e_ = (expr);                                                                      \
    if (e_ != hipSuccess) return fail(ZO_E_DEVICE, "%s: %s", #expr, hipGetErrorString(e_));      \
  } while (0)

#define ZO_CHECK(cond, code, ...)                 \
  do {                                            \
    if (!(cond)) return fail(code, __VA_ARGS__);  \
  } while (0)

// ---- launch timing (zo_profile_begin / zo_profile_end) -------------------------
struct Prof {
  bool on = false;
  uint32_t mask = ~0u;        // classes recorded
  std::vector<hipEvent_t> pool;
  size_t used = 0;
  struct Rec { int cls; size_t ev; };
  std::vector<Rec> recs;
};
Prof g_prof;

// Records the start event of a launch of class `cls`; returns the record index or -1.
long prof_start(int cls, hipStream_t s) {
  if (!g_prof.on || !((g_prof.mask >> cls) & 1u)) return -1;
  if (g_prof.used + 2 > g_prof.pool.size()) {
    for (int i = 0; i < 256; ++i) {
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) return -1;
      g_prof.pool.push_back(e);
    }
  }
  const size_t ev = g_prof.used;
  g_prof.used += 2;
  if (hipEventRecord(g_prof.pool[ev], s) != hipSuccess) return -1;
  g_prof.recs.push_back({cls, ev});
  return (long)g_prof.recs.size() - 1;
}
void prof_stop(long rec, hipStream_t s) {
  if (rec < 0) return;
  (void)hipEventRecord(g_prof.pool[g_prof.recs[rec].ev + 1], s);
}
struct ProfScope {
  long rec;
  hipStream_t s;
  ProfScope(int cls, hipStream_t st) : rec(prof_start(cls, st)), s(st) {}
  ~ProfScope() { prof_stop(rec, s); }
};

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

// ---- parameters and layout -----------------------------------------------------
enum { G_TOK = 0, G_POS = 1, G_FNW = 2, G_FNB = 3, G_HEAD = 4, N_GLOBAL = 5 };
enum {
  P_LN1W = 0, P_LN1B, P_WQ, P_BQ, P_WK, P_BK, P_WV, P_BV, P_WO, P_BO, P_LN2W, P_LN2B,
  P_W1, P_B1, P_W2, P_B2, P_WDOWN, P_QNW, P_KNW, N_LAYER_PARAMS
};

struct TLoc {
  bool present = false;
  size_t off = 0;
  int64_t rows = 0, cols = 0;
  int32_t dtype = ZO_DTYPE_F32;
  int32_t layout = 0;   // 0 plain, 1 gate / 2 up of a 16-row interleave
  bool gain = false;    // initialised as 1 + 0.02 z
};

struct Layout {
  size_t bytes = 0;
  std::array<TLoc, N_GLOBAL> g;
  std::vector<std::array<TLoc, N_LAYER_PARAMS>> L;
};

bool is_opt(const zo_model_desc& d) { return d.arch == ZO_ARCH_OPT; }
// bf16 and fp8 models share the bf16 kernels (activations, attention, side path, head);
// fp8 models differ only in their layer linears and those linears' inputs
bool bf16_like(const zo_model_desc& d) { return d.dtype == ZO_DTYPE_BF16 || d.dtype == ZO_DTYPE_FP8; }
bool is_fp8(const zo_model_desc& d) { return d.dtype == ZO_DTYPE_FP8; }
int n_kinds_of(const zo_model_desc& d) { return is_opt(d) ? 6 : 7; }

int validate_desc(const zo_model_desc* d) {
  ZO_CHECK(d, ZO_E_INVAL, "null model descriptor");
  ZO_CHECK(d->abi_version == ZO_ABI_VERSION, ZO_E_ABI, "descriptor ABI %d, library ABI %d", d->abi_version,
           ZO_ABI_VERSION);
  ZO_CHECK(d->arch == ZO_ARCH_OPT || d->arch == ZO_ARCH_QWEN3, ZO_E_INVAL, "unknown arch %d", d->arch);
  ZO_CHECK(d->dtype == ZO_DTYPE_F32 || d->dtype == ZO_DTYPE_BF16 || d->dtype == ZO_DTYPE_FP8, ZO_E_INVAL,
           "unknown dtype %d", d->dtype);
  ZO_CHECK(d->n_layers >= 1 && d->d_model >= 1 && d->n_heads >= 1 && d->n_kv_heads >= 1 && d->head_dim >= 1 &&
               d->d_ffn >= 1 && d->vocab >= 2 && d->max_pos >= 1,
           ZO_E_INVAL, "model sizes must be positive");
  ZO_CHECK(d->n_heads % d->n_kv_heads == 0, ZO_E_INVAL, "n_heads must be a multiple of n_kv_heads");
  ZO_CHECK(is_opt(*d) ? d->n_kv_heads == d->n_heads : true, ZO_E_INVAL, "OPT has n_kv_heads == n_heads");
  ZO_CHECK(d->head_dim == 16 || d->head_dim == 32 || d->head_dim == 64 || d->head_dim == 128, ZO_E_INVAL,
           "head_dim must be 16, 32, 64 or 128");
  ZO_CHECK(d->dtype == ZO_DTYPE_F32 || d->head_dim >= 32, ZO_E_INVAL, "bf16 attention needs head_dim >= 32");
  ZO_CHECK(d->d_model <= 6144 && d->d_model % 4 == 0, ZO_E_INVAL,
           "d_model must be a multiple of 4 and at most 6144 (norm kernels)");
  ZO_CHECK(std::isfinite(d->norm_eps) && d->norm_eps > 0, ZO_E_INVAL, "norm_eps must be > 0");
  ZO_CHECK(is_opt(*d) || (std::isfinite(d->rope_theta) && d->rope_theta > 1.0), ZO_E_INVAL,
           "rope_theta must be > 1");
  ZO_CHECK(is_opt(*d) || d->d_ffn % 16 == 0, ZO_E_INVAL, "Qwen3 d_ffn must be a multiple of 16");
  ZO_CHECK(d->dtype != ZO_DTYPE_FP8 || (d->d_model % 128 == 0 && d->d_ffn % 128 == 0 &&
                                        (d->n_heads * d->head_dim) % 128 == 0),
           ZO_E_INVAL, "fp8 models: d_model, d_ffn and n_heads * head_dim multiples of 128 (the e4m3 K-step)");
  return ZO_OK;
}

Layout make_layout(const zo_model_desc& d) {
  Layout Lo;
  size_t off = 0;
  const int mdt = d.dtype;                                   // layer linears
  const int gdt = d.dtype == ZO_DTYPE_FP8 ? ZO_DTYPE_BF16 : mdt;   // embeddings and head
  auto esz = [](int dt) { return dt == ZO_DTYPE_FP8 ? (size_t)1 : dt == ZO_DTYPE_BF16 ? (size_t)2 : (size_t)4; };
  auto place = [&](TLoc& t, int64_t rows, int64_t cols, int dt, bool aligned, bool gain = false) {
    if (aligned) off = align_up(off, 256);
    t.present = true; t.off = off; t.rows = rows; t.cols = cols; t.dtype = dt; t.gain = gain;
    off += (size_t)rows * cols * esz(dt);
  };
  const int64_t D = d.d_model, V = d.vocab, F = d.d_ffn;
  const int64_t NQ = (int64_t)d.n_heads * d.head_dim, NKV = (int64_t)d.n_kv_heads * d.head_dim;
  place(Lo.g[G_TOK], V, D, gdt, true);
  if (is_opt(d)) place(Lo.g[G_POS], d.max_pos, D, gdt, true);
  place(Lo.g[G_FNW], 1, D, ZO_DTYPE_F32, true, true);
  if (is_opt(d)) place(Lo.g[G_FNB], 1, D, ZO_DTYPE_F32, true);
  if (!is_opt(d)) place(Lo.g[G_HEAD], V, D, gdt, true);
  Lo.L.resize(d.n_layers);
  for (int l = 0; l < d.n_layers; ++l) {
    auto& P = Lo.L[l];
    if (is_opt(d)) {
      place(P[P_LN1W], 1, D, ZO_DTYPE_F32, true, true);
      place(P[P_LN1B], 1, D, ZO_DTYPE_F32, true);
      place(P[P_WQ], NQ, D, mdt, true);
      place(P[P_WK], NKV, D, mdt, false);
      place(P[P_WV], NKV, D, mdt, false);
      place(P[P_BQ], 1, NQ, ZO_DTYPE_F32, true);
      place(P[P_BK], 1, NKV, ZO_DTYPE_F32, false);
      place(P[P_BV], 1, NKV, ZO_DTYPE_F32, false);
      place(P[P_WO], D, NQ, mdt, true);
      place(P[P_BO], 1, D, ZO_DTYPE_F32, true);
      place(P[P_LN2W], 1, D, ZO_DTYPE_F32, true, true);
      place(P[P_LN2B], 1, D, ZO_DTYPE_F32, true);
      place(P[P_W1], F, D, mdt, true);
      place(P[P_B1], 1, F, ZO_DTYPE_F32, true);
      place(P[P_W2], D, F, mdt, true);
      place(P[P_B2], 1, D, ZO_DTYPE_F32, true);
    } else {
      place(P[P_LN1W], 1, D, ZO_DTYPE_F32, true, true);
      place(P[P_WQ], NQ, D, mdt, true);
      place(P[P_WK], NKV, D, mdt, false);
      place(P[P_WV], NKV, D, mdt, false);
      place(P[P_QNW], 1, d.head_dim, ZO_DTYPE_F32, true, true);
      place(P[P_KNW], 1, d.head_dim, ZO_DTYPE_F32, true, true);
      place(P[P_WO], D, NQ, mdt, true);
      place(P[P_LN2W], 1, D, ZO_DTYPE_F32, true, true);
      // gate/up: one packed [2F x D] matrix, 16-row interleave
      place(P[P_W1], 2 * F, D, mdt, true);
      P[P_W1].rows = F; P[P_W1].layout = 1;
      P[P_W2] = P[P_W1]; P[P_W2].layout = 2;
      place(P[P_WDOWN], D, F, mdt, true);
    }
  }
  Lo.bytes = align_up(off, 256);
  return Lo;
}

// ---- kinds ---------------------------------------------------------------------
struct KindShape { int64_t n_out, n_in; };
KindShape kind_shape(const zo_model_desc& d, int kind) {
  const int64_t D = d.d_model, F = d.d_ffn;
  const int64_t NQ = (int64_t)d.n_heads * d.head_dim, NKV = (int64_t)d.n_kv_heads * d.head_dim;
  switch (kind) {
    case ZO_KIND_Q: return {NQ, D};
    case ZO_KIND_K: return {NKV, D};
    case ZO_KIND_V: return {NKV, D};
    case ZO_KIND_O: return {D, NQ};
    case 4: return {F, D};                              // fc1 / gate
    case 5: return is_opt(d) ? KindShape{D, F} : KindShape{F, D};   // fc2 / up
    default: return {D, F};                             // down
  }
}

inline uint32_t dir_tag(int layer, int kind, int factor) {
  return ((uint32_t)layer << 8) | ((uint32_t)kind << 1) | (uint32_t)factor;
}
inline uint32_t weight_tag(int slot, int param) { return (1u << 30) | ((uint32_t)slot << 8) | (uint32_t)param; }

}  // namespace

// ---- opaque objects --------------------------------------------------------------
// The forward launch sequence of zo_score captured as a HIP graph, with what its kernel
// arguments were derived from (see graph_key).
struct GraphCache {
  bool on = false;                 // zo_model_set_graphs
  std::vector<int64_t> key;
  std::vector<int64_t> pending;    // the last eager call's key: captured when it repeats
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  void reset() {
    if (exec) (void)hipGraphExecDestroy(exec);
    if (graph) (void)hipGraphDestroy(graph);
    exec = nullptr;
    graph = nullptr;
    key.clear();
    pending.clear();
  }
};

struct zo_model {
  zo_model_desc d;
  Layout lo;
  unsigned char* w = nullptr;
  size_t w_bytes = 0;
  float2* rope = nullptr;   // [rope_len x head_dim/2] (cos, sin), Qwen3
  int rope_len = 0;
  int device = 0;
  int n_cu = 0;        // compute units of the device (0: unknown, no split-tail projections)
  GraphCache gc;       // zo_score's forward pass
  GraphCache gcd;      // a decode step of zo_generate
};

struct zo_plan_s {
  zo_model_desc md;
  uint64_t t;
  uint32_t nu;
  int rank;
  double eps, eps_tilde;
  std::vector<uint64_t> seeds;
  std::vector<int32_t> cdir, csign;
  uint32_t mask, flags;
  uint64_t window() const { return t / nu; }
};

struct zo_bank {
  zo_model_desc md;
  int n_slots, rank;
  uint32_t mask;
  float* u = nullptr;
  size_t bytes = 0;
  std::vector<uint64_t> seeds;
  std::vector<int64_t> windows;
  std::vector<int> kinds;            // target kinds, increasing
  std::vector<int64_t> kind_off;     // floats within a layer
  int64_t layer_stride = 0;          // floats per layer
  int64_t slot_stride = 0;           // floats per slot
};

namespace {

int bank_geometry(const zo_model_desc& d, int rank, uint32_t mask, std::vector<int>& kinds,
                  std::vector<int64_t>& koff, int64_t& layer_stride) {
  kinds.clear(); koff.clear();
  int64_t o = 0;
  for (int k = 0; k < n_kinds_of(d); ++k)
    if (mask & (1u << k)) {
      kinds.push_back(k);
      koff.push_back(o);
      o += kind_shape(d, k).n_out * rank;
    }
  layer_stride = o;
  return ZO_OK;
}

// A plan or a bank made for one model describes shapes (kinds, n_out, n_in, layers) that
// the launches of another model would index with; every call that takes a plan or bank
// together with a model checks that they were made for the same shapes.
bool same_shape(const zo_model_desc& a, const zo_model_desc& b) {
  return a.arch == b.arch && a.dtype == b.dtype && a.n_layers == b.n_layers && a.d_model == b.d_model &&
         a.n_heads == b.n_heads && a.n_kv_heads == b.n_kv_heads && a.head_dim == b.head_dim && a.d_ffn == b.d_ffn;
}

int check_objects(const zo_model* m, const zo_plan_s* p, const zo_bank* bank) {
  ZO_CHECK(!p || same_shape(p->md, m->d), ZO_E_STATE, "plan was made for another model");
  ZO_CHECK(!bank || same_shape(bank->md, m->d), ZO_E_STATE, "bank was made for another model");
  return ZO_OK;
}

// GEMM input groups of a layer: which kinds read the same activations.
struct Group {
  std::vector<int> kinds;   // kind of each column block of the side input
  bool interleaved = false; // gate/up packed GEMM (both kinds in one tile)
};

std::vector<Group> layer_groups(const zo_model_desc& d) {
  std::vector<Group> g(4);
  g[0].kinds = {ZO_KIND_Q, ZO_KIND_K, ZO_KIND_V};
  g[1].kinds = {ZO_KIND_O};
  if (is_opt(d)) {
    g[2].kinds = {4};
    g[3].kinds = {5};
  } else {
    g[2].kinds = {4, 5};
    g[2].interleaved = true;
    g[3].kinds = {6};
  }
  return g;
}

// ---- workspace bump allocator ------------------------------------------------------
struct Bump {
  unsigned char* base;
  size_t off = 0;
  explicit Bump(void* b) : base((unsigned char*)b) {}
  template <typename T>
  T* take(size_t count) {
    off = align_up(off, 256);
    T* p = base ? (T*)(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
};

// Everything zo_score needs to know about one batch under one plan and bank.
struct Packing {
  int n_phys = 0;
  int64_t M = 0, n_scored = 0;
  std::vector<int32_t> phys_seq, phys_cand, phys_cu, phys_first;
  std::vector<int32_t> row_src, row_pos, row_cand;
  std::vector<int32_t> sc_row, sc_lab_src;
  std::vector<int32_t> work;
  int max_len = 0;
};

int validate_batch(const zo_model_desc& d, const zo_batch* b) {
  ZO_CHECK(b, ZO_E_INVAL, "null batch");
  ZO_CHECK(b->n_seq >= 0, ZO_E_INVAL, "n_seq < 0");
  if (b->n_seq == 0) return ZO_OK;
  ZO_CHECK(b->cu_seqlens && b->role && b->score_mode, ZO_E_INVAL, "null batch array");
  ZO_CHECK(b->cu_seqlens[0] == 0, ZO_E_SHAPE, "cu_seqlens[0] must be 0");
  for (int i = 0; i < b->n_seq; ++i) {
    const int len = b->cu_seqlens[i + 1] - b->cu_seqlens[i];
    ZO_CHECK(len >= 1, ZO_E_SHAPE, "sequence %d has length %d", i, len);
    ZO_CHECK(b->role[i] == ZO_ROLE_PROBE || b->role[i] == ZO_ROLE_FOREGROUND, ZO_E_INVAL, "bad role");
    ZO_CHECK(b->score_mode[i] == ZO_SCORE_LAST_LABEL || b->score_mode[i] == ZO_SCORE_ALL_NEXT, ZO_E_INVAL,
             "bad score mode");
    ZO_CHECK(b->score_mode[i] != ZO_SCORE_LAST_LABEL || len >= 2, ZO_E_SHAPE,
             "LAST_LABEL sequence %d needs length >= 2", i);
    ZO_CHECK(len <= d.max_pos, ZO_E_SHAPE, "sequence %d longer than max_pos", i);
    ZO_CHECK(len <= 4095 * 64, ZO_E_SHAPE, "sequence %d too long", i);
  }
  ZO_CHECK(b->tokens_dev || b->cu_seqlens[b->n_seq] == 0, ZO_E_INVAL, "null tokens");
  return ZO_OK;
}

void build_packing(const zo_plan_s& p, const zo_batch& b, Packing& pk) {
  pk = Packing();
  auto add = [&](int li, int c) {
    pk.phys_seq.push_back(li);
    pk.phys_cand.push_back(c);
  };
  for (int i = 0; i < b.n_seq; ++i)
    if (b.role[i] == ZO_ROLE_FOREGROUND) add(i, -1);
  for (int c = 0; c < (int)p.cdir.size(); ++c)
    for (int i = 0; i < b.n_seq; ++i)
      if (b.role[i] == ZO_ROLE_PROBE) add(i, c);
  pk.n_phys = (int)pk.phys_seq.size();
  pk.phys_cu.assign(1, 0);
  pk.phys_first.assign(1, 0);
  for (int q = 0; q < pk.n_phys; ++q) {
    const int li = pk.phys_seq[q], c = pk.phys_cand[q];
    const int start = b.cu_seqlens[li], len = b.cu_seqlens[li + 1] - start;
    const int prow0 = (int)pk.M;
    for (int t = 0; t < len; ++t) {
      pk.row_src.push_back(start + t);
      pk.row_pos.push_back(t);
      pk.row_cand.push_back(c);
    }
    if (b.score_mode[li] == ZO_SCORE_LAST_LABEL) {
      pk.sc_row.push_back(prow0 + len - 2);
      pk.sc_lab_src.push_back(start + len - 1);
    } else {
      for (int t = 0; t + 1 < len; ++t) {
        pk.sc_row.push_back(prow0 + t);
        pk.sc_lab_src.push_back(start + t + 1);
      }
    }
    for (int qb = 0; qb * 64 < len; ++qb) pk.work.push_back((q << 12) | qb);
    pk.M += len;
    pk.max_len = std::max(pk.max_len, len);
    pk.phys_cu.push_back((int32_t)pk.M);
    pk.phys_first.push_back((int32_t)pk.sc_row.size());
  }
  pk.n_scored = (int64_t)pk.sc_row.size();
}

// Side-path geometry of a plan + bank (independent of the batch contents).
// Side-path geometry.  Per target kind, As holds (E + q) blocks of r columns (E bank
// entries, then one block per direction; ks columns with padding) and Bs the matching
// [U_j | G_d].  The side-input projection computes t only for the distinct V factors:
// a direction whose (seed, window) is a bank entry's key has the entry's V, so its t is
// the entry's and is not computed twice (nc = E + directions without an entry).
struct SideGeom {
  bool any = false;
  int E = 0, q = 0, r = 0;
  int used = 0, ks = 0;             // As columns per kind: (E + q) r, padded to ks
  int nc = 0, ks_c = 0;             // computed t slots and their columns per kind (padded)
  std::vector<int> entry_slots;     // active bank slots in slot order
  std::vector<int> dslot;           // per direction: its computed t slot (< E: an entry's)
  std::vector<int> cdirs;           // computed slots >= E: their direction
  std::vector<Group> groups;
  std::vector<bool> group_on;       // group has at least one target kind
  std::vector<int64_t> vt_rows;     // rows of the group's V^T block = computed t columns (per layer)
  std::vector<int64_t> as_cols;     // As columns of the group (kinds x ks)
  std::vector<int64_t> bs_cols;     // ks_tile of the group's GEMM
  std::vector<int64_t> bs_rows;     // physical output rows of the group's GEMM
  std::vector<int64_t> n_in;
};

int side_geometry(const zo_model* m, const zo_plan_s& p, const zo_bank* bank, SideGeom& sg) {
  const zo_model_desc& d = m->d;
  sg = SideGeom();
  if (int rc = check_objects(m, &p, bank)) return rc;
  sg.q = (int)p.seeds.size();
  sg.r = p.rank;
  if (bank) {
    ZO_CHECK(bank->rank == p.rank, ZO_E_STATE, "bank rank %d != plan rank %d", bank->rank, p.rank);
    ZO_CHECK(bank->mask == p.mask, ZO_E_STATE, "bank target mask differs from the plan's");
    for (int s = 0; s < bank->n_slots; ++s)
      if (bank->windows[s] >= 0) sg.entry_slots.push_back(s);
  }
  sg.E = (int)sg.entry_slots.size();
  const int bk = gemm_bk(bf16_like(d));
  sg.used = (sg.E + sg.q) * sg.r;
  sg.ks = (int)round_up(sg.used, bk);
  sg.nc = sg.E;
  for (int dd = 0; dd < sg.q; ++dd) {
    int slot = -1;
    for (int j = 0; j < sg.E && bank; ++j)
      if (bank->seeds[sg.entry_slots[j]] == p.seeds[dd] && bank->windows[sg.entry_slots[j]] == (int64_t)p.window())
        slot = j;
    if (slot < 0) {
      slot = sg.nc++;
      sg.cdirs.push_back(dd);
    }
    sg.dslot.push_back(slot);
  }
  // computed t columns per kind: an output width of the side-input projection (any
  // multiple of 32 serves), not a K extent like ks
  sg.ks_c = (int)round_up(sg.nc * sg.r, bf16_like(d) ? 32 : bk);
  sg.groups = layer_groups(d);
  const int64_t D = d.d_model, F = d.d_ffn;
  const int64_t NQ = (int64_t)d.n_heads * d.head_dim, NKV = (int64_t)d.n_kv_heads * d.head_dim;
  const int64_t nin[4] = {D, NQ, D, F};
  const int64_t nrows[4] = {NQ + 2 * NKV, D, is_opt(d) ? F : 2 * F, D};
  for (int g = 0; g < 4; ++g) {
    bool on = false;
    for (int k : sg.groups[g].kinds) on |= (p.mask >> k) & 1u;
    sg.group_on.push_back(on);
    sg.any |= on;
    const int nb = (int)sg.groups[g].kinds.size();
    sg.vt_rows.push_back(on ? (int64_t)nb * sg.ks_c : 0);
    sg.as_cols.push_back(on ? (int64_t)nb * sg.ks : 0);
    sg.bs_cols.push_back(on ? (sg.groups[g].interleaved ? (int64_t)nb * sg.ks : sg.ks) : 0);
    sg.bs_rows.push_back(nrows[g]);
    sg.n_in.push_back(nin[g]);
    ZO_CHECK(!is_fp8(d) || sg.vt_rows[g] <= 128, ZO_E_SHAPE,
             "fp8 models: side-input projection of %lld columns (rank x computed slots per kind, at most 128)",
             (long long)sg.vt_rows[g]);
  }
  return ZO_OK;
}

constexpr int kMaxDecodeSplit = 8;   // K-slices of a decode-step projection, at most

struct WsPtrs {
  int32_t *row_src, *row_pos, *row_cand, *phys_cu, *phys_first, *sc_row, *sc_lab_src, *work, *labels;
  int32_t* cand_dir;
  int32_t* cand_slot;           // computed t slot of the candidate's direction
  int32_t* bad_ids;             // [0]: set by the kernels when a token id lies outside [0, vocab);
                                // [1]: set by a split-tail projection whose wait gave up
  float* sk_part = nullptr;     // split-tail projections: accumulator images and flags (null: none)
  int32_t* sk_flag = nullptr;
  float* cand_scale;
  SideJob* jobs;
  int64_t as_ld;                // As row pitch (elements), the same for every group
  float* h;
  void *xa, *qkv, *attn, *hid, *as, *xs;
  std::vector<void*> vt, bs;   // per layer*4 + group
  unsigned char* side_begin = nullptr;
  size_t side_bytes = 0;
  float* tp_partial;
  float* sf_part;               // partial sums of the FFN input's side input (fc1 / gate-up epilogue)
  float2* part;
  float* lab_logit;
  double *tok64, *seq_logp;
  // generation only: per-layer K and V caches, cache row of every packed row, first cache
  // row of every physical sequence, current tokens, first column of each tile's maximum
  void *kcache = nullptr, *vcache = nullptr;
  int64_t kv_layer_elems = 0;
  int32_t *kv_first = nullptr, *row_cache = nullptr, *gen_tok = nullptr, *part_idx = nullptr;
  float* proj_partial = nullptr;   // K-slice partial sums of decode-step projections
  size_t bytes;
};

// K-split of the side-input projection: only for the narrow case (one column tile),
// chosen from N and K alone so that a row's result never depends on the batch.
int tproj_split(const zo_model_desc& d, int64_t n_cols, int64_t k) {
  if (!bf16_like(d) || n_cols == 0) return 1;
  // wide outputs (the pipelined kernel, 256 x 256 tiles): two K-slices, so that a few
  // column tiles over the batch's row tiles still fill the CUs
  if (n_cols > 128) return (k % 128 == 0 && k / 128 >= 8) ? 2 : 1;
  // the 128 x 32 tile (n_cols <= 32) has half as many row tiles as the 64 x 128 one
  int s = n_cols <= 32 ? 8 : 4;
  while (s > 1 && (k % (64 * s) != 0 || k / (64 * s) < 8)) s >>= 1;
  return s;
}

// bytes per activation element (fp8 models: bf16 except the e4m3 linear inputs, which
// take the same buffers at one byte an element)
// Decode steps of generation (one row per sequence, no batch invariance to keep): narrow
// side-input projections in K-slices of two to four 64-deep steps, up to 32 slices; the
// K loop of the register-staged kernel is latency-bound at these few rows.
int tproj_split_decode(const zo_model_desc& d, int64_t n_cols, int64_t k) {
  if (!bf16_like(d) || n_cols == 0 || n_cols > 128) return tproj_split(d, n_cols, k);
  int s = 32;
  while (s > 1 && (k % (64 * s) != 0 || k / (64 * s) < 2)) s >>= 1;
  return s;
}

size_t act_size(const zo_model_desc& d) { return bf16_like(d) ? 2 : 4; }
// Two-term rounding sites of a plan (ZO_PLAN_ACT_SPLIT = all of them)
uint32_t split_sites(const zo_plan_s& p) {
  return (p.flags & ZO_PLAN_ACT_SPLIT) ? (uint32_t)ZO_PLAN_SPLIT_SITES : (p.flags & ZO_PLAN_SPLIT_SITES);
}
bool split_act(const zo_plan_s& p) { return split_sites(p) != 0; }
// input of the projections of side group g (0 q|k|v, 1 o, 2 fc1 / gate-up, 3 fc2 / down)
bool split_group(const zo_plan_s& p, int g) {
  static const uint32_t site[4] = {ZO_PLAN_SPLIT_QKV_IN, ZO_PLAN_SPLIT_ATTN, ZO_PLAN_SPLIT_FC1_IN,
                                   ZO_PLAN_SPLIT_FC2_IN};
  return (split_sites(p) & site[g]) != 0;
}
bool split_head(const zo_plan_s& p) { return (split_sites(p) & ZO_PLAN_SPLIT_HEAD) != 0; }
// As columns per row: the widest group.  Every group writes, for a given row, the same
// column offsets inside each ks-wide block, so one zero fill per call keeps the
// columns that no group writes at zero.
int64_t as_stride(const SideGeom& sg) {
  int64_t c = 0;
  for (int g = 0; g < 4; ++g) c = std::max(c, sg.as_cols[g]);
  return c;
}

// The side input of the last projection of the FFN (fc2 / down) formed in the epilogue of the
// projection that writes its input (GELU / SwiGLU): bf16 and fp8 models, one-term
// activations, at most 4 used factor columns.
bool side_in_ffn_epilogue(const zo_model_desc& d, const zo_plan_s& p, const SideGeom& sg) {
  return bf16_like(d) && !split_group(p, 3) && sg.group_on.size() == 4 && sg.group_on[3] &&
         (sg.vt_rows[3] / sg.ks_c) * (int64_t)(sg.nc * sg.r) <= 4;
}

int n_side_jobs(const zo_model_desc& d, const zo_plan_s& p, const SideGeom& sg) {
  if (!sg.any) return 0;
  int per_kind = 0;
  per_kind += sg.nc;         // V rows of the computed t slots
  per_kind += sg.E + sg.q;   // Bs columns (U entries, G directions)
  int kinds = 0;
  for (int k = 0; k < n_kinds_of(d); ++k) kinds += (p.mask >> k) & 1u;
  return d.n_layers * kinds * per_kind;
}

// Split-tail projections (q|k|v, o and fc2 / down of bf16 models, 256x256 tiles) need room
// for two 256 x 256 fp32 accumulator images and two flags per workgroup; reserved when the
// widest of them spans at least one round of ZO_SK_MAX_WG tiles at this batch.
bool sk_workspace(const zo_model_desc& d, int64_t M) {
  if (d.dtype != ZO_DTYPE_BF16) return false;
  const int64_t nqkv = (int64_t)(d.n_heads + 2 * d.n_kv_heads) * d.head_dim;
  return ((M + 255) / 256) * ((std::max<int64_t>(nqkv, d.d_model) + 255) / 256) >= ZO_SK_MAX_WG;
}

// kv_rows > 0: a generation call whose caches hold kv_rows rows per layer
void carve(const zo_model* m, const zo_plan_s& p, const Packing& pk, const SideGeom& sg, void* base, WsPtrs& w,
           int64_t kv_rows = 0) {
  const zo_model_desc& d = m->d;
  const size_t as = act_size(d);
  Bump b(base);
  const int64_t M = std::max<int64_t>(pk.M, 1), S = std::max<int64_t>(pk.n_scored, 1);
  const int nc = (int)p.cdir.size();
  w.row_src = b.take<int32_t>(M);
  w.row_pos = b.take<int32_t>(M);
  w.row_cand = b.take<int32_t>(M);
  w.phys_cu = b.take<int32_t>(pk.n_phys + 1);
  w.phys_first = b.take<int32_t>(pk.n_phys + 1);
  w.sc_row = b.take<int32_t>(S);
  w.sc_lab_src = b.take<int32_t>(S);
  w.work = b.take<int32_t>(std::max<size_t>(pk.work.size(), 1));
  w.labels = b.take<int32_t>(S);
  w.cand_dir = b.take<int32_t>(nc);
  w.cand_slot = b.take<int32_t>(nc);
  w.bad_ids = b.take<int32_t>(2);
  w.cand_scale = b.take<float>(nc);
  w.jobs = b.take<SideJob>(std::max(n_side_jobs(d, p, sg), 1));
  const int64_t D = d.d_model, F = d.d_ffn;
  const int64_t NQ = (int64_t)d.n_heads * d.head_dim, NKV = (int64_t)d.n_kv_heads * d.head_dim;
  // two-term activations at a site: [hi | lo] rows (x2), fp32 q|k|v, factor blocks
  // hi | hi | lo (x3) of the groups that read a split site
  auto x2g = [&](int g) -> int64_t { return split_group(p, g) ? 2 : 1; };
  auto x3g = [&](int g) -> int64_t { return split_group(p, g) ? 3 : 1; };
  const int64_t x2n = (split_group(p, 0) || split_group(p, 2)) ? 2 : 1;   // the two norm outputs share xa
  w.h = b.take<float>(M * D);
  w.xa = b.take<unsigned char>(M * D * as * x2n);
  w.qkv = b.take<unsigned char>(M * (NQ + 2 * NKV) * (split_group(p, 1) ? sizeof(float) : as));
  w.attn = b.take<unsigned char>(M * NQ * as * x2g(1));
  w.hid = b.take<unsigned char>(M * F * as * x2g(3));
  w.as_ld = std::max<int64_t>(as_stride(sg), 1) * (split_act(p) ? 2 : 1);
  w.as = b.take<unsigned char>(M * w.as_ld * as);
  w.vt.assign((size_t)d.n_layers * 4, nullptr);
  w.bs.assign((size_t)d.n_layers * 4, nullptr);
  b.off = align_up(b.off, 256);
  const size_t side0 = b.off;
  for (int l = 0; l < d.n_layers; ++l)
    for (int g = 0; g < 4; ++g)
      if (sg.group_on[g]) {
        w.vt[l * 4 + g] = b.take<unsigned char>(sg.vt_rows[g] * sg.n_in[g] * as * x3g(g));
        w.bs[l * 4 + g] = b.take<unsigned char>(sg.bs_rows[g] * sg.bs_cols[g] * as * x3g(g));
      }
  w.side_begin = base ? (unsigned char*)base + side0 : nullptr;
  w.side_bytes = b.off - side0;
  w.xs = b.take<unsigned char>(S * D * as * (split_head(p) ? 2 : 1));
  if (sk_workspace(d, pk.M)) {
    w.sk_part = b.take<float>((int64_t)2 * ZO_SK_MAX_WG * 256 * 256);
    w.sk_flag = b.take<int32_t>(3 * ZO_SK_MAX_WG);
  }
  {
    int64_t np = 0, npd = 0;
    for (int g = 0; g < 4; ++g) {
      np = std::max(np, (int64_t)tproj_split(d, sg.vt_rows[g], sg.n_in[g] * x3g(g)) * sg.vt_rows[g]);
      npd = std::max(npd, (int64_t)tproj_split_decode(d, sg.vt_rows[g], sg.n_in[g]) * sg.vt_rows[g]);
    }
    const int64_t n = std::max<int64_t>(np * M, kv_rows > 0 ? npd * std::max(pk.n_phys, 1) : 0);
    w.tp_partial = b.take<float>(std::max<int64_t>(n, 1));
  }
  {
    const int64_t n1 = is_opt(d) ? F : 2 * F;           // columns of the fc1 / gate-up projection
    w.sf_part = side_in_ffn_epilogue(d, p, sg) ? b.take<float>(M * ((n1 + 127) / 128) * 4) : nullptr;
  }
  const int bn_head = gemm_cfg_bn(GEMM_CFG_HEAD, bf16_like(d));
  const int64_t n_vt = (d.vocab + bn_head - 1) / bn_head;
  w.part = b.take<float2>(S * n_vt);
  w.lab_logit = b.take<float>(S);
  w.tok64 = b.take<double>(S);
  w.seq_logp = b.take<double>(std::max(pk.n_phys, 1));
  if (kv_rows > 0) {
    w.kv_first = b.take<int32_t>(pk.n_phys + 1);
    w.row_cache = b.take<int32_t>(M);
    w.gen_tok = b.take<int32_t>(std::max(pk.n_phys, 1));
    w.part_idx = b.take<int32_t>(S * n_vt);
    w.kv_layer_elems = kv_rows * NKV;
    w.kcache = b.take<unsigned char>(d.n_layers * w.kv_layer_elems * as);
    w.vcache = b.take<unsigned char>(d.n_layers * w.kv_layer_elems * as);
    const int64_t max_n = std::max<int64_t>(NQ + 2 * NKV, std::max<int64_t>(D, is_opt(d) ? F : 2 * F));
    w.proj_partial = b.take<float>((int64_t)kMaxDecodeSplit * std::max(pk.n_phys, 1) * max_n);
  }
  w.bytes = align_up(b.off, 256);
}

int check_i32(int64_t elems, const char* what) {
  ZO_CHECK(elems < ((int64_t)1 << 31), ZO_E_SHAPE, "%s has %lld elements; the GEMM uses 32-bit offsets", what,
           (long long)elems);
  return ZO_OK;
}

int run_gemm(const zo_model_desc& d, const GemmParams& gp, int cfg, hipStream_t s) {
  ProfScope ps(cfg == GEMM_CFG_BIG ? ZO_PROF_GEMM_BASE : (cfg == GEMM_CFG_NARROW ? ZO_PROF_GEMM_SIDE : ZO_PROF_GEMM_HEAD),
               s);
  if (bf16_like(d)) {
    const int bn = gemm_cfg_bn(cfg, true);
    for (int i = 0; i < gp.n_bounds; ++i)
      ZO_CHECK(gp.bounds[i] % bn == 0, ZO_E_SHAPE, "kind boundary %d not a multiple of the %d-column tile",
               gp.bounds[i], bn);
    const int bk = (gp.a_e4m3 && gp.b_e4m3) ? 128 : gemm_cfg_bk(cfg, true);
    ZO_CHECK(gp.ks_tile % gemm_cfg_bk(cfg, true) == 0, ZO_E_SHAPE, "side K (%d) not a multiple of %d", gp.ks_tile,
             gemm_cfg_bk(cfg, true));
    ZO_CHECK(cfg != GEMM_CFG_BIG || (gp.N % 16 == 0 && gp.ldc % 4 == 0 && gp.ldh % 4 == 0), ZO_E_SHAPE,
             "projection N must be a multiple of 16");
    ZO_CHECK(gp.K % bk == 0, ZO_E_SHAPE, "K (%d) not a multiple of %d", gp.K, bk);
    ZO_CHECK(gp.kwa % bk == 0 && gp.kwb % bk == 0 && gp.kwas % bk == 0 && (!gp.kwa || gp.K <= 2 * gp.kwa) &&
                 (!gp.kwb || gp.K <= 2 * gp.kwb) && (!gp.kwas || gp.ks_tile <= 2 * gp.kwas),
             ZO_E_SHAPE, "operand wrap does not fit the K extent");
    int rc;
    if ((rc = check_i32((int64_t)gp.M * gp.lda, "A")) != ZO_OK) return rc;
    if ((rc = check_i32((int64_t)gp.N * gp.ldb, "B")) != ZO_OK) return rc;
    if ((rc = check_i32((int64_t)gp.M * gp.ldas, "As")) != ZO_OK) return rc;
    if ((rc = check_i32((int64_t)gp.N * gp.ldbs, "Bs")) != ZO_OK) return rc;
    ZO_HIP(gemm_launch_bf16(gp, cfg, s));
  } else {
    const int bn = gemm_cfg_bn(cfg, false);
    for (int i = 0; i < gp.n_bounds; ++i)
      ZO_CHECK(gp.bounds[i] % bn == 0, ZO_E_SHAPE, "kind boundary not a multiple of the tile");
    ZO_CHECK(gp.K % gemm_bk(false) == 0 && gp.ks_tile % gemm_bk(false) == 0, ZO_E_SHAPE,
             "K not a multiple of 16");
    ZO_HIP(gemm_launch_f32(gp, cfg, s));
  }
  return ZO_OK;
}

GemmParams gemm_base(const void* A, int64_t lda, const void* B, int64_t ldb, int M, int N, int K) {
  GemmParams g;
  memset(&g, 0, sizeof g);
  g.A = A; g.lda = lda; g.B = B; g.ldb = ldb; g.M = M; g.N = N; g.K = K;
  return g;
}

// Generation calls: every packed row's k and v also go to the cache (row w.row_cache[r]);
// decode steps (one row per physical sequence) attend over the cache instead of the packed
// rows, and the head also records each tile's first maximum column.
struct GenCtx {
  bool decode;
  int max_keys;       // decode: the longest sequence's key count this step
};

template <typename T>
int forward(zo_model* m, const zo_plan_s& p, const Packing& pk, const SideGeom& sg, const WsPtrs& w,
            const int32_t* tokens, hipStream_t s, const GenCtx* gen = nullptr) {
  const zo_model_desc& d = m->d;
  const bool bf = bf16_like(d);
  const bool f8 = is_fp8(d);
  const Layout& Lo = m->lo;
  auto W = [&](const TLoc& t) -> const void* { return t.present ? (const void*)(m->w + t.off) : nullptr; };
  auto Wf = [&](const TLoc& t) -> const float* { return (const float*)W(t); };
  const int M = (int)pk.M;
  const int D = d.d_model, F = d.d_ffn;
  const int NQ = d.n_heads * d.head_dim, NKV = d.n_kv_heads * d.head_dim;
  const int NQKV = NQ + 2 * NKV;
  const float eps = (float)d.norm_eps;
  const bool rms = !is_opt(d);
  const int big = GEMM_CFG_BIG, narrow = GEMM_CFG_NARROW;
  // Two-term activations (bf16 only), per site: a split projection input is [hi | lo] of
  // width 2K and the GEMM wraps B at K; with the attention site q|k|v stay fp32 for the
  // fp32 attention; the side-input projection of a split group reads A = [hi | lo] wrapped
  // at 2K against V^T = [hi | hi | lo] (K' = 3K), and its side segment reads
  // As = [t_hi | t_lo] per unit wrapped at 2 units against Bs = [U_hi | U_hi | U_lo].
  const bool sp = split_act(p);
  bool spg[4];
  for (int g = 0; g < 4; ++g) spg[g] = split_group(p, g);
  const bool sph = split_head(p);
  const int xn = (spg[0] || spg[2]) ? 2 : 1;        // pitch factor of the shared norm-output rows
  auto x3g = [&](int g) { return spg[g] ? 3 : 1; };
  // row pitch of the input buffer of group g (K its width)
  auto lda_of = [&](int g, int K) -> int64_t { return (int64_t)K * ((g == 0 || g == 2) ? xn : (spg[g] ? 2 : 1)); };
  int rc;

  if (M > 0) {
    ProfScope ps(ZO_PROF_NORM, s);
    if (bf)
      ZO_HIP(launch_embed_t<bf16_t>((const bf16_t*)W(Lo.g[G_TOK]), (const bf16_t*)W(Lo.g[G_POS]), tokens,
                                    w.row_src, w.row_pos, M, D, d.vocab, w.h, w.bad_ids, s));
    else
      ZO_HIP(launch_embed_t<float>((const float*)W(Lo.g[G_TOK]), (const float*)W(Lo.g[G_POS]), tokens, w.row_src,
                                   w.row_pos, M, D, d.vocab, w.h, w.bad_ids, s));
  }

  // the side input of a group formed inside the norm kernel that produces its activations
  // (bf16 and fp8 models, one-term activations, at most 16 used factor columns)
  auto side_in_norm = [&](int g) {
    return bf && !spg[g] && sg.group_on[g] && (sg.vt_rows[g] / sg.ks_c) * (int64_t)(sg.nc * sg.r) <= 16;
  };
  auto tproj_params = [&](int l, int g, const void* X, int K) {
    GemmParams gp = gemm_base(X, lda_of(g, K), w.vt[l * 4 + g], (int64_t)K * x3g(g), M, (int)sg.vt_rows[g],
                              K * x3g(g));
    gp.epi = EPI_TPROJ;
    gp.C = w.as; gp.ldc = w.as_ld;
    gp.row_cand = w.row_cand; gp.cand_dir = w.cand_dir; gp.cand_slot = w.cand_slot; gp.cand_scale = w.cand_scale;
    gp.tp_ks = sg.ks_c; gp.tp_rank = sg.r; gp.tp_entries = sg.E; gp.tp_used = sg.nc * sg.r; gp.tp_as_ks = sg.ks;
    return gp;
  };
  auto tproj = [&](int l, int g, const void* X, int K) -> int {
    if (!sg.group_on[g]) return ZO_OK;
    GemmParams gp = gemm_base(X, lda_of(g, K), w.vt[l * 4 + g], (int64_t)K * x3g(g), M, (int)sg.vt_rows[g],
                              K * x3g(g));
    if (spg[g]) { gp.kwa = 2 * K; gp.tp_unit = (int)sg.bs_cols[g]; }
    gp.epi = EPI_TPROJ;
    gp.C = w.as; gp.ldc = w.as_ld;
    gp.row_cand = w.row_cand; gp.cand_dir = w.cand_dir; gp.cand_slot = w.cand_slot; gp.cand_scale = w.cand_scale;
    gp.tp_ks = sg.ks_c; gp.tp_rank = sg.r; gp.tp_entries = sg.E; gp.tp_used = sg.nc * sg.r; gp.tp_as_ks = sg.ks;
    gp.ksplit = (gen && gen->decode && !sp) ? tproj_split_decode(d, sg.vt_rows[g], K)
                                            : tproj_split(d, sg.vt_rows[g], K * x3g(g));
    gp.partial = w.tp_partial;
    gp.a_e4m3 = f8;                        // fp8 models: every layer-linear input is e4m3
    return run_gemm(d, gp, narrow, s);
  };
  // projection over activations X [M x K] (or [hi | lo] when `split`; row pitch lda) with the
  // exact weight B [N x K] (fp8 models: e4m3 X and e4m3 codes of B * 2^11)
  auto proj = [&](const void* X, int64_t lda, bool split, const void* B, int N, int K) {
    GemmParams gp = gemm_base(X, lda, B, K, M, N, K * (split ? 2 : 1));
    if (split) gp.kwb = K;
    gp.a_e4m3 = gp.b_e4m3 = f8;
    if (w.sk_part && !f8) {
      gp.sk_part = w.sk_part; gp.sk_flag = w.sk_flag; gp.sk_err = w.bad_ids + 1; gp.sk_ncu = m->n_cu;
    }
    if (gen && gen->decode && !sp && bf) {
      // decode steps (one row per sequence): K-slices until the 128x128 tiles fill the
      // CUs, at least four K-steps (64 bf16 or 128 e4m3 deep) a slice
      const int64_t tiles = (int64_t)((M + 127) / 128) * ((N + 127) / 128);
      const int nks = K / (f8 ? 128 : 64);
      int ks = 1;
      while (ks < kMaxDecodeSplit && tiles * ks < 256 && nks % (2 * ks) == 0 && nks / (2 * ks) >= 4) ks *= 2;
      if (ks > 1) { gp.ksplit = ks; gp.partial = w.proj_partial; }
    }
    return gp;
  };
  // LayerNorm / RMSNorm of the residual stream into the input of the next linears (group g),
  // with the group's side input t when side_in_norm(g)
  auto norm_in = [&](const float* nw, const float* nb, int l, int g) -> hipError_t {
    if (side_in_norm(g)) {
      const GemmParams gp = tproj_params(l, g, w.xa, D);
      const int n_used = (int)(sg.vt_rows[g] / sg.ks_c) * sg.nc * sg.r;
      if (f8) return launch_norm_side<e4m3_t>(w.h, M, D, nw, nb, eps, rms, (e4m3_t*)w.xa, D, gp, n_used, s);
      if constexpr (std::is_same<T, bf16_t>::value)
        return launch_norm_side<bf16_t>(w.h, M, D, nw, nb, eps, rms, (bf16_t*)w.xa, (int64_t)D * xn, gp, n_used, s);
    }
    if (f8) return launch_norm<e4m3_t>(w.h, nullptr, M, D, nw, nb, eps, rms, (e4m3_t*)w.xa, D, 0, s);
    return launch_norm<T>(w.h, nullptr, M, D, nw, nb, eps, rms, (T*)w.xa, (int64_t)D * xn, spg[g] ? D : 0, s);
  };
  auto with_side = [&](GemmParams& gp, int l, int g) {
    if (!sg.group_on[g]) return;
    gp.As = w.as; gp.ldas = w.as_ld;
    gp.Bs = w.bs[l * 4 + g]; gp.ldbs = sg.bs_cols[g] * x3g(g);
    gp.ks_tile = (int)sg.bs_cols[g] * x3g(g);
    if (spg[g]) { gp.as_stride = 2 * (int)sg.bs_cols[g]; gp.kwas = 2 * (int)sg.bs_cols[g]; }
  };

  for (int l = 0; l < d.n_layers && M > 0; ++l) {
    const auto& P = Lo.L[l];
    // attention block
    {
      ProfScope ps(ZO_PROF_NORM, s);
      ZO_HIP(norm_in(Wf(P[P_LN1W]), Wf(P[P_LN1B]), l, 0));
    }
    if (!side_in_norm(0) && (rc = tproj(l, 0, w.xa, D)) != ZO_OK) return rc;
    {
      GemmParams gp = proj(w.xa, lda_of(0, D), spg[0], W(P[P_WQ]), NQKV, D);
      with_side(gp, l, 0);
      if (sg.group_on[0]) { gp.n_bounds = 2; gp.bounds[0] = NQ; gp.bounds[1] = NQ + NKV; }
      gp.epi = EPI_STORE; gp.bias = Wf(P[P_BQ]); gp.C = w.qkv; gp.ldc = NQKV; gp.c_f32 = spg[1];
      if ((rc = run_gemm(d, gp, big, s)) != ZO_OK) return rc;
    }
    if (!is_opt(d)) {
      ProfScope ps(ZO_PROF_NORM, s);
      if (spg[1])
        ZO_HIP(launch_qknorm_rope<float>((float*)w.qkv, M, NQKV, d.n_heads, d.n_kv_heads, d.head_dim, Wf(P[P_QNW]),
                                         Wf(P[P_KNW]), eps, m->rope, w.row_pos, s));
      else
        ZO_HIP(launch_qknorm_rope<T>((T*)w.qkv, M, NQKV, d.n_heads, d.n_kv_heads, d.head_dim, Wf(P[P_QNW]),
                                     Wf(P[P_KNW]), eps, m->rope, w.row_pos, s));
    }
    {
      ProfScope ps(gen && gen->decode ? ZO_PROF_DECODE_ATTN : ZO_PROF_ATTENTION, s);
      T* kc = gen ? (T*)w.kcache + (int64_t)l * w.kv_layer_elems : nullptr;
      T* vc = gen ? (T*)w.vcache + (int64_t)l * w.kv_layer_elems : nullptr;
      if (gen) ZO_HIP(launch_kv_append<T>((const T*)w.qkv, NQKV, M, w.row_cache, NQ, NKV, kc, vc, s));
      if (gen && gen->decode) {
        hipError_t e;
        if constexpr (std::is_same<T, bf16_t>::value) {
          if (f8)
            e = launch_decode_attention<T, e4m3_t>((const T*)w.qkv, NQKV, kc, vc, w.kv_first, w.row_pos, M,
                                                   d.n_heads, d.n_kv_heads, d.head_dim, (e4m3_t*)w.attn, NQ,
                                                   gen->max_keys, s);
          else
            e = launch_decode_attention<T, T>((const T*)w.qkv, NQKV, kc, vc, w.kv_first, w.row_pos, M, d.n_heads,
                                              d.n_kv_heads, d.head_dim, (T*)w.attn, NQ, gen->max_keys, s);
        } else {
          e = launch_decode_attention<T, T>((const T*)w.qkv, NQKV, kc, vc, w.kv_first, w.row_pos, M, d.n_heads,
                                            d.n_kv_heads, d.head_dim, (T*)w.attn, NQ, gen->max_keys, s);
        }
        ZO_HIP(e);
      }
      else if (spg[1])
        ZO_HIP(launch_attention_split((const float*)w.qkv, NQKV, (bf16_t*)w.attn, 2 * NQ, NQ, w.phys_cu, w.work,
                                      (int)pk.work.size(), d.n_heads, d.n_kv_heads, d.head_dim, s));
      else if (f8)
        ZO_HIP(launch_attention_e4m3((const bf16_t*)w.qkv, NQKV, (e4m3_t*)w.attn, NQ, w.phys_cu, w.work,
                                     (int)pk.work.size(), d.n_heads, d.n_kv_heads, d.head_dim, s));
      else
        ZO_HIP(launch_attention<T>((const T*)w.qkv, NQKV, (T*)w.attn, NQ, w.phys_cu, pk.n_phys, w.work,
                                   (int)pk.work.size(), d.n_heads, d.n_kv_heads, d.head_dim, s));
    }
    if ((rc = tproj(l, 1, w.attn, NQ)) != ZO_OK) return rc;
    {
      GemmParams gp = proj(w.attn, lda_of(1, NQ), spg[1], W(P[P_WO]), D, NQ);
      with_side(gp, l, 1);
      gp.epi = EPI_RESID; gp.bias = Wf(P[P_BO]); gp.H = w.h; gp.ldh = D;
      if ((rc = run_gemm(d, gp, big, s)) != ZO_OK) return rc;
    }
    // FFN block
    {
      ProfScope ps(ZO_PROF_NORM, s);
      ZO_HIP(norm_in(Wf(P[P_LN2W]), Wf(P[P_LN2B]), l, 2));
    }
    if (!side_in_norm(2) && (rc = tproj(l, 2, w.xa, D)) != ZO_OK) return rc;
    // the FFN output projection's side input: in the fc1 / gate-up epilogue (not in the
    // K-sliced decode-step projections)
    const bool ffn_fused = w.sf_part && !(gen && gen->decode);
    {
      const int N1 = is_opt(d) ? F : 2 * F;
      GemmParams gp = proj(w.xa, lda_of(2, D), spg[2], W(P[P_W1]), N1, D);
      with_side(gp, l, 2);
      gp.C = w.hid; gp.ldc = lda_of(3, F); gp.c_lo = spg[3] ? F : 0;
      if (is_opt(d)) { gp.epi = EPI_GELU; gp.bias = Wf(P[P_B1]); }
      else gp.epi = EPI_SWIGLU;
      if (ffn_fused) {
        gp.sf_n = sg.nc * sg.r; gp.sf_used = sg.nc * sg.r; gp.sf_ks = sg.ks_c;
        gp.sf_groups = (N1 + 127) / 128;                 // units of two 64-column wave tiles
        gp.sf_vt = w.vt[l * 4 + 3]; gp.sf_ldv = F;
        gp.sf_part = w.sf_part;
      }
      if ((rc = run_gemm(d, gp, big, s)) != ZO_OK) return rc;
      if (ffn_fused) {
        GemmParams rp = tproj_params(l, 3, w.hid, F);
        rp.sf_n = gp.sf_n; rp.sf_groups = gp.sf_groups; rp.sf_part = w.sf_part;
        ProfScope ps(ZO_PROF_GEMM_SIDE, s);
        ZO_HIP(launch_side_part_reduce(rp, s));
      }
    }
    if (!ffn_fused && (rc = tproj(l, 3, w.hid, F)) != ZO_OK) return rc;
    {
      const TLoc& w2 = is_opt(d) ? P[P_W2] : P[P_WDOWN];
      GemmParams gp = proj(w.hid, lda_of(3, F), spg[3], W(w2), D, F);
      with_side(gp, l, 3);
      gp.epi = EPI_RESID; gp.bias = is_opt(d) ? Wf(P[P_B2]) : nullptr; gp.H = w.h; gp.ldh = D;
      if ((rc = run_gemm(d, gp, big, s)) != ZO_OK) return rc;
    }
  }
  const int S = (int)pk.n_scored;
  if (S > 0) {
    {
      ProfScope ps(ZO_PROF_NORM, s);
      ZO_HIP(launch_norm<T>(w.h, w.sc_row, S, D, Wf(Lo.g[G_FNW]), Wf(Lo.g[G_FNB]), eps, rms, (T*)w.xs,
                            (int64_t)D * (sph ? 2 : 1), sph ? D : 0, s));
      ZO_HIP(launch_gather_labels(tokens, w.sc_lab_src, S, d.vocab, w.labels, w.bad_ids, s));
    }
    const TLoc& head = is_opt(d) ? Lo.g[G_TOK] : Lo.g[G_HEAD];
    GemmParams gp = gemm_base(w.xs, (int64_t)D * (sph ? 2 : 1), W(head), D, S, d.vocab, D * (sph ? 2 : 1));
    if (sph) gp.kwb = D;
    const int bn = gemm_cfg_bn(GEMM_CFG_HEAD, bf);
    gp.epi = EPI_LMHEAD; gp.labels = w.labels; gp.part = w.part; gp.lab_logit = w.lab_logit;
    gp.part_idx = gen ? w.part_idx : nullptr;
    gp.n_ntiles = (d.vocab + bn - 1) / bn;
    if ((rc = run_gemm(d, gp, GEMM_CFG_HEAD, s)) != ZO_OK) return rc;
  }
  return ZO_OK;
}

}  // namespace

// Runs `launch` (a fixed launch sequence whose arguments follow from `key`) on stream s: a
// new key eagerly once, captured into a graph when the next call repeats it, and replayed
// from the graph while the key repeats.
template <typename F>
static int launch_cached(GraphCache& gc, const std::vector<int64_t>& key, hipStream_t s, F&& launch) {
  if (gc.exec && gc.key == key) {
    ZO_HIP(hipGraphLaunch(gc.exec, s));
    return ZO_OK;
  }
  if (gc.pending != key) {
    const int rc = launch();
    if (rc == ZO_OK) gc.pending = key;
    return rc;
  }
  gc.reset();
  ZO_HIP(hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal));
  const int rc = launch();
  hipGraph_t g = nullptr;
  const hipError_t e = hipStreamEndCapture(s, &g);      // always leave capture mode
  if (rc != ZO_OK) {
    if (g) (void)hipGraphDestroy(g);
    return rc;
  }
  if (e != hipSuccess) return fail(ZO_E_DEVICE, "graph capture: %s", hipGetErrorString(e));
  gc.graph = g;
  if (hipGraphInstantiate(&gc.exec, g, nullptr, nullptr, 0) != hipSuccess) {
    gc.reset();
    return fail(ZO_E_DEVICE, "graph instantiation failed");
  }
  gc.key = key;
  ZO_HIP(hipGraphLaunch(gc.exec, s));
  return ZO_OK;
}

// Everything the kernel arguments of forward() are derived from, besides the model: the
// workspace (whose carve follows from the sizes below), the token buffer, the packing's
// sizes and the side geometry.  The packing tables and side factors themselves live in the
// workspace and are rewritten before every launch, so they are not part of the key.
static std::vector<int64_t> graph_key(const zo_plan_s& p, const Packing& pk, const SideGeom& sg, const void* ws,
                                      size_t ws_bytes, const void* tokens) {
  std::vector<int64_t> k = {(int64_t)(intptr_t)ws, (int64_t)ws_bytes, (int64_t)(intptr_t)tokens, pk.M, pk.n_phys,
                            pk.n_scored, (int64_t)pk.work.size(), (int64_t)p.cdir.size(), (int64_t)p.flags,
                            (int64_t)p.mask, sg.any, sg.E, sg.q, sg.r, sg.used, sg.ks, sg.nc, sg.ks_c};
  for (int g = 0; g < (int)sg.group_on.size(); ++g) k.push_back(sg.group_on[g]);
  return k;
}

// =====================================================================================
extern "C" {

int zo_abi_version(void) { return ZO_ABI_VERSION; }
const char* zo_last_error(void) { return g_err.c_str(); }

int zo_weights_size(const zo_model_desc* desc, size_t* bytes) {
  int rc = validate_desc(desc);
  if (rc) return rc;
  ZO_CHECK(bytes, ZO_E_INVAL, "null output");
  *bytes = make_layout(*desc).bytes;
  return ZO_OK;
}

int zo_weight_locate(const zo_model_desc* desc, int32_t slot, int32_t param, size_t* offset, int64_t* rows,
                     int64_t* cols, int32_t* dtype, int32_t* layout) {
  int rc = validate_desc(desc);
  if (rc) return rc;
  ZO_CHECK(offset && rows && cols && dtype && layout, ZO_E_INVAL, "null output");
  Layout Lo = make_layout(*desc);
  const TLoc* t = nullptr;
  if (slot == 0) {
    ZO_CHECK(param >= 0 && param < N_GLOBAL, ZO_E_INVAL, "bad global param %d", param);
    t = &Lo.g[param];
  } else {
    ZO_CHECK(slot >= 1 && slot <= desc->n_layers, ZO_E_INVAL, "bad slot %d", slot);
    ZO_CHECK(param >= 0 && param < N_LAYER_PARAMS, ZO_E_INVAL, "bad layer param %d", param);
    t = &Lo.L[slot - 1][param];
  }
  ZO_CHECK(t->present, ZO_E_INVAL, "param %d absent for this architecture", param);
  *offset = t->off; *rows = t->rows; *cols = t->cols; *dtype = t->dtype; *layout = t->layout;
  return ZO_OK;
}

int zo_model_create(const zo_model_desc* desc, void* weights_dev, size_t bytes, zo_model** out) {
  int rc = validate_desc(desc);
  if (rc) return rc;
  ZO_CHECK(weights_dev && out, ZO_E_INVAL, "null argument");
  Layout Lo = make_layout(*desc);
  ZO_CHECK(bytes >= Lo.bytes, ZO_E_SHAPE, "weight blob has %zu bytes, needs %zu", bytes, Lo.bytes);
  zo_model* m = new (std::nothrow) zo_model();
  ZO_CHECK(m, ZO_E_NOMEM, "out of host memory");
  m->d = *desc;
  m->lo = std::move(Lo);
  m->w = (unsigned char*)weights_dev;
  m->w_bytes = bytes;
  if (hipGetDevice(&m->device) != hipSuccess) m->device = 0;
  if (hipDeviceGetAttribute(&m->n_cu, hipDeviceAttributeMultiprocessorCount, m->device) != hipSuccess) m->n_cu = 0;
  (void)scratch_init(m->device);        // the device is current: record its scratch address
  if (!is_opt(*desc)) {
    // RoPE table: inv_freq_i = theta^(-2i/hd); angle = pos * inv_freq_i, in fp64, stored fp32
    const int half = desc->head_dim / 2;
    m->rope_len = desc->max_pos;
    std::vector<float2> tab((size_t)m->rope_len * half);
    std::vector<double> inv(half);
    for (int i = 0; i < half; ++i) inv[i] = std::pow(desc->rope_theta, -(2.0 * i) / desc->head_dim);
    for (int pos = 0; pos < m->rope_len; ++pos)
      for (int i = 0; i < half; ++i) {
        const double a = (double)pos * inv[i];
        tab[(size_t)pos * half + i] = make_float2((float)std::cos(a), (float)std::sin(a));
      }
    hipError_t e = hipMalloc((void**)&m->rope, tab.size() * sizeof(float2));
    if (e == hipSuccess) e = hipMemcpy(m->rope, tab.data(), tab.size() * sizeof(float2), hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      if (m->rope) (void)hipFree(m->rope);
      delete m;
      return fail(ZO_E_DEVICE, "RoPE table: %s", hipGetErrorString(e));
    }
  }
  *out = m;
  return ZO_OK;
}

int zo_model_destroy(zo_model* m) {
  if (!m) return ZO_OK;
  m->gc.reset();
  m->gcd.reset();
  if (m->rope) (void)hipFree(m->rope);
  delete m;
  return ZO_OK;
}

int zo_init_weights(zo_model* m, uint64_t seed, void* stream) {
  CallRange range_("zo_init_weights");
  ZO_CHECK(m, ZO_E_INVAL, "null model");
  hipStream_t s = (hipStream_t)stream;
  std::vector<NormalJob> jobs;
  int64_t max_blocks = 0;
  auto add = [&](const TLoc& t, int slot, int param) {
    if (!t.present) return;
    NormalJob j;
    memset(&j, 0, sizeof j);
    j.dst = m->w + t.off;
    j.rows = t.rows; j.cols = t.cols; j.ld = t.cols;
    j.seed = seed; j.tau = 0; j.tag = weight_tag(slot, param);
    j.mode = t.gain ? 1 : 0;
    j.dtype = t.dtype == ZO_DTYPE_FP8 ? 2 : t.dtype == ZO_DTYPE_BF16 ? 1 : 0;
    j.aux = t.layout;
    jobs.push_back(j);
    max_blocks = std::max<int64_t>(max_blocks, (t.rows * t.cols + 3) / 4);
  };
  for (int p = 0; p < N_GLOBAL; ++p) add(m->lo.g[p], 0, p);
  for (int l = 0; l < m->d.n_layers; ++l)
    for (int p = 0; p < N_LAYER_PARAMS; ++p) add(m->lo.L[l][p], l + 1, p);
  NormalJob* dj = nullptr;
  ZO_HIP(hipMalloc((void**)&dj, jobs.size() * sizeof(NormalJob)));
  hipError_t e = hipMemcpyAsync(dj, jobs.data(), jobs.size() * sizeof(NormalJob), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = launch_normal_jobs(dj, (int)jobs.size(), max_blocks, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  (void)hipFree(dj);
  if (e != hipSuccess) return fail(ZO_E_DEVICE, "weight init: %s", hipGetErrorString(e));
  return ZO_OK;
}

int zo_plan(const zo_model* m, const zo_plan_desc* desc, zo_plan_t** out) {
  CallRange range_("zo_plan");
  ZO_CHECK(m && desc && out, ZO_E_INVAL, "null argument");
  const zo_plan_desc& d = *desc;
  ZO_CHECK(d.nu >= 1, ZO_E_INVAL, "nu must be >= 1");
  ZO_CHECK(d.rank >= 1, ZO_E_INVAL, "rank must be >= 1");
  ZO_CHECK((d.flags & ~(ZO_PLAN_SCALE_INV_SQRT_R | ZO_PLAN_ALLOW_ZERO_EPS | ZO_PLAN_ACT_SPLIT |
                        ZO_PLAN_SPLIT_SITES)) == 0,
           ZO_E_INVAL, "unknown plan flag");
  ZO_CHECK(!(d.flags & (ZO_PLAN_ACT_SPLIT | ZO_PLAN_SPLIT_SITES)) || m->d.dtype == ZO_DTYPE_BF16, ZO_E_INVAL,
           "ZO_PLAN_ACT_SPLIT and ZO_PLAN_SPLIT_* apply to bf16 models only");
  ZO_CHECK(std::isfinite(d.eps) && (d.eps > 0 || (d.eps == 0 && (d.flags & ZO_PLAN_ALLOW_ZERO_EPS))), ZO_E_INVAL,
           "eps must be finite and > 0");
  ZO_CHECK(d.n_dirs >= 1 && d.dir_seeds, ZO_E_INVAL, "need at least one direction");
  ZO_CHECK(d.n_cand >= 1 && d.cand_dir && d.cand_sign, ZO_E_INVAL, "need at least one candidate");
  for (int i = 0; i < d.n_dirs; ++i)
    for (int j = 0; j < i; ++j)
      ZO_CHECK(d.dir_seeds[i] != d.dir_seeds[j], ZO_E_INVAL, "direction seeds must be distinct");
  for (int i = 0; i < d.n_cand; ++i) {
    ZO_CHECK(d.cand_dir[i] >= 0 && d.cand_dir[i] < d.n_dirs, ZO_E_INVAL, "candidate %d: direction out of range",
             i);
    ZO_CHECK(d.cand_sign[i] == 1 || d.cand_sign[i] == -1, ZO_E_INVAL, "candidate %d: sign must be +1 or -1", i);
  }
  ZO_CHECK((d.target_mask >> n_kinds_of(m->d)) == 0, ZO_E_INVAL, "target mask names a kind this arch lacks");
  zo_plan_s* p = new (std::nothrow) zo_plan_s();
  ZO_CHECK(p, ZO_E_NOMEM, "out of host memory");
  p->md = m->d;
  p->t = d.step; p->nu = d.nu; p->rank = d.rank; p->eps = d.eps;
  p->eps_tilde = (d.flags & ZO_PLAN_SCALE_INV_SQRT_R) ? d.eps / std::sqrt((double)d.rank) : d.eps;
  p->seeds.assign(d.dir_seeds, d.dir_seeds + d.n_dirs);
  p->cdir.assign(d.cand_dir, d.cand_dir + d.n_cand);
  p->csign.assign(d.cand_sign, d.cand_sign + d.n_cand);
  p->mask = d.target_mask;
  p->flags = d.flags;
  *out = p;
  return ZO_OK;
}

int zo_plan_destroy(zo_plan_t* p) {
  delete p;
  return ZO_OK;
}

int zo_bank_size(const zo_model* m, int32_t n_slots, int32_t rank, uint32_t target_mask, size_t* bytes) {
  ZO_CHECK(m && bytes, ZO_E_INVAL, "null argument");
  ZO_CHECK(n_slots >= 1 && rank >= 1, ZO_E_INVAL, "n_slots and rank must be >= 1");
  ZO_CHECK((target_mask >> n_kinds_of(m->d)) == 0, ZO_E_INVAL, "bad target mask");
  std::vector<int> kinds;
  std::vector<int64_t> koff;
  int64_t ls;
  bank_geometry(m->d, rank, target_mask, kinds, koff, ls);
  *bytes = (size_t)n_slots * m->d.n_layers * ls * sizeof(float);
  return ZO_OK;
}

int zo_bank_create(const zo_model* m, int32_t n_slots, int32_t rank, uint32_t target_mask, void* u_dev,
                   size_t bytes, zo_bank** out) {
  size_t need;
  int rc = zo_bank_size(m, n_slots, rank, target_mask, &need);
  if (rc) return rc;
  ZO_CHECK(out && (u_dev || need == 0), ZO_E_INVAL, "null argument");
  ZO_CHECK(bytes >= need, ZO_E_SHAPE, "bank memory has %zu bytes, needs %zu", bytes, need);
  zo_bank* b = new (std::nothrow) zo_bank();
  ZO_CHECK(b, ZO_E_NOMEM, "out of host memory");
  b->md = m->d; b->n_slots = n_slots; b->rank = rank; b->mask = target_mask;
  b->u = (float*)u_dev; b->bytes = bytes;
  b->seeds.assign(n_slots, 0);
  b->windows.assign(n_slots, -1);
  bank_geometry(m->d, rank, target_mask, b->kinds, b->kind_off, b->layer_stride);
  b->slot_stride = b->layer_stride * m->d.n_layers;
  *out = b;
  return ZO_OK;
}

int zo_bank_destroy(zo_bank* b) {
  delete b;
  return ZO_OK;
}

int zo_bank_keys(const zo_bank* b, uint64_t* seeds, int64_t* windows) {
  ZO_CHECK(b && seeds && windows, ZO_E_INVAL, "null argument");
  std::copy(b->seeds.begin(), b->seeds.end(), seeds);
  std::copy(b->windows.begin(), b->windows.end(), windows);
  return ZO_OK;
}

int zo_bank_set_keys(zo_bank* b, const uint64_t* seeds, const int64_t* windows) {
  ZO_CHECK(b && seeds && windows, ZO_E_INVAL, "null argument");
  for (int i = 0; i < b->n_slots; ++i) ZO_CHECK(windows[i] >= -1, ZO_E_INVAL, "bad window");
  b->seeds.assign(seeds, seeds + b->n_slots);
  b->windows.assign(windows, windows + b->n_slots);
  return ZO_OK;
}

int zo_bank_entry_offset(const zo_bank* b, int32_t slot, int32_t layer, int32_t kind, size_t* offset) {
  ZO_CHECK(b && offset, ZO_E_INVAL, "null argument");
  ZO_CHECK(slot >= 0 && slot < b->n_slots && layer >= 0 && layer < b->md.n_layers, ZO_E_INVAL, "out of range");
  for (size_t i = 0; i < b->kinds.size(); ++i)
    if (b->kinds[i] == kind) {
      *offset = ((size_t)slot * b->slot_stride + (size_t)layer * b->layer_stride + b->kind_off[i]) * sizeof(float);
      return ZO_OK;
    }
  return fail(ZO_E_INVAL, "kind %d is not a target of this bank", kind);
}

int zo_batch_layout(const zo_model* m, const zo_plan_t* p, const zo_bank* bank, const zo_batch* b, int32_t* n_phys,
                    int64_t* n_rows, int64_t* n_scored, size_t* ws_bytes) {
  ZO_CHECK(m && p, ZO_E_INVAL, "null argument");
  int rc = validate_batch(m->d, b);
  if (rc) return rc;
  Packing pk;
  build_packing(*p, *b, pk);
  SideGeom sg;
  if ((rc = side_geometry(m, *p, bank, sg)) != ZO_OK) return rc;
  WsPtrs w;
  carve(m, *p, pk, sg, nullptr, w);
  if (n_phys) *n_phys = pk.n_phys;
  if (n_rows) *n_rows = pk.M;
  if (n_scored) *n_scored = pk.n_scored;
  if (ws_bytes) *ws_bytes = w.bytes;
  return ZO_OK;
}

int zo_pack(const zo_plan_t* p, const zo_batch* b, int32_t* phys_seq, int32_t* phys_cand,
            int32_t* phys_first_scored) {
  ZO_CHECK(p && phys_seq && phys_cand && phys_first_scored, ZO_E_INVAL, "null argument");
  int rc = validate_batch(p->md, b);
  if (rc) return rc;
  Packing pk;
  build_packing(*p, *b, pk);
  std::copy(pk.phys_seq.begin(), pk.phys_seq.end(), phys_seq);
  std::copy(pk.phys_cand.begin(), pk.phys_cand.end(), phys_cand);
  std::copy(pk.phys_first.begin(), pk.phys_first.end(), phys_first_scored);
  return ZO_OK;
}

// Set-up shared by scoring and generation calls: packing, side geometry, workspace
// carve, host tables to the device and the side factors.  gen_new > 0: a generation call
// (scored rows = the last row of every physical sequence, KV caches in the workspace).
static int64_t gen_kv_rows(const Packing& pk, int gen_new) {
  int64_t n = 0;
  for (int q = 0; q < pk.n_phys; ++q) n += (pk.phys_cu[q + 1] - pk.phys_cu[q]) + gen_new - 1;
  return n;
}

static void gen_scored_rows(Packing& pk) {
  pk.sc_row.clear();
  pk.sc_lab_src.clear();
  pk.phys_first.assign(1, 0);
  for (int q = 0; q < pk.n_phys; ++q) {
    pk.sc_row.push_back(pk.phys_cu[q + 1] - 1);
    pk.sc_lab_src.push_back(0);          // labels are not used; any valid index
    pk.phys_first.push_back(q + 1);
  }
  pk.n_scored = pk.n_phys;
}

// host copies that queued transfers read (kept by the caller until its stream synchronisation)
struct HostKeep {
  std::vector<int32_t> cdir, cslot;
  std::vector<float> cscale;
  std::vector<SideJob> jobs;
  std::deque<std::vector<int32_t>> steps;   // a deque: references stay valid as it grows
};

static int prepare_call(zo_model* m, const zo_plan_t* p, const zo_bank* bank, const zo_batch* b, void* ws_dev,
                        size_t ws_bytes, hipStream_t s, int gen_new, Packing& pk, SideGeom& sg, WsPtrs& w,
                        HostKeep& keep) {
  int rc = validate_batch(m->d, b);
  if (rc) return rc;
  const zo_model_desc& d = m->d;
  const bool bf = bf16_like(d);
  build_packing(*p, *b, pk);
  if (gen_new > 0) gen_scored_rows(pk);
  if ((rc = side_geometry(m, *p, bank, sg)) != ZO_OK) return rc;
  const int64_t kv_rows = gen_new > 0 ? gen_kv_rows(pk, gen_new) : 0;
  carve(m, *p, pk, sg, nullptr, w, kv_rows);
  ZO_CHECK(ws_dev && ws_bytes >= w.bytes, ZO_E_SHAPE, "workspace has %zu bytes, needs %zu", ws_bytes, w.bytes);
  carve(m, *p, pk, sg, ws_dev, w, kv_rows);
  const int nc = (int)p->cdir.size();

  // ---- host tables -> device
  std::vector<int32_t>& cdir = keep.cdir;
  cdir = p->cdir;
  std::vector<float>& cscale = keep.cscale;
  cscale.assign(nc, 0.f);
  for (int c = 0; c < nc; ++c) cscale[c] = (float)((double)p->csign[c] * p->eps_tilde);
  auto h2d = [&](void* dst, const void* src, size_t n) -> hipError_t {
    if (n == 0) return hipSuccess;
    return hipMemcpyAsync(dst, src, n, hipMemcpyHostToDevice, s);
  };
  ZO_HIP(h2d(w.row_src, pk.row_src.data(), pk.row_src.size() * 4));
  ZO_HIP(h2d(w.row_pos, pk.row_pos.data(), pk.row_pos.size() * 4));
  ZO_HIP(h2d(w.row_cand, pk.row_cand.data(), pk.row_cand.size() * 4));
  ZO_HIP(h2d(w.phys_cu, pk.phys_cu.data(), pk.phys_cu.size() * 4));
  ZO_HIP(h2d(w.phys_first, pk.phys_first.data(), pk.phys_first.size() * 4));
  ZO_HIP(h2d(w.sc_row, pk.sc_row.data(), pk.sc_row.size() * 4));
  ZO_HIP(h2d(w.sc_lab_src, pk.sc_lab_src.data(), pk.sc_lab_src.size() * 4));
  ZO_HIP(h2d(w.work, pk.work.data(), pk.work.size() * 4));
  ZO_HIP(hipMemsetAsync(w.bad_ids, 0, 2 * sizeof(int32_t), s));
  if (w.sk_flag) ZO_HIP(hipMemsetAsync(w.sk_flag, 0, 2 * ZO_SK_MAX_WG * sizeof(int32_t), s));
  std::vector<int32_t>& cslot = keep.cslot;
  cslot.assign(nc, -1);
  for (int c = 0; c < nc && !sg.dslot.empty(); ++c) cslot[c] = sg.dslot[cdir[c]];
  ZO_HIP(h2d(w.cand_dir, cdir.data(), cdir.size() * 4));
  ZO_HIP(h2d(w.cand_slot, cslot.data(), cslot.size() * 4));
  ZO_HIP(h2d(w.cand_scale, cscale.data(), cscale.size() * 4));

  // ---- side factors: V^T rows for the input projections, [U | G] columns for the GEMMs
  std::vector<SideJob>& jobs = keep.jobs;
  int64_t max_items = 0;
  if (sg.any && pk.M > 0) {
    const uint64_t win = p->window();
    const int dt = bf ? 1 : 0;
    const int64_t NQ = (int64_t)d.n_heads * d.head_dim, NKV = (int64_t)d.n_kv_heads * d.head_dim;
    ZO_HIP(hipMemsetAsync(w.side_begin, 0, w.side_bytes, s));   // padding rows/columns must be zero
    ZO_HIP(hipMemsetAsync(w.as, 0, (size_t)pk.M * w.as_ld * act_size(d), s));   // columns no row writes
    for (int l = 0; l < d.n_layers; ++l)
      for (int g = 0; g < 4; ++g) {
        if (!sg.group_on[g]) continue;
        const Group& G = sg.groups[g];
        const size_t asz = act_size(d);
        const bool sp = split_group(*p, g);            // factor blocks hi | hi | lo
        const int64_t x3 = sp ? 3 : 1;
        for (size_t kb = 0; kb < G.kinds.size(); ++kb) {
          const int kind = G.kinds[kb];
          if (!((p->mask >> kind) & 1u)) continue;
          const KindShape ksh = kind_shape(d, kind);
          // V^T: block kb of the group's V^T, computed slot j at rows kb*ks_c + j*r
          unsigned char* vt = (unsigned char*)w.vt[l * 4 + g];
          unsigned char* bs = (unsigned char*)w.bs[l * 4 + g];
          int64_t row_base = 0;
          int row_map = 0;
          int64_t col_base = 0;
          if (g == 0) row_base = kind == ZO_KIND_Q ? 0 : (kind == ZO_KIND_K ? NQ : NQ + NKV);
          if (G.interleaved) { row_map = kind == 4 ? 1 : 2; col_base = (int64_t)kb * sg.ks; }
          // V^T rows of the computed t slots: entries, then directions without an entry
          for (int j = 0; j < sg.nc; ++j) {
            const bool entry = j < sg.E;
            const uint64_t seed = entry ? bank->seeds[sg.entry_slots[j]] : p->seeds[sg.cdirs[j - sg.E]];
            const uint64_t vwin = entry ? (uint64_t)bank->windows[sg.entry_slots[j]] : win;
            SideJob v;
            memset(&v, 0, sizeof v);
            v.dst = vt + ((int64_t)kb * sg.ks_c + (int64_t)j * sg.r) * sg.n_in[g] * x3 * asz;
            v.ld = sg.n_in[g] * x3;
            v.split = sp ? sg.n_in[g] : 0;
            v.seed = seed; v.tau = vwin; v.tag = dir_tag(l, kind, 1);
            v.src = 0; v.n = ksh.n_in; v.r = sg.r; v.dtype = dt;
            jobs.push_back(v);
            max_items = std::max<int64_t>(max_items, (ksh.n_in * sg.r + 3) / 4);
          }
          // Bs columns: U of every entry, then G of every direction
          for (int j = 0; j < sg.E + sg.q; ++j) {
            const bool entry = j < sg.E;
            const uint64_t seed = entry ? bank->seeds[sg.entry_slots[j]] : p->seeds[j - sg.E];
            SideJob u;
            memset(&u, 0, sizeof u);
            u.dst = bs + row_base * sg.bs_cols[g] * x3 * asz;
            u.ld = sg.bs_cols[g] * x3;
            u.split = sp ? sg.bs_cols[g] : 0;
            u.col0 = (int32_t)(col_base + (int64_t)j * sg.r);
            u.row_map = row_map;
            u.n = ksh.n_out; u.r = sg.r;
            u.dtype = is_fp8(d) ? 2 : dt;     // fp8 models: in the 2^11 units of the e4m3 weights
            if (entry) {
              size_t off;
              if ((rc = zo_bank_entry_offset(bank, sg.entry_slots[j], l, kind, &off)) != ZO_OK) return rc;
              u.src = 2;
              u.u_src = (const float*)((const unsigned char*)bank->u + off);
              max_items = std::max<int64_t>(max_items, ksh.n_out * sg.r);
            } else {
              u.src = 1;
              u.seed = seed; u.tau = p->t; u.tag = dir_tag(l, kind, 0);
              max_items = std::max<int64_t>(max_items, (ksh.n_out * sg.r + 3) / 4);
            }
            jobs.push_back(u);
          }
        }
      }
    ZO_CHECK((int)jobs.size() <= std::max(n_side_jobs(d, *p, sg), 1), ZO_E_SHAPE, "side job table overflow");
    ZO_HIP(h2d(w.jobs, jobs.data(), jobs.size() * sizeof(SideJob)));
    ProfScope ps(ZO_PROF_SIDE_PREP, s);
    ZO_HIP(launch_side_jobs(w.jobs, (int)jobs.size(), max_items, s));
  }

  return ZO_OK;
}

int zo_model_set_graphs(zo_model* m, int32_t enable) {
  ZO_CHECK(m, ZO_E_INVAL, "null model");
  m->gc.reset();
  m->gcd.reset();
  m->gc.on = enable != 0;
  return ZO_OK;
}

int zo_score(zo_model* m, const zo_plan_t* p, const zo_bank* bank, const zo_batch* b, void* ws_dev,
             size_t ws_bytes, double* seq_logp_dev, float* tok_logp_dev, double* S_host, void* stream) {
  CallRange range_("zo_score");
  ZO_CHECK(m && p && S_host, ZO_E_INVAL, "null argument");
  hipStream_t s = (hipStream_t)stream;
  const zo_model_desc& d = m->d;
  const bool bf = bf16_like(d);
  Packing pk;
  SideGeom sg;
  WsPtrs w;
  HostKeep keep;
  int rc = prepare_call(m, p, bank, b, ws_dev, ws_bytes, s, 0, pk, sg, w, keep);
  if (rc != ZO_OK) return rc;
  const int nc = (int)p->cdir.size();

  // ---- forward and head: eagerly, or replayed from the captured graph while everything its
  // launches were derived from repeats (graph_key); the tables it reads were copied above
  // (a new key runs eagerly once, which also does any first-use set-up of the kernels)
  if (m->gc.on && s != nullptr && !g_prof.on) {
    rc = launch_cached(m->gc, graph_key(*p, pk, sg, ws_dev, ws_bytes, b->tokens_dev), s, [&]() {
      return bf ? forward<bf16_t>(m, *p, pk, sg, w, b->tokens_dev, s) : forward<float>(m, *p, pk, sg, w, b->tokens_dev, s);
    });
    if (rc != ZO_OK) return rc;
  } else {
    if (bf) rc = forward<bf16_t>(m, *p, pk, sg, w, b->tokens_dev, s);   // bf16 and fp8 models
    else rc = forward<float>(m, *p, pk, sg, w, b->tokens_dev, s);
    if (rc != ZO_OK) return rc;
  }
  double* seq_out = seq_logp_dev ? seq_logp_dev : w.seq_logp;
  const int bn = gemm_cfg_bn(GEMM_CFG_HEAD, bf);
  ProfScope ps_red(ZO_PROF_REDUCE, s);
  ZO_HIP(launch_logp_reduce(w.part, (d.vocab + bn - 1) / bn, w.lab_logit, (int)pk.n_scored, w.phys_first,
                            pk.n_phys, w.tok64, tok_logp_dev, seq_out, s));
  prof_stop(ps_red.rec, s);
  ps_red.rec = -1;
  std::vector<double> seq(pk.n_phys);
  int32_t bad[2] = {0, 0};
  if (pk.n_phys > 0)
    ZO_HIP(hipMemcpyAsync(seq.data(), seq_out, pk.n_phys * sizeof(double), hipMemcpyDeviceToHost, s));
  ZO_HIP(hipMemcpyAsync(bad, w.bad_ids, sizeof bad, hipMemcpyDeviceToHost, s));
  ZO_HIP(hipStreamSynchronize(s));
  ZO_CHECK(!bad[0], ZO_E_INVAL, "a token id of the batch lies outside [0, vocab)");
  if (bad[1]) {
    m->n_cu = 0;        // split-tail projections off for this model from now on
    m->gc.reset();
    m->gcd.reset();
    return fail(ZO_E_DEVICE, "a split-tail projection %s; turned off for this model, call again",
                bad[1] == 2 ? "found a handover between XCDs" : "gave up waiting for a partial tile");
  }
  for (int c = 0; c < nc; ++c) S_host[c] = 0.0;
  for (int q = 0; q < pk.n_phys; ++q)
    if (pk.phys_cand[q] >= 0) S_host[pk.phys_cand[q]] += seq[q];
  return ZO_OK;
}

int zo_score_noalloc(zo_model* m, const zo_plan_t* p, const zo_bank* bank, const zo_batch* b,
                     double* seq_logp_dev, float* tok_logp_dev, double* S_host, void* stream) {
  CallRange range_("zo_score_noalloc");
  ZO_CHECK(m && p && S_host, ZO_E_INVAL, "null argument");
  size_t need = 0;
  int rc = zo_batch_layout(m, p, bank, b, nullptr, nullptr, nullptr, &need);
  if (rc != ZO_OK) return rc;
  ZO_CHECK(need <= (size_t)ZO_NOALLOC_SCRATCH_BYTES, ZO_E_SHAPE,
           "batch needs %zu bytes of workspace; the no-allocation scratch holds %zu", need,
           (size_t)ZO_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (m->device >= 0 && m->device < kMaxDevices) ws = g_scratch_ptr[m->device];
  }
  ZO_CHECK(ws, ZO_E_DEVICE, "no scratch address for device %d (hipGetSymbolAddress failed at model creation)",
           m->device);
  return zo_score(m, p, bank, b, ws, (size_t)ZO_NOALLOC_SCRATCH_BYTES, seq_logp_dev, tok_logp_dev, S_host, stream);
}

static int check_generate(const zo_model* m, const zo_plan_t* p, const zo_batch* b, int32_t n_new) {
  const zo_model_desc& d = m->d;
  ZO_CHECK(!split_act(*p), ZO_E_INVAL, "generation: not with ZO_PLAN_ACT_SPLIT or ZO_PLAN_SPLIT_*");
  ZO_CHECK(n_new >= 1, ZO_E_INVAL, "n_new must be >= 1");
  int rc = validate_batch(d, b);
  if (rc) return rc;
  for (int i = 0; i < b->n_seq; ++i) {
    const int len = b->cu_seqlens[i + 1] - b->cu_seqlens[i];
    ZO_CHECK((int64_t)len + n_new - 1 <= d.max_pos, ZO_E_SHAPE,
             "sequence %d: %d prompt + %d generated tokens exceed max_pos %d", i, len, n_new, d.max_pos);
  }
  return ZO_OK;
}

int zo_generate_layout(const zo_model* m, const zo_plan_t* p, const zo_bank* bank, const zo_batch* b,
                       int32_t n_new, int32_t* n_phys, size_t* ws_bytes) {
  ZO_CHECK(m && p, ZO_E_INVAL, "null argument");
  int rc = check_generate(m, p, b, n_new);
  if (rc) return rc;
  Packing pk;
  build_packing(*p, *b, pk);
  gen_scored_rows(pk);
  SideGeom sg;
  if ((rc = side_geometry(m, *p, bank, sg)) != ZO_OK) return rc;
  WsPtrs w;
  carve(m, *p, pk, sg, nullptr, w, gen_kv_rows(pk, n_new));
  if (n_phys) *n_phys = pk.n_phys;
  if (ws_bytes) *ws_bytes = w.bytes;
  return ZO_OK;
}

int zo_generate(zo_model* m, const zo_plan_t* p, const zo_bank* bank, const zo_batch* b, int32_t n_new,
                void* ws_dev, size_t ws_bytes, int32_t* tokens_dev, float* logp_dev, double* S_host, void* stream) {
  CallRange range_("zo_generate");
  ZO_CHECK(m && p && tokens_dev && logp_dev && S_host, ZO_E_INVAL, "null argument");
  int rc = check_generate(m, p, b, n_new);
  if (rc) return rc;
  hipStream_t s = (hipStream_t)stream;
  const zo_model_desc& d = m->d;
  const bool bf = bf16_like(d);
  Packing pk;
  SideGeom sg;
  WsPtrs w;
  HostKeep keep;
  if ((rc = prepare_call(m, p, bank, b, ws_dev, ws_bytes, s, n_new, pk, sg, w, keep)) != ZO_OK) return rc;
  const int nc = (int)p->cdir.size(), nq = pk.n_phys;
  if (nq == 0) {
    for (int c = 0; c < nc; ++c) S_host[c] = 0.0;
    return ZO_OK;
  }
  auto h2d = [&](void* dst, const std::vector<int32_t>& v) -> hipError_t {
    return v.empty() ? hipSuccess : hipMemcpyAsync(dst, v.data(), v.size() * 4, hipMemcpyHostToDevice, s);
  };
  // cache rows: sequence q owns len_q + n_new - 1 rows (the last generated token is never fed back)
  keep.steps.emplace_back(nq + 1, 0);
  std::vector<int32_t>& kv_first = keep.steps.back();
  for (int q = 0; q < nq; ++q) kv_first[q + 1] = kv_first[q] + (pk.phys_cu[q + 1] - pk.phys_cu[q]) + n_new - 1;
  keep.steps.emplace_back(pk.M, 0);
  std::vector<int32_t>& row_cache = keep.steps.back();
  for (int q = 0; q < nq; ++q)
    for (int r = pk.phys_cu[q]; r < pk.phys_cu[q + 1]; ++r) row_cache[r] = kv_first[q] + (r - pk.phys_cu[q]);
  ZO_HIP(h2d(w.kv_first, kv_first));
  ZO_HIP(h2d(w.row_cache, row_cache));
  const int bn = gemm_cfg_bn(GEMM_CFG_HEAD, bf);
  const int n_tiles = (d.vocab + bn - 1) / bn;
  // prefill: the prompts (the first token comes from each prompt's last row)
  const GenCtx prefill{false, 0};
  GenCtx decode{true, 0};
  rc = bf ? forward<bf16_t>(m, *p, pk, sg, w, b->tokens_dev, s, &prefill)
          : forward<float>(m, *p, pk, sg, w, b->tokens_dev, s, &prefill);
  if (rc != ZO_OK) return rc;
  ZO_HIP(launch_greedy_reduce(w.part, w.part_idx, n_tiles, nq, w.gen_tok, tokens_dev, logp_dev, n_new, 0, s));
  // decode steps: one row per physical sequence, token j - 1 at position len + j - 1
  Packing pd;
  pd.n_phys = nq;
  pd.M = nq;
  pd.n_scored = nq;
  pd.phys_cand = pk.phys_cand;
  pd.phys_seq = pk.phys_seq;
  for (int j = 1; j < n_new; ++j) {
    keep.steps.emplace_back(nq);
    std::vector<int32_t>& ident = keep.steps.back();
    keep.steps.emplace_back(nq);
    std::vector<int32_t>& pos = keep.steps.back();
    keep.steps.emplace_back(nq);
    std::vector<int32_t>& cache = keep.steps.back();
    keep.steps.emplace_back(nq, 0);
    std::vector<int32_t>& zeros = keep.steps.back();
    decode.max_keys = 0;
    for (int q = 0; q < nq; ++q) {
      ident[q] = q;
      pos[q] = (pk.phys_cu[q + 1] - pk.phys_cu[q]) + j - 1;
      cache[q] = kv_first[q] + pos[q];
      decode.max_keys = std::max(decode.max_keys, pos[q] + 1);
    }
    ZO_HIP(h2d(w.row_src, ident));
    ZO_HIP(h2d(w.row_pos, pos));
    ZO_HIP(h2d(w.row_cand, pk.phys_cand));
    ZO_HIP(h2d(w.sc_row, ident));
    ZO_HIP(h2d(w.sc_lab_src, zeros));
    ZO_HIP(h2d(w.row_cache, cache));
    if (sg.any) ZO_HIP(hipMemsetAsync(w.as, 0, (size_t)nq * w.as_ld * act_size(d), s));   // rows change meaning
    auto step = [&]() {
      return bf ? forward<bf16_t>(m, *p, pd, sg, w, w.gen_tok, s, &decode)
                : forward<float>(m, *p, pd, sg, w, w.gen_tok, s, &decode);
    };
    if (m->gc.on && s != nullptr && !g_prof.on) {
      // every decode step launches the same sequence (the step's tables were copied above);
      // only the wide / narrow form of the decode attention follows the key count
      std::vector<int64_t> key = graph_key(*p, pd, sg, ws_dev, ws_bytes, w.gen_tok);
      key.push_back(decode.max_keys > 512);
      rc = launch_cached(m->gcd, key, s, step);
    } else {
      rc = step();
    }
    if (rc != ZO_OK) return rc;
    ZO_HIP(launch_greedy_reduce(w.part, w.part_idx, n_tiles, nq, w.gen_tok, tokens_dev, logp_dev, n_new, j, s));
  }
  std::vector<float> lp((size_t)nq * n_new);
  int32_t bad[2] = {0, 0};
  ZO_HIP(hipMemcpyAsync(lp.data(), logp_dev, lp.size() * sizeof(float), hipMemcpyDeviceToHost, s));
  ZO_HIP(hipMemcpyAsync(bad, w.bad_ids, sizeof bad, hipMemcpyDeviceToHost, s));
  ZO_HIP(hipStreamSynchronize(s));
  ZO_CHECK(!bad[0], ZO_E_INVAL, "a token id of the batch lies outside [0, vocab)");
  if (bad[1]) {
    m->n_cu = 0;        // split-tail projections off for this model from now on
    m->gc.reset();
    m->gcd.reset();
    return fail(ZO_E_DEVICE, "a split-tail projection %s; turned off for this model, call again",
                bad[1] == 2 ? "found a handover between XCDs" : "gave up waiting for a partial tile");
  }
  for (int c = 0; c < nc; ++c) S_host[c] = 0.0;
  for (int q = 0; q < nq; ++q)
    if (pk.phys_cand[q] >= 0)
      for (int j = 0; j < n_new; ++j) S_host[pk.phys_cand[q]] += (double)lp[(size_t)q * n_new + j];
  return ZO_OK;
}

int zo_estimate(const zo_plan_t* p, const double* S_host, const int64_t* n_scored, uint32_t flags,
                double* c_out) {
  CallRange range_("zo_estimate");
  ZO_CHECK(p && S_host && c_out, ZO_E_INVAL, "null argument");
  ZO_CHECK((flags & ~(ZO_EST_INV_RANK | ZO_EST_MEAN)) == 0, ZO_E_INVAL, "unknown estimate flag");
  ZO_CHECK(!(flags & ZO_EST_MEAN) || n_scored, ZO_E_INVAL, "ZO_EST_MEAN needs n_scored");
  const int nc = (int)p->cdir.size(), q = (int)p->seeds.size();
  for (int c = 0; c < nc; ++c)
    ZO_CHECK(std::isfinite(S_host[c]), ZO_E_NONFINITE, "score of candidate %d is not finite", c);
  std::vector<double> c(q);
  const double two_eps = 2.0 * p->eps;
  ZO_CHECK(two_eps > 0, ZO_E_STATE, "eps is zero: the estimate is undefined");
  for (int dd = 0; dd < q; ++dd) {
    int ip = -1, im = -1, np = 0, nm = 0;
    for (int i = 0; i < nc; ++i)
      if (p->cdir[i] == dd) {
        if (p->csign[i] > 0) { ip = i; ++np; } else { im = i; ++nm; }
      }
    ZO_CHECK(np == 1 && nm == 1, ZO_E_STATE, "direction %d needs exactly one + and one - candidate", dd);
    double Lp = -S_host[ip], Lm = -S_host[im];
    if (flags & ZO_EST_MEAN) {
      ZO_CHECK(n_scored[ip] > 0 && n_scored[im] > 0, ZO_E_INVAL, "n_scored must be > 0");
      Lp = Lp / (double)n_scored[ip];
      Lm = Lm / (double)n_scored[im];
    }
    double cd = (Lp - Lm) / two_eps;
    if (flags & ZO_EST_INV_RANK) cd = cd / (double)p->rank;
    c[dd] = cd;
  }
  std::copy(c.begin(), c.end(), c_out);
  return ZO_OK;
}

int zo_update(zo_model* m, const zo_plan_t* p, zo_bank* bank, const double* c_host, double lr, void* stream) {
  CallRange range_("zo_update");
  ZO_CHECK(m && p && bank && c_host, ZO_E_INVAL, "null argument");
  ZO_CHECK(std::isfinite(lr), ZO_E_INVAL, "lr must be finite");
  if (int rc = check_objects(m, p, bank)) return rc;
  ZO_CHECK(bank->rank == p->rank && bank->mask == p->mask, ZO_E_STATE, "bank rank/targets differ from the plan's");
  const int q = (int)p->seeds.size();
  for (int dd = 0; dd < q; ++dd) ZO_CHECK(std::isfinite(c_host[dd]), ZO_E_NONFINITE, "c[%d] is not finite", dd);
  hipStream_t s = (hipStream_t)stream;
  const int64_t win = (int64_t)p->window();
  // find or allocate each direction's entry (keys change only after every check passed)
  std::vector<int> slot(q, -1);
  std::vector<int> fresh(q, 0);
  std::vector<bool> taken(bank->n_slots, false);
  for (int dd = 0; dd < q; ++dd)
    for (int sl = 0; sl < bank->n_slots; ++sl)
      if (bank->windows[sl] == win && bank->seeds[sl] == p->seeds[dd]) { slot[dd] = sl; taken[sl] = true; }
  for (int dd = 0; dd < q; ++dd) {
    if (slot[dd] >= 0) continue;
    for (int sl = 0; sl < bank->n_slots; ++sl)
      if (bank->windows[sl] < 0 && !taken[sl]) { slot[dd] = sl; taken[sl] = true; fresh[dd] = 1; break; }
    ZO_CHECK(slot[dd] >= 0, ZO_E_NOMEM, "bank has no free slot for direction %d window %lld", dd, (long long)win);
  }
  UpdateArgs a;
  memset(&a, 0, sizeof a);
  a.u_base = bank->u;
  a.layer_stride = bank->layer_stride;
  a.n_kinds = (int)bank->kinds.size();
  int64_t max_n = 0;
  for (int i = 0; i < a.n_kinds; ++i) {
    a.kind_id[i] = bank->kinds[i];
    a.kind_off[i] = bank->kind_off[i];
    a.kind_n[i] = kind_shape(m->d, bank->kinds[i]).n_out * bank->rank;
    max_n = std::max(max_n, a.kind_n[i]);
  }
  a.t = p->t;
  // the step follows the probed direction z_d = sigma G_d V_d^T (sigma = 1, or 1/sqrt(r) with
  // ZO_PLAN_SCALE_INV_SQRT_R): theta <- theta - (lr / q) sum_d c_d z_d
  const double sigma = (p->flags & ZO_PLAN_SCALE_INV_SQRT_R) ? 1.0 / std::sqrt((double)p->rank) : 1.0;
  for (int d0 = 0; d0 < q; d0 += ZO_MAX_UPDATE_DIRS) {
    a.n_dirs = std::min(ZO_MAX_UPDATE_DIRS, q - d0);
    for (int i = 0; i < a.n_dirs; ++i) {
      const int dd = d0 + i;
      a.seed[i] = p->seeds[dd];
      a.slot_off[i] = (int64_t)slot[dd] * bank->slot_stride;
      a.coef[i] = ((lr / (double)q) * c_host[dd]) * sigma;
      a.fresh[i] = fresh[dd];
    }
    ProfScope ps(ZO_PROF_UPDATE, s);
    ZO_HIP(launch_update(a, m->d.n_layers, max_n, s));
  }
  for (int dd = 0; dd < q; ++dd) {
    bank->seeds[slot[dd]] = p->seeds[dd];
    bank->windows[slot[dd]] = win;
  }
  return ZO_OK;
}

int zo_bank_fold_size(const zo_model* m, const zo_bank* bank, size_t* bytes) {
  ZO_CHECK(m && bank && bytes, ZO_E_INVAL, "null argument");
  size_t n = 0;
  for (int kind : bank->kinds) n += (size_t)kind_shape(m->d, kind).n_in * bank->rank;
  *bytes = std::max<size_t>(n * m->d.n_layers * sizeof(float), 256);
  return ZO_OK;
}

int zo_bank_fold(zo_model* m, zo_bank* bank, int32_t slot, void* ws_dev, size_t ws_bytes, void* stream) {
  CallRange range_("zo_bank_fold");
  ZO_CHECK(m && bank, ZO_E_INVAL, "null argument");
  ZO_CHECK(slot >= 0 && slot < bank->n_slots, ZO_E_INVAL, "slot %d out of range", slot);
  ZO_CHECK(bank->windows[slot] >= 0, ZO_E_STATE, "slot %d holds no entry", slot);
  if (int rc = check_objects(m, nullptr, bank)) return rc;
  size_t need = 0;
  int rc = zo_bank_fold_size(m, bank, &need);
  if (rc) return rc;
  ZO_CHECK(ws_dev && ws_bytes >= need, ZO_E_SHAPE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
  hipStream_t s = (hipStream_t)stream;
  const zo_model_desc& d = m->d;
  const int r = bank->rank;
  float* v = (float*)ws_dev;
  // V of every (layer, kind), regenerated from the entry's key
  std::vector<float*> vptr;
  for (int l = 0; l < d.n_layers; ++l)
    for (int kind : bank->kinds) {
      const KindShape ks = kind_shape(d, kind);
      SideJob jb;
      memset(&jb, 0, sizeof jb);
      jb.dst = v; jb.seed = bank->seeds[slot]; jb.tau = (uint64_t)bank->windows[slot];
      jb.tag = dir_tag(l, kind, 1); jb.n = ks.n_in; jb.r = r;
      ZO_HIP(launch_stream_rowmajor(jb, s));
      vptr.push_back(v);
      v += ks.n_in * r;
    }
  const int pk[7] = {P_WQ, P_WK, P_WV, P_WO, P_W1, P_W2, P_WDOWN};
  size_t vi = 0;
  for (int l = 0; l < d.n_layers; ++l)
    for (size_t kk = 0; kk < bank->kinds.size(); ++kk) {
      const int kind = bank->kinds[kk];
      const KindShape ks = kind_shape(d, kind);
      const TLoc& t = m->lo.L[l][pk[kind]];
      ZO_CHECK(t.present && t.rows == ks.n_out && t.cols == ks.n_in, ZO_E_STATE, "weight of kind %d not found",
               kind);
      FoldArgs a;
      memset(&a, 0, sizeof a);
      a.w = m->w + t.off;
      a.ld = t.cols;
      a.n_out = ks.n_out; a.n_in = ks.n_in;
      a.layout = t.layout;
      a.dtype = t.dtype == ZO_DTYPE_BF16 ? 1 : t.dtype == ZO_DTYPE_FP8 ? 2 : 0;
      a.r = r;
      a.u = bank->u + (size_t)slot * bank->slot_stride + (size_t)l * bank->layer_stride + bank->kind_off[kk];
      a.v = vptr[vi++];
      ZO_HIP(launch_fold(a, s));
    }
  ZO_HIP(hipStreamSynchronize(s));
  bank->windows[slot] = -1;
  bank->seeds[slot] = 0;
  return ZO_OK;
}

int zo_bank_cap(zo_model* m, zo_bank* bank, const zo_plan_t* p, int32_t max_frozen, void* ws_dev, size_t ws_bytes,
                void* stream, int32_t* n_folded) {
  CallRange range_("zo_bank_cap");
  ZO_CHECK(m && bank && p, ZO_E_INVAL, "null argument");
  ZO_CHECK(max_frozen >= 0, ZO_E_INVAL, "max_frozen must be >= 0");
  if (int rc = check_objects(m, p, bank)) return rc;
  const int64_t win = (int64_t)p->window();
  // frozen entries (windows other than the plan's), oldest window first, then slot order
  std::vector<std::pair<int64_t, int>> frozen;
  for (int s = 0; s < bank->n_slots; ++s)
    if (bank->windows[s] >= 0 && bank->windows[s] != win) frozen.push_back({bank->windows[s], s});
  std::sort(frozen.begin(), frozen.end());
  int folded = 0;
  if ((int)frozen.size() > max_frozen) {
    size_t need = 0;
    int rc = zo_bank_fold_size(m, bank, &need);
    if (rc) return rc;
    ZO_CHECK(ws_dev && ws_bytes >= need, ZO_E_SHAPE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
    for (size_t i = 0; i + max_frozen < frozen.size(); ++i) {
      if ((rc = zo_bank_fold(m, bank, frozen[i].second, ws_dev, ws_bytes, stream)) != ZO_OK) return rc;
      ++folded;
    }
  }
  if (n_folded) *n_folded = folded;
  return ZO_OK;
}

int zo_profile_select(uint32_t class_mask) {
  g_prof.mask = class_mask;
  return ZO_OK;
}

int zo_profile_begin(void) {
  g_prof.on = true;
  g_prof.used = 0;
  g_prof.recs.clear();
  return ZO_OK;
}

int zo_profile_end(int32_t n_classes, int64_t* counts, double* total_ms) {
  ZO_CHECK(n_classes >= 0 && n_classes <= ZO_PROF_N_CLASSES && (n_classes == 0 || (counts && total_ms)),
           ZO_E_INVAL, "bad argument");
  g_prof.on = false;
  for (int c = 0; c < n_classes; ++c) { counts[c] = 0; total_ms[c] = 0.0; }
  for (const auto& r : g_prof.recs) {
    ZO_HIP(hipEventSynchronize(g_prof.pool[r.ev + 1]));
    float ms = 0.f;
    ZO_HIP(hipEventElapsedTime(&ms, g_prof.pool[r.ev], g_prof.pool[r.ev + 1]));
    if (r.cls < n_classes) { counts[r.cls] += 1; total_ms[r.cls] += ms; }
  }
  g_prof.recs.clear();
  g_prof.used = 0;
  return ZO_OK;
}

int zo_philox_words(uint64_t seed, uint32_t tag, uint64_t tau, int64_t first_block, int64_t n_blocks,
                    uint32_t* out_dev, void* stream) {
  ZO_CHECK(n_blocks >= 0 && first_block >= 0 && (out_dev || n_blocks == 0), ZO_E_INVAL, "bad argument");
  ZO_CHECK(first_block + n_blocks <= ((int64_t)1 << 32), ZO_E_INVAL, "block index beyond 2^32");
  ZO_HIP(launch_words_fill(seed, tag, tau, first_block, n_blocks, out_dev, (hipStream_t)stream));
  return ZO_OK;
}

int zo_normal_fill(uint64_t seed, uint32_t tag, uint64_t tau, int64_t first, int64_t n, double* out_dev,
                   void* stream) {
  ZO_CHECK(n >= 0 && first >= 0 && (out_dev || n == 0), ZO_E_INVAL, "bad argument");
  ZO_CHECK(first + n <= ((int64_t)1 << 34), ZO_E_INVAL, "element index beyond 2^34");
  ZO_HIP(launch_normal_fill_f64(seed, tag, tau, first, n, out_dev, (hipStream_t)stream));
  return ZO_OK;
}

int zo_direction(const zo_model* m, const zo_plan_t* p, int32_t dir, int32_t layer, int32_t kind, int32_t which,
                 float* out_dev, void* stream) {
  ZO_CHECK(m && p && out_dev, ZO_E_INVAL, "null argument");
  if (int rc = check_objects(m, p, nullptr)) return rc;
  ZO_CHECK(dir >= 0 && dir < (int)p->seeds.size(), ZO_E_INVAL, "direction out of range");
  ZO_CHECK(layer >= 0 && layer < m->d.n_layers, ZO_E_INVAL, "layer out of range");
  ZO_CHECK(kind >= 0 && kind < n_kinds_of(m->d), ZO_E_INVAL, "kind out of range");
  ZO_CHECK(which == 0 || which == 1, ZO_E_INVAL, "which must be 0 (G) or 1 (V)");
  const KindShape ks = kind_shape(m->d, kind);
  SideJob j;
  memset(&j, 0, sizeof j);
  j.dst = out_dev;
  j.seed = p->seeds[dir];
  j.tau = which == 0 ? p->t : p->window();
  j.tag = dir_tag(layer, kind, which);
  j.n = which == 0 ? ks.n_out : ks.n_in;
  j.r = p->rank;
  ZO_HIP(launch_stream_rowmajor(j, (hipStream_t)stream));
  return ZO_OK;
}

}  // extern "C"
