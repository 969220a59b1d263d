// Host side of the PHOTON C ABI: validation, weight-blob layout, workspace
// planning, and the launch sequences of prefill and one decode chunk.
//
// Method (PHOTON explainer, mokumoku.ipfde.com, Fujitsu PHOTON vertical
// scan): module table -- Context Chunker (concatenate C vectors, project),
// Context Encoder (causal Transformer on the coarse stream; the top one holds
// the only global K/V), Context Converter (1-D convolution, one vector -> C
// conditioning vectors), Context Decoder (causal Transformer with attention
// confined to the chunk); recursive-generation section -- HierGen re-encodes
// each generated chunk bottom-up, RecGen feeds the decoder's bottleneck
// reconstruction straight to the top encoder and drops the lower encoder
// caches after prefill.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/photon.h"
#include "kernels.h"

using namespace photon;

namespace {

thread_local std::string g_err;

photon_status fail(photon_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

photon_status ok() {
  return PHOTON_OK;
}

constexpr uint64_t kAlign = 256;
uint64_t align_up(uint64_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ------------------------------------------------------------ config checks
photon_status check_config(const photon_config* c) {
  if (!c) return fail(PHOTON_EINVAL, "config is NULL");
  if (c->n_levels != 2) return fail(PHOTON_EUNSUPPORTED, "n_levels must be 2 (got %d)", c->n_levels);
  if (c->chunk[0] < 1 || c->chunk[1] < 1) return fail(PHOTON_ESHAPE, "chunk sizes must be >= 1");
  if (c->chunk[0] > 16 || c->chunk[1] > 16)
    return fail(PHOTON_EUNSUPPORTED, "chunk sizes above 16 are not supported");
  if (c->d_model < 1 || c->n_heads < 1) return fail(PHOTON_ESHAPE, "d_model and n_heads must be >= 1");
  if (c->d_model % c->n_heads) return fail(PHOTON_ESHAPE, "d_model %% n_heads != 0");
  const int hd = c->d_model / c->n_heads;
  if (hd != 32 && hd != 64 && hd != 96 && hd != 128)
    return fail(PHOTON_EUNSUPPORTED, "head_dim %d not in {32, 64, 96, 128}", hd);
  if (c->d_model % 64) return fail(PHOTON_EUNSUPPORTED, "d_model must be a multiple of 64");
  if (c->mlp_mult < 1 || c->vocab < 1) return fail(PHOTON_ESHAPE, "mlp_mult and vocab must be >= 1");
  if (c->vocab % 16) return fail(PHOTON_EUNSUPPORTED, "vocab must be a multiple of 16");
  if (c->n_top < 1 || c->n_enc1 < 1 || c->n_dec1 < 1 || c->n_dec0 < 1)
    return fail(PHOTON_ESHAPE, "every stack needs at least one layer");
  if (c->dtype != PHOTON_F32 && c->dtype != PHOTON_BF16) return fail(PHOTON_EINVAL, "dtype must be F32 or BF16");
  if (!(c->norm_eps > 0.f) || !(c->rope_theta > 1.f)) return fail(PHOTON_EINVAL, "norm_eps/rope_theta out of range");
  return ok();
}

int elem_bytes(const photon_config* c) { return c->dtype == PHOTON_BF16 ? 2 : 4; }

// ------------------------------------------------------------ weight layout
struct TensorDesc {
  std::string name;
  int blob;
  int is_gain;
  int64_t rows, cols;
  uint64_t offset;
};

void add_stack(std::vector<TensorDesc>& v, const char* pre, int n, int blob, int64_t d, int64_t F) {
  for (int l = 0; l < n; ++l) {
    char p[32];
    snprintf(p, sizeof p, "%s.%d.", pre, l);
    const std::string s = p;
    v.push_back({s + "g1", blob, 1, d, 1, 0});
    v.push_back({s + "Wq", blob, 0, d, d, 0});
    v.push_back({s + "Wk", blob, 0, d, d, 0});
    v.push_back({s + "Wv", blob, 0, d, d, 0});
    v.push_back({s + "Wo", blob, 0, d, d, 0});
    v.push_back({s + "g2", blob, 1, d, 1, 0});
    v.push_back({s + "W1", blob, 0, F, d, 0});
    v.push_back({s + "W2", blob, 0, d, F, 0});
  }
  v.push_back({std::string(pre) + ".gf", blob, 1, d, 1, 0});
}

// Blob order follows the decode call order (decode blob) and prefill order.
std::vector<TensorDesc> layout(const photon_config* c, uint64_t* dec_bytes, uint64_t* pre_bytes) {
  const int64_t d = c->d_model, F = (int64_t)c->mlp_mult * d, V = c->vocab;
  const int64_t C1 = c->chunk[0], C2 = c->chunk[1];
  std::vector<TensorDesc> v;
  v.push_back({"E", 0, 0, V, d, 0});
  v.push_back({"W_ch2", 0, 0, d, C2 * d, 0});
  add_stack(v, "top", c->n_top, 0, d, F);
  v.push_back({"W_cv2", 0, 0, C2 * d, d, 0});
  add_stack(v, "dec1", c->n_dec1, 0, d, F);
  v.push_back({"W_cv1", 0, 0, C1 * d, d, 0});
  add_stack(v, "dec0", c->n_dec0, 0, d, F);
  v.push_back({"W_out", 0, 0, V, d, 0});
  v.push_back({"W_ch1", 1, 0, d, C1 * d, 0});
  add_stack(v, "enc1", c->n_enc1, 1, d, F);
  uint64_t off[2] = {0, 0};
  const int eb = elem_bytes(c);
  for (auto& t : v) {
    const uint64_t bytes = (uint64_t)t.rows * t.cols * (t.is_gain ? 4 : eb);
    t.offset = align_up(off[t.blob]);
    off[t.blob] = t.offset + bytes;
  }
  if (dec_bytes) *dec_bytes = align_up(off[0]);
  if (pre_bytes) *pre_bytes = align_up(off[1]);
  return v;
}

// ------------------------------------------------------------ workspace plan
struct Region {
  uint64_t off = 0, bytes = 0;
};

struct WsPlan {
  int64_t top_cap = 0, low_cap = 0, rope_pos = 0;
  int nsplit_top = 1, nsplit_low = 1;
  int head_tiles = 1;
  // persistent
  Region top_kv, low_kv, dec_kv, h, counter, rope, prev, tok;
  // decode scratch, set A (top branch) and set B (token branch)
  Region xA, aA, qkvA, qA, oA, hidA, partA, eA, AA;
  Region xB, aB, qkvB, qB, oB, hidB, c0, Ahat, zB, kv1tmp, amv, ami;
  uint64_t state_bytes = 0, scratch_bytes = 0, total = 0;
  uint64_t off_state = 0, off_scratch = 0;
};

struct Cursor {
  uint64_t pos = 0;
  Region take(uint64_t bytes) {
    Region r;
    r.off = align_up(pos);
    r.bytes = bytes;
    pos = r.off + bytes;
    return r;
  }
};

WsPlan plan_workspace(const photon_config* c, int64_t B, int64_t tokens, int mode) {
  WsPlan p;
  const int64_t d = c->d_model, H = c->n_heads, hd = d / H, F = (int64_t)c->mlp_mult * d, V = c->vocab;
  const int64_t C1 = c->chunk[0], C2 = c->chunk[1], S = C1 * C2;
  const uint64_t eb = elem_bytes(c);
  const bool hier = mode == PHOTON_HIERGEN;
  p.top_cap = cdiv(tokens, S);
  p.low_cap = hier ? cdiv(tokens, C1) : 0;
  p.rope_pos = std::max<int64_t>({p.top_cap, p.low_cap, C1, C2});
  p.nsplit_top = attn_decode_splits((int)B, (int)H, (int)p.top_cap);
  p.nsplit_low = hier ? attn_decode_splits((int)B, (int)H, (int)p.low_cap) : 1;
  p.head_tiles = gemm_argmax_tiles(c->dtype, (int)(B * C2), (int)V, (int)d);
  Cursor cur;
  p.top_kv = cur.take((uint64_t)c->n_top * 2 * B * H * p.top_cap * hd * eb);
  p.low_kv = cur.take((uint64_t)c->n_enc1 * 2 * B * H * p.low_cap * hd * eb);
  p.dec_kv = cur.take((uint64_t)c->n_dec0 * 2 * B * C2 * H * C1 * hd * eb);
  p.off_state = align_up(cur.pos);
  p.h = cur.take((uint64_t)B * d * eb);
  p.counter = cur.take(sizeof(int));
  p.rope = cur.take((uint64_t)p.rope_pos * (hd / 2) * 2 * sizeof(float));
  p.prev = cur.take((uint64_t)B * C2 * sizeof(int));
  p.tok = cur.take((uint64_t)B * S * sizeof(int));
  p.off_scratch = align_up(cur.pos);
  p.state_bytes = p.off_scratch - p.off_state;
  const int64_t MA = hier ? B * C2 : B, MB = B * C2;
  p.xA = cur.take((uint64_t)MA * d * 4);
  p.aA = cur.take((uint64_t)MA * d * eb);
  p.qkvA = cur.take((uint64_t)MA * 3 * d * 4);
  p.qA = cur.take((uint64_t)MA * d * 4);
  p.oA = cur.take((uint64_t)MA * d * eb);
  p.hidA = cur.take((uint64_t)MA * F * eb);
  const int64_t parts = std::max<int64_t>((int64_t)B * H * p.nsplit_top, hier ? (int64_t)B * H * C2 * p.nsplit_low : 0);
  p.partA = cur.take((uint64_t)parts * (hd + 2) * 4);
  p.eA = cur.take(hier ? (uint64_t)B * S * d * eb : 0);
  p.AA = cur.take(hier ? (uint64_t)B * C2 * d * eb : 0);
  p.xB = cur.take((uint64_t)MB * d * 4);
  p.aB = cur.take((uint64_t)MB * d * eb);
  p.qkvB = cur.take((uint64_t)MB * 3 * d * 4);
  p.qB = cur.take((uint64_t)MB * d * 4);
  p.oB = cur.take((uint64_t)MB * d * eb);
  p.hidB = cur.take((uint64_t)MB * F * eb);
  p.c0 = cur.take((uint64_t)MB * C1 * d * 4);
  p.Ahat = cur.take((uint64_t)MB * d * eb);
  p.zB = cur.take((uint64_t)MB * d * eb);
  p.kv1tmp = cur.take((uint64_t)2 * B * H * C2 * hd * eb);
  p.amv = cur.take((uint64_t)p.head_tiles * MB * 4);
  p.ami = cur.take((uint64_t)p.head_tiles * MB * 4);
  p.total = align_up(cur.pos);
  p.scratch_bytes = p.total - p.off_scratch;
  return p;
}

// prefill scratch: one batch slice of bs sequences at a time
constexpr int64_t kPrefillRows = 65536;

struct PrePlan {
  int64_t bs = 1, n1 = 0, n = 0;
  Region e, x, a, qkv, q, o, hid, A1, kv1, rope1;
  uint64_t total = 0;
};

PrePlan plan_prefill(const photon_config* c, int64_t B, int64_t P, int mode) {
  PrePlan p;
  const int64_t d = c->d_model, H = c->n_heads, hd = d / H, F = (int64_t)c->mlp_mult * d;
  const int64_t C1 = c->chunk[0], S = C1 * c->chunk[1];
  const uint64_t eb = elem_bytes(c);
  p.n1 = P / C1;
  p.n = P / S;
  p.bs = std::max<int64_t>(1, std::min<int64_t>(B, kPrefillRows / std::max<int64_t>(1, p.n1)));
  const int64_t R = p.bs * p.n1;
  Cursor cur;
  p.e = cur.take((uint64_t)p.bs * P * d * eb);
  p.x = cur.take((uint64_t)R * d * 4);
  p.a = cur.take((uint64_t)R * d * eb);
  p.qkv = cur.take((uint64_t)R * 3 * d * 4);
  p.q = cur.take((uint64_t)R * d * 4);
  p.o = cur.take((uint64_t)R * d * eb);
  p.hid = cur.take((uint64_t)R * F * eb);
  p.A1 = cur.take((uint64_t)R * d * eb);
  p.kv1 = cur.take(mode == PHOTON_HIERGEN ? 0 : (uint64_t)2 * p.bs * H * p.n1 * hd * eb);
  p.rope1 = cur.take((uint64_t)std::max<int64_t>(p.n1, 1) * (hd / 2) * 2 * 4);
  p.total = align_up(cur.pos);
  return p;
}

// ------------------------------------------------------------ context
struct LayerW {
  const float* g1;
  const void* Wqkv;
  const void* Wo;
  const float* g2;
  const void* W1;
  const void* W2;
};
struct StackW {
  std::vector<LayerW> layers;
  const float* gf = nullptr;
};

struct TraceRec {
  int cls;
  hipEvent_t a, b;
  double bytes, flops;
};

struct Tracer {
  uint32_t mask = 0;
  std::vector<TraceRec> recs;
  std::vector<hipEvent_t> pool;
  size_t used = 0;
  hipError_t get(hipEvent_t* e) {
    if (used == pool.size()) {
      hipEvent_t n;
      hipError_t r = hipEventCreate(&n);
      if (r != hipSuccess) return r;
      pool.push_back(n);
    }
    *e = pool[used++];
    return hipSuccess;
  }
  void clear() {
    recs.clear();
    used = 0;
  }
  ~Tracer() {
    for (auto e : pool) (void)hipEventDestroy(e);
  }
};

}  // namespace

struct photon_ctx {
  photon_config cfg;
  const unsigned char* wdec = nullptr;
  const unsigned char* wpre = nullptr;
  std::vector<TensorDesc> tensors;
  const void* E = nullptr;
  const void *W_ch1 = nullptr, *W_ch2 = nullptr, *W_cv2 = nullptr, *W_cv1 = nullptr, *W_out = nullptr;
  StackW enc1, top, dec1, dec0;
  // decode state
  bool prefilled = false;
  int mode = 0;
  int64_t B = 0, max_tokens = 0, top_len = 0, tokens = 0, prompt_tokens = 0;
  unsigned char* ws = nullptr;
  WsPlan plan;
  Tracer tr;
};

namespace {

const unsigned char* tensor_ptr(photon_ctx* c, const std::string& name) {
  for (const auto& t : c->tensors)
    if (t.name == name) {
      const unsigned char* base = t.blob ? c->wpre : c->wdec;
      return base ? base + t.offset : nullptr;
    }
  return nullptr;
}

void bind_stack(photon_ctx* c, StackW& s, const char* pre, int n) {
  s.layers.clear();
  for (int l = 0; l < n; ++l) {
    char p[32];
    snprintf(p, sizeof p, "%s.%d.", pre, l);
    const std::string b = p;
    LayerW w;
    w.g1 = (const float*)tensor_ptr(c, b + "g1");
    w.Wqkv = tensor_ptr(c, b + "Wq");
    w.Wo = tensor_ptr(c, b + "Wo");
    w.g2 = (const float*)tensor_ptr(c, b + "g2");
    w.W1 = tensor_ptr(c, b + "W1");
    w.W2 = tensor_ptr(c, b + "W2");
    s.layers.push_back(w);
  }
  s.gf = (const float*)tensor_ptr(c, std::string(pre) + ".gf");
}

void bind_weights(photon_ctx* c) {
  c->E = tensor_ptr(c, "E");
  c->W_ch2 = tensor_ptr(c, "W_ch2");
  c->W_cv2 = tensor_ptr(c, "W_cv2");
  c->W_cv1 = tensor_ptr(c, "W_cv1");
  c->W_out = tensor_ptr(c, "W_out");
  c->W_ch1 = tensor_ptr(c, "W_ch1");
  bind_stack(c, c->top, "top", c->cfg.n_top);
  bind_stack(c, c->dec1, "dec1", c->cfg.n_dec1);
  bind_stack(c, c->dec0, "dec0", c->cfg.n_dec0);
  bind_stack(c, c->enc1, "enc1", c->cfg.n_enc1);
}

#define HIP_TRY(expr)                                                                    \
  do {                                                                                   \
    hipError_t e_ = (expr);                                                              \
    if (e_ != hipSuccess) return fail(PHOTON_EHIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

#define PH_TRY(expr)            \
  do {                          \
    photon_status s_ = (expr);  \
    if (s_ != PHOTON_OK) return s_; \
  } while (0)

// Launch `f` (returning hipError_t); when class `cls` is traced, bracket it
// with HIP events on the same stream and keep its algorithmic bytes/flops.
template <class F>
photon_status traced(photon_ctx* c, int cls, double bytes, double flops, hipStream_t st, const char* what, F&& f) {
  const bool on = (c->tr.mask >> cls) & 1u;
  hipEvent_t a = nullptr, b = nullptr;
  if (on) {
    HIP_TRY(c->tr.get(&a));
    HIP_TRY(hipEventRecord(a, st));
  }
  const hipError_t e = f();
  if (e != hipSuccess) return fail(PHOTON_EHIP, "%s: %s", what, hipGetErrorString(e));
  if (on) {
    HIP_TRY(c->tr.get(&b));
    HIP_TRY(hipEventRecord(b, st));
    c->tr.recs.push_back({cls, a, b, bytes, flops});
  }
  return PHOTON_OK;
}

// Algorithmic bytes of one GEMM launch: W and A read once, C written (and
// read too for the residual update); the head writes its argmax partials.
double gemm_bytes(const GemmCall& g) {
  const double eb = g.dtype ? 2 : 4;
  double b = (double)g.N * g.K * eb + (double)g.M * g.K * eb;
  switch (g.epi) {
    case EPI_STORE: b += (double)g.M * g.N * 4; break;
    case EPI_ADD: b += 2.0 * g.M * g.N * 4; break;
    case EPI_GELU: b += (double)g.M * g.N * eb; break;
    default:
      b += (double)gemm_argmax_tiles(g.dtype, g.M, g.N, g.K) * g.M * 8;
      if (g.C) b += (double)g.M * g.N * 4;
  }
  return b;
}

photon_status run_gemm(photon_ctx* c, int cls, const GemmCall& g, hipStream_t st) {
  return traced(c, cls, gemm_bytes(g), 2.0 * g.M * g.N * g.K, st, "gemm", [&] { return launch_gemm(g, st); });
}

// Where a stack's K/V live.
struct KvTarget {
  unsigned char* base;   // layer 0 K plane
  int64_t plane_elems;   // elements per K (or V) plane
  bool per_layer;        // false: every layer reuses the same planes
  int64_t seq_stride;    // H*cap*hd
  int cap, seq0;
};

enum AttnKind { ATT_PREFILL, ATT_DECODE, ATT_CHUNK };

struct StackBufs {
  float* x;
  void* a;
  float* qkv;
  float* q;
  void* o;
  void* hid;
  float* part;
};

struct StackRun {
  int M, rows_per_seq, G;
  KvTarget kv;
  int pos_add; const int* pos_dev; int pos_mul;
  const float* rope;
  AttnKind kind;
  int Q, L_host; const int* L_dev; int L_mul, L_add; int nsplit;
  int L_acct;  // keys visible to the last query (host mirror, for accounting)
  // final norm: rows out_rows, input row r*in_stride + in_off
  void* out; int out_rows; int64_t in_stride, in_off;
};

photon_status run_stack(photon_ctx* c, const StackW& sw, const StackBufs& b, const StackRun& r, hipStream_t st) {
  const photon_config& cf = c->cfg;
  const int dt = cf.dtype, d = cf.d_model, H = cf.n_heads, hd = d / H, F = cf.mlp_mult * d;
  const int eb = elem_bytes(&cf);
  const double norm_bytes = (double)r.M * d * (4 + eb) + d * 4.0;
  for (size_t l = 0; l < sw.layers.size(); ++l) {
    const LayerW& w = sw.layers[l];
    PH_TRY(traced(c, PHOTON_K_NORM, norm_bytes, 4.0 * r.M * d, st, "rmsnorm",
                  [&] { return launch_rmsnorm(dt, b.x, 1, 0, w.g1, b.a, r.M, d, cf.norm_eps, st); }));
    GemmCall g{};
    g.dtype = dt; g.A = b.a; g.lda = d; g.W = w.Wqkv; g.M = r.M; g.N = 3 * d; g.K = d;
    g.epi = EPI_STORE; g.C = b.qkv; g.ldc = 3 * d;
    PH_TRY(run_gemm(c, PHOTON_K_GEMM_QKV, g, st));
    unsigned char* kbase = r.kv.base + (r.kv.per_layer ? (int64_t)l * 2 * r.kv.plane_elems * eb : 0);
    void* Kc = kbase;
    void* Vc = kbase + r.kv.plane_elems * eb;
    RopeKvCall rc{dt, b.qkv, r.M, d, H, hd, b.q, Kc, Vc, r.kv.seq_stride, r.kv.cap, r.rows_per_seq, r.kv.seq0,
                  r.pos_add, r.pos_dev, r.pos_mul, r.rope};
    PH_TRY(traced(c, PHOTON_K_ROPE_KV, (double)r.M * d * (12 + 4 + 2 * eb), 6.0 * r.M * d, st, "rope_kv",
                  [&] { return launch_rope_kv(rc, st); }));
    AttnCall ac{dt, r.G, r.Q, H, hd, b.q, d, Kc, Vc, r.kv.seq_stride, r.kv.cap, r.kv.seq0,
                r.L_host, r.L_dev, r.L_mul, r.L_add, b.o, d, b.part, r.nsplit};
    // K and V of every visible key read once, q read, output written
    double abytes = (double)r.G * H * r.L_acct * hd * eb * 2 + (double)r.M * d * (4 + eb);
    if (r.kind == ATT_DECODE && r.nsplit > 1) abytes += 2.0 * r.G * H * r.Q * r.nsplit * (hd + 2) * 4;
    const double aflops = 4.0 * r.G * H * r.Q * (double)r.L_acct * hd;
    if (r.kind == ATT_PREFILL)
      PH_TRY(traced(c, PHOTON_K_ATTN_PREFILL, abytes, aflops / 2, st, "attn_prefill",
                    [&] { return launch_attn_prefill(ac, st); }));
    else if (r.kind == ATT_DECODE)
      PH_TRY(traced(c, PHOTON_K_ATTN_TOP, abytes, aflops, st, "attn_decode",
                    [&] { return launch_attn_decode(ac, st); }));
    else
      PH_TRY(traced(c, PHOTON_K_ATTN_CHUNK, abytes, aflops, st, "attn_chunk",
                    [&] { return launch_attn_chunk(ac, st); }));
    g = GemmCall{};
    g.dtype = dt; g.A = b.o; g.lda = d; g.W = w.Wo; g.M = r.M; g.N = d; g.K = d;
    g.epi = EPI_ADD; g.C = b.x; g.ldc = d;
    PH_TRY(run_gemm(c, PHOTON_K_GEMM_O, g, st));
    PH_TRY(traced(c, PHOTON_K_NORM, norm_bytes, 4.0 * r.M * d, st, "rmsnorm",
                  [&] { return launch_rmsnorm(dt, b.x, 1, 0, w.g2, b.a, r.M, d, cf.norm_eps, st); }));
    g = GemmCall{};
    g.dtype = dt; g.A = b.a; g.lda = d; g.W = w.W1; g.M = r.M; g.N = F; g.K = d;
    g.epi = EPI_GELU; g.Cb = b.hid; g.ldc = F;
    PH_TRY(run_gemm(c, PHOTON_K_GEMM_UP, g, st));
    g = GemmCall{};
    g.dtype = dt; g.A = b.hid; g.lda = F; g.W = w.W2; g.M = r.M; g.N = d; g.K = F;
    g.epi = EPI_ADD; g.C = b.x; g.ldc = d;
    PH_TRY(run_gemm(c, PHOTON_K_GEMM_DOWN, g, st));
  }
  PH_TRY(traced(c, PHOTON_K_NORM, (double)r.out_rows * d * (4 + eb) + d * 4.0, 4.0 * r.out_rows * d, st, "rmsnorm",
                [&] { return launch_rmsnorm(dt, b.x, r.in_stride, r.in_off, sw.gf, r.out, r.out_rows, d, cf.norm_eps, st); }));
  return ok();
}

photon_status gemm_plain(photon_ctx* c, int cls, const void* A, int64_t lda, const void* W, int M, int N, int K,
                         float* C, int64_t ldc, hipStream_t st) {
  GemmCall g{};
  g.dtype = c->cfg.dtype; g.A = A; g.lda = lda; g.W = W; g.M = M; g.N = N; g.K = K;
  g.epi = EPI_STORE; g.C = C; g.ldc = ldc;
  return run_gemm(c, cls, g, st);
}

photon_status check_gemms(const photon_config* c, int64_t B, int64_t R1, int64_t R2, int mode) {
  const int dt = c->dtype, d = c->d_model, F = c->mlp_mult * d, V = c->vocab;
  const int C1 = c->chunk[0], C2 = c->chunk[1];
  struct S3 { int64_t M; int N, K; };
  std::vector<S3> shapes = {{B, C2 * d, d}, {B * C2, C1 * d, d}, {B * C2, V, d}, {B, d, C2 * d},
                            {R1, d, C1 * d}, {R2, d, C2 * d}};
  for (int64_t M : {B, B * C2, R1, R2}) {
    shapes.push_back({M, 3 * d, d});
    shapes.push_back({M, d, d});
    shapes.push_back({M, F, d});
    shapes.push_back({M, d, F});
  }
  if (mode == PHOTON_HIERGEN) shapes.push_back({B * C2, d, C1 * d});
  for (const auto& s : shapes)
    if (s.M > 0x7fffffff || !gemm_supported(dt, (int)s.M, s.N, s.K))
      return fail(PHOTON_EUNSUPPORTED, "GEMM shape M=%lld N=%d K=%d is not supported", (long long)s.M, s.N, s.K);
  return ok();
}

}  // namespace

// ====================================================================== ABI
extern "C" {

const char* photon_last_error(void) { return g_err.c_str(); }

photon_status photon_kv_bytes(const photon_config* cfg, int32_t batch, int64_t tokens, int32_t mode,
                              photon_kv_report* out) {
  photon_status s = check_config(cfg);
  if (s) return s;
  if (!out) return fail(PHOTON_EINVAL, "out is NULL");
  if (mode != PHOTON_RECGEN && mode != PHOTON_HIERGEN) return fail(PHOTON_EINVAL, "bad mode %d", mode);
  if (batch < 1) return fail(PHOTON_ESHAPE, "batch must be >= 1");
  if (tokens < 1) return fail(PHOTON_ESHAPE, "tokens must be >= 1");
  const WsPlan p = plan_workspace(cfg, batch, tokens, mode);
  memset(out, 0, sizeof *out);
  out->top_len = p.top_cap;
  out->lower_len = mode == PHOTON_HIERGEN ? p.low_cap : 0;
  out->top_kv = p.top_kv.bytes;
  out->lower_kv = p.low_kv.bytes;
  out->dec_kv = p.dec_kv.bytes;
  out->state = p.state_bytes;
  out->decode_scratch = p.scratch_bytes;
  out->workspace_total = p.total;
  layout(cfg, &out->weights_decode, &out->weights_prefill_only);
  out->off_top_kv = p.top_kv.off;
  out->off_lower_kv = p.low_kv.off;
  out->off_dec_kv = p.dec_kv.off;
  out->off_state = p.h.off;
  out->off_scratch = p.off_scratch;
  return ok();
}

photon_status photon_prefill_scratch_bytes(const photon_config* cfg, int32_t batch, int32_t prompt_len, int32_t mode,
                                           uint64_t* out) {
  photon_status s = check_config(cfg);
  if (s) return s;
  if (!out) return fail(PHOTON_EINVAL, "out is NULL");
  if (mode != PHOTON_RECGEN && mode != PHOTON_HIERGEN) return fail(PHOTON_EINVAL, "bad mode %d", mode);
  if (batch < 1) return fail(PHOTON_ESHAPE, "batch must be >= 1");
  const int S = cfg->chunk[0] * cfg->chunk[1];
  if (prompt_len < S || prompt_len % S)
    return fail(PHOTON_ESHAPE, "prompt_len %d must be a positive multiple of C1*C2 = %d", prompt_len, S);
  *out = plan_prefill(cfg, batch, prompt_len, mode).total;
  return ok();
}

photon_status photon_weight_layout(const photon_config* cfg, uint64_t* decode_bytes, uint64_t* prefill_only_bytes,
                                   int32_t* n_tensors) {
  photon_status s = check_config(cfg);
  if (s) return s;
  auto v = layout(cfg, decode_bytes, prefill_only_bytes);
  if (n_tensors) *n_tensors = (int32_t)v.size();
  return ok();
}

photon_status photon_weight_tensor(const photon_config* cfg, int32_t index, photon_tensor_info* out) {
  photon_status s = check_config(cfg);
  if (s) return s;
  if (!out) return fail(PHOTON_EINVAL, "out is NULL");
  auto v = layout(cfg, nullptr, nullptr);
  if (index < 0 || index >= (int32_t)v.size()) return fail(PHOTON_EINVAL, "tensor index %d out of range", index);
  const TensorDesc& t = v[index];
  memset(out, 0, sizeof *out);
  snprintf(out->name, sizeof out->name, "%s", t.name.c_str());
  out->blob = t.blob;
  out->dtype = t.is_gain ? PHOTON_F32 : cfg->dtype;
  out->offset = t.offset;
  out->rows = t.rows;
  out->cols = t.cols;
  return ok();
}

photon_status photon_open(const photon_config* cfg, const void* d_w_decode, const void* d_w_prefill_only,
                          photon_ctx** out) {
  photon_status s = check_config(cfg);
  if (s) return s;
  if (!out) return fail(PHOTON_EINVAL, "out is NULL");
  if (!d_w_decode) return fail(PHOTON_EINVAL, "decode weight blob is NULL");
  if (((uintptr_t)d_w_decode | (uintptr_t)d_w_prefill_only) % kAlign)
    return fail(PHOTON_EINVAL, "weight blobs must be 256-byte aligned");
  photon_ctx* c = new (std::nothrow) photon_ctx();
  if (!c) return fail(PHOTON_EINVAL, "out of host memory");
  c->cfg = *cfg;
  c->wdec = (const unsigned char*)d_w_decode;
  c->wpre = (const unsigned char*)d_w_prefill_only;
  c->tensors = layout(cfg, nullptr, nullptr);
  bind_weights(c);
  *out = c;
  return ok();
}

photon_status photon_release_prefill_weights(photon_ctx* c) {
  if (!c) return fail(PHOTON_EINVAL, "ctx is NULL");
  c->wpre = nullptr;
  bind_weights(c);
  return ok();
}

photon_status photon_close(photon_ctx* c) {
  delete c;
  return ok();
}

photon_status photon_position(const photon_ctx* c, int64_t* top_len, int64_t* tokens) {
  if (!c) return fail(PHOTON_EINVAL, "ctx is NULL");
  if (top_len) *top_len = c->prefilled ? c->top_len : 0;
  if (tokens) *tokens = c->prefilled ? c->tokens : 0;
  return ok();
}

photon_status photon_prefill(photon_ctx* c, int32_t mode, void* d_workspace, uint64_t ws_bytes, void* d_scratch,
                             uint64_t scratch_bytes, const int32_t* d_prompt, int32_t batch, int32_t prompt_len,
                             int64_t max_tokens, void* stream) {
  if (!c) return fail(PHOTON_EINVAL, "ctx is NULL");
  if (mode != PHOTON_RECGEN && mode != PHOTON_HIERGEN) return fail(PHOTON_EINVAL, "bad mode %d", mode);
  if (!d_workspace || !d_scratch || !d_prompt) return fail(PHOTON_EINVAL, "NULL device pointer");
  if (((uintptr_t)d_workspace | (uintptr_t)d_scratch) % kAlign)
    return fail(PHOTON_EINVAL, "workspace and scratch must be 256-byte aligned");
  if (!c->wpre) return fail(PHOTON_ESTATE, "prefill needs the prefill-only weights, which were released");
  const photon_config& cf = c->cfg;
  const int C1 = cf.chunk[0], C2 = cf.chunk[1], S = C1 * C2;
  if (batch < 1) return fail(PHOTON_ESHAPE, "batch must be >= 1");
  if (prompt_len < S || prompt_len % S)
    return fail(PHOTON_ESHAPE, "prompt_len %d must be a positive multiple of C1*C2 = %d", prompt_len, S);
  if (max_tokens < prompt_len) return fail(PHOTON_ECAPACITY, "max_tokens %lld < prompt_len %d", (long long)max_tokens, prompt_len);
  const WsPlan wp = plan_workspace(&cf, batch, max_tokens, mode);
  if (ws_bytes < wp.total)
    return fail(PHOTON_ECAPACITY, "workspace holds %llu bytes, needs %llu", (unsigned long long)ws_bytes,
                (unsigned long long)wp.total);
  const PrePlan pp = plan_prefill(&cf, batch, prompt_len, mode);
  if (scratch_bytes < pp.total)
    return fail(PHOTON_ECAPACITY, "prefill scratch holds %llu bytes, needs %llu", (unsigned long long)scratch_bytes,
                (unsigned long long)pp.total);
  {
    photon_status s = check_gemms(&cf, batch, pp.bs * pp.n1, pp.bs * pp.n, mode);
    if (s) return s;
  }
  hipStream_t st = (hipStream_t)stream;
  const int dt = cf.dtype, d = cf.d_model, H = cf.n_heads, hd = d / H;
  const int eb = elem_bytes(&cf);
  unsigned char* ws = (unsigned char*)d_workspace;
  unsigned char* sc = (unsigned char*)d_scratch;
  c->prefilled = false;
  c->ws = ws;
  c->plan = wp;
  c->mode = mode;
  c->B = batch;
  c->max_tokens = max_tokens;

  float* rope_ws = (float*)(ws + wp.rope.off);
  float* rope1 = (float*)(sc + pp.rope1.off);
  HIP_TRY(launch_rope_table(rope_ws, (int)wp.rope_pos, hd, cf.rope_theta, st));
  HIP_TRY(launch_rope_table(rope1, (int)std::max<int64_t>(pp.n1, 1), hd, cf.rope_theta, st));

  const int64_t n1 = pp.n1, n = pp.n;
  StackBufs bufs{(float*)(sc + pp.x.off), sc + pp.a.off, (float*)(sc + pp.qkv.off), (float*)(sc + pp.q.off),
                 sc + pp.o.off, sc + pp.hid.off, nullptr};
  for (int64_t b0 = 0; b0 < batch; b0 += pp.bs) {
    const int bs = (int)std::min<int64_t>(pp.bs, batch - b0);
    // embedding rows of bs*P tokens == Chunker^1 input [bs*n1][C1*d]
    PH_TRY(traced(c, PHOTON_K_EMBED, (double)bs * prompt_len * (4 + 2.0 * d * eb), 0, st, "embed_gather", [&] {
      return launch_embed_gather(dt, d_prompt + b0 * prompt_len, (int64_t)bs * prompt_len, c->E, d, cf.vocab,
                                 sc + pp.e.off, st);
    }));
    {
      photon_status s = gemm_plain(c, PHOTON_K_GEMM_CHUNK, sc + pp.e.off, (int64_t)C1 * d, c->W_ch1, (int)(bs * n1), d, C1 * d, bufs.x, d, st);
      if (s) return s;
    }
    StackRun r{};
    r.M = (int)(bs * n1); r.rows_per_seq = (int)n1; r.G = bs;
    if (mode == PHOTON_HIERGEN) {
      r.kv = KvTarget{ws + wp.low_kv.off, (int64_t)batch * H * wp.low_cap * hd, true, (int64_t)H * wp.low_cap * hd,
                      (int)wp.low_cap, (int)b0};
    } else {
      r.kv = KvTarget{sc + pp.kv1.off, (int64_t)pp.bs * H * n1 * hd, false, (int64_t)H * n1 * hd, (int)n1, 0};
    }
    r.pos_add = 0; r.pos_dev = nullptr; r.pos_mul = 0; r.rope = rope1;
    r.kind = ATT_PREFILL; r.Q = (int)n1; r.L_host = (int)n1; r.nsplit = 1; r.L_acct = (int)n1;
    r.out = sc + pp.A1.off; r.out_rows = (int)(bs * n1); r.in_stride = 1; r.in_off = 0;
    {
      photon_status s = run_stack(c, c->enc1, bufs, r, st);
      if (s) return s;
    }
    // Chunker^2 over groups of C2 level-1 states
    {
      photon_status s = gemm_plain(c, PHOTON_K_GEMM_CHUNK, sc + pp.A1.off, (int64_t)C2 * d, c->W_ch2, (int)(bs * n), d, C2 * d, bufs.x, d, st);
      if (s) return s;
    }
    StackRun t{};
    t.M = (int)(bs * n); t.rows_per_seq = (int)n; t.G = bs;
    t.kv = KvTarget{ws + wp.top_kv.off, (int64_t)batch * H * wp.top_cap * hd, true, (int64_t)H * wp.top_cap * hd,
                    (int)wp.top_cap, (int)b0};
    t.pos_add = 0; t.pos_dev = nullptr; t.pos_mul = 0; t.rope = rope_ws;
    t.kind = ATT_PREFILL; t.Q = (int)n; t.L_host = (int)n; t.nsplit = 1; t.L_acct = (int)n;
    // final norm only for the last top state of each sequence: h_{n-1}
    t.out = ws + wp.h.off + (uint64_t)b0 * d * eb; t.out_rows = bs; t.in_stride = n; t.in_off = n - 1;
    {
      photon_status s = run_stack(c, c->top, bufs, t, st);
      if (s) return s;
    }
  }
  HIP_TRY(launch_set_int((int*)(ws + wp.counter.off), (int)n, st));
  c->top_len = n;
  c->tokens = prompt_len;
  c->prompt_tokens = prompt_len;
  c->prefilled = true;
  return ok();
}

photon_status photon_decode_chunk(photon_ctx* c, int32_t* d_tokens, float* d_logits, void* stream) {
  if (!c) return fail(PHOTON_EINVAL, "ctx is NULL");
  if (!d_tokens) return fail(PHOTON_EINVAL, "d_tokens is NULL");
  if (!c->prefilled) return fail(PHOTON_ESTATE, "decode before prefill");
  const photon_config& cf = c->cfg;
  const int C1 = cf.chunk[0], C2 = cf.chunk[1], S = C1 * C2;
  if (c->tokens + S > c->max_tokens)
    return fail(PHOTON_ECAPACITY, "chunk would pass max_tokens %lld", (long long)c->max_tokens);
  if (c->mode == PHOTON_HIERGEN && !c->wpre)
    return fail(PHOTON_ESTATE, "HierGen decoding needs the prefill-only weights, which were released");
  hipStream_t st = (hipStream_t)stream;
  const WsPlan& wp = c->plan;
  unsigned char* ws = c->ws;
  const int dt = cf.dtype, d = cf.d_model, H = cf.n_heads, hd = d / H, V = cf.vocab;
  const int B = (int)c->B, MB = B * C2;
  const int eb = elem_bytes(&cf);
  int* counter = (int*)(ws + wp.counter.off);
  const float* rope = (const float*)(ws + wp.rope.off);
  void* h = ws + wp.h.off;
  void* Ahat = ws + wp.Ahat.off;
  int* tok = (int*)(ws + wp.tok.off);
  int* prev = (int*)(ws + wp.prev.off);
  StackBufs sb{(float*)(ws + wp.xB.off), ws + wp.aB.off, (float*)(ws + wp.qkvB.off), (float*)(ws + wp.qB.off),
               ws + wp.oB.off, ws + wp.hidB.off, nullptr};
  StackBufs sa{(float*)(ws + wp.xA.off), ws + wp.aA.off, (float*)(ws + wp.qkvA.off), (float*)(ws + wp.qA.off),
               ws + wp.oA.off, ws + wp.hidA.off, (float*)(ws + wp.partA.off)};
  photon_status s;

  // Converter^2: h_{i-1} -> C2 conditioning vectors (rows of the level-1 decoder)
  if ((s = gemm_plain(c, PHOTON_K_GEMM_CONV, h, d, c->W_cv2, B, C2 * d, d, sb.x, (int64_t)C2 * d, st))) return s;
  // level-1 decoder over the C2 positions of the chunk -> A-hat_i
  {
    StackRun r{};
    r.M = MB; r.rows_per_seq = C2; r.G = B;
    r.kv = KvTarget{ws + wp.kv1tmp.off, (int64_t)B * H * C2 * hd, false, (int64_t)H * C2 * hd, C2, 0};
    r.pos_add = 0; r.rope = rope;
    r.kind = ATT_CHUNK; r.Q = C2; r.L_host = C2; r.nsplit = 1; r.L_acct = C2;
    r.out = Ahat; r.out_rows = MB; r.in_stride = 1; r.in_off = 0;
    if ((s = run_stack(c, c->dec1, sb, r, st))) return s;
  }
  // token branch: Converter^1 then C1 sequential token-decoder steps
  if ((s = gemm_plain(c, PHOTON_K_GEMM_CONV, Ahat, d, c->W_cv1, MB, C1 * d, d, (float*)(ws + wp.c0.off), (int64_t)C1 * d, st))) return s;
  for (int j = 0; j < C1; ++j) {
    PH_TRY(traced(c, PHOTON_K_EMBED, (double)MB * d * (8 + (j > 0 ? eb : 0)), (double)MB * d, st, "embed_add", [&] {
      return launch_embed_add(dt, (const float*)(ws + wp.c0.off), (int64_t)C1 * d, j, prev, c->E, MB, d, sb.x, st);
    }));
    StackRun r{};
    r.M = MB; r.rows_per_seq = 1; r.G = MB;
    r.kv = KvTarget{ws + wp.dec_kv.off, (int64_t)MB * H * C1 * hd, true, (int64_t)H * C1 * hd, C1, 0};
    r.pos_add = j; r.rope = rope;
    r.kind = ATT_CHUNK; r.Q = 1; r.L_host = j + 1; r.nsplit = 1; r.L_acct = j + 1;
    r.out = ws + wp.zB.off; r.out_rows = MB; r.in_stride = 1; r.in_off = 0;
    if ((s = run_stack(c, c->dec0, sb, r, st))) return s;
    GemmCall g{};
    g.dtype = dt; g.A = ws + wp.zB.off; g.lda = d; g.W = c->W_out; g.M = MB; g.N = V; g.K = d;
    g.epi = EPI_ARGMAX;
    g.C = d_logits ? d_logits + (int64_t)j * V : nullptr;
    g.ldc = (int64_t)C1 * V;
    g.amax_val = (float*)(ws + wp.amv.off); g.amax_idx = (int*)(ws + wp.ami.off);
    PH_TRY(run_gemm(c, PHOTON_K_GEMM_HEAD, g, st));
    PH_TRY(traced(c, PHOTON_K_ARGMAX, (double)wp.head_tiles * MB * 8 + MB * 8.0, 0, st, "argmax", [&] {
      return launch_argmax_finalize(g.amax_val, g.amax_idx, wp.head_tiles, MB, C1, C2, j, tok, prev, st);
    }));
  }
  // top branch
  if (c->mode == PHOTON_RECGEN) {
    // feedback: u_i = Chunker^2(A-hat_i), nothing re-encoded
    if ((s = gemm_plain(c, PHOTON_K_GEMM_CHUNK, Ahat, (int64_t)C2 * d, c->W_ch2, B, d, C2 * d, sa.x, d, st))) return s;
  } else {
    // HierGen: re-encode the chunk's tokens through Chunker^1 and one
    // level-1 encoder step, then Chunker^2 of the encoder summary A_i
    PH_TRY(traced(c, PHOTON_K_EMBED, (double)B * S * (4 + 2.0 * d * eb), 0, st, "embed_gather",
                  [&] { return launch_embed_gather(dt, tok, (int64_t)B * S, c->E, d, V, ws + wp.eA.off, st); }));
    if ((s = gemm_plain(c, PHOTON_K_GEMM_CHUNK, ws + wp.eA.off, (int64_t)C1 * d, c->W_ch1, MB, d, C1 * d, sa.x, d, st))) return s;
    StackRun r{};
    r.M = MB; r.rows_per_seq = C2; r.G = B;
    r.kv = KvTarget{ws + wp.low_kv.off, (int64_t)B * H * wp.low_cap * hd, true, (int64_t)H * wp.low_cap * hd,
                    (int)wp.low_cap, 0};
    r.pos_add = 0; r.pos_dev = counter; r.pos_mul = C2; r.rope = rope;
    r.kind = ATT_DECODE; r.Q = C2; r.L_dev = counter; r.L_mul = C2; r.L_add = C2; r.nsplit = wp.nsplit_low;
    r.L_acct = (int)((c->top_len + 1) * C2);
    r.out = ws + wp.AA.off; r.out_rows = MB; r.in_stride = 1; r.in_off = 0;
    if ((s = run_stack(c, c->enc1, sa, r, st))) return s;
    if ((s = gemm_plain(c, PHOTON_K_GEMM_CHUNK, ws + wp.AA.off, (int64_t)C2 * d, c->W_ch2, B, d, C2 * d, sa.x, d, st))) return s;
  }
  {
    StackRun r{};
    r.M = B; r.rows_per_seq = 1; r.G = B;
    r.kv = KvTarget{ws + wp.top_kv.off, (int64_t)B * H * wp.top_cap * hd, true, (int64_t)H * wp.top_cap * hd,
                    (int)wp.top_cap, 0};
    r.pos_add = 0; r.pos_dev = counter; r.pos_mul = 1; r.rope = rope;
    r.kind = ATT_DECODE; r.Q = 1; r.L_dev = counter; r.L_mul = 1; r.L_add = 1; r.nsplit = wp.nsplit_top;
    r.L_acct = (int)(c->top_len + 1);
    r.out = h; r.out_rows = B; r.in_stride = 1; r.in_off = 0;
    if ((s = run_stack(c, c->top, sa, r, st))) return s;
  }
  HIP_TRY(launch_add_int(counter, 1, st));
  HIP_TRY(hipMemcpyAsync(d_tokens, tok, (size_t)B * S * sizeof(int), hipMemcpyDeviceToDevice, st));
  c->top_len += 1;
  c->tokens += S;
  return ok();
}

photon_status photon_set_position(photon_ctx* c, int64_t tokens, void* stream) {
  if (!c) return fail(PHOTON_EINVAL, "ctx is NULL");
  if (!c->prefilled) return fail(PHOTON_ESTATE, "no prefill to rewind to");
  const int64_t S = (int64_t)c->cfg.chunk[0] * c->cfg.chunk[1];
  if (tokens % S || tokens < c->prompt_tokens || tokens > c->tokens)
    return fail(PHOTON_ESHAPE, "position %lld must be a multiple of %lld within [%lld, %lld]", (long long)tokens,
                (long long)S, (long long)c->prompt_tokens, (long long)c->tokens);
  HIP_TRY(launch_set_int((int*)(c->ws + c->plan.counter.off), (int)(tokens / S), (hipStream_t)stream));
  c->tokens = tokens;
  c->top_len = tokens / S;
  return ok();
}

photon_status photon_trace_enable(photon_ctx* c, uint32_t class_mask) {
  if (!c) return fail(PHOTON_EINVAL, "ctx is NULL");
  c->tr.mask = class_mask & ((1u << PHOTON_K_COUNT) - 1);
  c->tr.clear();
  return ok();
}

photon_status photon_trace_read(photon_ctx* c, photon_trace_stat* out) {
  if (!c || !out) return fail(PHOTON_EINVAL, "NULL argument");
  memset(out, 0, sizeof(photon_trace_stat) * PHOTON_K_COUNT);
  for (const auto& r : c->tr.recs) {
    HIP_TRY(hipEventSynchronize(r.b));
    float ms = 0.f;
    HIP_TRY(hipEventElapsedTime(&ms, r.a, r.b));
    photon_trace_stat& o = out[r.cls];
    o.launches += 1;
    o.ms += ms;
    o.bytes += r.bytes;
    o.flops += r.flops;
  }
  c->tr.clear();
  return ok();
}

}  // extern "C"
