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
#include <chrono>
#include <thread>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
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
// The levels of a (checked) configuration: C[l] for l = 1 .. L, span[l] =
// C1*...*C_l tokens per level-l state (span[0] = 1), enc[l] encoder layers
// (l = 1 .. L-1), dec[l] decoder layers (l = 0 .. L-1).
struct Levels {
  int L = 2;
  int C[PHOTON_MAX_LEVELS + 1] = {};
  int64_t span[PHOTON_MAX_LEVELS + 1] = {};
  int enc[PHOTON_MAX_LEVELS] = {};
  int dec[PHOTON_MAX_LEVELS] = {};
  int64_t S() const { return span[L]; }
  // level-l states per chunk (one top state); K1 = level-1 states
  int64_t per_chunk(int l) const { return span[L] / span[l]; }
  int64_t K1() const { return per_chunk(1); }
};

Levels levels(const photon_config* c) {
  Levels v;
  v.L = c->n_levels;
  v.span[0] = 1;
  for (int l = 1; l <= v.L; ++l) {
    v.C[l] = c->chunk[l - 1];
    v.span[l] = v.span[l - 1] * v.C[l];
  }
  v.enc[1] = c->n_enc1;
  v.dec[0] = c->n_dec0;
  v.dec[1] = c->n_dec1;
  for (int l = 2; l < v.L; ++l) {
    v.enc[l] = c->n_enc_hi[l - 2];
    v.dec[l] = c->n_dec_hi[l - 2];
  }
  return v;
}

photon_status check_config(const photon_config* c) {
  if (!c) return fail(PHOTON_EINVAL, "config is NULL");
  if (c->n_levels < 2 || c->n_levels > PHOTON_MAX_LEVELS)
    return fail(PHOTON_EUNSUPPORTED, "n_levels must be in [2, %d] (got %d)", PHOTON_MAX_LEVELS, c->n_levels);
  for (int l = 0; l < c->n_levels; ++l) {
    if (c->chunk[l] < 1) return fail(PHOTON_ESHAPE, "chunk sizes must be >= 1");
    if (c->chunk[l] > 16) return fail(PHOTON_EUNSUPPORTED, "chunk sizes above 16 are not supported");
  }
  for (int l = 2; l < c->n_levels; ++l)
    if (c->n_enc_hi[l - 2] < 1 || c->n_dec_hi[l - 2] < 1)
      return fail(PHOTON_ESHAPE, "every stack needs at least one layer (level %d)", l);
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

#define PH_CHECK(expr)            \
  do {                            \
    photon_status s_ = (expr);    \
    if (s_ != PHOTON_OK) return s_; \
  } while (0)

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

std::string lname(const char* pre, int l) {
  char b[16];
  snprintf(b, sizeof b, "%s%d", pre, l);
  return b;
}

// Blob order follows the decode call order (decode blob: the top chunker,
// the top, then converter and decoder level by level downwards, the head)
// and the prefill order (chunker and encoder level by level upwards).
std::vector<TensorDesc> layout(const photon_config* c, uint64_t* dec_bytes, uint64_t* pre_bytes) {
  const int64_t d = c->d_model, F = (int64_t)c->mlp_mult * d, V = c->vocab;
  const Levels lv = levels(c);
  const int L = lv.L;
  std::vector<TensorDesc> v;
  v.push_back({"E", 0, 0, V, d, 0});
  v.push_back({lname("W_ch", L), 0, 0, d, lv.C[L] * d, 0});
  add_stack(v, "top", c->n_top, 0, d, F);
  for (int l = L; l >= 1; --l) {
    v.push_back({lname("W_cv", l), 0, 0, lv.C[l] * d, d, 0});
    add_stack(v, lname("dec", l - 1).c_str(), lv.dec[l - 1], 0, d, F);
  }
  v.push_back({"W_out", 0, 0, V, d, 0});
  for (int l = 1; l < L; ++l) {
    v.push_back({lname("W_ch", l), 1, 0, d, lv.C[l] * d, 0});
    add_stack(v, lname("enc", l).c_str(), lv.enc[l], 1, d, F);
  }
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
  // low_cap: the level-1 capacity (HierGen), low_caps[l] every lower level's
  int64_t top_cap = 0, low_cap = 0, rope_pos = 0;
  int64_t low_caps[PHOTON_MAX_LEVELS] = {};
  int nsplit_top = 1;
  int nsplit_low[PHOTON_MAX_LEVELS] = {1, 1, 1, 1};
  int head_tiles = 1;
  // persistent; low_kv spans the lower levels' regions lowl[1 .. L-1]
  Region top_kv, low_kv, dec_kv, h, counter, rope, tok, tail;
  Region lowl[PHOTON_MAX_LEVELS];
  // decode scratch, set A (top branch) and set B (decoders + tokens);
  // Ahat[l] holds the level-l decoder outputs of the chunk (l = 1 .. L-1)
  Region xA, aA, partA, qA, oA, hidA, apartA, eA, AA;
  Region xB, aB, partB, qB, oB, hidB, c0, zB, kv1tmp, amv, ami;
  Region Ahat[PHOTON_MAX_LEVELS];
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

// bytes of the K-slab partials a STORE GEMM of this shape writes (with
// either tile preference)
uint64_t part_bytes(int dt, int64_t M, int64_t N, int64_t K) {
  const int ks = std::max(gemm_splits(dt, (int)M, (int)N, (int)K, 0), gemm_splits(dt, (int)M, (int)N, (int)K, 1));
  return (uint64_t)ks * M * N * 4;
}

// largest slab buffer any layer of a stack with M rows needs
uint64_t layer_part_bytes(const photon_config* c, int64_t M) {
  const int dt = c->dtype;
  const int64_t d = c->d_model, F = (int64_t)c->mlp_mult * d;
  return std::max({part_bytes(dt, M, 3 * d, d), part_bytes(dt, M, d, d), part_bytes(dt, M, d, F)});
}

WsPlan plan_workspace(const photon_config* c, int64_t B, int64_t tokens, int mode) {
  WsPlan p;
  const int dt = c->dtype;
  const int64_t d = c->d_model, H = c->n_heads, hd = d / H, F = (int64_t)c->mlp_mult * d, V = c->vocab;
  const Levels lv = levels(c);
  const int L = lv.L;
  const int64_t C1 = lv.C[1], CL = lv.C[L], S = lv.S(), K1 = lv.K1();
  const uint64_t eb = elem_bytes(c);
  const bool hier = mode == PHOTON_HIERGEN;
  p.top_cap = cdiv(tokens, S);
  p.rope_pos = p.top_cap;
  for (int l = 1; l <= L; ++l) p.rope_pos = std::max<int64_t>(p.rope_pos, lv.C[l]);
  for (int l = 1; l < L; ++l) {
    p.low_caps[l] = hier ? cdiv(tokens, lv.span[l]) : 0;
    p.rope_pos = std::max(p.rope_pos, p.low_caps[l]);
    p.nsplit_low[l] = hier ? attn_decode_splits((int)B, (int)H, (int)p.low_caps[l], (int)lv.per_chunk(l)) : 1;
  }
  p.low_cap = p.low_caps[1];
  p.nsplit_top = attn_decode_splits((int)B, (int)H, (int)p.top_cap, 1);
  p.head_tiles = gemm_argmax_tiles(dt, (int)(B * K1), (int)V, (int)d);
  Cursor cur;
  p.top_kv = cur.take((uint64_t)c->n_top * 2 * B * H * p.top_cap * hd * eb);
  p.low_kv.off = align_up(cur.pos);
  for (int l = 1; l < L; ++l) p.lowl[l] = cur.take((uint64_t)lv.enc[l] * 2 * B * H * p.low_caps[l] * hd * eb);
  p.low_kv.bytes = cur.pos - p.low_kv.off;
  p.dec_kv = cur.take((uint64_t)c->n_dec0 * 2 * B * K1 * H * C1 * hd * eb);
  p.off_state = align_up(cur.pos);
  p.h = cur.take((uint64_t)B * d * eb);
  p.counter = cur.take(sizeof(int));
  p.rope = cur.take((uint64_t)p.rope_pos * (hd / 2) * 2 * sizeof(float));
  p.tok = cur.take((uint64_t)B * S * sizeof(int));
  p.tail = cur.take((uint64_t)B * S * sizeof(int));   // a ragged prompt's tail tokens
  p.off_scratch = align_up(cur.pos);
  p.state_bytes = p.off_scratch - p.off_state;
  // Set A serves the top branch: the top (B rows), HierGen's re-encoding
  // (up to B*K1 rows at level 1) and RecGen's decoders for the next chunk
  // (up to B*K1 rows); set B the decoders and the token decoder (B*K1).
  // The level-l stacks run B*per_chunk(l) rows (fewer rows may take more K
  // slabs); the converters above level 1 and the chunkers store slabs too.
  const int64_t MA = B * K1, MB = B * K1;
  uint64_t stack_parts = layer_part_bytes(c, B);
  for (int l = 1; l < L; ++l) stack_parts = std::max(stack_parts, layer_part_bytes(c, B * lv.per_chunk(l)));
  for (int l = 2; l <= L; ++l) stack_parts = std::max(stack_parts, part_bytes(dt, B * lv.per_chunk(l), lv.C[l] * d, d));
  uint64_t partA = std::max(stack_parts, part_bytes(dt, B, d, CL * d));
  if (hier)
    for (int l = 1; l < L; ++l) partA = std::max(partA, part_bytes(dt, B * lv.per_chunk(l), d, lv.C[l] * d));
  p.xA = cur.take((uint64_t)MA * d * 4);
  p.aA = cur.take((uint64_t)MA * d * eb);
  p.partA = cur.take(partA);
  p.qA = cur.take((uint64_t)MA * d * 4);
  p.oA = cur.take((uint64_t)MA * d * eb);
  p.hidA = cur.take((uint64_t)MA * F * eb);
  int64_t parts = (int64_t)B * H * p.nsplit_top;
  if (hier)
    for (int l = 1; l < L; ++l) parts = std::max<int64_t>(parts, B * H * lv.per_chunk(l) * p.nsplit_low[l]);
  p.apartA = cur.take((uint64_t)parts * (hd + 2) * 4);
  p.eA = cur.take(hier ? (uint64_t)B * S * d * eb : 0);
  p.AA = cur.take(hier ? (uint64_t)B * K1 * d * eb : 0);
  const uint64_t partB = stack_parts;
  p.xB = cur.take((uint64_t)MB * d * 4);
  p.aB = cur.take((uint64_t)MB * d * eb);
  p.partB = cur.take(partB);
  p.qB = cur.take((uint64_t)MB * d * 4);
  p.oB = cur.take((uint64_t)MB * d * eb);
  p.hidB = cur.take((uint64_t)MB * F * eb);
  p.c0 = cur.take((uint64_t)MB * C1 * d * 4);
  for (int l = 1; l < L; ++l) p.Ahat[l] = cur.take((uint64_t)B * lv.per_chunk(l) * d * eb);
  p.zB = cur.take((uint64_t)MB * d * eb);
  // the chunk-confined decoders above the token decoder: C_l keys for each
  // of B*per_chunk(l) groups, at most B*K1 rows of K and V
  p.kv1tmp = cur.take((uint64_t)2 * B * H * K1 * hd * eb);
  p.amv = cur.take((uint64_t)p.head_tiles * MB * 4);
  p.ami = cur.take((uint64_t)p.head_tiles * MB * 4);
  p.total = align_up(cur.pos);
  p.scratch_bytes = p.total - p.off_scratch;
  return p;
}

// prefill scratch: one batch slice of bs sequences at a time
constexpr int64_t kPrefillRows = 65536;

// nl[l]: level-l states per sequence of the prompt (l = 1 .. L; n1 = nl[1],
// n = nl[L] top states).  One buffer A holds the output of the current
// encoder level: a level's chunker has read it before that level's stack
// writes it again.
struct PrePlan {
  int64_t bs = 1, n1 = 0, n = 0;
  int64_t nl[PHOTON_MAX_LEVELS + 1] = {};
  Region e, x, a, part, q, o, hid, A1, kv1, rope1;
  uint64_t total = 0;
};

PrePlan plan_prefill(const photon_config* c, int64_t B, int64_t P, int mode) {
  PrePlan p;
  const int dt = c->dtype;
  const int64_t d = c->d_model, H = c->n_heads, hd = d / H, F = (int64_t)c->mlp_mult * d;
  const Levels lv = levels(c);
  const uint64_t eb = elem_bytes(c);
  for (int l = 1; l <= lv.L; ++l) p.nl[l] = P / lv.span[l];
  p.n1 = p.nl[1];
  p.n = p.nl[lv.L];
  p.bs = std::max<int64_t>(1, std::min<int64_t>(B, kPrefillRows / std::max<int64_t>(1, p.n1)));
  const int64_t R = p.bs * p.n1;
  // the last slice may be shorter; its GEMMs plan their own slabs
  uint64_t part = 0;
  for (int64_t bs : {p.bs, B % p.bs}) {
    if (bs == 0) continue;
    for (int l = 1; l <= lv.L; ++l)
      part = std::max({part, layer_part_bytes(c, bs * p.nl[l]), part_bytes(dt, bs * p.nl[l], d, lv.C[l] * d)});
  }
  Cursor cur;
  p.e = cur.take((uint64_t)p.bs * P * d * eb);
  p.x = cur.take((uint64_t)R * d * 4);
  p.a = cur.take((uint64_t)R * d * eb);
  p.part = cur.take(part);
  p.q = cur.take((uint64_t)R * d * 4);
  p.o = cur.take((uint64_t)R * d * eb);
  p.hid = cur.take((uint64_t)R * F * eb);
  p.A1 = cur.take((uint64_t)R * d * eb);
  p.kv1 = cur.take(mode == PHOTON_HIERGEN ? 0 : (uint64_t)2 * p.bs * H * p.n1 * hd * eb);
  p.rope1 = cur.take((uint64_t)std::max<int64_t>(p.n1, 1) * (hd / 2) * 2 * 4);
  p.total = align_up(cur.pos);
  return p;
}

// ------------------------------------------------------- flat baseline plan
photon_status check_vconfig(const photon_vanilla_config* v) {
  if (!v) return fail(PHOTON_EINVAL, "config is NULL");
  photon_config c{};
  c.n_levels = 2;
  c.chunk[0] = 1; c.chunk[1] = 1;
  c.d_model = v->d_model; c.n_heads = v->n_heads; c.mlp_mult = v->mlp_mult; c.vocab = v->vocab;
  c.n_top = v->n_layers; c.n_enc1 = c.n_dec1 = c.n_dec0 = 1;
  c.dtype = v->dtype; c.norm_eps = v->norm_eps; c.rope_theta = v->rope_theta;
  PH_CHECK(check_config(&c));
  if (v->n_layers < 1) return fail(PHOTON_ESHAPE, "n_layers must be >= 1");
  if (v->steps < 1 || v->steps > 64) return fail(PHOTON_ESHAPE, "steps must be in [1, 64]");
  return ok();
}

// the photon_config the shared helpers read (dtype, widths, norm, rope)
photon_config vanilla_as_config(const photon_vanilla_config* v) {
  photon_config c{};
  c.n_levels = 2;
  c.chunk[0] = v->steps; c.chunk[1] = 1;
  c.d_model = v->d_model; c.n_heads = v->n_heads; c.mlp_mult = v->mlp_mult; c.vocab = v->vocab;
  c.n_top = v->n_layers; c.n_enc1 = c.n_dec1 = c.n_dec0 = 1;
  c.dtype = v->dtype; c.norm_eps = v->norm_eps; c.rope_theta = v->rope_theta;
  return c;
}

std::vector<TensorDesc> vlayout(const photon_vanilla_config* v, uint64_t* bytes) {
  const int64_t d = v->d_model, F = (int64_t)v->mlp_mult * d, V = v->vocab;
  std::vector<TensorDesc> t;
  t.push_back({"E", 0, 0, V, d, 0});
  add_stack(t, "layers", v->n_layers, 0, d, F);
  t.push_back({"W_out", 0, 0, V, d, 0});
  uint64_t off = 0;
  const int eb = v->dtype == PHOTON_BF16 ? 2 : 4;
  for (auto& x : t) {
    x.offset = align_up(off);
    off = x.offset + (uint64_t)x.rows * x.cols * (x.is_gain ? 4 : eb);
  }
  if (bytes) *bytes = align_up(off);
  return t;
}

struct VPlan {
  int64_t cap = 0;
  int nsplit = 1, head_tiles = 1;
  Region kv, z, counter, rope, tok;
  Region x, a, part, q, o, hid, apart, amv, ami;
  uint64_t state_bytes = 0, scratch_bytes = 0, total = 0, off_state = 0, off_scratch = 0;
};

VPlan plan_vworkspace(const photon_vanilla_config* v, int64_t B, int64_t tokens) {
  VPlan p;
  const photon_config c = vanilla_as_config(v);
  const int dt = c.dtype;
  const int64_t d = v->d_model, H = v->n_heads, hd = d / H, F = (int64_t)v->mlp_mult * d, V = v->vocab;
  const uint64_t eb = elem_bytes(&c);
  p.cap = tokens;
  p.nsplit = attn_decode_splits((int)B, (int)H, (int)tokens, 1);
  p.head_tiles = gemm_argmax_tiles(dt, (int)B, (int)V, (int)d);
  Cursor cur;
  p.kv = cur.take((uint64_t)v->n_layers * 2 * B * H * tokens * hd * eb);
  p.off_state = align_up(cur.pos);
  p.z = cur.take((uint64_t)B * d * eb);
  p.counter = cur.take(sizeof(int));
  p.rope = cur.take((uint64_t)tokens * (hd / 2) * 2 * sizeof(float));
  p.tok = cur.take((uint64_t)B * v->steps * sizeof(int));
  p.off_scratch = align_up(cur.pos);
  p.state_bytes = p.off_scratch - p.off_state;
  p.x = cur.take((uint64_t)B * d * 4);
  p.a = cur.take((uint64_t)B * d * eb);
  p.part = cur.take(layer_part_bytes(&c, B));
  p.q = cur.take((uint64_t)B * d * 4);
  p.o = cur.take((uint64_t)B * d * eb);
  p.hid = cur.take((uint64_t)B * F * eb);
  p.apart = cur.take((uint64_t)B * H * p.nsplit * (hd + 2) * 4);
  p.amv = cur.take((uint64_t)p.head_tiles * B * 4);
  p.ami = cur.take((uint64_t)p.head_tiles * B * 4);
  p.total = align_up(cur.pos);
  p.scratch_bytes = p.total - p.off_scratch;
  return p;
}

// prefill scratch: bs sequences of P tokens at a time (bs * P <= 65536 rows)
struct VPrePlan {
  int64_t bs = 1;
  Region x, a, part, q, o, hid;
  uint64_t total = 0;
};

VPrePlan plan_vprefill(const photon_vanilla_config* v, int64_t B, int64_t P) {
  VPrePlan p;
  const photon_config c = vanilla_as_config(v);
  const int64_t d = v->d_model, F = (int64_t)v->mlp_mult * d;
  const uint64_t eb = elem_bytes(&c);
  p.bs = std::max<int64_t>(1, std::min<int64_t>(B, kPrefillRows / std::max<int64_t>(1, P)));
  const int64_t R = p.bs * P;
  uint64_t part = 0;
  for (int64_t bs : {p.bs, B % p.bs})
    if (bs) part = std::max(part, layer_part_bytes(&c, bs * P));
  Cursor cur;
  p.x = cur.take((uint64_t)R * d * 4);
  p.a = cur.take((uint64_t)R * d * eb);
  p.part = cur.take(part);
  p.q = cur.take((uint64_t)R * d * 4);
  p.o = cur.take((uint64_t)R * d * eb);
  p.hid = cur.take((uint64_t)R * F * eb);
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
  // flat baseline context (photon_vanilla_open): cfg mirrors vcfg's widths
  bool vanilla = false;
  photon_vanilla_config vcfg{};
  StackW vlayers;
  VPlan vplan;
  const unsigned char* wdec = nullptr;
  const unsigned char* wpre = nullptr;
  std::vector<TensorDesc> tensors;
  const void* E = nullptr;
  // W_ch[l], W_cv[l] for l = 1 .. L; enc[l] for l = 1 .. L-1; dec[l] for
  // l = 0 .. L-1
  const void* W_ch[PHOTON_MAX_LEVELS + 1] = {};
  const void* W_cv[PHOTON_MAX_LEVELS + 1] = {};
  const void* W_out = nullptr;
  StackW top;
  StackW enc[PHOTON_MAX_LEVELS], dec[PHOTON_MAX_LEVELS];
  // decode state
  bool prefilled = false;
  int mode = 0;
  int64_t B = 0, max_tokens = 0, top_len = 0, tokens = 0, prompt_tokens = 0;
  // ragged prompt: tail_r = prompt_len mod S tokens open the next chunk as
  // given tokens; pending until that chunk is decoded
  int tail_r = 0;
  bool tail_pending = false;
  // RecGen: the workspace's A-hat buffers hold the decoders' outputs for
  // the next chunk (each chunk computes them for the one after it); false
  // after a prefill or a rewind, when the next chunk computes them first
  bool ahat_ready = false;
  unsigned char* ws = nullptr;
  WsPlan plan;
  Tracer tr;
  // sampling decode (photon_set_sampling): caller-owned workspace holding
  // one token step's logits and the chunk's log-likelihoods
  bool sampling = false;
  photon_sampling samp{};
  unsigned char* sws = nullptr;
  uint64_t sws_bytes = 0;
  // one decode chunk captured as HIP graphs, replayed for every chunk: each
  // graph is one chain of kernels (the runtime replays a chain from packets
  // it recorded at instantiation, a few tenths of a microsecond of host time
  // per kernel, while a graph with parallel branches is submitted kernel by
  // kernel at several microseconds each); RecGen's two branches are two
  // graphs on two streams, ordered by events.  Slots: the chunk's prefix
  // (or the whole chunk: HierGen, the flat baseline), the token branch, the
  // top branch.
  bool use_graph = true;
  // GEMMs enqueued meanwhile prefer their 8-wave tiles (WideGemms)
  bool wide = false;
  hipGraphExec_t graph[3] = {nullptr, nullptr, nullptr};
  hipStream_t cap[2] = {nullptr, nullptr};
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
  void drop_graphs() {
    for (auto& g : graph)
      if (g) {
        (void)hipGraphExecDestroy(g);
        g = nullptr;
      }
  }
  ~photon_ctx() {
    drop_graphs();
    for (auto s : cap)
      if (s) (void)hipStreamDestroy(s);
    if (ev_fork) (void)hipEventDestroy(ev_fork);
    if (ev_join) (void)hipEventDestroy(ev_join);
  }
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
  const Levels lv = levels(&c->cfg);
  c->E = tensor_ptr(c, "E");
  c->W_out = tensor_ptr(c, "W_out");
  bind_stack(c, c->top, "top", c->cfg.n_top);
  for (int l = 1; l <= lv.L; ++l) {
    c->W_ch[l] = tensor_ptr(c, lname("W_ch", l));
    c->W_cv[l] = tensor_ptr(c, lname("W_cv", l));
    bind_stack(c, c->dec[l - 1], lname("dec", l - 1).c_str(), lv.dec[l - 1]);
    if (l < lv.L) bind_stack(c, c->enc[l], lname("enc", l).c_str(), lv.enc[l]);
  }
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

// Sampling workspace: one token step's logits [B*K1][V] fp32, then the
// chunk's log-likelihoods [B][S] fp32.
uint64_t sampling_lp_off(const photon_config& cf, int64_t B) {
  return align_up((uint64_t)B * levels(&cf).K1() * cf.vocab * 4);
}
uint64_t sampling_bytes(const photon_config& cf, int64_t B) {
  return sampling_lp_off(cf, B) + align_up((uint64_t)B * levels(&cf).S() * 4);
}
photon_status check_sampling(const photon_sampling* sp, int vocab) {
  if (!(sp->temperature >= 1e-4f && sp->temperature <= 1e4f))
    return fail(PHOTON_EINVAL, "temperature %g must lie in [1e-4, 1e4]", (double)sp->temperature);
  if (sp->top_k < 0) return fail(PHOTON_EINVAL, "top_k %d must be >= 0", sp->top_k);
  if (!sample_supported(vocab)) return fail(PHOTON_EUNSUPPORTED, "sampling supports vocabularies up to 65536 (got %d)", vocab);
  return ok();
}

// Launch `f` (returning hipError_t); when class `cls` is traced, the kernel
// dispatches of `f` record a start event (first kernel) and a stop event
// (last kernel) themselves, and the launch keeps its algorithmic bytes and
// flops.
template <class F>
photon_status traced(photon_ctx* c, int cls, double bytes, double flops, hipStream_t st, const char* what, F&& f) {
  const bool on = (c->tr.mask >> cls) & 1u;
  hipEvent_t a = nullptr, b = nullptr;
  if (on) {
    HIP_TRY(c->tr.get(&a));
    HIP_TRY(c->tr.get(&b));
    launch_events() = LaunchEvents{a, b};
  }
  const hipError_t e = f();
  const bool launched = launch_events().start == nullptr;
  launch_events() = LaunchEvents{};
  if (e != hipSuccess) return fail(PHOTON_EHIP, "%s: %s", what, hipGetErrorString(e));
  if (on) {
    if (!launched) return fail(PHOTON_EHIP, "%s: traced operation launched no kernel", what);
    c->tr.recs.push_back({cls, a, b, bytes, flops});
  }
  return PHOTON_OK;
}

// Algorithmic bytes of one GEMM launch: W and A read once, the fp32 result
// written once (read too for a residual update; bf16 after GELU), the head
// its token ids (and logits when asked).  K slabs and the head's per-tile
// argmax partials are choices of this implementation and are not counted.
double gemm_bytes(const GemmCall& g) {
  const double eb = g.dtype ? 2 : 4;
  double b = (double)g.N * g.K * eb + (double)g.M * g.K * eb;
  switch (g.epi) {
    case EPI_STORE: b += (double)g.M * g.N * 4; break;
    case EPI_ADD: b += 2.0 * g.M * g.N * 4; break;
    case EPI_GELU: b += (double)g.M * g.N * eb; break;
    default:
      b += (double)g.M * 4;
      if (g.C) b += (double)g.M * g.N * 4;
  }
  return b;
}

photon_status run_gemm(photon_ctx* c, int cls, GemmCall g, hipStream_t st) {
  g.wide = c->wide;
  return traced(c, cls, gemm_bytes(g), 2.0 * g.M * g.N * g.K, st, "gemm", [&] { return launch_gemm(g, st); });
}

// While one is alive, the context's GEMMs prefer their 8-wave tiles: the
// decode chunk's top stack and the decoders above the token decoder, its
// critical path (the token decoder keeps the tiles that leave more of each
// CU to the top branch running beside it).  Both modes set it on the same
// GEMMs, so their top steps stay the same kernels.
struct WideGemms {
  photon_ctx* c;
  bool prev;
  explicit WideGemms(photon_ctx* c_) : c(c_), prev(c_->wide) { c->wide = true; }
  ~WideGemms() { c->wide = prev; }
};

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
  float* x;       // residual stream, fp32 [M][d]
  void* a;        // normalized GEMM operand [M][d]
  float* part;    // K-slab partials of the STORE GEMMs
  float* q;       // rotated queries, fp32 [M][d]
  void* o;        // attention output [M][d]
  void* hid;      // MLP hidden [M][F]
  float* apart;   // split-key attention partials
};

struct StackRun {
  int M, rows_per_seq, G;
  KvTarget kv;
  int pos_add; const int* pos_dev; int pos_mul;
  const float* rope;
  AttnKind kind;
  int Q, L_host; const int* L_dev; int L_mul, L_add; int nsplit;
  int L_acct;  // keys visible to the last query (host mirror, for accounting)
  // stack output round(norm(x; gf)) for rows i < out_rows taken from input
  // row i*in_stride + in_off
  void* out; int out_rows; int64_t in_stride, in_off;
};

// the producer's result read once (not its K slabs), residual and stream
double rows_epi_bytes(const RowsEpi& e, int eb) {
  double b = (double)e.R * e.d * 4 * (1 + (e.resid ? 1 : 0) + (e.x_out ? 1 : 0));
  if (e.ids) b += (double)e.R * (e.d * eb + 4);
  if (e.a_out) b += (double)e.R * e.d * eb + e.d * 4.0;
  return b;
}

photon_status rows_epi(photon_ctx* c, const RowsEpi& e, hipStream_t st) {
  return traced(c, PHOTON_K_NORM, rows_epi_bytes(e, elem_bytes(&c->cfg)), 6.0 * e.R * e.d, st, "rows_epilogue",
                [&] { return launch_rows_epilogue(c->cfg.dtype, e, st); });
}

// STORE GEMM into `part` (K slabs allowed); *ks receives the slab count.
photon_status gemm_slabs(photon_ctx* c, int cls, const void* A, int64_t lda, const void* W, int M, int N, int K,
                         float* part, int* ks, hipStream_t st) {
  GemmCall g{};
  g.dtype = c->cfg.dtype; g.A = A; g.lda = lda; g.W = W; g.M = M; g.N = N; g.K = K;
  g.epi = EPI_STORE; g.C = part; g.ldc = N; g.allow_split = 1;
  *ks = gemm_splits(g.dtype, M, N, K, c->wide);
  return run_gemm(c, cls, g, st);
}

// The stack input: x = sum of the producer GEMM's slabs (rows of d, row r at
// part + r*d), and its normalized form for the first layer.
photon_status stack_input(photon_ctx* c, const StackW& sw, const float* part, int ks, int R, float* x, void* a,
                          hipStream_t st) {
  RowsEpi e{};
  e.P = part; e.ksplit = ks; e.pstride = (int64_t)R * c->cfg.d_model; e.ldp = c->cfg.d_model;
  e.x_out = x; e.g = sw.layers[0].g1; e.a_out = a; e.a_ld = c->cfg.d_model;
  e.R = R; e.d = c->cfg.d_model; e.row_stride = 1; e.row_off = 0; e.eps = c->cfg.norm_eps;
  return rows_epi(c, e, st);
}

// One Transformer stack.  On entry b.x holds the stack input and b.a its
// normalized form for layer 0; on exit r.out holds the stack output rows.
photon_status run_stack(photon_ctx* c, const StackW& sw, const StackBufs& b, const StackRun& r, hipStream_t st) {
  const photon_config& cf = c->cfg;
  const int dt = cf.dtype, d = cf.d_model, H = cf.n_heads, hd = d / H, F = cf.mlp_mult * d;
  const int eb = elem_bytes(&cf);
  const int L = (int)sw.layers.size();
  for (int l = 0; l < L; ++l) {
    const LayerW& w = sw.layers[l];
    int ks = 1;
    unsigned char* kbase = r.kv.base + (r.kv.per_layer ? (int64_t)l * 2 * r.kv.plane_elems * eb : 0);
    void* Kc = kbase;
    void* Vc = kbase + r.kv.plane_elems * eb;
    // RoPE and the K/V append run inside the attention kernel (the new rows
    // are the last Q keys of every group) for the chunk-confined decoders and
    // for decode steps over caches of fewer than 1024 slots or whose
    // workgroups are all resident at once; otherwise the QKV projection
    // rotates q and k and appends K/V in its own epilogue where the kernel
    // supports the shape (prompts, decode steps of 64-512 rows), and else its
    // K slabs go to a RoPE + append launch of their own
    const bool fuse = r.rows_per_seq == r.Q &&
                      (r.kind == ATT_CHUNK ||
                       (r.kind == ATT_DECODE && attn_decode_rope_inside(r.G, H, (int)r.kv.cap, r.nsplit)));
    GemmCall gq{};
    gq.dtype = dt; gq.A = b.a; gq.lda = d; gq.W = w.Wqkv; gq.M = r.M; gq.N = 3 * d; gq.K = d;
    RopeKvCall rq{dt, nullptr, 1, 0, r.M, d, H, hd, b.q, Kc, Vc, r.kv.seq_stride, r.kv.cap,
                  r.rows_per_seq, r.kv.seq0, r.pos_add, r.pos_dev, r.pos_mul, r.rope};
    const bool qkv_rope = !fuse && r.kind != ATT_CHUNK && gemm_qkv_rope_supported(gq, rq);
    if (qkv_rope) {
      // W and the operand rows read once, q (fp32) and K, V written once
      const double qb = (double)gq.N * d * eb + (double)r.M * d * eb + (double)r.M * d * (4 + 2.0 * eb);
      PH_TRY(traced(c, PHOTON_K_GEMM_QKV, qb, 2.0 * r.M * gq.N * d, st, "gemm",
                    [&] { return launch_gemm_qkv_rope(gq, rq, st); }));
    } else {
      PH_TRY(gemm_slabs(c, PHOTON_K_GEMM_QKV, b.a, d, w.Wqkv, r.M, 3 * d, d, b.part, &ks, st));
    }
    if (!fuse && !qkv_rope) {
      RopeKvCall rc{dt, b.part, ks, (int64_t)r.M * 3 * d, r.M, d, H, hd, b.q, Kc, Vc, r.kv.seq_stride, r.kv.cap,
                    r.rows_per_seq, r.kv.seq0, r.pos_add, r.pos_dev, r.pos_mul, r.rope};
      PH_TRY(traced(c, PHOTON_K_ROPE_KV, (double)r.M * d * (12.0 + 4 + 2 * eb), 6.0 * r.M * d, st, "rope_kv",
                    [&] { return launch_rope_kv(rc, st); }));
    }
    AttnCall ac{dt, r.G, r.Q, H, hd, b.q, d, Kc, Vc, r.kv.seq_stride, r.kv.cap, r.kv.seq0,
                r.L_host, r.L_dev, r.L_mul, r.L_add, b.o, d, b.apart, r.nsplit};
    if (fuse) {
      ac.qkv = b.part; ac.ksplit = ks; ac.pstride = (int64_t)r.M * 3 * d; ac.d = d;
      ac.rope = r.rope; ac.pos_add = r.pos_add; ac.pos_dev = r.pos_dev; ac.pos_mul = r.pos_mul;
    }
    // K and V of every cached key read once, output written, and: q read
    // (separate RoPE launch), or the new rows' q, k, v read and their K, V
    // written (fused).  The split partials and the QKV GEMM's K slabs are
    // not counted.
    const double abytes = fuse ? (double)r.G * H * (r.L_acct - r.Q) * hd * eb * 2 + (double)r.M * d * (12 + 3 * eb)
                               : (double)r.G * H * r.L_acct * hd * eb * 2 + (double)r.M * d * (4 + eb);
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
    PH_TRY(gemm_slabs(c, PHOTON_K_GEMM_O, b.o, d, w.Wo, r.M, d, d, b.part, &ks, st));
    {
      RowsEpi e{};
      e.P = b.part; e.ksplit = ks; e.pstride = (int64_t)r.M * d; e.ldp = d;
      e.resid = b.x; e.x_out = b.x; e.g = w.g2; e.a_out = b.a; e.a_ld = d;
      e.R = r.M; e.d = d; e.row_stride = 1; e.row_off = 0; e.eps = cf.norm_eps;
      PH_TRY(rows_epi(c, e, st));
    }
    GemmCall g{};
    g.dtype = dt; g.A = b.a; g.lda = d; g.W = w.W1; g.M = r.M; g.N = F; g.K = d;
    g.epi = EPI_GELU; g.Cb = b.hid; g.ldc = F;
    PH_TRY(run_gemm(c, PHOTON_K_GEMM_UP, g, st));
    PH_TRY(gemm_slabs(c, PHOTON_K_GEMM_DOWN, b.hid, F, w.W2, r.M, d, F, b.part, &ks, st));
    {
      // residual add, then the next layer's first norm (or the final norm)
      const bool last = l + 1 == L;
      RowsEpi e{};
      e.P = b.part; e.ksplit = ks; e.pstride = (int64_t)r.M * d; e.ldp = d;
      e.resid = b.x; e.x_out = last ? nullptr : b.x;
      e.g = last ? sw.gf : sw.layers[l + 1].g1;
      e.a_out = last ? r.out : b.a; e.a_ld = d;
      e.R = last ? r.out_rows : r.M; e.d = d;
      e.row_stride = last ? r.in_stride : 1; e.row_off = last ? r.in_off : 0;
      e.eps = cf.norm_eps;
      PH_TRY(rows_epi(c, e, st));
    }
  }
  return ok();
}

// Every GEMM shape of prefill (slices of bs sequences, nl[l] level-l states
// each) and of the decode chunk, checked before anything is enqueued; and
// HierGen's encoder steps, which run S/span(l) queries per sequence through
// the global attention (1, 2 or 4).
photon_status check_gemms(const photon_config* c, int64_t B, const PrePlan& pp, int mode) {
  const int dt = c->dtype, d = c->d_model, F = c->mlp_mult * d, V = c->vocab;
  const Levels lv = levels(c);
  const int L = lv.L;
  struct S3 { int64_t M; int N, K; };
  std::vector<S3> shapes = {{B * lv.K1(), lv.C[1] * d, d}, {B * lv.K1(), V, d}, {B, d, lv.C[L] * d}};
  std::vector<int64_t> rows = {B};
  for (int l = 1; l <= L; ++l) {
    shapes.push_back({pp.bs * pp.nl[l], d, lv.C[l] * d});          // prefill chunkers
    rows.push_back(pp.bs * pp.nl[l]);
    if (l >= 2) shapes.push_back({B * lv.per_chunk(l), lv.C[l] * d, d});   // converters above level 1
    if (l < L) {
      rows.push_back(B * lv.per_chunk(l));
      if (mode == PHOTON_HIERGEN) {
        shapes.push_back({B * lv.per_chunk(l), d, lv.C[l] * d});  // re-encoding chunkers
        const int64_t q = lv.per_chunk(l);
        if (q != 1 && q != 2 && q != 4)
          return fail(PHOTON_EUNSUPPORTED, "HierGen's level-%d encoder step would take %lld queries per sequence "
                      "(1, 2 or 4 supported)", l, (long long)q);
      }
    }
  }
  for (int64_t M : rows) {
    shapes.push_back({M, 3 * d, d});
    shapes.push_back({M, d, d});
    shapes.push_back({M, F, d});
    shapes.push_back({M, d, F});
  }
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
  const int S = (int)levels(cfg).S();
  if (prompt_len < S)
    return fail(PHOTON_ESHAPE, "prompt_len %d must hold at least one chunk of S = %d tokens", prompt_len, S);
  *out = plan_prefill(cfg, batch, prompt_len / S * S, mode).total;   // whole chunks only
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
  if (c->vanilla) return fail(PHOTON_ESTATE, "a flat-baseline context has no prefill-only weights");
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
  if (c->vanilla) return fail(PHOTON_ESTATE, "a flat-baseline context (use photon_vanilla_prefill)");
  if (mode != PHOTON_RECGEN && mode != PHOTON_HIERGEN) return fail(PHOTON_EINVAL, "bad mode %d", mode);
  if (!d_workspace || !d_scratch || !d_prompt) return fail(PHOTON_EINVAL, "NULL device pointer");
  if (((uintptr_t)d_workspace | (uintptr_t)d_scratch) % kAlign)
    return fail(PHOTON_EINVAL, "workspace and scratch must be 256-byte aligned");
  if (!c->wpre) return fail(PHOTON_ESTATE, "prefill needs the prefill-only weights, which were released");
  const photon_config& cf = c->cfg;
  const Levels lv = levels(&cf);
  const int L = lv.L, S = (int)lv.S();
  if (batch < 1) return fail(PHOTON_ESHAPE, "batch must be >= 1");
  if (prompt_len < S)
    return fail(PHOTON_ESHAPE, "prompt_len %d must hold at least one chunk of S = %d tokens", prompt_len, S);
  if (max_tokens < prompt_len) return fail(PHOTON_ECAPACITY, "max_tokens %lld < prompt_len %d", (long long)max_tokens, prompt_len);
  const WsPlan wp = plan_workspace(&cf, batch, max_tokens, mode);
  if (ws_bytes < wp.total)
    return fail(PHOTON_ECAPACITY, "workspace holds %llu bytes, needs %llu", (unsigned long long)ws_bytes,
                (unsigned long long)wp.total);
  // whole chunks are encoded; a ragged tail opens the next chunk
  const int P_enc = prompt_len / S * S, tail_r = prompt_len - P_enc;
  const PrePlan pp = plan_prefill(&cf, batch, P_enc, mode);
  if (scratch_bytes < pp.total)
    return fail(PHOTON_ECAPACITY, "prefill scratch holds %llu bytes, needs %llu", (unsigned long long)scratch_bytes,
                (unsigned long long)pp.total);
  {
    photon_status s = check_gemms(&cf, batch, pp, mode);
    if (s) return s;
  }
  hipStream_t st = (hipStream_t)stream;
  const int dt = cf.dtype, d = cf.d_model, H = cf.n_heads, hd = d / H;
  const int eb = elem_bytes(&cf);
  unsigned char* ws = (unsigned char*)d_workspace;
  unsigned char* sc = (unsigned char*)d_scratch;
  c->prefilled = false;
  c->drop_graphs();
  c->ws = ws;
  c->plan = wp;
  c->mode = mode;
  c->B = batch;
  c->max_tokens = max_tokens;

  float* rope_ws = (float*)(ws + wp.rope.off);
  float* rope1 = (float*)(sc + pp.rope1.off);
  HIP_TRY(launch_rope_table(rope_ws, (int)wp.rope_pos, hd, cf.rope_theta, st));
  HIP_TRY(launch_rope_table(rope1, (int)std::max<int64_t>(pp.n1, 1), hd, cf.rope_theta, st));

  const int64_t n = pp.n;
  StackBufs bufs{(float*)(sc + pp.x.off), sc + pp.a.off, (float*)(sc + pp.part.off), (float*)(sc + pp.q.off),
                 sc + pp.o.off, sc + pp.hid.off, nullptr};
  for (int64_t b0 = 0; b0 < batch; b0 += pp.bs) {
    const int bs = (int)std::min<int64_t>(pp.bs, batch - b0);
    // embedding rows of bs*P tokens == Chunker^1 input [bs*n1][C1*d]
    PH_TRY(traced(c, PHOTON_K_EMBED, (double)bs * P_enc * (4 + 2.0 * d * eb), 0, st, "embed_gather", [&] {
      return launch_embed_gather_rows(dt, d_prompt + b0 * prompt_len, bs, P_enc, prompt_len, c->E, d, cf.vocab,
                                      sc + pp.e.off, st);
    }));
    // every level below the top: Chunker^l over groups of C_l states of the
    // level beneath (the embeddings for l = 1), then the level-l encoder;
    // its output replaces its input in buffer A
    int ks = 1;
    const unsigned char* in = sc + pp.e.off;
    for (int l = 1; l < L; ++l) {
      const int64_t nl = pp.nl[l];
      const int rows = (int)(bs * nl);
      PH_TRY(gemm_slabs(c, PHOTON_K_GEMM_CHUNK, in, (int64_t)lv.C[l] * d, c->W_ch[l], rows, d, lv.C[l] * d,
                        bufs.part, &ks, st));
      PH_TRY(stack_input(c, c->enc[l], bufs.part, ks, rows, bufs.x, bufs.a, st));
      StackRun r{};
      r.M = rows; r.rows_per_seq = (int)nl; r.G = bs;
      if (mode == PHOTON_HIERGEN) {
        const int64_t cap = wp.low_caps[l];
        r.kv = KvTarget{ws + wp.lowl[l].off, (int64_t)batch * H * cap * hd, true, (int64_t)H * cap * hd, (int)cap,
                        (int)b0};
      } else {
        r.kv = KvTarget{sc + pp.kv1.off, (int64_t)pp.bs * H * nl * hd, false, (int64_t)H * nl * hd, (int)nl, 0};
      }
      r.pos_add = 0; r.pos_dev = nullptr; r.pos_mul = 0; r.rope = rope1;
      r.kind = ATT_PREFILL; r.Q = (int)nl; r.L_host = (int)nl; r.nsplit = 1; r.L_acct = (int)nl;
      r.out = sc + pp.A1.off; r.out_rows = rows; r.in_stride = 1; r.in_off = 0;
      PH_TRY(run_stack(c, c->enc[l], bufs, r, st));
      in = sc + pp.A1.off;
    }
    // Chunker^L over groups of C_L states of level L-1
    PH_TRY(gemm_slabs(c, PHOTON_K_GEMM_CHUNK, in, (int64_t)lv.C[L] * d, c->W_ch[L], (int)(bs * n), d, lv.C[L] * d,
                      bufs.part, &ks, st));
    PH_TRY(stack_input(c, c->top, bufs.part, ks, (int)(bs * n), bufs.x, bufs.a, st));
    StackRun t{};
    t.M = (int)(bs * n); t.rows_per_seq = (int)n; t.G = bs;
    t.kv = KvTarget{ws + wp.top_kv.off, (int64_t)batch * H * wp.top_cap * hd, true, (int64_t)H * wp.top_cap * hd,
                    (int)wp.top_cap, (int)b0};
    t.pos_add = 0; t.pos_dev = nullptr; t.pos_mul = 0; t.rope = rope_ws;
    t.kind = ATT_PREFILL; t.Q = (int)n; t.L_host = (int)n; t.nsplit = 1; t.L_acct = (int)n;
    // final norm only for the last top state of each sequence: h_{n-1}
    t.out = ws + wp.h.off + (uint64_t)b0 * d * eb; t.out_rows = bs; t.in_stride = n; t.in_off = n - 1;
    PH_TRY(run_stack(c, c->top, bufs, t, st));
  }
  HIP_TRY(launch_set_int((int*)(ws + wp.counter.off), (int)n, st));
  if (tail_r)
    HIP_TRY(launch_copy_ids((int*)(ws + wp.tail.off), S, d_prompt + P_enc, prompt_len, batch, tail_r, cf.vocab, st));
  c->top_len = n;
  c->tokens = prompt_len;
  c->prompt_tokens = prompt_len;
  c->tail_r = tail_r;
  c->tail_pending = tail_r > 0;
  c->ahat_ready = false;
  c->prefilled = true;
  return ok();
}

// The chunk-confined decoders above the token decoder for the chunk after
// top state h: Converter^L expands h into C_L conditioning vectors and the
// level-(L-1) decoder gives A-hat (Ahat[L-1]); for l = L-1 .. 2 every level-l
// vector is expanded by Converter^l and the level-(l-1) decoder over its own
// C_l positions (attention confined to the group, positions 0 .. C_l-1, no
// cache kept), down to the level-1 vectors (Ahat[1]).  Only h is read.
photon_status enqueue_decoders(photon_ctx* c, const StackBufs& bufs, hipStream_t st) {
  WideGemms wide(c);
  const photon_config& cf = c->cfg;
  const Levels lv = levels(&cf);
  const WsPlan& wp = c->plan;
  unsigned char* ws = c->ws;
  const int d = cf.d_model, H = cf.n_heads, hd = d / H, B = (int)c->B;
  const float* rope = (const float*)(ws + wp.rope.off);
  int ks = 1;
  auto expand = [&](int l, const void* in, int M, void* out) -> photon_status {
    const int C = lv.C[l];
    PH_TRY(gemm_slabs(c, PHOTON_K_GEMM_CONV, in, d, c->W_cv[l], M, C * d, d, bufs.part, &ks, st));
    PH_TRY(stack_input(c, c->dec[l - 1], bufs.part, ks, M * C, bufs.x, bufs.a, st));
    StackRun r{};
    r.M = M * C; r.rows_per_seq = C; r.G = M;
    r.kv = KvTarget{ws + wp.kv1tmp.off, (int64_t)M * H * C * hd, false, (int64_t)H * C * hd, C, 0};
    r.pos_add = 0; r.rope = rope;
    r.kind = ATT_CHUNK; r.Q = C; r.L_host = C; r.nsplit = 1; r.L_acct = C;
    r.out = out; r.out_rows = M * C; r.in_stride = 1; r.in_off = 0;
    return run_stack(c, c->dec[l - 1], bufs, r, st);
  };
  PH_TRY(expand(lv.L, ws + wp.h.off, B, ws + wp.Ahat[lv.L - 1].off));
  for (int l = lv.L - 1; l >= 2; --l)
    PH_TRY(expand(l, ws + wp.Ahat[l].off, (int)(B * lv.per_chunk(l)), ws + wp.Ahat[l - 1].off));
  return ok();
}

// Enqueue one decode chunk.  The token decoder runs on `st`; with RecGen
// and st_top != st the top branch forks onto st_top once the token branch
// has its conditioning vectors, and joins back before the chunk ends.
// Everything reads positions from the device counter, so the same sequence
// serves every chunk.
//
// HierGen: the decoders of the chunk, the token steps, the bottom-up
// re-encoding and the top step, in that order.  RecGen: the decoders above
// the token decoder depend only on the previous top output, so each chunk's
// top branch ends with them for the next chunk (feedback Chunker^L(A-hat_i),
// top step i -> h_i, decoders -> A-hat_{i+1}), beside the token steps of
// chunk i; the chunk after a prefill or a rewind runs them first
// (`ahat_ready`, photon_decode_chunk_lp).  The results are those of the
// sequential order: the two branches share no buffer (A-hat_i is consumed by
// Converter^1 before the fork and by the feedback GEMM before the decoders
// of the top branch overwrite it).
// `parts` selects what is enqueued: the prefix (HierGen's decoders, then
// Converter^1 and the first token step's input), the token branch, the top
// branch, the position update; the fork and join events only when all four
// are (the graph replay orders its separately captured parts itself).
enum { kPartPre = 1, kPartTok = 2, kPartTop = 4, kPartEnd = 8, kPartAll = 15 };
photon_status enqueue_chunk(photon_ctx* c, float* d_logits, hipStream_t st, hipStream_t st_top, int given_r = 0,
                            int parts = kPartAll) {
  const photon_config& cf = c->cfg;
  const Levels lv = levels(&cf);
  const int L = lv.L, C1 = lv.C[1], CL = lv.C[L], K1 = (int)lv.K1();
  const WsPlan& wp = c->plan;
  unsigned char* ws = c->ws;
  const int dt = cf.dtype, d = cf.d_model, H = cf.n_heads, hd = d / H, V = cf.vocab;
  const int B = (int)c->B, MB = B * K1;
  const int eb = elem_bytes(&cf);
  const bool recgen = c->mode == PHOTON_RECGEN;
  int* counter = (int*)(ws + wp.counter.off);
  const float* rope = (const float*)(ws + wp.rope.off);
  void* h = ws + wp.h.off;
  void* Ahat_top = ws + wp.Ahat[L - 1].off;   // A-hat_i: the level-(L-1) decoder outputs
  int* tok = (int*)(ws + wp.tok.off);
  float* c0 = (float*)(ws + wp.c0.off);
  StackBufs sb{(float*)(ws + wp.xB.off), ws + wp.aB.off, (float*)(ws + wp.partB.off), (float*)(ws + wp.qB.off),
               ws + wp.oB.off, ws + wp.hidB.off, nullptr};
  StackBufs sa{(float*)(ws + wp.xA.off), ws + wp.aA.off, (float*)(ws + wp.partA.off), (float*)(ws + wp.qA.off),
               ws + wp.oA.off, ws + wp.hidA.off, (float*)(ws + wp.apartA.off)};
  int ks = 1;

  if ((parts & kPartPre) && !recgen) PH_TRY(enqueue_decoders(c, sb, st));
  // Converter^1 (all C1 conditioning vectors of every level-1 position) and
  // the first token step's input
  if (parts & kPartPre) {
    GemmCall g{};
    g.dtype = dt; g.A = ws + wp.Ahat[1].off; g.lda = d; g.W = c->W_cv[1]; g.M = MB; g.N = C1 * d; g.K = d;
    g.epi = EPI_STORE; g.C = c0; g.ldc = (int64_t)C1 * d;
    PH_TRY(run_gemm(c, PHOTON_K_GEMM_CONV, g, st));
    RowsEpi e{};   // step 0 input: x = c_0, no token yet
    e.P = c0; e.ksplit = 1; e.pstride = 0; e.ldp = (int64_t)C1 * d;
    e.x_out = sb.x; e.g = c->dec[0].layers[0].g1; e.a_out = sb.a; e.a_ld = d;
    e.R = MB; e.d = d; e.row_stride = 1; e.row_off = 0; e.eps = cf.norm_eps;
    PH_TRY(rows_epi(c, e, st));
  }
  const bool fork = recgen && st_top != st && parts == kPartAll;
  if (fork) {
    HIP_TRY(hipEventRecord(c->ev_fork, st));
    HIP_TRY(hipStreamWaitEvent(st_top, c->ev_fork, 0));
  }
  // token branch: C1 sequential token-decoder steps
  for (int j = 0; j < ((parts & kPartTok) ? C1 : 0); ++j) {
    StackRun r{};
    r.M = MB; r.rows_per_seq = 1; r.G = MB;
    r.kv = KvTarget{ws + wp.dec_kv.off, (int64_t)MB * H * C1 * hd, true, (int64_t)H * C1 * hd, C1, 0};
    r.pos_add = j; r.rope = rope;
    r.kind = ATT_CHUNK; r.Q = 1; r.L_host = j + 1; r.nsplit = 1; r.L_acct = j + 1;
    r.out = ws + wp.zB.off; r.out_rows = MB; r.in_stride = 1; r.in_off = 0;
    PH_TRY(run_stack(c, c->dec[0], sb, r, st));
    GemmCall g{};
    g.dtype = dt; g.A = ws + wp.zB.off; g.lda = d; g.W = c->W_out; g.M = MB; g.N = V; g.K = d;
    g.epi = EPI_ARGMAX;
    // sampling reads the logits back: the caller's buffer when it asked for
    // them, else the sampling workspace
    g.C = d_logits ? d_logits + (int64_t)j * V : c->sampling ? (float*)c->sws : nullptr;
    g.ldc = d_logits ? (int64_t)C1 * V : V;
    g.amax_val = (float*)(ws + wp.amv.off); g.amax_idx = (int*)(ws + wp.ami.off);
    PH_TRY(run_gemm(c, PHOTON_K_GEMM_HEAD, g, st));
    // rows m = b*K1 + k: sequence b, level-1 position k (token k*C1 + j)
    if (c->sampling) {
      // the sampler's id takes the place of the argmax tiles (one tile)
      SampleCall sc{g.C, g.ldc, MB, V, c->samp.temperature, c->samp.top_k, (uint32_t)c->samp.seed,
                    (uint32_t)(c->samp.seed >> 32), nullptr, nullptr, counter, C1, K1, j,
                    g.amax_idx, g.amax_val, (float*)(c->sws + sampling_lp_off(cf, B)),
                    (const int*)(ws + wp.tail.off), given_r};
      PH_TRY(traced(c, PHOTON_K_SAMPLE, (double)MB * V * 4 + (double)MB * 12, 0, st, "sample",
                    [&] { return launch_sample(sc, st); }));
    }
    const bool next = j + 1 < C1;
    ArgmaxNext an{g.amax_val, g.amax_idx, c->sampling ? 1 : wp.head_tiles, MB, C1, K1, j, tok,
                  c0, (int64_t)C1 * d, c->E, next ? sb.x : nullptr, sb.a, c->dec[0].layers[0].g1, d, cf.norm_eps,
                  (const int*)(ws + wp.tail.off), given_r, V};
    // the next step's input (conditioning row + embedding in, stream and its
    // norm out); the token ids are counted with the head
    const double nb = next ? (double)MB * d * (8 + 2 * eb) : 0;
    PH_TRY(traced(c, PHOTON_K_ARGMAX, nb, 0, st, "argmax_next", [&] { return launch_argmax_next(dt, an, st); }));
  }
  // top branch (RecGen: independent of the tokens, so it may run beside the
  // token branch on its own stream; its counter update closes it)
  const hipStream_t stt = fork ? st_top : st;
  if (!(parts & kPartTop)) {
    // not enqueued here
  } else if (recgen) {
    // feedback: u_i = Chunker^L(A-hat_i), nothing re-encoded
    WideGemms wide(c);
    PH_TRY(gemm_slabs(c, PHOTON_K_GEMM_CHUNK, Ahat_top, (int64_t)CL * d, c->W_ch[L], B, d, CL * d, sa.part, &ks, stt));
    PH_TRY(stack_input(c, c->top, sa.part, ks, B, sa.x, sa.a, stt));
  } else {
    // HierGen: re-encode the chunk's tokens bottom-up, through Chunker^l and
    // one level-l encoder step for l = 1 .. L-1 (the chunk's S/span(l) new
    // level-l positions over the kept level-l cache), then Chunker^L of the
    // encoder summary A_i
    PH_TRY(traced(c, PHOTON_K_EMBED, (double)B * lv.S() * (4 + 2.0 * d * eb), 0, stt, "embed_gather",
                  [&] { return launch_embed_gather(dt, tok, (int64_t)B * lv.S(), c->E, d, V, ws + wp.eA.off, stt); }));
    const void* in = ws + wp.eA.off;
    for (int l = 1; l < L; ++l) {
      const int q = (int)lv.per_chunk(l), M = B * q;
      const int64_t cap = wp.low_caps[l];
      PH_TRY(gemm_slabs(c, PHOTON_K_GEMM_CHUNK, in, (int64_t)lv.C[l] * d, c->W_ch[l], M, d, lv.C[l] * d, sa.part, &ks,
                        stt));
      PH_TRY(stack_input(c, c->enc[l], sa.part, ks, M, sa.x, sa.a, stt));
      StackRun r{};
      r.M = M; r.rows_per_seq = q; r.G = B;
      r.kv = KvTarget{ws + wp.lowl[l].off, (int64_t)B * H * cap * hd, true, (int64_t)H * cap * hd, (int)cap, 0};
      r.pos_add = 0; r.pos_dev = counter; r.pos_mul = q; r.rope = rope;
      r.kind = ATT_DECODE; r.Q = q; r.L_dev = counter; r.L_mul = q; r.L_add = q; r.nsplit = wp.nsplit_low[l];
      r.L_acct = (int)((c->top_len + 1) * q);
      r.out = ws + wp.AA.off; r.out_rows = M; r.in_stride = 1; r.in_off = 0;
      PH_TRY(run_stack(c, c->enc[l], sa, r, stt));
      in = ws + wp.AA.off;
    }
    WideGemms wide(c);
    PH_TRY(gemm_slabs(c, PHOTON_K_GEMM_CHUNK, in, (int64_t)CL * d, c->W_ch[L], B, d, CL * d, sa.part, &ks, stt));
    PH_TRY(stack_input(c, c->top, sa.part, ks, B, sa.x, sa.a, stt));
  }
  if (parts & kPartTop) {
    WideGemms wide(c);
    StackRun r{};
    r.M = B; r.rows_per_seq = 1; r.G = B;
    r.kv = KvTarget{ws + wp.top_kv.off, (int64_t)B * H * wp.top_cap * hd, true, (int64_t)H * wp.top_cap * hd,
                    (int)wp.top_cap, 0};
    r.pos_add = 0; r.pos_dev = counter; r.pos_mul = 1; r.rope = rope;
    r.kind = ATT_DECODE; r.Q = 1; r.L_dev = counter; r.L_mul = 1; r.L_add = 1; r.nsplit = wp.nsplit_top;
    r.L_acct = (int)(c->top_len + 1);
    r.out = h; r.out_rows = B; r.in_stride = 1; r.in_off = 0;
    PH_TRY(run_stack(c, c->top, sa, r, stt));
  }
  // RecGen: the next chunk's decoders from h_i, still in the top branch
  if ((parts & kPartTop) && recgen) PH_TRY(enqueue_decoders(c, sa, stt));
  // the position advances once both branches are done: the sampler of the
  // token branch reads it while the top branch runs
  if (fork) {
    HIP_TRY(hipEventRecord(c->ev_join, st_top));
    HIP_TRY(hipStreamWaitEvent(st, c->ev_join, 0));
  }
  if (parts & kPartEnd) HIP_TRY(launch_add_int(counter, 1, st));
  return ok();
}

// The chunk's token ids (and, when sampling, the log-likelihoods of the
// drawn tokens) into the caller's buffers, on stream st.
static photon_status copy_chunk_outputs(photon_ctx* c, int32_t* d_tokens, float* d_logprobs, hipStream_t st) {
  const int B = (int)c->B, S = (int)levels(&c->cfg).S();
  HIP_TRY(hipMemcpyAsync(d_tokens, c->ws + c->plan.tok.off, (size_t)B * S * sizeof(int), hipMemcpyDeviceToDevice, st));
  if (d_logprobs)
    HIP_TRY(hipMemcpyAsync(d_logprobs, c->sws + sampling_lp_off(c->cfg, B), (size_t)B * S * sizeof(float),
                           hipMemcpyDeviceToDevice, st));
  return ok();
}

// Capture what `enqueue` puts on the context's capture stream as a graph
// and instantiate it into *exec (left null on failure).
extern "C++" template <class F>
photon_status capture_graph(photon_ctx* c, hipGraphExec_t* exec, F&& enqueue) {
  HIP_TRY(hipStreamBeginCapture(c->cap[0], hipStreamCaptureModeRelaxed));
  const photon_status s = enqueue(c->cap[0]);
  hipGraph_t g = nullptr;
  const hipError_t e = hipStreamEndCapture(c->cap[0], &g);
  if (s != PHOTON_OK) {
    if (g) (void)hipGraphDestroy(g);
    return s;
  }
  if (e != hipSuccess) return fail(PHOTON_EHIP, "graph capture: %s", hipGetErrorString(e));
  const hipError_t ie = hipGraphInstantiate(exec, g, nullptr, nullptr, 0);
  (void)hipGraphDestroy(g);
  if (ie != hipSuccess) {
    *exec = nullptr;
    return fail(PHOTON_EHIP, "graph instantiate: %s", hipGetErrorString(ie));
  }
  return ok();
}

photon_status photon_decode_chunk(photon_ctx* c, int32_t* d_tokens, float* d_logits, void* stream) {
  return photon_decode_chunk_lp(c, d_tokens, d_logits, nullptr, stream);
}

photon_status photon_decode_chunk_lp(photon_ctx* c, int32_t* d_tokens, float* d_logits, float* d_logprobs,
                                     void* stream) {
  if (!c) return fail(PHOTON_EINVAL, "ctx is NULL");
  if (c->vanilla) return fail(PHOTON_ESTATE, "a flat-baseline context (use photon_vanilla_decode)");
  if (!d_tokens) return fail(PHOTON_EINVAL, "d_tokens is NULL");
  if (!c->prefilled) return fail(PHOTON_ESTATE, "decode before prefill");
  if (d_logprobs && !c->sampling) return fail(PHOTON_ESTATE, "log-likelihoods need a sampling context");
  const photon_config& cf = c->cfg;
  const int S = (int)levels(&cf).S();
  if ((c->top_len + 1) * S > c->max_tokens)
    return fail(PHOTON_ECAPACITY, "chunk would pass max_tokens %lld", (long long)c->max_tokens);
  if (c->mode == PHOTON_HIERGEN && !c->wpre)
    return fail(PHOTON_ESTATE, "HierGen decoding needs the prefill-only weights, which were released");
  if (c->sampling && c->sws_bytes < sampling_bytes(cf, c->B))
    return fail(PHOTON_ECAPACITY, "sampling workspace holds %llu bytes, batch %lld needs %llu",
                (unsigned long long)c->sws_bytes, (long long)c->B, (unsigned long long)sampling_bytes(cf, c->B));
  hipStream_t st = (hipStream_t)stream;
  if (c->mode == PHOTON_RECGEN && !c->ahat_ready) {
    // after a prefill or a rewind: this chunk's decoders from the current h
    // (afterwards every chunk leaves them ready for the next one)
    const WsPlan& wp = c->plan;
    unsigned char* ws = c->ws;
    const StackBufs sb{(float*)(ws + wp.xB.off), ws + wp.aB.off, (float*)(ws + wp.partB.off),
                       (float*)(ws + wp.qB.off), ws + wp.oB.off, ws + wp.hidB.off, nullptr};
    PH_TRY(enqueue_decoders(c, sb, st));
    c->ahat_ready = true;
  }
  if (c->tail_pending) {
    // the chunk a ragged prompt opened: its first tail_r tokens are given
    // (direct launches; the captured graphs serve the whole chunks)
    PH_TRY(enqueue_chunk(c, d_logits, st, st, c->tail_r));
    PH_TRY(copy_chunk_outputs(c, d_tokens, d_logprobs, st));
  } else if (c->use_graph && !d_logits && c->tr.mask == 0) {
    // RecGen: the prefix and the token branch on `st`, the top branch on a
    // stream of the context, forked after the prefix and joined before the
    // position update (the order enqueue_chunk's events give); HierGen: the
    // whole chunk as one chain
    const bool recgen = c->mode == PHOTON_RECGEN;
    if (!c->graph[0]) {
      for (auto& cs : c->cap)
        if (!cs) HIP_TRY(hipStreamCreateWithFlags(&cs, hipStreamNonBlocking));
      if (!c->ev_fork) HIP_TRY(hipEventCreateWithFlags(&c->ev_fork, hipEventDisableTiming));
      if (!c->ev_join) HIP_TRY(hipEventCreateWithFlags(&c->ev_join, hipEventDisableTiming));
      const int part[3] = {recgen ? (int)kPartPre : (int)kPartAll, kPartTok, kPartTop};
      for (int i = 0; i < (recgen ? 3 : 1); ++i) {
        const photon_status s = capture_graph(c, &c->graph[i], [&](hipStream_t cs) {
          return enqueue_chunk(c, nullptr, cs, cs, 0, part[i]);
        });
        if (s != PHOTON_OK) {
          c->drop_graphs();
          return s;
        }
      }
    }
    HIP_TRY(hipGraphLaunch(c->graph[0], st));
    if (recgen) {
      HIP_TRY(hipEventRecord(c->ev_fork, st));
      HIP_TRY(hipStreamWaitEvent(c->cap[1], c->ev_fork, 0));
      HIP_TRY(hipGraphLaunch(c->graph[2], c->cap[1]));
      HIP_TRY(hipEventRecord(c->ev_join, c->cap[1]));
      HIP_TRY(hipGraphLaunch(c->graph[1], st));
      // the token branch alone writes the chunk's tokens (and the sampler's
      // log-likelihoods): their copies overlap the top branch's tail
      PH_TRY(copy_chunk_outputs(c, d_tokens, d_logprobs, st));
      HIP_TRY(hipStreamWaitEvent(st, c->ev_join, 0));
      HIP_TRY(launch_add_int((int*)(c->ws + c->plan.counter.off), 1, st));
    } else {
      PH_TRY(copy_chunk_outputs(c, d_tokens, d_logprobs, st));
    }
  } else {
    PH_TRY(enqueue_chunk(c, d_logits, st, st));
    PH_TRY(copy_chunk_outputs(c, d_tokens, d_logprobs, st));
  }
  c->top_len += 1;
  c->tokens = c->top_len * S;
  c->tail_pending = false;
  return ok();
}

photon_status photon_consistency(photon_ctx* c, float* d_dist, void* d_ahat, void* d_a, void* stream) {
  if (!c) return fail(PHOTON_EINVAL, "ctx is NULL");
  if (c->vanilla) return fail(PHOTON_ESTATE, "a flat-baseline context has no hierarchy");
  if (!d_dist) return fail(PHOTON_EINVAL, "d_dist is NULL");
  if (!c->prefilled || c->mode != PHOTON_HIERGEN)
    return fail(PHOTON_ESTATE, "the diagnostic needs a HierGen context (RecGen never computes A_i)");
  if (c->tokens <= c->prompt_tokens) return fail(PHOTON_ESTATE, "no chunk decoded yet");
  const photon_config& cf = c->cfg;
  const Levels lv = levels(&cf);
  const int R = (int)c->B * lv.C[lv.L], d = cf.d_model;
  const size_t bytes = (size_t)R * d * elem_bytes(&cf);
  const void* Ahat = c->ws + c->plan.Ahat[lv.L - 1].off;
  const void* A = c->ws + c->plan.AA.off;
  hipStream_t st = (hipStream_t)stream;
  HIP_TRY(launch_cosine_distance(cf.dtype, Ahat, A, R, d, d_dist, st));
  if (d_ahat) HIP_TRY(hipMemcpyAsync(d_ahat, Ahat, bytes, hipMemcpyDeviceToDevice, st));
  if (d_a) HIP_TRY(hipMemcpyAsync(d_a, A, bytes, hipMemcpyDeviceToDevice, st));
  return ok();
}

photon_status photon_sampling_bytes(const photon_config* cfg, int32_t batch, uint64_t* bytes) {
  photon_status s = check_config(cfg);
  if (s) return s;
  if (!bytes) return fail(PHOTON_EINVAL, "bytes is NULL");
  if (batch < 1) return fail(PHOTON_ESHAPE, "batch must be >= 1");
  *bytes = sampling_bytes(*cfg, batch);
  return ok();
}

photon_status photon_set_sampling(photon_ctx* c, const photon_sampling* sp, void* d_ws, uint64_t ws_bytes) {
  if (!c) return fail(PHOTON_EINVAL, "ctx is NULL");
  if (c->vanilla) return fail(PHOTON_ESTATE, "sampling is not offered on a flat-baseline context");
  if (sp) {
    photon_status s = check_sampling(sp, c->cfg.vocab);
    if (s) return s;
    if (!d_ws) return fail(PHOTON_EINVAL, "sampling workspace is NULL");
    if ((uintptr_t)d_ws % kAlign) return fail(PHOTON_EINVAL, "sampling workspace must be 256-byte aligned");
  }
  c->drop_graphs();
  c->sampling = sp != nullptr;
  c->samp = sp ? *sp : photon_sampling{};
  c->sws = sp ? (unsigned char*)d_ws : nullptr;
  c->sws_bytes = sp ? ws_bytes : 0;
  return ok();
}

photon_status photon_sample(int32_t rows, int32_t vocab, const float* d_logits, int64_t ld, const photon_sampling* sp,
                            const int32_t* d_seq, const int32_t* d_pos, int32_t* d_ids, float* d_logprobs,
                            void* stream) {
  if (!sp) return fail(PHOTON_EINVAL, "sampling parameters are NULL");
  photon_status s = check_sampling(sp, vocab);
  if (s) return s;
  if (rows < 1 || vocab < 1 || ld < vocab)
    return fail(PHOTON_ESHAPE, "rows %d, vocab %d, ld %lld: need rows, vocab >= 1 and ld >= vocab", rows, vocab,
                (long long)ld);
  if (!d_logits || !d_seq || !d_pos || !d_ids) return fail(PHOTON_EINVAL, "NULL device pointer");
  SampleCall sc{d_logits, ld, rows, vocab, sp->temperature, sp->top_k, (uint32_t)sp->seed, (uint32_t)(sp->seed >> 32),
                d_seq, d_pos, nullptr, 1, 1, 0, d_ids, nullptr, d_logprobs};
  const hipError_t e = launch_sample(sc, (hipStream_t)stream);
  if (e != hipSuccess) return fail(PHOTON_EHIP, "sample: %s", hipGetErrorString(e));
  return ok();
}

photon_status photon_aggregate(int32_t batch, int32_t group, int32_t n_tok, const int32_t* d_tokens, int64_t tok_ld,
                               const float* d_logprobs, int64_t lp_ld, int32_t span_begin, int32_t span_end,
                               int32_t* d_best, int32_t* d_major, int32_t* d_votes, float* d_scores, void* stream) {
  if (batch < 1 || group < 1 || group > 64 || n_tok < 0)
    return fail(PHOTON_ESHAPE, "batch %d, group %d, n_tok %d: need batch >= 1, 1 <= group <= 64, n_tok >= 0", batch,
                group, n_tok);
  if (span_begin < 0 || span_end < span_begin || tok_ld < span_end || tok_ld < n_tok || lp_ld < n_tok)
    return fail(PHOTON_ESHAPE, "span [%d, %d), n_tok %d must fit rows of %lld tokens and %lld log-likelihoods",
                span_begin, span_end, n_tok, (long long)tok_ld, (long long)lp_ld);
  if (!d_tokens || !d_logprobs || !d_best || !d_major || !d_votes) return fail(PHOTON_EINVAL, "NULL device pointer");
  AggregateCall ac{d_tokens, tok_ld, d_logprobs, lp_ld, batch, group, n_tok, span_begin, span_end,
                   d_best, d_major, d_votes, d_scores};
  const hipError_t e = launch_aggregate(ac, (hipStream_t)stream);
  if (e != hipSuccess) return fail(PHOTON_EHIP, "aggregate: %s", hipGetErrorString(e));
  return ok();
}

photon_status photon_set_position(photon_ctx* c, int64_t tokens, void* stream) {
  if (!c) return fail(PHOTON_EINVAL, "ctx is NULL");
  if (!c->prefilled) return fail(PHOTON_ESTATE, "no prefill to rewind to");
  // a flat-baseline context counts tokens (steps per call), PHOTON top states
  const int64_t S = c->vanilla ? c->vcfg.steps : levels(&c->cfg).S();
  if ((tokens % S && tokens != c->prompt_tokens) || tokens < c->prompt_tokens || tokens > c->tokens)
    return fail(PHOTON_ESHAPE, "position %lld must be the prompt end or a multiple of %lld within [%lld, %lld]",
                (long long)tokens, (long long)S, (long long)c->prompt_tokens, (long long)c->tokens);
  int* counter = (int*)(c->ws + (c->vanilla ? c->vplan.counter.off : c->plan.counter.off));
  const int64_t pos = c->vanilla ? tokens : tokens / S;
  HIP_TRY(launch_set_int(counter, (int)pos, (hipStream_t)stream));
  c->tokens = tokens;
  c->top_len = pos;
  c->tail_pending = !c->vanilla && c->tail_r > 0 && tokens == c->prompt_tokens;
  c->ahat_ready = false;
  return ok();
}

photon_status photon_use_graphs(photon_ctx* c, int32_t enable) {
  if (!c) return fail(PHOTON_EINVAL, "ctx is NULL");
  c->use_graph = enable != 0;
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
    // wait with a deadline: a dispatch-recorded event that never completes
    // (e.g. under a tool that rewrites dispatch packets) is an error, not a hang
    const auto t0 = std::chrono::steady_clock::now();
    for (;;) {
      const hipError_t q = hipEventQuery(r.b);
      if (q == hipSuccess) break;
      if (q != hipErrorNotReady) return fail(PHOTON_EHIP, "trace event: %s", hipGetErrorString(q));
      if (std::chrono::steady_clock::now() - t0 > std::chrono::seconds(60))
        return fail(PHOTON_EHIP, "trace event did not complete within 60 s");
      std::this_thread::sleep_for(std::chrono::microseconds(50));
    }
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

// ------------------------------------------------------ stand-alone attention
namespace {
photon_status check_attention(int32_t kind, int32_t groups, int32_t heads, int32_t head_dim, int32_t queries,
                              int32_t cap) {
  if (kind != PHOTON_ATTN_GLOBAL && kind != PHOTON_ATTN_CHUNK && kind != PHOTON_ATTN_PREFILL)
    return fail(PHOTON_EINVAL, "unknown attention kind %d", kind);
  if (groups < 1 || heads < 1) return fail(PHOTON_ESHAPE, "groups and heads must be >= 1");
  if (head_dim != 32 && head_dim != 64 && head_dim != 96 && head_dim != 128)
    return fail(PHOTON_EUNSUPPORTED, "head_dim %d is not one of 32, 64, 96, 128", head_dim);
  if (queries < 1 || cap < queries) return fail(PHOTON_ESHAPE, "need 1 <= queries <= cap");
  if (kind == PHOTON_ATTN_GLOBAL && queries != 1 && queries != 2 && queries != 4)
    return fail(PHOTON_EUNSUPPORTED, "global attention takes 1, 2 or 4 queries per group (got %d)", queries);
  if ((int64_t)groups * heads * cap * head_dim > ((int64_t)1 << 40))
    return fail(PHOTON_ESHAPE, "cache too large");
  return ok();
}

uint64_t attention_part_bytes(int32_t kind, int32_t groups, int32_t heads, int32_t head_dim, int32_t queries,
                              int32_t cap, int* nsplit) {
  *nsplit = kind == PHOTON_ATTN_GLOBAL ? attn_decode_splits(groups, heads, cap, queries) : 1;
  return *nsplit > 1 ? (uint64_t)groups * heads * queries * *nsplit * (head_dim + 2) * sizeof(float) : 0;
}
}  // namespace

extern "C" {

photon_status photon_attention_scratch_bytes(int32_t kind, int32_t groups, int32_t heads, int32_t head_dim,
                                             int32_t queries, int32_t cap, uint64_t* bytes) {
  if (!bytes) return fail(PHOTON_EINVAL, "bytes is NULL");
  PH_TRY(check_attention(kind, groups, heads, head_dim, queries, cap));
  int ns = 1;
  *bytes = attention_part_bytes(kind, groups, heads, head_dim, queries, cap, &ns);
  return ok();
}

photon_status photon_attention(int32_t kind, int32_t dtype, const float* d_q, const void* d_k, const void* d_v,
                               void* d_out, int32_t groups, int32_t heads, int32_t head_dim, int32_t queries,
                               int32_t keys, int32_t cap, void* d_scratch, uint64_t scratch_bytes, void* stream) {
  PH_TRY(check_attention(kind, groups, heads, head_dim, queries, cap));
  if (dtype != PHOTON_F32 && dtype != PHOTON_BF16) return fail(PHOTON_EINVAL, "unknown dtype %d", dtype);
  if (!d_q || !d_k || !d_v || !d_out) return fail(PHOTON_EINVAL, "NULL buffer");
  if (keys < queries || keys > cap) return fail(PHOTON_ESHAPE, "need queries <= keys <= cap");
  if (kind == PHOTON_ATTN_CHUNK && keys > 16) return fail(PHOTON_EUNSUPPORTED, "chunk attention takes at most 16 keys");
  if (kind == PHOTON_ATTN_PREFILL && keys != queries)
    return fail(PHOTON_ESHAPE, "prefill attention needs queries == keys (got %d, %d)", queries, keys);
  int ns = 1;
  const uint64_t need = attention_part_bytes(kind, groups, heads, head_dim, queries, cap, &ns);
  if (need > 0 && (!d_scratch || scratch_bytes < need))
    return fail(PHOTON_ESHAPE, "scratch needs %llu bytes", (unsigned long long)need);
  if (need > 0 && ((uintptr_t)d_scratch % 256)) return fail(PHOTON_EINVAL, "scratch must be 256-byte aligned");
  AttnCall a{};
  a.dtype = dtype; a.G = groups; a.Q = queries; a.H = heads; a.hd = head_dim;
  a.q = d_q; a.q_ld = (int64_t)heads * head_dim;
  a.Kc = d_k; a.Vc = d_v; a.seq_stride = (int64_t)heads * cap * head_dim; a.cap = cap; a.seq0 = 0;
  a.L_host = keys; a.L_dev = nullptr; a.L_mul = 0; a.L_add = 0;
  a.out = d_out; a.out_ld = (int64_t)heads * head_dim;
  a.part = (float*)d_scratch; a.nsplit = ns;
  const hipStream_t st = (hipStream_t)stream;
  const hipError_t e = kind == PHOTON_ATTN_GLOBAL  ? launch_attn_decode(a, st)
                       : kind == PHOTON_ATTN_CHUNK ? launch_attn_chunk(a, st)
                                                   : launch_attn_prefill(a, st);
  if (e != hipSuccess) return fail(PHOTON_EHIP, "attention launch: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"

// ------------------------------------------- attention without allocation
// The split partials of photon_attention_noalloc live in this file-scope
// device array: every GPU the library runs on holds its own copy, for as
// long as the process lives.  Host code never passes `scratch` itself (on
// the host it is a stand-in, not a device address): each device's address
// comes from hipGetSymbolAddress, taken once per device with that device
// current, and kernels receive that pointer.
namespace {
constexpr uint64_t kNoallocScratchBytes = PHOTON_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
}  // namespace
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// The current device's address of `scratch` (looked up on its first use).
photon_status noalloc_scratch(void** out) {
  int dev = -1;
  HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(PHOTON_EUNSUPPORTED, "device index %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(PHOTON_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return ok();
}
}  // namespace

extern "C" {

photon_status photon_attention_noalloc(int32_t kind, int32_t dtype, const float* d_q, const void* d_k,
                                       const void* d_v, void* d_out, int32_t groups, int32_t heads,
                                       int32_t head_dim, int32_t queries, int32_t keys, int32_t cap, void* stream) {
  PH_TRY(check_attention(kind, groups, heads, head_dim, queries, cap));
  int ns = 1;
  const uint64_t need = attention_part_bytes(kind, groups, heads, head_dim, queries, cap, &ns);
  if (need > kNoallocScratchBytes)
    return fail(PHOTON_ECAPACITY, "split partials need %llu bytes; the built-in scratch holds %llu",
                (unsigned long long)need, (unsigned long long)kNoallocScratchBytes);
  void* p = nullptr;
  PH_TRY(noalloc_scratch(&p));
  // every split writes its whole partial before the combine reads it, so
  // nothing left by an earlier call needs clearing
  return photon_attention(kind, dtype, d_q, d_k, d_v, d_out, groups, heads, head_dim, queries, keys, cap, p,
                          kNoallocScratchBytes, stream);
}

}  // extern "C"

// ------------------------------------------------------- flat baseline
namespace {

// One decode call of the flat baseline: `steps` tokens per sequence.  Every
// position is read from the device counter, so one captured graph serves
// every call.
photon_status enqueue_vanilla(photon_ctx* c, float* d_logits, hipStream_t st) {
  const photon_config& cf = c->cfg;
  const photon_vanilla_config& v = c->vcfg;
  const VPlan& wp = c->vplan;
  unsigned char* ws = c->ws;
  const int dt = cf.dtype, d = cf.d_model, H = cf.n_heads, hd = d / H, V = cf.vocab;
  const int B = (int)c->B, steps = v.steps;
  int* counter = (int*)(ws + wp.counter.off);
  StackBufs b{(float*)(ws + wp.x.off), ws + wp.a.off, (float*)(ws + wp.part.off), (float*)(ws + wp.q.off),
              ws + wp.o.off, ws + wp.hid.off, (float*)(ws + wp.apart.off)};
  void* z = ws + wp.z.off;
  int* tok = (int*)(ws + wp.tok.off);
  const int eb = elem_bytes(&cf);
  for (int j = 0; j < steps; ++j) {
    GemmCall g{};
    g.dtype = dt; g.A = z; g.lda = d; g.W = c->W_out; g.M = B; g.N = V; g.K = d;
    g.epi = EPI_ARGMAX;
    g.C = d_logits ? d_logits + (int64_t)j * V : nullptr;
    g.ldc = (int64_t)steps * V;
    g.amax_val = (float*)(ws + wp.amv.off); g.amax_idx = (int*)(ws + wp.ami.off);
    PH_TRY(run_gemm(c, PHOTON_K_GEMM_HEAD, g, st));
    // token j of every sequence, then its embedding and norm as the stack input
    ArgmaxNext an{g.amax_val, g.amax_idx, wp.head_tiles, B, steps, 1, j, tok,
                  nullptr, 0, c->E, b.x, b.a, c->vlayers.layers[0].g1, d, cf.norm_eps, nullptr, 0, V};
    PH_TRY(traced(c, PHOTON_K_ARGMAX, (double)B * d * (4 + 2 * eb), 0, st, "argmax_next",
                  [&] { return launch_argmax_next(dt, an, st); }));
    StackRun r{};
    r.M = B; r.rows_per_seq = 1; r.G = B;
    r.kv = KvTarget{ws + wp.kv.off, (int64_t)B * H * wp.cap * hd, true, (int64_t)H * wp.cap * hd, (int)wp.cap, 0};
    r.pos_add = 0; r.pos_dev = counter; r.pos_mul = 1; r.rope = (const float*)(ws + wp.rope.off);
    r.kind = ATT_DECODE; r.Q = 1; r.L_dev = counter; r.L_mul = 1; r.L_add = 1; r.nsplit = wp.nsplit;
    r.L_acct = (int)(c->tokens + j + 1);
    r.out = z; r.out_rows = B; r.in_stride = 1; r.in_off = 0;
    PH_TRY(run_stack(c, c->vlayers, b, r, st));
    HIP_TRY(launch_add_int(counter, 1, st));
  }
  return ok();
}

}  // namespace

extern "C" {

photon_status photon_vanilla_kv_bytes(const photon_vanilla_config* cfg, int32_t batch, int64_t tokens,
                                      photon_kv_report* out) {
  PH_TRY(check_vconfig(cfg));
  if (!out) return fail(PHOTON_EINVAL, "out is NULL");
  if (batch < 1) return fail(PHOTON_ESHAPE, "batch must be >= 1");
  if (tokens < 1) return fail(PHOTON_ESHAPE, "tokens must be >= 1");
  const VPlan p = plan_vworkspace(cfg, batch, tokens);
  memset(out, 0, sizeof *out);
  out->top_len = p.cap;
  out->top_kv = p.kv.bytes;
  out->state = p.state_bytes;
  out->decode_scratch = p.scratch_bytes;
  out->workspace_total = p.total;
  vlayout(cfg, &out->weights_decode);
  out->off_top_kv = p.kv.off;
  out->off_state = p.z.off;
  out->off_scratch = p.off_scratch;
  return ok();
}

photon_status photon_vanilla_prefill_scratch_bytes(const photon_vanilla_config* cfg, int32_t batch,
                                                   int32_t prompt_len, uint64_t* out) {
  PH_TRY(check_vconfig(cfg));
  if (!out) return fail(PHOTON_EINVAL, "out is NULL");
  if (batch < 1) return fail(PHOTON_ESHAPE, "batch must be >= 1");
  if (prompt_len < cfg->steps || prompt_len % cfg->steps)
    return fail(PHOTON_ESHAPE, "prompt_len %d must be a positive multiple of steps = %d", prompt_len, cfg->steps);
  *out = plan_vprefill(cfg, batch, prompt_len).total;
  return ok();
}

photon_status photon_vanilla_weight_layout(const photon_vanilla_config* cfg, uint64_t* bytes, int32_t* n_tensors) {
  PH_TRY(check_vconfig(cfg));
  auto t = vlayout(cfg, bytes);
  if (n_tensors) *n_tensors = (int32_t)t.size();
  return ok();
}

photon_status photon_vanilla_weight_tensor(const photon_vanilla_config* cfg, int32_t index,
                                           photon_tensor_info* out) {
  PH_TRY(check_vconfig(cfg));
  if (!out) return fail(PHOTON_EINVAL, "out is NULL");
  auto v = vlayout(cfg, nullptr);
  if (index < 0 || index >= (int32_t)v.size()) return fail(PHOTON_EINVAL, "tensor index %d out of range", index);
  const TensorDesc& t = v[index];
  memset(out, 0, sizeof *out);
  snprintf(out->name, sizeof out->name, "%s", t.name.c_str());
  out->blob = 0;
  out->dtype = t.is_gain ? PHOTON_F32 : cfg->dtype;
  out->offset = t.offset;
  out->rows = t.rows;
  out->cols = t.cols;
  return ok();
}

photon_status photon_vanilla_open(const photon_vanilla_config* cfg, const void* d_weights, photon_ctx** out) {
  PH_TRY(check_vconfig(cfg));
  if (!out) return fail(PHOTON_EINVAL, "out is NULL");
  if (!d_weights) return fail(PHOTON_EINVAL, "weight blob is NULL");
  if ((uintptr_t)d_weights % kAlign) return fail(PHOTON_EINVAL, "weight blob must be 256-byte aligned");
  photon_ctx* c = new (std::nothrow) photon_ctx();
  if (!c) return fail(PHOTON_EINVAL, "out of host memory");
  c->vanilla = true;
  c->vcfg = *cfg;
  c->cfg = vanilla_as_config(cfg);
  c->wdec = (const unsigned char*)d_weights;
  c->tensors = vlayout(cfg, nullptr);
  c->E = tensor_ptr(c, "E");
  c->W_out = tensor_ptr(c, "W_out");
  bind_stack(c, c->vlayers, "layers", cfg->n_layers);
  *out = c;
  return ok();
}

photon_status photon_vanilla_prefill(photon_ctx* c, void* d_workspace, uint64_t ws_bytes, void* d_scratch,
                                     uint64_t scratch_bytes, const int32_t* d_prompt, int32_t batch,
                                     int32_t prompt_len, int64_t max_tokens, void* stream) {
  if (!c) return fail(PHOTON_EINVAL, "ctx is NULL");
  if (!c->vanilla) return fail(PHOTON_ESTATE, "not a flat-baseline context (use photon_prefill)");
  if (!d_workspace || !d_scratch || !d_prompt) return fail(PHOTON_EINVAL, "NULL device pointer");
  if (((uintptr_t)d_workspace | (uintptr_t)d_scratch) % kAlign)
    return fail(PHOTON_EINVAL, "workspace and scratch must be 256-byte aligned");
  const photon_vanilla_config& v = c->vcfg;
  const photon_config& cf = c->cfg;
  if (batch < 1) return fail(PHOTON_ESHAPE, "batch must be >= 1");
  if (prompt_len < v.steps || prompt_len % v.steps)
    return fail(PHOTON_ESHAPE, "prompt_len %d must be a positive multiple of steps = %d", prompt_len, v.steps);
  if (max_tokens < prompt_len) return fail(PHOTON_ECAPACITY, "max_tokens %lld < prompt_len %d", (long long)max_tokens, prompt_len);
  const VPlan wp = plan_vworkspace(&v, batch, max_tokens);
  if (ws_bytes < wp.total)
    return fail(PHOTON_ECAPACITY, "workspace holds %llu bytes, needs %llu", (unsigned long long)ws_bytes,
                (unsigned long long)wp.total);
  const VPrePlan pp = plan_vprefill(&v, batch, prompt_len);
  if (scratch_bytes < pp.total)
    return fail(PHOTON_ECAPACITY, "prefill scratch holds %llu bytes, needs %llu", (unsigned long long)scratch_bytes,
                (unsigned long long)pp.total);
  {
    const int d = cf.d_model, F = cf.mlp_mult * d;
    for (int64_t M : {(int64_t)batch, pp.bs * prompt_len, (batch % pp.bs) * (int64_t)prompt_len}) {
      if (M == 0) continue;
      for (auto nk : {std::pair<int, int>{3 * d, d}, {d, d}, {F, d}, {d, F}})
        if (M > 0x7fffffff || !gemm_supported(cf.dtype, (int)M, nk.first, nk.second))
          return fail(PHOTON_EUNSUPPORTED, "GEMM %lldx%dx%d unsupported", (long long)M, nk.first, nk.second);
    }
    if (!gemm_supported(cf.dtype, batch, cf.vocab, d)) return fail(PHOTON_EUNSUPPORTED, "head GEMM unsupported");
  }
  hipStream_t st = (hipStream_t)stream;
  const int dt = cf.dtype, d = cf.d_model, H = cf.n_heads, hd = d / H;
  const int eb = elem_bytes(&cf);
  unsigned char* ws = (unsigned char*)d_workspace;
  unsigned char* sc = (unsigned char*)d_scratch;
  c->prefilled = false;
  c->drop_graphs();
  c->ws = ws;
  c->vplan = wp;
  c->B = batch;
  c->max_tokens = max_tokens;
  float* rope = (float*)(ws + wp.rope.off);
  HIP_TRY(launch_rope_table(rope, (int)wp.cap, hd, cf.rope_theta, st));
  StackBufs bufs{(float*)(sc + pp.x.off), sc + pp.a.off, (float*)(sc + pp.part.off), (float*)(sc + pp.q.off),
                 sc + pp.o.off, sc + pp.hid.off, nullptr};
  for (int64_t b0 = 0; b0 < batch; b0 += pp.bs) {
    const int bs = (int)std::min<int64_t>(pp.bs, batch - b0);
    const int R = bs * prompt_len;
    // stack input: x = E[token], a = its first norm
    RowsEpi e{};
    e.P = bufs.x; e.ksplit = 0; e.pstride = 0; e.ldp = d;   // no slabs: x is the embedding alone
    e.ids = d_prompt + b0 * prompt_len; e.E = c->E;
    e.x_out = bufs.x; e.g = c->vlayers.layers[0].g1; e.a_out = bufs.a; e.a_ld = d;
    e.R = R; e.d = d; e.row_stride = 1; e.row_off = 0; e.eps = cf.norm_eps;
    PH_TRY(traced(c, PHOTON_K_EMBED, (double)R * (4 + d * (eb + 4.0 + eb)), 0, st, "rows_epilogue",
                  [&] { return launch_rows_epilogue(dt, e, st); }));
    StackRun r{};
    r.M = R; r.rows_per_seq = prompt_len; r.G = bs;
    r.kv = KvTarget{ws + wp.kv.off, (int64_t)batch * H * wp.cap * hd, true, (int64_t)H * wp.cap * hd, (int)wp.cap,
                    (int)b0};
    r.pos_add = 0; r.pos_dev = nullptr; r.pos_mul = 0; r.rope = rope;
    r.kind = ATT_PREFILL; r.Q = prompt_len; r.L_host = prompt_len; r.nsplit = 1; r.L_acct = prompt_len;
    // final norm only for the last position of each sequence: z
    r.out = ws + wp.z.off + (uint64_t)b0 * d * eb; r.out_rows = bs; r.in_stride = prompt_len;
    r.in_off = prompt_len - 1;
    PH_TRY(run_stack(c, c->vlayers, bufs, r, st));
  }
  HIP_TRY(launch_set_int((int*)(ws + wp.counter.off), prompt_len, st));
  c->top_len = prompt_len;
  c->tokens = prompt_len;
  c->prompt_tokens = prompt_len;
  c->prefilled = true;
  return ok();
}

photon_status photon_vanilla_decode(photon_ctx* c, int32_t* d_tokens, float* d_logits, void* stream) {
  if (!c) return fail(PHOTON_EINVAL, "ctx is NULL");
  if (!c->vanilla) return fail(PHOTON_ESTATE, "not a flat-baseline context (use photon_decode_chunk)");
  if (!d_tokens) return fail(PHOTON_EINVAL, "d_tokens is NULL");
  if (!c->prefilled) return fail(PHOTON_ESTATE, "decode before prefill");
  const int steps = c->vcfg.steps;
  if (c->tokens + steps > c->max_tokens)
    return fail(PHOTON_ECAPACITY, "decode would pass max_tokens %lld", (long long)c->max_tokens);
  hipStream_t st = (hipStream_t)stream;
  const int B = (int)c->B;
  int* tok = (int*)(c->ws + c->vplan.tok.off);
  if (c->use_graph && !d_logits && c->tr.mask == 0) {
    if (!c->graph[0]) {
      if (!c->cap[0]) HIP_TRY(hipStreamCreateWithFlags(&c->cap[0], hipStreamNonBlocking));
      PH_TRY(capture_graph(c, &c->graph[0], [&](hipStream_t cs) { return enqueue_vanilla(c, nullptr, cs); }));
    }
    HIP_TRY(hipGraphLaunch(c->graph[0], st));
  } else {
    PH_TRY(enqueue_vanilla(c, d_logits, st));
  }
  HIP_TRY(hipMemcpyAsync(d_tokens, tok, (size_t)B * steps * sizeof(int), hipMemcpyDeviceToDevice, st));
  c->tokens += steps;
  c->top_len = c->tokens;
  return ok();
}

}  // extern "C"
