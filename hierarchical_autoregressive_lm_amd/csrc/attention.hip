// Attention kernels for the PHOTON decode and prefill paths.
//
//  * attn_decode: the top encoder's step over the global coarse K/V cache
//    (and HierGen's level-1 step).  Memory-bound: every byte of K and V is
//    streamed once, with non-temporal loads (the cache is read once per
//    step; keeping it out of the caches leaves them to the weights and
//    activations).  One workgroup per (sequence, head, key split); the
//    threads form row slots of 16 lanes, each lane owning hd/16 contiguous
//    elements, so a wave reads 4 consecutive cache rows per instruction
//    (contiguous bytes).  Each row slot keeps its own online-softmax state
//    (max, sum, partial output) over the keys it visits; the slots are
//    merged through LDS at the end, and the splits by a combine kernel.
//  * attn_chunk: the decoders' attention confined to the chunk (at most a
//    few keys per query).  16 lanes per (sequence, head) pair hold every key
//    of the pair for hd/16 contiguous elements (non-temporal loads), so
//    scores need one 16-lane reduction and the output is lane-local; 4 pairs
//    per wave.
//  * attn_prefill: causal attention over a whole prompt with K/V tiles of
//    64 keys staged in LDS: MFMA on bf16 caches (128 queries per
//    workgroup), fp32 FMA on fp32 caches (64 queries per workgroup).
// q is fp32 everywhere; K and V are read in the storage dtype; softmax and
// accumulation are fp32; the output is rounded to the storage dtype.
#include "common.h"
#include "kernels.h"

namespace photon {
namespace {

// One cache row segment of CE elements held as raw dwords (bf16 pairs or
// fp32), loaded with plain or non-temporal loads and widened on use.
template <typename T, int CE, bool NT> struct Raw {
  static constexpr int W = CE * (int)sizeof(T) / 4;
  uint32_t w[W];
  __device__ __forceinline__ void load(const T* p) {
    const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
#pragma unroll
    for (int i = 0; i < W; ++i) w[i] = NT ? __builtin_nontemporal_load(q + i) : q[i];
  }
  __device__ __forceinline__ void unpack(float (&v)[CE]) const {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int i = 0; i < W; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int i = 0; i < W; ++i) v[i] = __uint_as_float(w[i]);
    }
  }
};

__device__ __forceinline__ int resolve_len(int L_host, const int* L_dev, int L_mul, int L_add) {
  return L_dev ? (*L_dev) * L_mul + L_add : L_host;
}

// Fused RoPE + K/V append: new row t of group g, head h, for lane c of its
// 16-lane group (elements [c*CE, (c+1)*CE)).  Sums the QKV GEMM's slabs in
// slab order; q and k turn by the rotate-half embedding at position pos(t)
// (pairs (i, i + hd/2): lanes c and c ^ 8 hold partners, exchanged by a
// DPP move inside the 16-lane row, so all 16 lanes must be active); k and v are rounded to the
// storage dtype (the values a cache read would give).  Returns pos(t).
// AHEAD (decode kernels, whose register peak lies in the key loop): every
// load goes out before the first sum waits (the table entries, then the
// slabs two at a time, summed in slab order all the same), so forming q
// costs one round trip instead of one per slab plus the table's.  The chunk
// kernel keeps the loads in step with the sums (the extra values in flight
// would cost it occupancy).
template <typename T, int HD, bool AHEAD = false>
__device__ __forceinline__ int new_row(const AttnCall& a, int g, int t, int h, int c, float (&q)[HD / 16],
                                       float (&k)[HD / 16], float (&v)[HD / 16]) {
  constexpr int CE = HD / 16, half = HD / 2;
  const float* p = a.qkv + ((int64_t)g * a.Q + t) * 3 * a.d + h * HD + c * CE;
  const int pos = a.pos_add + (a.pos_dev ? (*a.pos_dev) * a.pos_mul : 0) + t;
  const float* rt = a.rope + ((int64_t)pos * half + (c & 7) * CE) * 2;
  float cs[CE], sn[CE];
  if constexpr (AHEAD) {
#pragma unroll
    for (int e = 0; e < CE; ++e) { cs[e] = rt[2 * e]; sn[e] = rt[2 * e + 1]; }
  }
  float x[CE], y[CE];
#pragma unroll
  for (int e = 0; e < CE; ++e) { x[e] = 0.f; y[e] = 0.f; v[e] = 0.f; }
  int sl = 0;
  if constexpr (AHEAD) {
    for (; sl + 1 < a.ksplit; sl += 2) {
      const float* p0 = p + sl * a.pstride;
      const float* p1 = p0 + a.pstride;
      float x0[CE], y0[CE], v0[CE], x1[CE], y1[CE], v1[CE];
#pragma unroll
      for (int e = 0; e < CE; ++e) {
        x0[e] = p0[e]; y0[e] = p0[a.d + e]; v0[e] = p0[2 * a.d + e];
        x1[e] = p1[e]; y1[e] = p1[a.d + e]; v1[e] = p1[2 * a.d + e];
      }
#pragma unroll
      for (int e = 0; e < CE; ++e) {
        x[e] = (x[e] + x0[e]) + x1[e];
        y[e] = (y[e] + y0[e]) + y1[e];
        v[e] = (v[e] + v0[e]) + v1[e];
      }
    }
  }
  for (; sl < a.ksplit; ++sl) {
    const float* ps = p + sl * a.pstride;
#pragma unroll
    for (int e = 0; e < CE; ++e) {
      x[e] += ps[e];
      y[e] += ps[a.d + e];
      v[e] += ps[2 * a.d + e];
    }
  }
  if constexpr (!AHEAD) {
#pragma unroll
    for (int e = 0; e < CE; ++e) { cs[e] = rt[2 * e]; sn[e] = rt[2 * e + 1]; }
  }
#pragma unroll
  for (int e = 0; e < CE; ++e) {
    const float xp = row16_swap8(x[e]), yp = row16_swap8(y[e]);
    if (c < 8) {
      q[e] = x[e] * cs[e] - xp * sn[e];
      k[e] = St<T>::ld(St<T>::st(y[e] * cs[e] - yp * sn[e]));
    } else {
      q[e] = x[e] * cs[e] + xp * sn[e];
      k[e] = St<T>::ld(St<T>::st(y[e] * cs[e] + yp * sn[e]));
    }
    v[e] = St<T>::ld(St<T>::st(v[e]));
  }
  return pos;
}

// Store the lane's CE elements of a new key and value at cache slot pos.
template <typename T, int HD>
__device__ __forceinline__ void store_row(const AttnCall& a, int g, int h, int c, int pos, const float (&k)[HD / 16],
                                          const float (&v)[HD / 16]) {
  constexpr int CE = HD / 16;
  const int64_t off = (int64_t)(a.seq0 + g) * a.seq_stride + ((int64_t)h * a.cap + pos) * HD + c * CE;
  T* K = reinterpret_cast<T*>(const_cast<void*>(a.Kc)) + off;
  T* V = reinterpret_cast<T*>(const_cast<void*>(a.Vc)) + off;
#pragma unroll
  for (int e = 0; e < CE; ++e) {
    K[e] = St<T>::st(k[e]);
    V[e] = St<T>::st(v[e]);
  }
}

// ---------------------------------------------------------------- decode
// Merge nsplit partial results (num[hd], max, sum) of one (g, h, t) query.
template <typename T, int HD>
__device__ __forceinline__ void combine_splits(const AttnCall& a, int g, int h, int t, int e) {
  const float* pp = a.part + (((int64_t)g * a.H + h) * a.Q + t) * a.nsplit * (HD + 2);
  float M = -INFINITY;
  for (int s = 0; s < a.nsplit; ++s) M = fmaxf(M, pp[s * (HD + 2) + HD]);
  float den = 0.f, num = 0.f;
  for (int s = 0; s < a.nsplit; ++s) {
    const float ms = pp[s * (HD + 2) + HD];
    if (ms == -INFINITY) continue;
    const float w = expf(ms - M);
    den = fmaf(pp[s * (HD + 2) + HD + 1], w, den);
    num = fmaf(pp[s * (HD + 2) + e], w, num);
  }
  T* out = reinterpret_cast<T*>(a.out);
  out[(int64_t)(g * a.Q + t) * a.out_ld + h * HD + e] = St<T>::st(num / den);
}

// Second pass when the keys were split: one wave per (g, h, t).  (Merging in
// the last-arriving split instead would need agent-scope fences, which write
// back and invalidate the L2 and cost far more than this launch.)
template <typename T, int HD>
__global__ __launch_bounds__(64) void attn_combine_kernel(AttnCall a) {
  const int idx = blockIdx.x;
  const int t = idx % a.Q, h = (idx / a.Q) % a.H, g = idx / (a.Q * a.H);
  for (int e = threadIdx.x; e < HD; e += 64) combine_splits<T, HD>(a, g, h, t, e);
}

// One pass of a decode row slot: keys kb + r + SLOTS*u (u < U), clamped to
// k1 - 1 (in bounds; the scores mask them), K and V rows for this lane.
template <typename T, int CE, int U, int SLOTS, int HD>
__device__ __forceinline__ void load_pass(Raw<T, CE, true> (&kr)[U], Raw<T, CE, true> (&vr)[U], const T* Kb,
                                          const T* Vb, int kb, int r, int k1) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    int key = kb + r + SLOTS * u;
    key = key < k1 ? key : k1 - 1;
    kr[u].load(Kb + (int64_t)key * HD);
    vr[u].load(Vb + (int64_t)key * HD);
  }
}

template <typename T, int HD, int Q, int U, int SLOTS = 16, bool EARLY = SLOTS == 16>
__global__ __launch_bounds__(SLOTS * 16) void attn_decode_kernel(AttnCall a, float scale) {
  constexpr int CE = HD / 16;
  constexpr int NT = SLOTS * 16;
  const int tid = threadIdx.x;
  const int c = tid & 15, r = tid >> 4;
  const int nsplit = a.nsplit;
  const int split = blockIdx.x % nsplit;
  const int gh = blockIdx.x / nsplit;
  const int h = gh % a.H, g = gh / a.H;
  const int L = resolve_len(a.L_host, a.L_dev, a.L_mul, a.L_add);
  // fused: keys 0 .. Lc-1 come from the cache, the Q new rows' keys Lc ..
  // L-1 from registers (slot 0 of the last split folds them in below)
  const bool fused = a.qkv != nullptr;
  const int Lc = fused ? L - Q : L;
  int kps = (Lc + nsplit - 1) / nsplit;
  kps = (kps + 15) & ~15;
  const int k0 = split * kps;
  const int k1 = min(Lc, k0 + kps);
  const T* Kb = reinterpret_cast<const T*>(a.Kc) + (int64_t)(a.seq0 + g) * a.seq_stride + (int64_t)h * a.cap * HD + c * CE;
  const T* Vb = reinterpret_cast<const T*>(a.Vc) + (int64_t)(a.seq0 + g) * a.seq_stride + (int64_t)h * a.cap * HD + c * CE;
  // EARLY (short caches, and long ones that form q inside): the first
  // pass's K/V loads go out before the queries are formed and stay in
  // flight across the hand-over of q
  constexpr bool kEarly = EARLY;
  Raw<T, CE, true> kr[U], vr[U];
  if (kEarly && k0 < k1) load_pass<T, CE, U, SLOTS, HD>(kr, vr, Kb, Vb, k0, r, k1);

  // fused: slot 0 forms the queries from the QKV slabs (one read of them
  // per workgroup) and hands them to the other slots through LDS; with one
  // query it also keeps the new row's k and v, which the last split's slot
  // 0 stores and folds in after its pass
  const bool owner = fused && r == 0 && split == nsplit - 1;
  float qv[Q][CE], kn1[CE], vn1[CE];
  if (fused) {
    __shared__ float qs[Q][HD];
    if (r == 0) {
#pragma unroll
      for (int t = 0; t < Q; ++t) {
        float qn[CE], kn[CE], vn[CE];
        const int pos = new_row<T, HD, true>(a, g, t, h, c, qn, kn, vn);
#pragma unroll
        for (int e = 0; e < CE; ++e) qs[t][c * CE + e] = qn[e] * scale;
        if constexpr (Q == 1) {
#pragma unroll
          for (int e = 0; e < CE; ++e) { kn1[e] = kn[e]; vn1[e] = vn[e]; }
          if (owner) store_row<T, HD>(a, g, h, c, pos, kn, vn);
        }
      }
    }
    // LDS-only fences: the barrier orders q's hand-over without waiting
    // for the cache loads in flight
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
#pragma unroll
    for (int t = 0; t < Q; ++t)
#pragma unroll
      for (int e = 0; e < CE; ++e) qv[t][e] = qs[t][c * CE + e];
  } else {
#pragma unroll
    for (int t = 0; t < Q; ++t)
#pragma unroll
      for (int e = 0; e < CE; ++e)
        qv[t][e] = a.q[(int64_t)(g * Q + t) * a.q_ld + h * HD + c * CE + e] * scale;
  }

  float m[Q], l[Q], o[Q][CE];
#pragma unroll
  for (int t = 0; t < Q; ++t) {
    m[t] = -INFINITY; l[t] = 0.f;
#pragma unroll
    for (int e = 0; e < CE; ++e) o[t][e] = 0.f;
  }

  // Row slot r visits keys k0 + r, k0 + r + SLOTS, ...; U of them per
  // iteration, loaded together and folded into the slot's online softmax
  // with a single rescale.
  for (int kb = k0; kb < k1; kb += SLOTS * U) {
    if (!kEarly || kb != k0) load_pass<T, CE, U, SLOTS, HD>(kr, vr, Kb, Vb, kb, r, k1);
    float kv[U][CE], vv[U][CE];
#pragma unroll
    for (int u = 0; u < U; ++u) { kr[u].unpack(kv[u]); vr[u].unpack(vv[u]); }
#pragma unroll
    for (int t = 0; t < Q; ++t) {
      float sc[U];
      float mx = m[t];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < CE; ++e) s = fmaf(qv[t][e], kv[u][e], s);
        s = row16_sum(s);
        const int key = kb + r + SLOTS * u;
        sc[u] = (key < k1 && key <= L - Q + t) ? s : -INFINITY;
        mx = fmaxf(mx, sc[u]);
      }
      if (mx == -INFINITY) continue;       // nothing visible yet (uniform per slot)
      const float corr = expf(m[t] - mx);
      float ps = 0.f;
#pragma unroll
      for (int e = 0; e < CE; ++e) o[t][e] *= corr;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float p = expf(sc[u] - mx);
        ps += p;
#pragma unroll
        for (int e = 0; e < CE; ++e) o[t][e] = fmaf(p, vv[u][e], o[t][e]);
      }
      l[t] = l[t] * corr + ps;
      m[t] = mx;
    }
  }
  if (owner) {
    // the new rows' K/V (several queries: loaded again here, and stored)
    // into the state of every query t >= tn as key Lc + tn
    for (int tn = 0; tn < Q; ++tn) {
      float kn[CE], vn[CE];
      if constexpr (Q == 1) {
#pragma unroll
        for (int e = 0; e < CE; ++e) { kn[e] = kn1[e]; vn[e] = vn1[e]; }
      } else {
        float qd[CE];
        const int pos = new_row<T, HD, true>(a, g, tn, h, c, qd, kn, vn);
        store_row<T, HD>(a, g, h, c, pos, kn, vn);
      }
#pragma unroll
      for (int t = 0; t < Q; ++t) {
        if (t < tn) continue;
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < CE; ++e) s = fmaf(qv[t][e], kn[e], s);
        s = row16_sum(s);
        const float mx = fmaxf(m[t], s);
        const float corr = expf(m[t] - mx), p = expf(s - mx);
#pragma unroll
        for (int e = 0; e < CE; ++e) o[t][e] = fmaf(p, vn[e], o[t][e] * corr);
        l[t] = l[t] * corr + p;
        m[t] = mx;
      }
    }
  }

  // merge the row slots
  __shared__ float sm[SLOTS][Q], sl[SLOTS][Q];
  __shared__ float so[SLOTS][Q][HD];
#pragma unroll
  for (int t = 0; t < Q; ++t) {
    if (c == 0) { sm[r][t] = m[t]; sl[r][t] = l[t]; }
#pragma unroll
    for (int e = 0; e < CE; ++e) so[r][t][c * CE + e] = o[t][e];
  }
  __syncthreads();
  for (int idx = tid; idx < Q * HD; idx += NT) {
    const int t = idx / HD, e = idx % HD;
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < SLOTS; ++s) M = fmaxf(M, sm[s][t]);
    float den = 0.f, num = 0.f;
    if (M != -INFINITY) {
#pragma unroll 16
      for (int s = 0; s < SLOTS; ++s) {
        const float w = expf(sm[s][t] - M);
        den = fmaf(sl[s][t], w, den);
        num = fmaf(so[s][t][e], w, num);
      }
    }
    if (nsplit == 1) {
      T* out = reinterpret_cast<T*>(a.out);
      out[(int64_t)(g * Q + t) * a.out_ld + h * HD + e] = St<T>::st(num / den);
    } else {
      float* pp = a.part + ((((int64_t)g * a.H + h) * Q + t) * nsplit + split) * (HD + 2);
      pp[e] = num;
      if (e == 0) { pp[HD] = M; pp[HD + 1] = den; }
    }
  }
}

// ----------------------------------------------------------------- chunk
// Lanes 16*sub .. 16*sub+15 of a wave own pair 4*wave + sub; lane c holds
// elements [c*hd/16, (c+1)*hd/16) of every key of the pair.
template <typename T, int HD, int MAXL>
__global__ __launch_bounds__(256) void attn_chunk_kernel(AttnCall a, float scale) {
  constexpr int CE = HD / 16;
  using R = Raw<T, CE, true>;
  const int lane = threadIdx.x & 63, c = lane & 15, sub = lane >> 4;
  const int pair = (blockIdx.x * 4 + (threadIdx.x >> 6)) * 4 + sub;
  if (pair >= a.G * a.H) return;            // whole 16-lane groups exit together
  const int h = pair % a.H, g = pair / a.H;
  const int L = resolve_len(a.L_host, a.L_dev, a.L_mul, a.L_add);
  const bool fused = a.qkv != nullptr;
  const int Lc = fused ? L - a.Q : L;       // keys read from the cache
  const T* Kb = reinterpret_cast<const T*>(a.Kc) + (int64_t)(a.seq0 + g) * a.seq_stride + (int64_t)h * a.cap * HD + c * CE;
  const T* Vb = reinterpret_cast<const T*>(a.Vc) + (int64_t)(a.seq0 + g) * a.seq_stride + (int64_t)h * a.cap * HD + c * CE;
  R kr[MAXL], vr[MAXL];
#pragma unroll
  for (int j = 0; j < MAXL; ++j) {
    if (j < Lc) {
      kr[j].load(Kb + j * HD);
      vr[j].load(Vb + j * HD);
    } else {
#pragma unroll
      for (int w = 0; w < R::W; ++w) { kr[j].w[w] = 0u; vr[j].w[w] = 0u; }
    }
  }
  float kv[MAXL][CE], vv[MAXL][CE];
#pragma unroll
  for (int j = 0; j < MAXL; ++j) { kr[j].unpack(kv[j]); vr[j].unpack(vv[j]); }
  float q1[CE];                             // the query of a one-row step
  if (fused) {
    // the new rows: keys Lc .. L-1 from registers, and into the cache
    for (int t = 0; t < a.Q; ++t) {
      float kn[CE], vn[CE];
      const int pos = new_row<T, HD>(a, g, t, h, c, q1, kn, vn);
      store_row<T, HD>(a, g, h, c, pos, kn, vn);
#pragma unroll
      for (int j = 0; j < MAXL; ++j)
        if (j == Lc + t)
#pragma unroll
          for (int e = 0; e < CE; ++e) { kv[j][e] = kn[e]; vv[j][e] = vn[e]; }
    }
  }
  T* out = reinterpret_cast<T*>(a.out);
  for (int t = 0; t < a.Q; ++t) {
    float q[CE];
    if (fused) {
      if (a.Q > 1) {                        // several rows: their queries again
        float kn[CE], vn[CE];
        (void)new_row<T, HD>(a, g, t, h, c, q1, kn, vn);
      }
#pragma unroll
      for (int e = 0; e < CE; ++e) q[e] = q1[e] * scale;
    } else {
      const float* qp = a.q + (int64_t)(g * a.Q + t) * a.q_ld + h * HD + c * CE;
#pragma unroll
      for (int e = 0; e < CE; ++e) q[e] = qp[e] * scale;
    }
    const int last = L - a.Q + t;           // last visible key
    float s[MAXL];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < MAXL; ++j) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < CE; ++e) d = fmaf(q[e], kv[j][e], d);
      d = row16_sum(d);
      s[j] = d;
      if (j <= last) mx = fmaxf(mx, d);
    }
    float den = 0.f, num[CE];
#pragma unroll
    for (int e = 0; e < CE; ++e) num[e] = 0.f;
#pragma unroll
    for (int j = 0; j < MAXL; ++j) {
      if (j <= last) {
        const float p = expf(s[j] - mx);
        den += p;
#pragma unroll
        for (int e = 0; e < CE; ++e) num[e] = fmaf(p, vv[j][e], num[e]);
      }
    }
    T* op = out + (int64_t)(g * a.Q + t) * a.out_ld + h * HD + c * CE;
#pragma unroll
    for (int e = 0; e < CE; ++e) op[e] = St<T>::st(num[e] / den);
  }
}

// --------------------------------------------------------------- prefill
// 64 queries per workgroup, 4 threads per query.  Thread part pp computes
// the scores of keys pp, pp+4, ... of each 64-key tile and accumulates
// output elements [pp*HD/4, (pp+1)*HD/4).
template <typename T, int HD>
__global__ __launch_bounds__(256) void attn_prefill_kernel(AttnCall a, float scale) {
  constexpr int TK = 64, QB = 64, OE = HD / 4;
  __shared__ float Ks[TK][HD + 1];
  __shared__ float Vs[TK][HD];
  const int tid = threadIdx.x;
  const int qi = tid >> 2, pp = tid & 3;
  const int nqb = (a.Q + QB - 1) / QB;
  const int qb = blockIdx.x % nqb;
  const int gh = blockIdx.x / nqb;
  const int h = gh % a.H, g = gh / a.H;
  const int t = qb * QB + qi;                  // query index in sequence
  const bool qok = t < a.Q;
  float q[HD];
#pragma unroll
  for (int e = 0; e < HD; ++e)
    q[e] = qok ? a.q[(int64_t)(g * a.Q + t) * a.q_ld + h * HD + e] * scale : 0.f;
  float o[OE];
#pragma unroll
  for (int e = 0; e < OE; ++e) o[e] = 0.f;
  float m = -INFINITY, l = 0.f;
  const T* Kb = reinterpret_cast<const T*>(a.Kc) + (int64_t)(a.seq0 + g) * a.seq_stride + (int64_t)h * a.cap * HD;
  const T* Vb = reinterpret_cast<const T*>(a.Vc) + (int64_t)(a.seq0 + g) * a.seq_stride + (int64_t)h * a.cap * HD;
  const int kend = min(a.Q, (qb + 1) * QB);    // keys 0..kend-1 may be visible
  for (int k0 = 0; k0 < kend; k0 += TK) {
    __syncthreads();
    for (int idx = tid; idx < TK * HD; idx += 256) {
      const int j = idx / HD, e = idx % HD;
      const bool ok = k0 + j < kend;
      Ks[j][e] = ok ? St<T>::ld(Kb[(int64_t)(k0 + j) * HD + e]) : 0.f;
      Vs[j][e] = ok ? St<T>::ld(Vb[(int64_t)(k0 + j) * HD + e]) : 0.f;
    }
    __syncthreads();
    float s[TK / 4];
    float tmax = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < TK / 4; ++jj) {
      const int j = jj * 4 + pp;
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < HD; ++e) d = fmaf(q[e], Ks[j][e], d);
      const bool vis = (k0 + j) <= t && (k0 + j) < kend;
      s[jj] = vis ? d : -INFINITY;
      tmax = fmaxf(tmax, s[jj]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 1, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 2, 64));
    const float mn = fmaxf(m, tmax);
    if (mn == -INFINITY) continue;             // nothing visible yet (uniform per query)
    const float corr = expf(m - mn);
    float psum = 0.f;
#pragma unroll
    for (int jj = 0; jj < TK / 4; ++jj) {
      s[jj] = expf(s[jj] - mn);
      psum += s[jj];
    }
    psum += __shfl_xor(psum, 1, 64);
    psum += __shfl_xor(psum, 2, 64);
    l = l * corr + psum;
#pragma unroll
    for (int e = 0; e < OE; ++e) o[e] *= corr;
    const int base = (threadIdx.x & 63) & ~3;
#pragma unroll
    for (int j = 0; j < TK; ++j) {
      const float pj = __shfl(s[j / 4], base + (j & 3), 64);
#pragma unroll
      for (int e = 0; e < OE; ++e) o[e] = fmaf(pj, Vs[j][pp * OE + e], o[e]);
    }
    m = mn;
  }
  if (qok) {
    T* out = reinterpret_cast<T*>(a.out);
#pragma unroll
    for (int e = 0; e < OE; ++e)
      out[(int64_t)(g * a.Q + t) * a.out_ld + h * HD + pp * OE + e] = St<T>::st(o[e] / l);
  }
}

// ------------------------------------------------------- prefill (MFMA)
// Causal attention over a whole prompt on bf16 caches with
// v_mfma_f32_16x16x32_bf16.  Transposed products keep every softmax step in
// registers: S^T = K Q^T puts 4 consecutive keys of one query in each lane
// (lane l: keys 4(l/16)+r of a 16-key block, query l%16), so a query's max
// and sum need two shuffles across the lane's 4 groups and the running
// rescale of O^T = V^T P^T is lane-local; the probabilities a lane holds are
// directly the B operand of the P V product once the 32 keys of a k-step are
// ordered (4j..4j+3, 16+4j..16+4j+3) for lane group j, with V^T read from
// LDS in that same order.
// q and p are float32 in the rounding contract; each enters the products as
// hi + lo, two bf16 terms (hi = bf16(x), lo = bf16(x - hi): 16 significant
// bits), so every product is two MFMAs accumulating in float32.
// A workgroup: NWV waves x 16 queries of one (sequence, head); K and V
// tiles of 64 keys staged in LDS, double-buffered; query blocks run
// heaviest (last) first.
//
// LDS layout: both tiles are rows of 128 bytes, eight 16-byte chunks, with
// the chunk index XOR-ed by (row / 2) % 8, so that the 16 rows x 16 bytes
// one fragment read touches fall in distinct banks (measured on gfx950: 4
// cycles per 64-lane 16-byte read, no bank conflict; rows of 64 or 208 bytes
// took 8, and the V^T rows of 144 bytes read in 8-byte halves 16).
//   K: row = key, chunk = 8 dimensions; dims 64r .. 64r+63 in region r
//      (HD/64 rounded up regions of 64 rows).  Filled by direct global->LDS
//      loads (lane l of a load writes slot base + l, so each lane fetches the
//      chunk its slot holds); rows past the prompt repeat its last key (their
//      scores are masked) and unused chunks of a region repeat chunk 0.
//   V: row = key, like K (regions of 64 dims, direct global->LDS loads), with
//      chunk c of row r at position c ^ 2(r mod 4).  The P V products read it
//      with gfx950's transposing LDS reads (ds_read_b64_tr_b16): in each group
//      of 16 lanes, lanes 4a .. 4a+3 name 16 consecutive dims of one key row
//      a and lane i receives dim i of the four rows, so two such reads give a
//      lane the 8 keys of its V^T fragment (keys 32s+4j .. +3, then
//      32s+16+4j .. +3, the order of its probabilities).  The swizzle puts the
//      two chunks each of a group's four rows at eight distinct positions.
// Tile t+1's K and V loads go out at the start of tile t and land in LDS by
// themselves; one barrier per tile.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void attn_lds_t;
typedef __attribute__((address_space(1))) const void attn_glb_t;

__device__ __forceinline__ void split_hi_lo(float x, bf16_t& hi, bf16_t& lo) {
  hi = f2bf(x);
  lo = f2bf(x - bf2f(hi));
}

// Reductions over lanes l, l ^ 16, l ^ 32, l ^ 48 with gfx950's lane swaps
// (VALU, no trip through the LDS crossbar): with the same value as both
// operands, v_permlane16_swap leaves lane l's value and its l ^ 16 partner's
// in the two results (in some order), v_permlane32_swap likewise for l ^ 32.
// Each step combines the pair with a commutative operation, so every lane
// gets the same bits as a shuffle-based xor reduction.
__device__ __forceinline__ float xor16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 16-byte slot of (row, chunk) in a tile of 128-byte rows: K, and V
__device__ __forceinline__ int lds_slot(int row, int chunk) { return row * 8 + (chunk ^ ((row >> 1) & 7)); }
__device__ __forceinline__ int vlds_pos(int row, int chunk) { return chunk ^ (2 * (row & 3)); }

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

template <int HD, int NWV>
__global__ __launch_bounds__(NWV * 64, HD <= 96 ? 4 : 2) void attn_prefill_mfma_kernel(AttnCall a, float scale) {
  constexpr int NT = NWV * 64;           // threads
  constexpr int TK = 64;                 // keys per tile
  constexpr int BQ = 16 * NWV;           // queries per workgroup
  constexpr int KS = HD / 32;            // k-steps of S^T
  constexpr int HB = HD / 16;            // 16-row blocks of O^T
  constexpr int KR = (HD + 63) / 64;     // K regions of 64 dims
  constexpr int KSLOTS = KR * TK * 8;    // 16-byte K slots per tile
  static_assert(KSLOTS % (64 * NWV) == 0, "K tile fills whole direct loads per wave");
  constexpr int KI = KSLOTS / (64 * NWV);    // direct loads per wave per tile (K, and V)
  __shared__ __attribute__((aligned(16))) uint4 Ks[2][KSLOTS];
  __shared__ __attribute__((aligned(16))) uint4 Vs[2][KSLOTS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, j = lane >> 4;
  const int T = a.Q;                     // queries = keys = prompt rows
  const int nqb = (T + BQ - 1) / BQ;
  // consecutive workgroups go to different XCDs: give each XCD a contiguous
  // run of (sequence, head, query block) tiles, so that the query blocks of
  // one (sequence, head), which all stream its K/V, share one L2
  const int total = (int)gridDim.x;
  const int bid = (total % 8 == 0) ? (int)(blockIdx.x % 8) * (total / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
  const int qb = nqb - 1 - bid % nqb;    // heaviest first
  const int gh = bid / nqb;
  const int h = gh % a.H, g = gh / a.H;
  const int q0 = qb * BQ + wave * 16;
  // scores in base-2 units: q carries log2(e), the softmax uses exp2
  const float scale2 = scale * 1.44269504088896341f;
  const bf16_t* Kb = reinterpret_cast<const bf16_t*>(a.Kc) + (int64_t)(a.seq0 + g) * a.seq_stride + (int64_t)h * a.cap * HD;
  const bf16_t* Vb = reinterpret_cast<const bf16_t*>(a.Vc) + (int64_t)(a.seq0 + g) * a.seq_stride + (int64_t)h * a.cap * HD;

  // Q^T fragments (B operand): lane holds query q0 + c, dims 32ks + 8j .. +8,
  // read as two 16-byte loads per k-step where q's rows allow it (the 8
  // scalar loads a k-step otherwise takes touch each 128-byte line of the
  // row 8 times, and this prologue then cost about a sixth of a 2048-key
  // prompt's workgroup time)
  bf16x8_t qhi[KS], qlo[KS];
  f32x4_t o[HB];
  float m = -INFINITY, l = 0.f;
#pragma unroll
  for (int b = 0; b < HB; ++b) o[b] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

  const int kend = min(T, qb * BQ + BQ);  // keys any query of the block sees
  const int ntiles = (kend + TK - 1) / TK;
  // this lane's fragment slots (uint4 index inside a tile): K for the two
  // halves (k-steps 2r, 2r+1) of a region's row, V^T for the two k-steps
  const int kfr0 = lds_slot(c, j), kfr1 = lds_slot(c, 4 + j);
  // this lane's part of the transposing V reads: key row 4j + (c >> 2) of a
  // 16-key block, dims 4(c & 3) .. +3 of a 16-dim block (half of a chunk)
  const int vrow = 4 * j + (c >> 2), vsub = c & 3;
  // direct K loads: lane l of load i fills slot (wave*KI + i)*64 + l and
  // fetches the (key, dim chunk) that slot holds
  auto issue_k = [&](int t, uint4* Kdst) {
    const int k0 = t * TK;
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int slot = (wave * KI + i) * 64 + lane;
      const int key = (slot % (TK * 8)) / 8;
      const int c8 = 8 * (slot / (TK * 8)) + ((slot & 7) ^ ((key >> 1) & 7));
      const int row = k0 + key < T ? k0 + key : T - 1;
      const bf16_t* src = Kb + (int64_t)row * HD + 8 * (c8 < HD / 8 ? c8 : 0);
      __builtin_amdgcn_global_load_lds((attn_glb_t*)src, (attn_lds_t*)(Kdst + (wave * KI + i) * 64), 16, 0, 0);
    }
  };
  // direct V loads: the same slots as K, each holding chunk c of its row at
  // position vlds_pos(row, c)
  auto issue_v = [&](int t, uint4* Vdst) {
    const int k0 = t * TK;
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int slot = (wave * KI + i) * 64 + lane;
      const int key = (slot % (TK * 8)) / 8;
      const int c8 = 8 * (slot / (TK * 8)) + vlds_pos(key, slot & 7);
      const int row = k0 + key < T ? k0 + key : T - 1;
      const bf16_t* src = Vb + (int64_t)row * HD + 8 * (c8 < HD / 8 ? c8 : 0);
      __builtin_amdgcn_global_load_lds((attn_glb_t*)src, (attn_lds_t*)(Vdst + (wave * KI + i) * 64), 16, 0, 0);
    }
  };
  // V^T fragment of dims 16b .. 16b+15 and k-step s (8 keys per lane)
  auto v_frag = [&](const uint4* Vc, int s, int b) {
    const int cc = 2 * (b & 3) + (vsub >> 1);
    const uint4* base = Vc + (b >> 2) * TK * 8;
    const int r0 = 32 * s + vrow, r1 = r0 + 16;
    const char* p0 = reinterpret_cast<const char*>(base + r0 * 8 + vlds_pos(r0, cc)) + 8 * (vsub & 1);
    const char* p1 = reinterpret_cast<const char*>(base + r1 * 8 + vlds_pos(r1, cc)) + 8 * (vsub & 1);
    const v4i16_t t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)p0);
    const v4i16_t t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)p1);
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(t0, t1, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // one tile: products on buffer BUF while tile t+1 loads into the other
  auto step = [&](int BUF, int t) {
    const uint4* Kc = Ks[BUF];
    const uint4* Vc = Vs[BUF];
    const bool more = t + 1 < ntiles;
    if (more) {
      issue_k(t + 1, Ks[BUF ^ 1]);
      issue_v(t + 1, Vs[BUF ^ 1]);
    }
    const int k0 = t * TK;
    // S^T for 4 blocks of 16 keys x 16 queries.  The matrix-product runs
    // raise the wave's issue priority: of the two waves sharing a SIMD, the
    // one with products to issue goes first while the other runs its
    // softmax (1-2 % at 4096-8192 keys)
    __builtin_amdgcn_s_setprio(1);
    f32x4_t sc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) sc[kb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        // k-step outer, key block inner: consecutive products go to the
        // four independent accumulators (each one's order of terms, and so
        // its bits, as with the key block outer)
        const bf16x8_t kf = __builtin_bit_cast(
            bf16x8_t, Kc[(ks >> 1) * TK * 8 + kb * 16 * 8 + ((ks & 1) ? kfr1 : kfr0)]);
        sc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qhi[ks], sc[kb], 0, 0, 0);
        sc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qlo[ks], sc[kb], 0, 0, 0);
      }
    __builtin_amdgcn_s_setprio(0);
    // online softmax per query; p in place of the scores.  Only a tile that
    // reaches past this wave's first query or past the prompt needs masking.
    const bool masked = k0 + TK - 1 > q0 || k0 + TK > T;
    {
      const int qi = q0 + c;
      float mx = m;
      if (masked) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = k0 + 16 * kb + 4 * j + r;
            if (key > qi || key >= T) sc[kb][r] = -INFINITY;
          }
      }
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[kb][r]);
      mx = xor32_max(xor16_max(mx));
      // a query sees key 0 in the first tile, so mx is finite from then on
      const float corr = __builtin_amdgcn_exp2f(m - mx);
      float ps = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = __builtin_amdgcn_exp2f(sc[kb][r] - mx);
          sc[kb][r] = p;
          ps += p;
        }
      ps = xor32_sum(xor16_sum(ps));
      // the output rescale is skipped when no query of the wave has a new
      // maximum (corr = 1 for all of them, so nothing changes)
      const bool grew = __builtin_amdgcn_ballot_w64(mx != m) != 0;
      l = l * corr + ps;
      m = mx;
      if (grew) {
#pragma unroll
        for (int b = 0; b < HB; ++b) o[b] *= corr;
      }
    }
    // O^T += V^T P^T, two k-steps of 32 keys
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x8_t phi, plo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bf16_t hb, lb;
        split_hi_lo(sc[2 * s + (e >> 2)][e & 3], hb, lb);
        phi[e] = __builtin_bit_cast(__bf16, hb);
        plo[e] = __builtin_bit_cast(__bf16, lb);
      }
      // two row blocks at a time: both V fragment reads in flight, the hi
      // products of both, then the lo products (per accumulator the same
      // order of terms)
#pragma unroll
      for (int b = 0; b < HB; b += 2) {
        const bf16x8_t v0 = v_frag(Vc, s, b);
        const bf16x8_t v1 = v_frag(Vc, s, b + 1);
        o[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v0, phi, o[b], 0, 0, 0);
        o[b + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v1, phi, o[b + 1], 0, 0, 0);
        o[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v0, plo, o[b], 0, 0, 0);
        o[b + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v1, plo, o[b + 1], 0, 0, 0);
      }
    }
    // the next tile's direct K and V loads have landed for this wave, then
    // (the barrier) for all
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  // the first tile's K and V go out before the queries are formed, so the
  // two prologue latencies overlap
  issue_k(0, Ks[0]);
  issue_v(0, Vs[0]);
  {
    const int qi = q0 + c;
    const float* qp = a.q + (int64_t)(g * a.Q + (qi < T ? qi : T - 1)) * a.q_ld + h * HD + 8 * j;
    const bool vec = ((reinterpret_cast<uintptr_t>(a.q) | ((uintptr_t)a.q_ld * sizeof(float))) & 15) == 0;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      float x[8];
      if (vec) {
        const float4 v0 = *reinterpret_cast<const float4*>(qp + 32 * ks);
        const float4 v1 = *reinterpret_cast<const float4*>(qp + 32 * ks + 4);
        x[0] = v0.x; x[1] = v0.y; x[2] = v0.z; x[3] = v0.w;
        x[4] = v1.x; x[5] = v1.y; x[6] = v1.z; x[7] = v1.w;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = qp[32 * ks + e];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bf16_t hb, lb;
        split_hi_lo(qi < T ? x[e] * scale2 : 0.f, hb, lb);
        qhi[ks][e] = __builtin_bit_cast(__bf16, hb);
        qlo[ks][e] = __builtin_bit_cast(__bf16, lb);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) step(t & 1, t);

  // lane holds O^T[dims 16b + 4j + r][query c]
  bf16_t* out = reinterpret_cast<bf16_t*>(a.out);
  const int qi = q0 + c;
  if (qi < T) {
    const float inv = 1.f / l;
#pragma unroll
    for (int b = 0; b < HB; ++b) {
      uint2 pk;
      pk.x = (uint32_t)f2bf(o[b][0] * inv) | ((uint32_t)f2bf(o[b][1] * inv) << 16);
      pk.y = (uint32_t)f2bf(o[b][2] * inv) | ((uint32_t)f2bf(o[b][3] * inv) << 16);
      *reinterpret_cast<uint2*>(out + (int64_t)(g * a.Q + qi) * a.out_ld + h * HD + 16 * b + 4 * j) = pk;
    }
  }
}

template <typename T, int HD>
hipError_t decode_hd(const AttnCall& a, hipStream_t st) {
  const float scale = 1.0f / sqrtf((float)HD);
  dim3 grid(a.G * a.H * a.nsplit), block(256);
  switch (a.Q) {
    case 1:
      // long caches: 32 row slots x 8 keys in flight per workgroup; short
      // ones: 16 slots x 6 keys, so that the last pass over the keys is not
      // nearly empty and more workgroups share the chip.  A long cache's
      // step that forms q inside (one round of workgroups) takes 6 keys per
      // slot with the first pass issued early: 8 keys plus the early pass
      // need 148 registers, one workgroup per CU instead of two
      if (a.cap >= 1024 && a.qkv)
        PH_LAUNCH((attn_decode_kernel<T, HD, 1, 6, 32, true>), grid, dim3(512), 0, st, a, scale);
      else if (a.cap >= 1024)
        PH_LAUNCH((attn_decode_kernel<T, HD, 1, 8, 32>), grid, dim3(512), 0, st, a, scale);
      else
        PH_LAUNCH((attn_decode_kernel<T, HD, 1, 6>), grid, block, 0, st, a, scale);
      break;
    case 2: PH_LAUNCH((attn_decode_kernel<T, HD, 2, 4>), grid, block, 0, st, a, scale); break;
    case 4: PH_LAUNCH((attn_decode_kernel<T, HD, 4, 4>), grid, block, 0, st, a, scale); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;
  PH_LAUNCH((attn_combine_kernel<T, HD>), a.G * a.H * a.Q, 64, 0, st, a);
  return hipGetLastError();
}

template <typename T, int HD>
hipError_t chunk_hd(const AttnCall& a, hipStream_t st, int maxl) {
  const float scale = 1.0f / sqrtf((float)HD);
  dim3 grid((a.G * a.H + 15) / 16), block(256);
  if (maxl <= 2) PH_LAUNCH((attn_chunk_kernel<T, HD, 2>), grid, block, 0, st, a, scale);
  else if (maxl <= 4) PH_LAUNCH((attn_chunk_kernel<T, HD, 4>), grid, block, 0, st, a, scale);
  else if (maxl <= 8) PH_LAUNCH((attn_chunk_kernel<T, HD, 8>), grid, block, 0, st, a, scale);
  else if (maxl <= 16) PH_LAUNCH((attn_chunk_kernel<T, HD, 16>), grid, block, 0, st, a, scale);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

template <typename T, int HD>
hipError_t prefill_hd(const AttnCall& a, hipStream_t st) {
  const float scale = 1.0f / sqrtf((float)HD);
  if constexpr (sizeof(T) == 2 && HD % 32 == 0) {
    // bf16 caches: MFMA kernel, 16 queries per wave, 8 waves (two per SIMD,
    // so one's softmax overlaps the other's matrix products) sharing each
    // staged K/V tile: half the LDS fills per query of 4 waves
    constexpr int kWaves = 8;
    const int nqb = (a.Q + 16 * kWaves - 1) / (16 * kWaves);
    PH_LAUNCH((attn_prefill_mfma_kernel<HD, kWaves>), a.G * a.H * nqb, 64 * kWaves, 0, st, a, scale);
  } else {
    const int nqb = (a.Q + 63) / 64;
    PH_LAUNCH((attn_prefill_kernel<T, HD>), a.G * a.H * nqb, 256, 0, st, a, scale);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch_decode(const AttnCall& a, hipStream_t st) {
  switch (a.hd) {
    case 32: return decode_hd<T, 32>(a, st);
    case 64: return decode_hd<T, 64>(a, st);
    case 96: return decode_hd<T, 96>(a, st);
    case 128: return decode_hd<T, 128>(a, st);
    default: return hipErrorInvalidValue;
  }
}
template <typename T>
hipError_t dispatch_chunk(const AttnCall& a, hipStream_t st, int maxl) {
  switch (a.hd) {
    case 32: return chunk_hd<T, 32>(a, st, maxl);
    case 64: return chunk_hd<T, 64>(a, st, maxl);
    case 96: return chunk_hd<T, 96>(a, st, maxl);
    case 128: return chunk_hd<T, 128>(a, st, maxl);
    default: return hipErrorInvalidValue;
  }
}
template <typename T>
hipError_t dispatch_prefill(const AttnCall& a, hipStream_t st) {
  switch (a.hd) {
    case 32: return prefill_hd<T, 32>(a, st);
    case 64: return prefill_hd<T, 64>(a, st);
    case 96: return prefill_hd<T, 96>(a, st);
    case 128: return prefill_hd<T, 128>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool attn_decode_rope_inside(int G, int H, int cap, int nsplit) {
  // the forming of q (counter -> RoPE table -> QKV slabs) sits before every
  // workgroup's first scores: paid once by a launch whose workgroups are all
  // resident at once (short caches: 4 per CU; long: 2 per CU of 512
  // threads), once per round by a longer one, where a launch of its own is
  // cheaper
  return cap < 1024 || (int64_t)G * H * nsplit <= 2 * 256;
}

int attn_decode_splits(int G, int H, int cap, int Q) {
  const int pairs = G * H;
  if (Q == 1) {
    // one workgroup per (sequence, head) streams its whole cache once there
    // are enough pairs to fill the chip (measured: no split beats split +
    // combine from 256 pairs up); below that, split to ~256 workgroups
    if (pairs >= 128) return 1;
    int ns = (256 + pairs - 1) / pairs;
    const int max_ns = (cap + 255) / 256;
    return ns < 1 ? 1 : (ns > max_ns ? (max_ns < 1 ? 1 : max_ns) : ns);
  }
  // several queries per sequence (HierGen level-1 step): one round of
  // resident workgroups (~5 per CU), splits of at least 128 keys
  const int resident = 256 * 5;
  int ns = (resident + pairs / 2) / pairs;
  const int max_ns = (cap + 127) / 128;
  if (ns > max_ns) ns = max_ns;
  if (ns < 1) ns = 1;
  return ns;
}

hipError_t launch_attn_decode(const AttnCall& a, hipStream_t st) {
  return a.dtype ? dispatch_decode<bf16_t>(a, st) : dispatch_decode<float>(a, st);
}

hipError_t launch_attn_chunk(const AttnCall& a, hipStream_t st) {
  const int maxl = a.L_dev ? a.cap : a.L_host;
  return a.dtype ? dispatch_chunk<bf16_t>(a, st, maxl) : dispatch_chunk<float>(a, st, maxl);
}

hipError_t launch_attn_prefill(const AttnCall& a, hipStream_t st) {
  return a.dtype ? dispatch_prefill<bf16_t>(a, st) : dispatch_prefill<float>(a, st);
}

}  // namespace photon
