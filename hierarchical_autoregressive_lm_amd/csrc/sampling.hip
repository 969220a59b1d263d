// Sampling decode and multi-query aggregation.
//
// The PHOTON explainer's paragraph on quality recovery runs several slightly
// varied queries and binds them by majority vote or best-of-N.  Here the
// variation is stochastic decoding: each row of logits draws one id as the
// first maximum of logit / temperature + Gumbel noise over the ids a top-k
// cut keeps (every id whose logit reaches the k-th largest), which samples
// the tempered softmax restricted to them (the Gumbel-max identity).  The
// noise comes from Philox-4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel
// Random Numbers: As Easy as 1, 2, 3", SC 2011) keyed by the seed, counter
// (id / 4, absolute token position, sequence, 0), word id % 4, mapped to
// u = ((word >> 9) + 1/2) * 2^-23, exact in float32.
//
// One workgroup of 1024 threads per row keeps the row in registers (4*Q
// consecutive ids per thread, Q <= 16: vocabularies up to 65536), finds
// the row maximum and log-sum-exp, finds the k-th largest logit exactly by
// a 2-bits-per-pass search over order-preserving 32-bit keys (16 block
// counts), then reduces the perturbed scores of the kept ids.
#include "common.h"
#include "kernels.h"

namespace photon {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kCap = kThreads;   // band keys listed in LDS, one per thread
constexpr int kSmall = 64;       // band keys one wave ranks directly

// Philox-4x32 with 10 rounds: words 0 and 2 are multiplied by the two round
// constants; the high halves of the products are mixed with words 1 and 3
// and the round key; the key grows by the two Weyl increments per round.
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c.x;   // one 32x32 -> 64 multiply each
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
    c = make_uint4((uint32_t)(p1 >> 32) ^ c.y ^ k0, (uint32_t)p1, (uint32_t)(p0 >> 32) ^ c.w ^ k1, (uint32_t)p0);
  }
  return c;
}

// float -> unsigned key with the same order (-0 is folded into +0 first)
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t b = __float_as_uint(x + 0.0f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ uint32_t wave_min_u(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o, 64));
  return v;
}

// One band-search step: the counts n1 <= ... of keys >= the three
// candidates c1 < c2 < c3 pick the highest candidate still reached by k keys.
__device__ __forceinline__ void band_step(int n1, int n2, int n3, uint32_t c1, uint32_t c2, uint32_t c3, int k,
                                          uint32_t& t, int& nt, int& nu) {
  if (n3 >= k) { t = c3; nt = n3; }
  else if (n2 >= k) { t = c2; nt = n2; nu = n3; }
  else if (n1 >= k) { t = c1; nt = n1; nu = n2; }
  else { nu = n1; }
}

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Block reductions over the 16 waves; `buf` alternates between two halves so
// that one barrier per reduction suffices.
struct BlockRed {
  float* f;   // [2][kWaves]
  int* n;     // [2][3][kWaves]
  int par;
  __device__ float max(float v, int wave, int lane) {
    v = wave_max(v);
    float* b = f + par * kWaves;
    par ^= 1;
    if (lane == 0) b[wave] = v;
    __syncthreads();
    float r = b[0];
#pragma unroll
    for (int i = 1; i < kWaves; ++i) r = fmaxf(r, b[i]);
    return r;
  }
  __device__ float sum(float v, int wave, int lane) {
    v = wave_sum(v);
    float* b = f + par * kWaves;
    par ^= 1;
    if (lane == 0) b[wave] = v;
    __syncthreads();
    float r = b[0];
#pragma unroll
    for (int i = 1; i < kWaves; ++i) r += b[i];
    return r;
  }
  __device__ void count3(int& a, int& bb, int& c, int wave, int lane) {
    a = wave_sum_i(a);
    bb = wave_sum_i(bb);
    c = wave_sum_i(c);
    int* b = n + par * 3 * kWaves;
    par ^= 1;
    if (lane == 0) {
      b[wave] = a;
      b[kWaves + wave] = bb;
      b[2 * kWaves + wave] = c;
    }
    __syncthreads();
    a = bb = c = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
      a += b[i];
      bb += b[kWaves + i];
      c += b[2 * kWaves + i];
    }
  }
};

template <int Q>
__global__ __launch_bounds__(kThreads) void sample_kernel(SampleCall c) {
  __shared__ float redf[2 * kWaves];
  __shared__ int redn[2 * 3 * kWaves];
  __shared__ float arg_s[kWaves], arg_x[kWaves];
  __shared__ int arg_i[kWaves];
  __shared__ uint32_t cand[kCap], small[kSmall], t_sh;
  __shared__ int n_list[2];
  const int r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) n_list[0] = n_list[1] = 0;   // visible after the first block reduction
  const int V = c.V;
  const float* row = c.logits + (int64_t)r * c.ld;
  const bool vec = (c.ld % 4 == 0) && (reinterpret_cast<uintptr_t>(c.logits) % 16 == 0);
  BlockRed red{redf, redn, 0};

  // ids 4*(tid + kThreads*q) + w.  Up to 8 groups of 4 stay in registers;
  // past 32768 ids the other groups go to LDS, one float4 per thread and
  // group (consecutive threads, consecutive 16 bytes), and every pass visits
  // them in a rolled loop, so that a 1024-thread block keeps within its 128
  // registers per lane instead of spilling.
  constexpr int QR = Q <= 8 ? Q : 8, QL = Q - QR;
  __shared__ float4 xl[QL > 0 ? QL : 1][QL > 0 ? kThreads : 1];
  float xr[QR][4];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int base = 4 * (tid + kThreads * q);
    float4 v;
    if (vec && base + 3 < V) {
      v = *reinterpret_cast<const float4*>(row + base);
    } else {
      v.x = base < V ? row[base] : -INFINITY;
      v.y = base + 1 < V ? row[base + 1] : -INFINITY;
      v.z = base + 2 < V ? row[base + 2] : -INFINITY;
      v.w = base + 3 < V ? row[base + 3] : -INFINITY;
    }
    if (q < QR) {
      xr[q < QR ? q : 0][0] = v.x; xr[q < QR ? q : 0][1] = v.y;
      xr[q < QR ? q : 0][2] = v.z; xr[q < QR ? q : 0][3] = v.w;
    } else {
      xl[q < QR ? 0 : q - QR][tid] = v;   // read back by this thread only
    }
  }
  // f(q, x) for every group q of this thread, x its 4 values in id order
  auto each = [&](auto&& f) {
#pragma unroll
    for (int q = 0; q < QR; ++q) f(q, xr[q]);
#pragma unroll 1
    for (int q = QR; q < Q; ++q) {
      const float4 v = xl[q - QR][tid];
      const float x[4] = {v.x, v.y, v.z, v.w};
      f(q, x);
    }
  };

  // log-sum-exp of the row (the model's distribution, temperature 1)
  float m = -INFINITY;
  each([&](int, const float* x) {
#pragma unroll
    for (int w = 0; w < 4; ++w) m = fmaxf(m, x[w]);
  });
  m = red.max(m, wave, lane);
  float s = 0.f;
  each([&](int, const float* x) {
#pragma unroll
    for (int w = 0; w < 4; ++w) s += __expf(x[w] - m);   // padding: exp(-inf) = 0
  });
  s = red.sum(s, wave, lane);
  const float lse = m + logf(s);

  // The cut t = the k-th largest key (ids with key >= t are kept).  Band
  // search two bits a pass from the top: before the pass at bit b the k-th
  // largest key lies in the band [t, t + 2^(b+2)), with nt = #(key >= t) >= k
  // and nu = #(key >= band top) < k.  While the band is wide every element is
  // counted from registers; once it holds <= kCap keys they are listed in LDS
  // (one per thread) and the passes count that list; once <= kSmall remain,
  // one wave ranks them directly: a key is kept iff fewer than k keys are
  // strictly greater.  Padding ids are never counted.
  const bool cut = c.top_k > 0 && c.top_k < V;
  const int k = c.top_k;
  uint32_t t = 0;
  if (cut) {
    int nt = V, nu = 0, b = 30;
    const uint32_t kmax = order_key(m);   // no key exceeds the row maximum's
    for (; b >= 0 && nt - nu > kCap; b -= 2) {
      const uint32_t c1 = t | (1u << b), c2 = t | (2u << b), c3 = t | (3u << b);
      if (c1 > kmax) {   // every candidate above the maximum: digit 0, nothing to count
        band_step(0, 0, 0, c1, c2, c3, k, t, nt, nu);
        continue;
      }
      int n1 = 0, n2 = 0, n3 = 0;
      each([&](int q, const float* x) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t key = 4 * (tid + kThreads * q) + w < V ? order_key(x[w]) : 0u;
          n1 += key >= c1;
          n2 += key >= c2;
          n3 += key >= c3;
        }
      });
      red.count3(n1, n2, n3, wave, lane);
      band_step(n1, n2, n3, c1, c2, c3, k, t, nt, nu);
    }
    if (b >= 0) {
      // list the band's keys (nt - nu <= kCap of them)
      const uint64_t top = (uint64_t)t + (4ull << b);
      each([&](int q, const float* x) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t key = order_key(x[w]);
          if (4 * (tid + kThreads * q) + w < V && key >= t && (uint64_t)key < top) cand[atomicAdd(&n_list[0], 1)] = key;
        }
      });
      __syncthreads();
      const int n = n_list[0];
      const uint32_t mine = tid < n ? cand[tid] : 0u;
      const int nu0 = nu;   // keys above the listed band
      for (; b >= 0 && nt - nu > kSmall; b -= 2) {
        const uint32_t c1 = t | (1u << b), c2 = t | (2u << b), c3 = t | (3u << b);
        int n1 = tid < n && mine >= c1, n2 = tid < n && mine >= c2, n3 = tid < n && mine >= c3;
        red.count3(n1, n2, n3, wave, lane);
        band_step(nu0 + n1, nu0 + n2, nu0 + n3, c1, c2, c3, k, t, nt, nu);
      }
      if (b >= 0) {
        const uint64_t top2 = (uint64_t)t + (4ull << b);
        if (tid < n && mine >= t && (uint64_t)mine < top2) small[atomicAdd(&n_list[1], 1)] = mine;
        __syncthreads();
        if (wave == 0) {
          const int m2 = n_list[1];
          const uint32_t kk = lane < m2 ? small[lane] : 0u;
          int greater = 0;
          for (int j = 0; j < m2; ++j) greater += small[j] > kk;
          const uint32_t tk = wave_min_u(lane < m2 && nu + greater < k ? kk : 0xFFFFFFFFu);
          if (lane == 0) t_sh = tk;
        }
        __syncthreads();
        t = t_sh;
      }
    }
  }

  // this row's sequence and absolute token position
  int seq, pos;
  if (c.seq) {
    seq = c.seq[r];
    pos = c.pos[r];
  } else {
    const int S = c.C1 * c.C2;
    seq = r / c.C2;
    pos = *c.counter * S + (r % c.C2) * c.C1 + c.j;
  }

  // Gumbel-max over the kept ids: first maximum of x / T + g, with
  // g = -log(E), E = -log(u): E keeps full relative accuracy through the
  // library log (u near 1 gives the small E that win); the outer log only
  // needs absolute accuracy
  const float inv_t = 1.0f / c.temperature;
  float best = -INFINITY, bx = 0.f;
  int bi = 0x7fffffff;
  each([&](int q, const float* x) {
    const int base = 4 * (tid + kThreads * q);
    if (base >= V) return;
    bool any = false;
#pragma unroll
    for (int w = 0; w < 4; ++w) any |= base + w < V && (!cut || order_key(x[w]) >= t);
    if (!any) return;
    const uint4 rw = philox4x32_10(make_uint4((uint32_t)(base / 4), (uint32_t)pos, (uint32_t)seq, 0u), c.k0, c.k1);
    const uint32_t word[4] = {rw.x, rw.y, rw.z, rw.w};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int v = base + w;
      if (v >= V || (cut && order_key(x[w]) < t)) continue;
      const float u = ((float)(word[w] >> 9) + 0.5f) * 0x1p-23f;
      const float sc = x[w] * inv_t - __logf(-logf(u));
      if (sc > best) { best = sc; bi = v; bx = x[w]; }
    }
  });
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float os = __shfl_xor(best, o, 64), ox = __shfl_xor(bx, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    if (os > best || (os == best && oi < bi)) { best = os; bi = oi; bx = ox; }
  }
  if (lane == 0) { arg_s[wave] = best; arg_i[wave] = bi; arg_x[wave] = bx; }
  __syncthreads();
  if (tid == 0) {
    for (int i = 1; i < kWaves; ++i)
      if (arg_s[i] > best || (arg_s[i] == best && arg_i[i] < bi)) { best = arg_s[i]; bi = arg_i[i]; bx = arg_x[i]; }
    bi = bi < V ? bi : 0;
    if (!c.seq) {
      const int p = (r % c.C2) * c.C1 + c.j;
      if (p < c.given_r) {   // a given token (ragged prompt tail): no draw
        bi = c.given[(int64_t)(r / c.C2) * c.C1 * c.C2 + p];
        bx = row[bi];
      }
    }
    c.ids[r] = bi;
    if (c.val) c.val[r] = best;
    if (c.logprob) {
      int64_t li = r;
      if (!c.seq) li = (int64_t)(r / c.C2) * c.C1 * c.C2 + (r % c.C2) * c.C1 + c.j;
      c.logprob[li] = bx - lse;
    }
  }
}

// One workgroup per group of queries: summed log-likelihood per member (one
// wave per member, fixed reduction order), pairwise answer equality, then
// best-of-N and the majority answer.
__global__ __launch_bounds__(256) void aggregate_kernel(AggregateCall c) {
  __shared__ float sc[64];
  __shared__ unsigned long long eq[64];
  const int g = blockIdx.x;
  const int m0 = g * c.group;
  const int nm = min(c.group, c.B - m0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < 64) eq[tid] = 0ull;
  for (int m = wave; m < nm; m += 4) {
    const float* lp = c.logprobs + (int64_t)(m0 + m) * c.lp_ld;
    float s = 0.f;
    for (int t = lane; t < c.n_tok; t += 64) s += lp[t];
    s = wave_sum(s);
    if (lane == 0) {
      sc[m] = s;
      if (c.score) c.score[m0 + m] = s;
    }
  }
  __syncthreads();
  const int npairs = nm * (nm - 1) / 2;
  for (int p = tid; p < npairs; p += 256) {
    int a = 0, rem = p;
    while (rem >= nm - 1 - a) { rem -= nm - 1 - a; ++a; }
    const int b = a + 1 + rem;
    const int* ta = c.tokens + (int64_t)(m0 + a) * c.tok_ld;
    const int* tb = c.tokens + (int64_t)(m0 + b) * c.tok_ld;
    bool same = true;
    for (int t = c.span0; t < c.span1 && same; ++t) same = ta[t] == tb[t];
    if (same) {
      atomicOr(&eq[a], 1ull << b);
      atomicOr(&eq[b], 1ull << a);
    }
  }
  __syncthreads();
  if (tid == 0) {
    int best = 0, major = 0, mv = __popcll(eq[0]) + 1;
    for (int m = 1; m < nm; ++m) {
      if (sc[m] > sc[best]) best = m;
      const int v = __popcll(eq[m]) + 1;
      if (v > mv || (v == mv && sc[m] > sc[major])) { major = m; mv = v; }
    }
    c.best[g] = best;
    c.major[g] = major;
    c.votes[g] = mv;
  }
}

}  // namespace

int sample_supported(int V) { return V >= 1 && V <= 4 * kThreads * 16; }

hipError_t launch_sample(const SampleCall& c, hipStream_t st) {
  const int Q = (c.V + 4 * kThreads - 1) / (4 * kThreads);
  if (Q <= 1) PH_LAUNCH(sample_kernel<1>, c.rows, kThreads, 0, st, c);
  else if (Q <= 2) PH_LAUNCH(sample_kernel<2>, c.rows, kThreads, 0, st, c);
  else if (Q <= 4) PH_LAUNCH(sample_kernel<4>, c.rows, kThreads, 0, st, c);
  else if (Q <= 8) PH_LAUNCH(sample_kernel<8>, c.rows, kThreads, 0, st, c);
  else PH_LAUNCH(sample_kernel<16>, c.rows, kThreads, 0, st, c);
  return hipGetLastError();
}

hipError_t launch_aggregate(const AggregateCall& c, hipStream_t st) {
  const int groups = (c.B + c.group - 1) / c.group;
  PH_LAUNCH(aggregate_kernel, groups, 256, 0, st, c);
  return hipGetLastError();
}

}  // namespace photon
