// Row-wise and gather kernels of the PHOTON path: RMSNorm, rotary embedding
// with K/V cache append, embedding gather / conditioning add, the greedy
// argmax reduction and small state updates.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace photon {
namespace {


// Block-wide sum for the row kernels (blockDim.x a multiple of 64, <= 1024),
// once per kernel (red is not reused): one barrier, ordering only LDS, so
// no global access before it has to complete first.
__device__ __forceinline__ float block_sum_once(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}

// Four consecutive outputs in the storage dtype, one store (8 bytes for
// bf16; the column is a multiple of 4 and rows are 16-byte aligned).
template <typename T>
__device__ __forceinline__ void store4(T* p, float a, float b, float c, float d) {
  if constexpr (sizeof(T) == 2) {
    uint2 pk;
    pk.x = (uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16);
    pk.y = (uint32_t)f2bf(c) | ((uint32_t)f2bf(d) << 16);
    *reinterpret_cast<uint2*>(p) = pk;
  } else {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
  }
}

// Row epilogue, one workgroup per output row i (input row r = i*row_stride
// + row_off), one float4 column group per thread:
//   x = resid[r] + sum_s P[s][r] + E[ids[r]]  (each term optional; slabs
//   summed in order), x_out[r] = x, a_out[i] = round(g * x / rms(x)).
template <typename T>
__global__ __launch_bounds__(1024) void rows_epilogue_kernel(RowsEpi e) {
  __shared__ float red[16];
  const int i = blockIdx.x;
  const int64_t r = (int64_t)i * e.row_stride + e.row_off;
  const int d = e.d;
  const int c = threadIdx.x * 4;
  const bool act = c < d;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (act) {
    if (e.resid) acc = *reinterpret_cast<const float4*>(e.resid + r * d + c);
    const float* pp = e.P + r * e.ldp + c;
    int s = 0;
    if (e.ksplit >= 8) {                  // eight slabs in flight, added in order
      float4 p[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) p[k] = *reinterpret_cast<const float4*>(pp + k * e.pstride);
#pragma unroll
      for (int k = 0; k < 8; ++k) { acc.x += p[k].x; acc.y += p[k].y; acc.z += p[k].z; acc.w += p[k].w; }
      s = 8;
    }
    for (; s + 4 <= e.ksplit; s += 4) {   // four slabs in flight, added in order
      const float4 p0 = *reinterpret_cast<const float4*>(pp + (s + 0) * e.pstride);
      const float4 p1 = *reinterpret_cast<const float4*>(pp + (s + 1) * e.pstride);
      const float4 p2 = *reinterpret_cast<const float4*>(pp + (s + 2) * e.pstride);
      const float4 p3 = *reinterpret_cast<const float4*>(pp + (s + 3) * e.pstride);
      acc.x += p0.x; acc.y += p0.y; acc.z += p0.z; acc.w += p0.w;
      acc.x += p1.x; acc.y += p1.y; acc.z += p1.z; acc.w += p1.w;
      acc.x += p2.x; acc.y += p2.y; acc.z += p2.z; acc.w += p2.w;
      acc.x += p3.x; acc.y += p3.y; acc.z += p3.z; acc.w += p3.w;
    }
    for (; s < e.ksplit; ++s) {
      const float4 p0 = *reinterpret_cast<const float4*>(pp + s * e.pstride);
      acc.x += p0.x; acc.y += p0.y; acc.z += p0.z; acc.w += p0.w;
    }
    if (e.ids) {
      const T* erow = reinterpret_cast<const T*>(e.E) + (int64_t)e.ids[r] * d;
      acc.x += St<T>::ld(erow[c]); acc.y += St<T>::ld(erow[c + 1]);
      acc.z += St<T>::ld(erow[c + 2]); acc.w += St<T>::ld(erow[c + 3]);
    }
  }
  // both stores after the row's sum: a store still in flight would hold
  // the reduction up (the wait before it counts stores too)
  if (!e.a_out) {                         // uniform across the block
    if (act && e.x_out) *reinterpret_cast<float4*>(e.x_out + r * d + c) = acc;
    return;
  }
  float ss = act ? acc.x * acc.x + acc.y * acc.y + acc.z * acc.z + acc.w * acc.w : 0.f;
  ss = block_sum_once(ss, red);
  const float inv = 1.0f / sqrtf(ss / (float)d + e.eps);
  if (act) {
    if (e.x_out) *reinterpret_cast<float4*>(e.x_out + r * d + c) = acc;
    T* orow = reinterpret_cast<T*>(e.a_out) + (int64_t)i * e.a_ld;
    const float4 gg = *reinterpret_cast<const float4*>(e.g + c);
    store4<T>(orow + c, gg.x * (acc.x * inv), gg.y * (acc.y * inv), gg.z * (acc.z * inv), gg.w * (acc.w * inv));
  }
}

// one thread per (row, head, rotation pair)
template <typename T>
__global__ __launch_bounds__(256) void rope_kv_kernel(RopeKvCall c) {
  const int half = c.hd / 2;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per_row = (int64_t)c.H * half;
  if (idx >= (int64_t)c.M * per_row) return;
  const int m = (int)(idx / per_row);
  const int rem = (int)(idx % per_row);
  const int h = rem / half, i = rem % half;
  const int s = m / c.rows_per_seq, t = m % c.rows_per_seq;
  const int pos = c.pos_add + (c.pos_dev ? (*c.pos_dev) * c.pos_mul : 0) + t;
  const float cs = c.rope[((int64_t)pos * half + i) * 2];
  const float sn = c.rope[((int64_t)pos * half + i) * 2 + 1];
  const int ca = h * c.hd + i, cb = ca + half;
  float qa = 0.f, qb = 0.f, ka = 0.f, kb = 0.f, va = 0.f, vb = 0.f;
  for (int sl = 0; sl < c.ksplit; ++sl) {      // K slabs of the QKV GEMM, in order
    const float* row = c.qkv + sl * c.pstride + (int64_t)m * 3 * c.d;
    qa += row[ca]; qb += row[cb];
    ka += row[c.d + ca]; kb += row[c.d + cb];
    va += row[2 * c.d + ca]; vb += row[2 * c.d + cb];
  }
  c.q_out[(int64_t)m * c.d + ca] = qa * cs - qb * sn;
  c.q_out[(int64_t)m * c.d + cb] = qb * cs + qa * sn;
  const int64_t off = (int64_t)(c.seq0 + s) * c.seq_stride + ((int64_t)h * c.cap + pos) * c.hd;
  T* K = reinterpret_cast<T*>(c.Kc) + off;
  T* V = reinterpret_cast<T*>(c.Vc) + off;
  K[i] = St<T>::st(ka * cs - kb * sn);
  K[i + half] = St<T>::st(kb * cs + ka * sn);
  V[i] = St<T>::st(va);
  V[i + half] = St<T>::st(vb);
}

// ids outside [0, V) are clamped so that a bad caller id cannot read past E
__device__ __forceinline__ int64_t clamp_id(int id, int V) { return id < 0 ? 0 : (id >= V ? V - 1 : id); }

// id i of the gathered list sits at ids[(i / L) * ld + i % L]
template <typename T>
__global__ __launch_bounds__(256) void embed_gather_kernel(const int* ids, int64_t n, int L, int64_t ld, const T* E,
                                                           int d, int V, T* out) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n * d) return;
  const int64_t r = idx / d;
  const int e = (int)(idx % d);
  out[idx] = E[clamp_id(ids[(r / L) * ld + r % L], V) * d + e];
}

// The same, 16 bytes per thread (rows of d storage elements, d * sizeof(T)
// a multiple of 16, E and out 16-byte aligned).
template <typename T>
__global__ __launch_bounds__(256) void embed_gather16_kernel(const int* ids, int64_t n, int L, int64_t ld,
                                                             const T* E, int d, int V, T* out) {
  constexpr int PER = 16 / sizeof(T);
  const int dv = d / PER;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n * dv) return;
  const int64_t r = idx / dv;
  const int e = (int)(idx % dv) * PER;
  *reinterpret_cast<uint4*>(out + r * d + e) =
      *reinterpret_cast<const uint4*>(E + clamp_id(ids[(r / L) * ld + r % L], V) * d + e);
}

__global__ __launch_bounds__(256) void copy_ids_kernel(int* dst, int64_t dst_ld, const int* src, int64_t src_ld,
                                                       int rows, int cols, int V) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)rows * cols) return;
  const int64_t r = idx / cols;
  const int i = (int)(idx % cols);
  dst[r * dst_ld + i] = (int)clamp_id(src[r * src_ld + i], V);
}

// Greedy head, step j: one workgroup per row m = b*C2 + k reduces the
// column tiles to the first maximum (lowest id on ties), writes the token
// and, when a next step exists, that step's decoder input
// x = c0[m][j+1] + E[token] and its first norm a = round(g * x / rms(x)).
template <typename T>
__global__ __launch_bounds__(1024) void argmax_next_kernel(ArgmaxNext c) {
  __shared__ float red[16];
  __shared__ float bvs[16];
  __shared__ int bis[16];
  const int m = blockIdx.x;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  float best = -INFINITY;
  int bi = 0x7fffffff;
  for (int t = threadIdx.x; t < c.n_tiles; t += blockDim.x) {
    const float v = c.val[(int64_t)t * c.M + m];
    const int ix = c.idx[(int64_t)t * c.M + m];
    if (v > best || (v == best && ix < bi)) { best = v; bi = ix; }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(best, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    if (ov > best || (ov == best && oi < bi)) { best = ov; bi = oi; }
  }
  if (lane == 0) { bvs[w] = best; bis[w] = bi; }
  __syncthreads();
  best = bvs[0]; bi = bis[0];
  for (int i = 1; i < nw; ++i)
    if (bvs[i] > best || (bvs[i] == best && bis[i] < bi)) { best = bvs[i]; bi = bis[i]; }
  // a row with no ordered maximum (every logit NaN) leaves the initial id:
  // take 0, so the token and the embedding row read below stay in range
  if ((unsigned)bi >= (unsigned)c.V) bi = 0;
  {
    const int b = m / c.C2, p = (m % c.C2) * c.C1 + c.j;
    if (p < c.given_r) bi = c.given[(int64_t)b * c.C1 * c.C2 + p];   // block-uniform
    if (threadIdx.x == 0) c.tokens[(int64_t)b * c.C1 * c.C2 + p] = bi;
  }
  if (!c.x) return;                      // uniform across the block
  const int d = c.d;
  const int col = threadIdx.x * 4;
  const bool act = col < d;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (act) {
    if (c.c0) acc = *reinterpret_cast<const float4*>(c.c0 + (int64_t)m * c.c0_ld + (int64_t)(c.j + 1) * d + col);
    const T* erow = reinterpret_cast<const T*>(c.E) + (int64_t)bi * d;
    acc.x += St<T>::ld(erow[col]); acc.y += St<T>::ld(erow[col + 1]);
    acc.z += St<T>::ld(erow[col + 2]); acc.w += St<T>::ld(erow[col + 3]);
  }
  float ss = act ? acc.x * acc.x + acc.y * acc.y + acc.z * acc.z + acc.w * acc.w : 0.f;
  ss = block_sum_once(ss, red);           // the stores after it (see rows_epilogue_kernel)
  const float inv = 1.0f / sqrtf(ss / (float)d + c.eps);
  if (act) {
    *reinterpret_cast<float4*>(c.x + (int64_t)m * d + col) = acc;
    T* orow = reinterpret_cast<T*>(c.a) + (int64_t)m * d;
    const float4 gg = *reinterpret_cast<const float4*>(c.g + col);
    orow[col + 0] = St<T>::st(gg.x * (acc.x * inv));
    orow[col + 1] = St<T>::st(gg.y * (acc.y * inv));
    orow[col + 2] = St<T>::st(gg.z * (acc.z * inv));
    orow[col + 3] = St<T>::st(gg.w * (acc.w * inv));
  }
}

__global__ void rope_table_kernel(float* tab, int max_pos, int hd, double theta) {
  const int half = hd / 2;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)max_pos * half) return;
  const int p = (int)(idx / half), i = (int)(idx % half);
  const double ang = (double)p * pow(theta, -2.0 * (double)i / (double)hd);
  tab[idx * 2] = (float)cos(ang);
  tab[idx * 2 + 1] = (float)sin(ang);
}

__global__ void set_int_kernel(int* p, int v) { *p = v; }
__global__ void zero_ints_kernel(int* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}
__global__ void add_int_kernel(int* p, int v) { *p += v; }

inline unsigned blocks(int64_t n) { return (unsigned)((n + 255) / 256); }

// Cosine distance of row pairs, one wave per row: 1 - a.e / (|a| |e|) with
// float32 sums of the stored values.
template <typename T>
__global__ __launch_bounds__(256) void cosine_distance_kernel(const T* a, const T* e, int R, int d, float* out) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= R) return;
  const T* pa = a + (int64_t)row * d;
  const T* pe = e + (int64_t)row * d;
  float dot = 0.f, na = 0.f, ne = 0.f;
  for (int i = lane; i < d; i += 64) {
    const float x = St<T>::ld(pa[i]), y = St<T>::ld(pe[i]);
    dot = fmaf(x, y, dot);
    na = fmaf(x, x, na);
    ne = fmaf(y, y, ne);
  }
  dot = wave_sum(dot);
  na = wave_sum(na);
  ne = wave_sum(ne);
  if (lane == 0) out[row] = 1.0f - dot / (sqrtf(na) * sqrtf(ne));
}

}  // namespace

// threads for one row of d elements, one float4 each, whole waves
inline unsigned row_threads(int d) { return (unsigned)(((d / 4) + 63) / 64 * 64); }

hipError_t launch_rows_epilogue(int dtype, const RowsEpi& e, hipStream_t st) {
  if (e.d > 4096 || e.d % 4) return hipErrorInvalidValue;
  dim3 grid(e.R), block(row_threads(e.d));
  if (dtype) PH_LAUNCH((rows_epilogue_kernel<bf16_t>), grid, block, 0, st, e);
  else PH_LAUNCH((rows_epilogue_kernel<float>), grid, block, 0, st, e);
  return hipGetLastError();
}

hipError_t launch_rope_kv(const RopeKvCall& c, hipStream_t st) {
  const int64_t n = (int64_t)c.M * c.H * (c.hd / 2);
  if (c.dtype) PH_LAUNCH((rope_kv_kernel<bf16_t>), blocks(n), 256, 0, st, c);
  else PH_LAUNCH((rope_kv_kernel<float>), blocks(n), 256, 0, st, c);
  return hipGetLastError();
}

hipError_t launch_embed_gather_rows(int dtype, const int* ids, int64_t rows, int L, int64_t ld, const void* E, int d,
                                    int V, void* out, hipStream_t st) {
  const int64_t n = rows * L;
  if (n <= 0) return hipSuccess;
  const int eb = dtype ? 2 : 4;
  if ((d * eb) % 16 == 0 && (uintptr_t)E % 16 == 0 && (uintptr_t)out % 16 == 0) {
    const int64_t nv = n * (d * eb / 16);
    if (dtype)
      PH_LAUNCH((embed_gather16_kernel<bf16_t>), blocks(nv), 256, 0, st, ids, n, L, ld, (const bf16_t*)E, d, V,
                (bf16_t*)out);
    else
      PH_LAUNCH((embed_gather16_kernel<float>), blocks(nv), 256, 0, st, ids, n, L, ld, (const float*)E, d, V,
                (float*)out);
    return hipGetLastError();
  }
  if (dtype)
    PH_LAUNCH((embed_gather_kernel<bf16_t>), blocks(n * d), 256, 0, st, ids, n, L, ld, (const bf16_t*)E, d, V,
              (bf16_t*)out);
  else
    PH_LAUNCH((embed_gather_kernel<float>), blocks(n * d), 256, 0, st, ids, n, L, ld, (const float*)E, d, V,
              (float*)out);
  return hipGetLastError();
}

hipError_t launch_embed_gather(int dtype, const int* ids, int64_t n, const void* E, int d, int V, void* out,
                               hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (n > 0x7fffffff) return hipErrorInvalidValue;
  return launch_embed_gather_rows(dtype, ids, 1, (int)n, n, E, d, V, out, st);
}

hipError_t launch_copy_ids(int* dst, int64_t dst_ld, const int* src, int64_t src_ld, int rows, int cols, int V,
                           hipStream_t st) {
  const int64_t n = (int64_t)rows * cols;
  if (n <= 0) return hipSuccess;
  PH_LAUNCH((copy_ids_kernel), blocks(n), 256, 0, st, dst, dst_ld, src, src_ld, rows, cols, V);
  return hipGetLastError();
}

hipError_t launch_argmax_next(int dtype, const ArgmaxNext& c, hipStream_t st) {
  if (c.d > 4096 || c.d % 4) return hipErrorInvalidValue;
  dim3 grid(c.M), block(std::max(256u, row_threads(c.d)));
  if (dtype) PH_LAUNCH((argmax_next_kernel<bf16_t>), grid, block, 0, st, c);
  else PH_LAUNCH((argmax_next_kernel<float>), grid, block, 0, st, c);
  return hipGetLastError();
}

hipError_t launch_cosine_distance(int dtype, const void* a, const void* e, int R, int d, float* out, hipStream_t st) {
  const unsigned g = (unsigned)((R + 3) / 4);
  if (dtype) PH_LAUNCH((cosine_distance_kernel<bf16_t>), g, 256, 0, st, (const bf16_t*)a, (const bf16_t*)e, R, d, out);
  else PH_LAUNCH((cosine_distance_kernel<float>), g, 256, 0, st, (const float*)a, (const float*)e, R, d, out);
  return hipGetLastError();
}

hipError_t launch_rope_table(float* tab, int max_pos, int hd, float theta, hipStream_t st) {
  const int64_t n = (int64_t)max_pos * (hd / 2);
  PH_LAUNCH((rope_table_kernel), blocks(n), 256, 0, st, tab, max_pos, hd, (double)theta);
  return hipGetLastError();
}

hipError_t launch_set_int(int* p, int v, hipStream_t st) {
  PH_LAUNCH((set_int_kernel), 1, 1, 0, st, p, v);
  return hipGetLastError();
}

hipError_t launch_zero_ints(int* p, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  PH_LAUNCH((zero_ints_kernel), blocks(n), 256, 0, st, p, n);
  return hipGetLastError();
}

hipError_t launch_add_int(int* p, int v, hipStream_t st) {
  PH_LAUNCH((add_int_kernel), 1, 1, 0, st, p, v);
  return hipGetLastError();
}

}  // namespace photon
