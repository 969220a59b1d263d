// Row-wise and gather kernels of the PHOTON path: RMSNorm, rotary embedding
// with K/V cache append, embedding gather / conditioning add, the greedy
// argmax reduction and small state updates.
#include "common.h"
#include "kernels.h"

namespace photon {
namespace {

// one wave per row; fp32 sum of squares; output rounded to the storage type
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* x, int64_t in_stride, int64_t in_off,
                                                      const float* g, T* out, int rows, int d, float eps) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const float* xr = x + (row * in_stride + in_off) * (int64_t)d;
  float ss = 0.f;
  for (int e = lane * 4; e < d; e += 256) {
    const float4 v = *reinterpret_cast<const float4*>(xr + e);
    ss = fmaf(v.x, v.x, ss); ss = fmaf(v.y, v.y, ss);
    ss = fmaf(v.z, v.z, ss); ss = fmaf(v.w, v.w, ss);
  }
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / (float)d + eps);
  T* orow = out + (int64_t)row * d;
  for (int e = lane * 4; e < d; e += 256) {
    const float4 v = *reinterpret_cast<const float4*>(xr + e);
    const float4 gg = *reinterpret_cast<const float4*>(g + e);
    orow[e + 0] = St<T>::st(gg.x * (v.x * inv));
    orow[e + 1] = St<T>::st(gg.y * (v.y * inv));
    orow[e + 2] = St<T>::st(gg.z * (v.z * inv));
    orow[e + 3] = St<T>::st(gg.w * (v.w * inv));
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
  const float* row = c.qkv + (int64_t)m * 3 * c.d;
  const int ca = h * c.hd + i, cb = ca + half;
  const float qa = row[ca], qb = row[cb];
  const float ka = row[c.d + ca], kb = row[c.d + cb];
  const float va = row[2 * c.d + ca], vb = row[2 * c.d + cb];
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

template <typename T>
__global__ __launch_bounds__(256) void embed_gather_kernel(const int* ids, int64_t n, const T* E, int d, int V, T* out) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n * d) return;
  const int64_t r = idx / d;
  const int e = (int)(idx % d);
  out[idx] = E[clamp_id(ids[r], V) * d + e];
}

template <typename T>
__global__ __launch_bounds__(256) void embed_add_kernel(const float* c0, int64_t c0_ld, int j, const int* prev,
                                                        const T* E, int M, int d, float* x) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)M * d) return;
  const int m = (int)(idx / d), e = (int)(idx % d);
  float v = c0[(int64_t)m * c0_ld + (int64_t)j * d + e];
  if (j > 0) v += St<T>::ld(E[(int64_t)prev[m] * d + e]);
  x[idx] = v;
}

__global__ void argmax_finalize_kernel(const float* val, const int* idx, int n_tiles, int M, int C1, int C2, int j,
                                       int* tokens, int* prev) {
  const int m = blockIdx.x * blockDim.x + threadIdx.x;
  if (m >= M) return;
  float best = val[m];
  int bi = idx[m];
  for (int t = 1; t < n_tiles; ++t) {
    const float v = val[(int64_t)t * M + m];
    const int i = idx[(int64_t)t * M + m];
    if (v > best || (v == best && i < bi)) { best = v; bi = i; }
  }
  const int b = m / C2, k = m % C2;
  tokens[(int64_t)b * C1 * C2 + k * C1 + j] = bi;
  prev[m] = bi;
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
__global__ void add_int_kernel(int* p, int v) { *p += v; }

inline unsigned blocks(int64_t n) { return (unsigned)((n + 255) / 256); }

}  // namespace

hipError_t launch_rmsnorm(int dtype, const float* x, int64_t in_stride, int64_t in_off, const float* g, void* out,
                          int rows, int d, float eps, hipStream_t st) {
  dim3 grid((rows + 3) / 4), block(256);
  if (dtype) rmsnorm_kernel<bf16_t><<<grid, block, 0, st>>>(x, in_stride, in_off, g, (bf16_t*)out, rows, d, eps);
  else rmsnorm_kernel<float><<<grid, block, 0, st>>>(x, in_stride, in_off, g, (float*)out, rows, d, eps);
  return hipGetLastError();
}

hipError_t launch_rope_kv(const RopeKvCall& c, hipStream_t st) {
  const int64_t n = (int64_t)c.M * c.H * (c.hd / 2);
  if (c.dtype) rope_kv_kernel<bf16_t><<<blocks(n), 256, 0, st>>>(c);
  else rope_kv_kernel<float><<<blocks(n), 256, 0, st>>>(c);
  return hipGetLastError();
}

hipError_t launch_embed_gather(int dtype, const int* ids, int64_t n, const void* E, int d, int V, void* out,
                               hipStream_t st) {
  if (dtype) embed_gather_kernel<bf16_t><<<blocks(n * d), 256, 0, st>>>(ids, n, (const bf16_t*)E, d, V, (bf16_t*)out);
  else embed_gather_kernel<float><<<blocks(n * d), 256, 0, st>>>(ids, n, (const float*)E, d, V, (float*)out);
  return hipGetLastError();
}

hipError_t launch_embed_add(int dtype, const float* c0, int64_t c0_ld, int j, const int* prev, const void* E, int M,
                            int d, float* x, hipStream_t st) {
  const int64_t n = (int64_t)M * d;
  if (dtype) embed_add_kernel<bf16_t><<<blocks(n), 256, 0, st>>>(c0, c0_ld, j, prev, (const bf16_t*)E, M, d, x);
  else embed_add_kernel<float><<<blocks(n), 256, 0, st>>>(c0, c0_ld, j, prev, (const float*)E, M, d, x);
  return hipGetLastError();
}

hipError_t launch_argmax_finalize(const float* val, const int* idx, int n_tiles, int M, int C1, int C2, int j,
                                  int* tokens, int* prev, hipStream_t st) {
  argmax_finalize_kernel<<<(M + 255) / 256, 256, 0, st>>>(val, idx, n_tiles, M, C1, C2, j, tokens, prev);
  return hipGetLastError();
}

hipError_t launch_rope_table(float* tab, int max_pos, int hd, float theta, hipStream_t st) {
  const int64_t n = (int64_t)max_pos * (hd / 2);
  rope_table_kernel<<<blocks(n), 256, 0, st>>>(tab, max_pos, hd, (double)theta);
  return hipGetLastError();
}

hipError_t launch_set_int(int* p, int v, hipStream_t st) {
  set_int_kernel<<<1, 1, 0, st>>>(p, v);
  return hipGetLastError();
}

hipError_t launch_add_int(int* p, int v, hipStream_t st) {
  add_int_kernel<<<1, 1, 0, st>>>(p, v);
  return hipGetLastError();
}

}  // namespace photon
