// Launchers for the HIP kernels of the PHOTON decode path (gfx950).
// Every launcher enqueues on `st`, never synchronises and returns the
// launch status.  dtype: 0 = fp32 storage, 1 = bf16 storage.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace photon {

// Events that a tracer wants recorded by the kernel dispatches of one
// operation: `start` by its first kernel, `stop` by every kernel (the last
// one wins).  The dispatch itself records them (hipExtLaunchKernelGGL), so
// they time the kernels without marker packets between them.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
inline LaunchEvents& launch_events() {
  static thread_local LaunchEvents e;
  return e;
}

// Every kernel launch of the library goes through this macro.
#define PH_LAUNCH(kern, grid, block, shmem, st, ...)                                                  \
  do {                                                                                                 \
    photon::LaunchEvents& ev_ = photon::launch_events();                                               \
    if (ev_.stop) {                                                                                    \
      hipExtLaunchKernelGGL(kern, dim3(grid), dim3(block), shmem, st, ev_.start, ev_.stop, 0, __VA_ARGS__); \
      ev_.start = nullptr;                                                                             \
    } else {                                                                                           \
      hipLaunchKernelGGL(kern, dim3(grid), dim3(block), shmem, st, __VA_ARGS__);                      \
    }                                                                                                  \
  } while (0)

enum Epi { EPI_STORE = 0, EPI_ADD = 1, EPI_GELU = 2, EPI_ARGMAX = 3, EPI_ROPE = 4 };

// C[M,N] = A[M,K] W[N,K]^T with a fused epilogue:
//   STORE : C (fp32, row stride ldc) = acc
//   ADD   : C += acc                     (residual stream update)
//   GELU  : Cb (storage dtype, stride ldc) = round(gelu(acc))
//   ARGMAX: per-row (max, first index) over each column tile written to
//           amax_val/amax_idx [n_tiles][M]; logits stored to C if non-null.
//   With allow_split (STORE only) K may be cut into gemm_splits() slabs; slab
//   s then writes its raw partial sums to C + s*M*ldc and the consumer adds
//   the slabs in order (deterministic).
//   wide: prefer the 8-wave tiles where a shape has both (GEMMs on the
//   critical path; the others leave more of each CU to concurrent work).
struct GemmCall {
  int dtype;
  const void* A; int64_t lda;
  const void* W;           // [N][K] row-major, storage dtype
  int M, N, K;
  int epi;
  float* C; int64_t ldc;
  void* Cb;
  float* amax_val; int* amax_idx;
  int allow_split;
  int wide;
};
hipError_t launch_gemm(const GemmCall& g, hipStream_t st);
// K slabs launch_gemm uses for a STORE GEMM with allow_split (and wide) set.
int gemm_splits(int dtype, int M, int N, int K, int wide);
// Column tiles the ARGMAX epilogue produces for a GEMM of this shape.
int gemm_argmax_tiles(int dtype, int M, int N, int K);
// Host-side shape check: 0 when the GEMM kernels support (M, N, K).
int gemm_supported(int dtype, int M, int N, int K);

// Row epilogue of the GEMMs that feed a residual stream: for output row i
// (input row r = i*row_stride + row_off, i < R):
//   x = resid[r] + sum_{s<ksplit} P[s*pstride + r*ldp ..] + E[ids[r]]
// (resid, P, ids optional), x_out[r] = x (optional), and, if a_out is set,
// a_out[i*a_ld ..] = round(g * x / sqrt(mean(x^2) + eps)).  Rows have d
// (<= 4096, multiple of 4) fp32 elements.
struct RowsEpi {
  const float* P; int ksplit; int64_t pstride; int64_t ldp;
  const float* resid;
  const int* ids; const void* E;
  float* x_out;
  const float* g; void* a_out; int64_t a_ld;
  int R, d; int64_t row_stride, row_off;
  float eps;
};
hipError_t launch_rows_epilogue(int dtype, const RowsEpi& e, hipStream_t st);

// Positions: pos(t) = pos_add + (pos_dev ? *pos_dev * pos_mul : 0) + t for
// the t-th new row of a sequence; the K/V of that row go to cache slot pos.
struct RopeKvCall {
  int dtype;
  const float* qkv;        // ksplit slabs of [M][3d] fp32: q | k | v
  int ksplit; int64_t pstride;
  int M, d, H, hd;
  float* q_out;            // [M][d] fp32 rotated q
  void* Kc; void* Vc;      // cache planes [seq][H][cap][hd], storage dtype
  int64_t seq_stride;      // elements between sequences (H*cap*hd)
  int cap, rows_per_seq, seq0;
  int pos_add; const int* pos_dev; int pos_mul;
  const float* rope;       // [max_pos][hd/2][2] (cos, sin)
};
hipError_t launch_rope_kv(const RopeKvCall& c, hipStream_t st);

// QKV projection fused with launch_rope_kv's work: the GEMM g (A the
// normalized rows, W = Wqkv, N = 3d, no K slabs) writes rotated q to
// rc.q_out and rotated k and v, rounded to bf16, to the cache planes, with
// rc's row, sequence and position map, the device counter included
// (rc.qkv and rc.ksplit unused).  bf16 only, for prompt-sized GEMMs (M >=
// 2048; head size 64, 96 or 128) and decode steps of 64-512 rows (head
// size 64 or 96), an even number of heads in 3d and aligned buffers;
// gemm_qkv_rope_supported says whether a call qualifies.
int gemm_qkv_rope_supported(const GemmCall& g, const RopeKvCall& rc);
hipError_t launch_gemm_qkv_rope(const GemmCall& g, const RopeKvCall& rc, hipStream_t st);

// Attention of Q new queries per sequence over a K/V cache.  Query t of
// sequence g sees keys 0 .. L - Q + t, L = L_host or *L_dev*L_mul + L_add.
struct AttnCall {
  int dtype;
  int G, Q, H, hd;
  const float* q; int64_t q_ld;   // row g*Q + t, head h at column h*hd
  const void* Kc; const void* Vc; int64_t seq_stride; int cap; int seq0;
  int L_host; const int* L_dev; int L_mul; int L_add;
  void* out; int64_t out_ld;      // storage dtype, same row/col map as q
  float* part; int nsplit;        // decode split-K partials
  // Fused RoPE + K/V append (decode and chunk kernels, qkv != nullptr): the
  // Q new rows of group g are rows g*Q + t of the QKV GEMM's ksplit slabs
  // ([M][3d] fp32 each, q | k | v, pstride floats apart, summed in slab
  // order); q and k are rotated at position pos(t) = pos_add + (pos_dev ?
  // *pos_dev * pos_mul : 0) + t with the [pos][hd/2][2] (cos, sin) table
  // `rope`, K and V rounded to the storage dtype and written to cache slot
  // pos(t), which must be key L-Q+t; those keys are attended from
  // registers, and `q` is not read.
  const float* qkv; int ksplit; int64_t pstride; int d;
  const float* rope; int pos_add; const int* pos_dev; int pos_mul;
};
// Long caches: split over keys, then combine.  part holds
// G*H*Q*nsplit*(hd+2) floats when nsplit > 1.
hipError_t launch_attn_decode(const AttnCall& a, hipStream_t st);
// Short in-chunk caches (L <= 64).
hipError_t launch_attn_chunk(const AttnCall& a, hipStream_t st);
// Causal self-attention over a whole prompt (L = Q = rows per sequence).
hipError_t launch_attn_prefill(const AttnCall& a, hipStream_t st);

// out[i] = E[ids[i]] for i < n (storage dtype rows of length d); ids are
// clamped to [0, V)
hipError_t launch_embed_gather(int dtype, const int* ids, int64_t n,
                               const void* E, int d, int V, void* out,
                               hipStream_t st);
// The same over `rows` rows of L ids each, row r starting at ids + r*ld.
hipError_t launch_embed_gather_rows(int dtype, const int* ids, int64_t rows, int L, int64_t ld,
                                    const void* E, int d, int V, void* out, hipStream_t st);
// dst[r*dst_ld + i] = clamp(src[r*src_ld + i], 0, V-1) for i < cols, r < rows.
hipError_t launch_copy_ids(int* dst, int64_t dst_ld, const int* src, int64_t src_ld, int rows, int cols, int V,
                           hipStream_t st);
// Greedy head of token step j: reduce the ARGMAX tiles of row m = b*C2 + k
// to its token (tokens[b*S + k*C1 + j]); if x is set, also write the next
// step's input x[m] = c0[m*c0_ld + (j+1)*d ..] + E[token] (E[token] alone
// when c0 is null) and its norm a[m].
// Positions p = k*C1 + j < given_r take the token given[b*S + p] instead
// (the tail of a ragged prompt), ids already in [0, V).
struct ArgmaxNext {
  const float* val; const int* idx; int n_tiles, M, C1, C2, j;
  int* tokens;
  const float* c0; int64_t c0_ld; const void* E;
  float* x; void* a; const float* g; int d; float eps;
  const int* given; int given_r;
  int V;   // vocabulary: a reduced id outside [0, V) (all-NaN row) becomes 0
};
hipError_t launch_argmax_next(int dtype, const ArgmaxNext& c, hipStream_t st);
// out[r] = 1 - cos(a[r], e[r]) for R rows of d storage-dtype elements.
hipError_t launch_cosine_distance(int dtype, const void* a, const void* e, int R, int d, float* out, hipStream_t st);
// tab[p][i] = (cos, sin)(p * theta^(-2i/hd)), angles in double precision.
hipError_t launch_rope_table(float* tab, int max_pos, int hd, float theta,
                             hipStream_t st);
hipError_t launch_set_int(int* p, int v, hipStream_t st);
// p[0 .. n) = 0 with a kernel (also safe inside captured graphs).
hipError_t launch_zero_ints(int* p, int64_t n, hipStream_t st);
hipError_t launch_add_int(int* p, int v, hipStream_t st);

// Sampling: row r of logits [rows][ld] (vocab V <= 65536, sample_supported)
// draws ids[r] = first maximum over the top-k-kept ids (every id whose logit
// reaches the k-th largest; top_k = 0 or >= V keeps all) of
// logit / temperature + Gumbel(u), u from Philox-4x32-10 with key (k0, k1),
// counter (id / 4, pos, seq, 0), word id % 4, u = ((word >> 9) + 1/2) 2^-23.
// seq/pos per row from the arrays, or (decode layout, arrays null) row
// r = b*C2 + k: seq b, pos = *counter * C1*C2 + k*C1 + j.  val[r] (nullable)
// gets the perturbed score; logprob (nullable) the log-likelihood of the id
// under the whole-vocabulary softmax at temperature 1, at index r (arrays)
// or b*C1*C2 + k*C1 + j (decode layout).
struct SampleCall {
  const float* logits; int64_t ld;
  int rows, V;
  float temperature; int top_k; uint32_t k0, k1;
  const int* seq; const int* pos;
  const int* counter; int C1, C2, j;
  int* ids; float* val;
  float* logprob;
  const int* given; int given_r;   // decode layout: positions < given_r take given[b*S + p]
};
int sample_supported(int V);
hipError_t launch_sample(const SampleCall& c, hipStream_t st);

// Multi-query aggregation over groups of `group` (<= 64) consecutive
// sequences (the last group may be shorter): score[b] (nullable) = sum of
// logprobs[b][0 .. n_tok); per group g: best[g] = member with the highest
// score (lowest on ties), votes = members whose tokens[span0, span1) equal
// a member's, major[g] = the member with the most votes (then the higher
// score, then the lower index), votes[g] its count.
struct AggregateCall {
  const int* tokens; int64_t tok_ld;
  const float* logprobs; int64_t lp_ld;
  int B, group, n_tok, span0, span1;
  int* best; int* major; int* votes; float* score;
};
hipError_t launch_aggregate(const AggregateCall& c, hipStream_t st);

// Number of key splits the decode attention uses for G*H pairs with Q
// queries each over a cache of `cap` slots (plan-time, so one plan serves
// every length <= cap).
int attn_decode_splits(int G, int H, int cap, int Q);
// Whether a decode step's attention should form q and append the new K/V
// rows itself (AttnCall::qkv) rather than take them from a RoPE launch of
// their own: caches under 1024 slots, and longer ones whose G*H*nsplit
// workgroups are all resident at once.
bool attn_decode_rope_inside(int G, int H, int cap, int nsplit);

}  // namespace photon
