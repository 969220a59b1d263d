// Weight-streaming GEMMs for the PHOTON decode and prefill paths.
//
// C[M,N] = A[M,K] W[N,K]^T.  In decode, M is small (B or B*C2 rows) and the
// whole cost is streaming W from HBM once, so the kernel is organised around
// W: each workgroup owns a slab of W rows (output features) and keeps every
// activation row of its M tile in LDS, k-block by k-block.  bf16 operands go
// through v_mfma_f32_16x16x32_bf16 with W as the MFMA A operand (16 features
// x 32 k) and the activations as the B operand (32 k x 16 rows), so each
// lane ends with 4 consecutive features of one row and stores 16 bytes.
//
// Workgroup = 4 waves arranged WN (along N) x WK (along K).  Small M tiles
// use WK = 4 (each wave streams a quarter of every k-block, partial sums
// reduced through LDS at the end) so that narrow GEMMs still spread over
// many CUs; the largest M tile uses WK = 1.
#include "common.h"
#include "kernels.h"

namespace photon {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct GemmP {
  const bf16_t* A; int64_t lda;
  const bf16_t* W;
  int M, N, K;
  float* C; int64_t ldc;
  bf16_t* Cb;
  float* av; int* ai;
  int m_tiles, n_tiles;
  int ksplit; int64_t pstride;   // k slabs; elements between RAW slabs
};

template <int MB, int NI, int WK, int P, int EPI, int NKB, bool NTW>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmP p) {
  constexpr int WN = 4 / WK;
  constexpr int BM = 16 * MB;
  constexpr int BN = 16 * NI * WN;
  constexpr int KT = 64 * WK;             // k per iteration; 64 per wave
  constexpr int ROW = KT + 8;             // padded LDS row, bf16 elements
  constexpr int A_ELEMS = BM * ROW;
  constexpr int CHUNKS = BM * KT / 8;     // 16-byte A chunks per k-block
  constexpr int CH = (CHUNKS + 255) / 256;
  constexpr int RED = (WK > 1) ? (WK - 1) * WN * MB * NI * 4 * 64 : 0;
  constexpr int BYTES_A = 2 * A_ELEMS * 2;
  constexpr int BYTES = BYTES_A > RED * 4 ? BYTES_A : RED * 4;
  static_assert(P >= 2, "at least one k-block in flight");
  __shared__ __attribute__((aligned(16))) unsigned char smem[BYTES];
  bf16_t* As = reinterpret_cast<bf16_t*>(smem);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave % WN, wk = wave / WN;

  // XCD-aware tile order: consecutive workgroups land on different XCDs, so
  // give each XCD a contiguous run of tiles (M tiles of one W slab share L2).
  const int total = p.m_tiles * p.n_tiles;
  const int ks = blockIdx.x % p.ksplit;
  const int bid = blockIdx.x / p.ksplit;
  const int tile = (total % 8 == 0) ? (bid % 8) * (total / 8) + bid / 8 : bid;
  const int mt = tile % p.m_tiles, nt = tile / p.m_tiles;
  const int m0 = mt * BM, n0 = nt * BN;

  const int K = p.K, N = p.N, M = p.M;
  const int kl = (lane >> 4) * 8;
  const bf16_t* wp[NI];
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
    int row = n0 + wn * NI * 16 + ni * 16 + (lane & 15);
    row = row < N ? row : N - 1;          // clamp: columns >= N never stored
    wp[ni] = p.W + (int64_t)row * K + wk * 64 + kl;
  }

  f32x4 acc[MB][NI];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // Ring of P k-blocks: the A rows (global -> registers -> LDS, double
  // buffered in LDS) and this wave's W fragments (global -> registers).
  // k-block k lives in ring slot k % P; while block k is multiplied, the
  // loads of blocks k+1 .. k+P-1 are in flight.
  uint4 areg[P][CH];
  bf16x8 wreg[P][2][NI];
  auto load_a = [&](int kb, uint4 (&ar)[CH]) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = tid + i * 256;
      const int r = c / (KT / 8), c8 = c % (KT / 8);
      const int gm = m0 + r;
      if (c < CHUNKS && gm < M)
        ar[i] = *reinterpret_cast<const uint4*>(p.A + (int64_t)gm * p.lda + (int64_t)kb * KT + c8 * 8);
      else
        ar[i] = make_uint4(0, 0, 0, 0);
    }
  };
  auto store_a = [&](const uint4 (&ar)[CH], int buf) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = tid + i * 256;
      const int r = c / (KT / 8), c8 = c % (KT / 8);
      if (c < CHUNKS) *reinterpret_cast<uint4*>(As + buf * A_ELEMS + r * ROW + c8 * 8) = ar[i];
    }
  };
  auto load_w = [&](int kb, bf16x8 (&w)[2][NI]) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const bf16x8* src = reinterpret_cast<const bf16x8*>(wp[ni] + (int64_t)kb * KT + u * 32);
        w[u][ni] = NTW ? __builtin_nontemporal_load(src) : *src;
      }
  };

  // this workgroup's k slab: k-blocks [kb0, kb0 + nkb).  With NKB > 0 the
  // count is a compile-time constant and the loop below unrolls fully, which
  // lets the compiler wait for exactly the ring slot it needs (across a
  // loop back-edge it would wait for every load in flight).
  const int nkb = NKB > 0 ? NKB : K / KT / p.ksplit;
  const int kb0 = ks * nkb;
#pragma unroll
  for (int s = 0; s < P - 1; ++s)
    if (s < nkb) {
      load_a(kb0 + s, areg[s]);
      load_w(kb0 + s, wreg[s]);
    }
  store_a(areg[0], 0);
  __syncthreads();
#pragma unroll(NKB > 0 ? NKB : 1)
  for (int kb = 0; kb < nkb; kb += P) {
#pragma unroll
    for (int s = 0; s < P; ++s) {
      const int k = kb + s;
      if (k < nkb) {
        const int sp = (s + P - 1) % P;     // slot of block k + P - 1 (freed by block k - 1)
        if (k + P - 1 < nkb) {
          load_a(kb0 + k + P - 1, areg[sp]);
          load_w(kb0 + k + P - 1, wreg[sp]);
        }
        const int buf = k & 1;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int kk = wk * 64 + u * 32 + kl;
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                As + buf * A_ELEMS + (mb * 16 + (lane & 15)) * ROW + kk);
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
              acc[mb][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wreg[s][u][ni], a, acc[mb][ni], 0, 0, 0);
          }
        }
        if (k + 1 < nkb) store_a(areg[(s + 1) % P], buf ^ 1);
        __syncthreads();
      }
    }
  }

  // reduce the WK partial sums (fixed order: wk = 0, 1, 2, 3)
  if constexpr (WK > 1) {
    float* red = reinterpret_cast<float*>(smem);
    if (wk > 0) {
      float* dst = red + ((wk - 1) * WN + wn) * (MB * NI * 4 * 64);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
          for (int r = 0; r < 4; ++r) dst[((mb * NI + ni) * 4 + r) * 64 + lane] = acc[mb][ni][r];
    }
    __syncthreads();
    if (wk == 0) {
#pragma unroll
      for (int w = 1; w < WK; ++w) {
        const float* src = red + ((w - 1) * WN + wn) * (MB * NI * 4 * 64);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int ni = 0; ni < NI; ++ni)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[mb][ni][r] += src[((mb * NI + ni) * 4 + r) * 64 + lane];
      }
    }
  }

  // epilogue (waves with wk == 0 own the final sums)
  const int fl = (lane >> 4) * 4;
  if constexpr (EPI != EPI_ARGMAX) {
    if (wk == 0) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int row = m0 + mb * 16 + (lane & 15);
        if (row >= M) continue;
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const int f = n0 + wn * NI * 16 + ni * 16 + fl;
          if (f >= N) continue;
          const f32x4 v = acc[mb][ni];
          if constexpr (EPI == EPI_STORE) {
            *reinterpret_cast<float4*>(p.C + ks * p.pstride + (int64_t)row * p.ldc + f) =
                make_float4(v[0], v[1], v[2], v[3]);
          } else if constexpr (EPI == EPI_ADD) {
            float4* o = reinterpret_cast<float4*>(p.C + (int64_t)row * p.ldc + f);
            float4 c = *o;
            c.x += v[0]; c.y += v[1]; c.z += v[2]; c.w += v[3];
            *o = c;
          } else {  // GELU, rounded to bf16
            uint2 pk;
            pk.x = (uint32_t)f2bf(gelu_f(v[0])) | ((uint32_t)f2bf(gelu_f(v[1])) << 16);
            pk.y = (uint32_t)f2bf(gelu_f(v[2])) | ((uint32_t)f2bf(gelu_f(v[3])) << 16);
            *reinterpret_cast<uint2*>(p.Cb + (int64_t)row * p.ldc + f) = pk;
          }
        }
      }
    }
  } else {
    // greedy head: optional logits, then the per-row first maximum
    __shared__ float bv[WN][BM];
    __shared__ int bi[WN][BM];
    if (wk == 0) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int row = m0 + mb * 16 + (lane & 15);
        float best = -INFINITY;
        int bidx = 0x7fffffff;
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const int f = n0 + wn * NI * 16 + ni * 16 + fl;
          if (f >= N) continue;
          const f32x4 v = acc[mb][ni];
          if (p.C && row < M)
            *reinterpret_cast<float4*>(p.C + (int64_t)row * p.ldc + f) = make_float4(v[0], v[1], v[2], v[3]);
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (v[r] > best) { best = v[r]; bidx = f + r; }
        }
#pragma unroll
        for (int o = 16; o <= 32; o <<= 1) {
          const float ov = __shfl_xor(best, o, 64);
          const int oi = __shfl_xor(bidx, o, 64);
          if (ov > best || (ov == best && oi < bidx)) { best = ov; bidx = oi; }
        }
        if ((lane >> 4) == 0) { bv[wn][mb * 16 + lane] = best; bi[wn][mb * 16 + lane] = bidx; }
      }
    }
    __syncthreads();
    if (tid < BM) {
      const int row = m0 + tid;
      if (row < M) {
        float best = bv[0][tid];
        int bidx = bi[0][tid];
#pragma unroll
        for (int w = 1; w < WN; ++w)
          if (bv[w][tid] > best) { best = bv[w][tid]; bidx = bi[w][tid]; }
        p.av[(int64_t)nt * M + row] = best;
        p.ai[(int64_t)nt * M + row] = bidx;
      }
    }
  }
}

// ---- fp32 models: plain FMA kernel, one thread per output ----
struct GemmPF {
  const float* A; int64_t lda;
  const float* W;
  int M, N, K;
  float* C; int64_t ldc;
  float* Cf;
  float* av; int* ai;
};

template <int EPI>
__global__ __launch_bounds__(64) void gemm_f32_kernel(GemmPF p) {
  const int n = blockIdx.x * 64 + threadIdx.x;
  const int m = blockIdx.y;
  float acc = 0.f;
  if (n < p.N) {
    const float* a = p.A + (int64_t)m * p.lda;
    const float* w = p.W + (int64_t)n * p.K;
    for (int k = 0; k < p.K; ++k) acc = fmaf(a[k], w[k], acc);
  }
  if constexpr (EPI == EPI_STORE) {
    if (n < p.N) p.C[(int64_t)m * p.ldc + n] = acc;
  } else if constexpr (EPI == EPI_ADD) {
    if (n < p.N) p.C[(int64_t)m * p.ldc + n] += acc;
  } else if constexpr (EPI == EPI_GELU) {
    if (n < p.N) p.Cf[(int64_t)m * p.ldc + n] = gelu_f(acc);
  } else {
    if (n < p.N && p.C) p.C[(int64_t)m * p.ldc + n] = acc;
    float best = n < p.N ? acc : -INFINITY;
    int bidx = n < p.N ? n : 0x7fffffff;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float ov = __shfl_xor(best, o, 64);
      const int oi = __shfl_xor(bidx, o, 64);
      if (ov > best || (ov == best && oi < bidx)) { best = ov; bidx = oi; }
    }
    if (threadIdx.x == 0) {
      p.av[(int64_t)blockIdx.x * p.M + m] = best;
      p.ai[(int64_t)blockIdx.x * p.M + m] = bidx;
    }
  }
}

typedef void (*GemmKernel)(GemmP);

struct Plan {
  int MB, NI, WK, m_tiles, n_tiles, ksplit;
  GemmKernel fn;   // tuned instantiation (fully unrolled k loop), or null
};

// Tuned tiles for the decode GEMMs of the PHOTON model shapes (d = 768 and
// 1536, MLP 4d, vocab 32000, rows B or B*C2 from 16 to 512), measured on
// MI355X with the weights streamed from HBM (weights rotated past the
// Infinity Cache between launches).  Fields: M, N, K, epilogue, whether the
// entry splits K into slabs (usable only by callers that sum slabs), then
// MB, NI, WK, ring depth P, K slabs, k-blocks per workgroup, non-temporal W.
// Most winners run ~192-250 workgroups, about one per CU.
#define PHOTON_GEMM_TUNED(X) \
  X(16, 1536, 1536, EPI_STORE, 1, 1, 1, 1, 3, 8, 3, true) \
  X(16, 1536, 6144, EPI_STORE, 1, 1, 2, 4, 4, 4, 6, false) \
  X(16, 4608, 1536, EPI_STORE, 1, 1, 1, 1, 4, 6, 4, false) \
  X(16, 6144, 1536, EPI_GELU, 0, 1, 1, 2, 4, 1, 12, true) \
  X(16, 6144, 1536, EPI_STORE, 1, 1, 1, 2, 4, 4, 3, false) \
  X(32, 768, 768, EPI_STORE, 1, 1, 1, 2, 3, 2, 3, true) \
  X(32, 768, 3072, EPI_STORE, 1, 2, 1, 2, 4, 8, 3, true) \
  X(32, 2304, 768, EPI_STORE, 1, 2, 1, 1, 3, 6, 2, true) \
  X(32, 3072, 768, EPI_GELU, 0, 1, 1, 2, 4, 1, 6, true) \
  X(32, 3072, 768, EPI_STORE, 1, 2, 1, 2, 4, 2, 3, true) \
  X(64, 1536, 1536, EPI_STORE, 1, 4, 1, 1, 4, 8, 3, true) \
  X(64, 1536, 6144, EPI_STORE, 1, 4, 2, 2, 4, 8, 6, true) \
  X(64, 4608, 1536, EPI_STORE, 1, 4, 2, 2, 4, 3, 4, true) \
  X(64, 6144, 1536, EPI_GELU, 0, 2, 2, 2, 4, 1, 12, false) \
  X(64, 6144, 1536, EPI_STORE, 1, 4, 2, 1, 4, 4, 6, false) \
  X(64, 6144, 1536, EPI_STORE, 0, 2, 2, 2, 4, 1, 12, false) \
  X(64, 32000, 1536, EPI_ARGMAX, 0, 4, 2, 1, 4, 1, 24, false) \
  X(128, 768, 768, EPI_STORE, 1, 2, 1, 2, 3, 2, 3, true) \
  X(128, 768, 3072, EPI_STORE, 1, 4, 1, 1, 4, 8, 6, true) \
  X(128, 2304, 768, EPI_STORE, 1, 4, 1, 2, 3, 3, 2, true) \
  X(128, 3072, 768, EPI_GELU, 0, 2, 1, 1, 4, 1, 12, true) \
  X(128, 3072, 768, EPI_STORE, 1, 4, 1, 1, 4, 2, 6, true) \
  X(128, 3072, 768, EPI_STORE, 0, 2, 1, 1, 4, 1, 12, true) \
  X(128, 32000, 768, EPI_ARGMAX, 0, 8, 2, 1, 4, 1, 12, false) \
  X(256, 1536, 1536, EPI_STORE, 1, 4, 1, 1, 4, 2, 12, true) \
  X(256, 1536, 3072, EPI_STORE, 1, 8, 2, 1, 4, 8, 6, true) \
  X(256, 1536, 6144, EPI_STORE, 1, 8, 2, 1, 4, 8, 12, false) \
  X(256, 3072, 1536, EPI_STORE, 1, 4, 2, 1, 4, 2, 12, false) \
  X(256, 4608, 1536, EPI_STORE, 1, 8, 2, 1, 4, 3, 8, false) \
  X(256, 6144, 1536, EPI_GELU, 0, 4, 2, 1, 4, 1, 24, false) \
  X(256, 6144, 1536, EPI_STORE, 1, 8, 2, 1, 4, 2, 12, false) \
  X(256, 6144, 1536, EPI_STORE, 0, 4, 2, 1, 4, 1, 24, false) \
  X(256, 32000, 1536, EPI_ARGMAX, 0, 8, 4, 1, 3, 1, 24, false) \
  X(512, 1536, 1536, EPI_STORE, 1, 4, 2, 2, 4, 1, 12, true) \
  X(512, 1536, 3072, EPI_STORE, 1, 8, 2, 1, 4, 4, 12, false) \
  X(512, 1536, 6144, EPI_STORE, 1, 8, 2, 1, 4, 4, 24, false) \
  X(512, 3072, 1536, EPI_STORE, 1, 8, 2, 1, 4, 2, 12, true) \
  X(512, 3072, 1536, EPI_STORE, 0, 8, 2, 2, 4, 1, 12, true) \
  X(512, 4608, 1536, EPI_STORE, 1, 8, 4, 1, 3, 3, 8, false) \
  X(512, 6144, 1536, EPI_GELU, 0, 8, 2, 1, 4, 1, 24, false) \
  X(512, 32000, 1536, EPI_ARGMAX, 0, 8, 2, 1, 4, 1, 24, false)

struct Tuned {
  int M, N, K, epi, split, MB, NI, WK, P, ks, nkb;
  bool ntw;
  GemmKernel fn;
};
#define PHOTON_TUNED_ENTRY(M_, N_, K_, E_, S_, MB_, NI_, WK_, P_, KS_, NKB_, NT_) \
  {M_, N_, K_, E_, S_, MB_, NI_, WK_, P_, KS_, NKB_, NT_, gemm_bf16_kernel<MB_, NI_, WK_, P_, E_, NKB_, NT_>},
const Tuned kTuned[] = {PHOTON_GEMM_TUNED(PHOTON_TUNED_ENTRY)};
#undef PHOTON_TUNED_ENTRY

const Tuned* find_tuned(int M, int N, int K, int epi, bool allow_split) {
  const Tuned* hit = nullptr;
  for (const Tuned& t : kTuned) {
    if (t.M != M || t.N != N || t.K != K || t.epi != epi) continue;
    if (t.split && !allow_split) continue;
    if (!hit || (t.split && !hit->split)) hit = &t;   // slabs when the caller takes them
  }
  return hit;
}

// Waves along K: as many as the LDS budget of the M tile allows (4 for
// M tiles up to 64 rows, 2 for 128, 1 for 256) and K divides into.
int wk_of(int MB, int K) {
  int wk = MB >= 16 ? 1 : (MB >= 8 ? 2 : 4);
  while (wk > 1 && K % (64 * wk)) wk >>= 1;
  return wk;
}

// Tile plan.  Shapes in the tuned table take their measured tile; any other
// shape (prefill, other model sizes) gets a general plan: decode GEMMs are
// skinny (M = B or B*C2 rows) and their cost is streaming W once, so the
// plan looks for enough workgroups to keep every CU streaming: the widest
// column tile that still gives >= 256 workgroups, and otherwise a split of
// K into slabs (RAW partials, summed by the consumer).
Plan plan_bf16(int M, int N, int K, int epi, bool allow_split) {
  if (const Tuned* t = find_tuned(M, N, K, epi, allow_split)) {
    const int BM = 16 * t->MB, BN = 16 * t->NI * (4 / t->WK);
    return Plan{t->MB, t->NI, t->WK, (M + BM - 1) / BM, (N + BN - 1) / BN, t->ks, t->fn};
  }
  Plan best{};
  const int MB0 = M <= 16 ? 1 : M <= 32 ? 2 : M <= 64 ? 4 : M <= 128 ? 8 : 16;
  const int target = 256;
  long best_score = -1;
  // candidate M tiles: the one covering M (up to 256 rows) and, for tall
  // skinny GEMMs, half of it (two M tiles of one W slab are adjacent and land
  // on the same XCD, so the second read of the slab hits L2)
  for (int MB = MB0; MB >= 1 && MB >= MB0 / 2; MB >>= 1) {
    if (MB < MB0 && MB0 < 8) break;
    const int m_tiles = (M + 16 * MB - 1) / (16 * MB);
    const int wk_max = wk_of(MB, K);
    const int ni_max = MB >= 16 ? 2 : 4;
    for (int wk = wk_max; wk >= 1; wk >>= 1) {
      if (K % (64 * wk)) continue;
      const int WN = 4 / wk;
      const int nkb = K / (64 * wk);
      for (int ni = ni_max; ni >= 1; ni >>= 1) {
        const int n_tiles = (N + 16 * ni * WN - 1) / (16 * ni * WN);
        for (int ks = 1; ks <= (allow_split ? nkb : 1); ++ks) {
          if (nkb % ks) continue;
          const long wgs = (long)n_tiles * m_tiles * ks;
          // reach the target first; then fewest slabs, fewest M tiles, the
          // widest tile and the most waves along K
          const long score = wgs >= target
                                 ? (1L << 40) - (long)ks * (1L << 24) - (long)m_tiles * (1L << 18) + ni * WN * 16 * 8 + wk
                                 : wgs * 64 + ni;
          if (score > best_score) {
            best_score = score;
            best = Plan{MB, ni, wk, m_tiles, n_tiles, ks, nullptr};
          }
          if (wgs >= target) break;   // more slabs only add partial traffic
        }
      }
    }
  }
  return best;
}

template <int MB, int NI, int WK>
hipError_t run_bf16(const GemmP& p, int epi, hipStream_t st) {
  dim3 grid(p.m_tiles * p.n_tiles * p.ksplit), block(256);
  switch (epi) {
    case EPI_STORE: PH_LAUNCH((gemm_bf16_kernel<MB, NI, WK, 2, EPI_STORE, 0, false>), grid, block, 0, st, p); break;
    case EPI_ADD: PH_LAUNCH((gemm_bf16_kernel<MB, NI, WK, 2, EPI_ADD, 0, false>), grid, block, 0, st, p); break;
    case EPI_GELU: PH_LAUNCH((gemm_bf16_kernel<MB, NI, WK, 2, EPI_GELU, 0, false>), grid, block, 0, st, p); break;
    default: PH_LAUNCH((gemm_bf16_kernel<MB, NI, WK, 2, EPI_ARGMAX, 0, false>), grid, block, 0, st, p); break;
  }
  return hipGetLastError();
}

template <int MB, int WK>
hipError_t run_bf16_ni(const GemmP& p, int NI, int epi, hipStream_t st) {
  if constexpr (MB >= 16) {
    if (NI == 2) return run_bf16<MB, 2, WK>(p, epi, st);
    return run_bf16<MB, 1, WK>(p, epi, st);
  } else {
    if (NI == 4) return run_bf16<MB, 4, WK>(p, epi, st);
    if (NI == 2) return run_bf16<MB, 2, WK>(p, epi, st);
    return run_bf16<MB, 1, WK>(p, epi, st);
  }
}

template <int MB>
hipError_t run_bf16_wk(const GemmP& p, int NI, int WK, int epi, hipStream_t st) {
  if constexpr (MB <= 4) {
    if (WK == 4) return run_bf16_ni<MB, 4>(p, NI, epi, st);
  }
  if constexpr (MB <= 8) {
    if (WK == 2) return run_bf16_ni<MB, 2>(p, NI, epi, st);
  }
  return run_bf16_ni<MB, 1>(p, NI, epi, st);
}

}  // namespace

int gemm_supported(int dtype, int M, int N, int K) {
  if (M < 1 || N < 1 || K < 1) return 0;
  if (dtype == 0) return 1;
  return N % 16 == 0 && K % 64 == 0;
}

int gemm_argmax_tiles(int dtype, int M, int N, int K) {
  if (dtype == 0) return (N + 63) / 64;
  return plan_bf16(M, N, K, EPI_ARGMAX, false).n_tiles;
}

int gemm_splits(int dtype, int M, int N, int K) {
  if (dtype == 0) return 1;
  return plan_bf16(M, N, K, EPI_STORE, true).ksplit;
}

hipError_t launch_gemm(const GemmCall& g, hipStream_t st) {
  if (g.dtype == 0) {
    GemmPF p{(const float*)g.A, g.lda, (const float*)g.W, g.M, g.N, g.K,
             g.C, g.ldc, (float*)g.Cb, g.amax_val, g.amax_idx};
    dim3 grid((g.N + 63) / 64, g.M), block(64);
    switch (g.epi) {
      case EPI_STORE: PH_LAUNCH((gemm_f32_kernel<EPI_STORE>), grid, block, 0, st, p); break;
      case EPI_ADD: PH_LAUNCH((gemm_f32_kernel<EPI_ADD>), grid, block, 0, st, p); break;
      case EPI_GELU: PH_LAUNCH((gemm_f32_kernel<EPI_GELU>), grid, block, 0, st, p); break;
      default: PH_LAUNCH((gemm_f32_kernel<EPI_ARGMAX>), grid, block, 0, st, p); break;
    }
    return hipGetLastError();
  }
  const Plan pl = plan_bf16(g.M, g.N, g.K, g.epi, g.epi == EPI_STORE && g.allow_split);
  GemmP p{(const bf16_t*)g.A, g.lda, (const bf16_t*)g.W, g.M, g.N, g.K,
          g.C, g.ldc, (bf16_t*)g.Cb, g.amax_val, g.amax_idx, pl.m_tiles, pl.n_tiles,
          pl.ksplit, (int64_t)g.M * g.ldc};
  if (pl.fn) {
    PH_LAUNCH(pl.fn, pl.m_tiles * pl.n_tiles * pl.ksplit, 256, 0, st, p);
    return hipGetLastError();
  }
  switch (pl.MB) {
    case 1: return run_bf16_wk<1>(p, pl.NI, pl.WK, g.epi, st);
    case 2: return run_bf16_wk<2>(p, pl.NI, pl.WK, g.epi, st);
    case 4: return run_bf16_wk<4>(p, pl.NI, pl.WK, g.epi, st);
    case 8: return run_bf16_wk<8>(p, pl.NI, pl.WK, g.epi, st);
    default: return run_bf16_wk<16>(p, pl.NI, pl.WK, g.epi, st);
  }
}

}  // namespace photon
