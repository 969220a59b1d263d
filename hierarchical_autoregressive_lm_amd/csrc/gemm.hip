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
#include <utility>

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
  // EPI_ROPE (prompt QKV projection): rotated q to q (fp32 [M][d]), rotated
  // k and v rounded to bf16 into the cache planes Kc / Vc
  float* q; bf16_t* Kc; bf16_t* Vc; const float* rope;
  int64_t seq_stride; int cap, rows_per_seq, seq0, pos_add, d;
  const int* pos_dev; int pos_mul;   // positions also advance with a device counter (decode)
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

// ---- decode GEMM with the tiles streamed into LDS by direct loads ----
//
// gfx950's global_load_lds_dwordx4 writes 16 bytes per lane straight into
// LDS, so the prefetch depth costs LDS, not registers.  A ring of P stages,
// each one 64-wide k-block of the tile's A rows (first) and W rows (then),
// 128 bytes per row with the 16-byte chunks XOR-swizzled by the row so that
// the MFMA fragment reads spread over the banks.  Every wave issues its
// share of a stage's loads; before computing on stage kb it waits until at
// most the loads of the stages after kb are in flight (an explicit vmcnt)
// and its own LDS reads of the previous stage are done (lgkmcnt(0)), then
// meets the others at a barrier, which thereby frees the slot the next
// stage is loaded into.  Each ring slot is an LDS object of its own: the
// compiler then tells the slots apart and inserts no wait of its own.  The
// k loop is unrolled at compile time (NKB k-blocks per workgroup), so every
// slot index and wait count is a constant.
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void glb_void_t;

template <class F, int... I>
__device__ __forceinline__ void static_for(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}

// s_waitcnt immediate: vmcnt(n) and lgkmcnt(0), expcnt not waited on.  The
// lgkmcnt(0) matters: the barrier after it is what lets the other waves
// refill the slot this wave read last, and the compiler issues those LDS
// reads early but waits for them only where the products use them, which
// may be after the barrier; without the wait a refill that lands quickly
// (an L2 hit) can overwrite a slot before a wave held back on a busy CU
// has read it.
constexpr int vm_wait(int n) { return (n & 15) | (7 << 4) | (0 << 8) | (((n >> 4) & 3) << 14); }

#define PH_LDS_SLOTS(X) X(0) X(1) X(2) X(3) X(4) X(5)

template <int BM, int BN, int WM, int P, int EPI, int NKB, int NW = 4, bool PERSIST = false>
__global__ __launch_bounds__(NW * 64) void gemm_lds_kernel(GemmP p) {
  constexpr int WN = NW / WM, TM = BM / WM, TN = BN / WN, MF = TM / 16, NF = TN / 16;
  constexpr int ROWS = BM + BN;             // A rows, then W rows; 128 B each
  constexpr int SLOT_U4 = ROWS * 8;         // 16-byte units per slot
  constexpr int I = ROWS / (8 * NW);        // direct-load instructions per wave per stage
  static_assert(ROWS % (8 * NW) == 0 && TM % 16 == 0 && TN % 16 == 0 && P >= 2 && P <= 6, "tile");
  static_assert(EPI != EPI_ARGMAX || 2 * WN * BM * 4 <= ROWS * 128, "argmax partials fit a slot");
  static_assert(!PERSIST || (NKB == 0 && (EPI == EPI_STORE || EPI == EPI_GELU || EPI == EPI_ROPE)),
                "persistent workgroups: run-time k loop, epilogues that store only");
  static_assert(!PERSIST || (P - 2) * I + MF * NF <= 63, "waits fit the counter");
#define PH_DECL(s) __shared__ __attribute__((aligned(16))) uint4 L##s[s < P ? SLOT_U4 : 1];
  PH_LDS_SLOTS(PH_DECL)
#undef PH_DECL
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  const int total = p.m_tiles * p.n_tiles;
  const int ks = PERSIST ? 0 : blockIdx.x % p.ksplit;
  // XCD-aware tile order: consecutive workgroups land on different XCDs, so
  // each XCD takes a contiguous run of tiles.  Inside the run, row tiles in
  // groups of 1024 rows, the row tile fastest inside a group: while an XCD
  // walks a group's columns its A tiles stay in L2 and each W column slab
  // serves the whole group (prompt-sized GEMMs, whose A outgrows the
  // Infinity Cache: 5-17 % faster than walking every row tile per column;
  // groups of 512 or 2048 rows measured slower); at most 1024 rows (every
  // decode shape) this is the plain row-fastest order.  Persistent
  // workgroups take virtual tiles v, v + gridDim.x, ... (gridDim.x a
  // multiple of 8, so every one stays on its XCD's run).
  auto tile_of = [&](int v, int& tm0, int& tn0) {
    const int tile = (total % 8 == 0) ? (v % 8) * (total / 8) + v / 8 : v;
    constexpr int GR = 1024 / BM;
    const int grp = tile / (GR * p.n_tiles), base = grp * GR;
    const int gs = min(GR, p.m_tiles - base), r = tile - grp * GR * p.n_tiles;
    tm0 = (base + r % gs) * BM;
    tn0 = (r / gs) * BN;
  };
  int vt = PERSIST ? (int)blockIdx.x : (int)blockIdx.x / p.ksplit;
  int m0, n0;
  tile_of(vt, m0, n0);
  const int K = p.K;
  // k-blocks of this workgroup's slab: compile-time (fully unrolled loop) or,
  // with NKB = 0, K / 64 / ksplit at run time, a multiple of P
  const int nkb = NKB > 0 ? NKB : K / 64 / p.ksplit;
  const int kb0 = ks * nkb;

  // the source row of this lane in each of its load instructions (rows past
  // M or N are clamped: their results are never stored)
  const bf16_t* src[I];
  auto set_src = [&](int tm0, int tn0) {
#pragma unroll
    for (int q = 0; q < I; ++q) {
      const int row = (wave * I + q) * 8 + (lane >> 3);
      const int chunk = (lane & 7) ^ (row & 7);
      if (row < BM) src[q] = p.A + (int64_t)min(tm0 + row, p.M - 1) * p.lda + chunk * 8;
      else src[q] = p.W + (int64_t)min(tn0 + row - BM, p.N - 1) * K + chunk * 8;
    }
  };
  set_src(m0, n0);
  auto issue = [&](auto sc, int kb) {
    constexpr int s = decltype(sc)::value;
    uint4* Ls = s == 0 ? L0 : s == 1 ? L1 : s == 2 ? L2 : s == 3 ? L3 : s == 4 ? L4 : L5;
#pragma unroll
    for (int q = 0; q < I; ++q)
      __builtin_amdgcn_global_load_lds((glb_void_t*)(src[q] + (int64_t)kb * 64),
                                       (lds_void_t*)(Ls + (wave * I + q) * 64), 16, 0, 0);
  };

  f32x4 acc[MF][NF];
#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int j = 0; j < NF; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  auto compute = [&](auto sc) {
    constexpr int s = decltype(sc)::value;
    const uint4* Ls = s == 0 ? L0 : s == 1 ? L1 : s == 2 ? L2 : s == 3 ? L3 : s == 4 ? L4 : L5;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int kc = u * 4 + (lane >> 4);   // this lane's 8 k values
      bf16x8 a[MF], w[NF];
#pragma unroll
      for (int i = 0; i < MF; ++i) {
        const int row = wm * TM + i * 16 + (lane & 15);
        a[i] = *reinterpret_cast<const bf16x8*>(Ls + row * 8 + (kc ^ (row & 7)));
      }
#pragma unroll
      for (int j = 0; j < NF; ++j) {
        const int row = BM + wn * TN + j * 16 + (lane & 15);
        w[j] = *reinterpret_cast<const bf16x8*>(Ls + row * 8 + (kc ^ (row & 7)));
      }
#pragma unroll
      for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int j = 0; j < NF; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w[j], a[i], acc[i][j], 0, 0, 0);
    }
  };

  // the tile's results (every epilogue but the greedy head's): each lane
  // holds features 4*(lane>>4)..+3 of row (lane&15) of each fragment
  const int fl = (lane >> 4) * 4;
  auto store_tile = [&](int m0, int n0) {
    if constexpr (EPI == EPI_ROPE) {
      // A wave's TN columns are one head of q, k or v (TN = head size, the
      // tile starts on a head), so the rotate-half partner of feature c < TN/2,
      // c + TN/2, sits in the same lane, fragment j + NF/2.  Row r of the
      // product is new row t = r % rows_per_seq of sequence r / rows_per_seq,
      // at position pos_add + t; its K and V go to cache slot pos.
      static_assert(NF % 2 == 0, "rotation partners are half a head apart");
      constexpr int HALF = TN / 2;
      const int col0 = n0 + wn * TN;
      const int part = col0 / p.d;                 // 0 q, 1 k, 2 v (uniform per wave)
      const int h = (col0 - part * p.d) / TN;
      const int pos0 = p.pos_add + (p.pos_dev ? *p.pos_dev * p.pos_mul : 0);
  #pragma unroll
      for (int i = 0; i < MF; ++i) {
        const int row = m0 + wm * TM + i * 16 + (lane & 15);
        if (row >= p.M) continue;
        const int sq = row / p.rows_per_seq, t = row - sq * p.rows_per_seq;
        const int pos = pos0 + t;
        const int64_t slot = (int64_t)(p.seq0 + sq) * p.seq_stride + ((int64_t)h * p.cap + pos) * TN;
        if (part == 2) {
  #pragma unroll
          for (int j = 0; j < NF; ++j) {
            const f32x4 v = acc[i][j];
            uint2 pk;
            pk.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
            pk.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
            *reinterpret_cast<uint2*>(p.Vc + slot + j * 16 + fl) = pk;
          }
          continue;
        }
        const float* rp = p.rope + (int64_t)pos * TN;   // (cos, sin) of features 0 .. HALF-1
  #pragma unroll
        for (int j = 0; j < NF / 2; ++j) {
          const int cc = j * 16 + fl;
          const float4 r0 = *reinterpret_cast<const float4*>(rp + 2 * cc);
          const float4 r1 = *reinterpret_cast<const float4*>(rp + 2 * cc + 4);
          const float cs[4] = {r0.x, r0.z, r1.x, r1.z}, sn[4] = {r0.y, r0.w, r1.y, r1.w};
          const f32x4 a = acc[i][j], b = acc[i][j + NF / 2];
          float lo[4], hi[4];
  #pragma unroll
          for (int e = 0; e < 4; ++e) {
            lo[e] = a[e] * cs[e] - b[e] * sn[e];
            hi[e] = b[e] * cs[e] + a[e] * sn[e];
          }
          if (part == 0) {
            float* q = p.q + (int64_t)row * p.d + h * TN + cc;
            *reinterpret_cast<float4*>(q) = make_float4(lo[0], lo[1], lo[2], lo[3]);
            *reinterpret_cast<float4*>(q + HALF) = make_float4(hi[0], hi[1], hi[2], hi[3]);
          } else {
            uint2 pl, ph;
            pl.x = (uint32_t)f2bf(lo[0]) | ((uint32_t)f2bf(lo[1]) << 16);
            pl.y = (uint32_t)f2bf(lo[2]) | ((uint32_t)f2bf(lo[3]) << 16);
            ph.x = (uint32_t)f2bf(hi[0]) | ((uint32_t)f2bf(hi[1]) << 16);
            ph.y = (uint32_t)f2bf(hi[2]) | ((uint32_t)f2bf(hi[3]) << 16);
            *reinterpret_cast<uint2*>(p.Kc + slot + cc) = pl;
            *reinterpret_cast<uint2*>(p.Kc + slot + cc + HALF) = ph;
          }
        }
      }
    } else if constexpr (EPI != EPI_ARGMAX) {
  #pragma unroll
      for (int i = 0; i < MF; ++i) {
        const int row = m0 + wm * TM + i * 16 + (lane & 15);
        if (row >= p.M) continue;
  #pragma unroll
        for (int j = 0; j < NF; ++j) {
          const int f = n0 + wn * TN + j * 16 + fl;
          if (f >= p.N) continue;
          const f32x4 v = acc[i][j];
          if constexpr (EPI == EPI_STORE) {
            *reinterpret_cast<float4*>(p.C + ks * p.pstride + (int64_t)row * p.ldc + f) = make_float4(v[0], v[1], v[2], v[3]);
          } else if constexpr (EPI == EPI_ADD) {
            float4* o = reinterpret_cast<float4*>(p.C + (int64_t)row * p.ldc + f);
            float4 c = *o;
            c.x += v[0]; c.y += v[1]; c.z += v[2]; c.w += v[3];
            *o = c;
          } else {   // GELU, rounded to bf16
            uint2 pk;
            pk.x = (uint32_t)f2bf(gelu_f(v[0])) | ((uint32_t)f2bf(gelu_f(v[1])) << 16);
            pk.y = (uint32_t)f2bf(gelu_f(v[2])) | ((uint32_t)f2bf(gelu_f(v[3])) << 16);
            *reinterpret_cast<uint2*>(p.Cb + (int64_t)row * p.ldc + f) = pk;
          }
        }
      }
    }
  };

  if constexpr (NKB > 0) {
    static_for([&](auto sc) {
      constexpr int s = decltype(sc)::value;
      if constexpr (s < NKB) issue(sc, kb0 + s);
    }, std::make_integer_sequence<int, P - 1>{});
    static_for([&](auto kbc) {
      constexpr int kb = decltype(kbc)::value;
      constexpr int ahead = (P - 2 < NKB - 1 - kb) ? P - 2 : NKB - 1 - kb;   // later stages still in flight
      __builtin_amdgcn_s_waitcnt(vm_wait(ahead * I));
      __builtin_amdgcn_s_barrier();
      if constexpr (kb + P - 1 < NKB) issue(std::integral_constant<int, (kb + P - 1) % P>{}, kb0 + kb + P - 1);
      compute(std::integral_constant<int, kb % P>{});
    }, std::make_integer_sequence<int, NKB>{});
  } else if constexpr (!PERSIST) {
    // run-time loop over groups of P stages (slot s of a group is stage
    // kb + s, so slots stay compile-time constants); in every group but the
    // last each stage issues its successor P - 1 stages ahead, so P - 2
    // later stages are in flight at every wait; the last group is peeled
    static_for([&](auto sc) { issue(sc, kb0 + decltype(sc)::value); }, std::make_integer_sequence<int, P - 1>{});
    int kb = 0;
    for (; kb + P < nkb; kb += P) {
      static_for([&](auto sc) {
        constexpr int s = decltype(sc)::value;
        __builtin_amdgcn_s_waitcnt(vm_wait((P - 2) * I));
        __builtin_amdgcn_s_barrier();
        issue(std::integral_constant<int, (s + P - 1) % P>{}, kb0 + kb + s + P - 1);
        compute(sc);
      }, std::make_integer_sequence<int, P>{});
    }
    static_for([&](auto sc) {
      constexpr int s = decltype(sc)::value;
      constexpr int ahead = (P - 2 < P - 1 - s) ? P - 2 : P - 1 - s;
      __builtin_amdgcn_s_waitcnt(vm_wait(ahead * I));
      __builtin_amdgcn_s_barrier();
      if constexpr (s == 0) issue(std::integral_constant<int, P - 1>{}, kb0 + kb + P - 1);
      compute(sc);
    }, std::make_integer_sequence<int, P>{});
  } else {
    // Persistent workgroups (prompt-sized GEMMs): one workgroup per CU walks
    // its tiles with the same run-time k loop.  At the last stage of a tile,
    // once the barrier has freed slots 0 .. P-2, the next tile's first P-1
    // stages are issued, so they load while the last products and the
    // epilogue run and the epilogue's stores drain under the next tile's
    // first stages (a synchronised store burst from every CU at once would
    // otherwise leave the matrix cores idle).  The vector memory counter
    // retires in issue order, so a wait for a prefetched stage also counts
    // the E stores issued after it: while those stages are consumed the
    // wait allows E more, which holds only when the tile stored all of its
    // E results (a full tile); after a partial one the plain wait is used.
    // (A direct-to-LDS load under a branch makes the compiler wait for every
    // load before the next LDS read, so the tile's first stage also waits
    // for those stores in places: with two ring stages, whose waits drain
    // the ring anyway, this costs nothing, and only the two-stage QKV tile
    // of 96-wide heads runs persistent: 10 % faster at the 600M prompts,
    // where three-stage tiles measured 15-30 % slower.)
    constexpr int E = MF * NF;                  // stores per wave of a full tile
    static_for([&](auto sc) { issue(sc, decltype(sc)::value); }, std::make_integer_sequence<int, P - 1>{});
    bool behind = false;   // the previous tile's E stores sit behind the prefetched stages
    const int ngroups = nkb / P;
    for (;;) {
      const int cm0 = m0, cn0 = n0;
      const int vn = vt + (int)gridDim.x;
      const bool more = vn < total;
#pragma unroll
      for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int j = 0; j < NF; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
      for (int g = 0; g < ngroups; ++g) {
        const int kb = g * P;
        const bool last = g + 1 == ngroups;
        const bool extra = behind && g == 0;
        static_for([&](auto sc) {
          constexpr int s = decltype(sc)::value;
          constexpr int mid = P - 2;                                      // later stages issued before the wait
          constexpr int fin = (P - 2 < P - 1 - s) ? P - 2 : P - 1 - s;   // the same in the last group
          if (extra && s < P - 1) {
            if (last) __builtin_amdgcn_s_waitcnt(vm_wait(fin * I + E));
            else __builtin_amdgcn_s_waitcnt(vm_wait(mid * I + E));
          } else {
            if (last) __builtin_amdgcn_s_waitcnt(vm_wait(fin * I));
            else __builtin_amdgcn_s_waitcnt(vm_wait(mid * I));
          }
          __builtin_amdgcn_s_barrier();
          if (!last) {
            issue(std::integral_constant<int, (s + P - 1) % P>{}, kb + s + P - 1);
          } else {
            if constexpr (s == 0) issue(std::integral_constant<int, P - 1>{}, kb + P - 1);
            if constexpr (s == P - 1) {
              if (more) {
                tile_of(vn, m0, n0);
                set_src(m0, n0);
                static_for([&](auto nc) { issue(nc, decltype(nc)::value); }, std::make_integer_sequence<int, P - 1>{});
              }
            }
          }
          compute(sc);
        }, std::make_integer_sequence<int, P>{});
      }
      store_tile(cm0, cn0);
      if (!more) break;
      vt = vn;
      behind = cm0 + BM <= p.M;
    }
  }

  if constexpr (EPI != EPI_ARGMAX) {
    if constexpr (!PERSIST) store_tile(m0, n0);
  } else {
    // greedy head: optional logits, then the per-row first maximum of the
    // tile; the partials go through ring slot 0 once every wave is done
    // reading it (a full barrier: each wave's LDS reads complete first)
    __syncthreads();
    float* bv = reinterpret_cast<float*>(L0);
    int* bi = reinterpret_cast<int*>(L0) + WN * BM;
#pragma unroll
    for (int i = 0; i < MF; ++i) {
      const int rl = wm * TM + i * 16 + (lane & 15);
      const int row = m0 + rl;
      float best = -INFINITY;
      int bidx = 0x7fffffff;
#pragma unroll
      for (int j = 0; j < NF; ++j) {
        const int f = n0 + wn * TN + j * 16 + fl;
        if (f >= p.N) continue;
        const f32x4 v = acc[i][j];
        if (p.C && row < p.M)
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
      if ((lane >> 4) == 0) { bv[wn * BM + rl] = best; bi[wn * BM + rl] = bidx; }
    }
    __syncthreads();
    for (int rl = tid; rl < BM; rl += NW * 64) {
      const int row = m0 + rl;
      if (row >= p.M) continue;
      float best = bv[rl];
      int bidx = bi[rl];
#pragma unroll
      for (int w = 1; w < WN; ++w)
        if (bv[w * BM + rl] > best) { best = bv[w * BM + rl]; bidx = bi[w * BM + rl]; }
      p.av[(int64_t)(n0 / BN) * p.M + row] = best;
      p.ai[(int64_t)(n0 / BN) * p.M + row] = bidx;
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
  int threads = 256;
};

// Compute units of the current device (one persistent workgroup each).
int cu_count() {
  static int counts[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!counts[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    counts[dev] = n;
  }
  return counts[dev];
}

// Workgroups of a persistent launch over `total` tiles: one per CU, a
// multiple of 8 so that each stays on its XCD's run of tiles.
int persist_grid(int total) {
  const int g = cu_count() / 8 * 8;
  return total <= g || g < 8 ? total : g;
}

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

// Shapes where the LDS-streaming kernel (gemm_lds_kernel) measured faster
// than every register-streaming tile above, same conditions (weights
// rotated past the Infinity Cache).  Fields: M, N, K, epilogue, whether the
// entry splits K into slabs, then rows x features per workgroup (BM, BN),
// waves along M (WM; NW / WM along N), ring depth P, K slabs, k-blocks per
// workgroup, waves per workgroup (NW: 4, or 8 for two per SIMD); the
// comment gives the register kernel's time and this one's (a second pair,
// "8 waves, later run": the earlier 4-wave entry and this one, timed side by
// side on one box).  Entries marked "wide" are 8-wave alternatives of a
// 4-wave entry, taken when the caller asks for them (GemmCall::wide), with
// the 4-wave entry's time and theirs, alone on one box: faster alone, they
// speed up the decode chunk's critical path but slow its concurrent branch,
// where they take more of each CU from the critical kernels (measured at 64
// and 256 rows; at 128 rows they slowed the chunk in either branch, at 512
// rows they sped it up in both).
#define PHOTON_GEMM_LDS_TUNED(X) \
  X(16, 1536, 1536, EPI_STORE, 1, 32, 32, 2, 6, 4, 6, 4) /* 4.1 -> 3.1 us */ \
  X(16, 1536, 6144, EPI_STORE, 1, 32, 64, 2, 6, 8, 12, 4) /* 7.7 -> 6.0 us */ \
  X(16, 4608, 1536, EPI_STORE, 1, 32, 64, 2, 6, 2, 12, 4) /* 6.3 -> 5.6 us */ \
  X(16, 6144, 1536, EPI_GELU, 0, 32, 32, 2, 6, 1, 24, 4) /* 8.2 -> 6.8 us */ \
  X(32, 768, 768, EPI_STORE, 1, 32, 32, 2, 4, 4, 3, 4) /* 3.8 -> 2.7 us */ \
  X(32, 768, 3072, EPI_STORE, 1, 32, 32, 2, 6, 8, 6, 4) /* 4.5 -> 3.2 us */ \
  X(32, 2304, 768, EPI_STORE, 1, 32, 64, 1, 4, 4, 3, 4) /* 3.8 -> 3.2 us */ \
  X(32, 3072, 768, EPI_GELU, 0, 32, 32, 2, 6, 1, 12, 4) /* 5.4 -> 3.9 us */ \
  X(32, 3072, 768, EPI_STORE, 1, 32, 32, 2, 6, 2, 6, 4) /* 4.2 -> 3.2 us */ \
  X(64, 1536, 1536, EPI_STORE, 1, 32, 64, 1, 6, 4, 6, 4) /* 4.9 -> 3.5 us */ \
  X(64, 1536, 1536, EPI_STORE, 1, 64, 64, 2, 6, 4, 6, 8) /* wide: 4.7 -> 4.1 us */ \
  X(64, 1536, 6144, EPI_STORE, 1, 64, 64, 2, 6, 8, 12, 4) /* 10.0 -> 7.1 us */ \
  X(64, 1536, 6144, EPI_STORE, 1, 64, 64, 2, 6, 8, 12, 8) /* wide: 8.6 -> 7.8 us */ \
  X(64, 4608, 1536, EPI_STORE, 1, 64, 64, 2, 6, 2, 12, 4) /* 7.8 -> 5.3 us */ \
  X(64, 4608, 1536, EPI_STORE, 1, 64, 64, 2, 6, 2, 12, 8) /* wide: 7.8 -> 6.7 us */ \
  X(64, 6144, 1536, EPI_GELU, 0, 64, 32, 2, 6, 1, 24, 4) /* 12.9 -> 8.9 us */ \
  X(64, 6144, 1536, EPI_STORE, 1, 64, 64, 2, 6, 2, 12, 4) /* 9.9 -> 7.6 us */ \
  X(64, 6144, 1536, EPI_STORE, 0, 64, 32, 2, 6, 1, 24, 4) /* 10.9 -> 8.0 us */ \
  X(64, 32000, 1536, EPI_ARGMAX, 0, 64, 128, 2, 4, 1, 24, 4) /* 25.1 -> 22.8 us */ \
  X(128, 768, 768, EPI_STORE, 1, 32, 32, 2, 6, 2, 6, 4) /* 4.0 -> 3.1 us */ \
  X(128, 768, 3072, EPI_STORE, 1, 64, 32, 2, 6, 4, 12, 4) /* 6.1 -> 4.2 us */ \
  X(128, 2304, 768, EPI_STORE, 1, 32, 32, 2, 4, 2, 6, 4) /* 5.5 -> 4.0 us */ \
  X(128, 3072, 768, EPI_GELU, 0, 32, 32, 2, 6, 1, 12, 4) /* 7.8 -> 4.8 us */ \
  X(128, 3072, 768, EPI_STORE, 1, 64, 32, 4, 6, 1, 12, 4) /* 6.0 -> 4.1 us */ \
  X(128, 3072, 768, EPI_STORE, 0, 32, 64, 2, 6, 1, 12, 4) /* 7.1 -> 4.2 us */ \
  X(128, 32000, 768, EPI_ARGMAX, 0, 128, 128, 4, 4, 1, 12, 8) /* 20.4 -> 17.2 us; 8 waves, later run: 15.1 -> 13.7 us */ \
  X(256, 1536, 1536, EPI_STORE, 1, 64, 64, 2, 4, 2, 12, 4) /* 8.5 -> 5.2 us */ \
  X(256, 1536, 1536, EPI_STORE, 1, 64, 64, 2, 4, 2, 12, 8) /* wide: 7.3 -> 5.2 us */ \
  X(256, 32000, 1536, EPI_ARGMAX, 0, 256, 128, 4, 3, 1, 24, 8) /* 8 waves against the register tile: 44.3 -> 32.0 us */ \
  X(256, 1536, 3072, EPI_STORE, 1, 64, 64, 2, 6, 2, 24, 4) /* 12.0 -> 7.0 us */ \
  X(256, 1536, 6144, EPI_STORE, 1, 128, 128, 2, 4, 8, 12, 4) /* 17.0 -> 12.9 us */ \
  X(256, 1536, 6144, EPI_STORE, 1, 128, 128, 4, 4, 8, 12, 8) /* wide: 14.1 -> 13.0 us */ \
  X(256, 3072, 1536, EPI_STORE, 1, 64, 64, 2, 6, 1, 24, 4) /* 11.9 -> 7.0 us */ \
  X(256, 4608, 1536, EPI_STORE, 1, 128, 64, 4, 4, 1, 24, 4) /* 14.0 -> 9.7 us */ \
  X(256, 4608, 1536, EPI_STORE, 1, 128, 128, 4, 4, 2, 12, 8) /* wide: 15.1 -> 12.1 us */ \
  X(256, 6144, 1536, EPI_GELU, 0, 128, 64, 4, 4, 1, 24, 4) /* 22.2 -> 17.1 us */ \
  X(256, 6144, 1536, EPI_GELU, 0, 128, 64, 4, 4, 1, 24, 8) /* wide: 18.5 -> 15.0 us */ \
  X(256, 6144, 1536, EPI_STORE, 1, 128, 128, 2, 4, 2, 12, 4) /* 17.1 -> 13.3 us */ \
  X(256, 6144, 1536, EPI_STORE, 0, 128, 64, 4, 4, 1, 24, 4) /* 19.1 -> 13.8 us */ \
  X(512, 1536, 1536, EPI_STORE, 1, 128, 64, 4, 4, 2, 12, 8) /* 12.8 -> 6.9 us; 8 waves, later run: 10.3 -> 7.0 us */ \
  X(512, 1536, 3072, EPI_STORE, 1, 128, 64, 4, 4, 2, 24, 4) /* 16.5 -> 10.2 us */ \
  X(512, 1536, 6144, EPI_STORE, 1, 128, 128, 4, 4, 4, 24, 8) /* 25.7 -> 18.9 us; 8 waves, later run: 20.6 -> 19.3 us */ \
  X(512, 3072, 1536, EPI_STORE, 1, 128, 64, 4, 4, 1, 24, 4) /* 16.9 -> 9.9 us */ \
  X(512, 3072, 1536, EPI_STORE, 0, 128, 64, 4, 4, 1, 24, 4) /* 18.5 -> 10.1 us */ \
  X(512, 4608, 1536, EPI_STORE, 1, 256, 128, 4, 3, 2, 12, 8) /* 20.7 -> 15.0 us; 8 waves, later run: 22.9 -> 17.8 us */ \
  X(512, 6144, 1536, EPI_GELU, 0, 128, 128, 4, 4, 1, 24, 8) /* 32.5 -> 23.5 us; 8 waves, later run: 25.4 -> 21.2 us */ \
  X(512, 32000, 1536, EPI_ARGMAX, 0, 256, 128, 4, 3, 1, 24, 8) /* 83.0 -> 78.8 us; 8 waves, later run: 73.9 -> 53.8 us */

struct Tuned {
  int M, N, K, epi, split, MB, NI, WK, P, ks, nkb;
  bool ntw;
  GemmKernel fn;
};
struct TunedL {
  int M, N, K, epi, split, BM, BN, WM, P, ks, nkb, nw;
  GemmKernel fn;
};
#define PHOTON_LDS_ENTRY(M_, N_, K_, E_, S_, BM_, BN_, WM_, P_, KS_, NKB_, NW_) \
  {M_, N_, K_, E_, S_, BM_, BN_, WM_, P_, KS_, NKB_, NW_, gemm_lds_kernel<BM_, BN_, WM_, P_, E_, NKB_, NW_>},
const TunedL kTunedL[] = {PHOTON_GEMM_LDS_TUNED(PHOTON_LDS_ENTRY)};
#undef PHOTON_LDS_ENTRY

const TunedL* find_tuned_lds(int M, int N, int K, int epi, bool allow_split, bool wide) {
  const TunedL* hit = nullptr;
  int best = -1;
  for (const TunedL& t : kTunedL) {
    if (t.M != M || t.N != N || t.K != K || t.epi != epi) continue;
    if (t.split && !allow_split) continue;
    // slabs when the caller takes them, then the wave count it prefers
    const int score = (t.split ? 2 : 0) + ((t.nw == 8) == wide ? 1 : 0);
    if (score > best) {
      best = score;
      hit = &t;
    }
  }
  return hit;
}
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

constexpr int kBigM = 2048;   // rows from which the prompt-sized plan applies
constexpr int kBigP = 3;

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
Plan plan_bf16(int M, int N, int K, int epi, bool allow_split, bool wide) {
  if (const TunedL* t = find_tuned_lds(M, N, K, epi, allow_split, wide))
    return Plan{0, 0, 0, (M + t->BM - 1) / t->BM, (N + t->BN - 1) / t->BN, t->ks, t->fn, 64 * t->nw};
  if (const Tuned* t = find_tuned(M, N, K, epi, allow_split)) {
    const int BM = 16 * t->MB, BN = 16 * t->NI * (4 / t->WK);
    return Plan{t->MB, t->NI, t->WK, (M + BM - 1) / BM, (N + BN - 1) / BN, t->ks, t->fn};
  }
  // prompt-sized GEMMs (many row tiles): the LDS-streaming kernel with a run
  // time k loop and eight waves (two per SIMD, so one's LDS reads overlap
  // the other's matrix products): 256 x 256 tiles (4 x 2 waves of 64 x 128,
  // two 64 KB stages) for outputs at least 4096 wide, else 128 x 256 (2 x 4
  // waves of 64 x 64, three stages); 1.1-1.4x the four-wave 128 x 256 tile
  if (M >= kBigM && K % 64 == 0 && (epi == EPI_STORE || epi == EPI_GELU)) {
    if (N >= 4096 && (K / 64) % 2 == 0) {
      GemmKernel fn = epi == EPI_STORE ? gemm_lds_kernel<256, 256, 4, 2, EPI_STORE, 0, 8>
                                       : gemm_lds_kernel<256, 256, 4, 2, EPI_GELU, 0, 8>;
      return Plan{0, 0, 0, (M + 255) / 256, (N + 255) / 256, 1, fn, 512};
    }
    if ((K / 64) % kBigP == 0) {
      GemmKernel fn = epi == EPI_STORE ? gemm_lds_kernel<128, 256, 2, kBigP, EPI_STORE, 0, 8>
                                       : gemm_lds_kernel<128, 256, 2, kBigP, EPI_GELU, 0, 8>;
      return Plan{0, 0, 0, (M + 127) / 128, (N + 255) / 256, 1, fn, 512};
    }
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
  return plan_bf16(M, N, K, EPI_ARGMAX, false, false).n_tiles;
}

int gemm_splits(int dtype, int M, int N, int K, int wide) {
  if (dtype == 0) return 1;
  return plan_bf16(M, N, K, EPI_STORE, true, wide != 0).ksplit;
}

// QKV projection with RoPE and the K/V append in its epilogue.  Prompts:
// 256-row tiles two heads wide (8 waves, 4 along M; each wave's columns are
// one head), three ring stages where two fit the LDS, else two; persistent
// workgroups for the two-stage tile of 96-wide heads.  Decode steps of 64-512
// rows: 64-row tiles (below).
namespace {
GemmKernel qkv_rope_kernel(int hd, int K, int M, bool* persist, int* rows, int* threads) {
  GemmKernel fn = nullptr;
  int P = 0, BM = 256, NT = 512;
  bool pst = false;
  if (M >= kBigM) {
    if (hd == 64) { fn = gemm_lds_kernel<256, 128, 4, 3, EPI_ROPE, 0, 8>; P = 3; }
    if (hd == 96) { fn = gemm_lds_kernel<256, 192, 4, 2, EPI_ROPE, 0, 8, true>; P = 2; pst = true; }
    if (hd == 128) { fn = gemm_lds_kernel<256, 256, 4, 2, EPI_ROPE, 0, 8>; P = 2; }
  } else if (M >= 64 && M <= 512) {
    // decode steps of 64-512 rows: 64-row tiles of 4 waves (2 x 2, 32 rows x
    // one head each), four ring stages; M/64 x 3H/2 workgroups
    BM = 64;
    NT = 256;
    if (hd == 64) { fn = gemm_lds_kernel<64, 128, 2, 4, EPI_ROPE, 0, 4>; P = 4; }
    if (hd == 96) { fn = gemm_lds_kernel<64, 192, 2, 4, EPI_ROPE, 0, 4>; P = 4; }
  }
  if (!fn || K % 64 || (K / 64) % P) return nullptr;
  if (persist) *persist = pst;
  if (rows) *rows = BM;
  if (threads) *threads = NT;   // 64 x the tile's waves (its launch bound)
  return fn;
}
bool aligned(const void* ptr, int bytes) { return ((uintptr_t)ptr % bytes) == 0; }
}  // namespace

int gemm_qkv_rope_supported(const GemmCall& g, const RopeKvCall& rc) {
  if (g.dtype != 1 || rc.dtype != 1 || rc.M != g.M) return 0;
  if (!qkv_rope_kernel(rc.hd, g.K, g.M, nullptr, nullptr, nullptr) || rc.d != rc.H * rc.hd || g.N != 3 * rc.d || (3 * rc.H) % 2) return 0;
  if (g.lda % 8 || !aligned(g.A, 16) || !aligned(g.W, 16) || !aligned(rc.q_out, 16) || !aligned(rc.Kc, 8) ||
      !aligned(rc.Vc, 8) || !aligned(rc.rope, 16) || rc.seq_stride % 4 || rc.rows_per_seq < 1)
    return 0;
  return 1;
}

hipError_t launch_gemm_qkv_rope(const GemmCall& g, const RopeKvCall& rc, hipStream_t st) {
  if (!gemm_qkv_rope_supported(g, rc)) return hipErrorInvalidValue;
  bool pst = false;
  int BM = 256, NT = 512;
  GemmKernel fn = qkv_rope_kernel(rc.hd, g.K, g.M, &pst, &BM, &NT);
  const int BN = 2 * rc.hd;
  GemmP p{};
  p.A = (const bf16_t*)g.A; p.lda = g.lda; p.W = (const bf16_t*)g.W;
  p.M = g.M; p.N = g.N; p.K = g.K;
  p.m_tiles = (g.M + BM - 1) / BM; p.n_tiles = g.N / BN; p.ksplit = 1;
  p.q = rc.q_out; p.Kc = (bf16_t*)rc.Kc; p.Vc = (bf16_t*)rc.Vc; p.rope = rc.rope;
  p.seq_stride = rc.seq_stride; p.cap = rc.cap; p.rows_per_seq = rc.rows_per_seq; p.seq0 = rc.seq0;
  p.pos_add = rc.pos_add; p.d = rc.d; p.pos_dev = rc.pos_dev; p.pos_mul = rc.pos_mul;
  PH_LAUNCH(fn, pst ? persist_grid(p.m_tiles * p.n_tiles) : p.m_tiles * p.n_tiles, NT, 0, st, p);
  return hipGetLastError();
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
  const Plan pl = plan_bf16(g.M, g.N, g.K, g.epi, g.epi == EPI_STORE && g.allow_split, g.wide != 0);
  GemmP p{(const bf16_t*)g.A, g.lda, (const bf16_t*)g.W, g.M, g.N, g.K,
          g.C, g.ldc, (bf16_t*)g.Cb, g.amax_val, g.amax_idx, pl.m_tiles, pl.n_tiles,
          pl.ksplit, (int64_t)g.M * g.ldc};
  if (pl.fn) {
    PH_LAUNCH(pl.fn, pl.m_tiles * pl.n_tiles * pl.ksplit, pl.threads, 0, st, p);
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
