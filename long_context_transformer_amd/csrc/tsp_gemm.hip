// tsp_gemm.hip -- bf16 "NT" GEMM family on gfx950 MFMA for the TSP rank-shard layer.
//
// Every projection of the layer multiplies activations [M, K] by a weight stored
// [N, K] (out_features x in_features), so both operands are contiguous along the
// reduction: C[M, N] = A[M, K] B[N, K]^T. One kernel template serves the four uses
// (TSP summary §2: local QKV projections, W_O, and the gated-MLP shard passes), each
// with its own fused epilogue:
//   EpiQKV      Q to a dense buffer, K/V rows scattered to their global zigzag positions
//   EpiBf16     plain bf16 store (W_O)
//   EpiSwiGLU   two weights at once (W1, W3); stores silu(G) * U as bf16
//   EpiAcc      fp32 accumulator, overwrite or add (the down projection of a shard)
//
// Three kernels share the epilogues. gemm_p (the persistent path, below) takes the large
// shapes: 256 x 256 tiles (256 x 128 per weight for the gated pair; 256 x 128 for a single
// weight where 256 x 256 tiles would leave much of a round of CUs idle), one wave per SIMD,
// the 16 x 16 x 32 MFMA, one workgroup per CU walking its tiles. gemm_fast (the "fast
// path") serves the other operands that take 16-byte chunks, with smaller tiles or k extents
// gemm_p does not take; gemm_nt, register-staged, serves the rest (only the tiny workload's
// odd shard width):
// Tiling of gemm_nt: 256 threads = 4 waves in a 2 x 2 grid over a BM x BN output tile;
// each wave owns a (BM/2) x (BN/2) block made of 32 x 32 MFMA tiles
// (v_mfma_f32_32x32x16_bf16). K advances in stages of 64 through a double-buffered LDS
// tile: while the MFMAs run on stage k, the global loads of stage k+1 are in flight in
// registers, then written to the other LDS buffer; one barrier per stage. In LDS each
// operand row holds 64 bf16 as eight 16-byte chunks stored at position
// chunk ^ ((row / 2) % 8), so the 16-byte fragment reads of 16 consecutive rows at one
// chunk hit 16 distinct bank groups.
// Both kernels take the weight tile as the MFMA's A operand and the activation tile as B,
// so the 32 x 32 result gives each lane four consecutive output columns of one row
// (8-byte bf16 or 16-byte fp32 stores; gemm_fast pairs the half-waves for 16-byte bf16
// stores).
// Workgroup -> tile: XCD-contiguous ranges (xcd_remap), then groups of 8 row-tiles
// walked column-major so tiles running together on one XCD share A and B in its L2.
#include <algorithm>

#include "tsp_device.h"
#include "tsp_internal.h"

namespace tsp {
namespace {

constexpr int BK = 64;
constexpr int kThreads = 256;
constexpr int kGroupM = 8;

struct Operands {
  const bf16_t* a;
  int64_t lda;
  const bf16_t* b;
  const bf16_t* b2;  // second weight of the gated pair (same shape and stride as b)
  int64_t ldb;
  int M, N, K;
};

// 16-byte chunk (8 bf16) of `row`, elements k .. k+7, of an operand with `rows` rows;
// zero outside the operand. VEC: K % 8 == 0, ld % 8 == 0, 16-byte aligned base.
template <bool VEC>
__device__ __forceinline__ uint4 load_chunk(const bf16_t* base, int64_t ld, int row, int rows, int k,
                                            int K) {
  if constexpr (VEC) {
    if (row < rows && k < K) return *reinterpret_cast<const uint4*>(base + (int64_t)row * ld + k);
    return make_uint4(0u, 0u, 0u, 0u);
  } else {
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (row < rows) {
      const bf16_t* p = base + (int64_t)row * ld;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t v = (k + e < K) ? (uint32_t)p[k + e] : 0u;
        w[e >> 1] |= v << (16 * (e & 1));
      }
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
}

__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ ((row >> 1) & 7)) << 3); }

// ---------------------------------------------------------------------------- epilogues
// Epilogues with bf16 output (kWide) also take 8 columns at once, already packed (see the
// lane exchange in gemm_fast): one 16-byte store per lane where the row allows it.
__device__ __forceinline__ bf16_t bf16_at(const uint4& w, int e) {
  const uint32_t word = e < 2 ? w.x : e < 4 ? w.y : e < 6 ? w.z : w.w;
  return (bf16_t)(word >> (16 * (e & 1)));
}
__device__ __forceinline__ void store8_bf16(bf16_t* p, const uint4& w, int valid) {
  if (valid >= 8 && (reinterpret_cast<uintptr_t>(p) & 15u) == 0) {
    *reinterpret_cast<uint4*>(p) = w;
  } else {
    for (int e = 0; e < 8 && e < valid; ++e) p[e] = bf16_at(w, e);
  }
}

// Unchecked stores for whole tiles (the persistent kernel): row(m) does the per-row address
// work once, put8 / put4 store 8 bf16 or 4 fp32 columns at n without bounds or alignment
// tests; vec_ok says whether the destination takes 16-byte (bf16) or 16-byte fp32 stores at
// every multiple of 8 (4) columns.
struct EpiBf16 {
  static constexpr bool kWide = true;
  bf16_t* c;
  int64_t ldc;
  struct Row {
    bf16_t* p;
  };
  __device__ __forceinline__ bool vec_ok() const { return ((reinterpret_cast<uintptr_t>(c) & 15u) == 0) && ldc % 8 == 0; }
  __device__ __forceinline__ Row row(int m) const { return Row{c + (int64_t)m * ldc}; }
  __device__ __forceinline__ void put8(const Row& r, int n, const uint4& w) const {
    *reinterpret_cast<uint4*>(r.p + n) = w;
  }
  __device__ __forceinline__ static uint2 pack(const f32x4& v) { return pack_bf16x4(v[0], v[1], v[2], v[3]); }
  __device__ __forceinline__ void store8(int m, int n, const uint4& w, int M, int N) const {
    if (m >= M || n >= N) return;
    store8_bf16(c + (int64_t)m * ldc + n, w, N - n);
  }
  __device__ __forceinline__ void operator()(int m, int n, const f32x4& v, int M, int N) const {
    if (m >= M || n >= N) return;
    bf16_t* p = c + (int64_t)m * ldc + n;
    if (n + 4 <= N && (ldc & 3) == 0) {
      *reinterpret_cast<uint2*>(p) = pack_bf16x4(v[0], v[1], v[2], v[3]);
    } else {
      for (int e = 0; e < 4 && n + e < N; ++e) p[e] = to_bf16(v[e]);
    }
  }
};

struct EpiQKV {
  static constexpr bool kWide = true;
  bf16_t* q;  // may be null
  bf16_t* k;
  bf16_t* v;
  int d;       // model width (row stride of q, k, v)
  int dg;      // output columns [0,dg) are Q, [dg,2dg) K, [2dg,3dg) V (dg = d for all heads)
  int col0;    // model column of output column 0 of each part (a head group's first column)
  int R;       // local rows per sequence (2C)
  int64_t C;   // zigzag chunk length
  int rank, D;
  int64_t S;
  struct Row {
    bf16_t *q, *k, *v;  // row m's Q row and its K/V rows, at column col0
  };
  __device__ __forceinline__ bool vec_ok() const {
    const uintptr_t a = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v);
    return (a & 15u) == 0 && d % 8 == 0 && col0 % 8 == 0 && dg % 8 == 0;
  }
  __device__ __forceinline__ Row row(int m) const {
    const int b = m / R;
    const int64_t kv = ((int64_t)b * S + zigzag_pos(m - b * R, C, rank, D)) * d + col0;
    return Row{q ? q + (int64_t)m * d + col0 : nullptr, k + kv, v + kv};
  }
  __device__ __forceinline__ void put8(const Row& r, int n, const uint4& w) const {
    const int which = (n >= dg) + (n >= 2 * dg);
    bf16_t* p = which == 0 ? r.q : which == 1 ? r.k : r.v;
    if (p) *reinterpret_cast<uint4*>(p + (n - which * dg)) = w;
  }
  __device__ __forceinline__ void operator()(int m, int n, const f32x4& val, int M, int N) const {
    if (m >= M || n >= N) return;
    const int which = n / dg;
    const int col = col0 + n - which * dg;
    const uint2 packed = pack_bf16x4(val[0], val[1], val[2], val[3]);
    if (which == 0) {
      if (q) *reinterpret_cast<uint2*>(q + (int64_t)m * d + col) = packed;
      return;
    }
    const int b = m / R;
    const int i = m - b * R;
    const int64_t row = (int64_t)b * S + zigzag_pos(i, C, rank, D);
    bf16_t* dst = (which == 1 ? k : v) + row * d + col;
    *reinterpret_cast<uint2*>(dst) = packed;
  }
  __device__ __forceinline__ static uint2 pack(const f32x4& v) { return pack_bf16x4(v[0], v[1], v[2], v[3]); }
  // 8 columns never straddle Q/K/V: dg and n are multiples of 8.
  __device__ __forceinline__ void store8(int m, int n, const uint4& w, int M, int N) const {
    if (m >= M || n >= N) return;
    const int which = n / dg;
    const int col = col0 + n - which * dg;
    if (which == 0) {
      if (q) store8_bf16(q + (int64_t)m * d + col, w, N - n);
      return;
    }
    const int b = m / R;
    const int i = m - b * R;
    const int64_t row = (int64_t)b * S + zigzag_pos(i, C, rank, D);
    store8_bf16((which == 1 ? k : v) + row * d + col, w, N - n);
  }
};

struct EpiSwiGLU {
  static constexpr bool kWide = true;
  bf16_t* h;
  int64_t ldh;
  struct Row {
    bf16_t* p;
  };
  __device__ __forceinline__ bool vec_ok() const { return ((reinterpret_cast<uintptr_t>(h) & 15u) == 0) && ldh % 8 == 0; }
  __device__ __forceinline__ Row row(int m) const { return Row{h + (int64_t)m * ldh}; }
  __device__ __forceinline__ void put8(const Row& r, int n, const uint4& w) const {
    *reinterpret_cast<uint4*>(r.p + n) = w;
  }
  __device__ __forceinline__ void shift_cols(int64_t c) { h += c; }
  // silu(g) = g sigma(g), with the hardware reciprocal (about 1 ulp) instead of an IEEE division
  // (a ten-instruction sequence per value in the epilogue); g -> -inf gives g * rcp(inf) = -0.
  __device__ __forceinline__ static float silu(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }
  __device__ __forceinline__ static uint2 pack(const f32x4& g, const f32x4& u) {
    return pack_bf16x4(silu(g[0]) * u[0], silu(g[1]) * u[1], silu(g[2]) * u[2], silu(g[3]) * u[3]);
  }
  __device__ __forceinline__ void store8(int m, int n, const uint4& w, int M, int N) const {
    if (m >= M || n >= N) return;
    store8_bf16(h + (int64_t)m * ldh + n, w, N - n);
  }
  __device__ __forceinline__ void operator()(int m, int n, const f32x4& g, const f32x4& u, int M,
                                             int N) const {
    if (m >= M || n >= N) return;
    float r[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = silu(g[e]) * u[e];
    bf16_t* p = h + (int64_t)m * ldh + n;
    if (n + 4 <= N && (ldh & 3) == 0) {
      *reinterpret_cast<uint2*>(p) = pack_bf16x4(r[0], r[1], r[2], r[3]);
    } else {
      for (int e = 0; e < 4 && n + e < N; ++e) p[e] = to_bf16(r[e]);
    }
  }
};

// fp32 accumulator plus this partial, stored as bf16 (the last step of an fp32
// accumulation; first: the partial alone).
struct EpiAccBf16 {
  static constexpr bool kWide = false;
  const float* acc;
  bf16_t* out;
  int64_t ld;
  int first;
  struct Row {
    const float* a;
    bf16_t* o;
  };
  __device__ __forceinline__ bool vec_ok() const {
    return ((reinterpret_cast<uintptr_t>(acc) & 15u) == 0) && ((reinterpret_cast<uintptr_t>(out) & 7u) == 0) && ld % 4 == 0;
  }
  __device__ __forceinline__ Row row(int m) const { return Row{acc + (int64_t)m * ld, out + (int64_t)m * ld}; }
  __device__ __forceinline__ void put4(const Row& r, int n, const f32x4& v) const {
    f32x4 o = v;
    if (!first) o += *reinterpret_cast<const f32x4*>(r.a + n);
    *reinterpret_cast<uint2*>(r.o + n) = pack_bf16x4(o[0], o[1], o[2], o[3]);
  }
  __device__ __forceinline__ void operator()(int m, int n, const f32x4& v, int M, int N) const {
    if (m >= M || n >= N) return;
    f32x4 o = v;
    if (!first) o += *reinterpret_cast<const f32x4*>(acc + (int64_t)m * ld + n);
    *reinterpret_cast<uint2*>(out + (int64_t)m * ld + n) = pack_bf16x4(o[0], o[1], o[2], o[3]);
  }
};

struct EpiAcc {
  static constexpr bool kWide = false;
  float* c;
  int64_t ldc;
  int accumulate;
  struct Row {
    float* p;
  };
  __device__ __forceinline__ bool vec_ok() const { return ((reinterpret_cast<uintptr_t>(c) & 15u) == 0) && ldc % 4 == 0; }
  __device__ __forceinline__ Row row(int m) const { return Row{c + (int64_t)m * ldc}; }
  __device__ __forceinline__ void put4(const Row& r, int n, const f32x4& v) const {
    f32x4 o = v;
    if (accumulate) o += *reinterpret_cast<const f32x4*>(r.p + n);
    *reinterpret_cast<f32x4*>(r.p + n) = o;
  }
  __device__ __forceinline__ void operator()(int m, int n, const f32x4& v, int M, int N) const {
    if (m >= M || n >= N) return;
    float* p = c + (int64_t)m * ldc + n;
    if (n + 4 <= N && (ldc & 3) == 0) {
      f32x4 o = v;
      if (accumulate) o += *reinterpret_cast<const f32x4*>(p);
      *reinterpret_cast<f32x4*>(p) = o;
    } else {
      for (int e = 0; e < 4 && n + e < N; ++e) p[e] = accumulate ? p[e] + v[e] : v[e];
    }
  }
};

// ------------------------------------------------------------------------------- kernel
template <int BM, int BN, bool DUAL, bool VEC, class Epi>
__global__ __launch_bounds__(kThreads) void gemm_nt(Operands op, Epi epi, int tiles_m, int tiles_n) {
  constexpr int NB = DUAL ? 2 : 1;
  constexpr int WTM = BM / 2, WTN = BN / 2;
  constexpr int MI = WTM / 32, NI = WTN / 32;
  constexpr int AP = BM / 32, BP = BN / 32;  // load passes: 256 threads cover 32 rows x 8 chunks
  __shared__ __attribute__((aligned(16))) bf16_t smem[2][(BM + NB * BN) * BK];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, hl = lane >> 5;

  const int t = xcd_remap(blockIdx.x, tiles_m * tiles_n);
  const int span = kGroupM * tiles_n;
  const int first_m = (t / span) * kGroupM;
  const int gsz = min(tiles_m - first_m, kGroupM);
  const int in_g = t - (t / span) * span;
  const int m0 = (first_m + in_g % gsz) * BM;
  const int n0 = (in_g / gsz) * BN;

  const int lc = tid & 7;  // chunk this thread moves
  const int lr = tid >> 3;  // first row this thread moves

  uint4 ra[AP];
  uint4 rb[NB][BP];
  auto gload = [&](int k0) {
#pragma unroll
    for (int p = 0; p < AP; ++p) ra[p] = load_chunk<VEC>(op.a, op.lda, m0 + lr + 32 * p, op.M, k0 + 8 * lc, op.K);
#pragma unroll
    for (int p = 0; p < BP; ++p) rb[0][p] = load_chunk<VEC>(op.b, op.ldb, n0 + lr + 32 * p, op.N, k0 + 8 * lc, op.K);
    if constexpr (DUAL) {
#pragma unroll
      for (int p = 0; p < BP; ++p) rb[1][p] = load_chunk<VEC>(op.b2, op.ldb, n0 + lr + 32 * p, op.N, k0 + 8 * lc, op.K);
    }
  };
  auto sstore = [&](int buf) {
    bf16_t* sa = smem[buf];
#pragma unroll
    for (int p = 0; p < AP; ++p) *reinterpret_cast<uint4*>(sa + swz(lr + 32 * p, lc)) = ra[p];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      bf16_t* sb = sa + BM * BK + nb * BN * BK;
#pragma unroll
      for (int p = 0; p < BP; ++p) *reinterpret_cast<uint4*>(sb + swz(lr + 32 * p, lc)) = rb[nb][p];
    }
  };

  f32x16 acc[NB][MI][NI];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) acc[nb][mi][ni] = f32x16{};

  const int nk = (op.K + BK - 1) / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
    const bf16_t* sa = smem[cur];
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int ch = 2 * ks + hl;
      bf16x8 af[MI];
      bf16x8 bfr[NB][NI];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
        af[mi] = as_bf16x8(*reinterpret_cast<const uint4*>(sa + swz(wm * WTM + mi * 32 + l32, ch)));
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const bf16_t* sb = sa + BM * BK + nb * BN * BK;
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          bfr[nb][ni] = as_bf16x8(*reinterpret_cast<const uint4*>(sb + swz(wn * WTN + ni * 32 + l32, ch)));
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
          for (int ni = 0; ni < NI; ++ni) acc[nb][mi][ni] = mfma32x32x16(bfr[nb][ni], af[mi], acc[nb][mi][ni]);
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    const int m = m0 + wm * WTM + mi * 32 + l32;
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * WTN + ni * 32 + 8 * g + 4 * hl;
        const f32x4 v0 = {acc[0][mi][ni][4 * g], acc[0][mi][ni][4 * g + 1], acc[0][mi][ni][4 * g + 2],
                          acc[0][mi][ni][4 * g + 3]};
        if constexpr (DUAL) {
          const f32x4 v1 = {acc[1][mi][ni][4 * g], acc[1][mi][ni][4 * g + 1], acc[1][mi][ni][4 * g + 2],
                            acc[1][mi][ni][4 * g + 3]};
          epi(m, n, v0, v1, op.M, op.N);
        } else {
          epi(m, n, v0, op.M, op.N);
        }
      }
    }
  }
}

// ------------------------------------------------------------------- fast path (16-byte operands)
// Same contraction and epilogues, with the operand tiles moved straight from global memory
// into LDS (16-byte global_load_lds per lane, no register staging, no bounds predicates):
//   * k advances in stages of 64 through two LDS buffers: after the barrier of stage kt the
//     loads of stage kt+1 go to the other buffer while the MFMAs of stage kt run;
//   * a tile row holds 64 bf16 = eight 16-byte chunks, chunk c of row r stored at
//     c ^ ((r / 2) % 8), so the 16 rows read by 16 lanes at one chunk hit 16 distinct
//     bank groups;
//   * rows past M or N repeat the last row (their outputs are never stored); chunks past
//     K (the last stage when K % 64 != 0) come from a block of zeros;
//   * 8 waves per 256-wide tile (two per SIMD), each owning 128 x 64 outputs (128 x 32 per
//     weight for the gated pair), so one wave's MFMAs cover the other's LDS latency.

// Chunk swizzle of the stage tiles: rows of 4 chunks (k stage 32) rotate by (r / 4) % 4,
// rows of 8 chunks (k stage 64) by (r / 2) % 8, so the 16 rows read by 16 lanes at one
// chunk hit 16 distinct bank groups.
template <int CPR>
__device__ __forceinline__ int swz_chunk(int r) { return CPR == 4 ? (r >> 2) & 3 : (r >> 1) & 7; }

// Zeros read in place of chunks past K (16 bytes per lane). Never written.
__device__ __attribute__((aligned(16))) uint4 kZeroChunks[64];

// Shard tables of the fused MLP launches, which cover all D weight shards a rank sees in
// one launch each (passed by value in the kernel arguments).
//   SEG_N (gate/up): the column tiles are grouped by shard; a tile of shard j multiplies by
//     W1_j / W3_j (b[j], b2[j]; N = rows of one shard) and stores into column block j of H.
//   SEG_K (down): the reduction runs over the shards one after another in ring order, the
//     fp32 accumulators staying in registers; at ring step t the A columns start at a_col[t]
//     and the weight is b[t] (K = columns of one shard, zero-filled past K per shard).
// (Plain int constants and a named trait: an unnamed enum or std::conditional in a kernel's
// signature can mangle differently in the host and device compilations.)
constexpr int SEG_NONE = 0, SEG_N = 1, SEG_K = 2;
constexpr int kMaxShards = 32;
struct NoShards {};
struct Shards {
  const bf16_t* b[kMaxShards];
  const bf16_t* b2[kMaxShards];
  int64_t a_col[kMaxShards];
  int64_t out_col;  // SEG_N: columns between the output blocks of consecutive shards
  int tn;           // SEG_N: column tiles per shard
  int nks;          // SEG_K: 32-wide k stages per shard
  int count;        // number of shards
  // SEG_K in gemm_p only: parts > 1 splits the shards of every tile into `parts` equal runs,
  // each its own work item; run p (in ring order) writes its fp32 sum to the epilogue's output
  // (p = 0) or to part_c + (p - 1) part_stride (EpiAcc, overwrite), summed afterwards.
  int parts;
  float* part_c;
  int64_t part_stride;
};
template <int SEG>
struct SegArgOf {
  typedef Shards type;
};
template <>
struct SegArgOf<SEG_NONE> {
  typedef NoShards type;
};
template <int SEG>
using SegArg = typename SegArgOf<SEG>::type;

template <int BM, int BN, int WM, int WN, bool DUAL, int SEG, int KB, int GM, class Epi>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64)
__attribute__((amdgpu_waves_per_eu((BM / WM) * (BN / WN) / 4, (BM / WM) * (BN / WN) / 4)))
void gemm_fast(Operands op, Epi epi, int tiles_m, int tiles_n, SegArg<SEG> sg) {
  // KB: k extent of one LDS stage (2-stage ring). A tile row holds KB bf16 = CPR 16-byte
  // chunks; chunk c of row r sits at c ^ sw(r).
  constexpr int ROWB = KB * 2, CPR = KB / 8, RPI = 1024 / ROWB;  // rows per 1 KB DMA instruction
  static_assert(KB == 32 || KB == 64, "stage depth");
  auto sw = [](int r) { return swz_chunk<CPR>(r); };
  constexpr int NWN = BN / WN, NWAVE = (BM / WM) * NWN;
  constexpr int NB = DUAL ? 2 : 1;
  constexpr int MI = WM / 32, NI = WN / 32;
  constexpr int ATILE = BM * KB * 2, BTILE = BN * KB * 2;
  constexpr int STAGE = ATILE + NB * BTILE;
  constexpr int AINS = ATILE / 1024 / NWAVE;  // 1 KB DMA instructions per wave per stage
  constexpr int BINS = BTILE / 1024 / NWAVE;
  constexpr int LOADS = AINS + NB * BINS;     // per thread per stage
  static_assert(AINS >= 1 && AINS * NWAVE * 1024 == ATILE, "A tile split");
  static_assert(BINS >= 1 && BINS * NWAVE * 1024 == BTILE, "B tile split");
  __shared__ __attribute__((aligned(1024))) char s0[STAGE];
  __shared__ __attribute__((aligned(1024))) char s1[STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / NWN, wn = wave % NWN;
  const int l32 = lane & 31, hl = lane >> 5;

  const int t = xcd_remap(blockIdx.x, tiles_m * tiles_n);
  const int span = GM * tiles_n;
  const int first_m = (t / span) * GM;
  const int gsz = min(tiles_m - first_m, GM);
  const int in_g = t - (t / span) * span;
  const int m0 = (first_m + in_g % gsz) * BM;
  int n0 = (in_g / gsz) * BN;
  const char* abase = reinterpret_cast<const char*>(op.a);
  const char* bbase = reinterpret_cast<const char*>(op.b);
  const char* b2base = reinterpret_cast<const char*>(DUAL ? op.b2 : op.b);
  if constexpr (SEG == SEG_N) {
    const int nt = in_g / gsz;
    const int j = nt / sg.tn;
    n0 = (nt - j * sg.tn) * BN;
    bbase = reinterpret_cast<const char*>(sg.b[j]);
    b2base = reinterpret_cast<const char*>(sg.b2[j]);
    epi.shift_cols(j * sg.out_col);
  }

  // DMA instruction p of this wave covers tile rows 16 (p NWAVE + wave) + lane/4, physical
  // chunk lane%4, i.e. logical chunk (lane%4) ^ ((row/4)%4).
  uint32_t aoff[AINS], boff[BINS];
  int akc[AINS], bkc[BINS];
#pragma unroll
  for (int p = 0; p < AINS; ++p) {
    const int row = RPI * (p * NWAVE + wave) + lane / CPR;
    const int c = (lane % CPR) ^ sw(row);
    aoff[p] = (uint32_t)min(m0 + row, op.M - 1) * (uint32_t)(op.lda * 2) + 16 * c;
    akc[p] = 8 * c;
  }
#pragma unroll
  for (int p = 0; p < BINS; ++p) {
    const int row = RPI * (p * NWAVE + wave) + lane / CPR;
    const int c = (lane % CPR) ^ sw(row);
    boff[p] = (uint32_t)min(n0 + row, op.N - 1) * (uint32_t)(op.ldb * 2) + 16 * c;
    bkc[p] = 8 * c;
  }
  // Stages are issued strictly in order; under SEG_K (seg, kk) is the shard step and the
  // stage within it of the next one.
  // Under SEG_K the bases of the current shard step and of the next one are kept in
  // registers; the table is read once per shard step, a whole step before it is needed.
  int seg = 0, kk = 0;
  const char* seg_a = abase;
  const char* seg_b = bbase;
  const char* nxt_a = abase;
  const char* nxt_b = bbase;
  if constexpr (SEG == SEG_K) {
    seg_a = abase + sg.a_col[0] * 2;
    seg_b = reinterpret_cast<const char*>(sg.b[0]);
    if (sg.count > 1) {
      nxt_a = abase + sg.a_col[1] * 2;
      nxt_b = reinterpret_cast<const char*>(sg.b[1]);
    }
  }
  auto issue = [&] __device__(char* st, int kt) {
    const char* ab = abase;
    const char* bb = bbase;
    if constexpr (SEG == SEG_K) {
      ab = seg_a;
      bb = seg_b;
      kt = kk;
      if (++kk == sg.nks) {
        kk = 0;
        ++seg;
        seg_a = nxt_a;
        seg_b = nxt_b;
        if (seg + 1 < sg.count) {
          nxt_a = abase + sg.a_col[seg + 1] * 2;
          nxt_b = reinterpret_cast<const char*>(sg.b[seg + 1]);
        }
      }
    }
    const int k0 = kt * KB;
    ab += (size_t)k0 * 2;
    bb += (size_t)k0 * 2;
    const char* b2 = b2base + (size_t)k0 * 2;
    const uint32_t la = lds_addr(st) + wave * 1024;
    if (k0 + KB <= op.K) {
#pragma unroll
      for (int p = 0; p < AINS; ++p) dma16_sbase(ab, aoff[p], la + p * NWAVE * 1024);
#pragma unroll
      for (int p = 0; p < BINS; ++p) dma16_sbase(bb, boff[p], la + ATILE + p * NWAVE * 1024);
      if constexpr (DUAL) {
#pragma unroll
        for (int p = 0; p < BINS; ++p) dma16_sbase(b2, boff[p], la + ATILE + BTILE + p * NWAVE * 1024);
      }
    } else {  // last stage with K % 64 != 0: chunks past K read zeros
      const void* z = &kZeroChunks[lane];
#pragma unroll
      for (int p = 0; p < AINS; ++p)
        dma16_vaddr(k0 + akc[p] < op.K ? (const void*)(ab + aoff[p]) : z, la + p * NWAVE * 1024);
#pragma unroll
      for (int p = 0; p < BINS; ++p)
        dma16_vaddr(k0 + bkc[p] < op.K ? (const void*)(bb + boff[p]) : z, la + ATILE + p * NWAVE * 1024);
      if constexpr (DUAL) {
#pragma unroll
        for (int p = 0; p < BINS; ++p)
          dma16_vaddr(k0 + bkc[p] < op.K ? (const void*)(b2 + boff[p]) : z, la + ATILE + BTILE + p * NWAVE * 1024);
      }
    }
  };

  // Fragment byte offsets within a stage for each 16-wide k step (row l32 of a 32-row
  // block; the swizzle of a row depends only on its index within an aligned 32-row block).
  constexpr int KSTEPS = KB / 16;
  int fo[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) fo[ks] = l32 * ROWB + 16 * ((2 * ks + hl) ^ sw(l32));

  f32x16 acc[NB][MI][NI];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) acc[nb][mi][ni] = f32x16{};

  // The fragments of k step ks+1 are read from LDS while the MFMAs of step ks run (two
  // register sets), so only the first step of a stage waits for its reads.
  auto compute = [&] __device__(const char* st) {
    bf16x8 af[2][MI];
    bf16x8 bfr[2][NB][NI];
    auto load = [&] __device__(int ks, int b) {
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
        af[b][mi] = as_bf16x8(*reinterpret_cast<const uint4*>(st + (wm * WM + 32 * mi) * ROWB + fo[ks]));
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          bfr[b][nb][ni] = as_bf16x8(
              *reinterpret_cast<const uint4*>(st + ATILE + nb * BTILE + (wn * WN + 32 * ni) * ROWB + fo[ks]));
    };
    load(0, 0);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const int b = ks & 1;
      if (ks + 1 < KSTEPS) load(ks + 1, b ^ 1);
      // keep the next step's reads above this step's MFMAs (the scheduler would otherwise
      // sink them to their uses and reuse one register set)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
          for (int ni = 0; ni < NI; ++ni)
            acc[nb][mi][ni] = mfma32x32x16(bfr[b][nb][ni], af[b][mi], acc[nb][mi][ni]);
    }
  };

  int nk = (op.K + KB - 1) / KB;
  if constexpr (SEG == SEG_K) nk = sg.count * sg.nks;
  issue(s0, 0);
  {
    // Stage kt: wait for its loads, barrier, load stage kt+1 into the buffer of stage kt-1,
    // then the MFMAs of stage kt.
    auto body2 = [&] __device__(int kt, const char* cur, char* other) {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");  // no LDS read moves above the barrier
      if (kt + 1 < nk) issue(other, kt + 1);
      compute(cur);
    };
    for (int kt = 0; kt < nk; kt += 2) {
      body2(kt, s0, s1);
      if (kt + 1 < nk) body2(kt + 1, s1, s0);
    }
  }

  if constexpr (Epi::kWide) {
    // bf16 output: lane (row, hl) holds columns 8g + 4hl .. +3 of each 8-column block g of a
    // 32-column tile. The two half-waves swap halves so that lane hl holds whole blocks hl and
    // hl + 2, then store 16 bytes per lane (each row gets 32 contiguous bytes per store).
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int m = m0 + wm * WM + mi * 32 + l32;
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        uint2 pk[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 v0 = {acc[0][mi][ni][4 * g], acc[0][mi][ni][4 * g + 1], acc[0][mi][ni][4 * g + 2],
                            acc[0][mi][ni][4 * g + 3]};
          if constexpr (DUAL) {
            const f32x4 v1 = {acc[1][mi][ni][4 * g], acc[1][mi][ni][4 * g + 1], acc[1][mi][ni][4 * g + 2],
                              acc[1][mi][ni][4 * g + 3]};
            pk[g] = Epi::pack(v0, v1);
          } else {
            pk[g] = Epi::pack(v0);
          }
        }
        const uint2 s0 = hl ? pk[0] : pk[1];
        const uint2 s1 = hl ? pk[2] : pk[3];
        const uint2 r0 = make_uint2(__shfl_xor(s0.x, 32), __shfl_xor(s0.y, 32));
        const uint2 r1 = make_uint2(__shfl_xor(s1.x, 32), __shfl_xor(s1.y, 32));
        const uint4 b0 = hl ? make_uint4(r0.x, r0.y, pk[1].x, pk[1].y) : make_uint4(pk[0].x, pk[0].y, r0.x, r0.y);
        const uint4 b1 = hl ? make_uint4(r1.x, r1.y, pk[3].x, pk[3].y) : make_uint4(pk[2].x, pk[2].y, r1.x, r1.y);
        const int nt = n0 + wn * WN + ni * 32;
        epi.store8(m, nt + 8 * hl, b0, op.M, op.N);
        epi.store8(m, nt + 16 + 8 * hl, b1, op.M, op.N);
      }
    }
  } else {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int m = m0 + wm * WM + mi * 32 + l32;
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + wn * WN + ni * 32 + 8 * g + 4 * hl;
          const f32x4 v0 = {acc[0][mi][ni][4 * g], acc[0][mi][ni][4 * g + 1], acc[0][mi][ni][4 * g + 2],
                            acc[0][mi][ni][4 * g + 3]};
          if constexpr (DUAL) {
            const f32x4 v1 = {acc[1][mi][ni][4 * g], acc[1][mi][ni][4 * g + 1], acc[1][mi][ni][4 * g + 2],
                              acc[1][mi][ni][4 * g + 3]};
            epi(m, n, v0, v1, op.M, op.N);
          } else {
            epi(m, n, v0, op.M, op.N);
          }
        }
      }
    }
  }
}

// ------------------------------------------------------ persistent path (one wave per SIMD)
// 256 x 256 output tiles (256 x 128 per weight for the gated pair) computed by 4 waves, one
// per SIMD, each owning 128 x 128 outputs (128 x 64 per weight), on the 16 x 16 x 32 bf16
// MFMA: per 32-wide k step a wave reads 8 weight and 8 activation fragments (16 bytes per
// lane each) for its 64 MFMAs. Of the two bf16 MFMA shapes this one moves half the
// accumulator data per flop (k = 32 instead of 16), and on random data the matrix cores run
// at a clock some 15% higher with it than with 32 x 32 x 16 at the same issue rate.
// Registers: the 64 accumulators (64 x 4 fp32) fill a0..a255, fixed AGPRs named only in
// inline assembly (the MFMAs and the epilogue's read-out); every such statement lists them
// as clobbered, so the compiler keeps its own values out of them and never moves them. The
// fragments (two sets of 16) and everything else live in VGPRs.
// The grid holds one workgroup per CU (the two 64 KB stage buffers fill its LDS); workgroup
// b computes the tiles v = b, b + gridDim.x, ... (each XCD still walks a contiguous range of
// the grouped tile order, 32 tiles at a time). The k stages (64 wide) of consecutive tiles
// form one software pipeline over the two buffers: the workgroup's stage g lives in buffer
// g % 2, and the loads of stage g + 2 go into buffer g % 2 during stage g's second k step,
// whether g + 2 belongs to this tile or the next, so the next tile's first two stages load
// while this tile's epilogue runs.
// Stage g: k step 0 runs on fragments read during stage g-1 and reads those of step 1; then
// this wave waits for its reads and for its loads of stage g+1 and meets the other waves at
// the barrier (every wave has read stage g and every load of stage g+1 has landed); k step
// 1 then issues the 16 loads of stage g+2 and the 16 reads of stage g+1's step 0, one of
// each per four MFMAs. Scheduling barriers pin that placement.
// A k extent that is an odd multiple of 32 ends with a half stage (one k step): its loads
// take chunks 0..3 twice (in bounds; the copy is never read) and the barrier falls in the
// middle of its k step.
#define TSP_STR(x) #x
#define TSP_G10(p) TSP_STR(a##p##0), TSP_STR(a##p##1), TSP_STR(a##p##2), TSP_STR(a##p##3), TSP_STR(a##p##4), \
    TSP_STR(a##p##5), TSP_STR(a##p##6), TSP_STR(a##p##7), TSP_STR(a##p##8), TSP_STR(a##p##9)
// a0 .. a255
#define TSP_ACC_AGPRS "a0", "a1", "a2", "a3", "a4", "a5", "a6", "a7", "a8", "a9", TSP_G10(1), TSP_G10(2), TSP_G10(3), \
    TSP_G10(4), TSP_G10(5), TSP_G10(6), TSP_G10(7), TSP_G10(8), TSP_G10(9), TSP_G10(10), TSP_G10(11), TSP_G10(12),   \
    TSP_G10(13), TSP_G10(14), TSP_G10(15), TSP_G10(16), TSP_G10(17), TSP_G10(18), TSP_G10(19), TSP_G10(20),         \
    TSP_G10(21), TSP_G10(22), TSP_G10(23), TSP_G10(24), "a250", "a251", "a252", "a253", "a254", "a255"

// a[R .. R+3] (+)= A-fragment x B-fragment (16 x 16 x 32). Lane l supplies row l % 16 of A
// and column l % 16 of B, each with k = 8 (l / 16) .. + 7; the result holds rows
// 4 (l / 16) .. + 3 of column l % 16 in lane l.
template <int R>
__device__ __forceinline__ void gmma(const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 a[%2:%3], %0, %1, a[%2:%3]" ::"v"(a), "v"(b), "n"(R), "n"(R + 3)
               : TSP_ACC_AGPRS);
}
template <int R>
__device__ __forceinline__ void gmma0(const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 a[%2:%3], %0, %1, 0" ::"v"(a), "v"(b), "n"(R), "n"(R + 3)
               : TSP_ACC_AGPRS);
}
// a[R .. R+3] into VGPRs.
template <int R>
__device__ __forceinline__ f32x4 acc_read(void) {
  float x0, x1, x2, x3;
  asm volatile(
      "v_accvgpr_read_b32 %0, a[%4]\n\tv_accvgpr_read_b32 %1, a[%5]\n\tv_accvgpr_read_b32 %2, a[%6]\n\t"
      "v_accvgpr_read_b32 %3, a[%7]"
      : "=v"(x0), "=v"(x1), "=v"(x2), "=v"(x3)
      : "n"(R), "n"(R + 1), "n"(R + 2), "n"(R + 3)
      : TSP_ACC_AGPRS);
  return f32x4{x0, x1, x2, x3};
}

int device_cus() {
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

// Tile shapes: 256 x 256 (one weight), 256 x (128 + 128) (DUAL: two weights) and, NARROW,
// 256 x 128 (one weight; waves of 128 x 64) for launches where the 256 x 256 tiles would leave
// much of the last round of CUs idle.
template <bool DUAL, bool NARROW = false>
struct PGeom {
  static constexpr int KB = 64, ROWB = KB * 2, CPR = KB / 8, RPI = 1024 / ROWB;
  static constexpr int BM = 256, BN = DUAL || NARROW ? 128 : 256, WM = 128, WN = DUAL || NARROW ? 64 : 128;
  static constexpr int NWN = BN / WN, NWAVE = 4;
  static constexpr int NB = DUAL ? 2 : 1;
  static constexpr int MB = WM / 16, NBK = WN / 16, NW = NB * NBK;  // activation / weight blocks of 16
  static constexpr int ATILE = BM * KB * 2, BTILE = BN * KB * 2;
  static constexpr int STAGE = ATILE + NB * BTILE;
  static constexpr int AINS = ATILE / 1024 / NWAVE, BINS = BTILE / 1024 / NWAVE;
  // Per 32-wide k step and wave: MFMAs, fragment reads, and (per stage) 16-byte load instructions.
  static constexpr int NMF = MB * NW, NRD = MB + NW, NLD = AINS + NB * BINS;
  // One read (load) every RS (DS) MFMAs of a step; in the half step of a half stage, every RSH (DSH).
  static constexpr int RS = NMF / NRD, DS = NMF / NLD;
  static constexpr int RSH = NMF / 2 / NRD > 0 ? NMF / 2 / NRD : 1, DSH = NMF / 2 / NLD > 0 ? NMF / 2 / NLD : 1;
  static_assert(NWN * (BM / WM) == NWAVE && RS >= 1 && DS >= 1 && NRD <= NMF / 2 && NLD <= NMF / 2,
                "four waves; every read and load fits its step");
  static_assert(!(DUAL && NARROW), "the gated pair has one tile shape");
  // MFMA i of a k step: activation block mb = i / NW, weight block w = i % NW = (nb, nbk);
  // its accumulator a[4 (w MB + mb) ..].
  static constexpr int mb_of(int i) { return i / NW; }
  static constexpr int w_of(int i) { return i % NW; }
  static constexpr int acc_of(int i) { return 4 * (w_of(i) * MB + mb_of(i)); }
};

// Logical 16-byte chunk c of tile row r sits at physical chunk c ^ (r % 8): the 8 rows that
// 8 consecutive lanes of a fragment read hit 8 distinct bank groups.
__device__ __forceinline__ int swz8(int r) { return r & 7; }

// PF > 0: during each full stage g, one 4-byte load per activation row and wave pulls the
// activation lines of stage g + PF (same k segment) into the caches, so that its 16-byte
// stage loads two stages later find them there; the newest load of the wave is then such a
// prefetch, which the stage wait leaves in flight. It pays where the activation operand does
// not fit the MALL and comes from HBM (the down projection's gated hidden at 7B S=128K:
// 3600 -> 3310 cycles per stage); where the operands sit in the MALL it costs slightly.
template <bool DUAL, int SEG, int GM, class Epi, int PF = 0, bool NARROW = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_p(Operands op, Epi epi, int tiles_m, int tiles_n, SegArg<SEG> sg) {
  using G = PGeom<DUAL, NARROW>;
  constexpr int KB = G::KB, ROWB = G::ROWB, CPR = G::CPR, RPI = G::RPI;
  constexpr int BM = G::BM, BN = G::BN, WM = G::WM, WN = G::WN, NWN = G::NWN, NWAVE = G::NWAVE;
  constexpr int NB = G::NB, MB = G::MB, NBK = G::NBK, NW = G::NW;
  constexpr int ATILE = G::ATILE, BTILE = G::BTILE, STAGE = G::STAGE, AINS = G::AINS, BINS = G::BINS;
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];
  __shared__ __attribute__((aligned(256))) char pf_lds[PF > 0 ? NWAVE * 256 : 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / NWN, wn = wave % NWN;
  const int l16 = lane & 15, lg = lane >> 4;
  const int tiles = tiles_m * tiles_n;
  // Stages per k segment (the whole reduction, or one shard under SEG_K), segments, and the
  // runs of segments a tile is split into (SEG_K parts).
  const int nks = (op.K + KB - 1) / KB;
  int nseg = 1, parts = 1;
  if constexpr (SEG == SEG_K) {
    nseg = sg.count;
    parts = sg.parts > 1 ? sg.parts : 1;
  }
  const int total = tiles * parts;
  const bool khalf = (op.K % KB) != 0;
  if ((int)blockIdx.x >= total) return;
  auto seg_lo = [&](int p) { return p * nseg / parts; };

  // Work item v of the grouped order: row tile, column tile, (SEG_N) shard and (SEG_K) part;
  // the part is the slowest index.
  struct TileAt {
    int m0, n0, j, p;
  };
  auto tile_at = [&](int v) {
    int t = xcd_remap(v, total);
    const int pt = t / tiles;
    t -= pt * tiles;
    const int span = GM * tiles_n;
    const int first_m = (t / span) * GM;
    const int gsz = min(tiles_m - first_m, GM);
    const int in_g = t - (t / span) * span;
    TileAt r;
    r.p = pt;
    r.m0 = (first_m + in_g % gsz) * BM;
    int nt = in_g / gsz;
    r.j = 0;
    if constexpr (SEG == SEG_N) {
      r.j = nt / sg.tn;
      nt -= r.j * sg.tn;
    }
    r.n0 = nt * BN;
    return r;
  };

  // ---- load side. Per-lane byte offsets of the load instructions for the rows of the tile
  // the loads are working on: the current tile, or from the stage whose loads first reach
  // into the workgroup's next tile on, that one. The k position and the operand bases are
  // scalar. DMA instruction p of this wave covers tile rows RPI (p NWAVE + wave) + lane / CPR
  // at physical chunk lane % CPR, i.e. logical chunk (lane % CPR) ^ swz8(row), which is the
  // same chunk for every p (rows of one instruction step by RPI NWAVE, a multiple of 8).
  // Rows past M or N repeat the last row.
  auto row_of = [&](int p) { return RPI * (p * NWAVE + wave) + lane / CPR; };
  const int lc = (lane % CPR) ^ swz8(row_of(0));
  const uint32_t hsub = lc >= 4 ? 64u : 0u;  // bytes back to chunk c - 4 (half stages)
  uint32_t oa[AINS], ob[BINS];
  uint32_t opf = 0;  // prefetch: byte offset of activation row m0 + 64 wave + lane
  auto offsets = [&](int v) {
    const TileAt tl = tile_at(v);
    if constexpr (PF > 0) opf = (uint32_t)min(tl.m0 + wave * 64 + lane, op.M - 1) * (uint32_t)(op.lda * 2);
#pragma unroll
    for (int p = 0; p < AINS; ++p)
      oa[p] = (uint32_t)min(tl.m0 + row_of(p), op.M - 1) * (uint32_t)(op.lda * 2) + 16 * lc;
#pragma unroll
    for (int p = 0; p < BINS; ++p)
      ob[p] = (uint32_t)min(tl.n0 + row_of(p), op.N - 1) * (uint32_t)(op.ldb * 2) + 16 * lc;
  };
  const char* const abase = reinterpret_cast<const char*>(op.a);
  // Weight bases of tile v (SEG_N: its shard's).
  auto wbase = [&](int v, int w) -> const char* {
    if constexpr (SEG == SEG_N) {
      const int j = tile_at(v).j;
      return reinterpret_cast<const char*>(w ? sg.b2[j] : sg.b[j]);
    }
    return reinterpret_cast<const char*>(w && DUAL ? op.b2 : op.b);
  };
  const char* wb = wbase(blockIdx.x, 0);
  const char* wb2 = wbase(blockIdx.x, 1);
  // Loads of stage kt of segment s of the loads' tile, instruction by instruction
  // (p = 0 .. 15), into the stage buffer at LDS address la + 1 KB x wave.
  struct Ld {
    const char *a, *b, *b2;
    uint32_t hm;  // ~0 for a half stage
  };
  auto ld_of = [&](int s, int kt) {
    Ld l;
    const int k0 = kt * KB;
    const char* a = abase;
    const char* b = wb;
    if constexpr (SEG == SEG_K) {
      a = abase + sg.a_col[s] * 2;
      b = reinterpret_cast<const char*>(sg.b[s]);
    }
    l.a = a + (size_t)k0 * 2;
    l.b = b + (size_t)k0 * 2;
    l.b2 = wb2 + (size_t)k0 * 2;
    l.hm = k0 + KB <= op.K ? 0u : 0xffffffffu;
    return l;
  };
  auto dma = [&](int p, uint32_t la, const Ld& l) {
    const uint32_t back = hsub & l.hm;
    if (p < AINS) {
      dma16_sbase(l.a, oa[p] - back, la + p * NWAVE * 1024);
    } else {
      const int q = p - AINS;
      const int nb = q / BINS, pb = q % BINS;
      dma16_sbase(nb ? l.b2 : l.b, ob[pb] - back, la + ATILE + nb * BTILE + pb * NWAVE * 1024);
    }
  };

  // ---- compute side
  // Fragment byte offsets within a stage for each 32-wide k step: row l % 16 of a 16-row
  // block (every block starts at a multiple of 8, so the swizzle depends on l % 8 alone),
  // logical chunk 4 ks + l / 16.
  int fo[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) fo[ks] = l16 * ROWB + 16 * ((4 * ks + lg) ^ swz8(l16));
  bf16x8 fa[2][MB];  // activation fragments (MFMA B operand)
  bf16x8 fw[2][NW];  // weight fragments (MFMA A operand)
  // Read r (0..15) of k step ks from the stage at st into register set `set`: activation
  // block 0, the weight blocks, then activation blocks 1..7 (the order the MFMAs use them).
  auto rd = [&](int set, const char* st, int ks, int r) {
    if (r == 0 || r > NW) {
      const int mb = r == 0 ? 0 : r - NW;
      fa[set][mb] = as_bf16x8(*reinterpret_cast<const uint4*>(st + (wm * WM + 16 * mb) * ROWB + fo[ks]));
    } else {
      const int w = r - 1, nb = w / NBK, k = w % NBK;
      fw[set][w] = as_bf16x8(
          *reinterpret_cast<const uint4*>(st + ATILE + nb * BTILE + (wn * WN + 16 * k) * ROWB + fo[ks]));
    }
  };
  // MFMAs lo .. hi-1 of a k step on register set `set` (zero: the tile's first step, C = 0),
  // with, every rs-th MFMA from the first, read number (i - lo) / rs of k step rks of the
  // stage at rst into set rset (when rs != 0), and every ds-th MFMA from the (ds / 2)-th,
  // load number (i - lo) / ds of the stage *ld into the buffer at LDS address la (ds != 0).
  auto step = [&](const int set, const bool zero, auto LO, auto HI, const int rs, const char* rst, const int rset,
                  const int rks, const int ds, const Ld* ld, const uint32_t la) __attribute__((always_inline)) {
    static_for<G::NMF>([&](auto I) __attribute__((always_inline)) {
      constexpr int i = decltype(I)::value;
      if constexpr (i >= decltype(LO)::value && i < decltype(HI)::value) {
        constexpr int j = i - decltype(LO)::value;
        if (zero)
          gmma0<G::acc_of(i)>(fw[set][G::w_of(i)], fa[set][G::mb_of(i)]);
        else
          gmma<G::acc_of(i)>(fw[set][G::w_of(i)], fa[set][G::mb_of(i)]);
        if (rs && j % rs == 0 && j / rs < G::NRD) rd(rset, rst, rks, j / rs);
        if (ds && j % ds == ds / 2 && j / ds < G::NLD) dma(j / ds, la, *ld);
        __builtin_amdgcn_sched_barrier(0);
      }
    });
  };
  using I0 = std::integral_constant<int, 0>;
  using I32 = std::integral_constant<int, G::NMF / 2>;  // half a step
  using I64 = std::integral_constant<int, G::NMF>;      // a whole step

  // Prologue: stages 0 and 1 of the first tile (every tile has at least two), then the
  // first step's fragments.
  offsets(blockIdx.x);
  {
    const uint32_t base = lds_addr(smem) + wave * 1024;
    const int s0 = seg_lo(tile_at(blockIdx.x).p);
    const Ld l0 = ld_of(s0, 0);
    const Ld l1 = ld_of(s0, 1);
#pragma unroll
    for (int p = 0; p < G::NLD; ++p) dma(p, base, l0);
#pragma unroll
    for (int p = 0; p < G::NLD; ++p) dma(p, base + STAGE, l1);
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
#pragma unroll
  for (int r = 0; r < G::NRD; ++r) rd(0, smem, 0, r);

  // Waits for this wave's reads of the stage and its loads of the next one, then meets the
  // other waves: past it every wave has read the stage and every load of the next has landed.
  bool pf_out = false;  // the newest load of this wave is a prefetch
  auto sync = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    if (PF > 0 && pf_out) __builtin_amdgcn_s_waitcnt(waitcnt_vm(1));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  int g = 0;  // stages computed so far
  for (int v = blockIdx.x; v < total; v += gridDim.x) {
    const bool has_next = v + (int)gridDim.x < total;
    bool moved = false;  // the load offsets point at the next tile
    const int pv = tile_at(v).p;
    const int s_lo = seg_lo(pv), s_hi = seg_lo(pv + 1);
    const int s_next = has_next ? seg_lo(tile_at(v + gridDim.x).p) : 0;
    for (int s = s_lo; s < s_hi; ++s) {
      for (int kt = 0; kt < nks; ++kt, ++g) {
        const char* cur = smem + (g & 1) * STAGE;
        const char* nxt = smem + ((g + 1) & 1) * STAGE;
        const bool first = s == s_lo && kt == 0;
        // The stage two ahead: (s2, k2) of this tile or of the next; past the workgroup's
        // last stage, this stage again (into its own buffer, which nobody reads again).
        int s2 = s, k2 = kt + 2;
        bool nx = false;
        if (k2 >= nks) {
          k2 -= nks;
          if (++s2 == s_hi) {
            s2 = s_next;
            nx = true;
          }
        }
        if (nx && !has_next) {
          s2 = s;
          k2 = kt;
          nx = false;
        }
        if (nx && !moved) {
          offsets(v + gridDim.x);
          wb = wbase(v + gridDim.x, 0);
          wb2 = wbase(v + gridDim.x, 1);
          moved = true;
        }
        const Ld l2 = ld_of(s2, k2);
        const uint32_t la = lds_addr(cur) + wave * 1024;
        // Settle the scalar bookkeeping here, ahead of the MFMAs, not between a barrier and
        // the MFMAs that follow it.
        asm volatile("" ::"s"(l2.a), "s"(l2.b), "s"(l2.b2), "s"(l2.hm), "s"(la));
        if (kt + 1 < nks || !khalf) {
          if (first) step(0, true, I0{}, I64{}, G::RS, cur, 1, 1, 0, nullptr, 0u);
          else step(0, false, I0{}, I64{}, G::RS, cur, 1, 1, 0, nullptr, 0u);
          sync();
          step(1, false, I0{}, I64{}, G::RS, nxt, 0, 0, G::DS, &l2, la);
          if constexpr (PF > 0) {
            pf_out = kt + PF < nks;
            if (pf_out) {
              const char* ap = abase + (size_t)(kt + PF) * KB * 2;
              if constexpr (SEG == SEG_K) ap += sg.a_col[s] * 2;
              dma4_sbase(ap, opf, lds_addr(pf_lds) + wave * 256);
            }
          }
        } else {  // half stage: one k step, the barrier in its middle
          // Its second half still uses every weight fragment of set 0, so the next stage's
          // first fragments go to set 1 and move to set 0 afterwards.
          step(0, false, I0{}, I32{}, 0, cur, 0, 0, 0, nullptr, 0u);
          sync();
          step(0, false, I32{}, I64{}, G::RSH, nxt, 1, 0, G::DSH, &l2, la);
          pf_out = false;
#pragma unroll
          for (int w = 0; w < NW; ++w) fw[0][w] = fw[1][w];
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) fa[0][mb] = fa[1][mb];
        }
      }
    }
    // Epilogue: the accumulators of the last MFMAs are read many slots later; the nops
    // cover the read-after-write wait of the first ones read.
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::: TSP_ACC_AGPRS);
    const TileAt tl = tile_at(v);
    Epi e = epi;
    if constexpr (SEG == SEG_N) e.shift_cols(tl.j * sg.out_col);
    if constexpr (SEG == SEG_K && std::is_same<Epi, EpiAcc>::value)
      if (tl.p > 0) {
        e.c = sg.part_c + (int64_t)(tl.p - 1) * sg.part_stride;
        e.accumulate = 0;
      }
    const int m0 = tl.m0, n0 = tl.n0;
    // Activation block mb, weight blocks 2 q and 2 q + 1 of each weight: lane l holds outputs
    // (m = l % 16, n = 4 (l / 16) .. + 3) of each block. A tile wholly inside C whose
    // destination takes vector stores (FAST) does each row's address work once and stores
    // without per-store tests.
    auto tile = [&](auto FAST) __attribute__((always_inline)) {
      constexpr bool fast = decltype(FAST)::value;
      static_for<MB>([&](auto MBI) __attribute__((always_inline)) {
        constexpr int mb = decltype(MBI)::value;
        const int m = m0 + wm * WM + 16 * mb + l16;
        typename Epi::Row r{};
        if constexpr (fast) r = e.row(m);
        static_for<NBK / 2>([&](auto QI) __attribute__((always_inline)) {
          constexpr int q = decltype(QI)::value;
          constexpr int k0 = 2 * q, k1 = 2 * q + 1;
          const f32x4 g0 = acc_read<4 * (k0 * MB + mb)>();
          const f32x4 g1 = acc_read<4 * (k1 * MB + mb)>();
          f32x4 u0 = g0, u1 = g1;
          if constexpr (DUAL) {
            u0 = acc_read<4 * ((NBK + k0) * MB + mb)>();
            u1 = acc_read<4 * ((NBK + k1) * MB + mb)>();
          }
          const int nblk = n0 + wn * WN + 16 * k0;  // first column of the block pair
          if constexpr (Epi::kWide) {
            // Pack each block's 4 columns to bf16, then trade halves between lane groups:
            // after the swaps group 0 holds block 0 columns 0..7, group 1 block 1 columns
            // 0..7, group 2 block 0 columns 8..15, group 3 block 1 columns 8..15, with x the
            // lower 4 and y the upper 4 of the lane's 8: one 16-byte store each.
            uint2 p0, p1;
            if constexpr (DUAL) {
              p0 = Epi::pack(g0, u0);
              p1 = Epi::pack(g1, u1);
            } else {
              p0 = Epi::pack(g0);
              p1 = Epi::pack(g1);
            }
            uint32_t x0 = p0.x, x1 = p0.y, y0 = p1.x, y1 = p1.y;
            swap16(x0, y0);
            swap16(x1, y1);
            const uint4 w = make_uint4(x0, x1, y0, y1);
            const int col = nblk + 16 * (lg & 1) + 8 * (lg >> 1);
            if constexpr (fast) e.put8(r, col, w);
            else e.store8(m, col, w, op.M, op.N);
          } else {
            const int n = nblk + 4 * lg;
            if constexpr (DUAL) {
              e(m, n, g0, u0, op.M, op.N);
              e(m, n + 16, g1, u1, op.M, op.N);
            } else if constexpr (fast) {
              e.put4(r, n, g0);
              e.put4(r, n + 16, g1);
            } else {
              e(m, n, g0, op.M, op.N);
              e(m, n + 16, g1, op.M, op.N);
            }
          }
        });
      });
    };
    if (m0 + BM <= op.M && n0 + BN <= op.N && e.vec_ok()) tile(std::true_type{});
    else tile(std::false_type{});
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // the last stage's extra loads land before the LDS is freed
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <int BM, int BN, bool DUAL, bool VEC, class Epi>
hipError_t run_tiles(const Operands& op, const Epi& epi, hipStream_t s) {
  const int tm = (op.M + BM - 1) / BM;
  const int tn = (op.N + BN - 1) / BN;
  hipLaunchKernelGGL((gemm_nt<BM, BN, DUAL, VEC, Epi>), dim3(tm * tn), dim3(kThreads), 0, s, op, epi, tm, tn);
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, bool DUAL, int SEG = SEG_NONE, int GM = kGroupM, class Epi>
hipError_t run_fast(const Operands& op, const Epi& epi, hipStream_t s, SegArg<SEG> sg = {}) {
  constexpr int KB = 64;
  const int tm = (op.M + BM - 1) / BM;
  int tn = (op.N + BN - 1) / BN;
  if constexpr (SEG == SEG_N) {
    sg.tn = tn;
    tn *= sg.count;
  }
  if constexpr (SEG == SEG_K) sg.nks = (op.K + KB - 1) / KB;
  constexpr int threads = (BM / WM) * (BN / WN) * 64;
  hipLaunchKernelGGL((gemm_fast<BM, BN, WM, WN, DUAL, SEG, KB, GM, Epi>), dim3(tm * tn), dim3(threads), 0, s, op, epi, tm,
                     tn, sg);
  return hipGetLastError();
}

// The persistent kernel takes k extents (per shard under SEG_K) that are multiples of 32 and
// hold at least two 64-wide stages.
inline bool persist_ok(const Operands& op) { return op.K % 32 == 0 && op.K > 64; }

template <bool DUAL, int SEG = SEG_NONE, int GM = kGroupM, int PF = 0, bool NARROW = false, class Epi>
hipError_t run_persist(const Operands& op, const Epi& epi, hipStream_t s, SegArg<SEG> sg = {}) {
  constexpr int BM = PGeom<DUAL, NARROW>::BM, BN = PGeom<DUAL, NARROW>::BN, KB = 64;
  const int tm = (op.M + BM - 1) / BM;
  int tn = (op.N + BN - 1) / BN;
  if constexpr (SEG == SEG_N) {
    sg.tn = tn;
    tn *= sg.count;
  }
  if constexpr (SEG == SEG_K) sg.nks = (op.K + KB - 1) / KB;
  int total = tm * tn;
  if constexpr (SEG == SEG_K) total *= sg.parts > 1 ? sg.parts : 1;
  const int grid = total < device_cus() ? total : device_cus();
  hipLaunchKernelGGL((gemm_p<DUAL, SEG, GM, Epi, PF, NARROW>), dim3(grid), dim3(256), 0, s, op, epi, tm, tn, sg);
  return hipGetLastError();
}

// Operand requirements of the fast path: 16-byte chunks (K, strides multiples of 8
// elements, 16-byte aligned bases) and byte offsets of every row within 32 bits.
bool fast_ok(const Operands& op, bool dual) {
  const bool vec = (op.K % 8 == 0) && (op.lda % 8 == 0) && (op.ldb % 8 == 0) && aligned16(op.a) && aligned16(op.b) &&
                   (!dual || aligned16(op.b2));
  const uint64_t a_span = (uint64_t)(op.M - 1) * (uint64_t)op.lda * 2 + (uint64_t)op.K * 2;
  const uint64_t b_span = (uint64_t)(op.N - 1) * (uint64_t)op.ldb * 2 + (uint64_t)op.K * 2;
  return vec && a_span < (1ull << 32) && b_span < (1ull << 32);
}

// Large problems take the 256 x 256 tile (256 x 128 for the gated pair, which carries two
// accumulators); when that leaves fewer tiles than CUs the 128 x 128 (128 x 64) tile keeps
// the chip busy. Operands that cannot take 16-byte chunks (odd K or strides: only tiny
// shapes) use the register-staged kernel with element-wise loads.
constexpr int64_t kBigTileMin = 256;
// Single-weight GEMMs also have a 256 x 128 tile (64 x 64 per wave: one LDS fragment per MFMA
// against 0.75 for the 256 x 256 tile's 128 x 64 waves). Each tile fills one CU, so a launch
// runs in rounds of kCUs tiles; where the 256 x 256 tiles leave much of the last round idle
// (few row tiles: M of a few thousand) the 256 x 128 tile fills the rounds better.
constexpr int64_t kCUs = 256;
constexpr double kMidTileRate = 0.68;  // its per-CU rate relative to the 256 x 256 tile (measured)
enum class Tile { k256x256, k256x128, k128x128 };

double round_fill(int64_t tiles) {
  const int64_t rounds = (tiles + kCUs - 1) / kCUs;
  return (double)tiles / (double)(rounds * kCUs);
}

Tile choose_tile(int M, int N) {
  const int64_t tm = (M + 255) / 256;
  const int64_t t256 = tm * ((N + 255) / 256), t_mid = tm * ((N + 127) / 128);
  if (t256 >= kBigTileMin && round_fill(t256) >= kMidTileRate * round_fill(t_mid)) return Tile::k256x256;
  if (t_mid >= kCUs) return Tile::k256x128;
  return Tile::k128x128;
}

template <class Epi>
hipError_t run_single(const Operands& op, const Epi& epi, hipStream_t s) {
  if (!fast_ok(op, false)) {
    const bool vec = (op.K % 8 == 0) && (op.lda % 8 == 0) && (op.ldb % 8 == 0) && aligned16(op.a) && aligned16(op.b);
    return vec ? run_tiles<128, 128, false, true>(op, epi, s) : run_tiles<128, 128, false, false>(op, epi, s);
  }
  switch (choose_tile(op.M, op.N)) {
    case Tile::k256x256:
      if (persist_ok(op)) return run_persist<false>(op, epi, s);
      return run_fast<256, 256, 128, 64, false>(op, epi, s);
    case Tile::k256x128:
      if (persist_ok(op)) return run_persist<false, SEG_NONE, kGroupM, 0, true>(op, epi, s);
      return run_fast<256, 128, 64, 64, false>(op, epi, s);
    default: return run_fast<128, 128, 64, 64, false>(op, epi, s);
  }
}

template <class Epi>
hipError_t run_dual(const Operands& op, const Epi& epi, hipStream_t s) {
  if (!fast_ok(op, true)) {
    const bool vec = (op.K % 8 == 0) && (op.lda % 8 == 0) && (op.ldb % 8 == 0) && aligned16(op.a) &&
                     aligned16(op.b) && aligned16(op.b2);
    return vec ? run_tiles<128, 64, true, true>(op, epi, s) : run_tiles<128, 64, true, false>(op, epi, s);
  }
  const int64_t big = (int64_t)((op.M + 255) / 256) * ((op.N + 127) / 128);
  if (big >= kBigTileMin) {
    if (persist_ok(op)) return run_persist<true>(op, epi, s);
    return run_fast<256, 128, 128, 32, true>(op, epi, s);
  }
  return run_fast<128, 64, 64, 32, true>(op, epi, s);
}

}  // namespace

hipError_t launch_qkv(const void* x, const void* w_qkv, void* q_out, void* k_full, void* v_full, int B, int64_t S,
                      int D, int rank, int d, hipStream_t stream) {
  const int64_t C = S / (2 * D);
  const int R = (int)(2 * C);
  Operands op{static_cast<const bf16_t*>(x), d, static_cast<const bf16_t*>(w_qkv), nullptr, d, B * R, 3 * d, d};
  EpiQKV epi{static_cast<bf16_t*>(q_out), static_cast<bf16_t*>(k_full), static_cast<bf16_t*>(v_full), d, d, 0, R, C, rank,
             D, S};
  return run_single(op, epi, stream);
}

hipError_t launch_qkv_group(const void* x, const void* w_qkv_g, int group, int groups, void* q_out, void* k_full,
                            void* v_full, int B, int64_t S, int D, int rank, int d, hipStream_t stream) {
  const int64_t C = S / (2 * D);
  const int R = (int)(2 * C);
  const int dg = d / groups;
  Operands op{static_cast<const bf16_t*>(x), d, static_cast<const bf16_t*>(w_qkv_g), nullptr, d, B * R, 3 * dg, d};
  EpiQKV epi{static_cast<bf16_t*>(q_out), static_cast<bf16_t*>(k_full), static_cast<bf16_t*>(v_full), d, dg, group * dg, R,
             C, rank, D, S};
  return run_single(op, epi, stream);
}

hipError_t launch_wo_group(const void* o, const void* w_o_g, int group, int groups, float* acc, void* out, int M, int d,
                           int step, int steps, hipStream_t stream) {
  const int dg = d / groups;
  Operands op{static_cast<const bf16_t*>(o) + (int64_t)group * dg, d, static_cast<const bf16_t*>(w_o_g), nullptr, dg, M,
              d, dg};
  if (step == steps - 1) return run_single(op, EpiAccBf16{acc, static_cast<bf16_t*>(out), d, step == 0 ? 1 : 0}, stream);
  return run_single(op, EpiAcc{acc, d, step > 0 ? 1 : 0}, stream);
}

hipError_t launch_wo_pair(const void* o, const void* w_o_a, const void* w_o_b, int group, int groups, float* acc,
                          void* out, int M, int d, int first, int last, hipStream_t stream) {
  const int dg = d / groups;
  Operands op{static_cast<const bf16_t*>(o), d, static_cast<const bf16_t*>(w_o_a), nullptr, dg, M, d, dg};
  Shards sg{};
  sg.b[0] = static_cast<const bf16_t*>(w_o_a);
  sg.b[1] = static_cast<const bf16_t*>(w_o_b);
  sg.a_col[0] = (int64_t)group * dg;
  sg.a_col[1] = (int64_t)(group + 1) * dg;
  sg.count = 2;
  // Operands the 16-byte path cannot take run as two single-group launches.
  Operands chk = op;
  chk.a = op.a + sg.a_col[0];
  if (!fast_ok(chk, false) || !aligned16(w_o_b) || (dg * 2) % 16 != 0) {
    if (hipError_t e = launch_wo_group(o, w_o_a, group, groups, acc, out, M, d, first ? 0 : 1, 3, stream)) return e;
    return launch_wo_group(o, w_o_b, group + 1, groups, acc, out, M, d, last ? 2 : 1, 3, stream);
  }
  const bool big = choose_tile(M, d) == Tile::k256x256;
  if (last) {
    const EpiAccBf16 epi{acc, static_cast<bf16_t*>(out), d, first};
    if (big && persist_ok(op)) return run_persist<false, SEG_K>(op, epi, stream, sg);
    if (big) return run_fast<256, 256, 128, 64, false, SEG_K>(op, epi, stream, sg);
    return run_fast<128, 128, 64, 64, false, SEG_K>(op, epi, stream, sg);
  }
  const EpiAcc epi{acc, d, first ? 0 : 1};
  if (big && persist_ok(op)) return run_persist<false, SEG_K>(op, epi, stream, sg);
  if (big) return run_fast<256, 256, 128, 64, false, SEG_K>(op, epi, stream, sg);
  return run_fast<128, 128, 64, 64, false, SEG_K>(op, epi, stream, sg);
}

hipError_t launch_proj_bf16(const void* a, int64_t lda, const void* w, int64_t ldw, void* c, int64_t ldc, int M, int N,
                            int K, hipStream_t stream) {
  Operands op{static_cast<const bf16_t*>(a), lda, static_cast<const bf16_t*>(w), nullptr, ldw, M, N, K};
  EpiBf16 epi{static_cast<bf16_t*>(c), ldc};
  return run_single(op, epi, stream);
}

hipError_t launch_gate_up(const void* x, int64_t ldx, const void* w1, const void* w3, int64_t ldw, void* h, int64_t ldh,
                          int M, int Fs, int K, hipStream_t stream) {
  Operands op{static_cast<const bf16_t*>(x), ldx, static_cast<const bf16_t*>(w1), static_cast<const bf16_t*>(w3), ldw,
              M, Fs, K};
  EpiSwiGLU epi{static_cast<bf16_t*>(h), ldh};
  return run_dual(op, epi, stream);
}

hipError_t launch_down_acc(const void* h, int64_t ldh, const void* w2, int64_t ldw2, float* acc, int64_t ldacc, int M,
                           int N, int K, int accumulate, hipStream_t stream) {
  Operands op{static_cast<const bf16_t*>(h), ldh, static_cast<const bf16_t*>(w2), nullptr, ldw2, M, N, K};
  EpiAcc epi{acc, ldacc, accumulate};
  return run_single(op, epi, stream);
}

bool mlp_ring_fusable(const void* const* w1, const void* const* w3, const void* const* w2, int64_t ldw2, int D, int M,
                      int d, int Fs, int64_t ldh) {
  if (D < 1 || D > kMaxShards || Fs % 8 != 0 || d % 8 != 0 || ldw2 % 8 != 0 || ldh % 8 != 0) return false;
  for (int j = 0; j < D; ++j)
    if (!aligned16(w1[j]) || !aligned16(w3[j]) || !aligned16(w2[j])) return false;
  const uint64_t h_span = (uint64_t)(M - 1) * (uint64_t)ldh * 2 + (uint64_t)ldh * 2;
  const uint64_t w13_span = (uint64_t)Fs * (uint64_t)d * 2;
  const uint64_t w2_span = (uint64_t)(d - 1) * (uint64_t)ldw2 * 2 + (uint64_t)Fs * 2;
  const uint64_t x_span = (uint64_t)M * (uint64_t)d * 2;
  return h_span < (1ull << 32) && w13_span < (1ull << 32) && w2_span < (1ull << 32) && x_span < (1ull << 32);
}

hipError_t launch_gate_up_ring(const void* x, const void* const* w1, const void* const* w3, int D, void* h,
                               int64_t ldh, int64_t ldseg, int M, int Fs, int d, hipStream_t stream) {
  Operands op{static_cast<const bf16_t*>(x), d, nullptr, nullptr, d, M, Fs, d};
  EpiSwiGLU epi{static_cast<bf16_t*>(h), ldh};
  Shards sg{};
  for (int j = 0; j < D; ++j) {
    sg.b[j] = static_cast<const bf16_t*>(w1[j]);
    sg.b2[j] = static_cast<const bf16_t*>(w3[j]);
  }
  sg.out_col = ldseg;
  sg.count = D;
  op.b = sg.b[0];
  op.b2 = sg.b2[0];
  const int64_t big = (int64_t)((M + 255) / 256) * D * ((Fs + 127) / 128);
  if (big >= kBigTileMin) {
    if (persist_ok(op)) return run_persist<true, SEG_N>(op, epi, stream, sg);
    return run_fast<256, 128, 128, 32, true, SEG_N>(op, epi, stream, sg);
  }
  return run_fast<128, 64, 64, 32, true, SEG_N>(op, epi, stream, sg);
}

// out[m, :N] += part[m, :N]: the sum of the two halves of a split down projection.
__global__ __launch_bounds__(256) void add_rows_kernel(float* out, int64_t ldo, const float* part, int64_t ldp, int M,
                                                       int N4) {
  const int64_t n = (int64_t)M * N4;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t m = i / N4, c = (i - m * N4) * 4;
    f32x4* o = reinterpret_cast<f32x4*>(out + m * ldo + c);
    *o += *reinterpret_cast<const f32x4*>(part + m * ldp + c);
  }
}

hipError_t launch_down_ring(const void* h, int64_t ldh, int64_t ldseg, const void* const* w2, int64_t ldw2, int D,
                            int rank, float* out, int64_t ldout, int accumulate, int M, int N, int Fs, float* part,
                            hipStream_t stream) {
  Operands op{static_cast<const bf16_t*>(h), ldh, nullptr, nullptr, ldw2, M, N, Fs};
  EpiAcc epi{out, ldout, accumulate ? 1 : 0};
  Shards sg{};
  for (int t = 0; t < D; ++t) {
    const int j = ((rank - t) % D + D) % D;  // shard held at ring step t
    sg.b[t] = static_cast<const bf16_t*>(w2[j]);
    sg.a_col[t] = (int64_t)j * ldseg;
  }
  sg.count = D;
  op.b = sg.b[0];
  // Tiles in groups of 2 row tiles (16 column tiles of the 7B width run together on an XCD):
  // the hidden activation (361 MB at 7B S=128K) does not fit the 256 MB MALL, so each of its
  // row panels is read from HBM about once per group; the weights, which fit, are re-read
  // from the MALL instead (with the 8-wave kernel, 8-row groups: 3.76 ms of MLP, 2-row
  // groups: 3.68 ms; with the persistent kernel 1-, 2-, 4-, 8- and 16-row groups all time
  // within 2%).
  // With at most half a round of 256 x 256 tiles (7B S=16K: 128 tiles), each tile runs as two
  // work items over the two halves of the ring, one per CU, and a pass adds the halves
  // (230 -> 180 us against the 256 x 128 tile over the whole ring).
  const int64_t t256 = (int64_t)((M + 255) / 256) * ((N + 255) / 256);
  if (part && D % 2 == 0 && persist_ok(op) && 2 * t256 <= device_cus() && N % 4 == 0 && ldout % 4 == 0 &&
      aligned16(out) && aligned16(part)) {
    sg.parts = 2;
    sg.part_c = part;
    sg.part_stride = 0;
    if (hipError_t e = run_persist<false, SEG_K, 2, 3>(op, epi, stream, sg)) return e;
    const int64_t n4 = (int64_t)M * (N / 4);
    const int grid = (int)std::min<int64_t>((n4 + 255) / 256, 4 * (int64_t)device_cus());
    hipLaunchKernelGGL(add_rows_kernel, dim3(grid), dim3(256), 0, stream, out, ldout, part, ldout, M, N / 4);
    return hipGetLastError();
  }
  switch (choose_tile(M, N)) {
    case Tile::k256x256:
      if (persist_ok(op)) return run_persist<false, SEG_K, 2, 3>(op, epi, stream, sg);
      return run_fast<256, 256, 128, 64, false, SEG_K, 2>(op, epi, stream, sg);
    case Tile::k256x128: return run_fast<256, 128, 64, 64, false, SEG_K>(op, epi, stream, sg);
    default: return run_fast<128, 128, 64, 64, false, SEG_K>(op, epi, stream, sg);
  }
}

}  // namespace tsp
