// tsp_attn.hip -- causal attention of one TSP rank's zigzag queries against the
// full-sequence K/V, on gfx950 MFMA.
//
// TSP summary §2 (attention layers): after the K/V all-gather every rank runs
// FlashAttention for its own queries over the whole sequence, and the zigzag partition
// (chunk r with its mirror 2D-1-r) balances the causal work between ranks. This kernel
// is that step for one rank: online softmax in fp32, S x S never materialised.
//
// Work decomposition. One workgroup of 8 waves (two per SIMD) owns 256 consecutive local
// query rows of one (sequence, head); each wave owns one 32-row block of them (a build
// option gives 4 waves of two blocks each). Local rows ascend in position, so a tile's
// last row bounds its keys: the workgroup streams keys [0, pos(last)+1) in stages of 64
// and never reads a key row after the rank's last position (the final stage repeats that
// row instead; those keys are masked). A key-range launch reads only rows of its range:
// its first stage starts at the range's first key rounded down to 64, and the rows before
// that key repeat it (masked). Each XCD takes a contiguous range of (sequence,
// head) work, so the tiles running together on it stream the same K/V through its L2; it
// runs each head's heaviest tile first, or, with at most 4 tiles per CU, the longest tiles
// first across all its heads.
//
// Data movement. K and V stages go straight from global memory into LDS with 16-byte
// global_load_lds (no register staging), into a 4-deep ring of separate LDS buffers, two
// stages ahead of use; one barrier per stage. Rows are stored unpadded and XOR-swizzled
// in 16-byte chunks so the MFMA fragment reads are free of bank conflicts:
//   K: chunk c of row r lives at c ^ fk(r); 16 lanes read 16 rows at one chunk.
//   V: chunk c of row r lives at c ^ fv(r); V^T fragments come from ds_read_b64_tr_b16,
//      whose 16-lane groups each read a 4 key x 16 dim block and hand lane i the four
//      keys of dim i.
// The loads are issued from inline assembly (see dma16_sbase), so the compiler does not
// serialise fragment reads behind them; explicit vmcnt waits and one barrier per stage
// order them. The stage loop is unrolled by the ring depth so every stage offset is an
// immediate.
//
// MFMA formulation (v_mfma_f32_32x32x16_bf16, lane layout in tsp_device.h):
//   S^T = K Q^T     A = K rows (LDS), B = this wave's Q (registers). A lane holds 16 of the
//                   32 keys of a 32-key block for ITS query (column lane%32); the other 16
//                   sit in lane^32, so the row max needs one exchange per block.
//   O^T += V^T P^T  B = P straight from the S^T registers (bf16); A = V^T via transpose
//                   reads with the same key labelling. O^T keeps each lane on its own
//                   query, so the online-softmax rescale is a per-lane scalar.
// With two query blocks per wave, each K and V fragment feeds both.
//
// Pipeline inside a wave, per 32-key block j: the S MFMAs of block j+1 are issued as one
// block at raised wave priority, then the softmax of block j, the rare O rescale and the
// PV MFMAs of block j. With two waves per SIMD, the S MFMAs of one wave run on the matrix
// core while the other wave computes exponentials on the VALU.
// Softmax in base 2: p = exp2(s*c - m), c = scale*log2(e), m a running max of s*c. Q is
// pre-multiplied by c and every S MFMA chain starts from -m, so the MFMAs produce s*c - m
// and no FMA per score is needed. O is rescaled only when the running max grows by more
// than 8 (p <= 2^8 stays exact in fp32 and bf16); the row sum adds the bf16-rounded p with
// v_dot2, so numerator and denominator use the same p.
#include <math.h>

#include <algorithm>

#include "tsp_device.h"
#include "tsp_internal.h"

namespace tsp {
namespace {

// Tile shape. A workgroup owns BR = 256 consecutive local query rows of one (sequence, head)
// and streams keys through LDS in stages of BC = 64 (two 32-key softmax blocks), with a
// 4-stage ring. Two kernels:
//   attn_fwd      (head_dim 64)  8 waves of QB = 1 32-row block, two waves per SIMD, so one
//                                wave's softmax can overlap the other's MFMAs;
//   attn_fwd_w64  (head_dim 128) 4 waves of two 32-row blocks, one wave per SIMD; each K and
//                                V fragment read from LDS feeds both blocks, and the wave
//                                interleaves its own softmax with its MFMAs.
constexpr int BR = 256;
constexpr int BC = 64;
constexpr int QB = 1;
constexpr int RING = 4;
constexpr int NW = BR / (32 * QB);
constexpr int kThreads = 64 * NW;
constexpr int kWavesPerSimd = 2;
constexpr float kLazy = 8.0f;     // rescale O only when the max grows by more than this (log2)

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef const __attribute__((address_space(3))) s16x4 lds_cs16x4;

struct AttnArgs {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  bf16_t* o;     // full attention: bf16 O
  float* o32;    // key-range attention: fp32 O (normalised over the range's keys)
  float* lse;
  int key_lo, key_hi;  // key-range attention: key positions [key_lo, key_hi)
  int accumulate;      // key-range attention: merge into (o32, lse) instead of overwriting
  // Key-range attention, layout of o32 and lse: heads [oh0, oh0 + oH) of a [B, rows, oH, HD]
  // fp32 O and a [B, oH, rows] lse (oH = H, oh0 = 0 for the range entry point).
  int oH, oh0;
  // Split launch (key-range attention with split > 0): two items per tile, keys
  // [0, split) and [split, S); the item of half 1 writes o32 + part_o and lse + part_l.
  int split;
  int64_t part_o, part_l;
  // Fused split launch (split > 0, fused != 0): the key halves of the later chunk's tiles and
  // the earlier chunk's whole tiles in one launch; fused = later-chunk tiles per XCD, or -1
  // where heads do not divide over the XCDs.
  int fused;
  int64_t S;
  int64_t C;
  int rows;  // 2C local rows per sequence
  int D, rank, H;
  int n_qt;   // query tiles per (sequence, head)
  int qt_lo, qt_hi;  // tiles [qt_lo, qt_hi) of each (sequence, head) run (0, n_qt: all)
  int items;  // B * Hrun * (qt_hi - qt_lo), twice that for a split launch
  // Key-range attention: o32 and lse hold local rows [prow0, prow0 + prows) of each sequence.
  int prow0, prows;
  int h0, Hrun;  // heads [h0, h0 + Hrun) of the H in the layout
  int strided;   // 1: item = block index (consecutive items on different XCDs)
  int lpt;       // 1: longest tile first across an XCD's heads (set at launch)
  float scale_log2;
};

template <int HD, int THREADS = kThreads>
struct Lay {
  static constexpr int KS = HD / 16;            // 16-dim reduction steps of Q K^T
  static constexpr int DB = HD / 32;            // 32-dim output blocks
  static constexpr int ROWB = HD * 2;           // bytes per key row
  static constexpr int CPR = ROWB / 16;         // 16-byte chunks per row
  static constexpr int TILEB = BC * ROWB;       // bytes of one K (or V) tile
  static constexpr int NDMA = TILEB / (THREADS * 16);  // 16-byte loads per thread per tile
  static_assert(NDMA >= 1 && NDMA * THREADS * 16 == TILEB, "whole tile per stage");
  // K fragment reads touch 16 consecutive rows at one chunk; V transpose reads touch 4
  // consecutive rows (aligned to 4) x 4 chunks. Both swizzles spread those over all banks.
  __device__ static int fk(int r) { return HD == 128 ? (r & 15) : ((r >> 1) & 7); }
  __device__ static int fv(int r) { return HD == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
};

// The work item of this workgroup: (sequence, head, query tile), and for a split launch the
// key half with its partial outputs.
struct TileSel {
  int b, h, qt;
  int key_lo, key_hi;
  float* o32;    // key-range attention: fp32 O and log-sum-exp (nullptr: not written)
  float* lse32;
  bf16_t* o16;   // bf16 O (nullptr: not written)
};

// Item -> (sequence-head, query tile). A tile's work grows with its index (its last position
// bounds its keys). Each (sequence, head) runs its heaviest tile first. With few tiles per CU
// (lpt), an XCD's items instead go longest first across all its heads: the k-th heaviest tile
// of each head before any head's (k+1)-th, so the CUs that finish a heavy tile take the light
// ones; head-by-head order can give one CU two heavy tiles.
template <bool PART>
__device__ __forceinline__ TileSel select_tile(const AttnArgs& a) {
  TileSel t;
  int item = a.strided ? (int)blockIdx.x : xcd_remap(blockIdx.x, a.items);
  t.key_lo = a.key_lo;
  t.key_hi = a.key_hi;
  t.o32 = a.o32;
  t.lse32 = a.lse;
  t.o16 = a.o;
  if constexpr (PART) {
    if (a.fused != 0) {
      // fused > 0: XCD x receives blocks x, x + 8, ... in order. Its first 2 f blocks are the
      // two key halves of its f later-chunk tiles (whole heads), which start together; the
      // next f are the same heads' earlier-chunk tiles, heaviest first, each taken by the CU
      // that frees first: the one whose half over [split, end) was shortest. A later tile t
      // and the earlier tile n - 1 - t together see 2 D C + BR keys, so with
      // split = D C + BR / 2 a short half and its earlier tile take about as long as a first
      // half. fused < 0 (heads do not divide over the XCDs): the same items, halves first,
      // then the earlier tiles heaviest first, in block order.
      const int n_run = a.qt_hi - a.qt_lo;
      int f, x, k;
      if (a.fused > 0) {
        f = a.fused;
        x = (int)blockIdx.x % kNumXcd;
        k = (int)blockIdx.x / kNumXcd;
      } else {
        f = a.items / 3;
        x = 0;
        k = (int)blockIdx.x;
      }
      const int nbh = f / n_run;  // (sequence, head) pairs per XCD (all of them when fused < 0)
      int bh, qt;
      if (k < 2 * f) {
        const int half = k & 1;
        const int L = x * f + (k >> 1);
        bh = L / n_run;
        qt = a.qt_hi - 1 - (L - bh * n_run);
        t.key_lo = half ? a.split : 0;
        t.key_hi = half ? (int)a.S : a.split;
        t.o32 += half * a.part_o;
        t.lse32 += half * a.part_l;
        t.o16 = nullptr;
      } else {
        const int j = k - 2 * f;
        bh = x * nbh + j % nbh;
        qt = a.qt_lo - 1 - j / nbh;
        t.key_lo = 0;
        t.key_hi = (int)a.S;
        t.o32 = nullptr;
        t.lse32 = nullptr;
      }
      t.b = bh / a.Hrun;
      t.h = a.h0 + bh - t.b * a.Hrun;
      t.qt = qt;
      return t;
    }
    if (a.split > 0) {  // both halves of a tile are consecutive items
      const int half = item & 1;
      item >>= 1;
      t.key_lo = half ? a.split : 0;
      t.key_hi = half ? (int)a.S : a.split;
      t.o32 += half * a.part_o;
      t.lse32 += half * a.part_l;
    }
  }
  int bh, qt;
  const int n_run = a.qt_hi - a.qt_lo;
  if (a.lpt) {
    const int per_xcd = a.items / kNumXcd;
    const int nbh_x = per_xcd / n_run;
    const int x = item / per_xcd;
    const int L = item - x * per_xcd;
    const int k = L / nbh_x;
    bh = x * nbh_x + (L - k * nbh_x);
    qt = a.qt_hi - 1 - k;
  } else {
    bh = item / n_run;
    qt = a.qt_hi - 1 - (item - bh * n_run);
  }
  t.b = bh / a.Hrun;
  t.h = a.h0 + bh - t.b * a.Hrun;
  t.qt = qt;
  return t;
}

// A TileSel with every field read from the first lane (all lanes hold the same values).
__device__ __forceinline__ TileSel uniform_tile(const TileSel& v) {
  auto u = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
  auto up = [&](float* p) {
    const uint64_t x = (uint64_t)(uintptr_t)p;
    return (float*)(uintptr_t)(((uint64_t)(uint32_t)u((int)(uint32_t)(x >> 32)) << 32) | (uint32_t)u((int)(uint32_t)x));
  };
  TileSel t;
  t.b = u(v.b);
  t.h = u(v.h);
  t.qt = u(v.qt);
  t.key_lo = u(v.key_lo);
  t.key_hi = u(v.key_hi);
  t.o32 = up(v.o32);
  t.lse32 = up(v.lse32);
  t.o16 = reinterpret_cast<bf16_t*>(up(reinterpret_cast<float*>(v.o16)));
  return t;
}

// Key-range attention, a tile whose keys all lie outside the range: O = 0 and lse = -inf for
// its rows (accumulate: the range adds nothing; only the bf16 O is written if asked).
template <int HD, int QB>
__device__ __forceinline__ void store_no_keys(const AttnArgs& a, const TileSel& t, const int (&qi)[QB], int hl) {
  if (a.accumulate && t.o16 == nullptr) return;
  const int64_t tok = (int64_t)a.H * HD, otok = (int64_t)a.oH * HD;
  const int oh = t.h - a.oh0;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    if (qi[qb] >= a.rows) continue;
    const int64_t ro = ((int64_t)t.b * a.rows + qi[qb]) * tok + (int64_t)t.h * HD;
    float* op = t.o32 + ((int64_t)t.b * a.prows + (qi[qb] - a.prow0)) * otok + (int64_t)oh * HD;
#pragma unroll
    for (int db = 0; db < HD / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dim = db * 32 + 8 * g + 4 * hl;
        if (a.accumulate) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(op + dim);
          *reinterpret_cast<uint2*>(t.o16 + ro + dim) = pack_bf16x4(v[0], v[1], v[2], v[3]);
        } else {
          *reinterpret_cast<f32x4*>(op + dim) = f32x4{};
          if (t.o16 != nullptr) *reinterpret_cast<uint2*>(t.o16 + ro + dim) = make_uint2(0u, 0u);
        }
      }
    if (!a.accumulate && hl == 0) t.lse32[((int64_t)t.b * a.oH + oh) * a.prows + (qi[qb] - a.prow0)] = -INFINITY;
  }
}

// Normalise and store one wave's rows: QB blocks of 32 rows with O^T accumulators oacc[qb][db]
// (lane l32 + 32 hl: query l32 of block qb, dims 32 db + 8 (r / 4) + 4 hl + r % 4 in register
// r), running max m_s (log2 units) and the row sum in l_in: this half-wave's share, or with
// L_WHOLE the whole row's sum in both half-waves.
//   PART = false: bf16 O, and the log-sum-exp if a.lse is set.
//   PART = true:  fp32 O and log-sum-exp of the range (overwrite), or their log-sum-exp merge
//                 into the accumulator (accumulate); bf16 O too if a.o is set.
template <int HD, int QB, bool PART, bool L_WHOLE = false>
__device__ __forceinline__ void store_rows(const AttnArgs& a, const TileSel& t, const int (&qi)[QB],
                                           const f32x16 (&oacc)[QB][HD / 32], const float (&m_s)[QB],
                                           const float (&l_in)[QB], int hl) {
  constexpr int DB = HD / 32;
  const int64_t tok = (int64_t)a.H * HD;
  float inv[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = L_WHOLE ? l_in[qb] : l_in[qb] + __shfl_xor(l_in[qb], 32);
    inv[qb] = PART ? (l_tot > 0.0f ? 1.0f / l_tot : 0.0f) : 1.0f / l_tot;
    l_run[qb] = l_tot;
  }
  if constexpr (PART) {
    const int64_t otok = (int64_t)a.oH * HD;
    const int oh = t.h - a.oh0;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if (qi[qb] >= a.rows) continue;
      const int64_t ro = ((int64_t)t.b * a.rows + qi[qb]) * tok + (int64_t)t.h * HD;
      const bool w32 = t.o32 != nullptr;
      float* op = w32 ? t.o32 + ((int64_t)t.b * a.prows + (qi[qb] - a.prow0)) * otok + (int64_t)oh * HD : nullptr;
      float* lp = w32 ? t.lse32 + ((int64_t)t.b * a.oH + oh) * a.prows + (qi[qb] - a.prow0) : nullptr;
      const float lse_b = l_run[qb] > 0.0f ? (m_s[qb] + __log2f(l_run[qb])) * 0.69314718055994531f : -INFINITY;
      // Overwrite: weights (0, 1). Accumulate: the log-sum-exp merge with what the
      // accumulator holds (both lanes of the row read it before lane hl == 0 writes).
      float wa = 0.0f, wb = 1.0f, lse_new = lse_b;
      if (a.accumulate) {
        const float lse_a = *lp;
        const float mm = fmaxf(lse_a, lse_b);
        wb = 0.0f;
        if (mm != -INFINITY) {
          wa = __expf(lse_a - mm);
          wb = __expf(lse_b - mm);
          const float z = wa + wb;
          lse_new = mm + __logf(z);
          wa /= z;
          wb /= z;
        }
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int dim = db * 32 + 8 * g + 4 * hl;
          const f32x16& o = oacc[qb][db];
          const float s = wb * inv[qb];
          f32x4 val = {o[4 * g] * s, o[4 * g + 1] * s, o[4 * g + 2] * s, o[4 * g + 3] * s};
          if (a.accumulate) val += wa * *reinterpret_cast<const f32x4*>(op + dim);
          if (w32) *reinterpret_cast<f32x4*>(op + dim) = val;
          if (t.o16 != nullptr)
            *reinterpret_cast<uint2*>(t.o16 + ro + dim) = pack_bf16x4(val[0], val[1], val[2], val[3]);
        }
      }
      if (w32 && hl == 0) *lp = lse_new;
    }
    return;
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    if (qi[qb] >= a.rows) continue;
    bf16_t* op = a.o + ((int64_t)t.b * a.rows + qi[qb]) * tok + (int64_t)t.h * HD;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dim = db * 32 + 8 * g + 4 * hl;
        const f32x16& o = oacc[qb][db];
        *reinterpret_cast<uint2*>(op + dim) =
            pack_bf16x4(o[4 * g] * inv[qb], o[4 * g + 1] * inv[qb], o[4 * g + 2] * inv[qb], o[4 * g + 3] * inv[qb]);
      }
    }
    if (a.lse != nullptr && hl == 0)
      a.lse[((int64_t)t.b * a.H + t.h) * a.rows + qi[qb]] = (m_s[qb] + __log2f(l_run[qb])) * 0.69314718055994531f;
  }
}

// PART = false: every key up to the query's position, bf16 O. PART = true: only keys in
// [key_lo, key_hi) (a chunk of the sequence as the all-gather delivers it), fp32 O and the
// log-sum-exp for the merge; rows that see no key get O = 0 and lse = -inf.
template <int HD, bool PART>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWavesPerSimd, kWavesPerSimd))) void attn_fwd(AttnArgs a) {
  using L = Lay<HD>;
  constexpr int KS = L::KS, DB = L::DB, ROWB = L::ROWB, CPR = L::CPR, TILEB = L::TILEB, NDMA = L::NDMA;
  // K and V rings: stage st of K at kring + st * TILEB, of V at vring + st * TILEB. With
  // 4 stages each ring spans 64 KB, so every fragment address is a per-lane base plus an
  // immediate offset.
  __shared__ __attribute__((aligned(1024))) char kring[RING * TILEB];
  __shared__ __attribute__((aligned(1024))) char vring[RING * TILEB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hl = lane >> 5;

  const TileSel t = select_tile<PART>(a);
  const int b = t.b, h = t.h, key_lo = t.key_lo, key_hi = t.key_hi;
  const int row0 = t.qt * BR;
  int kv_end = (int)zigzag_pos(min(row0 + BR, a.rows) - 1, a.C, a.rank, a.D) + 1;
  int k_base = 0;  // position of the first key of stage 0
  if constexpr (PART) {
    kv_end = min(kv_end, key_hi);
    k_base = (key_lo / BC) * BC;
  }
  const int n_kt = (kv_end - k_base + BC - 1) / BC;

  const int wrow0 = row0 + wave * (32 * QB);
  const int wmin_pos = wrow0 < a.rows ? (int)zigzag_pos(wrow0, a.C, a.rank, a.D) : 0;
  const int64_t tok = (int64_t)a.H * HD;  // elements between consecutive tokens

  // This lane's query rows and their Q fragments (dims 16s + 8hl .. +7).
  int qi[QB], qpos[QB];
  bf16x8 qf[QB][KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    qi[qb] = wrow0 + 32 * qb + l32;
    const bool valid = qi[qb] < a.rows;
    const int qic = valid ? qi[qb] : a.rows - 1;
    qpos[qb] = (int)zigzag_pos(qic, a.C, a.rank, a.D);
    const bf16_t* qp = a.q + ((int64_t)b * a.rows + qic) * tok + (int64_t)h * HD + 8 * hl;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[qb][s] = valid ? as_bf16x8(*reinterpret_cast<const uint4*>(qp + 16 * s)) : bf16x8{};
  }
  // Q * scale * log2(e), rounded to bf16 (round to nearest even): S comes out in log2 units.
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[qb][s][e] = (__bf16)((float)qf[qb][s][e] * a.scale_log2);

  // A tile whose keys all lie outside the range: O = 0, lse = -inf, no LDS work (the whole
  // workgroup returns here, before any barrier).
  if constexpr (PART) {
    if (kv_end <= key_lo) {
      store_no_keys<HD, QB>(a, t, qi, hl);
      return;
    }
  }

  // ---- stage loads: global -> LDS, 16 bytes per lane, lane-linear within the 1 KB a wave
  // instruction writes. Load p of this wave covers linear chunks (NW p + wave) * 64 + lane.
  const char* kseq = reinterpret_cast<const char*>(a.k + (int64_t)b * a.S * tok + (int64_t)h * HD);
  const char* vseq = reinterpret_cast<const char*>(a.v + (int64_t)b * a.S * tok + (int64_t)h * HD);
  int drow[NDMA], dck[NDMA], dcv[NDMA];
#pragma unroll
  for (int p = 0; p < NDMA; ++p) {
    const int lin = (NW * p + wave) * 64 + lane;
    drow[p] = lin / CPR;
    const int pc = lin % CPR;
    dck[p] = 16 * (pc ^ L::fk(drow[p]));
    dcv[p] = 16 * (pc ^ L::fv(drow[p]));
  }
  const uint32_t tokb = (uint32_t)(tok * 2);
  auto issue = [&] __device__(int st, int t) {
    const int key0 = k_base + t * BC;
    const int lim = kv_end - 1 - key0;  // rows past the tile's last key repeat it (masked)
    // In a key range, rows of the first stage before key_lo repeat row key_lo (masked), so
    // no row outside [key_lo, kv_end) is addressed: K/V rows of chunks that have not arrived
    // may hold anything, and a masked P of 0 times a NaN V row would still poison O.
    const int low = PART ? key_lo - key0 : 0;  // <= 0 past the first stage
    const char* kb = kseq + (int64_t)key0 * tok * 2;
    const char* vb = vseq + (int64_t)key0 * tok * 2;
    const uint32_t lk = lds_addr(kring) + st * TILEB + wave * 1024;
    const uint32_t lv = lds_addr(vring) + st * TILEB + wave * 1024;
#pragma unroll
    for (int p = 0; p < NDMA; ++p) {
      const uint32_t roff = (uint32_t)(PART ? max(min(drow[p], lim), low) : min(drow[p], lim)) * tokb;
      dma16_sbase(kb, roff + dck[p], lk + NW * p * 1024);
      dma16_sbase(vb, roff + dcv[p], lv + NW * p * 1024);
    }
  };
  // Wait until at most `stages` later stages of this wave's loads are in flight, then a
  // bare barrier: every wave's earlier stage loads have landed in LDS.
  auto sync_stage = [&] __device__(int stages) {
    if (stages >= 2) {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(4 * NDMA));
    } else if (stages == 1) {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * NDMA));
    } else {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    }
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");  // no LDS read moves above the barrier
  };

  // ---- fragment addresses (bytes within a stage; block, half and part add constants)
  int kaddr[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) kaddr[s] = l32 * ROWB + 16 * ((2 * s + hl) ^ L::fk(l32));
  const int G = lane >> 4, j16 = lane & 15;
  // V^T fragment bases as LDS-typed pointers, so stage / block / part offsets fold into
  // the transpose reads' immediate offset field (units of 8 bytes).
  const lds_s16x4* vbase[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int r = 4 * hl + (j16 >> 2);  // row within an aligned group of 8 keys
    const int c = 4 * db + 2 * (G & 1) + ((j16 & 3) >> 1);
    vbase[db] = (const lds_s16x4*)(vring + r * ROWB + 16 * (c ^ L::fv(r)) + 8 * (j16 & 1));
  }

  f32x16 oacc[QB][DB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[qb][db] = f32x16{};
  float m_s[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_s[qb] = -INFINITY;
    l_run[qb] = 0.0f;
  }
  // Every S MFMA chain starts from -m_cm (m_cm = the reference max when the chain is
  // issued; 0 before the first block). m_at_*: m_cm of the two S buffers.
  float m_cm[QB], m_at_cur[QB], m_at_nxt[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) m_cm[qb] = m_at_cur[qb] = m_at_nxt[qb] = 0.0f;
  auto note = [&] __device__(float (&m_at)[QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) m_at[qb] = m_cm[qb];
  };
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  // K fragments of 32-key block kb (0/1) of a stage: 16 keys per lane group, dims of step s.
  auto load_k = [&] __device__(int st, int kb, bf16x8 (&kf)[KS]) {
#pragma unroll
    for (int s = 0; s < KS; ++s)
      kf[s] = as_bf16x8(*reinterpret_cast<const uint4*>(kring + st * TILEB + kaddr[s] + kb * 32 * ROWB));
  };
  // S^T of one 32-key block from its K fragments, both query blocks.
  auto qk = [&] __device__(const bf16x8 (&kf)[KS], f32x16 (&sacc)[QB]) {
    // The S MFMAs issue as one block of their own (no VALU interleaved) at raised wave
    // priority: with two waves per SIMD, one wave's MFMA block then runs while the other
    // wave does its softmax.
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[qb][r] = -m_cm[qb];
      sacc[qb] = mfma32x32x16(kf[0], qf[qb][0], sacc[qb]);
    }
#pragma unroll
    for (int s = 1; s < KS; ++s)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sacc[qb] = mfma32x32x16(kf[s], qf[qb][s], sacc[qb]);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto mask = [&] __device__(f32x16 (&sacc)[QB], int kstart) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kstart + 8 * (r >> 2) + 4 * hl + (r & 3) > qpos[qb] ||
            (PART && (kstart + 8 * (r >> 2) + 4 * hl + (r & 3) < key_lo ||
                      kstart + 8 * (r >> 2) + 4 * hl + (r & 3) >= key_hi)))
          sacc[qb][r] = -INFINITY;
  };
  // sacc = s*c - m_at (m_at: the reference max the block was computed against). Row max;
  // in the rare case that the max grew by more than kLazy or the block was computed
  // against an older reference, shift it to the current reference (and move the reference
  // and the chain start value); then exponentials, bf16 P and their sum. Returns whether
  // this lane needs the O rescale (then by the factors in alpha).
  auto softmax = [&] __device__(f32x16 (&sacc)[QB], const float (&m_at)[QB], bf16x8 (&pf)[QB][2],
                                float (&alpha)[QB]) {
    bool any = false, need = false;
    float mx[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float v = sacc[qb][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) v = fmaxf(v, sacc[qb][r]);
      mx[qb] = max_swap32(v);
      const float d = m_s[qb] - m_at[qb];  // 0 unless the reference moved since the MFMAs
      need |= (mx[qb] - d > kLazy) | (d != 0.0f);
      alpha[qb] = 1.0f;
    }
    if (__ballot(need)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float d = m_s[qb] - m_at[qb];
        const bool upd = mx[qb] - d > kLazy;
        const float m_new = upd ? m_at[qb] + mx[qb] : m_s[qb];
        alpha[qb] = upd ? __builtin_amdgcn_exp2f(m_s[qb] - m_new) : 1.0f;  // 0 on the first block
        // a row with no visible key so far keeps its scores (-inf) and reference
        const float shift = m_new == -INFINITY ? 0.0f : m_new - m_at[qb];
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[qb][r] -= shift;
        l_run[qb] *= alpha[qb];
        m_s[qb] = m_new;
        if (upd) m_cm[qb] = m_new;
        any |= upd;
      }
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float lsum = 0.0f;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(sacc[qb][8 * half + 2 * e]);
          const float p1 = __builtin_amdgcn_exp2f(sacc[qb][8 * half + 2 * e + 1]);
          w[e] = pack_bf16x2(p0, p1);
          lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[e]), ones, lsum, false);
        }
        pf[qb][half] = as_bf16x8(make_uint4(w[0], w[1], w[2], w[3]));
      }
      l_run[qb] += lsum;
    }
    return any;
  };
  // Pins P and the row sums in registers at the end of the softmax, so the exponentials
  // cannot sink below the rescale branch into the PV region.
  auto close_region = [&] __device__(const bf16x8 (&pf)[QB][2]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int half = 0; half < 2; ++half) asm volatile("" ::"v"(__builtin_bit_cast(u32x4, pf[qb][half])));
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) asm volatile("" ::"v"(l_run[qb]));
  };
  auto rescale = [&] __device__(const float (&alpha)[QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[qb][db] *= alpha[qb];
  };
  // V^T fragments of 32-key block kb of a stage (two 16-key halves x DB dim blocks), from
  // transpose reads.
  auto load_v = [&] __device__(int st, int kb, bf16x8 (&vf)[2][DB]) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const lds_s16x4* vr = vbase[db] + (st * TILEB + (32 * kb + 16 * half) * ROWB) / 8;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)vr);
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vr + ROWB));
        const uint2 ulo = __builtin_bit_cast(uint2, lo), uhi = __builtin_bit_cast(uint2, hi);
        vf[half][db] = as_bf16x8(make_uint4(ulo.x, ulo.y, uhi.x, uhi.y));
      }
    }
  };
  // O^T += V^T P^T for one 32-key block.
  auto pv = [&] __device__(const bf16x8 (&vf)[2][DB], const bf16x8 (&pf)[QB][2]) {
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) oacc[qb][db] = mfma32x32x16(vf[half][db], pf[qb][half], oacc[qb][db]);
  };

  // Prologue: stages 0..2 in flight, wait for stage 0, first S block.
  issue(0, 0);
  if (n_kt > 1) issue(1, 1);
  if (n_kt > 2) issue(2, 2);
  sync_stage(n_kt > 2 ? 2 : n_kt - 1);

  f32x16 s_cur[QB], s_nxt[QB];
  bf16x8 pf[QB][2];
  bf16x8 kf[KS];     // K fragments of the next S block, read one softmax ahead
  bf16x8 vf[2][DB];  // V^T fragments of the next PV block, read one softmax ahead
  float alpha[QB];
  load_k(0, 0, kf);
  qk(kf, s_cur);
  note(m_at_cur);
  load_k(0, 1, kf);

  // Stage t: `cur` holds it, `nxt` holds stage t+1 (its first block's S is computed here),
  // `refill` is the buffer of stage t-1, reloaded with stage t+3. Every LDS read is issued
  // one softmax before its MFMAs: the K of block 1 of stage t comes from the previous stage.
  auto body = [&] __device__(int t, int cur, int nxt, int refill) {
    sync_stage(t + 2 < n_kt ? 1 : 0);  // stage t+1 landed; stage t+2 may be in flight
    if (t + 3 < n_kt) issue(refill, t + 3);
    const int k0 = k_base + t * BC;
    // causal mask where a key may follow a row; in a key range also at its two ends
    if (k0 + 31 > wmin_pos || (PART && (k0 < key_lo || k0 + 32 > key_hi))) mask(s_cur, k0);
    qk(kf, s_nxt);  // block 1 of stage t
    note(m_at_nxt);
    load_v(cur, 0, vf);
    load_k(nxt, 0, kf);  // after the last stage this reads a stale buffer; the result is unused
    bool any = softmax(s_cur, m_at_cur, pf, alpha);
    close_region(pf);
    if (__ballot(any)) rescale(alpha);
    pv(vf, pf);
    if (k0 + 63 > wmin_pos || (PART && (k0 + 32 < key_lo || k0 + 64 > key_hi))) mask(s_nxt, k0 + 32);
    qk(kf, s_cur);  // block 0 of stage t+1
    note(m_at_cur);
    load_v(cur, 1, vf);
    load_k(nxt, 1, kf);
    any = softmax(s_nxt, m_at_nxt, pf, alpha);
    close_region(pf);
    if (__ballot(any)) rescale(alpha);
    pv(vf, pf);
  };
  // Unrolled by the ring depth so every stage buffer is named statically; guarded bodies
  // (no early exits) keep the accumulators in one register set.
  for (int t = 0; t < n_kt; t += 4) {
    body(t, 0, 1, 3);
    if (t + 1 < n_kt) body(t + 1, 1, 2, 0);
    if (t + 2 < n_kt) body(t + 2, 2, 3, 1);
    if (t + 3 < n_kt) body(t + 3, 3, 0, 2);
  }

  store_rows<HD, QB, PART>(a, t, qi, oacc, m_s, l_run, hl);
}

// ------------------------------------------------------------------- head_dim 128 kernel
// attn_fwd_w64: one wave per SIMD, 64 query rows per wave (two 32-row blocks that share every
// K and V^T fragment read from LDS: half the LDS bytes per MFMA of a 32-row wave).
// Registers: the O^T accumulators (2 x 4 x 16) sit in a0..a127 and the pre-scaled Q fragments
// (2 x 8 x 4) in a128..a191, fixed AGPRs named only inside inline assembly (the MFMAs, the
// zeroing, the rare rescale and the final read-out), so no compiler-placed copy ever moves
// them; every such statement lists a0..a191 as clobbered, which keeps the compiler's own values
// out of them. S of two key blocks, P of two key blocks and the K / V^T fragments stay in
// VGPRs.
// Per 32-key block j one pass issues 32 MFMAs, alternating the 16 of S_{j+1} = K Q^T with the
// 16 of O^T += V^T P_{j-1}^T, and puts the softmax of S_j (row max, exponentials, bf16 P_j)
// and the LDS reads of the next K and V^T fragments in fixed slots between them, so the
// matrix core and the VALU work side by side within the one wave. The row sums of P_{j-1}
// come from four small MFMAs beside its PV (mma_rowsum), not from the VALU. P_{j-1} meets
// V_{j-1} one pass late: the rescale of O^T and the row sums for block j (when its max moved)
// follows the pass's last PV MFMA, which is exactly when both hold blocks < j.
// The compiler's hazard checks do not see into inline assembly, so the waits are explicit:
// 2 wait states between a VALU write and an MFMA reading it (the S chains' start values, AGPR
// writes before an MFMA), 12 between an MFMA and a VALU read of its result (S before the
// softmax; O before a rescale or the read-out). A VALU or LDS write into an MFMA's A or B
// operand right after the MFMA needs none.
namespace w64 {
constexpr int HD = 128, QB = 2, NW = 4, THREADS = 64 * NW;
using L = Lay<HD, THREADS>;
constexpr int kOReg = 0;    // O^T[qb][db] in a[kOReg + 16 (4 qb + db) .. +15]
constexpr int kQReg = 128;  // Q[qb][ks] in a[kQReg + 4 (8 qb + ks) .. +3]
constexpr int kLReg = 192;  // row sums of query block qb in a[kLReg + 4 qb] (a[.. + 1 .. 3] stay 0)
}  // namespace w64

#define TSP_STR(x) #x
#define TSP_A10(p) TSP_STR(a##p##0), TSP_STR(a##p##1), TSP_STR(a##p##2), TSP_STR(a##p##3), TSP_STR(a##p##4), \
    TSP_STR(a##p##5), TSP_STR(a##p##6), TSP_STR(a##p##7), TSP_STR(a##p##8), TSP_STR(a##p##9)
// a0 .. a199
#define TSP_AGPRS "a0", "a1", "a2", "a3", "a4", "a5", "a6", "a7", "a8", "a9", TSP_A10(1), TSP_A10(2), TSP_A10(3), \
    TSP_A10(4), TSP_A10(5), TSP_A10(6), TSP_A10(7), TSP_A10(8), TSP_A10(9), TSP_A10(10), TSP_A10(11), TSP_A10(12), \
    TSP_A10(13), TSP_A10(14), TSP_A10(15), TSP_A10(16), TSP_A10(17), TSP_A10(18), TSP_A10(19)

// s += K-fragment x Q-fragment (Q in a[QR .. QR+3]); the first step of a chain also waits for
// the VALU write of its start value.
template <int QR>
__device__ __forceinline__ void mma_s(f32x16& s, const bf16x8& k) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, a[%2:%3], %0" : "+v"(s) : "v"(k), "n"(QR), "n"(QR + 3) : TSP_AGPRS);
}
template <int QR>
__device__ __forceinline__ void mma_s_first(f32x16& s, const bf16x8& k, const f32x16& start) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, a[%2:%3], %4" : "=&v"(s) : "v"(k), "n"(QR), "n"(QR + 3), "v"(start)
               : TSP_AGPRS);
}
// O^T in a[OR .. OR+15] += V^T-fragment x P-fragment.
template <int OR>
__device__ __forceinline__ void mma_pv(const bf16x8& v, const bf16x8& p) {
  asm volatile("v_mfma_f32_32x32x16_bf16 a[%2:%3], %0, %1, a[%2:%3]" ::"v"(v), "v"(p), "n"(OR), "n"(OR + 15)
               : TSP_AGPRS);
}
// Row sums on the matrix core: a[LR .. LR+3] += Sel x P-fragment with a 16x16x32 MFMA. P's
// B-operand layout for the 32x32x16 MFMA puts query l % 32, keys of group l / 32, in lane l;
// read as the B operand of the 16x16x32 MFMA, column n gathers lanes n, n+16, n+32, n+48, that
// is query n (k groups 0 and 2) and query n+16 (k groups 1 and 3). Sel (lane_sel) holds ones
// in rows 0 and 8 over k groups 0, 2 and in rows 4 and 12 over k groups 1, 3, zeros elsewhere;
// so output row 4 g of column n, which lane 16 g + n holds in its first register, is the sum
// of that lane's own query's 16 P values, and the other three registers stay zero. The
// products are exact (P times 1 or 0), so this adds the same bf16 values that enter O^T.
template <int LR>
__device__ __forceinline__ void mma_rowsum(const bf16x8& sel, const bf16x8& p) {
  asm volatile("v_mfma_f32_16x16x32_bf16 a[%2:%3], %0, %1, a[%2:%3]" ::"v"(sel), "v"(p), "n"(LR), "n"(LR + 3)
               : TSP_AGPRS);
}
__device__ __forceinline__ bf16x8 lane_sel(int lane) {
  const int g = lane >> 4, r = lane & 15;
  const bool on = (g & 1) ? (r == 4 || r == 12) : (r == 0 || r == 8);
  const uint32_t w = on ? 0x3f803f80u : 0u;
  return as_bf16x8(make_uint4(w, w, w, w));
}
// Both query blocks' row sums a[LR], a[LR + 4] times their alpha; for use after the O^T
// rescale (which provides the wait after the MFMAs), 2 wait states before an MFMA reads them.
template <int LR>
__device__ __forceinline__ void rescale_rowsums(float alpha0, float alpha1) {
  float t0, t1;
  asm volatile(
      "v_accvgpr_read_b32 %0, a[%4]\n\t"
      "v_accvgpr_read_b32 %1, a[%5]\n\t"
      "v_mul_f32 %0, %0, %2\n\t"
      "v_mul_f32 %1, %1, %3\n\t"
      "v_accvgpr_write_b32 a[%4], %0\n\t"
      "v_accvgpr_write_b32 a[%5], %1\n\t"
      "s_nop 1"
      : "=&v"(t0), "=&v"(t1)
      : "v"(alpha0), "v"(alpha1), "n"(LR), "n"(LR + 4)
      : TSP_AGPRS);
}
template <int R>
__device__ __forceinline__ float read_agpr(void) {
  float x;
  asm volatile("v_accvgpr_read_b32 %0, a[%1]" : "=v"(x) : "n"(R) : TSP_AGPRS);
  return x;
}
// Q fragment into a[QR .. QR+3].
template <int QR>
__device__ __forceinline__ void q_to_agpr(const bf16x8& q) {
  const uint4 u = __builtin_bit_cast(uint4, q);
  asm volatile(
      "v_accvgpr_write_b32 a[%4], %0\n\tv_accvgpr_write_b32 a[%5], %1\n\t"
      "v_accvgpr_write_b32 a[%6], %2\n\tv_accvgpr_write_b32 a[%7], %3" ::"v"(u.x),
      "v"(u.y), "v"(u.z), "v"(u.w), "n"(QR), "n"(QR + 1), "n"(QR + 2), "n"(QR + 3)
      : TSP_AGPRS);
}
// a[R .. R+63] *= alpha (one query block's O^T), after the MFMAs that wrote them (16 wait
// states), 2 wait states before an MFMA reads them again.
template <int R>
__device__ __forceinline__ void rescale_agprs(float alpha) {
  float t;
  asm volatile(
      "s_nop 7\n\ts_nop 7\n\t"
      ".set tsp_rr, %2\n\t"
      ".rept 64\n\t"
      "v_accvgpr_read_b32 %0, a[tsp_rr]\n\t"
      "v_mul_f32 %0, %0, %1\n\t"
      "v_accvgpr_write_b32 a[tsp_rr], %0\n\t"
      ".set tsp_rr, tsp_rr + 1\n\t"
      ".endr\n\t"
      "s_nop 1"
      : "=&v"(t)
      : "v"(alpha), "n"(R)
      : TSP_AGPRS);
}
// One O^T accumulator a[R .. R+15] read out (after the 16 wait states the caller provides).
template <int R>
__device__ __forceinline__ f32x16 read_agprs16(void) {
  float x0, x1, x2, x3, x4, x5, x6, x7, x8, x9, x10, x11, x12, x13, x14, x15;
  asm volatile(
      "v_accvgpr_read_b32 %0, a[%16]\n\tv_accvgpr_read_b32 %1, a[%17]\n\tv_accvgpr_read_b32 %2, a[%18]\n\t"
      "v_accvgpr_read_b32 %3, a[%19]\n\tv_accvgpr_read_b32 %4, a[%20]\n\tv_accvgpr_read_b32 %5, a[%21]\n\t"
      "v_accvgpr_read_b32 %6, a[%22]\n\tv_accvgpr_read_b32 %7, a[%23]\n\tv_accvgpr_read_b32 %8, a[%24]\n\t"
      "v_accvgpr_read_b32 %9, a[%25]\n\tv_accvgpr_read_b32 %10, a[%26]\n\tv_accvgpr_read_b32 %11, a[%27]\n\t"
      "v_accvgpr_read_b32 %12, a[%28]\n\tv_accvgpr_read_b32 %13, a[%29]\n\tv_accvgpr_read_b32 %14, a[%30]\n\t"
      "v_accvgpr_read_b32 %15, a[%31]"
      : "=v"(x0), "=v"(x1), "=v"(x2), "=v"(x3), "=v"(x4), "=v"(x5), "=v"(x6), "=v"(x7), "=v"(x8), "=v"(x9),
        "=v"(x10), "=v"(x11), "=v"(x12), "=v"(x13), "=v"(x14), "=v"(x15)
      : "n"(R), "n"(R + 1), "n"(R + 2), "n"(R + 3), "n"(R + 4), "n"(R + 5), "n"(R + 6), "n"(R + 7), "n"(R + 8),
        "n"(R + 9), "n"(R + 10), "n"(R + 11), "n"(R + 12), "n"(R + 13), "n"(R + 14), "n"(R + 15)
      : TSP_AGPRS);
  return f32x16{x0, x1, x2, x3, x4, x5, x6, x7, x8, x9, x10, x11, x12, x13, x14, x15};
}
#define TSP_SB() __builtin_amdgcn_sched_barrier(0)

template <bool PART>
__global__ __launch_bounds__(w64::THREADS) __attribute__((amdgpu_waves_per_eu(1, 1))) void attn_fwd_w64(AttnArgs a) {
  constexpr int HD = w64::HD, QB = w64::QB, NW = w64::NW, OR = w64::kOReg, QR = w64::kQReg, LR = w64::kLReg;
  using L = w64::L;
  constexpr int KS = L::KS, DB = L::DB, ROWB = L::ROWB, CPR = L::CPR, TILEB = L::TILEB, NDMA = L::NDMA;
  __shared__ __attribute__((aligned(1024))) char kring[RING * TILEB];
  __shared__ __attribute__((aligned(1024))) char vring[RING * TILEB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hl = lane >> 5;

  // The tile's indices come out of integer divisions, which the compiler leaves in VGPRs;
  // they are the same in every lane, so they are moved to SGPRs: the per-stage addresses,
  // loop bounds and mask tests then run on the scalar unit.
  const TileSel t = uniform_tile(select_tile<PART>(a));
  const int b = t.b, h = t.h, key_lo = t.key_lo, key_hi = t.key_hi;
  const int row0 = t.qt * BR;
  int kv_end = __builtin_amdgcn_readfirstlane((int)zigzag_pos(min(row0 + BR, a.rows) - 1, a.C, a.rank, a.D) + 1);
  int k_base = 0;  // position of the first key of stage 0
  if constexpr (PART) {
    kv_end = min(kv_end, key_hi);
    k_base = (key_lo / BC) * BC;
  }
  const int n_kt = (kv_end - k_base + BC - 1) / BC;

  const int wrow0 = row0 + wave * (32 * QB);
  const int wmin_pos =
      __builtin_amdgcn_readfirstlane(wrow0 < a.rows ? (int)zigzag_pos(wrow0, a.C, a.rank, a.D) : 0);
  const int64_t tok = (int64_t)a.H * HD;

  // This lane's query rows; their Q fragments (dims 16s + 8hl .. +7), times scale*log2(e) and
  // rounded to bf16 so that S comes out in log2 units, go to a[QR ..].
  int qi[QB], qpos[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    qi[qb] = wrow0 + 32 * qb + l32;
    qpos[qb] = (int)zigzag_pos(qi[qb] < a.rows ? qi[qb] : a.rows - 1, a.C, a.rank, a.D);
  }
  if constexpr (PART) {
    if (kv_end <= key_lo) {  // the whole workgroup returns here, before any barrier
      store_no_keys<HD, QB>(a, t, qi, hl);
      return;
    }
  }
  {
    bf16x8 qf[QB][KS];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const bool valid = qi[qb] < a.rows;
      const bf16_t* qp = a.q + ((int64_t)b * a.rows + (valid ? qi[qb] : a.rows - 1)) * tok + (int64_t)h * HD + 8 * hl;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        qf[qb][s] = valid ? as_bf16x8(*reinterpret_cast<const uint4*>(qp + 16 * s)) : bf16x8{};
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[qb][s][e] = (__bf16)((float)qf[qb][s][e] * a.scale_log2);
      }
    }
#define TSP_QW(qb, s) q_to_agpr<QR + 4 * (8 * (qb) + (s))>(qf[qb][s]);
    TSP_QW(0, 0) TSP_QW(0, 1) TSP_QW(0, 2) TSP_QW(0, 3) TSP_QW(0, 4) TSP_QW(0, 5) TSP_QW(0, 6) TSP_QW(0, 7)
    TSP_QW(1, 0) TSP_QW(1, 1) TSP_QW(1, 2) TSP_QW(1, 3) TSP_QW(1, 4) TSP_QW(1, 5) TSP_QW(1, 6) TSP_QW(1, 7)
#undef TSP_QW
  }
  // O^T = 0, row sums = 0
  asm volatile(
      ".set tsp_rr, %0\n\t"
      ".rept 128\n\t"
      "v_accvgpr_write_b32 a[tsp_rr], 0\n\t"
      ".set tsp_rr, tsp_rr + 1\n\t"
      ".endr\n\t"
      ".set tsp_rr, %1\n\t"
      ".rept 8\n\t"
      "v_accvgpr_write_b32 a[tsp_rr], 0\n\t"
      ".set tsp_rr, tsp_rr + 1\n\t"
      ".endr" ::"n"(OR), "n"(LR)
      : TSP_AGPRS);
  const bf16x8 lsel = lane_sel(lane);

  // ---- stage loads (as in attn_fwd): global -> LDS, 16 bytes per lane; load p of this wave
  // covers linear chunks (NW p + wave) * 64 + lane of a tile.
  const char* kseq = reinterpret_cast<const char*>(a.k + (int64_t)b * a.S * tok + (int64_t)h * HD);
  const char* vseq = reinterpret_cast<const char*>(a.v + (int64_t)b * a.S * tok + (int64_t)h * HD);
  // Load p of a lane covers tile row drow, 16-byte column chunk pc (stored swizzled); in a
  // tile whose rows are all keys of the range its source offsets are fixed (voffk, voffv).
  const uint32_t tokb = (uint32_t)(tok * 2);
  auto dma_slot = [&] __device__(int p, int& drow, int& dck, int& dcv) {
    const int lin = (NW * p + wave) * 64 + lane;
    drow = lin / CPR;
    const int pc = lin % CPR;
    dck = 16 * (pc ^ L::fk(drow));
    dcv = 16 * (pc ^ L::fv(drow));
  };
  uint32_t voffk[NDMA], voffv[NDMA];
#pragma unroll
  for (int p = 0; p < NDMA; ++p) {
    int drow, dck, dcv;
    dma_slot(p, drow, dck, dcv);
    voffk[p] = (uint32_t)drow * tokb + dck;
    voffv[p] = (uint32_t)drow * tokb + dcv;
  }
  auto issue = [&] __device__(int st, int tt) {
    const int key0 = k_base + tt * BC;
    const int lim = kv_end - 1 - key0;         // rows past the tile's last key repeat it (masked)
    const int low = PART ? key_lo - key0 : 0;  // a key range's rows before key_lo repeat key_lo
    const char* kb = kseq + (int64_t)key0 * tok * 2;
    const char* vb = vseq + (int64_t)key0 * tok * 2;
    const uint32_t lk = lds_addr(kring) + st * TILEB + wave * 1024;
    const uint32_t lv = lds_addr(vring) + st * TILEB + wave * 1024;
    if (lim >= BC - 1 && low <= 0) {
#pragma unroll
      for (int p = 0; p < NDMA; ++p) {
        dma16_sbase(kb, voffk[p], lk + NW * p * 1024);
        dma16_sbase(vb, voffv[p], lv + NW * p * 1024);
      }
    } else {  // the last tile, or the first of a key range: clamp the rows
#pragma unroll
      for (int p = 0; p < NDMA; ++p) {
        int drow, dck, dcv;
        dma_slot(p, drow, dck, dcv);
        const uint32_t roff = (uint32_t)(PART ? max(min(drow, lim), low) : min(drow, lim)) * tokb;
        dma16_sbase(kb, roff + dck, lk + NW * p * 1024);
        dma16_sbase(vb, roff + dcv, lv + NW * p * 1024);
      }
    }
  };
  // Stage u's buffer is read by the K fragment reads of body u-1 and the V^T fragment reads
  // of body u, which the first pass of body u+1 consumes; so the barrier at the start of body
  // u+2 is the first point where every wave is done with it, and body t refills the buffer of
  // stage t-2 with stage t+2 (4-stage ring, loads one body ahead). At that barrier the only
  // loads in flight are stage t+1's.
  auto sync_all = [&] __device__(int in_flight_stages) {
    if (in_flight_stages >= 1) {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * NDMA));
    } else {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    }
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");  // no LDS read moves above the barrier
  };

  // ---- fragment addresses (as in attn_fwd)
  int kaddr[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) kaddr[s] = l32 * ROWB + 16 * ((2 * s + hl) ^ L::fk(l32));
  const int G = lane >> 4, j16 = lane & 15;
  const lds_s16x4* vbase[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int r = 4 * hl + (j16 >> 2);
    const int c = 4 * db + 2 * (G & 1) + ((j16 & 3) >> 1);
    vbase[db] = (const lds_s16x4*)(vring + r * ROWB + 16 * (c ^ L::fv(r)) + 8 * (j16 & 1));
  }
  auto load_k1 = [&] __device__(int st, int kb, int s) {
    return as_bf16x8(*reinterpret_cast<const uint4*>(kring + st * TILEB + kaddr[s] + kb * 32 * ROWB));
  };
  auto load_v1 = [&] __device__(int st, int kb, int half, int db) {
    const lds_s16x4* vr = vbase[db] + (st * TILEB + (32 * kb + 16 * half) * ROWB) / 8;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)vr);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vr + ROWB));
    const uint2 ulo = __builtin_bit_cast(uint2, lo), uhi = __builtin_bit_cast(uint2, hi);
    return as_bf16x8(make_uint4(ulo.x, ulo.y, uhi.x, uhi.y));
  };

  // Online softmax state in log2 units: m_s the running max (the row sums, relative to it,
  // live in a[LR ..]), m_cm the value every newly started S chain subtracts (its start value
  // is -m_cm), m_at the m_cm a buffer's chain started from.
  float m_s[QB], m_cm[QB], m_at_a[QB], m_at_b[QB];
  // Wave-wide flags: some row has seen no key yet (its m_s is -inf while its chains start from
  // 0), and the block about to be processed was started before the last reference move. When
  // both are clear, every row's chain started from its current reference, so the scores of a
  // block are already relative to m_s and the lazy test is just "a score above kLazy".
  bool unseen = true, stale = false;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_s[qb] = -INFINITY;
    m_cm[qb] = m_at_a[qb] = m_at_b[qb] = 0.0f;
  }
  // Start value of every S chain: -m_cm in all 16 registers (the first MFMA of a chain reads it
  // as its accumulator input; rewritten only when m_cm moves).
  f32x16 start_t[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) start_t[qb] = f32x16{};
  auto mask = [&] __device__(f32x16 (&sacc)[QB], int kstart) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kstart + 8 * (r >> 2) + 4 * hl + (r & 3);
        if (key > qpos[qb] || (PART && (key < key_lo || key >= key_hi))) sacc[qb][r] = -INFINITY;
      }
  };

  // MFMA slot i (0..31): even i is S of the next block, step ks = i / 4, query block
  // (i / 2) % 2; odd i is PV of the previous block, half i / 16, dims block (i / 4) % 4, query
  // block (i / 2) % 2. K (V^T) fragments are read again once both query blocks used them.
#define TSP_MMA_S(i)                                                              \
  if ((i) / 4 == 0) {                                                            \
    mma_s_first<QR + 4 * (8 * (((i) / 2) % 2) + (i) / 4)>(sn[((i) / 2) % 2], kf[(i) / 4], start_t[((i) / 2) % 2]); \
  } else {                                                                       \
    mma_s<QR + 4 * (8 * (((i) / 2) % 2) + (i) / 4)>(sn[((i) / 2) % 2], kf[(i) / 4]);       \
  }                                                                              \
  TSP_SB();
#define TSP_MMA_PV(i)                                                                        \
  mma_pv<OR + 16 * (4 * (((i) / 2) % 2) + ((i) / 4) % 4)>(vf[(i) / 16][((i) / 4) % 4],       \
                                                         pp[((i) / 2) % 2][(i) / 16]);         \
  TSP_SB();
// Row sums of the previous block, with its PV: query block qb, key half hh.
#define TSP_MMA_L(qb, hh)                       \
  mma_rowsum<LR + 4 * (qb)>(lsel, pp[qb][hh]); \
  TSP_SB();
#define TSP_LOAD_K(i) kf[(i) / 4] = load_k1(kst, kkb, (i) / 4);
#define TSP_LOAD_V(i) vf[(i) / 16][((i) / 4) % 4] = load_v1(vst, vkb, (i) / 16, ((i) / 4) % 4);

  // ---- prologue: stages 0 and 1 in flight; S of block 0 once stage 0 has landed; K
  // fragments of block 1.
  issue(0, 0);
  if (n_kt > 1) issue(1, 1);
  sync_all(n_kt > 1 ? 1 : 0);
  f32x16 sa[QB], sb[QB];        // S chains of alternate blocks
  bf16x8 pa[QB][2], pb[QB][2];  // P of alternate blocks (two 16-key halves each)
  bf16x8 kf[KS];                // K fragments of the block whose S the next pass computes
  bf16x8 vf[2][DB];             // V^T fragments of the block whose PV the next pass computes
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    sa[qb] = f32x16{};
    sb[qb] = f32x16{};
    pb[qb][0] = pb[qb][1] = bf16x8{};  // the first pass's PV adds 0 (no block before block 0)
  }
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int db = 0; db < DB; ++db) vf[hh][db] = bf16x8{};
#pragma unroll
  for (int s = 0; s < KS; ++s) kf[s] = load_k1(0, 0, s);
  {
    f32x16 (&sn)[QB] = sa;
    TSP_MMA_S(0) TSP_MMA_S(2) TSP_MMA_S(4) TSP_MMA_S(6) TSP_MMA_S(8) TSP_MMA_S(10) TSP_MMA_S(12) TSP_MMA_S(14)
    TSP_MMA_S(16) TSP_MMA_S(18) TSP_MMA_S(20) TSP_MMA_S(22) TSP_MMA_S(24) TSP_MMA_S(26) TSP_MMA_S(28) TSP_MMA_S(30)
  }
#pragma unroll
  for (int s = 0; s < KS; ++s) kf[s] = load_k1(0, 1, s);

  // ---- one pass: softmax of block j (S in sc, chain started from -m_at), S of block j+1
  // into sn from kf, PV of block j-1 from vf and pp; kf <- K of block j+2 (stage kst, block
  // kkb), vf <- V^T of block j (stage vst, block vkb); P of block j -> pc; then sc restarts
  // as the chain of block j+2 from -m_cm.
  auto pass = [&] __device__(int k0, f32x16 (&sc)[QB], f32x16 (&sn)[QB], float (&m_at)[QB],
                             const bf16x8 (&pp)[QB][2], bf16x8 (&pc)[QB][2], int kst, int kkb, int vst,
                             int vkb) __attribute__((always_inline)) {
    TSP_SB();
    asm volatile("s_nop 11");  // the MFMAs that wrote sc: 12 wait states before a VALU read
    TSP_SB();
    // causal mask where a key may follow a row; in a key range also at its two ends
    if (k0 + 31 > wmin_pos || (PART && (k0 < key_lo || k0 + 32 > key_hi))) mask(sc, k0);
    TSP_SB();
    float tm[QB][5], mx[QB], alpha[QB];
    bool need = false, any = false;
    uint32_t w[QB][2][4];
    // slots 0-5: this half-wave's max of each row (16 of its 32 keys), three-way maxima
    TSP_MMA_S(0)
    tm[0][0] = fmaxf(fmaxf(sc[0][0], sc[0][1]), sc[0][2]);
    tm[0][1] = fmaxf(fmaxf(sc[0][3], sc[0][4]), sc[0][5]);
    tm[0][2] = fmaxf(fmaxf(sc[0][6], sc[0][7]), sc[0][8]);
    TSP_SB();
    TSP_MMA_PV(1)
    tm[0][3] = fmaxf(fmaxf(sc[0][9], sc[0][10]), sc[0][11]);
    tm[0][4] = fmaxf(fmaxf(sc[0][12], sc[0][13]), sc[0][14]);
    tm[1][0] = fmaxf(fmaxf(sc[1][0], sc[1][1]), sc[1][2]);
    TSP_SB();
    TSP_MMA_S(2)
    TSP_LOAD_K(2)
    tm[1][1] = fmaxf(fmaxf(sc[1][3], sc[1][4]), sc[1][5]);
    tm[1][2] = fmaxf(fmaxf(sc[1][6], sc[1][7]), sc[1][8]);
    tm[1][3] = fmaxf(fmaxf(sc[1][9], sc[1][10]), sc[1][11]);
    TSP_SB();
    TSP_MMA_PV(3)
    TSP_LOAD_V(3)
    tm[1][4] = fmaxf(fmaxf(sc[1][12], sc[1][13]), sc[1][14]);
    tm[0][0] = fmaxf(fmaxf(tm[0][0], tm[0][1]), tm[0][2]);
    tm[0][3] = fmaxf(fmaxf(tm[0][3], tm[0][4]), sc[0][15]);
    asm volatile("" ::"v"(tm[1][4]), "v"(tm[0][0]), "v"(tm[0][3]));
    TSP_SB();
    TSP_MMA_S(4)
    tm[1][0] = fmaxf(fmaxf(tm[1][0], tm[1][1]), tm[1][2]);
    tm[1][3] = fmaxf(fmaxf(tm[1][3], tm[1][4]), sc[1][15]);
    mx[0] = fmaxf(tm[0][0], tm[0][3]);
    asm volatile("" ::"v"(tm[1][0]), "v"(tm[1][3]), "v"(mx[0]));
    TSP_SB();
    TSP_MMA_PV(5)
    mx[1] = fmaxf(tm[1][0], tm[1][3]);
    asm volatile("" ::"v"(mx[1]));
    TSP_SB();
    // slot 6: does some row's reference move? With unseen and stale clear, only when one of
    // its scores exceeds kLazy (the half-wave maxima suffice: the row max exceeds kLazy iff
    // one half does); otherwise the branch takes the exact per-row test.
    TSP_MMA_S(6)
    TSP_LOAD_K(6)
    need = (mx[0] > kLazy) | (mx[1] > kLazy);
    alpha[0] = alpha[1] = 1.0f;
    TSP_SB();
    TSP_MMA_PV(7)
    TSP_LOAD_V(7)
    TSP_MMA_L(0, 0)
    if (__ballot(need) | unseen | stale) {  // rare: shift the scores to the new reference
      mx[0] = max_swap32(mx[0]);  // the row max over both half-waves
      mx[1] = max_swap32(mx[1]);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float d = m_s[qb] - m_at[qb];
        const bool upd = mx[qb] - d > kLazy;
        const float m_new = upd ? m_at[qb] + mx[qb] : m_s[qb];
        alpha[qb] = upd ? __builtin_amdgcn_exp2f(m_s[qb] - m_new) : 1.0f;  // 0 on the first block
        // a row with no visible key so far keeps its scores (-inf) and reference
        const float shift = m_new == -INFINITY ? 0.0f : m_new - m_at[qb];
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[qb][r] -= shift;
        m_s[qb] = m_new;
        if (upd) m_cm[qb] = m_new;
#pragma unroll
        for (int r = 0; r < 16; ++r) start_t[qb][r] = -m_cm[qb];
        any |= upd;
      }
      unseen = __ballot((m_s[0] == -INFINITY) | (m_s[1] == -INFINITY)) != 0;
    }
    TSP_SB();
    // slots 8-31: exponentials and bf16 P, two operations per slot (spread evenly: the MFMA
    // pipe stays fed only while each gap between MFMAs holds a few instructions). Operation n
    // (0..47) is exp, exp, convert of key pair n / 3, which is query block pr % 2, half
    // (pr / 2) / 4, register pair (pr / 2) % 4.
    float pv_[16][2];
#define TSP_OP(n)                                                                                    \
  {                                                                                                  \
    constexpr int pr_ = (n) / 3, op_ = (n) % 3, qb_ = pr_ % 2, hh_ = (pr_ / 2) / 4, e_ = (pr_ / 2) % 4; \
    if (op_ < 2) {                                                                                   \
      pv_[pr_][op_ % 2] = __builtin_amdgcn_exp2f(sc[qb_][8 * hh_ + 2 * e_ + op_ % 2]);               \
      asm volatile("" ::"v"(pv_[pr_][op_ % 2])); /* computed in this slot */                         \
    } else {                                                                                         \
      w[qb_][hh_][e_] = pack_bf16x2(pv_[pr_][0], pv_[pr_][1]);                                        \
      asm volatile("" ::"v"(w[qb_][hh_][e_]));                                                       \
    }                                                                                                \
  }
#define TSP_EXP(i) TSP_OP(2 * ((i) - 8)) TSP_OP(2 * ((i) - 8) + 1) TSP_SB();
    TSP_MMA_S(8)   TSP_EXP(8)
    TSP_MMA_PV(9)  TSP_EXP(9)
    TSP_MMA_S(10)  TSP_LOAD_K(10) TSP_EXP(10)
    TSP_MMA_PV(11) TSP_LOAD_V(11) TSP_EXP(11)
    TSP_MMA_S(12)  TSP_EXP(12)
    TSP_MMA_PV(13) TSP_EXP(13)
    TSP_MMA_S(14)  TSP_LOAD_K(14) TSP_EXP(14)
    TSP_MMA_PV(15) TSP_LOAD_V(15) TSP_MMA_L(1, 0) TSP_EXP(15)
    TSP_MMA_S(16)  TSP_EXP(16)
    TSP_MMA_PV(17) TSP_EXP(17)
    TSP_MMA_S(18)  TSP_LOAD_K(18) TSP_EXP(18)
    TSP_MMA_PV(19) TSP_LOAD_V(19) TSP_EXP(19)
    TSP_MMA_S(20)  TSP_EXP(20)
    TSP_MMA_PV(21) TSP_EXP(21)
    TSP_MMA_S(22)  TSP_LOAD_K(22) TSP_EXP(22)
    TSP_MMA_PV(23) TSP_LOAD_V(23) TSP_MMA_L(0, 1) TSP_EXP(23)
    TSP_MMA_S(24)  TSP_EXP(24)
    TSP_MMA_PV(25) TSP_EXP(25)
    TSP_MMA_S(26)  TSP_LOAD_K(26) TSP_EXP(26)
    TSP_MMA_PV(27) TSP_LOAD_V(27) TSP_EXP(27)
    TSP_MMA_S(28)  TSP_EXP(28)
    TSP_MMA_PV(29) TSP_EXP(29)
    TSP_MMA_S(30)  TSP_LOAD_K(30) TSP_EXP(30)
    TSP_MMA_PV(31) TSP_LOAD_V(31) TSP_MMA_L(1, 1) TSP_EXP(31)
#undef TSP_EXP
#undef TSP_OP
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) pc[qb][hh] = as_bf16x8(make_uint4(w[qb][hh][0], w[qb][hh][1], w[qb][hh][2], w[qb][hh][3]));
    }

#pragma unroll
    for (int qb = 0; qb < QB; ++qb) m_at[qb] = m_cm[qb];
    // O^T now holds the blocks before j: rescale it for block j's reference (rare)
    stale = __ballot(any) != 0;  // block j+1 was started from the old reference
    if (stale) {
      rescale_agprs<OR>(alpha[0]);
      rescale_agprs<OR + 64>(alpha[1]);
      rescale_rowsums<LR>(alpha[0], alpha[1]);
    }
    TSP_SB();
  };

  // ---- main loop: stage t holds blocks 2t and 2t+1; unrolled by the ring depth so every
  // stage buffer is named statically.
  auto body = [&] __device__(int tt, int cur, int nxt, int refill) __attribute__((always_inline)) {
    sync_all(0);  // stage tt+1 landed; every wave is done with the buffer of stage tt-2
    if (tt + 2 < n_kt) issue(refill, tt + 2);
    const int k0 = k_base + tt * BC;
    // block 2tt: S of 2tt+1 (kf: stage tt block 1), kf <- stage tt+1 block 0, vf <- stage tt block 0
    pass(k0, sa, sb, m_at_a, pb, pa, nxt, 0, cur, 0);
    // block 2tt+1: S of 2tt+2 (kf: stage tt+1 block 0, stale after the last stage: unused)
    pass(k0 + 32, sb, sa, m_at_b, pa, pb, nxt, 1, cur, 1);
  };
  for (int tt = 0; tt < n_kt; tt += 4) {
    body(tt, 0, 1, 2);
    if (tt + 1 < n_kt) body(tt + 1, 1, 2, 3);
    if (tt + 2 < n_kt) body(tt + 2, 2, 3, 0);
    if (tt + 3 < n_kt) body(tt + 3, 3, 0, 1);
  }
  // PV of the last block (its P in pb, its V^T fragments in vf)
  {
    const bf16x8 (&pp)[QB][2] = pb;
    TSP_MMA_PV(1) TSP_MMA_PV(3) TSP_MMA_PV(5) TSP_MMA_PV(7) TSP_MMA_PV(9) TSP_MMA_PV(11) TSP_MMA_PV(13)
    TSP_MMA_PV(15) TSP_MMA_PV(17) TSP_MMA_PV(19) TSP_MMA_PV(21) TSP_MMA_PV(23) TSP_MMA_PV(25) TSP_MMA_PV(27)
    TSP_MMA_PV(29) TSP_MMA_PV(31)
    TSP_MMA_L(0, 0) TSP_MMA_L(1, 0) TSP_MMA_L(0, 1) TSP_MMA_L(1, 1)
  }
#undef TSP_MMA_S
#undef TSP_MMA_PV
#undef TSP_MMA_L
#undef TSP_LOAD_K
#undef TSP_LOAD_V
  asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");  // 16 wait states before O^T is read out
  TSP_SB();
  f32x16 oacc[QB][DB];
  oacc[0][0] = read_agprs16<OR + 0>();
  oacc[0][1] = read_agprs16<OR + 16>();
  oacc[0][2] = read_agprs16<OR + 32>();
  oacc[0][3] = read_agprs16<OR + 48>();
  oacc[1][0] = read_agprs16<OR + 64>();
  oacc[1][1] = read_agprs16<OR + 80>();
  oacc[1][2] = read_agprs16<OR + 96>();
  oacc[1][3] = read_agprs16<OR + 112>();
  const float l_row[QB] = {read_agpr<LR>(), read_agpr<LR + 4>()};
  store_rows<HD, QB, PART, true>(a, t, qi, oacc, m_s, l_row, hl);
}
#undef TSP_SB

}  // namespace

namespace {

// Fields every launch sets the same way; the mode fields start as "full attention, all
// heads, no key range".
AttnArgs base_args(const void* q, const void* k_full, const void* v_full, int B, int64_t S, int D, int rank, int H,
                   int hd, float scale) {
  AttnArgs a;
  a.q = static_cast<const bf16_t*>(q);
  a.k = static_cast<const bf16_t*>(k_full);
  a.v = static_cast<const bf16_t*>(v_full);
  a.o = nullptr;
  a.o32 = nullptr;
  a.lse = nullptr;
  a.S = S;
  a.C = S / (2 * D);
  a.rows = (int)(2 * a.C);
  a.D = D;
  a.rank = rank;
  a.H = H;
  a.n_qt = (a.rows + BR - 1) / BR;
  a.qt_lo = 0;
  a.qt_hi = a.n_qt;
  a.prow0 = 0;
  a.prows = a.rows;
  a.h0 = 0;
  a.Hrun = H;
  a.strided = 0;
  a.lpt = 0;
  a.items = B * H * a.n_qt;
  a.key_lo = 0;
  a.key_hi = (int)S;
  a.accumulate = 0;
  a.oH = H;
  a.oh0 = 0;
  a.split = 0;
  a.part_o = 0;
  a.part_l = 0;
  a.fused = 0;
  const float sc = scale > 0.0f ? scale : 1.0f / sqrtf((float)hd);
  a.scale_log2 = sc * 1.4426950408889634f;
  return a;
}

// Heads [h0, h0 + h_run) only.
bool set_heads(AttnArgs& a, int B, int h0, int h_run) {
  if (h0 < 0 || h_run <= 0 || h0 + h_run > a.H) return false;
  a.h0 = h0;
  a.Hrun = h_run;
  a.items = B * h_run * (a.qt_hi - a.qt_lo);
  return true;
}

// Longest-first order across an XCD's heads pays when there are few tiles per CU (at 7B
// S=32K, two per CU: rank-to-rank spread of attention time 1.21x -> 1.01x). With many,
// head-by-head order already balances and keeps each head's K/V in the XCD's L2 (7B B=4
// S=64K, 16 per CU: 10% faster than longest first). Requires whole (sequence, head) ranges
// per XCD and one item per tile.
constexpr int kLptMaxItems = 4 * 256;

template <bool PART>
hipError_t launch(const AttnArgs& a_in, int hd, hipStream_t stream) {
  AttnArgs a = a_in;
  a.lpt = !a.strided && a.split == 0 && a.items <= kLptMaxItems && a.items % (kNumXcd * (a.qt_hi - a.qt_lo)) == 0;
  if (hd == 128) {
    hipLaunchKernelGGL((attn_fwd_w64<PART>), dim3(a.items), dim3(w64::THREADS), 0, stream, a);
  } else {
    hipLaunchKernelGGL((attn_fwd<64, PART>), dim3(a.items), dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn(const void* q, const void* k_full, const void* v_full, void* o, float* lse, int B, int64_t S,
                       int D, int rank, int H, int hd, float scale, hipStream_t stream) {
  AttnArgs a = base_args(q, k_full, v_full, B, S, D, rank, H, hd, scale);
  a.o = static_cast<bf16_t*>(o);
  a.lse = lse;
  return launch<false>(a, hd, stream);
}

hipError_t launch_attn_range(const void* q, const void* k_full, const void* v_full, float* o32, float* lse, int B,
                             int64_t S, int D, int rank, int H, int hd, float scale, int64_t key_lo, int64_t key_hi,
                             int accumulate, void* o_out, hipStream_t stream) {
  AttnArgs a = base_args(q, k_full, v_full, B, S, D, rank, H, hd, scale);
  a.o = static_cast<bf16_t*>(o_out);
  a.accumulate = accumulate;
  a.o32 = o32;
  a.lse = lse;
  a.key_lo = (int)key_lo;
  a.key_hi = (int)key_hi;
  if (accumulate && o_out == nullptr) {
    // Merging into the accumulator only: tiles whose rows all precede key_lo add nothing and
    // write nothing. Positions ascend with the local row, so those are the first tiles.
    int qt = 0;
    while (qt < a.n_qt && zigzag_pos(min((qt + 1) * BR, a.rows) - 1, a.C, a.rank, a.D) < key_lo) ++qt;
    if (qt == a.n_qt || key_lo >= key_hi) return hipSuccess;
    a.qt_lo = qt;
    a.items = B * H * (a.n_qt - qt);
  }
  return launch<true>(a, hd, stream);
}

hipError_t launch_attn_heads(const void* q, const void* k_full, const void* v_full, void* o, int B, int64_t S, int D,
                             int rank, int H, int hd, float scale, int h0, int h_run, hipStream_t stream) {
  AttnArgs a = base_args(q, k_full, v_full, B, S, D, rank, H, hd, scale);
  if (!set_heads(a, B, h0, h_run)) return hipErrorInvalidValue;
  a.o = static_cast<bf16_t*>(o);
  return launch<false>(a, hd, stream);
}

hipError_t launch_attn_split(const void* q, const void* k_full, const void* v_full, float* o32, float* lse, int B,
                             int64_t S, int D, int rank, int H, int hd, float scale, int h0, int h_run, int split,
                             hipStream_t stream) {
  AttnArgs a = base_args(q, k_full, v_full, B, S, D, rank, H, hd, scale);
  if (!set_heads(a, B, h0, h_run) || split <= 0 || split >= S) return hipErrorInvalidValue;
  a.o32 = o32;
  a.lse = lse;
  a.oH = a.Hrun;
  a.oh0 = a.h0;
  a.split = split;
  a.part_o = (int64_t)B * a.rows * a.Hrun * hd;
  a.part_l = (int64_t)B * a.Hrun * a.rows;
  a.items *= 2;
  // Strided (consecutive items on different XCDs), heaviest tiles first: every XCD gets an
  // even share of the heavy halves. (Measured faster than XCD-contiguous runs of a head's
  // tiles with heavy and light tiles alternating.)
  a.strided = 1;
  return launch<true>(a, hd, stream);
}

// Log-sum-exp merge of a partial attention into a running one, one wave per (sequence,
// row, head): lanes own hd / 64 consecutive dims; every lane reads the two lse values
// before lane 0 writes the merged one (one wave, in program order).
template <int HD>
__global__ __launch_bounds__(256) void attn_merge(float* o_acc, float* lse_acc, const float* o_part,
                                                  const float* lse_part, bf16_t* o_out, int64_t units, int rows, int H) {
  constexpr int PER = HD / 64;
  const int64_t u = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // (b * rows + row) * H + h
  if (u >= units) return;
  const int lane = threadIdx.x & 63;
  const int h = (int)(u % H);
  const int64_t br = u / H;
  const int row = (int)(br % rows);
  const int64_t b = br / rows;
  const int64_t li = (b * H + h) * rows + row;
  const float la = lse_acc[li], lb = lse_part[li];
  const float m = fmaxf(la, lb);
  float wa = 0.0f, wb = 0.0f, lnew = -INFINITY;
  if (m != -INFINITY) {
    wa = __expf(la - m);
    wb = __expf(lb - m);
    const float z = wa + wb;
    lnew = m + __logf(z);
    wa /= z;
    wb /= z;
  }
  float* pa = o_acc + u * HD + lane * PER;
  const float* pb = o_part + u * HD + lane * PER;
  float r[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) r[e] = wa * pa[e] + wb * pb[e];
#pragma unroll
  for (int e = 0; e < PER; ++e) pa[e] = r[e];
  if (o_out != nullptr) {
    bf16_t* po = o_out + u * HD + lane * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) po[e] = to_bf16(r[e]);
  }
  if (lane == 0) lse_acc[li] = lnew;
}

// The two halves of a split launch merged into bf16 O: one wave per (sequence, row, head
// of the group); partials in the group's [B, rows, h_run, HD] / [B, h_run, rows] layout,
// O in the [B, rows, H, HD] layout at heads h0 .. h0 + h_run - 1.
template <int HD>
__global__ __launch_bounds__(256) void attn_merge_halves(const float* o32, const float* lse, int64_t part_o,
                                                         int64_t part_l, bf16_t* o_out, int64_t units, int rows,
                                                         int h_run, int H, int h0, int out_rows, int out_row0) {
  constexpr int PER = HD / 64;
  const int64_t u = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // (b * rows + row) * h_run + h
  if (u >= units) return;
  const int lane = threadIdx.x & 63;
  const int h = (int)(u % h_run);
  const int64_t br = u / h_run;
  const int row = (int)(br % rows);
  const int64_t b = br / rows;
  const int64_t li = (b * h_run + h) * rows + row;
  const float la = lse[li], lb = lse[part_l + li];
  const float m = fmaxf(la, lb);  // finite: half 0 holds key 0, which every row sees
  const float ea = __expf(la - m), eb = __expf(lb - m);
  const float wa = ea / (ea + eb), wb = eb / (ea + eb);
  const float* pa = o32 + u * HD + lane * PER;
  const float* pb = o32 + part_o + u * HD + lane * PER;
  // row `row` of the partials is local row out_row0 + row of O ([B, out_rows, H, HD])
  bf16_t* po = o_out + ((b * out_rows + out_row0 + row) * H + h0 + h) * HD + lane * PER;
#pragma unroll
  for (int e = 0; e < PER; ++e) po[e] = to_bf16(wa * pa[e] + wb * pb[e]);
}

namespace {
hipError_t merge_halves_rows(const float* o32, const float* lse, void* o_out, int B, int rows, int H, int hd, int h0,
                             int h_run, int out_rows, int out_row0, hipStream_t stream) {
  if (h0 < 0 || h_run <= 0 || h0 + h_run > H || out_row0 < 0 || out_row0 + rows > out_rows)
    return hipErrorInvalidValue;
  const int64_t units = (int64_t)B * rows * h_run;
  const int64_t part_o = units * hd, part_l = units;
  const dim3 grid((unsigned)((units + 3) / 4));
  if (hd == 128) {
    hipLaunchKernelGGL(attn_merge_halves<128>, grid, dim3(256), 0, stream, o32, lse, part_o, part_l,
                       static_cast<bf16_t*>(o_out), units, rows, h_run, H, h0, out_rows, out_row0);
  } else {
    hipLaunchKernelGGL(attn_merge_halves<64>, grid, dim3(256), 0, stream, o32, lse, part_o, part_l,
                       static_cast<bf16_t*>(o_out), units, rows, h_run, H, h0, out_rows, out_row0);
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_attn_merge_halves(const float* o32, const float* lse, void* o_out, int B, int rows, int H, int hd,
                                    int h0, int h_run, hipStream_t stream) {
  return merge_halves_rows(o32, lse, o_out, B, rows, H, hd, h0, h_run, rows, 0, stream);
}

// Two-part attention for launches of at most one round of tiles (one per CU): the time of a
// plain launch is then that of the heaviest tile, a later zigzag chunk's tile that sees up to
// (2D - r) C keys. Instead, one launch runs each later-chunk tile as two items, keys
// [0, split) and [split, end), into fp32 partials of the later chunk's rows, and each
// earlier-chunk tile whole (bf16 O); the earlier tiles wait for the CUs whose second half
// ends first (the item order is in select_tile). A later tile t and the earlier tile
// n - 1 - t see 2 D C + BR keys together whatever the rank, so with split = D C + BR / 2 every
// CU sees about D C + BR / 2 keys. A log-sum-exp pass merges the halves into bf16 O. Every
// later-chunk row lies at or after split (split is clamped to the later chunk's start), so
// both halves see keys. Applies when chunks hold whole tiles and the tiles fill at most one
// round.
constexpr int kCus = 256;

int attn_two_part_split(int B, int64_t S, int D, int rank, int H) {
  const int64_t C = S / (2 * D);
  if (C <= 0 || C % BR != 0) return 0;
  const int64_t nt = C / BR;               // tiles per chunk and (sequence, head)
  const int64_t nl = (int64_t)B * H * nt;  // tiles per chunk over every (sequence, head)
  if (2 * nl > kCus) return 0;
  const int64_t split = std::min((int64_t)D * C + BR / 2, (2 * (int64_t)D - 1 - rank) * C) / BC * BC;
  if (split <= 0) return 0;
  return (int)split;
}

size_t attn_two_part_bytes(int B, int64_t S, int D, int H, int hd) {
  const size_t C = (size_t)(S / (2 * D));
  return 2 * (size_t)B * C * (size_t)H * ((size_t)hd + 1) * sizeof(float);
}

hipError_t launch_attn_two_part(const void* q, const void* k_full, const void* v_full, void* o, void* part, int B,
                                int64_t S, int D, int rank, int H, int hd, float scale, hipStream_t stream) {
  const int split = attn_two_part_split(B, S, D, rank, H);
  if (split <= 0) return hipErrorInvalidValue;
  AttnArgs l = base_args(q, k_full, v_full, B, S, D, rank, H, hd, scale);
  const int c_tiles = (int)(l.C / BR);
  const int64_t units = (int64_t)B * l.C * H;
  float* o32 = static_cast<float*>(part);
  l.o = static_cast<bf16_t*>(o);  // the earlier chunk's tiles
  l.o32 = o32;                    // the later chunk's halves: rows [C, 2C)
  l.lse = o32 + 2 * units * hd;
  l.qt_lo = c_tiles;
  l.prow0 = (int)l.C;
  l.prows = (int)l.C;
  l.split = split;
  l.part_o = units * hd;
  l.part_l = units;
  const int nl = B * H * c_tiles;
  l.fused = nl % kNumXcd == 0 && (nl / kNumXcd) % c_tiles == 0 ? nl / kNumXcd : -1;
  l.items = 3 * nl;
  l.strided = 1;
  if (hipError_t err = launch<true>(l, hd, stream)) return err;
  return merge_halves_rows(o32, l.lse, o, B, (int)l.C, H, hd, 0, H, l.rows, (int)l.C, stream);
}

hipError_t launch_attn_merge(float* o_acc, float* lse_acc, const float* o_part, const float* lse_part, void* o_out,
                             int B, int rows, int H, int hd, hipStream_t stream) {
  const int64_t units = (int64_t)B * rows * H;
  const dim3 grid((unsigned)((units + 3) / 4));
  if (hd == 128) {
    hipLaunchKernelGGL(attn_merge<128>, grid, dim3(256), 0, stream, o_acc, lse_acc, o_part, lse_part,
                       static_cast<bf16_t*>(o_out), units, rows, H);
  } else {
    hipLaunchKernelGGL(attn_merge<64>, grid, dim3(256), 0, stream, o_acc, lse_acc, o_part, lse_part,
                       static_cast<bf16_t*>(o_out), units, rows, H);
  }
  return hipGetLastError();
}

}  // namespace tsp
