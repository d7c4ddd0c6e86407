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

#include "tsp_device.h"
#include "tsp_internal.h"

namespace tsp {
namespace {

// Tile shape. Each wave owns QB 32-row query blocks; a workgroup owns BR rows (NW = BR /
// (32 QB) waves) and streams keys through LDS in stages of BC = 64 (two 32-key softmax
// blocks), with a 4-stage ring.
//   BR 256, QB 1: 8 waves sharing one ring; two waves per SIMD, so one wave's softmax can
//                 overlap the other's MFMAs (the default, fastest measured at 7B S=128K).
//   BR 256, QB 2: one wave per SIMD; each K/V fragment feeds two query blocks.
#ifndef TSP_ATTN_BR
#define TSP_ATTN_BR 256
#endif
#ifndef TSP_ATTN_QB
#define TSP_ATTN_QB 1
#endif
// CINIT 1: Q is pre-multiplied by scale*log2(e) (rounded to bf16) and every S MFMA chain
// starts from -m, so the MFMAs produce s*c - m directly and the softmax needs no FMA per
// score. CINIT 0: S = K Q^T, then one FMA per score.
#ifndef TSP_ATTN_CINIT
#define TSP_ATTN_CINIT 1
#endif
constexpr int BR = TSP_ATTN_BR;
constexpr int BC = 64;
constexpr int QB = TSP_ATTN_QB;
constexpr int RING = 4;
constexpr int NW = BR / (32 * QB);
constexpr int kThreads = 64 * NW;
constexpr int kWavesPerSimd = (QB == 1) ? 2 : 1;
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

template <int HD>
struct Lay {
  static constexpr int KS = HD / 16;            // 16-dim reduction steps of Q K^T
  static constexpr int DB = HD / 32;            // 32-dim output blocks
  static constexpr int ROWB = HD * 2;           // bytes per key row
  static constexpr int CPR = ROWB / 16;         // 16-byte chunks per row
  static constexpr int TILEB = BC * ROWB;       // bytes of one K (or V) tile
  static constexpr int NDMA = TILEB / (kThreads * 16);  // 16-byte loads per thread per tile
  static_assert(NDMA >= 1 && NDMA * kThreads * 16 == TILEB, "whole tile per stage");
  // K fragment reads touch 16 consecutive rows at one chunk; V transpose reads touch 4
  // consecutive rows (aligned to 4) x 4 chunks. Both swizzles spread those over all banks.
  __device__ static int fk(int r) { return HD == 128 ? (r & 15) : ((r >> 1) & 7); }
  __device__ static int fv(int r) { return HD == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
};

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

  int item = a.strided ? (int)blockIdx.x : xcd_remap(blockIdx.x, a.items);
  int key_lo = a.key_lo, key_hi = a.key_hi;
  float* o32 = a.o32;
  float* lse32 = a.lse;
  if constexpr (PART) {
    if (a.split > 0) {  // both halves of a tile are consecutive items
      const int half = item & 1;
      item >>= 1;
      key_lo = half ? a.split : 0;
      key_hi = half ? (int)a.S : a.split;
      o32 += half * a.part_o;
      lse32 += half * a.part_l;
    }
  }
  // Item -> (sequence-head, query tile). A tile's work grows with its index (its last
  // position bounds its keys). Each (sequence, head) runs its heaviest tile first. With few
  // tiles per CU (lpt), an XCD's items instead go longest first across all its heads: the
  // k-th heaviest tile of each head before any head's (k+1)-th, so the CUs that finish a
  // heavy tile take the light ones; head-by-head order can give one CU two heavy tiles.
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
  const int b = bh / a.Hrun, h = a.h0 + bh - (bh / a.Hrun) * a.Hrun;
  const int row0 = qt * BR;
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
  const int64_t otok = (int64_t)a.oH * HD;  // the same in o32
  const int oh = h - a.oh0;

  // This lane's two query rows and their Q fragments (dims 16s + 8hl .. +7).
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
#if TSP_ATTN_CINIT
  // Q * scale * log2(e), rounded to bf16 (round to nearest even): S comes out in log2 units.
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[qb][s][e] = (__bf16)((float)qf[qb][s][e] * a.scale_log2);
#endif

  // A tile whose keys all lie outside the range: O = 0, lse = -inf, no LDS work (the whole
  // workgroup returns here, before any barrier).
  if constexpr (PART) {
    if (kv_end <= key_lo) {
      // accumulate: the range adds nothing to these rows; only the bf16 O is written if asked
      if (a.accumulate && a.o == nullptr) return;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if (qi[qb] >= a.rows) continue;
        const int64_t ro = ((int64_t)b * a.rows + qi[qb]) * tok + (int64_t)h * HD;
        float* op = o32 + ((int64_t)b * a.prows + (qi[qb] - a.prow0)) * otok + (int64_t)oh * HD;
#pragma unroll
        for (int db = 0; db < HD / 32; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int dim = db * 32 + 8 * g + 4 * hl;
            if (a.accumulate) {
              const f32x4 v = *reinterpret_cast<const f32x4*>(op + dim);
              *reinterpret_cast<uint2*>(a.o + ro + dim) = pack_bf16x4(v[0], v[1], v[2], v[3]);
            } else {
              *reinterpret_cast<f32x4*>(op + dim) = f32x4{};
              if (a.o != nullptr) *reinterpret_cast<uint2*>(a.o + ro + dim) = make_uint2(0u, 0u);
            }
          }
        if (!a.accumulate && hl == 0) lse32[((int64_t)b * a.oH + oh) * a.prows + (qi[qb] - a.prow0)] = -INFINITY;
      }
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
  const float c2 = a.scale_log2;
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
      for (int r = 0; r < 16; ++r) sacc[qb][r] = TSP_ATTN_CINIT ? -m_cm[qb] : 0.0f;
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
#if TSP_ATTN_CINIT
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
#else
  // Row max, reference max, exponentials, bf16 P and their sum. Returns whether this lane
  // needs the O rescale (then by the factors in alpha).
  auto softmax = [&] __device__(f32x16 (&sacc)[QB], const float (&)[QB], bf16x8 (&pf)[QB][2],
                                float (&alpha)[QB]) {
    bool any = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = sacc[qb][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sacc[qb][r]);
      mx = max_swap32(mx);
      const float mxs = mx * c2;
      const bool upd = mxs > m_s[qb] + kLazy;
      const float m_new = upd ? mxs : m_s[qb];
      alpha[qb] = __builtin_amdgcn_exp2f(m_s[qb] - m_new);
      any |= upd;
      m_s[qb] = m_new;
      const float nm = -m_new;
      float lsum = 0.0f;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[qb][8 * half + 2 * e], c2, nm));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[qb][8 * half + 2 * e + 1], c2, nm));
          w[e] = pack_bf16x2(p0, p1);
          lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[e]), ones, lsum, false);
        }
        pf[qb][half] = as_bf16x8(make_uint4(w[0], w[1], w[2], w[3]));
      }
      l_run[qb] = __builtin_fmaf(l_run[qb], alpha[qb], lsum);
    }
    return any;
  };
#endif
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

  float inv[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = l_run[qb] + __shfl_xor(l_run[qb], 32);
    inv[qb] = PART ? (l_tot > 0.0f ? 1.0f / l_tot : 0.0f) : 1.0f / l_tot;
    l_run[qb] = l_tot;
  }
  if constexpr (PART) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if (qi[qb] >= a.rows) continue;
      const int64_t ro = ((int64_t)b * a.rows + qi[qb]) * tok + (int64_t)h * HD;
      float* op = o32 + ((int64_t)b * a.prows + (qi[qb] - a.prow0)) * otok + (int64_t)oh * HD;
      float* lp = lse32 + ((int64_t)b * a.oH + oh) * a.prows + (qi[qb] - a.prow0);
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
          *reinterpret_cast<f32x4*>(op + dim) = val;
          if (a.o != nullptr) *reinterpret_cast<uint2*>(a.o + ro + dim) = pack_bf16x4(val[0], val[1], val[2], val[3]);
        }
      }
      if (hl == 0) *lp = lse_new;
    }
    return;
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    if (qi[qb] >= a.rows) continue;
    bf16_t* op = a.o + ((int64_t)b * a.rows + qi[qb]) * tok + (int64_t)h * HD;
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
      a.lse[((int64_t)b * a.H + h) * a.rows + qi[qb]] = (m_s[qb] + __log2f(l_run[qb])) * 0.69314718055994531f;
  }
}

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
    hipLaunchKernelGGL((attn_fwd<128, PART>), dim3(a.items), dim3(kThreads), 0, stream, a);
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

// Two-part attention for launches of at most one round of tiles (one per CU): the time is
// then that of the heaviest tile, and the later zigzag chunk's tiles see up to (2D - r) C
// keys against at most (r + 1) C for the earlier chunk's. The earlier chunk's tiles run as
// they are (bf16 O); each later-chunk tile runs as two items, keys [0, split) and
// [split, end), with split at half of that chunk's key span, into fp32 partials of the later
// chunk's rows only, merged by log-sum-exp into bf16 O. Every later-chunk row lies at or after
// split, so both halves see keys. Applies when chunks hold whole tiles and the later chunk's
// span is at least twice the earlier one's (r <= (2D - 2) / 3).
constexpr int kCus = 256;

int attn_two_part_split(int B, int64_t S, int D, int rank, int H) {
  const int64_t C = S / (2 * D);
  if (C <= 0 || C % BR != 0) return 0;
  const int64_t n_qt = 2 * C / BR;
  if ((int64_t)B * H * n_qt > kCus) return 0;
  if (3 * (int64_t)rank > 2 * (int64_t)D - 2) return 0;
  const int64_t split = ((2 * (int64_t)D - rank) * C / 2) / BC * BC;
  if (split <= 0 || split > (2 * (int64_t)D - 1 - rank) * C) return 0;
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
  AttnArgs e = base_args(q, k_full, v_full, B, S, D, rank, H, hd, scale);
  const int c_tiles = (int)(e.C / BR);
  // earlier chunk: tiles [0, C / BR), bf16 O
  e.o = static_cast<bf16_t*>(o);
  e.qt_hi = c_tiles;
  e.items = B * H * c_tiles;
  if (hipError_t err = launch<false>(e, hd, stream)) return err;
  // later chunk: tiles [C / BR, 2C / BR), two key halves each, partials of rows [C, 2C)
  AttnArgs l = base_args(q, k_full, v_full, B, S, D, rank, H, hd, scale);
  const int64_t units = (int64_t)B * l.C * H;
  float* o32 = static_cast<float*>(part);
  l.o32 = o32;
  l.lse = o32 + 2 * units * hd;
  l.qt_lo = c_tiles;
  l.prow0 = (int)l.C;
  l.prows = (int)l.C;
  l.split = split;
  l.part_o = units * hd;
  l.part_l = units;
  l.items = 2 * B * H * (l.n_qt - c_tiles);
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
