// tsp_attn_bwd.hip -- gradients of the rank's causal attention: dq for its queries and its
// dk/dv contributions for every key position.
//
// Forward (per query row i at global position p_i, visible keys j <= p_i):
//   s_ij = scale q_i.k_j, P_ij = exp(s_ij - lse_i), o_i = sum_j P_ij v_j.
// Backward, with D_i = do_i . o_i (= sum_j P_ij dP_ij):
//   dv_j = sum_i P_ij do_i,  dP_ij = do_i . v_j,  ds_ij = P_ij (dP_ij - D_i),
//   dq_i = scale sum_j ds_ij k_j,  dk_j = scale sum_i ds_ij q_i.
// The forward's log-sum-exp gives P directly (no running max). Two kernels:
//   attn_bwd_dq    query-stationary: a wave owns 32 query rows and streams the key blocks
//                  its rows see; it also writes D_i for the second kernel.
//   attn_bwd_dkdv  key-stationary: a wave owns 32 keys and streams the rank's query rows
//                  that see them (a suffix of the local rows: they ascend in position).
// MFMA v_mfma_f32_32x32x16_bf16 throughout, in the forward kernel's formulation: S^T = K Q^T
// (and dP^T = V dO^T) leave each lane with one query's scores, which packed to bf16 are the
// B operand of dQ^T += K^T dS^T, whose A operand comes from LDS by transpose reads. The
// key-stationary kernel uses S = Q K^T instead, so that each lane holds one key's column.
// Both kernels stage their streamed operand by LDS DMA (global_load_lds): the K/V tiles of
// the query-stationary kernel in a three-stage ring, the Q/dO blocks (with their lse and D
// words) of the key-stationary kernel in a four-stage ring. The source address of each lane's 16 bytes is chosen so that
// the tile lands in LDS already swizzled.
#include <hip/hip_runtime.h>

#include "tsp_device.h"
#include "tsp_internal.h"

namespace tsp {
namespace {

constexpr int kDqWaves = 8;                 // query-stationary: 256 query rows per workgroup
constexpr int kDqThreads = 64 * kDqWaves;
constexpr int kDqRows = 32 * kDqWaves;
constexpr int kKvWaves = 8;                 // key-stationary: 8 waves x 32 keys (two per SIMD)
constexpr int kKvThreads = 64 * kKvWaves;
constexpr int kKeysPerWg = 32 * kKvWaves;
constexpr int kKvRing = 4;                  // key-stationary: Q/dO stages in the DMA ring
constexpr int kStage = 64;                  // query-stationary: keys staged per LDS fill
constexpr int kKvStage = 32;                // key-stationary: query rows per DMA stage
constexpr int kDqRing = 3;                  // query-stationary: K/V stages in the DMA ring
constexpr float kLog2e = 1.4426950408889634f;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// The 4-byte form of the LDS DMA copies (global_load_lds_dword): lane i's word lands at
// `lds` + 4 i (M0 holds `lds`). Like the 16-byte forms it is issued from inline assembly
// and ordered by explicit s_waitcnt vmcnt and s_barrier.
__device__ __forceinline__ void dma4_vaddr(const void* addr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(addr), "s"(lds) : "memory");
}

// s_waitcnt vmcnt(n) for a wave-uniform n known only at run time (s_waitcnt takes an
// immediate). Counts above 15 wait for 15: a smaller count only waits longer.
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
#define TSP_WAIT_VM_CASE(k)                    \
  case k:                                      \
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(k)); \
    break;
    TSP_WAIT_VM_CASE(0) TSP_WAIT_VM_CASE(1) TSP_WAIT_VM_CASE(2) TSP_WAIT_VM_CASE(3)
    TSP_WAIT_VM_CASE(4) TSP_WAIT_VM_CASE(5) TSP_WAIT_VM_CASE(6) TSP_WAIT_VM_CASE(7)
    TSP_WAIT_VM_CASE(8) TSP_WAIT_VM_CASE(9) TSP_WAIT_VM_CASE(10) TSP_WAIT_VM_CASE(11)
    TSP_WAIT_VM_CASE(12) TSP_WAIT_VM_CASE(13) TSP_WAIT_VM_CASE(14)
#undef TSP_WAIT_VM_CASE
    default:
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(15));
  }
}

template <int HD>
struct BLay {
  static constexpr int KS = HD / 16;   // 16-dim reduction steps
  static constexpr int DB = HD / 32;   // 32-dim output blocks
  static constexpr int ROWB = HD * 2;  // bytes per row
  static constexpr int CPR = ROWB / 16;
  static constexpr int TILEB = kStage * ROWB;
  // 16-byte chunk c of row r is stored at chunk c ^ sw(r). Each tile is read both ways: row
  // fragments (16 consecutive rows, one chunk) and transpose reads (4 rows aligned to 4 x 4
  // chunks aligned to 4). The swizzle's low bits separate the 16 rows of a row read and its
  // high bits the 4 rows of a transpose read, so that both cover 16 distinct 16-byte bank
  // groups (one 256-byte pass of the LDS).
  __device__ static int sw(int r) {
    return HD == 128 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
  }
  // A transpose read's second 8 rows (rows r + 8 for r < 8, in a 16-aligned group) have the
  // swizzle sw(r) ^ 2: their offset is the first read's with bit 5 flipped, 8 rows down.
  static constexpr int TR_HI_XOR = 32;
};

struct BwdArgs {
  const bf16_t* q;    // [B, rows, H, HD] the rank's queries
  const bf16_t* k;    // [B, S, H, HD]
  const bf16_t* v;
  const bf16_t* o;    // [B, rows, H, HD] forward output
  const bf16_t* d_o;  // [B, rows, H, HD]
  const float* lse;   // [B, H, rows] natural log
  float* dq;          // [B, rows, H, HD]
  float* dk;          // [B, S, H, HD]
  float* dv;
  float* dsum;        // [B, H, rows] D_i, written by attn_bwd_dq
  int64_t S, C;
  int rows, D, rank, H;
  float scale;
};

// A or B fragment of a 32-row block: lane (l32, hl) gets row rb + l32, dims 16 s + 8 hl .. +7.
template <int HD>
__device__ __forceinline__ bf16x8 row_frag(const char* tile, int rb, int l32, int hl, int s) {
  using L = BLay<HD>;
  const int r = rb + l32;
  return as_bf16x8(*reinterpret_cast<const uint4*>(tile + r * L::ROWB + 16 * ((2 * s + hl) ^ L::sw(r))));
}

// Transpose-read bases of the [32 dims x 16 rows] A fragments (dims block db): lane
// (G = lane / 16, j16 = lane % 16) reads row 4 hl + j16 / 4 of each group of 8, at the chunk
// that holds its dims; two reads 8 rows apart make one fragment. The row order this gives
// (rows 4 hl .. 4 hl + 3 and 8 + 4 hl .. 8 + 4 hl + 3 of a 16-row half) is the order in
// which an MFMA result's registers 8 half .. 8 half + 7 hold their rows, so the packed
// result of a previous MFMA serves directly as the B operand.
template <int HD>
__device__ __forceinline__ int tr_offset(int lane, int db) {
  using L = BLay<HD>;
  const int hl = lane >> 5, G = lane >> 4, j16 = lane & 15;
  const int r = 4 * hl + (j16 >> 2);
  const int c = 4 * db + 2 * (G & 1) + ((j16 & 3) >> 1);
  return r * L::ROWB + 16 * (c ^ L::sw(r)) + 8 * (j16 & 1);
}

template <int HD>
__device__ __forceinline__ bf16x8 tr_frag(const char* tile, int off, int rb) {
  using L = BLay<HD>;
  const char* base = tile + rb * L::ROWB;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + off));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + (off ^ L::TR_HI_XOR) + 8 * L::ROWB));
  const uint2 ulo = __builtin_bit_cast(uint2, lo), uhi = __builtin_bit_cast(uint2, hi);
  return as_bf16x8(make_uint4(ulo.x, ulo.y, uhi.x, uhi.y));
}

// Eight values (registers 8 half .. 8 half + 7 of an MFMA result) as bf16, rounded to
// nearest even: the B operand of the products that consume them.
__device__ __forceinline__ bf16x8 pack8(const float (&x)[8]) {
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(x[2 * e], x[2 * e + 1]);
  return as_bf16x8(make_uint4(w[0], w[1], w[2], w[3]));
}

// zigzag_pos in 32-bit arithmetic for the per-block tests (the positions of one sequence, and
// S itself, stay below 2^31: the launcher checks).
__device__ __forceinline__ int zz_pos(int i, int C, int r, int D) {
  return i < C ? r * C + i : (2 * D - 1 - r) * C + (i - C);
}

template <int HD>
__global__ __launch_bounds__(kDqThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_bwd_dq(BwdArgs a) {
  using L = BLay<HD>;
  constexpr int KS = L::KS, DB = L::DB;
  constexpr int CPR = L::CPR, TILEB = L::TILEB;
  constexpr int NDMA = TILEB / (kDqThreads * 16);  // 16-byte DMA loads per thread per tile
  static_assert(NDMA >= 1 && NDMA * kDqThreads * 16 == TILEB, "whole tile per stage");
  // K and V rings of kDqRing 64-key stages, filled by LDS DMA two stages ahead of the MFMAs
  __shared__ __attribute__((aligned(1024))) char kring[kDqRing * TILEB];
  __shared__ __attribute__((aligned(1024))) char vring[kDqRing * TILEB];
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hl = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n_qt = (a.rows + kDqRows - 1) / kDqRows;
  const int bh = blockIdx.x / n_qt;
  const int qt = n_qt - 1 - (int)(blockIdx.x - bh * n_qt);  // heaviest tile first
  const int b = bh / a.H, h = bh - (bh / a.H) * a.H;
  const int row0 = qt * kDqRows;
  const int kv_end = (int)zigzag_pos(min(row0 + kDqRows, a.rows) - 1, a.C, a.rank, a.D) + 1;
  const int64_t tok = (int64_t)a.H * HD;

  const int qi = row0 + 32 * wave + l32;
  const bool valid = qi < a.rows;
  const int qic = valid ? qi : a.rows - 1;
  const int qpos = (int)zigzag_pos(qic, a.C, a.rank, a.D);
  // the wave's first row has its lowest position (local rows ascend in position)
  const int wave_pos0 = (int)zigzag_pos(min(row0 + 32 * wave, a.rows - 1), a.C, a.rank, a.D);
  // and its last row the highest: key blocks past it add nothing to the wave's rows
  const int wave_pos1 = (int)zigzag_pos(min(row0 + 32 * wave + 31, a.rows - 1), a.C, a.rank, a.D);
  const int64_t rowoff = ((int64_t)b * a.rows + qic) * tok + (int64_t)h * HD + 8 * hl;
  bf16x8 qf[KS], df[KS];
  float dsum = 0.0f;
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    qf[s] = as_bf16x8(*reinterpret_cast<const uint4*>(a.q + rowoff + 16 * s));
    df[s] = as_bf16x8(*reinterpret_cast<const uint4*>(a.d_o + rowoff + 16 * s));
    const bf16x8 of = as_bf16x8(*reinterpret_cast<const uint4*>(a.o + rowoff + 16 * s));
#pragma unroll
    for (int e = 0; e < 8; ++e) dsum += (float)df[s][e] * (float)of[e];
  }
  dsum += __shfl_xor(dsum, 32);  // the other half of the row's dims
  const int64_t li = ((int64_t)b * a.H + h) * a.rows + qic;
  if (valid && hl == 0) a.dsum[li] = dsum;
  const float lse2 = a.lse[li] * kLog2e;
  const float c2 = a.scale * kLog2e;

  f32x16 dqacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dqacc[db] = f32x16{};
  int troff[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) troff[db] = tr_offset<HD>(lane, db);

  // ---- stage loads: global -> LDS by DMA, 16 bytes per lane, lane-linear within the 1 KB a
  // wave instruction writes; load p of this wave fills linear chunk (NW p + wave) 64 + lane
  // of the tile, whose source is the logical chunk that the swizzle puts there.
  const char* kseq = reinterpret_cast<const char*>(a.k + (int64_t)b * a.S * tok + (int64_t)h * HD);
  const char* vseq = reinterpret_cast<const char*>(a.v + (int64_t)b * a.S * tok + (int64_t)h * HD);
  const uint32_t tokb = (uint32_t)(tok * 2);
  int drow[NDMA], dch[NDMA];
#pragma unroll
  for (int p = 0; p < NDMA; ++p) {
    const int lin = (kDqWaves * p + wave) * 64 + lane;
    drow[p] = lin / CPR;
    dch[p] = 16 * ((lin % CPR) ^ L::sw(drow[p]));
  }
  auto issue = [&] __device__(int st, int key0) {
    const int lim = kv_end - 1 - key0;  // rows past the tile's last key repeat it (masked)
    const char* kb0 = kseq + (int64_t)key0 * tokb;
    const char* vb0 = vseq + (int64_t)key0 * tokb;
    const uint32_t lk = lds_addr(kring) + st * TILEB + wave * 1024;
    const uint32_t lv = lds_addr(vring) + st * TILEB + wave * 1024;
#pragma unroll
    for (int p = 0; p < NDMA; ++p) {
      const uint32_t roff = (uint32_t)min(drow[p], lim) * tokb + dch[p];
      dma16_sbase(kb0, roff, lk + kDqWaves * p * 1024);
      dma16_sbase(vb0, roff, lv + kDqWaves * p * 1024);
    }
  };
  const int n_st = (kv_end + kStage - 1) / kStage;
  issue(0, 0);
  if (n_st > 1) issue(1, kStage);
  int st = 0;
  for (int t = 0; t < n_st; ++t, st = (st + 1 == kDqRing ? 0 : st + 1)) {
    // this wave's loads of stage t have landed (those of stage t + 1 may be in flight), then
    // a bare barrier: every wave's have, and every wave is done with stage t - 1's buffer,
    // which stage t + 2 refills
    if (t + 1 < n_st) {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * NDMA));
    } else {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");  // no LDS read moves above the barrier
    if (t + 2 < n_st) issue(st + 2 >= kDqRing ? st + 2 - kDqRing : st + 2, (t + 2) * kStage);
    const char* ktile = kring + st * TILEB;
    const char* vtile = vring + st * TILEB;
    const int key0 = t * kStage;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int k0 = key0 + 32 * kb;
      if (k0 >= kv_end || k0 > wave_pos1) break;  // no row of the wave sees these keys
      f32x16 s = {}, dp = {};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s = mfma32x32x16(row_frag<HD>(ktile, 32 * kb, l32, hl, ks), qf[ks], s);
        dp = mfma32x32x16(row_frag<HD>(vtile, 32 * kb, l32, hl, ks), df[ks], dp);
      }
      // Where some row of the wave may not see some key of the block (a wave-uniform test), the
      // scores of keys past the row's position become -inf, so that their P is 0; other blocks
      // carry no mask.
      if (k0 + 31 > wave_pos0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 8 * (r >> 2) + 4 * hl + (r & 3);
          if (key > qpos) s[r] = -INFINITY;
        }
      }
      // dS one half of the block (registers 8 half .. 8 half + 7) at a time, packed and
      // consumed by the dQ products before the next half is computed
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        float ds[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 8 * half + e;
          const float p = __builtin_amdgcn_exp2f(s[r] * c2 - lse2);
          ds[e] = p * (dp[r] - dsum);
        }
        const bf16x8 dsf = pack8(ds);
#pragma unroll
        for (int db = 0; db < DB; ++db)
          dqacc[db] = mfma32x32x16(tr_frag<HD>(ktile, troff[db], 32 * kb + 16 * half), dsf, dqacc[db]);
      }
    }
  }
  if (!valid) return;
  float* out = a.dq + ((int64_t)b * a.rows + qi) * tok + (int64_t)h * HD;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x16& x = dqacc[db];
      *reinterpret_cast<f32x4*>(out + 32 * db + 8 * g + 4 * hl) =
          f32x4{x[4 * g] * a.scale, x[4 * g + 1] * a.scale, x[4 * g + 2] * a.scale, x[4 * g + 3] * a.scale};
    }
}

template <int HD>
__global__ __launch_bounds__(kKvThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_bwd_dkdv(BwdArgs a) {
  using L = BLay<HD>;
  constexpr int KS = L::KS, DB = L::DB, ROWB = L::ROWB, CPR = L::CPR;
  constexpr int STB = kKvStage * ROWB;                         // bytes of one staged Q (or dO) block
  constexpr int CHUNKS = STB / 16;                             // its 16-byte chunks
  constexpr int NDMA = (CHUNKS + kKvThreads - 1) / kKvThreads;  // DMA loads per thread per block
  static_assert(CHUNKS % 64 == 0, "whole waves per block");
  // Q and dO rings of kKvRing 32-row stages, and each stage's lse and D (64 words), filled
  // by LDS DMA up to kKvRing - 1 stages ahead of the MFMAs
  __shared__ __attribute__((aligned(1024))) char qring[kKvRing * STB];
  __shared__ __attribute__((aligned(1024))) char oring[kKvRing * STB];
  __shared__ __attribute__((aligned(256))) float lsed[kKvRing][2 * kKvStage];
  // V rows of the workgroup's keys: read as B fragments of dP = dO V^T each block (kept in
  // LDS rather than registers, so that two waves fit on a SIMD)
  __shared__ __attribute__((aligned(16))) char vkeys[kKeysPerWg * ROWB];
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hl = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n_kt = (int)((a.S + kKeysPerWg - 1) / kKeysPerWg);
  const int bh = blockIdx.x / n_kt;
  const int kt = (int)(blockIdx.x - bh * n_kt);
  const int b = bh / a.H, h = bh - (bh / a.H) * a.H;
  const int key0 = kt * kKeysPerWg;
  const int64_t tok = (int64_t)a.H * HD;

  const int C32 = (int)a.C, S32 = (int)a.S;
  const int kw0 = key0 + 32 * wave;  // the wave's first key
  const int kj = kw0 + l32;
  const int wave_klast = kw0 + 31;
  const bool kvalid = kj < a.S;
  const int kjc = kvalid ? kj : (int)a.S - 1;
  const int64_t keyoff = ((int64_t)b * a.S + kjc) * tok + (int64_t)h * HD + 8 * hl;
  bf16x8 kf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) kf[s] = as_bf16x8(*reinterpret_cast<const uint4*>(a.k + keyoff + 16 * s));
  {
    const bf16_t* vrows = a.v + (int64_t)b * a.S * tok + (int64_t)h * HD;
    for (int lin = tid; lin < kKeysPerWg * CPR; lin += kKvThreads) {
      const int r = lin / CPR, c = lin - (lin / CPR) * CPR;
      const int gr = (int)min((int64_t)key0 + r, a.S - 1);
      *reinterpret_cast<uint4*>(vkeys + r * ROWB + 16 * (c ^ L::sw(r))) =
          *reinterpret_cast<const uint4*>(vrows + (int64_t)gr * tok + 8 * c);
    }
  }
  __syncthreads();  // vkeys complete (the ring below synchronises with bare barriers)

  // The rank's local rows ascend in position (chunk r, then chunk 2D-1-r): the rows that see
  // any of this workgroup's keys are the suffix from the first row at position >= key0.
  const int64_t lo_a = (int64_t)a.rank * a.C, lo_b = (int64_t)(2 * a.D - 1 - a.rank) * a.C;
  int i0;
  if (key0 < lo_a + a.C) {
    i0 = (int)max((int64_t)0, key0 - lo_a);
  } else if (key0 < lo_b + a.C) {
    i0 = (int)(a.C + max((int64_t)0, key0 - lo_b));
  } else {
    i0 = a.rows;
  }
  const float c2 = a.scale * kLog2e;
  f32x16 dkacc[DB], dvacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dkacc[db] = dvacc[db] = f32x16{};
  int troff[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) troff[db] = tr_offset<HD>(lane, db);

  // ---- stage loads: global -> LDS by DMA, 16 bytes per lane, lane-linear within the 1 KB a
  // wave instruction writes. Load p of this wave fills linear chunk (NW p + wave) 64 + lane
  // of the block: row lin / CPR at physical chunk lin % CPR, which holds logical chunk
  // (lin % CPR) ^ sw(row); the source address is chosen accordingly. Wave 0 also copies
  // the stage's 32 lse and 32 D words.
  const char* qseq = reinterpret_cast<const char*>(a.q + (int64_t)b * a.rows * tok + (int64_t)h * HD);
  const char* oseq = reinterpret_cast<const char*>(a.d_o + (int64_t)b * a.rows * tok + (int64_t)h * HD);
  const uint32_t tokb = (uint32_t)(tok * 2);
  const int64_t lrow = ((int64_t)b * a.H + h) * a.rows;
  int drow[NDMA], dch[NDMA];
  int per_stage = wave == 0 ? 1 : 0;  // this wave's loads per stage
#pragma unroll
  for (int p = 0; p < NDMA; ++p) {
    const int lin = (kKvWaves * p + wave) * 64 + lane;
    drow[p] = lin / CPR;
    dch[p] = 16 * ((lin % CPR) ^ L::sw(drow[p] % kKvStage));
    if ((kKvWaves * p + wave) * 64 < CHUNKS) per_stage += 2;
  }
  auto issue = [&] __device__(int st, int q0) {
    const int lim = a.rows - 1 - q0;  // rows past the last local row repeat it (masked)
    const char* qb0 = qseq + (int64_t)q0 * tokb;
    const char* ob0 = oseq + (int64_t)q0 * tokb;
    const uint32_t lq = lds_addr(qring) + st * STB + wave * 1024;
    const uint32_t lo = lds_addr(oring) + st * STB + wave * 1024;
#pragma unroll
    for (int p = 0; p < NDMA; ++p) {
      if ((kKvWaves * p + wave) * 64 >= CHUNKS) break;  // the same for the whole wave
      const uint32_t roff = (uint32_t)min(drow[p], lim) * tokb + dch[p];
      dma16_sbase(qb0, roff, lq + kKvWaves * p * 1024);
      dma16_sbase(ob0, roff, lo + kKvWaves * p * 1024);
    }
    if (wave == 0) {
      const int ri = min(q0 + (lane & 31), a.rows - 1);
      dma4_vaddr((lane < 32 ? a.lse : a.dsum) + lrow + ri, lds_addr(&lsed[st][0]));
    }
  };
  const int n_st = i0 < a.rows ? (a.rows - i0 + kKvStage - 1) / kKvStage : 0;
  for (int t = 0; t < kKvRing - 1 && t < n_st; ++t) issue(t, i0 + t * kKvStage);
  int st = 0;
  for (int t = 0; t < n_st; ++t, st = (st + 1 == kKvRing ? 0 : st + 1)) {
    // this wave's loads of stage t have landed (later stages' may be in flight), then a bare
    // barrier: every wave's have, and every wave is done with stage t - 1's buffers, which
    // stage t + kKvRing - 1 refills
    wait_vm(min(kKvRing - 2, n_st - 1 - t) * per_stage);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");  // no LDS read moves above the barrier
    const int q0 = i0 + t * kKvStage;
    if (t + kKvRing - 1 < n_st) issue(st == 0 ? kKvRing - 1 : st - 1, q0 + (kKvRing - 1) * kKvStage);
    const char* qtile = qring + st * STB;
    const char* otile = oring + st * STB;
    const float* lse_s = &lsed[st][0];  // natural log
    const float* d_s = &lsed[st][kKvStage];
    // no row of the block sees the wave's keys (its last row has the highest position)
    if (kw0 > zz_pos(min(q0 + kKvStage - 1, a.rows - 1), C32, a.rank, a.D)) continue;
    f32x16 s = {}, dp = {};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s = mfma32x32x16(row_frag<HD>(qtile, 0, l32, hl, ks), kf[ks], s);
      dp = mfma32x32x16(row_frag<HD>(otile, 0, l32, hl, ks), row_frag<HD>(vkeys, 32 * wave, l32, hl, ks), dp);
    }
    // The block's first row has its lowest position: if that row sees the wave's last key,
    // every row sees every key (a wave-uniform test). Otherwise each register whose (row, key)
    // pair is not visible gets score -inf (so P = 0) and dP = D (so dP - D = 0: a key past
    // the rank's last position has K and V rows the caller need not fill, and its score and
    // dP may be NaN); the P and dS code below is then the same for every block, with no
    // per-register compare or select.
    const bool whole =
        q0 + 31 < a.rows && wave_klast < S32 && wave_klast <= zz_pos(q0, C32, a.rank, a.D);
    if (!whole) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qr = 8 * (r >> 2) + 4 * hl + (r & 3);  // query row of register r in the block
        const int row = q0 + qr;
        const bool ok =
            kvalid & (row < a.rows) & (kj <= zz_pos(min(row, a.rows - 1), C32, a.rank, a.D));
        if (!ok) {
          s[r] = -INFINITY;
          dp[r] = d_s[qr];
        }
      }
    }
    // P and dS one half of the block (registers 8 half .. 8 half + 7) at a time, each packed
    // and consumed by the dV and dK products before the next half is computed.
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      float p[8], ds[8];
      // registers 4 j .. 4 j + 3 hold query rows 8 j + 4 hl .. + 3: their lse and D as one
      // 16-byte read each
      f32x4 lq[2], dq4[2];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        lq[jj] = *reinterpret_cast<const f32x4*>(lse_s + 8 * (2 * half + jj) + 4 * hl);
        dq4[jj] = *reinterpret_cast<const f32x4*>(d_s + 8 * (2 * half + jj) + 4 * hl);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = 8 * half + e;
        const float ex = __builtin_amdgcn_exp2f(s[r] * c2 - lq[e >> 2][e & 3] * kLog2e);
        p[e] = ex;
        ds[e] = ex * (dp[r] - dq4[e >> 2][e & 3]);
      }
      const bf16x8 pf = pack8(p);
      const bf16x8 dsf = pack8(ds);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        dvacc[db] = mfma32x32x16(tr_frag<HD>(otile, troff[db], 16 * half), pf, dvacc[db]);
        dkacc[db] = mfma32x32x16(tr_frag<HD>(qtile, troff[db], 16 * half), dsf, dkacc[db]);
      }
    }
  }
  if (!kvalid) return;
  const int64_t ko = ((int64_t)b * a.S + kj) * tok + (int64_t)h * HD;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dim = 32 * db + 8 * g + 4 * hl;
      const f32x16& xk = dkacc[db];
      const f32x16& xv = dvacc[db];
      *reinterpret_cast<f32x4*>(a.dk + ko + dim) =
          f32x4{xk[4 * g] * a.scale, xk[4 * g + 1] * a.scale, xk[4 * g + 2] * a.scale, xk[4 * g + 3] * a.scale};
      *reinterpret_cast<f32x4*>(a.dv + ko + dim) = f32x4{xv[4 * g], xv[4 * g + 1], xv[4 * g + 2], xv[4 * g + 3]};
    }
}

}  // namespace

hipError_t launch_attn_bwd(const void* q, const void* k_full, const void* v_full, const void* o, const float* lse,
                           const void* d_o, float* dq, float* dk_full, float* dv_full, float* dsum, int B, int64_t S,
                           int D, int rank, int H, int hd, float scale, hipStream_t stream) {
  BwdArgs a;
  a.q = static_cast<const bf16_t*>(q);
  a.k = static_cast<const bf16_t*>(k_full);
  a.v = static_cast<const bf16_t*>(v_full);
  a.o = static_cast<const bf16_t*>(o);
  a.d_o = static_cast<const bf16_t*>(d_o);
  a.lse = lse;
  a.dq = dq;
  a.dk = dk_full;
  a.dv = dv_full;
  a.dsum = dsum;
  a.S = S;
  a.C = S / (2 * D);
  a.rows = (int)(2 * a.C);
  a.D = D;
  a.rank = rank;
  a.H = H;
  a.scale = scale > 0.0f ? scale : 1.0f / sqrtf((float)hd);
  const int n_qt = (a.rows + kDqRows - 1) / kDqRows;
  const int n_kt = (int)((S + kKeysPerWg - 1) / kKeysPerWg);
  const dim3 gq((unsigned)(B * H * n_qt)), gk((unsigned)(B * H * n_kt));
  if (hd == 128) {
    hipLaunchKernelGGL(attn_bwd_dq<128>, gq, dim3(kDqThreads), 0, stream, a);
    hipLaunchKernelGGL(attn_bwd_dkdv<128>, gk, dim3(kKvThreads), 0, stream, a);
  } else {
    hipLaunchKernelGGL(attn_bwd_dq<64>, gq, dim3(kDqThreads), 0, stream, a);
    hipLaunchKernelGGL(attn_bwd_dkdv<64>, gk, dim3(kKvThreads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace tsp
