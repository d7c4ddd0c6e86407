// tsp_attn.hip -- causal attention of one TSP rank's zigzag queries against the
// full-sequence K/V, on gfx950 MFMA.
//
// TSP summary §2 (attention layers): after the K/V all-gather every rank runs
// FlashAttention for its own queries over the whole sequence, and the zigzag partition
// (chunk r with its mirror 2D-1-r) balances the causal work between ranks. This kernel
// is that step for one rank: online softmax in fp32, S x S never materialised.
//
// Work decomposition. One workgroup (4 waves) owns 128 consecutive local query rows of
// one (sequence, head); each wave owns 32 of them. Local rows ascend in position, so a
// tile's last row bounds its keys: the tile streams keys [0, pos(last)+1) in stages of
// 64 and never reads a key row after the rank's last position. Stages at or before the
// tile's first position need no mask (only the last two or three are masked per
// element). Within one (sequence, head) the heaviest tile is dispatched first, and each
// XCD takes a contiguous range of (sequence, head) work so the query tiles running
// together on it stream the same K/V through its L2.
//
// MFMA formulation (v_mfma_f32_32x32x16_bf16, see tsp_device.h for the lane layout):
//   S^T = K Q^T   A = K rows from LDS, B = this wave's Q (registers). Each lane ends up
//                 holding 16 of the 32 keys of one 32-key block for ITS query
//                 (column lane%32); the other 16 sit in lane^32. Row max / row sum
//                 therefore need one exchange with lane^32 per stage.
//   O^T += V^T P^T  B = P straight from the S^T registers (converted to bf16); A = V^T
//                 read from LDS with the same key labelling. O^T keeps each lane on its
//                 own query, so the online-softmax rescale is a per-lane scalar.
// V is stored transposed in LDS ([dim][key], padded) so a lane's A fragment is two
// 8-byte reads; K is stored [key][dim] padded by 16 bytes so 16-byte fragment reads of
// consecutive keys fall in distinct banks. Both are double buffered: the global loads
// of stage t+1 are in flight while stage t computes.
// The softmax runs in base 2: s2 = s * scale * log2(e), p = exp2(s2 - m2).
#include <math.h>

#include "tsp_device.h"
#include "tsp_internal.h"

namespace tsp {
namespace {

constexpr int BR = 128;  // query rows per workgroup
constexpr int BC = 64;   // keys per stage
constexpr int kThreads = 256;

struct AttnArgs {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  bf16_t* o;
  float* lse;
  int64_t S;
  int64_t C;
  int rows;  // 2C local rows per sequence
  int D, rank, H;
  int n_qt;   // query tiles per (sequence, head)
  int items;  // B * H * n_qt
  float scale_log2;
};

// Element e (0..7) of x0 in the low half and of x1 in the high half of a word.
__device__ __forceinline__ uint32_t pair_elem(const uint4& x0, const uint4& x1, int e) {
  const uint32_t w0 = e < 2 ? x0.x : e < 4 ? x0.y : e < 6 ? x0.z : x0.w;
  const uint32_t w1 = e < 2 ? x1.x : e < 4 ? x1.y : e < 6 ? x1.z : x1.w;
  return (e & 1) ? ((w0 >> 16) | (w1 & 0xFFFF0000u)) : ((w0 & 0xFFFFu) | (w1 << 16));
}

template <int HD>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_fwd(AttnArgs a) {
  constexpr int KS = HD / 16;       // 16-dim reduction steps of Q K^T
  constexpr int DB = HD / 32;       // 32-dim output blocks
  constexpr int KSTR = HD + 8;      // padded K row (elements)
  constexpr int VSTR = BC + 4;      // padded V^T row (elements)
  constexpr int VCH = HD / 8;       // 16-byte chunks per key row
  constexpr int KCH = BC * VCH / kThreads;  // K chunks per thread per stage
  constexpr int KPT = HD / 32;      // keys per thread in the V^T fill (4 or 2)
  static_assert(KPT * (kThreads / VCH) == BC, "V^T fill must cover the stage");
  static_assert(KPT == 2 || KPT == 4, "head_dim 64 or 128");
  __shared__ __attribute__((aligned(16))) bf16_t ks[2][BC * KSTR];
  __shared__ __attribute__((aligned(16))) bf16_t vt[2][HD * VSTR];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hl = lane >> 5;

  const int item = xcd_remap(blockIdx.x, a.items);
  const int bh = item / a.n_qt;
  const int qt = a.n_qt - 1 - (item - bh * a.n_qt);  // heaviest tile of the (b, h) first
  const int b = bh / a.H, h = bh - (bh / a.H) * a.H;
  const int row0 = qt * BR;
  const int last_row = min(row0 + BR, a.rows) - 1;
  const int64_t pmin = zigzag_pos(row0, a.C, a.rank, a.D);
  const int64_t kv_end = zigzag_pos(last_row, a.C, a.rank, a.D) + 1;
  const int n_kt = (int)((kv_end + BC - 1) / BC);
  const int n_full = (int)((pmin + 1) / BC);

  const int qi = row0 + wave * 32 + l32;
  const bool qvalid = qi < a.rows;
  const int qic = qvalid ? qi : a.rows - 1;
  const int64_t qpos = zigzag_pos(qic, a.C, a.rank, a.D);
  const int64_t tok = (int64_t)a.H * HD;  // elements between consecutive tokens

  bf16x8 qf[KS];
  {
    const bf16_t* qp = a.q + ((int64_t)b * a.rows + qic) * tok + (int64_t)h * HD + 8 * hl;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[s] = qvalid ? as_bf16x8(*reinterpret_cast<const uint4*>(qp + 16 * s)) : bf16x8{};
  }

  const bf16_t* kbase = a.k + (int64_t)b * a.S * tok + (int64_t)h * HD;
  const bf16_t* vbase = a.v + (int64_t)b * a.S * tok + (int64_t)h * HD;

  uint4 rk[KCH];
  uint4 rv[KPT];
  const int vg = tid / VCH, vdc = tid % VCH;
  auto gload = [&](int t) {
    const int64_t key0 = (int64_t)t * BC;
#pragma unroll
    for (int p = 0; p < KCH; ++p) {
      const int c = tid + kThreads * p;
      const int64_t kg = key0 + c / VCH;
      rk[p] = kg < kv_end ? *reinterpret_cast<const uint4*>(kbase + kg * tok + 8 * (c % VCH)) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int kk = 0; kk < KPT; ++kk) {
      const int64_t kg = key0 + vg * KPT + kk;
      rv[kk] = kg < kv_end ? *reinterpret_cast<const uint4*>(vbase + kg * tok + 8 * vdc) : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int p = 0; p < KCH; ++p) {
      const int c = tid + kThreads * p;
      *reinterpret_cast<uint4*>(&ks[buf][(c / VCH) * KSTR + 8 * (c % VCH)]) = rk[p];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      bf16_t* dst = &vt[buf][(8 * vdc + e) * VSTR + vg * KPT];
      if constexpr (KPT == 4) {
        *reinterpret_cast<uint2*>(dst) = make_uint2(pair_elem(rv[0], rv[1], e), pair_elem(rv[2], rv[3], e));
      } else {
        *reinterpret_cast<uint32_t*>(dst) = pair_elem(rv[0], rv[1], e);
      }
    }
  };

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.0f;

  gload(0);
  sstore(0);
  __syncthreads();
  for (int t = 0; t < n_kt; ++t) {
    const int cur = t & 1;
    if (t + 1 < n_kt) gload(t + 1);

    f32x16 sacc[BC / 32];
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb) {
      sacc[kb] = f32x16{};
      const bf16_t* kr = &ks[cur][(kb * 32 + l32) * KSTR + 8 * hl];
#pragma unroll
      for (int s = 0; s < KS; ++s)
        sacc[kb] = mfma32x32x16(as_bf16x8(*reinterpret_cast<const uint4*>(kr + 16 * s)), qf[s], sacc[kb]);
    }

    float mx = m_run;
    const bool masked = t >= n_full;
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float sv = sacc[kb][r] * a.scale_log2;
        if (masked) {
          const int64_t key = (int64_t)t * BC + kb * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
          if (key > qpos) sv = -INFINITY;
        }
        sacc[kb][r] = sv;
        mx = fmaxf(mx, sv);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float alpha = __builtin_amdgcn_exp2f(m_run - mx);
    m_run = mx;

    float lsum = 0.0f;
    bf16x8 pf[BC / 16];
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = __builtin_amdgcn_exp2f(sacc[kb][8 * half + e] - mx);
          lsum += p;
          pf[2 * kb + half][e] = (__bf16)p;
        }
      }
    }
    l_run = l_run * alpha + lsum;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] *= alpha;

#pragma unroll
    for (int s = 0; s < BC / 16; ++s) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16_t* vr = &vt[cur][(db * 32 + l32) * VSTR + 16 * s + 4 * hl];
        const uint2 lo = *reinterpret_cast<const uint2*>(vr);
        const uint2 hi = *reinterpret_cast<const uint2*>(vr + 8);
        oacc[db] = mfma32x32x16(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), pf[s], oacc[db]);
      }
    }

    if (t + 1 < n_kt) sstore(cur ^ 1);
    __syncthreads();
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  if (qvalid) {
    bf16_t* op = a.o + ((int64_t)b * a.rows + qi) * tok + (int64_t)h * HD;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dim = db * 32 + 8 * g + 4 * hl;
        *reinterpret_cast<uint2*>(op + dim) = pack_bf16x4(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv,
                                                          oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
      }
    }
    if (a.lse != nullptr && hl == 0)
      a.lse[((int64_t)b * a.H + h) * a.rows + qi] = (m_run + __log2f(l_tot)) * 0.69314718055994531f;
  }
}

}  // namespace

hipError_t launch_attn(const void* q, const void* k_full, const void* v_full, void* o, float* lse, int B, int64_t S,
                       int D, int rank, int H, int hd, float scale, hipStream_t stream) {
  AttnArgs a;
  a.q = static_cast<const bf16_t*>(q);
  a.k = static_cast<const bf16_t*>(k_full);
  a.v = static_cast<const bf16_t*>(v_full);
  a.o = static_cast<bf16_t*>(o);
  a.lse = lse;
  a.S = S;
  a.C = S / (2 * D);
  a.rows = (int)(2 * a.C);
  a.D = D;
  a.rank = rank;
  a.H = H;
  a.n_qt = (a.rows + BR - 1) / BR;
  a.items = B * H * a.n_qt;
  const float sc = scale > 0.0f ? scale : 1.0f / sqrtf((float)hd);
  a.scale_log2 = sc * 1.4426950408889634f;
  if (hd == 128) {
    hipLaunchKernelGGL(attn_fwd<128>, dim3(a.items), dim3(kThreads), 0, stream, a);
  } else {
    hipLaunchKernelGGL(attn_fwd<64>, dim3(a.items), dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace tsp
