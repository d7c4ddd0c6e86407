// tsp_internal.h -- host-side launchers of the gfx950 kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tsp {

// QKV projection with the zigzag K/V scatter (step a2).
//   x [M, d] (M = B * 2C), w_qkv [3d, d]; q_out [M, d] or nullptr;
//   k_full, v_full [B, S, d]: rows b*S + zigzag_pos(i) receive the rank's K and V.
hipError_t launch_qkv(const void* x, const void* w_qkv, void* q_out, void* k_full, void* v_full,
                      int B, int64_t S, int D, int rank, int d, hipStream_t stream);

// QKV projection of head group `group` of `groups` (its packed shard w_qkv_g: [3 d/groups, d],
// the group's W_q, W_k and W_v rows): Q columns [group*dg, (group+1)*dg) of q_out, and the
// same columns of the rank's K/V rows.
hipError_t launch_qkv_group(const void* x, const void* w_qkv_g, int group, int groups, void* q_out, void* k_full,
                            void* v_full, int B, int64_t S, int D, int rank, int d, hipStream_t stream);

// Partial W_O of head group `group`: acc[M, d] (=, +=) O[:, group cols] w_o_g^T with w_o_g
// [d, d/groups] (the group's W_o columns); at the last step (step == steps - 1) the sum is
// stored as bf16 to out instead.
hipError_t launch_wo_group(const void* o, const void* w_o_g, int group, int groups, float* acc, void* out, int M, int d,
                           int step, int steps, hipStream_t stream);
// The same for head groups `group` and `group + 1` in one launch (their W_o columns w_o_a and
// w_o_b held apart), the two products summed in fp32 registers: acc (= when first, else +=);
// when last, out = bf16(acc + the pair's partial) instead (acc not written).
hipError_t launch_wo_pair(const void* o, const void* w_o_a, const void* w_o_b, int group, int groups, float* acc,
                          void* out, int M, int d, int first, int last, hipStream_t stream);

// Plain projection C[M, N] = A[M, K] W[N, K]^T, bf16 out (step a4, W_O).
hipError_t launch_proj_bf16(const void* a, int64_t lda, const void* w, int64_t ldw, void* c,
                            int64_t ldc, int M, int N, int K, hipStream_t stream);

// Gated hidden H[M, Fs] = silu(X W1^T) * (X W3^T), bf16 out (step a5, first half).
hipError_t launch_gate_up(const void* x, int64_t ldx, const void* w1, const void* w3, int64_t ldw,
                          void* h, int64_t ldh, int M, int Fs, int K, hipStream_t stream);

// Down projection into the fp32 accumulator: acc[M, N] (=, +=) H[M, K] W2[N, K]^T
// (step a5, second half).
hipError_t launch_down_acc(const void* h, int64_t ldh, const void* w2, int64_t ldw2, float* acc,
                           int64_t ldacc, int M, int N, int K, int accumulate, hipStream_t stream);

// The D-shard MLP ring of one rank in two launches (all shards resident on the device).
// mlp_ring_fusable: whether the shard operands suit them (at most 32 shards, 16-byte chunks,
// 32-bit row offsets); otherwise the caller loops over launch_gate_up / launch_down_acc.
bool mlp_ring_fusable(const void* const* w1, const void* const* w3, const void* const* w2, int64_t ldw2, int D,
                      int M, int d, int Fs, int64_t ldh);
// H[:, j*ldseg + n] = silu(X W1_j^T) * (X W3_j^T) for every shard j and n < Fs.
hipError_t launch_gate_up_ring(const void* x, const void* const* w1, const void* const* w3, int D, void* h,
                               int64_t ldh, int64_t ldseg, int M, int Fs, int d, hipStream_t stream);
// out[M, N] (+)= sum over ring steps t = 0..D-1 (shard j = (rank - t) mod D, in that order)
// of H[:, j*ldseg : j*ldseg + Fs] W2_j^T, the fp32 sum held in registers and stored (or added,
// accumulate != 0) once. part: NULL, or fp32 scratch [M, ldout] the call may use when the
// output tiles fill at most half the CUs: the first and second halves of the ring then run as
// separate work items (each summing its shards in ring order), the second into part, and
// out = (out +) first + second.
hipError_t launch_down_ring(const void* h, int64_t ldh, int64_t ldseg, const void* const* w2, int64_t ldw2, int D,
                            int rank, float* out, int64_t ldout, int accumulate, int M, int N, int Fs, float* part,
                            hipStream_t stream);

// Causal attention of the rank's queries against full-sequence K/V (step a3).
hipError_t launch_attn(const void* q, const void* k_full, const void* v_full, void* o, float* lse,
                       int B, int64_t S, int D, int rank, int H, int hd, float scale,
                       hipStream_t stream);

// Causal attention restricted to key positions [key_lo, key_hi): fp32 O (normalised over
// those keys) [B, 2C, H, hd] and lse [B, H, 2C]; rows with no such key get 0 and -inf.
// accumulate != 0: log-sum-exp merge into (o32, lse) instead (rows without such keys
// untouched); o_out (bf16, may be null) receives the resulting O of every row.
// Causal attention of heads [h0, h0 + h_run) as a split launch: two items per query tile,
// keys [0, split) and [split, S), each writing fp32 O (normalised over its keys) and the
// log-sum-exp; half 0 at o32 / lse, half 1 at o32 + B rows h_run hd / lse + B h_run rows,
// in the group's [B, rows, h_run, hd] / [B, h_run, rows] layout. Every item covers at most
// max(split, S - split) keys; launch_attn_merge_halves then writes bf16 O.
// Causal attention of heads [h0, h0 + h_run) only, bf16 O into the full-width o (the other
// heads' columns untouched).
hipError_t launch_attn_heads(const void* q, const void* k_full, const void* v_full, void* o, int B, int64_t S, int D,
                             int rank, int H, int hd, float scale, int h0, int h_run, hipStream_t stream);
hipError_t launch_attn_split(const void* q, const void* k_full, const void* v_full, float* o32, float* lse, int B,
                             int64_t S, int D, int rank, int H, int hd, float scale, int h0, int h_run, int split,
                             hipStream_t stream);
hipError_t launch_attn_merge_halves(const float* o32, const float* lse, void* o_out, int B, int rows, int H, int hd,
                                    int h0, int h_run, hipStream_t stream);
// Causal attention of all heads for launches of at most one tile per CU, in one launch: the
// earlier zigzag chunk's tiles write bf16 O directly; each later-chunk tile runs as two key
// halves split at attn_two_part_split(...) into fp32 partials of the later chunk's rows
// (`part`, 16-byte aligned, attn_two_part_bytes(...) bytes), then merged into bf16 O by a
// second launch. attn_two_part_split
// returns 0 where this does not apply (launch_attn serves those shapes).
int attn_two_part_split(int B, int64_t S, int D, int rank, int H);
size_t attn_two_part_bytes(int B, int64_t S, int D, int H, int hd);
hipError_t launch_attn_two_part(const void* q, const void* k_full, const void* v_full, void* o, void* part, int B,
                                int64_t S, int D, int rank, int H, int hd, float scale, hipStream_t stream);

// Gradients of the rank's causal attention (two launches: dq and the row sums D_i, then
// dk/dv of every key). lse [B, H, rows] natural log, from the forward; dsum [B, H, rows]
// fp32 scratch. dq [B, rows, H, hd], dk_full / dv_full [B, S, H, hd] fp32, overwritten.
hipError_t launch_attn_bwd(const void* q, const void* k_full, const void* v_full, const void* o, const float* lse,
                           const void* d_o, float* dq, float* dk_full, float* dv_full, float* dsum, int B, int64_t S,
                           int D, int rank, int H, int hd, float scale, hipStream_t stream);

// Memory-bound helpers of the layer backward (row-major, leading dimensions in elements).
// dst[c][r] = src[r][c] for an R x C source; fp32 sources are rounded to bf16.
hipError_t launch_transpose_bf16(const void* src, int64_t lds, void* dst, int64_t ldd, int R, int C,
                                 hipStream_t stream);
hipError_t launch_transpose_f32_bf16(const float* src, int64_t lds, void* dst, int64_t ldd, int R, int C,
                                     hipStream_t stream);
hipError_t launch_convert_f32_bf16(const float* src, int64_t lds, void* dst, int64_t ldd, int R, int C,
                                   hipStream_t stream);
// h = silu(g) u and dgu = [dh u silu'(g) | dh silu(g)] from gu = [g | u] and dh.
hipError_t launch_swiglu_bwd(const void* gu, int64_t ldgu, const float* dh, int64_t lddh, void* h, int64_t ldh,
                             void* dgu, int64_t lddgu, int M, int Fs, hipStream_t stream);

hipError_t launch_attn_range(const void* q, const void* k_full, const void* v_full, float* o32, float* lse, int B,
                             int64_t S, int D, int rank, int H, int hd, float scale, int64_t key_lo, int64_t key_hi,
                             int accumulate, void* o_out, hipStream_t stream);

// o_acc, lse_acc <- log-sum-exp merge with (o_part, lse_part); o_out (bf16, may be null)
// receives the merged O.
hipError_t launch_attn_merge(float* o_acc, float* lse_acc, const float* o_part, const float* lse_part, void* o_out,
                             int B, int rows, int H, int hd, hipStream_t stream);

}  // namespace tsp
