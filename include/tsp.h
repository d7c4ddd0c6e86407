/*
 * tsp.h -- C ABI of the TSP rank-shard layer forward for AMD MI355X (gfx950).
 *
 * Method: "Folding Tensor and Sequence Parallelism for Memory-Efficient Transformer
 * Training & Inference" (summary pages on gist.science, paper 2604.26294), cited here
 * as [TSP §n] for section n of that summary. TSP folds tensor and sequence parallelism
 * onto one axis of D ranks: each rank holds a zigzag shard of the tokens and sees the
 * weights as D shards [TSP §2, unified sharding]. This library computes ONE rank's share
 * of a transformer layer on one GPU:
 *
 *   a1  zigzag map      rank r's local rows are chunks r and 2D-1-r of 2D equal chunks
 *   a2  QKV projection  [Q|K|V] = X_r W_qkv^T; own K/V rows land in the full-sequence
 *                       K/V buffers at their global positions       [TSP §2, attention]
 *   a3  attention       causal softmax attention of the rank's queries against the
 *                       full-sequence K/V (what the all-gather delivers) [TSP §2]
 *   a4  W_O projection  A = O W_o^T
 *   a5  gated MLP ring  for each of the D ffn shards j seen in ring order,
 *                       acc (+)= (silu(A W1_j^T) * (A W3_j^T)) W2_j^T, fp32, no
 *                       all-reduce                                 [TSP §2, gated MLP]
 *
 * Conventions shared by every entry point
 *   - Element types: "bf16" is IEEE bfloat16 (uint16 storage); "f32" is float.
 *   - Layouts are row-major and dense unless a leading dimension is given.
 *     Weights are [out_features, in_features], so every GEMM operand is contiguous
 *     along its reduction dimension. W_qkv rows are [W_q; W_k; W_v]; head h owns rows
 *     h*hd .. h*hd+hd-1 of each block. Feature f of a token vector belongs to head
 *     f / hd.
 *   - Local row order: a rank's 2C = S/D rows per sequence list chunk r (positions
 *     r*C .. r*C+C-1) then chunk 2D-1-r, both ascending; C = S/(2D).
 *   - Device pointers are allocated and owned by the caller, must be 16-byte aligned,
 *     and outputs must not alias inputs. The library never allocates or frees memory,
 *     never synchronises, and keeps no state between calls (the opt-in timing hook at
 *     the end of this header aside).
 *   - `stream` is a hipStream_t (NULL = the default stream). Kernels are enqueued on it
 *     and run asynchronously; errors raised while they run surface at the caller's
 *     next synchronisation of that stream.
 *   - Empty problems (B = 0, S = 0, or M = 0 for the MLP step) are valid: after the
 *     shape checks the call returns TSP_OK without reading any pointer or launching
 *     anything (torch hands out NULL data pointers for empty tensors).
 *   - Every entry point returns a tsp_status. Argument errors are decided on the host
 *     before any HIP call, so they are deterministic and safe without a GPU. The
 *     message of the last error on the calling thread is tsp_last_error().
 *   - Numerics: bf16 inputs, fp32 accumulation, fp32 softmax; intermediates stored as
 *     bf16 use round-to-nearest-even; the MLP accumulator is fp32.
 */
#ifndef TSP_H
#define TSP_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define TSP_API __attribute__((visibility("default")))
#else
#define TSP_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef void* tsp_stream_t; /* a hipStream_t */

typedef enum {
  TSP_OK = 0,
  TSP_ERR_NULL = 1,        /* a required pointer is NULL */
  TSP_ERR_SHAPE = 2,       /* S % (2D) != 0, d != H*hd, F % D != 0, a size <= 0 ... */
  TSP_ERR_RANK = 3,        /* rank outside [0, D) */
  TSP_ERR_UNSUPPORTED = 4, /* head_dim not in {64, 128}, size beyond int32 limits */
  TSP_ERR_WORKSPACE = 5,   /* workspace smaller than the size query returns */
  TSP_ERR_ALIGN = 6,       /* a device pointer is not 16-byte aligned */
  TSP_ERR_HIP = 7          /* a HIP launch failed (message has the HIP error string) */
} tsp_status;

/* Shape of one rank's layer.  [TSP §2] */
typedef struct {
  int32_t batch;     /* B: sequences per call */
  int32_t fold;      /* D: number of ranks on the TSP axis */
  int64_t seq_len;   /* S: tokens per sequence over all ranks; S % (2D) == 0 */
  int32_t rank;      /* r in [0, D) */
  int32_t d_model;   /* d = n_heads * head_dim */
  int32_t n_heads;   /* H */
  int32_t head_dim;  /* hd in {64, 128} */
  int32_t ffn;       /* F: SwiGLU hidden size over all shards; F % D == 0 */
  int32_t reserved;  /* must be 0 */
  int64_t w2_ld;     /* row stride (elements) of each W2 shard; 0 means F/D (a
                        contiguous [d, F/D] shard); F for views into a full W2 */
  float scale;       /* softmax scale; <= 0 means 1/sqrt(head_dim) */
} tsp_layer_desc;

/* Library version, (major << 16) | minor. */
TSP_API int tsp_version(void);

/* Message of the last non-OK status returned on the calling thread ("" if none). */
TSP_API const char* tsp_last_error(void);

/*
 * a1  Zigzag index map.  [TSP §2, zigzag partitioning]
 * Writes the global positions of rank `rank`'s idx_len = S/D local rows to HOST memory
 * idx_out: idx[i] = r*C + i for i < C, and (2D-1-r)*C + (i-C) for C <= i < 2C, with
 * C = S/(2D). Pairing chunk r with its mirror 2D-1-r gives every rank C*(S+1) causal
 * (query, key) pairs per sequence and head. Exact integer arithmetic.
 * Errors: TSP_ERR_NULL (idx_out, when S > 0), TSP_ERR_SHAPE (S < 0, D <= 0,
 * S % 2D != 0, idx_len != S/D), TSP_ERR_RANK.
 */
TSP_API int tsp_zigzag_index(int64_t S, int32_t D, int32_t rank, int64_t* idx_out, int64_t idx_len);

/*
 * a2  Packed QKV projection of a rank's token shard.  [TSP §2, attention layers: local
 * projections with the packed W_Q/W_K/W_V shards]
 *   x      bf16 [B, 2C, d]   the rank's tokens in local row order
 *   w_qkv  bf16 [3d, d]      [W_q; W_k; W_v]
 *   q_out  bf16 [B, 2C, d]   Q in local row order (= [B, 2C, H, hd]); may be NULL when
 *                            only K/V are wanted (filling the rows of a peer rank)
 *   k_full, v_full bf16 [B, S, d]  full-sequence K and V in natural position order; the
 *                            call writes ONLY rows b*S + idx[i] (the rank's own rows)
 * This is also how a test or benchmark on one GPU stands in for the K/V all-gather:
 * calling it for every peer rank fills the peers' rows.
 */
TSP_API int tsp_qkv_fwd(const void* x, const void* w_qkv, void* q_out, void* k_full, void* v_full,
                int32_t B, int64_t S, int32_t D, int32_t rank, int32_t n_heads,
                int32_t head_dim, tsp_stream_t stream);

/*
 * a3  Causal attention of a rank's queries against the full-sequence K/V.
 * [TSP §2, attention layers: all-gathered K/V, FlashAttention, zigzag balance]
 *   q       bf16 [B, 2C, H, hd]  local row order
 *   k_full, v_full bf16 [B, S, H, hd]  natural order
 *   o       bf16 [B, 2C, H, hd]  output, local row order
 *   lse     f32  [B, H, 2C] natural-log sum of exp of the scaled visible scores, or
 *           NULL
 * Row i at position p = idx[i] attends keys 0..p (diagonal included) with weights
 * softmax(scale * q.k). Only key rows < (2D-rank)*C are read: rows after the rank's
 * last position are never touched, so the caller need not fill them.
 */
TSP_API int tsp_attn_fwd(const void* q, const void* k_full, const void* v_full, void* o, float* lse,
                 int32_t B, int64_t S, int32_t D, int32_t rank, int32_t n_heads,
                 int32_t head_dim, float scale, tsp_stream_t stream);

/*
 * Chunked-arrival attention: the consumer side of overlapping the K/V all-gather with
 * attention. [TSP §2, attention layers: the all-gather of K/V feeds FlashAttention;
 * §3, implementation and overlap: transfers hidden behind compute]
 *
 * tsp_attn_fwd_range: the rank's queries against the keys at positions [key_lo, key_hi)
 * only, e.g. one zigzag chunk of the sequence as soon as the all-gather has delivered it.
 *   q        bf16 [B, 2C, H, hd]  local row order
 *   k_full, v_full bf16 [B, S, H, hd]  natural order; only rows [key_lo, min(key_hi,
 *            last position of the rank + 1)) are read
 *   o_part   f32 [B, 2C, H, hd]  softmax-weighted mean of V over the keys j of the range
 *            with j <= the query's position; 0 for a row that sees no such key
 *   lse_part f32 [B, H, 2C]  natural log of the sum of exp(scale q.k_j) over those keys;
 *            -inf for a row that sees none
 *   0 <= key_lo <= key_hi <= S; scale as for tsp_attn_fwd.
 *   accumulate != 0: (o_part, lse_part) hold a running accumulator (start: 0, -inf) and
 *            the range's result is merged into it by log-sum-exp (as tsp_attn_merge does)
 *            instead of overwriting it; rows that see no key of the range, and whole row
 *            tiles without one, are left untouched.
 *   o_out    bf16 [B, 2C, H, hd] or NULL: receives the resulting O of every row (with
 *            accumulate, after the last range it is the output of tsp_attn_fwd).
 * tsp_attn_merge: (o_acc, lse_acc) <- their log-sum-exp merge with (o_part, lse_part):
 *   lse = log(exp(lse_acc) + exp(lse_part)),
 *   o_acc = exp(lse_acc - lse) o_acc + exp(lse_part - lse) o_part.
 *   Same layouts as above; start from o_acc = 0, lse_acc = -inf (or from the first
 *   range's outputs). o_out (bf16 [B, 2C, H, hd], may be NULL) receives the merged O;
 *   after every key range of [0, S) has been merged, in any order, it is the output of
 *   tsp_attn_fwd. o_part and lse_part must not alias the accumulators.
 * Errors: TSP_ERR_NULL, TSP_ERR_SHAPE (key range, fold), TSP_ERR_RANK,
 * TSP_ERR_UNSUPPORTED (head_dim), TSP_ERR_ALIGN (16 bytes; lse 4 bytes).
 */
TSP_API int tsp_attn_fwd_range(const void* q, const void* k_full, const void* v_full, float* o_part,
                               float* lse_part, int32_t B, int64_t S, int32_t D, int32_t rank,
                               int32_t n_heads, int32_t head_dim, float scale, int64_t key_lo,
                               int64_t key_hi, int32_t accumulate, void* o_out, tsp_stream_t stream);
TSP_API int tsp_attn_merge(float* o_acc, float* lse_acc, const float* o_part, const float* lse_part,
                           void* o_out, int32_t B, int64_t S, int32_t D, int32_t n_heads,
                           int32_t head_dim, tsp_stream_t stream);

/*
 * Gradients of the rank's causal attention (backward of tsp_attn_fwd). The pages name
 * training but do not describe the backward pass: this is the derivative of the forward
 * definition. With P_ij = exp(scale q_i.k_j - lse_i) over the visible keys j <= p_i and
 * D_i = do_i . o_i:
 *   dv_j = sum_i P_ij do_i,  ds_ij = P_ij (do_i . v_j - D_i),
 *   dq_i = scale sum_j ds_ij k_j,  dk_j = scale sum_i ds_ij q_i.
 *   q, o, d_o  bf16 [B, 2C, H, hd]  the rank's queries, forward output, output gradient
 *   k_full, v_full  bf16 [B, S, H, hd]  as given to tsp_attn_fwd
 *   lse        f32 [B, H, 2C]  the forward's log-sum-exp (natural log)
 *   dq         f32 [B, 2C, H, hd]  overwritten
 *   dk_full, dv_full  f32 [B, S, H, hd]  overwritten with this rank's contributions at
 *              every key position (zero where no query of the rank looks); the gradient
 *              of the sequence's K and V is their sum over the D ranks
 *   ws         device workspace of tsp_attn_bwd_workspace_size bytes (the D_i)
 *   scale      <= 0 means 1/sqrt(head_dim), as in the forward
 * Errors: as tsp_attn_fwd; TSP_ERR_NULL for a missing pointer, TSP_ERR_WORKSPACE.
 */
TSP_API size_t tsp_attn_bwd_workspace_size(int32_t B, int64_t S, int32_t D, int32_t n_heads);
TSP_API int tsp_attn_bwd(const void* q, const void* k_full, const void* v_full, const void* o,
                         const float* lse, const void* d_o, float* dq, float* dk_full, float* dv_full,
                         int32_t B, int64_t S, int32_t D, int32_t rank, int32_t n_heads,
                         int32_t head_dim, float scale, void* ws, size_t ws_bytes,
                         tsp_stream_t stream);

/* Workspace bytes tsp_mlp_shard_accum needs for M rows and shard width Fs: the gated hidden,
 * bf16 [M, round_up(Fs, 64)]. */
TSP_API size_t tsp_mlp_workspace_size(int64_t M, int32_t Fs);

/*
 * a5  One ring step of the gated MLP.  [TSP §2, gated MLP layers: the W1/W2/W3 shards
 * rotate; each rank accumulates the partial outputs locally, no all-reduce]
 *   x     bf16 [M, d]        MLP input rows (the W_O output)
 *   w1_j  bf16 [Fs, d]       gate rows of shard j
 *   w3_j  bf16 [Fs, d]       up rows of shard j
 *   w2_j  bf16 [d, Fs] with row stride ld_w2 >= Fs (Fs for a received contiguous
 *         shard, F for a column block of a full W2)
 *   acc   f32 [M, d]         accumulate == 0: acc = partial;  != 0: acc += partial
 *   ws    device workspace of at least tsp_mlp_workspace_size(M, Fs) bytes (holds the
 *         bf16 gated hidden H = silu(x W1_j^T) * (x W3_j^T), [M, Fs])
 * Calls on one stream applied in ring order give a deterministic fp32 sum.
 */
TSP_API int tsp_mlp_shard_accum(const void* x, const void* w1_j, const void* w3_j, const void* w2_j,
                        int64_t ld_w2, float* acc, int64_t M, int32_t d, int32_t Fs,
                        int32_t accumulate, void* ws, size_t ws_bytes, tsp_stream_t stream);

/*
 * tsp_mlp_shard_accum without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). Same arguments, semantics and errors as tsp_mlp_shard_accum; the gated hidden
 * lives in a scratch array of tsp_mlp_noalloc_max_bytes() bytes (64 MiB) that the library
 * holds on every GPU it runs on until the process ends. The call allocates and frees
 * nothing itself; its first call on a device looks up that device's scratch address
 * (hipGetSymbolAddress), which is when the HIP runtime materialises the 64 MiB on that
 * device. A caller that must not see that happen, e.g. before a graph capture, makes one
 * call first (M = 0 does not count: it returns before any HIP call).
 *   Limit: tsp_mlp_workspace_size(M, Fs) <= tsp_mlp_noalloc_max_bytes(), e.g. at most
 *   23831 rows at the 7B shard width Fs = 1376; larger calls return TSP_ERR_WORKSPACE
 *   before any HIP call (the rows are independent, so a caller may split them).
 *   The stream must belong to the current device. Every call on one GPU shares that GPU's
 *   scratch: calls that overlap on one GPU (different streams, host threads or graphs
 *   replayed concurrently) race; calls ordered on one stream do not.
 */
TSP_API size_t tsp_mlp_noalloc_max_bytes(void);
TSP_API int tsp_mlp_shard_accum_noalloc(const void* x, const void* w1_j, const void* w3_j,
                                        const void* w2_j, int64_t ld_w2, float* acc, int64_t M,
                                        int32_t d, int32_t Fs, int32_t accumulate,
                                        tsp_stream_t stream);

/* Workspace bytes tsp_layer_fwd needs for `desc` (0 if desc is invalid): Q and O of the
 * rank, bf16 [B, 2C, d] each, the gated hidden of all D shards, bf16
 * [B*2C, D * round_up(F/D, 64)], and, when D is even and ceil(B*2C/256) * ceil(d/256) <= 128
 * (short sequences), an fp32 [B*2C, d] partial sum of the down projection, in that order,
 * each starting at a multiple of 256 bytes (Q at offset 0, O at round_up(B*2C*d*2, 256)).
 * After a call O holds the rank's attention output, bf16 [B, 2C, H, hd] in local row order. */
TSP_API size_t tsp_layer_workspace_size(const tsp_layer_desc* desc);

/*
 * a2 -> a5  One rank's whole layer forward.  [TSP §2]
 *   x_shard  bf16 [B, 2C, d]  the rank's tokens, local row order
 *   w_qkv    bf16 [3d, d]; w_o bf16 [d, d]
 *   w1, w3   arrays of D device pointers; w1[j], w3[j] bf16 [F/D, d] = ffn shard j
 *   w2       array of D device pointers; w2[j] bf16 [d, F/D] with row stride
 *            desc->w2_ld (0 = F/D)
 *   k_full, v_full  bf16 [B, S, H, hd], IN/OUT: on entry the rows of the other ranks
 *            hold what the K/V all-gather delivers; the call writes the rank's own rows
 *   attn_out bf16 [B, 2C, d]  A = O W_o^T (the MLP input)
 *   mlp_out  f32  [B, 2C, d]  sum over the D shards, taken in ring order
 *            j = (r - t) mod D for t = 0 .. D-1
 *   ws       device workspace, at least tsp_layer_workspace_size(desc) bytes
 * The pointer arrays w1/w3/w2 live in HOST memory. With every shard on the device, the
 * MLP runs as two launches (gated hidden of all shards; one down projection whose
 * reduction takes the shards in the ring order above, fp32 in registers) when D <= 32,
 * F/D and d are multiples of 8 and every shard is 16-byte aligned; otherwise as D
 * tsp_mlp_shard_accum-style steps. Both give the same sum order over the shards.
 */
TSP_API int tsp_layer_fwd(const tsp_layer_desc* desc, const void* x_shard, const void* w_qkv,
                  const void* w_o, const void* const* w1, const void* const* w3,
                  const void* const* w2, void* k_full, void* v_full, void* attn_out,
                  float* mlp_out, void* ws, size_t ws_bytes, tsp_stream_t stream);

/*
 * Weight-streamed layer: the rank holds two receive slots per weight kind instead of all
 * D shards, and runs the layer as the pages' loops over packed shards.  [TSP §2 attention
 * and MLP layers, §3 overlap of weight transfers with compute]
 *
 * Packed attention shard j (j = 0 .. D-1, heads [j H/D, (j+1) H/D), dg = d/D columns):
 *   bf16, 4 dg d elements: [3 dg, d] = W_q rows, W_k rows, W_v rows of the group
 *   (rows j dg .. (j+1) dg - 1 of each), then [d, dg] = W_o columns j dg .. (j+1) dg - 1,
 *   row-major.
 * Packed MLP shard j (Fs = F/D, Fp = round_up(Fs, 8)):
 *   bf16, (2 Fs + Fp) d elements: [Fs, d] W1 rows of shard j, [Fs, d] W3 rows, then
 *   [d, Fs] W2 columns of shard j with row stride Fp (the pad columns are never read).
 *
 * Per call, on the streams of `streams` (n_streams = 4: [0] the caller's stream, [1] the
 * second attention stream, [2] the W_O stream, [3] the copy stream; a NULL entry means
 * streams[0]. n_streams = 1: everything on streams[0], in one order, no overlap):
 *   copy stream   copies the shards into the slots (hipMemcpyDeviceToDeviceNoCU: the copy
 *                 engines), the one-GPU stand-in for receiving the broadcast. An attention
 *                 slot is refilled in two parts: its QKV rows once the QKV launch that read
 *                 them is done, its W_o columns once the W_O launch that read them is done;
 *                 an MLP slot likewise: its W1/W3 rows after the gate/up launch, its W2
 *                 after the down projection. The MLP shards 0 and 1 are copied right after
 *                 the attention shards 0, 1.
 *   attention     head groups t = j = 0 .. D-1 in pairs (t, t+1), one per attention slot;
 *                 pair p runs on streams[p % 2]: the QKV of each group (its Q columns, its
 *                 columns of the rank's K/V rows), then causal attention of the pair's
 *                 heads as one launch. With D odd the last group runs alone, every query
 *                 tile's keys split at S/2 into two work items merged by log-sum-exp into
 *                 O. Two pairs overlap.
 *   W_O stream    per pair, O_pair W_o,pair^T (both groups' partials summed in fp32
 *                 registers) added to an fp32 accumulator, pairs in order; the last step
 *                 stores the sum as bf16 attn_out.
 *   streams[0]    the MLP ring after the last W_O step, t = 0 .. D-1 on shard
 *                 j = (r - t) mod D, one per MLP slot: the gated hidden of each step, and
 *                 after steps t and t+1 (t even) one down projection that sums both shards
 *                 in fp32 registers (step t first) and adds the sum to mlp_out. With D odd
 *                 the last step's down projection runs alone; shard widths that are not a
 *                 multiple of 8 run every step alone.
 * mlp_out doubles as the fp32 accumulator of the W_O partials before the MLP overwrites
 * it. The other streams first wait for the work already queued on streams[0]; on return
 * streams[0] waits for everything the call queued, so outputs are ready in its order.
 * Requires H % D == 0 (whole heads per group).
 *   w_attn, w_mlp  arrays (HOST memory) of D device pointers to packed shards, 16-byte
 *                  aligned; the other arguments as in tsp_layer_fwd (desc->w2_ld is
 *                  ignored: the packed layout fixes the W2 stride).
 * The library keeps a few HIP events per host thread and device between calls (created
 * on first use, never freed); calls that overlap on the same streams from different
 * threads are not supported.
 * Workspace (tsp_layer_streamed_workspace_size; 0 if desc is invalid): Q and O bf16
 * [B 2C, d] each, the gated hidden of two shards bf16 [B 2C, 2 round_up(Fs, 64)] (one shard
 * if D = 1; the down projections run over pairs of steps), two attention slots, two MLP slots and,
 * when D is odd, the fp32 O and log-sum-exp of the last group's attention over keys
 * [0, S/2) and [S/2, S) (merged into O).
 * Errors: as tsp_layer_fwd; TSP_ERR_SHAPE if H % D != 0 or n_streams is not 1 or 4.
 */
TSP_API size_t tsp_layer_streamed_workspace_size(const tsp_layer_desc* desc);
TSP_API int tsp_layer_fwd_streamed(const tsp_layer_desc* desc, const void* x_shard,
                                   const void* const* w_attn, const void* const* w_mlp,
                                   void* k_full, void* v_full, void* attn_out, float* mlp_out,
                                   void* ws, size_t ws_bytes, const tsp_stream_t* streams,
                                   int32_t n_streams);

/*
 * Backward of one rank's layer, in two parts around the exchange of K/V gradients. The
 * pages name training but do not describe the backward pass: this is the derivative of the
 * forward (attention as tsp_attn_bwd; with A = O W_o^T, G = A W1^T, U = A W3^T,
 * Y = (silu(G) U) W2^T, and dX = dQ W_q + dK W_k + dV W_v).
 * Part 1, tsp_layer_bwd_attn_mlp: from the output gradient d_y (f32 [B 2C, d], the rank's
 * rows) and the forward's q, o (bf16 [B 2C, d]) and lse (f32 [B, H, 2C]):
 *   recomputes A and, per MLP shard in ring order j = (r - t) mod D, its gate pair; writes
 *   dw13[j] (f32 [2 F/D, d]: the rank's share of dW1 rows then dW3 rows of shard j),
 *   dw2[j] (f32 [d, F/D]), dw_o (f32 [d, d]), dq (f32 [B 2C, d]) and dk_full, dv_full
 *   (f32 [B, S, d]: the rank's contributions at every position).
 *   w_o bf16 [d, d]; w_mlp: D packed MLP shards as for tsp_layer_fwd_streamed (host array).
 * Between the parts, each rank's dk/dv contributions are summed at the rank that owns the
 * rows (a reduce-scatter; outside this library).
 * Part 2, tsp_layer_bwd_qkv: from dq and the summed dk_own, dv_own (f32 [B 2C, d], the
 *   rank's rows in local order), writes dx (f32 [B 2C, d]) and dw_qkv (f32 [3d, d], the
 *   rank's share). x_shard and w_qkv as in tsp_layer_fwd.
 * Weight gradients are the rank's shares: the model's gradient is their sum over ranks.
 * Intermediates are rounded to bf16 before each GEMM (fp32 accumulation); outputs are f32.
 * Workspace: tsp_layer_bwd_workspace_size(desc) bytes, for either part.
 * Errors: as tsp_layer_fwd.
 */
TSP_API size_t tsp_layer_bwd_workspace_size(const tsp_layer_desc* desc);
TSP_API int tsp_layer_bwd_attn_mlp(const tsp_layer_desc* desc, const void* q, const void* o,
                                   const float* lse, const void* k_full, const void* v_full,
                                   const void* w_o, const void* const* w_mlp, const float* d_y,
                                   float* dq, float* dk_full, float* dv_full, float* dw_o,
                                   float* const* dw13, float* const* dw2, void* ws,
                                   size_t ws_bytes, tsp_stream_t stream);
TSP_API int tsp_layer_bwd_qkv(const tsp_layer_desc* desc, const void* x_shard, const void* w_qkv,
                              const float* dq, const float* dk_own, const float* dv_own,
                              float* dx, float* dw_qkv, void* ws, size_t ws_bytes,
                              tsp_stream_t stream);

/*
 * Measurement hook (outside the method): phase timing of tsp_layer_fwd with HIP events
 * recorded on the call's own stream, between its launches.
 *   tsp_timing_start(max_calls)  creates (4 + 1) * max_calls events and arms the hook:
 *       the next max_calls tsp_layer_fwd calls record an event before the QKV launch and
 *       after the QKV, attention, W_O and MLP launches. max_calls = 0 disarms and
 *       destroys the events. These events are the only objects the library creates.
 *   tsp_timing_read(ms, max_calls, n_calls)  waits for the last recorded event, writes
 *       ms[4 i + p] = milliseconds of phase p (0 QKV, 1 attention, 2 W_O, 3 MLP) of
 *       recorded call i for i < *n_calls = min(calls recorded, max_calls), then disarms.
 * Process-wide state behind a mutex; arm it only around calls that do not overlap.
 * Errors: TSP_ERR_SHAPE (max_calls < 0), TSP_ERR_NULL, TSP_ERR_HIP.
 */
TSP_API int tsp_timing_start(int32_t max_calls);
TSP_API int tsp_timing_read(float* ms, int32_t max_calls, int32_t* n_calls);

#ifdef __cplusplus
}
#endif

#endif /* TSP_H */
