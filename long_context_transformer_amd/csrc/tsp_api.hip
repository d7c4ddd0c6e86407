// tsp_api.hip -- the C ABI declared in include/tsp.h: argument checks on the host,
// workspace carving, and the launch sequence of one TSP rank's layer on the caller's
// stream(s). The library allocates no device memory. State kept between calls: the
// opt-in phase timing hook (tsp_timing_start / tsp_timing_read) used by measurements,
// and the per-thread, per-device HIP events of the weight-streamed layer.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <map>
#include <mutex>
#include <vector>

#include "tsp.h"
#include "tsp_device.h"
#include "tsp_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return TSP_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(TSP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return TSP_OK;
}

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

constexpr size_t kAlign = 256;
size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
constexpr int64_t kMaxI32 = 2147483647;

// Checks shared by every entry point that knows (B, S, D, rank): S % 2D == 0, rank
// in range, and local-row counts and key positions that fit the kernels' 32-bit indices.
// B = 0 or S = 0 is a valid empty problem (callers return before touching any pointer).
int check_fold(int64_t B, int64_t S, int64_t D, int64_t rank) {
  if (B < 0) return fail(TSP_ERR_SHAPE, "batch must be >= 0 (got %lld)", (long long)B);
  if (D < 1) return fail(TSP_ERR_SHAPE, "fold D must be >= 1 (got %lld)", (long long)D);
  if (S < 0 || S % (2 * D) != 0)
    return fail(TSP_ERR_SHAPE, "seq_len S=%lld must be a non-negative multiple of 2D=%lld", (long long)S,
                (long long)(2 * D));
  if (rank < 0 || rank >= D) return fail(TSP_ERR_RANK, "rank %lld outside [0, %lld)", (long long)rank, (long long)D);
  if (B * (S / D) > kMaxI32 / 4) return fail(TSP_ERR_UNSUPPORTED, "B*S/D too large for 32-bit row indices");
  if (S > kMaxI32 / 2) return fail(TSP_ERR_UNSUPPORTED, "S too large for 32-bit key positions");
  return TSP_OK;
}

int check_heads(int64_t H, int64_t hd) {
  if (H < 1) return fail(TSP_ERR_SHAPE, "n_heads must be >= 1 (got %lld)", (long long)H);
  if (hd != 64 && hd != 128) return fail(TSP_ERR_UNSUPPORTED, "head_dim %lld not in {64, 128}", (long long)hd);
  if (H * hd > 65536) return fail(TSP_ERR_UNSUPPORTED, "d_model = H*hd = %lld above 65536", (long long)(H * hd));
  return TSP_OK;
}

// Phase timing hook: events of armed tsp_layer_fwd calls, kPhases + 1 per call.
constexpr int kPhases = 4;  // QKV, attention, W_O, MLP
std::mutex g_tm_mu;
std::vector<hipEvent_t> g_tm_ev;
int g_tm_cap = 0, g_tm_used = 0;

void timing_destroy() {
  for (hipEvent_t e : g_tm_ev) (void)hipEventDestroy(e);
  g_tm_ev.clear();
  g_tm_cap = g_tm_used = 0;
}

// Events for the next armed call (kPhases + 1 of them), or nullptr when not armed.
hipEvent_t* timing_slot() {
  std::lock_guard<std::mutex> lk(g_tm_mu);
  if (g_tm_used >= g_tm_cap) return nullptr;
  return &g_tm_ev[(size_t)(g_tm_used++) * (kPhases + 1)];
}

// Row stride (elements) of one shard's block of the gated hidden: F/D rounded up to 64, so
// each row and each shard block starts on a 128-byte line and every 64-wide k stage of the
// down projection reads whole lines (with F/D = 1376, an odd multiple of 32, every other
// block would start mid-line; 0.1 ms of the 7B S=128K MLP).
int64_t hidden_ld(int64_t Fs) { return (int64_t)round_up((size_t)Fs, 64); }

size_t mlp_ws_bytes(int64_t M, int64_t Fs) { return round_up((size_t)M * (size_t)hidden_ld(Fs) * 2, kAlign); }

// Scratch of tsp_mlp_shard_accum_noalloc: the gated hidden of one ring step. A device global,
// so every GPU the library runs on holds its own copy from the module's load until the
// process ends. In host code `scratch` names a host-side stand-in, not device memory: the
// kernels get this device's address of it, taken once per device by hipGetSymbolAddress.
constexpr size_t kScratchBytes = (size_t)64 << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch (looked up on the first call per device).
int scratch_address(void** out) {
  int dev = 0;
  if (int rc = hip_status(hipGetDevice(&dev), "hipGetDevice")) return rc;
  if (dev < 0 || dev >= kMaxDevices) return fail(TSP_ERR_UNSUPPORTED, "device %d beyond the %d supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (int rc = hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress")) return rc;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return TSP_OK;
}

// Shape and pointer checks of one MLP ring step (everything but the workspace).
int check_mlp_step(const void* x, const void* w1_j, const void* w3_j, const void* w2_j, int64_t ld_w2, const float* acc,
                   int64_t M, int32_t d, int32_t Fs) {
  if (M < 0 || d < 1 || Fs < 1) return fail(TSP_ERR_SHAPE, "M must be >= 0, d and Fs >= 1");
  if (M > kMaxI32 / 4) return fail(TSP_ERR_UNSUPPORTED, "M too large for 32-bit row indices");
  if (ld_w2 < Fs) return fail(TSP_ERR_SHAPE, "ld_w2 %lld < Fs %d", (long long)ld_w2, Fs);
  if (M == 0) return TSP_OK;
  if (!x || !w1_j || !w3_j || !w2_j || !acc) return fail(TSP_ERR_NULL, "x, w1_j, w3_j, w2_j and acc must be non-NULL");
  if (misaligned(x) || misaligned(w1_j) || misaligned(w3_j) || misaligned(w2_j) || misaligned(acc))
    return fail(TSP_ERR_ALIGN, "device pointers must be 16-byte aligned");
  return TSP_OK;
}

// The two launches of one ring step: gated hidden into h, then its down projection into acc.
int launch_mlp_step(const void* x, const void* w1_j, const void* w3_j, const void* w2_j, int64_t ld_w2, float* acc,
                    int64_t M, int32_t d, int32_t Fs, int32_t accumulate, void* h, hipStream_t s) {
  const int64_t ldh = hidden_ld(Fs);
  if (int rc = hip_status(tsp::launch_gate_up(x, d, w1_j, w3_j, d, h, ldh, (int)M, Fs, d, s), "gate/up launch"))
    return rc;
  if (int rc = hip_status(tsp::launch_down_acc(h, ldh, w2_j, ld_w2, acc, d, (int)M, d, Fs, accumulate ? 1 : 0, s),
                          "down projection launch"))
    return rc;
  return ok();
}

}  // namespace

extern "C" {

int tsp_version(void) { return (1 << 16) | 0; }

int tsp_timing_start(int32_t max_calls) {
  std::lock_guard<std::mutex> lk(g_tm_mu);
  timing_destroy();
  if (max_calls < 0) return fail(TSP_ERR_SHAPE, "max_calls must be >= 0");
  if (max_calls == 0) return ok();
  g_tm_ev.resize((size_t)max_calls * (kPhases + 1));
  for (size_t i = 0; i < g_tm_ev.size(); ++i) {
    hipError_t e = hipEventCreate(&g_tm_ev[i]);
    if (e != hipSuccess) {
      g_tm_ev.resize(i);
      timing_destroy();
      return hip_status(e, "hipEventCreate");
    }
  }
  g_tm_cap = max_calls;
  return ok();
}

int tsp_timing_read(float* ms, int32_t max_calls, int32_t* n_calls) {
  if (!n_calls || (max_calls > 0 && !ms)) return fail(TSP_ERR_NULL, "ms and n_calls must be non-NULL");
  std::lock_guard<std::mutex> lk(g_tm_mu);
  const int n = g_tm_used < max_calls ? g_tm_used : (max_calls > 0 ? max_calls : 0);
  *n_calls = n;
  int rc = TSP_OK;
  if (g_tm_used > 0) {
    rc = hip_status(hipEventSynchronize(g_tm_ev[(size_t)g_tm_used * (kPhases + 1) - 1]), "hipEventSynchronize");
  }
  for (int i = 0; i < n && rc == TSP_OK; ++i)
    for (int p = 0; p < kPhases && rc == TSP_OK; ++p)
      rc = hip_status(hipEventElapsedTime(&ms[i * kPhases + p], g_tm_ev[(size_t)i * (kPhases + 1) + p],
                                          g_tm_ev[(size_t)i * (kPhases + 1) + p + 1]),
                      "hipEventElapsedTime");
  timing_destroy();
  return rc == TSP_OK ? ok() : rc;
}

const char* tsp_last_error(void) { return g_err; }

int tsp_zigzag_index(int64_t S, int32_t D, int32_t rank, int64_t* idx_out, int64_t idx_len) {
  if (int rc = check_fold(1, S, D, rank)) return rc;
  if (idx_len != S / D)
    return fail(TSP_ERR_SHAPE, "idx_len %lld != S/D = %lld", (long long)idx_len, (long long)(S / D));
  if (S == 0) return ok();
  if (!idx_out) return fail(TSP_ERR_NULL, "idx_out is NULL");
  const int64_t C = S / (2 * (int64_t)D);
  for (int64_t i = 0; i < 2 * C; ++i) idx_out[i] = tsp::zigzag_pos(i, C, rank, D);
  return ok();
}

int tsp_qkv_fwd(const void* x, const void* w_qkv, void* q_out, void* k_full, void* v_full, int32_t B, int64_t S,
                int32_t D, int32_t rank, int32_t n_heads, int32_t head_dim, tsp_stream_t stream) {
  if (int rc = check_fold(B, S, D, rank)) return rc;
  if (int rc = check_heads(n_heads, head_dim)) return rc;
  if (B == 0 || S == 0) return ok();
  if (!x || !w_qkv || !k_full || !v_full) return fail(TSP_ERR_NULL, "x, w_qkv, k_full and v_full must be non-NULL");
  if (misaligned(x) || misaligned(w_qkv) || misaligned(k_full) || misaligned(v_full) || misaligned(q_out))
    return fail(TSP_ERR_ALIGN, "device pointers must be 16-byte aligned");
  const int d = n_heads * head_dim;
  if (int rc = hip_status(tsp::launch_qkv(x, w_qkv, q_out, k_full, v_full, B, S, D, rank, d,
                                          static_cast<hipStream_t>(stream)),
                          "qkv projection launch"))
    return rc;
  return ok();
}

int tsp_attn_fwd(const void* q, const void* k_full, const void* v_full, void* o, float* lse, int32_t B, int64_t S,
                 int32_t D, int32_t rank, int32_t n_heads, int32_t head_dim, float scale, tsp_stream_t stream) {
  if (int rc = check_fold(B, S, D, rank)) return rc;
  if (int rc = check_heads(n_heads, head_dim)) return rc;
  if (!(scale == scale) || isinf(scale)) return fail(TSP_ERR_SHAPE, "scale must be finite");
  if (B == 0 || S == 0) return ok();
  if (!q || !k_full || !v_full || !o) return fail(TSP_ERR_NULL, "q, k_full, v_full and o must be non-NULL");
  if (misaligned(q) || misaligned(k_full) || misaligned(v_full) || misaligned(o) ||
      (reinterpret_cast<uintptr_t>(lse) & 3u))
    return fail(TSP_ERR_ALIGN, "q/k/v/o must be 16-byte aligned and lse 4-byte aligned");
  if (int rc = hip_status(tsp::launch_attn(q, k_full, v_full, o, lse, B, S, D, rank, n_heads, head_dim, scale,
                                           static_cast<hipStream_t>(stream)),
                          "attention launch"))
    return rc;
  return ok();
}

size_t tsp_attn_bwd_workspace_size(int32_t B, int64_t S, int32_t D, int32_t n_heads) {
  if (B < 0 || D < 1 || S < 0 || n_heads < 1 || S % (2 * (int64_t)D) != 0) return 0;
  return round_up((size_t)B * (size_t)n_heads * (size_t)(S / D) * 4, kAlign);
}

int tsp_attn_bwd(const void* q, const void* k_full, const void* v_full, const void* o, const float* lse,
                 const void* d_o, float* dq, float* dk_full, float* dv_full, int32_t B, int64_t S, int32_t D,
                 int32_t rank, int32_t n_heads, int32_t head_dim, float scale, void* ws, size_t ws_bytes,
                 tsp_stream_t stream) {
  if (int rc = check_fold(B, S, D, rank)) return rc;
  if (int rc = check_heads(n_heads, head_dim)) return rc;
  if (!(scale == scale) || isinf(scale)) return fail(TSP_ERR_SHAPE, "scale must be finite");
  if (B == 0 || S == 0) return ok();
  if (!q || !k_full || !v_full || !o || !lse || !d_o || !dq || !dk_full || !dv_full || !ws)
    return fail(TSP_ERR_NULL, "a required pointer is NULL");
  if (misaligned(q) || misaligned(k_full) || misaligned(v_full) || misaligned(o) || misaligned(d_o) ||
      misaligned(dq) || misaligned(dk_full) || misaligned(dv_full) || misaligned(ws) ||
      (reinterpret_cast<uintptr_t>(lse) & 3u))
    return fail(TSP_ERR_ALIGN, "tensors must be 16-byte aligned and lse 4-byte aligned");
  const size_t need = tsp_attn_bwd_workspace_size(B, S, D, n_heads);
  if (ws_bytes < need) return fail(TSP_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
  if (S > kMaxI32 / 2) return fail(TSP_ERR_UNSUPPORTED, "S too large for 32-bit key indices");
  return hip_status(tsp::launch_attn_bwd(q, k_full, v_full, o, lse, d_o, dq, dk_full, dv_full, static_cast<float*>(ws),
                                         B, S, D, rank, n_heads, head_dim, scale, static_cast<hipStream_t>(stream)),
                    "attention backward launch");
}

int tsp_attn_fwd_range(const void* q, const void* k_full, const void* v_full, float* o_part, float* lse_part,
                       int32_t B, int64_t S, int32_t D, int32_t rank, int32_t n_heads, int32_t head_dim, float scale,
                       int64_t key_lo, int64_t key_hi, int32_t accumulate, void* o_out, tsp_stream_t stream) {
  if (int rc = check_fold(B, S, D, rank)) return rc;
  if (int rc = check_heads(n_heads, head_dim)) return rc;
  if (!(scale == scale) || isinf(scale)) return fail(TSP_ERR_SHAPE, "scale must be finite");
  if (key_lo < 0 || key_lo > key_hi || key_hi > S)
    return fail(TSP_ERR_SHAPE, "key range [%lld, %lld) not within [0, S=%lld]", (long long)key_lo,
                (long long)key_hi, (long long)S);
  if (B == 0 || S == 0) return ok();
  if (!q || !k_full || !v_full || !o_part || !lse_part)
    return fail(TSP_ERR_NULL, "q, k_full, v_full, o_part and lse_part must be non-NULL");
  if (misaligned(q) || misaligned(k_full) || misaligned(v_full) || misaligned(o_part) || misaligned(o_out) ||
      (reinterpret_cast<uintptr_t>(lse_part) & 3u))
    return fail(TSP_ERR_ALIGN, "q/k/v/o_part/o_out must be 16-byte aligned and lse_part 4-byte aligned");
  return hip_status(tsp::launch_attn_range(q, k_full, v_full, o_part, lse_part, B, S, D, rank, n_heads, head_dim,
                                           scale, key_lo, key_hi, accumulate ? 1 : 0, o_out,
                                           static_cast<hipStream_t>(stream)),
                    "range attention launch") == TSP_OK
             ? ok()
             : TSP_ERR_HIP;
}

int tsp_attn_merge(float* o_acc, float* lse_acc, const float* o_part, const float* lse_part, void* o_out, int32_t B,
                   int64_t S, int32_t D, int32_t n_heads, int32_t head_dim, tsp_stream_t stream) {
  if (int rc = check_fold(B, S, D, 0)) return rc;
  if (int rc = check_heads(n_heads, head_dim)) return rc;
  if (B == 0 || S == 0) return ok();
  if (!o_acc || !lse_acc || !o_part || !lse_part)
    return fail(TSP_ERR_NULL, "o_acc, lse_acc, o_part and lse_part must be non-NULL");
  if (misaligned(o_acc) || misaligned(o_part) || misaligned(o_out) || (reinterpret_cast<uintptr_t>(lse_acc) & 3u) ||
      (reinterpret_cast<uintptr_t>(lse_part) & 3u))
    return fail(TSP_ERR_ALIGN, "o_acc/o_part/o_out must be 16-byte aligned and lse 4-byte aligned");
  if (o_acc == o_part || lse_acc == lse_part) return fail(TSP_ERR_SHAPE, "the partial must not alias the accumulator");
  return hip_status(tsp::launch_attn_merge(o_acc, lse_acc, o_part, lse_part, o_out, B, (int)(S / D), n_heads,
                                           head_dim, static_cast<hipStream_t>(stream)),
                    "merge launch") == TSP_OK
             ? ok()
             : TSP_ERR_HIP;
}

size_t tsp_mlp_workspace_size(int64_t M, int32_t Fs) {
  if (M < 0 || Fs < 1) return 0;
  return mlp_ws_bytes(M, Fs);
}

int tsp_mlp_shard_accum(const void* x, const void* w1_j, const void* w3_j, const void* w2_j, int64_t ld_w2, float* acc,
                        int64_t M, int32_t d, int32_t Fs, int32_t accumulate, void* ws, size_t ws_bytes,
                        tsp_stream_t stream) {
  if (int rc = check_mlp_step(x, w1_j, w3_j, w2_j, ld_w2, acc, M, d, Fs)) return rc;
  if (M == 0) return ok();
  if (!ws) return fail(TSP_ERR_NULL, "ws must be non-NULL");
  if (misaligned(ws)) return fail(TSP_ERR_ALIGN, "device pointers must be 16-byte aligned");
  if (ws_bytes < mlp_ws_bytes(M, Fs))
    return fail(TSP_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, mlp_ws_bytes(M, Fs));
  return launch_mlp_step(x, w1_j, w3_j, w2_j, ld_w2, acc, M, d, Fs, accumulate, ws, static_cast<hipStream_t>(stream));
}

size_t tsp_mlp_noalloc_max_bytes(void) { return kScratchBytes; }

int tsp_mlp_shard_accum_noalloc(const void* x, const void* w1_j, const void* w3_j, const void* w2_j, int64_t ld_w2,
                                float* acc, int64_t M, int32_t d, int32_t Fs, int32_t accumulate,
                                tsp_stream_t stream) {
  if (int rc = check_mlp_step(x, w1_j, w3_j, w2_j, ld_w2, acc, M, d, Fs)) return rc;
  if (M == 0) return ok();
  const size_t need = mlp_ws_bytes(M, Fs);
  if (need > kScratchBytes)
    return fail(TSP_ERR_WORKSPACE,
                "M=%lld rows of width Fs=%d need %zu bytes of scratch, above the %zu-byte maximum of the "
                "allocation-free entry point (use tsp_mlp_shard_accum with a workspace, or fewer rows per call)",
                (long long)M, Fs, need, kScratchBytes);
  void* h = nullptr;
  if (int rc = scratch_address(&h)) return rc;
  // Nothing in the scratch needs to start at zero: the gate/up launch writes every element of
  // the [M, Fs] hidden before the down projection reads it.
  return launch_mlp_step(x, w1_j, w3_j, w2_j, ld_w2, acc, M, d, Fs, accumulate, h, static_cast<hipStream_t>(stream));
}

namespace {

int check_desc(const tsp_layer_desc* desc) {
  if (!desc) return fail(TSP_ERR_NULL, "desc is NULL");
  if (desc->reserved != 0) return fail(TSP_ERR_SHAPE, "desc->reserved must be 0");
  if (int rc = check_fold(desc->batch, desc->seq_len, desc->fold, desc->rank)) return rc;
  if (int rc = check_heads(desc->n_heads, desc->head_dim)) return rc;
  if (desc->d_model != desc->n_heads * desc->head_dim)
    return fail(TSP_ERR_SHAPE, "d_model %d != n_heads*head_dim = %d", desc->d_model, desc->n_heads * desc->head_dim);
  if (desc->ffn < 1 || desc->ffn % desc->fold != 0)
    return fail(TSP_ERR_SHAPE, "ffn %d must be a positive multiple of D=%d", desc->ffn, desc->fold);
  const int64_t Fs = desc->ffn / desc->fold;
  if (desc->w2_ld != 0 && desc->w2_ld < Fs)
    return fail(TSP_ERR_SHAPE, "w2_ld %lld < F/D = %lld", (long long)desc->w2_ld, (long long)Fs);
  if (!(desc->scale == desc->scale) || isinf(desc->scale)) return fail(TSP_ERR_SHAPE, "scale must be finite");
  return TSP_OK;
}

struct LayerCarve {
  size_t q_off, o_off, h_off, p_off, total;  // p_off: 0 when there is no partial-sum region
};

// Whether the layer workspace carries an fp32 [M, d] partial sum for the down projection:
// when its 256 x 256 output tiles would fill at most half of the 256 CUs (7B S=16K: 128
// tiles), each tile runs as two work items over the two halves of the D-shard ring, and the
// second half's sum lands there before the two are added.
bool down_split_region(size_t M, size_t d, int D) {
  return D % 2 == 0 && ((M + 255) / 256) * ((d + 255) / 256) <= 128;
}

LayerCarve carve(const tsp_layer_desc* d) {
  const size_t M = (size_t)d->batch * (size_t)(d->seq_len / d->fold);
  const size_t act = round_up(M * (size_t)d->d_model * 2, kAlign);
  LayerCarve c;
  c.q_off = 0;
  c.o_off = act;
  c.h_off = 2 * act;
  // Gated hidden of all D shards: [M, D * hidden_ld(F/D)] bf16.
  c.total = 2 * act + round_up(M * (size_t)d->fold * (size_t)hidden_ld(d->ffn / d->fold) * 2, kAlign);
  c.p_off = 0;
  if (down_split_region(M, (size_t)d->d_model, d->fold)) {
    c.p_off = c.total;
    c.total += round_up(M * (size_t)d->d_model * 4, kAlign);
  }
  return c;
}

}  // namespace

size_t tsp_layer_workspace_size(const tsp_layer_desc* desc) {
  if (check_desc(desc) != TSP_OK) return 0;
  return carve(desc).total;
}

int tsp_layer_fwd(const tsp_layer_desc* desc, const void* x_shard, const void* w_qkv, const void* w_o,
                  const void* const* w1, const void* const* w3, const void* const* w2, void* k_full, void* v_full,
                  void* attn_out, float* mlp_out, void* ws, size_t ws_bytes, tsp_stream_t stream) {
  if (int rc = check_desc(desc)) return rc;
  if (desc->batch == 0 || desc->seq_len == 0) return ok();
  if (!x_shard || !w_qkv || !w_o || !w1 || !w3 || !w2 || !k_full || !v_full || !attn_out || !mlp_out || !ws)
    return fail(TSP_ERR_NULL, "a required pointer is NULL");
  const int D = desc->fold;
  for (int j = 0; j < D; ++j) {
    if (!w1[j] || !w3[j] || !w2[j]) return fail(TSP_ERR_NULL, "weight shard %d pointer is NULL", j);
    if (misaligned(w1[j]) || misaligned(w3[j]) || misaligned(w2[j]))
      return fail(TSP_ERR_ALIGN, "weight shard %d pointer is not 16-byte aligned", j);
  }
  if (misaligned(x_shard) || misaligned(w_qkv) || misaligned(w_o) || misaligned(k_full) || misaligned(v_full) ||
      misaligned(attn_out) || misaligned(mlp_out) || misaligned(ws))
    return fail(TSP_ERR_ALIGN, "device pointers must be 16-byte aligned");
  const LayerCarve c = carve(desc);
  if (ws_bytes < c.total) return fail(TSP_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, c.total);

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int B = desc->batch, H = desc->n_heads, hd = desc->head_dim, d = desc->d_model, r = desc->rank;
  const int64_t S = desc->seq_len;
  const int M = (int)(B * (S / D));
  const int Fs = desc->ffn / D;
  const int64_t ldw2 = desc->w2_ld ? desc->w2_ld : Fs;
  const int64_t ldseg = hidden_ld(Fs);  // H columns per shard block
  const int64_t ldh = ldseg * D;
  char* base = static_cast<char*>(ws);
  void* q = base + c.q_off;
  void* o = base + c.o_off;
  void* hbuf = base + c.h_off;
  hipEvent_t* tm = timing_slot();
  auto mark = [&](int p) -> int { return tm ? hip_status(hipEventRecord(tm[p], s), "hipEventRecord") : TSP_OK; };

  if (int rc = mark(0)) return rc;
  if (int rc = hip_status(tsp::launch_qkv(x_shard, w_qkv, q, k_full, v_full, B, S, D, r, d, s), "qkv launch"))
    return rc;
  if (int rc = mark(1)) return rc;
  // With at most one tile per CU the attention time is that of the heaviest tile: the later
  // chunk's tiles are then split in two key halves, whose fp32 partials use the MLP hidden
  // buffer (not yet written at this point) when it is large enough.
  if (tsp::attn_two_part_split(B, S, D, r, H) > 0 &&
      tsp::attn_two_part_bytes(B, S, D, H, hd) <= c.total - c.h_off) {
    if (int rc = hip_status(tsp::launch_attn_two_part(q, k_full, v_full, o, hbuf, B, S, D, r, H, hd, desc->scale, s),
                            "attention launch"))
      return rc;
  } else {
    if (int rc = hip_status(tsp::launch_attn(q, k_full, v_full, o, nullptr, B, S, D, r, H, hd, desc->scale, s),
                            "attention launch"))
      return rc;
  }
  if (int rc = mark(2)) return rc;
  if (int rc = hip_status(tsp::launch_proj_bf16(o, d, w_o, d, attn_out, d, M, d, d, s), "W_O launch")) return rc;
  if (int rc = mark(3)) return rc;
  // All D shards are resident here, so the ring runs as two launches: the gated hidden of
  // every shard, then one down projection whose reduction visits the shards in ring order
  // with the fp32 sums held in registers (stored once, no read-modify-write per shard).
  if (tsp::mlp_ring_fusable(w1, w3, w2, ldw2, D, M, d, Fs, ldh)) {
    if (int rc = hip_status(tsp::launch_gate_up_ring(attn_out, w1, w3, D, hbuf, ldh, ldseg, M, Fs, d, s),
                            "gate/up launch"))
      return rc;
    float* part = c.p_off ? reinterpret_cast<float*>(base + c.p_off) : nullptr;
    if (int rc = hip_status(tsp::launch_down_ring(hbuf, ldh, ldseg, w2, ldw2, D, r, mlp_out, d, 0, M, d, Fs, part, s),
                            "down projection launch"))
      return rc;
    if (int rc = mark(4)) return rc;
    return ok();
  }
  for (int t = 0; t < D; ++t) {
    const int j = ((r - t) % D + D) % D;  // shard held at ring step t
    if (int rc = hip_status(tsp::launch_gate_up(attn_out, d, w1[j], w3[j], d, hbuf, ldseg, M, Fs, d, s),
                            "gate/up launch"))
      return rc;
    if (int rc = hip_status(tsp::launch_down_acc(hbuf, ldseg, w2[j], ldw2, mlp_out, d, M, d, Fs, t > 0 ? 1 : 0, s),
                            "down projection launch"))
      return rc;
  }
  if (int rc = mark(4)) return rc;
  return ok();
}


namespace {

// Workspace of the layer backward (both parts share one size: the larger).
struct BwdCarve {
  // part 1 (MLP, W_O, attention)
  size_t a, at, dyb, dyt, da, gu, t2, dh, hb, dgu, t13, dgut, ht, dab, dat, wot, dob, ot, dsum;
  // part 2 (QKV)
  size_t dqkv, dqkvt, xt, wqkvt;
  size_t total;
};

BwdCarve carve_bwd(const tsp_layer_desc* d) {
  const size_t M = (size_t)d->batch * (size_t)(d->seq_len / d->fold);
  const size_t dm = (size_t)d->d_model;
  const size_t Fs = (size_t)(d->ffn / d->fold);
  const size_t R = (size_t)(d->seq_len / d->fold);
  BwdCarve c;
  size_t at = 0;
  auto take = [&](size_t bytes) {
    const size_t off = at;
    at += round_up(bytes, kAlign);
    return off;
  };
  c.a = take(M * dm * 2);
  c.at = take(M * dm * 2);
  c.dyb = take(M * dm * 2);
  c.dyt = take(M * dm * 2);
  c.da = take(M * dm * 4);
  c.gu = take(M * 2 * Fs * 2);
  c.t2 = take(Fs * dm * 2);
  c.dh = take(M * Fs * 4);
  c.hb = take(M * Fs * 2);
  c.dgu = take(M * 2 * Fs * 2);
  c.t13 = take(2 * Fs * dm * 2);
  c.dgut = take(M * 2 * Fs * 2);
  c.ht = take(M * Fs * 2);
  c.dab = take(M * dm * 2);
  c.dat = take(M * dm * 2);
  c.wot = take(dm * dm * 2);
  c.dob = take(M * dm * 2);
  c.ot = take(M * dm * 2);
  c.dsum = take((size_t)d->batch * (size_t)d->n_heads * R * 4);
  const size_t part1 = at;
  at = 0;
  c.dqkv = take(M * 3 * dm * 2);
  c.dqkvt = take(M * 3 * dm * 2);
  c.xt = take(M * dm * 2);
  c.wqkvt = take(3 * dm * dm * 2);
  c.total = part1 > at ? part1 : at;
  return c;
}

}  // namespace

size_t tsp_layer_bwd_workspace_size(const tsp_layer_desc* desc) {
  if (check_desc(desc) != TSP_OK) return 0;
  return carve_bwd(desc).total;
}

int tsp_layer_bwd_attn_mlp(const tsp_layer_desc* desc, const void* q, const void* o, const float* lse,
                           const void* k_full, const void* v_full, const void* w_o, const void* const* w_mlp,
                           const float* d_y, float* dq, float* dk_full, float* dv_full, float* dw_o,
                           float* const* dw13, float* const* dw2, void* ws, size_t ws_bytes, tsp_stream_t stream) {
  if (int rc = check_desc(desc)) return rc;
  if (desc->batch == 0 || desc->seq_len == 0) return ok();
  if (!q || !o || !lse || !k_full || !v_full || !w_o || !w_mlp || !d_y || !dq || !dk_full || !dv_full || !dw_o ||
      !dw13 || !dw2 || !ws)
    return fail(TSP_ERR_NULL, "a required pointer is NULL");
  const int D = desc->fold;
  for (int j = 0; j < D; ++j) {
    if (!w_mlp[j] || !dw13[j] || !dw2[j]) return fail(TSP_ERR_NULL, "shard %d pointer is NULL", j);
    if (misaligned(w_mlp[j]) || misaligned(dw13[j]) || misaligned(dw2[j]))
      return fail(TSP_ERR_ALIGN, "shard %d pointer is not 16-byte aligned", j);
  }
  if (misaligned(q) || misaligned(o) || misaligned(k_full) || misaligned(v_full) || misaligned(w_o) ||
      misaligned(d_y) || misaligned(dq) || misaligned(dk_full) || misaligned(dv_full) || misaligned(dw_o) ||
      misaligned(ws) || (reinterpret_cast<uintptr_t>(lse) & 3u))
    return fail(TSP_ERR_ALIGN, "device pointers must be 16-byte aligned (lse 4-byte)");
  const BwdCarve c = carve_bwd(desc);
  if (ws_bytes < c.total) return fail(TSP_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, c.total);

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int B = desc->batch, H = desc->n_heads, hd = desc->head_dim, d = desc->d_model, r = desc->rank;
  const int64_t S = desc->seq_len;
  const int M = (int)(B * (S / D));
  const int Fs = desc->ffn / D;
  const int64_t Fp = (int64_t)round_up((size_t)Fs, 8);  // W2 row stride in a packed MLP shard
  char* base = static_cast<char*>(ws);
  auto at = [&](size_t off) { return static_cast<void*>(base + off); };
  auto f32 = [&](size_t off) { return reinterpret_cast<float*>(base + off); };
  auto step = [](hipError_t e, const char* what) { return hip_status(e, what); };

  // Recompute A = O W_o^T; transposes of A and of dY (bf16) for the weight gradients.
  if (int rc = step(tsp::launch_proj_bf16(o, d, w_o, d, at(c.a), d, M, d, d, s), "W_O recompute")) return rc;
  if (int rc = step(tsp::launch_transpose_bf16(at(c.a), d, at(c.at), M, M, d, s), "transpose")) return rc;
  if (int rc = step(tsp::launch_convert_f32_bf16(d_y, d, at(c.dyb), d, M, d, s), "convert")) return rc;
  if (int rc = step(tsp::launch_transpose_f32_bf16(d_y, d, at(c.dyt), M, M, d, s), "transpose")) return rc;
  // MLP ring: shard j = (r - t) mod D at step t; dA summed in fp32 in that order.
  for (int t = 0; t < D; ++t) {
    const int j = ((r - t) % D + D) % D;
    const tsp::bf16_t* w13 = static_cast<const tsp::bf16_t*>(w_mlp[j]);  // [2 Fs, d]: W1 rows, W3 rows
    const tsp::bf16_t* w2j = w13 + 2 * (size_t)Fs * d;                   // [d, Fs], row stride Fp
    if (int rc = step(tsp::launch_proj_bf16(at(c.a), d, w13, d, at(c.gu), 2 * Fs, M, 2 * Fs, d, s), "gate/up"))
      return rc;
    if (int rc = step(tsp::launch_transpose_bf16(w2j, Fp, at(c.t2), d, d, Fs, s), "transpose")) return rc;
    if (int rc = step(tsp::launch_down_acc(at(c.dyb), d, at(c.t2), d, f32(c.dh), Fs, M, Fs, d, 0, s), "dH")) return rc;
    if (int rc = step(tsp::launch_swiglu_bwd(at(c.gu), 2 * Fs, f32(c.dh), Fs, at(c.hb), Fs, at(c.dgu), 2 * Fs, M, Fs, s),
                      "gate backward"))
      return rc;
    if (int rc = step(tsp::launch_transpose_bf16(w13, d, at(c.t13), 2 * Fs, 2 * Fs, d, s), "transpose")) return rc;
    if (int rc = step(tsp::launch_down_acc(at(c.dgu), 2 * Fs, at(c.t13), 2 * Fs, f32(c.da), d, M, d, 2 * Fs, t > 0 ? 1 : 0,
                                           s),
                      "dA"))
      return rc;
    if (int rc = step(tsp::launch_transpose_bf16(at(c.dgu), 2 * Fs, at(c.dgut), M, M, 2 * Fs, s), "transpose")) return rc;
    if (int rc = step(tsp::launch_down_acc(at(c.dgut), M, at(c.at), M, dw13[j], d, 2 * Fs, d, M, 0, s), "dW1/dW3"))
      return rc;
    if (int rc = step(tsp::launch_transpose_bf16(at(c.hb), Fs, at(c.ht), M, M, Fs, s), "transpose")) return rc;
    if (int rc = step(tsp::launch_down_acc(at(c.dyt), M, at(c.ht), M, dw2[j], Fs, d, Fs, M, 0, s), "dW2")) return rc;
  }
  // W_O: dO = dA W_o (bf16, for the attention backward); dW_o = dA^T O.
  if (int rc = step(tsp::launch_convert_f32_bf16(f32(c.da), d, at(c.dab), d, M, d, s), "convert")) return rc;
  if (int rc = step(tsp::launch_transpose_f32_bf16(f32(c.da), d, at(c.dat), M, M, d, s), "transpose")) return rc;
  if (int rc = step(tsp::launch_transpose_bf16(w_o, d, at(c.wot), d, d, d, s), "transpose")) return rc;
  if (int rc = step(tsp::launch_proj_bf16(at(c.dab), d, at(c.wot), d, at(c.dob), d, M, d, d, s), "dO")) return rc;
  if (int rc = step(tsp::launch_transpose_bf16(o, d, at(c.ot), M, M, d, s), "transpose")) return rc;
  if (int rc = step(tsp::launch_down_acc(at(c.dat), M, at(c.ot), M, dw_o, d, d, d, M, 0, s), "dW_o")) return rc;
  // Attention.
  return step(tsp::launch_attn_bwd(q, k_full, v_full, o, lse, at(c.dob), dq, dk_full, dv_full, f32(c.dsum), B, S, D, r,
                                   H, hd, desc->scale, s),
              "attention backward");
}

int tsp_layer_bwd_qkv(const tsp_layer_desc* desc, const void* x_shard, const void* w_qkv, const float* dq,
                      const float* dk_own, const float* dv_own, float* dx, float* dw_qkv, void* ws, size_t ws_bytes,
                      tsp_stream_t stream) {
  if (int rc = check_desc(desc)) return rc;
  if (desc->batch == 0 || desc->seq_len == 0) return ok();
  if (!x_shard || !w_qkv || !dq || !dk_own || !dv_own || !dx || !dw_qkv || !ws)
    return fail(TSP_ERR_NULL, "a required pointer is NULL");
  if (misaligned(x_shard) || misaligned(w_qkv) || misaligned(dq) || misaligned(dk_own) || misaligned(dv_own) ||
      misaligned(dx) || misaligned(dw_qkv) || misaligned(ws))
    return fail(TSP_ERR_ALIGN, "device pointers must be 16-byte aligned");
  const BwdCarve c = carve_bwd(desc);
  if (ws_bytes < c.total) return fail(TSP_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, c.total);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int d = desc->d_model;
  const int M = (int)(desc->batch * (desc->seq_len / desc->fold));
  char* base = static_cast<char*>(ws);
  auto at = [&](size_t off) { return static_cast<void*>(base + off); };
  auto step = [](hipError_t e, const char* what) { return hip_status(e, what); };
  // dQKV = [dq | dk_own | dv_own] (bf16 [M, 3d]); dX = dQKV W_qkv; dW_qkv = dQKV^T X.
  tsp::bf16_t* dqkv = static_cast<tsp::bf16_t*>(at(c.dqkv));
  if (int rc = step(tsp::launch_convert_f32_bf16(dq, d, dqkv, 3 * d, M, d, s), "convert")) return rc;
  if (int rc = step(tsp::launch_convert_f32_bf16(dk_own, d, dqkv + d, 3 * d, M, d, s), "convert")) return rc;
  if (int rc = step(tsp::launch_convert_f32_bf16(dv_own, d, dqkv + 2 * d, 3 * d, M, d, s), "convert")) return rc;
  if (int rc = step(tsp::launch_transpose_bf16(w_qkv, d, at(c.wqkvt), 3 * d, 3 * d, d, s), "transpose")) return rc;
  if (int rc = step(tsp::launch_down_acc(dqkv, 3 * d, at(c.wqkvt), 3 * d, dx, d, M, d, 3 * d, 0, s), "dX")) return rc;
  if (int rc = step(tsp::launch_transpose_bf16(dqkv, 3 * d, at(c.dqkvt), M, M, 3 * d, s), "transpose")) return rc;
  if (int rc = step(tsp::launch_transpose_bf16(x_shard, d, at(c.xt), M, M, d, s), "transpose")) return rc;
  return step(tsp::launch_down_acc(at(c.dqkvt), M, at(c.xt), M, dw_qkv, d, 3 * d, d, M, 0, s), "dW_qkv");
}

}  // extern "C"

namespace {

// Events of the weight-streamed layer, per host thread and device, created on first use.
// Re-recording an event is safe for waits already queued: a stream wait takes the
// event's most recent record at the time the wait is queued.
int stream_events(hipEvent_t** out, int n) {
  thread_local std::map<int, std::vector<hipEvent_t>> pool;
  int dev = 0;
  if (int rc = hip_status(hipGetDevice(&dev), "hipGetDevice")) return rc;
  std::vector<hipEvent_t>& ev = pool[dev];
  while ((int)ev.size() < n) {
    hipEvent_t e = nullptr;
    if (int rc = hip_status(hipEventCreateWithFlags(&e, hipEventDisableTiming), "hipEventCreateWithFlags")) return rc;
    ev.push_back(e);
  }
  *out = ev.data();
  return TSP_OK;
}

struct StreamedCarve {
  size_t q_off, o_off, h_off, slot_a[2], slot_m[2], part, total;
  size_t attn_shard, mlp_shard;  // elements of one packed shard
  int64_t fp;                    // W2 row stride in a packed MLP shard
  int64_t fh;                    // row stride of the gated hidden
};

StreamedCarve carve_streamed(const tsp_layer_desc* d) {
  const size_t M = (size_t)d->batch * (size_t)(d->seq_len / d->fold);
  const size_t dm = (size_t)d->d_model;
  const size_t dg = dm / (size_t)d->fold;
  const size_t Fs = (size_t)(d->ffn / d->fold);
  StreamedCarve c;
  c.fp = (int64_t)round_up(Fs, 8);
  c.fh = hidden_ld((int64_t)Fs);
  c.attn_shard = 4 * dg * dm;
  c.mlp_shard = (2 * Fs + (size_t)c.fp) * dm;
  const size_t act = round_up(M * dm * 2, kAlign);
  size_t at = 0;
  c.q_off = at;
  at += act;
  c.o_off = at;
  at += act;
  c.h_off = at;
  // Gated hidden of two shards (the MLP ring runs in pairs of steps), one with D = 1.
  at += round_up(M * (size_t)(d->fold >= 2 ? 2 : 1) * (size_t)c.fh * 2, kAlign);
  for (int i = 0; i < 2; ++i) {
    c.slot_a[i] = at;
    at += round_up(c.attn_shard * 2, kAlign);
  }
  for (int i = 0; i < 2; ++i) {
    c.slot_m[i] = at;
    at += round_up(c.mlp_shard * 2, kAlign);
  }
  // With D odd, the last head group runs alone and its attention is split into two key
  // halves: fp32 O [2, M, dg] and log-sum-exp [2, M * heads per group]. Pairs of groups
  // write O directly.
  const size_t hg = (size_t)(d->n_heads / d->fold);
  c.part = at;
  if (d->fold % 2) at += round_up(2 * M * dg * 4, kAlign) + round_up(2 * M * hg * 4, kAlign);
  c.total = at;
  return c;
}

int check_streamed_desc(const tsp_layer_desc* desc) {
  if (int rc = check_desc(desc)) return rc;
  if (desc->n_heads % desc->fold != 0)
    return fail(TSP_ERR_SHAPE, "n_heads %d must be a multiple of D=%d for head groups", desc->n_heads, desc->fold);
  return TSP_OK;
}

}  // namespace

extern "C" {

size_t tsp_layer_streamed_workspace_size(const tsp_layer_desc* desc) {
  if (check_streamed_desc(desc) != TSP_OK) return 0;
  return carve_streamed(desc).total;
}

int tsp_layer_fwd_streamed(const tsp_layer_desc* desc, const void* x_shard, const void* const* w_attn,
                           const void* const* w_mlp, void* k_full, void* v_full, void* attn_out, float* mlp_out,
                           void* ws, size_t ws_bytes, const tsp_stream_t* streams, int32_t n_streams) {
  if (int rc = check_streamed_desc(desc)) return rc;
  if (n_streams != 1 && n_streams != 4) return fail(TSP_ERR_SHAPE, "n_streams must be 1 or 4 (got %d)", n_streams);
  if (desc->batch == 0 || desc->seq_len == 0) return ok();
  if (!x_shard || !w_attn || !w_mlp || !k_full || !v_full || !attn_out || !mlp_out || !ws || !streams)
    return fail(TSP_ERR_NULL, "a required pointer is NULL");
  const int D = desc->fold;
  for (int j = 0; j < D; ++j) {
    if (!w_attn[j] || !w_mlp[j]) return fail(TSP_ERR_NULL, "packed shard %d pointer is NULL", j);
    if (misaligned(w_attn[j]) || misaligned(w_mlp[j]))
      return fail(TSP_ERR_ALIGN, "packed shard %d pointer is not 16-byte aligned", j);
  }
  if (misaligned(x_shard) || misaligned(k_full) || misaligned(v_full) || misaligned(attn_out) ||
      misaligned(mlp_out) || misaligned(ws))
    return fail(TSP_ERR_ALIGN, "device pointers must be 16-byte aligned");
  const StreamedCarve c = carve_streamed(desc);
  if (ws_bytes < c.total) return fail(TSP_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, c.total);

  const int B = desc->batch, H = desc->n_heads, hd = desc->head_dim, d = desc->d_model, r = desc->rank;
  const int64_t S = desc->seq_len;
  const int M = (int)(B * (S / D));
  const int Fs = desc->ffn / D;
  const int hg = H / D;  // heads per group
  const size_t dg = (size_t)(d / D);
  const size_t qkv_part = 3 * dg * (size_t)d;  // elements of a shard's [3 dg, d] QKV rows
  char* base = static_cast<char*>(ws);
  void* q = base + c.q_off;
  void* o = base + c.o_off;
  void* hbuf = base + c.h_off;
  tsp::bf16_t* slot_a[2] = {reinterpret_cast<tsp::bf16_t*>(base + c.slot_a[0]),
                            reinterpret_cast<tsp::bf16_t*>(base + c.slot_a[1])};
  tsp::bf16_t* slot_m[2] = {reinterpret_cast<tsp::bf16_t*>(base + c.slot_m[0]),
                            reinterpret_cast<tsp::bf16_t*>(base + c.slot_m[1])};
  float* part = reinterpret_cast<float*>(base + c.part);
  float* part_lse = reinterpret_cast<float*>(base + c.part + round_up(2 * (size_t)M * dg * 4, kAlign));
  hipStream_t s0 = static_cast<hipStream_t>(streams[0]);
  auto pick = [&](int i) { return n_streams == 4 && streams[i] ? static_cast<hipStream_t>(streams[i]) : s0; };
  hipStream_t comp[2] = {s0, pick(1)};
  hipStream_t s_wo = pick(2);
  hipStream_t cp = pick(3);

  hipEvent_t* ev = nullptr;
  if (int rc = stream_events(&ev, 20)) return rc;
  hipEvent_t ev_start = ev[0], wo_last = ev[1];
  hipEvent_t *q_full = ev + 2, *q_free = ev + 4;      // QKV part of an attention slot
  hipEvent_t *o_full = ev + 6, *o_free = ev + 8;      // W_o part of an attention slot
  hipEvent_t *g_full = ev + 10, *g_free = ev + 12;    // W1/W3 part of an MLP slot
  hipEvent_t *d_full = ev + 14, *d_free = ev + 16;    // W2 part of an MLP slot
  hipEvent_t* attn_done = ev + 18;                    // per attention stream
  auto rec = [](hipEvent_t e, hipStream_t st) { return hip_status(hipEventRecord(e, st), "hipEventRecord"); };
  auto wait = [](hipStream_t st, hipEvent_t e) {
    return hip_status(hipStreamWaitEvent(st, e, 0), "hipStreamWaitEvent");
  };
  // Copy `elems` bf16 into a slot after `free_ev` (if any), then record `full_ev`.
  auto fill = [&](void* dst, const void* src, size_t elems, hipEvent_t free_ev, hipEvent_t full_ev) -> int {
    if (free_ev)
      if (int rc = wait(cp, free_ev)) return rc;
    if (int rc = hip_status(hipMemcpyAsync(dst, src, elems * 2, hipMemcpyDeviceToDeviceNoCU, cp), "shard copy"))
      return rc;
    return rec(full_ev, cp);
  };
  auto fill_qkv = [&](int t) {
    return fill(slot_a[t & 1], w_attn[t], qkv_part, t >= 2 ? q_free[t & 1] : nullptr, q_full[t & 1]);
  };
  auto fill_wo = [&](int t) {
    return fill(slot_a[t & 1] + qkv_part, static_cast<const tsp::bf16_t*>(w_attn[t]) + qkv_part, dg * d,
                t >= 2 ? o_free[t & 1] : nullptr, o_full[t & 1]);
  };
  // An MLP slot is refilled in two parts: its W1/W3 rows once the gate/up launch that read
  // them is done, its W2 once the down projection is done.
  const size_t w13_part = 2 * (size_t)Fs * (size_t)d;
  auto fill_mlp13 = [&](int t) {
    const int j = ((r - t) % D + D) % D;  // ring order
    return fill(slot_m[t & 1], w_mlp[j], w13_part, t >= 2 ? g_free[t & 1] : nullptr, g_full[t & 1]);
  };
  auto fill_mlp2 = [&](int t) {
    const int j = ((r - t) % D + D) % D;
    return fill(slot_m[t & 1] + w13_part, static_cast<const tsp::bf16_t*>(w_mlp[j]) + w13_part,
                c.mlp_shard - w13_part, t >= 2 ? d_free[t & 1] : nullptr, d_full[t & 1]);
  };

  if (int rc = rec(ev_start, s0)) return rc;
  for (hipStream_t st : {comp[1], s_wo, cp})
    if (int rc = wait(st, ev_start)) return rc;
  for (int t = 0; t < 2 && t < D; ++t) {
    if (int rc = fill_qkv(t)) return rc;
    if (int rc = fill_wo(t)) return rc;
  }
  for (int t = 0; t < 2 && t < D; ++t) {
    if (int rc = fill_mlp13(t)) return rc;
    if (int rc = fill_mlp2(t)) return rc;
  }

  // Head groups in pairs (t, t+1), one group per slot: the pair's QKV launches, then its
  // attention as one launch over both groups' heads, on comp[(t / 2) % 2]; then one W_O
  // partial over both groups on s_wo (pairs in order, so the fp32 sum takes the groups in
  // order). A slot's QKV rows are refilled once its QKV launch is done, its W_o columns once
  // the pair's W_O launch is done. With D odd the last group runs alone, its attention split
  // into two key halves (one group is about one query tile per CU, and a tile of the later
  // zigzag chunk sees up to S keys) merged by log-sum-exp.
  for (int t = 0; t < D; t += 2) {
    const bool pair = t + 1 < D;
    const int pi = (t / 2) & 1;
    hipStream_t st = comp[pi];
    for (int u = t; u < t + (pair ? 2 : 1); ++u) {
      const int sl = u & 1;
      if (int rc = wait(st, q_full[sl])) return rc;
      if (int rc = hip_status(tsp::launch_qkv_group(x_shard, slot_a[sl], u, D, q, k_full, v_full, B, S, D, r, d, st),
                              "group qkv launch"))
        return rc;
      if (u + 2 < D) {
        if (int rc = rec(q_free[sl], st)) return rc;
        if (int rc = fill_qkv(u + 2)) return rc;
      }
    }
    if (pair) {
      if (int rc = hip_status(tsp::launch_attn_heads(q, k_full, v_full, o, B, S, D, r, H, hd, desc->scale, t * hg,
                                                     2 * hg, st),
                              "group pair attention launch"))
        return rc;
    } else {
      if (int rc = hip_status(tsp::launch_attn_split(q, k_full, v_full, part, part_lse, B, S, D, r, H, hd,
                                                     desc->scale, t * hg, hg, (int)(S / 2), st),
                              "group attention launch"))
        return rc;
      if (int rc = hip_status(tsp::launch_attn_merge_halves(part, part_lse, o, B, (int)(S / D), H, hd, t * hg,
                                                            hg, st),
                              "group attention merge launch"))
        return rc;
    }
    if (int rc = rec(attn_done[pi], st)) return rc;
    if (int rc = wait(s_wo, attn_done[pi])) return rc;
    if (int rc = wait(s_wo, o_full[0])) return rc;
    if (pair)
      if (int rc = wait(s_wo, o_full[1])) return rc;
    const hipError_t e = pair ? tsp::launch_wo_pair(o, slot_a[0] + qkv_part, slot_a[1] + qkv_part, t, D, mlp_out,
                                                    attn_out, M, d, t == 0 ? 1 : 0, t + 2 >= D ? 1 : 0, s_wo)
                              : tsp::launch_wo_group(o, slot_a[0] + qkv_part, t, D, mlp_out, attn_out, M, d, t == 0 ? 0 : 1,
                                                     t == 0 ? 1 : 2, s_wo);
    if (int rc = hip_status(e, "group W_O launch")) return rc;
    for (int u = t; u < t + (pair ? 2 : 1); ++u)
      if (u + 2 < D) {
        if (int rc = rec(o_free[u & 1], s_wo)) return rc;
        if (int rc = fill_wo(u + 2)) return rc;
      }
  }
  if (int rc = rec(wo_last, s_wo)) return rc;
  if (int rc = wait(s0, wo_last)) return rc;

  // MLP ring on streams[0], shard j = (r - t) mod D at step t, one per slot: the gated hidden
  // of each step into its own block of a two-shard hidden, and after every second step one
  // down projection whose fp32 sum runs over both steps' shards in registers (step t - 1
  // first) and is added to mlp_out once: half the read-modify-write passes over mlp_out. A
  // slot's W1/W3 rows refill once its gate/up launch is done (in time for the step two later,
  // a gate/up and a down projection later); its W2 once the pair's down projection is done.
  // A lone last step (D odd) runs its down projection alone; shard widths the two-shard
  // kernels cannot take run every step alone.
  auto w1_of = [&](int sl) -> const tsp::bf16_t* { return slot_m[sl]; };
  auto w3_of = [&](int sl) -> const tsp::bf16_t* { return slot_m[sl] + (size_t)Fs * d; };
  auto w2_of = [&](int sl) -> const tsp::bf16_t* { return slot_m[sl] + 2 * (size_t)Fs * d; };
  const void* w1p[2] = {w1_of(0), w1_of(1)};
  const void* w3p[2] = {w3_of(0), w3_of(1)};
  const void* w2p[2] = {w2_of(0), w2_of(1)};
  const bool pairs = D >= 2 && tsp::mlp_ring_fusable(w1p, w3p, w2p, c.fp, 2, M, d, Fs, 2 * c.fh);
  const int64_t ldh = pairs ? 2 * c.fh : c.fh;
  for (int t = 0; t < D; ++t) {
    const int sl = t & 1;
    tsp::bf16_t* hb = static_cast<tsp::bf16_t*>(hbuf) + (pairs ? (size_t)sl * (size_t)c.fh : 0);
    if (int rc = wait(s0, g_full[sl])) return rc;
    if (int rc = hip_status(tsp::launch_gate_up(attn_out, d, w1_of(sl), w3_of(sl), d, hb, ldh, M, Fs, d, s0),
                            "gate/up launch"))
      return rc;
    if (t + 2 < D) {
      if (int rc = rec(g_free[sl], s0)) return rc;
      if (int rc = fill_mlp13(t + 2)) return rc;
    }
    if (pairs && sl == 1) {  // steps t - 1 (slot 0) and t (slot 1): ring order is slot order
      for (int u = 0; u < 2; ++u)
        if (int rc = wait(s0, d_full[u])) return rc;
      if (int rc = hip_status(tsp::launch_down_ring(hbuf, ldh, c.fh, w2p, c.fp, 2, 0, mlp_out, d, t > 1 ? 1 : 0, M, d,
                                                    Fs, nullptr, s0),
                              "down projection launch"))
        return rc;
      for (int u = t - 1; u <= t; ++u)
        if (u + 2 < D) {
          if (int rc = rec(d_free[u & 1], s0)) return rc;
          if (int rc = fill_mlp2(u + 2)) return rc;
        }
    } else if (!pairs || t == D - 1) {
      if (int rc = wait(s0, d_full[sl])) return rc;
      if (int rc = hip_status(tsp::launch_down_acc(hb, ldh, w2_of(sl), c.fp, mlp_out, d, M, d, Fs, t > 0 ? 1 : 0, s0),
                              "down projection launch"))
        return rc;
      if (t + 2 < D) {
        if (int rc = rec(d_free[sl], s0)) return rc;
        if (int rc = fill_mlp2(t + 2)) return rc;
      }
    }
  }
  return ok();
}

}  // extern "C"
