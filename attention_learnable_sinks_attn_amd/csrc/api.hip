// C ABI of libattn_sink.so: argument checks, launch configuration, error mapping.
// Every check runs on the host before anything is enqueued; the library allocates nothing.
#include <math.h>
#include <stdint.h>

#include "attn_sink.h"
#include <algorithm>
#include <mutex>

#include "kernels.h"

using namespace attn_sink;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool head_dim_ok(int d) { return d == 64 || d == 128; }

// bf16_out: whether the call can store its output in bf16 (the forward can; the backward reads
// the forward's fp32 output).
int check_shape(const attn_sink_shape* s, bool bf16_out = false) {
  if (s == nullptr) return ATTN_SINK_ERR_NULL_PTR;
  if (s->total_tokens < 0 || s->num_seqs < 1 || s->num_heads_q < 1 || s->num_heads_kv < 1 ||
      s->max_seqlen < 0 || s->max_seqlen > s->total_tokens || s->num_heads_q % s->num_heads_kv != 0) {
    return ATTN_SINK_ERR_BAD_SHAPE;
  }
  if (!head_dim_ok(s->head_dim) ||
      (s->out_dtype != ATTN_SINK_F32 && !(bf16_out && s->out_dtype == ATTN_SINK_BF16))) {
    return ATTN_SINK_ERR_UNSUPPORTED;
  }
  // Element offsets are 64-bit in the kernels, but grid sizes and per-head row indices are
  // 32-bit.
  const long long rows_q = (long long)s->total_tokens * s->num_heads_q;
  if (rows_q > (1LL << 34)) return ATTN_SINK_ERR_BAD_SHAPE;
  // Within one sequence, element offsets (row * heads * 64) are 32-bit.
  if ((long long)s->max_seqlen * s->num_heads_q * s->head_dim >= (1LL << 31)) return ATTN_SINK_ERR_BAD_SHAPE;
  const long long nq = ((long long)s->max_seqlen + 63) / 64;
  if (nq * s->num_heads_q * (long long)s->num_seqs >= (1LL << 31)) return ATTN_SINK_ERR_BAD_SHAPE;
  return ATTN_SINK_OK;
}

// A window of at least the longest sequence sees every key, exactly as one of that length does;
// clamping keeps the kernels' index arithmetic (row + window) far from overflow.
int clamp_window(int window, int longest) { return window > 0 ? std::min(window, std::max(longest, 1)) : 0; }

int heads_per_group_split(int G) { return G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1); }

float resolve_scale(const attn_sink_shape* s) {
  return s->softmax_scale > 0.0f ? s->softmax_scale : 1.0f / sqrtf((float)s->head_dim);
}

int dsink_slots(const attn_sink_shape* s) { return s->total_tokens / kDqRowsPerWave + s->num_seqs + 1; }

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// The dK/dV pass splits each KV group's query heads over two workgroups only when its key blocks
// alone would not fill the GPU several times over (about 2048 workgroups); the halves' fp32
// partials are then added by the finish kernel. With one half the pass writes dK and dV itself.
int kv_halves(const attn_sink_shape* s) {
  const long long blocks = (long long)s->num_seqs * ((s->max_seqlen + kKvKeysPerBlock - 1) / kKvKeysPerBlock) *
                           s->num_heads_kv;
  return ((s->num_heads_q / s->num_heads_kv) % 2 == 0 && blocks < 2048) ? 2 : 1;
}

size_t dkv_part_bytes(const attn_sink_shape* s) {
  const int n = kv_halves(s);
  return n == 1 ? 0 : (size_t)2 * n * s->total_tokens * s->num_heads_kv * s->head_dim * sizeof(float);
}

// Workspace: -LSE/scale [Hq, T], -D [Hq, T] (both written by the dQ pass for the dK/dV pass), dSink
// partials [Hq, n_slots], dK/dV partials per head half, each 256-byte aligned.
size_t row_plane_bytes(const attn_sink_shape* s) {
  return round256((size_t)s->num_heads_q * s->total_tokens * sizeof(float));
}

size_t dsink_part_bytes(const attn_sink_shape* s) {
  return round256((size_t)s->num_heads_q * dsink_slots(s) * sizeof(float));
}

size_t workspace_bytes(const attn_sink_shape* s) {
  return 2 * row_plane_bytes(s) + dsink_part_bytes(s) + round256(dkv_part_bytes(s));
}

// Checks of the backward's shape and tensor pointers (everything but the workspace).
int check_bwd_args(const void* q, const void* k, const void* v, const float* sinks, const void* out, const float* lse,
                   const void* dout, const int32_t* cu_seqlens, const attn_sink_shape* shape, const float* dq,
                   const float* dk, const float* dv, const float* dsinks) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (sinks == nullptr || cu_seqlens == nullptr || dsinks == nullptr) return ATTN_SINK_ERR_NULL_PTR;
  const int T = shape->total_tokens;
  if (T > 0 && (!q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv)) return ATTN_SINK_ERR_NULL_PTR;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(dout) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv)) {
    return ATTN_SINK_ERR_ALIGN;
  }
  return ATTN_SINK_OK;
}

int bwd_impl(const void* q, const void* k, const void* v, const float* sinks, const void* out, const float* lse,
             const void* dout, int causal, int window, const int32_t* cu_seqlens, const attn_sink_shape* shape,
             void* workspace, size_t ws_bytes, float* dq, float* dk, float* dv, float* dsinks, hipStream_t stream,
             void* const* events, int num_events) {
  int rc = check_bwd_args(q, k, v, sinks, out, lse, dout, cu_seqlens, shape, dq, dk, dv, dsinks);
  if (rc) return rc;
  const int T = shape->total_tokens;
  const size_t need = workspace_bytes(shape);
  if (workspace == nullptr || ws_bytes < need || !aligned16(workspace)) return ATTN_SINK_ERR_WORKSPACE;
  if (events != nullptr && num_events != kBwdNumKernels + 1) return ATTN_SINK_ERR_BAD_SHAPE;

  BwdArgs a = {};
  a.q = static_cast<const __bf16*>(q);
  a.k = static_cast<const __bf16*>(k);
  a.v = static_cast<const __bf16*>(v);
  a.sinks = sinks;
  a.out = static_cast<const float*>(out);
  a.lse = lse;
  a.dout = static_cast<const __bf16*>(dout);
  a.cu = cu_seqlens;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dsinks = dsinks;
  a.nlse = static_cast<float*>(workspace);
  a.negd = reinterpret_cast<float*>(static_cast<char*>(workspace) + row_plane_bytes(shape));
  a.dsink_part = reinterpret_cast<float*>(static_cast<char*>(workspace) + 2 * row_plane_bytes(shape));
  a.dkv_part = reinterpret_cast<float*>(static_cast<char*>(workspace) + 2 * row_plane_bytes(shape) +
                                        dsink_part_bytes(shape));
  a.n_slots = dsink_slots(shape);
  // Head halves balance the causal triangle on short sequences; with a window every key block has
  // the same work, and one round of full-group workgroups (two per CU) beats two rounds of halves
  // plus the finish pass's sum. (The workspace is sized for the halves either way.)
  const long long kv_blocks =
      (long long)shape->num_seqs * ((shape->max_seqlen + kKvKeysPerBlock - 1) / kKvKeysPerBlock) * shape->num_heads_kv;
  a.n_halves = (window > 0 && kv_blocks >= 512) ? 1 : kv_halves(shape);
  a.T = T;
  a.B = shape->num_seqs;
  a.Hq = shape->num_heads_q;
  a.Hkv = shape->num_heads_kv;
  a.G = a.Hq / a.Hkv;
  a.hpw = heads_per_group_split(a.G);
  // Two key halves x two head streams per workgroup where the heads split evenly, two workgroups
  // per CU. (With a window, an 8-wave workgroup holding all of a group's heads as four streams, one
  // per CU, lost 37% of its step loop at the per-step barrier: at the window's edges the two key
  // halves of a stream have different numbers of live row blocks in a step, and with one
  // workgroup per CU nothing fills the wait. Two 4-wave workgroups per CU hide it: the pass took
  // 9-23% less time on the window-128 workloads.)
  a.kv_streams = (a.G / a.n_halves) % 2 == 0 ? 2 : 1;
  // At head_dim 128 a dK/dV wave needs more than half of a SIMD's registers, so a CU holds four
  // waves: two 2-wave workgroups (one head stream each) hide each other's per-step barrier waits,
  // one 4-wave workgroup does not (measured 8% less time for the pass at 4k causal, GQA 64/8).
  if (shape->head_dim == 128) a.kv_streams = 1;
  const int dq_rows = kDqRowsPerWave * (4 / a.hpw);  // rows per dQ workgroup
  a.n_qblocks = (shape->max_seqlen + dq_rows - 1) / dq_rows;
  a.n_kblocks = (shape->max_seqlen + kKvKeysPerBlock - 1) / kKvKeysPerBlock;
  a.causal = causal ? 1 : 0;
  a.window = clamp_window(window, shape->max_seqlen);
  a.scale = resolve_scale(shape);
  a.scale_log2 = a.scale * kLog2e;
  a.D = shape->head_dim;

  typedef hipError_t (*launcher)(const BwdArgs&, hipStream_t);
  const launcher steps[kBwdNumKernels] = {launch_bwd_dq, launch_bwd_dkdv, launch_bwd_finish};
  for (int i = 0; i < kBwdNumKernels; ++i) {
    if (events && events[i] && hipEventRecord(static_cast<hipEvent_t>(events[i]), stream) != hipSuccess) {
      return ATTN_SINK_ERR_HIP;
    }
    if (steps[i](a, stream) != hipSuccess) return ATTN_SINK_ERR_HIP;
  }
  if (events && events[kBwdNumKernels] &&
      hipEventRecord(static_cast<hipEvent_t>(events[kBwdNumKernels]), stream) != hipSuccess) {
    return ATTN_SINK_ERR_HIP;
  }
  return ATTN_SINK_OK;
}

// ---- decode ----
float resolve_decode_scale(const attn_sink_decode_shape* s) {
  return s->softmax_scale > 0.0f ? s->softmax_scale : 1.0f / sqrtf((float)s->head_dim);
}

int check_decode_shape(const attn_sink_decode_shape* s) {
  if (s == nullptr) return ATTN_SINK_ERR_NULL_PTR;
  if (s->total_q < 0 || s->total_k < 0 || s->num_seqs < 1 || s->max_q < 0 || s->max_k < 0 ||
      s->num_heads_q < 1 || s->num_heads_kv < 1 || s->num_heads_q % s->num_heads_kv != 0 ||
      s->max_q > s->total_q || s->max_k > s->total_k) {
    return ATTN_SINK_ERR_BAD_SHAPE;
  }
  if (!head_dim_ok(s->head_dim) || (s->out_dtype != ATTN_SINK_F32 && s->out_dtype != ATTN_SINK_BF16)) {
    return ATTN_SINK_ERR_UNSUPPORTED;
  }
  if ((long long)s->max_q * (s->num_heads_q / s->num_heads_kv) > kDecodeMaxCols) return ATTN_SINK_ERR_UNSUPPORTED;
  if ((long long)s->total_k * s->num_heads_kv * s->head_dim >= (1LL << 40) ||
      (long long)s->total_q * s->num_heads_q >= (1LL << 31) ||
      (long long)s->num_seqs * s->num_heads_kv * kDecodeMaxCols >= (1LL << 31) ||  // workgroups of one launch
      (s->total_q > 0 && s->max_q < 1)) {
    return ATTN_SINK_ERR_BAD_SHAPE;
  }
  return ATTN_SINK_OK;
}

// Key chunks: about 4096 (sequence, KV head, chunk) waves, five rounds of the 768 that fit the
// GPU at once (three 48 KB rings per CU), each chunk a whole number of 64-key tiles. `tiles` is
// the most tiles any sequence's new tokens see. Fewer, longer chunks leave the last round's CUs
// idle; more, shorter ones spend more time filling each wave's ring and merging partials.
void split_keys(long long pairs, long long tiles, long long* per, long long* n) {
  const long long target = pairs >= 4096 ? 1 : (4096 + pairs - 1) / pairs;
  *per = tiles <= 0 ? 1 : (tiles + target - 1) / target;
  *n = tiles <= 0 ? 1 : (tiles + *per - 1) / *per;
}

// Groups of 32 (new token, query head) columns per (sequence, KV head).
int decode_col_groups(const attn_sink_decode_shape* s) {
  const long long cols = (long long)s->max_q * (s->num_heads_q / s->num_heads_kv);
  return (int)std::max<long long>(1, (cols + 31) / 32);
}

// Chunks for a call with the given window. The workspace is sized for window 0; a window only
// shortens the span to chunk (the keys from the 64-aligned start of the first visible one), and the
// chunk count never exceeds the workspace's.
void decode_chunks(const attn_sink_decode_shape* s, int window, int* n_chunks, int* chunk_keys) {
  const long long pairs = (long long)s->num_seqs * s->num_heads_kv * decode_col_groups(s);
  long long per, n;
  split_keys(pairs, ((long long)s->max_k + 63) / 64, &per, &n);
  if (window > 0) {
    const long long span = std::min<long long>(s->max_k, (long long)window + s->max_q - 1 + 63);
    const long long tiles = (span + 63) / 64;
    long long per_w, n_w;
    split_keys(pairs, tiles, &per_w, &n_w);
    if (n_w > n) {
      per_w = (tiles + n - 1) / n;
      n_w = (tiles + per_w - 1) / per_w;
    }
    per = per_w;
    n = n_w;
  }
  *chunk_keys = (int)(64 * per);
  *n_chunks = (int)n;
}

size_t decode_part_o_bytes(const attn_sink_decode_shape* s, int n_chunks) {
  return round256((size_t)s->num_seqs * s->num_heads_kv * decode_col_groups(s) * n_chunks * s->head_dim * 32 *
                  sizeof(float));
}

size_t decode_workspace_bytes(const attn_sink_decode_shape* s) {
  int n, ck;
  decode_chunks(s, 0, &n, &ck);
  return decode_part_o_bytes(s, n) +
         round256((size_t)s->num_seqs * s->num_heads_kv * decode_col_groups(s) * n * 2 * 32 * sizeof(float));
}

}  // namespace

// ---- backward without a caller workspace ----
// Device memory for attn_sink_bwd_noalloc's workspace: a file-scope array of fixed size, one copy
// per GPU the library runs on, held until the process ends. Its name is only a host-side stand-in:
// host code must use the address hipGetSymbolAddress returns for the device (scratch_address).
static __device__ __align__(256) unsigned char scratch[ATTN_SINK_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, looked up once

// Device address of `scratch` on the device `stream` belongs to (the current device for the
// NULL stream). The first call per device makes that device current for the lookup and restores
// the caller's device afterwards.
int scratch_address(hipStream_t stream, void** out) {
  int dev = -1;
  if (stream != nullptr) {
    if (hipStreamGetDevice(stream, &dev) != hipSuccess) return ATTN_SINK_ERR_HIP;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return ATTN_SINK_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return ATTN_SINK_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return ATTN_SINK_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return ATTN_SINK_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return ATTN_SINK_ERR_HIP;
    if (e != hipSuccess || p == nullptr) return ATTN_SINK_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ATTN_SINK_OK;
}

}  // namespace

extern "C" {

int attn_sink_fwd(const void* q, const void* k, const void* v, const float* sinks, int causal, int window,
                  const int32_t* cu_seqlens, const attn_sink_shape* shape, void* out, float* lse,
                  hipStream_t stream) {
  int rc = check_shape(shape, true);
  if (rc) return rc;
  if (sinks == nullptr || cu_seqlens == nullptr) return ATTN_SINK_ERR_NULL_PTR;
  const int T = shape->total_tokens;
  if (T > 0 && (!q || !k || !v || !out || !lse)) return ATTN_SINK_ERR_NULL_PTR;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return ATTN_SINK_ERR_ALIGN;

  FwdArgs a = {};
  a.q = static_cast<const __bf16*>(q);
  a.k = static_cast<const __bf16*>(k);
  a.v = static_cast<const __bf16*>(v);
  a.sinks = sinks;
  a.cu = cu_seqlens;
  a.out = out;
  a.out_bf16 = shape->out_dtype == ATTN_SINK_BF16 ? 1 : 0;
  a.lse = lse;
  a.T = T;
  a.B = shape->num_seqs;
  a.Hq = shape->num_heads_q;
  a.Hkv = shape->num_heads_kv;
  a.G = a.Hq / a.Hkv;
  a.hpw = heads_per_group_split(a.G);
  a.D = shape->head_dim;
  const int fwd_rows = fwd_rows_per_wave(a.D) * (4 / a.hpw);  // rows per forward workgroup
  a.n_qblocks = (shape->max_seqlen + fwd_rows - 1) / fwd_rows;
  a.causal = causal ? 1 : 0;
  a.window = clamp_window(window, shape->max_seqlen);
  a.scale_log2 = resolve_scale(shape) * kLog2e;
  return launch_fwd(a, stream) == hipSuccess ? ATTN_SINK_OK : ATTN_SINK_ERR_HIP;
}

size_t attn_sink_bwd_workspace_bytes(const attn_sink_shape* shape) {
  if (check_shape(shape) != ATTN_SINK_OK) return 0;
  return workspace_bytes(shape);
}

int attn_sink_bwd(const void* q, const void* k, const void* v, const float* sinks, const void* out, const float* lse,
                  const void* dout, int causal, int window, const int32_t* cu_seqlens, const attn_sink_shape* shape,
                  void* workspace, size_t workspace_bytes, float* dq, float* dk, float* dv, float* dsinks,
                  hipStream_t stream) {
  return bwd_impl(q, k, v, sinks, out, lse, dout, causal, window, cu_seqlens, shape, workspace, workspace_bytes, dq,
                  dk, dv, dsinks, stream, nullptr, 0);
}

int attn_sink_bwd_timed(const void* q, const void* k, const void* v, const float* sinks, const void* out,
                        const float* lse, const void* dout, int causal, int window, const int32_t* cu_seqlens,
                        const attn_sink_shape* shape, void* workspace, size_t workspace_bytes, float* dq, float* dk,
                        float* dv, float* dsinks, hipStream_t stream, void* const* events, int num_events) {
  return bwd_impl(q, k, v, sinks, out, lse, dout, causal, window, cu_seqlens, shape, workspace, workspace_bytes, dq,
                  dk, dv, dsinks, stream, events, num_events);
}

int attn_sink_bwd_noalloc(const void* q, const void* k, const void* v, const float* sinks, const void* out,
                          const float* lse, const void* dout, int causal, int window, const int32_t* cu_seqlens,
                          const attn_sink_shape* shape, float* dq, float* dk, float* dv, float* dsinks,
                          hipStream_t stream) {
  int rc = check_bwd_args(q, k, v, sinks, out, lse, dout, cu_seqlens, shape, dq, dk, dv, dsinks);
  if (rc) return rc;
  if (workspace_bytes(shape) > (size_t)ATTN_SINK_NOALLOC_SCRATCH_BYTES) return ATTN_SINK_ERR_SCRATCH;
  void* ws = nullptr;
  rc = scratch_address(stream, &ws);
  if (rc) return rc;
  return bwd_impl(q, k, v, sinks, out, lse, dout, causal, window, cu_seqlens, shape, ws,
                  (size_t)ATTN_SINK_NOALLOC_SCRATCH_BYTES, dq, dk, dv, dsinks, stream, nullptr, 0);
}

size_t attn_sink_decode_workspace_bytes(const attn_sink_decode_shape* shape) {
  if (check_decode_shape(shape) != ATTN_SINK_OK) return 0;
  return decode_workspace_bytes(shape);
}

int attn_sink_decode_fwd_timed(const void* q, const void* k, const void* v, const float* sinks, int window,
                               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                               const attn_sink_decode_shape* shape, void* workspace, size_t workspace_bytes, void* out,
                               float* lse, hipStream_t stream, void* const* events, int num_events) {
  int rc = check_decode_shape(shape);
  if (rc) return rc;
  if (events != nullptr && num_events != kDecodeNumKernels + 1) return ATTN_SINK_ERR_BAD_SHAPE;
  if (window < 0) return ATTN_SINK_ERR_BAD_WINDOW;
  if (sinks == nullptr || cu_seqlens_q == nullptr || cu_seqlens_k == nullptr) return ATTN_SINK_ERR_NULL_PTR;
  if (shape->total_q > 0 && (!q || !out || !lse)) return ATTN_SINK_ERR_NULL_PTR;
  if (shape->total_k > 0 && (!k || !v)) return ATTN_SINK_ERR_NULL_PTR;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return ATTN_SINK_ERR_ALIGN;
  const size_t need = decode_workspace_bytes(shape);
  if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)) return ATTN_SINK_ERR_WORKSPACE;
  hipEvent_t const* ev = reinterpret_cast<hipEvent_t const*>(events);
  if (shape->total_q == 0) {  // nothing to compute; the events still mark the (empty) interval
    for (int i = 0; ev && i <= kDecodeNumKernels; ++i) {
      if (ev[i] && hipEventRecord(ev[i], stream) != hipSuccess) return ATTN_SINK_ERR_HIP;
    }
    return ATTN_SINK_OK;
  }

  DecodeArgs a = {};
  a.q = static_cast<const __bf16*>(q);
  a.k = static_cast<const __bf16*>(k);
  a.v = static_cast<const __bf16*>(v);
  a.sinks = sinks;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.out = out;
  a.lse = lse;
  decode_chunks(shape, window, &a.n_chunks, &a.chunk_keys);
  a.part_o = static_cast<float*>(workspace);
  a.part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + decode_part_o_bytes(shape, a.n_chunks));
  a.Tq = shape->total_q;
  a.B = shape->num_seqs;
  a.Hq = shape->num_heads_q;
  a.Hkv = shape->num_heads_kv;
  a.G = a.Hq / a.Hkv;
  a.n_cols = shape->max_q * a.G;
  a.n_cg = decode_col_groups(shape);
  a.window = clamp_window(window, shape->max_k);
  a.out_bf16 = shape->out_dtype == ATTN_SINK_BF16 ? 1 : 0;
  a.D = shape->head_dim;
  a.scale_log2 = resolve_decode_scale(shape) * kLog2e;
  return launch_decode(a, stream, ev) == hipSuccess ? ATTN_SINK_OK : ATTN_SINK_ERR_HIP;
}

int attn_sink_decode_fwd(const void* q, const void* k, const void* v, const float* sinks, int window,
                         const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, const attn_sink_decode_shape* shape,
                         void* workspace, size_t workspace_bytes, void* out, float* lse, hipStream_t stream) {
  return attn_sink_decode_fwd_timed(q, k, v, sinks, window, cu_seqlens_q, cu_seqlens_k, shape, workspace,
                                    workspace_bytes, out, lse, stream, nullptr, 0);
}

int attn_sink_decode_fwd_ordered(const void* q, const void* k, const void* v, const float* sinks, int window,
                                 const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                 const attn_sink_decode_shape* shape, void* out, float* lse, hipStream_t stream) {
  int rc = check_decode_shape(shape);
  if (rc) return rc;
  if (window < 0) return ATTN_SINK_ERR_BAD_WINDOW;
  if (sinks == nullptr || cu_seqlens_q == nullptr || cu_seqlens_k == nullptr) return ATTN_SINK_ERR_NULL_PTR;
  if (shape->total_q > 0 && (!q || !out || !lse)) return ATTN_SINK_ERR_NULL_PTR;
  if (shape->total_k > 0 && (!k || !v)) return ATTN_SINK_ERR_NULL_PTR;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return ATTN_SINK_ERR_ALIGN;
  if (shape->total_q == 0) return ATTN_SINK_OK;

  DecodeArgs a = {};
  a.q = static_cast<const __bf16*>(q);
  a.k = static_cast<const __bf16*>(k);
  a.v = static_cast<const __bf16*>(v);
  a.sinks = sinks;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.out = out;
  a.lse = lse;
  a.Tq = shape->total_q;
  a.B = shape->num_seqs;
  a.Hq = shape->num_heads_q;
  a.Hkv = shape->num_heads_kv;
  a.G = a.Hq / a.Hkv;
  a.n_cols = shape->max_q * a.G;
  a.n_cg = decode_col_groups(shape);
  a.window = clamp_window(window, shape->max_k);
  a.out_bf16 = shape->out_dtype == ATTN_SINK_BF16 ? 1 : 0;
  a.D = shape->head_dim;
  a.scale_log2 = resolve_decode_scale(shape) * kLog2e;
  return launch_decode_ordered(a, stream) == hipSuccess ? ATTN_SINK_OK : ATTN_SINK_ERR_HIP;
}

int attn_sink_decode_num_kernels(void) { return kDecodeNumKernels; }

const char* attn_sink_decode_kernel_name(int i) {
  static const char* const names[kDecodeNumKernels] = {"attn_sink_decode_partial_kernel",
                                                        "attn_sink_decode_combine_kernel"};
  return (i >= 0 && i < kDecodeNumKernels) ? names[i] : nullptr;
}

int attn_sink_check_cu_seqlens(const int32_t* cu, int32_t num_seqs, int32_t total_tokens, int32_t max_seqlen) {
  if (cu == nullptr) return ATTN_SINK_ERR_NULL_PTR;
  if (num_seqs < 1 || total_tokens < 0 || max_seqlen < 0) return ATTN_SINK_ERR_BAD_SHAPE;
  if (cu[0] != 0 || cu[num_seqs] != total_tokens) return ATTN_SINK_ERR_BAD_SEQLENS;
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int64_t len = (int64_t)cu[b + 1] - cu[b];
    if (len < 0 || len > max_seqlen) return ATTN_SINK_ERR_BAD_SEQLENS;
  }
  return ATTN_SINK_OK;
}

int attn_sink_bwd_num_kernels(void) { return kBwdNumKernels; }

const char* attn_sink_bwd_kernel_name(int i) {
  static const char* const names[kBwdNumKernels] = {"attn_sink_bwd_dq_kernel", "attn_sink_bwd_dkdv_kernel",
                                                    "attn_sink_bwd_finish_kernel"};
  return (i >= 0 && i < kBwdNumKernels) ? names[i] : nullptr;
}

const char* attn_sink_strerror(int code) {
  switch (code) {
    case ATTN_SINK_OK: return "success";
    case ATTN_SINK_ERR_NULL_PTR: return "a required pointer is NULL";
    case ATTN_SINK_ERR_BAD_SHAPE: return "invalid shape (sizes, head counts or max_seqlen)";
    case ATTN_SINK_ERR_UNSUPPORTED:
      return "unsupported head_dim or output dtype (head_dim 64 or 128; float32 outputs, bf16 also for forwards)";
    case ATTN_SINK_ERR_BAD_WINDOW: return "negative window";
    case ATTN_SINK_ERR_WORKSPACE:
      return "workspace missing, not 16-byte aligned, or smaller than attn_sink_bwd_workspace_bytes() "
             "(attn_sink_decode_workspace_bytes() for the decode forward)";
    case ATTN_SINK_ERR_HIP: return "a HIP launch failed";
    case ATTN_SINK_ERR_ALIGN: return "a tensor base pointer is not 16-byte aligned";
    case ATTN_SINK_ERR_SCRATCH:
      return "attn_sink_bwd_noalloc: the shape needs more workspace than its static scratch holds "
             "(attn_sink_bwd_workspace_bytes > ATTN_SINK_NOALLOC_SCRATCH_BYTES); use attn_sink_bwd";
    case ATTN_SINK_ERR_BAD_SEQLENS:
      return "cu_seqlens: not 0 at the start, decreasing, not ending at total_tokens, or a length above max_seqlen";
    default: return "unknown error code";
  }
}

}  // extern "C"
