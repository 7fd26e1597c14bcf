// Host-side launchers of the sink-attention kernels (one translation unit per pass).
#pragma once

#include "common.h"

namespace attn_sink {

// Queries per wave in the forward: 64 at head_dim 64, 32 at head_dim 128.
constexpr int fwd_rows_per_wave(int head_dim) { return head_dim == 128 ? 32 : 64; }
constexpr int kDqRowsPerWave = 32;    // queries per wave in the row-parallel dQ / dSink pass
constexpr int kKvKeysPerBlock = 64;   // keys per workgroup in the column-parallel dK / dV pass

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);

// Backward passes, in enqueue order.
constexpr int kBwdNumKernels = 3;
constexpr int kDecodeNumKernels = 2;  // partial, combine
constexpr int kDecodeMaxCols = 1024;  // (new token, query head) pairs per KV head: max_q * Hq / Hkv
hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t stream);      // dQ, -D_i, -LSE/scale, dSink partials
hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t stream);    // dK, dV (or partials per head half); dSink without halves
hipError_t launch_bwd_finish(const BwdArgs& a, hipStream_t stream);  // with head halves: dK, dV = sum of halves; dSink

// Inference-shaped forward: per-chunk partials, then the combine with the sink.
// events: NULL, or kDecodeNumKernels + 1 events recorded before, between and after the kernels
// (a NULL entry records nothing at that point).
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream, hipEvent_t const* events);

// Decode forward in the training forward's key order (no split over the keys, no workspace); uses
// q, k, v, sinks, cu_q, cu_k, out, lse, B, Hq, Hkv, G, n_cg, window, out_bf16, scale_log2, D.
hipError_t launch_decode_ordered(const DecodeArgs& a, hipStream_t stream);

}  // namespace attn_sink
