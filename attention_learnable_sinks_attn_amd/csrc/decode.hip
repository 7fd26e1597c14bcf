// Inference-shaped (decode) forward of attention with a learnable per-head sink, for gfx950.
//
// Each packed sequence b has Lk_b cached keys / values and its last Nq_b tokens as new queries;
// new query j sits at position Lk_b - Nq_b + j and sees the keys at positions <= its own (and,
// with a window W, > position - W), plus the sink (nmedialink.com "惊爆！GPT-OSS-20B强化学习…",
// section "GPT-OSS中的带注意力槽的注意力机制": the sink is one more logit in each row's softmax
// with no value row; section "数学公式深入解读", eq. P_ij).
//
// Split over the key axis. attn_sink_decode_partial_kernel: one wave per (sequence, KV head,
// group of 32 columns, chunk of keys). The columns are the group's (new query, query head) pairs,
// column c = j * G + (query head - g * G) for new token j, taken 32 at a time as the wave's MFMA
// columns, so the G query heads of a KV head share every K and V tile: S^T = K Q^T (32x32x16 MFMA, keys on the C
// rows), a sink-free online softmax per column (lane), O^T += V^T P^T, with K and V tiles of 64
// keys streamed through a 3-slot LDS ring of swizzled tiles (direct global->LDS copies two tiles
// ahead, transposing reads for V^T; see common.h). It writes the chunk's running max (log2
// units), denominator and unnormalised output per column. attn_sink_decode_combine_kernel merges
// the chunks of a (sequence, KV head, column) and adds the sink once: with M = max(S_h log2e, m_c),
// l = 2^(S_h log2e - M) + sum_c 2^(m_c - M) l_c and O = sum_c 2^(m_c - M) o_c / l; LSE = (M +
// log2 l) ln 2. O is stored in fp32 or bf16.
#include "kernels.h"

namespace attn_sink {

namespace {

constexpr int kDecTileKeys = 64;
constexpr int kDecTileBytes = kDecTileKeys * kHeadDim * 2;  // one swizzled 64-key tile (K or V)
constexpr int kDecSlotBytes = 2 * kDecTileBytes;             // K tile, then V tile
constexpr int kDecRing = 3;

__global__ __launch_bounds__(64) void attn_sink_decode_partial_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kDecRing * kDecSlotBytes];

  // The KV heads of one chunk of keys are neighbours in the launch, so that the rows they share
  // are read from HBM at about the same time; then the column groups of the same chunk.
  const int g = blockIdx.x % a.Hkv;
  const int rest = blockIdx.x / a.Hkv;  // = (b * n_cg + cg) * n_chunks + chunk
  const int chunk = rest % a.n_chunks;
  const int cg = (rest / a.n_chunks) % a.n_cg;
  const int b = rest / a.n_chunks / a.n_cg;
  const int pidx = ((b * a.Hkv + g) * a.n_cg + cg) * a.n_chunks + chunk;  // the partial's index
  const int cq = a.cu_q[b];
  const int nq = a.cu_q[b + 1] - cq;
  const int ck = a.cu_k[b];
  const int lk = a.cu_k[b + 1] - ck;

  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31;
  const int grp = lane >> 5;
  const int col = 32 * cg + l32;
  const int j = col / a.G;                 // column = (new query j, query head g*G + col % G)
  const int hq = g * a.G + col % a.G;
  const bool col_ok = j < nq;              // columns past the last pair repeat the last query
  const int pos = lk - nq + min(j, nq - 1);  // the column's query position (< 0: sees no key)

  // Keys of this chunk that some column can see. Chunks tile the keys from the 64-aligned start of
  // the first one any new query sees (key 0 without a window).
  const int k_vis = a.window > 0 ? max(0, lk - nq - a.window + 1) : 0;
  const int k_base = k_vis & ~(kDecTileKeys - 1);
  const int k_lo = max(k_vis, k_base + chunk * a.chunk_keys);
  const int k_hi = min(lk, k_base + (chunk + 1) * a.chunk_keys);

  float m = kNegInf, lsum = 0.0f;  // running max (log2 units) and denominator, without the sink
  f32x16 o[2];
  o[0] = o[1] = zero_f32x16();

  if (nq > 0 && k_lo < k_hi) {
    // Q^T as the B operand: lane holds column l32, d = 16c + 8grp + (0..7).
    bf16x8 qf[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      qf[c] = load_bf16x8(a.q + ((size_t)(cq + min(j, nq - 1)) * a.Hq + hq) * kHeadDim + 16 * c + 8 * grp);
    }
    const int kv_stride = a.Hkv * kHeadDim;
    const __bf16* kbase = a.k + (size_t)ck * kv_stride + (size_t)g * kHeadDim;
    const __bf16* vbase = a.v + (size_t)ck * kv_stride + (size_t)g * kHeadDim;
    // Full tiles go through buffer resources; in a partial last tile, keys past the end repeat
    // the last key (finite data; they are masked).
    const unsigned row_bytes = 2u * kv_stride;
    unsigned coff[2];
    tile_copy_offsets(lane, row_bytes, coff);
    auto issue = [&](int kt) {
      unsigned char* slot = ring + (kt % kDecRing) * kDecSlotBytes;
      const int row0 = kt * kDecTileKeys;
      if (row0 + kDecTileKeys <= lk) {
        const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(kbase + (size_t)row0 * kv_stride, kDecTileKeys * row_bytes);
        const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(vbase + (size_t)row0 * kv_stride, kDecTileKeys * row_bytes);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          tile_copy_full(rk, coff, row_bytes, slot, u);
          tile_copy_full(rv, coff, row_bytes, slot + kDecTileBytes, u);
        }
      } else {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          tile_copy(kbase, row0, lk - 1, kv_stride, slot, u, lane);
          tile_copy(vbase, row0, lk - 1, kv_stride, slot + kDecTileBytes, u, lane);
        }
      }
    };
    int aoff[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) aoff[c] = tile_frag_off(l32, grp, c);
    int toff[2][2];
    tile_tr_offsets(lane, toff);
    const unsigned ring_lds = lds_addr(ring);

    const int kt_begin = k_lo / kDecTileKeys;
    const int kt_end = (k_hi + kDecTileKeys - 1) / kDecTileKeys;
    issue(kt_begin);
    if (kt_begin + 1 < kt_end) issue(kt_begin + 1);
    for (int kt = kt_begin; kt < kt_end; ++kt) {
      if (kt + 1 < kt_end) {
        wait_vmcnt<16>();  // the copies of tile kt (those of kt + 1 may stay in flight)
      } else {
        wait_vmcnt<0>();
      }
      __syncthreads();
      if (kt + 2 < kt_end) issue(kt + 2);
      const unsigned char* slot = ring + (kt % kDecRing) * kDecSlotBytes;
      const unsigned vt_lds = ring_lds + (kt % kDecRing) * kDecSlotBytes + kDecTileBytes;
      const int k0 = kt * kDecTileKeys;

      f32x16 s[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        s[mb] = zero_f32x16();
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          s[mb] = mfma_32x32x16(*reinterpret_cast<const bf16x8*>(slot + 4096 * mb + aoff[c]), qf[c], s[mb]);
        }
      }
      // Per element: the key must lie in the chunk's range, exist, and be visible from the column.
      // Columns past the last (query, head) pair repeat the last query and are never stored.
      const bool need_mask =
          k0 < k_lo || k0 + kDecTileKeys > k_hi || k0 + kDecTileKeys - 1 > lk - nq || a.window > 0;
      if (need_mask) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int kj = k0 + 32 * mb + c_row(i, grp);
            const bool vis = (kj >= k_lo) & (kj < k_hi) & (kj <= pos) & ((a.window <= 0) | (kj > pos - a.window));
            s[mb][i] = vis ? s[mb][i] : kNegInf;
          }
        }
      }
      float t = kNegInf;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) t = fmaxf(t, s[mb][i]);
      }
      const float tmax = max_xor32(t) * a.scale_log2;
      if (wave_any(tmax > m)) {
        const float mnew = fmaxf(m, tmax);
        const float alpha = mnew == kNegInf ? 1.0f : fast_exp2(m - mnew);
        lsum *= alpha;
        o[0] *= alpha;
        o[1] *= alpha;
        m = mnew;
      }
      const float moff = m == kNegInf ? 0.0f : m;  // nothing visible yet: exp2(-inf) = 0
      bf16x8 pb[2][2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = fast_exp2(__builtin_fmaf(s[mb][i], a.scale_log2, -moff));
          s[mb][i] = p;
          lsum += p;
        }
        pb[mb][0] = pack8(s[mb], 0);
        pb[mb][1] = pack8(s[mb], 1);
      }
      u32x2 tr[16];  // V^T operands: [d block][key block][half][lo / hi]
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        tr[8 * db + 0] = ds_read_tr16_b64_asm<0>(vt_lds + toff[db][0]);
        tr[8 * db + 1] = ds_read_tr16_b64_asm<0>(vt_lds + toff[db][1]);
        tr[8 * db + 2] = ds_read_tr16_b64_asm<2048>(vt_lds + toff[db][0]);
        tr[8 * db + 3] = ds_read_tr16_b64_asm<2048>(vt_lds + toff[db][1]);
        tr[8 * db + 4] = ds_read_tr16_b64_asm<4096>(vt_lds + toff[db][0]);
        tr[8 * db + 5] = ds_read_tr16_b64_asm<4096>(vt_lds + toff[db][1]);
        tr[8 * db + 6] = ds_read_tr16_b64_asm<6144>(vt_lds + toff[db][0]);
        tr[8 * db + 7] = ds_read_tr16_b64_asm<6144>(vt_lds + toff[db][1]);
      }
      wait_lds_into(tr);
#pragma unroll
      for (int db = 0; db < 2; ++db) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
          for (int cc = 0; cc < 2; ++cc) {
            const u32x2* tt = tr + 8 * db + 4 * mb + 2 * cc;
            o[db] = mfma_32x32x16(join_tr(tt[0], tt[1]), pb[mb][cc], o[db]);
          }
        }
      }
    }
  }

  // This chunk's partial: running max, denominator, unnormalised output per column. Only the
  // columns of real (query, head) pairs are stored; the combine reads no other.
  const float ltot = sum_xor32(lsum);
  float* po = a.part_o + (size_t)pidx * 32 * kHeadDim + l32 * kHeadDim;  // [32 columns][64 d]
  float* pml = a.part_ml + (size_t)pidx * 2 * 32;                        // [max, denominator][32 columns]
  if (col_ok) {
#pragma unroll
    for (int db = 0; db < 2; ++db) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        *reinterpret_cast<f32x4*>(po + 32 * db + 8 * r4 + 4 * grp) =
            (f32x4){o[db][4 * r4], o[db][4 * r4 + 1], o[db][4 * r4 + 2], o[db][4 * r4 + 3]};
      }
    }
  }
  if (grp == 0) {
    pml[l32] = m;
    pml[32 + l32] = ltot;
  }
}

// One workgroup per (sequence, KV head, column): lane d of each of the four waves accumulates
// output element d over every fourth chunk; the waves' sums meet in LDS.
constexpr int kCombineWaves = 4;

__global__ __launch_bounds__(64 * kCombineWaves) void attn_sink_decode_combine_kernel(DecodeArgs a) {
  __shared__ float red[kCombineWaves][kHeadDim + 1];
  const int c = blockIdx.x % a.n_cols;
  const int rest = blockIdx.x / a.n_cols;  // = b * Hkv + g
  const int g = rest % a.Hkv;
  const int b = rest / a.Hkv;
  const int cq = a.cu_q[b];
  const int nq = a.cu_q[b + 1] - cq;
  const int j = c / a.G;
  if (j >= nq) return;  // uniform over the workgroup
  const int hq = g * a.G + c % a.G;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  // First partial of this (sequence, KV head, column group); chunk ch: max at ml[64 ch],
  // denominator at ml[64 ch + 32].
  const size_t p0 = ((size_t)rest * a.n_cg + c / 32) * a.n_chunks;
  const float* ml = a.part_ml + p0 * 64 + c % 32;

  // Largest running max over the chunks and the sink (log2 units).
  const float sink2 = a.sinks[hq] * kLog2e;
  float M = sink2;
  for (int ch = threadIdx.x; ch < a.n_chunks; ch += 64 * kCombineWaves) M = fmaxf(M, ml[(size_t)ch * 64]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  if (lane == 0) red[w][kHeadDim] = M;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kCombineWaves; ++i) M = fmaxf(M, red[i][kHeadDim]);
  const float Ms = M == kNegInf ? 0.0f : M;
  __syncthreads();  // red[.][kHeadDim] is reused below

  float acc = 0.0f, L = 0.0f;
  const float* po = a.part_o + p0 * 32 * kHeadDim + (c % 32) * kHeadDim + lane;
#pragma unroll 4
  for (int ch = w; ch < a.n_chunks; ch += kCombineWaves) {
    const float wt = fast_exp2(ml[(size_t)ch * 64] - Ms);  // 0 for an empty chunk (max -inf)
    L += wt * ml[(size_t)ch * 64 + 32];
    acc += wt * po[(size_t)ch * 32 * kHeadDim];
  }
  red[w][lane] = acc;
  if (lane == 0) red[w][kHeadDim] = L;
  __syncthreads();
  if (w != 0) return;
  L = fast_exp2(sink2 - Ms);
#pragma unroll
  for (int i = 0; i < kCombineWaves; ++i) L += red[i][kHeadDim];
  acc = 0.0f;
#pragma unroll
  for (int i = 0; i < kCombineWaves; ++i) acc += red[i][lane];
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  const size_t row = (size_t)(cq + j) * a.Hq + hq;
  if (a.out_bf16) {
    static_cast<__bf16*>(a.out)[row * kHeadDim + lane] = (__bf16)(acc * inv);
  } else {
    static_cast<float*>(a.out)[row * kHeadDim + lane] = acc * inv;
  }
  if (lane == 0) a.lse[(size_t)hq * a.Tq + cq + j] = L > 0.0f ? (Ms + fast_log2(L)) * kLn2 : kNegInf;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream, hipEvent_t const* events) {
  const long long parts = (long long)a.B * a.Hkv * a.n_cg * a.n_chunks;
  if (parts <= 0) return hipSuccess;
  hipError_t e;
  if (events && events[0] && (e = hipEventRecord(events[0], stream)) != hipSuccess) return e;
  hipLaunchKernelGGL(attn_sink_decode_partial_kernel, dim3((unsigned)parts), dim3(64), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (events && events[1] && (e = hipEventRecord(events[1], stream)) != hipSuccess) return e;
  hipLaunchKernelGGL(attn_sink_decode_combine_kernel, dim3((unsigned)(a.B * a.Hkv * a.n_cols)),
                     dim3(64 * kCombineWaves), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (events && events[2] && (e = hipEventRecord(events[2], stream)) != hipSuccess) return e;
  return hipSuccess;
}

}  // namespace attn_sink
