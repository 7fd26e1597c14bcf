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
// keys (32 at head_dim 128) streamed through a 3-slot LDS ring of swizzled tiles (direct global->LDS copies two tiles
// ahead, transposing reads for V^T; see common.h). It writes the chunk's running max (log2
// units), denominator and unnormalised output per column. attn_sink_decode_combine_kernel merges
// the chunks of a (sequence, KV head, column) and adds the sink once: with M = max(S_h log2e, m_c),
// l = 2^(S_h log2e - M) + sum_c 2^(m_c - M) l_c and O = sum_c 2^(m_c - M) o_c / l; LSE = (M +
// log2 l) ln 2. O is stored in fp32 or bf16.
#include "kernels.h"

namespace attn_sink {

namespace {

constexpr int kDecTileBytes = 8192;              // one swizzled K or V tile (64 keys at D = 64, 32 at D = 128)
constexpr int kDecSlotBytes = 2 * kDecTileBytes;  // K tile, then V tile
constexpr int kDecRing = 3;

// Head dim D = 64 or 128 (rows as 64-element panels in 8 KiB tiles; see Geo in common.h). Key chunks
// are whole numbers of 64 keys for either D.
template <int D>
__global__ __launch_bounds__(64) void attn_sink_decode_partial_kernel(DecodeArgs a) {
  using G_ = Geo<D>;
  constexpr int kDecTileKeys = G_::kTileRows;
  constexpr int MB = G_::kRowBlocks;
  constexpr int NTR = G_::kDBlocks * MB * 4;
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
  const int k_base = k_vis & ~63;
  const int k_lo = max(k_vis, k_base + chunk * a.chunk_keys);
  const int k_hi = min(lk, k_base + (chunk + 1) * a.chunk_keys);

  float m = kNegInf, lsum = 0.0f;  // running max (log2 units) and denominator, without the sink
  f32x16 o[G_::kDBlocks];
#pragma unroll
  for (int db = 0; db < G_::kDBlocks; ++db) o[db] = zero_f32x16();

  if (nq > 0 && k_lo < k_hi) {
    // Q^T as the B operand: lane holds column l32, d = 16c + 8grp + (0..7).
    bf16x8 qf[G_::kChunks];
#pragma unroll
    for (int c = 0; c < G_::kChunks; ++c) {
      qf[c] = load_bf16x8(a.q + ((size_t)(cq + min(j, nq - 1)) * a.Hq + hq) * D + 16 * c + 8 * grp);
    }
    const int kv_stride = a.Hkv * D;
    const __bf16* kbase = a.k + (size_t)ck * kv_stride + (size_t)g * D;
    const __bf16* vbase = a.v + (size_t)ck * kv_stride + (size_t)g * D;
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
          tile_copy_full_d<D>(rk, coff, row_bytes, slot, u);
          tile_copy_full_d<D>(rv, coff, row_bytes, slot + kDecTileBytes, u);
        }
      } else {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          tile_copy_d<D>(kbase, row0, lk - 1, kv_stride, slot, u, lane);
          tile_copy_d<D>(vbase, row0, lk - 1, kv_stride, slot + kDecTileBytes, u, lane);
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

      f32x16 s[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        s[mb] = zero_f32x16();
#pragma unroll
        for (int c = 0; c < G_::kChunks; ++c) {
          s[mb] = mfma_32x32x16(*reinterpret_cast<const bf16x8*>(slot + frag_off<D>(aoff, c, mb)), qf[c], s[mb]);
        }
      }
      // Per element: the key must lie in the chunk's range, exist, and be visible from the column.
      // Columns past the last (query, head) pair repeat the last query and are never stored.
      const bool need_mask =
          k0 < k_lo || k0 + kDecTileKeys > k_hi || k0 + kDecTileKeys - 1 > lk - nq || a.window > 0;
      if (need_mask) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
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
      for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) t = fmaxf(t, s[mb][i]);
      }
      const float tmax = max_xor32(t) * a.scale_log2;
      if (wave_any(tmax > m)) {
        const float mnew = fmaxf(m, tmax);
        const float alpha = mnew == kNegInf ? 1.0f : fast_exp2(m - mnew);
        lsum *= alpha;
#pragma unroll
        for (int db = 0; db < G_::kDBlocks; ++db) o[db] *= alpha;
        m = mnew;
      }
      const float moff = m == kNegInf ? 0.0f : m;  // nothing visible yet: exp2(-inf) = 0
      bf16x8 pb[MB][2];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = fast_exp2(__builtin_fmaf(s[mb][i], a.scale_log2, -moff));
          s[mb][i] = p;
          lsum += p;
        }
        pb[mb][0] = pack8(s[mb], 0);
        pb[mb][1] = pack8(s[mb], 1);
      }
      // V^T operands: tr[4 (db MB + mb) + 2 cc + lo/hi], from panel db / 2 at rows 32mb + 16cc.
      u32x2 tr[NTR];
      static_for<G_::kDBlocks>([&](auto db_tag) {
        constexpr int db = decltype(db_tag)::value;
        constexpr int PO = (db / 2) * G_::kPanelBytes;
        static_for<MB>([&](auto mb_tag) {
          constexpr int mb = decltype(mb_tag)::value;
          tr[4 * (db * MB + mb) + 0] = ds_read_tr16_b64_asm<PO + 4096 * mb>(vt_lds + toff[db % 2][0]);
          tr[4 * (db * MB + mb) + 1] = ds_read_tr16_b64_asm<PO + 4096 * mb>(vt_lds + toff[db % 2][1]);
          tr[4 * (db * MB + mb) + 2] = ds_read_tr16_b64_asm<PO + 4096 * mb + 2048>(vt_lds + toff[db % 2][0]);
          tr[4 * (db * MB + mb) + 3] = ds_read_tr16_b64_asm<PO + 4096 * mb + 2048>(vt_lds + toff[db % 2][1]);
        });
      });
      wait_lds_into(tr);
#pragma unroll
      for (int db = 0; db < G_::kDBlocks; ++db) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
          for (int cc = 0; cc < 2; ++cc) {
            const u32x2* tt = tr + 4 * (db * MB + mb) + 2 * cc;
            o[db] = mfma_32x32x16(join_tr(tt[0], tt[1]), pb[mb][cc], o[db]);
          }
        }
      }
    }
  }

  // This chunk's partial: running max, denominator, unnormalised output per column. Only the
  // columns of real (query, head) pairs are stored; the combine reads no other.
  const float ltot = sum_xor32(lsum);
  float* po = a.part_o + (size_t)pidx * 32 * D + l32 * D;  // [32 columns][D]
  float* pml = a.part_ml + (size_t)pidx * 2 * 32;                        // [max, denominator][32 columns]
  if (col_ok) {
#pragma unroll
    for (int db = 0; db < G_::kDBlocks; ++db) {
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

// One workgroup per (sequence, KV head, column): lane l of each of the four waves accumulates
// output elements l, l + 64, ... (D / 64 of them) over every fourth chunk; the waves' sums meet in
// LDS.
constexpr int kCombineWaves = 4;

template <int D>
__global__ __launch_bounds__(64 * kCombineWaves) void attn_sink_decode_combine_kernel(DecodeArgs a) {
  constexpr int E = D / 64;  // output elements per lane
  __shared__ float red[kCombineWaves][D + 1];
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
  if (lane == 0) red[w][D] = M;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kCombineWaves; ++i) M = fmaxf(M, red[i][D]);
  const float Ms = M == kNegInf ? 0.0f : M;
  __syncthreads();  // red[.][D] is reused below

  float acc[E], L = 0.0f;
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.0f;
  const float* po = a.part_o + p0 * 32 * D + (c % 32) * D + lane;
#pragma unroll 4
  for (int ch = w; ch < a.n_chunks; ch += kCombineWaves) {
    const float wt = fast_exp2(ml[(size_t)ch * 64] - Ms);  // 0 for an empty chunk (max -inf)
    L += wt * ml[(size_t)ch * 64 + 32];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] += wt * po[(size_t)ch * 32 * D + 64 * e];
  }
#pragma unroll
  for (int e = 0; e < E; ++e) red[w][lane + 64 * e] = acc[e];
  if (lane == 0) red[w][D] = L;
  __syncthreads();
  if (w != 0) return;
  L = fast_exp2(sink2 - Ms);
#pragma unroll
  for (int i = 0; i < kCombineWaves; ++i) L += red[i][D];
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  const size_t row = (size_t)(cq + j) * a.Hq + hq;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    float x = 0.0f;
#pragma unroll
    for (int i = 0; i < kCombineWaves; ++i) x += red[i][lane + 64 * e];
    if (a.out_bf16) {
      static_cast<__bf16*>(a.out)[row * D + lane + 64 * e] = (__bf16)(x * inv);
    } else {
      static_cast<float*>(a.out)[row * D + lane + 64 * e] = x * inv;
    }
  }
  if (lane == 0) a.lse[(size_t)hq * a.Tq + cq + j] = L > 0.0f ? (Ms + fast_log2(L)) * kLn2 : kNegInf;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream, hipEvent_t const* events) {
  const long long parts = (long long)a.B * a.Hkv * a.n_cg * a.n_chunks;
  if (parts <= 0) return hipSuccess;
  hipError_t e;
  if (events && events[0] && (e = hipEventRecord(events[0], stream)) != hipSuccess) return e;
  if (a.D == 128) {
    hipLaunchKernelGGL(attn_sink_decode_partial_kernel<128>, dim3((unsigned)parts), dim3(64), 0, stream, a);
  } else {
    hipLaunchKernelGGL(attn_sink_decode_partial_kernel<64>, dim3((unsigned)parts), dim3(64), 0, stream, a);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (events && events[1] && (e = hipEventRecord(events[1], stream)) != hipSuccess) return e;
  const dim3 cgrid((unsigned)(a.B * a.Hkv * a.n_cols)), cblock(64 * kCombineWaves);
  if (a.D == 128) {
    hipLaunchKernelGGL(attn_sink_decode_combine_kernel<128>, cgrid, cblock, 0, stream, a);
  } else {
    hipLaunchKernelGGL(attn_sink_decode_combine_kernel<64>, cgrid, cblock, 0, stream, a);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (events && events[2] && (e = hipEventRecord(events[2], stream)) != hipSuccess) return e;
  return hipSuccess;
}

}  // namespace attn_sink
