// Inference-shaped (decode) forward of attention with a learnable per-head sink, for gfx950.
//
// Each packed sequence b has Lk_b cached keys / values and its last Nq_b tokens as new queries;
// new query j sits at position Lk_b - Nq_b + j and sees the keys at positions <= its own (and,
// with a window W, > position - W), plus the sink (nmedialink.com "惊爆！GPT-OSS-20B强化学习…",
// section "GPT-OSS中的带注意力槽的注意力机制": the sink is one more logit in each row's softmax
// with no value row; section "数学公式深入解读", eq. P_ij).
//
// Split over the key axis. attn_sink_decode_partial_kernel: one wave per (sequence, KV head,
// chunk of keys). Its 32 MFMA columns are the group's (new query, query head) pairs, so the G
// query heads of a KV head share every K and V tile: S^T = K Q^T (32x32x16 MFMA, keys on the C
// rows), a sink-free online softmax per column (lane), O^T += V^T P^T, with K and V tiles of 64
// keys streamed through a 3-slot LDS ring of swizzled tiles (direct global->LDS copies two tiles
// ahead, transposing reads for V^T; see common.h). It writes the chunk's running max (log2
// units), denominator and unnormalised output per column. attn_sink_decode_combine_kernel merges
// the chunks of a (sequence, KV head) and adds the sink once: with M = max(S_h log2e, m_c),
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

  const int bid = blockIdx.x;  // = (b * Hkv + g) * n_chunks + chunk: the partial's index
  const int chunk = bid % a.n_chunks;
  const int rest = bid / a.n_chunks;
  const int g = rest % a.Hkv;
  const int b = rest / a.Hkv;
  const int cq = a.cu_q[b];
  const int nq = a.cu_q[b + 1] - cq;
  const int ck = a.cu_k[b];
  const int lk = a.cu_k[b + 1] - ck;

  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31;
  const int grp = lane >> 5;
  const int j = l32 / a.G;                 // column = (new query j, query head g*G + l32 % G)
  const int hq = g * a.G + l32 % a.G;
  const bool col_ok = j < nq;              // nq * G <= 32 (checked on the host)
  const int pos = lk - nq + min(j, nq - 1);  // the column's query position (< 0: sees no key)

  // Keys of this chunk that some column can see.
  int k_lo = chunk * a.chunk_keys;
  const int k_hi = min(lk, (chunk + 1) * a.chunk_keys);
  if (a.window > 0) k_lo = max(k_lo, lk - nq - a.window + 1);

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
    auto issue = [&](int kt) {
      unsigned char* slot = ring + (kt % kDecRing) * kDecSlotBytes;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        tile_copy(kbase, kt * kDecTileKeys, lk - 1, kv_stride, slot, u, lane);
        tile_copy(vbase, kt * kDecTileKeys, lk - 1, kv_stride, slot + kDecTileBytes, u, lane);
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
      const bool need_mask = k0 < k_lo || k0 + kDecTileKeys > k_hi || k0 + kDecTileKeys - 1 > lk - nq ||
                             a.window > 0 || nq * a.G < 32;
      if (need_mask) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int kj = k0 + 32 * mb + c_row(i, grp);
            const bool vis = col_ok & (kj >= k_lo) & (kj < k_hi) & (kj <= pos) &
                             ((a.window <= 0) | (kj > pos - a.window));
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

  // This chunk's partial: running max, denominator, unnormalised output per column.
  const float ltot = sum_xor32(lsum);
  float* po = a.part_o + (size_t)bid * kHeadDim * 32;  // [64 d][32 columns]
  float* pml = a.part_ml + (size_t)bid * 2 * 32;        // [max, denominator][32 columns]
#pragma unroll
  for (int db = 0; db < 2; ++db) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int d = 32 * db + 8 * (i >> 2) + 4 * grp + (i & 3);
      po[d * 32 + l32] = o[db][i];
    }
  }
  if (grp == 0) {
    pml[l32] = m;
    pml[32 + l32] = ltot;
  }
}

// One workgroup per (sequence, KV head): thread t merges column t % 32 for d = 8(t/32) .. +7.
__global__ __launch_bounds__(256) void attn_sink_decode_combine_kernel(DecodeArgs a) {
  const int g = blockIdx.x % a.Hkv;
  const int b = blockIdx.x / a.Hkv;
  const int cq = a.cu_q[b];
  const int nq = a.cu_q[b + 1] - cq;
  const int c = threadIdx.x & 31;
  const int dg = threadIdx.x >> 5;
  const int j = c / a.G;
  if (j >= nq) return;
  const int hq = g * a.G + c % a.G;
  const size_t p0 = (size_t)blockIdx.x * a.n_chunks;  // first partial of this (sequence, KV head)

  const float sink2 = a.sinks[hq] * kLog2e;
  float M = sink2;
  for (int ch = 0; ch < a.n_chunks; ++ch) M = fmaxf(M, a.part_ml[(p0 + ch) * 64 + c]);
  const float Ms = M == kNegInf ? 0.0f : M;
  float L = fast_exp2(sink2 - Ms);
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
  for (int ch = 0; ch < a.n_chunks; ++ch) {
    const float w = fast_exp2(a.part_ml[(p0 + ch) * 64 + c] - Ms);  // 0 for an empty chunk (max -inf)
    L += w * a.part_ml[(p0 + ch) * 64 + 32 + c];
    const float* po = a.part_o + (p0 + ch) * kHeadDim * 32;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += w * po[(8 * dg + i) * 32 + c];
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  const size_t row = (size_t)(cq + j) * a.Hq + hq;
  if (a.out_bf16) {
    bf16x8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (__bf16)(acc[i] * inv);
    *reinterpret_cast<bf16x8*>(static_cast<__bf16*>(a.out) + row * kHeadDim + 8 * dg) = v;
  } else {
    float* dst = static_cast<float*>(a.out) + row * kHeadDim + 8 * dg;
    *reinterpret_cast<f32x4*>(dst) = (f32x4){acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
    *reinterpret_cast<f32x4*>(dst + 4) = (f32x4){acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv};
  }
  if (dg == 0) a.lse[(size_t)hq * a.Tq + cq + j] = L > 0.0f ? (Ms + fast_log2(L)) * kLn2 : kNegInf;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  const long long parts = (long long)a.B * a.Hkv * a.n_chunks;
  if (parts <= 0) return hipSuccess;
  hipLaunchKernelGGL(attn_sink_decode_partial_kernel, dim3((unsigned)parts), dim3(64), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_sink_decode_combine_kernel, dim3((unsigned)(a.B * a.Hkv)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace attn_sink
