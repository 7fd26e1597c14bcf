// Forward of attention with a learnable per-head sink, for gfx950.
//
// Math (nmedialink.com "惊爆！GPT-OSS-20B强化学习…", section "GPT-OSS中的带注意力槽的注意力机制"
// and section "数学公式深入解读", eq. P_ij): each row's softmax runs over the visible scores plus
// one extra logit S_h, and the output only sums the visible keys' values. Written as an online
// softmax, the sink is simply the first element the row has seen: the running max starts at S_h
// and the running denominator at exp(S_h - S_h) = 1, while the output accumulator starts at 0
// because the sink has no value row. LSE = max + log(denominator) therefore includes the sink.
//
// Work split. A workgroup owns one block of 64 query rows of one sequence and `hpw` query heads
// that share one KV head (GQA); wave w handles head hs*hpw + w. K and V tiles of 64 keys are
// staged in LDS once and read by all of the workgroup's waves. Per tile each wave computes
//   S^T = K Q^T   (32x32x16 MFMA; keys on the C rows, the wave's 64 queries on the columns)
// so that each lane owns one query: the row max and row sum are mostly lane-local (one exchange
// with lane ^ 32), and the probabilities, rounded to bf16, are already laid out as the B operand
// of the second product
//   O^T += V^T P^T,
// whose A operand (V^T) is staged transposed in LDS. Causal and window tiles outside a block's
// key range are skipped; only boundary tiles evaluate the mask.
#include "kernels.h"

namespace attn_sink {

namespace {

constexpr int kTileKeys = 64;
constexpr int kLdsStride = 72;  // bf16 elements per staged row (64 + 8 pad: 16-byte aligned rows)

template <int NB>  // 32-query column blocks per wave
__global__ __launch_bounds__(256) void attn_sink_fwd_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) __bf16 k_lds[kTileKeys * kLdsStride];
  __shared__ __attribute__((aligned(16))) __bf16 vt_lds[kHeadDim * kLdsStride];

  constexpr int kRows = 32 * NB;
  const int n_hs = a.Hq / a.hpw;
  const int bid = blockIdx.x;
  const int inner = bid % n_hs;
  const int rest = bid / n_hs;
  // Consecutive block ids walk the KV groups first, so the round-robin placement of
  // workgroups on the 8 XCDs keeps each group's K/V in few L2s.
  const int spg = a.G / a.hpw;
  const int hs = (inner % a.Hkv) * spg + inner / a.Hkv;
  const int b = rest % a.B;
  const int qb = a.n_qblocks - 1 - rest / a.B;  // longest causal rows first

  const int cs = a.cu[b];
  const int len = a.cu[b + 1] - cs;
  const int q0 = qb * kRows;
  if (q0 >= len) return;

  const int tid = threadIdx.x;
  const int nthreads = blockDim.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int grp = lane >> 5;
  const int h = hs * a.hpw + wave;
  const int g = h / a.G;

  // Q^T as the B operand of S^T = K Q^T: lane holds query q0 + 32nb + l32, d = 16c + 8grp + (0..7).
  bf16x8 qf[NB][4];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int qi = q0 + 32 * nb + l32;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      qf[nb][c] = qi < len ? load_bf16x8(a.q + ((size_t)(cs + qi) * a.Hq + h) * kHeadDim + 16 * c + 8 * grp)
                           : zero_bf16x8();
    }
  }

  const float sink_log2 = a.sinks[h] * kLog2e;
  float m[NB], lsum[NB];
  f32x16 o[2][NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    m[nb] = sink_log2;
    // The sink contributes exp2(S_h*log2e - m) = 1 to the denominator; count it once per query.
    lsum[nb] = (grp == 0 && sink_log2 != kNegInf) ? 1.0f : 0.0f;
    o[0][nb] = zero_f32x16();
    o[1][nb] = zero_f32x16();
  }

  const int kend = a.causal ? min(len, q0 + kRows) : len;
  const int kbeg = a.window > 0 ? max(0, q0 - a.window + 1) : 0;
  const int kt_begin = kbeg / kTileKeys;
  const int kt_end = (kend + kTileKeys - 1) / kTileKeys;

  const __bf16* kbase = a.k + (size_t)cs * a.Hkv * kHeadDim + (size_t)g * kHeadDim;
  const __bf16* vbase = a.v + (size_t)cs * a.Hkv * kHeadDim + (size_t)g * kHeadDim;
  const size_t tok_stride = (size_t)a.Hkv * kHeadDim;

  for (int kt = kt_begin; kt < kt_end; ++kt) {
    const int k0 = kt * kTileKeys;
    __syncthreads();  // every wave is done reading the previous tile
    // K tile, natural layout [key][d].
    for (int u = tid; u < kTileKeys * 8; u += nthreads) {
      const int r = u >> 3, c8 = u & 7;
      const int key = k0 + r;
      bf16x8 val = key < len ? load_bf16x8(kbase + (size_t)key * tok_stride + 8 * c8) : zero_bf16x8();
      *reinterpret_cast<bf16x8*>(&k_lds[r * kLdsStride + 8 * c8]) = val;
    }
    // V tile, transposed [d][key]: each thread takes two keys and writes packed pairs.
    for (int u = tid; u < (kTileKeys / 2) * 8; u += nthreads) {
      const int c8 = u & 7, p = u >> 3;
      const int key = k0 + 2 * p;
      bf16x8 v0 = key < len ? load_bf16x8(vbase + (size_t)key * tok_stride + 8 * c8) : zero_bf16x8();
      bf16x8 v1 = key + 1 < len ? load_bf16x8(vbase + (size_t)(key + 1) * tok_stride + 8 * c8) : zero_bf16x8();
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        bf16x2 pr = {v0[j], v1[j]};
        *reinterpret_cast<bf16x2*>(&vt_lds[(8 * c8 + j) * kLdsStride + 2 * p]) = pr;
      }
    }
    __syncthreads();

    // S^T = K Q^T for two 32-key row blocks.
    f32x16 s[2][NB];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) s[mb][nb] = zero_f32x16();
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bf16x8 ka = load_bf16x8(&k_lds[(32 * mb + swap23(l32)) * kLdsStride + 16 * c + 8 * grp]);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) s[mb][nb] = mfma_32x32x16(ka, qf[nb][c], s[mb][nb]);
      }
    }

    const bool need_mask = (k0 + kTileKeys > len) || (a.causal && k0 + kTileKeys - 1 > q0) ||
                           (a.window > 0 && k0 <= q0 + kRows - 1 - a.window);
    if (need_mask) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int qi = q0 + 32 * nb + l32;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int kj = k0 + 32 * mb + c_row(i, grp);
            if (!visible(qi, kj, len, a.causal, a.window)) s[mb][nb][i] = kNegInf;
          }
        }
      }
    }

    bf16x8 pb[2][2][NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float tmax = kNegInf;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, s[mb][nb][i]);
      }
      tmax = fmaxf(tmax, xor32(tmax));
      const float mnew = fmaxf(m[nb], tmax * a.scale_log2);
      const float moff = mnew == kNegInf ? 0.0f : mnew;  // a row with nothing visible yet stays at 0
      const float alpha = fast_exp2(m[nb] - moff);
      float rs = 0.0f;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = fast_exp2(__builtin_fmaf(s[mb][nb][i], a.scale_log2, -moff));
          s[mb][nb][i] = p;
          rs += p;
        }
        pb[mb][0][nb] = pack8(s[mb][nb], 0);
        pb[mb][1][nb] = pack8(s[mb][nb], 1);
      }
      lsum[nb] = lsum[nb] * alpha + rs;
      o[0][nb] *= alpha;
      o[1][nb] *= alpha;
      m[nb] = mnew;
    }

    // O^T += V^T P^T, contracting over the tile's 64 keys in four 16-key chunks.
#pragma unroll
    for (int db = 0; db < 2; ++db) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const bf16x8 va = load_bf16x8(&vt_lds[(32 * db + l32) * kLdsStride + 32 * mb + 16 * cc + 8 * grp]);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) o[db][nb] = mfma_32x32x16(va, pb[mb][cc][nb], o[db][nb]);
        }
      }
    }
  }

  // Epilogue: combine the two lane halves' partial denominators, normalise, store.
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float ltot = lsum[nb] + xor32(lsum[nb]);
    const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
    const int qi = q0 + 32 * nb + l32;
    if (qi < len) {
      float* orow = a.out + ((size_t)(cs + qi) * a.Hq + h) * kHeadDim;
#pragma unroll
      for (int db = 0; db < 2; ++db) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          f32x4 val = {o[db][nb][4 * r4] * inv, o[db][nb][4 * r4 + 1] * inv, o[db][nb][4 * r4 + 2] * inv,
                       o[db][nb][4 * r4 + 3] * inv};
          *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * r4 + 4 * grp) = val;
        }
      }
      if (grp == 0) {
        a.lse[(size_t)h * a.T + cs + qi] = ltot > 0.0f ? (m[nb] + fast_log2(ltot)) * kLn2 : kNegInf;
      }
    }
  }
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  constexpr int NB = kFwdRowsPerWave / 32;
  const long long nblocks = (long long)a.n_qblocks * (a.Hq / a.hpw) * a.B;
  if (nblocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(attn_sink_fwd_kernel<NB>, dim3((unsigned)nblocks), dim3(64 * a.hpw), 0, stream, a);
  return hipGetLastError();
}

}  // namespace attn_sink
