// Backward of attention with a learnable per-head sink, for gfx950.
//
// Math. With the sink-inclusive LSE saved by the forward, P_ij = exp(S_ij - LSE_i) is the
// sink-aware probability and P_{i,h} = exp(S_h - LSE_i) the sink's. Differentiating the softmax
// over [scores | sink] with upstream gradients dP_ij = dO_i . v_j for content keys and 0 for the
// sink (it has no value row) gives
//   dS_ij = P_ij (dP_ij - D_i),   D_i = sum_j P_ij dP_ij = dO_i . O_i,
//   dL/dS_h = -sum_i P_{i,h} D_i
// (nmedialink.com "惊爆！GPT-OSS-20B强化学习…", section "反向传播的实现", simplified equation,
// with its dL/dS_ij read as the upstream probability gradient), and the usual
//   dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO.
//
// Passes (all on the caller's stream, no atomics, bitwise reproducible):
//  1. prep:  D_i = rowsum(dO * O) for every (row, head); clear the dSink partial sums.
//  2. dkdv:  column-parallel. A workgroup owns 64 keys of one KV head; its waves split the
//            query heads of the group and stream 32-row query tiles, keeping dK^T and dV^T of
//            their keys in registers; the waves' partial sums are added in LDS at the end.
//  3. dq:    row-parallel. A workgroup owns 64 query rows of `hpw` heads of one group (one head
//            per wave) and streams 64-key tiles of K, V and K^T through LDS. Besides dQ it
//            accumulates D~_i = sum_j P_ij dP_ij from the fp32 P and dP it already holds and
//            writes sum_i P_{i,h} D~_i for its rows. D~ equals D mathematically but does not
//            carry the bf16 rounding of the forward's P.V product, which matters because the
//            terms of dL/dS_h cancel heavily.
//  4. dsink: dL/dS_h = -(sum of the partials of head h), summed in a fixed order.
#include "kernels.h"

namespace attn_sink {

namespace {

constexpr int kLdsStride = 72;  // bf16 per staged 64-element row (16-byte aligned, 8 pad)

// ------------------------------------------------------------------------------------------
// 1. D_i = sum_d dO[i,h,d] * O[i,h,d]; 16 lanes per (row, head), 4 elements each.
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void attn_sink_bwd_prep_kernel(BwdArgs a) {
  const long long rows = (long long)a.T * a.Hq;
  const long long row = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int part = threadIdx.x & 15;
  float acc = 0.0f;
  if (row < rows) {
    const f32x4 o = *reinterpret_cast<const f32x4*>(a.out + row * kHeadDim + 4 * part);
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    const bf16x4 d = *reinterpret_cast<const bf16x4*>(a.dout + row * kHeadDim + 4 * part);
    acc = o[0] * (float)d[0] + o[1] * (float)d[1] + o[2] * (float)d[2] + o[3] * (float)d[3];
  }
  acc += __shfl_xor(acc, 8, 16);
  acc += __shfl_xor(acc, 4, 16);
  acc += __shfl_xor(acc, 2, 16);
  acc += __shfl_xor(acc, 1, 16);
  if (row < rows && part == 0) {
    const long long t = row / a.Hq;
    const int h = (int)(row - t * a.Hq);
    a.dws[(size_t)h * a.T + t] = acc;
  }
  // Clear the dSink partials (rows of the dq pass that exit early never write theirs).
  const long long nparts = (long long)a.Hq * a.n_slots;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < nparts;
       i += (long long)gridDim.x * blockDim.x) {
    a.dsink_part[i] = 0.0f;
  }
}

// ------------------------------------------------------------------------------------------
// 2. dK, dV: column-parallel over 64-key blocks.
// ------------------------------------------------------------------------------------------
constexpr int kKvQTile = 32;                    // query rows per step
constexpr int kKvStageStride = kKvQTile + 8;    // transposed staging row: 32 queries + pad
constexpr int kKvStageElems = kHeadDim * kKvStageStride;
constexpr int kKvRedStride = kHeadDim + 4;      // fp32 reduction row

__global__ __launch_bounds__(256, 1) void attn_sink_bwd_dkdv_kernel(BwdArgs a) {
  // Per wave: Q^T and dO^T of the current query tile, [d][query]. Reused afterwards for the
  // cross-wave reduction of dK / dV ([key][d] fp32).
  __shared__ __attribute__((aligned(16))) unsigned char smem[4 * 2 * kKvStageElems * 2];
  static_assert(sizeof(smem) >= kKvKeysPerBlock * kKvRedStride * 4, "reduction buffer fits");

  const int nw = a.kv_waves;
  const int bid = blockIdx.x;
  const int g = bid % a.Hkv;
  const int rest = bid / a.Hkv;
  const int b = rest % a.B;
  const int kb = rest / a.B;  // ascending: under a causal mask the first key blocks carry the most rows
  const int cs = a.cu[b];
  const int len = a.cu[b + 1] - cs;
  const int k0 = kb * kKvKeysPerBlock;
  if (k0 >= len) return;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int grp = lane >> 5;

  __bf16* qt_lds = reinterpret_cast<__bf16*>(smem) + wave * 2 * kKvStageElems;
  __bf16* dot_lds = qt_lds + kKvStageElems;

  // K^T and V^T as B operands (k = d, n = key): lane holds key k0 + 32nb + l32, d = 16c + 8grp.
  bf16x8 kf[2][4], vf[2][4];
  const size_t kv_tok = (size_t)a.Hkv * kHeadDim;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int key = k0 + 32 * nb + l32;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const size_t off = (size_t)(cs + key) * kv_tok + (size_t)g * kHeadDim + 16 * c + 8 * grp;
      kf[nb][c] = key < len ? load_bf16x8(a.k + off) : zero_bf16x8();
      vf[nb][c] = key < len ? load_bf16x8(a.v + off) : zero_bf16x8();
    }
  }

  f32x16 dk[2][2], dv[2][2];  // [d block][key block], C layout of dK^T / dV^T
#pragma unroll
  for (int x = 0; x < 2; ++x) {
#pragma unroll
    for (int y = 0; y < 2; ++y) {
      dk[x][y] = zero_f32x16();
      dv[x][y] = zero_f32x16();
    }
  }

  // Query rows that can see any key of [k0, k0+64).
  const int kmax = min(len, k0 + kKvKeysPerBlock) - 1;
  const int i_begin = a.causal ? k0 : 0;
  const int i_end = a.window > 0 ? min(len, kmax + a.window) : len;  // exclusive
  const int t_begin = i_begin / kKvQTile;
  const int t_end = (i_end + kKvQTile - 1) / kKvQTile;

  for (int hh = wave; hh < a.G; hh += nw) {
    const int h = g * a.G + hh;
    for (int t = t_begin; t < t_end; ++t) {
      const int i0 = t * kKvQTile;
      // Q and dO rows as A operands (m = query, k = d); row r holds query i0 + swap23(r).
      const int qrow = i0 + swap23(l32);
      bf16x8 qa[4], da[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const size_t off = ((size_t)(cs + qrow) * a.Hq + h) * kHeadDim + 16 * c + 8 * grp;
        qa[c] = qrow < len ? load_bf16x8(a.q + off) : zero_bf16x8();
        da[c] = qrow < len ? load_bf16x8(a.dout + off) : zero_bf16x8();
      }
      // LSE (log2 units) and D of the 16 query rows this lane's C registers hold.
      float lse2[16], dd[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int qi = i0 + c_row(i, grp);
        const bool ok = qi < len;
        lse2[i] = ok ? a.lse[(size_t)h * a.T + cs + qi] * kLog2e : 0.0f;
        dd[i] = ok ? a.dws[(size_t)h * a.T + cs + qi] : 0.0f;
      }
      // Stage Q^T and dO^T ([d][query], query slot = local row index) for the second products.
      const int lrow = swap23(l32);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          qt_lds[(16 * c + 8 * grp + e) * kKvStageStride + lrow] = qa[c][e];
          dot_lds[(16 * c + 8 * grp + e) * kKvStageStride + lrow] = da[c][e];
        }
      }

      // S = Q K^T and dP = dO V^T, C layout: lane = key column, registers = query rows.
      f32x16 s[2], dp[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        s[nb] = zero_f32x16();
        dp[nb] = zero_f32x16();
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          s[nb] = mfma_32x32x16(qa[c], kf[nb][c], s[nb]);
          dp[nb] = mfma_32x32x16(da[c], vf[nb][c], dp[nb]);
        }
      }

      const bool need_mask = (i0 + kKvQTile > len) || (k0 + kKvKeysPerBlock > len) ||
                             (a.causal && k0 + kKvKeysPerBlock - 1 > i0) ||
                             (a.window > 0 && k0 <= i0 + kKvQTile - 1 - a.window);
      bf16x8 pb[2][2], dsb[2][2];  // [key block][query chunk]
      float pmax = 0.0f;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int kj = k0 + 32 * nb + l32;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float p = fast_exp2(__builtin_fmaf(s[nb][i], a.scale_log2, -lse2[i]));
          if (need_mask) {
            const int qi = i0 + c_row(i, grp);
            if (!(qi < len && visible(qi, kj, len, a.causal, a.window))) p = 0.0f;
          }
          pmax = fmaxf(pmax, p);
          s[nb][i] = p;
          dp[nb][i] = p * (dp[nb][i] - dd[i]);
        }
        pb[nb][0] = pack8(s[nb], 0);
        pb[nb][1] = pack8(s[nb], 1);
        dsb[nb][0] = pack8(dp[nb], 0);
        dsb[nb][1] = pack8(dp[nb], 1);
      }
      // Large probabilities: add the products of the bf16 rounding residuals of P and dS.
      const bool split = wave_any(pmax > kSplitThreshold);

      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

      // dV^T += dO^T P and dK^T += Q^T dS (contract over the tile's 32 queries).
#pragma unroll
      for (int db = 0; db < 2; ++db) {
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const bf16x8 doa = load_bf16x8(&dot_lds[(32 * db + l32) * kKvStageStride + 16 * cc + 8 * grp]);
          const bf16x8 qta = load_bf16x8(&qt_lds[(32 * db + l32) * kKvStageStride + 16 * cc + 8 * grp]);
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            dv[db][nb] = mfma_32x32x16(doa, pb[nb][cc], dv[db][nb]);
            dk[db][nb] = mfma_32x32x16(qta, dsb[nb][cc], dk[db][nb]);
          }
          if (split) {
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
              dv[db][nb] = mfma_32x32x16(doa, residual8(s[nb], cc, pb[nb][cc]), dv[db][nb]);
              dk[db][nb] = mfma_32x32x16(qta, residual8(dp[nb], cc, dsb[nb][cc]), dk[db][nb]);
            }
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }

  // Sum the waves' partial dK^T / dV^T in LDS, then store [key][d] rows (dK scaled).
  float* red = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    for (int w = 0; w < nw; ++w) {
      __syncthreads();
      if (wave == w) {
#pragma unroll
        for (int db = 0; db < 2; ++db) {
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            const f32x16& acc = which == 0 ? dk[db][nb] : dv[db][nb];
            const int key = 32 * nb + l32;
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              f32x4* dst = reinterpret_cast<f32x4*>(&red[key * kKvRedStride + 32 * db + 8 * r4 + 4 * grp]);
              f32x4 val = {acc[4 * r4], acc[4 * r4 + 1], acc[4 * r4 + 2], acc[4 * r4 + 3]};
              if (w == 0) {
                *dst = val;
              } else {
                *dst = *dst + val;
              }
            }
          }
        }
      }
    }
    __syncthreads();
    float* dst = which == 0 ? a.dk : a.dv;
    const float mul = which == 0 ? a.scale : 1.0f;
    for (int u = tid; u < kKvKeysPerBlock * (kHeadDim / 4); u += blockDim.x) {
      const int key = u / (kHeadDim / 4);
      const int c4 = u % (kHeadDim / 4);
      if (k0 + key < len) {
        f32x4 val = *reinterpret_cast<const f32x4*>(&red[key * kKvRedStride + 4 * c4]);
        *reinterpret_cast<f32x4*>(dst + ((size_t)(cs + k0 + key) * a.Hkv + g) * kHeadDim + 4 * c4) = val * mul;
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// 3. dQ and the dSink partials: row-parallel over 64-row query blocks.
// ------------------------------------------------------------------------------------------
constexpr int kDqTileKeys = 64;

template <int NB>
__global__ __launch_bounds__(256) void attn_sink_bwd_dq_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) __bf16 k_lds[kDqTileKeys * kLdsStride];
  __shared__ __attribute__((aligned(16))) __bf16 v_lds[kDqTileKeys * kLdsStride];
  __shared__ __attribute__((aligned(16))) __bf16 kt_lds[kHeadDim * kLdsStride];

  constexpr int kRows = 32 * NB;
  const int n_hs = a.Hq / a.hpw;
  const int bid = blockIdx.x;
  const int inner = bid % n_hs;
  const int rest = bid / n_hs;
  const int spg = a.G / a.hpw;
  const int hs = (inner % a.Hkv) * spg + inner / a.Hkv;
  const int b = rest % a.B;
  const int qb = a.n_qblocks - 1 - rest / a.B;
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

  // Q^T and dO^T as B operands: lane holds query q0 + 32nb + l32, d = 16c + 8grp + (0..7).
  bf16x8 qf[NB][4], df[NB][4];
  float lse2[NB], dd[NB], dsum[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int qi = q0 + 32 * nb + l32;
    const bool ok = qi < len;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const size_t off = ((size_t)(cs + qi) * a.Hq + h) * kHeadDim + 16 * c + 8 * grp;
      qf[nb][c] = ok ? load_bf16x8(a.q + off) : zero_bf16x8();
      df[nb][c] = ok ? load_bf16x8(a.dout + off) : zero_bf16x8();
    }
    lse2[nb] = ok ? a.lse[(size_t)h * a.T + cs + qi] * kLog2e : 0.0f;
    dd[nb] = ok ? a.dws[(size_t)h * a.T + cs + qi] : 0.0f;
    dsum[nb] = 0.0f;
  }

  f32x16 acc[2][NB];  // dQ^T, [d block][query block]
#pragma unroll
  for (int db = 0; db < 2; ++db) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[db][nb] = zero_f32x16();
  }

  const int kend = a.causal ? min(len, q0 + kRows) : len;
  const int kbeg = a.window > 0 ? max(0, q0 - a.window + 1) : 0;
  const int kt_begin = kbeg / kDqTileKeys;
  const int kt_end = (kend + kDqTileKeys - 1) / kDqTileKeys;
  const size_t tok_stride = (size_t)a.Hkv * kHeadDim;
  const __bf16* kbase = a.k + (size_t)cs * tok_stride + (size_t)g * kHeadDim;
  const __bf16* vbase = a.v + (size_t)cs * tok_stride + (size_t)g * kHeadDim;

  for (int kt = kt_begin; kt < kt_end; ++kt) {
    const int k0 = kt * kDqTileKeys;
    __syncthreads();
    for (int u = tid; u < kDqTileKeys * 8; u += nthreads) {
      const int r = u >> 3, c8 = u & 7;
      const int key = k0 + r;
      const bool ok = key < len;
      *reinterpret_cast<bf16x8*>(&k_lds[r * kLdsStride + 8 * c8]) =
          ok ? load_bf16x8(kbase + (size_t)key * tok_stride + 8 * c8) : zero_bf16x8();
      *reinterpret_cast<bf16x8*>(&v_lds[r * kLdsStride + 8 * c8]) =
          ok ? load_bf16x8(vbase + (size_t)key * tok_stride + 8 * c8) : zero_bf16x8();
    }
    for (int u = tid; u < (kDqTileKeys / 2) * 8; u += nthreads) {
      const int c8 = u & 7, p = u >> 3;
      const int key = k0 + 2 * p;
      bf16x8 k0v = key < len ? load_bf16x8(kbase + (size_t)key * tok_stride + 8 * c8) : zero_bf16x8();
      bf16x8 k1v = key + 1 < len ? load_bf16x8(kbase + (size_t)(key + 1) * tok_stride + 8 * c8) : zero_bf16x8();
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        bf16x2 pr = {k0v[j], k1v[j]};
        *reinterpret_cast<bf16x2*>(&kt_lds[(8 * c8 + j) * kLdsStride + 2 * p]) = pr;
      }
    }
    __syncthreads();

    // S^T = K Q^T and dP^T = V dO^T (rows = keys, loaded with the swap23 permutation).
    f32x16 s[2][NB], dp[2][NB];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        s[mb][nb] = zero_f32x16();
        dp[mb][nb] = zero_f32x16();
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int row = (32 * mb + swap23(l32)) * kLdsStride + 16 * c + 8 * grp;
        const bf16x8 ka = load_bf16x8(&k_lds[row]);
        const bf16x8 va = load_bf16x8(&v_lds[row]);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          s[mb][nb] = mfma_32x32x16(ka, qf[nb][c], s[mb][nb]);
          dp[mb][nb] = mfma_32x32x16(va, df[nb][c], dp[mb][nb]);
        }
      }
    }

    const bool need_mask = (k0 + kDqTileKeys > len) || (a.causal && k0 + kDqTileKeys - 1 > q0) ||
                           (a.window > 0 && k0 <= q0 + kRows - 1 - a.window);
    bf16x8 dsb[2][2][NB];
    float pmax = 0.0f;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int qi = q0 + 32 * nb + l32;
      float part = 0.0f;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float p = fast_exp2(__builtin_fmaf(s[mb][nb][i], a.scale_log2, -lse2[nb]));
          if (need_mask) {
            const int kj = k0 + 32 * mb + c_row(i, grp);
            if (!visible(qi, kj, len, a.causal, a.window)) p = 0.0f;
          }
          pmax = fmaxf(pmax, p);
          const float pdp = p * dp[mb][nb][i];
          part += pdp;
          dp[mb][nb][i] = pdp - p * dd[nb];
        }
        dsb[mb][0][nb] = pack8(dp[mb][nb], 0);
        dsb[mb][1][nb] = pack8(dp[mb][nb], 1);
      }
      dsum[nb] += part;
    }

    // Large probabilities: also multiply the bf16 rounding residual of dS.
    const bool split = wave_any(pmax > kSplitThreshold);
    // dQ^T += K^T dS^T (A = K^T from LDS, contracting over the tile's keys).
#pragma unroll
    for (int db = 0; db < 2; ++db) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const bf16x8 kta = load_bf16x8(&kt_lds[(32 * db + l32) * kLdsStride + 32 * mb + 16 * cc + 8 * grp]);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) acc[db][nb] = mfma_32x32x16(kta, dsb[mb][cc][nb], acc[db][nb]);
          if (split) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
              acc[db][nb] = mfma_32x32x16(kta, residual8(dp[mb][nb], cc, dsb[mb][cc][nb]), acc[db][nb]);
            }
          }
        }
      }
    }
  }

  // dQ rows, and this wave's share of sum_i P_{i,h} D~_i.
  const float sink = a.sinks[h];
  float wsum = 0.0f;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int qi = q0 + 32 * nb + l32;
    const float dtot = dsum[nb] + xor32(dsum[nb]);
    if (qi < len) {
      float* qrow = a.dq + ((size_t)(cs + qi) * a.Hq + h) * kHeadDim;
#pragma unroll
      for (int db = 0; db < 2; ++db) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          f32x4 val = {acc[db][nb][4 * r4], acc[db][nb][4 * r4 + 1], acc[db][nb][4 * r4 + 2],
                       acc[db][nb][4 * r4 + 3]};
          *reinterpret_cast<f32x4*>(qrow + 32 * db + 8 * r4 + 4 * grp) = val * a.scale;
        }
      }
      if (grp == 0) wsum += fast_exp2(__builtin_fmaf(sink, kLog2e, -lse2[nb])) * dtot;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) wsum += __shfl_xor(wsum, off);
  if (lane == 0) {
    // Unique slot per (sequence, row block): floor(cs / rows) + b + qb never collides.
    const int slot = cs / kRows + b + qb;
    a.dsink_part[(size_t)h * a.n_slots + slot] = wsum;
  }
}

// ------------------------------------------------------------------------------------------
// 4. dL/dS_h = -sum of the head's partials (one wave per head, fixed summation order).
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(64) void attn_sink_bwd_dsink_kernel(BwdArgs a) {
  const int h = blockIdx.x;
  float acc = 0.0f;
  for (int i = threadIdx.x; i < a.n_slots; i += 64) acc += a.dsink_part[(size_t)h * a.n_slots + i];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if (threadIdx.x == 0) a.dsinks[h] = -acc;
}

}  // namespace

hipError_t launch_bwd_prep(const BwdArgs& a, hipStream_t stream) {
  const long long rows = (long long)a.T * a.Hq;
  long long nblocks = (rows + 15) / 16;
  if (nblocks < 1) nblocks = 1;  // still clears the dSink partials when T = 0
  hipLaunchKernelGGL(attn_sink_bwd_prep_kernel, dim3((unsigned)nblocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t stream) {
  const long long nblocks = (long long)a.n_kblocks * a.B * a.Hkv;
  if (nblocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(attn_sink_bwd_dkdv_kernel, dim3((unsigned)nblocks), dim3(64 * a.kv_waves), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t stream) {
  constexpr int NB = kDqRowsPerWave / 32;
  const long long nblocks = (long long)a.n_qblocks * (a.Hq / a.hpw) * a.B;
  if (nblocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(attn_sink_bwd_dq_kernel<NB>, dim3((unsigned)nblocks), dim3(64 * a.hpw), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dsink(const BwdArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(attn_sink_bwd_dsink_kernel, dim3((unsigned)a.Hq), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace attn_sink
