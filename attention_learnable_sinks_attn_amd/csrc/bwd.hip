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
//  2. dkdv:  column-parallel. A workgroup owns 64 keys of one KV head and one half of the
//            group's query heads: two key halves of 32 times one or two "head streams".
//            For each step (head, 64 query rows) the Q, dO, LSE and D rows are staged once per
//            stream in LDS, double-buffered with the next step's global loads issued ahead;
//            the transposed Q^T / dO^T operands come from transposing LDS loads. dK^T and dV^T of each wave's 32 keys stay in
//            registers; the two streams' partial sums are added in LDS at the end, and each
//            head half writes its own fp32 partial. Splitting the heads doubles the number of
//            workgroups, so that (launched longest first) they keep two per CU busy under a
//            causal mask instead of leaving a long block alone on its CU.
//  2b. dkdv_sum: dK = scale * (sum of the halves), dV = sum of the halves.
//  3. dq:    row-parallel. A workgroup owns 32 query rows of `hpw` heads of one group (one head
//            per wave) and streams double-buffered 64-key tiles of K and V through LDS (K^T
//            operands come from transposing LDS loads of the K tile).
//            Besides dQ it accumulates D~_i = sum_j P_ij dP_ij from the fp32 P and dP it already
//            holds and writes sum_i P_{i,h} D~_i for its rows. D~ equals D mathematically but
//            does not carry the bf16 rounding of the forward's P.V product, which matters
//            because the terms of dL/dS_h cancel heavily.
//  4. dsink: dL/dS_h = -(sum of the partials of head h), summed in a fixed order.
#include "kernels.h"

namespace attn_sink {

namespace {

constexpr int kLdsStride = 72;  // bf16 per staged 64-element row (16-byte aligned, 8 pad)
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

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
constexpr int kKvSub = 32;                             // query rows per product block
constexpr int kKvStageRows = 64;                       // query rows staged per step (2 blocks)
constexpr int kKvNatElems = kKvStageRows * kLdsStride; // [query][d] tile
// One stream's stage: Q and dO rows (natural layout), then LSE (log2 units) and D of those rows.
constexpr int kKvStageBytes = 2 * kKvNatElems * 2 + 2 * kKvStageRows * 4;
constexpr int kKvRedStride = kHeadDim + 4;             // fp32 reduction row

template <int NS>  // head streams: 1 or 2 (waves = 2 * NS)
__global__ __launch_bounds__(128 * NS, 2) void attn_sink_bwd_dkdv_kernel(BwdArgs a) {
  constexpr int NW = 2 * NS;
  constexpr int NT = 64 * NW;
  constexpr int kRR = kKvStageRows * 8 / NT;  // 16-byte pieces per thread and staged tile
  static_assert(NT == NS * 2 * kKvStageRows, "one LSE or D value per thread and stage");
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * NS * kKvStageBytes];
  static_assert(sizeof(smem) >= 4 * 32 * kKvRedStride * 4, "reduction buffer fits");

  // Block order: KV group fastest (consecutive ids land on different XCDs, each XCD keeps few
  // groups' rows in its L2), then head half, sequence, and key block ascending: under a causal
  // mask the first key blocks carry the most query rows, so the longest blocks start first and
  // the short ones fill in as slots free up.
  const int bid = blockIdx.x;
  const int g = bid % a.Hkv;
  int rest = bid / a.Hkv;
  const int hh = rest % a.n_halves;
  rest /= a.n_halves;
  const int b = rest % a.B;
  const int kb = rest / a.B;
  const int cs = a.cu[b];
  const int len = a.cu[b + 1] - cs;
  const int kblk = kb * kKvKeysPerBlock;
  if (kblk >= len) return;

  const int tid = threadIdx.x;
  const int wave = wave_id();
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int grp = lane >> 5;
  const int kh = wave & 1;        // key half
  const int st = wave >> 1;       // head stream
  const int k0 = kblk + 32 * kh;  // this wave's 32 keys
  const int heads_half = a.G / a.n_halves;
  const int heads_per_stream = heads_half / NS;
  const int h_base = g * a.G + hh * heads_half;  // stream s takes heads h_base + s + NS * j

  // K^T and V^T as B operands (k = d, n = key): lane holds key k0 + l32, d = 16c + 8grp + (0..7).
  bf16x8 kf[4], vf[4];
  const size_t kv_tok = (size_t)a.Hkv * kHeadDim;
  {
    const int key = min(k0 + l32, len - 1);  // keys past the end are masked
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const size_t off = (size_t)(cs + key) * kv_tok + (size_t)g * kHeadDim + 16 * c + 8 * grp;
      kf[c] = load_bf16x8(a.k + off);
      vf[c] = load_bf16x8(a.v + off);
    }
  }
  f32x16 dk[2], dv[2];  // [d block], C layout of dK^T / dV^T (rows d, columns this wave's keys)
  dk[0] = dk[1] = dv[0] = dv[1] = zero_f32x16();

  // Query rows that can see a key of [kblk, kblk + 64), in 64-row stages.
  const int kmax = min(len, kblk + kKvKeysPerBlock) - 1;
  const int i_begin = a.causal ? kblk : 0;
  const int i_end = a.window > 0 ? min(len, kmax + a.window) : len;  // exclusive
  const int t_begin = i_begin / kKvStageRows;
  const int n_t = (i_end + kKvStageRows - 1) / kKvStageRows - t_begin;
  const int n_steps = heads_per_stream * n_t;

  // Staging: per thread, row (tid >> 3) + (NT / 8) * rr, chunk (tid & 7) of each of the 2 * NS
  // tiles (stream t >> 1, Q or dO by t & 1), plus one LSE or D value. Rows past the sequence end
  // are clamped onto its last row (finite data; those rows are masked out).
  bf16x8 pre[2 * NS][kRR];
  float pre_ld = 0.0f;
  auto stage_ptr = [&](int buf, int s) { return smem + (size_t)(buf * NS + s) * kKvStageBytes; };
  const int prow = tid >> 3, pc8 = tid & 7;
  auto prefetch = [&](int hj, int i0) {
#pragma unroll
    for (int t = 0; t < 2 * NS; ++t) {
      const int h = h_base + (t >> 1) + NS * hj;
      const __bf16* base = ((t & 1) ? a.dout : a.q) + ((size_t)cs * a.Hq + h) * kHeadDim;
#pragma unroll
      for (int rr = 0; rr < kRR; ++rr) {
        const int qi = min(i0 + prow + (NT / 8) * rr, len - 1);
        pre[t][rr] = load_bf16x8(base + (unsigned)(qi * a.Hq * kHeadDim + 8 * pc8));
      }
    }
    {  // exactly one LSE or D value per thread (NT == NS * 2 * kKvStageRows)
      const int s = tid / (2 * kKvStageRows);
      const int which = (tid / kKvStageRows) & 1;
      const int h = h_base + s + NS * hj;
      const int qi = min(i0 + (tid & (kKvStageRows - 1)), len - 1);
      pre_ld = (which ? a.dws : a.lse)[(size_t)h * a.T + cs + qi];  // consumed only in commit
    }
  };
  auto commit = [&](int buf) {
#pragma unroll
    for (int t = 0; t < 2 * NS; ++t) {
      __bf16* nat = reinterpret_cast<__bf16*>(stage_ptr(buf, t >> 1)) + (t & 1) * kKvNatElems;
#pragma unroll
      for (int rr = 0; rr < kRR; ++rr) {
        *reinterpret_cast<bf16x8*>(&nat[(prow + (NT / 8) * rr) * kLdsStride + 8 * pc8]) = pre[t][rr];
      }
    }
    {
      float* f = reinterpret_cast<float*>(stage_ptr(buf, tid / (2 * kKvStageRows)) + 2 * kKvNatElems * 2);
      f[tid & (2 * kKvStageRows - 1)] = ((tid / kKvStageRows) & 1) ? pre_ld : pre_ld * kLog2e;  // LSE in log2 units
    }
  };

  // Stages run from the last query rows backwards: every workgroup's causal range ends at the
  // sequence end, so workgroups of one KV group stream the same rows at about the same time and
  // mostly hit in L2.
  auto stage_row = [&](int t) { return (t_begin + n_t - 1 - t) * kKvStageRows; };
  int hj = 0, ti = 0;  // current step = (head index within the stream, stage index)
  // Unconditional (n_steps > 0 here): every load issued so far, including K and V, is complete
  // on every path into the loop, so the loop only waits on its prefetch when committing it.
  prefetch(0, stage_row(0));
  commit(0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): nothing issued before the loop stays in flight
  __syncthreads();

  for (int step = 0; step < n_steps; ++step) {
    const int cur = step & 1;
    const bool has_next = step + 1 < n_steps;
    const int hj_n = ti + 1 < n_t ? hj : hj + 1;
    const int ti_n = ti + 1 < n_t ? ti + 1 : 0;
    if (has_next) prefetch(hj_n, stage_row(ti_n));

    const unsigned char* sp = stage_ptr(cur, st);
    const __bf16* qn = reinterpret_cast<const __bf16*>(sp);
    const __bf16* dn = qn + kKvNatElems;
    const float* lsep = reinterpret_cast<const float*>(sp + 2 * kKvNatElems * 2);
    const float* ddp = lsep + kKvStageRows;

#pragma unroll
    for (int sub = 0; sub < kKvStageRows / kKvSub; ++sub) {
      const int i0 = stage_row(ti) + kKvSub * sub;
      // Skip blocks in which no (query, key) pair of this wave is visible (wave-uniform).
      const bool live = (!a.causal || k0 <= i0 + kKvSub - 1) && (a.window <= 0 || i0 <= k0 + 30 + a.window) &&
                        k0 < len && i0 < len;
      if (!live) continue;
      const __bf16* qs = qn + kKvSub * sub * kLdsStride;
      const __bf16* ds = dn + kKvSub * sub * kLdsStride;

      // S = Q K^T and dP = dO V^T: A rows hold query swap23(r); C: lane = key, registers = queries.
      f32x16 s = zero_f32x16(), dp = zero_f32x16();
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int off = swap23(l32) * kLdsStride + 16 * c + 8 * grp;
        s = mfma_32x32x16(load_bf16x8(&qs[off]), kf[c], s);
        dp = mfma_32x32x16(load_bf16x8(&ds[off]), vf[c], dp);
      }
      // LSE / D of the 16 query rows held in this lane's registers: rows 16(i/8) + 8grp + (i%8).
      const f32x4* l4 = reinterpret_cast<const f32x4*>(lsep + kKvSub * sub);
      const f32x4* d4 = reinterpret_cast<const f32x4*>(ddp + kKvSub * sub);
      const f32x4 la = l4[2 * grp], lb = l4[2 * grp + 1], lc = l4[4 + 2 * grp], ld = l4[4 + 2 * grp + 1];
      const f32x4 da_ = d4[2 * grp], db_ = d4[2 * grp + 1], dc = d4[4 + 2 * grp], dd_ = d4[4 + 2 * grp + 1];
      const float lse2[16] = {la[0], la[1], la[2], la[3], lb[0], lb[1], lb[2], lb[3],
                              lc[0], lc[1], lc[2], lc[3], ld[0], ld[1], ld[2], ld[3]};
      const float dd[16] = {da_[0], da_[1], da_[2], da_[3], db_[0], db_[1], db_[2], db_[3],
                            dc[0], dc[1], dc[2], dc[3], dd_[0], dd_[1], dd_[2], dd_[3]};

      const bool need_mask = (i0 + kKvSub > len) || (k0 + 32 > len) || (a.causal && k0 + 31 > i0) ||
                             (a.window > 0 && k0 <= i0 + kKvSub - 1 - a.window);
      if (need_mask) {  // wave-uniform: only diagonal, window-edge and ragged blocks
        const int kj = k0 + l32;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int qi = i0 + c_row(i, grp);
          if (!(qi < len && visible(qi, kj, len, a.causal, a.window))) s[i] = kNegInf;
        }
      }
      float pmax = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(__builtin_fmaf(s[i], a.scale_log2, -lse2[i]));
        pmax = fmaxf(pmax, p);
        s[i] = p;
        dp[i] = p * (dp[i] - dd[i]);
      }
      const bf16x8 pb0 = pack8(s, 0), pb1 = pack8(s, 1);
      const bf16x8 ds0 = pack8(dp, 0), ds1 = pack8(dp, 1);
      // Large probabilities: add the products of the bf16 rounding residuals of P and dS.
      const bool split = wave_any(pmax > kSplitThreshold);

      // dV^T += dO^T P and dK^T += Q^T dS over the block's 32 queries; the transposed operands
      // come straight from the natural tiles through transposing LDS loads.
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const bf16x8 doa0 = load_tr8(ds, kLdsStride, 0, 32 * db), doa1 = load_tr8(ds, kLdsStride, 16, 32 * db);
        const bf16x8 qta0 = load_tr8(qs, kLdsStride, 0, 32 * db), qta1 = load_tr8(qs, kLdsStride, 16, 32 * db);
        dv[db] = mfma_32x32x16(doa0, pb0, dv[db]);
        dv[db] = mfma_32x32x16(doa1, pb1, dv[db]);
        dk[db] = mfma_32x32x16(qta0, ds0, dk[db]);
        dk[db] = mfma_32x32x16(qta1, ds1, dk[db]);
        if (split) {
          // The opaque copies of the packed values keep the residual arithmetic inside this
          // rarely taken branch (it depends on them), without copying the fp32 tiles.
          bf16x8 h0 = pb0, h1 = pb1, e0 = ds0, e1 = ds1;
          opaque(h0);
          opaque(h1);
          opaque(e0);
          opaque(e1);
          dv[db] = mfma_32x32x16(doa0, residual8(s, 0, h0), dv[db]);
          dv[db] = mfma_32x32x16(doa1, residual8(s, 1, h1), dv[db]);
          dk[db] = mfma_32x32x16(qta0, residual8(dp, 0, e0), dk[db]);
          dk[db] = mfma_32x32x16(qta1, residual8(dp, 1, e1), dk[db]);
        }
      }
    }

    if (has_next) commit(cur ^ 1);
    hj = hj_n;
    ti = ti_n;
    __syncthreads();
  }

  // Add the second stream's partial sums (LDS, [key][d] fp32 per key half), then store rows.
  float* red = reinterpret_cast<float*>(smem) + kh * 32 * kKvRedStride;
  if (NS == 2 && st == 1) {
#pragma unroll
    for (int db = 0; db < 2; ++db) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = 32 * db + 8 * r4 + 4 * grp;
        *reinterpret_cast<f32x4*>(&red[l32 * kKvRedStride + d]) =
            (f32x4){dk[db][4 * r4], dk[db][4 * r4 + 1], dk[db][4 * r4 + 2], dk[db][4 * r4 + 3]};
        *reinterpret_cast<f32x4*>(&red[(64 + l32) * kKvRedStride + d]) =
            (f32x4){dv[db][4 * r4], dv[db][4 * r4 + 1], dv[db][4 * r4 + 2], dv[db][4 * r4 + 3]};
      }
    }
  }
  if (NS == 2) __syncthreads();
  if (st == 0) {
    const int key = k0 + l32;
    if (key < len) {
      // This head half's partial sums (unscaled); attn_sink_bwd_dkdv_sum_kernel adds the halves.
      const size_t plane = (size_t)a.T * a.Hkv * kHeadDim;
      float* dkrow = a.dkv_part + hh * plane + ((size_t)(cs + key) * a.Hkv + g) * kHeadDim;
      float* dvrow = a.dkv_part + (a.n_halves + hh) * plane + ((size_t)(cs + key) * a.Hkv + g) * kHeadDim;
#pragma unroll
      for (int db = 0; db < 2; ++db) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int d = 32 * db + 8 * r4 + 4 * grp;
          f32x4 kv = {dk[db][4 * r4], dk[db][4 * r4 + 1], dk[db][4 * r4 + 2], dk[db][4 * r4 + 3]};
          f32x4 vv = {dv[db][4 * r4], dv[db][4 * r4 + 1], dv[db][4 * r4 + 2], dv[db][4 * r4 + 3]};
          if (NS == 2) {
            kv += *reinterpret_cast<const f32x4*>(&red[l32 * kKvRedStride + d]);
            vv += *reinterpret_cast<const f32x4*>(&red[(64 + l32) * kKvRedStride + d]);
          }
          *reinterpret_cast<f32x4*>(dkrow + d) = kv;
          *reinterpret_cast<f32x4*>(dvrow + d) = vv;
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// 2b. dK = scale * (sum of the head halves' partials), dV = sum of the partials.
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void attn_sink_bwd_dkdv_sum_kernel(BwdArgs a) {
  const size_t plane4 = (size_t)a.T * a.Hkv * (kHeadDim / 4);  // float4 per partial plane
  const f32x4* p = reinterpret_cast<const f32x4*>(a.dkv_part);
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < plane4; i += (size_t)gridDim.x * blockDim.x) {
    f32x4 k4 = p[i], v4 = p[a.n_halves * plane4 + i];
    for (int hh = 1; hh < a.n_halves; ++hh) {
      k4 += p[hh * plane4 + i];
      v4 += p[(a.n_halves + hh) * plane4 + i];
    }
    reinterpret_cast<f32x4*>(a.dk)[i] = k4 * a.scale;
    reinterpret_cast<f32x4*>(a.dv)[i] = v4;
  }
}

// ------------------------------------------------------------------------------------------
// 3. dQ and the dSink partials: row-parallel over 32-row query blocks.
// ------------------------------------------------------------------------------------------
constexpr int kDqTileKeys = 64;
constexpr int kDqTileElems = kDqTileKeys * kLdsStride;

template <int HPW>
__global__ __launch_bounds__(64 * HPW, 2) void attn_sink_bwd_dq_kernel(BwdArgs a) {
  constexpr int NT = 64 * HPW;
  constexpr int kRows = kDqRowsPerWave;
  constexpr int KU = kDqTileKeys * 8 / NT;  // 16-byte K (and V) pieces per thread and tile
  __shared__ __attribute__((aligned(16))) __bf16 k_lds[2 * kDqTileElems];
  __shared__ __attribute__((aligned(16))) __bf16 v_lds[2 * kDqTileElems];

  const int n_hs = a.Hq / HPW;
  const int bid = blockIdx.x;
  const int inner = bid % n_hs;
  const int rest = bid / n_hs;
  const int spg = a.G / HPW;
  const int hs = (inner % a.Hkv) * spg + inner / a.Hkv;
  const int b = rest % a.B;
  const int qb = a.n_qblocks - 1 - rest / a.B;
  const int cs = a.cu[b];
  const int len = a.cu[b + 1] - cs;
  const int q0 = qb * kRows;
  if (q0 >= len) return;

  const int tid = threadIdx.x;
  const int wave = wave_id();
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int grp = lane >> 5;
  const int h = hs * HPW + wave;
  const int g = h / a.G;

  // Q^T and dO^T as B operands: lane holds query q0 + l32, d = 16c + 8grp + (0..7).
  const int qi = q0 + l32;
  const bool qok = qi < len;
  const int qc = min(qi, len - 1);  // rows past the end compute on the last row and are not stored
  bf16x8 qf[4], df[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const size_t off = ((size_t)(cs + qc) * a.Hq + h) * kHeadDim + 16 * c + 8 * grp;
    qf[c] = load_bf16x8(a.q + off);
    df[c] = load_bf16x8(a.dout + off);
  }
  const float lse2 = a.lse[(size_t)h * a.T + cs + qc] * kLog2e;
  const float dd = a.dws[(size_t)h * a.T + cs + qc];
  float dsum = 0.0f;
  f32x16 acc[2];  // dQ^T, [d block]
  acc[0] = acc[1] = zero_f32x16();

  const int kend = a.causal ? min(len, q0 + kRows) : len;
  const int kbeg = a.window > 0 ? max(0, q0 - a.window + 1) : 0;
  const int kt_begin = kbeg / kDqTileKeys;
  const int kt_end = (kend + kDqTileKeys - 1) / kDqTileKeys;
  const size_t tok_stride = (size_t)a.Hkv * kHeadDim;
  const __bf16* kbase = a.k + (size_t)cs * tok_stride + (size_t)g * kHeadDim;
  const __bf16* vbase = a.v + (size_t)cs * tok_stride + (size_t)g * kHeadDim;

  // K and V tiles in natural [key][d] layout; K^T operands come from transposing LDS loads.
  // Keys past the sequence end are clamped onto its last key (finite data; they are masked).
  bf16x8 kpre[KU], vpre[KU];
  auto prefetch = [&](int kt) {
    const int kk = kt * kDqTileKeys;
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int idx = tid + u * NT;
      const unsigned off = (unsigned)(min(kk + (idx >> 3), len - 1) * (int)tok_stride + 8 * (idx & 7));
      kpre[u] = load_bf16x8(kbase + off);
      vpre[u] = load_bf16x8(vbase + off);
    }
  };
  auto commit = [&](int buf) {
    __bf16* kl = k_lds + buf * kDqTileElems;
    __bf16* vl = v_lds + buf * kDqTileElems;
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int idx = tid + u * NT;
      const int off = (idx >> 3) * kLdsStride + 8 * (idx & 7);
      *reinterpret_cast<bf16x8*>(&kl[off]) = kpre[u];
      *reinterpret_cast<bf16x8*>(&vl[off]) = vpre[u];
    }
  };

  // Unconditional (the range is never empty here): every load issued so far is complete on every
  // path into the loop, so the loop only waits on its prefetch when committing it.
  prefetch(kt_begin);
  commit(0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): nothing issued before the loop stays in flight
  __syncthreads();

  for (int kt = kt_begin; kt < kt_end; ++kt) {
    const int cur = (kt - kt_begin) & 1;
    const bool has_next = kt + 1 < kt_end;
    if (has_next) prefetch(kt + 1);
    const __bf16* kl = k_lds + cur * kDqTileElems;
    const __bf16* vl = v_lds + cur * kDqTileElems;
    const int k0 = kt * kDqTileKeys;

    // S^T = K Q^T and dP^T = V dO^T (rows = keys, loaded with the swap23 permutation).
    f32x16 s[2], dp[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      s[mb] = zero_f32x16();
      dp[mb] = zero_f32x16();
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int row = (32 * mb + swap23(l32)) * kLdsStride + 16 * c + 8 * grp;
        s[mb] = mfma_32x32x16(load_bf16x8(&kl[row]), qf[c], s[mb]);
        dp[mb] = mfma_32x32x16(load_bf16x8(&vl[row]), df[c], dp[mb]);
      }
    }

    const bool need_mask = (k0 + kDqTileKeys > len) || (a.causal && k0 + kDqTileKeys - 1 > q0) ||
                           (a.window > 0 && k0 <= q0 + kRows - 1 - a.window);
    if (need_mask) {  // uniform: only diagonal, window-edge and ragged tiles
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kj = k0 + 32 * mb + c_row(i, grp);
          if (!visible(qi, kj, len, a.causal, a.window)) s[mb][i] = kNegInf;
        }
      }
    }
    bf16x8 dsb[2][2];
    float pmax = 0.0f, part = 0.0f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(__builtin_fmaf(s[mb][i], a.scale_log2, -lse2));
        pmax = fmaxf(pmax, p);
        const float pdp = p * dp[mb][i];
        part += pdp;
        dp[mb][i] = __builtin_fmaf(-p, dd, pdp);
      }
      dsb[mb][0] = pack8(dp[mb], 0);
      dsb[mb][1] = pack8(dp[mb], 1);
    }
    dsum += part;
    // Large probabilities: also multiply the bf16 rounding residual of dS.
    const bool split = wave_any(pmax > kSplitThreshold);

    // dQ^T += K^T dS^T (A = K^T from LDS, contracting over the tile's keys).
#pragma unroll
    for (int db = 0; db < 2; ++db) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const bf16x8 kta = load_tr8(kl, kLdsStride, 32 * mb + 16 * cc, 32 * db);  // K^T rows d, keys
          acc[db] = mfma_32x32x16(kta, dsb[mb][cc], acc[db]);
          if (split) {
            bf16x8 hi = dsb[mb][cc];
            opaque(hi);  // keeps the residual arithmetic inside this rarely taken branch
            acc[db] = mfma_32x32x16(kta, residual8(dp[mb], cc, hi), acc[db]);
          }
        }
      }
    }

    if (has_next) commit(cur ^ 1);
    __syncthreads();
  }

  // dQ row, and this wave's share of sum_i P_{i,h} D~_i.
  const float dtot = sum_xor32(dsum);
  float wsum = 0.0f;
  if (qok) {
    float* qrow = a.dq + ((size_t)(cs + qi) * a.Hq + h) * kHeadDim;
#pragma unroll
    for (int db = 0; db < 2; ++db) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        f32x4 val = {acc[db][4 * r4], acc[db][4 * r4 + 1], acc[db][4 * r4 + 2], acc[db][4 * r4 + 3]};
        *reinterpret_cast<f32x4*>(qrow + 32 * db + 8 * r4 + 4 * grp) = val * a.scale;
      }
    }
    if (grp == 0) wsum = fast_exp2(__builtin_fmaf(a.sinks[h], kLog2e, -lse2)) * dtot;
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

hipError_t launch_bwd_dkdv_sum(const BwdArgs& a, hipStream_t stream) {
  const long long n4 = (long long)a.T * a.Hkv * (kHeadDim / 4);
  if (n4 <= 0) return hipSuccess;
  long long nblocks = (n4 + 255) / 256;
  if (nblocks > 8192) nblocks = 8192;
  hipLaunchKernelGGL(attn_sink_bwd_dkdv_sum_kernel, dim3((unsigned)nblocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t stream) {
  const long long nblocks = (long long)a.n_kblocks * a.B * a.Hkv * a.n_halves;
  if (nblocks <= 0) return hipSuccess;
  if (a.kv_waves == 4) {
    hipLaunchKernelGGL(attn_sink_bwd_dkdv_kernel<2>, dim3((unsigned)nblocks), dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL(attn_sink_bwd_dkdv_kernel<1>, dim3((unsigned)nblocks), dim3(128), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t stream) {
  const long long nblocks = (long long)a.n_qblocks * (a.Hq / a.hpw) * a.B;
  if (nblocks <= 0) return hipSuccess;
  const dim3 grid((unsigned)nblocks), block(64 * a.hpw);
  switch (a.hpw) {
    case 4: hipLaunchKernelGGL(attn_sink_bwd_dq_kernel<4>, grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL(attn_sink_bwd_dq_kernel<2>, grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL(attn_sink_bwd_dq_kernel<1>, grid, block, 0, stream, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_bwd_dsink(const BwdArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(attn_sink_bwd_dsink_kernel, dim3((unsigned)a.Hq), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace attn_sink
