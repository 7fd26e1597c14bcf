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
//  1. dq:    row-parallel. A workgroup of four waves owns `hpw` heads of one group and 4 / hpw
//            blocks of 32 query rows (one head and row block per wave) and streams 64-key tiles
//            of K and V in pairs through a 4-slot LDS ring filled by direct copies one pair ahead
//            (swizzled like the dkdv tiles; K^T operands come from transposing LDS loads of the K
//            tile). Each wave first forms D_i = dO_i . O_i for its rows from the dO it holds as
//            an operand and O, and leaves -D_i and -LSE_i / scale in the workspace for pass 2.
//            Besides dQ it accumulates D~_i = sum_j P_ij dP_ij from the fp32 P and dP it already
//            holds and writes sum_i P_{i,h} D~_i for its rows. D~ equals D mathematically but
//            does not carry the bf16 rounding of the forward's P.V product, which matters
//            because the terms of dL/dS_h cancel heavily.
//  2. dkdv:  column-parallel. A workgroup owns 64 keys of one KV head and all, or one half, of
//            the group's query heads: two key halves of 32 (one per wave) times one or two "head
//            streams". Each stream walks its query rows 64 at a time through a 2-slot LDS ring
//            filled by direct global->LDS copies issued one step ahead (the two key halves of a
//            stream split the copies and share the tiles); one barrier per step. The row tiles
//            are stored with an XOR swizzle of their 16-byte chunks, which keeps both the
//            fragment reads (rows permuted by swap23) and the transposing reads of Q^T / dO^T
//            free of bank conflicts. dK^T and dV^T of each wave's 32 keys stay in registers; the
//            two streams' partial sums are added in LDS at the end. With all heads in one
//            workgroup it writes dK and dV; with head halves each half writes its own fp32
//            partial. Halves double the number of workgroups, so that (launched longest first)
//            short sequences still keep two per CU busy under a causal mask.
//  3. finish: with head halves, dK = scale * (sum of the halves), dV = sum of the halves.
//  dL/dS_h = -(sum of the partials of head h), in a fixed order, by one workgroup per query head
//  at the end of the finish launch; or, for a dK/dV launch without halves of at most
//  kDsinkFoldMaxBlocks workgroups, at the end of that launch, which then needs no finish launch
//  (one launch more cost such a step more than its work).
#include <type_traits>

#include "kernels.h"

namespace attn_sink {

namespace {

// ------------------------------------------------------------------------------------------
// 2. dK, dV: column-parallel over 64-key blocks.
// ------------------------------------------------------------------------------------------
constexpr int kKvSub = 32;        // query rows per product block
constexpr int kKvRing = 2;        // LDS ring slots per head stream
constexpr int kKvTileBytes = 8192;  // one Q or dO row tile (64 rows at D = 64, 32 at D = 128)

// Head dim D = 64 or 128. A step is one 8 KiB row tile: 64 rows (two product blocks) at D = 64,
// 32 rows at D = 128, whose dK/dV accumulators and K/V operands take twice the registers; that
// instance runs one wave per SIMD and one head stream per workgroup (two workgroups per CU).
// dL/dS_h = -(sum of head h's partials src[0 .. n_slots)), in a fixed order: each thread sums its
// slots in batches of eight loads in flight, then a shuffle tree per wave, then the waves in
// order. The dQ pass wrote every slot (a partial or a zero) whenever there are rows (T > 0, as
// cu[B] - cu[0] = T); it ran to completion before this launch began. Not inlined and given plain
// scalars: inlined into the dK/dV kernel, it changed how the compiler kept that kernel's
// arguments, and one more scalar value was reloaded inside the main loop.
template <int kWaves>
__device__ __attribute__((noinline)) void dsink_reduce(const float* src, int n_slots, int T, float* dst,
                                                       float* part) {
  constexpr int kThreads = 64 * kWaves, kBatch = 8;
  float acc = 0.0f;
  if (T > 0) {
    for (int base = threadIdx.x; base < n_slots; base += kBatch * kThreads) {
      float v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) v[u] = base + u * kThreads < n_slots ? src[base + u * kThreads] : 0.0f;
#pragma unroll
      for (int u = 0; u < kBatch; ++u) acc += v[u];
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    float sum = part[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) sum += part[w];
    *dst = -sum;
  }
}

// kDsink: the launch ends with the dSink workgroups (no head halves, few key-block workgroups).
// An instance of its own: the branch costs each workgroup two more scalar loads in a row before
// its first tile (the compiler sinks the sequence-offset loads below it), which a small launch
// repays by saving the finish launch, and a long one (thousands of workgroups) does not.
template <int NS, int D, bool kDsink>  // head streams per workgroup: 1 or 2 (waves = 2 key halves x NS)
__global__ __launch_bounds__(128 * NS, D == 64 ? 2 : 1) void attn_sink_bwd_dkdv_kernel(BwdArgs a) {
  using G_ = Geo<D>;
  constexpr int kKvRows = G_::kTileRows;                            // query rows per step
  constexpr int kSubs = kKvRows / kKvSub;                           // product blocks per step
  constexpr int kKvSlotBytes = 2 * kKvTileBytes + 2 * kKvRows * 4;  // Q, dO, -LSE/scale, -D
  constexpr int kKvStreamBytes = kKvRing * kKvSlotBytes;
  constexpr int kKvRedStride = D + 4;                               // fp32 row of the final sum
  constexpr int kRedBytes = (NS - 1) * 2 * 2 * 32 * kKvRedStride * 4;  // partials of streams 1 .. NS-1
  constexpr int kNtr = 8 * G_::kDBlocks;                            // transposing reads per block
  __shared__ __attribute__((aligned(1024)))
  unsigned char smem[NS * kKvStreamBytes > kRedBytes ? NS * kKvStreamBytes : kRedBytes];
  static_assert(kKvRing == 2, "the waits below assume one step in flight");

  // Block order: KV group fastest (consecutive ids go to different XCDs, so each XCD works on
  // few groups and their query rows stay in its L2), then head half, then the key blocks of one
  // sequence back to back, sequence after sequence. The workgroups in flight then stream the rows
  // of one or two sequences, which stay in L2 and the last-level cache between them; interleaving
  // the sequences (key block 0 of every sequence, then key block 1, ...) made the pass fetch
  // about 31 times its algorithmic bytes on 16 packed sequences of up to 8k tokens, against 5
  // times in this order, and took 40% longer. Under a causal mask the first key blocks of a
  // sequence see the most query rows, so each sequence's longest workgroups start first.
  const int bid = blockIdx.x;
  if constexpr (kDsink) {
    const int n_dkdv = a.n_kblocks * a.B * a.Hkv;
    if (bid >= n_dkdv) {  // the last Hq workgroups: dL/dS_h of one head each
      const int h = bid - n_dkdv;
      dsink_reduce<2 * NS>(a.dsink_part + (size_t)h * a.n_slots, a.n_slots, a.T, a.dsinks + h,
                           reinterpret_cast<float*>(smem));
      return;
    }
  }
  const int g = bid % a.Hkv;
  int rest = bid / a.Hkv;
  const int hh = rest % a.n_halves;
  rest /= a.n_halves;
  const int b = rest / a.n_kblocks;
  const int kblk = (rest % a.n_kblocks) * kKvKeysPerBlock;
  const int cs = a.cu[b];
  const int len = a.cu[b + 1] - cs;
  if (kblk >= len) return;  // uniform over the workgroup

  const int wave = wave_id();
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31;
  const int grp = lane >> 5;
  const int kh = wave & 1;        // key half
  const int st = wave >> 1;       // head stream
  const int k0 = kblk + 32 * kh;  // this wave's 32 keys
  const int heads_half = a.G / a.n_halves;
  const int hps = heads_half / NS;
  const int h0 = g * a.G + hh * heads_half + st;  // stream st takes heads h0 + NS * j

  // K^T and V^T as B operands (k = d, n = key): lane holds key k0 + l32, d = 16c + 8grp + 0..7.
  bf16x8 kf[G_::kChunks], vf[G_::kChunks];
  {
    const int key = min(k0 + l32, len - 1);  // keys past the end are masked
#pragma unroll
    for (int c = 0; c < G_::kChunks; ++c) {
      const size_t off = ((size_t)(cs + key) * a.Hkv + g) * D + 16 * c + 8 * grp;
      kf[c] = load_bf16x8(a.k + off);
      vf[c] = load_bf16x8(a.v + off);
    }
  }
  f32x16 dk[G_::kDBlocks], dv[G_::kDBlocks];  // [d block], C layout of dK^T / dV^T (rows d, columns keys)
#pragma unroll
  for (int db = 0; db < G_::kDBlocks; ++db) dk[db] = dv[db] = zero_f32x16();

  // Query rows that can see a key of [kblk, kblk + 64), in steps of kKvRows from the last backwards
  // (every workgroup's causal range ends at the sequence end, so the workgroups of one KV group
  // stream the same rows at about the same time and mostly hit in L2). Both key halves and both
  // streams run the same number of steps, so one barrier per step serves the whole workgroup.
  const int kmax = min(len, kblk + kKvKeysPerBlock) - 1;
  const int i_begin = a.causal ? kblk : (a.window > 0 ? max(0, kblk - a.window + 1) : 0);
  const int i_end = a.window > 0 ? min(len, kmax + a.window) : len;  // exclusive
  const int n_sub = (i_end - i_begin + kKvRows - 1) / kKvRows;
  const int n_steps = hps * n_sub;

  // Each stream owns a ring of 2 slots; step s lives in slot s % 2. The two key halves of a
  // stream split the copies of a step: half 0 copies the Q tile and the -LSE/scale, -D rows,
  // half 1 the dO tile (tile_copy_d layout). Full tiles go through buffer resources; in the last,
  // partial tile rows past the end repeat the last row (they are masked).
  unsigned char* ring = smem + st * kKvStreamBytes;
  const int qstride = a.Hq * D;  // elements per token row of q / dout
  const unsigned qrow_bytes = 2u * qstride;
  unsigned coff[2];
  tile_copy_offsets(lane, qrow_bytes, coff);
  // Step (head j, tile t) starts at row i0 = i_begin + 64 (n_sub - 1 - t) of head h0 + NS j; its
  // Q / dO rows start at element qoff = ((cs + i0) Hq + h) 64 and its -LSE/scale, -D rows at
  // roff = h T + cs + i0. The loop below steps these offsets instead of recomputing them.
  auto issue = [&](int i0, size_t qoff, size_t roff, int slot) {
    unsigned char* dst = ring + slot * kKvSlotBytes + kh * kKvTileBytes;
    const __bf16* src = (kh ? a.dout : a.q) + qoff;
    unsigned char* rows = ring + slot * kKvSlotBytes + 2 * kKvTileBytes;
    const float* nl = a.nlse + roff;
    const float* nd = a.negd + roff;
    if (i0 + kKvRows <= len) {
      const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(src, kKvRows * qrow_bytes);
#pragma unroll
      for (int u = 0; u < kKvTileBytes / 1024; ++u) tile_copy_full_d<D>(rs, coff, qrow_bytes, dst, u);
      if (kh == 0) {  // -LSE/scale rows, then -D rows (kKvRows each)
        if constexpr (kKvRows == 64) {
          bdma4(buffer_rsrc(nl, 4 * kKvRows), 4 * lane, 0, rows);
          bdma4(buffer_rsrc(nd, 4 * kKvRows), 4 * lane, 0, rows + 4 * kKvRows);
        } else {  // 32 rows of each: one copy, lanes 32-63 fetch the -D rows
          dma4(lane < 32 ? nl + lane : nd + (lane - 32), rows);
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < kKvTileBytes / 1024; ++u) tile_copy_d<D>(src, 0, len - 1 - i0, qstride, dst, u, lane);
      if (kh == 0) {
        if constexpr (kKvRows == 64) {
          dma4(nl + min(lane, len - 1 - i0), rows);
          dma4(nd + min(lane, len - 1 - i0), rows + 4 * kKvRows);
        } else {
          dma4(lane < 32 ? nl + min(lane, len - 1 - i0) : nd + min(lane - 32, len - 1 - i0), rows);
        }
      }
    }
  };
  auto wait_own_step = [&]() { wait_vmcnt<0>(); };  // this wave's copies of the current step

  // Per-lane LDS byte offsets within a 32-row block of a swizzled tile: A-operand fragments
  // (k = d) and transposing reads (k = query rows).
  int aoff[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) aoff[c] = tile_frag_off(l32, grp, c);
  int toff[2][2];  // [d block][+0 / +4 rows]
  tile_tr_offsets(lane, toff);
  // Transposed operands (see ds_read_tr16_b64_asm): Q^T (tile 0) or dO^T (tile 1) rows d = 32db + l32, k
  // slots = query rows 16*half + 8grp + 0..7 of the slot at LDS address `slot_lds`.
  // The slot and the 32-row block are compile-time constants below (the step loop is unrolled
  // over the two ring slots), so their LDS offset goes into the reads' offset fields.
  unsigned trb[2][2];  // LDS addresses of the transposing reads at offset 0 of the ring
#pragma unroll
  for (int db = 0; db < 2; ++db) {
    trb[db][0] = lds_addr(ring) + toff[db][0];
    trb[db][1] = lds_addr(ring) + toff[db][1];
  }
  // d block db lives in panel db / 2 of the tile, as d block db % 2 of that panel.
  auto tr8 = [&](auto base_tag, auto tile_tag, auto db_tag, auto half_tag, u32x2& lo, u32x2& hi) {
    constexpr int db = decltype(db_tag)::value;
    constexpr int OFF = decltype(base_tag)::value + decltype(tile_tag)::value * kKvTileBytes +
                        (db / 2) * G_::kPanelBytes + 2048 * decltype(half_tag)::value;
    lo = ds_read_tr16_b64_asm<OFF>(trb[db % 2][0]);
    hi = ds_read_tr16_b64_asm<OFF>(trb[db % 2][1]);
  };
  auto tr_all = [&](auto base_tag, u32x2 (&tr)[kNtr]) {  // [d block][query half][Q / dO][lo / hi]
    static_for<G_::kDBlocks>([&](auto db_tag) {
      constexpr int db = decltype(db_tag)::value;
      using Z = std::integral_constant<int, 0>;
      using O = std::integral_constant<int, 1>;
      tr8(base_tag, Z(), db_tag, Z(), tr[8 * db], tr[8 * db + 1]);
      tr8(base_tag, O(), db_tag, Z(), tr[8 * db + 2], tr[8 * db + 3]);
      tr8(base_tag, Z(), db_tag, O(), tr[8 * db + 4], tr[8 * db + 5]);
      tr8(base_tag, O(), db_tag, O(), tr[8 * db + 6], tr[8 * db + 7]);
    });
  };

  // One step: S' = Q K^T - LSE/scale and dP' = dO V^T - D for the 32 rows x 32 keys (the row
  // values preloaded as the accumulators; C: lane = key, registers = rows 16(i/8) + 8grp + i%8),
  // P = exp2(S' * scale * log2e), dS = P dP'; then dV^T += dO^T P and dK^T += Q^T dS. When some
  // probability of the step exceeds kSplitThresholdDk (kSplitThreshold), the bf16 rounding
  // residuals of dS (and of P) are multiplied too, right after the main products.
  auto step = [&](auto si_tag, auto sub_tag, int i0, bool need_mask) {
    constexpr int SI = decltype(si_tag)::value, SUB = decltype(sub_tag)::value;
    constexpr int SO = SI * kKvSlotBytes + 4096 * SUB;  // 32-row block SUB of slot SI's tiles
    const unsigned char* slot = ring + SO;
    const float* lp = reinterpret_cast<const float*>(ring + SI * kKvSlotBytes + 2 * kKvTileBytes) + kKvSub * SUB;
    f32x16 sc = load_rows16(lp, grp);
    f32x16 dp = load_rows16(lp + kKvRows, grp);  // -D rows follow the kKvRows -LSE/scale rows
#pragma unroll
    for (int c = 0; c < G_::kChunks; ++c) {
      sc = mfma_32x32x16(*reinterpret_cast<const bf16x8*>(slot + frag_off<D>(aoff, c, 0)), kf[c], sc);
      dp = mfma_32x32x16(*reinterpret_cast<const bf16x8*>(slot + kKvTileBytes + frag_off<D>(aoff, c, 0)), vf[c],
                         dp);
    }
    u32x2 tr[kNtr];
    tr_all(std::integral_constant<int, SO>(), tr);
    if (need_mask) {
      // Row of register i: i0 + 8grp + r_i with r_i = 16(i/8) + i%8. Key kj is seen by the
      // rows lo .. hi: from the key itself (causal) or W - 1 rows before it (a non-causal
      // window), up to W - 1 rows after it (any window), within the sequence; none if the key
      // is past the end. (The empty asm keeps the arithmetic in this branch.)
      int kj = k0 + l32;
      asm volatile("" : "+v"(kj));
      const int lo = a.causal ? kj : (a.window > 0 ? kj - a.window + 1 : 0);
      const int hi = kj >= len ? lo - 1 : (a.window > 0 ? min(len - 1, kj + a.window - 1) : len - 1);
      const unsigned cnt = (unsigned)max(hi - lo + 1, 0);
      const int base = i0 + 8 * grp - lo;  // row - lo for r_i = 0
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sc[i] = in_span(base + 16 * (i >> 3) + (i & 7), cnt) ? sc[i] : kNegInf;
      }
    }
    float pmax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = fast_exp2(sc[i] * a.scale_log2);
      pmax = fmaxf(pmax, p);
      sc[i] = p;
      dp[i] *= p;
    }
    const bf16x8 pb0 = pack8(sc, 0), pb1 = pack8(sc, 1);
    const bf16x8 sb0 = pack8(dp, 0), sb1 = pack8(dp, 1);
    wait_lds_into(tr);
#pragma unroll
    for (int db = 0; db < G_::kDBlocks; ++db) {
      const u32x2* t = tr + 8 * db;
      dv[db] = mfma_32x32x16(join_tr(t[2], t[3]), pb0, dv[db]);
      dv[db] = mfma_32x32x16(join_tr(t[6], t[7]), pb1, dv[db]);
      dk[db] = mfma_32x32x16(join_tr(t[0], t[1]), sb0, dk[db]);
      dk[db] = mfma_32x32x16(join_tr(t[4], t[5]), sb1, dk[db]);
    }
    if (wave_any(pmax > kSplitThresholdDk)) {
      const bf16x8 sl0 = residual8(dp, 0, sb0), sl1 = residual8(dp, 1, sb1);
#pragma unroll
      for (int db = 0; db < G_::kDBlocks; ++db) {
        const u32x2* t = tr + 8 * db;
        dk[db] = mfma_32x32x16(join_tr(t[0], t[1]), sl0, dk[db]);
        dk[db] = mfma_32x32x16(join_tr(t[4], t[5]), sl1, dk[db]);
      }
      if (wave_any(pmax > kSplitThreshold)) {
        const bf16x8 pl0 = residual8(sc, 0, pb0), pl1 = residual8(sc, 1, pb1);
#pragma unroll
        for (int db = 0; db < G_::kDBlocks; ++db) {
          const u32x2* t = tr + 8 * db;
          dv[db] = mfma_32x32x16(join_tr(t[2], t[3]), pl0, dv[db]);
          dv[db] = mfma_32x32x16(join_tr(t[6], t[7]), pl1, dv[db]);
        }
      }
    }
  };

  // The next step to issue (wave-uniform): tile index, first row and offsets.
  int nx_t = 0;
  int nx_i0 = i_begin + kKvRows * (n_sub - 1);
  size_t nx_qoff = ((size_t)(cs + nx_i0) * a.Hq + h0) * D;
  size_t nx_roff = (size_t)h0 * a.T + cs + nx_i0;
  const size_t tile_q = (size_t)kKvRows * qstride;                            // one tile back
  const size_t head_q = (size_t)NS * D + (size_t)(n_sub - 1) * tile_q;  // next head's last tile
  const size_t head_r = (size_t)NS * a.T + (size_t)(n_sub - 1) * kKvRows;
  auto issue_next = [&](int slot) {
    issue(nx_i0, nx_qoff, nx_roff, slot);
    if (++nx_t == n_sub) {
      nx_t = 0;
      nx_i0 += kKvRows * (n_sub - 1);
      nx_qoff += head_q;
      nx_roff += head_r;
    } else {
      nx_i0 -= kKvRows;
      nx_qoff -= tile_q;
      nx_roff -= kKvRows;
    }
  };

  // Which 32-row blocks (first row i0) a wave computes, and which of them need the mask, as
  // ranges of i0 fixed per wave: live iff live_lo <= i0 <= live_hi (causal: the block reaches the
  // wave's first key; window: it starts before the last key's window ends; band: it ends after the
  // first key's window starts; inside the sequence, and no block when the keys are past its end).
  // The mask is needed iff i0 < mask_lo (diagonal, band's left edge) or i0 > mask_hi (sequence
  // end, window's right edge), or always when some key is past the end.
  constexpr int kBig = 1 << 29;
  const int W = a.window;
  int live_lo = a.causal ? k0 - (kKvSub - 1) : (W > 0 ? k0 - (kKvSub - 2) - W : -kBig);
  const int live_hi = min(len - 1, W > 0 ? k0 + 30 + W : kBig);
  if (k0 >= len) live_lo = kBig;
  const int mask_lo = k0 + 32 > len ? kBig : (a.causal ? k0 + 31 : (W > 0 ? k0 + 32 - W : -kBig));
  const int mask_hi = min(len - kKvSub - 1, W > 0 ? k0 + W - 32 : kBig);

  int cur_i0 = nx_i0;  // first row of the current step
  issue_next(0);
  static_assert(kKvRing == 2 && kKvRows % kKvSub == 0, "two slots, whole 32-row blocks per step");
  auto do_step = [&](int s, auto si_tag) {  // step s, held in slot SI = s % 2
    constexpr int SI = decltype(si_tag)::value;
    wait_own_step();
    // Both halves of step s have landed, and every wave is done with step s - 1, whose slot
    // receives step s + 1.
    __syncthreads();
    const int i0 = cur_i0;
    if (s + 1 < n_steps) {
      cur_i0 = nx_i0;
      issue_next(1 - SI);
    }
    // Wave-uniform: skip blocks without visible pairs.
    if (i0 >= live_lo && i0 <= live_hi) {
      step(si_tag, std::integral_constant<int, 0>(), i0, i0 < mask_lo || i0 > mask_hi);
    }
    if constexpr (kSubs == 2) {
      const int i1 = i0 + kKvSub;
      if (i1 >= live_lo && i1 <= live_hi) {
        step(si_tag, std::integral_constant<int, 1>(), i1, i1 < mask_lo || i1 > mask_hi);
      }
    }
  };
  for (int s = 0; s < n_steps; s += 2) {
    do_step(s, std::integral_constant<int, 0>());
    if (s + 1 < n_steps) do_step(s + 1, std::integral_constant<int, 1>());
  }

  // Streams 1 .. NS-1 leave their partial sums in LDS ([dk, dv][key][d] fp32 per (stream, key
  // half)); stream 0 adds them in stream order and stores the rows.
  float* red = reinterpret_cast<float*>(smem);
  constexpr int kRedPlane = 2 * 32 * kKvRedStride;
  if (NS > 1) {
    __syncthreads();  // every wave is done with its ring
    if (st > 0) {
      float* r = red + ((st - 1) * 2 + kh) * kRedPlane;
#pragma unroll
      for (int db = 0; db < G_::kDBlocks; ++db) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int d = 32 * db + 8 * r4 + 4 * grp;
          *reinterpret_cast<f32x4*>(&r[l32 * kKvRedStride + d]) =
              (f32x4){dk[db][4 * r4], dk[db][4 * r4 + 1], dk[db][4 * r4 + 2], dk[db][4 * r4 + 3]};
          *reinterpret_cast<f32x4*>(&r[(32 + l32) * kKvRedStride + d]) =
              (f32x4){dv[db][4 * r4], dv[db][4 * r4 + 1], dv[db][4 * r4 + 2], dv[db][4 * r4 + 3]};
        }
      }
    }
    __syncthreads();
  }
  if (st == 0) {
    const int key = k0 + l32;
    if (key < len) {
      // With one head half these are dK (scaled here) and dV; otherwise this half's unscaled
      // partial sums, which attn_sink_bwd_finish_kernel adds and scales.
      const size_t plane = (size_t)a.T * a.Hkv * D;
      const size_t row = ((size_t)(cs + key) * a.Hkv + g) * D;
      const bool direct = a.n_halves == 1;
      float* dkrow = direct ? a.dk + row : a.dkv_part + hh * plane + row;
      float* dvrow = direct ? a.dv + row : a.dkv_part + (a.n_halves + hh) * plane + row;
      const float kscale = direct ? a.scale : 1.0f;
#pragma unroll
      for (int db = 0; db < G_::kDBlocks; ++db) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int d = 32 * db + 8 * r4 + 4 * grp;
          f32x4 kv = {dk[db][4 * r4], dk[db][4 * r4 + 1], dk[db][4 * r4 + 2], dk[db][4 * r4 + 3]};
          f32x4 vv = {dv[db][4 * r4], dv[db][4 * r4 + 1], dv[db][4 * r4 + 2], dv[db][4 * r4 + 3]};
#pragma unroll
          for (int o = 0; o < NS - 1; ++o) {
            const float* r = red + (o * 2 + kh) * kRedPlane;
            kv += *reinterpret_cast<const f32x4*>(&r[l32 * kKvRedStride + d]);
            vv += *reinterpret_cast<const f32x4*>(&r[(32 + l32) * kKvRedStride + d]);
          }
          *reinterpret_cast<f32x4*>(dkrow + d) = kv * kscale;
          *reinterpret_cast<f32x4*>(dvrow + d) = vv;
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// 1. dQ, D and the dSink partials: row-parallel over 32-row query blocks.
// ------------------------------------------------------------------------------------------
constexpr int kDqTileBytes = 8192;             // one swizzled K or V tile (64 keys at D = 64, 32 at D = 128)
constexpr int kDqSlotBytes = 2 * kDqTileBytes;  // K tile, then V tile
constexpr int kDqRing = 4;                      // LDS ring slots (two pairs of tiles)

// HPW query heads of one KV group x RPW = 4 / HPW blocks of 32 rows per workgroup (four waves).
template <int HPW, int D>
__global__ __launch_bounds__(256, 2) void attn_sink_bwd_dq_kernel(BwdArgs a) {
  using G_ = Geo<D>;
  constexpr int kDqTileKeys = G_::kTileRows;
  constexpr int MB = G_::kRowBlocks;                    // 32-key blocks per tile
  constexpr int kRows = kDqRowsPerWave;                 // query rows per wave
  constexpr int RPW = 4 / HPW;                          // row blocks per workgroup
  constexpr int CPW = 2 * (kDqTileBytes / 1024) / 4;    // copies per wave and tile (K and V)
  constexpr int NTR = G_::kDBlocks * MB * 4;            // transposing reads of K^T per tile
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kDqRing * kDqSlotBytes];

  const int n_hs = a.Hq / HPW;
  const int bid = blockIdx.x;
  const int inner = bid % n_hs;
  const int rest = bid / n_hs;
  const int spg = a.G / HPW;
  const int hs = (inner % a.Hkv) * spg + inner / a.Hkv;
  // Row blocks of one sequence back to back (its K/V tiles stay in L2), the last (longest under
  // a causal mask) first; sequence after sequence.
  const int b = rest / a.n_qblocks;
  const int cs = a.cu[b];
  const int len = a.cu[b + 1] - cs;
  const int qw0 = (a.n_qblocks - 1 - rest % a.n_qblocks) * kRows * RPW;  // longest causal rows first
  if (qw0 >= len) return;

  const int wave = wave_id();
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31;
  const int grp = lane >> 5;
  const int h = hs * HPW + wave % HPW;
  const int g = h / a.G;
  const int q0 = qw0 + kRows * (wave / HPW);  // this wave's first row
  const int qb = q0 / kRows;                   // its row block within the sequence
  const bool rows_live = RPW == 1 || q0 < len;  // waves past the sequence end only copy

  // Q^T and dO^T as B operands: lane holds query q0 + l32, d = 16c + 8grp + (0..7).
  const int qi = q0 + l32;
  const bool qok = qi < len;
  const int qc = min(qi, len - 1);  // rows past the end compute on the last row and are not stored
  bf16x8 qf[G_::kChunks], df[G_::kChunks];
#pragma unroll
  for (int c = 0; c < G_::kChunks; ++c) {
    const size_t off = ((size_t)(cs + qc) * a.Hq + h) * D + 16 * c + 8 * grp;
    qf[c] = load_bf16x8(a.q + off);
    df[c] = load_bf16x8(a.dout + off);
  }
  // D_i = dO_i . O_i: this lane's 32 products (the d positions of its dO operand), then the other
  // half of the row from lane ^ 32. -D_i and -LSE_i / scale go to the workspace for the dK/dV pass.
  float dpart = 0.0f;
  {
    const float* orow = a.out + ((size_t)(cs + qc) * a.Hq + h) * D + 8 * grp;
#pragma unroll
    for (int c = 0; c < G_::kChunks; ++c) {
      const f32x4 o0 = *reinterpret_cast<const f32x4*>(orow + 16 * c);
      const f32x4 o1 = *reinterpret_cast<const f32x4*>(orow + 16 * c + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dpart = __builtin_fmaf(o0[e], (float)df[c][e], dpart);
        dpart = __builtin_fmaf(o1[e], (float)df[c][4 + e], dpart);
      }
    }
  }
  const float nd = -sum_xor32(dpart);                              // -D_i
  const float nl = -a.lse[(size_t)h * a.T + cs + qc] / a.scale;   // -LSE_i / scale
  const float lse2 = -nl * a.scale_log2;                           // LSE_i * log2(e)
  if (qok && grp == 0) a.nlse[(size_t)h * a.T + cs + qi] = nl;
  float dsum = 0.0f;
  f32x16 acc[G_::kDBlocks];  // dQ^T, [d block]
#pragma unroll
  for (int db = 0; db < G_::kDBlocks; ++db) acc[db] = zero_f32x16();

  // Keys a row range can see (as in the forward): the workgroup streams its whole range's tiles,
  // each wave computes only its own.
  auto key_end = [&](int r1) {  // rows before r1
    return a.causal ? min(len, r1) : (a.window > 0 ? min(len, r1 - 1 + a.window) : len);
  };
  auto key_begin = [&](int r0) { return a.window > 0 ? max(0, r0 - a.window + 1) : 0; };
  const int kt_begin = key_begin(qw0) / kDqTileKeys;
  const int kt_end = (key_end(qw0 + kRows * RPW) + kDqTileKeys - 1) / kDqTileKeys;
  const int kw_begin = key_begin(q0);
  const int kw_end = rows_live ? key_end(q0 + kRows) : 0;
  const int kv_stride = a.Hkv * D;
  const __bf16* kbase = a.k + (size_t)cs * kv_stride + (size_t)g * D;
  const __bf16* vbase = a.v + (size_t)cs * kv_stride + (size_t)g * D;

  // K and V tiles of kDqTileKeys keys, swizzled (see tile_swz), in a 4-slot ring filled by direct
  // global->LDS copies issued one pair of tiles ahead; the waves split each tile's 16 copies (waves 0-1
  // the K tile, 2-3 the V tile). Full tiles go through a buffer resource; in the last, partial
  // tile keys past the sequence end repeat its last key (finite data; they are masked).
  static_assert(8 % CPW == 0, "a wave's copies stay within one tile");
  const unsigned row_bytes = 2u * kv_stride;
  unsigned coff[2];
  tile_copy_offsets(lane, row_bytes, coff);
  // Tiles are issued in order, so the next one's source advances by a tile per issue.
  const int u0 = wave * CPW;  // copies u0 .. u0 + CPW - 1 of 16: K for u < 8, V after
  const bool is_v = u0 >= 8;
  const size_t tile_elems = (size_t)kDqTileKeys * kv_stride;
  const __bf16* nx_src = (is_v ? vbase : kbase) + (size_t)kt_begin * tile_elems;
  int nx_kt = kt_begin;
  auto issue_next = [&]() {
    unsigned char* tile = ring + ((unsigned)(nx_kt - kt_begin) % kDqRing) * kDqSlotBytes + (is_v ? kDqTileBytes : 0);
    const int row0 = nx_kt * kDqTileKeys;
    if (row0 + kDqTileKeys <= len) {
      const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(nx_src, kDqTileKeys * row_bytes);
#pragma unroll
      for (int i = 0; i < CPW; ++i) tile_copy_full_d<D>(rs, coff, row_bytes, tile, (u0 + i) & 7);
    } else {
#pragma unroll
      for (int i = 0; i < CPW; ++i) tile_copy_d<D>(nx_src, 0, len - 1 - row0, kv_stride, tile, (u0 + i) & 7, lane);
    }
    nx_src += tile_elems;
    ++nx_kt;
  };

  int aoff[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) aoff[c] = tile_frag_off(l32, grp, c);
  int toff[2][2];
  tile_tr_offsets(lane, toff);
  const unsigned ring_lds = lds_addr(ring);

  // Tiles (first key k0) that need the mask, as ranges fixed per wave: k0 > mask_hi when the
  // sequence end, the diagonal or a band's right edge reaches into the tile, k0 < mask_lo when a
  // window's left edge does.
  constexpr int kBig = 1 << 29;
  const int mask_hi = min(len - kDqTileKeys - 1,
                          a.causal ? q0 - kDqTileKeys : (a.window > 0 ? q0 + a.window - kDqTileKeys : kBig));
  const int mask_lo = a.window > 0 ? q0 + kRows - a.window : -kBig;

  issue_next();
  if (kt_begin + 1 < kt_end) issue_next();

  for (int kt = kt_begin; kt < kt_end; ++kt) {
    const unsigned j = kt - kt_begin;  // tiles go in pairs: one wait and one barrier per pair
    if ((j & 1) == 0) {
      wait_vmcnt<0>();  // this wave's copies of tiles kt and kt + 1
      // Every wave's copies of tiles kt and kt + 1 have landed, and every wave is done with tiles
      // kt - 2 and kt - 1, whose slots receive tiles kt + 2 and kt + 3.
      __syncthreads();
      if (kt + 2 < kt_end) issue_next();
      if (kt + 3 < kt_end) issue_next();
    }
    const int k0 = kt * kDqTileKeys;
    // Wave-uniform: skip a tile that holds none of this wave's keys.
    if (RPW > 1 && (k0 >= kw_end || k0 + kDqTileKeys <= kw_begin)) continue;

    const bool need_mask = k0 > mask_hi || k0 < mask_lo;
    // One tile: S^T = K Q^T and dP^T = V dO^T (rows = keys, loaded with the swap23 permutation),
    // P = exp2(S*scale*log2e - LSE*log2e), dS = P (dP - D), dQ^T += K^T dS^T, one 32-key block
    // after the other so that block 1's softmax overlaps block 0's dQ products. A block whose
    // largest probability exceeds kSplitThreshold also multiplies the bf16 rounding residual of
    // its dS.
    auto tile = [&](unsigned lds_off) {
      const unsigned char* slot = ring + lds_off;
      const unsigned slot_lds = ring_lds + lds_off;
      f32x16 s[MB], dp[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        s[mb] = zero_f32x16();
        dp[mb] = zero_f32x16();
#pragma unroll
        for (int c = 0; c < G_::kChunks; ++c) {
          s[mb] = mfma_32x32x16(*reinterpret_cast<const bf16x8*>(slot + frag_off<D>(aoff, c, mb)), qf[c], s[mb]);
          dp[mb] = mfma_32x32x16(*reinterpret_cast<const bf16x8*>(slot + kDqTileBytes + frag_off<D>(aoff, c, mb)),
                                 df[c], dp[mb]);
        }
      }
      // K^T operands for dQ^T (rows d = 32db + l32, k slots = keys 32mb + 16cc + 8grp + 0..7):
      // tr[4 (db MB + mb) + 2 cc + lo/hi], from panel db / 2 at rows 32mb + 16cc.
      u32x2 tr[NTR];
      static_for<G_::kDBlocks>([&](auto db_tag) {
        constexpr int db = decltype(db_tag)::value;
        constexpr int PO = (db / 2) * G_::kPanelBytes;
        static_for<MB>([&](auto mb_tag) {
          constexpr int mb = decltype(mb_tag)::value;
          tr[4 * (db * MB + mb) + 0] = ds_read_tr16_b64_asm<PO + 4096 * mb>(slot_lds + toff[db % 2][0]);
          tr[4 * (db * MB + mb) + 1] = ds_read_tr16_b64_asm<PO + 4096 * mb>(slot_lds + toff[db % 2][1]);
          tr[4 * (db * MB + mb) + 2] = ds_read_tr16_b64_asm<PO + 4096 * mb + 2048>(slot_lds + toff[db % 2][0]);
          tr[4 * (db * MB + mb) + 3] = ds_read_tr16_b64_asm<PO + 4096 * mb + 2048>(slot_lds + toff[db % 2][1]);
        });
      });
      float part = 0.0f;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        float pmax = 0.0f;
        if (need_mask) {  // uniform: only diagonal, window-edge and ragged tiles
          const KeyBounds kb = key_bounds(qi, len, a.causal, a.window);
          const unsigned cnt = (unsigned)max(kb.hi - kb.lo, 0);  // visible keys kb.lo + 1 .. kb.hi
          const int base = k0 + 32 * mb + 8 * grp - kb.lo - 1;   // key - (kb.lo + 1) for register 0
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            s[mb][i] = in_span(base + 16 * (i >> 3) + (i & 7), cnt) ? s[mb][i] : kNegInf;
          }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = fast_exp2(__builtin_fmaf(s[mb][i], a.scale_log2, -lse2));
          pmax = fmaxf(pmax, p);
          const float pdp = p * dp[mb][i];
          part += pdp;
          dp[mb][i] = __builtin_fmaf(p, nd, pdp);
        }
        const bf16x8 d0 = pack8(dp[mb], 0), d1 = pack8(dp[mb], 1);
        if (mb == 0) wait_lds_into(tr);
#pragma unroll
        for (int db = 0; db < G_::kDBlocks; ++db) {
          const u32x2* t = tr + 4 * (db * MB + mb);
          acc[db] = mfma_32x32x16(join_tr(t[0], t[1]), d0, acc[db]);
          acc[db] = mfma_32x32x16(join_tr(t[2], t[3]), d1, acc[db]);
        }
        if (wave_any(pmax > kSplitThreshold)) {
          const bf16x8 d0l = residual8(dp[mb], 0, d0), d1l = residual8(dp[mb], 1, d1);
#pragma unroll
          for (int db = 0; db < G_::kDBlocks; ++db) {
            const u32x2* t = tr + 4 * (db * MB + mb);
            acc[db] = mfma_32x32x16(join_tr(t[0], t[1]), d0l, acc[db]);
            acc[db] = mfma_32x32x16(join_tr(t[2], t[3]), d1l, acc[db]);
          }
        }
      }
      dsum += part;
    };
    tile((j % kDqRing) * kDqSlotBytes);
  }

  // dQ row, -D~_i for the dK/dV pass, and this wave's share of sum_i P_{i,h} D~_i.
  const float dtot = sum_xor32(dsum);
  if (qok && grp == 0) a.negd[(size_t)h * a.T + cs + qi] = -dtot;
  float wsum = 0.0f;
  if (qok && grp == 0) wsum = fast_exp2(__builtin_fmaf(a.sinks[h], kLog2e, -lse2)) * dtot;
  // dQ goes through LDS: a lane holds 4-float pieces of one row, so direct stores would put
  // 32-byte pieces of 32 rows in each store instruction; from LDS each instruction writes whole
  // rows. Each wave stages its kRows x D tile in its part of the ring (free once every wave is
  // done with the last tile), 16-byte chunk k of row r at chunk k ^ (r % kCpr).
  {
    constexpr int kCpr = D / 4;      // 16-byte chunks per dQ row
    constexpr int kRpi = 64 / kCpr;  // rows per store instruction
    static_assert(4 * kRows * D * 4 <= kDqRing * kDqSlotBytes, "four staged tiles fit in the ring");
    __syncthreads();
    float* stage = reinterpret_cast<float*>(ring) + wave * kRows * D;
#pragma unroll
    for (int db = 0; db < G_::kDBlocks; ++db) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int k = 8 * db + 2 * r4 + grp;  // d = 4k .. 4k + 3
        const f32x4 val = {acc[db][4 * r4], acc[db][4 * r4 + 1], acc[db][4 * r4 + 2], acc[db][4 * r4 + 3]};
        *reinterpret_cast<f32x4*>(stage + l32 * D + 4 * (k ^ (l32 % kCpr))) = val * a.scale;
      }
    }
    const int k = lane % kCpr;
#pragma unroll
    for (int it = 0; it < kRows / kRpi; ++it) {
      const int r = kRpi * it + lane / kCpr;
      const f32x4 val = *reinterpret_cast<const f32x4*>(stage + r * D + 4 * (k ^ (r % kCpr)));
      if (q0 + r < len) *reinterpret_cast<f32x4*>(a.dq + ((size_t)(cs + q0 + r) * a.Hq + h) * D + 4 * k) = val;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) wsum += __shfl_xor(wsum, off);
  if (lane == 0 && rows_live) {  // a wave past the sequence end has no slot
    // Unique slot per (sequence, row block): floor(cs / rows) + b + qb never collides.
    const int slot = cs / kRows + b + qb;
    a.dsink_part[(size_t)h * a.n_slots + slot] = wsum;
  }
  // The slots no row block maps to (a few between consecutive sequences with rows, those before
  // the first and after the last) get zeros from the neighbouring first / last row blocks, so
  // that every slot is written exactly once and the dSink workgroups can sum all of them.
  if (rows_live) {
    float* part = a.dsink_part + (size_t)h * a.n_slots;
    if (q0 + kRows >= len) {  // last row block: up to the first slot of the next sequence with rows
      int nb = b + 1;
      while (nb < a.B && a.cu[nb + 1] == a.cu[nb]) ++nb;
      const int to = nb < a.B ? a.cu[nb] / kRows + nb : a.n_slots;
      for (int j = cs / kRows + b + qb + 1 + lane; j < to; j += 64) part[j] = 0.0f;
    }
    if (q0 == 0 && cs == a.cu[0]) {  // first row block of the first sequence with rows
      for (int j = lane; j < cs / kRows + b; j += 64) part[j] = 0.0f;
    }
  }
}

// ------------------------------------------------------------------------------------------
// 3. Finish (head halves only): dK = scale * (sum of the halves' partials), dV = sum of the
//    partials (blocks below n_sum_blocks, grid-stride over float4s), then dL/dS_h (one block
//    per head after those).
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void attn_sink_bwd_finish_kernel(BwdArgs a, int n_sum_blocks) {
  if ((int)blockIdx.x >= n_sum_blocks) {
    __shared__ float part[4];
    const int h = blockIdx.x - n_sum_blocks;
    dsink_reduce<4>(a.dsink_part + (size_t)h * a.n_slots, a.n_slots, a.T, a.dsinks + h, part);
    return;
  }
  const size_t plane4 = (size_t)a.T * a.Hkv * (a.D / 4);  // float4 per partial plane
  const f32x4* p = reinterpret_cast<const f32x4*>(a.dkv_part);
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < plane4; i += (size_t)n_sum_blocks * blockDim.x) {
    f32x4 k4 = p[i], v4 = p[a.n_halves * plane4 + i];
    for (int hh = 1; hh < a.n_halves; ++hh) {
      k4 += p[hh * plane4 + i];
      v4 += p[(a.n_halves + hh) * plane4 + i];
    }
    reinterpret_cast<f32x4*>(a.dk)[i] = k4 * a.scale;
    reinterpret_cast<f32x4*>(a.dv)[i] = v4;
  }
}

}  // namespace

static constexpr long long kDsinkFoldMaxBlocks = 2048;

// Whether the dK/dV launch reduces dSink itself (and no finish kernel is launched).
static bool dsink_in_dkdv(const BwdArgs& a) {
  return a.n_halves == 1 && (long long)a.n_kblocks * a.B * a.Hkv <= kDsinkFoldMaxBlocks;
}

template <int D, bool kDsink>
void launch_dkdv_d(const BwdArgs& a, dim3 grid, hipStream_t stream) {
  if (D == 64 && a.kv_streams == 2) {  // head_dim 128 always runs one stream per workgroup
    hipLaunchKernelGGL((attn_sink_bwd_dkdv_kernel<2, 64, kDsink>), grid, dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL((attn_sink_bwd_dkdv_kernel<1, D, kDsink>), grid, dim3(128), 0, stream, a);
  }
}

hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t stream) {
  // key-block workgroups, then possibly one dSink workgroup per query head
  const bool with_dsink = dsink_in_dkdv(a);
  const long long nblocks = (long long)a.n_kblocks * a.B * a.Hkv * a.n_halves + (with_dsink ? a.Hq : 0);
  if (nblocks <= 0) return hipSuccess;
  const dim3 grid((unsigned)nblocks);
  if (a.D == 128) {
    with_dsink ? launch_dkdv_d<128, true>(a, grid, stream) : launch_dkdv_d<128, false>(a, grid, stream);
  } else {
    with_dsink ? launch_dkdv_d<64, true>(a, grid, stream) : launch_dkdv_d<64, false>(a, grid, stream);
  }
  return hipGetLastError();
}

template <int D>
void launch_dq_d(const BwdArgs& a, dim3 grid, hipStream_t stream) {
  const dim3 block(256);
  switch (a.hpw) {
    case 4: hipLaunchKernelGGL((attn_sink_bwd_dq_kernel<4, D>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((attn_sink_bwd_dq_kernel<2, D>), grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL((attn_sink_bwd_dq_kernel<1, D>), grid, block, 0, stream, a); break;
  }
}

hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t stream) {
  const long long nblocks = (long long)a.n_qblocks * (a.Hq / a.hpw) * a.B;
  if (nblocks <= 0) return hipSuccess;
  if (a.D == 128) {
    launch_dq_d<128>(a, dim3((unsigned)nblocks), stream);
  } else {
    launch_dq_d<64>(a, dim3((unsigned)nblocks), stream);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_finish(const BwdArgs& a, hipStream_t stream) {
  if (dsink_in_dkdv(a)) return hipSuccess;  // the dK/dV launch wrote dK, dV and dSink itself
  const long long n4 = (long long)a.T * a.Hkv * (a.D / 4);
  long long nsum = (n4 + 255) / 256;
  if (nsum > 4096) nsum = 4096;
  if (a.n_halves == 1) nsum = 0;  // the dK/dV pass wrote dK and dV itself
  hipLaunchKernelGGL(attn_sink_bwd_finish_kernel, dim3((unsigned)(nsum + a.Hq)), dim3(256), 0, stream, a, (int)nsum);
  return hipGetLastError();
}

}  // namespace attn_sink
