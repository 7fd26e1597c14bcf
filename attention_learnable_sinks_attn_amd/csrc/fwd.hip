// Forward of attention with a learnable per-head sink, for gfx950.
//
// Math (nmedialink.com "惊爆！GPT-OSS-20B强化学习…", section "GPT-OSS中的带注意力槽的注意力机制"
// and section "数学公式深入解读", eq. P_ij): each row's softmax runs over the visible scores plus
// one extra logit S_h, and the output only sums the visible keys' values. Written as an online
// softmax, the sink is simply the first element the row has seen: the running max starts at S_h
// and the running denominator at exp(S_h - S_h) = 1, while the output accumulator starts at 0
// because the sink has no value row. LSE = max + log(denominator) therefore includes the sink.
//
// Head dim D = 64 or 128 (rows stored as 64-element panels, tiles of 8 KiB: 64 keys at D = 64, 32
// at D = 128; see Geo in common.h). Per wave 64 query rows at D = 64, 32 at D = 128 (whose O^T
// accumulators are twice as tall).
//
// Work split. A workgroup of four waves owns HPW query heads that share one KV head (GQA) and
// 4 / HPW consecutive blocks of query rows of one sequence; wave w handles head hs*HPW + w%HPW
// and row block w/HPW. K and V tiles of 64 keys pass in pairs through a 4-slot LDS ring shared by
// the workgroup's waves, filled by direct global->LDS copies one pair ahead (the waves split the
// copies); one barrier per pair of tiles; a wave skips the tiles its rows cannot see. The tiles are stored with
// an XOR swizzle of their 16-byte chunks (tile_swz), so that neither the K fragment reads nor the
// transposing V^T reads have bank conflicts. Per tile each wave computes
//   S^T = K Q^T   (32x32x16 MFMA; keys on the C rows, the wave's 64 queries on the columns)
// so that each lane owns one query: the row max and row sum are lane-local plus one exchange
// with lane ^ 32, and the probabilities, rounded to bf16, are already laid out as the B operand
// of the second product
//   O^T += V^T P^T,
// whose V^T operand is read from the natural [key][d] V tile with transposing LDS loads.
// The two 32-query column blocks are processed one after the other, so the second block's
// softmax (VALU) can overlap the first block's P.V products (MFMA).
//
// The reference max is lazy: the sum and the accumulator are only rescaled when some row of a
// 32-query block sees a score more than 2^8 above its reference, so the unnormalised values
// exp2(s - m) stay below 256 and most tiles skip the rescale. Their bf16 rounding is then not
// exact for a row's largest value, and tiles where a value can reach an eighth of its row's
// probability mass also multiply the rounding residuals (see the tile body).
#include <type_traits>

#include "kernels.h"

namespace attn_sink {

namespace {

constexpr int kTileBytes = 8192;              // one swizzled K or V tile (64 keys at D = 64, 32 at D = 128)
constexpr int kSlotBytes = 2 * kTileBytes;    // K tile, then V tile
constexpr int kRing = 4;                      // LDS ring slots (two pairs of tiles)
// Probabilities above this share of their row get the residual P.V product (see the tile body).
// The largest ones dominate the rounding error of O, and through D = dO . O that of every dS of
// the row in the dQ pass, which grows with head_dim and the softmax scale: at a quarter, a
// head_dim-128 batch with three times the default scale put dQ at 1.08e-2; at an eighth, 3.7e-3.
// On N(0,1) inputs at the default scale about a tenth of the (row block, tile) units take it.
constexpr float kFwdSplitThreshold = 0.125f;
// Growth of a row's maximum (log2 units) that forces a rescale of its sum and accumulator.
constexpr float kLazyMax = 8.0f;

// The online softmax of one wave over NB blocks of 32 query columns: the queries' Q^T operands,
// the running maxima (log2 units), partial denominators (this lane's half of the keys) and O^T
// accumulators, and the work on one K/V tile. A column's arithmetic depends only on its own
// scores: the rescale and the residual product are decided per wave (one branch) but applied only
// to the columns that need them (the others multiply by exactly 1 and add exactly 0), and tiles
// without a visible key leave a column unchanged. So a column's result is the same, bit for bit,
// in whatever wave, next to whatever other columns, it is computed, as long as it sees the same
// tiles in the same order; the order-preserving decode kernel relies on this.
template <int D, int NB>
struct FwdCols {
  using G_ = Geo<D>;
  static constexpr int MB = G_::kRowBlocks;              // 32-key blocks per tile
  static constexpr int NTR = G_::kDBlocks * MB * 4;      // transposing reads of V^T per tile
  bf16x8 qf[NB][G_::kChunks];
  float m[NB], lsum[NB];
  f32x16 o[G_::kDBlocks][NB];

  // sink_log2[nb] = S_h log2(e) of the column's head. The sink contributes exp2(S_h log2e - m) = 1
  // to the denominator; it is counted once per query (lane half 0).
  __device__ __forceinline__ void init(const float (&sink_log2)[NB], int grp) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      m[nb] = sink_log2[nb];
      lsum[nb] = (grp == 0 && sink_log2[nb] != kNegInf) ? 1.0f : 0.0f;
#pragma unroll
      for (int db = 0; db < G_::kDBlocks; ++db) o[db][nb] = zero_f32x16();
    }
  }

  // One tile of keys k0 .. k0 + kTileRows - 1: its K rows at `slot`, its V rows VT bytes from the
  // pair base (transposing reads at trb + pair_off + VT). `need_mask`: some column of the wave may
  // not see some key of the tile; row_of(nb) is then the position whose visible keys
  // (key_bounds(row, len, causal, window)) column block nb's lane holds.
  template <int VT, typename RowOf>
  __device__ __forceinline__ void tile(const unsigned char* slot, const int (&aoff)[4], const unsigned (&trb)[2][2],
                                       unsigned pair_off, int k0, bool need_mask, RowOf row_of, int len, int causal,
                                       int window, float scale_log2, int grp) {
    // S^T = K Q^T for the tile's 32-key row blocks.
    f32x16 s[MB][NB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) s[mb][nb] = zero_f32x16();
#pragma unroll
      for (int c = 0; c < G_::kChunks; ++c) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(slot + frag_off<D>(aoff, c, mb));
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) s[mb][nb] = mfma_32x32x16(ka, qf[nb][c], s[mb][nb]);
      }
    }
    if (need_mask) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const KeyBounds kb = key_bounds(row_of(nb), len, causal, window);
        const unsigned cnt = (unsigned)max(kb.hi - kb.lo, 0);  // visible keys kb.lo + 1 .. kb.hi
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int base = k0 + 32 * mb + 8 * grp - kb.lo - 1;  // key - (kb.lo + 1) for register 0
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            s[mb][nb][i] = in_span(base + 16 * (i >> 3) + (i & 7), cnt) ? s[mb][nb][i] : kNegInf;
          }
        }
      }
    }

    // Row maxima of the tile (raw scores; the scale is positive).
    float tmax[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float t = kNegInf;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) t = fmaxf(t, s[mb][nb][i]);
      }
      tmax[nb] = max_xor32(t) * scale_log2;
    }
    // A column moves its reference maximum only when the tile holds a score more than kLazyMax
    // above it (lazily: most tiles of long rows skip the rescale); below that the tile's values
    // exp2(s - m) stay under 2^kLazyMax. The branch is taken per 32-column block; inside it the
    // columns that do not need it keep their reference (alpha = 1).
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      if (wave_any(tmax[nb] > m[nb] + kLazyMax)) {
        const bool up = tmax[nb] > m[nb] + kLazyMax;
        const float mnew = up ? fmaxf(m[nb], tmax[nb]) : m[nb];
        const float alpha = (!up || mnew == kNegInf) ? 1.0f : fast_exp2(m[nb] - mnew);
        lsum[nb] *= alpha;
#pragma unroll
        for (int db = 0; db < G_::kDBlocks; ++db) o[db][nb] *= alpha;
        m[nb] = mnew;
      }
    }

    // V^T operands for O^T += V^T P^T (rows d = 32db + l32, k slots = keys 32mb + 16cc + 8grp + 0..7):
    // tr[4 (db MB + mb) + 2 cc + lo/hi], from panel db / 2 at rows 32mb + 16cc.
    u32x2 tr[NTR];
    static_for<G_::kDBlocks>([&](auto db_tag) {
      constexpr int db = decltype(db_tag)::value;
      constexpr int PO = VT + (db / 2) * G_::kPanelBytes;
      const unsigned t0 = trb[db % 2][0] + pair_off, t1 = trb[db % 2][1] + pair_off;
      static_for<MB>([&](auto mb_tag) {
        constexpr int mb = decltype(mb_tag)::value;
        tr[4 * (db * MB + mb) + 0] = ds_read_tr16_b64_asm<PO + 4096 * mb + 0>(t0);
        tr[4 * (db * MB + mb) + 1] = ds_read_tr16_b64_asm<PO + 4096 * mb + 0>(t1);
        tr[4 * (db * MB + mb) + 2] = ds_read_tr16_b64_asm<PO + 4096 * mb + 2048>(t0);
        tr[4 * (db * MB + mb) + 3] = ds_read_tr16_b64_asm<PO + 4096 * mb + 2048>(t1);
      });
    });

#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const float moff = m[nb] == kNegInf ? 0.0f : m[nb];  // nothing visible yet: exp2(-inf) = 0
      // A row's final probabilities are its values in this tile divided by at least its
      // denominator so far (later tiles only add to it), and those values are at most
      // 2^(tile max - running max). So when a row's largest value here does not reach
      // kFwdSplitThreshold of its denominator before this tile, no probability of the tile will
      // exceed that share for it. Otherwise the row also gets the product of the bf16 rounding
      // residuals of its P: O then carries about 16 significant bits of its largest
      // probabilities, which matters twice downstream, in O itself and in D = dO . O of the
      // backward, where an error in D scales every dS of the row (dQ of peaked rows crossed 1e-2
      // through it without this product, and at head_dim 128 with a large scale with it at a
      // threshold of a quarter). The test needs only values known before the softmax,
      // which keeps it off the common path's critical chain; on N(0,1) inputs it is mostly a row
      // block's first tile that takes the extra products, and rows that a large sink dominates
      // never do.
      const float pm = fast_exp2(tmax[nb] - moff);  // 0 for a fully masked row
      const bool need = pm > kFwdSplitThreshold * sum_xor32(lsum[nb]);
      const bool split = wave_any(need);
      float rs = 0.0f;
      bf16x8 pb[MB][2];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = fast_exp2(__builtin_fmaf(s[mb][nb][i], scale_log2, -moff));
          s[mb][nb][i] = p;
          rs += p;
        }
        pb[mb][0] = pack8(s[mb][nb], 0);
        pb[mb][1] = pack8(s[mb][nb], 1);
      }
      lsum[nb] += rs;
      // O^T += V^T P^T for this column block, contracting over the tile's keys.
      if (nb == 0) wait_lds_into(tr);
#pragma unroll
      for (int db = 0; db < G_::kDBlocks; ++db) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
          for (int cc = 0; cc < 2; ++cc) {
            const u32x2* t = tr + 4 * (db * MB + mb) + 2 * cc;
            o[db][nb] = mfma_32x32x16(join_tr(t[0], t[1]), pb[mb][cc], o[db][nb]);
          }
        }
      }
      if (split) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
          for (int cc = 0; cc < 2; ++cc) {
            bf16x8 pl = residual8(s[mb][nb], cc, pb[mb][cc]);
            if (!need) pl = zero_bf16x8();  // adds exactly 0 to the other columns
#pragma unroll
            for (int db = 0; db < G_::kDBlocks; ++db) {
              const u32x2* t = tr + 4 * (db * MB + mb) + 2 * cc;
              o[db][nb] = mfma_32x32x16(join_tr(t[0], t[1]), pl, o[db][nb]);
            }
          }
        }
      }
    }
  }

  // Stores column block nb (the lane's column) as O row `orow` (element offset) and its LSE at
  // `lse_at`: the two lane halves' partial denominators combined, O normalised.
  __device__ __forceinline__ void store(int nb, void* out, int out_bf16, size_t orow, float* lse_at, int grp) const {
    const float ltot = sum_xor32(lsum[nb]);
    const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
#pragma unroll
    for (int db = 0; db < G_::kDBlocks; ++db) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        f32x4 val = {o[db][nb][4 * r4] * inv, o[db][nb][4 * r4 + 1] * inv, o[db][nb][4 * r4 + 2] * inv,
                     o[db][nb][4 * r4 + 3] * inv};
        const size_t e = orow + 32 * db + 8 * r4 + 4 * grp;
        if (out_bf16) {  // round to nearest even, as a separate conversion of the fp32 result would
          typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
          *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(out) + e) = __builtin_convertvector(val, bf16x4);
        } else {
          *reinterpret_cast<f32x4*>(static_cast<float*>(out) + e) = val;
        }
      }
    }
    if (grp == 0) *lse_at = ltot > 0.0f ? (m[nb] + fast_log2(ltot)) * kLn2 : kNegInf;
  }
};

// HPW query heads of one KV group x RPW = 4 / HPW blocks of query rows per workgroup (four waves),
// so that groups of fewer than four heads still share each K/V tile among four waves.
template <int HPW, int D>
__global__ __launch_bounds__(256, 2) void attn_sink_fwd_kernel(FwdArgs a) {
  using G_ = Geo<D>;
  constexpr int kTileKeys = G_::kTileRows;
  constexpr int NB = D == 64 ? 2 : 1;                   // 32-query column blocks per wave
  constexpr int kRows = 32 * NB;                        // query rows per wave
  constexpr int RPW = 4 / HPW;                          // row blocks per workgroup
  constexpr int CPW = 2 * (kTileBytes / 1024) / 4;      // copies per wave and tile (K and V)
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kRing * kSlotBytes];

  const int n_hs = a.Hq / HPW;
  const int bid = blockIdx.x;
  const int inner = bid % n_hs;
  const int rest = bid / n_hs;
  // Consecutive block ids walk the KV groups first, so the round-robin placement of
  // workgroups on the 8 XCDs keeps each group's K/V in few L2s.
  const int spg = a.G / HPW;
  const int hs = (inner % a.Hkv) * spg + inner / a.Hkv;
  // Row blocks of one sequence back to back (its K/V tiles stay in L2 and the last-level cache),
  // the last (longest under a causal mask) first; sequence after sequence.
  const int b = rest / a.n_qblocks;
  const int qb = a.n_qblocks - 1 - rest % a.n_qblocks;  // longest causal rows first

  const int cs = a.cu[b];
  const int len = a.cu[b + 1] - cs;
  const int qw0 = qb * kRows * RPW;  // first row of the workgroup
  if (qw0 >= len) return;

  const int tid = threadIdx.x;
  const int wave = wave_id();
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int grp = lane >> 5;
  const int h = hs * HPW + wave % HPW;
  const int g = h / a.G;
  const int q0 = qw0 + kRows * (wave / HPW);  // this wave's first row
  const bool rows_live = RPW == 1 || q0 < len;  // waves past the sequence end only copy

  FwdCols<D, NB> cols;
  // Q^T as the B operand of S^T = K Q^T: lane holds query q0 + 32nb + l32, d = 16c + 8grp + (0..7).
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int qi = q0 + 32 * nb + l32;
#pragma unroll
    for (int c = 0; c < G_::kChunks; ++c) {
      // Rows past the end compute on the last row; their results are not stored.
      cols.qf[nb][c] = load_bf16x8(a.q + ((size_t)(cs + min(qi, len - 1)) * a.Hq + h) * D + 16 * c + 8 * grp);
    }
  }
  float sink_log2[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) sink_log2[nb] = a.sinks[h] * kLog2e;
  cols.init(sink_log2, grp);

  // Keys some row of a row range can see: up to the last row (causal), or up to W - 1 past it (a
  // non-causal window), and from W - 1 before the first row (any window). The workgroup streams
  // the tiles of its whole range; each wave computes only the tiles of its own.
  auto key_end = [&](int r1) {  // rows before r1
    return a.causal ? min(len, r1) : (a.window > 0 ? min(len, r1 - 1 + a.window) : len);
  };
  auto key_begin = [&](int r0) { return a.window > 0 ? max(0, r0 - a.window + 1) : 0; };
  const int kt_begin = key_begin(qw0) / kTileKeys;
  const int kt_end = (key_end(qw0 + kRows * RPW) + kTileKeys - 1) / kTileKeys;
  const int kw_begin = key_begin(q0);
  const int kw_end = rows_live ? key_end(q0 + kRows) : 0;

  const int kv_stride = a.Hkv * D;
  const __bf16* kbase = a.k + (size_t)cs * kv_stride + (size_t)g * D;
  const __bf16* vbase = a.v + (size_t)cs * kv_stride + (size_t)g * D;

  // K and V tiles of kTileKeys keys, swizzled (see tile_swz), in a 4-slot ring filled by direct
  // global->LDS copies issued one pair of tiles ahead; the waves split each tile's 16 copies (waves 0-1
  // the K tile, 2-3 the V tile). Full tiles go through a buffer resource; in the last, partial
  // tile keys past the sequence end repeat its last key (finite data; they are masked). V^T
  // operands come from transposing LDS loads of the V tile.
  static_assert(8 % CPW == 0, "a wave's copies stay within one tile");
  const unsigned row_bytes = 2u * kv_stride;
  unsigned coff[2];
  tile_copy_offsets(lane, row_bytes, coff);
  // Tiles are issued in order, so the next one's source advances by a tile per issue.
  const int u0 = wave * CPW;  // copies u0 .. u0 + CPW - 1 of 16: K for u < 8, V after
  const bool is_v = u0 >= 8;
  const size_t tile_elems = (size_t)kTileKeys * kv_stride;
  const __bf16* nx_src = (is_v ? vbase : kbase) + (size_t)kt_begin * tile_elems;
  int nx_kt = kt_begin;
  auto issue_next = [&]() {
    unsigned char* tile = ring + ((unsigned)(nx_kt - kt_begin) % kRing) * kSlotBytes + (is_v ? kTileBytes : 0);
    const int row0 = nx_kt * kTileKeys;
    if (row0 + kTileKeys <= len) {
      const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(nx_src, kTileKeys * row_bytes);
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
  const int mask_hi = min(len - kTileKeys - 1,
                          a.causal ? q0 - kTileKeys : (a.window > 0 ? q0 + a.window - kTileKeys : kBig));
  const int mask_lo = a.window > 0 ? q0 + kRows - a.window : -kBig;

  issue_next();
  if (kt_begin + 1 < kt_end) issue_next();

  unsigned trb[2][2];  // LDS addresses of the transposing reads at offset 0 of the ring
#pragma unroll
  for (int db = 0; db < 2; ++db) {
    trb[db][0] = ring_lds + toff[db][0];
    trb[db][1] = ring_lds + toff[db][1];
  }
  auto row_of = [&](int nb) { return q0 + 32 * nb + l32; };
  // The work on tile kt, held in the ring slot at byte offset pair_off + K (K a compile-time
  // constant: 0 for the first tile of a pair, one slot for the second).
  auto tile = [&](int kt, unsigned pair_off, auto k_tag) {
    constexpr int K = decltype(k_tag)::value;
    const int k0 = kt * kTileKeys;
    // Wave-uniform: skip a tile that holds none of this wave's keys.
    if (RPW > 1 && (k0 >= kw_end || k0 + kTileKeys <= kw_begin)) return;
    cols.template tile<K + kTileBytes>(ring + pair_off + K, aoff, trb, pair_off, k0, k0 > mask_hi || k0 < mask_lo,
                                       row_of, len, a.causal, a.window, a.scale_log2, grp);
  };

  // Tiles go in pairs, one wait and one barrier per pair; a pair sits in slots 0-1 or 2-3, so the
  // second tile's LDS addresses are the first's plus a constant.
  static_assert(kRing == 4, "two pairs of slots");
  for (int kt = kt_begin; kt < kt_end; kt += 2) {
    wait_vmcnt<0>();  // this wave's copies of tiles kt and kt + 1
    // Every wave's copies of tiles kt and kt + 1 have landed, and every wave is done with tiles
    // kt - 2 and kt - 1, whose slots receive tiles kt + 2 and kt + 3.
    __syncthreads();
    if (kt + 2 < kt_end) issue_next();
    if (kt + 3 < kt_end) issue_next();
    const unsigned pair_off = ((unsigned)(kt - kt_begin) & 2) * kSlotBytes;
    tile(kt, pair_off, std::integral_constant<int, 0>());
    if (kt + 1 < kt_end) tile(kt + 1, pair_off, std::integral_constant<int, kSlotBytes>());
  }

  // Epilogue: combine the two lane halves' partial denominators, normalise, store.
  if (a.out_bf16) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int qi = q0 + 32 * nb + l32;
      if (qi < len) {  // also false for every lane of a wave past the sequence end
        cols.store(nb, a.out, a.out_bf16, ((size_t)(cs + qi) * a.Hq + h) * D, a.lse + (size_t)h * a.T + cs + qi, grp);
      }
    }
    return;
  }
  // fp32 O goes through LDS: a lane holds 4-float pieces of one row, so direct stores would put
  // 32-byte pieces of 32 rows in each store instruction; from LDS each instruction writes whole
  // rows. Each wave stages its kRows x D tile in its quarter of the ring (free once every wave is
  // done with the last tile), 16-byte chunk k of row r at chunk k ^ (r % kCpr), which spreads the
  // writes of the 32 lanes of a register (32 rows, one chunk) over the banks.
  constexpr int kCpr = D / 4;         // 16-byte chunks per O row
  constexpr int kRpi = 64 / kCpr;     // rows per store instruction
  static_assert(kRows * D * 4 * 4 <= kRing * kSlotBytes, "four staged tiles fit in the ring");
  __syncthreads();
  float* stage = reinterpret_cast<float*>(ring) + wave * kRows * D;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int r = 32 * nb + l32;
    const float ltot = sum_xor32(cols.lsum[nb]);
    const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
#pragma unroll
    for (int db = 0; db < G_::kDBlocks; ++db) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int k = 8 * db + 2 * r4 + grp;  // d = 4k .. 4k + 3
        const f32x4 val = {cols.o[db][nb][4 * r4] * inv, cols.o[db][nb][4 * r4 + 1] * inv,
                           cols.o[db][nb][4 * r4 + 2] * inv, cols.o[db][nb][4 * r4 + 3] * inv};
        *reinterpret_cast<f32x4*>(stage + r * D + 4 * (k ^ (r % kCpr))) = val;
      }
    }
    const int qi = q0 + r;
    if (grp == 0 && qi < len) {
      a.lse[(size_t)h * a.T + cs + qi] = ltot > 0.0f ? (cols.m[nb] + fast_log2(ltot)) * kLn2 : kNegInf;
    }
  }
  const int k = lane % kCpr;
#pragma unroll
  for (int it = 0; it < kRows / kRpi; ++it) {
    const int r = kRpi * it + lane / kCpr;
    const f32x4 val = *reinterpret_cast<const f32x4*>(stage + r * D + 4 * (k ^ (r % kCpr)));
    const int qi = q0 + r;
    if (qi < len) *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + ((size_t)(cs + qi) * a.Hq + h) * D + 4 * k) = val;
  }
}

// Inference-shaped forward that visits the keys the way attn_sink_fwd_kernel does, so that its
// results equal the training forward's rows bit for bit (the pages trace their RL training
// mismatch to the inference engine's sink forward and the training kernel disagreeing:
// nmedialink.com "惊爆！GPT-OSS-20B强化学习…", section "纠正训练与推理不一致问题", Fig. 4). One
// wave per (sequence, KV head, group of 32 (new token, query head) columns, as in the split-KV
// decode); it streams every tile its columns can see, in ascending order, through the same 4-slot
// ring of 8 KiB tiles, and runs FwdCols::tile on each: new token j of a sequence with Lk keys and
// Nq new tokens is the training forward's row Lk - Nq + j, and a column's arithmetic does not
// depend on the other columns of its wave (see FwdCols). No split over the keys, so it is slower
// than attn_sink_decode_partial_kernel on long caches.
template <int D>
__global__ __launch_bounds__(64) void attn_sink_decode_ordered_kernel(DecodeArgs a) {
  using G_ = Geo<D>;
  constexpr int kTileKeys = G_::kTileRows;
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kRing * kSlotBytes];

  const int g = blockIdx.x % a.Hkv;
  const int rest = blockIdx.x / a.Hkv;  // = b * n_cg + cg
  const int cg = rest % a.n_cg;
  const int b = rest / a.n_cg;
  const int cq = a.cu_q[b];
  const int nq = a.cu_q[b + 1] - cq;
  const int ck = a.cu_k[b];
  const int lk = a.cu_k[b + 1] - ck;
  if (nq <= 0 || 32 * cg >= nq * a.G) return;  // uniform: no real column in this group

  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31;
  const int grp = lane >> 5;
  const int col = 32 * cg + l32;
  const int j = col / a.G;                // column = (new query j, query head g*G + col % G)
  const int hq = g * a.G + col % a.G;
  const bool col_ok = j < nq;             // columns past the last pair repeat the last query
  const int pos = lk - nq + min(j, nq - 1);
  const int pos_lo = lk - nq + (32 * cg) / a.G;  // the wave's first and last query positions
  const int pos_hi = lk - nq + min((32 * cg + 31) / a.G, nq - 1);

  FwdCols<D, 1> cols;
#pragma unroll
  for (int c = 0; c < G_::kChunks; ++c) {
    cols.qf[0][c] = load_bf16x8(a.q + ((size_t)(cq + min(j, nq - 1)) * a.Hq + hq) * D + 16 * c + 8 * grp);
  }
  const float sink_log2[1] = {a.sinks[hq] * kLog2e};
  cols.init(sink_log2, grp);

  // Tiles some column sees, 64-aligned (D = 64) or 32-aligned (D = 128) from the sequence start as
  // in the training forward; earlier tiles that the training forward's wave also visits hold no
  // key the row sees and change nothing.
  const int kt_lo = (a.window > 0 ? max(0, pos_lo - a.window + 1) : 0) / kTileKeys;
  const int kt_hi = (pos_hi + kTileKeys) / kTileKeys;  // through the tile of key pos_hi
  const int kv_stride = a.Hkv * D;
  const __bf16* kbase = a.k + (size_t)ck * kv_stride + (size_t)g * D;
  const __bf16* vbase = a.v + (size_t)ck * kv_stride + (size_t)g * D;
  const unsigned row_bytes = 2u * kv_stride;
  unsigned coff[2];
  tile_copy_offsets(lane, row_bytes, coff);
  int nx_kt = kt_lo;
  auto issue_next = [&]() {  // all 16 copies of the next tile (this wave is alone in its workgroup)
    unsigned char* tile = ring + ((unsigned)(nx_kt - kt_lo) % kRing) * kSlotBytes;
    const int row0 = nx_kt * kTileKeys;
    if (row0 + kTileKeys <= lk) {
      const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(kbase + (size_t)row0 * kv_stride, kTileKeys * row_bytes);
      const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(vbase + (size_t)row0 * kv_stride, kTileKeys * row_bytes);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        tile_copy_full_d<D>(rk, coff, row_bytes, tile, u);
        tile_copy_full_d<D>(rv, coff, row_bytes, tile + kTileBytes, u);
      }
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        tile_copy_d<D>(kbase, row0, lk - 1, kv_stride, tile, u, lane);
        tile_copy_d<D>(vbase, row0, lk - 1, kv_stride, tile + kTileBytes, u, lane);
      }
    }
    ++nx_kt;
  };
  int aoff[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) aoff[c] = tile_frag_off(l32, grp, c);
  int toff[2][2];
  tile_tr_offsets(lane, toff);
  const unsigned ring_lds = lds_addr(ring);
  unsigned trb[2][2];
#pragma unroll
  for (int db = 0; db < 2; ++db) {
    trb[db][0] = ring_lds + toff[db][0];
    trb[db][1] = ring_lds + toff[db][1];
  }
  // A tile needs the mask when the cache end, the earliest column's diagonal or the latest
  // column's window edge reaches into it.
  constexpr int kBig = 1 << 29;
  const int mask_hi = min(lk - kTileKeys - 1, pos_lo - kTileKeys);
  const int mask_lo = a.window > 0 ? pos_hi + 1 - a.window : -kBig;
  auto row_of = [&](int) { return pos; };
  auto tile = [&](int kt, unsigned pair_off, auto k_tag) {
    constexpr int K = decltype(k_tag)::value;
    const int k0 = kt * kTileKeys;
    cols.template tile<K + kTileBytes>(ring + pair_off + K, aoff, trb, pair_off, k0, k0 > mask_hi || k0 < mask_lo,
                                       row_of, lk, 1, a.window, a.scale_log2, grp);
  };

  issue_next();
  if (kt_lo + 1 < kt_hi) issue_next();
  for (int kt = kt_lo; kt < kt_hi; kt += 2) {
    wait_vmcnt<0>();  // the copies of tiles kt and kt + 1
    __syncthreads();  // (one wave: orders its LDS reads of tiles kt - 2, kt - 1 before the next copies)
    if (kt + 2 < kt_hi) issue_next();
    if (kt + 3 < kt_hi) issue_next();
    const unsigned pair_off = ((unsigned)(kt - kt_lo) & 2) * kSlotBytes;
    tile(kt, pair_off, std::integral_constant<int, 0>());
    if (kt + 1 < kt_hi) tile(kt + 1, pair_off, std::integral_constant<int, kSlotBytes>());
  }
  if (col_ok) {
    cols.store(0, a.out, a.out_bf16, ((size_t)(cq + j) * a.Hq + hq) * D, a.lse + (size_t)hq * a.Tq + cq + j, grp);
  }
}

}  // namespace

template <int D>
void launch_fwd_d(const FwdArgs& a, dim3 grid, hipStream_t stream) {
  const dim3 block(256);
  switch (a.hpw) {
    case 4: hipLaunchKernelGGL((attn_sink_fwd_kernel<4, D>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((attn_sink_fwd_kernel<2, D>), grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL((attn_sink_fwd_kernel<1, D>), grid, block, 0, stream, a); break;
  }
}

hipError_t launch_decode_ordered(const DecodeArgs& a, hipStream_t stream) {
  const long long nblocks = (long long)a.B * a.Hkv * a.n_cg;
  if (nblocks <= 0) return hipSuccess;
  if (a.D == 128) {
    hipLaunchKernelGGL(attn_sink_decode_ordered_kernel<128>, dim3((unsigned)nblocks), dim3(64), 0, stream, a);
  } else {
    hipLaunchKernelGGL(attn_sink_decode_ordered_kernel<64>, dim3((unsigned)nblocks), dim3(64), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  const long long nblocks = (long long)a.n_qblocks * (a.Hq / a.hpw) * a.B;
  if (nblocks <= 0) return hipSuccess;
  if (a.D == 128) {
    launch_fwd_d<128>(a, dim3((unsigned)nblocks), stream);
  } else {
    launch_fwd_d<64>(a, dim3((unsigned)nblocks), stream);
  }
  return hipGetLastError();
}

}  // namespace attn_sink
