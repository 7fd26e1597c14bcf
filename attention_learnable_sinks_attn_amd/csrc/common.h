// Device-side building blocks shared by the sink-attention kernels (gfx950 / CDNA4 only).
//
// Matrix products use v_mfma_f32_32x32x16_bf16 (bf16 inputs, fp32 accumulation). Operand layout
// of one 64-lane wave for C[32x32] += A[32x16] * B[16x32]:
//   A: lane l holds row (l % 32), eight consecutive k slots 8*(l/32) .. 8*(l/32)+7
//   B: lane l holds column (l % 32), the same eight k slots
//   C: lane l holds column (l % 32), rows 8*(i/4) + 4*(l/32) + (i%4) for i = 0..15
// Only the pairing of k slots between A and B matters to the product, so a kernel may put any
// logical index in a slot as long as A and B agree.
//
// Row permutation used throughout: when a 32-row A block is loaded with row r holding element
// swap23(r) (bits 2 and 3 of r exchanged), lane group g = l/32 of the C result holds, in its
// registers 8c..8c+7, the eight CONSECUTIVE elements 16c + 8g + (0..7). That makes the C block
// directly usable as the B operand of a second product that contracts over those rows, and lets
// the matching A operand be read from LDS as one 16-byte vector.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace attn_sink {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ f32x16 mfma_32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int swap23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// Index (within a 32-row C block) of register i held by lane group g, after the swap23 load.
__device__ __forceinline__ int c_row(int i, int g) { return 16 * (i >> 3) + 8 * g + (i & 7); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Registers 8c..8c+7 of a C block, rounded to bf16 (round to nearest even).
__device__ __forceinline__ bf16x8 pack8(const f32x16& c, int chunk) {
  f32x8 v;
  if (chunk == 0) {
    v = (f32x8){c[0], c[1], c[2], c[3], c[4], c[5], c[6], c[7]};
  } else {
    v = (f32x8){c[8], c[9], c[10], c[11], c[12], c[13], c[14], c[15]};
  }
  return __builtin_convertvector(v, bf16x8);
}

// Rounding residual of pack8: bf16(c - hi), so that hi + lo carries about 16 significant bits.
__device__ __forceinline__ bf16x8 residual8(const f32x16& c, int chunk, const bf16x8& hi) {
  f32x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = c[8 * chunk + e] - (float)hi[e];
  return __builtin_convertvector(r, bf16x8);
}

// Probabilities above this value make the bf16 rounding of P and dS visible in the sums over
// query rows and heads (dV) and over keys (dQ); blocks that hold one get the residual product.
constexpr float kSplitThreshold = 0.0625f;
// dK sums dS Q over rows and heads, and on sharp rows (large |Q|) the rounding of dS shows from
// smaller probabilities on: its residual product starts at this one.
constexpr float kSplitThresholdDk = 0.03125f;

// Wave index within the workgroup, as a value the compiler knows to be wave-uniform (SGPR), so
// that branches and addresses derived from it stay scalar.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ bool wave_any(bool pred) { return __builtin_amdgcn_ballot_w64(pred) != 0; }

__device__ __forceinline__ bf16x8 load_bf16x8(const __bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  bf16x8 z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = (__bf16)0.0f;
  return z;
}

__device__ __forceinline__ f32x16 zero_f32x16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.0f;
  return z;
}

// Reductions over the lane pair (l, l ^ 32) with one v_permlane32_swap: the swap leaves the
// low-half values in both halves of one register and the high-half values in the other.
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Keys visible from query i of a sequence of `len` tokens (the sink is always visible): the
// interval lo < j <= hi. Causal attention sees j <= i and, with a window W, j > i - W;
// non-causal attention with a window sees the band i - W < j < i + W. A mask then tests each
// key with two comparisons.
struct KeyBounds {
  int lo, hi;
};
__device__ __forceinline__ KeyBounds key_bounds(int i, int len, int causal, int window) {
  int hi = len - 1;
  if (causal) {
    hi = min(hi, i);
  } else if (window > 0) {
    hi = min(hi, i + window - 1);
  }
  return {window > 0 ? i - window : -(1 << 30), hi};
}

// Membership of x in the interval first .. first + count - 1 as one unsigned comparison:
// in_span(x - first, count) (a negative offset wraps to a large unsigned value).
__device__ __forceinline__ bool in_span(int offset, unsigned count) { return (unsigned)offset < count; }

// Direct global -> LDS copies (gfx950): lane l's 16 (or 4) bytes at `src` land at LDS byte
// offset lds_dst + 16 * l (or 4 * l). `lds_dst` must be wave-uniform. The copy completes
// asynchronously; it is counted by vmcnt like any other vector memory load.
typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ void dma16(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_dst, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_dst, 4, 0, 0);
}

// The same copies addressed through a buffer resource: the 64-bit base sits in scalar registers,
// so a copy needs only a per-lane 32-bit offset `voff` and a wave-uniform offset `soff`, with no
// 64-bit address arithmetic in vector registers. Reads at or past `bytes` from the base return
// zero; the callers only use resources whose every read lies inside the tensor.
constexpr int kRawBufferWord3 = 0x00020000;  // raw (unswizzled) buffer, 32-bit data format
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRawBufferWord3);
}
__device__ __forceinline__ void bdma16(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff, void* lds_dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_dst, 16, (int)voff, (int)soff, 0, 0);
}
__device__ __forceinline__ void bdma4(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff, void* lds_dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_dst, 4, (int)voff, (int)soff, 0, 0);
}

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt left unconstrained).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Operand fragments of TRANSPOSED tiles come from ds_read_b64_tr_b16, which works on 16-lane
// groups: when the group's lanes address a 4-row x 16-column block of a row-major bf16 array X in
// LDS (lane s at row s/4, columns 4*(s%4)..+3), lane t of the group receives column t of the
// block, rows 0..3. Two such reads, 4 rows apart, give lane l the eight elements
// X[k0 + 8*(l/32) + e][m0 + l%32], e = 0..7: the MFMA operand whose row (or column) index runs
// along X's columns and whose k slots run along X's rows.
//
// The read is issued through inline asm: the compiler makes every transposing LDS read it knows
// about wait for all outstanding direct global->LDS copies (vmcnt(0)), which would serialise a
// kernel that keeps copies in flight into other LDS slots. The result is not tracked either:
// wait_lds_into must follow before any use.
template <int OFF>
__device__ __forceinline__ u32x2 ds_read_tr16_b64_asm(unsigned addr) {
  static_assert(OFF >= 0 && OFF < 65536, "16-bit DS offset");
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
// lgkmcnt(0), tied to the registers of 16 untracked LDS reads so that no use moves above it.
__device__ __forceinline__ void wait_lds_into(u32x2 (&t)[16]) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(t[0]), "+v"(t[1]), "+v"(t[2]), "+v"(t[3]), "+v"(t[4]), "+v"(t[5]), "+v"(t[6]), "+v"(t[7]),
                 "+v"(t[8]), "+v"(t[9]), "+v"(t[10]), "+v"(t[11]), "+v"(t[12]), "+v"(t[13]), "+v"(t[14]),
                 "+v"(t[15]));
}
__device__ __forceinline__ bf16x8 join_tr(const u32x2& lo, const u32x2& hi) {
  return __builtin_bit_cast(bf16x8, (u32x4){lo[0], lo[1], hi[0], hi[1]});
}

// The 16 fp32 values of rows 16(i/8) + 8g + i%8, i = 0..15 (the rows a C register block of lane
// group g holds after a swap23 load), from a row vector in LDS.
__device__ __forceinline__ f32x16 load_rows16(const float* p, int g) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p + 8 * g);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 8 * g + 4);
  const f32x4 c = *reinterpret_cast<const f32x4*>(p + 16 + 8 * g);
  const f32x4 d = *reinterpret_cast<const f32x4*>(p + 20 + 8 * g);
  return (f32x16){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3], c[0], c[1], c[2], c[3], d[0], d[1], d[2], d[3]};
}

// ---- Swizzled tiles of 64-element bf16 rows in LDS ----
// Rows of 64 bf16 (128 bytes) are stored back to back without padding; logical 16-byte chunk k of
// tile row r lives in chunk k ^ tile_swz(r). Over any 16 consecutive rows, rows of equal parity
// get distinct values, so the 16-byte A-operand fragment reads of a 32-row block (rows permuted by
// swap23, 16 lanes per LDS cycle) hit distinct banks; and rows r and r + 2 (r % 4 == 0) differ in
// bit 2, so the transposing 8-byte reads of 4 consecutive rows x 32 columns (32 lanes per cycle)
// do too. tile_swz(r + 16) == tile_swz(r), so 32-row blocks of a tile share one offset table.
__device__ __forceinline__ int tile_swz(int r) {
  const int x = (r >> 1) & 7;
  return ((x & 1) << 2) | (x >> 1);
}

// Byte offset, within a swizzled 32-row block, of the A-operand fragment of lane (l32, grp) for
// k slots 16c + 8grp .. +7: row swap23(l32).
__device__ __forceinline__ int tile_frag_off(int l32, int grp, int c) {
  const int r = swap23(l32);
  return r * 128 + (((2 * c + grp) ^ tile_swz(r)) << 4);
}

// Per-lane byte offsets of the transposing reads (see ds_read_tr16_b64_asm) of a swizzled tile:
// off[mb][h] addresses rows 8grp + (l%16)/4 + 4h, logical columns 32mb + 16((l>>4)&1) + 4(l%4).
// Rows k0 + ... (k0 a multiple of 16) add 128 * k0, which fits the instruction's offset field.
__device__ __forceinline__ void tile_tr_offsets(int lane, int (&off)[2][2]) {
  const int s16 = lane & 15;
  const int grp = lane >> 5;
  const int ch = 2 * ((lane >> 4) & 1) + ((s16 & 3) >> 1);
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = 8 * grp + (s16 >> 2) + 4 * h;
      off[mb][h] = r * 128 + (((4 * mb + ch) ^ tile_swz(r)) << 4) + 8 * (s16 & 1);
    }
  }
}

// Per-lane offsets for copies of a full tile through a buffer resource based at the tile's first
// row, rows `row_bytes` apart (tile_copy_full_d): off[h] is lane l's row l/8 and its swizzled
// chunk for the copies whose first row is 8h mod 16 (the swizzle of row 8u + l/8 depends on u only
// through u % 2); the uniform 8u rows are added per copy.
__device__ __forceinline__ void tile_copy_offsets(int lane, unsigned row_bytes, unsigned (&off)[2]) {
  const int r = lane >> 3;
  off[0] = r * row_bytes + 16 * ((lane & 7) ^ tile_swz(r));
  off[1] = r * row_bytes + 16 * ((lane & 7) ^ tile_swz(r + 8));
}

// f(std::integral_constant<int, i>()) for i = 0 .. N - 1, so that i can be a template argument
// (for instance an LDS offset folded into an instruction).
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>());
    static_for<N, I + 1>(std::forward<F>(f));
  }
}

// ---- Head dimensions 64 and 128 ----
// A row of D bf16 elements is stored in LDS as D / 64 "panels" of 64 elements, each panel laid out
// exactly like the 64-element tiles above (swizzled 128-byte rows), so every fragment and
// transposing read of a panel uses the same offsets. A K, V, Q or dO tile is always 8 KiB: 64 rows
// at D = 64, 32 rows at D = 128; its panels follow each other (panel p at p * kPanelBytes).
template <int D>
struct Geo {
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  static constexpr int kPanels = D / 64;             // 64-element panels per row
  static constexpr int kChunks = D / 16;             // 16-wide k slices of a contraction over d
  static constexpr int kDBlocks = D / 32;            // 32-row MFMA blocks over d (outputs)
  static constexpr int kTileRows = 4096 / D;         // rows of an 8 KiB tile
  static constexpr int kRowBlocks = kTileRows / 32;  // 32-row MFMA blocks of a tile
  static constexpr int kPanelBytes = kTileRows * 128;
  static constexpr int kTileBytes = 8192;
  static constexpr int kCopies = kTileBytes / 1024;  // 1 KiB copies per tile
  static constexpr int kCopiesPerPanel = kTileRows / 8;
};

// Byte offset, within an 8 KiB tile, of the A-operand fragment of contraction chunk c (d = 16c +
// 8grp + 0..7) for the 32-row block `rb` (rows swap23-permuted): panel c / 4, slice c % 4.
template <int D>
__device__ __forceinline__ int frag_off(const int (&aoff)[4], int c, int rb) {
  return (c / 4) * Geo<D>::kPanelBytes + 4096 * rb + aoff[c % 4];
}

// Copy u (0 .. kCopies - 1) of an 8 KiB swizzled tile of D-element rows: lane l fetches panel
// u / kCopiesPerPanel of tile row r = 8 (u % kCopiesPerPanel) + l / 8 (global row min(row0 + r,
// last), `stride` elements apart), logical 16-byte chunk (l % 8) ^ tile_swz(r), into LDS
// tile + 1024 u + 16 l, i.e. physical chunk l % 8 of that row.
template <int D>
__device__ __forceinline__ void tile_copy_d(const __bf16* base, int row0, int last, int stride, unsigned char* tile,
                                            int u, int lane) {
  const int p = u / Geo<D>::kCopiesPerPanel;
  const int r = 8 * (u % Geo<D>::kCopiesPerPanel) + (lane >> 3);
  dma16(base + (size_t)min(row0 + r, last) * stride + 64 * p + 8 * ((lane & 7) ^ tile_swz(r)), tile + 1024 * u);
}
// The same copy of a full tile (every row inside the sequence) through a buffer resource based at
// the tile's first row (offsets from tile_copy_offsets).
template <int D>
__device__ __forceinline__ void tile_copy_full_d(__amdgpu_buffer_rsrc_t rsrc, const unsigned (&off)[2],
                                                 unsigned row_bytes, unsigned char* tile, int u) {
  const int p = u / Geo<D>::kCopiesPerPanel;
  const int rb = u % Geo<D>::kCopiesPerPanel;
  bdma16(rsrc, off[rb & 1] + 128u * p, 8u * rb * row_bytes, tile + 1024 * u);
}

// lgkmcnt(0) for 32 untracked LDS reads (asm takes at most 30 operands: the second statement
// only orders the other 16 results after the wait).
__device__ __forceinline__ void wait_lds_into(u32x2 (&t)[32]) {
  u32x2(&a)[16] = *reinterpret_cast<u32x2(*)[16]>(&t[0]);
  u32x2(&b)[16] = *reinterpret_cast<u32x2(*)[16]>(&t[16]);
  wait_lds_into(a);
  asm volatile(""
               : "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]), "+v"(b[4]), "+v"(b[5]), "+v"(b[6]), "+v"(b[7]),
                 "+v"(b[8]), "+v"(b[9]), "+v"(b[10]), "+v"(b[11]), "+v"(b[12]), "+v"(b[13]), "+v"(b[14]),
                 "+v"(b[15]));
}

// Work descriptors (filled on the host).
struct FwdArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const float* sinks;
  const int32_t* cu;
  void* out;             // [T, Hq, D], fp32 or bf16 (out_bf16)
  float* lse;
  int out_bf16;
  int T, B, Hq, Hkv, G;  // G = Hq / Hkv
  int hpw;               // query heads per workgroup (= waves per workgroup), divides G
  int n_qblocks;         // ceil(max_seqlen / rows per workgroup)
  int causal, window;
  float scale_log2;      // softmax scale * log2(e)
  int D;                 // head_dim: 64 or 128
};

struct BwdArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const float* sinks;
  const float* out;
  const float* lse;
  const __bf16* dout;
  const int32_t* cu;
  float* dq;
  float* dk;
  float* dv;
  float* dsinks;
  float* nlse;       // workspace: -LSE_i / scale (score units), [Hq, T]
  float* negd;       // workspace: -D_i = -rowsum(dO * O), [Hq, T]
  float* dsink_part; // per (head, row-block slot) partial sums of P_sink * D~, [Hq, n_slots]
  float* dkv_part;   // dK / dV partial sums per head half: [2][n_halves][T][Hkv][D] (unscaled; unused with one half)
  int n_slots;
  int n_halves;      // query-head halves of a KV group processed by separate dK/dV workgroups
  int T, B, Hq, Hkv, G;
  int hpw;            // dQ kernel: query heads per workgroup
  int kv_streams;     // dK/dV kernel: head streams per workgroup (1 or 2; waves = 2 x streams)
  int n_qblocks;      // dQ kernel grid rows
  int n_kblocks;      // dK/dV kernel grid rows
  int causal, window;
  float scale;        // softmax scale
  float scale_log2;   // softmax scale * log2(e)
  int D;              // head_dim: 64 or 128
};

struct DecodeArgs {
  const __bf16* q;     // [Tq, Hq, D]: the new queries, packed by cu_q
  const __bf16* k;     // [Tk, Hkv, D]: the caches, packed by cu_k
  const __bf16* v;
  const float* sinks;
  const int32_t* cu_q;
  const int32_t* cu_k;
  void* out;           // [Tq, Hq, D], fp32 or bf16 (out_bf16)
  float* lse;          // [Hq, Tq]
  float* part_o;       // per (sequence, KV head, column group, chunk): [32 columns][D] unnormalised outputs
  float* part_ml;      // per (sequence, KV head, column group, chunk): [2][32] running max (log2), denominator
  int Tq, B, Hq, Hkv, G;
  int n_cols;          // max_q * G: the columns any (sequence, KV head) uses
  int n_cg;            // ceil(n_cols / 32): groups of 32 columns, one wave each per chunk
  int n_chunks;        // key chunks per sequence
  int chunk_keys;      // keys per chunk (multiple of 64)
  int window;
  int out_bf16;
  float scale_log2;
  int D;               // head_dim: 64 or 128
};

}  // namespace attn_sink
