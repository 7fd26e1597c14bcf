/*
 * attn_sink.h - C ABI of the MI355X (gfx950) sink-attention library (libattn_sink.so).
 *
 * Operation. Scaled dot-product attention in which every query head h owns one learnable
 * logit S_h (the "sink"). The sink joins each row's softmax denominator but has no value row,
 * so it takes probability mass without adding to the output:
 *     S_ij  = scale * q_i . k_j
 *     P_ij  = exp(S_ij) / (sum_{j' visible} exp(S_ij') + exp(S_h))
 *     O_i   = sum_{j visible} P_ij v_j
 * Defined on the nmedialink.com page "惊爆！GPT-OSS-20B强化学习，训练速度狂飙、超稳定！",
 * section "GPT-OSS中的带注意力槽的注意力机制" (concat the sink column, softmax, drop it,
 * multiply by V) and section "数学公式深入解读" (eq. P_ij and the sink probability P_{i,h}).
 * The backward returns dQ, dK, dV and dL/dS_h = -sum_i P_{i,h} D_i with
 * D_i = sum_j P_ij dO_i.v_j = dO_i.O_i (same page, section "反向传播的实现", simplified
 * equation).
 *
 * Conventions shared by every entry point
 *  - Packed varlen layout: B sequences are stored back to back; rows cu_seqlens[b] ..
 *    cu_seqlens[b+1]-1 belong to sequence b. Attention never crosses a sequence boundary
 *    (same page, section "结合Flash Attention V3的序列并行技术": padding removed, tokens
 *    packed into one list). A fixed-shape batch is B = 1, cu_seqlens = {0, N}.
 *  - Tensors (device pointers, contiguous, row-major, base 16-byte aligned); D = head_dim, 64 or
 *    128 (the pages' GPT-OSS layers use 64; 128 is the other common head size):
 *      q, dout   [T, Hq, D]   bfloat16
 *      k, v      [T, Hkv, D]  bfloat16
 *      sinks     [Hq]         float32 (one logit per query head, natural-log units, NOT scaled)
 *      out       [T, Hq, D]   float32 (attn_sink_fwd may store bf16 instead: out_dtype)
 *      lse       [Hq, T]      float32, natural log of the full denominator (sink included)
 *      dq        [T, Hq, D]   float32;  dk, dv [T, Hkv, D] float32;  dsinks [Hq] float32
 *      cu_seqlens [B+1] int32 on the device, cu[0] = 0, non-decreasing, cu[B] = T
 *  - GQA: query head h reads KV head h / (Hq / Hkv); Hq must be a multiple of Hkv.
 *  - Masks: causal != 0 lets query i see keys j <= i of its own sequence. window = W > 0 with
 *    causal further restricts to j > i - W, i.e. exactly the last W keys including itself; with
 *    causal = 0 it is the symmetric band i - W < j < i + W (the pages only use causal windows;
 *    the band is the plain non-causal reading). window <= 0 means no window. The sink is visible
 *    from every row, is never masked and does not count toward W. The sink is added after
 *    scaling: it is never multiplied by scale.
 *  - Outputs are overwritten, never accumulated into. The caller owns every buffer; the library
 *    allocates nothing, keeps no state between calls (apart from attn_sink_bwd_noalloc's static
 *    scratch array, described there), and only enqueues work on `stream` (NULL = the default
 *    stream). Calls return before the GPU work finishes; errors raised by the device
 *    surface at the caller's next synchronisation.
 *  - Errors: 0 on success, a negative ATTN_SINK_ERR_* code otherwise. All argument checks run on
 *    the host before anything is enqueued; a failing call enqueues nothing. The contents of
 *    cu_seqlens are trusted (they live on the device).
 */
#ifndef ATTN_SINK_H_
#define ATTN_SINK_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as HIP's hipStream_t; repeated here so that C callers need no HIP headers. */
typedef struct ihipStream_t* hipStream_t;

enum {
  ATTN_SINK_OK = 0,
  ATTN_SINK_ERR_NULL_PTR = -1,    /* a required pointer (or the shape struct) is NULL */
  ATTN_SINK_ERR_BAD_SHAPE = -2,   /* T < 0, B < 1, Hq < 1, Hkv < 1, Hq % Hkv != 0, max_seqlen < 0
                                     or max_seqlen > T, max_seqlen * Hq * D >= 2^31 (offsets
                                     inside one sequence are 32-bit), T * Hq > 2^34, or
                                     ceil(max_seqlen / 64) * Hq * B >= 2^31 (grid size) */
  ATTN_SINK_ERR_UNSUPPORTED = -3, /* head_dim not 64 or 128, or out_dtype not ATTN_SINK_F32 (attn_sink_bwd)
                                     or not ATTN_SINK_F32 / ATTN_SINK_BF16 (attn_sink_fwd) */
  ATTN_SINK_ERR_BAD_WINDOW = -4,  /* window < 0 (attn_sink_decode_fwd only) */
  ATTN_SINK_ERR_WORKSPACE = -5,   /* workspace NULL, not 16-byte aligned, or smaller than
                                     attn_sink_bwd_workspace_bytes() (attn_sink_decode_workspace_bytes()) */
  ATTN_SINK_ERR_HIP = -6,         /* a HIP launch failed (hipGetLastError after the launch) */
  ATTN_SINK_ERR_ALIGN = -7,       /* a tensor base pointer is not 16-byte aligned */
  ATTN_SINK_ERR_BAD_SEQLENS = -8, /* attn_sink_check_cu_seqlens: offsets inconsistent with the shape */
  ATTN_SINK_ERR_SCRATCH = -9      /* attn_sink_bwd_noalloc: workspace needed > its static scratch */
};

enum { ATTN_SINK_F32 = 0, ATTN_SINK_BF16 = 1 };

/* Problem description, passed by pointer; read on the host only, never retained. */
typedef struct attn_sink_shape {
  int32_t total_tokens;  /* T = cu_seqlens[B] */
  int32_t num_seqs;      /* B >= 1 */
  int32_t max_seqlen;    /* >= every cu[b+1]-cu[b]; sizes the grid (a larger value only adds idle blocks) */
  int32_t num_heads_q;   /* Hq */
  int32_t num_heads_kv;  /* Hkv, divides Hq */
  int32_t head_dim;      /* D: 64 or 128 */
  float softmax_scale;   /* <= 0 selects 1/sqrt(head_dim) */
  int32_t out_dtype;     /* ATTN_SINK_F32; attn_sink_fwd also takes ATTN_SINK_BF16 (out rounded to
                            bf16, nearest even, e.g. for inference prefill). attn_sink_bwd needs the
                            fp32 forward output: out, dq, dk, dv are float32 there */
} attn_sink_shape;

/*
 * Forward: writes out [T, Hq, D] (float32) and lse [Hq, T] (float32, natural log, sink included:
 * lse_i = log(sum_j exp(S_ij) + exp(S_h))). Rows of zero-length sequences are not touched (there
 * are none). Inputs are read only.
 */
int attn_sink_fwd(const void* q, const void* k, const void* v, const float* sinks, int causal, int window,
                  const int32_t* cu_seqlens, const attn_sink_shape* shape, void* out, float* lse,
                  hipStream_t stream);

/*
 * Bytes of device workspace attn_sink_bwd needs for this shape: -LSE_i/scale and -D_i for every
 * (head, row), one dSink partial sum per (head, 32-row block), and, when the dK/dV pass splits a
 * KV group's query heads over two workgroups (even Hq/Hkv and fewer than 2048 key blocks of 64
 * over all sequences and KV heads, counted as num_seqs * ceil(max_seqlen / 64) * Hkv), fp32
 * dK/dV partial sums for each half (2 * 2 * T * Hkv * D floats); each region 256-byte aligned.
 * Returns 0 if `shape` is NULL or invalid.
 */
size_t attn_sink_bwd_workspace_bytes(const attn_sink_shape* shape);

/*
 * Backward of L with upstream gradient dout = dL/dO, given the forward's out and lse:
 *   dq [T, Hq, D], dk / dv [T, Hkv, D] (float32, summed over the query heads of each KV group),
 *   dsinks [Hq] (float32, dL/dS_h summed over every row of every sequence).
 * workspace: caller-owned device memory of at least attn_sink_bwd_workspace_bytes(shape) bytes;
 * its contents on entry do not matter and are clobbered. The result is deterministic: no atomics
 * decide any output, so repeated calls on the same inputs give bitwise identical results.
 */
int attn_sink_bwd(const void* q, const void* k, const void* v, const float* sinks, const void* out,
                  const float* lse, const void* dout, int causal, int window, const int32_t* cu_seqlens,
                  const attn_sink_shape* shape, void* workspace, size_t workspace_bytes, float* dq, float* dk,
                  float* dv, float* dsinks, hipStream_t stream);

/*
 * attn_sink_bwd for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): same arguments, semantics and kernels,
 * minus the workspace, which comes from a static device array of ATTN_SINK_NOALLOC_SCRATCH_BYTES
 * (64 MiB) that the library holds on each GPU it runs on until the process ends. The caller still
 * passes every input and output. No hipMalloc, hipFree or other allocating call is made; the
 * first call on a device looks the array's address up once (hipGetSymbolAddress, with that device
 * made current for the lookup). Shapes whose attn_sink_bwd_workspace_bytes exceeds the array
 * return ATTN_SINK_ERR_SCRATCH before anything is enqueued (e.g. 4k tokens x 64/8 heads needs
 * about 34 MiB, 32k tokens about 16 MiB). Every call on one GPU shares that GPU's array and the
 * array keeps the last call's contents (the backward writes every workspace value before reading
 * it, so nothing needs clearing): calls that overlap on one GPU, on different streams or from
 * different threads, race and give wrong results; serialise them.
 */
#define ATTN_SINK_NOALLOC_SCRATCH_BYTES (64u << 20)
int attn_sink_bwd_noalloc(const void* q, const void* k, const void* v, const float* sinks, const void* out,
                          const float* lse, const void* dout, int causal, int window, const int32_t* cu_seqlens,
                          const attn_sink_shape* shape, float* dq, float* dk, float* dv, float* dsinks,
                          hipStream_t stream);

/*
 * Same as attn_sink_bwd, and additionally records events[0..num_events-1] on `stream` around the
 * backward's kernels (events[i] before kernel i, events[num_kernels] after the last), for
 * per-kernel timing. `events` holds hipEvent_t handles created by the caller; num_events must be
 * attn_sink_bwd_num_kernels() + 1. An entry may be NULL: nothing is recorded at that point (each
 * record costs a few microseconds of GPU time, so a caller timing one kernel passes only the two
 * events around it). Passing events == NULL behaves like attn_sink_bwd. A kernel the call does not
 * need is not launched and its two events are recorded back to back: the third kernel
 * (attn_sink_bwd_finish_kernel: the sum of the dK/dV head halves, if any, then the dSink
 * reduction) is left out when the dK/dV pass has no head halves and at most 2048 key blocks of 64
 * over all sequences and KV heads; that launch then reduces dSink itself. (The pass splits the
 * heads for an even Hq/Hkv with fewer than 2048 such blocks, or fewer than 512 with a window.)
 */
int attn_sink_bwd_timed(const void* q, const void* k, const void* v, const float* sinks, const void* out,
                        const float* lse, const void* dout, int causal, int window, const int32_t* cu_seqlens,
                        const attn_sink_shape* shape, void* workspace, size_t workspace_bytes, float* dq,
                        float* dk, float* dv, float* dsinks, hipStream_t stream, void* const* events,
                        int num_events);

/*
 * Inference-shaped (decode) forward: a few new query tokens per sequence against that sequence's
 * cached keys and values. Sequence b has Lk_b = cu_seqlens_k[b+1] - cu_seqlens_k[b] cached tokens
 * (k, v rows, including the new tokens' own keys) and Nq_b = cu_seqlens_q[b+1] - cu_seqlens_q[b]
 * new queries (q rows), which are the sequence's last Nq_b tokens: new query j sits at position
 * Lk_b - Nq_b + j and, as in the causal forward, sees the keys at positions <= its own (and, with
 * window = W > 0, only the last W of them), plus the sink. Same operation as attn_sink_fwd with
 * causal = 1 restricted to those rows (nmedialink.com "惊爆！GPT-OSS-20B强化学习…", section
 * "GPT-OSS中的带注意力槽的注意力机制"); results agree with attn_sink_fwd's rows to rounding, not
 * bitwise (the keys are summed in another order).
 *
 *   q      [Tq, Hq, D] bf16;  k, v [Tk, Hkv, D] bf16;  sinks [Hq] fp32 (D = head_dim, 64 or 128)
 *   out    [Tq, Hq, D] fp32 (out_dtype ATTN_SINK_F32) or bf16 (ATTN_SINK_BF16)
 *   lse    [Hq, Tq] fp32, natural log, sink included
 *   cu_seqlens_q / cu_seqlens_k  [B+1] int32 on the device, non-decreasing, Nq_b <= Lk_b (trusted)
 * Requires max_q * (Hq / Hkv) <= 1024 (the (new token, query head) pairs of one KV head, taken 32
 * at a time as MFMA columns), else ATTN_SINK_ERR_UNSUPPORTED. workspace: caller-owned device memory
 * of at least attn_sink_decode_workspace_bytes(shape) bytes (per-chunk partial results); its
 * contents on entry do not matter. Same ownership, asynchrony and error conventions as above.
 */
typedef struct attn_sink_decode_shape {
  int32_t total_q;      /* Tq = cu_seqlens_q[B] */
  int32_t total_k;      /* Tk = cu_seqlens_k[B] */
  int32_t num_seqs;     /* B >= 1 */
  int32_t max_q;        /* >= every Nq_b, >= 0 */
  int32_t max_k;        /* >= every Lk_b, >= 0 (sizes the key chunks) */
  int32_t num_heads_q;  /* Hq */
  int32_t num_heads_kv; /* Hkv, divides Hq */
  int32_t head_dim;     /* 64 or 128 */
  float softmax_scale;  /* <= 0 selects 1/sqrt(head_dim) */
  int32_t out_dtype;    /* ATTN_SINK_F32 or ATTN_SINK_BF16 */
} attn_sink_decode_shape;

size_t attn_sink_decode_workspace_bytes(const attn_sink_decode_shape* shape);

int attn_sink_decode_fwd(const void* q, const void* k, const void* v, const float* sinks, int window,
                         const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, const attn_sink_decode_shape* shape,
                         void* workspace, size_t workspace_bytes, void* out, float* lse, hipStream_t stream);

/*
 * attn_sink_decode_fwd with timing: events (hipEvent_t handles owned by the caller) are recorded on
 * `stream` before the first kernel, between the kernels and after the last; num_events must equal
 * attn_sink_decode_num_kernels() + 1, else ATTN_SINK_ERR_BAD_SHAPE; an entry may be NULL (nothing
 * is recorded there). events == NULL behaves like attn_sink_decode_fwd.
 * attn_sink_decode_kernel_name(i) names kernel i (static string, or NULL).
 */
int attn_sink_decode_fwd_timed(const void* q, const void* k, const void* v, const float* sinks, int window,
                               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                               const attn_sink_decode_shape* shape, void* workspace, size_t workspace_bytes, void* out,
                               float* lse, hipStream_t stream, void* const* events, int num_events);
int attn_sink_decode_num_kernels(void);
const char* attn_sink_decode_kernel_name(int i);

/*
 * Optional host-side validation of sequence offsets, for callers that cannot vouch for them.
 * The kernels trust cu_seqlens (it lives on the device): a max_seqlen below the longest sequence
 * leaves that sequence's later rows unwritten (the grid is sized from it), and offsets that are
 * not non-decreasing or that run past T make the kernels read and write outside the tensors.
 * This check takes a HOST copy of the offsets, cu_seqlens_host[0 .. num_seqs], and returns
 * ATTN_SINK_OK when cu[0] = 0, cu[b] <= cu[b+1] for every b, cu[num_seqs] = total_tokens and
 * every length cu[b+1] - cu[b] <= max_seqlen; ATTN_SINK_ERR_NULL_PTR for a NULL array,
 * ATTN_SINK_ERR_BAD_SHAPE for num_seqs < 1, total_tokens < 0 or max_seqlen < 0, and
 * ATTN_SINK_ERR_BAD_SEQLENS otherwise. For the decode forward, check cu_seqlens_q (total_q,
 * max_q) and cu_seqlens_k (total_k, max_k) separately. Pure host code: no HIP call, no
 * allocation, thread-safe. (The packing it describes: nmedialink.com "惊爆！GPT-OSS-20B强化学习…",
 * section "结合Flash Attention V3的序列并行技术", padding removed and sequences concatenated.)
 */
int attn_sink_check_cu_seqlens(const int32_t* cu_seqlens_host, int32_t num_seqs, int32_t total_tokens,
                               int32_t max_seqlen);

/*
 * Decode forward whose results equal the training forward's, bit for bit: out and lse of new
 * query j of sequence b are exactly attn_sink_fwd's (causal, same window, scale and out_dtype) for
 * row Lk_b - Nq_b + j of that sequence run over its whole cached K/V. Same arguments, shapes and
 * limits as attn_sink_decode_fwd (max_q * (Hq / Hkv) <= 1024), but no workspace: each (sequence,
 * KV head, group of 32 (new token, query head) pairs) is one wave that streams every key its
 * queries see in the training forward's tile order, with the training forward's own tile
 * arithmetic, instead of splitting the keys over waves; it is correspondingly slower on long
 * caches. For rollout engines that must reproduce the trainer's log-probabilities exactly: the
 * pages trace their RL training instability to the inference engine's sink forward and the
 * training kernel disagreeing (nmedialink.com "惊爆！GPT-OSS-20B强化学习…", section
 * "纠正训练与推理不一致问题", Fig. 4). Errors as attn_sink_decode_fwd (no ATTN_SINK_ERR_WORKSPACE).
 */
int attn_sink_decode_fwd_ordered(const void* q, const void* k, const void* v, const float* sinks, int window,
                                 const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                 const attn_sink_decode_shape* shape, void* out, float* lse, hipStream_t stream);

/* Number of kernels attn_sink_bwd enqueues, and the name of kernel i (static string, or NULL). */
int attn_sink_bwd_num_kernels(void);
const char* attn_sink_bwd_kernel_name(int i);

/* Static, human-readable description of an ATTN_SINK_* code (never NULL). */
const char* attn_sink_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_SINK_H_ */
