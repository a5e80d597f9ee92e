/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention hot path.
 *
 * The method (gated delta rule, one sequence, one head, state S of dk x dv,
 * row c = key channel, dv contiguous), per token, in the order the decode
 * kernel description lists the steps (page "Kimi K3 ... 昇腾 day-0 adaptation",
 * section "融合算子加速：KDA Prefill与Decode双路径"):
 *
 *   qh = q / sqrt(|q|^2 + 1e-6),  kh = k / sqrt(|k|^2 + 1e-6)    Q/K L2 norm
 *   alpha = exp(g)                       per key channel          gate
 *   S' = diag(alpha) S                                            state decay
 *   u  = beta * (v - S'^T kh)                                     delta rule, beta
 *   S  = S' + kh u^T                                              outer-product update
 *   o  = scale * S^T qh                                           output (updated state)
 *   S written back to its state-pool slot                         in-place write-back
 *
 * Conventions shared by every entry point:
 *  - Ownership: the caller owns every buffer.  No entry point allocates or frees
 *    memory or keeps state between calls; calls are thread-safe.  (Exception:
 *    kda_chunk_prefill_noalloc uses a library-owned static device array per GPU.)
 *  - All pointers are device pointers to contiguous row-major arrays, 16-byte
 *    aligned.  Index arrays (slot_idx, accepted_len, cu_seqlens) live on the device
 *    and are read by the kernels, not by the host.
 *  - Supported head dims: dk, dv in {64, 128}, for both dtypes and every entry point.
 *    Other values: KDA_ERR_UNSUPPORTED.
 *  - Every argument check runs on the host before any HIP call; on failure nothing
 *    is launched and the error code is returned.  Device-resident indices are not
 *    checked: a slot index >= num_slots, duplicate slots within one call, or
 *    cu_seqlens that do not match total_tokens are undefined behaviour.
 *  - Calls are asynchronous on `stream` (NULL = the null stream).  A launch failure
 *    returns KDA_ERR_HIP.
 *  - dtype KDA_BF16: q, k, v and o are bfloat16 (o rounded to nearest even); with
 *    KDA_F32 they are fp32.  g, beta, the state pool and records are always fp32.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARG = -1, /* null/misaligned pointer, bad size or dtype      */
    KDA_ERR_UNSUPPORTED = -2, /* dk or dv outside {64, 128} */
    KDA_ERR_WORKSPACE = -3,   /* prefill workspace null or too small             */
    KDA_ERR_HIP = -4          /* a HIP launch failed                             */
} kda_status;

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

/*
 * kda_decode_step -- fused decode / MTP step over state-pool slots.
 *
 * Follows the decode path of section "KDA Prefill与Decode双路径" (one fused kernel:
 * L2 norm, gate and beta, decay, delta rule, outer-product update, output, in-place
 * final-state write-back; work split by sequence x value head) and, with records,
 * the verification half of ReplaySSM (page "2.8倍性能提升！基于CANN实现Kimi K3高性能推理",
 * section 04): per token a record {kh | alpha | u} is written in place of a state.
 *
 *   q, k        [N, T, H, dk]   dtype
 *   v           [N, T, H, dv]   dtype
 *   g           [N, T, H, dk]   fp32, log of the per-key-channel decay (g <= 0 expected)
 *   beta        [N, T, H]       fp32
 *   state_pool  [num_slots, H, dk, dv] fp32
 *   slot_idx    [N] int32: sequence n uses slot slot_idx[n]; a negative index skips the
 *               sequence (no state read or write, its o is written as zeros, its records
 *               are not written).  Slots must be distinct within a call.
 *   o           [N, T, H, dv]   dtype (output)
 *   records     NULL: commit mode -- the T tokens are applied in order and the final
 *               state is written back to the slot in place.
 *               non-NULL: verify mode -- the slot is left untouched; fp32 records
 *               [N, T, H, 2*dk + dv] = {kh (dk) | alpha (dk) | u (dv)} are written for
 *               every token, and o is the output the token would have if committed.
 *   T >= 1 tokens per sequence (T = 1 decode, T > 1 MTP / speculative verify).
 *   scale       output scale (1/sqrt(dk) is the usual choice).
 *   use_qk_l2norm  1: normalise q and k as above; 0: use them as given.
 * Limit: N * H <= 2^22 (a launch's work-item count stays within 32 bits; 2^22 (sequence,
 * head) states are 256 GiB at dk = dv = 128), else KDA_ERR_INVALID_ARG.
 */
int kda_decode_step(const void* q, const void* k, const void* v, int dtype, const float* g,
                    const float* beta, float* state_pool, int64_t num_slots,
                    const int32_t* slot_idx, int N, int T, int H, int dk, int dv, float scale,
                    int use_qk_l2norm, void* o, float* records, hipStream_t stream);

/*
 * kda_replay_commit -- the commit half of ReplaySSM (page "2.8倍性能提升！基于CANN实现
 * Kimi K3高性能推理", section 04): the records of a sequence's accepted prefix update its
 * committed slot state in token order.
 *
 * For each sequence n with slot_idx[n] >= 0 and each head, starting from the slot's
 * committed state, applies records[n, t, h] for t = 0 .. accepted_len[n]-1:
 *     S <- diag(alpha) S + kh u^T
 * and writes the state back to the slot.  records are those written by
 * kda_decode_step in verify mode ([N, T, H, 2*dk + dv] fp32).  accepted_len [N] int32
 * on the device, each in 0..T (0 leaves the slot untouched; values outside 0..T are
 * undefined behaviour).  The fp32 arithmetic matches commit-mode kda_decode_step with
 * T >= 2, so replaying a prefix of two or more tokens reproduces, bit for bit, the state
 * that committing the same tokens gives (a one-token commit agrees up to fp32 rounding).
 * Limit: N * H <= 2^22, as for kda_decode_step.
 */
int kda_replay_commit(float* state_pool, int64_t num_slots, const int32_t* slot_idx,
                      const float* records, const int32_t* accepted_len, int N, int T, int H,
                      int dk, int dv, hipStream_t stream);

/*
 * kda_chunk_prefill_workspace_size -- bytes of device workspace kda_chunk_prefill
 * needs for these sizes (an upper bound that depends only on the arguments).
 */
size_t kda_chunk_prefill_workspace_size(int num_seqs, int64_t total_tokens, int H, int dk,
                                        int dv, int dtype);

/*
 * kda_chunk_prefill -- varlen chunked prefill (section "KDA Prefill与Decode双路径":
 * 64-token chunks, with Q/K normalisation, gate cumulation and the chunk recurrence
 * done as batched work).  The result equals running the token recurrence over each
 * sequence.
 *
 *   q, k        [total_tokens, H, dk]   dtype
 *   v           [total_tokens, H, dv]   dtype
 *   g           [total_tokens, H, dk]   fp32
 *   beta        [total_tokens, H]       fp32
 *   cu_seqlens  [num_seqs + 1] int32 on the device: sequence i is tokens
 *               cu_seqlens[i] .. cu_seqlens[i+1]-1; cu_seqlens[0] = 0,
 *               non-decreasing, cu_seqlens[num_seqs] = total_tokens.  Empty
 *               sequences are allowed (the state passes through).
 *   state_pool  [num_slots, H, dk, dv] fp32; slot_idx [num_seqs] int32 (distinct,
 *               >= 0).  h0_from_pool = 1: the initial state of sequence i is read from
 *               slot slot_idx[i]; 0: it is zero.  The final state is always written
 *               to slot slot_idx[i].
 *   o           [total_tokens, H, dv] dtype (output)
 *   workspace   device buffer of at least kda_chunk_prefill_workspace_size(...) bytes;
 *               its contents on entry do not matter.
 * Limits: H <= 65535 and (total_tokens / 64 + num_seqs) * H <= 2^22, else
 * KDA_ERR_INVALID_ARG (2^22 items take 176 GB of workspace or more).
 * Numerical range: the intra-chunk products split exp(G_t - G_s) (G the in-chunk cumulative
 * gate) at a reference between t and s; the one limit left is that, per key channel, the sum
 * of g over any 8 consecutive tokens of a 16-token block stays above about -85 (not checked;
 * beyond it exp overflows inside the product and the results are not finite).
 * Precision with bf16 inputs: the intra-chunk q.k and k.k products carry each operand as a
 * high and a low bf16 part (about 16 bits); the record operands of the chunk carry (W, U,
 * QG, Kt, P) and the carried state as an operand of the inter-chunk products are rounded to
 * bf16 (the state itself is kept in fp32).  fp32 inputs use fp32 operands throughout.
 */
int kda_chunk_prefill(const void* q, const void* k, const void* v, int dtype, const float* g,
                      const float* beta, const int32_t* cu_seqlens, int num_seqs,
                      int64_t total_tokens, float* state_pool, int64_t num_slots,
                      const int32_t* slot_idx, int h0_from_pool, int H, int dk, int dv,
                      float scale, int use_qk_l2norm, void* o, void* workspace,
                      size_t workspace_bytes, hipStream_t stream);

/*
 * kda_chunk_prefill_snapshots -- kda_chunk_prefill that also keeps prefix states, for a
 * KDA prefix cache (the Kimi K3 day-0 adaptation page, section "Kimi K3——面向长程智能体的
 * 开源旗舰大模型", infrastructure item: KDA Prefix-Cache reuses KDA states across shared
 * prefixes).  The page names the feature only; here it is read as states stored at
 * chunk-aligned positions, so a later request sharing the prefix resumes from the stored
 * state instead of recomputing it.
 *
 * Every argument of kda_chunk_prefill, plus:
 *   snap_every  snapshot interval in tokens, a positive multiple of 64 (chunk aligned)
 *   snap_slots  [num_seqs, max_snaps] int32 on the device: the state of sequence i after
 *               (j + 1) * snap_every tokens is written to pool slot snap_slots[i][j],
 *               for every j < max_snaps with (j + 1) * snap_every <= the sequence's
 *               length (at the full length it equals the final state); a negative entry
 *               skips that snapshot.  Snapshot slots must be distinct from each other
 *               and from the call's slot_idx (not checked: undefined behaviour).
 *   max_snaps   >= 1, the row length of snap_slots
 * The snapshot is the carried fp32 state at that chunk boundary (the same value the
 * following chunk starts from), so resuming a prefill or decode from the slot continues
 * the sequence exactly as the longer call would.
 * Errors: as kda_chunk_prefill; snap_every not a positive multiple of 64, max_snaps < 1,
 * a null or misaligned snap_slots, or num_seqs * max_snaps >= 2^31 give
 * KDA_ERR_INVALID_ARG.
 */
int kda_chunk_prefill_snapshots(const void* q, const void* k, const void* v, int dtype,
                                const float* g, const float* beta, const int32_t* cu_seqlens,
                                int num_seqs, int64_t total_tokens, float* state_pool,
                                int64_t num_slots, const int32_t* slot_idx, int h0_from_pool,
                                int H, int dk, int dv, float scale, int use_qk_l2norm, void* o,
                                void* workspace, size_t workspace_bytes, int snap_every,
                                const int32_t* snap_slots, int max_snaps, hipStream_t stream);

/*
 * kda_chunk_backward_workspace_size -- bytes of device workspace kda_chunk_backward needs for
 * these sizes (an upper bound that depends only on the arguments; 0 for invalid arguments).
 */
size_t kda_chunk_backward_workspace_size(int num_seqs, int64_t total_tokens, int H, int dk,
                                         int dv, int dtype);

/*
 * kda_chunk_backward -- gradients of the varlen chunked prefill, for training (the Kimi K3
 * day-0 adaptation page, section "基于昇腾实现Kimi K3训练基础功能适配与深度优化": the item on
 * forward and backward linear-attention kernels; the page gives no backward formula, so this
 * is the chain rule through the forward defined above).
 *
 * For o and the final states ht of kda_chunk_prefill on the same inputs (initial states h0),
 * returns the gradients of L = sum(dout * o) + sum(dht * ht):
 *   q, k, v, g, beta, cu_seqlens, num_seqs, total_tokens, H, dk, dv, scale, use_qk_l2norm
 *               as kda_chunk_prefill (same layouts and dtype)
 *   h0          [num_seqs, H, dk, dv] fp32 dense initial states, or NULL (zero)
 *   dout        [total_tokens, H, dv] dtype
 *   dht         [num_seqs, H, dk, dv] fp32, or NULL (zero)
 *   dq, dk_out  [total_tokens, H, dk] dtype;  dv_out [total_tokens, H, dv] dtype
 *   dg          [total_tokens, H, dk] fp32;   dbeta [total_tokens, H] fp32
 *   dh0         [num_seqs, H, dk, dv] fp32, or NULL (not written)
 *   workspace   at least kda_chunk_backward_workspace_size(...) bytes; contents on entry do not
 *               matter
 * The call runs the forward again (the state entering every 64-token chunk is kept in the
 * workspace), then the reverse chunk recurrence of the state gradient and the per-chunk input
 * gradients, all in fp32 arithmetic.  Supported shapes, limits and errors as kda_chunk_prefill
 * (the same numerical range).
 */
int kda_chunk_backward(const void* q, const void* k, const void* v, int dtype, const float* g,
                       const float* beta, const int32_t* cu_seqlens, int num_seqs,
                       int64_t total_tokens, const float* h0, const void* dout, const float* dht,
                       int H, int dk, int dv, float scale, int use_qk_l2norm, void* dq,
                       void* dk_out, void* dv_out, float* dg, float* dbeta, float* dh0,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * kda_chunk_prefill_noalloc -- kda_chunk_prefill without a caller workspace, for callers that
 * cannot allocate device memory: code under HIP graph capture, serving loops that must not
 * allocate, harnesses that forbid hipMalloc.  The call itself allocates nothing.
 *
 * Arguments, results and errors are those of kda_chunk_prefill minus workspace and
 * workspace_bytes.  The workspace is a library-owned static device array of
 * KDA_NOALLOC_SCRATCH_BYTES per GPU (held from the library's first use of the GPU until the
 * process ends); its address is looked up on the first call on each device.  A call whose
 * kda_chunk_prefill_workspace_size(...) exceeds KDA_NOALLOC_SCRATCH_BYTES returns
 * KDA_ERR_WORKSPACE before any HIP call (about 3,000 (64-token chunk, head) items at
 * dk = dv = 128: e.g. 4,096 tokens x 32 heads, or 8,192 x 16).  Every call on one GPU uses
 * the same array: calls that overlap in time on one GPU (on different streams or from
 * different host threads) race and give undefined results; calls ordered on one stream are
 * safe.  The array's contents between calls do not matter (nothing needs clearing).
 */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
int kda_chunk_prefill_noalloc(const void* q, const void* k, const void* v, int dtype,
                              const float* g, const float* beta, const int32_t* cu_seqlens,
                              int num_seqs, int64_t total_tokens, float* state_pool,
                              int64_t num_slots, const int32_t* slot_idx, int h0_from_pool, int H,
                              int dk, int dv, float scale, int use_qk_l2norm, void* o,
                              hipStream_t stream);

/*
 * kda_front -- the input front of the recurrence, for the fused entry points below.  The
 * CANN Kimi K3 inference page (section 03, MegaKDA) moves the steps in front of KDA -- the
 * input projections, ShortConv, and the gate and beta processing -- into the same operator,
 * without giving their formulas.  The front here takes the gate and beta processing and
 * ShortConv, read as:
 *   q, k, v    each convolved along the tokens of its sequence, channel by channel (causal
 *              depthwise, width W = conv_width in 1..4):
 *                  y_t[c] = sum_{j < W} w[h][c][j] x_{t-(W-1)+j}[c]
 *              the W - 1 inputs before the call's first token taken from the slot's
 *              convolution state; with conv_silu = 1, y <- y / (1 + e^-y) (SiLU).  The
 *              convolved q, k, v then enter the recurrence (L2 norm included).
 *   g          the log-decay is -gate_scale[h] * softplus(z) for the raw gate z passed in g's
 *              place (softplus(z) = log(1 + e^z)); the workloads' g = -0.1 softplus(N(0, 1))
 *              is gate_scale = 0.1.
 *   beta       1 / (1 + e^-b) for the raw value b passed in beta's place.
 * The input projections are not included (the pages give no weight shapes).
 *
 *   gate_scale  [H] fp32, >= 0
 *   conv_q      [H, dk, conv_width] fp32;  conv_k [H, dk, conv_width] fp32;
 *   conv_v      [H, dv, conv_width] fp32   (w[h][c][j] above; j = W - 1 is the current token)
 *   conv_state  [num_slots, H, conv_width - 1, 2*dk + dv] in the io dtype (channels q | k | v,
 *               row 0 the oldest input): read for the slot's sequence and replaced by its last
 *               W - 1 inputs (earlier rows kept where the call has fewer tokens).  May be NULL
 *               when conv_width = 1.
 *   conv_width  1..4;  conv_silu 0 or 1
 * The struct is read on the host during the call; the arrays it points to are device memory,
 * 16-byte aligned.
 */
typedef struct {
    const float* gate_scale;
    const float* conv_q;
    const float* conv_k;
    const float* conv_v;
    void* conv_state;
    int conv_width;
    int conv_silu;
} kda_front;

/*
 * kda_decode_step_front -- kda_decode_step in commit mode with the input front fused in: the
 * convolution, the gate and beta processing, the convolution state's update and the decode
 * step run in one kernel per (sequence, head).  q, k, v [N, T, H, *] are the raw inputs of the
 * convolution, g [N, T, H, dk] the raw gates z, beta [N, T, H] the raw b (see kda_front);
 * the other arguments and the results are those of kda_decode_step with records = NULL (the
 * front has no verify mode).  1 <= T <= 8 tokens are applied in order (longer inputs take the
 * prefill).  A skipped sequence
 * (negative slot) keeps its convolution state.
 * Errors: as kda_decode_step; front NULL, a null or misaligned gate_scale or conv weight,
 * conv_width outside 1..4, conv_silu not 0 or 1, (conv_width > 1) a null or misaligned
 * conv_state, or T > 8 give KDA_ERR_INVALID_ARG.
 */
int kda_decode_step_front(const void* q, const void* k, const void* v, int dtype, const float* g,
                          const float* beta, const kda_front* front, float* state_pool,
                          int64_t num_slots, const int32_t* slot_idx, int N, int T, int H, int dk,
                          int dv, float scale, int use_qk_l2norm, void* o, hipStream_t stream);

/*
 * kda_chunk_prefill_front -- kda_chunk_prefill with the input front fused in: the chunk kernel
 * convolves each 64-token chunk's raw q, k, v in its registers (the three inputs before the
 * chunk from the previous chunk or, at a sequence start, from the slot's convolution state)
 * and processes the raw gates and beta values there, and the output pass writes each
 * sequence's convolution state back to its slot.  q, k, v [total_tokens, H, *] are the raw
 * inputs of the convolution, g [total_tokens, H, dk] the raw gates z, beta [total_tokens, H]
 * the raw b (see kda_front); the other arguments and the results are those of
 * kda_chunk_prefill.  h0_from_pool = 1 reads both the recurrent and the convolution state
 * from the slot; 0 starts both from zero.  With bf16 inputs the convolved q, k, v are rounded
 * to bf16 before the chunk products (the decode front keeps them in fp32).
 * Errors: as kda_chunk_prefill, plus the kda_front checks of kda_decode_step_front.
 */
int kda_chunk_prefill_front(const void* q, const void* k, const void* v, int dtype, const float* g,
                            const float* beta, const kda_front* front, const int32_t* cu_seqlens,
                            int num_seqs, int64_t total_tokens, float* state_pool,
                            int64_t num_slots, const int32_t* slot_idx, int h0_from_pool, int H,
                            int dk, int dv, float scale, int use_qk_l2norm, void* o,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * kda_diag_state_stream -- a diagnostic, not part of the method: reads the fp32 state of each
 * sequence's slot (slot_idx [N] int32 on the device, negative skips) with the access pattern of
 * kda_decode_step's T = 1 kernel (a workgroup per (sequence, head), 512 threads at dv = 128, the
 * whole state held in registers, 16-byte non-temporal accesses) and writes it back unchanged.  Its time is
 * the floor that the decode step's state traffic sets on the GPU; the benchmark reports it beside
 * the decode kernel.  Errors and limits as kda_decode_step.
 */
int kda_diag_state_stream(float* state_pool, int64_t num_slots, const int32_t* slot_idx, int N, int H,
                          int dk, int dv, hipStream_t stream);

/* Human-readable name of a kda_status value (static string, never NULL). */
const char* kda_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
