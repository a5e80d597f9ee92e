// kda_api.cpp -- the extern "C" entry points declared in include/kda.h.
//
// Every argument check runs here, on the host, before any HIP call: an invalid
// call returns its error code without touching the device.  The launchers in
// the kernel translation units only see validated arguments.
#include "kda.h"

#include <math.h>

#include "kda_internal.hpp"

#define KDA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool supported_dim(int d) { return d == 64 || d == 128; }
bool valid_dtype(int dt) { return dt == KDA_F32 || dt == KDA_BF16; }

// Total element count of a product of non-negative sizes, or -1 on int64 overflow.
int64_t checked_mul(int64_t a, int64_t b) {
    if (a < 0 || b < 0) return -1;
    if (a != 0 && b > INT64_MAX / a) return -1;
    return a * b;
}

int to_status(hipError_t e) { return e == hipSuccess ? KDA_OK : KDA_ERR_HIP; }

}  // namespace

KDA_EXPORT int kda_decode_step(const void* q, const void* k, const void* v, int dtype,
                               const float* g, const float* beta, float* state_pool,
                               int64_t num_slots, const int32_t* slot_idx, int N, int T, int H,
                               int dk, int dv, float scale, int use_qk_l2norm, void* o,
                               float* records, hipStream_t stream) {
    if (!valid_dtype(dtype)) return KDA_ERR_INVALID_ARG;
    if (N < 0 || T < 1 || H < 1 || num_slots < 1) return KDA_ERR_INVALID_ARG;
    if (!isfinite(scale)) return KDA_ERR_INVALID_ARG;
    if (use_qk_l2norm != 0 && use_qk_l2norm != 1) return KDA_ERR_INVALID_ARG;
    if (!supported_dim(dk) || !supported_dim(dv)) return KDA_ERR_UNSUPPORTED;
    const void* ptrs[] = {q, k, v, g, beta, state_pool, slot_idx, o};
    for (const void* p : ptrs)
        if (!p || !aligned16(p)) return KDA_ERR_INVALID_ARG;
    if (records && !aligned16(records)) return KDA_ERR_INVALID_ARG;
    const int64_t tokens = checked_mul(checked_mul(N, T), H);
    if (tokens < 0 || checked_mul(tokens, 2 * dk + dv) < 0) return KDA_ERR_INVALID_ARG;
    if (checked_mul(checked_mul(num_slots, H), static_cast<int64_t>(dk) * dv) < 0)
        return KDA_ERR_INVALID_ARG;
    // launch size: up to 2 dv tiles per head, 256 threads each, within 32-bit work-items
    if (checked_mul(N, H) > (1ll << 22)) return KDA_ERR_INVALID_ARG;
    if (N == 0) return KDA_OK;

    kda::DecodeArgs a{q, k, v, g, beta, state_pool, slot_idx, o, records,
                      N, T, H, scale, use_qk_l2norm};
    return to_status(kda::launch_decode(a, dtype == KDA_BF16, dk, dv, stream));
}

namespace {

// Checks a kda_front and copies it into the launcher's arguments; KDA_OK or the error.
int front_args(const kda_front* f, kda::FrontArgs& out) {
    if (!f) return KDA_ERR_INVALID_ARG;
    if (f->conv_width < 1 || f->conv_width > 4) return KDA_ERR_INVALID_ARG;
    if (f->conv_silu != 0 && f->conv_silu != 1) return KDA_ERR_INVALID_ARG;
    const void* ptrs[] = {f->gate_scale, f->conv_q, f->conv_k, f->conv_v};
    for (const void* p : ptrs)
        if (!p || !aligned16(p)) return KDA_ERR_INVALID_ARG;
    if (f->conv_width > 1 && (!f->conv_state || !aligned16(f->conv_state))) return KDA_ERR_INVALID_ARG;
    out = kda::FrontArgs{f->gate_scale, f->conv_q,     f->conv_k,    f->conv_v,
                         f->conv_state, f->conv_width, f->conv_silu};
    return KDA_OK;
}

}  // namespace

KDA_EXPORT int kda_decode_step_front(const void* q, const void* k, const void* v, int dtype,
                                     const float* g, const float* beta, const kda_front* front,
                                     float* state_pool, int64_t num_slots, const int32_t* slot_idx,
                                     int N, int T, int H, int dk, int dv, float scale,
                                     int use_qk_l2norm, void* o, hipStream_t stream) {
    if (!valid_dtype(dtype)) return KDA_ERR_INVALID_ARG;
    if (N < 0 || T < 1 || H < 1 || num_slots < 1) return KDA_ERR_INVALID_ARG;
    if (!isfinite(scale)) return KDA_ERR_INVALID_ARG;
    if (use_qk_l2norm != 0 && use_qk_l2norm != 1) return KDA_ERR_INVALID_ARG;
    if (!supported_dim(dk) || !supported_dim(dv)) return KDA_ERR_UNSUPPORTED;
    const void* ptrs[] = {q, k, v, g, beta, state_pool, slot_idx, o};
    for (const void* p : ptrs)
        if (!p || !aligned16(p)) return KDA_ERR_INVALID_ARG;
    if (T > 8) return KDA_ERR_INVALID_ARG;  // the front's tokens form one block of at most 8
    kda::FrontArgs fa;
    if (const int st = front_args(front, fa); st != KDA_OK) return st;
    const int64_t tokens = checked_mul(checked_mul(N, T), H);
    if (tokens < 0 || checked_mul(tokens, 2 * dk + dv) < 0) return KDA_ERR_INVALID_ARG;
    if (checked_mul(checked_mul(num_slots, H), static_cast<int64_t>(dk) * dv) < 0)
        return KDA_ERR_INVALID_ARG;
    if (checked_mul(checked_mul(checked_mul(num_slots, H), 3), 2 * dk + dv) < 0)
        return KDA_ERR_INVALID_ARG;
    if (checked_mul(N, H) > (1ll << 22)) return KDA_ERR_INVALID_ARG;
    if (N == 0) return KDA_OK;

    kda::DecodeArgs a{q, k, v, g, beta, state_pool, slot_idx, o, nullptr,
                      N, T, H, scale, use_qk_l2norm, fa};
    return to_status(kda::launch_decode(a, dtype == KDA_BF16, dk, dv, stream));
}

KDA_EXPORT int kda_diag_state_stream(float* state_pool, int64_t num_slots, const int32_t* slot_idx,
                                     int N, int H, int dk, int dv, hipStream_t stream) {
    if (N < 0 || H < 1 || num_slots < 1) return KDA_ERR_INVALID_ARG;
    if (!supported_dim(dk) || !supported_dim(dv)) return KDA_ERR_UNSUPPORTED;
    if (!state_pool || !aligned16(state_pool) || !slot_idx || !aligned16(slot_idx)) return KDA_ERR_INVALID_ARG;
    if (checked_mul(checked_mul(num_slots, H), static_cast<int64_t>(dk) * dv) < 0)
        return KDA_ERR_INVALID_ARG;
    if (checked_mul(N, H) > (1ll << 22)) return KDA_ERR_INVALID_ARG;
    if (N == 0) return KDA_OK;
    return to_status(kda::launch_state_stream(state_pool, slot_idx, N, H, dk, dv, stream));
}

KDA_EXPORT int kda_replay_commit(float* state_pool, int64_t num_slots, const int32_t* slot_idx,
                                 const float* records, const int32_t* accepted_len, int N, int T,
                                 int H, int dk, int dv, hipStream_t stream) {
    if (N < 0 || T < 1 || H < 1 || num_slots < 1) return KDA_ERR_INVALID_ARG;
    if (!supported_dim(dk) || !supported_dim(dv)) return KDA_ERR_UNSUPPORTED;
    const void* ptrs[] = {state_pool, slot_idx, records, accepted_len};
    for (const void* p : ptrs)
        if (!p || !aligned16(p)) return KDA_ERR_INVALID_ARG;
    const int64_t tokens = checked_mul(checked_mul(N, T), H);
    if (tokens < 0 || checked_mul(tokens, 2 * dk + dv) < 0) return KDA_ERR_INVALID_ARG;
    if (checked_mul(checked_mul(num_slots, H), static_cast<int64_t>(dk) * dv) < 0)
        return KDA_ERR_INVALID_ARG;
    if (checked_mul(N, H) > (1ll << 22)) return KDA_ERR_INVALID_ARG;  // as for decode
    if (N == 0) return KDA_OK;

    kda::ReplayArgs a{state_pool, slot_idx, records, accepted_len, N, T, H};
    return to_status(kda::launch_replay(a, dk, dv, stream));
}

KDA_EXPORT size_t kda_chunk_prefill_workspace_size(int num_seqs, int64_t total_tokens, int H,
                                                   int dk, int dv, int dtype) {
    if (num_seqs < 0 || total_tokens < 0 || H < 1 || !supported_dim(dk) || !supported_dim(dv) ||
        !valid_dtype(dtype))
        return 0;
    return kda::prefill_workspace_bytes(num_seqs, total_tokens, H, dk, dv, dtype == KDA_BF16);
}

namespace {

int chunk_prefill_impl(const void* q, const void* k, const void* v, int dtype, const float* g,
                       const float* beta, const int32_t* cu_seqlens, int num_seqs,
                       int64_t total_tokens, float* state_pool, int64_t num_slots,
                       const int32_t* slot_idx, int h0_from_pool, int H, int dk, int dv,
                       float scale, int use_qk_l2norm, void* o, void* workspace,
                       size_t workspace_bytes, int snap_every, const int32_t* snap_slots,
                       int max_snaps, bool use_static, hipStream_t stream,
                       const kda::FrontArgs* front = nullptr) {
    if (!valid_dtype(dtype)) return KDA_ERR_INVALID_ARG;
    if (num_seqs < 0 || total_tokens < 0 || H < 1 || num_slots < 1) return KDA_ERR_INVALID_ARG;
    if (num_seqs == 0 && total_tokens != 0) return KDA_ERR_INVALID_ARG;
    if (!isfinite(scale)) return KDA_ERR_INVALID_ARG;
    if (use_qk_l2norm != 0 && use_qk_l2norm != 1) return KDA_ERR_INVALID_ARG;
    if (h0_from_pool != 0 && h0_from_pool != 1) return KDA_ERR_INVALID_ARG;
    if (!supported_dim(dk) || !supported_dim(dv)) return KDA_ERR_UNSUPPORTED;
    if (!kda::prefill_supported(dtype == KDA_BF16, dk, dv)) return KDA_ERR_UNSUPPORTED;
    if (total_tokens > (1ll << 31) - 1) return KDA_ERR_INVALID_ARG;  // int32 cu_seqlens
    // (chunk, head) items: 32-bit counts and offsets, and every launch's work-item count
    // within 32 bits (the segment kernels run one 512-thread block per (segment, head));
    // 2^22 items already take 176 GB of workspace or more
    if (H > 65535) return KDA_ERR_INVALID_ARG;
    if (checked_mul(total_tokens / 64 + num_seqs, H) > (1ll << 22)) return KDA_ERR_INVALID_ARG;
    if (checked_mul(checked_mul(total_tokens, H), 2 * dk + dv) < 0) return KDA_ERR_INVALID_ARG;
    if (checked_mul(checked_mul(num_slots, H), static_cast<int64_t>(dk) * dv) < 0)
        return KDA_ERR_INVALID_ARG;
    if (num_seqs == 0) return KDA_OK;
    const void* ptrs[] = {cu_seqlens, state_pool, slot_idx};
    for (const void* p : ptrs)
        if (!p || !aligned16(p)) return KDA_ERR_INVALID_ARG;
    if (total_tokens > 0) {
        const void* tp[] = {q, k, v, g, beta, o};
        for (const void* p : tp)
            if (!p || !aligned16(p)) return KDA_ERR_INVALID_ARG;
    }
    const size_t need =
        kda::prefill_workspace_bytes(num_seqs, total_tokens, H, dk, dv, dtype == KDA_BF16);
    if (use_static) {
        // the library's static array: sizes beyond it are rejected before any HIP call
        if (need > KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_WORKSPACE;
        workspace = kda::prefill_noalloc_scratch();
        if (!workspace) return KDA_ERR_HIP;
        workspace_bytes = KDA_NOALLOC_SCRATCH_BYTES;
    }
    if (!workspace || !aligned16(workspace) || workspace_bytes < need) return KDA_ERR_WORKSPACE;

    kda::PrefillArgs a{q, k, v, g, beta, cu_seqlens, num_seqs, total_tokens, state_pool,
                       slot_idx, h0_from_pool, H, scale, use_qk_l2norm, o, workspace,
                       snap_every, snap_slots, max_snaps};
    if (front) a.front = *front;
    return to_status(kda::launch_prefill(a, dtype == KDA_BF16, dk, dv, stream));
}

}  // namespace


KDA_EXPORT int kda_chunk_prefill(const void* q, const void* k, const void* v, int dtype,
                                 const float* g, const float* beta, const int32_t* cu_seqlens,
                                 int num_seqs, int64_t total_tokens, float* state_pool,
                                 int64_t num_slots, const int32_t* slot_idx, int h0_from_pool,
                                 int H, int dk, int dv, float scale, int use_qk_l2norm, void* o,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return chunk_prefill_impl(q, k, v, dtype, g, beta, cu_seqlens, num_seqs, total_tokens,
                              state_pool, num_slots, slot_idx, h0_from_pool, H, dk, dv, scale,
                              use_qk_l2norm, o, workspace, workspace_bytes, 0, nullptr, 0, false,
                              stream);
}

KDA_EXPORT int kda_chunk_prefill_noalloc(const void* q, const void* k, const void* v, int dtype,
                                         const float* g, const float* beta,
                                         const int32_t* cu_seqlens, int num_seqs,
                                         int64_t total_tokens, float* state_pool,
                                         int64_t num_slots, const int32_t* slot_idx,
                                         int h0_from_pool, int H, int dk, int dv, float scale,
                                         int use_qk_l2norm, void* o, hipStream_t stream) {
    return chunk_prefill_impl(q, k, v, dtype, g, beta, cu_seqlens, num_seqs, total_tokens,
                              state_pool, num_slots, slot_idx, h0_from_pool, H, dk, dv, scale,
                              use_qk_l2norm, o, nullptr, 0, 0, nullptr, 0, true, stream);
}

KDA_EXPORT int kda_chunk_prefill_front(const void* q, const void* k, const void* v, int dtype,
                                       const float* g, const float* beta, const kda_front* front,
                                       const int32_t* cu_seqlens, int num_seqs, int64_t total_tokens,
                                       float* state_pool, int64_t num_slots, const int32_t* slot_idx,
                                       int h0_from_pool, int H, int dk, int dv, float scale,
                                       int use_qk_l2norm, void* o, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
    kda::FrontArgs fa;
    if (const int st = front_args(front, fa); st != KDA_OK) return st;
    if (checked_mul(checked_mul(checked_mul(num_slots, H), 3), 2 * dk + dv) < 0)
        return KDA_ERR_INVALID_ARG;
    return chunk_prefill_impl(q, k, v, dtype, g, beta, cu_seqlens, num_seqs, total_tokens,
                              state_pool, num_slots, slot_idx, h0_from_pool, H, dk, dv, scale,
                              use_qk_l2norm, o, workspace, workspace_bytes, 0, nullptr, 0, false,
                              stream, &fa);
}

KDA_EXPORT int kda_chunk_prefill_snapshots(
    const void* q, const void* k, const void* v, int dtype, const float* g, const float* beta,
    const int32_t* cu_seqlens, int num_seqs, int64_t total_tokens, float* state_pool,
    int64_t num_slots, const int32_t* slot_idx, int h0_from_pool, int H, int dk, int dv,
    float scale, int use_qk_l2norm, void* o, void* workspace, size_t workspace_bytes,
    int snap_every, const int32_t* snap_slots, int max_snaps, hipStream_t stream) {
    if (snap_every < 64 || snap_every % 64 != 0 || max_snaps < 1) return KDA_ERR_INVALID_ARG;
    if (!snap_slots || !aligned16(snap_slots)) return KDA_ERR_INVALID_ARG;
    if (checked_mul(num_seqs, max_snaps) > (1ll << 31) - 1) return KDA_ERR_INVALID_ARG;
    return chunk_prefill_impl(q, k, v, dtype, g, beta, cu_seqlens, num_seqs, total_tokens,
                              state_pool, num_slots, slot_idx, h0_from_pool, H, dk, dv, scale,
                              use_qk_l2norm, o, workspace, workspace_bytes, snap_every,
                              snap_slots, max_snaps, false, stream);
}

KDA_EXPORT size_t kda_chunk_backward_workspace_size(int num_seqs, int64_t total_tokens, int H,
                                                    int dk, int dv, int dtype) {
    if (num_seqs < 0 || total_tokens < 0 || H < 1 || !supported_dim(dk) || !supported_dim(dv) ||
        !valid_dtype(dtype))
        return 0;
    return kda::backward_workspace_bytes(num_seqs, total_tokens, H, dk, dv, dtype == KDA_BF16);
}

KDA_EXPORT int kda_chunk_backward(const void* q, const void* k, const void* v, int dtype,
                                  const float* g, const float* beta, const int32_t* cu_seqlens,
                                  int num_seqs, int64_t total_tokens, const float* h0,
                                  const void* dout, const float* dht, int H, int dk, int dv,
                                  float scale, int use_qk_l2norm, void* dq, void* dk_out,
                                  void* dv_out, float* dg, float* dbeta, float* dh0,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!valid_dtype(dtype)) return KDA_ERR_INVALID_ARG;
    if (num_seqs < 0 || total_tokens < 0 || H < 1) return KDA_ERR_INVALID_ARG;
    if (num_seqs == 0 && total_tokens != 0) return KDA_ERR_INVALID_ARG;
    if (!isfinite(scale)) return KDA_ERR_INVALID_ARG;
    if (use_qk_l2norm != 0 && use_qk_l2norm != 1) return KDA_ERR_INVALID_ARG;
    if (!supported_dim(dk) || !supported_dim(dv)) return KDA_ERR_UNSUPPORTED;
    if (!kda::prefill_supported(dtype == KDA_BF16, dk, dv)) return KDA_ERR_UNSUPPORTED;
    if (total_tokens > (1ll << 31) - 1) return KDA_ERR_INVALID_ARG;
    if (H > 65535) return KDA_ERR_INVALID_ARG;
    if (checked_mul(total_tokens / 64 + num_seqs, H) > (1ll << 22)) return KDA_ERR_INVALID_ARG;
    if (checked_mul(checked_mul(total_tokens, H), 2 * dk + dv) < 0) return KDA_ERR_INVALID_ARG;
    if (checked_mul(checked_mul(num_seqs, H), static_cast<int64_t>(dk) * dv) < 0)
        return KDA_ERR_INVALID_ARG;
    if (num_seqs == 0) return KDA_OK;
    if (!cu_seqlens || !aligned16(cu_seqlens)) return KDA_ERR_INVALID_ARG;
    const void* opt[] = {h0, dht, dh0};
    for (const void* p : opt)
        if (p && !aligned16(p)) return KDA_ERR_INVALID_ARG;
    if (total_tokens > 0) {
        const void* tp[] = {q, k, v, g, beta, dout, dq, dk_out, dv_out, dg, dbeta};
        for (const void* p : tp)
            if (!p || !aligned16(p)) return KDA_ERR_INVALID_ARG;
    }
    const size_t need =
        kda::backward_workspace_bytes(num_seqs, total_tokens, H, dk, dv, dtype == KDA_BF16);
    if (!workspace || !aligned16(workspace) || workspace_bytes < need) return KDA_ERR_WORKSPACE;

    kda::BackwardArgs b{};
    b.fwd = kda::PrefillArgs{q, k, v, g, beta, cu_seqlens, num_seqs, total_tokens, nullptr,
                             nullptr, 1, H, scale, use_qk_l2norm, nullptr, workspace};
    b.h0 = h0;
    b.dout = dout;
    b.dht = dht;
    b.dq = dq;
    b.dk = dk_out;
    b.dv = dv_out;
    b.dg = dg;
    b.dbeta = dbeta;
    b.dh0 = dh0;
    kda::backward_setup(b, dk, dv, dtype == KDA_BF16);
    return to_status(kda::launch_backward(b, dtype == KDA_BF16, dk, dv, stream));
}

KDA_EXPORT const char* kda_status_string(int status) {
    switch (status) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_INVALID_ARG: return "KDA_ERR_INVALID_ARG: invalid argument";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: dk and dv must be 64 or 128";
        case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE: prefill workspace missing or too small";
        case KDA_ERR_HIP: return "KDA_ERR_HIP: a HIP launch failed";
        default: return "unknown kda_status";
    }
}
