// kda_internal.hpp -- launcher interface between the C ABI (kda_api.cpp) and the
// kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

// The input front (kda_front in include/kda.h): gate_scale == nullptr means none.  With a
// front, the g argument holds raw gates z (g = -gate_scale[h] softplus(z)), beta raw values
// (beta = sigmoid), and q, k, v the inputs of the causal depthwise convolution.
struct FrontArgs {
    const float* gate_scale = nullptr;  // [H]
    const float* conv_q = nullptr;      // [H, dk, conv_width]
    const float* conv_k = nullptr;      // [H, dk, conv_width]
    const float* conv_v = nullptr;      // [H, dv, conv_width]
    void* conv_state = nullptr;         // [num_slots, H, conv_width - 1, 2 dk + dv], io dtype
    int conv_width = 1;
    int conv_silu = 0;
};

struct DecodeArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    float* pool;
    const int32_t* slot_idx;
    void* o;
    float* records;  // nullptr: commit mode
    int N, T, H;
    float scale;
    int use_l2;
    FrontArgs front = {};
};

struct ReplayArgs {
    float* pool;
    const int32_t* slot_idx;
    const float* records;
    const int32_t* accepted;
    int N, T, H;
};

struct PrefillArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    const int32_t* cu_seqlens;
    int num_seqs;
    int64_t total_tokens;
    float* pool;
    const int32_t* slot_idx;
    int h0_from_pool;
    int H;
    float scale;
    int use_l2;
    // output [T][H][dv]; nullptr (internal: the backward's forward pass, which keeps only the
    // chunk states) computes no O, and the intra-chunk records then skip QG and P
    void* o;
    void* workspace;
    // prefix snapshots (0 / nullptr / 0: none): the state after (j + 1) * snap_every tokens of
    // sequence i goes to slot snap_slots[i * max_snaps + j] (negative: skipped)
    int snap_every = 0;
    const int32_t* snap_slots = nullptr;
    int max_snaps = 0;
    // chunk states (nullptr: none): the fp32 [dk][dv] state entering chunk c of the batch
    // (global chunk index, head h) goes to chunk_states + (c * H + h) * chunk_state_stride
    float* chunk_states = nullptr;
    size_t chunk_state_stride = 0;  // floats
    FrontArgs front = {};
};

struct BackwardArgs {
    PrefillArgs fwd;   // the forward's inputs; its pool, slots, o and chunk states are set by
                       // backward_setup to parts of the backward workspace
    const float* h0;   // [num_seqs, H, dk, dv] or nullptr (zero)
    const void* dout;  // [T, H, dv] dtype
    const float* dht;  // [num_seqs, H, dk, dv] or nullptr (zero)
    void* dq;          // [T, H, dk] dtype
    void* dk;          // [T, H, dk] dtype
    void* dv;          // [T, H, dv] dtype
    float* dg;         // [T, H, dk]
    float* dbeta;      // [T, H]
    float* dh0;        // [num_seqs, H, dk, dv] or nullptr
};

// Each launcher returns hipSuccess or the launch error.
hipError_t launch_decode(const DecodeArgs& a, int bf16, int dk, int dv, hipStream_t stream);
hipError_t launch_replay(const ReplayArgs& a, int dk, int dv, hipStream_t stream);
hipError_t launch_state_stream(float* pool, const int32_t* slot_idx, int N, int H, int dk, int dv,
                               hipStream_t stream);
size_t prefill_workspace_bytes(int num_seqs, int64_t total_tokens, int H, int dk, int dv,
                               int bf16);
// False where the prefill LDS plan does not fit a CU (every dk, dv in {64, 128} fits).
bool prefill_supported(int bf16, int dk, int dv);
hipError_t launch_prefill(const PrefillArgs& a, int bf16, int dk, int dv, hipStream_t stream);
// The static prefill workspace of kda_chunk_prefill_noalloc (KDA_NOALLOC_SCRATCH_BYTES per
// GPU): its device address on the current device, looked up once per device; nullptr if the
// lookup fails.
void* prefill_noalloc_scratch();
size_t backward_workspace_bytes(int num_seqs, int64_t total_tokens, int H, int dk, int dv, int bf16);
void backward_setup(BackwardArgs& b, int dk, int dv, int bf16);
hipError_t launch_backward(const BackwardArgs& b, int bf16, int dk, int dv, hipStream_t stream);

}  // namespace kda
