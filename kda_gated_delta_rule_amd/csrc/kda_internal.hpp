// kda_internal.hpp -- launcher interface between the C ABI (kda_api.cpp) and the
// kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

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
    void* o;
    void* workspace;
    // prefix snapshots (0 / nullptr / 0: none): the state after (j + 1) * snap_every tokens of
    // sequence i goes to slot snap_slots[i * max_snaps + j] (negative: skipped)
    int snap_every = 0;
    const int32_t* snap_slots = nullptr;
    int max_snaps = 0;
};

// Each launcher returns hipSuccess or the launch error.
hipError_t launch_decode(const DecodeArgs& a, int bf16, int dk, int dv, hipStream_t stream);
hipError_t launch_replay(const ReplayArgs& a, int dk, int dv, hipStream_t stream);
size_t prefill_workspace_bytes(int num_seqs, int64_t total_tokens, int H, int dk, int dv,
                               int bf16);
// False where the prefill LDS plan does not fit (fp32 inputs need dk = 64).
bool prefill_supported(int bf16, int dk, int dv);
hipError_t launch_prefill(const PrefillArgs& a, int bf16, int dk, int dv, hipStream_t stream);
// The static prefill workspace of kda_chunk_prefill_noalloc (KDA_NOALLOC_SCRATCH_BYTES per
// GPU): its device address on the current device, looked up once per device; nullptr if the
// lookup fails.
void* prefill_noalloc_scratch();

}  // namespace kda
