// kda_diag.hip -- a diagnostic memory pass with the decode kernel's state access pattern.
//
// For each (sequence, head) of a one-token decode call, a workgroup of the decode kernel's shape
// (512 threads for dv = 128, 256 for dv = 64) loads the head's fp32 state from the sequence's
// slot exactly as decode_kernel does (16-byte non-temporal loads, thread (row group, column
// quad) owning rows rg, rg + RG, ...), holds it in registers, and stores it back unchanged.  No token inputs, no arithmetic, no outputs: its time is the floor
// the decode step's state traffic sets with this access pattern on this GPU, which the
// benchmark reports beside the decode kernel.  The pool's contents are left as they were.
#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {

namespace {

template <int DK, int DV, int NTHR>
__global__ __launch_bounds__(NTHR) void state_stream_kernel(float* pool, const int32_t* slot_idx, int H) {
    constexpr int NC4 = DV / 4, RG = NTHR / NC4, RPT = DK / RG;
    const int tid = threadIdx.x, nh = blockIdx.x;
    const int h = nh % H, n = nh / H;
    const int slot = slot_idx[n];
    if (slot < 0) return;
    float* S = pool + (static_cast<int64_t>(slot) * H + h) * (DK * DV);
    const int c4 = tid % NC4, rg = tid / NC4, col0 = 4 * c4;
    float4 s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) s[i] = load_stream4(S + (rg + RG * i) * DV + col0);
    // opaque to the compiler (no instruction), which would otherwise drop a store of the value
    // just loaded from the same address, and the load with it
#pragma unroll
    for (int i = 0; i < RPT; ++i) asm volatile("" : "+v"(s[i].x), "+v"(s[i].y), "+v"(s[i].z), "+v"(s[i].w));
#pragma unroll
    for (int i = 0; i < RPT; ++i) store_stream4(S + (rg + RG * i) * DV + col0, s[i]);
}

template <int DK, int DV>
hipError_t launch_d(float* pool, const int32_t* slot_idx, int N, int H, hipStream_t stream) {
    constexpr int NTHR = DV == 128 ? 512 : 256;  // as decode_kernel at T = 1
    hipLaunchKernelGGL((state_stream_kernel<DK, DV, NTHR>), dim3(static_cast<unsigned>(N) * H), dim3(NTHR), 0,
                       stream, pool, slot_idx, H);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_state_stream(float* pool, const int32_t* slot_idx, int N, int H, int dk, int dv,
                               hipStream_t stream) {
    if (dk == 128 && dv == 128) return launch_d<128, 128>(pool, slot_idx, N, H, stream);
    if (dk == 128 && dv == 64) return launch_d<128, 64>(pool, slot_idx, N, H, stream);
    if (dk == 64 && dv == 128) return launch_d<64, 128>(pool, slot_idx, N, H, stream);
    if (dk == 64 && dv == 64) return launch_d<64, 64>(pool, slot_idx, N, H, stream);
    return hipErrorInvalidValue;
}

}  // namespace kda
