// kda_decode.hip -- fused KDA decode / MTP / verify kernel and the ReplaySSM
// commit kernel for gfx950.
//
// Decode follows the fused decode path of the Kimi K3 day-0 adaptation page
// (section "融合算子加速：KDA Prefill与Decode双路径"): one launch does the Q/K L2
// norm, gate and beta processing, state decay, delta rule, outer-product update,
// output and in-place write-back, with work split by sequence x value head.
// Replay follows section 04 (ReplaySSM) of the CANN Kimi K3 inference page.
//
// Design (MI355X-first, not the NPU's Unified-Buffer scheme):
//  * One workgroup of 256 threads (4 wave64) per (sequence, head, dv tile of BV
//    columns).  The fp32 state tile (dk x BV) is streamed once from HBM into
//    VGPRs with 16-byte non-temporal loads, kept there for all T tokens, and
//    written back once with non-temporal stores.  The step is HBM-bound (about 0.9 flop per byte), so nothing goes
//    through MFMA.
//  * Thread (rg, c4) owns columns 4*c4..4*c4+3 of rows rg, rg+RG, rg+2RG, ...;
//    a wave's load instruction covers whole adjacent rows, so every access is
//    a fully used 16-byte-per-lane coalesced transaction.
//  * Both reductions over dk (S'^T k and S'^T q) come from one pass over the
//    decayed state, using o = scale * (S'^T q + (k.q) u): the output needs no
//    second pass over the updated state.  Partial sums are combined with wave
//    butterflies (xor shuffles) and one LDS exchange across the 4 waves, i.e. one
//    barrier per token.
//  * Per-token vectors (qh, kh, alpha, v, beta, k.q) are prepared by one wave per
//    token into LDS (a block of TB tokens at a time), stored row-permuted so each
//    thread reads its rows with 16-byte LDS loads.
#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr float kNormEps = 1e-6f;

template <int DK, int DV, int BV>
struct Tile {
    static constexpr int NC4 = BV / 4;          // float4 column groups per tile
    static constexpr int RG = kThreads / NC4;   // row groups
    static constexpr int RPT = DK / RG;         // rows per thread
    static constexpr int NT = DV / BV;          // tiles per head
    static constexpr int EPL = DK / kWave;      // key channels per lane in the prep
    static constexpr int VPL = (BV + kWave - 1) / kWave;  // v columns per lane in the prep
    static_assert(kThreads % NC4 == 0 && DK % RG == 0 && RPT % 4 == 0, "tile shape");
    static_assert(EPL >= 1 && BV % 4 == 0 && DV % BV == 0, "tile shape");
    // LDS slot of key channel c: rows of one thread are contiguous.
    __device__ static constexpr int pos(int c) { return (c % RG) * RPT + c / RG; }
};

// Per-token vectors prepared in LDS.
template <int DK, int BV, int TB>
struct TokenLds {
    float q[TB][DK];
    float k[TB][DK];
    float a[TB][DK];
    float v[TB][BV];
    float beta[TB];
    float kq[TB];
};

// Prepares token t (local slot j) by one wave: L2 norms, alpha = exp(g), k.q.
template <int DK, int DV, int BV, int TB, class TIn, bool VERIFY>
__device__ __forceinline__ void prep_token(const DecodeArgs& a, TokenLds<DK, BV, TB>& L, int j,
                                           int n, int t, int h, int tile, int lane) {
    using C = Tile<DK, DV, BV>;
    const int64_t tok = (static_cast<int64_t>(n) * a.T + t) * a.H + h;
    const int64_t rowk = tok * DK;
    float qv[C::EPL], kv[C::EPL], gv[C::EPL];
    if constexpr (C::EPL == 2) {
        const int c = lane * 2;
        const float2 x = load2<TIn>(a.q, rowk + c);
        const float2 y = load2<TIn>(a.k, rowk + c);
        const float2 z = *reinterpret_cast<const float2*>(a.g + rowk + c);
        qv[0] = x.x; qv[1] = x.y;
        kv[0] = y.x; kv[1] = y.y;
        gv[0] = z.x; gv[1] = z.y;
    } else {
        static_assert(C::EPL == 1, "dk is 64 or 128");
        qv[0] = load1<TIn>(a.q, rowk + lane);
        kv[0] = load1<TIn>(a.k, rowk + lane);
        gv[0] = a.g[rowk + lane];
    }
    float vv[C::VPL];
#pragma unroll
    for (int e = 0; e < C::VPL; ++e) {
        const int col = lane + e * kWave;
        vv[e] = 0.f;
        if (col < BV) {
            const int64_t idx = tok * DV + tile * BV + col;
            vv[e] = load1<TIn>(a.v, idx);
        }
    }
    const float b = a.beta[tok];

    float iq = 1.f, ik = 1.f;
    if (a.use_l2) {
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int e = 0; e < C::EPL; ++e) {
            sq = fmaf(qv[e], qv[e], sq);
            sk = fmaf(kv[e], kv[e], sk);
        }
        sq = wave_sum(sq);
        sk = wave_sum(sk);
        iq = 1.f / sqrtf(sq + kNormEps);
        ik = 1.f / sqrtf(sk + kNormEps);
    }
    float kq = 0.f;
    float* rec = VERIFY ? a.records + tok * (2 * DK + DV) : nullptr;
#pragma unroll
    for (int e = 0; e < C::EPL; ++e) {
        const int c = lane * C::EPL + e;
        const float qh = qv[e] * iq, kh = kv[e] * ik, al = expf(gv[e]);
        kq = fmaf(qh, kh, kq);
        L.q[j][C::pos(c)] = qh;
        L.k[j][C::pos(c)] = kh;
        L.a[j][C::pos(c)] = al;
        if (VERIFY && tile == 0) {
            rec[c] = kh;
            rec[DK + c] = al;
        }
    }
    kq = wave_sum(kq);
#pragma unroll
    for (int e = 0; e < C::VPL; ++e) {
        const int col = lane + e * kWave;
        if (col < BV) L.v[j][col] = vv[e];
    }
    if (lane == 0) {
        L.beta[j] = b;
        L.kq[j] = kq;
    }
}

template <int DK, int DV, int BV, int TB, class TIn, bool VERIFY>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
    using C = Tile<DK, DV, BV>;
    __shared__ TokenLds<DK, BV, TB> L;
    __shared__ float4 red[2][kWaves][C::NC4][2];

    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int tile = blockIdx.x % C::NT;
    const int nh = blockIdx.x / C::NT;
    const int h = nh % a.H, n = nh / a.H;
    const int c4 = tid % C::NC4, rg = tid / C::NC4;
    const int col0 = tile * BV + 4 * c4;
    const int slot = a.slot_idx[n];

    if (slot < 0) {  // skipped sequence: zero outputs, no state access
        for (int idx = tid; idx < a.T * C::NC4; idx += kThreads) {
            const int t = idx / C::NC4, c = idx % C::NC4;
            const int64_t tok = (static_cast<int64_t>(n) * a.T + t) * a.H + h;
            store4<TIn>(a.o, tok * DV + tile * BV + 4 * c, make_float4(0.f, 0.f, 0.f, 0.f));
        }
        return;
    }
    float* S = a.pool + (static_cast<int64_t>(slot) * a.H + h) * (DK * DV);

    float4 s[C::RPT];
    for (int tb = 0; tb < a.T; tb += TB) {
        const int nb = min(TB, a.T - tb);
        for (int j = wave; j < nb; j += kWaves)
            prep_token<DK, DV, BV, TB, TIn, VERIFY>(a, L, j, n, tb + j, h, tile, lane);
        if (tb == 0) {
#pragma unroll
            for (int i = 0; i < C::RPT; ++i)
                s[i] = load_stream4(S + (rg + C::RG * i) * DV + col0);
        }
        __syncthreads();

        for (int j = 0; j < nb; ++j) {
            const int t = tb + j;
            const float4* a4 = reinterpret_cast<const float4*>(&L.a[j][rg * C::RPT]);
            const float4* k4 = reinterpret_cast<const float4*>(&L.k[j][rg * C::RPT]);
            const float4* q4 = reinterpret_cast<const float4*>(&L.q[j][rg * C::RPT]);
            float4 pk = make_float4(0.f, 0.f, 0.f, 0.f), pq = pk;
#pragma unroll
            for (int i4 = 0; i4 < C::RPT / 4; ++i4) {
                const float4 av = a4[i4], kv = k4[i4], qv = q4[i4];
                const float al[4] = {av.x, av.y, av.z, av.w};
                const float kk[4] = {kv.x, kv.y, kv.z, kv.w};
                const float qq[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float4& x = s[4 * i4 + r];
                    x = f4_mul(x, al[r]);            // decay
                    pk = f4_scale_fma(kk[r], x, pk);  // S'^T k
                    pq = f4_scale_fma(qq[r], x, pq);  // S'^T q
                }
            }
#pragma unroll
            for (int m = C::NC4; m < kWave; m <<= 1) {
                pk = f4_add(pk, f4_shfl_xor(pk, m));
                pq = f4_add(pq, f4_shfl_xor(pq, m));
            }
            const int buf = t & 1;
            if (lane < C::NC4) {
                red[buf][wave][c4][0] = pk;
                red[buf][wave][c4][1] = pq;
            }
            __syncthreads();
            pk = red[buf][0][c4][0];
            pq = red[buf][0][c4][1];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) {
                pk = f4_add(pk, red[buf][w][c4][0]);
                pq = f4_add(pq, red[buf][w][c4][1]);
            }
            const float4 vv = *reinterpret_cast<const float4*>(&L.v[j][4 * c4]);
            const float b = L.beta[j], kq = L.kq[j];
            const float4 u = f4_mul(f4_sub(vv, pk), b);                 // beta * delta
            const float4 ov = f4_mul(f4_scale_fma(kq, u, pq), a.scale);  // scale S^T q
#pragma unroll
            for (int i4 = 0; i4 < C::RPT / 4; ++i4) {
                const float4 kv = k4[i4];
                const float kk[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
                for (int r = 0; r < 4; ++r) s[4 * i4 + r] = f4_scale_fma(kk[r], u, s[4 * i4 + r]);
            }
            if (tid < C::NC4) {
                const int64_t tok = (static_cast<int64_t>(n) * a.T + t) * a.H + h;
                store4<TIn>(a.o, tok * DV + col0, ov);
                if (VERIFY)
                    *reinterpret_cast<float4*>(a.records + tok * (2 * DK + DV) + 2 * DK + col0) = u;
            }
        }
        if (tb + TB < a.T) __syncthreads();  // LDS token block is reused
    }
    if (!VERIFY) {
#pragma unroll
        for (int i = 0; i < C::RPT; ++i) store_stream4(S + (rg + C::RG * i) * DV + col0, s[i]);
    }
}

// ReplaySSM commit: S <- diag(alpha) S + kh u^T for the accepted records, with the
// same fp32 operation order as the decode kernel's decay and update.
template <int DK, int DV, int BV, int TB>
__global__ __launch_bounds__(kThreads) void replay_kernel(ReplayArgs a) {
    using C = Tile<DK, DV, BV>;
    __shared__ float Lk[TB][DK];
    __shared__ float La[TB][DK];
    __shared__ float Lu[TB][BV];

    const int tid = threadIdx.x;
    const int tile = blockIdx.x % C::NT;
    const int nh = blockIdx.x / C::NT;
    const int h = nh % a.H, n = nh / a.H;
    const int c4 = tid % C::NC4, rg = tid / C::NC4;
    const int col0 = tile * BV + 4 * c4;
    const int slot = a.slot_idx[n];
    const int acc = min(a.accepted[n], a.T);
    if (slot < 0 || acc <= 0) return;
    float* S = a.pool + (static_cast<int64_t>(slot) * a.H + h) * (DK * DV);

    float4 s[C::RPT];
#pragma unroll
    for (int i = 0; i < C::RPT; ++i) s[i] = load_stream4(S + (rg + C::RG * i) * DV + col0);

    for (int tb = 0; tb < acc; tb += TB) {
        const int nb = min(TB, acc - tb);
        for (int idx = tid; idx < nb * (2 * DK + BV); idx += kThreads) {
            const int j = idx / (2 * DK + BV), e = idx % (2 * DK + BV);
            const int64_t tok = (static_cast<int64_t>(n) * a.T + tb + j) * a.H + h;
            const float* rec = a.records + tok * (2 * DK + DV);
            if (e < DK)
                Lk[j][C::pos(e)] = rec[e];
            else if (e < 2 * DK)
                La[j][C::pos(e - DK)] = rec[e];
            else
                Lu[j][e - 2 * DK] = rec[2 * DK + tile * BV + (e - 2 * DK)];
        }
        __syncthreads();
        for (int j = 0; j < nb; ++j) {
            const float4* a4 = reinterpret_cast<const float4*>(&La[j][rg * C::RPT]);
            const float4* k4 = reinterpret_cast<const float4*>(&Lk[j][rg * C::RPT]);
            const float4 u = *reinterpret_cast<const float4*>(&Lu[j][4 * c4]);
#pragma unroll
            for (int i4 = 0; i4 < C::RPT / 4; ++i4) {
                const float4 av = a4[i4], kv = k4[i4];
                const float al[4] = {av.x, av.y, av.z, av.w};
                const float kk[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float4& x = s[4 * i4 + r];
                    x = f4_scale_fma(kk[r], u, f4_mul(x, al[r]));
                }
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < C::RPT; ++i) store_stream4(S + (rg + C::RG * i) * DV + col0, s[i]);
}

template <int DK, int DV, int BV, int TB, class TIn>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
    using C = Tile<DK, DV, BV>;
    const dim3 grid(static_cast<unsigned>(a.N) * a.H * C::NT), block(kThreads);
    if (a.records)
        hipLaunchKernelGGL((decode_kernel<DK, DV, BV, TB, TIn, true>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((decode_kernel<DK, DV, BV, TB, TIn, false>), grid, block, 0, stream, a);
    return hipGetLastError();
}

// dv tiles of 64 columns: twice the workgroups of whole-head tiles with half the
// registers each, measured faster on MI355X for a 64 x 32 x 128 x 128 pool step.  The
// tile shape fixes the order of the dk reductions, so every T uses the same one: the u a
// verify call records is then bit-identical to the u a commit call computes, and replaying
// records reproduces a commit exactly.
template <int DK, int DV, class TIn>
hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t stream) {
    constexpr int BV = DV < 64 ? DV : 64;
    if (a.T == 1) return launch_decode_t<DK, DV, BV, 1, TIn>(a, stream);
    return launch_decode_t<DK, DV, BV, 8, TIn>(a, stream);
}

template <class TIn>
hipError_t launch_decode_dt(const DecodeArgs& a, int dk, int dv, hipStream_t stream) {
    if (dk == 128 && dv == 128) return launch_decode_d<128, 128, TIn>(a, stream);
    if (dk == 128 && dv == 64) return launch_decode_d<128, 64, TIn>(a, stream);
    if (dk == 64 && dv == 128) return launch_decode_d<64, 128, TIn>(a, stream);
    if (dk == 64 && dv == 64) return launch_decode_d<64, 64, TIn>(a, stream);
    return hipErrorInvalidValue;
}

// Replay has no reductions (elementwise fma per state entry), so its tile shape does not
// affect the result; whole-head tiles measured faster.
template <int DK, int DV>
hipError_t launch_replay_d(const ReplayArgs& a, hipStream_t stream) {
    constexpr int BV = DV;
    using C = Tile<DK, DV, BV>;
    const dim3 grid(static_cast<unsigned>(a.N) * a.H * C::NT), block(kThreads);
    hipLaunchKernelGGL((replay_kernel<DK, DV, BV, 8>), grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int bf16, int dk, int dv, hipStream_t stream) {
    return bf16 ? launch_decode_dt<BF16>(a, dk, dv, stream)
                : launch_decode_dt<F32>(a, dk, dv, stream);
}

hipError_t launch_replay(const ReplayArgs& a, int dk, int dv, hipStream_t stream) {
    if (dk == 128 && dv == 128) return launch_replay_d<128, 128>(a, stream);
    if (dk == 128 && dv == 64) return launch_replay_d<128, 64>(a, stream);
    if (dk == 64 && dv == 128) return launch_replay_d<64, 128>(a, stream);
    if (dk == 64 && dv == 64) return launch_replay_d<64, 64>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace kda
