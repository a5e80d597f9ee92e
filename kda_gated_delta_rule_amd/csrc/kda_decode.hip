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
//  * The fp32 state tile (dk x BV, BV = 64 columns) of a (sequence, head, dv tile) is
//    streamed once from HBM into VGPRs with 16-byte non-temporal loads (each wave load
//    instruction covers whole 256-byte tile rows), kept there for all T tokens, and
//    written back once with non-temporal stores.  The step is about 0.9 flop per byte,
//    so nothing goes through MFMA.
//  * Both reductions over dk (S'^T k and S'^T q) come from one pass over the decayed
//    state, using o = scale * (S'^T q + (k.q) u): the output needs no second pass.
//  * The rows of a tile form 16 row groups (group g = rows g, g + 16, ...), group 4w + rq
//    at lane position rq (0..3) of slice w (0..3).  Each group's sum runs down its rows
//    in order; the four groups of a lane position are added in order w = 0..3; the four
//    lane positions are then combined pairwise ((r0 + r1) + (r2 + r3)) with the gfx950
//    row-swap instructions (v_permlane16_swap, v_permlane32_swap).  Both kernels below
//    follow exactly this order, so the u a verify call records is bit-identical to the u
//    a commit computes, and replaying records reproduces a commit exactly.
//  * T = 1 (decode_kernel, HBM-bound): 256 threads (4 waves) per tile; thread (w, rq, c4)
//    owns columns 4 c4 .. 4 c4 + 3 of row group 4w + rq; the slices meet through one LDS
//    exchange (one barrier per token).  Per-token vectors (qh, kh, alpha, v, beta, k.q)
//    are prepared by one wave per token into LDS, row-permuted for 16-byte LDS loads.
//  * T > 1 (decode_multi_kernel, MTP / verify): the token steps are VALU-bound (fp32 at
//    one wave64 instruction per 4 cycles), so one wave holds the whole tile (128
//    registers) and lane (rq, c4) owns columns 4 c4 .. 4 c4 + 3 of row groups 4w + rq
//    for all w: no LDS exchange and no barrier per token, and the 2,048-tile
//    verify workload fits the GPU in one round (two waves per SIMD).  The state loads
//    go out first; token inputs are loaded two tokens at a time while they stream.
//  * Replay: 256-thread workgroups per (sequence, head), elementwise (no reductions).
#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr float kNormEps = 1e-6f;
constexpr int kBufFlags = 0x00020000;  // raw buffer resource word 3 (gfx9 family)
constexpr int kNonTemporal = 2;        // buffer access cache policy: streaming (nt)

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// State tile accesses through a buffer resource: one VGPR offset per lane for the whole
// tile, the row offsets (compile-time constants) in the scalar offset field.
__device__ __forceinline__ float4 state_load4(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kNonTemporal);
    return make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]), __uint_as_float(v[3]));
}
__device__ __forceinline__ void state_store4(__amdgpu_buffer_rsrc_t r, int voff, int soff, float4 x) {
    const u32x4_t v = {__float_as_uint(x.x), __float_as_uint(x.y), __float_as_uint(x.z), __float_as_uint(x.w)};
    __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, soff, kNonTemporal);
}

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

// x + (x of the lane 16 apart in the other row of the pair): v_permlane16_swap exchanges
// rows 1 and 3 of one copy with rows 0 and 2 of the other, so the two results hold
// both rows of each pair and their sum is the pair sum in every lane.
__device__ __forceinline__ float pair_sum16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Likewise across the two 32-lane halves (v_permlane32_swap).
__device__ __forceinline__ float pair_sum32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float4 quad_sum(float4 x) {
    x = make_float4(pair_sum16(x.x), pair_sum16(x.y), pair_sum16(x.z), pair_sum16(x.w));
    return make_float4(pair_sum32(x.x), pair_sum32(x.y), pair_sum32(x.z), pair_sum32(x.w));
}

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
__global__ __launch_bounds__(kThreads, 5) void decode_kernel(DecodeArgs a) {
    using C = Tile<DK, DV, BV>;
    __shared__ TokenLds<DK, BV, TB> L;
    __shared__ float4 red[2][kWaves][kWave][2];

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
            // row groups 4w + rq of this lane position, in order w = 0..3, then its four
            // lane positions rq pairwise
            const int buf = t & 1;
            red[buf][wave][lane][0] = pk;
            red[buf][wave][lane][1] = pq;
            __syncthreads();
            pk = red[buf][0][lane][0];
            pq = red[buf][0][lane][1];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) {
                pk = f4_add(pk, red[buf][w][lane][0]);
                pq = f4_add(pq, red[buf][w][lane][1]);
            }
            pk = quad_sum(pk);
            pq = quad_sum(pq);
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

// Tile of decode_multi_kernel (one wave): see the file header for the lane mapping.
template <int DK, int DV, int BV>
struct DecTile {
    static constexpr int NC4 = BV / 4;                    // float4 column groups
    static constexpr int RQ = kWave / NC4;                // lanes per column group
    static constexpr int NRG = 16;                        // row groups of the dk reductions
    static constexpr int NW = NRG / RQ;                   // row groups per lane
    static constexpr int RPT = DK / NRG;                  // rows per row group
    static constexpr int NT = DV / BV;                    // tiles per head
    static constexpr int EPL = DK / kWave;                // key channels per lane in the prep
    static constexpr int VPL = (BV + kWave - 1) / kWave;  // v columns per lane in the prep
    static_assert(NC4 == 16 && RQ == 4 && RPT % 4 == 0 && DV % BV == 0, "decode tile");
    static_assert(EPL >= 1, "dk is 64 or 128");
    // LDS slot of key channel c: the rows of one row group are contiguous.
    __device__ static constexpr int pos(int c) { return (c % NRG) * RPT + c / NRG; }
};


// One token's inputs as this lane loads them (key channels EPL lane .. EPL lane + EPL - 1,
// v column lane of the tile).
template <int DK, int DV, int BV>
struct PrepIn {
    float q[DecTile<DK, DV, BV>::EPL], k[DecTile<DK, DV, BV>::EPL], g[DecTile<DK, DV, BV>::EPL];
    float v[DecTile<DK, DV, BV>::VPL];
    float b;
};

template <int DK, int DV, int BV, class TIn>
__device__ __forceinline__ PrepIn<DK, DV, BV> prep_load(const DecodeArgs& a, int n, int t, int h, int tile,
                                                        int lane) {
    using C = DecTile<DK, DV, BV>;
    PrepIn<DK, DV, BV> x;
    const int64_t tok = (static_cast<int64_t>(n) * a.T + t) * a.H + h;
    const int64_t rowk = tok * DK;
    if constexpr (C::EPL == 2) {
        const int c = lane * 2;
        const float2 qq = load2<TIn>(a.q, rowk + c);
        const float2 kk = load2<TIn>(a.k, rowk + c);
        const float2 gg = *reinterpret_cast<const float2*>(a.g + rowk + c);
        x.q[0] = qq.x; x.q[1] = qq.y;
        x.k[0] = kk.x; x.k[1] = kk.y;
        x.g[0] = gg.x; x.g[1] = gg.y;
    } else {
        x.q[0] = load1<TIn>(a.q, rowk + lane);
        x.k[0] = load1<TIn>(a.k, rowk + lane);
        x.g[0] = a.g[rowk + lane];
    }
#pragma unroll
    for (int e = 0; e < C::VPL; ++e) {
        const int col = lane + e * kWave;
        x.v[e] = col < BV ? load1<TIn>(a.v, tok * DV + tile * BV + col) : 0.f;
    }
    x.b = a.beta[tok];
    return x;
}

// Token t (local slot j): L2 norms, alpha = exp(g), k.q into LDS (and the k, alpha
// records of a verify call, written by tile 0).
template <int DK, int DV, int BV, int TB, bool VERIFY>
__device__ __forceinline__ void prep_store(const DecodeArgs& a, TokenLds<DK, BV, TB>& L, int j, int n, int t,
                                           int h, int tile, int lane, const PrepIn<DK, DV, BV>& x) {
    using C = DecTile<DK, DV, BV>;
    const int64_t tok = (static_cast<int64_t>(n) * a.T + t) * a.H + h;
    float iq = 1.f, ik = 1.f;
    if (a.use_l2) {
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int e = 0; e < C::EPL; ++e) {
            sq = fmaf(x.q[e], x.q[e], sq);
            sk = fmaf(x.k[e], x.k[e], sk);
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
        const float qh = x.q[e] * iq, kh = x.k[e] * ik, al = expf(x.g[e]);
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
        if (col < BV) L.v[j][col] = x.v[e];
    }
    if (lane == 0) {
        L.beta[j] = x.b;
        L.kq[j] = kq;
    }
}

// Orders this wave's LDS accesses in the compiler's schedule (the hardware completes one
// wave's LDS operations in issue order, so a single-wave workgroup needs no s_barrier).
__device__ __forceinline__ void wave_lds_order() {
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
}

template <int DK, int DV, int BV, int TB, class TIn, bool VERIFY>
__global__ __launch_bounds__(kWave, 2) void decode_multi_kernel(DecodeArgs a) {
    using C = DecTile<DK, DV, BV>;
    __shared__ TokenLds<DK, BV, TB> L;

    const int lane = threadIdx.x;
    const int tile = blockIdx.x % C::NT;
    const int nh = blockIdx.x / C::NT;
    const int h = nh % a.H, n = nh / a.H;
    const int c4 = lane % C::NC4, rq = lane / C::NC4;
    const int col0 = tile * BV + 4 * c4;
    const int slot = a.slot_idx[n];

    if (slot < 0) {  // skipped sequence: zero outputs, no state access
        for (int idx = lane; idx < a.T * C::NC4; idx += kWave) {
            const int t = idx / C::NC4, c = idx % C::NC4;
            const int64_t tok = (static_cast<int64_t>(n) * a.T + t) * a.H + h;
            store4<TIn>(a.o, tok * DV + tile * BV + 4 * c, make_float4(0.f, 0.f, 0.f, 0.f));
        }
        return;
    }
    float* S = a.pool + (static_cast<int64_t>(slot) * a.H + h) * (DK * DV);
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(S, 0, DK * DV * 4, kBufFlags);
    const int voff = (rq * DV + col0) * 4;

    // The state tile's loads go out first and stream while the tokens are prepared, PG
    // tokens at a time (their input loads all issued before any is used).
    constexpr int PG = TB < 2 ? TB : 2;  // tokens whose input loads are in flight together
    auto prep_block = [&](int tb, int nb) {
        for (int j0 = 0; j0 < nb; j0 += PG) {
            PrepIn<DK, DV, BV> pin[PG];
#pragma unroll
            for (int j = 0; j < PG; ++j)
                if (j0 + j < nb) pin[j] = prep_load<DK, DV, BV, TIn>(a, n, tb + j0 + j, h, tile, lane);
#pragma unroll
            for (int j = 0; j < PG; ++j)
                if (j0 + j < nb) prep_store<DK, DV, BV, TB, VERIFY>(a, L, j0 + j, n, tb + j0 + j, h, tile, lane, pin[j]);
        }
    };
    float4 s[C::NW][C::RPT];
    auto load_state = [&]() {
#pragma unroll
        for (int w = 0; w < C::NW; ++w)
#pragma unroll
            for (int i = 0; i < C::RPT; ++i) s[w][i] = state_load4(srs, voff, (4 * w + C::NRG * i) * DV * 4);
    };
    load_state();

    for (int tb = 0; tb < a.T; tb += TB) {
        const int nb = min(TB, a.T - tb);
        prep_block(tb, nb);
        wave_lds_order();

        for (int j = 0; j < nb; ++j) {
            const int t = tb + j;
            float4 tk, tq;
#pragma unroll
            for (int w = 0; w < C::NW; ++w) {
                const int g0 = (4 * w + rq) * C::RPT;
                const float4* a4 = reinterpret_cast<const float4*>(&L.a[j][g0]);
                const float4* k4 = reinterpret_cast<const float4*>(&L.k[j][g0]);
                const float4* q4 = reinterpret_cast<const float4*>(&L.q[j][g0]);
                float4 pk = make_float4(0.f, 0.f, 0.f, 0.f), pq = pk;
#pragma unroll
                for (int i4 = 0; i4 < C::RPT / 4; ++i4) {
                    const float4 av = a4[i4], kv = k4[i4], qv = q4[i4];
                    const float al[4] = {av.x, av.y, av.z, av.w};
                    const float kk[4] = {kv.x, kv.y, kv.z, kv.w};
                    const float qq[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float4& x = s[w][4 * i4 + r];
                        x = f4_mul(x, al[r]);            // decay
                        pk = f4_scale_fma(kk[r], x, pk);  // S'^T k
                        pq = f4_scale_fma(qq[r], x, pq);  // S'^T q
                    }
                }
                // row groups 4w + rq in order w = 0..3
                if (w == 0) {
                    tk = pk;
                    tq = pq;
                } else {
                    tk = f4_add(tk, pk);
                    tq = f4_add(tq, pq);
                }
            }
            tk = quad_sum(tk);  // then the four lane positions rq pairwise
            tq = quad_sum(tq);
            const float4 vv = *reinterpret_cast<const float4*>(&L.v[j][4 * c4]);
            const float b = L.beta[j], kq = L.kq[j];
            const float4 u = f4_mul(f4_sub(vv, tk), b);                 // beta * delta
            const float4 ov = f4_mul(f4_scale_fma(kq, u, tq), a.scale);  // scale S^T q
#pragma unroll
            for (int w = 0; w < C::NW; ++w) {
                const float4* k4 = reinterpret_cast<const float4*>(&L.k[j][(4 * w + rq) * C::RPT]);
#pragma unroll
                for (int i4 = 0; i4 < C::RPT / 4; ++i4) {
                    const float4 kv = k4[i4];
                    const float kk[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
                    for (int r = 0; r < 4; ++r) s[w][4 * i4 + r] = f4_scale_fma(kk[r], u, s[w][4 * i4 + r]);
                }
            }
            if (rq == 0) {
                const int64_t tok = (static_cast<int64_t>(n) * a.T + t) * a.H + h;
                store4<TIn>(a.o, tok * DV + col0, ov);
                if (VERIFY)
                    *reinterpret_cast<float4*>(a.records + tok * (2 * DK + DV) + 2 * DK + col0) = u;
            }
        }
        if (tb + TB < a.T) wave_lds_order();  // the next block's vectors overwrite L
    }
    if (!VERIFY) {
#pragma unroll
        for (int w = 0; w < C::NW; ++w)
#pragma unroll
            for (int i = 0; i < C::RPT; ++i) state_store4(srs, voff, (4 * w + C::NRG * i) * DV * 4, s[w][i]);
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

// T = 1: four-wave workgroups (HBM-bound); T > 1: one wave per tile (the token steps
// are VALU-bound, and a wave-local reduction needs no barrier).  Both reduce over dk in the
// same order, so their results are bit-identical.
template <int DK, int DV, int BV, int TB, class TIn>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(a.N) * a.H * (DV / BV));
    if constexpr (TB == 1) {
        if (a.records)
            hipLaunchKernelGGL((decode_kernel<DK, DV, BV, TB, TIn, true>), grid, dim3(kThreads), 0, stream, a);
        else
            hipLaunchKernelGGL((decode_kernel<DK, DV, BV, TB, TIn, false>), grid, dim3(kThreads), 0, stream, a);
    } else {
        if (a.records)
            hipLaunchKernelGGL((decode_multi_kernel<DK, DV, BV, TB, TIn, true>), grid, dim3(kWave), 0, stream, a);
        else
            hipLaunchKernelGGL((decode_multi_kernel<DK, DV, BV, TB, TIn, false>), grid, dim3(kWave), 0, stream, a);
    }
    return hipGetLastError();
}

// dv tiles of 64 columns, one wave each.  The tile fixes the order of the dk reductions, so
// every T uses the same one: the u a verify call records is then bit-identical to the u a
// commit call computes, and replaying records reproduces a commit exactly.
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
