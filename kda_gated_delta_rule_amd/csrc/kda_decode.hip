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
//  * The fp32 state tile (dk x BV) of a (sequence, head, dv tile) is streamed once from HBM
//    into VGPRs with 16-byte non-temporal loads (each wave load instruction covers whole
//    tile rows), kept there for all T tokens, and written back once with non-temporal
//    stores.  A one-token step is about 0.9 flop
//    per byte and runs on the VALU; only the multi-token blocks use MFMA.
//  * T = 1 (decode_kernel, HBM-bound): both reductions over dk (S'^T k and S'^T q) come
//    from one pass over the decayed state, using o = scale * (S'^T q + (k.q) u): the
//    output needs no second pass.  One workgroup per (sequence, head) holds the whole head:
//    at dv = 128, 512 threads (8 waves), thread (w, rq, c4) owning columns 4 c4 .. 4 c4 + 3
//    of row group 2w + rq (group g = rows g, g + 16, ...), so each wave instruction covers
//    two whole 512-byte rows (a bare memory pass measured 5.6% faster in this shape than
//    with 64-column tiles of 4 waves); at dv = 64, 256 threads and four lane positions per
//    column quad.  Each group's sum runs down its rows, the waves' sums meet through one LDS
//    exchange (one barrier per token), and the lane positions of a column quad are combined
//    pairwise with the gfx950 row-swap instructions (v_permlane16_swap, v_permlane32_swap).
//    Per-token vectors (qh, kh, alpha, v, beta, k.q) are prepared by one wave per token
//    into LDS.
//  * T > 1 (wy_multi_kernel, MTP / verify): the WY form of 8-token blocks (see the
//    kernel), one workgroup per head with a wave per 64-column tile (the waves split the
//    block's preparation): one fp32 MFMA pass over the register-resident tile gives the 16 products
//    with the entering state, a per-column 8x8 triangular solve gives u and o, and the
//    state is updated only when it is kept (commit, or between blocks) -- with the
//    replay kernel's fp32 operations, so replaying verify records reproduces a commit of
//    two or more tokens exactly.
//  * Replay: one workgroup per (sequence, head) (512 threads at dv = 128), elementwise (no
//    reductions).
#include "kda_device.hpp"
#include "kda_internal.hpp"

#include <type_traits>

namespace kda {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kFrontTB = 8;  // with the input front: at most 8 tokens, prepared as one block
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

template <int DK, int DV, int BV, int NTHR = kThreads>
struct Tile {
    static constexpr int NC4 = BV / 4;          // float4 column groups per tile
    static constexpr int RG = NTHR / NC4;       // row groups
    static constexpr int RPT = DK / RG;         // rows per thread
    static constexpr int NT = DV / BV;          // tiles per head
    static constexpr int EPL = DK / kWave;      // key channels per lane in the prep
    static constexpr int VPL = (BV + kWave - 1) / kWave;  // v columns per lane in the prep
    static_assert(NTHR % NC4 == 0 && DK % RG == 0 && RPT % 4 == 0, "tile shape");
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
// Sum over the lane positions of a wave that hold the same column quad: 4 (lanes 16 apart)
// for 16 column quads per tile, 2 (lanes 32 apart) for 32.
template <int NC4>
__device__ __forceinline__ float4 lane_pos_sum(float4 x) {
    if constexpr (NC4 == 16) {
        return quad_sum(x);
    } else {
        static_assert(NC4 == 32, "16 or 32 column quads per tile");
        return make_float4(pair_sum32(x.x), pair_sum32(x.y), pair_sum32(x.z), pair_sum32(x.w));
    }
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

// Prepares token t (local slot j) by one wave: L2 norms, alpha = exp(g), k.q.  With the
// input front (FRONT), q, k and v are first convolved along the tokens (the inputs before
// the call come from the slot's convolution state), g = -a_h softplus(z), beta = sigmoid(b).
template <int DK, int DV, int BV, int TB, class TIn, bool VERIFY, bool FRONT, int NTHR>
__device__ __forceinline__ void prep_token(const DecodeArgs& a, TokenLds<DK, BV, TB>& L, int j,
                                           int n, int t, int h, int tile, int lane, int slot) {
    using C = Tile<DK, DV, BV, NTHR>;
    const int64_t tok = (static_cast<int64_t>(n) * a.T + t) * a.H + h;
    const int64_t rowk = tok * DK;
    float qv[C::EPL], kv[C::EPL], gv[C::EPL];
    float vv[C::VPL];
    float b;
    if constexpr (FRONT) {
        const FrontArgs& f = a.front;
        const int W = f.conv_width;
        constexpr int CW = 2 * DK + DV;
        // channel c of input u of the call (u >= 0), or of row u + W - 1 of the state: the
        // source and index are selected, so each tap is one load
        auto raw = [&](const void* x, int D, int off, int u, int c) -> float {
            const bool in = u >= 0;
            const int64_t idx = in ? ((static_cast<int64_t>(n) * a.T + u) * a.H + h) * D + c
                                   : ((static_cast<int64_t>(slot) * a.H + h) * (W - 1) + u + W - 1) * CW + off + c;
            return load1<TIn>(in ? x : f.conv_state, idx);
        };
        // unrolled to the largest width with every tap's loads unconditional (taps past the
        // width re-read the last one and are not added), so they are all in flight together
        auto conv = [&](const void* x, const float* w, int D, int off, int c) -> float {
            const float* wc = w + (static_cast<int64_t>(h) * D + c) * W;
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ii = i < W ? i : W - 1;
                const float xv = raw(x, D, off, t - (W - 1) + ii, c), wv = wc[ii];
                acc = i < W ? fmaf(wv, xv, acc) : acc;
            }
            return f.conv_silu ? front_silu(acc) : acc;
        };
        const float gs = f.gate_scale[h];
#pragma unroll
        for (int e = 0; e < C::EPL; ++e) {
            const int c = lane * C::EPL + e;
            qv[e] = conv(a.q, f.conv_q, DK, 0, c);
            kv[e] = conv(a.k, f.conv_k, DK, DK, c);
            gv[e] = -gs * front_softplus(a.g[rowk + c]);
        }
#pragma unroll
        for (int e = 0; e < C::VPL; ++e) {
            const int col = lane + e * kWave;
            vv[e] = col < BV ? conv(a.v, f.conv_v, DV, 2 * DK, tile * BV + col) : 0.f;
        }
        b = front_sigmoid(a.beta[tok]);
    } else if constexpr (C::EPL == 2) {
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
    if constexpr (!FRONT) {
#pragma unroll
        for (int e = 0; e < C::VPL; ++e) {
            const int col = lane + e * kWave;
            vv[e] = 0.f;
            if (col < BV) {
                const int64_t idx = tok * DV + tile * BV + col;
                vv[e] = load1<TIn>(a.v, idx);
            }
        }
        b = a.beta[tok];
    }

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

template <int DK, int DV, int BV, int TB, class TIn, bool VERIFY, bool FRONT = false, int NTHR = kThreads>
__global__ __launch_bounds__(NTHR, FRONT ? 4 : 5 * kThreads / NTHR) void decode_kernel(DecodeArgs a) {
    using C = Tile<DK, DV, BV, NTHR>;
    constexpr int NW = NTHR / kWave;
    __shared__ __attribute__((aligned(16))) TokenLds<DK, BV, TB> L;  // read as float4
    __shared__ float4 red[2][NW][kWave][2];

    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int tile = blockIdx.x % C::NT;
    const int nh = blockIdx.x / C::NT;
    const int h = nh % a.H, n = nh / a.H;
    const int c4 = tid % C::NC4, rg = tid / C::NC4;
    const int col0 = tile * BV + 4 * c4;
    const int slot = a.slot_idx[n];

    if (slot < 0) {  // skipped sequence: zero outputs, no state access
        for (int idx = tid; idx < a.T * C::NC4; idx += NTHR) {
            const int t = idx / C::NC4, c = idx % C::NC4;
            const int64_t tok = (static_cast<int64_t>(n) * a.T + t) * a.H + h;
            store4<TIn>(a.o, tok * DV + tile * BV + 4 * c, make_float4(0.f, 0.f, 0.f, 0.f));
        }
        return;
    }
    float* S = a.pool + (static_cast<int64_t>(slot) * a.H + h) * (DK * DV);

    float4 s[C::RPT];
    // With the front (T <= TB) the tokens form one block: every token is prepared before the
    // (whole-head) state tile is loaded, so the preparation's temporaries and the tile are
    // never live together.
    for (int tb = 0; tb < (FRONT ? 1 : a.T); tb += TB) {
        const int nb = min(TB, a.T - tb);
        for (int j = wave; j < nb; j += NW)
            prep_token<DK, DV, BV, TB, TIn, VERIFY, FRONT, NTHR>(a, L, j, n, tb + j, h, tile, lane, slot);
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
            for (int w = 1; w < NW; ++w) {
                pk = f4_add(pk, red[buf][w][lane][0]);
                pq = f4_add(pq, red[buf][w][lane][1]);
            }
            pk = lane_pos_sum<C::NC4>(pk);
            pq = lane_pos_sum<C::NC4>(pq);
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
    if constexpr (FRONT) {
        // the convolution state after the call: its last W - 1 inputs, earlier state rows
        // where the call has fewer tokens.  The workgroup owns the whole head (one tile), so
        // its prep reads of the state (done before the first barrier) precede these writes.
        const FrontArgs& f = a.front;
        const int W = f.conv_width;
        if (W > 1) {
            static_assert(C::NT == 1, "the front runs one workgroup per head");
            constexpr int CW = 2 * DK + DV, NV = (3 * CW + NTHR - 1) / NTHR;
            const int nv = (W - 1) * CW;
            const int64_t st0 = (static_cast<int64_t>(slot) * a.H + h) * (W - 1) * CW;
            float keep[NV];
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const int idx = tid + i * NTHR;
                keep[i] = 0.f;
                if (idx < nv) {
                    const int r = idx / CW, c = idx % CW, u = a.T - (W - 1) + r;
                    const int64_t tk = (static_cast<int64_t>(n) * a.T + u) * a.H + h;
                    keep[i] = u < 0 ? load1<TIn>(f.conv_state, st0 + static_cast<int64_t>(u + W - 1) * CW + c)
                              : c < DK ? load1<TIn>(a.q, tk * DK + c)
                              : c < 2 * DK ? load1<TIn>(a.k, tk * DK + c - DK)
                              : load1<TIn>(a.v, tk * DV + c - 2 * DK);
                }
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const int idx = tid + i * NTHR;
                if (idx < nv) store1<TIn>(f.conv_state, st0 + idx, keep[i]);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// T > 1 (MTP, verify): the WY form of a block of up to 8 tokens on one state tile.  For
// the tokens t of a block entering with state S0, G_t = g_1 + ... + g_t per key channel:
//   S'_t^T kh_t = S0^T (kh_t e^{G_t}) + sum_{s<t} (kh_s . e^{G_t - G_s} kh_t) u_s
// so with R = S0^T [kh_t e^{G_t} | qh_t e^{G_t}] (16 vectors of dk, one fp32 MFMA pass
// over the tile) and, per column,
//   u_t = beta_t (v_t - RK_t - sum_{s<t} kk_ts u_s),  kk_ts = sum_c kh_tc kh_sc e^{G_tc - G_sc}
//   o_t = scale (RQ_t + sum_{s<=t} qk_ts u_s),        qk_ts = sum_c qh_tc kh_sc e^{G_tc - G_sc}
// (the token recurrence rearranged, exact in exact arithmetic).  A verify call never
// writes the pool.  A commit, and any call of more than 8 tokens between its blocks (on the
// register copy), applies S <- diag(alpha_t) S + kh_t u_t^T in token order with the replay
// kernel's fp32 operations, so replaying a verify call's records gives, bit for bit, the
// state a commit of the same two or more tokens gives.
//
// A wave per (sequence, head, 64-column tile).  The state tile is loaded with 16-byte
// loads, lane l holding rows 4 s + l / 16 (s = 0 .. dk/4 - 1), columns 4 (l % 16) .. + 3:
// component e of the k-step-s register is exactly the A operand of a 16x16x4 fp32 MFMA
// (row m = l % 16 <-> tile column 4 m + e, k = l / 16), so the product needs no
// re-layout.  The 64 dot products kk and qk of a block are reduced over the wave with a
// shuffle reduce-scatter (lane l ends with value l).
// ---------------------------------------------------------------------------
constexpr int kWyTB = 8;  // tokens per block
constexpr int kWyRt = 20; // R^T row stride (floats): 16 vectors, rows 16-byte aligned
constexpr float kLog2e = 1.4426950408889634f;

// LDS of one head: the block's operands (shared by the head's waves) and each wave's R^T and
// u areas.
template <int DK, int NW>
struct WyLds {
    static constexpr int KS = DK / 4;  // fp32 MFMA k-steps over dk
    struct Wave {
        float rt[64][kWyRt];           // R^T: tile column j, vector n
        float ut[kWyTB][64];           // v, then u, of the tile's columns
    };
    float xp[16][4][KS];               // X[4 s + q][n] at [n][q][s]: n < 8 kh_n e^G_n, n >= 8 qh e^G
    float kr[kWyTB][4][KS];            // kh_t of row 4 s + q at [t][q][s]
    float ar[kWyTB][4][KS];            // alpha_t likewise
    float pq[64];                      // dot products of the raw q and k (index: see wy_pair)
    float nf[2 * kWyTB];               // norm factors: 1/|q_t| at t, 1/|k_t| at 8 + t
    Wave w[NW];
};

// Dot-product index of the pair (a, b), a > b: kk_ab at wy_pair(a, b), qk_ab at 32 + that;
// the diagonal qk_aa at 28 + a (a < 4) and 56 + a (a >= 4).
__host__ __device__ constexpr int wy_pair(int a, int b) { return a * (a - 1) / 2 + b; }
__host__ __device__ constexpr int wy_diag(int a) { return a < 4 ? 28 + a : 56 + a; }

// Orders this wave's LDS accesses in the compiler's schedule (the hardware completes one
// wave's LDS operations in issue order, so a single-wave workgroup needs no s_barrier).
__device__ __forceinline__ void wave_lds_order() {
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
}

// One reduce-scatter step over lane bit M: 2N values per lane -> N, the lane keeping the
// upper half when its bit M is set.
template <int N, int M>
__device__ __forceinline__ void rs_step(const float (&v)[2 * N], float (&w)[N], int lane) {
    const bool hi = (lane & M) != 0;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const float keep = hi ? v[i + N] : v[i];
        const float send = hi ? v[i] : v[i + N];
        w[i] = keep + __shfl_xor(send, M, kWave);
    }
}

// One workgroup per (sequence, head): wave w holds the 64-column tile w.  The block's
// preparation is split between the waves: wave 0 forms the norms and the X, kh and alpha
// rows, wave 1 the 64 dot products of the raw q and k (scaled by the norms in the solve);
// with a single tile (dv = 64) one wave does both.
// ONEBLK: a verify call of at most 8 tokens (one block, no state update), where the state
// registers are free after the MFMA pass.
template <int DK, int DV, class TIn, bool VERIFY, bool ONEBLK>
__global__ __launch_bounds__(kWave * (DV / 64), 2) void wy_multi_kernel(DecodeArgs a) {
    constexpr int BV = 64, NW = DV / BV, EPL = DK / kWave;
    using LD = WyLds<DK, NW>;
    constexpr int KS = LD::KS;
    __shared__ __attribute__((aligned(16))) LD L;  // read as f32x4

    const int lane = threadIdx.x & (kWave - 1);
    const int tile = NW == 1 ? 0 : __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    const bool norm_role = NW == 1 || tile == 0, dot_role = NW == 1 || tile == 1;
    const int h = blockIdx.x % a.H, n = blockIdx.x / a.H;
    const int slot = a.slot_idx[n];
    const int64_t tok0 = static_cast<int64_t>(n) * a.T * a.H + h;  // token t: tok0 + t * H
    auto& Wv = L.w[tile];

    if (slot < 0) {  // skipped sequence (the whole workgroup): zero outputs, no state access
        for (int t = 0; t < a.T; ++t) store1<TIn>(a.o, (tok0 + static_cast<int64_t>(t) * a.H) * DV + tile * BV + lane, 0.f);
        return;
    }
    float* S = a.pool + (static_cast<int64_t>(slot) * a.H + h) * (DK * DV);
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(S, 0, DK * DV * 4, kBufFlags);
    const int lq = lane >> 4, lm = lane & 15;
    const int voff = (lq * DV + tile * BV + 4 * lm) * 4;
    // orders the head's LDS exchanges: a workgroup barrier with two waves, program order with one
    auto sync = [&]() {
        if constexpr (NW > 1) lds_barrier();
        else wave_lds_order();
    };

    float4 sv[KS];
    // one block of tokens; the first one (FIRST, a compile-time flag, so its loads stay in
    // straight-line code) also issues the state tile's loads
    auto block = [&](int tb, auto first) {
        constexpr bool FIRST = decltype(first)::value;
        const int nb = min(kWyTB, a.T - tb);
        // (1) token inputs of the block: lane l owns key channels EPL l .. EPL l + EPL - 1
        float kh[kWyTB][EPL], qh[kWyTB][EPL], G[kWyTB][EPL], vt[kWyTB], bt[kWyTB];
        // bf16 inputs arrive as raw words (a dword holds a lane's two channels) and are
        // widened only after the state loads are issued
        constexpr bool kBf = std::is_same<TIn, BF16>::value;
        uint32_t qw[kWyTB], kw[kWyTB], vw[kWyTB];
        // branch-free: tokens past the block's end load the last token's inputs (a valid
        // address) and are zeroed afterwards, so every load is in flight before the first wait
#pragma unroll
        for (int t = 0; t < kWyTB; ++t) {
            const int64_t tok = tok0 + static_cast<int64_t>(tb + min(t, nb - 1)) * a.H;
            const int64_t rowk = tok * DK + EPL * lane;
            const int64_t iv = tok * DV + tile * BV + lane;
            if constexpr (kBf) {
                const uint16_t* q16 = static_cast<const uint16_t*>(a.q);
                const uint16_t* k16 = static_cast<const uint16_t*>(a.k);
                if constexpr (EPL == 2) {
                    qw[t] = *reinterpret_cast<const uint32_t*>(q16 + rowk);
                    kw[t] = *reinterpret_cast<const uint32_t*>(k16 + rowk);
                } else {
                    qw[t] = q16[rowk];
                    kw[t] = k16[rowk];
                }
                vw[t] = static_cast<const uint16_t*>(a.v)[iv];
            } else {
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    qh[t][e] = static_cast<const float*>(a.q)[rowk + e];
                    kh[t][e] = static_cast<const float*>(a.k)[rowk + e];
                }
                vt[t] = static_cast<const float*>(a.v)[iv];
            }
#pragma unroll
            for (int e = 0; e < EPL; ++e) G[t][e] = a.g[rowk + e];
            bt[t] = a.beta[tok];
        }
        __builtin_amdgcn_sched_barrier(0);  // every load above is in flight before any use
        // the state tile's loads go out after the first block's token loads: loads complete
        // in issue order, so the token preparation below overlaps the tile's arrival
        if constexpr (FIRST) {
#pragma unroll
            for (int st = 0; st < KS; ++st) sv[st] = state_load4(srs, voff, 4 * st * DV * 4);
            // ... issued here, before the preparation: nothing is scheduled across this point
            // (widening the token words above the state loads would make them wait for the
            // token loads)
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (kBf) {
#pragma unroll
            for (int t = 0; t < kWyTB; ++t) {
                qh[t][0] = __uint_as_float(qw[t] << 16);
                kh[t][0] = __uint_as_float(kw[t] << 16);
                if constexpr (EPL == 2) {
                    qh[t][1] = __uint_as_float(qw[t] & 0xffff0000u);
                    kh[t][1] = __uint_as_float(kw[t] & 0xffff0000u);
                }
                vt[t] = __uint_as_float(vw[t] << 16);
            }
        }
        // tokens past the block's end become zeros; the gates go to log2 units and their
        // in-block cumsum; v waits in this wave's u slots until the solve
#pragma unroll
        for (int t = 0; t < kWyTB; ++t) {
            const bool live = t < nb;
            Wv.ut[t][lane] = live ? vt[t] : 0.f;
            bt[t] = live ? bt[t] : 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                const int c = EPL * lane + e;
                const float g2 = live ? G[t][e] * kLog2e : 0.f;
                if (norm_role) L.ar[t][c & 3][c >> 2] = __builtin_amdgcn_exp2f(g2);  // alpha
                G[t][e] = t == 0 ? g2 : G[t - 1][e] + g2;
                kh[t][e] = live ? kh[t][e] : 0.f;
                qh[t][e] = live ? qh[t][e] : 0.f;
            }
        }

        // (2a) the 64 dot products of the raw q and k: partial sums over this lane's channels,
        // values i and i + 32 together, then the reduce-scatter (lane l keeps value l)
        if (dot_role) {
            float r32[32];
            const bool up = (lane & 32) != 0;
            auto first_step = [&](int i, float lo, float hi) {
                const float keep = up ? hi : lo, send = up ? lo : hi;
                r32[i] = keep + __shfl_xor(send, 32, kWave);
            };
#pragma unroll
            for (int ta = 1; ta < kWyTB; ++ta)
#pragma unroll
                for (int sb = 0; sb < ta; ++sb) {
                    float kk = 0.f, qk = 0.f;
#pragma unroll
                    for (int e = 0; e < EPL; ++e) {
                        const float w = kh[sb][e] * __builtin_amdgcn_exp2f(G[ta][e] - G[sb][e]);
                        kk = fmaf(kh[ta][e], w, kk);
                        qk = fmaf(qh[ta][e], w, qk);
                    }
                    first_step(wy_pair(ta, sb), kk, qk);
                }
#pragma unroll
            for (int t = 0; t < 4; ++t) {  // the diagonal qk_tt (t < 4) and qk_{t+4, t+4}
                float d0 = 0.f, d1 = 0.f;
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    d0 = fmaf(qh[t][e], kh[t][e], d0);
                    d1 = fmaf(qh[t + 4][e], kh[t + 4][e], d1);
                }
                first_step(wy_diag(t), d0, d1);
            }
            float r16[16], r8[8], r4[4], r2[2], r1[1];
            rs_step<16, 16>(r32, r16, lane);
            rs_step<8, 8>(r16, r8, lane);
            rs_step<4, 4>(r8, r4, lane);
            rs_step<2, 2>(r4, r2, lane);
            rs_step<1, 1>(r2, r1, lane);
            L.pq[lane] = r1[0];
        }
        // (2b) the norms (16 sums of squares in one reduce-scatter: lane l ends with sum l >> 2),
        // then kh and X = [kh e^G | qh e^G] rows into LDS (alpha went there above)
        if (norm_role) {
            float nrm[2 * kWyTB];
#pragma unroll
            for (int t = 0; t < kWyTB; ++t) {
                float sq = 0.f, sk = 0.f;
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    sq = fmaf(qh[t][e], qh[t][e], sq);
                    sk = fmaf(kh[t][e], kh[t][e], sk);
                }
                nrm[t] = sq;
                nrm[kWyTB + t] = sk;
            }
            float n8[8], n4[4], n2[2], n1[1];
            rs_step<8, 32>(nrm, n8, lane);
            rs_step<4, 16>(n8, n4, lane);
            rs_step<2, 8>(n4, n2, lane);
            rs_step<1, 4>(n2, n1, lane);
            float tot = n1[0];
            tot += __shfl_xor(tot, 2, kWave);
            tot += __shfl_xor(tot, 1, kWave);
            const float f = a.use_l2 ? __builtin_amdgcn_rsqf(tot + kNormEps) : 1.f;
            if ((lane & 3) == 0) L.nf[lane >> 2] = f;
#pragma unroll
            for (int t = 0; t < kWyTB; ++t) {
                const float iq = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), 4 * t));
                const float ik = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), 4 * (kWyTB + t)));
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    const int c = EPL * lane + e;
                    const float k1 = kh[t][e] * ik, q1 = qh[t][e] * iq;
                    const float eg = __builtin_amdgcn_exp2f(G[t][e]);
                    L.xp[t][c & 3][c >> 2] = k1 * eg;
                    L.xp[8 + t][c & 3][c >> 2] = q1 * eg;
                    L.kr[t][c & 3][c >> 2] = k1;
                }
            }
        }
        sync();
        if (VERIFY && tile == 0) {  // the kh and alpha parts of the records, from LDS
#pragma unroll
            for (int t = 0; t < kWyTB; ++t) {
                if (t < nb) {
                    float* rec = a.records + (tok0 + static_cast<int64_t>(tb + t) * a.H) * (2 * DK + DV);
#pragma unroll
                    for (int e = 0; e < EPL; ++e) {
                        const int c = EPL * lane + e;
                        rec[c] = L.kr[t][c & 3][c >> 2];
                        rec[DK + c] = L.ar[t][c & 3][c >> 2];
                    }
                }
            }
        }

        // (3) R = S0^T X on fp32 MFMA: acc[e] holds R rows (tile columns) 16 lq + 4 i + e,
        // i = 0..3, of vector lm
        f32x4 acc[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < KS / 4; ++i) {
            const f32x4 bx = *reinterpret_cast<const f32x4*>(&L.xp[lm][lq][4 * i]);
#pragma unroll
            for (int k4 = 0; k4 < 4; ++k4) {
                const float4 x = sv[4 * i + k4];
                acc[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(x.x, bx[k4], acc[0], 0, 0, 0);
                acc[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(x.y, bx[k4], acc[1], 0, 0, 0);
                acc[2] = __builtin_amdgcn_mfma_f32_16x16x4f32(x.z, bx[k4], acc[2], 0, 0, 0);
                acc[3] = __builtin_amdgcn_mfma_f32_16x16x4f32(x.w, bx[k4], acc[3], 0, 0, 0);
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int i = 0; i < 4; ++i) Wv.rt[16 * lq + 4 * i + e][lm] = acc[e][i];
        wave_lds_order();

        // (4) per column j = lane: u and o of the block's tokens, the dot products scaled by
        // the norm factors (kk_ts = ik_t ik_s kk_raw, qk_ts = iq_t ik_s qk_raw)
        float rk[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(&Wv.rt[lane][4 * i]);
            rk[4 * i] = x[0]; rk[4 * i + 1] = x[1]; rk[4 * i + 2] = x[2]; rk[4 * i + 3] = x[3];
        }
        if constexpr (ONEBLK) {
            // branch-free over the 8 tokens, so the coefficient reads of later tokens overlap
            // the chain of earlier ones (the registers allow it once the state is dead): tokens
            // past the block's end have beta = 0 and zero operands, so their u is 0, and their o
            // is never stored.  Live tokens take the same operations as the branch below.
            float u[kWyTB], ov[kWyTB];
#pragma unroll
            for (int t = 0; t < kWyTB; ++t) {
                const float iq = L.nf[t], ik = L.nf[kWyTB + t];
                float d = Wv.ut[t][lane] - rk[t];
#pragma unroll
                for (int sb = 0; sb < t; ++sb)
                    d = fmaf(-(L.pq[wy_pair(t, sb)] * ik * L.nf[kWyTB + sb]), u[sb], d);
                u[t] = bt[t] * d;
                float o = rk[8 + t];
#pragma unroll
                for (int sb = 0; sb < t; ++sb)
                    o = fmaf(L.pq[32 + wy_pair(t, sb)] * iq * L.nf[kWyTB + sb], u[sb], o);
                ov[t] = fmaf(L.pq[wy_diag(t)] * iq * ik, u[t], o) * a.scale;
            }
            wave_lds_order();  // the v reads above precede the u writes into the same slots
#pragma unroll
            for (int t = 0; t < kWyTB; ++t) {
                Wv.ut[t][lane] = u[t];
                if (t < nb) {
                    const int64_t tok = tok0 + static_cast<int64_t>(tb + t) * a.H;
                    store1<TIn>(a.o, tok * DV + tile * BV + lane, ov[t]);
                    if (VERIFY) a.records[tok * (2 * DK + DV) + 2 * DK + tile * BV + lane] = u[t];
                }
            }
        } else {
            float u[kWyTB];
#pragma unroll
            for (int t = 0; t < kWyTB; ++t) {
                u[t] = 0.f;
                if (t < nb) {
                    const float iq = L.nf[t], ik = L.nf[kWyTB + t];
                    float d = Wv.ut[t][lane] - rk[t];
#pragma unroll
                    for (int sb = 0; sb < t; ++sb)
                        d = fmaf(-(L.pq[wy_pair(t, sb)] * ik * L.nf[kWyTB + sb]), u[sb], d);
                    u[t] = bt[t] * d;
                    float o = rk[8 + t];
#pragma unroll
                    for (int sb = 0; sb < t; ++sb)
                        o = fmaf(L.pq[32 + wy_pair(t, sb)] * iq * L.nf[kWyTB + sb], u[sb], o);
                    o = fmaf(L.pq[wy_diag(t)] * iq * ik, u[t], o);
                    const int64_t tok = tok0 + static_cast<int64_t>(tb + t) * a.H;
                    store1<TIn>(a.o, tok * DV + tile * BV + lane, o * a.scale);
                    if (VERIFY) a.records[tok * (2 * DK + DV) + 2 * DK + tile * BV + lane] = u[t];
                    Wv.ut[t][lane] = u[t];
                }
            }
        }

        // (5) the state update, in token order with the replay kernel's operations
        if (!VERIFY || (!ONEBLK && tb + kWyTB < a.T)) {
            wave_lds_order();
            for (int t = 0; t < nb; ++t) {
                const float4 uu = *reinterpret_cast<const float4*>(&Wv.ut[t][4 * lm]);
#pragma unroll
                for (int i = 0; i < KS / 4; ++i) {
                    const f32x4 alv = *reinterpret_cast<const f32x4*>(&L.ar[t][lq][4 * i]);
                    const f32x4 kv = *reinterpret_cast<const f32x4*>(&L.kr[t][lq][4 * i]);
#pragma unroll
                    for (int k4 = 0; k4 < 4; ++k4) {
                        float4& x = sv[4 * i + k4];
                        x = f4_scale_fma(kv[k4], uu, f4_mul(x, alv[k4]));
                    }
                }
            }
        }
        sync();  // the next block's writes follow every read of this one, in both waves
    };
    block(0, std::true_type{});
    if constexpr (!ONEBLK)
        for (int tb = kWyTB; tb < a.T; tb += kWyTB) block(tb, std::false_type{});
    if (!VERIFY) {
#pragma unroll
        for (int st = 0; st < KS; ++st) state_store4(srs, voff, 4 * st * DV * 4, sv[st]);
    }
}

// ReplaySSM commit: S <- diag(alpha) S + kh u^T for the accepted records, with the
// same fp32 operation order as the decode kernel's decay and update.
template <int DK, int DV, int BV, int TB, int NTHR = kThreads>
__global__ __launch_bounds__(NTHR) void replay_kernel(ReplayArgs a) {
    using C = Tile<DK, DV, BV, NTHR>;
    __shared__ __attribute__((aligned(16))) float Lk[TB][DK];  // read as float4
    __shared__ __attribute__((aligned(16))) float La[TB][DK];
    __shared__ __attribute__((aligned(16))) float Lu[TB][BV];

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

    // a block's records as 16-byte loads, all in flight before the first LDS store (records
    // are 16-byte aligned: 2 dk + dv floats per token, a multiple of 4)
    constexpr int RV = (2 * DK + BV) / 4, MV = (TB * RV + NTHR - 1) / NTHR;
    float4 rv[MV];
    auto fetch = [&](int tb, int nb) {
#pragma unroll
        for (int m = 0; m < MV; ++m) {
            const int idx = tid + m * NTHR, j = idx / RV, e = 4 * (idx % RV);
            rv[m] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (j < nb) {
                const int64_t tok = (static_cast<int64_t>(n) * a.T + tb + j) * a.H + h;
                const float* rec = a.records + tok * (2 * DK + DV);
                rv[m] = *reinterpret_cast<const float4*>(e < 2 * DK ? rec + e : rec + 2 * DK + tile * BV + (e - 2 * DK));
            }
        }
    };
    // the first block's records go out ahead of the state tile (loads complete in issue
    // order, so they are in LDS while the tile streams in)
    fetch(0, min(TB, acc));
    float4 s[C::RPT];
#pragma unroll
    for (int i = 0; i < C::RPT; ++i) s[i] = load_stream4(S + (rg + C::RG * i) * DV + col0);

    for (int tb = 0; tb < acc; tb += TB) {
        const int nb = min(TB, acc - tb);
        if (tb > 0) fetch(tb, nb);
#pragma unroll
        for (int m = 0; m < MV; ++m) {
            const int idx = tid + m * NTHR, j = idx / RV, e = 4 * (idx % RV);
            if (j < nb) {
                const float x[4] = {rv[m].x, rv[m].y, rv[m].z, rv[m].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (e < DK)
                        Lk[j][C::pos(e + i)] = x[i];
                    else if (e < 2 * DK)
                        La[j][C::pos(e - DK + i)] = x[i];
                    else
                        Lu[j][e - 2 * DK + i] = x[i];
                }
            }
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

// T = 1: a workgroup per (sequence, head) holding the whole state (HBM-bound, decode_kernel).
// T > 1: one workgroup per head, a wave per 64-column tile, the WY form of 8-token blocks
// (wy_multi_kernel).
template <int DK, int DV, class TIn>
hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t stream) {
    const dim3 hgrid(static_cast<unsigned>(a.N) * a.H);  // one workgroup per (sequence, head)
    if (a.front.gate_scale) {
        // the input front: the workgroup owns the head's convolution state; up to kFrontTB
        // tokens as one block, commit mode only (four waves: eight measured slower)
        hipLaunchKernelGGL((decode_kernel<DK, DV, DV, kFrontTB, TIn, false, true>), hgrid, dim3(kThreads), 0,
                           stream, a);
    } else if (a.T == 1) {
        // the whole head's state per workgroup: eight waves for dv = 128 (each row group's
        // 128 columns are one 512-byte access), four for dv = 64
        constexpr int NT1 = DV == 128 ? 2 * kThreads : kThreads;
        if (a.records)
            hipLaunchKernelGGL((decode_kernel<DK, DV, DV, 1, TIn, true, false, NT1>), hgrid, dim3(NT1), 0, stream, a);
        else
            hipLaunchKernelGGL((decode_kernel<DK, DV, DV, 1, TIn, false, false, NT1>), hgrid, dim3(NT1), 0, stream, a);
    } else {
        const dim3 hblock(kWave * (DV / 64));
        if (a.records && a.T <= kWyTB)
            hipLaunchKernelGGL((wy_multi_kernel<DK, DV, TIn, true, true>), hgrid, hblock, 0, stream, a);
        else if (a.records)
            hipLaunchKernelGGL((wy_multi_kernel<DK, DV, TIn, true, false>), hgrid, hblock, 0, stream, a);
        else
            hipLaunchKernelGGL((wy_multi_kernel<DK, DV, TIn, false, false>), hgrid, hblock, 0, stream, a);
    }
    return hipGetLastError();
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
// affect the result; whole-head tiles measured faster, and 512 threads at dv = 128 (two whole
// rows per wave access) faster than 256: replay 27.7 -> 26.2 us on the verify workload.
template <int DK, int DV>
hipError_t launch_replay_d(const ReplayArgs& a, hipStream_t stream) {
    constexpr int BV = DV, RT = DV == 128 ? 2 * kThreads : kThreads;  // as decode_kernel at T = 1
    using C = Tile<DK, DV, BV, RT>;
    const dim3 grid(static_cast<unsigned>(a.N) * a.H * C::NT), block(RT);
    hipLaunchKernelGGL((replay_kernel<DK, DV, BV, 8, RT>), grid, block, 0, stream, a);
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
