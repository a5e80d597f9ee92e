// kda_backward.hip -- chunked backward of the KDA recurrence for gfx950 (training).
//
// The Kimi K3 day-0 adaptation page names forward and backward linear-attention kernels for
// training (section "基于昇腾实现Kimi K3训练基础功能适配与深度优化", the Triton-Ascend item) but
// prints no formula.  The gradients here are the chain rule through the 64-token chunk form of
// the forward (the chunk algebra of kda_prefill.hip), for a chunk entering with state S:
//
//   forward  A = beta (.) Ag,  Ag_ts = sum_c kh_tc kh_sc e^(G_tc - G_sc)  (s < t)
//            P_ts = sum_c qh_tc kh_sc e^(G_tc - G_sc)  (s <= t),  T = (I + A)^-1
//            BK = beta kh e^G,  BV = beta v,  W = T BK,  Ut = T BV,  U = Ut - W S
//            O = scale (QG S + P U),  QG = qh e^G;  S' = e^(G_L) S + Kt^T U,  Kt = kh e^(G_L - G)
//   backward (dH = dL/dS', dO = dL/dO)
//            dU = scale P^T dO + Kt dH;  dS = e^(G_L) dH - W^T dU + scale QG^T dO
//                                          = Mt dH + b,  Mt = e^(G_L) - W^T Kt,  b = scale (QG - P W)^T dO
//            dQG = scale dO S^T,  dP = scale dO U^T (s <= t),  dW = -dU S^T,  dKt = U dH^T
//            dT = dW BK^T + dU BV^T,  dBK = T^T dW,  dBV = T^T dU,  dA = -(T^T dT T^T) (s < t)
//            dv = beta dBV,  dbeta = sum(v dBV) + sum(kh e^G dBK) + sum_s dA Ag,  dAg = beta dA
//            dkh = beta e^G dBK + e^(G_L - G) dKt + X1 + X2 + X3,   dqh = e^G dQG + X4
//              X1_t = sum_s dAg_ts kh_s e^(G_t - G_s),  X2_s = sum_t dAg_ts kh_t e^(G_t - G_s)
//              X3_s = sum_t dP_ts qh_t e^(G_t - G_s),   X4_t = sum_s dP_ts kh_s e^(G_t - G_s)
//            dG = QG dQG + BK dBK - Kt dKt + kh X1 - kh X2 + qh X4 - kh X3   (per token, channel)
//            dG_L = e^(G_L) sum_j S dH + sum_t Kt dKt;  dg_t = sum_(t' >= t) dG_t' + dG_L
//            dq = (dqh - qh (qh . dqh)) / |q|,  dk likewise (identity without the L2 norm)
//
// Launches on the caller's stream (all arithmetic fp32; bf16 inputs are widened):
//   0. bwd_init        identity slot map and the initial states for the forward pass
//   1. the forward prefill (kda_prefill.hip) with its carry storing every chunk's entering state
//      (and no output O: its intra-chunk records skip QG and P)
//   2. bwd_intra       per (chunk, head): Ag, P, T (forward substitution), W, Ut, exp(G_L)
//   3. bwd_prep        per (chunk, head): Mt and b of the reverse state recurrence
//   4. bwd_scan        per (sequence, head, 16 columns): dS_c = Mt_c dS_(c+1) + b_c from the
//                      last chunk back, keeping each chunk's exit-state gradient; dh0
//   5. bwd_state       per (chunk, head): the products with S and dH (U, dU, dQG, dW, dKt, dP,
//                      the e^(G_L) part of dG_L), over 32-column blocks of the state
//   6. bwd_ut          per (chunk, head): dT, dBK, dBV, dA; writes dv and dbeta
//   7. bwd_final       per (chunk, head): X1..X4, dkh, dqh, dG, the reverse cumsum and the
//                      norm backward; writes dq, dk and dg
// Every e^(G_t - G_s) is split at a reference inside its 16-token block pair, as in the
// forward: off-diagonal block pairs at a block end (both factors at most 1), diagonal blocks
// at the block's 8th token.
#include "kda.h"
#include "kda_device.hpp"
#include "kda_internal.hpp"
#include "kda_layout.hpp"

namespace kda {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kC = 64;
constexpr int kXcd = 8;  // XCDs of the GPU (workgroups are dispatched to them round-robin)
constexpr int kT = 256;  // threads of every per-chunk kernel (4 waves)
constexpr float kL2e = 1.4426950408889634f;
constexpr float kEps = 1e-6f;

__host__ __device__ constexpr size_t al256(size_t x) { return (x + 255) / 256 * 256; }

// ---------------------------------------------------------------------------
// Workspace: the forward prefill's workspace first (its chunk table is read here), then
//   pool [ns][H][dk][dv] f32, slots [ns] i32,
//   per (chunk, head) item (fp32, row-major):
//     S [dk][dv]   state entering the chunk (forward carry)
//     dX [dk][dv]  gradient of the chunk's exit state (scan)
//     Mt [dk][dk], b [dk][dv]
//     T, Ag, P [64][64];  W [64][dk], Ut [64][dv];  gl [dk] = e^(G_L)
//     dU [64][dv], dQG, dW, dKt [64][dk], dP [64][64], dgl [dk];  dBK [64][dk], dAg [64][64]
// ---------------------------------------------------------------------------
struct BwLayout {
    size_t fwd, off_pool, off_slots, off_items, item, total;
    size_t S, dX, Mt, b, T, Ag, P, W, Ut, gl, dU, dQG, dW, dKt, dP, dgl, dBK, dAg;
    int64_t max_items;
    __host__ __device__ BwLayout(int ns, int64_t T_tot, int H, int dk, int dv, int e) {
        fwd = al256(WsLayout(ns, T_tot, H, dk, dv, e).total);
        off_pool = fwd;
        off_slots = off_pool + al256(sizeof(float) * ns * H * dk * dv);
        off_items = off_slots + al256(sizeof(int32_t) * ns);
        size_t o = 0;
        auto take = [&](size_t n) {
            const size_t at = o;
            o += al256(sizeof(float) * n);
            return at;
        };
        S = take(dk * dv), dX = take(dk * dv), Mt = take(dk * dk), b = take(dk * dv);
        T = take(kC * kC), Ag = take(kC * kC), P = take(kC * kC), W = take(kC * dk), Ut = take(kC * dv);
        gl = take(dk), dU = take(kC * dv), dQG = take(kC * dk), dW = take(kC * dk), dKt = take(kC * dk);
        dP = take(kC * kC), dgl = take(dk), dBK = take(kC * dk), dAg = take(kC * kC);
        item = o;
        max_items = (T_tot / kC + ns) * H;
        total = off_items + item * static_cast<size_t>(max_items);
    }
};

// The forward's chunk offsets (at 0 of its workspace) and chunk table (kda_layout.hpp).
struct FwdTables {
    const int32_t* chunk_off;
    const int4* table;
};

// fp32 MFMA 16x16 tile: C(m, n) += sum_k A(m, k) B(k, n), k in [0, K) (K a multiple of 16);
// A(m, k) = A[m * am + k * ak], B(k, n) = B[k * bk + n * bn].  Lane l holds C(4 (l / 16) + i,
// l % 16), i = 0..3.
// Of every 16 k values, lane (r, q) supplies k = 16 s + 4 q + j to step j (the order of the
// k sum is free), so an operand whose k index is contiguous (ak = 1 or bk = 1: every call
// passes these as constants) is read as one 16-byte LDS load per four steps.  One
// accumulator: the matrix core takes back-to-back accumulation into the same registers, and
// more chains only add initialisation and combining instructions.  Every base, stride and offset
// here is a multiple of 4 floats of a 16-byte aligned array.
__device__ __forceinline__ f32x4 mm16(const float* A, int am, int ak, const float* B, int bk, int bn, int K,
                                      int lane, f32x4 c) {
    const int r = lane & 15, q = lane >> 4;
    f32x4 acc = c;
    for (int k0 = 0; k0 < K; k0 += 16) {
        const int kb = k0 + 4 * q;
        f32x4 av, bv;
        if (ak == 1) {
            av = *reinterpret_cast<const f32x4*>(A + r * am + kb);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) av[j] = A[r * am + (kb + j) * ak];
        }
        if (bk == 1) {
            bv = *reinterpret_cast<const f32x4*>(B + r * bn + kb);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) bv[j] = B[(kb + j) * bk + r * bn];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[j], bv[j], acc, 0, 0, 0);
    }
    return acc;
}

// Inclusive prefix sum over the 64 lanes of a wave (lane i gets x_0 + ... + x_i): a scan in
// each 16-lane row by DPP row shifts (lanes shifted in from outside the row add 0), then the
// totals of the rows before carried in with row_bcast:15 (into rows 1 and 3) and
// row_bcast:31 (into rows 2 and 3).
__device__ __forceinline__ float wave_prefix64(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x142, 0xa, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x143, 0xc, 0xf, false));
    return x;
}

template <class TIn>
__device__ __forceinline__ float ld_in(const void* p, int64_t i) {
    return load1<TIn>(p, i);
}
__device__ __forceinline__ void st_out(void* p, int64_t i, float x, F32) { static_cast<float*>(p)[i] = x; }
__device__ __forceinline__ void st_out(void* p, int64_t i, float x, BF16) {
    static_cast<uint16_t*>(p)[i] = f32_to_bf16(x);
}

struct Item {
    int seq, t0, L, h, chunk;
};

__device__ __forceinline__ bool item_of(const PrefillArgs& a, const char* ws, const FwdTables& ft, int item,
                                        Item& it) {
    const int nch = ft.chunk_off[a.num_seqs];
    if (item >= nch * a.H) return false;
    it.chunk = item / a.H;
    it.h = item % a.H;
    const int4 e = ft.table[it.chunk];
    it.seq = e.x;
    it.t0 = e.y;
    it.L = e.z;
    return true;
}

// The copies below issue every load of a thread before any of its stores (16-byte accesses,
// compile-time counts), so the loads are in flight together instead of each waiting in turn.

// Columns c0 .. c0 + W - 1 of rows t0 .. t0 + L - 1 of head h of a [T][H][D] input into LDS
// dst [64][ld] (fp32; rows from L on are zero): rows_fetch issues the loads into registers,
// rows_store writes them (so a caller can keep the loads in flight across other work).
template <class TIn, int W, int NT = kT>
struct RowCopy {
    static constexpr int EPG = 16 / TIn::bytes;  // elements per 16-byte access
    static constexpr int GPR = W / EPG, N = (kC * GPR + NT - 1) / NT;
    static_assert(W % EPG == 0, "row copy shape");
};
template <class TIn, int D, int W = D, int NT = kT>
__device__ __forceinline__ void rows_fetch(const void* src, u32x4 (&v)[RowCopy<TIn, W, NT>::N], const Item& it, int H,
                                           int c0 = 0) {
    using RC = RowCopy<TIn, W, NT>;
#pragma unroll
    for (int i = 0; i < RC::N; ++i) {
        const int idx = threadIdx.x + i * NT, t = idx / RC::GPR, c = c0 + RC::EPG * (idx % RC::GPR);
        v[i] = u32x4{0u, 0u, 0u, 0u};
        if (idx < kC * RC::GPR && t < it.L)
            v[i] = *reinterpret_cast<const u32x4*>(static_cast<const char*>(src) +
                                                   ((static_cast<int64_t>(it.t0 + t) * H + it.h) * D + c) * TIn::bytes);
    }
}
template <class TIn, int W, int NT = kT>
__device__ __forceinline__ void rows_store(const u32x4 (&v)[RowCopy<TIn, W, NT>::N], float* dst, int ld) {
    using RC = RowCopy<TIn, W, NT>;
#pragma unroll
    for (int i = 0; i < RC::N; ++i) {
        const int idx = threadIdx.x + i * NT, t = idx / RC::GPR, c = RC::EPG * (idx % RC::GPR);
        if (idx >= kC * RC::GPR) break;
        float* d = dst + t * ld + c;
        if constexpr (TIn::bytes == 2) {
            auto wide = [](uint32_t a, uint32_t b) {
                return f32x4{__uint_as_float(a << 16), __uint_as_float(a & 0xffff0000u), __uint_as_float(b << 16),
                             __uint_as_float(b & 0xffff0000u)};
            };
            reinterpret_cast<f32x4*>(d)[0] = wide(v[i][0], v[i][1]);
            reinterpret_cast<f32x4*>(d)[1] = wide(v[i][2], v[i][3]);
        } else {
            *reinterpret_cast<f32x4*>(d) = __builtin_bit_cast(f32x4, v[i]);
        }
    }
}
template <class TIn, int D, int W = D, int NT = kT>
__device__ void load_rows(const void* src, float* dst, int ld, const Item& it, int H, int c0 = 0) {
    u32x4 v[RowCopy<TIn, W, NT>::N];
    rows_fetch<TIn, D, W, NT>(src, v, it, H, c0);
    rows_store<TIn, W, NT>(v, dst, ld);
}

// f(t, c) for every 4-column group (t < 64, c = 0, 4, .., D - 4) of a 64 x D block, the
// workgroup's threads taking consecutive groups (16-byte LDS accesses in f).
template <int D, int NT = kT, class F>
__device__ __forceinline__ void for_groups(F f) {
    constexpr int GPR = D / 4;
    for (int i = threadIdx.x; i < kC * GPR; i += NT) f(i / GPR, 4 * (i % GPR));
}

// In place x_t <- x_t / sqrt(|x_t|^2 + eps) (when use_l2); inv[t] gets the factor.  NT / 64
// adjacent lanes share a row: each sums and then scales its own D / (NT / 64) channels (16-byte
// LDS accesses; ld and the offsets are multiples of 4 floats), the partial sums meet by lane
// shuffles, so only the final barrier is needed.
template <int NT = kT>
__device__ void normalize_rows(float* x, int ld, int D, float* inv, int use_l2) {
    constexpr int TPR = NT / kC;  // threads per row
    const int t = threadIdx.x / TPR, p = threadIdx.x % TPR, w = D / TPR;
    float* row = x + t * ld + p * w;
    float s = 0.f;
    for (int c = 0; c < w; c += 4) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(row + c);
        s = fmaf(v[0], v[0], fmaf(v[1], v[1], fmaf(v[2], v[2], fmaf(v[3], v[3], s))));
    }
#pragma unroll
    for (int m = 1; m < TPR; m <<= 1) s += __shfl_xor(s, m, 64);
    const float f = use_l2 ? 1.f / sqrtf(s + kEps) : 1.f;
    if (p == 0) inv[t] = f;
    if (use_l2) {
        for (int c = 0; c < w; c += 4) {
            f32x4 v = *reinterpret_cast<const f32x4*>(row + c);
            *reinterpret_cast<f32x4*>(row + c) = v * f;
        }
    }
    lds_barrier();
}

// G [64][ld] = in-chunk inclusive cumsum of g, in log2 units (rows from L on repeat G_L).
// The chunk's gates are first copied into G by all threads (coalesced), then each wave scans
// columns across its 64 lanes (lane = token).  The caller synchronises before reading G.
template <int DK, int NT = kT>
__device__ void gate_scan(float* G, int ld) {
    lds_barrier();
    // a wave scans four adjacent columns per pass (one 16-byte LDS access per lane)
    const int lane = threadIdx.x & 63;
    for (int c = 4 * (threadIdx.x >> 6); c < DK; c += 4 * (NT / 64)) {
        f32x4* p = reinterpret_cast<f32x4*>(G + lane * ld + c);
        f32x4 v = *p;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = wave_prefix64(v[e] * kL2e);
        *p = v;
    }
}
template <int DK, int NT = kT>
__device__ void gate_cumsum(const float* g, float* G, int ld, const Item& it, int H) {
    load_rows<F32, DK, DK, NT>(g, G, ld, it, H);
    gate_scan<DK, NT>(G, ld);
}

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// Decayed Gram tiles (t block i, s block j <= i) of the key and the query rows against the key
// rows: ta(t, s) = sum_c K_tc K_sc 2^(G_tc - G_sc), tp(t, s) = sum_c Q_tc K_sc 2^(G_tc - G_sc),
// the factor split at row R = 16 i - 1 (j < i) or 16 i + 7 (j = i).  The two share every
// exponential and the s-side operand.  Lane holds (t = 16 i + 4q + ii, s = 16 j + r).
__device__ void dgram_pair(const float* K, const float* Q, const float* G, int ld, int DK, int i, int j, int lane,
                           f32x4& ta, f32x4& tp) {
    const int r = lane & 15, q = lane >> 4;
    const int R = j < i ? 16 * i - 1 : 16 * i + 7;
    // of every 16 channels, lane (r, q) supplies channels 16 s + 4 q + e to step e, so each
    // operand row is read as 16-byte LDS loads (ld and every offset are multiples of 4 floats)
    f32x4 ca = {0.f, 0.f, 0.f, 0.f}, cp = ca;
    for (int k0 = 0; k0 < DK; k0 += 16) {
        const int ch = k0 + 4 * q;
        const f32x4 ref = *reinterpret_cast<const f32x4*>(G + R * ld + ch);
        const f32x4 kt = *reinterpret_cast<const f32x4*>(K + (16 * i + r) * ld + ch);
        const f32x4 qt = *reinterpret_cast<const f32x4*>(Q + (16 * i + r) * ld + ch);
        const f32x4 gt = *reinterpret_cast<const f32x4*>(G + (16 * i + r) * ld + ch);
        const f32x4 ks = *reinterpret_cast<const f32x4*>(K + (16 * j + r) * ld + ch);
        const f32x4 gs = *reinterpret_cast<const f32x4*>(G + (16 * j + r) * ld + ch);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float ft = ex2(gt[e] - ref[e]);
            const float bv = ks[e] * ex2(ref[e] - gs[e]);
            ca = __builtin_amdgcn_mfma_f32_16x16x4f32(kt[e] * ft, bv, ca, 0, 0, 0);
            cp = __builtin_amdgcn_mfma_f32_16x16x4f32(qt[e] * ft, bv, cp, 0, 0, 0);
        }
    }
    ta = ca;
    tp = cp;
}

// Decayed token products over a 16 x 16 (rows, channels) output tile.
//  t mode: Y(t, c) = sum_(s <= t) X(t, s) Z(s, c) 2^(G_tc - G_sc), t in block i
//  s mode: Y(s, c) = sum_(t >= s) X(t, s) Z(t, c) 2^(G_tc - G_sc), s in block i
// X [64][ldx] is stored lower triangular (zero above the diagonal).  Block pairs off the
// diagonal split the factor at a block end (t mode: the end of block i - 1; s mode: the end
// of block i), the diagonal block at its 8th token.  Lane holds (row 16 i + 4q + ii, channel
// 16 cb + r).
// Two such products of one mode are formed together, sharing their exponentials: ya from
// (Xa, Za), yb from (Xb, Zb); with SAMEZ (Zb = Za) they also share the B operand.
template <bool TMODE, bool SAMEZ>
__device__ void dtok_pair(const float* Xa, const float* Xb, int ldx, const float* Za, const float* Zb,
                          const float* G, int ld, int i, int cb, int lane, f32x4& ya, f32x4& yb) {
    const int r = lane & 15, q = lane >> 4, ch = 16 * cb + r;
    const int Roff = TMODE ? 16 * i - 1 : 16 * i + 15, M = 16 * i + 7;
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    // one accumulator per product for the off-diagonal and one for the diagonal part (the two
    // products' chains alternate, so consecutive MFMAs do not wait for each other)
    f32x4 oa = z4, ob = z4, da = z4, db = z4;
    // a 16-token block: lane (r, q) supplies token k0 + 4q + e to step e (the order of the sum
    // is free), so in t mode its X row segment is one 16-byte LDS read
    auto kblock = [&](int k0, float ref, f32x4& ca, f32x4& cb2) {
        f32x4 xa, xb;
        if constexpr (TMODE) {
            xa = *reinterpret_cast<const f32x4*>(Xa + (16 * i + r) * ldx + k0 + 4 * q);
            xb = *reinterpret_cast<const f32x4*>(Xb + (16 * i + r) * ldx + k0 + 4 * q);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                xa[e] = Xa[(k0 + 4 * q + e) * ldx + 16 * i + r];
                xb[e] = Xb[(k0 + 4 * q + e) * ldx + 16 * i + r];
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int k = k0 + 4 * q + e;
            const float g = G[k * ld + ch];
            const float zf = TMODE ? ex2(ref - g) : ex2(g - ref);
            const float za = Za[k * ld + ch] * zf;
            const float zb = SAMEZ ? za : Zb[k * ld + ch] * zf;
            ca = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[e], za, ca, 0, 0, 0);
            cb2 = __builtin_amdgcn_mfma_f32_16x16x4f32(xb[e], zb, cb2, 0, 0, 0);
        }
    };
    // off-diagonal blocks: t mode the s blocks before i, s mode the t blocks after i
    const int kb = TMODE ? 0 : 16 * (i + 1), ke = TMODE ? 16 * i : kC;
    if (ke > kb) {
        const float ref = G[Roff * ld + ch];
        for (int k0 = kb; k0 < ke; k0 += 16) kblock(k0, ref, oa, ob);
    }
    kblock(16 * i, G[M * ld + ch], da, db);
    const f32x4 offa = oa, offb = ob, dga = da, dgb = db;
    const float ro = ke > kb ? G[Roff * ld + ch] : 0.f, rm = G[M * ld + ch];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
        const float gr = G[(16 * i + 4 * q + ii) * ld + ch];
        const float fo = ke > kb ? (TMODE ? ex2(gr - ro) : ex2(ro - gr)) : 0.f;
        const float fm = TMODE ? ex2(gr - rm) : ex2(rm - gr);
        ya[ii] = offa[ii] * fo + dga[ii] * fm;
        yb[ii] = offb[ii] * fo + dgb[ii] * fm;
    }
}

// Stores a 16 x 16 accumulator tile (rows 16 rb + 4q + ii, columns 16 cb + r) to a row-major
// fp32 matrix of leading dimension ld.
__device__ __forceinline__ void put_tile(float* M, int ld, int rb, int cb, f32x4 v, int lane) {
    const int r = lane & 15, q = lane >> 4;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) M[(16 * rb + 4 * q + ii) * ld + 16 * cb + r] = v[ii];
}
__device__ __forceinline__ f32x4 get_tile(const float* M, int ld, int rb, int cb, int lane) {
    const int r = lane & 15, q = lane >> 4;
    f32x4 v;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) v[ii] = M[(16 * rb + 4 * q + ii) * ld + 16 * cb + r];
    return v;
}

// T = (I + A)^-1 for A = diag(beta) Ag (Ag [64][68] strictly lower, fp32), into T [64][68],
// by 16 x 16 blocks: wave w inverts diagonal block w by forward substitution (one lane per
// column, the block's rows read as vectors, the column in registers); then for d = 1, 2, 3
// the waves w >= d form T_(w, w-d) = -T_ww sum_(k = w-d .. w-1) A_wk T_(k, w-d) on fp32 MFMA.
// Y is a per-wave 16 x 20 scratch.  Ends with a barrier.
__device__ void unit_lower_inverse(const float* Ag, const float* beta, float* T, float* Y, int lane, int wave) {
    constexpr int LC = kC + 4, LY = 20;
    const int r = lane & 15, q = lane >> 4;
    // waves 0..3 own the four row blocks; further waves of the caller only join the barriers
    const bool on = wave < 4;
    // zero the blocks above the diagonal of this wave's rows (4 columns per store)
    for (int i = lane; on && i < 16 * (kC / 4); i += 64) {
        const int row = 16 * wave + i / (kC / 4), c = 4 * (i % (kC / 4));
        if (c >= 16 * (wave + 1)) *reinterpret_cast<f32x4*>(T + row * LC + c) = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (on) {
        const int col = r, b0 = 16 * wave;
        float x[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            const float bt = beta[b0 + rr];
            f32x4 row[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) row[m] = *reinterpret_cast<const f32x4*>(Ag + (b0 + rr) * LC + b0 + 4 * m);
            float acc = rr == col ? 1.f : 0.f;
#pragma unroll
            for (int s = 0; s < rr; ++s) acc = fmaf(-bt * row[s >> 2][s & 3], x[s], acc);
            x[rr] = acc;
        }
        if (q == 0) {
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) T[(b0 + rr) * LC + b0 + col] = x[rr];
        }
    }
    lds_barrier();
    float* y = Y + (on ? wave : 0) * 16 * LY;
    for (int d = 1; d < 4; ++d) {
        if (on && wave >= d) {
            const int jb = wave - d;
            // y = A_(wave, jb .. wave-1) T_(jb .. wave-1, jb): k over 16 d rows of T
            f32x4 acc = mm16(Ag + 16 * wave * LC + 16 * jb, LC, 1, T + 16 * jb * LC + 16 * jb, LC, 1, 16 * d, lane,
                             f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) acc[ii] *= beta[16 * wave + 4 * q + ii];
            put_tile(y, LY, 0, 0, acc, lane);
            // z = T_(wave, wave) y (this wave's own scratch, so no workgroup barrier is needed)
            const f32x4 z = mm16(T + 16 * wave * LC + 16 * wave, LC, 1, y, LY, 1, 16, lane, f32x4{0.f, 0.f, 0.f, 0.f});
            put_tile(T + 16 * wave * LC + 16 * jb, LC, 0, 0, -z, lane);
        }
        lds_barrier();
    }
}

// Global <-> LDS copies of a row-major fp32 [ROWS][COLS] matrix (leading dimensions and base
// addresses multiples of 4 floats).
template <int ROWS, int COLS, int NT = kT>
struct MatCopy {
    static constexpr int C4 = COLS / 4, N = ROWS * C4 / NT;
    static_assert(COLS % 4 == 0 && (ROWS * C4) % NT == 0, "copy shape");
};
template <int ROWS, int COLS, int NT = kT>
__device__ __forceinline__ void g2r(const float* g, int gld, f32x4 (&v)[MatCopy<ROWS, COLS, NT>::N]) {
    using MC = MatCopy<ROWS, COLS, NT>;
#pragma unroll
    for (int i = 0; i < MC::N; ++i) {
        const int idx = threadIdx.x + i * NT;
        v[i] = *reinterpret_cast<const f32x4*>(g + (idx / MC::C4) * gld + 4 * (idx % MC::C4));
    }
}
template <int ROWS, int COLS, int NT = kT>
__device__ __forceinline__ void r2s(const f32x4 (&v)[MatCopy<ROWS, COLS, NT>::N], float* s, int sld) {
    using MC = MatCopy<ROWS, COLS, NT>;
#pragma unroll
    for (int i = 0; i < MC::N; ++i) {
        const int idx = threadIdx.x + i * NT;
        *reinterpret_cast<f32x4*>(s + (idx / MC::C4) * sld + 4 * (idx % MC::C4)) = v[i];
    }
}
template <int ROWS, int COLS, int NT = kT>
__device__ void g2s(const float* g, int gld, float* s, int sld) {
    f32x4 v[MatCopy<ROWS, COLS, NT>::N];
    g2r<ROWS, COLS, NT>(g, gld, v);
    r2s<ROWS, COLS, NT>(v, s, sld);
}
template <int ROWS, int COLS, int NT = kT>
__device__ void s2g(const float* s, int sld, float* g, int gld) {
    constexpr int C4 = COLS / 4, N = ROWS * C4 / NT;
    static_assert(COLS % 4 == 0 && (ROWS * C4) % NT == 0, "copy shape");
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const int idx = threadIdx.x + i * NT;
        *reinterpret_cast<f32x4*>(g + (idx / C4) * gld + 4 * (idx % C4)) =
            *reinterpret_cast<const f32x4*>(s + (idx / C4) * sld + 4 * (idx % C4));
    }
}

// The opening operands of a per-chunk kernel: every global load is issued before the first
// LDS store (load_rows and g2s each wait for their own loads before storing, so a sequence of
// them pays one memory latency per call).
template <class TIn, int D, int NT = kT>
struct Rows {
    u32x4 v[RowCopy<TIn, D, NT>::N];
    __device__ void fetch(const void* src, const Item& it, int H) { rows_fetch<TIn, D, D, NT>(src, v, it, H); }
    __device__ void store(float* dst, int ld) const { rows_store<TIn, D, NT>(v, dst, ld); }
};
template <int ROWS, int COLS, int NT = kT>
struct Mat {
    f32x4 v[MatCopy<ROWS, COLS, NT>::N];
    __device__ void fetch(const float* g, int gld) { g2r<ROWS, COLS, NT>(g, gld, v); }
    __device__ void store(float* s, int sld) const { r2s<ROWS, COLS, NT>(v, s, sld); }
};

struct BwCtx {
    BwLayout bw;
    FwdTables ft;
    char* items;
    __device__ BwCtx(const PrefillArgs& a, int dk, int dv, int e)
        : bw(a.num_seqs, a.total_tokens, a.H, dk, dv, e) {
        const char* base = static_cast<const char*>(a.workspace);
        ft.chunk_off = reinterpret_cast<const int32_t*>(base);
        ft.table = reinterpret_cast<const int4*>(base + WsLayout(a.num_seqs, a.total_tokens, a.H, dk, dv, e).off_table);
        items = static_cast<char*>(a.workspace) + bw.off_items;
    }
    __device__ float* blk(int item, size_t off) const {
        return reinterpret_cast<float*>(items + bw.item * static_cast<size_t>(item) + off);
    }
};

// ---------------------------------------------------------------------------
// 0. initial states and the identity slot map for the forward pass
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kT) void bwd_init_kernel(BackwardArgs b, int dk, int dv, int e) {
    const BwLayout bw(b.fwd.num_seqs, b.fwd.total_tokens, b.fwd.H, dk, dv, e);
    char* base = static_cast<char*>(b.fwd.workspace);
    float* pool = reinterpret_cast<float*>(base + bw.off_pool);
    int32_t* slots = reinterpret_cast<int32_t*>(base + bw.off_slots);
    const int64_t n = static_cast<int64_t>(b.fwd.num_seqs) * b.fwd.H * dk * dv;
    for (int64_t i = blockIdx.x * static_cast<int64_t>(kT) + threadIdx.x; i < n; i += static_cast<int64_t>(gridDim.x) * kT)
        pool[i] = b.h0 ? b.h0[i] : 0.f;
    for (int64_t i = blockIdx.x * static_cast<int64_t>(kT) + threadIdx.x; i < b.fwd.num_seqs;
         i += static_cast<int64_t>(gridDim.x) * kT)
        slots[i] = static_cast<int32_t>(i);
}

// ---------------------------------------------------------------------------
// 2. bwd_intra: Ag, P, T, W, Ut, exp(G_L) of one (chunk, head)
// ---------------------------------------------------------------------------
constexpr int kTI = 512;  // threads of bwd_intra
template <int DK, int DV, class TIn>
__global__ __launch_bounds__(kTI) void bwd_intra_kernel(BackwardArgs b) {
    const PrefillArgs& a = b.fwd;
    constexpr int LK = DK + 4, LV = DV + 4, LC = kC + 4, LM = LK > LV ? LK : LV;
    __shared__ __attribute__((aligned(16))) float sK[kC * LM], sQ[kC * LK], sG[kC * LK], sA[kC * LC], sT[kC * LC], sY[4 * 16 * 20], inv[kC],
        sB[kC];
    const BwCtx X(a, DK, DV, TIn::bytes);
    Item it;
    if (!item_of(a, static_cast<const char*>(a.workspace), X.ft, blockIdx.x, it)) return;
    // eight waves (two per SIMD): the Gram tiles spread over all of them; wave (tb, half) takes
    // token block tb and half of the column tiles of W and Ut; the UT inverse runs on waves 0..3
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, H = a.H;
    const int tb = wave & 3, half = wave >> 2;
    const int item = blockIdx.x;
    {
        Rows<TIn, DK, kTI> rk, rq;
        Rows<F32, DK, kTI> rg;
        rk.fetch(a.k, it, H);
        rq.fetch(a.q, it, H);
        rg.fetch(a.g, it, H);
        const float bt = threadIdx.x < it.L ? a.beta[static_cast<int64_t>(it.t0 + threadIdx.x) * H + it.h] : 0.f;
        rk.store(sK, LK);
        rq.store(sQ, LK);
        rg.store(sG, LK);
        if (threadIdx.x < kC) sB[threadIdx.x] = bt;
    }
    gate_scan<DK, kTI>(sG, LK);
    lds_barrier();
    // v is first needed after T and W: its loads, issued once the first operands are in,
    // stay in flight (registers) until then
    u32x4 rV[RowCopy<TIn, DV, kTI>::N];
    rows_fetch<TIn, DV, DV, kTI>(a.v, rV, it, H);
    normalize_rows<kTI>(sK, LK, DK, inv, a.use_l2);
    normalize_rows<kTI>(sQ, LK, DK, inv, a.use_l2);
    // Ag (strictly lower) and P (lower with the diagonal): the ten tiles (i, j <= i), at most
    // two per wave (wave 0: (0,0) (3,0); 1: (1,0) (3,1); 2: (1,1) (3,2); 3: (2,0) (3,3);
    // 4: (2,1); 5: (2,2); wave 6 the six zero tiles above the diagonal)
    float* Pg = X.blk(item, X.bw.P);
    float* Ag = X.blk(item, X.bw.Ag);
    {
        const int w = __builtin_amdgcn_readfirstlane(wave);
        const int r = lane & 15, q = lane >> 4;
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            // tile index 4 i + j of this wave's slot n (-1: none)
            const int ij = w == 0 ? (n == 0 ? 0 : 12)
                         : w == 1 ? (n == 0 ? 4 : 13)
                         : w == 2 ? (n == 0 ? 5 : 14)
                         : w == 3 ? (n == 0 ? 8 : 15)
                         : w == 4 ? (n == 0 ? 9 : -1)
                         : w == 5 ? (n == 0 ? 10 : -1)
                                  : -1;
            if (ij < 0) break;
            const int i = ij >> 2, j = ij & 3;
            f32x4 ta, tp;
            dgram_pair(sK, sQ, sG, LK, DK, i, j, lane, ta, tp);
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int t = 16 * i + 4 * q + ii, s = 16 * j + r;
                ta[ii] = s < t ? ta[ii] : 0.f;
                tp[ii] = s <= t ? tp[ii] : 0.f;
            }
            put_tile(sA, LC, i, j, ta, lane);
            put_tile(Pg, kC, i, j, tp, lane);
            put_tile(Ag, kC, i, j, ta, lane);
        }
        if (w == 6) {
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < 3; ++i)
#pragma unroll
                for (int j = i + 1; j < 4; ++j) {
                    put_tile(sA, LC, i, j, z, lane);
                    put_tile(Pg, kC, i, j, z, lane);
                    put_tile(Ag, kC, i, j, z, lane);
                }
        }
    }
    lds_barrier();
    // BK = beta kh 2^G into sQ (P is done) by waves 4..7 while waves 0..3 invert (I + A); the
    // inverse's barriers order these writes before W = T BK
    if (wave >= 4) {
        constexpr int GPR = DK / 4, NB = kTI - 256;
        for (int i = threadIdx.x - 256; i < kC * GPR; i += NB) {
            const int t = i / GPR, c = 4 * (i % GPR);
            const f32x4 k4 = *reinterpret_cast<const f32x4*>(sK + t * LK + c);
            const f32x4 g4 = *reinterpret_cast<const f32x4*>(sG + t * LK + c);
            f32x4 b4;
#pragma unroll
            for (int e = 0; e < 4; ++e) b4[e] = sB[t] * k4[e] * ex2(g4[e]);
            *reinterpret_cast<f32x4*>(sQ + t * LK + c) = b4;
        }
        if (threadIdx.x - 256 < DK) X.blk(item, X.bw.gl)[threadIdx.x - 256] = ex2(sG[(kC - 1) * LK + threadIdx.x - 256]);
    }
    unit_lower_inverse(sA, sB, sT, sY, lane, wave);
    s2g<kC, kC, kTI>(sT, LC, X.blk(item, X.bw.T), kC);
    float* Wg = X.blk(item, X.bw.W);
    for (int cb = half * (DK / 32); cb < (half + 1) * (DK / 32); ++cb) {
        const f32x4 w = mm16(sT + 16 * tb * LC, LC, 1, sQ + 16 * cb, LK, 1, kC, lane, f32x4{0.f, 0.f, 0.f, 0.f});
        put_tile(Wg, DK, tb, cb, w, lane);
    }
    lds_barrier();
    // BV = beta v into sK, then Ut = T BV
    rows_store<TIn, DV, kTI>(rV, sK, LV);
    lds_barrier();
    for_groups<DV, kTI>([&](int t, int c) {
        f32x4* x = reinterpret_cast<f32x4*>(sK + t * LV + c);
        *x = *x * sB[t];
    });
    lds_barrier();
    float* Ug = X.blk(item, X.bw.Ut);
    for (int cb = half * (DV / 32); cb < (half + 1) * (DV / 32); ++cb) {
        const f32x4 u = mm16(sT + 16 * tb * LC, LC, 1, sK + 16 * cb, LV, 1, kC, lane, f32x4{0.f, 0.f, 0.f, 0.f});
        put_tile(Ug, DV, tb, cb, u, lane);
    }
}

// Kt = kh 2^(G_L - G) and QG = qh 2^G in place (the raw normalised rows on entry).
template <int DK, int NT = kT>
__device__ void to_kt(float* K, const float* G, int ld) {
    for_groups<DK, NT>([&](int t, int c) {
        const f32x4 gl = *reinterpret_cast<const f32x4*>(G + (kC - 1) * ld + c);
        const f32x4 g = *reinterpret_cast<const f32x4*>(G + t * ld + c);
        f32x4* x = reinterpret_cast<f32x4*>(K + t * ld + c);
        f32x4 v = *x;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] *= ex2(gl[e] - g[e]);
        *x = v;
    });
}
template <int DK, int NT = kT>
__device__ void to_qg(float* Q, const float* G, int ld) {
    for_groups<DK, NT>([&](int t, int c) {
        const f32x4 g = *reinterpret_cast<const f32x4*>(G + t * ld + c);
        f32x4* x = reinterpret_cast<f32x4*>(Q + t * ld + c);
        f32x4 v = *x;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] *= ex2(g[e]);
        *x = v;
    });
}

// ---------------------------------------------------------------------------
// 3. bwd_prep: Mt = diag(e^(G_L)) - W^T Kt,  b = scale (QG - P W)^T dO.  Sixteen waves (four
//    per SIMD) share the output tiles.
// ---------------------------------------------------------------------------
constexpr int kTP = 1024;  // threads of bwd_prep
template <int DK, int DV, class TIn>
__global__ __launch_bounds__(kTP) void bwd_prep_kernel(BackwardArgs b) {
    const PrefillArgs& a = b.fwd;
    constexpr int LK = DK + 4, LV = DV + 4, LC = kC + 4, NW = kTP / 64, NQ = (DK / 16) / (NW / 4);
    __shared__ __attribute__((aligned(16))) float sK[kC * LK], sQ[kC * LK], sW[kC * LK], sO[kC * LV], sP[kC * LC], inv[kC],
        sgl[DK];
    float* sG = sW;  // the gate cumsum lives where W goes once Kt and QG are formed
    const BwCtx X(a, DK, DV, TIn::bytes);
    Item it;
    if (!item_of(a, static_cast<const char*>(a.workspace), X.ft, blockIdx.x, it)) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, H = a.H, item = blockIdx.x;
    const int tb = wave & 3, part = wave >> 2;
    {
        Rows<TIn, DK, kTP> rk, rq;
        Rows<TIn, DV, kTP> ro;
        Rows<F32, DK, kTP> rg;
        Mat<kC, kC, kTP> rp;
        rk.fetch(a.k, it, H);
        rq.fetch(a.q, it, H);
        ro.fetch(b.dout, it, H);
        rg.fetch(a.g, it, H);
        rp.fetch(X.blk(item, X.bw.P), kC);
        const float gv = threadIdx.x < DK ? X.blk(item, X.bw.gl)[threadIdx.x] : 0.f;
        rk.store(sK, LK);
        rq.store(sQ, LK);
        ro.store(sO, LV);
        rg.store(sG, LK);
        rp.store(sP, LC);
        if (threadIdx.x < DK) sgl[threadIdx.x] = gv;
    }
    gate_scan<DK, kTP>(sG, LK);
    lds_barrier();
    // W goes where the gate cumsum is until Kt and QG are formed: its loads stay in flight
    // (registers) until then
    f32x4 rW[MatCopy<kC, DK, kTP>::N];
    g2r<kC, DK, kTP>(X.blk(item, X.bw.W), DK, rW);
    normalize_rows<kTP>(sK, LK, DK, inv, a.use_l2);
    normalize_rows<kTP>(sQ, LK, DK, inv, a.use_l2);
    to_kt<DK, kTP>(sK, sG, LK);
    to_qg<DK, kTP>(sQ, sG, LK);
    lds_barrier();
    r2s<kC, DK, kTP>(rW, sW, LK);
    lds_barrier();
    // Mt (dk x dk): tile (rb, cb), rows c = W's columns, k over tokens
    float* Mt = X.blk(item, X.bw.Mt);
    for (int tI = wave; tI < (DK / 16) * (DK / 16); tI += NW) {
        const int rb = tI / (DK / 16), cb = tI % (DK / 16);
        f32x4 m = mm16(sW + 16 * rb, 1, LK, sK + 16 * cb, LK, 1, kC, lane, f32x4{0.f, 0.f, 0.f, 0.f});
        const int r = lane & 15, q = lane >> 4;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int row = 16 * rb + 4 * q + ii, col = 16 * cb + r;
            m[ii] = (row == col ? sgl[row] : 0.f) - m[ii];
        }
        put_tile(Mt, DK, rb, cb, m, lane);
    }
    // Q' = QG - P W in place over QG: wave (tb, part) takes token block tb and a quarter of the
    // channel tiles (only it reads or writes those tiles of sQ here)
    for (int i = 0; i < NQ; ++i) {
        const int cb = NQ * part + i;
        const f32x4 pw = mm16(sP + 16 * tb * LC, LC, 1, sW + 16 * cb, LK, 1, kC, lane, f32x4{0.f, 0.f, 0.f, 0.f});
        put_tile(sQ, LK, tb, cb, get_tile(sQ, LK, tb, cb, lane) - pw, lane);
    }
    lds_barrier();
    // b = scale Q'^T dO (dk x dv)
    float* bb = X.blk(item, X.bw.b);
    for (int tI = wave; tI < (DK / 16) * (DV / 16); tI += NW) {
        const int rb = tI / (DV / 16), cb = tI % (DV / 16);
        const f32x4 v = mm16(sQ + 16 * rb, 1, LK, sO + 16 * cb, LV, 1, kC, lane, f32x4{0.f, 0.f, 0.f, 0.f});
        put_tile(bb, DV, rb, cb, v * a.scale, lane);
    }
}

// ---------------------------------------------------------------------------
// 4. bwd_scan: per (sequence, head, 16-column tile), from the last chunk back:
//    dX_c = X (the gradient of chunk c's exit state), X <- Mt_c X + b_c; dh0 = X.
//    DK / 16 waves, wave w owns rows 16 w .. 16 w + 15.
// ---------------------------------------------------------------------------
template <int DK, int DV>
__global__ __launch_bounds__(64 * (DK / 16)) void bwd_scan_kernel(BackwardArgs b, int e) {
    const PrefillArgs& a = b.fwd;
    constexpr int NTS = DV / 16, LX = DK + 4;
    // X^T [16 columns][DK], double-buffered by step parity: a step writes one buffer while no
    // wave can still be reading it (its last reads were before the previous step's barrier),
    // so each step needs one barrier
    __shared__ __attribute__((aligned(16))) float xs2[2][16 * LX];
    const BwCtx X(a, DK, DV, e);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 15, q4 = 4 * (lane >> 4);
    // The NTS column tiles of one (sequence, head) read the same Mt: their block ids are
    // congruent mod kXcd, so they run on one XCD and read each Mt from its L2 (round-robin
    // dispatch over the XCDs by block id); the grid is padded to whole groups of kXcd.
    const int H = a.H, j = blockIdx.x / kXcd, tile = j % NTS, grp = (j / NTS) * kXcd + blockIdx.x % kXcd;
    const int seq = grp / H, h = grp % H;
    if (seq >= a.num_seqs) return;
    const int c0 = X.ft.chunk_off[seq], nch = X.ft.chunk_off[seq + 1] - c0;
    const int col = 16 * tile + r;
    const size_t SZ = static_cast<size_t>(DK) * DV;
    f32x4 x;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
        x[rr] = b.dht ? b.dht[(static_cast<size_t>(seq) * H + h) * SZ + (16 * wave + q4 + rr) * DV + col] : 0.f;
    // Mt rows and b of a chunk for this wave, loaded two chunks ahead of their use (the three
    // operand sets rotate by name, the loop unrolled three times, so no copy waits for loads
    // still in flight)
    struct Ops {
        f32x4 mt[DK / 16], bb;
    };
    auto load = [&](Ops& o, int c) {
        const int item = (c0 + c) * H + h;
        const float* Mt = X.blk(item, X.bw.Mt);
        const float* bb = X.blk(item, X.bw.b);
#pragma unroll
        for (int kb = 0; kb < DK / 16; ++kb)
            o.mt[kb] = *reinterpret_cast<const f32x4*>(Mt + (16 * wave + r) * DK + 16 * kb + q4);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) o.bb[rr] = bb[(16 * wave + q4 + rr) * DV + col];
    };
    auto step = [&](int c, const Ops& cur, Ops& fill) {
        if (c < 0) return false;
        float* dX = X.blk((c0 + c) * H + h, X.bw.dX);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) dX[(16 * wave + q4 + rr) * DV + col] = x[rr];
        load(fill, c >= 2 ? c - 2 : 0);  // (a valid chunk when none is left)
        float* xs = xs2[c & 1];
        *reinterpret_cast<f32x4*>(xs + r * LX + 16 * wave + q4) = x;
        // LDS-only barrier: a __syncthreads() would also wait for the loads just issued
        lds_barrier();
        // lane (r, q) supplies k = 16 kb + 4q + ks of Mt row 16 wave + r and of X column r;
        // one accumulator (the matrix core accumulates back to back into the same registers)
        f32x4 acc = cur.bb;
#pragma unroll
        for (int kb = 0; kb < DK / 16; ++kb) {
            const f32x4 xb = *reinterpret_cast<const f32x4*>(xs + r * LX + 16 * kb + q4);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(cur.mt[kb][ks], xb[ks], acc, 0, 0, 0);
        }
        x = acc;
        return true;
    };
    if (nch > 0) {
        Ops o0, o1, o2;
        load(o0, nch - 1);
        load(o1, nch >= 2 ? nch - 2 : 0);
        // whole groups of three steps with no exit inside the loop body, the last zero to two
        // chunks after it: with exits between the steps the compiler's load-wait placement
        // gave up on the two-ahead distance and waited for every load in flight
        int c = nch - 1;
        for (; c >= 2; c -= 3) {
            step(c, o0, o2);
            step(c - 1, o1, o0);
            step(c - 2, o2, o1);
        }
        if (c >= 0) step(c, o0, o2);
        if (c >= 1) step(c - 1, o1, o0);
    }
    if (b.dh0) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
            b.dh0[(static_cast<size_t>(seq) * H + h) * SZ + (16 * wave + q4 + rr) * DV + col] = x[rr];
    }
}

// ---------------------------------------------------------------------------
// 5. bwd_state: U = Ut - W S, dU = scale P^T dO + Kt dX; dQG = scale dO S^T, dW = -dU S^T,
//    dKt = U dX^T, dP = scale dO U^T (s <= t); dgl = e^(G_L) sum_j S dX.  Over 32-column
//    blocks of S and dX.  Eight waves (two per SIMD): wave w owns token block w & 3 of every
//    output, and half w >> 2 of its column tiles.
// ---------------------------------------------------------------------------
constexpr int kVB = 32;
constexpr int kTS = 512;  // threads of bwd_state
template <int DK, int DV, class TIn>
__global__ __launch_bounds__(kTS) void bwd_state_kernel(BackwardArgs b) {
    const PrefillArgs& a = b.fwd;
    constexpr int LK = DK + 4, LC = kC + 4, LB = kVB + 4;
    constexpr int NKB = DK / 16, HK = NKB / 2;  // dk tiles, per half
    __shared__ __attribute__((aligned(16))) float sW[kC * LK], sK[kC * LK], sP[kC * LC], sS[DK * LB], sX[DK * LB], sO[kC * LB],
        sU[kC * LB], sdU[kC * LB], inv[kC], sgl[DK];
    float* sG = sW;
    const BwCtx X(a, DK, DV, TIn::bytes);
    Item it;
    if (!item_of(a, static_cast<const char*>(a.workspace), X.ft, blockIdx.x, it)) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, H = a.H, item = blockIdx.x;
    const int tb = wave & 3, half = wave >> 2;
    const int r = lane & 15, q = lane >> 4;
    {
        Rows<TIn, DK, kTS> rk;
        Rows<F32, DK, kTS> rg;
        Mat<kC, kC, kTS> rp;
        rk.fetch(a.k, it, H);
        rg.fetch(a.g, it, H);
        rp.fetch(X.blk(item, X.bw.P), kC);
        rk.store(sK, LK);
        rg.store(sG, LK);
        rp.store(sP, LC);
    }
    // W goes where the gate cumsum is once Kt is formed: its loads go out once the opening
    // operands are stored and stay in flight (registers) through the scan and the norms
    Mat<kC, DK, kTS> rw;
    rw.fetch(X.blk(item, X.bw.W), DK);
    gate_scan<DK, kTS>(sG, LK);
    lds_barrier();
    normalize_rows<kTS>(sK, LK, DK, inv, a.use_l2);
    to_kt<DK, kTS>(sK, sG, LK);
    lds_barrier();
    rw.store(sW, LK);
    if (threadIdx.x < DK) sgl[threadIdx.x] = 0.f;
    const float* S = X.blk(item, X.bw.S);
    const float* dX = X.blk(item, X.bw.dX);
    const float* Ut = X.blk(item, X.bw.Ut);
    float* dUg = X.blk(item, X.bw.dU);
    f32x4 dqg[HK], dw[HK], dkt[HK], dp[2];
    for (int i = 0; i < HK; ++i) dqg[i] = dw[i] = dkt[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < 2; ++i) dp[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    // a column block's S, dX, Ut and dO: loaded into registers one block ahead (during the
    // previous block's contractions), stored to LDS at the block's start
    f32x4 rS[MatCopy<DK, kVB, kTS>::N], rX[MatCopy<DK, kVB, kTS>::N], rU[MatCopy<kC, kVB, kTS>::N];
    u32x4 rO[RowCopy<TIn, kVB, kTS>::N];
    auto fetch = [&](int jb) {
        g2r<DK, kVB, kTS>(S + kVB * jb, DV, rS);
        g2r<DK, kVB, kTS>(dX + kVB * jb, DV, rX);
        rows_fetch<TIn, DV, kVB, kTS>(b.dout, rO, it, H, kVB * jb);
        g2r<kC, kVB, kTS>(Ut + kVB * jb, DV, rU);
    };
    fetch(0);
    for (int jb = 0; jb < DV / kVB; ++jb) {
        lds_barrier();
        r2s<DK, kVB, kTS>(rS, sS, LB);
        r2s<DK, kVB, kTS>(rX, sX, LB);
        rows_store<TIn, kVB, kTS>(rO, sO, LB);
        r2s<kC, kVB, kTS>(rU, sU, LB);
        if (jb + 1 < DV / kVB) fetch(jb + 1);
        lds_barrier();
        // U and dU of this wave's token block and column tile (one of the block's two); each
        // wave reads and writes only its own tile of sU and sdU here
        {
            const int cb = half;
            const f32x4 ws = mm16(sW + 16 * tb * LK, LK, 1, sS + 16 * cb, LB, 1, DK, lane, f32x4{0.f, 0.f, 0.f, 0.f});
            const f32x4 u = get_tile(sU, LB, tb, cb, lane) - ws;
            f32x4 du = mm16(sP + 16 * tb, 1, LC, sO + 16 * cb, LB, 1, kC, lane, f32x4{0.f, 0.f, 0.f, 0.f}) * a.scale;
            du = mm16(sK + 16 * tb * LK, LK, 1, sX + 16 * cb, LB, 1, DK, lane, du);
            put_tile(sU, LB, tb, cb, u, lane);
            put_tile(sdU, LB, tb, cb, du, lane);
        }
        lds_barrier();
        for_groups<kVB, kTS>([&](int t, int c) {
            *reinterpret_cast<f32x4*>(dUg + t * DV + kVB * jb + c) = *reinterpret_cast<const f32x4*>(sdU + t * LB + c);
        });
        if (threadIdx.x < DK) {
            float s = 0.f;
            for (int j = 0; j < kVB; j += 4) {
                const f32x4 sv = *reinterpret_cast<const f32x4*>(sS + threadIdx.x * LB + j);
                const f32x4 xv = *reinterpret_cast<const f32x4*>(sX + threadIdx.x * LB + j);
#pragma unroll
                for (int e = 0; e < 4; ++e) s = fmaf(sv[e], xv[e], s);
            }
            sgl[threadIdx.x] += s;
        }
        // contractions over this block's columns (k = the block's 32 value columns): the wave's
        // rows of dO, dU and U are read once per 16 k values and serve its half of the output
        // tiles; of every 16 k values lane (r, q) supplies k = 16 s + 4 q + e to step e, so every
        // operand row is read as 16-byte LDS loads
        for (int k0 = 0; k0 < kVB; k0 += 16) {
            const int kb = k0 + 4 * q;
            const f32x4 ao = *reinterpret_cast<const f32x4*>(sO + (16 * tb + r) * LB + kb);
            const f32x4 adu = *reinterpret_cast<const f32x4*>(sdU + (16 * tb + r) * LB + kb);
            const f32x4 au = *reinterpret_cast<const f32x4*>(sU + (16 * tb + r) * LB + kb);
#pragma unroll
            for (int i = 0; i < HK; ++i) {
                const int cb = HK * half + i;
                const f32x4 bs = *reinterpret_cast<const f32x4*>(sS + (16 * cb + r) * LB + kb);
                const f32x4 bx = *reinterpret_cast<const f32x4*>(sX + (16 * cb + r) * LB + kb);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    dqg[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(ao[e], bs[e], dqg[i], 0, 0, 0);
                    dw[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(adu[e], bs[e], dw[i], 0, 0, 0);
                    dkt[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(au[e], bx[e], dkt[i], 0, 0, 0);
                }
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const f32x4 bu = *reinterpret_cast<const f32x4*>(sU + (16 * (2 * half + i) + r) * LB + kb);
#pragma unroll
                for (int e = 0; e < 4; ++e) dp[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(ao[e], bu[e], dp[i], 0, 0, 0);
            }
        }
    }
    float* dQG = X.blk(item, X.bw.dQG);
    float* dW = X.blk(item, X.bw.dW);
    float* dKt = X.blk(item, X.bw.dKt);
    float* dP = X.blk(item, X.bw.dP);
    for (int i = 0; i < HK; ++i) {
        const int cb = HK * half + i;
        put_tile(dQG, DK, tb, cb, dqg[i] * a.scale, lane);
        put_tile(dW, DK, tb, cb, -dw[i], lane);
        put_tile(dKt, DK, tb, cb, dkt[i], lane);
    }
    for (int i = 0; i < 2; ++i) {
        const int sb = 2 * half + i;
        f32x4 v = dp[i] * a.scale;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) v[ii] = 16 * sb + r <= 16 * tb + 4 * q + ii ? v[ii] : 0.f;
        put_tile(dP, kC, tb, sb, v, lane);
    }
    lds_barrier();
    if (threadIdx.x < DK) X.blk(item, X.bw.dgl)[threadIdx.x] = X.blk(item, X.bw.gl)[threadIdx.x] * sgl[threadIdx.x];
}

// ---------------------------------------------------------------------------
// 6. bwd_ut: dT = dW BK^T + dU BV^T, dBK = T^T dW, dBV = T^T dU, dA = -(T^T dT T^T) (s < t);
//    dv = beta dBV, dbeta = sum v dBV + sum kh 2^G dBK + sum_s dA Ag, dAg = beta dA.
// ---------------------------------------------------------------------------
constexpr int kTU = 1024;  // threads of bwd_ut
template <int DK, int DV, class TIn>
__global__ __launch_bounds__(kTU) void bwd_ut_kernel(BackwardArgs b) {
    const PrefillArgs& a = b.fwd;
    constexpr int LK = DK + 4, LV = DV + 4, LC = kC + 4;
    constexpr int LM = LK > LV ? LK : LV;
    __shared__ __attribute__((aligned(16))) float sT[kC * LC], sM1[kC * LM], sM2[kC * LM], sDE[2 * kC * LC], inv[kC], sB[kC],
        sDB[kTU / 256][kC];
    float* sD = sDE;
    float* sE = sDE + kC * LC;
    float* sG = sDE;  // the gate cumsum (DK wide) spans sD and sE while KG is formed
    const BwCtx X(a, DK, DV, TIn::bytes);
    Item it;
    if (!item_of(a, static_cast<const char*>(a.workspace), X.ft, blockIdx.x, it)) return;
    // NP = kTU / 256 waves per token block: wave (tb, pw) takes token block tb (the rows of
    // every output tile) and part pw of its column tiles; dbeta adds the parts' row
    // sums through LDS
    constexpr int NP = kTU / 256, NS = 4 / NP;  // parts, s tiles of a part
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, H = a.H, item = blockIdx.x;
    const int tb = wave & 3, pw = wave >> 2;
    const int r = lane & 15, q = lane >> 4;
    static_assert(2 * kC * LC >= kC * LK, "gate cumsum fits sD + sE");
    // KG = kh 2^G (sM2) and dW (sM1); dW's loads stay in flight (registers) until sM1 is free
    f32x4 rW[MatCopy<kC, DK, kTU>::N];
    {
        Rows<TIn, DK, kTU> rk;
        Rows<F32, DK, kTU> rg;
        Mat<kC, kC, kTU> rt;
        rk.fetch(a.k, it, H);
        rg.fetch(a.g, it, H);
        rt.fetch(X.blk(item, X.bw.T), kC);
        g2r<kC, DK, kTU>(X.blk(item, X.bw.dW), DK, rW);
        const float bt = threadIdx.x < it.L ? a.beta[static_cast<int64_t>(it.t0 + threadIdx.x) * H + it.h] : 0.f;
        rk.store(sM2, LK);
        rg.store(sG, LK);
        rt.store(sT, LC);
        if (threadIdx.x < kC) sB[threadIdx.x] = bt;
    }
    gate_scan<DK, kTU>(sG, LK);
    lds_barrier();
    normalize_rows<kTU>(sM2, LK, DK, inv, a.use_l2);
    to_qg<DK, kTU>(sM2, sG, LK);  // kh 2^G
    r2s<kC, DK, kTU>(rW, sM1, LK);
    lds_barrier();
    // v and dU load during the dT and dBK products
    u32x4 rV[RowCopy<TIn, DV, kTU>::N];
    f32x4 rU[MatCopy<kC, DV, kTU>::N];
    rows_fetch<TIn, DV, DV, kTU>(a.v, rV, it, H);
    g2r<kC, DV, kTU>(X.blk(item, X.bw.dU), DV, rU);
    // dT (part 1: dW BK^T, BK = beta KG, so column s takes beta_s; this wave's tiles (tb, sb),
    // sb = NS pw .. NS pw + NS - 1) and dBK of its rows; dbeta part sum_c KG dBK
    f32x4 dT[NS];
    for (int i = 0; i < NS; ++i) {
        const int sb = NS * pw + i;
        dT[i] = mm16(sM1 + 16 * tb * LK, LK, 1, sM2 + 16 * sb * LK, 1, LK, DK, lane, f32x4{0.f, 0.f, 0.f, 0.f}) *
                sB[16 * sb + r];
    }
    float* dBK = X.blk(item, X.bw.dBK);
    float part[4] = {0.f, 0.f, 0.f, 0.f};
    for (int cb = pw * (DK / 16 / NP); cb < (pw + 1) * (DK / 16 / NP); ++cb) {
        const f32x4 v = mm16(sT + 16 * tb, 1, LC, sM1 + 16 * cb, LK, 1, kC, lane, f32x4{0.f, 0.f, 0.f, 0.f});
        put_tile(dBK, DK, tb, cb, v, lane);
        const f32x4 kg = get_tile(sM2, LK, tb, cb, lane);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) part[ii] = fmaf(kg[ii], v[ii], part[ii]);
    }
    lds_barrier();
    // BV = beta v (sM2) and dU (sM1)
    rows_store<TIn, DV, kTU>(rV, sM2, LV);
    r2s<kC, DV, kTU>(rU, sM1, LV);
    lds_barrier();
    // the raw v stays in sV (over sD and sE, free until dT goes there) for the dbeta part
    float* sV = sDE;
    static_assert(kC * LV <= 2 * kC * LC, "v fits sD + sE");
    for_groups<DV, kTU>([&](int t, int c) {
        f32x4* x = reinterpret_cast<f32x4*>(sM2 + t * LV + c);
        const f32x4 raw = *x;
        *reinterpret_cast<f32x4*>(sV + t * LV + c) = raw;
        *x = raw * sB[t];
    });
    lds_barrier();
    for (int i = 0; i < NS; ++i)
        dT[i] = mm16(sM1 + 16 * tb * LV, LV, 1, sM2 + 16 * (NS * pw + i) * LV, 1, LV, DV, lane, dT[i]);
    // dBV = T^T dU: dv = beta dBV, dbeta part sum_j v dBV
    for (int cb = pw * (DV / 16 / NP); cb < (pw + 1) * (DV / 16 / NP); ++cb) {
        const f32x4 v = mm16(sT + 16 * tb, 1, LC, sM1 + 16 * cb, LV, 1, kC, lane, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int t = 16 * tb + 4 * q + ii, j = 16 * cb + r;
            part[ii] = fmaf(sV[t * LV + j], v[ii], part[ii]);  // rows past the end: v = 0
            if (t < it.L) st_out(b.dv, (static_cast<int64_t>(it.t0 + t) * H + it.h) * DV + j, sB[t] * v[ii], TIn{});
        }
    }
    // this wave's rows of Ag for the dbeta part of dA (global), loaded during E
    const float* Ag = X.blk(item, X.bw.Ag);
    f32x4 agt[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) agt[i] = get_tile(Ag, kC, tb, NS * pw + i, lane);
    lds_barrier();  // every wave's reads of sV precede the dT stores over it
    // dT to LDS; E = T^T dT; dA = -(E T^T) (s < t)
    for (int i = 0; i < NS; ++i) put_tile(sD, LC, tb, NS * pw + i, dT[i], lane);
    lds_barrier();
    for (int i = 0; i < NS; ++i) {
        const int sb = NS * pw + i;
        put_tile(sE, LC, tb, sb, mm16(sT + 16 * tb, 1, LC, sD + 16 * sb, LC, 1, kC, lane, f32x4{0.f, 0.f, 0.f, 0.f}), lane);
    }
    lds_barrier();
    float* dAg = X.blk(item, X.bw.dAg);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        const int sb = NS * pw + i;
        f32x4 v = mm16(sE + 16 * tb * LC, LC, 1, sT + 16 * sb * LC, 1, LC, kC, lane, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int t = 16 * tb + 4 * q + ii, s = 16 * sb + r;
            const float da = s < t ? -v[ii] : 0.f;
            part[ii] = fmaf(da, agt[i][ii], part[ii]);
            v[ii] = sB[t] * da;
        }
        put_tile(dAg, kC, tb, sb, v, lane);
    }
    // dbeta: reduce the partial sums over the 16 lanes of each row group, then add the parts
    // (in the same order for every row)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
        float x = part[ii];
        x += __shfl_xor(x, 1, 64);
        x += __shfl_xor(x, 2, 64);
        x += __shfl_xor(x, 4, 64);
        x += __shfl_xor(x, 8, 64);
        if (r == 0) sDB[pw][16 * tb + 4 * q + ii] = x;
    }
    lds_barrier();
    if (threadIdx.x < it.L) {
        float x = sDB[0][threadIdx.x];
#pragma unroll
        for (int pp = 1; pp < NP; ++pp) x += sDB[pp][threadIdx.x];
        b.dbeta[static_cast<int64_t>(it.t0 + threadIdx.x) * H + it.h] = x;
    }
}

// ---------------------------------------------------------------------------
// 7. bwd_final: X1..X4, dkh, dqh, dG, reverse cumsum, norm backward; dq, dk, dg.
//    Eight waves: wave (tb, half) owns token block tb (rows of every output tile) and half of
//    the channel tiles.
// ---------------------------------------------------------------------------
constexpr int kTF = 512;  // threads of bwd_final
template <int DK, int DV, class TIn>
__global__ __launch_bounds__(kTF) void bwd_final_kernel(BackwardArgs b) {
    const PrefillArgs& a = b.fwd;
    constexpr int LK = DK + 4, LC = kC + 4, NKB = DK / 16, NH = NKB / 2;
    __shared__ __attribute__((aligned(16))) float sK[kC * LK], sQ[kC * LK], sG[kC * LK], sA[kC * LC], sP[kC * LC], iq[kC], ik[kC], sB[kC],
        sGL[DK], sNB[2][2][kC];
    const BwCtx X(a, DK, DV, TIn::bytes);
    Item it;
    if (!item_of(a, static_cast<const char*>(a.workspace), X.ft, blockIdx.x, it)) return;
    // eight waves (two per SIMD): wave (tb, half) takes token block tb and half of the channel
    // tiles of every per-row result
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, H = a.H, item = blockIdx.x;
    const int tb = wave & 3, half = wave >> 2, cb0 = NH * half;
    const int r = lane & 15, q = lane >> 4;
    {
        Rows<TIn, DK, kTF> rk, rq;
        Rows<F32, DK, kTF> rg;
        Mat<kC, kC, kTF> ra, rp;
        rk.fetch(a.k, it, H);
        rq.fetch(a.q, it, H);
        rg.fetch(a.g, it, H);
        ra.fetch(X.blk(item, X.bw.dAg), kC);
        rp.fetch(X.blk(item, X.bw.dP), kC);
        const float bt = threadIdx.x < it.L ? a.beta[static_cast<int64_t>(it.t0 + threadIdx.x) * H + it.h] : 0.f;
        rk.store(sK, LK);
        rq.store(sQ, LK);
        rg.store(sG, LK);
        ra.store(sA, LC);
        rp.store(sP, LC);
        if (threadIdx.x < kC) sB[threadIdx.x] = bt;
    }
    gate_scan<DK, kTF>(sG, LK);
    lds_barrier();
    normalize_rows<kTF>(sK, LK, DK, ik, a.use_l2);
    normalize_rows<kTF>(sQ, LK, DK, iq, a.use_l2);
    const float* dBK = X.blk(item, X.bw.dBK);
    const float* dQG = X.blk(item, X.bw.dQG);
    const float* dKt = X.blk(item, X.bw.dKt);
    // per channel tile of this wave: dkh, dqh and dG of its 16 rows
    f32x4 dkh[NH], dqh[NH], dG[NH];
    float ktdkt[NH];  // sum over this lane's rows of Kt dKt (for dG_L)
    // the channel tile's dBK, dQG and dKt (global) are loaded one tile ahead
    f32x4 nbk = get_tile(dBK, DK, tb, cb0, lane), nqg = get_tile(dQG, DK, tb, cb0, lane);
    f32x4 nkt = get_tile(dKt, DK, tb, cb0, lane);
#pragma unroll 1
    for (int i = 0; i < NH; ++i) {
        const int cb = cb0 + i;
        const f32x4 dbk = nbk, dqg = nqg, dkt = nkt;
        if (i + 1 < NH) {
            nbk = get_tile(dBK, DK, tb, cb + 1, lane);
            nqg = get_tile(dQG, DK, tb, cb + 1, lane);
            nkt = get_tile(dKt, DK, tb, cb + 1, lane);
        }
        f32x4 x1, x2, x3, x4;
        dtok_pair<true, true>(sA, sP, LC, sK, sK, sG, LK, tb, cb, lane, x1, x4);
        dtok_pair<false, false>(sA, sP, LC, sK, sQ, sG, LK, tb, cb, lane, x2, x3);
        const int c = 16 * cb + r;
        const float gL = sG[(kC - 1) * LK + c];
        ktdkt[i] = 0.f;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int t = 16 * tb + 4 * q + ii;
            const float kh = sK[t * LK + c], qh = sQ[t * LK + c], Gt = sG[t * LK + c];
            const float eg = ex2(Gt), el = ex2(gL - Gt);
            const float bk = sB[t] * kh * eg, kt = kh * el, qg = qh * eg;
            dkh[i][ii] = sB[t] * eg * dbk[ii] + el * dkt[ii] + x1[ii] + x2[ii] + x3[ii];
            dqh[i][ii] = eg * dqg[ii] + x4[ii];
            dG[i][ii] = qg * dqg[ii] + bk * dbk[ii] - kt * dkt[ii] + kh * (x1[ii] - x2[ii] - x3[ii]) + qh * x4[ii];
            ktdkt[i] = fmaf(kt, dkt[ii], ktdkt[i]);
        }
    }
    // norm backward: row dot products over this wave's channel tiles and the 16 lanes of a row
    // group, then the two halves' sums added through LDS (in the same order by both)
    float pq[4], pk[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
        float x = 0.f, y = 0.f;
        for (int i = 0; i < NH; ++i) {
            const int t = 16 * tb + 4 * q + ii, c = 16 * (cb0 + i) + r;
            x = fmaf(sQ[t * LK + c], dqh[i][ii], x);
            y = fmaf(sK[t * LK + c], dkh[i][ii], y);
        }
        for (int m = 1; m < 16; m <<= 1) {
            x += __shfl_xor(x, m, 64);
            y += __shfl_xor(y, m, 64);
        }
        if (r == 0) {
            sNB[half][0][16 * tb + 4 * q + ii] = x;
            sNB[half][1][16 * tb + 4 * q + ii] = y;
        }
    }
    lds_barrier();
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
        const int t = 16 * tb + 4 * q + ii;
        pq[ii] = sNB[0][0][t] + sNB[1][0][t];
        pk[ii] = sNB[0][1][t] + sNB[1][1][t];
    }
    for (int i = 0; i < NH; ++i) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int t = 16 * tb + 4 * q + ii, c = 16 * (cb0 + i) + r;
            if (t < it.L) {
                const int64_t o = (static_cast<int64_t>(it.t0 + t) * H + it.h) * DK + c;
                const float vq = a.use_l2 ? iq[t] * (dqh[i][ii] - sQ[t * LK + c] * pq[ii]) : dqh[i][ii];
                const float vk = a.use_l2 ? ik[t] * (dkh[i][ii] - sK[t * LK + c] * pk[ii]) : dkh[i][ii];
                st_out(b.dq, o, vq, TIn{});
                st_out(b.dk, o, vk, TIn{});
            }
        }
    }
    // dG_L = dgl + sum_t Kt dKt: the per-lane sums reduced over q (the 4 row groups of a wave)
    // and over the waves through LDS
    lds_barrier();  // sG's values are no longer read below this point
    if (threadIdx.x < DK) sGL[threadIdx.x] = X.blk(item, X.bw.dgl)[threadIdx.x];
    lds_barrier();
    for (int i = 0; i < NH; ++i) {
        float x = ktdkt[i];
        x += __shfl_xor(x, 16, 64);
        x += __shfl_xor(x, 32, 64);
        if (q == 0) atomicAdd(&sGL[16 * (cb0 + i) + r], x);
    }
    // dG into sG (rows of this wave's token block), then the reverse cumsum per channel plus dG_L
    for (int i = 0; i < NH; ++i) put_tile(sG, LK, tb, cb0 + i, dG[i], lane);
    lds_barrier();
    // suffix sums over the live rows (lane = token): total - inclusive prefix + own value; a
    // wave takes four adjacent columns per pass (one 16-byte LDS access per lane)
    for (int c = 4 * wave; c < DK; c += 4 * (kTF / 64)) {
        f32x4* p = reinterpret_cast<f32x4*>(sG + lane * LK + c);
        const f32x4 v4 = *p;
        f32x4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float v = lane < it.L ? v4[e] : 0.f;
            const float incl = wave_prefix64(v);
            const float tot = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(incl), 63));
            o4[e] = (tot - incl + v) + sGL[c + e];
        }
        *p = o4;
    }
    lds_barrier();
    for_groups<DK, kTF>([&](int t, int c) {
        if (t < it.L)
            *reinterpret_cast<f32x4*>(b.dg + (static_cast<int64_t>(it.t0 + t) * H + it.h) * DK + c) =
                *reinterpret_cast<const f32x4*>(sG + t * LK + c);
    });
}

template <int DK, int DV, class TIn>
hipError_t launch_backward_t(const BackwardArgs& b, hipStream_t stream) {
    constexpr int E = TIn::bytes;
    const PrefillArgs& a = b.fwd;
    const BwLayout bw(a.num_seqs, a.total_tokens, a.H, DK, DV, E);
    // 0: initial states and slots for the forward pass
    const int64_t n0 = static_cast<int64_t>(a.num_seqs) * a.H * DK * DV;
    const int g0 = static_cast<int>(n0 / kT + 1 < 4096 ? n0 / kT + 1 : 4096);
    hipLaunchKernelGGL(bwd_init_kernel, dim3(g0), dim3(kT), 0, stream, b, DK, DV, E);
    // 1: the forward with chunk states
    hipError_t err = launch_prefill(a, E == 2, DK, DV, stream);
    if (err != hipSuccess) return err;
    const dim3 grid(static_cast<unsigned>(bw.max_items));
    if (bw.max_items > 0) {
        hipLaunchKernelGGL((bwd_intra_kernel<DK, DV, TIn>), grid, dim3(kTI), 0, stream, b);
        hipLaunchKernelGGL((bwd_prep_kernel<DK, DV, TIn>), grid, dim3(kTP), 0, stream, b);
    }
    const int sgroups = (a.num_seqs * a.H + kXcd - 1) / kXcd;
    hipLaunchKernelGGL((bwd_scan_kernel<DK, DV>), dim3(static_cast<unsigned>(sgroups) * kXcd * (DV / 16)),
                       dim3(64 * (DK / 16)), 0, stream, b, E);
    if (bw.max_items > 0) {
        hipLaunchKernelGGL((bwd_state_kernel<DK, DV, TIn>), grid, dim3(kTS), 0, stream, b);
        hipLaunchKernelGGL((bwd_ut_kernel<DK, DV, TIn>), grid, dim3(kTU), 0, stream, b);
        hipLaunchKernelGGL((bwd_final_kernel<DK, DV, TIn>), grid, dim3(kTF), 0, stream, b);
    }
    return hipGetLastError();
}

template <class TIn>
hipError_t launch_backward_dt(const BackwardArgs& b, int dk, int dv, hipStream_t stream) {
    if (dk == 128 && dv == 128) return launch_backward_t<128, 128, TIn>(b, stream);
    if (dk == 128 && dv == 64) return launch_backward_t<128, 64, TIn>(b, stream);
    if (dk == 64 && dv == 128) return launch_backward_t<64, 128, TIn>(b, stream);
    if (dk == 64 && dv == 64) return launch_backward_t<64, 64, TIn>(b, stream);
    return hipErrorInvalidValue;
}

}  // namespace

size_t backward_workspace_bytes(int num_seqs, int64_t total_tokens, int H, int dk, int dv, int bf16) {
    return BwLayout(num_seqs, total_tokens, H, dk, dv, bf16 ? 2 : 4).total;
}

// Points the forward pass of a backward call at its part of the workspace.
void backward_setup(BackwardArgs& b, int dk, int dv, int bf16) {
    const BwLayout bw(b.fwd.num_seqs, b.fwd.total_tokens, b.fwd.H, dk, dv, bf16 ? 2 : 4);
    char* base = static_cast<char*>(b.fwd.workspace);
    b.fwd.pool = reinterpret_cast<float*>(base + bw.off_pool);
    b.fwd.slot_idx = reinterpret_cast<const int32_t*>(base + bw.off_slots);
    b.fwd.h0_from_pool = 1;
    b.fwd.o = nullptr;  // the forward pass keeps only the chunk states
    b.fwd.chunk_states = reinterpret_cast<float*>(base + bw.off_items + bw.S);
    b.fwd.chunk_state_stride = bw.item / sizeof(float);
}

hipError_t launch_backward(const BackwardArgs& b, int bf16, int dk, int dv, hipStream_t stream) {
    return bf16 ? launch_backward_dt<BF16>(b, dk, dv, stream) : launch_backward_dt<F32>(b, dk, dv, stream);
}

}  // namespace kda
