// kda_prefill.hip -- varlen chunked prefill of the KDA recurrence for gfx950.
//
// The Kimi K3 day-0 adaptation page (section "融合算子加速：KDA Prefill与Decode双路径")
// gives the prefill path as 64-token chunks with Q/K normalisation, gate
// cumulation and the chunk recurrence organised as batched work.  The chunk
// algebra used here (derived from the token recurrence; for a chunk of L <= 64
// tokens entering with state S0, G = inclusive cumulative sum of g inside the
// chunk):
//
//   A_ts = beta_t sum_c kh_tc kh_sc exp(G_tc - G_sc)   (s < t)     "KK^T" with decay
//   P_ts =        sum_c qh_tc kh_sc exp(G_tc - G_sc)   (s <= t)    "QK^T" with decay
//   T = (I + A)^-1,  W = T diag(beta) kh exp(G),  Ut = T diag(beta) V   (UT transform)
//   U  = Ut - W S0
//   O  = scale (QG S0 + P U),   QG = qh exp(G)
//   S  = diag(exp(G_L)) S0 + (kh exp(G_L - G))^T U
//
// Five launches on the caller's stream:
//   1. chunk_map    cu_seqlens -> per-sequence chunk and segment offsets, the chunk
//                   table (sequence, first token, length; chunks restart at every
//                   sequence start, the last one may be short) and the segment table.
//   2. chunk_intra  persistent, two workgroups per CU walking the (chunk, head) items:
//                   Q/K norm, gate cumsum (DPP scan), A and P on MFMA, T by blocked
//                   substitution in fp32, W and Ut on MFMA; writes W, QG, Kt =
//                   (kh exp(G_L - G))^T, Ut, P and exp(G_L) to a per-(chunk, head)
//                   workspace record.
//   3. seg_carry<LOCAL>  the chunk map is affine in S, so a segment of chunks maps its
//                   entering state to Phi S_start + S_loc: per (segment, head), the chunk
//                   steps on [S | Phi] from [0 | I] (section 3 below).
//   4. seg_scan     per (sequence, head, 16-column tile): S_start(k + 1) = Phi_k
//                   S_start(k) + S_loc(k) in fp32, from the initial state.
//   5. seg_carry<OUT>  per (segment, head): the chunk steps from S_start, writing O and,
//                   for a sequence's last segment, the final state to its slot.
// Every product of the carries is on MFMA with the fp32 state in registers.
//
// The record is stored in the carries' MFMA fragment order ("granules": the 16
// bytes one lane feeds one MFMA k-step, 64 lanes contiguous), so every carry
// load is a contiguous 1 KiB per wave, and the chunk_intra kernel produces most
// granules straight from its MFMA accumulators: a 16x16 accumulator tile holds
// four consecutive rows of one column per lane, which is the operand layout of
// the next product over that dimension when the k index of both operands is
// permuted the same way (two tiles per bf16 granule, one per fp32 granule).
//
// A and P are MFMA products of 16x16 tiles whose exp(G_t - G_s) factor is split
// at a reference inside the tile's span, so both factors stay bounded: an
// off-diagonal tile (t and s in different 16-token blocks) splits at the end of
// the block before t's, where both factors are at most 1; a diagonal tile at its
// block's 8th token, so each factor covers at most 8 tokens' gates.  The only
// range limit left: per key channel, 8 consecutive tokens' gates must sum to more
// than about -85 (else exp2 overflows inside the diagonal tile).  W, QG, Kt and
// exp(G_L) only use factors at most 1.
//
// MFMA operands are bf16 for bf16 inputs and fp32 for fp32 inputs; with bf16
// inputs the A and P operands are each carried as a high and a low bf16 part
// (three MFMAs per product), so every A and P entry is accurate to about 2^-16 of
// its terms.  Every accumulation, the cumsum and the triangular solve are fp32.
#include <atomic>
#include <mutex>
#include <type_traits>

#include "kda.h"
#include "kda_device.hpp"
#include "kda_internal.hpp"
#include "kda_layout.hpp"

namespace kda {

namespace {

constexpr int kThreads = 256;
constexpr int kCarryBV = 32;  // dv columns per Ut record tile
// chunks of record granules a carry wave holds in registers: with 1, a chunk's granules load
// right after the previous step (measured faster than 2, whose extra registers cost the
// step its batching of LDS operand reads)
constexpr int kCarryNB = 1;
constexpr int kNumXcd = 8;    // MI355X: 8 XCDs, workgroups dispatched round-robin
constexpr float kNormEps = 1e-6f;
constexpr int kBufFlags = 0x00020000;  // raw buffer resource word 3 (gfx9 family)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));


// ---------------------------------------------------------------------------
// Fragment geometry per operand type.  A granule is 16 bytes: 8 bf16 (one
// v_mfma_f32_16x16x32_bf16 k-step) or 4 fp32 (four v_mfma_f32_16x16x4_f32 k-steps).
// In accumulator terms a granule spans CT 16x16 tiles along k.
// ---------------------------------------------------------------------------
template <class TIn>
struct Geo;
template <>
struct Geo<BF16> {
    using elem = uint16_t;
    static constexpr int E = 2;
    static constexpr int GW = 8;  // elements per granule
    static constexpr int CT = 2;  // accumulator tiles per granule
};
template <>
struct Geo<F32> {
    using elem = float;
    static constexpr int E = 4;
    static constexpr int GW = 4;
    static constexpr int CT = 1;
};

// C += A B over one granule (both operands list their k values in the same order).
__device__ __forceinline__ f32x4 gmma(u32x4 a, u32x4 b, f32x4 c, BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 gmma(u32x4 a, u32x4 b, f32x4 c, F32) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[e]), __uint_as_float(b[e]), c, 0, 0, 0);
    return c;
}

// x = hi + lo, both bf16 granules (hi = x rounded to bf16, lo = the remainder rounded),
// so hi*hi + hi*lo + lo*hi carries about 16 bits of each product; fp32 keeps x in hi.
__device__ __forceinline__ u32x4 f32_to_gran(const float* x, BF16);
__device__ __forceinline__ u32x4 f32_to_gran(const float* x, F32);
__device__ __forceinline__ void gran_to_f32(u32x4 g, float* x, BF16);
__device__ __forceinline__ void split_gran(const float* x, u32x4& hi, u32x4& lo, BF16 tag) {
    hi = f32_to_gran(x, tag);
    float h[8];
    gran_to_f32(hi, h, tag);
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = x[e] - h[e];
    lo = f32_to_gran(h, tag);
}
__device__ __forceinline__ void split_gran(const float* x, u32x4& hi, u32x4& lo, F32 tag) {
    hi = f32_to_gran(x, tag);
    lo = hi;
}
// C += A B with both operands as (hi, lo) pairs: three bf16 MFMAs, one fp32 granule product.
__device__ __forceinline__ f32x4 smma(u32x4 ah, u32x4 al, u32x4 bh, u32x4 bl, f32x4 c, BF16 tag) {
    c = gmma(ah, bh, c, tag);
    c = gmma(ah, bl, c, tag);
    return gmma(al, bh, c, tag);
}
__device__ __forceinline__ f32x4 smma(u32x4 ah, u32x4, u32x4 bh, u32x4, f32x4 c, F32 tag) {
    return gmma(ah, bh, c, tag);
}

// Accumulator tiles -> granule: bf16 packs 4 values of each of two tiles, fp32
// takes one tile.
__device__ __forceinline__ u32x4 tiles_to_gran(f32x4 t0, f32x4 t1, BF16) {
    return u32x4{pack_bf16x2(t0[0], t0[1]), pack_bf16x2(t0[2], t0[3]), pack_bf16x2(t1[0], t1[1]),
                 pack_bf16x2(t1[2], t1[3])};
}
__device__ __forceinline__ u32x4 tiles_to_gran(f32x4 t0, f32x4, F32) {
    return u32x4{__float_as_uint(t0[0]), __float_as_uint(t0[1]), __float_as_uint(t0[2]), __float_as_uint(t0[3])};
}

// Granule <-> GW fp32 values.
__device__ __forceinline__ void gran_to_f32(u32x4 g, float* x, BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(g[i] << 16);
        x[2 * i + 1] = __uint_as_float(g[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void gran_to_f32(u32x4 g, float* x, F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(g[i]);
}
__device__ __forceinline__ u32x4 f32_to_gran(const float* x, BF16) {
    return u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
}
__device__ __forceinline__ u32x4 f32_to_gran(const float* x, F32) {
    return u32x4{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])};
}

// Four consecutive elements to LDS: 8 bytes (bf16) or 16 bytes (fp32).
__device__ __forceinline__ void lds_store4(uint16_t* p, float x0, float x1, float x2, float x3) {
    *reinterpret_cast<u32x2*>(p) = u32x2{pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
}
__device__ __forceinline__ void lds_store4(float* p, float x0, float x1, float x2, float x3) {
    *reinterpret_cast<f32x4*>(p) = f32x4{x0, x1, x2, x3};
}

// One MFMA k-step with both operands read from LDS in the natural order
// (row r = lane % 16, k contiguous): bf16 16 bytes per lane, fp32 4 bytes.
__device__ __forceinline__ f32x4 lmma(const uint16_t* A, const uint16_t* B, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(A),
                                                   *reinterpret_cast<const bf16x8*>(B), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 lmma(const float* A, const float* B, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(*A, *B, c, 0, 0, 0);
}

// Inclusive prefix sum over the 16 lanes of each row (DPP row_shr 1, 2, 4, 8; lanes
// shifted in from outside the row contribute 0).
__device__ __forceinline__ float row_scan16(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xf, 0xf, false));
    return x;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), kBufFlags);
}

// Granule counts of the record, shared by its producer and its consumer.
template <int DK, int DV, class TIn>
struct RecGeo {
    static constexpr int CT = Geo<TIn>::CT, E = Geo<TIn>::E;
    static constexpr int GK = DK / (16 * CT);      // granules along dk
    static constexpr int GT = kChunk / (16 * CT);  // granules along the chunk's tokens
    static constexpr int BV = kCarryBV, NT = DV / BV, NCB = BV / 16;
    static constexpr int UB = NCB * 4 * E;         // bytes of one Ut tile per lane
    static_assert(DV % BV == 0 && DK % 64 == 0 && UB % 16 == 0, "record geometry");
};

// ---------------------------------------------------------------------------
// 1. chunk map (single workgroup): chunk and segment offsets per sequence and the
//    chunk and segment tables.
// ---------------------------------------------------------------------------
// Exclusive scan of f(i) over i < n in blocks of kThreads; out[n] = total.
template <class F>
__device__ void block_exclusive_scan(int n, F f, int32_t* out, int32_t* part, int32_t* carry) {
    const int tid = threadIdx.x;
    if (tid == 0) *carry = 0;
    __syncthreads();
    for (int base = 0; base < n; base += kThreads) {
        const int i = base + tid;
        const int x0 = i < n ? f(i) : 0;
        part[tid] = x0;
        __syncthreads();
        for (int off = 1; off < kThreads; off <<= 1) {  // Hillis-Steele inclusive scan
            const int x = tid >= off ? part[tid - off] : 0;
            __syncthreads();
            part[tid] += x;
            __syncthreads();
        }
        if (i < n) out[i] = *carry + part[tid] - x0;
        __syncthreads();
        if (tid == kThreads - 1) *carry += part[kThreads - 1];
        __syncthreads();
    }
    if (tid == 0) out[n] = *carry;
    __syncthreads();
}

// The chunk table (sequence, first token, length) and the segment table (sequence, first
// chunk, chunks, 2 k + last) from the chunk and segment offsets: one wave per sequence (its
// lanes over the sequence's chunks and segments), so the sequences' loads overlap.
__device__ void write_chunk_tables(const int32_t* cu, int num_seqs, int seg_chunks, const int32_t* chunk_off,
                                   const int32_t* seg_off, int4* table, int4* segtab) {
    const int lane = threadIdx.x % kWave;
    for (int i = threadIdx.x / kWave; i < num_seqs; i += kThreads / kWave) {
        const int bos = cu[i], eos = cu[i + 1];
        const int first = chunk_off[i], nch = chunk_off[i + 1] - first;
        const int s0 = seg_off[i], ns = seg_off[i + 1] - s0;
        for (int c = lane; c < nch; c += kWave) {
            const int t0 = bos + c * kChunk;
            table[first + c] = make_int4(i, t0, min(kChunk, eos - t0), 0);
        }
        for (int k = lane; k < ns; k += kWave)
            segtab[s0 + k] = make_int4(i, first + k * seg_chunks, min(seg_chunks, nch - k * seg_chunks),
                                       2 * k + (k == ns - 1 ? 1 : 0));
    }
}

// Batches of at most kThreads sequences need no chunk_map launch: every intra-chunk
// workgroup scans the chunk counts itself, and workgroup 0 writes the tables above.
__host__ __device__ inline bool map_inline(int num_seqs) { return num_seqs <= kThreads; }

__global__ __launch_bounds__(kThreads) void chunk_map_kernel(const int32_t* __restrict__ cu, int num_seqs,
                                                             int seg_chunks, int32_t* chunk_off, int32_t* seg_off,
                                                             int4* table, int4* segtab) {
    __shared__ int32_t part[kThreads];
    __shared__ int32_t carry;
    auto nchunks = [&](int i) {
        const int len = cu[i + 1] - cu[i];
        return len > 0 ? (len + kChunk - 1) / kChunk : 0;
    };
    block_exclusive_scan(num_seqs, nchunks, chunk_off, part, &carry);
    block_exclusive_scan(num_seqs, [&](int i) { return (nchunks(i) + seg_chunks - 1) / seg_chunks; }, seg_off, part,
                         &carry);
    write_chunk_tables(cu, num_seqs, seg_chunks, chunk_off, seg_off, table, segtab);
}

// ---------------------------------------------------------------------------
// 2. chunk_intra
//
// Wave w owns tokens 16w .. 16w+15 of the chunk; lane (r = lane % 16, q = lane / 16)
// holds token 16w + r and, of every row vector, the granules j of channels
// GW (4j + q) .. + GW - 1.  LDS regions (reused by phase):
//   phases 2-3: s-operand copies [96][DK] (copy i = rows 0 .. 16 i - 1 for the
//          off-diagonal tiles of token block i, from row 8 i (i - 1)); bf16: their low
//          parts in the next [96][DK]; over R1 .. R2.  From phase 4:
//     R1  T fp32 [64][LDA]
//     RD  the diagonal 16x16 blocks of A, fp32 [4][16][LDD]
//     RT  T' = T diag(beta) [64][LDT]
//     R2  KG^T [DK][LDT]
//   R3  V^T [DV][LDT]
//   RM  beta [64], key norm factors [64], per-wave gate totals, in-wave gate cumsums at
//       token 7, 2^totals [4][DK] each, and per wave 2^(G at its start) [4][DK]
// (bf16, dk = dv = 128: 72.5 KiB, so two workgroups share a CU.)  The rest of A stays in
// the registers of the wave that owns its rows; the QG and Kt record granules are built
// in registers by MFMA products with a 0/1 selector (exact), without an LDS transpose.
// ---------------------------------------------------------------------------
template <int DK, int DV, class TIn>
struct IntraPlan {
    using G = Geo<TIn>;
    using elem = typename G::elem;
    static constexpr int E = G::E, GW = G::GW;
    static constexpr int PAD = E == 2 ? 8 : 4;  // rows stay 16-byte aligned and bank-spread
    static constexpr int LDK = DK + PAD;
    static constexpr int LDT = kChunk + PAD;
    static constexpr int LDA = kChunk + 4;
    static constexpr int NGK = DK / (4 * GW), NGV = DV / (4 * GW);  // granules per lane
    static constexpr size_t R1 = align_up(cmax(64ull * LDK * E, 64ull * LDA * 4), 16);
    static constexpr size_t R2 = align_up(1ull * DK * LDT * E, 16);
    static constexpr size_t R3 = align_up(1ull * DV * LDT * E, 16);
    static constexpr int LDD = 20;  // fp32 diagonal-block rows (16 + 4, 16-byte aligned)
    static constexpr size_t RD = align_up(4ull * 16 * LDD * 4, 16);
    static constexpr size_t RT = align_up(64ull * LDT * E, 16);
    static constexpr size_t RM = align_up(4ull * (2 * 64 + 17 * DK), 16);
    static constexpr size_t O1 = 0, OD = O1 + R1, OT = OD + RD, O2 = OT + RT, O3 = O2 + R2;
    static constexpr size_t OM = O3 + R3;
    static constexpr size_t BYTES = OM + RM;
    static constexpr bool fits = BYTES <= 160 * 1024;
    // the s-operand copies of phases 2-3 (96 rows; bf16: high and low parts) overlay R1,
    // RD, RT and R2 (first written in phase 4)
    static_assert(96ull * DK * E * (E == 2 ? 2 : 1) <= O3, "s-operand copies exceed R1 .. R2");
    static_assert(DK / GW >= 8, "copy swizzle needs 8 granules per row");
};

// One item's inputs, as loaded (granules of q, k, v; fp32 gate; beta).
template <int DK, int DV, class TIn>
struct IntraIn {
    using P = IntraPlan<DK, DV, TIn>;
    u32x4 q[P::NGK], k[P::NGK], v[P::NGV];
    f32x4 g[P::NGK][P::GW / 4];
    float beta;
};

// Loads item (chunk, head)'s rows through buffer resources bounded at the chunk's
// last token, so rows past it read as zero (neutral padding).
template <int DK, int DV, class TIn>
__device__ __forceinline__ void intra_fetch(IntraIn<DK, DV, TIn>& X, const PrefillArgs& a, int t0, int L, int h,
                                            int wave, int lane) {
    using P = IntraPlan<DK, DV, TIn>;
    constexpr int E = P::E, GW = P::GW;
    const int H = a.H, r = lane & 15, q = lane >> 4, t = 16 * wave + r;
    const int64_t tok = static_cast<int64_t>(t0) * H + h;
    const int rows = (L - 1) * H + 1;
    const auto rq = buf_rsrc(static_cast<const char*>(a.q) + tok * DK * E, static_cast<int64_t>(rows) * DK * E);
    const auto rk = buf_rsrc(static_cast<const char*>(a.k) + tok * DK * E, static_cast<int64_t>(rows) * DK * E);
    const auto rv = buf_rsrc(static_cast<const char*>(a.v) + tok * DV * E, static_cast<int64_t>(rows) * DV * E);
    const auto rg = buf_rsrc(a.g + tok * DK, static_cast<int64_t>(rows) * DK * 4);
    const auto rb = buf_rsrc(a.beta + tok, static_cast<int64_t>(rows) * 4);
#pragma unroll
    for (int j = 0; j < P::NGK; ++j) {
        const int off = (t * H * DK + GW * (4 * j + q)) * E;
        X.q[j] = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
        X.k[j] = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < P::NGV; ++j)
        X.v[j] = __builtin_amdgcn_raw_buffer_load_b128(rv, (t * H * DV + GW * (4 * j + q)) * E, 0, 0);
#pragma unroll
    for (int j = 0; j < P::NGK; ++j)
#pragma unroll
        for (int m = 0; m < GW / 4; ++m)
            X.g[j][m] = __builtin_bit_cast(
                f32x4, __builtin_amdgcn_raw_buffer_load_b128(rg, (t * H * DK + GW * (4 * j + q) + 4 * m) * 4, 0, 0));
    X.beta = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, t * H * 4, 0, 0));
}

// ---------------------------------------------------------------------------
// Input front (kda_chunk_prefill_front): before phase 1, the item's raw q, k, v are convolved
// along the tokens of their sequence (causal depthwise, width W <= 4:
// y_t[c] = sum_j w[c][j] x_{t-(W-1)+j}[c]), optionally passed through SiLU, and the raw
// gates and beta values processed (g = -a_h softplus(z), beta = sigmoid(b)), all in the
// item's registers.  Lane (r, q) of wave w holds token 16 w + r, so the input d tokens back
// is lane r - d of the same wave (a DPP row shift keeps the channels) or, for the wave's
// first d tokens, one of the previous wave's last three tokens, which each wave leaves in
// LDS; wave 0 fetches the three tokens before the chunk (the previous chunk's, or at the
// sequence start the slot's convolution state, or zeros).  Rows past the chunk's end are
// zeroed, gates included, as the plain prefill reads them.  With bf16 inputs the convolved
// q, k, v are rounded to bf16 (the granules the phases read).
// ---------------------------------------------------------------------------
template <int DK, int DV, class TIn>
struct FrontTails {
    static constexpr int CW = 2 * DK + DV;                        // channels q | k | v
    static constexpr size_t BYTES = 5ull * 3 * CW * Geo<TIn>::E;  // [slot 5][row 3][CW]
    static_assert(BYTES <= IntraPlan<DK, DV, TIn>::R1, "front tails exceed region R1");
};

template <int D>
__device__ __forceinline__ u32x4 row_shift_gran(u32x4 x) {
    u32x4 y;
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x[i]), 0x110 + D, 0xf, 0xf, false));
    return y;
}

template <int DK, int DV, class TIn>
__device__ __forceinline__ void intra_front(IntraIn<DK, DV, TIn>& X, char* smem, const PrefillArgs& a, int t0, int L,
                                            int bos, int seq, int h, int wave, int lane) {
    using P = IntraPlan<DK, DV, TIn>;
    using FT = FrontTails<DK, DV, TIn>;
    constexpr int E = P::E, GW = P::GW, NGK = P::NGK, NGV = P::NGV, CW = FT::CW;
    constexpr TIn tag{};
    const FrontArgs& f = a.front;
    const int W = f.conv_width, H = a.H;
    const int r = lane & 15, q = lane >> 4, t = 16 * wave + r;
    char* tails = smem + P::O1;
    auto tail_at = [&](int slot, int row, int chan) { return tails + ((slot * 3 + row) * CW + chan) * E; };

    if (W > 1) {
        // this wave's last three tokens -> tail slot wave + 1
        if (r >= 13) {
#pragma unroll
            for (int j = 0; j < NGK; ++j) {
                *reinterpret_cast<u32x4*>(tail_at(wave + 1, r - 13, GW * (4 * j + q))) = X.q[j];
                *reinterpret_cast<u32x4*>(tail_at(wave + 1, r - 13, DK + GW * (4 * j + q))) = X.k[j];
            }
#pragma unroll
            for (int j = 0; j < NGV; ++j)
                *reinterpret_cast<u32x4*>(tail_at(wave + 1, r - 13, 2 * DK + GW * (4 * j + q))) = X.v[j];
        }
        // the three tokens before the chunk -> slot 0
        if (wave == 0 && r >= 13) {
            const int u = t0 - 16 + r;  // its token index
            const bool in_seq = u >= bos;
            const int crow = u - bos + W - 1;  // its row of the convolution state (if >= 0)
            const bool from_state = !in_seq && a.h0_from_pool && crow >= 0;
            const char* src = nullptr;
            if (from_state)
                src = static_cast<const char*>(f.conv_state) +
                      ((static_cast<int64_t>(a.slot_idx[seq]) * H + h) * (W - 1) + crow) * CW * E;
            auto fetch = [&](const void* x, int D, int off, int chan) -> u32x4 {
                if (in_seq)
                    return *reinterpret_cast<const u32x4*>(static_cast<const char*>(x) +
                                                           ((static_cast<int64_t>(u) * H + h) * D + chan) * E);
                if (from_state) return *reinterpret_cast<const u32x4*>(src + (off + chan) * E);
                return u32x4{0u, 0u, 0u, 0u};
            };
#pragma unroll
            for (int j = 0; j < NGK; ++j) {
                const int c = GW * (4 * j + q);
                *reinterpret_cast<u32x4*>(tail_at(0, r - 13, c)) = fetch(a.q, DK, 0, c);
                *reinterpret_cast<u32x4*>(tail_at(0, r - 13, DK + c)) = fetch(a.k, DK, DK, c);
            }
#pragma unroll
            for (int j = 0; j < NGV; ++j) {
                const int c = GW * (4 * j + q);
                *reinterpret_cast<u32x4*>(tail_at(0, r - 13, 2 * DK + c)) = fetch(a.v, DV, 2 * DK, c);
            }
        }
        lds_barrier();
    }
    // one granule: channels c0 .. c0 + GW - 1 of the block at channel offset off (q | k | v)
    auto conv = [&](u32x4& G, const float* w, int D, int off, int c0) {
        const float* wc = w + (static_cast<int64_t>(h) * D + c0) * W;
        // wt[e][d]: the weight of the input d tokens back (zero beyond the width); width 4
        // reads each channel's taps as one 16-byte load
        float wt[GW][4];
        if (W == 4) {
#pragma unroll
            for (int e = 0; e < GW; ++e) {
                const f32x4 w4 = *reinterpret_cast<const f32x4*>(wc + 4 * e);
#pragma unroll
                for (int d = 0; d < 4; ++d) wt[e][d] = w4[3 - d];
            }
        } else {
#pragma unroll
            for (int e = 0; e < GW; ++e)
#pragma unroll
                for (int d = 0; d < 4; ++d) wt[e][d] = d < W ? wc[e * W + W - 1 - d] : 0.f;
        }
        float x[GW], acc[GW];
        gran_to_f32(G, x, tag);
#pragma unroll
        for (int e = 0; e < GW; ++e) acc[e] = wt[e][0] * x[e];
        auto tap = [&](auto dtag) {
            constexpr int d = decltype(dtag)::value;
            if (d < W) {
                const u32x4 sh = row_shift_gran<d>(G);
                // lanes r < d: token 16 wave + r - d, row 3 + r - d of the previous wave's tail
                const u32x4 tv = *reinterpret_cast<const u32x4*>(tail_at(wave, 3 + min(r, d - 1) - d, off + c0));
                const u32x4 xv = r >= d ? sh : tv;
                float xd[GW];
                gran_to_f32(xv, xd, tag);
#pragma unroll
                for (int e = 0; e < GW; ++e) acc[e] = fmaf(wt[e][d], xd[e], acc[e]);
            }
        };
        tap(std::integral_constant<int, 1>{});
        tap(std::integral_constant<int, 2>{});
        tap(std::integral_constant<int, 3>{});
#pragma unroll
        for (int e = 0; e < GW; ++e) {
            const float y = f.conv_silu ? front_silu(acc[e]) : acc[e];
            acc[e] = t < L ? y : 0.f;
        }
        G = f32_to_gran(acc, tag);
    };
#pragma unroll
    for (int j = 0; j < NGK; ++j) {
        conv(X.q[j], f.conv_q, DK, 0, GW * (4 * j + q));
        conv(X.k[j], f.conv_k, DK, DK, GW * (4 * j + q));
    }
#pragma unroll
    for (int j = 0; j < NGV; ++j) conv(X.v[j], f.conv_v, DV, 2 * DK, GW * (4 * j + q));
    const float gs = f.gate_scale[h];
#pragma unroll
    for (int j = 0; j < NGK; ++j)
#pragma unroll
        for (int m = 0; m < GW / 4; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e) X.g[j][m][e] = t < L ? -gs * front_softplus(X.g[j][m][e]) : 0.f;
    X.beta = t < L ? front_sigmoid(X.beta) : 0.f;
}

template <int DK, int DV, class TIn>
__device__ __forceinline__ void intra_compute(const IntraIn<DK, DV, TIn>& X, char* smem, const PrefillArgs& a,
                                              char* rec, const WsLayout& ws, int wave, int lane, int tid) {
    using P = IntraPlan<DK, DV, TIn>;
    using RG = RecGeo<DK, DV, TIn>;
    using elem = typename P::elem;
    constexpr int E = P::E, GW = P::GW, NGK = P::NGK, NGV = P::NGV;
    constexpr int LDT = P::LDT, LDA = P::LDA;
    constexpr int KS = Mma<TIn>::KS, KST = kChunk / KS;  // natural k-steps over tokens
    constexpr TIn tag{};
    // phases 2-3: s-operand copies, rows of DK elements without padding; the 16-byte
    // granule index is XORed with the row's low 3 bits, so the 16 rows one MFMA operand
    // read touches spread over the LDS banks
    elem* sKS = reinterpret_cast<elem*>(smem + P::O1);
    auto ks_at = [](int row, int gran) { return row * DK + GW * (gran ^ (row & 7)); };
    float* sT = reinterpret_cast<float*>(smem + P::O1);
    elem* sKGt = reinterpret_cast<elem*>(smem + P::O2);
    elem* sVt = reinterpret_cast<elem*>(smem + P::O3);
    float* sD = reinterpret_cast<float*>(smem + P::OD);
    elem* sTp = reinterpret_cast<elem*>(smem + P::OT);
    float* sBeta = reinterpret_cast<float*>(smem + P::OM);
    float* sIk = sBeta + 64;      // key norm factors per token
    float* sTot = sIk + 64;       // [wave][DK] the wave's gate total (log2 units)
    float* sMid = sTot + 4 * DK;  // [wave][DK] the in-wave gate cumsum at the wave's token 7
    float* sT2 = sMid + 4 * DK;   // [1 + wave][DK] 2^(the wave's gate total); row 0 = 1
    float* sPW = sT2 + 5 * DK + wave * DK;  // [wave][DK] 2^(G_end(wave - 1) - chunk start)

    const int r = lane & 15, q = lane >> 4, t = 16 * wave + r;
    // no output (the backward's forward pass): the QG and P records are never read, so
    // neither they nor the P tiles are formed
    const bool with_o = a.o != nullptr;

    // ---- 1. norms, gate cumsum inside the wave, per-wave gate tables ------------------
    // The gates are scaled by log2(e) before the scan, so each exponential below is a
    // single exp2.
    constexpr float kLog2e = 1.4426950408889634f;
    // q and k stay packed (unpacked again where used); only the norms' scale factors live on
    float gf[NGK][GW];
#pragma unroll
    for (int j = 0; j < NGK; ++j)
#pragma unroll
        for (int m = 0; m < GW / 4; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e) gf[j][4 * m + e] = X.g[j][m][e] * kLog2e;
    float iq = 1.f, ik = 1.f;
    if (a.use_l2) {
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int j = 0; j < NGK; ++j) {
            float qv[GW], kv[GW];
            gran_to_f32(X.q[j], qv, tag);
            gran_to_f32(X.k[j], kv, tag);
#pragma unroll
            for (int e = 0; e < GW; ++e) {
                sq = fmaf(qv[e], qv[e], sq);
                sk = fmaf(kv[e], kv[e], sk);
            }
        }
        sq += __shfl_xor(sq, 16, 64);
        sk += __shfl_xor(sk, 16, 64);
        sq += __shfl_xor(sq, 32, 64);
        sk += __shfl_xor(sk, 32, 64);
        iq = 1.f / sqrtf(sq + kNormEps);
        ik = 1.f / sqrtf(sk + kNormEps);
    }
#pragma unroll
    for (int j = 0; j < NGK; ++j)
#pragma unroll
        for (int e = 0; e < GW; ++e) gf[j][e] = row_scan16(gf[j][e]);
    if (r == 15 || r == 7) {
        float* dst = r == 15 ? sTot : sMid;
#pragma unroll
        for (int j = 0; j < NGK; ++j)
#pragma unroll
            for (int m = 0; m < GW / 4; ++m) {
                const int c = wave * DK + GW * (4 * j + q) + 4 * m;
                const f32x4 x = {gf[j][4 * m], gf[j][4 * m + 1], gf[j][4 * m + 2], gf[j][4 * m + 3]};
                *reinterpret_cast<f32x4*>(dst + c) = x;
                if (r == 15)
                    *reinterpret_cast<f32x4*>(sT2 + DK + c) =
                        f32x4{__builtin_amdgcn_exp2f(x[0]), __builtin_amdgcn_exp2f(x[1]),
                              __builtin_amdgcn_exp2f(x[2]), __builtin_amdgcn_exp2f(x[3])};
            }
    }
    if (q == 0) {
        sBeta[t] = X.beta;
        sIk[t] = ik;
    }
    if (tid < DK) sT2[tid] = 1.f;
    lds_barrier();

    // ---- 2. exponentials, operands, records, the diagonal tiles -----------------------
    // exp(G_t - G_s) is never formed as a product of one large and one small factor:
    //  - record operands and W use the chunk start as reference: 2^G_t <= 1 (QG, KG) and
    //    2^(G_L - G_t) <= 1 (Kt);
    //  - an off-diagonal tile (t in block i, s in block j < i) splits at the end of block
    //    i - 1: t side 2^(G_t - G_end(i-1)) = 2^gf_t <= 1 (KB, QB), s side
    //    2^(G_end(i-1) - G_s) <= 1, stored by the wave owning s once per later block i
    //    (row s of copy i = 2^(G_end(j) - G_s) times the gate factors of blocks j+1..i-1);
    //  - a diagonal tile (t, s in one block) splits at the block's token 7, so each factor
    //    spans at most 8 tokens' gates.
    // The operands are the raw q and k (exact for bf16 inputs wherever the factor is 1);
    // the norm factors scale the finished tiles.  With bf16 inputs every A and P operand is
    // carried as a high and a low bf16 part (products hi*hi + hi*lo + lo*hi, three MFMAs),
    // so an entry's error is about 2^-16 of its terms, and an entry whose terms cancel
    // (q.k near 0) keeps its own size's accuracy instead of 2^-8 of |q||k|.
    const bool odd = r & 1;
    const int te = t & ~1;
    // v_perm_b32 selectors for the adjacent-token pairs of the transposed copies: even
    // lanes write (own, neighbour) low halves, odd lanes (neighbour, own) high halves
    const uint32_t psel = odd ? 0x03020706u : 0x05040100u;
    auto pair_store = [&](elem* dstT, u32x4 wv, int j) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t nbr = static_cast<uint32_t>(
                __builtin_amdgcn_update_dpp(0, static_cast<int>(wv[i]), 0xB1, 0xf, 0xf, false));
            const int c = GW * (4 * j + q) + 2 * i + (odd ? 1 : 0);
            *reinterpret_cast<uint32_t*>(dstT + c * LDT + te) = __builtin_amdgcn_perm(nbr, wv[i], psel);
        }
    };
    // V^T first, so the V registers are free for the rest of the phase
#pragma unroll
    for (int j = 0; j < NGV; ++j) {
        if constexpr (E == 2) {
            pair_store(sVt, X.v[j], j);
        } else {
#pragma unroll
            for (int e = 0; e < GW; ++e) sVt[(GW * (4 * j + q) + e) * LDT + t] = __uint_as_float(X.v[j][e]);
        }
    }
    // sel[h]: the 0/1 granule whose row n picks channel 16 h + n of a 32-channel bf16
    // granule (fp32: channel n of a 16-channel granule, one 0/1 value per k-step).  A
    // product with it copies values exactly and leaves them in accumulator layout, which
    // gives the Kt and QG record granules without an LDS transpose.
    u32x4 sel[RG::CT];
#pragma unroll
    for (int h = 0; h < RG::CT; ++h) {
        float x[GW];
#pragma unroll
        for (int e = 0; e < GW; ++e) x[e] = (E == 2 ? (8 * q + e == 16 * h + r) : (4 * q + e == r)) ? 1.f : 0.f;
        sel[h] = f32_to_gran(x, tag);
    }
    // gate-table rows (wave-uniform): 2^(total of block w) is row w + 1, a block outside
    // the chunk reads the row of ones; the blocks before this one give the chunk-start
    // reference, the blocks after it Kt and the s-operand copies
    auto trow = [&](int w) { return (w >= 0 && w < 4 ? w + 1 : 0) * DK; };
    const int p1 = trow(wave - 1), p2 = trow(wave - 2), p3 = trow(wave - 3);
    const int n1 = trow(wave + 1), n2 = trow(wave + 2), n3 = trow(wave + 3);
    // s-operand copy rows of this wave's token for copies wave + 1, wave + 2, wave + 3
    const int c1 = 8 * (wave + 1) * wave + t, c2 = 8 * (wave + 2) * (wave + 1) + t, c3 = 48 + t;
    u32x4 KBh[NGK], KBl[NGK], QBh[NGK], QBl[NGK];
    f32x4 Adg = {0.f, 0.f, 0.f, 0.f}, Pdg = Adg;
    // this wave's chunk-start factors per channel, formed once (not by each of the 16 lanes
    // holding a channel); only this wave reads them, after its own writes
    for (int c = lane; c < DK; c += kWave) sPW[c] = sT2[p1 + c] * sT2[p2 + c] * sT2[p3 + c];
    asm volatile("" ::: "memory");
    {
        float* gl_out = reinterpret_cast<float*>(rec + ws.o_gl);
#pragma unroll
        for (int j = 0; j < NGK; ++j) {
            float qv[GW], kv[GW], ks0[GW], ks1[GW], ks2[GW], kb[GW], qb[GW], qg[GW], kt[GW];
            float sd[GW], kd[GW], qd[GW];
            gran_to_f32(X.q[j], qv, tag);
            gran_to_f32(X.k[j], kv, tag);
#pragma unroll
            for (int m = 0; m < GW / 4; ++m) {
                const int c = GW * (4 * j + q) + 4 * m;
                const f32x4 PW = *reinterpret_cast<const f32x4*>(sPW + c);
                const f32x4 N1 = *reinterpret_cast<const f32x4*>(sT2 + n1 + c);
                const f32x4 N2 = *reinterpret_cast<const f32x4*>(sT2 + n2 + c);
                const f32x4 N3 = *reinterpret_cast<const f32x4*>(sT2 + n3 + c);
                const f32x4 tw = *reinterpret_cast<const f32x4*>(sTot + wave * DK + c);
                const f32x4 md = *reinterpret_cast<const f32x4*>(sMid + wave * DK + c);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 4 * m + e;
                    const float G = gf[j][i];
                    // 2^(G_t - chunk start) and 2^(G_L - G_t) from the block factors
                    const float pw = PW[e];
                    const float kw = N1[e] * N2[e] * N3[e];
                    const float et = __builtin_amdgcn_exp2f(G);           // 2^(G_t - G_end(i-1))
                    const float kif = __builtin_amdgcn_exp2f(tw[e] - G);  // 2^(G_end(i) - G_t)
                    const float e1 = __builtin_amdgcn_exp2f(G - md[e]);   // diagonal tile, t side
                    const float e2 = __builtin_amdgcn_exp2f(md[e] - G);   // diagonal tile, s side
                    kb[i] = kv[i] * et;
                    qb[i] = qv[i] * et;
                    qg[i] = qb[i] * (iq * pw);
                    ks0[i] = kv[i] * kif;
                    kt[i] = ks0[i] * (ik * kw);
                    ks1[i] = ks0[i] * N1[e];
                    ks2[i] = ks1[i] * N2[e];
                    sd[i] = kv[i] * e2;
                    kd[i] = kv[i] * e1;
                    qd[i] = qv[i] * e1;
                }
                if (wave == 0 && r == 0) {
                    const f32x4 t0 = *reinterpret_cast<const f32x4*>(sTot + c);
                    const f32x4 t1 = *reinterpret_cast<const f32x4*>(sTot + DK + c);
                    const f32x4 t2 = *reinterpret_cast<const f32x4*>(sTot + 2 * DK + c);
                    const f32x4 t3 = *reinterpret_cast<const f32x4*>(sTot + 3 * DK + c);
                    f32x4 gl;
#pragma unroll
                    for (int e = 0; e < 4; ++e) gl[e] = __builtin_amdgcn_exp2f(((t0[e] + t1[e]) + t2[e]) + t3[e]);
                    *reinterpret_cast<f32x4*>(gl_out + c) = gl;
                }
            }
            split_gran(kb, KBh[j], KBl[j], tag);
            if (with_o) split_gran(qb, QBh[j], QBl[j], tag);
            // s-operand copies of this wave's rows for every later block i (copy i holds
            // rows 0 .. 16 i - 1 from KS row 8 i (i - 1); the low parts 96 rows further)
            auto put = [&](int row, const float* x) {
                u32x4 h, l;
                split_gran(x, h, l, tag);
                *reinterpret_cast<u32x4*>(sKS + ks_at(row, 4 * j + q)) = h;
                if constexpr (E == 2) *reinterpret_cast<u32x4*>(sKS + ks_at(96 + row, 4 * j + q)) = l;
            };
            if (wave < 3) put(c1, ks0);
            if (wave < 2) put(c2, ks1);
            if (wave < 1) put(c3, ks2);
            // records: granule j spans the dk blocks CT j .. CT j + CT - 1
            const u32x4 ktg = f32_to_gran(kt, tag);
            const u32x4 qgg = f32_to_gran(qg, tag);
            f32x4 qt[RG::CT] = {};
#pragma unroll
            for (int h = 0; h < RG::CT; ++h) {
                const int cb = RG::CT * j + h;
                // Kt tile (rows t of this token block, columns c): lane holds tokens
                // 16 wave + 4q + rr of channel 16 cb + r -> its half of the Kt granule
                const f32x4 kt4 = gmma(ktg, sel[h], f32x4{0.f, 0.f, 0.f, 0.f}, tag);
                char* dk = rec + ws.o_kt + ((static_cast<size_t>(cb) * RG::GT + wave / RG::CT) * 64 + lane) * 16;
                if constexpr (E == 2)
                    *reinterpret_cast<u32x2*>(dk + (wave % RG::CT) * 8) =
                        u32x2{pack_bf16x2(kt4[0], kt4[1]), pack_bf16x2(kt4[2], kt4[3])};
                else
                    *reinterpret_cast<f32x4*>(dk) = kt4;
                // QG^T tile (rows c, columns t): lane holds channels 16 cb + 4q + rr of token t
                if (with_o) qt[h] = gmma(sel[h], qgg, f32x4{0.f, 0.f, 0.f, 0.f}, tag);
            }
            // QG and P are read once, by the output pass: streaming stores, so the Infinity
            // Cache keeps more of the W, Kt, Ut granules that both carries read
            if (with_o)
                __builtin_nontemporal_store(
                    tiles_to_gran(qt[0], qt[RG::CT - 1], tag),
                    reinterpret_cast<u32x4*>(rec + ws.o_q + ((static_cast<size_t>(wave) * RG::GK + j) * 64 + lane) * 16));
            // the diagonal tiles from this lane's own rows (s and t both in this block) on fp32
            // MFMA (no operand split): step e takes channel GW (4 j + q) + e of lane (r, q) as
            // its k index q
#pragma unroll
            for (int e = 0; e < GW; ++e) {
                Adg = __builtin_amdgcn_mfma_f32_16x16x4f32(sd[e], kd[e], Adg, 0, 0, 0);
                if (with_o) Pdg = __builtin_amdgcn_mfma_f32_16x16x4f32(sd[e], qd[e], Pdg, 0, 0, 0);
            }
            // one granule at a time: interleaving the unrolled iterations runs out of registers
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    lds_barrier();
    // ---- 3. A^T and P^T tiles of this wave's rows t over the four s blocks; P record.
    //      The off-diagonal tiles read this block's s-operand copy; the tile of this block
    //      is the diagonal one; later blocks are zero.
    f32x4 Areg[4], Preg[4];
    {
        const int kbase = 8 * wave * (wave - 1);  // this block's copy (rows 0 .. 16 wave - 1)
        const float ab = X.beta * ik;             // A_ts = beta_t ik_t ik_s (raw product)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accP = accA;
            if (jj < 3 && jj < wave) {
                const int row = kbase + 16 * jj + r;
#pragma unroll
                for (int j = 0; j < NGK; ++j) {
                    const u32x4 bh = *reinterpret_cast<const u32x4*>(sKS + ks_at(row, 4 * j + q));
                    const u32x4 bl =
                        E == 2 ? *reinterpret_cast<const u32x4*>(sKS + ks_at(96 + row, 4 * j + q)) : bh;
                    accA = smma(bh, bl, KBh[j], KBl[j], accA, tag);
                    if (with_o) accP = smma(bh, bl, QBh[j], QBl[j], accP, tag);
                }
            }
            const f32x4 iks = *reinterpret_cast<const f32x4*>(sIk + 16 * jj + 4 * q);
            // lane holds (s = 16 jj + 4q + rr, t)
            float a4[4], p4[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int s = 16 * jj + 4 * q + rr;
                const float xa = jj == wave ? Adg[rr] : accA[rr];
                const float xp = jj == wave ? Pdg[rr] : accP[rr];
                a4[rr] = s < t ? ab * iks[rr] * xa : 0.f;
                p4[rr] = s <= t ? iq * iks[rr] * xp : 0.f;
            }
            Areg[jj] = f32x4{a4[0], a4[1], a4[2], a4[3]};
            Preg[jj] = f32x4{p4[0], p4[1], p4[2], p4[3]};
        }
    }
    // P granules (rows t of this token block, k over tokens) to the record
#pragma unroll
    for (int g = 0; g < RG::GT; ++g)
        if (with_o)
            __builtin_nontemporal_store(
                tiles_to_gran(Preg[RG::CT * g], Preg[RG::CT * g + RG::CT - 1], tag),
                reinterpret_cast<u32x4*>(rec + ws.o_p + ((static_cast<size_t>(wave) * RG::GT + g) * 64 + lane) * 16));
    lds_barrier();

    // ---- 4. (the s-operand copies are dead) KG^T for phase 6, KG = 2^G kh from KB =
    //      2^gf k (its high and low parts); this wave's diagonal block of A to LDS and the
    //      upper blocks of its T' rows zeroed (both read only by this wave until the next
    //      barrier)
#pragma unroll
    for (int j = 0; j < NGK; ++j) {
        float kg[GW], lo[GW];
        gran_to_f32(KBh[j], kg, tag);
        gran_to_f32(KBl[j], lo, tag);
#pragma unroll
        for (int m = 0; m < GW / 4; ++m) {
            const int c = GW * (4 * j + q) + 4 * m;
            const f32x4 PW = *reinterpret_cast<const f32x4*>(sPW + c);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 4 * m + e;
                kg[i] = (E == 2 ? kg[i] + lo[i] : kg[i]) * (ik * PW[e]);
            }
        }
        const u32x4 KG = f32_to_gran(kg, tag);
        if constexpr (E == 2) {
            pair_store(sKGt, KG, j);
        } else {
#pragma unroll
            for (int e = 0; e < GW; ++e) sKGt[(GW * (4 * j + q) + e) * LDT + t] = kg[e];
        }
    }
    {
        f32x4 dg = Areg[0];
#pragma unroll
        for (int jj = 1; jj < 4; ++jj)
            if (jj == wave) dg = Areg[jj];
        *reinterpret_cast<f32x4*>(sD + (16 * wave + r) * P::LDD + 4 * q) = dg;
    }
    for (int jj = wave + 1; jj < 4; ++jj) lds_store4(sTp + t * LDT + 16 * jj + 4 * q, 0.f, 0.f, 0.f, 0.f);

    // ---- 5. T = (I + A)^-1 by 16x16 blocks ----------------------------------------------
    // 5a. diagonal block of this wave by forward substitution, one lane per column
    {
        const int col = r;
        const float* Ab = sD + (16 * wave) * P::LDD;
        float x[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            f32x4 row[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) row[m] = *reinterpret_cast<const f32x4*>(Ab + rr * P::LDD + 4 * m);
            float acc = rr == col ? 1.f : 0.f;
#pragma unroll
            for (int s = 0; s < rr; ++s) acc = fmaf(-row[s >> 2][s & 3], x[s], acc);
            x[rr] = acc;
        }
        if (q == 0) {
            const float bc = sBeta[16 * wave + col];
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                sT[(16 * wave + rr) * LDA + 16 * wave + col] = x[rr];
                sTp[(16 * wave + rr) * LDT + 16 * wave + col] = Mma<TIn>::from_f32(x[rr] * bc);
            }
        }
    }
    lds_barrier();
    // 5b. T_{w, w-d} = -T_ww sum_{k = w-d}^{w-1} A_wk T_{k, w-d}, one block diagonal at a time
#pragma unroll
    for (int d = 1; d < 4; ++d) {
        if (wave >= d) {
            const int jb = wave - d;
            // y = sum over k blocks jb .. wave - 1 of A_{wave,kb} T_{kb,jb}; A comes from the
            // registers (lane (r, q) supplies k = 4q + ks: A[16 wave + r][16 kb + 4q + ks]);
            // blocks outside the range are masked to zero in both operands
            f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < 3; ++kb) {
                const bool in = kb >= jb && kb < wave;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const float av = in ? Areg[kb][ks] : 0.f;
                    const float tv = in ? sT[(16 * kb + 4 * q + ks) * LDA + 16 * jb + r] : 0.f;
                    y = __builtin_amdgcn_mfma_f32_16x16x4f32(av, tv, y, 0, 0, 0);
                }
            }
            // z = T_ww y; lane (r, q) supplies k = 4q + ks of both operands
            f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                z = __builtin_amdgcn_mfma_f32_16x16x4f32(sT[(16 * wave + r) * LDA + 16 * wave + 4 * q + ks], y[ks], z,
                                                         0, 0, 0);
            const float bc = sBeta[16 * jb + r];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int row = 16 * wave + 4 * q + rr;
                sT[row * LDA + 16 * jb + r] = -z[rr];
                sTp[row * LDT + 16 * jb + r] = Mma<TIn>::from_f32(-z[rr] * bc);
            }
        }
        lds_barrier();
    }

    // ---- 6. W^T = KG^T T'^T and Ut = T' V, straight to the record (each granule stored as
    //      soon as its tiles are done) -------------------------------------------------
    {
        const elem* Tr = sTp + (16 * wave + r) * LDT + (KS / 4) * q;
#pragma unroll
        for (int g = 0; g < RG::GK; ++g) {
            f32x4 wt[RG::CT];
#pragma unroll
            for (int h = 0; h < RG::CT; ++h) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                const elem* Kr = sKGt + (16 * (RG::CT * g + h) + r) * LDT + (KS / 4) * q;
#pragma unroll
                for (int ks = 0; ks < KST; ++ks) acc = lmma(Kr + KS * ks, Tr + KS * ks, acc);  // tile (c, t)
                wt[h] = acc;
            }
            *reinterpret_cast<u32x4*>(rec + ws.o_w + ((static_cast<size_t>(wave) * RG::GK + g) * 64 + lane) * 16) =
                tiles_to_gran(wt[0], wt[RG::CT - 1], tag);
        }
        // Ut: per dv tile, its NCB column blocks' 4 values each
#pragma unroll
        for (int tile = 0; tile < RG::NT; ++tile) {
            char* dst = rec + ws.o_u + (static_cast<size_t>(tile * 4 + wave) * 64 + lane) * RG::UB;
#pragma unroll
            for (int n = 0; n < RG::UB / 16; ++n) {
                f32x4 ut[RG::CT];
#pragma unroll
                for (int h = 0; h < RG::CT; ++h) {
                    const int jb = RG::NCB * tile + RG::CT * n + h;
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                    const elem* Vr = sVt + (16 * jb + r) * LDT + (KS / 4) * q;
#pragma unroll
                    for (int ks = 0; ks < KST; ++ks) acc = lmma(Tr + KS * ks, Vr + KS * ks, acc);  // tile (t, j)
                    ut[h] = acc;
                }
                *reinterpret_cast<u32x4*>(dst + 16 * n) = tiles_to_gran(ut[0], ut[RG::CT - 1], tag);
            }
        }
    }
}

// Persistent: workgroup b takes items b, b + grid, ... (item = chunk * H + head); two
// workgroups share a CU (bf16), so one computes while the other waits for its inputs.
// The table entry of the next item is read with a vector load one item ahead, so the
// LDS barriers (which wait for scalar loads) never wait for it.
template <int DK, int DV, class TIn, bool FRONT>
__global__ __launch_bounds__(kThreads, 2) void chunk_intra_kernel(PrefillArgs a) {
    using P = IntraPlan<DK, DV, TIn>;
    static_assert(P::fits, "LDS plan exceeds 160 KiB");
    __shared__ __attribute__((aligned(16))) char smem[P::BYTES];
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int H = a.H, ns = a.num_seqs;
    const WsLayout ws(ns, a.total_tokens, H, DK, DV, P::E);
    int32_t* chunk_off = static_cast<int32_t*>(a.workspace);
    int4* table = reinterpret_cast<int4*>(static_cast<char*>(a.workspace) + ws.off_table);
    char* recs = static_cast<char*>(a.workspace) + ws.off_rec;
    const int stride = gridDim.x;

    // Batches of up to kThreads sequences: the chunk offsets are scanned into LDS here (from
    // cu_seqlens, copied once), and workgroup 0 also writes the workspace tables the segment
    // kernels read.  Larger batches: chunk_map_kernel ran first and each item reads its entry
    // of the chunk table.
    __shared__ int32_t m_cu[kThreads + 1], m_coff[kThreads + 1];
    __shared__ int32_t m_carry;
    // used only before the item loop: over the phase regions
    int32_t* m_soff = reinterpret_cast<int32_t*>(smem);
    int32_t* m_part = m_soff + kThreads + 1;
    static_assert(sizeof(int32_t) * (2 * kThreads + 1) <= P::BYTES, "scan arrays exceed the phase regions");
    const bool inl = map_inline(ns);
    if (inl) {
        for (int i = tid; i <= ns; i += kThreads) m_cu[i] = a.cu_seqlens[i];
        __syncthreads();
        auto nchunks = [&](int i) {
            const int len = m_cu[i + 1] - m_cu[i];
            return len > 0 ? (len + kChunk - 1) / kChunk : 0;
        };
        block_exclusive_scan(ns, nchunks, m_coff, m_part, &m_carry);
        if (blockIdx.x == 0) {
            const int seg = ws.seg_chunks;
            block_exclusive_scan(ns, [&](int i) { return (nchunks(i) + seg - 1) / seg; }, m_soff, m_part, &m_carry);
            int32_t* seg_off = reinterpret_cast<int32_t*>(static_cast<char*>(a.workspace) + ws.off_segoff);
            for (int i = tid; i <= ns; i += kThreads) {
                chunk_off[i] = m_coff[i];
                seg_off[i] = m_soff[i];
            }
            write_chunk_tables(m_cu, ns, seg, m_coff, m_soff, table,
                               reinterpret_cast<int4*>(static_cast<char*>(a.workspace) + ws.off_segtab));
        }
        __syncthreads();  // m_soff and m_part are dead before any phase writes their LDS
    }
    const int total = (inl ? m_coff[ns] : chunk_off[ns]) * H;
    for (int item = blockIdx.x; item < total; item += stride) {
        const int c = item / H;
        int t0, L, seq;
        if (inl) {
            // the sequence lo with m_coff[lo] <= c < m_coff[lo + 1] (it has chunks)
            int lo = 0, hi = ns;
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (m_coff[mid] <= c)
                    lo = mid;
                else
                    hi = mid;
            }
            t0 = __builtin_amdgcn_readfirstlane(m_cu[lo] + kChunk * (c - m_coff[lo]));
            L = __builtin_amdgcn_readfirstlane(min(kChunk, m_cu[lo + 1] - t0));
            seq = lo;
        } else {
            const int4 e = table[c];
            seq = e.x;
            t0 = e.y;
            L = e.z;
        }
        // Lane-derived offsets and masks are formed again for every item: opaque copies of
        // the lane and wave indices keep the compiler from hoisting them out of the item
        // loop, where they would stay live across all phases (and spill).
        int ln = lane, wv = wave;
        asm volatile("" : "+v"(ln));
        asm volatile("" : "+s"(wv));
        IntraIn<DK, DV, TIn> X;
        intra_fetch(X, a, t0, L, item % H, wv, ln);
        if constexpr (FRONT)
            intra_front(X, smem, a, t0, L, inl ? m_cu[seq] : a.cu_seqlens[seq], seq, item % H, wv, ln);
        intra_compute(X, smem, a, recs + ws.rec_bytes * static_cast<size_t>(item), ws, wv, ln, tid);
    }
}

// ---------------------------------------------------------------------------
// 3. Segment carries.  The chunk recurrence S_{c+1} = M_c S_c + B_c (M_c =
//    diag(exp(G_L)) - Kt W, B_c = Kt Ut) is affine in S, so a segment of chunks maps
//    its entering state to S_end = Phi S_start + S_loc.  Three launches:
//      seg_carry<LOCAL>  per (segment, head), every segment but a sequence's last:
//                        runs the chunk steps on [S | Phi] from [0 | I] and stores
//                        S_loc and Phi;
//      seg_scan          per (sequence, head, 16-column tile): S_start of segment 0
//                        is the initial state, S_start(k+1) = Phi_k S_start(k) +
//                        S_loc(k) in fp32;
//      seg_carry<OUT>    per (segment, head): runs the chunk steps from S_start,
//                        writes O, and the sequence's last segment writes the
//                        final state to its slot.
//    A seg_carry workgroup has 8 waves and owns all state columns: wave w computes
//    token block w & 3 of U (w < 4) or of O [OUT] / of the Phi columns' U [LOCAL]
//    (w >= 4), and the state rows of dk block w % (DK/16) for its column blocks.
//    Where [S | Phi] does not fit one CU's LDS (fp32 inputs, dk = 128), the local pass
//    splits the columns over two workgroups (SPLIT = 2; the columns are independent
//    through a chunk step): each takes half of the column blocks, and wave w computes
//    token block w & 3 of U for half of its workgroup's blocks.  A wave's record
//    granules go from the workspace into registers for the next NB chunks (issued
//    unconditionally, clamped to the segment's last chunk); ragged output rows are
//    dropped by the buffer range check.  S and U cross between waves
//    through LDS as whole granules.
// ---------------------------------------------------------------------------
constexpr int kSegThreads = 512;
constexpr int kLocal = 0, kOut = 1;

template <int DK, int DV, class TIn, int MODE, int SPLIT_ = 1>
struct SegPlan {
    using RG = RecGeo<DK, DV, TIn>;
    static constexpr int E = RG::E, CT = RG::CT, GK = RG::GK, GT = RG::GT, NT = RG::NT, TB = RG::NCB;
    static constexpr int NUB = RG::UB / 16;
    static constexpr int VB = DV / 16, KB = DK / 16;
    static constexpr int SPLIT = SPLIT_;
    static constexpr bool OUT = MODE == kOut;
    static constexpr int NCB = MODE == kOut ? VB : VB + KB;  // 16-column blocks of the state
    static constexpr int NCW = NCB / SPLIT;                  // ... held by one workgroup
    static constexpr int HB = NCW / 2;                       // U blocks per wave (SPLIT = 2)
    static constexpr int WPC = 8 / KB;                       // waves per dk block (1 or 2)
    static constexpr int SJB = NCW / WPC;                    // state column blocks per wave
    static constexpr size_t O_SX = 0, O_UX = 16ull * GK * NCW * 64;
    static constexpr size_t BYTES = O_UX + 16ull * GT * NCW * 64;
    static constexpr bool fits = BYTES <= 160 * 1024;
    static_assert(8 % KB == 0 && NCB % SPLIT == 0 && NCW % WPC == 0, "segment plan");
    static_assert(SPLIT == 1 || (SPLIT == 2 && MODE == kLocal && E == 4 && NCW % 2 == 0),
                  "the column split serves the fp32 local pass");
};

// Column split of the local pass: 1 where [S | Phi] fits one workgroup, else 2.
template <int DK, int DV, class TIn>
constexpr int local_split() {
    return SegPlan<DK, DV, TIn, kLocal>::fits || Geo<TIn>::E != 4 ? 1 : 2;
}

// The prefill supports a shape when every kernel's LDS plan fits a CU.
template <int DK, int DV, class TIn>
constexpr bool prefill_fits() {
    return IntraPlan<DK, DV, TIn>::fits && SegPlan<DK, DV, TIn, kLocal, local_split<DK, DV, TIn>()>::fits &&
           SegPlan<DK, DV, TIn, kOut>::fits;
}

// One chunk's operands for one wave.
template <class SP>
struct SegOps {
    u32x4 a[SP::GK];             // W (U task) or QG (O task) granules of the token block
    u32x4 uo[SP::NT][SP::NUB];   // Ut of the token block, every dv tile (U task)
    u32x4 p[SP::GT];             // P granules of the token block (O task)
    u32x4 kt[SP::GT];            // Kt granules of the wave's dk block
    f32x4 gl;                    // exp(G_L) of the wave's rows
    f32x4 us[SP::SPLIT == 2 ? SP::HB : 1];  // SPLIT = 2: Ut of the wave's U blocks (0: Phi)
};

// A record granule: a streaming load in the output pass (the record's last read), so the
// records the output pass has not reached yet stay in the Infinity Cache; a plain load in
// the local pass (the output pass reads the same granules again).
template <bool NTL, class T>
__device__ __forceinline__ T rec_load(const char* p) {
    if constexpr (NTL)
        return __builtin_nontemporal_load(reinterpret_cast<const T*>(p));
    else
        return *reinterpret_cast<const T*>(p);
}

template <class SP>
__device__ __forceinline__ void seg_fetch(SegOps<SP>& F, const char* rec, const WsLayout& ws, int tb, int task,
                                          int cb, int lane, int ub0 = 0) {
    // task (wave-uniform): 0 = U (W, Ut), 1 = O (QG, P), 2 = W alone (the Phi columns' U),
    // 3 = none (the O waves of an output pass without output);
    // SPLIT = 2: W, and Ut of the global column blocks ub0 .. ub0 + HB - 1 that are state
    // columns (zero for Phi columns)
    if constexpr (SP::SPLIT == 2) {
#pragma unroll
        for (int i = 0; i < SP::HB; ++i) {
            const int g = ub0 + i;  // wave-uniform
            F.us[i] = g < SP::VB ? *reinterpret_cast<const f32x4*>(
                                       rec + ws.o_u +
                                       (static_cast<size_t>((g / SP::TB) * 4 + tb) * 64 + lane) * (SP::NUB * 16) +
                                       16 * (g % SP::TB))
                                 : f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    if (task != 3) {
        const char* ab = rec + (task == 1 ? ws.o_q : ws.o_w);
#pragma unroll
        for (int g = 0; g < SP::GK; ++g) {
            const char* pa = ab + ((static_cast<size_t>(tb) * SP::GK + g) * 64 + lane) * 16;
            F.a[g] = rec_load<SP::OUT, u32x4>(pa);
        }
    }
    if (SP::SPLIT == 1 && task == 0) {
#pragma unroll
        for (int t = 0; t < SP::NT; ++t)
#pragma unroll
            for (int n = 0; n < SP::NUB; ++n)
                F.uo[t][n] = rec_load<SP::OUT, u32x4>(
                    rec + ws.o_u + (static_cast<size_t>(t * 4 + tb) * 64 + lane) * (SP::NUB * 16) + 16 * n);
    } else if (task == 1) {
#pragma unroll
        for (int g = 0; g < SP::GT; ++g)
            F.p[g] = rec_load<SP::OUT, u32x4>(rec + ws.o_p + ((static_cast<size_t>(tb) * SP::GT + g) * 64 + lane) * 16);
    }
#pragma unroll
    for (int g = 0; g < SP::GT; ++g)
        F.kt[g] = rec_load<SP::OUT, u32x4>(rec + ws.o_kt + ((static_cast<size_t>(cb) * SP::GT + g) * 64 + lane) * 16);
    F.gl = rec_load<SP::OUT, f32x4>(rec + ws.o_gl + (16 * cb + 4 * (lane >> 4)) * 4);
}

// Value (column block jb, row rr) of a U/O part held as granules, one tile of
// kCarryBV columns per granule set.
__device__ __forceinline__ float uo_val(const u32x4* p, int cb, int rr, BF16) {
    const uint32_t w = p[(cb * 4 + rr) >> 3][((cb * 4 + rr) >> 1) & 3];
    return __uint_as_float((rr & 1) ? (w & 0xffff0000u) : (w << 16));
}
__device__ __forceinline__ float uo_val(const u32x4* p, int cb, int rr, F32) { return __uint_as_float(p[cb][rr]); }

__device__ __forceinline__ void store_out(__amdgpu_buffer_rsrc_t r, int off_elems, float x, F32) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, off_elems * 4, 0, 0);
}

// Accumulator tile (4 values) into its granule slot in LDS: the 8-byte half of a
// bf16 granule, or a whole fp32 granule.
__device__ __forceinline__ void lds_tile_to_gran(char* base, int gran_idx, int half, f32x4 v, BF16) {
    *reinterpret_cast<u32x2*>(base + gran_idx * 16 + half * 8) =
        u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}
__device__ __forceinline__ void lds_tile_to_gran(char* base, int gran_idx, int, f32x4 v, F32) {
    *reinterpret_cast<f32x4*>(base + gran_idx * 16) = v;
}

// O rows 4 (lane/16) + rr of column 16 jb + lane%16 (bf16: lanes r, r ^ 1 store column
// pairs, the even lane rows 0, 1 and the odd lane rows 2, 3, one dword each).
__device__ __forceinline__ void store_o4(__amdgpu_buffer_rsrc_t orsrc, int trow, int orow, int col, f32x4 ov, int r,
                                         BF16) {
    const bool odd = r & 1;
    const uint32_t p01 = pack_bf16x2(ov[0], ov[1]), p23 = pack_bf16x2(ov[2], ov[3]);
    const uint32_t own = odd ? p23 : p01;
    const uint32_t nbr = static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(odd ? p01 : p23), 0xB1, 0xf, 0xf, false));
    const int row = trow + (odd ? 2 : 0), c = col - (r & 1);
    const uint32_t d0 = __builtin_amdgcn_perm(nbr, own, odd ? 0x01000504u : 0x05040100u);
    const uint32_t d1 = __builtin_amdgcn_perm(nbr, own, odd ? 0x03020706u : 0x07060302u);
    __builtin_amdgcn_raw_buffer_store_b32(d0, orsrc, (row * orow + c) * 2, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b32(d1, orsrc, ((row + 1) * orow + c) * 2, 0, 0);
}
__device__ __forceinline__ void store_o4(__amdgpu_buffer_rsrc_t orsrc, int trow, int orow, int col, f32x4 ov, int,
                                         F32) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) store_out(orsrc, (trow + rr) * orow + col, ov[rr], F32{});
}

// Input front: the slot's convolution state after sequence seq (tokens bos .. eos - 1): its
// last W - 1 inputs, earlier state rows (or zeros without h0_from_pool) where the sequence is
// shorter.  Every read precedes every write (a barrier between), since the rows move.
template <int DK, int DV, class TIn>
__device__ void front_state_out(const PrefillArgs& a, int seq, int h, int bos, int eos, int tid) {
    using elem = typename Geo<TIn>::elem;
    constexpr int CW = 2 * DK + DV, NV = (3 * CW + kSegThreads - 1) / kSegThreads;
    const int W = a.front.conv_width, H = a.H;
    elem* cs = static_cast<elem*>(a.front.conv_state) + (static_cast<int64_t>(a.slot_idx[seq]) * H + h) * (W - 1) * CW;
    elem keep[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int idx = tid + i * kSegThreads;
        keep[i] = 0;
        if (idx < (W - 1) * CW) {
            const int r = idx / CW, c = idx % CW, u = eos - (W - 1) + r;
            const int64_t tk = static_cast<int64_t>(u) * H + h;
            if (u >= bos)
                keep[i] = c < DK       ? static_cast<const elem*>(a.q)[tk * DK + c]
                          : c < 2 * DK ? static_cast<const elem*>(a.k)[tk * DK + c - DK]
                                       : static_cast<const elem*>(a.v)[tk * DV + c - 2 * DK];
            else if (a.h0_from_pool)
                keep[i] = cs[(u - bos + W - 1) * CW + c];
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int idx = tid + i * kSegThreads;
        if (idx < (W - 1) * CW) cs[idx] = keep[i];
    }
}

// One chunk on the segment state.
template <class SP, class TIn, int MODE>
__device__ __forceinline__ void seg_step(const SegOps<SP>& F, f32x4 (&S)[SP::SJB], char* sx, char* ux,
                                         __amdgpu_buffer_rsrc_t orsrc, int orow, int ocol, float scale, int tb,
                                         int part, bool with_o, int cb, int jb0, int lane) {
    constexpr TIn tag{};
    constexpr int NCW = SP::NCW;  // column blocks of this workgroup (block indices below are its own)
    const int r = lane & 15, q4 = 4 * (lane >> 4);

    // (1) this wave's state tiles -> S granules (k over dk) in LDS
#pragma unroll
    for (int j = 0; j < SP::SJB; ++j)
        lds_tile_to_gran(sx, ((cb / SP::CT) * NCW + jb0 + j) * 64 + lane, cb % SP::CT, S[j], tag);
    lds_barrier();

    // (2) the token block's U (part 0), and QG S [OUT] or the Phi columns' U [LOCAL] (part 1)
    auto prod = [&](int jb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int g = 0; g < SP::GK; ++g)
            acc = gmma(F.a[g], *reinterpret_cast<const u32x4*>(sx + ((g * NCW + jb) * 64 + lane) * 16), acc, tag);
        return acc;
    };
    const int ug = ((tb / SP::CT) * NCW) * 64 + lane, uh = tb % SP::CT;
    if constexpr (SP::SPLIT == 2) {
        // blocks part * HB .. of this workgroup: U = Ut - W S (Ut zero for Phi columns)
#pragma unroll
        for (int i = 0; i < SP::HB; ++i) {
            const int jb = part * SP::HB + i;
            lds_tile_to_gran(ux, ug + jb * 64, uh, F.us[i] - prod(jb), tag);
        }
    } else if (part == 0) {
#pragma unroll
        for (int jb = 0; jb < SP::VB; ++jb) {
            const f32x4 acc = prod(jb);
            f32x4 uv;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) uv[rr] = uo_val(F.uo[jb / SP::TB], jb % SP::TB, rr, tag) - acc[rr];
            lds_tile_to_gran(ux, ug + jb * 64, uh, uv, tag);
        }
    }
    if constexpr (MODE == kLocal && SP::SPLIT == 1) {
        // the Phi columns' U (no Ut term)
        if (part == 1) {
#pragma unroll
            for (int jb = SP::VB; jb < SP::NCB; ++jb) lds_tile_to_gran(ux, ug + jb * 64, uh, -prod(jb), tag);
        }
    }
    // O task, first half: QG S (the P U half needs this chunk's U)
    f32x4 oacc[MODE == kOut ? SP::VB : 1];
    if constexpr (MODE == kOut) {
        if (part == 1 && with_o) {
#pragma unroll
            for (int jb = 0; jb < SP::VB; ++jb) oacc[jb] = prod(jb);
        }
    }
    lds_barrier();

    // (3) S = exp(G_L) S + Kt U; O = scale (QG S + P U)
#pragma unroll
    for (int j = 0; j < SP::SJB; ++j) {
        f32x4 acc = S[j] * F.gl;
#pragma unroll
        for (int g = 0; g < SP::GT; ++g)
            acc = gmma(F.kt[g], *reinterpret_cast<const u32x4*>(ux + ((g * NCW + jb0 + j) * 64 + lane) * 16),
                       acc, tag);
        S[j] = acc;
    }
    if constexpr (MODE == kOut) {
        if (part == 1 && with_o) {
            const int trow = 16 * tb + q4;
#pragma unroll
            for (int jb = 0; jb < SP::VB; ++jb) {
                f32x4 acc = oacc[jb];
#pragma unroll
                for (int g = 0; g < SP::GT; ++g)
                    acc = gmma(F.p[g], *reinterpret_cast<const u32x4*>(ux + ((g * NCW + jb) * 64 + lane) * 16),
                               acc, tag);
                store_o4(orsrc, trow, orow, ocol + 16 * jb + r, acc * scale, r, tag);
            }
        }
    }
}

template <int DK, int DV, class TIn, int MODE, int NB, int SPLIT>
__global__ __launch_bounds__(kSegThreads) void seg_carry_kernel(PrefillArgs a) {
    using SP = SegPlan<DK, DV, TIn, MODE, SPLIT>;
    constexpr int E = SP::E;
    __shared__ __attribute__((aligned(16))) char smem[SP::BYTES];
    char* sx = smem + SP::O_SX;
    char* ux = smem + SP::O_UX;

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tb = wave & 3, part = wave >> 2;
    const int cb = wave % SP::KB, jb0 = (wave / SP::KB) * SP::SJB;
    // SPLIT = 2: the two workgroups of a (segment, head) have block ids congruent mod
    // kNumXcd (so they run on one XCD and read each record from its L2); half 0 holds the
    // column blocks 0 .. NCW - 1, half 1 the rest
    int pair = blockIdx.x, half = 0;
    if constexpr (SPLIT == 2) {
        pair = (blockIdx.x / (2 * kNumXcd)) * kNumXcd + blockIdx.x % kNumXcd;
        half = (blockIdx.x / kNumXcd) & 1;
    }
    const int cw0 = half * SP::NCW;  // first global column block of this workgroup
    const int H = a.H, s = pair / H, h = pair % H;
    const WsLayout ws(a.num_seqs, a.total_tokens, H, DK, DV, E);
    const char* base = static_cast<const char*>(a.workspace);
    const int32_t* chunk_off = reinterpret_cast<const int32_t*>(base);
    const int32_t* seg_off = reinterpret_cast<const int32_t*>(base + ws.off_segoff);
    if (s >= seg_off[a.num_seqs]) return;
    const int4 sg = reinterpret_cast<const int4*>(base + ws.off_segtab)[s];
    const int seq = sg.x, c_first = sg.y, nc = sg.z, last = sg.w & 1;
    if (MODE == kLocal && last) return;  // the last segment's transition is never used
    char* blk = const_cast<char*>(base) + ws.off_seg + ws.seg_bytes * (static_cast<size_t>(s) * H + h);
    const int r = lane & 15, q4 = 4 * (lane >> 4);

    // state tiles: S[j] holds rows 16 cb + q4 + rr of columns 16 (jb0 + j) + r
    f32x4 S[SP::SJB];
    if constexpr (MODE == kOut) {
        const float* Ss = reinterpret_cast<const float*>(blk + ws.s_start);
#pragma unroll
        for (int j = 0; j < SP::SJB; ++j)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) S[j][rr] = Ss[(16 * cb + q4 + rr) * DV + 16 * (jb0 + j) + r];
    } else {
#pragma unroll
        for (int j = 0; j < SP::SJB; ++j)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                S[j][rr] = (cw0 + jb0 + j >= SP::VB && 16 * cb + q4 + rr == 16 * (cw0 + jb0 + j - SP::VB) + r) ? 1.f
                                                                                                            : 0.f;
    }

    const char* recs = base + ws.off_rec;
    auto rec_of = [&](int c) { return recs + ws.rec_bytes * (static_cast<size_t>(c) * H + h); };
    const bool with_o = a.o != nullptr;  // nullptr: chunk states only (the backward's forward pass)
    const int task = SPLIT == 2 || part == 0 ? 0 : (MODE == kOut ? (with_o ? 1 : 3) : 2);
    const int ub0 = cw0 + part * SP::HB;  // SPLIT = 2: the wave's first U column block
    const int c_last = c_first + nc - 1;
    const int bos = a.cu_seqlens[seq], eos = a.cu_seqlens[seq + 1], cs0 = chunk_off[seq];
    const int orow = H * DV, ocol = h * DV;
    // Prefix snapshot [OUT]: the state after p tokens of the sequence (p > 0, a multiple of
    // snap_every) goes to its snapshot slot, if one is given.  p is wave-uniform.
    auto snapshot = [&](int p) {
        if (p <= 0 || p % a.snap_every != 0) return;
        const int j = p / a.snap_every - 1;
        if (j >= a.max_snaps) return;
        const int slot = a.snap_slots[static_cast<int64_t>(seq) * a.max_snaps + j];
        if (slot < 0) return;
        float* Sn = a.pool + (static_cast<int64_t>(slot) * H + h) * (DK * DV);
#pragma unroll
        for (int j2 = 0; j2 < SP::SJB; ++j2)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) Sn[(16 * cb + q4 + rr) * DV + 16 * (jb0 + j2) + r] = S[j2][rr];
    };
    SegOps<SP> F[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k)
        seg_fetch(F[k], rec_of(min(c_first + k, c_last)), ws, tb, task, cb, lane, ub0);
    for (int c = c_first; c <= c_last; c += NB) {
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            const int cc = c + k;
            if (cc <= c_last) {
                // output rows of this chunk (an empty range in LOCAL mode, which stores nothing)
                const int t0 = bos + kChunk * (cc - cs0), L = min(kChunk, eos - t0);
                const __amdgpu_buffer_rsrc_t orsrc =
                    buf_rsrc(with_o ? static_cast<char*>(a.o) + static_cast<int64_t>(t0) * orow * E : nullptr,
                             MODE == kOut && with_o ? static_cast<int64_t>(L) * orow * E : 0);
                if (MODE == kOut && a.snap_every > 0) snapshot(t0 - bos);  // S = state before this chunk
                if (MODE == kOut && a.chunk_states) {
                    float* Sc = a.chunk_states + (static_cast<size_t>(cc) * H + h) * a.chunk_state_stride;
#pragma unroll
                    for (int j2 = 0; j2 < SP::SJB; ++j2)
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr) Sc[(16 * cb + q4 + rr) * DV + 16 * (jb0 + j2) + r] = S[j2][rr];
                }
                seg_step<SP, TIn, MODE>(F[k], S, sx, ux, orsrc, orow, ocol, a.scale, tb, part, with_o, cb, jb0, lane);
            }
            seg_fetch(F[k], rec_of(min(cc + NB, c_last)), ws, tb, task, cb, lane, ub0);
        }
    }

    // results
    if constexpr (MODE == kOut) {
        if (last) {
            float* Sg = a.pool + (static_cast<int64_t>(a.slot_idx[seq]) * H + h) * (DK * DV);
#pragma unroll
            for (int j = 0; j < SP::SJB; ++j)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) Sg[(16 * cb + q4 + rr) * DV + 16 * (jb0 + j) + r] = S[j][rr];
            if (a.snap_every > 0) snapshot(eos - bos);  // a snapshot at the full length
            if (a.front.gate_scale && a.front.conv_width > 1) front_state_out<DK, DV, TIn>(a, seq, h, bos, eos, tid);
        }
    } else {
        float* Sl = reinterpret_cast<float*>(blk + ws.s_loc);
        float* Ph = reinterpret_cast<float*>(blk + ws.s_phi);
#pragma unroll
        for (int j = 0; j < SP::SJB; ++j) {
            const int jb = cw0 + jb0 + j;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int row = 16 * cb + q4 + rr;
                if (jb < SP::VB)
                    Sl[row * DV + 16 * jb + r] = S[j][rr];
                else
                    Ph[row * DK + 16 * (jb - SP::VB) + r] = S[j][rr];
            }
        }
    }
}

// seg_scan: one workgroup of DK / 16 waves per (sequence, head, 16-column tile); wave w
// owns the tile's rows 16 w .. 16 w + 15 (one row block, so each wave's chain of
// dependent fp32 MFMAs per segment step is DK / 4 long).  X (fp32) -> S_start of each
// segment; X = Phi X + S_loc on fp32 MFMA, X crossing the waves through LDS transposed.
// One column tile of the segment scan of one (sequence, head): walks the segments in
// order, storing S_start(k) and forming S_start(k+1) = Phi_k S_start(k) + S_loc(k).
template <int DK, int DV, int E>
__device__ __forceinline__ void scan_group(const PrefillArgs& a, int group, int tile, float* xs, int lane, int wave) {
    constexpr int KB = DK / 16, RW = 1, LDX = DK + 4;  // one row block per wave
    const int H = a.H;
    const int r = lane & 15, q4 = 4 * (lane >> 4);
    const int seq = group / H, h = group % H;
    const WsLayout ws(a.num_seqs, a.total_tokens, H, DK, DV, E);
    const char* base = static_cast<const char*>(a.workspace);
    const int32_t* seg_off = reinterpret_cast<const int32_t*>(base + ws.off_segoff);
    const int s0 = seg_off[seq], nseg = seg_off[seq + 1] - s0;
    float* Sg = a.pool + (static_cast<int64_t>(a.slot_idx[seq]) * H + h) * (DK * DV) + 16 * tile;
    const int col = 16 * tile + r;

    f32x4 X[RW];
#pragma unroll
    for (int i = 0; i < RW; ++i)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
            X[i][rr] = a.h0_from_pool ? Sg[(16 * (RW * wave + i) + q4 + rr) * DV + r] : 0.f;
    // the initial state has arrived before the loop: otherwise the compiler, merging this
    // path with the loop's back edge, waits for every load in flight at each loop entry
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), the other counters unconstrained
    if (nseg == 0) {
        // no tokens: the final state is the initial state (zero unless read from the slot),
        // and so is the input front's convolution state
        if (!a.h0_from_pool) {
#pragma unroll
            for (int i = 0; i < RW; ++i)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) Sg[(16 * (RW * wave + i) + q4 + rr) * DV + r] = 0.f;
            if (a.front.gate_scale && a.front.conv_width > 1 && tile == 0) {
                const int n = (a.front.conv_width - 1) * (2 * DK + DV) * E;  // bytes
                char* cs = static_cast<char*>(a.front.conv_state) +
                           (static_cast<int64_t>(a.slot_idx[seq]) * H + h) * n;
                for (int i = 64 * wave + lane; i < n / 4; i += 64 * (DK / 16)) reinterpret_cast<uint32_t*>(cs)[i] = 0u;
            }
        }
        return;
    }
    // Phi_k and S_loc(k) rows of this wave, loaded one segment ahead of their use
    struct Ops {
        f32x4 ph[RW][KB], sl[RW];
    };
    auto blk_of = [&](int k) {
        return const_cast<char*>(base) + ws.off_seg + ws.seg_bytes * (static_cast<size_t>(s0 + k) * H + h);
    };
    auto load = [&](Ops& o, int k) {
        const char* blk = blk_of(k);
        const float* Sl = reinterpret_cast<const float*>(blk + ws.s_loc);
        const float* Ph = reinterpret_cast<const float*>(blk + ws.s_phi);
#pragma unroll
        for (int i = 0; i < RW; ++i) {
            const int rb = RW * wave + i;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
                o.ph[i][kb] = *reinterpret_cast<const f32x4*>(Ph + (16 * rb + r) * DK + 16 * kb + q4);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) o.sl[i][rr] = Sl[(16 * rb + q4 + rr) * DV + col];
        }
    };
    // Two segments in flight: step k uses the operands loaded two steps earlier and issues
    // the loads of step k + 2.  The three operand sets rotate by name (the loop is unrolled
    // three times), so no register copy forces a wait for loads still in flight.  X^T goes
    // through LDS buffer k & 1: a step writes the buffer whose last reads (two steps back)
    // ended before the previous step's barrier, so one barrier per step suffices.
    auto step = [&](int k, const Ops& cur, Ops& fill, bool may_end) {
        float* Ss = reinterpret_cast<float*>(blk_of(k) + ws.s_start);
#pragma unroll
        for (int i = 0; i < RW; ++i)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) Ss[(16 * (RW * wave + i) + q4 + rr) * DV + col] = X[i][rr];
        if (may_end && k == nseg - 1) return false;
        load(fill, min(k + 2, nseg - 2));  // the last segment has no transition; repeat a valid one
        float* xb = xs + (k & 1) * 16 * LDX;
#pragma unroll
        for (int i = 0; i < RW; ++i)
            *reinterpret_cast<f32x4*>(xb + r * LDX + 16 * (RW * wave + i) + q4) = X[i];
        lds_barrier();
        // lane (r, q) supplies k = 16 kb + 4q + ks of Phi row 16 rb + r and of X column r
#pragma unroll
        for (int i = 0; i < RW; ++i) {
            f32x4 acc = cur.sl[i];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const f32x4 pb = *reinterpret_cast<const f32x4*>(xb + r * LDX + 16 * kb + q4);
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(cur.ph[i][kb][ks], pb[ks], acc, 0, 0, 0);
            }
            X[i] = acc;
        }
        return true;
    };
    Ops o0, o1, o2;
    if (nseg > 1) {
        load(o0, 0);
        load(o1, min(1, nseg - 2));
    }
    // whole groups of three steps that are not the last (no exit inside the loop body, which
    // lets the compiler keep the loads two steps ahead), then the last one to three steps
    int k = 0;
    for (; k + 3 <= nseg - 1; k += 3) {
        step(k, o0, o2, false);
        step(k + 1, o1, o0, false);
        step(k + 2, o2, o1, false);
    }
    if (step(k, o0, o2, true) && step(k + 1, o1, o0, true)) step(k + 2, o2, o1, true);
    // the next group's first step writes buffer 0: every wave's reads of this group end here
    lds_barrier();
}

template <int DK, int DV, int E>
__global__ __launch_bounds__(64 * (DK / 16)) void seg_scan_kernel(PrefillArgs a) {
    constexpr int NTS = DV / 16, LDX = DK + 4;
    __shared__ __attribute__((aligned(16))) float xs[2 * 16 * LDX];  // X^T [16 columns][DK], two buffers
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // The NTS column tiles of one (sequence, head) all read the same Phi blocks: they get
    // virtual block ids congruent mod kNumXcd, so they run on one XCD and share its L2
    // (the grid is a multiple of kNumXcd, so the grid stride keeps the congruence).
    const int H = a.H, NG = a.num_seqs * H;
    const int nvb = (NG + kNumXcd - 1) / kNumXcd * kNumXcd * NTS;
    for (int vb = blockIdx.x; vb < nvb; vb += gridDim.x) {
        const int j = vb / kNumXcd, tile = j % NTS, group = (j / NTS) * kNumXcd + vb % kNumXcd;
        if (group < NG) scan_group<DK, DV, E>(a, group, tile, xs, lane, wave);
    }
}

constexpr int kMaxDevices = 64;

// Compute units of the current device (looked up once per device; the cache entries are
// atomics, so concurrent first calls only repeat the lookup).
int device_cu_count() {
    static std::atomic<int> cached[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

template <int DK, int DV, class TIn>
hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t stream) {
    if constexpr (!prefill_fits<DK, DV, TIn>()) {
        return hipErrorInvalidConfiguration;
    } else {
        constexpr int E = Geo<TIn>::E;
        const WsLayout ws(a.num_seqs, a.total_tokens, a.H, DK, DV, E);
        char* base = static_cast<char*>(a.workspace);
        const int64_t items = ws.max_chunks * a.H;
        if (!map_inline(a.num_seqs) || items == 0)
            hipLaunchKernelGGL(chunk_map_kernel, dim3(1), dim3(kThreads), 0, stream, a.cu_seqlens, a.num_seqs,
                           ws.seg_chunks, reinterpret_cast<int32_t*>(base), reinterpret_cast<int32_t*>(base + ws.off_segoff),
                           reinterpret_cast<int4*>(base + ws.off_table), reinterpret_cast<int4*>(base + ws.off_segtab));
        if (items > 0) {
            const int slots = 2 * device_cu_count();
            const int grid = static_cast<int>(items < slots ? items : slots);
            if (a.front.gate_scale)
                hipLaunchKernelGGL((chunk_intra_kernel<DK, DV, TIn, true>), dim3(grid), dim3(kThreads), 0, stream, a);
            else
                hipLaunchKernelGGL((chunk_intra_kernel<DK, DV, TIn, false>), dim3(grid), dim3(kThreads), 0, stream, a);
            constexpr int LS = local_split<DK, DV, TIn>();
            const int64_t pairs = ws.max_segs * a.H;
            const dim3 lgrid(static_cast<unsigned>(
                LS == 1 ? pairs : (pairs + kNumXcd - 1) / kNumXcd * kNumXcd * LS));
            hipLaunchKernelGGL((seg_carry_kernel<DK, DV, TIn, kLocal, kCarryNB, LS>), lgrid, dim3(kSegThreads), 0,
                               stream, a);
        }
        // one block per (sequence, head, 16-column tile), padded to whole XCD groups;
        // beyond 4096 such groups the blocks loop
        const int groups = (a.num_seqs * a.H + kNumXcd - 1) / kNumXcd;
        const int sblocks = (groups < 4096 ? groups : 4096) * kNumXcd * (DV / 16);
        hipLaunchKernelGGL((seg_scan_kernel<DK, DV, E>), dim3(sblocks), dim3(64 * (DK / 16)), 0, stream, a);
        if (items > 0)
            hipLaunchKernelGGL((seg_carry_kernel<DK, DV, TIn, kOut, kCarryNB, 1>),
                               dim3(static_cast<unsigned>(ws.max_segs * a.H)), dim3(kSegThreads), 0, stream, a);
        return hipGetLastError();
    }
}

template <class TIn>
hipError_t launch_prefill_dt(const PrefillArgs& a, int dk, int dv, hipStream_t stream) {
    if (dk == 128 && dv == 128) return launch_prefill_t<128, 128, TIn>(a, stream);
    if (dk == 128 && dv == 64) return launch_prefill_t<128, 64, TIn>(a, stream);
    if (dk == 64 && dv == 128) return launch_prefill_t<64, 128, TIn>(a, stream);
    if (dk == 64 && dv == 64) return launch_prefill_t<64, 64, TIn>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace

// The workspace of kda_chunk_prefill_noalloc: one array per GPU, in the code object's
// device memory.  In host code `scratch` names a host-side stand-in, not the device array:
// kernels get the address hipGetSymbolAddress returns on each device, never the name.
static __device__ __attribute__((aligned(256))) char scratch[KDA_NOALLOC_SCRATCH_BYTES];

void* prefill_noalloc_scratch() {
    static std::atomic<void*> addr[kMaxDevices];
    static std::mutex mu;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void* p = addr[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(mu);
    p = addr[dev].load(std::memory_order_relaxed);
    if (!p) {
        // with device `dev` current: its own copy of the array
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        addr[dev].store(p, std::memory_order_release);
    }
    return p;
}

size_t prefill_workspace_bytes(int num_seqs, int64_t total_tokens, int H, int dk, int dv, int bf16) {
    return WsLayout(num_seqs, total_tokens, H, dk, dv, bf16 ? 2 : 4).total;
}

bool prefill_supported(int bf16, int dk, int dv) {
    if (bf16) return true;
    if (dk == 64 && dv == 64) return prefill_fits<64, 64, F32>();
    if (dk == 64 && dv == 128) return prefill_fits<64, 128, F32>();
    if (dk == 128 && dv == 64) return prefill_fits<128, 64, F32>();
    return prefill_fits<128, 128, F32>();
}

hipError_t launch_prefill(const PrefillArgs& a, int bf16, int dk, int dv, hipStream_t stream) {
    return bf16 ? launch_prefill_dt<BF16>(a, dk, dv, stream) : launch_prefill_dt<F32>(a, dk, dv, stream);
}

}  // namespace kda
