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
//   (I + A) W  = beta kh exp(G)          (I + A) Ut = beta V      (UT transform, WY factor)
//   U  = Ut - W S0
//   O  = scale ((qh exp(G) - P W) S0 + P Ut)  =  scale (Q' S0 + Ot)
//   S  = diag(exp(G_L)) S0 + (kh exp(G_L - G))^T U
//
// Three kernels:
//   1. chunk_map    cu_seqlens -> per-sequence chunk offsets and a chunk table
//                   (sequence, first token, length); chunks restart at every
//                   sequence start, the last one may be short.
//   2. chunk_intra  one workgroup per (chunk, head), all chunks in parallel:
//                   Q/K norm, gate cumsum, A and P on MFMA, forward substitution
//                   for W and Ut in fp32, Q' = qh exp(G) - P W and Ot = P Ut on
//                   MFMA; writes W, Q', Kt = (kh exp(G_L - G))^T, Ut, Ot and
//                   exp(G_L) to the workspace.
//   3. chunk_carry  one workgroup per (sequence, head, 32-column dv tile),
//                   sequential over the sequence's chunks: U = Ut - W S,
//                   O = scale (Q' S + Ot), S = exp(G_L) S + Kt U, all on MFMA
//                   from LDS with the next chunk's operands prefetched; the
//                   fp32 state stays in registers and is written to its slot
//                   at the end.
//
// The exp(G_t - G_s) factor is split as exp(G_t) * exp(-G_s) (chunk-start
// reference) so A and P are plain MFMA products.  exp(-G_s) grows along the
// chunk; this is exact up to rounding as long as the within-chunk gate sum stays
// above about -80 (fp32/bf16 exponent range), far outside the gates these
// kernels are fed (a 64-token gate sum of a few units).
//
// MFMA operands are bf16 for bf16 inputs and fp32 for fp32 inputs; every
// accumulation, the cumsum and the triangular solve are fp32.
#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {

namespace {

constexpr int kChunk = 64;
constexpr int kThreads = 256;
constexpr int kCarryBV = 32;  // dv columns per carry workgroup
constexpr int kNumXcd = 8;    // MI355X: 8 XCDs, workgroups dispatched round-robin
constexpr float kNormEps = 1e-6f;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__host__ __device__ constexpr size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---------------------------------------------------------------------------
// Workspace layout (all offsets 256-byte aligned):
//   chunk_off  int32 [num_seqs + 1]     first chunk of each sequence; [num_seqs] = count
//   table      int4  [max_chunks]       {sequence, first token, length, 0}
//   records    [max_chunks * H] of     W [64][DK] | Q' [64][DK] | Kt [DK][64] |
//                                       Ut [64][DV] | Ot [64][DV]  (element e bytes)
//                                       | exp(G_L) [DK] fp32
// ---------------------------------------------------------------------------
struct WsLayout {
    int64_t max_chunks;
    size_t off_table, off_rec, rec_bytes, total;
    size_t o_w, o_q, o_kt, o_u, o_o, o_gl;
    __host__ __device__ WsLayout(int num_seqs, int64_t total_tokens, int H, int dk, int dv, int e) {
        max_chunks = total_tokens / kChunk + num_seqs;
        off_table = align_up(sizeof(int32_t) * (num_seqs + 1), 256);
        off_rec = off_table + align_up(sizeof(int32_t) * 4 * max_chunks, 256);
        o_w = 0;
        o_q = o_w + static_cast<size_t>(kChunk) * dk * e;
        o_kt = o_q + static_cast<size_t>(kChunk) * dk * e;
        o_u = o_kt + static_cast<size_t>(dk) * kChunk * e;
        o_o = o_u + static_cast<size_t>(kChunk) * dv * e;
        o_gl = o_o + static_cast<size_t>(kChunk) * dv * e;
        rec_bytes = align_up(o_gl + sizeof(float) * dk, 256);
        total = off_rec + rec_bytes * static_cast<size_t>(max_chunks) * H;
    }
};

// ---------------------------------------------------------------------------
// 1. chunk map (single workgroup)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void chunk_map_kernel(const int32_t* __restrict__ cu,
                                                             int num_seqs, int32_t* chunk_off,
                                                             int4* table) {
    __shared__ int32_t part[kThreads];
    __shared__ int32_t carry;
    const int tid = threadIdx.x;
    if (tid == 0) carry = 0;
    __syncthreads();
    // exclusive scan of ceil(len / 64) over sequences, in blocks of kThreads
    for (int base = 0; base < num_seqs; base += kThreads) {
        const int i = base + tid;
        int nch = 0;
        if (i < num_seqs) {
            const int len = cu[i + 1] - cu[i];
            nch = len > 0 ? (len + kChunk - 1) / kChunk : 0;
        }
        part[tid] = nch;
        __syncthreads();
        for (int off = 1; off < kThreads; off <<= 1) {  // Hillis-Steele inclusive scan
            const int x = tid >= off ? part[tid - off] : 0;
            __syncthreads();
            part[tid] += x;
            __syncthreads();
        }
        if (i < num_seqs) chunk_off[i] = carry + part[tid] - nch;
        __syncthreads();
        if (tid == kThreads - 1) carry += part[kThreads - 1];
        __syncthreads();
    }
    if (tid == 0) chunk_off[num_seqs] = carry;
    __syncthreads();
    // chunk table
    for (int i = 0; i < num_seqs; ++i) {
        const int bos = cu[i], eos = cu[i + 1];
        const int first = chunk_off[i];
        const int nch = eos > bos ? (eos - bos + kChunk - 1) / kChunk : 0;
        for (int c = tid; c < nch; c += kThreads) {
            const int t0 = bos + c * kChunk;
            table[first + c] = make_int4(i, t0, min(kChunk, eos - t0), 0);
        }
    }
}

// ---------------------------------------------------------------------------
// 2. chunk_intra: LDS plan (bytes), per instantiation
// ---------------------------------------------------------------------------
template <int DK, int DV, class TIn>
struct IntraPlan {
    using M = Mma<TIn>;
    using elem = typename M::elem;
    static constexpr int E = sizeof(elem);
    static constexpr int PAD = E == 2 ? 8 : 4;  // row pad: 16-byte rows stay bank-spread
    static constexpr int LDK = DK + PAD;        // [64][DK] tiles
    static constexpr int LDV = DV + PAD;        // [64][DV] tiles
    static constexpr int LDT = kChunk + PAD;    // transposed [D][64] tiles
    static constexpr int LDG = DK + 4;          // fp32 G
    static constexpr int LDA = kChunk + 4;      // fp32 A
    static constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }
    // regions
    static constexpr size_t R_G = align_up(cmax(64ull * LDG * 4, 64ull * LDA * 4), 16);  // G, then A
    static constexpr size_t R_KG = align_up(cmax(64ull * LDK * E, 64ull * LDK * E), 16);   // KG, then Q'
    static constexpr size_t R_KI = align_up(cmax(64ull * LDK * E, 64ull * LDV * E), 16);   // KI, then Ot
    static constexpr size_t R_QG = align_up(64ull * LDK * E, 16);
    static constexpr size_t R_KT = align_up(cmax(64ull * LDK * E, 1ull * DK * LDT * E), 16);  // Kt rows, then W^T
    static constexpr size_t R_UT = align_up(1ull * DV * LDT * E, 16);
    static constexpr size_t R_PM = align_up(64ull * LDT * E, 16);
    static constexpr size_t R_SM = align_up(4ull * (64 + DK + DK + 4 * DK), 16);  // beta, GL, eGL, totals
    static constexpr size_t O_G = 0, O_KG = O_G + R_G, O_KI = O_KG + R_KG, O_QG = O_KI + R_KI;
    static constexpr size_t O_KT = O_QG + R_QG, O_UT = O_KT + R_KT, O_PM = O_UT + R_UT;
    static constexpr size_t O_SM = O_PM + R_PM;
    static constexpr size_t BYTES = O_SM + R_SM;
    static constexpr bool fits = BYTES <= 160 * 1024;
};

template <int DK, int DV, class TIn>
__global__ __launch_bounds__(kThreads) void chunk_intra_kernel(PrefillArgs a) {
    using P = IntraPlan<DK, DV, TIn>;
    using M = typename P::M;
    using elem = typename P::elem;
    constexpr int E = P::E;
    static_assert(P::fits, "LDS plan exceeds 160 KiB");
    __shared__ __attribute__((aligned(16))) char smem[P::BYTES];
    float* sG = reinterpret_cast<float*>(smem + P::O_G);    // [64][LDG]
    float* sA = reinterpret_cast<float*>(smem + P::O_G);    // [64][LDA] (after G is dead)
    elem* sKG = reinterpret_cast<elem*>(smem + P::O_KG);    // [64][LDK]  kh exp(G)
    elem* sQo = reinterpret_cast<elem*>(smem + P::O_KG);    // [64][LDK]  Q' staging
    elem* sKI = reinterpret_cast<elem*>(smem + P::O_KI);    // [64][LDK]  kh exp(-G)
    elem* sOo = reinterpret_cast<elem*>(smem + P::O_KI);    // [64][LDV]  Ot staging
    elem* sQG = reinterpret_cast<elem*>(smem + P::O_QG);    // [64][LDK]  qh exp(G)
    elem* sKt = reinterpret_cast<elem*>(smem + P::O_KT);    // [64][LDK]  kh exp(G_L - G)
    elem* sWt = reinterpret_cast<elem*>(smem + P::O_KT);    // [DK][LDT]  W^T
    elem* sUt = reinterpret_cast<elem*>(smem + P::O_UT);    // [DV][LDT]  Ut^T
    elem* sPm = reinterpret_cast<elem*>(smem + P::O_PM);    // [64][LDT]  P
    float* sBeta = reinterpret_cast<float*>(smem + P::O_SM);  // [64]
    float* sGL = sBeta + 64;                                   // [DK] G_L
    float* sTot = sGL + DK;                                    // [4][DK] cumsum part totals

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int chunk = blockIdx.x, h = blockIdx.y, H = a.H;
    const WsLayout ws(a.num_seqs, a.total_tokens, H, DK, DV, E);
    const int32_t* chunk_off = static_cast<const int32_t*>(a.workspace);
    if (chunk >= chunk_off[a.num_seqs]) return;
    const int4 info = reinterpret_cast<const int4*>(static_cast<const char*>(a.workspace) +
                                                    ws.off_table)[chunk];
    const int t0 = info.y, L = info.z;
    char* rec = static_cast<char*>(a.workspace) + ws.off_rec +
                ws.rec_bytes * (static_cast<size_t>(chunk) * H + h);

    // ---- 1. rows: load q, k, g; L2 norm; beta --------------------------------
    constexpr int NCH = DK / 4;  // channels per thread (4 threads per row)
    const int r = tid >> 2, sg = tid & 3, c0 = sg * NCH;
    const bool valid = r < L;
    const int64_t tok = static_cast<int64_t>(t0) + r;
    float qv[NCH], kv[NCH];
    {
        const int64_t base = (tok * H + h) * DK + c0;
#pragma unroll
        for (int i = 0; i < NCH; i += 4) {
            float4 x = make_float4(0.f, 0.f, 0.f, 0.f), y = x, z = x;
            if (valid) {
                x = load4<TIn>(a.q, base + i);
                y = load4<TIn>(a.k, base + i);
                z = *reinterpret_cast<const float4*>(a.g + base + i);
            }
            qv[i] = x.x; qv[i + 1] = x.y; qv[i + 2] = x.z; qv[i + 3] = x.w;
            kv[i] = y.x; kv[i + 1] = y.y; kv[i + 2] = y.z; kv[i + 3] = y.w;
            *reinterpret_cast<float4*>(&sG[r * P::LDG + c0 + i]) = z;
        }
    }
    if (a.use_l2) {
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            sq = fmaf(qv[i], qv[i], sq);
            sk = fmaf(kv[i], kv[i], sk);
        }
        sq += __shfl_xor(sq, 1, 64);
        sk += __shfl_xor(sk, 1, 64);
        sq += __shfl_xor(sq, 2, 64);
        sk += __shfl_xor(sk, 2, 64);
        const float iq = 1.f / sqrtf(sq + kNormEps), ik = 1.f / sqrtf(sk + kNormEps);
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            qv[i] *= iq;
            kv[i] *= ik;
        }
    }
    if (sg == 0) sBeta[r] = valid ? a.beta[tok * H + h] : 0.f;
    // P's strictly-upper tiles that the k-loops of step 5 touch must be zero
    for (int idx = tid; idx < 64 * kChunk; idx += kThreads) {
        const int t = idx / kChunk, s = idx % kChunk;
        if ((s >> 4) > (t >> 4)) sPm[t * P::LDT + s] = M::from_f32(0.f);
    }
    __syncthreads();

    // ---- 2. gate cumsum over the chunk's tokens, per key channel --------------
    {
        constexpr int NP = kThreads / DK;  // parts per column
        constexpr int RP = 64 / NP;        // rows per part
        const int c = tid % DK, part = tid / DK;
        float x[RP];
        float run = 0.f;
#pragma unroll
        for (int i = 0; i < RP; ++i) {
            run += sG[(part * RP + i) * P::LDG + c];
            x[i] = run;
        }
        sTot[part * DK + c] = run;
        __syncthreads();
        float off = 0.f;
        for (int p = 0; p < part; ++p) off += sTot[p * DK + c];
#pragma unroll
        for (int i = 0; i < RP; ++i) sG[(part * RP + i) * P::LDG + c] = x[i] + off;
        if (part == NP - 1) sGL[c] = x[RP - 1] + off;  // G at the last row (= G_{L-1}: padded rows add 0)
    }
    __syncthreads();

    // ---- 3. operands: kh exp(G), kh exp(-G), qh exp(G), kh exp(G_L - G) --------
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int c = c0 + i;
        const float G = sG[r * P::LDG + c];
        const float eg = __expf(G), ei = __expf(-G), et = __expf(sGL[c] - G);
        sKG[r * P::LDK + c] = M::from_f32(kv[i] * eg);
        sKI[r * P::LDK + c] = M::from_f32(kv[i] * ei);
        sQG[r * P::LDK + c] = M::from_f32(qv[i] * eg);
        sKt[r * P::LDK + c] = M::from_f32(kv[i] * et);
    }
    __syncthreads();

    // ---- 4a. Kt = (kh exp(G_L - G))^T to the workspace; exp(G_L) -------------------
    {
        elem* gKt = reinterpret_cast<elem*>(rec + ws.o_kt);
        constexpr int VE = 16 / E;                 // elements per 16-byte vector
        constexpr int NV = DK * kChunk / VE;       // vectors in the tile
        for (int v = tid; v < NV; v += kThreads) {
            const int c = v / (kChunk / VE), t = (v % (kChunk / VE)) * VE;
            elem tmp[VE];
#pragma unroll
            for (int e = 0; e < VE; ++e) tmp[e] = sKt[(t + e) * P::LDK + c];
            *reinterpret_cast<uint4*>(gKt + c * kChunk + t) = *reinterpret_cast<const uint4*>(tmp);
        }
        float* gGL = reinterpret_cast<float*>(rec + ws.o_gl);
        for (int c = tid; c < DK; c += kThreads) gGL[c] = __expf(sGL[c]);
    }
    // ---- 4b. A = beta (KG KI^T) strictly lower, P = QG KI^T lower, on MFMA ----------
    {
        // 10 lower-triangular 16x16 tiles for each of A and P: 20 tile jobs, 5 per wave
        for (int job = wave; job < 20; job += 4) {
            const int which = job / 10, tix = job % 10;  // 0: A, 1: P
            int ti = 0, tj = tix;
            while (tj > ti) { tj -= ti + 1; ++ti; }      // tix -> (ti, tj), tj <= ti
            const elem* Aop = (which == 0 ? sKG : sQG) + ti * 16 * P::LDK;
            const elem* Bop = sKI + tj * 16 * P::LDK;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mma_nt<TIn>(Aop, P::LDK, Bop, P::LDK, 0, DK, acc, lane);
            const int s = tj * 16 + (lane & 15);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int t = ti * 16 + 4 * (lane >> 4) + rr;
                if (which == 0)
                    sA[t * P::LDA + s] = s < t ? sBeta[t] * acc[rr] : 0.f;
                else
                    sPm[t * P::LDT + s] = M::from_f32(s <= t ? acc[rr] : 0.f);
            }
        }
    }
    __syncthreads();

    // ---- 5. forward substitution: (I + A) X = [beta KG | beta V], one column per thread
    {
        const int j = tid;
        if (j < DK + DV) {
            float x[kChunk];
            if (j < DK) {
#pragma unroll
                for (int t = 0; t < kChunk; ++t) x[t] = sBeta[t] * M::to_f32(sKG[t * P::LDK + j]);
            } else {
                // unconditional loads (rows past the chunk end re-read its last row and
                // are zeroed by beta = 0), so all 64 are in flight together
                const int jv = j - DK;
#pragma unroll
                for (int t = 0; t < kChunk; ++t) {
                    const int tc = t < L ? t : L - 1;
                    x[t] = load1<TIn>(a.v, ((static_cast<int64_t>(t0) + tc) * H + h) * DV + jv);
                }
#pragma unroll
                for (int t = 0; t < kChunk; ++t) x[t] *= sBeta[t];
            }
            // row t: x_t -= sum_{s<t} A_ts x_s, with 4 independent partial sums
#pragma unroll
            for (int t = 1; t < kChunk; ++t) {
                const float* Arow = sA + t * P::LDA;
                float acc[4] = {x[t], 0.f, 0.f, 0.f};
#pragma unroll
                for (int s4 = 0; s4 < t; s4 += 4) {
                    const float4 av = *reinterpret_cast<const float4*>(Arow + s4);
                    acc[0] = fmaf(-av.x, x[s4], acc[0]);
                    if (s4 + 1 < t) acc[1] = fmaf(-av.y, x[s4 + 1], acc[1]);
                    if (s4 + 2 < t) acc[2] = fmaf(-av.z, x[s4 + 2], acc[2]);
                    if (s4 + 3 < t) acc[3] = fmaf(-av.w, x[s4 + 3], acc[3]);
                }
                x[t] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
            }
            elem* dst = j < DK ? sWt + j * P::LDT : sUt + (j - DK) * P::LDT;
#pragma unroll
            for (int t = 0; t < kChunk; ++t) dst[t] = M::from_f32(x[t]);
        }
    }
    __syncthreads();

    // ---- 6. Q' = QG - P W and Ot = P Ut on MFMA (row block = wave) -------------------
    {
        const int ti = wave;                 // token rows 16 ti .. 16 ti + 15
        const int kend = 32 * (ti / 2 + 1);  // P is lower triangular: s <= t
        const elem* Aop = sPm + ti * 16 * P::LDT;
        for (int cb = 0; cb < DK / 16; ++cb) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mma_nt<TIn>(Aop, P::LDT, sWt + cb * 16 * P::LDT, P::LDT, 0, kend, acc, lane);
            const int c = cb * 16 + (lane & 15);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int t = ti * 16 + 4 * (lane >> 4) + rr;
                sQo[t * P::LDK + c] = M::from_f32(M::to_f32(sQG[t * P::LDK + c]) - acc[rr]);
            }
        }
        for (int cb = 0; cb < DV / 16; ++cb) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mma_nt<TIn>(Aop, P::LDT, sUt + cb * 16 * P::LDT, P::LDT, 0, kend, acc, lane);
            const int c = cb * 16 + (lane & 15);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int t = ti * 16 + 4 * (lane >> 4) + rr;
                sOo[t * P::LDV + c] = M::from_f32(acc[rr]);
            }
        }
    }
    __syncthreads();

    // ---- 7. write W, Q', Ut, Ot (row-major) to the workspace with 16-byte stores ---------
    {
        constexpr int VE = 16 / E;
        elem* gW = reinterpret_cast<elem*>(rec + ws.o_w);
        elem* gQ = reinterpret_cast<elem*>(rec + ws.o_q);
        elem* gU = reinterpret_cast<elem*>(rec + ws.o_u);
        elem* gO = reinterpret_cast<elem*>(rec + ws.o_o);
        for (int v = tid; v < kChunk * DK / VE; v += kThreads) {
            const int t = v / (DK / VE), c = (v % (DK / VE)) * VE;
            elem tmp[VE];
#pragma unroll
            for (int e = 0; e < VE; ++e) tmp[e] = sWt[(c + e) * P::LDT + t];
            *reinterpret_cast<uint4*>(gW + t * DK + c) = *reinterpret_cast<const uint4*>(tmp);
            *reinterpret_cast<uint4*>(gQ + t * DK + c) =
                *reinterpret_cast<const uint4*>(sQo + t * P::LDK + c);
        }
        for (int v = tid; v < kChunk * DV / VE; v += kThreads) {
            const int t = v / (DV / VE), c = (v % (DV / VE)) * VE;
            elem tmp[VE];
#pragma unroll
            for (int e = 0; e < VE; ++e) tmp[e] = sUt[(c + e) * P::LDT + t];
            *reinterpret_cast<uint4*>(gU + t * DV + c) = *reinterpret_cast<const uint4*>(tmp);
            *reinterpret_cast<uint4*>(gO + t * DV + c) =
                *reinterpret_cast<const uint4*>(sOo + t * P::LDV + c);
        }
    }
}

// ---------------------------------------------------------------------------
// 3. chunk_carry
// ---------------------------------------------------------------------------
template <int DK, int DV, class TIn>
struct CarryPlan {
    using M = Mma<TIn>;
    using elem = typename M::elem;
    static constexpr int E = sizeof(elem);
    static constexpr int BV = kCarryBV;
    static constexpr int PAD = E == 2 ? 8 : 4;
    static constexpr int LDK = DK + PAD;      // W, Q' [64][LDK]; S^T [BV][LDK]
    static constexpr int LDT = kChunk + PAD;  // Kt [DK][LDT]; U^T [BV][LDT]
    static constexpr int LDB = BV + PAD;      // Ut, Ot tiles [64][LDB]
    // one operand buffer (per chunk)
    static constexpr size_t B_W = 64ull * LDK * E, B_Q = B_W, B_KT = 1ull * DK * LDT * E;
    static constexpr size_t B_U = 64ull * LDB * E, B_O = B_U, B_GL = 4ull * DK;
    static constexpr size_t O_W = 0, O_Q = O_W + B_W, O_KT = O_Q + B_Q, O_U = O_KT + B_KT;
    static constexpr size_t O_O = O_U + B_U, O_GL = O_O + B_O;
    static constexpr size_t BUF = align_up(O_GL + B_GL, 16);
    static constexpr size_t O_ST = 2 * BUF, O_UT = O_ST + align_up(1ull * BV * LDK * E, 16);
    static constexpr size_t BYTES = O_UT + align_up(1ull * BV * LDT * E, 16);
    static constexpr bool fits = BYTES <= 160 * 1024;
    // 16-byte vectors per chunk to stage, per operand (each a multiple of kThreads
    // except exp(G_L))
    static constexpr int VE = 16 / E;
    static constexpr int NV_W = 64 * DK / VE, NV_KT = DK * 64 / VE, NV_U = 64 * BV / VE;
    static constexpr int NV_GL = DK / 4;
    static constexpr int PT_W = NV_W / kThreads, PT_KT = NV_KT / kThreads, PT_U = NV_U / kThreads;
    static_assert(NV_W % kThreads == 0 && NV_KT % kThreads == 0 && NV_U % kThreads == 0, "");
    static_assert(NV_GL <= kThreads, "");
};

// One chunk's operands in flight: fetched from the workspace into registers while
// the previous chunk computes, then stored to an LDS buffer.
template <class CP>
struct CarryRegs {
    u32x4 w[CP::PT_W], q[CP::PT_W], kt[CP::PT_KT], u[CP::PT_U], o[CP::PT_U], gl;
};

template <class CP>
__device__ __forceinline__ void carry_fetch(CarryRegs<CP>& R, const char* rec, const WsLayout& ws,
                                            int tile, int tid, int DV) {
    const u32x4* gw = reinterpret_cast<const u32x4*>(rec + ws.o_w);
    const u32x4* gq = reinterpret_cast<const u32x4*>(rec + ws.o_q);
    const u32x4* gk = reinterpret_cast<const u32x4*>(rec + ws.o_kt);
#pragma unroll
    for (int i = 0; i < CP::PT_W; ++i) {
        R.w[i] = gw[tid + i * kThreads];
        R.q[i] = gq[tid + i * kThreads];
    }
#pragma unroll
    for (int i = 0; i < CP::PT_KT; ++i) R.kt[i] = gk[tid + i * kThreads];
#pragma unroll
    for (int i = 0; i < CP::PT_U; ++i) {
        const int w = tid + i * kThreads;
        const int t = w / (CP::BV / CP::VE), c = (w % (CP::BV / CP::VE)) * CP::VE;
        const size_t off = (static_cast<size_t>(t) * DV + tile * CP::BV + c) * CP::E;
        R.u[i] = *reinterpret_cast<const u32x4*>(rec + ws.o_u + off);
        R.o[i] = *reinterpret_cast<const u32x4*>(rec + ws.o_o + off);
    }
    if (tid < CP::NV_GL) R.gl = reinterpret_cast<const u32x4*>(rec + ws.o_gl)[tid];
}

template <class CP>
__device__ __forceinline__ void carry_stage(const CarryRegs<CP>& R, char* buf, int tid) {
    constexpr int DK = CP::LDK - CP::PAD;
#pragma unroll
    for (int i = 0; i < CP::PT_W; ++i) {
        const int v = tid + i * kThreads;
        const int t = v / (DK / CP::VE), c = (v % (DK / CP::VE)) * CP::VE;
        const size_t off = (static_cast<size_t>(t) * CP::LDK + c) * CP::E;
        *reinterpret_cast<u32x4*>(buf + CP::O_W + off) = R.w[i];
        *reinterpret_cast<u32x4*>(buf + CP::O_Q + off) = R.q[i];
    }
#pragma unroll
    for (int i = 0; i < CP::PT_KT; ++i) {
        const int v = tid + i * kThreads;
        const int c = v / (kChunk / CP::VE), t = (v % (kChunk / CP::VE)) * CP::VE;
        *reinterpret_cast<u32x4*>(buf + CP::O_KT + (static_cast<size_t>(c) * CP::LDT + t) * CP::E) = R.kt[i];
    }
#pragma unroll
    for (int i = 0; i < CP::PT_U; ++i) {
        const int v = tid + i * kThreads;
        const int t = v / (CP::BV / CP::VE), c = (v % (CP::BV / CP::VE)) * CP::VE;
        const size_t off = (static_cast<size_t>(t) * CP::LDB + c) * CP::E;
        *reinterpret_cast<u32x4*>(buf + CP::O_U + off) = R.u[i];
        *reinterpret_cast<u32x4*>(buf + CP::O_O + off) = R.o[i];
    }
    if (tid < CP::NV_GL) reinterpret_cast<u32x4*>(buf + CP::O_GL)[tid] = R.gl;
}

template <int DK, int DV, class TIn>
__global__ __launch_bounds__(kThreads) void chunk_carry_kernel(PrefillArgs a) {
    using CP = CarryPlan<DK, DV, TIn>;
    using M = typename CP::M;
    using elem = typename CP::elem;
    constexpr int BV = CP::BV, NT = DV / BV;
    static_assert(CP::fits, "LDS plan exceeds 160 KiB");
    __shared__ __attribute__((aligned(16))) char smem[CP::BYTES];
    elem* sSt = reinterpret_cast<elem*>(smem + CP::O_ST);  // S^T [BV][LDK]
    elem* sUt = reinterpret_cast<elem*>(smem + CP::O_UT);  // U^T [BV][LDT]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int H = a.H;
    // XCD-aware mapping: the NT dv tiles of one (sequence, head) share an XCD (and its L2)
    const int groups = a.num_seqs * H;
    const int b = blockIdx.x, xcd = b % kNumXcd, local = b / kNumXcd;
    const int group = (local / NT) * kNumXcd + xcd, tile = local % NT;
    if (group >= groups) return;
    const int seq = group / H, h = group % H;

    const WsLayout ws(a.num_seqs, a.total_tokens, H, DK, DV, CP::E);
    const int32_t* chunk_off = static_cast<const int32_t*>(a.workspace);
    const int4* table = reinterpret_cast<const int4*>(static_cast<const char*>(a.workspace) + ws.off_table);
    const char* recs = static_cast<const char*>(a.workspace) + ws.off_rec;
    const int c_begin = chunk_off[seq], c_end = chunk_off[seq + 1];
    const int slot = a.slot_idx[seq];
    float* Sg = a.pool + (static_cast<int64_t>(slot) * H + h) * (DK * DV) + tile * BV;

    // state tiles owned by this wave: dk row blocks 2 wave, 2 wave + 1 (x DK/128) and both
    // 16-column blocks of the dv tile.  S[rb][cb] holds rows 16 rb + 4 (lane/16) + r.
    constexpr int RB = DK / 16 / 4;  // row blocks per wave (2 for DK = 128, 1 for 64)
    f32x4 S[RB][2];
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            const int col = cb * 16 + (lane & 15);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int row = (wave * RB + i) * 16 + 4 * (lane >> 4) + rr;
                S[i][cb][rr] = a.h0_from_pool ? Sg[row * DV + col] : 0.f;
            }
        }

    CarryRegs<CP> regs;
    if (c_begin < c_end) {
        carry_fetch<CP>(regs, recs + ws.rec_bytes * (static_cast<size_t>(c_begin) * H + h), ws, tile,
                        tid, DV);
        carry_stage<CP>(regs, smem, tid);
    }
    __syncthreads();

    for (int c = c_begin; c < c_end; ++c) {
        char* buf = smem + ((c - c_begin) & 1) * CP::BUF;
        const elem* bW = reinterpret_cast<const elem*>(buf + CP::O_W);
        const elem* bQ = reinterpret_cast<const elem*>(buf + CP::O_Q);
        const elem* bKt = reinterpret_cast<const elem*>(buf + CP::O_KT);
        const elem* bU = reinterpret_cast<const elem*>(buf + CP::O_U);
        const elem* bO = reinterpret_cast<const elem*>(buf + CP::O_O);
        const float* bGL = reinterpret_cast<const float*>(buf + CP::O_GL);
        // next chunk's operands (the last iteration re-fetches its own chunk, unused)
        const int cn = c + 1 < c_end ? c + 1 : c;
        carry_fetch<CP>(regs, recs + ws.rec_bytes * (static_cast<size_t>(cn) * H + h), ws, tile, tid, DV);
        const int4 info = table[c];
        const int t0 = info.y, L = info.z;

        // (1) S (fp32 registers) -> S^T operand in LDS
#pragma unroll
        for (int i = 0; i < RB; ++i)
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
                const int col = cb * 16 + (lane & 15);
                const int row = (wave * RB + i) * 16 + 4 * (lane >> 4);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) sSt[col * CP::LDK + row + rr] = M::from_f32(S[i][cb][rr]);
            }
        __syncthreads();

        // (2) U = Ut - W S and O = scale (Q' S + Ot): token rows 16 wave .. +15
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            f32x4 u = {0.f, 0.f, 0.f, 0.f}, o = u;
            u = mma_nt<TIn>(bW + wave * 16 * CP::LDK, CP::LDK, sSt + cb * 16 * CP::LDK, CP::LDK, 0, DK, u, lane);
            o = mma_nt<TIn>(bQ + wave * 16 * CP::LDK, CP::LDK, sSt + cb * 16 * CP::LDK, CP::LDK, 0, DK, o, lane);
            const int col = cb * 16 + (lane & 15);
            const int trow = wave * 16 + 4 * (lane >> 4);
            float uv[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int t = trow + rr;
                uv[rr] = M::to_f32(bU[t * CP::LDB + col]) - u[rr];
                const float ov = a.scale * (o[rr] + M::to_f32(bO[t * CP::LDB + col]));
                if (t < L) {
                    const int64_t oi = ((static_cast<int64_t>(t0) + t) * H + h) * DV + tile * BV + col;
                    if constexpr (CP::E == 2)
                        static_cast<uint16_t*>(a.o)[oi] = f32_to_bf16(ov);
                    else
                        static_cast<float*>(a.o)[oi] = ov;
                }
            }
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) sUt[col * CP::LDT + trow + rr] = M::from_f32(uv[rr]);
        }
        __syncthreads();

        // (3) S = exp(G_L) S + Kt U
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            const int rb = wave * RB + i;
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
                f32x4 acc;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) acc[rr] = S[i][cb][rr] * bGL[rb * 16 + 4 * (lane >> 4) + rr];
                S[i][cb] = mma_nt<TIn>(bKt + rb * 16 * CP::LDT, CP::LDT, sUt + cb * 16 * CP::LDT, CP::LDT, 0,
                                       kChunk, acc, lane);
            }
        }
        carry_stage<CP>(regs, smem + ((c + 1 - c_begin) & 1) * CP::BUF, tid);
        __syncthreads();
    }

    // final state back to the slot
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            const int col = cb * 16 + (lane & 15);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int row = (wave * RB + i) * 16 + 4 * (lane >> 4) + rr;
                Sg[row * DV + col] = S[i][cb][rr];
            }
        }
}

template <int DK, int DV, class TIn>
hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t stream) {
    if constexpr (!IntraPlan<DK, DV, TIn>::fits || !CarryPlan<DK, DV, TIn>::fits) {
        return hipErrorInvalidConfiguration;
    } else {
        constexpr int E = sizeof(typename Mma<TIn>::elem);
        const WsLayout ws(a.num_seqs, a.total_tokens, a.H, DK, DV, E);
        int32_t* chunk_off = static_cast<int32_t*>(a.workspace);
        int4* table = reinterpret_cast<int4*>(static_cast<char*>(a.workspace) + ws.off_table);
        hipLaunchKernelGGL(chunk_map_kernel, dim3(1), dim3(kThreads), 0, stream, a.cu_seqlens,
                           a.num_seqs, chunk_off, table);
        if (ws.max_chunks > 0)
            hipLaunchKernelGGL((chunk_intra_kernel<DK, DV, TIn>),
                               dim3(static_cast<unsigned>(ws.max_chunks), a.H), dim3(kThreads), 0,
                               stream, a);
        const int groups = a.num_seqs * a.H;
        const int grid = (groups + kNumXcd - 1) / kNumXcd * kNumXcd * (DV / kCarryBV);
        hipLaunchKernelGGL((chunk_carry_kernel<DK, DV, TIn>), dim3(grid), dim3(kThreads), 0, stream, a);
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

size_t prefill_workspace_bytes(int num_seqs, int64_t total_tokens, int H, int dk, int dv, int bf16) {
    return WsLayout(num_seqs, total_tokens, H, dk, dv, bf16 ? 2 : 4).total;
}

bool prefill_supported(int bf16, int dk, int dv) {
    if (bf16) return true;
    if (dk == 64 && dv == 64) return IntraPlan<64, 64, F32>::fits && CarryPlan<64, 64, F32>::fits;
    if (dk == 64 && dv == 128) return IntraPlan<64, 128, F32>::fits && CarryPlan<64, 128, F32>::fits;
    if (dk == 128 && dv == 64) return IntraPlan<128, 64, F32>::fits && CarryPlan<128, 64, F32>::fits;
    return IntraPlan<128, 128, F32>::fits && CarryPlan<128, 128, F32>::fits;
}

hipError_t launch_prefill(const PrefillArgs& a, int bf16, int dk, int dv, hipStream_t stream) {
    return bf16 ? launch_prefill_dt<BF16>(a, dk, dv, stream) : launch_prefill_dt<F32>(a, dk, dv, stream);
}

}  // namespace kda
