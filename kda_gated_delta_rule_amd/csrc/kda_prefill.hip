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
//                                       Ut^T [DV][64] | Ot^T [DV][64]  (element e bytes)
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
// 2. chunk_intra: one workgroup per (chunk, head)
//
// LDS regions are reused by phase (row-major tiles [64][LDK], transposed tiles
// [D][LDT], fp32 tiles [64][LDA]):
//   X1: G (fp32)            | KG, KI          | T (fp32)        | W^T, Ut^T
//   X2: QG
//   X3: KG^T                                   | Q' staging
//   X4: V^T                                    | Ot^T staging
//   X5: Kt^T (write-out)    | A (fp32)        | T' = T diag(beta)
//   X6: P
//   X7: beta, G_L, cumsum part totals, per-wave 16x16 fp32 scratch
// ---------------------------------------------------------------------------
template <int DK, int DV, class TIn>
struct IntraPlan {
    using M = Mma<TIn>;
    using elem = typename M::elem;
    static constexpr int E = sizeof(elem);
    static constexpr int PAD = E == 2 ? 8 : 4;  // rows stay 16-byte aligned and bank-spread
    static constexpr int LDK = DK + PAD;
    static constexpr int LDT = kChunk + PAD;
    static constexpr int LDG = DK + 4;
    static constexpr int LDA = kChunk + 4;
    static constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }
    static constexpr size_t X1 = align_up(cmax(cmax(64ull * LDG * 4, 2ull * 64 * LDK * E),
                                               cmax(64ull * LDA * 4, 1ull * (DK + DV) * LDT * E)), 16);
    static constexpr size_t X2 = align_up(64ull * LDK * E, 16);
    static constexpr size_t X3 = align_up(cmax(1ull * DK * LDT * E, 64ull * LDK * E), 16);
    static constexpr size_t X4 = align_up(1ull * DV * LDT * E, 16);
    static constexpr size_t X5 = align_up(cmax(cmax(1ull * DK * LDT * E, 64ull * LDA * 4), 64ull * LDT * E), 16);
    static constexpr size_t X6 = align_up(64ull * LDT * E, 16);
    static constexpr size_t X7 = align_up(4ull * (64 + DK + 4 * DK) + 4ull * 4 * 16 * 16, 16);
    static constexpr size_t O1 = 0, O2 = O1 + X1, O3 = O2 + X2, O4 = O3 + X3, O5 = O4 + X4;
    static constexpr size_t O6 = O5 + X5, O7 = O6 + X6;
    static constexpr size_t BYTES = O7 + X7;
    static constexpr bool fits = BYTES <= 160 * 1024;
};

// fp32 16x16 block product with both operands row-major:
// C[m][n] += sum_{k < 16} A[m][k] * B[k][n] (v_mfma_f32_16x16x4_f32, 4 steps).
__device__ __forceinline__ f32x4 mma16_nn_f32(const float* A, int lda, const float* B, int ldb,
                                              f32x4 c, int lane) {
    const int r = lane & 15, kq = lane >> 4;
#pragma unroll
    for (int k0 = 0; k0 < 16; k0 += 4)
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(A[r * lda + k0 + kq], B[(k0 + kq) * ldb + r], c, 0, 0, 0);
    return c;
}

// Stores a 16x16 accumulator tile (times s) row-major into fp32 LDS.
__device__ __forceinline__ void store16_f32(float* D, int ld, f32x4 c, float s, int lane) {
    const int col = lane & 15, row = 4 * (lane >> 4);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) D[(row + rr) * ld + col] = s * c[rr];
}

template <int DK, int DV, class TIn>
__global__ __launch_bounds__(kThreads) void chunk_intra_kernel(PrefillArgs a) {
    using P = IntraPlan<DK, DV, TIn>;
    using M = typename P::M;
    using elem = typename P::elem;
    constexpr int E = P::E, LDK = P::LDK, LDT = P::LDT, LDG = P::LDG, LDA = P::LDA;
    static_assert(P::fits, "LDS plan exceeds 160 KiB");
    __shared__ __attribute__((aligned(16))) char smem[P::BYTES];
    float* sG = reinterpret_cast<float*>(smem + P::O1);
    elem* sKG = reinterpret_cast<elem*>(smem + P::O1);
    elem* sKI = reinterpret_cast<elem*>(smem + P::O1 + 64 * LDK * E);
    float* sT = reinterpret_cast<float*>(smem + P::O1);
    elem* sWt = reinterpret_cast<elem*>(smem + P::O1);
    elem* sUt = reinterpret_cast<elem*>(smem + P::O1 + DK * LDT * E);
    elem* sQG = reinterpret_cast<elem*>(smem + P::O2);
    elem* sKGt = reinterpret_cast<elem*>(smem + P::O3);
    elem* sQo = reinterpret_cast<elem*>(smem + P::O3);
    elem* sVt = reinterpret_cast<elem*>(smem + P::O4);
    elem* sOt = reinterpret_cast<elem*>(smem + P::O4);
    elem* sKtt = reinterpret_cast<elem*>(smem + P::O5);
    float* sA = reinterpret_cast<float*>(smem + P::O5);
    elem* sTp = reinterpret_cast<elem*>(smem + P::O5);
    elem* sPm = reinterpret_cast<elem*>(smem + P::O6);
    float* sBeta = reinterpret_cast<float*>(smem + P::O7);
    float* sGL = sBeta + 64;
    float* sTot = sGL + DK;
    float* sScr = sTot + 4 * DK;

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

    // ---- 1. rows (4 threads per token row): q, k, g, v loads; L2 norm; beta ----------
    constexpr int NCH = DK / 4, NCV = DV / 4;
    const int r = tid >> 2, sg = tid & 3, c0 = sg * NCH, j0 = sg * NCV;
    const bool valid = r < L;
    const int64_t tok = static_cast<int64_t>(t0) + r;
    float qv[NCH], kv[NCH];
    {
        const int64_t bk = (tok * H + h) * DK + c0, bv = (tok * H + h) * DV + j0;
#pragma unroll
        for (int i = 0; i < NCH; i += 4) {
            float4 x = make_float4(0.f, 0.f, 0.f, 0.f), y = x, z = x;
            if (valid) {
                x = load4<TIn>(a.q, bk + i);
                y = load4<TIn>(a.k, bk + i);
                z = *reinterpret_cast<const float4*>(a.g + bk + i);
            }
            qv[i] = x.x; qv[i + 1] = x.y; qv[i + 2] = x.z; qv[i + 3] = x.w;
            kv[i] = y.x; kv[i + 1] = y.y; kv[i + 2] = y.z; kv[i + 3] = y.w;
            *reinterpret_cast<float4*>(&sG[r * LDG + c0 + i]) = z;
        }
#pragma unroll
        for (int i = 0; i < NCV; i += 4) {
            float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
            if (valid) x = load4<TIn>(a.v, bv + i);
            sVt[(j0 + i) * LDT + r] = M::from_f32(x.x);
            sVt[(j0 + i + 1) * LDT + r] = M::from_f32(x.y);
            sVt[(j0 + i + 2) * LDT + r] = M::from_f32(x.z);
            sVt[(j0 + i + 3) * LDT + r] = M::from_f32(x.w);
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
    // P's strictly-upper 16x16 blocks are read by the k-loops of phase 7: zero them
    for (int idx = tid; idx < 64 * kChunk; idx += kThreads) {
        const int t = idx / kChunk, s = idx % kChunk;
        if ((s >> 4) > (t >> 4)) sPm[t * LDT + s] = M::from_f32(0.f);
    }
    lds_barrier();

    // ---- 2. gate cumsum over the chunk's tokens, per key channel ----------------------
    {
        constexpr int NP = kThreads / DK, RP = 64 / NP;
        const int c = tid % DK, part = tid / DK;
        float x[RP];
        float run = 0.f;
#pragma unroll
        for (int i = 0; i < RP; ++i) {
            run += sG[(part * RP + i) * LDG + c];
            x[i] = run;
        }
        sTot[part * DK + c] = run;
        lds_barrier();
        float off = 0.f;
        for (int p = 0; p < part; ++p) off += sTot[p * DK + c];
#pragma unroll
        for (int i = 0; i < RP; ++i) sG[(part * RP + i) * LDG + c] = x[i] + off;
        if (part == NP - 1) sGL[c] = x[RP - 1] + off;  // G at row 63 = G_{L-1} (padded rows add 0)
    }
    lds_barrier();

    // ---- 3. operands: KG = kh e^G, KI = kh e^-G, QG = qh e^G, Kt = kh e^(G_L - G) ------
    {
        float gr[NCH];
#pragma unroll
        for (int i = 0; i < NCH; i += 4) {
            const float4 z = *reinterpret_cast<const float4*>(&sG[r * LDG + c0 + i]);
            gr[i] = z.x; gr[i + 1] = z.y; gr[i + 2] = z.z; gr[i + 3] = z.w;
        }
        lds_barrier();  // G (X1) is dead from here: KG and KI take its place
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int c = c0 + i;
            const float eg = __expf(gr[i]), ei = __expf(-gr[i]), et = __expf(sGL[c] - gr[i]);
            const elem kg = M::from_f32(kv[i] * eg);
            sKG[r * LDK + c] = kg;
            sKGt[c * LDT + r] = kg;
            sKI[r * LDK + c] = M::from_f32(kv[i] * ei);
            sQG[r * LDK + c] = M::from_f32(qv[i] * eg);
            sKtt[c * LDT + r] = M::from_f32(kv[i] * et);
        }
    }
    lds_barrier();

    // ---- 4. Kt^T and exp(G_L) to the workspace; A and P on MFMA -------------------------
    {
        constexpr int VE = 16 / E;
        elem* gKt = reinterpret_cast<elem*>(rec + ws.o_kt);
        for (int v = tid; v < DK * kChunk / VE; v += kThreads) {
            const int c = v / (kChunk / VE), t = (v % (kChunk / VE)) * VE;
            *reinterpret_cast<u32x4*>(gKt + c * kChunk + t) =
                *reinterpret_cast<const u32x4*>(sKtt + c * LDT + t);
        }
        float* gGL = reinterpret_cast<float*>(rec + ws.o_gl);
        for (int c = tid; c < DK; c += kThreads) gGL[c] = __expf(sGL[c]);
    }
    {
        // 10 lower-triangular 16x16 tiles for each of A and P: 20 jobs, 5 per wave
        // lower-triangular tile index -> (row block, column block), as bit fields: no
        // data-dependent control flow between the MFMAs and the reads of their results
        f32x4 acc[5];
#pragma unroll
        for (int n = 0; n < 5; ++n) {
            const int job = wave + 4 * n;
            const int which = job / 10, tix = job % 10;
            const int ti = static_cast<int>((0x3333222110ull >> (4 * tix)) & 15);
            const int tj = static_cast<int>((0x3210210100ull >> (4 * tix)) & 15);
            const elem* Aop = (which == 0 ? sKG : sQG) + ti * 16 * LDK;
            acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
            acc[n] = mma_nt<TIn>(Aop, LDK, sKI + tj * 16 * LDK, LDK, 0, DK, acc[n], lane);
        }
        lds_barrier();  // Kt^T (X5) has been copied out: A takes its place
#pragma unroll
        for (int n = 0; n < 5; ++n) {
            const int job = wave + 4 * n;
            const int which = job / 10, tix = job % 10;
            const int ti = static_cast<int>((0x3333222110ull >> (4 * tix)) & 15);
            const int tj = static_cast<int>((0x3210210100ull >> (4 * tix)) & 15);
            const int s = tj * 16 + (lane & 15);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int t = ti * 16 + 4 * (lane >> 4) + rr;
                if (which == 0)
                    sA[t * LDA + s] = s < t ? sBeta[t] * acc[n][rr] : 0.f;
                else
                    sPm[t * LDT + s] = M::from_f32(s <= t ? acc[n][rr] : 0.f);
            }
        }
    }
    lds_barrier();

    // ---- 5. T = (I + A)^-1 (unit lower triangular) in fp32, by 16x16 blocks ------------
    // 5a. diagonal blocks by forward substitution (one thread per block column); the
    //     strictly-upper blocks of T are zero.
    if (wave == 0) {
        const int bi = lane >> 4, col = lane & 15;
        const float* Ab = sA + (16 * bi) * LDA + 16 * bi;
        float x[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            float acc = rr == col ? 1.f : 0.f;
#pragma unroll
            for (int s = 0; s < rr; ++s) acc = fmaf(-Ab[rr * LDA + s], x[s], acc);
            x[rr] = rr < col ? 0.f : acc;
        }
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) sT[(16 * bi + rr) * LDA + 16 * bi + col] = x[rr];
    } else {
        for (int idx = tid - 64; idx < 64 * 64; idx += kThreads - 64) {
            const int t = idx / 64, s = idx % 64;
            if ((s >> 4) > (t >> 4)) sT[t * LDA + s] = 0.f;
        }
    }
    lds_barrier();
    // 5b-d. off-diagonal blocks, one diagonal of blocks at a time:
    //   T_ij = -T_ii * sum_{k=j}^{i-1} A_ik T_kj
    for (int d = 1; d < 4; ++d) {
        if (wave < 4 - d) {
            const int i = wave + d, j = wave;
            f32x4 y = {0.f, 0.f, 0.f, 0.f};
            for (int k = j; k < i; ++k)
                y = mma16_nn_f32(sA + (16 * i) * LDA + 16 * k, LDA, sT + (16 * k) * LDA + 16 * j, LDA, y, lane);
            float* scr = sScr + wave * 256;
            store16_f32(scr, 16, y, 1.f, lane);
            f32x4 z = {0.f, 0.f, 0.f, 0.f};
            z = mma16_nn_f32(sT + (16 * i) * LDA + 16 * i, LDA, scr, 16, z, lane);
            store16_f32(sT + (16 * i) * LDA + 16 * j, LDA, z, -1.f, lane);
        }
        lds_barrier();
    }
    // 5e. T' = T diag(beta) in the MFMA operand type (A, in X5, is dead)
    for (int idx = tid; idx < 64 * 64; idx += kThreads) {
        const int t = idx / 64, s = idx % 64;
        sTp[t * LDT + s] = M::from_f32(sT[t * LDA + s] * sBeta[s]);
    }
    lds_barrier();

    // ---- 6. W = T' KG and Ut = T' V on MFMA -> W^T, Ut^T (T is dead: X1 reused) ----------
    {
        constexpr int NCB = (DK + DV) / 16;
        for (int job = wave; job < 4 * NCB; job += 4) {
            const int ti = job & 3, cb = job >> 2;
            const int kend = 32 * (ti / 2 + 1);  // T' is lower triangular
            const bool isw = cb < DK / 16;
            const elem* Bop = isw ? sKGt + cb * 16 * LDT : sVt + (cb - DK / 16) * 16 * LDT;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mma_nt<TIn>(sTp + ti * 16 * LDT, LDT, Bop, LDT, 0, kend, acc, lane);
            elem* D = isw ? sWt + cb * 16 * LDT : sUt + (cb - DK / 16) * 16 * LDT;
            const int col = lane & 15, t = ti * 16 + 4 * (lane >> 4);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) D[col * LDT + t + rr] = M::from_f32(acc[rr]);
        }
    }
    lds_barrier();

    // ---- 7. Q' = QG - P W -> row-major staging; Ot = P Ut -> Ot^T staging -------------
    {
        constexpr int NCB = (DK + DV) / 16;
        for (int job = wave; job < 4 * NCB; job += 4) {
            const int ti = job & 3, cb = job >> 2;
            const int kend = 32 * (ti / 2 + 1);
            const bool isq = cb < DK / 16;
            const elem* Bop = isq ? sWt + cb * 16 * LDT : sUt + (cb - DK / 16) * 16 * LDT;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mma_nt<TIn>(sPm + ti * 16 * LDT, LDT, Bop, LDT, 0, kend, acc, lane);
            const int col = lane & 15, t = ti * 16 + 4 * (lane >> 4);
            if (isq) {
                const int c = cb * 16 + col;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    sQo[(t + rr) * LDK + c] = M::from_f32(M::to_f32(sQG[(t + rr) * LDK + c]) - acc[rr]);
            } else {
                const int j = (cb - DK / 16) * 16 + col;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) sOt[j * LDT + t + rr] = M::from_f32(acc[rr]);
            }
        }
    }
    lds_barrier();

    // ---- 8. W, Q' (row-major) and Ut^T, Ot^T to the workspace, 16-byte stores ----------
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
            for (int e = 0; e < VE; ++e) tmp[e] = sWt[(c + e) * LDT + t];
            *reinterpret_cast<u32x4*>(gW + t * DK + c) = *reinterpret_cast<const u32x4*>(tmp);
            *reinterpret_cast<u32x4*>(gQ + t * DK + c) = *reinterpret_cast<const u32x4*>(sQo + t * LDK + c);
        }
        for (int v = tid; v < DV * kChunk / VE; v += kThreads) {
            const int j = v / (kChunk / VE), t = (v % (kChunk / VE)) * VE;
            *reinterpret_cast<u32x4*>(gU + j * kChunk + t) = *reinterpret_cast<const u32x4*>(sUt + j * LDT + t);
            *reinterpret_cast<u32x4*>(gO + j * kChunk + t) = *reinterpret_cast<const u32x4*>(sOt + j * LDT + t);
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
    // one operand buffer (per chunk); Ut^T, Ot^T tiles are [BV][LDT]
    static constexpr size_t B_W = 64ull * LDK * E, B_Q = B_W, B_KT = 1ull * DK * LDT * E;
    static constexpr size_t B_U = 1ull * BV * LDT * E, B_O = B_U, B_GL = 4ull * DK;
    static constexpr size_t O_W = 0, O_Q = O_W + B_W, O_KT = O_Q + B_Q, O_U = O_KT + B_KT;
    static constexpr size_t O_O = O_U + B_U, O_GL = O_O + B_O;
    static constexpr size_t BUF = align_up(O_GL + B_GL, 16);
    static constexpr size_t O_ST = 2 * BUF, O_UT = O_ST + align_up(1ull * BV * LDK * E, 16);
    static constexpr size_t BYTES = O_UT + align_up(1ull * BV * LDT * E, 16);
    static constexpr bool fits = BYTES <= 160 * 1024;
    // 16-byte vectors per chunk to stage, per operand (each a multiple of kThreads
    // except exp(G_L))
    static constexpr int VE = 16 / E;
    static constexpr int NV_W = 64 * DK / VE, NV_KT = DK * 64 / VE, NV_U = BV * 64 / VE;
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
    // the tile's rows of Ut^T / Ot^T are contiguous
    const size_t toff = static_cast<size_t>(tile) * CP::BV * kChunk * CP::E;
#pragma unroll
    for (int i = 0; i < CP::PT_U; ++i) {
        const size_t off = toff + static_cast<size_t>(tid + i * kThreads) * 16;
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
        const int j = v / (kChunk / CP::VE), t = (v % (kChunk / CP::VE)) * CP::VE;
        const size_t off = (static_cast<size_t>(j) * CP::LDT + t) * CP::E;
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
    lds_barrier();

    for (int c = c_begin; c < c_end; ++c) {
        char* buf = smem + ((c - c_begin) & 1) * CP::BUF;
        const elem* bW = reinterpret_cast<const elem*>(buf + CP::O_W);
        const elem* bQ = reinterpret_cast<const elem*>(buf + CP::O_Q);
        const elem* bKt = reinterpret_cast<const elem*>(buf + CP::O_KT);
        const elem* bU = reinterpret_cast<const elem*>(buf + CP::O_U);
        const elem* bO = reinterpret_cast<const elem*>(buf + CP::O_O);
        const float* bGL = reinterpret_cast<const float*>(buf + CP::O_GL);
        // this chunk's token range first: vmcnt retires in order, so a load issued after
        // the prefetch below would make its first use wait for the whole prefetch
        const int4 info = table[c];
        const int t0 = info.y, L = info.z;
        // next chunk's operands (the last iteration re-fetches its own chunk, unused)
        const int cn = c + 1 < c_end ? c + 1 : c;
        carry_fetch<CP>(regs, recs + ws.rec_bytes * (static_cast<size_t>(cn) * H + h), ws, tile, tid, DV);

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
        lds_barrier();

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
                uv[rr] = M::to_f32(bU[col * CP::LDT + t]) - u[rr];
                const float ov = a.scale * (o[rr] + M::to_f32(bO[col * CP::LDT + t]));
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
        lds_barrier();

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
        lds_barrier();
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
