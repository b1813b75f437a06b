// prefill_mfma.hip -- chunked KDA prefill on MFMA (gfx950): a prep kernel
// and a scan kernel.
//
// Method: the chunk unrolling of the Kimi K3 explainer's FlashKDA paragraph
// (Q_decay, K_restore, causal M_qk, UT transform for the pseudo-values U).
// With a = in-chunk cumulative log-decay, gamma = exp(a_last):
//     Kd = k * exp(a),  Qd = q * exp(a),  Kr = k * exp(a_last - a)
//     Mqk[t,s] = sum_c q_t k_s exp(a_t - a_s)   (s <= t)
//     L[t,s]   = beta_t sum_c k_t k_s exp(a_t - a_s)   (s < t)
//     IB       = (I + L)^{-1} Diag(beta)
// and per chunk of one (sequence, head), with the state M = S^T:
//     U     = IB (V - Kd M)
//     O     = Qd M + Mqk U
//     M_out = Diag(gamma) M + Kr^T U
//
// prep  (persistent, one workgroup per CU walking the (chunk, head) items,
//       all chunks in parallel): decays as products of alpha = exp(g) inside
//       16-token blocks; L and Mqk with the diagonal 16x16 blocks on fp32
//       MFMA and the off-diagonal ones on fp16 MFMA (every factor <= 1 there);
//       the unit-lower-triangular inverse by substitution on the diagonal
//       blocks and fp32 MFMA products off it; and a record of the scan's
//       operands in fp16, laid out as MFMA fragments so that the scan loads
//       them with 16-byte coalesced reads.
// scan  (one workgroup per (sequence, head, 16- or 32-column value tile), its
//       chunks in order): four recurrence wavefronts keep the fp32 state tile
//       in registers and form X = Kd M, U = IB (V - X) and the state update on
//       fp16 MFMA with the right operand (state, V - X, U) split into fp16
//       hi + lo and fp32 accumulation; four output wavefronts form o from the
//       state and U the recurrence shares in LDS.
//
// Every decay factor that is formed is <= 1, except on the diagonal 16x16
// blocks of L and Mqk, which use the block's own start as reference: their
// factors exp(a_start - a_s) are bounded by 1 / (whole-block decay), and a
// block whose decay leaves the fp32 normal range takes an exact per-element
// path instead.
#include <algorithm>

#include "kda_chunks.h"
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int D = 128;       // Dk == Dv
constexpr int C = 64;        // chunk length
constexpr int NTHR = 256;    // scan: 4 recurrence wavefronts, one per SIMD ...
constexpr int SCAN_THR = 2 * NTHR;   // ... and 4 output wavefronts beside them
constexpr float kTiny = 1.17549435e-38f;  // FLT_MIN

// Which right-hand operands of the scan's fp16 contractions are split into
// hi + lo (two MFMAs) rather than rounded once. The state update keeps ~22
// bits in every operand that feeds back into the state (X, V - X, U). The
// output-only products (formed by the output wavefronts) are split too on
// 16-column tiles, where those wavefronts have the time (measured slightly
// faster, o error 2.5e-3 -> 1.4e-3 x RMS on the 8k workload), and round once
// (11 bits) on 32-column tiles, where splitting them lengthened the step;
// KDA_SPLIT_OI / KDA_SPLIT_UO = 1 split them on both.
#ifndef KDA_SPLIT_X
#define KDA_SPLIT_X 1     // the state in X = Kd M
#endif
#ifndef KDA_SPLIT_OI
#define KDA_SPLIT_OI 0    // the state in O = Qd M on 32-column tiles (o only: its error is not fed back)
#endif
#ifndef KDA_SPLIT_Y
#define KDA_SPLIT_Y 1     // V - X in U = IB (V - X)
#endif
#ifndef KDA_SPLIT_U
#define KDA_SPLIT_U 1     // U in M += Kr^T U
#endif
#ifndef KDA_SCAN_MIN_WAVES
#define KDA_SCAN_MIN_WAVES 1  // scan waves per SIMD its registers must allow (4: two workgroups per CU, 128 registers)
#endif
#ifndef KDA_SCAN_BUFS
#define KDA_SCAN_BUFS 3   // scan operand buffers in rotation (loads two chunks ahead)
#endif
#ifndef KDA_SPLIT_UO
#define KDA_SPLIT_UO 0    // U in O += Mqk U on 32-column tiles (o only)
#endif

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 lds8(const __bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }
__device__ __forceinline__ f16x8 lds8h(const _Float16 *p) { return *reinterpret_cast<const f16x8 *>(p); }
__device__ __forceinline__ float bf2f(__bf16 x) { return static_cast<float>(x); }

// Raw buffer access (buf_rsrc): the ragged tail of a sequence needs no branch,
// and no per-lane 64-bit address arithmetic is spent per access.
template <typename T>
__device__ __forceinline__ T buf_ld16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
template <typename T> __device__ __forceinline__ void buf_st(__amdgpu_buffer_rsrc_t r, int voff, float x);
template <> __device__ __forceinline__ void buf_st<float>(__amdgpu_buffer_rsrc_t r, int voff, float x) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x), r, voff, 0, 0);
}
template <> __device__ __forceinline__ void buf_st<bf16_t>(__amdgpu_buffer_rsrc_t r, int voff, float x) {
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, static_cast<__bf16>(x)), r, voff, 0, 0);
}

template <typename T> __device__ __forceinline__ float ld_scalar(const T *p, size_t i);
template <> __device__ __forceinline__ float ld_scalar<float>(const float *p, size_t i) { return p[i]; }
template <> __device__ __forceinline__ float ld_scalar<bf16_t>(const bf16_t *p, size_t i) {
    return bf16_to_f32(p[i]);
}
template <typename T> __device__ __forceinline__ void st_scalar(T *p, size_t i, float x);
template <> __device__ __forceinline__ void st_scalar<float>(float *p, size_t i, float x) { p[i] = x; }
template <> __device__ __forceinline__ void st_scalar<bf16_t>(bf16_t *p, size_t i, float x) {
    p[i] = __builtin_bit_cast(bf16_t, static_cast<__bf16>(x));
}

// x = hi + lo, hi = bf16(x), lo = bf16(x - hi): about 16 significant bits
#define SPLIT2(x, HI, LO)                                   \
    do {                                                    \
        const float x_ = (x);                               \
        const __bf16 h_ = static_cast<__bf16>(x_);          \
        (HI) = h_;                                          \
        (LO) = static_cast<__bf16>(x_ - bf2f(h_));          \
    } while (0)
// the same in fp16: about 22 significant bits (|x| < 65504)
#define SPLITH(x, HI, LO)                                   \
    do {                                                    \
        const float x_ = (x);                               \
        const _Float16 h_ = static_cast<_Float16>(x_);      \
        (HI) = h_;                                          \
        (LO) = static_cast<_Float16>(x_ - static_cast<float>(h_)); \
    } while (0)

// ---------------------------------------------------------------- record
// Per (chunk, head): for each wavefront role w (tokens 16w..16w+15 and
// channels 32w..32w+31) 16 KB of fp16 fragments [operand][k-step][lane][8],
// then d_t = q_t . k_t (fp32 [64]) and gamma (fp32 [128]). Records are
// stored head-major (index head * records-per-head + chunk), so the records a
// scan chain walks through are contiguous in memory.
struct Rec {
    static constexpr int WAVE = 16384;
    static constexpr int KD = 0, QD = 4096, IB = 8192, MQ = 10240, KR = 12288;
    static constexpr int DG = 4 * WAVE, GAM = DG + C * 4, BYTES = GAM + D * 4;
};

// ---------------------------------------------------------------- prep
template <int N> struct IC { static constexpr int value = N; };    // an int as a type (compile-time argument)
constexpr int PTHR = 512;        // prep: 8 wavefronts, two per SIMD to hide latency
constexpr int SQ = D + 8;        // bf16 row stride of q, k           [64][136]
constexpr int SE = D + 4;        // fp32 row stride of the decays     [64][132]
constexpr int SL = C + 4;        // fp32 row stride of L / INV^T      [64][68]
constexpr int SMQ = C + 8;       // fp16 row stride of Mqk            [64][72]
constexpr int SKR = C + 8;       // fp16 row stride of Kr^T           [128][72]

struct PrepLds {
    static constexpr int Q = 0;
    static constexpr int K = Q + C * SQ * 2;
    static constexpr int E = K + C * SQ * 2;         // fp32 in-block prefix decay
    static constexpr int F = E + C * SE * 4;         // fp32 in-block suffix decay
    static constexpr int LI = F + C * SE * 4;        // fp32 L (strictly lower) and INV^T (upper, with diagonal)
    static constexpr int MQK = LI + C * SL * 4;      // fp16 strictly lower Mqk
    static constexpr int DG = MQK + C * SMQ * 2;     // fp32 [64]
    static constexpr int BETA = DG + C * 4;          // fp32 [64]
    static constexpr int GB = BETA + C * 4;          // fp32 [4][128] block decays
    static constexpr int G = GB + 4 * D * 4;         // fp32 [4][128] decay chunk start -> block start
    static constexpr int GAM = G + 4 * D * 4;        // fp32 [128]
    static constexpr int RQ = GAM + D * 4;           // fp32 [64] 1 / ||q_t|| (L2-normalised input)
    static constexpr int RK = RQ + C * 4;            // fp32 [64] 1 / ||k_t||
    static constexpr int FLAG = RK + C * 4;          // int [4]
    static constexpr int T3 = FLAG + 16;             // fp32 [4][256] inverse scratch
    static constexpr int KRT = T3 + 4 * 256 * 4;     // fp16 [128][SKR] Kr^T, channel-major
    static constexpr int SIZE = KRT + D * SKR * 2;
};

struct PrepParams {
    const bf16_t *q, *k;
    const float *g;
    const void *beta;
    SeqView sv;
    const int2 *meta;            // packed sequences: {first token, length} of every chunk
    int H;
    char *rec;
    long long rec_stride;        // records per head (head-major record layout)
    float norm_eps;              // NORM: q_t / sqrt(||q_t||^2 + eps), the same for k_t
};

// {first token, length} of every chunk of packed sequences (zeros past the last)
__global__ __launch_bounds__(256) void chunk_meta_kernel(SeqView sv, int2 *meta, int maxc) {
    const int ci = blockIdx.x * 256 + threadIdx.x;
    if (ci >= maxc) return;
    if (ci >= sv.total_chunks()) { meta[ci] = int2{0, 0}; return; }
    const int n = sv.seq_of_chunk(ci);
    const int tok0 = sv.seq_start(n) + (ci - sv.first_chunk(n)) * C;
    meta[ci] = int2{tok0, min(C, sv.seq_end(n) - tok0)};
}

// GHEAD: one log-decay per (token, head), g [T][H] or none (nullptr), instead
// of one per key channel. NORM: q and k are L2-normalised over the channels on
// the fly: the staged rows stay the bf16 inputs, and 1/||q_t||, 1/||k_t|| (fp32)
// scale every product they enter before its operands are rounded.
template <typename TB, bool VARLEN, bool GHEAD, bool NORM>
__global__ __launch_bounds__(PTHR) void chunk_prep_kernel(PrepParams p) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    using Lo = PrepLds;
    static_assert(Lo::SIZE <= 163840, "LDS budget");
    __bf16 *sQ = reinterpret_cast<__bf16 *>(smem + Lo::Q);
    __bf16 *sK = reinterpret_cast<__bf16 *>(smem + Lo::K);
    float *sE = reinterpret_cast<float *>(smem + Lo::E);
    float *sF = reinterpret_cast<float *>(smem + Lo::F);
    float *sLI = reinterpret_cast<float *>(smem + Lo::LI);
    _Float16 *sMqk = reinterpret_cast<_Float16 *>(smem + Lo::MQK);
    float *sDg = reinterpret_cast<float *>(smem + Lo::DG);
    float *sBeta = reinterpret_cast<float *>(smem + Lo::BETA);
    float *sGB = reinterpret_cast<float *>(smem + Lo::GB);
    float *sG = reinterpret_cast<float *>(smem + Lo::G);
    float *sGam = reinterpret_cast<float *>(smem + Lo::GAM);
    float *sRQ = reinterpret_cast<float *>(smem + Lo::RQ);
    float *sRK = reinterpret_cast<float *>(smem + Lo::RK);
    int *sFlag = reinterpret_cast<int *>(smem + Lo::FLAG);
    float *sT3 = reinterpret_cast<float *>(smem + Lo::T3);
    _Float16 *sKrt = reinterpret_cast<_Float16 *>(smem + Lo::KRT);

    const int tid0 = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid0 >> 6);   // 8 wavefronts
    const int H = p.H;
    const int items = p.sv.total_chunks() * H;

    // Inputs of one (chunk, head) item, fetched one item ahead. The loads are
    // issued unmasked (rows past the end read the last row) and masked when
    // staged, and the next fetch is unconditional (clamped item index): a load
    // that is used right away or issued under a branch makes the compiler wait
    // for every load in flight.
    // {first token, length} of global chunk ci: arithmetic for dense batches; for
    // packed sequences from the chunk table, read one fetch ahead so that the
    // value is never waited for right after its load (such a wait would also
    // wait for the previous item's record stores)
    auto dense_meta = [&](int ci) {
        const int n = ci / p.sv.dense_chunks();
        const int tok0 = n * p.sv.T + (ci - n * p.sv.dense_chunks()) * C;
        return int2{tok0, min(C, (n + 1) * p.sv.T - tok0)};
    };
    int2 meta_ahead = {0, 0};
    if constexpr (VARLEN)
        if ((int)blockIdx.x < items) meta_ahead = p.meta[(int)blockIdx.x / H];
    u32x4 rq[2], rk[2];
    float rg[16];                // g of (token 16 (tid >> 7) + tt, channel tid & 127), tt < 16
    TB rbeta = TB(0);
    int nx_h = 0, nx_tok0 = 0, nx_Lc = 0;
    // part 0: chunk bounds, q and k; part 1: g; part 2: beta; -1: all. The
    // parts go out in different phases of the current item, so that no phase
    // stalls on a full vector-memory queue.
    auto fetch = [&](int item, int part) {
        if (part <= 0) {
            const int ci = item / H;
            int2 m;
            if constexpr (VARLEN) {
                m = meta_ahead;
                meta_ahead = p.meta[min(item + (int)gridDim.x, items - 1) / H];
            } else {
                m = dense_meta(ci);
            }
            nx_h = item % H;
            nx_tok0 = m.x;
            nx_Lc = m.y;
        }
        const int h = nx_h, tok0 = nx_tok0, Lc = nx_Lc;
        if (part <= 0) {
#pragma unroll
            for (int it = 0; it < 2; ++it) {
                const int idx = tid0 + it * PTHR, row = idx >> 4, part = idx & 15;
                const size_t off = ((size_t)(tok0 + min(row, Lc - 1)) * H + h) * D + 8 * part;
                rq[it] = *reinterpret_cast<const u32x4 *>(p.q + off);
                rk[it] = *reinterpret_cast<const u32x4 *>(p.k + off);
            }
        }
        if (part == -1 || part == 1) {
            // thread (block I, channel c) takes the 16 rows of its block at its
            // channel: for each row the 128 threads of a block read 512
            // contiguous bytes, and the decay products then stay in registers
            const int I = tid0 >> 7, c = tid0 & (D - 1);
            if constexpr (GHEAD) {
                // one value per row, broadcast over the channels; without a gate the
                // range is empty and every load reads 0 (alpha = 1)
                const auto rgh = buf_rsrc(p.g ? p.g + (size_t)tok0 * H + h : nullptr, p.g ? ((Lc - 1) * H + 1) * 4 : 0);
#pragma unroll
                for (int tt = 0; tt < 16; ++tt)
                    rg[tt] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rgh, min(16 * I + tt, Lc - 1) * H * 4, 0, 0));
            } else {
                const auto rgc = buf_rsrc(p.g + ((size_t)tok0 * H + h) * D, ((Lc - 1) * H + 1) * D * 4);
#pragma unroll
                for (int tt = 0; tt < 16; ++tt)
                    rg[tt] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rgc, (min(16 * I + tt, Lc - 1) * H * D + c) * 4, 0, 0));
            }
        }
        if (part == -1 || part == 2)
            rbeta = static_cast<const TB *>(p.beta)[(size_t)(tok0 + min(tid0 & 63, Lc - 1)) * H + h];
    };
    // One item: stage, decays, L / Mqk, inverse, record. The first item is a
    // separate copy of the body, so that the loop is entered only from the end of
    // an item: the compiler's wait for the next item's inputs then counts the
    // record stores issued after them and does not wait for those stores.
    auto body = [&](int item) __attribute__((always_inline)) {
        const int ci = item / H, h = nx_h, tok0 = nx_tok0, Lc = nx_Lc;
        // per-thread LDS addresses are recomputed every item instead of being
        // hoisted out of the loop and held in registers for its whole length
        int tid = tid0;
        asm volatile("" : "+v"(tid));
        const int lane = tid & 63, l16 = lane & 15, lq = lane >> 4;

        // ================= stage the chunk in LDS (rows past the end: zeros, alpha = 1)
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int idx = tid + it * PTHR, row = idx >> 4, part = idx & 15;
            const u32x4 z0 = {0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4 *>(sQ + row * SQ + 8 * part) = row < Lc ? rq[it] : z0;
            *reinterpret_cast<u32x4 *>(sK + row * SQ + 8 * part) = row < Lc ? rk[it] : z0;
            if constexpr (NORM) {
                // sums of squares over the 16 threads of the row (lanes 16j..16j+15)
                const bf16x8 qx = __builtin_bit_cast(bf16x8, rq[it]), kx = __builtin_bit_cast(bf16x8, rk[it]);
                float sq = 0.f, sk = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    sq += bf2f(qx[e]) * bf2f(qx[e]);
                    sk += bf2f(kx[e]) * bf2f(kx[e]);
                }
#pragma unroll
                for (int o = 1; o < 16; o <<= 1) {
                    sq += __shfl_xor(sq, o, 64);
                    sk += __shfl_xor(sk, o, 64);
                }
                if (part == 0) {
                    sRQ[row] = row < Lc ? 1.f / sqrtf(sq + p.norm_eps) : 1.f;
                    sRK[row] = row < Lc ? 1.f / sqrtf(sk + p.norm_eps) : 1.f;
                }
            }
        }
        // in-block suffix (F) and prefix (E) products of alpha = exp(g), one
        // (block, channel) per thread, from the registers (rows past the end: alpha = 1)
        {
            const int I = tid >> 7, c = tid & 127;
            float al[16];
#pragma unroll
            for (int tt = 0; tt < 16; ++tt) al[tt] = 16 * I + tt < Lc ? __expf(rg[tt]) : 1.f;
            float f = 1.f;
#pragma unroll
            for (int tt = 15; tt >= 0; --tt) {
                sF[(16 * I + tt) * SE + c] = f;
                f *= al[tt];
            }
            float e = 1.f;
#pragma unroll
            for (int tt = 0; tt < 16; ++tt) {
                e *= al[tt];
                sE[(16 * I + tt) * SE + c] = e;
            }
            sGB[I * D + c] = e;
            if (!(e >= kTiny)) atomicOr(&sFlag[I], 1);     // flags were cleared during the previous item
        }
        if (tid < C) sBeta[tid] = tid < Lc ? ld_scalar<TB>(&rbeta, 0) : 0.f;
        __syncthreads();
        // the next item's inputs, in flight while this one is computed
        const int next = min(item + (int)gridDim.x, items - 1);
        fetch(next, 0);
        if (tid < D) {
            const int c = tid;
            const float g0 = sGB[c], g1 = sGB[D + c], g2 = sGB[2 * D + c], g3 = sGB[3 * D + c];
            sG[c] = 1.f; sG[D + c] = g0; sG[2 * D + c] = g0 * g1; sG[3 * D + c] = g0 * g1 * g2;
            sGam[c] = g0 * g1 * g2 * g3;
        }

        // ================= L and Mqk on MFMA, the 10 16x16 blocks with I >= J
        // Left operands x_t E_t (x = k for L, q for Mqk), t in block I.
        // Diagonal blocks (wavefronts 0-3, I = J = wavefront): right operands k_s / E_s
        // (start of block as reference, bounded by 1 / Gamma_I; a block with Gamma_I
        // below FLT_MIN takes the exact path instead), multiplied in fp32 on
        // v_mfma_f32_16x16x4f32: near-diagonal entries dominate o, and fp32
        // operands need no hi/lo splitting on the vector ALU.
        // Off-diagonal blocks (wavefronts 4-7): right operands k_s F_s
        // prod_{J<K<I} Gamma_K; every factor is <= 1, so both operands are rounded
        // once to fp16 (11-bit significand) and multiplied on fp16 MFMA. A wave's
        // blocks share their row block, so its left operands are built once.
        //   wavefront 4: (3,0) (3,1)   5: (3,2)   6: (2,0) (2,1)   7: (1,0)
        // the four flags in one LDS read (a serial read per block cost a round trip each)
        const int4 flags = *reinterpret_cast<const int4 *>(sFlag);
        if (wave < 4) {
            const int I = wave;
            if (!(I == 0 ? flags.x : I == 1 ? flags.y : I == 2 ? flags.z : flags.w)) {
                const int t = 16 * I + l16;
                const float nq = NORM ? sRQ[t] : 1.f, nk = NORM ? sRK[t] : 1.f;
                f32x4 accL = {0.f, 0.f, 0.f, 0.f}, accM = accL;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    // lane: row / column t, channels 32ks + 8lq + e; product e contracts
                    // channels 32ks + 8j + e over the four k-slots j
                    const int c0 = 32 * ks + 8 * lq;
                    const bf16x8 qv = lds8(sQ + t * SQ + c0), kv = lds8(sK + t * SQ + c0);
                    const f32x4 e0 = *reinterpret_cast<const f32x4 *>(sE + t * SE + c0);
                    const f32x4 e1 = *reinterpret_cast<const f32x4 *>(sE + t * SE + c0 + 4);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float ee = e < 4 ? e0[e] : e1[e - 4];
                        const float kk = NORM ? bf2f(kv[e]) * nk : bf2f(kv[e]);
                        const float qq = NORM ? bf2f(qv[e]) * nq : bf2f(qv[e]);
                        const float bk = kk * __builtin_amdgcn_rcpf(ee);
                        accL = __builtin_amdgcn_mfma_f32_16x16x4f32(kk * ee, bk, accL, 0, 0, 0);
                        accM = __builtin_amdgcn_mfma_f32_16x16x4f32(qq * ee, bk, accM, 0, 0, 0);
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tr = 16 * I + 4 * lq + i, sc = 16 * I + l16;
                    const bool lower = sc < tr;
                    // masked entries may hold inf / nan: select, do not scale
                    if (lower) sLI[tr * SL + sc] = sBeta[tr] * accL[i];
                    sMqk[tr * SMQ + sc] = static_cast<_Float16>(lower ? accM[i] : 0.f);
                }
            }
            // Kr = k F H for the block's 16 tokens, written channel-major (Kr^T) so that
            // the record's Kr^T fragments are single 16-byte reads. This wave is
            // otherwise idle until the off-diagonal blocks are done. A lane takes a
            // token pair (16I + 2(lane & 7), +1) and eight-channel groups lane >> 3 and
            // (lane >> 3) + 8, and writes each (channel, token pair) as one dword.
            {
                const int t0 = 16 * I + 2 * (lane & 7);
                float nk0 = 1.f, nk1 = 1.f;
                if constexpr (NORM) { nk0 = sRK[t0]; nk1 = sRK[t0 + 1]; }
#pragma unroll
                for (int gg = 0; gg < 2; ++gg) {
                    const int c0 = 8 * ((lane >> 3) + 8 * gg);
                    // H (block I end -> chunk end) = product of the later block decays
                    f32x4 h0 = {1.f, 1.f, 1.f, 1.f}, h1 = h0;
#pragma unroll
                    for (int K = 1; K < 4; ++K)
                        if (K > I) {                                      // uniform
                            h0 *= *reinterpret_cast<const f32x4 *>(sGB + K * D + c0);
                            h1 *= *reinterpret_cast<const f32x4 *>(sGB + K * D + c0 + 4);
                        }
                    const bf16x8 ka = lds8(sK + t0 * SQ + c0), kb = lds8(sK + (t0 + 1) * SQ + c0);
                    const f32x4 fa0 = *reinterpret_cast<const f32x4 *>(sF + t0 * SE + c0);
                    const f32x4 fa1 = *reinterpret_cast<const f32x4 *>(sF + t0 * SE + c0 + 4);
                    const f32x4 fb0 = *reinterpret_cast<const f32x4 *>(sF + (t0 + 1) * SE + c0);
                    const f32x4 fb1 = *reinterpret_cast<const f32x4 *>(sF + (t0 + 1) * SE + c0 + 4);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float hh = e < 4 ? h0[e] : h1[e - 4];
                        const float xa = bf2f(ka[e]) * nk0 * (e < 4 ? fa0[e] : fa1[e - 4]) * hh;
                        const float xb = bf2f(kb[e]) * nk1 * (e < 4 ? fb0[e] : fb1[e - 4]) * hh;
                        typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
                        const f16x2 pr = {static_cast<_Float16>(xa), static_cast<_Float16>(xb)};
                        *reinterpret_cast<f16x2 *>(sKrt + (c0 + e) * SKR + t0) = pr;
                    }
                }
            }
            // exact diagonal d_t = q_t . k_t (4 lanes per row, 32 channels each)
            {
                const int row = tid >> 2, seg = tid & 3;
                float acc = 0.f;
#pragma unroll
                for (int hh = 0; hh < 4; ++hh) {
                    const bf16x8 qa = lds8(sQ + row * SQ + 32 * seg + 8 * hh), ka = lds8(sK + row * SQ + 32 * seg + 8 * hh);
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc += bf2f(qa[e]) * bf2f(ka[e]);
                }
                acc += __shfl_xor(acc, 1, 64);
                acc += __shfl_xor(acc, 2, 64);
                if constexpr (NORM) acc *= sRQ[row] * sRK[row];
                if (seg == 0) sDg[row] = acc;
            }
        } else {
            // the wavefront's blocks (I, J0) and, when NB = 2, (I, 1), with the block
            // indices known at compile time: the decay factors between the blocks and
            // the loop bounds then cost no selects, multiplications by one or branches
            auto offdiag = [&](auto Ic, auto J0c, auto NBc) {
                constexpr int I = decltype(Ic)::value, J0 = decltype(J0c)::value, NB = decltype(NBc)::value;
                f32x4 accL[NB], accM[NB];
#pragma unroll
                for (int bb = 0; bb < NB; ++bb) { accL[bb] = f32x4{0.f, 0.f, 0.f, 0.f}; accM[bb] = accL[bb]; }
                const int t = 16 * I + l16;
                const float nq = NORM ? sRQ[t] : 1.f, nk = NORM ? sRK[t] : 1.f;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const int c0 = 32 * ks + 8 * lq;
                    const bf16x8 qv = lds8(sQ + t * SQ + c0), kv = lds8(sK + t * SQ + c0);
                    const f32x4 a0 = *reinterpret_cast<const f32x4 *>(sE + t * SE + c0);
                    const f32x4 a1 = *reinterpret_cast<const f32x4 *>(sE + t * SE + c0 + 4);
                    f16x8 aq, ak;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float fa = e < 4 ? a0[e] : a1[e - 4];
                        aq[e] = static_cast<_Float16>(NORM ? bf2f(qv[e]) * nq * fa : bf2f(qv[e]) * fa);
                        ak[e] = static_cast<_Float16>(NORM ? bf2f(kv[e]) * nk * fa : bf2f(kv[e]) * fa);
                    }
#pragma unroll
                    for (int bb = 0; bb < NB; ++bb) {
                        const int J = bb ? 1 : J0, sr = 16 * J + l16;
                        const bf16x8 sv = lds8(sK + sr * SQ + c0);
                        f32x4 b0 = *reinterpret_cast<const f32x4 *>(sF + sr * SE + c0);
                        f32x4 b1 = *reinterpret_cast<const f32x4 *>(sF + sr * SE + c0 + 4);
                        // prod_{J<K<I} Gamma_K (none for adjacent blocks)
#pragma unroll
                        for (int K = J + 1; K < I; ++K) {
                            b0 *= *reinterpret_cast<const f32x4 *>(sGB + K * D + c0);
                            b1 *= *reinterpret_cast<const f32x4 *>(sGB + K * D + c0 + 4);
                        }
                        const float ns = NORM ? sRK[sr] : 1.f;
                        f16x8 bk;
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            bk[e] = static_cast<_Float16>((NORM ? bf2f(sv[e]) * ns : bf2f(sv[e])) * (e < 4 ? b0[e] : b1[e - 4]));
                        accL[bb] = mfma_f16(ak, bk, accL[bb]);
                        accM[bb] = mfma_f16(aq, bk, accM[bb]);
                    }
                }
#pragma unroll
                for (int bb = 0; bb < NB; ++bb) {
                    const int J = bb ? 1 : J0;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int tr = 16 * I + 4 * lq + i, sc = 16 * J + l16;
                        sLI[tr * SL + sc] = sBeta[tr] * accL[bb][i];
                        sMqk[tr * SMQ + sc] = static_cast<_Float16>(accM[bb][i]);
                    }
                }
            };
            //   wavefront 4: (3,0) (3,1)   5: (3,2)   6: (2,0) (2,1)   7: (1,0)
            if (wave == 4) offdiag(IC<3>{}, IC<0>{}, IC<2>{});
            else if (wave == 5) offdiag(IC<3>{}, IC<2>{}, IC<1>{});
            else if (wave == 6) offdiag(IC<2>{}, IC<0>{}, IC<2>{});
            else offdiag(IC<1>{}, IC<0>{}, IC<1>{});
        }
        // exact path for diagonal blocks whose in-block decay leaves the fp32 normal range
        for (int I = 0; I < 4 && (flags.x | flags.y | flags.z | flags.w); ++I) {
            if (!(I == 0 ? flags.x : I == 1 ? flags.y : I == 2 ? flags.z : flags.w)) continue;   // uniform
            if (wave == I) {
                for (int tr = 1; tr < 16; ++tr)
                    for (int sc = 0; sc < tr; ++sc) {
                        const int T_ = 16 * I + tr, S_ = 16 * I + sc;
                        float accl = 0.f, accm = 0.f;
                        for (int c = lane; c < D; c += 64) {
                            float lg = 0.f;
                            for (int rho = S_ + 1; rho <= T_; ++rho)
                                if (rho < Lc) lg += GateRow(p.g, GHEAD, (size_t)(tok0 + rho) * H + h, D).at(c);
                            const float w = expf(lg), kk = bf2f(sK[S_ * SQ + c]);
                            accl += bf2f(sK[T_ * SQ + c]) * kk * w;
                            accm += bf2f(sQ[T_ * SQ + c]) * kk * w;
                        }
                        accl = warp_sum(accl);
                        accm = warp_sum(accm);
                        if constexpr (NORM) {
                            accl *= sRK[T_] * sRK[S_];
                            accm *= sRQ[T_] * sRK[S_];
                        }
                        if (lane == 0) {
                            sLI[T_ * SL + S_] = sBeta[T_] * accl;
                            sMqk[T_ * SMQ + S_] = static_cast<_Float16>(accm);
                        }
                    }
                for (int e = lane; e < 256; e += 64)
                    if ((e & 15) >= (e >> 4)) sMqk[(16 * I + (e >> 4)) * SMQ + 16 * I + (e & 15)] = static_cast<_Float16>(0.f);
            }
        }
        __syncthreads();
        fetch(next, 1);
        // the flags were read above (into registers); clear them for the next item
        if (tid < 4) sFlag[tid] = 0;

        // ================= INV = (I + L)^{-1}, stored transposed in the upper triangle
        // diagonal 16x16 blocks: wave = block, lane < 16 = column of INV_II, by
        // column-oriented substitution: once x[sc] is final it is eliminated from
        // every later row at once, so the updates of a step are independent and the
        // L column reads (wave-uniform addresses) do not wait on the arithmetic.
        // Entries above the diagonal stay 0 (they only ever see x[sc] = 0).
        // Meanwhile waves 4-7, idle until the record, build their role's Kd and
        // Qd fragments (which do not depend on the inverse) and keep them in
        // registers until the record is stored. (Qd moved into the first
        // inverse level measured slower: that level then set the pace.)
        f16x8 fr[8];
        // x_t e^{a_t} (Kd from k, Qd from q) for the role's 16 tokens as four fp16
        // A fragments: the chunk-start decay is G (chunk start -> block start)
        // times E (block start -> t); rs: 1 / ||x_t|| (normalised input) or null
        auto build_decayed = [&](const __bf16 *sx, const float *rs, f16x8 *dst) {
            const int role = wave & 3, t = 16 * role + l16;
            const float nr = NORM ? rs[t] : 1.f;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int c0 = 32 * ks + 8 * lq;
                const bf16x8 xv = lds8(sx + t * SQ + c0);
                const f32x4 e0 = *reinterpret_cast<const f32x4 *>(sE + t * SE + c0);
                const f32x4 e1 = *reinterpret_cast<const f32x4 *>(sE + t * SE + c0 + 4);
                const f32x4 g0 = *reinterpret_cast<const f32x4 *>(sG + role * D + c0);
                const f32x4 g1 = *reinterpret_cast<const f32x4 *>(sG + role * D + c0 + 4);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float dec = e < 4 ? g0[e] * e0[e] : g1[e - 4] * e1[e - 4];
                    dst[ks][e] = static_cast<_Float16>((NORM ? bf2f(xv[e]) * nr : bf2f(xv[e])) * dec);
                }
            }
        };
        if (wave < 4 && lane < 16) {
            const int I = wave, col = lane;
            float x[16];
#pragma unroll
            for (int tr = 0; tr < 16; ++tr) x[tr] = (tr == col) ? 1.f : 0.f;
#pragma unroll
            for (int sc = 0; sc < 15; ++sc)
#pragma unroll
                for (int tr = sc + 1; tr < 16; ++tr) x[tr] -= sLI[(16 * I + tr) * SL + 16 * I + sc] * x[sc];
#pragma unroll
            for (int tr = 0; tr < 16; ++tr)
                if (tr >= col) sLI[(16 * I + col) * SL + 16 * I + tr] = x[tr];
        } else if (wave >= 4) {
            build_decayed(sK, NORM ? sRK : nullptr, fr);
            build_decayed(sQ, NORM ? sRQ : nullptr, fr + 4);
        }
        __syncthreads();
        fetch(next, 2);
        // off-diagonal blocks on fp32 MFMA (exact products), with the 64 x 64 inverse
        // taken as 2 x 2 blocks of 32 (A, D its diagonal halves, C = L[32:64][0:32]):
        //   stage 1:  INV_10 = -INV_11 L_10 INV_00,  INV_32 = -INV_33 L_32 INV_22
        //   stage 2a: P = C A^{-1}    (P_IJ = sum_{J<=K<=1} L_IK INV_KJ, I in {2,3}, J in {0,1})
        //   stage 2b: INV_IJ = -sum_{2<=K<=I} INV_IK P_KJ
        // Four dependent products on the critical path instead of six for three
        // levels of INV_IJ = -INV_II sum_K L_IK INV_KJ. Operands: a 16x16x4 fragment
        // gives lane (l16, lq) A[row = l16][k] and B[k][col = l16], k = 4 sl + lq.
        // INV_XY[a][b] lives at sLI[(16Y + b) * SL + 16X + a]; for X == Y only a >= b is stored.
        {
            const int row = l16, kk = lq;
            // INV_XY[r][c] (X >= Y, zero above the diagonal of a diagonal block)
            auto inv_at = [&](int X, int Y, int r, int c) {
                return (X == Y && c > r) ? 0.f : sLI[(16 * Y + c) * SL + 16 * X + r];
            };
            if (wave < 2) {                                     // stage 1
                const int J = 2 * wave, I = J + 1;
                f32x4 T4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int sl = 0; sl < 4; ++sl) {
                    const int k = 4 * sl + kk;
                    T4 = __builtin_amdgcn_mfma_f32_16x16x4f32(sLI[(16 * I + row) * SL + 16 * J + k],   // L_IJ[row][k]
                                                              inv_at(J, J, k, row), T4, 0, 0, 0);      // INV_JJ[k][col]
                }
                float *tw = sT3 + wave * 256;
#pragma unroll
                for (int i = 0; i < 4; ++i) tw[(4 * lq + i) * 16 + l16] = T4[i];
                __builtin_amdgcn_s_waitcnt(0xc07f);     // lgkmcnt(0): scratch written before it is read
                f32x4 O4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int sl = 0; sl < 4; ++sl) {
                    const int k = 4 * sl + kk;
                    O4 = __builtin_amdgcn_mfma_f32_16x16x4f32(inv_at(I, I, row, k), tw[k * 16 + l16], O4, 0, 0, 0);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) sLI[(16 * J + l16) * SL + 16 * I + 4 * lq + i] = -O4[i];
            }
            __syncthreads();
            // stage 2a: wave w < 4 takes P_IJ with I = 2 + (w >> 1), J = w & 1
            if (wave < 4) {
                const int I = 2 + (wave >> 1), J = wave & 1;
                f32x4 P4 = {0.f, 0.f, 0.f, 0.f};
                for (int K = J; K < 2; ++K) {
#pragma unroll
                    for (int sl = 0; sl < 4; ++sl) {
                        const int k = 4 * sl + kk;
                        P4 = __builtin_amdgcn_mfma_f32_16x16x4f32(sLI[(16 * I + row) * SL + 16 * K + k],  // L_IK[row][k]
                                                                  inv_at(K, J, k, row), P4, 0, 0, 0);     // INV_KJ[k][col]
                    }
                }
                float *pw = sT3 + wave * 256;                   // P_IJ, [row][col]
#pragma unroll
                for (int i = 0; i < 4; ++i) pw[(4 * lq + i) * 16 + l16] = P4[i];
            }
            __syncthreads();
            // stage 2b: wave w < 4 takes INV_IJ with I = 2 + (w >> 1), J = w & 1
            if (wave < 4) {
                const int I = 2 + (wave >> 1), J = wave & 1;
                f32x4 O4 = {0.f, 0.f, 0.f, 0.f};
                for (int K = 2; K <= I; ++K) {
                    const float *pk = sT3 + ((K - 2) * 2 + J) * 256;    // P_KJ
#pragma unroll
                    for (int sl = 0; sl < 4; ++sl) {
                        const int k = 4 * sl + kk;
                        O4 = __builtin_amdgcn_mfma_f32_16x16x4f32(inv_at(I, K, row, k), pk[k * 16 + l16], O4, 0, 0, 0);
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) sLI[(16 * J + l16) * SL + 16 * I + 4 * lq + i] = -O4[i];
            }
            __syncthreads();
        }

        // ================= record: fp16 fragments of the scan's left operands
        // Record role r = wave & 3 (tokens 16r..16r+15, channels 32r..32r+31).
        // Waves 4-7 built Kd and Qd above; waves 0-3 build Kr^T, IB and Mqk here.
        // Both store eight fragments from the same code after the branch: stores
        // inside role branches would leave the compiler a path without them, and
        // its wait for the next item's inputs would then also wait for the stores.
        {
            const int role = wave & 3;
            const int t = 16 * role + l16;
            if (wave < 4) {
                // Kr^T fragments (channel rows, tokens 32ks + 8lq .. +7), from the
                // channel-major tile written during the L / Mqk phase
#pragma unroll
                for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks)
                        fr[rt * 2 + ks] = lds8h(sKrt + (32 * role + 16 * rt + l16) * SKR + 32 * ks + 8 * lq);
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const f32x4 be0 = *reinterpret_cast<const f32x4 *>(sBeta + 32 * ks + 8 * lq);
                    const f32x4 be1 = *reinterpret_cast<const f32x4 *>(sBeta + 32 * ks + 8 * lq + 4);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int sc = 32 * ks + 8 * lq + e;
                        // INV[t][sc] is stored at (sc, t); zero for sc > t. The read is
                        // unconditional (in bounds), so no branch waits on each of them.
                        const float x = sLI[sc * SL + t] * (e < 4 ? be0[e] : be1[e - 4]);
                        fr[4 + ks][e] = static_cast<_Float16>(sc <= t ? x : 0.f);
                    }
                    // Mqk blocks above the diagonal block are never written: select zeros
                    // there (a select, so stale LDS contents cannot leak in)
                    const f16x8 mq = *reinterpret_cast<const f16x8 *>(sMqk + t * SMQ + 32 * ks + 8 * lq);
                    fr[6 + ks] = 2 * ks + (lq >> 1) > role ? f16x8{} : mq;
                }
            }
            // fragment i: waves 4-7 Kd (i < 4) and Qd, contiguous from KD; waves 0-3
            // Kr (i < 4), then IB and Mqk, contiguous from IB
            static_assert(Rec::QD == Rec::KD + 4096 && Rec::MQ == Rec::IB + 2048, "record layout");
            char *rec = p.rec + ((size_t)h * p.rec_stride + ci) * Rec::BYTES;
            char *rw = rec + (size_t)role * Rec::WAVE + lane * 16;
            const int o_lo = wave >= 4 ? Rec::KD : Rec::KR, o_hi = wave >= 4 ? Rec::KD : Rec::IB - 4096;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                *reinterpret_cast<f16x8 *>(rw + (i < 4 ? o_lo : o_hi) + i * 1024) = fr[i];
            // d (64 floats) then gamma (128 floats): one float per thread, every
            // thread issues the store and the range check drops those past the end
            static_assert(Rec::GAM == Rec::DG + C * 4, "record layout");
            const float tv = tid < C ? sDg[tid] : sGam[min(tid - C, D - 1) & (D - 1)];
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, tv),
                                                  buf_rsrc(rec + Rec::DG, (C + D) * 4), tid * 4, 0, 0);
        }
        __syncthreads();      // LDS is restaged by the next item
    };
    if (tid0 < 4) sFlag[tid0] = 0;
    __syncthreads();
    if ((int)blockIdx.x < items) {
        fetch(blockIdx.x, -1);
        body(blockIdx.x);
    }
    for (int item = blockIdx.x + gridDim.x; item < items; item += gridDim.x) body(item);
}

// ---------------------------------------------------------------- scan
constexpr int SMS = D + 8;       // fp16 row stride of the state       [col][136]
constexpr int SYU = C + 8;       // fp16 row stride of Y and U         [col][72]
constexpr int SVT = C + 8;       // bf16 row stride of the V tile      [col][72]

template <int TV>
struct ScanLds {
    static constexpr int M = 0;                      // fp16 [2][TV][SMS] state hi / lo, [col][channel]
    static constexpr int Y = M + 2 * TV * SMS * 2;   // fp16 [2][TV][SYU] (V - Kd M) hi / lo, [col][token]
    static constexpr int U = Y + 2 * TV * SYU * 2;   // fp16 [2][TV][SYU] U hi / lo, [col][token]
    static constexpr int V = U + 2 * TV * SYU * 2;   // bf16 [2][TV][SVT] V of a chunk, [col][token], double-buffered
    static constexpr int DG = V + 2 * TV * SVT * 2;  // fp32 [2][C + D] d then gamma of a chunk, double-buffered
    static constexpr int SIZE = DG + 2 * (C + D) * 4;
};

struct ScanParams {
    const bf16_t *v;
    const float *S0;
    void *out;
    float *S_out;
    SeqView sv;
    int H, chains;
    const char *rec;
    long long rec_stride;        // records per head
    SnapView snap;
};

template <typename T> __device__ __forceinline__ void buf_st4(__amdgpu_buffer_rsrc_t r, int voff, f32x4 x);
template <> __device__ __forceinline__ void buf_st4<float>(__amdgpu_buffer_rsrc_t r, int voff, f32x4 x) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r, voff, 0, 0);
}
template <> __device__ __forceinline__ void buf_st4<bf16_t>(__amdgpu_buffer_rsrc_t r, int voff, f32x4 x) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const uint32_t lo = __builtin_bit_cast(uint16_t, static_cast<__bf16>(x[0])) |
                        (uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(x[1]))) << 16);
    const uint32_t hi = __builtin_bit_cast(uint16_t, static_cast<__bf16>(x[2])) |
                        (uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(x[3]))) << 16);
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{lo, hi}, r, voff, 0, 0);
}

template <int TV, typename TO>
__global__ __launch_bounds__(SCAN_THR, KDA_SCAN_MIN_WAVES) void chunk_scan_kernel(ScanParams p) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    using Lo = ScanLds<TV>;
    constexpr int NT = TV / 16;
    constexpr int TEAM = D / TV;
    static_assert(TV == 16 || TV == 32, "value columns per workgroup");
    constexpr int XP = NT;               // 16-byte pieces of V, d and gamma per lane and chunk
    _Float16 *sMh = reinterpret_cast<_Float16 *>(smem + Lo::M);
    _Float16 *sMl = sMh + TV * SMS;
    _Float16 *sYh = reinterpret_cast<_Float16 *>(smem + Lo::Y);
    _Float16 *sYl = sYh + TV * SYU;
    _Float16 *sUh = reinterpret_cast<_Float16 *>(smem + Lo::U);
    _Float16 *sUl = sUh + TV * SYU;
    bf16_t *sV = reinterpret_cast<bf16_t *>(smem + Lo::V);
    float *sDG = reinterpret_cast<float *>(smem + Lo::DG);

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, lq = lane >> 4;
    // XCD-aware placement: block b runs on XCD b % 8; the TEAM workgroups of
    // one chain share b % 8 and so one L2, where the chain's records are read.
    const int b = blockIdx.x;
    const int xcd = b & 7, r = b >> 3;
    const int member = r % TEAM, grp = r / TEAM;
    const int chain = grp * 8 + xcd;
    if (chain >= p.chains) return;
    const int H = p.H, n = chain / H, h = chain % H;
    const int col0 = member * TV;
    const int start = p.sv.seq_start(n), end = p.sv.seq_end(n);
    const int nch = (end - start + C - 1) / C, c0 = p.sv.first_chunk(n);
    const size_t st_off = ((size_t)n * H + h) * D * D;
    const int tb = 16 * (wave & 3);
    // bytes from a chunk's first row to the end of its last valid row
    auto chunk_bytes = [&](int Lc, int elem) { return ((Lc - 1) * H * D + D) * elem; };

    if (wave >= 4) {
        // Output wavefronts: o = Qd M + Mqk U + d U for token tile tb, from the
        // state and U that the recurrence wavefronts put in LDS, so that the
        // recurrence's own steps carry only what the next chunk depends on. Their
        // operands (Qd, Mqk) are loaded two chunks ahead, like the recurrence's;
        // they pass the same barriers (one before the first chunk, three per
        // chunk).
        struct OFrags {
            f16x8 qd[4], mq[2];
            // 16-byte pieces of the chunk's V tile and of its d and gamma (adjacent
            // in the record, 192 floats), staged through LDS one chunk ahead for
            // the whole workgroup (stid: thread index in this group). TV = 16: one
            // piece, wavefronts 4-5 V (token stid >> 1, columns 8 (stid & 1) ..
            // +7), 6-7 d and gamma (floats 4 (stid - 128) .. +3; lanes past them
            // repeat the last piece). TV = 32: piece 0 V (token stid >> 2, columns
            // 8 (stid & 3) .. +7), piece 1 d and gamma (floats 4 stid .. +3,
            // repeated past them).
            u32x4 x[XP];
        };
        const int stid = tid - NTHR;
        const bool x_is_v = TV == 32 || wave < 6;                  // uniform (piece 0)
        static_assert(Rec::GAM == Rec::DG + C * 4, "d and gamma adjacent in the record");
        constexpr int VL = TV / 8;                                 // lanes per V row
        int x_off[XP];
        x_off[0] = x_is_v ? ((stid / VL) * H * D + col0 + 8 * (stid % VL)) * 2
                          : Rec::DG + 16 * min(stid - 128, (C + D) / 4 - 1);
        if constexpr (XP == 2) x_off[XP - 1] = Rec::DG + 16 * min(stid, (C + D) / 4 - 1);
        // the V / gamma piece of chunk j into LDS buffer j & 1 (read during step j)
        auto stage = [&](const OFrags &f, int j) {
            const int bsel = j & 1;
            if (x_is_v) {
                // transposed into [col][token]: one column of eight per 16-bit store
                bf16_t *dst = sV + bsel * TV * SVT + (8 * (stid % VL)) * SVT + (stid / VL);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    dst[e * SVT] = static_cast<bf16_t>(e & 1 ? f.x[0][e >> 1] >> 16 : f.x[0][e >> 1] & 0xffffu);
            }
            const int dl = XP == 2 ? stid : stid - 128;            // lane's d / gamma piece
            if ((XP == 2 || !x_is_v) && dl < (C + D) / 4)
                *reinterpret_cast<u32x4 *>(sDG + bsel * (C + D) + 4 * dl) = f.x[XP - 1];
        };
        const int r_frag = (wave & 3) * Rec::WAVE + lane * 16;
        // this lane's output: token tb + l16, columns col0 + 4lq .. +3 (O is formed transposed)
        const int o_off = ((tb + l16) * H * D + col0 + 4 * lq) * (int)sizeof(TO);
        auto oissue = [&](int j, OFrags &f) {
            const auto rr = buf_rsrc(p.rec + ((size_t)h * p.rec_stride + c0 + j) * Rec::BYTES, Rec::BYTES);
            const int tok0 = start + j * C, Lc = min(C, end - tok0);
            // V rows past the end of the sequence read 0 (outside the range): their
            // values never matter, because beta = 0 there makes the matching columns
            // of IB zero
            const auto rv = buf_rsrc(p.v + ((size_t)tok0 * H + h) * D, chunk_bytes(Lc, 2));
#pragma unroll
            for (int pc = 0; pc < XP; ++pc) f.x[pc] = buf_ld16<u32x4>(pc == 0 && x_is_v ? rv : rr, x_off[pc], 0);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) f.qd[ks] = buf_ld16<f16x8>(rr, r_frag, Rec::QD + ks * 1024);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) f.mq[ks] = buf_ld16<f16x8>(rr, r_frag, Rec::MQ + ks * 1024);
        };
        auto ostep = [&](const OFrags &f, int j, const OFrags &f1, OFrags &nf, int nj) {
            oissue(nj, nf);
            stage(f1, j + 1);    // read by the recurrence in the next step
            const int tok0 = start + j * C, Lc = min(C, end - tok0);
            const auto ro = buf_rsrc(static_cast<TO *>(p.out) + ((size_t)tok0 * H + h) * D, chunk_bytes(Lc, sizeof(TO)));
            const int bsel = j & 1;
            __syncthreads();     // Y = V - Kd M is in LDS
            // O^T = M^T Qd^T from the state at the chunk start (published before the
            // barrier that ended the previous step, replaced only after the next
            // one), while the recurrence forms U
            f32x4 accO[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                accO[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const f16x8 bh = lds8h(sMh + (16 * nt + l16) * SMS + 32 * ks + 8 * lq);
                    accO[nt] = mfma_f16(bh, f.qd[ks], accO[nt]);
                    if constexpr (KDA_SPLIT_OI || TV == 16) {
                        const f16x8 bl = lds8h(sMl + (16 * nt + l16) * SMS + 32 * ks + 8 * lq);
                        accO[nt] = mfma_f16(bl, f.qd[ks], accO[nt]);
                    }
                }
            }
            __syncthreads();     // U is in LDS
            const float dt = sDG[bsel * (C + D) + tb + l16];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    // O^T += U^T Mqk^T (Mqk strictly lower)
                    const f16x8 bh = lds8h(sUh + (16 * nt + l16) * SYU + 32 * ks + 8 * lq);
                    accO[nt] = mfma_f16(bh, f.mq[ks], accO[nt]);
                    if constexpr (KDA_SPLIT_UO || TV == 16) {
                        const f16x8 bl = lds8h(sUl + (16 * nt + l16) * SYU + 32 * ks + 8 * lq);
                        accO[nt] = mfma_f16(bl, f.mq[ks], accO[nt]);
                    }
                }
                // + d_t U_t in fp32 for token tb + l16, columns 4lq .. +3, with U as its
                // hi + lo parts (U to 2^-22 relative); one vector store (rows past
                // the end are dropped)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int at = (16 * nt + 4 * lq + i) * SYU + tb + l16;
                    accO[nt][i] += dt * (static_cast<float>(sUh[at]) + static_cast<float>(sUl[at]));
                }
                buf_st4<TO>(ro, o_off + 16 * nt * (int)sizeof(TO), accO[nt]);
            }
            __syncthreads();     // the next state is in LDS
        };
        if (nch > 0) {
            const int last = nch - 1;
            OFrags A, B, Cb;
            oissue(0, A);
            oissue(min(1, last), B);
            stage(A, 0);
            __syncthreads();     // the initial state and chunk 0's V / gamma are in LDS
            for (int j = 0; j < nch; j += 3) {
                ostep(A, j, B, Cb, min(j + 2, last));
                if (j + 1 >= nch) break;
                ostep(B, j + 1, Cb, A, min(j + 3, last));
                if (j + 2 >= nch) break;
                ostep(Cb, j + 2, A, B, min(j + 4, last));
            }
        }
        return;
    }

    // state tile: wave w owns channels 32w..32w+31 (two 16-row tiles)
    f32x4 Macc[2][NT];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int chn = 32 * wave + 16 * rt + 4 * lq + i, col = col0 + 16 * nt + l16;
                Macc[rt][nt][i] = p.S0 ? p.S0[st_off + (size_t)chn * D + col] : 0.f;
            }
    auto publish_state = [&]() {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                f16x4 hi, lo;
#pragma unroll
                for (int i = 0; i < 4; ++i) SPLITH(Macc[rt][nt][i], hi[i], lo[i]);
                const int col = 16 * nt + l16, chn = 32 * wave + 16 * rt + 4 * lq;
                *reinterpret_cast<f16x4 *>(sMh + col * SMS + chn) = hi;
                *reinterpret_cast<f16x4 *>(sMl + col * SMS + chn) = lo;
            }
    };
    publish_state();

    // operands of one chunk, loaded two chunks ahead
    struct Frags {
        f16x8 kd[4], ib[2], kr[2][2];
    };
    // loop-invariant byte offsets of this lane's record fragments
    const int r_frag = wave * Rec::WAVE + lane * 16;

    // The loads of one chunk's operands, as NLD slots in the order they are
    // consumed: Kd by k-step, IB, Kr. issue() sends slots [s0, s1); the step
    // spreads them over its phases, so that no wave stalls on a full
    // vector-memory queue with work of its own waiting.
    constexpr int NLD = 10;
    auto issue = [&](int j, Frags &f, int s0, int s1) {
        const auto rr = buf_rsrc(p.rec + ((size_t)h * p.rec_stride + c0 + j) * Rec::BYTES, Rec::BYTES);
#pragma unroll
        for (int sl = 0; sl < NLD; ++sl) {
            if (sl < s0 || sl >= s1) continue;
            if (sl < 4) {
                f.kd[sl] = buf_ld16<f16x8>(rr, r_frag, Rec::KD + sl * 1024);
            } else if (sl < 6) {
                f.ib[sl - 4] = buf_ld16<f16x8>(rr, r_frag, Rec::IB + (sl - 4) * 1024);
            } else {
                const int e = sl - 6;
                f.kr[e >> 1][e & 1] = buf_ld16<f16x8>(rr, r_frag, Rec::KR + e * 1024);
            }
            // keep the slot order: the in-order vmcnt then lets each use wait
            // for its own load only
            __builtin_amdgcn_sched_barrier(0x048F);
        }
    };
    // where a step issues the next operands: Kd before its first product (START),
    // IB after the first k-step of U (U0), Kr after the first k-step of the state
    // update (M0)
    enum { START, U0, M0 };
    auto issue_at = [&](int nj, Frags &nf, int point) {
        const int a = point == START ? 0 : point == U0 ? 4 : 6;
        const int b = point == START ? 4 : point == U0 ? 6 : NLD;
        issue(nj, nf, a, b);
        // the loads stay where they are issued; compute and LDS traffic may cross
        __builtin_amdgcn_sched_barrier(0x048F);
    };
    // Three operand buffers, used round-robin without copies: the loads for a chunk
    // are issued two chunks before it is consumed (its V tile, d and gamma are put
    // in LDS by the output wavefronts during the step before).
    auto step = [&](const Frags &f, int j, const Frags &f1, Frags &nf, int nj) {
        issue_at(nj, nf, START);
        const int bsel = j & 1;

        // X = Kd M for tokens tb..tb+15 (state split hi + lo)
        f32x4 accX[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            accX[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const f16x8 bh = lds8h(sMh + (16 * nt + l16) * SMS + 32 * ks + 8 * lq);
                accX[nt] = mfma_f16(f.kd[ks], bh, accX[nt]);
#if KDA_SPLIT_X
                const f16x8 bl = lds8h(sMl + (16 * nt + l16) * SMS + 32 * ks + 8 * lq);
                accX[nt] = mfma_f16(f.kd[ks], bl, accX[nt]);
#endif
            }
            // V of tokens tb + 4lq .. +3 at this lane's column
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            const u32x2 vv = *reinterpret_cast<const u32x2 *>(sV + bsel * TV * SVT + (16 * nt + l16) * SVT + tb + 4 * lq);
            f16x4 hi, lo;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t w = vv[i >> 1];
                const float v = __uint_as_float(i & 1 ? w & 0xffff0000u : w << 16);
                SPLITH(v - accX[nt][i], hi[i], lo[i]);
            }
            const int col = 16 * nt + l16, t = tb + 4 * lq;
            *reinterpret_cast<f16x4 *>(sYh + col * SYU + t) = hi;
            *reinterpret_cast<f16x4 *>(sYl + col * SYU + t) = lo;
        }
        __syncthreads();
        // U = IB Y (Y split hi + lo)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            f32x4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const f16x8 bh = lds8h(sYh + (16 * nt + l16) * SYU + 32 * ks + 8 * lq);
                const f16x8 bl = lds8h(sYl + (16 * nt + l16) * SYU + 32 * ks + 8 * lq);
                u = mfma_f16(f.ib[ks], bh, u);
#if KDA_SPLIT_Y
                u = mfma_f16(f.ib[ks], bl, u);
#endif
                if (nt == 0 && ks == 0) issue_at(nj, nf, U0);
            }
            f16x4 hi, lo;
#pragma unroll
            for (int i = 0; i < 4; ++i) SPLITH(u[i], hi[i], lo[i]);
            const int col = 16 * nt + l16, t = tb + 4 * lq;
            *reinterpret_cast<f16x4 *>(sUh + col * SYU + t) = hi;
            *reinterpret_cast<f16x4 *>(sUl + col * SYU + t) = lo;
        }
        __syncthreads();
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            // M = Diag(gamma) M + Kr^T U for channels 32w..32w+31
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const f32x4 gm = *reinterpret_cast<const f32x4 *>(sDG + bsel * (C + D) + C + 32 * wave + 16 * rt + 4 * lq);
#pragma unroll
                for (int i = 0; i < 4; ++i) Macc[rt][nt][i] *= gm[i];
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const f16x8 bh = lds8h(sUh + (16 * nt + l16) * SYU + 32 * ks + 8 * lq);
                const f16x8 bl = lds8h(sUl + (16 * nt + l16) * SYU + 32 * ks + 8 * lq);
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    Macc[rt][nt] = mfma_f16(f.kr[rt][ks], bh, Macc[rt][nt]);
#if KDA_SPLIT_U
                    Macc[rt][nt] = mfma_f16(f.kr[rt][ks], bl, Macc[rt][nt]);
#endif
                }
                if (nt == 0 && ks == 0) issue_at(nj, nf, M0);
            }
        }
        if (float *sp = p.snap.slot(n, h, H, j + 1, end - start, C, D * D)) {   // uniform across the workgroup
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int chn = 32 * wave + 16 * rt + 4 * lq + i, col = col0 + 16 * nt + l16;
                        sp[(size_t)chn * D + col] = Macc[rt][nt][i];
                    }
        }
        publish_state();
        __syncthreads();
    };
    // The prefetches are unconditional (the chunk index is clamped, so the tail
    // re-reads the last record): conditional loads would make every later wait
    // on vector memory conservative and defeat the prefetch.
#if KDA_SCAN_BUFS == 3
    Frags A, B, Cb;
    if (nch > 0) {
        const int last = nch - 1;
        issue(0, A, 0, NLD);
        issue(min(1, last), B, 0, NLD);
        __syncthreads();
        for (int j = 0; j < nch; j += 3) {
            step(A, j, B, Cb, min(j + 2, last));
            if (j + 1 >= nch) break;
            step(B, j + 1, Cb, A, min(j + 3, last));
            if (j + 2 >= nch) break;
            step(Cb, j + 2, A, B, min(j + 4, last));
        }
    }
#else
    // two operand buffers: a chunk's loads are issued during the step before it
#error "the V / gamma staging needs the next chunk's operands during a step: KDA_SCAN_BUFS must be 3"
#endif

    if (p.S_out) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int chn = 32 * wave + 16 * rt + 4 * lq + i, col = col0 + 16 * nt + l16;
                    p.S_out[st_off + (size_t)chn * D + col] = Macc[rt][nt][i];
                }
    }
}

// ---------------------------------------------------------------- host
// Compute units of the device the launch goes to (the caller's current
// device). Queried on every call: the library keeps no per-process cache, so
// concurrent first calls and several devices need no synchronisation.
hipError_t device_cus(int *cus) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess && *cus < 1) e = hipErrorInvalidDevice;
    return e;
}

// workspace: chunk offsets (N + 1 int32), the chunk table (maxc int2), records
size_t ws_offs(int N) { return ((sizeof(int32_t) * (size_t)(N + 1) + 255) / 256) * 256; }
size_t ws_meta(long long maxc) { return ((sizeof(int2) * (size_t)maxc + 255) / 256) * 256; }

template <typename TB, typename TO>
hipError_t run(const PrefillArgs &a) {
    const long long maxc = max_chunks(a.N, (long long)a.B * a.T, C);
    char *ws = static_cast<char *>(a.ws);
    int32_t *chunk_off = reinterpret_cast<int32_t *>(ws);
    int2 *meta = reinterpret_cast<int2 *>(ws + ws_offs(a.N));
    char *recs = ws + ws_offs(a.N) + ws_meta(maxc);
    SeqView sv{a.cu_seqlens, chunk_off, a.N, a.T, C};
    const bool varlen = a.cu_seqlens != nullptr;
    int cus = 0;
    if (const hipError_t e = device_cus(&cus); e != hipSuccess) return e;
    if (varlen) {
        hipError_t e = launch_chunk_plan(a.cu_seqlens, a.N, C, chunk_off, a.stream);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(chunk_meta_kernel, dim3((unsigned)((maxc + 255) / 256)), dim3(256), 0, a.stream,
                           sv, meta, (int)maxc);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    {
        // kernel variant [varlen][per-head gate][L2-normalised q, k]
        using Kern = void (*)(PrepParams);
        const Kern kerns[2][2][2] = {
            {{chunk_prep_kernel<TB, false, false, false>, chunk_prep_kernel<TB, false, false, true>},
             {chunk_prep_kernel<TB, false, true, false>, chunk_prep_kernel<TB, false, true, true>}},
            {{chunk_prep_kernel<TB, true, false, false>, chunk_prep_kernel<TB, true, false, true>},
             {chunk_prep_kernel<TB, true, true, false>, chunk_prep_kernel<TB, true, true, true>}}};
        const Kern kern = kerns[varlen][a.g_head][a.qk_norm];
        // set on every call (idempotent; no process-wide "already set" flag to race on)
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, PrepLds::SIZE);
        if (e != hipSuccess) return e;
        PrepParams pp{static_cast<const bf16_t *>(a.q), static_cast<const bf16_t *>(a.k), a.g, a.beta, sv, meta,
                      a.H, recs, maxc, a.norm_eps};
        // persistent: one workgroup per CU walks the (chunk, head) items
        const long long items = maxc * a.H;
        const unsigned grid = (unsigned)std::min<long long>(items, cus);
        if (items > 0) {
            hipLaunchKernelGGL(kern, dim3(grid), dim3(PTHR), PrepLds::SIZE, a.stream, pp);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    {
        // 16 value columns per workgroup, or 32 when the 16-column workgroups would
        // fill the CUs four times over or more (many chains, e.g. packed batches):
        // a CU then reads each record once per 32 columns instead of per 16
        const int chains = a.N * a.H;
        const bool wide = (long long)chains * (D / 16) >= 4LL * cus;
        const int team = wide ? D / 32 : D / 16;
        const unsigned blocks = (unsigned)((chains + 7) / 8) * 8u * (unsigned)team;
        ScanParams sp{static_cast<const bf16_t *>(a.v), a.S0, a.out, a.S_out, sv, a.H, chains, recs, maxc,
                      SnapView{a.snaps, a.snap_every, a.max_snaps}};
        if (wide)
            hipLaunchKernelGGL((chunk_scan_kernel<32, TO>), dim3(blocks), dim3(SCAN_THR), ScanLds<32>::SIZE, a.stream, sp);
        else
            hipLaunchKernelGGL((chunk_scan_kernel<16, TO>), dim3(blocks), dim3(SCAN_THR), ScanLds<16>::SIZE, a.stream, sp);
        return hipGetLastError();
    }
}

template <typename TB>
hipError_t run_o(const PrefillArgs &a) {
    return a.out_dt == Dt::F32 ? run<TB, float>(a) : run<TB, bf16_t>(a);
}

}  // namespace

size_t prefill_mfma_workspace(int N, long long T_total, int H, int Dk, int Dv, int C_) {
    if (Dk == D && Dv == D && C_ == C)
        return ws_offs(N) + ws_meta(max_chunks(N, T_total, C)) + (size_t)max_chunks(N, T_total, C) * H * Rec::BYTES;
    return prefill_f32_workspace(N, T_total, H, Dk, Dv, C_);
}

hipError_t launch_prefill_mfma(const PrefillArgs &a) {
    // The MFMA kernels cover Dk = Dv = 128 with C = 64; other supported
    // shapes run the fp32-arithmetic kernels on the same bf16 inputs.
    if (a.Dk == D && a.C == C) return a.beta_dt == Dt::F32 ? run_o<float>(a) : run_o<bf16_t>(a);
    return launch_prefill_f32(a);
}

}  // namespace kda
