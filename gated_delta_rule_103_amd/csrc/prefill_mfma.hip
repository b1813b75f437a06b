// prefill_mfma.hip -- chunked KDA prefill on MFMA (gfx950): a prep kernel
// and a scan kernel.
//
// Method: the chunk unrolling of the Kimi K3 explainer's FlashKDA paragraph
// (Q_decay, K_restore, causal M_qk, UT transform for the pseudo-values U).
// With a = in-chunk cumulative log-decay, gamma = exp(a_last):
//     Kd = k * exp(a),  Qd = q * exp(a),  Kr = k * exp(a_last - a)
//     Mqk[t,s] = sum_c q_t k_s exp(a_t - a_s)   (s <= t)
//     L[t,s]   = beta_t sum_c k_t k_s exp(a_t - a_s)   (s < t)
//     IB       = (I + L)^{-1} Diag(beta),   W = IB Kd,   U~ = IB V
// and per chunk of one (sequence, head), with M = S^T (S [Dv][Dk] is the state
// as it is stored; the kernels work on its transpose):
//     U     = U~ - W M
//     O     = Qd M + Mqk U
//     M_out = Diag(gamma) M + Kr^T U
//
// prep  (persistent, one workgroup of twelve wavefronts per CU walking the
//       (chunk, head) items, all chunks in parallel; eight take an item's main
//       work, four help with Mqk's diagonal blocks, Kr^T and the Qd / Mqk
//       record fragments): decays as products of alpha = exp(g) inside
//       16-token blocks; L and Mqk with the diagonal 16x16 blocks on fp32
//       MFMA and the off-diagonal ones on fp16 MFMA (every factor <= 1 there);
//       the unit-lower-triangular inverse by substitution on the diagonal
//       blocks and fp32 MFMA products off it; W = IB Kd on fp16 MFMA; and a
//       record of the scan's operands in fp16, laid out as MFMA fragments in
//       the register order of the scan's accumulators.
// scan  (one workgroup of eight wavefronts per (sequence, head, 16- or
//       32-column value tile), its chunks in order): four recurrence
//       wavefronts keep 32 rows of the fp32 state each in registers and form
//       U = U~ - W M, the state update and the next chunk's U~; four output
//       wavefronts form o = Qd M + Mqk U + d U for 16 tokens each. The state
//       and U meet in LDS at two barriers per chunk. Contractions on fp16 MFMA
//       with the state and U split into fp16 hi + lo, fp32 accumulation; V and
//       S0 scaled by a power of two from their running maximum.
// One long sequence runs as a pipeline over windows of chunks: the prep of the
// next window (second stream, the CUs the scan leaves free) beside the scan of
// the current one, with the records of two windows in the workspace.
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
constexpr float kTiny = 1.17549435e-38f;  // FLT_MIN

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

// four consecutive outputs with one store (16 bytes fp32, 8 bytes bf16)
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

template <typename T> __device__ __forceinline__ float ld_scalar(const T *p, size_t i);
template <> __device__ __forceinline__ float ld_scalar<float>(const float *p, size_t i) { return p[i]; }
template <> __device__ __forceinline__ float ld_scalar<bf16_t>(const bf16_t *p, size_t i) {
    return bf16_to_f32(p[i]);
}

// x = hi + lo, hi = fp16(x), lo = fp16(x - hi): about 22 significant bits for
// |x| in [2^-2, 2^15] (below, lo loses bits to fp16's subnormal range)
#define SPLITH(x, HI, LO)                                   \
    do {                                                    \
        const float x_ = (x);                               \
        const _Float16 h_ = static_cast<_Float16>(x_);      \
        (HI) = h_;                                          \
        (LO) = static_cast<_Float16>(x_ - static_cast<float>(h_)); \
    } while (0)

// ---------------------------------------------------------------- record
// Per (chunk, head): for each scan wavefront w (state channels 32w..32w+31,
// tokens 16w..16w+15) 16 KB of fp16 MFMA fragments [operand][lane][8]:
//   NW  (-W) for token tile tt = 0..3, k = w's channels    (W = IB Kd)
//   QD  Qd for token tile tt = 0..3, k = w's channels
//   KR  Kr^T for channel tile rt of w and token k-step ks   (index 2 rt + ks)
//   IB  IB for w's tokens, token k-step ks (natural token order)
//   MQ  strictly lower Mqk for w's tokens, token k-step ks
// then d_t = q_t . k_t (fp32 [64]) and gamma (fp32 [128]). A "channel" k-step
// gives lane (l16, lq) the channels 32w + 4lq + {0..3} and 32w + 16 + 4lq +
// {0..3}, a "token" k-step ks of KR and MQ the tokens 32ks + 4lq + {0..3} and
// 32ks + 16 + 4lq + {0..3}: exactly what that lane holds of two 16-row tiles
// of the state (or of U) in MFMA output layout, so the scan feeds its own
// accumulators to the next product without moving them. Records are stored
// head-major (index head * records-per-head + chunk), so the records a scan
// chain walks through are contiguous in memory.
struct Rec {
    static constexpr int WAVE = 16384;
    static constexpr int NW = 0, QD = 4096, KR = 8192, IB = 12288, MQ = 14336;
    static constexpr int DG = 4 * WAVE, GAM = DG + C * 4, BYTES = GAM + D * 4;
};

// ---------------------------------------------------------------- prep
template <int N> struct IC { static constexpr int value = N; };    // an int as a type (compile-time argument)
constexpr int PTHR = 768;        // prep: 12 wavefronts, three per SIMD to hide latency:
constexpr int PWORK = 512;       // wavefronts 0-7 take an item's main work, 8-11 help (below)
constexpr int SQ = D + 8;        // bf16 row stride of q, k           [64][136]
constexpr int SL = C + 4;        // fp32 row stride of L / INV^T      [64][68]
constexpr int SMQ = C + 8;       // fp16 row stride of Mqk            [64][72]
// The decayed tiles (fp32 [64][128]) and Kr^T / Kd^T (fp16 [128][64]) are not
// padded; their 16-byte blocks are XOR-ed with a function of the row instead,
// chosen by measuring the bank-conflict counter of every access pattern of the
// kernel on gfx950 (operand reads of 16 rows at one block, the channel-major
// writes of the transposes): all of them are then conflict-free but the
// transposes' row-pair reads (half as many conflict cycles as before).
__device__ __forceinline__ int e_at(int t, int c) { return t * D + (c ^ ((t & 15) << 2)); }
__device__ __forceinline__ int kt_at(int ch, int t) {
    return ch * C + (t ^ ((((ch & 7) ^ (5 * (ch >> 3))) & 7) << 3));
}

// The decayed operand tiles, formed once per item (fp32 [64][128], the L2 norm
// of q and k applied when requested): KE = k E and QE = q E (E: the in-block
// prefix decay, block start -> token), KF = k F (F: the in-block suffix decay,
// token -> block end). Every operand of the products is one of them times at
// most one per-channel factor.
struct PrepLds {
    static constexpr int KE = 0;
    static constexpr int QE = KE + C * D * 4;
    static constexpr int KF = QE + C * D * 4;
    static constexpr int LI = KF + C * D * 4;        // fp32 L (strictly lower) and INV^T (upper, with diagonal)
    static constexpr int MQK = LI + C * SL * 4;      // fp16 strictly lower Mqk
    static constexpr int DG = MQK + C * SMQ * 2;     // fp32 [64]
    static constexpr int BETA = DG + C * 4;          // fp32 [64]
    static constexpr int GB = BETA + C * 4;          // fp32 [4][128] block decays Gamma
    static constexpr int IGB = GB + 4 * D * 4;       // fp32 [4][128] 1 / Gamma (used where Gamma >= FLT_MIN)
    static constexpr int G = IGB + 4 * D * 4;        // fp32 [4][128] decay chunk start -> block start
    static constexpr int GAM = G + 4 * D * 4;        // fp32 [128]
    static constexpr int RQ = GAM + D * 4;           // fp32 [64] 1 / ||q_t|| (L2-normalised input)
    static constexpr int RK = RQ + C * 4;            // fp32 [64] 1 / ||k_t||
    static constexpr int FLAG = RK + C * 4;          // int [4]
    static constexpr int KRT = (FLAG + 16 + 255) / 256 * 256;   // fp16 [128][64] Kr^T, channel-major
    static constexpr int SIZE = KRT + (D * C > C * SQ ? D * C : C * SQ) * 2;
    // the bf16 rows of q and k are staged in the L and Kr^T tiles, free until the
    // decayed tiles have been formed
    static constexpr int QS = LI, KS = KRT;
};
static_assert(C * SQ * 2 <= C * SL * 4, "q staging");

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
    int cw0, cwn;                // window: global chunks cw0 .. cw0 + cwn - 1; record index chunk - cw0
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

// Packed sequences (N <= ORDER_MAX): order[rank] = n, ranked by decreasing chunk
// count, ties by index (a strict total order, so order is a permutation). The
// scan maps its chains through it: its workgroups are dispatched in block order,
// so the longest chains start first and the short ones fill in behind them
// (longest-processing-time-first list scheduling) instead of the last long
// sequences starting when the CUs are nearly drained.
constexpr int ORDER_MAX = 1024;
__global__ __launch_bounds__(ORDER_MAX) void chain_order_kernel(SeqView sv, int32_t *order) {
    __shared__ int s_nc[ORDER_MAX];
    const int N = sv.N, n = threadIdx.x;
    if (n < N) s_nc[n] = sv.first_chunk(n + 1) - sv.first_chunk(n);
    __syncthreads();
    if (n >= N) return;
    const int c = s_nc[n];
    int rank = 0;
    for (int m = 0; m < N; ++m) {
        const int d = s_nc[m];
        rank += (d > c) || (d == c && m < n);
    }
    order[rank] = n;
}

// GHEAD: one log-decay per (token, head), g [T][H] or none (nullptr), instead
// of one per key channel. NORM: q and k are L2-normalised over the channels on
// the fly: 1/||q_t||, 1/||k_t|| (fp32, from the staged bf16 rows) scale the
// decayed tiles as they are formed.
template <typename TB, bool VARLEN, bool GHEAD, bool NORM>
__global__ __launch_bounds__(PTHR) void chunk_prep_kernel(PrepParams p) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    using Lo = PrepLds;
    __shared__ int s_hand[2];            // item + 1 once INV_32^T / INV_10 are in the 1 / Gamma tile (inverse phase)
    static_assert(Lo::SIZE <= 163840, "LDS budget");
    __bf16 *sQs = reinterpret_cast<__bf16 *>(smem + Lo::QS);
    __bf16 *sKs = reinterpret_cast<__bf16 *>(smem + Lo::KS);
    float *sKE = reinterpret_cast<float *>(smem + Lo::KE);
    float *sQE = reinterpret_cast<float *>(smem + Lo::QE);
    float *sKF = reinterpret_cast<float *>(smem + Lo::KF);
    float *sLI = reinterpret_cast<float *>(smem + Lo::LI);
    _Float16 *sMqk = reinterpret_cast<_Float16 *>(smem + Lo::MQK);
    float *sDg = reinterpret_cast<float *>(smem + Lo::DG);
    float *sBeta = reinterpret_cast<float *>(smem + Lo::BETA);
    float *sGB = reinterpret_cast<float *>(smem + Lo::GB);
    float *sIGB = reinterpret_cast<float *>(smem + Lo::IGB);
    float *sG = reinterpret_cast<float *>(smem + Lo::G);
    float *sGam = reinterpret_cast<float *>(smem + Lo::GAM);
    float *sRQ = reinterpret_cast<float *>(smem + Lo::RQ);
    float *sRK = reinterpret_cast<float *>(smem + Lo::RK);
    int *sFlag = reinterpret_cast<int *>(smem + Lo::FLAG);
    _Float16 *sKrt = reinterpret_cast<_Float16 *>(smem + Lo::KRT);
    // Kd^T [128][64] fp16, channel-major, built over the KF tile once it is dead
    _Float16 *sKdT = reinterpret_cast<_Float16 *>(smem + Lo::KF);
    static_assert(D * C * 2 <= C * D * 4, "Kd^T fits over the KF tile");

    const int tid0 = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid0 >> 6);   // 8 wavefronts
    const int H = p.H;
    // the chunks of this launch's window that exist
    const int wn = max(0, min(p.sv.total_chunks(), p.cw0 + p.cwn) - p.cw0);
    const int items = wn * H;
    // Items run from the last chunk to the first: the scan then starts on the
    // records written last, which are still in the device's last-level cache
    // (256 MB) when the whole set is larger.
    auto chunk_of = [&](int item) { return p.cw0 + wn - 1 - item / H; };

    // X_I (KF_I / Gamma_I)^T for diagonal block I on fp32 MFMA (X = KE gives L's
    // block, X = QE Mqk's): lane (l16, lq) gets rows 16I + 4lq + i of column
    // 16I + l16, over the 128 channels in four k-steps of 32; four partial sums
    // (k-slot e & 3) make four independent MFMA chains.
    auto diag_product = [&](const float *sX, int I, int lane) {
        const int l16 = lane & 15, lq = lane >> 4, t = 16 * I + l16;
        f32x4 a[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) a[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            // lane: row / column t, channels 32ks + 8lq + e; product e contracts
            // channels 32ks + 8j + e over the four k-slots j
            const int c0 = 32 * ks + 8 * lq;
            f32x4 x[2], bk[2];
#pragma unroll
            for (int hv = 0; hv < 2; ++hv) {
                x[hv] = *reinterpret_cast<const f32x4 *>(sX + e_at(t, c0 + 4 * hv));
                bk[hv] = *reinterpret_cast<const f32x4 *>(sKF + e_at(t, c0 + 4 * hv)) *
                         *reinterpret_cast<const f32x4 *>(sIGB + I * D + c0 + 4 * hv);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e)
                a[e & 3] = __builtin_amdgcn_mfma_f32_16x16x4f32(x[e >> 2][e & 3], bk[e >> 2][e & 3], a[e & 3], 0, 0, 0);
        }
        return (a[0] + a[1]) + (a[2] + a[3]);
    };
    // Kr^T fragment (rt, ks) of scan wavefront w: rows = channels 32w + 16rt +
    // l16, k = tokens of U's order (32ks + 4lq + {0..3}, 32ks + 16 + 4lq + {0..3})
    auto kr_frag = [&](int w, int rt, int ks, int lane) {
        typedef _Float16 f16x4_ __attribute__((ext_vector_type(4)));
        const int ch = 32 * w + 16 * rt + (lane & 15), lq = lane >> 4;
        const f16x4_ a = *reinterpret_cast<const f16x4_ *>(sKrt + kt_at(ch, 32 * ks + 4 * lq));
        const f16x4_ b = *reinterpret_cast<const f16x4_ *>(sKrt + kt_at(ch, 32 * ks + 16 + 4 * lq));
        return f16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    };

    // Inputs of one (chunk, head) item, fetched one item ahead, and the record
    // stores, carry the non-temporal hint (each byte is touched once here; the
    // hint keeps them from displacing lines the scan still reads). The loads are
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
        if ((int)blockIdx.x < items) meta_ahead = p.meta[chunk_of(blockIdx.x)];
    u32x4 rq[2], rk[2];
    float rg[16];                // g of (token 16 (tid >> 7) + tt, channel tid & 127), tt < 16
    TB rbeta = TB(0);
    int nx_h = 0, nx_tok0 = 0, nx_Lc = 0;
    // part 0: chunk bounds, q and k; part 1: g; part 2: beta; -1: all. The
    // parts go out in different phases of the current item, so that no phase
    // stalls on a full vector-memory queue.
    auto fetch = [&](int item, int part) {
        if (part <= 0) {
            const int ci = chunk_of(item);
            int2 m;
            if constexpr (VARLEN) {
                m = meta_ahead;
                meta_ahead = p.meta[chunk_of(min(item + (int)gridDim.x, items - 1))];
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
                const int idx = tid0 + it * PWORK, row = idx >> 4, part = idx & 15;
                const size_t off = ((size_t)(tok0 + min(row, Lc - 1)) * H + h) * D + 8 * part;
                rq[it] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p.q + off));
                rk[it] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p.k + off));
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
                    rg[tt] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rgc, (min(16 * I + tt, Lc - 1) * H * D + c) * 4, 0, 2));
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
        const int ci = chunk_of(item), h = nx_h, tok0 = nx_tok0, Lc = nx_Lc;
        // per-thread LDS addresses are recomputed every item instead of being
        // hoisted out of the loop and held in registers for its whole length
        int tid = tid0;
        asm volatile("" : "+v"(tid));
        const int lane = tid & 63, l16 = lane & 15, lq = lane >> 4;

        // ================= stage q and k in LDS (rows past the end: zeros, alpha = 1)
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int idx = tid + it * PWORK, row = idx >> 4, part = idx & 15;
            const u32x4 z0 = {0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4 *>(sQs + row * SQ + 8 * part) = row < Lc ? rq[it] : z0;
            *reinterpret_cast<u32x4 *>(sKs + row * SQ + 8 * part) = row < Lc ? rk[it] : z0;
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
        // (block, channel) per thread, kept in registers (rows past the end: alpha = 1)
        const int bI = tid >> 7, bc = tid & 127;
        float ev[16], fv[16];
        {
            float al[16];
#pragma unroll
            for (int tt = 0; tt < 16; ++tt) al[tt] = 16 * bI + tt < Lc ? __expf(rg[tt]) : 1.f;
            float f = 1.f;
#pragma unroll
            for (int tt = 15; tt >= 0; --tt) {
                fv[tt] = f;
                f *= al[tt];
            }
            float e = 1.f;
#pragma unroll
            for (int tt = 0; tt < 16; ++tt) {
                e *= al[tt];
                ev[tt] = e;
            }
            sGB[bI * D + bc] = e;
            sIGB[bI * D + bc] = __builtin_amdgcn_rcpf(e);     // read only for blocks with e >= FLT_MIN
            if (!(e >= kTiny)) atomicOr(&sFlag[bI], 1);     // flags were cleared during the previous item
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
        // the decayed tiles KE, QE, KF: thread (block, channel) forms its 16 rows
        // from the decays in its registers
#pragma unroll
        for (int tt = 0; tt < 16; ++tt) {
            const int t = 16 * bI + tt;
            const float kk = NORM ? bf2f(sKs[t * SQ + bc]) * sRK[t] : bf2f(sKs[t * SQ + bc]);
            const float qq = NORM ? bf2f(sQs[t * SQ + bc]) * sRQ[t] : bf2f(sQs[t * SQ + bc]);
            sKE[e_at(t, bc)] = kk * ev[tt];
            sQE[e_at(t, bc)] = qq * ev[tt];
            sKF[e_at(t, bc)] = kk * fv[tt];
        }
        __syncthreads();

        // ================= L and Mqk on MFMA, the 10 16x16 blocks with I >= J
        // Left operands x_t E_t (KE for L, QE for Mqk), t in block I.
        // Diagonal blocks (L's on wavefronts 0-3, I = J = wavefront; Mqk's on the
        // helper wavefronts 8-11): right operands k_s / E_s = KF_s / Gamma_I (start
        // of block as reference, bounded by 1 / Gamma_I; a block with Gamma_I below
        // FLT_MIN takes the exact path instead), multiplied in fp32 on
        // v_mfma_f32_16x16x4f32: near-diagonal entries dominate o, and fp32
        // operands need no hi/lo splitting.
        // Off-diagonal blocks (wavefronts 4-7): right operands KF_s
        // prod_{J<K<I} Gamma_K; every factor is <= 1, so both operands are rounded
        // once to fp16 (11-bit significand) and multiplied on fp16 MFMA. A wave's
        // blocks share their row block, so its left operands are built once.
        //   wavefront 4: (3,0) (3,1)   5: (3,2)   6: (2,0) (2,1)   7: (1,0)
        // Then waves 0-3 invert their diagonal block of I + L (the helpers form
        // Kr^T meanwhile).
        // the four flags in one LDS read (a serial read per block cost a round trip each)
        const int4 flags = *reinterpret_cast<const int4 *>(sFlag);
        if (wave < 4) {
            const int I = wave;
            if (!(I == 0 ? flags.x : I == 1 ? flags.y : I == 2 ? flags.z : flags.w)) {
                // L's block; the helper wavefront on the same SIMD forms Mqk's
                const f32x4 accL = diag_product(sKE, I, lane);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tr = 16 * I + 4 * lq + i, sc = 16 * I + l16;
                    // masked entries may hold inf / nan: select, do not scale; the
                    // block's upper triangle and diagonal are stored as zeros (the
                    // substitution below relies on them)
                    sLI[tr * SL + sc] = sc < tr ? sBeta[tr] * accL[i] : 0.f;
                }
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
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const int c0 = 32 * ks + 8 * lq;
                    const f32x4 ka0 = *reinterpret_cast<const f32x4 *>(sKE + e_at(t, c0));
                    const f32x4 ka1 = *reinterpret_cast<const f32x4 *>(sKE + e_at(t, c0 + 4));
                    const f32x4 qa0 = *reinterpret_cast<const f32x4 *>(sQE + e_at(t, c0));
                    const f32x4 qa1 = *reinterpret_cast<const f32x4 *>(sQE + e_at(t, c0 + 4));
                    f16x8 aq, ak;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        aq[e] = static_cast<_Float16>(e < 4 ? qa0[e] : qa1[e - 4]);
                        ak[e] = static_cast<_Float16>(e < 4 ? ka0[e] : ka1[e - 4]);
                    }
#pragma unroll
                    for (int bb = 0; bb < NB; ++bb) {
                        const int J = bb ? 1 : J0, sr = 16 * J + l16;
                        f32x4 b0 = *reinterpret_cast<const f32x4 *>(sKF + e_at(sr, c0));
                        f32x4 b1 = *reinterpret_cast<const f32x4 *>(sKF + e_at(sr, c0 + 4));
                        // prod_{J<K<I} Gamma_K (none for adjacent blocks)
#pragma unroll
                        for (int K = J + 1; K < I; ++K) {
                            b0 *= *reinterpret_cast<const f32x4 *>(sGB + K * D + c0);
                            b1 *= *reinterpret_cast<const f32x4 *>(sGB + K * D + c0 + 4);
                        }
                        f16x8 bk;
#pragma unroll
                        for (int e = 0; e < 8; ++e) bk[e] = static_cast<_Float16>(e < 4 ? b0[e] : b1[e - 4]);
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
                // strictly lower L and Mqk, and the diagonal d_t (sc == tr: no decay)
                for (int tr = 0; tr < 16; ++tr)
                    for (int sc = 0; sc <= tr; ++sc) {
                        const int T_ = 16 * I + tr, S_ = 16 * I + sc;
                        float accl = 0.f, accm = 0.f;
                        // raw q and k from memory (the tiles hold them decayed); rows past
                        // the end count as zeros (their loads read the last row)
                        const size_t rT = ((size_t)(tok0 + min(T_, Lc - 1)) * H + h) * D;
                        const size_t rS = ((size_t)(tok0 + min(S_, Lc - 1)) * H + h) * D;
                        const float mT = T_ < Lc ? 1.f : 0.f, mS = S_ < Lc ? 1.f : 0.f;
                        for (int c = lane; c < D; c += 64) {
                            float lg = 0.f;
                            for (int rho = S_ + 1; rho <= T_; ++rho)
                                if (rho < Lc) lg += GateRow(p.g, GHEAD, (size_t)(tok0 + rho) * H + h, D).at(c);
                            const float w = expf(lg);
                            const float kk = mS * bf16_to_f32(p.k[rS + c]);
                            accl += mT * bf16_to_f32(p.k[rT + c]) * kk * w;
                            accm += mT * bf16_to_f32(p.q[rT + c]) * kk * w;
                        }
                        accl = warp_sum(accl);
                        accm = warp_sum(accm);
                        if constexpr (NORM) {
                            accl *= sRK[T_] * sRK[S_];
                            accm *= sRQ[T_] * sRK[S_];
                        }
                        if (lane == 0) {
                            if (sc < tr) {
                                sLI[T_ * SL + S_] = sBeta[T_] * accl;
                                sMqk[T_ * SMQ + S_] = static_cast<_Float16>(accm);
                            } else {
                                sDg[T_] = accm;
                            }
                        }
                    }
                for (int e = lane; e < 256; e += 64)
                    if ((e & 15) >= (e >> 4)) {
                        sMqk[(16 * I + (e >> 4)) * SMQ + 16 * I + (e & 15)] = static_cast<_Float16>(0.f);
                        sLI[(16 * I + (e >> 4)) * SL + 16 * I + (e & 15)] = 0.f;   // L_II's upper triangle and diagonal
                    }
            }
        }
        // INV_II = (I + L_II)^{-1} of the diagonal blocks, as soon as L_II is final:
        // wave = block, by column-oriented substitution on all 64 lanes: lane
        // 4 col + g holds rows g, g + 4, g + 8, g + 12 of column col of INV_II.
        // Once x[sc] is final it is broadcast within the quad (DPP) and eliminated
        // from the lane's four rows at once; L_II's zeros on and above the
        // diagonal leave the rows at or above sc unchanged. The lane's four rows
        // of L_II are read first (16-byte rows, written by this wave). INV_II is
        // stored transposed in the block's upper triangle; entries above the
        // diagonal stay 0 (they only ever see x[sc] = 0).
        if (wave < 4) {
            const int I = wave, col = lane >> 2, g = lane & 3;
            const float *Lb = sLI + 16 * I * SL + 16 * I;    // L_II[tr][sc] = Lb[tr * SL + sc]
            f32x4 Lr[4][4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int q = 0; q < 4; ++q) Lr[k][q] = *reinterpret_cast<const f32x4 *>(Lb + (g + 4 * k) * SL + 4 * q);
            float x[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) x[k] = (g + 4 * k == col) ? 1.f : 0.f;
            auto bcast = [&](auto Sc) {                      // x[sc] of this column, from lane 4 col + sc % 4
                constexpr int sc = decltype(Sc)::value;
                return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x[sc >> 2]), 85 * (sc & 3), 0xf, 0xf, false));
            };
            auto eliminate = [&](auto Sc) {
                constexpr int sc = decltype(Sc)::value;
                const float xs = bcast(Sc);
#pragma unroll
                for (int k = 0; k < 4; ++k) x[k] -= Lr[k][sc >> 2][sc & 3] * xs;
            };
            eliminate(IC<0>{}); eliminate(IC<1>{}); eliminate(IC<2>{}); eliminate(IC<3>{}); eliminate(IC<4>{});
            eliminate(IC<5>{}); eliminate(IC<6>{}); eliminate(IC<7>{}); eliminate(IC<8>{}); eliminate(IC<9>{});
            eliminate(IC<10>{}); eliminate(IC<11>{}); eliminate(IC<12>{}); eliminate(IC<13>{}); eliminate(IC<14>{});
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (g + 4 * k >= col) sLI[(16 * I + col) * SL + 16 * I + g + 4 * k] = x[k];
        }
        __syncthreads();
        fetch(next, 1);
        // the flags were read above (into registers); clear them for the next item
        if (tid < 4) sFlag[tid] = 0;

        // ================= INV = (I + L)^{-1} off the diagonal blocks, and Kd^T
        // Waves 0-3 form the off-diagonal blocks of INV; waves 4-7 (token tile
        // tt = wave - 4) build Kd^T for the W product (into LDS, over the F tile,
        // which is dead now). The helpers build and store the Qd and Mqk record
        // fragments meanwhile.
        if (wave >= 4) {
            const int tt = wave & 3;
            // Kd^T = (k e^{a})^T = (KE G)^T, channel-major: a lane takes a token pair
            // (16 tt + 2 (lane & 7), +1) and eight-channel groups lane >> 3 and
            // (lane >> 3) + 8, and writes each (channel, token pair) as one dword.
            // The chunk-start decay of token t is G (chunk start -> block start)
            // times E (block start -> t).
            {
                const int t0 = 16 * tt + 2 * (lane & 7);
#pragma unroll
                for (int gg = 0; gg < 2; ++gg) {
                    const int c0 = 8 * ((lane >> 3) + 8 * gg);
                    const f32x4 g0 = *reinterpret_cast<const f32x4 *>(sG + tt * D + c0);
                    const f32x4 g1 = *reinterpret_cast<const f32x4 *>(sG + tt * D + c0 + 4);
                    const f32x4 ea0 = *reinterpret_cast<const f32x4 *>(sKE + e_at(t0, c0));
                    const f32x4 ea1 = *reinterpret_cast<const f32x4 *>(sKE + e_at(t0, c0 + 4));
                    const f32x4 eb0 = *reinterpret_cast<const f32x4 *>(sKE + e_at(t0 + 1, c0));
                    const f32x4 eb1 = *reinterpret_cast<const f32x4 *>(sKE + e_at(t0 + 1, c0 + 4));
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float gg_ = e < 4 ? g0[e] : g1[e - 4];
                        const float xa = (e < 4 ? ea0[e] : ea1[e - 4]) * gg_;
                        const float xb = (e < 4 ? eb0[e] : eb1[e - 4]) * gg_;
                        typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
                        const f16x2 pr = {static_cast<_Float16>(xa), static_cast<_Float16>(xb)};
                        *reinterpret_cast<f16x2 *>(sKdT + kt_at(c0 + e, t0)) = pr;
                    }
                }
            }
        }
        // off-diagonal blocks of INV on fp32 MFMA (exact products). With the 64 x 64
        // inverse taken as 2 x 2 blocks of 32 (A, D its diagonal halves, C its
        // lower-left block), INV = [[A^-1, 0], [-D^-1 C A^-1, D^-1]]:
        //   INV_10 = -INV_11 L_10 INV_00,  INV_32 = -INV_33 L_32 INV_22
        //   P_IJ = sum_{J<=K<=1} L_IK INV_KJ      (P = C A^-1; I in {2,3}, J in {0,1})
        //   INV_IJ = -sum_{2<=K<=I} INV_IK P_KJ
        // Wavefront w < 4 forms one of INV_20, INV_21, INV_30, INV_31 on its own,
        // with no barrier: what it needs of the others' blocks (INV_10, INV_32, P_2J)
        // it forms again itself, and every intermediate product stays in registers.
        // A 16x16x4 fragment in step sl takes A[row = l16][k] and B[k][col = l16]
        // from lane (l16, lq) with k = 4 lq + sl (the order of k inside a product is
        // free) and leaves C[4 lq + i][l16] there, so a product held in that layout
        // is the right operand of the next one as it stands (element sl), and the
        // transpose of such a product is a left operand. Most operands are then one
        // 16-byte LDS read: the rows of L, and the rows of INV^T (INV_XY[a][b]
        // lives at sLI[(16Y + b) * SL + 16X + a]; for X == Y only a >= b is stored,
        // the rest is selected as zero).
        if (wave < 4) {
            auto mm = [](f32x4 acc, f32x4 a, f32x4 b) {
#pragma unroll
                for (int sl = 0; sl < 4; ++sl) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[sl], b[sl], acc, 0, 0, 0);
                return acc;
            };
            const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
            const int k0 = 4 * lq;
            // L_XY[l16][k] (row-major)
            auto l_rk = [&](int X, int Y) { return *reinterpret_cast<const f32x4 *>(sLI + (16 * X + l16) * SL + 16 * Y + k0); };
            // INV_XX[k][l16], which is also INV_XX^T[l16][k]
            auto inv_kc = [&](int X) {
                f32x4 v = *reinterpret_cast<const f32x4 *>(sLI + (16 * X + l16) * SL + 16 * X + k0);
#pragma unroll
                for (int sl = 0; sl < 4; ++sl) v[sl] = k0 + sl < l16 ? 0.f : v[sl];
                return v;
            };
            // INV_XX[l16][k]
            auto inv_rk = [&](int X) {
                f32x4 v;
#pragma unroll
                for (int sl = 0; sl < 4; ++sl) {
                    const float x = sLI[(16 * X + k0 + sl) * SL + 16 * X + l16];
                    v[sl] = k0 + sl > l16 ? 0.f : x;
                }
                return v;
            };
            const int I = 2 + (wave >> 1), J = wave & 1;        // this wavefront's INV_IJ
            f32x4 inv10 = z4, inv32t = z4;
            // INV_32^T = -INV_22^T (L_32^T INV_33^T), needed by wavefronts 2 and 3, is
            // formed by wavefront 1, whose own block takes the fewest products, and
            // INV_10, needed by wavefronts 0 and 2, by wavefront 0 first; both are
            // handed over through LDS (the 1 / Gamma tile, dead in this phase) with
            // the item's number as the flag. A reader waits only where it needs the
            // block, and a writer reaches its flag with no barrier or wait on the
            // way, so the bounded waits always end.
            auto hand_over = [&](int slot, f32x4 v) {
                reinterpret_cast<f32x4 *>(sIGB)[64 * slot + lane] = v;
                asm volatile("" ::: "memory");                  // the tile's write stays before the flag's
                if (lane == 0)                                  // (and LDS keeps a wavefront's order)
                    __hip_atomic_store(&s_hand[slot], item + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            };
            auto take_over = [&](int slot) {
                for (int it = 0; it < (1 << 22) &&
                                 __hip_atomic_load(&s_hand[slot], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != item + 1;
                     ++it)
                    __builtin_amdgcn_s_sleep(1);
                asm volatile("" ::: "memory");
                return reinterpret_cast<const f32x4 *>(sIGB)[64 * slot + lane];
            };
            if (wave == 1) {
                f32x4 a, b;                                     // L_32^T[l16][k], INV_33^T[k][l16]
#pragma unroll
                for (int sl = 0; sl < 4; ++sl) {
                    a[sl] = sLI[(48 + k0 + sl) * SL + 32 + l16];
                    const float x = sLI[(48 + k0 + sl) * SL + 48 + l16];
                    b[sl] = k0 + sl > l16 ? 0.f : x;
                }
                hand_over(0, -mm(z4, inv_kc(2), mm(z4, a, b)));
            }
            if (wave == 0) {                                    // INV_10 = -INV_11 (L_10 INV_00)
                inv10 = -mm(z4, inv_rk(1), mm(z4, l_rk(1, 0), inv_kc(0)));
                hand_over(1, inv10);
            }
            // P_XJ = L_XJ INV_JJ (+ L_X1 INV_10 when J == 0)
            const f32x4 bJ = inv_kc(J);
            // the parts of P_2J and P_3J without INV_10 first
            f32x4 p2 = mm(z4, l_rk(2, J), bJ), p3 = z4;
            if (I == 3) p3 = mm(z4, l_rk(3, J), bJ);
            if (J == 0) {
                if (wave == 2) inv10 = take_over(1);
                p2 = mm(p2, l_rk(2, 1), inv10);
                if (I == 3) p3 = mm(p3, l_rk(3, 1), inv10);
            }
            f32x4 o = mm(z4, inv_rk(I), I == 2 ? p2 : p3);
            if (I == 3) {
                inv32t = take_over(0);
                o = mm(o, inv32t, p2);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) sLI[(16 * J + l16) * SL + 16 * I + 4 * lq + i] = -o[i];
            // the blocks formed on the way that are stored once
            if (wave == 0)
#pragma unroll
                for (int i = 0; i < 4; ++i) sLI[l16 * SL + 16 + 4 * lq + i] = inv10[i];          // INV_10
            if (wave == 3)
#pragma unroll
                for (int i = 0; i < 4; ++i) sLI[(32 + 4 * lq + i) * SL + 48 + l16] = inv32t[i];  // INV_32
        }
        __syncthreads();
        fetch(next, 2);

        // ================= record: fp16 fragments of the scan's operands
        // Wavefront p: token tile tt = p & 3. Every wave builds the IB fragments of
        // its token tile, which are also the right operand of W^T = Kd^T IB^T,
        // forms W for the channel tiles 4 (p >> 2) .. +3 (scan wavefronts 2 (p >> 2)
        // and 2 (p >> 2) + 1), and stores IB's token k-step p >> 2: three stores on
        // every path (a path with fewer stores than another would make the
        // compiler's wait for the next item's inputs also wait for stores). The
        // helpers store the Kr^T fragments meanwhile.
        {
            const int tt = wave & 3;
            const int t = 16 * tt + l16;
            // IB[t][s] = INV[t][s] beta_s for s = 32ks + 8lq + e; INV[t][s] is stored
            // at (s, t), zero for s > t. The read is unconditional (in bounds), so no
            // branch waits on each of them.
            f16x8 ib[2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const f32x4 be0 = *reinterpret_cast<const f32x4 *>(sBeta + 32 * ks + 8 * lq);
                const f32x4 be1 = *reinterpret_cast<const f32x4 *>(sBeta + 32 * ks + 8 * lq + 4);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int sc = 32 * ks + 8 * lq + e;
                    const float x = sLI[sc * SL + t] * (e < 4 ? be0[e] : be1[e - 4]);
                    ib[ks][e] = static_cast<_Float16>(sc <= t ? x : 0.f);
                }
            }
            f16x8 wf[2];
            // W^T tiles (channels 16 ct .. +15) x (tokens of tile tt): Kd^T rows times
            // IB^T; IB is lower triangular, so token tiles 0 and 1 need only the first
            // 32 tokens. Output layout: lane (token t, channels 16ct + 4lq + {0..3}),
            // which is the scan's channel order: channel tiles 2w and 2w + 1 give
            // elements 0-3 and 4-7 of scan wavefront w's fragment.
            {
                const int ct0 = 4 * (wave >> 2);
                f32x4 acc[4];
                static_assert(PWORK == 512, "eight main wavefronts: channel tiles 0-7");
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
                    acc[c] = mfma_f16(lds8h(sKdT + kt_at(16 * (ct0 + c) + l16, 8 * lq)), ib[0], acc[c]);
                }
                if (tt >= 2) {                                              // uniform
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        acc[c] = mfma_f16(lds8h(sKdT + kt_at(16 * (ct0 + c) + l16, 32 + 8 * lq)), ib[1], acc[c]);
                }
                // stored negated: the scan forms U = U~ + (-W) M
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int e = 0; e < 8; ++e) wf[j][e] = static_cast<_Float16>(-acc[2 * j + (e >> 2)][e & 3]);
            }
            // (scan wavefront, byte offset in its part) of every fragment:
            //   IB ks = p >> 2 -> (tt, IB + ks KB);  W j -> (2 (p >> 2) + j, NW + tt KB)
            char *rec = p.rec + ((size_t)h * p.rec_stride + ci - p.cw0) * Rec::BYTES + lane * 16;
            auto put = [&](f16x8 x, int w_s, int off) {
                __builtin_nontemporal_store(x, reinterpret_cast<f16x8 *>(rec + (size_t)w_s * Rec::WAVE + off));
            };
            put(wave >> 2 ? ib[1] : ib[0], tt, Rec::IB + (wave >> 2) * 1024);
#pragma unroll
            for (int j = 0; j < 2; ++j) put(wf[j], 2 * (wave >> 2) + j, Rec::NW + tt * 1024);
            // d (64 floats) then gamma (128 floats): one float per thread, every
            // thread issues the store and the range check drops those past the end
            static_assert(Rec::GAM == Rec::DG + C * 4, "record layout");
            const float tv = tid < C ? sDg[tid] : sGam[min(tid - C, D - 1) & (D - 1)];
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, tv),
                                                  buf_rsrc(p.rec + ((size_t)h * p.rec_stride + ci - p.cw0) * Rec::BYTES + Rec::DG,
                                                           (C + D) * 4),
                                                  tid * 4, 0, 2);
        }
        __syncthreads();      // LDS is restaged by the next item
    };
    if (tid0 < 4) sFlag[tid0] = 0;
    if (tid0 < 2) s_hand[tid0] = 0;
    __syncthreads();
    if (wave >= 8) {
        // Helper wavefronts 8-11 (block and token tile wave - 8), through the same
        // five barriers per item as the main ones: Kr^T of their block during the
        // L / Mqk phase, then the Qd and Mqk record fragments of their token tile,
        // built and stored during the inverse phase, then the Kr^T fragments of
        // scan wavefront wave - 8 during the record phase.
        const int lane = tid0 & 63, l16 = lane & 15, lq = lane >> 4;
        for (int item = blockIdx.x; item < items; item += gridDim.x) {
            const int ci = chunk_of(item), h = item % H;
            __syncthreads();                             // stage and decays
            __syncthreads();                             // decayed tiles
            // Kr^T first (vector ALU and LDS work, beside the MFMA products of the
            // diagonal wavefronts), then Mqk's diagonal block (MFMA, beside their
            // substitution, which is vector ALU work)
            // Kr = KF H for the 16 tokens of block I = wave - 8, written channel-major
            // (Kr^T) so that the record's Kr^T fragments are single 16-byte reads. A
            // lane takes a token pair (16I + 2(lane & 7), +1) and eight-channel groups
            // lane >> 3 and (lane >> 3) + 8, and writes each (channel, token pair) as
            // one dword.
            {
                const int I = wave & 3;
                const int t0 = 16 * I + 2 * (lane & 7);
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
                    const f32x4 fa0 = *reinterpret_cast<const f32x4 *>(sKF + e_at(t0, c0));
                    const f32x4 fa1 = *reinterpret_cast<const f32x4 *>(sKF + e_at(t0, c0 + 4));
                    const f32x4 fb0 = *reinterpret_cast<const f32x4 *>(sKF + e_at(t0 + 1, c0));
                    const f32x4 fb1 = *reinterpret_cast<const f32x4 *>(sKF + e_at(t0 + 1, c0 + 4));
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float hh = e < 4 ? h0[e] : h1[e - 4];
                        const float xa = (e < 4 ? fa0[e] : fa1[e - 4]) * hh;
                        const float xb = (e < 4 ? fb0[e] : fb1[e - 4]) * hh;
                        typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
                        const f16x2 pr = {static_cast<_Float16>(xa), static_cast<_Float16>(xb)};
                        *reinterpret_cast<f16x2 *>(sKrt + kt_at(c0 + e, t0)) = pr;
                    }
                }
            }
            // Mqk's diagonal block I = wave - 8 (strictly lower part, zeros on and
            // above the diagonal) and d_t = q_t . k_t, its diagonal: (q_t E_t)(k_t F_t /
            // Gamma_I) in fp32. A block on the exact path is left to its diagonal
            // wavefront.
            {
                const int4 flags = *reinterpret_cast<const int4 *>(sFlag);
                const int I = wave & 3;
                if (!(I == 0 ? flags.x : I == 1 ? flags.y : I == 2 ? flags.z : flags.w)) {
                    const f32x4 accM = diag_product(sQE, I, lane);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int tr = 16 * I + 4 * lq + i, sc = 16 * I + l16;
                        sMqk[tr * SMQ + sc] = static_cast<_Float16>(sc < tr ? accM[i] : 0.f);
                        if (sc == tr) sDg[tr] = accM[i];
                    }
                }
            }
            __syncthreads();                             // L / Mqk, diagonal inverse
            {
                f16x8 fr[6];
                const int tt = wave & 3;
                // Qd = q e^{a} = QE G for token tile tt, one fragment per scan wavefront w,
                // in that wavefront's state-channel order (channels 32w + 4lq + {0..3},
                // 32w + 16 + 4lq + {0..3})
                {
                    const int t = 16 * tt + l16;
#pragma unroll
                    for (int w = 0; w < 4; ++w)
#pragma unroll
                        for (int hh = 0; hh < 2; ++hh) {
                            const int c0 = 32 * w + 16 * hh + 4 * lq;
                            const f32x4 x4 = *reinterpret_cast<const f32x4 *>(sQE + e_at(t, c0));
                            const f32x4 g4 = *reinterpret_cast<const f32x4 *>(sG + tt * D + c0);
#pragma unroll
                            for (int i = 0; i < 4; ++i) fr[w][4 * hh + i] = static_cast<_Float16>(x4[i] * g4[i]);
                        }
                }
                // strictly lower Mqk for token tile tt in the scan's token order of U
                // (tokens 32ks + 4lq + {0..3}, 32ks + 16 + 4lq + {0..3}); blocks above
                // the diagonal block are never written and are selected as zeros (a
                // select, so stale LDS contents cannot leak in)
                {
                    const int t = 16 * tt + l16;
                    typedef _Float16 f16x4_ __attribute__((ext_vector_type(4)));
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                        for (int hh = 0; hh < 2; ++hh) {
                            const f16x4_ mq = *reinterpret_cast<const f16x4_ *>(sMqk + t * SMQ + 32 * ks + 16 * hh + 4 * lq);
                            const bool zero = 2 * ks + hh > tt;
#pragma unroll
                            for (int i = 0; i < 4; ++i) fr[4 + ks][4 * hh + i] = zero ? static_cast<_Float16>(0.f) : mq[i];
                        }
                }
                // Qd w -> (w, QD + tt KB); Mqk ks -> (tt, MQ + ks KB)
                char *rec = p.rec + ((size_t)h * p.rec_stride + ci - p.cw0) * Rec::BYTES + lane * 16;
#pragma unroll
                for (int i = 0; i < 6; ++i)
                    __builtin_nontemporal_store(fr[i], reinterpret_cast<f16x8 *>(
                        rec + (size_t)(i < 4 ? i : tt) * Rec::WAVE + (i < 4 ? Rec::QD + tt * 1024 : Rec::MQ + (i - 4) * 1024)));
            }
            __syncthreads();                             // off-diagonal inverse
            // the Kr^T fragments of scan wavefront wave - 8: (wave - 8, KR + (2 rt + ks) KB)
            {
                char *rec = p.rec + ((size_t)h * p.rec_stride + ci - p.cw0) * Rec::BYTES + lane * 16;
#pragma unroll
                for (int f = 0; f < 4; ++f)
                    __builtin_nontemporal_store(kr_frag(wave & 3, f >> 1, f & 1, lane),
                                                reinterpret_cast<f16x8 *>(rec + (size_t)(wave & 3) * Rec::WAVE + Rec::KR + f * 1024));
            }
            __syncthreads();                             // record
        }
        return;
    }
    if ((int)blockIdx.x < items) {
        fetch(blockIdx.x, -1);
        body(blockIdx.x);
    }
    for (int item = blockIdx.x + gridDim.x; item < items; item += gridDim.x) body(item);
}

// ---------------------------------------------------------------- scan
// One workgroup per (sequence, head, TV-column tile); the chunks of the
// sequence in order. Two roles of four wavefronts (one of each per SIMD),
// sharing two barriers per chunk:
//   recurrence wavefront w keeps state rows (channels) 32w..32w+31 in fp32
//   accumulators. After barrier A (the state is in LDS) it forms U for its 16
//   tokens, U = U~ - W M over all 128 channels, and puts U in LDS; after
//   barrier B it updates its rows, M <- Diag(gamma) M + Kr^T U, puts them in
//   LDS for the next chunk, and forms that chunk's U~ = IB V for its tokens
//   (off the dependency chain, kept in registers).
//   output wavefront w (tokens 16w..16w+15) forms o = Qd M + Mqk U + d U from
//   the same LDS copies (Qd M between A and B, the rest after B) and stages
//   the next chunk's V in LDS.
// The two dependent contraction stages (U, then the state) are the whole
// serial chain of a chunk. The state and U are split into fp16 hi + lo when
// they are put in LDS (two products each, ~22 significant bits); the record's
// fragments follow their register order, so every LDS read is one 16-byte read.
//
// Scale: the recurrence is linear in (V, S0), so the workgroup runs on V and
// S0 scaled by a power of two 2^e chosen from the running maximum R of |S0|
// and |V| (over its columns, up to the next chunk), such that R 2^e lies in
// [64, 128): the fp16 parts keep their relative precision however small the
// inputs are and do not overflow however large (65504 = 2^16 leaves 2^9 of
// headroom for the state's growth over R). A change of e rescales the state
// exactly (powers of two), and o, S_out and snapshots are scaled back.
constexpr int NREC = 256;                // recurrence wavefronts, one per SIMD ...
constexpr int SCAN_THR = 2 * NREC;       // ... and as many output wavefronts
// LDS tiles are [col][k] rows of 16-byte blocks, the block index XOR-ed with
// the row: an MFMA operand read (16 lanes per bank cycle, 64 banks) then takes
// 16 rows at one block index from 16 distinct bank groups. Measured on gfx950,
// a plain padded row stride costs one extra cycle per 16 lanes on these reads.
constexpr int SMS = D;                   // fp16 row of the state   [col][128], blocks ^ (col & 15)
constexpr int SUS = C;                   // fp16 row of U           [col][64],  blocks ^ (col & 7)
constexpr int SVT = C;                   // bf16 row of the V tile  [col][64],  blocks ^ vsw(col)
// the V tile's block swizzle: the column's low three bits XOR-ed with the next
// three, so that the four lanes staging one token (columns TV / 4 apart) write
// to four distinct blocks at every tile width
__device__ __forceinline__ int vsw(int col) { return (col ^ (col >> 3)) & 7; }

template <int TV>
struct ScanLds {
    static constexpr int M = 0;                          // fp16 [2][TV][SMS] state hi / lo, [col][channel, register order]
    static constexpr int U = M + 2 * TV * SMS * 2;       // fp16 [2][TV][SUS] U hi / lo, [col][token, register order]
    static constexpr int UF = U + 2 * TV * SUS * 2;      // fp32 [C][TV + 4] U, [token][col] (the output's d U term)
    static constexpr int V = UF + C * (TV + 4) * 4;      // bf16 [2][TV][SVT] V of a chunk, [col][token]
    static constexpr int VMAX = V + 2 * TV * SVT * 2;    // fp32 [2][4] max |v| per output wavefront, then [4] max |S0|
    static constexpr int SIZE = VMAX + 12 * 4;
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
    // window: global chunks cw0 .. cw0 + cwn - 1 (record index chunk - cw0). A
    // chain whose chunks continue past the window leaves its state in S_run, and
    // one whose chunks began before it takes its state from there.
    float *S_run;
    int cw0, cwn;
    // packed sequences: order[i] = the sequence with the i-th most chunks (ties
    // by index), so that the workgroups of the longest chains are dispatched
    // first; nullptr: sequence order
    const int32_t *order;
};

// exponent e with R 2^e in [64, 128) (R > 0), clamped; 7 for R == 0
__device__ __forceinline__ int scale_exp(float R) {
    return min(100, max(-100, 7 - __builtin_amdgcn_frexp_expf(R)));
}

template <int CTRL> __device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
// max over the wavefront, on the vector ALU: rotations within rows of 16 lanes
// (DPP row_ror 1, 2, 4, 8), then the four row maxima read as scalars
__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, dpp_f<0x121>(x));
    x = fmaxf(x, dpp_f<0x122>(x));
    x = fmaxf(x, dpp_f<0x124>(x));
    x = fmaxf(x, dpp_f<0x128>(x));
    const int b = __float_as_int(x);
    return fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 0)), __int_as_float(__builtin_amdgcn_readlane(b, 16))),
                 fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 32)), __int_as_float(__builtin_amdgcn_readlane(b, 48))));
}

__device__ __forceinline__ float max4(f32x4 x) { return fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])); }

template <int TV, typename TO>
__global__ __launch_bounds__(SCAN_THR) void chunk_scan_kernel(ScanParams p) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    using Lo = ScanLds<TV>;
    constexpr int NT = TV / 16;
    constexpr int TEAM = D / TV;
    constexpr int VW = TV / 8;           // dwords of V per output thread and chunk (TV / 4 columns of one token)
    static_assert(TV == 16 || TV == 32 || TV == 64, "value columns per workgroup");
    _Float16 *sMh = reinterpret_cast<_Float16 *>(smem + Lo::M);
    _Float16 *sMl = sMh + TV * SMS;
    _Float16 *sUh = reinterpret_cast<_Float16 *>(smem + Lo::U);
    _Float16 *sUl = sUh + TV * SUS;
    float *sUf = reinterpret_cast<float *>(smem + Lo::UF);
    bf16_t *sV = reinterpret_cast<bf16_t *>(smem + Lo::V);
    float *sVmax = reinterpret_cast<float *>(smem + Lo::VMAX);

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, lq = lane >> 4;
    const int w4 = wave & 3;             // token tile (both roles) and state rows (recurrence)
    // XCD-aware placement: block b runs on XCD b % 8; the TEAM workgroups of
    // one chain share b % 8 and so one L2, where the chain's records are read.
    const int b = blockIdx.x;
    const int xcd = b & 7, r = b >> 3;
    const int member = r % TEAM, grp = r / TEAM;
    const int chain = grp * 8 + xcd;
    if (chain >= p.chains) return;
    const int H = p.H, n = p.order ? p.order[chain / H] : chain / H, h = chain % H;
    const int col0 = member * TV;
    const int start = p.sv.seq_start(n), end = p.sv.seq_end(n);
    const int nch = (end - start + C - 1) / C, c0 = p.sv.first_chunk(n);
    // this launch's chunks j0 .. j1 - 1 of the sequence, and where its state
    // comes from and goes to
    const int j0 = min(nch, max(0, p.cw0 - c0)), j1 = min(nch, max(0, p.cw0 + p.cwn - c0));
    const int last = j1 - 1;
    const float *S_in = j0 == 0 ? p.S0 : p.S_run;
    float *S_fin = j1 == nch ? p.S_out : p.S_run;
    const size_t st_off = ((size_t)n * H + h) * D * D;
    // bytes from a chunk's first row to the end of its last valid row
    auto chunk_bytes = [&](int Lc, int elem) { return ((Lc - 1) * H * D + D) * elem; };
    auto rec_rsrc = [&](int j) {
        return buf_rsrc(p.rec + ((size_t)h * p.rec_stride + c0 + j - p.cw0) * Rec::BYTES, Rec::BYTES);
    };
    const int r_lane = lane * 16;
    // B-operand fragments from LDS: the state's k-step kk (channels of
    // recurrence wavefront kk), U's token k-step ks
    auto m_frag = [&](const _Float16 *base, int nt, int kk) {
        return lds8h(base + (16 * nt + l16) * SMS + 8 * ((4 * kk + lq) ^ l16));
    };
    auto u_frag = [&](const _Float16 *base, int nt, int ks) {
        return lds8h(base + (16 * nt + l16) * SUS + 8 * ((4 * ks + lq) ^ (l16 & 7)));
    };
    // U's position for token 16tt + 4lq + i: 32 (tt >> 1) + 8lq + 4 (tt & 1) + i
    const int u_at = (l16 * SUS) + 8 * ((4 * (w4 >> 1) + lq) ^ (l16 & 7)) + 4 * (w4 & 1);

    if (wave < 4) {
        // ============================ recurrence
        // the state S [Dv][Dk] in memory: this lane's four channels 32w + 16rt + 4lq
        // .. +3 of value column col are one 16-byte piece of row col
        auto st_at = [&](int rt, int nt) {
            return st_off + (size_t)(col0 + 16 * nt + l16) * D + 32 * w4 + 16 * rt + 4 * lq;
        };
        f32x4 Macc[2][NT];
        float m0 = 0.f;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                Macc[rt][nt] = S_in ? *reinterpret_cast<const f32x4 *>(S_in + st_at(rt, nt)) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i < 4; ++i) m0 = fmaxf(m0, fabsf(Macc[rt][nt][i]));
            }
        if (j0 >= j1) {
            // nothing to scan in this launch; an empty sequence: S_out = S0 exactly
            if (nch == 0 && p.S_out)
#pragma unroll
                for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) *reinterpret_cast<f32x4 *>(p.S_out + st_at(rt, nt)) = Macc[rt][nt];
            return;
        }
        m0 = wave_max(m0);
        if (lane == 0) sVmax[8 + w4] = m0;
        // the state into LDS (hi / lo, register order: channel 32w + 16rt + 4lq + i
        // at position 32w + 8lq + 4rt + i)
        auto publish = [&]() {
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    f16x4 hi, lo;
#pragma unroll
                    for (int i = 0; i < 4; ++i) SPLITH(Macc[rt][nt][i], hi[i], lo[i]);
                    const int at = (16 * nt + l16) * SMS + 8 * ((4 * w4 + lq) ^ l16) + 4 * rt;
                    *reinterpret_cast<f16x4 *>(sMh + at) = hi;
                    *reinterpret_cast<f16x4 *>(sMl + at) = lo;
                }
        };
        struct Frags {
            f16x8 nw[4], ib[2], kr[2][2];
            f32x4 gm[2];
        };
        // The operand loads of one chunk as 12 slots: -W for this wavefront's
        // token tile (k-step kk in recurrence wavefront kk's part of the
        // record), IB, Kr^T and gamma (its own part). A step issues the next
        // chunk's slots one at a time between its products: a burst of loads
        // right after a barrier, from every wavefront at once, fills the CU's
        // vector-memory queue and stalls the wavefronts in order.
        auto issue = [&](__amdgpu_buffer_rsrc_t rr, Frags &f, int sl) __attribute__((always_inline)) {
            if (sl < 4) f.nw[sl] = buf_ld16<f16x8>(rr, r_lane, sl * Rec::WAVE + Rec::NW + w4 * 1024);
            else if (sl < 6) f.ib[sl - 4] = buf_ld16<f16x8>(rr, r_lane, w4 * Rec::WAVE + Rec::IB + (sl - 4) * 1024);
            else if (sl < 10) f.kr[(sl - 6) >> 1][(sl - 6) & 1] = buf_ld16<f16x8>(rr, r_lane, w4 * Rec::WAVE + Rec::KR + (sl - 6) * 1024);
            else f.gm[sl - 10] = buf_ld16<f32x4>(rr, Rec::GAM + (32 * w4 + 4 * lq) * 4, (sl - 10) * 64);
            __builtin_amdgcn_sched_barrier(0);
        };
        auto issue_all = [&](int j, Frags &f) {
            const auto rr = rec_rsrc(j);
#pragma unroll
            for (int sl = 0; sl < 12; ++sl) issue(rr, f, sl);
        };
        // U~ = IB (2^ex V) for this wavefront's tokens, from V in LDS buffer bsel
        f32x4 ut[NT];
        auto pseudo_values = [&](const Frags &f, int bsel, float sc) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                ut[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const bf16x8 vv = lds8(reinterpret_cast<const __bf16 *>(sV) + bsel * TV * SVT + (16 * nt + l16) * SVT +
                                           8 * ((4 * ks + lq) ^ vsw(16 * nt + l16)));
                    f16x8 vb;
#pragma unroll
                    for (int e = 0; e < 8; ++e) vb[e] = static_cast<_Float16>(bf2f(vv[e]) * sc);
                    ut[nt] = mfma_f16(f.ib[ks], vb, ut[nt]);
                }
            }
        };
        float R = 0.f;
        int ex = 0;
        auto step = [&](Frags &f, int j, Frags &f1, Frags &nf, int nj) {
            const auto rn = rec_rsrc(nj);
            const int bsel = j & 1;
            // U = U~ + (-W) M for tokens 16w4 .. +15
            // (the hi and lo products accumulate in two chains of four)
            f32x4 u[NT], ul_[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                u[nt] = ut[nt];
                ul_[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    u[nt] = mfma_f16(f.nw[kk], m_frag(sMh, nt, kk), u[nt]);
                    ul_[nt] = mfma_f16(f.nw[kk], m_frag(sMl, nt, kk), ul_[nt]);
                }
                issue(rn, nf, kk);
            }
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) u[nt] += ul_[nt];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                f16x4 hi, lo;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    SPLITH(u[nt][i], hi[i], lo[i]);
                    sUf[(16 * w4 + 4 * lq + i) * (TV + 4) + 16 * nt + l16] = u[nt][i];
                }
                *reinterpret_cast<f16x4 *>(sUh + u_at + 16 * nt * SUS) = hi;
                *reinterpret_cast<f16x4 *>(sUl + u_at + 16 * nt * SUS) = lo;
            }
            issue(rn, nf, 4);
            issue(rn, nf, 5);
            __syncthreads();                                 // B: U (and the next chunk's V) are in LDS
            R = fmaxf(R, max4(*reinterpret_cast<const f32x4 *>(sVmax + (bsel ^ 1) * 4)));
            const int ex1 = scale_exp(R);
            const float fs = __builtin_amdgcn_ldexpf(1.f, ex1 - ex);
            // M <- Diag(gamma) M + Kr^T U for channels 32w4 .. +31, then into the
            // next chunk's scale
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) Macc[rt][nt] *= f.gm[rt];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) {
                        Macc[rt][nt] = mfma_f16(f.kr[rt][ks], u_frag(sUh, nt, ks), Macc[rt][nt]);
                        Macc[rt][nt] = mfma_f16(f.kr[rt][ks], u_frag(sUl, nt, ks), Macc[rt][nt]);
                    }
                    issue(rn, nf, 6 + 2 * rt + ks);
                }
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) Macc[rt][nt] *= fs;
            ex = ex1;
            if (float *sp = p.snap.slot(n, h, H, j + 1, end - start, C, D * D)) {   // uniform across the workgroup
                const float inv = __builtin_amdgcn_ldexpf(1.f, -ex);
#pragma unroll
                for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
                        *reinterpret_cast<f32x4 *>(sp + (st_at(rt, nt) - st_off)) = Macc[rt][nt] * inv;
            }
            publish();
            issue(rn, nf, 10);
            issue(rn, nf, 11);
            // the next chunk's U~ (its V is in LDS since barrier B), in its scale
            pseudo_values(f1, bsel ^ 1, __builtin_amdgcn_ldexpf(1.f, ex));
            __syncthreads();                                 // A: the next state is in LDS
        };
        Frags A, B, Cb;
        issue_all(j0, A);
        issue_all(min(j0 + 1, last), B);
        __syncthreads();                                     // S0 and chunk 0's V (and their maxima) are in LDS
        R = fmaxf(max4(*reinterpret_cast<const f32x4 *>(sVmax + 8)), max4(*reinterpret_cast<const f32x4 *>(sVmax)));
        ex = scale_exp(R);
        {
            const float s0 = __builtin_amdgcn_ldexpf(1.f, ex);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) Macc[rt][nt] *= s0;
            publish();
            pseudo_values(A, 0, s0);
        }
        __syncthreads();                                     // A: the initial state is in LDS
        // Rounds of six steps (two turns of the three operand buffers): at the
        // loop's back edge the compiler waits for more of the prefetched
        // operands than a step needs, so the back edge is kept rare.
        for (int j = j0; j < j1; j += 6) {
            step(A, j, B, Cb, min(j + 2, last));
            if (j + 1 >= j1) break;
            step(B, j + 1, Cb, A, min(j + 3, last));
            if (j + 2 >= j1) break;
            step(Cb, j + 2, A, B, min(j + 4, last));
            if (j + 3 >= j1) break;
            step(A, j + 3, B, Cb, min(j + 5, last));
            if (j + 4 >= j1) break;
            step(B, j + 4, Cb, A, min(j + 6, last));
            if (j + 5 >= j1) break;
            step(Cb, j + 5, A, B, min(j + 7, last));
        }
        if (S_fin) {
            const float inv = __builtin_amdgcn_ldexpf(1.f, -ex);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) *reinterpret_cast<f32x4 *>(S_fin + st_at(rt, nt)) = Macc[rt][nt] * inv;
        }
        return;
    }

    // ============================ output
    if (j0 >= j1) return;
    const int stid = tid - NREC;         // 0 .. 255
    // the operands of chunk c; vr holds the V of chunk c as well, loaded three
    // chunks ahead (it comes from HBM, the records mostly from cache)
    struct OFrags {
        f16x8 qd[4], mq[2];
        float dv;                        // d of token 16w4 + l16
        uint32_t vr[VW];                 // V of token stid >> 2, columns col0 + (TV / 4)(stid & 3) ..
    };
    const int v_off = ((stid >> 2) * H * D + col0 + (TV / 4) * (stid & 3)) * 2;
    auto vissue = [&](int j, OFrags &f) {
        const int tok0 = start + j * C, Lc = min(C, end - tok0);
        // V rows past the end of the sequence read 0 (outside the range)
        const auto rv = buf_rsrc(p.v + ((size_t)tok0 * H + h) * D, chunk_bytes(Lc, 2));
        if constexpr (VW == 2) {
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            const u32x2 x = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rv, v_off, 0, 0));
            f.vr[0] = x[0]; f.vr[1] = x[1];
        } else {
#pragma unroll
            for (int q = 0; q < VW / 4; ++q) {
                const u32x4 x = buf_ld16<u32x4>(rv, v_off + 16 * q, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i) f.vr[4 * q + i] = x[i];
            }
        }
        __builtin_amdgcn_sched_barrier(0x048F);
    };
    // the record loads as 7 slots: Qd (k-step kk in recurrence wavefront kk's
    // part), Mqk, d; issued one at a time between the products, like the
    // recurrence's
    auto oissue = [&](__amdgpu_buffer_rsrc_t rr, OFrags &f, int sl) __attribute__((always_inline)) {
        if (sl < 4) f.qd[sl] = buf_ld16<f16x8>(rr, r_lane, sl * Rec::WAVE + Rec::QD + w4 * 1024);
        else if (sl < 6) f.mq[sl - 4] = buf_ld16<f16x8>(rr, r_lane, w4 * Rec::WAVE + Rec::MQ + (sl - 4) * 1024);
        else f.dv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rr, Rec::DG + (16 * w4 + l16) * 4, 0, 0));
        __builtin_amdgcn_sched_barrier(0);
    };
    auto oissue_all = [&](int j, OFrags &f) {
        const auto rr = rec_rsrc(j);
#pragma unroll
        for (int sl = 0; sl < 7; ++sl) oissue(rr, f, sl);
    };
    // V of a chunk into LDS buffer bsel, transposed to [col][token], and this
    // wavefront's max |v| of it into slot bsel
    auto stage_v = [&](const OFrags &f, int bsel) {
        const int t = stid >> 2, c0 = (TV / 4) * (stid & 3);
        bf16_t *dst = sV + bsel * TV * SVT + (t & 7);
        float vm = 0.f;
#pragma unroll
        for (int e = 0; e < 2 * VW; ++e) {
            const uint32_t wv = f.vr[e >> 1];
            const bf16_t x = static_cast<bf16_t>(e & 1 ? wv >> 16 : wv & 0xffffu);
            const int c = c0 + e;
            dst[c * SVT + 8 * ((t >> 3) ^ vsw(c))] = x;
            vm = fmaxf(vm, fabsf(bf16_to_f32(x)));
        }
        vm = wave_max(vm);
        if (lane == 0) sVmax[bsel * 4 + w4] = vm;
    };
    // this lane's outputs: token 16w4 + l16, columns col0 + 16nt + 4lq .. +3
    const int o_base = ((16 * w4 + l16) * H * D + col0 + 4 * lq) * (int)sizeof(TO);
    float R = 0.f;
    int ex = 0;
    // L2 warming: the TEAM workgroups of a chain read every record, on one XCD.
    // Three chunks ahead, each output wavefront touches one dword of every
    // 128-byte line of its share of the record, so that the records' lines are
    // in L2 when the operand loads arrive. The touched values are folded into a
    // register one step later (that load is then long complete) and kept alive
    // to the end by an empty asm that takes them as input. Not with 64-column
    // workgroups: they run where the chains fill the CUs many times over, 16
    // chains per XCD, and three chunks of their records in flight would nearly
    // fill the XCD's 4 MB L2, so that lines were evicted before the team's
    // second workgroup read them.
    constexpr int LPW = Rec::DG / 128 / (4 * TEAM);                 // lines per wavefront
    const int touch_off = ((member * 4 + w4) * LPW + lane % LPW) * 128;  // < Rec::DG
    uint32_t touch_acc = 0, touch_prev = 0;
    auto ostep = [&](OFrags &f, int j, OFrags &nf, int nj) {
        const int bsel = j & 1;
        touch_acc ^= touch_prev;
        if constexpr (TV < 64)
            touch_prev = __builtin_amdgcn_raw_buffer_load_b32(rec_rsrc(min(j + 3, last)), touch_off, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        vissue(min(j + 3, last), f);     // this buffer's chunk after next: j + 3
        // o^T (part) = M^T Qd^T from the state at the chunk start (in LDS since
        // barrier A), formed transposed so that a lane holds four consecutive
        // columns of one token; the hi and lo products in two chains
        // (o only: the state's fp16 hi part, 11 significant bits, is enough here)
        const auto rn = rec_rsrc(nj);
        f32x4 acc[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc[nt] = mfma_f16(m_frag(sMh, nt, kk), f.qd[kk], acc[nt]);
            oissue(rn, nf, kk);
        }
        __syncthreads();                                     // B: U (and the next chunk's V) are in LDS
        R = fmaxf(R, max4(*reinterpret_cast<const f32x4 *>(sVmax + (bsel ^ 1) * 4)));
        // o = Qd M + Mqk U + d U in this chunk's scale; back to input units
        const int tok0 = start + j * C, Lc = min(C, end - tok0);
        const auto ro = buf_rsrc(static_cast<TO *>(p.out) + ((size_t)tok0 * H + h) * D, chunk_bytes(Lc, sizeof(TO)));
        const float inv = __builtin_amdgcn_ldexpf(1.f, -ex);
        const float d_t = f.dv;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            // o^T += U^T Mqk^T (U's hi part), then d_t U[t] in fp32: token
            // t = 16w4 + l16, columns 16nt + 4lq + i
            f32x4 o = acc[nt];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                o = mfma_f16(u_frag(sUh, nt, ks), f.mq[ks], o);
                if (nt == NT - 1) oissue(rn, nf, 4 + ks);
            }
            const f32x4 uf = *reinterpret_cast<const f32x4 *>(sUf + (16 * w4 + l16) * (TV + 4) + 16 * nt + 4 * lq);
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = (o[i] + d_t * uf[i]) * inv;
            buf_st4<TO>(ro, o_base + 16 * nt * (int)sizeof(TO), o);
        }
        oissue(rn, nf, 6);
        // V of chunk j + 2 and its max into the buffer chunk j's V has left (read
        // before barrier A of this step); staged here, after barrier B, where
        // this wavefront waits for the recurrence anyway
        stage_v(nf, bsel);
        ex = scale_exp(R);
        __syncthreads();                                     // A: the next state is in LDS
    };
    OFrags A, B, Cb;
    vissue(j0, A);
    oissue_all(j0, A);
    vissue(min(j0 + 1, last), B);
    oissue_all(min(j0 + 1, last), B);
    vissue(min(j0 + 2, last), Cb);
    stage_v(A, 0);
    stage_v(B, 1);
    __syncthreads();                                         // S0 and chunk 0's V (and their maxima) are in LDS
    R = fmaxf(max4(*reinterpret_cast<const f32x4 *>(sVmax + 8)), max4(*reinterpret_cast<const f32x4 *>(sVmax)));
    ex = scale_exp(R);
    __syncthreads();                                         // A: the initial state is in LDS
    // rounds of six steps, as for the recurrence
    for (int j = j0; j < j1; j += 6) {
        ostep(A, j, Cb, min(j + 2, last));
        if (j + 1 >= j1) break;
        ostep(B, j + 1, A, min(j + 3, last));
        if (j + 2 >= j1) break;
        ostep(Cb, j + 2, B, min(j + 4, last));
        if (j + 3 >= j1) break;
        ostep(A, j + 3, Cb, min(j + 5, last));
        if (j + 4 >= j1) break;
        ostep(B, j + 4, A, min(j + 6, last));
        if (j + 5 >= j1) break;
        ostep(Cb, j + 5, B, min(j + 7, last));
    }
    asm volatile("" ::"v"(touch_acc ^ touch_prev));
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

// workspace: chunk offsets (N + 1 int32) and the chains' order (N int32), the
// chunk table (maxc int2), records
size_t ws_offs(int N) { return ((sizeof(int32_t) * (size_t)(2 * N + 1) + 255) / 256) * 256; }
size_t ws_meta(long long maxc) { return ((sizeof(int2) * (size_t)maxc + 255) / 256) * 256; }

// One long sequence runs as a pipeline over windows of WIN chunks: the prep of
// window w + 1 (on a second stream, on the CUs the scan leaves free) overlaps
// the scan of window w, and the records of only two windows exist at a time.
// The chain's state passes from window to window through S_run.
constexpr long long WIN = 512;
// window starts stay even: the scan's V double buffer is indexed by chunk parity
// from a prologue that stages the first chunk's V into buffer 0
static_assert(WIN % 2 == 0, "even window length");
// (maxc - 1: the chunks of one sequence; max_chunks counts one more per sequence)
bool windowed(int N, long long maxc) { return N == 1 && maxc - 1 >= 4 * WIN; }
size_t ws_records(int N, long long maxc, int H) {
    return (size_t)(windowed(N, maxc) ? 2 * WIN : maxc) * H * Rec::BYTES;
}
size_t ws_state(int N, long long maxc, int H) {
    return windowed(N, maxc) ? (size_t)H * D * D * sizeof(float) : 0;
}

// The events and the stream of one pipelined call, released on every exit
// path. Destruction does not wait: the runtime releases them once the work
// queued on them has completed.
struct Pipeline {
    hipStream_t side = nullptr;
    hipEvent_t ev[5] = {};
    ~Pipeline() {
        for (hipEvent_t e : ev)
            if (e) (void)hipEventDestroy(e);
        if (side) (void)hipStreamDestroy(side);
    }
    hipError_t init() {
        for (hipEvent_t &e : ev)
            if (const hipError_t r = hipEventCreateWithFlags(&e, hipEventDisableTiming); r != hipSuccess) return r;
        return hipStreamCreateWithFlags(&side, hipStreamNonBlocking);
    }
};

template <typename TB, typename TO>
hipError_t run(const PrefillArgs &a) {
    const long long maxc = max_chunks(a.N, (long long)a.B * a.T, C);
    char *ws = static_cast<char *>(a.ws);
    int32_t *chunk_off = reinterpret_cast<int32_t *>(ws);
    int2 *meta = reinterpret_cast<int2 *>(ws + ws_offs(a.N));
    char *recs = ws + ws_offs(a.N) + ws_meta(maxc);
    float *S_run = reinterpret_cast<float *>(recs + ws_records(a.N, maxc, a.H));
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
        if (a.N > 1 && a.N <= ORDER_MAX) {
            hipLaunchKernelGGL(chain_order_kernel, dim3(1), dim3(ORDER_MAX), 0, a.stream, sv, chunk_off + a.N + 1);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    // kernel variant [varlen][per-head gate][L2-normalised q, k]
    using PrepKern = void (*)(PrepParams);
    const PrepKern kerns[2][2][2] = {
        {{chunk_prep_kernel<TB, false, false, false>, chunk_prep_kernel<TB, false, false, true>},
         {chunk_prep_kernel<TB, false, true, false>, chunk_prep_kernel<TB, false, true, true>}},
        {{chunk_prep_kernel<TB, true, false, false>, chunk_prep_kernel<TB, true, false, true>},
         {chunk_prep_kernel<TB, true, true, false>, chunk_prep_kernel<TB, true, true, true>}}};
    const PrepKern prep_kern = kerns[varlen][a.g_head][a.qk_norm];
    // Value columns per scan workgroup: one workgroup fits on a CU, so the
    // scan takes about (rounds of workgroups over the CUs) x (steps of the
    // longest chain) x (time of a step). A step of a 16-, 32- or 64-column
    // workgroup takes about 1.3, 1.8 and 2.9 us on MI355X: wider tiles read each
    // record once for more columns, narrower ones put more CUs on a chain. The
    // width with the fewest rounds x step time is taken (the narrower on a tie).
    const int chains = a.N * a.H;
    int tv = 16;
    {
        long long best = -1;
        for (const int w : {16, 32, 64}) {
            const long long rounds = ((long long)chains * (D / w) + cus - 1) / cus;
            const long long cost = rounds * (w == 16 ? 13 : w == 32 ? 18 : 29);
            if (best < 0 || cost < best) { best = cost; tv = w; }
        }
    }
    const int team = D / tv;
    const unsigned scan_blocks = (unsigned)((chains + 7) / 8) * 8u * (unsigned)team;
    using ScanKern = void (*)(ScanParams);
    const ScanKern scan_kern = tv == 64 ? chunk_scan_kernel<64, TO> : tv == 32 ? chunk_scan_kernel<32, TO> : chunk_scan_kernel<16, TO>;
    const int scan_lds = tv == 64 ? ScanLds<64>::SIZE : tv == 32 ? ScanLds<32>::SIZE : ScanLds<16>::SIZE;
    // set on every call (idempotent; no process-wide "already set" flag to race on)
    if (hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(prep_kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, PrepLds::SIZE);
        e != hipSuccess)
        return e;
    if (hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(scan_kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, scan_lds);
        e != hipSuccess)
        return e;

    // prep of global chunks cw0 .. cw0 + cwn - 1 into `slot` (cwn records per head)
    auto prep = [&](long long cw0, long long cwn, char *slot, unsigned max_grid, hipStream_t st) {
        PrepParams pp{static_cast<const bf16_t *>(a.q), static_cast<const bf16_t *>(a.k), a.g, a.beta, sv, meta,
                      a.H, slot, cwn, a.norm_eps, (int)cw0, (int)cwn};
        // persistent: at most one workgroup per CU walks the (chunk, head) items
        const unsigned grid = (unsigned)std::min<long long>(cwn * a.H, max_grid);
        hipLaunchKernelGGL(prep_kern, dim3(grid), dim3(PTHR), PrepLds::SIZE, st, pp);
        return hipGetLastError();
    };
    auto scan = [&](long long cw0, long long cwn, const char *slot, hipStream_t st) {
        ScanParams sp{static_cast<const bf16_t *>(a.v), a.S0, a.out, a.S_out, sv, a.H, chains, slot, cwn,
                      SnapView{a.snaps, a.snap_every, a.max_snaps}, S_run, (int)cw0, (int)cwn,
                      varlen && a.N > 1 && a.N <= ORDER_MAX ? chunk_off + a.N + 1 : nullptr};
        hipLaunchKernelGGL(scan_kern, dim3(scan_blocks), dim3(SCAN_THR), scan_lds, st, sp);
        return hipGetLastError();
    };

    if (!windowed(a.N, maxc)) {
        if (maxc * a.H > 0)
            if (hipError_t e = prep(0, maxc, recs, (unsigned)cus, a.stream); e != hipSuccess) return e;
        return scan(0, maxc, recs, a.stream);
    }

    // Windowed pipeline. Slot w % 2 holds window w's records; the prep of window
    // w waits for the scan of window w - 2 (the slot's previous reader), the
    // scan of window w for the prep of window w. The preps overlap the scans
    // only where the scan's workgroups, one per CU, leave half of the CUs free
    // (a prep that took CUs the scan needs would hold back part of its chains
    // for a whole window); otherwise, and while a stream capture is under way
    // on the caller's stream or for a caller that asked for it (in_order),
    // everything runs in order on that stream (same results, bounded workspace).
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipError_t e = hipStreamIsCapturing(a.stream, &cap); e != hipSuccess) return e;
    const bool concurrent = !a.in_order && cap == hipStreamCaptureStatusNone && scan_blocks * 2 <= (unsigned)cus;
    Pipeline pl;     // created only outside a capture
    if (concurrent)
        if (hipError_t e = pl.init(); e != hipSuccess) return e;
    hipStream_t ps = concurrent ? pl.side : a.stream;
    hipEvent_t ev_in = pl.ev[0], ev_prep[2] = {pl.ev[1], pl.ev[2]}, ev_scan[2] = {pl.ev[3], pl.ev[4]};
    // the prep stream starts after the caller's earlier work (inputs, chunk table)
    if (concurrent) {
        if (hipError_t e = hipEventRecord(ev_in, a.stream); e != hipSuccess) return e;
        if (hipError_t e = hipStreamWaitEvent(ps, ev_in, 0); e != hipSuccess) return e;
    }
    // the scan's workgroups, spread one per CU, leave cus - scan_blocks CUs to the
    // preps that overlap it
    const unsigned side_grid = concurrent ? (unsigned)cus - scan_blocks : (unsigned)cus;
    const long long nwin = (maxc + WIN - 1) / WIN;
    auto windows = [&]() -> hipError_t {
        for (long long w = 0; w < nwin; ++w) {
            char *slot = recs + (size_t)(w & 1) * WIN * a.H * Rec::BYTES;
            const long long cw0 = w * WIN, cwn = std::min(WIN, maxc - cw0);
            if (concurrent && w >= 2)
                if (hipError_t e = hipStreamWaitEvent(ps, ev_scan[w & 1], 0); e != hipSuccess) return e;
            if (hipError_t e = prep(cw0, cwn, slot, w == 0 ? (unsigned)cus : side_grid, ps); e != hipSuccess)
                return e;
            if (concurrent) {
                if (hipError_t e = hipEventRecord(ev_prep[w & 1], ps); e != hipSuccess) return e;
                if (hipError_t e = hipStreamWaitEvent(a.stream, ev_prep[w & 1], 0); e != hipSuccess) return e;
            }
            if (hipError_t e = scan(cw0, cwn, slot, a.stream); e != hipSuccess) return e;
            if (concurrent)
                if (hipError_t e = hipEventRecord(ev_scan[w & 1], a.stream); e != hipSuccess) return e;
        }
        return hipSuccess;
    };
    const hipError_t err = windows();
    // whatever happened, later work on the caller's stream follows everything
    // queued on the side stream
    if (concurrent && hipEventRecord(ev_in, ps) == hipSuccess) (void)hipStreamWaitEvent(a.stream, ev_in, 0);
    return err;
}

template <typename TB>
hipError_t run_o(const PrefillArgs &a) {
    return a.out_dt == Dt::F32 ? run<TB, float>(a) : run<TB, bf16_t>(a);
}

}  // namespace

size_t prefill_mfma_workspace(int N, long long T_total, int H, int Dk, int Dv, int C_) {
    if (Dk == D && Dv == D && C_ == C) {
        const long long maxc = max_chunks(N, T_total, C);
        return ws_offs(N) + ws_meta(maxc) + ws_records(N, maxc, H) + ws_state(N, maxc, H);
    }
    return prefill_f32_workspace(N, T_total, H, Dk, Dv, C_);
}

hipError_t launch_prefill_mfma(const PrefillArgs &a) {
    // The MFMA kernels cover Dk = Dv = 128 with C = 64; other supported
    // shapes run the fp32-arithmetic kernels on the same bf16 inputs.
    if (a.Dk == D && a.C == C) return a.beta_dt == Dt::F32 ? run_o<float>(a) : run_o<bf16_t>(a);
    return launch_prefill_f32(a);
}

}  // namespace kda
