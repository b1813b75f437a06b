// prefill_f32.hip -- chunked KDA prefill with fp32 arithmetic throughout.
//
// Follows the chunk unrolling of the Kimi K3 explainer's FlashKDA paragraph:
// a "prep" kernel handles every (chunk, head) in parallel and a "scan"
// kernel carries the state across the chunks of each (sequence, head,
// value-column tile). With a = in-chunk cumulative log-decay:
//   Qd    = q * exp(a)                 (Q_decay)
//   Kr    = k * exp(a_last - a)        (K_restore = D_{j:t+1} k_t)
//   gamma = exp(a_last)
//   Mqk[t,s] = sum_c q_t k_s exp(a_t - a_s), s <= t   (causal M_qk)
//   L[t,s]   = beta_t sum_c k_t k_s exp(a_t - a_s), s < t
//   INV = (I + L)^{-1}                 (UT transform, forward substitution)
//   Ut = INV Diag(beta) V,  W = INV Diag(beta) (k * exp(a))
// scan, per chunk: U = Ut - W M;  O = Qd M + Mqk U;  M = Diag(gamma) M + Kr^T U.
// Every exponent is <= 0, so nothing overflows (the page's K_inv = k*exp(-a)
// factorisation is avoided for that reason).
//
// This path is exact to fp32 rounding and simple; it is the io_dtype=f32
// path of the library. The bf16 path (prefill_mfma.hip) is the fast one.
#include "kda_chunks.h"
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

// chunk_off[n] = number of chunks in sequences 0..n-1 (chunks restart at
// each sequence start; a sequence of length len has ceil(len/C) chunks).
__global__ __launch_bounds__(256) void plan_kernel(const int32_t *__restrict__ cu, int N, int C,
                                                   int32_t *__restrict__ chunk_off) {
    __shared__ int32_t part[256];
    const int t = threadIdx.x;
    const int per = (N + 255) / 256;
    const int lo = min(N, t * per), hi = min(N, lo + per);
    int32_t s = 0;
    for (int n = lo; n < hi; ++n) s += (cu[n + 1] - cu[n] + C - 1) / C;
    part[t] = s;
    __syncthreads();
    if (t == 0) {
        int32_t run = 0;
        for (int i = 0; i < 256; ++i) { const int32_t x = part[i]; part[i] = run; run += x; }
        chunk_off[N] = run;
    }
    __syncthreads();
    int32_t run = part[t];
    for (int n = lo; n < hi; ++n) { chunk_off[n] = run; run += (cu[n + 1] - cu[n] + C - 1) / C; }
}


// Per (chunk, head) record of fp32 operands in the workspace.
template <int C, int D>
struct Rec {
    static constexpr size_t QD = 0, KR = QD + C * D, W = KR + C * D, UT = W + C * D, MQK = UT + C * D,
                            GAM = MQK + C * C, SIZE = GAM + D;
};

template <int C, int D, typename TI, typename TB>
__global__ __launch_bounds__(256) void prep_kernel(const TI *__restrict__ q, const TI *__restrict__ k,
                                                   const TI *__restrict__ v, const float *__restrict__ g,
                                                   const TB *__restrict__ beta, SeqView sv, int H,
                                                   float *__restrict__ rec_base, bool g_head, bool qk_norm,
                                                   float norm_eps) {
    using R = Rec<C, D>;
    __shared__ float s_a[C][D];
    __shared__ float s_L[C][C];
    __shared__ float s_inv[C][C];
    __shared__ float s_beta[C];
    __shared__ float s_rq[C], s_rk[C];   // 1 / ||q_t||, 1 / ||k_t|| when q and k are L2-normalised, else 1

    const int ci = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
    if (ci >= sv.total_chunks()) return;
    const int n = sv.seq_of_chunk(ci);
    const int s0 = sv.seq_start(n) + (ci - sv.first_chunk(n)) * C;
    const int Lc = min(C, sv.seq_end(n) - s0);
    float *rec = rec_base + ((size_t)ci * H + h) * R::SIZE;
    auto row = [&](int tau) -> size_t { return ((size_t)(s0 + tau) * H + h) * D; };

    // cumulative log-decay over the chunk, one thread per key channel; rows
    // past the end of the sequence repeat the last value (no decay)
    if (t < D) {
        float acc = 0.f;
        for (int tau = 0; tau < C; ++tau) {
            if (tau < Lc) acc += GateRow(g, g_head, (size_t)(s0 + tau) * H + h, D).at(t);
            s_a[tau][t] = acc;
        }
    }
    if (t < C) s_beta[t] = t < Lc ? io<TB>::load(beta, (size_t)(s0 + t) * H + h) : 0.f;
    if (t < C) {
        float sq = 0.f, sk = 0.f;
        if (qk_norm && t < Lc)
            for (int c = 0; c < D; ++c) {
                const float a = io<TI>::load(q, row(t) + c), b = io<TI>::load(k, row(t) + c);
                sq += a * a;
                sk += b * b;
            }
        s_rq[t] = qk_norm && t < Lc ? 1.f / sqrtf(sq + norm_eps) : 1.f;
        s_rk[t] = qk_norm && t < Lc ? 1.f / sqrtf(sk + norm_eps) : 1.f;
    }
    __syncthreads();

    // Mqk (to the record) and L (to LDS), exact per-element exponentials
    for (int p = t; p < C * C; p += 256) {
        const int tau = p / C, sig = p % C;
        float mq = 0.f, lk = 0.f;
        if (sig <= tau && tau < Lc) {
            for (int c = 0; c < D; ++c) {
                const float e = expf(s_a[tau][c] - s_a[sig][c]);
                const float ks = io<TI>::load(k, row(sig) + c);
                mq += io<TI>::load(q, row(tau) + c) * ks * e;
                lk += io<TI>::load(k, row(tau) + c) * ks * e;
            }
        }
        mq *= s_rq[tau] * s_rk[sig];
        lk *= s_rk[tau] * s_rk[sig];
        rec[R::MQK + p] = mq;
        s_L[tau][sig] = sig < tau ? s_beta[tau] * lk : 0.f;
    }
    __syncthreads();

    // INV = (I + L)^{-1}, unit lower triangular, row by row
    for (int tau = 0; tau < C; ++tau) {
        if (t < C) {
            float x = (t == tau) ? 1.f : 0.f;
            if (t < tau) {
                for (int sig = t; sig < tau; ++sig) x -= s_L[tau][sig] * s_inv[sig][t];
            }
            s_inv[tau][t] = x;
        }
        __syncthreads();
    }

    // Qd, Kr, gamma
    for (int p = t; p < C * D; p += 256) {
        const int tau = p / D, c = p % D;
        float qd = 0.f, kr = 0.f;
        if (tau < Lc) {
            qd = io<TI>::load(q, row(tau) + c) * s_rq[tau] * expf(s_a[tau][c]);
            kr = io<TI>::load(k, row(tau) + c) * s_rk[tau] * expf(s_a[C - 1][c] - s_a[tau][c]);
        }
        rec[R::QD + p] = qd;
        rec[R::KR + p] = kr;
    }
    if (t < D) rec[R::GAM + t] = expf(s_a[C - 1][t]);

    // W = INV Diag(beta) Kdec and Ut = INV Diag(beta) V
    for (int p = t; p < C * D; p += 256) {
        const int tau = p / D, c = p % D;
        float w = 0.f, ut = 0.f;
        if (tau < Lc) {
            for (int sig = 0; sig <= tau; ++sig) {
                const float ib = s_inv[tau][sig] * s_beta[sig];
                w += ib * io<TI>::load(k, row(sig) + c) * s_rk[sig] * expf(s_a[sig][c]);
                ut += ib * io<TI>::load(v, row(sig) + c);
            }
        }
        rec[R::W + p] = w;
        rec[R::UT + p] = ut;
    }
}

template <int C, int D, int TV, typename TO>
__global__ __launch_bounds__(256) void scan_kernel(const float *__restrict__ rec_base, const float *__restrict__ S0,
                                                   TO *__restrict__ out, float *__restrict__ S_out, SeqView sv,
                                                   int H, SnapView snap) {
    using R = Rec<C, D>;
    __shared__ float s_M[D][TV];
    __shared__ float s_U[C][TV];
    const int n = blockIdx.x, h = blockIdx.y, j0 = blockIdx.z * TV, t = threadIdx.x;
    const size_t st = ((size_t)n * H + h) * D * D;

    // the state S [Dv][Dk] in memory: row j0 + j, key channel c
    for (int p = t; p < D * TV; p += 256) {
        const int j = p / D, c = p % D;
        s_M[c][j] = S0 ? S0[st + (size_t)(j0 + j) * D + c] : 0.f;
    }
    __syncthreads();

    const int start = sv.seq_start(n), len = sv.seq_end(n) - start;
    const int nch = (len + C - 1) / C, c0 = sv.first_chunk(n);
    for (int j = 0; j < nch; ++j) {
        const float *rec = rec_base + ((size_t)(c0 + j) * H + h) * R::SIZE;
        const int Lc = min(C, len - j * C);
        // U = Ut - W M
        for (int p = t; p < C * TV; p += 256) {
            const int tau = p / TV, jj = p % TV;
            float u = rec[R::UT + tau * D + j0 + jj];
            for (int c = 0; c < D; ++c) u -= rec[R::W + tau * D + c] * s_M[c][jj];
            s_U[tau][jj] = u;
        }
        __syncthreads();
        // O = Qd M + Mqk U
        for (int p = t; p < C * TV; p += 256) {
            const int tau = p / TV, jj = p % TV;
            if (tau < Lc) {
                float o = 0.f;
                for (int c = 0; c < D; ++c) o += rec[R::QD + tau * D + c] * s_M[c][jj];
                for (int sig = 0; sig <= tau; ++sig) o += rec[R::MQK + tau * C + sig] * s_U[sig][jj];
                io<TO>::store(out, ((size_t)(start + j * C + tau) * H + h) * D + j0 + jj, o);
            }
        }
        __syncthreads();
        // M = Diag(gamma) M + Kr^T U
        for (int p = t; p < D * TV; p += 256) {
            const int c = p / TV, jj = p % TV;
            float m = rec[R::GAM + c] * s_M[c][jj];
            for (int tau = 0; tau < C; ++tau) m += rec[R::KR + tau * D + c] * s_U[tau][jj];
            s_M[c][jj] = m;
        }
        __syncthreads();
        if (float *sp = snap.slot(n, h, H, j + 1, len, C, D * D)) {     // uniform across the workgroup
            for (int p = t; p < D * TV; p += 256) {
                const int jj = p / D, c = p % D;
                sp[(size_t)(j0 + jj) * D + c] = s_M[c][jj];
            }
        }
    }
    if (S_out) {
        for (int p = t; p < D * TV; p += 256) {
            const int j = p / D, c = p % D;
            S_out[st + (size_t)(j0 + j) * D + c] = s_M[c][j];
        }
    }
}

template <int C, int D, typename TI, typename TB, typename TO>
hipError_t run(const PrefillArgs &a) {
    constexpr int TV = 32;
    using R = Rec<C, D>;
    const long long T_total = (long long)a.B * a.T;
    const long long maxc = max_chunks(a.N, T_total, C);
    char *ws = static_cast<char *>(a.ws);
    int32_t *chunk_off = reinterpret_cast<int32_t *>(ws);
    float *recs = reinterpret_cast<float *>(ws + ((sizeof(int32_t) * (a.N + 1) + 255) / 256) * 256);
    SeqView sv{a.cu_seqlens, chunk_off, a.N, a.T, C};
    if (a.cu_seqlens) {
        const hipError_t e = launch_chunk_plan(a.cu_seqlens, a.N, C, chunk_off, a.stream);
        if (e != hipSuccess) return e;
    }
    if (maxc > 0) {
        hipLaunchKernelGGL((prep_kernel<C, D, TI, TB>), dim3((unsigned)maxc, a.H), dim3(256), 0, a.stream,
                           static_cast<const TI *>(a.q), static_cast<const TI *>(a.k),
                           static_cast<const TI *>(a.v), a.g, static_cast<const TB *>(a.beta), sv, a.H, recs, a.g_head, a.qk_norm,
                           a.norm_eps);
        if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    }
    (void)sizeof(R);
    hipLaunchKernelGGL((scan_kernel<C, D, TV, TO>), dim3(a.N, a.H, D / TV), dim3(256), 0, a.stream, recs, a.S0,
                       static_cast<TO *>(a.out), a.S_out, sv, a.H, SnapView{a.snaps, a.snap_every, a.max_snaps});
    return hipGetLastError();
}

template <int C, int D>
hipError_t run_types(const PrefillArgs &a) {
    if (a.io == Dt::F32) return run<C, D, float, float, float>(a);
    // bf16 inputs through the fp32-arithmetic kernels
    if (a.beta_dt == Dt::F32)
        return a.out_dt == Dt::F32 ? run<C, D, bf16_t, float, float>(a) : run<C, D, bf16_t, float, bf16_t>(a);
    return a.out_dt == Dt::F32 ? run<C, D, bf16_t, bf16_t, float>(a) : run<C, D, bf16_t, bf16_t, bf16_t>(a);
}

template <int C>
hipError_t run_d(const PrefillArgs &a) {
    return a.Dk == 64 ? run_types<C, 64>(a) : run_types<C, 128>(a);
}

}  // namespace

hipError_t launch_chunk_plan(const int32_t *cu, int N, int C, int32_t *chunk_off, hipStream_t stream) {
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, stream, cu, N, C, chunk_off);
    return hipGetLastError();
}

size_t prefill_f32_workspace(int N, long long T_total, int H, int Dk, int Dv, int C) {
    (void)Dv;
    const size_t head = ((sizeof(int32_t) * (size_t)(N + 1) + 255) / 256) * 256;
    const size_t rec = (size_t)(4 * C * Dk + C * C + Dk) * sizeof(float);
    return head + (size_t)max_chunks(N, T_total, C) * H * rec;
}

hipError_t launch_prefill_f32(const PrefillArgs &a) {
    switch (a.C) {
        case 16: return run_d<16>(a);
        case 32: return run_d<32>(a);
        default: return run_d<64>(a);
    }
}

}  // namespace kda
