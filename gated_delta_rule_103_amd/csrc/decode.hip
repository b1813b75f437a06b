// decode.hip -- single-token KDA decode, state updated in place.
//
// One step of the recurrence in the Kimi K3 explainer's FlashKDA paragraph
// (decode follows the D_t / u_t form): M' = Diag(exp g) M, u = beta (v - M'^T k),
// M = M' + k u^T, o = M^T q. The explainer's cost model for it is about 7*D^2
// FLOPs and 8*D^2 bytes per head: the fp32 state is read once and written
// once, so the kernel is a stream over HBM.
//
// Layout of the work: the D value columns of one (sequence, head) chain are
// split over two workgroups (the reductions run over key rows, so column
// slices are independent). A thread owns one float4 column group of every
// (NT*4/W)-th row of its slice; each wavefront reads whole 256-byte row
// slices, and the state stays in registers between the read and the write.
// o is formed from the same pass: o = M'^T q + (q.k) u, so only one reduction
// round is needed. The state is read with ordinary loads and written with
// streaming (non-temporal) stores, which measured fastest.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

template <int D, int NT, int W, typename TI, typename TB, typename TO>
__global__ __launch_bounds__(NT) void decode_kernel(const TI *__restrict__ q, const TI *__restrict__ k,
                                                    const TI *__restrict__ v, const float *__restrict__ g,
                                                    const TB *__restrict__ beta, float *__restrict__ S,
                                                    TO *__restrict__ out, bool g_head, bool qk_norm, float norm_eps) {
    // NT threads cover W columns of one chain: the reductions over key rows stay
    // inside the workgroup, so the columns of a chain are split over D / W
    // workgroups.
    constexpr int CG = W / 4;         // float4 column groups per workgroup
    constexpr int RG = NT / CG;       // row groups (threads sharing a column group)
    constexpr int RPT = D / RG;       // rows per thread
    static_assert(CG * RG == NT && RG * RPT == D, "decode tiling");
    __shared__ float s_q[D], s_k[D], s_a[D], s_u[W];
    __shared__ float s_red[2][RG][W];
    __shared__ float s_qk, s_nq, s_nk;

    constexpr int SPLIT = D / W;
    const size_t chain = blockIdx.x / SPLIT;
    const int col0 = (blockIdx.x % SPLIT) * W;
    const int t = threadIdx.x;
    const int cg = t % CG, rg = t / CG;
    f32x4 *Sp = reinterpret_cast<f32x4 *>(S + chain * D * D + col0);

    f32x4 m[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) m[i] = Sp[(rg + RG * i) * (D / 4) + cg];

    for (int c = t; c < D; c += NT) {
        s_q[c] = io<TI>::load(q, chain * D + c);
        s_k[c] = io<TI>::load(k, chain * D + c);
        s_a[c] = expf(GateRow(g, g_head, chain, D).at(c));
    }
    __syncthreads();
    if (t < 64) {
        float x = 0.f, xq = 0.f, xk = 0.f;
        for (int c = t; c < D; c += 64) {
            x += s_q[c] * s_k[c];
            xq += s_q[c] * s_q[c];
            xk += s_k[c] * s_k[c];
        }
        x = warp_sum(x);
        xq = warp_sum(xq);
        xk = warp_sum(xk);
        if (t == 0) {
            // L2-normalised q and k: x / sqrt(sum x^2 + eps), applied as two scalars
            const float nq = qk_norm ? 1.f / sqrtf(xq + norm_eps) : 1.f;
            const float nk = qk_norm ? 1.f / sqrtf(xk + norm_eps) : 1.f;
            s_qk = x * nq * nk;
            s_nq = nq;
            s_nk = nk;
        }
    }
    float nq = 1.f, nk = 1.f;
    if (qk_norm) {                                     // uniform
        __syncthreads();
        nq = s_nq;
        nk = s_nk;
    }

    float4 pk = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rg + RG * i;
        const float a = s_a[r], kr = s_k[r] * nk, qr = s_q[r] * nq;
        m[i].x *= a; m[i].y *= a; m[i].z *= a; m[i].w *= a;
        pk.x += kr * m[i].x; pk.y += kr * m[i].y; pk.z += kr * m[i].z; pk.w += kr * m[i].w;
        pq.x += qr * m[i].x; pq.y += qr * m[i].y; pq.z += qr * m[i].z; pq.w += qr * m[i].w;
    }
    *reinterpret_cast<float4 *>(&s_red[0][rg][4 * cg]) = pk;
    *reinterpret_cast<float4 *>(&s_red[1][rg][4 * cg]) = pq;
    __syncthreads();
    if (t < W) {
        float p = 0.f, r = 0.f;
#pragma unroll
        for (int j = 0; j < RG; ++j) { p += s_red[0][j][t]; r += s_red[1][j][t]; }
        const float b = io<TB>::load(beta, chain);
        const float u = b * (io<TI>::load(v, chain * D + col0 + t) - p);
        s_u[t] = u;
        io<TO>::store(out, chain * D + col0 + t, r + s_qk * u);
    }
    __syncthreads();
    const float4 u4 = *reinterpret_cast<const float4 *>(&s_u[4 * cg]);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rg + RG * i;
        const float kr = s_k[r] * nk;
        f32x4 x = m[i];
        x.x += kr * u4.x; x.y += kr * u4.y; x.z += kr * u4.z; x.w += kr * u4.w;
        __builtin_nontemporal_store(x, &Sp[r * (D / 4) + cg]);
    }
}

// 128 threads per workgroup, each workgroup one half (64 value columns) of a
// chain's state: two workgroups per (sequence, head)
template <int D, typename TI, typename TB, typename TO>
hipError_t launch_t(const DecodeArgs &a) {
    constexpr int NT = 128, W = D / 2;
    const unsigned chains = static_cast<unsigned>(a.N) * static_cast<unsigned>(a.H);
    hipLaunchKernelGGL((decode_kernel<D, NT, W, TI, TB, TO>), dim3(chains * (D / W)), dim3(NT), 0, a.stream,
                       static_cast<const TI *>(a.q), static_cast<const TI *>(a.k), static_cast<const TI *>(a.v),
                       a.g, static_cast<const TB *>(a.beta), a.S, static_cast<TO *>(a.out), a.g_head, a.qk_norm,
                       a.norm_eps);
    return hipGetLastError();
}

template <int D, typename TI, typename TB>
hipError_t launch_o(const DecodeArgs &a) {
    return a.out_dt == Dt::F32 ? launch_t<D, TI, TB, float>(a) : launch_t<D, TI, TB, bf16_t>(a);
}

template <int D, typename TI>
hipError_t launch_b(const DecodeArgs &a) {
    return a.beta_dt == Dt::F32 ? launch_o<D, TI, float>(a) : launch_o<D, TI, bf16_t>(a);
}

template <int D>
hipError_t launch_i(const DecodeArgs &a) {
    return a.io == Dt::F32 ? launch_b<D, float>(a) : launch_b<D, bf16_t>(a);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a) {
    return a.Dk == 64 ? launch_i<64>(a) : launch_i<128>(a);
}

}  // namespace kda
