// decode.hip -- single-token KDA decode, state updated in place.
//
// One step of the recurrence in the Kimi K3 explainer's FlashKDA paragraph
// (decode follows the D_t / u_t form), on the state S [Dv][Dk] (row c = value
// channel, column = key channel):
//     S' = S Diag(exp g),  u = beta (v - S' k),  S = S' + u k^T,  o = S q.
// The explainer's cost model for it is about 7*D^2 FLOPs and 8*D^2 bytes per
// head: the fp32 state is read once and written once, so the kernel is a
// stream over HBM.
//
// Layout of the work: every quantity of a row reduces over that row's key
// channels, and a row is D*4 contiguous bytes. D/4 consecutive lanes own a
// row (four key channels, one float4, each), so both reductions (S'k and S'q)
// are sums over those lanes by cross-lane shuffles: no LDS, no barrier. A
// thread holds four rows, a workgroup 4 x (threads / (D/4)) rows, and each
// wavefront instruction reads or writes whole adjacent rows (1 KB at D = 128).
// o = S'q + (q.k) u is formed from the same pass. The state is read and
// written with the non-temporal hint (each byte is touched once).
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

// sum over each group of W consecutive lanes (W a power of two, at most 64)
template <int W>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
    for (int o = 1; o < W; o <<= 1) x += __shfl_xor(x, o, W);
    return x;
}
__device__ __forceinline__ float dot4(f32x4 a, f32x4 b) { return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w; }

template <int D, int NT, typename TI, typename TB, typename TO>
__global__ __launch_bounds__(NT) void decode_kernel(const TI *__restrict__ q, const TI *__restrict__ k,
                                                    const TI *__restrict__ v, const float *__restrict__ g,
                                                    const TB *__restrict__ beta, float *__restrict__ S,
                                                    TO *__restrict__ out, bool g_head, bool qk_norm, float norm_eps) {
    constexpr int LPR = D / 4;            // lanes per state row
    constexpr int SLOTS = NT / LPR;       // rows a workgroup takes per pass
    constexpr int ROWS = 4 * SLOTS;       // rows per workgroup
    constexpr int SPLIT = D / ROWS;       // workgroups per chain
    static_assert(NT % LPR == 0 && D % ROWS == 0 && (LPR & (LPR - 1)) == 0 && 64 % LPR == 0, "decode tiling");
    const size_t chain = blockIdx.x / SPLIT;
    const int r0 = (blockIdx.x % SPLIT) * ROWS, t = threadIdx.x, kq = t % LPR, slot = t / LPR;
    f32x4 *Sp = reinterpret_cast<f32x4 *>(S + chain * D * D);

    f32x4 s[4];
    float vr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = r0 + slot + SLOTS * i;
        s[i] = __builtin_nontemporal_load(&Sp[row * (D / 4) + kq]);
        vr[i] = io<TI>::load(v, chain * D + row);
    }
    const float b = io<TB>::load(beta, chain);
    // this lane's key channels 4kq .. 4kq + 3
    const GateRow gate(g, g_head, chain, D);
    f32x4 q4, k4, a4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        q4[e] = io<TI>::load(q, chain * D + 4 * kq + e);
        k4[e] = io<TI>::load(k, chain * D + 4 * kq + e);
        a4[e] = expf(gate.at(4 * kq + e));
    }
    if (qk_norm) {                                       // uniform
        // L2-normalised q and k: x / sqrt(sum x^2 + eps)
        q4 *= 1.f / sqrtf(group_sum<LPR>(dot4(q4, q4)) + norm_eps);
        k4 *= 1.f / sqrtf(group_sum<LPR>(dot4(k4, k4)) + norm_eps);
    }
    const float qk = group_sum<LPR>(dot4(q4, k4));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = r0 + slot + SLOTS * i;
        const f32x4 x = s[i] * a4;                       // S' = S Diag(exp g)
        const float pk = group_sum<LPR>(dot4(x, k4));    // (S' k)_row
        const float pq = group_sum<LPR>(dot4(x, q4));    // (S' q)_row
        const float u = b * (vr[i] - pk);
        __builtin_nontemporal_store(x + k4 * u, &Sp[row * (D / 4) + kq]);
        if (kq == 0) io<TO>::store(out, chain * D + row, pq + qk * u);
    }
}

// D = 128: 512 threads, two workgroups of 64 rows per (sequence, head);
// D = 64: 256 threads, one workgroup of 64 rows
template <int D, typename TI, typename TB, typename TO>
hipError_t launch_t(const DecodeArgs &a) {
    constexpr int NT = D == 128 ? 512 : 256, SPLIT = D / (4 * NT / (D / 4));
    const unsigned chains = static_cast<unsigned>(a.N) * static_cast<unsigned>(a.H);
    hipLaunchKernelGGL((decode_kernel<D, NT, TI, TB, TO>), dim3(chains * SPLIT), dim3(NT), 0, a.stream,
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
