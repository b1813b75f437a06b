// output_gate.hip -- the output side of the KDA block: per-head RMS norm of
// the attention output o, scaled by a per-channel weight and by a sigmoid
// output gate.
//
// The Kimi K3 explainer (input/output paragraph of its KDA section) states
// that KDA's output is normalised per head and then controlled by an output
// forget gate, whose pre-activation comes from a projection (linear in K3,
// low-rank in Kimi Linear). The projection needs trained weights and stays
// outside this library; this kernel takes its result z as input. Per (row,
// head), over the Dv channels j:
//     out_j = o_j / sqrt(mean_j o_j^2 + eps) * w_j * sigmoid(z_j)
//
// The op reads o and z once and writes out once, so it is bound by HBM. A
// head row of Dv values is spread over Dv / 8 lanes, each holding eight
// consecutive channels (one 16-byte load of bf16, two of fp32); the sum of
// squares is reduced with cross-lane shuffles inside those lanes.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int OG_THREADS = 256;

template <typename T> struct vec8;
template <> struct vec8<float> {
    __device__ static f32x8 load(const float *p) {
        const f32x4 a = *reinterpret_cast<const f32x4 *>(p), b = *reinterpret_cast<const f32x4 *>(p + 4);
        return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    }
    __device__ static void store(float *p, f32x8 x) {
        *reinterpret_cast<f32x4 *>(p) = f32x4{x[0], x[1], x[2], x[3]};
        *reinterpret_cast<f32x4 *>(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
    }
};
template <> struct vec8<bf16_t> {
    __device__ static f32x8 load(const bf16_t *p) {
        const u32x4 u = *reinterpret_cast<const u32x4 *>(p);
        f32x8 x;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(u[i] << 16);
            x[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
        }
        return x;
    }
    __device__ static void store(bf16_t *p, f32x8 x) {
        u32x4 u;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            u[i] = static_cast<uint32_t>(f32_to_bf16(x[2 * i])) | (static_cast<uint32_t>(f32_to_bf16(x[2 * i + 1])) << 16);
        *reinterpret_cast<u32x4 *>(p) = u;
    }
};

// LR lanes per head row (LR = Dv / 8, a power of two dividing 64).
template <int DV, typename TO_IN, typename TG, typename TOUT>
__global__ __launch_bounds__(OG_THREADS) void output_gate_kernel(const TO_IN *__restrict__ o, const TG *__restrict__ z,
                                                                 const float *__restrict__ w, TOUT *out,
                                                                 long long rowheads, float eps) {
    constexpr int LR = DV / 8;
    constexpr int RPB = OG_THREADS / LR;             // head rows per workgroup
    const int t = threadIdx.x, part = t % LR;
    const long long rh = (long long)blockIdx.x * RPB + t / LR;
    const bool live = rh < rowheads;                 // uniform over the LR lanes of a row
    const size_t off = (size_t)(live ? rh : 0) * DV + 8 * part;
    f32x8 x = live ? vec8<TO_IN>::load(o + off) : f32x8{};
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ss += x[i] * x[i];
#pragma unroll
    for (int m = 1; m < LR; m <<= 1) ss += __shfl_xor(ss, m, 64);
    if (!live) return;
    const f32x8 g = vec8<TG>::load(z + off);
    f32x8 wv = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
    if (w) wv = vec8<float>::load(w + 8 * part);
    const float r = 1.f / sqrtf(ss * (1.f / DV) + eps);
    f32x8 y;
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = x[i] * r * wv[i] / (1.f + __expf(-g[i]));
    vec8<TOUT>::store(out + off, y);
}

template <int DV, typename TI, typename TG, typename TO>
hipError_t launch_t(const OutputGateArgs &a) {
    constexpr int RPB = OG_THREADS / (DV / 8);
    const long long rowheads = (long long)a.rows * a.H;
    if (rowheads == 0) return hipSuccess;
    const unsigned grid = static_cast<unsigned>((rowheads + RPB - 1) / RPB);
    hipLaunchKernelGGL((output_gate_kernel<DV, TI, TG, TO>), dim3(grid), dim3(OG_THREADS), 0, a.stream,
                       static_cast<const TI *>(a.o), static_cast<const TG *>(a.gate), a.weight,
                       static_cast<TO *>(a.out), rowheads, a.eps);
    return hipGetLastError();
}

template <int DV, typename TI, typename TG>
hipError_t launch_o(const OutputGateArgs &a) {
    return a.out_dt == Dt::F32 ? launch_t<DV, TI, TG, float>(a) : launch_t<DV, TI, TG, bf16_t>(a);
}

template <int DV, typename TI>
hipError_t launch_g(const OutputGateArgs &a) {
    return a.gate_dt == Dt::F32 ? launch_o<DV, TI, float>(a) : launch_o<DV, TI, bf16_t>(a);
}

template <int DV>
hipError_t launch_i(const OutputGateArgs &a) {
    return a.o_dt == Dt::F32 ? launch_g<DV, float>(a) : launch_g<DV, bf16_t>(a);
}

}  // namespace

hipError_t launch_output_gate(const OutputGateArgs &a) {
    return a.Dv == 64 ? launch_i<64>(a) : launch_i<128>(a);
}

}  // namespace kda
