// kda_device.h -- small device helpers shared by the libkda HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// bf16 is carried as its raw 16 bits; conversions are explicit.
typedef uint16_t bf16_t;
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round-to-nearest-even float -> bf16 (NaN kept quiet).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<bf16_t>(u >> 16);
}

template <typename T> struct io;
template <> struct io<float> {
    __device__ __forceinline__ static float load(const float *p, size_t i) { return p[i]; }
    __device__ __forceinline__ static void store(float *p, size_t i, float x) { p[i] = x; }
};
template <> struct io<bf16_t> {
    __device__ __forceinline__ static float load(const bf16_t *p, size_t i) { return bf16_to_f32(p[i]); }
    __device__ __forceinline__ static void store(bf16_t *p, size_t i, float x) { p[i] = f32_to_bf16(x); }
};

// Raw buffer access: a wave-uniform base and byte range held in scalar
// registers, plus a 32-bit per-lane offset. A load past the range reads 0 and
// a store past it is dropped; an empty range (base may be null) never touches
// memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, 0x00020000);
}
__device__ __forceinline__ float buf_ld_f32(__amdgpu_buffer_rsrc_t r, int voff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0));
}

// Log-decay gate of one chain (sequence or token row, head): per key channel,
// g[row][h][0..D) (KDA); per head, g[row][h] broadcast over the channels (Gated
// DeltaNet); or none, g == nullptr (DeltaNet, alpha = 1). row_h = row * H + h.
struct GateRow {
    __amdgpu_buffer_rsrc_t r;
    bool per_head;
    __device__ GateRow(const float *g, bool head, size_t row_h, int D)
        : r(buf_rsrc(g ? g + (head ? row_h : row_h * D) : nullptr, g ? (head ? 4 : D * 4) : 0)), per_head(head) {}
    __device__ float at(int c) const { return buf_ld_f32(r, per_head ? 0 : c * 4); }
};

__device__ __forceinline__ float warp_sum(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

}  // namespace kda
