// kda_chunks.h -- how sequences are cut into chunks (device side).
//
// Chunks of C tokens restart at every sequence start and the last chunk of a
// sequence may be short. Dense input (no cu_seqlens) is N sequences of T
// tokens; packed input uses cu_seqlens and a chunk-offset table that the
// plan kernel builds on the device (chunk_off[n] = chunks in sequences < n,
// chunk_off[N] = total).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

struct SeqView {
    const int32_t *cu;        // nullptr => dense
    const int32_t *chunk_off; // valid when cu != nullptr
    int N, T, C;
    __device__ int dense_chunks() const { return (T + C - 1) / C; }
    __device__ int total_chunks() const { return cu ? chunk_off[N] : N * dense_chunks(); }
    __device__ int seq_start(int n) const { return cu ? cu[n] : n * T; }
    __device__ int seq_end(int n) const { return cu ? cu[n + 1] : (n + 1) * T; }
    __device__ int first_chunk(int n) const { return cu ? chunk_off[n] : n * dense_chunks(); }
    // sequence holding global chunk ci (0 <= ci < total_chunks): the largest n
    // with chunk_off[n] <= ci, which skips empty sequences
    __device__ int seq_of_chunk(int ci) const {
        if (!cu) return ci / dense_chunks();
        int lo = 0, hi = N - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (chunk_off[mid] <= ci) lo = mid; else hi = mid - 1;
        }
        return lo;
    }
};

// Optional state snapshots for prefix caching: the state of a chain after the
// first k * every chunks of its sequence (k = 1, 2, ..., up to max) goes to
// base[((n * H + h) * max + k - 1) * Dk * Dv + ...]. Only boundaries inside the
// sequence (k * every * C <= length) are written.
struct SnapView {
    float *base;    // [N][H][max][Dv][Dk] fp32, or nullptr
    int every;      // chunks between snapshots (> 0 when base is set)
    int max;        // snapshots per sequence
    __device__ float *slot(int n, int h, int H, int chunks_done, int len, int C, int DD) const {
        if (!base || chunks_done % every != 0 || chunks_done * C > len) return nullptr;
        const int k = chunks_done / every;
        if (k > max) return nullptr;
        return base + (((size_t)n * H + h) * max + (k - 1)) * DD;
    }
};

}  // namespace kda
