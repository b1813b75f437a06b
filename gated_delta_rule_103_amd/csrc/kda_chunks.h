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

}  // namespace kda
