// kda_launch.h -- host-side launchers implemented in the .hip files and
// called by the argument-checking layer in kda_abi.cpp. Every launcher
// assumes its arguments were already validated and returns a hipError_t.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

enum class Dt : int { F32 = 0, BF16 = 1 };

struct PrefillArgs {
    const void *q, *k, *v;
    const float *g;
    const void *beta;
    const float *S0;
    void *out;
    float *S_out;
    const int32_t *cu_seqlens;  // device, or nullptr (dense)
    int N, B, T, H, Dk, Dv, C;
    Dt io, beta_dt, out_dt;
    void *ws;
    size_t ws_bytes;
    hipStream_t stream;
    // optional state snapshots: [N][H][max_snaps][Dv][Dk] fp32, one every
    // snap_every chunks of each sequence (nullptr: none)
    float *snaps = nullptr;
    int snap_every = 0, max_snaps = 0;
    // gate layout: false: g [T_total][H][Dk], one log-decay per key channel (KDA);
    // true: g [T_total][H], one per head broadcast over the channels (Gated
    // DeltaNet), and g == nullptr means no decay (DeltaNet)
    bool g_head = false;
    // L2-normalise q and k over Dk inside the kernels: x / sqrt(sum x^2 + norm_eps)
    bool qk_norm = false;
    float norm_eps = 0.f;
    // run everything on `stream` (no side stream or events created), as for
    // callers that must not create runtime objects (the no-allocation entry)
    bool in_order = false;
};

struct DecodeArgs {
    const void *q, *k, *v;
    const float *g;
    const void *beta;
    float *S;
    void *out;
    int N, H, Dk, Dv;
    Dt io, beta_dt, out_dt;
    hipStream_t stream;
    bool g_head = false;        // as in PrefillArgs: g [N][H] or nullptr
    bool qk_norm = false;       // as in PrefillArgs
    float norm_eps = 0.f;
};

struct OutputGateArgs {
    const void *o, *gate;
    const float *weight;        // [Dv] or nullptr (ones)
    void *out;
    int rows, H, Dv;
    float eps;
    Dt o_dt, gate_dt, out_dt;
    hipStream_t stream;
};

// Upper bound on the number of chunks of all sequences (each sequence adds at
// most one partial chunk).
inline long long max_chunks(int N, long long T_total, int C) {
    return (T_total + C - 1) / C + N;
}

// Device-side chunk table of packed sequences: chunk_off[n] for n <= N.
hipError_t launch_chunk_plan(const int32_t *cu, int N, int C, int32_t *chunk_off, hipStream_t stream);

// fp32-arithmetic chunked prefill (plan + prep + scan kernels).
size_t prefill_f32_workspace(int N, long long T_total, int H, int Dk, int Dv, int C);
hipError_t launch_prefill_f32(const PrefillArgs &a);

// MFMA chunked prefill for bf16 inputs (fp16 and fp32 MFMA, fp32 accumulation).
size_t prefill_mfma_workspace(int N, long long T_total, int H, int Dk, int Dv, int C);
hipError_t launch_prefill_mfma(const PrefillArgs &a);

// kda_prefill_noalloc: the size of its fixed device workspace, and the address
// of that workspace on the current device (looked up once per device).
constexpr size_t kNoAllocScratchBytes = size_t(128) << 20;
hipError_t noalloc_scratch(void **ptr);

// single-token decode.
hipError_t launch_decode(const DecodeArgs &a);

// per-head RMS norm and sigmoid output gate of o.
hipError_t launch_output_gate(const OutputGateArgs &a);

}  // namespace kda
