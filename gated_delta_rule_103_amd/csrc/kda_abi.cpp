// kda_abi.cpp -- the extern "C" boundary of libkda: argument checks,
// workspace sizing and kernel selection. Declarations and the contract of
// every entry point are in include/kda.h.
#include "../../include/kda.h"

#include <climits>

#include "kda_launch.h"

using kda::Dt;

namespace {

bool dtype_ok(int d) { return d == KDA_F32 || d == KDA_BF16; }

bool head_dims_supported(int Dk, int Dv) { return Dk == Dv && (Dk == 64 || Dk == 128); }

bool chunk_supported(int C) { return C == 16 || C == 32 || C == 64; }

// Which prefill kernels serve this dtype combination.
bool use_mfma(kda_dtype io) { return io == KDA_BF16; }

size_t workspace_for(int N, long long T_total, int H, int Dk, int Dv, int C, kda_dtype io) {
    return use_mfma(io) ? kda::prefill_mfma_workspace(N, T_total, H, Dk, Dv, C)
                        : kda::prefill_f32_workspace(N, T_total, H, Dk, Dv, C);
}

// options: NULL = defaults; a bad gate or a norm without eps > 0 is an argument error
bool options_ok(const kda_options *o) {
    if (!o) return true;
    if (o->gate != KDA_GATE_CHANNEL && o->gate != KDA_GATE_HEAD) return false;
    if (o->qk_l2norm && !(o->l2norm_eps > 0.f)) return false;      // also rejects NaN
    return true;
}

}  // namespace

extern "C" {

int kda_version(void) { return (0 << 16) | (1 << 8) | 0; }

const char *kda_status_string(int status) {
    switch (status) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_INVALID_ARG: return "KDA_ERR_INVALID_ARG";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
        case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE";
        case KDA_ERR_HIP: return "KDA_ERR_HIP";
        default: return "KDA_UNKNOWN_STATUS";
    }
}

size_t kda_prefill_workspace_size(int N, int T_total, int H, int Dk, int Dv, int C, kda_dtype io_dtype) {
    if (N < 1 || T_total < 0 || H < 1 || !dtype_ok(io_dtype)) return 0;
    if (!head_dims_supported(Dk, Dv) || !chunk_supported(C)) return 0;
    return workspace_for(N, T_total, H, Dk, Dv, C, io_dtype);
}

}  // extern "C"

namespace {

int prefill_impl(const void *q, const void *k, const void *v, const float *g, const void *beta,
                 const float *S0, void *out, float *S_out, const int32_t *cu_seqlens, int N, int B, int T,
                 int H, int Dk, int Dv, int C, kda_dtype io_dtype, kda_dtype beta_dtype, kda_dtype out_dtype,
                 int snapshot_every, int max_snapshots, float *snapshots, void *workspace,
                 size_t workspace_bytes, void *stream, bool g_head = false, bool qk_norm = false,
                 float norm_eps = 0.f, bool noalloc = false) {
    // a per-head gate may be absent (no decay); a per-channel gate may not
    if (!q || !k || !v || (!g && !g_head) || !beta || !out) return KDA_ERR_INVALID_ARG;
    if (N < 1 || B < 1 || T < 0 || H < 1 || Dk < 1 || Dv < 1 || C < 1) return KDA_ERR_INVALID_ARG;
    if (!dtype_ok(io_dtype) || !dtype_ok(beta_dtype) || !dtype_ok(out_dtype)) return KDA_ERR_INVALID_ARG;
    if (cu_seqlens ? B != 1 : N != B) return KDA_ERR_INVALID_ARG;
    const long long T_total = (long long)B * T;
    if (T_total > INT_MAX / 2 || (long long)N * H > INT_MAX / 2) return KDA_ERR_INVALID_ARG;
    // q, k, v and a per-channel g are read with 16-byte vector loads; out is
    // written with vector stores of up to 16 bytes
    if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v) |
         reinterpret_cast<uintptr_t>(out) | (g_head ? 0u : reinterpret_cast<uintptr_t>(g))) & 15u)
        return KDA_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(g) & 3u) return KDA_ERR_INVALID_ARG;
    if (snapshots) {
        if (snapshot_every < 1 || max_snapshots < 1) return KDA_ERR_INVALID_ARG;
        if ((long long)N * H * max_snapshots > INT_MAX / 2) return KDA_ERR_INVALID_ARG;
    }
    if (!head_dims_supported(Dk, Dv) || !chunk_supported(C)) return KDA_ERR_UNSUPPORTED;
    if ((long long)H * Dv * C * 4 > INT_MAX) return KDA_ERR_UNSUPPORTED;
    if (io_dtype == KDA_F32 && (beta_dtype != KDA_F32 || out_dtype != KDA_F32)) return KDA_ERR_UNSUPPORTED;
    if (snapshots && snapshot_every % C != 0) return KDA_ERR_UNSUPPORTED;
    const size_t need = workspace_for(N, T_total, H, Dk, Dv, C, io_dtype);
    if (noalloc) {
        // the library's fixed per-device array serves as the workspace
        if (need > kda::kNoAllocScratchBytes) return KDA_ERR_WORKSPACE;
        if (kda::noalloc_scratch(&workspace) != hipSuccess) return KDA_ERR_HIP;
        workspace_bytes = kda::kNoAllocScratchBytes;
    }
    if (need > 0 && (!workspace || workspace_bytes < need)) return KDA_ERR_WORKSPACE;
    if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 255u)) return KDA_ERR_WORKSPACE;

    kda::PrefillArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.S0 = S0; a.out = out; a.S_out = S_out;
    a.cu_seqlens = cu_seqlens; a.N = N; a.B = B; a.T = T; a.H = H; a.Dk = Dk; a.Dv = Dv; a.C = C;
    a.io = static_cast<Dt>(io_dtype); a.beta_dt = static_cast<Dt>(beta_dtype);
    a.out_dt = static_cast<Dt>(out_dtype);
    a.ws = workspace; a.ws_bytes = workspace_bytes;
    a.stream = static_cast<hipStream_t>(stream);
    a.g_head = g_head;
    a.qk_norm = qk_norm;
    a.norm_eps = norm_eps;
    a.in_order = noalloc;
    if (snapshots) {
        a.snaps = snapshots;
        a.snap_every = snapshot_every / C;
        a.max_snaps = max_snapshots;
    }
    const hipError_t e = use_mfma(io_dtype) ? kda::launch_prefill_mfma(a) : kda::launch_prefill_f32(a);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // namespace

extern "C" {

int kda_prefill(const void *q, const void *k, const void *v, const float *g, const void *beta,
                const float *S0, void *out, float *S_out, const int32_t *cu_seqlens, int N, int B,
                int T, int H, int Dk, int Dv, int C, kda_dtype io_dtype, kda_dtype beta_dtype,
                kda_dtype out_dtype, void *workspace, size_t workspace_bytes, void *stream) {
    return prefill_impl(q, k, v, g, beta, S0, out, S_out, cu_seqlens, N, B, T, H, Dk, Dv, C, io_dtype,
                        beta_dtype, out_dtype, 0, 0, nullptr, workspace, workspace_bytes, stream);
}

int kda_prefill_noalloc(const void *q, const void *k, const void *v, const float *g, const void *beta,
                        const float *S0, void *out, float *S_out, const int32_t *cu_seqlens, int N, int B,
                        int T, int H, int Dk, int Dv, int C, kda_dtype io_dtype, kda_dtype beta_dtype,
                        kda_dtype out_dtype, void *stream) {
    // every argument is checked first, then the workspace size against the
    // fixed array, and only then is the array's address on the current device
    // taken: no allocation
    return prefill_impl(q, k, v, g, beta, S0, out, S_out, cu_seqlens, N, B, T, H, Dk, Dv, C, io_dtype,
                        beta_dtype, out_dtype, 0, 0, nullptr, nullptr, 0, stream, false, false, 0.f, true);
}

int kda_prefill_snapshots(const void *q, const void *k, const void *v, const float *g, const void *beta,
                          const float *S0, void *out, float *S_out, const int32_t *cu_seqlens, int N, int B,
                          int T, int H, int Dk, int Dv, int C, kda_dtype io_dtype, kda_dtype beta_dtype,
                          kda_dtype out_dtype, int snapshot_every, int max_snapshots, float *snapshots,
                          void *workspace, size_t workspace_bytes, void *stream) {
    if (!snapshots) return KDA_ERR_INVALID_ARG;
    return prefill_impl(q, k, v, g, beta, S0, out, S_out, cu_seqlens, N, B, T, H, Dk, Dv, C, io_dtype,
                        beta_dtype, out_dtype, snapshot_every, max_snapshots, snapshots, workspace,
                        workspace_bytes, stream);
}

int gdn_prefill(const void *q, const void *k, const void *v, const float *g, const void *beta,
                const float *S0, void *out, float *S_out, const int32_t *cu_seqlens, int N, int B,
                int T, int H, int Dk, int Dv, int C, kda_dtype io_dtype, kda_dtype beta_dtype,
                kda_dtype out_dtype, void *workspace, size_t workspace_bytes, void *stream) {
    return prefill_impl(q, k, v, g, beta, S0, out, S_out, cu_seqlens, N, B, T, H, Dk, Dv, C, io_dtype,
                        beta_dtype, out_dtype, 0, 0, nullptr, workspace, workspace_bytes, stream, true);
}

}  // extern "C"

namespace {

int decode_impl(const void *q, const void *k, const void *v, const float *g, const void *beta, float *S,
                void *out, int N, int H, int Dk, int Dv, kda_dtype io_dtype, kda_dtype beta_dtype,
                kda_dtype out_dtype, void *stream, bool g_head, bool qk_norm = false, float norm_eps = 0.f) {
    if (!q || !k || !v || (!g && !g_head) || !beta || !S || !out) return KDA_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(g) & 3u) return KDA_ERR_INVALID_ARG;
    if (N < 1 || H < 1 || Dk < 1 || Dv < 1) return KDA_ERR_INVALID_ARG;
    if (!dtype_ok(io_dtype) || !dtype_ok(beta_dtype) || !dtype_ok(out_dtype)) return KDA_ERR_INVALID_ARG;
    if ((long long)N * H > INT_MAX) return KDA_ERR_INVALID_ARG;
    if (!head_dims_supported(Dk, Dv)) return KDA_ERR_UNSUPPORTED;
    kda::DecodeArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.S = S; a.out = out;
    a.N = N; a.H = H; a.Dk = Dk; a.Dv = Dv;
    a.io = static_cast<Dt>(io_dtype); a.beta_dt = static_cast<Dt>(beta_dtype);
    a.out_dt = static_cast<Dt>(out_dtype);
    a.stream = static_cast<hipStream_t>(stream);
    a.g_head = g_head;
    a.qk_norm = qk_norm;
    a.norm_eps = norm_eps;
    return kda::launch_decode(a) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // namespace

extern "C" {

int kda_decode(const void *q, const void *k, const void *v, const float *g, const void *beta, float *S,
               void *out, int N, int H, int Dk, int Dv, kda_dtype io_dtype, kda_dtype beta_dtype,
               kda_dtype out_dtype, void *stream) {
    return decode_impl(q, k, v, g, beta, S, out, N, H, Dk, Dv, io_dtype, beta_dtype, out_dtype, stream, false);
}

int gdn_decode(const void *q, const void *k, const void *v, const float *g, const void *beta, float *S,
               void *out, int N, int H, int Dk, int Dv, kda_dtype io_dtype, kda_dtype beta_dtype,
               kda_dtype out_dtype, void *stream) {
    return decode_impl(q, k, v, g, beta, S, out, N, H, Dk, Dv, io_dtype, beta_dtype, out_dtype, stream, true);
}

}  // extern "C"

extern "C" {

int kda_prefill_ex(const void *q, const void *k, const void *v, const float *g, const void *beta,
                   const float *S0, void *out, float *S_out, const int32_t *cu_seqlens, int N, int B, int T,
                   int H, int Dk, int Dv, int C, kda_dtype io_dtype, kda_dtype beta_dtype,
                   kda_dtype out_dtype, const kda_options *opt, void *workspace, size_t workspace_bytes,
                   void *stream) {
    if (!options_ok(opt)) return KDA_ERR_INVALID_ARG;
    const kda_options o = opt ? *opt : kda_options{};
    if (o.snapshots && (o.snapshot_every < 1 || o.max_snapshots < 1)) return KDA_ERR_INVALID_ARG;
    return prefill_impl(q, k, v, g, beta, S0, out, S_out, cu_seqlens, N, B, T, H, Dk, Dv, C, io_dtype,
                        beta_dtype, out_dtype, o.snapshots ? o.snapshot_every : 0,
                        o.snapshots ? o.max_snapshots : 0, o.snapshots, workspace, workspace_bytes, stream,
                        o.gate == KDA_GATE_HEAD, o.qk_l2norm != 0, o.l2norm_eps);
}

int kda_decode_ex(const void *q, const void *k, const void *v, const float *g, const void *beta, float *S,
                  void *out, int N, int H, int Dk, int Dv, kda_dtype io_dtype, kda_dtype beta_dtype,
                  kda_dtype out_dtype, const kda_options *opt, void *stream) {
    if (!options_ok(opt)) return KDA_ERR_INVALID_ARG;
    const kda_options o = opt ? *opt : kda_options{};
    if (o.snapshots) return KDA_ERR_INVALID_ARG;                  // prefill only
    return decode_impl(q, k, v, g, beta, S, out, N, H, Dk, Dv, io_dtype, beta_dtype, out_dtype, stream,
                       o.gate == KDA_GATE_HEAD, o.qk_l2norm != 0, o.l2norm_eps);
}

}  // extern "C"

extern "C" {

int kda_output_gate(const void *o, const void *gate, const float *weight, void *out, int rows, int H, int Dv,
                    float eps, kda_dtype o_dtype, kda_dtype gate_dtype, kda_dtype out_dtype, void *stream) {
    if (rows < 0 || H < 1 || Dv < 1 || !(eps > 0.f)) return KDA_ERR_INVALID_ARG;     // also rejects NaN eps
    if (rows > 0 && (!o || !gate || !out)) return KDA_ERR_INVALID_ARG;          // empty tensors may be NULL
    if (!dtype_ok(o_dtype) || !dtype_ok(gate_dtype) || !dtype_ok(out_dtype)) return KDA_ERR_INVALID_ARG;
    if ((long long)rows * H > INT_MAX) return KDA_ERR_INVALID_ARG;
    // eight channels per lane: 16-byte vector loads and stores
    if ((reinterpret_cast<uintptr_t>(o) | reinterpret_cast<uintptr_t>(gate) | reinterpret_cast<uintptr_t>(out) |
         reinterpret_cast<uintptr_t>(weight)) & 15u)
        return KDA_ERR_INVALID_ARG;
    // in place only with the same element type (each lane rewrites what it read)
    if (rows > 0 && out == o && out_dtype != o_dtype) return KDA_ERR_INVALID_ARG;
    if (Dv != 64 && Dv != 128) return KDA_ERR_UNSUPPORTED;
    kda::OutputGateArgs a;
    a.o = o; a.gate = gate; a.weight = weight; a.out = out;
    a.rows = rows; a.H = H; a.Dv = Dv; a.eps = eps;
    a.o_dt = static_cast<Dt>(o_dtype); a.gate_dt = static_cast<Dt>(gate_dtype);
    a.out_dt = static_cast<Dt>(out_dtype);
    a.stream = static_cast<hipStream_t>(stream);
    return kda::launch_output_gate(a) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // extern "C"
