// Internal interface between the C-ABI layer (la_api.cpp) and the kernel
// translation units. Nothing here is exported from the shared library.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "linattn.h"

namespace la {

// A validated, planned call. Pointers are device pointers.
struct Problem {
    int B = 0, H = 0, N = 0, dk = 0, dv = 0;
    int variant = 0;
    bool io_bf16 = false, gate_bf16 = false;
    float eps = 0.f;
    int path = LA_PATH_VALU;  // resolved: VALU or MFMA
    int chunk = 16;           // resolved chunk size
    int segments = 1;         // resolved segment count (KATH / GLA matrix-core path)
    // Sequences: B * H of them (B = the batch, or the number of packed sequences). N is
    // the token count of one head's rows in the layout, L the longest sequence (N for a
    // dense batch), cu the packed batch's cumulative lengths (device, B + 1) or null.
    int L = 0;
    const int32_t* cu = nullptr;
    bool packed = false;      // a packed variable-length batch (set for its size query too)
    const void *q = nullptr, *k = nullptr, *v = nullptr, *g = nullptr, *beta = nullptr;
    const float *S0 = nullptr, *z0 = nullptr;
    void* o = nullptr;
    float *S = nullptr, *z = nullptr;
    void* ws = nullptr;
    size_t ws_bytes = 0;
    hipStream_t stream = nullptr;
};

constexpr int kValuChunk = 16;
constexpr int kMfmaChunk = 64;

// decode.hip
hipError_t launch_decode(const Problem& p);
// compute units of the current device (queried once per device)
int device_cus();
// prefill_valu.hip
hipError_t launch_prefill_valu(const Problem& p);
// state_init.hip: S_final <- S0 (or 0), z_final <- z0 (or 0), for N = 0
hipError_t launch_state_init(const Problem& p);
// prefill_kath_mfma.hip (KATH)
bool kath_mfma_supported(int dk, int dv, bool io_bf16);
size_t kath_mfma_workspace_bytes(const Problem& p);
int kath_mfma_auto_segments(const Problem& p);
hipError_t launch_prefill_kath_mfma(const Problem& p);
// prefill_kda_mfma.hip (KDA)
bool kda_mfma_supported(int dk, int dv, bool io_bf16);
size_t kda_mfma_workspace_bytes(const Problem& p);
hipError_t launch_prefill_kda_mfma(const Problem& p);
// prefill_gla_mfma.hip (GLA)
bool gla_mfma_supported(int dk, int dv, bool io_bf16);
size_t gla_mfma_workspace_bytes(const Problem& p);
int gla_mfma_auto_segments(const Problem& p);
hipError_t launch_prefill_gla_mfma(const Problem& p);
// prefill_ssd_mfma.hip (SSD in one pass: d_k = 128, bf16 io; segments as for GLA)
size_t ssd_mfma_workspace_bytes(const Problem& p);
hipError_t launch_prefill_ssd_mfma(const Problem& p);
// prefill_gdn_mfma.hip (GDN)
bool gdn_mfma_supported(int dk, int dv, bool io_bf16);
size_t gdn_mfma_workspace_bytes(const Problem& p);
hipError_t launch_prefill_gdn_mfma(const Problem& p);

// backward_valu.hip (backward of the prefill: GLA, SSD and KATH here, GDN and KDA through
// backward_gdn_valu.hip), a validated call
struct BwdProblem {
    Problem p;                       // the forward call (inputs, shapes, workspace, stream)
    const void* dO = nullptr;        // dL/do [B,H,N,dv] io
    const float* dS_final = nullptr; // dL/dS_final [B,H,dk,dv] or null (zero)
    void *dq = nullptr, *dk = nullptr, *dv = nullptr, *dg = nullptr;
    void* dbeta = nullptr;           // GDN: dL/dbeta [B,H,N] gate dtype
    float* dS0 = nullptr;
    const float* dz_final = nullptr; // KATH: dL/dz_final [B,H,dk] or null (zero)
    float* dz0 = nullptr;            // KATH: dL/dz0 [B,H,dk]
};
bool backward_supported(int variant);
size_t backward_workspace_bytes(const Problem& p);
hipError_t launch_backward(const BwdProblem& p);
// backward_gdn_valu.hip (GDN and KDA backward, fp32 vector ALUs); called through
// launch_backward
size_t gdn_backward_workspace_bytes(const Problem& p);
hipError_t launch_backward_gdn(const BwdProblem& p);
// backward_ssd_mfma.hip (SSD backward on the matrix cores: bf16, d_k = 128, d_v = 64)
bool ssd_backward_mfma_supported(const Problem& p);
size_t ssd_backward_mfma_workspace_bytes(const Problem& p);
hipError_t launch_backward_ssd_mfma(const BwdProblem& p);
// backward_gdn_mfma.hip (GDN backward on the matrix cores: bf16, d_k = 128, d_v = 64 or 128)
bool gdn_backward_mfma_supported(const Problem& p);
size_t gdn_backward_mfma_workspace_bytes(const Problem& p);
hipError_t launch_backward_gdn_mfma(const BwdProblem& p);

// selective_scan.hip (Mamba-1 selective scan), a validated call
struct ScanProblem {
    int Bt = 0, T = 0, D = 0, n = 0;
    bool io_bf16 = false;
    int dt_softplus = 0;
    const void *dt = nullptr, *Bm = nullptr, *Cm = nullptr, *x = nullptr;
    const float *A = nullptr, *Dskip = nullptr, *dt_bias = nullptr, *h0 = nullptr;
    void* y = nullptr;
    float* hT = nullptr;
    hipStream_t stream = nullptr;
};
bool selective_scan_supported(int n);
hipError_t launch_selective_scan(const ScanProblem& p);

}  // namespace la
