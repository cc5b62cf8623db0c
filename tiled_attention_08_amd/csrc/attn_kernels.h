// attn_kernels.h - launchers of the attention kernels (internal to libattn.so).
// Each launcher assumes validated arguments (see attn_api.hip) and only
// enqueues work on `stream`; it returns hipGetLastError() of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "attn_device.h"

namespace attn {


// causal != 0: query i sees keys j <= i. kv_len (device, B ints, or null):
// keys j >= kv_len[b] are hidden from every query of batch entry b (values are
// clamped to [0, N] on the device).
// 16-bit storage: bf16, or fp16 when f16 is true.
// sq: strides of q, k and v; so: of o.
hipError_t launch_fwd_16(bool f16, const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse,
                         int B, int H, int N, int d, float scale, int causal, const int* kv_len, Strides sq, Strides so,
                         hipStream_t stream);

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H, int N,
                          int d, float scale, hipStream_t stream);

// Workspace layout: lse * log2(e) [B*H*N] fp32, then (256-byte aligned) -delta [B*H*N] fp32.
size_t bwd_workspace_bytes(int B, int H, int N, int d);

// One backward stage: 0 = lse * log2(e) and -delta, 1 = dK and dV, 2 = dQ,
// 3 = stages 1 and 2 in one launch (only where bwd_can_fuse).
// Masks as for launch_fwd_16; st[0..3]: strides of (q, k, v), o, dO and (dq, dk, dv).
hipError_t launch_bwd_16_stage(bool f16, int stage, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                 const uint16_t* o, const float* lse, const uint16_t* dO, uint16_t* dq, uint16_t* dk,
                                 uint16_t* dv, int B, int H, int N, int d, float scale, int causal,
                                 const int* kv_len, const Strides* st, void* workspace, hipStream_t stream);

// Whether stages 1 and 2 may run as the single launch "stage 3" (same results, bit for bit).
bool bwd_can_fuse(int B, int H, int N, int d);

// fp32 backward stage (vector ALU; same stages and workspace as the 16-bit one).
hipError_t launch_bwd_f32_stage(int stage, const float* q, const float* k, const float* v, const float* o,
                                const float* lse, const float* dO, float* dq, float* dk, float* dv, int B, int H, int N,
                                int d, float scale, void* workspace, hipStream_t stream);

// Query/key/value projection: qkv[tokens, HD3] = x[tokens, D] w[D, HD3] (HD3 = 3 H d);
// backward dx = dqkv w^T and dw = x^T dqkv. The backward's workspace (its
// size from proj_bwd_workspace_bytes, 0 when no product splits its
// contraction) holds the float32 partial sums of split products.
hipError_t launch_proj_fwd(bool f16, const uint16_t* x, const uint16_t* w, uint16_t* qkv, long tokens, int D, int HD3,
                           hipStream_t stream);
size_t proj_bwd_workspace_bytes(long tokens, int D, int HD3);
hipError_t launch_proj_bwd(bool f16, const uint16_t* x, const uint16_t* w, const uint16_t* dqkv, uint16_t* dx,
                           uint16_t* dw, long tokens, int D, int HD3, void* ws, hipStream_t stream);

}  // namespace attn
