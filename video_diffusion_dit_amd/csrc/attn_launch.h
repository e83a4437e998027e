// Internal interface between the C-ABI layer (attn_api.cpp) and the gfx950 kernels
// (attn_fwd_gfx950.hip). Arguments are already validated when these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn_impl {

// Compile-time tile shape of the forward kernel.
int tile_rows();   // query rows per workgroup (BM)
int tile_keys();   // keys per inner K/V tile (BN)

// Dense [B,H,N,128] BF16 forward; lse may be null.
hipError_t launch_dense(const void* q, const void* k, const void* v, void* out, float* lse,
                        int B, int H, int N, float scale, hipStream_t stream);

// Workspace layout of the varlen schedule (bytes).
size_t varlen_workspace_bytes(int nseg, int total_tokens);

// Packed THD [T,H,128] BF16 forward over segments cu_seqlens[0..nseg]; lse [H,T] may be null.
hipError_t launch_varlen(const void* q, const void* k, const void* v, void* out, float* lse,
                         const int32_t* cu_seqlens, int nseg, int H, int total_tokens, float scale,
                         void* workspace, hipStream_t stream);

}  // namespace attn_impl
