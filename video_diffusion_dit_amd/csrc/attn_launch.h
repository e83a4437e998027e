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

// Split-KV plan of a dense launch for `slots` concurrently resident workgroups: the first D
// query tiles run whole; the last R are shared evenly by G workgroups (G = 0: no split).
struct SplitPlan {
    long items, D, R, G;
    int ntk;
    size_t workspace_bytes;
};
SplitPlan split_plan(int B, int H, int N, int slots);
// Workgroups the current device runs at once (0 if it cannot be queried).
int concurrent_workgroups();
// Dense forward under plan p (workspace >= p.workspace_bytes, 256-byte aligned).
hipError_t launch_dense_split(const void* q, const void* k, const void* v, void* out, float* lse,
                              int B, int H, int N, float scale, const SplitPlan& p, void* workspace,
                              hipStream_t stream);

// Block-skip attention. Key-tile lists: kv_idx [B*H*ntq][block_list_stride(N)] int32,
// kv_cnt [B*H*ntq]; item (b*H + h)*ntq + query tile.
int block_list_stride(int N);
hipError_t launch_block_sparse(const void* q, const void* k, const void* v, void* out, float* lse,
                               const int32_t* kv_idx, const int32_t* kv_cnt, const int32_t* order, int B, int H,
                               int N, float scale, hipStream_t stream);
// Routing of block-skip attention into those lists (block_route_gfx950.hip); workspace holds
// the pooled query and key tiles (route_workspace_bytes, 256-byte aligned); at most
// route_max_tiles() key tiles per sequence.
size_t route_workspace_bytes(int B, int H, int N);
int route_max_tiles();
// order (may be null): the items sorted by list length, longest first.
hipError_t launch_block_route(const void* q, const void* k, int B, int H, int N, float scale, float tau,
                              int sink_tokens, int32_t* kv_idx, int32_t* kv_cnt, int32_t* order, void* workspace,
                              hipStream_t stream);

// Packed (varlen) block-skip: query tiles (256 rows) and key tiles (64 keys) counted per
// segment and numbered segment by segment; at most varlen_tiles_q(nseg, T) query tiles.
// Lists: kv_idx [tiles_q * H][block_list_stride(T)], kv_cnt [tiles_q * H], row (tile * H + h).
size_t varlen_tiles_q(int nseg, int T);
size_t tile_offsets_bytes(int nseg);
// first query and key tile of each segment ([nseg + 1] ints each, 256-byte aligned) into dst
hipError_t launch_tile_offsets(const int32_t* cu, int nseg, int T, void* dst, hipStream_t stream);
size_t route_varlen_workspace_bytes(int nseg, int H, int T);
hipError_t launch_block_route_varlen(const void* q, const void* k, const int32_t* cu, int nseg, int H, int T,
                                     float scale, float tau, int sink_tokens, int32_t* kv_idx, int32_t* kv_cnt,
                                     int32_t* order, void* workspace, hipStream_t stream);
size_t block_sparse_varlen_workspace_bytes(int nseg, int total_tokens);
hipError_t launch_block_sparse_varlen(const void* q, const void* k, const void* v, void* out, float* lse,
                                      const int32_t* cu_seqlens, const int32_t* kv_idx, const int32_t* kv_cnt,
                                      const int32_t* order, int nseg, int H, int total_tokens, float scale,
                                      void* workspace, hipStream_t stream);

// Workspace layout of the varlen schedule (bytes).
size_t varlen_workspace_bytes(int nseg, int total_tokens);

// Device address of the library's fixed scratch array (ATTN_NOALLOC_SCRATCH_BYTES bytes,
// 256-byte aligned) on the calling thread's current device, looked up once per device.
hipError_t noalloc_scratch(void** ptr);

// Packed THD [T,H,128] BF16 forward over segments cu_seqlens[0..nseg]; lse [H,T] may be null.
hipError_t launch_varlen(const void* q, const void* k, const void* v, void* out, float* lse,
                         const int32_t* cu_seqlens, int nseg, int H, int total_tokens, float scale,
                         void* workspace, hipStream_t stream);

// Packed forward with split-KV of the schedule's tail (slots >= 2 resident workgroups): the
// plan is made on the device from the segment lengths; workspace >=
// varlen_split_workspace_bytes(nseg, T, slots), 256-byte aligned.
size_t varlen_split_workspace_bytes(int nseg, int total_tokens, int slots);
hipError_t launch_varlen_split(const void* q, const void* k, const void* v, void* out, float* lse,
                               const int32_t* cu_seqlens, int nseg, int H, int total_tokens, float scale, int slots,
                               void* workspace, hipStream_t stream);

// Prologue: per-head RMSNorm + interleaved 3-D RoPE on xq/xk (token-major [B,N,H,128] BF16)
// into q/k ([B,H,N,128] BF16); xv -> v re-laid only (both may be null). N = F * Hp * Wp.
hipError_t launch_qk_prologue(const void* xq, const void* xk, const void* xv, void* q, void* k, void* v,
                              const float* wq, const float* wk, int B, int N, int H, int Hp, int Wp,
                              float eps, float theta, hipStream_t stream);

// Packed prologue: per-head RMSNorm of THD [T,H,128] BF16 Q and K rows into THD outputs (q == xq
// and k == xk allowed).
hipError_t launch_qk_norm_packed(const void* xq, const void* xk, void* q, void* k, const float* wq, const float* wk,
                                 int T, int H, float eps, hipStream_t stream);

// Linear attention: q, k (ReLU'd), q_rot, k_rot, v, out BF16 [B,N,H,128] token-major;
// workspace >= linear_workspace_bytes(B, N, H), 256-byte aligned.
size_t linear_workspace_bytes(int B, int N, int H);
hipError_t launch_linear(const void* q, const void* k, const void* qr, const void* kr, const void* v, void* out,
                         int B, int N, int H, float eps, void* workspace, hipStream_t stream);

}  // namespace attn_impl
