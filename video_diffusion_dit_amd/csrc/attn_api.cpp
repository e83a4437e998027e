// C ABI of libattn (declared in include/attn.h): host-side validation, then one launch.
// No HIP call happens before every argument has been checked, so invalid requests are
// rejected on any machine, GPU or not.
#include <limits.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>

#include "attn.h"
#include "attn_launch.h"

namespace {

thread_local char g_last_error[256] = "";

int fail(int status, const char* msg) {
    snprintf(g_last_error, sizeof(g_last_error), "%s", msg);
    return status;
}

bool overlaps(const void* a, size_t abytes, const void* b, size_t bbytes) {
    if (a == nullptr || b == nullptr || abytes == 0 || bbytes == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + bbytes && b0 < a0 + abytes;
}

// Elements of a [d0, d1, d2, d3] tensor, or -1 past 2^62.
long long product(long long a, long long b, long long c, long long d) {
    const long long lim = 1LL << 62;
    long long r = a;
    for (long long x : {b, c, d}) {
        if (x != 0 && r > lim / x) return -1;
        r *= x;
    }
    return r;
}

// The attention kernels read one sequence's K and V rows through buffer resources whose
// record count is a signed 32-bit byte count, so the bytes from a sequence's first key row to
// its end must stay within INT_MAX. Dense rows of one (b, h) are d*2 bytes apart, so N*d*2
// bytes; packed rows are H*d*2 apart, and any segment is at most total_tokens long.
int check_kv_span(long long tokens, long long row_bytes) {
    const long long span = product(tokens, row_bytes, 1, 1);
    if (span < 0 || span > INT_MAX)
        return fail(ATTN_ERR_UNSUPPORTED, "a sequence's K/V rows span more than 2^31 - 1 bytes");
    return ATTN_OK;
}

int check_common(const void* q, const void* k, const void* v, void* out, int H, int d, float scale) {
    if (q == nullptr || k == nullptr || v == nullptr || out == nullptr)
        return fail(ATTN_ERR_INVALID_ARG, "q, k, v and out must be non-null device pointers");
    if (H <= 0) return fail(ATTN_ERR_INVALID_ARG, "H must be >= 1");
    if (!isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, "scale must be finite");
    if (d <= 0) return fail(ATTN_ERR_INVALID_ARG, "d must be >= 1");
    if (d != 128) return fail(ATTN_ERR_UNSUPPORTED, "only head dimension 128 is supported");
    return ATTN_OK;
}

int check_aliasing(const void* q, const void* k, const void* v, void* out, float* lse,
                   size_t tensor_bytes, size_t lse_bytes) {
    if (overlaps(out, tensor_bytes, q, tensor_bytes) || overlaps(out, tensor_bytes, k, tensor_bytes) ||
        overlaps(out, tensor_bytes, v, tensor_bytes))
        return fail(ATTN_ERR_INVALID_ARG, "out overlaps q, k or v");
    if (lse != nullptr &&
        (overlaps(lse, lse_bytes, out, tensor_bytes) || overlaps(lse, lse_bytes, q, tensor_bytes) ||
         overlaps(lse, lse_bytes, k, tensor_bytes) || overlaps(lse, lse_bytes, v, tensor_bytes)))
        return fail(ATTN_ERR_INVALID_ARG, "lse overlaps q, k, v or out");
    return ATTN_OK;
}

int hip_status(hipError_t e) {
    if (e == hipSuccess) return ATTN_OK;
    return fail(ATTN_ERR_HIP, hipGetErrorString(e));
}

// Checks shared by the two packed block-skip entry points (total_tokens >= 1 here).
int check_varlen_lists(const int32_t* cu, const int32_t* kv_idx, const int32_t* kv_cnt, int nseg, int H,
                              int total_tokens, size_t& idx_bytes, size_t& cnt_bytes) {
    if (cu == nullptr) return fail(ATTN_ERR_INVALID_ARG, "cu_seqlens must be a non-null device pointer");
    if (kv_idx == nullptr || kv_cnt == nullptr)
        return fail(ATTN_ERR_INVALID_ARG, "kv_idx and kv_cnt must be non-null device pointers");
    const long long rows = product((long long)attn_impl::varlen_tiles_q(nseg, total_tokens), H, 1, 1);
    const long long entries = product(rows, attn_impl::block_list_stride(total_tokens), 1, 1);
    if (rows < 0 || rows > INT_MAX || entries < 0) return fail(ATTN_ERR_UNSUPPORTED, "too many query tiles for one launch");
    idx_bytes = (size_t)entries * 4;
    cnt_bytes = (size_t)rows * 4;
    return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H,
             int N, int d, float scale, void* stream) {
    g_last_error[0] = '\0';
    int st = check_common(q, k, v, out, H, d, scale);
    if (st != ATTN_OK) return st;
    if (B <= 0 || N <= 0) return fail(ATTN_ERR_INVALID_ARG, "B and N must be >= 1");
    const long long elems = product(B, H, N, d);
    if (elems < 0) return fail(ATTN_ERR_UNSUPPORTED, "tensor too large");
    st = check_kv_span(N, 2LL * d);
    if (st != ATTN_OK) return st;
    const long long tiles = product(B, H, (N + attn_impl::tile_rows() - 1) / attn_impl::tile_rows(), 1);
    if (tiles < 0 || tiles > INT_MAX) return fail(ATTN_ERR_UNSUPPORTED, "too many query tiles for one launch");
    st = check_aliasing(q, k, v, out, lse, (size_t)elems * 2, (size_t)product(B, H, N, 1) * 4);
    if (st != ATTN_OK) return st;
    return hip_status(attn_impl::launch_dense(q, k, v, out, lse, B, H, N, scale,
                                              static_cast<hipStream_t>(stream)));
}

size_t attn_fwd_splitkv_workspace_bytes(int B, int H, int N, int d, int slots) {
    if (B <= 0 || H <= 0 || N <= 0 || d != 128 || slots > ATTN_MAX_SLOTS) return 0;
    if (product(B, H, (N + attn_impl::tile_rows() - 1) / attn_impl::tile_rows(), 1) < 0) return 0;
    if (slots <= 0) slots = attn_impl::concurrent_workgroups();
    return attn_impl::split_plan(B, H, N, slots).workspace_bytes;
}

int attn_fwd_splitkv(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H,
                     int N, int d, float scale, int slots, void* workspace, size_t workspace_bytes,
                     void* stream) {
    g_last_error[0] = '\0';
    int st = check_common(q, k, v, out, H, d, scale);
    if (st != ATTN_OK) return st;
    if (B <= 0 || N <= 0) return fail(ATTN_ERR_INVALID_ARG, "B and N must be >= 1");
    if (slots > ATTN_MAX_SLOTS) return fail(ATTN_ERR_INVALID_ARG, "slots exceeds ATTN_MAX_SLOTS");
    const long long elems = product(B, H, N, d);
    if (elems < 0) return fail(ATTN_ERR_UNSUPPORTED, "tensor too large");
    st = check_kv_span(N, 2LL * d);
    if (st != ATTN_OK) return st;
    const long long tiles = product(B, H, (N + attn_impl::tile_rows() - 1) / attn_impl::tile_rows(), 1);
    if (tiles < 0 || tiles + ATTN_MAX_SLOTS > INT_MAX / 16)
        return fail(ATTN_ERR_UNSUPPORTED, "too many query tiles for one launch");
    st = check_aliasing(q, k, v, out, lse, (size_t)elems * 2, (size_t)product(B, H, N, 1) * 4);
    if (st != ATTN_OK) return st;
    if (slots <= 0) slots = attn_impl::concurrent_workgroups();
    const attn_impl::SplitPlan plan = attn_impl::split_plan(B, H, N, slots);
    if (plan.G > 0) {
        if (workspace == nullptr || workspace_bytes < plan.workspace_bytes)
            return fail(ATTN_ERR_WORKSPACE, "workspace missing or smaller than attn_fwd_splitkv_workspace_bytes()");
        if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
            return fail(ATTN_ERR_WORKSPACE, "workspace must be 256-byte aligned");
        const size_t need = plan.workspace_bytes;
        if (overlaps(workspace, need, out, (size_t)elems * 2) || overlaps(workspace, need, q, (size_t)elems * 2) ||
            overlaps(workspace, need, k, (size_t)elems * 2) || overlaps(workspace, need, v, (size_t)elems * 2) ||
            overlaps(workspace, need, lse, (size_t)product(B, H, N, 1) * 4))
            return fail(ATTN_ERR_INVALID_ARG, "workspace overlaps a tensor argument");
    }
    return hip_status(attn_impl::launch_dense_split(q, k, v, out, lse, B, H, N, scale, plan, workspace,
                                                    static_cast<hipStream_t>(stream)));
}

int attn_qk_prologue(const void* xq, const void* xk, const void* xv, void* q, void* k, void* v,
                     const float* weight_q, const float* weight_k, int B, int N, int H, int d,
                     int frames, int grid_h, int grid_w, float eps, float theta, void* stream) {
    g_last_error[0] = '\0';
    if (xq == nullptr || xk == nullptr || q == nullptr || k == nullptr)
        return fail(ATTN_ERR_INVALID_ARG, "xq, xk, q and k must be non-null device pointers");
    if ((xv == nullptr) != (v == nullptr)) return fail(ATTN_ERR_INVALID_ARG, "xv and v must both be given or both be null");
    if (B <= 0 || N <= 0 || H <= 0) return fail(ATTN_ERR_INVALID_ARG, "B, N and H must be >= 1");
    if (d <= 0) return fail(ATTN_ERR_INVALID_ARG, "d must be >= 1");
    if (d != 128) return fail(ATTN_ERR_UNSUPPORTED, "only head dimension 128 is supported");
    if (frames <= 0 || grid_h <= 0 || grid_w <= 0 || product(frames, grid_h, grid_w, 1) != N)
        return fail(ATTN_ERR_INVALID_ARG, "frames * grid_h * grid_w must equal N (all >= 1)");
    if (!isfinite(eps) || eps < 0.f) return fail(ATTN_ERR_INVALID_ARG, "eps must be finite and >= 0");
    if (!isfinite(theta) || theta <= 0.f) return fail(ATTN_ERR_INVALID_ARG, "theta must be finite and > 0");
    const long long elems = product(B, N, H, d);
    if (elems < 0 || product(B, N, 1, 1) > 4LL * INT_MAX) return fail(ATTN_ERR_UNSUPPORTED, "tensor too large");
    const size_t bytes = (size_t)elems * 2;
    const void* outs[3] = {q, k, v};
    const void* ins[3] = {xq, xk, xv};
    for (int i = 0; i < 3; ++i) {
        for (int j = 0; j < 3; ++j)
            if (overlaps(outs[i], bytes, ins[j], bytes)) return fail(ATTN_ERR_INVALID_ARG, "an output overlaps an input");
        for (int j = i + 1; j < 3; ++j)
            if (overlaps(outs[i], bytes, outs[j], bytes)) return fail(ATTN_ERR_INVALID_ARG, "q, k and v overlap");
        if (overlaps(outs[i], bytes, weight_q, 512) || overlaps(outs[i], bytes, weight_k, 512))
            return fail(ATTN_ERR_INVALID_ARG, "an output overlaps a weight");
    }
    return hip_status(attn_impl::launch_qk_prologue(xq, xk, xv, q, k, v, weight_q, weight_k, B, N, H,
                                                    grid_h, grid_w, eps, theta,
                                                    static_cast<hipStream_t>(stream)));
}

int attn_qk_norm_packed(const void* xq, const void* xk, void* q, void* k, const float* weight_q,
                        const float* weight_k, int total_tokens, int H, int d, float eps, void* stream) {
    g_last_error[0] = '\0';
    if (xq == nullptr || xk == nullptr || q == nullptr || k == nullptr)
        return fail(ATTN_ERR_INVALID_ARG, "xq, xk, q and k must be non-null device pointers");
    if (total_tokens < 0) return fail(ATTN_ERR_INVALID_ARG, "total_tokens must be >= 0");
    if (H <= 0) return fail(ATTN_ERR_INVALID_ARG, "H must be >= 1");
    if (d <= 0) return fail(ATTN_ERR_INVALID_ARG, "d must be >= 1");
    if (d != 128) return fail(ATTN_ERR_UNSUPPORTED, "only head dimension 128 is supported");
    if (!isfinite(eps) || eps < 0.f) return fail(ATTN_ERR_INVALID_ARG, "eps must be finite and >= 0");
    const long long elems = product(total_tokens, H, d, 1);
    if (elems < 0 || product(total_tokens, H, 1, 1) > INT_MAX) return fail(ATTN_ERR_UNSUPPORTED, "tensor too large");
    if (total_tokens == 0) return ATTN_OK;
    const size_t bytes = (size_t)elems * 2;
    // in place is allowed (q == xq, k == xk); any other overlap is not
    if ((q != xq && overlaps(q, bytes, xq, bytes)) || overlaps(q, bytes, xk, bytes) || overlaps(q, bytes, k, bytes) ||
        (k != xk && overlaps(k, bytes, xk, bytes)) || overlaps(k, bytes, xq, bytes))
        return fail(ATTN_ERR_INVALID_ARG, "an output overlaps another tensor (only q == xq and k == xk may share memory)");
    if (overlaps(q, bytes, weight_q, 512) || overlaps(q, bytes, weight_k, 512) || overlaps(k, bytes, weight_q, 512) ||
        overlaps(k, bytes, weight_k, 512))
        return fail(ATTN_ERR_INVALID_ARG, "an output overlaps a weight");
    return hip_status(attn_impl::launch_qk_norm_packed(xq, xk, q, k, weight_q, weight_k, total_tokens, H, eps,
                                                       static_cast<hipStream_t>(stream)));
}

size_t attn_linear_workspace_bytes(int B, int N, int H, int d) {
    if (B <= 0 || N <= 0 || H <= 0 || d != 128 || product(B, N, H, d) < 0) return 0;
    return attn_impl::linear_workspace_bytes(B, N, H);
}

int attn_linear_fwd(const void* q, const void* k, const void* q_rot, const void* k_rot, const void* v, void* out,
                    int B, int N, int H, int d, float eps, void* workspace, size_t workspace_bytes,
                    void* stream) {
    g_last_error[0] = '\0';
    if (q == nullptr || k == nullptr || q_rot == nullptr || k_rot == nullptr || v == nullptr || out == nullptr)
        return fail(ATTN_ERR_INVALID_ARG, "q, k, q_rot, k_rot, v and out must be non-null device pointers");
    if (B <= 0 || N <= 0 || H <= 0) return fail(ATTN_ERR_INVALID_ARG, "B, N and H must be >= 1");
    if (d <= 0) return fail(ATTN_ERR_INVALID_ARG, "d must be >= 1");
    if (d != 128) return fail(ATTN_ERR_UNSUPPORTED, "only head dimension 128 is supported");
    if (!isfinite(eps) || eps < 0.f) return fail(ATTN_ERR_INVALID_ARG, "eps must be finite and >= 0");
    const long long elems = product(B, N, H, d);
    if (elems < 0 || product(B, H, (N + 255) / 256, 1) > INT_MAX / 2 || product(B, H, 512, 1) > INT_MAX)
        return fail(ATTN_ERR_UNSUPPORTED, "tensor too large");
    if (product(N, H, d, 2) > INT_MAX)   // one (b, h) slice is addressed with 32-bit buffer offsets
        return fail(ATTN_ERR_UNSUPPORTED, "N * H * d * 2 bytes exceeds 2^31 - 1");
    const size_t bytes = (size_t)elems * 2;
    const void* ins[5] = {q, k, q_rot, k_rot, v};
    for (int i = 0; i < 5; ++i)
        if (overlaps(out, bytes, ins[i], bytes)) return fail(ATTN_ERR_INVALID_ARG, "out overlaps an input");
    const size_t need = attn_impl::linear_workspace_bytes(B, N, H);
    if (workspace == nullptr || workspace_bytes < need)
        return fail(ATTN_ERR_WORKSPACE, "workspace missing or smaller than attn_linear_workspace_bytes()");
    if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
        return fail(ATTN_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (overlaps(workspace, need, out, bytes))
        return fail(ATTN_ERR_INVALID_ARG, "workspace overlaps out");
    for (int i = 0; i < 5; ++i)
        if (overlaps(workspace, need, ins[i], bytes)) return fail(ATTN_ERR_INVALID_ARG, "workspace overlaps an input");
    return hip_status(attn_impl::launch_linear(q, k, q_rot, k_rot, v, out, B, N, H, eps, workspace,
                                               static_cast<hipStream_t>(stream)));
}

int attn_block_list_stride(int N) { return N > 0 ? attn_impl::block_list_stride(N) : 0; }

size_t attn_block_route_workspace_bytes(int B, int H, int N, int d) {
    if (B <= 0 || H <= 0 || N <= 0 || d != 128) return 0;
    if (product(B, H, N, d) < 0) return 0;
    return attn_impl::route_workspace_bytes(B, H, N);
}

int attn_block_route(const void* q, const void* k, int B, int H, int N, int d, float scale, float tau,
                     int sink_tokens, int32_t* kv_idx, int32_t* kv_cnt, int32_t* order, void* workspace,
                     size_t workspace_bytes, void* stream) {
    g_last_error[0] = '\0';
    if (q == nullptr || k == nullptr || kv_idx == nullptr || kv_cnt == nullptr)
        return fail(ATTN_ERR_INVALID_ARG, "q, k, kv_idx and kv_cnt must be non-null device pointers");
    if (B <= 0 || H <= 0 || N <= 0) return fail(ATTN_ERR_INVALID_ARG, "B, H and N must be >= 1");
    if (d <= 0) return fail(ATTN_ERR_INVALID_ARG, "d must be >= 1");
    if (d != 128) return fail(ATTN_ERR_UNSUPPORTED, "only head dimension 128 is supported");
    if (!isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, "scale must be finite");
    if (isnan(tau) || tau < 0.f) return fail(ATTN_ERR_INVALID_ARG, "tau must be >= 0 (+inf keeps every key tile)");
    if (sink_tokens < 0) return fail(ATTN_ERR_INVALID_ARG, "sink_tokens must be >= 0");
    const long long elems = product(B, H, N, d);
    if (elems < 0) return fail(ATTN_ERR_UNSUPPORTED, "tensor too large");
    const int ntk = (N + attn_impl::tile_keys() - 1) / attn_impl::tile_keys();
    if (ntk > attn_impl::route_max_tiles())
        return fail(ATTN_ERR_UNSUPPORTED, "sequence longer than the routing supports (route_max_tiles key tiles)");
    const long long items = product(B, H, (N + attn_impl::tile_rows() - 1) / attn_impl::tile_rows(), 1);
    if (items < 0 || items > INT_MAX) return fail(ATTN_ERR_UNSUPPORTED, "too many query tiles for one launch");
    const size_t need = attn_impl::route_workspace_bytes(B, H, N);
    if (workspace == nullptr || workspace_bytes < need)
        return fail(ATTN_ERR_WORKSPACE, "workspace missing or smaller than attn_block_route_workspace_bytes()");
    if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
        return fail(ATTN_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    const size_t tb = (size_t)elems * 2;
    const size_t idx_bytes = (size_t)items * attn_impl::block_list_stride(N) * 4, cnt_bytes = (size_t)items * 4;
    const void* outs[4] = {kv_idx, kv_cnt, workspace, order};
    const size_t outb[4] = {idx_bytes, cnt_bytes, need, cnt_bytes};
    for (int i = 0; i < 4; ++i) {
        if (overlaps(outs[i], outb[i], q, tb) || overlaps(outs[i], outb[i], k, tb))
            return fail(ATTN_ERR_INVALID_ARG, "kv_idx, kv_cnt, order or workspace overlaps q or k");
        for (int j = 0; j < i; ++j)
            if (overlaps(outs[i], outb[i], outs[j], outb[j]))
                return fail(ATTN_ERR_INVALID_ARG, "kv_idx, kv_cnt, order and workspace must not overlap");
    }
    return hip_status(attn_impl::launch_block_route(q, k, B, H, N, scale, tau, sink_tokens, kv_idx, kv_cnt, order,
                                                    workspace, static_cast<hipStream_t>(stream)));
}

int attn_fwd_block_sparse(const void* q, const void* k, const void* v, void* out, float* lse,
                          const int32_t* kv_idx, const int32_t* kv_cnt, const int32_t* order, int B, int H,
                          int N, int d, float scale, void* stream) {
    g_last_error[0] = '\0';
    int st = check_common(q, k, v, out, H, d, scale);
    if (st != ATTN_OK) return st;
    if (kv_idx == nullptr || kv_cnt == nullptr)
        return fail(ATTN_ERR_INVALID_ARG, "kv_idx and kv_cnt must be non-null device pointers");
    if (B <= 0 || N <= 0) return fail(ATTN_ERR_INVALID_ARG, "B and N must be >= 1");
    const long long elems = product(B, H, N, d);
    if (elems < 0) return fail(ATTN_ERR_UNSUPPORTED, "tensor too large");
    st = check_kv_span(N, 2LL * d);
    if (st != ATTN_OK) return st;
    const long long items = product(B, H, (N + attn_impl::tile_rows() - 1) / attn_impl::tile_rows(), 1);
    if (items < 0 || items > INT_MAX) return fail(ATTN_ERR_UNSUPPORTED, "too many query tiles for one launch");
    const size_t tb = (size_t)elems * 2, lb = (size_t)product(B, H, N, 1) * 4;
    st = check_aliasing(q, k, v, out, lse, tb, lb);
    if (st != ATTN_OK) return st;
    const size_t idx_bytes = (size_t)items * attn_impl::block_list_stride(N) * 4, cnt_bytes = (size_t)items * 4;
    if (overlaps(out, tb, kv_idx, idx_bytes) || overlaps(out, tb, kv_cnt, cnt_bytes) ||
        overlaps(lse, lb, kv_idx, idx_bytes) || overlaps(lse, lb, kv_cnt, cnt_bytes) ||
        overlaps(out, tb, order, cnt_bytes) || overlaps(lse, lb, order, cnt_bytes))
        return fail(ATTN_ERR_INVALID_ARG, "out or lse overlaps kv_idx, kv_cnt or order");
    return hip_status(attn_impl::launch_block_sparse(q, k, v, out, lse, kv_idx, kv_cnt, order, B, H, N, scale,
                                                     static_cast<hipStream_t>(stream)));
}

int attn_block_varlen_tiles(int nseg, int total_tokens) {
    if (nseg <= 0 || total_tokens < 0) return 0;
    const size_t t = attn_impl::varlen_tiles_q(nseg, total_tokens);
    return t > (size_t)INT_MAX ? 0 : (int)t;
}

size_t attn_block_route_varlen_workspace_bytes(int nseg, int H, int total_tokens, int d) {
    if (nseg <= 0 || H <= 0 || total_tokens < 0 || d != 128) return 0;
    return attn_impl::route_varlen_workspace_bytes(nseg, H, total_tokens);
}

int attn_block_route_varlen(const void* q, const void* k, const int32_t* cu_seqlens, int nseg, int H,
                            int total_tokens, int d, float scale, float tau, int sink_tokens, int32_t* kv_idx,
                            int32_t* kv_cnt, int32_t* order, void* workspace, size_t workspace_bytes, void* stream) {
    g_last_error[0] = '\0';
    if (total_tokens < 0) return fail(ATTN_ERR_INVALID_ARG, "total_tokens must be >= 0");
    if (nseg <= 0) return fail(ATTN_ERR_INVALID_ARG, "nseg must be >= 1");
    if (H <= 0) return fail(ATTN_ERR_INVALID_ARG, "H must be >= 1");
    if (d <= 0) return fail(ATTN_ERR_INVALID_ARG, "d must be >= 1");
    if (d != 128) return fail(ATTN_ERR_UNSUPPORTED, "only head dimension 128 is supported");
    if (!isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, "scale must be finite");
    if (isnan(tau) || tau < 0.f) return fail(ATTN_ERR_INVALID_ARG, "tau must be >= 0 (+inf keeps every key tile)");
    if (sink_tokens < 0) return fail(ATTN_ERR_INVALID_ARG, "sink_tokens must be >= 0");
    if (total_tokens == 0) return ATTN_OK;
    if (q == nullptr || k == nullptr) return fail(ATTN_ERR_INVALID_ARG, "q and k must be non-null device pointers");
    const long long elems = product(total_tokens, H, d, 1);
    if (elems < 0) return fail(ATTN_ERR_UNSUPPORTED, "tensor too large");
    if ((total_tokens + attn_impl::tile_keys() - 1) / attn_impl::tile_keys() > attn_impl::route_max_tiles())
        return fail(ATTN_ERR_UNSUPPORTED, "packed batch longer than the routing supports (route_max_tiles key tiles)");
    size_t idx_bytes = 0, cnt_bytes = 0;
    int st = check_varlen_lists(cu_seqlens, kv_idx, kv_cnt, nseg, H, total_tokens, idx_bytes, cnt_bytes);
    if (st != ATTN_OK) return st;
    const size_t need = attn_impl::route_varlen_workspace_bytes(nseg, H, total_tokens);
    if (workspace == nullptr || workspace_bytes < need)
        return fail(ATTN_ERR_WORKSPACE, "workspace missing or smaller than attn_block_route_varlen_workspace_bytes()");
    if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
        return fail(ATTN_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    const size_t tb = (size_t)elems * 2;
    const void* outs[4] = {kv_idx, kv_cnt, workspace, order};
    const size_t outb[4] = {idx_bytes, cnt_bytes, need, cnt_bytes};
    for (int i = 0; i < 4; ++i) {
        if (overlaps(outs[i], outb[i], q, tb) || overlaps(outs[i], outb[i], k, tb) ||
            overlaps(outs[i], outb[i], cu_seqlens, sizeof(int32_t) * ((size_t)nseg + 1)))
            return fail(ATTN_ERR_INVALID_ARG, "kv_idx, kv_cnt, order or workspace overlaps q, k or cu_seqlens");
        for (int j = 0; j < i; ++j)
            if (overlaps(outs[i], outb[i], outs[j], outb[j]))
                return fail(ATTN_ERR_INVALID_ARG, "kv_idx, kv_cnt, order and workspace must not overlap");
    }
    return hip_status(attn_impl::launch_block_route_varlen(q, k, cu_seqlens, nseg, H, total_tokens, scale, tau,
                                                           sink_tokens, kv_idx, kv_cnt, order, workspace,
                                                           static_cast<hipStream_t>(stream)));
}

size_t attn_fwd_block_sparse_varlen_workspace_bytes(int nseg, int H, int total_tokens) {
    if (nseg <= 0 || H <= 0 || total_tokens < 0) return 0;
    return attn_impl::block_sparse_varlen_workspace_bytes(nseg, total_tokens);
}

int attn_fwd_block_sparse_varlen(const void* q, const void* k, const void* v, void* out, float* lse,
                                 const int32_t* cu_seqlens, const int32_t* kv_idx, const int32_t* kv_cnt,
                                 const int32_t* order, int nseg, int H, int total_tokens, int d, float scale,
                                 void* workspace, size_t workspace_bytes, void* stream) {
    g_last_error[0] = '\0';
    if (total_tokens < 0) return fail(ATTN_ERR_INVALID_ARG, "total_tokens must be >= 0");
    if (nseg <= 0) return fail(ATTN_ERR_INVALID_ARG, "nseg must be >= 1");
    if (total_tokens == 0) {
        if (H <= 0) return fail(ATTN_ERR_INVALID_ARG, "H must be >= 1");
        if (!isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, "scale must be finite");
        if (d != 128) return fail(d <= 0 ? ATTN_ERR_INVALID_ARG : ATTN_ERR_UNSUPPORTED,
                                  "only head dimension 128 is supported");
        return ATTN_OK;
    }
    int st = check_common(q, k, v, out, H, d, scale);
    if (st != ATTN_OK) return st;
    const long long elems = product(total_tokens, H, d, 1);
    if (elems < 0) return fail(ATTN_ERR_UNSUPPORTED, "tensor too large");
    st = check_kv_span(total_tokens, 2LL * H * d);
    if (st != ATTN_OK) return st;
    size_t idx_bytes = 0, cnt_bytes = 0;
    st = check_varlen_lists(cu_seqlens, kv_idx, kv_cnt, nseg, H, total_tokens, idx_bytes, cnt_bytes);
    if (st != ATTN_OK) return st;
    const size_t need = attn_impl::block_sparse_varlen_workspace_bytes(nseg, total_tokens);
    if (workspace == nullptr || workspace_bytes < need)
        return fail(ATTN_ERR_WORKSPACE, "workspace missing or smaller than attn_fwd_block_sparse_varlen_workspace_bytes()");
    if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
        return fail(ATTN_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    const size_t tb = (size_t)elems * 2, lb = (size_t)product(H, total_tokens, 1, 1) * 4;
    st = check_aliasing(q, k, v, out, lse, tb, lb);
    if (st != ATTN_OK) return st;
    if (overlaps(out, tb, kv_idx, idx_bytes) || overlaps(out, tb, kv_cnt, cnt_bytes) ||
        overlaps(lse, lb, kv_idx, idx_bytes) || overlaps(lse, lb, kv_cnt, cnt_bytes) ||
        overlaps(out, tb, order, cnt_bytes) || overlaps(lse, lb, order, cnt_bytes))
        return fail(ATTN_ERR_INVALID_ARG, "out or lse overlaps kv_idx, kv_cnt or order");
    const void* ins[8] = {q, k, v, out, lse, kv_idx, kv_cnt, order};
    const size_t inb[8] = {tb, tb, tb, tb, lb, idx_bytes, cnt_bytes, cnt_bytes};
    for (int i = 0; i < 8; ++i)
        if (overlaps(workspace, need, ins[i], inb[i]))
            return fail(ATTN_ERR_INVALID_ARG, "workspace overlaps a tensor argument");
    if (overlaps(workspace, need, cu_seqlens, sizeof(int32_t) * ((size_t)nseg + 1)))
        return fail(ATTN_ERR_INVALID_ARG, "workspace overlaps cu_seqlens");
    return hip_status(attn_impl::launch_block_sparse_varlen(q, k, v, out, lse, cu_seqlens, kv_idx, kv_cnt, order,
                                                            nseg, H, total_tokens, scale, workspace,
                                                            static_cast<hipStream_t>(stream)));
}

int attn_block_skip_use_dense(int step, int layer, int dense_steps, const char* dense_layers) {
    g_last_error[0] = '\0';
    if (step < 0 || layer < 0 || dense_steps < 0)
        return fail(ATTN_ERR_INVALID_ARG, "step, layer and dense_steps must be >= 0");
    bool dense = step < dense_steps;
    // dense_layers: comma-separated items "a" or "a-b" (inclusive, a <= b), blanks allowed
    const char* p = dense_layers != nullptr ? dense_layers : "";
    auto blank = [](char c) { return c == ' ' || c == '\t'; };
    auto number = [&](long& out) {
        while (blank(*p)) ++p;
        if (*p < '0' || *p > '9') return false;
        long v = 0;
        while (*p >= '0' && *p <= '9') {
            v = v * 10 + (*p - '0');
            if (v > INT_MAX) return false;
            ++p;
        }
        while (blank(*p)) ++p;
        out = v;
        return true;
    };
    while (blank(*p)) ++p;
    while (*p != '\0') {
        long a, b;
        if (!number(a)) return fail(ATTN_ERR_INVALID_ARG, "dense_layers: expected a layer number");
        b = a;
        if (*p == '-') {
            ++p;
            if (!number(b) || b < a) return fail(ATTN_ERR_INVALID_ARG, "dense_layers: bad range");
        }
        if (layer >= a && layer <= b) dense = true;
        if (*p == ',') {
            ++p;
            while (blank(*p)) ++p;
            if (*p == '\0') return fail(ATTN_ERR_INVALID_ARG, "dense_layers: trailing comma");
        } else if (*p != '\0') {
            return fail(ATTN_ERR_INVALID_ARG, "dense_layers: unexpected character");
        }
    }
    return dense ? 1 : 0;
}

size_t attn_fwd_varlen_workspace_bytes(int nseg, int H, int total_tokens) {
    if (nseg <= 0 || H <= 0 || total_tokens < 0) return 0;
    return attn_impl::varlen_workspace_bytes(nseg, total_tokens);
}

}  // extern "C"

namespace {

// Validation shared by attn_fwd_varlen and attn_fwd_varlen_noalloc, everything but the
// workspace. Returns ATTN_OK with `empty` set for the T = 0 no-op, else the tensor size.
int check_varlen(const void* q, const void* k, const void* v, void* out, float* lse, const int32_t* cu_seqlens,
                 int nseg, int H, int total_tokens, int d, float scale, bool& empty, long long& elems) {
    empty = false;
    if (total_tokens < 0) return fail(ATTN_ERR_INVALID_ARG, "total_tokens must be >= 0");
    if (nseg <= 0) return fail(ATTN_ERR_INVALID_ARG, "nseg must be >= 1");
    if (total_tokens == 0) {
        // nothing to compute; still reject requests that would be invalid at any size
        if (H <= 0) return fail(ATTN_ERR_INVALID_ARG, "H must be >= 1");
        if (!isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, "scale must be finite");
        if (d != 128) return fail(d <= 0 ? ATTN_ERR_INVALID_ARG : ATTN_ERR_UNSUPPORTED,
                                  "only head dimension 128 is supported");
        empty = true;
        return ATTN_OK;
    }
    int st = check_common(q, k, v, out, H, d, scale);
    if (st != ATTN_OK) return st;
    if (cu_seqlens == nullptr) return fail(ATTN_ERR_INVALID_ARG, "cu_seqlens must be a non-null device pointer");
    elems = product(total_tokens, H, d, 1);
    if (elems < 0) return fail(ATTN_ERR_UNSUPPORTED, "tensor too large");
    st = check_kv_span(total_tokens, 2LL * H * d);
    if (st != ATTN_OK) return st;
    const long long grid = product((long long)total_tokens / attn_impl::tile_rows() + nseg, H, 1, 1);
    if (grid < 0 || grid > INT_MAX) return fail(ATTN_ERR_UNSUPPORTED, "too many query tiles for one launch");
    return check_aliasing(q, k, v, out, lse, (size_t)elems * 2, (size_t)product(H, total_tokens, 1, 1) * 4);
}

}  // namespace

extern "C" {

int attn_fwd_varlen(const void* q, const void* k, const void* v, void* out, float* lse,
                    const int32_t* cu_seqlens, int nseg, int H, int total_tokens, int d, float scale,
                    void* workspace, size_t workspace_bytes, void* stream) {
    g_last_error[0] = '\0';
    bool empty;
    long long elems = 0;
    int st = check_varlen(q, k, v, out, lse, cu_seqlens, nseg, H, total_tokens, d, scale, empty, elems);
    if (st != ATTN_OK || empty) return st;
    const size_t need = attn_impl::varlen_workspace_bytes(nseg, total_tokens);
    if (workspace == nullptr || workspace_bytes < need)
        return fail(ATTN_ERR_WORKSPACE, "workspace missing or smaller than attn_fwd_varlen_workspace_bytes()");
    if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
        return fail(ATTN_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (overlaps(workspace, need, out, (size_t)elems * 2) || overlaps(workspace, need, q, (size_t)elems * 2) ||
        overlaps(workspace, need, k, (size_t)elems * 2) || overlaps(workspace, need, v, (size_t)elems * 2) ||
        overlaps(workspace, need, cu_seqlens, sizeof(int32_t) * ((size_t)nseg + 1)))
        return fail(ATTN_ERR_INVALID_ARG, "workspace overlaps a tensor argument");
    return hip_status(attn_impl::launch_varlen(q, k, v, out, lse, cu_seqlens, nseg, H, total_tokens,
                                               scale, workspace, static_cast<hipStream_t>(stream)));
}

size_t attn_fwd_varlen_splitkv_workspace_bytes(int nseg, int H, int total_tokens, int d, int slots) {
    if (nseg <= 0 || H <= 0 || total_tokens < 0 || d != 128 || slots > ATTN_MAX_SLOTS) return 0;
    if (slots <= 0) slots = attn_impl::concurrent_workgroups();
    if (slots < 2) return attn_impl::varlen_workspace_bytes(nseg, total_tokens);
    return attn_impl::varlen_split_workspace_bytes(nseg, total_tokens, slots);
}

int attn_fwd_varlen_splitkv(const void* q, const void* k, const void* v, void* out, float* lse,
                            const int32_t* cu_seqlens, int nseg, int H, int total_tokens, int d, float scale,
                            int slots, void* workspace, size_t workspace_bytes, void* stream) {
    g_last_error[0] = '\0';
    bool empty;
    long long elems = 0;
    int st = check_varlen(q, k, v, out, lse, cu_seqlens, nseg, H, total_tokens, d, scale, empty, elems);
    if (st != ATTN_OK || empty) return st;
    if (slots > ATTN_MAX_SLOTS) return fail(ATTN_ERR_INVALID_ARG, "slots exceeds ATTN_MAX_SLOTS");
    if (slots <= 0) slots = attn_impl::concurrent_workgroups();
    const size_t need = slots < 2 ? attn_impl::varlen_workspace_bytes(nseg, total_tokens)
                                  : attn_impl::varlen_split_workspace_bytes(nseg, total_tokens, slots);
    if (workspace == nullptr || workspace_bytes < need)
        return fail(ATTN_ERR_WORKSPACE, "workspace missing or smaller than attn_fwd_varlen_splitkv_workspace_bytes()");
    if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
        return fail(ATTN_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (overlaps(workspace, need, out, (size_t)elems * 2) || overlaps(workspace, need, q, (size_t)elems * 2) ||
        overlaps(workspace, need, k, (size_t)elems * 2) || overlaps(workspace, need, v, (size_t)elems * 2) ||
        overlaps(workspace, need, cu_seqlens, sizeof(int32_t) * ((size_t)nseg + 1)) ||
        overlaps(workspace, need, lse, lse ? (size_t)product(H, total_tokens, 1, 1) * 4 : 0))
        return fail(ATTN_ERR_INVALID_ARG, "workspace overlaps a tensor argument");
    if (slots < 2)
        return hip_status(attn_impl::launch_varlen(q, k, v, out, lse, cu_seqlens, nseg, H, total_tokens, scale,
                                                   workspace, static_cast<hipStream_t>(stream)));
    return hip_status(attn_impl::launch_varlen_split(q, k, v, out, lse, cu_seqlens, nseg, H, total_tokens, scale,
                                                     slots, workspace, static_cast<hipStream_t>(stream)));
}

int attn_fwd_varlen_noalloc(const void* q, const void* k, const void* v, void* out, float* lse,
                            const int32_t* cu_seqlens, int nseg, int H, int total_tokens, int d, float scale,
                            void* stream) {
    g_last_error[0] = '\0';
    bool empty;
    long long elems = 0;
    int st = check_varlen(q, k, v, out, lse, cu_seqlens, nseg, H, total_tokens, d, scale, empty, elems);
    if (st != ATTN_OK || empty) return st;
    if (attn_impl::varlen_workspace_bytes(nseg, total_tokens) > (size_t)ATTN_NOALLOC_SCRATCH_BYTES)
        return fail(ATTN_ERR_UNSUPPORTED,
                    "the tile schedule exceeds the library's fixed scratch (ATTN_NOALLOC_SCRATCH_BYTES); "
                    "use attn_fwd_varlen with a workspace");
    void* scratch = nullptr;
    st = hip_status(attn_impl::noalloc_scratch(&scratch));
    if (st != ATTN_OK) return st;
    return hip_status(attn_impl::launch_varlen(q, k, v, out, lse, cu_seqlens, nseg, H, total_tokens,
                                               scale, scratch, static_cast<hipStream_t>(stream)));
}

const char* attn_status_string(int status) {
    switch (status) {
        case ATTN_OK: return "ok";
        case ATTN_ERR_INVALID_ARG: return "invalid argument";
        case ATTN_ERR_UNSUPPORTED: return "unsupported (valid request outside what this library implements)";
        case ATTN_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
        case ATTN_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* attn_last_error(void) { return g_last_error; }

int attn_tile_rows(void) { return attn_impl::tile_rows(); }
int attn_tile_keys(void) { return attn_impl::tile_keys(); }

}  // extern "C"
