/*
 * attn.h -- C ABI of libattn: non-causal scaled-dot-product attention forward,
 * BF16 Q/K/V at head_dim 128, written for AMD CDNA4 (gfx950).
 *
 * What is computed (per query row i of one sequence, over the keys j of that sequence):
 *     x_ij = scale * <q_i, k_j>,   o_i = sum_j softmax_j(x_ij) v_j,   lse_i = ln sum_j exp(x_ij)
 * Page "[sglang] SANA-Video 2.0 anchor attention ... FP32 upcast" (blog on sglang PR #49219),
 * code analysis item 1: scaled_dot_product_attention(q, k, v, dropout_p=0.0) on 4-D,
 * equal-shape BF16 tensors -- non-causal, no mask, no dropout. Its "lessons" list: QK^T,
 * softmax and PV accumulate in FP32 from BF16 inputs. Its documentation item: the
 * probabilities are rounded to BF16 before the PV product. Page "PR #33702 report",
 * motivation and breakdown item 2: packed variable-length batches (THD layout, segment
 * offsets) attend within each segment only; head size 128 only.
 *
 * Numerics: QK^T in FP32 (BF16 MFMA), softmax statistics in FP32, probabilities
 * exp(x - m_ref) rounded to BF16 (round-to-nearest-even) before the PV product, where
 * m_ref is a per-row reference the kernel moves only when some probability of a 64-key
 * tile would make a lane's tile sum exceed 2^24 (then to about the row's running maximum
 * plus 48 log2 units); l sums the FP32 probabilities and gives the LSE. O = (PV
 * accumulator) / (l + C) rounded to BF16 RNE, where C adds, for the tiles that hold more
 * than half of a lane's running sum (or move the reference), the difference between the
 * sum of their BF16 probabilities and their FP32 sum: the keys that dominate a row are
 * normalised by the same BF16 values their products used, so their rounding cancels (a
 * row dominated by one key returns that key's v up to the final rounding). Any reference
 * gives the same softmax; this one keeps the work of moving it rare.
 *
 * Value range (every attention entry point): accepted probabilities never exceed 2^24, so
 * before normalisation |O| < N * 2^24 * max|v| (N: keys of the sequence): FP32 holds it while
 * N * max|v| < 2^104, e.g. max|v| < 2^87 at N = 2^17. Right after a move the probabilities
 * are at most 2^-48, so keys whose weight is below 2^-78 of the row maximum's may fall under
 * the FP32 normal range (their share of the output is far below its precision), and the
 * products p * v keep full precision while max|v| >= 2^-78. Q and K: any finite BF16 values
 * (logits up to the FP32 range; the tests use up to about +-1150).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library keeps no
 *     reference after the call returns and allocates nothing (scratch comes from the
 *     caller's workspace argument; attn_fwd_varlen_noalloc alone uses a fixed array of the
 *     library instead).
 *   - Launches are asynchronous on `stream` (a hipStream_t; NULL = the null stream).
 *     Only launch failures are reported (ATTN_ERR_HIP).
 *   - All argument validation happens on the host before any HIP call; on an error
 *     nothing is launched and no output is touched.
 *   - Deterministic: the same inputs on the same device give the same output bits.
 *   - Thread-safe and re-entrant; concurrent calls must not share output buffers.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_INVALID_ARG = -1,  /* null pointer, non-positive size, non-finite scale,
                                   aliasing output, malformed segment arguments */
    ATTN_ERR_UNSUPPORTED = -2,  /* valid request this library does not implement (d != 128,
                                   sizes beyond the kernel's index range); callers may fall back */
    ATTN_ERR_WORKSPACE = -3,    /* workspace null, misaligned or smaller than the *_workspace_bytes() query */
    ATTN_ERR_HIP = -4           /* the HIP runtime rejected a launch; see attn_last_error() */
} attn_status_t;

/*
 * Dense attention forward.
 *   q, k, v : BF16 [B, H, N, d], contiguous (d fastest), read only.
 *   out     : BF16 [B, H, N, d], contiguous; every element is written. Must not overlap
 *             q, k, v or lse.
 *   lse     : FP32 [B, H, N] log-sum-exp of the scaled logits (natural log), or NULL.
 *   B, H, N : batch, heads, tokens; each >= 1. N * d * 2 must not exceed 2^31 - 1
 *             (N <= 8388607 at d = 128: the kernels address one sequence's K/V rows with
 *             32-bit byte offsets); larger N returns ATTN_ERR_UNSUPPORTED.
 *   d       : head dimension; only 128 is supported (else ATTN_ERR_UNSUPPORTED).
 *   scale   : multiplier of q.k (finite; 1/sqrt(d) is the usual value).
 *   stream  : hipStream_t to launch on.
 * Returns an attn_status_t.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
             int B, int H, int N, int d, float scale, void* stream);

/* Largest `slots` value attn_fwd_splitkv accepts. */
#define ATTN_MAX_SLOTS 65536

/*
 * Dense attention forward with the key range of the last query tiles split across
 * workgroups (split-KV), merged through each piece's running statistics. Page "PR #33702
 * report", implementation breakdown item 2: the varlen backend there splits the key
 * sequence of long sequences (a kv_splits setting chosen from the device and the length).
 * Here the split serves the workgroups' last round on the device: the query tiles that
 * would leave most compute units idle at the end are cut into equal shares of
 * (query tile, key tile) pairs, one share per resident workgroup, and the pieces of a cut
 * tile are combined as o = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) (l_p + C_p) and
 * lse = (M + log2 sum_p 2^(m_p - M) l_p) ln 2 (M = max_p m_p; l_p + C_p the piece's
 * normaliser as in the numerics note above). The result equals attn_fwd's within rounding (BF16 P is taken relative to each piece's own
 * reference); for the same inputs, slots and device it is bitwise repeatable.
 *   q, k, v, out, lse, B, H, N, d, scale, stream : as for attn_fwd.
 *   slots  : workgroups that run at once; <= 0 means the current device's compute units
 *            (one workgroup each); at most ATTN_MAX_SLOTS.
 *   workspace : DEVICE scratch of at least attn_fwd_splitkv_workspace_bytes(B, H, N, d, slots)
 *            bytes, 256-byte aligned, holding the cut tiles' partial results between the
 *            two kernels of the call; no initialisation needed; not to be shared by calls
 *            that may run concurrently. May be NULL when that size is 0 (no tile is cut:
 *            the call is then exactly attn_fwd).
 * Returns an attn_status_t (ATTN_ERR_WORKSPACE for a missing, short or misaligned workspace).
 */
int attn_fwd_splitkv(const void* q, const void* k, const void* v, void* out, float* lse,
                     int B, int H, int N, int d, float scale, int slots,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes attn_fwd_splitkv needs (0: no split for these sizes, or invalid sizes). */
size_t attn_fwd_splitkv_workspace_bytes(int B, int H, int N, int d, int slots);

/*
 * Packed variable-length attention forward (THD layout), attention confined to each segment.
 *   q, k, v     : BF16 [T, H, d], contiguous, T = total_tokens (token-major, then head).
 *   out         : BF16 [T, H, d]; every element of every token is written.
 *   lse         : FP32 [H, T] or NULL.
 *   cu_seqlens  : DEVICE int32 [nseg + 1] segment offsets: cu[0] = 0, non-decreasing,
 *                 cu[nseg] = T. Empty segments are allowed. The kernel trusts these values;
 *                 callers validate them (the Python binding does, on a host copy).
 *   nseg        : number of segments, >= 1.
 *   H, d        : heads (>= 1) and head dim (only 128).
 *   total_tokens: T >= 0; T = 0 is a no-op that returns ATTN_OK. T * H * d * 2 must not
 *                 exceed 2^31 - 1 (a segment's K/V rows, H * d * 2 bytes apart, are addressed
 *                 with 32-bit byte offsets); larger batches return ATTN_ERR_UNSUPPORTED.
 *   workspace   : DEVICE scratch of at least attn_fwd_varlen_workspace_bytes(nseg, H, T)
 *                 bytes, 256-byte aligned; holds the tile schedule (longest segment first).
 *                 Its contents need no initialisation; it must not be shared by calls that
 *                 may run concurrently.
 * Returns an attn_status_t.
 */
int attn_fwd_varlen(const void* q, const void* k, const void* v, void* out, float* lse,
                    const int32_t* cu_seqlens, int nseg, int H, int total_tokens, int d,
                    float scale, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes attn_fwd_varlen needs for these sizes (0 if the sizes are invalid). */
size_t attn_fwd_varlen_workspace_bytes(int nseg, int H, int total_tokens);

/*
 * Packed variable-length forward with split-KV of the schedule's tail. Page "PR #33702
 * report", implementation breakdown item 2: the varlen backend there splits the key range of
 * long sequences (kv_splits, chosen from the device and the lengths). Here the split is
 * planned on the device from the segment lengths, for `slots` resident workgroups: items
 * (segment query tile, head) cost their segment's key tiles and run longest segment first;
 * the leading whole rounds of slots equal-cost items run whole, and the remaining items are
 * cut into equal shares of (item, key tile) pairs, one per workgroup, when a share is shorter
 * than the longest remaining item (otherwise nothing is split and the call equals
 * attn_fwd_varlen). The pieces of a cut item are merged as attn_fwd_splitkv merges them.
 * The result equals attn_fwd_varlen's within rounding (each piece takes its BF16
 * probabilities against its own reference); items that are not cut are bit-identical to it;
 * for the same inputs, slots and device it is bitwise repeatable.
 *   q, k, v, out, lse, cu_seqlens, nseg, H, total_tokens, d, scale, stream : as attn_fwd_varlen.
 *   slots      : workgroups that run at once; <= 0 means the current device's compute units;
 *                1 means no split; at most ATTN_MAX_SLOTS.
 *   workspace  : DEVICE scratch of at least attn_fwd_varlen_splitkv_workspace_bytes(nseg, H,
 *                total_tokens, d, slots) bytes, 256-byte aligned (schedule, plan, cost
 *                prefix, partial results of cut items); no initialisation needed; not to be
 *                shared by calls that may run concurrently.
 * Returns an attn_status_t.
 */
int attn_fwd_varlen_splitkv(const void* q, const void* k, const void* v, void* out, float* lse,
                            const int32_t* cu_seqlens, int nseg, int H, int total_tokens, int d,
                            float scale, int slots, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes attn_fwd_varlen_splitkv needs (0 if the sizes are invalid). */
size_t attn_fwd_varlen_splitkv_workspace_bytes(int nseg, int H, int total_tokens, int d, int slots);

/* Bytes of the fixed device scratch array behind attn_fwd_varlen_noalloc (per device). */
#define ATTN_NOALLOC_SCRATCH_BYTES 524288

/*
 * attn_fwd_varlen for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same kernels and the
 * same result bits, but the tile schedule lives in a fixed library array of
 * ATTN_NOALLOC_SCRATCH_BYTES bytes per device instead of a caller workspace. No allocation
 * happens in this call (no hipMalloc/hipFree, no allocating library routine).
 *   Arguments: as attn_fwd_varlen, without workspace/workspace_bytes. The device is the calling
 *   thread's current device, which must own `stream` and the tensors.
 *   Limit: attn_fwd_varlen_workspace_bytes(nseg, H, total_tokens) must not exceed
 *   ATTN_NOALLOC_SCRATCH_BYTES -- every nseg <= 16384 fits at any valid total_tokens --
 *   else ATTN_ERR_UNSUPPORTED (use attn_fwd_varlen with a workspace).
 *   Sharing: every call on one device uses that device's one array, and the array keeps what
 *   the last call wrote (nothing in it needs clearing: each call rebuilds the schedule before
 *   reading it). Calls that may overlap on one device (different streams or threads) race on
 *   it and must be serialised by the caller.
 *   The first call on a device looks up the array's device address (hipGetSymbolAddress);
 *   a failure there returns ATTN_ERR_HIP.
 * Returns an attn_status_t.
 */
int attn_fwd_varlen_noalloc(const void* q, const void* k, const void* v, void* out, float* lse,
                            const int32_t* cu_seqlens, int nseg, int H, int total_tokens, int d,
                            float scale, void* stream);

/*
 * Attention prologue: per-head RMSNorm and interleaved 3-D rotary embedding (RoPE) of the
 * projected Q and K, rounded to BF16 once and written in the head-major layout attn_fwd
 * reads; V is only re-laid. Page "PR #35728 report", key source excerpts (sana_video.py
 * forward: RMSNorm on Q and K, [B, N, H, D] view, interleaved rotary embedding on Q and K
 * only) and page "[sglang] SANA-Video 2.0 anchor attention ... FP32 upcast", introduction
 * (Q/K/V reach attention in BF16 after RMSNorm and RoPE). Per token n and head h, in FP32:
 *   y = x / sqrt(mean(x^2) + eps) * w                     (w = 1 when the weight is NULL)
 *   pair i (channels 2i, 2i+1) turns by phi = pos_a(n) * theta^(-k/P_a), where the 64 pairs
 *   split (22, 21, 21) over the axes a = (t, h, w), k is the pair's index within its axis,
 *   and pos(n) = (n / (grid_h*grid_w), (n / grid_w) % grid_h, n % grid_w):
 *   (y_2i, y_2i+1) -> (y_2i cos phi - y_2i+1 sin phi, y_2i sin phi + y_2i+1 cos phi).
 *   xq, xk     : BF16 [B, N, H, d], contiguous (token-major, as the QKV projection writes them).
 *   xv         : BF16 [B, N, H, d] or NULL; copied unchanged to v.
 *   q, k       : BF16 [B, H, N, d] outputs (the layout of attn_fwd's q and k).
 *   v          : BF16 [B, H, N, d] output, NULL exactly when xv is NULL.
 *   weight_q/k : FP32 [d] RMSNorm weights or NULL (all ones). Device pointers.
 *   B, N, H, d : sizes; d must be 128 (ATTN_ERR_UNSUPPORTED otherwise).
 *   frames, grid_h, grid_w : the token grid, frames * grid_h * grid_w == N.
 *   eps        : >= 0 (1e-6 in the workloads); theta: > 0 (10000 in the workloads).
 * No output may overlap an input, a weight or another output (ATTN_ERR_INVALID_ARG).
 * Asynchronous on `stream`; allocates nothing. Returns an attn_status_t.
 */
int attn_qk_prologue(const void* xq, const void* xk, const void* xv, void* q, void* k, void* v,
                     const float* weight_q, const float* weight_k, int B, int N, int H, int d,
                     int frames, int grid_h, int grid_w, float eps, float theta, void* stream);

/*
 * Prologue of the packed (varlen) path: per-head RMSNorm of the projected Q and K rows, rounded
 * to BF16 once, in the THD layout attn_fwd_varlen reads -- which is the projection's own
 * token-major layout, so nothing is re-laid and V needs no pass at all. Page "PR #35728 report",
 * key source excerpts (RMSNorm on Q and K before attention); page "PR #33702 report",
 * motivation (packed tokens reach the varlen forward in THD). The pages give no positions for
 * packed segments, so no rotation is applied. Per token t and head h, in FP32:
 *   y = x / sqrt(mean(x^2) + eps) * w                     (w = 1 when the weight is NULL)
 *   xq, xk      : BF16 [T, H, d] inputs, contiguous.
 *   q, k        : BF16 [T, H, d] outputs; q == xq and k == xk run in place, any other overlap
 *                 (and any overlap with a weight) is ATTN_ERR_INVALID_ARG.
 *   weight_q/k  : FP32 [d] RMSNorm weights or NULL (all ones). Device pointers.
 *   total_tokens: T >= 0 (0 is a no-op); H >= 1; d must be 128 (ATTN_ERR_UNSUPPORTED otherwise).
 *   eps         : finite, >= 0 (1e-6 in the workloads).
 * Asynchronous on `stream`; allocates nothing. Returns an attn_status_t.
 */
int attn_qk_norm_packed(const void* xq, const void* xk, void* q, void* k, const float* weight_q,
                        const float* weight_k, int total_tokens, int H, int d, float eps, void* stream);

/*
 * SANA-Video linear attention (ReLU feature map, rotated Q/K in the numerator, un-rotated Q/K
 * in the normaliser), per batch b and head h over the N tokens:
 *   ksum = sum_m k_m;  den_n = q_n . ksum + eps;  kv = sum_m v_m k_rot_m^T (d x d);
 *   out_n = (kv q_rot_n) / den_n.
 * Page "PR #35728 report", key source excerpts (sana_video.py forward: normaliser
 * 1 / (K.sum(-1)^T Q + 1e-15) from the un-rotated ReLU'd K and Q, then (V K_rot^T) Q_rot times
 * it, flattened back to [B, N, H*D]; try_sana_video_linear_attention: the first product with
 * BF16 inputs and FP32 accumulation, the second in FP32). Here kv and ksum accumulate in FP32
 * (BF16 MFMA for kv), the second product runs on FP32 values (kv split exactly into three
 * BF16 terms on the matrix cores), den and the division in FP32; out is rounded to BF16.
 *   q, k        : BF16 [B, N, H, d], the ReLU-activated (un-rotated) rows, token-major.
 *   q_rot, k_rot: BF16 [B, N, H, d], the same rows after the rotary embedding.
 *   v           : BF16 [B, N, H, d].
 *   out         : BF16 [B, N, H, d] (the page's [B, N, H*D] after its transpose).
 *   B, N, H, d  : sizes, d must be 128 (ATTN_ERR_UNSUPPORTED otherwise).
 *   eps         : finite, >= 0 (the page's 1e-15).
 *   workspace   : DEVICE scratch of at least attn_linear_workspace_bytes(B, N, H, d) bytes,
 *                 256-byte aligned (per-chunk partial sums, then kv and ksum); no
 *                 initialisation needed; not to be shared by calls that may run concurrently.
 * out may not overlap an input, nor the workspace any tensor (ATTN_ERR_INVALID_ARG).
 * Asynchronous on `stream`; allocates nothing. Deterministic for the same inputs.
 * Returns an attn_status_t.
 */
int attn_linear_fwd(const void* q, const void* k, const void* q_rot, const void* k_rot, const void* v,
                    void* out, int B, int N, int H, int d, float eps, void* workspace,
                    size_t workspace_bytes, void* stream);

/* Workspace bytes attn_linear_fwd needs (0 if the sizes are invalid). The kv pass's token
 * chunks fill whole rounds of the current device's resident workgroups, so query it with the
 * device that will run the call current (without a device, 256 compute units are assumed). */
size_t attn_linear_workspace_bytes(int B, int N, int H, int d);

/*
 * Block-skip attention (a block-sparse hook in the key loop). Page "PR #33702 report" (the
 * Sol-Attn backend for MiniMax-H3), motivation and breakdown: inside the online-softmax pass,
 * KV blocks are routed by a threshold (knob tau) and the rest skipped, without a full proxy
 * score map; sink tokens stay in; a dense guard keeps the first dense_steps denoising steps and
 * the dense_layers layers dense; head size 128 and BF16 only. The page gives no routing
 * formula; the one implemented here is stated at attn_block_route.
 *
 * Key-tile lists (the hook's interface): for dense [B, H, N, 128] inputs, query tile I =
 * rows 256*I .. 256*I+255 of one (b, h) (ntq = ceil(N/256) tiles), key tile J = keys
 * 64*J .. 64*J+63 (ntk = ceil(N/64) tiles). Item = (b*H + h)*ntq + I.
 *   kv_idx : int32 [B*H*ntq][attn_block_list_stride(N)]; row `item` holds kv_cnt[item]
 *            strictly ascending key-tile indices in [0, ntk); the entries after them are read
 *            (up to 8) but never attended to.
 *   kv_cnt : int32 [B*H*ntq].
 * A list that breaks these rules is processed memory-safely (each index is clamped to
 * [previous index, ntk], the count to [0, ntk]) with an unspecified result.
 *   order  : int32 [B*H*ntq] or NULL: the order in which the items are started. The routing
 *            writes, for each (b, h) in turn, its query tiles sorted by list length, longest
 *            first: the last round of the GPU then holds short items, and the workgroups in
 *            flight stay within one or two heads (on the 720p grid 7.5 % faster than item
 *            order, which a sort over all heads was slower than). NULL starts the items in
 *            item order. Results do not depend on it; entries outside the item range are
 *            clamped.
 */

/* Row stride of kv_idx in entries: ceil(N/64) + 8 (0 if N <= 0). */
int attn_block_list_stride(int N);

/*
 * Block-skip attention forward over given key-tile lists: the rows of query tile I attend
 * to the keys of the tiles kv_idx[item][0 .. kv_cnt[item]-1] only (exact softmax over them,
 * the numerics of attn_fwd). With every tile listed the result equals attn_fwd bit for bit.
 * A tile with kv_cnt <= 0 gets O = 0 and LSE = -inf.
 *   q, k, v, out, lse, B, H, N, d, scale, stream : as attn_fwd.
 *   kv_idx, kv_cnt : DEVICE lists as above (read only); out and lse must not overlap them.
 * Returns an attn_status_t.
 */
int attn_fwd_block_sparse(const void* q, const void* k, const void* v, void* out, float* lse,
                          const int32_t* kv_idx, const int32_t* kv_cnt, const int32_t* order, int B, int H,
                          int N, int d, float scale, void* stream);

/*
 * Key-tile routing of block-skip attention: writes kv_idx and kv_cnt for dense [B, H, N, 128]
 * BF16 q and k. Rule (a reading of the page, which names the knobs only): with qbar_I the
 * mean of the valid query rows of tile I and kbar_J that of the valid keys of tile J (FP32),
 *     z_IJ = scale * qbar_I . kbar_J,   J is kept for I  iff  z_IJ >= max_J' z_IJ' - tau
 *                                                       or  64*J < sink_tokens.
 * The tile with the largest z is always kept, so kv_cnt >= 1. The z values are evaluated in
 * FP32; a tile within FP32 rounding of the threshold may go either way.
 *   tau         : >= 0; +inf keeps every tile (dense attention). NaN is rejected.
 *   sink_tokens : >= 0; the key tiles holding keys 0 .. sink_tokens-1 are always kept.
 *   kv_idx, kv_cnt : DEVICE outputs (sizes above); entries after each count up to 8 are set
 *                 to ntk.
 *   order       : DEVICE output [B*H*ntq]: for each (b, h) in order, its ntq items by list
 *                 length, longest first (a counting sort over 4096 bins of length; items in
 *                 one bin, which holds one length while ntk <= 4095, in no fixed order), or
 *                 NULL to skip it.
 *   workspace   : DEVICE scratch of attn_block_route_workspace_bytes(B, H, N, d) bytes,
 *                 256-byte aligned (the pooled tiles); no initialisation needed.
 * Sequences of more than 15360 key tiles (N > 983040) return ATTN_ERR_UNSUPPORTED.
 * Returns an attn_status_t.
 */
int attn_block_route(const void* q, const void* k, int B, int H, int N, int d, float scale, float tau,
                     int sink_tokens, int32_t* kv_idx, int32_t* kv_cnt, int32_t* order, void* workspace,
                     size_t workspace_bytes, void* stream);

/* Workspace bytes attn_block_route needs (0 if the sizes are invalid). */
size_t attn_block_route_workspace_bytes(int B, int H, int N, int d);

/*
 * Block-skip attention on packed (varlen) batches: segment s = rows cu_seqlens[s] ..
 * cu_seqlens[s+1]-1 of THD [total_tokens, H, 128] tensors, attended to within the segment
 * only (as attn_fwd_varlen). Query tiles (256 rows) and key tiles (64 keys) are counted per
 * segment from its first row, and query tiles are numbered segment by segment: tile i of
 * segment s is g = sum over s' < s of ceil(len_s' / 256), plus i. List row (g * H + h) of
 * kv_idx holds that tile's key-tile indices (counted from the segment's first key, ascending,
 * below ceil(len_s / 64)); kv_cnt[g * H + h] their number. The lists hold
 * attn_block_varlen_tiles(nseg, total_tokens) * H rows of attn_block_list_stride(total_tokens)
 * entries. The routing rule is attn_block_route's, applied to each segment on its own.
 */

/* Upper bound of the number of query tiles of a packed batch: total_tokens / 256 + nseg. */
int attn_block_varlen_tiles(int nseg, int total_tokens);

/*
 * Key-tile routing of a packed batch into kv_idx / kv_cnt (layout above), q and k BF16 THD.
 * cu_seqlens: DEVICE int32 [nseg + 1] as attn_fwd_varlen takes it (not checked by the
 * kernels; offsets outside [0, total_tokens] are clamped). tau, sink_tokens: as
 * attn_block_route (sinks counted from each segment's first key). order: DEVICE output
 * [tiles * H] (items tile * H + h by list length, longest first; only the first
 * (number of query tiles) * H entries are written) or NULL. workspace: DEVICE scratch of
 * attn_block_route_varlen_workspace_bytes(nseg, H, total_tokens, d) bytes, 256-byte aligned.
 * total_tokens = 0 is a no-op; more than 983040 tokens return ATTN_ERR_UNSUPPORTED.
 * Returns an attn_status_t.
 */
int attn_block_route_varlen(const void* q, const void* k, const int32_t* cu_seqlens, int nseg, int H,
                            int total_tokens, int d, float scale, float tau, int sink_tokens, int32_t* kv_idx,
                            int32_t* kv_cnt, int32_t* order, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes attn_block_route_varlen needs (0 if the sizes are invalid). */
size_t attn_block_route_varlen_workspace_bytes(int nseg, int H, int total_tokens, int d);

/*
 * Block-skip attention forward of a packed batch over given key-tile lists (layout above):
 * as attn_fwd_varlen, except that each query tile attends to its listed key tiles only. With
 * every tile listed the result equals attn_fwd_varlen bit for bit; a tile with kv_cnt <= 0
 * gets O = 0 and LSE = -inf. order: as attn_block_route_varlen writes it, or NULL (the
 * varlen schedule's order: longest segments first). workspace: DEVICE scratch of
 * attn_fwd_block_sparse_varlen_workspace_bytes(nseg, H, total_tokens) bytes, 256-byte aligned
 * (the varlen schedule and the tile numbering). Returns an attn_status_t.
 */
int attn_fwd_block_sparse_varlen(const void* q, const void* k, const void* v, void* out, float* lse,
                                 const int32_t* cu_seqlens, const int32_t* kv_idx, const int32_t* kv_cnt,
                                 const int32_t* order, int nseg, int H, int total_tokens, int d, float scale,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes attn_fwd_block_sparse_varlen needs (0 if the sizes are invalid). */
size_t attn_fwd_block_sparse_varlen_workspace_bytes(int nseg, int H, int total_tokens);

/*
 * The dense guard of block-skip attention (host only): 1 if denoising step `step` of layer
 * `layer` should run dense attention -- step < dense_steps, or layer listed in dense_layers
 * ("a" or "a-b" inclusive items separated by commas, blanks allowed; NULL or "" lists none)
 * -- else 0; ATTN_ERR_INVALID_ARG for negative arguments or a malformed list.
 */
int attn_block_skip_use_dense(int step, int layer, int dense_steps, const char* dense_layers);

/* Static text for a status code. */
const char* attn_status_string(int status);

/* Detail message of the most recent failing call on the calling thread ("" if none). */
const char* attn_last_error(void);

/* Query rows per workgroup tile and keys per inner tile of the compiled kernel. */
int attn_tile_rows(void);
int attn_tile_keys(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
