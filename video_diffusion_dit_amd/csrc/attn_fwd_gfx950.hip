// Non-causal BF16 attention forward for CDNA4 (gfx950), head_dim 128.
//
// Method: blockwise softmax with running row statistics (online softmax), so the N x N
// score matrix never leaves registers; QK^T and PV are BF16 MFMA contractions with FP32
// accumulation, the probabilities are rounded to BF16 before PV. Sources: page "[sglang]
// SANA-Video 2.0 anchor attention ... FP32 upcast" (blog on sglang PR #49219), "lessons"
// list (flash attention accumulates QK^T, softmax and PV in FP32 from BF16 inputs) and
// documentation item (probabilities rounded to BF16 before the PV GEMM); page "PR #33702
// report", motivation (online softmax over KV blocks; packed varlen forward, THD layout).
//
// Work decomposition: one workgroup = 4 waves, one per SIMD, = 256 query rows of one
// (batch, head) or (segment, head); each wave owns 64 query rows (two 32-row blocks) for its
// whole key range. Per 64-key tile:
//
//   S^T[key, q] = K_tile . Q_w^T      v_mfma_f32_32x32x16_bf16, A = K rows from LDS,
//                                     B = the wave's Q rows, held in AGPRs all along
//   P = exp2(S*c - m_ref)             c = scale*log2(e); FP32 VALU
//   O^T[dv, q] += V^T_tile . P^T      A = V^T from LDS by transposing reads, B = P (BF16)
//                                     packed in place in the S^T accumulator registers
//
// Computing S and O transposed puts one query row in each lane (plus its partner lane
// l^32), so row statistics need no cross-lane reductions except one lane-pair exchange.
// The MFMA C layout holds, in register r of lane (n = l%32, g = l/32), row
// m = 8(r/4) + 4g + r%4. Loading K row swap23(m) (bits 2 and 3 of m exchanged) into A row m
// makes register r hold key 16(r/8) + 8g + r%8: registers 8h..8h+7 of lane group g are then
// exactly 8 consecutive keys, which is the B-operand layout of the PV MFMA for key step h.
// The same exchange on the value dims makes each lane's O^T registers 8 consecutive dims.
//
// Data movement: K and V tiles ([64 keys][128 dims] BF16, 16 KiB each) go from HBM/L2
// straight into LDS with buffer loads (no VGPR staging); lanes fetch the 16-byte chunk
// that belongs at their LDS slot, so the XOR-swizzled layouts cost nothing to build.
// Keys past the sequence end fall outside the buffer resource and read as zeros. V stays
// key-major in LDS; ds_read_b64_tr_b16 delivers it transposed: within 16 lanes, lane 4r+c
// reads 4 dims of key row r and lane j receives dim j of the 4 rows. Four LDS stages hold
// tiles t..t+3; the loads of a tile are issued three tiles ahead.
//
// The key loop is hand-scheduled (key_loop_gfx950.inc, written by gen_key_loop.py): with one
// wave per SIMD, the wave itself keeps the matrix core busy by issuing, per tile t,
//   QK(t+1) (32 MFMAs) beside the exp work of keys 32..63 of tile t, then the rescale check
//   PV(t)   (32 MFMAs) beside the exp work of keys 0..31 of tile t+1
// so that about 3.5 VALU instructions follow every MFMA; a second wave on the same SIMD
// issuing VALU work slows the MFMAs of the first, which the one-wave layout avoids.
//
// Row statistics: m_ref (per row, in log2 units of the scaled logit) and l (per-lane
// partial). The common path computes P with the current m_ref and only checks that no
// lane's tile sum exceeds 2^24 (then no probability exceeds 2^24, far from FP32 overflow);
// otherwise (always on a row's first tile, where m_ref = -inf) the wave recomputes S from
// LDS and takes the exact path: m_ref = true row max + 32 (so the largest probability is
// 2^-32 and a later key must beat the max by 56 before the next exact path), rescale of O
// and l, recompute of P. The result
// is the same softmax; only the reference the BF16 probabilities are taken against differs,
// and BF16 rounding is relative, so its error bound does not depend on it.
#include <hip/hip_runtime.h>
#include <limits.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include <mutex>

#include "attn.h"
#include "attn_launch.h"

// Fixed scratch of attn_fwd_varlen_noalloc (the varlen tile schedule), for callers that cannot
// allocate. Each device holds its own copy; host code never passes this name to a kernel, only
// the device address noalloc_scratch() looks up.
static __device__ __align__(256) char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr int D = 128;          // head dim
constexpr int BN = 64;          // keys per tile
constexpr int QW = 64;          // query rows per wave
constexpr int NW = 4;           // waves per workgroup (one per SIMD)
constexpr int BM = NW * QW;     // query rows per workgroup
constexpr int NT = NW * 64;     // threads per workgroup

constexpr int ROW_BYTES = D * 2;                 // one key row in LDS
constexpr int LDS_BYTES = 131072;                // K stages 0-3 at 16 KiB each, then V stages
constexpr int V_LDS = 65536;                     // byte offset of the V stages
constexpr int BUF_FLAGS = 0x00020000;            // raw buffer, 32-bit data format
constexpr float LN2 = 0.693147180559945309f;

__device__ __forceinline__ int swap23(int m) {
    return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// LDS layout of a K tile: key row r, 16-byte chunk c (dims 8c..8c+7) at r*256 + 16*(c ^ (r%16)).
__device__ __forceinline__ int k_swz(int r) { return r & 15; }
// LDS layout of a V tile: key row r, chunk c at r*256 + 16*(c ^ v_swz(r)); chosen so that
// the transposing reads (4 key rows x 2 chunks per 16 lanes) hit 32 distinct bank pairs.
__device__ __forceinline__ int v_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Row stride (floats) of a partial result: 128 unnormalised O values, then m_ref, l (the FP32
// sum of the probabilities) and the correction that makes l + correction the sum of the BF16
// probabilities O was accumulated with on the tiles that hold a lane's dominant keys.
constexpr int PART_STRIDE = 132;
constexpr size_t PART_BYTES = sizeof(float) * PART_STRIDE * BM;   // one workgroup's rows

// One workgroup: query rows q0 .. q0+BM-1 of a sequence of n tokens whose rows are rs
// elements apart (Q/K/V/O point at the sequence's first row; LSE at its first entry), over
// key tiles kt0 .. kt1-1 (kt0 < kt1). With part == nullptr the range is all keys and O (and
// LSE) get the final rows; otherwise the workgroup's unnormalised O, m_ref, l and correction
// go to part (PART_STRIDE floats per row) for a later merge. O is divided by l + correction,
// the LSE takes l. Rows past n are computed on row n-1 and
// not written. Every thread of the workgroup must call this (the key loop has barriers).
// LIST: the key tiles are the kt1 entries of klist (ascending tile indices, readable 8
// entries past kt1; kt0 is unused); the tile-list key loop clamps every entry to
// [previous entry, ntk], so loads stay inside the sequence whatever the list holds.
template <bool LIST>
__device__ __forceinline__ void attn_rows(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                                          const bf16* __restrict__ V, bf16* __restrict__ O,
                                          float* __restrict__ LSE, long rs, int n, int q0, float c,
                                          int kt0, int kt1, float* __restrict__ part,
                                          const int32_t* __restrict__ klist = nullptr) {
    __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int m = lane & 31, g = lane >> 5;
    const long rs_bytes = rs * 2;
    const unsigned sbase = (unsigned)(uintptr_t)(lds_char*)smem;

    // LDS read addresses (stage 0): K fragment for d-step s; transposing V reads for dim
    // block b, half t. The loop adds stage and key-block offsets as immediates.
    const int row = swap23(m);
    unsigned ka[8], va[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) ka[s] = sbase + row * ROW_BYTES + (((2 * s + g) ^ k_swz(row)) << 4);
    {
        const int j = lane & 15, r = j >> 2, c4 = j & 3, mh = (lane >> 4) & 1;
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int vrow = 8 * g + 4 * t + r;   // + 16h, which does not change v_swz
                const int chunk = 4 * b + 2 * mh + (c4 & 1);
                va[2 * b + t] = sbase + V_LDS + vrow * ROW_BYTES + ((chunk ^ v_swz(vrow)) << 4) + ((c4 >> 1) << 3);
            }
    }
    // Buffer->LDS loads: this wave fills 4 KiB of each 16 KiB tile, 1 KiB (4 key rows) per
    // instruction; ko/vo are the lanes' byte offsets of their chunks within the tile.
    int ko[4], vo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int slot_row = 4 * (4 * w + i) + (lane >> 4);
        const int slot_chunk = lane & 15;
        ko[i] = slot_row * (int)rs_bytes + ((slot_chunk ^ k_swz(slot_row)) << 4);
        vo[i] = slot_row * (int)rs_bytes + ((slot_chunk ^ v_swz(slot_row)) << 4);
    }
    const unsigned ldsw = sbase + 4096u * w;
    const int tb = (int)(BN * rs_bytes);
    const int ntile = LIST ? kt1 : kt1 - kt0;
    [[maybe_unused]] const int ntk = (n + BN - 1) / BN;
    int first = kt0, last = kt1 - 1;
    if constexpr (LIST) {
        first = min(max(klist[0], 0), ntk - 1);
        last = min(max(klist[kt1 - 1], first), ntk - 1);
    }
    [[maybe_unused]] const int idx0 = first;
    [[maybe_unused]] const unsigned lp[2] = {(unsigned)(uintptr_t)klist, (unsigned)((uint64_t)(uintptr_t)klist >> 32)};
    // Buffer resources start at the first tile and end at the sequence end.
    const long skip = (long)first * BN * rs_bytes;
    const long left = (long)n * rs_bytes - skip;
    const int nbytes = left > 0x7fffffffL ? 0x7fffffff : (left < 0 ? 0 : (int)left);
    const uint64_t kbase = (uint64_t)(uintptr_t)K + skip, vbase = (uint64_t)(uintptr_t)V + skip;
    const unsigned rk[4] = {(unsigned)kbase, (unsigned)(kbase >> 32) & 0xffffu, (unsigned)nbytes, (unsigned)BUF_FLAGS};
    const unsigned rv[4] = {(unsigned)vbase, (unsigned)(vbase >> 32) & 0xffffu, (unsigned)nbytes, (unsigned)BUF_FLAGS};
    // Keys of the last tile of the range at or past n are masked: key 32kb + 16(r/8) + 8g + r%8
    // of S register r is valid while 32kb + 16(r/8) + r%8 < klim.
    const int valid = min(BN, n - last * BN);
    const int klim = valid - 8 * g;
    int qrow[2];
    uint64_t qa[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        qrow[rb] = q0 + QW * w + 32 * rb + m;
        const int qr = min(qrow[rb], n - 1);
        qa[rb] = (uint64_t)(uintptr_t)(Q + (long)qr * rs + 8 * g);
    }
    const int bperm = (lane ^ 32) << 2;
    f32x16 o[4][2];
    float mref[2], lsum[2], lcor[2];
    if constexpr (LIST) {
#include "key_loop_idx_gfx950.inc"
    } else {
#include "key_loop_gfx950.inc"
    }

#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const float ltot = lsum[rb] + __shfl_xor(lsum[rb], 32);
        const float ctot = lcor[rb] + __shfl_xor(lcor[rb], 32);
        const bool qvalid = qrow[rb] < n;
        if (part != nullptr) {
            if (qvalid) {
                float* prow = part + (long)(qrow[rb] - q0) * PART_STRIDE;
#pragma unroll
                for (int b = 0; b < 4; ++b)
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        float4* d = reinterpret_cast<float4*>(prow + 32 * b + 16 * hh + 8 * g);
                        d[0] = make_float4(o[b][rb][8 * hh + 0], o[b][rb][8 * hh + 1], o[b][rb][8 * hh + 2], o[b][rb][8 * hh + 3]);
                        d[1] = make_float4(o[b][rb][8 * hh + 4], o[b][rb][8 * hh + 5], o[b][rb][8 * hh + 6], o[b][rb][8 * hh + 7]);
                    }
                if (g == 0) {
                    prow[128] = mref[rb];
                    prow[129] = ltot;
                    prow[130] = ctot;
                }
            }
            continue;
        }
        const float inv = 1.0f / (ltot + ctot);
        if (qvalid) {
            bf16* orow = O + (long)qrow[rb] * rs;
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    bf16x8 ov;
#pragma unroll
                    for (int i = 0; i < 8; ++i) ov[i] = (bf16)(o[b][rb][8 * hh + i] * inv);
                    *reinterpret_cast<bf16x8*>(orow + 32 * b + 16 * hh + 8 * g) = ov;
                }
            if (LSE != nullptr && g == 0) LSE[qrow[rb]] = (mref[rb] + __log2f(ltot)) * LN2;
        }
    }
}

struct DenseArgs {
    const bf16* q;
    const bf16* k;
    const bf16* v;
    bf16* o;
    float* lse;
    int N, ntq;
    float c;
};

// Workgroups are dispatched to the 8 XCDs in turn (workgroup x on XCD x % 8), each XCD with its
// own L2. Workgroup x takes item xcd_item(x): the first 8*(n/8) items are dealt so that each XCD
// walks a contiguous run of them (the query tiles of one or two heads, whose K/V its L2 then
// shares); the last n % 8 keep their index. A bijection on [0, n).
__device__ __forceinline__ int xcd_item(int x, int n) {
    const int per = n / 8;
    return x < 8 * per ? (x % 8) * per + x / 8 : x;
}

__global__ __launch_bounds__(NT, 1) void attn_fwd_dense_kernel(DenseArgs a) {
    const int item = xcd_item(blockIdx.x, gridDim.x);
    const int bh = item / a.ntq, qt = item - bh * a.ntq;
    const long base = (long)bh * a.N * D;
    attn_rows<false>(a.q + base, a.k + base, a.v + base, a.o + base, a.lse ? a.lse + (long)bh * a.N : nullptr,
                     D, a.N, qt * BM, a.c, 0, (a.N + BN - 1) / BN, nullptr);
}

// Block-skip attention over caller-given key-tile lists: item = (b*H + h) * ntq + query tile,
// its kv_cnt entry gives how many tiles of its kv_idx row (stride entries) it attends to.
// Workgroup x takes item order[x] (clamped to a valid item), or item x without an order. A
// tile with no keys gets O = 0 and LSE = -inf (softmax over an empty set).
struct SparseArgs {
    const bf16* q;
    const bf16* k;
    const bf16* v;
    bf16* o;
    float* lse;
    const int32_t* kidx;
    const int32_t* kcnt;
    const int32_t* order;
    int N, ntq, ntk, stride;
    float c;
};

__global__ __launch_bounds__(NT, 1) void attn_fwd_block_sparse_kernel(SparseArgs a) {
    const int item = a.order != nullptr ? min(max(a.order[blockIdx.x], 0), (int)gridDim.x - 1) : (int)blockIdx.x;
    const int bh = item / a.ntq, qt = item - bh * a.ntq;
    const long base = (long)bh * a.N * D;
    const int cnt = min(a.kcnt[item], a.ntk);
    if (cnt <= 0) {
        const int row = qt * BM + (int)threadIdx.x;
        if (row < a.N) {
            uint4* orow = reinterpret_cast<uint4*>(a.o + base + (long)row * D);
#pragma unroll
            for (int i = 0; i < D / 8; ++i) orow[i] = make_uint4(0, 0, 0, 0);
            if (a.lse != nullptr) a.lse[(long)bh * a.N + row] = -INFINITY;
        }
        return;
    }
    attn_rows<true>(a.q + base, a.k + base, a.v + base, a.o + base, a.lse ? a.lse + (long)bh * a.N : nullptr,
                    D, a.N, qt * BM, a.c, 0, cnt, nullptr, a.kidx + (long)item * a.stride);
}

// Split-KV launch (see attn_impl::split_plan): the plain kernel takes whole query tiles
// 0 .. D-1 (D is a whole number of rounds). The last R query tiles are shared by the G
// workgroups of attn_fwd_dense_split_kernel: each covers an equal contiguous share of the
// R*ntk (query tile, key tile) pairs, so every workgroup of the last round does the same work. A workgroup's share is at least one query
// tile long, so a tile is cut at most once per share boundary; a cut tile's pieces write
// partial results (workspace slot 2g for the first piece of share g, 2g+1 for its last) that
// merge_kernel combines.
struct SplitArgs {
    int D, R, G, ntk;
    float* part;
};
constexpr int SPLIT_MIN_TILES = 16;   // no piece shorter than this many key tiles

__device__ __forceinline__ long share_begin(const SplitArgs& sp, int g) {
    return (long)g * sp.R * sp.ntk / sp.G;
}

__global__ __launch_bounds__(NT, 1) void attn_fwd_dense_split_kernel(DenseArgs a, SplitArgs sp) {
    const int g = blockIdx.x;
    const long lo = share_begin(sp, g), hi = share_begin(sp, g + 1);
    const int i0 = (int)(lo / sp.ntk), i1 = (int)((hi - 1) / sp.ntk);
    for (int i = i0; i <= i1; ++i) {
        const long t0 = lo > (long)i * sp.ntk ? lo - (long)i * sp.ntk : 0;
        const long t1 = hi < (long)(i + 1) * sp.ntk ? hi - (long)i * sp.ntk : sp.ntk;
        const int item = sp.D + i;
        const int bh = item / a.ntq, qt = item - bh * a.ntq;
        const long base = (long)bh * a.N * D;
        float* part = nullptr;
        if (t0 != 0 || t1 != sp.ntk) part = sp.part + (size_t)(2 * g + (i == i0 ? 0 : 1)) * (PART_BYTES / sizeof(float));
        if (i != i0) __syncthreads();   // the previous piece's waves are done with LDS
        attn_rows<false>(a.q + base, a.k + base, a.v + base, a.o + base, a.lse ? a.lse + (long)bh * a.N : nullptr,
                         D, a.N, qt * BM, a.c, (int)t0, (int)t1, part);
    }
}

// One block per (cut query tile, 16 rows): combines the tile's partial results,
// O = sum_p 2^(m_p - M) O_p / sum_p 2^(m_p - M) (l_p + c_p) with M = max_p m_p,
// LSE = (M + log2 sum_p 2^(m_p - M) l_p) ln 2.
// Thread (row r, 8-dim chunk k) handles O[r, 8k .. 8k+7].
__global__ __launch_bounds__(256) void merge_kernel(DenseArgs a, SplitArgs sp) {
    const int i = blockIdx.x >> 4, rblk = blockIdx.x & 15;
    const long first = (long)i * sp.ntk, last = first + sp.ntk - 1;
    // shares containing the tile's first and last key tile
    int g0 = (int)((first * sp.G) / ((long)sp.R * sp.ntk));
    while (g0 + 1 < sp.G && share_begin(sp, g0 + 1) <= first) ++g0;
    while (g0 > 0 && share_begin(sp, g0) > first) --g0;
    int g1 = (int)((last * sp.G) / ((long)sp.R * sp.ntk));
    while (g1 + 1 < sp.G && share_begin(sp, g1 + 1) <= last) ++g1;
    while (g1 > 0 && share_begin(sp, g1) > last) --g1;
    if (g0 == g1) return;   // the tile was computed whole

    const int item = sp.D + i;
    const int bh = item / a.ntq, qt = item - bh * a.ntq;
    const int r = rblk * 16 + (threadIdx.x >> 4), k = threadIdx.x & 15;
    const int row = qt * BM + r;
    if (row >= a.N) return;
    // the tile's piece in share g sits in slot 2g when the tile is g's first, else in 2g+1
    float M = -INFINITY;
    for (int g = g0; g <= g1; ++g) {
        const int slot = 2 * g + (share_begin(sp, g) / sp.ntk == i ? 0 : 1);
        M = fmaxf(M, sp.part[(size_t)slot * (PART_BYTES / sizeof(float)) + (size_t)r * PART_STRIDE + 128]);
    }
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float l = 0.f, lb = 0.f;
    for (int g = g0; g <= g1; ++g) {
        const int slot = 2 * g + (share_begin(sp, g) / sp.ntk == i ? 0 : 1);
        const float* prow = sp.part + (size_t)slot * (PART_BYTES / sizeof(float)) + (size_t)r * PART_STRIDE;
        const float wgt = exp2_hw(prow[128] - M);
        l += wgt * prow[129];
        lb += wgt * (prow[129] + prow[130]);
        const float4 x0 = reinterpret_cast<const float4*>(prow + 8 * k)[0];
        const float4 x1 = reinterpret_cast<const float4*>(prow + 8 * k)[1];
        acc[0] += wgt * x0.x; acc[1] += wgt * x0.y; acc[2] += wgt * x0.z; acc[3] += wgt * x0.w;
        acc[4] += wgt * x1.x; acc[5] += wgt * x1.y; acc[6] += wgt * x1.z; acc[7] += wgt * x1.w;
    }
    const float inv = 1.0f / lb;
    bf16x8 ov;
#pragma unroll
    for (int e = 0; e < 8; ++e) ov[e] = (bf16)(acc[e] * inv);
    const long base = (long)bh * a.N * D;
    *reinterpret_cast<bf16x8*>(a.o + base + (long)row * D + 8 * k) = ov;
    if (a.lse != nullptr && k == 0) a.lse[(long)bh * a.N + row] = (M + __log2f(l)) * LN2;
}
// Varlen schedule in the workspace: a 256-byte header, then order[nseg] (segment ids, longest
// first), then entries (segment, query tile) in that order. Header: int [0] entry count,
// [1] items the plain kernel runs (item = entry * H + head; all of them unless a split plan
// took the tail), [2] workgroups of the split kernel (0: no split); int64 at byte 16 the cost
// (key tiles) of the items before the split ones, at byte 24 the cost of the split ones;
// [3] 1 when every entry was listed (offsets that overrun the list cap are not split).
constexpr size_t WS_HEADER = 256;
constexpr int SORT_LIMIT = 8192;   // above this many segments keep the given order

__host__ __device__ inline size_t ws_align(size_t x) { return (x + 255) & ~size_t(255); }
__host__ __device__ inline size_t ws_list_offset(int nseg) {
    return WS_HEADER + ws_align(sizeof(int) * (size_t)nseg);
}
__host__ __device__ inline long max_entries(int nseg, int T) { return (long)T / BM + nseg; }

__device__ __forceinline__ int seg_len(const int32_t* cu, int s, int T) {
    const int a = min(max(cu[s], 0), T);
    const int e = min(max(cu[s + 1], a), T);
    return e - a;
}

// cum (if not null): int64 [entries + 1], the key tiles of the entries before each entry
// (an entry's cost is its segment's key-tile count, the same for every head).
__global__ __launch_bounds__(1024) void build_varlen_schedule(const int32_t* __restrict__ cu,
                                                              int nseg, int T, char* ws, int H,
                                                              long long* __restrict__ cum) {
    __shared__ int chunk[16];
    __shared__ long long cost_chunk[16];
    int* count = reinterpret_cast<int*>(ws);
    int* order = reinterpret_cast<int*>(ws + WS_HEADER);
    int2* list = reinterpret_cast<int2*>(ws + ws_list_offset(nseg));
    const long cap = max_entries(nseg, T);
    const int tid = threadIdx.x;
    const bool sort = nseg <= SORT_LIMIT;

    for (int s = tid; s < nseg; s += 1024) {
        const int len = seg_len(cu, s, T);
        int rank = s;
        if (sort) {
            rank = 0;
            for (int t = 0; t < nseg; ++t) {
                const int lt = seg_len(cu, t, T);
                rank += (lt > len) || (lt == len && t < s);
            }
        }
        order[rank] = s;
    }
    __syncthreads();

    const int per = (nseg + 1023) / 1024;
    const int r0 = min(tid * per, nseg), r1 = min(r0 + per, nseg);
    int sum = 0;
    long long csum = 0;
    for (int r = r0; r < r1; ++r) {
        const int len = seg_len(cu, order[r], T);
        sum += (len + BM - 1) / BM;
        csum += (long long)((len + BM - 1) / BM) * ((len + BN - 1) / BN);
    }
    // exclusive prefix of (sum, csum) over the threads: within each wave by shuffles, then
    // over the 16 wave totals
    const int lane = tid & 63, wv = tid >> 6;
    int s_in = sum;
    long long c_in = csum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int sv = __shfl_up(s_in, o);
        const long long cv = __shfl_up(c_in, o);
        if (lane >= o) {
            s_in += sv;
            c_in += cv;
        }
    }
    if (lane == 63) {
        chunk[wv] = s_in;
        cost_chunk[wv] = c_in;
    }
    __syncthreads();
    int base = 0;
    long long cbase = 0;
    for (int i = 0; i < wv; ++i) {
        base += chunk[i];
        cbase += cost_chunk[i];
    }
    if (tid == 1023) {
        const int acc = base + s_in;
        const long long cacc = cbase + c_in;
        const int n = (int)min((long)acc, cap);   // malformed offsets cannot push readers past the list
        count[0] = n;
        count[1] = (int)min((long long)n * H, (long long)INT_MAX);   // every item runs whole
        count[2] = 0;
        count[3] = n == acc;   // every entry listed (the cost prefix is whole)
        if (cum != nullptr && n == acc) cum[n] = cacc;
    }
    long off = base + s_in - sum;
    long long cc = cbase + c_in - csum;
    for (int r = r0; r < r1; ++r) {
        const int s = order[r];
        const int len = seg_len(cu, s, T);
        const int nt = (len + BM - 1) / BM, ntk = (len + BN - 1) / BN;
        for (int i = 0; i < nt; ++i)
            if (off + i < cap) {
                list[off + i] = make_int2(s, i);
                if (cum != nullptr) cum[off + i] = cc + (long long)i * ntk;
            }
        off += nt;
        cc += (long long)nt * ntk;
    }
}

// Split-KV plan of a packed call for `slots` resident workgroups (one workgroup, after
// build_varlen_schedule). Items (entry e, head h) = e * H + h cost their segment's key tiles;
// the list runs longest segments first. The leading whole rounds of slots items of equal cost
// run whole in the plain kernel (they finish together); the rest is shared by G workgroups in
// equal contiguous shares of (item, key tile) pairs, if a share is shorter than the tail's
// longest item (else splitting would not shorten the tail, and nothing is split).
__global__ __launch_bounds__(64) void varlen_split_plan(char* ws, const long long* __restrict__ cum, int H,
                                                        int slots) {
    if (threadIdx.x != 0) return;
    int* hdr = reinterpret_cast<int*>(ws);
    long long* hdr64 = reinterpret_cast<long long*>(ws + 16);
    const long long n = hdr[0];
    const long long items = n * H;
    auto cost = [&](long long item) { const long long e = item / H; return cum[e + 1] - cum[e]; };
    if (!hdr[3]) return;
    long long r = 0;
    while ((r + 1) * slots <= items && cost(r * slots) == cost((r + 1) * slots - 1)) ++r;
    const long long D = r * slots;
    hdr[2] = 0;
    if (!hdr[3] || D >= items || items > INT_MAX) return;
    auto cum_item = [&](long long item) { const long long e = item / H; return H * cum[e] + (item - e * H) * (cum[e + 1] - cum[e]); };
    const long long base = cum_item(D), W = H * cum[n] - base;
    long long cmax = 0;
    for (long long e = D / H; e < n; ++e) cmax = max(cmax, cum[e + 1] - cum[e]);
    const long long G = min((long long)slots, W / SPLIT_MIN_TILES);
    if (G < 2 || W / G >= cmax) return;
    hdr[1] = (int)D;
    hdr[2] = (int)G;
    hdr64[0] = base;
    hdr64[1] = W;
}

struct VarlenArgs {
    const bf16* q;
    const bf16* k;
    const bf16* v;
    bf16* o;
    float* lse;
    const int32_t* cu;
    const char* ws;
    int nseg, H, T;
    float c;
};

__global__ __launch_bounds__(NT, 1) void attn_fwd_varlen_kernel(VarlenArgs a) {
    const int e = blockIdx.x / a.H, h = blockIdx.x - e * a.H;
    if (e >= reinterpret_cast<const int*>(a.ws)[0] || (int)blockIdx.x >= reinterpret_cast<const int*>(a.ws)[1]) return;
    const int2 t = reinterpret_cast<const int2*>(a.ws + ws_list_offset(a.nseg))[e];
    const int start = min(max(a.cu[t.x], 0), a.T);
    const int n = seg_len(a.cu, t.x, a.T);
    if (t.y * BM >= n) return;
    const long base = ((long)start * a.H + h) * D;
    attn_rows<false>(a.q + base, a.k + base, a.v + base, a.o + base, a.lse ? a.lse + (long)h * a.T + start : nullptr,
                     (long)a.H * D, n, t.y * BM, a.c, 0, (n + BN - 1) / BN, nullptr);
}

// Split-KV of a packed call (the plan of varlen_split_plan): workgroup g covers the cost units
// [lo(g), lo(g+1)) of the split items, lo(g) = base + W g / G; an item's units are its key
// tiles. Whole items write O and LSE; a cut item's piece writes its partial rows to slot 2g if
// the item is the share's first, else 2g+1 (only a share's first and last items can be cut).
struct VarlenSplitArgs {
    const long long* cum;
    float* part;
};

__device__ __forceinline__ long long vs_cost(const long long* cum, int H, long long item) {
    const long long e = item / H;
    return cum[e + 1] - cum[e];
}
__device__ __forceinline__ long long vs_cum_item(const long long* cum, int H, long long item) {
    const long long e = item / H;
    return H * cum[e] + (item - e * H) * (cum[e + 1] - cum[e]);
}
// the item holding cost unit u (0 <= u < H * cum[n])
__device__ __forceinline__ long long vs_item_at(const long long* cum, int H, int n, long long u) {
    int lo = 0, hi = n;   // H*cum[lo] <= u < H*cum[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (H * cum[mid] <= u) lo = mid;
        else hi = mid;
    }
    return (long long)lo * H + (u - H * cum[lo]) / (cum[lo + 1] - cum[lo]);
}
__device__ __forceinline__ long long vs_share_begin(long long base, long long W, int G, int g) {
    return base + W * g / G;
}
// the share holding unit u (base <= u < base + W)
__device__ __forceinline__ int vs_share_of(long long base, long long W, int G, long long u) {
    int g = (int)((u - base) * G / W);
    while (g + 1 < G && vs_share_begin(base, W, G, g + 1) <= u) ++g;
    while (g > 0 && vs_share_begin(base, W, G, g) > u) --g;
    return g;
}

__global__ __launch_bounds__(NT, 1) void attn_fwd_varlen_split_kernel(VarlenArgs a, VarlenSplitArgs sp) {
    const int* hdr = reinterpret_cast<const int*>(a.ws);
    const int G = hdr[2], g = blockIdx.x;
    if (g >= G) return;
    const int n_ent = hdr[0];
    const long long base = reinterpret_cast<const long long*>(a.ws + 16)[0];
    const long long W = reinterpret_cast<const long long*>(a.ws + 16)[1];
    const long long lo = vs_share_begin(base, W, G, g), hi = vs_share_begin(base, W, G, g + 1);
    const int2* list = reinterpret_cast<const int2*>(a.ws + ws_list_offset(a.nseg));
    const long long first = vs_item_at(sp.cum, a.H, n_ent, lo);
    for (long long it = first; it < (long long)n_ent * a.H; ++it) {
        const long long ci = vs_cum_item(sp.cum, a.H, it);
        if (ci >= hi) break;
        const long long c = vs_cost(sp.cum, a.H, it);
        const long long t0 = lo > ci ? lo - ci : 0, t1 = hi < ci + c ? hi - ci : c;
        const int e = (int)(it / a.H), h = (int)(it - (long long)e * a.H);
        const int2 t = list[e];
        const int start = min(max(a.cu[t.x], 0), a.T);
        const int n = seg_len(a.cu, t.x, a.T);
        const long base_el = ((long)start * a.H + h) * D;
        float* part = nullptr;
        if (t0 != 0 || t1 != c) part = sp.part + (size_t)(2 * g + (it == first ? 0 : 1)) * (PART_BYTES / sizeof(float));
        if (it != first) __syncthreads();   // the previous piece's waves are done with LDS
        attn_rows<false>(a.q + base_el, a.k + base_el, a.v + base_el, a.o + base_el,
                         a.lse ? a.lse + (long)h * a.T + start : nullptr, (long)a.H * D, n, t.y * BM, a.c,
                         (int)t0, (int)t1, part);
    }
}

// One block per (share boundary b = 1 .. G-1, 16 rows): the item cut by boundary b is merged
// by the block of the first boundary inside it, O = sum_p 2^(m_p - M) O_p / sum_p 2^(m_p - M) l_p.
__global__ __launch_bounds__(256) void varlen_merge_kernel(VarlenArgs a, VarlenSplitArgs sp) {
    const int* hdr = reinterpret_cast<const int*>(a.ws);
    const int G = hdr[2], b = blockIdx.x / 16 + 1, rblk = blockIdx.x & 15;
    if (b >= G) return;
    const int n_ent = hdr[0];
    const long long base = reinterpret_cast<const long long*>(a.ws + 16)[0];
    const long long W = reinterpret_cast<const long long*>(a.ws + 16)[1];
    const long long u = vs_share_begin(base, W, G, b);
    const long long it = vs_item_at(sp.cum, a.H, n_ent, u);
    const long long ci = vs_cum_item(sp.cum, a.H, it), c = vs_cost(sp.cum, a.H, it);
    if (u == ci) return;                                   // the boundary falls between items
    const int g0 = vs_share_of(base, W, G, ci);
    if (b != g0 + 1) return;                               // an earlier boundary's block merges it
    const int g1 = vs_share_of(base, W, G, ci + c - 1);
    const int e = (int)(it / a.H), h = (int)(it - (long long)e * a.H);
    const int2 t = reinterpret_cast<const int2*>(a.ws + ws_list_offset(a.nseg))[e];
    const int start = min(max(a.cu[t.x], 0), a.T);
    const int n = seg_len(a.cu, t.x, a.T);
    const int r = rblk * 16 + (threadIdx.x >> 4), k = threadIdx.x & 15;
    const int row = t.y * BM + r;
    if (row >= n) return;
    auto slot_row = [&](int g) {
        const int slot = 2 * g + (vs_item_at(sp.cum, a.H, n_ent, vs_share_begin(base, W, G, g)) == it ? 0 : 1);
        return sp.part + (size_t)slot * (PART_BYTES / sizeof(float)) + (size_t)r * PART_STRIDE;
    };
    float M = -INFINITY;
    for (int g = g0; g <= g1; ++g) M = fmaxf(M, slot_row(g)[128]);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float l = 0.f, lb = 0.f;
    for (int g = g0; g <= g1; ++g) {
        const float* prow = slot_row(g);
        const float wgt = exp2_hw(prow[128] - M);
        l += wgt * prow[129];
        lb += wgt * (prow[129] + prow[130]);
        const float4 x0 = reinterpret_cast<const float4*>(prow + 8 * k)[0];
        const float4 x1 = reinterpret_cast<const float4*>(prow + 8 * k)[1];
        acc[0] += wgt * x0.x; acc[1] += wgt * x0.y; acc[2] += wgt * x0.z; acc[3] += wgt * x0.w;
        acc[4] += wgt * x1.x; acc[5] += wgt * x1.y; acc[6] += wgt * x1.z; acc[7] += wgt * x1.w;
    }
    const float inv = 1.0f / lb;
    bf16x8 ov;
#pragma unroll
    for (int x = 0; x < 8; ++x) ov[x] = (bf16)(acc[x] * inv);
    *reinterpret_cast<bf16x8*>(a.o + ((long)(start + row) * a.H + h) * D + 8 * k) = ov;
    if (a.lse != nullptr && k == 0) a.lse[(long)h * a.T + start + row] = (M + __log2f(l)) * LN2;
}

// Block-skip attention over a packed batch: the varlen schedule's entry (segment s, query
// tile i) and head h attend to the key tiles of list row (off_q[s] + i) * H + h, key-tile
// indices counted from the segment's first key (off_q: first query tile of each segment,
// numbered segment by segment, as the routing writes them).
struct SparseVarlenArgs {
    const bf16* q;
    const bf16* k;
    const bf16* v;
    bf16* o;
    float* lse;
    const int32_t* cu;
    const char* ws;       // varlen schedule
    const int* off_q;
    const int32_t* kidx;
    const int32_t* kcnt;
    const int32_t* order; // item order (item = tile * H + h), or null: the schedule's order
    int nseg, H, T, stride;
    float c;
};

// segment holding query tile g of the numbering segment by segment (off ascending, off[0] = 0)
__device__ __forceinline__ int tile_segment_of(const int* off, int nseg, int g) {
    int lo = 0, hi = nseg;   // off[lo] <= g < off[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (off[mid] <= g) lo = mid;
        else hi = mid;
    }
    return lo;
}

__global__ __launch_bounds__(NT, 1) void attn_fwd_block_sparse_varlen_kernel(SparseVarlenArgs a) {
    int2 t;   // (segment, query tile)
    int h;
    if (a.order != nullptr) {
        const int items = a.off_q[a.nseg] * a.H;
        if ((int)blockIdx.x >= items) return;
        const int it = min(max(a.order[blockIdx.x], 0), items - 1);
        const int g = it / a.H;
        h = it - g * a.H;
        t.x = tile_segment_of(a.off_q, a.nseg, g);
        t.y = g - a.off_q[t.x];
    } else {
        const int e = blockIdx.x / a.H;
        h = blockIdx.x - e * a.H;
        if (e >= *reinterpret_cast<const int*>(a.ws)) return;
        t = reinterpret_cast<const int2*>(a.ws + ws_list_offset(a.nseg))[e];
    }
    const int start = min(max(a.cu[t.x], 0), a.T);
    const int n = seg_len(a.cu, t.x, a.T);
    if (t.y * BM >= n) return;
    const long base = ((long)start * a.H + h) * D;
    const long row = ((long)a.off_q[t.x] + t.y) * a.H + h;
    const int cnt = min(a.kcnt[row], (n + BN - 1) / BN);
    float* lse = a.lse ? a.lse + (long)h * a.T + start : nullptr;
    if (cnt <= 0) {
        const int r = t.y * BM + (int)threadIdx.x;
        if (r < n) {
            uint4* orow = reinterpret_cast<uint4*>(a.o + base + (long)r * a.H * D);
#pragma unroll
            for (int i = 0; i < D / 8; ++i) orow[i] = make_uint4(0, 0, 0, 0);
            if (lse != nullptr) lse[r] = -INFINITY;
        }
        return;
    }
    attn_rows<true>(a.q + base, a.k + base, a.v + base, a.o + base, lse, (long)a.H * D, n, t.y * BM, a.c, 0, cnt,
                    nullptr, a.kidx + row * a.stride);
}

inline float log2e_scale(float scale) { return (float)((double)scale * 1.4426950408889634074); }

}  // namespace

namespace attn_impl {

int tile_rows() { return BM; }
int tile_keys() { return BN; }

hipError_t launch_dense(const void* q, const void* k, const void* v, void* out, float* lse,
                        int B, int H, int N, float scale, hipStream_t stream) {
    DenseArgs a;
    a.q = static_cast<const bf16*>(q);
    a.k = static_cast<const bf16*>(k);
    a.v = static_cast<const bf16*>(v);
    a.o = static_cast<bf16*>(out);
    a.lse = lse;
    a.N = N;
    a.ntq = (N + BM - 1) / BM;
    a.c = log2e_scale(scale);
    const long grid = (long)B * H * a.ntq;
    hipLaunchKernelGGL(attn_fwd_dense_kernel, dim3((unsigned)grid), dim3(NT), 0, stream, a);
    return hipGetLastError();
}

SplitPlan split_plan(int B, int H, int N, int slots) {
    SplitPlan p{};
    const long ntq = (N + BM - 1) / BM, items = (long)B * H * ntq;
    const int ntk = (N + BN - 1) / BN;
    p.items = items;
    p.D = items;
    p.ntk = ntk;
    if (slots < 2 || items <= 0) return p;
    const long full = items / slots, r = items % slots;
    if (r == 0 || ntk < SPLIT_MIN_TILES) return p;
    long R, G;
    if (full >= 1) {
        R = slots + r;
        G = slots;
    } else {
        R = items;
        G = std::min<long>(slots, R * ntk / SPLIT_MIN_TILES);
        if (G <= R) return p;   // no workgroup would be added
    }
    p.D = items - R;
    p.R = R;
    p.G = G;
    p.workspace_bytes = 2 * (size_t)G * PART_BYTES;
    return p;
}

int concurrent_workgroups() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return cus;   // one workgroup (4 waves, one per SIMD) per compute unit
}

hipError_t launch_dense_split(const void* q, const void* k, const void* v, void* out, float* lse,
                              int B, int H, int N, float scale, const SplitPlan& p, void* workspace,
                              hipStream_t stream) {
    if (p.G == 0) return launch_dense(q, k, v, out, lse, B, H, N, scale, stream);
    DenseArgs a;
    a.q = static_cast<const bf16*>(q);
    a.k = static_cast<const bf16*>(k);
    a.v = static_cast<const bf16*>(v);
    a.o = static_cast<bf16*>(out);
    a.lse = lse;
    a.N = N;
    a.ntq = (N + BM - 1) / BM;
    a.c = log2e_scale(scale);
    SplitArgs sp;
    sp.D = (int)p.D;
    sp.R = (int)p.R;
    sp.G = (int)p.G;
    sp.ntk = p.ntk;
    sp.part = static_cast<float*>(workspace);
    hipError_t e;
    if (p.D > 0) {   // whole tiles: the plain kernel, whose grid index is the tile index
        hipLaunchKernelGGL(attn_fwd_dense_kernel, dim3((unsigned)p.D), dim3(NT), 0, stream, a);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(attn_fwd_dense_split_kernel, dim3((unsigned)p.G), dim3(NT), 0, stream, a, sp);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(merge_kernel, dim3((unsigned)(p.R * 16)), dim3(256), 0, stream, a, sp);
    return hipGetLastError();
}

int block_list_stride(int N) { return (N + BN - 1) / BN + 8; }

hipError_t launch_block_sparse(const void* q, const void* k, const void* v, void* out, float* lse,
                               const int32_t* kv_idx, const int32_t* kv_cnt, const int32_t* order, int B, int H,
                               int N, float scale, hipStream_t stream) {
    SparseArgs a;
    a.q = static_cast<const bf16*>(q);
    a.k = static_cast<const bf16*>(k);
    a.v = static_cast<const bf16*>(v);
    a.o = static_cast<bf16*>(out);
    a.lse = lse;
    a.kidx = kv_idx;
    a.kcnt = kv_cnt;
    a.order = order;
    a.N = N;
    a.ntq = (N + BM - 1) / BM;
    a.ntk = (N + BN - 1) / BN;
    a.stride = block_list_stride(N);
    a.c = log2e_scale(scale);
    const long grid = (long)B * H * a.ntq;
    hipLaunchKernelGGL(attn_fwd_block_sparse_kernel, dim3((unsigned)grid), dim3(NT), 0, stream, a);
    return hipGetLastError();
}

size_t varlen_workspace_bytes(int nseg, int total_tokens) {
    return ws_list_offset(nseg) + ws_align(sizeof(int2) * (size_t)max_entries(nseg, total_tokens));
}

size_t block_sparse_varlen_workspace_bytes(int nseg, int total_tokens) {
    return varlen_workspace_bytes(nseg, total_tokens) + tile_offsets_bytes(nseg);
}

hipError_t launch_block_sparse_varlen(const void* q, const void* k, const void* v, void* out, float* lse,
                                      const int32_t* cu_seqlens, const int32_t* kv_idx, const int32_t* kv_cnt,
                                      const int32_t* order, int nseg, int H, int total_tokens, float scale,
                                      void* workspace, hipStream_t stream) {
    char* ws = static_cast<char*>(workspace);
    hipLaunchKernelGGL(build_varlen_schedule, dim3(1), dim3(1024), 0, stream, cu_seqlens, nseg, total_tokens, ws, H,
                       (long long*)nullptr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    char* offs = ws + varlen_workspace_bytes(nseg, total_tokens);
    e = launch_tile_offsets(cu_seqlens, nseg, total_tokens, offs, stream);
    if (e != hipSuccess) return e;
    SparseVarlenArgs a;
    a.q = static_cast<const bf16*>(q);
    a.k = static_cast<const bf16*>(k);
    a.v = static_cast<const bf16*>(v);
    a.o = static_cast<bf16*>(out);
    a.lse = lse;
    a.cu = cu_seqlens;
    a.ws = ws;
    a.off_q = reinterpret_cast<const int*>(offs);
    a.kidx = kv_idx;
    a.kcnt = kv_cnt;
    a.order = order;
    a.nseg = nseg;
    a.H = H;
    a.T = total_tokens;
    a.stride = block_list_stride(total_tokens);
    a.c = log2e_scale(scale);
    const long grid = max_entries(nseg, total_tokens) * H;
    hipLaunchKernelGGL(attn_fwd_block_sparse_varlen_kernel, dim3((unsigned)grid), dim3(NT), 0, stream, a);
    return hipGetLastError();
}

hipError_t noalloc_scratch(void** ptr) {
    constexpr int MAX_DEVICES = 64;
    static std::mutex lock;
    static void* addr[MAX_DEVICES] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> guard(lock);
    if (addr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

size_t varlen_split_workspace_bytes(int nseg, int total_tokens, int slots) {
    return varlen_workspace_bytes(nseg, total_tokens) + ws_align(sizeof(long long) * (size_t)(max_entries(nseg, total_tokens) + 1)) +
           2 * (size_t)slots * PART_BYTES;
}

hipError_t launch_varlen_split(const void* q, const void* k, const void* v, void* out, float* lse,
                               const int32_t* cu_seqlens, int nseg, int H, int total_tokens, float scale, int slots,
                               void* workspace, hipStream_t stream) {
    char* ws = static_cast<char*>(workspace);
    long long* cum = reinterpret_cast<long long*>(ws + varlen_workspace_bytes(nseg, total_tokens));
    float* part = reinterpret_cast<float*>(reinterpret_cast<char*>(cum) +
                                           ws_align(sizeof(long long) * (size_t)(max_entries(nseg, total_tokens) + 1)));
    hipLaunchKernelGGL(build_varlen_schedule, dim3(1), dim3(1024), 0, stream, cu_seqlens, nseg, total_tokens, ws, H, cum);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(varlen_split_plan, dim3(1), dim3(64), 0, stream, ws, (const long long*)cum, H, slots);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    VarlenArgs a;
    a.q = static_cast<const bf16*>(q);
    a.k = static_cast<const bf16*>(k);
    a.v = static_cast<const bf16*>(v);
    a.o = static_cast<bf16*>(out);
    a.lse = lse;
    a.cu = cu_seqlens;
    a.ws = ws;
    a.nseg = nseg;
    a.H = H;
    a.T = total_tokens;
    a.c = log2e_scale(scale);
    VarlenSplitArgs sp;
    sp.cum = cum;
    sp.part = part;
    const long grid = max_entries(nseg, total_tokens) * H;
    hipLaunchKernelGGL(attn_fwd_varlen_kernel, dim3((unsigned)grid), dim3(NT), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_fwd_varlen_split_kernel, dim3((unsigned)slots), dim3(NT), 0, stream, a, sp);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(varlen_merge_kernel, dim3((unsigned)(slots - 1) * 16), dim3(256), 0, stream, a, sp);
    return hipGetLastError();
}

hipError_t launch_varlen(const void* q, const void* k, const void* v, void* out, float* lse,
                         const int32_t* cu_seqlens, int nseg, int H, int total_tokens, float scale,
                         void* workspace, hipStream_t stream) {
    char* ws = static_cast<char*>(workspace);
    hipLaunchKernelGGL(build_varlen_schedule, dim3(1), dim3(1024), 0, stream, cu_seqlens, nseg,
                       total_tokens, ws, H, (long long*)nullptr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    VarlenArgs a;
    a.q = static_cast<const bf16*>(q);
    a.k = static_cast<const bf16*>(k);
    a.v = static_cast<const bf16*>(v);
    a.o = static_cast<bf16*>(out);
    a.lse = lse;
    a.cu = cu_seqlens;
    a.ws = ws;
    a.nseg = nseg;
    a.H = H;
    a.T = total_tokens;
    a.c = log2e_scale(scale);
    const long grid = max_entries(nseg, total_tokens) * H;
    hipLaunchKernelGGL(attn_fwd_varlen_kernel, dim3((unsigned)grid), dim3(NT), 0, stream, a);
    return hipGetLastError();
}

}  // namespace attn_impl
