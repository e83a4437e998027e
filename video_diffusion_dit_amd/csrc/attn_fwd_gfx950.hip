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
// Work decomposition: one workgroup = 4 waves = 128 query rows of one (batch, head) or
// (segment, head); each wave owns 32 query rows for the whole key loop. Per 64-key tile:
//
//   S^T[key, q] = K_tile . Q_w^T      v_mfma_f32_32x32x16_bf16, A = K rows from LDS,
//                                     B = the wave's Q rows, held in VGPRs all along
//   P = exp2(S*c - m_ref)             c = scale*log2(e); FP32 VALU
//   O^T[dv, q] += V^T_tile . P^T      A = V^T rows from LDS, B = P (BF16) straight from
//                                     the S^T accumulator registers
//
// Computing S and O transposed puts one query row in each lane (plus its partner lane
// l^32), so row statistics need no cross-lane reductions except one lane-pair exchange.
// The MFMA C layout holds, in register r of lane (n = l%32, g = l/32), row
// m = 8(r/4) + 4g + r%4. Loading K row swap23(m) (bits 2 and 3 of m exchanged) into A row m
// makes register r hold key 16(r/8) + 8g + r%8: registers 8h..8h+7 of lane group g are then
// exactly 8 consecutive keys, which is the B-operand layout of the PV MFMA for key step h.
// The same exchange on V^T rows makes each lane's O^T registers 8 consecutive output dims.
//
// K tiles sit in LDS row-major [64 keys][128 dims]; V tiles are transposed on their way
// into LDS ([128 dims][64 keys]) so that the PV A operand is one 16-byte LDS read.
// 16-byte chunks are XOR-swizzled so those reads are bank-conflict free. Two LDS stages:
// tile j+1 is fetched from HBM/L2 into VGPRs while tile j is computed, then written to the
// other stage; one barrier per tile.
//
// Row statistics: m_ref (per row, in log2 units of the scaled logit) and l (per lane
// partial). The common path computes P with the current m_ref and only checks that no
// lane's partial tile sum exceeds 2^8 (then no probability exceeds 2^8 and FP32/BF16 stay
// exact in relative terms); otherwise (always on a row's first tile, where m_ref = -inf)
// the wave takes the exact path: true row max, rescale of O and l, recompute of P. The
// result is the same softmax; only the reference the BF16 probabilities are relative to
// differs, which BF16 rounding (relative) does not see.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "attn_launch.h"

namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int D = 128;          // head dim
constexpr int BN = 64;          // keys per tile
constexpr int QW = 32;          // query rows per wave
constexpr int NW = 4;           // waves per workgroup
constexpr int BM = NW * QW;     // query rows per workgroup
constexpr int NT = NW * 64;     // threads per workgroup

constexpr int K_BYTES = BN * D * 2;
constexpr int V_BYTES = BN * D * 2;
constexpr int STAGE_BYTES = K_BYTES + V_BYTES;
constexpr float RESCALE_LIMIT = 256.0f;
constexpr float LN2 = 0.693147180559945309f;

static_assert(BN * D / 8 == 4 * NT, "K tile: four 16-byte chunks per thread");
static_assert((BN / 2) * (D / 8) == 2 * NT, "V tile: two key pairs x 8 dims per thread");

__device__ __forceinline__ int swap23(int m) {
    return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// Byte offset of 16-byte chunk c (dims 8c..8c+7) of key row r in a K tile.
__device__ __forceinline__ int k_off(int r, int c) { return r * 256 + ((c ^ (r & 15)) << 4); }

// Byte offset of 16-byte chunk c (keys 8c..8c+7) of value-dim row r in a V^T tile.
__device__ __forceinline__ int vt_off(int r, int c) {
    return r * 128 + ((c ^ (((r >> 1) ^ (r >> 4)) & 7)) << 4);
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// One tile's worth of K and V held in VGPRs between its global load and its LDS store.
struct Staged {
    u32x4 k[4];
    u32x4 va[2], vb[2];
};

__device__ __forceinline__ void load_tile(Staged& st, const bf16* __restrict__ K,
                                          const bf16* __restrict__ V, long rs, int key0, int n,
                                          int tid) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int idx = tid + NT * i, r = idx >> 4, c = idx & 15;
        const int key = min(key0 + r, n - 1);
        st.k[i] = *reinterpret_cast<const u32x4*>(K + key * rs + c * 8);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int idx = tid + NT * i, kp = idx >> 4, c = idx & 15;
        const int ka = min(key0 + 2 * kp, n - 1), kb = min(key0 + 2 * kp + 1, n - 1);
        st.va[i] = *reinterpret_cast<const u32x4*>(V + ka * rs + c * 8);
        st.vb[i] = *reinterpret_cast<const u32x4*>(V + kb * rs + c * 8);
    }
}

__device__ __forceinline__ void store_tile(const Staged& st, char* lds, int tid) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int idx = tid + NT * i, r = idx >> 4, c = idx & 15;
        *reinterpret_cast<u32x4*>(lds + k_off(r, c)) = st.k[i];
    }
    char* vt = lds + K_BYTES;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int idx = tid + NT * i, kp = idx >> 4, c = idx & 15;
        const int kchunk = kp >> 2, kbyte = (kp & 3) * 4;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint32_t a = st.va[i][w], b = st.vb[i][w];
            const uint32_t lo = (a & 0xffffu) | (b << 16);          // dim 8c+2w, keys 2kp, 2kp+1
            const uint32_t hi = (a >> 16) | (b & 0xffff0000u);      // dim 8c+2w+1
            const int r0 = 8 * c + 2 * w;
            *reinterpret_cast<uint32_t*>(vt + vt_off(r0, kchunk) + kbyte) = lo;
            *reinterpret_cast<uint32_t*>(vt + vt_off(r0 + 1, kchunk) + kbyte) = hi;
        }
    }
}

// Key (within the tile) held by register r of lane group g in an S^T accumulator block kb.
__device__ __forceinline__ int key_of(int kb, int r, int g) {
    return 32 * kb + 16 * (r >> 3) + 8 * g + (r & 7);
}

template <bool MASK>
__device__ __forceinline__ void tile_step(const char* __restrict__ lds, const bf16x8 (&qf)[8],
                                          f32x16 (&oacc)[4], float& mref, float& lsum, float c,
                                          int valid, int m, int g) {
    // S^T = K_tile . Q^T
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        sacc[kb] = f32x16{};
        const int row = 32 * kb + swap23(m);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const bf16x8 kf = *reinterpret_cast<const bf16x8*>(lds + k_off(row, 2 * s + g));
            sacc[kb] = mfma(kf, qf[s], sacc[kb]);
        }
    }

    __builtin_amdgcn_sched_barrier(0);
    // P = exp2(S*c - m_ref) with the current reference
    float p[2][16];
    float ts = 0.f;
    float negm = -mref;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float x = exp2_hw(__builtin_fmaf(sacc[kb][r], c, negm));
            if (MASK && key_of(kb, r, g) >= valid) x = 0.f;
            p[kb][r] = x;
            ts += x;
        }

    if (__any(!(ts <= RESCALE_LIMIT))) {
        // exact path: new reference = running max, rescale accumulators, recompute P
        float tmax = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float t = sacc[kb][r] * c;
                if (MASK && key_of(kb, r, g) >= valid) t = -INFINITY;
                tmax = fmaxf(tmax, t);
            }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float mnew = fmaxf(mref, tmax);
        const float alpha = exp2_hw(mref - mnew);
        lsum *= alpha;
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[b][r] *= alpha;
        mref = mnew;
        negm = -mnew;
        ts = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float x = exp2_hw(__builtin_fmaf(sacc[kb][r], c, negm));
                if (MASK && key_of(kb, r, g) >= valid) x = 0.f;
                p[kb][r] = x;
                ts += x;
            }
    }
    lsum += ts;

    // P^T fragments (BF16, round to nearest even)
    bf16x8 pb[4];
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
        for (int i = 0; i < 8; ++i) pb[h][i] = (bf16)p[h >> 1][8 * (h & 1) + i];

    __builtin_amdgcn_sched_barrier(0);
    // O^T += V^T_tile . P^T
    const char* vt = lds + K_BYTES;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int row = 32 * b + swap23(m);
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const bf16x8 vf = *reinterpret_cast<const bf16x8*>(vt + vt_off(row, 2 * h + g));
            oacc[b] = mfma(vf, pb[h], oacc[b]);
        }
    }
}

// One workgroup: query rows q0 .. q0+BM-1 of a sequence of n tokens whose rows are rs
// elements apart (Q/K/V/O point at the sequence's first row; L at its first LSE entry).
__device__ __forceinline__ void attn_block(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                                           const bf16* __restrict__ V, bf16* __restrict__ O,
                                           float* __restrict__ L, long rs, int n, int q0, float c) {
    __shared__ __attribute__((aligned(16))) char smem[2 * STAGE_BYTES];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int m = lane & 31, g = lane >> 5;

    const int qrow = q0 + w * QW + m;
    const bool qvalid = qrow < n;
    const int qr = min(qrow, n - 1);
    bf16x8 qf[8];
#pragma unroll
    for (int s = 0; s < 8; ++s)
        qf[s] = *reinterpret_cast<const bf16x8*>(Q + qr * rs + 16 * s + 8 * g);

    f32x16 oacc[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) oacc[b] = f32x16{};
    float mref = -INFINITY, lsum = 0.f;

    // full tiles in the loop, a ragged last tile (if any) peeled after it
    const int ntiles = (n + BN - 1) / BN;
    const int nfull = n / BN;
    Staged st;
    load_tile(st, K, V, rs, 0, n, tid);
    store_tile(st, smem, tid);
    __syncthreads();

    for (int j = 0; j < nfull; ++j) {
        const char* cur = smem + (j & 1) * STAGE_BYTES;
        const bool more = j + 1 < ntiles;
        if (more) load_tile(st, K, V, rs, (j + 1) * BN, n, tid);
        tile_step<false>(cur, qf, oacc, mref, lsum, c, BN, m, g);
        if (more) store_tile(st, smem + ((j + 1) & 1) * STAGE_BYTES, tid);
        __syncthreads();
    }
    if (nfull < ntiles)
        tile_step<true>(smem + (nfull & 1) * STAGE_BYTES, qf, oacc, mref, lsum, c, n - nfull * BN, m, g);

    const float ltot = lsum + __shfl_xor(lsum, 32);
    const float inv = 1.0f / ltot;
    if (qvalid) {
        bf16* orow = O + qrow * rs;
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                bf16x8 ov;
#pragma unroll
                for (int i = 0; i < 8; ++i) ov[i] = (bf16)(oacc[b][8 * hh + i] * inv);
                *reinterpret_cast<bf16x8*>(orow + 32 * b + 16 * hh + 8 * g) = ov;
            }
        if (L != nullptr && g == 0) L[qrow] = (mref + __log2f(ltot)) * LN2;
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

__global__ __launch_bounds__(NT, 2) void attn_fwd_dense_kernel(DenseArgs a) {
    const int bh = blockIdx.x / a.ntq, qt = blockIdx.x - bh * a.ntq;
    const long base = (long)bh * a.N * D;
    attn_block(a.q + base, a.k + base, a.v + base, a.o + base,
               a.lse ? a.lse + (long)bh * a.N : nullptr, D, a.N, qt * BM, a.c);
}

// Varlen schedule in the workspace: [0] entry count, then order[nseg] (segment ids, longest
// first), then entries (segment, query tile) in that order.
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

__global__ __launch_bounds__(1024) void build_varlen_schedule(const int32_t* __restrict__ cu,
                                                              int nseg, int T, char* ws) {
    __shared__ int chunk[1024];
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
    for (int r = r0; r < r1; ++r) sum += (seg_len(cu, order[r], T) + BM - 1) / BM;
    chunk[tid] = sum;
    __syncthreads();
    if (tid == 0) {
        int acc = 0;
        for (int i = 0; i < 1024; ++i) {
            const int v = chunk[i];
            chunk[i] = acc;
            acc += v;
        }
        *count = (int)min((long)acc, cap);   // malformed offsets cannot push readers past the list
    }
    __syncthreads();
    long off = chunk[tid];
    for (int r = r0; r < r1; ++r) {
        const int s = order[r];
        const int nt = (seg_len(cu, s, T) + BM - 1) / BM;
        for (int i = 0; i < nt; ++i)
            if (off + i < cap) list[off + i] = make_int2(s, i);
        off += nt;
    }
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

__global__ __launch_bounds__(NT, 2) void attn_fwd_varlen_kernel(VarlenArgs a) {
    const int e = blockIdx.x / a.H, h = blockIdx.x - e * a.H;
    if (e >= *reinterpret_cast<const int*>(a.ws)) return;
    const int2 t = reinterpret_cast<const int2*>(a.ws + ws_list_offset(a.nseg))[e];
    const int start = min(max(a.cu[t.x], 0), a.T);
    const int n = seg_len(a.cu, t.x, a.T);
    if (t.y * BM >= n) return;
    const long base = ((long)start * a.H + h) * D;
    attn_block(a.q + base, a.k + base, a.v + base, a.o + base,
               a.lse ? a.lse + (long)h * a.T + start : nullptr, (long)a.H * D, n, t.y * BM, a.c);
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

size_t varlen_workspace_bytes(int nseg, int total_tokens) {
    return ws_list_offset(nseg) + ws_align(sizeof(int2) * (size_t)max_entries(nseg, total_tokens));
}

hipError_t launch_varlen(const void* q, const void* k, const void* v, void* out, float* lse,
                         const int32_t* cu_seqlens, int nseg, int H, int total_tokens, float scale,
                         void* workspace, hipStream_t stream) {
    char* ws = static_cast<char*>(workspace);
    hipLaunchKernelGGL(build_varlen_schedule, dim3(1), dim3(1024), 0, stream, cu_seqlens, nseg,
                       total_tokens, ws);
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
