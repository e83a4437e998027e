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
// Work decomposition: one workgroup = 8 waves = 256 query rows of one (batch, head) or
// (segment, head); each wave owns 32 query rows for the whole key loop. Per 64-key tile:
//
//   S^T[key, q] = K_tile . Q_w^T      v_mfma_f32_32x32x16_bf16, A = K rows from LDS,
//                                     B = the wave's Q rows, held in VGPRs all along
//   P = exp2(S*c - m_ref)             c = scale*log2(e); FP32 VALU
//   O^T[dv, q] += V^T_tile . P^T      A = V^T from LDS by transposing reads, B = P (BF16)
//                                     straight from the S^T accumulator registers
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
// reads 4 dims of key row r and lane j receives dim j of the 4 rows. Two LDS stages: the
// loads of tile j+1 are in flight while tile j is computed; one barrier per tile.
//
// Schedule inside a tile (per wave), so the exp work issues while the matrix core is busy:
//   QK(keys 0-31) | QK(keys 32-63) + exp(0-31) | PV(0-31) + exp(32-63) | PV(32-63)
// every MFMA is followed by its share of exp work and the LDS reads one region ahead.
// Two waves share each SIMD (w and w + NW/2). Issue arbitration favours the older one, which
// would finish its tile early and wait at the barrier while the younger runs alone; the
// younger wave therefore runs at raised priority (s_setprio) until its last exp block.
//
// Row statistics: m_ref (per row, in log2 units of the scaled logit) and l (per-lane
// partial). The common path computes P with the current m_ref and only checks that no
// lane's partial tile sum exceeds 2^8 (then no probability exceeds 2^8 and FP32/BF16 stay
// exact in relative terms); otherwise (always on a row's first tile, where m_ref = -inf)
// the wave recomputes S from LDS and takes the exact path: true row max, rescale of O and
// l, recompute of P. The result is the same softmax; only the reference the BF16
// probabilities are relative to differs, which BF16 rounding (relative) does not see.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "attn_launch.h"

namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int D = 128;          // head dim
constexpr int BN = 64;          // keys per tile
constexpr int QW = 32;          // query rows per wave
constexpr int NW = 8;           // waves per workgroup (two per SIMD)
constexpr int BM = NW * QW;     // query rows per workgroup
constexpr int NT = NW * 64;     // threads per workgroup

constexpr int ROW_BYTES = D * 2;                 // one key row in LDS
constexpr int K_BYTES = BN * ROW_BYTES;          // 16 KiB
constexpr int STAGE_BYTES = 2 * K_BYTES;         // K then V
constexpr int LOADS_PER_WAVE = K_BYTES / 1024 / NW;   // 1 KiB per buffer-load instruction
constexpr int BUF_FLAGS = 0x00020000;            // raw buffer, 32-bit data format
constexpr float RESCALE_LIMIT = 256.0f;
constexpr float LN2 = 0.693147180559945309f;

static_assert(LOADS_PER_WAVE * NW * 1024 == K_BYTES, "tile load split");

__device__ __forceinline__ int swap23(int m) {
    return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// LDS layout of a K tile: key row r, 16-byte chunk c (dims 8c..8c+7) at r*256 + 16*(c ^ (r%16)).
__device__ __forceinline__ int k_swz(int r) { return r & 15; }
// LDS layout of a V tile: key row r, chunk c at r*256 + 16*(c ^ v_swz(r)); chosen so that
// the transposing reads (4 key rows x 2 chunks per 16 lanes) hit 32 distinct bank pairs.
__device__ __forceinline__ int v_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const bf16* base, long bytes) {
    const int nbytes = bytes > 0x7fffffffL ? 0x7fffffff : (bytes < 0 ? 0 : (int)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(base), (short)0, nbytes, BUF_FLAGS);
}

// Per-lane constants of one workgroup-slot of the kernel.
struct Lane {
    int m, g;
    int kld[8];          // LDS byte offset of K fragment for d-step s (key block 0)
    int vld[4][2];       // LDS byte offset of the transposing V read for dim block b, half t
    int koff[LOADS_PER_WAVE], voff[LOADS_PER_WAVE];   // global byte offsets within a tile
};

__device__ __forceinline__ void init_lane(Lane& L, int tid, int rs_bytes) {
    const int lane = tid & 63, w = tid >> 6;
    L.m = lane & 31;
    L.g = lane >> 5;
    const int row = swap23(L.m);
#pragma unroll
    for (int s = 0; s < 8; ++s) L.kld[s] = row * ROW_BYTES + (((2 * s + L.g) ^ k_swz(row)) << 4);
    const int j = lane & 15, r = j >> 2, c4 = j & 3, mh = (lane >> 4) & 1;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int vrow = 8 * L.g + 4 * t + r;   // + 16h, which does not change v_swz
            const int chunk = 4 * b + 2 * mh + (c4 & 1);
            L.vld[b][t] = vrow * ROW_BYTES + ((chunk ^ v_swz(vrow)) << 4) + ((c4 >> 1) << 3);
        }
#pragma unroll
    for (int i = 0; i < LOADS_PER_WAVE; ++i) {
        const int slot_row = 4 * (LOADS_PER_WAVE * w + i) + (lane >> 4);
        const int slot_chunk = lane & 15;
        L.koff[i] = slot_row * rs_bytes + ((slot_chunk ^ k_swz(slot_row)) << 4);
        L.voff[i] = slot_row * rs_bytes + ((slot_chunk ^ v_swz(slot_row)) << 4);
    }
}

// Issue the buffer->LDS loads of key tile `tile` (this wave's quarter of K and of V).
__device__ __forceinline__ void load_tile(const Lane& L, char* stage, const bf16* K, const bf16* V,
                                          long rs_bytes, long seq_bytes, int tile, int w) {
    const long skip = (long)tile * BN * rs_bytes;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc((const bf16*)((const char*)K + skip), seq_bytes - skip);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc((const bf16*)((const char*)V + skip), seq_bytes - skip);
#pragma unroll
    for (int i = 0; i < LOADS_PER_WAVE; ++i) {
        char* dk = stage + (LOADS_PER_WAVE * w + i) * 1024;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)dk, 16, L.koff[i], 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(dk + K_BYTES), 16, L.voff[i], 0, 0, 0);
    }
}

__device__ __forceinline__ bf16x8 lds_b128(const char* p) { return *reinterpret_cast<const bf16x8*>(p); }

__device__ __forceinline__ bf16x8 lds_vt(const char* p0, const char* p1) {
    const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p0);
    const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p1);
    const s16x8 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, ab);
}

// Key (within the tile) held by register r of lane group g in S^T accumulator block kb.
__device__ __forceinline__ int key_of(int kb, int r, int g) {
    return 32 * kb + 16 * (r >> 3) + 8 * g + (r & 7);
}

// S^T block kb (keys 32kb..32kb+31 of the tile) = K_block . Q^T: 8 MFMAs.
__device__ __forceinline__ f32x16 qk_block(const char* __restrict__ kt, const Lane& L,
                                           const bf16x8 (&qf)[8], int kb) {
    f32x16 acc = f32x16{};
#pragma unroll
    for (int s = 0; s < 8; ++s) acc = mfma(lds_b128(kt + L.kld[s] + kb * 32 * ROW_BYTES), qf[s], acc);
    return acc;
}

// In place: p = exp2(S*c - m_ref) for one 32-key block; returns the lane's partial sum.
template <bool MASK>
__device__ __forceinline__ float exp_block(f32x16& sb, float c, float negm, int valid, int kb, int g) {
    float ts[4] = {0.f, 0.f, 0.f, 0.f};   // independent partial sums: no serial add chain
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        float x = exp2_hw(__builtin_fmaf(sb[r], c, negm));
        if (MASK && key_of(kb, r, g) >= valid) x = 0.f;
        sb[r] = x;
        ts[r & 3] += x;
    }
    return (ts[0] + ts[1]) + (ts[2] + ts[3]);
}

// Exact path for one 32-key block (rare): recompute its scores from LDS, move the
// reference to the running max, rescale O and l, recompute the probabilities.
template <bool MASK>
__device__ __forceinline__ float exact_block(const char* __restrict__ kt, const Lane& L,
                                                       const bf16x8 (&qf)[8], f32x16& sb,
                                                       f32x16 (&oacc)[4], float& mref, float& lsum,
                                                       float c, int valid, int kb) {
    sb = qk_block(kt, L, qf, kb);
    float tmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        float t = sb[r] * c;
        if (MASK && key_of(kb, r, L.g) >= valid) t = -INFINITY;
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
    return exp_block<MASK>(sb, c, -mnew, valid, kb, L.g);
}

__device__ __forceinline__ void to_bf16(const f32x16& sb, bf16x8 (&pb)[2]) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int i = 0; i < 8; ++i) pb[hh][i] = (bf16)sb[8 * hh + i];
}

// O^T += V^T . P^T over the 32 keys of block kb: 8 MFMAs (4 dim blocks x 2 key steps).
__device__ __forceinline__ void pv_block(const char* __restrict__ vt, const Lane& L,
                                         const bf16x8 (&pb)[2], f32x16 (&oacc)[4], int kb) {
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int h = 2 * kb + hh;
            oacc[b] = mfma(lds_vt(vt + L.vld[b][0] + h * 16 * ROW_BYTES, vt + L.vld[b][1] + h * 16 * ROW_BYTES),
                           pb[hh], oacc[b]);
        }
}

// Two probabilities of one 32-key block, in place, accumulating the lane's partial sums.
template <bool MASK>
__device__ __forceinline__ void exp_pair(f32x16& sb, float c, float negm, int valid, int kb, int g,
                                         int r0, float (&ts)[4]) {
#pragma unroll
    for (int r = r0; r < r0 + 2; ++r) {
        float x = exp2_hw(__builtin_fmaf(sb[r], c, negm));
        if (MASK && key_of(kb, r, g) >= valid) x = 0.f;
        sb[r] = x;
        ts[r & 3] += x;
    }
}

__device__ __forceinline__ bf16x8 vt_frag(const char* __restrict__ vt, const Lane& L, int b, int h) {
    return lds_vt(vt + L.vld[b][0] + h * 16 * ROW_BYTES, vt + L.vld[b][1] + h * 16 * ROW_BYTES);
}

// One 64-key tile, software-pipelined inside the wave so that the exp work of one 32-key
// block issues while the matrix core runs the MFMAs of the other, and every LDS fragment
// is read one region ahead of its MFMA:
//   QK(b0) [+ read K b1] | QK(b1) + exp(b0) [+ read V b0] | check b0 |
//   PV(b0) + exp(b1) [+ read V b1] | check b1 | PV(b1)
// Every MFMA is followed by its share of VALU and LDS work; sched_barrier keeps that order.
template <bool MASK>
__device__ __forceinline__ void tile_step(const char* __restrict__ stage, const Lane& L,
                                          const bf16x8 (&qf)[8], f32x16 (&oacc)[4], float& mref,
                                          float& lsum, float c, int valid, bool young) {
    const char* vt = stage + K_BYTES;
    bf16x8 kf0[8], kf1[8], vf0[8], vf1[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) kf0[s] = lds_b128(stage + L.kld[s]);
    __builtin_amdgcn_sched_barrier(0);

    // QK(b0), reading K b1
    f32x16 s0 = f32x16{};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        s0 = mfma(kf0[s], qf[s], s0);
        kf1[s] = lds_b128(stage + L.kld[s] + 32 * ROW_BYTES);
        __builtin_amdgcn_sched_barrier(0);
    }

    // QK(b1) beside exp(b0), reading V for PV(b0)
    float negm = -mref;
    float t0[4] = {0.f, 0.f, 0.f, 0.f};
    f32x16 s1 = f32x16{};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        s1 = mfma(kf1[s], qf[s], s1);
        exp_pair<MASK>(s0, c, negm, valid, 0, L.g, 2 * s, t0);
        vf0[s] = vt_frag(vt, L, s & 3, s >> 2);
        __builtin_amdgcn_sched_barrier(0);
    }
    float ts0 = (t0[0] + t0[1]) + (t0[2] + t0[3]);
    if (__any(!(ts0 <= RESCALE_LIMIT))) ts0 = exact_block<MASK>(stage, L, qf, s0, oacc, mref, lsum, c, valid, 0);
    lsum += ts0;
    bf16x8 p0[2];
    to_bf16(s0, p0);
    __builtin_amdgcn_sched_barrier(0);

    // PV(b0) beside exp(b1), reading V for PV(b1)
    negm = -mref;
    float t1[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        oacc[i & 3] = mfma(vf0[i], p0[i >> 2], oacc[i & 3]);
        exp_pair<MASK>(s1, c, negm, valid, 1, L.g, 2 * i, t1);
        vf1[i] = vt_frag(vt, L, i & 3, 2 + (i >> 2));
        __builtin_amdgcn_sched_barrier(0);
    }
    // the younger wave of the SIMD drops back to normal priority (raised at the tile start)
    if (young) __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
    float ts1 = (t1[0] + t1[1]) + (t1[2] + t1[3]);
    if (__any(!(ts1 <= RESCALE_LIMIT))) ts1 = exact_block<MASK>(stage, L, qf, s1, oacc, mref, lsum, c, valid, 1);
    lsum += ts1;
    bf16x8 p1[2];
    to_bf16(s1, p1);
    __builtin_amdgcn_sched_barrier(0);

    // PV(b1)
#pragma unroll
    for (int i = 0; i < 8; ++i) oacc[i & 3] = mfma(vf1[i], p1[i >> 2], oacc[i & 3]);
}

// One full-tile iteration on LDS stage STAGE: wait for tile j, start tile j+1, compute j.
template <int STAGE>
__device__ __forceinline__ void full_step(char* smem, const Lane& L, const bf16* K, const bf16* V,
                                          long rs_bytes, long seq_bytes, int j, int ntiles, int w,
                                          const bf16x8 (&qf)[8], f32x16 (&oacc)[4], float& mref,
                                          float& lsum, float c) {
    // Waves w and w + NW/2 share a SIMD. The older one wins issue arbitration and would run
    // ahead, then idle at the barrier while the younger finishes alone; raising the younger
    // wave's priority for the first three quarters of the tile keeps the two in step.
    const bool young = w >= NW / 2;
    wait_vmem();
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    if (young) __builtin_amdgcn_s_setprio(1);
    __builtin_amdgcn_sched_barrier(0);
    if (j + 1 < ntiles) load_tile(L, smem + (1 - STAGE) * STAGE_BYTES, K, V, rs_bytes, seq_bytes, j + 1, w);
    tile_step<false>(smem + STAGE * STAGE_BYTES, L, qf, oacc, mref, lsum, c, BN, young);
}

// Row stride (floats) of a partial result: 128 unnormalised O values, then m_ref and l.
constexpr int PART_STRIDE = 132;
constexpr size_t PART_BYTES = sizeof(float) * PART_STRIDE * BM;   // one workgroup's rows

// One workgroup: query rows q0 .. q0+BM-1 of a sequence of n tokens whose rows are rs
// elements apart (Q/K/V/O point at the sequence's first row; LSE at its first entry), over
// key tiles kt0 .. kt1-1. With part == nullptr the range is all keys and O (and LSE) get the
// final rows; otherwise the workgroup's unnormalised O, m_ref and l go to part (PART_STRIDE
// floats per row) for a later merge.
__device__ __forceinline__ void attn_block_range(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                                                 const bf16* __restrict__ V, bf16* __restrict__ O,
                                                 float* __restrict__ LSE, long rs, int n, int q0, float c,
                                                 int kt0, int kt1, float* __restrict__ part) {
    __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE_BYTES];
    const int tid = threadIdx.x, w = tid >> 6;
    const long rs_bytes = rs * 2;
    const long seq_bytes = (long)n * rs_bytes;
    Lane L;
    init_lane(L, tid, (int)rs_bytes);
    const int ntiles = kt1;
    const int nfull = min(n / BN, kt1);
    load_tile(L, smem, K, V, rs_bytes, seq_bytes, kt0, w);

    const int qrow = q0 + w * QW + L.m;
    const bool qvalid = qrow < n;
    const int qr = min(qrow, n - 1);
    bf16x8 qf[8];
#pragma unroll
    for (int s = 0; s < 8; ++s)
        qf[s] = *reinterpret_cast<const bf16x8*>(Q + qr * rs + 16 * s + 8 * L.g);

    f32x16 oacc[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) oacc[b] = f32x16{};
    float mref = -INFINITY, lsum = 0.f;

    // LDS stage of tile j is (j - kt0) & 1: tile kt0 went to stage 0.
    int j = kt0;
    for (; j + 1 < nfull; j += 2) {
        full_step<0>(smem, L, K, V, rs_bytes, seq_bytes, j, ntiles, w, qf, oacc, mref, lsum, c);
        full_step<1>(smem, L, K, V, rs_bytes, seq_bytes, j + 1, ntiles, w, qf, oacc, mref, lsum, c);
    }
    if (j < nfull) {
        full_step<0>(smem, L, K, V, rs_bytes, seq_bytes, j, ntiles, w, qf, oacc, mref, lsum, c);
        ++j;
    }
    if (j < ntiles) {   // ragged last tile, keys >= n masked (and read as zeros)
        wait_vmem();
        __syncthreads();
        tile_step<true>(smem + ((j - kt0) & 1) * STAGE_BYTES, L, qf, oacc, mref, lsum, c, n - j * BN, false);
    }

    const float ltot = lsum + __shfl_xor(lsum, 32);
    if (part != nullptr) {
        if (qvalid) {
            float* prow = part + (long)(qrow - q0) * PART_STRIDE;
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    float4* d = reinterpret_cast<float4*>(prow + 32 * b + 16 * hh + 8 * L.g);
                    d[0] = make_float4(oacc[b][8 * hh + 0], oacc[b][8 * hh + 1], oacc[b][8 * hh + 2], oacc[b][8 * hh + 3]);
                    d[1] = make_float4(oacc[b][8 * hh + 4], oacc[b][8 * hh + 5], oacc[b][8 * hh + 6], oacc[b][8 * hh + 7]);
                }
            if (L.g == 0) {
                prow[128] = mref;
                prow[129] = ltot;
            }
        }
        return;
    }
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
                *reinterpret_cast<bf16x8*>(orow + 32 * b + 16 * hh + 8 * L.g) = ov;
            }
        if (LSE != nullptr && L.g == 0) LSE[qrow] = (mref + __log2f(ltot)) * LN2;
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

__device__ __forceinline__ void attn_block(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                                           const bf16* __restrict__ V, bf16* __restrict__ O,
                                           float* __restrict__ LSE, long rs, int n, int q0, float c) {
    attn_block_range(Q, K, V, O, LSE, rs, n, q0, c, 0, (n + BN - 1) / BN, nullptr);
}

__global__ __launch_bounds__(NT, NW / 4) void attn_fwd_dense_kernel(DenseArgs a) {
    const int bh = blockIdx.x / a.ntq, qt = blockIdx.x - bh * a.ntq;
    const long base = (long)bh * a.N * D;
    attn_block(a.q + base, a.k + base, a.v + base, a.o + base,
               a.lse ? a.lse + (long)bh * a.N : nullptr, D, a.N, qt * BM, a.c);
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

__global__ __launch_bounds__(NT, NW / 4) void attn_fwd_dense_split_kernel(DenseArgs a, SplitArgs sp) {
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
        attn_block_range(a.q + base, a.k + base, a.v + base, a.o + base,
                         a.lse ? a.lse + (long)bh * a.N : nullptr, D, a.N, qt * BM, a.c, (int)t0, (int)t1, part);
    }
}

// One block per (cut query tile, 16 rows): combines the tile's partial results,
// O = sum_p 2^(m_p - M) O_p / sum_p 2^(m_p - M) l_p with M = max_p m_p, LSE = (M + log2 l) ln 2.
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
    float l = 0.f;
    for (int g = g0; g <= g1; ++g) {
        const int slot = 2 * g + (share_begin(sp, g) / sp.ntk == i ? 0 : 1);
        const float* prow = sp.part + (size_t)slot * (PART_BYTES / sizeof(float)) + (size_t)r * PART_STRIDE;
        const float wgt = exp2_hw(prow[128] - M);
        l += wgt * prow[129];
        const float4 x0 = reinterpret_cast<const float4*>(prow + 8 * k)[0];
        const float4 x1 = reinterpret_cast<const float4*>(prow + 8 * k)[1];
        acc[0] += wgt * x0.x; acc[1] += wgt * x0.y; acc[2] += wgt * x0.z; acc[3] += wgt * x0.w;
        acc[4] += wgt * x1.x; acc[5] += wgt * x1.y; acc[6] += wgt * x1.z; acc[7] += wgt * x1.w;
    }
    const float inv = 1.0f / l;
    bf16x8 ov;
#pragma unroll
    for (int e = 0; e < 8; ++e) ov[e] = (bf16)(acc[e] * inv);
    const long base = (long)bh * a.N * D;
    *reinterpret_cast<bf16x8*>(a.o + base + (long)row * D + 8 * k) = ov;
    if (a.lse != nullptr && k == 0) a.lse[(long)bh * a.N + row] = (M + __log2f(l)) * LN2;
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

__global__ __launch_bounds__(NT, NW / 4) void attn_fwd_varlen_kernel(VarlenArgs a) {
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
    return cus;   // one 512-thread workgroup per compute unit (VGPR-bound)
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
