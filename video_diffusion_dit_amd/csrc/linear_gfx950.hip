// SANA-Video linear attention for CDNA4 (gfx950): ReLU-feature-map attention with rotated
// Q/K in the numerator and un-rotated Q/K in the normaliser, per (batch, head):
//
//   ksum  = sum_m k_m                     den_n = q_n . ksum + eps   (eps = 1e-15)
//   kv    = sum_m v_m k_rot_m^T  [d x d]  out_n = (kv q_rot_n) / den_n
//
// Source: page "PR #35728 report", key source excerpts: sana_video.py forward (normaliser
// 1 / (K.sum(-1)^T Q + 1e-15) from the un-rotated K and Q, then (V K_rot^T) Q_rot times the
// normaliser, output flattened back to [B, N, H*D]) and the site file
// try_sana_video_linear_attention (first product: BF16 inputs, FP32 accumulation and
// output; second product in FP32).
//
// Inputs q, k, q_rot, k_rot, v and the output are BF16 rows in the token-major layout the
// QKV projection writes, [B, N, H, 128]. Three kernels:
//   linear_kv_partial_kernel  one workgroup per (b, h, chunk of tokens): the chunk's
//       kv (v_mfma_f32_32x32x16_bf16, FP32 accumulation) and ksum (FP32 VALU) into the
//       workspace. V and K_rot tiles go through LDS; transposing LDS reads
//       (ds_read_b64_tr_b16) give each lane 8 consecutive tokens of one dim, the MFMA's
//       operand layout for both A = V^T and B = K_rot.
//   linear_kv_reduce_kernel   sums the chunk partials in a fixed order (deterministic) and
//       splits kv exactly into three BF16 terms. The chunk (a multiple of 64 tokens, 256 to
//       4096) is the shortest that lets the kv pass's B*H*chunks workgroups fill whole rounds
//       of the device's resident workgroups (three per compute unit): one round where 4096-token
//       chunks suffice, else the fewest rounds that allow them. So calls with few heads (one
//       GPU's share of a head-sharded call) still fill the compute units, and no round runs
//       part-empty; the chunk depends on B*H, N and the device's compute-unit count.
//   linear_out_kernel         one workgroup per (b, h, 1024 tokens): out = kv q_rot / den;
//       each wave keeps 32 rows of kv in registers, q_rot arrives in LDS by buffer->LDS loads.
//       The FP32 product runs on the BF16 matrix cores: kv = hi + mid + lo with three BF16
//       terms (8 bits each, together every bit of the FP32 value), q_rot is BF16 exactly,
//       so each of the three MFMA products is exact and the accumulation is FP32, the same
//       arithmetic as an FP32 GEMM up to summation order.
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
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int D = 128;
constexpr int NT = 256;              // threads per workgroup (4 waves)
constexpr int TILE = 64;             // tokens per LDS tile in the kv pass
constexpr int KV_CHUNK_MAX = 4096;   // tokens per workgroup in the kv pass (multiples of TILE)
constexpr int KV_CHUNK_MIN = 256;    // shorter chunks pay their partial write and setup more often
constexpr int KV_PER_CU = 3;         // kv-pass workgroups resident per compute unit (LDS bound)
constexpr int ROW = D * 2 + 32;      // LDS row stride in bytes (padded: 8-bank shift per row)
constexpr int KV_TERMS = 3;          // BF16 terms of the FP32 kv in the output pass
#define LIN_OUT_SUB 128              // tokens per sub-block of the output pass (a multiple of 64)
constexpr int OUT_SUB = LIN_OUT_SUB;
constexpr int OUT_SUBS = 1024 / OUT_SUB;   // sub-blocks per workgroup
constexpr int RPW = OUT_SUB / 4;           // rows of a sub-block each wave stages, normalises, stores
constexpr int NI = RPW / 4;                // instructions for them (four rows each)
constexpr int OUT_TOK = OUT_SUB * OUT_SUBS;

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 8 consecutive tokens (4 from each transposing read) of one dim from a [token][dim] LDS tile.
__device__ __forceinline__ bf16x8 lds_tokens8(const char* p0, const char* p1) {
    const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p0);
    const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p1);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

struct LinearArgs {
    const bf16* q;
    const bf16* k;
    const bf16* qr;
    const bf16* kr;
    const bf16* v;
    bf16* out;
    float* part;      // [BH][S][D*D + D] chunk partials (kv then ksum)
    bf16* terms;      // [BH][KV_TERMS][D][D] kv = hi + mid + lo, BF16
    float* ksum;      // [BH][D]
    int N, H, S;      // tokens, heads, chunks per sequence
    int chunk;        // tokens per chunk
    float eps;
};

// ---------------------------------------------------------------- kv and ksum of a chunk
// Waves in a 2 x 2 grid: wave (wi, wj) owns the 32x32 output blocks (2wi + a, 2wj + b).
__global__ __launch_bounds__(NT) void linear_kv_partial_kernel(LinearArgs a) {
    __shared__ __attribute__((aligned(16))) char smem[2 * TILE * ROW + NT * 8 * 4];
    char* vt = smem;
    char* kt = smem + TILE * ROW;
    float* red = reinterpret_cast<float*>(smem + 2 * TILE * ROW);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wi = w >> 1, wj = w & 1;
    // heads fastest: the workgroups running together read the same token rows of every head
    // (whole 4 KiB token rows of the [B, N, H, 128] tensors instead of one 256-byte slice each)
    const int nbh = gridDim.x / a.S;
    const int s = blockIdx.x / nbh, bh = blockIdx.x - s * nbh;
    const int b = bh / a.H, h = bh - b * a.H;
    const long row_stride = (long)a.H * D;                       // elements between tokens
    const long base = ((long)b * a.N * a.H + h) * D;             // (b, token 0, h)
    const int m0 = s * a.chunk, m1 = min(a.N, m0 + a.chunk);

    // loads: thread -> (row tid/16 (+16, +32, +48), 8-dim chunk tid%16)
    const int lr = tid >> 4, lc = tid & 15;
    // transposing reads: lane L, read t -> token row 8g + 4t + r, dims d0 + 16*((L/16)&1) + 4c
    const int g = lane >> 5, r = (lane & 15) >> 2, c = lane & 3, half = (lane >> 4) & 1;
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
    float ks[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

    for (int t0 = m0; t0 < m1; t0 += TILE) {
        // stage V and K_rot rows t0..t0+63 (zeros past m1), sum K rows
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int row = lr + 16 * u, tok = t0 + row;
            u32x4 vv = {0u, 0u, 0u, 0u}, kk = {0u, 0u, 0u, 0u}, k0 = {0u, 0u, 0u, 0u};
            if (tok < m1) {
                const long off = base + (long)tok * row_stride + 8 * lc;
                vv = *reinterpret_cast<const u32x4*>(a.v + off);
                kk = *reinterpret_cast<const u32x4*>(a.kr + off);
                k0 = *reinterpret_cast<const u32x4*>(a.k + off);
            }
            *reinterpret_cast<u32x4*>(vt + row * ROW + 16 * lc) = vv;
            *reinterpret_cast<u32x4*>(kt + row * ROW + 16 * lc) = kk;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ks[2 * e] += __uint_as_float(k0[e] << 16);
                ks[2 * e + 1] += __uint_as_float(k0[e] & 0xffff0000u);
            }
        }
        __syncthreads();
#pragma unroll
        for (int st = 0; st < TILE / 16; ++st) {          // 16-token MFMA steps
            bf16x8 fa[2], fb[2];
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const int di = 32 * (2 * wi + x) + 16 * half + 4 * c;
                const int dj = 32 * (2 * wj + x) + 16 * half + 4 * c;
                const int tr0 = 16 * st + 8 * g + r, tr1 = tr0 + 4;
                fa[x] = lds_tokens8(vt + tr0 * ROW + 2 * di, vt + tr1 * ROW + 2 * di);
                fb[x] = lds_tokens8(kt + tr0 * ROW + 2 * dj, kt + tr1 * ROW + 2 * dj);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) acc[i][j] = mfma(fa[i], fb[j], acc[i][j]);
        }
        __syncthreads();
    }

    float* pk = a.part + ((long)bh * a.S + s) * (D * D + D);
    // C layout: lane (column n = lane%32, g), register q -> row 8(q/4) + 4g + q%4
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = 32 * (2 * wj + j) + (lane & 31);
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int rowi = 32 * (2 * wi + i) + 8 * (q >> 2) + 4 * g + (q & 3);
                pk[rowi * D + col] = acc[i][j][q];
            }
        }
    // ksum: 16 threads (rows lr) share each 8-dim chunk lc
#pragma unroll
    for (int e = 0; e < 8; ++e) red[tid * 8 + e] = ks[e];
    __syncthreads();
    if (tid < D) {
        const int ch = tid >> 3, e = tid & 7;
        float sum = 0.f;
        for (int rr = 0; rr < 16; ++rr) sum += red[(rr * 16 + ch) * 8 + e];
        pk[D * D + tid] = sum;
    }
}

// ---------------------------------------------------------------- chunk partials -> kv, ksum
// A partial is (D*D + D) FP32 values, read as groups of 4 (16-byte loads). RS threads share a
// group: thread sl sums chunks sl, sl + RS, ... in order, then the RS sums are added in sl
// order (a fixed order, so the result is deterministic). A wave reads whole 256-byte rows of
// 64 / RG partials at once, so RS chunks are in flight per group.
#ifndef LIN_REDUCE_SPLIT
#define LIN_REDUCE_SPLIT 16
#endif
constexpr int RS = LIN_REDUCE_SPLIT;
constexpr int RG = NT / RS;                      // 4-value groups per workgroup
constexpr int PART_GROUPS = (D * D + D) / 4;
constexpr int REDUCE_BLOCKS = (PART_GROUPS + RG - 1) / RG;
static_assert((D * D + D) % 4 == 0 && RG >= 16 && 64 % RG == 0, "reduce layout");

__device__ __forceinline__ void split_terms(float sum, bf16* t) {
    // exact split of the FP32 sum into three BF16 terms (8 significant bits each)
    const bf16 hi = (bf16)sum;
    const float r1 = sum - (float)hi;
    const bf16 mid = (bf16)r1;
    const bf16 lo = (bf16)(r1 - (float)mid);
    t[0] = hi;
    t[D * D] = mid;
    t[2 * D * D] = lo;
}

__global__ __launch_bounds__(NT) void linear_kv_reduce_kernel(LinearArgs a) {
    __shared__ float4 red[RS][RG];
    const int bh = blockIdx.x / REDUCE_BLOCKS, blk = blockIdx.x - bh * REDUCE_BLOCKS;
    const int gl = threadIdx.x % RG, sl = threadIdx.x / RG;
    const int grp = blk * RG + gl;
    float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
    if (grp < PART_GROUPS) {
        const float4* p = reinterpret_cast<const float4*>(a.part + (long)bh * a.S * (D * D + D)) + grp;
        for (int s = sl; s < a.S; s += RS) {
            const float4 x = p[(long)s * PART_GROUPS];
            sum.x += x.x;
            sum.y += x.y;
            sum.z += x.z;
            sum.w += x.w;
        }
    }
    red[sl][gl] = sum;
    __syncthreads();
    if (sl != 0 || grp >= PART_GROUPS) return;
    for (int r = 1; r < RS; ++r) {
        const float4 x = red[r][gl];
        sum.x += x.x;
        sum.y += x.y;
        sum.z += x.z;
        sum.w += x.w;
    }
    const float v[4] = {sum.x, sum.y, sum.z, sum.w};
    const int e0 = 4 * grp;                      // D*D is a multiple of 4: a group is all kv or all ksum
    if (e0 < D * D) {
        bf16* t = a.terms + (long)bh * KV_TERMS * D * D + e0;
#pragma unroll
        for (int i = 0; i < 4; ++i) split_terms(v[i], t + i);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) a.ksum[(long)bh * D + e0 - D * D + i] = v[i];
    }
}

// ---------------------------------------------------------------- out = kv q_rot / den
// A workgroup takes OUT_TOK tokens of one (b, h) in sub-blocks of OUT_SUB tokens; two
// workgroups share a compute unit (64 KiB of LDS and at most 256 registers per lane each), so
// one computes while the other waits on memory. Wave w owns output dims 32w .. 32w+31: its A
// fragments (rows 32w.. of the three kv terms, all 128 dims) stay in registers for the whole
// workgroup. q_rot of a sub-block goes from HBM straight into LDS (buffer->LDS loads: each
// instruction moves four whole token rows, 1 KiB, fully coalesced), double-buffered and
// XOR-swizzled (row r, 16-byte chunk c at r*256 + 16*(c ^ (r % 16))), and every wave reads the
// B fragments of all OUT_SUB tokens from it. The normaliser of a token: 16 lanes load its q row
// (one 16-byte chunk each, coalesced), dot it with ksum and add across the 16 lanes; wave w
// does tokens RPW*w .. RPW*w+RPW-1 of the next sub-block into LDS while its MFMAs run. The
// grid runs heads fastest, so the workgroups in flight read whole 4 KiB token rows of the
// token-major tensors together.
constexpr int QROW = D * 2;                  // LDS bytes per staged q_rot row (swizzled, no pad)
constexpr int QBUF = OUT_SUB * QROW;         // one sub-block of q_rot
// s_waitcnt vmcnt(0) (expcnt and lgkmcnt at their maxima) as a builtin, which the compiler's
// wait-count bookkeeping sees (an asm statement would be opaque to it)
constexpr int WAIT_VMCNT0 = 0x0F70;

constexpr unsigned BUF_FLAGS = 0x00020000;   // raw buffer, 32-bit data format

// Buffer resource over tokens n .. N-1 of the (b, h) slice of a token-major [B, N, H, 128]
// tensor (p points at token n; token n + r at byte r * row_stride * 2). Every load below puts
// its whole offset in the VGPR (soffset 0), which the bounds check covers: rows past the last
// token read zeros.
__device__ __forceinline__ u32x4 rows_rsrc(const bf16* p, int rows, long row_stride) {
    const uint64_t a = (uint64_t)(uintptr_t)p;
    return u32x4{(unsigned)a, (unsigned)(a >> 32) & 0xffffu, (unsigned)(((long)(rows - 1) * row_stride + D) * 2),
                 BUF_FLAGS};
}

// Per-lane byte offsets of the q_rot staging: instruction i of wave w moves rows
// RPW*w + 4i .. +3 (lane: row 4i + lane/16, LDS slot lane%16, global chunk slot ^ row%16).
// The swizzle repeats every 4 instructions: offset = v[i % 4] + (i / 4) * 16 rows... written
// as v[i % 4] + i' * step4 with the row step added in the asm.
struct StageOffsets {
    unsigned v[4];
};

// The lane index passed through an empty asm: values derived from it are recomputed where
// they are used (a few VALU ops) instead of being hoisted out of the sub-block loop, where
// they would not fit in registers and would be spilled.
__device__ __forceinline__ int fresh_lane(int lane) {
    asm volatile("" : "+v"(lane));
    return lane;
}

__device__ __forceinline__ StageOffsets stage_offsets(long row_stride, int w, int lane_in) {
    const int lane = fresh_lane(lane_in);
    StageOffsets o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * i + (lane >> 4);           // row within a group of 16 (swizzle key)
        const int c = (lane & 15) ^ (r & 15);
        o.v[i] = (unsigned)((((long)(RPW * w + 4 * i + (lane >> 4))) * row_stride + 8 * c) * 2);
    }
    return o;
}

// q_rot rows of the resource (one sub-block) into LDS buffer dst. Instruction i = 4m + k uses
// offset v[k] + m * step16 (16 rows), formed by one v_add in the asm. One asm block, so the
// compiler puts no wait for these LDS writes in front of unrelated LDS reads: the caller waits
// (vmcnt(0), then a barrier) before any wave reads dst. M0 (the LDS destination) is saved and
// restored around it.
__device__ __forceinline__ void stage_qrot(u32x4 rsrc, unsigned step16, const StageOffsets& o, char* dst, int w) {
    const unsigned lds = (unsigned)(uintptr_t)(__attribute__((address_space(3))) char*)(dst + RPW * w * QROW);
    unsigned saved, st, t;
#define STAGE_LOAD(k) "v_add_u32 %[t], %[st], %[o" #k "]\n" "buffer_load_dwordx4 %[t], %[rs], 0 offen lds\n" \
                      "s_add_u32 m0, m0, 1024\n" "s_nop 0\n"
#define STAGE_GROUP STAGE_LOAD(0) STAGE_LOAD(1) STAGE_LOAD(2) STAGE_LOAD(3) "s_add_u32 %[st], %[st], %[s16]\n"
    asm volatile(
        "s_mov_b32 %[sv], m0\n"
        "s_mov_b32 m0, %[l]\n"
        "s_mov_b32 %[st], 0\n"
        "s_nop 0\n"
        STAGE_GROUP STAGE_GROUP
#if LIN_OUT_SUB == 256
        STAGE_GROUP STAGE_GROUP
#endif
        "s_mov_b32 m0, %[sv]\n"
        : [sv] "=&s"(saved), [st] "=&s"(st), [t] "=&v"(t)
        : [l] "s"(lds), [rs] "s"(rsrc), [s16] "s"(step16), [o0] "v"(o.v[0]), [o1] "v"(o.v[1]), [o2] "v"(o.v[2]),
          [o3] "v"(o.v[3])
        : "memory");
#undef STAGE_LOAD
#undef STAGE_GROUP
}

// q rows of tokens RPW*w .. +RPW-1 of the resource: lane (row 4i + lane/16, chunk lane%16), NI
// loads (zeros past the last token).
struct QRows {
    u32x4 v[NI];
};

__device__ __forceinline__ void load_q_rows(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned step4, QRows& qrw) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
        qrw.v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)(voff + i * step4), 0, 0));
}

// Sum over the 16 lanes of a DPP row (each lane ends with the total): xor 1 and xor 2 within
// quads, then the mirrored half-row and the mirrored row.
__device__ __forceinline__ float row16_sum(float p) {
    p += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, p), 0xB1, 0xF, 0xF, false));
    p += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, p), 0x4E, 0xF, 0xF, false));
    p += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, p), 0x141, 0xF, 0xF, false));
    p += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, p), 0x140, 0xF, 0xF, false));
    return p;
}

// den of those RPW tokens -> den_s[RPW*w + row]; lane (row group lane/16, chunk c) ends holding
// the sums of rows 4i + lane/16 for every i and writes the one with i = c.
__device__ __forceinline__ void write_den(const QRows& qrw, const float* ksum_s, float eps, float* den_s, int w,
                                          int lane) {
    const int c = lane & 15;
    float ks8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) ks8[e] = ksum_s[8 * c + e];
    float mine = 0.f;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        float p = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            p = fmaf(__uint_as_float(qrw.v[i][e] << 16), ks8[2 * e], p);
            p = fmaf(__uint_as_float(qrw.v[i][e] & 0xffff0000u), ks8[2 * e + 1], p);
        }
        p = row16_sum(p);
        mine = c == i ? p : mine;
    }
    const int fl = fresh_lane(lane);
    if (c < NI) den_s[RPW * w + 4 * (fl & 15) + (fl >> 4)] = mine + eps;
}

__global__ __launch_bounds__(NT, LIN_OUT_SUB == 128 ? 2 : 1) void linear_out_kernel(LinearArgs a) {
    __shared__ __attribute__((aligned(1024))) char qbuf[2][QBUF];
    __shared__ float den_s[2][OUT_SUB];
    __shared__ float ksum_s[D];
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ntb = (a.N + OUT_TOK - 1) / OUT_TOK;
    const int nbh = gridDim.x / ntb;   // heads fastest, as in the kv pass
    const int tb = blockIdx.x / nbh, bh = blockIdx.x - tb * nbh;
    const int b = bh / a.H, h = bh - b * a.H;
    const long row_stride = (long)a.H * D;
    const long base = ((long)b * a.N * a.H + h) * D;
    const int n0 = tb * OUT_TOK;
    const int nsub = min(OUT_SUBS, (a.N - n0 + OUT_SUB - 1) / OUT_SUB);
    const int g = lane >> 5, col = lane & 31;

    // resources per sub-block (from its first token); per-lane offsets fixed for the kernel
    auto q_rsrc = [&](int n) {
        return __builtin_amdgcn_make_buffer_rsrc((void*)(a.q + base + (long)n * row_stride), (short)0,
                                                 (int)(((long)(a.N - n - 1) * row_stride + D) * 2), (int)BUF_FLAGS);
    };
    // per-lane offsets (recomputed where used: a few VALU ops, cheaper than keeping them live)
    auto qoff = [&]() {
        const int l = fresh_lane(lane);
        return (unsigned)((((long)(RPW * w + (l >> 4))) * row_stride + 8 * (l & 15)) * 2);
    };
    const unsigned step4 = (unsigned)(4 * row_stride * 2), step16 = 4 * step4;
    stage_qrot(rows_rsrc(a.qr + base + (long)n0 * row_stride, a.N - n0, row_stride), step16,
               stage_offsets(row_stride, w, lane), qbuf[0], w);
    QRows qrw;
    load_q_rows(q_rsrc(n0), qoff(), step4, qrw);
    // A fragments: kv term rows 32w + col, dims 16ks + 8g .. +7
    bf16x8 af[KV_TERMS][8];
    const bf16* tm = a.terms + (long)bh * KV_TERMS * D * D + (long)(32 * w + col) * D + 8 * g;
#pragma unroll
    for (int t = 0; t < KV_TERMS; ++t)
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) af[t][ks] = *reinterpret_cast<const bf16x8*>(tm + (long)t * D * D + 16 * ks);
    if (tid < D) ksum_s[tid] = a.ksum[(long)bh * D + tid];
    __syncthreads();
    __builtin_amdgcn_s_waitcnt(WAIT_VMCNT0);   // this wave's q_rot rows are in LDS, af and q loaded
    write_den(qrw, ksum_s, a.eps, den_s[0], w, lane);

    for (int sub = 0; sub < nsub; ++sub) {
        const int cur = sub & 1;
        const int n_first = n0 + OUT_SUB * sub;
        // every wave waited for its q_rot rows of this sub-block and wrote its den before
        // arriving; every wave is done reading the other buffer
        __syncthreads();
        const bool more = sub + 1 < nsub;
        if (more) {
            const int nn = n_first + OUT_SUB;
            stage_qrot(rows_rsrc(a.qr + base + (long)nn * row_stride, a.N - nn, row_stride), step16,
                       stage_offsets(row_stride, w, lane), qbuf[cur ^ 1], w);
            load_q_rows(q_rsrc(nn), qoff(), step4, qrw);
        }
        const char* qb = qbuf[cur];
        f32x16 acc[OUT_SUB / 32];
#pragma unroll
        for (int cb = 0; cb < OUT_SUB / 32; ++cb) acc[cb] = f32x16{};
#if LIN_OUT_SUB == 256
        // B fragments of column block cb (row 32cb + col, chunks 2ks + g), read one block ahead
        bf16x8 bq[2][8];
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
            bq[0][ks] = *reinterpret_cast<const bf16x8*>(qb + col * QROW + 16 * ((2 * ks + g) ^ (col & 15)));
#pragma unroll
        for (int cb = 0; cb < OUT_SUB / 32; ++cb) {
            if (cb + 1 < OUT_SUB / 32) {
                const int r = 32 * (cb + 1) + col;
#pragma unroll
                for (int ks = 0; ks < 8; ++ks)
                    bq[(cb + 1) & 1][ks] =
                        *reinterpret_cast<const bf16x8*>(qb + r * QROW + 16 * ((2 * ks + g) ^ (r & 15)));
            }
#pragma unroll
            for (int ks = 0; ks < 8; ++ks)
#pragma unroll
                for (int t = 0; t < KV_TERMS; ++t) acc[cb] = mfma(af[t][ks], bq[cb & 1][ks], acc[cb]);
        }
#else
        // B fragment (row 32cb + col, chunk 2ks + g) per step; the other wave of the SIMD
        // covers the LDS latency
#pragma unroll
        for (int cb = 0; cb < OUT_SUB / 32; ++cb) {
            const int r = 32 * cb + col;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                const bf16x8 bq = *reinterpret_cast<const bf16x8*>(qb + r * QROW + 16 * ((2 * ks + g) ^ (r & 15)));
#pragma unroll
                for (int t = 0; t < KV_TERMS; ++t) acc[cb] = mfma(af[t][ks], bq, acc[cb]);
            }
        }
#endif
        if (more) {   // the next sub-block's loads had the MFMA phase to land
            __builtin_amdgcn_s_waitcnt(WAIT_VMCNT0);
            write_den(qrw, ksum_s, a.eps, den_s[cur ^ 1], w, lane);
        }
        // Output through LDS, so that the global stores move whole rows: once every wave is done
        // with this sub-block's q_rot, each writes its 32 dims of the 256 tokens (scaled by
        // 1/den, BF16) into that buffer, laid out like q_rot (row t, 16-byte chunk c at
        // t*256 + 16*(c ^ (t % 16))), then moves RPW whole rows to HBM, 4 per instruction.
        // C layout: lane (token column col, g), register q -> dim 32w + 8(q/4) + 4g + q%4.
        __syncthreads();
        char* ob = qbuf[cur];
#pragma unroll
        for (int cb = 0; cb < OUT_SUB / 32; ++cb) {
            const int t = 32 * cb + col;
            const float inv = 1.0f / den_s[cur][t];
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                const bf16 e0 = (bf16)(acc[cb][4 * qq + 0] * inv), e1 = (bf16)(acc[cb][4 * qq + 1] * inv);
                const bf16 e2 = (bf16)(acc[cb][4 * qq + 2] * inv), e3 = (bf16)(acc[cb][4 * qq + 3] * inv);
                const unsigned lo = (unsigned)__builtin_bit_cast(unsigned short, e0) |
                                    ((unsigned)__builtin_bit_cast(unsigned short, e1) << 16);
                const unsigned hi = (unsigned)__builtin_bit_cast(unsigned short, e2) |
                                    ((unsigned)__builtin_bit_cast(unsigned short, e3) << 16);
                const int chunk = (4 * w + qq) ^ (t & 15);     // dims 32w + 8qq .. +7
                *reinterpret_cast<uint2*>(ob + t * QROW + 16 * chunk + 8 * g) = make_uint2(lo, hi);
            }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int r = RPW * w + 4 * i + (lane >> 4), c = lane & 15;
            const u32x4 val = *reinterpret_cast<const u32x4*>(ob + r * QROW + 16 * (c ^ (r & 15)));
            if (n_first + r < a.N)
                *reinterpret_cast<u32x4*>(a.out + base + (long)(n_first + r) * row_stride + 8 * c) = val;
        }
    }
}

}  // namespace

namespace attn_impl {

// Resident kv-pass workgroups of the current device (compute units x KV_PER_CU); without a
// device (a host-only query) an MI355X's 256 compute units are assumed.
static long kv_slots() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                 hipSuccess || cus <= 0) {
        (void)hipGetLastError();
        cus = 256;
    }
    return (long)cus * KV_PER_CU;
}

// Tokens per kv-pass chunk: the shortest multiple of TILE (at least KV_CHUNK_MIN, at most
// KV_CHUNK_MAX) whose B*H*chunks workgroups fit in r whole rounds of the resident slots, for the
// smallest r that allows chunks of at most KV_CHUNK_MAX.
static int kv_chunk(size_t bh, int N) {
    const long slots = kv_slots();
    const long need = (N + KV_CHUNK_MAX - 1) / KV_CHUNK_MAX;          // chunks per sequence at the cap
    long r = std::max(1L, (long)((need * (long)bh + slots - 1) / slots));
    for (;; ++r) {
        const long cps = r * slots / (long)bh;                        // chunks per sequence in r rounds
        if (cps < 1) continue;
        long c = (N + cps - 1) / cps;
        c = std::max((long)KV_CHUNK_MIN, (c + TILE - 1) / TILE * TILE);
        if (c <= KV_CHUNK_MAX) return (int)c;
    }
}

static int linear_chunks(size_t bh, int N) {
    const int c = kv_chunk(bh, N);
    return (N + c - 1) / c;
}

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// [partials: BH x S x (D*D + D) FP32][terms: BH x 3 x D x D BF16][ksum: BH x D FP32]
size_t linear_workspace_bytes(int B, int N, int H) {
    const size_t bh = (size_t)B * H;
    return align256(bh * (size_t)linear_chunks(bh, N) * (D * D + D) * sizeof(float)) +
           align256(bh * KV_TERMS * D * D * sizeof(bf16)) + align256(bh * D * sizeof(float));
}

hipError_t launch_linear(const void* q, const void* k, const void* qr, const void* kr, const void* v, void* out,
                         int B, int N, int H, float eps, void* workspace, hipStream_t stream) {
    LinearArgs a;
    a.q = static_cast<const bf16*>(q);
    a.k = static_cast<const bf16*>(k);
    a.qr = static_cast<const bf16*>(qr);
    a.kr = static_cast<const bf16*>(kr);
    a.v = static_cast<const bf16*>(v);
    a.out = static_cast<bf16*>(out);
    a.N = N;
    a.H = H;
    const size_t bh = (size_t)B * H;
    a.chunk = kv_chunk(bh, N);
    a.S = (N + a.chunk - 1) / a.chunk;
    a.eps = eps;
    char* ws = static_cast<char*>(workspace);
    const size_t part = align256(bh * (size_t)a.S * (D * D + D) * sizeof(float));
    const size_t terms = align256(bh * KV_TERMS * D * D * sizeof(bf16));
    a.part = reinterpret_cast<float*>(ws);
    a.terms = reinterpret_cast<bf16*>(ws + part);
    a.ksum = reinterpret_cast<float*>(ws + part + terms);
    hipLaunchKernelGGL(linear_kv_partial_kernel, dim3((unsigned)(bh * a.S)), dim3(NT), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(linear_kv_reduce_kernel, dim3((unsigned)(bh * REDUCE_BLOCKS)), dim3(NT), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long ntb = (N + OUT_TOK - 1) / OUT_TOK;
    hipLaunchKernelGGL(linear_out_kernel, dim3((unsigned)(bh * ntb)), dim3(NT), 0, stream, a);
    return hipGetLastError();
}

}  // namespace attn_impl
