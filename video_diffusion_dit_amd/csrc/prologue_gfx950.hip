// Attention prologue for CDNA4 (gfx950): per-head RMSNorm and interleaved 3-D RoPE on Q and K,
// V passed through, from the projection's token-major [B, N, H, 128] BF16 rows to the
// attention kernel's head-major [B, H, N, 128] BF16 layout, in one pass over memory.
//
// What is computed, per token n of batch b and head h (x = the BF16 input row; FP32 math):
//   r = 1 / sqrt(mean_c x_c^2 + eps);  y_c = x_c * r * w_c  (w = 1 without a weight)
//   pair i (channels 2i, 2i+1) on axis a(i) with index k < P_a turns by
//   phi = pos_a(n) * theta^(-k/P_a):  (y_2i, y_2i+1) -> (y_2i c - y_2i+1 s, y_2i s + y_2i+1 c)
//   the 64 pairs split (22, 21, 21) over (t, h, w); pos(n) = (n / (Hp Wp), (n / Wp) % Hp, n % Wp)
//   the result is rounded to BF16 (nearest even) once.
// Sources: page "PR #35728 report", key source excerpts (sana_video.py forward: RMSNorm on
// Q and K, view as [B, N, H, D], interleaved rotary embedding on Q and K only, V only
// reshaped); page "[sglang] SANA-Video 2.0 anchor attention ... FP32 upcast", introduction
// (Q/K/V reach attention in BF16 after RMSNorm and RoPE); page "PR #35728 report", related
// context (a fused 3-D RoPE kernel for the LTX-2.5 decoder).
//
// Work decomposition: a 16-lane group owns one 256-byte row at a time (lane j: channels
// 8j..8j+7, i.e. RoPE pairs 4j..4j+3), so one wave instruction moves four rows; each group
// keeps four rows in flight (loads issued before any use). The row's sum of squares is reduced
// across its 16 lanes. With more than 4 heads a wave takes one token and its four groups split
// the token's rows; with 4 heads or fewer (a token has at most 8 Q/K rows, e.g. one GPU's share
// of a head-sharded call) each group takes a token of its own, so no group idles. The token's angles are the same for every head
// and for Q and K: each lane computes its four (cos, sin) once per token, from FP64 angles
// (theta^(-k/P) and pos * freq in FP64, then sincos), so the angle error stays near 1e-16
// rad instead of the ~1e-5 that FP32 products reach at pos ~ 80. Memory-bound: 256 bytes
// read and 256 written per token-head row.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "attn_launch.h"

namespace {

typedef __bf16 bf16;
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int D = 128;
constexpr int WAVES = 4;        // tokens per workgroup
constexpr int ROWS = 4;         // rows in flight per 16-lane group

struct PrologueArgs {
    const bf16* xq;
    const bf16* xk;
    const bf16* xv;
    bf16* q;
    bf16* k;
    bf16* v;
    const float* wq;
    const float* wk;
    long tokens;                // B * N
    int N, H, Hp, Wp;
    float eps;
    double log2_theta;
};

// Interleaved pair index i (0..63) -> (axis, k, P).
__device__ __forceinline__ void pair_axis(int i, int& axis, int& k, int& P) {
    if (i < 22) { axis = 0; k = i; P = 22; }
    else if (i < 43) { axis = 1; k = i - 22; P = 21; }
    else { axis = 2; k = i - 43; P = 21; }
}

__device__ __forceinline__ f32x8 load_row(const bf16* p) {
    const u32x4 u = *reinterpret_cast<const u32x4*>(p);
    f32x8 x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(u[i] << 16);
        x[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
    return x;
}

// RMSNorm (over the 16-lane group), weight, rotation; 8 BF16 results (RNE) packed in 4 dwords.
__device__ __forceinline__ u32x4 norm_rope(f32x8 x, const float (&w)[8], const float (&c)[4],
                                           const float (&s)[4], float eps) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = fmaf(x[i], x[i], ss);
    ss += __shfl_xor(ss, 1, 16);
    ss += __shfl_xor(ss, 2, 16);
    ss += __shfl_xor(ss, 4, 16);
    ss += __shfl_xor(ss, 8, 16);
    const float r = 1.0f / sqrtf(ss * (1.0f / D) + eps);
    u32x4 out;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const float ye = x[2 * p] * r * w[2 * p], yo = x[2 * p + 1] * r * w[2 * p + 1];
        const float oe = fmaf(ye, c[p], -yo * s[p]);
        const float oo = fmaf(ye, s[p], yo * c[p]);
        const bf16 be = (bf16)oe, bo = (bf16)oo;   // round to nearest even
        out[p] = (unsigned)__builtin_bit_cast(unsigned short, be) |
                 ((unsigned)__builtin_bit_cast(unsigned short, bo) << 16);
    }
    return out;
}

// A token's Q/K/V rows are split over GROUPS 16-lane groups (4: one token per wave; 1: one
// token per group).
template <int GROUPS>
__global__ __launch_bounds__(WAVES * 64) void qk_prologue_kernel(PrologueArgs a) {
    const int lane = threadIdx.x & 63;
    const int j = lane & 15;
    const int grp = GROUPS == 4 ? lane >> 4 : 0;
    const long tok = GROUPS == 4 ? (long)blockIdx.x * WAVES + (threadIdx.x >> 6)
                                 : (long)blockIdx.x * WAVES * 4 + (threadIdx.x >> 4);
    if (tok >= a.tokens) return;   // a whole group (16 lanes) leaves together
    const long b = tok / a.N;
    const int n = (int)(tok - b * a.N);
    const int pos[3] = {n / (a.Hp * a.Wp), (n / a.Wp) % a.Hp, n % a.Wp};

    // this lane's four pairs: angles in FP64, then FP32 cos/sin
    float c[4], s[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        int axis, k, P;
        pair_axis(4 * j + p, axis, k, P);
        const double phi = (double)pos[axis] * exp2(-a.log2_theta * (double)k / (double)P);
        double sd, cd;
        sincos(phi, &sd, &cd);
        c[p] = (float)cd;
        s[p] = (float)sd;
    }
    float wq[8], wk[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        wq[i] = a.wq ? a.wq[8 * j + i] : 1.0f;
        wk[i] = a.wk ? a.wk[8 * j + i] : 1.0f;
    }

    const long in_row = (long)tok * a.H;                  // first row of this token in [B*N, H]
    const long out_tok = (long)b * a.H * a.N + n;         // row (b, 0, n) of [B, H, N]
    // Q and K: rows r = 0..2H-1 (r < H: Q head r, else K head r - H), four per group in flight
    for (int r0 = grp * ROWS; r0 < 2 * a.H; r0 += GROUPS * ROWS) {
        f32x8 x[ROWS];
#pragma unroll
        for (int u = 0; u < ROWS; ++u) {
            const int r = r0 + u;
            if (r < 2 * a.H) {
                const bf16* src = r < a.H ? a.xq + (in_row + r) * D : a.xk + (in_row + r - a.H) * D;
                x[u] = load_row(src + 8 * j);
            }
        }
#pragma unroll
        for (int u = 0; u < ROWS; ++u) {
            const int r = r0 + u;
            if (r < 2 * a.H) {
                const bool isq = r < a.H;
                const int h = isq ? r : r - a.H;
                const u32x4 o = norm_rope(x[u], isq ? wq : wk, c, s, a.eps);
                bf16* dst = (isq ? a.q : a.k) + (out_tok + (long)h * a.N) * D + 8 * j;
                *reinterpret_cast<u32x4*>(dst) = o;
            }
        }
    }
    if (a.xv == nullptr) return;
    for (int r0 = grp * ROWS; r0 < a.H; r0 += GROUPS * ROWS) {
        u32x4 x[ROWS];
#pragma unroll
        for (int u = 0; u < ROWS; ++u)
            if (r0 + u < a.H) x[u] = *reinterpret_cast<const u32x4*>(a.xv + (in_row + r0 + u) * D + 8 * j);
#pragma unroll
        for (int u = 0; u < ROWS; ++u)
            if (r0 + u < a.H) *reinterpret_cast<u32x4*>(a.v + (out_tok + (long)(r0 + u) * a.N) * D + 8 * j) = x[u];
    }
}

// Packed (THD) prologue: per-head RMSNorm of the Q and K rows, which stay in their token-major
// layout -- the layout the packed attention reads -- with no rotation (the pages give no
// positions for packed segments). Rows 0 .. TH-1 are Q, TH .. 2TH-1 K; each 16-lane group
// normalises 4 consecutive rows, all loads issued before any store, so q == xq (and
// k == xk) works in place.
struct NormArgs {
    const bf16* xq;
    const bf16* xk;
    bf16* q;
    bf16* k;
    const float* wq;
    const float* wk;
    long rows;                  // T * H
    float eps;
};

__global__ __launch_bounds__(256) void qk_norm_packed_kernel(NormArgs a) {
    const int j = threadIdx.x & 15;
    const long r0 = ((long)blockIdx.x * 16 + (threadIdx.x >> 4)) * ROWS;
    if (r0 >= 2 * a.rows) return;   // a whole group (16 lanes) leaves together
    float wq[8], wk[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        wq[i] = a.wq ? a.wq[8 * j + i] : 1.0f;
        wk[i] = a.wk ? a.wk[8 * j + i] : 1.0f;
    }
    f32x8 x[ROWS];
#pragma unroll
    for (int u = 0; u < ROWS; ++u) {
        const long r = r0 + u;
        if (r < 2 * a.rows) x[u] = load_row((r < a.rows ? a.xq + r * D : a.xk + (r - a.rows) * D) + 8 * j);
    }
#pragma unroll
    for (int u = 0; u < ROWS; ++u) {
        const long r = r0 + u;
        if (r >= 2 * a.rows) continue;
        const bool isq = r < a.rows;
        const float* w = isq ? wq : wk;
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) ss = fmaf(x[u][i], x[u][i], ss);
        ss += __shfl_xor(ss, 1, 16);
        ss += __shfl_xor(ss, 2, 16);
        ss += __shfl_xor(ss, 4, 16);
        ss += __shfl_xor(ss, 8, 16);
        const float rn = 1.0f / sqrtf(ss * (1.0f / D) + a.eps);
        u32x4 out;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const bf16 be = (bf16)(x[u][2 * p] * rn * w[2 * p]), bo = (bf16)(x[u][2 * p + 1] * rn * w[2 * p + 1]);
            out[p] = (unsigned)__builtin_bit_cast(unsigned short, be) |
                     ((unsigned)__builtin_bit_cast(unsigned short, bo) << 16);
        }
        *reinterpret_cast<u32x4*>((isq ? a.q + r * D : a.k + (r - a.rows) * D) + 8 * j) = out;
    }
}

}  // namespace

namespace attn_impl {

hipError_t launch_qk_norm_packed(const void* xq, const void* xk, void* q, void* k, const float* wq, const float* wk,
                                 int T, int H, float eps, hipStream_t stream) {
    NormArgs a;
    a.xq = static_cast<const bf16*>(xq);
    a.xk = static_cast<const bf16*>(xk);
    a.q = static_cast<bf16*>(q);
    a.k = static_cast<bf16*>(k);
    a.wq = wq;
    a.wk = wk;
    a.rows = (long)T * H;
    a.eps = eps;
    const long grid = (2 * a.rows + 16 * ROWS - 1) / (16 * ROWS);
    hipLaunchKernelGGL(qk_norm_packed_kernel, dim3((unsigned)grid), dim3(256), 0, stream, a);
    return hipGetLastError();
}


hipError_t launch_qk_prologue(const void* xq, const void* xk, const void* xv, void* q, void* k, void* v,
                              const float* wq, const float* wk, int B, int N, int H, int Hp, int Wp,
                              float eps, float theta, hipStream_t stream) {
    PrologueArgs a;
    a.xq = static_cast<const bf16*>(xq);
    a.xk = static_cast<const bf16*>(xk);
    a.xv = static_cast<const bf16*>(xv);
    a.q = static_cast<bf16*>(q);
    a.k = static_cast<bf16*>(k);
    a.v = static_cast<bf16*>(v);
    a.wq = wq;
    a.wk = wk;
    a.tokens = (long)B * N;
    a.N = N;
    a.H = H;
    a.Hp = Hp;
    a.Wp = Wp;
    a.eps = eps;
    a.log2_theta = log2((double)theta);
    if (H <= 4) {
        const long grid = (a.tokens + 4 * WAVES - 1) / (4 * WAVES);
        hipLaunchKernelGGL(qk_prologue_kernel<1>, dim3((unsigned)grid), dim3(WAVES * 64), 0, stream, a);
    } else {
        const long grid = (a.tokens + WAVES - 1) / WAVES;
        hipLaunchKernelGGL(qk_prologue_kernel<4>, dim3((unsigned)grid), dim3(WAVES * 64), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace attn_impl
