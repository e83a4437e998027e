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
//   linear_kv_partial_kernel  one workgroup per (b, h, chunk of KV_CHUNK tokens): the chunk's
//       kv (v_mfma_f32_32x32x16_bf16, FP32 accumulation) and ksum (FP32 VALU) into the
//       workspace. V and K_rot tiles go through LDS; transposing LDS reads
//       (ds_read_b64_tr_b16) give each lane 8 consecutive tokens of one dim, the MFMA's
//       operand layout for both A = V^T and B = K_rot.
//   linear_kv_reduce_kernel   sums the chunk partials in chunk order (deterministic) and
//       splits kv exactly into three BF16 terms.
//   linear_out_kernel         one workgroup per (b, h, 1024 tokens): out = kv q_rot / den.
//       The FP32 product runs on the BF16 matrix cores: kv = hi + mid + lo with three BF16
//       terms (8 bits each, together every bit of the FP32 value), q_rot is BF16 exactly,
//       so each of the three MFMA products is exact and the accumulation is FP32, the same
//       arithmetic as an FP32 GEMM up to summation order.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

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
constexpr int KV_CHUNK = 2048;       // tokens per workgroup in the kv pass (a multiple of TILE)
constexpr int ROW = D * 2 + 32;      // LDS row stride in bytes (padded: 8-bank shift per row)
constexpr int KV_TERMS = 3;          // BF16 terms of the FP32 kv in the output pass
constexpr int OUT_SUB = 256;         // tokens per sub-block of the output pass (64 per wave)
constexpr int OUT_SUBS = 4;          // sub-blocks per workgroup
constexpr int OUT_TOK = OUT_SUB * OUT_SUBS;
constexpr int KVROW = D * 2 + 16;    // LDS row stride of a BF16 kv term

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
    const int bh = blockIdx.x / a.S, s = blockIdx.x - bh * a.S;
    const int b = bh / a.H, h = bh - b * a.H;
    const long row_stride = (long)a.H * D;                       // elements between tokens
    const long base = ((long)b * a.N * a.H + h) * D;             // (b, token 0, h)
    const int m0 = s * KV_CHUNK, m1 = min(a.N, m0 + KV_CHUNK);

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
__global__ __launch_bounds__(NT) void linear_kv_reduce_kernel(LinearArgs a) {
    const int per = (D * D + D + NT - 1) / NT;
    const int bh = blockIdx.x / per, blk = blockIdx.x - bh * per;
    const int e = blk * NT + threadIdx.x;
    if (e >= D * D + D) return;
    const float* p = a.part + (long)bh * a.S * (D * D + D) + e;
    float sum = 0.f;
    for (int s = 0; s < a.S; ++s) sum += p[(long)s * (D * D + D)];
    if (e < D * D) {
        // exact split of the FP32 sum into three BF16 terms (8 significant bits each)
        const bf16 hi = (bf16)sum;
        const float r1 = sum - (float)hi;
        const bf16 mid = (bf16)r1;
        const bf16 lo = (bf16)(r1 - (float)mid);
        bf16* t = a.terms + (long)bh * KV_TERMS * D * D + e;
        t[0] = hi;
        t[D * D] = mid;
        t[2 * D * D] = lo;
    } else {
        a.ksum[(long)bh * D + e - D * D] = sum;
    }
}

// ---------------------------------------------------------------- out = kv q_rot / den
// A workgroup takes OUT_TOK tokens of one (b, h) in OUT_SUBS sub-blocks; in each, wave w owns
// 64 tokens (two 32-token column blocks) against all four 32-row blocks of kv. A fragments
// (kv terms) come from LDS; the B fragments (q_rot) and the q rows of the normaliser are
// loaded in the MFMA operand layout (lane: token column, 8 dims), the next sub-block's while
// the current one computes.
struct OutFrags {
    bf16x8 qr[2][8];   // q_rot: [column block][16-dim step]
    bf16x8 q[2][8];    // q (normaliser)
};

__device__ __forceinline__ void load_out_frags(const LinearArgs& a, long base, long row_stride, int n_first,
                                               int col, int g, OutFrags& f) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
        const int nn = min(n_first + 32 * cb + col, a.N - 1);
        const bf16* qr = a.qr + base + (long)nn * row_stride + 8 * g;
        const bf16* q = a.q + base + (long)nn * row_stride + 8 * g;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            f.qr[cb][ks] = *reinterpret_cast<const bf16x8*>(qr + 16 * ks);
            f.q[cb][ks] = *reinterpret_cast<const bf16x8*>(q + 16 * ks);
        }
    }
}

__global__ __launch_bounds__(NT, 1) void linear_out_kernel(LinearArgs a) {
    __shared__ __attribute__((aligned(16))) char kvs[KV_TERMS * D * KVROW];
    __shared__ float ksum_s[D];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int ntb = (a.N + OUT_TOK - 1) / OUT_TOK;
    const int bh = blockIdx.x / ntb, tb = blockIdx.x - bh * ntb;
    const int b = bh / a.H, h = bh - b * a.H;
    const long row_stride = (long)a.H * D;
    const long base = ((long)b * a.N * a.H + h) * D;
    const int n0 = tb * OUT_TOK;
    const int g = lane >> 5, col = lane & 31;

    OutFrags cur, nxt;
    load_out_frags(a, base, row_stride, n0 + 64 * w, col, g, cur);
    // kv terms -> LDS (row i of term t at t*D*KVROW + i*KVROW), 16 bytes per thread and step
    // (straight-line batches of 8 loads, so the waits count the loads in flight instead of
    // draining the queue after each one)
    const u32x4* src = reinterpret_cast<const u32x4*>(a.terms + (long)bh * KV_TERMS * D * D);
    constexpr int PER = KV_TERMS * D * (D / 8) / NT;      // 24 chunks of 16 bytes per thread
    static_assert(PER % 8 == 0, "copy batches");
#pragma unroll
    for (int bt = 0; bt < PER; bt += 8) {
        u32x4 tmp[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) tmp[u] = src[tid + (bt + u) * NT];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int cidx = tid + (bt + u) * NT;
            const int row = cidx >> 4, ch = cidx & 15;      // row = term * D + i
            *reinterpret_cast<u32x4*>(kvs + row * KVROW + 16 * ch) = tmp[u];
        }
    }
    if (tid < D) ksum_s[tid] = a.ksum[(long)bh * D + tid];
    __syncthreads();

#pragma unroll
    for (int sub = 0; sub < OUT_SUBS; ++sub) {
        const int n_first = n0 + OUT_SUB * sub + 64 * w;
        if (sub + 1 < OUT_SUBS) load_out_frags(a, base, row_stride, n_first + OUT_SUB, col, g, nxt);

        // normaliser: lane (col, g) sums its 64 dims of q . ksum, the partner lane the other 64
        float den[2];
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            float p = 0.f;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks)
#pragma unroll
                for (int t = 0; t < 8; ++t) p = fmaf((float)cur.q[cb][ks][t], ksum_s[16 * ks + 8 * g + t], p);
            den[cb] = p + __shfl_xor(p, 32) + a.eps;
        }

        f32x16 acc[4][2];
#pragma unroll
        for (int ib = 0; ib < 4; ++ib)
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) acc[ib][cb] = f32x16{};
#pragma unroll
        for (int term = 0; term < KV_TERMS; ++term)
#pragma unroll
            for (int ks = 0; ks < 8; ++ks)
#pragma unroll
                for (int ib = 0; ib < 4; ++ib) {
                    // A: kv term, rows 32ib + col, dims 16ks + 8g .. +7
                    const bf16x8 fa = *reinterpret_cast<const bf16x8*>(
                        kvs + (term * D + 32 * ib + col) * KVROW + 2 * (16 * ks + 8 * g));
#pragma unroll
                    for (int cb = 0; cb < 2; ++cb) acc[ib][cb] = mfma(fa, cur.qr[cb][ks], acc[ib][cb]);
                }

        // C layout: lane (token column col, g), register q -> dim 32ib + 8(q/4) + 4g + q%4
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            const int n = n_first + 32 * cb + col;
            if (n < a.N) {
                const float inv = 1.0f / den[cb];
                bf16* orow = a.out + base + (long)n * row_stride;
#pragma unroll
                for (int ib = 0; ib < 4; ++ib)
#pragma unroll
                    for (int qq = 0; qq < 4; ++qq) {
                        const int d0 = 32 * ib + 8 * qq + 4 * g;
                        const bf16 e0 = (bf16)(acc[ib][cb][4 * qq + 0] * inv), e1 = (bf16)(acc[ib][cb][4 * qq + 1] * inv);
                        const bf16 e2 = (bf16)(acc[ib][cb][4 * qq + 2] * inv), e3 = (bf16)(acc[ib][cb][4 * qq + 3] * inv);
                        const unsigned lo = (unsigned)__builtin_bit_cast(unsigned short, e0) |
                                            ((unsigned)__builtin_bit_cast(unsigned short, e1) << 16);
                        const unsigned hi = (unsigned)__builtin_bit_cast(unsigned short, e2) |
                                            ((unsigned)__builtin_bit_cast(unsigned short, e3) << 16);
                        *reinterpret_cast<uint2*>(orow + d0) = make_uint2(lo, hi);
                    }
            }
        }
        if (sub + 1 < OUT_SUBS) cur = nxt;
    }
}

}  // namespace

namespace attn_impl {

int linear_chunks(int N) { return (N + KV_CHUNK - 1) / KV_CHUNK; }

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// [partials: BH x S x (D*D + D) FP32][terms: BH x 3 x D x D BF16][ksum: BH x D FP32]
size_t linear_workspace_bytes(int B, int N, int H) {
    const size_t bh = (size_t)B * H;
    return align256(bh * (size_t)linear_chunks(N) * (D * D + D) * sizeof(float)) +
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
    a.S = linear_chunks(N);
    a.eps = eps;
    const size_t bh = (size_t)B * H;
    char* ws = static_cast<char*>(workspace);
    const size_t part = align256(bh * (size_t)a.S * (D * D + D) * sizeof(float));
    const size_t terms = align256(bh * KV_TERMS * D * D * sizeof(bf16));
    a.part = reinterpret_cast<float*>(ws);
    a.terms = reinterpret_cast<bf16*>(ws + part);
    a.ksum = reinterpret_cast<float*>(ws + part + terms);
    hipLaunchKernelGGL(linear_kv_partial_kernel, dim3((unsigned)(bh * a.S)), dim3(NT), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int per = (D * D + D + NT - 1) / NT;
    hipLaunchKernelGGL(linear_kv_reduce_kernel, dim3((unsigned)(bh * per)), dim3(NT), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long ntb = (N + OUT_TOK - 1) / OUT_TOK;
    hipLaunchKernelGGL(linear_out_kernel, dim3((unsigned)(bh * ntb)), dim3(NT), 0, stream, a);
    return hipGetLastError();
}

}  // namespace attn_impl
