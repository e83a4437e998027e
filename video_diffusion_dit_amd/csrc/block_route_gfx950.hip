// Key-block routing of block-skip attention for gfx950: for every query tile of 256 rows,
// the list of the 64-key tiles its rows attend to.
//
// Method: page "PR #33702 report" (the Sol-Attn backend for MiniMax-H3), motivation and
// breakdown: KV blocks are routed by a threshold (knob tau) so that the attention skips most
// of them, without building a full proxy score map; sink tokens stay in. The page gives no
// formula; the rule taken here:
//   qbar_I = mean of the valid query rows of tile I, kbar_J = mean of the valid keys of tile J
//   z_IJ   = scale * qbar_I . kbar_J
//   keep J for I  iff  z_IJ >= max_J' z_IJ' - tau  or  J*64 < sink_tokens
// Only the per-tile lists leave the chip (the z of a tile row live in LDS), in the layout the
// block-sparse attention kernel reads: kv_idx[item][stride] ascending tile indices and
// kv_cnt[item], item = (b*H + h)*ntq + I, stride = ntk + 8; the 8 entries after the count
// hold ntk.
//
// Kernels (HBM-bound pooling, then L2-resident routing):
//   pool_kernel<RB, KT>: one workgroup per 256 rows of one (b, h); thread (row lane rl, 16-byte
//     chunk ch) sums rows rl, rl+16, ... of each RB-row block in FP32, the 16 row lanes are
//     added in order through LDS, and the sum is divided by the block's valid rows. The query
//     means are stored row by row ([BH][ntq][128]); the key means (KT) by groups of four
//     dimensions, tile-minor ([BH][32][ntk] float4), so that the lanes of a wave, which take
//     consecutive key tiles, read one contiguous kilobyte per load.
//   route_kernel<QPW>: one workgroup per QPW query tiles of one (b, h); thread J computes the
//     QPW proxies of key tile J (128-term FP32 dot products, dimensions in order, the query
//     means read through scalar loads) into LDS;
//     then per query tile a block-wide max, the threshold, and an ordered compaction (each
//     thread owns a contiguous run of tiles; a wave-level scan of the run counts gives the
//     write offsets).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "attn_launch.h"

namespace {

typedef __bf16 bf16;

constexpr int D = 128;
constexpr int BMQ = 256;   // query rows per tile (the attention kernel's workgroup rows)
constexpr int BNK = 64;    // keys per tile (the attention kernel's key tile)
constexpr int LIST_PAD = 8;
constexpr int ROUTE_LDS_LIMIT = 61440;   // bytes of proxies a workgroup keeps in LDS

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <int RB, bool KT>
__global__ __launch_bounds__(256) void pool_kernel(const bf16* __restrict__ x, float* __restrict__ out, int N,
                                                   int nblk) {
    constexpr int NB = 256 / RB;    // pooled blocks per workgroup
    constexpr int PER = RB / 16;    // rows per thread and block
    __shared__ float red[16][NB][D];
    const int wpb = (N + 255) / 256;
    const int bh = blockIdx.x / wpb, w = blockIdx.x - bh * wpb;
    const int tid = threadIdx.x, ch = tid & 15, rl = tid >> 4;
    const bf16* xb = x + (long)bh * N * D;
    for (int b = 0; b < NB; ++b) {
        float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int i = 0; i < PER; ++i) {
            const int r = w * 256 + b * RB + rl + 16 * i;
            if (r < N) {
                const uint4 u = *reinterpret_cast<const uint4*>(xb + (long)r * D + 8 * ch);
                acc[0] += bf16_lo(u.x);
                acc[1] += bf16_hi(u.x);
                acc[2] += bf16_lo(u.y);
                acc[3] += bf16_hi(u.y);
                acc[4] += bf16_lo(u.z);
                acc[5] += bf16_hi(u.z);
                acc[6] += bf16_lo(u.w);
                acc[7] += bf16_hi(u.w);
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) red[rl][b][8 * ch + e] = acc[e];
    }
    __syncthreads();
    for (int t = tid; t < NB * D; t += 256) {
        // KT: 4 consecutive threads take 4 dimensions of one block, the next 4 the next block
        const int b = KT ? (t >> 2) % NB : t / D;
        const int c = KT ? 4 * (t / (4 * NB)) + (t & 3) : t - b * D;
        const int blk = w * NB + b;
        const int rows = min(RB, N - blk * RB);
        if (rows <= 0) continue;
        float s = 0.f;
        for (int j = 0; j < 16; ++j) s += red[j][b][c];
        const long o = KT ? (((long)bh * (D / 4) + (c >> 2)) * nblk + blk) * 4 + (c & 3) : ((long)bh * nblk + blk) * D + c;
        out[o] = s / (float)rows;
    }
}

struct RouteArgs {
    const float* qbar;   // [BH][ntq][128]
    const float* kbar;   // [BH][32][ntk][4]: dimensions 4c..4c+3 of key tile J at [bh][c][J]
    int32_t* kidx;
    int32_t* kcnt;
    int ntq, ntk, stride, nsink;
    float scale, tau;
};

__device__ __forceinline__ float block_max(float v, float* red) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    const int tid = threadIdx.x;
    __syncthreads();
    if ((tid & 63) == 0) red[tid >> 6] = v;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

template <int QPW>
__global__ __launch_bounds__(256) void route_kernel(RouteArgs a) {
    extern __shared__ float zs[];   // [QPW][ntk]
    __shared__ float red[4];
    __shared__ int wsum[4];
    const int gpb = (a.ntq + QPW - 1) / QPW;
    const int bh = blockIdx.x / gpb, g = blockIdx.x - bh * gpb;
    const int qt0 = g * QPW, nq = min(QPW, a.ntq - qt0);
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    // the query means are the same for every lane: read at wave-uniform addresses (scalar
    // loads); a group's missing last tiles repeat tile ntq - 1 and are never compacted
    const float* __restrict__ qg[QPW];
#pragma unroll
    for (int qi = 0; qi < QPW; ++qi) qg[qi] = a.qbar + ((long)bh * a.ntq + min(qt0 + qi, a.ntq - 1)) * D;
    const float4* kb = reinterpret_cast<const float4*>(a.kbar) + (long)bh * (D / 4) * a.ntk;
    for (int J = tid; J < a.ntk; J += 256) {
        float z[QPW];
#pragma unroll
        for (int qi = 0; qi < QPW; ++qi) z[qi] = 0.f;
#pragma unroll 4
        for (int c4 = 0; c4 < D / 4; ++c4) {
            const float4 kv = kb[(long)c4 * a.ntk + J];
#pragma unroll
            for (int qi = 0; qi < QPW; ++qi) {
                z[qi] = fmaf(qg[qi][4 * c4 + 0], kv.x, z[qi]);
                z[qi] = fmaf(qg[qi][4 * c4 + 1], kv.y, z[qi]);
                z[qi] = fmaf(qg[qi][4 * c4 + 2], kv.z, z[qi]);
                z[qi] = fmaf(qg[qi][4 * c4 + 3], kv.w, z[qi]);
            }
        }
#pragma unroll
        for (int qi = 0; qi < QPW; ++qi) zs[qi * a.ntk + J] = z[qi] * a.scale;
    }
    __syncthreads();
    const int run = (a.ntk + 255) / 256;
    const int j0 = min(tid * run, a.ntk), j1 = min(j0 + run, a.ntk);
    for (int qi = 0; qi < nq; ++qi) {
        const float* z = zs + qi * a.ntk;
        float m = -INFINITY;
        for (int J = tid; J < a.ntk; J += 256) m = fmaxf(m, z[J]);
        const float thr = block_max(m, red) - a.tau;
        int cnt = 0;
        for (int J = j0; J < j1; ++J) cnt += (z[J] >= thr || J < a.nsink) ? 1 : 0;
        // exclusive prefix of the run counts: within the wave, then across the 4 waves
        int incl = cnt;
        for (int o = 1; o < 64; o <<= 1) {
            const int t = __shfl_up(incl, o);
            if (lane >= o) incl += t;
        }
        if (lane == 63) wsum[wv] = incl;
        __syncthreads();
        int off = incl - cnt;
        for (int k = 0; k < wv; ++k) off += wsum[k];
        const int total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
        const long item = (long)bh * a.ntq + qt0 + qi;
        int32_t* dst = a.kidx + item * a.stride;
        for (int J = j0; J < j1; ++J)
            if (z[J] >= thr || J < a.nsink) dst[off++] = J;
        if (tid < LIST_PAD) dst[total + tid] = a.ntk;
        if (tid == 0) a.kcnt[item] = total;
        __syncthreads();   // wsum and red are reused by the next query tile
    }
}

// ---------------------------------------------------------------- packed (varlen) batches
// Segment s = rows cu[s] .. cu[s+1]-1 of THD [T, H, 128] tensors (row stride H*128). Query
// tiles (256 rows) and key tiles (64 keys) are counted per segment from its first row and
// numbered segment by segment: tile i of segment s is tile off[s] + i.

__device__ __forceinline__ int seg_bound(const int32_t* cu, int s, int T) { return min(max(cu[s], 0), T); }

// off_q[s] / off_k[s]: first query / key tile of segment s ([nseg + 1], last = totals). One
// workgroup: each thread sums a contiguous run of segments, a serial scan orders the runs.
__global__ __launch_bounds__(1024) void tile_offsets_kernel(const int32_t* __restrict__ cu, int nseg, int T,
                                                            int* __restrict__ off_q, int* __restrict__ off_k) {
    __shared__ int pq[1024], pk[1024];
    const int tid = threadIdx.x;
    const int per = (nseg + 1023) / 1024;
    const int s0 = min(tid * per, nseg), s1 = min(s0 + per, nseg);
    int sq = 0, sk = 0;
    for (int s = s0; s < s1; ++s) {
        const int a = seg_bound(cu, s, T), e = max(seg_bound(cu, s + 1, T), a);
        sq += (e - a + BMQ - 1) / BMQ;
        sk += (e - a + BNK - 1) / BNK;
    }
    pq[tid] = sq;
    pk[tid] = sk;
    __syncthreads();
    if (tid == 0) {
        int aq = 0, ak = 0;
        for (int i = 0; i < 1024; ++i) {
            const int vq = pq[i], vk = pk[i];
            pq[i] = aq;
            pk[i] = ak;
            aq += vq;
            ak += vk;
        }
        off_q[nseg] = aq;
        off_k[nseg] = ak;
    }
    __syncthreads();
    int aq = pq[tid], ak = pk[tid];
    for (int s = s0; s < s1; ++s) {
        off_q[s] = aq;
        off_k[s] = ak;
        const int a = seg_bound(cu, s, T), e = max(seg_bound(cu, s + 1, T), a);
        aq += (e - a + BMQ - 1) / BMQ;
        ak += (e - a + BNK - 1) / BNK;
    }
}

// segment holding tile g: the last s with off[s] <= g (off ascending, off[0] = 0)
__device__ __forceinline__ int tile_segment(const int* off, int nseg, int g) {
    int lo = 0, hi = nseg;   // off[lo] <= g < off[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (off[mid] <= g) lo = mid;
        else hi = mid;
    }
    return lo;
}

// Mean of one RB-row tile of one head: workgroup (tile g, head h); thread (row lane rl, chunk
// ch) sums rows rl, rl+16, ...; the 16 row lanes are added in order through LDS. Stored at
// [g][h][128] (kt = 0), or, for the key means, by groups of four dimensions, tile-minor, at
// [h][32][kt][4] (kt = the tile capacity), as pool_kernel stores them.
template <int RB>
__global__ __launch_bounds__(256) void pool_varlen_kernel(const bf16* __restrict__ x, float* __restrict__ out,
                                                          const int32_t* __restrict__ cu, const int* __restrict__ off,
                                                          int nseg, int H, int T, int kt) {
    __shared__ float red[16][D];
    const int g = blockIdx.x / H, h = blockIdx.x - g * H;
    if (g >= off[nseg]) return;
    const int s = tile_segment(off, nseg, g);
    const int a = seg_bound(cu, s, T), e = max(seg_bound(cu, s + 1, T), a);
    const int r0 = a + RB * (g - off[s]), rows = min(RB, e - r0);
    const int tid = threadIdx.x, ch = tid & 15, rl = tid >> 4;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int r = rl; r < rows; r += 16) {
        const uint4 u = *reinterpret_cast<const uint4*>(x + ((long)(r0 + r) * H + h) * D + 8 * ch);
        acc[0] += bf16_lo(u.x);
        acc[1] += bf16_hi(u.x);
        acc[2] += bf16_lo(u.y);
        acc[3] += bf16_hi(u.y);
        acc[4] += bf16_lo(u.z);
        acc[5] += bf16_hi(u.z);
        acc[6] += bf16_lo(u.w);
        acc[7] += bf16_hi(u.w);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) red[rl][8 * ch + i] = acc[i];
    __syncthreads();
    if (tid < D) {
        float sum = 0.f;
        for (int j = 0; j < 16; ++j) sum += red[j][tid];
        const long o = kt > 0 ? (((long)h * (D / 4) + (tid >> 2)) * kt + g) * 4 + (tid & 3) : ((long)g * H + h) * D + tid;
        out[o] = sum / (float)rows;
    }
}

struct RouteVarlenArgs {
    const float* qbar;   // [tiles_q][H][128]
    const float* kbar;   // [H][32][ktiles][4]: dimensions 4c..4c+3 of key tile j at [h][c][j]
    const int* off_q;
    const int* off_k;
    int32_t* kidx;       // [tiles_q * H][stride]
    int32_t* kcnt;       // [tiles_q * H]
    int nseg, H, stride, nsink, ktiles;
    float scale, tau;
};

// One workgroup per (query tile g, head h): the proxies of the segment's key tiles into LDS,
// then the threshold and the ordered compaction as route_kernel does.
__global__ __launch_bounds__(256) void route_varlen_kernel(RouteVarlenArgs a) {
    extern __shared__ float zs[];
    __shared__ float red[4];
    __shared__ int wsum[4];
    const int g = blockIdx.x / a.H, h = blockIdx.x - g * a.H;
    if (g >= a.off_q[a.nseg]) return;
    const int s = tile_segment(a.off_q, a.nseg, g);
    const int k0 = a.off_k[s], ntk = a.off_k[s + 1] - k0;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const float* __restrict__ qg = a.qbar + ((long)g * a.H + h) * D;   // wave-uniform (scalar loads)
    const float4* kb = reinterpret_cast<const float4*>(a.kbar) + (long)h * (D / 4) * a.ktiles + k0;
    for (int J = tid; J < ntk; J += 256) {
        float z = 0.f;
#pragma unroll 4
        for (int c4 = 0; c4 < D / 4; ++c4) {
            const float4 kv = kb[(long)c4 * a.ktiles + J];
            z = fmaf(qg[4 * c4 + 0], kv.x, z);
            z = fmaf(qg[4 * c4 + 1], kv.y, z);
            z = fmaf(qg[4 * c4 + 2], kv.z, z);
            z = fmaf(qg[4 * c4 + 3], kv.w, z);
        }
        zs[J] = z * a.scale;
    }
    __syncthreads();
    float m = -INFINITY;
    for (int J = tid; J < ntk; J += 256) m = fmaxf(m, zs[J]);
    const float thr = block_max(m, red) - a.tau;
    const int run = (ntk + 255) / 256;
    const int j0 = min(tid * run, ntk), j1 = min(j0 + run, ntk);
    int cnt = 0;
    for (int J = j0; J < j1; ++J) cnt += (zs[J] >= thr || J < a.nsink) ? 1 : 0;
    int incl = cnt;
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
    }
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    int off = incl - cnt;
    for (int k = 0; k < wv; ++k) off += wsum[k];
    const int total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    const long item = (long)g * a.H + h;
    int32_t* dst = a.kidx + item * a.stride;
    for (int J = j0; J < j1; ++J)
        if (zs[J] >= thr || J < a.nsink) dst[off++] = J;
    if (tid < LIST_PAD) dst[total + tid] = ntk;
    if (tid == 0) a.kcnt[item] = total;
}

// count * H into dst (one thread): the number of (query tile, head) items of a packed batch
__global__ void scale_count_kernel(const int* __restrict__ count, int H, int* __restrict__ dst) {
    *dst = *count * H;
}

// ---------------------------------------------------------------- dispatch order
// Items sorted by their list length, longest first (a bucket sort per workgroup), so that
// the block-sparse kernel starts the long items first and the last round is made of short
// ones. Workgroup g sorts items [g*group, (g+1)*group) among themselves: with group = the
// query tiles of one (b, h), the heads keep their order (the workgroups in flight then share
// one or two heads' K/V in L2, and items of similar length walk the key range in step);
// with group = all items, the sort is global. Within a bucket the order depends on the timing
// of LDS atomics; the attention results do not depend on the order at all.
constexpr int ORDER_BINS = 4096;

__global__ __launch_bounds__(1024) void lpt_order_kernel(const int32_t* __restrict__ kcnt, int items,
                                                         const int* __restrict__ items_dev, int max_cnt,
                                                         int group, int32_t* __restrict__ order) {
    __shared__ int hist[ORDER_BINS];
    __shared__ int part[1024];
    const int tid = threadIdx.x;
    const int n_all = items_dev != nullptr ? min(*items_dev, items) : items;
    const long lo = (long)blockIdx.x * group;
    if (lo >= n_all) return;   // uniform across the workgroup
    const int n = (int)min((long)group, (long)n_all - lo);
    kcnt += lo;
    order += lo;
    const int mc = max(max_cnt, 1);
    auto bin = [&](int c) {   // descending: the longest lists in bin 0
        c = min(max(c, 0), mc);
        return (int)((long)(mc - c) * (ORDER_BINS - 1) / mc);
    };
    for (int b = tid; b < ORDER_BINS; b += 1024) hist[b] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += 1024) atomicAdd(&hist[bin(kcnt[i])], 1);
    __syncthreads();
    constexpr int PER = ORDER_BINS / 1024;
    int local = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) local += hist[tid * PER + j];
    part[tid] = local;
    __syncthreads();
    if (tid == 0) {
        int acc = 0;
        for (int i = 0; i < 1024; ++i) {
            const int v = part[i];
            part[i] = acc;
            acc += v;
        }
    }
    __syncthreads();
    int acc = part[tid];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int v = hist[tid * PER + j];
        hist[tid * PER + j] = acc;
        acc += v;
    }
    __syncthreads();
    for (int i = tid; i < n; i += 1024) order[atomicAdd(&hist[bin(kcnt[i])], 1)] = (int)(lo + i);
}

}  // namespace

namespace attn_impl {

// group: items sorted among themselves per workgroup (0: all items in one workgroup)
hipError_t launch_lpt_order(const int32_t* kv_cnt, int items, const int* items_dev, int max_cnt, int32_t* order,
                            hipStream_t stream, int group = 0) {
    if (group <= 0 || group >= items) group = items > 0 ? items : 1;
    const unsigned grid = (unsigned)(((long)items + group - 1) / group);
    hipLaunchKernelGGL(lpt_order_kernel, dim3(grid > 0 ? grid : 1), dim3(1024), 0, stream, kv_cnt, items, items_dev,
                       max_cnt, group, order);
    return hipGetLastError();
}

size_t route_workspace_bytes(int B, int H, int N) {
    const size_t bh = (size_t)B * H;
    const size_t ntq = (size_t)(N + BMQ - 1) / BMQ, ntk = (size_t)(N + BNK - 1) / BNK;
    const size_t qb = (bh * ntq * D * sizeof(float) + 255) & ~size_t(255);
    return qb + bh * ntk * D * sizeof(float);
}

int route_max_tiles() { return ROUTE_LDS_LIMIT / (int)sizeof(float); }

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

size_t varlen_tiles_q(int nseg, int T) { return (size_t)T / BMQ + (size_t)nseg; }
static size_t varlen_tiles_k(int nseg, int T) { return (size_t)T / BNK + (size_t)nseg; }

// [off_q: nseg + 1][off_k: nseg + 1][item count of the order], each 256-byte aligned
size_t tile_offsets_bytes(int nseg) { return 2 * align256(sizeof(int) * ((size_t)nseg + 1)) + 256; }

hipError_t launch_tile_offsets(const int32_t* cu, int nseg, int T, void* dst, hipStream_t stream) {
    int* off_q = static_cast<int*>(dst);
    int* off_k = reinterpret_cast<int*>(static_cast<char*>(dst) + align256(sizeof(int) * ((size_t)nseg + 1)));
    hipLaunchKernelGGL(tile_offsets_kernel, dim3(1), dim3(1024), 0, stream, cu, nseg, T, off_q, off_k);
    return hipGetLastError();
}

size_t route_varlen_workspace_bytes(int nseg, int H, int T) {
    return tile_offsets_bytes(nseg) + align256(varlen_tiles_q(nseg, T) * H * D * sizeof(float)) +
           varlen_tiles_k(nseg, T) * H * D * sizeof(float);
}

hipError_t launch_block_route_varlen(const void* q, const void* k, const int32_t* cu, int nseg, int H, int T,
                                     float scale, float tau, int sink_tokens, int32_t* kv_idx, int32_t* kv_cnt,
                                     int32_t* order, void* workspace, hipStream_t stream) {
    char* ws = static_cast<char*>(workspace);
    hipError_t e = launch_tile_offsets(cu, nseg, T, ws, stream);
    if (e != hipSuccess) return e;
    const int* off_q = reinterpret_cast<const int*>(ws);
    const int* off_k = reinterpret_cast<const int*>(ws + align256(sizeof(int) * ((size_t)nseg + 1)));
    const size_t tq = varlen_tiles_q(nseg, T), tk = varlen_tiles_k(nseg, T);
    float* qbar = reinterpret_cast<float*>(ws + tile_offsets_bytes(nseg));
    float* kbar = reinterpret_cast<float*>(ws + tile_offsets_bytes(nseg) + align256(tq * H * D * sizeof(float)));
    hipLaunchKernelGGL(pool_varlen_kernel<BMQ>, dim3((unsigned)(tq * H)), dim3(256), 0, stream,
                       static_cast<const bf16*>(q), qbar, cu, off_q, nseg, H, T, 0);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(pool_varlen_kernel<BNK>, dim3((unsigned)(tk * H)), dim3(256), 0, stream,
                       static_cast<const bf16*>(k), kbar, cu, off_k, nseg, H, T, (int)tk);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    RouteVarlenArgs a;
    a.qbar = qbar;
    a.kbar = kbar;
    a.off_q = off_q;
    a.off_k = off_k;
    a.kidx = kv_idx;
    a.kcnt = kv_cnt;
    a.nseg = nseg;
    a.H = H;
    a.ktiles = (int)tk;
    a.stride = (T + BNK - 1) / BNK + LIST_PAD;
    a.nsink = sink_tokens > 0 ? (int)(((long)sink_tokens + BNK - 1) / BNK) : 0;
    a.scale = scale;
    a.tau = tau;
    const size_t lds = (size_t)((T + BNK - 1) / BNK) * sizeof(float);
    hipLaunchKernelGGL(route_varlen_kernel, dim3((unsigned)(tq * H)), dim3(256), lds, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess || order == nullptr) return e;
    // items = (number of query tiles) * H, known on the device only: written into the slot
    // after the offsets, read by the sort
    int* items_dev = reinterpret_cast<int*>(ws + 2 * align256(sizeof(int) * ((size_t)nseg + 1)));
    hipLaunchKernelGGL(scale_count_kernel, dim3(1), dim3(1), 0, stream, off_q + nseg, H, items_dev);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_lpt_order(kv_cnt, (int)(tq * H), items_dev, (T + BNK - 1) / BNK, order, stream);
}

hipError_t launch_block_route(const void* q, const void* k, int B, int H, int N, float scale, float tau,
                              int sink_tokens, int32_t* kv_idx, int32_t* kv_cnt, int32_t* order, void* workspace,
                              hipStream_t stream) {
    const long bh = (long)B * H;
    const int ntq = (N + BMQ - 1) / BMQ, ntk = (N + BNK - 1) / BNK;
    float* qbar = static_cast<float*>(workspace);
    const size_t qb = ((size_t)bh * ntq * D * sizeof(float) + 255) & ~size_t(255);
    float* kbar = reinterpret_cast<float*>(static_cast<char*>(workspace) + qb);
    const unsigned pool_grid = (unsigned)(bh * ((N + 255) / 256));
    hipLaunchKernelGGL((pool_kernel<BMQ, false>), dim3(pool_grid), dim3(256), 0, stream, static_cast<const bf16*>(q), qbar,
                       N, ntq);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((pool_kernel<BNK, true>), dim3(pool_grid), dim3(256), 0, stream, static_cast<const bf16*>(k), kbar,
                       N, ntk);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    RouteArgs a;
    a.qbar = qbar;
    a.kbar = kbar;
    a.kidx = kv_idx;
    a.kcnt = kv_cnt;
    a.ntq = ntq;
    a.ntk = ntk;
    a.stride = ntk + LIST_PAD;
    a.nsink = sink_tokens > 0 ? (int)(((long)sink_tokens + BNK - 1) / BNK) : 0;
    a.scale = scale;
    a.tau = tau;
    if (4 * ntk * (int)sizeof(float) <= ROUTE_LDS_LIMIT) {
        const size_t lds = (size_t)4 * ntk * sizeof(float);
        hipLaunchKernelGGL(route_kernel<4>, dim3((unsigned)(bh * ((ntq + 3) / 4))), dim3(256), lds, stream, a);
    } else {
        const size_t lds = (size_t)ntk * sizeof(float);
        hipLaunchKernelGGL(route_kernel<1>, dim3((unsigned)(bh * ntq)), dim3(256), lds, stream, a);
    }
    e = hipGetLastError();
    if (e != hipSuccess || order == nullptr) return e;
    return launch_lpt_order(kv_cnt, (int)(bh * ntq), nullptr, ntk, order, stream, ntq);
}

}  // namespace attn_impl
