// Selection-stage kernels for gfx950 (CDNA4): pooling, head means, the pooled
// score product on fp32 MFMA, and the per-row top-k with CSR compaction.
//
// What is computed follows the page "automatic/modules/attention/sparse/selector.py"
// (pool_blocks, score_blocks, diagonal_blocks, selection_plan, select_blocks).
// How it is computed is designed for CDNA4: one 64-lane wavefront per pooled
// tile or per selection row, 16-byte coalesced loads, MFMA for the dense
// contraction, ballot/popcount for the compaction.
#include "nsa_internal.h"

#include <float.h>

namespace nsa {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Order LDS traffic between the lanes of one wavefront (no workgroup barrier:
// waves of a workgroup progress independently here).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Wavefront reductions and scans on DPP lane moves (no LDS round trips):
// within each quad by quad permutes, then the half-row and row mirrors give
// every lane its 16-lane row's result, and the four row results are read out.
template <int CTRL>
__device__ __forceinline__ int dpp(int x) { return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false); }
template <typename T, typename F>
__device__ __forceinline__ T wave_reduce(T x, F op) {
    auto bits = [](T v) { return __builtin_bit_cast(int, v); };
    auto val = [](int v) { return __builtin_bit_cast(T, v); };
    x = op(x, val(dpp<0xB1>(bits(x))));   // quad_perm [1, 0, 3, 2]
    x = op(x, val(dpp<0x4E>(bits(x))));   // quad_perm [2, 3, 0, 1]
    x = op(x, val(dpp<0x141>(bits(x))));  // row_half_mirror
    x = op(x, val(dpp<0x140>(bits(x))));  // row_mirror
    auto rd = [&](int l) -> T { return val(__builtin_amdgcn_readlane(bits(x), l)); };
    return op(op(rd(0), rd(16)), op(rd(32), rd(48)));
}
__device__ __forceinline__ int wave_sum_i(int x) { return wave_reduce(x, [](int a, int b) { return a + b; }); }
__device__ __forceinline__ float wave_min_f(float x) { return wave_reduce(x, [](float a, float b) { return fminf(a, b); }); }
__device__ __forceinline__ float wave_max_f(float x) { return wave_reduce(x, [](float a, float b) { return fmaxf(a, b); }); }
// Inclusive prefix sum over the 64 lanes: shifts within each 16-lane row, then
// the last lane of rows 0 / 2 is added to rows 1 / 3 and lane 31 to rows 2 and 3.
__device__ __forceinline__ int wave_prefix_sum(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false); // row_bcast:15 into rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false); // row_bcast:31 into rows 2, 3
    return x;
}

// ---------------------------------------------------------------- pooling
//
// One wavefront pools one tile of `block` token rows of one head. A token row
// of D elements is split into CPR 16-byte chunks; the 64 lanes cover RG = 64/CPR
// rows at a time, so each load instruction of the wave reads 1 KiB of
// contiguous memory. Per lane the sum runs in fp32 over its rows, then the RG
// partial sums are added across lanes and divided by the tile's real length.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void pool_kernel(const void* __restrict__ xv, float* __restrict__ out,
                                                   int S, int block, int ntiles, int64_t total, int64_t x_head_rows,
                                                   int tile0, int64_t out_head_tiles) {
    constexpr int ESZ = BF16 ? 2 : 4;
    constexpr int VEC = 16 / ESZ;      // elements per 16-byte chunk
    constexpr int CPR = D / VEC;       // chunks per token row
    constexpr int RG = 64 / CPR;       // rows in flight per wave instruction
    static_assert(CPR <= 64 && 64 % CPR == 0, "row must split evenly over the wave");
    const int lane = threadIdx.x & 63;
    const int64_t tile = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (tile >= total) return;
    const int64_t head = tile / ntiles;
    const int i = tile0 + (int)(tile - head * ntiles);  // tile index within the head
    const int c = lane % CPR, rg = lane / CPR;
    const int t0 = i * block;
    const int len = min(block, S - t0);
    const char* base = (const char*)xv + ((head * x_head_rows + t0) * (int64_t)D + (int64_t)c * VEC) * ESZ;
    const int64_t row_bytes = (int64_t)D * ESZ;

    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.f;

    auto add = [&](u32x4 w) {
        if constexpr (BF16) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[2 * e] += bf16lo(w[e]);
                acc[2 * e + 1] += bf16hi(w[e]);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] += __uint_as_float(w[e]);
        }
    };

    int r = rg;
    constexpr int U = 8;  // loads in flight per lane
    for (; r + (U - 1) * RG < len; r += U * RG) {
        u32x4 w[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            w[u] = __builtin_nontemporal_load((const u32x4*)(base + (int64_t)(r + u * RG) * row_bytes));
#pragma unroll
        for (int u = 0; u < U; ++u) add(w[u]);
    }
    for (; r < len; r += RG) add(*(const u32x4*)(base + (int64_t)r * row_bytes));

#pragma unroll
    for (int off = CPR; off < 64; off <<= 1) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] += __shfl_xor(acc[e], off);
    }
    if (rg == 0) {
        const float n = (float)len;
        float* o = out + (head * out_head_tiles + i) * D + c * VEC;
#pragma unroll
        for (int e = 0; e < VEC; e += 4) {
            f32x4 v = {acc[e] / n, acc[e + 1] / n, acc[e + 2] / n, acc[e + 3] / n};
            *(f32x4*)(o + e) = v;
        }
    }
}

// ---------------------------------------------------------------- head means
// in: (B, H, Ns, D) with the first N of Ns rows per head used; out: (B, N, D).
__global__ __launch_bounds__(256) void head_mean_kernel(const float* __restrict__ in, float* __restrict__ out,
                                                        int B, int H, int N, int Ns, int D) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t per_b = (int64_t)N * D;
    if (idx >= (int64_t)B * per_b) return;
    const int64_t b = idx / per_b, nd = idx - b * per_b;
    const int64_t head_stride = (int64_t)Ns * D;
    const float* p = in + b * H * head_stride + nd;
    float s = 0.f;
    for (int h = 0; h < H; ++h) s += p[(int64_t)h * head_stride];
    out[idx] = s / (float)H;
}

// ---------------------------------------------------------------- scores
//
// One wavefront computes a 64 x 64 block of one head's score matrix with
// v_mfma_f32_32x32x2_f32 (2 x 2 blocks of 32 x 32). The contraction index is
// split between the two lane halves: at step s lane half hf supplies
// d = kc + 8*hf + s, so every lane reads 8 consecutive floats of its row. The
// pooled operands are small and stay in L2.
template <int D>
__global__ __launch_bounds__(256) void score_kernel(const float* __restrict__ qh, const float* __restrict__ kh,
                                                    int Hsel, int Hk, int group, int h0, int nh, int NQ,
                                                    int NK, int NKs, int nbi, int nbj, float* __restrict__ s) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nbj4 = (nbj + 3) >> 2;
    int64_t wid = blockIdx.x;
    const int bj = (int)(wid % nbj4) * 4 + wave;
    wid /= nbj4;
    const int bi = (int)(wid % nbi);
    wid /= nbi;
    const int hl = (int)(wid % nh);
    const int b = (int)(wid / nh);
    if (bj >= nbj) return;
    const int h = h0 + hl;
    const int hk = (Hk == 1) ? 0 : h / group;
    const float* A = qh + ((int64_t)b * Hsel + h) * NQ * D;
    const float* Bm = kh + ((int64_t)b * Hk + hk) * NKs * D;  // NKs >= NK rows per head
    const int i0 = bi * 64, j0 = bj * 64;
    const int l32 = lane & 31, hf = lane >> 5;
    const float* a0p = A + (int64_t)min(i0 + l32, NQ - 1) * D + 8 * hf;
    const float* a1p = A + (int64_t)min(i0 + 32 + l32, NQ - 1) * D + 8 * hf;
    const float* b0p = Bm + (int64_t)min(j0 + l32, NK - 1) * D + 8 * hf;
    const float* b1p = Bm + (int64_t)min(j0 + 32 + l32, NK - 1) * D + 8 * hf;

    f32x16 c00 = {}, c01 = {}, c10 = {}, c11 = {};
    // Operands of 16 contraction indices per lane-half group: 8 x 16 bytes per
    // lane. Chunks are loaded two ahead of their products (three buffers),
    // so the L2 latency of a chunk overlaps the products of the two before it.
    constexpr int NC = D / 16;
    f32x4 buf[3][8];
    auto load = [&](f32x4 (&o)[8], int kc) {
#pragma unroll
        for (int v = 0; v < 2; ++v) {
            o[0 + v] = *(const f32x4*)(a0p + kc + 4 * v);
            o[2 + v] = *(const f32x4*)(a1p + kc + 4 * v);
            o[4 + v] = *(const f32x4*)(b0p + kc + 4 * v);
            o[6 + v] = *(const f32x4*)(b1p + kc + 4 * v);
        }
    };
    load(buf[0], 0);
    if (NC > 1) load(buf[1], 16);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        if (c + 2 < NC) load(buf[(c + 2) % 3], 16 * (c + 2));
        __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the products
        const f32x4 (&o)[8] = buf[c % 3];
#pragma unroll
        for (int st = 0; st < 8; ++st) {
            const float x0 = o[0 + (st >> 2)][st & 3], x1 = o[2 + (st >> 2)][st & 3];
            const float y0 = o[4 + (st >> 2)][st & 3], y1 = o[6 + (st >> 2)][st & 3];
            c00 = __builtin_amdgcn_mfma_f32_32x32x2f32(x0, y0, c00, 0, 0, 0);
            c01 = __builtin_amdgcn_mfma_f32_32x32x2f32(x0, y1, c01, 0, 0, 0);
            c10 = __builtin_amdgcn_mfma_f32_32x32x2f32(x1, y0, c10, 0, 0, 0);
            c11 = __builtin_amdgcn_mfma_f32_32x32x2f32(x1, y1, c11, 0, 0, 0);
        }
    }
    // Accumulator layout of a 32 x 32 block: lane holds column l32 and rows
    // 8*q + 4*hf + e at element 4*q + e.
    float* out = s + ((int64_t)b * nh + hl) * NQ * NK;
    auto store = [&](const f32x16& c, int ib, int jb) {
        const int col = j0 + jb + l32;
        if (col >= NK) return;
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = i0 + ib + 8 * q + 4 * hf + e;
                if (row < NQ) out[(int64_t)row * NK + col] = c[4 * q + e];
            }
    };
    store(c00, 0, 0);
    store(c01, 0, 32);
    store(c10, 32, 0);
    store(c11, 32, 32);
}

// The same product for many query rows (NQ > 64), one 128 x 256 block per
// workgroup: wave w takes query rows 64 (w / 2) .. + 63 and key columns
// 128 (w % 2) .. + 127 (2 x 4 blocks of 32 x 32 as above). Loading each lane's
// own rows from L2 touches a cache line per lane and every wave of a workgroup
// reloads the rows it shares with the others, so here the operands go through
// LDS in chunks of 32 contraction indices: the workgroup loads the chunk's 128
// pooled-query rows and 256 pooled-key rows with 8 lanes per 128-byte row
// segment, one chunk ahead in registers, and stores them to LDS with rows
// padded to 36 floats (16-byte reads of 16 consecutive rows then fall in
// distinct banks). At step (g, e) of a chunk, lane half hf supplies
// contraction index 16*hf + 4*g + e.
template <int D>
__global__ __launch_bounds__(256) void score_lds_kernel(const float* __restrict__ qh, const float* __restrict__ kh,
                                                        int Hsel, int Hk, int group, int h0, int nh, int NQ,
                                                        int NK, int NKs, int nbi, int nbj, float* __restrict__ s) {
    constexpr int KC = 32, PAD = 36, ROWS = 128, COLS = 256;
    __shared__ __attribute__((aligned(16))) float As[ROWS * PAD];
    __shared__ __attribute__((aligned(16))) float Bs[COLS * PAD];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int64_t wid = blockIdx.x;
    const int bj = (int)(wid % nbj);
    wid /= nbj;
    const int bi = (int)(wid % nbi);
    wid /= nbi;
    const int hl = (int)(wid % nh);
    const int b = (int)(wid / nh);
    const int h = h0 + hl;
    const int hk = (Hk == 1) ? 0 : h / group;
    const float* A = qh + ((int64_t)b * Hsel + h) * NQ * D;
    const float* Bm = kh + ((int64_t)b * Hk + hk) * NKs * D;  // NKs >= NK rows per head
    const int i0 = bi * ROWS, j0 = bj * COLS;

    // Global loads: thread t takes rows t / 8 + 32 x (x < 4), floats 4 (t % 8) .. + 3
    // of the chunk (rows past the end repeat the last row; their results are not stored).
    const int lr = tid >> 3, lq = tid & 7;
    const float* ag[4];
    const float* bg[8];
#pragma unroll
    for (int x = 0; x < 4; ++x) ag[x] = A + (int64_t)min(i0 + lr + 32 * x, NQ - 1) * D + 4 * lq;
#pragma unroll
    for (int x = 0; x < 8; ++x) bg[x] = Bm + (int64_t)min(j0 + lr + 32 * x, NK - 1) * D + 4 * lq;
    f32x4 ra[4], rb[8];
    auto gload = [&](int kc) {
#pragma unroll
        for (int x = 0; x < 4; ++x) ra[x] = *(const f32x4*)(ag[x] + kc);
#pragma unroll
        for (int x = 0; x < 8; ++x) rb[x] = *(const f32x4*)(bg[x] + kc);
    };
    auto lstore = [&]() {
#pragma unroll
        for (int x = 0; x < 4; ++x) *(f32x4*)(As + (lr + 32 * x) * PAD + 4 * lq) = ra[x];
#pragma unroll
        for (int x = 0; x < 8; ++x) *(f32x4*)(Bs + (lr + 32 * x) * PAD + 4 * lq) = rb[x];
    };
    const int wi = wave >> 1, wj = wave & 1;
    const int l32 = lane & 31, hf = lane >> 5;
    const float* a0l = As + (wi * 64 + l32) * PAD + 16 * hf;
    const float* a1l = a0l + 32 * PAD;
    const float* b0l = Bs + (wj * 128 + l32) * PAD + 16 * hf;

    f32x16 c0[4] = {}, c1[4] = {};
    gload(0);
#pragma unroll
    for (int kc = 0; kc < D; kc += KC) {
        __syncthreads();  // the previous chunk's LDS reads are done
        lstore();
        __syncthreads();
        if (kc + KC < D) gload(kc + KC);  // in flight under this chunk's products
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x4 x0 = *(const f32x4*)(a0l + 4 * g), x1 = *(const f32x4*)(a1l + 4 * g);
            f32x4 y[4];
#pragma unroll
            for (int jb = 0; jb < 4; ++jb) y[jb] = *(const f32x4*)(b0l + jb * 32 * PAD + 4 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int jb = 0; jb < 4; ++jb) {
                    c0[jb] = __builtin_amdgcn_mfma_f32_32x32x2f32(x0[e], y[jb][e], c0[jb], 0, 0, 0);
                    c1[jb] = __builtin_amdgcn_mfma_f32_32x32x2f32(x1[e], y[jb][e], c1[jb], 0, 0, 0);
                }
        }
    }
    // Accumulator layout of a 32 x 32 block: lane holds column l32 and rows
    // 8*q + 4*hf + e at element 4*q + e.
    float* out = s + ((int64_t)b * nh + hl) * NQ * NK;
    const int r0 = i0 + wi * 64, cb = j0 + wj * 128;
    auto store = [&](const f32x16& c, int ib, int jb) {
        const int col = cb + jb + l32;
        if (col >= NK) return;
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = r0 + ib + 8 * q + 4 * hf + e;
                if (row < NQ) out[(int64_t)row * NK + col] = c[4 * q + e];
            }
    };
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
        store(c0[jb], 0, 32 * jb);
        store(c1[jb], 32, 32 * jb);
    }
}

// Scores of a few query rows (NQ <= 8, e.g. while decoding): a 64 x 64 MFMA
// block would be almost all padding. A workgroup takes 64 kv tiles of one
// selection head: it stages their pooled keys in LDS with coalesced 16-byte
// loads (rows padded by 4 floats) next to the (at most 8) pooled query rows;
// then four consecutive threads share a tile, each summing a quarter of the
// contraction, and two DPP steps add the four partial sums.
// QIN says what qh holds: 0 the pooled queries (fp32); 1 or 2 the query rows
// themselves (bf16 or fp32), when every query tile is a single token. Such a
// tile's pooled query is 0 + row / 1 in fp32, which is what is staged.
template <int D, int QIN>
__global__ __launch_bounds__(256) void score_rows_kernel(const void* __restrict__ qh, const float* __restrict__ kh,
                                                         int Hsel, int Hk, int group, int h0, int nh, int NQ,
                                                         int NK, int NKs, float* __restrict__ s) {
    constexpr int KP = D + 4, QD = D / 4;
    __shared__ __attribute__((aligned(16))) float qs[8 * D];
    __shared__ __attribute__((aligned(16))) float ks[64 * KP];
    const int tid = threadIdx.x;
    const int nbj = (NK + 63) / 64;
    int64_t wid = blockIdx.x;
    const int jb = (int)(wid % nbj);
    wid /= nbj;
    const int hl = (int)(wid % nh);
    const int b = (int)(wid / nh);
    const int h = h0 + hl;
    const int hk = (Hk == 1) ? 0 : h / group;
    const int64_t qoff = ((int64_t)b * Hsel + h) * NQ * D;
    const float* Bm = kh + ((int64_t)b * Hk + hk) * NKs * D;
    const int j0 = jb * 64;
    if constexpr (QIN == 0) {
        const float* A = (const float*)qh + qoff;
        for (int x = tid; x < NQ * D / 4; x += 256) *(f32x4*)(qs + 4 * x) = *(const f32x4*)(A + 4 * x);
    } else if constexpr (QIN == 1) {
        const uint16_t* A = (const uint16_t*)qh + qoff;
        for (int x = tid; x < NQ * D; x += 256) qs[x] = 0.f + __uint_as_float((uint32_t)A[x] << 16);
    } else {
        const float* A = (const float*)qh + qoff;
        for (int x = tid; x < NQ * D; x += 256) qs[x] = 0.f + A[x];
    }
    for (int x = tid; x < 64 * D / 4; x += 256) {
        const int row = x / (D / 4), c4 = x % (D / 4);
        const int j = min(j0 + row, NK - 1);  // rows past NK repeat the last one and are not stored
        *(f32x4*)(ks + row * KP + 4 * c4) = *(const f32x4*)(Bm + (int64_t)j * D + 4 * c4);
    }
    __syncthreads();
    const int t = tid >> 2, part = tid & 3;
    const float* kr = ks + t * KP + part * QD;
    const float* qr = qs + part * QD;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll 4
    for (int d = 0; d < QD; d += 4) {
        const f32x4 kv = *(const f32x4*)(kr + d);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (i < NQ) {
                const f32x4 qv = *(const f32x4*)(qr + i * D + d);
                acc[i] = __builtin_fmaf(qv[0], kv[0], acc[i]);
                acc[i] = __builtin_fmaf(qv[1], kv[1], acc[i]);
                acc[i] = __builtin_fmaf(qv[2], kv[2], acc[i]);
                acc[i] = __builtin_fmaf(qv[3], kv[3], acc[i]);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if (i < NQ) {
            float v = acc[i];
            v += __builtin_bit_cast(float, dpp<0xB1>(__builtin_bit_cast(int, v)));  // quad_perm [1, 0, 3, 2]
            v += __builtin_bit_cast(float, dpp<0x4E>(__builtin_bit_cast(int, v)));  // quad_perm [2, 3, 0, 1]
            acc[i] = v;
        }
    }
    const int j = j0 + t;
    if (j >= NK) return;
    float* out = s + ((int64_t)b * nh + hl) * NQ * NK;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        if (i < NQ && (i & 3) == part) out[(int64_t)i * NK + j] = acc[i];
}

// ---------------------------------------------------------------- top-k
//
// One wavefront per selection row. Element j = 64*t + lane sits in register
// slot t of lane `lane`, so the 64-bit ballot of slot t is exactly word t of
// the row's bit masks (pins, drops, keep).
//
// Exact top-k by value bucketing: every candidate is mapped to one of 256
// buckets by a function of its score that never decreases as the score grows
// (fp32 subtract and multiply by a positive constant, truncation; the row
// maximum gets the top bucket). Buckets strictly above the bucket holding the
// k-th largest score are taken whole, the rest dropped, and the search repeats
// inside that bucket until what is left is either exactly what is needed or a
// set of equal scores, which is then taken in ascending kv index order. This
// picks the first k candidates in (score descending, index ascending) order;
// -0.0 and +0.0 fall into the same bucket and tie.
template <int EPL>
struct MaskT { typedef uint32_t type; };
template <>
struct MaskT<64> { typedef uint64_t type; };

// Bits lo..hi (clipped to 0..63) of a 64-bit word; empty when lo > hi.
__device__ __forceinline__ uint64_t range_bits(int lo, int hi) {
    lo = lo < 0 ? 0 : lo;
    hi = hi > 63 ? 63 : hi;
    if (lo > hi) return 0ull;
    const uint64_t upto = hi == 63 ? ~0ull : ((1ull << (hi + 1)) - 1ull);
    return upto & ~((1ull << lo) - 1ull);
}

template <int EPL>
__device__ typename MaskT<EPL>::type select_top(const float (&s)[EPL], typename MaskT<EPL>::type active,
                                                int need, uint32_t* hist, int lane) {
    typedef typename MaskT<EPL>::type M;
    constexpr int NB = (EPL + 3) / 4;  // packed bucket bytes
    M picked = 0;
    uint32_t bk[NB];
    for (int iter = 0; iter < 64 && need > 0; ++iter) {
        const int na = wave_sum_i(__builtin_popcountll((uint64_t)active));
        if (na <= need) {
            picked |= active;
            need = 0;
            break;
        }
        float lo = FLT_MAX, hi = -FLT_MAX;
#pragma unroll
        for (int t = 0; t < EPL; ++t) {
            const bool on = (active >> t) & 1;
            lo = fminf(lo, on ? s[t] : FLT_MAX);
            hi = fmaxf(hi, on ? s[t] : -FLT_MAX);
        }
        lo = wave_min_f(lo);
        hi = wave_max_f(hi);
        if (!(hi > lo)) break;  // every remaining score is equal: index order below
        const bool half = !(hi - lo <= FLT_MAX);
        const float lo_u = half ? 0.5f * lo : lo;
        const float range = half ? 0.5f * hi - 0.5f * lo : hi - lo;
        float scale = 255.0f / range;
        if (!(scale <= FLT_MAX)) scale = FLT_MAX;
        for (int q = lane; q < 256; q += 64) hist[q] = 0;
        wave_lds_sync();
#pragma unroll
        for (int w = 0; w < NB; ++w) bk[w] = 0;
#pragma unroll
        for (int t = 0; t < EPL; ++t) {
            // after the first pass few elements remain: slots with none are skipped
            const bool on = (active >> t) & 1;
            if (__ballot(on) == 0) continue;
            const float x = s[t];
            const float u = ((half ? 0.5f * x : x) - lo_u) * scale;
            int b = (int)u;
            b = b > 254 ? 254 : (b < 0 ? 0 : b);
            b = (x == hi) ? 255 : b;
            bk[t >> 2] |= (uint32_t)b << (8 * (t & 3));
            if (on) atomicAdd(&hist[b], 1u);
        }
        wave_lds_sync();
        // Lane L owns buckets 4L .. 4L+3. Count what lies strictly above each.
        const uint32_t h0 = hist[4 * lane], h1 = hist[4 * lane + 1], h2 = hist[4 * lane + 2],
                       h3 = hist[4 * lane + 3];
        const int own = (int)(h0 + h1 + h2 + h3);
        const int incl = wave_prefix_sum(own);
        int ab = __builtin_amdgcn_readlane(incl, 63) - incl;  // sum over lanes with a larger index
        int found = -1, found_above = 0;
        const uint32_t hh[4] = {h3, h2, h1, h0};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (found < 0 && ab < need && need <= ab + (int)hh[e]) {
                found = 4 * lane + 3 - e;
                found_above = ab;
            }
            ab += (int)hh[e];
        }
        wave_lds_sync();
        const uint64_t who = __ballot(found >= 0);
        const int src = __builtin_ctzll(who);
        const int bstar = __builtin_amdgcn_readlane(found, src);
        const int above = __builtin_amdgcn_readlane(found_above, src);
        M next = 0;
#pragma unroll
        for (int t = 0; t < EPL; ++t) {
            const int b = (bk[t >> 2] >> (8 * (t & 3))) & 0xff;
            const M on = (active >> t) & 1;
            picked |= (on & (M)(b > bstar)) << t;
            next |= (on & (M)(b == bstar)) << t;
        }
        active = next;
        need -= above;
    }
    if (need > 0) {
        const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
        for (int t = 0; t < EPL; ++t) {
            const bool on = (active >> t) & 1;
            const uint64_t m = __ballot(on);
            const int cnt = __builtin_popcountll(m);
            if (cnt <= need) {
                if (on) picked |= (M)1 << t;
                need -= cnt;
            } else {
                if (on && __builtin_popcountll(m & below) < need) picked |= (M)1 << t;
                need = 0;
            }
            if (need == 0) break;
        }
    }
    return picked;
}

template <int EPL>
// Up to 2048 kv tiles per row the register budget is held to four waves per
// SIMD: the kernel waits on loads and LDS atomics, and more resident waves
// hide that.
__global__ __launch_bounds__(256, (EPL <= 32 ? 4 : 1)) void topk_kernel(TopkArgs a) {
    typedef typename MaskT<EPL>::type M;
    __shared__ uint32_t hist_all[4][256];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar row math
    uint32_t* hist = hist_all[wave];
    const int64_t lr = (int64_t)blockIdx.x * 4 + wave;
    const int64_t nrows = (int64_t)a.B * a.nh * a.NQ;
    if (lr >= nrows) return;
    const int i = (int)(lr % a.NQ);
    const int64_t bh = lr / a.NQ;
    const int hl = (int)(bh % a.nh);
    const int b = (int)(bh / a.nh);
    const int h = a.h0 + hl;
    const int64_t r = ((int64_t)b * a.Hsel + h) * a.NQ + i;
    const float* srow = a.scores + lr * a.NK;
    const uint64_t* pw =
        a.pin_words ? a.pin_words + (((int64_t)(b % a.pb) * a.ph + (h % a.ph)) * a.NQ + i) * a.NKW : nullptr;
    const uint64_t* dw =
        a.drop_words ? a.drop_words + (((int64_t)(b % a.db) * a.dh + (h % a.dh)) * a.NQ + i) * a.NKW : nullptr;
    // Diagonal: kv tiles j with o + i*bq < (j+1)*bkv and j*bkv < o + (i+1)*bq
    // (o = q_off, the absolute position of the first query token), i.e.
    // floor((o + i*bq)/bkv) <= j <= ceil((o + (i+1)*bq)/bkv) - 1.
    const int dlo = (int)((a.q_off + (int64_t)i * a.block_q) / a.block_kv);
    const int dhi = (int)((a.q_off + (int64_t)(i + 1) * a.block_q + a.block_kv - 1) / a.block_kv) - 1;

    // Scores: slot t of lane L is element 64t + L (index clamped in range;
    // slots past NK are never candidates).
    float s[EPL];
#pragma unroll
    for (int t = 0; t < EPL; ++t) s[t] = srow[min(64 * t + lane, a.NK - 1)];
    // Masks: wave-uniform 64-bit words per slot (bit = lane), built one slot
    // at a time on the scalar unit.
    // The row's mask words arrive with one vector load (lane t holds word t)
    // and are read back per slot with readlane.
    M cand = 0, must_kept = 0;
    int c = 0;
    const int nw = (a.NK + 63) / 64;
    // Mask words from device memory, or (masks shared by every row) from the launch arguments.
    uint64_t pin_l = 0ull, drop_l = 0ull;
    if (lane < nw) {
        if (pw) pin_l = pw[lane];
        else if (a.pin_at >= 0) pin_l = a.words[a.pin_at + lane];
        if (dw) drop_l = dw[lane];
        else if (a.drop_at >= 0) drop_l = a.words[a.drop_at + lane];
    }
#pragma unroll 1
    for (int t = 0; t < EPL; ++t) {
        const int base = 64 * t;
        const int rem = a.NK - base;
        const uint64_t valid = rem >= 64 ? ~0ull : (rem > 0 ? (1ull << rem) - 1ull : 0ull);
        const uint64_t diag = range_bits(dlo - base, dhi - base);
        const uint64_t pin = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(pin_l >> 32), t) << 32) |
                             (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)pin_l, t);
        const uint64_t drop = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(drop_l >> 32), t) << 32) |
                              (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)drop_l, t);
        const uint64_t must = (diag | pin) & valid;
        const uint64_t cw = valid & ~must & ~drop;
        const uint64_t mk = must & ~drop;
        c += __builtin_popcountll(cw);
        cand |= (M)((cw >> lane) & 1ull) << t;
        must_kept |= (M)((mk >> lane) & 1ull) << t;
    }
    // k_r = ceil(fl32(c) * fl32(budget)): the product rounds to fp32 first.
    const float kf = ceilf(__fmul_rn((float)c, a.budget));
    const int k = (kf >= (float)c) ? c : (int)kf;
    M picked = 0;
    if (k >= c) picked = cand;
    else if (k > 0) picked = select_top<EPL>(s, cand, k, hist, lane);
    const M keepm = must_kept | picked;

    int8_t* krow = a.keep + r * a.NK;
    const int32_t row_begin = a.row_src ? a.row_src[r] : (int32_t)(r * a.row_step);
    const int32_t row_end = a.row_src ? a.row_src[r + 1] : (int32_t)((r + 1) * a.row_step);
    const int32_t row_len = row_end - row_begin;  // planned on the host from the same rule
    if (lane == 0) {  // the caller's row offsets (the last row also writes the end)
        a.row_ptr[r] = row_begin;
        if (r + 1 == (int64_t)a.B * a.Hsel * a.NQ) a.row_ptr[r + 1] = row_end;
    }
    int32_t* crow = a.col_idx + row_begin;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int pos = 0;
#pragma unroll
    for (int t = 0; t < EPL; ++t) {
        const int j = 64 * t + lane;
        const bool kb = (keepm >> t) & 1;
        if (j < a.NK) krow[j] = kb ? 1 : 0;
        const uint64_t m = __ballot(kb);
        const int slot = pos + __builtin_popcountll(m & below);
        if (kb && slot < row_len) crow[slot] = j;  // never write past the planned row
        pos += __builtin_popcountll(m);
    }
}

// Top-k of few rows (e.g. decoding: one row per query head): one workgroup
// of four waves per row, so that the row's work is spread over 256 lanes
// instead of the 64 of topk_kernel. Element j = 256 t + 64 w + lane sits in
// slot t of lane `lane` of wave w; the ballot of slot t in wave w is word
// 4 t + w of the row's bit masks. The selection is the bucketing of
// select_top, with candidate counts, extremes, the bucket histogram and the
// index-ordered tie break and compaction reduced over the workgroup in LDS.
template <int EPT>
__global__ __launch_bounds__(256) void topk_rows_kernel(TopkArgs a) {
    typedef uint32_t M;
    __shared__ uint32_t hist[256];
    __shared__ int red_i[4];
    __shared__ float red_lo[4], red_hi[4];
    __shared__ int bsel[2];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t lr = blockIdx.x;
    const int i = (int)(lr % a.NQ);
    const int64_t bh = lr / a.NQ;
    const int hl = (int)(bh % a.nh);
    const int b = (int)(bh / a.nh);
    const int h = a.h0 + hl;
    const int64_t r = ((int64_t)b * a.Hsel + h) * a.NQ + i;
    const float* srow = a.scores + lr * a.NK;
    const uint64_t* pw =
        a.pin_words ? a.pin_words + (((int64_t)(b % a.pb) * a.ph + (h % a.ph)) * a.NQ + i) * a.NKW : nullptr;
    const uint64_t* dw =
        a.drop_words ? a.drop_words + (((int64_t)(b % a.db) * a.dh + (h % a.dh)) * a.NQ + i) * a.NKW : nullptr;
    const int dlo = (int)((a.q_off + (int64_t)i * a.block_q) / a.block_kv);
    const int dhi = (int)((a.q_off + (int64_t)(i + 1) * a.block_q + a.block_kv - 1) / a.block_kv) - 1;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

    auto block_sum = [&](int x) -> int {  // x wave-uniform
        if (lane == 0) red_i[wave] = x;
        __syncthreads();
        const int t = red_i[0] + red_i[1] + red_i[2] + red_i[3];
        __syncthreads();
        return t;
    };

    float sc[EPT];
#pragma unroll
    for (int t = 0; t < EPT; ++t) sc[t] = srow[min(256 * t + 64 * wave + lane, a.NK - 1)];

    // Masks: word 4 t + w of the row (lane x < EPT holds word 4 x + w).
    const int nw = (a.NK + 63) / 64;
    const int wx = 4 * lane + wave;
    // Mask words from device memory, or (masks shared by every row) from the launch arguments.
    uint64_t pin_l = 0ull, drop_l = 0ull;
    if (lane < EPT && wx < nw) {
        if (pw) pin_l = pw[wx];
        else if (a.pin_at >= 0) pin_l = a.words[a.pin_at + wx];
        if (dw) drop_l = dw[wx];
        else if (a.drop_at >= 0) drop_l = a.words[a.drop_at + wx];
    }
    M cand = 0, must_kept = 0;
    int cw_count = 0;
#pragma unroll
    for (int t = 0; t < EPT; ++t) {
        const int base = 64 * (4 * t + wave);
        const int rem = a.NK - base;
        const uint64_t valid = rem >= 64 ? ~0ull : (rem > 0 ? (1ull << rem) - 1ull : 0ull);
        const uint64_t diag = range_bits(dlo - base, dhi - base);
        const uint64_t pin = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(pin_l >> 32), t) << 32) |
                             (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)pin_l, t);
        const uint64_t drop = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(drop_l >> 32), t) << 32) |
                              (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)drop_l, t);
        const uint64_t must = (diag | pin) & valid;
        const uint64_t cw = valid & ~must & ~drop;
        const uint64_t mk = must & ~drop;
        cw_count += __builtin_popcountll(cw);
        cand |= (M)((cw >> lane) & 1ull) << t;
        must_kept |= (M)((mk >> lane) & 1ull) << t;
    }
    const int c = block_sum(cw_count);
    const float kf = ceilf(__fmul_rn((float)c, a.budget));
    const int k = (kf >= (float)c) ? c : (int)kf;

    M picked = 0;
    if (k >= c) {
        picked = cand;
    } else if (k > 0) {
        M active = cand;
        int need = k;
        uint32_t bk[(EPT + 3) / 4];
        for (int iter = 0; iter < 64 && need > 0; ++iter) {
            const int na = block_sum(wave_sum_i(__builtin_popcount(active)));
            if (na <= need) {
                picked |= active;
                need = 0;
                break;
            }
            float lo = FLT_MAX, hi = -FLT_MAX;
#pragma unroll
            for (int t = 0; t < EPT; ++t) {
                const bool on = (active >> t) & 1;
                lo = fminf(lo, on ? sc[t] : FLT_MAX);
                hi = fmaxf(hi, on ? sc[t] : -FLT_MAX);
            }
            lo = wave_min_f(lo);
            hi = wave_max_f(hi);
            if (lane == 0) {
                red_lo[wave] = lo;
                red_hi[wave] = hi;
            }
            hist[tid] = 0;
            __syncthreads();
            lo = fminf(fminf(red_lo[0], red_lo[1]), fminf(red_lo[2], red_lo[3]));
            hi = fmaxf(fmaxf(red_hi[0], red_hi[1]), fmaxf(red_hi[2], red_hi[3]));
            if (!(hi > lo)) break;  // every remaining score is equal: index order below (uniform)
            const bool half = !(hi - lo <= FLT_MAX);
            const float lo_u = half ? 0.5f * lo : lo;
            const float range = half ? 0.5f * hi - 0.5f * lo : hi - lo;
            float scale = 255.0f / range;
            if (!(scale <= FLT_MAX)) scale = FLT_MAX;
#pragma unroll
            for (int w = 0; w < (EPT + 3) / 4; ++w) bk[w] = 0;
#pragma unroll
            for (int t = 0; t < EPT; ++t) {
                const bool on = (active >> t) & 1;
                const float x = sc[t];
                const float u = ((half ? 0.5f * x : x) - lo_u) * scale;
                int bb = (int)u;
                bb = bb > 254 ? 254 : (bb < 0 ? 0 : bb);
                bb = (x == hi) ? 255 : bb;
                bk[t >> 2] |= (uint32_t)bb << (8 * (t & 3));
                if (on) atomicAdd(&hist[bb], 1u);
            }
            __syncthreads();
            if (wave == 0) {  // lane L owns buckets 4L .. 4L+3; count what lies strictly above each
                const uint32_t h0 = hist[4 * lane], h1 = hist[4 * lane + 1], h2 = hist[4 * lane + 2],
                               h3 = hist[4 * lane + 3];
                const int own = (int)(h0 + h1 + h2 + h3);
                const int incl = wave_prefix_sum(own);
                int ab = __builtin_amdgcn_readlane(incl, 63) - incl;
                int found = -1, found_above = 0;
                const uint32_t hh[4] = {h3, h2, h1, h0};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (found < 0 && ab < need && need <= ab + (int)hh[e]) {
                        found = 4 * lane + 3 - e;
                        found_above = ab;
                    }
                    ab += (int)hh[e];
                }
                if (found >= 0) {  // exactly one lane
                    bsel[0] = found;
                    bsel[1] = found_above;
                }
            }
            __syncthreads();
            const int bstar = bsel[0], above = bsel[1];
            M next = 0;
#pragma unroll
            for (int t = 0; t < EPT; ++t) {
                const int bb = (bk[t >> 2] >> (8 * (t & 3))) & 0xff;
                const M on = (active >> t) & 1;
                picked |= (on & (M)(bb > bstar)) << t;
                next |= (on & (M)(bb == bstar)) << t;
            }
            active = next;
            need -= above;
            __syncthreads();  // bsel and hist are rewritten by the next pass
        }
        if (need > 0) {  // equal scores: the lowest kv indices first
            for (int t = 0; t < EPT && need > 0; ++t) {
                const bool on = (active >> t) & 1;
                const uint64_t m = __ballot(on);
                if (lane == 0) red_i[wave] = __builtin_popcountll(m);
                __syncthreads();
                int prior = 0;
                for (int w = 0; w < wave; ++w) prior += red_i[w];
                const int total = red_i[0] + red_i[1] + red_i[2] + red_i[3];
                __syncthreads();
                if (total <= need) {
                    if (on) picked |= (M)1 << t;
                    need -= total;
                } else {
                    if (on && prior + __builtin_popcountll(m & below) < need) picked |= (M)1 << t;
                    need = 0;
                }
            }
        }
    }
    const M keepm = must_kept | picked;

    int8_t* krow = a.keep + r * a.NK;
    const int32_t row_begin = a.row_src ? a.row_src[r] : (int32_t)(r * a.row_step);
    const int32_t row_end = a.row_src ? a.row_src[r + 1] : (int32_t)((r + 1) * a.row_step);
    const int32_t row_len = row_end - row_begin;  // planned on the host from the same rule
    if (tid == 0) {  // the caller's row offsets (the last row also writes the end)
        a.row_ptr[r] = row_begin;
        if (r + 1 == (int64_t)a.B * a.Hsel * a.NQ) a.row_ptr[r + 1] = row_end;
    }
    int32_t* crow = a.col_idx + row_begin;
    int pos = 0;
#pragma unroll
    for (int t = 0; t < EPT; ++t) {
        const int j = 256 * t + 64 * wave + lane;
        const bool kb = (keepm >> t) & 1;
        if (j < a.NK) krow[j] = kb ? 1 : 0;
        const uint64_t m = __ballot(kb);
        if (lane == 0) red_i[wave] = __builtin_popcountll(m);
        __syncthreads();
        int prior = 0;
        for (int w = 0; w < wave; ++w) prior += red_i[w];
        const int total = red_i[0] + red_i[1] + red_i[2] + red_i[3];
        __syncthreads();
        const int slot = pos + prior + __builtin_popcountll(m & below);
        if (kb && slot < row_len) crow[slot] = j;  // never write past the planned row
        pos += total;
    }
}

}  // namespace

// ---------------------------------------------------------------- launchers

hipError_t launch_pool_range(const void* x, int bf16, int64_t heads, int S, int64_t x_head_rows, int D, int block,
                             int tile0, int ntiles, float* out, int64_t out_head_tiles, hipStream_t stream) {
    const int64_t total = heads * ntiles;
    if (total == 0) return hipSuccess;
    const dim3 grid((unsigned)((total + 3) / 4));
#define NSA_POOL(DD, BB)                                                                                 \
    hipLaunchKernelGGL((pool_kernel<DD, BB>), grid, dim3(256), 0, stream, x, out, S, block, ntiles, total, \
                       x_head_rows, tile0, out_head_tiles)
    if (bf16) {
        if (D == 64) NSA_POOL(64, true);
        else if (D == 128) NSA_POOL(128, true);
        else if (D == 256) NSA_POOL(256, true);
        else return hipErrorInvalidValue;
    } else {
        if (D == 64) NSA_POOL(64, false);
        else if (D == 128) NSA_POOL(128, false);
        else if (D == 256) NSA_POOL(256, false);
        else return hipErrorInvalidValue;
    }
#undef NSA_POOL
    return hipGetLastError();
}

hipError_t launch_pool(const void* x, int bf16, int64_t heads, int S, int D, int block, float* out,
                       hipStream_t stream) {
    const int ntiles = (S + block - 1) / block;
    return launch_pool_range(x, bf16, heads, S, S, D, block, 0, ntiles, out, ntiles, stream);
}

hipError_t launch_head_mean(const float* in, int B, int H, int N, int D, float* out, hipStream_t stream,
                            int Ns) {
    const int64_t total = (int64_t)B * N * D;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(head_mean_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, in,
                       out, B, H, N, Ns > 0 ? Ns : N, D);
    return hipGetLastError();
}

hipError_t launch_scores(const void* qh, const float* kh, int B, int Hsel, int Hk, int group, int h0, int nh,
                         int NQ, int NK, int D, float* s, hipStream_t stream, int NKs, int q_rows) {
    if (NKs <= 0) NKs = NK;
    if (NQ == 0 || NK == 0 || nh == 0 || B == 0) return hipSuccess;
    if (q_rows != 0 && NQ > 8) return hipErrorInvalidValue;
    if (NQ <= 8) {
        const dim3 g((unsigned)((int64_t)B * nh * ((NK + 63) / 64)));
#define NSA_ROWS(DD, QI)                                                                                          \
    hipLaunchKernelGGL((score_rows_kernel<DD, QI>), g, dim3(256), 0, stream, qh, kh, Hsel, Hk, group, h0, nh, NQ, \
                       NK, NKs, s)
#define NSA_ROWS_D(QI)                      \
    if (D == 64) NSA_ROWS(64, QI);          \
    else if (D == 128) NSA_ROWS(128, QI);   \
    else if (D == 256) NSA_ROWS(256, QI);   \
    else return hipErrorInvalidValue;
        if (q_rows == 0) NSA_ROWS_D(0)
        else if (q_rows == 1) NSA_ROWS_D(1)
        else NSA_ROWS_D(2)
#undef NSA_ROWS_D
#undef NSA_ROWS
        return hipGetLastError();
    }
    const float* qf = (const float*)qh;
    if (NQ > 64) {
        const int nbi = (NQ + 127) / 128, nbj = (NK + 255) / 256;
        const dim3 grid((unsigned)((int64_t)B * nh * nbi * nbj));
#define NSA_SCORE_LDS(DD)                                                                                     \
    hipLaunchKernelGGL((score_lds_kernel<DD>), grid, dim3(256), 0, stream, qf, kh, Hsel, Hk, group, h0, nh, NQ, \
                       NK, NKs, nbi, nbj, s)
        if (D == 64) NSA_SCORE_LDS(64);
        else if (D == 128) NSA_SCORE_LDS(128);
        else if (D == 256) NSA_SCORE_LDS(256);
        else return hipErrorInvalidValue;
#undef NSA_SCORE_LDS
        return hipGetLastError();
    }
    const int nbi = (NQ + 63) / 64, nbj = (NK + 63) / 64;
    const int64_t blocks = (int64_t)B * nh * nbi * ((nbj + 3) / 4);
    const dim3 grid((unsigned)blocks);
#define NSA_SCORE(DD)                                                                                 \
    hipLaunchKernelGGL((score_kernel<DD>), grid, dim3(256), 0, stream, qf, kh, Hsel, Hk, group, h0, nh, NQ, \
                       NK, NKs, nbi, nbj, s)
    if (D == 64) NSA_SCORE(64);
    else if (D == 128) NSA_SCORE(128);
    else if (D == 256) NSA_SCORE(256);
    else return hipErrorInvalidValue;
#undef NSA_SCORE
    return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t stream) {
    const int64_t rows = (int64_t)a.B * a.nh * a.NQ;
    if (rows == 0 || a.NK == 0) return hipSuccess;
    if (rows <= 1024 && a.NK <= 4096) {  // few rows: a workgroup per row
        const int ept = (a.NK + 255) / 256;
#define NSA_TOPK_ROWS(E) hipLaunchKernelGGL((topk_rows_kernel<E>), dim3((unsigned)rows), dim3(256), 0, stream, a)
        if (ept <= 1) NSA_TOPK_ROWS(1);
        else if (ept <= 2) NSA_TOPK_ROWS(2);
        else if (ept <= 4) NSA_TOPK_ROWS(4);
        else if (ept <= 8) NSA_TOPK_ROWS(8);
        else NSA_TOPK_ROWS(16);
#undef NSA_TOPK_ROWS
        return hipGetLastError();
    }
    const dim3 grid((unsigned)((rows + 3) / 4));
    const int epl = (a.NK + 63) / 64;
#define NSA_TOPK(E) hipLaunchKernelGGL((topk_kernel<E>), grid, dim3(256), 0, stream, a)
    if (epl <= 1) NSA_TOPK(1);
    else if (epl <= 2) NSA_TOPK(2);
    else if (epl <= 4) NSA_TOPK(4);
    else if (epl <= 8) NSA_TOPK(8);
    else if (epl <= 16) NSA_TOPK(16);
    else if (epl <= 32) NSA_TOPK(32);
    else if (epl <= 64) NSA_TOPK(64);
    else return hipErrorInvalidValue;
#undef NSA_TOPK
    return hipGetLastError();
}

}  // namespace nsa
