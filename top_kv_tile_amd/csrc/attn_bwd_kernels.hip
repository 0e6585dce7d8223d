// Gradients of block-sparse attention for gfx950 (CDNA4).
//
// The forward is softmax attention of each query over the keys of the kv
// tiles its query tile keeps (keep flags / CSR of the selection defined on the
// page "automatic/modules/attention/sparse/selector.py", BlockSelection), with
// GQA, an optional causal mask and scale D^-1/2. Given dO and the forward's
// LSE, with P_tu = exp(scale q_t.k_u - LSE_t) on visible pairs:
//   Delta_t = dO_t . O_t
//   dP_tu = dO_t . v_u,  dS_tu = P_tu (dP_tu - Delta_t)
//   dQ_t = scale sum_u dS_tu k_u
//   dK_u = scale sum_t dS_tu q_t,  dV_u = sum_t P_tu dO_t   (summed over the heads of a GQA group)
// Tiles entirely in the causal future are skipped as in the forward.
//
// Kernels:
//  * delta_kernel: Delta per query row.
//  * colcount_kernel / colscan_kernel / colfill_kernel: the kv-tile-major
//    index of the keep flags (for each selection head and kv tile, the query
//    tiles that keep it, ascending).
//  * bwd_dq_mfma_kernel: one workgroup per (batch, query head, query tile),
//    walking the query-major CSR like the forward. S^T = K Q^T and
//    dP^T = V dO^T, then dQ^T += K^T dS^T with K^T read from the row-major K
//    tile by transposing LDS reads.
//  * bwd_dkdv_mfma_kernel: one workgroup per (batch, kv head, kv tile),
//    walking the kv-tile-major index over the query heads of the group in
//    64-query chunks. S = Q K^T and dP = dO V^T, then dV^T += dO^T P and
//    dK^T += Q^T dS with Q^T / dO^T read by transposing LDS reads.
//  * bwd_dq_simt_kernel / bwd_dkdv_simt_kernel: fp32 FMA fallback for fp32
//    inputs and block sizes the MFMA kernels do not take.
#include "nsa_internal.h"
#include "device_common.h"

#include <math.h>
#include <type_traits>

namespace nsa {
namespace {

constexpr float kPosInf = __builtin_huge_valf();
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLog2e = 1.44269504088896340736f;

// LSE in log2 units as the exponent offset of P; an empty row (LSE = -inf)
// maps to +inf so that every P of that row is exactly 0.
__device__ __forceinline__ float lse_offset(float lse) { return lse == kNegInf ? kPosInf : lse * kLog2e; }

__device__ __forceinline__ float load_elem(const void* base, int64_t idx, bool bf16) {
    if (bf16) return __uint_as_float((uint32_t)((const uint16_t*)base)[idx] << 16);
    return ((const float*)base)[idx];
}
__device__ __forceinline__ uint16_t to_bf16_bits(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// ============================================================ preprocessing

// Delta[r] = sum_d dO[r, d] * O[r, d] in fp32; D / 8 lanes per row, 8 elements per lane.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void delta_kernel(const void* out, const void* dout, float* delta, int64_t rows) {
    constexpr int LPR = D / 8;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t r = t / LPR;
    const int part = (int)(t % LPR);
    float acc = 0.f;
    if (r < rows) {
        const int64_t base = r * D + part * 8;
#pragma unroll
        for (int x = 0; x < 8; ++x) acc += load_elem(dout, base + x, BF16) * load_elem(out, base + x, BF16);
    }
#pragma unroll
    for (int o = LPR / 2; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
    if (r < rows && part == 0) delta[r] = acc;
}

// Column index of the keep flags. A workgroup takes 64 columns of one slab
// (one lane per column, so each wave load reads 64 consecutive flags) and its
// four waves take a quarter of the query tiles each.
// counts4[(bh * NK + j) * 4 + w] = query tiles i of quarter w with keep[bh, i, j] != 0.
__global__ __launch_bounds__(256) void colcount_kernel(const int8_t* keep, int NQ, int NK, int32_t* counts4) {
    const int per = (NK + 63) / 64;
    const int64_t bh = blockIdx.x / per;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int j = (int)(blockIdx.x % per) * 64 + lane;
    if (j >= NK) return;
    const int q = (NQ + 3) / 4;
    const int i0 = min(NQ, w * q), i1 = min(NQ, i0 + q);
    const int8_t* col = keep + bh * NQ * (int64_t)NK + j;
    int c = 0;
#pragma unroll 8
    for (int i = i0; i < i1; ++i) c += col[(int64_t)i * NK] != 0;
    counts4[(bh * NK + j) * 4 + w] = c;
}

// Exclusive prefix sum over columns of the column totals (sum of the four
// quarters): col_ptr[0 .. n], in three launches. Block b of colscan_block
// scans 2048 columns and writes its total to sums[b]; colscan_sums scans the
// block totals (one workgroup); colscan_add adds each block's offset. Offsets
// are clamped to cap (the capacity of row_idx) so that flags that disagree
// with the CSR cannot index past it.
__device__ __forceinline__ int32_t block_scan_256(int32_t v, int32_t* sh, int32_t& total) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    int32_t x = v;  // inclusive scan within the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int32_t y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) sh[w] = x;
    __syncthreads();
    int32_t off = 0;
    for (int u = 0; u < w; ++u) off += sh[u];
    total = sh[0] + sh[1] + sh[2] + sh[3];
    __syncthreads();
    return off + x - v;  // exclusive
}
__global__ __launch_bounds__(256) void colscan_block_kernel(const int32_t* counts4, int64_t n, int32_t* col_ptr,
                                                            int32_t* sums) {
    __shared__ int32_t sh[4];
    const int64_t base = (int64_t)blockIdx.x * 2048 + threadIdx.x * 8;
    int32_t v[8], t = 0;
#pragma unroll
    for (int x = 0; x < 8; ++x) {
        const int64_t c = base + x;
        if (c < n) {
            const int4 q = *(const int4*)(counts4 + c * 4);
            v[x] = q.x + q.y + q.z + q.w;
        } else {
            v[x] = 0;
        }
        t += v[x];
    }
    int32_t total;
    int32_t run = block_scan_256(t, sh, total);
#pragma unroll
    for (int x = 0; x < 8; ++x) {
        if (base + x < n) col_ptr[base + x] = run;
        run += v[x];
    }
    if (threadIdx.x == 0) sums[blockIdx.x] = total;
}
__global__ __launch_bounds__(256) void colscan_sums_kernel(int32_t* sums, int nb) {
    __shared__ int32_t sh[4];
    int32_t carry = 0;
    for (int b0 = 0; b0 < nb; b0 += 256) {
        const int b = b0 + threadIdx.x;
        const int32_t v = b < nb ? sums[b] : 0;
        int32_t total;
        const int32_t ex = block_scan_256(v, sh, total);
        if (b < nb) sums[b] = carry + ex;  // exclusive offset of block b
        carry += total;
    }
    if (threadIdx.x == 0) sums[nb] = carry;
}
__global__ __launch_bounds__(256) void colscan_add_kernel(int32_t* col_ptr, const int32_t* sums, int64_t n,
                                                          int nb, int32_t cap) {
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c < n) col_ptr[c] = min(col_ptr[c] + sums[c / 2048], cap);
    if (c == n) col_ptr[n] = min(sums[nb], cap);
}

// row_idx[col_ptr[bh * NK + j] ..] = the query tiles keeping (bh, j), ascending:
// the same geometry as colcount, each wave starting after the flags of the
// quarters before it.
__global__ __launch_bounds__(256) void colfill_kernel(const int8_t* keep, int NQ, int NK, const int32_t* counts4,
                                                      const int32_t* col_ptr, int32_t* row_idx) {
    const int per = (NK + 63) / 64;
    const int64_t bh = blockIdx.x / per;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int j = (int)(blockIdx.x % per) * 64 + lane;
    if (j >= NK) return;
    const int q = (NQ + 3) / 4;
    const int i0 = min(NQ, w * q), i1 = min(NQ, i0 + q);
    const int64_t c = bh * NK + j;
    int32_t p = col_ptr[c];
    for (int u = 0; u < w; ++u) p += counts4[c * 4 + u];
    const int32_t p_end = col_ptr[c + 1];
    const int8_t* col = keep + bh * NQ * (int64_t)NK + j;
    for (int i = i0; i < i1 && p < p_end; ++i)
        if (col[(int64_t)i * NK] != 0) row_idx[p++] = i;
}

// ============================================================ shared helpers

// Range of query-major CSR entries for query tile (b, h, i) up to query q_last.
__device__ __forceinline__ void q_tile_range(const AttnBwdArgs& a, int b, int h, int i, int q_last, int& start,
                                             int& end) {
    if (a.row_ptr) {
        const int hs = (a.Hsel == 1) ? 0 : h;
        const int64_t r = ((int64_t)(a.Bsel == 1 ? 0 : b) * a.Hsel + hs) * a.NQ + i;
        start = a.row_ptr[r];
        end = a.row_ptr[r + 1];
        if (a.causal) {
            int lo = start, hi = end;  // first entry starting after q_last
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if ((int64_t)a.col_idx[mid] * a.block_kv > q_last) hi = mid;
                else lo = mid + 1;
            }
            end = lo;
        }
    } else {
        start = 0;
        end = a.NK;
        if (a.causal) end = min(a.NK, q_last / a.block_kv + 1);
    }
}

// The same range found by a whole wavefront before any tile is in flight: the
// causal end is counted 64 entries at a time with one vector load and a ballot
// (visible entries form a prefix of the ascending list).
__device__ __forceinline__ void q_tile_range_wave(const AttnBwdArgs& a, int b, int h, int i, int q_last, int lane,
                                                  int& start, int& end) {
    if (!a.row_ptr || !a.causal) {
        q_tile_range(a, b, h, i, q_last, start, end);
        return;
    }
    const int hs = (a.Hsel == 1) ? 0 : h;
    const int64_t r = ((int64_t)(a.Bsel == 1 ? 0 : b) * a.Hsel + hs) * a.NQ + i;
    start = a.row_ptr[r];
    const int row_end = a.row_ptr[r + 1];
    end = start;
    for (int base = start; base < row_end; base += 64) {
        const int e = base + lane;
        const bool vis = e < row_end && (int64_t)a.col_idx[e] * a.block_kv <= q_last;
        const int nvis = __builtin_popcountll(__ballot(vis));
        end = base + nvis;
        if (nvis < min(64, row_end - base)) break;
    }
}

// Range of kv-tile-major entries for kv tile (b, selection head hs, j), trimmed
// under causal to query tiles whose last row reaches key0. Dense: all tiles.
__device__ __forceinline__ void kv_tile_range(const AttnBwdArgs& a, int b, int hs, int j, int key0, int& start,
                                              int& end) {
    if (a.col_ptr) {
        const int64_t c = ((int64_t)(a.Bsel == 1 ? 0 : b) * a.Hsel + hs) * a.NK + j;
        start = ld_scalar(a.col_ptr, c);
        end = ld_scalar(a.col_ptr, c + 1);
        if (a.causal) {
            int lo = start, hi = end;  // first entry whose tile ends at or after key0
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if ((int64_t)ld_scalar(a.row_idx, mid) * a.block_q + a.block_q - 1 >= key0) hi = mid;
                else lo = mid + 1;
            }
            start = lo;
        }
    } else {
        start = a.causal ? key0 / a.block_q : 0;
        end = a.NQ;
    }
}
__device__ __forceinline__ int kv_entry(const AttnBwdArgs& a, int e) { return a.row_idx ? ld_scalar(a.row_idx, e) : e; }

// ============================================================ MFMA geometry
//
// A 64-row tile of D bf16 per row, row-major in LDS, filled by buffer-to-LDS
// DMA (1 KiB per wave instruction). Rows are XOR-swizzled in 16-byte chunks.
// Tiles read only as rows (16 bytes per lane, 32 consecutive rows per
// instruction) use rswz = x = (row / RPB) % CH. Tiles read both as rows and
// transposed (ds_read_b64_tr_b16: 4 consecutive rows x 4 columns of 8 bytes
// per 16 lanes) use bswz = x ^ 4 (x % 4) (x % 2 at D = 64): the row-read
// swizzle combined with the one that makes transposed reads conflict-free.
// Measured with SQ_LDS_BANK_CONFLICT on gfx950 at D = 128: x alone costs ~6
// conflict cycles per transposed read, 4 (x % 4) alone ~6 per row read, and
// x ^ 4 (x % 4) none for either.
template <int D>
struct Geo {
    static constexpr int ROWB = D * 2;
    static constexpr int CH = ROWB / 16;
    static constexpr int RPB = 256 / ROWB;
    static constexpr int TILEB = 64 * ROWB;
    static constexpr int RPI = 1024 / ROWB;
    static constexpr int NINSTR = TILEB / 1024;
    __device__ static int rswz(int row) { return (row / RPB) % CH; }
    __device__ static int bswz(int row) {
        const int x = (row / RPB) % CH;
        return x ^ ((4 * (x % 4)) % CH);
    }
};

// DMA of one 64-row tile (rows row0 .. row0 + 63 of a head, clamped to S - 1)
// into `dst`, by the NW waves of the workgroup. `swz` picks the swizzle.
template <int D, int NW, bool BOTH>
__device__ __forceinline__ void dma_tile(__amdgpu_buffer_rsrc_t rs, char* dst, int row0, int S, int wave, int lane) {
    using G = Geo<D>;
#pragma unroll
    for (int x = 0; x < (G::NINSTR + NW - 1) / NW; ++x) {
        const int ii = wave + NW * x;
        if (G::NINSTR % NW == 0 || ii < G::NINSTR) {
            const int row = ii * G::RPI + lane / G::CH, pc = lane % G::CH;
            const int chunk = pc ^ (BOTH ? G::bswz(row) : G::rswz(row));
            const int off = min(row0 + row, S - 1) * G::ROWB + chunk * 16;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + ii * 1024), 16, off, 0, 0, 0);
        }
    }
}

// 16-byte row fragment: row `row`, logical chunk `chunk`.
template <int D, bool BOTH>
__device__ __forceinline__ bf16x8 row_frag(const char* tile, int row, int chunk) {
    using G = Geo<D>;
    const int pc = chunk ^ (BOTH ? G::bswz(row) : G::rswz(row));
    return __builtin_bit_cast(bf16x8, *(const u32x4*)(tile + row * G::ROWB + pc * 16));
}

// Transposed A fragment for a 32x32x16 MFMA whose contraction runs over tile
// rows: lane (l32, hf) receives column d = 32 m + l32 at rows
// r0 + 4 hf + (0..3) and r0 + 8 + 4 hf + (0..3). Within each 16-lane group,
// ds_read_b64_tr_b16 gives result element e of lane i from element (i mod 4)
// of the 8 bytes addressed by lane 4e + i/4.
template <int D>
__device__ __forceinline__ bf16x8 tr_frag(const char* tile, int r0, int m, int lane) {
    using G = Geo<D>;
    const int vg = lane >> 4, vs = lane & 15, hf = lane >> 5;
    const int d = 32 * m + 16 * (vg & 1) + 4 * (vs & 3);
    const int row0 = r0 + 4 * hf + (vs >> 2);
    const int row1 = row0 + 8;
    const int c = d >> 3, b = (d & 7) * 2;
    const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s4*)(tile + row0 * G::ROWB + ((c ^ G::bswz(row0)) * 16) + b));
    const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s4*)(tile + row1 * G::ROWB + ((c ^ G::bswz(row1)) * 16) + b));
    const short8_t w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, w);
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) { return mfma32(a, b, c); }

// DMA of one 64-row tile (rows row0 .. row0 + 63 of a head, clamped to S - 1)
// into LDS byte address dst, by the NW waves of the workgroup (bswz layout).
template <int D, int NW>
__device__ __forceinline__ void dma_tile_asm(u32x4 rs, uint32_t dst, int row0, int S, int wave, int lane) {
    using G = Geo<D>;
    static_assert(G::NINSTR % NW == 0, "every wave issues the same number of DMA instructions");
#pragma unroll
    for (int x = 0; x < G::NINSTR / NW; ++x) {
        const int ii = wave + NW * x;
        const int row = ii * G::RPI + lane / G::CH, pc = lane % G::CH;
        const int chunk = pc ^ G::bswz(row);
        dma16(rs, dst + ii * 1024, min(row0 + row, S - 1) * G::ROWB + chunk * 16);
    }
}

// ============================================================ dQ (MFMA)
//
// Work item order as in the forward: kv-head major, query tile descending,
// query head fastest, runs of 64 blocks spread over the 8 XCDs.
struct Work {
    int b, h, g, i;
};
__device__ __forceinline__ Work decode_q_work(int64_t n, int64_t total, int Hq, int Hkv, int NQ) {
    int64_t w = n;
    const int64_t full = (total / 64) * 64;
    if (n < full) {
        const int64_t run = n >> 6;
        const int r = (int)(n & 63);
        w = run * 64 + (r & 7) * 8 + (r >> 3);
    }
    const int G = Hq / Hkv;
    Work wk;
    const int hh = (int)(w % G);
    w /= G;
    wk.i = NQ - 1 - (int)(w % NQ);
    w /= NQ;
    wk.g = (int)(w % Hkv);
    wk.b = (int)(w / Hkv);
    wk.h = wk.g * G + hh;
    return wk;
}

template <int D, int NW>
__global__ __launch_bounds__(64 * NW, 2) void bwd_dq_mfma_kernel(AttnBwdArgs a) {
    constexpr int KSTEPS = D / 16;
    constexpr int DBLK = D / 32;
    using G = Geo<D>;
    extern __shared__ __attribute__((aligned(1024))) char lds[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hf = lane >> 5;
    const int64_t total = (int64_t)a.B * a.Hq * a.NQ;
    const Work wk = decode_q_work(blockIdx.x, total, a.Hq, a.Hkv, a.NQ);
    const int bq = a.block_q;
    const int q0 = wk.i * bq;
    const int qw0 = q0 + wave * 32;
    const int q_last = min(q0 + bq, a.S) - 1;
    const int qrow = qw0 + l32;
    const bool qvalid = qrow < a.S && (wave * 32 + l32) < bq;

    const int head_bytes = a.S * G::ROWB;
    const int64_t qhead = ((int64_t)wk.b * a.Hq + wk.h) * a.S;
    const int64_t khead = ((int64_t)wk.b * a.Hkv + wk.g) * a.S;
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc((const uint16_t*)a.q + qhead * D, head_bytes);
    const __amdgpu_buffer_rsrc_t dors = make_rsrc((const uint16_t*)a.dout + qhead * D, head_bytes);
    const __amdgpu_buffer_rsrc_t krs = make_rsrc((const uint16_t*)a.k + khead * D, head_bytes);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc((const uint16_t*)a.v + khead * D, head_bytes);

    // B operands of S^T = K Q^T and dP^T = V dO^T: this lane's query row.
    bf16x8 qf[KSTEPS], dof[KSTEPS];
    {
        const int off = (wave * 32 + l32) < bq ? (qrow * D + 8 * hf) * 2 : head_bytes;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            qf[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qrs, off + 32 * ks, 0, 0));
            dof[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(dors, off + 32 * ks, 0, 0));
        }
    }
    const float lse_l2 = qvalid ? lse_offset(a.lse[qhead + qrow]) : kPosInf;
    const float delta = qvalid ? a.delta[qhead + qrow] : 0.f;

    int e_begin, e_end;
    q_tile_range_wave(a, wk.b, wk.h, wk.i, q_last, lane, e_begin, e_end);
    const int ntiles = e_end - e_begin;
    int col_base = e_begin, col_lane = 0;
    auto fetch_cols = [&](int base) {
        col_base = base;
        const int e = base + lane;
        col_lane = a.row_ptr ? (e < e_end ? a.col_idx[e] : 0) : e;
    };
    fetch_cols(e_begin);
    auto tile_of = [&](int n) -> int {
        const int e = e_begin + n;
        if (e - col_base >= 64) fetch_cols(e);
        return __builtin_amdgcn_readlane(col_lane, e - col_base);
    };

    // LDS: K stages 0/1 then V stages 0/1, one 64-key tile each.
    auto kst = [&](int st) -> char* { return lds + st * G::TILEB; };
    auto vst = [&](int st) -> char* { return lds + (2 + st) * G::TILEB; };

    f32x16 dq[DBLK];
#pragma unroll
    for (int m = 0; m < DBLK; ++m) dq[m] = (f32x16){};

    // Tile DMA through the instruction itself (the compiler does not track it,
    // so the transposed K reads of step n do not wait for the tiles of step
    // n + 1); every wait on it is explicit.
    // Per-lane source offsets inside a tile (independent of the tile); the
    // tile is selected by the base of the buffer resource, whose record count
    // ends at the last key, so rows of a ragged last tile past it read as
    // zeros (their keys are masked: P = 0, dS = 0).
    constexpr int IPW = (G::NINSTR + NW - 1) / NW;
    const uint16_t* kbase = (const uint16_t*)a.k + khead * D;
    const uint16_t* vbase = (const uint16_t*)a.v + khead * D;
    const uint32_t lds0 = lds_address(lds);
    int kvo[IPW], vvo[IPW];
#pragma unroll
    for (int x = 0; x < IPW; ++x) {
        const int ii = wave + NW * x;
        const int row = ii * G::RPI + lane / G::CH, pc = lane % G::CH;
        kvo[x] = row * G::ROWB + (pc ^ G::bswz(row)) * 16;
        vvo[x] = row * G::ROWB + (pc ^ G::rswz(row)) * 16;
    }
    auto dma = [&](const uint16_t* base, const int (&vo)[IPW], int st_off, int j) {
        const uint32_t off = (uint32_t)j * (64 * G::ROWB);
        const u32x4 rs = rsrc_words((const char*)base + off, (uint32_t)head_bytes - off);
#pragma unroll
        for (int x = 0; x < IPW; ++x) {
            const int ii = wave + NW * x;
            if (G::NINSTR % NW == 0 || ii < G::NINSTR) dma16(rs, lds0 + st_off + ii * 1024, vo[x]);
        }
    };
    auto dma_k = [&](int st, int j) { dma(kbase, kvo, st * G::TILEB, j); };
    auto dma_v = [&](int st, int j) { dma(vbase, vvo, (2 + st) * G::TILEB, j); };

    int j_cur = 0;
    // The Q / dO loads are the only loads the compiler tracks: settle them
    // before the first DMA on every path, so none of its waits counts tiles.
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    if (ntiles > 0) {
        j_cur = tile_of(0);
        dma_k(0, j_cur);
        dma_v(0, j_cur);
    }
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    bare_barrier();

    for (int n = 0; n < ntiles; ++n) {
        const int st = n & 1;
        const int j_next = (n + 1 < ntiles) ? tile_of(n + 1) : 0;
        if (n + 1 < ntiles) {  // stage st ^ 1 was last read in step n - 1
            dma_k(st ^ 1, j_next);
            dma_v(st ^ 1, j_next);
        }
        const char* kt = kst(st);
        const char* vt = vst(st);
        f32x16 s[2], dp[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            s[mb] = (f32x16){};
            dp[mb] = (f32x16){};
        }
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
                s[mb] = mfma(row_frag<D, true>(kt, 32 * mb + l32, 2 * ks + hf), qf[ks], s[mb]);
                dp[mb] = mfma(row_frag<D, false>(vt, 32 * mb + l32, 2 * ks + hf), dof[ks], dp[mb]);
            }
        // Lane holds query qrow and keys 32 mb + 8 (x / 4) + 4 hf + (x % 4) of the tile at [mb][x].
        // Partial tiles (causal diagonal, ragged tail) only: keys past the
        // lane's query row or past S get S = -inf, hence P = 0. Key offset of
        // element x is c(x) + 4 hf: compare the constant c(x) with lim - 4 hf.
        const int key0 = j_cur * 64;
        const bool need_mask = (a.causal && key0 + 63 > qw0) || (key0 + 64 > a.S);
        if (need_mask) {
            int lim = min(63, a.S - 1 - key0);
            if (a.causal) lim = min(lim, qrow - key0);
            const int limh = lim - 4 * hf;
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int x = 0; x < 16; ++x) {
                    const int c = 32 * mb + 8 * (x >> 2) + (x & 3);
                    s[mb][x] = c <= limh ? s[mb][x] : kNegInf;
                }
        }
        bf16x8 dsf[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int mb = kk >> 1, q4 = 8 * (kk & 1);
#pragma unroll
            for (int x = 0; x < 8; ++x) {
                const float p = fast_exp2(__builtin_fmaf(s[mb][q4 + x], a.scale_log2, -lse_l2));
                dsf[kk][x] = (__bf16)(p * (dp[mb][q4 + x] - delta));
            }
        }
        // dQ^T += K^T dS^T; contraction over keys 16 kk + 4 hf + (0..3), 16 kk + 8 + 4 hf + (0..3).
        bf16x8 tf[2][DBLK];
        auto load_t = [&](int kk, int buf) {
#pragma unroll
            for (int m = 0; m < DBLK; ++m) tf[buf][m] = tr_frag<D>(kt, 16 * kk, m, lane);
        };
        load_t(0, 0);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            if (kk + 1 < 4) load_t(kk + 1, (kk + 1) & 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int m = 0; m < DBLK; ++m) dq[m] = mfma(tf[kk & 1][m], dsf[kk], dq[m]);
            __builtin_amdgcn_sched_barrier(0);
        }
        j_cur = j_next;
        __builtin_amdgcn_s_waitcnt(kVmcnt0);  // tile n + 1 has landed
        bare_barrier();
    }

    if (qvalid) {
        uint16_t* op = (uint16_t*)a.dq + (qhead + qrow) * D;
#pragma unroll
        for (int m = 0; m < DBLK; ++m)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                bf16x4 w;
#pragma unroll
                for (int x = 0; x < 4; ++x) w[x] = (__bf16)(dq[m][4 * q + x] * a.scale);
                *(bf16x4*)(op + 32 * m + 8 * q + 4 * hf) = w;
            }
    }
}

// ============================================================ dK / dV (MFMA)
//
// Workgroup = 8 waves on one kv tile of 64 keys, two per SIMD. A unit is 64
// queries (a "chunk") of one query head of the group; each 32-key x 32-query
// block of it (key half kb, query half qs) belongs to a pair of waves:
//  - the P wave (waves 0..3) computes S = Q K^T and P = exp(S scale - LSE),
//    hands P to its partner through LDS and accumulates dV^T += dO^T P;
//  - the dS wave (waves 4..7) computes dP = dO V^T, takes P, forms
//    dS = P (dP - Delta) and accumulates dK^T += Q^T dS.
// Each wave thus runs half the products of its block, and the two waves of a
// pair sit on one SIMD (wave w and w + 4), so the vector work and the waits
// of one overlap the matrix products of the other. K (P waves) or V (dS
// waves) fragments stay in registers.
// Units are walked head by head over the group, each head's query tiles
// ascending, and streamed through four LDS stages (Q chunk, dO chunk, and per
// wave the LSE or Delta of its 32 queries, all by buffer-to-LDS DMA): units
// n + 1 .. n + 3 are in flight while unit n is computed, and every wave
// issues the same number of loads per unit, so a partial vmcnt wait tells
// unit n has landed. Two barriers per unit: the first ends every wave's reads
// of the stage refilled next, the second publishes P. At the end the two
// query halves of each key half add their partial dK^T / dV^T through LDS.
// Workgroups run kv-tile major (tile 0 of every kv head first): under causal,
// early tiles are seen by the most query tiles, and a pinned tile (a sink) by
// every one of them, so the longest work starts first.
struct Unit {
    int hh, e, e_end, c, nch, i;
};

template <int D>
struct DkdvLds {
    static constexpr int TILEB = 64 * D * 2;
    static constexpr int NST = 4;                    // stages: the unit in work, the next one, two in flight
    static constexpr int SIDE = 8 * 64 * 4;          // per stage: 8 waves x 64 floats (LSE or Delta)
    static constexpr int STAGEB = 2 * TILEB + SIDE;  // a stage: Q chunk, dO chunk, side values
    static constexpr int PX = 4 * 16 * 64 * 4;       // P of the four blocks, fp32, 16 per lane
    static constexpr int BYTES = NST * STAGEB + PX;
    static_assert(2 * 2 * 2 * (D / 32) * 16 * 64 * 4 <= BYTES, "reduction buffer fits");
};

template <int D>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_mfma_kernel(AttnBwdArgs a) {
    constexpr int KSTEPS = D / 16;
    constexpr int DBLK = D / 32;
    constexpr int NW = 8;
    using G = Geo<D>;
    using L = DkdvLds<D>;
    static_assert(G::NINSTR % NW == 0, "every wave issues the same number of DMA instructions");
    constexpr int IPW = G::NINSTR / NW;
    constexpr int PER_UNIT = 2 * IPW + 1;  // vector memory instructions per wave per unit
    extern __shared__ __attribute__((aligned(1024))) char lds[];
    const uint32_t lds0 = lds_address(lds);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool pwave = wave < 4;  // P wave (S, P, dV) or dS wave (dP, dS, dK)
    const int l32 = lane & 31, hf = lane >> 5;
    const int kb = wave & 1, qs = (wave >> 1) & 1;
    const int64_t BH = (int64_t)a.B * a.Hkv;
    const int j = (int)(blockIdx.x / BH);
    const int g = (int)(blockIdx.x % BH % a.Hkv);
    const int b = (int)(blockIdx.x % BH / a.Hkv);
    const int GRP = a.Hq / a.Hkv;
    const int key0 = j * 64;
    const int mykey = key0 + 32 * kb + l32;
    const int bq = a.block_q;

    const int head_bytes = a.S * G::ROWB;
    const int64_t khead = ((int64_t)b * a.Hkv + g) * a.S;
    // K fragments (P waves) or V fragments (dS waves) of this wave's 32 keys.
    bf16x8 kvf[KSTEPS];
    {
        const __amdgpu_buffer_rsrc_t rs =
            make_rsrc((const uint16_t*)(pwave ? a.k : a.v) + khead * D, head_bytes);
        const int off = (mykey * D + 8 * hf) * 2;  // past S: zeros
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks)
            kvf[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 32 * ks, 0, 0));
        // Settle these before any DMA: from here on every vmcnt wait is explicit.
        __builtin_amdgcn_s_waitcnt(kVmcnt0);
    }

    // Cursor over units (query head of the group, entry of its kv-tile list,
    // 64-query chunk); indices come from scalar loads.
    auto setup_entry = [&](Unit& u) {
        u.i = kv_entry(a, u.e);
        const int t0 = u.i * bq;
        const int rows = min(bq, a.S - t0);
        u.nch = (rows + 63) >> 6;
        // Under causal, chunk c can see key0 only if its last query t0 + 64 c + 63 >= key0.
        u.c = (a.causal && key0 > t0 + 63) ? (key0 - t0) / 64 : 0;
    };
    // Moves `u` to the first unit at or after its position; false when none is left.
    auto settle = [&](Unit& u) -> bool {
        for (;;) {
            if (u.e < u.e_end) {
                if (u.c < u.nch) return true;
                ++u.e;
                if (u.e < u.e_end) setup_entry(u);
                continue;
            }
            ++u.hh;
            if (u.hh >= GRP) return false;
            const int h = g * GRP + u.hh;
            const int hs = (a.Hsel == 1) ? 0 : h;
            kv_tile_range(a, b, hs, j, key0, u.e, u.e_end);
            if (u.e < u.e_end) setup_entry(u);
        }
    };
    auto advance = [&](Unit u, bool& ok) -> Unit {
        ++u.c;
        ok = settle(u);
        return u;
    };

    // Loads of unit u into stage st: Q and dO chunks and, for this wave's 32
    // queries, the raw LSE (P waves) or Delta (dS waves). Per-lane offsets
    // inside a chunk are the same for every unit (bswz layout); a chunk is
    // selected by the base of its buffer resource, whose record count ends at
    // query S - 1, so rows past it read as zeros (those queries are masked:
    // P = 0, dS = 0). Every lane of every wave takes part, so each wave
    // issues PER_UNIT loads.
    int tvo[IPW];
#pragma unroll
    for (int x = 0; x < IPW; ++x) {
        const int ii = wave + NW * x;
        const int row = ii * G::RPI + lane / G::CH, pc = lane % G::CH;
        tvo[x] = row * G::ROWB + (pc ^ G::bswz(row)) * 16;
    }
    // Query rows are counted from the first row of the group's first head.
    const int64_t grow0 = ((int64_t)b * a.Hq + g * GRP) * a.S;
    // Group base addresses; a unit's byte offsets from them fit in 32 bits
    // (the host keeps the group's rows below 2^32 bytes).
    const uint64_t qgrp = (uint64_t)a.q + (uint64_t)grow0 * G::ROWB;
    const uint64_t dgrp = (uint64_t)a.dout + (uint64_t)grow0 * G::ROWB;
    const uint64_t sgrp = (uint64_t)(pwave ? a.lse : a.delta) + (uint64_t)grow0 * 4;
    auto words = [](uint64_t base, uint32_t off, uint32_t bytes) -> u32x4 {
        const uint64_t p = base + off;
        return (u32x4){(uint32_t)p, (uint32_t)(p >> 32) & 0xFFFFu, bytes, 0x00020000u};
    };
    auto issue = [&](const Unit& u, int st) {
        const int row0 = u.i * bq + 64 * u.c;
        const uint32_t trow = (uint32_t)(u.hh * a.S + row0);
        const uint32_t tbytes = (uint32_t)(a.S - row0) * G::ROWB;
        const u32x4 rq = words(qgrp, trow * G::ROWB, tbytes);
        const u32x4 rd = words(dgrp, trow * G::ROWB, tbytes);
        const uint32_t lq = lds0 + st * L::STAGEB;
#pragma unroll
        for (int x = 0; x < IPW; ++x) dma16(rq, lq + (wave + NW * x) * 1024, tvo[x]);
#pragma unroll
        for (int x = 0; x < IPW; ++x) dma16(rd, lq + G::TILEB + (wave + NW * x) * 1024, tvo[x]);
        const int srow = 32 * qs;  // lanes 32..63 fetch values no one reads
        const uint32_t sbytes = (uint32_t)max(a.S - row0 - srow, 0) * 4;
        dma4(words(sgrp, (trow + srow) * 4u, sbytes), lq + 2 * G::TILEB + wave * 256, lane * 4);
    };

    f32x16 acc[DBLK];  // dV^T (P waves) or dK^T (dS waves), partial over this wave's queries
#pragma unroll
    for (int m = 0; m < DBLK; ++m) acc[m] = (f32x16){};

    // Per-lane LDS offsets within a stage, the same for every unit: row
    // fragments of this wave's queries (Q for P waves, dO for dS waves: chunk
    // 2 ks + hf of row qr), and the two halves of the transposed fragments
    // (dO for P waves, Q for dS waves: rows 32 qs + 4 hf + (0..3) and + 8,
    // column block m; the second k-step is 16 rows further on).
    const int qr = 32 * qs + l32;
    const int rbase = pwave ? 0 : G::TILEB;  // row-read tile
    const int tbase = pwave ? G::TILEB : 0;  // transposed-read tile
    int roff[KSTEPS], tlo[DBLK], thi[DBLK];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) roff[ks] = rbase + qr * G::ROWB + ((2 * ks + hf) ^ G::bswz(qr)) * 16;
    {
        const int vg = lane >> 4, vs = lane & 15;
        const int r0 = 32 * qs + 4 * hf + (vs >> 2), r1 = r0 + 8;
#pragma unroll
        for (int m = 0; m < DBLK; ++m) {
            const int d = 32 * m + 16 * (vg & 1) + 4 * (vs & 3);
            const int c = d >> 3, bo = (d & 7) * 2;
            tlo[m] = tbase + r0 * G::ROWB + (c ^ G::bswz(r0)) * 16 + bo;
            thi[m] = tbase + r1 * G::ROWB + (c ^ G::bswz(r1)) * 16 + bo;
        }
    }
    const int soff = 2 * G::TILEB + wave * 256 + 16 * hf;  // this wave's LSE or Delta
    // P of this wave's block (written by the P wave, read by the dS wave of
    // the pair): element x of lane l at float (x / 4) * 256 + 4 l + x % 4.
    float* px = (float*)(lds + L::NST * L::STAGEB) + (wave & 3) * 1024 + 4 * lane;
    auto rowf = [&](const char* p, int ks) -> bf16x8 {
        return __builtin_bit_cast(bf16x8, *(const u32x4*)(p + roff[ks]));
    };
    auto trf = [&](const char* p, int m, int s3) -> bf16x8 {
        const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p + tlo[m] + s3 * 16 * G::ROWB));
        const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p + thi[m] + s3 * 16 * G::ROWB));
        const short8_t w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        return __builtin_bit_cast(bf16x8, w);
    };
    // Software pipeline over units, one unit deep: an iteration finishes unit
    // `cur` while it computes S (P waves) or dP (dS waves) of the next unit.
    // Unit cur sits in stage st, the next units nx[0], nx[1], ... in the
    // following stages (valid while hv[]). When an iteration starts, cur and
    // nx[0] are resident and nx[1] is in flight; it issues one more unit into
    // the stage of the unit before cur.
    constexpr int NST = L::NST;
    static_assert(NST == 4, "the waits below assume four stages");
    Unit cur;
    cur.hh = -1;
    cur.e = cur.e_end = 0;
    cur.c = cur.nch = 0;
    cur.i = 0;
    bool have = settle(cur);
    Unit nx[NST - 1];
    bool hv[NST - 1];
#pragma unroll
    for (int x = 0; x < NST - 1; ++x) {
        nx[x] = cur;
        hv[x] = false;
    }
    if (have) {
        issue(cur, 0);
        bool ok = true;
        Unit prev = cur;
#pragma unroll
        for (int x = 0; x < NST - 2; ++x) {
            if (ok) {
                prev = advance(prev, ok);
                if (ok) {
                    nx[x] = prev;
                    hv[x] = true;
                    issue(prev, x + 1);
                }
            }
        }
    }
    // S (or dP) of the first unit (stage 0), for this wave's 32 queries x 32 keys.
    f32x16 sc = (f32x16){};
    if (have) {
        // unit cur has landed once at most the units issued after it are outstanding
        if (hv[1]) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * PER_UNIT));
        else if (hv[0]) __builtin_amdgcn_s_waitcnt(vmcnt_imm(PER_UNIT));
        else __builtin_amdgcn_s_waitcnt(kVmcnt0);
        bare_barrier();
        bf16x8 ra[KSTEPS];
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) ra[ks] = rowf(lds, ks);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) sc = mfma(ra[ks], kvf[ks], sc);
    }
    int st = 0;
    while (have) {
        // Unit nx[0] (if any) has landed once at most the unit issued after it
        // is outstanding; the barrier also ends every wave's reads of the stage
        // of the unit before cur.
        if (hv[1]) __builtin_amdgcn_s_waitcnt(vmcnt_imm(PER_UNIT));
        else __builtin_amdgcn_s_waitcnt(kVmcnt0);
        bare_barrier();
        // The walk to the unit after nx[1] and its loads (into the stage of
        // the unit before cur, free since the barrier), placed after this
        // wave's products are issued so that its scalar work runs beside them.
        auto next_unit = [&]() {
            if (hv[1]) {
                bool ok = false;
                const Unit u = advance(nx[1], ok);
                if (ok) {
                    nx[2] = u;
                    hv[2] = true;
                    issue(u, (st + 3) & 3);
                }
            }
        };
        const int st1 = (st + 1) & 3;
        const char* sp = lds + st * L::STAGEB;
        const char* sp1 = lds + st1 * L::STAGEB;
        // Side values of unit cur, then the row fragments of the next unit
        // (stale but harmless when there is none: its products are then discarded).
        f32x4 side[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) side[q] = *(const f32x4*)(sp + soff + 32 * q);
        bf16x8 ra[KSTEPS];
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) ra[ks] = rowf(sp1, ks);
        f32x16 sn = (f32x16){};
        bf16x8 opf[2];  // bf16 operand of this wave's product: P or dS
        if (pwave) {
            // Lane holds key mykey (column) and queries 32 qs + 8 q + 4 hf + e
            // (chunk rows) at [4 q + e]. Element masks only where this block is
            // partial: under causal when a key may follow a query, and past the
            // tile end or S. A query with LSE = -inf sees no key at all, so
            // under causal every pair of its row here is masked, and without
            // causal it cannot occur in a kept tile.
            const int tq0 = cur.i * bq + 64 * cur.c + 32 * qs;
            const int t_lim = min(a.S, cur.i * bq + bq);  // queries of this unit are below t_lim
            const bool need_mask = (a.causal && key0 + 32 * kb + 31 > tq0) || (tq0 + 31 >= t_lim);
            const int key_lim = a.causal ? mykey : -1;
            auto step = [&](auto masked) {
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    f32x4 pq;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int x = 4 * q + e;
                        float p = fast_exp2(__builtin_fmaf(sc[x], a.scale_log2, -kLog2e * side[q][e]));
                        if (decltype(masked)::value) {
                            const int t = tq0 + 8 * q + 4 * hf + e;
                            p = (t < t_lim && key_lim <= t) ? p : 0.f;
                        }
                        pq[e] = p;
                        opf[x >> 3][x & 7] = (__bf16)p;
                    }
                    *(f32x4*)(px + 256 * q) = pq;
                }
#pragma unroll
                for (int ks = 0; ks < KSTEPS; ++ks) sn = mfma(ra[ks], kvf[ks], sn);
                // One product, then a share of the vector work, eight times over.
#pragma unroll
                for (int x = 0; x < KSTEPS; ++x) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, decltype(masked)::value ? 9 : 6, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            };
            // Two copies, so that full blocks (the common case) carry no mask arithmetic.
            if (need_mask) step(std::true_type{});
            else step(std::false_type{});
            next_unit();
            bare_barrier();  // P of this unit is in LDS for the dS waves
        } else {
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) sn = mfma(ra[ks], kvf[ks], sn);
            next_unit();
            bare_barrier();  // P of this unit is in LDS
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 pq = *(const f32x4*)(px + 256 * q);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int x = 4 * q + e;
                    opf[x >> 3][x & 7] = (__bf16)(pq[e] * (sc[x] - side[q][e]));
                }
            }
        }
        // dV^T += dO^T P (P waves) or dK^T += Q^T dS (dS waves); contraction
        // over this wave's queries, k-step s3 covering rows 32 qs + 16 s3 +
        // 4 hf + (0..3) and + 8.
#pragma unroll
        for (int s3 = 0; s3 < 2; ++s3) {
            bf16x8 ta[DBLK];  // read ahead of the products
#pragma unroll
            for (int m = 0; m < DBLK; ++m) ta[m] = trf(sp, m, s3);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int m = 0; m < DBLK; ++m) acc[m] = mfma(ta[m], opf[s3], acc[m]);
        }
        sc = sn;
        cur = nx[0];
        have = hv[0];
#pragma unroll
        for (int x = 0; x < NST - 2; ++x) {
            nx[x] = nx[x + 1];
            hv[x] = hv[x + 1];
        }
        hv[NST - 2] = false;
        st = st1;
    }
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    __syncthreads();  // every wave is done with the stages (nothing is in flight any more)

    // Add the query-half partials: waves with qs = 1 park theirs in LDS.
    float* red = (float*)lds;  // [pwave][kb][DBLK][16][64] floats
    const int rw = (pwave ? 0 : 2) + kb;
    if (qs == 1) {
#pragma unroll
        for (int m = 0; m < DBLK; ++m)
#pragma unroll
            for (int x = 0; x < 16; ++x) red[((rw * DBLK + m) * 16 + x) * 64 + lane] = acc[m][x];
    }
    __syncthreads();
    if (qs == 0 && mykey < a.S) {
        uint16_t* op = (uint16_t*)(pwave ? a.dv : a.dk) + (khead + mykey) * D;
        const float sc_out = pwave ? 1.0f : a.scale;
#pragma unroll
        for (int m = 0; m < DBLK; ++m)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                bf16x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int x = 4 * q + e;
                    w[e] = (__bf16)((acc[m][x] + red[((rw * DBLK + m) * 16 + x) * 64 + lane]) * sc_out);
                }
                // rows d = 32 m + 8 q + 4 hf + e of column mykey
                *(bf16x4*)(op + 32 * m + 8 * q + 4 * hf) = w;
            }
    }
}

// ============================================================ SIMT fallback
//
// Four lanes per row, each holding a quarter of D in fp32.

template <int D, bool BF16>
__global__ __launch_bounds__(256) void bwd_dq_simt_kernel(AttnBwdArgs a) {
    constexpr int QD = D / 4;
    constexpr int KC = 32;
    __shared__ float Ks[KC][D + 4];
    __shared__ float Vs[KC][D + 4];
    const int tid = threadIdx.x;
    const int64_t total = (int64_t)a.B * a.Hq * a.NQ;
    const Work wk = decode_q_work(blockIdx.x, total, a.Hq, a.Hkv, a.NQ);
    const int t0 = wk.i * a.block_q;
    const int t_end = min(t0 + a.block_q, a.S);
    const int64_t qhead = ((int64_t)wk.b * a.Hq + wk.h) * a.S;
    const int64_t khead = ((int64_t)wk.b * a.Hkv + wk.g) * a.S;
    const int part = tid & 3;

    for (int rc = t0; rc < t_end; rc += 64) {
        const int row = rc + (tid >> 2);
        const bool rvalid = row < t_end;
        const int chunk_last = min(rc + 64, t_end) - 1;
        float qv[QD], dov[QD], dqv[QD];
#pragma unroll
        for (int d = 0; d < QD; ++d) {
            const int64_t x = (qhead + row) * D + part * QD + d;
            qv[d] = rvalid ? load_elem(a.q, x, BF16) : 0.f;
            dov[d] = rvalid ? load_elem(a.dout, x, BF16) : 0.f;
            dqv[d] = 0.f;
        }
        const float lse_l2 = rvalid ? lse_offset(a.lse[qhead + row]) : kPosInf;
        const float delta = rvalid ? a.delta[qhead + row] : 0.f;
        int e_begin, e_end;
        q_tile_range(a, wk.b, wk.h, wk.i, chunk_last, e_begin, e_end);
        for (int e = e_begin; e < e_end; ++e) {
            const int jt = a.row_ptr ? a.col_idx[e] : e;
            const int k0 = jt * a.block_kv;
            const int k1 = min(k0 + a.block_kv, a.S);
            for (int kc = k0; kc < k1; kc += KC) {
                if (a.causal && kc > chunk_last) break;
                const int nkeys = min(KC, k1 - kc);
                __syncthreads();
                for (int x = tid; x < KC * D; x += 256) {
                    const int kr = x / D, d = x % D;
                    const bool ok = kr < nkeys;
                    Ks[kr][d] = ok ? load_elem(a.k, (khead + kc + kr) * D + d, BF16) : 0.f;
                    Vs[kr][d] = ok ? load_elem(a.v, (khead + kc + kr) * D + d, BF16) : 0.f;
                }
                __syncthreads();
                for (int kr = 0; kr < nkeys; ++kr) {
                    float sd = 0.f, pd = 0.f;
#pragma unroll
                    for (int d = 0; d < QD; ++d) {
                        sd += qv[d] * Ks[kr][part * QD + d];
                        pd += dov[d] * Vs[kr][part * QD + d];
                    }
                    sd += __shfl_xor(sd, 1);
                    sd += __shfl_xor(sd, 2);
                    pd += __shfl_xor(pd, 1);
                    pd += __shfl_xor(pd, 2);
                    const int key = kc + kr;
                    float p = exp2f(sd * a.scale_log2 - lse_l2);
                    if (a.causal && key > row) p = 0.f;
                    const float ds = p * (pd - delta);
#pragma unroll
                    for (int d = 0; d < QD; ++d) dqv[d] += ds * Ks[kr][part * QD + d];
                }
            }
        }
        if (rvalid) {
            const int64_t o = (qhead + row) * D + part * QD;
#pragma unroll
            for (int d = 0; d < QD; ++d) {
                if constexpr (BF16) ((uint16_t*)a.dq)[o + d] = to_bf16_bits(dqv[d] * a.scale);
                else ((float*)a.dq)[o + d] = dqv[d] * a.scale;
            }
        }
    }
}

template <int D, bool BF16>
__global__ __launch_bounds__(256) void bwd_dkdv_simt_kernel(AttnBwdArgs a) {
    constexpr int QD = D / 4;
    constexpr int QC = 32;
    __shared__ float Qs[QC][D + 4];
    __shared__ float Ds[QC][D + 4];
    __shared__ float Ls[QC], Dl[QC];
    const int tid = threadIdx.x;
    const int j = (int)(blockIdx.x % a.NK);
    const int g = (int)((blockIdx.x / a.NK) % a.Hkv);
    const int b = (int)(blockIdx.x / ((int64_t)a.NK * a.Hkv));
    const int GRP = a.Hq / a.Hkv;
    const int k0 = j * a.block_kv;
    const int k_end = min(k0 + a.block_kv, a.S);
    const int64_t khead = ((int64_t)b * a.Hkv + g) * a.S;
    const int part = tid & 3;

    for (int kc0 = k0; kc0 < k_end; kc0 += 64) {
        const int key = kc0 + (tid >> 2);
        const bool kvalid = key < k_end;
        float kv_[QD], vv[QD], dkv[QD], dvv[QD];
#pragma unroll
        for (int d = 0; d < QD; ++d) {
            const int64_t x = (khead + key) * D + part * QD + d;
            kv_[d] = kvalid ? load_elem(a.k, x, BF16) : 0.f;
            vv[d] = kvalid ? load_elem(a.v, x, BF16) : 0.f;
            dkv[d] = 0.f;
            dvv[d] = 0.f;
        }
        for (int hh = 0; hh < GRP; ++hh) {
            const int h = g * GRP + hh;
            const int hs = (a.Hsel == 1) ? 0 : h;
            const int64_t qhead = ((int64_t)b * a.Hq + h) * a.S;
            int e_begin, e_end;
            kv_tile_range(a, b, hs, j, kc0, e_begin, e_end);
            for (int e = e_begin; e < e_end; ++e) {
                const int i = kv_entry(a, e);
                const int t0 = i * a.block_q;
                const int t1 = min(t0 + a.block_q, a.S);
                for (int tc = t0; tc < t1; tc += QC) {
                    if (a.causal && tc + QC - 1 < kc0) continue;
                    const int nq = min(QC, t1 - tc);
                    __syncthreads();
                    for (int x = tid; x < QC * D; x += 256) {
                        const int r = x / D, d = x % D;
                        const bool ok = r < nq;
                        Qs[r][d] = ok ? load_elem(a.q, (qhead + tc + r) * D + d, BF16) : 0.f;
                        Ds[r][d] = ok ? load_elem(a.dout, (qhead + tc + r) * D + d, BF16) : 0.f;
                    }
                    if (tid < QC) {
                        const bool ok = tid < nq;
                        Ls[tid] = ok ? lse_offset(a.lse[qhead + tc + tid]) : kPosInf;
                        Dl[tid] = ok ? a.delta[qhead + tc + tid] : 0.f;
                    }
                    __syncthreads();
                    for (int r = 0; r < nq; ++r) {
                        float sd = 0.f, pd = 0.f;
#pragma unroll
                        for (int d = 0; d < QD; ++d) {
                            sd += Qs[r][part * QD + d] * kv_[d];
                            pd += Ds[r][part * QD + d] * vv[d];
                        }
                        sd += __shfl_xor(sd, 1);
                        sd += __shfl_xor(sd, 2);
                        pd += __shfl_xor(pd, 1);
                        pd += __shfl_xor(pd, 2);
                        float p = exp2f(sd * a.scale_log2 - Ls[r]);
                        if (a.causal && key > tc + r) p = 0.f;
                        const float ds = p * (pd - Dl[r]);
#pragma unroll
                        for (int d = 0; d < QD; ++d) {
                            dvv[d] += p * Ds[r][part * QD + d];
                            dkv[d] += ds * Qs[r][part * QD + d];
                        }
                    }
                }
            }
        }
        if (kvalid) {
            const int64_t o = (khead + key) * D + part * QD;
#pragma unroll
            for (int d = 0; d < QD; ++d) {
                if constexpr (BF16) {
                    ((uint16_t*)a.dk)[o + d] = to_bf16_bits(dkv[d] * a.scale);
                    ((uint16_t*)a.dv)[o + d] = to_bf16_bits(dvv[d]);
                } else {
                    ((float*)a.dk)[o + d] = dkv[d] * a.scale;
                    ((float*)a.dv)[o + d] = dvv[d];
                }
            }
        }
    }
}

}  // namespace

// ============================================================ launchers

hipError_t launch_bwd_delta(const void* out, const void* dout, int bf16, int64_t rows, int D, float* delta,
                            hipStream_t stream) {
    if (rows == 0) return hipSuccess;
    const int64_t threads = rows * (D / 8);
    const dim3 grid((unsigned)((threads + 255) / 256));
#define NSA_DELTA(DD, BB) hipLaunchKernelGGL((delta_kernel<DD, BB>), grid, dim3(256), 0, stream, out, dout, delta, rows)
    if (D == 128) {
        if (bf16) NSA_DELTA(128, true);
        else NSA_DELTA(128, false);
    } else if (D == 64) {
        if (bf16) NSA_DELTA(64, true);
        else NSA_DELTA(64, false);
    } else {
        return hipErrorInvalidValue;
    }
#undef NSA_DELTA
    return hipGetLastError();
}

hipError_t launch_kv_major_index(const int8_t* keep, int BH, int NQ, int NK, int32_t cap, int32_t* counts4,
                                 int32_t* col_ptr, int32_t* sums, int32_t* row_idx, hipStream_t stream) {
    const int64_t n = (int64_t)BH * NK;
    const int nb = (int)((n + 2047) / 2048);
    if (n > 0) {
        const dim3 grid((unsigned)((int64_t)BH * ((NK + 63) / 64)));
        hipLaunchKernelGGL(colcount_kernel, grid, dim3(256), 0, stream, keep, NQ, NK, counts4);
        hipLaunchKernelGGL(colscan_block_kernel, dim3((unsigned)nb), dim3(256), 0, stream, counts4, n, col_ptr,
                           sums);
    }
    hipLaunchKernelGGL(colscan_sums_kernel, dim3(1), dim3(256), 0, stream, sums, nb);
    hipLaunchKernelGGL(colscan_add_kernel, dim3((unsigned)((n + 1 + 255) / 256)), dim3(256), 0, stream, col_ptr,
                       sums, n, nb, cap);
    if (n > 0) {
        const dim3 grid((unsigned)((int64_t)BH * ((NK + 63) / 64)));
        hipLaunchKernelGGL(colfill_kernel, grid, dim3(256), 0, stream, keep, NQ, NK, counts4, col_ptr, row_idx);
    }
    return hipGetLastError();
}

bool attn_bwd_mfma_supported(const AttnBwdArgs& a, int bf16) {
    const bool fits = ((int64_t)a.S + 128) * a.D * 2 < ((int64_t)1 << 31);
    // dK / dV address a unit by its 32-bit byte offset from its GQA group's first row
    const bool group_fits = (int64_t)(a.Hq / a.Hkv) * ((int64_t)a.S + 128) * a.D * 2 < ((int64_t)1 << 32);
    return bf16 && fits && group_fits && a.block_kv == 64 && a.block_q % 32 == 0 && a.block_q >= 32 && a.block_q <= 128 &&
           (a.D == 64 || a.D == 128);
}

size_t attn_bwd_dkdv_lds_bytes(int D) { return D == 128 ? DkdvLds<128>::BYTES : DkdvLds<64>::BYTES; }

hipError_t launch_attn_bwd_mfma(const AttnBwdArgs& a, hipStream_t stream) {
    const int64_t qwork = (int64_t)a.B * a.Hq * a.NQ;
    const int64_t kvwork = (int64_t)a.B * a.Hkv * a.NK;
    const int nw = a.block_q / 32;
    if (qwork > 0) {
#define NSA_DQ(DD, NWW)                                                                                 \
    hipLaunchKernelGGL((bwd_dq_mfma_kernel<DD, NWW>), dim3((unsigned)qwork), dim3(64 * NWW), \
                       (size_t)(4 * 64 * DD * 2), stream, a)
        if (a.D == 128) {
            if (nw == 4) NSA_DQ(128, 4);
            else if (nw == 3) NSA_DQ(128, 3);
            else if (nw == 2) NSA_DQ(128, 2);
            else NSA_DQ(128, 1);
        } else {
            if (nw == 4) NSA_DQ(64, 4);
            else if (nw == 3) NSA_DQ(64, 3);
            else if (nw == 2) NSA_DQ(64, 2);
            else NSA_DQ(64, 1);
        }
#undef NSA_DQ
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    hipError_t e = stage_mark("dq", stream);
    if (e != hipSuccess) return e;
    if (kvwork > 0) {
        if (a.D == 128)
            hipLaunchKernelGGL((bwd_dkdv_mfma_kernel<128>), dim3((unsigned)kvwork), dim3(512),
                               attn_bwd_dkdv_lds_bytes(128), stream, a);
        else
            hipLaunchKernelGGL((bwd_dkdv_mfma_kernel<64>), dim3((unsigned)kvwork), dim3(512),
                               attn_bwd_dkdv_lds_bytes(64), stream, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return stage_mark("dkdv", stream);
}

hipError_t launch_attn_bwd_simt(const AttnBwdArgs& a, int bf16, hipStream_t stream) {
    const int64_t qwork = (int64_t)a.B * a.Hq * a.NQ;
    const int64_t kvwork = (int64_t)a.B * a.Hkv * a.NK;
#define NSA_BSIMT(DD, BB)                                                                                    \
    do {                                                                                                     \
        if (qwork > 0)                                                                                       \
            hipLaunchKernelGGL((bwd_dq_simt_kernel<DD, BB>), dim3((unsigned)qwork), dim3(256), 0, stream, a); \
        if (kvwork > 0)                                                                                      \
            hipLaunchKernelGGL((bwd_dkdv_simt_kernel<DD, BB>), dim3((unsigned)kvwork), dim3(256), 0, stream, \
                               a);                                                                           \
    } while (0)
    if (a.D == 64) {
        if (bf16) NSA_BSIMT(64, true);
        else NSA_BSIMT(64, false);
    } else if (a.D == 128) {
        if (bf16) NSA_BSIMT(128, true);
        else NSA_BSIMT(128, false);
    } else {
        return hipErrorInvalidValue;
    }
#undef NSA_BSIMT
    return hipGetLastError();
}

}  // namespace nsa
