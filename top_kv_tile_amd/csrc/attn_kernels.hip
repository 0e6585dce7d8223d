// Block-sparse attention forward for gfx950 (CDNA4).
//
// Semantics: softmax attention of every query over the keys of the kv tiles
// its query tile keeps (the keep flags / CSR produced by the selection, whose
// definition is the page "automatic/modules/attention/sparse/selector.py",
// BlockSelection), with GQA, an optional causal mask and scale D^-1/2; the
// output is O and the natural-log logsumexp. Tiles entirely in the causal
// future are skipped, and element masks are applied only on tiles that are
// partly masked (the full-tile / partial-tile distinction the thread "Optimal
// ordering with block mask" describes for block masks). Rows whose running
// maximum is still -inf are guarded so they never produce NaN (the NaN reports
// of the "todo" list on native-sparse-attention-pytorch issue #1).
//
// Two kernels:
//  * attn_mfma_kernel: bf16 inputs, 64-key tiles, D in {64, 128}. One
//    workgroup per (batch, query head, query tile), one wavefront per 32 query
//    rows. S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_32x32x16_bf16, so each
//    lane owns one query row of both accumulators and the softmax needs a
//    single cross-lane exchange. K/V tiles are double-buffered in LDS; V is
//    transposed on its way into LDS.
//  * attn_simt_kernel: any dtype / block size (fp32 path), plain fp32 FMA.
#include "nsa_internal.h"

#include <float.h>
#include <math.h>

namespace nsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;  // NaN stays NaN
    u += 0x7fffu + ((u >> 16) & 1u);                                 // round to nearest even
    return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Work item of a workgroup. Workgroups are dispatched round-robin over the 8
// XCDs (block n runs on XCD n % 8); inside each run of 64 consecutive blocks,
// XCD x receives the 8 consecutive work items 8x .. 8x+7 of that run, so the
// query heads of one GQA group (which share the diagonal and pinned tiles) hit
// the same L2. Work items are ordered kv-head major, then query tile
// descending (longest causal rows first), then query head within the group:
// the whole chip works on one kv head at a time and its K/V stays in the
// shared last-level cache.
struct Work {
    int b, h, g, i;
};
__device__ __forceinline__ Work decode_work(int64_t n, int64_t total, int Hq, int Hkv, int NQ) {
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

// Range [start, end) of CSR entries to visit for query rows up to q_last
// (inclusive). Column lists are ascending, so under causal the visited prefix
// ends at the first tile that starts after q_last.
__device__ __forceinline__ void tile_range(const AttnArgs& a, int b, int h, int i, int q_last, int& start,
                                           int& end) {
    if (a.row_ptr) {
        const int hs = (a.Hsel == 1) ? 0 : h;
        const int64_t r = ((int64_t)b * a.Hsel + hs) * a.NQ + i;
        start = a.row_ptr[r];
        end = a.row_ptr[r + 1];
        if (a.causal) {
            int lo = start, hi = end;  // first entry with col * bkv > q_last
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

// ============================================================ MFMA kernel
//
// LDS layout per buffer (bf16):
//   Ks [64][D + 8]   key-major, row pitch padded by 16 bytes
//   Vt [D][64 + 8]   d-major; inside each group of 16 keys the two middle
//                    quads are swapped (key quads 0,2,1,3), so the 8 keys one
//                    lane feeds to an MFMA k-slot are 16 contiguous bytes.
template <int D>
struct MfmaLds {
    static constexpr int KP = D + 8;        // Ks row pitch (elements)
    static constexpr int VP = 64 + 8;       // Vt row pitch (elements)
    static constexpr int KS = 64 * KP;      // Ks elements
    static constexpr int VS = D * VP;       // Vt elements
    static constexpr int BUF = KS + VS;     // one stage
    static constexpr int BYTES = 2 * BUF * 2;
};

__device__ __forceinline__ int vt_pos(int key) {  // key 0..63 -> position in a Vt row
    const int quad = (key >> 2) & 3;
    const int pq = ((quad & 1) << 1) | (quad >> 1);  // 0,1,2,3 -> 0,2,1,3
    return (key & ~15) | (pq << 2) | (key & 3);
}

template <int D, int NW>
__global__ __launch_bounds__(64 * NW, 2) void attn_mfma_kernel(AttnArgs a) {
    constexpr int NT = 64 * NW;
    constexpr int BKV = 64;
    constexpr int KSTEPS = D / 16;      // QK^T contraction steps of 16
    constexpr int DBLK = D / 32;        // O^T row blocks of 32
    constexpr int KCH = D / 8;          // 16-byte chunks per K row
    constexpr int KLOADS = BKV * KCH / NT;
    constexpr int VUNITS = 16 * (D / 8);  // (key quad, d chunk) units
    constexpr int VLOADS = (VUNITS + NT - 1) / NT;
    static_assert(KLOADS * NT == BKV * KCH, "K tile must split evenly");
    using L = MfmaLds<D>;
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hf = lane >> 5;
    const int64_t total = (int64_t)a.B * a.Hq * a.NQ;
    const Work wk = decode_work(blockIdx.x, total, a.Hq, a.Hkv, a.NQ);
    const int bq = a.block_q;
    const int q0 = wk.i * bq;
    const int qw0 = q0 + wave * 32;                  // first query row of this wave
    const int q_last = min(q0 + bq, a.S) - 1;        // last real query row of the tile
    const int qrow = qw0 + l32;                      // this lane's query row
    const bool qvalid = qrow < a.S && (wave * 32 + l32) < bq;

    const uint16_t* qp = (const uint16_t*)a.q + (((int64_t)wk.b * a.Hq + wk.h) * a.S) * D;
    const uint16_t* kp = (const uint16_t*)a.k + (((int64_t)wk.b * a.Hkv + wk.g) * a.S) * D;
    const uint16_t* vp = (const uint16_t*)a.v + (((int64_t)wk.b * a.Hkv + wk.g) * a.S) * D;

    // Q^T operand: lane holds q[qrow][16*ks + 8*hf .. +8] for every ks.
    bf16x8 qf[KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
        u32x4 w = {0u, 0u, 0u, 0u};
        if (qvalid) w = *(const u32x4*)(qp + (int64_t)qrow * D + 16 * ks + 8 * hf);
        qf[ks] = __builtin_bit_cast(bf16x8, w);
    }

    int e_begin, e_end;
    tile_range(a, wk.b, wk.h, wk.i, q_last, e_begin, e_end);

    f32x16 oacc[DBLK];
#pragma unroll
    for (int m = 0; m < DBLK; ++m) oacc[m] = (f32x16){};
    float m_run = kNegInf;  // running max (log2 domain) of this lane's query row
    float l_run = 0.f;      // partial sum over this lane's half of every tile

    u32x4 kreg[KLOADS];
    u32x4 vreg[VLOADS][4];

    auto tile_of = [&](int e) -> int { return a.row_ptr ? a.col_idx[e] : e; };
    auto load_tile = [&](int j) {
        const int key0 = j * BKV;
#pragma unroll
        for (int x = 0; x < KLOADS; ++x) {
            const int c = tid + NT * x;
            const int row = c / KCH, ch = c % KCH;
            u32x4 w = {0u, 0u, 0u, 0u};
            if (key0 + row < a.S) w = *(const u32x4*)(kp + (int64_t)(key0 + row) * D + ch * 8);
            kreg[x] = w;
        }
#pragma unroll
        for (int x = 0; x < VLOADS; ++x) {
            const int u = tid + NT * x;
            const int kq = u & 15, dc = u >> 4;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = key0 + 4 * kq + r;
                u32x4 w = {0u, 0u, 0u, 0u};
                if (key < a.S && u < VUNITS) w = *(const u32x4*)(vp + (int64_t)key * D + dc * 8);
                vreg[x][r] = w;
            }
        }
    };
    auto store_tile = [&](int buf) {
        uint16_t* ks = lds + buf * L::BUF;
        uint16_t* vt = ks + L::KS;
#pragma unroll
        for (int x = 0; x < KLOADS; ++x) {
            const int c = tid + NT * x;
            const int row = c / KCH, ch = c % KCH;
            *(u32x4*)(ks + row * L::KP + ch * 8) = kreg[x];
        }
#pragma unroll
        for (int x = 0; x < VLOADS; ++x) {
            const int u = tid + NT * x;
            if (VUNITS % NT != 0 && u >= VUNITS) break;
            const int kq = u & 15, dc = u >> 4;
            const int pos = vt_pos(4 * kq);
#pragma unroll
            for (int e = 0; e < 4; ++e) {  // dword e holds d = 8*dc + 2e (low) and 2e+1 (high)
                const uint32_t k0 = vreg[x][0][e], k1 = vreg[x][1][e], k2 = vreg[x][2][e], k3 = vreg[x][3][e];
                u32x2 lo, hi;
                lo[0] = (k0 & 0xffffu) | (k1 << 16);
                lo[1] = (k2 & 0xffffu) | (k3 << 16);
                hi[0] = (k0 >> 16) | (k1 & 0xffff0000u);
                hi[1] = (k2 >> 16) | (k3 & 0xffff0000u);
                *(u32x2*)(vt + (8 * dc + 2 * e) * L::VP + pos) = lo;
                *(u32x2*)(vt + (8 * dc + 2 * e + 1) * L::VP + pos) = hi;
            }
        }
    };

    if (e_begin < e_end) {
        load_tile(tile_of(e_begin));
        store_tile(0);
    }
    __syncthreads();

    for (int e = e_begin; e < e_end; ++e) {
        const int cur = (e - e_begin) & 1;
        const int j = tile_of(e);
        const bool has_next = e + 1 < e_end;
        if (has_next) load_tile(tile_of(e + 1));

        const int key0 = j * BKV;
        // Whole tile masked for this wave: every key is after every query row.
        const bool wave_dead = a.causal && key0 > qw0 + 31;
        if (!wave_dead) {
            const uint16_t* ks = lds + cur * L::BUF;
            const uint16_t* vt = ks + L::KS;
            // S^T = K Q^T : two 32-key blocks.
            f32x16 sacc[2] = {(f32x16){}, (f32x16){}};
#pragma unroll
            for (int ks_ = 0; ks_ < KSTEPS; ++ks_) {
#pragma unroll
                for (int mb = 0; mb < 2; ++mb) {
                    const bf16x8 kf = __builtin_bit_cast(
                        bf16x8, *(const u32x4*)(ks + (32 * mb + l32) * L::KP + 16 * ks_ + 8 * hf));
                    sacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks_], sacc[mb], 0, 0, 0);
                }
            }
            // Lane holds query qrow and keys key0 + 32*mb + 8*q + 4*hf + e at sacc[mb][4q + e].
            const bool need_mask = (a.causal && key0 + BKV - 1 > qw0) || (key0 + BKV > a.S);
            float mx = kNegInf;
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int x = 0; x < 16; ++x) {
                    float sv = sacc[mb][x] * a.scale_log2;
                    if (need_mask) {
                        const int key = key0 + 32 * mb + 8 * (x >> 2) + 4 * hf + (x & 3);
                        if (key >= a.S || (a.causal && key > qrow)) sv = kNegInf;
                    }
                    sacc[mb][x] = sv;
                    mx = fmaxf(mx, sv);
                }
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m_run, mx);
            const float m_use = (m_new == kNegInf) ? 0.f : m_new;  // no visible key yet: keep zeros
            const float alpha = fast_exp2(m_run - m_use);
            m_run = m_new;
            float psum = 0.f;
            bf16x8 pf[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int mb = kk >> 1, q4 = 8 * (kk & 1);
                float p[8];
#pragma unroll
                for (int x = 0; x < 8; ++x) {
                    p[x] = fast_exp2(sacc[mb][q4 + x] - m_use);
                    psum += p[x];
                }
                u32x4 w;
#pragma unroll
                for (int x = 0; x < 4; ++x) w[x] = pack_bf16x2(p[2 * x], p[2 * x + 1]);
                pf[kk] = __builtin_bit_cast(bf16x8, w);
            }
            l_run = l_run * alpha + psum;
#pragma unroll
            for (int m = 0; m < DBLK; ++m) oacc[m] *= alpha;
            // O^T += V^T P^T
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
                for (int m = 0; m < DBLK; ++m) {
                    const bf16x8 vf = __builtin_bit_cast(
                        bf16x8, *(const u32x4*)(vt + (32 * m + l32) * L::VP + 16 * kk + 8 * hf));
                    oacc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[kk], oacc[m], 0, 0, 0);
                }
            }
        }
        if (has_next) store_tile(cur ^ 1);
        __syncthreads();
    }

    // Finish: combine the two lane halves of the row sum.
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const bool empty = !(l_tot > 0.f);
    const float inv = empty ? 0.f : 1.0f / l_tot;
    if (qvalid) {
        uint16_t* op = (uint16_t*)a.out + (((int64_t)wk.b * a.Hq + wk.h) * a.S + qrow) * D;
#pragma unroll
        for (int m = 0; m < DBLK; ++m)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                u32x2 w;
                w[0] = pack_bf16x2(oacc[m][4 * q] * inv, oacc[m][4 * q + 1] * inv);
                w[1] = pack_bf16x2(oacc[m][4 * q + 2] * inv, oacc[m][4 * q + 3] * inv);
                *(u32x2*)(op + 32 * m + 8 * q + 4 * hf) = w;
            }
        if (hf == 0) {
            a.lse[((int64_t)wk.b * a.Hq + wk.h) * a.S + qrow] =
                empty ? kNegInf : (m_run + __log2f(l_tot)) * kLn2;
        }
    }
}

// ============================================================ SIMT kernel
//
// General fallback (fp32 inputs, or block sizes the MFMA kernel does not take).
// Two lanes share a query row, each holding half of D; keys are staged in LDS
// 32 at a time as fp32.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void attn_simt_kernel(AttnArgs a) {
    constexpr int HALF = D / 2;
    constexpr int KC = 32;
    __shared__ float Ks[KC][D + 4];
    __shared__ float Vs[KC][D + 4];
    const int tid = threadIdx.x;
    const int64_t total = (int64_t)a.B * a.Hq * a.NQ;
    const Work wk = decode_work(blockIdx.x, total, a.Hq, a.Hkv, a.NQ);
    const int q_tile0 = wk.i * a.block_q;
    const int q_tile_end = min(q_tile0 + a.block_q, a.S);
    const char* qbase = (const char*)a.q;
    const int esz = BF16 ? 2 : 4;
    auto ld = [&](const void* base, int64_t idx) -> float {
        if constexpr (BF16) return __uint_as_float((uint32_t)((const uint16_t*)base)[idx] << 16);
        else return ((const float*)base)[idx];
    };
    (void)qbase;
    (void)esz;
    const int64_t kvoff = ((int64_t)wk.b * a.Hkv + wk.g) * a.S * D;
    const int64_t qoff = ((int64_t)wk.b * a.Hq + wk.h) * a.S * D;

    for (int rc = q_tile0; rc < q_tile_end; rc += 128) {
        const int row = rc + (tid >> 1);
        const int half = tid & 1;
        const bool rvalid = row < q_tile_end;
        const int chunk_last = min(rc + 128, q_tile_end) - 1;
        float qv[HALF], ov[HALF];
#pragma unroll
        for (int d = 0; d < HALF; ++d) {
            qv[d] = rvalid ? ld(a.q, qoff + (int64_t)row * D + half * HALF + d) : 0.f;
            ov[d] = 0.f;
        }
        float m_run = kNegInf, l_run = 0.f;
        int e_begin, e_end;
        tile_range(a, wk.b, wk.h, wk.i, chunk_last, e_begin, e_end);
        for (int e = e_begin; e < e_end; ++e) {
            const int j = a.row_ptr ? a.col_idx[e] : e;
            const int kt0 = j * a.block_kv;
            const int kt1 = min(kt0 + a.block_kv, a.S);
            for (int kc = kt0; kc < kt1; kc += KC) {
                if (a.causal && kc > chunk_last) break;
                const int nkeys = min(KC, kt1 - kc);
                __syncthreads();
                for (int x = tid; x < KC * D; x += 256) {
                    const int kr = x / D, d = x % D;
                    const bool ok = kr < nkeys;
                    Ks[kr][d] = ok ? ld(a.k, kvoff + (int64_t)(kc + kr) * D + d) : 0.f;
                    Vs[kr][d] = ok ? ld(a.v, kvoff + (int64_t)(kc + kr) * D + d) : 0.f;
                }
                __syncthreads();
                float sv[KC];
                float mx = kNegInf;
#pragma unroll
                for (int kr = 0; kr < KC; ++kr) {
                    float dot = 0.f;
#pragma unroll
                    for (int d = 0; d < HALF; ++d) dot += qv[d] * Ks[kr][half * HALF + d];
                    dot += __shfl_xor(dot, 1);
                    float x = dot * a.scale_log2;
                    const int key = kc + kr;
                    if (kr >= nkeys || (a.causal && key > row)) x = kNegInf;
                    sv[kr] = x;
                    mx = fmaxf(mx, x);
                }
                const float m_new = fmaxf(m_run, mx);
                const float m_use = (m_new == kNegInf) ? 0.f : m_new;
                const float alpha = exp2f(m_run - m_use);
                m_run = m_new;
                l_run *= alpha;
#pragma unroll
                for (int d = 0; d < HALF; ++d) ov[d] *= alpha;
#pragma unroll
                for (int kr = 0; kr < KC; ++kr) {
                    const float p = exp2f(sv[kr] - m_use);
                    l_run += p;
#pragma unroll
                    for (int d = 0; d < HALF; ++d) ov[d] += p * Vs[kr][half * HALF + d];
                }
            }
        }
        if (rvalid) {
            const bool empty = !(l_run > 0.f);
            const float inv = empty ? 0.f : 1.0f / l_run;
            const int64_t o = qoff + (int64_t)row * D + half * HALF;
            if constexpr (BF16) {
                uint16_t* op = (uint16_t*)a.out;
#pragma unroll
                for (int d = 0; d < HALF; ++d) op[o + d] = (uint16_t)f32_to_bf16_bits(ov[d] * inv);
            } else {
                float* op = (float*)a.out;
#pragma unroll
                for (int d = 0; d < HALF; ++d) op[o + d] = ov[d] * inv;
            }
            if (half == 0)
                a.lse[((int64_t)wk.b * a.Hq + wk.h) * a.S + row] =
                    empty ? kNegInf : (m_run + log2f(l_run)) * kLn2;
        }
    }
}

}  // namespace

bool attn_mfma_supported(const AttnArgs& a, int bf16) {
    return bf16 && a.block_kv == 64 && a.block_q % 32 == 0 && a.block_q >= 32 && a.block_q <= 128 &&
           (a.D == 64 || a.D == 128);
}

hipError_t launch_attn_mfma(const AttnArgs& a, hipStream_t stream) {
    const int64_t total = (int64_t)a.B * a.Hq * a.NQ;
    if (total == 0) return hipSuccess;
    const dim3 grid((unsigned)total);
    const int nw = a.block_q / 32;
#define NSA_ATTN(DD, NWW)                                                                             \
    do {                                                                                              \
        const size_t lds_bytes = MfmaLds<DD>::BYTES;                                                 \
        hipLaunchKernelGGL((attn_mfma_kernel<DD, NWW>), grid, dim3(64 * NWW), lds_bytes, stream, a); \
    } while (0)
    if (a.D == 128) {
        if (nw == 4) NSA_ATTN(128, 4);
        else if (nw == 2) NSA_ATTN(128, 2);
        else if (nw == 1) NSA_ATTN(128, 1);
        else return hipErrorInvalidValue;
    } else if (a.D == 64) {
        if (nw == 4) NSA_ATTN(64, 4);
        else if (nw == 2) NSA_ATTN(64, 2);
        else if (nw == 1) NSA_ATTN(64, 1);
        else return hipErrorInvalidValue;
    } else {
        return hipErrorInvalidValue;
    }
#undef NSA_ATTN
    return hipGetLastError();
}

hipError_t launch_attn_simt(const AttnArgs& a, int bf16, hipStream_t stream) {
    const int64_t total = (int64_t)a.B * a.Hq * a.NQ;
    if (total == 0) return hipSuccess;
    const dim3 grid((unsigned)total);
#define NSA_SIMT(DD, BB) hipLaunchKernelGGL((attn_simt_kernel<DD, BB>), grid, dim3(256), 0, stream, a)
    if (a.D == 64) {
        if (bf16) NSA_SIMT(64, true);
        else NSA_SIMT(64, false);
    } else if (a.D == 128) {
        if (bf16) NSA_SIMT(128, true);
        else NSA_SIMT(128, false);
    } else {
        return hipErrorInvalidValue;
    }
#undef NSA_SIMT
    return hipGetLastError();
}

}  // namespace nsa
