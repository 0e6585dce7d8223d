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
#include "device_common.h"

#include <algorithm>
#include <float.h>
#include <math.h>
#include <mutex>
#include <vector>

namespace nsa {

// Split partials of the allocation-free decode call (nsa_decode_attn_static):
// one copy per GPU, held while the process runs. Host code must never pass
// this name to a kernel (on the host it is only a stand-in); it uses the
// device address that decode_scratch() looks up.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void** ptr) {
    static std::mutex mu;
    static std::vector<void*> addr;  // per device ordinal
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(mu);
    if ((size_t)dev >= addr.size()) addr.resize((size_t)dev + 1, nullptr);
    if (!addr[dev]) {
        void* p = nullptr;
        if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;  // NaN stays NaN
    u += 0x7fffu + ((u >> 16) & 1u);                                 // round to nearest even
    return u >> 16;
}


// Work item of a workgroup. Workgroups are dispatched round-robin over the 8
// XCDs (block n runs on XCD n % 8); inside each run of 64 consecutive blocks,
// XCD x receives the 8 consecutive work items 8x .. 8x+7 of that run, so the
// query heads of one GQA group (which share the diagonal and pinned tiles) hit
// the same L2. Work items are ordered kv-head major, then query tile
// descending (longest causal rows first), then query head within the group,
// so the whole chip works on one kv head (64 MiB of K/V at 128k tokens) at a
// time. Measured on MI355X, scattered 32 KiB tile reads from a 64 MiB region
// stream no faster than from HBM (the last-level cache adds no bandwidth for
// this pattern); only the per-XCD L2 hits that the GQA grouping creates
// (shared diagonal and pinned tiles) save HBM traffic.
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

// Range [start, end) of CSR entries to visit for query rows up to absolute key
// position q_last (inclusive). Column lists are ascending, so under causal the
// visited prefix ends at the first tile that starts after q_last.
__device__ __forceinline__ void tile_range(const AttnArgs& a, int b, int h, int i, int q_last, int& start,
                                           int& end) {
    if (a.row_ptr) {
        const int hs = (a.Hsel == 1) ? 0 : h;
        const int64_t r = a.qpack ? (int64_t)(a.Bsel == 1 ? 0 : b)  // shared selection, one query tile
                                  : ((int64_t)(a.Bsel == 1 ? 0 : b) * a.Hsel + hs) * a.NQ + i;
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

// The same range computed by a whole wavefront: the causal end is found 64
// entries at a time with one vector load and a ballot (the visible entries
// form a prefix of the ascending list), instead of a chain of dependent
// scalar loads. `lane` is the lane index; the result is wave-uniform.
__device__ __forceinline__ void tile_range_wave(const AttnArgs& a, int b, int h, int i, int q_last, int lane,
                                                int& start, int& end) {
    if (!a.row_ptr || !a.causal) {
        tile_range(a, b, h, i, q_last, start, end);
        return;
    }
    const int hs = (a.Hsel == 1) ? 0 : h;
    const int64_t r = a.qpack ? (int64_t)(a.Bsel == 1 ? 0 : b)
                              : ((int64_t)(a.Bsel == 1 ? 0 : b) * a.Hsel + hs) * a.NQ + i;
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

// ============================================================ MFMA kernel
//
// LDS, per workgroup: two K stages and two V stages of one 64-key tile each,
// row-major (64 x D bf16, no padding), filled by buffer-to-LDS DMA. Rows are
// XOR-swizzled in 16-byte chunks so both read patterns are bank-conflict free:
//   K (read 16 bytes per lane, 16 rows per pass):  chunk ^= (row / RPB) % CH
//   V (transposed 8-byte reads, 4 rows per pass):  chunk ^= 4 * ((row / RPB) % 4) % CH
// (RPB = token rows per 256-byte bank row, CH = 16-byte chunks per token row).
//
// Per tile n the loop issues S(n+1) = K(n+1) Q^T on the matrix cores before the
// softmax of tile n, so the exponentials of one tile run under the QK^T of the
// next, then O^T += V(n)^T P(n)^T. V^T fragments come straight from the
// row-major V tile with ds_read_b64_tr_b16: within each 16-lane group, result
// element e of lane i is element (i mod 4) of the 8 bytes addressed by lane
// 4e + i/4, so lane i receives one d column over four keys.
template <int D>
struct MfmaGeo {
    static constexpr int ROWB = D * 2;            // bytes per token row
    static constexpr int CH = ROWB / 16;          // 16-byte chunks per row
    static constexpr int RPB = 256 / ROWB;        // rows per 256-byte bank row
    static constexpr int TILEB = 64 * ROWB;       // bytes per 64-row tile
    static constexpr int RPI = 1024 / ROWB;       // rows per 1 KiB DMA instruction
    static constexpr int NINSTR = TILEB / 1024;   // DMA instructions per tile
    static constexpr int BYTES = 4 * TILEB;       // 2 K stages + 2 V stages
    __device__ static int kswz(int row) { return (row / RPB) % CH; }
    __device__ static int vswz(int row) { return (4 * ((row / RPB) % 4)) % CH; }
};

template <int D, int NW>
__global__ __launch_bounds__(64 * NW, 2) void attn_mfma_kernel(AttnArgs a) {
    constexpr int NT = 64 * NW;
    constexpr int BKV = 64;
    constexpr int KSTEPS = D / 16;      // QK^T contraction steps of 16
    constexpr int DBLK = D / 32;        // O^T row blocks of 32
    using G = MfmaGeo<D>;
    constexpr int IPW = (G::NINSTR + NW - 1) / NW;  // DMA instructions per wave per tile
    extern __shared__ __attribute__((aligned(1024))) char lds[];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hf = lane >> 5;
    const int64_t total = (int64_t)a.B * a.Hq * a.NQ;
    const int split = (int)(blockIdx.x % a.nsplit);
    const Work wk = decode_work(blockIdx.x / a.nsplit, total, a.Hq, a.Hkv, a.NQ);
    const int bq = a.block_q;
    const int q0 = wk.i * bq;
    const int qw0 = q0 + wave * 32;                  // first query row of this wave
    const int q_last = min(q0 + bq, a.S) - 1;        // last real query row of the tile
    const int qrow = qw0 + l32;                      // this lane's query row
    const bool qvalid = qrow < a.S && (wave * 32 + l32) < bq;

    // Per-head buffer resources: 32-bit offsets, and reads past the end of the
    // head return zeros (ragged tails need no branches). The host guarantees
    // (S + 64) * D * 2 < 2^31.
    const int head_bytes = a.S * G::ROWB;          // one query head
    const int kv_bytes = a.Skv * G::ROWB;          // the keys of one kv head
    const __amdgpu_buffer_rsrc_t qrs =
        make_rsrc((const uint16_t*)a.q + (((int64_t)wk.b * a.Hq + wk.h) * a.S) * D, head_bytes);
    const uint16_t* kbase = (const uint16_t*)a.k + ((int64_t)wk.b * a.Hkv + wk.g) * a.kv_rows * D;
    const uint16_t* vbase = (const uint16_t*)a.v + ((int64_t)wk.b * a.Hkv + wk.g) * a.kv_rows * D;

    // Q^T operand: lane holds q[qrow][16*ks + 8*hf .. +8] for every ks (zeros past S).
    bf16x8 qf[KSTEPS];
    {
        const int qoff = (wave * 32 + l32) < bq ? (qrow * D + 8 * hf) * 2 : head_bytes;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks)
            qf[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qrs, qoff + 32 * ks, 0, 0));
    }

    // Token position of this lane's row and the last position of the tile
    // (packed heads: every head's tokens 0 .. qpack - 1 may be in the tile).
    const int qpos = a.qpack ? qrow % a.qpack : qrow;
    int e_begin, e_end;
    tile_range_wave(a, wk.b, wk.h, wk.i, a.q_off + (a.qpack ? a.qpack - 1 : q_last), lane, e_begin, e_end);
    if (a.nsplit > 1) {  // this workgroup's share of the row's tiles
        const int per = (e_end - e_begin + a.nsplit - 1) / a.nsplit;
        e_begin = min(e_end, e_begin + split * per);
        e_end = min(e_end, e_begin + per);
    }
    const int ntiles = e_end - e_begin;

    // The row's kv-tile indices, 64 at a time: lane x holds entry base + x and
    // the loop reads them with readlane (no memory access per tile).
    int col_base = e_begin;
    int col_lane = 0;
    auto fetch_cols = [&](int base) {
        col_base = base;
        const int e = base + lane;
        col_lane = a.row_ptr ? (e < e_end ? a.col_idx[e] : 0) : e;
    };
    fetch_cols(e_begin);
    auto tile_of = [&](int n) -> int {  // n-th visited tile (n uniform)
        const int e = e_begin + n;
        if (e - col_base >= 64) fetch_cols(e);
        return __builtin_amdgcn_readlane(col_lane, e - col_base);
    };

    // DMA: wave w issues instructions w, w + NW, ...; lane L of instruction ii
    // fills LDS bytes ii*1024 + 16L, i.e. row ii*RPI + L/CH, physical chunk L%CH,
    // from the logical chunk given by the row's swizzle.
    // The DMA is issued by the instruction itself and every wait on it is
    // explicit (vmcnt(0) at the end of a step), so the tiles of step n + 1 stay
    // in flight through the whole of step n, transposed V reads included.
    char* kst[2] = {lds, lds + G::TILEB};
    char* vst[2] = {lds + 2 * G::TILEB, lds + 3 * G::TILEB};
    const uint32_t lds0 = lds_address(lds);
    // Per-lane source offsets inside a tile of this wave's DMA instructions
    // (they do not depend on the tile); the tile itself is selected by the
    // base of the buffer resource, whose record count ends at the last key,
    // so the rows of a ragged last tile past it read as zeros (their keys
    // are masked, so P = 0 for them).
    int kvo[IPW], vvo[IPW];
#pragma unroll
    for (int x = 0; x < IPW; ++x) {
        const int ii = wave + NW * x;
        const int row = ii * G::RPI + lane / G::CH, pc = lane % G::CH;
        kvo[x] = row * G::ROWB + (pc ^ G::kswz(row)) * 16;
        vvo[x] = row * G::ROWB + (pc ^ G::vswz(row)) * 16;
    }
    auto dma = [&](const uint16_t* base, const int (&vo)[IPW], char* stage_base, int j) {
        const uint32_t off = (uint32_t)j * (BKV * G::ROWB);
        const u32x4 rs = rsrc_words((const char*)base + off, (uint32_t)kv_bytes - off);
        const uint32_t sb = lds0 + (uint32_t)(stage_base - lds);
#pragma unroll
        for (int x = 0; x < IPW; ++x) {
            const int ii = wave + NW * x;
            if (G::NINSTR % NW == 0 || ii < G::NINSTR) dma16(rs, sb + ii * 1024, vo[x]);
        }
    };
    auto dma_k = [&](int j, int stage) { dma(kbase, kvo, kst[stage], j); };
    auto dma_v = [&](int j, int stage) { dma(vbase, vvo, vst[stage], j); };

    // LDS read offsets (bytes) that do not depend on the tile.
    // K: lane reads row 32*mb + l32, logical chunk 2*ks + hf.
    // V^T: lane (group g = lane/16, s = lane%16) addresses row 16*kk + 4*hf + s/4
    // (+8 for the second half) at d = 32*m + 16*(g%2) + 4*(s%4).
    const int vg = lane >> 4, vs = lane & 15;
    const int v_e = vs >> 2, v_q = vs & 3;
    // The swizzles depend on the row only through bits that the tile-relative
    // steps (32 rows between K row blocks, 16 rows between V k-steps, 8 rows
    // between the two halves of a V^T fragment) leave unchanged, so each read
    // is a per-lane offset below plus a compile-time constant.
    int koff[KSTEPS];  // K: row l32, logical chunk 2*ks + hf
#pragma unroll
    for (int ks_ = 0; ks_ < KSTEPS; ++ks_) koff[ks_] = l32 * G::ROWB + (((2 * ks_ + hf) ^ G::kswz(l32)) * 16);
    int voff[DBLK];    // V^T: row 4*hf + v_e, column d = 32*m + 16*(vg&1) + 4*v_q
#pragma unroll
    for (int m = 0; m < DBLK; ++m) {
        const int r = 4 * hf + v_e;
        const int d = 32 * m + 16 * (vg & 1) + 4 * v_q;
        voff[m] = r * G::ROWB + (((d >> 3) ^ G::vswz(r)) * 16) + (d & 7) * 2;
    }

    f32x16 oacc[DBLK];
#pragma unroll
    for (int m = 0; m < DBLK; ++m) oacc[m] = (f32x16){};
    float m_ref = kNegInf;  // exponent reference of this lane's query row (raw dot-product units)
    float l_run = 0.f;      // partial sum over this lane's half of every tile

    // Masks of a partial tile (causal diagonal or ragged tail): keys past the
    // lane's query row or past S get -inf. Only partial tiles take this branch.
    auto mask_tile = [&](f32x16 (&sacc)[2], int key0) {
        const bool need_mask = (a.causal && key0 + BKV - 1 > a.q_off + (a.qpack ? 0 : qw0)) || (key0 + BKV > a.Skv);
        if (need_mask) {
            int lim = min(BKV - 1, a.Skv - 1 - key0);         // last visible key offset
            if (a.causal) lim = min(lim, a.q_off + qpos - key0);
            // Key offset of element x is c(x) + 4 * hf: compare c(x), a
            // compile-time constant, with lim - 4 * hf.
            const int limh = lim - 4 * hf;
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int x = 0; x < 16; ++x) {
                    const int c = 32 * mb + 8 * (x >> 2) + (x & 3);
                    sacc[mb][x] = c <= limh ? sacc[mb][x] : kNegInf;
                }
        }
    };
    // S^T = K Q^T for the tile in K stage `stage` (raw dot products).
    auto qk_frag = [&](const char* ks, int ks_, int mb) -> bf16x8 {
        return __builtin_bit_cast(bf16x8, *(const u32x4*)(ks + 32 * mb * G::ROWB + koff[ks_]));
    };
    // One straight-line block: the matrix cores compute S(next) while the
    // vector ALUs turn S(cur) into P (exponentials, bf16 pack, row sum). Lane
    // holds query qrow and keys 32*mb + 8*q + 4*hf + e at sacc[mb][4q + e];
    // the softmax scale is folded into one FMA per logit.
    // Reference: the exponentials are taken against the row's current
    // reference m_ref (raw units) without a row maximum. Only when a row's
    // exponentials of this tile sum past 2^20 (some p beyond 2^20 / 64), or the
    // row has no reference yet, does the wave take the row maximum: those
    // rows move their reference to it and recompute the tile. Any reference
    // gives the same normalised result and LSE adds it back; bounding p keeps
    // O and the row sum far from overflow.
    auto qk_softmax = [&](f32x16 (&scur)[2], f32x16 (&snext)[2], int kstage, bf16x8 (&pf)[4]) -> float {
        const char* ks = kst[kstage];
        snext[0] = (f32x16){};
        snext[1] = (f32x16){};
        const float mref_s = (m_ref == kNegInf) ? 0.f : m_ref * a.scale_log2;
        float psum = 0.f;
        // K fragments one k-step ahead of their products (two buffers),
        // fenced so the reads of step ks + 1 are in flight under step ks.
        bf16x8 kf[2][2];
        kf[0][0] = qk_frag(ks, 0, 0);
        kf[0][1] = qk_frag(ks, 0, 1);
#pragma unroll
        for (int ks_ = 0; ks_ < KSTEPS; ++ks_) {
            if (ks_ + 1 < KSTEPS) {
                kf[(ks_ + 1) & 1][0] = qk_frag(ks, ks_ + 1, 0);
                kf[(ks_ + 1) & 1][1] = qk_frag(ks, ks_ + 1, 1);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
                snext[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks_ & 1][mb], qf[ks_], snext[mb], 0, 0, 0);
            if (ks_ < 4) {  // four of the eight k-steps carry the softmax of one P fragment each
                const int kk = ks_, mb = kk >> 1, q4 = 8 * (kk & 1);
#pragma unroll
                for (int x = 0; x < 8; ++x) {
                    const float pv = fast_exp2(__builtin_fmaf(scur[mb][q4 + x], a.scale_log2, -mref_s));
                    psum += pv;
                    pf[kk][x] = (__bf16)pv;
                }
                // Keep this fragment's exponentials here, under the products,
                // rather than sunk to their use in O^T += V^T P^T.
                u32x4 pw = __builtin_bit_cast(u32x4, pf[kk]);
                asm volatile("" : "+v"(pw), "+v"(psum));
                pf[kk] = __builtin_bit_cast(bf16x8, pw);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // The row's sum over both lane halves (the other half holds its other
        // keys): the swap returns this lane's and the other half's value, in an
        // order that depends on the half, and their sum is the same in both.
        const auto ps = __builtin_amdgcn_permlane32_swap(__float_as_uint(psum), __float_as_uint(psum), false, false);
        const float prow = __uint_as_float(ps[0]) + __uint_as_float(ps[1]);
        const bool redo = !(prow <= 1048576.0f) || m_ref == kNegInf;  // 2^20; also catches inf
        float alpha = 1.0f;
        if (__ballot(redo)) {  // wave-uniform; rare after a row's first tile
            float mx = kNegInf;
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int x = 0; x < 16; ++x) mx = fmaxf(mx, scur[mb][x]);
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
            mx = fmaxf(mx, fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])));
            if (redo) {
                const float m_new = fmaxf(mx, m_ref);
                alpha = (m_new > m_ref) ? fast_exp2((m_ref - m_new) * a.scale_log2) : 1.0f;  // 0 from -inf
                const float ms = (m_new == kNegInf) ? 0.f : m_new * a.scale_log2;
                psum = 0.f;
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const int mb = kk >> 1, q4 = 8 * (kk & 1);
#pragma unroll
                    for (int x = 0; x < 8; ++x) {
                        const float pv = fast_exp2(__builtin_fmaf(scur[mb][q4 + x], a.scale_log2, -ms));
                        psum += pv;
                        pf[kk][x] = (__bf16)pv;
                    }
                }
                m_ref = m_new;
            }
        }
        l_run = l_run * alpha + psum;
        return alpha;
    };
    // O^T += V^T P^T ; the V^T fragment of k-step kk, row block m is two
    // transposed reads: keys 16kk + 4hf + (0..3) and 16kk + 8 + 4hf + (0..3).
    auto pv = [&](const bf16x8 (&pf)[4], int vstage) {
        const char* vt = vst[vstage];
        // V^T fragments of k-step kk + 1 are read while the products of k-step
        // kk run (two buffers, fenced as the K fragments above).
        short4_t vlo[2][DBLK], vhi[2][DBLK];
        auto load_v = [&](int kk, int buf) {
#pragma unroll
            for (int m = 0; m < DBLK; ++m) {
                const char* p0 = vt + 16 * kk * G::ROWB + voff[m];
                vlo[buf][m] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)p0);
                vhi[buf][m] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p0 + 8 * G::ROWB));
            }
        };
        load_v(0, 0);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            if (kk + 1 < 4) load_v(kk + 1, (kk + 1) & 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int m = 0; m < DBLK; ++m) {
                const short4_t lo = vlo[kk & 1][m], hi = vhi[kk & 1][m];
                const short8_t w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                oacc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w), pf[kk],
                                                                   oacc[m], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Prologue: K(0), V(0), K(1) in flight; S(0) once K(0) has landed.
    int j_cur = 0, j_next = 0;
    if (ntiles > 0) {
        j_cur = tile_of(0);
        dma_k(j_cur, 0);
        dma_v(j_cur, 0);
    }
    if (ntiles > 1) {
        j_next = tile_of(1);
        dma_k(j_next, 1);
    }
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    __syncthreads();
    f32x16 sa[2], sb[2];
    sa[0] = (f32x16){};
    sa[1] = (f32x16){};
    if (ntiles > 0) {
#pragma unroll
        for (int ks_ = 0; ks_ < KSTEPS; ++ks_)
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
                sa[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qk_frag(kst[0], ks_, mb), qf[ks_], sa[mb], 0, 0, 0);
    }
    __syncthreads();  // K stage 0 is refilled by the first step

    // One step: tile n with S(n) in scur, K(n+1) in K stage (n+1)&1, V(n) in V stage n&1.
    // Tiles entirely after this wave's rows are computed like any other and
    // come out fully masked (p = 0); they are rare (the causal diagonal).
    auto step = [&](int n, f32x16 (&scur)[2], f32x16 (&snext)[2]) {
        const int kst_next = (n + 1) & 1, vst_cur = n & 1;
        const int j_after = (n + 2 < ntiles) ? tile_of(n + 2) : 0;
        if (n + 2 < ntiles) dma_k(j_after, n & 1);          // K(n) stage is free again
        if (n + 1 < ntiles) dma_v(j_next, kst_next);        // V(n-1) stage is free again
        mask_tile(scur, j_cur * BKV);
        bf16x8 pf[4];
        const float alpha = qk_softmax(scur, snext, kst_next, pf);
        if (__ballot(alpha != 1.0f)) {  // wave-uniform: some row moved its reference
#pragma unroll
            for (int m = 0; m < DBLK; ++m) oacc[m] *= alpha;
        }
        pv(pf, vst_cur);
        j_cur = j_next;
        j_next = j_after;
        __builtin_amdgcn_s_waitcnt(kVmcnt0);  // K(n + 2) and V(n + 1) have landed
        bare_barrier();
    };
    int n = 0;
    for (; n + 1 < ntiles; n += 2) {
        step(n, sa, sb);
        step(n + 1, sb, sa);
    }
    if (n < ntiles) step(n, sa, sb);

    // Finish: combine the two lane halves of the row sum.
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const bool empty = !(l_tot > 0.f);
    if (a.nsplit > 1) {  // partial result of this split: unnormalised O, reference and sum
        if (qvalid) {
            const int64_t prow = (((int64_t)wk.b * a.Hq + wk.h) * a.S + qrow) * a.nsplit + split;
            float* po = a.part_o + prow * D;
#pragma unroll
            for (int m = 0; m < DBLK; ++m)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 w = {oacc[m][4 * q], oacc[m][4 * q + 1], oacc[m][4 * q + 2], oacc[m][4 * q + 3]};
                    *(f32x4*)(po + 32 * m + 8 * q + 4 * hf) = w;
                }
            if (hf == 0) {
                a.part_ml[2 * prow] = empty ? kNegInf : m_ref * a.scale_log2;
                a.part_ml[2 * prow + 1] = l_tot;
            }
        }
        return;
    }
    const float inv = empty ? 0.f : 1.0f / l_tot;
    if (qvalid) {
        uint16_t* op = (uint16_t*)a.out + (((int64_t)wk.b * a.Hq + wk.h) * a.S + qrow) * D;
#pragma unroll
        for (int m = 0; m < DBLK; ++m)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                bf16x4 w;
#pragma unroll
                for (int x = 0; x < 4; ++x) w[x] = (__bf16)(oacc[m][4 * q + x] * inv);
                *(bf16x4*)(op + 32 * m + 8 * q + 4 * hf) = w;
            }
        if (hf == 0) {
            a.lse[((int64_t)wk.b * a.Hq + wk.h) * a.S + qrow] =
                empty ? kNegInf : (m_ref * a.scale_log2 + __log2f(l_tot)) * kLn2;
        }
    }
}

// ============================================================ decode kernel
//
// Few query rows over many kv tiles (decoding): one wave of 32 query rows per
// workgroup, as attn_mfma_kernel<D, 1>, but with K read straight into
// registers (in the A-operand layout of S^T = K Q^T: lane (l32, hf) takes 16
// bytes of key row 32*mb + l32 per k-step) and only V staged in LDS (two
// stages, for the transposed reads). A workgroup then needs 2 * 64 * D * 2
// bytes of LDS, so five fit a CU where two of attn_mfma_kernel do, and five
// tile pairs are in flight per CU.
// Per tile n: S(n) from the K(n) registers; V(n+1) is issued into the free V
// stage and K(n+1) into the K registers; then the softmax of tile n and
// O^T += V(n)^T P(n)^T. The compiler's wait for K(n+1) before the next S also
// covers V(n+1), which was issued just before it.
template <int D>
__global__ __launch_bounds__(64, 2) void attn_decode_kernel(AttnArgs a) {
    constexpr int BKV = 64;
    constexpr int KSTEPS = D / 16;
    constexpr int DBLK = D / 32;
    using G = MfmaGeo<D>;
    extern __shared__ __attribute__((aligned(1024))) char lds[];

    const int lane = threadIdx.x & 63;
    const int l32 = lane & 31, hf = lane >> 5;
    const int64_t total = (int64_t)a.B * a.Hq * a.NQ;
    const int split = (int)(blockIdx.x % a.nsplit);
    const Work wk = decode_work(blockIdx.x / a.nsplit, total, a.Hq, a.Hkv, a.NQ);
    const int q0 = wk.i * a.block_q;              // a tile holds at most 32 rows (host-checked)
    const int q_last = min(q0 + 32, a.S) - 1;
    const int qrow = q0 + l32;
    const bool qvalid = qrow < a.S;

    const int head_bytes = a.S * G::ROWB;
    const int kv_bytes = a.Skv * G::ROWB;
    const __amdgpu_buffer_rsrc_t qrs =
        make_rsrc((const uint16_t*)a.q + (((int64_t)wk.b * a.Hq + wk.h) * a.S) * D, head_bytes);
    const __amdgpu_buffer_rsrc_t krs =
        make_rsrc((const uint16_t*)a.k + ((int64_t)wk.b * a.Hkv + wk.g) * a.kv_rows * D, kv_bytes);
    const u32x4 vrs = rsrc_words((const uint16_t*)a.v + ((int64_t)wk.b * a.Hkv + wk.g) * a.kv_rows * D, kv_bytes);

    bf16x8 qf[KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
        qf[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qrs, (qrow * D + 8 * hf) * 2 + 32 * ks,
                                                                                   0, 0));
    __builtin_amdgcn_s_waitcnt(kVmcnt0);  // Q settled before any tile DMA

    const int qpos = a.qpack ? qrow % a.qpack : qrow;
    int e_begin, e_end;
    tile_range_wave(a, wk.b, wk.h, wk.i, a.q_off + (a.qpack ? a.qpack - 1 : q_last), lane, e_begin, e_end);
    if (a.nsplit > 1) {
        const int per = (e_end - e_begin + a.nsplit - 1) / a.nsplit;
        e_begin = min(e_end, e_begin + split * per);
        e_end = min(e_end, e_begin + per);
    }
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

    // V DMA into stage st (rows past Skv read row Skv - 1, weighted by p = 0).
    const uint32_t lds0 = lds_address(lds);
    auto dma_v = [&](int j, int st) {
        const int key0 = j * BKV;
        const uint32_t base = lds0 + st * G::TILEB;
#pragma unroll
        for (int ii = 0; ii < G::NINSTR; ++ii) {
            const int row = ii * G::RPI + lane / G::CH, pc = lane % G::CH;
            const int chunk = pc ^ G::vswz(row);
            dma16(vrs, base + ii * 1024, min(key0 + row, a.Skv - 1) * G::ROWB + chunk * 16);
        }
    };
    // K(j) into registers: kf[mb][ks] = key row 32*mb + l32, elements 16*ks + 8*hf .. + 8.
    bf16x8 kf[2][KSTEPS];
    auto load_k = [&](int j) {
        const int key0 = j * BKV;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            const int off = min(key0 + 32 * mb + l32, a.Skv - 1) * G::ROWB + 16 * hf;
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks)
                kf[mb][ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(krs, off + 32 * ks, 0, 0));
        }
    };

    const int vg = lane >> 4, vs = lane & 15;
    const int v_e = vs >> 2, v_q = vs & 3;
    int voff[DBLK];
#pragma unroll
    for (int m = 0; m < DBLK; ++m) {
        const int r = 4 * hf + v_e;
        const int d = 32 * m + 16 * (vg & 1) + 4 * v_q;
        voff[m] = r * G::ROWB + (((d >> 3) ^ G::vswz(r)) * 16) + (d & 7) * 2;
    }

    f32x16 oacc[DBLK];
#pragma unroll
    for (int m = 0; m < DBLK; ++m) oacc[m] = (f32x16){};
    float m_ref = kNegInf, l_run = 0.f;
    const float tau_raw = 8.0f / a.scale_log2;

    int j_cur = 0, j_next = 0;
    if (ntiles > 0) {
        j_cur = tile_of(0);
        dma_v(j_cur, 0);
        load_k(j_cur);
    }
    for (int n = 0; n < ntiles; ++n) {
        // S^T(n) = K(n) Q^T (the compiler waits here for K(n), and with it for V(n)).
        f32x16 sc[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            sc[mb] = (f32x16){};
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) sc[mb] = mfma32(kf[mb][ks], qf[ks], sc[mb]);
        }
        if (n + 1 < ntiles) {
            j_next = tile_of(n + 1);
            dma_v(j_next, (n + 1) & 1);  // that stage was last read by PV(n - 1)
            load_k(j_next);
        }
        // Masks of a partial tile (causal diagonal or ragged tail).
        const int key0 = j_cur * BKV;
        if ((a.causal && key0 + BKV - 1 > a.q_off + (a.qpack ? 0 : q0)) || (key0 + BKV > a.Skv)) {
            int lim = min(BKV - 1, a.Skv - 1 - key0);
            if (a.causal) lim = min(lim, a.q_off + qpos - key0);
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int x = 0; x < 16; ++x) {
                    const int off = 32 * mb + 8 * (x >> 2) + 4 * hf + (x & 3);
                    sc[mb][x] = off <= lim ? sc[mb][x] : kNegInf;
                }
        }
        // Online softmax with a lazy reference (as attn_mfma_kernel).
        float mx = kNegInf;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int x = 0; x < 16; ++x) mx = fmaxf(mx, sc[mb][x]);
        {  // the other half-wave holds the row's other keys
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
            mx = fmaxf(mx, fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])));
        }
        const bool grow = mx > m_ref + tau_raw;
        const float m_new = grow ? mx : m_ref;
        const float alpha = grow ? fast_exp2((m_ref - m_new) * a.scale_log2) : 1.0f;
        const float mref_s = (m_new == kNegInf) ? 0.f : m_new * a.scale_log2;
        bf16x8 pf[4];
        float psum = 0.f;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int mb = kk >> 1, q4 = 8 * (kk & 1);
#pragma unroll
            for (int x = 0; x < 8; ++x) {
                const float pv = fast_exp2(__builtin_fmaf(sc[mb][q4 + x], a.scale_log2, -mref_s));
                psum += pv;
                pf[kk][x] = (__bf16)pv;
            }
        }
        l_run = l_run * alpha + psum;
        m_ref = m_new;
        if (__ballot(alpha != 1.0f)) {
#pragma unroll
            for (int m = 0; m < DBLK; ++m) oacc[m] *= alpha;
        }
        // O^T += V(n)^T P(n)^T
        const char* vt = lds + (n & 1) * G::TILEB;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
            for (int m = 0; m < DBLK; ++m) {
                const char* p0 = vt + 16 * kk * G::ROWB + voff[m];
                const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)p0);
                const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p0 + 8 * G::ROWB));
                const short8_t w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                oacc[m] = mfma32(__builtin_bit_cast(bf16x8, w), pf[kk], oacc[m]);
            }
        }
        // The V stage read here is refilled two tiles on: its reads must be
        // done before that DMA is issued.
        __builtin_amdgcn_s_waitcnt(kLgkmcnt0);
        j_cur = j_next;
    }
    __builtin_amdgcn_s_waitcnt(kVmcnt0);

    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const bool empty = !(l_tot > 0.f);
    if (a.nsplit > 1) {
        if (qvalid) {
            const int64_t prow = (((int64_t)wk.b * a.Hq + wk.h) * a.S + qrow) * a.nsplit + split;
            float* po = a.part_o + prow * D;
#pragma unroll
            for (int m = 0; m < DBLK; ++m)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 w = {oacc[m][4 * q], oacc[m][4 * q + 1], oacc[m][4 * q + 2], oacc[m][4 * q + 3]};
                    *(f32x4*)(po + 32 * m + 8 * q + 4 * hf) = w;
                }
            if (hf == 0) {
                a.part_ml[2 * prow] = empty ? kNegInf : m_ref * a.scale_log2;
                a.part_ml[2 * prow + 1] = l_tot;
            }
        }
        return;
    }
    const float inv = empty ? 0.f : 1.0f / l_tot;
    if (qvalid) {
        uint16_t* op = (uint16_t*)a.out + (((int64_t)wk.b * a.Hq + wk.h) * a.S + qrow) * D;
#pragma unroll
        for (int m = 0; m < DBLK; ++m)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                bf16x4 w;
#pragma unroll
                for (int x = 0; x < 4; ++x) w[x] = (__bf16)(oacc[m][4 * q + x] * inv);
                *(bf16x4*)(op + 32 * m + 8 * q + 4 * hf) = w;
            }
        if (hf == 0) {
            a.lse[((int64_t)wk.b * a.Hq + wk.h) * a.S + qrow] =
                empty ? kNegInf : (m_ref * a.scale_log2 + __log2f(l_tot)) * kLn2;
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
    const int64_t kvoff = ((int64_t)wk.b * a.Hkv + wk.g) * a.kv_rows * D;
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
        tile_range(a, wk.b, wk.h, wk.i, a.q_off + chunk_last, e_begin, e_end);
        for (int e = e_begin; e < e_end; ++e) {
            const int j = a.row_ptr ? a.col_idx[e] : e;
            const int kt0 = j * a.block_kv;
            const int kt1 = min(kt0 + a.block_kv, a.Skv);
            for (int kc = kt0; kc < kt1; kc += KC) {
                if (a.causal && kc > a.q_off + chunk_last) break;
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
                    if (kr >= nkeys || (a.causal && key > a.q_off + row)) x = kNegInf;
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

// Merges the split partials of one query row: with M the largest reference,
// w_s = 2^(m_s - M), O = sum_s w_s O_s / sum_s w_s l_s and
// LSE = (M + log2 sum_s w_s l_s) ln 2. One workgroup per row: its four waves
// take every fourth split (D / 64 elements per lane) and add up through LDS.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
    constexpr int PER = D / 64;
    __shared__ float sm[4], sl[4];
    __shared__ float so[4][D];
    const int64_t row = blockIdx.x;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int ns = a.nsplit;
    const float* ml = a.part_ml + row * ns * 2;
    float m = kNegInf;
    for (int s = threadIdx.x; s < ns; s += 256) m = fmaxf(m, ml[2 * s]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if (lane == 0) sm[w] = m;
    __syncthreads();
    const float M = fmaxf(fmaxf(sm[0], sm[1]), fmaxf(sm[2], sm[3]));
    float lsum = 0.f, acc[PER];
#pragma unroll
    for (int x = 0; x < PER; ++x) acc[x] = 0.f;
#pragma unroll 4
    for (int s = w; s < ns; s += 4) {
        const float ms = ml[2 * s];
        const float ws = ms == kNegInf ? 0.f : exp2f(ms - M);  // splits that saw no key add nothing
        lsum += ws * ml[2 * s + 1];
        const float* po = a.part_o + (row * ns + s) * D;
#pragma unroll
        for (int x = 0; x < PER; ++x) acc[x] += ws * po[lane + 64 * x];
    }
#pragma unroll
    for (int x = 0; x < PER; ++x) so[w][lane + 64 * x] = acc[x];
    if (lane == 0) sl[w] = lsum;
    __syncthreads();
    if (w != 0) return;
    const float L = (sl[0] + sl[1]) + (sl[2] + sl[3]);
    const bool empty = !(L > 0.f);
    const float inv = empty ? 0.f : 1.0f / L;
#pragma unroll
    for (int x = 0; x < PER; ++x) {
        const int d = lane + 64 * x;
        const float o = ((so[0][d] + so[1][d]) + (so[2][d] + so[3][d])) * inv;
        if constexpr (BF16) ((__bf16*)a.out)[row * D + d] = (__bf16)o;
        else ((float*)a.out)[row * D + d] = o;
    }
    if (lane == 0) a.lse[row] = empty ? kNegInf : (M + __log2f(L)) * kLn2;
}

}  // namespace

bool attn_decode_supported(const AttnArgs& a, int bf16) {
    return attn_mfma_supported(a, bf16) && (a.block_q == 32 || (a.NQ == 1 && a.S <= 32));
}

hipError_t launch_attn_decode(const AttnArgs& a, hipStream_t stream) {
    const int64_t total = (int64_t)a.B * a.Hq * a.NQ * std::max(1, a.nsplit);
    if (total == 0) return hipSuccess;
    if (!(a.block_q == 32 || (a.NQ == 1 && a.S <= 32))) return hipErrorInvalidValue;
    if (a.D == 128)
        hipLaunchKernelGGL((attn_decode_kernel<128>), dim3((unsigned)total), dim3(64), 2 * MfmaGeo<128>::TILEB,
                           stream, a);
    else if (a.D == 64)
        hipLaunchKernelGGL((attn_decode_kernel<64>), dim3((unsigned)total), dim3(64), 2 * MfmaGeo<64>::TILEB,
                           stream, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_attn_combine(const AttnArgs& a, int bf16, hipStream_t stream) {
    const int64_t rows = (int64_t)a.B * a.Hq * a.S;
    if (rows == 0) return hipSuccess;
    const dim3 grid((unsigned)rows);
    if (a.D == 128) {
        if (bf16) hipLaunchKernelGGL((attn_combine_kernel<128, true>), grid, dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((attn_combine_kernel<128, false>), grid, dim3(256), 0, stream, a);
    } else if (a.D == 64) {
        if (bf16) hipLaunchKernelGGL((attn_combine_kernel<64, true>), grid, dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((attn_combine_kernel<64, false>), grid, dim3(256), 0, stream, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

bool attn_mfma_supported(const AttnArgs& a, int bf16) {
    // Buffer offsets are 32-bit: one head plus a tile of slack must stay below 2^31 bytes.
    const bool fits = ((int64_t)std::max(a.S, a.Skv) + 64) * a.D * 2 < ((int64_t)1 << 31);
    return bf16 && fits && a.block_kv == 64 && a.block_q % 32 == 0 && a.block_q >= 32 && a.block_q <= 128 &&
           (a.D == 64 || a.D == 128);
}

hipError_t launch_attn_mfma(const AttnArgs& a, hipStream_t stream) {
    const int64_t total = (int64_t)a.B * a.Hq * a.NQ * std::max(1, a.nsplit);
    if (total == 0) return hipSuccess;
    const dim3 grid((unsigned)total);
    const int nw = a.block_q / 32;
#define NSA_ATTN(DD, NWW)                                                                             \
    do {                                                                                              \
        const size_t lds_bytes = MfmaGeo<DD>::BYTES;                                                 \
        hipLaunchKernelGGL((attn_mfma_kernel<DD, NWW>), grid, dim3(64 * NWW), lds_bytes, stream, a); \
    } while (0)
    if (a.D == 128) {
        if (nw == 4) NSA_ATTN(128, 4);
        else if (nw == 3) NSA_ATTN(128, 3);
        else if (nw == 2) NSA_ATTN(128, 2);
        else if (nw == 1) NSA_ATTN(128, 1);
        else return hipErrorInvalidValue;
    } else if (a.D == 64) {
        if (nw == 4) NSA_ATTN(64, 4);
        else if (nw == 3) NSA_ATTN(64, 3);
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
