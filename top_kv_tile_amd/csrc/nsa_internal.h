// Internal launch interface between the C ABI (nsa_api.cpp) and the HIP
// kernels. Every launcher enqueues on `stream` and returns the hipError_t of
// the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nsa {

// ---- selection stage -------------------------------------------------------

// Mean over blocks of `block` tokens: x (heads, S, D) -> out (heads, N, D) fp32.
hipError_t launch_pool(const void* x, int bf16, int64_t heads, int S, int D, int block,
                       float* out, hipStream_t stream);
// The same for tiles [tile0, tile0 + ntiles) of heads laid out x_head_rows rows
// apart (S valid rows each), into out tiles laid out out_head_tiles apart.
hipError_t launch_pool_range(const void* x, int bf16, int64_t heads, int S, int64_t x_head_rows, int D, int block,
                             int tile0, int ntiles, float* out, int64_t out_head_tiles, hipStream_t stream);

// out[b, n, :] = mean over h of in[b, h, n, :]  (in: (B, H, Ns, D) fp32, rows n < N
// used; Ns = 0 means Ns = N).
hipError_t launch_head_mean(const float* in, int B, int H, int N, int D, float* out,
                            hipStream_t stream, int Ns = 0);

// Scores for selection heads [h0, h0 + nh): s[b, h - h0, i, j] = qh[b, h, i] . kh[b, h / group, j]
// qh: (B, Hsel, NQ, D) fp32, kh: (B, Hk, NK, D) fp32, s: (B, nh, NQ, NK) fp32.
// kh rows of one head are NKs apart (NKs = 0 means NK).
// q_rows = 1 or 2: qh holds query rows (bf16 or fp32) of single-token tiles,
// pooled on the fly (NQ <= 8 only).
hipError_t launch_scores(const void* qh, const float* kh, int B, int Hsel, int Hk, int group,
                         int h0, int nh, int NQ, int NK, int D, float* s, hipStream_t stream, int NKs = 0,
                         int q_rows = 0);

// Per-row top-k over the score chunk of heads [h0, h0 + nh) and CSR emission.
constexpr int kInlineMaskWords = 64;  // mask words a top-k launch can carry in its arguments
struct TopkArgs {
    const float* scores;       // (B, nh, NQ, NK)
    int B, Hsel, h0, nh, NQ, NK, NKW;
    int block_q, block_kv;
    int64_t q_off = 0;         // absolute key position of query token 0 (diagonal)
    float budget;
    const uint64_t* pin_words; // (pb, ph, NQ, NKW) or null; bit (j % 64) of word j / 64
    int pb, ph;
    const uint64_t* drop_words;
    int db, dh;
    int pin_at = -1, drop_at = -1;  // with pin_words / drop_words null: the words start at
                                    // words[pin_at] / words[drop_at] (-1: no such mask)
    uint64_t words[kInlineMaskWords];
    const int32_t* row_src;    // (B*Hsel*NQ + 1) row offsets (planned on the host), read; or null:
    int32_t row_step;          //   then row r starts at r * row_step (every row keeps row_step tiles)
    int32_t* row_ptr;          // (B*Hsel*NQ + 1) the caller's row offsets, written from row_src
    int8_t* keep;              // (B, Hsel, NQ, NK)
    int32_t* col_idx;
};
hipError_t launch_topk(const TopkArgs& a, hipStream_t stream);

// ---- attention stage -------------------------------------------------------

struct AttnArgs {
    const void* q;            // (B, Hq, S, D): S query tokens
    const void* k;            // (B, Hkv, kv_rows, D): the first Skv rows of each head are keys
    const void* v;
    void* out;                // (B, Hq, S, D), dtype of q
    float* lse;               // (B, Hq, S)
    int Skv;                  // keys per head (== S outside decoding)
    int64_t kv_rows;          // rows per kv head in memory (>= Skv; a cache's capacity)
    int q_off;                // absolute key position of query token 0 (causal: u <= q_off + t)
    int nsplit = 1;           // > 1: each row's tiles are split over nsplit workgroups (MFMA path)
    float* part_o = nullptr;  // split partials: (B*Hq*S, nsplit, D) unnormalised O
    float* part_ml = nullptr; // (B*Hq*S, nsplit, 2): exponent reference (log2 units) and sum
    // > 0 (MFMA path): query heads packed per kv head. The call then describes
    // Hq = Hkv heads of S = G * qpack rows each, row r being token r % qpack of
    // query head g * G + r / qpack (the same memory, since a GQA group's heads
    // are adjacent); every row uses selection row (b, 0, 0), so the selection
    // is shared by the heads and has one query tile.
    int qpack = 0;
    const int32_t* row_ptr;   // null = dense
    const int32_t* col_idx;
    int B, Hq, Hkv, Hsel, S, D, NQ, NK, block_q, block_kv;
    int Bsel;                 // selection batch: B, or 1 (one selection for every batch entry)
    int causal;
    float scale_log2;         // D^-1/2 * log2(e)
};
// bf16 MFMA path: block_q in {32, 64, 96, 128}, block_kv == 64, D in {64, 128}.
bool attn_mfma_supported(const AttnArgs& a, int bf16);
hipError_t launch_attn_mfma(const AttnArgs& a, hipStream_t stream);
// Decoding: one wave of 32 query rows per workgroup with K read into registers
// (bf16, block_q == 32, block_kv == 64, D in {64, 128}); split rows as above.
bool attn_decode_supported(const AttnArgs& a, int bf16);
hipError_t launch_attn_decode(const AttnArgs& a, hipStream_t stream);
// Merges the nsplit partials of every query row into out (dtype of q) and lse.
hipError_t launch_attn_combine(const AttnArgs& a, int bf16, hipStream_t stream);
// General path (fp32 or bf16 inputs, any block sizes, D in {64, 128}).
hipError_t launch_attn_simt(const AttnArgs& a, int bf16, hipStream_t stream);
// Device address of the library's static split-partial buffer on the current
// device (kDecodeScratchBytes bytes, 256-byte aligned), looked up once per device.
constexpr size_t kDecodeScratchBytes = size_t(16) << 20;
hipError_t decode_scratch(void** ptr);

// ---- attention gradients ---------------------------------------------------

struct AttnBwdArgs {
    const void* q;            // (B, Hq, S, D)
    const void* k;            // (B, Hkv, S, D)
    const void* v;
    const float* lse;         // (B, Hq, S), natural log
    const void* dout;         // (B, Hq, S, D)
    const float* delta;       // (B, Hq, S): dO . O
    void* dq;                 // (B, Hq, S, D)
    void* dk;                 // (B, Hkv, S, D)
    void* dv;
    const int32_t* row_ptr;   // query-major CSR; null = dense
    const int32_t* col_idx;
    const int32_t* col_ptr;   // kv-tile-major index: (B*Hsel*NK + 1); null = dense
    const int32_t* row_idx;   // query tiles per (b, h', j), ascending
    int B, Hq, Hkv, Hsel, S, D, NQ, NK, block_q, block_kv;
    int Bsel;                 // selection batch: B, or 1 (one selection for every batch entry)
    int causal;
    float scale;              // D^-1/2
    float scale_log2;         // D^-1/2 * log2(e)
};
// delta[r] = dout[r] . out[r] over D for `rows` rows (D in {64, 128}).
hipError_t launch_bwd_delta(const void* out, const void* dout, int bf16, int64_t rows, int D, float* delta,
                            hipStream_t stream);
// kv-tile-major index of keep (BH slabs of NQ x NK int8): counts4 (BH*NK*4,
// per column and quarter of the query tiles), col_ptr (BH*NK + 1), sums
// (ceil(BH*NK / 2048) + 1), row_idx (cap entries; offsets are clamped to cap).
hipError_t launch_kv_major_index(const int8_t* keep, int BH, int NQ, int NK, int32_t cap, int32_t* counts4,
                                 int32_t* col_ptr, int32_t* sums, int32_t* row_idx, hipStream_t stream);
// bf16 MFMA path: block_q in {32, 64, 96, 128}, block_kv == 64, D in {64, 128}.
bool attn_bwd_mfma_supported(const AttnBwdArgs& a, int bf16);
hipError_t launch_attn_bwd_mfma(const AttnBwdArgs& a, hipStream_t stream);
// Stage timing: records an event named `name` on `stream` while timing is on
// (nsa_stage_timing_begin / _end), else does nothing.
hipError_t stage_mark(const char* name, hipStream_t stream);
// General path (fp32 or bf16, any block sizes, D in {64, 128}).
hipError_t launch_attn_bwd_simt(const AttnBwdArgs& a, int bf16, hipStream_t stream);

// ---- token reordering --------------------------------------------------------

// y[bh, m] = x[bh, perm[m]] (inverse = 0) or y[bh, perm[m]] = x[bh, m] (inverse = 1)
// for `slabs` slabs of S rows of row_bytes bytes (a multiple of 16, at most 1024).
hipError_t launch_permute_rows(const void* x, const int32_t* perm, int inverse, int64_t slabs, int S,
                               int row_bytes, void* y, hipStream_t stream);

}  // namespace nsa
