// Token reordering for gfx950: gather / scatter of whole token rows by a
// permutation, so that tokens of an image or video grid can be laid out along a
// space-filling curve once before a series of attention calls (the thread
// "Optimal ordering with block mask": ordering by small patches, Morton or
// Hilbert curves, leaves fewer non-empty blocks for a local pattern).
//
// y[bh, m, :] = x[bh, perm[m], :]   (apply)
// y[bh, perm[m], :] = x[bh, m, :]   (undo)
//
// Each token row (D elements) is moved by LPR lanes with 16-byte loads and
// stores; one 256-thread workgroup moves 256 / LPR rows of one (b, h) slab.
// Rows whose permutation entry is outside [0, S) are skipped.
#include "nsa_internal.h"

namespace nsa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int LPR>
__global__ __launch_bounds__(256) void permute_rows_kernel(const u32x4* x, const int32_t* perm, int inverse,
                                                           int64_t slabs, int S, u32x4* y) {
    constexpr int RPB = 256 / LPR;  // rows per block
    const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
    const int part = threadIdx.x % LPR;
    const int64_t total = slabs * S;
    if (row >= total) return;
    const int64_t bh = row / S;
    const int m = (int)(row % S);
    const int p = perm[m];
    if (p < 0 || p >= S) return;
    const int64_t src = inverse ? row : bh * S + p;
    const int64_t dst = inverse ? bh * S + p : row;
    y[dst * LPR + part] = __builtin_nontemporal_load(x + src * LPR + part);
}

}  // namespace

hipError_t launch_permute_rows(const void* x, const int32_t* perm, int inverse, int64_t slabs, int S,
                               int row_bytes, void* y, hipStream_t stream) {
    const int64_t rows = slabs * S;
    if (rows == 0) return hipSuccess;
    const int lpr = row_bytes / 16;
#define NSA_PERM(L)                                                                                           \
    hipLaunchKernelGGL((permute_rows_kernel<L>), dim3((unsigned)((rows + (256 / L) - 1) / (256 / L))),      \
                       dim3(256), 0, stream, (const u32x4*)x, perm, inverse, slabs, S, (u32x4*)y)
    switch (lpr) {
        case 4: NSA_PERM(4); break;
        case 8: NSA_PERM(8); break;
        case 16: NSA_PERM(16); break;
        case 32: NSA_PERM(32); break;
        case 64: NSA_PERM(64); break;
        default: return hipErrorInvalidValue;
    }
#undef NSA_PERM
    return hipGetLastError();
}

}  // namespace nsa
