// fused.hip -- one-launch forward (lora_forward) and its multi-slice form
// (lora_forward_multi) on gfx950.  The kernel is in fused.h.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "fused.h"
#include "fused_decode.h"
#include "host_checks.h"
#include "lora_batch.h"

using namespace lora;

namespace lora {
// forward.hip: the 16-row-tile shrink (needs no workspace)
int run_dec_shrink(int dtype, const void* x, int64_t ldx, int32_t T, int32_t d_in, const lora_adapter* adapters,
                   int32_t num_adapters, int32_t r_max, const lora_segments& seg, float* v, int64_t ldv,
                   int32_t v_by_pos, hipStream_t st);
}  // namespace lora

namespace {

constexpr int64_t kFusedMaxGrid = 8192;
constexpr int64_t kNumCus = 256;  // MI355X compute units

template <int DT, int S>
void launch_fused(int nmb, const FusedParams& p, unsigned grid, hipStream_t st) {
    const dim3 block(kFusedThreads);
    if (nmb == 1) {
        hipLaunchKernelGGL((fused_forward_kernel<DT, 1, 1, S>), dim3(grid), block, 0, st, p);
    } else if (nmb == 2) {
        hipLaunchKernelGGL((fused_forward_kernel<DT, 1, 2, S>), dim3(grid), block, 0, st, p);
    } else if (nmb == 4) {
        hipLaunchKernelGGL((fused_forward_kernel<DT, 2, 4, S>), dim3(grid), block, 0, st, p);
    } else {
        if constexpr (S == 1) hipLaunchKernelGGL((fused_forward_kernel<DT, 4, 8, 1>), dim3(grid), block, 0, st, p);
    }
}

template <int DT>
void launch_fused_s(int n_slices, int nmb, const FusedParams& p, unsigned grid, hipStream_t st) {
    if (n_slices == 1)
        launch_fused<DT, 1>(nmb, p, grid, st);
    else if (n_slices == 2)
        launch_fused<DT, 2>(nmb, p, grid, st);
    else
        launch_fused<DT, 3>(nmb, p, grid, st);
}

static_assert(LORA_MAX_SLICES <= kFdMaxSlices && LORA_MAX_SLICES <= kFusedMaxSlices, "slices per launch");

// Column ranges per tile of the decode kernel (0: from the batch's bounds).
#ifndef LORA_FD_NSPLIT
#define LORA_FD_NSPLIT 0
#endif

// Decode batches (at most 32 rows per adapter on average) of rank <= 16
// adapters take fused_decode_kernel: enough column ranges per tile for about
// one 16-wave workgroup per CU, at least 16 output chunks per range.
bool fused_decode_fits(int dtype, int32_t T, int32_t num_adapters, int32_t r_max) {
    return r_max <= kFdMaxRank && use_decode_path(dtype, T, num_adapters);
}

int fused_decode_run(const void* x, int64_t ldx, int32_t T, int32_t d_in, const lora_slice* slices, int32_t n_slices,
                     int32_t num_adapters, int32_t r_max, const lora_segments& seg, hipStream_t st) {
    FdParams p{};
    p.x = x;
    p.ldx = ldx;
    p.x_bytes = (uint32_t)(((int64_t)(T - 1) * ldx + d_in) * 2);
    p.K = d_in;
    p.r_max = r_max;
    p.perm = seg.perm;
    p.sched = seg.sched;
    p.tiles16_off = SchedLayout::make(T, num_adapters).tiles16;
    const int64_t max_tiles = SchedLayout::max_tiles16(T, num_adapters);
    p.max_tiles = (int32_t)max_tiles;
    int64_t nch = 0;
    for (int32_t q = 0; q < n_slices; ++q) {
        const lora_slice& sl = slices[q];
        p.sl[q] = FdSlice{sl.adapters, sl.y, sl.ldy, (uint32_t)(((int64_t)(T - 1) * sl.ldy + sl.d_out) * 2),
                          sl.d_out, sl.v, sl.ldv, (int32_t)nch};
        nch += (sl.d_out + kFdChunk - 1) / kFdChunk;
    }
    p.nch = (int32_t)nch;
    const int64_t ns = LORA_FD_NSPLIT > 0 ? LORA_FD_NSPLIT
                                          : std::min<int64_t>((kNumCus + max_tiles - 1) / max_tiles, nch / kFdWaves);
    p.nsplit = (int32_t)std::max<int64_t>(1, std::min<int64_t>(ns, nch));
    if (nch * (p.nsplit + 1) > 0x7fffffff) return LORA_ERR_UNSUPPORTED;
    p.err = seg.err;
    // tile t -> XCD t % 8: 8 x nsplit workgroups per 8 tiles
    const int64_t grid = kNumXcd * p.nsplit * ((max_tiles + kNumXcd - 1) / kNumXcd);
    if (grid > 0x7fffffff) return LORA_ERR_UNSUPPORTED;
    const dim3 g((unsigned)grid), block(kFdThreads);
    if (n_slices == 1)
        hipLaunchKernelGGL(fused_decode_kernel<1>, g, block, 0, st, p);
    else if (n_slices == 2)
        hipLaunchKernelGGL(fused_decode_kernel<2>, g, block, 0, st, p);
    else
        hipLaunchKernelGGL(fused_decode_kernel<3>, g, block, 0, st, p);
    return hipGetLastError() == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

int fused_run(int dtype, const void* x, int64_t ldx, int32_t T, int32_t d_in, const lora_slice* slices,
              int32_t n_slices, int32_t num_adapters, int32_t r_max, const lora_segments& seg, void* stream) {
    if (n_slices < 1 || n_slices > LORA_MAX_SLICES || !slices) return LORA_ERR_INVALID_ARG;
    int rc = check_common(dtype, T, num_adapters, r_max, slices[0].adapters, seg);
    if (rc != LORA_OK) return rc;
    if (d_in < 1) return LORA_ERR_INVALID_ARG;
    for (int32_t q = 0; q < n_slices; ++q) {
        const lora_slice& sl = slices[q];
        if (!sl.adapters || ((uintptr_t)sl.adapters & 7u) || sl.d_out < 1 || sl.reserved != 0)
            return LORA_ERR_INVALID_ARG;
    }
    // the LDS of several slices' v rows and fragments fits up to rank 64
    if (n_slices > 1 && r_max > 64) return LORA_ERR_UNSUPPORTED;
    if (T == 0) return LORA_OK;
    if ((rc = check_matrix(x, d_in, ldx)) != LORA_OK) return rc;
    for (int32_t q = 0; q < n_slices; ++q) {
        const lora_slice& sl = slices[q];
        if ((rc = check_matrix(sl.y, sl.d_out, sl.ldy)) != LORA_OK) return rc;
        if (sl.v && (rc = check_f32_rows(sl.v, sl.ldv, r_max)) != LORA_OK) return rc;
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    bool dec = fused_decode_fits(dtype, T, num_adapters, r_max) && dec_offsets_fit((int64_t)T * ldx * 2, d_in, r_max);
    for (int32_t q = 0; q < n_slices; ++q)
        dec = dec && dec_offsets_fit((int64_t)T * slices[q].ldy * 2, slices[q].d_out, r_max);
    if (dec) return fused_decode_run(x, ldx, T, d_in, slices, n_slices, num_adapters, r_max, seg, st);
    // Slices with v given: where the split kernels need no workspace -- the
    // 16-row-tile shrink on decode batches or at r_max <= 16, then the expand
    // -- they are faster than the 64-row-tile kernel, which walks all of d_in
    // per tile; such a slice runs them (v passes through HBM, results as
    // lora_shrink + lora_expand_add bit for bit), the others the one-launch
    // kernel below.
    lora_slice rest[LORA_MAX_SLICES];
    if ((use_decode_path(dtype, T, num_adapters) || (dtype == LORA_BF16 && r_max <= 16)) &&
        dec_offsets_fit((int64_t)T * ldx * 2, d_in, r_max)) {
        int32_t n_rest = 0;
        for (int32_t q = 0; q < n_slices; ++q) {
            const lora_slice& sl = slices[q];
            if (!sl.v) {
                rest[n_rest++] = sl;
                continue;
            }
            rc = run_dec_shrink(dtype, x, ldx, T, d_in, sl.adapters, num_adapters, r_max, seg, sl.v, sl.ldv, 0, st);
            if (rc != LORA_OK) return rc;
            rc = lora_expand_add(dtype, sl.v, sl.ldv, T, sl.d_out, sl.adapters, num_adapters, r_max, seg, sl.y,
                                 sl.ldy, stream);
            if (rc != LORA_OK) return rc;
        }
        if (n_rest == 0) return LORA_OK;
        slices = rest;
        n_slices = n_rest;
    }
    FusedParams p{};
    int64_t nch = 0;
    for (int32_t q = 0; q < n_slices; ++q) {
        const lora_slice& sl = slices[q];
        p.sl[q] = FusedSlice{sl.adapters, sl.y, sl.ldy, sl.v, sl.ldv, sl.d_out, (int32_t)nch};
        nch += (sl.d_out + 63) / 64;
    }
    if (nch > 0x7fffffff) return LORA_ERR_UNSUPPORTED;
    p.x = x;
    p.ldx = ldx;
    p.K = d_in;
    p.r_max = r_max;
    p.perm = seg.perm;
    p.sched = seg.sched;
    p.tiles64_off = SchedLayout::make(T, num_adapters).tiles64;
    p.nch = (int32_t)nch;
    p.err = seg.err;
    // column ranges per tile: enough tasks for one per CU (each range
    // recomputes v; at most one range per eight 64-column chunks)
    const int64_t max_tiles = SchedLayout::max_tiles64(T, num_adapters);
    p.nsplit = (int32_t)std::max<int64_t>(1, std::min<int64_t>(kNumCus / max_tiles, std::max<int64_t>(1, nch / 8)));
    const unsigned grid = grid_for(max_tiles * p.nsplit, 1, kFusedMaxGrid);
    // 16-rank blocks of phase 1: 1 (r_max <= 16), 2, 4 or 8
    const int nmb = r_max <= 16 ? 1 : (r_max <= 32 ? 2 : (r_max <= 64 ? 4 : 8));
    if (dtype == LORA_BF16)
        launch_fused_s<LORA_BF16>(n_slices, nmb, p, grid, st);
    else
        launch_fused_s<LORA_F32>(n_slices, nmb, p, grid, st);
    return hipGetLastError() == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

}  // namespace

extern "C" int lora_forward(int dtype, const void* x, int64_t ldx, int32_t T, int32_t d_in, int32_t d_out,
                            const lora_adapter* adapters, int32_t num_adapters, int32_t r_max, lora_segments seg,
                            void* y, int64_t ldy, float* v, int64_t ldv, void* stream) {
    const lora_slice one{adapters, y, ldy, v, ldv, d_out, 0};
    return fused_run(dtype, x, ldx, T, d_in, &one, 1, num_adapters, r_max, seg, stream);
}

extern "C" int lora_forward_multi(int dtype, const void* x, int64_t ldx, int32_t T, int32_t d_in,
                                  const lora_slice* slices, int32_t n_slices, int32_t num_adapters, int32_t r_max,
                                  lora_segments seg, void* stream) {
    return fused_run(dtype, x, ldx, T, d_in, slices, n_slices, num_adapters, r_max, seg, stream);
}
