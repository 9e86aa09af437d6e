// forward.hip -- lora_shrink and lora_expand_add entry points.
//
// The forward of one LoRA layer over a mixed batch: v = A_a x (shrink), then
// y += s_a B_a v (expand-add), for every row with an adapter (MOLT section 2.1,
// h(x) = W x + B A x; DeltaServe section 2.2, multi-LoRA batching).  Both
// kernels are MFMA tiles over the rows of one adapter at a time, walking the
// tile records of lora_segments_build.
#include "host_checks.h"
#include "lora_kernels.h"

using namespace lora;

namespace {

constexpr int64_t kMaxGrid = 8192;

template <int DT>
int launch_shrink_t(bool trans_w, const ShrinkParams& p, unsigned grid, hipStream_t st) {
    if (trans_w)
        hipLaunchKernelGGL((shrink_kernel<DT, true>), dim3(grid), dim3(kShrinkThreads), 0, st, p);
    else
        hipLaunchKernelGGL((shrink_kernel<DT, false>), dim3(grid), dim3(kShrinkThreads), 0, st, p);
    return hipGetLastError() == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

template <int DT, bool TRANS_W>
int launch_expand_t(int ks, const ExpandParams& p, unsigned grid, hipStream_t st) {
    const dim3 block(kExpandWaves * kWave);
    if (ks == 1)
        hipLaunchKernelGGL((expand_kernel<DT, TRANS_W, 1>), dim3(grid), block, 0, st, p);
    else if (ks == 2)
        hipLaunchKernelGGL((expand_kernel<DT, TRANS_W, 2>), dim3(grid), block, 0, st, p);
    else
        hipLaunchKernelGGL((expand_kernel<DT, TRANS_W, 4>), dim3(grid), block, 0, st, p);
    return hipGetLastError() == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

}  // namespace

namespace lora {

// Shared by the forward and the backward (declared in backward.hip).
int run_shrink(int dtype, bool trans_w, const ShrinkParams& p, int32_t T, int32_t num_adapters, hipStream_t st) {
    const int64_t tasks = SchedLayout::max_tiles16(T, num_adapters) * p.rgroups;
    const unsigned grid = grid_for(tasks, 1, kMaxGrid);
    return dtype == LORA_BF16 ? launch_shrink_t<LORA_BF16>(trans_w, p, grid, st)
                              : launch_shrink_t<LORA_F32>(trans_w, p, grid, st);
}

int run_expand(int dtype, bool trans_w, const ExpandParams& p, int32_t T, int32_t num_adapters, int32_t r_max,
               hipStream_t st) {
    const int ks = r_max <= 32 ? 1 : (r_max <= 64 ? 2 : 4);
    const int64_t tasks = SchedLayout::max_tiles64(T, num_adapters) * ((p.N + kExpandCols - 1) / kExpandCols);
    const unsigned grid = grid_for(tasks, 1, kMaxGrid);
    if (dtype == LORA_BF16)
        return trans_w ? launch_expand_t<LORA_BF16, true>(ks, p, grid, st)
                       : launch_expand_t<LORA_BF16, false>(ks, p, grid, st);
    return trans_w ? launch_expand_t<LORA_F32, true>(ks, p, grid, st)
                   : launch_expand_t<LORA_F32, false>(ks, p, grid, st);
}

}  // namespace lora

extern "C" int lora_shrink(int dtype, const void* x, int64_t ldx, int32_t T, int32_t d_in,
                           const lora_adapter* adapters, int32_t num_adapters, int32_t r_max, lora_segments seg,
                           float* v, int64_t ldv, void* stream) {
    int rc = check_common(dtype, T, num_adapters, r_max, adapters, seg);
    if (rc != LORA_OK) return rc;
    if (d_in < 1) return LORA_ERR_INVALID_ARG;
    if (T == 0) return LORA_OK;
    if ((rc = check_matrix(x, d_in, ldx)) != LORA_OK) return rc;
    if ((rc = check_f32_rows(v, ldv, r_max)) != LORA_OK) return rc;
    const SchedLayout sl = SchedLayout::make(T, num_adapters);
    ShrinkParams p{};
    p.x = x;
    p.ldx = ldx;
    p.K = d_in;
    p.adapters = adapters;
    p.r_max = r_max;
    p.perm = seg.perm;
    p.sched = seg.sched;
    p.tiles16_off = sl.tiles16;
    p.out = v;
    p.ldo = ldv;
    p.out_by_pos = 0;
    p.outT = nullptr;
    p.ldT = 0;
    p.err = seg.err;
    p.rgroups = rank_groups(r_max);
    return run_shrink(dtype, false, p, T, num_adapters, static_cast<hipStream_t>(stream));
}

extern "C" int lora_expand_add(int dtype, const float* v, int64_t ldv, int32_t T, int32_t d_out,
                               const lora_adapter* adapters, int32_t num_adapters, int32_t r_max, lora_segments seg,
                               void* y, int64_t ldy, void* stream) {
    int rc = check_common(dtype, T, num_adapters, r_max, adapters, seg);
    if (rc != LORA_OK) return rc;
    if (d_out < 1) return LORA_ERR_INVALID_ARG;
    if (T == 0) return LORA_OK;
    if ((rc = check_matrix(y, d_out, ldy)) != LORA_OK) return rc;
    if ((rc = check_f32_rows(v, ldv, r_max)) != LORA_OK) return rc;
    const SchedLayout sl = SchedLayout::make(T, num_adapters);
    ExpandParams p{};
    p.v = v;
    p.ldv = ldv;
    p.v_by_pos = 0;
    p.adapters = adapters;
    p.r_max = r_max;
    p.perm = seg.perm;
    p.sched = seg.sched;
    p.tiles64_off = sl.tiles64;
    p.y = y;
    p.ldy = ldy;
    p.N = d_out;
    p.err = seg.err;
    return run_expand(dtype, false, p, T, num_adapters, r_max, static_cast<hipStream_t>(stream));
}
