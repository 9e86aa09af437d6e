// backward.hip -- lora_backward entry point.
//
// The LoRA gradients of the fine-tuning rows (DeltaServe, section 3.2: the
// backward computes the LoRA gradients from the saved layer input).  For
// y = y0 + s B A x and a given dY:
//   g  = B^T dy                      shrink kernel, weights read transposed
//   v  = A x                         shrink kernel (or the caller's saved v)
//   dX += s A^T g                    expand kernel, weights read transposed
//   dA += s sum g x^T, dB += s sum dy v^T   token-contraction kernel
// The workspace holds g (by sorted position, row- and rank-major), v
// (rank-major), the shrinks' split-K partials and the contraction's partial
// tiles of tiles cut between workgroups.
//
// Launches: the g shrink and its reduce (which also lays out a saved v
// rank-major), then one launch in which the contraction and the dX expand
// run side by side on their own workgroups (both read only g, v and the
// inputs), then the contraction's fix-up of its cut tiles.  Run one after the
// other, the two middle kernels each paid their own ramp-up and tail: 4096
// fine-tuning rows, rank 16, 5120 -> 5120: backward 59.4 against 64.4 us;
// the mixed batch's 2048 rows, 4096 -> 14336: 49.8 against 51.8 us.
//
// For bf16 calls with r_max <= 16 and dY the wider stream (d_out >= 2 d_in)
// the two products that read dY run in one pass over it (dy_pass_kernel: g
// partials and dB); g's partials are summed by the shrink's reduce kernel,
// the contraction computes dA only, and the dB tiles cut between workgroups
// are added in the x-side launch.
#include <algorithm>

#include "host_checks.h"
#include "shrink.h"
#include "expand.h"
#include "contract.h"
#include "bwd_stream.h"

using namespace lora;

namespace lora {
int run_shrink(int dtype, bool trans_w, const ShrinkParams& p, const ReduceParams& rp, int32_t T, int32_t num_adapters,
               hipStream_t st);
int64_t shrink_part_ld(int32_t r_max);
int64_t shrink_part_floats(int dtype, int32_t T, int32_t K, int32_t r_max);
int expand_plan(const ExpandParams& p, int32_t T, int32_t num_adapters, int32_t r_max, ExpandParams* q,
                unsigned* grid);
int launch_shrink_reduce(int32_t r_max, const ReduceParams& rp, int32_t T, int32_t num_adapters, hipStream_t st);

// Contraction workgroups (4 waves each) of the x-side launch: one per CU.
#ifndef LORA_XSIDE_CTR
#define LORA_XSIDE_CTR 256
#endif
constexpr int kXsideCtrGrid = LORA_XSIDE_CTR;
static_assert(kXsideCtrGrid % kNumXcd == 0, "whole rounds of the 8 XCDs");

// Workspace layout of lora_backward (fp32 elements): g by sorted position
// (row-major and rank-major), v rank-major (two-pass path) or by sorted
// position (streaming path, recomputed v), the split-K partials of the shrinks
// or the streaming path's g partials (reused by the passes, which run one
// after the other), and the partial tiles of the stream-K kernels.
struct BwdWs {
    int64_t ldg, ldT;               // pitch of g rows; pitch of the rank-major arrays
    int64_t g, gT, vT, vpos, part, fix, fix_meta, dyfix, dymeta, total; // offsets
    static int32_t dy_slices(int64_t d_out) { return (int32_t)((d_out + kDyCols - 1) / kDyCols); }
    static BwdWs make(int dtype, int64_t T, int64_t d_in, int64_t d_out, int64_t r_max) {
        BwdWs w;
        w.ldg = round_up(r_max, 8);
        w.ldT = round_up(T > 0 ? T : 1, 32);
        w.g = 0;
        w.gT = round_up(w.g + T * w.ldg, 64);
        w.vT = round_up(w.gT + r_max * w.ldT, 64);
        w.vpos = round_up(w.vT + r_max * w.ldT, 64);
        w.part = round_up(w.vpos + T * w.ldg, 64);
        int64_t np = std::max(shrink_part_floats(dtype, (int32_t)T, (int32_t)d_in, (int32_t)r_max),
                              shrink_part_floats(dtype, (int32_t)T, (int32_t)d_out, (int32_t)r_max));
        np = std::max(np, (int64_t)dy_slices(d_out) * (T > 0 ? T : 1) * 16);
        w.fix = round_up(w.part + np, 64);
        w.fix_meta = w.fix + (int64_t)kXsideCtrGrid * 2 * kFixFloats;
        w.dyfix = round_up(w.fix_meta + (int64_t)kXsideCtrGrid * 2 * kFixMeta, 64);
        w.dymeta = w.dyfix + (int64_t)kStGrid * 2 * kDyFixFloats;
        w.total = round_up(w.dymeta + (int64_t)kStGrid * 2 * kStFixMeta, 64);
        return w;
    }
};
}  // namespace lora

namespace {
// The x side of the backward in one launch: the contraction (dA; on the
// two-pass route dA and dB) on the first n_ctr workgroups, dX += s A^T g on
// the next n_expand and (streaming route) the fix-up of the dB tiles cut by
// dy_pass_kernel on the rest.  Each reads only what earlier launches wrote
// (g, v, the dY pass's partial tiles), so the three run side by side instead
// of one after the other; the contraction's own cut tiles are added by
// contract_fixup_kernel in the next launch.  The contraction and the expand
// use one LDS buffer (a workgroup runs one of them).
// (fp32: one workgroup per CU by its LDS, so no register limit for more)
template <int DT, int KS, bool NT>
__global__ __launch_bounds__(4 * kWave) __attribute__((amdgpu_waves_per_eu(DT == LORA_F32 ? 1 : (KS == 4 ? 2 : 3))))
void xside_kernel(ContractParams cp, int n_ctr, ExpandParams ep, int n_expand, DyParams dp) {
    constexpr int kC = ContractLds<DT, 4>::kBytes, kE = ExpandLds<KS>::kBytes;
    __shared__ __attribute__((aligned(16))) char s_lds[kC > kE ? kC : kE];
    const int b = (int)blockIdx.x;
    if (b < n_ctr)
        contract_body<DT, NT, 4>(cp, b, n_ctr, s_lds);
    else if (b < n_ctr + n_expand)
        expand_body<DT, true, KS>(ep, b - n_ctr, n_expand, s_lds);
    else
        dy_fixup_body(dp, b - n_ctr - n_expand);
}

template <int DT, bool NT>
void launch_xside(int ks, const ContractParams& cp, const ExpandParams& ep, const DyParams& dp, unsigned n_expand,
                  unsigned n_dy, hipStream_t st) {
    const dim3 grid(kXsideCtrGrid + n_expand + n_dy), block(4 * kWave);
    if (ks == 1)
        hipLaunchKernelGGL((xside_kernel<DT, 1, NT>), grid, block, 0, st, cp, kXsideCtrGrid, ep, (int)n_expand, dp);
    else if (ks == 2)
        hipLaunchKernelGGL((xside_kernel<DT, 2, NT>), grid, block, 0, st, cp, kXsideCtrGrid, ep, (int)n_expand, dp);
    else
        hipLaunchKernelGGL((xside_kernel<DT, 4, NT>), grid, block, 0, st, cp, kXsideCtrGrid, ep, (int)n_expand, dp);
}
}  // namespace

extern "C" size_t lora_backward_workspace_bytes(int dtype, int32_t T_ft, int32_t d_in, int32_t d_out, int32_t r_max) {
    if (!valid_dtype(dtype) || T_ft < 0 || d_in < 1 || d_out < 1 || r_max < 1 || r_max > LORA_MAX_RANK) return 0;
    return (size_t)BwdWs::make(dtype, T_ft, d_in, d_out, r_max).total * sizeof(float);
}

namespace {

// Backward preemption gate (one thread): status = 1 ("yield") when the grant
// has been withdrawn (*grant == 0) or an earlier gate of the same call has
// already yielded; otherwise 0.  The grant is read with a system-scope load,
// so a flag in host memory mapped for the device, or in device memory updated
// by a copy, is read fresh.
__global__ __launch_bounds__(kWave) void bwd_gate_kernel(const int32_t* grant, int32_t* status, int32_t first) {
    if (threadIdx.x != 0) return;
    const int32_t g = __hip_atomic_load(grant, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    const int32_t before = first ? 0 : __hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(status, (before != 0 || g == 0) ? 1 : 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The streaming pass over dY (dy_pass_kernel) for bf16 calls whose adapters
// all have rank <= 16 and whose dY rows are at least twice as wide as their x
// rows, when its 32-bit buffer offsets cover dY, v and the g partials.  (It
// replaces the g shrink and the dB half of the contraction; measured on one
// MI355X it wins where dY is the dominant stream, e.g. 4096 -> 14336, and
// loses where the two halves are equal, e.g. 5120 -> 5120, to its fixed
// per-workgroup latency.)
bool use_stream_path(int dtype, int32_t T, int64_t lddy, int32_t d_in, int32_t d_out, int32_t r_max,
                     const float* v_saved, int64_t ldv) {
    const int64_t lim = (int64_t)1 << 31;
    return dtype == LORA_BF16 && r_max <= kStMaxRank && d_out >= 2 * (int64_t)d_in && (int64_t)T * lddy * 2 < lim &&
           (int64_t)BwdWs::dy_slices(d_out) * T * 64 < lim && (!v_saved || (int64_t)T * ldv * 4 < lim);
}

int backward_impl(int dtype, const void* x, int64_t ldx, const void* dy, int64_t lddy, void* dx, int64_t lddx,
                  int32_t T_ft, int32_t d_in, int32_t d_out, const lora_adapter* adapters,
                  const lora_adapter_grad* grads, int32_t num_adapters, int32_t r_max, lora_segments seg_ft,
                  const float* v_saved, int64_t ldv, void* ws, size_t ws_bytes, const int32_t* grant,
                  int32_t* status, void* stream) {
    int rc = check_common(dtype, T_ft, num_adapters, r_max, adapters, seg_ft);
    if (rc != LORA_OK) return rc;
    if (d_in < 1 || d_out < 1 || !grads || ((uintptr_t)grads & 7u)) return LORA_ERR_INVALID_ARG;
    if (T_ft == 0) return LORA_OK;
    if ((rc = check_matrix(x, d_in, ldx)) != LORA_OK) return rc;
    if ((rc = check_matrix(dy, d_out, lddy)) != LORA_OK) return rc;
    if (dx && (rc = check_matrix(dx, d_in, lddx)) != LORA_OK) return rc;
    if (v_saved && (rc = check_f32_rows(v_saved, ldv, r_max)) != LORA_OK) return rc;
    if (!seg_ft.offsets) return LORA_ERR_INVALID_ARG;
    const BwdWs w = BwdWs::make(dtype, T_ft, d_in, d_out, r_max);
    if (!ws || !aligned16(ws) || ws_bytes < (size_t)w.total * sizeof(float)) return LORA_ERR_WORKSPACE;

    hipStream_t st = static_cast<hipStream_t>(stream);
    const SchedLayout sl = SchedLayout::make(T_ft, num_adapters);
    float* wsf = static_cast<float*>(ws);
    const bool one_pass = use_stream_path(dtype, T_ft, lddy, d_in, d_out, r_max, v_saved, ldv);
    // Preemption: a gate at the start, and one more after a recompute of v;
    // everything after the last gate (every kernel that writes dA, dB or dX)
    // runs completely or skips its work.
    if (grant) {
        hipLaunchKernelGGL(bwd_gate_kernel, dim3(1), dim3(kWave), 0, st, grant, status, 1);
        if (hipGetLastError() != hipSuccess) return LORA_ERR_HIP;
    }
    const int32_t* stop = grant ? status : nullptr;
    float* g = wsf + w.g;
    float* gT = wsf + w.gT;
    float* vT = wsf + w.vT;
    float* vpos = wsf + w.vpos;

    // Split-K shrink over the rows' sorted positions (g = B^T dy, or v = A x).
    ShrinkParams sp{};
    sp.adapters = adapters;
    sp.r_max = r_max;
    sp.perm = seg_ft.perm;
    sp.sched = seg_ft.sched;
    sp.tiles64_off = sl.tiles64;
    sp.part = wsf + w.part;
    sp.ldp = shrink_part_ld(r_max);
    sp.slice_stride = (int64_t)T_ft * sp.ldp;
    sp.err = seg_ft.err;
    sp.rgroups = rank_groups(r_max);
    sp.stop = stop;
    ReduceParams rp{};
    rp.part = sp.part;
    rp.ldp = sp.ldp;
    rp.slice_stride = sp.slice_stride;
    rp.adapters = adapters;
    rp.r_max = r_max;
    rp.perm = seg_ft.perm;
    rp.sched = seg_ft.sched;
    rp.tiles16_off = sl.tiles16;
    rp.out_by_pos = 1;
    rp.ldT = w.ldT;
    rp.stop = stop;

    // v = A x when the caller did not save it: by sorted position for the
    // one-pass kernel, rank-major for the contraction.
    if (!v_saved) {
        ShrinkParams vp = sp;
        vp.x = x;
        vp.ldx = ldx;
        vp.K = d_in;
        vp.nslices = shrink_slices(dtype, d_in);
        ReduceParams vr = rp;
        vr.nslices = vp.nslices;
        vr.out = one_pass ? vpos : nullptr;
        vr.ldo = w.ldg;
        vr.outT = one_pass ? nullptr : vT;
        if ((rc = run_shrink(dtype, false, vp, vr, T_ft, num_adapters, st)) != LORA_OK) return rc;
        if (grant) {
            hipLaunchKernelGGL(bwd_gate_kernel, dim3(1), dim3(kWave), 0, st, grant, status, 0);
            if (hipGetLastError() != hipSuccess) return LORA_ERR_HIP;
        }
    }

    DyParams dp{};
    if (one_pass) {
        // g partials and dB from one read of dY, then g = the sum of the partials.
        dp.dy = dy;
        dp.lddy = lddy;
        dp.dy_bytes = (uint32_t)(((int64_t)(T_ft - 1) * lddy + d_out) * 2);
        dp.d_out = d_out;
        dp.v = v_saved ? v_saved : vpos;
        dp.ldv = v_saved ? ldv : w.ldg;
        dp.v_bytes = (uint32_t)(((int64_t)(T_ft - 1) * dp.ldv + r_max) * 4);
        dp.v_by_pos = v_saved ? 0 : 1;
        dp.grads = grads;
        dp.perm = seg_ft.perm;
        dp.T = T_ft;
        dp.gpart = wsf + w.part;
        dp.fix = wsf + w.dyfix;
        dp.walk.sched = seg_ft.sched;
        dp.walk.active_off = sl.active;
        dp.walk.adapters = adapters;
        dp.walk.offsets = seg_ft.offsets;
        dp.walk.r_max = r_max;
        dp.walk.nslices = BwdWs::dy_slices(d_out);
        dp.walk.fix_meta = reinterpret_cast<int32_t*>(wsf + w.dymeta);
        dp.gpart_bytes = (uint32_t)((int64_t)dp.walk.nslices * T_ft * 64);
        dp.err = seg_ft.err;
        dp.stop = stop;
        hipLaunchKernelGGL(dy_pass_kernel, dim3(kStGrid), dim3(kStWaves * kWave), 0, st, dp);
        if (hipGetLastError() != hipSuccess) return LORA_ERR_HIP;
        ReduceParams gr = rp;
        gr.part = dp.gpart;
        gr.ldp = 16;
        gr.slice_stride = (int64_t)T_ft * 16;
        gr.nslices = dp.walk.nslices;
        gr.out = g;
        gr.ldo = w.ldg;
        gr.outT = gT;
        if ((rc = launch_shrink_reduce(r_max, gr, T_ft, num_adapters, st)) != LORA_OK) return rc;
    } else {
        // g = B^T dy by the split-K shrink; its reduce also lays out a saved v
        // rank-major for the contraction.
        ShrinkParams gp = sp;
        gp.x = dy;
        gp.ldx = lddy;
        gp.K = d_out;
        gp.nslices = shrink_slices(dtype, d_out);
        ReduceParams gr = rp;
        gr.nslices = gp.nslices;
        gr.out = g;
        gr.ldo = w.ldg;
        gr.outT = gT;
        if (v_saved) {
            gr.vsrc = v_saved;
            gr.ldvsrc = ldv;
            gr.vT = vT;
        }
        if ((rc = run_shrink(dtype, true, gp, gr, T_ft, num_adapters, st)) != LORA_OK) return rc;
    }

    // dA += s g^T x (and, on the two-pass path, dB += s dy^T v).
    ContractParams cp{};
    cp.x = x;
    cp.ldx = ldx;
    cp.dy = dy;
    cp.lddy = lddy;
    cp.gT = gT;
    cp.vT = vT;
    cp.ldT = w.ldT;
    cp.adapters = adapters;
    cp.grads = grads;
    cp.r_max = r_max;
    cp.offsets = seg_ft.offsets;
    cp.perm = seg_ft.perm;
    cp.sched = seg_ft.sched;
    cp.active_off = sl.active;
    cp.d_in = d_in;
    cp.d_out = d_out;
    cp.ncb_in = (d_in + 63) / 64;
    cp.ncb_out = one_pass ? 0 : (d_out + 63) / 64;
    cp.rgroups = (r_max + 16 * kContractMB - 1) / (16 * kContractMB);
    cp.err = seg_ft.err;
    cp.fix = wsf + w.fix;
    cp.fix_meta = reinterpret_cast<int32_t*>(wsf + w.fix_meta);
    cp.stop = stop;
    // dX += s A^T g, the contraction and the dB fix-up in one launch, then the
    // contraction's fix-up.
    const unsigned n_dy = one_pass ? kStGrid * kDyFixParts : 0;
    ExpandParams q{};
    unsigned n_expand = 0;
    int ks = 1;
    if (dx) {
        ExpandParams ep{};
        ep.v = g;
        ep.ldv = w.ldg;
        ep.v_by_pos = 1;
        ep.adapters = adapters;
        ep.r_max = r_max;
        ep.perm = seg_ft.perm;
        ep.sched = seg_ft.sched;
        ep.y = dx;
        ep.ldy = lddx;
        ep.N = d_in;
        ep.err = seg_ft.err;
        ep.stop = stop;
        ks = expand_plan(ep, T_ft, num_adapters, r_max, &q, &n_expand);
    }
    if (dtype == LORA_BF16 && !one_pass)
        launch_xside<LORA_BF16, true>(ks, cp, q, dp, n_expand, n_dy, st);
    else if (dtype == LORA_BF16)
        launch_xside<LORA_BF16, false>(ks, cp, q, dp, n_expand, n_dy, st);
    else
        launch_xside<LORA_F32, false>(ks, cp, q, dp, n_expand, n_dy, st);
    if (hipGetLastError() != hipSuccess) return LORA_ERR_HIP;
    hipLaunchKernelGGL(contract_fixup_kernel, dim3(kXsideCtrGrid), dim3(4 * kWave), 0, st, cp, (int)kXsideCtrGrid);
    return hipGetLastError() == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

}  // namespace

extern "C" int lora_backward(int dtype, const void* x, int64_t ldx, const void* dy, int64_t lddy, void* dx,
                             int64_t lddx, int32_t T_ft, int32_t d_in, int32_t d_out, const lora_adapter* adapters,
                             const lora_adapter_grad* grads, int32_t num_adapters, int32_t r_max,
                             lora_segments seg_ft, const float* v_saved, int64_t ldv, void* ws, size_t ws_bytes,
                             void* stream) {
    return backward_impl(dtype, x, ldx, dy, lddy, dx, lddx, T_ft, d_in, d_out, adapters, grads, num_adapters, r_max,
                         seg_ft, v_saved, ldv, ws, ws_bytes, nullptr, nullptr, stream);
}

extern "C" int lora_backward_preemptible(int dtype, const void* x, int64_t ldx, const void* dy, int64_t lddy,
                                         void* dx, int64_t lddx, int32_t T_ft, int32_t d_in, int32_t d_out,
                                         const lora_adapter* adapters, const lora_adapter_grad* grads,
                                         int32_t num_adapters, int32_t r_max, lora_segments seg_ft,
                                         const float* v_saved, int64_t ldv, void* ws, size_t ws_bytes,
                                         const int32_t* grant, int32_t* status, void* stream) {
    if (!grant || !status || ((uintptr_t)grant & 3u) || ((uintptr_t)status & 3u)) return LORA_ERR_INVALID_ARG;
    return backward_impl(dtype, x, ldx, dy, lddy, dx, lddx, T_ft, d_in, d_out, adapters, grads, num_adapters, r_max,
                         seg_ft, v_saved, ldv, ws, ws_bytes, grant, status, stream);
}
