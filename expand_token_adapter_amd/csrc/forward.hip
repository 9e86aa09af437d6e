// forward.hip -- lora_shrink and lora_expand_add entry points.
//
// The forward of one LoRA layer over a mixed batch: v = A_a x (shrink), then
// y += s_a B_a v (expand-add), for every row with an adapter (MOLT section 2.1,
// h(x) = W x + B A x; DeltaServe section 2.2, multi-LoRA batching).  Both
// kernels are MFMA tiles over the rows of one adapter at a time, walking the
// tile records of lora_segments_build.
#include <algorithm>

#include "host_checks.h"
#include "shrink.h"
#include "expand.h"
#include "decode.h"


using namespace lora;

namespace {

constexpr int64_t kMaxGrid = 8192;
// Split-K shrink: at most two workgroups per CU, the number the 64-rank
// variant's LDS keeps resident (mixed batch: 28.6 us at 512 workgroups, 29.8
// at 1024, 30.4 at 768, 31.8 at 2048).
constexpr int64_t kShrinkMaxGrid = 512;

template <int DT, int RB>
void launch_shrink_rb(bool trans_w, const ShrinkParams& p, unsigned grid, hipStream_t st) {
    if (trans_w)
        hipLaunchKernelGGL((shrink_kernel<DT, true, RB>), dim3(grid), dim3(kShrinkThreads), 0, st, p);
    else
        hipLaunchKernelGGL((shrink_kernel<DT, false, RB>), dim3(grid), dim3(kShrinkThreads), 0, st, p);
}

// 16-rank blocks per task: 1 (r_max <= 16), 2 (<= 32), else 4 (64-rank groups)
template <int DT>
int launch_shrink_t(bool trans_w, const ShrinkParams& p, unsigned grid, hipStream_t st) {
    if (p.r_max <= 16)
        launch_shrink_rb<DT, 1>(trans_w, p, grid, st);
    else if (p.r_max <= 32)
        launch_shrink_rb<DT, 2>(trans_w, p, grid, st);
    else
        launch_shrink_rb<DT, 4>(trans_w, p, grid, st);
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

// One task per workgroup up to this many tasks: the hardware dispatcher then
// hands out tasks of very different sizes (and the empty ones) as slots free
// up, instead of each workgroup walking a fixed share.
constexpr int64_t kDecShrinkMaxGrid = 1 << 16;

// Balanced mode: at least this many tasks (bound from the row and adapter
// counts), on a grid of two 4-wave workgroups per CU, all resident at once.
// Measured on the zipf-320 decode batch (2048 rows, 8192 -> 8192): two per CU
// 65.8 us; four per CU (at most three resident, the rest started late) 71.8;
// three 72.9; one 73.7; 1.5 or 2.5 per CU (CUs unevenly loaded) 83.8 / 73.7.
// With more workgroups in flight the memory system serves the same 1 KB row
// pieces more slowly; with fewer, too few loads are in flight.
constexpr int64_t kDecShrinkPlanTasks = 2048;
constexpr unsigned kDecShrinkPlanGrid = 256 * 2;
static_assert(kDecShrinkPlanGrid % kNumXcd == 0, "balanced ranges are numbered XCD by XCD");

template <int DT>
void launch_dec_shrink(const DecShrinkParams& p, int64_t tasks, hipStream_t st) {
    if (p.balanced) {
        hipLaunchKernelGGL((dec_shrink_kernel<DT, 4>), dim3(kDecShrinkPlanGrid), dim3(4 * kWave), 0, st, p);
        return;
    }
    const unsigned grid = grid_for(tasks, 1, kDecShrinkMaxGrid);
    // few tasks: more waves per workgroup (each takes a shorter run of d_in)
    if (tasks < 512)
        hipLaunchKernelGGL((dec_shrink_kernel<DT, 16>), dim3(grid), dim3(16 * kWave), 0, st, p);
    else if (tasks < 1024)
        hipLaunchKernelGGL((dec_shrink_kernel<DT, 8>), dim3(grid), dim3(8 * kWave), 0, st, p);
    else
        hipLaunchKernelGGL((dec_shrink_kernel<DT, 4>), dim3(grid), dim3(4 * kWave), 0, st, p);
}

}  // namespace

namespace lora {


// v = A x on 16-row tiles (decode.h), written straight to v.
int run_dec_shrink(int dtype, const void* x, int64_t ldx, int32_t T, int32_t d_in, const lora_adapter* adapters,
                   int32_t num_adapters, int32_t r_max, const lora_segments& seg, float* v, int64_t ldv,
                   int32_t v_by_pos, hipStream_t st) {
    DecShrinkParams p{};
    p.x = x;
    p.ldx = ldx;
    p.x_bytes = (uint32_t)(((int64_t)(T - 1) * ldx + d_in) * 2);
    p.K = d_in;
    p.adapters = adapters;
    p.r_max = r_max;
    p.perm = seg.perm;
    p.sched = seg.sched;
    p.tiles16_off = SchedLayout::make(T, num_adapters).tiles16;
    p.v = v;
    p.ldv = ldv;
    p.v_by_pos = v_by_pos;
    p.rblocks = (r_max + 15) / 16;
    p.err = seg.err;
    const int64_t tiles = SchedLayout::max_tiles16(T, num_adapters);
    const int64_t tasks = tiles * p.rblocks;
    p.balanced = tasks >= kDecShrinkPlanTasks && tiles <= kShrPlanMaxTiles;
    if (dtype != LORA_BF16) return LORA_ERR_UNSUPPORTED;
    launch_dec_shrink<LORA_BF16>(p, tasks, st);
    return hipGetLastError() == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

// y += s B v on 16-row tiles (decode.h): one launch of a fixed grid, each
// workgroup a byte-balanced share of the (tile, chunk) units.
constexpr int kDecExpandGrid = 256 * 3;  // three workgroups per CU (the kernel's occupancy)
static_assert(kDecExpandGrid % kNumXcd == 0, "balanced ranges are numbered XCD by XCD");

int run_dec_expand(int dtype, const float* v, int64_t ldv, int32_t v_by_pos, int32_t T, int32_t d_out,
                   const lora_adapter* adapters, int32_t num_adapters, int32_t r_max, const lora_segments& seg,
                   void* y, int64_t ldy, hipStream_t st) {
    if (dtype != LORA_BF16) return LORA_ERR_UNSUPPORTED;
    DecExpandParams p{};
    p.v = v;
    p.ldv = ldv;
    p.v_by_pos = v_by_pos;
    p.adapters = adapters;
    p.r_max = r_max;
    p.perm = seg.perm;
    p.sched = seg.sched;
    p.tiles16_off = SchedLayout::make(T, num_adapters).tiles16;
    p.y = y;
    p.ldy = ldy;
    p.y_bytes = (uint32_t)(((int64_t)(T - 1) * ldy + d_out) * 2);
    p.N = d_out;
    p.err = seg.err;
    // small batches (or more tiles than the plan holds): one tile slice per
    // workgroup; otherwise a fixed grid with byte-balanced ranges
    const int64_t nch = (d_out + kDecChunk - 1) / kDecChunk;
    const int64_t tiles = SchedLayout::max_tiles16(T, num_adapters);
    p.balanced = tiles * nch > 8192 && tiles <= kPlanMaxTiles;
    const unsigned grid = p.balanced ? (unsigned)kDecExpandGrid
                                     : grid_for(tiles * ((nch + kDirectChunks - 1) / kDirectChunks), 1, INT32_MAX);
    hipLaunchKernelGGL(dec_expand_kernel<LORA_BF16>, dim3(grid), dim3(kDecExpWaves * kWave), 0, st, p);
    return hipGetLastError() == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

// Fixed-order sum of the K-slice partials of one 16-row tile per workgroup.
// Lane (n, q) = (lane % 16, lane / 16) holds ranks 16 j + 4 q .. + 3 of row
// n; wave w sums the slices [w ns / 4, (w + 1) ns / 4) in slice order with
// all its loads in flight, and wave 0 adds the four wave sums in wave order,
// so the result does not depend on timing.
constexpr int kReduceWaves = 4;

// NJ: 16-rank blocks covered (16 NJ >= r_max).  Every partial is loaded
// unconditionally (quads at or past r read quad 0 of the row, which exists,
// and are dropped where they are added): conditional loads are waited for one
// at a time, these are all in flight together.
template <int NJ>
__global__ __launch_bounds__(kReduceWaves * kWave) void shrink_reduce_kernel(ReduceParams p) {
    __shared__ f32x4_t s_acc[kReduceWaves - 1][NJ][kWave];
    if (p.stop && *p.stop) return;
    const int wave = wave_id();
    const int lane = threadIdx.x & (kWave - 1);
    const int n = lane & 15;
    const int q = lane >> 4;
    const int64_t ntiles = p.sched[0];
    const int s0 = wave * p.nslices / kReduceWaves;
    const int s1 = (wave + 1) * p.nslices / kReduceWaves;
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const TileRec rec = load_tile(p.sched, p.tiles16_off, tile);
        const lora_adapter ad = load_adapter(p.adapters, rec.adapter);
        if (!adapter_ok(ad, p.r_max)) continue;  // bad entries are counted by the shrink
        const int r = ad.rank;
        const int nj = (r + 15) / 16;
        const bool row_ok = n < rec.rows;
        const int pos = rec.pos0 + (row_ok ? n : 0);
        const int64_t orow = wave == 0 && p.out && !p.out_by_pos ? p.perm[pos] : pos;
        const int64_t vrow = wave == 1 && p.vsrc ? p.perm[pos] : 0;
        const float* src = p.part + (int64_t)pos * p.ldp;
        bool qok[NJ];
        int qoff[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            qok[j] = 16 * j + 4 * q < r;
            qoff[j] = qok[j] ? 16 * j + 4 * q : 0;
        }
        f32x4_t acc[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll(NJ <= 4 ? 2 : 1)
        for (int sl = s0; sl < s1; ++sl) {
            f32x4_t part[NJ];
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                part[j] = *gptr(reinterpret_cast<const f32x4_t*>(src + (int64_t)sl * p.slice_stride + qoff[j]));
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                if (qok[j]) acc[j] += part[j];
        }
        if (wave > 0) {
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                if (j < nj) s_acc[wave - 1][j][lane] = acc[j];
        }
        lds_barrier();
        if (wave == 1 && p.vsrc && row_ok) {
            // rank-major copy of the caller's v rows of this tile (quads below
            // round_up(r, 4) <= the caller's pitch)
            f32x4_t vv[NJ];
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                vv[j] = *gptr(reinterpret_cast<const f32x4_t*>(p.vsrc + vrow * p.ldvsrc + qoff[j]));
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int k = 16 * j + 4 * q;
                if (qok[j]) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (k + i < r) gptr(p.vT)[(int64_t)(k + i) * p.ldT + pos] = vv[j][i];
                }
            }
        }
        if (wave == 0 && row_ok) {
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                if (j < nj) {
                    f32x4_t sum = acc[j];
#pragma unroll
                    for (int w = 0; w < kReduceWaves - 1; ++w) sum += s_acc[w][j][lane];
                    const int k = 16 * j + 4 * q;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (k + i >= r) sum[i] = 0.f;
                    // quads below round_up(r, 8) <= round_up(r_max, 8) <= ldo
                    if (p.out && k < (r + 7) / 8 * 8)
                        *gptr(reinterpret_cast<f32x4_t*>(p.out + orow * p.ldo + k)) = sum;
                    if (p.outT) {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (k + i < r) gptr(p.outT)[(int64_t)(k + i) * p.ldT + pos] = sum[i];
                    }
                }
            }
        }
        lds_barrier();  // s_acc is reused by the next tile
    }
}

int launch_shrink_reduce(int32_t r_max, const ReduceParams& rp, int32_t T, int32_t num_adapters, hipStream_t st);

// Shared by the forward and the backward (declared in backward.hip): the
// split-K shrink into partials, then their fixed-order sum.
int run_shrink(int dtype, bool trans_w, const ShrinkParams& p, const ReduceParams& rp, int32_t T, int32_t num_adapters,
               hipStream_t st) {
    // at most two workgroups per CU: the later tasks of a workgroup overlap
    // their metadata loads with the current task's data
    const int64_t tasks = SchedLayout::max_tiles64(T, num_adapters) * p.rgroups * p.nslices;
    const unsigned grid = grid_for(tasks, 1, kShrinkMaxGrid);
    const int rc = dtype == LORA_BF16 ? launch_shrink_t<LORA_BF16>(trans_w, p, grid, st)
                                      : launch_shrink_t<LORA_F32>(trans_w, p, grid, st);
    if (rc != LORA_OK) return rc;
    return launch_shrink_reduce(rp.r_max, rp, T, num_adapters, st);
}

// The fixed-order sum of split-K partials (one workgroup per 16-row tile).
int launch_shrink_reduce(int32_t r_max, const ReduceParams& rp, int32_t T, int32_t num_adapters, hipStream_t st) {
    const unsigned rgrid = (unsigned)std::min<int64_t>(SchedLayout::max_tiles16(T, num_adapters), kMaxGrid);
    const dim3 rb(kReduceWaves * kWave);
    if (r_max <= 16)
        hipLaunchKernelGGL(shrink_reduce_kernel<1>, dim3(rgrid), rb, 0, st, rp);
    else if (r_max <= 32)
        hipLaunchKernelGGL(shrink_reduce_kernel<2>, dim3(rgrid), rb, 0, st, rp);
    else if (r_max <= 64)
        hipLaunchKernelGGL(shrink_reduce_kernel<4>, dim3(rgrid), rb, 0, st, rp);
    else
        hipLaunchKernelGGL(shrink_reduce_kernel<8>, dim3(rgrid), rb, 0, st, rp);
    return hipGetLastError() == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

// Workspace of the split-K partials: [slices][T][round_up(r_max, 8)] fp32.
int64_t shrink_part_ld(int32_t r_max) { return round_up(r_max, 8); }
int64_t shrink_part_floats(int dtype, int32_t T, int32_t K, int32_t r_max) {
    return (int64_t)shrink_slices(dtype, K) * (T > 0 ? T : 1) * shrink_part_ld(r_max);
}

// Rank-split, tile offset and grid of an expand launch (shared with the
// backward, which runs the dX expand together with another kernel).
int expand_plan(const ExpandParams& p, int32_t T, int32_t num_adapters, int32_t r_max, ExpandParams* q,
                unsigned* grid) {
    *q = p;
    q->tiles64_off = SchedLayout::make(T, num_adapters).tiles64;
    const int64_t tasks = SchedLayout::max_tiles64(T, num_adapters) * ((p.N + kExpandCols - 1) / kExpandCols);
    *grid = grid_for(tasks, 1, kMaxGrid);
    return r_max <= 32 ? 1 : (r_max <= 64 ? 2 : 4);
}

int run_expand(int dtype, const ExpandParams& p, int32_t T, int32_t num_adapters, int32_t r_max, hipStream_t st) {
    ExpandParams q;
    unsigned grid;
    const int ks = expand_plan(p, T, num_adapters, r_max, &q, &grid);
    return dtype == LORA_BF16 ? launch_expand_t<LORA_BF16, false>(ks, q, grid, st)
                              : launch_expand_t<LORA_F32, false>(ks, q, grid, st);
}

}  // namespace lora

extern "C" size_t lora_shrink_workspace_bytes(int dtype, int32_t T, int32_t d_in, int32_t r_max) {
    if (!valid_dtype(dtype) || T < 0 || d_in < 1 || r_max < 1 || r_max > LORA_MAX_RANK) return 0;
    return (size_t)shrink_part_floats(dtype, T, d_in, r_max) * sizeof(float);
}

namespace lora {
// lora_shrink with its workspace given; shared with the entry point whose
// workspace is the library's static device scratch.
// Every check of lora_shrink except the workspace's (T == 0 passes).
int shrink_check(int dtype, const void* x, int64_t ldx, int32_t T, int32_t d_in, const lora_adapter* adapters,
                 int32_t num_adapters, int32_t r_max, const lora_segments& seg, const float* v, int64_t ldv) {
    int rc = check_common(dtype, T, num_adapters, r_max, adapters, seg);
    if (rc != LORA_OK) return rc;
    if (d_in < 1) return LORA_ERR_INVALID_ARG;
    if (T == 0) return LORA_OK;
    if ((rc = check_matrix(x, d_in, ldx)) != LORA_OK) return rc;
    return check_f32_rows(v, ldv, r_max);
}

int shrink_entry(int dtype, const void* x, int64_t ldx, int32_t T, int32_t d_in, const lora_adapter* adapters,
                 int32_t num_adapters, int32_t r_max, lora_segments seg, float* v, int64_t ldv, void* ws,
                 size_t ws_bytes, void* stream) {
    const int rc = shrink_check(dtype, x, ldx, T, d_in, adapters, num_adapters, r_max, seg, v, ldv);
    if (rc != LORA_OK || T == 0) return rc;
    if (!ws || !aligned16(ws) || ws_bytes < (size_t)shrink_part_floats(dtype, T, d_in, r_max) * sizeof(float))
        return LORA_ERR_WORKSPACE;
    // 16-row tiles on decode batches, and for rank <= 16 tables at any row
    // count: with one rank block per tile the full-K task reads each x row
    // once and needs no partial sums (4096 rows, one rank-16 adapter, 5120
    // -> 5120: 14.1 us against 18.6 us for the split-K shrink and its
    // reduce; with four rank blocks per tile, on the mixed batch, it reads x
    // four times and is slower, 34.0 against 29.9 us)
    if ((use_decode_path(dtype, T, num_adapters) || (dtype == LORA_BF16 && r_max <= 16)) &&
        dec_offsets_fit((int64_t)T * ldx * 2, d_in, r_max))
        return run_dec_shrink(dtype, x, ldx, T, d_in, adapters, num_adapters, r_max, seg, v, ldv, 0,
                              static_cast<hipStream_t>(stream));
    const SchedLayout sl = SchedLayout::make(T, num_adapters);
    ShrinkParams p{};
    p.x = x;
    p.ldx = ldx;
    p.K = d_in;
    p.adapters = adapters;
    p.r_max = r_max;
    p.perm = seg.perm;
    p.sched = seg.sched;
    p.tiles64_off = sl.tiles64;
    p.part = static_cast<float*>(ws);
    p.ldp = shrink_part_ld(r_max);
    p.slice_stride = (int64_t)T * p.ldp;
    p.nslices = shrink_slices(dtype, d_in);
    p.err = seg.err;
    p.rgroups = rank_groups(r_max);
    ReduceParams rp{};
    rp.part = p.part;
    rp.ldp = p.ldp;
    rp.slice_stride = p.slice_stride;
    rp.nslices = p.nslices;
    rp.adapters = adapters;
    rp.r_max = r_max;
    rp.perm = seg.perm;
    rp.sched = seg.sched;
    rp.tiles16_off = sl.tiles16;
    rp.out = v;
    rp.ldo = ldv;
    rp.out_by_pos = 0;
    rp.outT = nullptr;
    rp.ldT = 0;
    return run_shrink(dtype, false, p, rp, T, num_adapters, static_cast<hipStream_t>(stream));
}
}  // namespace lora

extern "C" int lora_shrink(int dtype, const void* x, int64_t ldx, int32_t T, int32_t d_in,
                           const lora_adapter* adapters, int32_t num_adapters, int32_t r_max, lora_segments seg,
                           float* v, int64_t ldv, void* ws, size_t ws_bytes, void* stream) {
    return shrink_entry(dtype, x, ldx, T, d_in, adapters, num_adapters, r_max, seg, v, ldv, ws, ws_bytes, stream);
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
    ExpandParams p{};
    p.v = v;
    p.ldv = ldv;
    p.v_by_pos = 0;
    p.adapters = adapters;
    p.r_max = r_max;
    p.perm = seg.perm;
    p.sched = seg.sched;
    p.y = y;
    p.ldy = ldy;
    p.N = d_out;
    p.err = seg.err;
    if (use_decode_path(dtype, T, num_adapters) && dec_offsets_fit((int64_t)T * ldy * 2, d_out, r_max))
        return run_dec_expand(dtype, v, ldv, 0, T, d_out, adapters, num_adapters, r_max, seg, y, ldy,
                              static_cast<hipStream_t>(stream));
    return run_expand(dtype, p, T, num_adapters, r_max, static_cast<hipStream_t>(stream));
}

