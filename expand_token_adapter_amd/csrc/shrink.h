// shrink.h -- shrink kernel: rows times an adapter factor into a rank-r fp32 result (gfx950).
//
// Walks the scheduling records written by the segment builder, so every
// workgroup touches one adapter's weights and that adapter's rows only
// (multi-LoRA batching: each row applies its own adapter, DeltaServe section
// 2.2).  Dense work goes to 16x16 MFMA tiles; every reduction runs in a fixed
// order, so results are bit-reproducible.
#pragma once

#include "device_common.h"

namespace lora {

// ============================================================== shrink
//
// out[row][k] = sum_i X[row][i] * W(k, i) for the rows of one adapter, where
//   W(k, i) = A_a[k][i]     (A_a is [r, K]; v = A x, the "A x" of h(x) = Wx + BAx)
//   W(k, i) = B_a[i][k]     (TRANS_W: B_a is [K, r]; g = B^T dy in the backward)
// Split over K.  One workgroup = one tile of up to 64 rows x one group of up
// to 64 ranks x one slice of up to 512 (bf16) or 256 (fp32) elements of K;
// it writes the slice's partial sums, and shrink_reduce_kernel adds the
// slices in order.  The workgroup first copies the weight slice into LDS
// with row-contiguous loads (B_a is transposed on the way), so its waves
// read each weight byte from L2 once.  Its eight waves are four 16-row blocks
// x two halves of the slice: each issues the loads of its whole x half-slice
// at once, then runs up to four 16x16 MFMA tiles per 32 elements of K (A
// operand = weight rows from LDS, B operand = its rows); the second half's
// tiles are added to the first's through LDS, in that order.  Within a
// 64-element chunk, lane group g and half h take K offsets 8 g + 32 h .. + 7.
// The next task's tile record, adapter entry and row indices are fetched
// while the current task's loads are in flight.
//
// LDS layout of the weight slice: one 1 KB row per rank, 64 units of 16
// bytes; unit u of rank row j sits at position u ^ (j % 16), so the 16 rank
// rows of one MFMA operand read fall on distinct banks.

constexpr int kShrinkWaves = 8;
constexpr int kShrinkThreads = kShrinkWaves * kWave;

// 64-element K chunks per slice (the slice's rank rows, up to 64, fill up to 64 KB of LDS).
__host__ __device__ constexpr int shrink_slice_chunks(int dtype) { return dtype == LORA_BF16 ? 8 : 4; }
__host__ __device__ constexpr int shrink_slices(int dtype, int K) {
    return (int)((((int64_t)K + 63) / 64 + shrink_slice_chunks(dtype) - 1) / shrink_slice_chunks(dtype));
}

struct ShrinkParams {
    const void* x;   // rows gathered through perm
    int64_t ldx;
    int32_t K;       // reduction length (d_in, or d_out for g)
    const lora_adapter* adapters;
    int32_t r_max;
    const int32_t* perm;
    const int32_t* sched;
    int64_t tiles64_off;
    float* part;     // partial sums [slice][sorted position][ldp]
    int64_t ldp;
    int64_t slice_stride;
    int32_t nslices;
    int32_t* err;
    int32_t rgroups; // ceil(r_max / 64)
    // backward preemption: when set and *stop != 0 at the start, the
    // workgroup does nothing (null in the forward)
    const int32_t* stop;
};

// acc[mb] += W(rank block mb) x X over chunks cc0 .. cc0 + SCH - 1 of the slice
// (chunks >= nch and K offsets >= klen contribute nothing).
template <int DT, int SCH, int NMB>
__device__ __forceinline__ void shrink_slice_mma(f32x4_t* acc, const Frag<DT> (*xr)[2], const u32x4_t* s_w, int cc0,
                                                 int nch, int klen, int lr, int lg) {
    using F = Frag<DT>;
#pragma unroll
    for (int c = 0; c < SCH; ++c) {
        const int cc = cc0 + c;
        if (cc < nch) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int kk = cc * 64 + 8 * lg + 32 * h;
                const F xf = kk < klen ? xr[c][h] : F::zero();
#pragma unroll
                for (int mb = 0; mb < NMB; ++mb) {
                    const u32x4_t* wrow = s_w + (16 * mb + lr) * 64;
                    F wf;
                    if constexpr (DT == LORA_BF16) {
                        wf.q = wrow[(8 * cc + 4 * h + lg) ^ lr];
                    } else {
                        const int u0 = 16 * cc + 8 * h + 2 * lg;
                        wf.q0 = wrow[u0 ^ lr];
                        wf.q1 = wrow[(u0 + 1) ^ lr];
                    }
                    acc[mb] = mma(wf, xf, acc[mb]);
                }
            }
        }
    }
}

// RB: 16-rank blocks a task covers (1, 2 or 4, from r_max): the weight slice
// in LDS (16 RB rank rows of 1 KB) and the accumulators are sized for it, so
// small ranks leave room for more workgroups per CU.
template <int DT, bool TRANS_W, int RB>
__global__ __launch_bounds__(kShrinkThreads) __attribute__((amdgpu_waves_per_eu(4)))
void shrink_kernel(ShrinkParams p) {
    using F = Frag<DT>;
    constexpr int EB = F::kBytes;
    constexpr int EPU = 16 / EB;                 // elements per 16-byte unit
    constexpr int SC = shrink_slice_chunks(DT);  // 64-element chunks per slice
    constexpr int SCH = SC / 2;                  // chunks per wave (half a slice)
    static_assert(RB == 1 || RB == 2 || RB == 4, "rank blocks per task");
    constexpr int NU = 16 * RB * 64 / kShrinkThreads; // row-major weight rows x units per thread
    constexpr int kTB = 4;                       // transposed weight units per thread and batch
    __shared__ __attribute__((aligned(16))) u32x4_t s_w[16 * RB * 64];
    char* s_wb = reinterpret_cast<char*>(s_w);
    f32x4_t* s_red = reinterpret_cast<f32x4_t*>(s_w);  // reused after the MFMA pass

    if (p.stop && *p.stop) return;
    const int wave = wave_id();
    const int lane = threadIdx.x & (kWave - 1);
    const int lr = lane & 15;  // MFMA row / column within the 16x16 tile
    const int lg = lane >> 4;  // K group of this lane
    const int rb = wave & 3;   // 16-row block of the tile
    const int kh = wave >> 2;  // half of the slice
    const int ntiles = p.sched[1];
    const int64_t n_tasks = (int64_t)ntiles * p.rgroups * p.nslices;
    const TaskSlice ts = xcd_slice(n_tasks, 1, 0);
    const int nkc = (p.K + 63) / 64;

    // Metadata of the next task (consecutive tasks: consecutive tiles of the
    // same slice and rank group).
    TileRec rec_n{0, 0, 0};
    lora_adapter ad_n{};
    int64_t xrow_n = 0;
    auto fetch = [&](int64_t t) {
        rec_n = load_tile(p.sched, p.tiles64_off, (int)(t % ntiles));
        const int rr = 16 * rb + lr;  // rows past the tile read its first row
        xrow_n = p.perm[rec_n.pos0 + (rr < rec_n.rows ? rr : 0)];
        ad_n = load_adapter(p.adapters, rec_n.adapter);
    };
    if (ts.begin < ts.end) fetch(ts.begin);

    for (int64_t task = ts.begin; task < ts.end; task += ts.stride) {
        const TileRec rec = rec_n;
        const lora_adapter ad = ad_n;
        const int64_t xrow = xrow_n;
        const int rg = (int)((task / ntiles) % p.rgroups);
        const int sl = (int)(task / ((int64_t)ntiles * p.rgroups));
        const bool ok = adapter_ok(ad, p.r_max);
        if (!ok && rg == 0 && sl == 0 && threadIdx.x == 0) atomicAdd(p.err, 1);
        const int r = ad.rank;
        const int rank0 = rg * 64;
        const bool work = ok && rank0 < r;
        const int nr = min(64, r - rank0);
        const int nmb = (nr + 15) / 16;
        const int pos0 = rec.pos0;
        const int nrows = rec.rows;
        const int c0 = sl * SC;
        const int nch = min(SC, nkc - c0);
        const int k0 = c0 * 64;
        const int klen = min(nch * 64, p.K - k0);  // elements of K in this slice
        const char* wbase = static_cast<const char*>(TRANS_W ? ad.B : ad.A);

        // Transposed B_a with 16-byte aligned rows: batches of kTB units per
        // thread, unit u = K row u / upr, ranks EPU (u % upr) .. + EPU - 1.
        const bool trans_units = TRANS_W && (r % EPU) == 0;
        const int upr = nr / EPU;
        const int tunits = nch * 64 * upr;
        u32x4_t wu[kTB];
        auto load_tbatch = [&](int b) {
#pragma unroll
            for (int i = 0; i < kTB; ++i) {
                const int u = threadIdx.x + kShrinkThreads * (kTB * b + i);
                const int kk = u / upr;
                const int kr = kk < klen ? kk : 0;
                const int q = u - kk * upr;
                wu[i] = *gptr(reinterpret_cast<const u32x4_t*>(wbase + ((int64_t)(k0 + kr) * r + rank0 + q * EPU) * EB));
            }
        };
        auto store_tbatch = [&](int b) {
#pragma unroll
            for (int i = 0; i < kTB; ++i) {
                const int u = threadIdx.x + kShrinkThreads * (kTB * b + i);
                const int kk = u / upr;
                if (u < tunits) {
                    const int q = u - kk * upr;
                    const int upos = kk / EPU;
                    const int eoff = (kk % EPU) * EB;
#pragma unroll
                    for (int e = 0; e < EPU; ++e) {
                        const int j = q * EPU + e;
                        char* dst = s_wb + j * 1024 + ((upos ^ (j & 15)) * 16) + eoff;
                        if constexpr (EB == 2)
                            *reinterpret_cast<uint16_t*>(dst) = (uint16_t)(wu[i][e >> 1] >> (16 * (e & 1)));
                        else
                            *reinterpret_cast<uint32_t*>(dst) = wu[i][e];
                    }
                }
            }
        };

        // 1. This wave's x half-slice (chunk c, half h; chunks past the slice
        //    re-read its start), then the weight slice loads (16-byte units).
        F xr[SCH][2];
        if (work) {
            const char* xp = static_cast<const char*>(p.x) + xrow * p.ldx * EB;
#pragma unroll
            for (int c = 0; c < SCH; ++c)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int cc = kh * SCH + c;
                    const int kk = (cc < nch ? cc * 64 : 0) + 8 * lg + 32 * h;
                    xr[c][h] = F::load(xp + (int64_t)(k0 + (kk < klen ? kk : 0)) * EB);
                }
            if constexpr (!TRANS_W) {
                // Straight into LDS, issued last (the compiler does not track
                // these loads; the barrier below waits for them): rank row
                // j = wave + 8 i; lane L fetches unit L ^ (j % 16) of the row,
                // which lands in slot L of the LDS row.  Rows past the group are
                // not loaded (their MFMA outputs are discarded).
#pragma unroll
                for (int i = 0; i < NU; ++i) {
                    const int j = wave + kShrinkWaves * i;
                    if (j < nr) {
                        const int q = lane ^ (j & 15);
                        const int kq = q * EPU < klen ? q * EPU : 0;
                        lds_dma16_async(wbase + ((int64_t)(rank0 + j) * p.K + k0 + kq) * EB, s_w + j * 64);
                    }
                }
            } else {
                if (trans_units) load_tbatch(0);
            }
        }

        // 2. Next task's metadata, while this task's loads are in flight.
        if (task + ts.stride < ts.end) fetch(task + ts.stride);
        if (!work) continue;

        // 3. Weight slice -> LDS (swizzled rows), then one barrier.
        if constexpr (!TRANS_W) {
            // this wave's weight loads into LDS (and its x loads) have landed
            // before the barrier; a barrier alone does not wait for them
            wait_vmcnt_le<0>();
        } else if (trans_units) {
            store_tbatch(0);
            for (int b = 1; kShrinkThreads * kTB * b < tunits; ++b) {
                load_tbatch(b);
                store_tbatch(b);
            }
        } else {
            // transposed weights whose rows are not 16-byte aligned: element by element
            for (int e = threadIdx.x; e < nch * 64 * nr; e += kShrinkThreads) {
                const int kk = e / nr;
                const int j = e - kk * nr;
                const int kr = kk < klen ? kk : 0;
                char* dst = s_wb + j * 1024 + (((kk / EPU) ^ (j & 15)) * 16) + (kk % EPU) * EB;
                const char* src = wbase + ((int64_t)(k0 + kr) * r + rank0 + j) * EB;
                if constexpr (EB == 2)
                    *reinterpret_cast<uint16_t*>(dst) = *gptr(reinterpret_cast<const uint16_t*>(src));
                else
                    *reinterpret_cast<uint32_t*>(dst) = *gptr(reinterpret_cast<const uint32_t*>(src));
            }
        }
        __syncthreads();

        // 4. MFMA over this wave's half-slice (row blocks past the tile skip it).
        const bool rows_ok = 16 * rb < nrows;
        f32x4_t acc[RB];
#pragma unroll
        for (int mb = 0; mb < RB; ++mb) acc[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (rows_ok) {
            switch (nmb) {
                case 1: shrink_slice_mma<DT, SCH, 1>(acc, xr, s_w, kh * SCH, nch, klen, lr, lg); break;
                case 2: if constexpr (RB >= 2) shrink_slice_mma<DT, SCH, 2>(acc, xr, s_w, kh * SCH, nch, klen, lr, lg); break;
                case 3: if constexpr (RB >= 4) shrink_slice_mma<DT, SCH, 3>(acc, xr, s_w, kh * SCH, nch, klen, lr, lg); break;
                default: if constexpr (RB >= 4) shrink_slice_mma<DT, SCH, 4>(acc, xr, s_w, kh * SCH, nch, klen, lr, lg); break;
            }
        }
        __syncthreads();  // weight slice no longer read: its LDS holds the second half's tiles
        if (kh == 1 && rows_ok) {
#pragma unroll
            for (int mb = 0; mb < RB; ++mb) s_red[(rb * RB + mb) * kWave + lane] = acc[mb];
        }
        __syncthreads();
        if (kh == 0 && rows_ok) {
            // D rows 4 (l / 16) + i of block mb = ranks, column l % 16 = row of the block.
            float* part = p.part + (int64_t)sl * p.slice_stride;
            const int row = 16 * rb + lr;
#pragma unroll
            for (int mb = 0; mb < RB; ++mb) {
                const int rk = rank0 + 16 * mb + 4 * lg;
                const f32x4_t sum = acc[mb] + s_red[(rb * RB + mb) * kWave + lane];
                if (mb < nmb && row < nrows && rk < r)
                    *gptr(reinterpret_cast<f32x4_t*>(part + (int64_t)(pos0 + row) * p.ldp + rk)) = sum;
            }
        }
        __syncthreads();  // the weight slice is rewritten by the next task
    }
}

// Sum of the K-slice partials, in slice order, for every row with an adapter:
//   out[row][k] (row = original row, or sorted position if out_by_pos) and,
//   if outT is given, outT[k][sorted position], for k < r_a; ranks r_a ..
//   round_up(r_a, 8) - 1 of out are written as zeros.  One wave per 16-row
//   tile record; lane (row n, group g) handles ranks 8 (g + 4 i) .. + 7.
struct ReduceParams {
    const float* part;
    int64_t ldp;
    int64_t slice_stride;
    int32_t nslices;
    const lora_adapter* adapters;
    int32_t r_max;
    const int32_t* perm;
    const int32_t* sched;
    int64_t tiles16_off;
    float* out;
    int64_t ldo;
    int32_t out_by_pos;
    float* outT;
    int64_t ldT;
    // optional rank-major copy of a caller's v: vT[k][pos] = vsrc[perm[pos]][k]
    // for k < r_a (pitch ldT), written alongside the sum of the same tile
    const float* vsrc;
    int64_t ldvsrc;
    float* vT;
    // backward preemption: when set and *stop != 0 at the start, the
    // workgroup does nothing (null in the forward)
    const int32_t* stop;
};

// shrink_reduce_kernel(ReduceParams) is defined in forward.hip.

}  // namespace lora
