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
// to 64 ranks x one slice of kSliceChunks 64-wide K chunks; it writes the
// slice's partial sums, and shrink_reduce_kernel adds the slices in order.
// The eight waves cover the tile's 16-row blocks x sub-slices of the K slice
// (1 x 8, 2 x 4 or 4 x 2, by the tile's row count): every weight chunk is
// read from L2 once per tile and shared by the row-block waves through L1.
// Each wave runs up to four 16x16 MFMA tiles (A operand = weight rows,
// B operand = the block's rows), two chunks per iteration with their loads
// issued first; the sub-slice tiles of a row block are summed in wave order
// through LDS.  Within a chunk, lane group g and half h take K offsets
// 8 g + 32 h .. + 7, so each load instruction reads one contiguous 64-byte
// half line per row.  With TRANS_W and bf16, each chunk's weight block (64
// rows of B_a) is staged in the wave's LDS region as loaded and read back
// transposed with ds_read_b64_tr_b16.

constexpr int kShrinkWaves = 8;
constexpr int kShrinkThreads = kShrinkWaves * kWave;
#ifndef LORA_SHRINK_SLICE_CHUNKS
#define LORA_SHRINK_SLICE_CHUNKS 16  // K slice = 1024 elements
#endif
constexpr int kSliceChunks = LORA_SHRINK_SLICE_CHUNKS;
constexpr int kWPitch = 72;       // staged weight row: up to 64 ranks + 8 elements of padding

__host__ __device__ constexpr int shrink_slices(int K) { return (K + 64 * kSliceChunks - 1) / (64 * kSliceChunks); }

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
};

// Registers of one 64-wide K chunk in flight: the tile's rows (B operand)
// and, for row-major weights, the weight rows (A operand); for staged
// transposed weights, the raw 16-byte segments of the weight block.
template <int DT>
struct ShrinkStage {
    Frag<DT> x[2];
    Frag<DT> w[4][2];
};
template <int NSEG>
struct ShrinkStageTr {
    Frag<LORA_BF16> x[2];
    u32x4_t wr[NSEG];
};

template <int DT>
__device__ __forceinline__ void shrink_load_x(Frag<DT>* x, const char* xp, int kc, int lg, int K) {
    constexpr int EB = Frag<DT>::kBytes;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int kk = kc * 64 + 8 * lg + 32 * h;
        x[h] = Frag<DT>::load(xp + (int64_t)(kk < K ? kk : 0) * EB);  // past K: position 0, zeroed on use
    }
}

template <int DT>
__device__ __forceinline__ void shrink_mask_x(Frag<DT>* xf, const Frag<DT>* x, int kc, int lg, int K) {
#pragma unroll
    for (int h = 0; h < 2; ++h) xf[h] = kc * 64 + 8 * lg + 32 * h < K ? x[h] : Frag<DT>::zero();
}

// Row-major weights W(k, i) = A_a[k][i]; or, for fp32 transposed weights,
// element-wise loads of B_a[i][k].
template <int DT, bool TRANS_W, int NMB = 4>
__device__ __forceinline__ void shrink_load(ShrinkStage<DT>& S, const char* xp, const char* wbase, int kc, int lg,
                                            int lr, int K, int r, int rank0) {
    constexpr int EB = Frag<DT>::kBytes;
    shrink_load_x<DT>(S.x, xp, kc, lg, K);
    // The first NMB M-blocks are loaded unconditionally (ranks past r read
    // row r - 1: finite, outputs discarded), which keeps the stage in
    // registers.
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
        const int rk = min(rank0 + 16 * mb + lr, r - 1);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int kk = kc * 64 + 8 * lg + 32 * h;
            const int kq = kk < K ? kk : 0;
            if (TRANS_W)
                S.w[mb][h] = Frag<DT>::load_strided(wbase + ((int64_t)kq * r + rk) * EB, r, min(8, K - kq));
            else
                S.w[mb][h] = Frag<DT>::load(wbase + ((int64_t)rk * K + kq) * EB);
        }
    }
}

template <int DT, int NMB = 4>
__device__ __forceinline__ void shrink_compute(const ShrinkStage<DT>& S, f32x4_t* acc, int kc, int lg, int K) {
    Frag<DT> xf[2];
    shrink_mask_x<DT>(xf, S.x, kc, lg, K);
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int h = 0; h < 2; ++h) acc[mb] = mma(S.w[mb][h], xf[h], acc[mb]);
}

// Chunk i (0 <= i < n) of a wave's slice [kc0, kc0 + n), visited from a
// tile-dependent starting point so that the tiles of one adapter, which read
// the same weight rows, do not all read the same lines at the same time.
// The order is fixed per tile, so results stay bit-reproducible.
__device__ __forceinline__ int rotated(int kc0, int n, int rot, int i) {
    const int j = i + rot;
    return kc0 + (j < n ? j : j - n);
}

// Row-major weights, NMB rank blocks: two chunks per iteration, all loads first.
template <int DT, int NMB>
__device__ __forceinline__ void shrink_rows_loop(f32x4_t* acc, const char* xp, const char* wbase, int kc0, int kc1,
                                                 int rot, int lg, int lr, int K, int r, int rank0) {
    const int n = kc1 - kc0;
    for (int i = 0; i < n; i += 2) {
        const bool two = i + 1 < n;
        const int ka = rotated(kc0, n, rot, i);
        const int kb = two ? rotated(kc0, n, rot, i + 1) : ka;
        ShrinkStage<DT> S0, S1;
        shrink_load<DT, false, NMB>(S0, xp, wbase, ka, lg, lr, K, r, rank0);
        shrink_load<DT, false, NMB>(S1, xp, wbase, kb, lg, lr, K, r, rank0);
        shrink_compute<DT, NMB>(S0, acc, ka, lg, K);
        if (two) shrink_compute<DT, NMB>(S1, acc, kb, lg, K);
    }
}

// Transposed bf16 weights: the chunk's 64 rows of B_a (ranks rank0 ..
// rank0 + nr) are one contiguous block when nr = r, or row pieces of nr
// ranks; lanes load 16-byte segments of it (nr a power of two, 8..64).
template <int NSEG>
__device__ __forceinline__ void shrink_load_tr(ShrinkStageTr<NSEG>& S, const char* xp, const char* wbase, int kc,
                                               int lane, int K, int r, int rank0, int nr) {
    shrink_load_x<LORA_BF16>(S.x, xp, kc, lane >> 4, K);
    const int nseg = nr >> 3;  // a power of two: 1, 2, 4 or 8
    const int lseg = __builtin_ctz(nseg);
    // Segments i >= nseg repeat segment 0 of this lane (in bounds; not staged).
#pragma unroll
    for (int i = 0; i < NSEG; ++i) {
        const int sg = lane + kWave * (i < nseg ? i : 0);
        const int j = sg >> lseg;
        const int row = kc * 64 + j < K ? kc * 64 + j : 0;
        S.wr[i] = *gptr(reinterpret_cast<const u32x4_t*>(wbase + ((int64_t)row * r + rank0 + 8 * (sg & (nseg - 1))) * 2));
    }
}

template <int NSEG>
__device__ __forceinline__ void shrink_compute_tr(const ShrinkStageTr<NSEG>& S, f32x4_t* acc, uint16_t* wst, int kc,
                                                  int lane, int K, int nr, int nmb) {
    const int lg = lane >> 4;
    Frag<LORA_BF16> xf[2];
    shrink_mask_x<LORA_BF16>(xf, S.x, kc, lg, K);
    const int nseg = nr >> 3;
    const int lseg = __builtin_ctz(nseg);
#pragma unroll
    for (int i = 0; i < NSEG; ++i) {
        if (i < nseg) {
            const int sg = lane + kWave * i;
            *reinterpret_cast<u32x4_t*>(wst + (sg >> lseg) * kWPitch + 8 * (sg & (nseg - 1))) = S.wr[i];
        }
    }
    const int e = (lane & 15) >> 2;
    const int c = lane & 3;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
        if (mb < nmb) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                // rows 8 lg + 32 h + 0..7 of rank column 16 mb + (lane % 16)
                const uint16_t* base = wst + (8 * lg + 32 * h + e) * kWPitch + 16 * mb + 4 * c;
                const uint2 a = lds_read_tr16(base);
                const uint2 b = lds_read_tr16(base + 4 * kWPitch);
                Frag<LORA_BF16> wf;
                wf.q = u32x4_t{a.x, a.y, b.x, b.y};
                acc[mb] = mma(wf, xf[h], acc[mb]);
            }
        }
    }
}

template <int DT, bool TRANS_W>
__global__ __launch_bounds__(kShrinkThreads) __attribute__((amdgpu_waves_per_eu(DT == LORA_BF16 ? 4 : 2)))
void shrink_kernel(ShrinkParams p) {
    using F = Frag<DT>;
    constexpr int EB = F::kBytes;
    constexpr bool kTr = TRANS_W && DT == LORA_BF16;
    constexpr int kRedBytes = kShrinkWaves * 4 * kWave * 16;
    constexpr int kStageBytes = kTr ? kShrinkWaves * 64 * kWPitch * 2 : 0;
    __shared__ __attribute__((aligned(16))) char s_mem[kRedBytes > kStageBytes ? kRedBytes : kStageBytes];
    f32x4_t* s_red = reinterpret_cast<f32x4_t*>(s_mem);

    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int lr = lane & 15;  // MFMA row / column within the 16x16 tile
    const int lg = lane >> 4;  // K group of this lane
    uint16_t* wst = reinterpret_cast<uint16_t*>(s_mem) + wave * 64 * kWPitch;  // this wave's staging rows
    const int ntiles = p.sched[1];
    const int64_t n_tasks = (int64_t)ntiles * p.rgroups * p.nslices;
    const TaskSlice ts = xcd_slice(n_tasks, 1, 0);
    const int nkc = (p.K + 63) / 64;

    for (int64_t task = ts.begin; task < ts.end; task += ts.stride) {
        // consecutive tasks: consecutive tiles of the same (slice, rank group)
        const int tile = (int)(task % ntiles);
        const int rg = (int)((task / ntiles) % p.rgroups);
        const int sl = (int)(task / ((int64_t)ntiles * p.rgroups));
        const TileRec rec = load_tile(p.sched, p.tiles64_off, tile);
        const lora_adapter ad = load_adapter(p.adapters, rec.adapter);
        if (!adapter_ok(ad, p.r_max)) {
            if (rg == 0 && sl == 0 && threadIdx.x == 0) atomicAdd(p.err, 1);
            continue;
        }
        const int r = ad.rank;
        const int rank0 = rg * 64;
        if (rank0 >= r) continue;
        const int nr = min(64, r - rank0);
        const int nmb = (nr + 15) / 16;
        const int pos0 = rec.pos0;
        const int nrows = rec.rows;

        // Wave roles: nbw row blocks x (8 / nbw) sub-slices of this K slice.
        const int nnb = (nrows + 15) >> 4;
        const int nbw = nnb == 1 ? 1 : (nnb == 2 ? 2 : 4);
        const int nsub = kShrinkWaves / nbw;
        const int nb = wave % nbw;
        const int sub = wave / nbw;
        const int c0 = sl * kSliceChunks;
        const int nch = min(kSliceChunks, nkc - c0);
        const int kc0 = c0 + sub * nch / nsub;
        const int kc1 = c0 + (sub + 1) * nch / nsub;
        const bool active = nb < nnb;

        // Rows past the tile read the tile's first row (finite data; outputs discarded).
        const int rr = 16 * nb + lr;
        const int64_t xrow = p.perm[pos0 + (rr < nrows ? rr : 0)];
        const char* xp = static_cast<const char*>(p.x) + xrow * p.ldx * EB;
        const char* wbase = static_cast<const char*>(TRANS_W ? ad.B : ad.A);

        f32x4_t acc[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) acc[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        // Staged path: bf16 and the group's rank count a power of two >= 8.
        const bool staged = kTr && nr >= 8 && (nr & (nr - 1)) == 0 && (r & 7) == 0;
        if (active) {
            if (TRANS_W && !staged) {
                // transposed weights that cannot be staged in 16-byte segments
                // (fp32, or a rank that is not a multiple of 8): one chunk at a time
                for (int kc = kc0; kc < kc1; ++kc) {
                    F xr[2], xf[2];
                    shrink_load_x<DT>(xr, xp, kc, lg, p.K);
                    shrink_mask_x<DT>(xf, xr, kc, lg, p.K);
                    for (int mb = 0; mb < nmb; ++mb) {
                        const int rk = min(rank0 + 16 * mb + lr, r - 1);
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const int kk = kc * 64 + 8 * lg + 32 * h;
                            const int kq = kk < p.K ? kk : 0;
                            const F wf = F::load_strided(wbase + ((int64_t)kq * r + rk) * EB, r, min(8, p.K - kq));
#pragma unroll
                            for (int m = 0; m < 4; ++m)
                                if (m == mb) acc[m] = mma(wf, xf[h], acc[m]);
                        }
                    }
                }
            } else if (kTr && nr <= 32) {
                for (int kc = kc0; kc < kc1; kc += 2) {
                    const bool two = kc + 1 < kc1;
                    ShrinkStageTr<4> S0, S1;
                    shrink_load_tr(S0, xp, wbase, kc, lane, p.K, r, rank0, nr);
                    shrink_load_tr(S1, xp, wbase, two ? kc + 1 : kc, lane, p.K, r, rank0, nr);
                    shrink_compute_tr(S0, acc, wst, kc, lane, p.K, nr, nmb);
                    if (two) shrink_compute_tr(S1, acc, wst, kc + 1, lane, p.K, nr, nmb);
                }
            } else if (kTr) {
                for (int kc = kc0; kc < kc1; ++kc) {
                    ShrinkStageTr<8> S0;
                    shrink_load_tr(S0, xp, wbase, kc, lane, p.K, r, rank0, nr);
                    shrink_compute_tr(S0, acc, wst, kc, lane, p.K, nr, nmb);
                }
            } else if (!TRANS_W) {
                switch (nmb) {
                    case 1: shrink_rows_loop<DT, 1>(acc, xp, wbase, kc0, kc1, 0, lg, lr, p.K, r, rank0); break;
                    case 2: shrink_rows_loop<DT, 2>(acc, xp, wbase, kc0, kc1, 0, lg, lr, p.K, r, rank0); break;
                    case 3: shrink_rows_loop<DT, 3>(acc, xp, wbase, kc0, kc1, 0, lg, lr, p.K, r, rank0); break;
                    default: shrink_rows_loop<DT, 4>(acc, xp, wbase, kc0, kc1, 0, lg, lr, p.K, r, rank0); break;
                }
            }
        }

        __syncthreads();  // staging rows are reused as the reduction buffer
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) s_red[(wave * 4 + mb) * kWave + lane] = acc[mb];
        __syncthreads();
        // Waves 0 .. nbw-1 finish row block nb = wave: sub-slices summed in order.
        if (wave < nbw && active) {
            float* part = p.part + (int64_t)sl * p.slice_stride;
            const int n = lr;
            const int row = 16 * nb + n;
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
                if (mb < nmb) {
                    f32x4_t sum = s_red[(wave * 4 + mb) * kWave + lane];
                    for (int q = 1; q < nsub; ++q) sum += s_red[((wave + q * nbw) * 4 + mb) * kWave + lane];
                    const int rk = rank0 + 16 * mb + 4 * lg;  // D rows 4*(l/16)+i
                    if (row < nrows && rk < r)
                        *gptr(reinterpret_cast<f32x4_t*>(part + (int64_t)(pos0 + row) * p.ldp + rk)) = sum;
                }
            }
        }
        __syncthreads();
    }
}

// Sum of the K-slice partials, in slice order, for every row with an adapter:
//   out[row][k] (row = original row, or sorted position if out_by_pos) and,
//   if outT is given, outT[k][sorted position], for k < r_a.
// One workgroup per 16-row tile; thread (row n, group q) handles ranks
// 8 q .. 8 q + 7.
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
};

// shrink_reduce_kernel(ReduceParams) is defined in forward.hip.

}  // namespace lora
