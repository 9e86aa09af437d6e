// lora_kernels.h -- shrink, expand-add and token-contraction kernels (gfx950).
//
// All three walk the scheduling records written by the segment builder, so
// every workgroup touches one adapter's weights and that adapter's rows only
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

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

// Four 16-bit values of one LDS column: lane i of each 16-lane group gets
// rows row0 + 0..3 of column col0 + i, when lane 4e + c of the group passes
// the address of (row0 + e, col0 + 4c).  (gfx950 ds_read_b64_tr_b16.)
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
    const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4_t*)((__attribute__((address_space(3))) uint16_t*)(p)));
    return __builtin_bit_cast(uint2, v);
}

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

// ============================================================== expand-add
//
// Y[row][c] += s_a * sum_k V[row][k] * W(c, k) for the rows of one adapter:
//   W(c, k) = B_a[c][k]     (B_a is [N, r]; y += s B v, forward)
//   W(c, k) = A_a[k][c]     (TRANS_W: A_a is [r, N]; dX += s A^T g, backward)
// One workgroup = one 64-row tile x 256 output columns; each of its four
// waves owns 64 columns and keeps that weight block (A operand, KS x 32
// ranks) in registers.  The fp32 V rows of the tile are converted once per
// workgroup into MFMA B-operand fragments in LDS (bf16: hi = bf16(v),
// lo = bf16(v - hi)).  Every wave issues all of its y loads for the tile up
// front, then runs the tile in 16-row steps.  Output columns are assigned to
// MFMA rows so that each lane owns two runs of 8 columns of one row (see
// expand_col): 128 contiguous bytes per row and wave.

constexpr int kExpandWaves = 4;
constexpr int kExpandCols = kExpandWaves * 64;

struct ExpandParams {
    const float* v;  // [row][ldv]; row = original row, or sorted position if v_by_pos
    int64_t ldv;
    int32_t v_by_pos;
    const lora_adapter* adapters;
    int32_t r_max;
    const int32_t* perm;
    const int32_t* sched;
    int64_t tiles64_off;
    void* y;         // [row][ldy], rows through perm
    int64_t ldy;
    int32_t N;       // output columns (d_out, or d_in for dX)
    int32_t* err;
};

// Output column of MFMA row m in column block mb (0..3) of a 64-column block:
// lane group g ends up owning columns 8 g + 0..7 and 32 + 8 g + 0..7, so the
// four lane groups read and write one contiguous 64-byte half line per row
// and instruction.
__device__ __forceinline__ int expand_col(int mb, int m) { return 8 * (m >> 2) + 32 * (mb >> 1) + 4 * (mb & 1) + (m & 3); }

template <int DT, bool TRANS_W, int KS>
__global__ __launch_bounds__(kExpandWaves * kWave) void expand_kernel(ExpandParams p) {
    using F = Frag<DT>;
    using E = Elem<DT>;
    using O = F32Operand<DT>;
    constexpr int EB = F::kBytes;
    constexpr int YQ = EB;  // 16-byte quads per lane per 16-row step (16 columns)
    constexpr int kThreads = kExpandWaves * kWave;
    constexpr int kFragPerThread = 4 * KS * kWave / kThreads;  // = KS
    static_assert(sizeof(O) == 32, "fragment pair is two quads");
    __shared__ u32x4_t s_frag[4 * KS * kWave * 2];

    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int lr = lane & 15;
    const int lg = lane >> 4;
    const int ncg = (p.N + kExpandCols - 1) / kExpandCols;
    const int64_t n_tasks = (int64_t)p.sched[1] * ncg;
    const TaskSlice ts = xcd_slice(n_tasks, 1, 0);
    const char* ybase = static_cast<const char*>(p.y);

    for (int64_t task = ts.begin; task < ts.end; task += ts.stride) {
        const int tile = (int)(task / ncg);
        const int cg = (int)(task % ncg);
        const TileRec rec = load_tile(p.sched, p.tiles64_off, tile);
        const lora_adapter ad = load_adapter(p.adapters, rec.adapter);
        if (!adapter_ok(ad, p.r_max)) {
            if (cg == 0 && threadIdx.x == 0) atomicAdd(p.err, 1);
            continue;
        }
        const int r = ad.rank;
        const float s = ad.scale;
        const int pos0 = rec.pos0;
        const int nrows = rec.rows;
        const int nsub = (nrows + 15) >> 4;
        const int c0 = cg * kExpandCols + wave * 64;
        const bool cols_ok = c0 < p.N;

        // Row indices first (one round trip), for the y rows of this lane and
        // for the V rows whose fragments this thread converts.
        int64_t yrow[4];
        bool yok[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            yok[st] = cols_ok && 16 * st + lr < nrows;
            yrow[st] = p.perm[yok[st] ? pos0 + 16 * st + lr : pos0];
        }
        int64_t vrow[kFragPerThread];
        bool vok[kFragPerThread];
#pragma unroll
        for (int i = 0; i < kFragPerThread; ++i) {
            const int f = threadIdx.x + kThreads * i;
            const int row = 16 * (f / (KS * kWave)) + (f & 15);
            vok[i] = row < nrows;
            const int pos = pos0 + (vok[i] ? row : 0);
            vrow[i] = p.v_by_pos ? pos : p.perm[pos];
        }

        // V rows first: the fragment conversion waits for them while the weight
        // and y loads issued after them stay in flight.
        // (The pitch of V is a multiple of 8 and >= r_max, so 8 values from any
        // rank group that starts below r stay inside the row.)
        f32x4_t vq[kFragPerThread][2];
#pragma unroll
        for (int i = 0; i < kFragPerThread; ++i) {
            const int f = threadIdx.x + kThreads * i;
            const int kk = 32 * ((f / kWave) % KS) + 8 * ((f >> 4) & 3);
            const bool ld = vok[i] && kk < r;
            const LORA_GLOBAL f32x4_t* src = gptr(reinterpret_cast<const f32x4_t*>(p.v + (ld ? vrow[i] * p.ldv + kk : 0)));
            vq[i][0] = src[0];
            vq[i][1] = src[1];
        }
        // 1. Weight block: wf[mb][ks] holds W(c0 + expand_col(mb, lr), 32 ks + 8 lg + 0..7).
        F wf[4][KS];
        const char* wbase = static_cast<const char*>(TRANS_W ? ad.A : ad.B);
        if (!TRANS_W && (r & 7) == 0) {
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
                const int col = c0 + expand_col(mb, lr);
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int kk = 32 * ks + 8 * lg;
                    const bool ok = col < p.N && kk < r;
                    const F w = F::load(wbase + (ok ? (int64_t)col * r + kk : 0) * EB);
                    wf[mb][ks] = ok ? w : F::zero();
                }
            }
        } else {
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
                const int col = c0 + expand_col(mb, lr);
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int kk = 32 * ks + 8 * lg;
                    const int nval = (col < p.N) ? max(0, min(8, r - kk)) : 0;
                    if (TRANS_W)
                        wf[mb][ks] = F::load_strided(wbase + ((int64_t)(nval ? kk : 0) * p.N + (nval ? col : 0)) * EB,
                                                     p.N, nval);
                    else
                        wf[mb][ks] = F::load_strided(wbase + (nval ? (int64_t)col * r + kk : 0) * EB, 1, nval);
                }
            }
        }

        // 2. All y loads of this wave for the tile: row 16 st + lr, columns c0 + 8 lg + 32 h + 0..7.
        u32x4_t yq[4][YQ];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int col = c0 + 8 * lg + 32 * h;
                const bool ok = yok[st] && col < p.N;
                const LORA_GLOBAL u32x4_t* src =
                    gptr(reinterpret_cast<const u32x4_t*>(ybase + (ok ? yrow[st] * p.ldy + col : 0) * EB));
#pragma unroll
                for (int q = 0; q < YQ / 2; ++q) yq[st][h * (YQ / 2) + q] = src[q];
            }
        }

        // 3. V fragments of the tile -> LDS (once per workgroup).
#pragma unroll
        for (int i = 0; i < kFragPerThread; ++i) {
            const int f = threadIdx.x + kThreads * i;
            const int kk = 32 * ((f / kWave) % KS) + 8 * ((f >> 4) & 3);
            float fv[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                fv[e] = (vok[i] && kk + e < r) ? vq[i][0][e] : 0.f;
                fv[4 + e] = (vok[i] && kk + 4 + e < r) ? vq[i][1][e] : 0.f;
            }
            const O o = O::make(fv);
            const u32x4_t* oq = reinterpret_cast<const u32x4_t*>(&o);
            s_frag[2 * f] = oq[0];
            s_frag[2 * f + 1] = oq[1];
        }
        lds_barrier();

        // 4. MFMA and epilogue, 16 rows at a time.
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            if (st < nsub) {
                f32x4_t acc[4];
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) acc[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int f = (st * KS + ks) * kWave + lane;
                    O o;
                    u32x4_t* oq = reinterpret_cast<u32x4_t*>(&o);
                    oq[0] = s_frag[2 * f];
                    oq[1] = s_frag[2 * f + 1];
#pragma unroll
                    for (int mb = 0; mb < 4; ++mb) acc[mb] = o.mma_right(wf[mb][ks], acc[mb]);
                }
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int col = c0 + 8 * lg + 32 * h;
                    if (yok[st] && col < p.N) {
                        float yv[8];
                        E::unpack8(&yq[st][h * (YQ / 2)], yv);
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const int j = 8 * h + e;  // column offset 4 mb + i
                            yv[e] = yv[e] + s * acc[j >> 2][j & 3];
                        }
                        E::store8(static_cast<char*>(p.y) + (yrow[st] * p.ldy + col) * EB, yv);
                    }
                }
            }
        }
        lds_barrier();
    }
}

// ============================================================== token contraction
//
// For each adapter a with fine-tuning rows, each group of 32 ranks and each
// block of 64 columns:
//   dA_a[k][c] += s_a * sum_rows g[row][k] * x[row][c]      (c < d_in)
//   dB_a[c][k] += s_a * sum_rows dy[row][c] * v[row][k]     (c < d_out)
// The contraction runs over rows, so the row-major x / dy tiles (32 rows x
// 64 columns per wave and step) become MFMA B operands through LDS: bf16
// tiles are stored as loaded and read back transposed with
// ds_read_b64_tr_b16; fp32 tiles are written transposed element by element.
// g and v come rank-major ([k][sorted position]) from the shrink kernel.
// Four waves split the adapter's rows into contiguous ranges, two 32-row
// windows per iteration with all loads issued first; their partial tiles
// are summed in wave order through LDS and added to dA / dB, which no other
// workgroup touches.

constexpr int kContractWaves = 4;
constexpr int kContractMB = 2;    // 16-rank blocks per task (32 ranks)
constexpr int kCtPitch = 32 + 8;  // fp32 path: LDS pitch (elements) of a transposed column
constexpr int kQPitch = 64 + 8;   // bf16 path: LDS pitch (elements) of a staged row

struct ContractParams {
    const void* x;
    int64_t ldx;
    const void* dy;
    int64_t lddy;
    const float* gT;  // [r_max][ldT] by sorted position
    const float* vT;
    int64_t ldT;
    const lora_adapter* adapters;
    const lora_adapter_grad* grads;
    int32_t r_max;
    const int32_t* offsets;
    const int32_t* perm;
    const int32_t* sched;
    int64_t active_off;
    int32_t d_in, d_out;
    int32_t ncb_in, ncb_out;
    int32_t rgroups;  // ceil(r_max / 32)
    int32_t* err;
};

template <int DT>
struct ContractLds {
    static constexpr int EB = Frag<DT>::kBytes;
    // per wave: two window tiles
    static constexpr int kTileBytes = DT == LORA_BF16 ? 32 * kQPitch * 2 : 64 * kCtPitch * 4;
    static constexpr int kTransBytes = kContractWaves * 2 * kTileBytes;
    static constexpr int kRedBytes = kContractWaves * kContractMB * 4 * kWave * 16;
    static constexpr int kBytes = kTransBytes > kRedBytes ? kTransBytes : kRedBytes;
};

// Raw loads of one 32-row window: this lane's 4 rows x 8 columns of Q and,
// per rank block, 8 positions of P.
template <int DT>
struct ContractWin {
    Frag<DT> q[4];
    f32x4_t pv[kContractMB][2];
};

template <int DT>
__device__ __forceinline__ void contract_load(ContractWin<DT>& W, const char* q, int64_t ldq, const float* PT,
                                              int64_t ldT, const int32_t* perm, int win, int lo, int hi, int c0,
                                              int lcol, int lrow, int rank0, int r, int lane) {
    constexpr int EB = Frag<DT>::kBytes;
    int64_t rows[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int pos = win + lrow + j;
        rows[j] = perm[pos >= lo && pos < hi ? pos : lo];  // outside the range: row lo (finite, P is zero there)
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) W.q[j] = Frag<DT>::load(q + (rows[j] * ldq + c0 + lcol) * EB);
    const int pp = win + 8 * (lane >> 4);
#pragma unroll
    for (int mb = 0; mb < kContractMB; ++mb) {
        const int rk = min(rank0 + 16 * mb + (lane & 15), r - 1);  // ranks past r: discarded rows
        const LORA_GLOBAL f32x4_t* src = gptr(reinterpret_cast<const f32x4_t*>(PT + (int64_t)rk * ldT + pp));
        W.pv[mb][0] = src[0];
        W.pv[mb][1] = src[1];
    }
}

template <int DT>
__device__ __forceinline__ void contract_compute(const ContractWin<DT>& W, char* tile, f32x4_t (*acc)[4], int win,
                                                 int lo, int hi, int lcol, int lrow, int nmb, int lane) {
    using F = Frag<DT>;
    const int lr = lane & 15;
    const int lg = lane >> 4;
    // 1. Q tile -> LDS;  2. B operands: column 16 nb + lr, window rows 8 lg .. 8 lg + 7.
    F qf[4];
    if constexpr (DT == LORA_BF16) {
        uint16_t* t = reinterpret_cast<uint16_t*>(tile);
#pragma unroll
        for (int j = 0; j < 4; ++j) *reinterpret_cast<u32x4_t*>(t + (lrow + j) * kQPitch + lcol) = W.q[j].q;
        const int e = lr >> 2;
        const int c = lane & 3;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            const uint16_t* base = t + (8 * lg + e) * kQPitch + 16 * nb + 4 * c;
            const uint2 a = lds_read_tr16(base);
            const uint2 b = lds_read_tr16(base + 4 * kQPitch);
            qf[nb].q = u32x4_t{a.x, a.y, b.x, b.y};
        }
    } else {
        float* t = reinterpret_cast<float*>(tile);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e) t[(lcol + e) * kCtPitch + lrow + j] = W.q[j].get(e);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) qf[nb] = F::load_lds(t + (16 * nb + lr) * kCtPitch + 8 * lg);
    }
    // 3. A operands from P^T (zero outside [lo, hi)), hi/lo split for bf16.
    const int pp = win + 8 * lg;
#pragma unroll
    for (int mb = 0; mb < kContractMB; ++mb) {
        if (mb < nmb) {
            float f[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                f[e] = (pp + e >= lo && pp + e < hi) ? W.pv[mb][0][e] : 0.f;
                f[4 + e] = (pp + 4 + e >= lo && pp + 4 + e < hi) ? W.pv[mb][1][e] : 0.f;
            }
            const F32Operand<DT> po = F32Operand<DT>::make(f);
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = po.mma_left(qf[nb], acc[mb][nb]);
        }
    }
}

template <int DT>
__global__ __launch_bounds__(kContractWaves * kWave) void contract_kernel(ContractParams p) {
    using F = Frag<DT>;
    __shared__ __attribute__((aligned(16))) char s_mem[ContractLds<DT>::kBytes];

    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int lr = lane & 15;
    const int lg = lane >> 4;
    const int ncb = p.ncb_in + p.ncb_out;
    const int64_t n_tasks = (int64_t)p.sched[2] * p.rgroups * ncb;
    const TaskSlice ts = xcd_slice(n_tasks, 1, 0);
    char* tileA = s_mem + (2 * wave) * ContractLds<DT>::kTileBytes;
    char* tileB = s_mem + (2 * wave + 1) * ContractLds<DT>::kTileBytes;
    // Loader role: lane covers window rows 4*(lane/8)+j (j < 4), columns 8*(lane%8)+e (e < 8).
    const int lrow = 4 * (lane >> 3);
    const int lcol = 8 * (lane & 7);

    for (int64_t task = ts.begin; task < ts.end; task += ts.stride) {
        const int cb_all = (int)(task % ncb);
        const int rg = (int)((task / ncb) % p.rgroups);
        const int act = (int)(task / ((int64_t)ncb * p.rgroups));
        const int a = p.sched[p.active_off + act];
        const lora_adapter ad = load_adapter(p.adapters, a);
        const lora_adapter_grad gr = load_grad(p.grads, a);
        const bool is_dA = cb_all < p.ncb_in;
        if (!adapter_ok(ad, p.r_max) || gr.dA == nullptr || gr.dB == nullptr) {
            if (cb_all == 0 && rg == 0 && threadIdx.x == 0) atomicAdd(p.err, 1);
            continue;
        }
        const int r = ad.rank;
        const int rank0 = rg * 16 * kContractMB;
        if (rank0 >= r) continue;
        const int nmb = min(kContractMB, (r - rank0 + 15) / 16);
        const int cb = is_dA ? cb_all : cb_all - p.ncb_in;
        const int c0 = cb * 64;
        const int N = is_dA ? p.d_in : p.d_out;
        const char* q = static_cast<const char*>(is_dA ? p.x : p.dy);
        const int64_t ldq = is_dA ? p.ldx : p.lddy;
        const float* PT = is_dA ? p.gT : p.vT;
        // Columns past N (N is a multiple of 8) read column block 0 of the row; never written back.
        const int cq = c0 + lcol < N ? c0 : -lcol;

        const int lo = p.offsets[a];
        const int hi = p.offsets[a + 1];
        // 32-aligned windows of sorted positions covering [lo, hi), split over the waves.
        const int w0 = lo & ~31;
        const int nwin = (hi - w0 + 31) / 32;
        const int wa = w0 + 32 * (int)((int64_t)wave * nwin / kContractWaves);
        const int wb = w0 + 32 * (int)((int64_t)(wave + 1) * nwin / kContractWaves);

        f32x4_t acc[kContractMB][4];
#pragma unroll
        for (int mb = 0; mb < kContractMB; ++mb)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        // Windows visited from a task-dependent start (the column blocks of one
        // adapter read the same g / v windows); fixed order per task.
        const int nw = (wb - wa) / 32;
        const int rot = nw > 0 ? (int)(task % nw) : 0;
        for (int i = 0; i < nw; i += 2) {
            const bool two = i + 1 < nw;
            const int wa0 = wa + 32 * (rotated(0, nw, rot, i));
            const int wa1 = two ? wa + 32 * (rotated(0, nw, rot, i + 1)) : wa0;
            ContractWin<DT> W0, W1;
            contract_load<DT>(W0, q, ldq, PT, p.ldT, p.perm, wa0, lo, hi, cq, lcol, lrow, rank0, r, lane);
            contract_load<DT>(W1, q, ldq, PT, p.ldT, p.perm, wa1, lo, hi, cq, lcol, lrow, rank0, r, lane);
            contract_compute<DT>(W0, tileA, acc, wa0, lo, hi, lcol, lrow, nmb, lane);
            if (two) contract_compute<DT>(W1, tileB, acc, wa1, lo, hi, lcol, lrow, nmb, lane);
        }

        // Fixed-order sum of the four waves' tiles.
        __syncthreads();
        f32x4_t* red = reinterpret_cast<f32x4_t*>(s_mem);
#pragma unroll
        for (int mb = 0; mb < kContractMB; ++mb)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) red[((wave * kContractMB + mb) * 4 + nb) * kWave + lane] = acc[mb][nb];
        __syncthreads();
        {
            const int nb = wave;  // this wave finishes column block nb
            const float s = ad.scale;
#pragma unroll
            for (int mb = 0; mb < kContractMB; ++mb) {
                if (mb < nmb) {
                    f32x4_t sum = red[(mb * 4 + nb) * kWave + lane];
#pragma unroll
                    for (int w = 1; w < kContractWaves; ++w) sum += red[((w * kContractMB + mb) * 4 + nb) * kWave + lane];
                    const int col = c0 + 16 * nb + lr;
                    if (col < N) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int rk = rank0 + 16 * mb + 4 * lg + i;
                            if (rk < r) {
                                float* dst = is_dA ? gr.dA + (int64_t)rk * p.d_in + col : gr.dB + (int64_t)col * r + rk;
                                *gptr(dst) += s * sum[i];
                            }
                        }
                    }
                }
            }
        }
        __syncthreads();
    }
}

}  // namespace lora
