// expand.h -- expand-add kernel: y += s W v for the rows of each adapter (gfx950).
//
// Walks the scheduling records written by the segment builder, so every
// workgroup touches one adapter's weights and that adapter's rows only
// (multi-LoRA batching: each row applies its own adapter, DeltaServe section
// 2.2).  Dense work goes to 16x16 MFMA tiles; every reduction runs in a fixed
// order, so results are bit-reproducible.
#pragma once

#include "device_common.h"

namespace lora {

// ============================================================== expand-add
//
// Y[row][c] += s_a * sum_k V[row][k] * W(c, k) for the rows of one adapter:
//   W(c, k) = B_a[c][k]     (B_a is [N, r]; y += s B v, forward)
//   W(c, k) = A_a[k][c]     (TRANS_W: A_a is [r, N]; dX += s A^T g, backward)
// One workgroup = one tile record of up to 64 rows x 256 output columns;
// each of its four waves owns 64 columns and keeps that weight block (MFMA A
// operand, KS x 32 ranks) in registers for the whole tile.  At the start of a
// tile the workgroup converts the tile's fp32 V rows once into MFMA B-operand
// fragments in LDS (bf16: hi = bf16(v), lo = bf16(v - hi)).  The tile is then
// finished 16 rows at a time while the y rows of the next steps are already
// in flight (a ring of kYBuf steps; for bf16 the whole tile).  Taller tiles
// (fewer weight-block loads) measured slower: fewer workgroups in flight.  y is read and written row-contiguously:
// lane L of a wave owns columns 8 (L % 8) .. + 7 of rows L / 8 and 8 + L / 8
// of a 16-row step, so eight consecutive lanes cover 128 contiguous bytes of
// a bf16 row; the MFMA accumulators are brought into that layout through a
// small per-wave LDS buffer.

constexpr int kExpandWaves = 4;
constexpr int kExpandCols = kExpandWaves * 64;
constexpr int kTPitch = 68;  // floats per row of the per-wave transpose buffer (16 rows x 64 columns)

struct ExpandParams {
    const float* v;  // [row][ldv]; row = original row, or sorted position if v_by_pos
    int64_t ldv;
    int32_t v_by_pos;
    const lora_adapter* adapters;
    int32_t r_max;
    const int32_t* perm;
    const int32_t* sched;
    int64_t tiles64_off;
    void* y;            // [row][ldy], rows through perm
    int64_t ldy;
    int32_t N;          // output columns (d_out, or d_in for dX)
    int32_t* err;
    // backward preemption: when set and *stop != 0 at the start, the
    // workgroup does nothing (null in the forward)
    const int32_t* stop;
};

// Raw element type of the weights read element by element, and the fragment
// of 8 such elements (elements n .. 7 zeroed).
template <int DT>
struct GatherElem;
template <>
struct GatherElem<LORA_BF16> {
    using type = uint16_t;
    __device__ __forceinline__ static Frag<LORA_BF16> frag(const uint32_t (&h)[8], int n) {
        u32x4_t q;
#pragma unroll
        for (int j = 0; j < 4; ++j) q[j] = (2 * j < n ? h[2 * j] : 0u) | ((2 * j + 1 < n ? h[2 * j + 1] : 0u) << 16);
        return Frag<LORA_BF16>{q};
    }
};
template <>
struct GatherElem<LORA_F32> {
    using type = uint32_t;
    __device__ __forceinline__ static Frag<LORA_F32> frag(const uint32_t (&h)[8], int n) {
        u32x4_t a, b;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            a[j] = j < n ? h[j] : 0u;
            b[j] = j + 4 < n ? h[j + 4] : 0u;
        }
        return Frag<LORA_F32>{a, b};
    }
};

// The kernel's work as workgroup blk of nblk (nblk a multiple of 8, the
// workgroup at launch index blk), so that another kernel can run it on part
// of its grid.
template <int KS>
struct ExpandLds {
    static constexpr int kFragBytes = (64 / 16) * KS * kWave * 2 * 16;   // s_frag: STEPS x KS x 64 x 2 quads
    static constexpr int kTBytes = kExpandWaves * 16 * kTPitch * 4;      // s_t: per-wave transpose buffers
    static constexpr int kRowBytes = 64 * 4;                             // s_row
    static constexpr int kBytes = kFragBytes + kTBytes + kRowBytes;
};

// (s_lds: ExpandLds<KS>::kBytes of LDS, 16-byte aligned)
template <int DT, bool TRANS_W, int KS>
__device__ __forceinline__ void expand_body(const ExpandParams& p, int blk, int nblk, char* s_lds) {
    using F = Frag<DT>;
    using E = Elem<DT>;
    using O = F32Operand<DT>;
    constexpr int EB = F::kBytes;
    constexpr int YQ = EB / 2;                   // 16-byte quads per 8 elements
    constexpr int ROWS = 64;
    constexpr int STEPS = ROWS / 16;
    constexpr int kThreads = kExpandWaves * kWave;
    constexpr int NF = STEPS * KS * kWave / kThreads;  // V fragments converted per thread
    constexpr int kYBuf = DT == LORA_BF16 ? 4 : 2;     // y steps held in registers
    static_assert(sizeof(O) == 32, "fragment pair is two quads");
    static_assert(ExpandLds<KS>::kFragBytes == STEPS * KS * kWave * 2 * 16, "LDS layout");
    u32x4_t* s_frag = reinterpret_cast<u32x4_t*>(s_lds);
    float(*s_t)[16 * kTPitch] = reinterpret_cast<float(*)[16 * kTPitch]>(s_lds + ExpandLds<KS>::kFragBytes);
    int32_t* s_row = reinterpret_cast<int32_t*>(s_lds + ExpandLds<KS>::kFragBytes + ExpandLds<KS>::kTBytes);

    const int wave = wave_id();
    const int lane = threadIdx.x & (kWave - 1);
    const int lr = lane & 15;
    const int lg = lane >> 4;
    const int yr = lane >> 3;       // row (and row + 8) of the step in the row-contiguous layout
    const int yc = 8 * (lane & 7);  // first column (of the wave's 64) in that layout
    if (p.stop && *p.stop) return;
    const int ncg = (p.N + kExpandCols - 1) / kExpandCols;
    const int64_t n_tasks = (int64_t)p.sched[1] * ncg;
    const TaskSlice ts = xcd_slice_of(blk, nblk, n_tasks, 1, 0);
    char* ybase = static_cast<char*>(p.y);
    float* tw = &s_t[wave][0];

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
        const int nst = (nrows + 15) >> 4;
        const int c0 = cg * kExpandCols + wave * 64;

        // 1. Original rows of the tile (rows past the tile repeat its first row).
        int32_t my_row = 0;
        if (threadIdx.x < ROWS) my_row = p.perm[pos0 + (int)threadIdx.x < pos0 + nrows ? pos0 + threadIdx.x : pos0];

        // 2. Weight block: wf[mb][ks] holds W(c0 + 16 mb + lr, 32 ks + 8 lg + 0..7).
        F wf[4][KS];
        const char* wbase = static_cast<const char*>(TRANS_W ? ad.A : ad.B);
        if (!TRANS_W && (r & 7) == 0) {
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
                const int col = c0 + 16 * mb + lr;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int kk = 32 * ks + 8 * lg;
                    const bool ok = col < p.N && kk < r;
                    const F w = F::load(wbase + (ok ? (int64_t)col * r + kk : 0) * EB);
                    wf[mb][ks] = ok ? w : F::zero();
                }
            }
        } else if constexpr (!TRANS_W) {
            // rows of B_a not in whole 16-byte units (rare): element by element
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
                const int col = c0 + 16 * mb + lr;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int kk = 32 * ks + 8 * lg;
                    const int nval = (col < p.N) ? max(0, min(8, r - kk)) : 0;
                    wf[mb][ks] = F::load_strided(wbase + (nval ? (int64_t)col * r + kk : 0) * EB, 1, nval);
                }
            }
        } else {
            // A_a read transposed, element by element: every element load of
            // the block is issued before any is packed, with clamped indices
            // and no branches (a conditional load is waited for where its
            // branch joins, which made this one round trip per pair of
            // elements).
            using ET = typename GatherElem<DT>::type;
            const int64_t stride = p.N;
            uint32_t h[4][KS][8];
            int nv[4][KS];
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
                const int col = c0 + 16 * mb + lr;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int kk = 32 * ks + 8 * lg;
                    const int nval = (col < p.N) ? max(0, min(8, r - kk)) : 0;
                    nv[mb][ks] = nval;
                    const int64_t e0 = nval ? (int64_t)kk * p.N + col : 0;
                    const LORA_GLOBAL ET* src = gptr(reinterpret_cast<const ET*>(wbase)) + e0;
#pragma unroll
                    for (int i = 0; i < 8; ++i) h[mb][ks][i] = src[(i < nval ? i : 0) * stride];
                }
            }
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) wf[mb][ks] = GatherElem<DT>::frag(h[mb][ks], nv[mb][ks]);
        }
        if (threadIdx.x < ROWS) s_row[threadIdx.x] = my_row;
        __syncthreads();

        // 3. V rows of the whole tile (converted below), then the y rows of the
        //    first kYBuf steps.  (The pitch of V is a multiple of 8 and >= r_max,
        //    so 8 values from any rank group that starts below r stay inside the row.)
        f32x4_t vq[NF][2];
        bool vok[NF];
#pragma unroll
        for (int i = 0; i < NF; ++i) {
            const int f = threadIdx.x + kThreads * i;
            const int row = 16 * (f / (KS * kWave)) + (f & 15);
            const int kk = 32 * ((f / kWave) % KS) + 8 * ((f >> 4) & 3);
            vok[i] = row < nrows && kk < r;
            const int64_t vrow = p.v_by_pos ? pos0 + (row < nrows ? row : 0) : s_row[row];
            const LORA_GLOBAL f32x4_t* src = gptr(reinterpret_cast<const f32x4_t*>(p.v + vrow * p.ldv + (vok[i] ? kk : 0)));
            vq[i][0] = src[0];
            vq[i][1] = src[1];
        }
        const bool col_ok = c0 + yc < p.N;
        const int ycol = col_ok ? c0 + yc : 0;
        u32x4_t yq[kYBuf][2][YQ];
        auto load_y = [&](u32x4_t (&dst)[2][YQ], int st) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int64_t row = s_row[16 * st + 8 * u + yr];
                const LORA_GLOBAL u32x4_t* src =
                    gptr(reinterpret_cast<const u32x4_t*>(ybase + (row * p.ldy + ycol) * EB));
                // y is read once and written once: streaming (nontemporal) accesses
#pragma unroll
                for (int q = 0; q < YQ; ++q) dst[u][q] = __builtin_nontemporal_load(src + q);
            }
        };
#pragma unroll
        for (int b = 0; b < kYBuf; ++b)
            if (b < STEPS) load_y(yq[b], b < nst ? b : 0);

        // 4. V fragments of the tile -> LDS.
#pragma unroll
        for (int i = 0; i < NF; ++i) {
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

        // 5. 16 rows at a time: MFMA, accumulators to the row-contiguous layout
        //    through LDS, y += s * acc with one rounding, then the y loads of
        //    the step kYBuf ahead go into the freed registers.
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
            if (st < nst) {
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
                // D[m][n] of block mb: column 16 mb + m, row n; this lane has m = 4 lg + i, n = lr.
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) *reinterpret_cast<f32x4_t*>(tw + lr * kTPitch + 16 * mb + 4 * lg) = acc[mb];
                __builtin_amdgcn_wave_barrier();
                u32x4_t(&yb)[2][YQ] = yq[st % kYBuf];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int row_in_tile = 16 * st + 8 * u + yr;
                    const f32x4_t a0 = *reinterpret_cast<const f32x4_t*>(tw + (8 * u + yr) * kTPitch + yc);
                    const f32x4_t a1 = *reinterpret_cast<const f32x4_t*>(tw + (8 * u + yr) * kTPitch + yc + 4);
                    float yv[8];
                    E::unpack8(&yb[u][0], yv);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        yv[e] = yv[e] + s * a0[e];
                        yv[4 + e] = yv[4 + e] + s * a1[e];
                    }
                    if (col_ok && row_in_tile < nrows) {
                        const int64_t row = s_row[row_in_tile];
                        E::store8_nt(ybase + (row * p.ldy + ycol) * EB, yv);
                    }
                }
                __builtin_amdgcn_wave_barrier();
                if (st + kYBuf < STEPS && st + kYBuf < nst) load_y(yb, st + kYBuf);
            }
        }
        __syncthreads();  // s_row / s_frag are rewritten by the next task
    }
}

template <int DT, bool TRANS_W, int KS>
__global__ __launch_bounds__(kExpandWaves * kWave) __attribute__((amdgpu_waves_per_eu(KS == 4 ? 2 : 3)))
void expand_kernel(ExpandParams p) {
    __shared__ __attribute__((aligned(16))) char s_lds[ExpandLds<KS>::kBytes];
    expand_body<DT, TRANS_W, KS>(p, blockIdx.x, gridDim.x, s_lds);
}

}  // namespace lora
