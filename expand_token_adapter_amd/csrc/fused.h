// fused.h -- one-launch forward: y += s B (A x) for batches of short row groups (gfx950).
//
// h(x) = W x + B A x with each row applying its own adapter (MOLT section 2.1;
// DeltaServe section 2.2, multi-LoRA batching).  The split path runs the
// shrink (K split into slices), the sum of the slices and the expand as three
// launches with v in HBM between them; that suits tiles of many rows, whose
// y traffic needs the whole chip.  When adapters have few rows each (decode),
// the work is the weights A_a and B_a plus launch latency, and a workgroup can
// carry a tile from x to y.  A task = (64-row tile, one of `nsplit` column
// ranges of d_out):
//   phase 1  v = A_a x for the tile's rows and ranks (16 NMB of them).  The
//            waves cover the tile's 16-row blocks (1, 2 or 4 of them) times
//            equal parts of d_in (8, 4 or 2), with several 32-element K chunks
//            in flight; the parts are added in order through LDS.  v stays in
//            LDS (the task of column range 0 also writes it out on request).
//            Each task of a tile computes v itself: A_a is read once per
//            column range (from L2 after the first).  The weight block and y
//            rows of the task's first output chunk are requested before phase
//            1 starts: they do not depend on v.
//   phase 2  the waves walk the range's 64-column chunks (up to 32 KS ranks):
//            for bf16 with KS <= 2 the next chunk's weight block (and, for
//            KS = 1 and at most two slices, its y rows) is in flight while
//            the current chunk's MFMA tiles (16 columns x 16 rows, v as hi/lo
//            bf16 fragments) are added to y in fp32 and rounded once.
// Several projections that read the same x (multi-slice: e.g. the q, k and v
// projections, each with its own adapters; DeltaServe section 4.1 adapts all
// attention projections) go through one launch: phase 1 multiplies each x
// chunk it loads by the A blocks of every slice (x read once per tile for all
// of them), and phase 2 walks the output chunks of all slices, one after the
// other.
// The arithmetic per output is the split path's: fp32 accumulation, MFMA
// 16x16x32 bf16 (fp32 operands split into hi/lo bf16 pairs), one rounding of
// y.  Only the association of the sum over d_in differs, and it is fixed by
// the tile's row count: results are bit-reproducible.
#pragma once

#include "device_common.h"

namespace lora {

constexpr int kFusedWaves = 8;
constexpr int kFusedThreads = kFusedWaves * kWave;
constexpr int kFusedPitch = 68;  // LDS pitch (floats) of a 16-row transpose buffer

constexpr int kFusedMaxSlices = 3;

// One projection (slice) of a fused call.
struct FusedSlice {
    const lora_adapter* adapters;  // this projection's adapter table
    void* y;                       // [row][ldy], rows through perm
    int64_t ldy;
    float* v;                      // optional [row][ldv]: v as lora_shrink writes it
    int64_t ldv;
    int32_t N;                     // d_out of the projection
    int32_t ch0;                   // its first 64-column chunk in the concatenated range
};

struct FusedParams {
    const void* x;       // [row][ldx], rows through perm
    int64_t ldx;
    int32_t K;           // d_in
    int32_t r_max;       // over every slice's adapters
    const int32_t* perm;
    const int32_t* sched;
    int64_t tiles64_off;
    int32_t nsplit;      // column ranges per tile
    int32_t nch;         // 64-column chunks of all slices together
    FusedSlice sl[kFusedMaxSlices];
    int32_t* err;
};

template <int DT, int KS, int S>
struct FusedLds {
    static constexpr int NMB = 2 * KS;
    static constexpr int kTBytes = kFusedWaves * 16 * kFusedPitch * 4;  // phase 2 transposes
    static constexpr int kRedBytes = 7 * NMB * kWave * 16;             // phase 1: up to 7 parts of one row block
    static constexpr int kScratch = kTBytes > kRedBytes ? kTBytes : kRedBytes;
    static constexpr int kFragSlice = 4 * KS * kWave * 2;               // 16-byte quads: v as MFMA B fragments
    static constexpr int kFrag = S * kFragSlice * 16;
    static constexpr int kVPitch = 32 * KS + 4;                         // floats
    static constexpr int kVSlice = 64 * kVPitch;                        // floats
    static constexpr int kV = S * kVSlice * 4;
    static constexpr int kBytes = kScratch + kFrag + kV + 64 * 4;
    static_assert(kBytes <= 160 * 1024, "LDS of one workgroup");
};

// Value of slice s (uniform) from a small array indexed by constants only.
template <int S, typename T>
__device__ __forceinline__ T slice_pick(int s, const T (&a)[S]) {
    if constexpr (S == 1) return a[0];
    else if constexpr (S == 2) return s == 0 ? a[0] : a[1];
    else return s == 0 ? a[0] : (s == 1 ? a[1] : a[2]);
}

// KS: 32-rank steps of phase 2 (32 KS >= r_max); NMB: 16-rank blocks of
// phase 1 (16 NMB >= r_max, NMB <= 2 KS); S: slices (projections sharing x).
template <int DT, int KS, int NMB, int S>
__global__ __launch_bounds__(kFusedThreads) __attribute__((amdgpu_waves_per_eu(2)))
void fused_forward_kernel(FusedParams p) {
    using F = Frag<DT>;
    using E = Elem<DT>;
    using O = F32Operand<DT>;
    using L = FusedLds<DT, KS, S>;
    constexpr int EB = F::kBytes;
    constexpr int YQ = EB / 2;          // 16-byte quads per 8 elements
    constexpr int NF = (4 * KS * kWave + kFusedThreads - 1) / kFusedThreads;  // v fragments built per thread
    // K chunks in flight per wave in phase 1 (each: an x fragment and S x NMB
    // weight fragments); the next chunk's weight block and y rows in flight in
    // phase 2 (where the registers allow it)
    constexpr int kUnits = 1 + S * NMB;
    constexpr int NPF = S == 1 ? (DT == LORA_BF16 ? (NMB == 1 ? 8 : (NMB <= 2 ? 4 : 2)) : (NMB <= 2 ? 2 : 1))
                               : (DT == LORA_BF16 ? (12 / kUnits > 1 ? 12 / kUnits : 1) : 1);
    static_assert(NMB >= 1 && NMB <= 2 * KS, "phase 1 covers at most the ranks of phase 2");
    static_assert(S >= 1 && S <= kFusedMaxSlices, "slices");
    constexpr bool PFW = DT == LORA_BF16 && KS <= 2;  // next chunk's weight block in flight
    constexpr bool PFY = DT == LORA_BF16 && KS == 1 && S < 3;  // and its y rows
    static_assert(sizeof(O) == 32, "fragment pair is two quads");
    __shared__ __attribute__((aligned(16))) char s_mem[L::kBytes];
    char* scratch = s_mem;
    u32x4_t* s_frag = reinterpret_cast<u32x4_t*>(s_mem + L::kScratch);
    float* s_v = reinterpret_cast<float*>(s_mem + L::kScratch + L::kFrag);
    int32_t* s_row = reinterpret_cast<int32_t*>(s_mem + L::kScratch + L::kFrag + L::kV);

    const int wave = wave_id();
    const int lane = threadIdx.x & (kWave - 1);
    const int lr = lane & 15;
    const int lg = lane >> 4;
    const int yr = lane >> 3;       // phase 2: row (and row + 8) of a step in the row-contiguous layout
    const int yc = 8 * (lane & 7);  // phase 2: first column of the chunk in that layout
    const int ntiles = p.sched[1];
    const int64_t ntasks = (int64_t)ntiles * p.nsplit;
    const TaskSlice ts = xcd_slice(ntasks, 1, 0);
    const int nkc = (p.K + 31) / 32;          // 32-element K chunks
    const int nch = p.nch;                    // 64-column chunks of all slices
    float* tw = reinterpret_cast<float*>(scratch) + wave * 16 * kFusedPitch;
    // per-slice constants (arrays indexed by constants or through slice_pick)
    char* ybase_s[S];
    int64_t ldy_s[S];
    int N_s[S], ch0_s[S];
#pragma unroll
    for (int q = 0; q < S; ++q) {
        ybase_s[q] = static_cast<char*>(p.sl[q].y);
        ldy_s[q] = p.sl[q].ldy;
        N_s[q] = p.sl[q].N;
        ch0_s[q] = p.sl[q].ch0;
    }
    auto slice_of = [&](int ch) {  // slice of a chunk of the concatenated range
        int q = 0;
#pragma unroll
        for (int k = 1; k < S; ++k) q += ch >= ch0_s[k] ? 1 : 0;
        return q;
    };

    for (int64_t task = ts.begin; task < ts.end; task += ts.stride) {
        const int tile = (int)(task / p.nsplit);
        const int split = (int)(task % p.nsplit);
        const TileRec rec = load_tile(p.sched, p.tiles64_off, tile);
        // each slice's adapter entry; a bad one is counted and its slice skipped
        // (its operands then point at x, valid memory, and nothing is stored)
        bool ok_s[S];
        int r_s[S];
        float sc_s[S];
        const char* A_s[S];
        const char* B_s[S];
        bool any = false;
#pragma unroll
        for (int q = 0; q < S; ++q) {
            const lora_adapter ad = load_adapter(p.sl[q].adapters, rec.adapter);
            ok_s[q] = adapter_ok(ad, p.r_max);
            if (!ok_s[q] && split == 0 && threadIdx.x == 0) atomicAdd(p.err, 1);
            r_s[q] = ok_s[q] ? ad.rank : 1;
            sc_s[q] = ad.scale;
            A_s[q] = ok_s[q] ? static_cast<const char*>(ad.A) : static_cast<const char*>(p.x);
            B_s[q] = ok_s[q] ? static_cast<const char*>(ad.B) : static_cast<const char*>(p.x);
            any |= ok_s[q];
        }
        if (!any) continue;
        const int nrows = rec.rows;
        const int nst = (nrows + 15) >> 4;
        if (threadIdx.x < 64)
            s_row[threadIdx.x] = p.perm[rec.pos0 + ((int)threadIdx.x < nrows ? (int)threadIdx.x : 0)];
        __syncthreads();

        // Phase 2 walks the chunks of this task's column range, ch = lo + wave,
        // lo + wave + 8, ...  Its first chunk's weight block and y rows do not
        // depend on v: they are issued here, before phase 1.
        const int ch_lo = split * nch / p.nsplit, ch_hi = (split + 1) * nch / p.nsplit;
        // Rows of B_a in whole 16-byte units: the loads only clamp addresses
        // (columns past N or the range read B_a's first unit and are not
        // stored); groups past rank r are zeroed where they are used, so the
        // next chunk's loads are not waited for early.  Otherwise elements are
        // read one by one.
        auto load_w = [&](int ch, F (&wf)[4][KS]) {
            const int q = slice_of(ch);
            const int r = slice_pick(q, r_s);
            const char* B = slice_pick(q, B_s);
            const bool sok = ch < ch_hi && slice_pick(q, ok_s);
            const int N = slice_pick(q, N_s);
            const int c0 = 64 * (ch - slice_pick(q, ch0_s));
            const bool b_units = (r & 7) == 0;
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
                const int col = c0 + 16 * mb + lr;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int kk = 32 * ks + 8 * lg;
                    const bool ok = sok && col < N && kk < r;
                    const char* src = B + (ok ? (int64_t)col * r + kk : 0) * EB;
                    wf[mb][ks] = b_units ? F::load(src) : F::load_strided(src, 1, ok ? wkeep(r, kk) : 0);
                }
            }
        };
        // y rows of a chunk (the tile's 16-row steps; columns past N and
        // chunks past the range re-read column 0 of the rows)
        auto load_y_step = [&](int ch, int st, u32x4_t (&yq)[2][YQ]) {
            const int q = slice_of(ch);
            const int c = 64 * (ch - slice_pick(q, ch0_s)) + yc;
            const int col = ch < ch_hi && c < slice_pick(q, N_s) ? c : 0;
            const char* yb = slice_pick(q, ybase_s);
            const int64_t ldy = slice_pick(q, ldy_s);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int64_t row = s_row[16 * st + 8 * u + yr];
                const LORA_GLOBAL u32x4_t* src =
                    gptr(reinterpret_cast<const u32x4_t*>(yb + (row * ldy + col) * EB));
#pragma unroll
                for (int q = 0; q < YQ; ++q) yq[u][q] = __builtin_nontemporal_load(src + q);
            }
        };
        auto load_y = [&](int ch, u32x4_t (&yq)[4][2][YQ]) {
#pragma unroll
            for (int st = 0; st < 4; ++st)
                if (st < nst) load_y_step(ch, st, yq[st]);
        };
        // (the empty asm statements with a memory clobber keep the prefetches
        // where they are issued, as in phase 1)
        F wcur[4][KS], wnext[4][KS];
        u32x4_t ycur[4][2][YQ], ynext[4][2][YQ];
        if constexpr (PFW) load_w(ch_lo + wave, wcur);
        if constexpr (PFY) load_y(ch_lo + wave, ycur);
        asm volatile("" ::: "memory");

        // ---- phase 1: v = A x.  A operand: rank rows of A_a, B operand: x rows.
        {
            const int nrb = nst == 1 ? 1 : (nst == 2 ? 2 : 4);  // row blocks
            const int nkp = kFusedWaves / nrb;                  // parts of d_in
            const int rb = wave % nrb;
            const int kp = wave / nrb;
            const int kc0 = kp * nkc / nkp, kc1 = (kp + 1) * nkc / nkp;
            const char* xr = static_cast<const char*>(p.x) + (int64_t)s_row[16 * rb + lr] * p.ldx * EB;
            f32x4_t acc[S][NMB];
#pragma unroll
            for (int q = 0; q < S; ++q)
#pragma unroll
                for (int mb = 0; mb < NMB; ++mb) acc[q][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            // Loads only clamp addresses: rank rows past r read row r - 1 (their
            // sums are dropped below), K past the part reads K 0.  The x operand
            // of a chunk past the part is zeroed where it is used, so that the
            // chunks in flight are not waited for when they are issued.
            auto load_chunk = [&](int kc, F& xf, F (&af)[S][NMB]) {
                const int k = 32 * kc + 8 * lg;
                const int ks = kc < kc1 && k < p.K ? k : 0;
                xf = F::load(xr + (int64_t)ks * EB);
#pragma unroll
                for (int q = 0; q < S; ++q)
#pragma unroll
                    for (int mb = 0; mb < NMB; ++mb) {
                        const int rk = 16 * mb + lr;
                        af[q][mb] = F::load(A_s[q] + ((int64_t)(rk < r_s[q] ? rk : r_s[q] - 1) * p.K + ks) * EB);
                    }
                // keeps the loads where they are issued: without it the loads of
                // the prologue and of the loop body merge into one load at the
                // top of the loop, which is then waited for at once
                asm volatile("" ::: "memory");
            };
            F xq[NPF];
            F aq[NPF][S][NMB];
#pragma unroll
            for (int i = 0; i < NPF; ++i) load_chunk(kc0 + i, xq[i], aq[i]);
            for (int kc = kc0; kc < kc1; kc += NPF) {
#pragma unroll
                for (int i = 0; i < NPF; ++i) {
                    const F xv = xq[i].masked((kc + i < kc1) & (32 * (kc + i) + 8 * lg < p.K));
#pragma unroll
                    for (int q = 0; q < S; ++q)
#pragma unroll
                        for (int mb = 0; mb < NMB; ++mb) acc[q][mb] = mma(aq[i][q][mb], xv, acc[q][mb]);
                    load_chunk(kc + NPF + i, xq[i], aq[i]);
                }
            }
            // D rows 4 (l / 16) + i of block mb = ranks, column l % 16 = row of the block.
            // Parts 1 .. nkp - 1 go through LDS; part 0 adds them in order (slice by slice).
            f32x4_t* red = reinterpret_cast<f32x4_t*>(scratch);
#pragma unroll
            for (int q = 0; q < S; ++q) {
                if (kp > 0) {
#pragma unroll
                    for (int mb = 0; mb < NMB; ++mb)
                        red[(((kp - 1) * nrb + rb) * NMB + mb) * kWave + lane] = acc[q][mb];
                }
                __syncthreads();
                if (kp == 0) {
                    const int row = 16 * rb + lr;
                    const int r = r_s[q];
                    float* sv = s_v + q * L::kVSlice;
                    const FusedSlice& sl = p.sl[q];
                    for (int pt = 1; pt < nkp; ++pt)
#pragma unroll
                        for (int mb = 0; mb < NMB; ++mb)
                            acc[q][mb] += red[(((pt - 1) * nrb + rb) * NMB + mb) * kWave + lane];
#pragma unroll
                    for (int mb = 0; mb < NMB; ++mb) {
                        f32x4_t sum = acc[q][mb];
                        const int rk = 16 * mb + 4 * lg;
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (rk + i >= r) sum[i] = 0.f;
                        *reinterpret_cast<f32x4_t*>(sv + row * L::kVPitch + rk) = sum;
                        // v as lora_shrink writes it: ranks < r, zeros up to round_up(r, 8)
                        if (sl.v && ok_s[q] && split == 0 && row < nrows && rk < (r + 7) / 8 * 8)
                            *gptr(reinterpret_cast<f32x4_t*>(sl.v + (int64_t)s_row[row] * sl.ldv + rk)) = sum;
                    }
                    // ranks past the blocks of phase 1 (and so past r) enter phase 2 as zeros
#pragma unroll
                    for (int mb = NMB; mb < 2 * KS; ++mb)
                        *reinterpret_cast<f32x4_t*>(sv + row * L::kVPitch + 16 * mb + 4 * lg) =
                            f32x4_t{0.f, 0.f, 0.f, 0.f};
                }
                __syncthreads();
            }
        }

        // ---- v fragments: step st (16 rows), rank step ks: lane (row lr, ranks 32 ks + 8 lg .. + 7),
        //      for the tile's steps only.
#pragma unroll
        for (int q = 0; q < S; ++q)
#pragma unroll
            for (int i = 0; i < NF; ++i) {
                const int f = threadIdx.x + kFusedThreads * i;
                const int st = f / (KS * kWave);
                if (f < 4 * KS * kWave && st < nst) {
                    const int ks = (f / kWave) % KS;
                    const int row = 16 * st + (f & 15);
                    const int kk = 32 * ks + 8 * ((f >> 4) & 3);
                    float fv[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) fv[e] = s_v[q * L::kVSlice + row * L::kVPitch + kk + e];
                    const O o = O::make(fv);
                    const u32x4_t* oq = reinterpret_cast<const u32x4_t*>(&o);
                    s_frag[q * L::kFragSlice + 2 * f] = oq[0];
                    s_frag[q * L::kFragSlice + 2 * f + 1] = oq[1];
                }
            }
        __syncthreads();

        // ---- phase 2: chunks of this task's column range, ch = lo + wave, lo + wave + 8, ...
        for (int ch = ch_lo + wave; ch < ch_hi; ch += kFusedWaves) {
            if constexpr (PFW)
                load_w(ch + kFusedWaves, wnext);
            else
                load_w(ch, wcur);
            // without prefetch the y rows of one step are read just before
            // they are needed (fewer registers live)
            if constexpr (PFY) load_y(ch + kFusedWaves, ynext);
            asm volatile("" ::: "memory");
            const int q = slice_of(ch);
            const int r = slice_pick(q, r_s);
            const float s = slice_pick(q, sc_s);
            const bool b_units = (r & 7) == 0;
            const int c = 64 * (ch - slice_pick(q, ch0_s)) + yc;
            const bool col_ok = c < slice_pick(q, N_s) && slice_pick(q, ok_s);
            char* ybase = slice_pick(q, ybase_s);
            const int64_t ldy = slice_pick(q, ldy_s);
            const u32x4_t* frag = s_frag + q * L::kFragSlice;
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                if (st < nst) {
                    if constexpr (!PFY) load_y_step(ch, st, ycur[st]);
                    f32x4_t acc[4];
#pragma unroll
                    for (int mb = 0; mb < 4; ++mb) acc[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        const int f = (st * KS + ks) * kWave + lane;
                        O o;
                        u32x4_t* oq = reinterpret_cast<u32x4_t*>(&o);
                        oq[0] = frag[2 * f];
                        oq[1] = frag[2 * f + 1];
                        const bool keep = !b_units || 32 * ks + 8 * lg < r;
#pragma unroll
                        for (int mb = 0; mb < 4; ++mb) acc[mb] = o.mma_right(wcur[mb][ks].masked(keep), acc[mb]);
                    }
                    // D[m][n] of block mb: column 16 mb + m, row n; this lane has m = 4 lg + i, n = lr.
#pragma unroll
                    for (int mb = 0; mb < 4; ++mb)
                        *reinterpret_cast<f32x4_t*>(tw + lr * kFusedPitch + 16 * mb + 4 * lg) = acc[mb];
                    __builtin_amdgcn_wave_barrier();
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const int row_in_tile = 16 * st + 8 * u + yr;
                        const f32x4_t a0 = *reinterpret_cast<const f32x4_t*>(tw + (8 * u + yr) * kFusedPitch + yc);
                        const f32x4_t a1 =
                            *reinterpret_cast<const f32x4_t*>(tw + (8 * u + yr) * kFusedPitch + yc + 4);
                        float yv[8];
                        E::unpack8(&ycur[st][u][0], yv);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            yv[e] = yv[e] + s * a0[e];
                            yv[4 + e] = yv[4 + e] + s * a1[e];
                        }
                        if (col_ok && row_in_tile < nrows)
                            E::store8_nt(ybase + ((int64_t)s_row[row_in_tile] * ldy + c) * EB, yv);
                    }
                    __builtin_amdgcn_wave_barrier();
                }
            }
            if constexpr (PFW) {
#pragma unroll
                for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) wcur[mb][ks] = wnext[mb][ks];
            }
            if constexpr (PFY) {
#pragma unroll
                for (int st = 0; st < 4; ++st)
#pragma unroll
                    for (int u = 0; u < 2; ++u)
#pragma unroll
                        for (int q = 0; q < YQ; ++q) ycur[st][u][q] = ynext[st][u][q];
            }
        }
        __syncthreads();  // s_row, s_v and s_frag are rewritten by the next task
    }
}

}  // namespace lora
