// fused_decode.h -- one-launch forward for decode batches of adapters of rank
// <= 16 (gfx950, bf16), for one to three projections that read the same x.
//
// h(x) = W x + B A x with each row applying its own adapter (MOLT section 2.1;
// DeltaServe section 2.2).  When every adapter serves a few rows and the
// weights are small (decode), the work is a handful of dependent memory round
// trips per tile, and the kernel is built to have as few of them as possible:
// a workgroup = (16-row tile, one of `nsplit` column ranges of the output
// chunks) with 16 waves, and every load it needs -- the tile's A_a blocks and
// x rows for phase 1, the first output chunk's B_a block and y rows for
// phase 2 -- is issued as soon as the tile record, then the adapter entries
// and the row indices (scalar loads, requested together) have arrived: three
// round trips in all, plus the result's store.
//   phase 1  v = A_a x: wave w takes the w-th sixteenth of d_in's 32-element
//            steps and loads its x fragments and every slice's A fragments
//            straight into registers in MFMA operand layout (lane (lr, lg):
//            rank row / tile row lr, elements 8 lg .. 8 lg + 7 of the step),
//            a round of steps in flight at a time; the waves' 16x16 tiles are
//            added through LDS in wave order.  v stays in LDS (the task of
//            column range 0 also writes it out on request).
//   phase 2  the waves take the range's 64-column chunks in turn (chunk
//            wave, wave + 16, ...; the chunks of all slices one after the
//            other), each chunk's B_a block and y rows in flight while the
//            previous chunk is added; the MFMA's 32-deep reduction carries two
//            16-rank groups, each owning 16 columns (the decode expand's
//            layout for ranks <= 16), so every loaded byte of B_a is used;
//            results reach y through a per-wave LDS transpose and are rounded
//            once.
// The tasks of one tile sit on one XCD (their A_a reads after the first hit
// its L2); tiles are spread over the XCDs in tile order.
// Sums run in a fixed order (per 32-element step inside one MFMA, steps in
// order within a wave, waves in order), the same for every slice count:
// results are bit-reproducible, and a slice computed with others equals the
// slice computed alone bit for bit.
#pragma once

#include "device_common.h"

namespace lora {

constexpr int kFdWaves = 16;
constexpr int kFdThreads = kFdWaves * kWave;
constexpr int kFdChunk = 64;    // phase 2: output columns per chunk
constexpr int kFdPitch = 68;    // floats per row of a wave's transpose buffer
constexpr int kFdMaxRank = 16;
constexpr int kFdMaxSlices = 3;

// 32-element steps per wave and round of phase 1: x and S A fragments per
// step, at most 16 loads (64 registers) in flight.
template <int S>
constexpr int fd_steps() { return S == 1 ? 8 : (S == 2 ? 5 : 4); }

struct FdSlice {
    const lora_adapter* adapters;  // this projection's adapter table
    void* y;                       // [row][ldy], rows through perm
    int64_t ldy;
    uint32_t y_bytes;              // bytes from y to the end of its last row (< 2^31)
    int32_t N;                     // d_out of the projection
    float* v;                      // optional [row][ldv]: v as lora_shrink writes it
    int64_t ldv;
    int32_t ch0;                   // its first 64-column chunk in the concatenated range
};

struct FdParams {
    const void* x;        // [row][ldx], rows through perm
    int64_t ldx;
    uint32_t x_bytes;     // bytes from x to the end of its last row (< 2^31)
    int32_t K;            // d_in
    int32_t r_max;        // <= 16, over every slice's adapters
    const int32_t* perm;
    const int32_t* sched;
    int64_t tiles16_off;
    int32_t max_tiles;    // the host's bound on the 16-row tile count
    int32_t nsplit;       // column ranges per tile
    int32_t nch;          // 64-column chunks of all slices together
    FdSlice sl[kFdMaxSlices];
    int32_t* err;
};

// Value of slice q (uniform) from a small array indexed by constants only.
template <int S, typename T>
__device__ __forceinline__ T fd_pick(int q, const T (&a)[S]) {
    if constexpr (S == 1) return a[0];
    else if constexpr (S == 2) return q == 0 ? a[0] : a[1];
    else return q == 0 ? a[0] : (q == 1 ? a[1] : a[2]);
}

template <int S>
__global__ __launch_bounds__(kFdThreads) void fused_decode_kernel(FdParams p) {
    using F = Frag<LORA_BF16>;
    using E = Elem<LORA_BF16>;
    using O = F32Operand<LORA_BF16>;
    constexpr int EB = 2;
    constexpr int NST = fd_steps<S>();
    // phase 1's per-wave tiles (per slice), then (reused) phase 2's transpose buffers
    constexpr int kRedBytes = S * kFdWaves * kWave * 16;
    constexpr int kTBytes = kFdWaves * 16 * kFdPitch * 4;
    __shared__ __attribute__((aligned(16))) char s_mem[kRedBytes > kTBytes ? kRedBytes : kTBytes];
    __shared__ __attribute__((aligned(16))) float s_v[S][16][kFdMaxRank + 4];  // v[slice][row][rank]

    const int wave = wave_id();
    const int lane = threadIdx.x & (kWave - 1);
    const int lr = lane & 15;
    const int lg = lane >> 4;

    // Task of this workgroup: tile t goes to XCD t % 8, its nsplit ranges to
    // consecutive slots of that XCD; slots are handed out in tile order.
    const int b = blockIdx.x;
    const int j = b / kNumXcd;
    const int c = j % p.nsplit;
    const int t = (j / p.nsplit) * kNumXcd + b % kNumXcd;
    if (t >= p.max_tiles) return;
    // The record (in the schedule for every t below the bound) is requested
    // together with the tile count: the empty asm reads both before the test.
    const TileRec rec = load_tile(p.sched, p.tiles16_off, t);
    const int n16 = *cptr(p.sched);
    asm volatile("" ::"s"(rec.adapter), "s"(rec.pos0), "s"(rec.rows), "s"(n16));
    if (t >= n16) return;
    const int nrows = rec.rows;
    // The tile's rows (rows past it repeat its first) through scalar loads,
    // requested with the adapter entries (the empty asm below reads both
    // before the entries are tested): they do not queue behind the vector
    // loads of the other workgroups' weights.
    int32_t prow[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) prow[k] = *cptr(p.perm + rec.pos0 + (k < nrows ? k : 0));
    // each slice's adapter entry; a bad one is counted and its slice skipped
    bool ok_s[S];
    int r_s[S];
    float sc_s[S];
    const char* A_s[S];
    const char* B_s[S];
    bool any = false;
    lora_adapter ad_s[S];
#pragma unroll
    for (int q = 0; q < S; ++q) ad_s[q] = load_adapter(p.sl[q].adapters, rec.adapter);
    asm volatile("" ::"s"(prow[0]), "s"(prow[1]), "s"(prow[2]), "s"(prow[3]), "s"(prow[4]), "s"(prow[5]),
                 "s"(prow[6]), "s"(prow[7]), "s"(prow[8]), "s"(prow[9]), "s"(prow[10]), "s"(prow[11]),
                 "s"(prow[12]), "s"(prow[13]), "s"(prow[14]), "s"(prow[15]), "s"(ad_s[0].rank),
                 "s"(ad_s[S - 1].rank));
#pragma unroll
    for (int q = 0; q < S; ++q) {
        const lora_adapter& ad = ad_s[q];
        ok_s[q] = adapter_ok(ad, p.r_max);
        if (!ok_s[q] && c == 0 && threadIdx.x == 0) atomicAdd(p.err, 1);
        r_s[q] = ok_s[q] ? ad.rank : 0;
        sc_s[q] = ad.scale;
        A_s[q] = static_cast<const char*>(ad.A);
        B_s[q] = static_cast<const char*>(ad.B);
        any |= ok_s[q];
    }
    if (!any) return;
    // lane lr takes row lr
    int32_t row_lr = prow[0];
#pragma unroll
    for (int k = 1; k < 16; ++k) row_lr = lr == k ? prow[k] : row_lr;

    // ---- phase 2 addressing (G = 2 rank groups of 16 per MFMA)
    // Chunk columns c0 .. c0 + 63 of slice q; MFMA nb (0, 1) covers columns
    // c0 + 32 nb .. + 31: lane (lr, lg) loads B[c0 + 32 nb + 16 g + lr][j0 ..
    // j0 + 7], g = lg / 2, j0 = 8 (lg % 2).  y layout: lane (yr, yc) holds
    // rows yr and yr + 8, columns c0 + yc .. + 7.
    const int ch0 = (int)((uint32_t)(p.nch * c) / (uint32_t)p.nsplit);  // nch * nsplit < 2^31 (host)
    const int ch1 = (int)((uint32_t)(p.nch * (c + 1)) / (uint32_t)p.nsplit);
    // per-slice constants (arrays indexed by constants or through fd_pick)
    int N_s[S], cb_s[S];
    char* y_s[S];
    int64_t ldy_s[S];
    uint32_t yb_s[S];
#pragma unroll
    for (int q = 0; q < S; ++q) {
        N_s[q] = p.sl[q].N;
        cb_s[q] = p.sl[q].ch0;
        y_s[q] = static_cast<char*>(p.sl[q].y);
        ldy_s[q] = p.sl[q].ldy;
        yb_s[q] = p.sl[q].y_bytes;
    }
    auto slice_of = [&](int ch) {
        int q = 0;
#pragma unroll
        for (int k = 1; k < S; ++k) q += ch >= cb_s[k] ? 1 : 0;
        return q;
    };
    const int g2 = lg >> 1;
    const int j0 = 8 * (lg & 1);
    const int yr = lane >> 3;
    const int yc = 8 * (lane & 7);
    int64_t yrow0 = prow[0], yrow1 = prow[8];  // rows yr and yr + 8
#pragma unroll
    for (int k = 1; k < 8; ++k) {
        yrow0 = yr == k ? prow[k] : yrow0;
        yrow1 = yr == k ? prow[k + 8] : yrow1;
    }
    // this wave's chunks: ch0 + wave, ch0 + wave + 16, ...; -1: none
    auto chunk_of = [&](int k) {
        const int ch = ch0 + wave + kFdWaves * k;
        return ch < ch1 ? ch : -1;
    };
    auto load_w = [&](int ch, F (&wf)[2]) {
        const int q = ch >= 0 ? slice_of(ch) : 0;
        const int r = fd_pick(q, r_s);
        const int N = fd_pick(q, N_s);
        const char* B = fd_pick(q, B_s);
        const bool live = ch >= 0 && fd_pick(q, ok_s);
        const int c0 = kFdChunk * (ch - fd_pick(q, cb_s));
        if ((r & 7) == 0) {  // B rows in whole 16-byte units
            const buf_rsrc_t br = make_rsrc(B, (uint32_t)((int64_t)N * r * EB));
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                const int col = c0 + 32 * nb + 16 * g2 + lr;
                wf[nb].q = buf_load16(br, live ? (uint32_t)(col * r + j0) * EB : kBufOff, 0);
            }
        } else {
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                const int col = c0 + 32 * nb + 16 * g2 + lr;
                const bool ok = live && col < N && j0 < r;
                wf[nb] = F::load_strided(B + (ok ? (int64_t)col * r + j0 : 0) * EB, 1, ok ? wkeep(r, j0) : 0);
            }
        }
    };
    auto load_y = [&](int ch, u32x4_t (&yq)[2]) {
        const int q = ch >= 0 ? slice_of(ch) : 0;
        const buf_rsrc_t yres = make_rsrc(fd_pick(q, y_s), fd_pick(q, yb_s));
        const int c0 = kFdChunk * (ch - fd_pick(q, cb_s));
        const int64_t ldy = fd_pick(q, ldy_s);
        const bool ok = ch >= 0 && fd_pick(q, ok_s) && c0 + yc < fd_pick(q, N_s);
        yq[0] = buf_load16(yres, ok && yr < nrows ? (uint32_t)((yrow0 * ldy + c0 + yc) * EB) : kBufOff, 0);
        yq[1] = buf_load16(yres, ok && yr + 8 < nrows ? (uint32_t)((yrow1 * ldy + c0 + yc) * EB) : kBufOff, 0);
    };

    // ---- phase 1 addressing: this wave's share [sb0, sb1) of d_in's steps
    const int nsteps = (p.K + 31) / 32;
    const int sb0 = nsteps * wave / kFdWaves, sb1 = nsteps * (wave + 1) / kFdWaves;
    const buf_rsrc_t xr = make_rsrc(p.x, p.x_bytes);
    buf_rsrc_t ar[S];
    uint32_t ao[S];
#pragma unroll
    for (int q = 0; q < S; ++q) {
        ar[q] = make_rsrc(A_s[q], (uint32_t)((int64_t)r_s[q] * p.K * EB));
        ao[q] = lr < r_s[q] ? (uint32_t)((int64_t)lr * p.K * EB) + 16u * lg : kBufOff;
    }
    F af[S][NST], xf[NST];
    // steps past this wave's share load nothing (zeros)
    auto issue_a = [&](int st0) {
#pragma unroll
        for (int i = 0; i < NST; ++i)
#pragma unroll
            for (int q = 0; q < S; ++q)
                af[q][i].q = buf_load16(ar[q], st0 + i < sb1 && ao[q] != kBufOff ? ao[q] + (uint32_t)(st0 + i) * 64u
                                                                                   : kBufOff, 0);
    };
    auto issue_x = [&](int st0, uint32_t xo) {
#pragma unroll
        for (int i = 0; i < NST; ++i)
            xf[i].q = buf_load16(xr, st0 + i < sb1 && xo != kBufOff ? xo + (uint32_t)(st0 + i) * 64u : kBufOff, 0);
    };
    f32x4_t acc[S];
#pragma unroll
    for (int q = 0; q < S; ++q) acc[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    auto mma_round = [&](int st0) {
#pragma unroll
        for (int i = 0; i < NST; ++i) {
            // elements past K (the next row's data) are dropped with the x fragment
            const bool ok = 32 * (st0 + i) + 8 * lg < p.K;
            const F xm = xf[i].masked(ok);
#pragma unroll
            for (int q = 0; q < S; ++q) acc[q] = mma(af[q][i], xm, acc[q]);
        }
    };

    // Every load of the tile in one batch: the first chunk's weights, the
    // first round's A and x fragments, the first chunk's y rows.
    F wf[2];
    u32x4_t yq[2];
    const uint32_t xo = lr < nrows ? (uint32_t)((int64_t)row_lr * p.ldx * EB) + 16u * lg : kBufOff;
    load_w(chunk_of(0), wf);
    issue_a(sb0);
    issue_x(sb0, xo);
    load_y(chunk_of(0), yq);
    asm volatile("" ::: "memory");

    // ---- phase 1: v = A x over this wave's share of d_in
    mma_round(sb0);
    for (int st0 = sb0 + NST; st0 < sb1; st0 += NST) {
        issue_a(st0);
        issue_x(st0, xo);
        mma_round(st0);
    }
    // waves' tiles in wave order: D row 4 lg + e = rank, column lr = row;
    // wave q adds slice q's tiles
    f32x4_t* s_red = reinterpret_cast<f32x4_t*>(s_mem);
#pragma unroll
    for (int q = 0; q < S; ++q) s_red[(q * kFdWaves + wave) * kWave + lane] = acc[q];
    lds_barrier();
    if (wave < S) {
        const int q = wave;
        f32x4_t sum = s_red[q * kFdWaves * kWave + lane];
#pragma unroll
        for (int w = 1; w < kFdWaves; ++w) sum += s_red[(q * kFdWaves + w) * kWave + lane];
        const int r = fd_pick(q, r_s);
        const int k = 4 * lg;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (k + e >= r) sum[e] = 0.f;
            s_v[q][lr][k + e] = sum[e];
        }
        // v as lora_shrink writes it (ranks below round_up(r, 8) <= ldv)
        float* v_s[S];
        int64_t ldv_s[S];
#pragma unroll
        for (int qq = 0; qq < S; ++qq) {
            v_s[qq] = p.sl[qq].v;
            ldv_s[qq] = p.sl[qq].ldv;
        }
        float* v = fd_pick(q, v_s);
        if (v != nullptr && fd_pick(q, ok_s) && c == 0 && lr < nrows && k < (r + 7) / 8 * 8)
            *gptr(reinterpret_cast<f32x4_t*>(v + (int64_t)row_lr * fd_pick(q, ldv_s) + k)) = sum;
    }
    lds_barrier();

    // ---- phase 2: y += s B v over the range's chunks
    float* tw = reinterpret_cast<float*>(s_mem) + wave * 16 * kFdPitch;
    const int nk = (ch1 - ch0 - wave + kFdWaves - 1) / kFdWaves;  // chunks of this wave
    for (int k = 0; k < nk; ++k) {
        const int ch = chunk_of(k);
        const int q = slice_of(ch);
        const int c0 = kFdChunk * (ch - fd_pick(q, cb_s));
        const int N = fd_pick(q, N_s);
        // the next chunk's weights and y rows go in flight before this one is used
        F wn[2];
        u32x4_t yn[2];
        load_w(chunk_of(k + 1), wn);
        load_y(chunk_of(k + 1), yn);
        asm volatile("" ::: "memory");
        if (fd_pick(q, ok_s)) {  // wave-uniform
            const int r = fd_pick(q, r_s);
            const float s = fd_pick(q, sc_s);
            // v operand of sub-block sb (rows 8 sb .. 8 sb + 7): lane (lr, lg)
            // holds v[8 sb + lr % 8][j0 .. j0 + 7] when its rank group g2
            // equals the column group lr / 8, else zeros.  D[m][n] lands at
            // row 8 sb + n % 8, column 32 nb + 16 (n / 8) + m (m = 4 lg + e,
            // n = lr).
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {
                if (8 * sb < nrows) {  // wave-uniform
                    const int row = 8 * sb + (lr & 7);
                    const bool on = g2 == (lr >> 3) && row < nrows;
                    float f[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) f[e] = on ? s_v[q][row][j0 + e] : 0.f;
                    const O vo = O::make(f);
#pragma unroll
                    for (int nb = 0; nb < 2; ++nb) {
                        const bool keep = c0 + 32 * nb + 16 * g2 + lr < N && j0 < r;
                        const f32x4_t d = vo.mma_right(wf[nb].masked(keep), f32x4_t{0.f, 0.f, 0.f, 0.f});
                        *reinterpret_cast<f32x4_t*>(tw + (8 * sb + (lr & 7)) * kFdPitch + 32 * nb +
                                                    16 * (lr >> 3) + 4 * lg) = d;
                    }
                }
            }
            __builtin_amdgcn_wave_barrier();
            if (c0 + yc < N) {
                char* ybase = fd_pick(q, y_s);
                const int64_t ldy = fd_pick(q, ldy_s);
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int rt = 8 * u + yr;
                    if (rt < nrows) {
                        const f32x4_t a0 = *reinterpret_cast<const f32x4_t*>(tw + rt * kFdPitch + yc);
                        const f32x4_t a1 = *reinterpret_cast<const f32x4_t*>(tw + rt * kFdPitch + yc + 4);
                        float yv[8];
                        E::unpack8(&yq[u], yv);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            yv[e] = yv[e] + s * a0[e];
                            yv[4 + e] = yv[4 + e] + s * a1[e];
                        }
                        const int64_t row = u == 0 ? yrow0 : yrow1;
                        E::store8_nt(ybase + (row * ldy + c0 + yc) * EB, yv);
                    }
                }
            }
            __builtin_amdgcn_wave_barrier();
        }
        wf[0] = wn[0];
        wf[1] = wn[1];
        yq[0] = yn[0];
        yq[1] = yn[1];
    }
}

}  // namespace lora
