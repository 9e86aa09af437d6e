// contract.h -- token-contraction kernel of the backward: dA and dB (gfx950).
//
// Walks the scheduling records written by the segment builder, so every
// workgroup touches one adapter's weights and that adapter's rows only
// (multi-LoRA batching: each row applies its own adapter, DeltaServe section
// 2.2).  Dense work goes to 16x16 MFMA tiles; every reduction runs in a fixed
// order, so results are bit-reproducible.
#pragma once

#include "device_common.h"

namespace lora {

// Window i (0 <= i < n) of a wave's range, visited from a per-workgroup
// starting point so that concurrent workgroups do not all read the same
// lines at the same time.  The order is fixed per task, so results stay
// bit-reproducible.
__device__ __forceinline__ int rotated(int kc0, int n, int rot, int i) {
    const int j = i + rot;
    return kc0 + (j < n ? j : j - n);
}

// ============================================================== token contraction
//
// For each adapter a with fine-tuning rows, each group of 16 ranks and each
// block of 64 columns (a "tile"):
//   dA_a[k][c] += s_a * sum_rows g[row][k] * x[row][c]      (c < d_in)
//   dB_a[c][k] += s_a * sum_rows dy[row][c] * v[row][k]     (c < d_out)
// The contraction runs over rows, so the row-major x / dy tiles (32 rows x
// 64 columns per wave and step) become MFMA B operands through LDS: bf16
// tiles are stored as loaded and read back transposed with
// ds_read_b64_tr_b16; fp32 tiles are written transposed element by element.
// g and v come rank-major ([k][sorted position]) from the shrink kernel.
//
// Work split ("stream-K"): the work is the list of (tile, 32-row window)
// units, ordered by active adapter, rank group, column block, window; the
// contraction's workgroups (one per CU, four waves each, in the backward's
// x-side launch beside the dX expand) take equal contiguous ranges of it, so
// no CU waits on another's second tile.  Inside a workgroup the waves split
// the windows of each tile they meet into contiguous ranges.  Each wave runs two interleaved streams of windows:
// while one window is multiplied, the next window of the other stream is in
// flight, and the row indices (perm) of each stream are fetched one window
// ahead of its data.  The waves' partial tiles are summed in wave order
// through LDS.  A tile whose windows all fall in one workgroup is added to
// dA / dB there; a tile cut by workgroup boundaries leaves one partial tile
// per workgroup, and contract_fixup_kernel adds those in workgroup order.
// Every sum therefore runs in an order fixed by the shapes alone.

constexpr int kContractMB = 1;    // 16-rank blocks per task
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
    int32_t rgroups;  // ceil(r_max / 16)
    int32_t* err;
    float* fix;       // [grid][2] partial tiles of cut tiles (kFixFloats floats each)
    int32_t* fix_meta;  // [grid][2][kFixMeta]: first unit of the tile (lo, hi; -1: none, -2: empty
                        // range), adapter, rank group, column block, owner
    // backward preemption: when set and *stop != 0 at the start, the
    // workgroup does nothing (null in the forward)
    const int32_t* stop;
};

constexpr int kFixFloats = kContractMB * 4 * kWave * 4;
constexpr int kFixMeta = 8;

// One active adapter's share of the contraction: rank groups x column blocks
// x 32-row windows of its sorted rows (no units for an invalid entry).
struct ContractAct {
    int a, rgroups, nwin, lo, hi;
    int64_t units;
};
__device__ __forceinline__ ContractAct contract_act(const ContractParams& p, int i, int ncb) {
    ContractAct c;
    c.a = p.sched[p.active_off + i];
    const lora_adapter ad = load_adapter(p.adapters, c.a);
    const lora_adapter_grad gr = load_grad(p.grads, c.a);
    const bool ok = adapter_ok(ad, p.r_max) && gr.dA != nullptr && gr.dB != nullptr;
    c.rgroups = ok ? min(p.rgroups, (ad.rank + 16 * kContractMB - 1) / (16 * kContractMB)) : 0;
    c.lo = p.offsets[c.a];
    c.hi = p.offsets[c.a + 1];
    c.nwin = (c.hi - (c.lo & ~31) + 31) / 32;
    c.units = (int64_t)c.rgroups * ncb * c.nwin;
    return c;
}

// The same, for a wave-uniform index: every field wave-uniform (scalar).
__device__ __forceinline__ ContractAct contract_act_uniform(const ContractParams& p, int i, int ncb) {
    ContractAct c = contract_act(p, i, ncb);
    c.a = __builtin_amdgcn_readfirstlane(c.a);
    c.rgroups = __builtin_amdgcn_readfirstlane(c.rgroups);
    c.nwin = __builtin_amdgcn_readfirstlane(c.nwin);
    c.lo = __builtin_amdgcn_readfirstlane(c.lo);
    c.hi = __builtin_amdgcn_readfirstlane(c.hi);
    c.units = uniform64(c.units);
    return c;
}


template <int DT, int NW>
struct ContractLds {
    static constexpr int EB = Frag<DT>::kBytes;
    // per wave: two window tiles
    static constexpr int kTileBytes = DT == LORA_BF16 ? 32 * kQPitch * 2 : 64 * kCtPitch * 4;
    static constexpr int kTransBytes = NW * 2 * kTileBytes;
    static constexpr int kRedBytes = NW * kContractMB * 4 * kWave * 16;
    static constexpr int kBytes = kTransBytes > kRedBytes ? kTransBytes : kRedBytes;
};

// Raw loads of one 32-row window: this lane's 4 rows x 8 columns of Q and,
// per rank block, 8 positions of P.
template <int DT>
struct ContractWin {
    Frag<DT> q[4];
    f32x4_t pv[kContractMB][2];
};

// Row indices of this lane's 4 rows of a window (positions outside [lo, hi)
// read row lo: finite data, P is zero there).
__device__ __forceinline__ void contract_rows(int32_t* rows, const int32_t* perm, int win, int lo, int hi, int lrow) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int pos = win + lrow + j;
        rows[j] = perm[pos >= lo && pos < hi ? pos : lo];
    }
}

// NT: the window's x / dY rows are loaded with the nontemporal hint.
template <int DT, bool NT>
__device__ __forceinline__ void contract_load(ContractWin<DT>& W, const char* q, int64_t ldq, const float* PT,
                                              int64_t ldT, const int32_t* rows, int win, int c0, int lcol, int rank0,
                                              int r, int lane) {
    constexpr int EB = Frag<DT>::kBytes;
    if constexpr (NT && DT == LORA_BF16) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            W.q[j].q = __builtin_nontemporal_load(
                gptr(reinterpret_cast<const u32x4_t*>(q + ((int64_t)rows[j] * ldq + c0 + lcol) * EB)));
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) W.q[j] = Frag<DT>::load(q + ((int64_t)rows[j] * ldq + c0 + lcol) * EB);
    }
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

// NT: nontemporal loads of the x / dY windows.  The two-pass backward (dA and
// dB tiles) takes it: those streams then leave the g / v windows and the other
// tiles' rows in L2 (4096 fine-tuning rows, 5120 -> 5120: backward 65.5
// against 67.6 us, measured with the contraction in a launch of its own);
// the dA-only contraction after the streaming pass is faster with ordinary
// loads (52.0 against 53.7 us).
//
// Body of workgroup blk of the G workgroups (NW waves each, G a multiple of
// the 8 XCDs, workgroup blk placed at a launch index congruent to blk modulo
// 8) that share the contraction; s_mem holds ContractLds<DT, NW>::kBytes.
template <int DT, bool NT, int NW>
__device__ __forceinline__ void contract_body(const ContractParams& p, int blk, int G, char* s_mem) {
    static_assert(NW >= 4, "waves 0..3 finish the four 16-column blocks of a tile");
    if (p.stop && *p.stop) return;

    const int wave = wave_id();
    const int lane = threadIdx.x & (kWave - 1);
    const int lr = lane & 15;
    const int lg = lane >> 4;
    const int ncb = p.ncb_in + p.ncb_out;
    const int n_act = p.sched[2];
    // Workgroups of one XCD take neighbouring ranges (workgroup b runs on XCD b % 8).
    const int vg = (blk % kNumXcd) * (G / kNumXcd) + blk / kNumXcd;
    int32_t* meta = p.fix_meta + (int64_t)vg * 2 * kFixMeta;
    if (threadIdx.x == 0) {
        meta[0] = -1;
        meta[kFixMeta] = -1;
    }

    // Total units (every wave, 64 adapters per pass); workgroup 0 counts the bad entries.
    int64_t U = 0;
    for (int b = 0; b < n_act; b += kWave) {
        const int i = b + lane;
        ContractAct c{};
        if (i < n_act) c = contract_act(p, i, ncb);
        U += uniform64(wave_sum64(c.units));
        if (blk == 0 && wave == 0 && i < n_act && c.rgroups == 0) atomicAdd(p.err, 1);
    }
    const int64_t begin = U * vg / G;
    const int64_t end = U * (vg + 1) / G;
    if (begin >= end) {  // (fewer units than workgroups) the fix-up steps over this one
        if (threadIdx.x == 0) meta[0] = -2;
        return;
    }
    // The active adapter holding unit `begin` and the units before it.
    int act = 0;
    int64_t abase = 0;
    for (int b = 0; b < n_act; b += kWave) {
        const int i = b + lane;
        const int64_t un = i < n_act ? contract_act(p, i, ncb).units : 0;
        int64_t incl = un;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const int64_t o = __shfl_up(incl, d, kWave);
            if (lane >= d) incl += o;
        }
        const uint64_t hit = __ballot(i < n_act && abase + incl - un <= begin && begin < abase + incl);
        if (hit) {
            const int l = __ffsll((long long)hit) - 1;
            act = b + l;
            abase += uniform64(__shfl(incl - un, l, kWave));
            break;
        }
        abase += uniform64(__shfl(incl, kWave - 1, kWave));
    }

    char* tileA = s_mem + (2 * wave) * ContractLds<DT, NW>::kTileBytes;
    char* tileB = s_mem + (2 * wave + 1) * ContractLds<DT, NW>::kTileBytes;
    // Loader role: lane covers window rows 4*(lane/8)+j (j < 4), columns 8*(lane%8)+e (e < 8).
    const int lrow = 4 * (lane >> 3);
    const int lcol = 8 * (lane & 7);

    ContractAct c = contract_act_uniform(p, act, ncb);
    int slot = 0;
    for (int64_t u = begin; u < end;) {
        if (u >= abase + c.units) {  // next adapter (u < end <= U: one exists)
            abase += c.units;
            c = contract_act_uniform(p, ++act, ncb);
            continue;
        }
        const int64_t local = u - abase;
        const int tile_in = (int)(local / c.nwin);  // rank group major, then column block
        const int w0 = (int)(local - (int64_t)tile_in * c.nwin);
        const int w1 = (int)min((int64_t)c.nwin, w0 + (end - u));
        const int rg = tile_in / ncb;
        const int cb_all = tile_in - rg * ncb;
        const int a = c.a;
        const lora_adapter ad = load_adapter(p.adapters, a);
        const lora_adapter_grad gr = load_grad(p.grads, a);
        const bool is_dA = cb_all < p.ncb_in;
        const int r = ad.rank;
        const int rank0 = rg * 16 * kContractMB;
        const int nmb = min(kContractMB, (r - rank0 + 15) / 16);
        const int cb = is_dA ? cb_all : cb_all - p.ncb_in;
        const int c0 = cb * 64;
        const int N = is_dA ? p.d_in : p.d_out;
        const char* q = static_cast<const char*>(is_dA ? p.x : p.dy);
        const int64_t ldq = is_dA ? p.ldx : p.lddy;
        const float* PT = is_dA ? p.gT : p.vT;
        // Columns past N (N is a multiple of 8) read column block 0 of the row; never written back.
        const int cq = c0 + lcol < N ? c0 : -lcol;
        const int lo = c.lo;
        const int hi = c.hi;
        // This wave's windows: a contiguous share of [w0, w1) of the 32-aligned
        // windows of sorted positions covering [lo, hi).
        const int wbase = lo & ~31;
        const int nwt = w1 - w0;
        const int wa = wbase + 32 * (w0 + nwt * wave / NW);
        const int wb = wbase + 32 * (w0 + nwt * (wave + 1) / NW);

        f32x4_t acc[kContractMB][4];
#pragma unroll
        for (int mb = 0; mb < kContractMB; ++mb)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        // Windows visited from a tile-dependent start (the column blocks of one
        // adapter read the same g / v windows); fixed order per tile.  Two
        // streams: A takes windows 0, 2, 4, ..., B takes 1, 3, 5, ...; indices
        // past the range repeat the last window (loaded, never multiplied).
        const int nw = (wb - wa) / 32;
        if (nw > 0) {
            const int rot = cb_all % nw;
            auto win_at = [&](int i) { return wa + 32 * rotated(0, nw, rot, i < nw ? i : nw - 1); };
            int32_t rowsA[4], rowsB[4];
            ContractWin<DT> WA, WB;
            contract_rows(rowsA, p.perm, win_at(0), lo, hi, lrow);
            contract_rows(rowsB, p.perm, win_at(1), lo, hi, lrow);
            contract_load<DT, NT>(WA, q, ldq, PT, p.ldT, rowsA, win_at(0), cq, lcol, rank0, r, lane);
            contract_rows(rowsA, p.perm, win_at(2), lo, hi, lrow);
            contract_load<DT, NT>(WB, q, ldq, PT, p.ldT, rowsB, win_at(1), cq, lcol, rank0, r, lane);
            contract_rows(rowsB, p.perm, win_at(3), lo, hi, lrow);
            // (B's multiply is unconditional inside the loop, so the compiler
            // keeps B's loads where they are issued, a window ahead)
            int i = 0;
            for (; i + 1 < nw; i += 2) {
                contract_compute<DT>(WA, tileA, acc, win_at(i), lo, hi, lcol, lrow, nmb, lane);
                contract_load<DT, NT>(WA, q, ldq, PT, p.ldT, rowsA, win_at(i + 2), cq, lcol, rank0, r, lane);
                contract_rows(rowsA, p.perm, win_at(i + 4), lo, hi, lrow);
                contract_compute<DT>(WB, tileB, acc, win_at(i + 1), lo, hi, lcol, lrow, nmb, lane);
                contract_load<DT, NT>(WB, q, ldq, PT, p.ldT, rowsB, win_at(i + 3), cq, lcol, rank0, r, lane);
                contract_rows(rowsB, p.perm, win_at(i + 5), lo, hi, lrow);
            }
            if (i < nw) contract_compute<DT>(WA, tileA, acc, win_at(i), lo, hi, lcol, lrow, nmb, lane);
        }

        // Fixed-order sum of the waves' tiles; wave nb (< 4) finishes column block nb.
        __syncthreads();
        f32x4_t* red = reinterpret_cast<f32x4_t*>(s_mem);
#pragma unroll
        for (int mb = 0; mb < kContractMB; ++mb)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) red[((wave * kContractMB + mb) * 4 + nb) * kWave + lane] = acc[mb][nb];
        __syncthreads();
        const bool whole = w0 == 0 && w1 == c.nwin;
        if (wave < 4) {
            const int nb = wave;
            const float s = ad.scale;
#pragma unroll
            for (int mb = 0; mb < kContractMB; ++mb) {
                f32x4_t sum = red[(mb * 4 + nb) * kWave + lane];
#pragma unroll 4
                for (int w = 1; w < NW; ++w) sum += red[((w * kContractMB + mb) * 4 + nb) * kWave + lane];
                if (!whole) {
                    // partial tile for contract_fixup_kernel
                    float* f = p.fix + ((int64_t)vg * 2 + slot) * kFixFloats;
                    *gptr(reinterpret_cast<f32x4_t*>(f) + (mb * 4 + nb) * kWave + lane) = sum;
                } else if (mb < nmb) {
                    // the four read-modify-writes of a lane: loads first (entries
                    // outside [0, r) x [0, N) read the tile's first entry and are
                    // not written), then the stores
                    const int col = c0 + 16 * nb + lr;
                    float* dst[4];
                    bool ok[4];
                    float old[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int rk = rank0 + 16 * mb + 4 * lg + i;
                        ok[i] = col < N && rk < r;
                        const int rk_ = ok[i] ? rk : rank0;
                        const int col_ = ok[i] ? col : c0;
                        dst[i] = is_dA ? gr.dA + (int64_t)rk_ * p.d_in + col_ : gr.dB + (int64_t)col_ * r + rk_;
                        old[i] = *gptr(dst[i]);
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (ok[i]) *gptr(dst[i]) = old[i] + s * sum[i];
                }
            }
        }
        if (!whole) {
            if (threadIdx.x == 0) {
                const int64_t tile_u = abase + (int64_t)tile_in * c.nwin;  // first unit: the tile's id
                int32_t* m = meta + slot * kFixMeta;
                m[0] = (int32_t)(tile_u & 0x7fffffff);
                m[1] = (int32_t)(tile_u >> 31);
                m[2] = a;
                m[3] = rg;
                m[4] = cb_all;
                m[5] = w0 == 0;  // owner: holds the tile's first window, runs its fix-up
            }
            slot = 1;  // only a workgroup's first and last tiles can be cut
        } else {
            slot = 1;
        }
        u += w1 - w0;
        __syncthreads();
    }
}

// Adds the partial tiles of each cut tile in workgroup order, then s times
// the sum to dA / dB.  Workgroup g handles the tile it owns (if any); the
// later workgroups that hold the same tile follow g in order.
// (as workgroup g0 of a 4-wave grid part)
__device__ __forceinline__ void contract_fixup_body(const ContractParams& p, int G, int g0) {
    if (p.stop && *p.stop) return;
    const int nb = wave_id();
    const int lane = threadIdx.x & (kWave - 1);
    const int lr = lane & 15;
    const int lg = lane >> 4;
    for (int sl = 0; sl < 2; ++sl) {
        const int32_t* m = p.fix_meta + ((int64_t)g0 * 2 + sl) * kFixMeta;
        if (m[0] < 0 || !m[5]) continue;
        const int32_t id0 = m[0], id1 = m[1];
        const int a = m[2], rg = m[3], cb_all = m[4];
        // Requested together: the adapter's entries, this workgroup's partial
        // tile and the records of the 64 workgroups after g0 (lane j reads
        // workgroup g0 + 1 + j's first slot).
        const lora_adapter ad = load_adapter(p.adapters, a);
        const lora_adapter_grad gr = load_grad(p.grads, a);
        f32x4_t sum[kContractMB];
#pragma unroll
        for (int mb = 0; mb < kContractMB; ++mb)
            sum[mb] = *gptr(reinterpret_cast<const f32x4_t*>(p.fix + ((int64_t)g0 * 2 + sl) * kFixFloats) +
                            (mb * 4 + nb) * kWave + lane);
        auto records = [&](int g, int32_t& m0, int32_t& m1) {
            const int gj = g + lane;
            m0 = -3;
            m1 = 0;
            if (gj < G) {
                const int32_t* mg = p.fix_meta + (int64_t)gj * 2 * kFixMeta;
                m0 = mg[0];
                m1 = mg[1];
            }
        };
        int32_t m0, m1;
        records(g0 + 1, m0, m1);
        // The dA / dB entries' old values, requested before the followers'
        // partial tiles (addresses clamped, stores masked).
        const bool is_dA = cb_all < p.ncb_in;
        const int r = ad.rank;
        const int rank0 = rg * 16 * kContractMB;
        const int nmb = min(kContractMB, (r - rank0 + 15) / 16);
        const int c0 = (is_dA ? cb_all : cb_all - p.ncb_in) * 64;
        const int N = is_dA ? p.d_in : p.d_out;
        const int col = c0 + 16 * nb + lr;
        float old[kContractMB][4];
        float* dst[kContractMB][4];
        bool ok[kContractMB][4];
#pragma unroll
        for (int mb = 0; mb < kContractMB; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rk = rank0 + 16 * mb + 4 * lg + i;
                ok[mb][i] = mb < nmb && col < N && rk < r;
                const int rk_ = ok[mb][i] ? rk : 0, col_ = ok[mb][i] ? col : 0;
                dst[mb][i] = is_dA ? gr.dA + (int64_t)rk_ * p.d_in + col_ : gr.dB + (int64_t)col_ * r + rk_;
                old[mb][i] = *gptr(dst[mb][i]);
            }
        // The later workgroups holding the tile (their first slot) form a run
        // after g0, workgroups without units skipped: a run of up to 64 costs
        // one round trip for the records; the partial tiles are then loaded
        // eight at a time and added in workgroup order.
        for (int g = g0 + 1; g < G; g += kWave) {
            if (g > g0 + 1) records(g, m0, m1);
            const bool same = m0 == id0 && m1 == id1;
            const uint64_t same_mask = __ballot(same);
            const uint64_t end_mask = __ballot(!same && m0 != -2);  // another tile, or past the grid
            const int n = end_mask ? __ffsll((long long)end_mask) - 1 : kWave;
            for (int j0 = 0; j0 < n; j0 += 8) {
                f32x4_t pv[8][kContractMB];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int gg = min(g + j0 + j, G - 1);
#pragma unroll
                    for (int mb = 0; mb < kContractMB; ++mb)
                        pv[j][mb] = *gptr(reinterpret_cast<const f32x4_t*>(p.fix + (int64_t)gg * 2 * kFixFloats) +
                                          (mb * 4 + nb) * kWave + lane);
                }
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (j0 + j < n && ((same_mask >> (j0 + j)) & 1))
#pragma unroll
                        for (int mb = 0; mb < kContractMB; ++mb) sum[mb] += pv[j][mb];
            }
            if (n < kWave) break;
        }
#pragma unroll
        for (int mb = 0; mb < kContractMB; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (ok[mb][i]) *gptr(dst[mb][i]) = old[mb][i] + ad.scale * sum[mb][i];
    }
}

__global__ __launch_bounds__(4 * kWave) void contract_fixup_kernel(ContractParams p, int G) {
    contract_fixup_body(p, G, blockIdx.x);
}

}  // namespace lora
