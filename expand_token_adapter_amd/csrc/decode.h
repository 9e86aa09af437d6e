// decode.h -- shrink and expand-add kernels for batches whose adapters have few
// rows each (decode), on gfx950.
//
// When each adapter serves a handful of rows, the forward's bytes are the
// adapter weights themselves (DeltaServe section 2.1: decode is bound by
// memory bandwidth; the adapter-caching page: the adapters' cost grows with
// their number and size).  Both kernels therefore stream each weight byte from
// HBM once, into registers in MFMA operand layout, with many loads in flight
// per wave, and work on 16-row tiles (the segment builder's 16-row records),
// so a decode row group costs one tile, not a mostly-empty 64-row one.
//
// Shrink (v = A x): a workgroup = (16-row tile, 16-rank block of the tile's
// adapter).  Its waves split d_in into equal runs of 32-element steps; each
// wave keeps kShrPD steps of A-rows and x-rows in flight and accumulates one
// 16x16 MFMA tile (ranks x rows); the waves' tiles are added in wave order
// through LDS and written straight to v: no partial sums leave the workgroup,
// no second kernel, no workspace.
//
// Expand (y += s B v): a workgroup = (16-row tile, range of kDecRange output
// columns); each of its waves walks 64-column chunks of the range with the
// chunks' weight blocks and y rows in flight, as many as its registers allow
// for the adapter's rank.  For ranks <= 16 one 16-byte operand load carries
// 16-byte rows of B for different columns: the MFMA's 32-deep reduction is
// split into 32 / r_pad groups of r_pad ranks, each group owning 16 columns,
// and the v operand carries each row's values in its own group only (zeros
// elsewhere), so every loaded byte is used.  Results are added to y through a
// per-wave LDS transpose, in the row-contiguous layout of the other expand.
//
// Sums run in a fixed order (per 32-element step inside one MFMA, then steps
// in order, then waves in order): results are bit-reproducible.
#pragma once

#include "device_common.h"

namespace lora {

// ============================================================== shrink
//
// Workgroups of 8 or 16 waves (few tasks): a wave reads its run of d_in in
// groups of 128 elements (4 MFMA steps): the group's 16 rank rows of A_a and
// 16 x rows are 256-byte pieces of rows, read with coalesced loads (16
// neighbouring lanes take the 16 consecutive 16-byte units of one row piece,
// 4 rows per load), two groups in flight in registers.  An arrived group is
// written to the wave's own LDS region, unit u of row j at slot u ^ j, and
// read back in MFMA operand layout (lane (lr, lg) takes unit 4 t + lg of row
// lr at step t), which the XOR spreads over distinct banks.  Workgroups of 4
// waves (many tasks) share 512-element groups: every load is one contiguous
// 1 KB piece of a row (the same LDS layout, 64 units per row).  Loads of rows
// past the adapter's rank or the tile fetch nothing (their offsets lie past
// the buffer).

constexpr int kShrGS = 4;                   // MFMA steps (of 32 elements) per group
constexpr int kShrUnits = 2 * kShrGS * 2;   // 16-byte units per row piece (16)
constexpr int kShrLoads = 16 / (kWave / kShrUnits);  // coalesced loads per 16 rows (4)

struct DecShrinkParams {
    const void* x;        // rows gathered through perm
    int64_t ldx;
    uint32_t x_bytes;     // bytes from x to the end of its last row (< 2^31)
    int32_t K;            // d_in
    const lora_adapter* adapters;
    int32_t r_max;
    const int32_t* perm;
    const int32_t* sched;
    int64_t tiles16_off;
    float* v;             // [row][ldv], row = original row (or sorted position if v_by_pos)
    int64_t ldv;
    int32_t v_by_pos;
    int32_t rblocks;      // ceil(r_max / 16)
    int32_t balanced;     // 1: cost-balanced task ranges (plan); 0: one task per workgroup
    int32_t* err;
};

// Balanced mode (many tasks): workgroup w of G (numbered XCD by XCD) takes the
// tasks whose start falls in [w C / G, (w + 1) C / G) of the total cost C, in
// task order; a task (tile t, rank block b) costs its A rows plus its x rows,
// min(16, r - 16 b) + rows(t) rows of d_in elements, plus a fixed
// kShrTaskCost rows.  Wave 0 builds the
// tiles' cost prefix in LDS as the expand's plan does; each XCD then holds
// one contiguous eighth of the work, so the tiles of an adapter share A_a
// through one L2 and the rank blocks of a tile share its x rows.  Direct
// mode (few tasks): workgroups take tasks by index, XCD by XCD.
constexpr int kShrPlanMaxTiles = 2048;  // tiles per call in balanced mode (LDS prefix)
// A task's time is set mostly by its chain of sequential 512-element groups,
// whatever its live rows, so the plan prices each task at a fixed 512 rows
// plus its rows: the ranges then hold nearly equal task counts (zipf-320
// decode batch, forward per call: 135.3 / 133.2 / 130.6 / 128.9 / 129.0 us
// with a fixed cost of 0 / 32 / 256 / 512 / 1024 rows).
#ifndef LORA_SHR_TASK_COST
#define LORA_SHR_TASK_COST 512
#endif
constexpr uint32_t kShrTaskCost = LORA_SHR_TASK_COST;  // fixed cost of a task, in rows
#ifndef LORA_SHR_DEPTH
#define LORA_SHR_DEPTH 2
#endif
constexpr int kShrDepth = LORA_SHR_DEPTH;  // 4-wave kernel: 512-element groups in flight per wave

// Records of tiles t0 + 64 i + lane (i < NB; tile 0 past n16) and their
// table entries: the records' loads all in flight, then the entries' loads.
// Each record (16 bytes, one word unused) and entry (the scale unused) is
// read whole by an empty asm statement: no register of a value is reused
// while its load is in flight, which would make every load wait for the
// previous one.
template <int NB>
__device__ __forceinline__ void plan_loads(const int32_t* sched, int64_t off, const lora_adapter* table, int t0,
                                           int n16, int lane, TileRec (&rec)[NB], lora_adapter (&ads)[NB]) {
    u32x4_t raw[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int t = t0 + kWave * i + lane;
        raw[i] = *cptr(reinterpret_cast<const u32x4_t*>(sched + off + 4 * (int64_t)(t < n16 ? t : 0)));
    }
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        asm volatile("" ::"v"(raw[i]));
        rec[i] = TileRec{(int)raw[i][0], (int)raw[i][1], (int)raw[i][2]};
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) ads[i] = load_adapter(table, rec[i].adapter);
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < NB; ++i) asm volatile("" ::"v"(ads[i].scale));
}

// Returns {first tile, first rank block, end tile, end rank block} (end
// exclusive).  s_pre / s_inf: LDS arrays of n16 entries.
__device__ __forceinline__ int4 dec_shrink_plan(const DecShrinkParams& p, int n16, int lane, uint32_t* s_pre,
                                                uint32_t* s_inf) {
    constexpr int kBlocks = 8;
    for (int t0 = 0; t0 < n16; t0 += kBlocks * kWave) {
        // every record, then every table entry, in flight together: two
        // memory round trips per round of 512 tiles
        TileRec rec[kBlocks];
        lora_adapter ads[kBlocks];
        plan_loads<kBlocks>(p.sched, p.tiles16_off, p.adapters, t0, n16, lane, rec, ads);
        uint32_t carry = t0 > 0 ? s_pre[t0 - 1] : 0u;
#pragma unroll
        for (int i = 0; i < kBlocks; ++i) {
            const int t = t0 + kWave * i + lane;
            const lora_adapter& ad = ads[i];
            const bool ok = t < n16 && adapter_ok(ad, p.r_max);
            if (t < n16 && !ok && blockIdx.x == 0) atomicAdd(p.err, 1);
            const uint32_t nrb = ok ? (uint32_t)(ad.rank + 15) / 16 : 0u;
            const uint32_t c = ok ? (uint32_t)ad.rank + nrb * ((uint32_t)rec[i].rows + kShrTaskCost) : 0u;
            uint32_t incl = c;
#pragma unroll
            for (int d = 1; d < kWave; d <<= 1) {
                const uint32_t o = __shfl_up(incl, d, kWave);
                if (lane >= d) incl += o;
            }
            if (t < n16) {
                s_pre[t] = carry + incl;
                s_inf[t] = (uint32_t)rec[i].rows | (nrb << 8);
            }
            carry += __shfl(incl, kWave - 1, kWave);
        }
    }
    __builtin_amdgcn_wave_barrier();
    const uint64_t total = n16 > 0 ? s_pre[n16 - 1] : 0;
    const uint64_t G = gridDim.x;
    const uint64_t w = (uint64_t)(blockIdx.x % kNumXcd) * (G / kNumXcd) + blockIdx.x / kNumXcd;
    const uint64_t lo = total * w / G, hi = total * (w + 1) / G;
    // first task whose start is at or past x: tile = first with prefix > x;
    // its tasks start at st + b (16 + rows), b < nrb
    auto locate = [&](uint64_t x, int& tt, int& bb) {
        int l = 0, h = n16;
        while (l < h) {
            const int m = (l + h) >> 1;
            if ((uint64_t)s_pre[m] > x) h = m;
            else l = m + 1;
        }
        if (l >= n16) {
            tt = n16;
            bb = 0;
            return;
        }
        const uint64_t st = l > 0 ? s_pre[l - 1] : 0;
        const uint32_t inf = s_inf[l];
        const uint64_t q = 16 + (inf & 255u) + kShrTaskCost;
        const uint64_t b = (x - st + q - 1) / q;
        tt = b < (inf >> 8) ? l : l + 1;
        bb = b < (inf >> 8) ? (int)b : 0;
    };
    int4 plan;
    locate(lo, plan.x, plan.y);
    locate(hi, plan.z, plan.w);
    if (hi >= total) plan.z = n16, plan.w = 0;
    return plan;
}

// NW: waves per workgroup (4, 8 or 16).
template <int DT, int NW>
__global__ __launch_bounds__(NW * kWave) void dec_shrink_kernel(DecShrinkParams p) {
    static_assert(DT == LORA_BF16, "the 16-row-tile kernels are built for bf16 elements");
    using F = Frag<DT>;
    constexpr int EB = F::kBytes;
    // per wave: A rows and x rows of one group, 16 x 16 units each
    __shared__ __attribute__((aligned(16))) u32x4_t s_grp[NW][2][16 * kShrUnits];
    __shared__ f32x4_t s_red[NW][kWave];

    const int wave = wave_id();
    const int lane = threadIdx.x & (kWave - 1);
    const int lr = lane & 15;  // MFMA: A rank row of the block / x row of the tile
    const int lg = lane >> 4;  // MFMA: 8-element group of the step
    const int cu = lane & (kShrUnits - 1);  // coalesced load: unit of the row piece
    const int cr = lane / kShrUnits;        // coalesced load: row within the load's 4 rows
    const int n16 = p.sched[0];
    // wave w takes groups w, w + NW, w + 2 NW, ...: at any time the waves of a
    // workgroup read neighbouring pieces of the same rows
    const int ngroups = (p.K + 32 * kShrGS - 1) / (32 * kShrGS);
    u32x4_t* sA = &s_grp[wave][0][0];
    u32x4_t* sX = &s_grp[wave][1][0];

    // one task: rank block rb of tile rec (adapter ad, a valid entry)
    auto task = [&](const TileRec& rec, const lora_adapter& ad, int rb) {
        const int r = ad.rank;
        const int rank0 = 16 * rb;
        if (rank0 >= r) return;  // wave-uniform: the whole workgroup skips
        const int nrows = rec.rows;
        const int nranks = min(16, r - rank0);
        // Byte offsets inside the x and A_a buffers stay below 2^31 (checked
        // on the host); a piece that runs past K reads the next row (or zeros
        // past the buffer) and is zeroed where it is used.  Rows past the tile
        // or the rank take an offset past the end of the buffer: the hardware
        // returns zeros without touching memory, and no branch splits the
        // loads (a branch would make the compiler wait for every load at its
        // join).  Row indices come through scalar loads: no vector load may
        // sit between the buffer loads, or the compiler's waits lose their
        // count.
        const buf_rsrc_t xr = make_rsrc(p.x, p.x_bytes);
        const buf_rsrc_t ar = make_rsrc(ad.A, (uint32_t)((int64_t)r * p.K * EB));
        f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if constexpr (NW == 4) {
            // Four waves share each group of 512 elements (16 MFMA steps):
            // wave w loads rows w, w + 4, w + 8, w + 12 of A's block and of the
            // tile, one contiguous 1 KB piece of a row per load (lane l: unit
            // l), and writes them to the workgroup's LDS group (unit u of row j
            // at slot u ^ j); after a barrier each wave multiplies its quarter
            // of the steps (4 w .. 4 w + 3) for all 16 rows.  kShrDepth
            // groups are in flight in registers.
            constexpr int kU = 64;  // 16-byte units per 1 KB row piece
            u32x4_t* gA = &s_grp[0][0][0];
            u32x4_t* gX = gA + 16 * kU;
            const int ng = (p.K + 511) / 512;
            uint32_t xo[4], ao[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = wave + 4 * i;
                const int32_t xrow = *cptr(p.perm + rec.pos0 + (row < nrows ? row : 0));
                xo[i] = row < nrows ? (uint32_t)((int64_t)xrow * p.ldx * EB) + 16u * lane : kBufOff;
                ao[i] = row < nranks ? (uint32_t)((int64_t)(rank0 + row) * p.K * EB) + 16u * lane : kBufOff;
            }
            constexpr int D = kShrDepth;  // groups in flight
            u32x4_t xq[D][4], wq[D][4];
            auto issue4 = [&](int b, int g) {
                const uint32_t kb = (uint32_t)g * 1024u;
                const bool in = g < ng;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    // many tasks: an A_a block is read by few tiles, the tile's
                    // x rows by each of its rank blocks; A streams past L2
                    // (nontemporal) so the x rows stay (zipf-320 decode batch:
                    // 64.0 against 66.2 us)
                    xq[b][i] = buf_load16(xr, in && xo[i] != kBufOff ? xo[i] + kb : kBufOff, 0);
                    wq[b][i] = buf_load16_nt(ar, in && ao[i] != kBufOff ? ao[i] + kb : kBufOff, 0);
                }
            };
#pragma unroll
            for (int b = 0; b < D; ++b) {
                issue4(b, b);
                asm volatile("" ::: "memory");
            }
            for (int g = 0; g < ng; g += D) {
#pragma unroll
                for (int b = 0; b < D; ++b) {
                    const int gg = g + b;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int row = wave + 4 * i;
                        gA[row * kU + (lane ^ row)] = wq[b][i];
                        gX[row * kU + (lane ^ row)] = xq[b][i];
                    }
                    issue4(b, gg + D);
                    asm volatile("" ::: "memory");
                    lds_barrier();
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const int step = 4 * wave + t;
                        const int u = 4 * step + lg;
                        const bool ok = gg < ng && 512 * gg + 32 * step + 8 * lg < p.K;
                        const F wf{gA[lr * kU + (u ^ lr)]};
                        const F xf{gX[lr * kU + (u ^ lr)]};
                        acc = mma(wf, xf.masked(ok), acc);
                    }
                    lds_barrier();
                }
            }
        } else {
        // Each wave takes its own 128-element groups.  Coalesced loads: load i
        // covers rows 4 i + cr (A: rank rows of the block; x: rows of the
        // tile), unit cu of the group's row piece.  Registers of two groups
        // in flight.
        int32_t prow[16];  // the tile's rows (rows past it repeat its first)
#pragma unroll
        for (int j = 0; j < 16; ++j) prow[j] = *cptr(p.perm + rec.pos0 + (j < nrows ? j : 0));
        uint32_t xoff[kShrLoads], aoff[kShrLoads];
        bool xon[kShrLoads], aon[kShrLoads];
#pragma unroll
        for (int i = 0; i < kShrLoads; ++i) {
            const int row = 4 * i + cr;
            xon[i] = row < nrows;
            aon[i] = row < nranks;
            const int32_t xrow = cr == 0 ? prow[4 * i] : cr == 1 ? prow[4 * i + 1] : cr == 2 ? prow[4 * i + 2]
                                                                                        : prow[4 * i + 3];
            xoff[i] = (uint32_t)((int64_t)xrow * p.ldx * EB) + 16u * cu;
            aoff[i] = (uint32_t)((int64_t)(rank0 + (aon[i] ? row : 0)) * p.K * EB) + 16u * cu;
        }
        u32x4_t xa[2][kShrLoads], wa[2][kShrLoads];
        auto issue = [&](int b, int g) {
            const uint32_t kb = (uint32_t)g * (32 * kShrGS * EB);
            const bool in = g < ngroups;  // groups past K fetch nothing
#pragma unroll
            for (int i = 0; i < kShrLoads; ++i) {
                xa[b][i] = buf_load16(xr, xon[i] && in ? xoff[i] + kb : kBufOff, 0);
                wa[b][i] = buf_load16(ar, aon[i] && in ? aoff[i] + kb : kBufOff, 0);
            }
        };
        // The loop has no branch but its own: groups past K are loaded at an
        // offset past the buffer (zeros, no fetch) and multiplied by zero, so
        // the compiler's waits stay exact (a conditional load would make it
        // wait for all loads where the paths join).
        // (the empty asm statements keep the two groups' loads in issue order:
        // the waits below count on group g0's loads being the older ones)
        issue(0, wave);
        asm volatile("" ::: "memory");
        issue(1, wave + NW);
        asm volatile("" ::: "memory");
        for (int g = wave; g < ngroups; g += 2 * NW) {
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const int gg = g + b * NW;
                // group gg -> LDS (unit cu of row 4 i + cr at slot cu ^ row)
#pragma unroll
                for (int i = 0; i < kShrLoads; ++i) {
                    const int row = 4 * i + cr;
                    sA[row * kShrUnits + (cu ^ row)] = wa[b][i];
                    sX[row * kShrUnits + (cu ^ row)] = xa[b][i];
                }
                __builtin_amdgcn_wave_barrier();
                // its registers are free: the group two ahead goes in flight
                issue(b, gg + 2 * NW);
                asm volatile("" ::: "memory");
#pragma unroll
                for (int t = 0; t < kShrGS; ++t) {
                    const int u = 4 * t + lg;
                    const bool ok = 32 * (kShrGS * gg + t) + 8 * lg < p.K;
                    const F wf{sA[lr * kShrUnits + (u ^ lr)]};
                    const F xf{sX[lr * kShrUnits + (u ^ lr)]};
                    acc = mma(wf, xf.masked(ok), acc);
                }
                __builtin_amdgcn_wave_barrier();
            }
        }
        }

        // waves' tiles in wave order: D rows 4 lg + e = ranks, column lr = row
        s_red[wave][lane] = acc;
        lds_barrier();
        if (wave == 0 && lr < nrows) {
            f32x4_t sum = s_red[0][lane];
#pragma unroll
            for (int w = 1; w < NW; ++w) sum += s_red[w][lane];
            const int k = rank0 + 4 * lg;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (k + e >= r) sum[e] = 0.f;
            // ranks below round_up(r, 8) <= round_up(r_max, 8) <= ldv: v as lora_shrink writes it
            if (k < (r + 7) / 8 * 8) {
                const int64_t vrow = p.v_by_pos ? (int64_t)rec.pos0 + lr : (int64_t)p.perm[rec.pos0 + lr];
                *gptr(reinterpret_cast<f32x4_t*>(p.v + vrow * p.ldv + k)) = sum;
            }
        }
        lds_barrier();  // s_red is rewritten by the next task
    };

    if (p.balanced) {
        // the plan's prefix arrays live in the group buffers until the tasks start
        static_assert(sizeof(s_grp) >= 2 * kShrPlanMaxTiles * sizeof(uint32_t), "plan arrays fit the group buffers");
        __shared__ int4 s_plan;
        if (wave == 0) {
            uint32_t* s_pre = reinterpret_cast<uint32_t*>(&s_grp[0][0][0]);
            const int4 pl = dec_shrink_plan(p, min(n16, kShrPlanMaxTiles), lane, s_pre, s_pre + kShrPlanMaxTiles);
            if (lane == 0) s_plan = pl;
        }
        __syncthreads();
        const int4 plan = s_plan;
        __syncthreads();  // the group buffers are rewritten by the tasks
        for (int t = plan.x; t <= plan.z && t < n16; ++t) {
            const TileRec rec = load_tile(p.sched, p.tiles16_off, t);
            const lora_adapter ad = load_adapter(p.adapters, rec.adapter);
            if (!adapter_ok(ad, p.r_max)) continue;  // counted by the plan
            const int b0 = t == plan.x ? plan.y : 0;
            const int b1 = t == plan.z ? plan.w : (ad.rank + 15) / 16;
            for (int rb = b0; rb < b1; ++rb) task(rec, ad, rb);
        }
        return;
    }
    const int64_t ntasks = (int64_t)n16 * p.rblocks;
    const TaskSlice ts = xcd_slice(ntasks, 1, 0);
    for (int64_t i = ts.begin; i < ts.end; i += ts.stride) {
        const int tile = (int)(i / p.rblocks);
        const int rb = (int)(i % p.rblocks);
        const TileRec rec = load_tile(p.sched, p.tiles16_off, tile);
        const lora_adapter ad = load_adapter(p.adapters, rec.adapter);
        if (!adapter_ok(ad, p.r_max)) {
            if (rb == 0 && threadIdx.x == 0) atomicAdd(p.err, 1);
            continue;
        }
        task(rec, ad, rb);
    }
}

// ============================================================== expand-add

constexpr int kDecExpWaves = 4;
constexpr int kDecChunk = 64;                                  // columns per chunk
constexpr int kDecPitch = 68;                                  // floats per row of the per-wave transpose buffer

struct DecExpandParams {
    const float* v;       // [row][ldv]
    int64_t ldv;
    int32_t v_by_pos;
    const lora_adapter* adapters;
    int32_t r_max;
    const int32_t* perm;
    const int32_t* sched;
    int64_t tiles16_off;
    void* y;              // [row][ldy], rows through perm
    int64_t ldy;
    uint32_t y_bytes;     // bytes from y to the end of its last row (< 2^31)
    int32_t N;            // d_out
    int32_t balanced;     // 1: byte-balanced ranges (plan); 0: one tile slice per workgroup
    int32_t* err;
};

// Rank classes: r_pad = 8, 16 (several column groups per MFMA), 32, 64, 128.
//   G   column groups per MFMA (32 / r_pad for r_pad <= 32, else 1)
//   KS  32-rank steps (r_pad / 32 for r_pad >= 32, else 1)
//   SB  row sub-blocks of 16 / G rows covering the tile's 16 rows
//   NB  MFMAs per 64-column chunk and sub-block (64 / (16 G))... per KS step
//   LPC operand loads per chunk = NB * KS
//   DEPTH chunks whose loads are issued together
template <int CLS>
struct DecClass {
    static constexpr int r_pad = 8 << CLS;
    static constexpr int G = r_pad <= 32 ? 32 / r_pad : 1;
    static constexpr int KS = r_pad >= 32 ? r_pad / 32 : 1;
    static constexpr int SB = G;            // 16 rows in sub-blocks of 16 / G
    static constexpr int NB = 4 / G;        // 16 G columns per MFMA
    static constexpr int LPC = NB * KS;
    // at most 8 operand loads (32 registers) per batch: whole chunks for
    // ranks <= 64, half chunks for rank 128
    static constexpr int DEPTH = LPC <= 2 ? 4 : (LPC <= 4 ? 2 : 1);
    static constexpr int NBL = LPC > 8 ? NB / 2 : NB;  // MFMA blocks per batch of loads
};

template <int DT, int CLS>
__device__ __forceinline__ void dec_expand_task(const DecExpandParams& p, const lora_adapter& ad, const TileRec& rec,
                                                int cbeg, int cend, int wave, int lane, float* tw) {
    using F = Frag<DT>;
    using E = Elem<DT>;
    using O = F32Operand<DT>;
    using C = DecClass<CLS>;
    constexpr int EB = F::kBytes;
    constexpr int YQ = EB / 2;  // 16-byte quads per 8 elements
    constexpr int G = C::G, KS = C::KS, SB = C::SB, NB = C::NB, NBL = C::NBL;
    constexpr int DEPTH = C::DEPTH;
    constexpr int NH = NB / NBL;  // load batches per chunk
    static_assert(NH == 1 || DEPTH == 1, "chunks split into load batches are issued one at a time");
    static_assert(DT == LORA_BF16, "the 16-row-tile kernels are built for bf16 elements");
    constexpr int RPS = 16 / G;  // rows per sub-block
    const int lr = lane & 15;
    const int lg = lane >> 4;
    const int yr = lane >> 3;       // y layout: rows yr and yr + 8
    const int yc = 8 * (lane & 7);  // y layout: first of 8 columns in the chunk
    const int r = ad.rank;
    const float s = ad.scale;
    const int nrows = rec.rows;
    const bool units = (r & 7) == 0;  // B rows in whole 16-byte units
    const char* B = static_cast<const char*>(ad.B);
    char* ybase = static_cast<char*>(p.y);

    // Row indices: lane lr holds row lr of the tile (rows past the tile repeat
    // its first row); the y layout's rows come from it by lane exchange.
    const int pos_lr = rec.pos0 + (lr < nrows ? lr : 0);
    const int32_t row_lr = p.perm[pos_lr];
    const int64_t yrow0 = __shfl(row_lr, yr, kWave);
    const int64_t yrow1 = __shfl(row_lr, yr + 8, kWave);

    // v as the MFMA B operand (hi / lo bf16 pairs for bf16 weights).
    //   G == 1: sub-block 0 = the 16 rows, k step ks: lane (lr, lg) holds
    //           v[row lr][32 ks + 8 lg .. + 7].
    //   G > 1:  sub-block sb = rows RPS sb .. + RPS - 1; lane (lr, lg) holds
    //           v[row RPS sb + lr % RPS][j0 .. j0 + 7] when its rank group
    //           g = 8 lg / r_pad equals the column group lr / RPS, else zeros
    //           (j0 = 8 lg % r_pad).
    O vo[SB][KS];
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            int row, j0;
            bool on;
            if constexpr (G == 1) {
                row = lr;
                j0 = 32 * ks + 8 * lg;
                on = true;
            } else {
                row = RPS * sb + lr % RPS;
                j0 = (8 * lg) % C::r_pad;
                on = (8 * lg) / C::r_pad == lr / RPS;
            }
            const bool ok = on && row < nrows && j0 < r;
            float f[8];
            if (RPS * sb < nrows) {  // wave-uniform
                const int64_t vrow = p.v_by_pos ? (int64_t)rec.pos0 + (ok ? row : 0)
                                                : (int64_t)__shfl(row_lr, row, kWave);
                const LORA_GLOBAL f32x4_t* src =
                    gptr(reinterpret_cast<const f32x4_t*>(p.v + vrow * p.ldv + (ok ? j0 : 0)));
                const f32x4_t a = src[0], b = src[1];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    f[e] = (ok && j0 + e < r) ? a[e] : 0.f;
                    f[4 + e] = (ok && j0 + 4 + e < r) ? b[e] : 0.f;
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) f[e] = 0.f;
            }
            vo[sb][ks] = O::make(f);
        }
    }

    // Operand loads of one chunk (columns c0 .. c0 + 63): for MFMA nb and step
    // ks, lane (lr, lg) loads B[col][j0 .. j0 + 7] with
    //   G == 1: col = c0 + 16 nb + lr,            j0 = 32 ks + 8 lg
    //   G > 1:  col = c0 + 16 G nb + 16 g + lr,   j0 = 8 lg % r_pad, g = 8 lg / r_pad
    // Columns past N and groups past r load B's first unit and are zeroed
    // where they are used.
    auto col_of = [&](int c0, int nb) {
        if constexpr (G == 1) return c0 + 16 * nb + lr;
        else return c0 + 16 * G * nb + 16 * ((8 * lg) / C::r_pad) + lr;
    };
    auto j0_of = [&](int ks) {
        if constexpr (G == 1) return 32 * ks + 8 * lg;
        else return (8 * lg) % C::r_pad;
    };
    // B_a as a buffer: bytes past its end read as zeros (columns past N).
    const buf_rsrc_t br = make_rsrc(B, (uint32_t)((int64_t)p.N * r * EB));
    auto load_w = [&](int c0, int h, F (&wf)[NBL][KS]) {
#pragma unroll
        for (int b = 0; b < NBL; ++b)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int nb = h * NBL + b;
                const int col = col_of(c0, nb);
                const int j0 = j0_of(ks);
                if (units) {
                    // the whole offset in the lane's register: the buffer's range
                    // check covers that offset (and the instruction's immediate)
                    wf[b][ks].q = buf_load16(br, (uint32_t)(col * r + j0) * EB, 0);
                } else {
                    const bool ok = col < p.N && j0 < r;
                    const char* src = B + (ok ? (int64_t)col * r + j0 : 0) * EB;
                    wf[b][ks] = F::load_strided(src, 1, ok ? wkeep(r, j0) : 0);
                }
            }
    };
    // y through a buffer resource: chunks past this wave's range (c0 = -1)
    // and columns past N take an offset past the buffer (zeros, no fetch).
    const buf_rsrc_t yres = make_rsrc(p.y, p.y_bytes);
    auto load_y = [&](int c0, u32x4_t (&yq)[2][YQ]) {
        const bool ok = c0 >= 0 && c0 + yc < p.N;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int64_t row = u == 0 ? yrow0 : yrow1;
            const uint32_t off = ok ? (uint32_t)((row * p.ldy + c0 + yc) * EB) : kBufOff;
#pragma unroll
            // y is read once (nontemporal: B_a blocks re-read by an adapter's
            // tiles stay in L2; zipf-320 decode batch 71.8 against 73.5 us)
            for (int q = 0; q < YQ; ++q) yq[u][q] = buf_load16_nt(yres, off + 16u * q, 0);
        }
    };

    // this wave's chunks: cbeg + wave, cbeg + wave + kDecExpWaves, ... < cend;
    // a chunk past the range has c0 = -1 (loads fetch nothing, nothing stored)
    auto chunk_c0 = [&](int k) {
        const int ch = cbeg + wave + kDecExpWaves * k;
        return ch < cend ? ch * kDecChunk : -1;
    };
    const int nk = (cend - cbeg - wave + kDecExpWaves - 1) / kDecExpWaves;  // chunks of this wave
    for (int cb = 0; cb < nk; cb += DEPTH) {
        F wf[DEPTH][NBL][KS];
        u32x4_t yq[DEPTH][2][YQ];
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const int c0 = chunk_c0(cb + d);
            load_w(c0 < 0 ? p.N : c0, 0, wf[d]);
            load_y(c0, yq[d]);
        }
        asm volatile("" ::: "memory");
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const int c0 = chunk_c0(cb + d);
            if (c0 < 0) break;  // wave-uniform
            // MFMAs of the chunk; D[m][n] lands in the transpose buffer at
            //   G == 1: row n, column 16 nb + m
            //   G > 1:  row RPS sb + n % RPS, column 16 G nb + 16 (n / RPS) + m
            // (m = 4 lg + e, n = lr).
#pragma unroll
            for (int h = 0; h < NH; ++h) {
                if (h > 0) {
                    load_w(c0, h, wf[d]);
                    asm volatile("" ::: "memory");
                }
#pragma unroll
                for (int sb = 0; sb < SB; ++sb) {
                    if (RPS * sb < nrows) {  // wave-uniform
#pragma unroll
                        for (int b = 0; b < NBL; ++b) {
                            const int nb = h * NBL + b;
                            f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                            for (int ks = 0; ks < KS; ++ks) {
                                const bool keep = col_of(c0, nb) < p.N && j0_of(ks) < r;
                                acc = vo[sb][ks].mma_right(wf[d][b][ks].masked(keep), acc);
                            }
                            int trow, tcol;
                            if constexpr (G == 1) {
                                trow = lr;
                                tcol = 16 * nb + 4 * lg;
                            } else {
                                trow = RPS * sb + lr % RPS;
                                tcol = 16 * G * nb + 16 * (lr / RPS) + 4 * lg;
                            }
                            *reinterpret_cast<f32x4_t*>(tw + trow * kDecPitch + tcol) = acc;
                        }
                    }
                }
            }
            __builtin_amdgcn_wave_barrier();
            const bool col_ok = c0 + yc < p.N;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int rt = 8 * u + yr;
                if (rt < nrows && col_ok) {
                    const f32x4_t a0 = *reinterpret_cast<const f32x4_t*>(tw + rt * kDecPitch + yc);
                    const f32x4_t a1 = *reinterpret_cast<const f32x4_t*>(tw + rt * kDecPitch + yc + 4);
                    float yv[8];
                    E::unpack8(&yq[d][u][0], yv);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        yv[e] = yv[e] + s * a0[e];
                        yv[4 + e] = yv[4 + e] + s * a1[e];
                    }
                    const int64_t row = u == 0 ? yrow0 : yrow1;
                    E::store8_nt(ybase + (row * p.ldy + c0 + yc) * EB, yv);
                }
            }
            __builtin_amdgcn_wave_barrier();
        }
    }
}

// Cost of one 64-column chunk of a tile, in bytes moved: its block of B_a
// (64 r elements), its y rows read and written, and a fixed share for the
// tile's setup (records, row indices, v).
__device__ __forceinline__ int64_t dec_chunk_cost(int r, int rows) {
    return 128 * (int64_t)r + 256 * (int64_t)rows + 1024;
}

// Work units of the expand are (16-row tile, 64-column chunk), in tile order.
// Balanced mode: workgroup w of G takes the units whose first byte falls in
// [w C / G, (w + 1) C / G) of the total cost C, so every workgroup moves the
// same number of bytes whatever the ranks and row counts of the tiles it
// meets; w numbers the workgroups XCD by XCD.  Wave 0 loads every tile
// record and table entry (kPlanBlocks x 64 tiles per round: the records
// together, then the entries together), writes the inclusive prefix of the
// tiles' costs (in units of kPlanUnit bytes) to LDS, and the range's ends
// are found there by binary search.  Bad table entries
// cost nothing (workgroup 0 counts them).  Direct mode (small batches, where
// the plan's latency would dominate): workgroup w takes chunks
// [16 c, 16 c + 16) of tile w / ncr, c = w % ncr.
constexpr int kPlanBlocks = 8;
constexpr int kPlanMaxTiles = 2048;  // tiles per call in balanced mode (LDS prefix)
constexpr int kPlanUnit = 256;       // bytes per cost unit in the LDS prefix
constexpr int kDirectChunks = 16;    // chunks per workgroup in direct mode

// Returns {first tile, first chunk, end tile, end chunk} (end exclusive).
__device__ __forceinline__ int4 dec_expand_plan(const DecExpandParams& p, int n16, int nch, int lane,
                                                uint32_t* s_pre) {
    for (int t0 = 0; t0 < n16; t0 += kPlanBlocks * kWave) {
        TileRec rec[kPlanBlocks];
        lora_adapter ads[kPlanBlocks];
        plan_loads<kPlanBlocks>(p.sched, p.tiles16_off, p.adapters, t0, n16, lane, rec, ads);
        uint32_t carry = t0 > 0 ? s_pre[t0 - 1] : 0u;
#pragma unroll
        for (int i = 0; i < kPlanBlocks; ++i) {
            const int t = t0 + kWave * i + lane;
            const lora_adapter& ad = ads[i];
            const bool ok = t < n16 && adapter_ok(ad, p.r_max);
            if (t < n16 && !ok && blockIdx.x == 0) atomicAdd(p.err, 1);
            uint32_t c = ok ? (uint32_t)((nch * dec_chunk_cost(ad.rank, rec[i].rows) + kPlanUnit - 1) / kPlanUnit) : 0u;
            uint32_t incl = c;
#pragma unroll
            for (int d = 1; d < kWave; d <<= 1) {
                const uint32_t o = __shfl_up(incl, d, kWave);
                if (lane >= d) incl += o;
            }
            if (t < n16) s_pre[t] = carry + incl;
            carry += __shfl(incl, kWave - 1, kWave);
        }
    }
    __builtin_amdgcn_wave_barrier();
    const uint64_t total = n16 > 0 ? s_pre[n16 - 1] : 0;
    // ranges in XCD order: the workgroups of one XCD (same blockIdx % 8) take
    // one contiguous eighth of the cost, so the tiles of an adapter share its
    // B_a blocks through one L2 (the grid is a multiple of 8)
    const uint64_t G = gridDim.x;
    const uint64_t w = (uint64_t)(blockIdx.x % kNumXcd) * (G / kNumXcd) + blockIdx.x / kNumXcd;
    const uint64_t lo = total * w / G, hi = total * (w + 1) / G;
    // first unit whose start is at or past x: tile = first with prefix > x,
    // chunk = ceil((x - tile's start) / unit cost)
    auto locate = [&](uint64_t x, int& tt, int& cc) {
        int l = 0, h = n16;  // first t with s_pre[t] > x
        while (l < h) {
            const int m = (l + h) >> 1;
            if ((uint64_t)s_pre[m] > x) h = m;
            else l = m + 1;
        }
        if (l >= n16) {
            tt = n16;
            cc = 0;
            return;
        }
        const uint64_t st = l > 0 ? s_pre[l - 1] : 0;
        const uint64_t tc = s_pre[l] - st;               // tile cost (units)
        const uint64_t c = ((x - st) * nch + tc - 1) / tc;  // ceil((x - st) / (tc / nch))
        tt = c < (uint64_t)nch ? l : l + 1;
        cc = c < (uint64_t)nch ? (int)c : 0;
    };
    int4 plan;
    locate(lo, plan.x, plan.y);
    locate(hi, plan.z, plan.w);
    if (hi >= total) plan.z = n16, plan.w = 0;
    return plan;
}

template <int DT>
__global__ __launch_bounds__(kDecExpWaves * kWave) __attribute__((amdgpu_waves_per_eu(3)))
void dec_expand_kernel(DecExpandParams p) {
    __shared__ __attribute__((aligned(16))) float s_t[kDecExpWaves][16 * kDecPitch];
    __shared__ uint32_t s_pre[kPlanMaxTiles];
    __shared__ int4 s_plan;
    const int wave = wave_id();
    const int lane = threadIdx.x & (kWave - 1);
    const int n16 = p.sched[0];
    const int nch = (p.N + kDecChunk - 1) / kDecChunk;
    int4 plan;
    if (p.balanced) {
        if (wave == 0) {
            const int4 pl = dec_expand_plan(p, min(n16, kPlanMaxTiles), nch, lane, s_pre);
            if (lane == 0) s_plan = pl;
        }
        __syncthreads();
        plan = s_plan;
    } else {
        const int ncr = (nch + kDirectChunks - 1) / kDirectChunks;
        const int t = (int)(blockIdx.x / ncr);
        const int c = (int)(blockIdx.x % ncr) * kDirectChunks;
        plan = t < n16 ? make_int4(t, c, t, min(c + kDirectChunks, nch)) : make_int4(n16, 0, n16, 0);
        // a bad entry is counted by the workgroup of its first chunks
        if (t < n16 && c == 0 && threadIdx.x == 0) {
            const TileRec rec = load_tile(p.sched, p.tiles16_off, t);
            if (!adapter_ok(load_adapter(p.adapters, rec.adapter), p.r_max)) atomicAdd(p.err, 1);
        }
    }
    float* tw = &s_t[wave][0];
    for (int t = plan.x; t <= plan.z && t < n16; ++t) {
        const int cbeg = t == plan.x ? plan.y : 0;
        const int cend = t == plan.z ? plan.w : nch;
        if (cbeg >= cend) continue;
        const TileRec rec = load_tile(p.sched, p.tiles16_off, t);
        const lora_adapter ad = load_adapter(p.adapters, rec.adapter);
        if (!adapter_ok(ad, p.r_max)) continue;  // counted above
        const int r = ad.rank;
        if (r <= 8)
            dec_expand_task<DT, 0>(p, ad, rec, cbeg, cend, wave, lane, tw);
        else if (r <= 16)
            dec_expand_task<DT, 1>(p, ad, rec, cbeg, cend, wave, lane, tw);
        else if (r <= 32)
            dec_expand_task<DT, 2>(p, ad, rec, cbeg, cend, wave, lane, tw);
        else if (r <= 64)
            dec_expand_task<DT, 3>(p, ad, rec, cbeg, cend, wave, lane, tw);
        else
            dec_expand_task<DT, 4>(p, ad, rec, cbeg, cend, wave, lane, tw);
    }
}

}  // namespace lora
