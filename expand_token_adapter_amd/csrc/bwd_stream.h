// bwd_stream.h -- one streaming pass over dY for the backward of adapters of
// rank <= 16 (gfx950, bf16).
//
// Two of the backward's products read dY (DeltaServe section 3.2: the
// backward computes the LoRA gradients):
//   g  = B^T dy               (a reduction over d_out, per row)
//   dB += s sum_rows dy v^T   (a reduction over rows, per column of d_out)
// dy_pass_kernel computes both from one read of each dY byte: g as partial
// sums per 256-column slice (summed by shrink_reduce_kernel), dB directly.
//
// It cuts dY into (adapter, 256-column slice, 32-row window) units and gives
// the grid's workgroups (one per CU) equal contiguous ranges of them
// (stream-K), so a workgroup holds a run of windows of one or two (adapter,
// slice) pairs.  A pair's B_a block is loaded once per workgroup into LDS
// and each wave keeps it in registers as its MFMA operand; the pair's dB tile
// (256 columns x 16 ranks) accumulates in registers over the workgroup's windows:
// a pair whose windows all fall in one workgroup is added to dB there, a pair
// cut by workgroup boundaries leaves one partial tile per workgroup, added in
// workgroup order by the fix-up (dy_fixup_body).  Every sum runs in an order
// fixed by the shapes alone.
//
// Inside a workgroup the four waves take interleaved windows.  A window's dY
// rows (32 rows x 512 bytes, gathered through perm) and its v rows are loaded
// straight into the wave's LDS tiles, two windows in flight, and read back
// row-wise (g) or transposed (ds_read_b64_tr_b16, dB) as MFMA operands; v
// (fp32) enters the bf16 MFMAs as an exact hi/lo pair.
//
// Why rank <= 16 only: the g partials cost 2 r / C of the dY bytes each way
// (C = slice width), and the dB accumulators (C x r fp32 per wave) bound C by
// the register file; at rank 16 that is 12.5% each way, while at rank 32 or
// 64 the partials would cost as much as a second read of dY.  Larger ranks
// take the two-pass backward.
#pragma once

#include "device_common.h"

namespace lora {

constexpr int kStWaves = 4;
// Units a pair costs before its first window in the stream-K split: starting
// a pair (its B_a block, row indices and first windows) takes a workgroup
// about as long as a few windows do, so a workgroup whose range crosses into
// a second pair gets that many windows fewer.  Mixed batch (2048 rows, 56
// slices of 64 windows): backward 48.8 / 48.5 / 47.6 / 46.7 / 46.7 / 48.2 us
// with 0 / 2 / 4 / 6 / 8 / 10 set-up units (14 and 20: 48.2 us).
#ifndef LORA_ST_SETUP
#define LORA_ST_SETUP 6
#endif
constexpr int kStSetupUnits = LORA_ST_SETUP;
constexpr int kStGrid = 256;          // one workgroup per CU
constexpr int kStMaxRank = 16;
constexpr int kStChunk = 1056;        // one load's 1 KB (8 rows x 128 bytes) plus 32 bytes of bank offset
constexpr int kStChunks = 16;         // chunks of a window tile
constexpr int kStTileBytes = kStChunks * kStChunk;
constexpr int kStSmallBytes = 2048;   // a window's rank-16 fp32 rows
constexpr int kStRingBytes = 4 * 256; // row indices of four windows
constexpr int kStFixMeta = 8;
constexpr int kStFixChunk = 1024;     // floats per fix-up workgroup
constexpr int kStBBytes = 256 * 16 * 2;  // a pair's B_a block
static_assert(kStWaves * (2 * (kStTileBytes + kStSmallBytes) + kStRingBytes) + kStBBytes <= 160 * 1024,
              "fits the LDS of a CU");

constexpr int kDyCols = 256;                  // d_out columns per slice
constexpr int kDyFixFloats = kDyCols * 16;    // a cut pair's partial dB tile
static_assert(kStWaves * kStTileBytes >= kStWaves * (kDyCols / 16) * kWave * 16, "the dB sums reuse a buffer's tiles");

// A buffer load of `bytes` (4 or 16) per lane straight into LDS: lane L's
// bytes land at lds + bytes * L (lds wave-uniform); bytes past the buffer
// (voff) are not fetched.  soff (wave-uniform) adds to the memory address
// only.  Issued from assembly: the compiler does not track it, so the caller
// waits (vmcnt) before any read of those LDS bytes and before reusing them.
__device__ __forceinline__ void dma_lds(buf_rsrc_t r, uint32_t voff, uint32_t soff, void* lds, int bytes) {
    const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds;
    if (bytes == 16)
        asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                     :
                     : "s"(m0), "v"(voff), "s"(r), "s"(soff)
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                     :
                     : "s"(m0), "v"(voff), "s"(r), "s"(soff)
                     : "memory", "m0");
}
// The same for 16 bytes with the nontemporal hint: dY is read once, and its
// stream then leaves in L2 the g partials, cut dB tiles, B_a and v that the
// next kernels re-read (mixed batch: backward 52.2 against 55.3 us).
__device__ __forceinline__ void dma_lds16_nt(buf_rsrc_t r, uint32_t voff, uint32_t soff, void* lds) {
    const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds;
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
                 :
                 : "s"(m0), "v"(voff), "s"(r), "s"(soff)
                 : "memory", "m0");
}
__device__ __forceinline__ void buf_store_f32(float x, buf_rsrc_t r, uint32_t voff) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, (int)voff, 0, 0);
}

// ---------------------------------------------------------------- the pair walk
//
// One active adapter's units: slices x 32-row windows of its sorted rows
// (none for an entry the kernels cannot use).
struct StAct {
    int a, lo, hi, nwin;
    int64_t units;
};
struct StWalk {
    const int32_t* sched;
    int64_t active_off;
    const lora_adapter* adapters;
    const int32_t* offsets;
    int32_t r_max;
    int32_t nslices;
    int32_t* fix_meta;  // [grid][2][kStFixMeta]: pair id (lo, hi; -1: none, -2: empty range),
                        // adapter, slice, owner
};
__device__ __forceinline__ StAct st_act(const StWalk& w, int i) {
    StAct c;
    c.a = w.sched[w.active_off + i];
    const lora_adapter ad = load_adapter(w.adapters, c.a);
    c.lo = w.offsets[c.a];
    c.hi = w.offsets[c.a + 1];
    c.nwin = (c.hi - (c.lo & ~31) + 31) / 32;
    c.units = adapter_ok(ad, w.r_max) ? (int64_t)w.nslices * (c.nwin + kStSetupUnits) : 0;
    return c;
}

// Calls pair(c, slice, w0, w1, slot, pair_id) for each (adapter, slice) pair
// of this workgroup's range of units, windows [w0, w1) of the pair; slot 0
// for the range's first pair, 1 for the others (only the first and last can
// be cut).  vg: this workgroup's place in the order.
template <class PairFn>
__device__ __forceinline__ void walk_pairs(const StWalk& w, int vg, int G, PairFn&& pair) {
    const int lane = threadIdx.x & (kWave - 1);
    const int n_act = w.sched[2];
    int32_t* meta = w.fix_meta + (int64_t)vg * 2 * kStFixMeta;
    if (threadIdx.x == 0) {
        meta[0] = -1;
        meta[kStFixMeta] = -1;
    }
    // Total units, this workgroup's range and the active adapter holding its
    // first unit.  Up to 64 active adapters (one per lane) in one pass whose
    // per-lane results also serve every pair below; more adapters in passes of
    // 64, the pairs' adapters then reloaded.
    const bool per_lane = n_act <= kWave;
    StAct mine{};
    int64_t incl = 0, U = 0;
    if (per_lane) {
        if (lane < n_act) mine = st_act(w, lane);
        incl = mine.units;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const int64_t o = __shfl_up(incl, d, kWave);
            if (lane >= d) incl += o;
        }
        U = uniform64(__shfl(incl, kWave - 1, kWave));
    } else {
        for (int b = 0; b < n_act; b += kWave) {
            const int i = b + lane;
            const int64_t un = i < n_act ? st_act(w, i).units : 0;
            U += uniform64(wave_sum64(un));
        }
    }
    const int64_t begin = U * vg / G;
    const int64_t end = U * (vg + 1) / G;
    if (begin >= end) {  // (fewer units than workgroups) the fix-up steps over this one
        if (threadIdx.x == 0) meta[0] = -2;
        return;
    }
    int act = 0;
    int64_t abase = 0;
    if (per_lane) {
        const uint64_t hit = __ballot(lane < n_act && incl - mine.units <= begin && begin < incl);
        act = __ffsll((long long)hit) - 1;
        abase = uniform64(__shfl(incl - mine.units, act, kWave));
    } else {
        for (int b = 0; b < n_act; b += kWave) {
            const int i = b + lane;
            const int64_t un = i < n_act ? st_act(w, i).units : 0;
            int64_t inc = un;
#pragma unroll
            for (int d = 1; d < kWave; d <<= 1) {
                const int64_t o = __shfl_up(inc, d, kWave);
                if (lane >= d) inc += o;
            }
            const uint64_t h = __ballot(i < n_act && abase + inc - un <= begin && begin < abase + inc);
            if (h) {
                const int l = __ffsll((long long)h) - 1;
                act = b + l;
                abase += uniform64(__shfl(inc - un, l, kWave));
                break;
            }
            abase += uniform64(__shfl(inc, kWave - 1, kWave));
        }
    }
    // record of active adapter i: from the lanes in one pass, else reloaded
    auto act_at = [&](int i) -> StAct {
        StAct c;
        if (!per_lane) {
            c = st_act(w, i);
            c.a = __builtin_amdgcn_readfirstlane(c.a);
            c.lo = __builtin_amdgcn_readfirstlane(c.lo);
            c.hi = __builtin_amdgcn_readfirstlane(c.hi);
            c.nwin = __builtin_amdgcn_readfirstlane(c.nwin);
            c.units = uniform64(c.units);
            return c;
        }
        c.a = __builtin_amdgcn_readlane(mine.a, i);
        c.lo = __builtin_amdgcn_readlane(mine.lo, i);
        c.hi = __builtin_amdgcn_readlane(mine.hi, i);
        c.nwin = __builtin_amdgcn_readlane(mine.nwin, i);
        const uint32_t ul = __builtin_amdgcn_readlane((uint32_t)mine.units, i);
        const uint32_t uh = __builtin_amdgcn_readlane((uint32_t)(mine.units >> 32), i);
        c.units = (int64_t)(((uint64_t)uh << 32) | ul);
        return c;
    };
    StAct c = act_at(act);
    int slot = 0;
    for (int64_t u = begin; u < end;) {
        if (u >= abase + c.units) {  // next adapter (u < end <= U: one exists)
            abase += c.units;
            c = act_at(++act);
            continue;
        }
        // a pair is kStSetupUnits set-up units, then its windows
        const int64_t local = u - abase;
        const int per = c.nwin + kStSetupUnits;
        const int cs = (int)(local / per);
        const int v0 = (int)(local - (int64_t)cs * per);
        const int v1 = (int)min((int64_t)per, v0 + (end - u));
        const int w0 = max(v0 - kStSetupUnits, 0), w1 = max(v1 - kStSetupUnits, 0);
        if (w1 > w0) {  // (a range that ends inside a pair's set-up units leaves it to the next workgroup)
            pair(c, cs, w0, w1, slot, abase + (int64_t)cs * per);
            slot = 1;
        }
        u += v1 - v0;
    }
}

// Records a cut pair's partial tile for the fix-up (thread 0).
__device__ __forceinline__ void st_meta(int32_t* fix_meta, int vg, int slot, int64_t pair_id, int a, int cs,
                                        bool owner) {
    if (threadIdx.x != 0) return;
    int32_t* m = fix_meta + ((int64_t)vg * 2 + slot) * kStFixMeta;
    m[0] = (int32_t)(pair_id & 0x7fffffff);
    m[1] = (int32_t)(pair_id >> 31);
    m[2] = a;
    m[3] = cs;
    m[5] = owner;  // holds the pair's first window: runs its fix-up
}

// ---------------------------------------------------------------- window pipeline
//
// LDS of a wave (buffer b = 0, 1): a window tile of kStChunks chunks and a
// small tile (rank-16 fp32 rows), plus a ring of four windows' row indices.
// A chunk is one load: lanes 8 k .. 8 k + 7 take 16 bytes each of row 4 k + m
// of the window, so a lane's rows are 4 (lane / 8) + 0..3 and one 16-byte read
// of the ring gives their indices.  Chunk (4 q + m) of a 512-byte-wide tile
// holds bytes 128 q .. 128 q + 127 of rows 4 k + m; the 32-byte stagger of the
// chunks puts rows 4 k + m (m = 0..3) on different banks, so both the
// row-wise reads (16 rows of one 16-byte unit) and the transposed reads (4
// rows x 32 bytes) are free of bank conflicts.
//
// Every load of a window has a fixed count (a window past the wave's last,
// a row outside the adapter's range or bytes past the matrix load at an
// offset past the buffer: no fetch), issued in this order:
//   prologue  perm(0) perm(1) perm(2) data(0) data(1)
//   window i  [wait data(i)] compute [wait perm(i+2)] perm(i+3) data(i+2) stores(i)
// with perm = 1 load, data = 18 loads, stores = 8 stores.  The compiler does
// not see these loads, so the waits are written out (the constants below);
// a window's row indices arrive before the window ahead of it is issued, so
// waiting for them never waits for data in flight.
struct StLds {
    char* tile;   // [2][kStWaves] window tiles
    char* small;  // [2][kStWaves] small tiles
    char* ring;   // [kStWaves]
    uint16_t* bblk;  // the pair's B_a block, [kDyCols columns][16 ranks] bf16 (workgroup-wide)
};
__device__ __forceinline__ char* st_tile(const StLds& l, int b, int wave) {
    return l.tile + (b * kStWaves + wave) * kStTileBytes;
}
__device__ __forceinline__ char* st_small(const StLds& l, int b, int wave) {
    return l.small + (b * kStWaves + wave) * kStSmallBytes;
}
// waits before window i's data and before window i + 2's row indices
__device__ __forceinline__ void st_wait_data(int i) {
    if (i == 0)
        wait_vmcnt_le<18>();
    else if (i == 1)
        wait_vmcnt_le<27>();
    else
        wait_vmcnt_le<35>();
}
__device__ __forceinline__ void st_wait_perm(int i) {
    if (i == 0)
        wait_vmcnt_le<36>();
    else
        wait_vmcnt_le<26>();
}

// ---------------------------------------------------------------- the dY pass

struct DyParams {
    const void* dy;        // [T][lddy] bf16, rows through perm
    int64_t lddy;
    uint32_t dy_bytes;     // bytes from dy to the end of its last row (< 2^31)
    int32_t d_out;
    const float* v;        // [row][ldv]: row = original row, or sorted position if v_by_pos
    int64_t ldv;
    uint32_t v_bytes;      // bytes from v to the end of its last row (< 2^31)
    int32_t v_by_pos;
    const lora_adapter_grad* grads;
    const int32_t* perm;
    int32_t T;
    float* gpart;          // [nslices][T][16]
    uint32_t gpart_bytes;  // nslices * T * 64 (< 2^31)
    float* fix;            // [grid][2][kDyFixFloats] partial dB tiles of cut pairs
    StWalk walk;           // nslices = ceil(d_out / kDyCols)
    int32_t* err;          // counts active adapters with a bad entry or no gradient entry
    const int32_t* stop;   // backward preemption: the workgroup does nothing when *stop != 0
};

// Windows [w0, w1) of pair (adapter c.a, slice cs): g partials, dB tile.
__device__ __forceinline__ void dy_pair(const DyParams& p, const StAct& c, int cs, int w0, int w1, int slot, int vg,
                                        int64_t pair_id, const StLds& L, int wave, int lane) {
    using F = Frag<LORA_BF16>;
    using O = F32Operand<LORA_BF16>;
    constexpr int CT = kDyCols / 16;  // 16-column tiles (16)
    constexpr int KS = kDyCols / 32;  // 32-column steps of g (8)
    const int lr = lane & 15;
    const int lg = lane >> 4;
    const int c0 = cs * kDyCols;
    const int lo = c.lo, hi = c.hi;
    const int wbase = lo & ~31;

    f32x4_t accB[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) accB[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const buf_rsrc_t dyr = make_rsrc(p.dy, p.dy_bytes);
    const buf_rsrc_t vr = make_rsrc(p.v, p.v_bytes);
    const buf_rsrc_t pr = make_rsrc(p.perm, (uint32_t)p.T * 4u);
    const buf_rsrc_t gpr = make_rsrc(p.gpart, p.gpart_bytes);
    // loads: chunk (4 q + m), q < 4: dY bytes 128 q.. of rows 4 lk + m; the
    // v rows (64 bytes) in two loads j: 16 bytes (unit lane % 4) of row
    // 4 lk + 2 j + (lane / 4) % 2, into the small tile at 1024 j + 16 lane
    const int lk = lane >> 3;
    const int l8 = lane & 7;
    const int vt = (lane >> 2) & 1;
    const int vu = lane & 3;
    const uint32_t coff = (uint32_t)c0 * 2u + 16u * l8;
    const uint32_t ldy2 = (uint32_t)p.lddy * 2u;
    const uint32_t ldv4 = (uint32_t)p.ldv * 4u;
    const int sunits = min(kDyCols, p.d_out - c0) / 8;  // 16-byte units of the slice inside d_out
    const int nw = (w1 - w0 - wave + kStWaves - 1) / kStWaves;  // windows w0 + wave + 4 i, i < nw
    auto wpos_of = [&](int i) { return wbase + 32 * (w0 + wave + kStWaves * i); };
    char* ring = L.ring + wave * kStRingBytes;
    auto issue_perm = [&](int i) {
        const int pos = wpos_of(i) + lane;
        dma_lds(pr, i < nw && lane < 32 ? (uint32_t)pos * 4u : kBufOff, 0u, ring + (i & 3) * 256, 4);
    };
    auto read_perm = [&](int i) -> u32x4_t {
        return *reinterpret_cast<const u32x4_t*>(ring + (i & 3) * 256 + 16 * lk);
    };
    auto issue = [&](int b, int i, const u32x4_t& prow) {
        const int pos0 = wpos_of(i) + 4 * lk;
        char* tile = st_tile(L, b, wave);
        char* small = st_small(L, b, wave);
        uint32_t off[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int pos = pos0 + m;
            off[m] = i < nw && pos >= lo && pos < hi ? prow[m] * ldy2 + coff : kBufOff;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int m = 0; m < 4; ++m)
                dma_lds16_nt(dyr, 8 * q + l8 < sunits ? off[m] : kBufOff, 128u * q, tile + (4 * q + m) * kStChunk);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int pos = pos0 + 2 * j + vt;
            const bool ok = i < nw && pos >= lo && pos < hi;
            const uint32_t vrow = p.v_by_pos ? (uint32_t)pos : (vt ? prow[2 * j + 1] : prow[2 * j]);
            dma_lds(vr, ok ? vrow * ldv4 + 16u * vu : kBufOff, 0u, small + j * 1024, 16);
        }
    };
    // The first windows' row indices go out before anything that needs the
    // adapter's entry; then the B_a block (16 two-byte loads per thread for
    // the whole workgroup) and the first two windows' data are in flight
    // together.  (With the block gathered by every wave in operand layout,
    // 64 loads per lane behind the entry and ahead of the row indices, a
    // pair took 5.5 us from its start to its first window's data.)
    issue_perm(0);
    issue_perm(1);
    issue_perm(2);
    const lora_adapter ad = load_adapter(p.walk.adapters, c.a);
    const lora_adapter_grad gr = load_grad(p.grads, c.a);
    const int r = ad.rank;
    uint32_t hb[kStBBytes / 2 / (kStWaves * kWave)];
    {
        const buf_rsrc_t brs = make_rsrc(ad.B, (uint32_t)((int64_t)p.d_out * r * 2));
        // element e = column e / 16, rank e % 16 of the block; ranks past r and
        // columns past d_out read zeros (offset past the buffer, no fetch)
#pragma unroll
        for (int j = 0; j < kStBBytes / 2 / (kStWaves * kWave); ++j) {
            const int e = (int)threadIdx.x + kStWaves * kWave * j;
            const int col = c0 + (e >> 4), rk = e & 15;
            const bool ok = rk < r && col < p.d_out;
            hb[j] = __builtin_amdgcn_raw_buffer_load_b16(brs, ok ? (uint32_t)((col * r + rk) * 2) : kBufOff, 0, 0);
        }
    }
    constexpr int kB = kStBBytes / 2 / (kStWaves * kWave);  // B loads issued after the row indices
    wait_vmcnt_le<2 + kB>();                                  // perm(0)
    issue(0, 0, read_perm(0));
    wait_vmcnt_le<1 + kB + 18>();                             // perm(1)
    issue(1, 1, read_perm(1));
    // The block to LDS (the compiler waits for its loads, and with them for
    // the windows' loads issued before them), then every wave's B operand:
    // rank lr, columns c0 + 32 ks + 8 lg + 0..7, read transposed.
#pragma unroll
    for (int j = 0; j < kB; ++j) L.bblk[threadIdx.x + kStWaves * kWave * j] = (uint16_t)hb[j];
    __syncthreads();
    F bf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const uint16_t* base = L.bblk + (32 * ks + 8 * lg + (lr >> 2)) * 16 + 4 * (lane & 3);
        const uint2 x0 = lds_read_tr16(base);
        const uint2 x1 = lds_read_tr16(base + 4 * 16);
        bf[ks].q = u32x4_t{x0.x, x0.y, x1.x, x1.y};
    }

    // per-lane LDS offsets of the operand reads
    const int e = lr >> 2;
    const int cc = lane & 3;
    const int g_off = (lr & 3) * kStChunk + 128 * (lr >> 2) + 16 * lg;         // rows 16 rt + lr, unit 4 ks + lg
    const int t_off = e * kStChunk + 256 * lg + 16 * (cc >> 1) + 8 * (cc & 1);  // transposed: rows 8 lg + e
    const int v_off = 256 * lg + 4 * lr;                                         // v: rank lr, rows 8 lg + jj
    for (int ii = 0; ii < nw; ++ii) {
        const int b = ii & 1;
        const int wpos = wpos_of(ii);
        st_wait_data(ii);
        const char* tile = st_tile(L, b, wave);
        const char* small = st_small(L, b, wave);

        // g partial: window rows 16 rt + lr x slice columns (A), B_a block (B)
        f32x4_t ag[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
                ag[rt] = mma(F::load_lds(tile + g_off + 4 * (ks >> 1) * kStChunk + 512 * rt + 64 * (ks & 1)), bf[ks],
                             ag[rt]);
        // v operand of dB: rank lr, window rows 8 lg + jj (ranks past r hold
        // other data; they only reach dB columns that are never stored)
        float vf[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
            vf[jj] = *reinterpret_cast<const float*>(small + v_off + 1024 * ((jj >> 1) & 1) + 128 * (jj >> 2) +
                                                     64 * (jj & 1));
        const O vo = O::make(vf);
        // dB: A operand = the window transposed (column 16 ct + lr, rows
        // 8 lg .. 8 lg + 7), B operand = v (rank lr, the same rows)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const uint16_t* base =
                reinterpret_cast<const uint16_t*>(tile + t_off + 4 * (ct >> 2) * kStChunk + 32 * (ct & 3));
            const uint2 x0 = lds_read_tr16(base);
            const uint2 x1 = lds_read_tr16(base + 64);  // rows + 4: the next 128-byte block
            accB[ct] = vo.mma_right(F{u32x4_t{x0.x, x0.y, x1.x, x1.y}}, accB[ct]);
        }
        // every read of this window's tiles has returned: they take window ii + 2
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        st_wait_perm(ii);
        const u32x4_t prow = read_perm(ii + 2);
        issue_perm(ii + 3);
        issue(b, ii + 2, prow);
        // D rows 4 lg + q = window rows, column lr = rank; rows outside the
        // adapter's range are not stored (offset past the buffer)
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int pos = wpos + 16 * rt + 4 * lg + q;
                const bool ok = pos >= lo && pos < hi;
                const uint32_t off = ((uint32_t)cs * (uint32_t)p.T + (uint32_t)pos) * 64u + 4u * lr;
                buf_store_f32(ag[rt][q], gpr, ok ? off : kBufOff);
            }
        asm volatile("" ::: "memory");
    }
    wait_vmcnt_le<0>();  // loads past the last window still write the tiles

    // The waves' dB tiles in wave order; wave w finishes tiles 4 w .. 4 w + 3.
    __syncthreads();
    f32x4_t* red = reinterpret_cast<f32x4_t*>(L.tile);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) red[(wave * CT + ct) * kWave + lane] = accB[ct];
    __syncthreads();
    const bool whole = w0 == 0 && w1 == c.nwin;
    constexpr int kPer = CT / kStWaves;
    f32x4_t sum[kPer];
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const int ct = kPer * wave + q;
        sum[q] = red[ct * kWave + lane];
#pragma unroll
        for (int w = 1; w < kStWaves; ++w) sum[q] += red[(w * CT + ct) * kWave + lane];
    }
    if (!whole) {
        f32x4_t* f = reinterpret_cast<f32x4_t*>(p.fix + ((int64_t)vg * 2 + slot) * kDyFixFloats);
#pragma unroll
        for (int q = 0; q < kPer; ++q) *gptr(f + (kPer * wave + q) * kWave + lane) = sum[q];
        st_meta(p.walk.fix_meta, vg, slot, pair_id, c.a, cs, w0 == 0);
    } else if (gr.dA && gr.dB) {
        // D rows 4 lg + i = columns, column lr = rank: dB[col][rank] += s sum.
        // Loads first (entries outside the matrix read its first entry and
        // are not written), then the stores.
        float* dst[kPer][4];
        bool ok[kPer][4];
        float old[kPer][4];
#pragma unroll
        for (int q = 0; q < kPer; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int col = c0 + 16 * (kPer * wave + q) + 4 * lg + i;
                ok[q][i] = col < p.d_out && lr < r;
                dst[q][i] = gr.dB + (ok[q][i] ? (int64_t)col * r + lr : 0);
                old[q][i] = *gptr(dst[q][i]);
            }
#pragma unroll
        for (int q = 0; q < kPer; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (ok[q][i]) *gptr(dst[q][i]) = old[q][i] + ad.scale * sum[q][i];
    }
    __syncthreads();  // the tiles' LDS is rewritten by the next pair
}

// ---------------------------------------------------------------- kernels

// XCD-aware place of this workgroup (workgroup b runs on XCD b % 8):
// workgroups of one XCD take neighbouring ranges.
__device__ __forceinline__ int st_place() {
    const int G = gridDim.x;
    return (int)(blockIdx.x % kNumXcd) * (G / kNumXcd) + (int)(blockIdx.x / kNumXcd);
}

#define LORA_ST_LDS                                                                   \
    __shared__ __attribute__((aligned(16))) char s_t[2 * kStWaves * kStTileBytes];    \
    __shared__ __attribute__((aligned(16))) char s_s[2 * kStWaves * kStSmallBytes];   \
    __shared__ __attribute__((aligned(16))) char s_r[kStWaves * kStRingBytes];        \
    __shared__ __attribute__((aligned(16))) uint16_t s_b[kStBBytes / 2];              \
    const StLds L{s_t, s_s, s_r, s_b};

__global__ __launch_bounds__(kStWaves * kWave) __attribute__((amdgpu_waves_per_eu(1, 1)))
void dy_pass_kernel(DyParams p) {
    LORA_ST_LDS
    if (p.stop && *p.stop) return;
    const int wave = wave_id();
    const int lane = threadIdx.x & (kWave - 1);
    const int vg = st_place();
    if (blockIdx.x == 0 && wave == 0) {  // entries the passes skip, once each
        const int n_act = p.walk.sched[2];
        for (int i = lane; i < n_act; i += kWave) {
            const int a = p.walk.sched[p.walk.active_off + i];
            const lora_adapter ad = load_adapter(p.walk.adapters, a);
            const lora_adapter_grad gr = load_grad(p.grads, a);
            if (!adapter_ok(ad, p.walk.r_max) || !gr.dA || !gr.dB) atomicAdd(p.err, 1);
        }
    }
    walk_pairs(p.walk, vg, gridDim.x, [&](const StAct& c, int cs, int w0, int w1, int slot, int64_t id) {
        dy_pair(p, c, cs, w0, w1, slot, vg, id, L, wave, lane);
    });
}

#undef LORA_ST_LDS

// ---------------------------------------------------------------- fix-up
//
// Adds the partial tiles of each cut pair in workgroup order, then s times
// the sum to the gradient.  A 256-thread workgroup handles kStFixChunk floats
// (one quad per thread) of the pair that pass workgroup g0 owns, if any: the
// later workgroups holding the same pair are found from their records, 64 at
// a time, and their partial tiles added in workgroup order.  apply(a, cs,
// quad, sum) adds one quad of the tile to the gradient.
template <class Apply>
__device__ __forceinline__ void st_fixup(const float* fix, const int32_t* fix_meta, int tile_floats, int G, int g0,
                                         int chunk, Apply&& apply) {
    const int t = threadIdx.x;
    const int lane = t & (kWave - 1);
    for (int sl = 0; sl < 2; ++sl) {
        const int32_t* m = fix_meta + ((int64_t)g0 * 2 + sl) * kStFixMeta;
        if (m[0] < 0 || !m[5]) continue;
        const int32_t id0 = m[0], id1 = m[1];
        const int a = m[2], cs = m[3];
        const int64_t q0 = (int64_t)chunk * (kStFixChunk / 4) + t;  // this thread's quad of the tile
        f32x4_t sum = *gptr(reinterpret_cast<const f32x4_t*>(fix + ((int64_t)g0 * 2 + sl) * tile_floats) + q0);
        // followers: workgroups after g0 whose first pair is this one (those
        // with an empty range are stepped over), up to the first that differs
        for (int gb = g0 + 1; gb < G; gb += kWave) {
            const int gl = gb + lane;
            int32_t m0 = -1, m1 = -1;
            if (gl < G) {
                m0 = fix_meta[(int64_t)gl * 2 * kStFixMeta];
                m1 = fix_meta[(int64_t)gl * 2 * kStFixMeta + 1];
            }
            const bool match = gl < G && m0 == id0 && m1 == id1;
            const bool stop = !(match || (gl < G && m0 == -2));
            const uint64_t stops = __ballot(stop);
            uint64_t take = __ballot(match);
            if (stops) take &= (stops & (0 - stops)) - 1;  // lanes before the first stop
            take = (uint64_t)uniform64((int64_t)take);
            while (take) {  // eight partial tiles in flight at a time, added in workgroup order
                int ls[8];
                f32x4_t pv[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    ls[j] = take ? __ffsll((long long)take) - 1 : -1;
                    take &= take - 1;
                }
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    pv[j] = *gptr(reinterpret_cast<const f32x4_t*>(fix + (int64_t)(gb + max(ls[j], 0)) * 2 * tile_floats) +
                                  q0);
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (ls[j] >= 0) sum += pv[j];
            }
            if (stops) break;
        }
        apply(a, cs, (int)q0, sum);
    }
}

constexpr int kDyFixParts = kDyFixFloats / kStFixChunk;  // fix-up workgroups per pass workgroup (4)

// The fix-up of pass 1's cut dB tiles, as workgroup `part` of a 256-thread
// grid part of kStGrid * kDyFixParts workgroups.
__device__ __forceinline__ void dy_fixup_body(const DyParams& q, int part) {
    if (q.stop && *q.stop) return;
    st_fixup(q.fix, q.walk.fix_meta, kDyFixFloats, kStGrid, part / kDyFixParts, part % kDyFixParts,
             [&](int a, int cs, int quad, f32x4_t sum) {
                 const lora_adapter ad = load_adapter(q.walk.adapters, a);
                 const lora_adapter_grad gr = load_grad(q.grads, a);
                 if (!gr.dA || !gr.dB) return;
                 const int r = ad.rank;
                 // quad = tile ct, lane ln of the pass: columns 16 ct + 4 (ln / 16) + i, rank ln % 16
                 const int ct = quad / kWave, ln = quad % kWave, rk = ln & 15;
                 float* dst[4];
                 bool ok[4];
                 float old[4];
#pragma unroll
                 for (int i = 0; i < 4; ++i) {
                     const int col = cs * kDyCols + 16 * ct + 4 * (ln >> 4) + i;
                     ok[i] = col < q.d_out && rk < r;
                     dst[i] = gr.dB + (ok[i] ? (int64_t)col * r + rk : 0);
                     old[i] = *gptr(dst[i]);
                 }
#pragma unroll
                 for (int i = 0; i < 4; ++i)
                     if (ok[i]) *gptr(dst[i]) = old[i] + ad.scale * sum[i];
             });
}

}  // namespace lora
