// segments.hip -- group the rows of a batch by adapter.
//
// Multi-LoRA batching applies each row's own adapter inside one shared pass
// (DeltaServe, section 2.2).  The compute kernels therefore need, for every
// adapter, the list of its rows: a counting sort of the rows by adapter id.
//
// General path: three kernels, all deterministic (the order inside an
// adapter is the row order, never the order in which threads happen to run):
//   1. seg_count   one workgroup per chunk of kChunk rows: each row's rank
//                  among the earlier rows of its chunk with the same id, and
//                  the per-(adapter, chunk) counts.
//   2. seg_scan    one workgroup: per-adapter prefix over chunks, exclusive
//                  scans over adapters (offsets, tile prefixes, active list).
//   3. seg_scatter one workgroup per chunk: perm[pos] = row, plus the tile
//                  records the shrink / expand / backward kernels walk.
#include "device_common.h"

namespace lora {

constexpr int kChunk = 256;
constexpr int kScanThreads = 1024;

// Workspace layout (int32 elements), regions aligned to 64 elements.
struct SegWs {
    int64_t hist, rank, errc, pre16, pre64, total;
    static SegWs make(int64_t T, int64_t A) {
        auto al = [](int64_t n) { return (n + 63) / 64 * 64; };
        const int64_t nchunks = (T + kChunk - 1) / kChunk;
        SegWs w;
        w.hist = 0;
        w.rank = w.hist + al(A * nchunks);
        w.errc = w.rank + al(T);
        w.pre16 = w.errc + al(nchunks);
        w.pre64 = w.pre16 + al(A);
        w.total = w.pre64 + al(A);
        return w;
    }
};

__global__ __launch_bounds__(kChunk) void seg_count_kernel(const int32_t* __restrict__ ids, int32_t T, int32_t A,
                                                           int32_t nchunks, int32_t* __restrict__ hist,
                                                           int32_t* __restrict__ rank, int32_t* __restrict__ errc) {
    __shared__ int32_t s_ids[kChunk];
    __shared__ int32_t s_err[kChunk / kWave];
    const int c = blockIdx.x;
    const int tid = threadIdx.x;
    const int64_t t = (int64_t)c * kChunk + tid;
    const int32_t id = t < T ? ids[t] : -1;
    const bool valid = id >= 0 && id < A;
    const bool bad = t < T && !valid && id != -1;
    s_ids[tid] = valid ? id : -1;
    // This workgroup owns column c of hist[A][nchunks]; clear it first.
    for (int a = tid; a < A; a += kChunk) hist[(int64_t)a * nchunks + c] = 0;
    __syncthreads();
    int before = 0, same = 0;
#pragma unroll 16
    for (int j = 0; j < kChunk; ++j) {
        const int eq = s_ids[j] == id;
        same += eq;
        before += eq & (j < tid);
    }
    if (valid) {
        rank[t] = before;
        if (before + 1 == same) hist[(int64_t)id * nchunks + c] = same;  // last row of this id in the chunk
    }
    const uint64_t m = __ballot(bad);
    if ((tid & (kWave - 1)) == 0) s_err[tid / kWave] = __popcll(m);
    __syncthreads();
    if (tid == 0) {
        int e = 0;
        for (int w = 0; w < kChunk / kWave; ++w) e += s_err[w];
        errc[c] = e;
    }
}

__device__ __forceinline__ int wave_inclusive_scan(int v) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int o = __shfl_up(v, d, kWave);
        if (lane >= d) v += o;
    }
    return v;
}

// Exclusive scan of one int per thread across the workgroup; returns the
// exclusive prefix and writes the workgroup total to *total.
__device__ __forceinline__ int block_exclusive_scan(int v, int* s_tot, int* total) {
    constexpr int kWaves = kScanThreads / kWave;
    const int w = wave_id();
    const int lane = threadIdx.x & (kWave - 1);
    const int incl = wave_inclusive_scan(v);
    if (lane == kWave - 1) s_tot[w] = incl;
    __syncthreads();
    int before = 0, all = 0;
    for (int i = 0; i < kWaves; ++i) {
        const int x = s_tot[i];
        before += i < w ? x : 0;
        all += x;
    }
    __syncthreads();
    *total = all;
    return before + incl - v;
}

__global__ __launch_bounds__(kScanThreads) void seg_scan_kernel(int32_t A, int32_t nchunks, int32_t* __restrict__ hist,
                                                                const int32_t* __restrict__ errc,
                                                                int32_t* __restrict__ counts,
                                                                int32_t* __restrict__ offsets,
                                                                int32_t* __restrict__ sched,
                                                                int32_t* __restrict__ pre16,
                                                                int32_t* __restrict__ pre64, int32_t* __restrict__ err,
                                                                int64_t active_off) {
    __shared__ int s_tot[4][kScanThreads / kWave];
    const int tid = threadIdx.x;
    // Per adapter: exclusive prefix of its chunk counts (in place), total = count.
    for (int a = tid; a < A; a += kScanThreads) {
        int32_t* h = hist + (int64_t)a * nchunks;
        int run = 0;
        for (int c = 0; c < nchunks; ++c) {
            const int x = h[c];
            h[c] = run;
            run += x;
        }
        counts[a] = run;
    }
    __syncthreads();
    int carry_c = 0, carry16 = 0, carry64 = 0, carry_act = 0;
    int32_t* active = sched + active_off;
    for (int base = 0; base < A; base += kScanThreads) {
        const int a = base + tid;
        const int c = a < A ? counts[a] : 0;
        int tc, t16, t64, tact;
        const int ec = block_exclusive_scan(c, s_tot[0], &tc);
        const int e16 = block_exclusive_scan((c + 15) / 16, s_tot[1], &t16);
        const int e64 = block_exclusive_scan((c + 63) / 64, s_tot[2], &t64);
        const int eact = block_exclusive_scan(c > 0 ? 1 : 0, s_tot[3], &tact);
        if (a < A) {
            offsets[a] = carry_c + ec;
            pre16[a] = carry16 + e16;
            pre64[a] = carry64 + e64;
            if (c > 0) active[carry_act + eact] = a;
        }
        carry_c += tc;
        carry16 += t16;
        carry64 += t64;
        carry_act += tact;
    }
    if (tid == 0) {
        offsets[A] = carry_c;
        sched[0] = carry16;
        sched[1] = carry64;
        sched[2] = carry_act;
        sched[3] = 0;
        int e = 0;
        for (int c = 0; c < nchunks; ++c) e += errc[c];
        err[0] = e;
    }
}

__global__ __launch_bounds__(kChunk) void seg_scatter_kernel(const int32_t* __restrict__ ids, int32_t T, int32_t A,
                                                             int32_t nchunks, const int32_t* __restrict__ hist,
                                                             const int32_t* __restrict__ rank,
                                                             const int32_t* __restrict__ counts,
                                                             const int32_t* __restrict__ offsets,
                                                             const int32_t* __restrict__ pre16,
                                                             const int32_t* __restrict__ pre64,
                                                             int32_t* __restrict__ perm, int32_t* __restrict__ sched,
                                                             int64_t tiles16_off, int64_t tiles64_off) {
    const int c = blockIdx.x;
    const int64_t t = (int64_t)c * kChunk + threadIdx.x;
    if (t >= T) return;
    const int32_t id = ids[t];
    if (id < 0 || id >= A) return;
    const int32_t local = hist[(int64_t)id * nchunks + c] + rank[t];  // position inside the adapter's group
    const int32_t pos = offsets[id] + local;
    perm[pos] = (int32_t)t;
    const int32_t cnt = counts[id];
    if ((local & 15) == 0) {
        int32_t* rec = sched + tiles16_off + 4 * (int64_t)(pre16[id] + local / 16);
        const int32_t rows = cnt - local < 16 ? cnt - local : 16;
        *reinterpret_cast<int4*>(rec) = make_int4(id, pos, rows, 0);
    }
    if ((local & 63) == 0) {
        int32_t* rec = sched + tiles64_off + 4 * (int64_t)(pre64[id] + local / 64);
        const int32_t rows = cnt - local < 64 ? cnt - local : 64;
        *reinterpret_cast<int4*>(rec) = make_int4(id, pos, rows, 0);
    }
}

// ---------------------------------------------------------------- one workgroup
//
// For batches of up to kSmallMaxT rows and kSmallMaxA adapters the whole
// build runs in one workgroup of 16 waves (one launch instead of three).
// Wave w owns a contiguous range of rows; its first 512 ids are loaded once,
// before anything else, and stay in registers for both passes together with
// each lane's match inside its group (longer ranges load and match the rest
// again in the second pass; the matching is most of the kernel's ALU work):
//   1. wave w counts its ids into its own LDS histogram row hist[w][a], one
//      update per distinct id of each 64-row group (a group holding one id is
//      matched by one ballot; other groups by one ballot per id bit);
//   2. per adapter: counts = sum over w, hist[w][a] becomes the exclusive
//      prefix over waves; one scan of four values per adapter (within wave 0
//      when the adapters fit in one wave, else across the workgroup) gives
//      offsets, both tile prefixes and the active list;
//   3. wave w walks its rows in order, 64 at a time; inside a group the lanes
//      that share an id are ranked by lane order (the same ballot match), and
//      the wave's cursor for that id advances by the group's count.  Every row's
//      position is therefore its rank in row order: the same stable grouping
//      as the three-kernel path.
// Only LDS is waited on at the barriers; the global stores of one phase
// never hold up the next.

// Lanes of this wave holding the same valid id as the calling lane (0 for an
// invalid one), from one ballot per bit of the ids (ids < 2^nbits): a lane
// matches when it agrees on every bit.
__device__ __forceinline__ uint64_t same_id_lanes(int id, bool valid, int nbits) {
    uint64_t m = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (id >> b) & 1;
        const uint64_t set = __ballot(valid && bit);
        m &= bit ? set : ~set;
    }
    return valid ? m : 0ull;
}


// Inclusive scan of four ints across the first n (a power of two) lanes of a wave.
template <int n>
__device__ __forceinline__ int4 wave_inclusive_scan4(int4 v, int lane) {
    int4 incl = v;
#pragma unroll
    for (int d = 1; d < n; d <<= 1) {
        const int4 o = make_int4(__shfl_up(incl.x, d, kWave), __shfl_up(incl.y, d, kWave),
                                 __shfl_up(incl.z, d, kWave), __shfl_up(incl.w, d, kWave));
        if (lane >= d) incl = incl + o;
    }
    return incl;
}

// Exclusive scan of four ints per thread across the workgroup.  Each wave
// scans its lanes; wave 0 then scans the wave totals (s_tot[0, W) in, their
// exclusive prefixes to s_tot[W, 2W), the workgroup totals to s_tot[2W]),
// and every wave reads back its own prefix and the totals: two LDS barriers
// and two reads per wave, instead of every wave summing all W totals.
// s_tot holds 2W + 1 entries (W waves) and is used once.  Returns the
// exclusive prefixes and writes the workgroup totals to *total.
__device__ __forceinline__ int4 block_exclusive_scan4(int4 v, int4* s_tot, int4* total) {
    constexpr int kWaves = kScanThreads / kWave;
    const int w = wave_id();
    const int lane = threadIdx.x & (kWave - 1);
    const int4 incl = wave_inclusive_scan4<kWave>(v, lane);
    if (lane == kWave - 1) s_tot[w] = incl;
    lds_barrier();
    if (w == 0) {
        const int4 t = lane < kWaves ? s_tot[lane] : make_int4(0, 0, 0, 0);
        const int4 ti = wave_inclusive_scan4<kWaves>(t, lane);
        if (lane < kWaves) s_tot[kWaves + lane] = ti - t;
        if (lane == kWaves - 1) s_tot[2 * kWaves] = ti;
    }
    lds_barrier();
    *total = s_tot[2 * kWaves];
    return s_tot[kWaves + w] + incl - v;
}

constexpr int kSmallMaxA = 1024;
constexpr int kSmallMaxT = 1 << 16;
constexpr int kSmallWaves = kScanThreads / kWave;
constexpr int kSmallBatch = 8;  // 64-row groups per load batch

// One build of the one-workgroup path; a launch carries up to kSegBatchMax
// independent builds, one workgroup each (blockIdx.x selects the build).
struct SegSmallJob {
    const int32_t* ids;
    int32_t T;
    int32_t* counts;
    int32_t* offsets;
    int32_t* perm;
    int32_t* sched;
    int32_t* err;
    int64_t active_off, tiles16_off, tiles64_off;
};
constexpr int kSegBatchMax = LORA_SEG_BATCH_MAX;
struct SegSmallJobs {
    SegSmallJob job[kSegBatchMax];
};

__global__ __launch_bounds__(kScanThreads) void seg_small_kernel(SegSmallJobs jobs, int32_t A) {
    const SegSmallJob& job = jobs.job[blockIdx.x];
    const int32_t* __restrict__ ids = job.ids;
    const int32_t T = job.T;
    int32_t* __restrict__ counts = job.counts;
    int32_t* __restrict__ offsets = job.offsets;
    int32_t* __restrict__ perm = job.perm;
    int32_t* __restrict__ sched = job.sched;
    int32_t* __restrict__ err = job.err;
    const int64_t active_off = job.active_off, tiles16_off = job.tiles16_off, tiles64_off = job.tiles64_off;
    __shared__ int s_hist[kSmallWaves][kSmallMaxA];
    __shared__ int4 s_info[kSmallMaxA];  // offset, count, 16-row tile prefix, 64-row tile prefix
    __shared__ int4 s_tot[2 * kSmallWaves + 1];
    __shared__ int s_err[kSmallWaves];
    const int tid = threadIdx.x;
    const int w = wave_id();
    const int lane = tid & (kWave - 1);
    const int per = (T + kSmallWaves - 1) / kSmallWaves;
    const int r0 = min(T, w * per);
    const int r1 = min(T, r0 + per);
    const int nbits = A > 1 ? 32 - __clz(A - 1) : 1;  // bits of the largest id
    constexpr int kStep = kSmallBatch * kWave;

    auto load_batch = [&](int b, int* idv) {
#pragma unroll
        for (int g = 0; g < kSmallBatch; ++g) {
            const int t = b + g * kWave + lane;
            idv[g] = t < r1 ? ids[t] : -1;
        }
    };
    int id0[kSmallBatch];
    load_batch(r0, id0);
    // Each wave clears its own histogram row (no other wave touches it before the barrier).
    for (int a = lane; a < A; a += kWave) s_hist[w][a] = 0;

    // A lane's match inside its 64-row group: rank among the lanes with its id
    // (bits 0-7), their number (bits 8-15), bit 16 set on the lowest of them;
    // 0 for a lane without a valid id.
    auto match = [&](int id, bool valid) {
        // A group whose valid lanes all hold one id (a run of prefill or
        // fine-tuning rows) matches on the valid lanes at once; only mixed
        // groups take one ballot per id bit.  (Wave-uniform branch.)
        const uint64_t vm = __ballot(valid);
        const int l0 = vm ? __ffsll((long long)vm) - 1 : 0;
        const int id0 = __builtin_amdgcn_readlane(id, l0);
        const uint64_t m = __ballot(valid && id == id0) == vm ? (valid ? vm : 0ull) : same_id_lanes(id, valid, nbits);
        const int rank = __popcll(m & ((1ull << lane) - 1));
        return valid ? rank | (__popcll(m) << 8) | (rank == 0 ? 1 << 16 : 0) : 0;
    };
    // 1. count: the lowest lane holding each id adds the group's count of that id.
    int bad = 0;
    int mt0[kSmallBatch];
    auto count_batch = [&](int b, const int* idv, int* mt) {
#pragma unroll
        for (int g = 0; g < kSmallBatch; ++g) {
            mt[g] = 0;
            if (b + g * kWave < r1) {  // wave-uniform: skip empty groups
                const int id = idv[g];
                const bool valid = id >= 0 && id < A;
                bad += (!valid && id != -1) ? 1 : 0;
                mt[g] = match(id, valid);
                if (mt[g] & (1 << 16)) s_hist[w][id] += mt[g] >> 8 & 0xff;
            }
        }
    };
    count_batch(r0, id0, mt0);
    for (int b = r0 + kStep; b < r1; b += kStep) {
        int idv[kSmallBatch], mt[kSmallBatch];
        load_batch(b, idv);
        count_batch(b, idv, mt);
    }
    bad = __reduce_add_sync(~0ull, bad);
    if (lane == 0) s_err[w] = bad;
    lds_barrier();

    // 2. per adapter: total and exclusive prefix over the waves, then the scans over adapters
    const int a = tid;
    int c = 0;
    if (a < A) {
        for (int v = 0; v < kSmallWaves; ++v) {
            const int h = s_hist[v][a];
            s_hist[v][a] = c;
            c += h;
        }
    }
    // (rows, 16-row tiles, 64-row tiles, active) of adapter a, scanned over the adapters
    const int4 v4 = make_int4(c, (c + 15) / 16, (c + 63) / 64, c > 0 ? 1 : 0);
    int4 tot = make_int4(0, 0, 0, 0), ex = make_int4(0, 0, 0, 0);
    if (A <= kWave) {
        // every adapter is a lane of wave 0: one wave-level scan, no barrier
        if (w == 0) {
            const int4 incl = wave_inclusive_scan4<kWave>(v4, lane);
            ex = incl - v4;
            tot = make_int4(__shfl(incl.x, kWave - 1, kWave), __shfl(incl.y, kWave - 1, kWave),
                            __shfl(incl.z, kWave - 1, kWave), __shfl(incl.w, kWave - 1, kWave));
        }
    } else {
        ex = block_exclusive_scan4(v4, s_tot, &tot);
    }
    if (a < A) s_info[a] = make_int4(ex.x, c, ex.y, ex.z);
    lds_barrier();
    if (a < A) {
        counts[a] = c;
        offsets[a] = ex.x;
        if (c > 0) sched[active_off + ex.w] = a;
    }
    if (tid == 0) {
        offsets[A] = tot.x;
        *reinterpret_cast<int4*>(sched) = make_int4(tot.y, tot.z, tot.w, 0);
        int e = 0;
        for (int v = 0; v < kSmallWaves; ++v) e += s_err[v];
        err[0] = e;
    }

    // 3. stable scatter: s_hist[w][a] is wave w's cursor for adapter a.
    auto scatter_batch = [&](int b, const int* idv, const int* mt) {
#pragma unroll
        for (int g = 0; g < kSmallBatch; ++g) {
            if (b + g * kWave >= r1) break;  // wave-uniform
            const int t = b + g * kWave + lane;
            const int id = idv[g];
            const bool valid = mt[g] != 0;
            int cur = 0;
            if (valid) {
                cur = s_hist[w][id];
                const int4 info = s_info[id];
                const int rank = mt[g] & 0xff;
                const int local = cur + rank;  // position inside the adapter's group
                const int pos = info.x + local;
                const int cnt = info.y;
                perm[pos] = t;
                if ((local & 15) == 0) {
                    const int rows = cnt - local < 16 ? cnt - local : 16;
                    *reinterpret_cast<int4*>(sched + tiles16_off + 4 * (int64_t)(info.z + local / 16)) =
                        make_int4(id, pos, rows, 0);
                }
                if ((local & 63) == 0) {
                    const int rows = cnt - local < 64 ? cnt - local : 64;
                    *reinterpret_cast<int4*>(sched + tiles64_off + 4 * (int64_t)(info.w + local / 64)) =
                        make_int4(id, pos, rows, 0);
                }
            }
            // every lane has read its cursor: the lowest lane of each id advances it
            __builtin_amdgcn_wave_barrier();
            if (mt[g] & (1 << 16)) s_hist[w][id] = cur + (mt[g] >> 8 & 0xff);
        }
    };
    scatter_batch(r0, id0, mt0);
    for (int b = r0 + kStep; b < r1; b += kStep) {
        int idv[kSmallBatch], mt[kSmallBatch];
        load_batch(b, idv);
#pragma unroll
        for (int g = 0; g < kSmallBatch; ++g) {
            const bool valid = idv[g] >= 0 && idv[g] < A;
            mt[g] = b + g * kWave < r1 ? match(idv[g], valid) : 0;
        }
        scatter_batch(b, idv, mt);
    }
}

}  // namespace lora

using namespace lora;

extern "C" size_t lora_segments_workspace_bytes(int32_t T, int32_t num_adapters) {
    if (T < 0 || num_adapters < 1) return 0;
    return (size_t)SegWs::make(T, num_adapters).total * sizeof(int32_t);
}

namespace {
// Host-side checks of one build (nothing enqueued on failure).
int seg_check(const int32_t* adapter_ids, int32_t T, int32_t num_adapters, const lora_segments& seg, const void* ws,
              size_t ws_bytes) {
    if (T < 0 || num_adapters < 1) return LORA_ERR_INVALID_ARG;
    if (T == 0) return LORA_OK;
    if (!adapter_ids || !seg.counts || !seg.offsets || !seg.perm || !seg.err || !seg.sched) return LORA_ERR_INVALID_ARG;
    if (((uintptr_t)seg.sched & 15u) != 0) return LORA_ERR_INVALID_ARG;
    if (!ws || ws_bytes < (size_t)SegWs::make(T, num_adapters).total * sizeof(int32_t)) return LORA_ERR_WORKSPACE;
    return LORA_OK;
}
bool seg_small(int32_t T, int32_t num_adapters) { return T <= kSmallMaxT && num_adapters <= kSmallMaxA; }
SegSmallJob small_job(const int32_t* adapter_ids, int32_t T, int32_t num_adapters, const lora_segments& seg) {
    const SchedLayout sl = SchedLayout::make(T, num_adapters);
    return SegSmallJob{adapter_ids, T, seg.counts, seg.offsets, seg.perm, seg.sched, seg.err,
                       sl.active, sl.tiles16, sl.tiles64};
}
// The three-kernel path for batches beyond the one-workgroup limits.
void seg_large(const int32_t* adapter_ids, int32_t T, int32_t num_adapters, const lora_segments& seg, void* ws,
               hipStream_t st) {
    const SegWs w = SegWs::make(T, num_adapters);
    const int32_t nchunks = (int32_t)(((int64_t)T + kChunk - 1) / kChunk);
    const SchedLayout sl = SchedLayout::make(T, num_adapters);
    int32_t* wsi = static_cast<int32_t*>(ws);
    hipLaunchKernelGGL(seg_count_kernel, dim3(nchunks), dim3(kChunk), 0, st, adapter_ids, T, num_adapters, nchunks,
                       wsi + w.hist, wsi + w.rank, wsi + w.errc);
    hipLaunchKernelGGL(seg_scan_kernel, dim3(1), dim3(kScanThreads), 0, st, num_adapters, nchunks, wsi + w.hist,
                       wsi + w.errc, seg.counts, seg.offsets, seg.sched, wsi + w.pre16, wsi + w.pre64, seg.err,
                       sl.active);
    hipLaunchKernelGGL(seg_scatter_kernel, dim3(nchunks), dim3(kChunk), 0, st, adapter_ids, T, num_adapters, nchunks,
                       wsi + w.hist, wsi + w.rank, seg.counts, seg.offsets, wsi + w.pre16, wsi + w.pre64, seg.perm,
                       seg.sched, sl.tiles16, sl.tiles64);
}
}  // namespace

extern "C" int lora_segments_build(const int32_t* adapter_ids, int32_t T, int32_t num_adapters, lora_segments seg,
                                   void* ws, size_t ws_bytes, void* stream) {
    const int rc = seg_check(adapter_ids, T, num_adapters, seg, ws, ws_bytes);
    if (rc != LORA_OK || T == 0) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (seg_small(T, num_adapters)) {
        SegSmallJobs jobs{};
        jobs.job[0] = small_job(adapter_ids, T, num_adapters, seg);
        hipLaunchKernelGGL(seg_small_kernel, dim3(1), dim3(kScanThreads), 0, st, jobs, num_adapters);
    } else {
        seg_large(adapter_ids, T, num_adapters, seg, ws, st);
    }
    return hipGetLastError() == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

extern "C" int lora_segments_build_batch(const lora_segments_job* jobs, int32_t n_jobs, int32_t num_adapters,
                                         void* stream) {
    if (n_jobs < 0 || (n_jobs > 0 && !jobs)) return LORA_ERR_INVALID_ARG;
    if (n_jobs == 0) return LORA_OK;
    for (int32_t i = 0; i < n_jobs; ++i) {
        const lora_segments_job& j = jobs[i];
        const int rc = seg_check(j.adapter_ids, j.T, num_adapters, j.seg, j.ws, j.ws_bytes);
        if (rc != LORA_OK) return rc;
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    SegSmallJobs batch{};
    int nb = 0;
    auto flush = [&]() {
        if (nb > 0) hipLaunchKernelGGL(seg_small_kernel, dim3(nb), dim3(kScanThreads), 0, st, batch, num_adapters);
        nb = 0;
    };
    for (int32_t i = 0; i < n_jobs; ++i) {
        const lora_segments_job& j = jobs[i];
        if (j.T == 0) continue;
        if (seg_small(j.T, num_adapters)) {
            batch.job[nb++] = small_job(j.adapter_ids, j.T, num_adapters, j.seg);
            if (nb == kSegBatchMax) flush();
        } else {
            seg_large(j.adapter_ids, j.T, num_adapters, j.seg, j.ws, st);
        }
    }
    flush();
    return hipGetLastError() == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}
