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
