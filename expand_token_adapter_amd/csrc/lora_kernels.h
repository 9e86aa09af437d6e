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
// One workgroup = one 16-row tile x one group of up to 64 ranks.  Its eight
// waves split K into contiguous slices; each wave runs 16x16 MFMA tiles
// (A operand = weight rows, B operand = the tile's rows), then the eight
// partial tiles are summed in wave order through LDS.

constexpr int kShrinkWaves = 8;
constexpr int kShrinkThreads = kShrinkWaves * kWave;

struct ShrinkParams {
    const void* x;   // rows gathered through perm
    int64_t ldx;
    int32_t K;       // reduction length (d_in, or d_out for g)
    const lora_adapter* adapters;
    int32_t r_max;
    const int32_t* perm;
    const int32_t* sched;
    int64_t tiles16_off;
    float* out;      // [row][ldo] or nullptr; row = original row, or sorted position if out_by_pos
    int64_t ldo;
    int32_t out_by_pos;
    float* outT;     // [k][ldT] indexed by sorted position, or nullptr
    int64_t ldT;
    int32_t* err;
    int32_t rgroups; // ceil(r_max / 64)
};

template <int DT, bool TRANS_W>
__global__ __launch_bounds__(kShrinkThreads) void shrink_kernel(ShrinkParams p) {
    using F = Frag<DT>;
    constexpr int EB = F::kBytes;
    __shared__ f32x4_t s_red[kShrinkWaves][4][kWave];

    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int lr = lane & 15;  // MFMA row / column within the 16x16 tile
    const int lg = lane >> 4;  // K group of this lane
    const int64_t n_tasks = (int64_t)p.sched[0] * p.rgroups;
    const TaskSlice ts = xcd_slice(n_tasks, 1, 0);
    const int nkc = (p.K + 63) / 64;
    const int kc0 = (int)((int64_t)wave * nkc / kShrinkWaves);
    const int kc1 = (int)((int64_t)(wave + 1) * nkc / kShrinkWaves);

    for (int64_t task = ts.begin; task < ts.end; task += ts.stride) {
        const int tile = (int)(task / p.rgroups);
        const int rg = (int)(task % p.rgroups);
        const int4 rec = *reinterpret_cast<const int4*>(p.sched + p.tiles16_off + 4 * (int64_t)tile);
        const lora_adapter ad = p.adapters[rec.x];
        if (!adapter_ok(ad, p.r_max)) {
            if (rg == 0 && threadIdx.x == 0) atomicAdd(p.err, 1);
            continue;
        }
        const int r = ad.rank;
        const int rank0 = rg * 64;
        if (rank0 >= r) continue;
        const int nmb = min(4, (r - rank0 + 15) / 16);
        const int pos0 = rec.y;
        const int nrows = rec.z;

        const bool row_ok = lr < nrows;
        const int64_t xrow = row_ok ? p.perm[pos0 + lr] : 0;
        const char* xp = static_cast<const char*>(p.x) + xrow * p.ldx * EB;
        const char* wbase = static_cast<const char*>(TRANS_W ? ad.B : ad.A);

        f32x4_t acc[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) acc[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        for (int kc = kc0; kc < kc1; ++kc) {
            F xf[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int kk = kc * 64 + 16 * lg + 8 * h;
                xf[h] = (row_ok && kk < p.K) ? F::load(xp + (int64_t)kk * EB) : F::zero();
            }
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
                if (mb < nmb) {
                    const int rk = rank0 + 16 * mb + lr;
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int kk = kc * 64 + 16 * lg + 8 * h;
                        F wf = F::zero();
                        if (rk < r && kk < p.K) {
                            if (TRANS_W)
                                wf = F::load_strided(wbase + ((int64_t)kk * r + rk) * EB, r, min(8, p.K - kk));
                            else
                                wf = F::load(wbase + ((int64_t)rk * p.K + kk) * EB);
                        }
                        acc[mb] = mma(wf, xf[h], acc[mb]);
                    }
                }
            }
        }

#pragma unroll
        for (int mb = 0; mb < 4; ++mb) s_red[wave][mb][lane] = acc[mb];
        __syncthreads();
        if (threadIdx.x < 4 * kWave) {
            const int mb = threadIdx.x / kWave;
            const int l = threadIdx.x & (kWave - 1);
            if (mb < nmb) {
                f32x4_t s = s_red[0][mb][l];
#pragma unroll
                for (int w = 1; w < kShrinkWaves; ++w) s += s_red[w][mb][l];
                const int n = l & 15;
                const int rk = rank0 + 16 * mb + 4 * (l >> 4);  // D rows 4*(l/16)+i
                if (n < nrows && rk < r) {
                    const int pos = pos0 + n;
                    if (p.out) {
                        const int64_t row = p.out_by_pos ? pos : p.perm[pos];
                        *reinterpret_cast<f32x4_t*>(p.out + row * p.ldo + rk) = s;
                    }
                    if (p.outT) {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (rk + i < r) p.outT[(int64_t)(rk + i) * p.ldT + pos] = s[i];
                    }
                }
            }
        }
        __syncthreads();
    }
}

// ============================================================== expand-add
//
// Y[row][c] += s_a * sum_k V[row][k] * W(c, k) for the rows of one adapter:
//   W(c, k) = B_a[c][k]     (B_a is [N, r]; y += s B v, forward)
//   W(c, k) = A_a[k][c]     (TRANS_W: A_a is [r, N]; dX += s A^T g, backward)
// One wave = one 64-row tile x 64 output columns.  The wave loads the
// weight block once (A operand, KS x 32 ranks) and keeps it in registers
// while it walks the tile in 16-row steps.  Output columns are assigned to
// MFMA rows so that each lane ends up owning 16 consecutive columns of one
// row: 32-byte (bf16) read-modify-write of y per lane, 128 bytes per row.

constexpr int kExpandWaves = 4;

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
    int32_t ncb;     // column blocks of 64
};

// Output column of MFMA row m in column block mb (0..3) of a 64-column block.
__device__ __forceinline__ int expand_col(int mb, int m) { return 16 * (m >> 2) + 4 * mb + (m & 3); }

template <int DT, bool TRANS_W, int KS>
__global__ __launch_bounds__(kExpandWaves * kWave) void expand_kernel(ExpandParams p) {
    using F = Frag<DT>;
    using E = Elem<DT>;
    constexpr int EB = F::kBytes;
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int lr = lane & 15;
    const int lg = lane >> 4;
    const int64_t n_tasks = (int64_t)p.sched[1] * p.ncb;
    const TaskSlice ts = xcd_slice(n_tasks, kExpandWaves, wave);

    for (int64_t task = ts.begin; task < ts.end; task += ts.stride) {
        const int tile = (int)(task / p.ncb);
        const int cb = (int)(task % p.ncb);
        const int4 rec = *reinterpret_cast<const int4*>(p.sched + p.tiles64_off + 4 * (int64_t)tile);
        const lora_adapter ad = p.adapters[rec.x];
        if (!adapter_ok(ad, p.r_max)) {
            if (cb == 0 && lane == 0) atomicAdd(p.err, 1);
            continue;
        }
        const int r = ad.rank;
        const float s = ad.scale;
        const int c0 = cb * 64;
        const int pos0 = rec.y;
        const int nrows = rec.z;

        // Weight block: wf[mb][ks] holds W(col(mb, lr), 32 ks + 8 lg + 0..7).
        F wf[4][KS];
        const char* wbase = static_cast<const char*>(TRANS_W ? ad.A : ad.B);
        const bool vec_w = !TRANS_W && (r & 7) == 0;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const int col = c0 + expand_col(mb, lr);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int kk = 32 * ks + 8 * lg;
                const int nval = min(8, r - kk);
                F w = F::zero();
                if (col < p.N && nval > 0) {
                    if (TRANS_W)
                        w = F::load_strided(wbase + ((int64_t)kk * p.N + col) * EB, p.N, nval);
                    else if (vec_w && nval == 8)
                        w = F::load(wbase + ((int64_t)col * r + kk) * EB);
                    else
                        w = F::load_strided(wbase + ((int64_t)col * r + kk) * EB, 1, nval);
                }
                wf[mb][ks] = w;
            }
        }

        for (int st = 0; st * 16 < nrows; ++st) {
            const bool row_ok = st * 16 + lr < nrows;
            const int pos = pos0 + st * 16 + lr;
            const int64_t t = row_ok ? p.perm[pos] : 0;
            const int64_t vrow = p.v_by_pos ? pos : t;
            const float* vp = p.v + vrow * p.ldv;

            f32x4_t acc[4];
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) acc[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int kk = 32 * ks + 8 * lg;
                float f[8];
                if (row_ok && kk + 8 <= r) {
                    const f32x4_t a = *reinterpret_cast<const f32x4_t*>(vp + kk);
                    const f32x4_t b = *reinterpret_cast<const f32x4_t*>(vp + kk + 4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        f[e] = a[e];
                        f[4 + e] = b[e];
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) f[e] = (row_ok && kk + e < r) ? vp[kk + e] : 0.f;
                }
                const F32Operand<DT> vo = F32Operand<DT>::make(f);
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) acc[mb] = vo.mma_right(wf[mb][ks], acc[mb]);
            }

            if (row_ok) {
                char* yp = static_cast<char*>(p.y) + (t * p.ldy + c0 + 16 * lg) * EB;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    if (c0 + 16 * lg + 8 * h < p.N) {
                        float yv[8];
                        E::load8(yp + 8 * h * EB, yv);
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const int j = 8 * h + e;  // column offset 4 mb + i
                            yv[e] = yv[e] + s * acc[j >> 2][j & 3];
                        }
                        E::store8(yp + 8 * h * EB, yv);
                    }
                }
            }
        }
    }
}

// ============================================================== token contraction
//
// For each adapter a with fine-tuning rows and each block of 64 columns:
//   dA_a[k][c] += s_a * sum_rows g[row][k] * x[row][c]      (c < d_in)
//   dB_a[c][k] += s_a * sum_rows dy[row][c] * v[row][k]     (c < d_out)
// The contraction runs over rows, so the row-major x / dy tiles are
// transposed through LDS (per wave, 32 rows x 64 columns) into MFMA B
// operands; g and v come pre-transposed ([k][sorted position]) from the
// shrink kernel.  Four waves split the adapter's rows into contiguous
// ranges; their partial tiles are summed in wave order through LDS and
// added to dA / dB, which no other workgroup touches.

constexpr int kContractWaves = 4;
constexpr int kCtPitch = 32 + 8;  // LDS row pitch (elements) of a transposed column

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
    int32_t rgroups;
    int32_t* err;
};

template <int DT>
struct ContractLds {
    static constexpr int EB = Frag<DT>::kBytes;
    static constexpr int kTransBytes = kContractWaves * 64 * kCtPitch * EB;
    static constexpr int kRedBytes = kContractWaves * 16 * kWave * 16;
    static constexpr int kBytes = kTransBytes > kRedBytes ? kTransBytes : kRedBytes;
};

template <int DT>
__global__ __launch_bounds__(kContractWaves * kWave) void contract_kernel(ContractParams p) {
    using F = Frag<DT>;
    constexpr int EB = F::kBytes;
    __shared__ __attribute__((aligned(16))) char s_mem[ContractLds<DT>::kBytes];

    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int lr = lane & 15;
    const int lg = lane >> 4;
    const int ncb = p.ncb_in + p.ncb_out;
    const int64_t n_tasks = (int64_t)p.sched[2] * p.rgroups * ncb;
    const TaskSlice ts = xcd_slice(n_tasks, 1, 0);
    char* trans = s_mem + wave * (64 * kCtPitch * EB);  // this wave's [64 columns][kCtPitch] tile

    for (int64_t task = ts.begin; task < ts.end; task += ts.stride) {
        const int cb_all = (int)(task % ncb);
        const int rg = (int)((task / ncb) % p.rgroups);
        const int act = (int)(task / ((int64_t)ncb * p.rgroups));
        const int a = p.sched[p.active_off + act];
        const lora_adapter ad = p.adapters[a];
        const lora_adapter_grad gr = p.grads[a];
        const bool is_dA = cb_all < p.ncb_in;
        if (!adapter_ok(ad, p.r_max) || gr.dA == nullptr || gr.dB == nullptr) {
            if (cb_all == 0 && rg == 0 && threadIdx.x == 0) atomicAdd(p.err, 1);
            continue;
        }
        const int r = ad.rank;
        const int rank0 = rg * 64;
        if (rank0 >= r) continue;
        const int nmb = min(4, (r - rank0 + 15) / 16);
        const int cb = is_dA ? cb_all : cb_all - p.ncb_in;
        const int c0 = cb * 64;
        const int N = is_dA ? p.d_in : p.d_out;
        const char* q = static_cast<const char*>(is_dA ? p.x : p.dy);
        const int64_t ldq = is_dA ? p.ldx : p.lddy;
        const float* PT = is_dA ? p.gT : p.vT;

        const int lo = p.offsets[a];
        const int hi = p.offsets[a + 1];
        // 32-aligned windows of sorted positions covering [lo, hi), split over the waves.
        const int w0 = lo & ~31;
        const int nwin = (hi - w0 + 31) / 32;
        const int wa = w0 + 32 * (int)((int64_t)wave * nwin / kContractWaves);
        const int wb = w0 + 32 * (int)((int64_t)(wave + 1) * nwin / kContractWaves);

        f32x4_t acc[4][4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        // Loader role: lane covers positions 4*(lane/8)+j (j < 4), columns 8*(lane%8)+e (e < 8).
        const int lrow = 4 * (lane >> 3);
        const int lcol = 8 * (lane & 7);
        for (int win = wa; win < wb; win += 32) {
            // 1. Q tile -> LDS, transposed to [column][position].
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int pos = win + lrow + j;
                const bool ok = pos >= lo && pos < hi && c0 + lcol < N;
                F f = F::zero();
                if (ok) {
                    const int64_t row = p.perm[pos];
                    f = F::load(q + (row * ldq + c0 + lcol) * EB);
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    char* dst = trans + ((lcol + e) * kCtPitch + lrow + j) * EB;
                    if constexpr (EB == 2)
                        *reinterpret_cast<uint16_t*>(dst) = (uint16_t)f.raw(e);
                    else
                        *reinterpret_cast<uint32_t*>(dst) = f.raw(e);
                }
            }
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // 2. B operands: column 16 nb + lr, positions 8 lg .. 8 lg + 7.
            F qf[4];
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) qf[nb] = F::load(trans + ((16 * nb + lr) * kCtPitch + 8 * lg) * EB);
            // 3. A operands from P^T: rank rank0 + 16 mb + lr, same positions.
            const int pp = win + 8 * lg;
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
                if (mb < nmb) {
                    const int rk = rank0 + 16 * mb + lr;
                    float f[8];
                    if (rk < r) {
                        const float* src = PT + (int64_t)rk * p.ldT + pp;
                        const f32x4_t a0 = *reinterpret_cast<const f32x4_t*>(src);
                        const f32x4_t a1 = *reinterpret_cast<const f32x4_t*>(src + 4);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            f[e] = (pp + e >= lo && pp + e < hi) ? a0[e] : 0.f;
                            f[4 + e] = (pp + 4 + e >= lo && pp + 4 + e < hi) ? a1[e] : 0.f;
                        }
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e) f[e] = 0.f;
                    }
                    const F32Operand<DT> po = F32Operand<DT>::make(f);
#pragma unroll
                    for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = po.mma_left(qf[nb], acc[mb][nb]);
                }
            }
            __builtin_amdgcn_wave_barrier();
        }

        // Fixed-order sum of the four waves' tiles.
        __syncthreads();
        f32x4_t* red = reinterpret_cast<f32x4_t*>(s_mem);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) red[((wave * 4 + mb) * 4 + nb) * kWave + lane] = acc[mb][nb];
        __syncthreads();
        {
            const int nb = wave;  // this wave finishes column block nb
            const float s = ad.scale;
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
                if (mb < nmb) {
                    f32x4_t sum = red[((0 * 4 + mb) * 4 + nb) * kWave + lane];
#pragma unroll
                    for (int w = 1; w < kContractWaves; ++w) sum += red[((w * 4 + mb) * 4 + nb) * kWave + lane];
                    const int col = c0 + 16 * nb + lr;
                    if (col < N) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int rk = rank0 + 16 * mb + 4 * lg + i;
                            if (rk < r) {
                                float* dst = is_dA ? gr.dA + (int64_t)rk * p.d_in + col : gr.dB + (int64_t)col * r + rk;
                                *dst += s * sum[i];
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
