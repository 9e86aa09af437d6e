// device_common.h -- gfx950 building blocks shared by the LoRA kernels:
// bf16 conversion, MFMA wrappers, per-lane operand fragments and the
// XCD-aware task walk.
//
// MFMA lane layout used throughout (16x16 output tiles, wave64):
//   A operand (16 x K):  lane l supplies row  m = l % 16, a group of K values
//   B operand (K x 16):  lane l supplies column n = l % 16, the same K group
//   C/D (16 x 16 fp32):  lane l holds D[4 * (l / 16) + i][l % 16], i = 0..3
// The K values a lane supplies for A and for B are taken from the same K
// positions, so the product is the full sum over K whatever order the
// hardware walks them in.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lora_batch.h"

namespace lora {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Pointers into device memory that the compiler cannot prove global (e.g.
// the adapter weights, read from the device-resident table) would otherwise
// be accessed with FLAT instructions; gptr() casts them to the global
// address space so loads and stores are global_* instructions.
#define LORA_GLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ const LORA_GLOBAL T* gptr(const T* p) {
    return (const LORA_GLOBAL T*)(p);
}
template <typename T>
__device__ __forceinline__ LORA_GLOBAL T* gptr(T* p) {
    return (LORA_GLOBAL T*)(p);
}

constexpr int kWave = 64;
constexpr int kNumXcd = 8;  // MI355X: 8 accelerator dies, one L2 each

// ---------------------------------------------------------------- scalars

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Two fp32 values -> packed bf16 pair (first value in the low half), round to
// nearest even by the hardware conversion (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// Wait for this wave's LDS operations, then barrier the workgroup.  Global
// loads still in flight stay in flight (unlike __syncthreads, which also
// drains them).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Index of the calling wave in its workgroup, as a wave-uniform (scalar)
// value: branches on it stay scalar branches instead of exec-masked ones.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave)); }
// Lane 0's value, as a wave-uniform (scalar) value.
__device__ __forceinline__ int64_t uniform64(int64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Sum over the wave's lanes (every lane gets it).
__device__ __forceinline__ int64_t wave_sum64(int64_t v) {
#pragma unroll
    for (int d = kWave / 2; d >= 1; d >>= 1) v += __shfl_xor(v, d, kWave);
    return v;
}

// ---------------------------------------------------------------- MFMA

__device__ __forceinline__ f32x4_t mfma_bf16(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t mfma_f32(float a, float b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- fragments
// A fragment is the 8 K-consecutive elements one lane feeds to one 16x16
// tile step.  bf16: one 16-byte register quad, consumed by one
// 16x16x32 MFMA.  fp32: two quads, consumed by eight 16x16x4 MFMAs.

template <int DT>
struct Frag;

template <>
struct Frag<LORA_BF16> {
    u32x4_t q;
    static constexpr int kBytes = 2;
    __device__ __forceinline__ static Frag zero() { return Frag{u32x4_t{0, 0, 0, 0}}; }
    // 8 elements at p in device memory (16-byte aligned).
    __device__ __forceinline__ static Frag load(const void* p) {
        return Frag{*gptr(reinterpret_cast<const u32x4_t*>(p))};
    }
    // 8 elements at p in LDS.
    __device__ __forceinline__ static Frag load_lds(const void* p) {
        return Frag{*reinterpret_cast<const u32x4_t*>(p)};
    }
    // Elements p[i * stride] (device memory) for i < n (n <= 8), zeros after.
    __device__ __forceinline__ static Frag load_strided(const void* p, int64_t stride, int n) {
        const LORA_GLOBAL uint16_t* s = gptr(reinterpret_cast<const uint16_t*>(p));
        uint32_t h[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) h[i] = (i < n) ? (uint32_t)s[i * stride] : 0u;
        return Frag{u32x4_t{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                            h[6] | (h[7] << 16)}};
    }
    // From 8 fp32 values, rounded to bf16 (nearest even).
    __device__ __forceinline__ static Frag from_f32(const float* f) {
        return Frag{u32x4_t{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                            pack_bf16x2(f[6], f[7])}};
    }
    __device__ __forceinline__ float get(int i) const {
        uint32_t w = q[i >> 1];
        return bf16_bits_to_f32((i & 1) ? (w >> 16) : (w & 0xffffu));
    }
    // Raw 16-bit pattern of element i.
    __device__ __forceinline__ uint32_t raw(int i) const { return (q[i >> 1] >> (16 * (i & 1))) & 0xffffu; }
    // The fragment where ok holds, else zeros (a mask, not a branch).
    __device__ __forceinline__ Frag masked(bool ok) const {
        const uint32_t m = 0u - (uint32_t)ok;
        return Frag{u32x4_t{q[0] & m, q[1] & m, q[2] & m, q[3] & m}};
    }
};

template <>
struct Frag<LORA_F32> {
    u32x4_t q0, q1;
    static constexpr int kBytes = 4;
    __device__ __forceinline__ static Frag zero() {
        return Frag{u32x4_t{0, 0, 0, 0}, u32x4_t{0, 0, 0, 0}};
    }
    __device__ __forceinline__ static Frag load(const void* p) {
        const LORA_GLOBAL u32x4_t* v = gptr(reinterpret_cast<const u32x4_t*>(p));
        return Frag{v[0], v[1]};
    }
    __device__ __forceinline__ static Frag load_lds(const void* p) {
        const u32x4_t* v = reinterpret_cast<const u32x4_t*>(p);
        return Frag{v[0], v[1]};
    }
    __device__ __forceinline__ static Frag load_strided(const void* p, int64_t stride, int n) {
        const LORA_GLOBAL uint32_t* s = gptr(reinterpret_cast<const uint32_t*>(p));
        uint32_t h[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) h[i] = (i < n) ? s[i * stride] : 0u;
        return Frag{u32x4_t{h[0], h[1], h[2], h[3]}, u32x4_t{h[4], h[5], h[6], h[7]}};
    }
    __device__ __forceinline__ static Frag from_f32(const float* f) {
        return Frag{u32x4_t{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                            __float_as_uint(f[3])},
                    u32x4_t{__float_as_uint(f[4]), __float_as_uint(f[5]), __float_as_uint(f[6]),
                            __float_as_uint(f[7])}};
    }
    __device__ __forceinline__ float get(int i) const {
        return __uint_as_float(i < 4 ? q0[i & 3] : q1[i & 3]);
    }
    __device__ __forceinline__ uint32_t raw(int i) const { return i < 4 ? q0[i & 3] : q1[i & 3]; }
    __device__ __forceinline__ Frag masked(bool ok) const {
        const uint32_t m = 0u - (uint32_t)ok;
        return Frag{u32x4_t{q0[0] & m, q0[1] & m, q0[2] & m, q0[3] & m},
                    u32x4_t{q1[0] & m, q1[1] & m, q1[2] & m, q1[3] & m}};
    }
};

// Elements of an 8-element rank group starting at kk that lie below rank r.
__device__ __forceinline__ int wkeep(int r, int kk) { return max(0, min(8, r - kk)); }

// acc += A_frag (rows) x B_frag (columns) over the 8-element K group of each lane.
__device__ __forceinline__ f32x4_t mma(const Frag<LORA_BF16>& a, const Frag<LORA_BF16>& b, f32x4_t c) {
    return mfma_bf16(a.q, b.q, c);
}
__device__ __forceinline__ f32x4_t mma(const Frag<LORA_F32>& a, const Frag<LORA_F32>& b, f32x4_t c) {
#pragma unroll
    for (int e = 0; e < 4; ++e) c = mfma_f32(__uint_as_float(a.q0[e]), __uint_as_float(b.q0[e]), c);
#pragma unroll
    for (int e = 0; e < 4; ++e) c = mfma_f32(__uint_as_float(a.q1[e]), __uint_as_float(b.q1[e]), c);
    return c;
}

// An fp32 operand (v, g) fed against element-typed weights.  For bf16 the
// value is split into hi = bf16(v) and lo = bf16(v - hi), two exact-product
// MFMAs whose sum carries about 16 significant bits of v; for fp32 the value
// is used as is.
template <int DT>
struct F32Operand;

template <>
struct F32Operand<LORA_BF16> {
    Frag<LORA_BF16> hi, lo;
    __device__ __forceinline__ static F32Operand make(const float* f) {
        F32Operand o;
        float r[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t h = pack_bf16x2(f[2 * i], f[2 * i + 1]);
            o.hi.q[i] = h;
            r[2 * i] = f[2 * i] - __uint_as_float(h << 16);
            r[2 * i + 1] = f[2 * i + 1] - __uint_as_float(h & 0xffff0000u);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) o.lo.q[i] = pack_bf16x2(r[2 * i], r[2 * i + 1]);
        return o;
    }
    // acc += W x operand   (W as the A operand, this as the B operand)
    __device__ __forceinline__ f32x4_t mma_right(const Frag<LORA_BF16>& w, f32x4_t c) const {
        c = mma(w, hi, c);
        return mma(w, lo, c);
    }
    // acc += operand x Q   (this as the A operand, Q as the B operand)
    __device__ __forceinline__ f32x4_t mma_left(const Frag<LORA_BF16>& q, f32x4_t c) const {
        c = mma(hi, q, c);
        return mma(lo, q, c);
    }
};

template <>
struct F32Operand<LORA_F32> {
    Frag<LORA_F32> f;
    __device__ __forceinline__ static F32Operand make(const float* v) {
        F32Operand o;
        o.f = Frag<LORA_F32>::from_f32(v);
        return o;
    }
    __device__ __forceinline__ f32x4_t mma_right(const Frag<LORA_F32>& w, f32x4_t c) const { return mma(w, f, c); }
    __device__ __forceinline__ f32x4_t mma_left(const Frag<LORA_F32>& q, f32x4_t c) const { return mma(f, q, c); }
};

// ---------------------------------------------------------------- element IO

template <int DT>
struct Elem;

template <>
struct Elem<LORA_BF16> {
    __device__ __forceinline__ static float get(const void* p, int64_t i) {
        return bf16_bits_to_f32(gptr(reinterpret_cast<const uint16_t*>(p))[i]);
    }
    // Read 8 consecutive elements (16-byte aligned) as fp32.
    __device__ __forceinline__ static void load8(const void* p, float* f) {
        u32x4_t q = *gptr(reinterpret_cast<const u32x4_t*>(p));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = bf16_bits_to_f32(q[i] & 0xffffu);
            f[2 * i + 1] = bf16_bits_to_f32(q[i] >> 16);
        }
    }
    // 8 elements held in one 16-byte quad, as fp32.
    __device__ __forceinline__ static void unpack8(const u32x4_t* q, float* f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(q[0][i] << 16);
            f[2 * i + 1] = __uint_as_float(q[0][i] & 0xffff0000u);
        }
    }
    // Write 8 fp32 values, each rounded once to bf16.
    __device__ __forceinline__ static void store8(void* p, const float* f) {
        u32x4_t q;
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
        *gptr(reinterpret_cast<u32x4_t*>(p)) = q;
    }
    // The same as a nontemporal (streaming) store.
    __device__ __forceinline__ static void store8_nt(void* p, const float* f) {
        u32x4_t q;
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
        __builtin_nontemporal_store(q, gptr(reinterpret_cast<u32x4_t*>(p)));
    }
};

template <>
struct Elem<LORA_F32> {
    __device__ __forceinline__ static float get(const void* p, int64_t i) {
        return gptr(reinterpret_cast<const float*>(p))[i];
    }
    __device__ __forceinline__ static void load8(const void* p, float* f) {
        const LORA_GLOBAL f32x4_t* v = gptr(reinterpret_cast<const f32x4_t*>(p));
        f32x4_t a = v[0], b = v[1];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[i] = a[i];
            f[4 + i] = b[i];
        }
    }
    // 8 elements held in two 16-byte quads.
    __device__ __forceinline__ static void unpack8(const u32x4_t* q, float* f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[i] = __uint_as_float(q[0][i]);
            f[4 + i] = __uint_as_float(q[1][i]);
        }
    }
    __device__ __forceinline__ static void store8(void* p, const float* f) {
        LORA_GLOBAL f32x4_t* v = gptr(reinterpret_cast<f32x4_t*>(p));
        v[0] = f32x4_t{f[0], f[1], f[2], f[3]};
        v[1] = f32x4_t{f[4], f[5], f[6], f[7]};
    }
    __device__ __forceinline__ static void store8_nt(void* p, const float* f) {
        LORA_GLOBAL f32x4_t* v = gptr(reinterpret_cast<f32x4_t*>(p));
        __builtin_nontemporal_store(f32x4_t{f[0], f[1], f[2], f[3]}, v);
        __builtin_nontemporal_store(f32x4_t{f[4], f[5], f[6], f[7]}, v + 1);
    }
};

// ---------------------------------------------------------------- tasks

// Scheduling metadata written by the segment builder (int32 offsets into
// lora_segments.sched).  Tile records are {adapter, first sorted position,
// rows, 0}.
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

// 16 bytes per lane from global memory straight into LDS: lane L's bytes
// land at lds_row + 16 L (gfx950 global_load_lds_dwordx4; counted in vmcnt).
__device__ __forceinline__ void lds_dma16(const void* src, void* lds_row) {
    __builtin_amdgcn_global_load_lds((const LORA_GLOBAL void*)src,
                                     (__attribute__((address_space(3))) void*)lds_row, 16, 0, 0);
}

// The same load issued from inline assembly: the compiler does not track it,
// so it does not order consecutive such loads behind one another (its waits
// for LDS writes it cannot tell apart).  The caller waits (vmcnt) before any
// wave reads the bytes; lds_row must be wave-uniform.
__device__ __forceinline__ void lds_dma16_async(const void* src, void* lds_row) {
    const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds_row;
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "global_load_lds_dwordx4 %1, off"
        :
        : "s"(m0), "v"(src)
        : "memory", "m0");
}

// Buffer resources (raw, untyped): loads through them take a 32-bit byte
// offset from a wave-uniform base, and the hardware returns zeros for bytes at
// or past num_records instead of touching memory there.
typedef __amdgpu_buffer_rsrc_t buf_rsrc_t;
constexpr int kBufDword3 = 0x00020000;  // gfx9 family: raw buffer, no format conversion
__device__ __forceinline__ buf_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufDword3);
}
// A byte offset past every buffer the kernels build (they all hold fewer than
// 2^31 bytes): a load at it returns zeros and touches no memory.
constexpr uint32_t kBufOff = 0x80000000u;
// 16 bytes at base + soff + voff (soff wave-uniform).  The range check
// covers voff and the instruction's immediate offset, not soff: offsets that
// may fall past the buffer go in voff.
__device__ __forceinline__ u32x4_t buf_load16(buf_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
}
// The same with the nontemporal hint, for data read once (a stream that
// should not push out of L2 the lines other workgroups still re-read).
__device__ __forceinline__ u32x4_t buf_load16_nt(buf_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 2);
}

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding:
// vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt_le() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

struct SchedLayout {
    int64_t active;    // [A] adapters with at least one row, ascending
    int64_t tiles16;   // [n16_max] records of up to 16 rows
    int64_t tiles64;   // [n64_max] records of up to 64 rows
    int64_t total;     // int32 elements
    __host__ __device__ static SchedLayout make(int64_t T, int64_t A) {
        SchedLayout s;
        s.active = 4;
        s.tiles16 = s.active + ((A + 3) / 4) * 4;
        s.tiles64 = s.tiles16 + 4 * max_tiles16(T, A);
        s.total = s.tiles64 + 4 * max_tiles64(T, A);
        return s;
    }
    __host__ __device__ static int64_t max_tiles16(int64_t T, int64_t A) { return (T + 15) / 16 + A; }
    __host__ __device__ static int64_t max_tiles64(int64_t T, int64_t A) { return (T + 63) / 64 + A; }
};
// sched[0] = number of 16-row tiles, sched[1] = number of 64-row tiles,
// sched[2] = number of active adapters.

// Contiguous slice of a task range for the calling wave group.  Workgroups
// are handed to the 8 XCDs round-robin by index, so workgroups b with the
// same b % 8 share an L2; giving each such set one contiguous slice keeps
// neighbouring tasks (same adapter, same weights) in one L2.
struct TaskSlice {
    int64_t begin, end, stride;
};
// (for workgroup b of G, G a multiple of 8, placed at launch index b)
__device__ __forceinline__ TaskSlice xcd_slice_of(int b, int G, int64_t n, int units_per_wg, int unit) {
    const int x = b % kNumXcd;
    const int64_t per = (n + kNumXcd - 1) / kNumXcd;
    TaskSlice s;
    s.begin = (int64_t)x * per;
    s.end = s.begin + per < n ? s.begin + per : n;
    s.begin += (int64_t)(b / kNumXcd) * units_per_wg + unit;
    s.stride = (int64_t)(G / kNumXcd) * units_per_wg;
    return s;
}
__device__ __forceinline__ TaskSlice xcd_slice(int64_t n, int units_per_wg, int unit) {
    return xcd_slice_of(blockIdx.x, gridDim.x, n, units_per_wg, unit);
}

// Table entries and tile records, read with global loads.
// Tables and tile records are read-only while a kernel runs and are indexed
// with wave-uniform values: read through the constant address space, so
// they become scalar loads whose waits (lgkmcnt) do not hold up the vector
// memory pipeline.
#define LORA_CONST __attribute__((address_space(4)))
template <class T>
__device__ __forceinline__ const LORA_CONST T* cptr(const T* p) {
    return (const LORA_CONST T*)(p);
}

__device__ __forceinline__ lora_adapter load_adapter(const lora_adapter* table, int a) {
    // One 16-byte and one 8-byte load, issued together.
    const LORA_CONST u32x4_t* q4 = cptr(reinterpret_cast<const u32x4_t*>(table + a));
    const LORA_CONST uint64_t* q = cptr(reinterpret_cast<const uint64_t*>(table + a));
    const u32x4_t ab = q4[0];
    const uint64_t w2 = q[2];
    const uint64_t w0 = (uint64_t)ab[0] | ((uint64_t)ab[1] << 32);
    const uint64_t w1 = (uint64_t)ab[2] | ((uint64_t)ab[3] << 32);
    lora_adapter ad;
    ad.A = reinterpret_cast<const void*>(w0);
    ad.B = reinterpret_cast<const void*>(w1);
    ad.rank = (int32_t)(uint32_t)w2;
    ad.scale = __uint_as_float((uint32_t)(w2 >> 32));
    return ad;
}
__device__ __forceinline__ lora_adapter_grad load_grad(const lora_adapter_grad* table, int a) {
    const LORA_CONST uint64_t* q = cptr(reinterpret_cast<const uint64_t*>(table + a));
    lora_adapter_grad g;
    g.dA = reinterpret_cast<float*>(q[0]);
    g.dB = reinterpret_cast<float*>(q[1]);
    return g;
}
struct TileRec {
    int adapter, pos0, rows;
};
__device__ __forceinline__ TileRec load_tile(const int32_t* sched, int64_t off, int64_t tile) {
    const u32x4_t v = *cptr(reinterpret_cast<const u32x4_t*>(sched + off + 4 * tile));
    return TileRec{(int)v[0], (int)v[1], (int)v[2]};
}

__device__ __forceinline__ bool adapter_ok(const lora_adapter& ad, int r_max) {
    return ad.rank >= 1 && ad.rank <= r_max && ad.A != nullptr && ad.B != nullptr &&
           (((uintptr_t)ad.A | (uintptr_t)ad.B) & 15u) == 0;
}

}  // namespace lora
