// host_checks.h -- argument checks run on the host before anything is
// enqueued, plus launch-size helpers.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "lora_batch.h"

namespace lora {

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline bool valid_dtype(int dt) { return dt == LORA_BF16 || dt == LORA_F32; }
inline int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

// Check one element matrix argument: pointer, row length, pitch.
// Returns LORA_OK, LORA_ERR_INVALID_ARG or LORA_ERR_UNSUPPORTED.
inline int check_matrix(const void* p, int64_t cols, int64_t ld) {
    if (!p || cols < 1 || ld < cols) return LORA_ERR_INVALID_ARG;
    if (!aligned16(p)) return LORA_ERR_INVALID_ARG;
    if (cols % 8 != 0 || ld % 8 != 0) return LORA_ERR_UNSUPPORTED;
    return LORA_OK;
}

inline int check_common(int dtype, int32_t T, int32_t num_adapters, int32_t r_max, const lora_adapter* adapters,
                        const lora_segments& seg) {
    if (!valid_dtype(dtype) || T < 0 || num_adapters < 1) return LORA_ERR_INVALID_ARG;
    if (r_max < 1 || r_max > LORA_MAX_RANK) return LORA_ERR_INVALID_ARG;
    if (!adapters || ((uintptr_t)adapters & 7u)) return LORA_ERR_INVALID_ARG;
    if (!seg.offsets || !seg.perm || !seg.err || !seg.sched || !aligned16(seg.sched)) return LORA_ERR_INVALID_ARG;
    return LORA_OK;
}

inline int check_f32_rows(const float* p, int64_t ld, int32_t r_max) {
    if (!p || !aligned16(p) || ld < r_max || ld % 8 != 0) return LORA_ERR_INVALID_ARG;
    return LORA_OK;
}

// Grid size (multiple of the XCD count) for `units` independent work units
// handled `per_wg` at a time, capped at `cap` workgroups.
inline unsigned grid_for(int64_t units, int per_wg, int64_t cap) {
    int64_t g = (units + per_wg - 1) / per_wg;
    if (g > cap) g = cap;
    if (g < 1) g = 1;
    return (unsigned)round_up(g, 8);
}

inline int rank_groups(int32_t r_max) { return (r_max + 63) / 64; }

// Batches with at most this many rows per adapter (T <= this * num_adapters)
// take the 16-row-tile kernels (decode.h, fused_decode.h); others the
// 64-row-tile kernels.
#ifndef LORA_DECODE_ROWS_PER_ADAPTER
#define LORA_DECODE_ROWS_PER_ADAPTER 32
#endif

inline bool use_decode_path(int dtype, int32_t T, int32_t num_adapters) {
    return dtype == LORA_BF16 && (int64_t)T <= (int64_t)LORA_DECODE_ROWS_PER_ADAPTER * num_adapters;
}

// The 16-row-tile kernels address x, A_a and B_a (or y and B_a) through
// buffer resources with 32-bit byte offsets, and use offsets from 2^31 up as
// "past the buffer": every buffer they address must hold fewer than 2^31
// bytes.
inline bool dec_offsets_fit(int64_t rows_bytes, int64_t d, int32_t r_max) {
    const int64_t lim = ((int64_t)1 << 31) - 65536;
    return rows_bytes < lim && d * r_max * 2 < lim;
}

}  // namespace lora
