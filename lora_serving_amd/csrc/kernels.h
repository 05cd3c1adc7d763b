// Host-side launchers of the gfx950 kernels (one .hip file each), called by api.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mlora {

constexpr int SORT_UNIT = 1024;   // entries per wave in the counting sort

// ---- plan.hip ----------------------------------------------------------------------------
size_t sort_workspace_bytes(int64_t n, int32_t nkeys);
hipError_t launch_stable_sort(const int32_t *keys, int64_t n, int32_t nkeys, int32_t *perm,
                              int32_t *seg_key, int32_t *seg_start, int32_t *seg_len,
                              int32_t *counts, int32_t *cnt_ws, hipStream_t stream);

// ---- slot geometry passed to kernels by value ----------------------------------------------
struct SlotGeom {
    const uint16_t *A;      // [S][n_slices][R][n_in]
    const uint16_t *B;      // [S][n_out][R]
    const float *factor;    // [S]
    int32_t S, R, n_slices;
    int32_t slice_start[5];
};

// ---- bgmv.hip: per-pair shrink and per-token expand (decode / any T) -----------------------
// v[j][t][:] = scale*factor * A[a] x[t]  (zeros for -1 pairs)
hipError_t launch_shrink_pairs(const uint16_t *x, int64_t T, int64_t n_in, const SlotGeom &g,
                               const int32_t *idx, int32_t K, const float *scale, float *v,
                               hipStream_t stream);
// y[t][n] = bf16(base + delta): base = y (accumulate) or the sum of n_part fp32 partials
// part[n_part][T][n_out]; rows whose slots are all -1 get exactly base.
hipError_t launch_expand_tokens(const float *v, int64_t T, int64_t n_out, const SlotGeom &g,
                                const int32_t *idx, int32_t K, const float *part, int32_t n_part,
                                uint16_t *y, hipStream_t stream);

// ---- gemm_decode.hip: skinny base GEMM for T <= 128 -------------------------------------------
struct DecodeCfg {
    int tt;        // token tiles of 16
    int sk;        // split of n_in across workgroups
    int kr;        // n_in per workgroup (multiple of 128)
    int n_tiles;   // row tiles of 64
};
DecodeCfg decode_config(int64_t T, int64_t n_in, int64_t n_out);
size_t decode_partial_bytes(int64_t T, int64_t n_in, int64_t n_out);
// part[sk][T][n_out] = x[:, krange] W[:, krange]^T ; if v != nullptr the same launch also runs
// the per-pair shrink (horizontal fusion: no dependency between the two halves).
hipError_t launch_decode_gemm(const uint16_t *x, const uint16_t *W, int64_t T, int64_t n_in,
                              int64_t n_out, float *part, const DecodeCfg &cfg,
                              const SlotGeom *g, const int32_t *idx, int32_t K,
                              const float *scale, float *v, hipStream_t stream);

}  // namespace mlora
