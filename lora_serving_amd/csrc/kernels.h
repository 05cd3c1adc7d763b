// Host-side launchers of the gfx950 kernels (one .hip file each), called by api.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mlora {

constexpr int SORT_UNIT = 1024;   // entries per wave in the counting sort
constexpr int MI355X_CUS = 256;   // CUs assumed when no device can be asked (host-only callers)
constexpr size_t LDS_BYTES = 160 * 1024;   // LDS per CU on gfx950

// ---- device_props.hip: per-device facts, cached under a lock ------------------------------
// CUs of the current device (MI355X_CUS when there is no device to ask).
int device_cu_count();
// Static (__shared__) LDS of a kernel.
size_t kernel_static_lds(const void *fn);
// Workgroups of a kernel (threads each, dyn_lds bytes of dynamic LDS) that one CU holds at once
// (its register and LDS use; looked up on the first call per device and kernel, at least 1).
int kernel_resident_blocks(const void *fn, int threads, size_t dyn_lds);
// Raises the kernel's dynamic-LDS limit on the current device to at least `bytes` (once).
hipError_t ensure_dynamic_lds(const void *fn, size_t bytes);
constexpr int MLORA_MAX_SLICES_DEV = 4;
constexpr int MLORA_MAX_RANK_DEV = 512;
constexpr int MLORA_MAX_K_DEV = 8;

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
    const int32_t *rank;    // [S] true ranks (device), or nullptr: every slot R wide
    int32_t S, R, n_slices;
    int32_t slice_start[5];
};

// ---- bgmv.hip: per-pair shrink and per-token expand (decode / any T) -----------------------
// v[j][t][:] = scale*factor * A[a] x[t]  (zeros for -1 pairs); pieces: A[a] x[t] unscaled, in
// the decode finish's layout of shrink pieces with one split (per 64-token chunk c a block
// [K][Tc][wd], Tc = the chunk's tokens, the blocks K 64 wd floats apart)
hipError_t launch_shrink_pairs(const uint16_t *x, int64_t T, int64_t n_in, const SlotGeom &g,
                               const int32_t *idx, int32_t K, const float *scale, float *v,
                               hipStream_t stream, bool pieces = false);
// One workgroup per (token, block of output rows):
//   y[t][n] = bf16(y[t][n] + sum_j B[a_j][n][:] . v[j][t][slice(n)*R ..]); rows of a token whose
//   slots are all -1 are left untouched.  hipErrorInvalidValue past the grid's limits
//   (T >= 2^31, more than 65535 blocks of 256 rows).
hipError_t launch_expand_tokens(const float *v, int64_t T, int64_t n_out, const SlotGeom &g,
                                const int32_t *idx, int32_t K, uint16_t *y, hipStream_t stream);

// ---- gemm_decode.hip: skinny base GEMM for T <= 64 -------------------------------------------
struct DecodeCfg {
    int tt;        // token tiles of 16
    int sk;        // split of n_in across workgroups
    int kr;        // n_in per workgroup (multiple of 128)
    int n_tiles;   // row tiles of 64
};
DecodeCfg decode_config(int64_t T, int64_t n_in, int64_t n_out);
size_t decode_partial_bytes(int64_t T, int64_t n_in, int64_t n_out);
// part[s][tile][t][0:64] = x[t, split s] . W[tile*64 + (0:64), split s]; with upart != nullptr
// the same launch writes the unscaled shrink partials upart[s][j][t][0:n_slices*R] of every
// pair (-1 pairs skipped).  T above 64: chunks of 64 tokens in one launch, each with its own
// part and upart blocks (token stride 64; decode_partial_bytes covers them all).
// W: row-major [n_out][n_in], or the packed layout of pack.hip when `packed`.  With many more
// (chunk, tile, split) items than CUs the launch takes a persistent grid of one workgroup per
// CU (decode_gemm_persistent), which holds every CU until it ends.
hipError_t launch_decode_gemm(const uint16_t *x, const uint16_t *W, bool packed, int64_t T,
                              int64_t n_in, int64_t n_out, float *part, const DecodeCfg &cfg,
                              const SlotGeom *g, const int32_t *idx, int32_t K, float *upart,
                              hipStream_t stream);
// Whether launch_decode_gemm takes the persistent grid for these sizes.
bool decode_gemm_persistent(int64_t T, int64_t n_in, int64_t n_out);
// Whether the decode path's shrink runs apart from the GEMM (launch_shrink_pairs, pieces
// layout) for a launch of T tokens, K slots, n_out rows and slots of wd rows.
bool decode_shrink_apart(int64_t T, int32_t K, int64_t n_out, int32_t wd);
// ---- decode_finish.hip: y = bf16(sum of the split partials + LoRA delta), T <= 64 ----------
// part: fp32 [sk][n_tiles][T][64] (launch_decode_gemm); upart: fp32 [usk][K][T][wd] unscaled
// shrink pieces, usk = the GEMM's sk or 1 when the shrink ran apart (nullptr: base only, g
// unused); ysum: fp32 [T][n_out], the same sums before rounding, or nullptr
hipError_t launch_decode_finish(const float *part, int32_t sk, int32_t n_tiles, const float *upart,
                                int32_t usk, const float *scale, int64_t T, int64_t n_out,
                                const SlotGeom *g, const int32_t *idx, int32_t K, uint16_t *y,
                                float *ysum, hipStream_t stream);

// ---- pack.hip: W in the matrix cores' fragment order ------------------------------------------
// Wp[rg][kb][lane][8] = W[16 rg + lane % 16][32 kb + 8 (lane / 16) + e], zero padded.
int64_t packed_weight_elems(int64_t n_out, int64_t n_in);
hipError_t launch_pack_weight(const uint16_t *W, int64_t n_out, int64_t n_in, uint16_t *Wp,
                              hipStream_t stream);

// ---- slot_load.hip: zero padding of a loaded slot and its scale factor ----------------------
// A_slot: bf16 [n_slices][R][n_in] of the slot; B_slot: bf16 [n_out][R]; rows/columns >= r.
hipError_t launch_slot_pad(uint16_t *A_slot, uint16_t *B_slot, float *factor, int32_t R,
                           int32_t r, int32_t n_slices, int64_t n_in, int64_t n_out, float f,
                           hipStream_t stream);

// ---- gemm_prefill.hip: tiled MFMA GEMM with the LoRA delta as extra K-steps ---------------
struct PrefillCfg {
    int n_mtiles, n_ntiles;   // 256-token x 256-row output tiles
    int list_stride;          // max distinct adapters per token tile
    int64_t vcat_tile_elems;  // bf16 elements of one tile's V block
    int sc_cap;               // scattered tiles whose expand runs outside the GEMM
    int64_t n_out;
    int tok_stride;           // bytes of a tile's per-adapter token lists in the tile plan's LDS (256 K)
    int sd_cap_slots;         // fp32 partial blocks of the dense shrink items (256 x 128 each)
    int grp_stride;           // group records per tile (scattered tiles' 16-token groups)
    bool may_scatter;         // some tile could be scattered (else no expand launches)
};
PrefillCfg prefill_config(int64_t T, int32_t K, int64_t n_in, int64_t n_out, int32_t S, int32_t R,
                          int32_t n_slices);
size_t prefill_workspace_bytes(const PrefillCfg &c);
// Whether the tiled kernels are estimated faster than the decode kernels for these sizes
// (host only: a model of both paths' measured rates).
bool prefill_worth_it(int64_t T, int64_t n_in, int64_t n_out, int32_t K, int32_t wd);
bool grouped_decode_worth_it(int64_t T, int32_t K, int64_t n_in, int64_t n_out, int32_t wd,
                             int32_t R);
// y = bf16(x W^T + LoRA delta); g == nullptr: base only.  ws: prefill_workspace_bytes(c).
// Profiling hook (mlora_trace_start): records the begin/end event of the main product kernel.
void trace_mark(hipStream_t stream, bool begin);

hipError_t launch_prefill(const uint16_t *x, const uint16_t *W, bool packed, int64_t T,
                          int64_t n_in, int64_t n_out, const SlotGeom *g, const int32_t *idx,
                          int32_t K, const float *scale, uint16_t *y, const PrefillCfg &c,
                          void *ws, hipStream_t stream);

// Grouped decode: the decode kernels' base product with the LoRA terms computed per adapter
// group by the tiled path's scattered-tile kernels (every 256-token tile scattered).  Order:
// launch_grouped_shrink (tile plan, group items into V), the decode GEMM and finish without
// LoRA (the finish also leaves the fp32 sums in grouped_base_sums(c, ws), [T][n_out]), then
// launch_grouped_expand (adds each token's delta, rounds y).  Only while
// grouped_decode_fits(c) (every tile's fp32 sums kept); c: grouped_config(T, ...), ws:
// prefill_workspace_bytes(c).
// the tiled path's configuration for a grouped-decode launch of T tokens (no dense regions)
PrefillCfg grouped_config(int64_t T, int32_t K, int64_t n_in, int64_t n_out, int32_t S, int32_t R,
                          int32_t n_slices);
bool grouped_decode_fits(const PrefillCfg &c);
hipError_t launch_grouped_shrink(const uint16_t *x, int64_t T, int64_t n_in, int64_t n_out,
                                 const SlotGeom &g, const int32_t *idx, int32_t K,
                                 const float *scale, const PrefillCfg &c, void *ws,
                                 hipStream_t stream);
float *grouped_base_sums(const PrefillCfg &c, void *ws);
hipError_t launch_grouped_expand(int64_t T, int64_t n_out, const SlotGeom &g, const int32_t *idx,
                                 int32_t K, uint16_t *y, const PrefillCfg &c, void *ws,
                                 hipStream_t stream);

// ---- noalloc.hip: the fixed per-device scratch of mlora_linear_noalloc ----------------------
// Device address of this library's scratch array on the stream's device (looked up once per
// device with hipGetSymbolAddress), MLORA_NOALLOC_SCRATCH_BYTES long.
hipError_t noalloc_scratch(hipStream_t stream, void **ptr);

}  // namespace mlora
