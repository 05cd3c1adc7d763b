// Decode path (T <= 64 per launch): skinny base GEMM, LoRA shrink and, in the fused variant,
// LoRA expand and the final rounding, all in one launch.
//
// "Multi-LoRA Serving Explained" (sevydevy.com): every token of the batch is multiplied by the
// shared base weight in one product, then each token's side path (shrink by its own A, expand
// by its own B, found through its slot id) is added.  At decode sizes the base product reads W
// (n_out x n_in bf16) once and is bound by HBM bandwidth, so this kernel is built to stream W:
//
//  - a workgroup owns 64 rows of W ("tile") and one split of n_in (up to 8 x 128 columns)
//    and has 8 waves; wave w owns the w-th 128 columns of the split for all 64 rows;
//  - each lane first loads its share of x (all T tokens of the wave's 128 columns, read once
//    per workgroup with whole cache lines per instruction), then the A rows of its
//    workgroup's share of the LoRA shrink, then all of its W fragments (16 x 16 bytes); vmcnt
//    is in order, so the x and A data are usable while W streams in.  x is moved into the
//    MFMA operand layout through the wave's own 16 KB of LDS (XOR-swizzled, conflict-free);
//  - the products run on the matrix cores (v_mfma_f32_16x16x32_bf16: W rows = A operand,
//    16-token tiles of x = B operand).  The order in which a lane's bytes map onto the MFMA's
//    k positions is a permutation shared by both operands, which a sum allows;
//  - the shrink of a (token, slot) pair is the same kind of product with A[a]'s rows in place
//    of W's: one extra MFMA per 32 columns against the x fragments already in registers,
//    keeping the pair's token column;
//  - the 8 waves' partial tiles are added in LDS in a fixed order (deterministic) and the
//    split's partial tile goes to fp32 scratch.
// Two-kernel variant: the expand kernel then adds the splits in order, adds the LoRA delta
// and rounds y once.  Fused variant (one launch; every workgroup of the grid must be resident
// at once, which the host checks with the occupancy API): each workgroup publishes its shrink
// pieces and its split's partial tile with L2-bypassing (sc1) stores, waits for its own stores
// to complete, and then adds 1 to its tile's counter in the workspace.  It then waits (bounded)
// until every tile counter has reached sk -- all shrink partials and all partial tiles exist --
// and finishes 64/sk of its tile's rows: the split partials summed in split order,
// v = s*f * (the shrink partials summed in split order), delta = B[a] v, y = bf16(base + delta).
// Two counter sets alternate from call to call (a parity word in the workspace says which);
// workgroup 0 zeroes the other set and flips the parity once every workgroup has started, so
// no counter is ever shared by more than sk writers and no cache-wide flush is needed.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace mlora {

constexpr int DEC_ROWS = 64;    // rows of W per workgroup
constexpr int DEC_WK = 128;     // columns of n_in per wave
constexpr int DEC_WAVES = 8;
constexpr uint32_t DEC_SPIN_LIMIT = 1u << 22;   // bounded wait (~1 s) in the fused kernel
constexpr int DEC_CSTRIDE = 8184;               // counter words per set (max tiles)

// 8 bf16 (packed in a u32x4) times 8 fp32, summed in order
__device__ __forceinline__ float dot8_bf16_f32(const u32x4 b, const float *v)
{
    float d = 0.f;
    d += bf16_lo(b.x) * v[0];
    d += bf16_hi(b.x) * v[1];
    d += bf16_lo(b.y) * v[2];
    d += bf16_hi(b.y) * v[3];
    d += bf16_lo(b.z) * v[4];
    d += bf16_hi(b.z) * v[5];
    d += bf16_lo(b.w) * v[6];
    d += bf16_hi(b.w) * v[7];
    return d;
}

// Agent-coherent (L2-bypassing) accesses for data handed between workgroups.
__device__ __forceinline__ void st_agent(float *p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float *p)
{
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_agent_u32(uint32_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Shrink piece of pair p, A rows r0..r0+15: D[16 rows][16 tokens] = A rows x (the token tile
// holding t), one MFMA per 32 columns on fragments already in registers; the pair's token
// column is summed over the 8 waves (fixed order) and written to upart[s][j][t][r0..].
template <int TT, bool AGENT>
__device__ __forceinline__ void decode_shrink_piece(const u32x4 (&xf)[TT][4], const u32x4 (&af)[4],
                                                    int p, int r0, int K, int T, int wd, int s,
                                                    int wave, int r, int gq,
                                                    float (*sred)[16], float *upart)
{
    const int t = p / K;
    const int tt = t >> 4;
    f32x4 d = {0.f, 0.f, 0.f, 0.f};
    // uniform branch per token tile with compile-time indices: a runtime index into xf would
    // put the fragments in scratch memory
#pragma unroll
    for (int q = 0; q < TT; ++q) {
        if (q == tt) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af[ks]),
                                                            __builtin_bit_cast(bf16x8, xf[q][ks]),
                                                            d, 0, 0, 0);
        }
    }
    if (r == (t & 15)) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            sred[wave][gq * 4 + i] = d[i];
    }
    lds_barrier();
    if (threadIdx.x < 16 && r0 + (int)threadIdx.x < wd) {
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < DEC_WAVES; ++w)
            sum += sred[w][threadIdx.x];
        const int j = p - t * K;
        float *dst = upart + (((int64_t)s * K + j) * T + t) * wd + r0 + threadIdx.x;
        if constexpr (AGENT)
            st_agent(dst, sum);
        else
            *dst = sum;
    }
    lds_barrier();
}

struct DecodeArgs {
    const uint16_t *x, *W;
    int T, n_in, n_out, n_tiles, ks_cols, sk;
    SlotGeom g;
    const int32_t *idx;
    int K;
    const float *scale;
    float *part;       // two-kernel: [sk][T][n_out]; fused: [sk][n_tiles][T][64]
    float *upart;      // [sk][K][T][wd] or nullptr (no LoRA)
    int n_pairs;
    uint32_t *sync;    // fused: [0] parity, [1] spin timeouts, counter set p at [16 + p*DEC_CSTRIDE]
    uint16_t *y;       // fused: output
};

// One output of the fused epilogue: y[t][n] = bf16(sum of the split partials + LoRA delta).
// With pre, the B chunks come from eb (chunk u = B[a_j][n][rho..rho+8), u*8 = j*R + rho).
template <int BPRE, typename Args>
__device__ __forceinline__ void decode_output(const Args &P, const SlotGeom &g,
                                              const float *upart, const float *vsh, int tile,
                                              int t, int rl, int wd, bool pre,
                                              const u32x4 (&eb)[BPRE])
{
    const int n_out = P.n_out, n_tiles = P.n_tiles, T = P.T, K = P.K, R = g.R;
    const int64_t n = (int64_t)tile * 64 + rl;
    float base = 0.f;
    for (int sp = 0; sp < P.sk; ++sp)
        base += ld_agent(P.part + (((int64_t)sp * n_tiles + tile) * T + t) * 64 + rl);
    float delta = 0.f;
    if (upart != nullptr) {
        int sg = 0;
        while (sg + 1 < g.n_slices && n >= g.slice_start[sg + 1])
            ++sg;
        if (pre) {
            // -1 slots have zero B chunks and zero v, so every chunk can be added
#pragma unroll
            for (int u = 0; u < BPRE; ++u) {
                const int j = (u * 8) / R;
                if (j < K) {
                    const int rho = u * 8 - j * R;
                    delta += dot8_bf16_f32(eb[u], vsh + (j * T + t) * wd + sg * R + rho);
                }
            }
        } else {
            for (int j = 0; j < K; ++j) {
                const int a = P.idx[t * K + j];
                if (a < 0)
                    continue;
                const float *vv = vsh + (j * T + t) * wd + sg * R;
                const uint16_t *brow = g.B + ((int64_t)a * n_out + n) * R;
                float dj = 0.f;
                for (int rho = 0; rho < R; rho += 8)
                    dj += dot8_bf16_f32(*(const u32x4 *)(brow + rho), vv + rho);
                delta += dj;
            }
        }
    }
    P.y[(int64_t)t * n_out + n] = f32_to_bf16(base + delta);
}

template <int TT, bool FUSED>
__global__ __launch_bounds__(512) void decode_gemm_kernel(DecodeArgs P)
{
    extern __shared__ __attribute__((aligned(16))) float red[];   // [8][4][TT][64] float4
    __shared__ float sred[DEC_WAVES][16];
    const uint16_t *__restrict__ x = P.x;
    const uint16_t *__restrict__ W = P.W;
    const int T = P.T, n_in = P.n_in, n_out = P.n_out, n_tiles = P.n_tiles, K = P.K;
    const SlotGeom &g = P.g;
    const int tile = blockIdx.x % n_tiles;
    const int s = blockIdx.x / n_tiles;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int r = lane & 15;     // row (A operand) / token (B operand) within a 16-tile
    const int gq = lane >> 4;    // which 16-byte chunk group of the k-step this lane supplies
    const int kw = s * P.ks_cols + wave * DEC_WK;      // first column of this wave
    const bool wave_on = kw < n_in && wave * DEC_WK < P.ks_cols;
    float *upart = P.upart;
    // counter set of this call (fused): the parity word only changes after every workgroup of
    // the call has read it
    uint32_t par = 0;
    if constexpr (FUSED)
        par = ld_agent_u32(&P.sync[0]) & 1u;

    // column of the chunk this lane supplies at k-step ks: the 4 lanes of a row read 64
    // contiguous bytes per instruction (16 cache lines per wave instruction)
    auto col = [&](int ks) { return kw + (ks * 4 + gq) * 8; };

    // ---- x: the wave's T x 128 slice, loaded line-friendly (lane l reads 16 bytes of row
    //      tt*16 + ks*4 + l/16 at chunk l%16: 8 full cache lines per instruction), then moved
    //      through this wave's own 16 KB of LDS into the MFMA layout (fragment (tt, ks): token
    //      tt*16 + r, chunk ks*4 + gq).  LDS chunk (row, c) is stored at c ^ (row & 15).
    uint16_t *xl = (uint16_t *)(red + wave * (4 * TT * 64 * 4));   // [16*TT rows][16 chunks]
    u32x4 xf[TT][4];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int row = tt * 16 + ks * 4 + gq;
            const int c = kw + r * 8;
            xf[tt][ks] = (wave_on && row < T && c < n_in)
                             ? *(const u32x4 *)(x + (int64_t)row * n_in + c)
                             : u32x4{0u, 0u, 0u, 0u};
        }
    // ---- first shrink piece of this workgroup: pair p = tile, rows 0..15 of A[a]
    const int wd = g.n_slices * g.R;
    int a0 = -1;
    if (upart != nullptr && tile < P.n_pairs)
        a0 = P.idx[tile];
    u32x4 af[4];
    if (a0 >= 0) {
        const int arow = min(r, wd - 1);
        const uint16_t *ap = g.A + ((int64_t)a0 * wd + arow) * n_in;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int c = col(ks);
            af[ks] = (wave_on && c < n_in && r < wd) ? *(const u32x4 *)(ap + c)
                                                     : u32x4{0u, 0u, 0u, 0u};
        }
    }

    // ---- W fragments: row tile rt, k-step ks
    u32x4 wf[4][4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
        const int row = tile * DEC_ROWS + rt * 16 + r;
        const uint16_t *wrow = W + (int64_t)min(row, n_out - 1) * n_in;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int c = col(ks);
            wf[rt][ks] = (wave_on && c < n_in && row < n_out) ? *(const u32x4 *)(wrow + c)
                                                              : u32x4{0u, 0u, 0u, 0u};
        }
    }

#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int row = tt * 16 + ks * 4 + gq;
            *(u32x4 *)(xl + (row * 16 + (r ^ (row & 15))) * 8) = xf[tt][ks];
        }
    // the reads below take other lanes' writes: complete them and keep the compiler from
    // moving the reads above them (LDS executes one wave's operations in order)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int row = tt * 16 + r;
            const int c = ks * 4 + gq;
            xf[tt][ks] = *(const u32x4 *)(xl + (row * 16 + (c ^ (row & 15))) * 8);
        }

    if (a0 >= 0)
        decode_shrink_piece<TT, FUSED>(xf, af, tile, 0, K, T, wd, s, wave, r, gq, sred, upart);

    // ---- base products
    f32x4 acc[4][TT];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
            acc[rt][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int tt = 0; tt < TT; ++tt)
                acc[rt][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, wf[rt][ks]), __builtin_bit_cast(bf16x8, xf[tt][ks]),
                    acc[rt][tt], 0, 0, 0);

    // ---- remaining shrink pieces (other row groups, other pairs of this tile)
    if (upart != nullptr) {
        for (int p = tile; p < P.n_pairs; p += n_tiles) {
            const int a = P.idx[p];
            if (a < 0)
                continue;
            for (int r0 = (p == tile ? 16 : 0); r0 < wd; r0 += 16) {
                u32x4 afr[4];
                const int arow = r0 + r;
                const uint16_t *ap = g.A + ((int64_t)a * wd + min(arow, wd - 1)) * n_in;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const int c = col(ks);
                    afr[ks] = (wave_on && c < n_in && arow < wd) ? *(const u32x4 *)(ap + c)
                                                                 : u32x4{0u, 0u, 0u, 0u};
                }
                decode_shrink_piece<TT, FUSED>(xf, afr, p, r0, K, T, wd, s, wave, r, gq, sred, upart);
            }
        }
    }

    // ---- add the 8 waves' tiles in a fixed order and store the split's partial tile
    float4 *red4 = (float4 *)red;
    constexpr int SLOTS = 4 * TT * 64;   // float4 outputs of the workgroup
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
            red4[wave * SLOTS + (rt * TT + tt) * 64 + lane] =
                float4{acc[rt][tt][0], acc[rt][tt][1], acc[rt][tt][2], acc[rt][tt][3]};
    lds_barrier();
    for (int sl = threadIdx.x; sl < SLOTS; sl += 512) {
        float4 sum = red4[sl];
#pragma unroll
        for (int w = 1; w < DEC_WAVES; ++w) {
            const float4 v = red4[w * SLOTS + sl];
            sum.x += v.x;
            sum.y += v.y;
            sum.z += v.z;
            sum.w += v.w;
        }
        const int ln = sl & 63;
        const int rt = sl / (64 * TT);
        const int tt = (sl / 64) % TT;
        const int tok = tt * 16 + (ln & 15);
        const int rloc = rt * 16 + (ln >> 4) * 4;   // row within the tile
        if (tok < T) {
            if constexpr (FUSED) {
                float *dst = P.part + (((int64_t)s * n_tiles + tile) * T + tok) * DEC_ROWS + rloc;
                st_agent(dst + 0, sum.x);
                st_agent(dst + 1, sum.y);
                st_agent(dst + 2, sum.z);
                st_agent(dst + 3, sum.w);
            } else {
                const int nb = tile * DEC_ROWS + rloc;
                float *dst = P.part + ((int64_t)s * T + tok) * n_out + nb;
                if (nb + 3 < n_out && (n_out & 3) == 0) {
                    *(float4 *)dst = sum;
                } else {
                    const float v4[4] = {sum.x, sum.y, sum.z, sum.w};
                    for (int q = 0; q < 4; ++q)
                        if (nb + q < n_out)
                            dst[q] = v4[q];
                }
            }
        }
    }
    if constexpr (!FUSED)
        return;

    // ================= fused epilogue =================
    // every store above has completed before the counter moves
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    uint32_t *cnt = P.sync + 16 + par * DEC_CSTRIDE;
    if (threadIdx.x == 0)
        __hip_atomic_fetch_add(&cnt[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    // rows [r_lo, r_hi) of the tile are finished by this workgroup; thread o handles outputs
    // o and o + 512 (token t = o / nr, row r_lo + o % nr).  Inputs that do not depend on other
    // workgroups are fetched before the wait.
    const int rows_per = (DEC_ROWS + P.sk - 1) / P.sk;
    const int r_lo = s * rows_per;
    const int r_hi = min(min(DEC_ROWS, r_lo + rows_per), n_out - tile * DEC_ROWS);
    const int nr = max(r_hi - r_lo, 0);
    const int R = g.R;
    const bool lora = upart != nullptr;
    constexpr int EPQ = 2;                     // outputs per thread
    constexpr int BPRE = 4;                    // prefetched 16-byte B chunks per output
    const bool bpre = lora && K * R <= BPRE * 8;
    int eo_t[EPQ], eo_r[EPQ];
    u32x4 eb[EPQ][BPRE];
#pragma unroll
    for (int q = 0; q < EPQ; ++q) {
        const int o = threadIdx.x + q * 512;
        eo_t[q] = -1;
        eo_r[q] = 0;
        if (o < nr * T) {
            eo_t[q] = o / nr;
            eo_r[q] = r_lo + (o - eo_t[q] * nr);
        }
        if (bpre) {
            // chunk u holds B[a_j][n][rho..rho+8) with u*8 = j*R + rho (zeros for -1 slots)
            const int64_t n = (int64_t)tile * DEC_ROWS + eo_r[q];
#pragma unroll
            for (int u = 0; u < BPRE; ++u) {
                const int j = (u * 8) / R;
                const int rho = u * 8 - j * R;
                const int a = (eo_t[q] >= 0 && j < K) ? P.idx[eo_t[q] * K + j] : -1;
                eb[q][u] = (a >= 0) ? *(const u32x4 *)(g.B + ((int64_t)a * n_out + n) * R + rho)
                                    : u32x4{0u, 0u, 0u, 0u};
            }
        }
    }

    // wait until every tile counter has reached sk (wave 0 polls them, one per lane)
    if (wave == 0) {
        uint32_t it = 0;
        bool all = false;
        while (!all && it < DEC_SPIN_LIMIT) {
            bool mine = true;
            for (int i = lane; i < n_tiles; i += 64)
                mine &= ld_agent_u32(&cnt[i]) >= (uint32_t)P.sk;
            all = __ballot(!mine) == 0ull;
            if (!all) {
                __builtin_amdgcn_s_sleep(2);
                ++it;
            }
        }
        if (lane == 0 && !all)
            atomicAdd(&P.sync[1], 1u);   // recorded for the host; the kernel still ends
        if (blockIdx.x == 0 && all) {
            // every workgroup has started (they all published): prepare the other counter set
            // for the next call and flip the parity word that all of them read at their start
            uint32_t *other = P.sync + 16 + (1 - par) * DEC_CSTRIDE;
            for (int i = lane; i < n_tiles; i += 64)
                __hip_atomic_store(&other[i], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            if (lane == 0)
                __hip_atomic_store(&P.sync[0], (uint32_t)(1 - par), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    asm volatile("" ::: "memory");
    __syncthreads();

    // v of every (slot, token) pair, in LDS: vsh[(j*T + t)*wd + c]
    float *vsh = red;
    if (lora && nr > 0) {
        const int nv = K * T * wd;
        for (int e = threadIdx.x; e < nv; e += blockDim.x) {
            const int c = e % wd;
            const int jt = e / wd;
            const int t = jt % T;
            const int j = jt / T;
            const int a = P.idx[t * K + j];
            float v = 0.f;
            if (a >= 0) {
                float sum = 0.f;
                for (int sp = 0; sp < P.sk; ++sp)
                    sum += ld_agent(upart + (((int64_t)sp * K + j) * T + t) * wd + c);
                v = (P.scale ? P.scale[t * K + j] : 1.f) * g.factor[a] * sum;
            }
            vsh[e] = v;
        }
    }
    lds_barrier();
    // the first EPQ outputs of each thread use their prefetched B chunks; any further outputs
    // (more than EPQ*512 of them when sk < 4) load theirs here
    const u32x4 none[BPRE] = {};
#pragma unroll
    for (int q = 0; q < EPQ; ++q)
        if (eo_t[q] >= 0)
            decode_output(P, g, upart, vsh, tile, eo_t[q], eo_r[q], wd, bpre, eb[q]);
    for (int o = threadIdx.x + EPQ * 512; o < nr * T; o += 512) {
        const int t = o / nr;
        decode_output(P, g, upart, vsh, tile, t, r_lo + (o - t * nr), wd, false, none);
    }
}

DecodeCfg decode_config(int64_t T, int64_t n_in, int64_t n_out)
{
    DecodeCfg c;
    c.tt = T <= 16 ? 1 : T <= 32 ? 2 : 4;   // callers pass T <= 64
    c.n_tiles = (int)((n_out + DEC_ROWS - 1) / DEC_ROWS);
    const int64_t wblocks = (n_in + DEC_WK - 1) / DEC_WK;          // 128-column blocks
    // each workgroup takes up to 8 blocks (one per wave); split further while the grid is
    // smaller than the 256 CUs
    int per = DEC_WAVES;
    while (per > 1 && c.n_tiles * ((wblocks + per - 1) / per) < 256)
        per >>= 1;
    c.kr = per * DEC_WK;
    c.sk = (int)((n_in + c.kr - 1) / c.kr);
    return c;
}

size_t decode_partial_bytes(int64_t T, int64_t n_in, int64_t n_out)
{
    const DecodeCfg c = decode_config(T, n_in, n_out);
    const size_t a = (size_t)c.sk * (size_t)T * (size_t)n_out * sizeof(float);
    const size_t b = (size_t)c.sk * c.n_tiles * (size_t)T * DEC_ROWS * sizeof(float);
    return std::max(a, b);
}

size_t decode_sync_words(int64_t n_out)
{
    return 16 + 2 * (size_t)DEC_CSTRIDE + 0 * (size_t)n_out;
}

bool decode_tiles_fit_sync(int64_t n_out) { return (n_out + DEC_ROWS - 1) / DEC_ROWS <= DEC_CSTRIDE; }

template <int TT, bool FUSED>
static hipError_t launch_tf(DecodeArgs &a, const DecodeCfg &c, hipStream_t stream)
{
    const size_t lds = (size_t)DEC_WAVES * 4 * TT * 64 * sizeof(float4);
    static size_t lds_allowed = 64 * 1024;
    if (lds > lds_allowed) {
        hipError_t e = hipFuncSetAttribute((const void *)decode_gemm_kernel<TT, FUSED>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess)
            return e;
        lds_allowed = lds;
    }
    const dim3 grid((unsigned)(c.n_tiles * c.sk)), block(512);
    hipLaunchKernelGGL((decode_gemm_kernel<TT, FUSED>), grid, block, lds, stream, a);
    return hipGetLastError();
}

static DecodeArgs make_args(const uint16_t *x, const uint16_t *W, int64_t T, int64_t n_in,
                            int64_t n_out, float *part, const DecodeCfg &c, const SlotGeom *g,
                            const int32_t *idx, int32_t K, const float *scale, float *upart)
{
    DecodeArgs a{};
    a.x = x;
    a.W = W;
    a.T = (int)T;
    a.n_in = (int)n_in;
    a.n_out = (int)n_out;
    a.n_tiles = c.n_tiles;
    a.ks_cols = c.kr;
    a.sk = c.sk;
    a.idx = idx;
    a.K = K;
    a.scale = scale;
    a.part = part;
    if (g != nullptr && upart != nullptr) {
        a.g = *g;
        a.upart = upart;
        a.n_pairs = (int)(T * K);
    }
    return a;
}

hipError_t launch_decode_gemm(const uint16_t *x, const uint16_t *W, int64_t T, int64_t n_in,
                              int64_t n_out, float *part, const DecodeCfg &cfg,
                              const SlotGeom *g, const int32_t *idx, int32_t K, float *upart,
                              hipStream_t stream)
{
    DecodeArgs a = make_args(x, W, T, n_in, n_out, part, cfg, g, idx, K, nullptr, upart);
    switch (cfg.tt) {
    case 1: return launch_tf<1, false>(a, cfg, stream);
    case 2: return launch_tf<2, false>(a, cfg, stream);
    case 4: return launch_tf<4, false>(a, cfg, stream);
    default: return hipErrorInvalidValue;
    }
}

// Workgroups of the fused kernel that the device keeps resident at once (0 if unknown).
template <int TT>
static int fused_capacity()
{
    static int cap = -1;
    if (cap < 0) {
        int dev = 0, cus = 0, per_cu = 0;
        const size_t lds = (size_t)DEC_WAVES * 4 * TT * 64 * sizeof(float4);
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipFuncSetAttribute((const void *)decode_gemm_kernel<TT, true>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &per_cu, (const void *)decode_gemm_kernel<TT, true>, 512, lds) != hipSuccess) {
            (void)hipGetLastError();
            cap = 0;
        } else {
            cap = cus * per_cu;
        }
    }
    return cap;
}

bool decode_fused_fits(int64_t T, int32_t K, int32_t wd, const DecodeCfg &cfg)
{
    // v of all pairs must fit the reduction buffer (LDS); every workgroup finishes >= 1 row;
    // the whole grid must be resident at once
    const size_t lds = (size_t)DEC_WAVES * 4 * cfg.tt * 64 * sizeof(float4);
    if ((size_t)K * T * wd * sizeof(float) > lds || cfg.sk > DEC_ROWS)
        return false;
    const int cap = cfg.tt == 1 ? fused_capacity<1>() : cfg.tt == 2 ? fused_capacity<2>()
                                                                    : fused_capacity<4>();
    return cfg.n_tiles * cfg.sk <= cap;
}

hipError_t launch_decode_fused(const uint16_t *x, const uint16_t *W, int64_t T, int64_t n_in,
                               int64_t n_out, float *part, const DecodeCfg &cfg, const SlotGeom *g,
                               const int32_t *idx, int32_t K, const float *scale, float *upart,
                               uint32_t *sync, uint16_t *y, hipStream_t stream)
{
    DecodeArgs a = make_args(x, W, T, n_in, n_out, part, cfg, g, idx, K, scale, upart);
    a.sync = sync;
    a.y = y;
    switch (cfg.tt) {
    case 1: return launch_tf<1, true>(a, cfg, stream);
    case 2: return launch_tf<2, true>(a, cfg, stream);
    case 4: return launch_tf<4, true>(a, cfg, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace mlora
