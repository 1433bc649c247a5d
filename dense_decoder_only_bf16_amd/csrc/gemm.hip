// MFMA matrix product C = A[M,K] B[N,K]^T for gfx950 with fused epilogues (prefill).
//
// All linear layers of the model are bias-free products with weights stored [out, in]
// (apidog.com/th "How to train your own ChatGPT for $50", part 3 on precision: the weight
// is cast to the activation dtype and applied with a plain linear map; yelogs.com
// architecture answer: no bias in any linear layer).  Because RMSNorm has no parameters,
// norm(x) W^T = r (x W^T) with r = 1/sqrt(mean(x^2) + eps) per row, so the norm that
// precedes a projection is applied as a row scale in the epilogue, from per-row sums of
// squares that the producer of x left behind.
//
// Compensated operands: a bf16 operand carries a relative rounding error of up to 2^-9, and
// in the MLP that error is amplified by the squared ReLU and summed over d_ff terms.  For
// the MLP products and the LM head the activation is therefore carried as a high part
// hi = bf16(a) and a low part lo = a - hi, and multiplied as hi W^T + lo W^T with fp32
// accumulation.  The low part is stored as an e4m3 byte (lo 2^8) and its product runs on
// the fp8 matrix cores against an e4m3 copy of the weight made in registers: the operand
// error left is about 2^-12 of a at worst, against 2^-9 for a plain bf16 operand.  The
// producing epilogue writes both parts.
//
// Tiling: a workgroup computes a 256 x 256 tile.  bf16: 2 x 4 waves (two per SIMD, so one
// wave's MFMAs cover the other's waits at barriers and LDS reads), each owning a 128 x 64
// sub-tile of 4 x 2 MFMA 32x32 tiles; fp32: 2 x 2 waves of 128 x 128.  Operands are
// staged in LDS in the MFMA-blocked form [rows/32][K/16][32][16]: one 32x16 block is
// exactly one wave's 16-deep operand, so every LDS operand read is 1 KB contiguous.
// Weights arrive in that blocked form from global memory (see kernels.h).
//
// Three main loops:
//  * bf16 (the model's dtype): global -> LDS with the gfx950 direct-to-LDS load
//    (global_load_lds_dwordx4), a ring of 5 LDS stages of 32 K-columns (all 160 KB), loads
//    issued four stages ahead; no staging registers and no LDS store instructions.  The operand
//    fragments of the next 16-deep step (also across a K-tile boundary) are read from LDS
//    while the MFMAs of the current step run (fragments double-buffered in registers,
//    reads interleaved one per MFMA).
//  * bf16 with a compensated operand (gemm_bf16_comp_kernel): 7 stages of one 16-deep step
//    holding the A and weight blocks, beside 3 slots of 64-deep groups of e4m3 low parts.
//  * fp32 (the small fp32 check model): loads staged through registers into two LDS
//    buffers (A kept row-major with an XOR swizzle).
// Workgroups are dealt round-robin to the 8 dies (XCDs), each with its own L2; tiles are
// renumbered so each die works on a contiguous range, walked in groups of 8 row tiles so
// tiles running together share A rows and weight columns in the die's L2.
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace nc {


template <typename T> struct KT {
    static constexpr int BK = 128 / (int)sizeof(T);  // elements per 128-byte row slice
    static constexpr int CPR = BK / 8;               // chunks per row slice
    static constexpr int KS = BK / 16;               // 16-deep MFMA steps per slice
};

constexpr int TBM = 256, TBN = 256;  // workgroup tile

// (m0, n0, tile column index) of this workgroup's tile, and its K tiles [kt0, kt1) of nk.
// The first tiles - p.tail workgroups take whole tiles, numbered XCD-aware: workgroup ids
// go round-robin over the 8 XCDs, so each XCD gets a contiguous run of tile numbers and its
// L2 sees whole row groups.  The last 2 p.tail workgroups, dispatched last, take one K half
// each of the last p.tail tiles (tail split, GemmArgs): workgroups 2 s and 2 s + 1 of them
// share tail tile s (`slot`; -1 for a whole tile).  `even`: the halves split at an even K
// tile.
struct TileWork {
    int m0, n0, tn, kt0, kt1, slot;
};
__device__ __forceinline__ TileWork tile_work(const GemmArgs& p, int nk, bool even) {
    constexpr int GM = 8;
    const int ntn = (p.N + TBN - 1) / TBN, ntm = (p.M + TBM - 1) / TBM;
    const int whole = ntn * ntm - p.tail;
    const int pid = blockIdx.x;
    TileWork w;
    w.kt0 = 0;
    w.kt1 = nk;
    w.slot = -1;
    int t;
    if (pid < whole) {
        const int xcd = pid % 8, loc = pid / 8, q8 = whole / 8, r8 = whole % 8;
        t = (xcd < r8) ? xcd * (q8 + 1) + loc : r8 * (q8 + 1) + (xcd - r8) * q8 + loc;
    } else {  // a K half of a tail tile
        const int v = pid - whole;
        w.slot = v / 2;
        t = whole + w.slot;
        const int mid = even ? (nk / 2) & ~1 : nk / 2;
        if (v % 2 == 0) w.kt1 = mid;
        else w.kt0 = mid;
    }
    const int grp = t / (GM * ntn), first_m = grp * GM;
    const int gsize = min(ntm - first_m, GM);
    const int tm = first_m + (t % (GM * ntn)) % gsize;
    w.tn = (t % (GM * ntn)) / gsize;
    w.n0 = w.tn * TBN;
    w.m0 = tm * TBM;
    return w;
}

// Row scales r_m of the tile (RELU2 / SOFTCAP), computed once into LDS.
__device__ __forceinline__ void tile_row_scales(const GemmArgs& p, int m0, float* rs, int nt) {
    for (int r = threadIdx.x; r < TBM; r += nt) {
        const int m = m0 + r;
        float s = 0.f;
        if (m < p.M)
            for (int q = 0; q < p.ss_in_parts; ++q) s += p.ss_in[(long long)q * p.ss_stride + m];
        rs[r] = 1.0f / sqrtf(s / (float)p.K + p.eps);
    }
}

// Transpose of a 4 x 4 block held by a lane quad: lane a (= lane % 4) holds x[k] = B[k][a]
// and leaves with x[k] = B[a][k].  Two rounds of quad DPP exchanges (lane xor 1, then xor 2);
// in each, a lane keeps the two entries whose bit already matches its own and takes the
// other two from its partner, one exchange per pair.
__device__ __forceinline__ void quad_transpose4(float (&x)[4], int a) {
#pragma unroll
    for (int k0 = 0; k0 < 4; k0 += 2) {  // bit 0: pairs (0, 1), (2, 3)
        const bool hi = a & 1;
        const float r = dpp_lane<DPP_QUAD_XOR1>(hi ? x[k0] : x[k0 + 1]);
        if (hi) x[k0] = r;
        else x[k0 + 1] = r;
    }
#pragma unroll
    for (int k0 = 0; k0 < 2; ++k0) {  // bit 1: pairs (0, 2), (1, 3)
        const bool hi = a & 2;
        const float r = dpp_lane<DPP_QUAD_XOR2>(hi ? x[k0] : x[k0 + 2]);
        if (hi) x[k0] = r;
        else x[k0 + 2] = r;
    }
}

// bf16 RELU2 / RESID epilogue of the 2 x 4-wave kernels with each lane finishing 4
// consecutive columns of one row.  In the accumulator layout a lane holds one column and
// rows 8 q + 4 hh + k (k < 4) of each 32-row block; a quad transpose turns every such 4 x 4
// block around, so lane 4 c + e holds row 8 q + 4 hh + e, columns 4 c .. 4 c + 3.  Then x
// moves as 16-byte loads and stores and the blocked bf16 outputs as 8-byte stores (4
// columns of one 16-column chunk), a quarter of the memory instructions of the column
// layout.  N and ldo are multiples of 4 (host check), so a lane's 4 columns all exist or
// none does.
template <int EPI>
__device__ __forceinline__ void tile_epilogue4(const GemmArgs& p, f32x16 (&acc)[4][2], int m0, int n0, const float* rs,
                                               float (*red)[TBM]) {
    constexpr int WN = 4, IM = 4, JN = 2;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int l32 = lane & 31, hh = lane >> 5;
    const int e = l32 & 3, cq = l32 & ~3;
#pragma unroll
    for (int i = 0; i < IM; ++i) {
        const int rb = wm * 128 + i * 32 + 4 * hh + e;  // + 8 q: this lane's rows in the tile
        // RESID: the old residual of every row and column this lane finishes in this row
        // block, all loaded before any store (the stores write the same array)
        f32x4 xold[4][JN];
        if (EPI == EPI_RESID) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int j = 0; j < JN; ++j) {
                    const int m = min(m0 + rb + 8 * q, p.M - 1);
                    const int n = min(n0 + wn * 64 + j * 32 + cq, p.N - 4);
                    xold[q][j] = *(const f32x4*)(p.out_f32 + (long long)m * p.ldo + n);
                }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int rl = rb + 8 * q, m = m0 + rl;
            float sq = 0.f;
#pragma unroll
            for (int j = 0; j < JN; ++j) {
                float v[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) v[k] = acc[i][j][4 * q + k];
                quad_transpose4(v, e);
                const int n = n0 + wn * 64 + j * 32 + cq;
                const bool ok = m < p.M && n < p.N;
                const long long ot = blocked_index(m, n, p.ldo);
                bf16x4 hi;
                float lo[4];
                if (EPI == EPI_RELU2) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const float t = fmaxf(v[k] * rs[rl], 0.f);
                        hi[k] = (bf16)(t * t);
                        lo[k] = t * t - (float)hi[k];
                    }
                } else {  // EPI_RESID
                    const long long o = (long long)m * p.ldo + n;
                    f32x4 xn;
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        xn[k] = ok ? resid_value(p.rx, o + k, xold[q][j][k], v[k]) : 0.f;
                        hi[k] = (bf16)xn[k];
                        lo[k] = xn[k] - (float)hi[k];
                        sq += xn[k] * xn[k];
                    }
                    if (ok) *(f32x4*)(p.out_f32 + o) = xn;
                }
                if (ok) {
                    *(bf16x4*)((bf16*)p.out_t + ot) = hi;
                    // the low parts as e4m3 in the lo8 layout: 4 consecutive bytes (n % 4 == 0)
                    if (p.out_lo)
                        *(uint32_t*)((unsigned char*)p.out_lo + lo8_index(m, n, p.ldo)) =
                            e4m3x4(lo[0], lo[1], lo[2], lo[3], (float)(1 << LO8_SHIFT));
                }
            }
            if (EPI == EPI_RESID) {  // the row's sum over the wave's 64 columns: the 8 quads
                sq += __shfl_xor(sq, 4, 64);
                sq += __shfl_xor(sq, 8, 64);
                sq += __shfl_xor(sq, 16, 64);
                if (cq == 0) red[wn][rl] = sq;
            }
        }
    }
    if (EPI == EPI_RESID) {
        __syncthreads();
        for (int r = tid; r < TBM; r += 512) {
            const int m = m0 + r;
            float s = 0.f;
#pragma unroll
            for (int w = 0; w < WN; ++w) s += red[w][r];
            if (m < p.M) p.ss_out[(long long)(n0 / TBN) * p.ss_stride + m] = s;
        }
    }
}

// Epilogue on the accumulators of a workgroup of WM x WN waves: wave (wm, wn) owns rows
// m0 + wm (256/WM) + [0, 256/WM) and columns n0 + wn (256/WN) + [0, 256/WN); its lane holds
// column n0 + wn (256/WN) + 32 j + l32 and rows ... + 32 i + 8 (r/4) + 4 hh + (r%4) of
// acc[i][j][r].  RESID leaves one sum of squares per row and tile in ss_out.
template <typename T, int EPI, int WM, int WN>
__device__ __forceinline__ void tile_epilogue(const GemmArgs& p, f32x16 (&acc)[256 / WM / 32][256 / WN / 32],
                                              int m0, int n0, int tn, const float* rs, float (*red)[TBM]) {
    constexpr int IM = 256 / WM / 32, JN = 256 / WN / 32, NT = 64 * WM * WN;
    const float inv_cap = 1.0f / p.cap;  // SOFTCAP
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int l32 = lane & 31, hh = lane >> 5;
#pragma unroll
    for (int i = 0; i < IM; ++i) {
        // RESID: the old residual of this row tile, all loaded before any store (the stores
        // write the same array, so the compiler could not move a later load above them and
        // every element would wait a full memory round trip)
        float xold[16][JN];
        if (EPI == EPI_RESID) {
#pragma unroll
            for (int jr = 0; jr < 16; ++jr) {
                const int m = min(m0 + wm * (256 / WM) + i * 32 + 8 * (jr / 4) + 4 * hh + (jr % 4), p.M - 1);
#pragma unroll
                for (int j = 0; j < JN; ++j) {
                    const int n = min(n0 + wn * (256 / WN) + j * 32 + l32, p.N - 1);
                    xold[jr][j] = p.out_f32[(long long)m * p.ldo + n];
                }
            }
        }
#pragma unroll
        for (int jr = 0; jr < 16; ++jr) {
            const int rl = wm * (256 / WM) + i * 32 + 8 * (jr / 4) + 4 * hh + (jr % 4);
            const int m = m0 + rl;
            float sq = 0.f;
#pragma unroll
            for (int j = 0; j < JN; ++j) {
                const int n = n0 + wn * (256 / WN) + j * 32 + l32;
                const bool ok = (m < p.M) && (n < p.N);
                const float v = acc[i][j][jr];
                const long long o = (long long)m * p.ldo + n;
                if (EPI == EPI_STORE) {
                    if (ok) p.out_f32[(long long)blockIdx.z * p.z_stride + o] = v;
                } else if (EPI == EPI_RELU2) {
                    const float t = fmaxf(v * rs[rl], 0.f);
                    const T hi = from_f32<T>(t * t);
                    const long long ot = sizeof(T) == 2 ? blocked_index(m, n, p.ldo) : o;
                    if (ok) ((T*)p.out_t)[ot] = hi;
                    if (ok && p.out_lo) ((T*)p.out_lo)[ot] = from_f32<T>(t * t - to_f32(hi));
                } else if (EPI == EPI_SOFTCAP) {
                    if (ok) p.out_f32[o] = softcap_f32(v * rs[rl], p.cap, inv_cap);
                } else {  // EPI_RESID
                    if (ok) {
                        const float xn = resid_value(p.rx, o, xold[jr][j], v);
                        p.out_f32[o] = xn;
                        const T hi = from_f32<T>(xn);
                        const long long ot = sizeof(T) == 2 ? blocked_index(m, n, p.ldo) : o;
                        ((T*)p.out_t)[ot] = hi;
                        if (p.out_lo) ((T*)p.out_lo)[ot] = from_f32<T>(xn - to_f32(hi));
                        sq += xn * xn;
                    }
                }
            }
            if (EPI == EPI_RESID) {  // the row's sum over the wave's 32 columns: lanes 16, 48
                sq = half_sum_hi_rows(sq);
                if (l32 == 16) red[wn][rl] = sq;
            }
        }
    }
    if (EPI == EPI_RESID) {
        __syncthreads();
        for (int r = tid; r < TBM; r += NT) {
            const int m = m0 + r;
            float s = 0.f;
#pragma unroll
            for (int w = 0; w < WN; ++w) s += red[w][r];
            if (m < p.M) p.ss_out[(long long)tn * p.ss_stride + m] = s;
        }
    }
}

// Tail split join (all 512 threads; after the main loop, with the ring free).  For a whole
// tile (slot < 0) it adds nothing.  Of the two halves of tail tile `slot`, the first to
// arrive stores its accumulators (device scope, thread-major so each 16-byte store is
// coalesced), waits for the stores and sets the ready flag, and is done (false); the other
// waits for the flag (bounded: the first is already running), adds the stored sums to its
// own and clears both words for the next launch (true).  A flag that never comes makes the
// tile NaN rather than wrong.  Every workgroup runs the same add, a whole tile's through a
// zero-size buffer (its loads return 0 without touching memory): one straight path keeps
// the accumulators in place for the epilogue instead of merging two versions of them.
__device__ __forceinline__ bool tail_join(const GemmArgs& p, int slot, f32x16 (&acc)[4][2], int* lflag) {
    const int tid = threadIdx.x;
    float* part = p.tail_part + (long long)(slot < 0 ? 0 : slot) * GEMM_TAIL_FLOATS;
    int32_t* ctr = p.tail_ctr + 2 * (slot < 0 ? 0 : slot);
    bool bad = false;
    if (slot >= 0) {
        if (tid == 0) lflag[0] = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0;
        __syncthreads();
        if (lflag[0]) {
            const __amdgpu_buffer_rsrc_t w = buffer_rsrc(part, GEMM_TAIL_FLOATS * 4);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        f32x4 v;
#pragma unroll
                        for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e];
                        store_device4(w, 16 * (((i * 2 + j) * 4 + q) * 512 + tid), v);
                    }
            wait_stores_complete();  // the sums are visible device-wide before the flag
            __syncthreads();
            if (tid == 0) __hip_atomic_store(ctr + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return false;
        }
        if (tid == 0) {
            int v = 0;
            for (int it = 0; it < (1 << 22); ++it) {
                v = __hip_atomic_load(ctr + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (v) break;
                __builtin_amdgcn_s_sleep(2);
            }
            lflag[1] = v ? 0 : 1;
            __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(ctr + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        bad = lflag[1] != 0;
        __syncthreads();  // every thread has read lflag before the epilogue reuses the LDS
    }
    const __amdgpu_buffer_rsrc_t r = buffer_rsrc(part, slot < 0 ? 0 : GEMM_TAIL_FLOATS * 4);
    const float keep = bad ? __builtin_nanf("") : 1.f;
    // A quarter of the sums at a time (32 registers in flight), so the accumulators and the
    // loads fit beside each other.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 v = load_device4(r, 16 * (((i * 2 + j) * 4 + q) * 512 + tid));
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[i][j][4 * q + e] = acc[i][j][4 * q + e] * keep + v[e];
            }
        __builtin_amdgcn_sched_barrier(0);
    }
    return true;
}

// ---------------------------------------------------------------------- bf16 ----------

template <int EPI>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_bf16_kernel(GemmArgs p) {
    constexpr int BK = 32, KB = BK / 16, NS = 5;
    constexpr int STAGE = (TBM + TBN) * BK;       // elements per stage (A then B)
    // The ring takes all 160 KB of LDS; after the main loop it holds the row scales and the
    // RESID row sums instead.
    __shared__ __attribute__((aligned(1024))) bf16 lds[NS * STAGE];
    float* rs = (float*)lds;
    float (*red)[TBM] = (float (*)[TBM])((float*)lds + TBM);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / 4, wn = wave % 4;       // 2 x 4 waves, 128 x 64 each
    const int l32 = lane & 31, hh = lane >> 5;
    const int ksteps = p.K / 16;
    // A compensated product runs twice as many K tiles: tile 2k takes A's columns of tile
    // k, tile 2k + 1 the same columns of A_lo, both against the same weight block.
    const bool comp = p.A_lo != nullptr;
    const TileWork tw = tile_work(p, comp ? 2 * (p.K / BK) : p.K / BK, comp);
    const int m0 = tw.m0, n0 = tw.n0, tn = tw.tn;
    const int kt0 = tw.kt0, nk = tw.kt1 - tw.kt0;  // this workgroup's K tiles kt0 + [0, nk)
    const bf16* A = (const bf16*)p.A;
    const bf16* A_lo = (const bf16*)p.A_lo;
    const bf16* B = (const bf16*)p.B;

    // RELU2 / SOFTCAP: the partial sums of squares of row m0 + (tid % 256) are loaded now and
    // reduced to the row scale after the main loop, so their latency overlaps it.
    constexpr int MAXP = 16;  // partial sums per row: one per 256 columns of d <= 4096
    float ssp[MAXP];
#pragma unroll
    for (int q = 0; q < MAXP; ++q) ssp[q] = 0.f;
    if (EPI == EPI_RELU2 || EPI == EPI_SOFTCAP) {
        const int m = min(m0 + (tid & (TBM - 1)), p.M - 1);
#pragma unroll
        for (int q = 0; q < MAXP; ++q)
            if (q < p.ss_in_parts) ssp[q] = p.ss_in[(long long)q * p.ss_stride + m];
    }

    // Stage layout: 16 A blocks (row block rb = b/2, k block b%2) then 16 B blocks.  Wave w
    // loads A blocks 2w, 2w+1 and B blocks 2w, 2w+1.  A and B are both stored blocked, so
    // each block is one contiguous 1 KB load (8 cache lines, fully used).  In LDS a block is
    // held in MFMA lane order: bytes [16 l, 16 l + 16) are what lane l of an operand read
    // takes, row l % 32, k half l / 32 (memory chunk 2 (l % 32) + l / 32), so each group of
    // 8 lanes that LDS serves together reads 128 contiguous bytes from all 32 banks (the
    // memory order would put two lanes of a group on the same banks).  A holds ceil(M/32)
    // whole 32-row blocks (rows past M are padding); a tile's row blocks past the last one
    // and weight blocks past Npad read a clamped block.  Their outputs are masked in the
    // epilogue.
    const int lchunk = 2 * l32 + hh;  // the memory chunk this lane moves into LDS chunk `lane`
    auto issue = [&](int kt) {
        bf16* sbase = lds + (kt % NS) * STAGE;
        const int kg = kt0 + kt;
        const int k0 = (comp ? kg >> 1 : kg) * BK;
        const bf16* As = (comp && (kg & 1)) ? A_lo : A;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int b = wave * 2 + u;
            const int rb = b / KB, kb = b % KB;
            int mb = m0 / 32 + rb;
            mb = mb < (p.M + 31) / 32 ? mb : (p.M + 31) / 32 - 1;  // tiles reach past the last block
            const bf16* src = As + ((long long)mb * (p.K / 16) + (k0 / 16 + kb)) * 512 + lchunk * 8;
            __builtin_amdgcn_global_load_lds((gvoid*)src, (lvoid*)(sbase + b * 512), 16, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int b = wave * 2 + u;
            const int rb = b / KB, kb = b % KB;
            int nb = n0 / 32 + rb;
            nb = nb < p.Npad / 32 ? nb : p.Npad / 32 - 1;
            const bf16* src = B + ((long long)nb * ksteps + k0 / 16 + kb) * 512 + lchunk * 8;
            __builtin_amdgcn_global_load_lds((gvoid*)src, (lvoid*)(sbase + (16 + b) * 512), 16, 0, 0);
        }
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = zero_vec<f32x16>();

    // Operand fragments of one 16-deep step: 4 A blocks and 2 B blocks.
    typedef bf16x8 FragA[4];
    typedef bf16x8 FragB[2];
    auto fload = [&](int kt, int s, FragA& fa, FragB& fb) {
        const bf16* sa = lds + (kt % NS) * STAGE;
        const bf16* sb = sa + TBM * BK;
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[i] = *(const bf16x8*)(sa + ((wm * 4 + i) * KB + s) * 512 + lane * 8);
#pragma unroll
        for (int j = 0; j < 2; ++j) fb[j] = *(const bf16x8*)(sb + ((wn * 2 + j) * KB + s) * 512 + lane * 8);
    };
    // 8 MFMAs of one step, with the 6 LDS reads of the next step interleaved (one read per
    // MFMA) so the reads' latency hides behind the matrix cores.
    auto mfmas = [&](FragA& fa, FragB& fb, bool interleave) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[i][j] = mma32(fa[i], fb[j], acc[i][j]);
        if (interleave) {
#pragma unroll
            for (int g = 0; g < 6; ++g) {
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        }
    };

    // Prologue: tiles 0 .. NS-2 in flight (4 loads per wave each), fragments of tile 0,
    // step 0 in registers.
#pragma unroll
    for (int kt = 0; kt < NS - 1; ++kt)
        if (kt < nk) issue(kt);
    if (nk > 3) NC_WAIT_VM(12);
    else if (nk > 2) NC_WAIT_VM(8);
    else if (nk > 1) NC_WAIT_VM(4);
    else NC_WAIT_VM(0);
    __builtin_amdgcn_s_barrier();
    FragA a0, a1;
    FragB b0, b1;
    fload(0, 0, a0, b0);
    for (int kt = 0; kt < nk; ++kt) {
        // step 0 of tile kt; read step 1 of tile kt meanwhile
        fload(kt, 1, a1, b1);
        mfmas(a0, b0, true);
        // Tile kt+1: own loads done (tiles kt+2, kt+3 may still be in flight), then a
        // barrier: every wave's loads of kt+1 are in LDS and every wave is done with tile
        // kt-1, whose stage the next issue overwrites.
        const bool more = kt + 1 < nk;
        if (more) {
            if (kt + 3 < nk) NC_WAIT_VM(8);
            else if (kt + 2 < nk) NC_WAIT_VM(4);
            else NC_WAIT_VM(0);
            __builtin_amdgcn_s_barrier();
            if (kt + NS - 1 < nk) issue(kt + NS - 1);
            fload(kt + 1, 0, a0, b0);  // step 0 of tile kt+1
        }
        mfmas(a1, b1, more);
    }
    __syncthreads();  // every wave is done with the ring (all its loads have landed)
    if (p.tail && !tail_join(p, tw.slot, acc, (int*)lds + 8192)) return;  // workgroup-uniform
    if (EPI == EPI_RELU2 || EPI == EPI_SOFTCAP) {
        if (tid < TBM) {
            float s = 0.f;
#pragma unroll
            for (int q = 0; q < MAXP; ++q) s += ssp[q];
            rs[tid] = 1.0f / sqrtf(s / (float)p.K + p.eps);
        }
        __syncthreads();
    }
    if constexpr (EPI == EPI_RELU2 || EPI == EPI_RESID) tile_epilogue4<EPI>(p, acc, m0, n0, rs, red);
    else tile_epilogue<bf16, EPI, 2, 4>(p, acc, m0, n0, tn, rs, red);
}

// Compensated products (A + A_lo against one weight: the MLP products and the LM head).  The
// high part runs the bf16 MFMAs of the plain kernel; the low part, a correction near 2^-9 of
// the operand, runs at fp8 rate: A_lo arrives as e4m3 bytes (lo8 layout, kernels.h), the
// weight fragments of every 16-deep step are converted to e4m3 in registers (w 2^w8_exp),
// and after four steps one scaled 32x32x64 e4m3 MFMA per accumulator tile adds
// lo W^T 2^-LO8_SHIFT 2^-w8_exp into the same fp32 accumulators.  Per 64 deep a wave then
// issues 32 bf16 and 8 fp8 MFMAs (the time of 48 bf16 ones, against 64 with a bf16 low
// part), and a 16-deep step moves 20 KB into LDS instead of 24 KB.
// LDS: a ring of 7 stages of one 16-deep step (the tile's 8 A and 8 weight blocks, 16 KB;
// wave w loads block w of each, loads issued six stages ahead) and a ring of 3 slots of one
// 64-deep group of low parts (8 row blocks x 2 KB).  A group's 16 KB low-part block loads
// are spread over its four steps' stages (waves 0-3 take one each), so it has landed when its
// last step's stage has, and its slot is refilled only two steps after that step's reads.
// Operand error of the product: the e4m3 rounding of lo (2^-4 relative) and of the weight
// copy (2^-4 relative) act on a term 2^-9 the size of a, leaving about 2^-12 of a at worst
// and far less on average, against 2^-9 for a plain bf16 operand.
template <int EPI>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_bf16_comp_kernel(GemmArgs p) {
    constexpr int NSM = 7, NSL = 3;  // main stages, low-part group slots
    constexpr int MST = 16 * 512;    // bf16 elements per main stage
    constexpr int LST = 16 * 1024;   // bytes per low-part slot
    __shared__ __attribute__((aligned(1024))) unsigned char lds[NSM * MST * 2 + NSL * LST];
    bf16* const ring = (bf16*)lds;
    unsigned char* const lring = lds + NSM * MST * 2;
    float* rs = (float*)lds;
    float (*red)[TBM] = (float (*)[TBM])((float*)lds + TBM);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / 4, wn = wave % 4;  // 2 x 4 waves, 128 x 64 each
    const int l32 = lane & 31, hh = lane >> 5;
    const int ksteps = p.K / 16, ngroups = p.K / 64;
    const TileWork tw = tile_work(p, ngroups, false);  // K tiles of 64 (K halves for the tail split)
    const int m0 = tw.m0, n0 = tw.n0, tn = tw.tn;
    const int g0 = tw.kt0;              // first 64-deep group
    const int nk = 4 * (tw.kt1 - g0);   // this workgroup's 16-deep steps (stages), from step 4 g0

    constexpr int MAXP = 16;
    float ssp[MAXP];
#pragma unroll
    for (int q = 0; q < MAXP; ++q) ssp[q] = 0.f;
    if (EPI == EPI_RELU2 || EPI == EPI_SOFTCAP) {
        const int m = min(m0 + (tid & (TBM - 1)), p.M - 1);
#pragma unroll
        for (int q = 0; q < MAXP; ++q)
            if (q < p.ss_in_parts) ssp[q] = p.ss_in[(long long)q * p.ss_stride + m];
    }

    // Wave w moves row block w of A and weight block w; lane l takes memory chunk
    // 2 (l % 32) + l / 32 of a block into LDS chunk l (MFMA lane order, as above).  The low
    // parts are already in lane order in memory and move as plain 1 KB copies.  Row blocks
    // past A's last and weight blocks past Npad read a clamped block; their outputs are
    // masked in the epilogue.
    const int lchunk = 2 * l32 + hh;
    const int mblast = (p.M + 31) / 32 - 1;
    const int mb = min(m0 / 32 + wave, mblast);
    const int nb = min(n0 / 32 + wave, p.Npad / 32 - 1);
    const bf16* srcA = (const bf16*)p.A + ((long long)mb * ksteps + 4 * g0) * 512 + lchunk * 8;
    const bf16* srcB = (const bf16*)p.B + ((long long)nb * ksteps + 4 * g0) * 512 + lchunk * 8;
    const unsigned char* lo8 = (const unsigned char*)p.A_lo + (long long)g0 * 2048 + lane * 16;
    auto issue = [&](int kt) {
        bf16* s = ring + (kt % NSM) * MST;
        __builtin_amdgcn_global_load_lds((gvoid*)(srcA + (long long)kt * 512), (lvoid*)(s + wave * 512), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((gvoid*)(srcB + (long long)kt * 512), (lvoid*)(s + (8 + wave) * 512), 16, 0, 0);
        if (wave < 4) {  // 1 KB half h of row block r of group kt / 4: load 4 (kt % 4) + wave
            const int g = kt >> 2, i = 4 * (kt & 3) + wave, r = i >> 1, h = i & 1;
            const int mbr = min(m0 / 32 + r, mblast);
            const unsigned char* src = lo8 + ((long long)mbr * ngroups + g) * 2048 + h * 1024;
            __builtin_amdgcn_global_load_lds((gvoid*)src, (lvoid*)(lring + (g % NSL) * LST + r * 2048 + h * 1024), 16, 0, 0);
        }
    };
    // this wave's loads per stage: 3 (waves 0-3) or 2; wait until at most n stages are in flight
    auto wait_stages = [&](int n) {
        if (wave < 4) {
            switch (n) {
                case 5: NC_WAIT_VM(15); break;
                case 4: NC_WAIT_VM(12); break;
                case 3: NC_WAIT_VM(9); break;
                case 2: NC_WAIT_VM(6); break;
                case 1: NC_WAIT_VM(3); break;
                default: NC_WAIT_VM(0); break;
            }
        } else {
            switch (n) {
                case 5: NC_WAIT_VM(10); break;
                case 4: NC_WAIT_VM(8); break;
                case 3: NC_WAIT_VM(6); break;
                case 2: NC_WAIT_VM(4); break;
                case 1: NC_WAIT_VM(2); break;
                default: NC_WAIT_VM(0); break;
            }
        }
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = zero_vec<f32x16>();
    i32x8 wq[2];  // e4m3 copies of this wave's two weight blocks over the current group's 4 steps
    const float winv = ldexpf(1.0f, -p.w8_exp);
    const int sa = 127 - LO8_SHIFT, sb = 127 - p.w8_exp;

    // A blocks 0..3, weight blocks 4..5, as raw 32-bit words: carried through the loop's
    // branches as vectors of bf16, the fragments were split into 16-bit halves and packed
    // again at every step (48 extra VALU instructions per step)
    typedef u32x4 Frag[6];
    auto fload = [&](int kt, Frag& f) {
        const bf16* s = ring + (kt % NSM) * MST + lane * 8;
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = *(const u32x4*)(s + (wm * 4 + i) * 512);
#pragma unroll
        for (int j = 0; j < 2; ++j) f[4 + j] = *(const u32x4*)(s + (8 + wn * 2 + j) * 512);
    };
    // One stage (step kt, q = kt % 4): wait until this wave's loads of stage kt + 1 have
    // landed (later stages, at most 4, may stay in flight), barrier (every wave's loads of
    // kt + 1 are in LDS and every wave is done with stage kt - 1, whose slot the next issue
    // refills), refill, then the 8 bf16 MFMAs of stage kt with the fragment reads of stage
    // kt + 1 interleaved, the weight blocks' e4m3 copy, and after the group's last step its
    // 8 e4m3 MFMAs.
    auto step = [&](auto qc, int kt, Frag& cur, Frag& nxt) {
        constexpr int q = decltype(qc)::value;
        const bool more = kt + 1 < nk;
        if (more) {
            wait_stages(min(NSM - 3, nk - 2 - kt));
            __builtin_amdgcn_s_barrier();
            if (kt + NSM - 1 < nk) issue(kt + NSM - 1);
            fload(kt + 1, nxt);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[i][j] = mma32(__builtin_bit_cast(bf16x8, cur[i]), __builtin_bit_cast(bf16x8, cur[4 + j]), acc[i][j]);
        if (more) {
#pragma unroll
            for (int g = 0; g < 6; ++g) {
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            int d0, d1;
            e4m3x8_bf16(__builtin_bit_cast(bf16x8, cur[4 + j]), winv, d0, d1);
            asm volatile("" ::"v"(d0), "v"(d1));  // converted in this step, not all at the group's end
            wq[j][2 * q] = d0;
            wq[j][2 * q + 1] = d1;
        }
        if constexpr (q == 3) {
            const unsigned char* ls = lring + ((kt >> 2) % NSL) * LST + lane * 32;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bf16x8 l0 = *(const bf16x8*)(ls + (wm * 4 + i) * 2048);
                const bf16x8 l1 = *(const bf16x8*)(ls + (wm * 4 + i) * 2048 + 16);
                const u32x4 u0 = __builtin_bit_cast(u32x4, l0), u1 = __builtin_bit_cast(u32x4, l1);
                const i32x8 la = {(int)u0[0], (int)u0[1], (int)u0[2], (int)u0[3], (int)u1[0], (int)u1[1], (int)u1[2], (int)u1[3]};
#pragma unroll
                for (int j = 0; j < 2; ++j) acc[i][j] = mma32_e4m3(la, wq[j], acc[i][j], sa, sb);
            }
        }
    };

    // Prologue: stages 0 .. NSM-2 in flight, stage 0's fragments.
#pragma unroll
    for (int kt = 0; kt < NSM - 1; ++kt)
        if (kt < nk) issue(kt);
    wait_stages(min(NSM - 2, nk - 1));
    // (the row statistics were loaded before the stages, so they have landed too: one
    // register instead of MAXP stays live across the main loop)
    float ssum = 0.f;
#pragma unroll
    for (int q = 0; q < MAXP; ++q) ssum += ssp[q];
    __builtin_amdgcn_s_barrier();
    Frag f0, f1;
    fload(0, f0);
    for (int kt = 0; kt < nk; kt += 4) {  // nk is a multiple of 4
        step(std::integral_constant<int, 0>{}, kt, f0, f1);
        step(std::integral_constant<int, 1>{}, kt + 1, f1, f0);
        step(std::integral_constant<int, 2>{}, kt + 2, f0, f1);
        step(std::integral_constant<int, 3>{}, kt + 3, f1, f0);
    }
    __syncthreads();  // every wave is done with the rings (all its loads have landed)
    if (p.tail && !tail_join(p, tw.slot, acc, (int*)lds + 8192)) return;  // workgroup-uniform
    if (EPI == EPI_RELU2 || EPI == EPI_SOFTCAP) {
        if (tid < TBM) rs[tid] = 1.0f / sqrtf(ssum / (float)p.K + p.eps);
        __syncthreads();
    }
    if constexpr (EPI == EPI_RELU2 || EPI == EPI_RESID) tile_epilogue4<EPI>(p, acc, m0, n0, rs, red);
    else tile_epilogue<bf16, EPI, 2, 4>(p, acc, m0, n0, tn, rs, red);
}

// ---------------------------------------------------------------------- fp32 ----------
template <int EPI>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_f32_kernel(GemmArgs p) {
    typedef float T;
    typedef typename Chunk<T>::type CT;
    constexpr int NT = 256;
    constexpr int BK = KT<T>::BK, CPR = KT<T>::CPR, KS = KT<T>::KS;
    constexpr int AL = TBM * CPR / NT, BL = TBN * CPR / NT;
    constexpr int KB16 = BK / 16;
    __shared__ __attribute__((aligned(32))) T As[2][TBM * BK];
    __shared__ __attribute__((aligned(32))) T Bs[2][TBN * BK];
    __shared__ float rs[TBM];
    __shared__ float red[2][TBM];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / 2, wn = wave % 2;
    const int l32 = lane & 31, hh = lane >> 5;
    const TileWork tw = tile_work(p, 1, false);  // no tail split: p.tail is 0
    const int m0 = tw.m0, n0 = tw.n0, tn = tw.tn;
    const int kspan = p.K / p.k_split;
    const int kbeg = blockIdx.z * kspan;
    const int nk = kspan / BK;
    const int ksteps = p.K / 16;
    const T* A = (const T*)p.A;
    const T* B = (const T*)p.B;

    if (EPI == EPI_RELU2 || EPI == EPI_SOFTCAP) tile_row_scales(p, m0, rs, NT);

    CT ra[AL], rb[BL];
    auto gload = [&](int kt) {
        const int k0 = kbeg + kt * BK;
#pragma unroll
        for (int i = 0; i < AL; ++i) {
            int q = tid + i * NT, r = q / CPR, c = q % CPR;
            int gm = m0 + r;
            const bool ok = gm < p.M;
            ra[i] = load_masked(A + (long long)(ok ? gm : 0) * p.lda + k0 + c * 8, ok);
        }
#pragma unroll
        for (int i = 0; i < BL; ++i) {
            int q = tid + i * NT, bq = q / 64, w = q % 64;
            int rbk = bq / KB16, kb = bq % KB16;
            int gn = n0 + 32 * rbk;
            const bool ok = gn < p.Npad;
            rb[i] = load_masked(B + ((long long)((ok ? gn : 0) / 32) * ksteps + k0 / 16 + kb) * 512 + w * 8, ok);
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < AL; ++i) {
            int q = tid + i * NT, r = q / CPR, c = q % CPR;
            *(CT*)(&As[buf][r * BK + ((c ^ (r % CPR)) * 8)]) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < BL; ++i) *(CT*)(&Bs[buf][(tid + i * NT) * 8]) = rb[i];
    };

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = zero_vec<f32x16>();

    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const int c = 2 * s + hh;
            CT a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                int r = wm * 128 + i * 32 + l32;
                a[i] = *(const CT*)(&As[buf][r * BK + ((c ^ (r % CPR)) * 8)]);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
                b[j] = *(const CT*)(&Bs[buf][((wn * 4 + j) * KB16 + s) * 512 + l32 * 16 + 8 * hh]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mma32(a[i], b[j], acc[i][j]);
        }
        if (kt + 1 < nk) sstore(buf ^ 1);
        __syncthreads();
    }
    tile_epilogue<T, EPI, 2, 2>(p, acc, m0, n0, tn, rs, red);
}

// Tail split (GemmArgs): the last round of workgroups (256 CUs, one 160 KB workgroup each)
// holds tiles % 256 tiles; when that is at most half a round they run as 2 K halves each, so
// the round is twice as full and ends in about half the time.  With the split on, every
// workgroup runs the join's add (a whole tile's through an empty buffer), about a microsecond
// per tile, so it is kept to K of at least 64 K tiles (2048), where half a round is worth
// far more: d26's MLP down-projection (K 6656) 1488 -> 1362 us, its attention output
// projection (K 1664) 349 -> 345 us.
static int tail_tiles(const GemmArgs& a, int tiles, int ktiles) {
    if (!a.tail_part || !a.tail_ctr || ktiles < 64) return 0;
    const int r = tiles % 256;
    return (r > 0 && r <= 128 && r <= GEMM_TAIL_SLOTS) ? r : 0;
}

template <int EPI>
static hipError_t launch_e(DType dt, const GemmArgs& a_in, hipStream_t st) {
    GemmArgs a = a_in;
    const int tiles = ((a.N + TBN - 1) / TBN) * ((a.M + TBM - 1) / TBM);
    a.tail = dt == BF16 ? tail_tiles(a, tiles, a.K / 32) : 0;
    dim3 grid(tiles + a.tail, 1, a.k_split);
    if (dt == BF16) {
        if (a.k_split != 1 || a.K % 32) return hipErrorInvalidValue;
        if ((EPI == EPI_RELU2 || EPI == EPI_RESID) && (a.N % 4 || a.ldo % 4)) return hipErrorInvalidValue;
        if ((a.A_lo && a.K % 64) || (a.out_lo && a.ldo % 64)) return hipErrorInvalidValue;  // lo8 layout
        if constexpr (EPI != EPI_STORE) {
            if (a.A_lo) {
                NC_TLAUNCH((gemm_bf16_comp_kernel<EPI>), grid, dim3(512), 0, st, a);
                return hipGetLastError();
            }
        }
        NC_TLAUNCH((gemm_bf16_kernel<EPI>), grid, dim3(512), 0, st, a);
    } else {
        if (a.A_lo || a.out_lo) return hipErrorInvalidValue;  // fp32 operands need no compensation
        NC_TLAUNCH((gemm_f32_kernel<EPI>), grid, dim3(256), 0, st, a);
    }
    return hipGetLastError();
}

// Largest |w| of a bf16 weight: grid-stride maximum, one atomic per wave on the float's bit
// pattern (non-negative floats order like their bit patterns).
__global__ __launch_bounds__(256) void absmax_kernel(const bf16* w, long long n, unsigned* out) {
    float m = 0.f;
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256)
        m = fmaxf(m, fabsf((float)w[i]));
    m = wave_max(m);
    if ((threadIdx.x & 63) == 0) atomicMax(out, __float_as_uint(m));
}

hipError_t launch_absmax(const void* w, long long n, unsigned* out, hipStream_t st) {
    if (n < 1) return hipSuccess;
    const long long blocks = std::min<long long>(1024, (n + 255) / 256);
    hipLaunchKernelGGL(absmax_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (const bf16*)w, n, out);
    return hipGetLastError();
}

int lo8_weight_exp(float absmax) {
    if (!(absmax > 0.f)) return 16;       // all zero (or NaN)
    if (!(absmax <= 3.0e38f)) return -16;  // infinite weights: the smallest scale
    const int s = (int)std::floor(std::log2(448.0 / (double)absmax));
    return std::max(-16, std::min(16, s));
}

int gemm_tile_n() { return TBN; }
int gemm_tile_k(DType dt) { return dt == BF16 ? 32 : KT<float>::BK; }

hipError_t launch_gemm(DType dt, Epi epi, const GemmArgs& a, hipStream_t st) {
    if (a.M < 1 || a.N < 1 || a.Npad < a.N || a.Npad % 32) return hipErrorInvalidValue;
    switch (epi) {
        case EPI_STORE: return launch_e<EPI_STORE>(dt, a, st);
        case EPI_RELU2: return launch_e<EPI_RELU2>(dt, a, st);
        case EPI_RESID: return launch_e<EPI_RESID>(dt, a, st);
        case EPI_SOFTCAP: return launch_e<EPI_SOFTCAP>(dt, a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace nc
