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
// the MLP products and the LM head the activation is therefore passed as two bf16 arrays,
// hi = bf16(a) and lo = bf16(a - hi), and multiplied as hi W^T + lo W^T with fp32
// accumulation, which leaves a relative operand error near 2^-17 (the weights are exact
// bf16 values).  The producing epilogue writes both parts.
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
//  * bf16 with a compensated operand (gemm_bf16_comp_kernel): 6 stages of one 16-deep step
//    holding A, A_lo and the weight block, so each weight block is loaded once.
//  * fp32 (the small fp32 check model): loads staged through registers into two LDS
//    buffers (A kept row-major with an XOR swizzle).
// Workgroups are dealt round-robin to the 8 dies (XCDs), each with its own L2; tiles are
// renumbered so each die works on a contiguous range, walked in groups of 8 row tiles so
// tiles running together share A rows and weight columns in the die's L2.
#include "common.h"
#include "kernels.h"

namespace nc {


template <typename T> struct KT {
    static constexpr int BK = 128 / (int)sizeof(T);  // elements per 128-byte row slice
    static constexpr int CPR = BK / 8;               // chunks per row slice
    static constexpr int KS = BK / 16;               // 16-deep MFMA steps per slice
};

constexpr int TBM = 256, TBN = 256;  // workgroup tile

// (m0, n0, tile column index) of this workgroup's tile.
__device__ __forceinline__ void tile_coords(const GemmArgs& p, int& m0, int& n0, int& tn) {
    constexpr int GM = 8;
    const int ntn = (p.N + TBN - 1) / TBN, ntm = (p.M + TBM - 1) / TBM;
    const int total = ntn * ntm;
    const int pid = blockIdx.x;
    const int xcd = pid % 8, loc = pid / 8, q8 = total / 8, r8 = total % 8;
    const int t = (xcd < r8) ? xcd * (q8 + 1) + loc : r8 * (q8 + 1) + (xcd - r8) * q8 + loc;
    const int grp = t / (GM * ntn), first_m = grp * GM;
    const int gsize = min(ntm - first_m, GM);
    const int tm = first_m + (t % (GM * ntn)) % gsize;
    tn = (t % (GM * ntn)) / gsize;
    n0 = tn * TBN;
    m0 = tm * TBM;
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
    int m0, n0, tn;
    tile_coords(p, m0, n0, tn);
    const int ksteps = p.K / 16;
    // A compensated product runs twice as many K tiles: tile 2k takes A's columns of tile
    // k, tile 2k + 1 the same columns of A_lo, both against the same weight block.
    const bool comp = p.A_lo != nullptr;
    const int nk = comp ? 2 * (p.K / BK) : p.K / BK;
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
        const int k0 = (comp ? kt >> 1 : kt) * BK;
        const bf16* As = (comp && (kt & 1)) ? A_lo : A;
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
    if (EPI == EPI_RELU2 || EPI == EPI_SOFTCAP) {
        if (tid < TBM) {
            float s = 0.f;
#pragma unroll
            for (int q = 0; q < MAXP; ++q) s += ssp[q];
            rs[tid] = 1.0f / sqrtf(s / (float)p.K + p.eps);
        }
        __syncthreads();
    }
    tile_epilogue<bf16, EPI, 2, 4>(p, acc, m0, n0, tn, rs, red);
}

// Compensated products (A + A_lo against one weight: the MLP products and the LM head).  A
// stage is one 16-deep step holding the tile's 8 A blocks, its 8 A_lo blocks and its 8
// weight blocks (24 KB; wave w loads block w of each), so a weight block is brought into
// LDS once for both MFMAs that use it: 24 KB of loads per 16 MFMAs of each wave, where
// running A_lo as extra K tiles of the kernel above loads 32 KB (the weight twice).  The
// loads into LDS, not the matrix cores, bound these products.  Six stages (144 KB), five
// in flight; a stage's 8 hi MFMAs come before its 8 lo MFMAs, so the two updates of an
// accumulator are 8 MFMAs apart, and the next stage's 10 fragment reads are interleaved
// with them.
template <int EPI>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_bf16_comp_kernel(GemmArgs p) {
    constexpr int NS = 6, BPS = 24;   // stages, 1 KB blocks per stage
    constexpr int STAGE = BPS * 512;  // elements per stage
    __shared__ __attribute__((aligned(1024))) bf16 lds[NS * STAGE];
    float* rs = (float*)lds;
    float (*red)[TBM] = (float (*)[TBM])((float*)lds + TBM);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / 4, wn = wave % 4;  // 2 x 4 waves, 128 x 64 each
    const int l32 = lane & 31, hh = lane >> 5;
    int m0, n0, tn;
    tile_coords(p, m0, n0, tn);
    const int nk = p.K / 16;  // stages

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

    // Wave w moves row block w of A and A_lo and weight block w; lane l takes memory chunk
    // 2 (l % 32) + l / 32 of a block into LDS chunk l (MFMA lane order, as above).  Row
    // blocks past A's last and weight blocks past Npad read a clamped block; their outputs
    // are masked in the epilogue.
    const int lchunk = 2 * l32 + hh;
    const int mb = min(m0 / 32 + wave, (p.M + 31) / 32 - 1);
    const int nb = min(n0 / 32 + wave, p.Npad / 32 - 1);
    const bf16* srcA = (const bf16*)p.A + (long long)mb * nk * 512 + lchunk * 8;
    const bf16* srcL = (const bf16*)p.A_lo + (long long)mb * nk * 512 + lchunk * 8;
    const bf16* srcB = (const bf16*)p.B + (long long)nb * nk * 512 + lchunk * 8;
    auto issue = [&](int kt) {
        bf16* s = lds + (kt % NS) * STAGE;
        __builtin_amdgcn_global_load_lds((gvoid*)(srcA + (long long)kt * 512), (lvoid*)(s + wave * 512), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((gvoid*)(srcL + (long long)kt * 512), (lvoid*)(s + (8 + wave) * 512), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((gvoid*)(srcB + (long long)kt * 512), (lvoid*)(s + (16 + wave) * 512), 16, 0, 0);
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = zero_vec<f32x16>();

    typedef bf16x8 Frag[10];  // A blocks 0..3, A_lo blocks 4..7, weight blocks 8..9
    auto fload = [&](int kt, Frag& f) {
        const bf16* s = lds + (kt % NS) * STAGE + lane * 8;
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = *(const bf16x8*)(s + (wm * 4 + i) * 512);
#pragma unroll
        for (int i = 0; i < 4; ++i) f[4 + i] = *(const bf16x8*)(s + (8 + wm * 4 + i) * 512);
#pragma unroll
        for (int j = 0; j < 2; ++j) f[8 + j] = *(const bf16x8*)(s + (16 + wn * 2 + j) * 512);
    };
    auto mfmas = [&](Frag& f, bool interleave) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[i][j] = mma32(f[i], f[8 + j], acc[i][j]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[i][j] = mma32(f[4 + i], f[8 + j], acc[i][j]);
        if (interleave) {
#pragma unroll
            for (int g = 0; g < 10; ++g) {
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
        }
    };
    // One stage: wait until this wave's loads of stage kt + 1 have landed (later stages,
    // at most 3, may stay in flight), barrier (every wave's loads of kt + 1 are in LDS and
    // every wave is done with stage kt - 1, whose slot the next issue refills), refill, then
    // the MFMAs of stage kt with the fragment reads of stage kt + 1.
    auto step = [&](int kt, Frag& cur, Frag& nxt) {
        const bool more = kt + 1 < nk;
        if (more) {
            const int ahead = min(NS - 3, nk - 2 - kt);
            if (ahead >= 3) NC_WAIT_VM(9);
            else if (ahead == 2) NC_WAIT_VM(6);
            else if (ahead == 1) NC_WAIT_VM(3);
            else NC_WAIT_VM(0);
            __builtin_amdgcn_s_barrier();
            if (kt + NS - 1 < nk) issue(kt + NS - 1);
            fload(kt + 1, nxt);
        }
        mfmas(cur, more);
    };

    // Prologue: stages 0 .. NS-2 in flight (3 loads per wave each), stage 0's fragments.
#pragma unroll
    for (int kt = 0; kt < NS - 1; ++kt)
        if (kt < nk) issue(kt);
    if (nk > 4) NC_WAIT_VM(12);
    else if (nk > 3) NC_WAIT_VM(9);
    else if (nk > 2) NC_WAIT_VM(6);
    else if (nk > 1) NC_WAIT_VM(3);
    else NC_WAIT_VM(0);
    __builtin_amdgcn_s_barrier();
    Frag f0, f1;
    fload(0, f0);
    for (int kt = 0; kt < nk; kt += 2) {
        step(kt, f0, f1);
        if (kt + 1 < nk) step(kt + 1, f1, f0);
    }
    __syncthreads();  // every wave is done with the ring (all its loads have landed)
    if (EPI == EPI_RELU2 || EPI == EPI_SOFTCAP) {
        if (tid < TBM) {
            float s = 0.f;
#pragma unroll
            for (int q = 0; q < MAXP; ++q) s += ssp[q];
            rs[tid] = 1.0f / sqrtf(s / (float)p.K + p.eps);
        }
        __syncthreads();
    }
    tile_epilogue<bf16, EPI, 2, 4>(p, acc, m0, n0, tn, rs, red);
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
    int m0, n0, tn;
    tile_coords(p, m0, n0, tn);
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

template <int EPI>
static hipError_t launch_e(DType dt, const GemmArgs& a, hipStream_t st) {
    dim3 grid(((a.N + TBN - 1) / TBN) * ((a.M + TBM - 1) / TBM), 1, a.k_split);
    if (dt == BF16) {
        if (a.k_split != 1 || a.K % 32) return hipErrorInvalidValue;
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
