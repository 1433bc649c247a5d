// Decode projections: C[M, N] = A[M, K] W[N, K]^T for the few rows of one decode step
// (M = batch <= 128), with the elementwise epilogues of the layer fused.
//
// In decode the weights are read once per step and dominate the traffic, so this kernel is
// built to stream W.  A workgroup owns 32 output columns and all M rows; its waves split K,
// and each wave loads its W and A operands straight from memory into registers (no LDS
// staging): the weights are stored MFMA-blocked, so one 16-deep step's W operand is a
// contiguous 1 KB block, and loads run two groups of steps ahead of the MFMAs.  The waves'
// partial tiles are summed in LDS in a fixed order (deterministic; a product with long K
// and few column tiles also splits K over workgroups, see dec_gemm_kernel), then each
// wave finishes whole rows:
//   STORE   raw fp32 product                              (QKV; finished by qkv_post)
//   RELU2   relu(r_m c)^2 -> dtype                        (MLP up-projection)
//   RESID   x += c, dtype copy of x, per-row sum of x^2 over the 32 columns
//   SOFTCAP cap tanh(r_m c / cap) -> fp32 logits          (LM head)
// with r_m = 1/sqrt(mean(x_m^2) + eps) the parameter-free RMSNorm folded into a row scale.
// Sources: yelogs.com launch write-up, architecture answer (norms without parameters,
// ReLU^2, no biases, untied head, logit softcap); apidog.com/th "How to train your own
// ChatGPT for $50", part 3 (weights cast to the activation dtype for a plain linear map).
#include <algorithm>

#include "common.h"
#include "finish.h"
#include "kernels.h"

namespace nc {

constexpr int DEC_BN = 32;  // output columns per workgroup (both tile shapes below)

// Finish one row of the tile: `v` is column n0 + lane of row m (lanes >= tile width hold 0),
// `r` the row's norm scale (RELU2, SOFTCAP), `x_old` the residual at (m, n0 + lane) (RESID).
template <typename T, int EPI>
__device__ __forceinline__ void dec_row_epilogue(const DecGemmArgs& p, int m, int n0, int width,
                                                 int lane, float v, float r, float x_old) {
    const int nn = n0 + lane;
    const bool ok = lane < width && nn < p.N;
    const long long o = (long long)m * p.ldo + nn;      // fp32 outputs, row-major
    const long long ob = blocked_index(m, ok ? nn : 0, p.N);  // dtype outputs, blocked
    if (EPI == EPI_STORE) {
        if (ok) p.out_f32[o] = v;
    } else if (EPI == EPI_RELU2) {
        const float t = fmaxf(v * r, 0.f);
        const T hi = from_f32<T>(t * t);
        if (ok) ((T*)p.out_t)[ob] = hi;
        if (ok && p.out_lo) ((T*)p.out_lo)[ob] = from_f32<T>(t * t - to_f32(hi));
    } else if (EPI == EPI_SOFTCAP) {
        if (ok) p.out_f32[o] = softcap_f32(v * r, p.cap, 1.0f / p.cap);
    } else {  // EPI_RESID
        float xn = 0.f;
        if (ok) {
            xn = resid_value(p.rx, o, x_old, v);
            p.out_f32[o] = xn;
            const T hi = from_f32<T>(xn);
            ((T*)p.out_t)[ob] = hi;
            if (p.out_lo) ((T*)p.out_lo)[ob] = from_f32<T>(xn - to_f32(hi));
        }
        const float sq = wave_sum(xn * xn);
        if (lane == 0) p.ss_out[(long long)blockIdx.x * p.ss_stride + m] = sq;
    }
}


// 32 x 32 MFMA tiles: FM row tiles (M <= 32 FM), 32 columns, NW waves splitting K.
// Each wave walks its K range in groups of U 16-deep steps with two register buffers: the
// loads of group g + 1 are issued before the MFMAs of group g, so 2U steps (2U KB of
// weights per wave for bf16) are in flight.  The weight operand of a step is one
// contiguous 32x16 block of the blocked layout.  LO: compensated operand (A + A_lo), one
// more MFMA per step against the same weight registers.
// K slices: with gridDim.z = KS > 1, workgroup z covers the z-th of KS equal ranges of K
// and stores its tile sum to `part`; the workgroup that finds itself the last of the tile
// to arrive (a counter per tile at the head of `part`, which it sets back to zero) adds the KS slices
// in slice order and runs the epilogue.  Every other workgroup only stores and leaves,
// so no workgroup ever waits on another.  The slice sums are stored and loaded with
// device-scope accesses (written through to, and read from, the level where the dies'
// caches are coherent), and each workgroup waits for its stores to complete before it
// counts itself, so no cache-wide write-back or invalidation is needed; such fences
// would flush the whole L2 of a die under the other workgroups' weight streams.
// FIN (QKV, one row block): the tile's raw rows are stored at device scope, and the last
// workgroup to store a tile of a head (an arrival counter per head slot, which it sets back
// to zero) finishes that head for every row (qkv_finish_head), one wave per row.
struct NoFinish {};
template <typename T, int FM, int NW, int U, int EPI, bool LO, bool FIN, typename FA>
__device__ __forceinline__ void dec_gemm_body(const DecGemmArgs& p, const FA& f) {
    typedef typename Chunk<T>::type CT;
    constexpr int BM = 32 * FM, BN = 32, TP = BN + 1;
    __shared__ float red[NW * BM * TP];
    __shared__ int last_in;

    if (p.lens_inc && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0)
        for (int r = threadIdx.x; r < p.M; r += NW * 64) p.lens_inc[r] += 1;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int l32 = lane & 31, hh = lane >> 5;
    const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
    const int rows = min(BM, p.M - m0);  // >= 1
    const int ksteps = p.K / 16;  // K is a multiple of 16 (checked on the host)

    // Wave w finishes rows w, w + NW, ... of the tile.  What their epilogue reads from
    // memory is loaded now, all rows at once, so the latency hides behind the weight
    // stream: RELU2 / SOFTCAP this lane's share of the row's partial sums of squares, RESID
    // the residual x at (row, n0 + lane).  Addresses are clamped into the tile; rows past
    // the tile are dropped below.
    constexpr int RPW = (BM + NW - 1) / NW;
    float pre[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) pre[i] = 0.f;
    if (EPI == EPI_RELU2 || EPI == EPI_SOFTCAP) {
        for (int q = lane; q < p.ss_in_parts; q += 64) {
#pragma unroll
            for (int i = 0; i < RPW; ++i) {
                const int ml = wave + NW * i;
                const float v = p.ss_in[(long long)q * p.ss_stride + m0 + min(ml, rows - 1)];
                pre[i] += ml < rows ? v : 0.f;
            }
        }
    } else if (EPI == EPI_RESID) {
        const int nn = min(n0 + (lane & 31), p.N - 1);
#pragma unroll
        for (int i = 0; i < RPW; ++i)
            pre[i] = p.out_f32[(long long)(m0 + min(wave + NW * i, rows - 1)) * p.ldo + nn];
    }
    const int KS = gridDim.z;
    const int z0 = (int)((long long)ksteps * blockIdx.z / KS), z1 = (int)((long long)ksteps * (blockIdx.z + 1) / KS);
    const int s0 = z0 + (z1 - z0) * wave / NW, s1 = z0 + (z1 - z0) * (wave + 1) / NW;
    const T* A = (const T*)p.A;
    const T* wb = (const T*)p.W + (long long)(n0 / 32) * ksteps * 512 + l32 * 16 + 8 * hh;
    // A is blocked like W: the operand of step s for row block i is 1 KB at
    // arow[i] + 512 s.  Lanes of rows past M read row 0 of the block (the same cache lines
    // as lane 0, so a short last block costs no extra traffic) and zero what they read.
    const T* arow[FM];
    const T* lrow[FM];
    bool mok[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        mok[i] = m0 + 32 * i + l32 < p.M;
        const int rb = min(m0 / 32 + i, (p.M - 1) / 32);  // row block (clamped into the buffer)
        const long long off = (long long)rb * ksteps * 512 + (mok[i] ? l32 : 0) * 16 + 8 * hh;
        arow[i] = A + off;
        lrow[i] = LO ? (const T*)p.A_lo + off : arow[i];
    }

    f32x16 acc[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) acc[i] = zero_vec<f32x16>();
    constexpr int NA = LO ? 2 : 1;  // activation parts
    CT wf0[U], wf1[U], af0[U][NA][FM], af1[U][NA][FM];
    // Loads are unconditional (addresses clamped into valid memory); rows past M are zeroed
    // with a bit mask and steps past the wave's range (a wave-uniform condition) with a
    // select, so no load sits behind a divergent branch.
    auto load = [&](CT (&wf)[U], CT (&af)[U][NA][FM], int sb) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int s = sb + u;
            const bool ok = s < s1;
            const int sc = ok ? s : s1 - 1;
            wf[u] = load_masked(wb + (long long)sc * 512, ok);
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                af[u][0][i] = load_masked(arow[i] + (long long)sc * 512, ok && mok[i]);
                if (LO) af[u][NA - 1][i] = load_masked(lrow[i] + (long long)sc * 512, ok && mok[i]);
            }
        }
    };
    auto mma = [&](CT (&wf)[U], CT (&af)[U][NA][FM]) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int h = 0; h < NA; ++h)
#pragma unroll
                for (int i = 0; i < FM; ++i) acc[i] = mma32(af[u][h][i], wf[u], acc[i]);
    };
    if (s1 > s0) load(wf0, af0, s0);
    for (int sb = s0; sb < s1; sb += 2 * U) {
        load(wf1, af1, sb + U);
        mma(wf0, af0);
        if (sb + U >= s1) break;
        load(wf0, af0, sb + 2 * U);
        mma(wf1, af1);
    }

    float* mine = red + wave * BM * TP;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            mine[(32 * i + 8 * (r / 4) + 4 * hh + (r % 4)) * TP + l32] = acc[i][r];
    __syncthreads();
    for (int e = tid; e < rows * BN; e += NW * 64) {
        const int r = e / BN, c = e % BN;
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) sum += red[w * BM * TP + r * TP + c];
        red[r * TP + c] = sum;
    }
    if (KS > 1) {
        const int tile = blockIdx.y * gridDim.x + blockIdx.x;  // < DEC_PART_CTRS (host check)
        int32_t* done = (int32_t*)p.part;
        float* pt = p.part + DEC_PART_CTRS + (long long)tile * KS * BM * BN;  // [tile][slice][BM][BN]
        for (int e = tid; e < rows * BN; e += NW * 64)
            store_device(pt + blockIdx.z * BM * BN + e, red[(e / BN) * TP + e % BN]);
        wait_stores_complete();  // this slice is visible device-wide before it is counted
        __syncthreads();
        if (tid == 0) {
            const int before = __hip_atomic_fetch_add(done + tile, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            last_in = before == KS - 1;
            if (before == KS - 1) __hip_atomic_store(done + tile, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        if (!last_in) return;  // workgroup-uniform
        for (int e = tid; e < rows * BN; e += NW * 64) {
            float sum = 0.f;
            for (int zb = 0; zb < KS; zb += 8) {  // 8 independent loads at a time
                float t[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) t[u] = load_device(pt + min(zb + u, KS - 1) * BM * BN + e);
#pragma unroll
                for (int u = 0; u < 8; ++u) sum += zb + u < KS ? t[u] : 0.f;
            }
            red[(e / BN) * TP + e % BN] = sum;
        }
    }
    __syncthreads();
    if constexpr (FIN) {
        const int nn = n0 + (lane & 31);
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int ml = wave + NW * i;
            if (ml < rows && lane < BN && nn < p.N)
                store_device(p.out_f32 + (long long)(m0 + ml) * p.ldo + nn, red[ml * TP + lane]);
        }
        wait_stores_complete();  // the tile is visible device-wide before it is counted
        __syncthreads();
        const int hd = f.hd, head = n0 / hd;
        if (tid == 0) {
            const int before = __hip_atomic_fetch_add(f.head_ctr + head, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            last_in = before == hd / BN - 1;
            if (before == hd / BN - 1) __hip_atomic_store(f.head_ctr + head, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        if (!last_in) return;  // workgroup-uniform
        const int half = hd / 2, ii = lane < half ? lane : 0;
        for (int b = wave; b < p.M; b += NW) {
            const float* src = p.out_f32 + (long long)b * p.ldo + head * hd;
            qkv_finish_head<T>(f, b, head, lane, load_device(src + ii), load_device(src + ii + half));
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int ml = wave + NW * i;
        if (ml < rows) {  // wave-uniform
            float r = 1.f;
            if (EPI == EPI_RELU2 || EPI == EPI_SOFTCAP) r = 1.0f / sqrtf(wave_sum(pre[i]) / (float)p.K + p.eps);
            dec_row_epilogue<T, EPI>(p, m0 + ml, n0, BN, lane, lane < BN ? red[ml * TP + lane] : 0.f, r, pre[i]);
        }
    }
}

template <typename T, int FM, int NW, int U, int EPI, bool LO>
__global__ __launch_bounds__(NW * 64) void dec_gemm_kernel(DecGemmArgs p) {
    dec_gemm_body<T, FM, NW, U, EPI, LO, false>(p, NoFinish{});
}
template <typename T, int NW, int U>
__global__ __launch_bounds__(NW * 64) void dec_gemm_fin_kernel(DecGemmArgs p, DecFinishArgs f) {
    dec_gemm_body<T, 1, NW, U, EPI_STORE, false, true>(p, f);
}

// LM head of a decode step with at most 32 rows (softcap epilogue).  One wave per 32-column
// tile over the whole K, 4 waves (4 independent tiles) per workgroup: the vocabulary's
// tiles then run as one round of independent waves, each streaming its weight column
// block with 2U steps of loads in flight, with no reduction across waves and no barrier.
// (With 8 waves splitting K per tile, the head ran as four rounds of whole workgroups,
// each round a full latency chain: d12, 8 rows, 1 ms more per 256 steps; U = 8 measured
// the same as U = 4.)
template <typename T, bool LO, int U>
__global__ __launch_bounds__(256) void dec_head_kernel(DecGemmArgs p) {
    typedef typename Chunk<T>::type CT;
    __shared__ float rsc[4][32];  // each wave's copy of the rows' norm scales
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, hh = lane >> 5;
    if (p.lens_inc && blockIdx.x == 0)
        for (int r = threadIdx.x; r < p.M; r += 256) p.lens_inc[r] += 1;
    const int n0 = (blockIdx.x * 4 + wave) * 32;
    if (n0 >= p.N) return;  // wave-uniform; no barrier follows
    const int ksteps = p.K / 16;

    // norm scale of row `lane` (< M): its partial sums of squares, loads issued together
    float s = 0.f;
    if (lane < p.M)
        for (int q = 0; q < p.ss_in_parts; ++q) s += p.ss_in[(long long)q * p.ss_stride + lane];
    if (lane < 32) rsc[wave][lane] = 1.0f / sqrtf(s / (float)p.K + p.eps);

    // A and W blocked; lanes of rows past M read row 0 of the block (its cache lines) and
    // zero what they read
    const bool mok = l32 < p.M;
    const long long aoff = (long long)(mok ? l32 : 0) * 16 + 8 * hh;
    const T* arow = (const T*)p.A + aoff;
    const T* lrow = LO ? (const T*)p.A_lo + aoff : arow;
    const T* wb = (const T*)p.W + (long long)(n0 / 32) * ksteps * 512 + l32 * 16 + 8 * hh;
    constexpr int NA = LO ? 2 : 1;
    f32x16 acc = zero_vec<f32x16>();
    CT wf0[U], wf1[U], af0[U][NA], af1[U][NA];
    auto load = [&](CT (&wf)[U], CT (&af)[U][NA], int sb) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int st = sb + u;
            const bool ok = st < ksteps;
            const int sc = ok ? st : ksteps - 1;
            wf[u] = load_masked(wb + (long long)sc * 512, ok);
            af[u][0] = load_masked(arow + (long long)sc * 512, ok && mok);
            if (LO) af[u][NA - 1] = load_masked(lrow + (long long)sc * 512, ok && mok);
        }
    };
    auto mma = [&](CT (&wf)[U], CT (&af)[U][NA]) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int h = 0; h < NA; ++h) acc = mma32(af[u][h], wf[u], acc);
    };
    load(wf0, af0, 0);
    for (int sb = 0; sb < ksteps; sb += 2 * U) {
        load(wf1, af1, sb + U);
        mma(wf0, af0);
        if (sb + U >= ksteps) break;
        load(wf0, af0, sb + 2 * U);
        mma(wf1, af1);
    }

    // lane holds column n0 + l32 of rows 8 (r / 4) + 4 hh + r % 4
    const int n = n0 + l32;
    const float inv_cap = 1.0f / p.cap;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int m = 8 * (r / 4) + 4 * hh + (r % 4);
        if (m < p.M && n < p.N)
            p.out_f32[(long long)m * p.ldo + n] = softcap_f32(acc[r] * rsc[wave][m], p.cap, inv_cap);
    }
}

// K slices of the one-row-block kernel: a product with long K and few column tiles (the
// MLP down-projection: d_model columns, K = d_ff) is split so that each workgroup takes
// 64 16-deep steps, 8 per wave, all of a wave's loads in flight at once (d12, 8 rows:
// 8.0 us against 10.3 us for 16 waves with 12 steps each in one workgroup per tile; 32
// or 16 steps per workgroup measured no faster).
static int dec_ksplit(int M, int N, int K) {
    if (M > 32 || K <= 1024 || N > 2048) return 1;
    return (K / 16 + 63) / 64;
}

// Launch shape.  `variant` picks alternative (waves, steps-in-flight) choices for tuning.
template <typename T, int EPI, bool LO>
static hipError_t dec_t(const DecGemmArgs& a, hipStream_t st, int variant, const DecFinishArgs* fin) {
    const unsigned gx = (a.N + DEC_BN - 1) / DEC_BN;
    const int fm = a.M <= 32 ? 1 : (a.M <= 64 ? 2 : 4);
    const unsigned gy = (a.M + 32 * fm - 1) / (32 * fm);
    const int ks = dec_ksplit(a.M, a.N, a.K);
    if (ks > 1 && (!a.part || (int)(gx * gy) > DEC_PART_CTRS)) return hipErrorInvalidValue;
    dim3 g(gx, gy, ks);
    if (EPI == EPI_SOFTCAP && fm == 1 && variant == 0) {
        NC_TLAUNCH((dec_head_kernel<T, LO, 4>), dim3((gx + 3) / 4), dim3(256), 0, st, a);
        return hipGetLastError();
    }
#define NC_DG(FMV, NWV, UV) NC_TLAUNCH((dec_gemm_kernel<T, FMV, NWV, UV, EPI, LO>), g, dim3(NWV * 64), 0, st, a)
    // one row block and at most 8 steps per wave (K <= 1024, or a K slice): all of a
    // wave's weight steps in flight at once (one memory round trip), except for the wide
    // LM head
    if (fm == 1 && variant == 0 && (ks > 1 || a.K <= 1024) && a.N <= 16384) variant = 2;
    if (fin) {  // QKV with its finish (EPI_STORE, one row block)
        if (variant == 2) NC_TLAUNCH((dec_gemm_fin_kernel<T, 8, 8>), g, dim3(512), 0, st, a, *fin);
        else NC_TLAUNCH((dec_gemm_fin_kernel<T, 8, 4>), g, dim3(512), 0, st, a, *fin);
        return hipGetLastError();
    }
    if (fm == 1) {
        if (variant == 1) NC_DG(1, 16, 4);
        else if (variant == 2) NC_DG(1, 8, 8);
        else if (variant == 3) NC_DG(1, 4, 16);
        else if (variant == 4) NC_DG(1, 4, 8);
        else NC_DG(1, 8, 4);
    } else if (fm == 2) {
        if (variant == 1) NC_DG(2, 16, 2);
        else if (variant == 2) NC_DG(2, 4, 8);
        else if (variant == 3) NC_DG(2, 4, 4);
        else if (variant == 4) NC_DG(2, 8, 2);
        else NC_DG(2, 8, 4);
    } else {
        if (variant == 1) NC_DG(4, 4, 4);
        else if (variant == 2) NC_DG(4, 8, 1);
        else if (variant == 3) NC_DG(4, 4, 2);
        else if (variant == 4) NC_DG(4, 2, 4);
        else NC_DG(4, 8, 2);
    }
#undef NC_DG
    return hipGetLastError();
}


// ------------------------------------------------------------ wide (32 < M <= 128) -------
// With up to 128 rows, a 32-column workgroup that reads all of A moves several times more
// activation bytes (out of L2) than weight bytes, and the L2s become the bound.  For bf16
// and M > 32 a workgroup therefore owns 256 or 128 columns (8 or 4 waves x one 32-column
// weight block) and one slice of K, and its waves share the activation operand through
// LDS: every stage of an LDS ring holds WKC 16-deep steps of the A blocks (both parts when
// compensated) and of the waves' weight blocks, all filled by direct-to-LDS 1 KB loads
// issued WNS - 1 stages ahead.  The ring is short (3 stages) so that two or three workgroups fit a CU:
// that measured 5-10% faster on the projections than one workgroup with a 6-stage ring,
// and 40% faster on the LM head, whose hundreds of tiles then run in one round.  The LM head (softcap; N = vocab gives hundreds of column tiles) runs its
// whole K in one workgroup and its epilogue here.  The other products split K into slices
// so that there are a few hundred workgroups; their fp32 partial products go to `part` and
// dec_reduce4_kernel (or, for the raw QKV product, the QKV finish) adds the slices in a
// fixed order and runs the epilogue.
// Waves per workgroup (one 32-column weight block each) for FM row tiles: 8 at up to 64
// rows, where the activation operand is small and sharing it over twice the columns halves
// its LDS fills per weight byte (d20, 64 rows: decode projections 9.57 -> 9.06 us per
// operation); 4 at more rows, where 8 waves measured slower (d30, 128 rows: 13.5 -> 14.3 us).
constexpr int wide_waves(int fm) { return fm <= 2 ? 8 : 4; }
// 16-deep steps per LDS stage: 2, or 4 where a 2-step stage's blocks would not split
// evenly over the waves (ablk: A blocks per step)
constexpr int wide_wkc(int ablk, int nw) { return (2 * (ablk + nw)) % nw == 0 ? 2 : 4; }
constexpr int WNS = 3;    // stages in the ring (two or three resident workgroups per CU)

struct WideShape {
    int tiles, splits, per;  // column tiles, K slices, 16-deep steps per slice
};
// Slices: a workgroup streams its A slice (the activation rows, both parts when
// compensated) and its W tile at a roughly fixed rate, and each slice leaves an fp32 partial
// product that is written and read back once more.  The slice count S minimises the
// estimate  (A / S + W / (tiles S)) / 50 GB/s  +  2 S M N 4 / 5 TB/s  over 2 <= S, each
// slice at least 2 stages long and every workgroup in one round of slots (256 CUs, one or
// two resident workgroups each by LDS size).  The LM head (softcap) is never split.
static WideShape wide_shape(Epi epi, int M, bool lo, int N, int K) {
    WideShape w;
    const int ksteps = K / 16;  // >= 4 (K >= 64)
    const int fm = M <= 64 ? 2 : 4, nw = wide_waves(fm);
    w.tiles = (N + 32 * nw - 1) / (32 * nw);
    if (epi == EPI_SOFTCAP) {
        w.splits = 1;
        w.per = ksteps;
        return w;
    }
    const int ablk = fm * (lo ? 2 : 1), WKC = wide_wkc(ablk, nw);
    const int stage_kb = WKC * (ablk + nw);
    const int slots = 256 * std::max(1, 160 / (WNS * stage_kb));
    const int smax = std::max(2, std::min(slots / w.tiles, ksteps / (2 * WKC)));
    const double a_bytes = (double)M * K * 2 * (lo ? 2 : 1), w_bytes = (double)N * K * 2;
    int best = 2;
    double best_t = 1e30;
    for (int s = 2; s <= smax; ++s) {
        const double t = (a_bytes / s + w_bytes / ((double)w.tiles * s)) / 50e9 + 2.0 * s * M * N * 4 / 5e12;
        if (t < best_t) {
            best_t = t;
            best = s;
        }
    }
    w.per = (ksteps + best - 1) / best;
    w.splits = (ksteps + w.per - 1) / w.per;  // every slice non-empty, >= 2
    return w;
}

template <int FM, bool LO, int EPI>
__global__ __launch_bounds__(64 * wide_waves(FM)) void dec_gemm_wide_kernel(DecGemmArgs p, int splits, int per) {
    constexpr int WNW = wide_waves(FM), WBN = 32 * WNW;
    constexpr int NA = LO ? 2 : 1;
    constexpr int ABLK = FM * NA;          // A blocks per 16-deep step
    constexpr int WKC = wide_wkc(ABLK, WNW);
    constexpr int BPS = WKC * (ABLK + WNW);  // 1 KB blocks per stage: A blocks, then W blocks
    constexpr int BPW = BPS / WNW;           // blocks each wave loads per stage
    static_assert(BPS % WNW == 0, "stage must split evenly over the waves");
    static_assert((WNS - 2) * BPW <= 63, "vmcnt range");
    constexpr int STAGE = BPS * 512;       // bf16 elements per stage
    // one LDS object (the ring, then the LM head's row scales): with a second one the
    // compiler cannot tell its reads from the ring's in-flight loads and waits for them all
    __shared__ __attribute__((aligned(1024))) bf16 lds[WNS * STAGE + 64 * FM];
    float* const rs = (float*)(lds + WNS * STAGE);  // 32 FM row scales

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hh = lane >> 5;
    const int n0 = blockIdx.x * WBN;
    const int ksteps = p.K / 16;
    const int s0 = blockIdx.y * per, s1 = min(ksteps, s0 + per);  // s0 < s1 (host)
    const int nstg = (s1 - s0 + WKC - 1) / WKC;
    const int nblk_w = (p.N + 31) / 32;
    const int mblk = (p.M + 31) / 32;
    const bf16* A = (const bf16*)p.A;
    const bf16* AL = LO ? (const bf16*)p.A_lo : A;
    const bf16* W = (const bf16*)p.W;
    (void)splits;
    if (p.lens_inc && blockIdx.x == 0 && blockIdx.y == 0)  // end of a decode step
        for (int r = tid; r < p.M; r += 64 * WNW) p.lens_inc[r] += 1;

    if (EPI == EPI_SOFTCAP) {  // row scales of the final norm: wave w does rows w + WNW j,
        // lanes over the partial sums, every load of every row issued before any sum
        constexpr int RW = 32 * FM / WNW;
        float s[RW];
#pragma unroll
        for (int j = 0; j < RW; ++j) s[j] = 0.f;
        for (int q = lane; q < p.ss_in_parts; q += 64)
#pragma unroll
            for (int j = 0; j < RW; ++j) s[j] += p.ss_in[(long long)q * p.ss_stride + min(wave + WNW * j, p.M - 1)];
#pragma unroll
        for (int j = 0; j < RW; ++j) {
            const float t = wave_sum(s[j]);
            if (lane == 0) rs[wave + WNW * j] = 1.0f / sqrtf(t / (float)p.K + p.eps);
        }
        __syncthreads();
    }

    // Stage t: block q < WKC ABLK is A (step q / ABLK, row block (q % ABLK) / NA, part
    // q % NA); the rest are W (step (q - WKC ABLK) / WNW, column block of wave
    // (q - WKC ABLK) % WNW).  Steps past the slice and blocks past the matrices load clamped
    // addresses whose data is never used.
    auto issue = [&](int t) {
        bf16* sb = lds + (t % WNS) * STAGE;
#pragma unroll
        for (int u = 0; u < BPW; ++u) {
            const int q = u * WNW + wave;
            const bf16* src;
            if (q < WKC * ABLK) {
                const int kc = q / ABLK, r = q % ABLK;
                const int step = min(s0 + t * WKC + kc, s1 - 1);
                const int rb = min(r / NA, mblk - 1);
                src = ((r % NA) ? AL : A) + ((long long)rb * ksteps + step) * 512 + lane * 8;
            } else {
                const int q2 = q - WKC * ABLK;
                const int step = min(s0 + t * WKC + q2 / WNW, s1 - 1);
                const int nb = min(n0 / 32 + q2 % WNW, nblk_w - 1);
                src = W + ((long long)nb * ksteps + step) * 512 + lane * 8;
            }
            __builtin_amdgcn_global_load_lds((gvoid*)src, (lvoid*)(sb + q * 512), 16, 0, 0);
        }
    };

    f32x16 acc[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) acc[i] = zero_vec<f32x16>();
#pragma unroll
    for (int t = 0; t < WNS - 1; ++t) issue(t);
    for (int t = 0; t < nstg; ++t) {
        NC_WAIT_VM((WNS - 2) * BPW);  // this wave's share of stage t is in LDS
        __builtin_amdgcn_s_barrier(); // everyone's share is; everyone is done with stage t-1
        issue(t + WNS - 1);           // refills the slot of stage t-1
        const bf16* sb = lds + (t % WNS) * STAGE;
#pragma unroll
        for (int kc = 0; kc < WKC; ++kc) {
            if (s0 + t * WKC + kc < s1) {
                const bf16x8 wf = *(const bf16x8*)(sb + (WKC * ABLK + kc * WNW + wave) * 512 + l32 * 16 + 8 * hh);
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int h = 0; h < NA; ++h) {
                        const bf16x8 af = *(const bf16x8*)(sb + (kc * ABLK + i * NA + h) * 512 + l32 * 16 + 8 * hh);
                        acc[i] = mma32(af, wf, acc[i]);
                    }
            }
        }
    }
    NC_WAIT_VM_ALL();  // the ring's trailing loads land before the workgroup's LDS is released

    // lane holds column n = n0 + 32 wave + l32 and rows 32 i + 8 (r / 4) + 4 hh + r % 4
    const int nb = n0 / 32 + wave;
    const int n = nb * 32 + l32;
    const bool nok = n < p.N;
    if constexpr (EPI != EPI_SOFTCAP) {  // split K: this slice's partial product
        float* dst = p.part + (long long)blockIdx.y * p.M * p.N;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = 32 * i + 8 * (r / 4) + 4 * hh + (r % 4);
                if (m < p.M && nok) dst[(long long)m * p.N + n] = acc[i][r];
            }
    } else {  // whole K: logits = cap tanh(r_m c / cap)
        const float inv_cap = 1.0f / p.cap;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = 32 * i + 8 * (r / 4) + 4 * hh + (r % 4);
                if (m < p.M && nok) p.out_f32[(long long)m * p.ldo + n] = softcap_f32(acc[i][r] * rs[m], p.cap, inv_cap);
            }
    }
}

// Split-K finish of the wide products, four columns per lane: workgroup (256 columns,
// 4 rows), wave w finishes row 4 blockIdx.y + w.  Each lane adds its 4 columns' slices in
// slice order with 16-byte loads (8 slices per batch of independent loads), then runs the
// row epilogue on them (N is a multiple of 4):
//   RELU2  relu(r_m c)^2 -> bf16 hi / lo (blocked)
//   RESID  x += c, bf16 hi / lo copies of x (blocked), per-row sums of x^2 over each 32
//          columns (the same partial sums the other decode kernels leave)
template <int EPI>
__global__ __launch_bounds__(256) void dec_reduce4_kernel(DecGemmArgs p, int splits) {
    const int lane = threadIdx.x & 63;
    const int m = blockIdx.y * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (m >= p.M) return;  // wave-uniform; no workgroup barrier below
    const int n = blockIdx.x * 256 + 4 * lane;
    const bool ok = n < p.N;
    const int nc = ok ? n : 0;
    const long long slice = (long long)p.M * p.N;
    const float* src = p.part + (long long)m * p.N + nc;
    f32x4 x_old = zero_vec<f32x4>();
    if (EPI == EPI_RESID) x_old = *(const f32x4*)(p.out_f32 + (long long)m * p.ldo + nc);
    float pre = 0.f;
    if (EPI == EPI_RELU2)
        for (int q = lane; q < p.ss_in_parts; q += 64) pre += p.ss_in[(long long)q * p.ss_stride + m];
    f32x4 v = zero_vec<f32x4>();
    for (int s0 = 0; s0 < splits; s0 += 8) {
        f32x4 t[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) t[u] = *(const f32x4*)(src + min(s0 + u, splits - 1) * slice);
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (s0 + u < splits) v += t[u];
    }
    const long long ob = blocked_index(m, nc, p.N);  // 4 consecutive bf16 (n % 4 == 0)
    if (EPI == EPI_RELU2) {
        const float r = 1.0f / sqrtf(wave_sum(pre) / (float)p.K + p.eps);
        bf16x4 hi, lo;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float t = fmaxf(v[e] * r, 0.f);
            hi[e] = (bf16)(t * t);
            lo[e] = (bf16)(t * t - (float)hi[e]);
        }
        if (ok) {
            *(bf16x4*)((bf16*)p.out_t + ob) = hi;
            if (p.out_lo) *(bf16x4*)((bf16*)p.out_lo + ob) = lo;
        }
    } else {  // EPI_RESID
        const long long o = (long long)m * p.ldo + nc;
        f32x4 xn;
        float sq = 0.f;
        bf16x4 hi, lo;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            xn[e] = ok ? resid_value(p.rx, o + e, x_old[e], v[e]) : 0.f;
            hi[e] = (bf16)xn[e];
            lo[e] = (bf16)(xn[e] - (float)hi[e]);
            sq += xn[e] * xn[e];
        }
        if (ok) {
            *(f32x4*)(p.out_f32 + o) = xn;
            *(bf16x4*)((bf16*)p.out_t + ob) = hi;
            if (p.out_lo) *(bf16x4*)((bf16*)p.out_lo + ob) = lo;
        }
        sq += __shfl_xor(sq, 1, 64);  // the 8 lanes of a 32-column tile
        sq += __shfl_xor(sq, 2, 64);
        sq += __shfl_xor(sq, 4, 64);
        if ((lane & 7) == 0 && ok) p.ss_out[(long long)(n / 32) * p.ss_stride + m] = sq;
    }
}

template <int EPI, bool LO>
static hipError_t wide_t(const DecGemmArgs& args, hipStream_t st) {
    const WideShape w = wide_shape((Epi)EPI, args.M, LO, args.N, args.K);
    if (w.splits > 1 && !args.part) return hipErrorInvalidValue;
    DecGemmArgs a = args;
    if (a.part) a.part += DEC_PART_CTRS;  // the partials follow the counters
    dim3 g(w.tiles, w.splits);
    if (a.M <= 64) NC_TLAUNCH((dec_gemm_wide_kernel<2, LO, EPI>), g, dim3(64 * wide_waves(2)), 0, st, a, w.splits, w.per);
    else NC_TLAUNCH((dec_gemm_wide_kernel<4, LO, EPI>), g, dim3(64 * wide_waves(4)), 0, st, a, w.splits, w.per);
    // the raw QKV product's slices are added by the QKV finish (dec_gemm_store_slices)
    if ((EPI == EPI_RELU2 || EPI == EPI_RESID) && w.splits > 1) {
        if (a.N % 4) return hipErrorInvalidValue;
        NC_TLAUNCH((dec_reduce4_kernel<EPI == EPI_RELU2 ? EPI_RELU2 : EPI_RESID>), dim3((a.N + 255) / 256, (a.M + 3) / 4),
                   dim3(256), 0, st, a, w.splits);
    }
    return hipGetLastError();
}

int dec_gemm_store_slices(DType dt, int M, int N, int K) {
    if (dt != BF16 || M <= 32) return 0;
    return wide_shape(EPI_STORE, M, false, N, K).splits;
}

long long dec_gemm_part_elems(DType dt, Epi epi, int M, int N, int K) {
    if (M <= 32) {
        const int ks = dec_ksplit(M, N, K);
        return ks > 1 ? DEC_PART_CTRS + (long long)ks * ((N + DEC_BN - 1) / DEC_BN) * 32 * DEC_BN : 0;
    }
    if (dt != BF16) return 0;
    const bool lo = epi != EPI_STORE;  // compensated operands: MLP products and LM head
    const WideShape w = std::max(wide_shape(epi, M, lo, N, K), wide_shape(epi, M, false, N, K),
                                 [](const WideShape& x, const WideShape& y) { return x.splits < y.splits; });
    return w.splits > 1 ? DEC_PART_CTRS + (long long)w.splits * M * N : 0;
}

int dec_gemm_tile_n() { return DEC_BN; }

bool dec_gemm_fuses_finish(DType dt, int M, int hd, int slots) {
    (void)dt;
    return M <= 32 && hd % DEC_BN == 0 && slots <= DEC_FIN_SLOTS;
}

template <typename T>
static hipError_t dec_dt(Epi epi, const DecGemmArgs& a, hipStream_t st, int variant, const DecFinishArgs* fin) {
    // compensated operands exist for the MLP products and the LM head (bf16 only)
    const bool lo = a.A_lo != nullptr;
    if (lo && (sizeof(T) != 2 || epi == EPI_STORE)) return hipErrorInvalidValue;
    if (fin) {
        if (epi != EPI_STORE || !fin->head_ctr || fin->B != a.M || a.N != (fin->H + 2 * fin->nkv) * fin->hd ||
            a.ldo != a.N || !dec_gemm_fuses_finish(sizeof(T) == 2 ? BF16 : F32, a.M, fin->hd, fin->H + 2 * fin->nkv))
            return hipErrorInvalidValue;
        return dec_t<T, EPI_STORE, false>(a, st, variant, fin);
    }
    if (sizeof(T) == 2 && a.M > 32) {
        switch (epi) {
            case EPI_STORE: return wide_t<EPI_STORE, false>(a, st);
            case EPI_RELU2: return lo ? wide_t<EPI_RELU2, true>(a, st) : wide_t<EPI_RELU2, false>(a, st);
            case EPI_RESID: return lo ? wide_t<EPI_RESID, true>(a, st) : wide_t<EPI_RESID, false>(a, st);
            case EPI_SOFTCAP: return lo ? wide_t<EPI_SOFTCAP, true>(a, st) : wide_t<EPI_SOFTCAP, false>(a, st);
            default: return hipErrorInvalidValue;
        }
    }
    switch (epi) {
        case EPI_STORE: return dec_t<T, EPI_STORE, false>(a, st, variant, nullptr);
        case EPI_RELU2:
            return lo ? dec_t<T, EPI_RELU2, sizeof(T) == 2>(a, st, variant, nullptr)
                      : dec_t<T, EPI_RELU2, false>(a, st, variant, nullptr);
        case EPI_RESID:
            return lo ? dec_t<T, EPI_RESID, sizeof(T) == 2>(a, st, variant, nullptr)
                      : dec_t<T, EPI_RESID, false>(a, st, variant, nullptr);
        case EPI_SOFTCAP:
            return lo ? dec_t<T, EPI_SOFTCAP, sizeof(T) == 2>(a, st, variant, nullptr)
                      : dec_t<T, EPI_SOFTCAP, false>(a, st, variant, nullptr);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_dec_gemm(DType dt, Epi epi, const DecGemmArgs& a, hipStream_t st, int variant,
                           const DecFinishArgs* fin) {
    if (a.M < 1 || a.M > 128 || a.K % 16) return hipErrorInvalidValue;
    return dt == BF16 ? dec_dt<bf16>(epi, a, st, variant, fin) : dec_dt<float>(epi, a, st, variant, fin);
}

}  // namespace nc
