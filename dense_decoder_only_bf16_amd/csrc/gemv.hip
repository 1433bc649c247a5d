// Decode projections: C[M, N] = A[M, K] W[N, K]^T for the few rows of one decode step
// (M = batch <= 128), with the elementwise epilogues of the layer fused.
//
// In decode the weights are read once per step and dominate the traffic, so this kernel is
// built to stream W.  A workgroup owns 32 output columns and all M rows; its waves split K,
// and each wave loads its W and A operands straight from memory into registers (no LDS
// staging): the weights are stored MFMA-blocked, so one 16-deep step's W operand is a
// contiguous 1 KB block, and loads run two groups of steps ahead of the MFMAs.  The eight partial tiles are summed in LDS in a fixed order
// (deterministic, and no communication between workgroups, whose L2 caches are not
// coherent with each other), then each wave finishes whole rows:
//   STORE   raw fp32 product                              (QKV; finished by qkv_post)
//   RELU2   relu(r_m c)^2 -> dtype                        (MLP up-projection)
//   RESID   x += c, dtype copy of x, per-row sum of x^2 over the 32 columns
//   SOFTCAP cap tanh(r_m c / cap) -> fp32 logits          (LM head)
// with r_m = 1/sqrt(mean(x_m^2) + eps) the parameter-free RMSNorm folded into a row scale.
// Sources: yelogs.com launch write-up, architecture answer (norms without parameters,
// ReLU^2, no biases, untied head, logit softcap); apidog.com/th "How to train your own
// ChatGPT for $50", part 3 (weights cast to the activation dtype for a plain linear map).
#include "common.h"
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
        if (ok) p.out_f32[o] = p.cap * tanh_f32(v * r / p.cap);
    } else {  // EPI_RESID
        float xn = 0.f;
        if (ok) {
            xn = x_old + v;
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
template <typename T, int FM, int NW, int U, int EPI, bool LO>
__global__ __launch_bounds__(NW * 64) void dec_gemm_kernel(DecGemmArgs p) {
    typedef typename Chunk<T>::type CT;
    constexpr int BM = 32 * FM, BN = 32, TP = BN + 1;
    __shared__ float red[NW * BM * TP];

    if (p.lens_inc && blockIdx.x == 0 && blockIdx.y == 0)
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
    const int s0 = ksteps * wave / NW, s1 = ksteps * (wave + 1) / NW;
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
    __syncthreads();
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

// Launch shape.  `variant` picks alternative (waves, steps-in-flight) choices for tuning.
template <typename T, int EPI, bool LO>
static hipError_t dec_t(const DecGemmArgs& a, hipStream_t st, int variant) {
    const unsigned gx = (a.N + DEC_BN - 1) / DEC_BN;
    const int fm = a.M <= 32 ? 1 : (a.M <= 64 ? 2 : 4);
    const unsigned gy = (a.M + 32 * fm - 1) / (32 * fm);
    dim3 g(gx, gy);
#define NC_DG(FMV, NWV, UV) NC_TLAUNCH((dec_gemm_kernel<T, FMV, NWV, UV, EPI, LO>), g, dim3(NWV * 64), 0, st, a)
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

int dec_gemm_tile_n() { return DEC_BN; }

template <typename T>
static hipError_t dec_dt(Epi epi, const DecGemmArgs& a, hipStream_t st, int variant) {
    // compensated operands exist for the MLP products only (bf16 RELU2 and RESID)
    const bool lo = a.A_lo != nullptr;
    if (lo && (sizeof(T) != 2 || (epi != EPI_RELU2 && epi != EPI_RESID))) return hipErrorInvalidValue;
    switch (epi) {
        case EPI_STORE: return dec_t<T, EPI_STORE, false>(a, st, variant);
        case EPI_RELU2:
            return lo ? dec_t<T, EPI_RELU2, sizeof(T) == 2>(a, st, variant) : dec_t<T, EPI_RELU2, false>(a, st, variant);
        case EPI_RESID:
            return lo ? dec_t<T, EPI_RESID, sizeof(T) == 2>(a, st, variant) : dec_t<T, EPI_RESID, false>(a, st, variant);
        case EPI_SOFTCAP: return dec_t<T, EPI_SOFTCAP, false>(a, st, variant);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_dec_gemm(DType dt, Epi epi, const DecGemmArgs& a, hipStream_t st, int variant) {
    if (a.M < 1 || a.M > 128 || a.K % 16) return hipErrorInvalidValue;
    return dt == BF16 ? dec_dt<bf16>(epi, a, st, variant) : dec_dt<float>(epi, a, st, variant);
}

}  // namespace nc
