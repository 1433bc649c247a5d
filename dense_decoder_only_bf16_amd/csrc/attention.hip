// Causal multi-query attention for gfx950: a flash-style prefill kernel and a split-context
// decode kernel with a combine kernel.
//
// Multi-query attention: one K/V head serves every query head (yelogs.com launch write-up,
// architecture answer).  Causal softmax of q.k/sqrt(hd) over keys at positions <= the
// query's; the pages run these through FlashAttention-3 (`flash_attn_func` with
// causal=True for training/prefill, `flash_attn_with_kvcache` for decode -- apidog.com/th
// "How to train your own ChatGPT for $50", parts 5 and 6).  Here both are written for
// wave64 MFMA tiles.
//
// Layout trick shared by both kernels: scores are produced transposed, S^T = K Q^T, so that
// in the MFMA output each lane owns one query (column) and a run of keys (rows).  The
// softmax statistics of a query then live in one lane (plus its partner half-wave), and
// the probabilities already sit in the B-operand layout of O^T = V^T P^T once the keys of a
// 16/32-deep contraction step are taken in the order the output layout holds them.  V is
// kept transposed in the cache ([hd][positions]) so that the A operand of O^T (8 keys of
// one feature) is two short contiguous reads.
#include "common.h"
#include "kernels.h"

namespace nc {

// ------------------------------------------------------------------ prefill ---------
// Workgroup: 4 waves, 256 query positions of one (row, head); wave w owns 64 queries as two
// 32-column MFMA tiles.  K/V advance in blocks of 64 keys staged in LDS; blocks past the
// last query of the workgroup are never loaded, and a wave whose queries all precede a
// block skips its MFMAs.
template <typename T, int HD>
__global__ __launch_bounds__(256) void attn_prefill_kernel(const T* __restrict__ q,
                                                           const T* __restrict__ kc,
                                                           const T* __restrict__ vtc,
                                                           T* __restrict__ y, int Tn, int H,
                                                           int S, float scale_log2) {
    typedef typename Chunk<T>::type CT;
    typedef typename Chunk<T>::half HT;
    constexpr int BQ = 256, KB = 64;
    constexpr int CPRK = HD / 8;      // chunks per K row
    constexpr int KSTEPS = HD / 16;   // 16-deep steps over the head dim
    constexpr int MD = HD / 32;       // 32-row tiles of O^T

    __shared__ __attribute__((aligned(32))) T Ks[KB * HD];
    __shared__ __attribute__((aligned(32))) T Vs[HD * KB];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const int qb = gridDim.x - 1 - blockIdx.x;  // longest (latest) query blocks first
    const int head = blockIdx.y, b = blockIdx.z;
    const int q0 = qb * BQ;
    const int q0w = q0 + wave * 64;

    const T* kb_base = kc + (long long)b * S * HD;
    const T* vb_base = vtc + (long long)b * HD * S;

    // Query operands: B operand of S^T, lane holds query (q0w + jn*32 + l32), dims 16s+8hh..
    CT qf[2][KSTEPS];
#pragma unroll
    for (int jn = 0; jn < 2; ++jn) {
        const int qi = q0w + jn * 32 + l32;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
            if (qi < Tn)
                qf[jn][s] = *(const CT*)(q + (((long long)b * Tn + qi) * H + head) * HD + 16 * s + 8 * hh);
            else
                qf[jn][s] = zero_vec<CT>();
        }
    }

    f32x16 oacc[MD][2];
#pragma unroll
    for (int i = 0; i < MD; ++i) {
        oacc[i][0] = zero_vec<f32x16>();
        oacc[i][1] = zero_vec<f32x16>();
    }
    float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};

    const int kend = min(Tn, q0 + BQ);
    const int nkb = (kend + KB - 1) / KB;
    constexpr int KCH = KB * CPRK / 256;  // K chunks per thread
    constexpr int VCH = HD * (KB / 8) / 256;
    static_assert(KCH >= 1 && VCH >= 1, "block too small for 256 threads");

    for (int kbi = 0; kbi < nkb; ++kbi) {
        const int k0 = kbi * KB;
        CT rk[KCH], rv[VCH];
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            int c = tid + i * 256, key = c / CPRK, ch = c % CPRK;
            rk[i] = (k0 + key < Tn) ? *(const CT*)(kb_base + (long long)(k0 + key) * HD + ch * 8) : zero_vec<CT>();
        }
#pragma unroll
        for (int i = 0; i < VCH; ++i) {
            int c = tid + i * 256, d = c / (KB / 8), ch = c % (KB / 8);
            const T* src = vb_base + (long long)d * S + k0 + ch * 8;
            if (k0 + ch * 8 + 8 <= Tn) {
                rv[i] = *(const CT*)src;
            } else {
                CT t = zero_vec<CT>();
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (k0 + ch * 8 + e < Tn) t[e] = src[e];
                rv[i] = t;
            }
        }
        __syncthreads();  // previous block's LDS reads are complete
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            int c = tid + i * 256, key = c / CPRK, ch = c % CPRK;
            *(CT*)(&Ks[key * HD + ((ch ^ (key & 7)) * 8)]) = rk[i];
        }
#pragma unroll
        for (int i = 0; i < VCH; ++i) {
            int c = tid + i * 256, d = c / (KB / 8), ch = c % (KB / 8);
            *(CT*)(&Vs[d * KB + ((ch ^ (d & 7)) * 8)]) = rv[i];
        }
        __syncthreads();

        if (k0 > q0w + 63) continue;  // every query of this wave precedes the block

        f32x16 sacc[2][2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            sacc[mt][0] = zero_vec<f32x16>();
            sacc[mt][1] = zero_vec<f32x16>();
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s) {
                const int key = mt * 32 + l32, ch = 2 * s + hh;
                CT kf = *(const CT*)(&Ks[key * HD + ((ch ^ (key & 7)) * 8)]);
                sacc[mt][0] = mma32(kf, qf[0][s], sacc[mt][0]);
                sacc[mt][1] = mma32(kf, qf[1][s], sacc[mt][1]);
            }
        }

        // Online softmax (base 2).  Row index of register r in a 32x32 output tile:
        // 8*(r/4) + 4*hh + (r%4).
#pragma unroll
        for (int jn = 0; jn < 2; ++jn) {
            const int qi = q0w + jn * 32 + l32;
            float mx = -INFINITY;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + mt * 32 + 8 * (r / 4) + 4 * hh + (r % 4);
                    float v = sacc[mt][jn][r] * scale_log2;
                    v = (key <= qi && key < Tn) ? v : -INFINITY;
                    sacc[mt][jn][r] = v;
                    mx = fmaxf(mx, v);
                }
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            const float m_new = fmaxf(m_run[jn], mx);
            const float alpha = fast_exp2(m_run[jn] - m_new);
            float ls = 0.f;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float pv = fast_exp2(sacc[mt][jn][r] - m_new);
                    sacc[mt][jn][r] = pv;
                    ls += pv;
                }
            ls += __shfl_xor(ls, 32, 64);
            l_run[jn] = l_run[jn] * alpha + ls;
            m_run[jn] = m_new;
#pragma unroll
            for (int md = 0; md < MD; ++md) oacc[md][jn] *= alpha;
        }

        // O^T += V^T P^T over the block's 64 keys in four 16-deep steps.
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int mt = t / 2, rb = 8 * (t % 2);
            CT pf[2];
#pragma unroll
            for (int jn = 0; jn < 2; ++jn)
#pragma unroll
                for (int i = 0; i < 8; ++i) pf[jn][i] = from_f32<T>(sacc[mt][jn][rb + i]);
#pragma unroll
            for (int md = 0; md < MD; ++md) {
                const int d = md * 32 + l32;
                const int u1 = 4 * t + hh, u2 = 4 * t + 2 + hh;  // 4-key units of this lane
                const int sw = 2 * (d & 7);
                HT lo = *(const HT*)(&Vs[d * KB + ((u1 ^ sw) * 4)]);
                HT hi = *(const HT*)(&Vs[d * KB + ((u2 ^ sw) * 4)]);
                CT vf;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    vf[i] = lo[i];
                    vf[4 + i] = hi[i];
                }
                oacc[md][0] = mma32(vf, pf[0], oacc[md][0]);
                oacc[md][1] = mma32(vf, pf[1], oacc[md][1]);
            }
        }
    }

    // Normalise and store: lane holds query (l32 + 32 jn), features 32md + 8(r/4) + 4hh + 0..3.
#pragma unroll
    for (int jn = 0; jn < 2; ++jn) {
        const int qi = q0w + jn * 32 + l32;
        if (qi >= Tn) continue;
        const float inv = 1.0f / l_run[jn];
        T* dst = y + (((long long)b * Tn + qi) * H + head) * HD;
#pragma unroll
        for (int md = 0; md < MD; ++md)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                HT o;
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = from_f32<T>(oacc[md][jn][4 * g + e] * inv);
                *(HT*)(dst + md * 32 + 8 * g + 4 * hh) = o;
            }
    }
}

hipError_t launch_attn_prefill(DType dt, int hd, const void* q, const void* kc, const void* vtc,
                               void* y, int B, int T, int H, int S, hipStream_t st) {
    dim3 grid((T + 255) / 256, H, B);
    const float sl = 1.4426950408889634f / sqrtf((float)hd);
#define NC_AP(TT, HDV)                                                                        \
    hipLaunchKernelGGL((attn_prefill_kernel<TT, HDV>), grid, dim3(256), 0, st, (const TT*)q, \
                       (const TT*)kc, (const TT*)vtc, (TT*)y, T, H, S, sl)
    if (dt == BF16 && hd == 128) NC_AP(bf16, 128);
    else if (dt == BF16 && hd == 64) NC_AP(bf16, 64);
    else if (dt == F32 && hd == 128) NC_AP(float, 128);
    else if (dt == F32 && hd == 64) NC_AP(float, 64);
    else return hipErrorInvalidValue;
#undef NC_AP
    return hipGetLastError();
}

// ------------------------------------------------------------------ decode ----------
// Split kernel.  Workgroup (chunk c, row b): 4 waves x 64 keys = keys [256c, 256c + 256)
// limited to positions 0..lens[b].  All query heads of the row (padded to 16) form the 16
// columns of 16x16 MFMA tiles, so each K/V element is read from memory once for the whole
// head group.  Every wave issues all of its K and V^T loads (straight from the cache into
// registers) before any arithmetic, so a wave keeps 32 KB in flight.  The four waves'
// softmax states are merged in LDS and the workgroup writes its chunk's partial
// (max, sum, o[16][hd]); the combine kernel merges the chunks of each row.
constexpr int DEC_KPW = 64, DEC_CHUNK = 4 * DEC_KPW;
int attn_decode_chunk() { return DEC_CHUNK; }

template <typename T, int HD>
__global__ __launch_bounds__(256) void attn_decode_split_kernel(
    const T* __restrict__ q, const T* __restrict__ kc, const T* __restrict__ vtc,
    const int32_t* __restrict__ lens, float* __restrict__ part, int H, int S, int max_chunks,
    float scale_log2) {
    typedef typename Chunk<T>::type CT;
    typedef typename Chunk<T>::half HT;
    constexpr int DS = HD / 32;   // 32-deep steps over head dim for S^T
    constexpr int DT = HD / 16;   // 16-row tiles of O^T
    constexpr int PSZ = 16 * (HD + 2);

    __shared__ float sm[4][16], sl[4][16];
    __shared__ float so[4][16][HD + 1];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, g = lane >> 4;
    const int c = blockIdx.x, b = blockIdx.y;
    const int pos = lens[b];  // keys 0..pos are visible
    const int nkeys = min(pos + 1, S);
    const int nchunks = (nkeys + DEC_CHUNK - 1) / DEC_CHUNK;
    if (c >= nchunks) return;
    const int kbeg = c * DEC_CHUNK + wave * DEC_KPW;

    const T* kb_base = kc + (long long)b * S * HD;
    const T* vb_base = vtc + (long long)b * HD * S;

    // ---- issue every load of this wave
    CT qf[DS];
#pragma unroll
    for (int s = 0; s < DS; ++s)
        qf[s] = (col < H) ? *(const CT*)(q + ((long long)b * H + col) * HD + 32 * s + 8 * g) : zero_vec<CT>();
    CT kf[4][DS];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
        const int key = kbeg + 16 * kt + col;
#pragma unroll
        for (int s = 0; s < DS; ++s)
            kf[kt][s] = (key < nkeys) ? *(const CT*)(kb_base + (long long)key * HD + 32 * s + 8 * g) : zero_vec<CT>();
    }
    // V^T operands: slot 8g+i of 32-key step u <-> key 32u + 4g + i (i < 4) or
    // 32u + 16 + 4g + (i - 4) (i >= 4); loaded whole when in range, else element-wise.
    HT vlo[2][DT], vhi[2][DT];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int ka = kbeg + 32 * u + 4 * g, kb2 = ka + 16;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const T* src = vb_base + (long long)(dt * 16 + col) * S;
            if (ka + 4 <= nkeys) vlo[u][dt] = *(const HT*)(src + ka);
            else
#pragma unroll
                for (int e = 0; e < 4; ++e) vlo[u][dt][e] = (ka + e < nkeys) ? src[ka + e] : from_f32<T>(0.f);
            if (kb2 + 4 <= nkeys) vhi[u][dt] = *(const HT*)(src + kb2);
            else
#pragma unroll
                for (int e = 0; e < 4; ++e) vhi[u][dt][e] = (kb2 + e < nkeys) ? src[kb2 + e] : from_f32<T>(0.f);
        }
    }

    // ---- scores S^T (lane: head `col`, keys kbeg + 16kt + 4g + j), softmax (base 2)
    f32x4 sacc[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
        sacc[kt] = zero_vec<f32x4>();
#pragma unroll
        for (int s = 0; s < DS; ++s) sacc[kt] = mma16(kf[kt][s], qf[s], sacc[kt]);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int key = kbeg + 16 * kt + 4 * g + j;
            float v = (key < nkeys) ? sacc[kt][j] * scale_log2 : -INFINITY;
            sacc[kt][j] = v;
            mx = fmaxf(mx, v);
        }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mref = (mx == -INFINITY) ? 0.f : mx;  // a wave past the last key has no mass
    float ls = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float pv = fast_exp2(sacc[kt][j] - mref);
            sacc[kt][j] = pv;
            ls += pv;
        }
    ls += __shfl_xor(ls, 16, 64);
    ls += __shfl_xor(ls, 32, 64);

    // ---- O^T[d][head] over the wave's 64 keys (two 32-deep steps)
    f32x4 oacc[DT];
#pragma unroll
    for (int i = 0; i < DT; ++i) oacc[i] = zero_vec<f32x4>();
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        CT pf;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pf[i] = from_f32<T>(sacc[2 * u][i]);
            pf[4 + i] = from_f32<T>(sacc[2 * u + 1][i]);
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            CT vf;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                vf[i] = vlo[u][dt][i];
                vf[4 + i] = vhi[u][dt][i];
            }
            oacc[dt] = mma16(vf, pf, oacc[dt]);
        }
    }

    // ---- merge the four waves into this chunk's partial
    if (g == 0) {
        sm[wave][col] = mx;
        sl[wave][col] = ls;
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) so[wave][col][dt * 16 + 4 * g + j] = oacc[dt][j];
    __syncthreads();
    float* pb = part + ((long long)b * max_chunks + c) * PSZ;
    for (int i = tid; i < 16 * HD; i += 256) {
        const int h = i / HD, d = i % HD;
        const float M = fmaxf(fmaxf(sm[0][h], sm[1][h]), fmaxf(sm[2][h], sm[3][h]));
        float o = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w)
            if (sm[w][h] != -INFINITY) o += fast_exp2(sm[w][h] - M) * so[w][h][d];
        pb[32 + h * HD + d] = o;
    }
    if (tid < 16) {
        const int h = tid;
        const float M = fmaxf(fmaxf(sm[0][h], sm[1][h]), fmaxf(sm[2][h], sm[3][h]));
        float l = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w)
            if (sm[w][h] != -INFINITY) l += fast_exp2(sm[w][h] - M) * sl[w][h];
        pb[h] = M;
        pb[16 + h] = l;
    }

}

// Combine kernel: workgroup (head h, row b), one thread per feature d:
// y[b][h][d] = sum_c 2^(m_c - M) o_c[d] / sum_c 2^(m_c - M) l_c.
template <typename T, int HD>
__global__ __launch_bounds__(HD) void attn_decode_combine_kernel(const float* __restrict__ part,
                                                                 const int32_t* __restrict__ lens,
                                                                 T* __restrict__ y, int H, int S,
                                                                 int max_chunks) {
    constexpr int PSZ = 16 * (HD + 2);
    const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
    const int nkeys = min(lens[b] + 1, S);
    const int nch = (nkeys + DEC_CHUNK - 1) / DEC_CHUNK;
    const float* prow = part + (long long)b * max_chunks * PSZ;
    float M = -INFINITY;
    for (int cc = 0; cc < nch; ++cc) M = fmaxf(M, prow[(long long)cc * PSZ + h]);
    float o = 0.f, l = 0.f;
    for (int cc = 0; cc < nch; ++cc) {
        const float* pc = prow + (long long)cc * PSZ;
        const float w = fast_exp2(pc[h] - M);
        l += w * pc[16 + h];
        o += w * pc[32 + h * HD + d];
    }
    y[((long long)b * H + h) * HD + d] = from_f32<T>(o / l);
}

hipError_t launch_attn_decode(DType dt, int hd, const void* q, const void* kc, const void* vtc,
                              const int32_t* lens, void* y, float* part, int B, int H, int S,
                              int max_chunks, hipStream_t st) {
    const float sl = 1.4426950408889634f / sqrtf((float)hd);
    dim3 g1(max_chunks, B), g2(H, B);
#define NC_AD(TT, HDV)                                                                         \
    do {                                                                                       \
        hipLaunchKernelGGL((attn_decode_split_kernel<TT, HDV>), g1, dim3(256), 0, st,          \
                           (const TT*)q, (const TT*)kc, (const TT*)vtc, lens, part, H, S,      \
                           max_chunks, sl);                                                    \
        hipLaunchKernelGGL((attn_decode_combine_kernel<TT, HDV>), g2, dim3(HDV), 0, st,        \
                           (const float*)part, lens, (TT*)y, H, S, max_chunks);                \
    } while (0)
    if (dt == BF16 && hd == 128) NC_AD(bf16, 128);
    else if (dt == BF16 && hd == 64) NC_AD(bf16, 64);
    else if (dt == F32 && hd == 128) NC_AD(float, 128);
    else if (dt == F32 && hd == 64) NC_AD(float, 64);
    else return hipErrorInvalidValue;
#undef NC_AD
    return hipGetLastError();
}

}  // namespace nc
