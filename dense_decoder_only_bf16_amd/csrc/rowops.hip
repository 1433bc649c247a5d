// Row-wise kernels: embedding + norm, the QKV finish of prefill (RoPE, QK-norm, KV-cache
// write), greedy argmax and small cache utilities.
//
// RMSNorm has no learnable parameters and sits after the token embedding (yelogs.com
// launch write-up, architecture answer); RoPE with precomputed tables (geoz.com.cn
// development-tricks section) and QK-norm (yelogs.com architecture answer; apidog.com/th
// part 1) finish the query and key projections.  Each of these is one wave per row (or
// per row and head) with wavefront reductions for the sums of squares.
#include <algorithm>

#include "common.h"
#include "finish.h"
#include "kernels.h"

namespace nc {

// ------------------------------------------------------------------ embedding -------
// One wave per row; each lane moves 8 consecutive elements per 16/32-byte access.
// Normalised embedding e of a token: chunks in v[], returned scale r (e = r wte[tok]).
template <typename T>
__device__ __forceinline__ float embed_row(const T* __restrict__ wte, int t, int nch, int d, float eps,
                                           int lane, typename Chunk<T>::type (&v)[8]) {
    typedef typename Chunk<T>::type CT;
    const T* e = wte + (long long)t * d;
    float s = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int cidx = lane + 64 * u;
        v[u] = load_masked(e + (cidx < nch ? cidx : 0) * 8, cidx < nch);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float f = to_f32(v[u][k]);
            s += f * f;
        }
    }
    s = wave_sum(s);
    return 1.0f / sqrtf(s / (float)d + eps);
}

// Row m is token m % T of batch row b = m / T at position pos = lens[b] + m % T (lens null:
// 0).  x = scale0 e' with e' = e, or with smear e + lambda sigmoid(e[:C] . g) e_prev (e_prev
// the normalised embedding of the row's previous token: the chunk's previous token, else
// hist[b][pos - 1]; none at position 0); x0 = e' and xb = x where requested; hist[b][pos] =
// token.
template <typename T>
__global__ __launch_bounds__(256) void embed_kernel(EmbedArgs a) {
    typedef typename Chunk<T>::type CT;
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= a.M) return;
    auto clamp_tok = [&](int t) { return t < 0 ? 0 : (t >= a.vocab ? a.vocab - 1 : t); };
    const int t = clamp_tok(a.tok[row]);
    const int nch = a.d / 8;  // d is a multiple of 64; up to 8 chunks per lane: d <= 4096
    const T* wte = (const T*)a.wte;
    CT v[8];
    const float r = embed_row<T>(wte, t, nch, a.d, a.eps, lane, v);
    float xs[8][8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int k = 0; k < 8; ++k) xs[u][k] = to_f32(v[u][k]) * r;
    const int T_ = a.T > 0 ? a.T : 1;
    const int b = row / T_, ti = row % T_;
    const int pos = ti + (a.lens ? a.lens[b] : 0);
    const bool in_cache = a.hist && pos >= 0 && pos < a.S;
    if (a.smear_gate) {
        const int prev = ti > 0 ? clamp_tok(a.tok[row - 1])
                                : ((in_cache && pos > 0) ? clamp_tok(a.hist[(long long)b * a.S + pos - 1]) : -1);
        if (prev >= 0) {  // wave-uniform
            const T* g = (const T*)a.smear_gate;
            float dot = 0.f;
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int c = (lane + 64 * u) * 8 + k;
                    dot += c < a.smear_ch ? xs[u][k] * to_f32(g[c]) : 0.f;
                }
            dot = wave_sum(dot);
            const float gate = a.smear_lambda / (1.0f + expf(-dot));
            const float rp = embed_row<T>(wte, prev, nch, a.d, a.eps, lane, v);
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int k = 0; k < 8; ++k) xs[u][k] += gate * to_f32(v[u][k]) * rp;
        }
    }
    if (in_cache && lane == 0) a.hist[(long long)b * a.S + pos] = t;
    if (a.tok_out && lane == 0) a.tok_out[row] = t;
    float s2 = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int cidx = lane + 64 * u;
        if (cidx < nch) {
            f32x8 xo, x0o;
            CT ao;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float f = xs[u][k] * a.scale0;
                x0o[k] = xs[u][k];
                xo[k] = f;
                ao[k] = from_f32<T>(f);
                s2 += f * f;
            }
            const long long o = (long long)row * a.d + cidx * 8;
            *(f32x8*)(a.x + o) = xo;
            if (a.x0) *(f32x8*)(a.x0 + o) = x0o;
            if (a.xb) *(f32x8*)(a.xb + o) = xo;
            *(CT*)((T*)a.act + (a.blocked ? blocked_index(row, cidx * 8, a.d) : o)) = ao;
        }
    }
    s2 = wave_sum(s2);
    if (lane == 0) a.ss[row] = s2;
}

hipError_t launch_embed(DType dt, const EmbedArgs& a, hipStream_t st) {
    if (a.d % 64 || a.d > 4096 || a.smear_ch > a.d) return hipErrorInvalidValue;
    dim3 grid((a.M + 3) / 4);
    if (dt == BF16)
        hipLaunchKernelGGL(embed_kernel<bf16>, grid, dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL(embed_kernel<float>, grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

// ------------------------------------------------------------------ QKV finish ------
// Workgroup (head slot j, 64 consecutive tokens of one batch row); slots 0..H-1 are query
// heads, H..H+nkv-1 the key heads, H+nkv..H+2nkv-1 the value heads.  Wave w takes tokens
// 16 w .. 16 w + 15 of the tile one after another; lane i < hd/2 holds the RoPE pair
// (i, i + hd/2).  The 16 row scales of a wave are computed up front, one token per lane.
// Value heads go through LDS so that each row d of the transposed V cache is written as
// 64 consecutive positions.
constexpr int QP_TILE = 64;

template <typename T>
__global__ __launch_bounds__(256) void qkv_post_kernel(QkvPostArgs a) {
    __shared__ T vs[128][QP_TILE];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int j = blockIdx.x;
    const int tpr = (a.T + QP_TILE - 1) / QP_TILE;
    const int b = blockIdx.y / tpr, t0 = (blockIdx.y % tpr) * QP_TILE;
    const int off = a.lens ? a.lens[b] : 0;  // position of the row's token 0
    const int half = a.hd / 2;
    const int slots = a.H + 2 * a.nkv;
    const int N = slots * a.hd;
    const bool act = lane < half;
    const int i = act ? lane : 0;
    const bool is_v = j >= a.H + a.nkv;

    // row scales of this wave's 16 tokens: lane k < 16 takes token 16 wave + k
    float rl = 1.f;
    {
        const int tk = t0 + 16 * wave + (lane & 15);
        const int m = b * a.T + min(tk, a.T - 1);
        constexpr int MAXP = 16;  // partial sums per row (prefill: one per 256 columns)
        float sp[MAXP];
#pragma unroll
        for (int q = 0; q < MAXP; ++q)
            sp[q] = q < a.ss_in_parts ? a.ss_in[(long long)q * a.ss_stride + m] : 0.f;
        float ssum = 0.f;
#pragma unroll
        for (int q = 0; q < MAXP; ++q) ssum += sp[q];
        for (int q = MAXP; q < a.ss_in_parts; ++q) ssum += a.ss_in[(long long)q * a.ss_stride + m];
        rl = 1.0f / sqrtf(ssum / (float)a.norm_dim + a.eps);
    }
    // One product slice (prefill): the 16 tokens' values and rotation tables are all loaded
    // before any arithmetic (rows past the tile's last token read a clamped row).
    const bool one = a.splits == 1;
    float pv1[16], pv2[16], pc[16], ps[16];
    if (one) {
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int t = min(t0 + 16 * wave + k, a.T - 1);
            const float* src = a.part + (long long)(b * a.T + t) * N + j * a.hd;
            pv1[k] = src[i];
            pv2[k] = src[i + half];
            const int pos = min(max(off + t, 0), a.S - 1);
            pc[k] = a.rope_cos[(long long)pos * half + i];
            ps[k] = a.rope_sin[(long long)pos * half + i];
        }
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const int tl = 16 * wave + k, t = t0 + tl;
        const float r = __shfl(rl, k, 64);
        if (t >= a.T) break;  // wave-uniform
        const int m = b * a.T + t;
        const int pos = off + t;
        float v1 = 0.f, v2 = 0.f;
        if (one) {
            v1 = act ? pv1[k] * r : 0.f;
            v2 = act ? pv2[k] * r : 0.f;
        } else {   // the K-split slices, in order, 8 independent loads per batch
            const float* src = a.part + (long long)m * N + j * a.hd;
            for (int z0 = 0; z0 < a.splits; z0 += 8) {
                float t1[8], t2[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const long long o = (long long)min(z0 + u, a.splits - 1) * a.z_stride;
                    t1[u] = src[o + i];
                    t2[u] = src[o + i + half];
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    v1 += (z0 + u < a.splits) ? t1[u] : 0.f;
                    v2 += (z0 + u < a.splits) ? t2[u] : 0.f;
                }
            }
            v1 = act ? v1 * r : 0.f;
            v2 = act ? v2 * r : 0.f;
        }
        if (is_v) {
            if (a.vemb.ve) {  // the layer's value embedding
                const ValueEmbed& ve = a.vemb;
                const int jj = j - a.H - a.nkv;
                const float g = value_embed_gate<T>((const T*)ve.ve_gate, jj, ve.ve_ch,
                                                    ve.xin + (long long)m * ve.xin_stride, r, lane);
                const T* e = (const T*)ve.ve + ((long long)ve.tok[m] * a.nkv + jj) * a.hd;
                v1 += act ? g * to_f32(e[i]) : 0.f;
                v2 += act ? g * to_f32(e[i + half]) : 0.f;
            }
            if (act) {
                vs[i][tl] = from_f32<T>(v1);
                vs[i + half][tl] = from_f32<T>(v2);
            }
            continue;
        }
        if (pos < 0 || pos >= a.S) continue;  // capacity is checked by the host
        float c = 0.f, sn = 0.f;
        if (act) {
            c = one ? pc[k] : a.rope_cos[(long long)pos * half + i];
            sn = one ? ps[k] : a.rope_sin[(long long)pos * half + i];
        }
        float o1 = v1 * c - v2 * sn;
        float o2 = v1 * sn + v2 * c;
        const float ms = wave_sum(o1 * o1 + o2 * o2) / (float)a.hd;
        const float rr = 1.0f / sqrtf(ms + a.eps);
        if (act) {
            T* dst;
            if (j < a.H)
                dst = (T*)a.q + ((long long)m * a.H + j) * a.hd;
            else
                dst = (T*)a.kc + (((long long)b * a.nkv + (j - a.H)) * a.S + pos) * a.hd;
            dst[i] = from_f32<T>(o1 * rr);
            dst[i + half] = from_f32<T>(o2 * rr);
        }
    }
    if (is_v) {  // workgroup-uniform: V^T rows, 64 consecutive positions each
        __syncthreads();
        T* vt = (T*)a.vtc + ((long long)b * a.nkv + (j - a.H - a.nkv)) * a.hd * a.S;
        for (int e = threadIdx.x; e < a.hd * QP_TILE; e += 256) {
            const int d = e / QP_TILE, p = e % QP_TILE;
            const int pos = off + t0 + p;
            if (t0 + p < a.T && pos >= 0 && pos < a.S) vt[(long long)d * a.S + pos] = vs[d][p];
        }
    }
}

hipError_t launch_qkv_post(DType dt, const QkvPostArgs& a, hipStream_t st) {
    if (a.nkv < 1 || a.H % a.nkv || a.hd > 128 || a.T < 1 || a.M % a.T) return hipErrorInvalidValue;
    const int B = a.M / a.T, tpr = (a.T + QP_TILE - 1) / QP_TILE;
    dim3 grid(a.H + 2 * a.nkv, B * tpr);
    if (dt == BF16)
        hipLaunchKernelGGL(qkv_post_kernel<bf16>, grid, dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL(qkv_post_kernel<float>, grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

// Decode step: one token per row at position lens[b].  Workgroup (4 head slots, row b),
// one wave per slot; lane i < hd/2 holds the RoPE pair (i, i + hd/2).  The slices' loads
// of a batch are all issued before they are added, in slice order.
template <typename T>
__global__ __launch_bounds__(256) void qkv_finish_decode_kernel(DecFinishArgs a) {
    const int lane = threadIdx.x & 63;
    const int j = 4 * blockIdx.x + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int b = blockIdx.y;
    if (j >= a.H + 2 * a.nkv) return;  // wave-uniform; no workgroup barrier below
    const int half = a.hd / 2;
    const int i = lane < half ? lane : 0;
    const float* src = a.part + (long long)b * (a.H + 2 * a.nkv) * a.hd + j * a.hd;
    float v1 = 0.f, v2 = 0.f;
    for (int z0 = 0; z0 < a.splits; z0 += 8) {
        float t1[8], t2[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const long long o = (long long)min(z0 + u, a.splits - 1) * a.z_stride;
            t1[u] = src[o + i];
            t2[u] = src[o + i + half];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            v1 += (z0 + u < a.splits) ? t1[u] : 0.f;
            v2 += (z0 + u < a.splits) ? t2[u] : 0.f;
        }
    }
    qkv_finish_head<T>(a, b, j, lane, v1, v2);
}

hipError_t launch_qkv_finish_decode(DType dt, const DecFinishArgs& a, hipStream_t st) {
    if (a.nkv < 1 || a.H % a.nkv || a.hd > 128 || a.hd % 2 || a.B < 1 || a.splits < 1 || !a.part || !a.lens)
        return hipErrorInvalidValue;
    dim3 grid((a.H + 2 * a.nkv + 3) / 4, a.B);
    if (dt == BF16)
        hipLaunchKernelGGL(qkv_finish_decode_kernel<bf16>, grid, dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL(qkv_finish_decode_kernel<float>, grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

// ------------------------------------------------------------------ argmax ----------
// Lowest index wins ties; NaN never wins against a number.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
    if (v != v) return false;
    if (bv != bv) return true;
    return v > bv || (v == bv && i < bi);
}

// One 1024-thread workgroup per row; 16-byte loads when the row allows it.
__global__ __launch_bounds__(1024) void argmax_kernel(const float* __restrict__ logits, int V,
                                                      int32_t* __restrict__ out) {
    __shared__ float sv[16];
    __shared__ int si[16];
    const int b = blockIdx.x, tid = threadIdx.x;
    const float* row = logits + (long long)b * V;
    float bv = __builtin_nanf("");
    int bi = 0x7fffffff;
    const bool vec = ((V & 3) == 0) && ((((uintptr_t)row) & 15) == 0);
    if (vec) {
        const f32x4* r4 = (const f32x4*)row;
        const int n4 = V >> 2;
        for (int i0 = tid; i0 < n4; i0 += 16 * 1024) {  // 16 independent loads per batch
            f32x4 v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) v[u] = r4[min(i0 + 1024 * u, n4 - 1)];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int i = i0 + 1024 * u;
                if (i < n4) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (better(v[u][e], 4 * i + e, bv, bi)) { bv = v[u][e]; bi = 4 * i + e; }
                }
            }
        }
    } else {
        for (int i = tid; i < V; i += 1024) {
            float v = row[i];
            if (better(v, i, bv, bi)) { bv = v; bi = i; }
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        float ov = __shfl_xor(bv, o, 64);
        int oi = __shfl_xor(bi, o, 64);
        if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    if ((tid & 63) == 0) { sv[tid >> 6] = bv; si[tid >> 6] = bi; }
    __syncthreads();
    if (tid == 0) {
        for (int w = 1; w < 16; ++w)
            if (better(sv[w], si[w], bv, bi)) { bv = sv[w]; bi = si[w]; }
        out[b] = (bi == 0x7fffffff) ? 0 : bi;
    }
}

hipError_t launch_argmax(const float* logits, int B, int V, int32_t* out, hipStream_t st) {
    hipLaunchKernelGGL(argmax_kernel, dim3(B), dim3(1024), 0, st, logits, V, out);
    return hipGetLastError();
}

// ------------------------------------------------------------------ sampling --------
// Order-preserving map of a float to an unsigned key (larger float, larger key); NaN maps
// to 0, below every number.
__device__ __forceinline__ uint32_t order_key(float x) {
    if (x != x) return 0u;
    const uint32_t b = __float_as_uint(x);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// One 1024-thread workgroup per row.  The row is taken in tiles of 65536 tokens held in
// registers: thread t holds the 16 four-token chunks j 1024 + t of the tile (64 values),
// loaded with independent 16-byte loads; a row of at most one tile is loaded once and
// every pass runs on registers (longer rows reload their tiles per pass).  Tokens past V
// are masked by index.
//  1. Threshold: the key of the top_k-th largest logit (keys: order_key), found bit by
//     bit from the top by counting the keys at or above each candidate (32 steps of one
//     comparison per value); top_k <= 0 or >= V keeps every logit.
//  2. m = the row's largest logit (always kept).
//  3. Weights w_i = 2^((x_i - m) scale) for kept, non-NaN logits (scale = log2(e) / T).
//     Range (tile, j) is the 4096 contiguous tokens of chunk column j; with the range
//     totals in token order and target = u Z, the last range with mass whose preceding
//     total is <= target is scanned over its threads (4 tokens each, in token order), and
//     the last thread with mass whose preceding sum is <= the remainder walks its 4
//     tokens to the first whose running sum exceeds it (rounding past the end: its last
//     token with mass).
constexpr int SMP_J = 16;                  // four-token chunks per thread in a tile
constexpr int SMP_TILE = SMP_J * 1024 * 4; // tokens per tile
constexpr int SMP_MAX_TILES = 16;          // rows up to 2^20 tokens

__device__ __forceinline__ void sample_load(const float* row, int V, int t0, bool vec, int tid,
                                            f32x4 (&v)[SMP_J]) {
#pragma unroll
    for (int j = 0; j < SMP_J; ++j) {
        const int i = t0 + 4 * (j * 1024 + tid);
        if (vec && i + 3 < V) {
            v[j] = *(const f32x4*)(row + i);
        } else {
            f32x4 t;
#pragma unroll
            for (int e = 0; e < 4; ++e) t[e] = (i + e < V) ? row[i + e] : __builtin_nanf("");
            v[j] = t;
        }
    }
}

template <bool MT>  // MT: more than one tile (V > 65536)
__global__ __launch_bounds__(1024) void sample_kernel(const float* __restrict__ logits, int V,
                                                      float scale, int top_k,
                                                      const float* __restrict__ u,
                                                      int32_t* __restrict__ out) {
    __shared__ int cntbuf[2][16];
    __shared__ float wred[16][SMP_J];
    __shared__ float rtot[SMP_MAX_TILES * SMP_J];
    __shared__ float wsc[16];
    __shared__ int wbest[16];
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float* row = logits + (long long)b * V;
    const bool vec = ((V & 3) == 0) && ((((uintptr_t)row) & 15) == 0);
    const int ntiles = MT ? (V + SMP_TILE - 1) / SMP_TILE : 1;
    f32x4 v[SMP_J];
    sample_load(row, V, 0, vec, tid, v);
    auto valid = [&](int t0, int j, int e) { return t0 + 4 * (j * 1024 + tid) + e < V; };

    uint32_t thresh = 0;
    if (top_k > 0 && top_k < V) {
        // The largest key t with at least top_k keys >= t, one bit at a time from the top
        // (per-lane counts, one wave sum per step).  The values are
        // turned into keys in place (padding and NaN: key 0, never counted) and back after.
        if (ntiles == 1) {
#pragma unroll
            for (int j = 0; j < SMP_J; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    v[j][e] = __uint_as_float(valid(0, j, e) ? order_key(v[j][e]) : 0u);
        }
        uint32_t prefix = 0;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = prefix | (1u << bit);
            int cnt = 0;
            for (int tl = 0; tl < ntiles; ++tl) {
                if (ntiles > 1) {
                    sample_load(row, V, tl * SMP_TILE, vec, tid, v);
#pragma unroll
                    for (int j = 0; j < SMP_J; ++j)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            v[j][e] = __uint_as_float(valid(tl * SMP_TILE, j, e) ? order_key(v[j][e]) : 0u);
                }
#pragma unroll
                for (int j = 0; j < SMP_J; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) cnt += (__float_as_uint(v[j][e]) >= cand) ? 1 : 0;
            }
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o, 64);
            if (lane == 0) cntbuf[bit & 1][wave] = cnt;
            __syncthreads();  // one barrier a step: the two parities alternate
            int total = 0;
#pragma unroll
            for (int w = 0; w < 16; ++w) total += cntbuf[bit & 1][w];
            if (total >= top_k) prefix = cand;
        }
        thresh = prefix;
        if (ntiles == 1) {  // keys back to values (key 0 -> a NaN)
#pragma unroll
            for (int j = 0; j < SMP_J; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t k = __float_as_uint(v[j][e]);
                    v[j][e] = __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
                }
        } else {
            sample_load(row, V, 0, vec, tid, v);
        }
    }

    float m = -INFINITY;  // fmaxf skips NaN (padding included)
    for (int tl = 0; tl < ntiles; ++tl) {
        if (ntiles > 1) sample_load(row, V, tl * SMP_TILE, vec, tid, v);
#pragma unroll
        for (int j = 0; j < SMP_J; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) m = fmaxf(m, v[j][e]);
    }
    m = wave_max(m);
    if (lane == 0) wsc[wave] = m;
    __syncthreads();
    m = wsc[0];
#pragma unroll
    for (int w = 1; w < 16; ++w) m = fmaxf(m, wsc[w]);
    if (m == -INFINITY) {  // no logit with mass
        if (tid == 0) out[b] = 0;
        return;
    }
    auto weight = [&](float x) {
        return (x == x && order_key(x) >= thresh) ? exp2f((x - m) * scale) : 0.f;
    };
    // range totals (tile, j), in token order
    for (int tl = 0; tl < ntiles; ++tl) {
        if (ntiles > 1) sample_load(row, V, tl * SMP_TILE, vec, tid, v);
        __syncthreads();  // wred of the previous tile has been read
#pragma unroll
        for (int j = 0; j < SMP_J; ++j) {
            float t = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) t += weight(v[j][e]);
            t = wave_sum(t);
            if (lane == 0) wred[wave][j] = t;
        }
        __syncthreads();
        if (tid < SMP_J) {
            float t = 0.f;
            for (int w = 0; w < 16; ++w) t += wred[w][tid];
            rtot[tl * SMP_J + tid] = t;
        }
    }
    __syncthreads();
    const int nr = ntiles * SMP_J;
    float Z = 0.f;
    for (int r = 0; r < nr; ++r) Z += rtot[r];
    float uu = u[b];
    uu = (uu >= 0.f) ? (uu < 1.f ? uu : 0x1.fffffep-1f) : 0.f;  // into [0, 1); NaN -> 0
    const float target = uu * Z;
    float pre = 0.f, rem = 0.f;
    int rsel = 0;
    for (int r = 0; r < nr; ++r) {
        if (rtot[r] > 0.f && pre <= target) {
            rsel = r;
            rem = target - pre;
        }
        pre += rtot[r];
    }
    const int tl = rsel / SMP_J, js = rsel % SMP_J;
    if (ntiles > 1) sample_load(row, V, tl * SMP_TILE, vec, tid, v);
    float w4[4], st = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f32x4 c = v[0];
#pragma unroll
        for (int j = 1; j < SMP_J; ++j) c = (j == js) ? v[j] : c;
        w4[e] = weight(c[e]);
        st += w4[e];
    }
    // exclusive scan of the threads' sums over the range (thread order = token order)
    float incl = st;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const float t = __shfl_up(incl, o, 64);
        if (lane >= o) incl += t;
    }
    if (lane == 63) wsc[wave] = incl;
    __syncthreads();
    float wpre = 0.f;
#pragma unroll
    for (int w = 0; w < 16; ++w) wpre += (w < wave) ? wsc[w] : 0.f;
    const float r = rem - (wpre + (incl - st));
    const bool ok = r >= 0.f && st > 0.f;
    int best = ok ? tid : -1;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) best = max(best, __shfl_xor(best, o, 64));
    if (lane == 0) wbest[wave] = best;
    __syncthreads();
    int tbest = -1;
#pragma unroll
    for (int w = 0; w < 16; ++w) tbest = max(tbest, wbest[w]);
    if (tid == tbest) {
        const int base = tl * SMP_TILE + 4 * (js * 1024 + tid);
        int pick = -1, last = -1;
        float loc = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            loc += w4[e];
            if (w4[e] > 0.f) {
                last = base + e;
                if (pick < 0 && loc > r) pick = base + e;
            }
        }
        out[b] = min(max(pick >= 0 ? pick : last, 0), V - 1);
    } else if (tbest < 0 && tid == 0) {
        out[b] = 0;
    }
}

hipError_t launch_sample(const float* logits, int B, int V, float scale, int top_k, const float* u,
                         int32_t* out, hipStream_t st) {
    if (V > SMP_MAX_TILES * SMP_TILE) return hipErrorInvalidValue;
    if (V <= SMP_TILE)
        hipLaunchKernelGGL(sample_kernel<false>, dim3(B), dim3(1024), 0, st, logits, V, scale, top_k, u, out);
    else
        hipLaunchKernelGGL(sample_kernel<true>, dim3(B), dim3(1024), 0, st, logits, V, scale, top_k, u, out);
    return hipGetLastError();
}

// ------------------------------------------------------------------ weight repack ---
// [N][K] row-major -> MFMA-blocked [Npad/32][K/16][32][16]; one thread per 8 elements.
template <typename T>
__global__ __launch_bounds__(256) void repack_kernel(const T* __restrict__ src, T* __restrict__ dst,
                                                     int N, int K) {
    typedef typename Chunk<T>::type CT;
    const long long c = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long total = blocked_elems(N, K) / 8;
    if (c >= total) return;
    const long long blk = c / 64;
    const int w = (int)(c % 64);
    const int ksteps = K / 16;
    const long long rbk = blk / ksteps;
    const int kb = (int)(blk % ksteps);
    const long long row = rbk * 32 + w / 2;
    const int k = kb * 16 + (w % 2) * 8;
    CT v = zero_vec<CT>();
    if (row < N) v = *(const CT*)(src + row * K + k);
    *(CT*)(dst + c * 8) = v;
}

hipError_t launch_repack(DType dt, const void* src, void* dst, int N, int K, hipStream_t st) {
    const long long total = blocked_elems(N, K) / 8;
    dim3 grid((unsigned)((total + 255) / 256));
    if (dt == BF16)
        hipLaunchKernelGGL(repack_kernel<bf16>, grid, dim3(256), 0, st, (const bf16*)src, (bf16*)dst, N, K);
    else
        hipLaunchKernelGGL(repack_kernel<float>, grid, dim3(256), 0, st, (const float*)src, (float*)dst, N, K);
    return hipGetLastError();
}

// ------------------------------------------------------------------ cache utilities -
__global__ void lens_kernel(int32_t* lens, int B, int32_t delta, int32_t set_value) {
    int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b < B) lens[b] = set_value >= 0 ? set_value : lens[b] + delta;
}

hipError_t launch_lens_add(int32_t* lens, int B, int32_t delta, int32_t set_value, hipStream_t st) {
    hipLaunchKernelGGL(lens_kernel, dim3((B + 255) / 256), dim3(256), 0, st, lens, B, delta, set_value);
    return hipGetLastError();
}

__global__ void zero_i32_kernel(int32_t* p, long long n) {
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x)
        p[i] = 0;
}

hipError_t launch_zero_i32(int32_t* p, long long n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    const long long blocks = std::min<long long>((n + 255) / 256, 1024);
    hipLaunchKernelGGL(zero_i32_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p, n);
    return hipGetLastError();
}

template <typename T>
__global__ __launch_bounds__(256) void kv_export_kernel(const T* __restrict__ kc, const T* __restrict__ vtc,
                                                        T* __restrict__ ko, T* __restrict__ vo, int B,
                                                        int S, int S_out, int hd) {
    long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    long long total = (long long)B * S_out * hd;
    if (i >= total) return;
    int d = (int)(i % hd);
    long long bs = i / hd;
    int s = (int)(bs % S_out);
    int b = (int)(bs / S_out);
    ko[i] = kc[((long long)b * S + s) * hd + d];
    vo[i] = vtc[((long long)b * hd + d) * S + s];
}

hipError_t launch_kv_export(DType dt, int hd, const void* kc, const void* vtc, void* k_out,
                            void* v_out, int B, int S, int S_out, hipStream_t st) {
    long long total = (long long)B * S_out * hd;
    dim3 grid((unsigned)((total + 255) / 256));
    if (dt == BF16)
        hipLaunchKernelGGL(kv_export_kernel<bf16>, grid, dim3(256), 0, st, (const bf16*)kc,
                           (const bf16*)vtc, (bf16*)k_out, (bf16*)v_out, B, S, S_out, hd);
    else
        hipLaunchKernelGGL(kv_export_kernel<float>, grid, dim3(256), 0, st, (const float*)kc,
                           (const float*)vtc, (float*)k_out, (float*)v_out, B, S, S_out, hd);
    return hipGetLastError();
}

// Row copy between caches of one model: workgroup (pair i, layer and K/V head, K or V).
// K of a (row, head) is len hd contiguous elements; V^T is hd rows of len positions with
// the cache's row stride.  Copies go in 16-byte units (the tail of a V^T row is rounded up
// to 16 bytes, which stays inside the row: S is a multiple of 64 positions).
__global__ __launch_bounds__(256) void kv_copy_rows_kernel(KvRowCopy rc, const char* __restrict__ ksrc,
                                                          const char* __restrict__ vsrc,
                                                          char* __restrict__ kdst, char* __restrict__ vdst,
                                                          int nkv, int hd, int es, int Bsrc, int Ssrc,
                                                          int Bdst, int Sdst, int32_t* lens_dst,
                                                          const int32_t* __restrict__ hsrc,
                                                          int32_t* __restrict__ hdst) {
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    const int i = blockIdx.x, l = blockIdx.y / nkv, kvh = blockIdx.y % nkv;
    const int len = rc.len[i];
    const long long us = ((long long)l * Bsrc + rc.src[i]) * nkv + kvh;  // (layer, row, head) unit
    const long long ud = ((long long)l * Bdst + rc.dst[i]) * nkv + kvh;
    if (blockIdx.z == 0) {
        const u4* s = (const u4*)(ksrc + us * Ssrc * hd * es);
        u4* d = (u4*)(kdst + ud * Sdst * hd * es);
        const long long n = (long long)len * hd * es / 16;
        for (long long e = threadIdx.x; e < n; e += 256) d[e] = s[e];
        if (l == 0 && kvh == 0 && threadIdx.x == 0) lens_dst[rc.dst[i]] = len;
    } else if (blockIdx.z == 2) {  // token history, once per pair
        if (l == 0 && kvh == 0)
            for (int e = threadIdx.x; e < len; e += 256)
                hdst[(long long)rc.dst[i] * Sdst + e] = hsrc[(long long)rc.src[i] * Ssrc + e];
    } else {
        const int per_row = (len * es + 15) / 16;
        const long long n = (long long)per_row * hd;
        for (long long e = threadIdx.x; e < n; e += 256) {
            const int row = (int)(e / per_row), c = (int)(e % per_row);
            const u4* s = (const u4*)(vsrc + ((us * hd + row) * Ssrc) * es) + c;
            u4* d = (u4*)(vdst + ((ud * hd + row) * Sdst) * es) + c;
            *d = *s;
        }
    }
}

hipError_t launch_kv_copy_rows(const KvRowCopy& rc, const void* ksrc, const void* vsrc, void* kdst,
                               void* vdst, int L, int nkv, int hd, int es, int Bsrc, int Ssrc, int Bdst,
                               int Sdst, int32_t* lens_dst, const int32_t* hsrc, int32_t* hdst,
                               hipStream_t st) {
    if (rc.n < 1 || rc.n > KvRowCopy::MAX || (!hsrc) != (!hdst)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kv_copy_rows_kernel, dim3(rc.n, L * nkv, hsrc ? 3 : 2), dim3(256), 0, st, rc,
                       (const char*)ksrc, (const char*)vsrc, (char*)kdst, (char*)vdst, nkv, hd, es,
                       Bsrc, Ssrc, Bdst, Sdst, lens_dst, hsrc, hdst);
    return hipGetLastError();
}

}  // namespace nc
