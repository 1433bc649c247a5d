// Causal multi-query attention for gfx950: a flash-style prefill kernel and a split-context
// decode kernel with a combine kernel.  Both write the attention output y in the layout the
// O product reads: MFMA-blocked (kernels.h, blocked_index) for bf16, row-major for fp32
// prefill.
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
// Workgroup: 256 query positions of one (row, head) over 8 / JN waves; wave w owns 32 JN
// queries as JN 32-column MFMA tiles.  The launcher uses JN = 1: 8 waves whose registers
// leave room for two waves per SIMD, so one wave's MFMAs overlap another's softmax
// (measured 1.35x faster than 4 waves of 64 queries at the d12 and d20 prefill shapes).  K/V advance in blocks of 64 keys staged in
// LDS; blocks past the last query of the workgroup, or before the window of its first
// query, are never loaded, and a wave whose queries all precede a block, or whose windows
// all start after it, skips its MFMAs.  Query i of row b sits at position off + i (off =
// offs[b]: the tokens already in the row's cache, 0 for a first prefill) and keys are
// cache positions.  Sliding window: a query at position p sees keys p - win .. p (win
// = 2^30: the whole causal context).
template <typename T, int HD, int JN>
__global__ __launch_bounds__(64 * 8 / JN) void attn_prefill_kernel(const T* __restrict__ q,
                                                           const T* __restrict__ kc,
                                                           const T* __restrict__ vtc,
                                                           T* __restrict__ y, int Tn, int H,
                                                           int nkv, int S, int win,
                                                           const int32_t* __restrict__ offs,
                                                           float scale_log2) {
    typedef typename Chunk<T>::type CT;
    typedef typename Chunk<T>::half HT;
    constexpr int BQ = 256, KB = 64, NT = 64 * 8 / JN;
    constexpr int CPRK = HD / 8;      // chunks per K row
    constexpr int KSTEPS = HD / 16;   // 16-deep steps over the head dim
    constexpr int MD = HD / 32;       // 32-row tiles of O^T

    // bf16: two buffers of a K block and a V^T block, filled by direct-to-LDS loads; fp32:
    // one buffer, filled through registers.  Both take 8 KB HD bytes.
    constexpr bool DIRECT = sizeof(T) == 2;
    constexpr int BUF_T = 2 * KB * HD;  // elements of one buffer (K block, then V^T block)
    __shared__ __attribute__((aligned(1024))) T smem[DIRECT ? 2 * BUF_T : BUF_T];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const int qb = gridDim.x - 1 - blockIdx.x;  // longest (latest) query blocks first
    const int head = blockIdx.y, b = blockIdx.z;
    const int q0 = qb * BQ;
    const int q0w = q0 + wave * 32 * JN;
    const int off = offs ? offs[b] : 0;  // position of query 0
    const int Kn = off + Tn;             // keys in the cache after this prefill

    const int kvh = head / (H / nkv);  // the K/V head this query head reads
    const T* kb_base = kc + ((long long)b * nkv + kvh) * S * HD;
    const T* vb_base = vtc + ((long long)b * nkv + kvh) * HD * S;

    // Query operands: B operand of S^T, lane holds query (q0w + jn*32 + l32), dims 16s+8hh..
    CT qf[JN][KSTEPS];
#pragma unroll
    for (int jn = 0; jn < JN; ++jn) {
        const int qi = q0w + jn * 32 + l32;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
            if (qi < Tn)
                qf[jn][s] = *(const CT*)(q + (((long long)b * Tn + qi) * H + head) * HD + 16 * s + 8 * hh);
            else
                qf[jn][s] = zero_vec<CT>();
        }
    }

    f32x16 oacc[MD][JN];
    float m_run[JN], l_run[JN];
#pragma unroll
    for (int jn = 0; jn < JN; ++jn) {
#pragma unroll
        for (int i = 0; i < MD; ++i) oacc[i][jn] = zero_vec<f32x16>();
        m_run[jn] = -INFINITY;
        l_run[jn] = 0.f;
    }

    const int kend = off + min(Tn, q0 + BQ);
    const int nkb = (kend + KB - 1) / KB;
    const int kb_first = max(0, off + q0 - win) / KB;  // earliest key any query here sees
    const int p0w = off + q0w;                          // position of this wave's first query
    const int plast_w = p0w + 32 * JN - 1;              // and of its last
    constexpr int KCH = KB * CPRK / NT;  // K chunks per thread
    constexpr int VCH = HD * (KB / 8) / NT;
    static_assert(KCH >= 1 && VCH >= 1, "block too small for the workgroup");

    // LDS layouts (16-byte chunks): K row `key` holds chunk ch at chunk position
    // ch ^ (key % 8); V^T row d (KB keys) holds chunk ch at position ch ^ (d % 8), so that
    // the operand reads below are spread over the banks.
    // bf16: block kbi goes straight into buffer `bufi` with 1 KB direct-to-LDS loads; lane l
    // of a load writes chunk position l of its 1 KB and so fetches the chunk that the
    // swizzle puts there.  Rows past Kn are loaded as they are (the cache holds finite
    // values everywhere): their scores are masked, so they weigh 0.
    constexpr int NWV = 8 / JN;                    // waves
    constexpr int KJ = KB * CPRK / 64 / NWV;       // 1 KB K loads per wave
    constexpr int VJ = HD * (KB / 8) / 64 / NWV;   // 1 KB V^T loads per wave
    auto issue = [&](int kbi, int bufi) {
        const int k0 = kbi * KB;
        T* kl = smem + bufi * BUF_T;
        T* vl = kl + KB * HD;
#pragma unroll
        for (int j = 0; j < KJ; ++j) {
            const int p = (wave * KJ + j) * 64 + lane;
            const int key = p / CPRK, ch = (p % CPRK) ^ (key & 7);
            __builtin_amdgcn_global_load_lds((gvoid*)(kb_base + (long long)(k0 + key) * HD + ch * 8),
                                             (lvoid*)(kl + (wave * KJ + j) * 512), 16, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < VJ; ++j) {
            const int p = (wave * VJ + j) * 64 + lane;
            const int d = p / (KB / 8), ch = (p % (KB / 8)) ^ (d & 7);
            __builtin_amdgcn_global_load_lds((gvoid*)(vb_base + (long long)d * S + k0 + ch * 8),
                                             (lvoid*)(vl + (wave * VJ + j) * 512), 16, 0, 0);
        }
    };
    // fp32: K/V block k0 into registers (zeros past Kn), then into LDS.
    CT rk[KCH], rv[VCH];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            int c = tid + i * NT, key = c / CPRK, ch = c % CPRK;
            const int kk = min(k0 + key, Kn - 1);
            rk[i] = load_masked(kb_base + (long long)kk * HD + ch * 8, k0 + key < Kn);
        }
#pragma unroll
        for (int i = 0; i < VCH; ++i) {
            int c = tid + i * NT, d = c / (KB / 8), ch = c % (KB / 8);
            const T* src = vb_base + (long long)d * S + k0 + ch * 8;
            if (k0 + ch * 8 + 8 <= Kn) {
                rv[i] = *(const CT*)src;
            } else {
                CT t = zero_vec<CT>();
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (k0 + ch * 8 + e < Kn) t[e] = src[e];
                rv[i] = t;
            }
        }
    };
    // bf16: block kbi + 1 streams into the other buffer while block kbi is worked on, with
    // one barrier per block.
    if (DIRECT && kb_first < nkb) issue(kb_first, 0);
    for (int kbi = kb_first; kbi < nkb; ++kbi) {
        const int k0 = kbi * KB;
        const T* Ks;
        const T* Vs;
        if constexpr (DIRECT) {
            const int bufi = (kbi - kb_first) & 1;
            NC_WAIT_VM_ALL();  // this wave's loads of block kbi have landed
            __syncthreads();   // every wave's have, and every wave is done with the other buffer
            if (kbi + 1 < nkb) issue(kbi + 1, bufi ^ 1);
            Ks = smem + bufi * BUF_T;
            Vs = Ks + KB * HD;
        } else {
            gload(k0);
            __syncthreads();  // previous block's LDS reads are complete
#pragma unroll
            for (int i = 0; i < KCH; ++i) {
                int c = tid + i * NT, key = c / CPRK, ch = c % CPRK;
                *(CT*)(&smem[key * HD + ((ch ^ (key & 7)) * 8)]) = rk[i];
            }
#pragma unroll
            for (int i = 0; i < VCH; ++i) {
                int c = tid + i * NT, d = c / (KB / 8), ch = c % (KB / 8);
                *(CT*)(&smem[KB * HD + d * KB + ((ch ^ (d & 7)) * 8)]) = rv[i];
            }
            __syncthreads();
            Ks = smem;
            Vs = smem + KB * HD;
        }

        // every query of this wave precedes the block, or its window starts after it
        if (k0 > plast_w || k0 + KB - 1 < p0w - win) continue;

        f32x16 sacc[2][JN];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
            for (int jn = 0; jn < JN; ++jn) sacc[mt][jn] = zero_vec<f32x16>();
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s) {
                const int key = mt * 32 + l32, ch = 2 * s + hh;
                CT kf = *(const CT*)(&Ks[key * HD + ((ch ^ (key & 7)) * 8)]);
#pragma unroll
                for (int jn = 0; jn < JN; ++jn) sacc[mt][jn] = mma32(kf, qf[jn][s], sacc[mt][jn]);
            }
        }

        // Online softmax in base 2 on unscaled scores: the running max m is kept unscaled and
        // p = 2^(c s - c m) with c = log2(e)/sqrt(hd), one FMA per score.  Only a block that
        // reaches past a query of this wave (the diagonal), past Kn, or before the window
        // start of a query of this wave needs the mask.  A query whose keys in the blocks
        // so far are all masked keeps an empty state (m = -inf, reference 0).  Row index of
        // register r in a 32x32 output tile: 8*(r/4) + 4*hh + (r%4).
        const bool need_mask = (k0 + KB - 1 > p0w) || (k0 + KB > Kn) || (k0 < plast_w - win);  // wave-uniform
#pragma unroll
        for (int jn = 0; jn < JN; ++jn) {
            const int qp = p0w + jn * 32 + l32;  // the query's position
            float mx = -INFINITY;
            if (need_mask) {
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = k0 + mt * 32 + 8 * (r / 4) + 4 * hh + (r % 4);
                        const float v = (key <= qp && key < Kn && key >= qp - win) ? sacc[mt][jn][r] : -INFINITY;
                        sacc[mt][jn][r] = v;
                        mx = fmaxf(mx, v);
                    }
            } else {
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[mt][jn][r]);
            }
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            // Lazy rescaling: the reference max moves only when the block's max exceeds it by
            // more than 8 in the base-2 exponent (or no key was visible yet), so p <= 2^8 and
            // the state is rescaled (64 multiplies) only when some lane of the wave moved.
            const float m_cand = fmaxf(m_run[jn], mx);
            const bool move = m_run[jn] == -INFINITY || scale_log2 * (m_cand - m_run[jn]) > 8.f;
            const float m_new = move ? m_cand : m_run[jn];
            const float cm = (m_new == -INFINITY) ? 0.f : scale_log2 * m_new;
            const float alpha = move ? fast_exp2(scale_log2 * m_run[jn] - cm) : 1.f;  // 0 on the first block
            float ls = 0.f;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float pv = fast_exp2(fmaf(sacc[mt][jn][r], scale_log2, -cm));
                    sacc[mt][jn][r] = pv;
                    ls += pv;
                }
            ls += __shfl_xor(ls, 32, 64);
            l_run[jn] = l_run[jn] * alpha + ls;
            m_run[jn] = m_new;
            if (__any(move)) {  // wave-uniform
#pragma unroll
                for (int md = 0; md < MD; ++md) oacc[md][jn] *= alpha;
            }
        }

        // O^T += V^T P^T over the block's 64 keys in four 16-deep steps.
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int mt = t / 2, rb = 8 * (t % 2);
            CT pf[JN];
#pragma unroll
            for (int jn = 0; jn < JN; ++jn)
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
#pragma unroll
                for (int jn = 0; jn < JN; ++jn) oacc[md][jn] = mma32(vf, pf[jn], oacc[md][jn]);
            }
        }
    }

    // Normalise and store: lane holds query (l32 + 32 jn), features 32md + 8(r/4) + 4hh + 0..3.
#pragma unroll
    for (int jn = 0; jn < JN; ++jn) {
        const int qi = q0w + jn * 32 + l32;
        if (qi >= Tn) continue;
        const float inv = 1.0f / l_run[jn];
        const long long row = (long long)b * Tn + qi;
#pragma unroll
        for (int md = 0; md < MD; ++md)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                HT o;
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = from_f32<T>(oacc[md][jn][4 * g + e] * inv);
                const int c = head * HD + md * 32 + 8 * g + 4 * hh;  // 4 features, 4-aligned
                // bf16: the O product's operand layout (blocked); fp32: row-major
                const long long o_idx = sizeof(T) == 2 ? blocked_index((int)row, c, H * HD) : row * H * HD + c;
                *(HT*)(y + o_idx) = o;
            }
    }
}

hipError_t launch_attn_prefill(DType dt, int hd, const void* q, const void* kc, const void* vtc,
                               void* y, int B, int T, int H, int nkv, int S, int window,
                               const int32_t* offs, hipStream_t st) {
    if (nkv < 1 || H % nkv) return hipErrorInvalidValue;
    const int win = (window < 0 || window >= S) ? (1 << 30) : window;  // 2^30: whole context
    dim3 grid((T + 255) / 256, H, B);
    const float sl = 1.4426950408889634f / sqrtf((float)hd);
#define NC_AP(TT, HDV)                                                                          \
    NC_TLAUNCH((attn_prefill_kernel<TT, HDV, 1>), grid, dim3(512), 0, st, (const TT*)q,        \
               (const TT*)kc, (const TT*)vtc, (TT*)y, T, H, nkv, S, win, offs, sl)
    if (dt == BF16 && hd == 128) NC_AP(bf16, 128);
    else if (dt == BF16 && hd == 64) NC_AP(bf16, 64);
    else if (dt == F32 && hd == 128) NC_AP(float, 128);
    else if (dt == F32 && hd == 64) NC_AP(float, 64);
    else return hipErrorInvalidValue;
#undef NC_AP
    return hipGetLastError();
}

// ------------------------------------------------------------------ decode ----------
// Split kernel.  Workgroup (chunk c, unit u = (row b, K/V head kvh)), NW = 2 or 4 waves: the
// keys [c CK, c CK + CK) of K/V head kvh of row b, CK = 64 NW R, limited to the visible
// positions lo..lens[b] (lo = lens[b] - window with a window, else 0), against the
// G = H / nkv query heads kvh G .. kvh G + G - 1 (G <= 16).  The grid's x index counts
// chunks from the one holding lo, so only chunks with visible keys are launched work;
// a wave's blocks wholly before lo are skipped.  Wave w takes the 64-key blocks
// (c R + i) NW + w, i < R, one after another and keeps an online-softmax state (running
// max, sum and o[16][hd]) across them; at the end the NW states are merged in LDS into the
// chunk's partial state, slot c of row b (with R = 1 each wave's state is a partial of its
// own, slot NW c + w, and the merge is left to the combine kernel).
//  1. Finish the QKV product of row b for this step (the row's attention-norm scale,
//     RoPE at position lens[b] and QK-norm of the group's query heads and of key head kvh;
//     value head kvh as is) into LDS.  Every workgroup of the row does this (a few hundred values);
//     the one whose chunk holds position lens[b] also writes the new key and value into the
//     cache for later steps.
//  2. All query heads of the row (padded to 16) form the 16 columns of 16x16 MFMA tiles,
//     so each cached K/V element is read from memory once for the whole head group.
//     bf16: a wave stages a block's K (64 x hd) and V^T (hd x 64) in its own LDS region
//     with 1 KB direct-to-LDS loads, XOR-swizzled so that the MFMA operand reads are free
//     of bank conflicts; once the block's operands are in registers, the next block's
//     loads are issued and overlap this block's arithmetic.  fp32 (small check model):
//     operands are loaded straight into registers.  Cached keys at or past lens[b] are
//     masked in the scores; the new key (position lens[b]) is not read from the cache but
//     added to the state of the wave whose block holds it, as one extra term from the
//     values in LDS.
constexpr int DEC_KPW = 64;
int attn_decode_span(int S, int window) { return (window < 0 || window >= S) ? S : window + 1; }
// Waves per workgroup: 4, or 2 when the work is small (more, smaller workgroups then).
// B here and below counts (row, K/V head) units; `span` bounds the keys a query sees.
int attn_decode_waves(int B, int span) { return (long long)B * ((span + 255) / 256) >= 128 ? 4 : 2; }
int attn_decode_iters(int B, int span) {
    // The largest R in {1, 2, 4} that still leaves 128 workgroups or more: a wave's blocks
    // run one after another at about one memory latency each, so longer chunks amortize
    // the QKV finish and the merge until too few workgroups are left to fill the chip
    // (measured at d12, d20 and d30 decode shapes).
    const int nw = attn_decode_waves(B, span);
    int r = 1;
    while (r < 4 && (long long)B * ((span + nw * 64 * 2 * r - 1) / (nw * 64 * 2 * r)) >= 128) r *= 2;
    return r;
}
// Slots are indexed by absolute chunk, so a unit needs as many as the whole cache has.
int attn_decode_slots(int B, int S, int span) {
    const int nw = attn_decode_waves(B, span), r = attn_decode_iters(B, span);
    const int ck = nw * DEC_KPW * r;
    return (S + ck - 1) / ck * (r == 1 ? nw : 1);  // one block per wave: a slot per wave
}

template <typename T, int HD, int NW>
__global__ __launch_bounds__(NW * 64) void attn_decode_split_kernel(DecAttnArgs a) {
    typedef typename Chunk<T>::type CT;
    typedef typename Chunk<T>::half HT;
    constexpr bool STAGE = sizeof(T) == 2;  // LDS staging for bf16
    constexpr int DS = HD / 32;   // 32-deep steps over head dim for S^T
    constexpr int DT = HD / 16;   // 16-row tiles of O^T
    constexpr int PSZ = 16 * (HD + 2);
    constexpr int HALF = HD / 2;
    constexpr int KREG = DEC_KPW * HD * 2;  // bytes of one block's K (and of its V^T), bf16
    constexpr int WREG = 2 * KREG;          // a wave's region: staging, then its final state
    static_assert(WREG >= PSZ * 4, "a wave's state fits its region");
    constexpr int NSLOT = (18 + NW - 1) / NW;  // QKV-finish slots per wave

    __shared__ __attribute__((aligned(1024))) unsigned char buf[NW * WREG];
    __shared__ __attribute__((aligned(32))) T qs[16][HD];
    __shared__ __attribute__((aligned(32))) T kv_new[2][HD];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, g = lane >> 4;
    const int u = blockIdx.y;  // unit u = b nkv + kvh
    const int b = u / a.nkv, kvh = u % a.nkv;
    const int S = a.S, H = a.H, R = a.iters;
    const int G = H / a.nkv;
    const int CK = NW * DEC_KPW * R;
    const int pos = a.lens[b];  // this step's position; keys lo..pos are visible
    if (pos < 0 || pos >= S) return;  // capacity is checked by the host; stay in bounds
    const int lo = (a.window < 0 || a.window >= pos) ? 0 : pos - a.window;
    const int c = blockIdx.x + lo / CK;
    const int nchunks = (pos + 1 + CK - 1) / CK;
    if (c >= nchunks) return;
    T* kb_base = (T*)a.kc + (long long)u * S * HD;
    T* vb_base = (T*)a.vtc + (long long)u * HD * S;
    unsigned char* kl = buf + wave * WREG;  // K: 64 keys x HD, 16-byte chunks swizzled
    unsigned char* vl = kl + KREG;           // V^T: HD rows x 64 keys (128 bytes a row)
    // first key of this wave's i-th block; a block starting past pos holds no visible key
    auto kbeg_of = [&](int i) { return ((c * R + i) * NW + wave) * DEC_KPW; };

    // ---- staging loads of one block of cached K and V^T (bf16)
    auto issue = [&](int kbeg) {
        if constexpr (STAGE) {
            constexpr int KCH = HD / 8;  // 16-byte chunks per K row
            // K: LDS byte 16 p holds key p / KCH, chunk (p % KCH) ^ (key % KCH)
#pragma unroll
            for (int j = 0; j < KREG / 1024; ++j) {
                const int p = j * 64 + lane;
                const int kidx = p / KCH, cch = (p % KCH) ^ (kidx % KCH);
                int key = kbeg + kidx;
                key = key < pos ? key : (pos > 0 ? pos - 1 : 0);  // keys >= pos are masked
                __builtin_amdgcn_global_load_lds((gvoid*)(kb_base + (long long)key * HD + cch * 8),
                                                 (lvoid*)(kl + j * 1024), 16, 0, 0);
            }
            // V^T: LDS byte 16 p holds row d = p / 8, keys 8 ((p % 8) ^ (d % 8)) .. +8
#pragma unroll
            for (int j = 0; j < KREG / 1024; ++j) {
                const int p = j * 64 + lane;
                const int d = p / 8;
                int k0 = kbeg + 8 * ((p % 8) ^ (d % 8));
                k0 = k0 <= S - 8 ? k0 : S - 8;  // a chunk starting at or past S is fully masked
                __builtin_amdgcn_global_load_lds((gvoid*)(vb_base + (long long)d * S + k0),
                                                 (lvoid*)(vl + j * 1024), 16, 0, 0);
            }
        }
    };
    // first block of this wave that reaches lo (blocks are R apart in NW 64-key steps)
    int i0 = 0;
    while (i0 < R && kbeg_of(i0) + DEC_KPW <= lo) ++i0;
    const bool first_live = i0 < R && kbeg_of(i0) <= pos;
    if (first_live) issue(kbeg_of(i0));

    // ---- 1. QKV finish for row b: slot j = wave + NW i (0..15 the group's query heads,
    //         padding past G; 16 key head kvh; 17 value head kvh).  All loads first, then
    //         arithmetic.
    {
        const float* raw = a.qkv + (long long)b * (H + 2 * a.nkv) * HD;
        const bool act = lane < HALF;
        const int i = act ? lane : 0;
        float v1[NSLOT], v2[NSLOT];
#pragma unroll
        for (int t = 0; t < NSLOT; ++t) {
            const int j = wave + NW * t;
            const int src = (j < G) ? kvh * G + j : (j == 16 ? H + kvh : (j == 17 ? H + a.nkv + kvh : 0));
            v1[t] = raw[src * HD + i];
            v2[t] = raw[src * HD + i + HALF];
        }
        const float cs = a.rope_cos[(long long)pos * HALF + i], sn = a.rope_sin[(long long)pos * HALF + i];
        const float r = row_scale_wave(a.ss_in, a.ss_in_parts, a.ss_stride, b, a.norm_dim, a.eps);
#pragma unroll
        for (int t = 0; t < NSLOT; ++t) {
            const int j = wave + NW * t;
            if (j >= 18) continue;
            if (j < G || j == 16) {  // rotate + normalise
                const float x1 = v1[t] * r, x2 = v2[t] * r;
                const float o1 = x1 * cs - x2 * sn, o2 = x1 * sn + x2 * cs;
                const float ss = wave_sum(act ? o1 * o1 + o2 * o2 : 0.f);
                const float rr = 1.0f / sqrtf(ss / (float)HD + a.eps);
                T* dst = (j < 16) ? qs[j] : kv_new[0];
                if (act) {
                    dst[i] = from_f32<T>(o1 * rr);
                    dst[i + HALF] = from_f32<T>(o2 * rr);
                }
            } else if (j == 17) {
                float w1 = v1[t] * r, w2 = v2[t] * r;
                if (a.vemb) {  // the layer's value embedding (wave-uniform)
                    const ValueEmbed& ve = *a.vemb;
                    const float g = value_embed_gate<T>((const T*)ve.ve_gate, kvh, ve.ve_ch,
                                                        ve.xin + (long long)b * ve.xin_stride, r, lane);
                    const T* e = (const T*)ve.ve + ((long long)ve.tok[b] * a.nkv + kvh) * HD;
                    w1 += g * to_f32(e[i]);
                    w2 += g * to_f32(e[i + HALF]);
                }
                if (act) {
                    kv_new[1][i] = from_f32<T>(w1);
                    kv_new[1][i + HALF] = from_f32<T>(w2);
                }
            } else {  // padding query slot
                if (act) {
                    qs[j][i] = from_f32<T>(0.f);
                    qs[j][i + HALF] = from_f32<T>(0.f);
                }
            }
        }
    }
    __syncthreads();
    if (c == nchunks - 1)  // the chunk holding `pos` stores the new key/value
        for (int e = tid; e < HD; e += NW * 64) {
            kb_base[(long long)pos * HD + e] = kv_new[0][e];
            vb_base[(long long)e * S + pos] = kv_new[1][e];
        }
    CT qf[DS];
#pragma unroll
    for (int s = 0; s < DS; ++s) qf[s] = *(const CT*)(&qs[col][32 * s + 8 * g]);

    // ---- 2. the wave's blocks, online softmax over them.  State per lane: head `col`;
    //         o_run[dt][j] holds O^T[d = 16 dt + 4 g + j][col].
    float m_run = -INFINITY, l_run = 0.f;
    f32x4 o_run[DT];
#pragma unroll
    for (int i = 0; i < DT; ++i) o_run[i] = zero_vec<f32x4>();
    for (int it = i0; it < R; ++it) {
        const int kbeg = kbeg_of(it);
        if (kbeg > pos) break;  // wave-uniform: this and later blocks hold no visible key
        CT kf[4][DS];
        // V^T operands: slot 8g+i of 32-key step u <-> key 32u + 4g + i (i < 4) or
        // 32u + 16 + 4g + (i - 4) (i >= 4).
        HT vlo[2][DT], vhi[2][DT];
        if constexpr (STAGE) {
            constexpr int KCH = HD / 8;
            NC_WAIT_VM_ALL();  // this wave's staging loads of the block have landed
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                const int kidx = 16 * kt + col;
#pragma unroll
                for (int s = 0; s < DS; ++s)
                    kf[kt][s] = *(const CT*)(kl + kidx * (HD * 2) + (((4 * s + g) ^ (kidx % KCH)) * 16));
            }
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const int d = dt * 16 + col;
                    const int k1 = 32 * u + 4 * g, k2 = k1 + 16;  // first keys (local) of the halves
                    vlo[u][dt] = *(const HT*)(vl + d * 128 + (((k1 / 8) ^ (d % 8)) * 16) + (k1 % 8) * 2);
                    vhi[u][dt] = *(const HT*)(vl + d * 128 + (((k2 / 8) ^ (d % 8)) * 16) + (k2 % 8) * 2);
                }
            // the operand reads are complete before the region is refilled
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
            __builtin_amdgcn_sched_barrier(0);
            if (it + 1 < R && kbeg_of(it + 1) <= pos) issue(kbeg_of(it + 1));
        } else {
            const int klast = pos > 0 ? pos - 1 : 0;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                int key = kbeg + 16 * kt + col;
                key = key < pos ? key : klast;
#pragma unroll
                for (int s = 0; s < DS; ++s) kf[kt][s] = *(const CT*)(kb_base + (long long)key * HD + 32 * s + 8 * g);
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                int ka = kbeg + 32 * u + 4 * g, kb2 = ka + 16;
                ka = ka <= S - 4 ? ka : S - 4;
                kb2 = kb2 <= S - 4 ? kb2 : S - 4;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const T* src = vb_base + (long long)(dt * 16 + col) * S;
                    vlo[u][dt] = *(const HT*)(src + ka);
                    vhi[u][dt] = *(const HT*)(src + kb2);
                }
            }
        }

        // scores S^T (lane: head `col`, keys kbeg + 16kt + 4g + j), cached keys < pos
        f32x4 sacc[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            sacc[kt] = zero_vec<f32x4>();
#pragma unroll
            for (int s = 0; s < DS; ++s) sacc[kt] = mma16(kf[kt][s], qf[s], sacc[kt]);
        }
        float mb = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int key = kbeg + 16 * kt + 4 * g + j;
                const float v = (key < pos && key >= lo) ? sacc[kt][j] * a.scale_log2 : -INFINITY;
                sacc[kt][j] = v;
                mb = fmaxf(mb, v);
            }
        mb = fmaxf(mb, __shfl_xor(mb, 16, 64));
        mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
        const float mn = fmaxf(m_run, mb);
        const float mref = (mn == -INFINITY) ? 0.f : mn;  // nothing visible yet: no mass
        const float al = fast_exp2(m_run - mref);           // 0 while the state is empty
        float ls = 0.f;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float pv = fast_exp2(sacc[kt][j] - mref);
                sacc[kt][j] = pv;
                ls += pv;
            }
        ls += __shfl_xor(ls, 16, 64);
        ls += __shfl_xor(ls, 32, 64);
        l_run = l_run * al + ls;
        m_run = mn;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int j = 0; j < 4; ++j) o_run[dt][j] *= al;
        // O^T[d][head] += V^T P over the block's 64 keys (two 32-deep steps)
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
                o_run[dt] = mma16(vf, pf, o_run[dt]);
            }
        }
        // the new key (position pos) joins the wave whose block holds it
        if (pos >= kbeg && pos < kbeg + DEC_KPW) {
            // score of head `col`: lane group g sums a quarter of the hd features
            float part = 0.f;
#pragma unroll
            for (int e = 0; e < HD / 4; ++e)
                part += to_f32(qs[col][g * (HD / 4) + e]) * to_f32(kv_new[0][g * (HD / 4) + e]);
            part += __shfl_xor(part, 16, 64);
            part += __shfl_xor(part, 32, 64);
            const float sp = part * a.scale_log2;
            const float mn2 = fmaxf(m_run, sp);
            const float al2 = fast_exp2(m_run - mn2);  // 0 when no cached key was visible
            const float be = fast_exp2(sp - mn2);
            l_run = l_run * al2 + be;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    o_run[dt][j] = o_run[dt][j] * al2 + be * to_f32(kv_new[1][dt * 16 + 4 * g + j]);
            m_run = mn2;
        }
    }

    // ---- 3a. one block per wave (R == 1): each wave's state is its own partial, slot
    //          NW c + w of row b; the combine kernel merges them with the other chunks'.
    if (R == 1) {
        float* pw = a.part + ((long long)u * a.max_slots + NW * c + wave) * PSZ;
        if (g == 0) {
            pw[col] = m_run;
            pw[16 + col] = l_run;
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) *(f32x4*)(pw + 32 + col * HD + dt * 16 + 4 * g) = o_run[dt];
        return;
    }
    // ---- 3b. merge the waves' states into the chunk's partial (slot c of row b)
    if constexpr (STAGE) NC_WAIT_VM_ALL();  // no staging load still in flight into the region
    __syncthreads();                        // every wave is done with its region
    float* st = (float*)(buf + wave * WREG);
    if (g == 0) {
        st[col] = m_run;
        st[16 + col] = l_run;
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) st[32 + col * HD + dt * 16 + 4 * g + j] = o_run[dt][j];
    __syncthreads();
    float* pb = a.part + ((long long)u * a.max_slots + c) * PSZ;
    for (int e = tid; e < 16 * HD; e += NW * 64) {
        const int h = e / HD;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, ((const float*)(buf + w * WREG))[h]);
        const float mref = (M == -INFINITY) ? 0.f : M;
        float o = 0.f, l = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float* sw = (const float*)(buf + w * WREG);
            const float f = fast_exp2(sw[h] - mref);
            o += f * sw[32 + e];
            l += f * sw[16 + h];
        }
        pb[32 + e] = o;
        if (e % HD == 0) {
            pb[h] = M;
            pb[16 + h] = l;
        }
    }
}

// Combine kernel: workgroup (head h, row b), one thread per feature d, over the row's
// chunks (slots) of `chunk` keys that hold visible keys (from the one holding lo):
// y[b][h][d] = sum_s 2^(m_s - M) o_s[d] / sum_s 2^(m_s - M) l_s over the row's slots.  The
// slot statistics are loaded lane-parallel (one slot per lane), the weights go through
// LDS, and the o_s[d] loads of consecutive slots are independent of each other.
template <typename T, int HD>
__global__ __launch_bounds__(HD) void attn_decode_combine_kernel(const float* __restrict__ part,
                                                                 const int32_t* __restrict__ lens,
                                                                 T* __restrict__ y, int H, int nkv,
                                                                 int S, int window, int max_slots,
                                                                 int chunk) {
    constexpr int PSZ = 16 * (HD + 2);
    __shared__ float wts[512];
    __shared__ float stat[1];
    const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
    const int G = H / nkv, hg = h % G;  // query head h is head hg of K/V head h / G's group
    const int pos = min(lens[b], S - 1);
    const int nsl = min((pos + 1 + chunk - 1) / chunk, 512);
    const int s_lo = ((window < 0 || window >= pos) ? 0 : pos - window) / chunk;
    const float* prow = part + ((long long)b * nkv + h / G) * max_slots * PSZ;
    if (d < 64) {  // wave 0: max, weights and normaliser
        float mloc = -INFINITY;
        for (int sl = s_lo + d; sl < nsl; sl += 64) mloc = fmaxf(mloc, prow[(long long)sl * PSZ + hg]);
        const float M = wave_max(mloc);
        float lsum = 0.f;
        for (int sl = s_lo + d; sl < nsl; sl += 64) {
            const float w = fast_exp2(prow[(long long)sl * PSZ + hg] - M);  // 0 for empty slots
            wts[sl] = w;
            lsum += w * prow[(long long)sl * PSZ + 16 + hg];
        }
        lsum = wave_sum(lsum);
        if (d == 0) stat[0] = 1.0f / lsum;
    }
    __syncthreads();
    const float* po = prow + 32 + hg * HD + d;
    float o = 0.f;
    for (int s0 = s_lo; s0 < nsl; s0 += 16) {  // 16 slots per batch of independent loads
        float t[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) t[u] = po[(long long)min(s0 + u, nsl - 1) * PSZ];
#pragma unroll
        for (int u = 0; u < 16; ++u) o += (s0 + u < nsl) ? wts[min(s0 + u, nsl - 1)] * t[u] : 0.f;
    }
    y[blocked_index(b, h * HD + d, H * HD)] = from_f32<T>(o * stat[0]);
}

hipError_t launch_attn_decode(DType dt, const DecAttnArgs& args, void* y, hipStream_t st) {
    DecAttnArgs a = args;
    a.scale_log2 = 1.4426950408889634f / sqrtf((float)a.hd);
    if (a.nkv < 1 || a.H % a.nkv || a.H / a.nkv > 16) return hipErrorInvalidValue;
    const int units = a.B * a.nkv;  // (row, K/V head) pairs
    const int span = attn_decode_span(a.S, a.window);
    const int nw = attn_decode_waves(units, span);
    if (a.iters != attn_decode_iters(units, span) || a.max_slots < attn_decode_slots(units, a.S, span))
        return hipErrorInvalidValue;
    const int ck = nw * DEC_KPW * a.iters;
    // chunks with visible keys: all of them, or those a window of span keys can touch
    const int all = (a.S + ck - 1) / ck;
    const int live = span == a.S ? all : std::min(all, (span - 1 + ck - 1) / ck + 1);
    dim3 g1(live, units), g2(a.H, a.B);
    // the combine sees slots of `chunk` keys: a wave's block when R == 1, else a chunk
    const int chunk = a.iters == 1 ? DEC_KPW : ck;
#define NC_AD(TT, HDV)                                                                         \
    do {                                                                                       \
        if (nw == 4) NC_TLAUNCH((attn_decode_split_kernel<TT, HDV, 4>), g1, dim3(256), 0, st, a); \
        else NC_TLAUNCH((attn_decode_split_kernel<TT, HDV, 2>), g1, dim3(128), 0, st, a);     \
        NC_TLAUNCH((attn_decode_combine_kernel<TT, HDV>), g2, dim3(HDV), 0, st,                \
                   (const float*)a.part, a.lens, (TT*)y, a.H, a.nkv, a.S,              \
                   span == a.S ? -1 : a.window, a.max_slots, chunk);                          \
    } while (0)
    if (dt == BF16 && a.hd == 128) NC_AD(bf16, 128);
    else if (dt == BF16 && a.hd == 64) NC_AD(bf16, 64);
    else if (dt == F32 && a.hd == 128) NC_AD(float, 128);
    else if (dt == F32 && a.hd == 64) NC_AD(float, 64);
    else return hipErrorInvalidValue;
#undef NC_AD
    return hipGetLastError();
}

}  // namespace nc
