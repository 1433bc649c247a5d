// Causal multi-query attention for gfx950: a flash-style prefill kernel and a decode kernel
// over balanced runs of 64-key blocks.  Both write the attention output y in the layout the
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
// kept transposed in the cache ([hd][positions]) so that the A operand of O^T (the keys of
// one feature that a step contracts) is contiguous: in prefill the score tile's rows are
// taken in a permuted key order (pf_kperm) so that it is one 16-byte read.
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
// Key order of a 32-key score tile: A-operand row i of S^T = K Q^T reads key pf_kperm(i)
// (bits 2 and 3 of i swapped).  Output register r of lane (l32, hh) then holds key
// 16 (r / 8) + 8 hh + r % 8, so the eight scores a lane feeds into one 16-deep step of
// O^T = V^T P^T are eight consecutive keys, whose V^T operand is one 16-byte read.
__device__ __forceinline__ int pf_kperm(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }
// K chunk swizzle: the eight rows that eight neighbouring lanes read (keys pf_kperm(8 g + j),
// j = 0..7) get eight different values, pf_kswz(pf_kperm(x)) = x % 8.
__device__ __forceinline__ int pf_kswz(int key) { return (key & 3) | ((key & 8) >> 1); }

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
    // Work order over the whole launch.  Workgroups are dispatched x fastest, then y, then z,
    // and dealt round-robin to the 8 XCDs; with the query block in x (8 blocks for a 2048-token
    // row) each XCD would always get the same block, the longest 8x the shortest's work.  So
    // query blocks go by decreasing length across every (row, head), head fastest: each
    // length spreads over all XCDs and the launch ends on the shortest blocks.
    const int lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    const int hb = gridDim.y * gridDim.z;
    const int qb = gridDim.x - 1 - lin / hb;
    const int head = (lin % hb) % gridDim.y, b = (lin % hb) / gridDim.y;
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

    // LDS layouts (8-element chunks): K row `key` holds chunk ch at chunk position
    // ch ^ pf_kswz(key); V^T row d (KB keys) holds chunk ch at position ch ^ (d % 8), so that
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
            const int key = p / CPRK, ch = (p % CPRK) ^ pf_kswz(key);
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
                *(CT*)(&smem[key * HD + ((ch ^ pf_kswz(key)) * 8)]) = rk[i];
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
                const int key = mt * 32 + pf_kperm(l32), ch = 2 * s + hh;
                CT kf = *(const CT*)(&Ks[key * HD + ((ch ^ (l32 & 7)) * 8)]);  // l32 % 8 = pf_kswz(key)
#pragma unroll
                for (int jn = 0; jn < JN; ++jn) sacc[mt][jn] = mma32(kf, qf[jn][s], sacc[mt][jn]);
            }
        }

        // Online softmax in base 2 on unscaled scores: the running max m is kept unscaled and
        // p = 2^(c s - c m) with c = log2(e)/sqrt(hd), one FMA per score.  Only a block that
        // reaches past a query of this wave (the diagonal), past Kn, or before the window
        // start of a query of this wave needs the mask.  A query whose keys in the blocks
        // so far are all masked keeps an empty state (m = -inf, reference 0).  Key of
        // register r in score tile mt: k0 + 32 mt + 16 (r / 8) + 8 hh + r % 8 (pf_kperm).
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
                        const int key = k0 + mt * 32 + 16 * (r / 8) + 8 * hh + (r % 8);
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

        // O^T += V^T P^T over the block's 64 keys in four 16-deep steps; step t contracts keys
        // 16 t + 8 hh .. 16 t + 8 hh + 7 in this lane (registers 8 (t % 2) .. + 7 of score
        // tile t / 2), which V^T row d holds as its chunk 2 t + hh.
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
                const CT vf = *(const CT*)(&Vs[d * KB + (((2 * t + hh) ^ (d & 7)) * 8)]);
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
// One query per row at position pos_b = lens[b] against the row's cached keys lo_b..pos_b
// (lo_b = pos_b - window with a window, else 0) of each K/V head, all query heads of a K/V
// head's group together, so each cached K/V element is read from memory once per step
// (multi-query attention, yelogs.com launch write-up, architecture answer; decode against
// the cache, apidog.com/th guide, part 6, flash_attn_with_kvcache).
//
// Work split.  A unit is (row b, K/V head g); unit u = b nkv + g covers the 64-key blocks
// lo_b / 64 .. pos_b / 64 of its cache.  The blocks of all units, unit after unit, form one
// sequence, cut into equal contiguous runs, one per workgroup, whatever the row lengths:
// the launch stays balanced when the rows' lengths differ (d30's mixed lengths), and a
// run that ends inside a unit leaves a partial softmax state (max m, sum l, o[hd] per
// query head) for the workgroup that finishes the unit.  The cut is computed in the kernel
// from the device lengths, so a captured step stays valid as the rows grow.
//
// Workgroup: 4 waves.  Its blocks stream through a ring of NS LDS stages (bf16: 64 keys of
// K rows and of V^T rows, 1 KB direct-to-LDS loads, NS - 1 stages in flight); wave w takes
// keys 16 w .. 16 w + 15 of every block: S^T = K Q^T by 16x16x32 MFMAs (keys = rows, the
// group's <= 16 query heads = columns), online softmax in base 2 per head, then
// O^T += V^T P^T by 16x16x16 MFMAs whose B operand is the score tile as it stands (each lane
// already holds the 4 keys of its column).  fp32 (small check models) loads the same
// fragments straight from memory.
//
// Queries.  The finished queries (qkv_finish_decode, which also put the new key and value
// into the cache) of a unit's group are copied into LDS by a fifth wave, the I/O wave, with
// direct-to-LDS loads: the first units' while the ring's first stages load, a later unit's
// while the run is still DEC_QSEG units before it.  The I/O wave also does the run's output
// stores, so the streaming waves never wait on them.
//
// End of a unit's run: the 4 waves' states merge in LDS; a unit inside one run is
// normalised and stored to y; otherwise the state goes to the unit's partial slot and, at
// the end of the run, the workgroup counts itself on the unit's arrival counter (device-
// scope stores completed first, no cache-wide fence); the last to arrive merges the unit's
// partials into y and resets the counter.  y is [B][H hd] stored blocked (blocked_index).
constexpr int DEC_KB = 64;       // keys per block (one ring stage)
constexpr int DEC_QSEG = 2;      // query slots in LDS (units whose queries are staged ahead)
constexpr int DEC_PER_MIN = 2;   // at least this many blocks per workgroup
constexpr int DEC_MAX_WG = 256;  // workgroups per launch (one per CU)
constexpr int DEC_MAX_B = 128;

int attn_decode_span(int S, int window) { return (window < 0 || window >= S) ? S : window + 1; }
int attn_decode_workgroups(int units, int S) {
    const long long most = (long long)units * (S / DEC_KB);  // every unit at full length
    return (int)std::max(1LL, std::min((long long)DEC_MAX_WG, most / DEC_PER_MIN));
}
int attn_decode_slots(int units, int S) {
    (void)units;
    return std::min(DEC_MAX_WG, (S / DEC_KB + DEC_PER_MIN - 1) / DEC_PER_MIN + 2);
}

__device__ __forceinline__ f32x4 mma16x16x16(bf16x4 a, bf16x4 b, f32x4 c) {
    typedef short s4 __attribute__((ext_vector_type(4)));
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4, a), __builtin_bit_cast(s4, b), c, 0, 0, 0);
}
// O^T += V^T P^T over 4 keys: bf16 one 16x16x16 MFMA; fp32 four 16x16x4 MFMAs, key j of
// every lane contracted in MFMA j (the same key assignment on both operands).
__device__ __forceinline__ f32x4 pv_step(bf16x4 v, f32x4 p, f32x4 c) {
    bf16x4 pb;
#pragma unroll
    for (int j = 0; j < 4; ++j) pb[j] = (bf16)p[j];
    return mma16x16x16(v, pb, c);
}
__device__ __forceinline__ f32x4 pv_step(f32x4 v, f32x4 p, f32x4 c) {
#pragma unroll
    for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(v[j], p[j], c, 0, 0, 0);
    return c;
}

template <typename T, int HD>
__global__ __launch_bounds__(320) void attn_decode_kernel(DecAttnArgs a) {
    typedef typename Chunk<T>::type CT;     // 8 elements
    typedef typename Chunk<T>::half HT;     // 4 elements
    constexpr bool STAGE = sizeof(T) == 2;  // LDS ring for bf16
    constexpr int NS = STAGE ? (HD == 128 ? 3 : 5) : 1;
    constexpr int NSW = 4;                                  // streaming waves; wave 4 does I/O
    constexpr int KBYTES = DEC_KB * HD * 2;                 // a block's K rows (bf16)
    constexpr int SBYTES = STAGE ? 2 * KBYTES : 16;         // a stage: K, then V^T
    constexpr int LK = KBYTES / 1024 / NSW;                 // 1 KB loads per wave, K (and V^T)
    constexpr int KCH = HD / 8;                             // 16-byte chunks of a K row
    constexpr int DS = HD / 32;                             // 32-deep steps of S^T
    constexpr int DT = HD / 16;                             // 16-row tiles of O^T
    constexpr int OP = HD + 4;                              // padded merge row
    constexpr int HALF = HD / 2;
    constexpr int PSZ = 16 * (HD + 2);
    constexpr int TPH = HD / 8;                             // merge threads per head, 8 features each
    constexpr int QBYTES = 16 * HD * (int)sizeof(T);        // a query slot: 16 heads
    constexpr int PFB = (PSZ * 4 + 1023) / 1024 * 1024;     // LDS of a prefetched partial state
    static_assert(!STAGE || LK >= 1, "stage split");

    // One LDS array, carved into regions (a single LDS object leaves the compiler's wait
    // insertion no alias scopes to track, so reads of a landed ring stage do not wait for
    // the stages still in flight; the explicit waits below order them):
    //   ring  NS stages of SBYTES (K rows, then V^T rows)
    //   mrg   per streaming wave: o[16][OP], m[16], l[16] (fp32)
    //   outb  a unit's merged state: m[16], l[16], o[16][HD] (fp32)
    //   qsl   DEC_QSEG x 16 x HD elements: query heads of a group
    //   pfb   a partial state of an earlier run, prefetched (PSZ floats)
    //   pre / jlo / posr / flag / desc  int tables
    constexpr int MRG_FL = 16 * OP + 32;
    constexpr int MRG_OFF = NS * SBYTES;
    constexpr int OUT_OFF = MRG_OFF + NSW * MRG_FL * 4;
    constexpr int QSL_OFF = OUT_OFF + PSZ * 4;
    constexpr int PFB_OFF = QSL_OFF + DEC_QSEG * QBYTES;
    constexpr int INT_OFF = PFB_OFF + PFB;
    constexpr int LDS_BYTES = INT_OFF + (3 * DEC_MAX_B + 1 + 2 + 4) * 4;
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    static_assert(QSL_OFF % 16 == 0 && QBYTES % 1024 == 0, "query slots: whole 1 KB loads");

    __shared__ __attribute__((aligned(1024))) unsigned char lds[LDS_BYTES];
    unsigned char* const ring = lds;
    float (*const mrg)[MRG_FL] = (float (*)[MRG_FL])(lds + MRG_OFF);
    float* const outb = (float*)(lds + OUT_OFF);
    T (*const qsl)[16][HD] = (T (*)[16][HD])(lds + QSL_OFF);
    float* const pfb = (float*)(lds + PFB_OFF);
    int* const pre = (int*)(lds + INT_OFF);  // DEC_MAX_B + 1
    int* const jlo = pre + DEC_MAX_B + 1;     // DEC_MAX_B
    int* const posr = jlo + DEC_MAX_B;        // DEC_MAX_B
    int* const flag = posr + DEC_MAX_B;       // 2: a partial state never came; states prefetched
    int* const desc = flag + 2;               // 4: first unit, its block; last unit, its block

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool io = wave == NSW;  // wave-uniform
    const int col = lane & 15, grp = lane >> 4;
    const int B = a.B, nkv = a.nkv, S = a.S, H = a.H, G = H / nkv;

    // ---- block counts per row and their prefix (I/O wave; B <= 128, two rows per lane)
    if (io) {
        int nb[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = 2 * lane + i;
            nb[i] = 0;
            if (r < B) {
                const int pos = min(max(a.lens[r], 0), S - 1);  // capacity is checked by the host
                const int lo = (a.window < 0 || a.window >= pos) ? 0 : pos - a.window;
                nb[i] = pos / DEC_KB - lo / DEC_KB + 1;
                jlo[r] = lo / DEC_KB;
                posr[r] = pos;
            }
        }
        int s = nb[0] + nb[1];
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int t = __shfl_up(s, d, 64);
            if (lane >= d) s += t;
        }
        if (2 * lane < B) pre[2 * lane] = s - nb[0] - nb[1];
        if (2 * lane + 1 < B) pre[2 * lane + 1] = s - nb[1];
        const int tot = __shfl(s, 63, 64);
        if (lane == 0) {
            pre[B] = tot;
            flag[0] = 0;
        }
        // this workgroup's run (the same formulas as below) and the units holding its first
        // and last block: the lane whose two rows hold block q answers, found by a ballot
        const int total = nkv * tot;
        const int nwg = max(1, min((int)gridDim.x, total / DEC_PER_MIN));
        const int w = blockIdx.x;
        if (w < nwg) {
            const int q_at[2] = {(int)((long long)w * total / nwg), (int)((long long)(w + 1) * total / nwg) - 1};
            const int p0 = nkv * (s - nb[0] - nb[1]), p1 = nkv * (s - nb[1]), p2 = nkv * s;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int q = q_at[e];
                const unsigned long long m = __ballot(p0 <= q && q < p2);
                const int L = __builtin_ctzll(m);
                const bool second = q >= p1;
                const int row = 2 * lane + (second ? 1 : 0);
                const int n = second ? nb[1] : nb[0];
                const int rel = q - (second ? p1 : p0);
                if (lane == L) {
                    desc[2 * e] = row * nkv + rel / n;  // unit
                    desc[2 * e + 1] = rel % n;          // block within the unit
                }
            }
        }
    }
    __syncthreads();
    // (LDS values are the same in every lane: read them as scalars, so that addresses built
    // from them stay in scalar registers)
    auto lds_s = [](const int* p) { return __builtin_amdgcn_readfirstlane(*p); };
    const int total = nkv * lds_s(&pre[B]);
    const int nwg = max(1, min((int)gridDim.x, total / DEC_PER_MIN));
    const int w = blockIdx.x;
    if (w >= nwg) return;  // workgroup-uniform
    // run of workgroup x: blocks [start(x), start(x + 1)), start(x) = floor(x total / nwg)
    auto start_of = [&](int x) { return (int)((long long)x * total / nwg); };
    auto wg_of = [&](int q) { return (int)(((long long)(q + 1) * nwg - 1) / total); };  // run holding block q
    const int g0 = start_of(w), g1 = start_of(w + 1);
    const int nblk = g1 - g0;  // >= 1

    // ---- processing order.  The run's blocks are F | M | X (F: blocks of its first unit,
    // which may continue a unit of earlier runs; X: blocks of its last unit, which may
    // continue into later runs; M: whole units).  They are processed as X, M, F: a unit
    // that continues into later runs leaves its partial state early, and the run that holds
    // a unit's last block (its owner, which merges the others' partial states into y) gets
    // to it last.  Segment k of the order is one unit's blocks [j, jend); units are linear
    // indices u = b nkv + g, consecutive in the run.
    const int u_first = lds_s(&desc[0]), jf = lds_s(&desc[1]);
    const int u_last = lds_s(&desc[2]), jl = lds_s(&desc[3]);
    const int nseg = u_last - u_first + 1;
    struct Cur { int k, u, b, g, j, jend, nb; };
    auto unit_nb = [&](int bb) { return lds_s(&pre[bb + 1]) - lds_s(&pre[bb]); };
    auto seg_begin = [&](Cur& c, int k) {
        c.k = k;
        int j0, je;
        if (nseg == 1) {
            c.u = u_first; j0 = jf; je = jl + 1;
        } else if (k == 0) {
            c.u = u_last; j0 = 0; je = jl + 1;
        } else if (k < nseg - 1) {
            c.u = u_first + k; j0 = 0; je = -1;
        } else {
            c.u = u_first; j0 = jf; je = -1;
        }
        c.b = c.u / nkv;
        c.g = c.u - c.b * nkv;
        c.nb = unit_nb(c.b);
        c.j = j0;
        c.jend = je < 0 ? c.nb : je;
    };
    auto cstart = [&]() { Cur c; seg_begin(c, 0); return c; };
    auto cadvance = [&](Cur& c) {  // next block in processing order
        if (++c.j == c.jend && c.k + 1 < nseg) seg_begin(c, c.k + 1);
    };
    // first block (global index) of unit (b, g)
    auto unit_first = [&](const Cur& c) { return nkv * lds_s(&pre[c.b]) + c.g * c.nb; };
    // the segment reaches the unit's last block: this run owns the unit
    auto owns = [&](const Cur& c) { return c.jend == c.nb; };

    // ---- query slot of segment k: heads g G .. g G + 15 of unit (b, g) (heads past the
    //      group repeat its last head; their scores are never used), 1 KB loads by the I/O wave
    const int nq = min(nseg, DEC_QSEG);
    auto issue_q = [&](const Cur& c, int sl) {
        unsigned char* dst = (unsigned char*)&qsl[sl][0][0];
        const unsigned char* src = (const unsigned char*)a.q + ((long long)c.b * H + c.g * G) * HD * sizeof(T);
#pragma unroll
        for (int ch = 0; ch < QBYTES / 1024; ++ch) {
            const int byte = ch * 1024 + lane * 16;
            const int h = min(byte / (HD * (int)sizeof(T)), G - 1);
            const int within = byte % (HD * (int)sizeof(T));
            __builtin_amdgcn_global_load_lds((gvoid*)(src + h * HD * sizeof(T) + within), (lvoid*)(dst + ch * 1024), 16, 0, 0);
        }
    };
    // ---- ring: stage t (t-th block in processing order) into slot t % NS.  A stage is 4 LK
    // chunks of 1 KB for K and as many for V^T; chunk c goes to LDS bytes 1024 c .. and lane
    // l of its load fetches the 16 bytes that land at 16 l (K: LDS chunk p = 64 c + l holds
    // key p / KCH, chunk (p % KCH) ^ (key % KCH); V^T: row d = p / 8, keys
    // 8 ((p % 8) ^ (d % 8)) .. + 8).  Streaming wave w loads chunks w LK .. w LK + LK - 1 of
    // every stage.
    auto issue = [&](int t, const Cur& c, int c0, int nc) {
        if constexpr (STAGE) {
            unsigned char* sb = ring + (t % NS) * SBYTES;
            const long long u = (long long)c.b * nkv + c.g;
            const int kbeg = (lds_s(&jlo[c.b]) + c.j) * DEC_KB;
            const unsigned char* kb = (const unsigned char*)a.kc + (u * S + kbeg) * HD * 2;
            const unsigned char* vb = (const unsigned char*)a.vtc + (u * HD * S + kbeg) * 2;
            for (int ch = c0; ch < c0 + nc; ++ch) {
                const int p = ch * 64 + lane;
                const int key = p / KCH, kch = (p % KCH) ^ (key % KCH);
                __builtin_amdgcn_global_load_lds((gvoid*)(kb + (unsigned)(key * HD + kch * 8) * 2u),
                                                 (lvoid*)(sb + ch * 1024), 16, 0, 0);
            }
            for (int ch = c0; ch < c0 + nc; ++ch) {
                const int p = ch * 64 + lane;
                const int d = p / 8, vch = (p % 8) ^ (d % 8);
                __builtin_amdgcn_global_load_lds((gvoid*)(vb + (unsigned)(d * S + vch * 8) * 2u),
                                                 (lvoid*)(sb + KBYTES + ch * 1024), 16, 0, 0);
            }
        }
    };
    // prologue: the I/O wave loads the first segments' queries; then (a CU returns its
    // loads in order, so the queries are not queued behind a stage) the streaming waves
    // issue their shares of the first NS - 1 stages while the I/O wave waits for the queries
    Cur ci = cstart();
    if (io)
        for (int k = 0; k < nq; ++k) {
            Cur c;
            seg_begin(c, k);
            issue_q(c, k);
        }
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int t = 0; t < NS - 1; ++t)
        if (t < nblk) {
            if (!io) issue(t, ci, wave * LK, LK);
            cadvance(ci);
        }
    if (io) NC_WAIT_VM(0);
    // (a full barrier: the streaming waves also wait for their prologue stages, which
    // measured faster overall than entering the loop with them in flight)
    __syncthreads();

    // ---- main loop
    const float scale = a.scale_log2;
    Cur cc = cstart();
    int seg = 0;
    int b = cc.b, g = cc.g, pos = lds_s(&posr[b]);
    int lo = (a.window < 0 || a.window >= pos) ? 0 : pos - a.window;
    CT qf[DS];
    auto load_q = [&](int sl) {
#pragma unroll
        for (int s = 0; s < DS; ++s) qf[s] = *(const CT*)(&qsl[sl][col][8 * (4 * s + grp)]);
    };
    if (!io) load_q(0);
    float m_run = -INFINITY, l_run = 0.f;
    f32x4 o_run[DT];
#pragma unroll
    for (int i = 0; i < DT; ++i) o_run[i] = zero_vec<f32x4>();
    int own_u = -1, own_ws0 = 0, own_n = 0;  // an owned unit shared with earlier runs (the last one processed)
    // I/O wave: a partial state stored, its flag not yet set (the flag waits until the
    // stores have completed, checked two blocks later so that the wave does not stall the
    // streaming waves at the next barrier)
    long long pend_flag = -1;
    int pend_t = 0;
    // The run's first unit, processed last, is owned by this run and shared with earlier
    // runs when the run starts inside it and holds its last block.  Those runs mostly store
    // their partial states early (a run's last unit comes first in its order), so the I/O
    // wave polls the flag of the first of them (slot 0) during the loop and, once it is set,
    // copies that state into pfb with device-scope direct-to-LDS loads.
    //   pf_st: -1 nothing to prefetch, 0 poll next, 1 poll in flight, 2 state loading
    int pf_st = -1, pf_fv = 0;
    const int32_t* pf_fl = nullptr;
    const unsigned char* pf_src = nullptr;
    if (io && jf > 0) {
        Cur c;
        seg_begin(c, nseg - 1);
        if (owns(c) && wg_of(unit_first(c)) < w) {
            const long long uf = (long long)c.b * nkv + c.g;
            pf_fl = a.flags + uf * a.max_slots;
            pf_src = (const unsigned char*)(a.part + uf * a.max_slots * PSZ);
            pf_st = 0;
        }
    }
    auto set_flag = [&]() {
        wait_stores_complete();
        if (lane == 0) __hip_atomic_store(a.flags + pend_flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        pend_flag = -1;
    };

    for (int t = 0; t < nblk; ++t) {
        if (io && pend_flag >= 0 && t >= pend_t + 2) set_flag();
        if constexpr (STAGE) {
            // wait for this wave's loads of stage t (its loads of the later stages may stay
            // in flight)
            if (!io) {
                const int ahead = min(NS - 2, nblk - 1 - t);
                if (ahead >= 3) NC_WAIT_VM(3 * 2 * LK);
                else if (ahead == 2) NC_WAIT_VM(2 * 2 * LK);
                else if (ahead == 1) NC_WAIT_VM(2 * LK);
                else NC_WAIT_VM(0);
            }
            __syncthreads();  // stage t is in LDS; every wave is done with stage t - 1
            if (t + NS - 1 < nblk) {
                if (!io) issue(t + NS - 1, ci, wave * LK, LK);
                cadvance(ci);
            }
        }
        if (io && pf_st == 1) {  // the flag polled one block ago
            if (__shfl(pf_fv, 0, 64) != 0) {
                if (pend_flag < 0) {  // (so that no wait of this wave holds up the loads)
                    __atomic_signal_fence(__ATOMIC_SEQ_CST);
                    constexpr int NCH = (PSZ * 4 + 1023) / 1024;
#pragma unroll
                    for (int ch = 0; ch < NCH; ++ch) {
                        const int byte = min(ch * 1024 + lane * 16, PSZ * 4 - 16);
                        __builtin_amdgcn_global_load_lds((gvoid*)(pf_src + byte), (lvoid*)((unsigned char*)pfb + ch * 1024),
                                                         16, 0, NC_CPOL_DEVICE);
                    }
                    pf_st = 2;
                }
            } else {
                pf_st = 0;
            }
        }
        if (io && pf_st == 0) {
            if (lane == 0) pf_fv = __hip_atomic_load(pf_fl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            pf_st = 1;
        }
        const long long u = (long long)b * nkv + g;
        if (!io) {
            const int kbeg = (lds_s(&jlo[b]) + cc.j) * DEC_KB;
            const int kw = kbeg + 16 * wave;          // first key of this wave
            // operands: K rows of keys kw + col (A of S^T), V^T rows d = 16 dt + col at keys
            // kw + 4 grp .. + 3 (A of O^T)
            CT kf[DS];
            HT vf[DT];
            if constexpr (STAGE) {
                const unsigned char* kl = ring + (t % NS) * SBYTES;
                const unsigned char* vl = kl + KBYTES;
                const int key = 16 * wave + col;
#pragma unroll
                for (int s = 0; s < DS; ++s) kf[s] = *(const CT*)(kl + key * HD * 2 + (((4 * s + grp) ^ (key % KCH)) * 16));
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const int d = 16 * dt + col, ch = 2 * wave + (grp >> 1);
                    vf[dt] = *(const HT*)(vl + d * 128 + ((ch ^ (d % 8)) * 16) + (grp & 1) * 8);
                }
            } else {
                const T* kb = (const T*)a.kc + (u * S + kw + col) * HD;
#pragma unroll
                for (int s = 0; s < DS; ++s) kf[s] = *(const CT*)(kb + 8 * (4 * s + grp));
                const T* vb = (const T*)a.vtc + u * HD * S + kw + 4 * grp;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) vf[dt] = *(const HT*)(vb + (long long)(16 * dt + col) * S);
            }
            // scores S^T: lane holds head col, keys kw + 4 grp + j
            f32x4 sc = zero_vec<f32x4>();
#pragma unroll
            for (int s = 0; s < DS; ++s) sc = mma16(kf[s], qf[s], sc);
            float mb = -INFINITY;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int key = kw + 4 * grp + j;
                const float v = (key <= pos && key >= lo) ? sc[j] * scale : -INFINITY;
                sc[j] = v;
                mb = fmaxf(mb, v);
            }
            mb = fmaxf(mb, __shfl_xor(mb, 16, 64));
            mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
            const float mn = fmaxf(m_run, mb);
            const float mref = (mn == -INFINITY) ? 0.f : mn;  // nothing visible yet: no mass
            const float al = fast_exp2(m_run - mref);           // 0 while the state is empty
            float ls = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                sc[j] = fast_exp2(sc[j] - mref);
                ls += sc[j];
            }
            ls += __shfl_xor(ls, 16, 64);
            ls += __shfl_xor(ls, 32, 64);
            l_run = l_run * al + ls;
            m_run = mn;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) o_run[dt] = pv_step(vf[dt], sc, o_run[dt] * al);
        }

        // ---- end of the unit's blocks in this run (workgroup-uniform)
        const bool unit_end = cc.j == cc.jend - 1;
        if (unit_end) {
            if (!io) {
                float* mw = mrg[wave];
                if (grp == 0) {
                    mw[16 * OP + col] = m_run;
                    mw[16 * OP + 16 + col] = l_run;
                }
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) *(f32x4*)(&mw[col * OP + 16 * dt + 4 * grp]) = o_run[dt];
            }
            lds_barrier();
            const int q0 = unit_first(cc);
            const int ws0 = wg_of(q0), ws1 = wg_of(q0 + cc.nb - 1);
            const int nsu = ws1 - ws0 + 1;  // runs holding blocks of this unit
            // the streaming waves merge their 4 states into outb (y values when the whole
            // unit is in this run, else this run's state)
            const int hh = tid / TPH, d0 = 8 * (tid % TPH);
            if (!io && hh < G) {
                float M = -INFINITY;
#pragma unroll
                for (int x = 0; x < NSW; ++x) M = fmaxf(M, mrg[x][16 * OP + hh]);
                const float mr = (M == -INFINITY) ? 0.f : M;
                float o[8], l = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] = 0.f;
#pragma unroll
                for (int x = 0; x < NSW; ++x) {
                    const float f = fast_exp2(mrg[x][16 * OP + hh] - mr);
                    l += f * mrg[x][16 * OP + 16 + hh];
#pragma unroll
                    for (int e = 0; e < 8; ++e) o[e] += f * mrg[x][hh * OP + d0 + e];
                }
                const float inv = nsu == 1 ? 1.0f / l : 1.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) outb[32 + hh * HD + d0 + e] = o[e] * inv;
                if (d0 == 0) {
                    outb[hh] = M;
                    outb[16 + hh] = l;
                }
            }
            // the next segment's queries were loaded by the I/O wave at an earlier unit's end
            // (or in the prologue, already waited for): they land before the barrier
            if (io && seg + 1 >= DEC_QSEG && t + 1 < nblk) NC_WAIT_VM(0);
            lds_barrier();  // outb is complete; the merge area is free again
            if (nsu > 1 && w == ws1) {  // owned, shared with earlier runs: merged after the loop
                own_u = (int)u;
                own_ws0 = ws0;
                own_n = nsu;
            } else if (io) {  // the stores: y, or this run's partial state in slot (unit, run - first run)
                if (nsu == 1) {
                    for (int e = lane; e < G * TPH; e += 64) {
                        const int h2 = e / TPH, f0 = 8 * (e % TPH);
                        CT yo;
#pragma unroll
                        for (int x = 0; x < 8; ++x) yo[x] = from_f32<T>(outb[32 + h2 * HD + f0 + x]);
                        *(CT*)((T*)a.y + blocked_index(b, (g * G + h2) * HD + f0, H * HD)) = yo;
                    }
                } else {
                    // 16-byte device-scope stores: few instructions, so that the wave does not
                    // queue long behind the ring's loads for vector-memory slots
                    const __amdgpu_buffer_rsrc_t ps = buffer_rsrc(a.part + (u * a.max_slots + (w - ws0)) * PSZ, PSZ * 4);
                    for (int e = lane; e < (32 + G * HD) / 4; e += 64) store_device4(ps, 16 * e, *(const f32x4*)&outb[4 * e]);
                    if (pend_flag >= 0) set_flag();  // (a run shares at most two units)
                    pend_flag = u * a.max_slots + (w - ws0);
                    pend_t = t;
                }
            }
            // this segment's slot is free (its queries are in the streaming waves' registers):
            // it takes the queries of the segment DEC_QSEG later
            if (io && seg + DEC_QSEG < nseg) {
                Cur c;
                seg_begin(c, seg + DEC_QSEG);
                issue_q(c, seg % DEC_QSEG);
            }
            // next unit
            if (t + 1 < nblk) {
                ++seg;
                m_run = -INFINITY;
                l_run = 0.f;
#pragma unroll
                for (int i = 0; i < DT; ++i) o_run[i] = zero_vec<f32x4>();
                cadvance(cc);
                b = cc.b;
                g = cc.g;
                pos = lds_s(&posr[b]);
                lo = (a.window < 0 || a.window >= pos) ? 0 : pos - a.window;
                if (!io) load_q(seg % DEC_QSEG);
            }
            continue;
        }
        cadvance(cc);
    }

    // ---- an owned unit shared with earlier runs: wait for their partial states (flags set
    // once each state is visible; they were written at the start of those runs), merge them
    // with this run's state (outb) into y, and clear the flags for the next launch
    if (io && pend_flag >= 0) set_flag();  // the state is visible device-wide before its flag
    if (own_u < 0) return;  // workgroup-uniform
    const long long u = own_u;
    const int nprev = own_n - 1;  // slots 0 .. nprev - 1
    int32_t* fl = a.flags + u * a.max_slots;
    if (io) {
        if (pf_st == 2) NC_WAIT_VM(0);  // the prefetched state has landed in pfb
        if (lane == 0) flag[1] = pf_st == 2 ? 1 : 0;
    }
    __syncthreads();
    const int npf = lds_s(&flag[1]);
    if (npf < nprev) {  // workgroup-uniform: wait for the other states (flags set once each
        // state is visible; they were written at the start of those runs, or at their end)
        if (tid >= npf && tid < nprev) {  // bounded wait
            int v = 0;
            for (int it = 0; it < (1 << 22); ++it) {
                v = __hip_atomic_load(fl + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (v) break;
                __builtin_amdgcn_s_sleep(2);
            }
            if (!v) flag[0] = 1;  // never set: the output is made NaN rather than wrong
        }
        __syncthreads();
    }
    if (io) return;
    // merge the earlier runs' states with this run's (outb) into y; clear the flags for the
    // next launch
    const bool bad = flag[0] != 0;
    const int hh = tid / TPH, d0 = 8 * (tid % TPH);
    if (hh < G) {
        const int bb = (int)(u / nkv), gg = (int)(u % nkv);
        const float* pu = a.part + u * a.max_slots * PSZ;
        float mt[4], lt[4], ot[4][8];
        auto fetch = [&](int s0) {  // 4 slots per batch of independent loads
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const int sl = min(s0 + x, nprev - 1);
                f32x4 o0, o1;
                if (sl < npf) {  // prefetched (wave-uniform)
                    mt[x] = pfb[hh];
                    lt[x] = pfb[16 + hh];
                    o0 = *(const f32x4*)&pfb[32 + hh * HD + d0];
                    o1 = *(const f32x4*)&pfb[32 + hh * HD + d0 + 4];
                } else {
                    const float* ps = pu + (long long)sl * PSZ;
                    const __amdgpu_buffer_rsrc_t r = buffer_rsrc(ps, PSZ * 4);
                    mt[x] = load_device(ps + hh);
                    lt[x] = load_device(ps + 16 + hh);
                    o0 = load_device4(r, 4 * (32 + hh * HD + d0));
                    o1 = load_device4(r, 4 * (32 + hh * HD + d0 + 4));
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    ot[x][e] = o0[e];
                    ot[x][4 + e] = o1[e];
                }
            }
        };
        float M = outb[hh];
        float l = 0.f, o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = 0.f;
        // running merge: scale what is summed so far whenever the maximum grows
        auto absorb = [&](float m, float lv, const float* ov) {
            const float Mn = fmaxf(M, m);
            const float mr = (Mn == -INFINITY) ? 0.f : Mn;
            const float fo = fast_exp2(M - mr), fn = fast_exp2(m - mr);
            l = l * fo + lv * fn;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = o[e] * fo + ov[e] * fn;
            M = Mn;
        };
        {
            float ov[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) ov[e] = outb[32 + hh * HD + d0 + e];
            M = -INFINITY;
            absorb(outb[hh], outb[16 + hh], ov);
        }
        for (int s0 = 0; s0 < nprev; s0 += 4) {
            fetch(s0);
#pragma unroll
            for (int x = 0; x < 4; ++x)
                if (s0 + x < nprev) absorb(mt[x], lt[x], ot[x]);
        }
        const float inv = bad ? __builtin_nanf("") : 1.0f / l;
        CT yo;
#pragma unroll
        for (int e = 0; e < 8; ++e) yo[e] = from_f32<T>(o[e] * inv);
        *(CT*)((T*)a.y + blocked_index(bb, (gg * G + hh) * HD + d0, H * HD)) = yo;
    }
    if (tid < nprev) __hip_atomic_store(fl + tid, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

hipError_t launch_attn_decode(DType dt, const DecAttnArgs& args, hipStream_t st) {
    DecAttnArgs a = args;
    a.scale_log2 = 1.4426950408889634f / sqrtf((float)a.hd);
    const int units = a.B * a.nkv;
    if (a.nkv < 1 || a.H % a.nkv || a.H / a.nkv > 16 || a.B < 1 || a.B > DEC_MAX_B || a.S % DEC_KB ||
        a.max_slots < attn_decode_slots(units, a.S) || !a.part || !a.flags || !a.y)
        return hipErrorInvalidValue;
    const dim3 grid(attn_decode_workgroups(units, a.S));
#define NC_AD(TT, HDV) NC_TLAUNCH((attn_decode_kernel<TT, HDV>), grid, dim3(320), 0, st, a)
    if (dt == BF16 && a.hd == 128) NC_AD(bf16, 128);
    else if (dt == BF16 && a.hd == 64) NC_AD(bf16, 64);
    else if (dt == F32 && a.hd == 128) NC_AD(float, 128);
    else if (dt == F32 && a.hd == 64) NC_AD(float, 64);
    else return hipErrorInvalidValue;
#undef NC_AD
    return hipGetLastError();
}

}  // namespace nc
