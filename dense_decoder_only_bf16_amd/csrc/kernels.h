// Host-side launchers of the gfx950 kernels (one definition per .hip file).  Every
// launcher enqueues on `st` and returns hipGetLastError() of the launch.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nc {

// Kernel-timing hook.  While the library times a kernel class it hands a launch helper of
// that class up to NC_MAX_STAMPS event pairs; each NC_TLAUNCH in the helper takes the next
// pair and launches through hipExtLaunchKernel, which stamps the pair with the kernel's
// own start and end (no pair left: launched without stamps).
#define NC_MAX_STAMPS 2
struct LaunchStamp {
    hipEvent_t ev[NC_MAX_STAMPS][2];
    int avail, used;
};
extern thread_local LaunchStamp t_stamp;
#define NC_TLAUNCH(K, grid, block, shm, st, ...)                                            \
    do {                                                                                    \
        ::nc::LaunchStamp& ts_ = ::nc::t_stamp;                                             \
        const bool on_ = ts_.used < ts_.avail;                                              \
        hipExtLaunchKernelGGL(K, grid, block, shm, st, on_ ? ts_.ev[ts_.used][0] : nullptr, \
                              on_ ? ts_.ev[ts_.used][1] : nullptr, 0, __VA_ARGS__);         \
        ts_.used += on_ ? 1 : 0;                                                            \
    } while (0)

enum DType { F32 = 0, BF16 = 1 };

// Epilogues of the matrix product C = A[M,K] B[N,K]^T (fp32 accumulation):
//   STORE   out_f32[z][m][n] = C            (raw product; z = K-split index)
//   RELU2   out_t[m][n] = relu(r_m C)^2     (r_m = 1/sqrt(sum_p ss_in[p][m]/K + eps))
//   RESID   x[m][n] += C; out_t[m][n] = x; ss_out[tile_n][m] = sum over the tile of x^2
//   SOFTCAP out_f32[m][n] = cap tanh(r_m C / cap)
enum Epi { EPI_STORE = 0, EPI_RELU2 = 1, EPI_RESID = 2, EPI_SOFTCAP = 3 };

// Weight layout used by every projection: MFMA-blocked [Npad/32][K/16][32][16], i.e.
// element (n, k) of an [N][K] nn.Linear weight sits at
//   ((n / 32) * (K / 16) + k / 16) * 512 + (n % 32) * 16 + k % 16,
// with rows n >= N (up to Npad = N rounded up to 32) zero.  A 32x16 block is the operand
// of one 16-deep MFMA step for one wave.
__host__ __device__ inline long long blocked_elems(int N, int K) { return (long long)((N + 31) / 32) * 32 * K; }
// Index of element (n, k) in that layout (K a multiple of 16).  Decode activations use the
// same layout, rows being token rows, so a wave's 16-deep A operand is 1 KB contiguous.
__host__ __device__ inline long long blocked_index(int n, int k, int K) {
    return ((long long)(n >> 5) * (K >> 4) + (k >> 4)) * 512 + (n & 31) * 16 + (k & 15);
}
hipError_t launch_repack(DType dt, const void* src, void* dst, int N, int K, hipStream_t st);

// Low parts of the compensated prefill operands (bf16 model): lo = a - bf16(a) is stored as
// one e4m3 byte, e4m3(lo 2^LO8_SHIFT) clamped to +-448 (|lo| <= 2^-8 |a|, so the scaled value
// stays in range for |a| < 448), in the operand layout of the 32x32x64 fp8 MFMA: row block
// m / 32 and 64-deep group k / 64 form a 2 KB block whose 64 lanes hold 32 bytes each;
// lane (m % 32) + 32 ((k % 16) / 8) holds byte (k % 64) / 16 * 8 + k % 8, i.e. the 8 values
// of its row and k half in each of the group's four 16-deep steps, in step order.  The
// weight side of that MFMA is made from the bf16 fragments of the same four steps in
// registers, so both operands pair the same k in the same lane byte.  K % 64 == 0.
constexpr int LO8_SHIFT = 8;
__host__ __device__ inline long long lo8_index(int m, int k, int K) {
    return ((long long)(m >> 5) * (K >> 6) + (k >> 6)) * 2048 + ((m & 31) + 32 * ((k >> 3) & 1)) * 32 +
           ((k >> 4) & 3) * 8 + (k & 7);
}
// Largest |w| of n bf16 values, as the bit pattern of a non-negative float, max-ed into *out
// (which the caller zeroes first).
hipError_t launch_absmax(const void* w, long long n, unsigned* out, hipStream_t st);
// Exponent s of the weight's e4m3 copy in the fp8 low-part product: e4m3(w 2^s) with
// |w| 2^s <= 448 for the largest |w| (s in [0, 12]).
int lo8_weight_exp(float absmax);

// RESID with the later version's blocks (x0 non-null): the new residual is
//   x = ra (x_old + C) + rb x0 + rc xb        (xb null: no last term)
// with x0, xb fp32 [M][ldo] like x; xb_out (if set) receives a copy of the new x.
struct ResidExtra {
    const float* x0; const float* xb; float* xb_out;
    float ra, rb, rc;
};
__host__ __device__ inline float resid_value(const ResidExtra& e, long long o, float x_old, float c) {
    if (!e.x0) return x_old + c;
    float x = e.ra * (x_old + c) + e.rb * e.x0[o];
    if (e.xb) x += e.rc * e.xb[o];
    if (e.xb_out) e.xb_out[o] = x;
    return x;
}
// Decode kernels take these blocks by pointer (device memory, null: off): their argument
// blocks stay small, which measurably shortens these few-microsecond kernels.
__device__ inline float resid_value(const ResidExtra* e, long long o, float x_old, float c) {
    return e ? resid_value(*e, o, x_old, c) : x_old + c;
}

struct GemmArgs {
    // bf16: blocked [ceil(M/32)][K/16][32][16] (whole 32-row blocks; lda unused);
    // fp32: [M][lda], K contiguous.  The same holds for the dtype outputs out_t of RELU2 and
    // RESID (blocked with K = ldo for bf16); low parts: see A_lo.
    const void* A;
    const void* B;  // blocked weight (see above), Npad rows
    int M, N, K, lda, Npad;
    int k_split;        // grid z; K / k_split must be a multiple of the K tile
    float* out_f32;     // STORE / SOFTCAP output, RESID residual x (fp32)
    void* out_t;        // RELU2 output, RESID dtype copy of x
    int ldo;            // row stride of the outputs (elements)
    long long z_stride; // STORE: elements between K-split slices
    const float* ss_in; // RELU2 / SOFTCAP row statistics: ss_in[p * M_stride + m]
    int ss_in_parts, ss_stride;
    float* ss_out;      // RESID: ss_out[tile_n * ss_stride + m]
    float eps, cap;
    // Compensated operand (bf16 only): A_lo holds a - bf16(a), and the product is taken over
    // both parts (A + A_lo) W^T.  Null: plain A.
    // bf16: A_lo holds the e4m3 low parts in the lo8 layout (see lo8_index), and w8_exp is
    // the exponent of B's e4m3 copy (lo8_weight_exp of B's largest |w|).
    const void* A_lo;
    // RELU2 / RESID: also write value - dtype(value) here (the low part a later
    // compensated product reads; bf16: e4m3 in the lo8 layout with K = ldo).  Null: not
    // written.
    void* out_lo;
    int w8_exp;
    ResidExtra rx;  // RESID: the later version's residual scaling and backout
    // Tail split (bf16): when the tiles leave the last round of workgroups (one per CU) at
    // most half full, that round's tiles run as two K halves each; the half that arrives
    // first on its tile leaves its partial sums in tail_part and sets a ready flag, the other
    // adds them and runs the epilogue.  Null tail_part: off.  tail is set by the launcher.
    float* tail_part;    // GEMM_TAIL_SLOTS x GEMM_TAIL_FLOATS fp32
    int32_t* tail_ctr;   // 2 per slot, zero before the launch; every launch leaves them zero
    int tail;
};
constexpr int GEMM_TAIL_SLOTS = 128;
constexpr long long GEMM_TAIL_FLOATS = 512 * 128;  // a tile's accumulators: 512 threads x 128

// Prefill product (M in the thousands): 256 x 256 tiles.
int gemm_tile_n();             // N extent of one tile (ss_out parts = ceil(N / tile_n))
int gemm_tile_k(DType dt);     // K granularity
hipError_t launch_gemm(DType dt, Epi epi, const GemmArgs& a, hipStream_t st);

// Decode projection of the raw QKV product (EPI_STORE): the number of K slices it leaves in
// `part` (after the DEC_PART_CTRS counters, slice z at z M N) for the QKV finish to add, or 0
// when it writes the sum to out_f32 itself.
int dec_gemm_store_slices(DType dt, int M, int N, int K);

// Decode projection (M <= 128 rows, K a multiple of 16) with the epilogue fused
// (STORE / RELU2 / RESID / SOFTCAP).  Tiles are dec_gemm_tile_n() columns; RESID writes
// ss_out[tile_n * ss_stride + m] (parts = ceil(N / tile_n)).
// Decode activations (A, A_lo and the dtype outputs out_t, out_lo) are stored blocked with
// rows rounded up to 32 (blocked_index); the fp32 outputs are row-major with stride ldo.
struct DecFinishArgs;
struct DecGemmArgs {  // pointers first, then 4-byte fields: no padding (120 bytes)
    const void* A;              // blocked [ceil(M/32)][K/16][32][16] dtype
    const void* W;              // blocked weight, Npad = N rounded up to 32 rows
    float* out_f32; void* out_t;
    const float* ss_in;
    float* ss_out;
    int32_t* lens_inc;  // if set, workgroup 0 adds one to lens_inc[0..M) (end of a decode step)
    const void* A_lo;   // compensated operand a - bf16(a), bf16 blocked like A (bf16 only; null: plain A)
    void* out_lo;       // RELU2 / RESID low-part output, bf16 blocked like out_t (null: not written)
    // split-K workspace, dec_gemm_part_elems(M, N, K) elements: DEC_PART_CTRS int32 arrival
    // counters (zero before the first launch; every launch leaves them at zero), then the
    // fp32 partial products
    float* part;
    const ResidExtra* rx;  // RESID: as in GemmArgs, in device memory (null: plain residual)
    int M, N, K, ldo;
    int ss_in_parts, ss_stride;
    float eps, cap;
};
int dec_gemm_tile_n();
constexpr int DEC_PART_CTRS = 64;
// Elements of DecGemmArgs::part that a product of this shape needs (0: none).
long long dec_gemm_part_elems(DType dt, Epi epi, int M, int N, int K);
// fin (EPI_STORE only, dec_gemm_fuses_finish): the QKV finish runs in the product's
// epilogue: the last workgroup to store a column tile of a head finishes that head for every
// row (fin->part, splits and z_stride unused: the raw product is out_f32).
hipError_t launch_dec_gemm(DType dt, Epi epi, const DecGemmArgs& a, hipStream_t st, int variant = 0,
                           const DecFinishArgs* fin = nullptr);

// x[m] = scale0 norm(wte[tok[m]]) (fp32, row-major), act[m] = dtype copy (row-major, or
// blocked with rows rounded up to 32 when `blocked`), ss[m] = sum(x^2); with the later
// version's smear, the previous token's normalised embedding is mixed in first (row m is
// token m % T of batch row m / T at position lens[b] + m % T; hist [B][S] holds each row's
// tokens by position), and the unscaled result is x0.
struct EmbedArgs {
    const int32_t* tok; int M, T;
    const void* wte; int vocab, d;
    float eps, scale0;
    float* x; void* act; float* ss; bool blocked;
    const int32_t* lens;          // positions of each row's first token (null: 0)
    int32_t* hist; int S;         // token history (null: none)
    const void* smear_gate; int smear_ch; float smear_lambda;  // null gate: no smear
    float* x0;                    // stream before the layer-0 scaling (null: not written)
    float* xb;                    // copy of x (backout source at layer 0; null: none)
    int32_t* tok_out;             // the clamped token of each row (null: not written)
};
hipError_t launch_embed(DType dt, const EmbedArgs& a, hipStream_t st);

// Pre-attention finish of the raw QKV product part[z][m][(H+2 nkv)*hd] (H query heads, then
// nkv key heads, then nkv value heads): scale row m by r_m, rotate the q and k heads at
// position pos(m), QK-normalise, write q [m][H][hd] and k, v into the cache of the layer.
// Token m is token m % T of batch row b = m / T, at position pos = lens[b] + m % T (the
// row's current length, 0 when lens is null).
// Value embedding of a layer (the later version's blocks; ve null: none): value head j of
// row m gains 3 sigmoid(r_m xin[m][:ve_ch] . ve_gate[j]) ve[tok[m]][j hd .. (j + 1) hd),
// r_m xin the row's attention input (xin fp32 with row stride xin_stride, ve_ch <= 64);
// ve [vocab][nkv hd] and ve_gate [nkv][ve_ch] in the model dtype; tok[m] the row's token
// (clamped into the vocabulary by the embedding kernel that writes it).
struct ValueEmbed {
    const void* ve; const void* ve_gate; int ve_ch, vocab;
    const int32_t* tok; const float* xin; int xin_stride;
};

struct QkvPostArgs {
    const float* part; int splits; long long z_stride;
    int M, T, H, hd, nkv;
    const float* ss_in; int ss_in_parts, ss_stride, norm_dim;
    const int32_t* lens;
    const float* rope_cos; const float* rope_sin; // [max_seq][hd/2]
    void* q;          // [M][H][hd]
    void* kc;         // K cache of this layer: [B][nkv][S][hd]
    void* vtc;        // V cache of this layer, transposed: [B][nkv][hd][S]
    int S;            // cache capacity (positions)
    float eps;
    ValueEmbed vemb;  // tok[m], xin row m
};
hipError_t launch_qkv_post(DType dt, const QkvPostArgs& a, hipStream_t st);

// QKV finish of a decode step (one token per row, at position lens[b]): adds the `splits`
// K slices of the raw product part[z * z_stride + b * (H + 2 nkv) hd + ...] in slice order,
// scales row b by its norm scale, rotates and QK-normalises the query and key heads, adds
// the layer's value embedding to the value heads; writes q [B][H][hd] and the key / value
// into this layer's cache at position lens[b].  One wave per (row, head slot).
struct DecFinishArgs {
    const float* part; long long z_stride;
    const float* ss_in;
    const int32_t* lens;
    const float* rope_cos; const float* rope_sin;  // [max_seq][hd/2]
    void* q;          // [B][H][hd]
    void* kc;         // [B][nkv][S][hd]
    void* vtc;        // [B][nkv][hd][S]
    const ValueEmbed* vemb;  // device memory (null: none); tok[b], xin row b
    int32_t* head_ctr;       // fused finish (launch_dec_gemm with a finish): one arrival
                             // counter per head slot, zero before the launch and left zero
    int splits, B, H, hd, nkv, S;
    int ss_in_parts, ss_stride, norm_dim;
    float eps;
};
hipError_t launch_qkv_finish_decode(DType dt, const DecFinishArgs& a, hipStream_t st);
// Whether the raw QKV product of M rows can finish in its own epilogue (launch_dec_gemm
// with `fin`): at most 32 rows, head_dim a multiple of 32, at most DEC_FIN_SLOTS head slots.
constexpr int DEC_FIN_SLOTS = 256;
bool dec_gemm_fuses_finish(DType dt, int M, int hd, int slots);

// Causal attention of a prefill of T tokens per row: q [B*T][H][hd], the queries of row b
// at positions off_b .. off_b + T - 1 (off_b = offs[b], or 0 when offs is null), the K/V
// of this layer in the cache (positions 0 .. off_b + T - 1, nkv heads; query head h reads
// K/V head h / (H / nkv)), y [B*T][H*hd].  window >= 0: a query at position p sees keys
// p - window .. p; window < 0: keys 0..p.
hipError_t launch_attn_prefill(DType dt, int hd, const void* q, const void* kc, const void* vtc,
                               void* y, int B, int T, int H, int nkv, int S, int window,
                               const int32_t* offs, hipStream_t st);

// Decode attention for one step: one query per row at position lens[b] against keys
// 0..lens[b] (or lens[b] - window .. lens[b] with a window >= 0) of each K/V head, the new
// key/value already in the cache (qkv_finish_decode).  The 64-key blocks of all (row, K/V
// head) units are split into equal runs, one per workgroup; a unit cut by run boundaries leaves partial softmax
// states that the run holding its last block merges.  y: [B][H hd] stored blocked
// (blocked_index, rows rounded up to 32).
struct DecAttnArgs {
    const void* q;        // finished queries [B][H][hd] (qkv_finish_decode)
    const int32_t* lens;  // position of each row's new token, already in the cache
    const void* kc; const void* vtc;  // this layer's cache: K [B][nkv][S][hd], V^T [B][nkv][hd][S]
    float* part;          // partial states [B nkv][max_slots][16 (hd + 2)]
    int32_t* flags;       // ready flags of the partial states [B nkv][max_slots]: zero before
                          // the first launch, and every launch leaves them zero
    void* y;              // attention output, blocked
    int B, H, hd, S, nkv; // query heads H = nkv G, G <= 16 per K/V head; B <= 128; S % 64 == 0
    int window;           // sliding window (< 0: the whole causal context)
    int max_slots;        // partial slots per unit, >= attn_decode_slots(B nkv, S)
    float scale_log2;     // set by the launcher
};
// Keys a query can see at most: min(S, window + 1), or S without a window.
int attn_decode_span(int S, int window);
int attn_decode_workgroups(int units, int S);  // grid of a launch over `units` (row, K/V head) units
int attn_decode_slots(int units, int S);       // partial slots per unit
hipError_t launch_attn_decode(DType dt, const DecAttnArgs& a, hipStream_t st);

hipError_t launch_argmax(const float* logits, int B, int V, int32_t* out, hipStream_t st);
// Token per row drawn with probabilities proportional to 2^(logit scale) over the logits at
// or above the top_k-th largest (top_k <= 0 or >= V: all), by the inverse of the
// cumulative distribution in token order at u[b] in [0, 1).
hipError_t launch_sample(const float* logits, int B, int V, float scale, int top_k, const float* u,
                         int32_t* out, hipStream_t st);
hipError_t launch_lens_add(int32_t* lens, int B, int32_t delta, int32_t set_value, hipStream_t st);
// p[0..n) = 0 (a fill kernel: no memset node when the caller captures the stream)
hipError_t launch_zero_i32(int32_t* p, long long n, hipStream_t st);
hipError_t launch_kv_export(DType dt, int hd, const void* kc, const void* vtc, void* k_out,
                            void* v_out, int B, int S, int S_out, hipStream_t st);

// Copy rows between two caches of one model (K [L][B][nkv][S][hd], V^T [L][B][nkv][hd][S],
// es bytes per element): pair i copies positions 0..len[i]-1 of source row src[i] into
// destination row dst[i] and sets lens_dst[dst[i]] = len[i].  The pairs' rows must not
// overlap when both caches are the same.
struct KvRowCopy {
    static constexpr int MAX = 128;
    int n;
    int32_t dst[MAX], src[MAX], len[MAX];
};
// hsrc / hdst: token histories [B][S] (both null: none), copied like the keys.
hipError_t launch_kv_copy_rows(const KvRowCopy& rc, const void* ksrc, const void* vsrc, void* kdst,
                               void* vdst, int L, int nkv, int hd, int es, int Bsrc, int Ssrc, int Bdst,
                               int Sdst, int32_t* lens_dst, const int32_t* hsrc, int32_t* hdst,
                               hipStream_t st);

}  // namespace nc
