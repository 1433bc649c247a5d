// QKV finish of a decode step for one head slot of one row (one wave), shared by the
// standalone finish kernel and the QKV product's fused epilogue.
//
// Head slot j of row b: slots 0..H-1 are query heads, H..H+nkv-1 key heads, the rest value
// heads.  Lane i < hd/2 holds the RoPE pair (i, i + hd/2): v1, v2 are the raw product at
// columns j hd + i and j hd + i + hd/2 (lanes past hd/2 pass anything).  Row b's norm
// scale comes from the partial sums of squares the previous residual epilogue left; a
// query / key head is rotated at position lens[b] and normalised over the head (QK-norm);
// a value head gets the layer's gated value embedding when there is one.  Query heads go
// to q, the new key / value into the cache at lens[b].  Sources: yelogs.com launch
// write-up, architecture answer (RoPE, QK-norm, norms without parameters); apidog.com/th
// guide, part 1 (value embeddings of the later version), part 6 (KV cache).
#pragma once
#include "common.h"
#include "kernels.h"

namespace nc {

template <typename T>
__device__ __forceinline__ void qkv_finish_head(const DecFinishArgs& a, int b, int j, int lane, float v1, float v2) {
    const int half = a.hd / 2;
    const bool act = lane < half;
    const int i = act ? lane : 0;
    const int pos = min(max(a.lens[b], 0), a.S - 1);  // capacity is checked by the host
    const bool is_q = j < a.H, is_k = !is_q && j < a.H + a.nkv;
    float c = 0.f, sn = 0.f;
    if (is_q || is_k) {
        c = a.rope_cos[(long long)pos * half + i];
        sn = a.rope_sin[(long long)pos * half + i];
    }
    float ssl = 0.f;
    for (int q = lane; q < a.ss_in_parts; q += 64) ssl += a.ss_in[(long long)q * a.ss_stride + b];
    const float r = 1.0f / sqrtf(wave_sum(ssl) / (float)a.norm_dim + a.eps);
    v1 = act ? v1 * r : 0.f;
    v2 = act ? v2 * r : 0.f;
    if (!is_q && !is_k) {  // value head: value embedding, then the transposed cache
        const int g = j - a.H - a.nkv;
        if (a.vemb) {
            const ValueEmbed& ve = *a.vemb;
            const float gt = value_embed_gate<T>((const T*)ve.ve_gate, g, ve.ve_ch,
                                                 ve.xin + (long long)b * ve.xin_stride, r, lane);
            const T* e = (const T*)ve.ve + ((long long)ve.tok[b] * a.nkv + g) * a.hd;
            v1 += act ? gt * to_f32(e[i]) : 0.f;
            v2 += act ? gt * to_f32(e[i + half]) : 0.f;
        }
        if (act) {
            T* vt = (T*)a.vtc + ((long long)b * a.nkv + g) * a.hd * a.S + pos;
            vt[(long long)i * a.S] = from_f32<T>(v1);
            vt[(long long)(i + half) * a.S] = from_f32<T>(v2);
        }
        return;
    }
    // query / key head: rotate, then normalise over the head
    const float o1 = v1 * c - v2 * sn;
    const float o2 = v1 * sn + v2 * c;
    const float rr = 1.0f / sqrtf(wave_sum(o1 * o1 + o2 * o2) / (float)a.hd + a.eps);
    if (act) {
        T* dst = is_q ? (T*)a.q + ((long long)b * a.H + j) * a.hd
                      : (T*)a.kc + (((long long)b * a.nkv + (j - a.H)) * a.S + pos) * a.hd;
        dst[i] = from_f32<T>(o1 * rr);
        dst[i + half] = from_f32<T>(o2 * rr);
    }
}

}  // namespace nc
