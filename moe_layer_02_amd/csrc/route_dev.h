// route_dev.h -- router top-k of one token by one wavefront (route.hip, prologue.hip).
//
// Softmax / sigmoid top-k and the DeepSeek-V3 biased grouped gate (SGLang PR #3191 "Add
// deepseek_v3 fused gate").  Each lane holds up to four experts (lane l: l, l+64, l+128,
// l+192, so the logit row is read with consecutive lanes on consecutive addresses); every
// selection is a 64-lane butterfly arg-max over (key descending, expert index ascending),
// which gives one reproducible slot order -- the review of that PR asks why the order
// varied between runs.  Keys are compared exactly in fp32; the sigmoid is evaluated in fp64
// and rounded once so that a bias added to it cannot flip a selection on its last bit.
#pragma once

#include <float.h>
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace route_dev {

enum { SOFTMAX = 0, SIGMOID = 1, GROUPED = 2 };

__device__ __forceinline__ bool ranks_before(float ka, int ia, float kb, int ib) {
    return ka > kb || (ka == kb && ia < ib);
}

// Butterfly arg-max over the wave; every lane ends with the winner and its payload.
__device__ __forceinline__ void wave_argmax(float &key, int &idx, float &val) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float ok = __shfl_xor(key, off, kWave);
        const int oi = __shfl_xor(idx, off, kWave);
        const float ov = __shfl_xor(val, off, kWave);
        if (ranks_before(ok, oi, key, idx)) {
            key = ok;
            idx = oi;
            val = ov;
        }
    }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
    return v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

__device__ __forceinline__ float sigmoid_f64_rounded(float x) {
    return (float)(1.0 / (1.0 + exp(-(double)x)));
}

// Route token t with the calling wavefront (every lane of the wave must call).
template <int EPL>
__device__ __forceinline__ void route_token(const RouteArgs &a, int t) {
    const int lane = lane_id();
    const int E = a.E;

    float key[EPL], val[EPL];
    bool live[EPL];   // expert exists, is allowed (grouped gate) and not yet taken
    float xmax = -FLT_MAX;
#pragma unroll
    for (int i = 0; i < EPL; i++) {
        const int e = lane + kWave * i;
        float x = -FLT_MAX;
        live[i] = e < E;
        if (live[i]) {
            x = a.logits_bf16 ? bf16_bits_to_f32(((const uint16_t *)a.logits)[(int64_t)t * E + e])
                              : ((const float *)a.logits)[(int64_t)t * E + e];
        }
        if (a.kind == SOFTMAX) {
            key[i] = live[i] ? x : -INFINITY;
            val[i] = x;
            if (live[i]) xmax = fmaxf(xmax, x);
        } else {
            const float s = live[i] ? sigmoid_f64_rounded(x) : 0.0f;
            key[i] = live[i] ? (a.bias ? s + a.bias[e] : s) : -INFINITY;
            val[i] = s;
        }
    }

    // softmax normaliser in fp64: p_e = exp(x_e - max) / sum_all exp(x_e' - max)
    double m = 0.0, z = 1.0;
    if (a.kind == SOFTMAX) {
        m = (double)wave_max(xmax);
        double part = 0.0;
#pragma unroll
        for (int i = 0; i < EPL; i++)
            if (live[i]) part += exp((double)key[i] - m);
        z = wave_sum(part);
    }

    if (a.kind == GROUPED && (E / a.n_group) <= kWave && ((E / a.n_group) & (E / a.n_group - 1)) == 0) {
        // Groups of G = 2^s <= 64 consecutive experts lie inside one slot on G consecutive
        // lanes, so every group's two largest keys come from segmented butterflies (xor
        // offsets < G) over all slots at once.
        const int G = E / a.n_group;
        float score[EPL];
#pragma unroll
        for (int i = 0; i < EPL; i++) {
            const int e = lane + kWave * i;
            float k1 = live[i] ? key[i] : -INFINITY;
            int i1 = live[i] ? e : INT32_MAX;
            for (int off = G >> 1; off >= 1; off >>= 1) {
                const float ok = __shfl_xor(k1, off, kWave);
                const int oi = __shfl_xor(i1, off, kWave);
                if (ranks_before(ok, oi, k1, i1)) { k1 = ok; i1 = oi; }
            }
            float k2 = (live[i] && e != i1) ? key[i] : -INFINITY;
            int i2 = (live[i] && e != i1) ? e : INT32_MAX;
            for (int off = G >> 1; off >= 1; off >>= 1) {
                const float ok = __shfl_xor(k2, off, kWave);
                const int oi = __shfl_xor(i2, off, kWave);
                if (ranks_before(ok, oi, k2, i2)) { k2 = ok; i2 = oi; }
            }
            score[i] = G >= 2 ? k1 + k2 : k1;
        }
        // keep the topk_group best groups; the first lane of each segment stands for its group
        uint64_t kept = 0;
        for (int q = 0; q < a.topk_group; q++) {
            float gk = -INFINITY, gv = 0.0f;
            int gi = INT32_MAX;
#pragma unroll
            for (int i = 0; i < EPL; i++) {
                const int e = lane + kWave * i, g = e / G;
                if (e < E && (lane % G) == 0 && !((kept >> g) & 1ull) && ranks_before(score[i], g, gk, gi)) {
                    gk = score[i];
                    gi = g;
                }
            }
            wave_argmax(gk, gi, gv);
            kept |= 1ull << gi;
        }
#pragma unroll
        for (int i = 0; i < EPL; i++) {
            const int e = lane + kWave * i;
            if (live[i] && !((kept >> (e / G)) & 1ull)) live[i] = false;
        }
    } else if (a.kind == GROUPED) {
        // general group size: group score = sum of the group's two largest keys, from two
        // wave-wide arg-max rounds per group; lane g keeps group g's score
        const int G = E / a.n_group;
        float my_score = -INFINITY;
        for (int g = 0; g < a.n_group; g++) {
            float k1 = -INFINITY, v1 = 0.0f;
            int i1 = INT32_MAX;
#pragma unroll
            for (int i = 0; i < EPL; i++) {
                const int e = lane + kWave * i;
                if (live[i] && e / G == g && ranks_before(key[i], e, k1, i1)) {
                    k1 = key[i];
                    i1 = e;
                }
            }
            wave_argmax(k1, i1, v1);
            float score = k1;
            if (G >= 2) {
                float k2 = -INFINITY, v2 = 0.0f;
                int i2 = INT32_MAX;
#pragma unroll
                for (int i = 0; i < EPL; i++) {
                    const int e = lane + kWave * i;
                    if (live[i] && e / G == g && e != i1 && ranks_before(key[i], e, k2, i2)) {
                        k2 = key[i];
                        i2 = e;
                    }
                }
                wave_argmax(k2, i2, v2);
                score = k1 + k2;
            }
            if (lane == g) my_score = score;
        }
        // keep the topk_group best groups
        uint64_t kept = 0;
        bool gfree = lane < a.n_group;
        for (int q = 0; q < a.topk_group; q++) {
            float gk = gfree ? my_score : -INFINITY;
            int gi = gfree ? lane : INT32_MAX;
            float gv = 0.0f;
            wave_argmax(gk, gi, gv);
            kept |= 1ull << gi;
            if (lane == gi) gfree = false;
        }
#pragma unroll
        for (int i = 0; i < EPL; i++) {
            const int e = lane + kWave * i;
            if (live[i] && !((kept >> (e / G)) & 1ull)) live[i] = false;
        }
    }

    // k rounds of arg-max; slot j is kept by lane j
    int my_id = 0;
    double my_val = 0.0, norm = 0.0;
    for (int j = 0; j < a.k; j++) {
        float bk = -INFINITY, bv = 0.0f;
        int bi = INT32_MAX;
#pragma unroll
        for (int i = 0; i < EPL; i++) {
            const int e = lane + kWave * i;
            if (live[i] && ranks_before(key[i], e, bk, bi)) {
                bk = key[i];
                bi = e;
                bv = val[i];
            }
        }
        wave_argmax(bk, bi, bv);
#pragma unroll
        for (int i = 0; i < EPL; i++)
            if (lane + kWave * i == bi) live[i] = false;
        const double v = a.kind == SOFTMAX ? exp((double)bv - m) / z : (double)bv;
        norm += v;
        if (lane == j) {
            my_id = bi;
            my_val = v;
        }
    }
    if (lane < a.k) {
        const double w = a.renorm ? my_val / norm : my_val;
        a.ids[(int64_t)t * a.k + lane] = my_id;
        a.weights[(int64_t)t * a.k + lane] = (float)(w * (double)a.scale);
    }
}

}  // namespace route_dev
}  // namespace moe
