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
// compiled variants: the routing mode, with the grouped gate split by its group size
enum { V_SOFTMAX = 0, V_SIGMOID = 1, V_GROUPED_POW2 = 2, V_GROUPED_ANY = 3 };

// The variant that routes cfg: the grouped gate's fast path needs groups of 2^g <= 64 experts.
__host__ __device__ inline int route_variant(int kind, int E, int n_group) {
    if (kind == SOFTMAX) return V_SOFTMAX;
    if (kind == SIGMOID) return V_SIGMOID;
    const int G = E / n_group;
    return (G <= 64 && (G & (G - 1)) == 0) ? V_GROUPED_POW2 : V_GROUPED_ANY;
}

// Lane exchanges without LDS: step S pairs every lane with one partner so that steps
// 0..g-1 combine all lanes of each aligned group of 2^g (g <= 6).  Steps 0-3 are DPP moves
// (xor 1, xor 2, mirror within 8, mirror within 16); steps 4 and 5 are gfx950's
// v_permlane16_swap / v_permlane32_swap, whose two results hold, for each lane, its own
// value and its partner's (lane l and l ^ 16, resp. l ^ 32); which of the two is the
// partner depends on the lane's half.
template <int S>
__device__ __forceinline__ int partner(int x) {
    if constexpr (S == 0) return __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xf, 0xf, false);    // quad_perm [1,0,3,2]
    if constexpr (S == 1) return __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xf, 0xf, false);    // quad_perm [2,3,0,1]
    if constexpr (S == 2) return __builtin_amdgcn_update_dpp(0, x, 0x141, 0xf, 0xf, false);   // row_half_mirror
    if constexpr (S == 3) return __builtin_amdgcn_update_dpp(0, x, 0x140, 0xf, 0xf, false);   // row_mirror
    if constexpr (S == 4) {
        const auto p = __builtin_amdgcn_permlane16_swap(x, x, false, false);
        return (lane_id() & 16) ? p[0] : p[1];
    }
    if constexpr (S == 5) {
        const auto p = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        return (lane_id() & 32) ? p[0] : p[1];
    }
    return x;
}
template <int S>
__device__ __forceinline__ float partner(float x) { return __int_as_float(partner<S>(__float_as_int(x))); }
template <int S>
__device__ __forceinline__ double partner(double x) {
    const int64_t b = __double_as_longlong(x);
    const int lo = partner<S>((int)b), hi = partner<S>((int)(b >> 32));
    return __longlong_as_double(((int64_t)hi << 32) | (uint32_t)lo);
}

template <int S>
__device__ __forceinline__ uint64_t partner(uint64_t x) {
    const uint32_t lo = (uint32_t)partner<S>((int)(uint32_t)x), hi = (uint32_t)partner<S>((int)(uint32_t)(x >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// A candidate (key, index) as one unsigned 64-bit rank whose integer order is the
// selection order (key descending, index ascending): the key's bits mapped to an
// order-preserving unsigned word (-0 folded into +0, so that equal keys stay equal) above
// the complement of the index.  0 ranks below every candidate: no candidate.  One wave
// step then moves two words and compares once, where moving key, index and payload and
// comparing (key, index) took about twice the instructions (four cycles each per wave).
__device__ __forceinline__ uint64_t rank_of(float key, int idx) {
    uint32_t u = __float_as_uint(key + 0.0f);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint32_t)~(uint32_t)idx;
}
__device__ __forceinline__ int rank_index(uint64_t r) { return r ? (int)~(uint32_t)r : INT32_MAX; }
__device__ __forceinline__ float rank_key(uint64_t r) {
    if (!r) return -INFINITY;
    const uint32_t u = (uint32_t)(r >> 32);
    return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// One arg-max step: both lanes of a pair keep the larger rank.
template <int S>
__device__ __forceinline__ void argmax_step(uint64_t &r) {
    const uint64_t o = partner<S>(r);
    if (o > r) r = o;
}

// Arg-max over each aligned group of 2^g lanes (g <= 6, wave-uniform) for N independent
// ranks, step by step over all N so that their dependency chains interleave; every lane of
// a group ends with the group's winner.
template <int N>
__device__ __forceinline__ void group_argmax_n(uint64_t (&r)[N], int g) {
#pragma unroll
    for (int i = 0; i < N; i++)
        if (g > 0) argmax_step<0>(r[i]);
#pragma unroll
    for (int i = 0; i < N; i++)
        if (g > 1) argmax_step<1>(r[i]);
#pragma unroll
    for (int i = 0; i < N; i++)
        if (g > 2) argmax_step<2>(r[i]);
#pragma unroll
    for (int i = 0; i < N; i++)
        if (g > 3) argmax_step<3>(r[i]);
#pragma unroll
    for (int i = 0; i < N; i++)
        if (g > 4) argmax_step<4>(r[i]);
#pragma unroll
    for (int i = 0; i < N; i++)
        if (g > 5) argmax_step<5>(r[i]);
}

__device__ __forceinline__ uint64_t wave_argmax(uint64_t r) {
    argmax_step<0>(r);
    argmax_step<1>(r);
    argmax_step<2>(r);
    argmax_step<3>(r);
    argmax_step<4>(r);
    argmax_step<5>(r);
    return r;
}

// A key's order-preserving unsigned image (-0 folded into +0, as in rank_of); 0 stands for
// no candidate (every key maps above it).  code_key inverts it.
__device__ __forceinline__ uint32_t key_code(float key) {
    const uint32_t u = __float_as_uint(key + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float code_key(uint32_t u) {
    if (!u) return -INFINITY;
    return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// Maximum of 32-bit codes over each aligned group of 2^g lanes (g <= 6), for N independent
// codes step by step; every lane of a group ends with the group's maximum.  A selection
// round is a 32-bit maximum followed by one ballot per slot that names the smallest index
// holding it -- the same (key descending, index ascending) order as the 64-bit ranks in
// about a quarter of the instructions of a 64-bit arg-max.
template <int S>
__device__ __forceinline__ void max_step(uint32_t &u) {
    const uint32_t o = (uint32_t)partner<S>((int)u);
    u = o > u ? o : u;
}
template <int N>
__device__ __forceinline__ void group_max_n(uint32_t (&u)[N], int g) {
#pragma unroll
    for (int i = 0; i < N; i++)
        if (g > 0) max_step<0>(u[i]);
#pragma unroll
    for (int i = 0; i < N; i++)
        if (g > 1) max_step<1>(u[i]);
#pragma unroll
    for (int i = 0; i < N; i++)
        if (g > 2) max_step<2>(u[i]);
#pragma unroll
    for (int i = 0; i < N; i++)
        if (g > 3) max_step<3>(u[i]);
#pragma unroll
    for (int i = 0; i < N; i++)
        if (g > 4) max_step<4>(u[i]);
#pragma unroll
    for (int i = 0; i < N; i++)
        if (g > 5) max_step<5>(u[i]);
}
__device__ __forceinline__ uint32_t wave_max_code(uint32_t u) {
    max_step<0>(u);
    max_step<1>(u);
    max_step<2>(u);
    max_step<3>(u);
    max_step<4>(u);
    max_step<5>(u);
    return u;
}
// The lowest lane of mask inside this lane's aligned group of 2^g lanes (64: none).
__device__ __forceinline__ int group_first_lane(uint64_t mask, int g) {
    const int base = g >= 6 ? 0 : (lane_id() & ~((1 << g) - 1));
    const uint64_t span = g >= 6 ? ~0ull : (((1ull << (1 << g)) - 1) << base);
    const uint64_t s = mask & span;
    return s ? __builtin_ctzll(s) : 64;
}

__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, partner<0>(v));
    v = fmaxf(v, partner<1>(v));
    v = fmaxf(v, partner<2>(v));
    v = fmaxf(v, partner<3>(v));
    v = fmaxf(v, partner<4>(v));
    return fmaxf(v, partner<5>(v));
}

// Sum over the wave in a fixed tree (lane pairs add in the same order on both sides, so
// every lane ends with the same value).
__device__ __forceinline__ double wave_sum(double v) {
    double o;
    o = partner<0>(v); v = (lane_id() & 1) ? o + v : v + o;
    o = partner<1>(v); v = (lane_id() & 2) ? o + v : v + o;
    o = partner<2>(v); v = (lane_id() & 4) ? o + v : v + o;
    o = partner<3>(v); v = (lane_id() & 8) ? o + v : v + o;
    o = partner<4>(v); v = (lane_id() & 16) ? o + v : v + o;
    o = partner<5>(v); v = (lane_id() & 32) ? o + v : v + o;
    return v;
}

__device__ __forceinline__ float sigmoid_f64_rounded(float x) {
    return (float)(1.0 / (1.0 + exp(-(double)x)));
}

// Route token t with the calling wavefront (every lane of the wave must call); V is
// route_variant(a.kind, a.E, a.n_group).  Returns, on lane j < k, the expert of slot j.
template <int EPL, int V>
__device__ __forceinline__ int route_token(const RouteArgs &a, int t) {
    constexpr bool softmax = V == V_SOFTMAX;
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
        if constexpr (softmax) {
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
    if constexpr (softmax) {
        m = (double)wave_max(xmax);
        double part = 0.0;
#pragma unroll
        for (int i = 0; i < EPL; i++)
            if (live[i]) part += exp((double)key[i] - m);
        z = wave_sum(part);
    }

    if constexpr (V == V_GROUPED_POW2) {
        // Groups of G = 2^g <= 64 consecutive experts lie inside one slot on G consecutive
        // lanes, so every group's two largest keys come from arg-max steps confined to
        // aligned groups of G lanes, for all slots at once.
        const int G = E / a.n_group;
        const int gbits = __builtin_ctz(G);
        float score[EPL];
        uint32_t u[EPL], m1[EPL], m2[EPL];
#pragma unroll
        for (int i = 0; i < EPL; i++) {
            u[i] = live[i] ? key_code(key[i]) : 0u;
            m1[i] = u[i];
        }
        group_max_n(m1, gbits);
        // the second key: the group's largest without its first (lowest-index) holder of the
        // largest, so a tie keeps the value
#pragma unroll
        for (int i = 0; i < EPL; i++) {
            const uint64_t at = __ballot(u[i] != 0u && u[i] == m1[i]);
            m2[i] = lane == group_first_lane(at, gbits) ? 0u : u[i];
        }
        group_max_n(m2, gbits);
#pragma unroll
        for (int i = 0; i < EPL; i++) score[i] = G >= 2 ? code_key(m1[i]) + code_key(m2[i]) : code_key(m1[i]);
        // keep the topk_group best groups (ties: the lower group); the first lane of each
        // segment stands for its group
        uint64_t kept = 0;
        for (int q = 0; q < a.topk_group; q++) {
            uint32_t sc[EPL], m = 0u;
#pragma unroll
            for (int i = 0; i < EPL; i++) {
                const int e = lane + kWave * i, g = e / G;
                sc[i] = (e < E && (lane % G) == 0 && !((kept >> g) & 1ull)) ? key_code(score[i]) : 0u;
                m = sc[i] > m ? sc[i] : m;
            }
            m = wave_max_code(m);
            if (!m) break;
#pragma unroll
            for (int i = 0; i < EPL; i++) {
                const uint64_t at = __ballot(sc[i] == m);
                if (at) {
                    kept |= 1ull << ((__builtin_ctzll(at) + kWave * i) / G);
                    break;
                }
            }
        }
#pragma unroll
        for (int i = 0; i < EPL; i++) {
            const int e = lane + kWave * i;
            if (live[i] && !((kept >> (e / G)) & 1ull)) live[i] = false;
        }
    } else if constexpr (V == V_GROUPED_ANY) {
        // general group size: group score = sum of the group's two largest keys, from two
        // wave-wide arg-max rounds per group; lane g keeps group g's score
        const int G = E / a.n_group;
        float my_score = -INFINITY;
        for (int g = 0; g < a.n_group; g++) {
            uint64_t r1 = 0;
#pragma unroll
            for (int i = 0; i < EPL; i++) {
                const int e = lane + kWave * i;
                if (live[i] && e / G == g) {
                    const uint64_t c = rank_of(key[i], e);
                    if (c > r1) r1 = c;
                }
            }
            r1 = wave_argmax(r1);
            float score = rank_key(r1);
            if (G >= 2) {
                const int i1 = rank_index(r1);
                uint64_t r2 = 0;
#pragma unroll
                for (int i = 0; i < EPL; i++) {
                    const int e = lane + kWave * i;
                    if (live[i] && e / G == g && e != i1) {
                        const uint64_t c = rank_of(key[i], e);
                        if (c > r2) r2 = c;
                    }
                }
                score = rank_key(r1) + rank_key(wave_argmax(r2));
            }
            if (lane == g) my_score = score;
        }
        // keep the topk_group best groups
        uint64_t kept = 0;
        bool gfree = lane < a.n_group;
        for (int q = 0; q < a.topk_group; q++) {
            const int gi = rank_index(wave_argmax(gfree ? rank_of(my_score, lane) : 0));
            kept |= 1ull << gi;
            if (lane == gi) gfree = false;
        }
#pragma unroll
        for (int i = 0; i < EPL; i++) {
            const int e = lane + kWave * i;
            if (live[i] && !((kept >> (e / G)) & 1ull)) live[i] = false;
        }
    }

    // k rounds of arg-max; slot j is kept by lane j (its expert and the winner's logit or
    // score).  The slot weights are computed afterwards, each on its own lane, so that the
    // fp64 exp of a softmax slot is not on the chain of arg-max rounds.
    int my_id = 0;
    float my_bv = 0.0f;
    uint32_t uk[EPL];   // the candidates' codes, 0 once taken or not allowed
#pragma unroll
    for (int i = 0; i < EPL; i++) uk[i] = live[i] ? key_code(key[i]) : 0u;
    for (int j = 0; j < a.k; j++) {
        uint32_t m = uk[0];
#pragma unroll
        for (int i = 1; i < EPL; i++) m = uk[i] > m ? uk[i] : m;
        m = wave_max_code(m);
        // the smallest index holding the largest key, and its payload (bi is the same on
        // every lane)
        int bi = INT32_MAX;
        float bv = 0.0f;
        if (m) {
#pragma unroll
            for (int i = 0; i < EPL; i++) {
                const uint64_t at = __ballot(uk[i] == m);
                if (at) {
                    const int l = __builtin_ctzll(at);
                    bi = l + kWave * i;
                    bv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(val[i]), l));
                    break;
                }
            }
        }
#pragma unroll
        for (int i = 0; i < EPL; i++)
            if (lane + kWave * i == bi) uk[i] = 0u;
        if (lane == j) {
            my_id = bi;
            my_bv = bv;
        }
    }
    const double my_val = softmax ? exp((double)my_bv - m) / z : (double)my_bv;
    double norm = 0.0;   // summed over the slots in order 0 .. k-1 (lane reads, not LDS shuffles)
    const int64_t vb = __double_as_longlong(my_val);
    for (int j = 0; j < a.k; j++) {
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)vb, j);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(vb >> 32), j);
        norm += __longlong_as_double((int64_t)(((uint64_t)hi << 32) | lo));
    }
    if (lane < a.k) {
        const double w = a.renorm ? my_val / norm : my_val;
        a.ids[(int64_t)t * a.k + lane] = my_id;
        a.weights[(int64_t)t * a.k + lane] = (float)(w * (double)a.scale);
    }
    return my_id;
}

}  // namespace route_dev
}  // namespace moe
