// reduce.hip -- unpermute and reduce: each token's k weighted expert rows summed back to
// token order, in a fixed order, with no floating-point atomics.
//
// TensorRT-LLM's unpermute_and_reduce (named in the last review comment of SGLang PR #3191
// "Add deepseek_v3 fused gate") returns the permuted rows to their tokens.  Here each thread
// owns 8 consecutive columns of one token and adds, for j = 0..k-1 and then split s =
// 0..S-1, the row inv_pos[t*k + j] -- the same order on every run, so the result is bitwise
// reproducible; SGLang PR #2333 ("[kernel] introduce fused_moe_triton_splitk", Background)
// shows what an unordered atomic_add of the same partial sums did to the output.  The same
// file finishes a K-split GEMM1: its split planes of gate and up sums are added in a fixed
// order before SiLU * up.
#include "common.h"
#include "kernels.h"
#include "quant_dev.h"

namespace moe {
namespace {

constexpr int kReduceMaxK = 8;   // top-k up to this: the rows' loads are issued together

__global__ __launch_bounds__(256) void k_reduce(ReduceArgs a) {
    const int c8 = a.H / 8;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t t = gid / c8;
    const int col = (int)(gid % c8) * 8;
    if (t >= a.T) return;
    // GEMM2's split tail: rows from tail_row0 on are tail_s fp32 planes
    int64_t tail_row0 = INT64_MAX, tail_plane = 0;
    int tail_s = 0;
    if (a.tail_info && a.tail_info[1] > 0) {
        tail_row0 = a.tail_info[0];
        tail_s = a.tail_info[1];
        tail_plane = a.tail_info[2];
    }
    if (a.direct && a.inv_pos[t] < tail_row0) return;   // top-1: GEMM2 wrote this token
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (a.split == 0 && a.k <= kReduceMaxK) {
        // bf16 rows: every row's load is issued before the first add, so a thread keeps k
        // loads in flight instead of one (the adds keep the order j = 0, 1, ...)
        int64_t row[kReduceMaxK];
        uint4 v[kReduceMaxK];
#pragma unroll
        for (int j = 0; j < kReduceMaxK; j++)
            if (j < a.k) row[j] = a.inv_pos[t * a.k + j];
#pragma unroll
        for (int j = 0; j < kReduceMaxK; j++)
            if (j < a.k && row[j] < tail_row0) v[j] = *(const uint4 *)((const uint16_t *)a.Y + row[j] * a.H + col);
#pragma unroll
        for (int j = 0; j < kReduceMaxK; j++) {
            if (j >= a.k) break;
            if (row[j] >= tail_row0) {
                for (int s = 0; s < tail_s; s++) {
                    const float *p = a.tail_P + s * tail_plane + (row[j] - tail_row0) * a.H + col;
                    const float4 lo = *(const float4 *)p, hi = *(const float4 *)(p + 4);
                    acc[0] += lo.x; acc[1] += lo.y; acc[2] += lo.z; acc[3] += lo.w;
                    acc[4] += hi.x; acc[5] += hi.y; acc[6] += hi.z; acc[7] += hi.w;
                }
            } else {
                const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    acc[2 * i] += __uint_as_float(w[i] << 16);
                    acc[2 * i + 1] += __uint_as_float(w[i] & 0xFFFF0000u);
                }
            }
        }
    } else {
    for (int j = 0; j < a.k; j++) {
        const int64_t row = a.inv_pos[t * a.k + j];
        if (row >= tail_row0) {
            for (int s = 0; s < tail_s; s++) {
                const float *p = a.tail_P + s * tail_plane + (row - tail_row0) * a.H + col;
                const float4 lo = *(const float4 *)p, hi = *(const float4 *)(p + 4);
                acc[0] += lo.x; acc[1] += lo.y; acc[2] += lo.z; acc[3] += lo.w;
                acc[4] += hi.x; acc[5] += hi.y; acc[6] += hi.z; acc[7] += hi.w;
            }
        } else if (a.split == 0) {
            const uint4 v = *(const uint4 *)((const uint16_t *)a.Y + row * a.H + col);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; i++) {
                acc[2 * i] += __uint_as_float(w[i] << 16);
                acc[2 * i + 1] += __uint_as_float(w[i] & 0xFFFF0000u);
            }
        } else {
            for (int s = 0; s < a.split; s++) {
                const float *p = (const float *)a.Y + s * a.partial_stride + row * a.H + col;
                const float4 lo = *(const float4 *)p, hi = *(const float4 *)(p + 4);
                acc[0] += lo.x; acc[1] += lo.y; acc[2] += lo.z; acc[3] += lo.w;
                acc[4] += hi.x; acc[5] += hi.y; acc[6] += hi.z; acc[7] += hi.w;
            }
        }
    }
    }
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    *(uint4 *)(a.out + t * a.H + col) = o;
}

// GEMM1 split K: h[r, c] = SiLU(sum_s G_s[r, c]) * sum_s U_s[r, c] over the split planes in
// order s = 0, 1, ... (the same SiLU as the unsplit epilogue), 8 columns per thread, valid
// rows only; fp32 h also folds its |h| maximum (one atomic per workgroup, max is exact).
__global__ __launch_bounds__(256) void k_gate_up_finish(GateUpFinishArgs a) {
    const int64_t c8 = a.I / 8;
    int64_t r0 = 0, plane = a.plane;
    int split = a.split;
    if (a.tail_info) {   // GEMM1's split tail: its rows only (the same for the whole grid)
        r0 = a.tail_info[0];
        split = a.tail_info[1];
        plane = a.tail_info[2];
        if (split == 0) return;
    }
    // the padded layout's rows up to its end (filler rows skipped), or the T*k rows of the
    // layout without padding (every one a pair)
    const int64_t rows = (a.ragged ? (int64_t)a.pairs : (int64_t)*a.npp) - r0;
    float m = 0.0f;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < rows * c8; i += (int64_t)gridDim.x * 256) {
        const int64_t pr = i / c8, r = r0 + pr;   // plane row, sorted row
        const int c = (int)(i % c8) * 8;
        if (!a.ragged && a.sorted[r] >= a.pairs) continue;
        float g[8], u[8];
        for (int s = 0; s < split; s++) {
            const float *p = a.P + s * plane + pr * 2 * (int64_t)a.I;
            const float4 g0 = *(const float4 *)(p + c), g1 = *(const float4 *)(p + c + 4);
            const float4 u0 = *(const float4 *)(p + a.I + c), u1 = *(const float4 *)(p + a.I + c + 4);
            const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
            const float uv[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
            for (int j = 0; j < 8; j++) {
                g[j] = s ? g[j] + gv[j] : gv[j];
                u[j] = s ? u[j] + uv[j] : uv[j];
            }
        }
        float h[8];
#pragma unroll
        for (int j = 0; j < 8; j++) h[j] = silu(g[j]) * u[j];
        if (a.h_kind == GATE_UP_H_F32) {
            float *o = (float *)a.h + r * a.I + c;
            *(float4 *)o = make_float4(h[0], h[1], h[2], h[3]);
            *(float4 *)(o + 4) = make_float4(h[4], h[5], h[6], h[7]);
#pragma unroll
            for (int j = 0; j < 8; j++) m = fmaxf(m, fabsf(h[j]));
        } else if (a.h_kind == GATE_UP_H_BF16_PERM) {   // bf16, order (0,4,1,5,2,6,3,7) in the 8
            *(uint4 *)((uint16_t *)a.h + r * a.I + c) =
                make_uint4(pack_bf16x2(h[0], h[4]), pack_bf16x2(h[1], h[5]), pack_bf16x2(h[2], h[6]),
                           pack_bf16x2(h[3], h[7]));
        } else {
            *(uint4 *)((uint16_t *)a.h + r * a.I + c) =
                make_uint4(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]), pack_bf16x2(h[4], h[5]),
                           pack_bf16x2(h[6], h[7]));
        }
    }
    if (a.h_kind == GATE_UP_H_F32 && a.amax) {
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
        __shared__ float wmax[4];
        if (lane_id() == 0) wmax[threadIdx.x >> 6] = m;
        __syncthreads();
        if (threadIdx.x == 0) amax_raise(a.amax, amax_peek(a.amax), fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3])));
    }
}

// A small fp8 batch: the finish above and the quantisation of h (quant.hip) in one
// workgroup -- every valid pair's h row (through inv_pos) in fp32 with |h| folded, then
// after a barrier the same rows as E4M3 codes with the scale of that maximum.  Codes,
// scale and h are those of the two separate kernels.
__global__ __launch_bounds__(1024) void k_gate_up_finish_quant(GateUpFinishArgs a, const int32_t *inv_pos,
                                                                uint8_t *hq, float *scale_out) {
    const int c8 = a.I / 8;
    const int items = a.pairs * c8;
    float m = 0.0f;
    for (int it = threadIdx.x; it < items; it += 1024) {
        const int64_t r = inv_pos[it / c8];
        const int c = (it % c8) * 8;
        float g[8], u[8];
        for (int s = 0; s < a.split; s++) {
            const float *p = a.P + s * a.plane + r * 2 * (int64_t)a.I;
            const float4 g0 = *(const float4 *)(p + c), g1 = *(const float4 *)(p + c + 4);
            const float4 u0 = *(const float4 *)(p + a.I + c), u1 = *(const float4 *)(p + a.I + c + 4);
            const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
            const float uv[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
            for (int j = 0; j < 8; j++) {
                g[j] = s ? g[j] + gv[j] : gv[j];
                u[j] = s ? u[j] + uv[j] : uv[j];
            }
        }
        float h[8];
#pragma unroll
        for (int j = 0; j < 8; j++) {
            h[j] = silu(g[j]) * u[j];
            m = fmaxf(m, fabsf(h[j]));
        }
        float *o = (float *)a.h + r * a.I + c;
        *(float4 *)o = make_float4(h[0], h[1], h[2], h[3]);
        *(float4 *)(o + 4) = make_float4(h[4], h[5], h[6], h[7]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
    __shared__ float wmax[16];
    if (lane_id() == 0) wmax[threadIdx.x >> 6] = m;
    __syncthreads();
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; i++) amax = fmaxf(amax, wmax[i]);
    float scale, inv;
    quant_dev::scales_from_amax(__float_as_uint(amax), &scale, &inv);
    if (threadIdx.x == 0) {
        *a.amax = __float_as_uint(amax);
        *scale_out = scale;
    }
    for (int it = threadIdx.x; it < items; it += 1024) {
        const int64_t r = inv_pos[it / c8];
        const int c = (it % c8) * 8;
        const float *o = (const float *)a.h + r * a.I + c;
        const float4 lo = *(const float4 *)o, hi = *(const float4 *)(o + 4);
        uint2 q;
        q.x = quant_dev::e4m3x4(lo.x, lo.y, lo.z, lo.w, inv);
        q.y = quant_dev::e4m3x4(hi.x, hi.y, hi.z, hi.w, inv);
        *(uint2 *)(hq + r * a.I + c) = q;
    }
}

}  // namespace

hipError_t launch_gate_up_finish_quant(const GateUpFinishArgs &a, const int32_t *inv_pos, uint8_t *hq, float *scale_out,
                                       hipStream_t s) {
    hipLaunchKernelGGL(k_gate_up_finish_quant, dim3(1), dim3(1024), 0, s, a, inv_pos, hq, scale_out);
    return hipGetLastError();
}

hipError_t launch_gate_up_finish(const GateUpFinishArgs &a, int64_t max_rows, hipStream_t s) {
    int64_t blocks = (max_rows * (a.I / 8) + 255) / 256;
    const int64_t cap = (int64_t)device_cu_count() * 8;
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(k_gate_up_finish, dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_reduce(const ReduceArgs &a, hipStream_t s) {
    const int64_t threads = (int64_t)a.T * (a.H / 8);
    hipLaunchKernelGGL(k_reduce, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
