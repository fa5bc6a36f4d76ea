// kernels.h -- host-side launchers of the libmoe kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

struct RouteArgs {
    int T, E, k, kind, renorm, n_group, topk_group;
    float scale;
    int logits_bf16;             // 1: bf16 bits, 0: fp32
    const void *logits;
    const float *bias;           // may be null
    int32_t *ids;
    float *weights;
    uint32_t *zero_ptr;          // words cleared by the launch (scratch counters), may be null
    int zero_n;                  // <= 256
    // the hidden states [T, x_cols] bf16 where the route also reads them: fp8, one word per
    // workgroup receiving the largest |x| of its tokens as float bits (x_parts); int4, the
    // rows in the nibble order of the int4 GEMM's A (x_perm, [T, x_cols]); null: neither
    const uint16_t *x;
    int64_t x_cols;
    uint32_t *x_parts;
    uint16_t *x_perm;
};
hipError_t launch_route(const RouteArgs &a, hipStream_t s);

struct AlignArgs {
    int T, k, E, BM, nbits;
    int64_t cap;
    const int32_t *ids;
    int32_t *sorted, *eids, *npp, *counts, *inv_pos;
    // null: the padded layout; else no padding -- sorted holds the T*k pairs expert by
    // expert, and blk_start[b] the first row of block b (blocks cut at expert ends; T*k for
    // b past the last block, capacity / BM + 1 entries)
    int32_t *blk_start;
};
// scratch: align_scratch_bytes() of device memory for the multi-launch path (T*k above
// 65536; zero bytes below), or null to run such batches on the one-workgroup kernel
int64_t align_scratch_bytes(int64_t pairs, int E);
hipError_t launch_align(const AlignArgs &a, int32_t *scratch, hipStream_t s);

// One grouped GEMM over the align layout.  Rows of the M dimension are the sorted rows;
// block b (block_m rows) multiplies by the weights of expert expert_ids[b].
struct GemmArgs {
    const void *A;               // gate/up: hidden [T, H] (gathered); down: h [cap, I]
    int64_t lda;                 // elements of A per row
    const void *B;               // expert weights, [E, rows, K]
    int64_t ldb;                 // bytes per B row  (K elements, packed for int4)
    int64_t b_expert_stride;     // bytes per expert
    const uint16_t *bs, *bz;     // int4: fp16 scales / zeros [E, rows, K/128]
    int64_t sz_expert_stride;    // int4: elements per expert of bs / bz
    void *C;                     // gate/up: h [cap, N] bf16 (fp8: fp32); down: out rows [cap, N] bf16 or fp32 partials
    int64_t ldc;                 // elements per row of C
    int64_t partial_stride;      // elements between split-K partial planes
    const int32_t *sorted, *eids, *npp;
    const int32_t *blk_start;    // null: padded layout (block b = rows b*BM ..); else block b = rows
                                 // [blk_start[b], blk_start[b + 1]) of one expert, at most BM
    const float *topk_w;         // down: pair weights
    int K, N;                    // reduction length; output columns
    int I;                       // gate/up: offset of the up rows in w13
    int top_k, pairs;            // pairs = T*k (the filler value)
    int split, ksplit;           // number of K splits and the K length of each
    const float *a_scale;        // fp8: activation scale (device scalar)
    const float *b_scale;        // fp8: per-expert weight scales [E]
    uint32_t *amax_out;          // fp8 gate/up: |h| max as float bits (atomicMax), may be null
    int group_m;                 // tile order: blocks per group (set by the launcher)
    int rotate_k;                // 1: each tile starts its K walk at its own offset
    int out_by_pair;             // down, no split: write row p = sorted[row] of C (top-1: the token's output row)
    // down, no split, pipelined bf16/fp8 tiles: an at most half-full last round of tiles is
    // computed as up to tail_split K splits into fp32 planes (tail_split < 2: never)
    int tail_split;
    int tail_cap;                // tiles x splits the planes hold (BM x BN fp32 each)
    float *tail_P;               // fp32 [S, tail rows, ldc]
    int32_t *tail_info;          // written by workgroup 0: first tail row, S (0: none), plane elements
    int expert_groups;           // > 0: tile groups of an expert's row blocks, at most this many (set by the launcher)
    int gather_a;                // down: A row of block row r is sorted[r] (not r); the grouped GEMM
};

enum GemmKind { GEMM_GATE_UP = 1, GEMM_DOWN = 2 };

// The rows [row0, row0 + n) of the intermediates (h, y, split planes) that row block mb
// covers: mb * BM and BM in the padded layout, the block table's entries without padding.
struct BlockRows {
    int row0, n;
};
__device__ __forceinline__ BlockRows block_rows(const GemmArgs &a, int mb, int BM) {
    if (a.blk_start) {
        const int s = a.blk_start[mb];
        return BlockRows{s, a.blk_start[mb + 1] - s};
    }
    return BlockRows{mb * BM, BM};
}
// The pair held by row r (0 <= r < BM) of the block: a.pairs (the filler value) for a
// padded layout's filler rows and for the rows past a block's end without padding (whose
// entries belong to the next block).
__device__ __forceinline__ int block_pair(const GemmArgs &a, BlockRows b, int r) {
    return r < b.n ? a.sorted[b.row0 + r] : a.pairs;
}
// The same without a branch around the load (a row past the block reads the block's first
// entry): the GEMM epilogues read a chunk of rows' pairs back to back.
__device__ __forceinline__ int block_pair_nb(const GemmArgs &a, BlockRows b, int r) {
    const int v = a.sorted[b.row0 + (r < b.n ? r : 0)];
    return r < b.n ? v : a.pairs;
}
// A loaded value taken into a register here: the wait for its load is placed at this point,
// once for a chunk of loads, instead of next to each row's stores, where the compiler would
// sink it and where it would also drain every store issued before (the wait counter counts
// stores too).  The GEMM epilogues read all of a chunk's pairs and weights, pin them, then
// store.
template <class T>
__device__ __forceinline__ void pin(T &v) {
    asm volatile("" : "+v"(v));
}
// Values of a chunk taken into registers G at a time, each group by one statement: the loads
// of a group are all in flight before its wait.  With a pin per value (G = 1) the compiler
// may, under register pressure, place the wait for one load (and the arithmetic that uses
// it) before it issues the next, one memory latency per value; a larger group keeps up to G
// more values live at once, which the register-tight tiles pay for in spills.
template <int G, class T, int N>
__device__ __forceinline__ void pin_groups(T (&v)[N]) {
    static_assert(N % G == 0 && (G == 1 || G == 4 || G == 8 || G == 16), "groups of 1, 4, 8 or 16");
#pragma unroll
    for (int c = 0; c < N; c += G) {
        if constexpr (G == 1) {
            asm volatile("" : "+v"(v[c]));
        } else if constexpr (G == 4) {
            asm volatile("" : "+v"(v[c]), "+v"(v[c + 1]), "+v"(v[c + 2]), "+v"(v[c + 3]));
        } else if constexpr (G == 8) {
            asm volatile("" : "+v"(v[c]), "+v"(v[c + 1]), "+v"(v[c + 2]), "+v"(v[c + 3]), "+v"(v[c + 4]),
                         "+v"(v[c + 5]), "+v"(v[c + 6]), "+v"(v[c + 7]));
        } else {
            asm volatile("" : "+v"(v[c]), "+v"(v[c + 1]), "+v"(v[c + 2]), "+v"(v[c + 3]), "+v"(v[c + 4]),
                         "+v"(v[c + 5]), "+v"(v[c + 6]), "+v"(v[c + 7]), "+v"(v[c + 8]), "+v"(v[c + 9]),
                         "+v"(v[c + 10]), "+v"(v[c + 11]), "+v"(v[c + 12]), "+v"(v[c + 13]), "+v"(v[c + 14]),
                         "+v"(v[c + 15]));
        }
    }
}
template <class T, int N>
__device__ __forceinline__ void pin_all(T (&v)[N]) {
    pin_groups<N>(v);
}

struct TileInfo {
    int BM, BN, BK, WM, WN;      // tile rows, B rows per tile, K step, wave grid
    int stages;                  // 0: register-staged double buffer; >= 2: direct-to-LDS stages
    int mfma;                    // MFMA output tile edge: 16 or 32
};

// Compiled tiles per weight type (MOE_DT_*).  Returns the count; fills info when non-null.
int gemm_tile_count(int wdtype);
bool gemm_tile_info(int wdtype, int tile, TileInfo *info);
// Workgroups the launch uses (persistent grid) for a given upper bound of tiles.
hipError_t launch_gemm(int wdtype, int tile, GemmKind kind, bool partial, const GemmArgs &a,
                       int64_t max_tiles, hipStream_t s);
// the direct-to-LDS pipelined tiles (gemm_pipe.hip), numbered after the staged ones
bool pipe_tile_info(int wdtype, int tile, TileInfo *info);
hipError_t launch_gemm_pipe(int wdtype, int tile, GemmKind kind, bool partial, const GemmArgs &a,
                            int64_t max_tiles, hipStream_t s);
// int4 tiles of the pipelined kind (gemm_i4.hip): A is bf16 in the (0,4,1,5,2,6,3,7) order
// inside every 8 columns (bf16x8_perm, written by the route or the prologue), and GEMM1
// writes h as bf16 in the same order
bool i4_tile_info(int tile, TileInfo *info);
hipError_t launch_gemm_i4(int tile, GemmKind kind, bool partial, const GemmArgs &a, int64_t max_tiles,
                          hipStream_t s);

struct ReduceArgs {
    const void *Y;               // bf16 [cap, H] or fp32 partials [split, cap, H]
    int64_t partial_stride;
    int split;                   // 0: bf16 rows; >=1: fp32 partial planes
    const int32_t *inv_pos;
    uint16_t *out;               // bf16 [T, H]
    int T, k, H;
    // GEMM2's split tail (null: none): rows from tail_info[0] on are the sum of tail_info[1]
    // fp32 planes of tail_info[2] elements at tail_P; with direct, GEMM2 wrote the other
    // rows' tokens itself (top-1) and only the tail's tokens are written here
    const int32_t *tail_info;
    const float *tail_P;
    int direct;
};
hipError_t launch_reduce(const ReduceArgs &a, hipStream_t s);

// GEMM1 split-K finish: h from the split planes of gate/up sums (fp32 [split, cap, 2I]).
enum { GATE_UP_H_BF16 = 0, GATE_UP_H_F32 = 1, GATE_UP_H_BF16_PERM = 2 };
struct GateUpFinishArgs {
    const float *P;
    int64_t plane;               // elements between split planes
    int split, I;
    const int32_t *sorted, *npp;
    int pairs;
    void *h;                     // [cap, I] in h_kind's format
    int h_kind;                  // GATE_UP_H_*
    uint32_t *amax;              // fp32 h: |h| max as float bits (atomicMax), may be null
    // GEMM1's split tail (null: the split-K planes of every row): rows from tail_info[0]
    // on, tail_info[1] planes (0: none, nothing to do) of tail_info[2] elements, whose row
    // r - tail_info[0] holds row r's sums; plane and split above are then unused
    const int32_t *tail_info;
    int ragged;                  // rows are the T*k pairs (no filler rows; sorted unused)
};
hipError_t launch_gate_up_finish(const GateUpFinishArgs &a, int64_t max_rows, hipStream_t s);
// fp32 h (GATE_UP_H_F32) of a small batch, finished and quantised to E4M3 in one workgroup:
// the pairs' rows through inv_pos; writes |h| max bits to a.amax and amax / 448 to scale_out
hipError_t launch_gate_up_finish_quant(const GateUpFinishArgs &a, const int32_t *inv_pos, uint8_t *hq, float *scale_out,
                                       hipStream_t s);

// fp8 activation quantisation

struct QuantArgs {
    const void *x;               // bf16 rows, or fp32 rows when x_f32
    int x_f32;
    uint8_t *q;                  // e4m3 codes
    int64_t rows, cols;
    const uint32_t *amax;        // float bits
    float *scale_out;            // amax/448 (or 1), written by block 0
    const int32_t *row_valid;    // optional: sorted ids; rows with value >= pairs are zeroed
    const int32_t *npp;          // optional: rows past *npp are skipped
    int pairs;
    // optional: the maximum comes as n_parts partial maxima (float bits) instead of *amax;
    // block 0 stores it to amax_out
    const uint32_t *amax_parts;
    int n_parts;
    uint32_t *amax_out;
};
hipError_t launch_quant(const QuantArgs &a, hipStream_t s);

// bf16 [n8 * 8] with each group of 8 reordered (0,4,1,5,2,6,3,7) (int4 GEMM1's A)

// Route + align (+ the activation pass) of a batch of at most kPrologueMaxT tokens in one
// launch (prologue.hip); results identical to launch_route, launch_align and the fp8 /
// fp16 activation kernels.
// Tokens: up to 64 (16 waves route 4 tokens each); 16 for layers whose routing per token is
// long (more than 64 experts, or top-k above 2).  The fp8 pass (the batch's amax, then its codes, in one workgroup whose threads
// hold the batch in registers) takes at most kPrologueFp8Elems elements.
constexpr int kPrologueMaxT = 64, kPrologueMaxTLongRoute = 16;
constexpr int kPrologueActRegs = 16;                                // 16-byte groups per thread
constexpr int64_t kPrologueFp8Elems = (int64_t)kPrologueActRegs * 1024 * 8;
enum { PROLOGUE_ACT_NONE = 0, PROLOGUE_ACT_FP8 = 1, PROLOGUE_ACT_BF16_PERM = 2 };
struct PrologueArgs {
    RouteArgs route;             // zero_ptr unused
    AlignArgs align;             // ids = route.ids
    int act;                     // PROLOGUE_ACT_*
    const uint16_t *x;           // bf16 hidden [n]
    int64_t n;                   // T * H
    uint8_t *xq;                 // fp8: codes [n]
    uint16_t *xperm;             // int4: bf16 [n] in the packed-nibble order
    uint32_t *x_amax;            // fp8: |x| max as float bits
    float *x_scale;              // fp8: amax / 448 (1 when amax is 0)
    uint32_t *h_amax;            // cleared to 0 (GEMM1's |h| maximum), may be null
};
hipError_t launch_prologue(const PrologueArgs &p, hipStream_t s);

// Block layout of a grouped GEMM over contiguous segments (grouped.hip): E <= 1024, BM a
// power of two; capacity = rows of sorted[].
struct SegmentArgs {
    const int32_t *m_sizes;      // [E] rows per segment (device)
    int E, M, BM, bm_shift;      // BM = 1 << bm_shift
    int32_t *sorted;             // [capacity] source row of each block row, M for padding
    int32_t *eids;               // [capacity / BM] segment of each block
    int32_t *npp;                // [1] block rows
};
hipError_t launch_segments(const SegmentArgs &a, int64_t capacity, hipStream_t s);

int device_cu_count();

}  // namespace moe
