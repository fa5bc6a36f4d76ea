// pipe.h -- device helpers of the direct-to-LDS pipelined GEMMs (gemm_pipe.hip, gemm_i4.hip).
#pragma once

#include "common.h"

namespace moe {

typedef __attribute__((address_space(3))) void *lds_ptr;
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Byte address of an LDS object in the LDS address space (what M0 holds for a DMA load).
template <class T>
__device__ __forceinline__ uint32_t lds_addr(T *p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)p;
}

// Direct-to-LDS load of 16 (or 4) bytes per lane: lane l's bytes land at LDS address
// lds + 16 l (4 l).  Issued as inline assembly: the compiler cannot tell which stage buffer
// such a load fills, and around its own builtin it may insert s_waitcnt vmcnt(0) before
// LDS reads, draining the stages in flight.  Stage order is kept by the kernels' explicit
// s_waitcnt vmcnt and s_barrier; the "memory" clobber keeps every memory access in program
// order around it.
// M0 is a register the compiler reserves (it warns that a clobber of it may not be
// preserved): the statement writes M0 itself, right before the load that reads it, and
// the kernels using it keep no other value in M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <int BYTES>
__device__ __forceinline__ void lds_dma(const void *g, uint32_t lds) {
    static_assert(BYTES == 16 || BYTES == 4, "dwordx4 or dword");
    const uint32_t m = __builtin_amdgcn_readfirstlane(lds);
    if constexpr (BYTES == 16)
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(m) : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(m) : "memory", "m0");
}

// A wave-uniform pointer as the compiler's uniform (SGPR) value.
template <class T>
__device__ __forceinline__ const T *uniform_ptr(const T *p) {
    const uint64_t b = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b), hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    return (const T *)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// The same load with a wave-uniform 64-bit base (SGPRs) and a 32-bit per-lane byte offset:
// one VGPR per load instead of a 64-bit address, and advancing the base is scalar work.
template <int BYTES>
__device__ __forceinline__ void lds_dma_off(const void *base, uint32_t voff, uint32_t lds) {
    static_assert(BYTES == 16 || BYTES == 4, "dwordx4 or dword");
    const void *sb = uniform_ptr((const char *)base);
    const uint32_t m = __builtin_amdgcn_readfirstlane(lds);
    if constexpr (BYTES == 16)
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sb), "s"(m) : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sb), "s"(m) : "memory", "m0");
}
#pragma clang diagnostic pop

// A wave-uniform 32-bit read through the scalar data cache, waited for in the same statement:
// the value lands in an SGPR, and the wait (lgkmcnt) leaves the wave's vector loads and
// stores in flight, where a vector load's vmcnt wait would drain them -- the stores of the
// previous tile's epilogue, or stages already issued.  For the tile walk's small read-only
// arrays (expert of each row block, block starts), written by an earlier launch.
__device__ __forceinline__ int sload(const int32_t *p) {
    const int32_t *q = uniform_ptr(p);
    int v;
    asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=&s"(v) : "s"(q) : "memory");
    return v;
}
// p[0] and p[1], both in flight before the one wait
__device__ __forceinline__ int2 sload_pair(const int32_t *p) {
    const int32_t *q = uniform_ptr(p);
    int v0, v1;
    asm volatile("s_load_dword %0, %2, 0x0\n\ts_load_dword %1, %2, 0x4\n\ts_waitcnt lgkmcnt(0)"
                 : "=&s"(v0), "=&s"(v1)
                 : "s"(q)
                 : "memory");
    return make_int2(v0, v1);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// wait until at most n (a multiple of LPW, n <= MAXS*LPW) of this wave's loads are pending
template <int LPW, int MAXS>
__device__ __forceinline__ void wait_stages(int later) {
    if constexpr (MAXS >= 3) {
        if (later >= 3) { wait_vmcnt<3 * LPW>(); return; }
    }
    if constexpr (MAXS >= 2) {
        if (later >= 2) { wait_vmcnt<2 * LPW>(); return; }
    }
    if constexpr (MAXS >= 1) {
        if (later >= 1) { wait_vmcnt<LPW>(); return; }
    }
    wait_vmcnt<0>();
}

// s_barrier without the fence of __syncthreads() (which would drain every pending load)
__device__ __forceinline__ void block_barrier() {
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// LDS position of 16-byte chunk c of tile row r is c ^ swz(r): a pair of rows shares a
// position in the two halves of the 64 banks, 8 pairs cover the 8 positions, so 16 lanes
// reading one chunk of 16 consecutive rows hit 64 distinct banks
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

// Other read patterns want other keys (measured on gfx950 with SQ_LDS_BANK_CONFLICT, which
// shows that a ds_read_b128 is not served as four groups of 16 consecutive lanes): where the
// four 16-lane groups read chunks 0, 2, 4, 6 (or 1, 3, 5, 7) of 16 rows -- an fp8 fragment
// takes 32 bytes a lane, chunks 2g and 2g + 1 -- swz costs 4 conflict cycles per read and
// key 1 = 2 (r & 3) + ((r >> 2) & 1) none; where groups read chunk c of a slab and c + 4 of
// the slab after it (int4's A fragments) key 2 = (r >> 1) & 3 has none.  Key 0 is swz.
template <int K>
__device__ __forceinline__ int swz_key(int r) {
    if constexpr (K == 1) return 2 * (r & 3) + ((r >> 2) & 1);
    else if constexpr (K == 2) return (r >> 1) & 3;
    else return swz(r);
}

// Slabs of SB = 64-byte rows (32 bf16 of K) pack two rows into each 128-byte line: row r
// is line r / 2, half r % 2, and its chunk c (0..3) sits at position (4 (r % 2) + c) ^ s
// with s = (line / 2) % 4.  16 lanes reading one chunk of 16 consecutive rows touch 8
// lines; lines alternate between the two halves of the banks, and within a half the four
// lines have four different s, so the 16 positions are all distinct: conflict-free like
// the 128-byte layout.
template <int SB, int K = 0>
__device__ __forceinline__ int slab_off(int r, int c) {
    static_assert(SB == 128 || K == 0, "the 64-byte slabs have one layout");
    if constexpr (SB == 128) return r * 128 + ((c ^ swz_key<K>(r)) << 4);
    else return (r >> 1) * 128 + (((((r & 1) << 2) | c) ^ ((r >> 2) & 3)) << 4);
}

// The row and chunk that lane `lane` of a DMA instruction filling the 1024 LDS bytes of
// rows rb .. rb + 1024 / SB - 1 (rb a multiple of that count) must load: lane l writes
// LDS bytes 16 l .. 16 l + 15 of the instruction's range, i.e. slab_off(row, chunk).
template <int SB, int K = 0>
__device__ __forceinline__ void dma_lane(int lane, int rb, int &row, int &chunk) {
    static_assert(SB == 128 || K == 0, "the 64-byte slabs have one layout");
    if constexpr (SB == 128) {
        row = rb + (lane >> 3);
        chunk = (lane & 7) ^ swz_key<K>(row);
    } else {
        const int line = (rb >> 1) + (lane >> 3);
        const int v = (lane & 7) ^ ((line >> 1) & 3);
        row = 2 * line + (v >> 2);
        chunk = v & 3;
    }
}

template <int MS> struct AccOf { typedef f32x4 type; };
template <> struct AccOf<32> { typedef f32x16 type; };

// Row of a 16x16 (32x32) MFMA output fragment held in accumulator value r of this lane;
// its column is lane % 16 (lane % 32).
template <int MS>
__device__ __forceinline__ int frag_row(int lane, int r) {
    if constexpr (MS == 32) return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    return 4 * (lane >> 4) + r;
}

// Persistent-grid tile walk shared by the grouped GEMMs: split outermost, then groups of
// group_m row blocks with the block index fastest inside a group.
struct TileCoord {
    int s, mb, nt;
};
__device__ __forceinline__ TileCoord tile_coord(int tile, int mn, int mblocks, int ntiles, int group_m) {
    TileCoord c;
    c.s = tile / mn;
    const int rest = tile - c.s * mn;
    const int gm0 = rest / (group_m * ntiles) * group_m;
    const int gsz = min(group_m, mblocks - gm0);
    const int local = rest - gm0 * ntiles;
    c.mb = gm0 + local % gsz;
    c.nt = local / gsz;
    return c;
}

// The same walk with groups aligned to experts: the row blocks of one expert, at most gmax
// per group (eids is non-decreasing over the row blocks), so that the tiles in flight on an
// XCD share the expert's weight tiles instead of straddling two experts.
__device__ __forceinline__ TileCoord tile_coord_expert(int tile, int mn, int mblocks, int ntiles,
                                                       const int32_t *eids, int gmax) {
    TileCoord c;
    c.s = tile / mn;
    const int rest = tile - c.s * mn;
    const int bt = rest / ntiles;                 // a block of rest's group (groups span all column tiles)
    const int e = sload(eids + bt);
    int lo = 0, hi = bt;                          // first block of expert e
    while (lo < hi) {
        const int m = (lo + hi) / 2;
        if (sload(eids + m) < e) lo = m + 1;
        else hi = m;
    }
    const int efirst = lo;
    lo = bt + 1;                                  // one past its last block below mblocks
    hi = mblocks;
    while (lo < hi) {
        const int m = (lo + hi) / 2;
        if (sload(eids + m) <= e) lo = m + 1;
        else hi = m;
    }
    const int b0 = efirst + (bt - efirst) / gmax * gmax;
    const int gsz = min(gmax, lo - b0);
    const int local = rest - b0 * ntiles;
    c.mb = b0 + local % gsz;
    c.nt = local / gsz;
    return c;
}

// workgroup b of a grid of G (a multiple of 8) starts at tile j0: consecutive tiles go to
// one XCD (workgroups are dealt to the 8 XCDs round-robin)
__device__ __forceinline__ int xcd_first_tile(int b, int G) {
    return (G % 8 == 0) ? (b % 8) * (G / 8) + b / 8 : b;
}

}  // namespace moe
