// Definitions shared by the attention sources: launch parameters, tile
// constants and the device helpers (lane exchanges, the key permutation,
// XCD-aware block order, LDS-DMA loads, wait-count encoding).
#pragma once

#include "common.hpp"

namespace focus {
namespace attn {

constexpr int kRowsPerBlock = 256;  // (query head, entry) rows per block
constexpr int kKeyTile = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazyRescale = 8.0f;
// Largest logit bound (scaled, log2 units) for which the softmax may use the
// bound itself as its fixed exponent offset: P >= 2^-120 stays normal.
constexpr float kFixedOffsetMax = 60.0f;
constexpr int kXcds = 8;

struct Params {
    int hq, hkv, ratio, hpb, nhg;  // ratio = hq/hkv; hpb heads per block; nhg = ratio/hpb
    int64_t n;
    int K, topk;
    int window;  // min(w, n)
    float c;     // scale * log2(e)
    const void *q;
    const void *kmat;  // row-major [hkv][krows][D]
    const void *vmat;  // bf16: [hkv][D][vcols] (transposed); fp32: [hkv][krows][D]
    int64_t krows, vcols;
    // group pass
    const int32_t *tokens;
    const int32_t *offsets;
    const uint32_t *gmask;
    const int32_t *etok;  // position of each bucket entry, [hkv][estride], INT_MAX padded
    const uint32_t *egm;  // gmask of each bucket entry's token, [hkv][estride], 0 padded
    int64_t estride;
    const int4 *tiles;
    // group pass: the work item of each block, heaviest first, when the grid
    // is small enough for its tail to matter (nullptr: XCD-contiguous order)
    const int32_t *order;
    const int32_t *ntiles;
    int max_tiles;
    int64_t E;
    void *part_o;  // normalised partial O per (query head, entry), I/O dtype
    float *part_lse;
    // window pass
    const int32_t *slot_entry;
    int merge;
    void *out;
    float *lse;
    int row_tiles;
    int total_blocks;
    // gated dense pass (training mode): bf16 assignment rows padded to 16
    // or 32 groups, [2][hkv][krows][16 or 32] (A, then -lambda log2(e) A);
    // far pairs (i - j >= gate_w) multiply their score by sigmoid(lambda a_ij)
    const void *apack;
    int gate_w;
    // per key/value head, kNormBlocks partial maxima of the keys' Euclidean
    // norms (their largest bounds every key of the head)
    const float *kpart;
};

constexpr int kNormBlocks = 64;

constexpr int kGateGroups = 32;  // widest assignment row of the gated pass

// ---------------------------------------------------------------------------
// small helpers

__device__ __forceinline__ float swap_halves_max(float x)
{
    auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                               false);
    return fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
}

__device__ __forceinline__ float swap_halves_sum(float x)
{
    auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                               false);
    return __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
}

// Row of the 32x32 accumulator held by lane half h in register r (the MFMA
// output layout), and the key that row carries after the sigma permutation.
__device__ __forceinline__ int sigma(int m)
{
    return ((m >> 2) & 1) * 16 + (m & 3) + 4 * (m >> 3);
}

// Remap of a linear block index so that each XCD (blocks are dealt to the 8
// XCDs round-robin) walks one contiguous range of the work list: tiles of one
// head and group then share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int b, int total_padded)
{
    const int per = total_padded / kXcds;
    return (b % kXcds) * per + b / kXcds;
}

// (Take the LDS address of an array itself and add offsets to the 32-bit
// result: converting "array + offset" back from a generic pointer costs a
// null test and keeps the 64-bit generic pointer alive.)
// LDS-DMA: each lane loads 16 (or 4) bytes from gbase + voff and the
// wavefront's 64 results land contiguously at LDS byte address lds_addr (via
// M0).  Issued from inline assembly so that the compiler neither tracks nor
// waits for these loads: the kernel waits for them itself (vmcnt) before the
// barrier that publishes a stage.  M0 is saved and restored around the load;
// writing M0 needs one wait state before the load reads it.
__device__ __forceinline__ uint32_t lds_address(const void *p)
{
    return __builtin_amdgcn_readfirstlane(
        (uint32_t)(size_t)(const __attribute__((address_space(3))) char *)p);
}

// (Both the LDS address and the global base are wave-uniform; readfirstlane
// puts them in the scalar registers the instruction reads them from.)
__device__ __forceinline__ const void *uniform_ptr(const void *p)
{
    const uint64_t v = (uint64_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const void *)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ void dma16(const void *gbase, uint32_t voff, uint32_t lds_addr)
{
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %2, %3\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(uniform_ptr(gbase))
                 : "memory");
}

__device__ __forceinline__ void dma4(const void *gbase, uint32_t voff, uint32_t lds_addr)
{
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
                 "global_load_lds_dword %2, %3\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(uniform_ptr(gbase))
                 : "memory");
}

// base + off as one vector add the compiler can neither hoist nor fold:
// for an address that would otherwise be kept, per stage, in registers
// across a loop (base wave-uniform, in a scalar register)
__device__ __forceinline__ uint32_t lds_add(uint32_t base, uint32_t off)
{
    uint32_t r;
    asm volatile("v_add_u32 %0, %1, %2" : "=v"(r) : "s"(base), "v"(off));
    return r;
}

// 16-byte LDS read at a 32-bit LDS byte address
__device__ __forceinline__ bf16x8 lds_read16(uint32_t addr)
{
    return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8 *>(addr);
}

// Immediate of "s_waitcnt vmcnt(n) lgkmcnt(0)" (expcnt untouched) on gfx9:
// vmcnt is split over bits 3:0 and 15:14, expcnt is bits 6:4, lgkmcnt 11:8.
constexpr int waitcnt_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70; }
static_assert(waitcnt_vm_lgkm0(0) == 0x70 && waitcnt_vm_lgkm0(20) == 0x4074, "encoding");

}  // namespace attn
}  // namespace focus
