// handoff.h -- passing fp32 partial sums between the workgroups that share
// one output block within a launch (split-K), the last of them to finish
// adding them up and writing the block.
//
// Where the partials travel.  Each of the eight XCDs has its own L2, and the
// L2s are not coherent with each other; within an XCD the one L2 serves
// every compute unit and the per-CU vector L1 is write-through, so a store
// that has completed (vmcnt) is in that L2, where a load from another CU of
// the same XCD that misses its L1 finds it.  Workgroups are dispatched to
// the XCDs round-robin, so workgroups whose ids are congruent mod 8 share an
// L2; the host places the parts of one block on such workgroups, one
// workgroup per part, all resident at once (grid <= compute units).
//
// The placement is checked, not assumed.  When a part starts it adds
// 1 << (8 * xcc) to its block's start word (xcc: the XCC_ID hardware
// register); once it has stored its partial it reads the word back.  If
// every part of the block registered on its own XCD the plain stores are
// enough.  Otherwise (another dispatch order, or a partner that has not
// started) it makes its stores visible device-wide with an agent-scope
// release fence and says so when it arrives; a last part that sees such an
// arrival performs an agent-scope acquire fence before it reads -- the
// memory model's own synchronisation, slower (it writes back and
// invalidates whole caches: about 5 us per launch on the short products
// measured) but correct wherever the parts run.  A part
// that skipped its fence saw all parts on its XCD, the last one included,
// so its partial is in the last part's L2.
//
// Arrivals are counted on the block's arrive word; the part that brings
// the count to the number of parts is last.  It reads every partner's
// partial, writes the block, and clears the record, so every launch finds
// it zero (it starts zeroed when the scratch is created).
#pragma once

#include "device_common.h"
#include "tile_schedule.h"

namespace gb {

// One output block's words, 16 bytes.
struct HandoffRecord {
    unsigned long long start;   // 8 bits per XCD: parts registered there
    unsigned long long arrive;  // bits 0-7: parts arrived, 8-15: of them fenced
};

// The XCD this wave runs on (0..7), or 8 when the register reads anything
// else (then the part never counts as placed on one XCD).
__device__ __forceinline__ int xcd_id() {
    uint32_t v;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
    v &= 0xFu;
    return v < 8u ? (int)v : 8;
}

// Thread 0 of a part, when the part starts.
__device__ __forceinline__ void handoff_register(HandoffRecord *rec, int xcd) {
    if (xcd < 8)
        __hip_atomic_fetch_add(&rec->start, 1ull << (8 * xcd), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Every thread of the part, after it has issued the stores of its partial.
// Returns true in the last part to arrive, whose loads then see every
// partner's partial.  fence_always: take the fenced path even when the
// placement check passes (for testing that path).  flag: a 4-byte LDS word,
// free until the next barrier of the caller.
__device__ __forceinline__ bool handoff_arrive(HandoffRecord *rec, int parts, int xcd, bool fence_always,
                                               uint32_t *flag) {
    wait_vmcnt<0>();  // this wave's stores have completed at its L2
    __syncthreads();  // and every wave's
    if (threadIdx.x == 0) {
        const unsigned long long start = __hip_atomic_load(&rec->start, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool local = !fence_always && xcd < 8 && start == ((unsigned long long)parts << (8 * xcd));
        if (!local) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        const unsigned long long old = __hip_atomic_fetch_add(&rec->arrive, local ? 1ull : 0x101ull,
                                                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = (int)(old & 0xFFu) + 1 == parts;
        const bool fenced = ((old >> 8) & 0xFFu) != 0u || !local;
        *flag = (last ? 1u : 0u) | (fenced ? 2u : 0u);
    }
    __syncthreads();
    const uint32_t f = *flag;
    if ((f & 1u) == 0u) return false;
    if ((f & 2u) != 0u) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    return true;
}

// Thread 0 of the last part, after its reads: the record is zero again.
__device__ __forceinline__ void handoff_reset(HandoffRecord *rec) {
    __hip_atomic_store(&rec->start, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&rec->arrive, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Slot of workgroup w when the grid (a multiple of 8) holds exactly one part
// per workgroup: the workgroups of XCD w % 8 take a contiguous run of slots,
// so when each XCD's run holds whole blocks, a block's parts share an L2.
__device__ __forceinline__ int handoff_slot(int w, int grid) {
    return (w % kNumXcds) * (grid / kNumXcds) + w / kNumXcds;
}

}  // namespace gb
