// Direct-to-LDS copies for gfx950 and the waits and barrier that go with
// them (shared by the MFMA router kernels).
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

namespace moe_route {

typedef __attribute__((address_space(3))) void lds_void;

// Direct-to-LDS copies (global_load_lds_dwordx4): lane l copies 16 bytes from
// its global address to LDS byte lds + 16 l (lds goes in M0).  They are inline asm
// so that the compiler neither waits for them on its own (its conservative
// waits drain a whole ring of copies) nor counts them; a ring waits for them
// explicitly with wait_vmcnt, which also counts every other vector-memory
// access of the wave issued before (so other accesses can only make it wait
// longer).  The instruction writes no register, so nothing of the wave is
// overwritten while a copy is in flight.
__device__ __forceinline__ void lds_copy16(const void* src, uint32_t lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" :: "v"(src), "{m0}"(lds)
                 : "memory");
}
__device__ __forceinline__ void lds_copy16(const void* base, uint32_t offset, uint32_t lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" :: "v"(offset), "s"(base),
                 "{m0}"(lds) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(void* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)p));
}

// Workgroup barrier without a memory fence.  A fence here would make every
// wave wait for all of its copies still in flight (they write LDS); a ring
// instead waits explicitly for exactly the copies a step consumes.
__device__ __forceinline__ void barrier_no_fence() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

}  // namespace moe_route
