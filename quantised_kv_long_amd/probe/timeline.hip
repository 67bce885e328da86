// timeline.hip -- the library with a per-workgroup timeline in the attention
// kernel (decode_mfma_kernel).  Not part of the decode path: it measures how
// the workgroups of one launch start and end, which no per-kernel profile
// shows (the static split of rows into workgroups leaves HBM idle while the
// last workgroups finish).
//
// The same kernels as the library: this file defines the timeline points the
// kernel source leaves empty and then compiles that source.  Thread 0 of each
// workgroup stores, with ordinary vector stores, the 100 MHz constant clock
// (s_memrealtime) at the timeline points of the kernel source (start, wave
// 0's last tile, end; in the four-wave merge also all loops done and merge
// area written), plus the XCC and hardware ids of the CU it ran on.  Every launch of the
// attention kernel overwrites the records of its workgroups, so after a run
// the buffer holds the last launch's timeline.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace kvq_timeline {
// per workgroup: clock at points 0, 1, 2, then (xcc_id << 32) | hw_id, then
// the clock at points 3 and 4, two words unused
constexpr int WORDS = 8;
constexpr int MAX_WG = 65536;
__device__ uint64_t records[WORDS * MAX_WG];

__device__ __forceinline__ int slot(int point) { return point < 3 ? point : point + 1; }

__device__ __forceinline__ void record(int point)
{
    if (threadIdx.x != 0) return;
    const unsigned id = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    if (id >= (unsigned)MAX_WG) return;
    const uint64_t t = __builtin_amdgcn_s_memrealtime();
    records[WORDS * id + slot(point)] = t;
    if (point == 0) {
        unsigned xcc, hw;
        asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
        asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
        // a split with no rows, or a kernel without the merge, records no
        // later points
        records[WORDS * id + slot(1)] = 0;
        records[WORDS * id + slot(3)] = 0;
        records[WORDS * id + slot(4)] = 0;
        records[WORDS * id + 3] = ((uint64_t)xcc << 32) | hw;
    }
}
}  // namespace kvq_timeline

#define KVQ_TL(point) kvq_timeline::record(point)
#include "decode_mfma.hip"

// Copies the first `bytes` of the records (8 x uint64 per workgroup, in
// launch order of blockIdx) to host memory; returns the hipError_t.
extern "C" int kvq_timeline_read(void* dst, size_t bytes)
{
    if (bytes > sizeof(kvq_timeline::records)) return (int)hipErrorInvalidValue;
    return (int)hipMemcpyFromSymbol(dst, HIP_SYMBOL(kvq_timeline::records), bytes, 0, hipMemcpyDeviceToHost);
}

extern "C" int kvq_timeline_capacity(void) { return kvq_timeline::MAX_WG; }
