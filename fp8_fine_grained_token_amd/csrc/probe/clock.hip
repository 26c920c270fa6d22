// Shader-clock probe for the benchmark (not part of the fp8blk library).
//
// One launch records, for each of its workgroups, the compute unit it ran
// on (XCD, shader engine, shader array and CU index from the XCC_ID and
// HW_ID registers), that unit's shader-clock counter (s_memtime, counting
// its core clock) and the constant 100 MHz real-time counter
// (s_memrealtime).  The shader-clock counters of different compute units
// are not aligned with each other, so two launches on the same stream, one
// before and one after a stretch of GPU work, are matched unit by unit: the
// ratio of one unit's two counter increments, times 100 MHz, is its mean
// shader clock over the stretch.  With several workgroups per compute unit
// in each launch, every unit shows up in both.  The probe reads counters
// only: it writes nothing but its own output array.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__global__ __launch_bounds__(64) void clock_probe_kernel(uint64_t *__restrict__ out, int n) {
    if (threadIdx.x != 0 || (int)blockIdx.x >= n) return;
    uint32_t xcc, hw;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
    const uint64_t t = __builtin_amdgcn_s_memtime();
    const uint64_t r = __builtin_amdgcn_s_memrealtime();
    uint64_t *o = out + 3 * (int64_t)blockIdx.x;
    // XCC_ID[3:0]: the XCD; HW_ID[11:8] CU, [12] shader array, [14:13]
    // shader engine
    o[0] = ((uint64_t)(xcc & 0xfu) << 8) | ((hw >> 8) & 0x7fu);
    o[1] = t;
    o[2] = r;
}

}  // namespace

// out: device array of 3 * workgroups uint64 (compute unit: XCD << 8 | SE
// << 5 | SH << 4 | CU; shader-clock count; real-time count; per workgroup);
// workgroups in [1, 4096].  Returns 0 when
// the launch was enqueued, 1 for bad arguments, 2 for a launch error.
extern "C" int fp8probe_clock(uint64_t *out, int workgroups, void *stream) {
    if (out == nullptr || workgroups < 1 || workgroups > 4096) return 1;
    (void)hipGetLastError();
    hipLaunchKernelGGL(clock_probe_kernel, dim3(workgroups), dim3(64), 0,
                       static_cast<hipStream_t>(stream), out, workgroups);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
