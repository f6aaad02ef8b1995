// probe.hip -- streaming-read probe: the HBM bandwidth a plain read of a
// large buffer draws on this device, as the yardstick next to which the
// decode kernels' KV-read rate is judged (decode time is the bytes of the
// cache read once per step, [B] "Two Costs: Capacity and Bandwidth").
//
// Every wave reads one contiguous chunk of the buffer exactly once, 16 bytes
// per lane and instruction, 8 instructions in flight per lane, with the
// non-temporal hint (each byte is read once), and folds what it read into a
// checksum so the loads cannot be dropped.  No work but the loads.
#include "pkv_device.hpp"
#include "pkv_kernels.hpp"

namespace pkv {
namespace {

constexpr int kProbeWavesPerGroup = 4;
constexpr int kProbeDepth = 8;           // 16-byte loads in flight per lane

__global__ __launch_bounds__(kProbeWavesPerGroup * kWave)
void stream_read_kernel(const u32x4* buf, long long per_wave, uint32_t* sink)
{
    const long long wave = (long long)blockIdx.x * kProbeWavesPerGroup + (threadIdx.x >> 6);
    const u32x4* p = buf + wave * per_wave + __lane_id();
    uint32_t acc = 0;
    // per_wave is a multiple of kWave * kProbeDepth (checked on the host):
    // every load is in bounds and unconditional
    for (long long i = 0; i < per_wave; i += kWave * kProbeDepth) {
        u32x4 v[kProbeDepth];
#pragma unroll
        for (int k = 0; k < kProbeDepth; ++k)
            v[k] = __builtin_nontemporal_load(p + i + k * kWave);
#pragma unroll
        for (int k = 0; k < kProbeDepth; ++k)
            acc ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
    }
    if (acc == 0x9E3779B9u)              // keeps the loads live; almost never true
        sink[__lane_id()] = acc;
}

} // namespace

hipError_t launch_stream_read(const void* buf, long long bytes, int waves, uint32_t* sink,
                              hipStream_t stream)
{
    const long long per_wave = bytes / 16 / waves;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)(waves / kProbeWavesPerGroup)),
                       dim3(kProbeWavesPerGroup * kWave), 0, stream, (const u32x4*)buf,
                       per_wave, sink);
    return hipGetLastError();
}

} // namespace pkv
