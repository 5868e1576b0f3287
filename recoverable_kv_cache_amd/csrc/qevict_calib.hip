// Measurement aid, not part of the method: a plain streaming read of a device buffer,
// to set the split kernel's bandwidth beside what one launch that only reads the same
// number of bytes achieves on the same machine.  Each byte is read once with 16-byte
// buffer loads (range-checked by the hardware, so the tail needs no per-lane branch),
// several loads in flight per wave; each workgroup folds what it read into one XOR word.
#include <hip/hip_ext.h>

#include "qevict_internal.h"

namespace qv {

constexpr int SR_LOADS = 4;   // 1 KB pieces in flight per wave

__device__ __forceinline__ uint32_t wave_xor(uint32_t x) {
    x ^= (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, true);    // quad [1,0,3,2]
    x ^= (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, true);    // quad [2,3,0,1]
    x ^= (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x141, 0xF, 0xF, true);   // row_half_mirror
    x ^= (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x140, 0xF, 0xF, true);   // row_mirror
    const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    x = a[0] ^ a[1];
    const auto c = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return c[0] ^ c[1];
}

__global__ void __launch_bounds__(256) k_stream_read(const uint8_t* __restrict__ buf, uint32_t bytes,
                                                     uint32_t* __restrict__ sink) {
    __shared__ uint32_t part[4];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(buf), (short)0,
                                                                        (int)bytes, 0x00020000);
    const uint32_t pieces = bytes / 1024, nw = gridDim.x * 4;
    uint32_t x = 0;
    for (uint32_t p0 = (blockIdx.x * 4 + wv) * SR_LOADS; p0 < pieces; p0 += nw * SR_LOADS) {
        uint32_t v[SR_LOADS][4];
#pragma unroll
        for (int k = 0; k < SR_LOADS; ++k) {   // pieces past the end read as zeros
            const auto t = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)((p0 + k) * 1024u + lane * 16u), 0, 0);
            v[k][0] = t[0], v[k][1] = t[1], v[k][2] = t[2], v[k][3] = t[3];
        }
#pragma unroll
        for (int k = 0; k < SR_LOADS; ++k) x ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
    }
    x = wave_xor(x);
    if (lane == 0) part[wv] = x;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

hipError_t launch_stream_read(const void* buf, uint32_t bytes, uint32_t* sink, hipStream_t s, hipEvent_t ev0,
                              hipEvent_t ev1) {
    const dim3 grid(STREAM_READ_WGS), block(256);
    if (ev0)
        hipExtLaunchKernelGGL(k_stream_read, grid, block, 0, s, ev0, ev1, 0, (const uint8_t*)buf, bytes, sink);
    else
        hipLaunchKernelGGL(k_stream_read, grid, block, 0, s, (const uint8_t*)buf, bytes, sink);
    return hipGetLastError();
}

}  // namespace qv
