// q4_floor.hip -- a measurement reference, not part of libq4: the plain
// streaming read of a packed matrix's bytes in one launch.
//
// The kernel reads two planes (codes, then scales) once, 16 bytes per lane
// per step, the grid sweeping memory together (unit g of step t is
// t * (grid threads) + g), with the same non-temporal buffer loads as the
// GEMV's weight stream, and does no arithmetic beyond folding the words it
// reads.  Its time is the floor a product reading the same bytes in one
// launch can reach on the machine; the benchmark times it beside each GEMV.
// Built into libq4floor.so, exported as q4floor_read.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint32_t read_plane(const void *p, uint32_t bytes, uint32_t first, uint32_t stride) {
    const __amdgpu_buffer_rsrc_t r = rsrc(p, bytes);
    uint32_t acc = 0;
    const uint32_t units = bytes >> 4;
    // Four units in flight per lane per trip (the last trip reads past the
    // plane's end through the buffer bounds, which returns zeros).
    for (uint32_t u = first; u < units; u += 4 * stride) {
        const u32x4_t a = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(u * 16u), 0, 2);
        const u32x4_t b = __builtin_amdgcn_raw_buffer_load_b128(r, (int)((u + stride) * 16u), 0, 2);
        const u32x4_t c = __builtin_amdgcn_raw_buffer_load_b128(r, (int)((u + 2 * stride) * 16u), 0, 2);
        const u32x4_t d = __builtin_amdgcn_raw_buffer_load_b128(r, (int)((u + 3 * stride) * 16u), 0, 2);
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w;
        acc ^= c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
    }
    return acc;
}

__global__ void read_kernel(const void *a, uint32_t abytes, const void *b, uint32_t bbytes, uint32_t *out,
                            uint32_t magic) {
    const uint32_t stride = gridDim.x * blockDim.x;
    const uint32_t g = blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = read_plane(a, abytes, g, stride);
    if (b) acc ^= read_plane(b, bbytes, g, stride);
    // A store the compiler cannot prove dead (the caller passes a value the
    // fold practically never equals), so every load is kept.
    if (acc == magic) out[g & 255u] = acc;
}

}  // namespace

extern "C" int q4floor_read(const void *a, uint64_t abytes, const void *b, uint64_t bbytes, uint32_t *out,
                            int grid, int block, void *stream) {
    // (out holds 256 words; grid * block <= 2^24 keeps every byte offset
    // below 2^32, so a read past a plane's end lands outside its buffer
    // range and returns zeros.)
    if (!a || !out || grid < 1 || block < 64 || block > 1024 || block % 64 != 0 ||
        (int64_t)grid * block > (1 << 24))
        return 1;
    if (abytes % 16 != 0 || bbytes % 16 != 0 || abytes >= (1ull << 31) || bbytes >= (1ull << 31)) return 2;
    if (b == nullptr) bbytes = 0;
    hipLaunchKernelGGL(read_kernel, dim3((unsigned)grid), dim3((unsigned)block), 0, (hipStream_t)stream, a,
                       (uint32_t)abytes, b, (uint32_t)bbytes, out, 0x9E3779B9u);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}
