// Gather-bandwidth probe: the decode's memory access pattern (whole tiles at scattered
// addresses, each read once with the non-temporal hint) with no arithmetic. The
// bandwidth it reaches is the practical ceiling for that pattern on the device, the
// yardstick for the decode kernels next to the HBM peak.
//
// Wave w of W takes tiles w, w + W, w + 2W, ... in trips of U tiles: the next trip's
// offsets are loaded while the current tiles' loads are in flight, then the tiles are
// folded into an XOR. A lane reads 16 bytes of every 1 KiB of a tile. A tile that does
// not lie wholly inside [0, base_bytes) is skipped.
#include "device_common.h"
#include "launchers.h"
#include "pagedkv.h"

namespace pkv {

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <int U, int CH>
__global__ __launch_bounds__(256) void read_tiles_kernel(const uint8_t* __restrict__ base,
                                                         size_t base_bytes,
                                                         const int64_t* __restrict__ offsets,
                                                         int num_tiles,
                                                         uint32_t* __restrict__ sink) {
    constexpr int64_t kTileBytes = CH * 1024;
    const int lane = threadIdx.x & 63;
    const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int waves = gridDim.x * 4;
    auto offset_of = [&](int64_t t) -> int64_t {
        if (t >= num_tiles) return -1;
        const int64_t off = offsets[t];
        return (off >= 0 && off % 16 == 0 && (uint64_t)off + kTileBytes <= base_bytes) ? off
                                                                                       : -1;
    };
    u32x4_t acc = {0u, 0u, 0u, 0u};
    int64_t off[U];
#pragma unroll
    for (int u = 0; u < U; ++u) off[u] = offset_of(wave + (int64_t)u * waves);
    for (int64_t t = wave; t < num_tiles; t += (int64_t)waves * U) {
        int64_t next[U];
#pragma unroll
        for (int u = 0; u < U; ++u) next[u] = offset_of(t + (int64_t)(U + u) * waves);
        u32x4_t v[U][CH];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                v[u][c] = u32x4_t{0u, 0u, 0u, 0u};
                if (off[u] >= 0)
                    v[u][c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(
                        base + off[u] + c * 1024 + lane * 16));
            }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int c = 0; c < CH; ++c) acc ^= v[u][c];
#pragma unroll
        for (int u = 0; u < U; ++u) off[u] = next[u];
    }
    // A store that random data practically never triggers keeps the loads alive.
    const uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (x == 0x9e3779b9u) sink[(size_t)wave * 64 + lane] = x;
}

template <int CH>
int launch_ch(const void* base, size_t base_bytes, const int64_t* offsets, int num_tiles,
              int workgroups, int unroll, uint32_t* sink, hipStream_t stream) {
    const uint8_t* b = static_cast<const uint8_t*>(base);
    switch (unroll) {
        case 1:
            hipLaunchKernelGGL((read_tiles_kernel<1, CH>), dim3(workgroups), dim3(256), 0, stream,
                               b, base_bytes, offsets, num_tiles, sink);
            break;
        case 2:
            hipLaunchKernelGGL((read_tiles_kernel<2, CH>), dim3(workgroups), dim3(256), 0, stream,
                               b, base_bytes, offsets, num_tiles, sink);
            break;
        case 4:
            hipLaunchKernelGGL((read_tiles_kernel<4, CH>), dim3(workgroups), dim3(256), 0, stream,
                               b, base_bytes, offsets, num_tiles, sink);
            break;
        default:
            return -1;
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

int launch_read_tiles(const void* base, size_t base_bytes, const int64_t* offsets,
                      int num_tiles, int tile_bytes, int workgroups, int unroll, uint32_t* sink,
                      hipStream_t stream) {
    if (tile_bytes == 2048)
        return launch_ch<2>(base, base_bytes, offsets, num_tiles, workgroups, unroll, sink,
                            stream);
    if (tile_bytes == 4096)
        return launch_ch<4>(base, base_bytes, offsets, num_tiles, workgroups, unroll, sink,
                            stream);
    return -1;
}

}  // namespace pkv
