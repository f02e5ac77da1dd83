// gemv_tile_g128.hip — the decode tile kernel instantiated for group size 128 (one translation
// unit per group size, so they compile in parallel).
#include "gemv_tile.h"
#include "q4_launch.h"

hipError_t q4k_gemv_tile_g128(int sym, int x_dtype, int m, int k, int upw, int waves, int wide,
                             const q4::GemvBatch& batch, int tiles, hipStream_t stream,
                             const char** kname) {
    return q4t::launch_tile<128>(sym, x_dtype, m, k, upw, waves, wide, batch, tiles, stream, kname);
}
