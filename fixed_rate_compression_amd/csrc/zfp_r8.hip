// Instantiation of the fused zfp-style kernels at 8 bits per value.
#include "zfp_kernels.hpp"

template hipError_t cgk::zfp_launch_rate<8>(bool, bool, int, const void *, const float *, void *,
                                             const cgk::TileArgs &, hipStream_t);
