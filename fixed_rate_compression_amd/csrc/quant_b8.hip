// Instantiation of the quantizer kernels at 8 bits per code.
#include "quant_launch.hpp"

template hipError_t cgq::quant_launch_bits<8>(bool, bool, int, int, const void *, const float *,
                                              void *, const void *, float *,
                                              const cgq::QuantArgs &, hipStream_t);
