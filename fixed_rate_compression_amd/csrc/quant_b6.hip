// Instantiation of the quantizer kernels at 6 bits per code.
#include "quant_launch.hpp"

template hipError_t cgq::quant_launch_bits<6>(bool, bool, int, int, const void *, const float *,
                                              void *, const void *, float *,
                                              const cgq::QuantArgs &, hipStream_t);
