// Internal interface of the DCT-statistics path.  Not part of the public ABI.
#pragma once

namespace cgh {
bool expm(int n, const double *M, double *E);
void set_error(const char *msg);
}  // namespace cgh
