// placeholder: statistics path is added next
#include <stddef.h>
#include <stdint.h>
#include "../../include/codec_gauge.h"
#include "cg_stats.hpp"
extern "C" int cg_stats_workspace_bytes(const cg_shape *, int32_t, int32_t, size_t *) { cgh::set_error("not built"); return CG_E_UNSUPPORTED; }
extern "C" int cg_gauge_fit_stats(const cg_shape *, const void *, int32_t, const double *, int32_t, float, float, float, void *, size_t, cg_stats *, double *, void *) { cgh::set_error("not built"); return CG_E_UNSUPPORTED; }
