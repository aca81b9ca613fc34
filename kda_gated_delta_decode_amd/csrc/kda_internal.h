// kda_internal.h -- declarations shared by the two translation units of the
// KDA decode library (host validation and kernel launch).  Internal header.
#pragma once

#include <stdint.h>

#include "kda_decode.h"

namespace kda {

// Checks shared by kda_decode_step and kda_validate: pointer to the pool,
// dtype admission and match, shape, rows per request, counts.  Returns
// KDA_OK or the first failing kda_status.
int check_common(const kda_pool* pool, int32_t n_req, int32_t n_rows, kda_dtype state_dtype);

}  // namespace kda
