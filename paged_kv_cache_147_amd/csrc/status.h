// Internal: status codes and the per-thread error detail behind pa_last_error().
#pragma once

#include <string>

#include "pagedkv.h"

namespace pkv {

// Records a failure detail for pa_last_error() and returns the status.
pa_status fail(pa_status code, const std::string& detail);

// Clears the detail; returns PA_OK.
pa_status ok();

}  // namespace pkv
