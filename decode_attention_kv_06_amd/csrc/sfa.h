// Internal interface of the sparse (MLA-absorb) decode path.
#pragma once

#include "ifa_decode.h"
#include "internal.h"

namespace ifa {

int sfa_workspace_size(const sfa_mla_args *a, size_t *bytes);
int sfa_run(const sfa_mla_args *a, void *ws, size_t ws_bytes, hipStream_t stream);

}  // namespace ifa
