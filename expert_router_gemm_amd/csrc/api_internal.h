// api_internal.h -- the layer entry's argument checks and launch sequence,
// shared by the exported layer entry points (moe_api.cpp, noalloc.hip).
// Not exported from the library.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// The argument checks of moe_layer_forward (shape, T, pointers and their
// alignment; not the workspace).  MOE_OK for T == 0 with a valid shape.
moe_status layer_forward_validate(const moe_shape *shape, const moe_weights *w,
                                  const moe_slot_map *map, int32_t T, const void *h, void *out);

// moe_layer_forward with optional stage events (prof may be NULL): checks
// the arguments and the workspace, then enqueues the layer on `stream`.
moe_status layer_forward_run(const moe_shape *shape, const moe_weights *w,
                             const moe_slot_map *map, int32_t T, const void *h, void *out,
                             void *ws, size_t ws_bytes, const moe_profile *prof, void *stream);

}  // namespace moe
