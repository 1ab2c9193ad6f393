// Host orchestration of the operations, shared by the C-ABI entry points.
#pragma once

#include "../../include/ortho.h"

namespace ortho {

// The Dion step sequence of dion_step_batched on an already validated group,
// with `ws` holding at least the planned workspace (no optional outputs).
ortho_status dion_run(int32_t batch, const ortho_mat* X, const ortho_mat* G, const ortho_mat* M,
                      const ortho_mat* Q, int32_t r, float mu, float lr, float scale, void* ws,
                      void* stream);

}  // namespace ortho
