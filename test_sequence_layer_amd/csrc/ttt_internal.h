// Internal declarations of libttt.so (not part of the C ABI): every kernel
// family's launch arguments and entry points, for the host-side dispatch.
#pragma once
#include "args_bwd.h"
#include "args_linear.h"
#include "args_mlp.h"
#include "args_mlp_bwd.h"
#include "args_primal.h"
#include "ttt_common.h"
