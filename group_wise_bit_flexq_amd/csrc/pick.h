// Host entry of the token-choice kernel, shared by flexq_argmax, flexq_pick and the
// model's output head.
#pragma once

#include "common.h"

namespace flexq {
// `fresh` ignores the incoming stopped flags (the first token of a sequence).
int launch_pick(const float* logits, int64_t M, int64_t N, const flexq_gen_config* gen,
                int32_t step, int32_t m0, int32_t* stopped, bool fresh, int32_t* next,
                hipStream_t stream);
}  // namespace flexq
