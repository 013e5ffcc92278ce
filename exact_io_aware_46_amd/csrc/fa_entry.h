// Backward entry shared by the C-ABI front ends (fa_api.cpp and the allocation-free
// variant): bwd_check validates every argument but the workspace and returns FA_OK or a
// fa_status; bwd_entry validates everything, lays out the workspace and launches.
#pragma once

#include <stdint.h>

namespace fa {

int bwd_check(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
              const float* lse, const uint16_t* dO, uint16_t* dq, uint16_t* dk, uint16_t* dv,
              int B, int H, int N, int d, float scale, const int32_t* kv_len, float dropout_p);
int bwd_entry(int dtype, const uint16_t* q, const uint16_t* k, const uint16_t* v,
              const uint16_t* o, const float* lse, const uint16_t* dO, uint16_t* dq,
              uint16_t* dk, uint16_t* dv, int B, int H, int N, int d, float scale, int causal,
              const uint8_t* blockmask, const int32_t* kv_len, int window_left,
              int window_right, float dropout_p, uint64_t seed, uint32_t offset,
              void* workspace, void* stream);

}  // namespace fa
