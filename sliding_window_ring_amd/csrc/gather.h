// gather.h -- arguments of the paged-cache gather (gather.hip), shared with
// the C ABI layer.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace swr {

// One call: request b's window (the positions max(0, pos[b]-W+1) .. pos[b])
// from the pages block_table[b][p / page_tokens] into ring slot p mod W.
struct GatherArgs {
  const uint16_t* k_pages;      // bf16 [n_pages][page_tokens][Hkv][D]
  const uint16_t* v_pages;
  const int32_t* block_table;   // [B][max_pages]
  const int32_t* pos;           // [B]
  uint8_t* k_base;
  uint8_t* v_base;
  const int64_t* k_off;
  const int64_t* v_off;
  int64_t n_pages;
  int page_tokens, max_pages, B, Hkv, D, W;
};

hipError_t launch_paged_gather(const GatherArgs& a, hipStream_t s);

}  // namespace swr
